/*
 * ssd_oracle.c -- plain, slow, fp64 CPU evaluation of the Mamba-2 SSD prefill.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this file; only the test suite, the smoke check and the CPU-baseline leg
 * of the benchmark use it.  It shares no code with the HIP library.
 *
 * Sources (cited by page title and section):
 *   [XLA] "Mamba-2状态空间模型的编译器优化与实现", section 1.1 (state space model
 *         basics): the discrete recurrence h_t = A_bar h_{t-1} + B_bar x_t,
 *         y_t = C h_t + D x_t, with B, C and the step size input dependent and A
 *         a per-head scalar.
 *   [HW]  "Mamba 硬件感知算法", section "块分解与状态传递" (chunk decomposition and
 *         state passing): intra-chunk output from a zero state, chunk-end states,
 *         state passing across chunks, output contribution of the passed state.
 *   [KF]  "Mamba-2炸裂升级！大模型推理飙升20%，效率翻2.5倍！" (repost of "Accelerating
 *         Mamba2 with Kernel Fusion"), section "Mamba-2核心操作与融合的必要性"
 *         (Mamba-2 core operations): the five SSD steps chunk_cumsum (per-token dt
 *         and in-chunk cumulative decay), chunk_state, state_passing, bmm and
 *         chunk_scan.
 *
 * Readings taken where the pages are silent (each also listed in the design notes):
 *   - the step size is dt = softplus(dt_raw + dt_bias) when dt_softplus != 0,
 *     else dt_raw + dt_bias; softplus is exact (no threshold, no clamp);
 *   - the decay over one token is exp(dt * A) and the input term is
 *     dt * x_t (outer) B_t (the Mamba-2 form, not the zero-order-hold B_bar);
 *   - the state of head h is a [P, N] matrix, S[p][n] += dt * x[p] * B[n];
 *   - head h reads the B/C group g = h / (H / G) (contiguous blocks of heads);
 *   - a null initial state means zeros; null D / dt_bias mean zeros;
 *   - every 16-bit input element is widened exactly to fp64 before use.
 *
 * Three formulations live here so that each can be checked against the others:
 *   ssd_oracle_recurrence  the definition itself (sequential, per token);
 *   ssd_oracle_chunked     the five-step chunked algorithm, exposing each step's
 *                          intermediate tensors.
 * The quadratic ("attention") form used as a third check is in quadratic.py.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };

typedef struct {
    int batch, seqlen, nheads, headdim, dstate, ngroups;
    int in_dtype;     /* dtype of x, dt, B, C (OR_*) */
    int state_dtype;  /* dtype of the initial state (OR_*) */
    int dt_softplus;  /* 1: dt = softplus(dt_raw + dt_bias); 0: dt = dt_raw + dt_bias */
    const void* x;    /* [B, L, H, P] */
    const void* dt;   /* [B, L, H]    */
    const float* A;   /* [H]          */
    const void* Bm;   /* [B, L, G, N] */
    const void* Cm;   /* [B, L, G, N] */
    const float* D;   /* [H] or NULL  */
    const float* dt_bias; /* [H] or NULL */
    const void* h0;   /* [B, H, P, N] or NULL */
} ssd_oracle_problem;

/* ---- exact widening of stored elements to fp64 ------------------------- */

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
static double half_bits_to_double(uint16_t h) {
    int sign = h >> 15;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);              /* subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);  /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16 is the upper half of an IEEE-754 binary32. */
static double bf16_bits_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double load_elem(const void* base, int dtype, size_t idx) {
    switch (dtype) {
    case OR_F32: return (double)((const float*)base)[idx];
    case OR_F16: return half_bits_to_double(((const uint16_t*)base)[idx]);
    default:     return bf16_bits_to_double(((const uint16_t*)base)[idx]);
    }
}

/* Exported so the tests can check the widening against an independent one. */
void ssd_oracle_widen(const void* src, int dtype, long n, double* out) {
    for (long i = 0; i < n; ++i) out[i] = load_elem(src, dtype, (size_t)i);
}

/* softplus(z) = log(1 + e^z), evaluated without overflow. */
static double softplus(double z) {
    return z > 0 ? z + log1p(exp(-z)) : log1p(exp(z));
}

static double step_size(const ssd_oracle_problem* pr, int b, int t, int h) {
    const size_t L = (size_t)pr->seqlen, H = (size_t)pr->nheads;
    double z = load_elem(pr->dt, pr->in_dtype, ((size_t)b * L + t) * H + h);
    if (pr->dt_bias) z += (double)pr->dt_bias[h];
    return pr->dt_softplus ? softplus(z) : z;
}

/* ---- the definition: sequential recurrence ------------------------------ */

/*
 * For every (b, h) in bh[0 .. nbh) (pairs, flattened as b * H + h), run
 *     S <- exp(dt_t A_h) S + dt_t x_t (outer) B_t,   y_t = S C_t + D_h x_t
 * over t = 0 .. L-1 from S = h0 (or 0).
 * Outputs (all optional): y[nbh][L][P], final[nbh][P][N], and, when snap_q > 0,
 * snaps[nbh][ceil(L / snap_q)][P][N] = the state after token min((k+1) snap_q, L) - 1.
 * Returns 0, or -1 for bad arguments.
 */
int ssd_oracle_recurrence(const ssd_oracle_problem* pr, const int* bh, int nbh,
                          double* y, double* final_state, int snap_q, double* snaps) {
    if (!pr || !bh || nbh < 0) return -1;
    const int L = pr->seqlen, H = pr->nheads, P = pr->headdim, N = pr->dstate, G = pr->ngroups;
    if (L < 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return -1;
    const int hpg = H / G;
    const int nsnap = snap_q > 0 ? (L + snap_q - 1) / snap_q : 0;

    int err = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int k = 0; k < nbh; ++k) {
        const int b = bh[k] / H, h = bh[k] % H, g = h / hpg;
        if (b < 0 || b >= pr->batch) { err = -1; continue; }
        double* S = (double*)calloc((size_t)P * N, sizeof(double));
        double* Bt = (double*)malloc((size_t)N * sizeof(double));
        double* Ct = (double*)malloc((size_t)N * sizeof(double));
        double* xt = (double*)malloc((size_t)P * sizeof(double));
        if (pr->h0) {
            const size_t base = ((size_t)b * H + h) * P * N;
            for (size_t i = 0; i < (size_t)P * N; ++i) S[i] = load_elem(pr->h0, pr->state_dtype, base + i);
        }
        const double Ah = (double)pr->A[h];
        const double Dh = pr->D ? (double)pr->D[h] : 0.0;
        for (int t = 0; t < L; ++t) {
            const double d = step_size(pr, b, t, h);
            const double a = exp(d * Ah);
            const size_t bc = (((size_t)b * L + t) * G + g) * N;
            const size_t xb = (((size_t)b * L + t) * H + h) * P;
            for (int n = 0; n < N; ++n) {
                Bt[n] = load_elem(pr->Bm, pr->in_dtype, bc + n);
                Ct[n] = load_elem(pr->Cm, pr->in_dtype, bc + n);
            }
            for (int p = 0; p < P; ++p) xt[p] = load_elem(pr->x, pr->in_dtype, xb + p);
            for (int p = 0; p < P; ++p) {
                double* Sp = S + (size_t)p * N;
                const double coef = d * xt[p];
                double acc = 0.0;
                for (int n = 0; n < N; ++n) {
                    Sp[n] = a * Sp[n] + coef * Bt[n];
                    acc += Sp[n] * Ct[n];
                }
                if (y) y[((size_t)k * L + t) * P + p] = acc + Dh * xt[p];
            }
            if (snaps && (t == L - 1 || (t + 1) % snap_q == 0)) {
                const int s = t / snap_q;
                memcpy(snaps + ((size_t)k * nsnap + s) * P * N, S, (size_t)P * N * sizeof(double));
            }
        }
        if (final_state) memcpy(final_state + (size_t)k * P * N, S, (size_t)P * N * sizeof(double));
        free(S); free(Bt); free(Ct); free(xt);
    }
    return err;
}

/* ---- the five-step chunked algorithm ------------------------------------ */

/*
 * Chunk size Q (any Q >= 1), nc = ceil(L / Q).  Positions past L inside the last
 * chunk do not exist: they carry dt = 0 and zero x, B, C, so they change nothing.
 * Outputs (each optional, all fp64, row-major):
 *   dt_out  [B][nc][H][Q]        step size per token (chunk_cumsum)
 *   acs_out [B][nc][H][Q]        inclusive in-chunk cumulative sum of dt * A (chunk_cumsum)
 *   cb_out  [B][nc][G][Q][Q]     CB[i][j] = C_i . B_j (bmm)
 *   s_out   [B][nc][H][P][N]     chunk-end state from a zero start (chunk_state)
 *   st_out  [B][nc+1][H][P][N]   state entering chunk c; slot nc is the final state (state_passing)
 *   y       [B][L][H][P]         output (chunk_scan)
 *   final_state [B][H][P][N]
 * Returns 0, or -1 for bad arguments / allocation failure.
 */
int ssd_oracle_chunked(const ssd_oracle_problem* pr, int Q,
                       double* dt_out, double* acs_out, double* cb_out, double* s_out,
                       double* st_out, double* y, double* final_state) {
    if (!pr || Q <= 0) return -1;
    const int Bn = pr->batch, L = pr->seqlen, H = pr->nheads, P = pr->headdim, N = pr->dstate, G = pr->ngroups;
    if (Bn <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G) return -1;
    const int hpg = H / G;
    const int nc = (L + Q - 1) / Q;
    const size_t PN = (size_t)P * N;

    double* dtc = (double*)calloc((size_t)Bn * nc * H * Q, sizeof(double));
    double* acs = (double*)calloc((size_t)Bn * nc * H * Q, sizeof(double));
    double* cb = (double*)calloc((size_t)Bn * nc * G * Q * Q, sizeof(double));
    double* s = (double*)calloc((size_t)Bn * nc * H * PN, sizeof(double));
    double* st = (double*)calloc((size_t)Bn * (nc + 1) * H * PN, sizeof(double));
    if (!dtc || !acs || !cb || !s || !st) {
        free(dtc); free(acs); free(cb); free(s); free(st);
        return -1;
    }
#define TOK(c, i) ((c) * Q + (i))
#define IDX_DT(b, c, h, i) ((((size_t)(b) * nc + (c)) * H + (h)) * Q + (i))
#define IDX_CB(b, c, g, i, j) (((((size_t)(b) * nc + (c)) * G + (g)) * Q + (i)) * Q + (j))
#define IDX_S(b, c, h) ((((size_t)(b) * nc + (c)) * H + (h)) * PN)
#define IDX_ST(b, c, h) ((((size_t)(b) * (nc + 1) + (c)) * H + (h)) * PN)
#define XV(b, t, h, p) load_elem(pr->x, pr->in_dtype, ((((size_t)(b) * L + (t)) * H + (h)) * P + (p)))
#define BV(b, t, g, n) load_elem(pr->Bm, pr->in_dtype, ((((size_t)(b) * L + (t)) * G + (g)) * N + (n)))
#define CV(b, t, g, n) load_elem(pr->Cm, pr->in_dtype, ((((size_t)(b) * L + (t)) * G + (g)) * N + (n)))

    /* step 1, chunk_cumsum: per-token dt and its in-chunk running sum of dt * A */
#pragma omp parallel for collapse(2)
    for (int b = 0; b < Bn; ++b)
        for (int c = 0; c < nc; ++c)
            for (int h = 0; h < H; ++h) {
                double run = 0.0;
                for (int i = 0; i < Q; ++i) {
                    const int t = TOK(c, i);
                    const double d = t < L ? step_size(pr, b, t, h) : 0.0;
                    run += d * (double)pr->A[h];
                    dtc[IDX_DT(b, c, h, i)] = d;
                    acs[IDX_DT(b, c, h, i)] = run;
                }
            }

    /* step 2, bmm: CB[i][j] = sum_n C[i][n] B[j][n] inside each chunk, per group */
#pragma omp parallel for collapse(3)
    for (int b = 0; b < Bn; ++b)
        for (int c = 0; c < nc; ++c)
            for (int g = 0; g < G; ++g)
                for (int i = 0; i < Q; ++i)
                    for (int j = 0; j < Q; ++j) {
                        const int ti = TOK(c, i), tj = TOK(c, j);
                        double acc = 0.0;
                        if (ti < L && tj < L)
                            for (int n = 0; n < N; ++n) acc += CV(b, ti, g, n) * BV(b, tj, g, n);
                        cb[IDX_CB(b, c, g, i, j)] = acc;
                    }

    /* step 3, chunk_state: the state each chunk reaches from a zero start,
       s[p][n] = sum_j exp(Acs[Q-1] - Acs[j]) dt[j] x[j][p] B[j][n] */
#pragma omp parallel for collapse(3)
    for (int b = 0; b < Bn; ++b)
        for (int c = 0; c < nc; ++c)
            for (int h = 0; h < H; ++h) {
                const int g = h / hpg;
                double* sp = s + IDX_S(b, c, h);
                const double last = acs[IDX_DT(b, c, h, Q - 1)];
                for (int j = 0; j < Q; ++j) {
                    const int t = TOK(c, j);
                    if (t >= L) break;
                    const double w = exp(last - acs[IDX_DT(b, c, h, j)]) * dtc[IDX_DT(b, c, h, j)];
                    for (int p = 0; p < P; ++p) {
                        const double xw = XV(b, t, h, p) * w;
                        for (int n = 0; n < N; ++n) sp[(size_t)p * N + n] += xw * BV(b, t, g, n);
                    }
                }
            }

    /* step 4, state_passing: S_0 = h0, S_{c+1} = exp(Acs_c[Q-1]) S_c + s_c (sequential over c) */
#pragma omp parallel for collapse(2)
    for (int b = 0; b < Bn; ++b)
        for (int h = 0; h < H; ++h) {
            double* s0 = st + IDX_ST(b, 0, h);
            if (pr->h0)
                for (size_t e = 0; e < PN; ++e)
                    s0[e] = load_elem(pr->h0, pr->state_dtype, ((size_t)b * H + h) * PN + e);
            for (int c = 0; c < nc; ++c) {
                const double a = exp(acs[IDX_DT(b, c, h, Q - 1)]);
                const double* cur = st + IDX_ST(b, c, h);
                const double* loc = s + IDX_S(b, c, h);
                double* nxt = st + IDX_ST(b, c + 1, h);
                for (size_t e = 0; e < PN; ++e) nxt[e] = a * cur[e] + loc[e];
            }
        }

    /* step 5, chunk_scan: y_i = exp(Acs_i) C_i . S_c  +  sum_{j<=i} CB[i][j] exp(Acs_i - Acs_j) dt_j x_j
                           + D x_i */
    if (y) {
#pragma omp parallel for collapse(3)
        for (int b = 0; b < Bn; ++b)
            for (int c = 0; c < nc; ++c)
                for (int h = 0; h < H; ++h) {
                    const int g = h / hpg;
                    const double* Sc = st + IDX_ST(b, c, h);
                    const double Dh = pr->D ? (double)pr->D[h] : 0.0;
                    for (int i = 0; i < Q; ++i) {
                        const int ti = TOK(c, i);
                        if (ti >= L) break;
                        const double ai = acs[IDX_DT(b, c, h, i)];
                        for (int p = 0; p < P; ++p) {
                            double off = 0.0;
                            for (int n = 0; n < N; ++n) off += CV(b, ti, g, n) * Sc[(size_t)p * N + n];
                            double diag = 0.0;
                            for (int j = 0; j <= i; ++j) {
                                const int tj = TOK(c, j);
                                diag += cb[IDX_CB(b, c, g, i, j)] * exp(ai - acs[IDX_DT(b, c, h, j)]) *
                                        dtc[IDX_DT(b, c, h, j)] * XV(b, tj, h, p);
                            }
                            y[(((size_t)b * L + ti) * H + h) * P + p] = exp(ai) * off + diag + Dh * XV(b, ti, h, p);
                        }
                    }
                }
    }

    if (dt_out) memcpy(dt_out, dtc, (size_t)Bn * nc * H * Q * sizeof(double));
    if (acs_out) memcpy(acs_out, acs, (size_t)Bn * nc * H * Q * sizeof(double));
    if (cb_out) memcpy(cb_out, cb, (size_t)Bn * nc * G * Q * Q * sizeof(double));
    if (s_out) memcpy(s_out, s, (size_t)Bn * nc * H * PN * sizeof(double));
    if (st_out) memcpy(st_out, st, (size_t)Bn * (nc + 1) * H * PN * sizeof(double));
    if (final_state)
        for (int b = 0; b < Bn; ++b)
            for (int h = 0; h < H; ++h)
                memcpy(final_state + ((size_t)b * H + h) * PN, st + IDX_ST(b, nc, h), PN * sizeof(double));
    free(dtc); free(acs); free(cb); free(s); free(st);
    return 0;
#undef TOK
#undef IDX_DT
#undef IDX_CB
#undef IDX_S
#undef IDX_ST
#undef XV
#undef BV
#undef CV
}

int ssd_oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
