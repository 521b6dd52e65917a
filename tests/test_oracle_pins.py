"""Pins for the fp64 oracle, each against something other than the oracle itself.

Sources: the recurrence h_t = exp(dt_t A) h_{t-1} + dt_t x_t (outer) B_t,
y_t = C_t h_t + D x_t ("Mamba-2状态空间模型的编译器优化与实现", section 1.1); the
chunk decomposition ("Mamba 硬件感知算法", section "块分解与状态传递"); the
quadratic / attention-like form ("Mamba 硬件感知算法", section "结构化状态空间对偶性");
the linear-attention special case ("Mamba-2炸裂升级！…", section "未来展望与应用拓展").
"""
import math

import numpy as np
import pytest
import torch

from mamba_ssd_prefill_amd.inputs import make_inputs

REL = 1e-12


def f64(t):
    """Independent widening through torch (not the oracle's decoder)."""
    return None if t is None else t.detach().to(torch.float64).numpy()


def rel_err(a, b):
    scale = max(np.max(np.abs(b)), 1e-300)
    return np.max(np.abs(a - b)) / scale


def small(seed=0, Bt=2, L=37, H=4, P=3, N=5, G=2, dtype="f32", h0=True, dt_scale=1.0, **kw):
    inp = make_inputs(Bt, L, H, P, N, G, dtype=dtype, state_dtype="f32", has_h0=h0, seed=seed, **kw)
    if dt_scale != 1.0:
        # push the per-head step sizes up so decays inside a chunk are substantial
        inp.dt_bias = inp.dt_bias + math.log(dt_scale)
    return inp


def quad(inp):
    return __import__("oracle").ssd_quadratic(
        f64(inp.x), f64(inp.dt), f64(inp.A), f64(inp.B), f64(inp.C), f64(inp.D), f64(inp.dt_bias),
        f64(inp.h0), inp.dt_softplus)


# ---------------------------------------------------------------------------------------------
def test_widening_matches_torch(oracle_mod):
    bits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
    for tdt in (torch.float16, torch.bfloat16):
        t = bits.view(tdt)
        got = oracle_mod.widen(t)
        ref = t.to(torch.float64).numpy()
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(got), nan)
        assert np.array_equal(got[~nan], ref[~nan])


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("softplus", [True, False])
def test_recurrence_matches_quadratic_form(oracle_mod, dtype, softplus):
    inp = small(seed=3, dtype=dtype, dt_scale=5.0)
    inp.dt_softplus = softplus
    if not softplus:  # keep dt positive and moderate without softplus
        inp.dt = (0.5 * inp.dt.float().abs()).to(inp.dt.dtype)
        inp.dt_bias = torch.full_like(inp.dt_bias, 0.05)
    y, fin = oracle_mod.recurrence_full(**inp.args())
    yq, finq = quad(inp)
    assert rel_err(y, yq) < REL
    assert rel_err(fin, finq) < REL


@pytest.mark.parametrize("Q", [1, 2, 3, 7, 8, 16, 64, 50])
def test_chunked_is_chunk_size_independent(oracle_mod, Q):
    inp = small(seed=5, L=50, dt_scale=3.0)
    y, fin = oracle_mod.recurrence_full(**inp.args())
    ch = oracle_mod.chunked(**inp.args(), chunk_size=Q)
    assert rel_err(ch["y"], y) < REL
    assert rel_err(ch["final"], fin) < REL


@pytest.mark.parametrize("Q", [4, 7, 16])
def test_chunk_entry_states_are_recurrence_states(oracle_mod, Q):
    inp = small(seed=6, L=45, dt_scale=2.0)
    Bt, L, H = inp.x.shape[:3]
    ch = oracle_mod.chunked(**inp.args(), chunk_size=Q)
    _, _, snaps = oracle_mod.recurrence(**inp.args(), snap_q=Q)
    nc = (L + Q - 1) // Q
    st = ch["states"]  # [B, nc+1, H, P, N]; slot c+1 = state after chunk c
    for k, (b, h) in enumerate([(b, h) for b in range(Bt) for h in range(H)]):
        for c in range(nc):
            assert rel_err(st[b, c + 1, h], snaps[k, c]) < REL
        assert rel_err(st[b, 0, h], f64(inp.h0)[b, h]) == 0.0


def test_local_chunk_state_is_zero_start_recurrence(oracle_mod):
    """s_c is the state a chunk reaches when the recurrence restarts from zero at its start."""
    Q = 8
    inp = small(seed=7, L=29, dt_scale=2.0)
    Bt, L, H = inp.x.shape[:3]
    ch = oracle_mod.chunked(**inp.args(), chunk_size=Q)
    for c in range((L + Q - 1) // Q):
        sl = slice(c * Q, min(L, (c + 1) * Q))
        part = dict(inp.args())
        for k in ("x", "dt", "B", "C"):
            part[k] = part[k][:, sl].contiguous()
        part["h0"] = None
        _, fin, _ = oracle_mod.recurrence(**part)
        fin = fin.reshape(Bt, H, *fin.shape[1:])
        assert rel_err(ch["s"][:, c], fin) < REL


def test_cumsum_and_bmm_steps_match_library_routines(oracle_mod):
    Q = 8
    inp = small(seed=8, L=30, dt_scale=2.0)
    Bt, L, H = inp.x.shape[:3]
    G = inp.B.shape[2]
    ch = oracle_mod.chunked(**inp.args(), chunk_size=Q)
    nc = (L + Q - 1) // Q
    pad = nc * Q - L
    z = f64(inp.dt) + f64(inp.dt_bias)[None, None, :]
    d = np.logaddexp(0.0, z)
    d = np.concatenate([d, np.zeros((Bt, pad, H))], axis=1).reshape(Bt, nc, Q, H).transpose(0, 1, 3, 2)
    assert rel_err(ch["dt"], d) < REL
    acs = np.cumsum(d * f64(inp.A)[None, None, :, None], axis=-1)
    assert rel_err(ch["acs"], acs) < REL
    Bp = np.concatenate([f64(inp.B), np.zeros((Bt, pad, G, inp.B.shape[3]))], axis=1)
    Cp = np.concatenate([f64(inp.C), np.zeros((Bt, pad, G, inp.C.shape[3]))], axis=1)
    for b in range(Bt):
        for c in range(nc):
            for g in range(G):
                ref = Cp[b, c * Q:(c + 1) * Q, g] @ Bp[b, c * Q:(c + 1) * Q, g].T
                assert np.max(np.abs(ch["cb"][b, c, g] - ref)) < 1e-14


def test_decay_only_closed_form(oracle_mod):
    """x = 0, h0 != 0: final = exp(A sum dt) h0 and y_t = exp(A sum_{k<=t} dt_k) (h0 C_t)."""
    inp = small(seed=9, dt_scale=4.0)
    inp.x = torch.zeros_like(inp.x)
    y, fin = oracle_mod.recurrence_full(**inp.args())
    d = np.logaddexp(0.0, f64(inp.dt) + f64(inp.dt_bias)[None, None, :])  # [B, L, H]
    A = f64(inp.A)
    cum = np.cumsum(d, axis=1) * A[None, None, :]
    h0 = f64(inp.h0)
    G = inp.B.shape[2]
    H = inp.x.shape[2]
    Cg = np.repeat(f64(inp.C), H // G, axis=2)  # [B, L, H, N]
    yref = np.exp(cum)[..., None] * np.einsum("bhpn,blhn->blhp", h0, Cg)
    finref = np.exp(cum[:, -1])[..., None, None] * h0
    assert rel_err(y, yref) < REL
    assert rel_err(fin, finref) < REL


def test_zero_step_leaves_state_unchanged(oracle_mod):
    """dt = 0 (no softplus, zero bias): final = h0 and y_t = h0 C_t + D x_t."""
    inp = small(seed=10)
    inp.dt = torch.zeros_like(inp.dt)
    inp.dt_bias = torch.zeros_like(inp.dt_bias)
    inp.dt_softplus = False
    y, fin = oracle_mod.recurrence_full(**inp.args())
    H, G = inp.x.shape[2], inp.B.shape[2]
    Cg = np.repeat(f64(inp.C), H // G, axis=2)
    yref = np.einsum("bhpn,blhn->blhp", f64(inp.h0), Cg) + f64(inp.D)[None, None, :, None] * f64(inp.x)
    assert np.array_equal(fin, f64(inp.h0))
    assert rel_err(y, yref) < REL


def test_zero_input_gives_exact_zero(oracle_mod):
    inp = small(seed=11, h0=False)
    inp.x = torch.zeros_like(inp.x)
    y, fin = oracle_mod.recurrence_full(**inp.args())
    assert np.all(y == 0.0) and np.all(fin == 0.0)
    ch = oracle_mod.chunked(**inp.args(), chunk_size=8)
    assert np.all(ch["y"] == 0.0) and np.all(ch["final"] == 0.0)


def test_geometric_series(oracle_mod):
    """Constant x, B, C, dt and h0 = 0: S_t = dt x (outer) B (1 - a^t) / (1 - a), a = exp(dt A)."""
    Bt, L, H, P, N = 1, 40, 2, 3, 4
    x = torch.randn(1, 1, H, P, generator=torch.Generator().manual_seed(1)).expand(Bt, L, H, P).contiguous()
    Bm = torch.randn(1, 1, 1, N, generator=torch.Generator().manual_seed(2)).expand(Bt, L, 1, N).contiguous()
    Cm = torch.randn(1, 1, 1, N, generator=torch.Generator().manual_seed(3)).expand(Bt, L, 1, N).contiguous()
    dt = torch.full((Bt, L, H), 0.3)
    A = torch.tensor([-0.7, -2.5])
    D = torch.tensor([0.5, -1.5])
    y, fin = oracle_mod.recurrence_full(x, dt, A, Bm, Cm, D=D, dt_softplus=False)
    dv = float(dt[0, 0, 0])  # the fp32 value actually stored
    for h in range(H):
        a = math.exp(dv * float(A[h]))
        outer = dv * np.outer(f64(x)[0, 0, h], f64(Bm)[0, 0, 0])
        for t in range(1, L + 1):
            S = outer * (1 - a ** t) / (1 - a)
            yt = S @ f64(Cm)[0, 0, 0] + float(D[h]) * f64(x)[0, 0, h]
            assert rel_err(y[0, t - 1, h], yt) < 1e-11
        assert rel_err(fin[0, h], outer * (1 - a ** L) / (1 - a)) < 1e-11


def test_linear_attention_special_case(oracle_mod):
    """No decay (A = 0) and dt = 1: y = tril(C B^T) x + D x, causal linear attention."""
    inp = small(seed=12, h0=False, G=1, H=3)
    inp.A = torch.zeros_like(inp.A)
    inp.dt = torch.ones_like(inp.dt)
    inp.dt_bias = torch.zeros_like(inp.dt_bias)
    inp.dt_softplus = False
    y, fin = oracle_mod.recurrence_full(**inp.args())
    X, Bm, Cm = f64(inp.x), f64(inp.B), f64(inp.C)
    for b in range(X.shape[0]):
        M = np.tril(Cm[b, :, 0] @ Bm[b, :, 0].T)
        for h in range(X.shape[2]):
            ref = M @ X[b, :, h] + float(inp.D[h]) * X[b, :, h]
            assert rel_err(y[b, :, h], ref) < REL
            assert rel_err(fin[b, h], X[b, :, h].T @ Bm[b, :, 0]) < REL


def test_linear_in_x_and_initial_state(oracle_mod):
    """y and the final state are jointly linear in (x, h0).  Integer-valued x and h0 keep the
    mixed inputs exactly representable, so the check is at fp64 rounding level."""
    base = small(seed=13, dt_scale=2.0)
    gen = torch.Generator().manual_seed(99)
    ints = lambda t: torch.randint(-8, 9, t.shape, generator=gen).float()  # noqa: E731
    x1, x2, h1, h2 = ints(base.x), ints(base.x), ints(base.h0), ints(base.h0)
    al, be = 3.0, -2.0

    def run(x, h0):
        a = dict(base.args())
        a["x"], a["h0"] = x, h0
        return oracle_mod.recurrence_full(**a)

    y1, f1 = run(x1, h1)
    y2, f2 = run(x2, h2)
    ym, fm = run(al * x1 + be * x2, al * h1 + be * h2)
    assert rel_err(ym, al * y1 + be * y2) < 1e-11
    assert rel_err(fm, al * f1 + be * f2) < 1e-11


def test_state_carry_equals_one_run(oracle_mod):
    inp = small(seed=15, L=48, dt_scale=2.0)
    L1 = 19
    y, fin = oracle_mod.recurrence_full(**inp.args())
    first = dict(inp.args())
    second = dict(inp.args())
    for k in ("x", "dt", "B", "C"):
        first[k] = first[k][:, :L1].contiguous()
        second[k] = second[k][:, L1:].contiguous()
    y1, f1 = oracle_mod.recurrence_full(**first)
    # the carried state enters as fp32 (the state dtype): its rounding (2^-24 relative)
    # bounds the difference, far below any error a wrong carry would make
    second["h0"] = torch.from_numpy(f1).float()
    y2, f2 = oracle_mod.recurrence_full(**second)
    assert rel_err(y1, y[:, :L1]) == 0.0
    assert rel_err(y2, y[:, L1:]) < 1e-6
    assert rel_err(f2, fin) < 1e-6


def test_grouped_bc_equals_replicated_per_head(oracle_mod):
    inp = small(seed=16, H=6, G=3, dt_scale=2.0)
    y, fin = oracle_mod.recurrence_full(**inp.args())
    rep = dict(inp.args())
    rep["B"] = inp.B.repeat_interleave(2, dim=2).contiguous()
    rep["C"] = inp.C.repeat_interleave(2, dim=2).contiguous()
    yr, fr = oracle_mod.recurrence_full(**rep)
    assert np.array_equal(y, yr) and np.array_equal(fin, fr)


def test_batch_rows_are_independent(oracle_mod):
    inp = small(seed=17, Bt=3, dt_scale=2.0)
    y, fin = oracle_mod.recurrence_full(**inp.args())
    perm = [2, 0, 1]
    pa = dict(inp.args())
    for k in ("x", "dt", "B", "C", "h0"):
        pa[k] = pa[k][perm].contiguous()
    yp, fp = oracle_mod.recurrence_full(**pa)
    assert np.array_equal(yp, y[perm]) and np.array_equal(fp, fin[perm])


def test_single_token_by_hand(oracle_mod):
    """L = 1: y = dt (B.C) x + exp(dt A) (h0 C) + D x, final = exp(dt A) h0 + dt x (outer) B."""
    inp = small(seed=18, Bt=1, L=1, H=2, G=1, dt_scale=3.0)
    y, fin = oracle_mod.recurrence_full(**inp.args())
    d = np.logaddexp(0.0, f64(inp.dt)[0, 0] + f64(inp.dt_bias))
    for h in range(2):
        a = math.exp(d[h] * float(inp.A[h]))
        xv, Bv, Cv, h0 = f64(inp.x)[0, 0, h], f64(inp.B)[0, 0, 0], f64(inp.C)[0, 0, 0], f64(inp.h0)[0, h]
        yref = d[h] * float(Bv @ Cv) * xv + a * (h0 @ Cv) + float(inp.D[h]) * xv
        fref = a * h0 + d[h] * np.outer(xv, Bv)
        assert rel_err(y[0, 0, h], yref) < REL
        assert rel_err(fin[0, h], fref) < REL


def test_sampled_pairs_match_full_run(oracle_mod):
    inp = small(seed=19, Bt=2, H=4)
    y, fin = oracle_mod.recurrence_full(**inp.args())
    ys, fs, _ = oracle_mod.recurrence(**inp.args(), bh=[(1, 3), (0, 2)])
    assert np.array_equal(ys[0], y[1, :, 3]) and np.array_equal(ys[1], y[0, :, 2])
    assert np.array_equal(fs[0], fin[1, 3]) and np.array_equal(fs[1], fin[0, 2])


def test_golden_hand_example(oracle_mod):
    """The fixture in tests/golden/hand_example.json is worked out by hand from the recurrence."""
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "hand_example.json")
    with open(path) as f:
        g = json.load(f)
    t = lambda k: torch.tensor(g[k], dtype=torch.float32)  # noqa: E731
    y, fin = oracle_mod.recurrence_full(t("x"), t("dt"), t("A"), t("B"), t("C"), D=t("D"),
                                        dt_softplus=False)
    assert np.allclose(y, np.array(g["y"]), rtol=0, atol=1e-12)
    assert np.allclose(fin, np.array(g["final"]), rtol=0, atol=1e-12)


def test_decode_steps_continue_a_prefill(oracle_mod):
    """The decode step ("Mamba-2状态空间模型的编译器优化与实现", section 2.1): k single-token
    steps from a prefix's final state reproduce the last k tokens of one long run."""
    inp = small(seed=20, Bt=2, L=29, H=4, G=2, dt_scale=2.0)
    y, fin = oracle_mod.recurrence_full(**inp.args())
    L0 = 25
    pre = dict(inp.args())
    for k in ("x", "dt", "B", "C"):
        pre[k] = pre[k][:, :L0].contiguous()
    _, state = oracle_mod.recurrence_full(**pre)
    for t in range(L0, 29):
        # the state enters as fp32 (its storage dtype): 2^-24 relative per step
        yt, state = oracle_mod.decode_step(inp.x[:, t].contiguous(), inp.dt[:, t].contiguous(), inp.A,
                                           inp.B[:, t].contiguous(), inp.C[:, t].contiguous(), inp.D, inp.dt_bias,
                                           torch.from_numpy(state).float(), inp.dt_softplus)
        assert yt.shape == (2, 4, 3)
        assert rel_err(yt, y[:, t]) < 1e-6
    assert rel_err(state, fin) < 1e-6


def test_decode_step_by_hand(oracle_mod):
    """One decode step for one (b, h), written out: S' = exp(dt A) S + dt x (outer) B,
    y = S' C + D x, with dt = softplus(dt_raw + dt_bias) and group g = h / (H / G)."""
    inp = small(seed=21, Bt=2, L=1, H=4, G=2, dt_scale=3.0)
    x, dt, Bm, Cm = inp.x[:, 0], inp.dt[:, 0], inp.B[:, 0], inp.C[:, 0]
    y, S = oracle_mod.decode_step(x, dt, inp.A, Bm, Cm, inp.D, inp.dt_bias, inp.h0, True)
    b, h = 1, 3
    g = h // 2
    d = math.log1p(math.exp(float(dt[b, h]) + float(inp.dt_bias[h])))
    a = math.exp(d * float(inp.A[h]))
    Sref = a * f64(inp.h0)[b, h] + d * np.outer(f64(x)[b, h], f64(Bm)[b, g])
    yref = Sref @ f64(Cm)[b, g] + float(inp.D[h]) * f64(x)[b, h]
    assert rel_err(S[b, h], Sref) < REL
    assert rel_err(y[b, h], yref) < REL


def _masked_quadratic(inp, seq):
    """Packed sequences in the SSD "attention" form ("Mamba 硬件感知算法", section
    "结构化状态空间对偶性"), with the mask of "Mamba-2炸裂升级！…", section "与vLLM的深度融合":
    y_i = sum_{j <= i, same sequence} (C_i . B_j) exp(sum_{j < k <= i} dA_k) dt_j x_j + D x_i
          + [i in the row's first sequence] exp(sum_{k <= i} dA_k) (h0 C_i);
    the final state is the same sum over the last sequence (plus the decayed h0 when the row
    holds one sequence).  Plain numpy, O(L^2) per (b, h)."""
    x, dtr, A, Bm, Cm, D, bias, h0 = (f64(t) for t in (inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.dt_bias, inp.h0))
    Bt, L, H, P = x.shape
    G, N = Bm.shape[2], Bm.shape[3]
    y = np.zeros((Bt, L, H, P))
    fin = np.zeros((Bt, H, P, N))
    for b in range(Bt):
        first = seq[b] == seq[b, 0]
        for h in range(H):
            g = h // (H // G)
            d = np.logaddexp(0.0, dtr[b, :, h] + bias[h])
            cum = np.concatenate([[0.0], np.cumsum(d * A[h])])  # cum[t + 1] = sum_{k <= t} dA_k
            for i in range(L):
                acc = D[h] * x[b, i, h]
                for j in range(i + 1):
                    if seq[b, j] == seq[b, i] and np.all(seq[b, j:i + 1] == seq[b, i]):
                        acc = acc + (Cm[b, i, g] @ Bm[b, j, g]) * np.exp(cum[i + 1] - cum[j + 1]) * d[j] * x[b, j, h]
                if first[i] and np.all(seq[b, :i + 1] == seq[b, 0]):
                    acc = acc + np.exp(cum[i + 1]) * (h0[b, h] @ Cm[b, i, g])
                y[b, i, h] = acc
            last = L - 1
            for j in range(L):
                if np.all(seq[b, j:] == seq[b, last]):
                    fin[b, h] += np.exp(cum[L] - cum[j + 1]) * d[j] * np.outer(x[b, j, h], Bm[b, j, g])
            if np.all(seq[b] == seq[b, 0]):
                fin[b, h] += np.exp(cum[L]) * h0[b, h]
    return y, fin


def test_varlen_matches_masked_quadratic_form(oracle_mod):
    inp = small(seed=22, Bt=2, L=30, H=4, P=3, N=5, G=2, dt_scale=2.0)
    seq = np.array([[0] * 7 + [1] * 1 + [2] * 12 + [3] * 10,
                    [5] * 30], dtype=np.int32)
    y, fin = oracle_mod.recurrence_varlen(**inp.args(), seq_idx=seq)
    yq, fq = _masked_quadratic(inp, seq)
    assert rel_err(y, yq) < REL
    assert rel_err(fin, fq) < REL
    # a row holding one sequence is the plain recurrence
    y1, f1 = oracle_mod.recurrence_full(**inp.args())
    assert np.array_equal(y[1], y1[1]) and np.array_equal(fin[1], f1[1])


def test_varlen_ids_only_matter_where_they_change(oracle_mod):
    inp = small(seed=23, Bt=1, L=24, H=2, G=1)
    a = np.array([[3] * 5 + [9] * 11 + [3] * 8], dtype=np.int32)
    b = np.array([[0] * 5 + [1] * 11 + [2] * 8], dtype=np.int32)
    ya, fa = oracle_mod.recurrence_varlen(**inp.args(), seq_idx=a)
    yb, fb = oracle_mod.recurrence_varlen(**inp.args(), seq_idx=b)
    assert np.array_equal(ya, yb) and np.array_equal(fa, fb)


def test_varlen_states_match_closed_form_sums(oracle_mod):
    """Per-sequence initial and final states, against the sums written out in numpy: for
    sequence q = tokens [s, e] of a row, with h0 = initial_states[q],
      y_i     = sum_{s <= j <= i} (C_i . B_j) exp(sum_{j < k <= i} dA_k) dt_j x_j
                + exp(sum_{s <= k <= i} dA_k) (h0 C_i) + D x_i,
      final_q = sum_{s <= j <= e} exp(sum_{j < k <= e} dA_k) dt_j x_j (outer) B_j
                + exp(sum_{s <= k <= e} dA_k) h0.
    A row's first token starts a sequence too, so no state crosses rows."""
    import torch
    inp = small(seed=24, Bt=2, L=26, H=4, P=3, N=5, G=2, dt_scale=2.0)
    seq = np.array([[4] * 6 + [0] * 1 + [2] * 9 + [1] * 10,
                    [3] * 11 + [5] * 15], dtype=np.int32)
    nseq = 7  # number 6 labels no run
    g0 = torch.Generator().manual_seed(5)
    h0s = 0.3 * torch.randn(nseq, 4, 3, 5, generator=g0, dtype=torch.float64).float()
    args = {k: v for k, v in inp.args().items() if k != "h0"}
    y, fin = oracle_mod.recurrence_varlen_states(**args, seq_idx=seq, nseq=nseq, initial_states=h0s)
    x, dtr, A, Bm, Cm, D, bias = (f64(t) for t in (inp.x, inp.dt, inp.A, inp.B, inp.C, inp.D, inp.dt_bias))
    H0 = h0s.double().numpy()
    L, H = 26, 4
    yref = np.zeros_like(y)
    fref = np.full_like(fin, np.nan)
    for b in range(2):
        runs, t = [], 0
        while t < L:
            e = t
            while e + 1 < L and seq[b, e + 1] == seq[b, t]:
                e += 1
            runs.append((t, e))
            t = e + 1
        for h in range(H):
            g = h // 2
            d = np.logaddexp(0.0, dtr[b, :, h] + bias[h])
            cum = np.concatenate([[0.0], np.cumsum(d * A[h])])
            for (s0, e0) in runs:
                q = seq[b, s0]
                for i in range(s0, e0 + 1):
                    acc = D[h] * x[b, i, h] + np.exp(cum[i + 1] - cum[s0]) * (H0[q, h] @ Cm[b, i, g])
                    for j in range(s0, i + 1):
                        acc = acc + (Cm[b, i, g] @ Bm[b, j, g]) * np.exp(cum[i + 1] - cum[j + 1]) * d[j] * x[b, j, h]
                    yref[b, i, h] = acc
                F = np.exp(cum[e0 + 1] - cum[s0]) * H0[q, h]
                for j in range(s0, e0 + 1):
                    F = F + np.exp(cum[e0 + 1] - cum[j + 1]) * d[j] * np.outer(x[b, j, h], Bm[b, j, g])
                fref[q, h] = F
    assert rel_err(y, yref) < REL
    assert np.all(np.isnan(fin[6])) and np.all(np.isnan(fref[6]))
    assert rel_err(fin[:6], fref[:6]) < REL


# ---- the convolution before and the norm after the SSD ("Mamba-2炸裂升级！…", section
# "未来展望与应用拓展"; the depthwise convolution of section "Mamba-2核心操作与融合的必要性") ----

def _silu(v):
    return v / (1.0 + np.exp(-v))


def test_conv_silu_equals_numpy_convolve_per_channel(oracle_mod):
    gen = torch.Generator().manual_seed(71)
    Bt, L, Ch, K = 2, 13, 6, 4
    x = torch.randn(Bt, L, Ch, generator=gen)
    w = torch.randn(Ch, K, generator=gen)
    bias = torch.randn(Ch, generator=gen)
    st = torch.randn(Bt, Ch, K - 1, generator=gen)
    out = oracle_mod.conv_silu(x, w, bias, st)
    X, W, Bv, S = (t.double().numpy() for t in (x, w, bias, st))
    for b in range(Bt):
        for ch in range(Ch):
            seq = np.concatenate([S[b, ch], X[b, :, ch]])
            # numpy's convolve flips its second argument: correlation with the taps = convolve
            # with the reversed taps; 'valid' keeps the L outputs that see K inputs
            v = np.convolve(seq, W[ch, ::-1], mode="valid") + Bv[ch]
            assert np.allclose(out[b, :, ch], _silu(v), rtol=1e-13, atol=1e-13)


def test_conv_impulse_response_and_zero_state(oracle_mod):
    Ch, K, L = 3, 4, 9
    w = torch.arange(1.0, Ch * K + 1).reshape(Ch, K) / 10
    x = torch.zeros(1, L, Ch)
    x[0, 2, :] = 1.0
    out = oracle_mod.conv_silu(x, w)
    for ch in range(Ch):
        for t in range(L):
            k = t - 2  # the impulse at token 2 reaches token t through tap K-1-k
            v = float(w[ch, K - 1 - k]) if 0 <= k < K else 0.0
            assert out[0, t, ch] == pytest.approx(_silu(v), abs=1e-15)


def test_conv_state_carries_across_a_split(oracle_mod):
    gen = torch.Generator().manual_seed(72)
    Bt, L, Ch, K = 2, 20, 5, 4
    x = torch.randn(Bt, L, Ch, generator=gen)
    w = torch.randn(Ch, K, generator=gen)
    bias = torch.randn(Ch, generator=gen)
    whole = oracle_mod.conv_silu(x, w, bias)
    s = 7
    tail = x[:, s - (K - 1):s, :].permute(0, 2, 1).contiguous()  # [B, Ch, K-1]: the state after token s-1
    second = oracle_mod.conv_silu(x[:, s:], w, bias, tail)
    assert np.allclose(second, whole[:, s:], rtol=1e-14, atol=1e-14)


def test_gated_rmsnorm_against_torch_rms_norm(oracle_mod):
    gen = torch.Generator().manual_seed(73)
    Bt, L, C, G = 2, 5, 24, 3
    y = torch.randn(Bt, L, C, generator=gen, dtype=torch.float64)
    z = torch.randn(Bt, L, C, generator=gen, dtype=torch.float64)
    w = torch.randn(C, generator=gen, dtype=torch.float64)
    eps = 1e-5
    out = oracle_mod.gated_rmsnorm(y, z, w, eps, G)
    g = (y * torch.nn.functional.silu(z)).reshape(Bt, L, G, C // G)
    ref = torch.nn.functional.rms_norm(g, (C // G,), None, eps).reshape(Bt, L, C) * w
    assert np.allclose(out, ref.numpy(), rtol=1e-12, atol=1e-12)


def test_gated_rmsnorm_closed_forms(oracle_mod):
    gen = torch.Generator().manual_seed(74)
    Bt, L, C, G = 1, 4, 16, 2
    y = torch.randn(Bt, L, C, generator=gen, dtype=torch.float64)
    z = torch.randn(Bt, L, C, generator=gen, dtype=torch.float64)
    ones = torch.ones(C, dtype=torch.float64)
    eps = 1e-3
    out = oracle_mod.gated_rmsnorm(y, z, ones, eps, G).reshape(Bt, L, G, C // G)
    g = (y.numpy() * _silu(z.numpy())).reshape(Bt, L, G, C // G)
    ms = np.mean(g * g, axis=3)
    # the mean square of the output of a group is ms / (ms + eps)
    assert np.allclose(np.mean(out * out, axis=3), ms / (ms + eps), rtol=1e-12)
    # without eps the result does not depend on the scale of y
    a = oracle_mod.gated_rmsnorm(y, z, ones, 0.0, G)
    b = oracle_mod.gated_rmsnorm(3.5 * y, z, ones, 0.0, G)
    assert np.allclose(a, b, rtol=1e-12, atol=1e-12)
    # a zero gate gives zero
    assert np.all(oracle_mod.gated_rmsnorm(y, torch.zeros_like(z), ones, eps, G) == 0.0)


def test_block_carries_conv_and_ssm_state_across_a_split(oracle_mod):
    """One call over L tokens = a call over the first s tokens, then a call over the rest with the
    first call's last K-1 raw inputs as the conv state and its final state as h0."""
    H, P, G, N, K = 4, 8, 2, 8, 4
    Bt, L, s = 2, 30, 11
    gen = torch.Generator().manual_seed(75)
    Ch = H * P + 2 * G * N
    xbc = torch.randn(Bt, L, Ch, generator=gen).to(torch.bfloat16)
    w = (0.5 * torch.randn(Ch, K, generator=gen))
    cb = 0.1 * torch.randn(Ch, generator=gen)
    inp = make_inputs(Bt, L, H, P, N, G, dtype="bf16", state_dtype="f32", has_h0=True, seed=76)
    z = torch.randn(Bt, L, H * P, generator=gen).to(torch.bfloat16)
    nw = 1.0 + 0.1 * torch.randn(H * P, generator=gen)
    kw = dict(nheads=H, headdim=P, ngroups=G, dstate=N, in_dtype="bf16")
    out, y, fin = oracle_mod.block(xbc, w, cb, None, inp.dt, inp.A, inp.D, inp.dt_bias, z, nw, 1e-5, h0=inp.h0, **kw)
    o1, y1, f1 = oracle_mod.block(xbc[:, :s], w, cb, None, inp.dt[:, :s], inp.A, inp.D, inp.dt_bias, z[:, :s], nw, 1e-5,
                              h0=inp.h0, **kw)
    st = xbc[:, s - (K - 1):s].permute(0, 2, 1).contiguous()
    o2, y2, f2 = oracle_mod.block(xbc[:, s:].contiguous(), w, cb, st, inp.dt[:, s:].contiguous(), inp.A, inp.D, inp.dt_bias,
                              z[:, s:].contiguous(), nw, 1e-5, h0=torch.from_numpy(f1).float(), **kw)
    assert rel_err(np.concatenate([y1, y2], axis=1), y) < 1e-6
    assert rel_err(np.concatenate([o1, o2], axis=1), out) < 1e-6
    assert rel_err(f2, fin) < 1e-6


def test_block_channel_layout_x_then_b_then_c(oracle_mod):
    """xBC = [x | B | C] along channels: with the B channels' inputs and bias zero, B = silu(0) = 0,
    so nothing enters the state (final state 0, y = D x); with the C channels zero instead, y is
    still D x but the state fills."""
    H, P, G, N, K = 2, 8, 1, 8, 4
    Bt, L = 1, 12
    HP, GN = H * P, G * N
    gen = torch.Generator().manual_seed(77)
    xbc = torch.randn(Bt, L, HP + 2 * GN, generator=gen)
    w = 0.5 * torch.randn(HP + 2 * GN, K, generator=gen)
    cb = 0.1 * torch.randn(HP + 2 * GN, generator=gen)
    inp = make_inputs(Bt, L, H, P, N, G, dtype="f32", state_dtype="f32", has_h0=False, seed=78)
    z = torch.randn(Bt, L, HP, generator=gen)
    nw = torch.ones(HP)
    kw = dict(nheads=H, headdim=P, ngroups=G, dstate=N, in_dtype="f32")
    xconv = oracle_mod.conv_silu(xbc, w, cb)[..., :HP].astype(np.float32).astype(np.float64)
    dx = inp.D.double().numpy()[None, None, :, None] * xconv.reshape(Bt, L, H, P)
    for part, state_fills in ((slice(HP, HP + GN), False), (slice(HP + GN, HP + 2 * GN), True)):
        xb, c2 = xbc.clone(), cb.clone()
        xb[..., part] = 0.0
        c2[part] = 0.0
        out, y, fin = oracle_mod.block(xb, w, c2, None, inp.dt, inp.A, inp.D, inp.dt_bias, z, nw, 1e-5, **kw)
        assert np.allclose(y, dx, rtol=1e-12, atol=1e-12)
        assert (np.max(np.abs(fin)) > 1e-3) == state_fills
