"""Brute-force quadratic ("attention") form of the SSD prefill, numpy fp64.

TEST INFRASTRUCTURE ONLY: used by the test suite to check the recurrence oracle.

Source: "Mamba 硬件感知算法", section "结构化状态空间对偶性" (structured state space
duality): the SSM matrix splits into attention-like diagonal blocks and low-rank
off-diagonal blocks; taken over one block covering the whole sequence it is the
plain masked matrix

    y_i = sum_{j <= i} (C_i . B_j) * prod_{j < k <= i} a_k * dt_j * x_j
          + (prod_{k <= i} a_k) * (h0 C_i) + D x_i,        a_k = exp(dt_k A).

The decay between positions is formed as a running product of per-token factors
(not as a difference of cumulative sums), so this form shares no arithmetic
shortcut with the recurrence or the chunked oracle.  O(L^2) per head: tiny inputs.
"""
import numpy as np


def _softplus(z):
    # numpy's logaddexp(0, z) = log(1 + e^z), an independent library evaluation.
    return np.logaddexp(0.0, z)


def ssd_quadratic(x, dt, A, B, C, D=None, dt_bias=None, h0=None, dt_softplus=True):
    """All arguments are fp64 numpy arrays: x[Bt,L,H,P], dt[Bt,L,H], A[H],
    B/C[Bt,L,G,N], D[H], dt_bias[H], h0[Bt,H,P,N].  Returns (y, final_state)."""
    Bt, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    z = dt + (dt_bias[None, None, :] if dt_bias is not None else 0.0)
    d = _softplus(z) if dt_softplus else z                      # [Bt, L, H]
    y = np.zeros((Bt, L, H, P))
    fin = np.zeros((Bt, H, P, N))
    for b in range(Bt):
        for h in range(H):
            g = h // hpg
            a = np.exp(d[b, :, h] * A[h])                        # per-token decay factor
            # decay[i, j] = prod_{j < k <= i} a_k  (1 on the diagonal, 0 above it)
            decay = np.zeros((L, L))
            for j in range(L):
                run = 1.0
                decay[j, j] = 1.0
                for i in range(j + 1, L):
                    run *= a[i]
                    decay[i, j] = run
            M = (C[b, :, g, :] @ B[b, :, g, :].T) * decay * d[b, :, h][None, :]
            yb = M @ x[b, :, h, :]                               # [L, P]
            # initial-state contribution: (prod_{k <= i} a_k) * h0 C_i
            lead = np.cumprod(a)
            if h0 is not None:
                yb += lead[:, None] * (C[b, :, g, :] @ h0[b, h].T)
            if D is not None:
                yb += D[h] * x[b, :, h, :]
            y[b, :, h, :] = yb
            # final state: sum_j decay[L-1, j] dt_j x_j (outer) B_j + lead[L-1] h0
            w = decay[L - 1, :] * d[b, :, h]
            fin[b, h] = (x[b, :, h, :] * w[:, None]).T @ B[b, :, g, :]
            if h0 is not None:
                fin[b, h] += lead[L - 1] * h0[b, h]
    return y, fin
