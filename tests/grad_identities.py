"""Identities between the gradients of attention that hold at any size.

Test infrastructure: the parity tests use these where the fp64 oracle cannot
compute every row (a key's gradient needs every query), and the oracle pins
check that the oracle satisfies them.

With P the softmax weights, W = P (times keep * s_keep under dropout) the
weights that form O = W V, and dS = P * (keep * s_keep * dP - D), D_i = dO_i . O_i
(the chain rule through the row softmax and O = W V):
  dQ_i = scale sum_j dS_ij k_j  and  dK_j = scale sum_i dS_ij q_i, so
      sum_i dQ_i q_i^T = sum_j k_j dK_j^T  (both scale sum_ij dS_ij k_j q_i^T);
  O_i = sum_j W_ij v_j  and  dV_j = sum_i W_ij dO_i, so
      sum_i O_i dO_i^T = sum_j v_j dV_j^T  (both sum_ij W_ij v_j dO_i^T);
  a live row of dS sums to zero (sum_j W_ij dP_ij = dO_i . O_i = D_i and
  sum_j P_ij = 1), so sum_j dK_j = 0.
A K/V head's sums over i run over every query head that uses it (query head
h reads K/V head h // G).  Rows that admit no key have O_i = dQ_i = 0 and
drop out of every sum.
"""
import numpy as np

__all__ = ["outer_identities", "identity_errors"]


def outer_identities(q, k, v, do, o, dq, dk, dv):
    """Both sides of the three identities per (batch, K/V head).

    q, do, o, dq: float64 [B, H, Nq, d]; k, v, dk, dv: float64 [B, Hkv, Nk, d].
    Returns {"dk": (K^T dK, dQ^T Q), "dv": (V^T dV, O^T dO), "dk_sum":
    (sum_j dK_j, sum_j |dK_j|)}, the matrices [B, Hkv, d, d], the sums
    [B, Hkv, d].
    """
    B, H, _, d = q.shape
    Hkv = k.shape[1]
    G = H // Hkv
    kdk = np.empty((B, Hkv, d, d))
    dqq = np.zeros((B, Hkv, d, d))
    vdv = np.empty((B, Hkv, d, d))
    odo = np.zeros((B, Hkv, d, d))
    for b in range(B):
        for hk in range(Hkv):
            kdk[b, hk] = k[b, hk].T @ dk[b, hk]
            vdv[b, hk] = v[b, hk].T @ dv[b, hk]
            for g in range(G):
                h = hk * G + g
                dqq[b, hk] += dq[b, h].T @ q[b, h]
                odo[b, hk] += o[b, h].T @ do[b, h]
    return {"dk": (kdk, dqq), "dv": (vdv, odo), "dk_sum": (dk.sum(axis=2), np.abs(dk).sum(axis=2))}


def identity_errors(q, k, v, do, o, dq, dk, dv):
    """Relative deviations: ||K^T dK - dQ^T Q|| / ||dQ^T Q||, the same for
    V^T dV against O^T dO (Frobenius, over all batches and K/V heads), and
    max |sum_j dK_j| / max sum_j |dK_j|."""
    r = outer_identities(q, k, v, do, o, dq, dk, dv)
    out = {}
    for name in ("dk", "dv"):
        left, right = r[name]
        out[name] = float(np.linalg.norm(left - right) / max(np.linalg.norm(right), 1e-300))
    s, a = r["dk_sum"]
    out["dk_sum"] = float(np.abs(s).max() / max(a.max(), 1e-300))
    return out
