"""Backward pass of the relative-position memory attention and of one layer step
(test infrastructure only: the tests, the smoke check and the benchmark's CPU
baseline use it; nothing in the HIP library imports it).

Plain numpy in fp64, written from the definitions of the forward pass that the
C oracle computes (Transformer-XL, arXiv 1901.02860v3, section 3.3: the score
A^rel with its content and position terms and the global biases u and v;
section 3.2: the memory enters with its gradient stopped, so no gradient
flows into the cached hidden states; Appendix B: key j of query i sits at
distance mem_len + i - j).  The forward values come from the C oracle
(oracle.py); the backward is the chain rule through each forward step:

  s_ij = scale ((q_i + u) . k_j + (q_i + v) . r_{mem_len + i - j}),  j <= mem_len + i
  P_i  = softmax_j(s_i),  O_i = sum_j P_ij v_j

  dV_j  = sum_i P_ij G_i                    (G = dL/dO)
  dS_ij = P_ij (G_i . v_j - G_i . O_i)      (softmax backward)
  dq_i  = scale sum_j dS_ij (k_j + r_{mem_len + i - j})
  dk_j  = scale sum_i dS_ij (q_i + u)
  dr_p  = scale sum over pairs at distance p of dS_ij (q_i + v)
  du    = scale sum_ij dS_ij k_j,  dv = scale sum_ij dS_ij r_{mem_len + i - j}

The layer step (section 3.3, no feed-forward) adds the projections, the output
projection with its residual, and LayerNorm (biased variance), whose backward
is the usual one:  dy = (dyhat - mean(dyhat) - yhat mean(dyhat yhat)) / sigma.
"""
import numpy as np

from . import oracle as O


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _softmax_masked(scores):
    """Row softmax of scores [..., T] with -inf where masked (every row has a key)."""
    m = np.max(scores, axis=-1, keepdims=True)
    e = np.exp(scores - m)
    return e / np.sum(e, axis=-1, keepdims=True)


def rel_attn_bwd(q, k, v, r, u, vb, mem_len, dout, scale=None):
    """Gradients of rel_attn's output with respect to its inputs.

    q [B,L,H,d]; k, v [B,T,H,d]; r [>=T,H,d]; u, vb [H,d]; dout [B,L,H,d].
    Returns dict dq [B,L,H,d], dk, dv [B,T,H,d], dr [T,H,d], du, dvb [H,d].
    """
    q, k, v, r, u, vb, dout = map(_f64, (q, k, v, r, u, vb, dout))
    B, L, H, d = q.shape
    T = mem_len + L
    r = r[:T]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out, scores = O.rel_attn(q, k, v, r, u, vb, mem_len, scale=scale, want_scores=True)
    # scores are the scaled A^rel with -inf where masked; P is their softmax
    P = _softmax_masked(scores)                      # [B,H,L,T]
    i_idx = np.arange(L)[:, None]
    j_idx = np.arange(T)[None, :]
    dist = mem_len + i_idx - j_idx                   # [L,T]
    valid = j_idx <= mem_len + i_idx
    dist_c = np.where(valid, dist, 0)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    dr = np.zeros((T, H, d))
    du = np.zeros((H, d))
    dvb = np.zeros((H, d))
    for b in range(B):
        for h in range(H):
            G = dout[b, :, h, :]                     # [L,d]
            Pbh = P[b, h]                            # [L,T]
            V = v[b, :, h, :]
            K = k[b, :, h, :]
            Obh = out[b, :, h, :]
            dv[b, :, h, :] = Pbh.T @ G
            dP = G @ V.T                             # [L,T]
            dS = Pbh * (dP - np.sum(G * Obh, axis=1, keepdims=True))
            dS = np.where(valid, dS, 0.0)
            Rrel = r[dist_c, h, :]                   # [L,T,d]: r at each pair's distance
            dqc = scale * (dS @ K)
            dqp = scale * np.einsum("ij,ijc->ic", dS, Rrel)
            dq[b, :, h, :] = dqc + dqp
            du[h] += dqc.sum(axis=0)
            dvb[h] += dqp.sum(axis=0)
            dk[b, :, h, :] = scale * (dS.T @ (q[b, :, h, :] + u[h]))
            qp = q[b, :, h, :] + vb[h]               # [L,d]
            contrib = scale * dS[:, :, None] * qp[:, None, :]   # [L,T,d]
            np.add.at(dr[:, h, :], dist_c[valid], contrib[valid])
    return {"dq": dq, "dk": dk, "dv": dv, "dr": dr, "du": du, "dvb": dvb}


def layer_step_bwd(h, mem, W, u, vb, R, dh_out, eps=1e-5):
    """Gradients of one layer step (oracle.layer_step) for the upstream gradient
    dh_out [B,L,D].  The memory's gradient is stopped: mem gets none, while the
    weights still collect the memory rows' contributions.  Returns dict dh,
    dW_q, dW_kE, dW_v, dW_kR, dW_o, du, dvb, dgamma, dbeta."""
    h = _f64(h)
    B, L, D = h.shape
    u = _f64(u)
    H, d = u.shape
    mem = _f64(mem) if mem is not None else np.zeros((B, 0, D))
    mem_len = mem.shape[1]
    T = mem_len + L
    R = _f64(R)[:T]
    Wd = {n: _f64(W[n]) for n in ("W_q", "W_kE", "W_v", "W_kR", "W_o", "gamma", "beta")}
    dh_out = _f64(dh_out)
    _, inter = O.layer_step(h, mem, W, u, vb, R, eps=eps, want_intermediates=True)
    a2 = inter["a"].reshape(B * L, H * d)
    h2 = h.reshape(B * L, D)
    # LayerNorm over y = a W_o^T + h
    y = a2 @ Wd["W_o"].T + h2
    mu = y.mean(axis=1, keepdims=True)
    var = ((y - mu) ** 2).mean(axis=1, keepdims=True)
    sig = np.sqrt(var + eps)
    yhat = (y - mu) / sig
    g2 = dh_out.reshape(B * L, D)
    dgamma = np.sum(g2 * yhat, axis=0)
    dbeta = np.sum(g2, axis=0)
    dyhat = g2 * Wd["gamma"]
    dy = (dyhat - dyhat.mean(axis=1, keepdims=True)
          - yhat * np.mean(dyhat * yhat, axis=1, keepdims=True)) / sig
    dW_o = dy.T @ a2
    da = (dy @ Wd["W_o"]).reshape(B, L, H, d)
    dh = dy.copy()                                   # the residual path
    g = rel_attn_bwd(inter["q"], inter["k"], inter["v"], inter["r"], u, vb, mem_len, da)
    htil = np.concatenate([mem, h], axis=1).reshape(B * T, D)
    dq2 = g["dq"].reshape(B * L, H * d)
    dk2 = g["dk"].reshape(B * T, H * d)
    dv2 = g["dv"].reshape(B * T, H * d)
    dW_q = dq2.T @ h2
    dW_kE = dk2.T @ htil
    dW_v = dv2.T @ htil
    dW_kR = g["dr"].reshape(T, H * d).T @ R
    dh += dq2 @ Wd["W_q"]
    dkv = (dk2 @ Wd["W_kE"] + dv2 @ Wd["W_v"]).reshape(B, T, D)
    dh += dkv[:, mem_len:, :].reshape(B * L, D)       # current rows only (memory: stopped)
    return {"dh": dh.reshape(B, L, D), "dW_q": dW_q, "dW_kE": dW_kE, "dW_v": dW_v,
            "dW_kR": dW_kR, "dW_o": dW_o, "du": g["du"], "dvb": g["dvb"],
            "dgamma": dgamma, "dbeta": dbeta}
