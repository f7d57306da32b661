"""Seeded synthetic inputs, shared by the HIP path's tests/benchmark and the oracle.

This module only draws and shapes data: it holds none of the method's
arithmetic.  Both sides receive the same arrays.

Workloads are named by what they are.  Their shapes follow the pages'
models (Transformer-XL, Dai et al. 2019: the 12-layer enwik8 model of
section 4.1, the WikiText-103 attention lengths 384 in training and 1600 at
evaluation of section 4.1, the 10-head 16-layer word model of Appendix D);
the value distributions are synthetic stand-ins for activations and trained
weights, which are not available:

  hidden states and memory ~ N(0, 1); weights, u and v ~ N(0, sigma_w)

The relative encoding R is the fixed sinusoid table (section 3.3: no
learnable parameters), here R[p, 2c] = sin(p * 10000^(-2c/D)) and
R[p, 2c+1] = cos(p * 10000^(-2c/D)).  The pages give no formula; any fixed
table is a valid input, because R enters only through W_kR R and both sides
receive the same R.

Draw order with numpy.random.default_rng(seed), all fp32:
  1. for each layer n: W_q, W_kE, W_v, W_kR [H*d, D], then W_o [D, H*d]
  2. u, v [H, d]
  3. for each layer n: memory [B, M, D]  (the stream starts with a full memory)
  4. segment inputs h0 [S, B, L, D]
gamma = 1 and beta = 0.  bf16 workloads round every array once, to nearest even.
"""
from dataclasses import dataclass, replace

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int          # batch
    D: int          # d_model
    H: int          # n_head
    d: int          # d_head
    L: int          # segment length
    M: int          # memory capacity
    n_layers: int
    n_segments: int
    dtype: str      # "fp32" or "bf16"
    sigma_w: float  # std of the weights
    sigma_uv: float  # std of u and v
    R_rows: int     # rows of the sinusoid table (covers distances 0 .. M+L-1)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 32, 2, 16, 16, 16, 1, 1, "fp32",
                     1.0 / np.sqrt(32.0), 0.1, 32),
    "charlm": Workload("charlm", 22, 512, 8, 64, 512, 512, 12, 4, "bf16", 0.02, 0.02, 1024),
    "wordlm": Workload("wordlm", 60, 410, 10, 41, 150, 150, 16, 8, "bf16", 0.02, 0.02, 300),
    "large_eval": Workload("large_eval", 1, 1024, 16, 64, 128, 1600, 18, 16, "bf16",
                           0.02, 0.02, 1728),
    "large_train": Workload("large_train", 8, 1024, 16, 64, 384, 384, 18, 4, "bf16",
                            0.02, 0.02, 768),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    if overrides:
        w = replace(w, **overrides)
        if "R_rows" not in overrides:
            w = replace(w, R_rows=max(w.R_rows, w.M + w.L))
    return w


def sinusoid_table(rows: int, D: int) -> np.ndarray:
    """The fixed sinusoid table described in the module docstring, fp32 [rows, D]."""
    p = np.arange(rows, dtype=np.float64)[:, None]
    c = np.arange((D + 1) // 2, dtype=np.float64)[None, :]
    ang = p * np.power(10000.0, -2.0 * c / D)
    R = np.zeros((rows, D), dtype=np.float64)
    R[:, 0::2] = np.sin(ang)[:, : (D + 1) // 2]
    R[:, 1::2] = np.cos(ang)[:, : D // 2]
    return R.astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round an fp32 array to bf16 (nearest even) and return it as fp32."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(
        torch.bfloat16).to(torch.float32).numpy()


def make_inputs(w: Workload, seed: int = 0, layers=None, segments=None):
    """Draw every array of workload w in the fixed order.

    layers / segments override how many layers and segments are drawn
    (the draw order is unchanged, so a prefix of layers matches the full draw
    only for the weights).  Returns a dict of fp32 numpy arrays:
      weights: list of dicts (W_q, W_kE, W_v, W_kR, W_o, gamma, beta)
      u, v [H, d]; mem: list of [B, M, D]; h0 [S, B, L, D]; R [R_rows, D]
    """
    n_layers = w.n_layers if layers is None else layers
    n_seg = w.n_segments if segments is None else segments
    rng = np.random.default_rng(seed)
    HD = w.H * w.d

    def normal(shape, std):
        return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)

    weights = []
    for _ in range(n_layers):
        lw = {
            "W_q": normal((HD, w.D), w.sigma_w),
            "W_kE": normal((HD, w.D), w.sigma_w),
            "W_v": normal((HD, w.D), w.sigma_w),
            "W_kR": normal((HD, w.D), w.sigma_w),
            "W_o": normal((w.D, HD), w.sigma_w),
            "gamma": np.ones(w.D, dtype=np.float32),
            "beta": np.zeros(w.D, dtype=np.float32),
        }
        weights.append(lw)
    u = normal((w.H, w.d), w.sigma_uv)
    v = normal((w.H, w.d), w.sigma_uv)
    mem = [normal((w.B, w.M, w.D), 1.0) for _ in range(n_layers)]
    h0 = normal((n_seg, w.B, w.L, w.D), 1.0)
    R = sinusoid_table(w.R_rows, w.D)
    out = {"weights": weights, "u": u, "v": v, "mem": mem, "h0": h0, "R": R}
    if w.dtype == "bf16":
        out = _round_all(out)
    return out


def _round_all(x):
    if isinstance(x, dict):
        return {k: _round_all(v) for k, v in x.items()}
    if isinstance(x, list):
        return [_round_all(v) for v in x]
    return round_bf16(x)


def attention_inputs(B, H, L, mem_len, d, seed=0, sigma=1.0, sigma_uv=0.1,
                     r_rows=None, dtype="fp32"):
    """Seeded q, k, v, r, u, v for the attention entry point alone.

    q [B,L,H,d], k/v [B,T,H,d], r [r_rows,H,d], u/vb [H,d], with T = mem_len+L.
    Draw order: q, k, v, r, u, vb.
    """
    rng = np.random.default_rng(seed)
    T = mem_len + L
    r_rows = T if r_rows is None else r_rows

    def normal(shape, std):
        return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)

    out = {
        "q": normal((B, L, H, d), sigma),
        "k": normal((B, T, H, d), sigma),
        "v": normal((B, T, H, d), sigma),
        "r": normal((r_rows, H, d), sigma),
        "u": normal((H, d), sigma_uv),
        "vb": normal((H, d), sigma_uv),
    }
    if dtype == "bf16":
        out = _round_all(out)
    return out
