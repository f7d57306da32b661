"""Python face of the CPU oracle (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this module.  It loads oracle/liboracle.so (plain C, fp64; see txl_oracle.c)
and converts numpy arrays to contiguous float64 before every call.  It shares
no code with the HIP library and imports nothing from it.

Transformer-XL (Dai et al., arXiv 1901.02860v3): section 3.2 (memory),
section 3.3 (relative score A^rel and the N-layer procedure), Appendix B
(distance range and the distance of key j for query i).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None
_LIB_PATH = _build.LIB
_i64 = ctypes.c_int64
_dbl = ctypes.c_double
_p = ctypes.c_void_p


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            _build.build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.txo_rel_attn.argtypes = [_i64] * 5 + [_p] * 6 + [_dbl, _p, _p]
        lib.txo_rel_attn.restype = None
        lib.txo_linear.argtypes = [_i64] * 3 + [_p] * 3
        lib.txo_linear.restype = None
        lib.txo_layer_norm.argtypes = [_i64, _i64, _p, _p, _p, _dbl, _p]
        lib.txo_layer_norm.restype = None
        lib.txo_layer_step.argtypes = [_i64] * 6 + [_dbl] + [_p] * 18
        lib.txo_layer_step.restype = ctypes.c_int
        lib.txo_layer_step_rows.argtypes = ([_i64] * 6 + [_dbl] + [_p] * 12
                                            + [_i64, _p, _p, _p])
        lib.txo_layer_step_rows.restype = ctypes.c_int
        lib.txo_mem_update.argtypes = [_i64] * 3 + [_p, _i64, _p, _i64, _p]
        lib.txo_mem_update.restype = _i64
        lib.txo_pos_ff.argtypes = [_i64] * 3 + [_p] * 7 + [_dbl, _p]
        lib.txo_pos_ff.restype = ctypes.c_int
        lib.txo_num_threads.argtypes = []
        lib.txo_num_threads.restype = ctypes.c_int
        lib.txo_set_num_threads.argtypes = [ctypes.c_int]
        lib.txo_set_num_threads.restype = None
        _LIB = lib
    return _LIB


def use_native_build() -> str:
    """Switch this process to the oracle compiled with -march=native for the
    host it runs on (built now, before the first call); returns its flags.
    Only the benchmark's CPU-baseline leg does this; results are the same."""
    global _LIB, _LIB_PATH
    if _LIB is not None and _LIB_PATH != _build.LIB:
        return _build.flags(native=True)
    _LIB_PATH = _build.build(native=True)
    _LIB = None
    _lib()
    return _build.flags(native=True)


def set_num_threads(n: int) -> None:
    _lib().txo_set_num_threads(int(n))


def _f64(x):
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return int(_lib().txo_num_threads())


def rel_attn(q, k, v, r, u, vb, mem_len, scale=None, want_scores=False):
    """Relative-position attention, direct definition (section 3.3, A^rel).

    q [B,L,H,d]; k, v [B,T,H,d] with T = mem_len + L (memory rows first);
    r [>=T,H,d] with row p the projected encoding of distance p; u, vb [H,d].
    Returns out [B,L,H,d] (and scores [B,H,L,T] with -inf where masked).
    """
    q, k, v, r, u, vb = map(_f64, (q, k, v, r, u, vb))
    B, L, H, d = q.shape
    T = mem_len + L
    assert k.shape == (B, T, H, d) and v.shape == (B, T, H, d)
    assert r.shape[0] >= T and r.shape[1:] == (H, d)
    r = np.ascontiguousarray(r[:T])
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    out = np.zeros((B, L, H, d))
    scores = np.zeros((B, H, L, T)) if want_scores else None
    _lib().txo_rel_attn(B, H, L, mem_len, d, _ptr(q), _ptr(k), _ptr(v), _ptr(r),
                        _ptr(u), _ptr(vb), float(scale), _ptr(out), _ptr(scores))
    return (out, scores) if want_scores else out


def linear(x, W):
    """y = x W^T over the last axis of x (the pages' h W^T convention)."""
    x, W = _f64(x), _f64(W)
    lead = x.shape[:-1]
    x2 = x.reshape(-1, x.shape[-1])
    y = np.zeros((x2.shape[0], W.shape[0]))
    _lib().txo_linear(x2.shape[0], W.shape[0], W.shape[1], _ptr(x2), _ptr(W), _ptr(y))
    return y.reshape(*lead, W.shape[0])


def pos_ff(x, W1, b1, W2, b2, gamma, beta, eps=1e-5):
    """Position-wise feed-forward (section 3.3's h = Positionwise-Feed-Forward(o)),
    read as LayerNorm(x + relu(x W1^T + b1) W2^T + b2) over the last axis of x.
    W1 [Di, D], b1 [Di], W2 [D, Di], b2 / gamma / beta [D]."""
    x = _f64(x)
    W1, b1, W2, b2 = _f64(W1), _f64(b1), _f64(W2), _f64(b2)
    gamma, beta = _f64(gamma), _f64(beta)
    D, Di = x.shape[-1], W1.shape[0]
    assert W1.shape == (Di, D) and W2.shape == (D, Di) and b1.shape == (Di,)
    x2 = x.reshape(-1, D)
    out = np.zeros_like(x2)
    rc = _lib().txo_pos_ff(x2.shape[0], D, Di, _ptr(x2), _ptr(W1), _ptr(b1), _ptr(W2), _ptr(b2),
                           _ptr(gamma), _ptr(beta), float(eps), _ptr(out))
    if rc != 0:
        raise MemoryError("oracle pos_ff: allocation failed")
    return out.reshape(x.shape)


def layer_norm(x, gamma, beta, eps=1e-5):
    x, gamma, beta = _f64(x), _f64(gamma), _f64(beta)
    D = x.shape[-1]
    y = np.zeros_like(x)
    _lib().txo_layer_norm(x.size // D, D, _ptr(x), _ptr(gamma), _ptr(beta), float(eps), _ptr(y))
    return y


def layer_step(h, mem, W, u, vb, R, eps=1e-5, want_intermediates=False):
    """One layer, one segment (section 3.3 N-layer procedure, no feed-forward).

    h [B,L,D]; mem [B,mem_len,D] in logical order (mem_len may be 0);
    W: dict with W_q, W_kE, W_v, W_kR [H*d,D], W_o [D,H*d], gamma, beta [D];
    u, vb [H,d]; R [>=mem_len+L, D].  Returns h_out [B,L,D] (and a dict of
    q, k, v, r, a when want_intermediates).
    """
    h = _f64(h)
    B, L, D = h.shape
    u = _f64(u)
    H, d = u.shape
    mem = _f64(mem) if mem is not None else np.zeros((B, 0, D))
    mem_len = mem.shape[1]
    T = mem_len + L
    R = _f64(R)
    assert R.shape[0] >= T and R.shape[1] == D
    Wd = {n: _f64(W[n]) for n in ("W_q", "W_kE", "W_v", "W_kR", "W_o", "gamma", "beta")}
    vb = _f64(vb)
    h_out = np.zeros((B, L, D))
    inter = None
    if want_intermediates:
        inter = {"q": np.zeros((B, L, H, d)), "k": np.zeros((B, T, H, d)),
                 "v": np.zeros((B, T, H, d)), "r": np.zeros((T, H, d)),
                 "a": np.zeros((B, L, H, d))}
    g = (lambda n: _ptr(inter[n])) if inter else (lambda n: None)
    rc = _lib().txo_layer_step(
        B, L, D, H, d, mem_len, float(eps), _ptr(h), _ptr(mem) if mem_len else None,
        _ptr(Wd["W_q"]), _ptr(Wd["W_kE"]), _ptr(Wd["W_v"]), _ptr(Wd["W_kR"]),
        _ptr(Wd["W_o"]), _ptr(Wd["gamma"]), _ptr(Wd["beta"]), _ptr(u), _ptr(vb),
        _ptr(R), _ptr(h_out), g("q"), g("k"), g("v"), g("r"), g("a"))
    if rc != 0:
        raise MemoryError("oracle layer_step: allocation failed")
    return (h_out, inter) if want_intermediates else h_out


def layer_step_rows(h, mem, W, u, vb, R, rows, eps=1e-5):
    """The layer step evaluated only at the sampled output rows [(b, i), ...].

    Same arithmetic as layer_step; returns [len(rows), D].
    """
    h = _f64(h)
    B, L, D = h.shape
    u = _f64(u)
    H, d = u.shape
    mem = _f64(mem) if mem is not None else np.zeros((B, 0, D))
    mem_len = mem.shape[1]
    R = _f64(R)
    assert R.shape[0] >= mem_len + L
    Wd = {n: _f64(W[n]) for n in ("W_q", "W_kE", "W_v", "W_kR", "W_o", "gamma", "beta")}
    rows = sorted(rows)
    bs = np.array([b for b, _ in rows], dtype=np.int64)
    is_ = np.array([i for _, i in rows], dtype=np.int64)
    out = np.zeros((len(rows), D))
    rc = _lib().txo_layer_step_rows(
        B, L, D, H, d, mem_len, float(eps), _ptr(h), _ptr(mem) if mem_len else None,
        _ptr(Wd["W_q"]), _ptr(Wd["W_kE"]), _ptr(Wd["W_v"]), _ptr(Wd["W_kR"]),
        _ptr(Wd["W_o"]), _ptr(Wd["gamma"]), _ptr(Wd["beta"]), _ptr(u), _ptr(_f64(vb)),
        _ptr(R), len(rows), _ptr(bs), _ptr(is_), _ptr(out))
    if rc != 0:
        raise MemoryError("oracle layer_step_rows: allocation failed")
    return rows, out


def mem_update(mem, h, M):
    """New memory = last min(M, mem_len+L) rows of [mem ; h] (section 3.2).

    mem [B,mem_len,D] logical order; h [B,L,D].  Returns [B,new_len,D].
    """
    h = _f64(h)
    B, L, D = h.shape
    mem = _f64(mem) if mem is not None else np.zeros((B, 0, D))
    out = np.zeros((B, M, D))
    n = _lib().txo_mem_update(B, M, D, _ptr(mem) if mem.shape[1] else None, mem.shape[1],
                              _ptr(h), L, _ptr(out))
    return np.ascontiguousarray(out[:, :n])
