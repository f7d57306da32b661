"""Thin ctypes binding of libtxl.so (declared in include/txl.h).

Argument marshalling only: torch supplies device memory (data_ptr), strides
and the current HIP stream; every step of the computation runs in the
library's HIP kernels.  Importing this module fails loudly if libtxl.so has
not been built (there is no fallback of any kind).
"""
import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtxl.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                      "(or python relative_position_memory_amd/build.py)")
_lib = ctypes.CDLL(LIB_PATH)

FP32, BF16 = 0, 1
OK, EINVAL, EUNSUPPORTED, EHIP, EWORKSPACE = 0, -1, -2, -3, -4

_i64, _p, _f, _sz = ctypes.c_int64, ctypes.c_void_p, ctypes.c_float, ctypes.c_size_t


class Ring(ctypes.Structure):
    """txl_ring: the memory of one layer as a ring over [B, capacity, d_model]."""
    _fields_ = [("data", _p), ("capacity", _i64), ("start", _i64), ("len", _i64)]


class LayerDims(ctypes.Structure):
    _fields_ = [("B", _i64), ("L", _i64), ("d_model", _i64), ("n_head", _i64),
                ("d_head", _i64), ("ln_eps", _f)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("W_q", _p), ("W_kE", _p), ("W_v", _p), ("W_kR", _p), ("W_o", _p),
                ("ln_gamma", _p), ("ln_beta", _p)]


_lib.txl_rel_attn_fwd.argtypes = ([_p, ctypes.c_int] + [_i64] * 5 + [_p, _i64, _i64, _i64]
                                  + [_p, _p, _i64, _i64, _i64] + [_p, _i64, _i64, _i64]
                                  + [_p, _p, _f] + [_p, _i64, _i64, _i64] + [_p, _p, _sz])
_lib.txl_rel_attn_fwd.restype = ctypes.c_int
_lib.txl_rel_attn_workspace_bytes.argtypes = [ctypes.c_int] + [_i64] * 5
_lib.txl_rel_attn_bwd.argtypes = ([_p, ctypes.c_int] + [_i64] * 5 + [_p, _i64, _i64, _i64]
                                  + [_p, _p, _i64, _i64, _i64] + [_p, _i64, _i64, _i64]
                                  + [_p, _p, ctypes.c_float] + [_p, _i64, _i64, _i64]
                                  + [_p] * 6 + [_p, ctypes.c_size_t])
_lib.txl_rel_attn_bwd.restype = ctypes.c_int
_lib.txl_rel_attn_bwd_workspace_bytes.argtypes = [ctypes.c_int] + [_i64] * 5
_lib.txl_rel_attn_bwd_workspace_bytes.restype = ctypes.c_size_t
_lib.txl_rel_attn_workspace_bytes.restype = _sz
_lib.txl_layer_workspace_bytes.argtypes = [ctypes.POINTER(LayerDims), _i64, ctypes.c_int]
_lib.txl_layer_workspace_bytes.restype = _sz
_lib.txl_layer_step.argtypes = [_p, ctypes.c_int, ctypes.POINTER(LayerDims), _p,
                                ctypes.POINTER(Ring), ctypes.POINTER(LayerWeights), _p, _p,
                                _p, _i64, _p, _p, _sz]
_lib.txl_layer_step.restype = ctypes.c_int
_lib.txl_mem_update.argtypes = [_p, ctypes.c_int, ctypes.POINTER(Ring), _i64, _i64, _p, _i64]
_lib.txl_mem_update.restype = ctypes.c_int
_lib.txl_status_string.argtypes = [ctypes.c_int]
_lib.txl_status_string.restype = ctypes.c_char_p


_lib.txl_attn_variant.argtypes = [ctypes.c_int]
_lib.txl_attn_variant.restype = ctypes.c_int


def attn_variant(variant: int) -> int:
    """txl_attn_variant: 0 by shape, 1 the 64-query kernel, 2 the 128-query kernel
    with key splits; returns the previous setting."""
    rc = _lib.txl_attn_variant(int(variant))
    if rc < 0:
        raise TxlError(rc, "txl_attn_variant")
    return rc


_lib.txl_attn_kernel.argtypes = [ctypes.c_int] + [_i64] * 5
_lib.txl_attn_kernel.restype = ctypes.c_int
ATTN_KERNEL_NAMES = {0: "attn_generic (vector unit)", 1: "attn_decode_kernel + merge",
                     2: "attn_mfma_kernel", 3: "attn_mfma_kernel + key-split merge",
                     4: "attn_q64_kernel"}


def attn_kernel(dtype: torch.dtype, B, H, L, mem_len, d_head) -> str:
    """txl_attn_kernel: the name of the kernel txl_rel_attn_fwd runs at these sizes."""
    rc = _lib.txl_attn_kernel(dtype_code(dtype), B, H, L, int(mem_len), d_head)
    if rc < 0:
        raise TxlError(rc, "txl_attn_kernel")
    return ATTN_KERNEL_NAMES[rc]


class TxlError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)}")
        self.status = status


def status_string(status: int) -> str:
    return _lib.txl_status_string(int(status)).decode()


def dtype_code(t: torch.dtype) -> int:
    if t == torch.float32:
        return FP32
    if t == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t}")


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(rc, what):
    if rc != OK:
        raise TxlError(rc, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def rel_attn_workspace_bytes(dtype, B, H, L, mem_len, d):
    """txl_rel_attn_workspace_bytes: scratch the key split can use (0 = no split)."""
    return int(_lib.txl_rel_attn_workspace_bytes(dtype_code(dtype), B, H, L, int(mem_len), d))


def rel_attn_fwd(q, k, v, r, u, vb, mem_len, out, scale=None, scores=None, stream=None,
                 workspace=None):
    """txl_rel_attn_fwd on torch tensors.

    q, out [B, L, H, d]; k, v [B, mem_len+L, H, d]; r [R_rows, H, d]; u, vb [H, d]
    (dense).  Any strides are passed through as long as the last dimension is
    contiguous.  scores: None or float32 [B, H, L, mem_len+L] contiguous.
    workspace: None or a uint8 device tensor of rel_attn_workspace_bytes() bytes.
    """
    B, L, H, d = q.shape
    for t in (q, k, v, r, out):
        if t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if scores is not None and (scores.dtype != torch.float32 or not scores.is_contiguous()):
        raise ValueError("scores must be a contiguous float32 tensor")
    rc = _lib.txl_rel_attn_fwd(
        _stream(stream), dtype_code(q.dtype), B, H, L, int(mem_len), d,
        _ptr(q), q.stride(0), q.stride(1), q.stride(2),
        _ptr(k), _ptr(v), k.stride(0), k.stride(1), k.stride(2),
        _ptr(r), r.stride(0), r.stride(1), r.shape[0],
        _ptr(u), _ptr(vb), float(scale),
        _ptr(out), out.stride(0), out.stride(1), out.stride(2), _ptr(scores),
        _ptr(workspace), 0 if workspace is None else workspace.numel() * workspace.element_size())
    _check(rc, "txl_rel_attn_fwd")
    return out


_lib.txl_rel_attn_fwd_noalloc.argtypes = _lib.txl_rel_attn_fwd.argtypes[:-2]
_lib.txl_rel_attn_fwd_noalloc.restype = ctypes.c_int
_lib.txl_rel_attn_noalloc_max_scratch_bytes.argtypes = []
_lib.txl_rel_attn_noalloc_max_scratch_bytes.restype = _sz


def rel_attn_noalloc_max_scratch_bytes() -> int:
    return int(_lib.txl_rel_attn_noalloc_max_scratch_bytes())


def rel_attn_fwd_noalloc(q, k, v, r, u, vb, mem_len, out, scale=None, scores=None, stream=None):
    """txl_rel_attn_fwd_noalloc: rel_attn_fwd without a workspace (the library's
    static device scratch holds the key-split partials)."""
    B, L, H, d = q.shape
    for t in (q, k, v, r, out):
        if t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if scores is not None and (scores.dtype != torch.float32 or not scores.is_contiguous()):
        raise ValueError("scores must be a contiguous float32 tensor")
    rc = _lib.txl_rel_attn_fwd_noalloc(
        _stream(stream), dtype_code(q.dtype), B, H, L, int(mem_len), d,
        _ptr(q), q.stride(0), q.stride(1), q.stride(2),
        _ptr(k), _ptr(v), k.stride(0), k.stride(1), k.stride(2),
        _ptr(r), r.stride(0), r.stride(1), r.shape[0],
        _ptr(u), _ptr(vb), float(scale),
        _ptr(out), out.stride(0), out.stride(1), out.stride(2), _ptr(scores))
    _check(rc, "txl_rel_attn_fwd_noalloc")
    return out


def rel_attn_bwd_workspace_bytes(dtype, B, H, L, mem_len, d):
    """txl_rel_attn_bwd_workspace_bytes."""
    return int(_lib.txl_rel_attn_bwd_workspace_bytes(dtype_code(dtype), B, H, L, int(mem_len), d))


def rel_attn_bwd(q, k, v, r, u, vb, mem_len, dout, scale=None, stream=None, workspace=None):
    """txl_rel_attn_bwd on torch tensors (layouts as rel_attn_fwd; dout like out).

    Returns a dict of fp32 gradients dq [B,L,H,d], dk, dv [B,T,H,d], dr [T,H,d],
    du, dvb [H,d].  workspace: None (allocated here) or a uint8 device tensor of
    at least rel_attn_bwd_workspace_bytes() bytes.
    """
    B, L, H, d = q.shape
    T = int(mem_len) + L
    for t in (q, k, v, r, dout):
        if t.stride(-1) != 1:
            raise ValueError("the head dimension must be contiguous")
    if k.stride() != v.stride():
        raise ValueError("k and v must share strides")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dev = q.device
    f32 = torch.float32
    g = {"dq": torch.empty((B, L, H, d), dtype=f32, device=dev),
         "dk": torch.empty((B, T, H, d), dtype=f32, device=dev),
         "dv": torch.empty((B, T, H, d), dtype=f32, device=dev),
         "dr": torch.empty((T, H, d), dtype=f32, device=dev),
         "du": torch.empty((H, d), dtype=f32, device=dev),
         "dvb": torch.empty((H, d), dtype=f32, device=dev)}
    if workspace is None:
        nb = rel_attn_bwd_workspace_bytes(q.dtype, B, H, L, mem_len, d)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev)
    rc = _lib.txl_rel_attn_bwd(
        _stream(stream), dtype_code(q.dtype), B, H, L, int(mem_len), d,
        _ptr(q), q.stride(0), q.stride(1), q.stride(2),
        _ptr(k), _ptr(v), k.stride(0), k.stride(1), k.stride(2),
        _ptr(r), r.stride(0), r.stride(1), r.shape[0],
        _ptr(u), _ptr(vb), float(scale),
        _ptr(dout), dout.stride(0), dout.stride(1), dout.stride(2),
        _ptr(g["dq"]), _ptr(g["dk"]), _ptr(g["dv"]), _ptr(g["dr"]), _ptr(g["du"]), _ptr(g["dvb"]),
        _ptr(workspace), workspace.numel() * workspace.element_size())
    _check(rc, "txl_rel_attn_bwd")
    return g


def layer_dims(B, L, d_model, n_head, d_head, ln_eps=1e-5):
    return LayerDims(B, L, d_model, n_head, d_head, ln_eps)


def workspace_bytes(dims: LayerDims, mem_capacity: int, dtype: torch.dtype) -> int:
    n = _lib.txl_layer_workspace_bytes(ctypes.byref(dims), int(mem_capacity), dtype_code(dtype))
    if n == 0:
        raise ValueError("invalid layer dims")
    return int(n)


def make_ring(data, start=0, length=0) -> Ring:
    """A Ring over a [B, capacity, d_model] device tensor (kept alive by the caller)."""
    return Ring(data.data_ptr(), data.shape[1], int(start), int(length))


def layer_weights(W) -> LayerWeights:
    """LayerWeights of raw device pointers into the tensors of W: they must outlive
    every call that takes the returned struct (it holds no reference to them)."""
    return LayerWeights(*[W[n].data_ptr() for n in
                          ("W_q", "W_kE", "W_v", "W_kR", "W_o", "gamma", "beta")])


def layer_step(dims, h_in, ring, W, u, vb, R, h_out, workspace, stream=None):
    """txl_layer_step; W is a LayerWeights (see layer_weights) or a dict of tensors."""
    lw = W if isinstance(W, LayerWeights) else layer_weights(W)
    rc = _lib.txl_layer_step(_stream(stream), dtype_code(h_in.dtype), ctypes.byref(dims),
                             _ptr(h_in), ctypes.byref(ring), ctypes.byref(lw), _ptr(u),
                             _ptr(vb), _ptr(R), R.shape[0], _ptr(h_out), _ptr(workspace),
                             workspace.numel() * workspace.element_size())
    _check(rc, "txl_layer_step")
    return h_out


def mem_update(ring, h_new, stream=None):
    """txl_mem_update: append the newest rows of h_new [B, L, d_model] to the ring."""
    B, L, D = h_new.shape
    rc = _lib.txl_mem_update(_stream(stream), dtype_code(h_new.dtype), ctypes.byref(ring),
                             B, D, _ptr(h_new), L)
    _check(rc, "txl_mem_update")
    return ring


STACK_MAX_STREAMS = 8
_lib.txl_stack_workspace_bytes.argtypes = [ctypes.POINTER(LayerDims), _i64, ctypes.c_int,
                                           ctypes.c_int]
_lib.txl_stack_workspace_bytes.restype = _sz
_lib.txl_stack_fwd.argtypes = [ctypes.POINTER(_p), ctypes.c_int, ctypes.c_int,
                               ctypes.POINTER(LayerDims), _i64, _i64, _p, ctypes.POINTER(Ring),
                               ctypes.POINTER(LayerWeights), _p, _p, _p, _i64, _p, _p, _sz]
_lib.txl_stack_fwd.restype = ctypes.c_int


def stack_workspace_bytes(dims: LayerDims, mem_capacity: int, dtype: torch.dtype,
                          n_streams: int) -> int:
    n = _lib.txl_stack_workspace_bytes(ctypes.byref(dims), int(mem_capacity), dtype_code(dtype),
                                       int(n_streams))
    if n == 0:
        raise ValueError("invalid dims, dtype or stream count")
    return int(n)


def stack_fwd(streams, dims, h_in, rings, lws, u, vb, R, h_out, workspace):
    """txl_stack_fwd: the layer stack over h_in's segments [S, B, L, D] on the given
    streams (a list; None entries mean the current stream).  rings (a list of Ring)
    are advanced in place; lws is a list of LayerWeights."""
    S = h_in.shape[0]
    n = len(rings)
    if len(lws) != n:
        raise ValueError("one LayerWeights per ring")
    sa = (_p * len(streams))(*[_stream(st).value for st in streams])
    ra = (Ring * n)(*rings)
    wa = (LayerWeights * n)(*lws)
    rc = _lib.txl_stack_fwd(sa, len(streams), dtype_code(h_in.dtype), ctypes.byref(dims), n, S,
                            _ptr(h_in), ra, wa, _ptr(u), _ptr(vb), _ptr(R), R.shape[0],
                            _ptr(h_out), _ptr(workspace),
                            workspace.numel() * workspace.element_size())
    for i in range(n):  # the library advanced the copies
        rings[i].start, rings[i].len = ra[i].start, ra[i].len
    _check(rc, "txl_stack_fwd")
    return h_out


class WorkspaceMap(ctypes.Structure):
    _fields_ = [("q", _sz), ("k", _sz), ("v", _sz), ("r", _sz), ("a", _sz), ("d_pad", _i64)]


_lib.txl_layer_workspace_map.argtypes = [ctypes.POINTER(LayerDims), _i64, ctypes.c_int,
                                         ctypes.POINTER(WorkspaceMap)]
_lib.txl_layer_workspace_map.restype = ctypes.c_int


class LayerGrads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("dh", "dW_q", "dW_kE", "dW_v", "dW_kR", "dW_o", "du", "dv_bias", "dgamma",
                 "dbeta")]


_lib.txl_layer_bwd_workspace_bytes.argtypes = [ctypes.POINTER(LayerDims), _i64, ctypes.c_int]
_lib.txl_layer_bwd_workspace_bytes.restype = _sz
_lib.txl_layer_step_bwd.argtypes = [_p, ctypes.c_int, ctypes.POINTER(LayerDims), _p,
                                    ctypes.POINTER(Ring), ctypes.POINTER(LayerWeights), _p, _p,
                                    _p, _i64, _p, ctypes.POINTER(LayerGrads), _p, _sz]
_lib.txl_layer_step_bwd.restype = ctypes.c_int


class LayerSaved(ctypes.Structure):
    """txl_layer_saved: the buffer, what it holds, and the call it belongs to."""
    _fields_ = [("data", ctypes.c_void_p), ("bytes", _sz), ("has_lse", ctypes.c_int),
                ("has_y", ctypes.c_int), ("mem_data", ctypes.c_void_p),
                ("mem_capacity", _i64), ("mem_start", _i64), ("mem_len", _i64),
                ("h_in", ctypes.c_void_p), ("B", _i64), ("L", _i64), ("d_model", _i64),
                ("n_head", _i64), ("d_head", _i64), ("dtype", ctypes.c_int)]


_lib.txl_layer_saved_bytes.argtypes = [ctypes.POINTER(LayerDims), _i64, ctypes.c_int]
_lib.txl_layer_saved_bytes.restype = _sz
_lib.txl_layer_step_save.argtypes = [_p, ctypes.c_int, ctypes.POINTER(LayerDims), _p,
                                     ctypes.POINTER(Ring), ctypes.POINTER(LayerWeights), _p, _p,
                                     _p, _i64, _p, ctypes.POINTER(LayerSaved)]
_lib.txl_layer_step_save.restype = ctypes.c_int
_lib.txl_layer_step_bwd_saved.argtypes = [_p, ctypes.c_int, ctypes.POINTER(LayerDims), _p,
                                          ctypes.POINTER(Ring), ctypes.POINTER(LayerWeights), _p,
                                          _p, _p, _i64, _p, ctypes.POINTER(LayerSaved),
                                          ctypes.POINTER(LayerGrads), _p, _sz]
_lib.txl_layer_step_bwd_saved.restype = ctypes.c_int


def layer_saved_bytes(dims: LayerDims, mem_capacity: int, dtype: torch.dtype) -> int:
    """txl_layer_saved_bytes."""
    return int(_lib.txl_layer_saved_bytes(ctypes.byref(dims), int(mem_capacity),
                                          dtype_code(dtype)))


def layer_step_save(dims, h_in, ring, W, u, vb, R, h_out, saved_buf, stream=None):
    """txl_layer_step_save into the device buffer saved_buf (uint8, 256-byte
    aligned); returns the LayerSaved to hand to layer_step_bwd(saved=...)."""
    lw = W if isinstance(W, LayerWeights) else layer_weights(W)
    sv = LayerSaved(data=_ptr(saved_buf), bytes=saved_buf.numel() * saved_buf.element_size())
    rc = _lib.txl_layer_step_save(_stream(stream), dtype_code(h_in.dtype), ctypes.byref(dims),
                                  _ptr(h_in), ctypes.byref(ring), ctypes.byref(lw), _ptr(u),
                                  _ptr(vb), _ptr(R), R.shape[0], _ptr(h_out), ctypes.byref(sv))
    _check(rc, "txl_layer_step_save")
    return sv


def layer_bwd_workspace_bytes(dims: LayerDims, mem_capacity: int, dtype: torch.dtype) -> int:
    """txl_layer_bwd_workspace_bytes."""
    return int(_lib.txl_layer_bwd_workspace_bytes(ctypes.byref(dims), int(mem_capacity),
                                                  dtype_code(dtype)))


def layer_step_bwd(dims, h, ring, W, u, vb, R, dh_out, workspace, grads=None, stream=None,
                   saved=None):
    """txl_layer_step_bwd, or txl_layer_step_bwd_saved when saved (a LayerSaved from
    layer_step_save) is given.  grads: None (fp32 tensors allocated here) or a
    dict with the keys of LayerGrads.  Returns the dict of gradient tensors."""
    dev = h.device
    D, H, d = dims.d_model, dims.n_head, dims.d_head
    f32 = torch.float32
    if grads is None:
        grads = {"dh": torch.empty((dims.B, dims.L, D), dtype=f32, device=dev),
                 "dW_q": torch.empty((H * d, D), dtype=f32, device=dev),
                 "dW_kE": torch.empty((H * d, D), dtype=f32, device=dev),
                 "dW_v": torch.empty((H * d, D), dtype=f32, device=dev),
                 "dW_kR": torch.empty((H * d, D), dtype=f32, device=dev),
                 "dW_o": torch.empty((D, H * d), dtype=f32, device=dev),
                 "du": torch.empty((H, d), dtype=f32, device=dev),
                 "dv_bias": torch.empty((H, d), dtype=f32, device=dev),
                 "dgamma": torch.empty((D,), dtype=f32, device=dev),
                 "dbeta": torch.empty((D,), dtype=f32, device=dev)}
    gs = LayerGrads(**{n: _ptr(t) for n, t in grads.items()})
    lw = W if isinstance(W, LayerWeights) else layer_weights(W)
    nbytes = workspace.numel() * workspace.element_size()
    if saved is None:
        rc = _lib.txl_layer_step_bwd(_stream(stream), dtype_code(h.dtype), ctypes.byref(dims),
                                     _ptr(h), ctypes.byref(ring), ctypes.byref(lw), _ptr(u),
                                     _ptr(vb), _ptr(R), R.shape[0], _ptr(dh_out),
                                     ctypes.byref(gs), _ptr(workspace), nbytes)
        _check(rc, "txl_layer_step_bwd")
    else:
        rc = _lib.txl_layer_step_bwd_saved(_stream(stream), dtype_code(h.dtype),
                                           ctypes.byref(dims), _ptr(h), ctypes.byref(ring),
                                           ctypes.byref(lw), _ptr(u), _ptr(vb), _ptr(R),
                                           R.shape[0], _ptr(dh_out), ctypes.byref(saved),
                                           ctypes.byref(gs), _ptr(workspace), nbytes)
        _check(rc, "txl_layer_step_bwd_saved")
    return grads


def workspace_views(dims, mem_len, workspace, dtype, padded=False):
    """Views of the intermediates txl_layer_step leaves in `workspace`
    (txl_layer_workspace_map): q [B,L,H,d], k/v [B,T,H,d], r [T,H,d], a [B,L,H,d].
    padded=True gives q, k, v, r with their whole d_pad-wide rows (the columns
    past d hold zeros)."""
    mp = WorkspaceMap()
    _check(_lib.txl_layer_workspace_map(ctypes.byref(dims), int(mem_len), dtype_code(dtype),
                                        ctypes.byref(mp)), "txl_layer_workspace_map")
    B, L, H, d, dp = dims.B, dims.L, dims.n_head, dims.d_head, mp.d_pad
    T = mem_len + L
    es = torch.tensor([], dtype=dtype).element_size()
    dq = dp if padded else d

    def view(off, shape):
        n = 1
        for s in shape:
            n *= s
        return workspace[off: off + n * es].view(dtype).view(*shape)

    q = view(mp.q, (B, H, L, dp))[..., :dq].permute(0, 2, 1, 3)
    k = view(mp.k, (B, H, T, dp))[..., :dq].permute(0, 2, 1, 3)
    v = view(mp.v, (B, H, T, dp))[..., :dq].permute(0, 2, 1, 3)
    r = view(mp.r, (H, T, dp))[..., :dq].permute(1, 0, 2)
    a = view(mp.a, (B, L, H, d))
    return {"q": q, "k": k, "v": v, "r": r, "a": a}


# ---- evaluation with cached keys and values ----------------------------------------------

class KVRing(ctypes.Structure):
    """txl_kv_ring: projected k and v of the memory rows, [B, H, capacity, d_pad] each."""
    _fields_ = [("k", _p), ("v", _p), ("capacity", _i64), ("start", _i64), ("len", _i64),
                ("mem_max", _i64)]


_lib.txl_kv_ring_bytes.argtypes = [ctypes.POINTER(LayerDims), _i64, ctypes.c_int]
_lib.txl_kv_ring_bytes.restype = _sz
_lib.txl_pos_proj.argtypes = [_p, ctypes.c_int, ctypes.POINTER(LayerDims), _p, _i64, _p, _p]
_lib.txl_pos_proj.restype = ctypes.c_int
_lib.txl_layer_kv_workspace_bytes.argtypes = [ctypes.POINTER(LayerDims), _i64, ctypes.c_int]
_lib.txl_layer_kv_workspace_bytes.restype = _sz
_lib.txl_layer_step_kv.argtypes = [_p, ctypes.c_int, ctypes.POINTER(LayerDims), _p,
                                   ctypes.POINTER(KVRing), ctypes.POINTER(LayerWeights), _p, _p,
                                   _p, _i64, _p, _p, _sz]
_lib.txl_layer_step_kv.restype = ctypes.c_int


def d_pad(d_head: int) -> int:
    return (int(d_head) + 7) // 8 * 8


def make_kv_ring(dims, mem_max, dtype, capacity=None, device="cuda"):
    """Allocates k, v [B, H, capacity, d_pad] (capacity defaults to mem_max + L) and
    returns (KVRing, k, v); the caller keeps k and v alive."""
    cap = int(mem_max + dims.L if capacity is None else capacity)
    if _lib.txl_kv_ring_bytes(ctypes.byref(dims), cap, dtype_code(dtype)) == 0:
        raise ValueError("invalid layer dims or capacity")
    shape = (dims.B, dims.n_head, cap, d_pad(dims.d_head))
    k = torch.empty(shape, dtype=dtype, device=device)
    v = torch.empty(shape, dtype=dtype, device=device)
    return KVRing(k.data_ptr(), v.data_ptr(), cap, 0, 0, int(mem_max)), k, v


def pos_proj(dims, R, W_kR, r_out=None, stream=None):
    """txl_pos_proj: r = R W_kR^T as [H, R_rows, d_pad]."""
    rows = R.shape[0]
    if r_out is None:
        r_out = torch.empty((dims.n_head, rows, d_pad(dims.d_head)), dtype=R.dtype,
                            device=R.device)
    rc = _lib.txl_pos_proj(_stream(stream), dtype_code(R.dtype), ctypes.byref(dims), _ptr(R),
                           rows, _ptr(W_kR), _ptr(r_out))
    _check(rc, "txl_pos_proj")
    return r_out


def kv_workspace_bytes(dims, mem_max, dtype) -> int:
    n = _lib.txl_layer_kv_workspace_bytes(ctypes.byref(dims), int(mem_max), dtype_code(dtype))
    if n == 0:
        raise ValueError("invalid layer dims")
    return int(n)


def layer_step_kv(dims, h_in, kv, W, u, vb, r, h_out, workspace, stream=None):
    """txl_layer_step_kv; r from pos_proj ([H, r_rows, d_pad]); kv is a KVRing."""
    lw = W if isinstance(W, LayerWeights) else layer_weights(W)
    rc = _lib.txl_layer_step_kv(_stream(stream), dtype_code(h_in.dtype), ctypes.byref(dims),
                                _ptr(h_in), ctypes.byref(kv), ctypes.byref(lw), _ptr(u), _ptr(vb),
                                _ptr(r), r.shape[1], _ptr(h_out), _ptr(workspace),
                                workspace.numel() * workspace.element_size())
    _check(rc, "txl_layer_step_kv")
    return h_out


# ---- position-wise feed-forward ----------------------------------------------------------

_lib.txl_pos_ff_workspace_bytes.argtypes = [_i64, _i64, _i64, ctypes.c_int]
_lib.txl_pos_ff_workspace_bytes.restype = _sz
_lib.txl_pos_ff.argtypes = ([_p, ctypes.c_int, _i64, _i64, _i64] + [_p] * 7
                            + [ctypes.c_float, _p, _p, _sz])
_lib.txl_pos_ff.restype = ctypes.c_int


def pos_ff_workspace_bytes(rows, d_model, d_inner, dtype) -> int:
    n = _lib.txl_pos_ff_workspace_bytes(int(rows), int(d_model), int(d_inner), dtype_code(dtype))
    if n == 0:
        raise ValueError("invalid feed-forward sizes")
    return int(n)


def pos_ff(x, W1, b1, W2, b2, gamma, beta, out, workspace=None, eps=1e-5, stream=None):
    """txl_pos_ff over the rows of x [..., d_model]."""
    D = x.shape[-1]
    rows = x.numel() // D
    Di = W1.shape[0]
    if workspace is None:
        workspace = torch.empty(pos_ff_workspace_bytes(rows, D, Di, x.dtype), dtype=torch.uint8,
                                device=x.device)
    rc = _lib.txl_pos_ff(_stream(stream), dtype_code(x.dtype), rows, D, Di, _ptr(x), _ptr(W1),
                         _ptr(b1), _ptr(W2), _ptr(b2), _ptr(gamma), _ptr(beta), float(eps),
                         _ptr(out), _ptr(workspace), workspace.numel() * workspace.element_size())
    _check(rc, "txl_pos_ff")
    return out
