"""Parity of the attention backward (txl_rel_attn_bwd, through the C ABI) with
the fp64 backward oracle.

Both sides consume the same inputs (bf16 cases: values rounded to bf16 once).
fp32 inputs: the HIP path computes in fp32, so every gradient must agree within
2e-3 of its largest magnitude (fp32 sums over at most a few thousand keys and
the exponential's rounding stay near 1e-5 relative; a dropped or misplaced term
is O(1)).  bf16 inputs: the key-side products dv = P^T dO and dk = dS^T (q + u)
run on the bf16 matrix cores, so P, dS and q + u enter them rounded to bf16
(relative 2^-9 each, as P enters the forward's P V); an fp64 emulation of that
rounding at these shapes stays below 4e-3 of the largest magnitude, and the bar
is 1e-2.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle_bwd as OB
from relative_position_memory_amd import inputs as I
from tests.gpu_util import dev, need_gpu

pytestmark = pytest.mark.gpu

GRAD_TOL = 2e-3
TOL = {"fp32": GRAD_TOL, "bf16": 1e-2}


def _txl():
    need_gpu()
    from relative_position_memory_amd import txl
    return txl


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _dout(B, L, H, d, seed, dtype):
    g = np.random.default_rng(seed).standard_normal((B, L, H, d)).astype(np.float32)
    if dtype == "bf16":
        g = torch.from_numpy(g).bfloat16().float().numpy()
    return g


def _close(name, got, ref, tol):
    scale = max(1.0, float(np.max(np.abs(ref))))
    err = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    assert err <= tol * scale, f"{name}: max err {err:.3e} (scale {scale:.3e})"


def _run(c, dout, M, dtype, layout="bthd"):
    txl = _txl()
    if layout == "bthd":
        q, k, v, r = (dev(c[n], dtype) for n in ("q", "k", "v", "r"))
        g = dev(dout, dtype)
    else:  # head-major storage passed as permuted views
        hm = lambda x: dev(x.transpose(0, 2, 1, 3), dtype).permute(0, 2, 1, 3)
        q, k, v, g = hm(c["q"]), hm(c["k"]), hm(c["v"]), hm(dout)
        r = dev(c["r"].transpose(1, 0, 2), dtype).permute(1, 0, 2)
    out = txl.rel_attn_bwd(q, k, v, r, dev(c["u"], dtype), dev(c["vb"], dtype), M, g)
    torch.cuda.synchronize()
    return {n: t.cpu().numpy().astype(np.float64) for n, t in out.items()}


@pytest.mark.parametrize("dtype,B,H,L,M,d,layout", [
    ("fp32", 1, 2, 16, 16, 16, "bthd"),     # the tiny workload's shape
    ("bf16", 2, 2, 37, 50, 64, "bhtd"),     # ragged tiles, head-major
    ("bf16", 1, 3, 130, 70, 41, "bthd"),    # d = 41, ragged query tail
    ("fp32", 2, 1, 65, 0, 32, "bthd"),      # no memory
    ("bf16", 1, 2, 1, 100, 64, "bthd"),     # one query over a memory
    ("fp32", 1, 1, 200, 333, 48, "bhtd"),   # memory longer than the segment
    ("bf16", 2, 1, 65, 0, 32, "bthd"),      # no memory, matrix-core path
    ("bf16", 1, 2, 200, 333, 64, "bhtd"),   # long memory, matrix-core path, T % 4 = 1
])
def test_attn_bwd_matches_oracle(dtype, B, H, L, M, d, layout):
    c = I.attention_inputs(B, H, L, M, d, seed=3 * L + M + d, sigma=1.0, sigma_uv=0.5,
                           dtype=dtype)
    dout = _dout(B, L, H, d, seed=L + d, dtype=dtype)
    _say(f"attn bwd dtype={dtype} B={B} H={H} L={L} M={M} d={d} layout={layout}")
    got = _run(c, dout, M, dtype, layout)
    ref = OB.rel_attn_bwd(c["q"], c["k"], c["v"], c["r"], c["u"], c["vb"], M, dout)
    for n in ("dq", "dk", "dv", "dr", "du", "dvb"):
        _close(n, got[n], ref[n], TOL[dtype])


def test_attn_bwd_large_train_shape_batch_row():
    """Large train-shape (B 8, H 16, L = M = 384, d 64, bf16): the query- and key-side
    gradients of one batch row depend only on that row, so batch row 0 is checked
    against the oracle run on it alone."""
    B, H, L, M, d = 8, 16, 384, 384, 64
    c = I.attention_inputs(B, H, L, M, d, seed=5, sigma=1.0, sigma_uv=0.5, dtype="bf16")
    dout = _dout(B, L, H, d, seed=9, dtype="bf16")
    _say("attn bwd large train shape")
    got = _run(c, dout, M, "bf16", "bhtd")
    c0 = {n: (c[n][:1] if n in ("q", "k", "v") else c[n]) for n in c}
    ref = OB.rel_attn_bwd(c0["q"], c0["k"], c0["v"], c0["r"], c0["u"], c0["vb"], M, dout[:1])
    for n in ("dq", "dk", "dv"):
        _close(n, got[n][:1], ref[n], TOL["bf16"])


def test_attn_bwd_rejects_bad_arguments():
    txl = _txl()
    B, H, L, M, d = 1, 1, 8, 8, 80
    x = torch.zeros((B, L, H, d), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((B, M + L, H, d), dtype=torch.bfloat16, device="cuda")
    r = torch.zeros((M + L, H, d), dtype=torch.bfloat16, device="cuda")
    u = torch.zeros((H, d), dtype=torch.bfloat16, device="cuda")
    assert txl.rel_attn_bwd_workspace_bytes(torch.bfloat16, B, H, L, M, d) == 0
    with pytest.raises(txl.TxlError):
        txl.rel_attn_bwd(x, kv, kv, r, u, u, M, x,
                         workspace=torch.empty(1 << 20, dtype=torch.uint8, device="cuda"))


# ---- layer step backward -----------------------------------------------------------------

# fp32: the HIP path's intermediates are fp32, so the gradients agree like the
# attention's.  bf16: q, k, v, r and a are rounded to bf16 between the kernels
# (relative 2^-9), the backward's products take their operands rounded to bf16
# (matrix cores, fp32 sums), and the scores, LayerNorm input and products that
# follow carry that rounding; 3e-2 of the largest magnitude bounds it with margin.
LAYER_TOL = {"fp32": GRAD_TOL, "bf16": 3e-2}
GRAD_NAMES = [("dh", "dh"), ("dW_q", "dW_q"), ("dW_kE", "dW_kE"), ("dW_v", "dW_v"),
              ("dW_kR", "dW_kR"), ("dW_o", "dW_o"), ("du", "du"), ("dv_bias", "dvb"),
              ("dgamma", "dgamma"), ("dbeta", "dbeta")]


@pytest.mark.parametrize("dtype,name,over,mem_len,start", [
    ("fp32", "tiny", {}, None, 0),
    ("fp32", "tiny", {}, 0, 0),                                                  # empty memory
    ("fp32", "tiny", {"B": 2, "L": 37, "M": 50, "d": 12, "H": 3, "D": 40}, 45, 31),  # ring wrap
    ("bf16", "charlm", {"B": 2, "L": 64, "M": 64, "D": 128, "H": 2, "d": 64}, 64, 0),
    ("bf16", "charlm", {"B": 3, "L": 50, "M": 50, "D": 82, "H": 2, "d": 41}, 50, 11),
    ("bf16", "charlm", {"B": 2, "L": 64, "M": 64, "D": 128, "H": 2, "d": 64}, 0, 0),  # empty memory
    # 128-wide product tiles with a ragged half tile
    ("bf16", "charlm", {"B": 2, "L": 96, "M": 160, "D": 192, "H": 3, "d": 64}, 160, 37),
    # weight gradients split along their summed rows (dW_o over B L = 200 > d_model;
    # dW_kE and dW_v over B T = 1,000 > 3 HD), partials summed after the grid
    ("bf16", "charlm", {"B": 2, "L": 100, "M": 400, "D": 192, "H": 3, "d": 64}, 400, 123),
    # d_model above 512: the backward reuses the forward's fp32 LayerNorm input y
    ("bf16", "charlm", {"B": 2, "L": 48, "M": 64, "D": 640, "H": 8, "d": 64}, 40, 30),
    # d_model a multiple of 256: the one-wave-per-row LayerNorm backward; 1,050 rows
    # (more than one row per wave, a partial last workgroup), 66 rows in fp32, and
    # four 256-column chunks per lane at d_model 1024
    ("bf16", "charlm", {"B": 3, "L": 350, "M": 50, "D": 256, "H": 4, "d": 64}, 50, 7),
    ("fp32", "tiny", {"B": 2, "L": 33, "M": 40, "D": 256, "H": 4, "d": 64}, 40, 5),
    ("bf16", "charlm", {"B": 1, "L": 40, "M": 24, "D": 1024, "H": 16, "d": 64}, 24, 3),
])
def test_layer_step_bwd_matches_oracle(dtype, name, over, mem_len, start):
    from tests.test_gpu_parity import _layer_setup
    w = I.workload(name, **over)
    _say(f"layer bwd {dtype} {w} mem_len={mem_len} start={start}")
    txl, x, W, data, ring, h, logical = _layer_setup(w, mem_len=mem_len, start=start)
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    nb = txl.layer_bwd_workspace_bytes(dims, w.M, h.dtype)
    assert nb > 0
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    g_out = np.random.default_rng(w.L + w.D).standard_normal((w.B, w.L, w.D)).astype(np.float32)
    if dtype == "bf16":
        g_out = torch.from_numpy(g_out).bfloat16().float().numpy()
    got = txl.layer_step_bwd(dims, h, ring, W, dev(x["u"], dtype), dev(x["v"], dtype),
                             dev(x["R"], dtype), dev(g_out, dtype), ws)
    torch.cuda.synchronize()
    ref = OB.layer_step_bwd(x["h0"][0], logical, x["weights"][0], x["u"], x["v"], x["R"], g_out)
    for gn, rn in GRAD_NAMES:
        g = got[gn].cpu().numpy().astype(np.float64)
        r = ref[rn]
        scale = max(1.0, float(np.max(np.abs(r))))
        err = float(np.max(np.abs(g - r)))
        assert err <= LAYER_TOL[dtype] * scale, f"{gn}: max err {err:.3e} (scale {scale:.3e})"


@pytest.mark.parametrize("dtype,name,over,mem_len,start", [
    ("fp32", "tiny", {"B": 2, "L": 37, "M": 50, "d": 12, "H": 3, "D": 40}, 45, 31),
    ("bf16", "charlm", {"B": 2, "L": 96, "M": 160, "D": 192, "H": 3, "d": 64}, 160, 37),
    ("bf16", "charlm", {"B": 3, "L": 50, "M": 50, "D": 82, "H": 2, "d": 41}, 50, 11),
    ("bf16", "charlm", {"B": 2, "L": 48, "M": 64, "D": 640, "H": 8, "d": 64}, 40, 30),
    # K-split output projection whose LayerNorm also writes the saved y
    ("bf16", "charlm", {"B": 1, "L": 40, "M": 24, "D": 1024, "H": 16, "d": 64}, 24, 3),
])
def test_layer_step_bwd_saved_matches_recompute(dtype, name, over, mem_len, start):
    """txl_layer_step_save + txl_layer_step_bwd_saved: the forward output equals
    txl_layer_step's and the gradients equal txl_layer_step_bwd's (same kernels on
    the same values; only the order of atomic sums may differ) and the oracle's."""
    from tests.test_gpu_parity import _layer_setup
    w = I.workload(name, **over)
    _say(f"layer bwd saved {dtype} {w} mem_len={mem_len} start={start}")
    txl, x, W, data, ring, h, logical = _layer_setup(w, mem_len=mem_len, start=start)
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    ws = torch.empty(txl.layer_bwd_workspace_bytes(dims, w.M, h.dtype), dtype=torch.uint8,
                     device="cuda")
    fws = torch.empty(txl.workspace_bytes(dims, w.M, h.dtype), dtype=torch.uint8, device="cuda")
    nsv = txl.layer_saved_bytes(dims, w.M, h.dtype)
    assert nsv > 0
    sbuf = torch.empty(nsv, dtype=torch.uint8, device="cuda")
    u, vb, R = dev(x["u"], dtype), dev(x["v"], dtype), dev(x["R"], dtype)
    g_out = np.random.default_rng(w.L + w.D).standard_normal((w.B, w.L, w.D)).astype(np.float32)
    if dtype == "bf16":
        g_out = torch.from_numpy(g_out).bfloat16().float().numpy()
    g_dev = dev(g_out, dtype)
    out_ref = torch.empty_like(h)
    txl.layer_step(dims, h, ring, W, u, vb, R, out_ref, fws)
    out_sv = torch.empty_like(h)
    sv = txl.layer_step_save(dims, h, ring, W, u, vb, R, out_sv, sbuf)
    torch.cuda.synchronize()
    assert torch.equal(out_sv, out_ref)
    got = txl.layer_step_bwd(dims, h, ring, W, u, vb, R, g_dev, ws, saved=sv)
    got = {n: t.clone() for n, t in got.items()}
    rec = txl.layer_step_bwd(dims, h, ring, W, u, vb, R, g_dev, ws)
    torch.cuda.synchronize()
    ref = OB.layer_step_bwd(x["h0"][0], logical, x["weights"][0], x["u"], x["v"], x["R"], g_out)
    for gn, rn in GRAD_NAMES:
        a, b = got[gn].cpu().double(), rec[gn].cpu().double()
        scale = max(1.0, float(b.abs().max()))
        assert float((a - b).abs().max()) <= 1e-5 * scale, gn
        r = ref[rn]
        scale = max(1.0, float(np.max(np.abs(r))))
        err = float(np.max(np.abs(a.numpy() - r)))
        assert err <= LAYER_TOL[dtype] * scale, f"{gn}: max err {err:.3e} (scale {scale:.3e})"
