"""Evaluation with cached keys and values (txl_layer_step_kv, txl_pos_proj).

The cached path must equal the recurrence of the plain definition: at every
segment the oracle runs a layer step over the hidden-state memory (the last M
layer inputs) and the memory update, and the cached path's output must match
it to the dtype's tolerance; it must also match txl_layer_step over a
hidden-state ring (the recompute path) on the same inputs.  Ring capacities that
are not multiples of the segment length make the rows wrap inside key tiles.
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from relative_position_memory_amd import inputs as I
from tests.gpu_util import TOL, dev, host, max_err

pytestmark = pytest.mark.gpu


def _txl():
    from relative_position_memory_amd import txl
    return txl


def _say(*a):
    print(*a, flush=True)


def _stream_case(w, segments, capacity_extra=0, seed=1):
    txl = _txl()
    dt = w.dtype
    x = I.make_inputs(w, seed=seed, layers=1, segments=segments)
    W = {n: dev(a, dt) for n, a in x["weights"][0].items()}
    u, vb, R = dev(x["u"], dt), dev(x["v"], dt), dev(x["R"], dt)
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    tdt = W["W_q"].dtype
    kv, kbuf, vbuf = txl.make_kv_ring(dims, w.M, tdt, capacity=w.M + w.L + capacity_extra)
    kv.start = (7 * capacity_extra) % kv.capacity
    r = txl.pos_proj(dims, R, W["W_kR"])
    ws = torch.empty(txl.kv_workspace_bytes(dims, w.M, tdt), dtype=torch.uint8, device="cuda")
    # the recompute path over a hidden-state ring
    data = torch.zeros((w.B, w.M, w.D), dtype=tdt, device="cuda")
    ring = txl.make_ring(data, 3 % w.M, 0)
    ws2 = torch.empty(txl.workspace_bytes(dims, w.M, tdt), dtype=torch.uint8, device="cuda")
    ref_mem = None
    for s in range(segments):
        h = dev(x["h0"][s], dt)
        out = torch.empty_like(h)
        txl.layer_step_kv(dims, h, kv, W, u, vb, r, out, ws)
        out2 = torch.empty_like(h)
        txl.layer_step(dims, h, ring, W, u, vb, R, out2, ws2)
        txl.mem_update(ring, h)
        ref = O.layer_step(x["h0"][s], ref_mem, x["weights"][0], x["u"], x["v"], x["R"])
        ref_mem = O.mem_update(ref_mem, x["h0"][s], w.M)
        torch.cuda.synchronize()
        assert kv.len == ref_mem.shape[1], (s, kv.len)
        e_ref, e_re = max_err(host(out), ref), max_err(host(out), host(out2))
        _say(f"  segment {s}: len {kv.len} start {kv.start}  |kv - oracle| {e_ref:.2e}  "
             f"|kv - recompute| {e_re:.2e}")
        assert e_ref <= TOL[dt], s
        assert e_re <= TOL[dt], s


@pytest.mark.parametrize("name,over,segments,extra", [
    ("tiny", {"M": 24}, 4, 0),
    ("tiny", {"M": 24, "L": 10}, 5, 13),
    ("charlm", {"B": 2, "L": 48, "M": 80, "D": 128, "H": 2, "d": 64}, 5, 22),
    ("charlm", {"B": 2, "L": 30, "M": 50, "D": 82, "H": 2, "d": 41}, 4, 7),
    ("charlm", {"B": 1, "L": 64, "M": 192, "D": 256, "H": 4, "d": 64}, 4, 0),
])
def test_kv_stream_matches_oracle(name, over, segments, extra):
    w = I.workload(name, **over)  # R_rows covers M + L
    _say(f"kv stream {w} segments={segments} capacity extra={extra}")
    _stream_case(w, segments, extra)


@pytest.mark.parametrize("over,segments", [
    ({"B": 2, "L": 1, "M": 100, "D": 128, "H": 2, "d": 64, "R_rows": 101}, 12),
    # the long-memory evaluation model's width: matrix-vector products over K = 1024
    ({"B": 1, "L": 1, "M": 300, "D": 1024, "H": 16, "d": 64, "R_rows": 301}, 6),
    # widths that are not multiples of 32: the products read zero-padded copies
    ({"B": 3, "L": 1, "M": 40, "D": 82, "H": 2, "d": 41, "R_rows": 41}, 5),
])
def test_kv_decode_one_token_at_a_time(over, segments):
    """L = 1: a memory of up to M tokens, one new token per step."""
    w = I.workload("charlm", **over)
    _say(f"kv decode {w}")
    _stream_case(w, segments=segments, capacity_extra=5, seed=4)


@pytest.mark.parametrize("dtype,over", [
    ("fp32", {"D": 32, "H": 2, "d": 16}),
    ("bf16", {"D": 82, "H": 2, "d": 41}),
    ("bf16", {"D": 512, "H": 8, "d": 64}),
])
def test_pos_proj_matches_oracle(dtype, over):
    txl = _txl()
    w = I.workload("charlm", B=1, L=8, M=120, dtype=dtype, **over)
    x = I.make_inputs(w, seed=2, layers=1, segments=1)
    dims = txl.layer_dims(1, w.L, w.D, w.H, w.d)
    R = dev(x["R"], dtype)
    W_kR = dev(x["weights"][0]["W_kR"], dtype)
    r = txl.pos_proj(dims, R, W_kR)
    torch.cuda.synchronize()
    got = host(r)  # [H, rows, d_pad]
    ref = x["R"].astype(np.float64) @ x["weights"][0]["W_kR"].astype(np.float64).T
    ref = ref.reshape(-1, w.H, w.d).transpose(1, 0, 2)
    assert max_err(got[..., :w.d], ref) <= TOL[dtype]
    assert np.all(got[..., w.d:] == 0), "padding columns must be zero"
