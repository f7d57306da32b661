"""txl_stack_fwd: the layer stack over several segments, on one or more streams.

The recurrence (Transformer-XL section 3.2) over the layer of section 3.3: for
every segment, each layer reads the previous layer's output and its own memory
as the previous segment left it, then caches its input.  The schedule across
streams must not change a single bit: every result is compared with the serial
composition of txl_layer_step and txl_mem_update (outputs, ring contents and
ring states), and the fp32 stack with the oracle's recurrence."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from relative_position_memory_amd import inputs as I
from tests.gpu_util import TOL, dev, host, max_err, ring_logical

pytestmark = pytest.mark.gpu

SHAPES = {
    # name: (workload, overrides)
    "fp32-tiny": ("tiny", {"M": 24, "n_layers": 3, "n_segments": 4}),
    "bf16-charlm-small": ("charlm", {"B": 2, "L": 40, "M": 56, "D": 128, "H": 2, "d": 64,
                                     "n_layers": 3, "n_segments": 5}),
    # ragged head size and d_model (zero-padded operand copies), memory shorter than L
    "bf16-ragged": ("wordlm", {"B": 3, "L": 30, "M": 20, "D": 82, "H": 2, "d": 41,
                               "n_layers": 2, "n_segments": 4}),
}


def _say(*a):
    print(*a, flush=True)


def _setup(name):
    from relative_position_memory_amd import txl
    wl, over = SHAPES[name]
    w = I.workload(wl, **over)
    dtype = "fp32" if w.dtype == "fp32" else "bf16"
    x = I.make_inputs(w, seed=5)
    Ws = [{k: dev(a, dtype) for k, a in lw.items()} for lw in x["weights"]]
    lws = [txl.layer_weights(W) for W in Ws]
    u, vb, R = dev(x["u"], dtype), dev(x["v"], dtype), dev(x["R"], dtype)
    h_in = dev(np.stack(x["h0"][:w.n_segments]), dtype)
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    # rings start half full (start 3, so the logical rows wrap round the slots)
    mem0 = [dev(m, dtype) for m in x["mem"]]
    return w, dtype, x, Ws, lws, u, vb, R, h_in, dims, mem0


def _rings(w, mem0):
    from relative_position_memory_amd import txl
    datas, rings = [], []
    for m in mem0:
        dd = torch.zeros_like(m)
        n0 = w.M // 2
        idx = [(3 + t) % w.M for t in range(n0)]
        dd[:, idx] = m[:, w.M - n0:]
        datas.append(dd)
        rings.append(txl.make_ring(dd, 3 % w.M, n0))
    return datas, rings


def _serial(w, lws, u, vb, R, h_in, dims, mem0, tdt):
    from relative_position_memory_amd import txl
    datas, rings = _rings(w, mem0)
    ws = torch.empty(txl.workspace_bytes(dims, w.M, tdt), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(h_in)
    for s in range(w.n_segments):
        h = h_in[s]
        for n in range(w.n_layers):
            o = torch.empty_like(h)
            txl.layer_step(dims, h, rings[n], lws[n], u, vb, R, o, ws)
            txl.mem_update(rings[n], h)
            h = o
        out[s].copy_(h)
    torch.cuda.synchronize()
    return out, datas, rings


@pytest.mark.parametrize("name", list(SHAPES))
@pytest.mark.parametrize("n_streams", [1, 2, 3])
def test_stack_is_bit_identical_to_the_serial_order(name, n_streams):
    from relative_position_memory_amd import txl
    w, dtype, x, Ws, lws, u, vb, R, h_in, dims, mem0 = _setup(name)
    tdt = h_in.dtype
    _say(f"stack {name} {w.n_layers} layers x {w.n_segments} segments, {n_streams} streams")
    ref, ref_datas, ref_rings = _serial(w, lws, u, vb, R, h_in, dims, mem0, tdt)
    datas, rings = _rings(w, mem0)
    streams = [torch.cuda.current_stream()] + [torch.cuda.Stream() for _ in range(n_streams - 1)]
    ws = torch.empty(txl.stack_workspace_bytes(dims, w.M, tdt, n_streams), dtype=torch.uint8,
                     device="cuda")
    out = torch.full_like(h_in, float("nan"))
    for rep in range(2):  # a second call continues the recurrence from where the first left it
        txl.stack_fwd(streams, dims, h_in, rings, lws, u, vb, R, out, ws)
        torch.cuda.synchronize()
        if rep == 0:
            assert torch.equal(out, ref), "outputs differ from the serial order"
            for n in range(w.n_layers):
                assert (rings[n].start, rings[n].len) == (ref_rings[n].start, ref_rings[n].len)
                assert torch.equal(ring_logical(datas[n], rings[n]),
                                   ring_logical(ref_datas[n], ref_rings[n])), n
            # the serial order again from here, for the second call
            ref2 = torch.empty_like(h_in)
            wsl = torch.empty(txl.workspace_bytes(dims, w.M, tdt), dtype=torch.uint8, device="cuda")
            for s in range(w.n_segments):
                h = h_in[s]
                for n in range(w.n_layers):
                    o = torch.empty_like(h)
                    txl.layer_step(dims, h, ref_rings[n], lws[n], u, vb, R, o, wsl)
                    txl.mem_update(ref_rings[n], h)
                    h = o
                ref2[s].copy_(h)
            torch.cuda.synchronize()
        else:
            assert torch.equal(out, ref2), "second call differs from the serial order"
            for n in range(w.n_layers):
                assert torch.equal(ring_logical(datas[n], rings[n]),
                                   ring_logical(ref_datas[n], ref_rings[n])), n


def test_fp32_stack_matches_the_oracle_recurrence():
    """fp32: the stack's per-segment outputs against the oracle run of the same
    recurrence from the same initial memories (errors compound over layers, still
    far inside the fp32 bar)."""
    from relative_position_memory_amd import txl
    w, dtype, x, Ws, lws, u, vb, R, h_in, dims, mem0 = _setup("fp32-tiny")
    datas, rings = _rings(w, mem0)
    ws = torch.empty(txl.stack_workspace_bytes(dims, w.M, torch.float32, 2), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(h_in)
    txl.stack_fwd([None, torch.cuda.Stream()], dims, h_in, rings, lws, u, vb, R, out, ws)
    torch.cuda.synchronize()
    n0 = w.M // 2
    mems = [np.asarray(m, np.float64)[:, w.M - n0:] for m in x["mem"]]
    for s in range(w.n_segments):
        h = np.asarray(x["h0"][s], np.float64)
        for n in range(w.n_layers):
            y = O.layer_step(h, mems[n], x["weights"][n], x["u"], x["v"], x["R"])
            mems[n] = O.mem_update(mems[n], h, w.M)
            h = y
        err = max_err(host(out[s]), h)
        _say(f"  segment {s}: max-abs error {err:.2e}")
        assert err <= TOL["fp32"], s


def test_bad_arguments_leave_the_rings_alone():
    from relative_position_memory_amd import txl
    w, dtype, x, Ws, lws, u, vb, R, h_in, dims, mem0 = _setup("bf16-charlm-small")
    datas, rings = _rings(w, mem0)
    before = [(r.start, r.len) for r in rings]
    ws = torch.empty(txl.stack_workspace_bytes(dims, w.M, h_in.dtype, 2) - 256,
                     dtype=torch.uint8, device="cuda")
    out = torch.empty_like(h_in)
    with pytest.raises(txl.TxlError) as e:
        txl.stack_fwd([None, None], dims, h_in, rings, lws, u, vb, R, out, ws)
    assert e.value.status == txl.EWORKSPACE
    assert [(r.start, r.len) for r in rings] == before
