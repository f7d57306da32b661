"""Position-wise feed-forward (txl_pos_ff) and the full layer stack with it,
against the oracle (fp32 within 1e-4, bf16 within 2e-2, element by element).
The weights are drawn with std 1/sqrt(fan_in) so that the feed-forward branch
is as large as the residual and an error in it cannot hide under the LayerNorm."""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from relative_position_memory_amd import inputs as I
from tests.gpu_util import TOL, dev, host, max_err

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _ff_weights(rng, D, Di, dtype):
    W = {"W1": rng.standard_normal((Di, D)) / np.sqrt(D),
         "b1": 0.5 * rng.standard_normal(Di),
         "W2": rng.standard_normal((D, Di)) / np.sqrt(Di),
         "b2": 0.5 * rng.standard_normal(D),
         "gamma": 1 + 0.2 * rng.standard_normal(D),
         "beta": 0.2 * rng.standard_normal(D)}
    W = {k: v.astype(np.float32) for k, v in W.items()}
    if dtype == "bf16":
        W = {k: I.round_bf16(v) for k, v in W.items()}
    return W


@pytest.mark.parametrize("dtype,rows,D,Di", [
    ("fp32", 37, 40, 72),       # generic kernels
    ("bf16", 300, 512, 2048),   # matrix cores, fused second layer + LayerNorm
    ("bf16", 77, 96, 200),      # ragged rows; d_inner 200 read as a zero-padded 224
    ("bf16", 150, 96, 256),     # D % 64 != 0: the fused kernel's ragged form, with bias
    ("bf16", 300, 410, 1640),   # the 10-head word-level model's widths, both padded
    ("bf16", 100, 1024, 4096),  # D > 512: unfused LayerNorm
    ("bf16", 3, 512, 2048),     # a decode step's rows: matrix-vector products
    ("bf16", 1, 1024, 4096),    # one token of the long-memory evaluation shape
    ("bf16", 4, 136, 200),      # 4 rows, column counts that end mid-workgroup
    ("bf16", 5, 512, 2048),     # 5 rows: the skinny matrix-core path
])
def test_pos_ff_matches_oracle(dtype, rows, D, Di):
    from relative_position_memory_amd import txl
    rng = np.random.default_rng(rows + D)
    W = _ff_weights(rng, D, Di, dtype)
    x = rng.standard_normal((rows, D)).astype(np.float32)
    if dtype == "bf16":
        x = I.round_bf16(x)
    _say(f"pos_ff {dtype} rows={rows} D={D} Di={Di}")
    Wd = {k: dev(v, dtype) for k, v in W.items()}
    xd = dev(x, dtype)
    out = torch.empty_like(xd)
    txl.pos_ff(xd, Wd["W1"], Wd["b1"], Wd["W2"], Wd["b2"], Wd["gamma"], Wd["beta"], out)
    torch.cuda.synchronize()
    ref = O.pos_ff(x, W["W1"], W["b1"], W["W2"], W["b2"], W["gamma"], W["beta"])
    err = max_err(host(out), ref)
    _say(f"  max-abs error {err:.2e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_full_stack_with_feed_forward(dtype):
    """N = 2 layers x S = 3 segments: each layer is the attention sublayer then the
    feed-forward; each memory caches its layer's input; against the oracle."""
    from relative_position_memory_amd import txl
    name = "tiny" if dtype == "fp32" else "charlm"
    over = {"M": 24, "n_layers": 2, "n_segments": 3} if dtype == "fp32" else \
        {"B": 2, "L": 40, "M": 56, "D": 128, "H": 2, "d": 64, "n_layers": 2, "n_segments": 3}
    w = I.workload(name, **over)
    x = I.make_inputs(w, seed=9)
    rng = np.random.default_rng(10)
    Di = 4 * w.D
    ffs = [_ff_weights(rng, w.D, Di, dtype) for _ in range(w.n_layers)]
    _say(f"stack with feed-forward {w} d_inner={Di}")
    Ws = [{n: dev(a, dtype) for n, a in lw.items()} for lw in x["weights"]]
    Fs = [{n: dev(a, dtype) for n, a in f.items()} for f in ffs]
    tdt = Ws[0]["W_q"].dtype
    datas = [torch.zeros((w.B, w.M, w.D), dtype=tdt, device="cuda") for _ in range(w.n_layers)]
    rings = [txl.make_ring(dd, 0, 0) for dd in datas]
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    ws = torch.empty(txl.workspace_bytes(dims, w.M, tdt), dtype=torch.uint8, device="cuda")
    u, vb, R = dev(x["u"], dtype), dev(x["v"], dtype), dev(x["R"], dtype)
    # Each layer is checked on the inputs the GPU actually gave it (its h and the
    # memory of the h it cached), so bf16 rounding does not compound over layers.
    ref_mems = [None] * w.n_layers
    for s in range(w.n_segments):
        h = dev(x["h0"][s], dtype)
        for n in range(w.n_layers):
            href = host(h).astype(np.float64)
            o = torch.empty_like(h)
            txl.layer_step(dims, h, rings[n], Ws[n], u, vb, R, o, ws)
            txl.mem_update(rings[n], h)
            hn = torch.empty_like(h)
            F = Fs[n]
            txl.pos_ff(o, F["W1"], F["b1"], F["W2"], F["b2"], F["gamma"], F["beta"], hn)
            oref = O.layer_step(href, ref_mems[n], x["weights"][n], x["u"], x["v"], x["R"])
            ref_mems[n] = O.mem_update(ref_mems[n], href, w.M)
            f = ffs[n]
            # the GPU path carries o in the working dtype between the two sublayers
            o_in = host(o)
            href_next = O.pos_ff(o_in, f["W1"], f["b1"], f["W2"], f["b2"], f["gamma"], f["beta"])
            torch.cuda.synchronize()
            e_o, e_h = max_err(host(o), oref), max_err(host(hn), href_next)
            _say(f"  segment {s} layer {n}: |o - oracle| {e_o:.2e}  |h - oracle| {e_h:.2e}")
            assert e_o <= TOL[dtype] and e_h <= TOL[dtype], (s, n)
            h = hn
