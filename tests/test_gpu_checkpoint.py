"""Checkpoint and resume of the recurrence (Transformer-XL section 3.2: between
segments the cached memory of each layer is the only state; section 3.3: the
score depends on relative distances only, so where a row sits in the ring does
not matter).

An N-layer stack runs S segments with the memory update after every layer.
The same stream is then run again, stopped after segment 2: each layer's
memory is read back in logical order (oldest row first), written to a file,
loaded into fresh ring buffers at a different physical offset, and the
remaining segments run from there.  Every output of the resumed segments must
be bit-identical to the uninterrupted run's.
"""
import sys

import numpy as np
import pytest
import torch

from relative_position_memory_amd import inputs as I
from tests.gpu_util import dev, need_gpu, ring_logical

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("dtype,over", [
    ("bf16", {"B": 2, "L": 48, "M": 80, "D": 128, "H": 2, "d": 64}),
    ("fp32", {"B": 2, "L": 20, "M": 36, "D": 40, "H": 2, "d": 12}),
])
def test_resume_from_saved_memory_is_bit_identical(dtype, over, tmp_path):
    need_gpu()
    from relative_position_memory_amd import txl
    w = I.workload("charlm", dtype=dtype, n_layers=2, n_segments=5, **over)
    _say(f"checkpoint/resume {w}")
    x = I.make_inputs(w, seed=9)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    Ws = [{n: dev(a, dtype) for n, a in lw.items()} for lw in x["weights"]]
    u, vb, R = dev(x["u"], dtype), dev(x["v"], dtype), dev(x["R"], dtype)
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    ws = torch.empty(txl.workspace_bytes(dims, w.M, tdt), dtype=torch.uint8, device="cuda")

    def run(rings, segs):
        outs = []
        for s in segs:
            h = dev(x["h0"][s], dtype)
            for n in range(w.n_layers):
                out = torch.empty_like(h)
                txl.layer_step(dims, h, rings[n][1], Ws[n], u, vb, R, out, ws)
                txl.mem_update(rings[n][1], h)
                h = out
            outs.append(h.clone())
        torch.cuda.synchronize()
        return outs

    def fresh(start, logical=None):
        data = torch.zeros((w.B, w.M, w.D), dtype=tdt, device="cuda")
        n = 0 if logical is None else logical.shape[1]
        for t in range(n):
            data[:, (start + t) % w.M] = logical[:, t]
        return [data, txl.make_ring(data, start if n else 0, n)]

    # uninterrupted: empty memory at segment 0, five segments
    full = run([fresh(0) for _ in range(w.n_layers)], range(5))
    # interrupted after segment 2 (three segments run), memory saved to a file
    rings = [fresh(0) for _ in range(w.n_layers)]
    first = run(rings, range(3))
    for a, b in zip(first, full[:3]):
        assert torch.equal(a, b)
    path = tmp_path / "memory.npz"
    saved = {f"layer{n}": ring_logical(d, r).float().cpu().numpy() for n, (d, r) in enumerate(rings)}
    np.savez(path, **saved)
    assert all(v.shape[1] == w.M for v in saved.values())  # 3 L >= M: the memory is full
    # resume in new buffers, each layer's rows placed at another physical offset
    loaded = np.load(path)
    starts = [(w.M * 2) // 3, w.M - 1]
    resumed = [fresh(starts[n], torch.from_numpy(loaded[f"layer{n}"]).to(tdt).cuda())
               for n in range(w.n_layers)]
    rest = run(resumed, range(3, 5))
    for s, (a, b) in enumerate(zip(rest, full[3:]), start=3):
        assert torch.equal(a, b), f"segment {s} differs after resume"
