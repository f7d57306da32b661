"""Parity at the workloads' full sizes, in the launch configuration bench.py uses.

One layer step per workload with a full memory placed at a wrapped ring offset;
the oracle evaluates sampled output rows one by one (same fp64 arithmetic as the
full oracle, cheaper), and the memory update that follows is checked bit-exactly
on every row.  Sampled rows cover both batch ends, the first and last query of
the segment and query-tile edges.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from relative_position_memory_amd import inputs as I
from tests.gpu_util import TOL, dev, host, need_gpu, ring_logical

pytestmark = pytest.mark.gpu


def _rows(w):
    qs = sorted({0, 1, 31, 32, 127, 128, w.L // 2, w.L - 2, w.L - 1} & set(range(w.L)))
    bs = sorted({0, w.B // 2, w.B - 1})
    return [(b, i) for b in bs for i in qs]


@pytest.mark.parametrize("name", ["charlm", "wordlm", "large_eval", "large_train"])
def test_full_size_layer_step(name):
    need_gpu()
    from relative_position_memory_amd import txl
    w = I.workload(name)
    print(f"full size {w}", flush=True)
    sys.stdout.flush()
    x = I.make_inputs(w, seed=0, layers=1, segments=1)
    W = {k: dev(v, "bf16") for k, v in x["weights"][0].items()}
    start = (w.M * 5) // 7
    data = torch.empty((w.B, w.M, w.D), dtype=torch.bfloat16, device="cuda")
    mem = dev(x["mem"][0], "bf16")
    idx = torch.tensor([(start + t) % w.M for t in range(w.M)], device="cuda")
    data[:, idx] = mem
    ring = txl.make_ring(data, start, w.M)
    h = dev(x["h0"][0], "bf16")
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    ws = torch.empty(txl.workspace_bytes(dims, w.M, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(h)
    txl.layer_step(dims, h, ring, W, dev(x["u"], "bf16"), dev(x["v"], "bf16"),
                   dev(x["R"], "bf16"), out, ws)
    txl.mem_update(ring, h)
    torch.cuda.synchronize()
    got = host(out)
    rows, ref = O.layer_step_rows(x["h0"][0], x["mem"][0], x["weights"][0], x["u"], x["v"],
                                  x["R"], _rows(w))
    errs = [float(np.abs(got[b, i] - ref[t]).max()) for t, (b, i) in enumerate(rows)]
    print(f"  sampled rows {len(rows)}, max-abs error {max(errs):.3e}", flush=True)
    assert max(errs) <= TOL["bf16"], list(zip(rows, errs))
    assert np.all(np.isfinite(got))
    # memory after the update: last M rows of [memory ; h], bit-exact
    want = O.mem_update(x["mem"][0], x["h0"][0], w.M)
    np.testing.assert_array_equal(host(ring_logical(data, ring)), want)
