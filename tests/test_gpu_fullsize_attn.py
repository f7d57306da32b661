"""Element-wise parity of the relative attention at the workloads' full sizes.

Transformer-XL section 3.3 (the score A^rel, masked softmax, P v) and
Appendix B (key j of query i at distance mem_len + i - j).

A full-size layer step leaves the q, k, v and r it projected, and the output of
its own attention launch, in its workspace.  The oracle recomputes the whole
attention from those same bf16 q, k, v, r (every output element, all batch
rows and heads), and two GPU results are compared with it element by element:
  * the layer step's attention output (the launch inside txl_layer_step, with
    the workspace and key-split plan the step uses: at the long-memory
    evaluation shape that is 9 key parts per query tile and the merge kernel);
  * txl_rel_attn_fwd called on the same views with the workspace the benchmark
    gives it (the launch the benchmark times alone).
Also the vanilla window recompute of the per-token evaluation comparison
(section 3.1's evaluation phase, Table 9): one sequence of 3,800 tokens with an
empty memory through a layer of the long-memory evaluation model, sampled rows
from every one of its 30 query tiles against the oracle.
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from relative_position_memory_amd import inputs as I
from tests.gpu_util import TOL, dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("name", ["charlm", "wordlm", "large_eval", "large_train"])
def test_full_size_attention_every_element(name):
    need_gpu()
    from relative_position_memory_amd import txl
    w = I.workload(name)
    _say(f"full-size attention, every element: {w}")
    x = I.make_inputs(w, seed=0, layers=1, segments=1)
    W = {k: dev(v, "bf16") for k, v in x["weights"][0].items()}
    start = (w.M * 3) // 5
    data = torch.empty((w.B, w.M, w.D), dtype=torch.bfloat16, device="cuda")
    idx = torch.tensor([(start + t) % w.M for t in range(w.M)], device="cuda")
    data[:, idx] = dev(x["mem"][0], "bf16")
    ring = txl.make_ring(data, start, w.M)
    h = dev(x["h0"][0], "bf16")
    u, vb = dev(x["u"], "bf16"), dev(x["v"], "bf16")
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    ws = torch.empty(txl.workspace_bytes(dims, w.M, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(h)
    txl.layer_step(dims, h, ring, W, u, vb, dev(x["R"], "bf16"), out, ws)
    torch.cuda.synchronize()
    views = txl.workspace_views(dims, w.M, ws, torch.bfloat16)
    a_layer = host(views["a"])
    # the standalone launch, configured as the benchmark configures it
    nws = txl.rel_attn_workspace_bytes(torch.bfloat16, w.B, w.H, w.L, w.M, w.d)
    aws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
    a_alone = torch.empty((w.B, w.L, w.H, w.d), dtype=torch.bfloat16, device="cuda")
    txl.rel_attn_fwd(views["q"], views["k"], views["v"], views["r"], u, vb, w.M, a_alone,
                     workspace=aws)
    torch.cuda.synchronize()
    a_alone = host(a_alone)
    q, k, v, r = (host(views[n]) for n in ("q", "k", "v", "r"))
    _say(f"  oracle over {w.B * w.H * w.L} query rows (split workspace {nws} bytes)")
    ref = O.rel_attn(q, k, v, r, x["u"], x["v"], w.M)
    for what, got in (("layer step launch", a_layer), ("standalone launch", a_alone)):
        err = np.abs(got - ref)
        worst = np.unravel_index(int(np.argmax(err)), err.shape)
        _say(f"  {what}: max-abs error {err.max():.3e} at (b, i, h, c) = {worst}")
        assert np.all(np.isfinite(got)), what
        assert err.max() <= TOL["bf16"], what


def test_vanilla_window_layer_step_3800():
    """The vanilla side of the evaluation-speed comparison at its longest window:
    B 1, d_model 1024, 16 heads of 64, L = 3800, empty memory (a ring of capacity
    1, as the benchmark passes it), the benchmark's workspace.  Rows sampled from
    each of the 30 query tiles of 128 (first, middle, last) against the oracle."""
    need_gpu()
    from relative_position_memory_amd import txl
    w = I.workload("large_eval", L=3800, M=0, n_layers=1, n_segments=1)
    _say(f"vanilla window layer step: {w}")
    x = I.make_inputs(w, seed=0)
    W = {k: dev(v, "bf16") for k, v in x["weights"][0].items()}
    h = dev(x["h0"][0], "bf16")
    empty = txl.make_ring(torch.zeros((1, 1, w.D), dtype=torch.bfloat16, device="cuda"), 0, 0)
    dims = txl.layer_dims(w.B, w.L, w.D, w.H, w.d)
    ws = torch.empty(txl.workspace_bytes(dims, 1, torch.bfloat16), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty_like(h)
    txl.layer_step(dims, h, empty, W, dev(x["u"], "bf16"), dev(x["v"], "bf16"),
                   dev(x["R"], "bf16"), out, ws)
    torch.cuda.synchronize()
    got = host(out)
    qs = sorted({min(w.L - 1, 128 * t + o) for t in range((w.L + 127) // 128) for o in (0, 61, 127)})
    assert len({i // 128 for i in qs}) == 30
    rows, ref = O.layer_step_rows(x["h0"][0], None, x["weights"][0], x["u"], x["v"], x["R"],
                                  [(0, i) for i in qs])
    errs = [float(np.abs(got[b, i] - ref[t]).max()) for t, (b, i) in enumerate(rows)]
    _say(f"  {len(rows)} rows, max-abs error {max(errs):.3e}")
    assert np.all(np.isfinite(got))
    assert max(errs) <= TOL["bf16"], [(r, e) for r, e in zip(rows, errs) if e > TOL["bf16"]]
