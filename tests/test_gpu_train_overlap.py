"""The training step's two-stream schedule (bench.train_runner): the backward of
segment s beside the forward of segment s + 1, with the stop-gradient memory of
Transformer-XL section 3.2.  Against the same work on one stream: the stack's
outputs are bit-identical (the forward kernels see the same operands), and the
gradients of the last segment agree up to the order of the atomic sums in the
backward's position-gradient kernel."""
import numpy as np
import pytest
import torch

from relative_position_memory_amd import inputs as I
from tests.gpu_util import need_gpu

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("over", [
    {"B": 2, "L": 64, "M": 64, "D": 128, "H": 2, "d": 64, "n_layers": 3, "n_segments": 4},
    # memory longer than the segment: each ring keeps rows of the previous memory
    {"B": 2, "L": 40, "M": 96, "D": 256, "H": 4, "d": 64, "n_layers": 2, "n_segments": 5},
])
def test_two_stream_training_step_matches_one_stream(over):
    need_gpu()
    import bench
    w = I.workload("charlm", **over)
    x = I.make_inputs(w, seed=3)
    print(f"train schedule {w}", flush=True)
    cur = torch.cuda.current_stream()
    step1, box1, out1, _ = bench.train_runner(w, x, [cur])
    step2, box2, out2, _ = bench.train_runner(w, x, [cur, torch.cuda.Stream()])
    for _ in range(2):  # the second step starts again from the initial memories
        step1()
        step2()
        torch.cuda.synchronize()
        assert torch.equal(out1, out2), "stack outputs differ"
        for k, g1 in box1["grads"].items():
            g2 = box2["grads"][k]
            a, b = g1.cpu().numpy().astype(np.float64), g2.cpu().numpy().astype(np.float64)
            scale = max(1.0, float(np.max(np.abs(a))))
            assert float(np.max(np.abs(a - b))) <= 1e-5 * scale, k
