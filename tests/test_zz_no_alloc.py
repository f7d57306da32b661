"""txl_rel_attn_fwd_noalloc (the entry point that allocates nothing: its key-split
partials live in the library's static device scratch) against txl_rel_attn_fwd
with a caller workspace, through the C ABI.

Two calls in a row, the second with a smaller input, each compared with the
workspace entry point on the same inputs: the plans are the same (the whole
split plan fits both scratches), so the results must be bit-identical, and
within 2e-2 of the fp64 oracle.  Also: a shape with no split (no scratch), and
a shape whose split needs more than the static scratch (rejected, nothing
written).
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as O
from relative_position_memory_amd import inputs as I
from tests.gpu_util import TOL, dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _case(B, H, L, M, d, seed):
    c = I.attention_inputs(B, H, L, M, d, seed=seed, sigma=1.0, sigma_uv=0.5, dtype="bf16")
    hm = lambda x: dev(x.transpose(0, 2, 1, 3), "bf16").permute(0, 2, 1, 3)
    t = {"q": hm(c["q"]), "k": hm(c["k"]), "v": hm(c["v"]),
         "r": dev(c["r"].transpose(1, 0, 2), "bf16").permute(1, 0, 2),
         "u": dev(c["u"], "bf16"), "vb": dev(c["vb"], "bf16")}
    return c, t


def _both(txl, B, H, L, M, d, seed):
    c, t = _case(B, H, L, M, d, seed)
    need = txl.rel_attn_workspace_bytes(torch.bfloat16, B, H, L, M, d)
    print(f"no-alloc case B={B} H={H} L={L} M={M} d={d}: split scratch {need} bytes", flush=True)
    sys.stdout.flush()
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda") if need else None
    ref = torch.empty((B, L, H, d), dtype=torch.bfloat16, device="cuda")
    txl.rel_attn_fwd(t["q"], t["k"], t["v"], t["r"], t["u"], t["vb"], M, ref, workspace=ws)
    got = torch.full((B, L, H, d), float("nan"), dtype=torch.bfloat16, device="cuda")
    txl.rel_attn_fwd_noalloc(t["q"], t["k"], t["v"], t["r"], t["u"], t["vb"], M, got)
    torch.cuda.synchronize()
    return c, need, ref, got


def test_noalloc_matches_workspace_entry_point_twice():
    need_gpu()
    from relative_position_memory_amd import txl
    cap = txl.rel_attn_noalloc_max_scratch_bytes()
    assert cap == 16 << 20
    # first call: the long-memory evaluation shape (9 key parts per query tile)
    c, need, ref, got = _both(txl, 1, 16, 128, 1600, 64, seed=11)
    assert 0 < need <= cap
    assert torch.equal(got, ref)
    oracle = O.rel_attn(c["q"], c["k"], c["v"], c["r"], c["u"], c["vb"], 1600)
    assert float(np.abs(host(got) - oracle).max()) <= TOL["bf16"]
    # second call, smaller: fewer heads, shorter memory (the scratch holds the
    # previous call's partials, which this call must not read)
    c, need2, ref, got = _both(txl, 1, 3, 70, 700, 64, seed=12)
    assert 0 < need2 < need
    assert torch.equal(got, ref)
    oracle = O.rel_attn(c["q"], c["k"], c["v"], c["r"], c["u"], c["vb"], 700)
    assert float(np.abs(host(got) - oracle).max()) <= TOL["bf16"]


def test_noalloc_without_a_split():
    need_gpu()
    from relative_position_memory_amd import txl
    c, need, ref, got = _both(txl, 22, 8, 512, 512, 64, seed=13)  # the character-model shape
    assert need == 0
    assert torch.equal(got, ref)


def test_noalloc_rejects_a_split_beyond_the_static_scratch():
    need_gpu()
    from relative_position_memory_amd import txl
    B, H, L, M, d = 1, 16, 1600, 1600, 64
    need = txl.rel_attn_workspace_bytes(torch.bfloat16, B, H, L, M, d)
    assert need > txl.rel_attn_noalloc_max_scratch_bytes()
    c, t = _case(B, H, L, M, d, seed=14)
    out = torch.full((B, L, H, d), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(txl.TxlError, match="static scratch"):
        txl.rel_attn_fwd_noalloc(t["q"], t["k"], t["v"], t["r"], t["u"], t["vb"], M, out)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
