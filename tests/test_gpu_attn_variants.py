"""Both bf16 matrix-core attention kernels on the same cases, against the oracle.

The library picks the 64-query kernel (three 4-wave workgroups per CU, no key
split) or the 128-query kernel (key splits planned for few query tiles) by
shape; txl_attn_variant forces either one, so each runs here on the ragged and
edge shapes that the by-shape rule would send to only one of them: query and key
tails, a wave with no query rows, head sizes 16 to 64 in padded rows, an empty
memory, a key ring (cached keys), the softmax statistics the backward takes from
the saved forward, and a layer step.  Same bars as the other parity tests."""
import pytest

from tests import test_gpu_bwd as PB
from tests import test_gpu_kvcache as PK
from tests import test_gpu_parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(params=[1, 2], ids=["q64", "q128"])
def variant(request):
    P.need_gpu()
    from relative_position_memory_amd import txl
    old = txl.attn_variant(request.param)
    yield request.param
    txl.attn_variant(old)


@pytest.mark.parametrize("B,H,L,M,d,dp", [
    (1, 2, 128, 128, 64, 64),     # whole tiles
    (1, 2, 513, 511, 64, 64),     # ragged query and key tails
    (1, 2, 65, 63, 64, 64),       # one query past a tile; the last tile's waves 1-3 idle
    (1, 2, 33, 1, 64, 64),        # waves without rows in the only tile
    (1, 1, 128, 1600, 64, 64),    # long memory, skinny query block
    (2, 2, 384, 384, 64, 64),
    (1, 2, 1, 0, 64, 64),         # a single query, no memory
    (1, 2, 1, 200, 64, 64),
    (1, 1, 300, 0, 32, 32),       # no memory, d 32
    (1, 2, 200, 50, 41, 48),      # ragged head size in padded rows
    (2, 1, 150, 150, 41, 48),     # the word model's head size and segment
    (1, 2, 70, 130, 16, 16),
])
def test_attn_layouts(variant, B, H, L, M, d, dp):
    P.test_attn_matrix_core_layouts(B, H, L, M, d, dp)


@pytest.mark.parametrize("dtype,B,H,L,M,d,layout", [
    ("bf16", 2, 2, 130, 70, 64, "bthd"),
    ("bf16", 2, 2, 130, 70, 64, "bhtd"),
    ("bf16", 1, 3, 150, 150, 41, "bthd"),
    ("bf16", 2, 1, 200, 0, 64, "bhtd"),
    ("bf16", 1, 2, 77, 333, 48, "bhtd"),
])
def test_attn_strided(variant, dtype, B, H, L, M, d, layout):
    P.test_attn_shapes(dtype, B, H, L, M, d, layout)


@pytest.mark.parametrize("over,mem_len,start", [
    ({"B": 2, "L": 100, "M": 130, "D": 96, "H": 3, "d": 32}, 130, 77),
    ({"B": 3, "L": 50, "M": 50, "D": 82, "H": 2, "d": 41}, 50, 11),
    ({"B": 1, "L": 33, "M": 200, "D": 128, "H": 2, "d": 64}, 17, 190),
])
def test_layer_step(variant, over, mem_len, start):
    P.test_layer_step_bf16(over, mem_len, start)


@pytest.mark.parametrize("name,over,segments,extra", [
    ("charlm", {"B": 2, "L": 48, "M": 80, "D": 128, "H": 2, "d": 64}, 5, 22),
    ("charlm", {"B": 2, "L": 30, "M": 50, "D": 82, "H": 2, "d": 41}, 4, 7),
])
def test_kv_ring(variant, name, over, segments, extra):
    PK.test_kv_stream_matches_oracle(name, over, segments, extra)


@pytest.mark.parametrize("dtype,name,over,mem_len,start", [
    ("bf16", "charlm", {"B": 2, "L": 96, "M": 160, "D": 192, "H": 3, "d": 64}, 160, 37),
    ("bf16", "charlm", {"B": 3, "L": 50, "M": 50, "D": 82, "H": 2, "d": 41}, 50, 11),
])
def test_saved_forward_statistics(variant, dtype, name, over, mem_len, start):
    PB.test_layer_step_bwd_saved_matches_recompute(dtype, name, over, mem_len, start)
