"""Host-side checks of the C ABI: the library loads, exports every function
include/txl.h declares, and rejects bad arguments before touching a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "txl.h")
LIB = os.path.join(ROOT, "relative_position_memory_amd", "libtxl.so")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(txl_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libtxl.so is not built (run __graft_entry__.build())")
    return ctypes.CDLL(LIB)


def test_header_declares_the_entry_points():
    names = _declared()
    for n in ("txl_rel_attn_fwd", "txl_layer_step", "txl_mem_update",
              "txl_layer_workspace_bytes", "txl_status_string"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared():
        assert hasattr(lib, n), n


def test_status_strings(lib):
    lib.txl_status_string.restype = ctypes.c_char_p
    for s in (0, -1, -2, -3, -4, 7):
        assert lib.txl_status_string(s)


def test_argument_errors_need_no_gpu():
    from relative_position_memory_amd import txl
    lib = txl._lib
    i64 = ctypes.c_int64
    # NULL tensors -> EINVAL, before any HIP call
    args = [None, txl.BF16, 1, 1, 4, 0, 16] + [None, 16, 16, 16] + [None, None, 16, 16, 16] \
        + [None, 16, 16, 4] + [None, None, 0.25] + [None, 16, 16, 16] + [None, None, 0]
    assert lib.txl_rel_attn_fwd(*args) == txl.EINVAL
    # unsupported dtype and d_head
    bad = list(args)
    bad[1] = 7
    assert lib.txl_rel_attn_fwd(*bad) == txl.EUNSUPPORTED
    bad = list(args)
    bad[6] = 200
    fake = ctypes.c_void_p(0x1000)
    for idx in (7, 11, 12, 16, 20, 21, 23):
        bad[idx] = fake
    assert lib.txl_rel_attn_fwd(*bad) == txl.EUNSUPPORTED
    assert "d_head" in txl.status_string(txl.EUNSUPPORTED)
    # workspace size is a pure host computation
    dims = txl.layer_dims(22, 512, 512, 8, 64)
    n = txl.workspace_bytes(dims, 512, __import__("torch").bfloat16)
    assert n >= 2 * (22 * 8 * 1024 * 64 * 2)
    assert lib.txl_layer_workspace_bytes(ctypes.byref(txl.layer_dims(1, 1, 1, 1, 300)), 1, 1) == 0
    # ring state errors
    ring = txl.Ring(0x1000, 4, 5, 0)
    assert lib.txl_mem_update(None, txl.BF16, ctypes.byref(ring), 1, 8, fake, 2) == txl.EINVAL
    ring = txl.Ring(0x1000, 4, 0, 0)
    assert lib.txl_mem_update(None, txl.BF16, ctypes.byref(ring), 1, 8, None, 2) == txl.EINVAL
    # h_new overlapping the ring
    assert lib.txl_mem_update(None, txl.BF16, ctypes.byref(ring), 1, 8,
                              ctypes.c_void_p(0x1000 + 8), 2) == txl.EINVAL
    assert ring.start == 0 and ring.len == 0


def test_kv_path_argument_errors_need_no_gpu():
    from relative_position_memory_amd import txl
    lib = txl._lib
    dims = txl.layer_dims(2, 16, 64, 2, 32)
    assert lib.txl_kv_ring_bytes(ctypes.byref(dims), 40, txl.BF16) == 2 * 2 * 40 * 32 * 2
    assert lib.txl_kv_ring_bytes(ctypes.byref(dims), 0, txl.BF16) == 0
    assert lib.txl_layer_kv_workspace_bytes(ctypes.byref(dims), 24, txl.FP32) > 0
    fake = ctypes.c_void_p(0x100000)
    W = txl.LayerWeights(*([fake] * 7))
    good = dict(k=fake, v=ctypes.c_void_p(0x200000), capacity=40, start=0, len=0, mem_max=24)

    def call(**ring_over):
        kv = txl.KVRing(**{**good, **ring_over})
        return lib.txl_layer_step_kv(None, txl.BF16, ctypes.byref(dims), fake, ctypes.byref(kv),
                                     ctypes.byref(W), fake, fake, fake, 64, fake,
                                     ctypes.c_void_p(0x400000), 1 << 20)
    assert call(capacity=39) == txl.EINVAL        # capacity < mem_max + L
    assert call(len=25) == txl.EINVAL             # len > mem_max
    assert call(start=40) == txl.EINVAL           # start outside the ring
    assert call(k=None) == txl.EINVAL
    # a failing call leaves the ring state alone
    kv = txl.KVRing(**{**good, "len": 25})
    lib.txl_layer_step_kv(None, txl.BF16, ctypes.byref(dims), fake, ctypes.byref(kv),
                          ctypes.byref(W), fake, fake, fake, 64, fake, fake, 1 << 20)
    assert (kv.start, kv.len) == (0, 25)
    # r too short for len + L
    kv = txl.KVRing(**{**good, "len": 20})
    assert lib.txl_layer_step_kv(None, txl.BF16, ctypes.byref(dims), fake, ctypes.byref(kv),
                                 ctypes.byref(W), fake, fake, fake, 35, fake,
                                 ctypes.c_void_p(0x400000), 1 << 20) == txl.EINVAL
    assert lib.txl_pos_proj(None, txl.BF16, ctypes.byref(dims), None, 64, fake, fake) == txl.EINVAL


def test_pos_ff_argument_errors_need_no_gpu():
    from relative_position_memory_amd import txl
    lib = txl._lib
    # hidden activations (bf16) + the fp32 pre-LayerNorm rows, each rounded up to 256 bytes
    assert lib.txl_pos_ff_workspace_bytes(10, 64, 256, txl.BF16) == 5120 + 2560
    assert lib.txl_pos_ff_workspace_bytes(0, 64, 256, txl.BF16) == 0
    fake = ctypes.c_void_p(0x100000)
    args = [None, txl.BF16, 10, 64, 256] + [fake] * 7 + [ctypes.c_float(1e-5), ctypes.c_void_p(0x900000),
                                                         ctypes.c_void_p(0xa00000), 1 << 20]
    bad = list(args)
    bad[5] = None                      # x
    assert lib.txl_pos_ff(*bad) == txl.EINVAL
    bad = list(args)
    bad[2] = 0                         # rows
    assert lib.txl_pos_ff(*bad) == txl.EINVAL
    bad = list(args)
    bad[1] = 5                         # dtype
    assert lib.txl_pos_ff(*bad) == txl.EUNSUPPORTED
    bad = list(args)
    bad[-1] = 16                       # workspace too small
    assert lib.txl_pos_ff(*bad) == txl.EWORKSPACE


def test_saved_state_argument_errors_need_no_gpu():
    """txl_layer_step_save / txl_layer_step_bwd_saved reject a missing, unaligned,
    short or overlapping saved state before any HIP call."""
    from relative_position_memory_amd import txl
    lib = txl._lib
    dims = txl.layer_dims(2, 16, 64, 2, 32)
    nsv = lib.txl_layer_saved_bytes(ctypes.byref(dims), 16, txl.BF16)
    assert nsv >= lib.txl_layer_workspace_bytes(ctypes.byref(dims), 16, txl.BF16) + 2 * 2 * 16 * 4
    assert lib.txl_layer_saved_bytes(ctypes.byref(txl.layer_dims(0, 16, 64, 2, 32)), 16,
                                     txl.BF16) == 0
    fake = ctypes.c_void_p(0x100000)
    W = txl.LayerWeights(*([fake] * 7))
    ring = txl.Ring(0x200000, 16, 0, 16)
    h_in, h_out = ctypes.c_void_p(0x300000), ctypes.c_void_p(0x400000)

    def save(sv):
        return lib.txl_layer_step_save(None, txl.BF16, ctypes.byref(dims), h_in,
                                       ctypes.byref(ring), ctypes.byref(W), fake, fake, fake, 64,
                                       h_out, ctypes.byref(sv) if sv is not None else None)

    assert save(None) == txl.EINVAL
    assert save(txl.LayerSaved(0x10000010, nsv, 0, 0)) == txl.EINVAL          # unaligned
    assert save(txl.LayerSaved(0x10000000, nsv - 256, 0, 0)) == txl.EWORKSPACE  # short
    assert save(txl.LayerSaved(0x300000 - 256, nsv, 0, 0)) == txl.EINVAL        # over h_in
    grads = txl.LayerGrads(*([ctypes.c_void_p(0x500000 + 0x10000 * i) for i in range(10)]))
    assert lib.txl_layer_step_bwd_saved(None, txl.BF16, ctypes.byref(dims), h_in,
                                        ctypes.byref(ring), ctypes.byref(W), fake, fake, fake,
                                        64, fake, None, ctypes.byref(grads),
                                        ctypes.c_void_p(0x20000000), 1 << 30) == txl.EINVAL

    # a state saved with the ring at (start 0, len 16): the backward refuses the
    # same ring after a memory update (start 5) and a different h_in
    def saved_as(**over):
        f = dict(data=0x10000000, bytes=nsv, has_lse=1, has_y=0, mem_data=0x200000,
                 mem_capacity=16, mem_start=0, mem_len=16, h_in=0x300000, B=2, L=16,
                 d_model=64, n_head=2, d_head=32, dtype=txl.BF16)
        f.update(over)
        return txl.LayerSaved(**f)

    def bwd(sv, rg):
        return lib.txl_layer_step_bwd_saved(None, txl.BF16, ctypes.byref(dims), h_in,
                                            ctypes.byref(rg), ctypes.byref(W), fake, fake, fake,
                                            64, fake, ctypes.byref(sv), ctypes.byref(grads),
                                            ctypes.c_void_p(0x20000000), 1 << 30)

    moved = txl.Ring(0x200000, 16, 5, 16)
    assert bwd(saved_as(), moved) == txl.EINVAL
    assert "memory differs" in txl.status_string(txl.EINVAL)
    assert bwd(saved_as(h_in=0x310000), ring) == txl.EINVAL
    assert "h_in" in txl.status_string(txl.EINVAL)
    assert bwd(saved_as(d_model=128), ring) == txl.EINVAL


def test_noalloc_entry_point_checks_need_no_gpu():
    """txl_rel_attn_fwd_noalloc: bad arguments and a split larger than the static
    scratch are rejected on the host, before any HIP call."""
    from relative_position_memory_amd import txl
    lib = txl._lib
    assert txl.rel_attn_noalloc_max_scratch_bytes() == 16 << 20
    args = [None, txl.BF16, 1, 1, 4, 0, 16] + [None, 16, 16, 16] + [None, None, 16, 16, 16] \
        + [None, 16, 16, 4] + [None, None, 0.25] + [None, 16, 16, 16] + [None]
    assert lib.txl_rel_attn_fwd_noalloc(*args) == txl.EINVAL
    # B 1, H 16, L = M = 1600, d 64, head-major bf16: the split plan needs more
    # than 16 MiB of partials
    B, H, L, M, d = 1, 16, 1600, 1600, 64
    T = M + L
    gb = 1 << 30
    base = lambda i: ctypes.c_void_p((i + 1) * gb)
    need = lib.txl_rel_attn_workspace_bytes(txl.BF16, B, H, L, M, d)
    assert need > 16 << 20
    args = [None, txl.BF16, B, H, L, M, d,
            base(0), H * L * d, d, L * d,
            base(1), base(2), H * T * d, d, T * d,
            base(3), d, T * d, T,
            base(4), base(5), 0.125,
            base(6), L * H * d, H * d, d, None]
    assert lib.txl_rel_attn_fwd_noalloc(*args) == txl.EWORKSPACE
    assert "static scratch" in txl.status_string(txl.EWORKSPACE)


def test_workspaces_cover_the_padded_copies_need_no_gpu():
    """bf16 widths that are not whole 32-element K steps (the word-level model's
    d_model 410, 10 heads of 41) are read through zero-padded copies that live in
    the caller's workspace: its size must cover them (pure host arithmetic)."""
    import torch
    from relative_position_memory_amd import txl
    B, L, M, D, H, d = 60, 150, 150, 410, 10, 41
    Dp, HDp, HD, T = 416, 416, H * d, M + L
    dims = txl.layer_dims(B, L, D, H, d)
    n = txl.workspace_bytes(dims, M, torch.bfloat16)
    dp = 48  # head rows padded to a multiple of 8
    base = 2 * (B * H * L * dp + 2 * B * H * T * dp + H * T * dp + B * L * HD) + 4 * B * L * D
    pads = 2 * (B * T * Dp + T * Dp + 4 * HD * Dp + D * HDp + B * L * HDp)
    assert n >= base + pads
    # the same model in fp32 takes no copies: its workspace is the plain layout
    r256 = lambda x: (x + 255) // 256 * 256
    n32 = txl.workspace_bytes(dims, M, torch.float32)
    assert n32 == sum(r256(4 * x) for x in (B * H * L * dp, B * H * T * dp, B * H * T * dp,
                                             H * T * dp, B * L * HD, B * L * D))
    # cached keys and values: h, W_q, W_kE, W_v and W_o, a padded
    nk = txl.kv_workspace_bytes(dims, M, torch.bfloat16)
    assert nk >= 2 * (B * L * Dp + 3 * HD * Dp + D * HDp + B * L * HDp)
    # feed-forward 410 x 1640: x, W1 (1664 rows), b1, W2 and f at a pitch of 1664
    rows, Di, Dip = 9000, 1640, 1664
    nf = txl.pos_ff_workspace_bytes(rows, D, Di, torch.bfloat16)
    assert nf >= 2 * (rows * Dip + rows * Dp + Dip * Dp + Dip + D * Dip) + 4 * rows * D
    # widths already whole K steps take no copies
    assert txl.pos_ff_workspace_bytes(rows, 512, 2048, torch.bfloat16) == \
        r256(rows * 2048 * 2) + r256(rows * 512 * 4)


def test_stack_argument_errors_need_no_gpu():
    """txl_stack_fwd checks every layer's arguments before it enqueues anything."""
    from relative_position_memory_amd import txl
    lib = txl._lib
    dims = txl.layer_dims(2, 16, 64, 2, 32)
    one = txl.stack_workspace_bytes(dims, 32, torch_bf16(), 1)
    assert txl._lib.txl_stack_workspace_bytes(ctypes.byref(dims), 32, txl.BF16, 2) == 2 * one
    assert txl._lib.txl_stack_workspace_bytes(ctypes.byref(dims), 32, txl.BF16, 0) == 0
    assert txl._lib.txl_stack_workspace_bytes(ctypes.byref(dims), 32, txl.BF16, 9) == 0
    seg = 2 * 16 * 64 * 2                  # one segment's [B][L][D] bf16
    ring_bytes = 2 * 32 * 64 * 2
    base = 0x100000000
    h_in, h_out, ws = base, base + 0x1000000, base + 0x2000000
    rdata = [base + 0x3000000 + i * 0x100000 for i in range(3)]
    fake = ctypes.c_void_p(base + 0x4000000)
    lw = txl.LayerWeights(*[fake.value] * 7)

    def call(n_streams=2, streams=True, n_layers=3, n_seg=2, rings=None, R_rows=200,
             ws_ptr=ws, ws_bytes=2 * one):
        rs = rings or [txl.Ring(rdata[i], 32, 0, 0) for i in range(3)]
        ra = (txl.Ring * 3)(*rs)
        wa = (txl.LayerWeights * 3)(lw, lw, lw)
        sa = (ctypes.c_void_p * 2)(None, None) if streams else None
        rc = lib.txl_stack_fwd(sa, n_streams, txl.BF16, ctypes.byref(dims), n_layers, n_seg,
                               h_in, ra, wa, fake, fake, fake, R_rows, h_out, ws_ptr, ws_bytes)
        return rc, [(r.start, r.len) for r in ra]

    assert call(n_streams=0)[0] == txl.EINVAL
    assert call(n_streams=9)[0] == txl.EINVAL
    assert call(streams=False)[0] == txl.EINVAL
    assert call(n_layers=0)[0] == txl.EINVAL
    assert call(n_seg=0)[0] == txl.EINVAL
    assert call(ws_ptr=ws + 8)[0] == txl.EINVAL               # not 256-byte aligned
    assert call(ws_bytes=2 * one - 1)[0] == txl.EWORKSPACE
    # R must cover the longest memory a layer reaches (len grows by L per segment up
    # to M) + L: from empty rings over 2 segments that is 16 + 16 rows
    assert call(R_rows=31)[0] == txl.EINVAL
    # bad ring state, and two layers sharing ring memory
    assert call(rings=[txl.Ring(rdata[0], 32, 32, 0)] * 3)[0] == txl.EINVAL
    rc, states = call(rings=[txl.Ring(rdata[0], 32, 0, 5), txl.Ring(rdata[0] + ring_bytes // 2, 32, 0, 5),
                             txl.Ring(rdata[2], 32, 0, 5)])
    assert rc == txl.EINVAL and states == [(0, 5)] * 3      # rejected, rings untouched
    # h_out overlapping h_in
    sa = (ctypes.c_void_p * 1)(None)
    ra = (txl.Ring * 1)(txl.Ring(rdata[0], 32, 0, 0))
    wa = (txl.LayerWeights * 1)(lw)
    assert lib.txl_stack_fwd(sa, 1, txl.BF16, ctypes.byref(dims), 1, 2, h_in, ra, wa, fake, fake,
                             fake, 200, h_in + seg, ws, one) == txl.EINVAL


def torch_bf16():
    import torch
    return torch.bfloat16


def test_attention_kernel_choice_needs_no_gpu():
    """txl_attn_kernel reports the kernel each workload's attention takes (the
    rule is one of sizes and CU count; without a device the count is 256, as on
    an MI355X), and txl_attn_variant forces one and rejects unknown settings."""
    import torch
    from relative_position_memory_amd import txl
    bf = torch.bfloat16
    assert txl.attn_kernel(bf, 22, 8, 512, 512, 64) == "attn_mfma_kernel"        # Char-LM
    assert txl.attn_kernel(bf, 60, 10, 150, 150, 48) == "attn_q64_kernel"        # Word-LM rows
    assert txl.attn_kernel(bf, 8, 16, 384, 384, 64) == "attn_q64_kernel"         # Large-train
    assert txl.attn_kernel(bf, 1, 16, 128, 1600, 64).startswith("attn_mfma_kernel + key-split")
    assert txl.attn_kernel(bf, 1, 16, 1, 3799, 64).startswith("attn_decode_kernel")
    assert txl.attn_kernel(torch.float32, 22, 8, 512, 512, 64).startswith("attn_generic")
    assert txl.attn_kernel(bf, 2, 2, 64, 64, 41).startswith("attn_generic")      # dense 41-wide rows
    with pytest.raises(txl.TxlError):
        txl.attn_kernel(bf, 0, 8, 512, 512, 64)
    old = txl.attn_variant(1)
    try:
        assert txl.attn_kernel(bf, 1, 16, 128, 1600, 64) == "attn_q64_kernel"
        assert txl.attn_variant(2) == 1
        assert txl.attn_kernel(bf, 8, 16, 384, 384, 64).startswith("attn_mfma_kernel")
        with pytest.raises(txl.TxlError):
            txl.attn_variant(3)
    finally:
        txl.attn_variant(old)
    assert txl.attn_kernel(bf, 8, 16, 384, 384, 64) == "attn_q64_kernel"
