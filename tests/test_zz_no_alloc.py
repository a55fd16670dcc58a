"""paged_attn_fwd_static (the entry point that allocates nothing: split
partials in the library's static per-GPU workspace) against paged_attn_fwd
with a caller workspace, through the C ABI: same bits, on two calls in a row
(the second on a smaller batch), and oversize plans rejected before any
launch."""
import ctypes

import pytest
import torch

import oracle
import tiled_online_softmax_attention_amd as attn
from tiled_online_softmax_attention_amd import inputs
from parity import check_close, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def call_both(pi, max_q, max_ctx):
    """paged_attn_fwd (caller workspace) and paged_attn_fwd_static on the same
    inputs; returns ((o, lse), (o_static, lse_static), workspace bytes)."""
    num_blocks, _, H_kv, bs, d = pi.pool.shape
    H = pi.q.shape[1]
    assert H_kv == H
    num_seqs, maxb = pi.block_table.shape
    k_ptr = pi.pool.data_ptr()
    v_ptr = k_ptr + H * bs * d * pi.pool.element_size()
    stride = 2 * H * bs * d
    need = attn.paged_attn_workspace_bytes(num_seqs, H, d, bs, max_q, max_ctx)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    outs = []
    for static in (False, True):
        o = torch.full_like(pi.q, float("nan"))
        lse = torch.full(pi.q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
        args = [attn._ptr(pi.q), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr), attn._ptr(pi.block_table),
                attn._ptr(pi.ctx_lens), attn._ptr(pi.q_lens), bs, attn._ptr(o), attn._ptr(lse), num_seqs, H, d,
                pi.scale, maxb, stride, num_blocks, max_q, max_ctx, attn.ATTN_BF16]
        if static:
            rc = attn.paged_attn_fwd_static(*args, attn._stream(None))
        else:
            rc = attn.paged_attn_fwd(*args, attn._ptr(ws), ws.numel(), attn._stream(None))
        assert rc == 0, attn.attn_strerror(rc)
        torch.cuda.synchronize()
        outs.append((o, lse))
    return outs[0], outs[1], need


def assert_same_bits(a, b):
    assert torch.equal(a[0].view(torch.int16), b[0].view(torch.int16))
    assert torch.equal(a[1].view(torch.int32), b[1].view(torch.int32))


def test_static_matches_caller_workspace_twice():
    """A 64-request decode batch with split contexts (the static workspace in
    use), then a smaller batch: the static entry point gives the bits of the
    caller-workspace one both times, and the first batch again after the
    second (whatever the array kept from the previous call)."""
    big = inputs.paged_inputs(inputs.C4, DEV)
    max_ctx_big = int(big.ctx_lens.max())
    log("no-alloc: 64-request decode batch, max ctx %d" % max_ctx_big)
    ref1, got1, need1 = call_both(big, 1, max_ctx_big)
    assert 0 < need1 <= attn.STATIC_WORKSPACE_BYTES
    assert_same_bits(ref1, got1)

    small = inputs.build_paged(torch.tensor([700, 33, 1500, 2100], dtype=torch.int32),
                               torch.tensor([1, 3, 64, 17], dtype=torch.int32), 32, 128, 16, 91, DEV)
    max_ctx_small = int(small.ctx_lens.max())
    log("no-alloc: 4-request mixed batch, max ctx %d" % max_ctx_small)
    ref2, got2, need2 = call_both(small, 64, max_ctx_small)
    # a smaller input (fewer requests, query rows and context tokens); its
    # plan (the tile kernel for 64-row queries) splits too, within the array
    assert small.ctx_lens.numel() < big.ctx_lens.numel()
    assert int(small.ctx_lens.sum()) < int(big.ctx_lens.sum())
    assert 0 < need2 <= attn.STATIC_WORKSPACE_BYTES
    assert_same_bits(ref2, got2)
    o_ref, l_ref = oracle.paged_attention(small.q, small.pool, small.block_table, small.ctx_lens, small.q_lens, 16,
                                          small.scale)
    check_close("no-alloc small batch", got2[0], o_ref, got2[1], l_ref, torch.bfloat16)

    ref3, got3, _ = call_both(big, 1, max_ctx_big)
    assert_same_bits(ref1, got3)
    assert_same_bits(ref3, got3)


def test_static_rejects_oversize_plan():
    """A plan needing more than the static workspace is ATTN_ERR_WORKSPACE,
    before anything is launched (the outputs keep their contents)."""
    num_seqs, H, d, bs, max_q, max_ctx = 8, 32, 128, 32, 512, 33280
    need = attn.paged_attn_workspace_bytes(num_seqs, H, d, bs, max_q, max_ctx)
    assert need > attn.STATIC_WORKSPACE_BYTES
    o = torch.full((16, H, d), 3.0, dtype=torch.bfloat16, device=DEV)
    dummy = torch.zeros(1 << 16, dtype=torch.uint8, device=DEV)
    p = attn._ptr(dummy)
    rc = attn.paged_attn_fwd_static(p, p, p, p, p, p, bs, attn._ptr(o), None, num_seqs, H, d, 0.1, 2048,
                                    2 * H * bs * d, 4, max_q, max_ctx, attn.ATTN_BF16, attn._stream(None))
    torch.cuda.synchronize()
    assert rc == -7, attn.attn_strerror(rc)   # ATTN_ERR_WORKSPACE
    assert bool((o == 3.0).all())
