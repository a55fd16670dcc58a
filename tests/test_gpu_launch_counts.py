"""Launches per call, counted from the device trace (torch.profiler records
every kernel the HIP runtime runs, the library's included): one launch for a
prefill, one for a paged step whose contexts fit one split and two (partial
attention + log-sum-exp combine) when some context is split, two for the
backward (dQ; dK and dV) and two for a KV append (allocation; copy)."""
import pytest
import torch
from torch.profiler import ProfilerActivity, profile

import tiled_online_softmax_attention_amd as attn
from tiled_online_softmax_attention_amd import inputs
from parity import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def library_launches(fn):
    """Names of the library's kernels (namespace attn::) that fn launched."""
    fn()   # warm: first-call work (code-object loading) stays out of the trace
    torch.cuda.synchronize()
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        fn()
        torch.cuda.synchronize()
    names = [e.name for e in prof.events() if e.device_type == torch.autograd.DeviceType.CUDA]
    return [n for n in names if "attn::" in n]


def test_prefill_one_launch():
    for dtype, kname in ((torch.bfloat16, "prefill_bf16_kernel"), (torch.float32, "prefill_f32_kernel")):
        cfg = inputs.PrefillConfig("launch", 1, 2, 300, 128, dtype, True, 1)
        q, k, v = inputs.prefill_inputs(cfg, DEV)
        got = library_launches(lambda: attn.prefill(q, k, v, True))
        log("prefill %s: %s" % (dtype, got))
        assert len(got) == 1 and kname in got[0], got


@pytest.mark.parametrize("ctx,ql,split", [
    ([900, 64, 1, 300], 1, True),        # decode, split contexts (at most 8 splits)
    ([5000, 64, 1, 300], 1, True),       # decode, more than 8 splits of one context
    ([40, 64, 1, 17], 1, False),         # decode, every context in one split
    ([3000, 600, 1300], 200, True),      # chunked prefill (tile kernel), split
    ([900, 600, 300], 200, False),       # chunked prefill, one split (1024 keys at least)
])
def test_paged_launches(ctx, ql, split):
    pi = inputs.build_paged(ctx, [min(ql, c) for c in ctx], 4, 128, 16, 3, DEV)
    max_q, max_ctx = int(pi.q_lens.max()), int(pi.ctx_lens.max())
    ws = attn.paged_attn_workspace_bytes(pi.num_seqs, pi.H, pi.d, pi.block_size, max_q, max_ctx)
    assert (ws > 0) == split   # the plan splits exactly when it asks for a workspace
    got = library_launches(lambda: attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, 16,
                                                        max_q_len=max_q, max_ctx_len=max_ctx))
    log("paged ctx=%s ql=%d: %s" % (ctx, ql, got))
    assert len(got) == (2 if split else 1), got
    if split:
        # the workspace holds (d + 1) fp32 per (row, head, split): at most 8
        # splits per row take the lane-groups-per-head combine, more a wave per head
        rows_heads = pi.num_seqs * max_q * pi.H
        max_splits = ws // (rows_heads * (pi.d + 1) * 4)
        kname = "paged_combine_kernel" if max_splits > 8 else "paged_combine_heads_kernel"
        log("max_splits=%d -> %s" % (max_splits, kname))
        assert kname in got[1], got


def test_backward_two_launches():
    cfg = inputs.PrefillConfig("launch_bwd", 1, 4, 200, 128, torch.bfloat16, True, 2, H_kv=2)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    do = inputs.grad_output(cfg, DEV)
    o, lse = attn.prefill(q, k, v, True)
    got = library_launches(lambda: attn.prefill_bwd(q, k, v, o, lse, do, True))
    log("bwd: %s" % got)
    assert len(got) == 2 and "bwd_dq_kernel" in got[0] and "bwd_dkdv_kernel" in got[1], got


def test_append_two_launches():
    ai = inputs.append_inputs([40, 0, 17], [5, 16, 1], 4, 128, 16, 9, DEV, slack_blocks=64)
    free = torch.tensor(ai.free_list + [-7] * (ai.pool.shape[0] - len(ai.free_list)), dtype=torch.int32,
                        device=DEV)   # the free list is [num_blocks]
    count = torch.tensor([len(ai.free_list)], dtype=torch.int32, device=DEV)
    ctx = ai.ctx_old.clone()

    def step():
        # append, then hand the blocks back so that every call starts alike
        nctx, _ = attn.kv_append(ai.k_new, ai.v_new, ctx, ai.new_lens, ai.pool, ai.block_table, free, count, 16,
                                 check=False)
        return nctx

    step()
    torch.cuda.synchronize()
    count.fill_(len(ai.free_list))
    got = library_launches(lambda: (count.fill_(len(ai.free_list)), step()))
    log("append: %s" % got)
    assert len(got) == 2, got
