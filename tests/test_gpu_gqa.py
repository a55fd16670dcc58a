"""GPU parity of grouped-query attention (attn_prefill_gqa_fwd, paged_attn_gqa_fwd
through the C ABI) against the fp64 oracle, and GQA == multi-head attention on
explicitly repeated K/V heads."""
import pytest
import torch

import oracle
import tiled_online_softmax_attention_amd as attn
from tiled_online_softmax_attention_amd import inputs
from parity import check_close, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def path_opts(split=None, path=None):
    """Launch options forcing the context split size and the decode path."""
    o = {}
    if split is not None:
        o["paged_split_tokens"] = int(split)
    if path is not None:
        o["paged_path"] = int(path)
    return o or None


@pytest.mark.parametrize("B,H,H_kv,N,d,causal,dtype", [
    (1, 8, 2, 300, 128, True, torch.bfloat16),
    (2, 4, 1, 257, 64, False, torch.bfloat16),        # MQA
    (1, 6, 3, 129, 128, True, torch.bfloat16),
    (1, 32, 4, 700, 128, True, torch.bfloat16),       # groups of 8
    (1, 4, 2, 100, 64, True, torch.float32),
    (1, 8, 8, 65, 128, True, torch.bfloat16),         # H_kv == H through the GQA entry point
])
def test_prefill_gqa_matches_oracle(B, H, H_kv, N, d, causal, dtype):
    cfg = inputs.PrefillConfig("gqa", B, H, N, d, dtype, causal, 500 + N + H_kv, H_kv=H_kv)
    log("prefill gqa B=%d H=%d H_kv=%d N=%d d=%d causal=%d %s" % (B, H, H_kv, N, d, causal, dtype))
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    assert k.shape[1] == H_kv
    if H_kv == H:
        o = torch.empty_like(q)
        lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
        rc = attn.attn_prefill_gqa_fwd(attn._ptr(q), attn._ptr(k), attn._ptr(v), attn._ptr(o), attn._ptr(lse), B, H,
                                       H_kv, N, d, cfg.scale, int(causal), attn._dtype_code(q), None,
                                       attn._stream(None))
        assert rc == 0
    else:
        o, lse = attn.prefill(q, k, v, causal, cfg.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, cfg.scale, causal)
    check_close("prefill gqa", o, o_ref, lse, l_ref, dtype)


def test_prefill_gqa_equals_repeated_heads():
    cfg = inputs.PrefillConfig("gqa_rep", 1, 8, 400, 128, torch.bfloat16, True, 77, H_kv=2)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    o1, l1 = attn.prefill(q, k, v, True, cfg.scale)
    o2, l2 = attn.prefill(q, k.repeat_interleave(4, 1).contiguous(), v.repeat_interleave(4, 1).contiguous(), True,
                          cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def make_gqa(ctx, ql, H, H_kv, d=128, bs=16, seed=1):
    return inputs.build_paged(torch.tensor(ctx, dtype=torch.int32), torch.tensor(ql, dtype=torch.int32), H_kv, d, bs,
                              seed, DEV, H_q=H)


def run_paged(pi, split=None, path=None):
    o, lse = attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size,
                                  pi.scale, options=path_opts(split, path))
    torch.cuda.synchronize()
    return o, lse


@pytest.mark.parametrize("H,H_kv", [(32, 4), (32, 8), (32, 16), (32, 1), (12, 4), (6, 2)])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("split", [None, 64])
@pytest.mark.parametrize("path", [0, 1, 2])
def test_paged_decode_gqa_matches_oracle(H, H_kv, bs, split, path):
    """Decode (q_len 1 to 3) on the three paths.  Vector kernel: one
    workgroup serves up to 8 (16-token pages) or 4 (32-token pages) query
    heads of a group, larger groups split across workgroups (MQA at 32 query
    heads, groups of 3).  MFMA tile kernel: a tile holds all heads of a group
    for 128 / G positions.  Decode MFMA kernel: where G x 3 <= 16 (else the
    launcher keeps its own choice)."""
    ctx = [700, 33, 1500, 5, 64]
    ql = [1, 3, 1, 1, 2]
    pi = make_gqa(ctx, ql, H, H_kv, bs=bs, seed=H + H_kv + bs)
    log("paged decode gqa H=%d H_kv=%d bs=%d split=%s path=%d" % (H, H_kv, bs, split, path))
    o, lse = run_paged(pi, split, path)
    o_ref, l_ref = oracle.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, bs, pi.scale)
    check_close("paged decode gqa", o, o_ref, lse, l_ref, torch.bfloat16)


@pytest.mark.parametrize("H,H_kv,ql", [(32, 4, 1), (32, 4, 2), (32, 2, 1), (16, 4, 4), (8, 8, 1), (6, 2, 5)])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("split", [None, 32, 400, 4096])
def test_paged_decode_mfma_matches_oracle(H, H_kv, ql, bs, d, split):
    """The decode MFMA kernel (paged_path 2): groups of 8 and 16 heads at one
    position, 8 x 2 and 4 x 4 rows (all 16), one plain head (1 row of 16), 3
    heads x 5 positions (15 rows); contexts shorter than a 16-key tile, tiles
    cut by the context end, splits of one or two pages, of a length that is
    not a whole number of tiles per wave, and above the 128-page cap (pages
    64-127 of a split come from the second table register)."""
    ctx = [1, 15, 16, 17, 300, 1030, 5000]
    qls = [min(ql, c) for c in ctx]
    pi = make_gqa(ctx, qls, H, H_kv, d=d, bs=bs, seed=H + 3 * H_kv + ql + bs + d)
    log("paged decode mfma H=%d H_kv=%d ql=%d bs=%d d=%d split=%s" % (H, H_kv, ql, bs, d, split))
    o, lse = run_paged(pi, split, 2)
    o_ref, l_ref = oracle.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, bs, pi.scale)
    check_close("paged decode mfma", o, o_ref, lse, l_ref, torch.bfloat16)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("split", [None, 256])
def test_paged_chunk_gqa_matches_oracle(d, split):
    ctx = [300, 1200, 40, 700]
    ql = [300, 260, 7, 129]
    pi = make_gqa(ctx, ql, 8, 2, d=d, bs=32, seed=9 + d)
    log("paged chunk gqa d=%d split=%s" % (d, split))
    o, lse = run_paged(pi, split)
    o_ref, l_ref = oracle.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, 32, pi.scale)
    check_close("paged chunk gqa", o, o_ref, lse, l_ref, torch.bfloat16)


def repeat_pool(pool, rep):
    """Pool with every K/V head repeated rep times (multi-head layout)."""
    return pool.repeat_interleave(rep, dim=2).contiguous()


@pytest.mark.parametrize("ql", [1, 2])
def test_paged_gqa_equals_repeated_heads(ql):
    """On the vector decode kernel, a group of query heads served by one
    workgroup gives the same bits as the same heads served one by one from a
    repeated-head pool (per-head arithmetic is independent of the other heads
    there; the MFMA kernel's lazy rescale is a per-wave decision, so its bits
    depend on which rows share a wave and it is checked against the oracle)."""
    ctx = [900, 65, 2000, 17 + ql]
    pi = make_gqa(ctx, [ql] * 4, 32, 4, seed=33 + ql)
    # the default split size depends on the workgroup count; fix it for both
    o1, l1 = run_paged(pi, split=256, path=0)
    o2, l2 = attn.paged_attention(pi.q, repeat_pool(pi.pool, 8), pi.block_table, pi.ctx_lens, pi.q_lens, 16,
                                  pi.scale, options=path_opts(256, 0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_gqa_mixed_batch():
    ctx = [4000, 1, 513, 77, 2048]
    ql = [1, 1, 40, 77, 4]
    pi = make_gqa(ctx, ql, 16, 4, seed=55)
    o, lse = run_paged(pi)
    o_ref, l_ref = oracle.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, 16, pi.scale)
    check_close("paged gqa mixed", o, o_ref, lse, l_ref, torch.bfloat16)


def test_c4_gqa8_full_size_sampled_rows():
    """The 64-request decode batch with 32 query heads on 4 K/V heads, in the
    benchmark's launch configuration (MFMA tile kernel, pipelined loop) and
    on the decode MFMA kernel; 64 seeded (request, head) pairs checked
    against the oracle; and, on the vector kernel, the whole output against
    the repeated-head pool bit for bit."""
    cfg = inputs.C4_GQA8
    pi = inputs.paged_inputs(cfg, DEV)
    log("c4 gqa8 full size: %d requests, sum ctx %d" % (pi.num_seqs, int(pi.ctx_lens.sum())))
    trip = inputs.sample_triples(cfg.seed, 64, (pi.num_seqs, cfg.H), edge=[(0, 0), (63, 31), (10, 7), (10, 8)])
    ridx = [r for r, _ in trip]
    hidx = [h for _, h in trip]
    o_ref, l_ref = oracle.paged_attention_rows(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, 16, pi.scale,
                                               ridx, hidx, [0] * len(trip))
    for path in (None, 2):
        o, lse = run_paged(pi, path=path)
        og = torch.stack([o[r, h] for r, h in trip])
        lg = torch.stack([lse[r, h] for r, h in trip])
        check_close("c4 gqa8 sampled path %s" % path, og, o_ref, lg, l_ref, torch.bfloat16)
    o1, l1 = run_paged(pi, split=512, path=0)
    o2, l2 = attn.paged_attention(pi.q, repeat_pool(pi.pool, 8), pi.block_table, pi.ctx_lens, pi.q_lens, 16,
                                  pi.scale, options=path_opts(512, 0))
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
