"""GPU parity of paged_attn_fwd and paged_kv_gather (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_attention_amd as attn
from tiled_online_softmax_attention_amd import inputs
from parity import check_close, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def split_opts(tokens, path=None):
    """Launch options forcing the context split size (tokens) and the decode
    path (0 vector kernel, 2 decode MFMA kernel), or None."""
    o = {}
    if tokens is not None:
        o["paged_split_tokens"] = int(tokens)
    if path is not None:
        o["paged_path"] = int(path)
    return o or None


def make(ctx, ql, H=4, d=128, bs=16, seed=1, **kw):
    return inputs.build_paged(torch.tensor(ctx, dtype=torch.int32), torch.tensor(ql, dtype=torch.int32), H, d, bs,
                              seed, DEV, **kw)


def run(pi, split=None, name="paged", path=None):
    log("%s: num_seqs=%d H=%d d=%d bs=%d ctx=%s q=%s split=%s path=%s" % (
        name, pi.num_seqs, pi.H, pi.d, pi.block_size, pi.ctx_lens.tolist()[:8], pi.q_lens.tolist()[:8], split, path))
    o, lse = attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size,
                                  pi.scale, options=split_opts(split, path))
    torch.cuda.synchronize()
    return o, lse


def check_full(pi, split=None, name="paged", path=None):
    o, lse = run(pi, split, name, path)
    o_ref, l_ref = oracle.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size,
                                          pi.scale)
    check_close(name, o, o_ref, lse, l_ref, torch.bfloat16)
    return o, lse


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("split", [None, 64])
@pytest.mark.parametrize("path", [None, 0, 2])
def test_decode_ragged(bs, d, split, path):
    # plain heads, one query row: the plan's kernel (the vector kernel here but
    # on 32-token pages), and each decode kernel forced
    ctx = [1, 15, 16, 17, 100, 513, 1030, 2047]
    pi = make(ctx, [1] * len(ctx), H=3, d=d, bs=bs, seed=bs + d)
    check_full(pi, split, "decode bs%d d%d" % (bs, d), path)


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("split", [None, 256])
@pytest.mark.parametrize("path", [None, 0])
def test_small_q_decode_path(bs, split, path):
    # q_len 2..4: the decode MFMA kernel by default (all of a request's rows
    # in one workgroup), the vector kernel (one query row per workgroup) forced
    ctx = [4, 40, 333, 1000]
    pi = make(ctx, [2, 4, 3, 4], H=2, bs=bs, seed=3)
    check_full(pi, split, "decode q<=4 bs%d" % bs, path)


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("split", [None, 128, 320])
def test_chunk_ragged(bs, d, split):
    ctx = [5, 129, 700, 1200]
    ql = [5, 129, 200, 77]
    pi = make(ctx, ql, H=2, d=d, bs=bs, seed=7 + bs)
    check_full(pi, split, "chunk bs%d d%d" % (bs, d))


@pytest.mark.parametrize("split", [64, 128, 192])
def test_chunk_split_tile_counts(split):
    """Splits of 64, 128 and 192 keys (2, 4 and 6 key tiles of 32), with
    ragged tails: several lengths of the double-buffered key loop, odd and
    even tile counts."""
    ctx = [300, 1200, 40, 130]
    ql = [300, 260, 7, 129]
    pi = make(ctx, ql, H=2, bs=32, seed=17)
    check_full(pi, split, "chunk split%d" % split)


@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("split", [None, 128, 320, 4096])
def test_chunk_tile_kernels_bit_identical(bs, d, split):
    """The tile kernel's three variants -- the plain key loop on 128-row
    workgroups, the pipelined loop (page-table entries read from a 64-page
    register window) on 128- and on 256-row workgroups -- give the same bits
    and match the oracle: ragged chunks of one to five 128-row tiles, a 1-row
    request, splits of 2 to 128 key tiles (4096 keys = 256 pages of 16
    tokens: the window moves several times per split)."""
    ctx = [5, 129, 700, 1200, 5000, 1]
    ql = [5, 129, 300, 77, 600, 1]
    pi = make(ctx, ql, H=2, d=d, bs=bs, seed=31 + bs + d)
    outs = []
    for kind in (0, 1, 2):
        log("chunk tile kernel %d bs%d d%d split %s" % (kind, bs, d, split))
        opts = {"paged_tile_kernel": kind, "paged_path": 1}
        if split is not None:
            opts["paged_split_tokens"] = split
        o, lse = attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size,
                                      pi.scale, options=opts)
        torch.cuda.synchronize()
        outs.append((o, lse))
    for o, l in outs[1:]:
        assert torch.equal(outs[0][0].view(torch.int16), o.view(torch.int16)) and torch.equal(outs[0][1], l)
    o_ref, l_ref = oracle.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size,
                                          pi.scale)
    check_close("chunk tile kernels", outs[2][0], o_ref, outs[2][1], l_ref, torch.bfloat16)


@pytest.mark.parametrize("H,H_kv,ql", [(32, 8, 130), (8, 1, 40), (6, 2, 100), (32, 4, 1), (32, 4, 4)])
def test_chunk_tile_kernels_grouped_heads(H, H_kv, ql):
    """The tile kernel's variants on grouped query heads (positions of 4, 8,
    3 and 8 heads per workgroup, down to decode rows: 8 or 32 valid rows of
    128): same bits, and the oracle."""
    ctx = [900, 2000, 300, 4100]
    qls = [min(ql, c) for c in ctx]
    pi = inputs.build_paged(ctx, qls, H_kv, 128, 16, 55 + H + ql, DEV, H_q=H)
    outs = []
    for kind in (0, 1, 2):
        log("grouped chunk tile kernel %d H=%d H_kv=%d ql=%d" % (kind, H, H_kv, ql))
        o, lse = attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size,
                                      pi.scale, options={"paged_tile_kernel": kind, "paged_split_tokens": 1024,
                                                         "paged_path": 1})
        torch.cuda.synchronize()
        outs.append((o, lse))
    for o, l in outs[1:]:
        assert torch.equal(outs[0][0].view(torch.int16), o.view(torch.int16)) and torch.equal(outs[0][1], l)
    o_ref, l_ref = oracle.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size,
                                          pi.scale)
    check_close("grouped chunk tile kernels", outs[1][0], o_ref, outs[1][1], l_ref, torch.bfloat16)


def test_chunk_mixed_with_decode_rows():
    ctx = [900, 64, 1, 300]
    ql = [300, 1, 1, 300]
    pi = make(ctx, ql, H=4, bs=32, seed=21)
    check_full(pi, None, "mixed")


def test_permutation_bit_identity_and_aliasing():
    """Same logical K/V in two different physical layouts (and with a second
    request aliasing the first one's blocks): bit-identical outputs."""
    H, d, bs = 4, 128, 16
    ctx = torch.tensor([777, 777, 50], dtype=torch.int32)
    ql = torch.tensor([1, 1, 1], dtype=torch.int32)
    a = inputs.build_paged(ctx, ql, H, d, bs, seed=31, device=DEV)
    # permuted copy: move every block to a new random slot
    perm = torch.randperm(a.num_blocks, generator=torch.Generator().manual_seed(99)).to(DEV)
    pool2 = torch.empty_like(a.pool)
    pool2[perm] = a.pool
    table2 = a.block_table.clone()
    valid = table2 >= 0
    table2[valid] = perm[table2[valid].long()].to(torch.int32)
    # alias: request 1 reads request 0's blocks (its own K/V are identical then)
    table_alias = a.block_table.clone()
    table_alias[1] = table_alias[0]
    q = a.q.clone()
    q[1] = q[0]
    for split in (None, 128):
        op = split_opts(split)
        o1, l1 = attn.paged_attention(q, a.pool, a.block_table, a.ctx_lens, a.q_lens, bs, options=op)
        o2, l2 = attn.paged_attention(q, pool2, table2, a.ctx_lens, a.q_lens, bs, options=op)
        o3, l3 = attn.paged_attention(q, a.pool, table_alias, a.ctx_lens, a.q_lens, bs, options=op)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        assert torch.equal(o3[0], o3[1]) and torch.equal(o3[0], o1[0]) and torch.equal(o3[2], o1[2])


def test_repeat_determinism():
    pi = make([3000, 10, 900], [1, 1, 1], H=8, seed=41)
    o1, l1 = run(pi, None)
    o2, l2 = run(pi, None)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    pc = make([3000, 300, 900], [200, 300, 5], H=4, bs=32, seed=42)
    o1, l1 = run(pc, 512)
    o2, l2 = run(pc, 512)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_split_count_independence():
    pi = make([5000, 2500, 100], [1, 1, 1], H=4, seed=51)
    base, bl = run(pi, 1 << 14)
    for s in (64, 256, 1024):
        o, l = run(pi, s)
        assert (o.float() - base.float()).abs().max() <= 2e-2
        assert (l - bl).abs().max() <= 1e-4


def test_paged_square_matches_prefill():
    """q_len == ctx: paged chunk attention equals causal prefill on the same data."""
    H, d, bs, N = 2, 128, 32, 700
    cfg = inputs.PrefillConfig("sq", 1, H, N, d, torch.bfloat16, True, 61)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    nb = (N + bs - 1) // bs
    perm = torch.randperm(nb + 2, generator=torch.Generator().manual_seed(3))
    pool = torch.full((nb + 2, 2, H, bs, d), float("nan"), dtype=torch.bfloat16, device=DEV)
    for t0 in range(0, N, bs):
        t1 = min(N, t0 + bs)
        pb = int(perm[t0 // bs])
        pool[pb, 0, :, :t1 - t0] = k[0, :, t0:t1]
        pool[pb, 1, :, :t1 - t0] = v[0, :, t0:t1]
    table = perm[:nb].to(torch.int32).view(1, nb).to(DEV)
    qp = q[0].permute(1, 0, 2).contiguous()
    lens = torch.tensor([N], dtype=torch.int32, device=DEV)
    op, lp = attn.paged_attention(qp, pool, table, lens, lens, bs)
    of, lf = attn.prefill(q, k, v, True)
    torch.cuda.synchronize()
    assert (op.float() - of[0].permute(1, 0, 2).float()).abs().max() <= 2e-2
    assert (lp - lf[0].T).abs().max() <= 5e-3


def test_scale_zero_bottom_right_alignment():
    ctx = [40, 333]
    ql = [7, 100]
    pi = make(ctx, ql, H=2, bs=16, seed=71)
    o, lse = attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, 16, scale=0.0)
    torch.cuda.synchronize()
    lse = lse.double().cpu()
    row = 0
    for c, q in zip(ctx, ql):
        for i in range(q):
            want = np.log(c - q + i + 1)
            assert abs(float(lse[row + i, 0]) - want) < 1e-4
        row += q


def test_gather_bit_exact():
    ctx = [1, 16, 17, 250, 1000]
    for bs in (16, 32):
        pi = make(ctx, [1] * 5, H=3, d=128, bs=bs, seed=81)
        k, v = attn.gather(pi.pool, pi.block_table, pi.ctx_lens, bs)
        torch.cuda.synchronize()
        ko, vo = oracle.paged_gather(pi.pool, pi.block_table, pi.ctx_lens, bs)
        assert np.array_equal(k.cpu().view(torch.int16).numpy().view(np.uint16), ko)
        assert np.array_equal(v.cpu().view(torch.int16).numpy().view(np.uint16), vo)


def test_c4_full():
    """64 requests, q_len 1, ctx U[512, 16384], 16-token pages: every row vs the oracle."""
    c = inputs.C4
    log("c4: building inputs")
    pi = inputs.paged_inputs(c, DEV)
    check_full(pi, None, "c4")


@pytest.mark.slow
def test_c5_sampled():
    """8 requests x 512-token chunks on ctx U[4096, 32768] + 512, 32-token pages;
    64 seeded (request, head, row) triples plus edge rows."""
    c = inputs.C5
    log("c5: building inputs")
    pi = inputs.paged_inputs(c, DEV)
    o, lse = run(pi, None, "c5")
    assert bool(torch.isfinite(o).all())
    trip = inputs.sample_triples(c.seed, 64, (c.num_seqs, c.H, c.q_len),
                                 edge=[(0, 0, 0), (0, 0, 511), (7, 31, 0), (7, 31, 511), (3, 4, 128)])
    r_idx = [t[0] for t in trip]
    h_idx = [t[1] for t in trip]
    i_idx = [t[2] for t in trip]
    o_ref, l_ref = oracle.paged_attention_rows(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens,
                                               pi.block_size, pi.scale, r_idx, h_idx, i_idx)
    rows = [r * c.q_len + i for r, i in zip(r_idx, i_idx)]
    og = torch.stack([o[rw, h] for rw, h in zip(rows, h_idx)])
    lg = torch.stack([lse[rw, h] for rw, h in zip(rows, h_idx)])
    check_close("c5 sampled", og, o_ref, lg, l_ref, torch.bfloat16)


@pytest.mark.parametrize("ql,split", [(1, None), (1, 64), (200, 128), (3, None)])
def test_outputs_and_workspace_in_bounds(ql, split):
    """Guard words around O, LSE and the workspace survive a call: the
    decode and tile paths, with and without context splits, write only
    inside the buffers they are given (the workspace exactly as large as
    paged_attn_workspace_bytes asks)."""
    ctx = [900, 64, 1, 300, 2000]
    pi = make(ctx, [min(ql, c) for c in ctx], H=4, d=128, bs=16, seed=50 + ql)
    G = 4096
    rows, H, d = pi.q.shape
    obuf = torch.full((2 * G + rows * H * d,), 7.0, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((2 * G + rows * H,), 3.0, dtype=torch.float32, device=DEV)
    o = obuf[G:G + rows * H * d].view(rows, H, d)
    lse = lbuf[G:G + rows * H].view(rows, H)
    op = split_opts(split)
    max_q, max_ctx = int(pi.q_lens.max()), int(pi.ctx_lens.max())
    ws_bytes = attn.paged_attn_gqa_workspace_bytes(pi.num_seqs, H, H, d, pi.block_size, max_q, max_ctx,
                                                   attn._opts(op))
    wbuf = torch.full((ws_bytes + 2 * G,), 0x5A, dtype=torch.uint8, device=DEV)
    ws = wbuf[G:G + ws_bytes] if ws_bytes else None   # offset G keeps the 256-byte alignment
    log("canaries ql=%d split=%s ws=%d" % (ql, split, ws_bytes))
    attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size, pi.scale,
                         max_q_len=max_q, max_ctx_len=max_ctx, out=o, lse=lse, workspace=ws, options=op)
    torch.cuda.synchronize()
    assert bool((obuf[:G] == 7.0).all()) and bool((obuf[-G:] == 7.0).all())
    assert bool((lbuf[:G] == 3.0).all()) and bool((lbuf[-G:] == 3.0).all())
    assert bool((wbuf[:G] == 0x5A).all()) and bool((wbuf[-G:] == 0x5A).all())
    assert bool(torch.isfinite(o.float()).all())


@pytest.mark.parametrize("ctx,ql,H,H_kv", [
    ([900, 64, 3000, 300, 1, 2100], 40, 32, 8),   # 48 (request, K/V head) pairs: pairs dealt to XCDs
    ([900, 2000, 300], 130, 8, 1),                 # 3 pairs: items dealt one by one
])
def test_chunk_work_mappings_bit_identical(ctx, ql, H, H_kv):
    """The tile kernel's three work mappings (XCD-contiguous ranges, pairs
    dealt round-robin, items dealt round-robin) only move items between
    workgroups: outputs are bit-identical, and they match the oracle."""
    qls = [min(ql, c) for c in ctx]
    pi = inputs.build_paged(ctx, qls, H_kv, 128, 16, 77, DEV, H_q=H)
    outs = []
    for m in (0, 1, 2):
        log("chunk mapping %d" % m)
        o, lse = attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size,
                                      pi.scale, options={"paged_split_tokens": 256, "paged_tile_map": m})
        torch.cuda.synchronize()
        outs.append((o, lse))
    for o, l in outs[1:]:
        assert torch.equal(o.view(torch.int16), outs[0][0].view(torch.int16)) and torch.equal(l, outs[0][1])
    o_ref, l_ref = oracle.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size,
                                          pi.scale)
    check_close("chunk mappings", outs[0][0], o_ref, outs[0][1], l_ref, torch.bfloat16)


def test_context_above_bound_reads_as_bound():
    """A ctx_lens[r] above the host bound max_ctx_len breaks the contract; the
    kernels read it as max_ctx_len, so no kernel reaches past the workspace
    (guard words) and the result is attention over the bound's context.
    Every table row holds the real contexts' pages, so table reads stay in the
    row either way; only the split count, which sizes the workspace, depends
    on the bound."""
    ctx, ql = [1500, 900, 2100], [1, 1, 1]
    pi = make(ctx, ql, H=4, d=128, bs=16, seed=61)
    bound = 1000
    op = {"paged_split_tokens": 256}
    ws_bytes = attn.paged_attn_gqa_workspace_bytes(pi.num_seqs, 4, 4, 128, 16, 1, bound, attn._opts(op))
    assert ws_bytes > 0
    G = 1 << 16
    wbuf = torch.full((ws_bytes + 2 * G,), 0x5A, dtype=torch.uint8, device=DEV)
    ws = wbuf[G:G + ws_bytes]
    o, lse = attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, 16, pi.scale,
                                  max_q_len=1, max_ctx_len=bound, workspace=ws, options=op)
    torch.cuda.synchronize()
    assert bool((wbuf[:G] == 0x5A).all()) and bool((wbuf[-G:] == 0x5A).all())
    clamped = torch.clamp(pi.ctx_lens, max=bound)
    o_ref, l_ref = oracle.paged_attention(pi.q, pi.pool, pi.block_table, clamped, pi.q_lens, 16, pi.scale)
    check_close("ctx above bound", o, o_ref, lse, l_ref, torch.bfloat16)


@pytest.mark.parametrize("H,H_kv", [(8, 8), (32, 4)])
def test_long_context_decode(H, H_kv):
    """Decode over very long contexts (262144 and 100003 tokens, 16-token
    pages scattered over the pool): hundreds of splits per row, so the
    combine walks its split partials in several batches of 64; plain heads
    (vector decode kernel) and eight query heads per K/V head (MFMA tile
    kernel).  Every row against the oracle."""
    ctx = [262144, 100003]
    pi = inputs.build_paged(ctx, [1, 1], H_kv, 128, 16, 91 + H, DEV, H_q=H)
    log("long decode H=%d H_kv=%d ctx=%s" % (H, H_kv, ctx))
    o, lse = attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size, pi.scale)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size,
                                          pi.scale)
    check_close("long decode", o, o_ref, lse, l_ref, torch.bfloat16)
