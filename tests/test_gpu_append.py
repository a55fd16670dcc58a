"""GPU parity of paged_kv_append / paged_kv_release (through the C ABI) against
the KV-append oracle (oracle/kv_cache.py): pool bytes, block tables, free
list and counts must match bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from oracle import kv_cache as kc
import tiled_online_softmax_attention_amd as attn
from tiled_online_softmax_attention_amd import inputs
from parity import check_close, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


class DeviceCache:
    """The device-side state of one append test, plus its oracle twin."""

    def __init__(self, ai: inputs.AppendInputs):
        self.ai = ai
        nb = ai.pool.shape[0]
        self.num_blocks = nb
        self.pool = ai.pool.to(DEV)
        self.table = ai.block_table.to(DEV).clone()
        self.free = torch.full((nb,), -7, dtype=torch.int32)
        self.free[:len(ai.free_list)] = torch.tensor(ai.free_list, dtype=torch.int32)
        self.free = self.free.to(DEV)
        self.count = torch.tensor([len(ai.free_list)], dtype=torch.int32, device=DEV)
        # oracle twin (bytes: bf16 as int16, fp32 as int32)
        iview = torch.int16 if ai.pool.dtype == torch.bfloat16 else torch.int32
        self.iview = iview
        self.o_pool = ai.pool.cpu().view(iview).numpy().copy()
        self.o_table = ai.block_table.cpu().numpy().copy()
        self.o_alloc = kc.BlockAllocator(nb, ai.block_size, free=list(ai.free_list))

    def append(self, ctx, new, k_new, v_new, check=True):
        ctx_d = torch.tensor(ctx, dtype=torch.int32, device=DEV)
        new_d = torch.tensor(new, dtype=torch.int32, device=DEV)
        nctx, status = attn.kv_append(k_new, v_new, ctx_d, new_d, self.pool, self.table, self.free, self.count,
                                      self.ai.block_size, check=check)
        torch.cuda.synchronize()
        return nctx.cpu().tolist(), int(status.item())

    def oracle_append(self, ctx, new, k_new, v_new):
        kn = k_new.cpu().view(self.iview).numpy()
        vn = v_new.cpu().view(self.iview).numpy()
        return kc.append(self.o_pool, self.o_table, ctx, new, kn, vn, self.o_alloc)

    def assert_matches_oracle(self, free_before):
        assert np.array_equal(self.table.cpu().numpy(), self.o_table)
        cnt = int(self.count.item())
        assert cnt == len(self.o_alloc.free)
        fr = self.free.cpu()
        assert fr[:cnt].tolist() == self.o_alloc.free
        assert torch.equal(fr, free_before)          # allocation never rewrites the stack
        assert np.array_equal(self.pool.cpu().view(self.iview).numpy(), self.o_pool)


CASES = [
    # (ctx_old, new_lens)
    ([0, 5, 16, 40], [3, 30, 0, 17]),
    ([1, 15, 31, 32, 33], [1, 1, 1, 1, 1]),          # decode step across block edges
    ([0, 0, 0], [64, 1, 100]),                        # prompts into an empty cache
    ([200, 7, 0, 64, 130, 9, 77, 1], [0, 0, 0, 0, 0, 0, 0, 0]),   # nothing to append
    ([300, 12, 513], [129, 250, 31]),
]


@pytest.mark.parametrize("case", range(len(CASES)))
@pytest.mark.parametrize("bs,d,dtype", [(16, 128, torch.bfloat16), (32, 64, torch.bfloat16), (16, 64, torch.float32)])
def test_append_matches_oracle(case, bs, d, dtype):
    ctx, new = CASES[case]
    log("append case %d bs=%d d=%d %s" % (case, bs, d, dtype))
    ai = inputs.append_inputs(ctx, new, 3, d, bs, 40 + case, dtype=dtype)
    dc = DeviceCache(ai)
    free0 = dc.free.cpu().clone()
    k_new, v_new = ai.k_new.to(DEV), ai.v_new.to(DEV)
    nctx, status = dc.append(ctx, new, k_new, v_new)
    assert status == attn.APPEND_OK
    assert nctx == dc.oracle_append(ctx, new, k_new, v_new)
    dc.assert_matches_oracle(free0)


@pytest.mark.parametrize("what", ["exhausted", "table_full", "negative"])
def test_failed_append_changes_nothing(what):
    ctx, new = [5, 40, 0], [30, 20, 16]
    ai = inputs.append_inputs(ctx, new, 2, 128, 16, 77, slack_blocks=0, table_slack=0)
    dc = DeviceCache(ai)
    if what == "exhausted":
        dc.count.fill_(len(ai.free_list) - 1)        # one block short
        expect = attn.APPEND_EXHAUSTED
    elif what == "table_full":
        new = [30, 20, 70]                           # request 2 needs 5 table entries, the table has 4
        expect = attn.APPEND_TABLE_FULL
    else:
        new = [30, -1, 16]
        expect = attn.APPEND_INVALID
    if what == "table_full":
        assert -(-(0 + 70) // 16) > dc.table.shape[1]
    snap = (dc.pool.clone(), dc.table.clone(), dc.free.clone(), dc.count.clone())
    k_new, v_new = ai.k_new.to(DEV), ai.v_new.to(DEV)
    if what != "exhausted":
        tot = sum(max(n, 0) for n in new)
        k_new = torch.randn(tot, 2, 128, device=DEV).to(torch.bfloat16)
        v_new = torch.randn(tot, 2, 128, device=DEV).to(torch.bfloat16)
    with pytest.raises(RuntimeError):
        dc.append(ctx, new, k_new, v_new)
    _, status = dc.append(ctx, new, k_new, v_new, check=False)
    assert status == expect
    assert torch.equal(snap[0].view(torch.int16), dc.pool.view(torch.int16))   # bitwise (the pool holds NaN)
    for a, b in zip(snap[1:], (dc.table, dc.free, dc.count)):
        assert torch.equal(a, b)


def test_append_length_above_bound_changes_nothing():
    """A new_lens[r] above the host bound max_new_len (which sizes the copy
    launch) is ATTN_APPEND_INVALID: no block is taken, no table entry, pool
    slot or count changes."""
    ctx, new = [5, 40, 0], [30, 20, 16]
    ai = inputs.append_inputs(ctx, new, 2, 128, 16, 78)
    dc = DeviceCache(ai)
    snap = (dc.pool.clone(), dc.table.clone(), dc.free.clone(), dc.count.clone())
    k_new, v_new = ai.k_new.to(DEV), ai.v_new.to(DEV)
    ctx_d = torch.tensor(ctx, dtype=torch.int32, device=DEV)
    new_d = torch.tensor(new, dtype=torch.int32, device=DEV)
    nctx = torch.full_like(ctx_d, -5)
    _, status = attn.kv_append(k_new, v_new, ctx_d, new_d, dc.pool, dc.table, dc.free, dc.count, 16,
                               max_new_len=29, new_ctx_lens=nctx, check=False)
    torch.cuda.synchronize()
    assert int(status.item()) == attn.APPEND_INVALID
    assert torch.equal(snap[0].view(torch.int16), dc.pool.view(torch.int16))
    for a, b in zip(snap[1:], (dc.table, dc.free, dc.count)):
        assert torch.equal(a, b)
    assert nctx.tolist() == [-5, -5, -5]
    # the same call with the true bound succeeds and matches the oracle
    free0 = dc.free.cpu().clone()
    nctx2, status2 = dc.append(ctx, new, k_new, v_new)
    assert status2 == attn.APPEND_OK and nctx2 == [35, 60, 16]
    dc.oracle_append(ctx, new, k_new, v_new)
    dc.assert_matches_oracle(free0)


def test_release_then_append_reuses_last_released():
    ai = inputs.append_inputs([0, 0], [40, 3], 2, 64, 16, 91)
    dc = DeviceCache(ai)
    free0 = dc.free.cpu().clone()
    k_new, v_new = ai.k_new.to(DEV), ai.v_new.to(DEV)
    dc.append([0, 0], [40, 3], k_new, v_new)
    dc.oracle_append([0, 0], [40, 3], k_new, v_new)
    dc.assert_matches_oracle(free0)
    # request 0 finishes: its three blocks go back, in table order
    rel = dc.table[0, :3].clone()
    attn.kv_release(rel, dc.free, dc.count, dc.num_blocks)
    dc.o_alloc.release(rel.cpu().tolist())
    torch.cuda.synchronize()
    cnt = int(dc.count.item())
    assert dc.free.cpu()[:cnt].tolist() == dc.o_alloc.free
    # a new request (reusing row 0 as empty) takes the last released first
    dc.table[0].fill_(-1)
    dc.o_table[0, :] = -1
    k2 = torch.randn(20, 2, 64, device=DEV).to(torch.bfloat16)
    v2 = torch.randn(20, 2, 64, device=DEV).to(torch.bfloat16)
    dc.append([0, 3], [20, 0], k2, v2)
    dc.oracle_append([0, 3], [20, 0], k2, v2)
    assert dc.table[0, 0].item() == rel[2].item() and dc.table[0, 1].item() == rel[1].item()
    assert np.array_equal(dc.table.cpu().numpy(), dc.o_table)
    assert np.array_equal(dc.pool.cpu().view(dc.iview).numpy(), dc.o_pool)


def test_release_rejects_overflow_and_bad_ids():
    free = torch.zeros(8, dtype=torch.int32, device=DEV)
    count = torch.tensor([6], dtype=torch.int32, device=DEV)
    snap = free.clone()
    st = attn.kv_release(torch.tensor([1, 2, 3], dtype=torch.int32, device=DEV), free, count, 8, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == attn.APPEND_EXHAUSTED and int(count.item()) == 6 and torch.equal(free, snap)
    st = attn.kv_release(torch.tensor([1, 9], dtype=torch.int32, device=DEV), free, count, 8, check=False)
    torch.cuda.synchronize()
    assert int(st.item()) == attn.APPEND_INVALID and int(count.item()) == 6 and torch.equal(free, snap)


def test_decode_loop_append_then_attend():
    """Prompts appended into an empty cache, then three decode steps of
    append-one-token + paged attention; every step's attention output is
    checked against the oracle run on the oracle's own cache."""
    bs, H, d = 16, 4, 128
    prompts = [37, 1, 64, 20]
    ai = inputs.append_inputs([0] * 4, prompts, H, d, bs, 123, slack_blocks=8, table_slack=2)
    dc = DeviceCache(ai)
    ctx = [0] * 4
    new = list(prompts)
    k_new, v_new = ai.k_new.to(DEV), ai.v_new.to(DEV)
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    for step in range(4):
        nctx, status = dc.append(ctx, new, k_new, v_new)
        o_ctx = dc.oracle_append(ctx, new, k_new, v_new)
        assert status == 0 and nctx == o_ctx
        q = torch.randn(sum(new), H, d, device=DEV, generator=g).to(torch.bfloat16)
        ctx_d = torch.tensor(nctx, dtype=torch.int32, device=DEV)
        ql_d = torch.tensor(new, dtype=torch.int32, device=DEV)
        scale = 1.0 / d ** 0.5
        o, lse = attn.paged_attention(q, dc.pool, dc.table, ctx_d, ql_d, bs, scale, max_q_len=max(new),
                                      max_ctx_len=max(nctx))
        torch.cuda.synchronize()
        o_pool = torch.from_numpy(dc.o_pool).view(torch.bfloat16)
        o_tab = torch.from_numpy(dc.o_table)
        o_ref, l_ref = oracle.paged_attention(q.cpu(), o_pool, o_tab, torch.tensor(nctx, dtype=torch.int32),
                                              torch.tensor(new, dtype=torch.int32), bs, scale)
        check_close("decode loop step %d" % step, o, o_ref, lse, l_ref, torch.bfloat16)
        ctx = nctx
        new = [1] * 4
        k_new = torch.randn(4, H, d, device=DEV, generator=g).to(torch.bfloat16)
        v_new = torch.randn(4, H, d, device=DEV, generator=g).to(torch.bfloat16)


@pytest.mark.parametrize("shape", ["chunk_c5", "decode_c4"])
def test_full_size_append_read_back(shape):
    """The append of the chunked-prefill workload (8 requests x 512 new
    tokens onto contexts U[4096, 32768], 32-token pages, 32 heads) and of one
    decode step of the decode workload (64 requests x 1 token onto contexts
    U[512, 16384], 16-token pages): allocation equals the oracle's, the new
    tokens read back through the table bit-exactly, and the old tokens are
    unchanged."""
    cfg = inputs.C5 if shape == "chunk_c5" else inputs.C4
    ctx, ql, _ = inputs.draw_lengths(cfg)
    ctx, ql = [int(c) for c in ctx], [int(q) for q in ql]
    ctx_old = [c - q for c, q in zip(ctx, ql)]
    log("full-size append %s: %d requests, %d new tokens" % (shape, len(ql), sum(ql)))
    ai = inputs.append_inputs(ctx_old, ql, cfg.H, cfg.d, cfg.block_size, cfg.seed, device=DEV)
    bs = cfg.block_size
    table0 = ai.block_table.clone()
    ctx_old_d = torch.tensor(ctx_old, dtype=torch.int32, device=DEV)
    k_old, v_old = attn.gather(ai.pool, ai.block_table, ctx_old_d, bs)
    free = torch.tensor(ai.free_list + [-7] * (ai.pool.shape[0] - len(ai.free_list)), dtype=torch.int32, device=DEV)
    count = torch.tensor([len(ai.free_list)], dtype=torch.int32, device=DEV)
    new_d = torch.tensor(ql, dtype=torch.int32, device=DEV)
    nctx, _ = attn.kv_append(ai.k_new, ai.v_new, ctx_old_d, new_d, ai.pool, ai.block_table, free, count, bs)
    # oracle allocation (no pool needed): one allocate per request in order
    o_alloc = kc.BlockAllocator(ai.pool.shape[0], bs, free=list(ai.free_list))
    o_table = table0.cpu().numpy().copy()
    for r, (c, n) in enumerate(zip(ctx_old, ql)):
        h, w = kc.blocks_for(c, bs), kc.blocks_for(c + n, bs)
        o_table[r, h:w] = o_alloc.allocate_blocks(w - h)
    assert np.array_equal(ai.block_table.cpu().numpy(), o_table)
    assert int(count.item()) == len(o_alloc.free)
    k_all, v_all = attn.gather(ai.pool, ai.block_table, nctx, bs)
    torch.cuda.synchronize()
    k_all, v_all, k_old, v_old = (t.view(torch.int16) for t in (k_all, v_all, k_old, v_old))
    k_nw, v_nw = ai.k_new.view(torch.int16), ai.v_new.view(torch.int16)
    row_old = row_new = row_all = 0
    for r, (c, n) in enumerate(zip(ctx_old, ql)):
        assert torch.equal(k_all[row_all:row_all + c], k_old[row_old:row_old + c])
        assert torch.equal(v_all[row_all:row_all + c], v_old[row_old:row_old + c])
        assert torch.equal(k_all[row_all + c:row_all + c + n], k_nw[row_new:row_new + n])
        assert torch.equal(v_all[row_all + c:row_all + c + n], v_nw[row_new:row_new + n])
        row_old += c
        row_new += n
        row_all += c + n
