"""The device-side check of the paged-attention contract (paged_attn_check)
and the ATTN_DEBUG=1 mode of the paged entry points.

The "bad" block ids the debug-mode tests hand to paged_attn_fwd are chosen
so that even an attention launch that went ahead would read only memory of
the test's own allocation: the pool tensor carries four blocks beyond the
declared num_blocks, and the out-of-contract id is the first of them."""
import ctypes
import os

import pytest
import torch

import tiled_online_softmax_attention_amd as attn
from tiled_online_softmax_attention_amd import inputs
from parity import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def small_case(seed=3, ql=1):
    ctx = [40, 700, 1, 257, 1024]
    qls = [min(ql, c) for c in ctx]
    return inputs.build_paged(ctx, qls, 4, 128, 16, seed, DEV, max_blocks_per_seq=70)


def check(pi, block_table=None, ctx_lens=None, q_lens=None, max_q_len=None, max_ctx_len=None, num_blocks=None):
    bt = pi.block_table if block_table is None else block_table
    cl = pi.ctx_lens if ctx_lens is None else ctx_lens
    qlen = pi.q_lens if q_lens is None else q_lens
    status = torch.full((1,), 0x7fffffff, dtype=torch.int32, device=DEV)   # must be overwritten
    attn.paged_check(bt, cl, qlen, pi.block_size, pi.num_blocks if num_blocks is None else num_blocks,
                     int(pi.q_lens.max()) if max_q_len is None else max_q_len,
                     int(pi.ctx_lens.max()) if max_ctx_len is None else max_ctx_len, status=status)
    torch.cuda.synchronize()
    return int(status.item())


def test_check_valid_inputs():
    pi = small_case()
    assert check(pi) == attn.CHECK_OK
    # entries past ceil(ctx / block_size) are never read: garbage there is fine
    bt = pi.block_table.clone()
    bt[2, 1:] = 123456789
    assert check(pi, block_table=bt) == attn.CHECK_OK


@pytest.mark.parametrize("value", [-1, "num_blocks", 1 << 30])
def test_check_flags_bad_table_entry(value):
    pi = small_case()
    bt = pi.block_table.clone()
    bt[1, 43] = pi.num_blocks if value == "num_blocks" else value   # request 1 uses 44 blocks
    log("check table entry %s" % value)
    assert check(pi, block_table=bt) == attn.CHECK_TABLE
    bt = pi.block_table.clone()
    bt[4, 0] = -7
    assert check(pi, block_table=bt) == attn.CHECK_TABLE


def test_check_flags_bad_lengths():
    pi = small_case(ql=1)
    cases = {
        "q_len 0": (None, torch.tensor([1, 0, 1, 1, 1], dtype=torch.int32)),
        "q_len > ctx": (None, torch.tensor([1, 1, 2, 1, 1], dtype=torch.int32)),
        "ctx > max_ctx_len": (torch.tensor([40, 700, 1, 257, 1025], dtype=torch.int32), None),
        "q_len > max_q_len": (None, torch.tensor([1, 1, 1, 2, 1], dtype=torch.int32)),
        "ctx past the table": (torch.tensor([40, 70 * 16 + 1, 1, 257, 1024], dtype=torch.int32), None),
    }
    for name, (cl, qlen) in cases.items():
        log("check " + name)
        got = check(pi, ctx_lens=None if cl is None else cl.to(DEV), q_lens=None if qlen is None else qlen.to(DEV),
                    max_q_len=1, max_ctx_len=1024 if name != "ctx past the table" else 70 * 16 + 1)
        assert got & attn.CHECK_LENGTHS, name
    # both problems at once
    bt = pi.block_table.clone()
    bt[0, 0] = pi.num_blocks
    got = check(pi, block_table=bt, q_lens=torch.tensor([1, 0, 1, 1, 1], dtype=torch.int32, device=DEV), max_q_len=1)
    assert got == attn.CHECK_LENGTHS | attn.CHECK_TABLE


def _raw_paged(pi, pool, block_table, num_blocks, out, lse, ws):
    H, bs, d = pi.H, pi.block_size, pi.d
    k_ptr = pool.data_ptr()
    v_ptr = k_ptr + H * bs * d * pool.element_size()
    return attn.paged_attn_fwd(
        ctypes.c_void_p(pi.q.data_ptr()), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr),
        ctypes.c_void_p(block_table.data_ptr()), ctypes.c_void_p(pi.ctx_lens.data_ptr()),
        ctypes.c_void_p(pi.q_lens.data_ptr()), bs, ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
        pi.num_seqs, H, d, pi.scale, block_table.shape[1], 2 * H * bs * d, num_blocks, int(pi.q_lens.max()),
        int(pi.ctx_lens.max()), attn.ATTN_BF16, ctypes.c_void_p(ws.data_ptr()), ws.numel(),
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


@pytest.fixture
def debug_env():
    old = os.environ.get("ATTN_DEBUG")
    os.environ["ATTN_DEBUG"] = "1"
    # the library reads the C environment; make sure the setting reached it
    libc = ctypes.CDLL(None)
    libc.getenv.restype = ctypes.c_char_p
    assert libc.getenv(b"ATTN_DEBUG") == b"1"
    yield
    if old is None:
        os.environ.pop("ATTN_DEBUG", None)
    else:
        os.environ["ATTN_DEBUG"] = old


@pytest.mark.parametrize("ql", [1, 3, 200])
def test_debug_mode_rejects_bad_table_without_launching(debug_env, ql):
    pi = small_case(seed=5, ql=ql)
    P = pi.num_blocks
    # four blocks beyond the declared pool, inside this allocation
    pool = torch.cat([pi.pool, torch.zeros((4,) + tuple(pi.pool.shape[1:]), dtype=pi.pool.dtype, device=DEV)])
    bt = pi.block_table.clone()
    bt[3, 5] = P
    ws_bytes = attn.paged_attn_workspace_bytes(pi.num_seqs, pi.H, pi.d, pi.block_size, int(pi.q_lens.max()),
                                               int(pi.ctx_lens.max()))
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=DEV)
    out = torch.full_like(pi.q, float("nan"))
    lse = torch.full(pi.q.shape[:2], float("nan"), dtype=torch.float32, device=DEV)
    log("debug mode, bad table, q_len %d" % ql)
    rc = _raw_paged(pi, pool, bt, P, out, lse, ws)
    torch.cuda.synchronize()
    assert rc == attn.ERR_BAD_TABLE
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()   # nothing was launched
    # a length that breaks the contract (request 2 has one cached token but
    # two query rows), with the total row count kept, so the q and o tensors
    # would still bound every row had a launch gone ahead
    qls = pi.q_lens.cpu().tolist()
    qls[2] = 2
    qls[0 if ql == 1 else 3] -= 1
    bad_q = torch.tensor(qls, dtype=torch.int32, device=DEV)
    with pytest.raises(attn.AttnError) as e:
        attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, bad_q, pi.block_size,
                             max_q_len=max(qls), max_ctx_len=1024, out=out, lse=lse)
    assert e.value.code == attn.ERR_BAD_TABLE
    torch.cuda.synchronize()
    assert torch.isnan(out.float()).all() and torch.isnan(lse).all()


@pytest.mark.parametrize("ql", [1, 200])
def test_debug_mode_valid_inputs_same_bits(debug_env, ql):
    pi = small_case(seed=6, ql=ql)
    o1, l1 = attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size)
    torch.cuda.synchronize()
    del os.environ["ATTN_DEBUG"]
    o2, l2 = attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size)
    torch.cuda.synchronize()
    os.environ["ATTN_DEBUG"] = "1"
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1, l2)
