"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every symbol include/attn.h declares, and rejects bad arguments with the
documented status codes before anything is launched."""
import ctypes
import re
from pathlib import Path

import pytest

import tiled_online_softmax_attention_amd as attn

ROOT = Path(__file__).resolve().parent.parent
HEADER = ROOT / "include" / "attn.h"

OK, E_NULL, E_SHAPE, E_HD, E_BS, E_DT, E_AL, E_WS, E_LAUNCH, E_SCALE, E_DEV, E_BAD_TABLE, E_OPT = \
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11, -12


def header_functions():
    text = HEADER.read_text()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_library_exports_every_declared_symbol():
    lib = attn.library()
    declared = header_functions()
    assert set(declared) == set(attn.exported_symbols), declared
    for name in declared:
        assert hasattr(lib, name), name


def test_strerror_and_version():
    assert attn.attn_strerror(0) == "ok"
    for code in (E_NULL, E_SHAPE, E_HD, E_BS, E_DT, E_AL, E_WS, E_LAUNCH, E_SCALE, E_DEV, E_BAD_TABLE, E_OPT):
        s = attn.attn_strerror(code)
        assert s and s != "unknown attn status"
    assert attn.attn_strerror(-1234) == "unknown attn status"
    assert attn.attn_version().startswith("attn_gfx950")


# fake, 256-aligned "device" addresses: never dereferenced, because every call
# below fails validation on the host
P = ctypes.c_void_p(1 << 20)
P2 = ctypes.c_void_p(2 << 20)
P3 = ctypes.c_void_p(3 << 20)
P4 = ctypes.c_void_p(4 << 20)
NULL = None


@pytest.fixture(autouse=True)
def _no_launch_on_fake_pointers(request):
    """A case whose arguments pass every host check ends at the device check
    (E_DEV) here; with a GPU present it would launch on the fake pointers
    these tests pass, so it is skipped there."""
    callspec = getattr(request.node, "callspec", None)
    if callspec is not None and callspec.params.get("code") == E_DEV:
        import torch
        if torch.cuda.device_count() > 0:
            pytest.skip("valid arguments on fake pointers would launch on the GPU")


def prefill(**kw):
    a = dict(q=P, k=P2, v=P3, o=P4, lse=NULL, B=1, H=2, N=64, d=128, scale=0.125, causal=1, dtype=0, stream=NULL)
    a.update(kw)
    return attn.attn_prefill_fwd(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), E_NULL), (dict(k=NULL), E_NULL), (dict(v=NULL), E_NULL), (dict(o=NULL), E_NULL),
    (dict(B=0), E_SHAPE), (dict(H=0), E_SHAPE), (dict(N=0), E_SHAPE), (dict(N=-5), E_SHAPE),
    (dict(d=96), E_HD), (dict(d=256), E_HD), (dict(d=0), E_HD),
    (dict(dtype=7), E_DT),
    (dict(q=ctypes.c_void_p((1 << 20) + 8)), E_AL), (dict(lse=ctypes.c_void_p((5 << 20) + 2)), E_AL),
    (dict(scale=float("nan")), E_SCALE), (dict(scale=float("inf")), E_SCALE), (dict(scale=-0.5), E_SCALE),
])
def test_prefill_rejects(kw, code):
    assert prefill(**kw) == code


def paged(**kw):
    a = dict(q=P, k_pool=P2, v_pool=P3, block_table=P4, ctx_lens=P, q_lens=P2, block_size=16, o=P3, lse=NULL,
             num_seqs=4, H=8, d=128, scale=0.1, max_blocks_per_seq=64, kv_block_stride=2 * 8 * 16 * 128,
             num_blocks=100, max_q_len=1, max_ctx_len=1024, dtype=0, workspace=NULL, workspace_bytes=0,
             stream=NULL)
    a.update(kw)
    return attn.paged_attn_fwd(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), E_NULL), (dict(k_pool=NULL), E_NULL), (dict(v_pool=NULL), E_NULL),
    (dict(block_table=NULL), E_NULL), (dict(ctx_lens=NULL), E_NULL), (dict(q_lens=NULL), E_NULL),
    (dict(o=NULL), E_NULL),
    (dict(num_seqs=0), E_SHAPE), (dict(H=0), E_SHAPE), (dict(max_q_len=0), E_SHAPE),
    (dict(max_ctx_len=0), E_SHAPE), (dict(max_q_len=2000), E_SHAPE), (dict(num_blocks=0), E_SHAPE),
    (dict(max_blocks_per_seq=10), E_SHAPE),              # 1024 / 16 = 64 pages needed
    (dict(kv_block_stride=100), E_SHAPE),
    (dict(d=80), E_HD), (dict(block_size=8), E_BS), (dict(block_size=64), E_BS),
    (dict(dtype=1), E_DT),
    (dict(o=ctypes.c_void_p((3 << 20) + 4)), E_AL),
    (dict(scale=-1.0), E_SCALE),
])
def test_paged_rejects(kw, code):
    assert paged(**kw) == code


def test_paged_workspace_required_when_split():
    need = attn.paged_attn_workspace_bytes(4, 8, 128, 16, 1, 1 << 16)
    assert need > 0
    assert paged(max_ctx_len=1 << 16, max_blocks_per_seq=4096, workspace=NULL, workspace_bytes=0) == E_WS
    assert paged(max_ctx_len=1 << 16, max_blocks_per_seq=4096, workspace=P, workspace_bytes=need - 1) == E_WS
    assert paged(max_ctx_len=1 << 16, max_blocks_per_seq=4096, workspace=ctypes.c_void_p((1 << 20) + 16),
                 workspace_bytes=need) == E_AL


def test_workspace_plan_is_pure_and_sane():
    # one split -> no workspace
    assert attn.paged_attn_workspace_bytes(64, 32, 128, 16, 1, 64) == 0
    a = attn.paged_attn_workspace_bytes(64, 32, 128, 16, 1, 16384)
    b = attn.paged_attn_workspace_bytes(64, 32, 128, 16, 1, 16384)
    assert a == b > 0
    # bad geometry -> 0
    assert attn.paged_attn_workspace_bytes(0, 32, 128, 16, 1, 100) == 0
    assert attn.paged_attn_workspace_bytes(4, 32, 128, 8, 1, 100) == 0


def _max_splits(num_seqs, H, H_kv, d, bs, max_q, max_ctx):
    """Splits per (row, head) the plan chose, read back from the workspace
    size: d + 1 fp32 per (row, head, split), the O part rounded up to 256 B."""
    ws = attn.paged_attn_gqa_workspace_bytes(num_seqs, H, H_kv, d, bs, max_q, max_ctx, None)
    return ws // (num_seqs * max_q * H * (d + 1) * 4) if ws else 1


@pytest.mark.parametrize("args,splits", [
    # 64-request decode on 16-token pages (decode MFMA kernel, plain heads at
    # d = 128 on 2048 pairs): 2048-key splits
    ((64, 32, 32, 128, 16, 1, 16384), 8),
    # ... 16 such requests (512 pairs): 1024-key splits
    ((16, 32, 32, 128, 16, 1, 16384), 16),
    # the same at d = 64 (vector kernel): 384-token splits
    ((64, 32, 32, 64, 16, 1, 16384), 43),
    # the same lengths on 4 K/V heads (tile kernel, decode-length rows): 1280-key splits
    ((64, 32, 4, 128, 16, 1, 16384), 13),
    # ... 128 such requests (512 pairs, still the tile kernel): 2368-key splits
    ((128, 32, 4, 128, 16, 1, 16384), 7),
    # ... and 256 (1024 pairs: decode MFMA kernel, 8 rows): 2048-key splits
    ((256, 32, 4, 128, 16, 1, 16384), 8),
    # chunked prefill, 8 x 512 rows on 32-token pages (tile kernel): 8192-key splits
    ((8, 32, 32, 128, 32, 512, 33280), 5),
    # small decode batches: splits halved down to one 16-token page per wave, no further
    ((4, 32, 32, 128, 16, 1, 900), 15),
    ((4, 32, 32, 128, 16, 1, 64), 1),
])
def test_split_plans(args, splits):
    """The split plans measured best on the benchmark shapes (host-side plan,
    read back through the workspace size)."""
    assert _max_splits(*args) == splits


def gather(**kw):
    a = dict(k_pool=P, v_pool=P2, block_table=P3, ctx_lens=P4, block_size=16, num_seqs=2, H=4, d=64,
             max_blocks_per_seq=8, kv_block_stride=2 * 4 * 16 * 64, max_ctx_len=100, dtype=0, k_out=P,
             v_out=P2, stream=NULL)
    a.update(kw)
    return attn.paged_kv_gather(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(k_pool=NULL), E_NULL), (dict(k_out=NULL), E_NULL), (dict(num_seqs=0), E_SHAPE),
    (dict(max_blocks_per_seq=2), E_SHAPE), (dict(d=32), E_HD), (dict(block_size=24), E_BS),
    (dict(dtype=3), E_DT), (dict(v_out=ctypes.c_void_p((2 << 20) + 2)), E_AL),
])
def test_gather_rejects(kw, code):
    assert gather(**kw) == code


def test_valid_call_without_gpu_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert prefill() == E_DEV


def append(**kw):
    a = dict(k_new=P, v_new=P2, ctx_lens=P3, new_lens=P4, k_pool=P, v_pool=P2, block_table=P3, free_blocks=P4,
             free_count=P, new_ctx_lens=P2, status=P3, block_size=16, num_seqs=4, H=8, d=128,
             max_blocks_per_seq=64, kv_block_stride=2 * 8 * 16 * 128, num_blocks=100, max_new_len=16, dtype=0,
             stream=NULL)
    a.update(kw)
    return attn.paged_kv_append(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(ctx_lens=NULL), E_NULL), (dict(new_lens=NULL), E_NULL), (dict(k_pool=NULL), E_NULL),
    (dict(v_pool=NULL), E_NULL), (dict(block_table=NULL), E_NULL), (dict(free_blocks=NULL), E_NULL),
    (dict(free_count=NULL), E_NULL), (dict(status=NULL), E_NULL), (dict(k_new=NULL), E_NULL),
    (dict(v_new=NULL), E_NULL),
    (dict(num_seqs=0), E_SHAPE), (dict(H=0), E_SHAPE), (dict(max_blocks_per_seq=0), E_SHAPE),
    (dict(num_blocks=0), E_SHAPE), (dict(max_new_len=-1), E_SHAPE), (dict(kv_block_stride=100), E_SHAPE),
    (dict(new_ctx_lens=P3), E_SHAPE),                    # aliases ctx_lens
    (dict(d=96), E_HD), (dict(block_size=8), E_BS), (dict(dtype=5), E_DT),
    (dict(k_pool=ctypes.c_void_p((1 << 20) + 8)), E_AL), (dict(v_new=ctypes.c_void_p((2 << 20) + 4)), E_AL),
    (dict(), E_DEV),                                    # valid arguments: only the device check is left
    (dict(k_new=NULL, v_new=NULL, max_new_len=0), E_DEV),
])
def test_append_rejects(kw, code):
    assert append(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(blocks=NULL), E_NULL), (dict(free_blocks=NULL), E_NULL), (dict(free_count=NULL), E_NULL),
    (dict(status=NULL), E_NULL), (dict(n=-1), E_SHAPE), (dict(num_blocks=0), E_SHAPE),
    (dict(blocks=NULL, n=0), E_DEV), (dict(), E_DEV),
])
def test_release_rejects(kw, code):
    a = dict(blocks=P, n=4, free_blocks=P2, free_count=P3, status=P4, num_blocks=100, stream=NULL)
    a.update(kw)
    assert attn.paged_kv_release(**a) == code


@pytest.mark.parametrize("kw,code", [
    (dict(H_kv=0), E_SHAPE), (dict(H_kv=3), E_SHAPE), (dict(H_kv=16), E_SHAPE), (dict(), E_DEV),
    (dict(k=NULL), E_NULL), (dict(d=80), E_HD),
])
def test_prefill_gqa_rejects(kw, code):
    a = dict(q=P, k=P2, v=P3, o=P4, lse=NULL, B=1, H=8, H_kv=2, N=64, d=128, scale=0.125, causal=1, dtype=0,
             opts=None, stream=NULL)
    a.update(kw)
    assert attn.attn_prefill_gqa_fwd(**a) == code


@pytest.mark.parametrize("kw,code", [
    (dict(H_kv=0), E_SHAPE), (dict(H_kv=3), E_SHAPE), (dict(H_kv=16), E_SHAPE),
    (dict(kv_block_stride=2 * 16 * 128 - 16), E_SHAPE),         # below H_kv * bs * d
    (dict(), E_DEV),
])
def test_paged_gqa_rejects(kw, code):
    a = dict(q=P, k_pool=P2, v_pool=P3, block_table=P4, ctx_lens=P, q_lens=P2, block_size=16, o=P3, lse=NULL,
             num_seqs=4, H=8, H_kv=2, d=128, scale=0.1, max_blocks_per_seq=64, kv_block_stride=2 * 2 * 16 * 128,
             num_blocks=100, max_q_len=1, max_ctx_len=1024, dtype=0, workspace=NULL, workspace_bytes=0,
             opts=None, stream=NULL)
    a.update(kw)
    if code == E_DEV and attn.paged_attn_gqa_workspace_bytes(4, 8, 2, 128, 16, 1, 1024):
        a["workspace"] = ctypes.c_void_p(8 << 20)
        a["workspace_bytes"] = attn.paged_attn_gqa_workspace_bytes(4, 8, 2, 128, 16, 1, 1024)
    assert attn.paged_attn_gqa_fwd(**a) == code


def test_gqa_workspace_matches_plain_at_equal_heads():
    for args in ((64, 32, 128, 16, 1, 16384), (8, 32, 128, 32, 512, 32768), (4, 8, 64, 16, 3, 100)):
        n, H, d, bs, mq, mc = args
        assert attn.paged_attn_gqa_workspace_bytes(n, H, H, d, bs, mq, mc) == attn.paged_attn_workspace_bytes(*args)
    assert attn.paged_attn_gqa_workspace_bytes(4, 8, 3, 128, 16, 1, 100) == 0


def bwd(**kw):
    a = dict(q=P, k=P2, v=P3, o=P4, lse=P, dout=P2, dq=P3, dk=P4, dv=P, B=2, H=8, H_kv=2, N=100, d=128, scale=0.125,
             causal=1, dtype=0, workspace=P2, workspace_bytes=2 * 8 * 100 * 8, opts=None, stream=NULL)
    a.update(kw)
    return attn.attn_prefill_bwd(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(q=NULL), E_NULL), (dict(lse=NULL), E_NULL), (dict(dout=NULL), E_NULL), (dict(dv=NULL), E_NULL),
    (dict(B=0), E_SHAPE), (dict(N=0), E_SHAPE), (dict(H_kv=3), E_SHAPE), (dict(H_kv=0), E_SHAPE),
    (dict(d=96), E_HD), (dict(dtype=1), E_DT),
    (dict(dq=ctypes.c_void_p((3 << 20) + 8)), E_AL), (dict(lse=ctypes.c_void_p((1 << 20) + 2)), E_AL),
    (dict(scale=-1.0), E_SCALE), (dict(scale=float("nan")), E_SCALE),
    (dict(workspace=NULL), E_WS), (dict(workspace_bytes=2 * 8 * 100 * 8 - 1), E_WS),
    (dict(workspace=ctypes.c_void_p((2 << 20) + 8)), E_AL),
    (dict(N=1 << 24), E_SHAPE),                                  # N * d * 2 bytes must stay below 4 GiB
    (dict(), E_DEV),
])
def test_bwd_rejects(kw, code):
    assert bwd(**kw) == code


def test_bwd_workspace_bytes():
    assert attn.attn_prefill_bwd_workspace_bytes(2, 8, 100) == 2 * 8 * 100 * 8
    assert attn.attn_prefill_bwd_workspace_bytes(16, 32, 8192) == 16 * 32 * 8192 * 8
    for bad in ((0, 8, 100), (2, 0, 100), (2, 8, 0), (-1, 8, 100)):
        assert attn.attn_prefill_bwd_workspace_bytes(*bad) == 0


def opts(**kw):
    return attn._opts(kw)


def test_launch_opts_default_values():
    o = attn.LaunchOpts()
    for name, _ in attn.LaunchOpts._fields_:
        setattr(o, name, 77)
    attn.attn_launch_opts_default(ctypes.byref(o))
    want = dict(prefill_kernel=-1, prefill_pair=-1, prefill_order=-1, paged_path=-1, paged_split_tokens=0,
                paged_decode_heads=0, paged_tile_map=-1, bwd_pair_q=-1, bwd_pair_kv=-1, paged_tile_kernel=-1)
    assert {name: getattr(o, name) for name, _ in attn.LaunchOpts._fields_} == want
    attn.attn_launch_opts_default(None)   # NULL is a no-op


@pytest.mark.parametrize("field,bad", [
    ("prefill_kernel", 2), ("prefill_kernel", -2), ("prefill_pair", 2), ("prefill_order", 2), ("prefill_order", 4),
    ("paged_path", 3), ("paged_split_tokens", -1), ("paged_decode_heads", 3), ("paged_decode_heads", 16),
    ("paged_tile_map", 3), ("bwd_pair_q", 5), ("bwd_pair_kv", -3), ("paged_tile_kernel", 3),
    ("paged_tile_kernel", -2),
])
def test_out_of_range_options_rejected(field, bad):
    """Every entry point that takes opts rejects an out-of-range field with
    ATTN_ERR_OPTION before anything is launched (and the workspace query
    answers 0)."""
    o = opts(**{field: bad})
    a = dict(q=P, k=P2, v=P3, o=P4, lse=NULL, B=1, H=8, H_kv=2, N=64, d=128, scale=0.125, causal=1, dtype=0,
             opts=o, stream=NULL)
    assert attn.attn_prefill_gqa_fwd(**a) == E_OPT
    b = dict(q=P, k_pool=P2, v_pool=P3, block_table=P4, ctx_lens=P, q_lens=P2, block_size=16, o=P3, lse=NULL,
             num_seqs=4, H=8, H_kv=2, d=128, scale=0.1, max_blocks_per_seq=64, kv_block_stride=2 * 2 * 16 * 128,
             num_blocks=100, max_q_len=1, max_ctx_len=1024, dtype=0, workspace=ctypes.c_void_p(8 << 20),
             workspace_bytes=1 << 30, opts=o, stream=NULL)
    assert attn.paged_attn_gqa_fwd(**b) == E_OPT
    assert attn.paged_attn_gqa_workspace_bytes(4, 8, 2, 128, 16, 1, 1024, o) == 0
    assert bwd(opts=o) == E_OPT


def test_decode_heads_option_must_divide_the_group():
    b = dict(q=P, k_pool=P2, v_pool=P3, block_table=P4, ctx_lens=P, q_lens=P2, block_size=16, o=P3, lse=NULL,
             num_seqs=4, H=12, H_kv=4, d=128, scale=0.1, max_blocks_per_seq=64, kv_block_stride=2 * 4 * 16 * 128,
             num_blocks=100, max_q_len=1, max_ctx_len=1024, dtype=0, workspace=ctypes.c_void_p(8 << 20),
             workspace_bytes=1 << 30, opts=opts(paged_decode_heads=2), stream=NULL)
    assert attn.paged_attn_gqa_fwd(**b) == E_OPT          # groups of 3
    b["opts"] = opts(paged_decode_heads=1)
    assert attn.paged_attn_gqa_fwd(**b) == E_DEV
    b.update(H=32, block_size=32, kv_block_stride=2 * 4 * 32 * 128, opts=opts(paged_decode_heads=8))
    assert attn.paged_attn_gqa_fwd(**b) == E_OPT          # 8 heads per workgroup needs 16-token pages


def test_split_option_sets_the_workspace():
    """A forced split size changes the plan and so the workspace the call
    needs; the automatic plan equals passing no options."""
    auto = attn.paged_attn_gqa_workspace_bytes(64, 32, 32, 128, 16, 1, 16384, None)
    assert attn.paged_attn_gqa_workspace_bytes(64, 32, 32, 128, 16, 1, 16384, opts()) == auto
    s256 = attn.paged_attn_gqa_workspace_bytes(64, 32, 32, 128, 16, 1, 16384, opts(paged_split_tokens=256))
    assert s256 == (64 * 32 * 64 * 128 * 4 + 255) // 256 * 256 + 64 * 32 * 64 * 4
    # on the vector kernel a split longer than every context is one split (the
    # decode MFMA kernel, this shape's default, caps a split at 128 pages)
    assert attn.paged_attn_gqa_workspace_bytes(64, 32, 32, 128, 16, 1, 16384,
                                               opts(paged_split_tokens=1 << 20, paged_path=0)) == 0


def test_decode_mfma_plan():
    """Decode on grouped heads (32 query heads on 4 K/V heads, one query row:
    8 rows of the decode MFMA kernel's 16) on that kernel splits the context
    into 1024-key splits for a 64-request batch (256 pairs: no doubling to
    2048 below 1024 pairs), caps a forced split at 128 pages, and the kernel
    is not taken for more rows than 16 (q_len 3 on groups of 8)."""
    def ws(splits, rows=64 * 1, H=32):
        return (rows * H * splits * 128 * 4 + 255) // 256 * 256 + rows * H * splits * 4
    assert attn.paged_attn_gqa_workspace_bytes(64, 32, 4, 128, 16, 1, 16384, opts(paged_path=2)) == ws(16)
    assert attn.paged_attn_gqa_workspace_bytes(64, 32, 4, 128, 16, 1, 16384,
                                               opts(paged_split_tokens=4096, paged_path=2)) == ws(8)
    assert attn.paged_attn_gqa_workspace_bytes(64, 32, 4, 128, 32, 1, 16384,
                                               opts(paged_split_tokens=8192, paged_path=2)) == ws(4)
    # 3 rows x 8 heads = 24 > 16: the tile kernel's plan (64-key units, no page cap)
    assert attn.paged_attn_gqa_workspace_bytes(64, 32, 4, 128, 16, 3, 16384,
                                               opts(paged_split_tokens=4096, paged_path=2)) == ws(4, rows=64 * 3)


def check_call(**kw):
    a = dict(block_table=P, ctx_lens=P2, q_lens=P3, num_seqs=4, block_size=16, max_blocks_per_seq=64, num_blocks=256,
             max_q_len=1, max_ctx_len=1024, status=P4, stream=NULL)
    a.update(kw)
    return attn.paged_attn_check(**a)


@pytest.mark.parametrize("kw,code", [
    (dict(block_table=NULL), E_NULL), (dict(ctx_lens=NULL), E_NULL), (dict(q_lens=NULL), E_NULL),
    (dict(status=NULL), E_NULL),
    (dict(num_seqs=0), E_SHAPE), (dict(max_blocks_per_seq=0), E_SHAPE), (dict(num_blocks=0), E_SHAPE),
    (dict(max_q_len=0), E_SHAPE), (dict(max_ctx_len=0), E_SHAPE),
    (dict(block_size=8), E_BS), (dict(block_size=64), E_BS),
    (dict(status=ctypes.c_void_p((4 << 20) + 2)), E_AL), (dict(block_table=ctypes.c_void_p((1 << 20) + 1)), E_AL),
    (dict(), E_DEV),
])
def test_paged_check_rejects(kw, code):
    assert check_call(**kw) == code


def test_debug_flag_does_not_change_host_checks(monkeypatch):
    """ATTN_DEBUG=1 adds a device check after the host checks; host errors
    come first, unchanged."""
    monkeypatch.setenv("ATTN_DEBUG", "1")
    assert paged(q=NULL) == E_NULL
    assert paged(block_size=8) == E_BS
