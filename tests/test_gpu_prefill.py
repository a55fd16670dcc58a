"""GPU parity of attn_prefill_fwd against the fp64 oracle (through the C ABI)."""
import math

import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_attention_amd as attn
from tiled_online_softmax_attention_amd import inputs
from parity import check_close, log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def run_case(B, H, N, d, dtype, causal, seed, options=None):
    cfg = inputs.PrefillConfig("case", B, H, N, d, dtype, causal, seed)
    log("prefill case B=%d H=%d N=%d d=%d %s causal=%d seed=%d options=%s"
        % (B, H, N, d, dtype, causal, seed, options))
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    o, lse = attn.prefill(q, k, v, causal, cfg.scale, options=options)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.attention(q, k, v, cfg.scale, causal)
    return check_close("B%dH%dN%dd%d" % (B, H, N, d), o, o_ref, lse, lse_ref, dtype), (q, k, v, o, lse)


def test_c1_fp32_noncausal_full():
    c = inputs.C1
    run_case(c.B, c.H, c.N, c.d, c.dtype, c.causal, c.seed)


def test_c2_bf16_causal_full():
    c = inputs.C2
    run_case(c.B, c.H, c.N, c.d, c.dtype, c.causal, c.seed)


@pytest.mark.parametrize("N", [1, 2, 31, 64, 127, 128, 129, 200, 257, 640])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_ragged_lengths(N, causal):
    run_case(1, 3, N, 128, torch.bfloat16, causal, 100 + N)


@pytest.mark.parametrize("N", [1, 65, 300])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_head_dim_64(N, causal):
    run_case(2, 2, N, 64, torch.bfloat16, causal, 200 + N)


@pytest.mark.parametrize("N,d", [(1, 64), (33, 128), (257, 64), (300, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_fp32_shapes(N, d, causal):
    run_case(1, 2, N, d, torch.float32, causal, 300 + N)


@pytest.mark.parametrize("pair", [False, True])
def test_pair_mode_matches_oracle(pair):
    run_case(2, 4, 1000, 128, torch.bfloat16, True, 7, options={"prefill_pair": int(pair)})


@pytest.mark.parametrize("B,H,N,d", [(1, 32, 2048, 128), (1, 8, 1000, 64), (2, 4, 640, 128), (1, 3, 700, 64),
                                     (1, 12, 1500, 128)])
def test_tile_order_bit_identical(B, H, N, d):
    """The tile orders (per-head heavy-first in XCD ranges, complementary,
    tile-major) only change which workgroup runs which query tile: output
    and LSE are bit-identical across them, and match the oracle."""
    cfg = inputs.PrefillConfig("order", B, H, N, d, torch.bfloat16, True, 12 + N)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    outs = []
    for order in (0, 1, 3):
        outs.append(attn.prefill(q, k, v, True, cfg.scale, options={"prefill_order": order}))
        torch.cuda.synchronize()
    o0, l0 = outs[0]
    for o1, l1 in outs[1:]:
        assert torch.equal(o0.view(torch.int16), o1.view(torch.int16)) and torch.equal(l0, l1)
    if B * H * N <= 8 * 1000:
        o_ref, l_ref = oracle.attention(q, k, v, cfg.scale, True)
        check_close("order", outs[-1][0], o_ref, outs[-1][1], l_ref, torch.bfloat16)


@pytest.mark.parametrize("N", [64, 65, 128, 192, 256, 320, 384])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_key_tile_counts(N, d, causal):
    """Two to twelve 32-key tiles per query tile: odd and even tile counts and
    the boundary between unmasked and masked tiles of the double-buffered
    key loop."""
    run_case(1, 2, N, d, torch.bfloat16, causal, 400 + N + d)


@pytest.mark.parametrize("N", [1, 31, 200, 256, 257, 640, 1100])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_pipelined_key_loop_matches_oracle(N, causal, d):
    """The software-pipelined key loop (prefill_kernel = 1): no full tile,
    partial 128-row tiles, pipelined runs of 4 and more key tiles followed by
    masked tiles, and rows past N in the last tile."""
    run_case(2, 3, N, d, torch.bfloat16, causal, 700 + N + d, options={"prefill_kernel": 1})


@pytest.mark.parametrize("B,H,H_kv,N,d,causal", [(1, 8, 8, 777, 128, True), (2, 4, 4, 300, 64, True),
                                                 (1, 8, 2, 1100, 128, True), (1, 4, 4, 640, 128, False),
                                                 (1, 32, 32, 2048, 128, True)])
def test_key_loops_bit_identical(B, H, H_kv, N, d, causal):
    """The plain and the pipelined key loop apply the same operations to O, l
    and the offset in the same order: identical bits, for every tile order
    and pairing they run under."""
    cfg = inputs.PrefillConfig("loops", B, H, N, d, torch.bfloat16, causal, 31 + N, H_kv=H_kv)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    ref = None
    for kernel in (0, 1):
        for pair in (0, 1):
            o, lse = attn.prefill(q, k, v, causal, cfg.scale, options={"prefill_kernel": kernel, "prefill_pair": pair})
            torch.cuda.synchronize()
            if ref is None:
                ref = (o, lse)
            else:
                assert torch.equal(ref[0].view(torch.int16), o.view(torch.int16)) and torch.equal(ref[1], lse), \
                    (kernel, pair)
    if B * H * N <= 8 * 1100:
        o_ref, l_ref = oracle.attention(q, k, v, cfg.scale, causal)
        check_close("loops", ref[0], o_ref, ref[1], l_ref, torch.bfloat16)


@pytest.mark.parametrize("N", [777, 1000])
def test_deterministic_and_pair_independent(N):
    """Repeat calls give the same bits, and so do one query tile per
    workgroup and paired tiles t / n-1-t (per-head ranges, where pairing
    applies; N = 777 has 7 tiles, so the middle tile runs alone)."""
    cfg = inputs.PrefillConfig("det", 1, 8, N, 128, torch.bfloat16, True, 9)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    o1, l1 = attn.prefill(q, k, v, True, cfg.scale)
    o2, l2 = attn.prefill(q, k, v, True, cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    res = {}
    for pair in (0, 1):
        res[pair] = attn.prefill(q, k, v, True, cfg.scale, options={"prefill_order": 0, "prefill_pair": pair})
        torch.cuda.synchronize()
    # same tiles, same order of key tiles within a tile: identical bits
    for o3, l3 in res.values():
        assert torch.equal(o1, o3) and torch.equal(l1, l3)


@pytest.mark.parametrize("N,H,H_kv,causal", [(131072, 1, 1, True), (65536, 4, 1, True), (65536, 2, 2, False)])
def test_long_context_sampled_rows(N, H, H_kv, causal):
    """Long contexts in the default launch configuration: 512 or 1024 query
    tiles against up to 4096 key tiles of one head (the first row's single key
    and the last row's full sum of fp32 probabilities both in the sample),
    four query heads on one K/V head, and a non-causal case.  32 seeded
    rows plus edge rows against the oracle."""
    cfg = inputs.PrefillConfig("long", 1, H, N, 128, torch.bfloat16, causal, 7 + N + H, H_kv=H_kv)
    log("long context N=%d H=%d H_kv=%d causal=%d" % (N, H, H_kv, causal))
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    o, lse = attn.prefill(q, k, v, causal, cfg.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    trip = inputs.sample_triples(cfg.seed, 32, (1, H, N),
                                 edge=[(0, 0, 0), (0, 0, 1), (0, H - 1, 127), (0, H - 1, 128), (0, 0, N - 128),
                                       (0, H - 1, N - 1)])
    qs, ks, vs = q.cpu(), k.cpu(), v.cpu()
    o_ref, l_ref = oracle.attention_rows(qs, ks, vs, cfg.scale, causal, [0] * len(trip), [h for _, h, _ in trip],
                                         [r for _, _, r in trip])
    og = torch.stack([o[0, h, r] for _, h, r in trip])
    lg = torch.stack([lse[0, h, r] for _, h, r in trip])
    check_close("long", og, o_ref, lg, l_ref, torch.bfloat16)


def test_scale_zero_closed_form():
    """scale 0: O_i = mean of V[0..i], LSE_i = ln(i+1)."""
    cfg = inputs.PrefillConfig("s0", 1, 2, 300, 128, torch.bfloat16, True, 10)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    o, lse = attn.prefill(q, k, v, True, 0.0)
    torch.cuda.synchronize()
    vv = v.double().cpu()
    cnt = torch.arange(1, 301, dtype=torch.float64)
    want = vv.cumsum(dim=2) / cnt[None, None, :, None]
    assert (o.double().cpu() - want).abs().max() < 2e-2
    assert (lse.double().cpu() - cnt.log()[None, None]).abs().max() < 1e-4


def test_constant_v_rows():
    cfg = inputs.PrefillConfig("cv", 1, 2, 500, 128, torch.bfloat16, True, 11)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    c = torch.randn(128, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16)
    v = c.to(DEV).expand(1, 2, 500, 128).contiguous()
    o, _ = attn.prefill(q, k, v, True, cfg.scale)
    torch.cuda.synchronize()
    err = (o.float() - c.float().to(DEV)).abs()
    ulp = (c.float().abs().to(DEV) * 2.0 ** -7).clamp_min(2.0 ** -133)
    assert bool((err <= ulp).all()), float((err / ulp).max())


def test_output_canaries_untouched():
    """Outputs written exactly in bounds: guard words around O and LSE survive."""
    B, H, N, d = 1, 2, 200, 128
    cfg = inputs.PrefillConfig("canary", B, H, N, d, torch.bfloat16, True, 12)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    G = 4096
    obuf = torch.full((2 * G + B * H * N * d,), 7.0, dtype=torch.bfloat16, device=DEV)
    lbuf = torch.full((2 * G + B * H * N,), 3.0, dtype=torch.float32, device=DEV)
    o = obuf[G:G + B * H * N * d].view(B, H, N, d)
    lse = lbuf[G:G + B * H * N].view(B, H, N)
    attn.prefill(q, k, v, True, cfg.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((obuf[:G] == 7.0).all()) and bool((obuf[-G:] == 7.0).all())
    assert bool((lbuf[:G] == 3.0).all()) and bool((lbuf[-G:] == 3.0).all())


@pytest.mark.slow
def test_c3_full_size_sampled_rows():
    """The 16x32x8192x128 causal workload in the benchmark's launch
    configuration; 64 seeded (b, h, row) triples plus edge rows checked."""
    c = inputs.C3
    log("c3 full size: generating inputs")
    q, k, v = inputs.prefill_inputs(c, DEV)
    o, lse = attn.prefill(q, k, v, True, c.scale)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    trip = inputs.sample_triples(c.seed, 64, (c.B, c.H, c.N),
                                 edge=[(0, 0, 0), (0, 0, 1), (3, 5, 127), (7, 9, 128), (15, 31, c.N - 1)])
    heads = sorted({(b, h) for b, h, _ in trip})
    idx = {bh: i for i, bh in enumerate(heads)}
    qs = torch.stack([q[b, h] for b, h in heads]).unsqueeze(0).cpu()
    ks = torch.stack([k[b, h] for b, h in heads]).unsqueeze(0).cpu()
    vs = torch.stack([v[b, h] for b, h in heads]).unsqueeze(0).cpu()
    o_ref, l_ref = oracle.attention_rows(qs, ks, vs, c.scale, True, [0] * len(trip),
                                         [idx[(b, h)] for b, h, _ in trip], [r for _, _, r in trip])
    og = torch.stack([o[b, h, r] for b, h, r in trip])
    lg = torch.stack([lse[b, h, r] for b, h, r in trip])
    check_close("c3 sampled", og, o_ref, lg, l_ref, torch.bfloat16)


def test_grid_past_32bit_work_items_is_a_shape_error():
    """A grid is a 32-bit count of work-items: 2^25 heads of one row need
    2^25 workgroups of 256 threads, 2^33 work-items, which the launcher
    rejects as ATTN_ERR_SHAPE (-2) before launching anything (the buffers are
    real, so a launch would still be a valid one)."""
    B, H, N, d = 1 << 17, 256, 1, 128
    log("grid guard: B=%d H=%d N=%d d=%d (32 GiB of buffers)" % (B, H, N, d))
    q = torch.empty((B, H, N, d), dtype=torch.bfloat16, device=DEV)
    k, v, o = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=DEV)
    rc = attn.attn_prefill_fwd(attn._ptr(q), attn._ptr(k), attn._ptr(v), attn._ptr(o), attn._ptr(lse), B, H, N, d,
                               1.0 / math.sqrt(d), 1, attn._dtype_code(q), attn._stream(None))
    torch.cuda.synchronize()
    assert rc == -2, rc
    del q, k, v, o, lse
    torch.cuda.empty_cache()
