"""GPU parity of the attention backward (attn_prefill_bwd through the C ABI)
against the fp64 oracle's gradients, on the forward's own O and LSE.

Tolerance (bf16 gradients; derived from the arithmetic, not given by the
pages).  The kernels round P and dS to bf16 before the dV, dK and dQ products
(relative error <= 2^-9 per term, accumulated in fp32), take D = dO . O from
the bf16-rounded forward output, and round each gradient to bf16 once at the
end (relative error <= 2^-9).  Per element:
    |g - r| <= 2^-7 |r| + 0.1 rms(r)
(2^-7: twice the output rounding plus the rounded-operand products; the
absolute term covers accumulations whose terms are much larger than their
sum), and over the tensor:
    mean |g - r| <= 4e-3 rms(r).
An emulation of this rounding scheme in fp64 on the CPU gives mean errors of
1.0e-3 to 1.8e-3 rms and per-element excesses over 2^-8 |r| up to 0.073 rms
at N = 2048 on these inputs.  rms is floored at 1e-3: where the exact
gradient vanishes (one key: P = 1, dS = P (dP - D) = 0) the kernel's dP and D
are the same fp32 dot product summed in different orders, so dS, and with it
dQ and dK, is a few fp32 roundings of |dO| |V| instead of 0.
"""
import numpy as np
import pytest
import torch

import oracle
import tiled_online_softmax_attention_amd as attn
from tiled_online_softmax_attention_amd import inputs
from parity import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"

REL = 2.0 ** -7
ABS_RMS = 0.1
MEAN_RMS = 4e-3
RMS_FLOOR = 1e-3


def check_grad(name, got, ref):
    g = got.detach().float().cpu().numpy().astype(np.float64) if isinstance(got, torch.Tensor) else got
    assert np.isfinite(g).all(), "%s: non-finite gradient" % name
    rms = max(float(np.sqrt(np.mean(ref ** 2))), RMS_FLOOR)
    err = np.abs(g - ref)
    excess = float((err - REL * np.abs(ref)).max())
    log("  %s: rms %.3e  max %.3e  mean %.3e (%.2e rms)  excess %.2e rms" %
        (name, rms, err.max(), err.mean(), err.mean() / max(rms, 1e-30), excess / max(rms, 1e-30)))
    assert excess <= ABS_RMS * rms, (name, excess, rms)
    assert err.mean() <= MEAN_RMS * rms, (name, float(err.mean()), rms)


def run(cfg, nan_outputs=True, scale=None):
    scale = cfg.scale if scale is None else scale
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    do = inputs.grad_output(cfg, DEV)
    o, lse = attn.prefill(q, k, v, cfg.causal, scale)
    dq = torch.full_like(q, float("nan")) if nan_outputs else None
    dk = torch.full_like(k, float("nan")) if nan_outputs else None
    dv = torch.full_like(v, float("nan")) if nan_outputs else None
    dq, dk, dv = attn.prefill_bwd(q, k, v, o, lse, do, cfg.causal, scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return (q, k, v, do), (dq, dk, dv)


@pytest.mark.parametrize("B,H,H_kv,N,d,causal", [
    (1, 2, 2, 300, 128, True),
    (1, 2, 2, 257, 64, False),
    (2, 4, 2, 129, 128, True),      # groups of 2
    (1, 8, 1, 200, 64, True),       # MQA
    (1, 2, 2, 33, 128, True),
    (1, 3, 3, 31, 64, True),        # one partial tile
    (1, 2, 2, 1, 128, True),        # a single key
    (1, 2, 2, 128, 128, True),      # exactly one key block
    (1, 4, 4, 1000, 128, True),
    (1, 6, 3, 511, 128, False),
])
def test_bwd_matches_oracle(B, H, H_kv, N, d, causal):
    cfg = inputs.PrefillConfig("bwd", B, H, N, d, torch.bfloat16, causal, 900 + N + H_kv, H_kv=H_kv)
    log("bwd B=%d H=%d H_kv=%d N=%d d=%d causal=%d" % (B, H, H_kv, N, d, causal))
    (q, k, v, do), (dq, dk, dv) = run(cfg)
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, cfg.scale, causal)
    check_grad("dq", dq, rq)
    check_grad("dk", dk, rk)
    check_grad("dv", dv, rv)


@pytest.mark.parametrize("N", [32, 64, 96, 160, 224, 250])
@pytest.mark.parametrize("H,H_kv", [(2, 2), (6, 2)])
@pytest.mark.parametrize("causal", [True, False])
def test_bwd_tile_stream_lengths(N, H, H_kv, causal):
    """The dK/dV loop runs its query-tile stream through three LDS buffers
    with the dS waves one tile behind: streams of 1, 2, 3, 5, 7 and 8 tiles
    per query head (every remainder modulo three, with and without a ragged
    last tile), one and three query heads per K/V head (each head's range of
    the stream starting at another buffer), causal and not."""
    cfg = inputs.PrefillConfig("bwd_len", 1, H, N, 128, torch.bfloat16, causal, 40 + N + H, H_kv=H_kv)
    log("bwd tile stream N=%d H=%d H_kv=%d causal=%d" % (N, H, H_kv, causal))
    (q, k, v, do), (dq, dk, dv) = run(cfg)
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, cfg.scale, causal)
    check_grad("dq", dq, rq)
    check_grad("dk", dk, rk)
    check_grad("dv", dv, rv)


def test_bwd_single_key_closed_form():
    """N = 1: P = 1, so dV = dO summed over the group and dQ = dK = 0 (up to
    the fp32 rounding of dP - D, two sums of the same 128 products)."""
    cfg = inputs.PrefillConfig("bwd1", 2, 4, 1, 128, torch.bfloat16, True, 5, H_kv=2)
    (q, k, v, do), (dq, dk, dv) = run(cfg)
    assert dq.abs().max() <= 1e-4 and dk.abs().max() <= 1e-4
    ref = do.float().view(2, 2, 2, 1, 128).sum(2)
    assert torch.allclose(dv.float(), ref, rtol=2.0 ** -8, atol=0)


def test_bwd_scale_zero():
    """scale = 0: P is uniform over the allowed keys, dQ = dK = 0."""
    cfg = inputs.PrefillConfig("bwd0", 1, 2, 70, 64, torch.bfloat16, True, 6)
    (q, k, v, do), (dq, dk, dv) = run(cfg, scale=0.0)
    assert torch.all(dq == 0) and torch.all(dk == 0)
    _, _, rv = oracle.attention_bwd(q, k, v, do, 0.0, True)
    check_grad("dv scale 0", dv, rv)


def test_bwd_deterministic():
    """Same inputs, same bits (no atomics; fixed accumulation order)."""
    cfg = inputs.PrefillConfig("bwd_det", 1, 8, 700, 128, torch.bfloat16, True, 7, H_kv=2)
    _, g1 = run(cfg)
    _, g2 = run(cfg, nan_outputs=False)
    for a, b in zip(g1, g2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("B,H,H_kv,N,d", [(1, 2, 2, 300, 128), (1, 8, 2, 700, 128), (2, 4, 4, 391, 64)])
def test_bwd_pairing_bit_identical(B, H, H_kv, N, d):
    """Paired dQ query tiles (t, n-1-t) and paired dK/dV key blocks (kb,
    nkb-1-kb) only change which workgroup runs which tile: every combination
    gives the bits of the unpaired launch (odd tile and block counts, so a
    middle tile / block runs alone; a grouped-query shape)."""
    cfg = inputs.PrefillConfig("bwd_pair", B, H, N, d, torch.bfloat16, True, 17 + N, H_kv=H_kv)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    do = inputs.grad_output(cfg, DEV)
    o, lse = attn.prefill(q, k, v, True, cfg.scale)
    ref = None
    for pq in (0, 1):
        for pkv in (0, 1):
            got = attn.prefill_bwd(q, k, v, o, lse, do, True, cfg.scale,
                                   options={"bwd_pair_q": pq, "bwd_pair_kv": pkv})
            torch.cuda.synchronize()
            if ref is None:
                ref = got
            for a, b in zip(ref, got):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), (pq, pkv)
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, cfg.scale, True)
    for name, g, r in zip(("dq", "dk", "dv"), ref, (rq, rk, rv)):
        check_grad(name, g, r)


def test_bwd_workspace_contents_ignored():
    """A workspace full of garbage on entry gives the same gradients."""
    cfg = inputs.PrefillConfig("bwd_ws", 1, 2, 300, 128, torch.bfloat16, True, 8)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    do = inputs.grad_output(cfg, DEV)
    o, lse = attn.prefill(q, k, v, True, cfg.scale)
    ref = attn.prefill_bwd(q, k, v, o, lse, do, True, cfg.scale)
    ws = torch.full((attn.attn_prefill_bwd_workspace_bytes(1, 2, 300) // 4,), float("nan"), device=DEV)
    got = attn.prefill_bwd(q, k, v, o, lse, do, True, cfg.scale, workspace=ws)
    torch.cuda.synchronize()
    for a, b in zip(ref, got):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_c3_bwd_full_size_sampled_rows():
    """The 16 x 32 x 8192 x 128 causal workload in the benchmark's launch
    configuration: 32 seeded dQ rows and 6 dK/dV key rows (key 0, which every
    query sees, and the last key among them) against the oracle."""
    cfg = inputs.C3
    log("c3 bwd full size")
    (q, k, v, do), (dq, dk, dv) = run(cfg, nan_outputs=False)
    N = cfg.N
    qs = inputs.sample_triples(cfg.seed + 50, 32, (cfg.B, cfg.H, N), edge=[(0, 0, 0), (15, 31, N - 1), (3, 7, 4095)])
    ks = inputs.sample_triples(cfg.seed + 51, 3, (cfg.B, cfg.H, N), edge=[(0, 0, 0), (15, 31, N - 1), (7, 3, 128)])
    log("  oracle: %d dq rows, %d dk/dv rows" % (len(qs), len(ks)))
    rq, rk, rv = oracle.attention_bwd_rows(q, k, v, do, cfg.scale, True, qs, ks)
    gq = torch.stack([dq[b, h, i] for b, h, i in qs])
    gk = torch.stack([dk[b, h, j] for b, h, j in ks])
    gv = torch.stack([dv[b, h, j] for b, h, j in ks])
    check_grad("c3 dq rows", gq, rq)
    check_grad("c3 dk rows", gk, rk)
    check_grad("c3 dv rows", gv, rv)


def test_c3_gqa8_bwd_full_size_sampled_rows():
    """The grouped-query variant of the same workload (32 query heads on 4
    K/V heads) at full size: 24 seeded dQ rows, and dK/dV rows of keys that
    the oracle can afford to visit with every query head of their group
    (the last key, one 100 keys from the end, one in the last quarter)."""
    cfg = inputs.C3_GQA8
    log("c3 gqa8 bwd full size")
    (q, k, v, do), (dq, dk, dv) = run(cfg, nan_outputs=False)
    N = cfg.N
    qs = inputs.sample_triples(cfg.seed + 60, 24, (cfg.B, cfg.H, N), edge=[(0, 31, N - 1), (9, 8, 0)])
    ks = [(0, 0, N - 1), (15, 3, N - 100), (7, 2, 7 * N // 8 + 13)]
    log("  oracle: %d dq rows, %d dk/dv rows" % (len(qs), len(ks)))
    rq, rk, rv = oracle.attention_bwd_rows(q, k, v, do, cfg.scale, True, qs, ks)
    gq = torch.stack([dq[b, h, i] for b, h, i in qs])
    gk = torch.stack([dk[b, h, j] for b, h, j in ks])
    gv = torch.stack([dv[b, h, j] for b, h, j in ks])
    check_grad("c3 gqa8 dq rows", gq, rq)
    check_grad("c3 gqa8 dk rows", gk, rk)
    check_grad("c3 gqa8 dv rows", gv, rv)


@pytest.mark.parametrize("H,H_kv,N,d", [(4, 2, 300, 128), (3, 3, 77, 64)])
def test_bwd_outputs_and_workspace_in_bounds(H, H_kv, N, d):
    """Guard words around dQ, dK, dV and the workspace survive: the backward
    writes only inside the buffers it is given (the workspace exactly
    attn_prefill_bwd_workspace_bytes long)."""
    cfg = inputs.PrefillConfig("bwd_guard", 1, H, N, d, torch.bfloat16, True, 31 + N, H_kv=H_kv)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    do = inputs.grad_output(cfg, DEV)
    o, lse = attn.prefill(q, k, v, True, cfg.scale)
    G = 4096

    def guarded(like, fill):
        buf = torch.full((2 * G + like.numel(),), fill, dtype=like.dtype, device=DEV)
        return buf, buf[G:G + like.numel()].view(like.shape)

    bq, dq = guarded(q, 7.0)
    bk, dk = guarded(k, 5.0)
    bv, dv = guarded(v, 3.0)
    ws_bytes = attn.attn_prefill_bwd_workspace_bytes(1, H, N)
    wbuf = torch.full((ws_bytes // 4 + 2 * G,), -9.0, dtype=torch.float32, device=DEV)
    ws = wbuf[G:G + ws_bytes // 4]
    log("bwd canaries H=%d H_kv=%d N=%d d=%d" % (H, H_kv, N, d))
    attn.prefill_bwd(q, k, v, o, lse, do, True, cfg.scale, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    for buf, fill in ((bq, 7.0), (bk, 5.0), (bv, 3.0), (wbuf, -9.0)):
        assert bool((buf[:G] == fill).all()) and bool((buf[-G:] == fill).all())
    rq, rk, rv = oracle.attention_bwd(q, k, v, do, cfg.scale, True)
    check_grad("dq", dq, rq)
    check_grad("dk", dk, rk)
    check_grad("dv", dv, rv)
