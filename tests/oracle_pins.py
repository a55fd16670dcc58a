"""Checks that pin the fp64 oracle to facts fixed outside itself.

Each check raises AssertionError when the oracle disagrees with:
  * hand-derived closed-form fixtures (tests/golden/*.json, each citing the
    passage it follows),
  * arbitrary-precision brute force (mpmath, no max shift) on tiny inputs,
  * closed forms (scale 0 -> mean of allowed values and LSE = ln #allowed;
    constant V rows; a dominant score -> one-hot),
  * a library routine for the special cases it covers (torch's CPU
    scaled_dot_product_attention in fp64 with an explicit boolean mask),
  * invariants of the method (rows of P sum to one; permutation equivariance;
    the block-wise online algorithm equals the two-pass definition for every
    block size; partial results merged by LSE equal the unsplit row; the paged
    path equals the contiguous path bit for bit under any block permutation;
    the gather copies bits exactly; poisoned slots are never read),
  * for the backward (gradients dQ, dK, dV of the same definition): central
    finite differences of the forward oracle; torch's fp64 autograd through an
    explicitly written masked softmax; the closed form of a two-key softmax
    (a logistic); and identities the gradients of this function obey at any
    size (shift invariance of the softmax in K, P rows summing to one in V,
    <V, dV> = <O, dO>, <Q, dQ> = <K, dK>).

They are plain functions so that the same list can be run both against the
real oracle (test_oracle_pins.py) and against deliberately broken copies of it
(test_oracle_mutants.py), which must each fail at least one check.
"""
from __future__ import annotations

import json
import math
from pathlib import Path

import numpy as np
import torch

import oracle

GOLDEN = Path(__file__).resolve().parent / "golden"


def _rng(seed):
    return np.random.default_rng(seed)


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
def check_golden_fixtures():
    files = sorted(GOLDEN.glob("*.json"))
    assert files, "no golden fixtures"
    for f in files:
        g = json.loads(f.read_text())
        tol = 1e-14
        if g["kind"] == "dense":
            q = _f64(g["q"])[None, None]
            k = _f64(g["k"])[None, None]
            v = _f64(g["v"])[None, None]
            o, lse = oracle.attention(q, k, v, g["scale"], g["causal"])
            assert np.allclose(o[0, 0], _f64(g["o"]), rtol=0, atol=tol), (f.name, o, g["o"])
            assert np.allclose(lse[0, 0], _f64(g["lse"]), rtol=0, atol=tol), (f.name, lse, g["lse"])
        elif g["kind"] == "paged":
            pool = np.array(g["pool"], dtype=object)
            pool = np.vectorize(lambda x: float("nan") if x == "nan" else float(x))(pool).astype(np.float64)
            o, lse = oracle.paged_attention(_f64(g["q"]), pool, np.array(g["block_table"], np.int32),
                                            np.array(g["ctx_lens"], np.int32), np.array(g["q_lens"], np.int32),
                                            g["block_size"], g["scale"])
            assert np.allclose(o, _f64(g["o"]), rtol=0, atol=tol), (f.name, o, g["o"])
            assert np.allclose(lse, _f64(g["lse"]), rtol=0, atol=tol), (f.name, lse, g["lse"])
        else:
            raise AssertionError("unknown fixture kind " + g["kind"])


# ---------------------------------------------------------------------------
def _brute_mp(q, k, v, scale, lim):
    """Arbitrary-precision direct evaluation: weights exp(scale*q.k) with no
    max shift, explicit sums; 40 significant digits."""
    import mpmath
    mpmath.mp.dps = 40
    nq, d = q.shape
    o = np.zeros((nq, d))
    lse = np.zeros(nq)
    for i in range(nq):
        w = []
        for j in range(lim[i]):
            s = mpmath.mpf(0)
            for c in range(d):
                s += mpmath.mpf(float(q[i, c])) * mpmath.mpf(float(k[j, c]))
            w.append(mpmath.exp(mpmath.mpf(scale) * s))
        tot = mpmath.fsum(w)
        for c in range(d):
            o[i, c] = float(mpmath.fsum(wj * mpmath.mpf(float(v[j, c])) for j, wj in enumerate(w)) / tot)
        lse[i] = float(mpmath.log(tot))
    return o, lse


def check_bruteforce_tiny():
    rng = _rng(11)
    for (nq, nk, d, causal) in [(1, 1, 1, False), (2, 3, 2, False), (5, 5, 4, True), (9, 9, 4, True),
                                (4, 7, 2, True), (3, 9, 1, False), (7, 7, 3, False)]:
        q = rng.standard_normal((nq, d))
        k = rng.standard_normal((nk, d))
        v = rng.standard_normal((nk, d))
        scale = 0.7
        if causal:
            lim = [nk - nq + i + 1 for i in range(nq)]
        else:
            lim = [nk] * nq
        if causal and nq != nk:
            # bottom-right causal on non-square shapes is exercised through the paged entry point
            nb = nk  # one token per block, identity table
            pool = np.zeros((nb, 2, 1, 1, d))
            pool[:, 0, 0, 0, :] = k
            pool[:, 1, 0, 0, :] = v
            o, lse = oracle.paged_attention(q[:, None, :], pool, np.arange(nb, dtype=np.int32)[None],
                                            np.array([nk], np.int32), np.array([nq], np.int32), 1, scale)
            o, lse = o[:, 0, :], lse[:, 0]
        else:
            o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal)
            o, lse = o[0, 0], lse[0, 0]
        ob, lb = _brute_mp(q, k, v, scale, lim)
        assert np.allclose(o, ob, rtol=0, atol=1e-13), (nq, nk, d, causal, np.abs(o - ob).max())
        assert np.allclose(lse, lb, rtol=0, atol=1e-13), (nq, nk, d, causal)


# ---------------------------------------------------------------------------
def check_rows_sum_to_one():
    """sum_j exp(S_ij - LSE_i) = 1, with S computed independently here."""
    rng = _rng(12)
    nq = nk = 33
    d = 8
    q, k, v = (rng.standard_normal((nq, d)) for _ in range(3))
    scale = 0.4
    for causal in (False, True):
        _, lse = oracle.attention(q[None, None], k[None, None], v[None, None], scale, causal)
        s = scale * (q @ k.T)
        if causal:
            s = np.where(np.tril(np.ones((nq, nk), bool)), s, -np.inf)
        tot = np.exp(s - lse[0, 0][:, None]).sum(axis=1)
        assert np.allclose(tot, 1.0, rtol=0, atol=1e-12), tot


def check_scale_zero_closed_form():
    """scale = 0: every allowed key gets equal weight, so O_i is the mean of
    the allowed V rows and LSE_i = ln(#allowed).  Pins the mask alignment."""
    rng = _rng(13)
    n, d = 37, 5
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], 0.0, True)
    cnt = np.arange(1, n + 1, dtype=np.float64)
    assert np.allclose(o[0, 0], np.cumsum(v, axis=0) / cnt[:, None], rtol=0, atol=1e-13)
    assert np.allclose(lse[0, 0], np.log(cnt), rtol=0, atol=1e-13)
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], 0.0, False)
    assert np.allclose(o[0, 0], np.broadcast_to(v.mean(axis=0), (n, d)), rtol=0, atol=1e-13)
    assert np.allclose(lse[0, 0], math.log(n), rtol=0, atol=1e-13)
    # paged, bottom-right: request with ctx 23, q_len 6 -> row i sees 23 - 6 + i + 1 keys
    ctx, ql, bs, H = 23, 6, 4, 2
    kv = rng.standard_normal((2, H, ctx, d))
    pool, table = _scatter(kv, bs, rng)
    qq = rng.standard_normal((ql, H, d))
    o, lse = oracle.paged_attention(qq, pool, table[None], np.array([ctx], np.int32),
                                    np.array([ql], np.int32), bs, 0.0)
    for i in range(ql):
        lim = ctx - ql + i + 1
        for h in range(H):
            assert np.allclose(o[i, h], kv[1, h, :lim].mean(axis=0), rtol=0, atol=1e-13)
            assert abs(lse[i, h] - math.log(lim)) < 1e-13


def check_constant_v():
    rng = _rng(14)
    n, d = 29, 6
    q, k = (rng.standard_normal((n, d)) for _ in range(2))
    c = rng.standard_normal(d)
    v = np.broadcast_to(c, (n, d)).copy()
    for causal in (False, True):
        o, _ = oracle.attention(q[None, None], k[None, None], v[None, None], 1.3, causal)
        assert np.allclose(o[0, 0], np.broadcast_to(c, (n, d)), rtol=0, atol=1e-13)


def check_one_hot_limit():
    """A score that dominates the rest of its row by > 60 nats makes the row
    a copy of that key's value (to far below fp64 resolution)."""
    rng = _rng(15)
    n, d = 6, 4
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    q = np.stack([200.0 * k[t] for t in (3, 0, 5, 1, 2, 4)])
    o, _ = oracle.attention(q[None, None], k[None, None], v[None, None], 1.0, False)
    s = q @ k.T
    srt = np.sort(s, axis=1)
    ok = (srt[:, -1] - srt[:, -2]) > 60.0
    assert ok.sum() >= 3
    assert np.allclose(o[0, 0][ok], v[np.argmax(s, axis=1)][ok], rtol=0, atol=1e-12)


def check_torch_sdpa_special_case():
    """torch's CPU fp64 scaled_dot_product_attention with an explicit mask."""
    rng = _rng(16)
    B, H, nq, nk, d = 2, 3, 11, 19, 8
    q = torch.from_numpy(rng.standard_normal((B, H, nq, d)))
    k = torch.from_numpy(rng.standard_normal((B, H, nk, d)))
    v = torch.from_numpy(rng.standard_normal((B, H, nk, d)))
    scale = 0.3
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    o, _ = oracle.attention(q, k, v, scale, False)
    assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    # square causal: top-left and bottom-right coincide
    q2 = torch.from_numpy(rng.standard_normal((B, H, nk, d)))
    ref = torch.nn.functional.scaled_dot_product_attention(q2, k, v, is_causal=True, scale=scale)
    o, _ = oracle.attention(q2, k, v, scale, True)
    assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-12)
    # paged, bottom-right limit given to torch as an explicit boolean mask
    ctx, ql, bs = nk, nq, 4
    kv = np.stack([k[0].numpy(), v[0].numpy()])           # [2, H, ctx, d]
    pool, table = _scatter(kv, bs, rng)
    qq = q[0].permute(1, 0, 2).contiguous().numpy()        # [ql, H, d]
    o, _ = oracle.paged_attention(qq, pool, table[None], np.array([ctx], np.int32),
                                  np.array([ql], np.int32), bs, scale)
    i = torch.arange(ql)[:, None]
    j = torch.arange(ctx)[None, :]
    mask = j <= (ctx - ql + i)
    ref = torch.nn.functional.scaled_dot_product_attention(q[0], k[0], v[0], attn_mask=mask, scale=scale)
    assert np.allclose(o, ref.permute(1, 0, 2).numpy(), rtol=0, atol=1e-12)


def check_equivariance():
    rng = _rng(17)
    n, d = 21, 7
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], 0.5, False)
    pk = rng.permutation(n)
    o2, lse2 = oracle.attention(q[None, None], k[pk][None, None], v[pk][None, None], 0.5, False)
    assert np.allclose(o, o2, rtol=0, atol=1e-13) and np.allclose(lse, lse2, rtol=0, atol=1e-13)
    pq = rng.permutation(n)
    o3, lse3 = oracle.attention(q[pq][None, None], k[None, None], v[None, None], 0.5, False)
    assert np.allclose(o3[0, 0], o[0, 0][pq], rtol=0, atol=1e-13)
    assert np.allclose(lse3[0, 0], lse[0, 0][pq], rtol=0, atol=1e-13)


def check_tiled_equals_two_pass():
    rng = _rng(18)
    n, d = 131, 16
    q, k, v = (rng.standard_normal((n, d)) for _ in range(3))
    for causal in (False, True):
        o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], 0.25, causal)
        for bsz in (1, 3, 16, 64, 128, n):
            ot, lt = oracle.tiled_online(q, k, v, 0.25, causal, bsz)
            assert np.allclose(ot, o[0, 0], rtol=0, atol=1e-12), (causal, bsz)
            assert np.allclose(lt, lse[0, 0], rtol=0, atol=1e-12), (causal, bsz)


def check_lse_merge_partition():
    rng = _rng(19)
    nk, d = 50, 9
    q = rng.standard_normal((1, d))
    k, v = (rng.standard_normal((nk, d)) for _ in range(2))
    o, lse = oracle.attention(q[None, None], k[None, None], v[None, None], 0.8, False)
    for nparts in (1, 2, 3, 7):
        cuts = np.sort(rng.choice(np.arange(1, nk), nparts - 1, replace=False))
        bounds = [0, *cuts.tolist(), nk]
        parts_o, parts_l = [], []
        for a, b in zip(bounds[:-1], bounds[1:]):
            po, pl = oracle.attention(q[None, None], k[a:b][None, None], v[a:b][None, None], 0.8, False)
            parts_o.append(po[0, 0, 0])
            parts_l.append(pl[0, 0, 0])
        mo, ml = oracle.lse_merge(np.array(parts_o), np.array(parts_l))
        assert np.allclose(mo, o[0, 0, 0], rtol=0, atol=1e-12), nparts
        assert abs(ml - lse[0, 0, 0]) < 1e-12


def _scatter(kv, bs, rng, spare=3, nan_fill=True):
    """Scatter contiguous kv [2, H, ctx, d] into a shuffled pool; returns (pool, table)."""
    _, H, ctx, d = kv.shape
    nb = -(-ctx // bs)
    num_blocks = nb + spare
    ids = rng.permutation(num_blocks)[:nb].astype(np.int32)
    pool = np.full((num_blocks, 2, H, bs, d), np.nan if nan_fill else 0.0)
    for t in range(ctx):
        pool[ids[t // bs], :, :, t % bs, :] = kv[:, :, t, :]
    return pool, ids


def check_paged_equals_contiguous_bitexact():
    rng = _rng(20)
    H, d, bs = 3, 8, 4
    ctx_lens = [13, 4, 29]
    q_lens = [5, 1, 29]
    kvs = [rng.standard_normal((2, H, c, d)) for c in ctx_lens]
    qs = [rng.standard_normal((ql, H, d)) for ql in q_lens]
    q = np.concatenate(qs)
    results = []
    for trial in range(3):
        pools, tables = [], []
        base = 0
        for kv in kvs:
            p, t = _scatter(kv, bs, rng)
            pools.append(p)
            tables.append(t + base)
            base += p.shape[0]
        pool = np.concatenate(pools)
        maxb = max(len(t) for t in tables)
        table = np.full((len(tables), maxb), -1, np.int32)
        for r, t in enumerate(tables):
            table[r, :len(t)] = t
        o, lse = oracle.paged_attention(q, pool, table, np.array(ctx_lens, np.int32),
                                        np.array(q_lens, np.int32), bs, 0.35)
        results.append((o, lse))
        assert np.isfinite(o).all()
    for o, lse in results[1:]:
        assert np.array_equal(o, results[0][0]) and np.array_equal(lse, results[0][1])
    # contiguous path (bottom-right causal) must agree bit for bit
    row = 0
    o_p, l_p = results[0]
    for r, (kv, qr) in enumerate(zip(kvs, qs)):
        for h in range(H):
            qc = qr[:, h, :][None, None]
            if q_lens[r] == ctx_lens[r]:
                oc, lc = oracle.attention(qc, kv[0, h][None, None], kv[1, h][None, None], 0.35, True)
                assert np.array_equal(oc[0, 0], o_p[row:row + q_lens[r], h]), (r, h)
                assert np.array_equal(lc[0, 0], l_p[row:row + q_lens[r], h])
            for i in range(q_lens[r]):
                lim = ctx_lens[r] - q_lens[r] + i + 1
                oc, lc = oracle.attention(qr[i, h][None, None, None], kv[0, h, :lim][None, None],
                                          kv[1, h, :lim][None, None], 0.35, False)
                assert np.array_equal(oc[0, 0, 0], o_p[row + i, h]), (r, h, i)
                assert lc[0, 0, 0] == l_p[row + i, h]
        row += q_lens[r]


def check_gather_bitexact():
    rng = _rng(21)
    H, d, bs = 2, 4, 16
    ctx_lens = [33, 16, 1, 70]
    kvs = [rng.standard_normal((2, H, c, d)).astype(np.float32) for c in ctx_lens]
    pools, tables, base = [], [], 0
    for kv in kvs:
        p, t = _scatter(kv, bs, rng)
        pools.append(p.astype(np.float32))
        tables.append(t + base)
        base += p.shape[0]
    pool = np.concatenate(pools)
    maxb = max(len(t) for t in tables)
    table = np.full((len(tables), maxb), -1, np.int32)
    for r, t in enumerate(tables):
        table[r, :len(t)] = t
    ko, vo = oracle.paged_gather(pool, table, np.array(ctx_lens, np.int32), bs)
    want_k = np.concatenate([kv[0].transpose(1, 0, 2) for kv in kvs])
    want_v = np.concatenate([kv[1].transpose(1, 0, 2) for kv in kvs])
    assert np.array_equal(ko.view(np.uint32), want_k.view(np.uint32))
    assert np.array_equal(vo.view(np.uint32), want_v.view(np.uint32))
    # bf16 storage: bits copied unchanged
    pb = torch.from_numpy(pool).to(torch.bfloat16)
    ko, vo = oracle.paged_gather(pb, table, np.array(ctx_lens, np.int32), bs)
    wk = torch.from_numpy(want_k).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ko, wk)


def check_bf16_upcast_exact():
    """bf16 inputs are read as their exact values (here: small integers and
    powers of two, all exact in bf16), via the golden running-mean example."""
    q = torch.zeros(1, 1, 3, 1, dtype=torch.bfloat16)
    k = torch.tensor([7.0, -2.0, 0.5], dtype=torch.bfloat16).view(1, 1, 3, 1)
    v = torch.tensor([3.0, 5.0, 10.0], dtype=torch.bfloat16).view(1, 1, 3, 1)
    o, lse = oracle.attention(q, k, v, 0.125, True)
    assert np.allclose(o[0, 0, :, 0], [3.0, 4.0, 6.0], rtol=0, atol=1e-15)
    assert np.allclose(lse[0, 0], [0.0, math.log(2), math.log(3)], rtol=0, atol=1e-15)
    vv = torch.tensor([1.0 + 2.0 ** -7], dtype=torch.float32).to(torch.bfloat16)   # exactly representable
    o, _ = oracle.attention(q[:, :, :1], k[:, :, :1], vv.view(1, 1, 1, 1), 1.0, False)
    assert o[0, 0, 0, 0] == 1.0 + 2.0 ** -7


def check_gqa_torch_sdpa():
    """Grouped-query attention ("Sequence length doubles ...", further
    optimisations: several query heads share one K/V head; MQA when all do)
    against torch's CPU fp64 SDPA with enable_gqa (consecutive query heads
    share a K/V head, the K/V heads repeated by repeat_interleave)."""
    rng = _rng(30)
    B, n, d, scale = 2, 9, 8, 0.4
    for H, Hkv in ((4, 2), (6, 3), (4, 1), (3, 3), (8, 2)):
        q = torch.from_numpy(rng.standard_normal((B, H, n, d)))
        k = torch.from_numpy(rng.standard_normal((B, Hkv, n, d)))
        v = torch.from_numpy(rng.standard_normal((B, Hkv, n, d)))
        for causal in (False, True):
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, scale=scale,
                                                                   enable_gqa=True)
            o, _ = oracle.attention(q, k, v, scale, causal)
            assert np.allclose(o, ref.numpy(), rtol=0, atol=1e-12), (H, Hkv, causal)
        # the same through sampled rows
        o, _ = oracle.attention(q, k, v, scale, True)
        orow, _ = oracle.attention_rows(q, k, v, scale, True, [1, 0], [H - 1, 0], [n - 1, 3])
        assert np.array_equal(orow[0], o[1, H - 1, n - 1]) and np.array_equal(orow[1], o[0, 0, 3])


def check_gqa_paged_equals_contiguous():
    """Paged GQA (pool holds Hkv heads) equals contiguous GQA bit for bit."""
    rng = _rng(31)
    H, Hkv, d, bs = 6, 2, 8, 4
    ctx_lens, q_lens = [13, 7], [5, 7]
    kvs = [rng.standard_normal((2, Hkv, c, d)) for c in ctx_lens]
    qs = [rng.standard_normal((ql, H, d)) for ql in q_lens]
    pools, tables, base = [], [], 0
    for kv in kvs:
        pl, t = _scatter(kv, bs, rng)
        pools.append(pl)
        tables.append(t + base)
        base += pl.shape[0]
    pool = np.concatenate(pools)
    table = np.full((2, max(len(t) for t in tables)), -1, np.int32)
    for r, t in enumerate(tables):
        table[r, :len(t)] = t
    cl, ql = np.array(ctx_lens, np.int32), np.array(q_lens, np.int32)
    o_p, l_p = oracle.paged_attention(np.concatenate(qs), pool, table, cl, ql, bs, 0.3)
    orow, lrow = oracle.paged_attention_rows(np.concatenate(qs), pool, table, cl, ql, bs, 0.3, [0, 1], [5, 2],
                                             [4, 0])
    assert np.array_equal(orow[0], o_p[4, 5]) and np.array_equal(orow[1], o_p[5, 2])
    row = 0
    for r, (kv, qr) in enumerate(zip(kvs, qs)):
        qc = qr.transpose(1, 0, 2)[None]                       # [1, H, ql, d]
        oc, lc = oracle.attention(qc, kv[0][None], kv[1][None], 0.3, True)   # bottom-right when ql < ctx
        assert np.array_equal(oc[0].transpose(1, 0, 2), o_p[row:row + q_lens[r]])
        assert np.array_equal(lc[0].T, l_p[row:row + q_lens[r]])
        row += q_lens[r]


# ---- backward ---------------------------------------------------------------

def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention(q, k, v, scale, causal)
    return float(np.sum(o * do))


def check_bwd_finite_differences():
    """Every gradient entry of L = sum(O * dO) against central differences of
    the forward oracle (h = 1e-5; truncation and rounding error both far below
    the 1e-7 tolerance at these magnitudes), square causal, bottom-right causal
    (fewer queries than keys) and unmasked, with two query heads on one K/V
    head."""
    rng = _rng(40)
    h = 1e-5
    for (Nq, Nk, causal) in ((5, 5, True), (3, 6, True), (4, 5, False)):
        B, H, Hkv, d, scale = 1, 2, 1, 3, 0.7
        q = rng.standard_normal((B, H, Nq, d))
        k = rng.standard_normal((B, Hkv, Nk, d))
        v = rng.standard_normal((B, Hkv, Nk, d))
        do = rng.standard_normal((B, H, Nq, d))
        grads = oracle.attention_bwd(q, k, v, do, scale, causal)
        for x, g in zip((q, k, v), grads):
            for idx in np.ndindex(*x.shape):
                keep = x[idx]
                x[idx] = keep + h
                up = _loss(q, k, v, do, scale, causal)
                x[idx] = keep - h
                dn = _loss(q, k, v, do, scale, causal)
                x[idx] = keep
                fd = (up - dn) / (2 * h)
                assert abs(fd - g[idx]) < 1e-7, (Nq, Nk, causal, idx, fd, g[idx])


def check_bwd_torch_autograd():
    """Against torch's fp64 autograd of softmax(scale Q K^T + mask) V written
    out explicitly (bottom-right causal mask as a boolean matrix, K/V heads
    repeated for grouped-query attention, so dK and dV come back summed over
    each group), for bf16 and fp32 stored inputs."""
    rng = _rng(41)
    for (B, H, Hkv, Nq, Nk, d, causal, dt) in ((2, 4, 2, 37, 37, 16, True, torch.bfloat16),
                                                (1, 3, 3, 11, 29, 8, True, torch.float32),
                                                (1, 4, 1, 13, 13, 8, False, torch.bfloat16),
                                                (1, 6, 2, 9, 9, 4, True, torch.float64)):
        scale = 1.0 / math.sqrt(d)
        q = torch.from_numpy(rng.standard_normal((B, H, Nq, d))).to(dt)
        k = torch.from_numpy(rng.standard_normal((B, Hkv, Nk, d))).to(dt)
        v = torch.from_numpy(rng.standard_normal((B, Hkv, Nk, d))).to(dt)
        do = torch.from_numpy(rng.standard_normal((B, H, Nq, d))).to(dt)
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, causal)
        qq, kk, vv = (t.double().requires_grad_() for t in (q, k, v))
        rep = H // Hkv
        kr, vr = kk.repeat_interleave(rep, 1), vv.repeat_interleave(rep, 1)
        s = torch.matmul(qq, kr.transpose(-1, -2)) * scale
        if causal:
            allowed = torch.arange(Nk)[None, :] <= torch.arange(Nq)[:, None] + (Nk - Nq)
            s = s.masked_fill(~allowed, float("-inf"))
        o = torch.matmul(torch.softmax(s, -1), vr)
        o.backward(do.double())
        for name, mine, ref in (("dq", dq, qq.grad), ("dk", dk, kk.grad), ("dv", dv, vv.grad)):
            assert np.allclose(mine, ref.numpy(), rtol=0, atol=1e-12), (name, B, H, Hkv, Nq, Nk, causal, dt)


def check_bwd_two_key_closed_form():
    """One query, two keys: P = (1 - s, s) with s = logistic(t), t = scale
    q.(k1 - k0), so O = v0 + s (v1 - v0) and, with s' = s (1 - s):
    dV0 = (1 - s) dO, dV1 = s dO, dQ = s' (dO.(v1 - v0)) scale (k1 - k0),
    dK1 = -dK0 = s' (dO.(v1 - v0)) scale q."""
    rng = _rng(42)
    d, scale = 5, 0.9
    q = rng.standard_normal((1, 1, 1, d))
    k = rng.standard_normal((1, 1, 2, d))
    v = rng.standard_normal((1, 1, 2, d))
    do = rng.standard_normal((1, 1, 1, d))
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, scale, False)
    q0, k0, k1, v0, v1, g = q[0, 0, 0], k[0, 0, 0], k[0, 0, 1], v[0, 0, 0], v[0, 0, 1], do[0, 0, 0]
    t = scale * q0 @ (k1 - k0)
    sg = 1.0 / (1.0 + math.exp(-t))
    ds = sg * (1 - sg) * (g @ (v1 - v0))
    tol = dict(rtol=0, atol=1e-14)
    assert np.allclose(dv[0, 0, 0], (1 - sg) * g, **tol) and np.allclose(dv[0, 0, 1], sg * g, **tol)
    assert np.allclose(dq[0, 0, 0], ds * scale * (k1 - k0), **tol)
    assert np.allclose(dk[0, 0, 1], ds * scale * q0, **tol) and np.allclose(dk[0, 0, 0], -ds * scale * q0, **tol)


def check_bwd_identities():
    """Identities of the gradient at any size, per K/V head (its group of
    query heads together):
      sum_j dK_j = 0             (a common shift of all keys moves every
                                  allowed score of a row by one constant)
      sum_j dV_j = sum_i dO_i    (every P row sums to one)
      <V, dV> = <O, dO>          (O is linear in V)
      <Q, dQ> = <K, dK>          (scaling Q or K scales S alike)
    plus: a causal row that sees one key has dQ = 0; constant V rows give
    dQ = dK = 0; scale 0 gives dQ = dK = 0 and dV_j = sum over rows i that
    see j of dO_i / (number of keys row i sees)."""
    rng = _rng(43)
    for (B, H, Hkv, Nq, Nk, d, causal) in ((2, 4, 2, 40, 40, 8, True), (1, 3, 1, 7, 33, 8, True),
                                          (1, 2, 2, 21, 21, 16, False)):
        q = rng.standard_normal((B, H, Nq, d))
        k = rng.standard_normal((B, Hkv, Nk, d))
        v = rng.standard_normal((B, Hkv, Nk, d))
        do = rng.standard_normal((B, H, Nq, d))
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.5, causal)
        o, _ = oracle.attention(q, k, v, 0.5, causal)
        G = H // Hkv
        for b in range(B):
            for hk in range(Hkv):
                hs = slice(hk * G, (hk + 1) * G)
                assert np.allclose(dk[b, hk].sum(0), 0.0, rtol=0, atol=1e-11)
                assert np.allclose(dv[b, hk].sum(0), do[b, hs].sum((0, 1)), rtol=0, atol=1e-11)
                assert abs(np.sum(v[b, hk] * dv[b, hk]) - np.sum(o[b, hs] * do[b, hs])) < 1e-10
                assert abs(np.sum(q[b, hs] * dq[b, hs]) - np.sum(k[b, hk] * dk[b, hk])) < 1e-10
        if causal and Nq == Nk:
            assert np.all(dq[:, :, 0] == 0.0)
        vc = np.broadcast_to(rng.standard_normal((B, Hkv, 1, d)), v.shape).copy()
        dq0, dk0, _ = oracle.attention_bwd(q, k, vc, do, 0.5, causal)
        assert np.allclose(dq0, 0.0, rtol=0, atol=1e-12) and np.allclose(dk0, 0.0, rtol=0, atol=1e-12)
        dqz, dkz, dvz = oracle.attention_bwd(q, k, v, do, 0.0, causal)
        assert np.all(dqz == 0.0) and np.allclose(dkz, 0.0, rtol=0, atol=1e-15)
        n_see = np.array([min(Nk, Nk - Nq + i + 1) if causal else Nk for i in range(Nq)], np.float64)
        sees = np.array([[j < n_see[i] for j in range(Nk)] for i in range(Nq)], np.float64)   # [Nq, Nk]
        for b in range(B):
            for hk in range(Hkv):
                ref = np.einsum("ij,hic->jc", sees / n_see[:, None], do[b, hk * G:(hk + 1) * G])
                assert np.allclose(dvz[b, hk], ref, rtol=0, atol=1e-12)


def check_bwd_rows_match_full():
    """Sampled rows of the backward equal the full backward (grouped heads,
    bottom-right causal, first/last rows and keys)."""
    rng = _rng(44)
    B, H, Hkv, Nq, Nk, d = 2, 6, 2, 9, 14, 8
    q = rng.standard_normal((B, H, Nq, d))
    k = rng.standard_normal((B, Hkv, Nk, d))
    v = rng.standard_normal((B, Hkv, Nk, d))
    do = rng.standard_normal((B, H, Nq, d))
    for causal in (True, False):
        dq, dk, dv = oracle.attention_bwd(q, k, v, do, 0.3, causal)
        qs = [(0, 0, 0), (1, 5, Nq - 1), (1, 2, 4), (0, 3, 7)]
        ks = [(0, 0, 0), (1, 1, Nk - 1), (0, 1, 6), (1, 0, 13), (1, 0, 2)]
        rq, rk, rv = oracle.attention_bwd_rows(q, k, v, do, 0.3, causal, qs, ks)
        for n, (b, h, i) in enumerate(qs):
            assert np.allclose(rq[n], dq[b, h, i], rtol=0, atol=1e-13)
        for n, (b, hk, j) in enumerate(ks):
            assert np.allclose(rk[n], dk[b, hk, j], rtol=0, atol=1e-13)
            assert np.allclose(rv[n], dv[b, hk, j], rtol=0, atol=1e-13)


ALL_CHECKS = [
    check_golden_fixtures,
    check_bruteforce_tiny,
    check_rows_sum_to_one,
    check_scale_zero_closed_form,
    check_constant_v,
    check_one_hot_limit,
    check_torch_sdpa_special_case,
    check_equivariance,
    check_tiled_equals_two_pass,
    check_lse_merge_partition,
    check_paged_equals_contiguous_bitexact,
    check_gather_bitexact,
    check_bf16_upcast_exact,
    check_gqa_torch_sdpa,
    check_gqa_paged_equals_contiguous,
    check_bwd_finite_differences,
    check_bwd_torch_autograd,
    check_bwd_two_key_closed_form,
    check_bwd_identities,
    check_bwd_rows_match_full,
]
