#!/usr/bin/env python3
"""Throughput of the tiled online-softmax attention hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * causal prefill, bf16, B=16 H=32 N=8192 d=128 (attn_prefill_fwd, one launch)
  * paged decode, bf16, 64 requests x 1 query, ctx ~ U[512, 16384], 16-token
    pages scattered in the pool (paged_attn_fwd: split kernel + combine kernel)
  * paged chunked prefill, bf16, 8 requests x 512 query rows on prior contexts
    ~ U[4096, 32768], 32-token pages (paged_attn_fwd: tile kernel + combine)
Inputs are generated on the GPU before timing (resident in HBM).  The line
printed reports prefill TFLOP/s as `value` (algorithmic FLOPs = 4*d per
allowed (query, key) pair, per launch, over the launch's average duration
measured with HIP events on the launch stream), the decode KV GB/s
(algorithmic bytes: K and V of every context token read once, plus q, o and
the block table) under "decode", the chunked prefill under "c5", and, timed
after the steps, the small causal prefill B=1 H=32 N=2048 under "c2" (warm,
and cold: 1 GiB written between launches), then a few calls each of the
grouped-query prefill and decode (32 query heads on 4 K/V heads) under "gqa8"
and of the prefill's backward under "bwd", and the KV append under "append".  The oracle (fp64, CPU) is timed
on a bounded sample of the same prefill and decode workloads as
`cpu_baseline`.

Other modes (--only): prefill, decode, c2, c5 (single workloads), append (KV
append), gqa (grouped-query prefill and decode), bwd (the backward of the
causal prefill, MHA and GQA-8).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0         # MI355X HBM3E
METRIC = "causal prefill TFLOP/s + paged-decode KV GB/s (and % roofline), 1 MI355X"
# Sources each measured kernel is built from (csrc/): a PMC summary in
# profiles/ is used only while these files are unchanged.
KERNEL_SOURCES = {
    "prefill_c3": ["attn_mfma_core.h", "attn_mfma_kernel.h", "attn_mfma_pipe.h", "prefill_gfx950.hip",
                   "attn_internal.h"],
    "decode_c4": ["attn_mfma_core.h", "attn_mfma_kernel.h", "attn_mfma_pipe.h", "paged_gfx950.hip", "attn_internal.h"],
    "chunk_c5": ["attn_mfma_core.h", "attn_mfma_kernel.h", "attn_mfma_pipe.h", "paged_gfx950.hip", "attn_internal.h"],
    "bwd_c3": ["attn_mfma_core.h", "bwd_gfx950.hip", "bwd_internal.h"],
}


def kernel_source_hash(kernel_key):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel_key]:
        h.update((ROOT / "tiled_online_softmax_attention_amd" / "csrc" / name).read_bytes())
    return h.hexdigest()[:16]


def read_traffic(kernel_key):
    """HBM bytes per launch from committed PMC summaries (profiles/pmc_*.txt),
    valid only if they were taken on the current kernel sources."""
    f = ROOT / "profiles" / ("pmc_%s.txt" % kernel_key)
    if not f.exists():
        return None
    kv = {}
    for line in f.read_text().splitlines():
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha") != kernel_source_hash(kernel_key):
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def prefill_flops(B, H, N, d, causal):
    pairs = N * (N + 1) // 2 if causal else N * N
    return 4.0 * d * pairs * B * H


def prefill_bytes(B, H, N, d, elem=2, H_kv=None):
    H_kv = H if H_kv is None else H_kv
    return B * N * d * elem * (2 * H + 2 * H_kv) + B * H * N * 4   # q, k, v read + o written + lse


def bwd_flops(B, H, N, d, causal):
    """Algorithmic FLOPs of the backward: five products (S recomputed, dP,
    dV, dK, dQ) of 2*d FLOPs per allowed (query, key) pair."""
    pairs = N * (N + 1) // 2 if causal else N * N
    return 10.0 * d * pairs * B * H


def bwd_bytes(B, H, N, d, elem=2, H_kv=None):
    """q, o, dO read and dQ written (H heads); k, v read and dK, dV written
    (H_kv heads); lse read; the per-row (lse, D) workspace written and read."""
    H_kv = H if H_kv is None else H_kv
    return B * N * d * elem * (4 * H + 4 * H_kv) + B * H * N * 4 + 2 * B * H * N * 8


def paged_bytes(ctx_lens, q_lens, H, d, block_size, elem=2, H_kv=None):
    """K and V of every context token once (for the H_kv K/V heads), q read
    and o, lse written (H query heads), one table entry per page."""
    H_kv = H if H_kv is None else H_kv
    ctx = sum(ctx_lens)
    tq = sum(q_lens)
    pages = sum((c + block_size - 1) // block_size for c in ctx_lens)
    return 2 * ctx * H_kv * d * elem + 2 * tq * H * d * elem + tq * H * 4 + pages * 4


def paged_flops(ctx_lens, q_lens, d, H):
    pairs = 0
    for c, q in zip(ctx_lens, q_lens):
        pairs += q * (c - q) + q * (q + 1) // 2
    return 4.0 * d * pairs * H


def probe_copy(torch, dev):
    """One 1 GiB device-to-device copy: the reference kernel whose PMC byte
    counters calibrate FETCH_SIZE / WRITE_SIZE."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    print("probe copy: 1073741824 bytes read and written", file=sys.stderr, flush=True)


class EventTimer:
    """Average duration of one region per step, from HIP events on the stream."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def start(self):
        e = self.torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    def stop(self, e0):
        e1 = self.torch.cuda.Event(enable_timing=True)
        e1.record()
        self.pairs.append((e0, e1))

    def times_ms(self):
        return sorted(a.elapsed_time(b) for a, b in self.pairs)

    def mean_ms(self):
        t = self.times_ms()
        return sum(t) / max(1, len(t))

    def median_ms(self):
        t = self.times_ms()
        return t[len(t) // 2] if len(t) % 2 else 0.5 * (t[len(t) // 2 - 1] + t[len(t) // 2])

    def min_ms(self):
        return self.times_ms()[0]


class ParityStats:
    """Max / mean |GPU - oracle| over the rows the CPU baseline evaluated
    (outside its timed region), reported beside the parity bounds of the bf16
    path (tests/parity.py): O max 2e-2 and mean 2e-3; LSE max 2.5e-3."""

    def __init__(self):
        self.n, self.max_o, self.sum_o, self.cnt_o, self.max_lse = 0, 0.0, 0.0, 0, 0.0

    def add(self, o_gpu, o_ref, lse_gpu, lse_ref):
        import numpy as np
        e = np.abs(np.asarray(o_gpu, dtype=np.float64) - np.asarray(o_ref, dtype=np.float64))
        self.n += e.shape[0]
        self.max_o = max(self.max_o, float(e.max()))
        self.sum_o += float(e.sum())
        self.cnt_o += e.size
        el = np.abs(np.asarray(lse_gpu, dtype=np.float64) - np.asarray(lse_ref, dtype=np.float64))
        self.max_lse = max(self.max_lse, float(el.max()))

    def report(self):
        return {"rows": self.n, "o_max_abs": self.max_o, "o_mean_abs": self.sum_o / max(1, self.cnt_o),
                "lse_max_abs": self.max_lse, "bounds": {"o_max_abs": 2e-2, "o_mean_abs": 2e-3, "lse_max_abs": 2.5e-3},
                "within": bool(self.max_o <= 2e-2 and self.sum_o / max(1, self.cnt_o) <= 2e-3
                               and self.max_lse <= 2.5e-3)}


def host_cpu():
    """CPU model and logical CPU count of the host the oracle runs on."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count()}


def cpu_baseline_prefill(q, k, v, cfg, budget_s, oracle, o=None, lse=None):
    """Oracle on sampled rows of the causal prefill until ~budget_s of CPU
    work: seeded (b, h) heads, 256 seeded rows of each (full-length fp64
    rows); TFLOP/s on the algorithmic FLOPs of the rows evaluated.  With the
    GPU's o and lse of the same inputs, the oracle rows also give the parity
    errors of those rows."""
    import torch
    from tiled_online_softmax_attention_amd import inputs
    heads = inputs.sample_triples(cfg.seed + 1000, 4096, (cfg.B, cfg.H))
    done_rows, done_heads, flops, t_total = 0, 0, 0.0, 0.0
    par = ParityStats()
    for hi, (b, h) in enumerate(heads):
        rows = inputs.sample_triples(cfg.seed + 2000 + hi, 256, (cfg.N,))
        rows = [r for (r,) in rows]
        qs, ks, vs = (x[b, h].unsqueeze(0).unsqueeze(0).cpu() for x in (q, k, v))
        t0 = time.perf_counter()
        o_ref, l_ref = oracle.attention_rows(qs, ks, vs, cfg.scale, True, [0] * len(rows), [0] * len(rows), rows)
        t_total += time.perf_counter() - t0
        if o is not None:
            idx = torch.tensor(rows, device=o.device)
            par.add(o[b, h].index_select(0, idx).float().cpu().numpy(), o_ref,
                    lse[b, h].index_select(0, idx).cpu().numpy(), l_ref)
        done_rows += len(rows)
        done_heads += 1
        flops += sum(4.0 * cfg.d * (r + 1) for r in rows)
        if t_total >= budget_s:
            break
    res = {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), **host_cpu(), "kind": "oracle",
           "sample": "%d seeded rows (256 per head, %d seeded heads) of the 16x32x8192x128 causal prefill, "
                     "full-length fp64 rows, %.1f s of oracle time" % (done_rows, done_heads, t_total)}
    if o is not None:
        res["parity"] = par.report()
    return res


def cpu_baseline_decode(pi, budget_s, oracle, o=None, lse=None):
    """Oracle on the first requests of the C4 batch until ~budget_s; KV GB/s.
    With the GPU's o and lse, also the parity errors of those rows."""
    import torch
    ctx = pi.ctx_lens.cpu().tolist()
    t_total, nbytes, nreq = 0.0, 0.0, 0
    pool_cpu = None
    par = ParityStats()
    q_cpu, bt_cpu, ctx_cpu, ql_cpu = pi.q.cpu(), pi.block_table.cpu(), pi.ctx_lens.cpu(), pi.q_lens.cpu()
    for r in range(len(ctx)):
        if pool_cpu is None:
            pool_cpu = pi.pool.cpu()
        rows = list(range(pi.H))
        t0 = time.perf_counter()
        o_ref, l_ref = oracle.paged_attention_rows(q_cpu, pool_cpu, bt_cpu, ctx_cpu, ql_cpu, pi.block_size, pi.scale,
                                                   [r] * pi.H, rows, [0] * pi.H)
        t_total += time.perf_counter() - t0
        if o is not None:   # one query row per request: packed row r
            par.add(o[r].float().cpu().numpy(), o_ref, lse[r].cpu().numpy(), l_ref)
        nbytes += paged_bytes([ctx[r]], [1], pi.H, pi.d, pi.block_size)
        nreq += 1
        if t_total >= budget_s:
            break
    res = {"value": nbytes / t_total / 1e9, "unit": "GB/s", "cores": oracle.num_threads(), **host_cpu(), "kind": "oracle",
           "sample": "%d of 64 decode requests (all 32 heads each), %.1f s" % (nreq, t_total)}
    if o is not None:
        res["parity"] = par.report()
    return res


def cpu_baseline_bwd(q, k, v, do, cfg, budget_s, oracle):
    """Oracle backward on sampled dQ rows of the causal workload until
    ~budget_s of CPU work: seeded (b, h) heads, 64 seeded rows each.  Each
    row's work is its S row, dP row and dQ row, i.e. three of the five
    products of the backward, counted as 6*d FLOPs per allowed key."""
    from tiled_online_softmax_attention_amd import inputs
    heads = inputs.sample_triples(cfg.seed + 3000, 4096, (cfg.B, cfg.H))
    done_rows, done_heads, flops, t_total = 0, 0, 0.0, 0.0
    for hi, (b, h) in enumerate(heads):
        rows = [r for (r,) in inputs.sample_triples(cfg.seed + 4000 + hi, 64, (cfg.N,))]
        hk = h // (cfg.H // (cfg.H_kv or cfg.H))
        qs, dos = (x[b, h].unsqueeze(0).unsqueeze(0).cpu() for x in (q, do))
        ks, vs = (x[b, hk].unsqueeze(0).unsqueeze(0).cpu() for x in (k, v))
        t0 = time.perf_counter()
        oracle.attention_bwd_rows(qs, ks, vs, dos, cfg.scale, True, [(0, 0, r) for r in rows], [])
        t_total += time.perf_counter() - t0
        done_rows += len(rows)
        done_heads += 1
        flops += sum(6.0 * cfg.d * (r + 1) for r in rows)
        if t_total >= budget_s:
            break
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(), **host_cpu(), "kind": "oracle",
            "sample": "%d seeded dQ rows (64 per head, %d seeded heads) of the 16x32x8192x128 causal backward, "
                      "full-length fp64 rows (S, dP, dQ products; 6*d FLOPs per allowed key), %.1f s of oracle "
                      "time" % (done_rows, done_heads, t_total)}



def time_bwd(torch, attn, inputs, dev, key, cfg, steps, warmup, keep=False):
    """One backward variant ("mha" or "gqa8"): the forward's O and LSE and dO
    resident in HBM, then `steps` calls of attn_prefill_bwd timed with HIP
    events on their stream.  Returns (entry, wall seconds of the timed calls,
    (q, k, v, dO) if keep else None)."""
    q, k, v = inputs.prefill_inputs(cfg, dev)
    do = inputs.grad_output(cfg, dev)
    o, lse = attn.prefill(q, k, v, True, cfg.scale)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(attn.attn_prefill_bwd_workspace_bytes(cfg.B, cfg.H, cfg.N), dtype=torch.uint8, device=dev)
    timer = EventTimer(torch)
    for _ in range(warmup):
        attn.prefill_bwd(q, k, v, o, lse, do, True, cfg.scale, dq=dq, dk=dk, dv=dv, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        e = timer.start()
        attn.prefill_bwd(q, k, v, o, lse, do, True, cfg.scale, dq=dq, dk=dk, dv=dv, workspace=ws)
        timer.stop(e)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = timer.mean_ms()
    fl = bwd_flops(cfg.B, cfg.H, cfg.N, cfg.d, True)
    tf = fl / (ms * 1e-3) / 1e12
    entry = {"launch_ms": round(ms, 4), "TFLOP/s": round(tf, 2),
             "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                          "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                          "traffic": read_traffic("bwd_c3") if key == "mha" else None,
                          "kernels": "bwd_dq_kernel<128, true> + bwd_dkdv_kernel<128, true>",
                          "flops_per_launch": fl,
                          "executed_flops_per_launch": fl * 7 / 5,
                          "algorithmic_bytes_per_launch": bwd_bytes(cfg.B, cfg.H, cfg.N, cfg.d, H_kv=cfg.H_kv)}}
    if key == "gqa8":
        entry["workload"] = "causal prefill backward bf16 16x32x8192x128, 32 query heads on 4 K/V heads"
    else:
        entry["workload"] = "causal prefill backward bf16 16x32x8192x128, dO iid N(0,1)"
    del o, lse, dq, dk, dv, ws
    kept = (q, k, v, do) if keep else None
    if not keep:
        del q, k, v, do
    torch.cuda.empty_cache()
    return entry, wall, kept

def bench_bwd(args):
    """Backward of the causal 16x32x8192x128 prefill (attn_prefill_bwd: dQ
    kernel + dK/dV kernel) and of its grouped-query variant (4 K/V heads);
    TFLOP/s on the algorithmic FLOPs of the backward (five products of 2*d
    FLOPs per allowed pair), the call's average duration from HIP events on
    its stream.  Inputs, the forward's O and LSE, and dO are resident in HBM
    before timing."""
    import torch
    import tiled_online_softmax_attention_amd as attn
    from tiled_online_softmax_attention_amd import inputs
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    attn.library()
    dev = torch.device("cuda:0")
    res = {"metric": "causal prefill backward TFLOP/s (dQ, dK, dV), 1 MI355X", "value": None, "unit": "TFLOP/s",
           "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "causal prefill backward bf16 16x32x8192x128, dO iid N(0,1)",
                      "global_batch": inputs.C3.B, "seq_len": inputs.C3.N, "parallelism": "none (1 GPU)"}}
    if args.probe_copy:
        probe_copy(torch, dev)
    variants = [("mha", inputs.C3), ("gqa8", inputs.C3_GQA8)]
    if args.bwd_mha_only:
        variants = variants[:1]
    for key, cfg in variants:
        entry, wall, kept = time_bwd(torch, attn, inputs, dev, key, cfg, args.steps, args.warmup,
                                     keep=(key == "mha" and not args.no_cpu_baseline))
        if key == "mha":
            res["value"] = entry["TFLOP/s"]
            res["ms_per_step"] = round(wall * 1e3 / args.steps, 4)
            res["roofline"] = entry["roofline"]
            res["launch_ms"] = entry["launch_ms"]
            if kept is not None:
                import oracle
                print("timing the fp64 oracle on the host", file=sys.stderr, flush=True)
                q, k, v, do = kept
                res["cpu_baseline"] = cpu_baseline_bwd(q, k, v, do, cfg, args.cpu_seconds, oracle)
                del q, k, v, do, kept
                torch.cuda.empty_cache()
        else:
            res["gqa8"] = entry
    print(json.dumps(res), flush=True)


def append_bytes(new_lens, H, d, elem=2):
    """Algorithmic bytes of one KV append: the new K and V rows read once and
    written once, plus each request's lengths and new table entries."""
    t = sum(new_lens)
    return 2 * t * H * d * elem * 2 + len(new_lens) * 12



def time_append(torch, attn, inputs, dev, steps, warmup):
    """KV append on the chunked-prefill shape and on one decode step; each
    timed call (HIP events on its stream) starts from the same cache state
    (table and free count restored, untimed).  Returns {"chunk_c5": ...,
    "decode_c4": ...}."""
    res = {}
    for name, cfg in (("chunk_c5", inputs.C5), ("decode_c4", inputs.C4)):
        ctx, ql, _ = inputs.draw_lengths(cfg)
        ctx, ql = [int(c) for c in ctx], [int(q) for q in ql]
        ctx_old = [c - q for c, q in zip(ctx, ql)]
        ai = inputs.append_inputs(ctx_old, ql, cfg.H, cfg.d, cfg.block_size, cfg.seed, device=dev)
        table0 = ai.block_table.clone()
        free = torch.tensor(ai.free_list + [0] * (ai.pool.shape[0] - len(ai.free_list)), dtype=torch.int32,
                            device=dev)
        count = torch.empty(1, dtype=torch.int32, device=dev)
        ctx_d = torch.tensor(ctx_old, dtype=torch.int32, device=dev)
        new_d = torch.tensor(ql, dtype=torch.int32, device=dev)
        nctx = torch.empty_like(ctx_d)
        status = torch.empty(1, dtype=torch.int32, device=dev)
        timer = EventTimer(torch)
        for i in range(warmup + steps):
            ai.block_table.copy_(table0)
            count.fill_(len(ai.free_list))
            e = timer.start() if i >= warmup else None
            attn.kv_append(ai.k_new, ai.v_new, ctx_d, new_d, ai.pool, ai.block_table, free, count,
                           cfg.block_size, max_new_len=max(ql), new_ctx_lens=nctx, status=status, check=False)
            if e is not None:
                timer.stop(e)
        torch.cuda.synchronize()
        assert int(status.item()) == 0
        ms = timer.mean_ms()
        nb = append_bytes(ql, cfg.H, cfg.d)
        res[name] = {"launch_ms": round(ms, 4), "bytes": nb, "GB/s": round(nb / (ms * 1e-3) / 1e9, 1),
                     "new_tokens": sum(ql), "requests": len(ql),
                     "roofline": {"bound": "hbm", "achieved": round(nb / (ms * 1e-3) / 1e9, 1),
                                  "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                  "frac": round(nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBPS, 4)}}
        del ai, table0, free
        torch.cuda.empty_cache()
    return res

def bench_append(args):
    """KV append (paged_kv_append: allocation launch + copy launch) on the
    chunked-prefill shape (8 requests x 512 tokens onto U[4096, 32768], 32-token
    pages) and on one decode step (64 requests x 1 token onto U[512, 16384],
    16-token pages).  Each timed call starts from the same cache state (table
    and free count restored, untimed), so it allocates and writes the same
    blocks every time."""
    import torch
    import tiled_online_softmax_attention_amd as attn
    from tiled_online_softmax_attention_amd import inputs
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    attn.library()
    dev = torch.device("cuda:0")
    res = {"metric": "paged KV append GB/s", "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "bf16", "data": "synthetic"}
    res.update(time_append(torch, attn, inputs, dev, args.steps, args.warmup))
    res["value"] = res["chunk_c5"]["GB/s"]
    res["config"] = {"workload": "KV append: 8 x 512 tokens (32-token pages) and 64 x 1 token (16-token pages), "
                                 "H=32, d=128"}
    print(json.dumps(res), flush=True)



def time_gqa(torch, attn, inputs, dev, steps, warmup):
    """Grouped-query variants (32 query heads on 4 K/V heads), inputs resident
    in HBM: the causal 16x32x8192x128 prefill (TFLOP/s) and the 64-request
    decode batch (KV GB/s, K/V of the 4 shared heads counted once), each call
    timed with HIP events on its stream."""
    c3, c4 = inputs.C3_GQA8, inputs.C4_GQA8
    q, k, v = inputs.prefill_inputs(c3, dev)
    o = torch.empty_like(q)
    lse = torch.empty((c3.B, c3.H, c3.N), dtype=torch.float32, device=dev)
    pi = inputs.paged_inputs(c4, dev)
    ctx_list, ql_list = pi.ctx_lens.cpu().tolist(), pi.q_lens.cpu().tolist()
    ws = torch.empty(max(1, attn.paged_attn_gqa_workspace_bytes(pi.num_seqs, c4.H, c4.H_kv, c4.d, c4.block_size, 1,
                                                                max(ctx_list))), dtype=torch.uint8, device=dev)
    od = torch.empty_like(pi.q)
    lsed = torch.empty(pi.q.shape[:2], dtype=torch.float32, device=dev)
    t_pre, t_dec = EventTimer(torch), EventTimer(torch)
    for i in range(warmup + steps):
        e = t_pre.start() if i >= warmup else None
        attn.prefill(q, k, v, True, c3.scale, out=o, lse=lse)
        if e is not None:
            t_pre.stop(e)
        e = t_dec.start() if i >= warmup else None
        attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size, pi.scale,
                             max_q_len=1, max_ctx_len=max(ctx_list), out=od, lse=lsed, workspace=ws)
        if e is not None:
            t_dec.stop(e)
    torch.cuda.synchronize()
    ms_p, ms_d = t_pre.mean_ms(), t_dec.mean_ms()
    fl = prefill_flops(c3.B, c3.H, c3.N, c3.d, True)
    nb = paged_bytes(ctx_list, ql_list, c4.H, c4.d, c4.block_size, H_kv=c4.H_kv)
    tf, gbs = fl / (ms_p * 1e-3) / 1e12, nb / (ms_d * 1e-3) / 1e9
    del q, k, v, o, lse, pi, ws, od, lsed
    torch.cuda.empty_cache()
    return {"workload": "causal prefill bf16 16x32x8192x128 with 4 K/V heads + paged decode bf16 64 req x "
                        "1 query, ctx U[512,16384], 16-token pages, 32 query heads on 4 K/V heads",
            "prefill": {"launch_ms": round(ms_p, 4), "TFLOP/s": round(tf, 2),
                        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}},
            "decode": {"launch_ms": round(ms_d, 4), "bytes_per_call": nb, "GB/s": round(gbs, 1),
                       "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                                    "frac": round(gbs / PEAK_HBM_GBPS, 4)}}}

def bench_gqa(args):
    """Grouped-query variants (32 query heads on 4 K/V heads): the causal
    16x32x8192x128 prefill (TFLOP/s) and the 64-request decode batch (KV GB/s,
    K/V of the 4 shared heads counted once)."""
    import torch
    import tiled_online_softmax_attention_amd as attn
    from tiled_online_softmax_attention_amd import inputs
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    attn.library()
    dev = torch.device("cuda:0")
    g = time_gqa(torch, attn, inputs, dev, args.steps, args.warmup)
    res = {"metric": "GQA-8 causal prefill TFLOP/s + paged-decode KV GB/s", "value": g["prefill"]["TFLOP/s"],
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": g["workload"]}, "prefill": g["prefill"], "decode": g["decode"]}
    print(json.dumps(res), flush=True)


# Kernels behind each measured workload, as the launchers pick them for these
# shapes (prefill: paired 128-row tiles in per-head ranges take the plain key
# loop; one-round causal grids take the complementary order and the
# pipelined key loop).
KERNELS = {
    "c3": "prefill_bf16_kernel<128, true, 0>",
    "c2": "prefill_bf16_kernel<128, false, 1>",
    "c4": "paged_decode_mfma_kernel<128, 16> + paged_combine_heads_kernel<128>",
    "c5": "paged_chunk_kernel<128, 32, 0> + paged_combine_heads_kernel<128>",
}


def single_gpu_or_exit(args):
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path; run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)


# timed calls (and untimed warm-up calls) of the GQA-8 and backward entries of
# the default run
EXTRA_STEPS, EXTRA_WARMUP = 5, 2

# warm C2 launches per timed block (time_c2)
C2_BLOCK = 50


def time_c2(torch, attn, inputs, dev, warm_launches, cold_launches):
    """The small causal prefill (1x32x2048x128): warm (inputs in the 256 MB
    last-level cache) and cold (1 GiB written before each launch, outside the
    timed events, so each launch starts from HBM).

    A launch takes ~50 us, about what one call through the Python binding
    costs on the host, so warm launches timed one by one would measure the
    host as well (the GPU idles between them, and a host stall between an
    event and its launch counts as kernel time).  Warm launches are therefore
    timed in blocks of C2_BLOCK back-to-back calls of the C entry point with
    its arguments marshalled once, one event pair per block: a block's time
    is its launches' kernel time plus the gaps the GPU itself leaves between
    them.  A cold launch follows a 1 GiB fill, which keeps the GPU ahead of
    the host, and is timed on its own."""
    c2 = inputs.C2
    q2, k2, v2 = inputs.prefill_inputs(c2, dev)
    o2 = torch.empty_like(q2)
    l2 = torch.empty((c2.B, c2.H, c2.N), dtype=torch.float32, device=dev)
    flush = torch.empty(1 << 28, dtype=torch.float32, device=dev)
    fl = prefill_flops(c2.B, c2.H, c2.N, c2.d, True)
    cargs = (attn._ptr(q2), attn._ptr(k2), attn._ptr(v2), attn._ptr(o2), attn._ptr(l2), c2.B, c2.H, c2.N, c2.d,
             c2.scale, 1, attn._dtype_code(q2), attn._stream(None))

    def launch():
        return attn.attn_prefill_fwd(*cargs)

    rc = launch()
    if rc != 0:
        raise attn.AttnError(rc, "attn_prefill_fwd")
    for _ in range(20):
        launch()
    torch.cuda.synchronize()
    warm, cold = EventTimer(torch), EventTimer(torch)
    for _ in range(max(1, warm_launches // C2_BLOCK)):
        e = warm.start()
        for _ in range(C2_BLOCK):
            launch()
        warm.stop(e)
    for _ in range(cold_launches):
        flush.fill_(1.0)
        e = cold.start()
        launch()
        cold.stop(e)
    torch.cuda.synchronize()

    def entry(t, per, note):
        ms = t.mean_ms() / per
        tf = fl / (ms * 1e-3) / 1e12
        return {"value": round(tf, 2), "unit": "TFLOP/s", "launch_ms": round(ms, 5),
                "launch_ms_median": round(t.median_ms() / per, 5), "launch_ms_min": round(t.min_ms() / per, 5),
                "launches": len(t.pairs) * per, "frac": round(tf / PEAK_BF16_TFLOPS, 4), "note": note}

    res = {"metric": "causal prefill TFLOP/s", "workload": "causal prefill bf16 1x32x2048x128",
           "kernel": KERNELS["c2"], "flops_per_launch": fl,
           "algorithmic_bytes_per_launch": prefill_bytes(c2.B, c2.H, c2.N, c2.d)}
    res["warm"] = entry(warm, C2_BLOCK, "inputs resident in the last-level cache; blocks of %d back-to-back "
                                        "launches through the C entry point, one event pair per block" % C2_BLOCK)
    res["cold"] = entry(cold, 1, "1 GiB written before each launch, outside the timed events")
    res["value"], res["unit"], res["frac"] = res["warm"]["value"], "TFLOP/s", res["warm"]["frac"]
    del q2, k2, v2, o2, l2, flush
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-c2", action="store_true", help="skip the small-prefill timing after the steps")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the GQA-8, backward and KV-append timings after the steps")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--probe-copy", action="store_true",
                    help="also run one 1 GiB device copy (reference kernel for PMC byte counters)")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "c2", "c5", "append", "gqa", "bwd"],
                    default="all")
    ap.add_argument("--bwd-mha-only", action="store_true",
                    help="--only bwd: skip the grouped-query variant (profiling runs)")
    args = ap.parse_args()

    if args.only == "append":
        return bench_append(args)
    if args.only == "gqa":
        return bench_gqa(args)
    if args.only == "bwd":
        return bench_bwd(args)
    single_gpu_or_exit(args)

    import torch
    import tiled_online_softmax_attention_amd as attn
    from tiled_online_softmax_attention_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    attn.library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    c3, c4, c5 = inputs.C3, inputs.C4, inputs.C5
    do_prefill = args.only in ("all", "prefill")
    do_decode = args.only in ("all", "decode")
    do_c5 = args.only in ("all", "c5")

    if args.probe_copy:
        probe_copy(torch, dev)

    print("generating inputs", file=sys.stderr, flush=True)
    if do_prefill:
        q, k, v = inputs.prefill_inputs(c3, dev)
        o = torch.empty_like(q)
        lse = torch.empty((c3.B, c3.H, c3.N), dtype=torch.float32, device=dev)
    if do_decode:
        pi = inputs.paged_inputs(c4, dev)
        ctx_list = pi.ctx_lens.cpu().tolist()
        ql_list = pi.q_lens.cpu().tolist()
        max_ctx = max(ctx_list)
        ws_bytes = attn.paged_attn_workspace_bytes(pi.num_seqs, pi.H, pi.d, pi.block_size, 1, max_ctx)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        od = torch.empty_like(pi.q)
        lsed = torch.empty(pi.q.shape[:2], dtype=torch.float32, device=dev)
    if do_c5:
        p5 = inputs.paged_inputs(c5, dev)
        ctx5 = p5.ctx_lens.cpu().tolist()
        ql5 = p5.q_lens.cpu().tolist()
        ws5 = torch.empty(max(1, attn.paged_attn_workspace_bytes(p5.num_seqs, p5.H, p5.d, p5.block_size,
                                                                  max(ql5), max(ctx5))), dtype=torch.uint8,
                          device=dev)
        o5 = torch.empty_like(p5.q)
        l5 = torch.empty(p5.q.shape[:2], dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    t_pre = EventTimer(torch)
    t_dec = EventTimer(torch)
    t_c5 = EventTimer(torch)

    def step(record):
        if do_prefill:
            e = t_pre.start() if record else None
            attn.prefill(q, k, v, True, c3.scale, out=o, lse=lse)
            if record:
                t_pre.stop(e)
        if do_decode:
            e = t_dec.start() if record else None
            attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size, pi.scale,
                                 max_q_len=1, max_ctx_len=max_ctx, out=od, lse=lsed, workspace=ws)
            if record:
                t_dec.stop(e)
        if do_c5:
            e = t_c5.start() if record else None
            attn.paged_attention(p5.q, p5.pool, p5.block_table, p5.ctx_lens, p5.q_lens, p5.block_size, p5.scale,
                                 max_q_len=max(ql5), max_ctx_len=max(ctx5), out=o5, lse=l5, workspace=ws5)
            if record:
                t_c5.stop(e)

    res = {"metric": METRIC, "value": None, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
           "warmup": args.warmup, "ms_per_step": None, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": "causal prefill bf16 16x32x8192x128 + paged decode bf16 64 req x 1 query, "
                                  "ctx U[512,16384], 16-token pages + paged chunked prefill bf16 8 x 512 rows, "
                                  "prev ctx U[4096,32768], 32-token pages; H=32, d=128",
                      "global_batch": c3.B, "seq_len": c3.N, "parallelism": "none (1 GPU)"}}
    if args.only == "c2":
        c2res = time_c2(torch, attn, inputs, dev, max(args.steps, 2000), max(args.steps, 200))
        res.update(value=c2res["value"], unit="TFLOP/s", steps=c2res["warm"]["launches"],
                   ms_per_step=c2res["warm"]["launch_ms"])
        res["config"].update(workload="causal prefill bf16 1x32x2048x128", global_batch=1, seq_len=2048)
        res["c2"] = c2res
        print(json.dumps(res), flush=True)
        return

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    print("timing %d steps" % args.steps, file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    res["ms_per_step"] = round(wall * 1e3 / args.steps, 4)

    if do_prefill:
        ms = t_pre.mean_ms()
        fl = prefill_flops(c3.B, c3.H, c3.N, c3.d, True)
        tf = fl / (ms * 1e-3) / 1e12
        res["value"] = round(tf, 2)
        res["roofline"] = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(tf / PEAK_BF16_TFLOPS, 4), "traffic": read_traffic("prefill_c3"),
                           "kernel": KERNELS["c3"], "launch_ms": round(ms, 4),
                           "launch_ms_median": round(t_pre.median_ms(), 4), "launch_ms_min": round(t_pre.min_ms(), 4),
                           "flops_per_launch": fl, "algorithmic_bytes_per_launch":
                               prefill_bytes(c3.B, c3.H, c3.N, c3.d)}
    if do_decode:
        ms = t_dec.mean_ms()
        nb = paged_bytes(ctx_list, ql_list, pi.H, pi.d, pi.block_size)
        gbs = nb / (ms * 1e-3) / 1e9
        res["decode"] = {"metric": "paged-decode KV GB/s", "value": round(gbs, 1), "unit": "GB/s",
                         "launch_ms": round(ms, 4), "launch_ms_median": round(t_dec.median_ms(), 4),
                         "launch_ms_min": round(t_dec.min_ms(), 4), "bytes_per_call": nb, "sum_ctx": sum(ctx_list),
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBPS,
                                      "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBPS, 4),
                                      "traffic": read_traffic("decode_c4"), "kernels": KERNELS["c4"]}}
        if not do_prefill:
            res["value"], res["unit"] = round(gbs, 1), "GB/s"
            res["config"].update(workload="paged decode bf16 64 req x 1 query, ctx U[512,16384], 16-token pages, "
                                          "H=32, d=128", global_batch=len(ctx_list), seq_len=1)
    if do_c5:
        ms = t_c5.mean_ms()
        fl = paged_flops(ctx5, ql5, p5.d, p5.H)
        nb = paged_bytes(ctx5, ql5, p5.H, p5.d, p5.block_size)
        tf = fl / (ms * 1e-3) / 1e12
        res["c5"] = {"metric": "paged chunked-prefill TFLOP/s", "value": round(tf, 2), "unit": "TFLOP/s",
                     "kv_gbps": round(nb / (ms * 1e-3) / 1e9, 1), "launch_ms": round(ms, 4),
                     "launch_ms_median": round(t_c5.median_ms(), 4), "launch_ms_min": round(t_c5.min_ms(), 4),
                     "flops_per_call": fl, "bytes_per_call": nb,
                     "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                                  "traffic": read_traffic("chunk_c5"), "kernels": KERNELS["c5"]}}
        if args.only == "c5":
            res["value"], res["unit"] = res["c5"]["value"], "TFLOP/s"
            res["config"].update(workload="paged chunked prefill bf16 8 x 512 rows, prev ctx U[4096,32768], "
                                          "32-token pages", global_batch=len(ql5), seq_len=max(ql5))
    if args.only == "all" and not args.no_c2:
        print("timing the 1x32x2048x128 prefill", file=sys.stderr, flush=True)
        res["c2"] = time_c2(torch, attn, inputs, dev, 2000, 200)
    if args.only == "all" and not args.no_extra:
        # the grouped-query prefill and decode and the backward, a few calls
        # each (their own --only modes time more and add the backward's oracle)
        print("timing the GQA-8 prefill and decode", file=sys.stderr, flush=True)
        res["gqa8"] = time_gqa(torch, attn, inputs, dev, EXTRA_STEPS, EXTRA_WARMUP)
        print("timing the backward", file=sys.stderr, flush=True)
        res["bwd"], _, _ = time_bwd(torch, attn, inputs, dev, "mha", inputs.C3, EXTRA_STEPS, EXTRA_WARMUP)
        print("timing the KV append", file=sys.stderr, flush=True)
        res["append"] = time_append(torch, attn, inputs, dev, 20, 5)

    if not args.no_cpu_baseline and args.only in ("all", "prefill", "decode"):
        import oracle
        print("timing the fp64 oracle on the host", file=sys.stderr, flush=True)
        if do_prefill:
            res["cpu_baseline"] = cpu_baseline_prefill(q, k, v, c3, args.cpu_seconds, oracle, o=o, lse=lse)
        if do_decode:
            cb = cpu_baseline_decode(pi, args.cpu_seconds * 0.5, oracle, o=od, lse=lsed)
            if do_prefill:
                res["cpu_baseline"]["decode"] = cb
            else:
                res["cpu_baseline"] = cb
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
