"""Seeded synthetic inputs for the attention workloads.

This module only draws random numbers and lays them out; it holds none of the
attention arithmetic.  Both the HIP path (through the tests and the benchmark)
and the fp64 oracle consume exactly the tensors built here.

Recipe (the same for every workload):
  * Q, K, V entries are iid N(0, 1), drawn in fp32 from a seeded torch
    Generator on the target device, then rounded to bf16 (round to nearest
    even) unless the workload is fp32.
  * Paged workloads draw their integer structure from a CPU Generator seeded
    with the same seed, in this order: context lengths (integers, inclusive at
    both ends), then one random permutation of all physical block ids.  The
    first sum(ceil(ctx_r / block_size)) ids of the permutation are handed to
    the requests in request order; the rest (1 % spares, at least one) stay
    unused.
  * Pool contents: every slot of the pool is drawn N(0,1); then spare blocks,
    and the slots past each request's context in its last block, are
    overwritten with NaN so that any stray read shows up in the output.
  * Unused block-table entries are -1.
  * The output gradient dO of a backward workload is iid N(0, 1) like Q,
    drawn from its own generator (seed + 7919), rounded to bf16.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class PrefillConfig:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: torch.dtype
    causal: bool
    seed: int
    tile: int | None = None  # key-tile size the workload names, if any
    H_kv: int | None = None  # K/V heads (grouped-query attention); None = H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


@dataclass(frozen=True)
class PagedConfig:
    name: str
    num_seqs: int
    q_len: int
    H: int
    d: int
    block_size: int
    ctx_lo: int          # inclusive bounds of the drawn length
    ctx_hi: int
    prefix_draw: bool    # True: draw the existing context, ctx = drawn + q_len
    seed: int
    dtype: torch.dtype = torch.bfloat16
    H_kv: int | None = None  # K/V heads in the pool (grouped-query attention); None = H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


# The five workloads (the pages profile a 7B-shaped model at seq 8192, batch 16;
# these synthetic shapes stand in for it -- no weights or datasets are used).
C1 = PrefillConfig("c1_fp32_noncausal_1x1x256x64", 1, 1, 256, 64, torch.float32, False, 1, tile=64)
C2 = PrefillConfig("c2_causal_bf16_1x32x2048x128", 1, 32, 2048, 128, torch.bfloat16, True, 2)
C3 = PrefillConfig("c3_causal_bf16_16x32x8192x128", 16, 32, 8192, 128, torch.bfloat16, True, 3)
C4 = PagedConfig("c4_paged_decode_64req_ctx512-16384_bs16", 64, 1, 32, 128, 16, 512, 16384, False, 4)
C5 = PagedConfig("c5_paged_chunk_8x512_prev4096-32768_bs32", 8, 512, 32, 128, 32, 4096, 32768, True, 5)

# Grouped-query variants of the long prefill and the decode batch: 32 query
# heads sharing 4 K/V heads (groups of 8, the grouping of the GQA example of
# "Sequence length doubles, inference time quadruples"); same seeds, so the
# decode variant draws C4's context lengths.
C3_GQA8 = PrefillConfig("c3_gqa8_causal_bf16_16x32x8192x128_kv4", 16, 32, 8192, 128, torch.bfloat16, True, 3,
                        H_kv=4)
C4_GQA8 = PagedConfig("c4_gqa8_paged_decode_64req_ctx512-16384_bs16_kv4", 64, 1, 32, 128, 16, 512, 16384, False, 4,
                      H_kv=4)

CONFIGS = {"c1": C1, "c2": C2, "c3": C3, "c4": C4, "c5": C5}


def _randn(shape, gen, device, dtype, chunk_elems=1 << 28):
    """iid N(0,1) drawn in fp32, rounded to dtype, filled in fixed-size chunks
    (so large tensors never need a full fp32 copy)."""
    out = torch.empty(shape, dtype=dtype, device=device)
    flat = out.view(-1)
    n = flat.numel()
    for s in range(0, n, chunk_elems):
        e = min(n, s + chunk_elems)
        flat[s:e] = torch.randn(e - s, generator=gen, device=device, dtype=torch.float32).to(dtype)
    return out


def device_generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def prefill_inputs(cfg: PrefillConfig, device="cpu", B=None, H=None, N=None, seed=None):
    """q of shape [B, H, N, d] and k, v of shape [B, H_kv, N, d] (H_kv = H
    unless the config names fewer K/V heads; overrides allow smaller variants)."""
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    N = cfg.N if N is None else N
    H_kv = H if cfg.H_kv is None else cfg.H_kv
    g = device_generator(cfg.seed if seed is None else seed, device)
    q = _randn((B, H, N, cfg.d), g, device, cfg.dtype)
    k = _randn((B, H_kv, N, cfg.d), g, device, cfg.dtype)
    v = _randn((B, H_kv, N, cfg.d), g, device, cfg.dtype)
    return q, k, v


def grad_output(cfg: PrefillConfig, device="cpu", B=None, H=None, N=None):
    """dO of shape [B, H, N, d] for a backward workload (own seeded stream)."""
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    N = cfg.N if N is None else N
    g = device_generator(cfg.seed + 7919, device)
    return _randn((B, H, N, cfg.d), g, device, cfg.dtype)


@dataclass
class PagedInputs:
    q: torch.Tensor            # packed [sum(q_lens), H, d]
    pool: torch.Tensor         # [num_blocks, 2, H, block_size, d]
    block_table: torch.Tensor  # int32 [num_seqs, max_blocks_per_seq], -1 padded
    ctx_lens: torch.Tensor     # int32 [num_seqs] (includes the new tokens)
    q_lens: torch.Tensor       # int32 [num_seqs]
    block_size: int
    scale: float
    spare_blocks: list = field(default_factory=list)

    @property
    def num_seqs(self):
        return self.block_table.shape[0]

    @property
    def H(self):
        return self.pool.shape[2]

    @property
    def d(self):
        return self.pool.shape[4]

    @property
    def num_blocks(self):
        return self.pool.shape[0]

    @property
    def max_blocks_per_seq(self):
        return self.block_table.shape[1]

    @property
    def max_ctx_len(self):
        return int(self.ctx_lens.max())

    @property
    def max_q_len(self):
        return int(self.q_lens.max())


def draw_lengths(cfg: PagedConfig, num_seqs=None, ctx_lo=None, ctx_hi=None):
    """(ctx_lens, q_lens, cpu generator positioned after the draw)."""
    n = cfg.num_seqs if num_seqs is None else num_seqs
    lo = cfg.ctx_lo if ctx_lo is None else ctx_lo
    hi = cfg.ctx_hi if ctx_hi is None else ctx_hi
    g = torch.Generator()
    g.manual_seed(cfg.seed)
    drawn = torch.randint(lo, hi + 1, (n,), generator=g, dtype=torch.int64)
    q_lens = torch.full((n,), cfg.q_len, dtype=torch.int64)
    ctx = drawn + cfg.q_len if cfg.prefix_draw else drawn
    return ctx.to(torch.int32), q_lens.to(torch.int32), g


def build_paged(ctx_lens, q_lens, H, d, block_size, seed, device="cpu", dtype=torch.bfloat16,
                cpu_gen=None, spare_frac=0.01, poison=True, max_blocks_per_seq=None, extra_blocks=0, H_q=None):
    """Lay out a scattered paged KV pool of H heads for the given lengths (plus
    extra_blocks unused blocks on top of the ~spare_frac spares); q gets H_q
    heads (default H; more for grouped-query attention)."""
    ctx_lens = torch.as_tensor(ctx_lens, dtype=torch.int32).cpu()
    q_lens = torch.as_tensor(q_lens, dtype=torch.int32).cpu()
    if cpu_gen is None:
        cpu_gen = torch.Generator()
        cpu_gen.manual_seed(seed)
    nblk = [(int(c) + block_size - 1) // block_size for c in ctx_lens]
    used = sum(nblk)
    spare = max(1, math.ceil(spare_frac * used)) + int(extra_blocks)
    num_blocks = used + spare
    perm = torch.randperm(num_blocks, generator=cpu_gen).to(torch.int32)
    maxb = max(nblk) if max_blocks_per_seq is None else max_blocks_per_seq
    table = torch.full((len(nblk), maxb), -1, dtype=torch.int32)
    pos = 0
    for r, nb in enumerate(nblk):
        table[r, :nb] = perm[pos:pos + nb]
        pos += nb
    spare_ids = perm[used:].tolist()

    g = device_generator(seed, device)
    pool = _randn((num_blocks, 2, H, block_size, d), g, device, dtype)
    q = _randn((int(q_lens.sum()), H if H_q is None else H_q, d), g, device, dtype)
    if poison:
        nan = float("nan")
        if spare_ids:
            pool[torch.tensor(spare_ids, dtype=torch.long, device=device)] = nan
        for r, c in enumerate(ctx_lens.tolist()):
            tail = c % block_size
            if tail:
                last = int(table[r, nblk[r] - 1])
                pool[last, :, :, tail:, :] = nan
    return PagedInputs(q=q, pool=pool, block_table=table.to(device), ctx_lens=ctx_lens.to(device),
                       q_lens=q_lens.to(device), block_size=block_size, scale=1.0 / math.sqrt(d),
                       spare_blocks=spare_ids)


def paged_inputs(cfg: PagedConfig, device="cpu", num_seqs=None, ctx_lo=None, ctx_hi=None, H=None):
    ctx, ql, g = draw_lengths(cfg, num_seqs, ctx_lo, ctx_hi)
    H = cfg.H if H is None else H
    H_kv = H if cfg.H_kv is None else cfg.H_kv
    return build_paged(ctx, ql, H_kv, cfg.d, cfg.block_size, cfg.seed, device, cfg.dtype, cpu_gen=g, H_q=H)


@dataclass
class AppendInputs:
    pool: torch.Tensor         # [num_blocks, 2, H, block_size, d]; spare blocks NaN
    block_table: torch.Tensor  # int32 [num_seqs, max_blocks]; entries past ceil(ctx_old/bs) are -1
    ctx_old: torch.Tensor      # int32 [num_seqs]: tokens cached before the append
    new_lens: torch.Tensor     # int32 [num_seqs]: tokens to append
    k_new: torch.Tensor        # packed [sum(new_lens), H, d]
    v_new: torch.Tensor
    free_list: list            # free block ids, bottom of the stack first
    block_size: int


def append_inputs(ctx_old, new_lens, H, d, block_size, seed, device="cpu", dtype=torch.bfloat16, slack_blocks=4,
                  table_slack=1):
    """A paged cache holding ctx_old tokens per request, a free list with
    enough blocks for appending new_lens tokens (plus slack_blocks), and the
    new K/V rows.  Free ids are the pool's spare blocks in seeded order."""
    ctx_old = [int(c) for c in ctx_old]
    new_lens = [int(n) for n in new_lens]
    bs = block_size
    need = sum(-(-(c + n) // bs) - (-(-c // bs)) for c, n in zip(ctx_old, new_lens))
    maxb = max(1, max(-(-(c + n) // bs) for c, n in zip(ctx_old, new_lens))) + table_slack
    pi = build_paged(ctx_old, [0] * len(ctx_old), H, d, bs, seed, device, dtype, spare_frac=0.0,
                     max_blocks_per_seq=maxb, extra_blocks=need + slack_blocks - 1)
    g = device_generator(seed + 7919, device)
    tot = sum(new_lens)
    k_new = _randn((tot, H, d), g, device, dtype)
    v_new = _randn((tot, H, d), g, device, dtype)
    return AppendInputs(pool=pi.pool, block_table=pi.block_table, ctx_old=pi.ctx_lens,
                        new_lens=torch.tensor(new_lens, dtype=torch.int32, device=device), k_new=k_new, v_new=v_new,
                        free_list=list(pi.spare_blocks), block_size=bs)


def sample_triples(seed: int, n: int, dims, edge=()):
    """n seeded index tuples uniform over the given dims, plus fixed edge tuples."""
    g = torch.Generator()
    g.manual_seed(seed)
    cols = [torch.randint(0, int(dm), (n,), generator=g) for dm in dims]
    out = [tuple(int(c[i]) for c in cols) for i in range(n)]
    out.extend(tuple(e) for e in edge)
    return out
