// attn_mfma_wide.h -- the bf16 MFMA attention forward with 64 query rows per
// wave: four waves per workgroup (256 query rows), one workgroup per CU.
//
// It computes what attn_mfma_kernel.h computes -- the block-wise forward with
// online softmax of "Flash Attention and Paged Attention" (section 2) -- from
// the same tile step pieces (attn_mfma_core.h), laid out differently:
//  * Each wave holds two 32-row query blocks.  Every K fragment and every V^T
//    fragment it reads from LDS feeds two MFMAs (one per block), so the LDS
//    operand reads per MFMA halve, and each K/V tile copied into LDS serves
//    256 query rows instead of 128 (half the copy traffic per FLOP).
//  * About 420 registers per wave (Q and O in AGPRs): one wave per SIMD.  A
//    wave's VALU work issues alongside its own MFMAs while they execute (they
//    do not depend on each other), so the key loop is software-pipelined by
//    one tile: the
//    MFMAs of S for tile j+1 run while the wave computes the exponentials of
//    tile j, and the P V MFMAs of tile j run while it takes the row maxima of
//    tile j+1 and decides the offset update for it.
//  * K/V tiles of 32 keys go through a ring of four LDS buffers (distinct
//    __shared__ objects, indexed statically by unrolling the key loop by four),
//    copied global -> LDS two tiles ahead, one barrier per tile.
//
// Key tiles [0, nf4) -- the full tiles rounded down to a multiple of four --
// take the pipelined step; the rest (the causal diagonal, the tail of the
// context and up to three full tiles) take a plain masked step.
//
// Measured on the 16x32x8192x128 causal prefill (same-box A/B and rocprofv3
// counters): the lower LDS and copy traffic per FLOP lets the chip hold
// ~2.1 GHz against ~1.7 GHz for the 32-row kernel, but a lone wave per SIMD
// keeps its matrix pipe busy only ~46-48 % of the cycles against ~60 % (the
// per-tile barrier, the exposed start of every workgroup and the unpipelined
// diagonal tiles have no other wave to cover them): 0.92-0.94 of the 32-row
// kernel's rate.  launch_prefill therefore takes it only when asked
// (PrefillArgs::wide = 1, ATTN_PREFILL_WIDE=1).
#pragma once

#include "attn_mfma_kernel.h"

namespace attn {

// Query rows per workgroup of the wide kernel: 4 waves x 64.
constexpr int kWideRows = 256;
constexpr int kWideBufs = 4;

// The four LDS buffers of the ring; tile t lives in b[t % 4].
struct WideBuffers {
    char* b[kWideBufs];
};

template <int D>
struct VReadOffsets;

// S^T = K Q^T for both query blocks of one key tile; each K fragment is read
// once from LDS and used by both blocks' MFMAs.
template <int D>
__device__ __forceinline__ void qk_tile2(TileScores<D> (&S)[2], const bf16x8 (&qf)[2][TileCfg<D>::KSTEPS],
                                         const char* lds_k, int lane)
{
    using C = TileCfg<D>;
    const int g = lane >> 5, r32 = lane & 31;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb) {
        bf16x8 kf[C::KSTEPS];
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
            kf[ks] = as_bf16x8(*(const u32x4*)(lds_k + k_ofs<D>(kb * 32 + r32, ks * 2 + g)));
        f32x16 a0 = f32x16{}, a1 = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            a0 = mfma32(kf[ks], qf[0][ks], a0);
            a1 = mfma32(kf[ks], qf[1][ks], a1);
        }
        // the scores feed VALU work (maxima, exponentials): ask for them in
        // VGPRs, which the VALU reads directly (an AGPR would need a copy)
        asm volatile("" : "+v"(a0), "+v"(a1));
        S[0].s[kb] = a0;
        S[1].s[kb] = a1;
    }
}

// V^T operands of one key tile (two transposing LDS reads each), read ahead
// of the MFMAs that use them: a lone wave per SIMD has no other wave to cover
// LDS latency.  Operand layout as pv_tile.
template <int D>
struct VOperands {
    bf16x8 a[TileCfg<D>::KBLK][2][TileCfg<D>::DBLK];
};

// Per-lane byte offsets of this lane's transposing V reads within a V tile,
// one per 32-wide d block: the XOR swizzle depends on the d block and on row
// bits that the 8-, 16- and 32-row steps of the reads leave unchanged, so the
// other reads of a tile are these plus immediates.
template <int D>
struct VReadOffsets {
    uint32_t o[TileCfg<D>::DBLK];
};

template <int D>
__device__ __forceinline__ void v_read_offsets(VReadOffsets<D>& vo, int lane)
{
    using C = TileCfg<D>;
    const int g = lane >> 5;
    const uint32_t tr_row = (uint32_t)(g * 4 + ((lane & 15) >> 2));
    const uint32_t tr_col = (uint32_t)((((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2);
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) {
        const uint32_t cb = tr_col + db * 64;
        vo.o[db] = v_ofs<D>(tr_row, cb >> 4) + (cb & 15u);
    }
}

// Per-wave constants: the driver's WaveCtx plus the key limit of the second
// query block and the lane's V read offsets.
template <int D>
struct WideCtx {
    WaveCtx cx;            // cx.q_lim: limit of block 0
    int q_lim1;            // limit of block 1
    int nf4;               // tiles taken by the pipelined step (a multiple of 4)
    VReadOffsets<D> vro;
};

template <int D>
__device__ __forceinline__ void read_v_tile(VOperands<D>& va, const char* lds_v, const VReadOffsets<D>& vo)
{
    using C = TileCfg<D>;
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db) {
                const char* p = lds_v + vo.o[db] + (kb * 32 + 16 * h) * C::ROW_BYTES;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p + 8 * C::ROW_BYTES));
                va.a[kb][h][db] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            }
}

// O^T += V^T P^T for both query blocks; each V^T operand is used by both
// blocks' MFMAs.
template <int D>
__device__ __forceinline__ void pv_tile2(WaveState<D> (&st)[2], const bf16x2 (&pk)[2][TileCfg<D>::KBLK][8],
                                         const VOperands<D>& va)
{
    using C = TileCfg<D>;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x8 b0 =
                cat8(pk[0][kb][4 * h + 0], pk[0][kb][4 * h + 1], pk[0][kb][4 * h + 2], pk[0][kb][4 * h + 3]);
            const bf16x8 b1 =
                cat8(pk[1][kb][4 * h + 0], pk[1][kb][4 * h + 1], pk[1][kb][4 * h + 2], pk[1][kb][4 * h + 3]);
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db) {
                st[0].o[db] = mfma32(va.a[kb][h][db], b0, st[0].o[db]);
                st[1].o[db] = mfma32(va.a[kb][h][db], b1, st[1].o[db]);
            }
        }
}

// Instruction order of a pipelined step (scheduling groups; mask bits: 0x2
// VALU, 0x8 MFMA, 0x20 global load, 0x100 LDS read): all LDS operand reads
// first, then the copies of a later tile, a few VALU instructions while the
// reads land, then each S MFMA of the next tile followed by
// exponential work of this tile, then each P V MFMA followed by maximum work
// of the next tile.
template <int D>
__device__ __forceinline__ void schedule_pipelined_step()
{
    using C = TileCfg<D>;
    constexpr int kReads = C::KBLK * (C::KSTEPS + 2 * 2 * C::DBLK);
    constexpr int kMfma = 2 * C::KBLK * C::KSTEPS;     // S MFMAs of both blocks (as many P V MFMAs)
    __builtin_amdgcn_sched_group_barrier(0x100, kReads, 0);
    __builtin_amdgcn_sched_group_barrier(0x020, C::COPIES_PER_GROUP, 0);   // copies, after the reads
    __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
}

// Offset update of one block inside the shared branch below: same rule as
// update_offset (O and l follow the offset; a block whose maximum did not move
// gets alpha = 1).
template <int D>
__device__ __forceinline__ void move_offset(WaveState<D>& ws, float mt, float c2)
{
    using C = TileCfg<D>;
    const float m_new = fmaxf(ws.m, mt);
    const float alpha = (ws.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ws.m - m_new) * c2);
    ws.m = m_new;
    ws.ms = (m_new == -INFINITY) ? 0.f : m_new * c2;
    ws.l *= alpha;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) scale_in_place(ws.o[db], alpha);
}

// Lazy offset update of both blocks with one wave-uniform branch: taken when
// some query of either block exceeds its offset by more than the headroom.
template <int D>
__device__ __forceinline__ void update_offset2(WaveState<D> (&st)[2], float mt0, float mt1, float c2, float thr)
{
    if (__builtin_amdgcn_ballot_w64((mt0 > st[0].m + thr) || (mt1 > st[1].m + thr)) != 0) {
        move_offset(st[0], mt0, c2);
        move_offset(st[1], mt1, c2);
    }
}

// Copies of one tile into `buf` (K at byte 0, V at TILE_BYTES; wave w < 2
// copies K group w, the others V group w - 2) from a contiguous [N, d] head
// slab.  The buffer descriptor starts at the group's first row (clamped to N)
// and covers the rest of the slab, so each lane's offset is the
// loop-invariant cx.voff plus a wave-uniform step per copy, and the range
// check (which covers that per-lane offset) returns zero for rows at or past
// N -- keys that the mask removes (p = 0), whose K and V values never matter.
// Branch-free and free of per-lane arithmetic, which keeps a step's copies in
// the same scheduling region as its LDS reads and MFMAs.
template <int D, class KV>
__device__ __forceinline__ void issue_tile_copies_flat(const KV& kv, const WaveCtx& cx, char* buf, int key_base)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using C = TileCfg<D>;
    const bool is_v = cx.w >= C::GROUPS;
    const int grp = is_v ? cx.w - C::GROUPS : cx.w;
    const int gkey = min(key_base + 16 * grp, cx.kv_end);   // uniform, <= N
    const uint32_t skip = (uint32_t)gkey * C::ROW_BYTES;     // < N * ROW_BYTES + 1 <= slab bytes + 1
    const char* base = (is_v ? kv.v_group(0, cx.kv_end) : kv.k_group(0, cx.kv_end)) + skip;
    const __amdgpu_buffer_rsrc_t r = raw_rsrc(base, kv.group_bytes() - skip);
    char* dst = buf + (is_v ? C::TILE_BYTES : 0) + grp * 16 * C::ROW_BYTES;
    const uint32_t step = is_v ? kVDmaStep : kKDmaStep;
#pragma unroll
    for (int i = 0; i < C::COPIES_PER_GROUP; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ATTN_LDS(dst + i * 1024), 16, cx.voff + i * step, 0, 0, 0);
#endif
}

// Copy protocol of the ring: the copies of tiles 0 and 1 are issued before
// the loop, and the step that publishes tile t issues the copies of tile
// t + 2 (into the buffer of tile t - 2, which every wave is done with once it
// has passed the barrier that publishes t), whether or not tile t + 2 exists.
// So at every publish exactly two tiles' copies are in flight, and waiting
// until one tile's worth remains means tile t has landed.
template <int D>
__device__ __forceinline__ void publish_tile()
{
    static_assert(TileCfg<D>::COPIES_PER_GROUP < 16, "vmcnt field");
    // The empty asm statements keep the compiler from moving memory accesses
    // across the barrier (s_barrier alone is not a memory operation to it);
    // unlike a workgroup fence they add no wait for the copies in flight.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x3f70 | TileCfg<D>::COPIES_PER_GROUP);   // vmcnt(one tile's copies)
    __builtin_amdgcn_s_waitcnt(0xc07f);                                  // lgkmcnt(0): this wave's LDS reads done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Pipelined step for tile j (in buffer I), whose scores S[cur] and offset
// update are done: publish tile j + 1, S of tile j + 1 into S[nxt], p of tile
// j, O += P V of tile j, maxima and offset update of tile j + 1.  Tile j + 1
// is a full tile (j + 1 < nf4).
template <int D, int I, class KV>
__device__ __forceinline__ void wide_step_next(WaveState<D> (&st)[2], TileScores<D> (&Scur)[2],
                                               TileScores<D> (&Snxt)[2], const bf16x8 (&qf)[2][TileCfg<D>::KSTEPS],
                                               const KV& kv, const WideCtx<D>& wc, const WideBuffers& buf, int j)
{
    using C = TileCfg<D>;
    constexpr int IN = (I + 1) % kWideBufs;
    publish_tile<D>();   // tile j + 1
    VOperands<D> va;
    read_v_tile(va, buf.b[I] + C::TILE_BYTES, wc.vro);
    qk_tile2(Snxt, qf, buf.b[IN], wc.cx.lane);
    issue_tile_copies_flat<D>(kv, wc.cx, buf.b[(I + 3) % kWideBufs], wc.cx.kv_begin + (j + 3) * C::BN);
    bf16x2 pk[2][C::KBLK][8];
    exp_tile(pk[0], Scur[0], st[0], wc.cx.c2);
    exp_tile(pk[1], Scur[1], st[1], wc.cx.c2);
    pv_tile2(st, pk, va);
    const int key1 = wc.cx.kv_begin + (j + 1) * C::BN;
    const float mt0 = tile_max<D, false>(Snxt[0], wc.cx.lane, key1, wc.cx.q_lim);
    const float mt1 = tile_max<D, false>(Snxt[1], wc.cx.lane, key1, wc.q_lim1);
    schedule_pipelined_step<D>();
    update_offset2(st, mt0, mt1, wc.cx.c2, wc.cx.thr);
}

// Last pipelined step (tile j = nf4 - 1): p and O += P V of tile j only.
template <int D, int I>
__device__ __forceinline__ void wide_step_last(WaveState<D> (&st)[2], TileScores<D> (&Scur)[2], const WideCtx<D>& wc,
                                               const WideBuffers& buf)
{
    using C = TileCfg<D>;
    VOperands<D> va;
    read_v_tile(va, buf.b[I] + C::TILE_BYTES, wc.vro);
    bf16x2 pk[2][C::KBLK][8];
    exp_tile(pk[0], Scur[0], st[0], wc.cx.c2);
    exp_tile(pk[1], Scur[1], st[1], wc.cx.c2);
    pv_tile2(st, pk, va);
}

// Plain step for tile t (in buffer I) with the causal / tail mask: publish it,
// S, mask and maxima, offset update, p, O += P V.
template <int D, int I, class KV>
__device__ __forceinline__ void wide_step_masked(WaveState<D> (&st)[2], const bf16x8 (&qf)[2][TileCfg<D>::KSTEPS],
                                                 const KV& kv, const WideCtx<D>& wc, const WideBuffers& buf, int t)
{
    using C = TileCfg<D>;
    publish_tile<D>();   // tile t
    TileScores<D> S[2];
    qk_tile2(S, qf, buf.b[I], wc.cx.lane);
    issue_tile_copies_flat<D>(kv, wc.cx, buf.b[(I + 2) % kWideBufs], wc.cx.kv_begin + (t + 2) * C::BN);
    const int key0 = wc.cx.kv_begin + t * C::BN;
    const float mt0 = tile_max<D, true>(S[0], wc.cx.lane, key0, wc.cx.q_lim);
    const float mt1 = tile_max<D, true>(S[1], wc.cx.lane, key0, wc.q_lim1);
    update_offset2(st, mt0, mt1, wc.cx.c2, wc.cx.thr);
    VOperands<D> va;
    read_v_tile(va, buf.b[I] + C::TILE_BYTES, wc.vro);
    bf16x2 pk[2][C::KBLK][8];
    exp_tile(pk[0], S[0], st[0], wc.cx.c2);
    exp_tile(pk[1], S[1], st[1], wc.cx.c2);
    pv_tile2(st, pk, va);
}

// The key loop of one wave (copy protocol above).
template <int D, class KV>
__device__ __forceinline__ void wide_key_loop(WaveState<D> (&st)[2], const bf16x8 (&qf)[2][TileCfg<D>::KSTEPS],
                                              const KV& kv, const WideCtx<D>& wc, const WideBuffers& buf)
{
    using C = TileCfg<D>;
    const int ntile = wc.cx.ntile, nf4 = wc.nf4;
    issue_tile_copies_flat<D>(kv, wc.cx, buf.b[0], wc.cx.kv_begin);
    issue_tile_copies_flat<D>(kv, wc.cx, buf.b[1], wc.cx.kv_begin + C::BN);
    if (nf4 > 0) {
        // prologue: publish tile 0, its scores, maxima and offset
        publish_tile<D>();
        TileScores<D> Sa[2], Sb[2];
        qk_tile2(Sa, qf, buf.b[0], wc.cx.lane);
        issue_tile_copies_flat<D>(kv, wc.cx, buf.b[2], wc.cx.kv_begin + 2 * C::BN);
        {
            const float mt0 = tile_max<D, false>(Sa[0], wc.cx.lane, wc.cx.kv_begin, wc.cx.q_lim);
            const float mt1 = tile_max<D, false>(Sa[1], wc.cx.lane, wc.cx.kv_begin, wc.q_lim1);
            update_offset2(st, mt0, mt1, wc.cx.c2, wc.cx.thr);
        }
        // tiles j .. j + 3 in buffers 0 .. 3; scores alternate Sa / Sb
        int j = 0;
        for (; j + 4 < nf4; j += 4) {
            wide_step_next<D, 0>(st, Sa, Sb, qf, kv, wc, buf, j);
            wide_step_next<D, 1>(st, Sb, Sa, qf, kv, wc, buf, j + 1);
            wide_step_next<D, 2>(st, Sa, Sb, qf, kv, wc, buf, j + 2);
            wide_step_next<D, 3>(st, Sb, Sa, qf, kv, wc, buf, j + 3);
        }
        // last group of four: tile nf4 - 1 has no pipelined successor
        wide_step_next<D, 0>(st, Sa, Sb, qf, kv, wc, buf, j);
        wide_step_next<D, 1>(st, Sb, Sa, qf, kv, wc, buf, j + 1);
        wide_step_next<D, 2>(st, Sa, Sb, qf, kv, wc, buf, j + 2);
        wide_step_last<D, 3>(st, Sb, wc, buf);
    }
    // masked tiles, from a multiple of four: static buffer indices again
    for (int t = nf4; t < ntile; t += 4) {
        wide_step_masked<D, 0>(st, qf, kv, wc, buf, t);
        if (t + 1 < ntile) wide_step_masked<D, 1>(st, qf, kv, wc, buf, t + 1);
        if (t + 2 < ntile) wide_step_masked<D, 2>(st, qf, kv, wc, buf, t + 2);
        if (t + 3 < ntile) wide_step_masked<D, 3>(st, qf, kv, wc, buf, t + 3);
    }
    // the last two tiles' copies (past the context) may still be in flight:
    // drain them before the workgroup's LDS can be handed on
    __builtin_amdgcn_s_waitcnt(0x3f70);
}

// One 256-row query tile: Q fragments of both blocks, the key loop, and the
// epilogue (O / l and the log-sum-exp of the valid rows).
template <int D, class KV>
__device__ __forceinline__ void run_wide_tile(const TileProblem& P, const KV& kv, const TileOut& out, float c2_in,
                                              const WideBuffers& buf)
{
    using C = TileCfg<D>;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    WideCtx<D> wc;
    bf16x8 qf[2][C::KSTEPS];
    int n_full;
    // block b of wave w is the 32-row block 2w + b of the tile
    WaveCtx c1;
    init_query_tile<D>(P, c1, qf[1], c2_in, 2 * w + 1, &n_full);
    wc.q_lim1 = c1.q_lim;
    wc.cx.ntile = init_query_tile<D>(P, wc.cx, qf[0], c2_in, 2 * w, &n_full);
    wc.cx.w = w;               // the copy role is the wave's own index
    wc.cx.kv_begin = P.kv_begin;
    wc.cx.kv_end = P.kv_end;
    wc.cx.voff = copy_voff<D>(w, wc.cx.lane);
    wc.nf4 = n_full & ~3;
    v_read_offsets<D>(wc.vro, wc.cx.lane);
    // Q fragments are only MFMA operands: keep them in AGPRs, leaving VGPRs
    // for the scores and the LDS operands
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) asm volatile("" : "+a"(qf[b][ks]));
    WaveState<D> st[2];
    clear_state(st[0]);
    clear_state(st[1]);
    // every wave computes (rows past n_rows run on zero queries, never stored)
    wide_key_loop<D>(st, qf, kv, wc, buf);
    WaveCtx sc = wc.cx;
    sc.w = 2 * w;
    store_query_rows(st[0], P, out, sc);
    sc.w = 2 * w + 1;
    store_query_rows(st[1], P, out, sc);
}

}  // namespace attn
