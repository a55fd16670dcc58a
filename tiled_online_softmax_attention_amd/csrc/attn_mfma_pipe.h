// attn_mfma_pipe.h -- the bf16 MFMA attention forward with a software-pipelined
// key loop: 32 query rows per wave, four or eight waves per workgroup, every
// K/V tile staged in LDS once for the workgroup's 128 or 256 rows.
//
// It computes what attn_mfma_kernel.h computes -- the block-wise forward with
// online softmax of "Flash Attention and Paged Attention" (section 2) -- from
// the same tile-step pieces (attn_mfma_core.h), in another order:
//  * The matrix pipe takes VALU work beside an MFMA best when both come from
//    the same wave; while a wave runs its softmax alone, the other waves of
//    its SIMD can only issue their own MFMAs.  So each wave interleaves its own
//    work: the MFMAs of S for tile j+1 run while the wave computes the
//    exponentials of tile j, and the P V MFMAs of tile j run while it takes
//    the row maxima of tile j+1 and decides the offset update for it.
//  * K/V tiles of 32 keys go through a ring of four LDS buffers (distinct
//    __shared__ objects, indexed statically by unrolling the key loop by
//    four), copied global -> LDS two tiles ahead, one barrier per tile.  A
//    step reads the K fragments of its S MFMAs first and spreads the V^T reads
//    over those MFMAs, so the first MFMA waits for 8 LDS reads, not 24.
//  * ~200 registers per wave: two waves per SIMD, i.e. two workgroups of four
//    waves or one of eight per CU.  Eight waves share each K/V tile between
//    two 128-row query tiles, which halves the copies (global -> LDS) per
//    MFMA and, where the K/V does not stay in L2, the K/V read from memory.
//  * The K/V source is a policy object (contiguous head slab or paged pool).
//    For the loop it has a small per-wave state, SrcWin (for the paged pool:
//    a window of 64 page-table entries in one register, lane l holding page
//    base + l), and three members: win_update(win, cx, key_lo, key_hi)
//    makes the window cover the copies of keys [key_lo, key_hi] (reloading
//    it from LDS when it does not), copy_src(win, cx, key_base) the value a
//    tile's copies need (a page entry, read out of the window register: no
//    memory access), and copy_tile<NW>(cx, buf, key_base, src), this wave's
//    share of the copies.  The window is updated once per four pipelined
//    steps, before a barrier whose wait covers its reload, so a step's
//    schedule holds no extra LDS read or wait.
//
// The operations on O, l and the offset are the plain loop's, in the same
// order, so the two loops give the same bits.  Key tiles [0, nf4) -- the full
// tiles rounded down to a multiple of four -- take the pipelined step; the
// rest (the causal diagonal, the tail of the context and up to three full
// tiles) take a plain masked step.
#pragma once

#include "attn_mfma_kernel.h"

namespace attn {

constexpr int kPipeBufs = 4;

// Copies of one K/V tile are split over the waves of a workgroup: the tile's
// four 16-row groups (K rows 0-15, K 16-31, V 0-15, V 16-31) go to waves
// w % 4, and wave w issues copies [(w / 4) * kPerWave, + kPerWave) of its
// group's COPIES_PER_GROUP wave-wide copies.
template <int D, int NW>
struct PipeCopies {
    static_assert(NW == 4 || NW == 8, "four or eight waves per workgroup");
    static_assert(TileCfg<D>::kWaves == 4, "four 16-row copy groups per tile");
    static constexpr int kPerWave = TileCfg<D>::COPIES_PER_GROUP * 4 / NW;
    static_assert(kPerWave >= 1, "at least one copy per wave");
};

// The four LDS buffers of the ring; tile t lives in b[t % 4].
struct PipeBuffers {
    char* b[kPipeBufs];
};

// V^T operands of one key tile (two transposing LDS reads each), read ahead
// of the MFMAs that use them.  Operand layout as pv_tile.
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

// Per-wave constants: the driver's WaveCtx plus the tiles of the pipelined
// step and the lane's V read offsets.
template <int D>
struct PipeCtx {
    WaveCtx cx;
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

// O^T += V^T P^T with the V^T operands already in registers (same MFMA order
// as pv_tile).
template <int D>
__device__ __forceinline__ void pv_tile_regs(WaveState<D>& ws, const bf16x2 (&pk)[TileCfg<D>::KBLK][8],
                                             const VOperands<D>& va)
{
    using C = TileCfg<D>;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x8 b = cat8(pk[kb][4 * h + 0], pk[kb][4 * h + 1], pk[kb][4 * h + 2], pk[kb][4 * h + 3]);
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db) ws.o[db] = mfma32(va.a[kb][h][db], b, ws.o[db]);
        }
}

// Instruction order of a pipelined step (scheduling groups; mask bits: 0x2
// VALU, 0x8 MFMA, 0x20 global load, 0x100 LDS read): the K reads first, then
// each S MFMA of the next tile with a share of the V^T reads and exponential
// work of this tile, the copies of a later tile, then each P V MFMA with
// maximum work of the next tile.
template <int D, int NW>
__device__ __forceinline__ void schedule_pipelined_step()
{
    using C = TileCfg<D>;
    constexpr int kKReads = C::KBLK * C::KSTEPS;
    constexpr int kVReads = C::KBLK * 2 * 2 * C::DBLK;
    constexpr int kMfma = C::KBLK * C::KSTEPS;     // S MFMAs (as many P V MFMAs)
    constexpr int kVPerMfma = (kVReads + kMfma - 1) / kMfma;
    __builtin_amdgcn_sched_group_barrier(0x100, kKReads, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kVPerMfma, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x020, PipeCopies<D, NW>::kPerWave, 0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
    }
}

// This wave's copies of one tile into `buf` (K at byte 0, V at TILE_BYTES;
// copy group w % 4: K group w % 4 below GROUPS, V group w % 4 - GROUPS
// above) from a contiguous [N, d] head slab.  The buffer descriptor starts at
// the group's first row (clamped to N) and covers the rest of the slab, so
// each lane's offset is the loop-invariant cx.voff plus a wave-uniform step
// per copy, and the range check (which covers that per-lane offset) returns
// zero for rows at or past N -- keys that the mask removes (p = 0), whose K
// and V values never matter.  Branch-free and free of per-lane arithmetic,
// which keeps a step's copies in the same scheduling region as its LDS reads
// and MFMAs.
template <int D, int NW, class KV>
__device__ __forceinline__ void issue_tile_copies_flat(const KV& kv, const WaveCtx& cx, char* buf, int key_base)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using C = TileCfg<D>;
    constexpr int CPW = PipeCopies<D, NW>::kPerWave;
    const int cw = cx.w & 3;
    const int i0 = (NW == 4) ? 0 : (cx.w >> 2) * CPW;
    const bool is_v = cw >= C::GROUPS;
    const int grp = is_v ? cw - C::GROUPS : cw;
    const int gkey = min(key_base + 16 * grp, cx.kv_end);   // uniform, <= N
    const uint32_t skip = (uint32_t)gkey * C::ROW_BYTES;     // < N * ROW_BYTES + 1 <= slab bytes + 1
    const char* base = (is_v ? kv.v_group(0, cx.kv_end) : kv.k_group(0, cx.kv_end)) + skip;
    const __amdgpu_buffer_rsrc_t r = raw_rsrc(base, kv.group_bytes() - skip);
    char* dst = buf + (is_v ? C::TILE_BYTES : 0) + grp * 16 * C::ROW_BYTES;
    const uint32_t step = is_v ? kVDmaStep : kKDmaStep;
    dst += i0 * 1024;
#pragma unroll
    for (int k = 0; k < CPW; ++k)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ATTN_LDS(dst + k * 1024), 16, cx.voff + (i0 + k) * step, 0, 0,
                                                 0);
#endif
}

// This wave's copies of one tile from a paged pool: the 16 rows of a group
// lie in one page (groups are 16-aligned, pages hold 16 or 32 tokens), whose
// table entry `page` the caller looked up for the group's first key clamped to
// kv_end - 1.  Rows at or past kv_end are fetched from row kv_end - 1 (valid
// data that the mask removes), so no copy reads outside the context; when the
// whole group lies past kv_end every row is that row, in the page looked up.
// K and V differ only in which lane fetches which row and 16-byte chunk (the
// layouts of k_dma_row / v_dma_row), so both go through the same branch-free code.
// CPOL: the copies' cache policy (0, or kCopyStream for K/V read once).
template <int D, int NW, int BS, int CPOL>
__device__ __forceinline__ void issue_tile_copies_paged(const char* kbase, const char* vbase, int64_t blk_bytes,
                                                        const WaveCtx& cx, char* buf, int key_base, int page)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using C = TileCfg<D>;
    constexpr int CPW = PipeCopies<D, NW>::kPerWave;
    const int cw = cx.w & 3;
    const int i0 = (NW == 4) ? 0 : (cx.w >> 2) * CPW;
    const bool is_v = cw >= C::GROUPS;
    const int grp = is_v ? cw - C::GROUPS : cw;
    const int gkey = key_base + 16 * grp;
    const int last = cx.kv_end - 1;
    const int64_t pg = __builtin_amdgcn_readfirstlane(page);
    const __amdgpu_buffer_rsrc_t r = raw_rsrc((is_v ? vbase : kbase) + pg * blk_bytes, (uint32_t)(BS * D * 2));
    char* dst = buf + (is_v ? C::TILE_BYTES : 0) + grp * 16 * C::ROW_BYTES + i0 * 1024;
    // K: lane l -> row l % 16, chunk 4 i + l / 16 (copy i steps 64 bytes);
    // V: lane l -> row i * ROWS_PER_DMA + l / KCPR, chunk as v_dma_col
    const int rstep = is_v ? C::ROWS_PER_DMA : 0;
    const uint32_t cstep = is_v ? 0u : kKDmaStep;
    const int lrow = (is_v ? v_dma_row<D>(cx.lane) : k_dma_row<D>(cx.lane)) + gkey + i0 * rstep;
    const uint32_t lcol = (is_v ? v_dma_col<D>(cx.lane) : k_dma_col<D>(cx.lane)) + i0 * cstep;
#pragma unroll
    for (int k = 0; k < CPW; ++k) {
        const int row = min(lrow + k * rstep, last) & (BS - 1);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ATTN_LDS(dst + k * 1024), 16,
                                                 (uint32_t)row * C::ROW_BYTES + lcol, k * cstep, 0, CPOL);
    }
#endif
}

// Copy protocol of the ring: the copies of tiles 0 and 1 are issued before
// the loop, and the step that publishes tile t issues the copies of tile
// t + 2 (into the buffer of tile t - 2, which every wave is done with once it
// has passed the barrier that publishes t), whether or not tile t + 2 exists.
// So at every publish exactly two tiles' copies are in flight, and waiting
// until one tile's worth remains means tile t has landed.
template <int D, int NW>
__device__ __forceinline__ void publish_tile()
{
    constexpr int CPW = PipeCopies<D, NW>::kPerWave;
    static_assert(CPW < 16, "vmcnt field");
    // The empty asm statements keep the compiler from moving memory accesses
    // across the barrier (s_barrier alone is not a memory operation to it);
    // unlike a workgroup fence they add no wait for the copies in flight.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x3f70 | CPW);   // vmcnt(one tile's copies)
    __builtin_amdgcn_s_waitcnt(0xc07f);                                  // lgkmcnt(0): this wave's LDS reads done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Pipelined step for tile j (in buffer I), whose scores Scur and offset
// update are done: publish tile j + 1, S of tile j + 1 into Snxt, p of tile
// j, O += P V of tile j, maximum and offset update of tile j + 1, and the
// copies of tile j + 3 (the window covers them).  Tile j + 1 is a full tile
// (j + 1 < nf4).
template <int D, int NW, int I, class KV>
__device__ __forceinline__ void pipe_step_next(WaveState<D>& ws, TileScores<D>& Scur, TileScores<D>& Snxt,
                                               const bf16x8 (&qf)[TileCfg<D>::KSTEPS], const KV& kv,
                                               const typename KV::SrcWin& win, const PipeCtx<D>& pc,
                                               const PipeBuffers& buf, int j)
{
    using C = TileCfg<D>;
    constexpr int IN = (I + 1) % kPipeBufs;
    const int copy_key = pc.cx.kv_begin + (j + 3) * C::BN;
    publish_tile<D, NW>();   // tile j + 1
    const int src = kv.copy_src(win, pc.cx, copy_key);
    qk_tile(Snxt, qf, buf.b[IN], pc.cx.lane);
    VOperands<D> va;
    read_v_tile(va, buf.b[I] + C::TILE_BYTES, pc.vro);
    kv.template copy_tile<NW>(pc.cx, buf.b[(I + 3) % kPipeBufs], copy_key, src);
    bf16x2 pk[C::KBLK][8];
    exp_tile(pk, Scur, ws, pc.cx.c2);
    pv_tile_regs(ws, pk, va);
    const float mt = tile_max<D, false>(Snxt, pc.cx.lane, pc.cx.kv_begin + (j + 1) * C::BN, pc.cx.q_lim);
    schedule_pipelined_step<D, NW>();
    update_offset(ws, mt, pc.cx.c2, pc.cx.thr);
}

// Last pipelined step (tile j = nf4 - 1): p and O += P V of tile j only.
template <int D, int I>
__device__ __forceinline__ void pipe_step_last(WaveState<D>& ws, TileScores<D>& Scur, const PipeCtx<D>& pc,
                                               const PipeBuffers& buf)
{
    using C = TileCfg<D>;
    VOperands<D> va;
    read_v_tile(va, buf.b[I] + C::TILE_BYTES, pc.vro);
    bf16x2 pk[C::KBLK][8];
    exp_tile(pk, Scur, ws, pc.cx.c2);
    pv_tile_regs(ws, pk, va);
}

// Plain step for tile t (in buffer I) with the causal / tail mask: publish it,
// S, mask and maximum, offset update, p, O += P V.
template <int D, int NW, int I, class KV>
__device__ __forceinline__ void pipe_step_masked(WaveState<D>& ws, const bf16x8 (&qf)[TileCfg<D>::KSTEPS],
                                                 const KV& kv, typename KV::SrcWin& win, const PipeCtx<D>& pc,
                                                 const PipeBuffers& buf, int t)
{
    using C = TileCfg<D>;
    const int copy_key = pc.cx.kv_begin + (t + 2) * C::BN;
    kv.win_update(win, pc.cx, copy_key, copy_key + C::BN - 1);
    publish_tile<D, NW>();   // tile t
    const int src = kv.copy_src(win, pc.cx, copy_key);
    TileScores<D> S;
    qk_tile(S, qf, buf.b[I], pc.cx.lane);
    kv.template copy_tile<NW>(pc.cx, buf.b[(I + 2) % kPipeBufs], copy_key, src);
    const float mt = tile_max<D, true>(S, pc.cx.lane, pc.cx.kv_begin + t * C::BN, pc.cx.q_lim);
    update_offset(ws, mt, pc.cx.c2, pc.cx.thr);
    VOperands<D> va;
    read_v_tile(va, buf.b[I] + C::TILE_BYTES, pc.vro);
    bf16x2 pk[C::KBLK][8];
    exp_tile(pk, S, ws, pc.cx.c2);
    pv_tile_regs(ws, pk, va);
}

// This wave's copies of the tile at key_base into buf, outside the
// pipelined steps.
template <int D, int NW, class KV>
__device__ __forceinline__ void pipe_copies(const KV& kv, typename KV::SrcWin& win, const WaveCtx& cx, char* buf,
                                            int key_base)
{
    kv.win_update(win, cx, key_base, key_base + TileCfg<D>::BN - 1);
    kv.template copy_tile<NW>(cx, buf, key_base, kv.copy_src(win, cx, key_base));
}

// The key loop of one wave (copy protocol above).
template <int D, int NW, class KV>
__device__ __forceinline__ void pipe_key_loop(WaveState<D>& ws, const bf16x8 (&qf)[TileCfg<D>::KSTEPS], const KV& kv,
                                              const PipeCtx<D>& pc, const PipeBuffers& buf)
{
    using C = TileCfg<D>;
    const int ntile = pc.cx.ntile, nf4 = pc.nf4;
    typename KV::SrcWin win = kv.empty_win();
    pipe_copies<D, NW>(kv, win, pc.cx, buf.b[0], pc.cx.kv_begin);
    pipe_copies<D, NW>(kv, win, pc.cx, buf.b[1], pc.cx.kv_begin + C::BN);
    if (nf4 > 0) {
        // prologue: publish tile 0, its scores, maximum and offset
        publish_tile<D, NW>();
        TileScores<D> Sa, Sb;
        qk_tile(Sa, qf, buf.b[0], pc.cx.lane);
        pipe_copies<D, NW>(kv, win, pc.cx, buf.b[2], pc.cx.kv_begin + 2 * C::BN);
        update_offset(ws, tile_max<D, false>(Sa, pc.cx.lane, pc.cx.kv_begin, pc.cx.q_lim), pc.cx.c2, pc.cx.thr);
        // tiles j .. j + 3 in buffers 0 .. 3; scores alternate Sa / Sb; the
        // four steps copy tiles j + 3 .. j + 6
        int j = 0;
        for (; j + 4 < nf4; j += 4) {
            kv.win_update(win, pc.cx, pc.cx.kv_begin + (j + 3) * C::BN, pc.cx.kv_begin + (j + 7) * C::BN - 1);
            pipe_step_next<D, NW, 0>(ws, Sa, Sb, qf, kv, win, pc, buf, j);
            pipe_step_next<D, NW, 1>(ws, Sb, Sa, qf, kv, win, pc, buf, j + 1);
            pipe_step_next<D, NW, 2>(ws, Sa, Sb, qf, kv, win, pc, buf, j + 2);
            pipe_step_next<D, NW, 3>(ws, Sb, Sa, qf, kv, win, pc, buf, j + 3);
        }
        // last group of four: tile nf4 - 1 has no pipelined successor
        kv.win_update(win, pc.cx, pc.cx.kv_begin + (j + 3) * C::BN, pc.cx.kv_begin + (j + 6) * C::BN - 1);
        pipe_step_next<D, NW, 0>(ws, Sa, Sb, qf, kv, win, pc, buf, j);
        pipe_step_next<D, NW, 1>(ws, Sb, Sa, qf, kv, win, pc, buf, j + 1);
        pipe_step_next<D, NW, 2>(ws, Sa, Sb, qf, kv, win, pc, buf, j + 2);
        pipe_step_last<D, 3>(ws, Sb, pc, buf);
    }
    // masked tiles, from a multiple of four: static buffer indices again
    for (int t = nf4; t < ntile; t += 4) {
        pipe_step_masked<D, NW, 0>(ws, qf, kv, win, pc, buf, t);
        if (t + 1 < ntile) pipe_step_masked<D, NW, 1>(ws, qf, kv, win, pc, buf, t + 1);
        if (t + 2 < ntile) pipe_step_masked<D, NW, 2>(ws, qf, kv, win, pc, buf, t + 2);
        if (t + 3 < ntile) pipe_step_masked<D, NW, 3>(ws, qf, kv, win, pc, buf, t + 3);
    }
    // the last two tiles' copies (past the context) may still be in flight:
    // drain them before the workgroup's LDS can be handed on
    __builtin_amdgcn_s_waitcnt(0x3f70);
}

// The loop of a wave with no valid query row: it takes part in the copies and
// the barriers of pipe_key_loop only.  Every wave of the workgroup publishes
// tile t (t = 0 .. ntile - 1) at one barrier and issues its copies of tile
// t + 2 right after it, the copies of tiles 0 and 1 before the first.
template <int D, int NW, class KV>
__device__ __forceinline__ void pipe_copy_loop(const KV& kv, const PipeCtx<D>& pc, const PipeBuffers& buf)
{
    using C = TileCfg<D>;
    const int ntile = pc.cx.ntile;
    typename KV::SrcWin win = kv.empty_win();
    pipe_copies<D, NW>(kv, win, pc.cx, buf.b[0], pc.cx.kv_begin);
    pipe_copies<D, NW>(kv, win, pc.cx, buf.b[1], pc.cx.kv_begin + C::BN);
    for (int t = 0; t < ntile; t += 4) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (t + i < ntile) {
                publish_tile<D, NW>();
                pipe_copies<D, NW>(kv, win, pc.cx, buf.b[(i + 2) % kPipeBufs], pc.cx.kv_begin + (t + i + 2) * C::BN);
            }
        }
    }
    __builtin_amdgcn_s_waitcnt(0x3f70);
}

// One query tile of 32 * NW rows: Q fragments, the key loop, and the epilogue
// (O / l and the log-sum-exp of the valid rows).  Waves with valid rows
// compute (rows past n_rows run on zero queries and are never stored); waves
// past the last valid row (the tail of a short tile, e.g. the few rows of a
// decode step on grouped heads) only copy.  The key tiles the
// workgroup runs are those its last row needs, and the full ones those its
// first row sees in full: rows of a later 128-row block may see more keys of
// a masked tile (the mask keeps exactly what each row sees), and a key tile
// wholly masked for a row adds exactly nothing to it, so a row gets the same
// bits in either tile size.
template <int D, int NW, class KV>
__device__ __forceinline__ void run_pipe_tile(const TileProblem& P, const KV& kv, const TileOut& out, float c2_in,
                                              const PipeBuffers& buf)
{
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    PipeCtx<D> pc;
    bf16x8 qf[TileCfg<D>::KSTEPS];
    int n_full = 0;
    pc.cx.ntile = init_query_tile<D>(P, pc.cx, qf, c2_in, w, &n_full);
    pc.cx.kv_begin = P.kv_begin;
    pc.cx.kv_end = P.kv_end;
    pc.cx.voff = copy_voff<D>(w & 3, pc.cx.lane);
    pc.nf4 = n_full & ~3;
    v_read_offsets<D>(pc.vro, pc.cx.lane);
    if (w * 32 >= P.n_rows) {
        pipe_copy_loop<D, NW>(kv, pc, buf);
        return;
    }
    WaveState<D> ws;
    clear_state(ws);
    pipe_key_loop<D, NW>(ws, qf, kv, pc, buf);
    store_query_rows(ws, P, out, pc.cx);
}

}  // namespace attn
