// attn_mfma_pipe.h -- the bf16 MFMA attention forward with a software-pipelined
// key loop: 32 query rows per wave, four waves per workgroup, every K/V tile
// staged in LDS once for the workgroup's 128 rows.
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
//  * ~200 registers per wave: two workgroups (two waves per SIMD) per CU.
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
template <int D>
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
    __builtin_amdgcn_sched_group_barrier(0x020, C::COPIES_PER_GROUP, 0);
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
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

// Pipelined step for tile j (in buffer I), whose scores Scur and offset
// update are done: publish tile j + 1, S of tile j + 1 into Snxt, p of tile
// j, O += P V of tile j, maximum and offset update of tile j + 1.  Tile j + 1
// is a full tile (j + 1 < nf4).
template <int D, int I, class KV>
__device__ __forceinline__ void pipe_step_next(WaveState<D>& ws, TileScores<D>& Scur, TileScores<D>& Snxt,
                                               const bf16x8 (&qf)[TileCfg<D>::KSTEPS], const KV& kv,
                                               const PipeCtx<D>& pc, const PipeBuffers& buf, int j)
{
    using C = TileCfg<D>;
    constexpr int IN = (I + 1) % kPipeBufs;
    publish_tile<D>();   // tile j + 1
    qk_tile(Snxt, qf, buf.b[IN], pc.cx.lane);
    VOperands<D> va;
    read_v_tile(va, buf.b[I] + C::TILE_BYTES, pc.vro);
    issue_tile_copies_flat<D>(kv, pc.cx, buf.b[(I + 3) % kPipeBufs], pc.cx.kv_begin + (j + 3) * C::BN);
    bf16x2 pk[C::KBLK][8];
    exp_tile(pk, Scur, ws, pc.cx.c2);
    pv_tile_regs(ws, pk, va);
    const float mt = tile_max<D, false>(Snxt, pc.cx.lane, pc.cx.kv_begin + (j + 1) * C::BN, pc.cx.q_lim);
    schedule_pipelined_step<D>();
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
template <int D, int I, class KV>
__device__ __forceinline__ void pipe_step_masked(WaveState<D>& ws, const bf16x8 (&qf)[TileCfg<D>::KSTEPS],
                                                 const KV& kv, const PipeCtx<D>& pc, const PipeBuffers& buf, int t)
{
    using C = TileCfg<D>;
    publish_tile<D>();   // tile t
    TileScores<D> S;
    qk_tile(S, qf, buf.b[I], pc.cx.lane);
    issue_tile_copies_flat<D>(kv, pc.cx, buf.b[(I + 2) % kPipeBufs], pc.cx.kv_begin + (t + 2) * C::BN);
    const float mt = tile_max<D, true>(S, pc.cx.lane, pc.cx.kv_begin + t * C::BN, pc.cx.q_lim);
    update_offset(ws, mt, pc.cx.c2, pc.cx.thr);
    VOperands<D> va;
    read_v_tile(va, buf.b[I] + C::TILE_BYTES, pc.vro);
    bf16x2 pk[C::KBLK][8];
    exp_tile(pk, S, ws, pc.cx.c2);
    pv_tile_regs(ws, pk, va);
}

// The key loop of one wave (copy protocol above).
template <int D, class KV>
__device__ __forceinline__ void pipe_key_loop(WaveState<D>& ws, const bf16x8 (&qf)[TileCfg<D>::KSTEPS], const KV& kv,
                                              const PipeCtx<D>& pc, const PipeBuffers& buf)
{
    using C = TileCfg<D>;
    const int ntile = pc.cx.ntile, nf4 = pc.nf4;
    issue_tile_copies_flat<D>(kv, pc.cx, buf.b[0], pc.cx.kv_begin);
    issue_tile_copies_flat<D>(kv, pc.cx, buf.b[1], pc.cx.kv_begin + C::BN);
    if (nf4 > 0) {
        // prologue: publish tile 0, its scores, maximum and offset
        publish_tile<D>();
        TileScores<D> Sa, Sb;
        qk_tile(Sa, qf, buf.b[0], pc.cx.lane);
        issue_tile_copies_flat<D>(kv, pc.cx, buf.b[2], pc.cx.kv_begin + 2 * C::BN);
        update_offset(ws, tile_max<D, false>(Sa, pc.cx.lane, pc.cx.kv_begin, pc.cx.q_lim), pc.cx.c2, pc.cx.thr);
        // tiles j .. j + 3 in buffers 0 .. 3; scores alternate Sa / Sb
        int j = 0;
        for (; j + 4 < nf4; j += 4) {
            pipe_step_next<D, 0>(ws, Sa, Sb, qf, kv, pc, buf, j);
            pipe_step_next<D, 1>(ws, Sb, Sa, qf, kv, pc, buf, j + 1);
            pipe_step_next<D, 2>(ws, Sa, Sb, qf, kv, pc, buf, j + 2);
            pipe_step_next<D, 3>(ws, Sb, Sa, qf, kv, pc, buf, j + 3);
        }
        // last group of four: tile nf4 - 1 has no pipelined successor
        pipe_step_next<D, 0>(ws, Sa, Sb, qf, kv, pc, buf, j);
        pipe_step_next<D, 1>(ws, Sb, Sa, qf, kv, pc, buf, j + 1);
        pipe_step_next<D, 2>(ws, Sa, Sb, qf, kv, pc, buf, j + 2);
        pipe_step_last<D, 3>(ws, Sb, pc, buf);
    }
    // masked tiles, from a multiple of four: static buffer indices again
    for (int t = nf4; t < ntile; t += 4) {
        pipe_step_masked<D, 0>(ws, qf, kv, pc, buf, t);
        if (t + 1 < ntile) pipe_step_masked<D, 1>(ws, qf, kv, pc, buf, t + 1);
        if (t + 2 < ntile) pipe_step_masked<D, 2>(ws, qf, kv, pc, buf, t + 2);
        if (t + 3 < ntile) pipe_step_masked<D, 3>(ws, qf, kv, pc, buf, t + 3);
    }
    // the last two tiles' copies (past the context) may still be in flight:
    // drain them before the workgroup's LDS can be handed on
    __builtin_amdgcn_s_waitcnt(0x3f70);
}

// One 128-row query tile: Q fragments, the key loop, and the epilogue (O / l
// and the log-sum-exp of the valid rows).  Every wave computes (rows past
// n_rows run on zero queries and are never stored).
template <int D, class KV>
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
    pc.cx.voff = copy_voff<D>(w, pc.cx.lane);
    pc.nf4 = n_full & ~3;
    v_read_offsets<D>(pc.vro, pc.cx.lane);
    WaveState<D> ws;
    clear_state(ws);
    pipe_key_loop<D>(ws, qf, kv, pc, buf);
    store_query_rows(ws, P, out, pc.cx);
}

}  // namespace attn
