// attn_mfma_kernel.h -- the per-workgroup driver of the bf16 MFMA attention
// forward: loads the query tile into registers, streams 32-key K/V tiles into
// LDS with direct global->LDS copies (one barrier per tile; each tile's
// copies go out after the S MFMAs of an earlier tile), runs the
// online-softmax tile step of attn_mfma_core.h, and writes O (bf16, or fp32
// partials) and the log-sum-exp.  The source of K/V rows is a policy object,
// so the same driver serves contiguous K/V ([B,H,N,d]) and the paged pool.
// Two copy schedules, chosen by the source's kCopiesAhead:
//   2: three LDS buffers, copies two tiles ahead (contiguous K/V);
//   1: two LDS buffers, copies one tile ahead (the paged pool, where copies
//      two tiles ahead were measured to fetch ~1.8x the pool bytes from
//      memory, against 1.14x, and to run no faster).
//
// K/V source policy interface (all members device functions):
//   static constexpr int kCopiesAhead (1 or 2, above)
//   for kCopiesAhead == 2 (the copy helpers are in attn_mfma_pipe.h, whose
//   key loop uses the same members):
//     SrcWin, SrcWin empty_win()
//         a small per-wave state that locates the rows of a range of keys.
//     void win_update(SrcWin&, const WaveCtx&, int key_lo, int key_hi)
//         make the state cover the copies of keys [key_lo, key_hi].
//     int copy_src(const SrcWin&, const WaveCtx&, int key_base)
//         what this wave's copies of the tile at key_base need.
//     template <int NW> void copy_tile(const WaveCtx&, char* buf, int key_base, int src)
//         this wave's share (of NW waves) of the branch-free copies of the
//         tile at key_base into buf: K at byte 0, V at TILE_BYTES, in the
//         layouts of attn_mfma_core.h.  Rows at or past kv_end hold data
//         that the mask removes; no copy reads outside the K/V allocation.
//   for kCopiesAhead == 1:
//     const char* k_group(int key, int kv_end) / v_group(...)
//         wave-uniform base address of the 16-row group holding key
//         min(key, kv_end - 1); rows of one group are contiguous (ROW_BYTES
//         apart) in memory, which holds for any page of 16 or 32 tokens
//         (groups are 16-aligned).
//     int group_row(int key, int kv_end)
//         row of key min(key, kv_end - 1) relative to that group base.
//     uint32_t group_bytes()
//         bytes addressable from a group base (range of the copy descriptor).
#pragma once

#include <type_traits>

#include "attn_mfma_core.h"

namespace attn {

// One query tile's problem, resolved per workgroup.  Tile row t is query
// position t / rows_per_pos and, within it, head t % rows_per_pos: the rows
// of the query heads that share one K/V head (grouped-query attention) sit
// side by side, so each K/V tile staged in LDS serves all of them.  With one
// row per position it is an ordinary query tile of one head.
struct TileProblem {
    const char* q;       // query row 0 of the tile (bytes)
    int64_t q_stride;    // bytes between query positions
    int64_t q_hstride;   // bytes between the heads of one position
    int rows_per_pos;    // heads per position in the tile (>= 1)
    int n_rows;          // valid query rows in this tile
    int q_pos0;          // position of row 0: a row at position p may see keys
                         // < min(kv_end, q_pos0 + p + 1) when causal
    int causal;
    int kv_begin;        // keys [kv_begin, kv_end) are this workgroup's share
    int kv_end;
};

// Output writer: normalised bf16 rows, or fp32 rows + lse for split partials.
// Rows are addressed like the query rows (position, head).
struct TileOut {
    char* o;             // output row 0 of the tile (bytes)
    int64_t o_stride;    // bytes between positions
    int64_t o_hstride;   // bytes between heads of one position
    float* lse;          // lse of row 0 (may be null)
    int64_t lse_stride;  // floats between positions
    int64_t lse_hstride; // floats between heads of one position
    int fp32_out;        // 1: write fp32 normalised O (partials), 0: bf16
};

// Query rows per workgroup: 4 waves x 32 queries.
constexpr int kTileRows = 128;

// LDS of one workgroup: three buffers (two, b2 unused, for copies one tile
// ahead), each holding one K tile then one V tile.  They are distinct
// __shared__ objects, so reads of one are not ordered behind copies in
// flight into another.
struct TileBuffers {
    char* b0;
    char* b1;
    char* b2;
};

#if defined(__HIP_DEVICE_COMPILE__)
// Buffer resource for raw 16-byte loads of `bytes` bytes from `base`
// (data format 32, no swizzle); loads at offsets >= bytes return zero.
// (The resource type exists only for the device target.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const char* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
#endif

// Wave-level constants of one query tile.
struct WaveCtx {
    int lane, w;
    float c2, thr;
    int q_lim;           // this lane's query sees keys < q_lim
    int kv_begin, kv_end, ntile;
    uint32_t voff;       // this lane's copy source offset within a full group
};

// Issue this wave's copies of one tile into buffer `buf` (K tile at byte 0, V
// tile at TILE_BYTES): wave w < GROUPS copies K group w, the others V group
// w - GROUPS.  Rows at or past kv_end are fetched from row kv_end - 1 (valid
// data, masked out of S), so no copy reads outside the context.  For a full
// group the per-lane source offset is loop-invariant (cx.voff) and the
// group's position goes in the scalar offset.
template <int D, class KV>
__device__ __forceinline__ void issue_tile_copies(const KV& kv, const WaveCtx& cx, char* buf, int key_base)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using C = TileCfg<D>;
    const bool is_v = cx.w >= C::GROUPS;                      // uniform
    const int grp = is_v ? cx.w - C::GROUPS : cx.w;
    const int kv_end = cx.kv_end;
    const int gkey = key_base + 16 * grp;                     // first key of the group (uniform)
    const __amdgpu_buffer_rsrc_t r =
        raw_rsrc(is_v ? kv.v_group(gkey, kv_end) : kv.k_group(gkey, kv_end), kv.group_bytes());
    char* dst = buf + (is_v ? C::TILE_BYTES : 0) + grp * 16 * C::ROW_BYTES;
    if (__builtin_expect(gkey + 16 <= kv_end, 1)) {
        const uint32_t soff = (uint32_t)kv.group_row(gkey, kv_end) * C::ROW_BYTES;
        const uint32_t step = is_v ? kVDmaStep : kKDmaStep;
#pragma unroll
        for (int i = 0; i < C::COPIES_PER_GROUP; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ATTN_LDS(dst + i * 1024), 16, cx.voff + i * step, soff, 0,
                                                     0);
    } else if (!is_v) {
        const uint32_t koff = (uint32_t)kv.group_row(gkey + k_dma_row<D>(cx.lane), kv_end) * C::ROW_BYTES +
                              k_dma_col<D>(cx.lane);
#pragma unroll
        for (int i = 0; i < C::COPIES_PER_GROUP; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ATTN_LDS(dst + i * 1024), 16, koff + i * kKDmaStep, 0, 0, 0);
    } else {
        const uint32_t vcol = v_dma_col<D>(cx.lane);
#pragma unroll
        for (int i = 0; i < C::COPIES_PER_GROUP; ++i) {
            const int vrow = kv.group_row(gkey + i * C::ROWS_PER_DMA + v_dma_row<D>(cx.lane), kv_end);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ATTN_LDS(dst + i * 1024), 16,
                                                     (uint32_t)vrow * C::ROW_BYTES + vcol, 0, 0, 0);
        }
    }
#endif
}

// Copies one tile ahead: wait until this wave's copies have landed, then the
// barrier that publishes the tile.
__device__ __forceinline__ void publish_copies()
{
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0)
    __syncthreads();
}

// Wait until this wave's copies of the next tile have landed -- the copies
// of the tile after it, this wave's last COPIES_PER_GROUP vector-memory
// instructions, may still be in flight -- then the barrier that publishes it.
template <int D>
__device__ __forceinline__ void publish_copies_ahead()
{
    constexpr int CPG = TileCfg<D>::COPIES_PER_GROUP;
    static_assert(CPG < 16, "vmcnt field");
    // A workgroup fence would wait for every copy in flight; the empty asm
    // statements instead keep the compiler from moving memory accesses
    // across the barrier.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0x3f70 | CPG);   // vmcnt(CPG)
    __builtin_amdgcn_s_waitcnt(0xc07f);         // lgkmcnt(0): this wave's LDS reads done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// One key tile (K at buf, V at buf + TILE_BYTES) for this wave's 32 queries.
// `copies` issues this wave's share of the next tile's copies; it runs after
// the S MFMAs, whose K reads it would otherwise queue behind.
template <int D, bool MASKED, class CP>
__device__ __forceinline__ void tile_step(WaveState<D>& ws, const bf16x8 (&qf)[TileCfg<D>::KSTEPS], const WaveCtx& cx,
                                          const char* buf, int key0, const CP& copies)
{
    using C = TileCfg<D>;
    TileScores<D> S;
    qk_tile(S, qf, buf, cx.lane);
    copies();
    const float mt = tile_max<D, MASKED>(S, cx.lane, key0, cx.q_lim);
    update_offset(ws, mt, cx.c2, cx.thr);
    bf16x2 pk[C::KBLK][8];
    exp_tile(pk, S, ws, cx.c2);
    pv_tile(ws, pk, buf + C::TILE_BYTES, cx.lane);
}

// The key loops of one wave: tiles [0, n_full) unmasked, the rest masked.
// COMPUTE false: the wave only copies its share of every tile and joins the
// barriers (it has no valid query row).
//
// Copies two tiles ahead.  Tile j lives in buffer j % 3.  The step of tile
// j issues the copies of tile min(j + 2, nt - 1) (into the buffer of tile
// j - 1, which every wave was done with at the barrier that ended step
// j - 1; past the last tile it fetches the last tile again, out of L2,
// rather than keys beyond the causal limit), and ends with "wait until only
// those copies are in flight, barrier", which publishes tile j + 1: each
// tile's copies have a step and a half to land.  The copies are the K/V
// source's branch-free ones (copy_tile, its source looked up in a window
// updated once per three tiles), and the buffers are chosen statically
// (unrolled by three): with a branch in the copies, the compiler orders the
// next LDS reads behind every copy in flight.
template <int D, bool COMPUTE, class KV>
__device__ __forceinline__ void key_loop_ahead2(WaveState<D>& ws, const bf16x8 (&qf)[TileCfg<D>::KSTEPS],
                                                const WaveCtx& cx, const KV& kv, const TileBuffers& buf, int n_full)
{
    using C = TileCfg<D>;
    const int nt = cx.ntile;
    if (nt == 0) return;
    const int last_kb = cx.kv_begin + (nt - 1) * C::BN;
    typename KV::SrcWin win = kv.empty_win();
    const auto copy = [&](char* dst, int key_base) {
        kv.template copy_tile<C::kWaves>(cx, dst, key_base, kv.copy_src(win, cx, key_base));
    };
    // the window covers the copies of the three tiles from tile j on
    const auto cover = [&](int j) {
        j = min(j, nt - 1);
        kv.win_update(win, cx, cx.kv_begin + j * C::BN, cx.kv_begin + (j + 3) * C::BN - 1);
    };
    cover(0);
    copy(buf.b0, cx.kv_begin);
    copy(buf.b1, cx.kv_begin + C::BN);
    publish_copies_ahead<D>();
    // step of tile j in buffer cur; tile j + 2 goes to buffer nxt2
    const auto step = [&](auto masked, char* cur, char* nxt2, int j) {
        const int kb0 = cx.kv_begin + j * C::BN;
        const auto cp = [&]() { copy(nxt2, min(kb0 + 2 * C::BN, last_kb)); };
        if (COMPUTE) tile_step<D, decltype(masked)::value>(ws, qf, cx, cur, kb0, cp);
        else cp();
        publish_copies_ahead<D>();
    };
    using Full = std::false_type;
    using Masked = std::true_type;
    int j = 0;
    for (; j + 3 <= n_full; j += 3) {
        cover(j + 2);
        step(Full{}, buf.b0, buf.b2, j);
        step(Full{}, buf.b1, buf.b0, j + 1);
        step(Full{}, buf.b2, buf.b1, j + 2);
    }
    // j is a multiple of three here, so tile j is in buffer 0
    for (; j < nt; j += 3) {
        cover(j + 2);
        step(Masked{}, buf.b0, buf.b2, j);
        if (j + 1 < nt) step(Masked{}, buf.b1, buf.b0, j + 1);
        if (j + 2 < nt) step(Masked{}, buf.b2, buf.b1, j + 2);
    }
    // the copies past the last tile may still be in flight: drain them
    // before the workgroup's LDS can be handed on
    __builtin_amdgcn_s_waitcnt(0x3f70);
}

// Copies one tile ahead.  Tile j lives in buffer j % 2; its copies are
// issued while tile j - 1 is being consumed; "wait for my copies, then
// barrier" publishes it.
template <int D, bool COMPUTE, class KV>
__device__ __forceinline__ void key_loop_ahead1(WaveState<D>& ws, const bf16x8 (&qf)[TileCfg<D>::KSTEPS],
                                                const WaveCtx& cx, const KV& kv, const TileBuffers& buf, int n_full)
{
    using C = TileCfg<D>;
    if (cx.ntile > 0) {
        issue_tile_copies<D>(kv, cx, buf.b0, cx.kv_begin);
        publish_copies();
    }
    int j = 0;
    for (; j + 2 <= n_full; j += 2) {
        const int kb0 = cx.kv_begin + j * C::BN;
        const auto c1 = [&]() { issue_tile_copies<D>(kv, cx, buf.b1, kb0 + C::BN); };
        if (COMPUTE) tile_step<D, false>(ws, qf, cx, buf.b0, kb0, c1);
        else c1();
        publish_copies();
        const auto c2 = [&]() {
            if (j + 2 < cx.ntile) issue_tile_copies<D>(kv, cx, buf.b0, kb0 + 2 * C::BN);
        };
        if (COMPUTE) tile_step<D, false>(ws, qf, cx, buf.b1, kb0 + C::BN, c2);
        else c2();
        publish_copies();
    }
    // j is even here, so tile j is in buffer 0
    for (; j < cx.ntile; j += 2) {
        const int kb0 = cx.kv_begin + j * C::BN;
        const auto c1 = [&]() {
            if (j + 1 < cx.ntile) issue_tile_copies<D>(kv, cx, buf.b1, kb0 + C::BN);
        };
        if (COMPUTE) tile_step<D, true>(ws, qf, cx, buf.b0, kb0, c1);
        else c1();
        publish_copies();
        if (j + 1 < cx.ntile) {
            const auto c2 = [&]() {
                if (j + 2 < cx.ntile) issue_tile_copies<D>(kv, cx, buf.b0, kb0 + 2 * C::BN);
            };
            if (COMPUTE) tile_step<D, true>(ws, qf, cx, buf.b1, kb0 + C::BN, c2);
            else c2();
            publish_copies();
        }
    }
}

template <int D, bool COMPUTE, class KV>
__device__ __forceinline__ void key_loop(WaveState<D>& ws, const bf16x8 (&qf)[TileCfg<D>::KSTEPS], const WaveCtx& cx,
                                         const KV& kv, const TileBuffers& buf, int n_full)
{
    static_assert(KV::kCopiesAhead == 1 || KV::kCopiesAhead == 2, "copy schedule");
    if constexpr (KV::kCopiesAhead == 2) key_loop_ahead2<D, COMPUTE>(ws, qf, cx, kv, buf, n_full);
    else key_loop_ahead1<D, COMPUTE>(ws, qf, cx, kv, buf, n_full);
}

// Per-wave set-up of one query tile: the Q^T fragments of this lane's query,
// its key limit, and the key tiles the whole tile needs.  Returns the number
// of key tiles from P.kv_begin; *n_full receives how many of them every row
// of the tile sees in full (below the diagonal of its first row and before
// kv_end).  cx.kv_begin / kv_end / ntile / voff are left to the caller.
template <int D>
__device__ __forceinline__ int init_query_tile(const TileProblem& P, WaveCtx& cx, bf16x8 (&qf)[TileCfg<D>::KSTEPS],
                                               float c2_in, int w, int* n_full)
{
    using C = TileCfg<D>;
    // scale * log2(e); a zero scale becomes a tiny positive factor (every
    // allowed key still gets p = 2^0 = 1 exactly, masked keys 2^-inf = 0)
    cx.c2 = fmaxf(c2_in, 1e-30f);
    cx.thr = kRescaleLog2 / cx.c2;
    cx.lane = threadIdx.x & 63;
    cx.w = w;
    const int g = cx.lane >> 5, r32 = cx.lane & 31;
    const int qrow = w * 32 + r32;            // this lane's query row in the tile
    const int qpos = qrow / P.rows_per_pos, qhead = qrow % P.rows_per_pos;
    const int64_t qoff = qpos * P.q_stride + qhead * P.q_hstride;
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (qrow < P.n_rows) val = *(const u32x4*)(P.q + qoff + (ks * 2 + g) * 16);
        qf[ks] = as_bf16x8(val);
    }
    // rows past n_rows run on zero queries and are never stored
    cx.q_lim = P.causal ? min(P.kv_end, P.q_pos0 + qpos + 1) : P.kv_end;
    // keys the whole tile needs
    const int t_end =
        P.causal ? min(P.kv_end, P.q_pos0 + (max(P.n_rows, 1) - 1) / P.rows_per_pos + 1) : P.kv_end;
    const int ntile = (t_end > P.kv_begin) ? (t_end - P.kv_begin + C::BN - 1) / C::BN : 0;
    // Tiles [0, n_full) are seen in full by every row of the tile (below the
    // diagonal of query row 0 and before kv_end).  The rest (diagonal and
    // tail) go through the masked step, for every wave: a tile fully masked
    // for a lane adds exactly nothing (p = 0, and the offset only moves on a
    // finite score), and waves past the last valid row run on zero queries
    // and never store.  Keeping the per-tile code free of per-wave branches
    // also keeps O in one register set across the loop.
    int nf = 0;
    {
        const int lim = P.causal ? min(P.kv_end, P.q_pos0 + 1) : P.kv_end;
        if (lim > P.kv_begin) nf = min(ntile, (lim - P.kv_begin) / C::BN);
    }
    *n_full = nf;
    return ntile;
}

template <int D>
__device__ __forceinline__ uint32_t copy_voff(int w, int lane)
{
    using C = TileCfg<D>;
    return (w >= C::GROUPS) ? (uint32_t)v_dma_row<D>(lane) * C::ROW_BYTES + v_dma_col<D>(lane)
                            : (uint32_t)k_dma_row<D>(lane) * C::ROW_BYTES + k_dma_col<D>(lane);
}

template <int D>
__device__ __forceinline__ void clear_state(WaveState<D>& ws)
{
#pragma unroll
    for (int db = 0; db < TileCfg<D>::DBLK; ++db) ws.o[db] = f32x16{};
    ws.m = -INFINITY;
    ws.ms = 0.f;
    ws.l = 0.f;
}

// Epilogue of one wave: O / l (bf16, or fp32 partials) and the log-sum-exp
// of its valid rows.
template <int D>
__device__ __forceinline__ void store_query_rows(const WaveState<D>& ws, const TileProblem& P, const TileOut& out,
                                                 const WaveCtx& cx)
{
    using C = TileCfg<D>;
    const int g = cx.lane >> 5, r32 = cx.lane & 31;
    const int qrow = cx.w * 32 + r32;
    const int qpos = qrow / P.rows_per_pos, qhead = qrow % P.rows_per_pos;
    const float l_tot = half_sum(ws.l);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < P.n_rows) {
        if (out.fp32_out) {
            float* orow = (float*)(out.o + qpos * out.o_stride + qhead * out.o_hstride);
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    f32x4 v4;
                    v4[0] = ws.o[db][a * 4 + 0] * inv;
                    v4[1] = ws.o[db][a * 4 + 1] * inv;
                    v4[2] = ws.o[db][a * 4 + 2] * inv;
                    v4[3] = ws.o[db][a * 4 + 3] * inv;
                    *(f32x4*)(orow + db * 32 + a * 8 + g * 4) = v4;
                }
        } else {
            char* orow = out.o + qpos * out.o_stride + qhead * out.o_hstride;
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    u32x2 w2;
                    w2[0] = pack_bf16(ws.o[db][a * 4 + 0] * inv, ws.o[db][a * 4 + 1] * inv);
                    w2[1] = pack_bf16(ws.o[db][a * 4 + 2] * inv, ws.o[db][a * 4 + 3] * inv);
                    *(u32x2*)(orow + (db * 32 + a * 8 + g * 4) * 2) = w2;
                }
        }
        if (out.lse && g == 0) {
            out.lse[qpos * out.lse_stride + qhead * out.lse_hstride] =
                (l_tot > 0.f) ? (ws.ms + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

template <int D, class KV>
__device__ __forceinline__ void run_query_tile(const TileProblem& P, const KV& kv, const TileOut& out, float c2_in,
                                               const TileBuffers& buf)
{
    WaveCtx cx;
    bf16x8 qf[TileCfg<D>::KSTEPS];
    int n_full;
    cx.ntile = init_query_tile<D>(P, cx, qf, c2_in, __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), &n_full);
    cx.kv_begin = P.kv_begin;
    cx.kv_end = P.kv_end;
    cx.voff = copy_voff<D>(cx.w, cx.lane);
    WaveState<D> ws;
    clear_state(ws);
    // Waves with no valid row (the tail of a partial tile, or the rows past a
    // short grouped-query tile) only take part in the copies and barriers.
    if (cx.w * 32 < P.n_rows) key_loop<D, true>(ws, qf, cx, kv, buf, n_full);
    else key_loop<D, false>(ws, qf, cx, kv, buf, n_full);
    store_query_rows(ws, P, out, cx);
}

}  // namespace attn
