// bwd_gfx950.hip -- backward of the fused causal/dense attention for gfx950
// (bf16 inputs, fp32 accumulation, bf16 gradients).
//
// "Flash Attention and Paged Attention" (section 2) keeps only O and the
// softmax normalisation statistics from the forward, so that the backward
// recomputes S and P tile by tile instead of reading an N x N matrix back.
// With the saved LSE the recomputed P = exp(scale q.k - LSE) is final for
// every tile on its own (no running maximum), and the gradients follow from
// the chain rule through the forward's three steps (section 1):
//   dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),  D_i = dO_i . O_i,
//   dQ = scale dS K,  dK = scale dS^T Q.
// (D_i = sum_j P_ij dP_ij because O_i = sum_j P_ij V_j.)
//
// Two kernels, both deterministic: every output element is accumulated by
// one lane in a fixed order, with no atomics.
//   bwd_dq_kernel    one workgroup per (batch, head, 128-query tile).  First
//                    writes (LSE log2 e, D) of its rows to the workspace, then
//                    streams 32-key K/V tiles through LDS as the forward does,
//                    recomputes S^T and dP^T and accumulates dQ^T += K^T dS^T.
//   bwd_dkdv_kernel  one workgroup of 8 waves per (batch, K/V head, 128-key
//                    block); 32-query tiles of Q, dO and the rows' (LSE log2 e,
//                    D), for every query head of the K/V head's group, stream
//                    through LDS.  Each 32-key block has two waves: the P wave
//                    (its keys' K in registers) computes S and P, passes P on
//                    through LDS and accumulates dV^T += dO^T P; the dS wave
//                    (V in registers), one query tile behind, computes dP,
//                    then dS = P (dP - D), and accumulates dK^T += Q^T dS.
// Computing dQ apart from dK/dV costs a second recomputation of S and dP (7
// matrix products per (query tile, key tile) pair instead of 5) and saves a
// float atomic read-modify-write of dQ for every such pair.
//
// MFMA layout (v_mfma_f32_32x32x16_bf16, one lane per output column):
//  * dQ kernel: S^T = K Q^T and dP^T = V dO^T put one query per lane (its Q
//    and dO fragments stay in registers, as Q does in the forward); dS^T is
//    the B operand of dQ^T += K^T dS^T straight from the accumulators, and
//    K^T comes from transposing LDS reads of the K tile.
//  * dK/dV kernel: S = Q K^T (P wave) and dP = dO V^T (dS wave) put one key
//    per lane (K or V fragments in registers); P and dS are the B operands of
//    dV^T += dO^T P and dK^T += Q^T dS, and dO^T, Q^T come from transposing
//    reads.
// Every streamed tile is read both ways -- MFMA row reads (16 consecutive
// rows at one 16-byte chunk) and transposing reads (4 consecutive rows x 4
// consecutive chunks) -- so tiles are stored row-major with an XOR swizzle of
// the chunk index that keeps both patterns free of LDS bank conflicts
// (dual_xor).  Tiles are copied global -> LDS directly (buffer loads to LDS,
// no registers) one tile ahead, one barrier per tile: into two buffers in
// the dQ kernel, three in the dK/dV kernel (whose dS waves read a tile one
// step after the P waves).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "attn_mfma_core.h"
#include "bwd_internal.h"
#include "attn_internal.h"

namespace attn {

namespace {


template <int D>
struct BwdCfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BT = 32;                     // rows per streamed tile
    static constexpr int BLK = 32 * kWaves;           // stationary rows per workgroup
    static constexpr int KCPR = D / 8;                // 16-byte chunks per row
    static constexpr int KSTEPS = D / 16;             // MFMA k-steps over the head dimension
    static constexpr int DBLK = D / 32;               // 32-wide blocks of the head dimension
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int TILE_BYTES = BT * ROW_BYTES;
    static constexpr int RPD = 1024 / ROW_BYTES;      // rows per wave-wide 16 B/lane copy
    static constexpr int COPIES = TILE_BYTES / 1024;  // wave-wide copies per tile
};

// XOR applied to the 16-byte chunk index of tile row `row`, chosen so that
//  (a) 16 consecutive 16-aligned rows at one logical chunk (an MFMA row read
//      by 16 lanes) fall on 16 distinct 16-byte bank groups, and
//  (b) 4 consecutive 4-aligned rows x 4 consecutive 4-aligned chunks (one
//      32-lane pass of a transposing read) fall on 16 distinct bank groups.
// D = 128: a row spans all 64 banks; xor = 4 (row & 3) + ((row >> 2) & 3).
// D = 64: two rows share a 256-byte bank window (row & 1 picks the half);
//         xor = 4 ((row >> 1) & 1) + ((row >> 2) & 3).
template <int D>
__device__ __forceinline__ uint32_t dual_xor(uint32_t row)
{
    return (D == 128) ? (((row & 3u) << 2) | ((row >> 2) & 3u)) : ((((row >> 1) & 1u) << 2) | ((row >> 2) & 3u));
}

template <int D>
__device__ __forceinline__ uint32_t dual_ofs(uint32_t row, uint32_t chunk)
{
    return row * (uint32_t)BwdCfg<D>::ROW_BYTES + ((chunk ^ dual_xor<D>(row)) << 4);
}

// Lane addressing of the transposing reads: lane (16-lane group G, i = lane
// % 16, half g = lane / 32) reads row 4g + i/4 (+16h per half-tile), the 4
// channels starting at 16 (G % 2) + 4 (i % 4) of the 32-channel block, so it
// receives channel 16 (G % 2) + i over rows 16h + 4g + {0..3, 8..11} -- the
// rows (keys or queries) that its accumulator registers 8h .. 8h + 7 hold.
__device__ __forceinline__ int tr_row_of(int lane) { return (lane >> 5) * 4 + ((lane & 15) >> 2); }
__device__ __forceinline__ uint32_t tr_col_of(int lane)
{
    return (uint32_t)((((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2);
}

// Per-lane byte offsets of every LDS read a tile step makes, relative to the
// tile (computed once per kernel).  The swizzle only looks at row bits 0..3,
// so tile row r32 + 32 sb and row tr_row + 16 h + 32 sb share the offsets of
// rows r32 and tr_row plus (32 sb + 16 h) * ROW_BYTES, which, like the tile's
// own position in LDS, goes into the read's immediate offset: no address
// arithmetic is left inside the loop.
template <int D>
struct LaneOfs {
    uint32_t row[BwdCfg<D>::KSTEPS];    // MFMA row reads: row r32, chunk 2 ks + g
    uint32_t tlo[BwdCfg<D>::DBLK];      // transposing reads: row tr_row, d-block db
    uint32_t thi[BwdCfg<D>::DBLK];      //                    row tr_row + 8
};

template <int D>
__device__ __forceinline__ LaneOfs<D> lane_offsets(int lane)
{
    LaneOfs<D> o;
    const int g = lane >> 5, r32 = lane & 31;
    const int tr_row = tr_row_of(lane);
    const uint32_t tr_col = tr_col_of(lane);
#pragma unroll
    for (int ks = 0; ks < BwdCfg<D>::KSTEPS; ++ks) o.row[ks] = dual_ofs<D>((uint32_t)r32, (uint32_t)(ks * 2 + g));
#pragma unroll
    for (int db = 0; db < BwdCfg<D>::DBLK; ++db) {
        const uint32_t col = tr_col + db * 64;
        o.tlo[db] = dual_ofs<D>((uint32_t)tr_row, col >> 4) + (col & 15u);
        o.thi[db] = dual_ofs<D>((uint32_t)tr_row + 8u, col >> 4) + (col & 15u);
    }
    return o;
}

__device__ __forceinline__ bf16x8 lds_row(const char* p)
{
    return as_bf16x8(*(const u32x4*)p);
}

__device__ __forceinline__ bf16x8 lds_tr(const char* lo, const char* hi)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)lo);
    const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)hi);
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Linear work id after the XCD-contiguous remap (workgroups are dealt to the
// 8 XCDs round-robin; the grid is padded to a multiple of 8): consecutive
// ids, i.e. the tiles of one head, share one XCD's L2.
__device__ __forceinline__ int xcd_linear_id(int bid, int grid)
{
    const int per = grid >> 3;
    return (bid & 7) * per + (bid >> 3);
}

__device__ __forceinline__ void publish_copies()
{
    __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this wave's copies have landed
    __syncthreads();
}

#if defined(__HIP_DEVICE_COMPILE__)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}

// Copies pieces c0 .. c0 + NC - 1 of the BT-row tile starting at row row0 of
// a row-major [n_rows][D] slab into `tile` in the dual layout; rows at or
// past n_rows are fetched from row n_rows - 1 (valid data, masked later).
// Piece c holds tile rows c * RPD .. c * RPD + RPD - 1: lane l lands at row
// c * RPD + l / KCPR, physical chunk l % KCPR, which holds logical chunk
// (l % KCPR) ^ dual_xor(row).
template <int D, int NC>
__device__ __forceinline__ void copy_tile(__amdgpu_buffer_rsrc_t r, char* tile, int row0, int n_rows, int c0,
                                          int lane)
{
    using C = BwdCfg<D>;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = c0 + i;
        const uint32_t row = (uint32_t)(c * C::RPD + lane / C::KCPR);
        const uint32_t src = (uint32_t)min(row0 + (int)row, n_rows - 1);
        const uint32_t voff = src * (uint32_t)C::ROW_BYTES + ((((uint32_t)lane % C::KCPR) ^ dual_xor<D>(row)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ATTN_LDS(tile + c * 1024), 16, voff, 0, 0, 0);
    }
}

#endif

// Runs tiles [tb, te) of a stream of nt tiles double-buffered in b0 / b1
// (tile t lives in buffer t % 2), all with one step variant.  On entry tile
// tb has been published; each step is preceded by the copies of the next
// tile into the other buffer and followed by "wait for my copies, barrier",
// which publishes that tile and frees the one just read.  The buffers are
// chosen statically (the loop is unrolled by two, with an odd first tile
// peeled), so LDS reads of one buffer are never ordered behind copies in
// flight into the other.
template <class Issue, class Step>
__device__ __forceinline__ void run_tiles(char* b0, char* b1, int tb, int te, int nt, const Issue& issue,
                                          const Step& step)
{
    int t = tb;
    if ((t & 1) && t < te) {
        if (t + 1 < nt) issue(b0, t + 1);
        step(b1, t);
        publish_copies();
        ++t;
    }
    for (; t + 2 <= te; t += 2) {
        issue(b1, t + 1);
        step(b0, t);
        publish_copies();
        if (t + 2 < nt) issue(b0, t + 2);
        step(b1, t + 1);
        publish_copies();
    }
    if (t < te) {
        if (t + 1 < nt) issue(b1, t + 1);
        step(b0, t);
        publish_copies();
    }
}

// Runs tiles [tb, te) of a stream of nt tiles in three buffers (tile t lives
// in buffer t % 3) for the two wave roles of the dK/dV kernel: the step of
// tile t issues the copies of tile t + 1 (into the buffer of tile t - 2,
// which both roles were done with at the last barrier), runs p(t) (the P
// waves) and d(t - 1) (the dS waves, one tile behind, reading the P the P
// waves left in the previous step), and ends with "wait for my copies,
// barrier", which publishes tile t + 1 and this step's P.  One barrier per
// tile.  On entry tile tb has been published.  Buffers are chosen
// statically (unrolled by three, the first tiles peeled to a multiple of
// three), so LDS reads of one buffer are never ordered behind copies in
// flight into another.
template <class Issue, class PStep, class DStep>
__device__ __forceinline__ void run_tiles_lag(char* b0, char* b1, char* b2, int tb, int te, int nt,
                                              const Issue& issue, const PStep& p, const DStep& d)
{
    const auto one = [&](char* bc, char* bp, char* bn, int t) {
        if (t + 1 < nt) issue(bn, t + 1);
        p(bc, t);
        if (t > 0) d(bp, t - 1);
        publish_copies();
    };
    int t = tb;
    if (t < te && t % 3 == 1) one(b1, b0, b2, t++);
    if (t < te && t % 3 == 2) one(b2, b1, b0, t++);
    for (; t + 3 <= te; t += 3) {
        one(b0, b2, b1, t);
        one(b1, b0, b2, t + 1);
        one(b2, b1, b0, t + 2);
    }
    if (t < te) one(b0, b2, b1, t++);
    if (t < te) one(b1, b0, b2, t++);
}

// ---------------------------------------------------------------------------
// dQ: one 32-key tile (K at buf, V at buf + TILE_BYTES) for this wave's 32
// queries.  Lane: query (lane % 32) with lse2 = its LSE * log2 e and dd = D;
// accumulator register i of S^T / dP^T holds key key0 + (i/4)*8 + 4g + i%4.
// MASKED: keys >= q_lim get P = 0.
template <int D, bool MASKED>
__device__ __forceinline__ void dq_tile(f32x16 (&dq)[BwdCfg<D>::DBLK], const bf16x8 (&qf)[BwdCfg<D>::KSTEPS],
                                        const bf16x8 (&df)[BwdCfg<D>::KSTEPS], float lse2, float dd, const char* buf,
                                        const LaneOfs<D>& lo, int lane, float c2, int key0, int q_lim)
{
    using C = BwdCfg<D>;
    const char* tk = buf;
    const char* tv = buf + C::TILE_BYTES;
    const int g = lane >> 5;
    // stages fenced as in the dK/dV kernel: row reads, then the S / dP
    // MFMAs, then the transposing K reads (ahead of the exponentials), then
    // the dQ MFMAs
    f32x16 s = f32x16{}, dp = f32x16{};
    {
        bf16x8 kf[C::KSTEPS], vf[C::KSTEPS];
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            kf[ks] = lds_row(tk + lo.row[ks]);
            vf[ks] = lds_row(tv + lo.row[ks]);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            s = mfma32(kf[ks], qf[ks], s);
            dp = mfma32(vf[ks], df[ks], dp);
        }
    }
    bf16x8 kt[2][C::DBLK];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const char* th = tk + 16 * h * C::ROW_BYTES;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) kt[h][db] = lds_tr(th + lo.tlo[db], th + lo.thi[db]);
    }
    __builtin_amdgcn_sched_barrier(0);
    bf16x2 dsk[8];
    const int lim_rel = q_lim - key0 - 4 * g;
#pragma unroll
    for (int i = 0; i < 16; i += 2) {
        float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, -lse2));
        float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i + 1], c2, -lse2));
        if (MASKED) {
            const int off = (i >> 2) * 8 + (i & 3);
            p0 = (off < lim_rel) ? p0 : 0.f;
            p1 = (off + 1 < lim_rel) ? p1 : 0.f;
        }
        dsk[i >> 1] = pack2(p0 * (dp[i] - dd), p1 * (dp[i + 1] - dd));
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const bf16x8 b = cat8(dsk[4 * h + 0], dsk[4 * h + 1], dsk[4 * h + 2], dsk[4 * h + 3]);
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) dq[db] = mfma32(kt[h][db], b, dq[db]);
    }
}

// dQ of one 128-query tile starting at q0 of head bh (the body of
// bwd_dq_kernel; a paired workgroup runs it for two tiles).
template <int D>
__device__ __forceinline__ void dq_query_tile(const BwdArgs& a, int bh, int q0, char* lds0, char* lds1)
{
    using C = BwdCfg<D>;
    const int N = a.N;
    const int G = a.H / a.H_kv;
    const int64_t head_off = (int64_t)bh * N * C::ROW_BYTES;
    const int64_t kv_off = ((int64_t)(bh / a.H) * a.H_kv + (bh % a.H) / G) * N * C::ROW_BYTES;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = lane >> 5, r32 = lane & 31;
    const int qi = q0 + 32 * w + r32;                       // this lane's query
    const bool valid = qi < N;
    const float c2 = fmaxf(a.scale * kLog2e, 1e-30f);

    // ---- Q and dO fragments (channels 16 ks + 8 g .. + 7), D = dO . O ----------
    bf16x8 qf[C::KSTEPS], df[C::KSTEPS];
    float dpart = 0.f;
    {
        const int64_t row = head_off + (int64_t)qi * C::ROW_BYTES;
        const char* qp = (const char*)a.q + row;
        const char* dp = (const char*)a.dout + row;
        const char* op = (const char*)a.o + row;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u}, z = {0u, 0u, 0u, 0u};
            if (valid) {
                x = *(const u32x4*)(qp + (ks * 2 + g) * 16);
                y = *(const u32x4*)(dp + (ks * 2 + g) * 16);
                z = *(const u32x4*)(op + (ks * 2 + g) * 16);
            }
            qf[ks] = as_bf16x8(x);
            df[ks] = as_bf16x8(y);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dpart = __builtin_fmaf(bf16lo(y[e]), bf16lo(z[e]), dpart);
                dpart = __builtin_fmaf(bf16hi(y[e]), bf16hi(z[e]), dpart);
            }
        }
    }
    const float dd = half_sum(dpart);
    float lse2 = INFINITY;                                  // rows past N: P = 0
    if (valid) {
        const float l = a.lse[(int64_t)bh * N + qi];
        lse2 = (l == -INFINITY) ? INFINITY : l * kLog2e;    // a row with no key has P = 0
        if (g == 0) {                                       // planar: lse2 of the head's rows, then D
            a.ws[(int64_t)bh * N * 2 + qi] = lse2;
            a.ws[(int64_t)bh * N * 2 + N + qi] = dd;
        }
    }

    // ---- key loop -------------------------------------------------------------
    f32x16 dq[C::DBLK];
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) dq[db] = f32x16{};
    const int kend = a.causal ? min(N, q0 + C::BLK) : N;    // keys this tile needs
    const int nt = (kend + C::BT - 1) / C::BT;
    const int q_lim = a.causal ? min(N, qi + 1) : N;
    const int sel = w >> 1;                                 // waves 0, 1 copy K; 2, 3 copy V
    const int c0 = (w & 1) * (C::COPIES / 2);
    // Tiles [0, n_full) are seen in full by every query of the tile (keys
    // below its first query, all inside the context); the rest (diagonal and
    // a ragged tail) are masked, for every wave: a tile wholly above a wave's
    // queries adds exactly nothing (P = 0).  Waves with no valid query only
    // take part in the copies and barriers.
    const int n_full = a.causal ? min(nt, q0 / C::BT) : N / C::BT;
    auto issue = [&](char* buf, int t) {
#if defined(__HIP_DEVICE_COMPILE__)
        const char* src = (const char*)(sel ? a.v : a.k) + kv_off;
        copy_tile<D, C::COPIES / 2>(raw_rsrc(src, (uint32_t)N * C::ROW_BYTES), buf + sel * C::TILE_BYTES, t * C::BT,
                                    N, c0, lane);
#endif
    };
    const LaneOfs<D> lo = lane_offsets<D>(lane);
    auto full = [&](const char* buf, int t) {
        dq_tile<D, false>(dq, qf, df, lse2, dd, buf, lo, lane, c2, t * C::BT, q_lim);
    };
    auto masked = [&](const char* buf, int t) {
        dq_tile<D, true>(dq, qf, df, lse2, dd, buf, lo, lane, c2, t * C::BT, q_lim);
    };
    auto none = [&](const char*, int) {};
    if (nt > 0) {
        issue(lds0, 0);
        publish_copies();
    }
    if (q0 + 32 * w < N) {
        run_tiles(lds0, lds1, 0, n_full, nt, issue, full);
        run_tiles(lds0, lds1, n_full, nt, nt, issue, masked);
    } else {
        run_tiles(lds0, lds1, 0, nt, nt, issue, none);
    }

    // ---- dQ = scale * dQ^T, bf16 ----------------------------------------------
    if (valid) {
        char* orow = (char*)a.dq + head_off + (int64_t)qi * C::ROW_BYTES;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                u32x2 w2;
                w2[0] = pack_bf16(dq[db][r * 4 + 0] * a.scale, dq[db][r * 4 + 1] * a.scale);
                w2[1] = pack_bf16(dq[db][r * 4 + 2] * a.scale, dq[db][r * 4 + 3] * a.scale);
                *(u32x2*)(orow + (db * 32 + r * 8 + g * 4) * 2) = w2;
            }
    }
}

// One workgroup per (b, h, 128-query tile), heaviest tile first within a
// head, or (PAIR, causal launches) per pair of tiles t and nqt-1-t, so that
// every workgroup does the same number of key tiles.
template <int D, bool PAIR>
__global__ __launch_bounds__(256, 2) void bwd_dq_kernel(BwdArgs a, int n_work)
{
    using C = BwdCfg<D>;
    __shared__ __attribute__((aligned(16))) char lds0[2 * C::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char lds1[2 * C::TILE_BYTES];
    const int L = xcd_linear_id(blockIdx.x, gridDim.x);
    if (L >= n_work) return;
    const int nqt = (a.N + C::BLK - 1) / C::BLK;
    const int per_bh = PAIR ? (nqt + 1) / 2 : nqt;
    const int bh = L / per_bh, t = L % per_bh;
    dq_query_tile<D>(a, bh, (nqt - 1 - t) * C::BLK, lds0, lds1);   // heaviest (most keys) first
    if (PAIR && t != nqt - 1 - t) {
        __syncthreads();   // LDS reuse across the two tiles
        dq_query_tile<D>(a, bh, t * C::BLK, lds0, lds1);
    }
}

// ---------------------------------------------------------------------------
// dK, dV with two wave roles per 32-key block.  A workgroup of 8 waves owns
// 128 keys; wave k (0..3) is the P wave of keys k0 + 32k .. + 31 and wave
// 4 + k its dS wave (the hardware puts both on SIMD k).  With one wave per
// key block holding K, V, dK and dV (~350 registers) only one wave fits a
// SIMD and nothing hides its exponentials; split in two, two waves fit.
// Per 32-query tile t:
//   P wave : S = Q K^T, P = exp2(s c2 - lse2) (masked), P to an LDS exchange
//            slot (bf16), dV^T += dO^T P
//   dS wave, one tile behind (tile t - 1, whose P the barrier ending the
//            previous step published): dP = dO V^T, dS = P (dP - D),
//            dK^T += Q^T dS
// so a tile step has one barrier (three tile buffers and two exchange slots;
// run_tiles_lag), and the two waves of a SIMD never wait for each other
// inside it.  Each wave holds half the stationary state (K or V, dV or dK),
// which leaves room for two waves per SIMD: one's exponentials or dS run
// beside the other's MFMAs.  The workspace rows are planar here: lse2 of a
// head's N rows, then D of its N rows.
constexpr int kRoleKB = 4;                     // 32-key blocks per workgroup
constexpr int kRoleWaves = 2 * kRoleKB;

#if defined(__HIP_DEVICE_COMPILE__)
// lse2 (lanes 0..31) and D (lanes 32..63) of rows row0 .. row0 + 31, clamped.
__device__ __forceinline__ void copy_rowstats(__amdgpu_buffer_rsrc_t r, char* dst, int row0, int n_rows, int lane)
{
    const uint32_t row = (uint32_t)min(row0 + (lane & 31), n_rows - 1);
    const uint32_t off = ((lane >> 5) ? (uint32_t)n_rows * 4u : 0u) + row * 4u;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, ATTN_LDS(dst), 4, off, 0, 0, 0);
}
#endif

template <int D>
struct RoleCfg {
    static constexpr int TILE_BYTES = 32 * BwdCfg<D>::ROW_BYTES;   // 32 rows of Q or of dO
    static constexpr int COPIES = TILE_BYTES / 1024;
    static constexpr int STAT_BYTES = 256;                          // lse2[32], D[32]
    static constexpr int BUF_BYTES = 2 * TILE_BYTES + STAT_BYTES;
    static constexpr int XCH_BYTES = 64 * 32;                       // P of one key block: 16 bf16 per lane
};

// P wave, one tile: S = Q K^T, P to its exchange slot in LDS (read by the
// dS wave one step later, after the barrier that ends this step), then
// dV^T += dO^T P.
template <int D, bool MASKED>
__device__ __forceinline__ void role_p_tile(f32x16 (&dv)[BwdCfg<D>::DBLK], const bf16x8 (&kf)[BwdCfg<D>::KSTEPS],
                                            const char* buf, char* xch, const LaneOfs<D>& lo, int lane, float c2,
                                            int q0, int key, int n, int causal)
{
    using C = BwdCfg<D>;
    using R = RoleCfg<D>;
    const char* tq = buf;
    const char* td = buf + R::TILE_BYTES;
    const float* st = (const float*)(buf + 2 * R::TILE_BYTES);
    const int g = lane >> 5;
    f32x16 s = f32x16{};
    {
        bf16x8 x[C::KSTEPS];
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) x[ks] = lds_row(tq + lo.row[ks]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) s = mfma32(x[ks], kf[ks], s);
    }
    bf16x8 tdo[2][C::DBLK];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db)
            tdo[h][db] = lds_tr(td + 16 * h * C::ROW_BYTES + lo.tlo[db], td + 16 * h * C::ROW_BYTES + lo.thi[db]);
    f32x4 l2[4];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) l2[a4] = *(const f32x4*)(st + a4 * 8 + 4 * g);
    __builtin_amdgcn_sched_barrier(0);
    bf16x2 pk[8];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
        float p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float pj = __builtin_amdgcn_exp2f(__builtin_fmaf(s[4 * a4 + j], c2, -l2[a4][j]));
            if (MASKED) {
                const int qq = q0 + a4 * 8 + 4 * g + j;
                pj = (qq < n && (!causal || key <= qq)) ? pj : 0.f;
            }
            p[j] = pj;
        }
        pk[2 * a4] = pack2(p[0], p[1]);
        pk[2 * a4 + 1] = pack2(p[2], p[3]);
    }
    *(bf16x8*)(xch + lane * 32) = cat8(pk[0], pk[1], pk[2], pk[3]);
    *(bf16x8*)(xch + lane * 32 + 16) = cat8(pk[4], pk[5], pk[6], pk[7]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const bf16x8 bp = cat8(pk[4 * h + 0], pk[4 * h + 1], pk[4 * h + 2], pk[4 * h + 3]);
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) dv[db] = mfma32(tdo[h][db], bp, dv[db]);
    }
}

// dS wave, one tile (the tile the P wave took one step earlier, whose P is
// in xch): dP = dO V^T, dS = P (dP - D), dK^T += Q^T dS.
template <int D>
__device__ __forceinline__ void role_ds_tile(f32x16 (&dk)[BwdCfg<D>::DBLK], const bf16x8 (&vf)[BwdCfg<D>::KSTEPS],
                                             const char* buf, const char* xch, const LaneOfs<D>& lo, int lane)
{
    using C = BwdCfg<D>;
    using R = RoleCfg<D>;
    const char* tq = buf;
    const char* td = buf + R::TILE_BYTES;
    const float* st = (const float*)(buf + 2 * R::TILE_BYTES);
    const int g = lane >> 5;
    f32x16 dp = f32x16{};
    {
        bf16x8 y[C::KSTEPS];
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) y[ks] = lds_row(td + lo.row[ks]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) dp = mfma32(y[ks], vf[ks], dp);
    }
    bf16x8 tqo[2][C::DBLK];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db)
            tqo[h][db] = lds_tr(tq + 16 * h * C::ROW_BYTES + lo.tlo[db], tq + 16 * h * C::ROW_BYTES + lo.thi[db]);
    f32x4 dd[4];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) dd[a4] = *(const f32x4*)(st + 32 + a4 * 8 + 4 * g);
    __builtin_amdgcn_sched_barrier(0);
    const u32x4 p0 = *(const u32x4*)(xch + lane * 32);
    const u32x4 p1 = *(const u32x4*)(xch + lane * 32 + 16);
    const uint32_t pw[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
    bf16x2 dsk[8];
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
        float ds[4];
#pragma unroll
        for (int j = 0; j < 4; j += 2) {
            const uint32_t w2 = pw[2 * a4 + j / 2];
            ds[j] = bf16lo(w2) * (dp[4 * a4 + j] - dd[a4][j]);
            ds[j + 1] = bf16hi(w2) * (dp[4 * a4 + j + 1] - dd[a4][j + 1]);
        }
        dsk[2 * a4] = pack2(ds[0], ds[1]);
        dsk[2 * a4 + 1] = pack2(ds[2], ds[3]);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const bf16x8 bs = cat8(dsk[4 * h + 0], dsk[4 * h + 1], dsk[4 * h + 2], dsk[4 * h + 3]);
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) dk[db] = mfma32(tqo[h][db], bs, dk[db]);
    }
}

// dK, dV of one key block of BLK keys starting at k0 of K/V head bhk (the
// body of bwd_dkdv_kernel; a paired workgroup runs it for two blocks).
template <int D>
__device__ __forceinline__ void dkdv_key_block(const BwdArgs& a, int bhk, int k0, char* lds0, char* lds1,
                                               char* lds2, char* xch_all)
{
    using C = BwdCfg<D>;
    using R = RoleCfg<D>;
    constexpr int KB = kRoleKB, BLK = 32 * KB;
    const int N = a.N;
    const int b = bhk / a.H_kv, hk = bhk % a.H_kv;
    const int G = a.H / a.H_kv;
    const int64_t kv_off = (int64_t)bhk * N * C::ROW_BYTES;
    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int kb = w % KB;                                  // key block of this wave
    const bool p_role = w < KB;
    const int g = lane >> 5, r32 = lane & 31;
    const int key = k0 + 32 * kb + r32;                     // this lane's key
    const bool kvalid = key < N;
    const float c2 = fmaxf(a.scale * kLog2e, 1e-30f);
    // P of tile t goes to exchange slot t % 2
    const auto xch = [&](int t) { return xch_all + ((t & 1) * KB + kb) * R::XCH_BYTES; };

    // K (P wave) or V (dS wave) fragments of the lane's key
    bf16x8 kvf[C::KSTEPS];
    {
        const char* src = (const char*)(p_role ? a.k : a.v) + kv_off + (int64_t)key * C::ROW_BYTES;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (kvalid) x = *(const u32x4*)(src + (ks * 2 + g) * 16);
            kvf[ks] = as_bf16x8(x);
        }
    }
    f32x16 acc[C::DBLK];                                    // dV (P wave) or dK (dS wave)
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) acc[db] = f32x16{};

    const int qt0 = a.causal ? k0 / 32 : 0;
    const int nqt = (N + 31) / 32;
    const int per_head = nqt - qt0;
    const int nt = G * per_head;
    const int sel = w / KB;                                 // P waves copy Q, dS waves copy dO
    const int c0 = (w % KB) * (R::COPIES / KB);
    auto issue = [&](char* buf, int t) {
#if defined(__HIP_DEVICE_COMPILE__)
        const int gh = t / per_head, qt = qt0 + t % per_head;
        const int64_t bh = (int64_t)b * a.H + hk * G + gh;
        const char* src = (const char*)(sel ? a.dout : a.q) + bh * N * C::ROW_BYTES;
        copy_tile<D, R::COPIES / KB>(raw_rsrc(src, (uint32_t)N * C::ROW_BYTES), buf + sel * R::TILE_BYTES, qt * 32,
                                     N, c0, lane);
        if (w == 0)
            copy_rowstats(raw_rsrc(a.ws + bh * N * 2, (uint32_t)N * 8u), buf + 2 * R::TILE_BYTES, qt * 32, N, lane);
#endif
    };
    auto q_of = [&](int t) { return (qt0 + t % per_head) * 32; };
    const LaneOfs<D> lo = lane_offsets<D>(lane);
    auto p_full = [&](const char* buf, int t) {
        role_p_tile<D, false>(acc, kvf, buf, xch(t), lo, lane, c2, q_of(t), key, N, a.causal);
    };
    auto p_masked = [&](const char* buf, int t) {
        role_p_tile<D, true>(acc, kvf, buf, xch(t), lo, lane, c2, q_of(t), key, N, a.causal);
    };
    auto ds_step = [&](const char* buf, int t) { role_ds_tile<D>(acc, kvf, buf, xch(t), lo, lane); };
    auto none = [&](const char*, int) {};
    const int n_head_masked = a.causal ? min(KB, per_head) : 0;
    const int n_tail_masked = (N % 32 != 0 && per_head - 1 >= n_head_masked) ? 1 : 0;
    if (nt > 0) {
        issue(lds0, 0);
        publish_copies();
    }
    if (k0 + 32 * kb >= N) {
        run_tiles_lag(lds0, lds1, lds2, 0, nt, nt, issue, none, none);
    } else if (p_role) {
        for (int gh = 0; gh < G; ++gh) {
            const int tb = gh * per_head;
            run_tiles_lag(lds0, lds1, lds2, tb, tb + n_head_masked, nt, issue, p_masked, none);
            run_tiles_lag(lds0, lds1, lds2, tb + n_head_masked, tb + per_head - n_tail_masked, nt, issue, p_full,
                          none);
            run_tiles_lag(lds0, lds1, lds2, tb + per_head - n_tail_masked, tb + per_head, nt, issue, p_masked,
                          none);
        }
    } else {
        run_tiles_lag(lds0, lds1, lds2, 0, nt, nt, issue, none, ds_step);
        // the last tile's dS step (its P was published by the last barrier;
        // no copies are in flight and nothing overwrites its buffer)
        if (nt > 0) {
            const int t = nt - 1;
            if (t % 3 == 0) ds_step(lds0, t);
            else if (t % 3 == 1) ds_step(lds1, t);
            else ds_step(lds2, t);
        }
    }

    if (kvalid) {
        char* row = (char*)(p_role ? a.dv : a.dk) + kv_off + (int64_t)key * C::ROW_BYTES;
        const float f = p_role ? 1.f : a.scale;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                u32x2 w2;
                w2[0] = pack_bf16(acc[db][r * 4 + 0] * f, acc[db][r * 4 + 1] * f);
                w2[1] = pack_bf16(acc[db][r * 4 + 2] * f, acc[db][r * 4 + 3] * f);
                *(u32x2*)(row + (db * 32 + r * 8 + g * 4) * 2) = w2;
            }
    }
}

// One workgroup per (b, K/V head, key block of BLK keys), the block with the
// most query tiles first, or (PAIR, causal launches) per pair of blocks kb
// and nkb-1-kb, so that every workgroup sees the same number of query tiles.
template <int D, bool PAIR>
__global__ __launch_bounds__(64 * kRoleWaves, 1) void bwd_dkdv_kernel(BwdArgs a, int n_work)
{
    using R = RoleCfg<D>;
    constexpr int KB = kRoleKB, BLK = 32 * KB;
    __shared__ __attribute__((aligned(16))) char lds0[R::BUF_BYTES];
    __shared__ __attribute__((aligned(16))) char lds1[R::BUF_BYTES];
    __shared__ __attribute__((aligned(16))) char lds2[R::BUF_BYTES];
    __shared__ __attribute__((aligned(16))) char xch_all[2 * KB * R::XCH_BYTES];
    const int L = xcd_linear_id(blockIdx.x, gridDim.x);
    if (L >= n_work) return;
    const int nkb = (a.N + BLK - 1) / BLK;
    const int per = PAIR ? (nkb + 1) / 2 : nkb;
    const int bhk = L / per, t = L % per;
    dkdv_key_block<D>(a, bhk, t * BLK, lds0, lds1, lds2, xch_all);
    if (PAIR && t != nkb - 1 - t) {
        __syncthreads();   // LDS reuse across the two blocks
        dkdv_key_block<D>(a, bhk, (nkb - 1 - t) * BLK, lds0, lds1, lds2, xch_all);
    }
}

}  // namespace

int launch_bwd(const BwdArgs& a, hipStream_t stream)
{
    constexpr int BLK = 128;
    const int64_t nblk = (a.N + BLK - 1) / BLK;
    // causal launches pair the dQ kernel's query tiles (t, nqt-1-t) and the
    // dK/dV kernel's key blocks (kb, nkb-1-kb); a.pair_q / a.pair_kv force it
    const bool pair = (a.pair_q < 0 ? a.causal != 0 : a.pair_q != 0) && nblk > 1;
    const int64_t n_dq = (int64_t)a.B * a.H * (pair ? (nblk + 1) / 2 : nblk);
    const int64_t nkb = (a.N + 32 * kRoleKB - 1) / (32 * kRoleKB);
    const bool pair_kv = (a.pair_kv < 0 ? a.causal != 0 : a.pair_kv != 0) && nkb > 1;
    const int64_t n_kv = (int64_t)a.B * a.H_kv * (pair_kv ? (nkb + 1) / 2 : nkb);
    if (!grid_fits((n_dq + 7) / 8 * 8, BwdCfg<128>::kThreads) || !grid_fits((n_kv + 7) / 8 * 8, 64 * kRoleWaves))
        return -2;
    const int grid_dq = (int)((n_dq + 7) / 8 * 8);
    const int grid_kv = (int)((n_kv + 7) / 8 * 8);
    if (a.d == 128) {
        if (pair)
            hipLaunchKernelGGL((bwd_dq_kernel<128, true>), dim3(grid_dq), dim3(BwdCfg<128>::kThreads), 0, stream, a,
                               (int)n_dq);
        else
            hipLaunchKernelGGL((bwd_dq_kernel<128, false>), dim3(grid_dq), dim3(BwdCfg<128>::kThreads), 0, stream, a,
                               (int)n_dq);
        if (pair_kv)
            hipLaunchKernelGGL((bwd_dkdv_kernel<128, true>), dim3(grid_kv), dim3(64 * kRoleWaves), 0, stream, a,
                               (int)n_kv);
        else
            hipLaunchKernelGGL((bwd_dkdv_kernel<128, false>), dim3(grid_kv), dim3(64 * kRoleWaves), 0, stream, a,
                               (int)n_kv);
    } else {
        if (pair)
            hipLaunchKernelGGL((bwd_dq_kernel<64, true>), dim3(grid_dq), dim3(BwdCfg<64>::kThreads), 0, stream, a,
                               (int)n_dq);
        else
            hipLaunchKernelGGL((bwd_dq_kernel<64, false>), dim3(grid_dq), dim3(BwdCfg<64>::kThreads), 0, stream, a,
                               (int)n_dq);
        if (pair_kv)
            hipLaunchKernelGGL((bwd_dkdv_kernel<64, true>), dim3(grid_kv), dim3(64 * kRoleWaves), 0, stream, a,
                               (int)n_kv);
        else
            hipLaunchKernelGGL((bwd_dkdv_kernel<64, false>), dim3(grid_kv), dim3(64 * kRoleWaves), 0, stream, a,
                               (int)n_kv);
    }
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace attn
