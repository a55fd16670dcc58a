// attn_mfma_kernel.h -- the per-workgroup driver of the bf16 MFMA attention
// forward: loads a 128-row query tile into registers, streams 64-key K/V
// tiles through LDS (global loads issued one tile ahead), runs the online
// softmax tile step of attn_mfma_core.h, and writes O (bf16, or fp32 partials)
// and the log-sum-exp.  The source of K/V rows is a policy object, so the same
// driver serves contiguous K/V ([B,H,N,d]) and the paged pool.
#pragma once

#include "attn_mfma_core.h"

namespace attn {

// One query tile's problem, resolved per workgroup.
struct TileProblem {
    const char* q;       // query row 0 of the tile (bytes)
    int64_t q_stride;    // bytes between query rows
    int n_rows;          // valid query rows in this tile (<= BM)
    int q_pos0;          // absolute key position of query row 0 minus nothing:
                         // row i may see keys < min(kv_end, q_pos0 + i + 1) when causal
    int causal;
    int kv_begin;        // keys [kv_begin, kv_end) are this workgroup's share
    int kv_end;
};

// Per-thread byte offsets of the rows this thread loads inside one K/V tile
// (identical for every tile).  K: load i covers tile rows [i*R, (i+1)*R) with
// R = 256 / (d/8) rows; thread tid takes row i*R + tid/(d/8), chunk tid%(d/8),
// so its offset is tid*16 + i*R*d*2.  V: keys vblock_quad(tid)*4 + 0..3,
// channels vblock_oct(tid)*8 .. +7.
template <int D>
struct TileOffsets {
    static constexpr int R = TileCfg<D>::kThreads / TileCfg<D>::KCPR;   // K rows per load
    uint32_t k0;      // tid * 16 (offset of load 0)
    int k_row0;       // tid / (d/8)
    int v_key;        // first key of this thread's V quad
    uint32_t v;       // v_key*D*2 + octet*16
    __device__ __forceinline__ TileOffsets(int tid)
    {
        k0 = (uint32_t)tid * 16u;
        k_row0 = tid / TileCfg<D>::KCPR;
        v_key = vblock_quad(tid) * 4;
        v = (uint32_t)(v_key * D * 2 + vblock_oct(tid) * 16);
    }
    __device__ __forceinline__ uint32_t k(int i) const { return k0 + (uint32_t)(i * R * D * 2); }
    __device__ __forceinline__ int k_row(int i) const { return k_row0 + i * R; }
};

// Zero the staged rows at or past kv_end (keys of the tail tile that do not
// exist, or belong to the next context split).
template <int D>
__device__ __forceinline__ void zero_tail(KVStage<D>& st, const TileOffsets<D>& off, int key_base, int kv_end,
                                          int tid)
{
    using C = TileCfg<D>;
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i)
        if (key_base + off.k_row(i) >= kv_end) st.k[i] = z;
    if (tid < C::V_QUADS) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
            if (key_base + off.v_key + r >= kv_end) st.v[r] = z;
    }
}

// Output writer: normalised bf16 rows, or fp32 rows + lse for split partials.
struct TileOut {
    char* o;             // output row 0 of the tile (bytes)
    int64_t o_stride;    // bytes between output rows
    float* lse;          // lse of row 0 (may be null)
    int64_t lse_stride;  // floats between rows
    int fp32_out;        // 1: write fp32 normalised O (partials), 0: bf16
};

template <int D, class KV>
__device__ __forceinline__ void run_query_tile(const TileProblem& P, const KV& kv, const TileOut& out, float c2_in,
                                               char* lds)
{
    // scale * log2(e); a zero scale becomes a tiny positive factor (every
    // allowed key still gets p = 2^0 = 1 exactly, masked keys 2^-inf = 0)
    const float c2 = fmaxf(c2_in, 1e-30f);
    using C = TileCfg<D>;
    const int tid = threadIdx.x;
    const int lane = tid & 63, w = tid >> 6, g = lane >> 5, r32 = lane & 31;

    // ---- Q^T fragments for this lane's query --------------------------------
    const int qrow = w * 32 + r32;
    bf16x8 qf[C::KSTEPS];
#pragma unroll
    for (int ks = 0; ks < C::KSTEPS; ++ks) {
        u32x4 val = {0u, 0u, 0u, 0u};
        if (qrow < P.n_rows) val = *(const u32x4*)(P.q + qrow * P.q_stride + (ks * 2 + g) * 16);
        qf[ks] = as_bf16x8(val);
    }
    // allowed keys for this lane's query: key < q_lim
    int q_lim = P.kv_end;
    if (P.causal) q_lim = min(q_lim, P.q_pos0 + qrow + 1);
    // bounds over the wave (rows past n_rows are never stored; they use the
    // last valid row's limit so they never widen the wave's key range)
    int wrow_lo = min(w * 32, max(P.n_rows - 1, 0));
    int wrow_hi = min(w * 32 + 31, max(P.n_rows - 1, 0));
    int w_lim_min = P.kv_end, w_lim_max = P.kv_end;
    if (P.causal) {
        w_lim_min = min(P.kv_end, P.q_pos0 + wrow_lo + 1);
        w_lim_max = min(P.kv_end, P.q_pos0 + wrow_hi + 1);
    }
    if (qrow >= P.n_rows) q_lim = w_lim_max;
    const bool wave_active = w * 32 < P.n_rows;   // waves past the last row only help load
    // keys the whole tile needs
    int t_end = P.kv_end;
    if (P.causal) t_end = min(P.kv_end, P.q_pos0 + P.n_rows);

    WaveState<D> ws;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) ws.o[db] = f32x16{};
    ws.m = -INFINITY;
    ws.l = 0.f;

    const float thr = kRescaleLog2 / c2;
    const TileOffsets<D> toff(tid);
    KVStage<D> st;
    // Two LDS buffers: while tile j is consumed from one, tile j+1 is written
    // into the other (its global loads were issued one tile earlier), so each
    // tile costs one barrier.
    const int ntile = (t_end > P.kv_begin) ? (t_end - P.kv_begin + C::BN - 1) / C::BN : 0;
    if (ntile > 0) {
        kv.load(st, toff, P.kv_begin, P.kv_end, tid);
        stage_to_lds<D>(st, lds, lds + C::LDS_K, tid);
        if (ntile > 1) kv.load(st, toff, P.kv_begin + C::BN, P.kv_end, tid);
        __syncthreads();
    }
    for (int j = 0; j < ntile; ++j) {
        const int key_base = P.kv_begin + j * C::BN;
        const char* lds_k = lds + (j & 1) * (C::LDS_K + C::LDS_V);
        const char* lds_v = lds_k + C::LDS_K;
        if (wave_active && key_base < w_lim_max) {
            if (key_base + C::BN > w_lim_min)
                tile_step<D, true>(ws, qf, lds_k, lds_v, lane, c2, thr, key_base, q_lim);
            else
                tile_step<D, false>(ws, qf, lds_k, lds_v, lane, c2, thr, key_base, q_lim);
        }
        if (j + 1 < ntile) {
            char* nk = lds + ((j + 1) & 1) * (C::LDS_K + C::LDS_V);
            stage_to_lds<D>(st, nk, nk + C::LDS_K, tid);
            if (j + 2 < ntile) kv.load(st, toff, key_base + 2 * C::BN, P.kv_end, tid);
        }
        __syncthreads();
    }

    // ---- epilogue -------------------------------------------------------------
    const float l_tot = half_sum(ws.l);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (qrow < P.n_rows) {
        if (out.fp32_out) {
            float* orow = (float*)(out.o + qrow * out.o_stride);
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
            char* orow = out.o + qrow * out.o_stride;
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
            const float ms = (ws.m == -INFINITY) ? 0.f : ws.m * c2;
            out.lse[qrow * out.lse_stride] = (l_tot > 0.f) ? (ms + __log2f(l_tot)) * kLn2 : -INFINITY;
        }
    }
}

}  // namespace attn
