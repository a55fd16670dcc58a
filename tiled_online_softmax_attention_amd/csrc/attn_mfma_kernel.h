// attn_mfma_kernel.h -- the per-workgroup driver of the bf16 MFMA attention
// forward: loads the query tile into registers, streams 64-key K/V tiles into
// LDS with direct global->LDS copies issued one tile ahead (two LDS buffers,
// one barrier per tile), runs the online-softmax tile step of
// attn_mfma_core.h, and writes O (bf16, or fp32 partials) and the
// log-sum-exp.  The source of K/V rows is a policy object, so the same driver
// serves contiguous K/V ([B,H,N,d]) and the paged pool.
//
// K/V source policy interface (all members device functions):
//   const char* k_group(int key, int kv_end) / v_group(...)
//       wave-uniform base address of the 16-row group holding key
//       min(key, kv_end - 1); rows of one group are contiguous (ROW_BYTES
//       apart) in memory, which holds for a contiguous head slab and for any
//       page of 16 or 32 tokens (groups are 16-aligned).
//   int group_row(int key, int kv_end)
//       row of key min(key, kv_end - 1) relative to that group base.
//   uint32_t group_bytes()
//       bytes addressable from a group base (range of the copy descriptor).
#pragma once

#include "attn_mfma_core.h"

namespace attn {

// One query tile's problem, resolved per workgroup.
struct TileProblem {
    const char* q;       // query row 0 of the tile (bytes)
    int64_t q_stride;    // bytes between query rows
    int n_rows;          // valid query rows in this tile
    int q_pos0;          // position of query row 0: row i may see keys
                         // < min(kv_end, q_pos0 + i + 1) when causal
    int causal;
    int kv_begin;        // keys [kv_begin, kv_end) are this workgroup's share
    int kv_end;
};

// Output writer: normalised bf16 rows, or fp32 rows + lse for split partials.
struct TileOut {
    char* o;             // output row 0 of the tile (bytes)
    int64_t o_stride;    // bytes between output rows
    float* lse;          // lse of row 0 (may be null)
    int64_t lse_stride;  // floats between rows
    int fp32_out;        // 1: write fp32 normalised O (partials), 0: bf16
};

// Query rows per workgroup: 4 waves x QB blocks of 32 queries.
template <int QB>
struct QueryTile {
    static constexpr int BM = 4 * 32 * QB;
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

// Issue this wave's direct copies of one K/V tile (16 rows of each) into an
// LDS buffer.  Rows at or past kv_end are fetched from row kv_end - 1 (valid
// data, masked out of S), so no copy reads outside the context.  For a full
// group the per-lane source offsets are loop-invariant (k_voff, v_voff) and
// the group's position goes in the scalar offset.
template <int D, class KV>
__device__ __forceinline__ void issue_tile_dma(const KV& kv, char* lds_k, char* lds_v, int key_base, int kv_end,
                                               int w, int lane, uint32_t k_voff, uint32_t v_voff)
{
#if defined(__HIP_DEVICE_COMPILE__)
    using C = TileCfg<D>;
    const int gkey = key_base + 16 * w;                 // this wave's first key (uniform)
    const __amdgpu_buffer_rsrc_t kr = raw_rsrc(kv.k_group(gkey, kv_end), kv.group_bytes());
    const __amdgpu_buffer_rsrc_t vr = raw_rsrc(kv.v_group(gkey, kv_end), kv.group_bytes());
    char* kdst = lds_k + w * 16 * C::ROW_BYTES;
    char* vdst = lds_v + w * 16 * C::ROW_BYTES;
    if (__builtin_expect(gkey + 16 <= kv_end, 1)) {
        const uint32_t soff = (uint32_t)kv.group_row(gkey, kv_end) * C::ROW_BYTES;
#pragma unroll
        for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, ATTN_LDS(kdst + i * 1024), 16, k_voff + i * kKDmaStep,
                                                     soff, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, ATTN_LDS(vdst + i * 1024), 16, v_voff + i * kVDmaStep,
                                                     soff, 0, 0);
        }
    } else {
        const uint32_t koff = (uint32_t)kv.group_row(gkey + k_dma_row<D>(lane), kv_end) * C::ROW_BYTES +
                              k_dma_col<D>(lane);
        const uint32_t vcol = v_dma_col<D>(lane);
#pragma unroll
        for (int i = 0; i < C::DMA_PER_WAVE; ++i) {
            const int vrow = kv.group_row(gkey + i * C::ROWS_PER_DMA + v_dma_row<D>(lane), kv_end);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, ATTN_LDS(kdst + i * 1024), 16, koff + i * kKDmaStep, 0,
                                                     0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, ATTN_LDS(vdst + i * 1024), 16,
                                                     (uint32_t)vrow * C::ROW_BYTES + vcol, 0, 0, 0);
        }
    }
#endif
}

// lds0 / lds1: the two LDS buffers (K tile then V tile in each); they must be
// distinct __shared__ objects so that reads of one are not ordered behind
// copies still in flight into the other.
template <int D, int QB, class KV>
__device__ __forceinline__ void run_query_tile(const TileProblem& P, const KV& kv, const TileOut& out, float c2_in,
                                               char* lds0, char* lds1)
{
    // scale * log2(e); a zero scale becomes a tiny positive factor (every
    // allowed key still gets p = 2^0 = 1 exactly, masked keys 2^-inf = 0)
    const float c2 = fmaxf(c2_in, 1e-30f);
    using C = TileCfg<D>;
    const int tid = threadIdx.x;
    const int lane = tid & 63, g = lane >> 5, r32 = lane & 31;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wrow0 = w * 32 * QB;            // first query row of this wave

    // ---- Q^T fragments, per-query key limits ----------------------------------
    bf16x8 qf[QB][C::KSTEPS];
    int q_lim[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = wrow0 + qb * 32 + r32;
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            u32x4 val = {0u, 0u, 0u, 0u};
            if (qrow < P.n_rows) val = *(const u32x4*)(P.q + qrow * P.q_stride + (ks * 2 + g) * 16);
            qf[qb][ks] = as_bf16x8(val);
        }
        // rows past n_rows run on zero queries and are never stored
        q_lim[qb] = P.causal ? min(P.kv_end, P.q_pos0 + qrow + 1) : P.kv_end;
    }
    // keys the whole tile needs
    int t_end = P.kv_end;
    if (P.causal) t_end = min(P.kv_end, P.q_pos0 + P.n_rows);

    WaveState<D, QB> ws;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) ws.o[qb][db] = f32x16{};
        ws.m[qb] = -INFINITY;
        ws.l[qb] = 0.f;
    }

    const float thr = kRescaleLog2 / c2;
    const uint32_t k_voff = (uint32_t)k_dma_row<D>(lane) * C::ROW_BYTES + k_dma_col<D>(lane);
    const uint32_t v_voff = (uint32_t)v_dma_row<D>(lane) * C::ROW_BYTES + v_dma_col<D>(lane);
    char* k0 = lds0;
    char* v0 = lds0 + C::TILE_BYTES;
    char* k1 = lds1;
    char* v1 = lds1 + C::TILE_BYTES;
    // Tile j lives in buffer j % 2.  Its copies are issued while tile j - 1 is
    // being consumed; "wait for my copies, then barrier" publishes it.
    const int ntile = (t_end > P.kv_begin) ? (t_end - P.kv_begin + C::BN - 1) / C::BN : 0;
    if (ntile > 0) {
        issue_tile_dma<D>(kv, k0, v0, P.kv_begin, P.kv_end, w, lane, k_voff, v_voff);
        __builtin_amdgcn_s_waitcnt(0x3f70);   // vmcnt(0): this wave's copies have landed
        __syncthreads();
    }
    // Phase 1: tiles that every row of the tile sees in full (below the
    // diagonal of query row 0 and before kv_end): no masking and no per-wave
    // skipping, so the loop body is straight-line apart from the rescale.
    // Waves past the last valid row compute on zero queries here and never
    // store.  This keeps O in one register set across the loop (branches
    // around the tile step make the allocator move O between register sets).
    int n_full = 0;
    {
        const int lim = P.causal ? min(P.kv_end, P.q_pos0 + 1) : P.kv_end;
        if (lim > P.kv_begin) n_full = min(ntile, (lim - P.kv_begin) / C::BN);
    }
    int j = 0;
    for (; j + 2 <= n_full; j += 2) {
        const int kb0 = P.kv_begin + j * C::BN;
        issue_tile_dma<D>(kv, k1, v1, kb0 + C::BN, P.kv_end, w, lane, k_voff, v_voff);
        tile_step<D, QB, false>(ws, qf, k0, v0, lane, c2, thr, kb0, q_lim);
        __builtin_amdgcn_s_waitcnt(0x3f70);
        __syncthreads();
        if (j + 2 < ntile) issue_tile_dma<D>(kv, k0, v0, kb0 + 2 * C::BN, P.kv_end, w, lane, k_voff, v_voff);
        tile_step<D, QB, false>(ws, qf, k1, v1, lane, c2, thr, kb0 + C::BN, q_lim);
        __builtin_amdgcn_s_waitcnt(0x3f70);
        __syncthreads();
    }
    // Phase 2: the rest (diagonal and tail tiles), always through the masked
    // step: a tile that is fully masked for a lane adds exactly nothing
    // (p = 0, and the running offset only moves on a finite score), so waves
    // whose rows see none of it need no separate skip path.  j is even here,
    // so tile j is in buffer 0.
    for (; j < ntile; j += 2) {
        const int kb0 = P.kv_begin + j * C::BN;
        if (j + 1 < ntile) issue_tile_dma<D>(kv, k1, v1, kb0 + C::BN, P.kv_end, w, lane, k_voff, v_voff);
        tile_step<D, QB, true>(ws, qf, k0, v0, lane, c2, thr, kb0, q_lim);
        __builtin_amdgcn_s_waitcnt(0x3f70);
        __syncthreads();
        if (j + 1 < ntile) {
            if (j + 2 < ntile) issue_tile_dma<D>(kv, k0, v0, kb0 + 2 * C::BN, P.kv_end, w, lane, k_voff, v_voff);
            tile_step<D, QB, true>(ws, qf, k1, v1, lane, c2, thr, kb0 + C::BN, q_lim);
            __builtin_amdgcn_s_waitcnt(0x3f70);
            __syncthreads();
        }
    }

    // ---- epilogue -------------------------------------------------------------
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int qrow = wrow0 + qb * 32 + r32;
        const float l_tot = half_sum(ws.l[qb]);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        if (qrow < P.n_rows) {
            if (out.fp32_out) {
                float* orow = (float*)(out.o + qrow * out.o_stride);
#pragma unroll
                for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        f32x4 v4;
                        v4[0] = ws.o[qb][db][a * 4 + 0] * inv;
                        v4[1] = ws.o[qb][db][a * 4 + 1] * inv;
                        v4[2] = ws.o[qb][db][a * 4 + 2] * inv;
                        v4[3] = ws.o[qb][db][a * 4 + 3] * inv;
                        *(f32x4*)(orow + db * 32 + a * 8 + g * 4) = v4;
                    }
            } else {
                char* orow = out.o + qrow * out.o_stride;
#pragma unroll
                for (int db = 0; db < C::DBLK; ++db)
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        u32x2 w2;
                        w2[0] = pack_bf16(ws.o[qb][db][a * 4 + 0] * inv, ws.o[qb][db][a * 4 + 1] * inv);
                        w2[1] = pack_bf16(ws.o[qb][db][a * 4 + 2] * inv, ws.o[qb][db][a * 4 + 3] * inv);
                        *(u32x2*)(orow + (db * 32 + a * 8 + g * 4) * 2) = w2;
                    }
            }
            if (out.lse && g == 0) {
                const float ms = (ws.m[qb] == -INFINITY) ? 0.f : ws.m[qb] * c2;
                out.lse[qrow * out.lse_stride] = (l_tot > 0.f) ? (ms + __log2f(l_tot)) * kLn2 : -INFINITY;
            }
        }
    }
}

}  // namespace attn
