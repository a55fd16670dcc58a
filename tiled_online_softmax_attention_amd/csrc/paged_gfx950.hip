// paged_gfx950.hip -- attention over a paged KV cache for gfx950: decode
// (a few query rows per request) and chunked prefill (an appended chunk of
// query rows per request), plus the log-sum-exp combine of context splits and
// the bit-exact gather used to check the address function.
//
// Address function ("Chunked attention ... 70x slower", section 2.1, and the
// pool layout of "Flash Attention and Paged Attention", section 3): token t of
// request r lives in physical block pb = block_table[r][t / bs] at offset
// t % bs; the [bs, d] slab of head h in that block is contiguous, so every
// page is read as whole 16-byte-per-lane rows, never element by element.
// Block offsets are 64-bit (a pool may exceed 2^31 elements).
//
// Work decomposition: each request's context is cut into splits of a fixed
// number of tokens (a whole number of pages).  One launch covers every
// (request, query row or tile, head, split) of the batch; a split writes a
// normalised fp32 partial and its log-sum-exp, and a second launch merges the
// partials of each (row, head).  Requests whose context fits one split write
// their final output directly.  The plan depends only on host bounds, so
// results never depend on where blocks sit in the pool.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>

#include "attn_internal.h"
#include "attn_mfma_kernel.h"
#include "attn_mfma_pipe.h"

namespace attn {

// Context length of request r as every paged kernel reads it: clamped to the
// host bound max_ctx_len, so that a length above the bound (a broken contract,
// which ATTN_DEBUG=1 reports) cannot make a kernel read block-table entries
// past max_blocks_per_seq or the combine read split slots past max_splits.
template <class A>
__device__ __forceinline__ int req_ctx(const A& a, int r)
{
    return min(a.ctx_lens[r], a.max_ctx_len);
}

// Query rows of request r that the kernels compute: clamped to max_q_len
// likewise (the grid and the split partials are sized by it).
template <class A>
__device__ __forceinline__ int req_ql(const A& a, int r)
{
    return min(a.q_lens[r], a.max_q_len);
}


// ---- small wave helpers ------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
// Sum over aligned groups of 16 (or 8) lanes, result in every lane of the group.
template <int LPR>
__device__ __forceinline__ float group_sum(float x)
{
    x += dpp<0xB1>(x);      // quad_perm [1,0,3,2]
    x += dpp<0x4E>(x);      // quad_perm [2,3,0,1]
    x += dpp<0x141>(x);     // row_half_mirror: pairs quad 0 with quad 1
    if (LPR == 16) x += dpp<0x140>(x);   // row_mirror: pairs the two halves of a row
    return x;
}

// sum_e a[e] * b[e] over 8 bf16 pairs, fp32 accumulation (bf16 dot2).  The
// pairs are taken with shufflevector from whole 8-element vectors; bit-casting
// single 32-bit elements of a loaded vector to bf16x2 is mis-lowered by the
// compiler (every pair ends up reading the first element).
__device__ __forceinline__ float dot8_bf16(bf16x8 a, bf16x8 b)
{
    float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 0, 1), __builtin_shufflevector(b, b, 0, 1), 0.f, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 2, 3), __builtin_shufflevector(b, b, 2, 3), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 4, 5), __builtin_shufflevector(b, b, 4, 5), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(a, a, 6, 7), __builtin_shufflevector(b, b, 6, 7), acc, false);
    return acc;
}

__device__ __forceinline__ int wave_sum_int(int x)
{
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

__device__ __forceinline__ float wave_max(float x)
{
    for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}

__device__ __forceinline__ float wave_sum(float x)
{
    for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
    return x;
}

// sum_{s<r} lens[s], computed by one wave (every lane gets the result)
__device__ __forceinline__ int64_t prefix_len(const int32_t* lens, int r, int lane)
{
    int64_t acc = 0;
    for (int s0 = 0; s0 < r; s0 += 64) {
        int s = s0 + lane;
        int v = (s < r) ? lens[s] : 0;
        acc += wave_sum_int(v);
    }
    return acc;
}

// ============================================================================
// Decode kernel: one workgroup (4 waves) per (request, query row, K/V head,
// group of GC query heads, split).  The GC query heads share that K/V head
// (grouped-query attention; GC = 1 for plain multi-head attention), so every
// K/V page is read once for all of them.  Lanes are grouped by LPR = d/8: a
// group of LPR lanes holds one token row of a page (16 bytes = 8 channels per
// lane), so each 16-byte-per-lane load covers 64/LPR consecutive tokens.  q.k
// uses bf16 dot2 on the raw pairs; the group reduction is DPP; the wave takes
// pages w, w+4, ... of the split with the next page's loads in flight while
// the current page is consumed; the four waves' partial (m, l, o) of every
// query head are merged through LDS.
// ============================================================================
template <int D, int BS, int GC>
__global__ __launch_bounds__(256) void paged_decode_kernel(PagedArgs a)
{
    constexpr int LPR = D / 8;
    constexpr int TPL = 64 / LPR;       // tokens per wave-load
    constexpr int LOADS = BS / TPL;     // loads per lane per page (each of K, V)
    __shared__ float red_o[4][GC][D];
    __shared__ float red_ml[4][GC][2];

    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int sub = lane / LPR, oct = lane % LPR;
    int bid = blockIdx.x;
    const int split = bid % a.max_splits;
    bid /= a.max_splits;
    const int chunk = bid % a.n_chunks;
    bid /= a.n_chunks;
    const int hk = bid % a.H_kv;
    bid /= a.H_kv;
    const int i = bid % a.max_q_len;
    const int r = bid / a.max_q_len;
    const int ctx = req_ctx(a, r), ql = a.q_lens[r];
    if (i >= ql) return;
    const int S = a.split_tokens;
    const int nsplit = (ctx + S - 1) / S;
    if (split >= nsplit) return;
    const int lim = ctx - ql + i + 1;             // keys [0, lim) are visible
    const int kbeg = split * S, kend = min(kbeg + S, lim);
    const int64_t row = prefix_len(a.q_lens, r, lane) + i;
    const float c2 = a.scale * kLog2e;
    const int h0 = hk * (a.H / a.H_kv) + chunk * GC;   // first query head of this workgroup

    bf16x8 qb[GC];
#pragma unroll
    for (int g = 0; g < GC; ++g)
        qb[g] = as_bf16x8(*(const u32x4*)((const char*)a.q + ((row * a.H + h0 + g) * D + oct * 8) * 2));
    const int32_t* table = a.block_table + (int64_t)r * a.max_blocks_per_seq;
    const int64_t blk_bytes = a.kv_block_stride * 2;
    const char* kbase = (const char*)a.k_pool + (int64_t)hk * BS * D * 2 + oct * 16;
    const char* vbase = (const char*)a.v_pool + (int64_t)hk * BS * D * 2 + oct * 16;

    float m[GC], l[GC], o[GC][8];
#pragma unroll
    for (int g = 0; g < GC; ++g) {
        m[g] = -INFINITY;
        l[g] = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[g][e] = 0.f;
    }

    const int pbeg = kbeg / BS;
    const int pend = (kend > kbeg) ? (kend + BS - 1) / BS : pbeg;
    // K/V loads are non-temporal: every page is read by this workgroup alone
    // (5.91 -> 6.23 TB/s on the 64-request decode batch)
    u32x4 kr[LOADS], vr[LOADS], kn[LOADS], vn[LOADS];
    int p = pbeg + w;
    if (p < pend) {
        const int64_t pb = table[p];
        const char* kp = kbase + pb * blk_bytes;
        const char* vp = vbase + pb * blk_bytes;
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            kr[j] = __builtin_nontemporal_load((const u32x4*)(kp + (j * TPL + sub) * D * 2));
            vr[j] = __builtin_nontemporal_load((const u32x4*)(vp + (j * TPL + sub) * D * 2));
        }
    }
    for (; p < pend; p += 4) {
        const int pn = p + 4;
        if (pn < pend) {
            const int64_t pb = table[pn];
            const char* kp = kbase + pb * blk_bytes;
            const char* vp = vbase + pb * blk_bytes;
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                kn[j] = __builtin_nontemporal_load((const u32x4*)(kp + (j * TPL + sub) * D * 2));
                vn[j] = __builtin_nontemporal_load((const u32x4*)(vp + (j * TPL + sub) * D * 2));
            }
        }
        // scores of this lane group's tokens, for every query head
        const bool tail = (p + 1) * BS > kend;
        bool dead[LOADS];
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            dead[j] = tail && (p * BS + j * TPL + sub >= kend);
            if (dead[j]) vr[j] = u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int g = 0; g < GC; ++g) {
            float s[LOADS];
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                s[j] = group_sum<LPR>(dot8_bf16(qb[g], as_bf16x8(kr[j])));
                if (dead[j]) s[j] = -INFINITY;
            }
            float mt = s[0];
#pragma unroll
            for (int j = 1; j < LOADS; ++j) mt = fmaxf(mt, s[j]);
#pragma unroll
            for (int x = LPR; x < 64; x <<= 1) mt = fmaxf(mt, __shfl_xor(mt, x, 64));
            const float m_new = fmaxf(m[g], mt);        // finite: every page has a visible key
            const float ms_new = m_new * c2;
            const float alpha = (m[g] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[g] * c2 - ms_new);
            m[g] = m_new;
            float ps = 0.f;
#pragma unroll
            for (int e = 0; e < 8; ++e) o[g][e] *= alpha;
#pragma unroll
            for (int j = 0; j < LOADS; ++j) {
                const float pj = dead[j] ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], c2, -ms_new));
                ps += pj;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    o[g][2 * e] = __builtin_fmaf(pj, bf16lo(vr[j][e]), o[g][2 * e]);
                    o[g][2 * e + 1] = __builtin_fmaf(pj, bf16hi(vr[j][e]), o[g][2 * e + 1]);
                }
            }
            l[g] = l[g] * alpha + ps;
        }
#pragma unroll
        for (int j = 0; j < LOADS; ++j) {
            kr[j] = kn[j];
            vr[j] = vn[j];
        }
    }
    // merge the lane groups of this wave (same channels, different tokens),
    // then the four waves through LDS
#pragma unroll
    for (int g = 0; g < GC; ++g) {
#pragma unroll
        for (int x = LPR; x < 64; x <<= 1) {
            l[g] += __shfl_xor(l[g], x, 64);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[g][e] += __shfl_xor(o[g][e], x, 64);
        }
        if (sub == 0) {
#pragma unroll
            for (int e = 0; e < 8; ++e) red_o[w][g][oct * 8 + e] = o[g][e];
        }
        if (lane == 0) {
            red_ml[w][g][0] = m[g];
            red_ml[w][g][1] = l[g];
        }
    }
    __syncthreads();
    if (w != 0) return;
    for (int g = 0; g < GC; ++g) {
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < 4; ++x) M = fmaxf(M, red_ml[x][g][0]);
        const float Ms = (M == -INFINITY) ? 0.f : M * c2;
        float sc[4], L = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            sc[x] = (red_ml[x][g][0] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(red_ml[x][g][0] * c2 - Ms);
            L += sc[x] * red_ml[x][g][1];
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const float lse = L > 0.f ? (Ms + __log2f(L)) * kLn2 : -INFINITY;
        const int h = h0 + g;
        // lane c writes channels c and c + 64 (d = 64 or 128)
        if (nsplit == 1) {
            __bf16* orow = (__bf16*)a.o + (row * a.H + h) * D;
            for (int c = lane; c < D; c += 64) {
                float acc = 0.f;
#pragma unroll
                for (int x = 0; x < 4; ++x) acc += sc[x] * red_o[x][g][c];
                orow[c] = (__bf16)(acc * inv);
            }
            if (a.lse && lane == 0) a.lse[row * a.H + h] = lse;
        } else {
            const int64_t slot = (((int64_t)r * a.max_q_len + i) * a.H + h) * a.max_splits + split;
            float* wo = a.ws_o + slot * D;
            for (int c = lane; c < D; c += 64) {
                float acc = 0.f;
#pragma unroll
                for (int x = 0; x < 4; ++x) acc += sc[x] * red_o[x][g][c];
                wo[c] = acc * inv;
            }
            if (lane == 0) a.ws_lse[slot] = lse;
        }
    }
}

// ============================================================================
// Decode on the matrix cores, for grouped query heads: the G = H / H_kv query
// heads of one K/V head at a few query positions give G x q_len <= 16 rows,
// which form the N side of 16x16 MFMAs:
//   S^T (16 keys x 16 rows)  = K (16 keys x d) Q^T      16x16x32 bf16, d/32 steps
//   O^T (d x 16 rows)       += V^T (d x 16 keys) P^T     16x16x16 bf16, d/16 blocks
// The S^T accumulator (lane l: row l % 16, keys 4 (l / 16) .. + 3) is the P^T
// operand as it stands.  One workgroup of four waves per (request, K/V head,
// split); each wave takes 16-key tiles w, w + 4, ... of the split and keeps
// two of them in flight beyond the one it computes: K straight into
// registers in the MFMA operand layout, V into a ring of three 16-row LDS
// tiles private to the wave (direct global -> LDS copies, landing row-major
// with the swizzle of v_ofs; read back transposed with ds_read_b64_tr_b16).
// A wave only waits for its own loads -- no barrier ties the waves together.
// The online softmax is the tile kernel's (base 2, lazy offset, p rounded to
// bf16 for the product, the sum in fp32); the four waves' (offset, sum, O)
// are merged through LDS at the end.
// ============================================================================
constexpr int kDecMfmaRows = 16;       // query rows (heads x positions) per workgroup
constexpr int kDecMfmaMinPairs = 512;  // (request, K/V head) pairs from which it is the default ...
constexpr int kDecMfmaMinPairsGrouped = 1024;   // ... for groups of kDecodeMfmaGroup heads and more

__device__ __forceinline__ f32x4 mfma16x32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16(i16x4 a, i16x4 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// max / sum over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes holding
// one row), through the row-swap permutes (no LDS traffic)
__device__ __forceinline__ float row4_max(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                    false, false);
    return half_max(fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1])));
}
__device__ __forceinline__ float row4_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                    false, false);
    return half_sum(__builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]));
}

template <int D, int BS>
__global__ __launch_bounds__(256, 3) void paged_decode_mfma_kernel(PagedArgs a)
{
    constexpr int KS = D / 32;         // S^T steps of 32 channels
    constexpr int DB = D / 16;         // O^T blocks of 16 channels
    constexpr int ROW = D * 2;         // bytes per K/V row
    constexpr int VC = TileCfg<D>::COPIES_PER_GROUP;   // wave-wide V copies per 16-key tile
    constexpr int PER = KS + VC;                        // loads per tile (vmcnt units)
    constexpr int VT = 16 * ROW;                        // bytes of a V tile
    constexpr int RED = 4 * DB * 4 * 64 * 4;            // merge buffer: every wave's O^T registers
    constexpr int LDS_BYTES = (4 * 3 * VT > RED) ? 4 * 3 * VT : RED;
    static_assert(PER * 2 < 64, "vmcnt field");
    __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];   // V rings, then the merge buffer
    __shared__ float red_ml[4][kDecMfmaRows][2];                     // per wave and row: offset, sum

    const int lane = threadIdx.x & 63;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    // split-major: consecutive blocks (dealt to the 8 XCDs in turn) take
    // different (request, K/V head) pairs, so that every XCD gets a share of
    // each split index -- with the split fastest, a split count that is a
    // multiple of 8 puts split s on XCD s mod 8, and the high splits exist
    // only for the longest contexts
    const int n_pairs = a.num_seqs * a.H_kv;
    const int split = (int)blockIdx.x / n_pairs;
    const int pair = (int)blockIdx.x % n_pairs;
    const int hk = pair % a.H_kv;
    const int r = pair / a.H_kv;
    const int ctx = req_ctx(a, r), ql = req_ql(a, r);
    const int S = a.split_tokens;
    const int nsplit = (ctx + S - 1) / S;
    if (split >= nsplit) return;
    const int G = a.H / a.H_kv;
    const int kbeg = split * S, kend = min(kbeg + S, ctx);
    const float c2 = fmaxf(a.scale * kLog2e, 1e-30f);
    const float thr = kRescaleLog2 / c2;

    // this lane's row t = l % 16: query position qi, query head hk * G + qg;
    // rows at or past G * q_len run on zero queries and are never stored
    const int t = lane & 15;
    const int qi = t / G, qg = t % G;
    const bool row_ok = qi < ql;
    const int vis_end = min(row_ok ? ctx - ql + qi + 1 : kend, kend);   // keys < vis_end are visible
    const int64_t prow0 = prefix_len(a.q_lens, r, lane);                // packed row of position 0
    bf16x8 qf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row_ok)
            v = *(const u32x4*)((const char*)a.q + (((prow0 + qi) * a.H + hk * G + qg) * D + 32 * ks + 8 * (lane >> 4)) * 2);
        qf[ks] = as_bf16x8(v);
    }

    // block-table entries of the split's pages (at most 128: the plan caps
    // the split) in two registers, lane i holding pages p0 + i and p0 + 64 + i
    const int p0 = kbeg / BS, np = (kend - 1) / BS - p0 + 1;
    const int32_t* trow = a.block_table + (int64_t)r * a.max_blocks_per_seq + p0;
    const int pgv0 = trow[min(lane, np - 1)];
    const int pgv1 = trow[min(64 + lane, np - 1)];
    const int64_t blk_bytes = a.kv_block_stride * 2;
    const char* kbase = (const char*)a.k_pool + (int64_t)hk * BS * ROW;
    const char* vbase = (const char*)a.v_pool + (int64_t)hk * BS * ROW;
    const int last = kend - 1;

    // Loads of 16-key tile tt (keys kbeg + 16 tt ..; a tile lies in one page):
    // K lane l: key l % 16, channels 32 ks + 8 (l / 16) .. + 7 (the A operand
    // of S^T); V: the copy layout of v_dma_row / v_dma_col for one 16-row
    // group, into the LDS tile vt.  Both non-temporal (read by this
    // workgroup alone).  Keys at or past kend are read from key kend - 1
    // (valid data; the mask removes them).  KS register loads, then VC copies.
    const auto load_tile = [&](int tt, u32x4 (&kr)[KS], char* vt) {
        const int key0 = kbeg + 16 * tt;
        const int pi = key0 / BS - p0;   // < 128, wave-uniform
        const int64_t pg = (pi < 64) ? __builtin_amdgcn_readlane(pgv0, pi) : __builtin_amdgcn_readlane(pgv1, pi - 64);
        const char* kp = kbase + pg * blk_bytes;
        const int krow = min(key0 + (lane & 15), last) & (BS - 1);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
            kr[ks] = __builtin_nontemporal_load((const u32x4*)(kp + krow * ROW + 64 * ks + 16 * (lane >> 4)));
#if defined(__HIP_DEVICE_COMPILE__)
        const __amdgpu_buffer_rsrc_t rv = raw_rsrc(vbase + pg * blk_bytes, (uint32_t)(BS * ROW));
        const uint32_t vcol = v_dma_col<D>(lane);
#pragma unroll
        for (int i = 0; i < VC; ++i) {
            const int vrow = min(key0 + i * TileCfg<D>::ROWS_PER_DMA + v_dma_row<D>(lane), last) & (BS - 1);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, ATTN_LDS(vt + i * 1024), 16, (uint32_t)vrow * ROW + vcol, 0,
                                                     0, kCopyStream);
        }
#endif
    };
    // wait for this wave's loads of a tile, `later` tiles having been issued
    // after it (vmcnt counts a wave's loads in issue order)
    const auto wait_tile = [](int later) {
        asm volatile("" ::: "memory");
        if (later >= 2) __builtin_amdgcn_s_waitcnt(0x3f70 | (2 * PER));
        else if (later == 1) __builtin_amdgcn_s_waitcnt(0x3f70 | PER);
        else __builtin_amdgcn_s_waitcnt(0x3f70);
        asm volatile("" ::: "memory");
    };

    f32x4 o[DB];
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m = -INFINITY, ms = 0.f, l = 0.f;
    char* vring = lds + w * 3 * VT;
    // this lane's transposing V read (A operand of O^T: channel 16 db + l % 16,
    // keys 4 (l / 16) .. + 3): row 4 (l / 16) + (l % 16) / 4, channels
    // 16 db + 4 (l % 4) .. + 3
    const uint32_t tr_row = 4u * (uint32_t)(lane >> 4) + (uint32_t)((lane & 15) >> 2);

    const auto compute = [&](int tt, const u32x4 (&kr)[KS], const char* vt) {
        const int key0 = kbeg + 16 * tt;
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) s = mfma16x32(as_bf16x8(kr[ks]), qf[ks], s);
        // keys key0 + 4 (l / 16) + i; visible while below vis_end
        const int nvis = vis_end - (key0 + 4 * (lane >> 4));
#pragma unroll
        for (int i = 0; i < 4; ++i) s[i] = (i < nvis) ? s[i] : -INFINITY;
        const float mt = row4_max(fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3])));
        if (__builtin_amdgcn_ballot_w64(mt > m + thr) != 0) {
            const float m_new = fmaxf(m, mt);
            const float alpha = (m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((m - m_new) * c2);
            m = m_new;
            ms = (m_new == -INFINITY) ? 0.f : m_new * c2;
            l *= alpha;
#pragma unroll
            for (int db = 0; db < DB; ++db) o[db] *= alpha;
        }
        float p[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], c2, -ms));
            l += p[i];
        }
        bf16x4 pb;
        pb[0] = (__bf16)p[0];
        pb[1] = (__bf16)p[1];
        pb[2] = (__bf16)p[2];
        pb[3] = (__bf16)p[3];
        const i16x4 pbi = __builtin_bit_cast(i16x4, pb);
        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            const uint32_t cb = (uint32_t)(32 * db + 8 * (lane & 3));    // byte column
            const i16x4 va = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_i16x4*)(vt + v_ofs<D>(tr_row, cb >> 4) + (cb & 15u)));
            o[db] = mfma16x16(va, pbi, o[db]);
        }
    };

    // this wave's tiles w + 4 k, k < nmine, in register sets / LDS tiles
    // k % 3; the loads of tiles k + 1 and k + 2 are in flight while tile k is
    // computed
    const int ntile = (kend - kbeg + 15) / 16;
    const int nmine = (w < ntile) ? (ntile - w + 3) / 4 : 0;
    u32x4 ka[KS], kb[KS], kc[KS];
    char* const v0 = vring;
    char* const v1 = vring + VT;
    char* const v2 = vring + 2 * VT;
    if (nmine > 0) load_tile(w, ka, v0);
    if (nmine > 1) load_tile(w + 4, kb, v1);
    for (int k = 0; k < nmine; k += 3) {
        // an LDS tile is reloaded only after the reads of its last use are done
        __builtin_amdgcn_s_waitcnt(0xc07f);
        if (k + 2 < nmine) load_tile(w + 4 * (k + 2), kc, v2);
        wait_tile(min(2, nmine - 1 - k));
        compute(w + 4 * k, ka, v0);
        if (k + 1 >= nmine) break;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        if (k + 3 < nmine) load_tile(w + 4 * (k + 3), ka, v0);
        wait_tile(min(2, nmine - 2 - k));
        compute(w + 4 * (k + 1), kb, v1);
        if (k + 2 >= nmine) break;
        __builtin_amdgcn_s_waitcnt(0xc07f);
        if (k + 4 < nmine) load_tile(w + 4 * (k + 4), kb, v1);
        wait_tile(min(2, nmine - 3 - k));
        compute(w + 4 * (k + 2), kc, v2);
    }

    // merge the four waves: O^T registers, offsets and row sums through LDS
    // (the V rings' space, once every wave is done with its ring)
    const float lrow = row4_sum(l);
    __syncthreads();
    float (*red_o)[DB][4][64] = (float (*)[DB][4][64])lds;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) red_o[w][db][i][lane] = o[db][i];
    if (lane < kDecMfmaRows) {
        red_ml[w][lane][0] = m;
        red_ml[w][lane][1] = lrow;
    }
    __syncthreads();
    const int64_t slot0 = (int64_t)r * a.max_q_len;
    for (int item = threadIdx.x; item < kDecMfmaRows * D; item += 256) {
        const int tr = item / D, c = item % D;
        const int pi = tr / G, pg = tr % G;
        if (pi >= ql) break;            // rows are ascending in item
        float M = -INFINITY;
#pragma unroll
        for (int x = 0; x < 4; ++x) M = fmaxf(M, red_ml[x][tr][0]);
        const float Ms = (M == -INFINITY) ? 0.f : M * c2;
        float L = 0.f, acc = 0.f;
        const int src_lane = tr + 16 * ((c & 15) >> 2);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const float mx = red_ml[x][tr][0];
            const float sc = (mx == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mx * c2 - Ms);
            L += sc * red_ml[x][tr][1];
            acc += sc * red_o[x][c >> 4][c & 3][src_lane];
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
        const float lse = L > 0.f ? (Ms + __log2f(L)) * kLn2 : -INFINITY;
        const int h = hk * G + pg;
        const int64_t row = prow0 + pi;
        if (nsplit == 1) {
            ((__bf16*)a.o)[(row * a.H + h) * D + c] = (__bf16)(acc * inv);
            if (a.lse && c == 0) a.lse[row * a.H + h] = lse;
        } else {
            const int64_t slot = ((slot0 + pi) * a.H + h) * a.max_splits + split;
            a.ws_o[slot * D + c] = acc * inv;
            if (c == 0) a.ws_lse[slot] = lse;
        }
    }
}

// ============================================================================
// Chunked-prefill kernel: the bf16 MFMA tile driver with K/V rows fetched
// through the block table.  One workgroup per (request, 128-row query tile,
// head, split); query tiles of one (request, head, split) are adjacent in the
// XCD-contiguous order so they share K/V pages in that XCD's L2.
// ============================================================================
// K/V rows through the block table.  A 16-row group of keys (16-aligned)
// lies inside one page of 16 or 32 tokens, so the group base is one scalar
// table read; keys are clamped to the last key of the context first, so no
// page past the context is ever looked up.  STREAM: the pipelined loop's
// copies are non-temporal (kCopyStream), for the decode-length variant,
// where a split's K/V tiles are read by its one workgroup.
template <int D, int BS, bool STREAM>
struct PagedKV {
    const char* kbase;       // k_pool + head offset (bytes)
    const char* vbase;
    const int32_t* ptab;     // LDS copy of the block-table entries of pages p0, p0 + 1, ...
    int p0;                  // first page of this workgroup's keys
    int64_t blk_bytes;
    // The plain key loop copies one tile ahead (two tiles ahead fetched
    // about 1.8x the pool bytes on the chunked-prefill batch).
    static constexpr int kCopiesAhead = 1;
    // The page of every key tile comes from the workgroup's LDS copy of its
    // pages' table entries (staged once; a global table read at the head of
    // each tile step would hold up that tile's copies by a memory latency).
    __device__ __forceinline__ int64_t page_of(int key, int kv_end) const
    {
        return (int64_t)__builtin_amdgcn_readfirstlane(ptab[min(key, kv_end - 1) / BS - p0]);
    }
    __device__ __forceinline__ const char* k_group(int key, int kv_end) const
    {
        return kbase + page_of(key, kv_end) * blk_bytes;
    }
    __device__ __forceinline__ const char* v_group(int key, int kv_end) const
    {
        return vbase + page_of(key, kv_end) * blk_bytes;
    }
    __device__ __forceinline__ int group_row(int key, int kv_end) const { return min(key, kv_end - 1) % BS; }
    __device__ __forceinline__ uint32_t group_bytes() const { return (uint32_t)(BS * D * 2); }
    // Copies of the pipelined key loop.  The window holds the table entries
    // of pages p0 + base .. p0 + base + 63 (lane l: base + l, clamped to the
    // last page of the context); a tile's copies take the entry of the page
    // holding the wave's copy group out of it with a lane read.
    struct SrcWin {
        int base;   // window start, relative to p0 (uniform)
        int pg;     // lane l: table entry of page p0 + base + l
    };
    __device__ __forceinline__ SrcWin empty_win() const { return SrcWin{-(1 << 30), 0}; }
    __device__ __forceinline__ void win_update(SrcWin& win, const WaveCtx& cx, int key_lo, int key_hi) const
    {
        const int last = (cx.kv_end - 1) / BS - p0;    // last page of the context, relative to p0
        const int lo = min(key_lo / BS - p0, last), hi = min(key_hi / BS - p0, last);
        if (lo < win.base || hi >= win.base + 64) {
            win.base = lo;
            win.pg = ptab[min(lo + cx.lane, last)];
        }
    }
    __device__ __forceinline__ int copy_src(const SrcWin& win, const WaveCtx& cx, int key_base) const
    {
        const int cw = cx.w & 3;
        const int gkey = key_base + 16 * (cw >= TileCfg<D>::GROUPS ? cw - TileCfg<D>::GROUPS : cw);
        return __builtin_amdgcn_readlane(win.pg, min(gkey, cx.kv_end - 1) / BS - p0 - win.base);
    }
    template <int NW>
    __device__ __forceinline__ void copy_tile(const WaveCtx& cx, char* buf, int key_base, int page) const
    {
        constexpr int CPOL = STREAM ? kCopyStream : 0;
        issue_tile_copies_paged<D, NW, BS, CPOL>(kbase, vbase, blk_bytes, cx, buf, key_base, page);
    }
};

// Work mapping.  An item is (request r, K/V head hk, context split, query
// tile); the items of one (r, hk) pair read that head's K/V, so they run on
// one XCD (workgroups are dealt to the 8 XCDs round-robin by block id) and
// share its L2, and the pairs are dealt to the XCDs round-robin (pair 8 m + x
// on XCD x), so that every XCD gets a similar mix of long and short
// requests.  (Contiguous per-XCD ranges hand an XCD whole requests -- one
// request per XCD for a batch of 8 -- and unequal contexts then leave most
// XCDs idle behind the longest; dealing (pair, split) units instead puts
// split s on XCD s mod 8 whenever max_splits is a multiple of 8, and the
// high splits exist only for the longest contexts.)  With fewer than
// kChunkPairsPerXcd pairs per XCD, items are dealt round-robin one by one
// instead, so that a small batch still spreads over all XCDs.
constexpr int kChunkPairsPerXcd = 4;
enum { kMapRanges = 0, kMapPairs = 1, kMapItems = 2 };

// KIND 0: 128-row query tiles, the plain key loop, three workgroups per CU;
// KIND 1: 128-row query tiles, the pipelined key loop (attn_mfma_pipe.h), two
// workgroups per CU; KIND 2: 256-row query tiles of eight waves, the
// pipelined loop, one workgroup per CU, each K/V tile staged once for 256
// rows.
template <int KIND>
constexpr int chunk_waves() { return KIND == 2 ? 8 : 4; }

template <int D, int BS, int KIND>
__global__ __launch_bounds__(64 * chunk_waves<KIND>(), KIND == 0 ? 3 : (KIND == 1 ? 2 : 1))
void paged_chunk_kernel(PagedArgs a, int n_work, int map)
{
    using C = TileCfg<D>;
    constexpr int NW = chunk_waves<KIND>();
    __shared__ __attribute__((aligned(16))) char lds0[2 * C::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char lds1[2 * C::TILE_BYTES];
    __shared__ int32_t ptab[kChunkMaxSplit / BS];
    const TileBuffers buf{lds0, lds1, nullptr};
    PipeBuffers pbuf{{lds0, lds1, nullptr, nullptr}};
    if constexpr (KIND != 0) {
        __shared__ __attribute__((aligned(16))) char lds2[2 * C::TILE_BYTES];
        __shared__ __attribute__((aligned(16))) char lds3[2 * C::TILE_BYTES];
        pbuf.b[2] = lds2;
        pbuf.b[3] = lds3;
    }
    // A tile holds ppt query positions x G query heads (the heads of one K/V
    // group), so each K/V tile staged in LDS serves the whole group.
    const int G = a.H / a.H_kv;
    const int ppt = 32 * NW / G;                       // positions per tile
    const int nqt = (a.max_q_len + ppt - 1) / ppt;
    int qt, split, pair;                               // pair = r * H_kv + hk
    if (map == kMapPairs) {
        const int per_pair = nqt * a.max_splits;       // items of one pair
        const int j = blockIdx.x >> 3;                 // position on this XCD
        pair = (blockIdx.x & 7) + 8 * (j / per_pair);
        if (pair >= a.num_seqs * a.H_kv) return;
        qt = (j % per_pair) % nqt;
        split = (j % per_pair) / nqt;
    } else if (map == kMapItems) {
        // item = block id, query tile fastest, then pair, then split (so that
        // the XCD an item lands on does not follow its split)
        int L = (int)blockIdx.x;
        if (L >= n_work) return;
        qt = L % nqt;
        L /= nqt;
        pair = L % (a.num_seqs * a.H_kv);
        split = L / (a.num_seqs * a.H_kv);
    } else {
        // XCD-contiguous ranges of (pair, split, query tile)
        int L = (blockIdx.x & 7) * (gridDim.x >> 3) + (blockIdx.x >> 3);
        if (L >= n_work) return;
        qt = L % nqt;
        L /= nqt;
        split = L % a.max_splits;
        pair = L / a.max_splits;
    }
    const int hk = pair % a.H_kv;
    const int r = pair / a.H_kv;
    const int ctx = req_ctx(a, r), ql = req_ql(a, r);
    if (qt * ppt >= ql) return;
    const int S = a.split_tokens;
    const int nsplit = (ctx + S - 1) / S;
    if (split >= nsplit) return;
    const int lane = threadIdx.x & 63;
    const int64_t pos0 = prefix_len(a.q_lens, r, lane) + (int64_t)qt * ppt;   // packed row of the tile's first position
    const int h0 = hk * G;                             // first query head of the group

    // this split's pages: [kv_begin, kv_end) is page-aligned at its start
    // and spans at most kChunkMaxSplit keys (the plan caps the split size)
    const int kb = split * S, ke = min(ctx, (split + 1) * S);
    const int p0 = kb / BS, np = (ke - 1) / BS - p0 + 1;
    const int32_t* table = a.block_table + (int64_t)r * a.max_blocks_per_seq;
    for (int i = threadIdx.x; i < np; i += 64 * NW) ptab[i] = table[p0 + i];
    __syncthreads();
    // decode-length rows (KIND 1 by default) read each K/V tile in one
    // workgroup; chunks share them between the query tiles of a request
    PagedKV<D, BS, KIND == 1> kv;
    kv.kbase = (const char*)a.k_pool + (int64_t)hk * BS * D * 2;
    kv.vbase = (const char*)a.v_pool + (int64_t)hk * BS * D * 2;
    kv.ptab = ptab;
    kv.p0 = p0;
    kv.blk_bytes = a.kv_block_stride * 2;

    TileProblem P;
    P.q = (const char*)a.q + (pos0 * a.H + h0) * D * 2;
    P.q_stride = (int64_t)a.H * D * 2;
    P.q_hstride = D * 2;
    P.rows_per_pos = G;
    P.n_rows = min(ppt, ql - qt * ppt) * G;
    P.q_pos0 = ctx - ql + qt * ppt;
    P.causal = 1;
    P.kv_begin = kb;
    P.kv_end = ke;
    TileOut out;
    if (nsplit == 1) {
        out.o = (char*)a.o + (pos0 * a.H + h0) * D * 2;
        out.o_stride = (int64_t)a.H * D * 2;
        out.o_hstride = D * 2;
        out.lse = a.lse ? a.lse + pos0 * a.H + h0 : nullptr;
        out.lse_stride = a.H;
        out.lse_hstride = 1;
        out.fp32_out = 0;
    } else {
        const int64_t slot = (((int64_t)r * a.max_q_len + qt * ppt) * a.H + h0) * a.max_splits + split;
        out.o = (char*)(a.ws_o + slot * D);
        out.o_stride = (int64_t)a.H * a.max_splits * D * 4;
        out.o_hstride = (int64_t)a.max_splits * D * 4;
        out.lse = a.ws_lse + slot;
        out.lse_stride = (int64_t)a.H * a.max_splits;
        out.lse_hstride = a.max_splits;
        out.fp32_out = 1;
    }
    if constexpr (KIND != 0) run_pipe_tile<D, NW>(P, kv, out, a.scale * kLog2e, pbuf);
    else run_query_tile<D>(P, kv, out, a.scale * kLog2e, buf);
}

// ============================================================================
// Combine for few splits (at most kCombineHeadsMaxSplits, e.g. chunked
// prefill): M = max_s lse_s, L = M + ln sum_s exp(lse_s - M),
// O = sum_s exp(lse_s - L) O_s, for every (request, query row, head) whose
// context was split.  One wave per (request, query row, group of 64 / (d/8)
// heads): d/8 lanes per head, 8 channels (two 16-byte loads of the fp32
// partial) per lane.  Each lane walks its head's log-sum-exps itself (a few
// values, the same for the lanes of a head), so no cross-lane reduction sits
// between the memory round trips, and the partial rows are read eight splits
// per batch with all their loads in flight; O is summed split by split in
// ascending order.
// ============================================================================
template <int D>
__global__ __launch_bounds__(256) void paged_combine_heads_kernel(PagedArgs a)
{
    constexpr int LPH = D / 8;          // lanes per head
    constexpr int HPW = 64 / LPH;       // heads per wave
    constexpr int BATCH = 8;            // splits whose partial rows are loaded together
    const int lane = threadIdx.x & 63;
    const int sub = lane / LPH, c = lane % LPH;
    const int hgroups = (a.H + HPW - 1) / HPW;
    const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t n_waves = (int64_t)a.num_seqs * a.max_q_len * hgroups;
    if (wid >= n_waves) return;
    const int hg = (int)(wid % hgroups);
    const int i = (int)((wid / hgroups) % a.max_q_len);
    const int r = (int)(wid / ((int64_t)hgroups * a.max_q_len));
    const int ctx = req_ctx(a, r), ql = a.q_lens[r];
    if (i >= ql) return;                                   // uniform over the wave
    const int nsplit = (ctx + a.split_tokens - 1) / a.split_tokens;
    if (nsplit <= 1) return;
    const int64_t row = prefix_len(a.q_lens, r, lane) + i;  // whole wave, one request
    const int h = hg * HPW + sub;
    if (h >= a.H) return;
    const int64_t slot0 = (((int64_t)r * a.max_q_len + i) * a.H + h) * a.max_splits;
    const float* lse_s = a.ws_lse + slot0;
    float M = -INFINITY;
    for (int s = 0; s < nsplit; ++s) M = fmaxf(M, lse_s[s]);
    float sum = 0.f;
    for (int s = 0; s < nsplit; ++s) sum += expf(lse_s[s] - M);
    const float Lse = M + logf(sum);
    const float* os = a.ws_o + slot0 * D + c * 8;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    int s = 0;
    for (; s + BATCH <= nsplit; s += BATCH) {
        f32x4 x0[BATCH], x1[BATCH];
        float wgt[BATCH];
#pragma unroll
        for (int u = 0; u < BATCH; ++u) {
            x0[u] = *(const f32x4*)(os + (int64_t)(s + u) * D);
            x1[u] = *(const f32x4*)(os + (int64_t)(s + u) * D + 4);
            wgt[u] = expf(lse_s[s + u] - Lse);
        }
#pragma unroll
        for (int u = 0; u < BATCH; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc0[e] = __builtin_fmaf(wgt[u], x0[u][e], acc0[e]);
                acc1[e] = __builtin_fmaf(wgt[u], x1[u][e], acc1[e]);
            }
    }
    for (; s < nsplit; ++s) {
        const f32x4 x0 = *(const f32x4*)(os + (int64_t)s * D);
        const f32x4 x1 = *(const f32x4*)(os + (int64_t)s * D + 4);
        const float wgt = expf(lse_s[s] - Lse);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            acc0[e] = __builtin_fmaf(wgt, x0[e], acc0[e]);
            acc1[e] = __builtin_fmaf(wgt, x1[e], acc1[e]);
        }
    }
    u32x4 packed;
    packed[0] = pack_bf16(acc0[0], acc0[1]);
    packed[1] = pack_bf16(acc0[2], acc0[3]);
    packed[2] = pack_bf16(acc1[0], acc1[1]);
    packed[3] = pack_bf16(acc1[2], acc1[3]);
    *(u32x4*)((__bf16*)a.o + (row * a.H + h) * D + c * 8) = packed;
    if (a.lse && c == 0) a.lse[row * a.H + h] = Lse;
}

// ============================================================================
// Combine for many splits (decode): one wave per (request, query row, head)
// whose context was split.
// M = max_s lse_s, L = M + ln sum_s exp(lse_s - M), O = sum_s exp(lse_s - L) O_s.
// Lane s of the wave computes the weight of split s (64 splits at a time) and
// the partial rows are read eight splits per batch, all eight loads in flight
// together; O is still summed split by split in ascending order.
// ============================================================================
template <int D>
__global__ __launch_bounds__(256) void paged_combine_kernel(PagedArgs a)
{
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t n_items = (int64_t)a.num_seqs * a.max_q_len * a.H;
    if (item >= n_items) return;
    const int h = (int)(item % a.H);
    const int i = (int)((item / a.H) % a.max_q_len);
    const int r = (int)(item / ((int64_t)a.H * a.max_q_len));
    const int ctx = req_ctx(a, r), ql = a.q_lens[r];
    if (i >= ql) return;
    const int nsplit = (ctx + a.split_tokens - 1) / a.split_tokens;
    if (nsplit <= 1) return;
    const int64_t slot0 = (((int64_t)r * a.max_q_len + i) * a.H + h) * a.max_splits;
    float M = -INFINITY;
    for (int s = lane; s < nsplit; s += 64) M = fmaxf(M, a.ws_lse[slot0 + s]);
    M = wave_max(M);
    float sum = 0.f;
    for (int s = lane; s < nsplit; s += 64) sum += expf(a.ws_lse[slot0 + s] - M);
    sum = wave_sum(sum);
    const float Lse = M + logf(sum);
    const int64_t row = prefix_len(a.q_lens, r, lane) + i;
    __bf16* orow = (__bf16*)a.o + (row * a.H + h) * D;
    constexpr int CPL = D / 64;      // channels per lane: lane and lane + 64
    constexpr int BATCH = 8;         // splits whose partial rows are loaded together
    float acc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) acc[c] = 0.f;
    for (int s0 = 0; s0 < nsplit; s0 += 64) {
        const int n = min(64, nsplit - s0);
        const float wl = (lane < n) ? expf(a.ws_lse[slot0 + s0 + lane] - Lse) : 0.f;
        const float* os = a.ws_o + (slot0 + s0) * D + lane;
        int s = 0;
        for (; s + BATCH <= n; s += BATCH) {
            float x[BATCH][CPL];
#pragma unroll
            for (int u = 0; u < BATCH; ++u)
#pragma unroll
                for (int c = 0; c < CPL; ++c) x[u][c] = os[(s + u) * D + 64 * c];
#pragma unroll
            for (int u = 0; u < BATCH; ++u) {
                const float wgt = __shfl(wl, s + u, 64);
#pragma unroll
                for (int c = 0; c < CPL; ++c) acc[c] = __builtin_fmaf(wgt, x[u][c], acc[c]);
            }
        }
        for (; s < n; ++s) {
            const float wgt = __shfl(wl, s, 64);
#pragma unroll
            for (int c = 0; c < CPL; ++c) acc[c] = __builtin_fmaf(wgt, os[s * D + 64 * c], acc[c]);
        }
    }
#pragma unroll
    for (int c = 0; c < D / 64; ++c) orow[lane + 64 * c] = (__bf16)acc[c];
    if (a.lse && lane == 0) a.lse[row * a.H + h] = Lse;
}

// ============================================================================
// Gather: one workgroup per (request, page, head); copies the page's [bs, d]
// K and V slabs (bytes as stored) to packed [sum(ctx), H, d] outputs.
// ============================================================================
__global__ __launch_bounds__(256) void paged_gather_kernel(GatherArgs a)
{
    const int max_pages = (a.max_ctx_len + a.block_size - 1) / a.block_size;
    int bid = blockIdx.x;
    const int h = bid % a.H;
    bid /= a.H;
    const int pg = bid % max_pages;
    const int r = bid / max_pages;
    const int ctx = a.ctx_lens[r];
    if (pg * a.block_size >= ctx) return;
    const int lane = threadIdx.x & 63;
    const int64_t tok0 = prefix_len(a.ctx_lens, r, lane);
    const int64_t pb = a.block_table[(int64_t)r * a.max_blocks_per_seq + pg];
    const int row_bytes = a.d * a.elem_bytes;
    const int chunks_per_row = row_bytes / 16;
    const int64_t src_off = pb * a.kv_block_stride * a.elem_bytes + (int64_t)h * a.block_size * row_bytes;
    for (int u = threadIdx.x; u < a.block_size * chunks_per_row; u += blockDim.x) {
        const int tok = u / chunks_per_row, ch = u % chunks_per_row;
        const int t = pg * a.block_size + tok;
        if (t >= ctx) continue;
        const int64_t dst = ((tok0 + t) * a.H + h) * (int64_t)row_bytes + ch * 16;
        *(u32x4*)((char*)a.k_out + dst) = *(const u32x4*)((const char*)a.k_pool + src_off + (int64_t)tok * row_bytes + ch * 16);
        *(u32x4*)((char*)a.v_out + dst) = *(const u32x4*)((const char*)a.v_pool + src_off + (int64_t)tok * row_bytes + ch * 16);
    }
}

// ============================================================================
// host side
// ============================================================================
// The combine of few splits per row (chunked prefill: C5 has at most 5; the
// 64-request decode on the decode MFMA kernel 8) runs lane groups per head,
// each lane walking its head's log-sum-exps itself; with many splits (the
// vector decode kernel's: up to 64) a wave per head reads them in parallel
// (same-machine A/B: heads kernel C5 call 920 -> 939 TFLOP/s, but 64-request
// decode on the vector kernel, 43 splits, 5.75 -> 5.69 TB/s).
constexpr int kCombineHeadsMaxSplits = 8;

PagedPlan plan_paged(int num_seqs, int H, int H_kv, int d, int block_size, int max_q_len, int max_ctx_len,
                     const attn_launch_opts_t& opts)
{
    PagedPlan p{};
    const int G = H / H_kv;
    // The vector decode kernel serves short queries of plain or lightly
    // grouped heads; from groups of kDecodeMfmaGroup heads up, the group's
    // rows go to the matrix cores: for batches of many (request, K/V head)
    // pairs the decode MFMA kernel, while the rows fit its 16, else the tile
    // kernel.  (Decode on 32 query heads / 4 K/V heads, contexts U[512,16384],
    // 16-token pages, TB/s for the tile kernel / the decode MFMA kernel: 64
    // requests 4.90 / 4.72, 256 requests 4.76 / 5.32, 512 requests 5.13 /
    // 5.22.)
    // Below kDecodeMfmaGroup heads per group the vector kernel is the
    // default, except where the decode MFMA kernel (its K/V loads
    // non-temporal, like the vector kernel's) measured faster: several query
    // positions (the vector kernel reads every page once per query row),
    // 32-token pages (two pages per lane crowd the vector kernel's
    // registers), and plain heads at d = 128 on batches of many pairs.  (Same
    // machine, 32 heads, contexts U[512,16384], TB/s vector / MFMA: 64 requests
    // 6.21 / 6.40, 16 requests 5.94 / 6.19, 256 requests 6.11 / 6.35, 8
    // requests 5.47 / 5.24; 32-token pages 4.73 / 6.48; 4 query positions
    // 1.55 / 5.77; d = 64 6.56 / 6.19; 16 K/V heads 6.42 / 6.06.)
    // From groups of kDecodeMfmaGroup heads up, the tile kernel leads up to
    // 512 pairs (GQA-8, 128 requests: tile 5.41, decode MFMA 5.27 TB/s) and
    // the decode MFMA kernel from 1024 (256 requests: 4.27 / 5.59).
    const bool dec_rows = (int64_t)max_q_len * G <= kDecMfmaRows;
    const int64_t pairs = (int64_t)num_seqs * H_kv;
    if (max_q_len <= kDecodeMaxQ && G < kDecodeMfmaGroup)
        p.path = (dec_rows && (max_q_len > 1 || block_size == 32 || (G == 1 && d == 128 && pairs >= kDecMfmaMinPairs)))
                     ? 2 : 0;
    else
        p.path = (dec_rows && pairs >= kDecMfmaMinPairsGrouped) ? 2 : 1;
    if ((opts.paged_path == 0 && max_q_len <= kDecodeMaxQ) || opts.paged_path == 1 ||
        (opts.paged_path == 2 && dec_rows))
        p.path = opts.paged_path;
    const int64_t rows = (int64_t)num_seqs * max_q_len;
    // decode workgroups serve gc query heads of one K/V group (the largest of
    // 8, 4, 2, 1 that divides the group; at most 4 with 32-token pages, whose
    // in-flight page registers leave less room)
    p.gc = 1;
    for (int c = (block_size == 32 ? 4 : 8); c > 1; c >>= 1)
        if (G % c == 0) {
            p.gc = c;
            break;
        }
    const int hc = opts.paged_decode_heads;
    if (hc == 1 || hc == 2 || hc == 4 || hc == 8)
        if (G % hc == 0 && !(block_size == 32 && hc == 8)) p.gc = hc;
    p.n_chunks = G / p.gc;
    int S;
    if (p.path == 0) {
        // decode: 4 waves x 6 pages of 16 tokens per split (measured on the
        // 64-request, 16-token-page decode batch: 384-token splits 5.90 TB/s,
        // 352 5.90, 256 5.77, 448 5.86, 512 5.35), 4 pages of 32 tokens;
        // halved while the batch would leave the chip short of workgroups,
        // down to 1 page per wave (2 for a workgroup serving several query
        // heads)
        const int64_t items = rows * H_kv * p.n_chunks;
        S = 4 * block_size * (block_size == 16 ? 6 : 4);
        const int s_min = (p.gc > 1 ? 2 : 1) * 4 * block_size;
        while (S > s_min && items * ((max_ctx_len + S - 1) / S) < 4096) S /= 2;
        if (S < s_min) S = s_min;
        p.nqt = 1;
        p.tile_kernel = 0;
    } else if (p.path == 2) {
        // decode MFMA kernel: 4 waves x 4 tiles of 16 keys, doubled while the
        // batch keeps the chip busy, up to 128 pages (the block-table entries
        // of a split sit in two registers) and 2048 keys, the last doubling
        // only from 1024 pairs (2048-key against 1024-key splits, TB/s: 64
        // requests x 32 heads 6.22 / 6.21-6.44, 256 x 32 6.52 / 6.37, 4 query
        // positions 6.02 / 5.79, GQA-8 256 requests 5.59 / 5.25; 16 x 32
        // heads 5.90 / 6.03-6.24)
        const int64_t items = (int64_t)num_seqs * H_kv;
        S = 256;
        const int s_max = min(128 * block_size, 2048);
        while (S < s_max && items * ((max_ctx_len + 2 * S - 1) / (2 * S)) >= 2048 && (S < 1024 || items >= 1024))
            S *= 2;
        p.nqt = 1;
        p.tile_kernel = 0;
    } else {
        // The plain key loop on 128-row workgroups (three per CU) unless asked
        // otherwise.  256-row workgroups (eight waves, the pipelined loop, one
        // per CU) read each K/V tile once for twice the rows but keep the
        // matrix cores less busy: 8 x 512-row chunks on 32 heads, contexts
        // of 9-33K keys, 128 rows 949 TFLOP/s with K/V fetched 1.27x the
        // algorithmic bytes (the four tiles of a request share it in L2 in
        // part), 256 rows 879 TFLOP/s at 1.00x.
        // Decode-length rows (one wave of the workgroup has rows) take the
        // pipelined loop: two workgroups per CU with two tiles in flight each
        // keep more K/V in flight than three with one (64 requests, 32 query
        // heads on 4 K/V heads: 4.92 against 4.76 TB/s).
        p.tile_kernel = (opts.paged_tile_kernel >= 0) ? opts.paged_tile_kernel : (max_q_len <= kDecodeMaxQ ? 1 : 0);
        const int ppt = (p.tile_kernel == 2 ? 2 * kTileRows : kTileRows) / G;   // query positions per tile
        p.nqt = (max_q_len + ppt - 1) / ppt;
        // the split plan counts 128-row tiles whatever the workgroup size, so
        // both sizes split the context alike (and give the same bits)
        const int ppt128 = kTileRows / G;
        const int64_t items = (int64_t)num_seqs * ((max_q_len + ppt128 - 1) / ppt128) * H_kv;
        // Decode-length queries (grouped heads on this path) leave one wave of
        // the tile with rows, so a workgroup is latency-bound and more, shorter
        // splits keep more of them in flight; longer queries have full tiles
        // and want fewer partials to combine.  The split count per (request,
        // K/V head, query tile) brings the grid to about `target` items, in
        // whole 64-key units between 1024 and 8192 keys (64 requests x 4 K/V
        // heads, 16-token pages, one query: 1280-key splits 4.84 TB/s, 1024
        // 4.75, 1536 4.54, 2048 3.50; 8 requests x 512 rows: 8192).
        const int64_t target = (max_q_len <= kDecodeMaxQ) ? 3200 : 2048;
        const int64_t per = (target + items - 1) / items;              // splits per item
        int64_t s = (max_ctx_len + per - 1) / per;
        s = (s + 63) / 64 * 64;
        S = (int)(s < 1024 ? 1024 : (s > 8192 ? 8192 : s));
    }
    if (opts.paged_split_tokens > 0) S = opts.paged_split_tokens;
    // a tile-path workgroup stages its split's block-table entries in LDS, a
    // decode-MFMA wave holds them in two registers
    if (p.path == 1 && S > kChunkMaxSplit) S = kChunkMaxSplit;
    if (p.path == 2 && S > 128 * block_size) S = 128 * block_size;
    // whole pages; on the tile path a multiple of 64 keys (whole pages of 16
    // or 32 tokens, so every split starts on a page boundary)
    const int unit = (p.path != 1) ? block_size : (block_size > 64 ? block_size : 64);
    S = ((S + unit - 1) / unit) * unit;
    p.split_tokens = S;
    p.max_splits = (max_ctx_len + S - 1) / S;
    if (p.max_splits < 1) p.max_splits = 1;
    if (p.max_splits > 1) {
        const int64_t slots = rows * H * p.max_splits;
        p.ws_o_bytes = (size_t)(slots * d * 4);
        p.ws_lse_bytes = (size_t)(slots * 4);
        p.ws_o_bytes = (p.ws_o_bytes + 255) / 256 * 256;
        p.ws_bytes = p.ws_o_bytes + p.ws_lse_bytes;
    }
    return p;
}

template <int D, int BS>
static int launch_paged_t(const PagedArgs& a, const PagedPlan& plan, hipStream_t stream)
{
    // the combine's grid is checked before the partial kernel is launched
    const int64_t comb_items = (int64_t)a.num_seqs * a.max_q_len * a.H;
    const int64_t comb_waves = (int64_t)a.num_seqs * a.max_q_len * ((a.H + 64 / (D / 8) - 1) / (64 / (D / 8)));
    if (a.max_splits > kCombineHeadsMaxSplits && !grid_fits((comb_items + 3) / 4, 256)) return -2;
    if (a.max_splits > 1 && a.max_splits <= kCombineHeadsMaxSplits && !grid_fits((comb_waves + 3) / 4, 256))
        return -2;
    if (plan.path == 2) {
        const int64_t grid = (int64_t)a.num_seqs * a.H_kv * a.max_splits;
        if (!grid_fits(grid, 256)) return -2;
        hipLaunchKernelGGL((paged_decode_mfma_kernel<D, BS>), dim3((unsigned)grid), dim3(256), 0, stream, a);
    } else if (plan.path == 0) {
        const int64_t grid = (int64_t)a.num_seqs * a.max_q_len * a.H_kv * plan.n_chunks * a.max_splits;
        if (!grid_fits(grid, 256)) return -2;
        const dim3 g((unsigned)grid), b(256);
        if (plan.gc == 8) hipLaunchKernelGGL((paged_decode_kernel<D, BS, 8>), g, b, 0, stream, a);
        else if (plan.gc == 4) hipLaunchKernelGGL((paged_decode_kernel<D, BS, 4>), g, b, 0, stream, a);
        else if (plan.gc == 2) hipLaunchKernelGGL((paged_decode_kernel<D, BS, 2>), g, b, 0, stream, a);
        else hipLaunchKernelGGL((paged_decode_kernel<D, BS, 1>), g, b, 0, stream, a);
    } else {
        const int64_t pairs = (int64_t)a.num_seqs * a.H_kv;
        const int64_t per_pair = (int64_t)plan.nqt * a.max_splits;
        const int64_t n_work = pairs * per_pair;
        int map = (pairs >= 8 * kChunkPairsPerXcd) ? kMapPairs : kMapItems;
        if (a.tile_map >= kMapRanges && a.tile_map <= kMapItems) map = a.tile_map;
        const int64_t grid = (map == kMapPairs) ? (pairs + 7) / 8 * 8 * per_pair
                           : (map == kMapRanges) ? (n_work + 7) / 8 * 8 : n_work;
        if (n_work > (int64_t)INT32_MAX || !grid_fits(grid, plan.tile_kernel == 2 ? 512 : 256)) return -2;
        if (plan.tile_kernel == 2)
            hipLaunchKernelGGL((paged_chunk_kernel<D, BS, 2>), dim3((unsigned)grid), dim3(512), 0, stream, a,
                               (int)n_work, map);
        else if (plan.tile_kernel == 1)
            hipLaunchKernelGGL((paged_chunk_kernel<D, BS, 1>), dim3((unsigned)grid), dim3(256), 0, stream, a,
                               (int)n_work, map);
        else
            hipLaunchKernelGGL((paged_chunk_kernel<D, BS, 0>), dim3((unsigned)grid), dim3(256), 0, stream, a,
                               (int)n_work, map);
    }
    if (a.max_splits > kCombineHeadsMaxSplits)
        hipLaunchKernelGGL((paged_combine_kernel<D>), dim3((unsigned)((comb_items + 3) / 4)), dim3(256), 0, stream, a);
    else if (a.max_splits > 1)
        hipLaunchKernelGGL((paged_combine_heads_kernel<D>), dim3((unsigned)((comb_waves + 3) / 4)), dim3(256), 0,
                           stream, a);
    return 0;
}

int launch_paged(const PagedArgs& a, const PagedPlan& plan, hipStream_t stream)
{
    int rc;
    if (a.d == 128) {
        if (a.block_size == 16) rc = launch_paged_t<128, 16>(a, plan, stream);
        else rc = launch_paged_t<128, 32>(a, plan, stream);
    } else {
        if (a.block_size == 16) rc = launch_paged_t<64, 16>(a, plan, stream);
        else rc = launch_paged_t<64, 32>(a, plan, stream);
    }
    if (rc) return rc;
    return hipGetLastError() == hipSuccess ? 0 : -8;
}

int launch_gather(const GatherArgs& a, hipStream_t stream)
{
    const int max_pages = (a.max_ctx_len + a.block_size - 1) / a.block_size;
    const int64_t grid = (int64_t)a.num_seqs * max_pages * a.H;
    if (!grid_fits(grid, 256)) return -2;
    hipLaunchKernelGGL(paged_gather_kernel, dim3((unsigned)grid), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // namespace attn
