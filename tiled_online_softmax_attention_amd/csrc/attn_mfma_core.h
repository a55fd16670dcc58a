// attn_mfma_core.h -- bf16 MFMA tile core of the fused attention forward for
// gfx950 (CDNA4), shared by the contiguous prefill kernel and the paged
// chunked-prefill kernel.
//
// The computation is the block-wise forward with online softmax of
// "Flash Attention and Paged Attention" (section 2): for each key tile,
// S = Q K^T * scale, m_new = max(m, rowmax S), p = exp(S - m_new),
// l = exp(m - m_new) l + sum p, O = exp(m - m_new) O + p V, and O / l once at
// the end.  Here it is laid out for 64-wide wavefronts and 32x32x16 bf16 MFMA:
//
//  * Each wave owns 32 query rows.  It computes S^T = K Q^T, so the MFMA
//    accumulator puts one query per lane (lane % 32) and that query's keys
//    down the 16 accumulator registers: the running max, sum and the rescale
//    factor are per-lane scalars, and the two lane halves (lane / 32) hold
//    disjoint key subsets of the same query.
//  * The P^T operand of O^T += V^T P^T is taken straight from the S^T
//    accumulators (8 consecutive registers = 8 keys per lane); the key order
//    inside each 16-key MFMA step is permuted consistently on the V side, which
//    leaves the contraction unchanged.
//  * K tiles sit in LDS row-major with rows padded by 16 bytes, so 16
//    consecutive rows start in 16 distinct bank groups and every read address
//    is one base plus an immediate.  V tiles are written to LDS transposed
//    (d-major, keys contiguous, in the permuted order) so that each lane reads
//    its 8 keys of one d-column with a single 16-byte LDS read; the V^T rows
//    use an XOR swizzle of 16-byte chunks within each 256-byte line.  Reads
//    and the transposing writes are both free of bank conflicts.
//  * Softmax runs in base 2: scores are scaled by scale*log2(e) inside one FMA
//    and exponentiated with the hardware exp2.  P is rounded to bf16 (round to
//    nearest even) for the MFMA and the running sum adds those rounded values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Byte offset of 16-byte chunk `chunk` of LDS row `row` (rows of `cpr` chunks)
// after the XOR swizzle: the linear chunk index is split into 256-byte lines
// of 16 chunks and the in-line index is XORed with the line number (mod 16).
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t chunk, uint32_t cpr)
{
    uint32_t L = row * cpr + chunk;
    return ((L & ~15u) | ((L & 15u) ^ ((L >> 4) & 15u))) * 16u;
}

// Position of key offset o (0..15) inside a 16-key MFMA step of the V^T tile:
// bits 2 and 3 are swapped, so that lane half g finds keys {4g..4g+3} and
// {8+4g..8+4g+3} -- exactly the keys its S^T accumulator registers hold --
// in 8 consecutive slots.
__device__ __forceinline__ uint32_t vperm16(uint32_t o)
{
    return (o & 3u) | ((o & 4u) << 1) | ((o & 8u) >> 1);
}

// max / sum of x over lanes l and l ^ 32 (the two halves holding one
// query's keys), through the gfx950 lane-half swap instead of an LDS permute
__device__ __forceinline__ float half_max(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                    false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float half_sum(float x)
{
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x), __builtin_bit_cast(uint32_t, x),
                                                    false, false);
    return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c)
{
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u)
{
    return __builtin_bit_cast(bf16x8, u);
}

// Pack two fp32 into bf16x2 (RNE) and return the packed bits.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Tile geometry: 4 waves x 32 query rows, 64-key tiles.
template <int D>
struct TileCfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BM = 32 * kWaves;          // query rows per workgroup
    static constexpr int BN = 64;                   // keys per tile
    static constexpr int KCPR = D / 8;              // 16-byte chunks per K row
    static constexpr int VCPR = BN / 8;             // 16-byte chunks per V^T row
    static constexpr int KSTEPS = D / 16;           // MFMA k-steps for Q K^T
    static constexpr int DBLK = D / 32;             // 32-wide d blocks of O^T
    static constexpr int KBLK = BN / 32;            // 32-key blocks of S^T
    static constexpr int K_LOADS = BN * KCPR / kThreads;    // 16 B K loads per thread
    static constexpr int V_QUADS = (BN / 4) * (D / 8);      // 4-key x 8-d V blocks
    static constexpr int KSTRIDE = D * 2 + 16;      // padded K row in LDS (bytes)
    static constexpr int LDS_K = BN * KSTRIDE;
    static constexpr int LDS_V = BN * D * 2;
    static constexpr int LDS_TOTAL = 2 * (LDS_K + LDS_V);   // double-buffered
    static_assert(BN * KCPR % kThreads == 0, "K tile must split evenly");
    static_assert(V_QUADS <= kThreads, "one V block per thread at most");
};

// The 4-key x 8-channel block of the V tile that thread `tid` stages: wave w
// takes channel octets 4w .. 4w+3 for all 16 key quads (lane % 4 picks the
// octet, lane / 4 the quad).  With this order every 32-lane pass of the
// transposing LDS writes hits 32 distinct bank pairs.
__device__ __forceinline__ int vblock_quad(int tid) { return (tid & 63) >> 2; }
__device__ __forceinline__ int vblock_oct(int tid) { return ((tid >> 6) << 2) | (tid & 3); }

// Per-thread registers holding the next K/V tile while the current one is
// being consumed (the global loads are issued one tile ahead).
template <int D>
struct KVStage {
    u32x4 k[TileCfg<D>::K_LOADS];
    u32x4 v[4];
};

// Write the staged K rows (swizzled) and the staged V block (transposed,
// permuted, swizzled) into LDS.
template <int D>
__device__ __forceinline__ void stage_to_lds(const KVStage<D>& st, char* lds_k, char* lds_v, int tid)
{
    using C = TileCfg<D>;
#pragma unroll
    for (int i = 0; i < C::K_LOADS; ++i) {
        int u = i * C::kThreads + tid;
        int row = u / C::KCPR, chunk = u % C::KCPR;
        *(u32x4*)(lds_k + row * C::KSTRIDE + chunk * 16) = st.k[i];
    }
    if (tid < C::V_QUADS) {
        const int kq = vblock_quad(tid), dof = vblock_oct(tid);
        int key0 = kq * 4;                                   // first of 4 keys
        uint32_t kp = (key0 & ~15) | vperm16(key0 & 15);     // permuted slot (4-aligned)
        uint32_t chunk = kp >> 3, half = (kp >> 2) & 1;
        // st.v[r] holds 8 bf16 of key key0 + r for d = dof*8 .. dof*8+7.
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            // d = dof*8 + 2*e2 (low halves) and dof*8 + 2*e2 + 1 (high halves)
            uint32_t a0 = st.v[0][e2], a1 = st.v[1][e2], a2 = st.v[2][e2], a3 = st.v[3][e2];
            u32x2 lo, hi;
            lo[0] = __builtin_amdgcn_perm(a1, a0, 0x05040100u);   // (key0, key1) low halves
            lo[1] = __builtin_amdgcn_perm(a3, a2, 0x05040100u);   // (key2, key3)
            hi[0] = __builtin_amdgcn_perm(a1, a0, 0x07060302u);
            hi[1] = __builtin_amdgcn_perm(a3, a2, 0x07060302u);
            uint32_t d_lo = dof * 8 + 2 * e2, d_hi = d_lo + 1;
            *(u32x2*)(lds_v + swz(d_lo, chunk, C::VCPR) + half * 8) = lo;
            *(u32x2*)(lds_v + swz(d_hi, chunk, C::VCPR) + half * 8) = hi;
        }
    }
}

// State of one wave: 32 queries, O^T accumulators, running offset / sum.
template <int D>
struct WaveState {
    f32x16 o[TileCfg<D>::DBLK];
    float m;      // offset of this lane's query, raw score units (-inf: none yet)
    float l;      // running sum of this lane-half's rounded probabilities
};

__device__ __forceinline__ bf16x2 pack2(float a, float b)
{
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return r;
}

__device__ __forceinline__ bf16x8 cat8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d)
{
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    bf16x4 hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Exponent headroom of the lazy rescale: the offset m only moves when a
// tile's maximum exceeds it by more than kRescaleLog2 in the base-2 exponent,
// so p = 2^(s*c2 - m*c2) stays <= 2^kRescaleLog2 (well inside fp32 and bf16
// range) and the O/l rescale is skipped on almost every tile.  O and l always
// share the same offset, so the final O/l and LSE = m + ln l are exact.
constexpr float kRescaleLog2 = 8.0f;

// One key tile for one wave.
//  qf      : Q^T operand fragments (bf16x8 per 16-wide d step)
//  c2      : scale * log2(e) (> 0);  thr = kRescaleLog2 / c2 in raw score units
//  key0    : absolute key index of tile row 0
//  q_lim   : this lane's query sees keys < q_lim
//  MASKED  : whether any key of this tile may be masked for a lane of the wave
//  (c2 > 0 always: a zero scale is passed as a tiny positive c2, which gives
//  the same p = 1 for every allowed key and keeps exp2(-inf) = 0 for masked ones)
template <int D, bool MASKED>
__device__ __forceinline__ void tile_step(WaveState<D>& ws, const bf16x8 (&qf)[TileCfg<D>::KSTEPS],
                                          const char* lds_k, const char* lds_v, int lane, float c2, float thr,
                                          int key0, int q_lim)
{
    using C = TileCfg<D>;
    const int g = lane >> 5, r32 = lane & 31;
    // ---- S^T = K Q^T --------------------------------------------------------
    f32x16 s[C::KBLK];
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb) {
        f32x16 acc = {};
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) {
            u32x4 a = *(const u32x4*)(lds_k + (kb * 32 + r32) * C::KSTRIDE + (ks * 2 + g) * 16);
            acc = mfma32(as_bf16x8(a), qf[ks], acc);
        }
        s[kb] = acc;
    }
    // ---- mask (diagonal / tail tiles only) and tile maximum -----------------
    // key of accumulator register i of block kb: key0 + kb*32 + (i/4)*8 + g*4 + i%4
    const int lim_rel = q_lim - key0 - g * 4;
    float mt = -INFINITY;
    if (MASKED) {
#pragma unroll
        for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = kb * 32 + (i >> 2) * 8 + (i & 3);
                s[kb][i] = (off < lim_rel) ? s[kb][i] : -INFINITY;
            }
    }
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mt = fmaxf(mt, fmaxf(s[kb][i], s[kb][i + 1]));
    mt = half_max(mt);
    // ---- lazy offset update (wave-uniform decision) --------------------------
    const bool need = mt > ws.m + thr;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = fmaxf(ws.m, mt);
        const float alpha = (ws.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ws.m - m_new) * c2);
        ws.m = m_new;
        ws.l *= alpha;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) ws.o[db] *= alpha;
    }
    const float ms = (ws.m == -INFINITY) ? 0.f : ws.m * c2;
    // ---- p = exp2(s*c2 - ms), rounded to bf16; l += sum of the rounded p -----
    bf16x2 pk[C::KBLK][8];
    const bf16x2 ones = pack2(1.f, 1.f);
    float ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const float t0 = __builtin_fmaf(s[kb][i], c2, -ms);
            const float t1 = __builtin_fmaf(s[kb][i + 1], c2, -ms);
            const bf16x2 w = pack2(__builtin_amdgcn_exp2f(t0), __builtin_amdgcn_exp2f(t1));
            pk[kb][i >> 1] = w;
            if ((i >> 1) & 1) ps1 = __builtin_amdgcn_fdot2_f32_bf16(w, ones, ps1, false);
            else ps0 = __builtin_amdgcn_fdot2_f32_bf16(w, ones, ps0, false);
        }
    ws.l += ps0 + ps1;
    // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x8 b = cat8(pk[kb][4 * h + 0], pk[kb][4 * h + 1], pk[kb][4 * h + 2], pk[kb][4 * h + 3]);
            const int chunk = kb * 4 + h * 2 + g;
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db) {
                u32x4 a = *(const u32x4*)(lds_v + swz(db * 32 + r32, chunk, C::VCPR));
                ws.o[db] = mfma32(as_bf16x8(a), b, ws.o[db]);
            }
        }
}

}  // namespace attn
