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
//  * K tiles sit in LDS row-major; V tiles are written to LDS transposed
//    (d-major, keys contiguous, in the permuted order) so that each lane reads
//    its 8 keys of one d-column with a single 16-byte LDS read.  Both tiles use
//    an XOR swizzle of 16-byte chunks so that 16 consecutive lanes hit 16
//    distinct chunks of a 256-byte LDS line (no bank conflicts on the reads).
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

__device__ __forceinline__ float xor32(float x)
{
    return __shfl_xor(x, 32, 64);
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
    static constexpr int LDS_K = BN * D * 2;
    static constexpr int LDS_V = BN * D * 2;
    static_assert(BN * KCPR % kThreads == 0, "K tile must split evenly");
    static_assert(V_QUADS <= kThreads, "one V block per thread at most");
};

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
        *(u32x4*)(lds_k + swz(row, chunk, C::KCPR)) = st.k[i];
    }
    if (tid < C::V_QUADS) {
        int kq = tid / (D / 8), dof = tid % (D / 8);
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

// State of one wave: 32 queries, O^T accumulators, running max / sum.
template <int D>
struct WaveState {
    f32x16 o[TileCfg<D>::DBLK];
    float m;      // running max of the raw (unscaled) scores of this lane's query
    float l;      // running sum of this lane-half's rounded probabilities
};

// One key tile for one wave.
//  qf       : Q^T operand fragments (bf16x8 per 16-wide d step)
//  c2       : scale * log2(e)
//  key0     : absolute key index of tile row 0
//  q_abs    : absolute position of this lane's query (for the causal test)
//  kv_len   : keys >= kv_len are masked
//  masked   : whether any mask test is needed for this wave on this tile
template <int D>
__device__ __forceinline__ void tile_step(WaveState<D>& ws, const bf16x8 (&qf)[TileCfg<D>::KSTEPS],
                                          const char* lds_k, const char* lds_v, int lane, float c2,
                                          int key0, int q_lim, bool masked)
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
            u32x4 a = *(const u32x4*)(lds_k + swz(kb * 32 + r32, ks * 2 + g, C::KCPR));
            acc = mfma32(as_bf16x8(a), qf[ks], acc);
        }
        s[kb] = acc;
    }
    // ---- mask + running max ------------------------------------------------
    // key of accumulator register i of block kb: kb*32 + (i/4)*8 + g*4 + i%4
    float mt = -INFINITY;
    if (masked) {
#pragma unroll
        for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int key = key0 + kb * 32 + (i >> 2) * 8 + g * 4 + (i & 3);
                if (key >= q_lim) s[kb][i] = -INFINITY;
                mt = fmaxf(mt, s[kb][i]);
            }
    } else {
#pragma unroll
        for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) mt = fmaxf(mt, s[kb][i]);
    }
    mt = fmaxf(mt, xor32(mt));
    const float m_new = fmaxf(ws.m, mt);
    // scaled maxima; a row that has seen no allowed key keeps max -inf and
    // uses 0 as its offset (all its p are 0 and its O, l are still 0)
    const float ms_new = (m_new == -INFINITY) ? 0.f : m_new * c2;
    const float ms_old = (ws.m == -INFINITY) ? 0.f : ws.m * c2;
    const float alpha = __builtin_amdgcn_exp2f(ms_old - ms_new);
    ws.m = m_new;
    // ---- p = exp2(s*c2 - m), rounded to bf16, summed -------------------------
    uint32_t pk[C::KBLK][8];
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i], c2, -ms_new));
            float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][i + 1], c2, -ms_new));
            if (masked) {
                if (s[kb][i] == -INFINITY) p0 = 0.f;
                if (s[kb][i + 1] == -INFINITY) p1 = 0.f;
            }
            uint32_t w = pack_bf16(p0, p1);
            pk[kb][i >> 1] = w;
            psum += bf16lo(w) + bf16hi(w);
        }
    ws.l = ws.l * alpha + psum;
#pragma unroll
    for (int db = 0; db < C::DBLK; ++db) ws.o[db] *= alpha;
    // ---- O^T += V^T P^T ------------------------------------------------------
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            u32x4 pw;
            pw[0] = pk[kb][4 * h + 0];
            pw[1] = pk[kb][4 * h + 1];
            pw[2] = pk[kb][4 * h + 2];
            pw[3] = pk[kb][4 * h + 3];
            bf16x8 b = as_bf16x8(pw);
            const int chunk = kb * 4 + h * 2 + g;
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db) {
                u32x4 a = *(const u32x4*)(lds_v + swz(db * 32 + r32, chunk, C::VCPR));
                ws.o[db] = mfma32(as_bf16x8(a), b, ws.o[db]);
            }
        }
}

}  // namespace attn
