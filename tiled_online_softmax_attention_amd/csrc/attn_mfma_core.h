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
//  * Each wave owns 32 query rows.  It computes S^T = K Q^T, so
//    the MFMA accumulator puts one query per lane (lane % 32) and that query's
//    keys down the 16 accumulator registers: the running offset, sum and the
//    rescale factor are per-lane scalars, and the two lane halves (lane / 32)
//    hold disjoint key subsets of the same query.
//  * The P^T operand of O^T += V^T P^T is taken straight from the S^T
//    accumulators (8 consecutive registers = 8 keys per lane).  The matching
//    V^T operand -- for each lane one d-column over those 8 keys -- is read
//    from the row-major V tile with two transposing LDS reads
//    (ds_read_b64_tr_b16): in each 16-lane group, lane i receives element j
//    from the 8-byte row segment addressed by lane 4j + i/4, at position i%4.
//  * K and V tiles are copied from global memory straight into LDS
//    (buffer_load_dwordx4 ... lds: lane l of a wave lands at base + 16*l),
//    so no registers stage them; the source each lane fetches is chosen so
//    that the tile lands in the layout its readers want.  K is stored in
//    16-row groups, chunk-major, so the MFMA K reads (16 consecutive rows,
//    one 16-byte chunk) are contiguous; V is row-major with an XOR swizzle
//    that makes the transposing reads (4 consecutive rows x 64 bytes per
//    32-lane pass) conflict-free.
//  * Softmax runs in base 2: scores are scaled by scale*log2(e) inside one FMA
//    and exponentiated with the hardware exp2.  P is rounded to bf16 (round to
//    nearest even) for the MFMA; the running sum adds the fp32 values.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define ATTN_LDS(p) ((__attribute__((address_space(3))) void*)(p))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

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

__device__ __forceinline__ bf16x2 pack2(float a, float b)
{
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return r;
}

__device__ __forceinline__ bf16x8 cat8(bf16x2 a, bf16x2 b, bf16x2 c, bf16x2 d)
{
    bf16x4 lo = __builtin_shufflevector(a, b, 0, 1, 2, 3);
    bf16x4 hi = __builtin_shufflevector(c, d, 0, 1, 2, 3);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Tile geometry: 4 waves, 32-key tiles of two 16-row groups.  Per tile, waves
// 0 and 1 copy the two K groups and waves 2 and 3 the two V groups.  Short
// tiles keep the per-wave registers low enough for three workgroups per CU
// (12 waves), which hides more of the latency of each wave's dependent chain
// (S MFMAs -> max -> exp -> PV MFMAs) than longer tiles at two per CU.
template <int D>
struct TileCfg {
    static constexpr int kWaves = 4;
    static constexpr int kThreads = 64 * kWaves;
    static constexpr int BN = 32;                   // keys per tile
    static constexpr int KCPR = D / 8;              // 16-byte chunks per row
    static constexpr int KSTEPS = D / 16;           // MFMA k-steps for Q K^T
    static constexpr int DBLK = D / 32;             // 32-wide d blocks of O^T
    static constexpr int KBLK = BN / 32;            // 32-key blocks of S^T
    static constexpr int ROW_BYTES = D * 2;
    static constexpr int TILE_BYTES = BN * ROW_BYTES;          // one of K or V
    static constexpr int GROUPS = BN / 16;                     // 16-row groups per tile
    static constexpr int ROWS_PER_DMA = 1024 / ROW_BYTES;      // rows per wave-wide 16 B/lane copy
    static constexpr int COPIES_PER_GROUP = 16 / ROWS_PER_DMA;
    static_assert(kWaves == 2 * GROUPS, "one wave per 16-row group of K or V");
};

// XOR applied to the 16-byte chunk index of V row `row`: 4 consecutive rows
// (4-aligned) map the same 4 logical chunks onto 4 distinct bank groups.
template <int D>
__device__ __forceinline__ uint32_t v_row_xor(uint32_t row)
{
    return (D == 128) ? ((row & 3u) << 2) : (((row >> 1) & 1u) << 2);
}

template <int D>
__device__ __forceinline__ uint32_t v_ofs(uint32_t row, uint32_t chunk)
{
    return row * (uint32_t)TileCfg<D>::ROW_BYTES + ((chunk ^ v_row_xor<D>(row)) << 4);
}

// K tile layout in LDS: 16-row groups, each stored chunk-major (for every
// 16-byte chunk of the row, the 16 rows' copies of it are contiguous).  The
// MFMA K reads (16 consecutive rows, one chunk per 16-lane quarter) then
// touch 256 contiguous bytes: conflict-free without a swizzle, and every
// read of a tile is one per-lane base plus an immediate.
template <int D>
__device__ __forceinline__ uint32_t k_ofs(uint32_t row, uint32_t chunk)
{
    return (row >> 4) * (16u * TileCfg<D>::ROW_BYTES) + chunk * 256u + (row & 15u) * 16u;
}

// Sources of the wave-wide LDS copies (lane l of a copy lands at the copy's
// LDS base + 16*l).  Offsets are bytes from the first row of the wave's
// 16-row group; copy i adds a wave-uniform step.
//  K: copy i fills chunks 4i..4i+3 of the group's 16 rows; lane l lands at
//     row l % 16 of chunk 4i + l / 16.  Step: 4 chunks = 64 source bytes.
//  V: copy i fills rows i*ROWS_PER_DMA onwards (row-major); lane l lands at
//     row i*ROWS_PER_DMA + l / KCPR, physical chunk l % KCPR, which holds
//     logical chunk (l % KCPR) ^ v_row_xor(row).  The XOR only looks at row
//     bits below ROWS_PER_DMA, so it does not depend on i.  Step: 1 KiB.
constexpr uint32_t kKDmaStep = 64;
constexpr uint32_t kVDmaStep = 1024;

// Cache policy (the aux operand of the direct global->LDS copies) for K/V
// that no other workgroup reads: non-temporal.  Streaming reads marked so
// move ~13 % more bytes per second on gfx950 (7.0 against 6.2 TB/s for a
// plain 8 GiB read); K/V that the query tiles of one head or request share
// through L2 must keep the default, which the hint would make miss.
constexpr int kCopyStream = 2;   // nt
template <int D>
__device__ __forceinline__ int k_dma_row(int lane) { return lane & 15; }
template <int D>
__device__ __forceinline__ uint32_t k_dma_col(int lane) { return (uint32_t)(lane >> 4) * 16u; }
template <int D>
__device__ __forceinline__ int v_dma_row(int lane) { return lane / TileCfg<D>::KCPR; }
template <int D>
__device__ __forceinline__ uint32_t v_dma_col(int lane)
{
    return (((uint32_t)(lane % TileCfg<D>::KCPR)) ^ v_row_xor<D>((uint32_t)(lane / TileCfg<D>::KCPR))) * 16u;
}

// State of one wave: 32 queries (one per lane % 32), O^T accumulators, the
// running offset and the running sum.
template <int D>
struct WaveState {
    f32x16 o[TileCfg<D>::DBLK];
    float m;   // offset of this lane's query, raw score units (-inf: none yet)
    float ms;  // the same offset in the exponent's base-2 units, m * c2 (0 while m = -inf)
    float l;   // running sum of this lane-half's probabilities (fp32)
};

// Scores of one key tile: S^T blocks of 32 keys (accumulator register i of
// block kb holds key kb*32 + (i/4)*8 + (lane/32)*4 + i%4 of the tile).
template <int D>
struct TileScores {
    f32x16 s[TileCfg<D>::KBLK];
};

// Exponent headroom of the lazy rescale: the offset m only moves when a
// tile's maximum exceeds it by more than kRescaleLog2 in the base-2 exponent,
// so p = 2^(s*c2 - m*c2) stays <= 2^kRescaleLog2 (well inside fp32 and bf16
// range) and the O/l rescale is skipped on almost every tile.  O and l always
// share the same offset, so the final O/l and LSE = m + ln l are exact.
constexpr float kRescaleLog2 = 8.0f;

// V^T operand of one PV MFMA step for this lane: its d-column, over keys
// row, row+1, row+2, row+3 and row+8 .. row+11 of the tile (row = the lane's
// transposed-read row), read with two transposing LDS reads.
template <int D>
__device__ __forceinline__ bf16x8 v_operand(const char* lds_v, int row, uint32_t col_byte)
{
    typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(lds_v + v_ofs<D>((uint32_t)row, col_byte >> 4) + (col_byte & 15u)));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (lds_i16x4*)(lds_v + v_ofs<D>((uint32_t)row + 8u, col_byte >> 4) + (col_byte & 15u)));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// acc *= alpha, register by register in the accumulator's own registers.
// (Written as a plain vector multiply, the rarely taken rescale branch puts
// the product in fresh registers, and the common path then pays a copy of the
// whole accumulator every tile to merge the two.)
__device__ __forceinline__ void scale_in_place(f32x16& acc, float alpha)
{
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float x = acc[i];
        asm("v_mul_f32 %0, %0, %1" : "+v"(x) : "v"(alpha));
        acc[i] = x;
    }
}

// The tile step of the block-wise forward, in stages: S MFMAs, mask and
// maximum, lazy offset update, exponentials, PV MFMAs.

// S^T = K Q^T for one key tile.  All K fragments of a 32-key block are read
// first, so the LDS latency is paid once per block rather than per MFMA.
template <int D>
__device__ __forceinline__ void qk_tile(TileScores<D>& S, const bf16x8 (&qf)[TileCfg<D>::KSTEPS], const char* lds_k,
                                        int lane)
{
    using C = TileCfg<D>;
    const int g = lane >> 5, r32 = lane & 31;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb) {
        bf16x8 kf[C::KSTEPS];
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks)
            kf[ks] = as_bf16x8(*(const u32x4*)(lds_k + k_ofs<D>(kb * 32 + r32, ks * 2 + g)));
        f32x16 acc = f32x16{};
#pragma unroll
        for (int ks = 0; ks < C::KSTEPS; ++ks) acc = mfma32(kf[ks], qf[ks], acc);
        S.s[kb] = acc;
    }
}

// Mask (MASKED: keys >= q_lim become -inf) and the tile maximum of this
// lane's query over both lane halves.
//  key0  : absolute key index of tile row 0
//  q_lim : this lane's query sees keys < q_lim
template <int D, bool MASKED>
__device__ __forceinline__ float tile_max(TileScores<D>& S, int lane, int key0, int q_lim)
{
    using C = TileCfg<D>;
    const int g = lane >> 5;
    if (MASKED) {
        const int lim_rel = q_lim - key0 - g * 4;
#pragma unroll
        for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int off = kb * 32 + (i >> 2) * 8 + (i & 3);
                S.s[kb][i] = (off < lim_rel) ? S.s[kb][i] : -INFINITY;
            }
    }
    // one chain of three-operand maxima (v_max3_f32 takes two new scores each)
    float x = fmaxf(S.s[0][0], S.s[0][1]);
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int i = (kb == 0) ? 2 : 0; i < 16; i += 2) x = fmaxf(fmaxf(x, S.s[kb][i]), S.s[kb][i + 1]);
    return half_max(x);
}

// Lazy offset update (wave-uniform decision): when some query's tile maximum
// mt exceeds its offset by more than the headroom, move the offsets and
// rescale O and l by exp2((m_old - m_new) * c2).
//  c2  : scale * log2(e) (> 0);  thr = kRescaleLog2 / c2 in raw score units
template <int D>
__device__ __forceinline__ void update_offset(WaveState<D>& ws, float mt, float c2, float thr)
{
    using C = TileCfg<D>;
    if (__builtin_amdgcn_ballot_w64(mt > ws.m + thr) != 0) {
        const float m_new = fmaxf(ws.m, mt);
        const float alpha = (ws.m == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ws.m - m_new) * c2);
        ws.m = m_new;
        ws.ms = (m_new == -INFINITY) ? 0.f : m_new * c2;
        ws.l *= alpha;
#pragma unroll
        for (int db = 0; db < C::DBLK; ++db) scale_in_place(ws.o[db], alpha);
    }
}

// p = exp2(s*c2 - m*c2), rounded to bf16 (packed in pairs, the P^T operand
// layout) for the P V product; l += the fp32 values of p, added one by one in
// key order.  (The bf16 dot-product instruction that would add the rounded
// pairs in one step occupies the matrix pipe -- it never issues beside an
// MFMA -- while plain fp32 adds do.)  (c2 > 0 always: a zero scale is passed
// as a tiny positive c2, which gives the same p = 1 for every allowed key and
// keeps exp2(-inf) = 0 for masked ones.)
template <int D>
__device__ __forceinline__ void exp_tile(bf16x2 (&pk)[TileCfg<D>::KBLK][8], const TileScores<D>& S, WaveState<D>& ws,
                                         float c2)
{
    using C = TileCfg<D>;
    const float ms = ws.ms;
    float l = ws.l;
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
            const float e0 = __builtin_amdgcn_exp2f(__builtin_fmaf(S.s[kb][i], c2, -ms));
            const float e1 = __builtin_amdgcn_exp2f(__builtin_fmaf(S.s[kb][i + 1], c2, -ms));
            pk[kb][i >> 1] = pack2(e0, e1);
            l += e0;
            l += e1;
        }
    ws.l = l;
}

// O^T += V^T P^T for one key tile.
// Lane (16-lane group G = lane/16, i = lane%16) addresses V row k0 + i/4 and
// the 4 channels d0 + 4*(i%4), d0 = db*32 + (G%2)*16, with
// k0 = kb*32 + 16h + 4g (+8 for the second read); the transposing read hands
// it keys k0..k0+3 of channel d0 + i -- the keys its P^T registers
// 8h..8h+7 hold.
template <int D>
__device__ __forceinline__ void pv_tile(WaveState<D>& ws, const bf16x2 (&pk)[TileCfg<D>::KBLK][8], const char* lds_v,
                                        int lane)
{
    using C = TileCfg<D>;
    const int g = lane >> 5;
    const int tr_row = g * 4 + ((lane & 15) >> 2);
    const uint32_t tr_col = (uint32_t)((((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2);
#pragma unroll
    for (int kb = 0; kb < C::KBLK; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const bf16x8 b = cat8(pk[kb][4 * h + 0], pk[kb][4 * h + 1], pk[kb][4 * h + 2], pk[kb][4 * h + 3]);
#pragma unroll
            for (int db = 0; db < C::DBLK; ++db) {
                const bf16x8 a = v_operand<D>(lds_v, kb * 32 + 16 * h + tr_row, tr_col + db * 64);
                ws.o[db] = mfma32(a, b, ws.o[db]);
            }
        }
}

}  // namespace attn
