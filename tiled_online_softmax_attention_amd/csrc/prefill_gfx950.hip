// prefill_gfx950.hip -- dense / causal prefill attention for gfx950.
//
//  * bf16: fused MFMA kernel, one workgroup of 4 waves per 128-row query tile
//    (or per pair of tiles, see below), K/V streamed through LDS in 32-key
//    tiles, causal key tiles above the diagonal never loaded.  Two key loops:
//    the plain one of attn_mfma_kernel.h (three LDS buffers, three workgroups
//    per CU) for grids of several dispatch rounds, and the software-pipelined
//    one of attn_mfma_pipe.h (four LDS buffers, two workgroups per CU) for
//    grids of about one round, whose few waves per SIMD need the MFMA and
//    softmax work of each wave interleaved (1x32x2048x128 causal: 560 -> 622
//    TFLOP/s; 16x32x8192x128: 1128 against 1111 for the pipelined loop).
//    Both give the same bits.
//  * fp32: a vector-ALU kernel with the same online softmax and 64-key tiles
//    (fp32 storage has no dense matrix path worth using at these sizes).
//
// Work mapping (bf16).  Workgroups are dealt to the 8 XCDs round-robin by
// block id; a causal launch picks one of three tile orders (launch_prefill):
//  * order 0, per-head ranges: the linear id is remapped so that each XCD
//    receives a contiguous range of (batch*head, query tile) work, heaviest
//    tile (most keys) first within each head; the query tiles of a head then
//    share that XCD's L2 for their K/V.  Non-causal launches, whose tiles
//    all weigh the same, always use it.
//  * order 3, tile-major: block id p takes head p % (B*H) and its
//    (p / (B*H))-th heaviest tile -- the heaviest tile of every head first,
//    then the next -- so the longest work starts first everywhere and every
//    XCD gets the same mix of tile weights, whatever B*H is.  All heads are
//    in flight at once, which pays while their K/V fits in the last-level
//    cache: 1x12x16384 870 -> 1036 TFLOP/s, 1x28x8192 853 -> 969, 2x32x8192
//    1000 -> 1045, but 16x32x8192 (2 GB of K/V) 1070 -> 722, and with grouped
//    heads per-head ranges win (their L2 serves a K/V head to all its query
//    heads): 16x32x8192 on 4 K/V heads 1075-1081 against 905-937.
//  * order 1, complementary: for a grid of about one dispatch round (all
//    its workgroups resident, two or three per CU) each XCD's tiles go heavy
//    half descending, then light half ascending, so that the workgroups one
//    CU receives together add up to the same work.
// In "pair" mode a workgroup instead takes tile t and tile n-1-t, so that
// every workgroup does the same number of key tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_mfma_kernel.h"
#include "attn_mfma_pipe.h"
#include "attn_internal.h"

namespace attn {

// K/V rows of one head of a contiguous [B, H, N, d] tensor: the copies
// address the head slab from its base (N * d * 2 < 4 GiB is checked on the
// host), and the descriptor's range check returns zero for rows past N.
template <int D>
struct ContigKV {
    const char* k;   // head base (bytes)
    const char* v;
    uint32_t head_bytes;
    static constexpr int kCopiesAhead = 2;
    __device__ __forceinline__ uint32_t group_bytes() const { return head_bytes; }
    __device__ __forceinline__ const char* k_group(int, int) const { return k; }
    __device__ __forceinline__ const char* v_group(int, int) const { return v; }
    // copies of the key loops: nothing to look up per tile
    struct SrcWin {};
    __device__ __forceinline__ SrcWin empty_win() const { return SrcWin{}; }
    __device__ __forceinline__ void win_update(SrcWin&, const WaveCtx&, int, int) const {}
    __device__ __forceinline__ int copy_src(const SrcWin&, const WaveCtx&, int) const { return 0; }
    template <int NW>
    __device__ __forceinline__ void copy_tile(const WaveCtx& cx, char* buf, int key_base, int) const
    {
        issue_tile_copies_flat<D, NW>(*this, cx, buf, key_base);
    }
};

// Linear work id for this workgroup after the XCD-contiguous remap; the grid
// is padded to a multiple of 8.
__device__ __forceinline__ int xcd_linear_id(int bid, int grid)
{
    const int per = grid >> 3;
    return (bid & 7) * per + (bid >> 3);
}

// KIND 0: the plain key loop (attn_mfma_kernel.h: three LDS buffers, three
// workgroups per CU).  KIND 1: the software-pipelined key loop of
// attn_mfma_pipe.h (four LDS buffers, two workgroups per CU).  (Eight waves
// on 256-row tiles, one workgroup per CU, each K/V tile copied once for 256
// rows, measured slower: 16x32x8192 1081 against 1102 TFLOP/s, 1x32x2048
// 498 against 610, the second for want of two workgroups per CU to balance
// the causal tiles.)
template <int D, bool PAIR, int KIND>
__global__ __launch_bounds__(256, KIND == 0 ? 3 : 2) void prefill_bf16_kernel(PrefillArgs a)
{
    using C = TileCfg<D>;
    constexpr bool PIPE = KIND != 0;
    constexpr int BM = kTileRows;
    __shared__ __attribute__((aligned(16))) char lds0[2 * C::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char lds1[2 * C::TILE_BYTES];
    __shared__ __attribute__((aligned(16))) char lds2[2 * C::TILE_BYTES];
    const TileBuffers buf{lds0, lds1, lds2};
    PipeBuffers pbuf{{lds0, lds1, lds2, nullptr}};
    if constexpr (PIPE) {
        __shared__ __attribute__((aligned(16))) char lds3[2 * C::TILE_BYTES];
        pbuf.b[3] = lds3;
    }
    const int L = xcd_linear_id(blockIdx.x, gridDim.x);
    if (L >= a.n_work && (PAIR || a.order != 3)) return;
    const int nqt = (a.N + BM - 1) / BM;
    const int per_bh = PAIR ? (nqt + 1) / 2 : nqt;
    int bh = L / per_bh, t = L % per_bh;
    if (!PAIR && a.order == 1) {
        // Complementary order: an XCD's share is whole heads; position j of
        // the share takes the (j / heads)-th tile of the sequence heaviest,
        // next heaviest, ... down to the middle, then lightest upwards, so
        // that positions j and j + share/2 (the two workgroups one CU
        // receives when the grid fits one dispatch round) sum to the same
        // work.
        const int per = gridDim.x >> 3, hpx = per / nqt;
        const int j = blockIdx.x >> 3, k = j / hpx, half = nqt / 2;
        bh = (blockIdx.x & 7) * hpx + j % hpx;
        t = (k < half) ? k : (nqt - 1) - (k - half);   // tiles[0] = nqt - 1 - t below
    }
    if (!PAIR && a.order == 3) {
        // tile-major: head p % (B*H), (p / (B*H))-th heaviest tile
        const int nbh = a.B * a.H;
        if ((int)blockIdx.x >= a.n_work) return;
        bh = (int)blockIdx.x % nbh;
        t = (int)blockIdx.x / nbh;
    }
    const int64_t head_off = (int64_t)bh * a.N * D * 2;   // bytes, q and o
    const int64_t kv_off =                                 // bytes, k and v of this head's K/V head
        ((int64_t)(bh / a.H) * a.H_kv + (bh % a.H) / (a.H / a.H_kv)) * a.N * D * 2;
    ContigKV<D> kv{(const char*)a.k + kv_off, (const char*)a.v + kv_off, (uint32_t)a.N * (uint32_t)(D * 2)};
    const float c2 = a.scale * kLog2e;

    int tiles[2];
    int ntiles = 1;
    tiles[0] = nqt - 1 - t;                 // heavy first
    if (PAIR) {
        tiles[1] = t;
        ntiles = (tiles[1] != tiles[0]) ? 2 : 1;
    }
#pragma unroll 1
    for (int it = 0; it < ntiles; ++it) {
        const int qt = tiles[it];
        const int q0 = qt * BM;
        TileProblem P;
        P.q = (const char*)a.q + head_off + (int64_t)q0 * D * 2;
        P.q_stride = D * 2;
        P.q_hstride = 0;
        P.rows_per_pos = 1;
        P.n_rows = min(BM, a.N - q0);
        P.q_pos0 = q0;
        P.causal = a.causal;
        P.kv_begin = 0;
        P.kv_end = a.N;
        TileOut out;
        out.o = (char*)a.o + head_off + (int64_t)q0 * D * 2;
        out.o_stride = D * 2;
        out.o_hstride = 0;
        out.lse_hstride = 0;
        out.lse = a.lse ? a.lse + (int64_t)bh * a.N + q0 : nullptr;
        out.lse_stride = 1;
        out.fp32_out = 0;
        if (it) __syncthreads();   // LDS reuse across the two tiles
        if constexpr (PIPE) run_pipe_tile<D, 4>(P, kv, out, c2, pbuf);
        else run_query_tile<D>(P, kv, out, c2, buf);
    }
}

// ---------------------------------------------------------------------------
// fp32 kernel: 64 query rows per workgroup, 4 threads per row (each owns d/4
// channels of q and of the output), 64-key K/V tiles staged in LDS as fp32 (the
// block size of the fp32 workload).
template <int D>
__global__ __launch_bounds__(256) void prefill_f32_kernel(PrefillArgs a)
{
    constexpr int BM = 64, BN = 64, SUB = D / 4;
    __shared__ float ks[BN][D + 4];
    __shared__ float vs[BN][D + 4];
    const int nqt = (a.N + BM - 1) / BM;
    const int bh = blockIdx.x / nqt, qt = nqt - 1 - (int)(blockIdx.x % nqt);
    const int tid = threadIdx.x, row = tid >> 2, part = tid & 3;
    const int q0 = qt * BM, qi = q0 + row;
    const int64_t head = (int64_t)bh * a.N * D;
    const int64_t kv_head = ((int64_t)(bh / a.H) * a.H_kv + (bh % a.H) / (a.H / a.H_kv)) * a.N * D;
    const float* qp = (const float*)a.q + head;
    const float* kp = (const float*)a.k + kv_head;
    const float* vp = (const float*)a.v + kv_head;
    const float c2 = a.scale * kLog2e;

    float qv[SUB], acc[SUB];
#pragma unroll
    for (int c = 0; c < SUB; ++c) {
        qv[c] = qi < a.N ? qp[(int64_t)qi * D + part * SUB + c] : 0.f;
        acc[c] = 0.f;
    }
    int lim = a.N;
    if (a.causal) lim = min(a.N, qi + 1);
    int t_end = a.causal ? min(a.N, q0 + BM) : a.N;
    float m = -INFINITY, l = 0.f;
    for (int kb = 0; kb < t_end; kb += BN) {
        __syncthreads();
        for (int e = tid; e < BN * D; e += 256) {
            int r = e / D, c = e % D, key = kb + r;
            ks[r][c] = key < a.N ? kp[(int64_t)key * D + c] : 0.f;
            vs[r][c] = key < a.N ? vp[(int64_t)key * D + c] : 0.f;
        }
        __syncthreads();
        float s[BN];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            float p = 0.f;
#pragma unroll
            for (int c = 0; c < SUB; ++c) p = __builtin_fmaf(qv[c], ks[j][part * SUB + c], p);
            p += __shfl_xor(p, 1, 64);
            p += __shfl_xor(p, 2, 64);
            s[j] = (kb + j < lim) ? p : -INFINITY;
            mt = fmaxf(mt, s[j]);
        }
        float m_new = fmaxf(m, mt);
        float ms_new = m_new == -INFINITY ? 0.f : m_new * c2;
        float ms_old = m == -INFINITY ? 0.f : m * c2;
        float alpha = __builtin_amdgcn_exp2f(ms_old - ms_new);
        m = m_new;
        l *= alpha;
#pragma unroll
        for (int c = 0; c < SUB; ++c) acc[c] *= alpha;
#pragma unroll
        for (int j = 0; j < BN; ++j) {
            float p = s[j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(__builtin_fmaf(s[j], c2, -ms_new));
            l += p;
#pragma unroll
            for (int c = 0; c < SUB; ++c) acc[c] = __builtin_fmaf(p, vs[j][part * SUB + c], acc[c]);
        }
    }
    if (qi < a.N) {
        float inv = l > 0.f ? 1.f / l : 0.f;
        float* op = (float*)a.o + head + (int64_t)qi * D + part * SUB;
#pragma unroll
        for (int c = 0; c < SUB; ++c) op[c] = acc[c] * inv;
        if (a.lse && part == 0) {
            float ms = m == -INFINITY ? 0.f : m * c2;
            a.lse[(int64_t)bh * a.N + qi] = l > 0.f ? (ms + __log2f(l)) * kLn2 : -INFINITY;
        }
    }
}

// Causal grids of at most this many query tiles (about one dispatch round)
// take the complementary tile order; larger ones take the tile-major order
// while the K/V of all heads fits in the last-level cache (256 MB) and no
// query heads share a K/V head, and per-head ranges otherwise.
constexpr int64_t kOrderMaxTiles = 1024;
constexpr int64_t kTileMajorMaxKV = (int64_t)256 << 20;

int launch_prefill(const PrefillArgs& in, hipStream_t stream)
{
    PrefillArgs a = in;
    if (a.dtype == 0) {
        const int BM = kTileRows;
        const int nqt = (a.N + BM - 1) / BM;
        const int64_t bh = (int64_t)a.B * a.H;
        // tile order, decided for one query tile per workgroup; the
        // complementary order needs whole heads per XCD share (a multiple of
        // 8 * nqt tiles)
        const int64_t n_tiles = bh * nqt;
        const bool can_order = a.causal && a.pair != 1 && n_tiles % 8 == 0 && (n_tiles / 8) % nqt == 0;
        if (a.order == 1 && !can_order) a.order = 0;
        if (a.order < 0) {
            const int64_t kv_bytes = (int64_t)a.B * a.H_kv * a.N * a.d * 2 * 2;
            // tile-major only without grouped heads: per-head ranges keep the
            // query heads of one K/V head on one XCD, whose L2 then serves
            // their K/V (16x32x8192x128 on 4 K/V heads, 256 MiB of K/V: per-head
            // ranges 1075-1081 TFLOP/s, tile-major 905-937)
            a.order = (can_order && n_tiles <= kOrderMaxTiles) ? 1
                    : ((kv_bytes <= kTileMajorMaxKV && a.H_kv == a.H) ? 3 : 0);
        }
        if (!a.causal) a.order = 0;
        // Pairing (tiles t and nqt-1-t in one workgroup, equal work per
        // workgroup) by default where a causal grid runs in per-head ranges:
        // 16x32x8192x128 1057-1064 -> 1077-1084 TFLOP/s, on 4 K/V heads
        // 1057-1067 -> 1079-1089; one-round grids keep the complementary
        // order (1x32x2048x128 paired: -2.5 %)
        if (a.pair < 0) a.pair = (a.causal && a.order == 0 && nqt > 1) ? 1 : 0;
        if (a.pair) a.order = 0;
        // the pipelined key loop for the one-round grids of the complementary
        // order, the plain one otherwise
        if (a.kernel < 0) a.kernel = (a.order == 1) ? 1 : 0;
        const int per_bh = a.pair ? (nqt + 1) / 2 : nqt;
        const int64_t n_work = bh * per_bh;
        if (n_work > (int64_t)INT32_MAX - 8) return -2;
        a.n_work = (int)n_work;
        if (!grid_fits((n_work + 7) / 8 * 8, TileCfg<128>::kThreads)) return -2;
        const int grid = (int)((n_work + 7) / 8 * 8);
#define ATTN_LAUNCH_PREFILL(DD, PP, KK) \
    hipLaunchKernelGGL((prefill_bf16_kernel<DD, PP, KK>), dim3(grid), dim3(TileCfg<DD>::kThreads), 0, stream, a)
#define ATTN_LAUNCH_PREFILL_K(DD, PP)               \
    do {                                            \
        if (a.kernel == 1) ATTN_LAUNCH_PREFILL(DD, PP, 1); \
        else ATTN_LAUNCH_PREFILL(DD, PP, 0);        \
    } while (0)
        if (a.d == 128) {
            if (a.pair) ATTN_LAUNCH_PREFILL_K(128, true);
            else ATTN_LAUNCH_PREFILL_K(128, false);
        } else {
            if (a.pair) ATTN_LAUNCH_PREFILL_K(64, true);
            else ATTN_LAUNCH_PREFILL_K(64, false);
        }
#undef ATTN_LAUNCH_PREFILL
#undef ATTN_LAUNCH_PREFILL_K
    } else {
        const int nqt = (a.N + 63) / 64;
        const int64_t grid = (int64_t)a.B * a.H * nqt;
        if (!grid_fits(grid, 256)) return -2;
        if (a.d == 128)
            hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3((unsigned)grid), dim3(256), 0, stream, a);
        else
            hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3((unsigned)grid), dim3(256), 0, stream, a);
    }
    return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // namespace attn
