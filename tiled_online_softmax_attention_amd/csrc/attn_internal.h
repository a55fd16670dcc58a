// attn_internal.h -- argument blocks and launchers shared between the C-ABI
// host code (attn_api.hip) and the kernel translation units.  Not installed;
// the public interface is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "attn.h"

namespace attn {

// A dispatch's grid size is a 32-bit count of work-items: `blocks`
// workgroups of `threads` each must fit in it (and in a positive int).
inline bool grid_fits(int64_t blocks, int threads)
{
    return blocks > 0 && blocks <= (int64_t)INT32_MAX && blocks * threads <= (int64_t)UINT32_MAX;
}

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, N, d;
    int H_kv;       // K/V heads (H a multiple of H_kv; query head h reads K/V head h / (H / H_kv))
    float scale;
    int causal;
    int dtype;      // 0 bf16, 1 fp32
    int pair;       // bf16 causal: one workgroup takes tiles t and n-1-t (-1: launcher decides)
    int order;      // bf16 causal: -1 automatic, 0 heaviest tile first per head in
                    // XCD-contiguous ranges, 1 complementary order within each XCD's share,
                    // 3 tile-major over the whole grid
    int kernel;     // bf16 key loop: -1 launcher decides, 0 plain, 1 software-pipelined
    int n_work;     // filled by the launcher
};

// Host-side plan of a paged launch: a pure function of the host bounds.
struct PagedPlan {
    int path;            // 0: vector decode kernel, 1: MFMA tile kernel, 2: decode MFMA kernel
    int split_tokens;    // keys per context split (multiple of the page size)
    int max_splits;      // ceil(max_ctx_len / split_tokens)
    int nqt;             // query tiles per request (chunk path)
    int tile_kernel;     // tile path: 0 plain loop, 128 rows; 1 pipelined loop, 128 rows; 2 pipelined, 256 rows
    int gc;              // decode path: query heads per workgroup (they share one K/V head)
    int n_chunks;        // decode path: workgroups per K/V head (= (H / H_kv) / gc)
    size_t ws_o_bytes;   // fp32 partial outputs
    size_t ws_lse_bytes; // fp32 partial log-sum-exps
    size_t ws_bytes;     // total (0 when max_splits == 1)
};

struct PagedArgs {
    const void* q;
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_table;
    const int32_t* ctx_lens;
    const int32_t* q_lens;
    int block_size;
    void* o;
    float* lse;
    int num_seqs, H, d;
    int H_kv;                  // K/V heads in the pool
    int n_chunks;              // decode path: workgroups per K/V head (from the plan)
    float scale;
    int max_blocks_per_seq;
    int64_t kv_block_stride;   // elements
    int num_blocks;
    int max_q_len, max_ctx_len;
    int split_tokens, max_splits;
    float* ws_o;     // [num_seqs*max_q_len][H][max_splits][d]
    float* ws_lse;   // [num_seqs*max_q_len][H][max_splits]
    int tile_map;    // tile kernel work mapping: -1 launcher decides, 0 ranges, 1 pairs, 2 items
};

struct GatherArgs {
    const void* k_pool;
    const void* v_pool;
    const int32_t* block_table;
    const int32_t* ctx_lens;
    int block_size, num_seqs, H, d, max_blocks_per_seq;
    int64_t kv_block_stride;
    int max_ctx_len;
    int elem_bytes;
    void* k_out;
    void* v_out;
};

constexpr int kDecodeMaxQ = 4;     // q_len up to this uses the vector decode kernel ...
constexpr int kDecodeMfmaGroup = 4; // ... unless this many query heads share a K/V head
constexpr int kChunkMaxSplit = 8192;  // most keys per split on the MFMA tile path (multiple of 64)

// opts: paged_path, paged_split_tokens and paged_decode_heads override the
// plan's choices (validated by the caller).
PagedPlan plan_paged(int num_seqs, int H, int H_kv, int d, int block_size, int max_q_len, int max_ctx_len,
                     const attn_launch_opts_t& opts);

int launch_prefill(const PrefillArgs& a, hipStream_t stream);
int launch_paged(const PagedArgs& a, const PagedPlan& plan, hipStream_t stream);
int launch_gather(const GatherArgs& a, hipStream_t stream);

}  // namespace attn
