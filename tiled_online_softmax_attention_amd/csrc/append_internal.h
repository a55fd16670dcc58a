// append_internal.h -- argument blocks, status codes and launchers of the KV
// append / release kernels (append_gfx950.hip), shared with the C-ABI host
// code (attn_api.hip).  Not installed; the public interface is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

struct AppendArgs {
    const void* k_new;
    const void* v_new;
    const int32_t* ctx_lens;
    const int32_t* new_lens;
    void* k_pool;
    void* v_pool;
    int32_t* block_table;
    int32_t* free_blocks;
    int32_t* free_count;
    int32_t* new_ctx_lens;   // may be null
    int32_t* status;
    int block_size, num_seqs, H, d, max_blocks_per_seq;
    int64_t kv_block_stride;   // elements
    int num_blocks, max_new_len, elem_bytes;
};

struct ReleaseArgs {
    const int32_t* blocks;
    int n;
    int32_t* free_blocks;
    int32_t* free_count;
    int32_t* status;
    int num_blocks;
};

// device status words of append / release (values of include/attn.h)
constexpr int kAppendOk = 0, kAppendExhausted = 1, kAppendTableFull = 2, kAppendInvalid = 3;

int launch_append(const AppendArgs& a, hipStream_t stream);
int launch_release(const ReleaseArgs& a, hipStream_t stream);

}  // namespace attn
