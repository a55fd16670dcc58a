// check_internal.h -- the device-side check of the paged-attention contract,
// shared between the C-ABI host code (attn_api.hip) and check_gfx950.hip.
// Not installed; the public interface is include/attn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Flag bits of the status word (ATTN_CHECK_* in attn.h).
constexpr int kCheckLengths = 1;
constexpr int kCheckTable = 2;

struct CheckArgs {
    const int32_t* block_table;   // [num_seqs, max_blocks_per_seq]
    const int32_t* ctx_lens;      // [num_seqs]
    const int32_t* q_lens;        // [num_seqs]
    int num_seqs, block_size, max_blocks_per_seq, num_blocks, max_q_len, max_ctx_len;
    int32_t* status;              // device word, written once per call
};

// Enqueue the check on `stream` (status written asynchronously).  0 / -1.
int launch_paged_check(const CheckArgs& a, hipStream_t stream);

// The ATTN_DEBUG form: check into the library's own status word, wait for
// the stream and return the flags in *flags.  0 / -1 (a HIP call failed).
int run_paged_debug_check(CheckArgs a, hipStream_t stream, int32_t* flags);

}  // namespace attn
