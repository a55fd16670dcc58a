// check_gfx950.hip -- device-side check of the paged-attention contract:
// every request's lengths (1 <= q_len <= ctx_len <= max_ctx_len, q_len <=
// max_q_len) and every block-table entry a request uses (logical blocks
// [0, ceil(ctx_len / block_size)), which must fit max_blocks_per_seq) lying in
// [0, num_blocks).  The attention kernels trust these values (checking them
// there would cost every step); this check is for debugging callers, either
// through paged_attn_check or, with ATTN_DEBUG=1, before every paged call.
//
// One workgroup walks the requests in order, its threads striding over each
// request's table entries, and folds what it finds into a shared flag word,
// which thread 0 stores once at the end: no global atomics, and the status
// word is fully written by every call (callers need not clear it).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "check_internal.h"

namespace attn {

namespace {

__global__ __launch_bounds__(256) void paged_check_kernel(CheckArgs a)
{
    __shared__ int flags;
    if (threadIdx.x == 0) flags = 0;
    __syncthreads();
    int found = 0;
    for (int r = 0; r < a.num_seqs; ++r) {
        const int ctx = a.ctx_lens[r], ql = a.q_lens[r];
        if (ql < 1 || ql > ctx || ctx > a.max_ctx_len || ql > a.max_q_len) found |= kCheckLengths;
        // table entries the attention would read, never past the row
        const int64_t need = ctx > 0 ? ((int64_t)ctx + a.block_size - 1) / a.block_size : 0;
        if (need > a.max_blocks_per_seq) found |= kCheckLengths;
        const int n = (int)(need < a.max_blocks_per_seq ? need : a.max_blocks_per_seq);
        const int32_t* row = a.block_table + (int64_t)r * a.max_blocks_per_seq;
        for (int j = threadIdx.x; j < n; j += blockDim.x) {
            const int32_t pb = row[j];
            if (pb < 0 || pb >= a.num_blocks) found |= kCheckTable;
        }
    }
    if (found) atomicOr(&flags, found);   // LDS atomic
    __syncthreads();
    if (threadIdx.x == 0) *a.status = flags;
}

}  // namespace

// Status word of the ATTN_DEBUG check inside the paged entry points (one per
// device, in the library's static device memory).
__device__ int32_t g_debug_status;

int launch_paged_check(const CheckArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL(paged_check_kernel, dim3(1), dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int run_paged_debug_check(CheckArgs a, hipStream_t stream, int32_t* flags)
{
    // device address of this device's status word (the symbol itself is only
    // a host-side handle)
    void* dev_status = nullptr;
    if (hipGetSymbolAddress(&dev_status, HIP_SYMBOL(g_debug_status)) != hipSuccess || !dev_status) return -1;
    a.status = (int32_t*)dev_status;
    hipLaunchKernelGGL(paged_check_kernel, dim3(1), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -1;
    int32_t host = 0;
    if (hipMemcpyAsync(&host, dev_status, sizeof(host), hipMemcpyDeviceToHost, stream) != hipSuccess) return -1;
    if (hipStreamSynchronize(stream) != hipSuccess) return -1;
    *flags = host;
    return 0;
}

}  // namespace attn
