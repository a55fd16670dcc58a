// noalloc_gfx950.hip -- paged_attn_fwd_static: paged_attn_fwd for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).  The split partials live in a file-scope
// device array instead of a caller workspace; everything else is
// paged_attn_fwd (same validation, plan, kernels and bits).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "attn.h"

namespace {

constexpr int kMaxDevices = 64;

// The workspace of paged_attn_fwd_static: one copy per GPU, held until the
// process ends.  In host code `scratch` names a host-side stand-in; device
// code is only ever handed the address hipGetSymbolAddress returns.
__device__ __align__(256) unsigned char scratch[ATTN_STATIC_WORKSPACE_BYTES];

// Device address of `scratch` on each device, looked up once per device.
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices];

// Address of this device's `scratch` (looked up on first use, with the device
// current), or an ATTN_ERR_* code.
int device_scratch(void** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_ERR_DEVICE;
    std::lock_guard<std::mutex> lock(g_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();   // leave no sticky error behind
            return ATTN_ERR_DEVICE;
        }
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

int paged_attn_fwd_static(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                          int block_size, void* o, float* lse,
                          int num_seqs, int H, int d, float scale, int max_blocks_per_seq,
                          int64_t kv_block_stride, int num_blocks, int max_q_len, int max_ctx_len,
                          attn_dtype_t dtype, void* stream)
{
    // 0 for arguments paged_attn_fwd rejects (it reports them below) and for
    // plans without split partials
    const size_t need = paged_attn_workspace_bytes(num_seqs, H, d, block_size, max_q_len, max_ctx_len);
    if (need > (size_t)ATTN_STATIC_WORKSPACE_BYTES) return ATTN_ERR_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) {
        const int rc = device_scratch(&ws);
        if (rc) return rc;
    }
    return paged_attn_fwd(q, k_pool, v_pool, block_table, ctx_lens, q_lens, block_size, o, lse, num_seqs, H, d,
                          scale, max_blocks_per_seq, kv_block_stride, num_blocks, max_q_len, max_ctx_len, dtype, ws,
                          need > 0 ? (size_t)ATTN_STATIC_WORKSPACE_BYTES : 0, stream);
}

}  // extern "C"
