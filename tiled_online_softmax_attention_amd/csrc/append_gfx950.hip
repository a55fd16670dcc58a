// append_gfx950.hip -- KV append into the paged cache, with the block
// allocator on the device ("Flash Attention and Paged Attention", section 3:
// a pool of fixed-size blocks, a free list, a page table per request that
// grows by whole blocks; "Sequence length doubles, inference time
// quadruples", decode stage: each new token's K and V join the cache).
//
// Two launches per append, both on the caller's stream:
//   kv_alloc_kernel  one workgroup: checks the whole batch, then takes the new
//                    blocks off the top of the free stack in request order
//                    (the ids, and their table slots, that one pop per block
//                    per request in order would give) and writes them into
//                    the page tables; status 0 on success, else an error code
//                    and nothing changed.
//   kv_write_kernel  copies every new token's K and V rows (16 bytes per
//                    lane) into their slots; does nothing unless status is 0.
// Release pushes ids back on the stack (kv_release_kernel, one workgroup).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "append_internal.h"
#include "attn_internal.h"

namespace attn {

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAllocThreads = 1024;
constexpr int kWriteThreads = 256;
constexpr int kTokPerGroup = 4;   // new tokens per write workgroup

__device__ __forceinline__ int wave_sum(int v)
{
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
    for (int o = 1; o < 64; o <<= 1) {
        const int t = __shfl_up(v, o, 64);
        if (lane >= o) v += t;
    }
    return v;
}

// Sum over the workgroup (kAllocThreads threads); every thread gets it.
__device__ int block_sum(int v, int* red)
{
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = wave_sum(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    int s = 0;
    for (int i = 0; i < kAllocThreads / 64; ++i) s += red[i];
    return s;
}

__device__ __forceinline__ int blocks_for(int tokens, int bs) { return (tokens + bs - 1) / bs; }

}  // namespace

__global__ __launch_bounds__(kAllocThreads) void kv_alloc_kernel(AppendArgs a)
{
    __shared__ int red[kAllocThreads / 64];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int bs = a.block_size;
    const int fc = *a.free_count;

    // pass 1: blocks wanted by the batch, and whether any request is invalid
    // or would outgrow its table
    int need_sum = 0, over = 0, bad = 0;
    for (int r = tid; r < a.num_seqs; r += kAllocThreads) {
        const int c = a.ctx_lens[r], n = a.new_lens[r];
        // n above the host bound max_new_len would allocate blocks for tokens
        // the write launch (sized by that bound) never copies
        if (c < 0 || n < 0 || n > a.max_new_len || c > INT32_MAX - n) {
            bad = 1;
            continue;
        }
        const int have = blocks_for(c, bs), want = blocks_for(c + n, bs);
        need_sum += want - have;
        over |= want > a.max_blocks_per_seq;
    }
    const int total = block_sum(need_sum, red);
    const int any_over = block_sum(over, red);
    const int any_bad = block_sum(bad, red) + (fc < 0 || fc > a.num_blocks);
    if (any_bad || any_over || total > fc) {
        if (tid == 0) *a.status = any_bad ? kAppendInvalid : (any_over ? kAppendTableFull : kAppendExhausted);
        return;
    }

    // pass 2: exclusive scan of the per-request block counts in request order;
    // request r's i-th new block is the (off_r + i)-th id from the top
    int base = 0;
    for (int r0 = 0; r0 < a.num_seqs; r0 += kAllocThreads) {
        const int r = r0 + tid;
        int c = 0, n = 0, have = 0, need = 0;
        if (r < a.num_seqs) {
            c = a.ctx_lens[r];
            n = a.new_lens[r];
            have = blocks_for(c, bs);
            need = blocks_for(c + n, bs) - have;
        }
        const int incl = wave_incl_scan(need, lane);
        __syncthreads();
        if (lane == 63) red[w] = incl;
        __syncthreads();
        int wofs = 0, chunk = 0;
        for (int i = 0; i < kAllocThreads / 64; ++i) {
            wofs += (i < w) ? red[i] : 0;
            chunk += red[i];
        }
        const int off = base + wofs + incl - need;
        if (r < a.num_seqs) {
            int32_t* row = a.block_table + (int64_t)r * a.max_blocks_per_seq;
            for (int i = 0; i < need; ++i) row[have + i] = a.free_blocks[fc - 1 - (off + i)];
            if (a.new_ctx_lens) a.new_ctx_lens[r] = c + n;
        }
        base += chunk;
    }
    __syncthreads();
    if (tid == 0) {
        *a.free_count = fc - total;
        *a.status = kAppendOk;
    }
}

// One workgroup per (request, group of kTokPerGroup new tokens); grid is
// flattened: blockIdx.x = r * tiles_per_seq + tile.
__global__ __launch_bounds__(kWriteThreads) void kv_write_kernel(AppendArgs a, int tiles_per_seq)
{
    if (*a.status != kAppendOk) return;
    const int r = blockIdx.x / tiles_per_seq;
    const int t0 = (blockIdx.x % tiles_per_seq) * kTokPerGroup;
    const int n = a.new_lens[r];
    if (t0 >= n) return;
    const int c = a.ctx_lens[r];
    const int lane = threadIdx.x & 63;
    int64_t row0 = 0;                          // packed row of request r's first new token
    for (int s0 = 0; s0 < r; s0 += 64) {
        const int s = s0 + lane;
        row0 += wave_sum((s < r) ? a.new_lens[s] : 0);
    }
    const int bs = a.block_size;
    const int64_t row_bytes = (int64_t)a.d * a.elem_bytes;
    const int cpr = (int)(row_bytes / 16);     // 16-byte chunks per row
    const int per_kv = a.H * cpr;
    const int per_tok = 2 * per_kv;
    const int ntok = min(kTokPerGroup, n - t0);
    const int32_t* table = a.block_table + (int64_t)r * a.max_blocks_per_seq;
    const int64_t blk_bytes = a.kv_block_stride * a.elem_bytes;
    for (int e = threadIdx.x; e < ntok * per_tok; e += kWriteThreads) {
        const int t = t0 + e / per_tok;
        int rem = e % per_tok;
        const int kv = rem / per_kv;
        rem %= per_kv;
        const int h = rem / cpr, ch = rem % cpr;
        const int p = c + t;
        const int pb = table[p / bs];
        if (pb < 0 || pb >= a.num_blocks) {    // a corrupt existing table entry
            *a.status = kAppendInvalid;
            continue;
        }
        const char* src = (const char*)(kv ? a.v_new : a.k_new) + ((row0 + t) * a.H + h) * row_bytes + ch * 16;
        char* dst = (char*)(kv ? a.v_pool : a.k_pool) + (int64_t)pb * blk_bytes + ((int64_t)h * bs + p % bs) * row_bytes +
                    ch * 16;
        *(u32x4*)dst = *(const u32x4*)src;
    }
}

__global__ __launch_bounds__(kAllocThreads) void kv_release_kernel(ReleaseArgs a)
{
    __shared__ int red[kAllocThreads / 64];
    const int tid = threadIdx.x;
    const int fc = *a.free_count;
    int bad = 0;
    for (int i = tid; i < a.n; i += kAllocThreads) {
        const int b = a.blocks[i];
        bad |= (b < 0 || b >= a.num_blocks);
    }
    const int any_bad = block_sum(bad, red) + (fc < 0 || fc > a.num_blocks);
    if (any_bad || a.n > a.num_blocks - fc) {
        if (tid == 0) *a.status = any_bad ? kAppendInvalid : kAppendExhausted;
        return;
    }
    for (int i = tid; i < a.n; i += kAllocThreads) a.free_blocks[fc + i] = a.blocks[i];
    __syncthreads();
    if (tid == 0) {
        *a.free_count = fc + a.n;
        *a.status = kAppendOk;
    }
}

int launch_append(const AppendArgs& a, hipStream_t stream)
{
    // the write grid is checked before the allocation is launched
    const int tiles = (a.max_new_len + kTokPerGroup - 1) / kTokPerGroup;
    const int64_t grid = (int64_t)a.num_seqs * tiles;
    if (a.max_new_len > 0 && !grid_fits(grid, kWriteThreads)) return -2;
    hipLaunchKernelGGL(kv_alloc_kernel, dim3(1), dim3(kAllocThreads), 0, stream, a);
    if (a.max_new_len > 0)
        hipLaunchKernelGGL(kv_write_kernel, dim3((unsigned)grid), dim3(kWriteThreads), 0, stream, a, tiles);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

int launch_release(const ReleaseArgs& a, hipStream_t stream)
{
    hipLaunchKernelGGL(kv_release_kernel, dim3(1), dim3(kAllocThreads), 0, stream, a);
    return hipGetLastError() == hipSuccess ? 0 : -1;
}

}  // namespace attn
