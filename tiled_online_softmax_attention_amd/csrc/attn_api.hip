// attn_api.hip -- the C ABI declared in include/attn.h: host-side validation,
// launch planning and kernel launches.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "attn.h"
#include "append_internal.h"
#include "bwd_internal.h"
#include "attn_internal.h"
#include "check_internal.h"

namespace {

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Cached "is the current device a gfx950" answer (per device ordinal).
int check_device()
{
    static int cached[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_DEVICE;
    if (dev < 0 || dev >= 64) return ATTN_ERR_DEVICE;
    if (cached[dev] == 0) {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_DEVICE;
        cached[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    }
    return cached[dev] == 1 ? ATTN_OK : ATTN_ERR_DEVICE;
}

// ATTN_DEBUG=1 (read at every call): the paged entry points check lengths
// and block-table entries on the device first, wait for the result and
// return ATTN_ERR_BAD_TABLE without launching anything else if they break
// the contract.
bool debug_checks()
{
    const char* env = getenv("ATTN_DEBUG");
    return env && *env && atoi(env) != 0;
}

int check_scale(float scale)
{
    if (!isfinite(scale) || scale < 0.f) return ATTN_ERR_SCALE;
    return ATTN_OK;
}

// Launch variants with every field in range (defaults where opts is NULL).
int read_opts(const attn_launch_opts_t* in, attn_launch_opts_t* out)
{
    attn_launch_opts_default(out);
    if (!in) return ATTN_OK;
    *out = *in;
    const attn_launch_opts_t& o = *out;
    const bool ok = (o.prefill_kernel >= -1 && o.prefill_kernel <= 1) &&
                    (o.prefill_pair >= -1 && o.prefill_pair <= 1) &&
                    (o.prefill_order == -1 || o.prefill_order == 0 || o.prefill_order == 1 ||
                     o.prefill_order == 3) &&
                    (o.paged_path >= -1 && o.paged_path <= 2) &&
                    (o.paged_split_tokens >= 0 && o.paged_split_tokens <= (1 << 24)) &&
                    (o.paged_decode_heads == 0 || o.paged_decode_heads == 1 || o.paged_decode_heads == 2 ||
                     o.paged_decode_heads == 4 || o.paged_decode_heads == 8) &&
                    (o.paged_tile_map >= -1 && o.paged_tile_map <= 2) &&
                    (o.bwd_pair_q >= -1 && o.bwd_pair_q <= 1) && (o.bwd_pair_kv >= -1 && o.bwd_pair_kv <= 1) &&
                    (o.paged_tile_kernel >= -1 && o.paged_tile_kernel <= 2);
    return ok ? ATTN_OK : ATTN_ERR_OPTION;
}

}  // namespace

extern "C" {

const char* attn_strerror(int status)
{
    switch (status) {
        case ATTN_OK: return "ok";
        case ATTN_ERR_NULL: return "a required pointer is NULL";
        case ATTN_ERR_SHAPE: return "invalid size (must be >= 1 and fit 32-bit grid indexing)";
        case ATTN_ERR_HEAD_DIM: return "head_dim must be 64 or 128";
        case ATTN_ERR_BLOCK_SIZE: return "block_size must be 16 or 32";
        case ATTN_ERR_DTYPE: return "element type not supported by this entry point";
        case ATTN_ERR_ALIGN: return "pointer or stride not 16-byte aligned";
        case ATTN_ERR_WORKSPACE: return "workspace missing or too small";
        case ATTN_ERR_LAUNCH: return "HIP kernel launch failed";
        case ATTN_ERR_SCALE: return "scale must be finite and >= 0";
        case ATTN_ERR_DEVICE: return "current device is not a gfx950 GPU";
        case ATTN_ERR_BAD_TABLE:
            return "a length or block-table entry breaks the paged-attention contract (ATTN_DEBUG check)";
        case ATTN_ERR_OPTION: return "a launch option is out of range";
        default: return "unknown attn status";
    }
}

const char* attn_version(void) { return "attn_gfx950 1.1"; }

void attn_launch_opts_default(attn_launch_opts_t* opts)
{
    if (!opts) return;
    opts->prefill_kernel = -1;
    opts->prefill_pair = -1;
    opts->prefill_order = -1;
    opts->paged_path = -1;
    opts->paged_split_tokens = 0;
    opts->paged_decode_heads = 0;
    opts->paged_tile_map = -1;
    opts->bwd_pair_q = -1;
    opts->bwd_pair_kv = -1;
    opts->paged_tile_kernel = -1;
}

int attn_prefill_gqa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int H_kv, int N, int d, float scale, int causal,
                         attn_dtype_t dtype, const attn_launch_opts_t* opts, void* stream)
{
    if (!q || !k || !v || !o) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || H_kv < 1 || H % H_kv != 0) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || ((uintptr_t)lse & 3u))
        return ATTN_ERR_ALIGN;
    int rc = check_scale(scale);
    if (rc) return rc;
    attn_launch_opts_t op;
    rc = read_opts(opts, &op);
    if (rc) return rc;
    if ((int64_t)B * H > INT32_MAX / 2) return ATTN_ERR_SHAPE;
    if ((int64_t)N * d * (dtype == ATTN_BF16 ? 2 : 4) >= ((int64_t)1 << 32)) return ATTN_ERR_SHAPE;  // 32-bit row offsets
    rc = check_device();
    if (rc) return rc;
    attn::PrefillArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.H = H; a.H_kv = H_kv; a.N = N; a.d = d;
    a.scale = scale;
    a.causal = causal ? 1 : 0;
    a.dtype = (dtype == ATTN_BF16) ? 0 : 1;
    // bf16: the launcher picks the key loop, the tile order and pairing for
    // the grid (-1); the options force them
    a.kernel = op.prefill_kernel;
    a.pair = (!a.causal || N <= 128) ? 0 : op.prefill_pair;
    a.order = op.prefill_order;
    rc = attn::launch_prefill(a, (hipStream_t)stream);
    return rc == 0 ? ATTN_OK : (rc == -2 ? ATTN_ERR_SHAPE : ATTN_ERR_LAUNCH);
}

int attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, float scale, int causal,
                     attn_dtype_t dtype, void* stream)
{
    return attn_prefill_gqa_fwd(q, k, v, o, lse, B, H, H, N, d, scale, causal, dtype, nullptr, stream);
}

size_t attn_prefill_bwd_workspace_bytes(int B, int H, int N)
{
    if (B < 1 || H < 1 || N < 1) return 0;
    return attn::bwd_workspace_bytes(B, H, N);
}

int attn_prefill_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv,
                     int B, int H, int H_kv, int N, int d, float scale, int causal,
                     attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                     const attn_launch_opts_t* opts, void* stream)
{
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv) return ATTN_ERR_NULL;
    if (B < 1 || H < 1 || N < 1 || H_kv < 1 || H % H_kv != 0) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
        !aligned16(dk) || !aligned16(dv) || ((uintptr_t)lse & 3u))
        return ATTN_ERR_ALIGN;
    int rc = check_scale(scale);
    if (rc) return rc;
    attn_launch_opts_t op;
    rc = read_opts(opts, &op);
    if (rc) return rc;
    if ((int64_t)B * H > INT32_MAX / 2) return ATTN_ERR_SHAPE;
    if ((int64_t)N * d * 2 >= ((int64_t)1 << 32)) return ATTN_ERR_SHAPE;   // 32-bit row offsets
    const size_t need = attn::bwd_workspace_bytes(B, H, N);
    if (!workspace || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
    if ((uintptr_t)workspace & 15u) return ATTN_ERR_ALIGN;
    rc = check_device();
    if (rc) return rc;
    attn::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
    a.dq = dq; a.dk = dk; a.dv = dv;
    a.ws = (float*)workspace;
    a.B = B; a.H = H; a.H_kv = H_kv; a.N = N; a.d = d;
    a.scale = scale;
    a.causal = causal ? 1 : 0;
    a.pair_q = op.bwd_pair_q;
    a.pair_kv = op.bwd_pair_kv;
    rc = attn::launch_bwd(a, (hipStream_t)stream);
    return rc == 0 ? ATTN_OK : (rc == -2 ? ATTN_ERR_SHAPE : ATTN_ERR_LAUNCH);
}

size_t paged_attn_gqa_workspace_bytes(int num_seqs, int H, int H_kv, int d, int block_size, int max_q_len,
                                      int max_ctx_len, const attn_launch_opts_t* opts)
{
    if (num_seqs < 1 || H < 1 || H_kv < 1 || H % H_kv != 0 || H / H_kv > 128 || (d != 64 && d != 128) ||
        (block_size != 16 && block_size != 32) || max_q_len < 1 || max_ctx_len < 1 || max_q_len > max_ctx_len)
        return 0;
    attn_launch_opts_t op;
    if (read_opts(opts, &op) != ATTN_OK) return 0;
    return attn::plan_paged(num_seqs, H, H_kv, d, block_size, max_q_len, max_ctx_len, op).ws_bytes;
}

size_t paged_attn_workspace_bytes(int num_seqs, int H, int d, int block_size, int max_q_len, int max_ctx_len)
{
    return paged_attn_gqa_workspace_bytes(num_seqs, H, H, d, block_size, max_q_len, max_ctx_len, nullptr);
}

int paged_attn_gqa_fwd(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                       int block_size, void* o, float* lse,
                       int num_seqs, int H, int H_kv, int d, float scale, int max_blocks_per_seq,
                       int64_t kv_block_stride, int num_blocks, int max_q_len, int max_ctx_len,
                       attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                       const attn_launch_opts_t* opts, void* stream)
{
    if (!q || !k_pool || !v_pool || !block_table || !ctx_lens || !q_lens || !o) return ATTN_ERR_NULL;
    if (num_seqs < 1 || H < 1 || max_blocks_per_seq < 1 || num_blocks < 1 || max_q_len < 1 ||
        max_ctx_len < 1 || max_q_len > max_ctx_len || H_kv < 1 || H % H_kv != 0 || H / H_kv > 128)
        return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (block_size != 16 && block_size != 32) return ATTN_ERR_BLOCK_SIZE;
    if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
    if (((int64_t)max_ctx_len + block_size - 1) / block_size > max_blocks_per_seq) return ATTN_ERR_SHAPE;
    if (kv_block_stride < (int64_t)H_kv * block_size * d) return ATTN_ERR_SHAPE;
    if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool) || !aligned16(o) ||
        ((kv_block_stride * 2) & 15) || ((uintptr_t)block_table & 3u) || ((uintptr_t)lse & 3u))
        return ATTN_ERR_ALIGN;
    int rc = check_scale(scale);
    if (rc) return rc;
    attn_launch_opts_t op;
    rc = read_opts(opts, &op);
    if (rc) return rc;
    if (op.paged_decode_heads > 0 &&
        ((H / H_kv) % op.paged_decode_heads != 0 || (block_size == 32 && op.paged_decode_heads == 8)))
        return ATTN_ERR_OPTION;
    const attn::PagedPlan plan = attn::plan_paged(num_seqs, H, H_kv, d, block_size, max_q_len, max_ctx_len, op);
    // grid sizes must fit 32 bits
    const int64_t rows = (int64_t)num_seqs * max_q_len;
    if (rows * H * plan.max_splits > (int64_t)INT32_MAX - 8) return ATTN_ERR_SHAPE;
    if (plan.ws_bytes > 0) {
        if (!workspace || workspace_bytes < plan.ws_bytes) return ATTN_ERR_WORKSPACE;
        if ((uintptr_t)workspace & 255u) return ATTN_ERR_ALIGN;
    }
    rc = check_device();
    if (rc) return rc;
    if (debug_checks()) {
        attn::CheckArgs c{block_table, ctx_lens, q_lens, num_seqs, block_size, max_blocks_per_seq, num_blocks,
                          max_q_len, max_ctx_len, nullptr};
        int32_t flags = 0;
        if (attn::run_paged_debug_check(c, (hipStream_t)stream, &flags) != 0) return ATTN_ERR_LAUNCH;
        if (flags) return ATTN_ERR_BAD_TABLE;
    }
    attn::PagedArgs a{};
    a.q = q; a.k_pool = k_pool; a.v_pool = v_pool;
    a.block_table = block_table; a.ctx_lens = ctx_lens; a.q_lens = q_lens;
    a.block_size = block_size; a.o = o; a.lse = lse;
    a.num_seqs = num_seqs; a.H = H; a.H_kv = H_kv; a.n_chunks = plan.n_chunks; a.d = d; a.scale = scale;
    a.max_blocks_per_seq = max_blocks_per_seq;
    a.kv_block_stride = kv_block_stride;
    a.num_blocks = num_blocks;
    a.max_q_len = max_q_len; a.max_ctx_len = max_ctx_len;
    a.split_tokens = plan.split_tokens;
    a.max_splits = plan.max_splits;
    a.ws_o = plan.ws_bytes ? (float*)workspace : nullptr;
    a.ws_lse = plan.ws_bytes ? (float*)((char*)workspace + plan.ws_o_bytes) : nullptr;
    a.tile_map = op.paged_tile_map;
    rc = attn::launch_paged(a, plan, (hipStream_t)stream);
    return rc == 0 ? ATTN_OK : (rc == -2 ? ATTN_ERR_SHAPE : ATTN_ERR_LAUNCH);
}

int paged_attn_fwd(const void* q, const void* k_pool, const void* v_pool,
                   const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                   int block_size, void* o, float* lse,
                   int num_seqs, int H, int d, float scale, int max_blocks_per_seq,
                   int64_t kv_block_stride, int num_blocks, int max_q_len, int max_ctx_len,
                   attn_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    return paged_attn_gqa_fwd(q, k_pool, v_pool, block_table, ctx_lens, q_lens, block_size, o, lse, num_seqs, H, H,
                              d, scale, max_blocks_per_seq, kv_block_stride, num_blocks, max_q_len, max_ctx_len,
                              dtype, workspace, workspace_bytes, nullptr, stream);
}

int paged_kv_gather(const void* k_pool, const void* v_pool, const int32_t* block_table,
                    const int32_t* ctx_lens, int block_size, int num_seqs, int H, int d,
                    int max_blocks_per_seq, int64_t kv_block_stride, int max_ctx_len,
                    attn_dtype_t dtype, void* k_out, void* v_out, void* stream)
{
    if (!k_pool || !v_pool || !block_table || !ctx_lens || !k_out || !v_out) return ATTN_ERR_NULL;
    if (num_seqs < 1 || H < 1 || max_blocks_per_seq < 1 || max_ctx_len < 1) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (block_size != 16 && block_size != 32) return ATTN_ERR_BLOCK_SIZE;
    if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
    if ((int64_t)(max_ctx_len + block_size - 1) / block_size > max_blocks_per_seq) return ATTN_ERR_SHAPE;
    if (kv_block_stride < (int64_t)H * block_size * d) return ATTN_ERR_SHAPE;
    const int eb = (dtype == ATTN_BF16) ? 2 : 4;
    if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_out) || !aligned16(v_out) ||
        ((kv_block_stride * eb) & 15))
        return ATTN_ERR_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    attn::GatherArgs a{};
    a.k_pool = k_pool; a.v_pool = v_pool; a.block_table = block_table; a.ctx_lens = ctx_lens;
    a.block_size = block_size; a.num_seqs = num_seqs; a.H = H; a.d = d;
    a.max_blocks_per_seq = max_blocks_per_seq; a.kv_block_stride = kv_block_stride;
    a.max_ctx_len = max_ctx_len; a.elem_bytes = eb; a.k_out = k_out; a.v_out = v_out;
    rc = attn::launch_gather(a, (hipStream_t)stream);
    return rc == 0 ? ATTN_OK : (rc == -2 ? ATTN_ERR_SHAPE : ATTN_ERR_LAUNCH);
}

int paged_kv_append(const void* k_new, const void* v_new, const int32_t* ctx_lens, const int32_t* new_lens,
                    void* k_pool, void* v_pool, int32_t* block_table, int32_t* free_blocks, int32_t* free_count,
                    int32_t* new_ctx_lens, int32_t* status, int block_size, int num_seqs, int H, int d,
                    int max_blocks_per_seq, int64_t kv_block_stride, int num_blocks, int max_new_len,
                    attn_dtype_t dtype, void* stream)
{
    if (!ctx_lens || !new_lens || !k_pool || !v_pool || !block_table || !free_blocks || !free_count || !status)
        return ATTN_ERR_NULL;
    if (max_new_len > 0 && (!k_new || !v_new)) return ATTN_ERR_NULL;
    if (num_seqs < 1 || H < 1 || max_blocks_per_seq < 1 || num_blocks < 1 || max_new_len < 0) return ATTN_ERR_SHAPE;
    if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
    if (block_size != 16 && block_size != 32) return ATTN_ERR_BLOCK_SIZE;
    if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
    if (kv_block_stride < (int64_t)H * block_size * d) return ATTN_ERR_SHAPE;
    if ((int64_t)num_seqs * ((max_new_len + 3) / 4) > INT32_MAX) return ATTN_ERR_SHAPE;
    const int eb = (dtype == ATTN_BF16) ? 2 : 4;
    if (!aligned16(k_pool) || !aligned16(v_pool) || (k_new && !aligned16(k_new)) || (v_new && !aligned16(v_new)) ||
        ((kv_block_stride * eb) & 15))
        return ATTN_ERR_ALIGN;
    if (new_ctx_lens && new_ctx_lens == ctx_lens) return ATTN_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    attn::AppendArgs a{};
    a.k_new = k_new; a.v_new = v_new; a.ctx_lens = ctx_lens; a.new_lens = new_lens;
    a.k_pool = k_pool; a.v_pool = v_pool; a.block_table = block_table; a.free_blocks = free_blocks;
    a.free_count = free_count; a.new_ctx_lens = new_ctx_lens; a.status = status;
    a.block_size = block_size; a.num_seqs = num_seqs; a.H = H; a.d = d; a.max_blocks_per_seq = max_blocks_per_seq;
    a.kv_block_stride = kv_block_stride; a.num_blocks = num_blocks; a.max_new_len = max_new_len; a.elem_bytes = eb;
    rc = attn::launch_append(a, (hipStream_t)stream);
    return rc == 0 ? ATTN_OK : (rc == -2 ? ATTN_ERR_SHAPE : ATTN_ERR_LAUNCH);
}

int paged_kv_release(const int32_t* blocks, int n, int32_t* free_blocks, int32_t* free_count, int32_t* status,
                     int num_blocks, void* stream)
{
    if (!free_blocks || !free_count || !status || (n > 0 && !blocks)) return ATTN_ERR_NULL;
    if (n < 0 || num_blocks < 1) return ATTN_ERR_SHAPE;
    int rc = check_device();
    if (rc) return rc;
    attn::ReleaseArgs a{};
    a.blocks = blocks; a.n = n; a.free_blocks = free_blocks; a.free_count = free_count; a.status = status;
    a.num_blocks = num_blocks;
    rc = attn::launch_release(a, (hipStream_t)stream);
    return rc == 0 ? ATTN_OK : ATTN_ERR_LAUNCH;
}

int paged_attn_check(const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens, int num_seqs,
                     int block_size, int max_blocks_per_seq, int num_blocks, int max_q_len, int max_ctx_len,
                     int32_t* status, void* stream)
{
    if (!block_table || !ctx_lens || !q_lens || !status) return ATTN_ERR_NULL;
    if (num_seqs < 1 || max_blocks_per_seq < 1 || num_blocks < 1 || max_q_len < 1 || max_ctx_len < 1)
        return ATTN_ERR_SHAPE;
    if (block_size != 16 && block_size != 32) return ATTN_ERR_BLOCK_SIZE;
    if (((uintptr_t)block_table & 3u) || ((uintptr_t)ctx_lens & 3u) || ((uintptr_t)q_lens & 3u) ||
        ((uintptr_t)status & 3u))
        return ATTN_ERR_ALIGN;
    int rc = check_device();
    if (rc) return rc;
    attn::CheckArgs c{block_table, ctx_lens, q_lens, num_seqs, block_size, max_blocks_per_seq, num_blocks,
                      max_q_len, max_ctx_len, status};
    return attn::launch_paged_check(c, (hipStream_t)stream) == 0 ? ATTN_OK : ATTN_ERR_LAUNCH;
}

}  // extern "C"
