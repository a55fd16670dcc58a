/*
 * attn.h -- C ABI of the MI355X (gfx950) tiled online-softmax attention library
 *           (libattn_gfx950.so).
 *
 * What is computed (the four web pages on tiled attention are the source):
 *   O = softmax(scale * Q K^T) V  row by row, with an optional causal mask
 *   ("Sequence length doubles, inference time quadruples", section "The
 *   mathematical nature of attention", attention equation), evaluated tile by
 *   tile with a running max m and running sum l so that no score matrix ever
 *   reaches memory ("Flash Attention and Paged Attention", section 2, the
 *   block-wise forward with online softmax).  Alongside O the library returns
 *   the per-row softmax statistic LSE = m + ln(l), the natural-log log-sum-exp
 *   of the row's masked, scaled scores (same page, section 2: the statistics
 *   kept for the backward pass).
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory),
 *     row-major and contiguous as described per function.  The caller owns all
 *     buffers.  The library allocates and frees nothing, keeps no pointer after
 *     it returns and holds no mutable global state besides a cached device
 *     property query.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Work is enqueued asynchronously; the function returns once the launches
 *     are issued.  Buffers must stay alive until the stream reaches them.
 *   - Return value: ATTN_OK (0) or a negative ATTN_ERR_* code.  Arguments are
 *     validated on the host before anything is launched; on error nothing is
 *     launched and no output is touched.  No exception or abort ever crosses
 *     the boundary.  attn_strerror() names a code.
 *   - Element types: ATTN_BF16 (bfloat16 storage, fp32 accumulation, bf16
 *     MFMA for the contractions) or ATTN_F32 (fp32 storage and arithmetic).
 *   - Scores are scaled by `scale` before the softmax; `scale` must be finite
 *     and >= 0 (the pages use 1/sqrt(d)).
 *   - head_dim d must be 64 or 128.  Pointers must be 16-byte aligned.
 */
#ifndef ATTN_GFX950_H
#define ATTN_GFX950_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type.  The two range markers are not types: they make every int a
   valid value of the enum, so a caller's out-of-range dtype is an argument
   error (ATTN_ERR_DTYPE), not undefined behaviour in the library's C++. */
typedef enum {
    ATTN_BF16 = 0,
    ATTN_F32 = 1,
    ATTN_DTYPE_RANGE_MIN_ = -2147483647 - 1,
    ATTN_DTYPE_RANGE_MAX_ = 2147483647
} attn_dtype_t;

enum {
    ATTN_OK = 0,
    ATTN_ERR_NULL = -1,        /* a required pointer is NULL */
    ATTN_ERR_SHAPE = -2,       /* a size is < 1, or too large for 32-bit grid indexing */
    ATTN_ERR_HEAD_DIM = -3,    /* d not in {64, 128} */
    ATTN_ERR_BLOCK_SIZE = -4,  /* block_size not in {16, 32} */
    ATTN_ERR_DTYPE = -5,       /* element type not supported by this entry point */
    ATTN_ERR_ALIGN = -6,       /* a pointer or stride is not 16-byte aligned */
    ATTN_ERR_WORKSPACE = -7,   /* workspace missing or smaller than required */
    ATTN_ERR_LAUNCH = -8,      /* the HIP runtime rejected a launch */
    ATTN_ERR_SCALE = -9,       /* scale is negative, NaN or infinite */
    ATTN_ERR_DEVICE = -10,     /* the current device is not a gfx950 GPU */
    ATTN_ERR_BAD_TABLE = -11,  /* ATTN_DEBUG=1 only: a length or block-table entry breaks the
                                  paged-attention contract (see paged_attn_check) */
    ATTN_ERR_OPTION = -12      /* a field of attn_launch_opts_t is out of range */
};

/*
 * Launch variants of the entry points that take an `opts` pointer.  NULL, or
 * a field left at its "automatic" value (-1, or 0 where stated), selects what
 * the library chooses for the shapes at hand (the measured fastest); the
 * other values force one variant, for tests and tuning.  Set every field:
 * start from attn_launch_opts_default().  Variants marked [same bits] give
 * bit-identical results; the others change only the floating-point summation
 * order (each is checked against the oracle like the default).
 *
 *   prefill_kernel : -1 auto; 0 the plain key loop (three LDS buffers, three
 *                    workgroups per CU); 1 the software-pipelined key loop
 *                    (four LDS buffers, two workgroups per CU) [same bits].
 *   prefill_pair   : -1 auto; 0 one 128-row query tile per workgroup; 1
 *                    query tiles t and n-1-t in one workgroup [same bits].
 *   prefill_order  : -1 auto; tile order of causal grids: 0 per-head ranges,
 *                    heaviest tile first; 1 complementary (heavy and light
 *                    tiles dealt together, for grids of one dispatch round);
 *                    3 tile-major [same bits].
 *   paged_path     : -1 auto; 0 the vector decode kernel (only for max_q_len
 *                    <= 4); 1 the MFMA tile kernel; 2 the decode MFMA
 *                    kernel (only for max_q_len * H / H_kv <= 16).
 *   paged_split_tokens : 0 auto; otherwise the keys per context split
 *                    (rounded up to whole pages, 64-key units on the tile
 *                    kernel; at most 8192 there and 128 pages on the decode
 *                    MFMA kernel).
 *   paged_decode_heads : 0 auto; 1, 2, 4 or 8 query heads of one K/V group
 *                    per vector-decode workgroup (must divide H / H_kv; at
 *                    most 4 with 32-token pages).
 *   paged_tile_map : -1 auto; work mapping of the tile kernel: 0 contiguous
 *                    ranges per XCD, 1 (request, K/V head) pairs dealt
 *                    round-robin, 2 single items round-robin [same bits].
 *   paged_tile_kernel: -1 auto; key loop and workgroup size of the tile
 *                    kernel: 0 the plain loop on 128-row workgroups (three
 *                    per CU); 1 the pipelined loop on 128-row workgroups
 *                    (two per CU); 2 the pipelined loop on 256-row
 *                    workgroups of eight waves (one per CU; each K/V tile
 *                    read once for 256 rows) [same bits].
 *   bwd_pair_q     : -1 auto (on for causal); 0 / 1: query tiles t and
 *                    n-1-t in one dQ workgroup [same bits].
 *   bwd_pair_kv    : -1 auto (on for causal); 0 / 1: key blocks kb and
 *                    nkb-1-kb in one dK/dV workgroup [same bits].
 */
typedef struct {
    int prefill_kernel;
    int prefill_pair;
    int prefill_order;
    int paged_path;
    int paged_split_tokens;
    int paged_decode_heads;
    int paged_tile_map;
    int bwd_pair_q;
    int bwd_pair_kv;
    int paged_tile_kernel;
} attn_launch_opts_t;

/* Fills *opts with the automatic values (no-op for NULL). */
void attn_launch_opts_default(attn_launch_opts_t* opts);

/*
 * Prefill / dense attention (the block-wise forward of "Flash Attention and
 * Paged Attention", section 2, with its is_causal flag).
 *
 *   q, k, v : [B, H, N, d] contiguous, element type `dtype`.
 *   o       : [B, H, N, d] output, same type.
 *   lse     : [B, H, N] fp32 output, natural log; may be NULL.
 *   causal  : 0 = every query sees all N keys; 1 = query i sees keys j <= i.
 *
 * bf16: one launch of the MFMA kernel; key tiles entirely above the diagonal
 * are skipped.  fp32: one launch of the fp32 vector kernel.
 * Requires N >= 1 (every causal row sees at least its own key).
 */
int attn_prefill_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                     int B, int H, int N, int d, float scale, int causal,
                     attn_dtype_t dtype, void* stream);

/*
 * Paged attention over a block-table KV cache: decode (q_len = 1) and chunked
 * prefill (q_len > 1) for a whole batch in one step.
 *
 * Pool ("Flash Attention and Paged Attention", section 3): one tensor
 * [num_blocks, 2, H, block_size, d], K at index 0 and V at index 1 of dim 1.
 * Address of token t of request r, head h ("Chunked attention ... 70x slower",
 * section 2.1): logical block lb = t / block_size, physical block
 * pb = block_table[r][lb], offset t % block_size; element
 *   k_pool + pb * kv_block_stride + (h * block_size + t % block_size) * d + c
 * and likewise from v_pool.  For the pages' pool, k_pool = pool,
 * v_pool = pool + H * block_size * d and kv_block_stride = 2 * H * block_size * d
 * (elements); any other pool with the same per-block [H, block_size, d]
 * layout works too.  Offsets are computed in 64-bit.
 *
 *   q           : packed [sum(q_lens), H, d] bf16; request r's rows start at
 *                 sum_{s<r} q_lens[s].
 *   block_table : int32 [num_seqs, max_blocks_per_seq] device; entries past
 *                 ceil(ctx_lens[r] / block_size) are never read.
 *   ctx_lens    : int32 [num_seqs] device: tokens in the cache for request r,
 *                 INCLUDING its q_lens[r] new tokens (already written).
 *   q_lens      : int32 [num_seqs] device: new query rows of request r.
 *                 Row i of request r sits at position ctx - q_len + i and sees
 *                 keys j <= ctx - q_len + i (causal, bottom-right aligned).
 *   o           : packed [sum(q_lens), H, d] bf16 output.
 *   lse         : packed [sum(q_lens), H] fp32 output; may be NULL.
 *   max_q_len, max_ctx_len : host upper bounds of q_lens and ctx_lens, used
 *                 only to size the grid (a larger bound costs only idle
 *                 workgroups).
 *   workspace   : device scratch of at least paged_attn_workspace_bytes(...)
 *                 bytes (partial results of split contexts); contents on entry
 *                 are ignored.  May be NULL when that function returns 0.
 *
 * Device-side contract: 1 <= q_lens[r] <= ctx_lens[r] <= max_ctx_len,
 * q_lens[r] <= max_q_len, every block-table entry needed lies in
 * [0, num_blocks), and ceil(max_ctx_len / block_size) <= max_blocks_per_seq.
 * The kernels do not check it (a bad entry reads outside the pool; a
 * ctx_lens[r] above max_ctx_len is read as max_ctx_len and a q_lens[r]
 * above max_q_len as max_q_len, so neither can reach past the table row or
 * the workspace, but the result is then wrong);
 * paged_attn_check does, and with the environment variable ATTN_DEBUG=1 every
 * paged call runs that check first, waits for it (the call then synchronises
 * `stream`) and returns ATTN_ERR_BAD_TABLE, launching nothing else, when the
 * contract is broken.  Slots of a request's last block past its context may
 * hold anything (NaN included); they are never used.  Several requests may
 * share (alias) physical blocks.
 *
 * Launches: one partial-attention kernel for the whole batch (per request,
 * head, query tile and context split), plus one log-sum-exp combine kernel
 * when some context is split.  Results do not depend on where the blocks sit
 * in the pool (bit-identical under any permutation of physical blocks).
 */
int paged_attn_fwd(const void* q, const void* k_pool, const void* v_pool,
                   const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                   int block_size, void* o, float* lse,
                   int num_seqs, int H, int d, float scale, int max_blocks_per_seq,
                   int64_t kv_block_stride, int num_blocks, int max_q_len, int max_ctx_len,
                   attn_dtype_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes paged_attn_fwd needs for these host bounds (0 if none). */
size_t paged_attn_workspace_bytes(int num_seqs, int H, int d, int block_size,
                                  int max_q_len, int max_ctx_len);

/*
 * For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: exactly
 * paged_attn_fwd (same arguments, validation, launches and bits), except
 * that the split partials go to a workspace the library owns, a static
 * device array of ATTN_STATIC_WORKSPACE_BYTES on each GPU it runs on (held
 * until the process ends; its address is looked up on the first call on each
 * device).  The call allocates and frees nothing.
 *   - If paged_attn_workspace_bytes(...) for these bounds exceeds
 *     ATTN_STATIC_WORKSPACE_BYTES the call returns ATTN_ERR_WORKSPACE and
 *     launches nothing (64 MiB holds, e.g., 64 decode rows x 32 heads x d 128
 *     with contexts up to ~30 K tokens; use paged_attn_fwd with a caller
 *     workspace beyond that).
 *   - Every call on one GPU uses that GPU's array, which keeps the last
 *     call's contents; nothing in it needs to start at zero (each call writes
 *     every slot it reads).  Calls that overlap on one GPU (other streams,
 *     other host threads) race on it: serialise them.
 */
#define ATTN_STATIC_WORKSPACE_BYTES (64u << 20)
int paged_attn_fwd_static(const void* q, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                          int block_size, void* o, float* lse,
                          int num_seqs, int H, int d, float scale, int max_blocks_per_seq,
                          int64_t kv_block_stride, int num_blocks, int max_q_len, int max_ctx_len,
                          attn_dtype_t dtype, void* stream);

/*
 * Grouped-query attention ("Sequence length doubles, inference time
 * quadruples", further optimisations: several query heads share one key and
 * value head; with one shared K/V head it is multi-query attention): H query
 * heads and H_kv K/V heads, H a multiple of H_kv; query head h uses K/V head
 * h / (H / H_kv) (groups of consecutive query heads).  Everything else is as
 * for the functions above, which are these with H_kv = H.
 *
 * attn_prefill_gqa_fwd: q, o [B, H, N, d]; k, v [B, H_kv, N, d]; lse [B, H, N].
 *   The query tiles of the heads of one group run next to each other, so K/V
 *   of a group is read from HBM once and reused through L2.
 * paged_attn_gqa_fwd: q, o packed [sum(q_lens), H, d], lse [sum(q_lens), H];
 *   the pool holds H_kv heads per block ([H_kv, block_size, d] per block, so
 *   kv_block_stride >= H_kv * block_size * d).  Each K/V page is read once
 *   for all the query heads of a group that one workgroup serves: all of them
 *   on the MFMA tile kernel (from 4 heads per group, or query lengths > 4),
 *   up to 8 on the vector decode kernel (groups of 2, q_len <= 4).
 * paged_attn_gqa_workspace_bytes: the workspace paged_attn_gqa_fwd needs.
 * H % H_kv != 0 or H_kv < 1 is ATTN_ERR_SHAPE.  `opts` selects launch
 * variants (see attn_launch_opts_t; NULL = automatic); an out-of-range field
 * is ATTN_ERR_OPTION.
 */
int attn_prefill_gqa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                         int B, int H, int H_kv, int N, int d, float scale, int causal,
                         attn_dtype_t dtype, const attn_launch_opts_t* opts, void* stream);
int paged_attn_gqa_fwd(const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens,
                       int block_size, void* o, float* lse,
                       int num_seqs, int H, int H_kv, int d, float scale, int max_blocks_per_seq,
                       int64_t kv_block_stride, int num_blocks, int max_q_len, int max_ctx_len,
                       attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                       const attn_launch_opts_t* opts, void* stream);
/* Workspace for paged_attn_gqa_fwd with the same bounds and opts (0 if none
   is needed or the arguments are invalid). */
size_t paged_attn_gqa_workspace_bytes(int num_seqs, int H, int H_kv, int d, int block_size,
                                      int max_q_len, int max_ctx_len, const attn_launch_opts_t* opts);

/*
 * Backward of the prefill attention ("Flash Attention and Paged Attention",
 * section 2: the forward keeps only O and the softmax statistics so that the
 * backward can recompute S and P tile by tile).  Gradients of
 * O = softmax(scale * Q K^T) V (causal or not, as in attn_prefill_gqa_fwd)
 * for an output gradient dO, by the chain rule through the forward's three
 * steps (same page, section 1):
 *   P  = exp(scale * Q K^T - LSE) (recomputed per tile from the saved LSE)
 *   dV = P^T dO,  dP = dO V^T,  D_i = dO_i . O_i,  dS = P * (dP - D),
 *   dQ = scale * dS K,  dK = scale * dS^T Q.
 * With H_kv < H the dK and dV of a K/V head sum over its group of query heads
 * (query head h uses K/V head h / (H / H_kv)).
 *
 *   q, o, dout, dq : [B, H, N, d] bf16 (o: the forward's output).
 *   k, v, dk, dv   : [B, H_kv, N, d] bf16.
 *   lse            : [B, H, N] fp32, the forward's log-sum-exp (natural log).
 *   workspace      : device scratch of at least attn_prefill_bwd_workspace_bytes
 *                    (B, H, N) bytes (8 bytes per query row), 16-byte aligned;
 *                    contents on entry are ignored.
 *   dtype          : ATTN_BF16 only (ATTN_ERR_DTYPE otherwise).
 * q, k, v, o and lse must be the inputs and outputs of one forward call with
 * the same scale and causal flag.  dq, dk, dv and the workspace must not
 * overlap each other or any input.  Every element of dq, dk and dv is
 * written (fp32 accumulation, one bf16 rounding at the end).
 *
 * Launches: one kernel for dQ (it also stores each row's LSE and D in the
 * workspace) and one for dK and dV.  Deterministic: the same inputs give the
 * same bits (no atomics), whatever opts->bwd_pair_q / bwd_pair_kv say.
 */
int attn_prefill_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv,
                     int B, int H, int H_kv, int N, int d, float scale, int causal,
                     attn_dtype_t dtype, void* workspace, size_t workspace_bytes,
                     const attn_launch_opts_t* opts, void* stream);

/* Workspace bytes attn_prefill_bwd needs (0 for invalid sizes). */
size_t attn_prefill_bwd_workspace_bytes(int B, int H, int N);

/*
 * Gather through the block table ("Chunked attention ... 70x slower",
 * section 2.1, the address function): copies K and V of every request,
 * tokens [0, ctx_lens[r]), into packed token-major [sum(ctx_lens), H, d]
 * outputs (request r's tokens start at sum_{s<r} ctx_lens[s]).  The copy is
 * bit-exact and uses the same address computation as paged_attn_fwd.  It is
 * a test and debug aid; the attention itself never gathers.
 *   max_ctx_len : host upper bound of ctx_lens (grid sizing).
 */
int paged_kv_gather(const void* k_pool, const void* v_pool, const int32_t* block_table,
                    const int32_t* ctx_lens, int block_size, int num_seqs, int H, int d,
                    int max_blocks_per_seq, int64_t kv_block_stride, int max_ctx_len,
                    attn_dtype_t dtype, void* k_out, void* v_out, void* stream);

/*
 * KV append with a device-side block allocator ("Flash Attention and Paged
 * Attention", section 3: fixed-size blocks, a free list, per-request page
 * tables that grow by whole blocks; "Sequence length doubles, inference time
 * quadruples", decode stage: every new token's K and V are added to the cache
 * after the tokens already there).  Appends new_lens[r] tokens to every
 * request r of a batch, in one allocation launch and one copy launch.
 *
 *   k_new, v_new : packed [sum(new_lens), H, d] (element type `dtype`); request
 *                  r's rows start at sum_{s<r} new_lens[s].  May be NULL when
 *                  max_new_len == 0.
 *   ctx_lens     : int32 [num_seqs] device: tokens already cached per request.
 *   new_lens     : int32 [num_seqs] device: tokens to append (>= 0).
 *   k_pool, v_pool, kv_block_stride, block_size : the pool and its addressing,
 *                  exactly as for paged_attn_fwd; token ctx_lens[r] + i lands
 *                  in logical block (ctx_lens[r] + i) / block_size, slot
 *                  (ctx_lens[r] + i) % block_size.
 *   block_table  : int32 [num_seqs, max_blocks_per_seq] device, in/out.  On
 *                  entry entries [0, ceil(ctx / block_size)) are the request's
 *                  blocks (ids in [0, num_blocks)); on success entries
 *                  [ceil(ctx / bs), ceil((ctx + new) / bs)) receive the newly
 *                  allocated blocks.  Other entries are untouched.
 *   free_blocks  : int32 [num_blocks] device, the free list as a stack: ids
 *                  free_blocks[0 .. *free_count) are free, the top is at
 *                  *free_count - 1.
 *   free_count   : int32 device scalar, in/out.
 *   new_ctx_lens : int32 [num_seqs] device output ctx + new, or NULL; must not
 *                  be ctx_lens itself.
 *   status       : int32 device scalar output, ATTN_APPEND_*.
 *   max_new_len  : host upper bound of new_lens (sizes the copy launch); a
 *                  new_lens[r] above it is ATTN_APPEND_INVALID.
 *
 * Allocation follows the pages' allocator: a request that needs k more blocks
 * takes k ids off the top of the stack, one pop per block, and requests are
 * served in order -- request r's i-th new block is
 * free_blocks[*free_count - 1 - (sum_{s<r} need_s + i)], and *free_count drops
 * by the batch total.  The append is all-or-nothing: if a request would need
 * more than max_blocks_per_seq table entries (ATTN_APPEND_TABLE_FULL), the
 * batch needs more blocks than are free (ATTN_APPEND_EXHAUSTED), or a length
 * or *free_count is out of range (ATTN_APPEND_INVALID), *status says so and
 * no table entry, pool slot, free_count or new_ctx_lens value changes.
 * Results reach *status asynchronously (read it after the stream reaches the
 * call); the allocator runs on the device so a step needs no host round trip.
 * If an existing table entry a new token lands in is outside [0, num_blocks)
 * that token is skipped and *status becomes ATTN_APPEND_INVALID after the
 * blocks were allocated.  Calls that overlap on the same pool or free list
 * race.
 */
enum {
    ATTN_APPEND_OK = 0,
    ATTN_APPEND_EXHAUSTED = 1,   /* not enough free blocks for the batch */
    ATTN_APPEND_TABLE_FULL = 2,  /* a request would need more than max_blocks_per_seq blocks */
    ATTN_APPEND_INVALID = 3      /* negative length, a length above max_new_len, *free_count out of
                                    range, or bad block id */
};
int paged_kv_append(const void* k_new, const void* v_new, const int32_t* ctx_lens, const int32_t* new_lens,
                    void* k_pool, void* v_pool, int32_t* block_table, int32_t* free_blocks, int32_t* free_count,
                    int32_t* new_ctx_lens, int32_t* status, int block_size, int num_seqs, int H, int d,
                    int max_blocks_per_seq, int64_t kv_block_stride, int num_blocks, int max_new_len,
                    attn_dtype_t dtype, void* stream);

/*
 * Return blocks to the free list (the pages' release): blocks[0 .. n) (int32
 * device) are pushed in order, so blocks[n-1] becomes the top of the stack
 * and is the next one allocated.  All-or-nothing: if *free_count + n would
 * exceed num_blocks (ATTN_APPEND_EXHAUSTED) or an id is outside [0,
 * num_blocks) or *free_count is out of range (ATTN_APPEND_INVALID), *status
 * says so and nothing changes.  Pushing an id that is already free is not
 * detected.
 */
int paged_kv_release(const int32_t* blocks, int n, int32_t* free_blocks, int32_t* free_count, int32_t* status,
                     int num_blocks, void* stream);

/*
 * Check of the paged-attention device-side contract (see paged_attn_fwd):
 * lengths and every block-table entry a request uses, on the device.  *status
 * (int32 device word) receives, asynchronously, ATTN_CHECK_OK (0) or an OR of
 * ATTN_CHECK_LENGTHS (some q_lens[r] < 1, q_lens[r] > ctx_lens[r],
 * ctx_lens[r] > max_ctx_len, q_lens[r] > max_q_len, or a context needing more
 * than max_blocks_per_seq blocks) and ATTN_CHECK_TABLE (an entry among the
 * first ceil(ctx_lens[r] / block_size) of a row, at most max_blocks_per_seq,
 * outside [0, num_blocks)).  It reads only those entries and the length
 * arrays, so it is safe on any inputs of the declared shapes, and it writes
 * *status on every call (no clearing needed).  One workgroup: a debugging aid,
 * not for the per-step path.  Host-side errors: ATTN_ERR_NULL, ATTN_ERR_SHAPE,
 * ATTN_ERR_BLOCK_SIZE, ATTN_ERR_ALIGN (pointers not 4-byte aligned),
 * ATTN_ERR_DEVICE, ATTN_ERR_LAUNCH.
 */
enum { ATTN_CHECK_OK = 0, ATTN_CHECK_LENGTHS = 1, ATTN_CHECK_TABLE = 2 };
int paged_attn_check(const int32_t* block_table, const int32_t* ctx_lens, const int32_t* q_lens, int num_seqs,
                     int block_size, int max_blocks_per_seq, int num_blocks, int max_q_len, int max_ctx_len,
                     int32_t* status, void* stream);

/* Human-readable name of a status code (static string, never NULL). */
const char* attn_strerror(int status);

/* Library version, e.g. "attn_gfx950 1.0". */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_GFX950_H */
