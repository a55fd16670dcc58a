"""MI355X (gfx950) tiled online-softmax attention: thin Python binding.

Every function here only marshals arguments into the C ABI of
``libattn_gfx950.so`` (declared in ``include/attn.h``); all of the attention
work runs in the library's HIP kernels.  PyTorch supplies device memory and
the current stream.  If the library has not been built, the first call raises
``RuntimeError`` -- there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
from pathlib import Path

__all__ = [
    "ATTN_BF16", "ATTN_F32", "AttnError", "library", "lib_path", "exported_symbols",
    "attn_prefill_fwd", "paged_attn_fwd", "paged_attn_workspace_bytes", "paged_attn_fwd_static", "paged_kv_gather",
    "STATIC_WORKSPACE_BYTES",
    "paged_kv_append", "paged_kv_release", "attn_prefill_gqa_fwd", "paged_attn_gqa_fwd",
    "paged_attn_gqa_workspace_bytes", "attn_prefill_bwd", "attn_prefill_bwd_workspace_bytes", "paged_attn_check",
    "attn_launch_opts_default", "LaunchOpts", "attn_strerror", "attn_version", "prefill", "prefill_bwd",
    "paged_attention", "paged_check", "CHECK_OK", "CHECK_LENGTHS", "CHECK_TABLE", "ERR_BAD_TABLE",
    "ERR_OPTION",
    "gather", "kv_append", "kv_release", "APPEND_OK", "APPEND_EXHAUSTED", "APPEND_TABLE_FULL",
    "APPEND_INVALID",
]

PKG = Path(__file__).resolve().parent
LIB_PATH = PKG / "libattn_gfx950.so"

ATTN_BF16 = 0
ATTN_F32 = 1

# device status words of paged_kv_append / paged_kv_release
APPEND_OK, APPEND_EXHAUSTED, APPEND_TABLE_FULL, APPEND_INVALID = 0, 1, 2, 3
# flag bits of paged_attn_check's status word, and the status the paged calls
# return under ATTN_DEBUG=1 when the check fails
CHECK_OK, CHECK_LENGTHS, CHECK_TABLE = 0, 1, 2
ERR_BAD_TABLE = -11
ERR_OPTION = -12
# size of the library-owned workspace of paged_attn_fwd_static (per GPU)
STATIC_WORKSPACE_BYTES = 64 << 20

# every symbol include/attn.h declares
exported_symbols = (
    "attn_prefill_fwd",
    "paged_attn_fwd",
    "paged_attn_workspace_bytes",
    "paged_attn_fwd_static",
    "paged_kv_gather",
    "paged_kv_append",
    "paged_kv_release",
    "attn_prefill_gqa_fwd",
    "paged_attn_gqa_fwd",
    "paged_attn_gqa_workspace_bytes",
    "attn_prefill_bwd",
    "attn_prefill_bwd_workspace_bytes",
    "paged_attn_check",
    "attn_launch_opts_default",
    "attn_strerror",
    "attn_version",
)

_lib = None


class LaunchOpts(ctypes.Structure):
    """attn_launch_opts_t: launch variants of the entry points that take opts
    (include/attn.h documents every field; -1 / 0 = automatic)."""
    _fields_ = [(name, ctypes.c_int) for name in (
        "prefill_kernel", "prefill_pair", "prefill_order", "paged_path", "paged_split_tokens",
        "paged_decode_heads", "paged_tile_map", "bwd_pair_q", "bwd_pair_kv", "paged_tile_kernel")]


def _opts(options):
    """ctypes pointer to an attn_launch_opts_t with the automatic values except
    the fields named in `options` (a dict), or None for options=None."""
    if options is None:
        return None
    o = LaunchOpts()
    library().attn_launch_opts_default(ctypes.byref(o))
    for k, v in options.items():
        if k not in dict(LaunchOpts._fields_):
            raise KeyError("unknown launch option %r" % k)
        setattr(o, k, int(v))
    return ctypes.pointer(o)


class AttnError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__("%s: %s (status %d)" % (what, attn_strerror(code), code))
        self.code = code


def lib_path() -> Path:
    return LIB_PATH


def library():
    """Load libattn_gfx950.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not LIB_PATH.exists():
        raise RuntimeError("libattn_gfx950.so is not built (run __graft_entry__.build() or "
                           "python -m tiled_online_softmax_attention_amd._build)")
    lib = ctypes.CDLL(str(LIB_PATH))
    P, I, F, I64, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_int64, ctypes.c_size_t
    lib.attn_prefill_fwd.argtypes = [P, P, P, P, P, I, I, I, I, F, I, I, P]
    lib.attn_prefill_fwd.restype = I
    lib.paged_attn_fwd.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, F, I, I64, I, I, I, I, P, SZ, P]
    lib.paged_attn_fwd.restype = I
    lib.paged_attn_workspace_bytes.argtypes = [I, I, I, I, I, I]
    lib.paged_attn_workspace_bytes.restype = SZ
    lib.paged_attn_fwd_static.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, F, I, I64, I, I, I, I, P]
    lib.paged_attn_fwd_static.restype = I
    lib.paged_kv_gather.argtypes = [P, P, P, P, I, I, I, I, I, I64, I, I, P, P, P]
    lib.paged_kv_gather.restype = I
    lib.paged_kv_append.argtypes = [P, P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, I64, I, I, I, P]
    lib.paged_kv_append.restype = I
    lib.paged_kv_release.argtypes = [P, I, P, P, P, I, P]
    lib.paged_kv_release.restype = I
    OP = ctypes.POINTER(LaunchOpts)
    lib.attn_launch_opts_default.argtypes = [OP]
    lib.attn_launch_opts_default.restype = None
    lib.attn_prefill_gqa_fwd.argtypes = [P, P, P, P, P, I, I, I, I, I, F, I, I, OP, P]
    lib.attn_prefill_gqa_fwd.restype = I
    lib.paged_attn_gqa_fwd.argtypes = [P, P, P, P, P, P, I, P, P, I, I, I, I, F, I, I64, I, I, I, I, P, SZ, OP, P]
    lib.paged_attn_gqa_fwd.restype = I
    lib.paged_attn_gqa_workspace_bytes.argtypes = [I, I, I, I, I, I, I, OP]
    lib.paged_attn_gqa_workspace_bytes.restype = SZ
    lib.attn_prefill_bwd.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, I, P, SZ, OP, P]
    lib.attn_prefill_bwd.restype = I
    lib.attn_prefill_bwd_workspace_bytes.argtypes = [I, I, I]
    lib.attn_prefill_bwd_workspace_bytes.restype = SZ
    lib.paged_attn_check.argtypes = [P, P, P, I, I, I, I, I, I, P, P]
    lib.paged_attn_check.restype = I
    lib.attn_strerror.argtypes = [I]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_strerror(code: int) -> str:
    return library().attn_strerror(int(code)).decode()


def attn_version() -> str:
    return library().attn_version().decode()


# ---- raw entry points (same names and argument order as the C ABI) -----------

def attn_prefill_fwd(q, k, v, o, lse, B, H, N, d, scale, causal, dtype, stream):
    return library().attn_prefill_fwd(q, k, v, o, lse, B, H, N, d, float(scale), int(causal), int(dtype),
                                      stream)


def paged_attn_fwd(q, k_pool, v_pool, block_table, ctx_lens, q_lens, block_size, o, lse, num_seqs, H, d,
                   scale, max_blocks_per_seq, kv_block_stride, num_blocks, max_q_len, max_ctx_len, dtype,
                   workspace, workspace_bytes, stream):
    return library().paged_attn_fwd(q, k_pool, v_pool, block_table, ctx_lens, q_lens, block_size, o, lse,
                                    num_seqs, H, d, float(scale), max_blocks_per_seq, kv_block_stride,
                                    num_blocks, max_q_len, max_ctx_len, int(dtype), workspace,
                                    workspace_bytes, stream)


def paged_attn_workspace_bytes(num_seqs, H, d, block_size, max_q_len, max_ctx_len) -> int:
    return int(library().paged_attn_workspace_bytes(num_seqs, H, d, block_size, max_q_len, max_ctx_len))


def paged_attn_fwd_static(q, k_pool, v_pool, block_table, ctx_lens, q_lens, block_size, o, lse, num_seqs, H, d,
                          scale, max_blocks_per_seq, kv_block_stride, num_blocks, max_q_len, max_ctx_len, dtype,
                          stream):
    return library().paged_attn_fwd_static(q, k_pool, v_pool, block_table, ctx_lens, q_lens, block_size, o, lse,
                                           num_seqs, H, d, float(scale), max_blocks_per_seq, kv_block_stride,
                                           num_blocks, max_q_len, max_ctx_len, int(dtype), stream)


def paged_kv_gather(k_pool, v_pool, block_table, ctx_lens, block_size, num_seqs, H, d, max_blocks_per_seq,
                    kv_block_stride, max_ctx_len, dtype, k_out, v_out, stream):
    return library().paged_kv_gather(k_pool, v_pool, block_table, ctx_lens, block_size, num_seqs, H, d,
                                     max_blocks_per_seq, kv_block_stride, max_ctx_len, int(dtype), k_out,
                                     v_out, stream)


def paged_kv_append(k_new, v_new, ctx_lens, new_lens, k_pool, v_pool, block_table, free_blocks, free_count,
                    new_ctx_lens, status, block_size, num_seqs, H, d, max_blocks_per_seq, kv_block_stride,
                    num_blocks, max_new_len, dtype, stream):
    return library().paged_kv_append(k_new, v_new, ctx_lens, new_lens, k_pool, v_pool, block_table, free_blocks,
                                     free_count, new_ctx_lens, status, block_size, num_seqs, H, d,
                                     max_blocks_per_seq, kv_block_stride, num_blocks, max_new_len, int(dtype),
                                     stream)


def attn_prefill_gqa_fwd(q, k, v, o, lse, B, H, H_kv, N, d, scale, causal, dtype, opts, stream):
    return library().attn_prefill_gqa_fwd(q, k, v, o, lse, B, H, H_kv, N, d, float(scale), int(causal), int(dtype),
                                          opts, stream)


def paged_attn_gqa_fwd(q, k_pool, v_pool, block_table, ctx_lens, q_lens, block_size, o, lse, num_seqs, H, H_kv, d,
                       scale, max_blocks_per_seq, kv_block_stride, num_blocks, max_q_len, max_ctx_len, dtype,
                       workspace, workspace_bytes, opts, stream):
    return library().paged_attn_gqa_fwd(q, k_pool, v_pool, block_table, ctx_lens, q_lens, block_size, o, lse,
                                        num_seqs, H, H_kv, d, float(scale), max_blocks_per_seq, kv_block_stride,
                                        num_blocks, max_q_len, max_ctx_len, int(dtype), workspace, workspace_bytes,
                                        opts, stream)


def paged_attn_gqa_workspace_bytes(num_seqs, H, H_kv, d, block_size, max_q_len, max_ctx_len, opts=None) -> int:
    return int(library().paged_attn_gqa_workspace_bytes(num_seqs, H, H_kv, d, block_size, max_q_len, max_ctx_len,
                                                        opts))


def attn_launch_opts_default(opts):
    library().attn_launch_opts_default(opts)


def paged_kv_release(blocks, n, free_blocks, free_count, status, num_blocks, stream):
    return library().paged_kv_release(blocks, n, free_blocks, free_count, status, num_blocks, stream)


def attn_prefill_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, N, d, scale, causal, dtype, workspace,
                     workspace_bytes, opts, stream):
    return library().attn_prefill_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, H, H_kv, N, d, float(scale),
                                      int(causal), int(dtype), workspace, workspace_bytes, opts, stream)


def attn_prefill_bwd_workspace_bytes(B, H, N) -> int:
    return int(library().attn_prefill_bwd_workspace_bytes(B, H, N))


# ---- torch-tensor conveniences (marshalling only) -----------------------------

def paged_attn_check(block_table, ctx_lens, q_lens, num_seqs, block_size, max_blocks_per_seq, num_blocks, max_q_len,
                     max_ctx_len, status, stream):
    return library().paged_attn_check(block_table, ctx_lens, q_lens, num_seqs, block_size, max_blocks_per_seq,
                                      num_blocks, max_q_len, max_ctx_len, status, stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float32:
        return ATTN_F32
    raise TypeError("attention tensors must be bfloat16 or float32, got %s" % t.dtype)


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def prefill(q, k, v, causal: bool, scale: float | None = None, out=None, lse=None, want_lse=True,
            stream=None, options=None):
    """O (and LSE) for q [B, H, N, d] and k, v [B, H_kv, N, d] on the GPU (H_kv < H:
    grouped-query attention, query head h reads K/V head h // (H // H_kv)).
    options: launch variants (a dict of attn_launch_opts_t fields) or None."""
    import torch
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (B, H_kv, N, d) or v.shape != k.shape or H % H_kv != 0:
        raise ValueError("q must be [B, H, N, d] and k, v [B, H_kv, N, d] with H a multiple of H_kv")
    for t in (q, k, v):
        if not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v must be contiguous, same dtype and device")
    if scale is None:
        scale = d ** -0.5
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if H_kv == H and options is None:
        rc = attn_prefill_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, scale,
                              1 if causal else 0, _dtype_code(q), _stream(stream))
    else:
        rc = attn_prefill_gqa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, H_kv, N, d, scale,
                                  1 if causal else 0, _dtype_code(q), _opts(options), _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_prefill_fwd")
    return out, lse


def prefill_bwd(q, k, v, o, lse, dout, causal: bool, scale: float | None = None, dq=None, dk=None, dv=None,
                workspace=None, stream=None, options=None):
    """Gradients (dq, dk, dv) of ``prefill`` for the output gradient dout, from
    the forward's q, k, v, o and lse (q, o, dout [B, H, N, d]; k, v [B, H_kv,
    N, d]; lse [B, H, N] fp32); bf16 only."""
    import torch
    B, H, N, d = q.shape
    H_kv = k.shape[1]
    if k.shape != (B, H_kv, N, d) or v.shape != k.shape or H % H_kv != 0:
        raise ValueError("q must be [B, H, N, d] and k, v [B, H_kv, N, d] with H a multiple of H_kv")
    for t in (q, k, v, o, dout):
        if not t.is_contiguous() or t.dtype != q.dtype or t.device != q.device:
            raise ValueError("q, k, v, o, dout must be contiguous, same dtype and device")
    if o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("o and dout must have q's shape")
    if lse.shape != (B, H, N) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    if scale is None:
        scale = d ** -0.5
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    need = attn_prefill_bwd_workspace_bytes(B, H, N)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    rc = attn_prefill_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                          B, H, H_kv, N, d, scale, 1 if causal else 0, _dtype_code(q), _ptr(workspace),
                          workspace.numel() * workspace.element_size(), _opts(options), _stream(stream))
    if rc != 0:
        raise AttnError(rc, "attn_prefill_bwd")
    return dq, dk, dv


def paged_attention(q, pool, block_table, ctx_lens, q_lens, block_size: int, scale: float | None = None,
                    max_q_len: int | None = None, max_ctx_len: int | None = None, out=None, lse=None,
                    want_lse=True, workspace=None, stream=None, options=None):
    """Paged attention over the pool [num_blocks, 2, H_kv, block_size, d] (K at 0, V at 1).

    q: packed [sum(q_lens), H, d] bf16 with H a multiple of H_kv (grouped-query
    attention when H_kv < H); block_table int32 [num_seqs, max_blocks];
    ctx_lens, q_lens int32 [num_seqs] on the device.  max_q_len / max_ctx_len are
    host bounds (read from the tensors with a device sync when omitted)."""
    import torch
    num_blocks, two, H_kv, bs, d = pool.shape
    H = q.shape[1]
    if two != 2 or bs != block_size or H % H_kv != 0:
        raise ValueError("pool must be [num_blocks, 2, H_kv, block_size, d] with H_kv dividing q's heads")
    if not pool.is_contiguous() or not q.is_contiguous() or not block_table.is_contiguous():
        raise ValueError("pool, q and block_table must be contiguous")
    num_seqs, maxb = block_table.shape
    if max_q_len is None:
        max_q_len = int(q_lens.max())
    if max_ctx_len is None:
        max_ctx_len = int(ctx_lens.max())
    if out is None:
        out = torch.empty_like(q)
    if lse is None and want_lse:
        lse = torch.empty(q.shape[:2], dtype=torch.float32, device=q.device)
    op = _opts(options)
    ws_bytes = paged_attn_gqa_workspace_bytes(num_seqs, H, H_kv, d, block_size, max_q_len, max_ctx_len, op)
    if ws_bytes and workspace is None:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=q.device)
    kv_stride = 2 * H_kv * block_size * d
    k_ptr = pool.data_ptr()
    v_ptr = k_ptr + H_kv * block_size * d * pool.element_size()
    sc = d ** -0.5 if scale is None else scale
    wsb = workspace.numel() if workspace is not None else 0
    if H_kv == H and options is None:
        rc = paged_attn_fwd(_ptr(q), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr), _ptr(block_table),
                            _ptr(ctx_lens), _ptr(q_lens), block_size, _ptr(out), _ptr(lse), num_seqs, H, d, sc,
                            maxb, kv_stride, num_blocks, max_q_len, max_ctx_len, _dtype_code(q), _ptr(workspace),
                            wsb, _stream(stream))
    else:
        rc = paged_attn_gqa_fwd(_ptr(q), ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr), _ptr(block_table),
                                _ptr(ctx_lens), _ptr(q_lens), block_size, _ptr(out), _ptr(lse), num_seqs, H, H_kv,
                                d, sc, maxb, kv_stride, num_blocks, max_q_len, max_ctx_len, _dtype_code(q),
                                _ptr(workspace), wsb, op, _stream(stream))
    if rc != 0:
        raise AttnError(rc, "paged_attn_fwd")
    return out, lse


def paged_check(block_table, ctx_lens, q_lens, block_size: int, num_blocks: int, max_q_len: int, max_ctx_len: int,
                status=None, stream=None):
    """Run paged_attn_check on the device; returns the int32 status tensor
    (one element: CHECK_OK, or an OR of CHECK_LENGTHS and CHECK_TABLE),
    written asynchronously on the stream."""
    import torch
    num_seqs, maxb = block_table.shape
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=block_table.device)
    rc = paged_attn_check(_ptr(block_table), _ptr(ctx_lens), _ptr(q_lens), num_seqs, block_size, maxb, num_blocks,
                          max_q_len, max_ctx_len, _ptr(status), _stream(stream))
    if rc != 0:
        raise AttnError(rc, "paged_attn_check")
    return status


def gather(pool, block_table, ctx_lens, block_size: int, total_tokens: int | None = None,
           max_ctx_len: int | None = None, stream=None):
    """K and V of every request through the block table, packed [sum(ctx), H, d]."""
    import torch
    num_blocks, two, H, bs, d = pool.shape
    num_seqs, maxb = block_table.shape
    if total_tokens is None:
        total_tokens = int(ctx_lens.to(torch.int64).sum())
    if max_ctx_len is None:
        max_ctx_len = int(ctx_lens.max())
    k_out = torch.empty((total_tokens, H, d), dtype=pool.dtype, device=pool.device)
    v_out = torch.empty_like(k_out)
    k_ptr = pool.data_ptr()
    v_ptr = k_ptr + H * block_size * d * pool.element_size()
    rc = paged_kv_gather(ctypes.c_void_p(k_ptr), ctypes.c_void_p(v_ptr), _ptr(block_table), _ptr(ctx_lens),
                         block_size, num_seqs, H, d, maxb, 2 * H * block_size * d, max_ctx_len,
                         _dtype_code(pool), _ptr(k_out), _ptr(v_out), _stream(stream))
    if rc != 0:
        raise AttnError(rc, "paged_kv_gather")
    return k_out, v_out


def _status_error(code: int, what: str) -> RuntimeError:
    names = {APPEND_EXHAUSTED: "KV cache exhausted (not enough free blocks)",
             APPEND_TABLE_FULL: "a request would outgrow its block table",
             APPEND_INVALID: "invalid length, free count or block id"}
    return RuntimeError("%s: %s" % (what, names.get(code, "status %d" % code)))


def kv_append(k_new, v_new, ctx_lens, new_lens, pool, block_table, free_blocks, free_count, block_size: int,
              max_new_len: int | None = None, new_ctx_lens=None, status=None, check: bool = True, stream=None):
    """Append new K/V rows to the paged pool [num_blocks, 2, H, bs, d], allocating
    blocks on the device (paged_kv_append).  With check=True the call waits for
    the stream and raises RuntimeError when the device reports a failure (the
    append then changed nothing); with check=False it returns the device status
    tensor without waiting.  Returns (new_ctx_lens, status)."""
    import torch
    num_blocks, two, H, bs, d = pool.shape
    num_seqs, maxb = block_table.shape
    if max_new_len is None:
        max_new_len = int(new_lens.max()) if new_lens.numel() else 0
    if new_ctx_lens is None:
        new_ctx_lens = torch.empty_like(ctx_lens)
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=pool.device)
    k_ptr = pool.data_ptr()
    v_ptr = k_ptr + H * block_size * d * pool.element_size()
    rc = paged_kv_append(_ptr(k_new), _ptr(v_new), _ptr(ctx_lens), _ptr(new_lens), ctypes.c_void_p(k_ptr),
                         ctypes.c_void_p(v_ptr), _ptr(block_table), _ptr(free_blocks), _ptr(free_count),
                         _ptr(new_ctx_lens), _ptr(status), block_size, num_seqs, H, d, maxb,
                         2 * H * block_size * d, num_blocks, max_new_len, _dtype_code(pool), _stream(stream))
    if rc != 0:
        raise AttnError(rc, "paged_kv_append")
    if check:
        code = int(status.item())
        if code != APPEND_OK:
            raise _status_error(code, "paged_kv_append")
    return new_ctx_lens, status


def kv_release(blocks, free_blocks, free_count, num_blocks: int, status=None, check: bool = True, stream=None):
    """Push block ids back on the device free list (paged_kv_release)."""
    import torch
    if status is None:
        status = torch.empty(1, dtype=torch.int32, device=free_blocks.device)
    rc = paged_kv_release(_ptr(blocks), int(blocks.numel()), _ptr(free_blocks), _ptr(free_count), _ptr(status),
                          num_blocks, _stream(stream))
    if rc != 0:
        raise AttnError(rc, "paged_kv_release")
    if check:
        code = int(status.item())
        if code != APPEND_OK:
            raise _status_error(code, "paged_kv_release")
    return status
