"""fp64 CPU oracle for tiled online-softmax attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product library never links, loads
or calls it, and it imports nothing from the product package.

The arithmetic lives in ``attn_oracle.c`` (plain C, fp64, OpenMP over
independent heads/rows); this module only builds that file with gcc and
marshals arrays through ctypes.  What each entry point computes, and which
passage of the source pages it follows, is stated in the C file's comments:

* ``attention``            -- softmax(scale * Q K^T) V with optional causal mask,
                              materialised S and P, two-pass softmax, plus LSE
                              (answer.freetools.me page, attention equation;
                              ipipp.com page, sections 1-2).
* ``attention_rows``       -- the same for sampled (b, h, row) triples.
* ``paged_attention``      -- per-token block-table gather (cf-1.com page,
                              section 2.1; pool layout of the ipipp.com page,
                              section 3), then the same definition with the
                              bottom-right causal limit.
* ``paged_attention_rows`` -- the same for sampled (request, head, row) triples.
* ``paged_gather``         -- the bit-exact byte copy the gather must reproduce.
* ``tiled_online``         -- the ipipp.com page's block-wise online-softmax
                              forward, in fp64, for the online == two-pass pin.
* ``lse_merge``            -- merge of partial (O_s, lse_s) over a key partition.
* ``attention_bwd``        -- gradients dQ, dK, dV of ``attention`` for a given
                              output gradient dO (chain rule through the three
                              forward steps; the ipipp.com page, section 2,
                              names recomputing S and P in the backward).
* ``attention_bwd_rows``   -- the same for sampled query rows (dQ) and key
                              rows (dK, dV).

The KV-append oracle (block allocator and per-token page writes) is plain
Python in ``oracle/kv_cache.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

_HERE = Path(__file__).resolve().parent
_SRC = _HERE / "attn_oracle.c"
_LIB = _HERE / "liboracle.so"

BF16, F32, F64 = 0, 1, 2

_lib = None


def build(force: bool = True, src: Path | None = None, out: Path | None = None, extra_flags=()) -> Path:
    """Compile the oracle with gcc (-O2, IEEE semantics, OpenMP); extra_flags
    are appended (the sanitizer test builds an instrumented copy this way)."""
    src = Path(src) if src else _SRC
    out = Path(out) if out else _LIB
    if not force and out.exists() and out.stat().st_mtime >= src.stat().st_mtime:
        return out
    tmp = out.with_suffix(".so.tmp%d" % os.getpid())
    cmd = ["gcc", "-O2", "-fno-fast-math", "-fPIC", "-shared", "-fopenmp", "-std=c11", *extra_flags,
           str(src), "-o", str(tmp), "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def _declare(lib):
    P = ctypes.c_void_p
    I = ctypes.c_int
    D = ctypes.c_double
    lib.oracle_attention.argtypes = [P, P, P, I, I, I, I, I, I, I, D, I, P, P]
    lib.oracle_attention_rows.argtypes = [P, P, P, I, I, I, I, I, I, I, D, I, I, P, P, P, P, P]
    lib.oracle_paged_attention.argtypes = [P, I, P, I, P, P, P, I, I, I, I, I, I, I, D, P, P]
    lib.oracle_paged_attention_rows.argtypes = [P, I, P, I, P, P, P, I, I, I, I, I, I, I, D, I, P, P, P, P, P]
    lib.oracle_paged_gather.argtypes = [P, I, P, P, I, I, I, I, I, I, P, P]
    lib.oracle_tiled_online.argtypes = [P, P, P, I, I, I, I, D, I, I, P, P]
    lib.oracle_lse_merge.argtypes = [I, I, P, P, P, P]
    lib.oracle_attention_bwd.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, I, P, P, P]
    lib.oracle_attention_bwd_rows.argtypes = [P, P, P, P, I, I, I, I, I, I, I, D, I,
                                              I, P, P, P, P, I, P, P, P, P, P]
    lib.oracle_num_threads.argtypes = []
    for name in ("oracle_attention", "oracle_attention_rows", "oracle_attention_bwd", "oracle_attention_bwd_rows",
                 "oracle_paged_attention",
                 "oracle_paged_attention_rows", "oracle_paged_gather", "oracle_tiled_online",
                 "oracle_lse_merge", "oracle_num_threads"):
        getattr(lib, name).restype = ctypes.c_int
    return lib


def load(path: Path | None = None):
    """Load (building first if absent) the oracle library."""
    global _lib
    if path is not None:
        return _declare(ctypes.CDLL(str(path)))
    if _lib is None:
        if not _LIB.exists() or _LIB.stat().st_mtime < _SRC.stat().st_mtime:
            build()
        _lib = _declare(ctypes.CDLL(str(_LIB)))
    return _lib


# ---- array marshalling ------------------------------------------------------

def _host_array(x):
    """Return (contiguous numpy array, oracle dtype code) holding x's stored bits."""
    try:
        import torch
        if isinstance(x, torch.Tensor):
            x = x.detach()
            if x.device.type != "cpu":
                x = x.cpu()
            x = x.contiguous()
            if x.dtype == torch.bfloat16:
                return x.view(torch.int16).numpy().view(np.uint16), BF16
            if x.dtype == torch.float32:
                return x.numpy(), F32
            if x.dtype == torch.float64:
                return x.numpy(), F64
            if x.dtype == torch.int32:
                return x.numpy(), None
            raise TypeError("unsupported tensor dtype %s" % x.dtype)
    except ImportError:  # pragma: no cover
        pass
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, BF16
    if x.dtype == np.float32:
        return x, F32
    if x.dtype == np.float64:
        return x, F64
    if x.dtype == np.int32:
        return x, None
    raise TypeError("unsupported array dtype %s" % x.dtype)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _i32(x):
    a, _ = _host_array(x) if not isinstance(x, (list, tuple)) else (np.asarray(x, dtype=np.int32), None)
    return np.ascontiguousarray(a, dtype=np.int32)


def _check(rc, what):
    if rc != 0:
        raise RuntimeError("oracle %s failed with code %d" % (what, rc))


def num_threads() -> int:
    return load().oracle_num_threads()


def attention(q, k, v, scale: float, causal: bool = False):
    """q: [B,H,Nq,d], k/v: [B,Hkv,Nk,d] with H a multiple of Hkv (groups of
    H/Hkv consecutive query heads share a K/V head; Hkv == H is plain
    multi-head attention).  bf16/fp32/fp64.  Returns (o fp64, lse fp64)."""
    qa, dt = _host_array(q)
    ka, dk = _host_array(k)
    va, dv = _host_array(v)
    assert dt == dk == dv is not None
    B, H, Nq, d = qa.shape
    Hkv, Nk = ka.shape[1], ka.shape[2]
    assert ka.shape == (B, Hkv, Nk, d) and va.shape == ka.shape
    o = np.empty((B, H, Nq, d), np.float64)
    lse = np.empty((B, H, Nq), np.float64)
    _check(load().oracle_attention(_ptr(qa), _ptr(ka), _ptr(va), dt, B, H, Hkv, Nq, Nk, d, float(scale),
                                   1 if causal else 0, _ptr(o), _ptr(lse)), "attention")
    return o, lse


def attention_rows(q, k, v, scale: float, causal: bool, bidx, hidx, rows):
    """Sampled rows of ``attention``.  Returns (o [n,d], lse [n])."""
    qa, dt = _host_array(q)
    ka, _ = _host_array(k)
    va, _ = _host_array(v)
    B, H, Nq, d = qa.shape
    Hkv, Nk = ka.shape[1], ka.shape[2]
    bi, hi, ri = _i32(bidx), _i32(hidx), _i32(rows)
    n = len(bi)
    o = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    _check(load().oracle_attention_rows(_ptr(qa), _ptr(ka), _ptr(va), dt, B, H, Hkv, Nq, Nk, d, float(scale),
                                        1 if causal else 0, n, _ptr(bi), _ptr(hi), _ptr(ri), _ptr(o),
                                        _ptr(lse)), "attention_rows")
    return o, lse


def _bwd_operands(q, k, v, do):
    qa, dt = _host_array(q)
    ka, dk = _host_array(k)
    va, dv = _host_array(v)
    oa, do_ = _host_array(do)
    assert dt == dk == dv == do_ is not None
    B, H, Nq, d = qa.shape
    Hkv, Nk = ka.shape[1], ka.shape[2]
    assert ka.shape == (B, Hkv, Nk, d) and va.shape == ka.shape and oa.shape == qa.shape
    return qa, ka, va, oa, dt, B, H, Hkv, Nq, Nk, d


def attention_bwd(q, k, v, do, scale: float, causal: bool = False):
    """Gradients of ``attention`` for output gradient do ([B,H,Nq,d], same dtype
    as q).  Returns (dq [B,H,Nq,d], dk [B,Hkv,Nk,d], dv [B,Hkv,Nk,d]), fp64; a
    K/V head's dk, dv sum over the query heads of its group."""
    qa, ka, va, oa, dt, B, H, Hkv, Nq, Nk, d = _bwd_operands(q, k, v, do)
    dq = np.empty((B, H, Nq, d), np.float64)
    dk = np.empty((B, Hkv, Nk, d), np.float64)
    dv = np.empty((B, Hkv, Nk, d), np.float64)
    _check(load().oracle_attention_bwd(_ptr(qa), _ptr(ka), _ptr(va), _ptr(oa), dt, B, H, Hkv, Nq, Nk, d,
                                       float(scale), 1 if causal else 0, _ptr(dq), _ptr(dk), _ptr(dv)),
           "attention_bwd")
    return dq, dk, dv


def attention_bwd_rows(q, k, v, do, scale: float, causal: bool, q_samples=(), k_samples=()):
    """Sampled rows of ``attention_bwd``: q_samples are (b, h, row) triples
    (rows of dq), k_samples (b, h_kv, key) triples (rows of dk and dv).
    Returns (dq_rows [nq,d], dk_rows [nk,d], dv_rows [nk,d]), fp64."""
    qa, ka, va, oa, dt, B, H, Hkv, Nq, Nk, d = _bwd_operands(q, k, v, do)
    qs = np.asarray(list(q_samples), dtype=np.int32).reshape(-1, 3)
    ks = np.asarray(list(k_samples), dtype=np.int32).reshape(-1, 3)
    qb, qh, qr = (np.ascontiguousarray(qs[:, i]) for i in range(3))
    kb, kh, kr = (np.ascontiguousarray(ks[:, i]) for i in range(3))
    dq = np.empty((len(qs), d), np.float64)
    dk = np.empty((len(ks), d), np.float64)
    dv = np.empty((len(ks), d), np.float64)
    _check(load().oracle_attention_bwd_rows(_ptr(qa), _ptr(ka), _ptr(va), _ptr(oa), dt, B, H, Hkv, Nq, Nk, d,
                                            float(scale), 1 if causal else 0,
                                            len(qs), _ptr(qb), _ptr(qh), _ptr(qr), _ptr(dq),
                                            len(ks), _ptr(kb), _ptr(kh), _ptr(kr), _ptr(dk), _ptr(dv)),
           "attention_bwd_rows")
    return dq, dk, dv


def paged_attention(q, pool, block_table, ctx_lens, q_lens, block_size: int, scale: float):
    """q: packed [sum(q_lens), H, d]; pool: [num_blocks, 2, Hkv, bs, d] with H a
    multiple of Hkv (query head h reads K/V head h // (H // Hkv)).
    Returns (o fp64 [sum(q_lens), H, d], lse fp64 [sum(q_lens), H])."""
    qa, dq = _host_array(q)
    pa, dp = _host_array(pool)
    bt = _i32(block_table)
    cl, ql = _i32(ctx_lens), _i32(q_lens)
    num_blocks, two, Hkv, bs, d = pa.shape
    assert two == 2 and bs == block_size
    num_seqs, maxb = bt.shape
    total_q = int(ql.sum())
    H = qa.shape[1]
    assert qa.shape == (total_q, H, d)
    o = np.empty((total_q, H, d), np.float64)
    lse = np.empty((total_q, H), np.float64)
    _check(load().oracle_paged_attention(_ptr(qa), dq, _ptr(pa), dp, _ptr(bt), _ptr(cl), _ptr(ql), num_seqs,
                                         H, Hkv, d, bs, maxb, num_blocks, float(scale), _ptr(o), _ptr(lse)),
           "paged_attention")
    return o, lse


def paged_attention_rows(q, pool, block_table, ctx_lens, q_lens, block_size: int, scale: float,
                         ridx, hidx, iidx):
    """Sampled (request, head, row-in-request) triples of ``paged_attention``."""
    qa, dq = _host_array(q)
    pa, dp = _host_array(pool)
    bt = _i32(block_table)
    cl, ql = _i32(ctx_lens), _i32(q_lens)
    num_blocks, two, Hkv, bs, d = pa.shape
    H = qa.shape[1]
    num_seqs, maxb = bt.shape
    ri, hi, ii = _i32(ridx), _i32(hidx), _i32(iidx)
    n = len(ri)
    o = np.empty((n, d), np.float64)
    lse = np.empty((n,), np.float64)
    _check(load().oracle_paged_attention_rows(_ptr(qa), dq, _ptr(pa), dp, _ptr(bt), _ptr(cl), _ptr(ql),
                                              num_seqs, H, Hkv, d, bs, maxb, num_blocks, float(scale), n,
                                              _ptr(ri), _ptr(hi), _ptr(ii), _ptr(o), _ptr(lse)),
           "paged_attention_rows")
    return o, lse


def paged_gather(pool, block_table, ctx_lens, block_size: int):
    """Bit-exact K and V of every request, packed [sum(ctx_lens), H, d], same
    storage dtype as the pool (uint16 bits for bf16)."""
    pa, dp = _host_array(pool)
    bt = _i32(block_table)
    cl = _i32(ctx_lens)
    num_blocks, two, H, bs, d = pa.shape
    num_seqs, maxb = bt.shape
    total = int(cl.astype(np.int64).sum())
    k_out = np.empty((total, H, d), pa.dtype)
    v_out = np.empty((total, H, d), pa.dtype)
    _check(load().oracle_paged_gather(_ptr(pa), dp, _ptr(bt), _ptr(cl), num_seqs, H, d, bs, maxb, num_blocks,
                                      _ptr(k_out), _ptr(v_out)), "paged_gather")
    return k_out, v_out


def tiled_online(q, k, v, scale: float, causal: bool, block_size: int):
    """The pages' block-wise online-softmax forward for one head: q [Nq,d], k/v [Nk,d]."""
    qa, dt = _host_array(q)
    ka, _ = _host_array(k)
    va, _ = _host_array(v)
    Nq, d = qa.shape
    Nk = ka.shape[0]
    o = np.empty((Nq, d), np.float64)
    lse = np.empty((Nq,), np.float64)
    _check(load().oracle_tiled_online(_ptr(qa), _ptr(ka), _ptr(va), dt, Nq, Nk, d, float(scale),
                                      1 if causal else 0, int(block_size), _ptr(o), _ptr(lse)),
           "tiled_online")
    return o, lse


def lse_merge(o_parts, lse_parts):
    """Merge partial (O_s [n,d], lse_s [n]) of one row.  Returns (o [d], lse)."""
    op = np.ascontiguousarray(o_parts, dtype=np.float64)
    lp = np.ascontiguousarray(lse_parts, dtype=np.float64)
    n, d = op.shape
    o = np.empty((d,), np.float64)
    lse = np.empty((1,), np.float64)
    _check(load().oracle_lse_merge(n, d, _ptr(op), _ptr(lp), _ptr(o), _ptr(lse)), "lse_merge")
    return o, float(lse[0])
