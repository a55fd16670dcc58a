"""The library on caller streams: every entry point enqueues on the stream it
is given and keeps no state between calls, so results on a side stream, on
two streams at once, and from a captured HIP graph replayed several times
are bit-identical to a plain call on the default stream.  (Streams are
created at the default priority.)"""
import pytest
import torch

import tiled_online_softmax_attention_amd as attn
from tiled_online_softmax_attention_amd import inputs
from parity import log

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def same(a, b):
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def prefill_case():
    cfg = inputs.PrefillConfig("streams", 2, 4, 700, 128, torch.bfloat16, True, 21, H_kv=2)
    q, k, v = inputs.prefill_inputs(cfg, DEV)
    return cfg, q, k, v


def paged_case():
    return inputs.build_paged([900, 64, 1, 3000, 257], [1, 1, 1, 1, 1], 4, 128, 16, 22, DEV)


def paged_call(pi, out, lse, ws, stream=None):
    return attn.paged_attention(pi.q, pi.pool, pi.block_table, pi.ctx_lens, pi.q_lens, pi.block_size, pi.scale,
                                max_q_len=1, max_ctx_len=3000, out=out, lse=lse, workspace=ws, stream=stream)


def paged_buffers(pi):
    ws_bytes = attn.paged_attn_workspace_bytes(pi.num_seqs, pi.H, pi.d, pi.block_size, 1, 3000)
    assert ws_bytes > 0   # this case splits its contexts: partial + combine launches
    return (torch.empty_like(pi.q), torch.empty(pi.q.shape[:2], dtype=torch.float32, device=DEV),
            torch.empty(ws_bytes, dtype=torch.uint8, device=DEV))


def test_side_stream_matches_default():
    cfg, q, k, v = prefill_case()
    pi = paged_case()
    o_ref, l_ref = attn.prefill(q, k, v, True, cfg.scale)
    po_ref, pl_ref = paged_call(pi, *paged_buffers(pi))
    do = inputs.grad_output(cfg, DEV)
    g_ref = attn.prefill_bwd(q, k, v, o_ref, l_ref, do, True, cfg.scale)
    torch.cuda.synchronize()

    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    po, pl, ws = paged_buffers(pi)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(attn.attn_prefill_bwd_workspace_bytes(cfg.B, cfg.H, cfg.N), dtype=torch.uint8, device=DEV)
    log("side stream")
    attn.prefill(q, k, v, True, cfg.scale, out=o, lse=lse, stream=side)
    paged_call(pi, po, pl, ws, stream=side)
    attn.prefill_bwd(q, k, v, o, lse, do, True, cfg.scale, dq=dq, dk=dk, dv=dv, workspace=bws, stream=side)
    side.synchronize()
    assert same(o, o_ref) and same(lse, l_ref)
    assert same(po, po_ref) and same(pl, pl_ref)
    for a, b in zip((dq, dk, dv), g_ref):
        assert same(a, b)


def test_two_streams_at_once():
    cfg, q, k, v = prefill_case()
    pi = paged_case()
    o_ref, l_ref = attn.prefill(q, k, v, True, cfg.scale)
    po_ref, pl_ref = paged_call(pi, *paged_buffers(pi))
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(device=DEV), torch.cuda.Stream(device=DEV)
    outs = []
    log("two streams, 4 rounds")
    for _ in range(4):
        o = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
        po, pl, ws = paged_buffers(pi)
        torch.cuda.synchronize()
        attn.prefill(q, k, v, True, cfg.scale, out=o, lse=lse, stream=s1)
        paged_call(pi, po, pl, ws, stream=s2)
        outs.append((o, lse, po, pl))
    torch.cuda.synchronize()
    for o, lse, po, pl in outs:
        assert same(o, o_ref) and same(lse, l_ref) and same(po, po_ref) and same(pl, pl_ref)


def test_graph_capture_replays():
    """A prefill and a split paged decode captured into one HIP graph: every
    replay, with the program's own eager work and synchronisations between
    replays, gives the eager result."""
    cfg, q, k, v = prefill_case()
    pi = paged_case()
    o_ref, l_ref = attn.prefill(q, k, v, True, cfg.scale)
    po_ref, pl_ref = paged_call(pi, *paged_buffers(pi))
    torch.cuda.synchronize()
    o = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    po, pl, ws = paged_buffers(pi)
    # warm on a side stream first (torch's capture recipe), then capture
    s = torch.cuda.Stream(device=DEV)
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        attn.prefill(q, k, v, True, cfg.scale, out=o, lse=lse)
        paged_call(pi, po, pl, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        attn.prefill(q, k, v, True, cfg.scale, out=o, lse=lse)
        paged_call(pi, po, pl, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        log("graph replay %d" % rep)
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        po.fill_(float("nan"))
        pl.fill_(float("nan"))
        ws.fill_(0xFF)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert same(o, o_ref) and same(lse, l_ref), rep
        assert same(po, po_ref) and same(pl, pl_ref), rep
        # eager work between replays
        attn.prefill(q[:, :1].contiguous(), k[:, :1].contiguous(), v[:, :1].contiguous(), True, cfg.scale)
        torch.cuda.synchronize()
