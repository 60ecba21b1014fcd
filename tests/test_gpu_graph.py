"""The HIP path under HIP-graph capture: a captured step replays to the eager result.

The library allocates nothing and sets no memory inside its launches, so a caller can capture
them.  The step here is the hot path plus the adjacent rows: rope_tables, the fused forward
(with lse), its backward, the KV-cache write and a decode step, all into preallocated buffers
(lse and the decode output come from the graph's own memory pool).  The graph is replayed
several times, with eager work, output clearing and synchronisation between the replays, and
every replay must match the eager run bit for bit.
"""

import dataclasses

import numpy as np
import pytest
import torch

import rope_flashattention_amd as rfa
from rope_flashattention_amd import workloads as wl
from gpu_common import device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def test_graph_replay_matches_eager():
    dev = device()
    w = dataclasses.replace(wl.SMALL[3], seed=6100)  # GQA, bf16, causal
    inp = wl.generate(w)
    D = w.head_dim
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    f = torch.from_numpy(rfa.inv_freq(w.base, D, [w.seqlen], w.trained_len)).to(dev)
    pos = torch.arange(w.seqlen, dtype=torch.int32, device=dev)
    lens = np.array([w.seqlen], dtype=np.int32)
    sin = torch.empty((w.seqlen, D), dtype=w.torch_dtype, device=dev)
    cos = torch.empty_like(sin)
    out = torch.empty_like(q)
    dout = wl.generate_dout(inp, 6101).to(dev)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    bws = torch.empty(4 * (q.numel() + k.numel()) * q.element_size() + (1 << 20), dtype=torch.uint8, device=dev)

    cw = wl.CACHE_CONFIGS["decode-small"]
    ci = wl.generate_cache(cw)
    kc, vc = ci.k_cache.to(dev), ci.v_cache.to(dev)
    ck, cvv = ci.k.to(dev), ci.v.to(dev)
    slots = torch.from_numpy(ci.slots).to(dev)
    gamma = ci.gamma.to(dev)
    cf = torch.from_numpy(rfa.inv_freq(cw.base, cw.head_dim)).to(dev)
    csin, ccos = rfa.rope_tables(torch.from_numpy(ci.pos).to(dev), cf, [cw.batch], cw.head_dim, 1.0, cw.torch_dtype)
    dlens = torch.from_numpy((ci.ctx + 1).astype(np.int32)).to(dev)
    bt = torch.from_numpy(ci.block_table.astype(np.int32)).to(dev)
    dq_in = ci.q.to(dev)
    dkw = dict(max_seqlen=int((ci.ctx + 1).max()), block_table=bt)
    dws = torch.empty(rfa.decode_workspace_size(dq_in, kc, vc, dlens, **dkw), dtype=torch.uint8, device=dev)
    dout_dec = torch.empty_like(dq_in)
    kc0, vc0 = kc.clone(), vc.clone()

    def step():
        rfa.rope_tables(pos, f, lens, D, w.pos_scale, w.torch_dtype, sin, cos)
        o, lse = rfa.rope_flash_attn_fwd(q, k, v, cos, sin, softmax_scale=w.softmax_scale, out=out, return_lse=True)
        rfa.rope_flash_attn_bwd(q, k, v, o, lse, dout, cos, sin, softmax_scale=w.softmax_scale, dq=dq, dk=dk, dv=dv,
                                workspace=bws)
        kc.copy_(kc0)
        vc.copy_(vc0)
        rfa.rope_kv_rms_norm_rope_cache(ck, cvv, ccos, csin, slots, kc, vc, gamma=gamma)
        rfa.rope_decode_attn_fwd(dq_in, kc, vc, dlens, ccos, csin, out=dout_dec, workspace=dws, **dkw)
        return lse

    outs = (out, dq, dk, dv, kc, vc, dout_dec)
    lse_e = step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs] + [lse_e.clone()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lse_g = step()

    junk = torch.randn(1024, 1024, device=dev)
    for rep in range(4):
        for x in outs:
            x.zero_()
        lse_g.zero_()
        junk = junk @ junk.T / 1024.0  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = list(outs) + [lse_g]
        same = [torch.equal(a, b) for a, b in zip(got, ref)]
        say(f"replay {rep}: out, dq, dk, dv, k_cache, v_cache, decode out, lse equal to eager: {same}")
        assert all(same)


def test_graph_replay_prepass_forward():
    """The forward with the k' pre-pass (two launches into a caller workspace) captured with the
    table pass; every replay equals the eager call and the in-loop call bit for bit."""
    dev = device()
    w = dataclasses.replace(wl.SMALL[5], seed=6200)  # GQA 8:1, S520: the plan takes the pre-pass
    inp = wl.generate(w)
    D = w.head_dim
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    f = torch.from_numpy(rfa.inv_freq(w.base, D, [w.seqlen], w.trained_len)).to(dev)
    pos = torch.arange(w.seqlen, dtype=torch.int32, device=dev)
    lens = np.array([w.seqlen], dtype=np.int32)
    sin = torch.empty((w.seqlen, D), dtype=w.torch_dtype, device=dev)
    cos = torch.empty_like(sin)
    rfa.rope_tables(pos, f, lens, D, w.pos_scale, w.torch_dtype, sin, cos)
    need = rfa.flash_attn_fwd_workspace_size(q, k, v, cos, sin)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.hq, inp.ntokens), dtype=torch.float32, device=dev)

    def step():
        rfa.rope_tables(pos, f, lens, D, w.pos_scale, w.torch_dtype, sin, cos)
        o, l = rfa.rope_flash_attn_fwd(q, k, v, cos, sin, softmax_scale=w.softmax_scale, out=out, return_lse=True,
                                       workspace=ws)
        lse.copy_(l)

    step()
    torch.cuda.synchronize()
    ref_o, ref_l = out.clone(), lse.clone()
    io, il = rfa.rope_flash_attn_fwd(q, k, v, cos, sin, softmax_scale=w.softmax_scale, return_lse=True,
                                     workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(io, ref_o) and torch.equal(il, ref_l)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()

    junk = torch.randn(1024, 1024, device=dev)
    for rep in range(4):
        out.zero_()
        lse.zero_()
        ws.zero_()
        junk = junk @ junk.T / 1024.0  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        same = torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        say(f"pre-pass forward replay {rep}: out and lse equal to eager: {same}")
        assert same
