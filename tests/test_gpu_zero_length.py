"""Packed (varlen) batches whose cu_seqlens hold zero-length sequences.

cu_seqlens lives in device memory, so the host cannot reject an empty sequence; the kernels
treat it as a sequence with no rows (nothing read, nothing written).  The forward (out and
lse) and the backward (dq, dk, dv) must equal, bit for bit, the results for the same batch
with the empty sequences left out (every output element is computed by the same arithmetic
in the same order), and must match the fp64 oracle on that batch at the attention tolerance.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle as orc
import rope_flashattention_amd as rfa
from rope_flashattention_amd import workloads as wl
from gpu_common import ATTN_TOL, device, gpu_tables, oracle_tables

pytestmark = pytest.mark.gpu

LENS = [0, 5, 0, 130, 0, 64, 0]


def say(*a):
    print(*a, flush=True)


def _inputs(dtype, seed):
    nz = [L for L in LENS if L > 0]
    w = wl.Workload("varlen with empty sequences", dtype, len(nz), 4, 2, 128, varlen=True, len_range=(1, 1),
                    base=1e4, seed=seed)
    inp = dataclasses.replace(wl.generate(w), seq_lens=np.asarray(nz, dtype=np.int32))
    T = int(sum(nz))
    g = torch.Generator().manual_seed(seed)
    inp.q = torch.randn(T, 4, 128, generator=g).to(w.torch_dtype)
    inp.k = torch.randn(T, 2, 128, generator=g).to(w.torch_dtype)
    inp.v = torch.randn(T, 2, 128, generator=g).to(w.torch_dtype)
    inp.pos = np.concatenate([np.arange(L, dtype=np.int32) for L in nz])
    return inp


def _cu(lens, dev):
    return torch.from_numpy(np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)).to(dev)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_forward_and_backward_with_empty_sequences(dtype):
    inp = _inputs(dtype, 7300 + (dtype == "f16"))
    w = inp.workload
    dev = device()
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    s, c, tsr = gpu_tables(inp, shared=False)
    assert tsr == 0
    dout = torch.randn(q.shape, generator=torch.Generator().manual_seed(7310)).to(w.torch_dtype).to(dev)
    kw = dict(causal=True, softmax_scale=w.softmax_scale, table_seq_rows=0, layout="TND", max_seqlen=max(LENS))
    res = {}
    for name, lens in (("with empty", LENS), ("without", inp.seq_lens.tolist())):
        say(f"varlen {dtype} {name}: lens {lens}")
        cu = _cu(lens, dev)
        o, lse = rfa.rope_flash_attn_fwd(q, k, v, c, s, return_lse=True, cu_seqlens=cu, **kw)
        dq, dk, dv = rfa.rope_flash_attn_bwd(q, k, v, o, lse, dout, c, s, cu_seqlens=cu, **kw)
        torch.cuda.synchronize()
        res[name] = (o, lse, dq, dk, dv)
    for nm, a, b in zip(("out", "lse", "dq", "dk", "dv"), res["with empty"], res["without"]):
        assert torch.equal(a, b), nm

    o, lse, dq, dk, dv = (x.to(torch.float64).cpu().numpy() for x in res["with empty"])
    qn, kn, vn = inp.packed()
    rs, rc = oracle_tables(inp, w.dtype)
    ro, rlse = orc.rope_attention(qn, kn, vn, rc, rs, inp.seq_lens, w.softmax_scale, True)
    tol = ATTN_TOL[w.dtype]
    err, lerr = np.abs(o - ro).max(), np.abs(lse - rlse).max()
    say(f"  out max-abs {err:.3e}, lse max-abs {lerr:.3e} (tol {tol})")
    assert np.all(np.isfinite(o)) and err <= tol and lerr <= tol
    don = dout.to(torch.float64).cpu().numpy()
    ref = orc.rope_attention_bwd(qn, kn, vn, don, rc, rs, inp.seq_lens, w.softmax_scale, True, "half")
    for nm, g_, r in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        e, bound = np.abs(g_ - r).max(), tol * max(1.0, np.abs(r).max())
        say(f"  {nm}: max-abs {e:.3e}, err/bound {e / bound:.3f}")
        assert np.all(np.isfinite(g_)) and e <= bound, nm
