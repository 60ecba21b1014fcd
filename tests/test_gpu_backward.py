"""GPU parity of the backward pass (rope_flash_attn_bwd) against the fp64 oracle.

The GPU forward runs first (its out and lse are the backward's inputs, as in training);
the oracle differentiates the exact forward.  Bar, element by element for each of dq, dk,
dv: |got - ref| <= u (8 |ref| + 64 rms(ref)) + 2^-16 with u the unit roundoff of the input type
(tests/bwd_bar.py: the kernels' rounding points - q', k', P, dS, the forward's O, the
stored gradients - emulated in float64 stay within half of it, tests/test_bwd_bar.py).
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle as orc
import rope_flashattention_amd as rfa
from rope_flashattention_amd import workloads as wl
from gpu_common import device, gpu_tables, packed_out, to_dev
from bwd_bar import backward_bar

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def run_bwd(inp, *, layout="BNSD", causal=None, pairing="half", rotate=True, seed=4242, check=True):
    w = inp.workload
    dev = device()
    causal = w.causal if causal is None else causal
    lay = "TND" if w.varlen else layout
    q, k, v = to_dev(inp, lay)
    dout_bnsd = wl.generate_dout(inp, seed)
    dout = dout_bnsd.to(dev)
    if lay == "BSND":
        dout = dout.transpose(1, 2).contiguous()
    if rotate:
        if pairing == "half":
            s, c, tsr = gpu_tables(inp, shared=False)
        else:
            f = torch.from_numpy(rfa.inv_freq(w.base, w.head_dim, inp.seq_lens, w.trained_len)).to(dev)
            s, c = rfa.rope_tables(torch.from_numpy(inp.pos).to(dev), f, inp.seq_lens, w.head_dim, w.pos_scale,
                                   w.torch_dtype, pairing=pairing)
            tsr = 0 if w.varlen else w.seqlen
    else:
        s = c = None
        tsr = 0
    kw = dict(causal=causal, softmax_scale=w.softmax_scale, table_seq_rows=tsr, pairing=pairing)
    if w.varlen:
        kw.update(layout="TND", cu_seqlens=torch.from_numpy(wl.cu_seqlens(inp.seq_lens)).to(dev),
                  max_seqlen=int(inp.seq_lens.max()))
    else:
        kw.update(layout=layout)
    say(f"backward {w.name} {lay} causal={causal} pairing={pairing} rotate={rotate}")
    o, lse = rfa.rope_flash_attn_fwd(q, k, v, c, s, return_lse=True, **kw)
    dq, dk, dv = rfa.rope_flash_attn_bwd(q, k, v, o, lse, dout, c, s, **kw)
    torch.cuda.synchronize()
    got = [packed_out(inp, x, lay) for x in (dq, dk, dv)]
    if not check:
        return got
    qn, kn, vn = inp.packed()
    don = packed_out(inp, dout, lay)
    if rotate:
        f = orc.inv_freq_per_sequence(w.base, inp.seq_lens, w.head_dim, w.trained_len)
        rs, rc = orc.rope_tables(inp.pos, f, inp.seq_lens, w.pos_scale, "fp32", pairing)
        rs, rc = orc.round_rne(rs, w.dtype), orc.round_rne(rc, w.dtype)
    else:
        rc = np.ones((inp.ntokens, w.head_dim))
        rs = np.zeros((inp.ntokens, w.head_dim))
    ref = orc.rope_attention_bwd(qn, kn, vn, don, rc, rs, inp.seq_lens, w.softmax_scale, causal, pairing)
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        err = np.abs(g - r)
        bar = backward_bar(r, w.dtype)
        ratio = float((err / bar).max())
        say(f"  {name}: max-abs {err.max():.3e}, max|ref| {np.abs(r).max():.3e}, "
            f"max over the elements of err / bar {ratio:.3f}")
        assert np.all(np.isfinite(g))
        assert np.all(err <= bar), name
    return got


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_backward_small(cfg):
    run_bwd(wl.generate(wl.SMALL[cfg]))


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f16", 64), ("f16", 128)])
def test_backward_dtypes_and_dims(dtype, D):
    w = dataclasses.replace(wl.SMALL[3], dtype=dtype, head_dim=D, seed=5100 + D)
    run_bwd(wl.generate(w))


def test_backward_non_causal_interleaved_plain():
    inp = wl.generate(dataclasses.replace(wl.SMALL[3], seed=5200))
    run_bwd(inp, causal=False)
    run_bwd(inp, pairing="interleaved")
    run_bwd(inp, rotate=False)


def test_backward_bsnd_layout():
    run_bwd(wl.generate(dataclasses.replace(wl.SMALL[2], seed=5300)), layout="BSND")


@pytest.mark.parametrize("batch,hq,hkv", [(3, 8, 8), (5, 16, 8), (3, 16, 4)])
def test_backward_xcd_group_counts(batch, hq, hkv):
    """(sequence, kv head) group counts of 24, 40 and 12: three and five groups per XCD (the
    dK/dV grid takes them two at a time and the dQ grid four at a time, so each has a
    partial last chunk) and a count that is not a multiple of 8 (plain order)."""
    w = wl.Workload(f"groups B{batch} H{hq}/{hkv}", "bf16", batch, hq, hkv, 128, seqlen=200, base=1e4,
                    seed=5600 + batch * hq)
    run_bwd(wl.generate(w))


@pytest.mark.parametrize("S", [1, 31, 32, 33, 127, 128, 129, 257])
def test_backward_edge_lengths(S):
    w = dataclasses.replace(wl.SMALL[3], seqlen=S, seed=5400 + S)
    run_bwd(wl.generate(w))


def test_backward_varlen_edges():
    # lengths 1, a tile multiple and ragged ones in one packed batch
    w = dataclasses.replace(wl.SMALL[4], batch=5, len_range=(1, 260), seed=5500)
    inp = wl.generate(w)
    inp.seq_lens[:] = np.array([1, 128, 129, 33, 64], dtype=np.int32)
    T = int(inp.seq_lens.sum())
    inp.q, inp.k, inp.v = inp.q[:T], inp.k[:T], inp.v[:T]
    inp.pos = np.concatenate([np.arange(L, dtype=np.int32) for L in inp.seq_lens.tolist()])
    run_bwd(inp)


def test_backward_full_size_gqa():
    """The llama3-8b-like GQA workload at its full size (B2 H32/8 S4096), every element."""
    run_bwd(wl.generate(wl.CONFIGS[3]))


def test_backward_deterministic():
    inp = wl.generate(dataclasses.replace(wl.SMALL[5], seed=5600))
    a = run_bwd(inp, check=False)
    b = run_bwd(inp, check=False)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
