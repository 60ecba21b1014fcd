"""Helpers for the GPU parity tests: run the HIP path and the oracle on one Inputs."""

import numpy as np
import torch

import oracle as orc
import rope_flashattention_amd as rfa
from rope_flashattention_amd import workloads as wl

DT_NAME = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}
ATTN_TOL = {"f32": 1e-4, "f16": 5e-3, "bf16": 2e-2}


def device():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a GPU")
    return torch.device("cuda:0")


def gpu_tables(inp: wl.Inputs, shared: bool = True, dtype=None):
    """Tables from the HIP path: inv_freq on the host (rope_inv_freq), then rope_tables.

    Dense + shared: one [seqlen, D] table (all sequences have positions 0..S-1).
    Otherwise one row per packed token.  Returns (sin, cos, table_seq_rows).
    """
    w = inp.workload
    dev = device()
    dtype = dtype or w.torch_dtype
    D = w.head_dim
    if not w.varlen and shared:
        f = rfa.inv_freq(w.base, D, [w.seqlen], w.trained_len)
        pos = torch.from_numpy(inp.pos[: w.seqlen]).to(dev)
        s, c = rfa.rope_tables(pos, torch.from_numpy(f).to(dev), [w.seqlen], D, w.pos_scale, dtype)
        return s, c, 0
    f = rfa.inv_freq(w.base, D, inp.seq_lens, w.trained_len)
    pos = torch.from_numpy(inp.pos).to(dev)
    s, c = rfa.rope_tables(pos, torch.from_numpy(f).to(dev), inp.seq_lens, D, w.pos_scale, dtype)
    return s, c, (0 if w.varlen else w.seqlen)


def oracle_tables(inp: wl.Inputs, table_dtype: str = None, mode="fp32"):
    """Oracle (sin, cos) float64 [T, D]; rounded to table_dtype when given (storage model)."""
    w = inp.workload
    f = orc.inv_freq_per_sequence(w.base, inp.seq_lens, w.head_dim, w.trained_len)
    s, c = orc.rope_tables(inp.pos, f, inp.seq_lens, w.pos_scale, mode)
    if table_dtype:
        s, c = orc.round_rne(s, table_dtype), orc.round_rne(c, table_dtype)
    return s, c


def to_dev(inp: wl.Inputs, layout: str = "BNSD"):
    dev = device()
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))
    if layout == "BSND":
        q, k, v = (x.transpose(1, 2).contiguous() for x in (q, k, v))
    return q, k, v


def gpu_attention(inp: wl.Inputs, layout: str = "BNSD", shared_table: bool = True, return_lse: bool = False,
                  rotate: bool = True, causal=None):
    w = inp.workload
    dev = device()
    q, k, v = to_dev(inp, "TND" if w.varlen else layout)
    s, c, tsr = gpu_tables(inp, shared_table)
    kw = dict(causal=w.causal if causal is None else causal, softmax_scale=w.softmax_scale,
              return_lse=return_lse, table_seq_rows=tsr)
    if w.varlen:
        kw.update(layout="TND", cu_seqlens=torch.from_numpy(wl.cu_seqlens(inp.seq_lens)).to(dev),
                  max_seqlen=int(inp.seq_lens.max()))
    else:
        kw.update(layout=layout)
    if rotate:
        return rfa.rope_flash_attn_fwd(q, k, v, c, s, **kw)
    return rfa.rope_flash_attn_fwd(q, k, v, None, None, **kw)


def packed_out(inp: wl.Inputs, o: torch.Tensor, layout: str = "BNSD") -> np.ndarray:
    """GPU output as float64 [T, Hq, D] in packed token order."""
    o = o.to(torch.float64).cpu()
    if inp.workload.varlen:
        return o.numpy()
    if layout == "BSND":
        return o.reshape(-1, o.shape[2], o.shape[3]).numpy()
    return o.permute(0, 2, 1, 3).reshape(-1, o.shape[1], o.shape[3]).numpy()


def oracle_attention(inp: wl.Inputs, causal=None):
    w = inp.workload
    q, k, v = inp.packed()
    s, c = oracle_tables(inp, w.dtype)
    return orc.rope_attention(q, k, v, c, s, inp.seq_lens, w.softmax_scale, w.causal if causal is None else causal)
