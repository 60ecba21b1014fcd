"""The allocation-free decode entry point against the workspace one.

rope_decode_attn_fwd_noalloc runs the same kernels as rope_decode_attn_fwd with the split
partials in the library's per-GPU scratch instead of a caller workspace, so its output and
lse must equal the workspace entry point's bit for bit.  Two calls in a row, the second
with a smaller input (the scratch keeps the first call's contents); the smaller case is
also held to the attention tolerance against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle as orc
import rope_flashattention_amd as rfa
from rope_flashattention_amd import workloads as wl
from gpu_common import ATTN_TOL, device

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def _case(name):
    w = wl.CACHE_CONFIGS[name]
    ci = wl.generate_cache(w)
    dev = device()
    f = orc.inv_freq(w.base, w.head_dim)[None, :]
    s64, c64 = orc.rope_tables(ci.pos, f, [ci.ntokens], 1.0)
    s64, c64 = orc.round_rne(s64, w.dtype), orc.round_rne(c64, w.dtype)
    lens = (ci.ctx + 1).astype(np.int32)
    t = dict(q=ci.q.to(dev), kc=ci.k_cache.to(dev), vc=ci.v_cache.to(dev),
             lens=torch.from_numpy(lens).to(dev), bt=torch.from_numpy(ci.block_table.astype(np.int32)).to(dev),
             cos=torch.from_numpy(c64).to(w.torch_dtype).to(dev), sin=torch.from_numpy(s64).to(w.torch_dtype).to(dev))
    return w, ci, lens, s64, c64, t


def test_noalloc_equals_workspace_entry_on_two_calls():
    for name in ("decode", "decode-small"):          # the second call is the smaller one
        w, ci, lens, s64, c64, t = _case(name)
        kw = dict(max_seqlen=int(lens.max()), block_table=t["bt"])
        ref_o, ref_l = rfa.rope_decode_attn_fwd(t["q"], t["kc"], t["vc"], t["lens"], t["cos"], t["sin"],
                                                return_lse=True, **kw)
        out = torch.full_like(t["q"], float("nan"))
        lse = torch.full(tuple(t["q"].shape[:2]), float("nan"), dtype=torch.float32, device=t["q"].device)
        rfa.rope_decode_attn_fwd_noalloc(t["q"], t["kc"], t["vc"], t["lens"], t["cos"], t["sin"], out=out, lse=lse,
                                         **kw)
        torch.cuda.synchronize()
        say(f"{w.name}: noalloc vs workspace entry: output equal {torch.equal(out, ref_o)}, "
            f"lse equal {torch.equal(lse, ref_l)}")
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        if name == "decode-small":
            nb, bs, H, D = ci.k_cache.shape
            kc = ci.k_cache.to(torch.float64).numpy().reshape(nb * bs, H, D)
            vc = ci.v_cache.to(torch.float64).numpy().reshape(nb * bs, H, D)
            ro, rl = orc.decode_attention(ci.q.to(torch.float64).numpy(), c64, s64, kc, vc, ci.block_table, lens, bs,
                                          1.0 / D ** 0.5)
            err = np.abs(out.to(torch.float64).cpu().numpy() - ro).max()
            lerr = np.abs(lse.cpu().numpy() - rl).max()
            say(f"{w.name}: noalloc vs oracle max-abs {err:.3e}, lse {lerr:.3e}")
            assert err <= ATTN_TOL[w.dtype] and lerr <= ATTN_TOL[w.dtype]


def test_noalloc_rejects_beyond_its_scratch():
    w, ci, lens, s64, c64, t = _case("decode-small")
    out = torch.empty_like(t["q"])
    # 256 splits of a 5 x 8-head batch need 5*8*256*(128+2)*4 bytes = 5.3 MB: fits; a batch
    # of 64 sequences repeated from it with 256 splits needs 68 MB: beyond the 16 MiB scratch
    q = t["q"].repeat(13, 1, 1)[:64].contiguous()
    lens64 = t["lens"].repeat(13)[:64].contiguous()
    bt = t["bt"].repeat(13, 1)[:64].contiguous()
    with pytest.raises(RuntimeError, match="ROPE_ERR_LIMIT"):
        rfa.rope_decode_attn_fwd_noalloc(q, t["kc"], t["vc"], lens64, t["cos"].repeat(13, 1)[:64].contiguous(),
                                         t["sin"].repeat(13, 1)[:64].contiguous(), out=torch.empty_like(q),
                                         max_seqlen=int(lens.max()), block_table=bt, num_splits=256)
    del out
