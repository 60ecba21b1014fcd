"""GPU parity at full size: every output element of the workloads against the oracle.

The fused forward (tables from rope_tables, one rope_flash_attn_fwd launch in the same
configuration the benchmark times) is compared with the fp64 oracle on every element of
O and of the log-sum-exp, for each (sequence, q head) of the workload.  The oracle runs
one (sequence, q head) per CPU worker (tests/oracle_pool.py).  Bars: max-abs 5e-3 (fp16),
2e-2 (bf16) ([FlashAttention blog], "Attention 的显存坑在哪", is the definition checked).
The long GQA workload is split by kv head so that each test stays short; together they
cover every q head.
"""

import time

import numpy as np
import pytest
import torch

import oracle as orc
import rope_flashattention_amd as rfa
from rope_flashattention_amd import workloads as wl
from gpu_common import ATTN_TOL, device, gpu_attention, oracle_tables, packed_out
from oracle_pool import map_heads

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


_CACHE = {}


def _gpu_run(cfg):
    """Inputs, oracle-side tables and the GPU's O, lse of a full workload (kept per module)."""
    if cfg not in _CACHE:
        w = wl.CONFIGS[cfg]
        inp = wl.generate(w)
        say(f"cfg{cfg}: {w.name}, T={inp.ntokens}, lens={inp.seq_lens.tolist() if w.varlen else w.seqlen}")
        o, lse = gpu_attention(inp, return_lse=True)
        torch.cuda.synchronize()
        got = packed_out(inp, o).astype(np.float32)          # exact: 16-bit values
        glse = lse.cpu().numpy()
        del o, lse
        q, k, v = (x.astype(np.float32) for x in inp.packed())
        s, c = oracle_tables(inp, w.dtype)
        _CACHE.clear()
        _CACHE[cfg] = (inp, q, k, v, s.astype(np.float32), c.astype(np.float32), got, glse)
    return _CACHE[cfg]


def _tasks(cfg, heads):
    inp, q, k, v, s, c, got, glse = _gpu_run(cfg)
    w = inp.workload
    g = w.hq // w.hkv
    starts = orc.segment_starts(inp.seq_lens)
    for b, L in enumerate(inp.seq_lens.tolist()):
        sl = slice(int(starts[b]), int(starts[b]) + L)
        for h in heads:
            yield (q[sl, h], k[sl, h // g], v[sl, h // g], c[sl], s[sl], w.softmax_scale, w.causal, "half",
                   got[sl, h], glse[h, sl])


def _check(cfg, heads):
    inp = _gpu_run(cfg)[0]
    w = inp.workload
    t0 = time.time()
    res = map_heads(_tasks(cfg, heads), int(inp.seq_lens.max()))
    err = max(r[0] for r in res)
    lerr = max(r[1] for r in res)
    say(f"cfg{cfg} {w.name}: heads {heads[0]}..{heads[-1]} x {w.batch} sequences, every element: "
        f"max-abs {err:.3e}, lse {lerr:.3e} (tol {ATTN_TOL[w.dtype]}); {len(res)} oracle heads in "
        f"{time.time() - t0:.1f} s")
    assert all(r[2] for r in res)
    assert err <= ATTN_TOL[w.dtype] and lerr <= ATTN_TOL[w.dtype]


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_full_size_every_element(cfg):
    _check(cfg, list(range(wl.CONFIGS[cfg].hq)))


@pytest.mark.parametrize("kvh", list(range(8)))
def test_full_size_long_gqa_every_element(kvh):
    """B1 H64/8 S16384: the 8 q heads of kv head kvh, all 16384 rows each."""
    w = wl.CONFIGS[5]
    g = w.hq // w.hkv
    _check(5, list(range(kvh * g, (kvh + 1) * g)))


def test_reduced_gqa_eight_head_groups():
    """H64/8 at S=520: eight workgroups along the head-group axis (as the full long GQA
    workload launches), full output against the oracle."""
    w = wl.Workload("reduced GQA B1 H64/8 D128 S520 s=2", "bf16", 1, 64, 8, 128, seqlen=520, base=1e6,
                    pos_scale=2.0, seed=2105)
    inp = wl.generate(w)
    o, lse = gpu_attention(inp, return_lse=True)
    got = packed_out(inp, o)
    qn, kn, vn = inp.packed()
    s, c = oracle_tables(inp, w.dtype)
    ro, rlse = orc.rope_attention(qn, kn, vn, c, s, inp.seq_lens, w.softmax_scale, True)
    err = np.abs(got - ro).max()
    lerr = np.abs(lse.cpu().numpy().astype(np.float64) - rlse).max()
    say(f"{w.name}: max-abs {err:.3e}, lse {lerr:.3e}")
    assert err <= ATTN_TOL[w.dtype] and lerr <= ATTN_TOL[w.dtype]


# --------------------------------------------------------------------------- clamped device lengths
def _varlen_inputs(ntokens, seed, H=4, D=128):
    g = torch.Generator().manual_seed(seed)
    return tuple(torch.randn(ntokens, H, D, generator=g).to(torch.bfloat16) for _ in range(3))


@pytest.mark.parametrize("case", ["above_max_seqlen", "past_ntokens"])
def test_varlen_lengths_clamped(case):
    """A device length above max_seqlen, or an end past ntokens, is clamped to
    L_b = min(cu[b+1] - s_b, max_seqlen, ntokens - s_b): the sequence is computed as its
    first L_b tokens and every row outside the clamped sequences stays unwritten."""
    dev = device()
    H, D = 4, 128
    if case == "above_max_seqlen":
        lens, ntok, maxlen = [100, 300], 400, 200      # sequence 1 clamped to 200 of its 300 rows
    else:
        lens, ntok, maxlen = [100, 400], 400, 400      # sequence 1 ends at 500 > ntokens: 300 rows
    q, k, v = _varlen_inputs(ntok, 77, H, D)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    eff = [min(L, maxlen, ntok - int(s0)) for L, s0 in zip(lens, cu[:-1])]
    n_in = sum(eff)
    pos = np.concatenate([np.arange(L) for L in eff] + [np.zeros(ntok - n_in)]).astype(np.int32)
    f = rfa.inv_freq(1e4, D, [ntok], None)
    s, c = rfa.rope_tables(torch.from_numpy(pos).to(dev), torch.from_numpy(f).to(dev), [ntok], D, 1.0,
                           torch.bfloat16)
    out = torch.full((ntok, H, D), float("nan"), dtype=torch.bfloat16, device=dev)
    _, lse = rfa.rope_flash_attn_fwd(q.to(dev), k.to(dev), v.to(dev), c, s, layout="TND",
                                     cu_seqlens=torch.from_numpy(cu).to(dev), max_seqlen=maxlen,
                                     softmax_scale=D ** -0.5, out=out, return_lse=True)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    assert np.isnan(got[n_in:]).all(), "rows outside the clamped sequences must stay unwritten"
    rs, rc = orc.rope_tables(pos[:n_in], orc.inv_freq_per_sequence(1e4, eff, D, None), eff, 1.0)
    rs, rc = orc.round_rne(rs, "bf16"), orc.round_rne(rc, "bf16")
    ro, rlse = orc.rope_attention(q[:n_in].double().numpy(), k[:n_in].double().numpy(), v[:n_in].double().numpy(),
                                  rc, rs, eff, D ** -0.5, True)
    err = np.abs(got[:n_in] - ro).max()
    lerr = np.abs(lse.cpu().numpy()[:, :n_in] - rlse).max()
    say(f"clamped lengths {case}: effective {eff}, max-abs {err:.3e}, lse {lerr:.3e}")
    assert err <= ATTN_TOL["bf16"] and lerr <= ATTN_TOL["bf16"]


def test_varlen_lengths_clamped_backward():
    """The backward clamps the same way: gradients of the clamped sequences match the
    backward of those sequences passed with exact lengths, and other rows stay unwritten."""
    dev = device()
    H, D = 4, 128
    ntok, maxlen = 400, 200
    q, k, v = (x.to(dev) for x in _varlen_inputs(ntok, 78, H, D))
    f = torch.from_numpy(rfa.inv_freq(1e4, D, [ntok], None)).to(dev)
    pos = torch.arange(ntok, dtype=torch.int32, device=dev) % 200
    s, c = rfa.rope_tables(pos, f, [ntok], D, 1.0, torch.bfloat16)
    dout = torch.randn(ntok, H, D, generator=torch.Generator().manual_seed(79)).to(torch.bfloat16).to(dev)
    cu_bad = torch.tensor([0, 100, 400], dtype=torch.int32, device=dev)   # 300 rows > max_seqlen
    cu_ok = torch.tensor([0, 100, 300], dtype=torch.int32, device=dev)
    kw = dict(layout="TND", max_seqlen=maxlen, softmax_scale=D ** -0.5)
    o, lse = rfa.rope_flash_attn_fwd(q, k, v, c, s, cu_seqlens=cu_ok, return_lse=True, **kw)
    grads = []
    for cu_d in (cu_ok, cu_bad):
        dq, dk, dv = (torch.full_like(x, float("nan")) for x in (q, k, v))
        rfa.rope_flash_attn_bwd(q, k, v, o, lse, dout, c, s, cu_seqlens=cu_d, dq=dq, dk=dk, dv=dv, **kw)
        grads.append((dq, dk, dv))
    torch.cuda.synchronize()
    for a, b in zip(*grads):
        assert torch.equal(a[:300], b[:300])
        assert torch.isnan(b[300:].float()).all()
