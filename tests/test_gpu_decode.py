"""GPU parity of decode-step RoPE + GQA attention over a paged KV cache (rope_decode_attn_fwd).

The caches handed to the kernel are built on the CPU: the seeded previous contents plus
each sequence's new token written by the oracle's RMSNorm + RoPE + cache step and rounded
to the cache dtype; the query tables are the oracle's, rounded likewise.  Both sides see
the same inputs.  Bar: output and lse max-abs within the attention tolerance of the
dtype (1e-4 fp32, 5e-3 fp16, 2e-2 bf16).  The end-to-end test instead runs the whole
decode step on the GPU (tables, cache write, attention) and compares with the oracle's
composition of the same steps.
"""

import dataclasses

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


def f64(t):
    return t.to(torch.float64).cpu().numpy()


def query_tables(ci):
    """Oracle tables of the new tokens' positions, rounded to the dtype: (sin, cos) [B, D]."""
    w = ci.workload
    f = orc.inv_freq(w.base, w.head_dim)[None, :]
    s, c = orc.rope_tables(ci.pos, f, [ci.ntokens], 1.0)
    return orc.round_rne(s, w.dtype), orc.round_rne(c, w.dtype)


def oracle_caches(ci, gamma=True):
    """Previous cache contents with every new token written by the oracle, rounded to dtype."""
    w = ci.workload
    nb, bs, H, D = ci.k_cache.shape
    s64, c64 = query_tables(ci)
    kc, vc = orc.kv_rms_norm_rope_cache(f64(ci.k), f64(ci.v), ci.gamma.double().numpy() if gamma else None, 1e-6,
                                        c64, s64, ci.slots, f64(ci.k_cache).reshape(nb * bs, H, D),
                                        f64(ci.v_cache).reshape(nb * bs, H, D))
    # only the written rows need rounding: the rest are the dtype's own values already
    kc[ci.slots] = orc.round_rne(kc[ci.slots], w.dtype)
    vc[ci.slots] = orc.round_rne(vc[ci.slots], w.dtype)
    return kc, vc


def run_decode(ci, *, lens=None, rotate=True, num_splits=0, layout="BSND", contiguous=False, q=None,
               max_seqlen=None, label="", check=True):
    w = ci.workload
    dev = device()
    nb, bs, H, D = ci.k_cache.shape
    B, Hq = w.batch, w.hq
    kc64, vc64 = oracle_caches(ci)
    s64, c64 = query_tables(ci)
    lens = (ci.ctx + 1).astype(np.int32) if lens is None else np.asarray(lens, dtype=np.int32)
    max_seqlen = int(max(1, lens.max())) if max_seqlen is None else max_seqlen
    table = ci.block_table
    if contiguous:
        table = np.arange(nb, dtype=np.int64).reshape(B, -1)
    q_cpu = ci.q if q is None else q
    scale = 1.0 / D ** 0.5
    eff = np.clip(lens, 0, max_seqlen)
    ro, rl = orc.decode_attention(f64(q_cpu.cpu()), c64 if rotate else np.ones_like(c64),
                                  s64 if rotate else np.zeros_like(s64), kc64, vc64, table,
                                  np.maximum(eff, 1), bs, scale)
    tdt = w.torch_dtype
    kc = torch.from_numpy(kc64.reshape(nb, bs, H, D)).to(tdt).to(dev)
    vc = torch.from_numpy(vc64.reshape(nb, bs, H, D)).to(tdt).to(dev)
    if layout == "BNSD":
        kc, vc = kc.permute(0, 2, 1, 3).contiguous(), vc.permute(0, 2, 1, 3).contiguous()
    cos = torch.from_numpy(c64).to(tdt).to(dev) if rotate else None
    sin = torch.from_numpy(s64).to(tdt).to(dev) if rotate else None
    bt = None if contiguous else torch.from_numpy(table.astype(np.int32)).to(dev)
    say(f"decode {label} {w.name} B={B} Hq={Hq} Hkv={H} D={D} lens[{eff.min()}..{eff.max()}] splits={num_splits} "
        f"layout={layout} rotate={rotate} paged={not contiguous}")
    o, lse = rfa.rope_decode_attn_fwd(q_cpu.to(dev), kc, vc, torch.from_numpy(lens).to(dev), cos, sin,
                                      max_seqlen=max_seqlen, block_table=bt, softmax_scale=scale, cache_layout=layout,
                                      num_splits=num_splits, return_lse=True)
    torch.cuda.synchronize()
    got, glse = f64(o), lse.cpu().numpy().astype(np.float64)
    if not check:
        return got, glse, ro, rl, eff
    live = eff > 0
    err = np.abs(got[live] - ro[live]).max() if live.any() else 0.0
    lerr = np.abs(glse[live] - rl[live]).max() if live.any() else 0.0
    say(f"  max-abs {err:.3e} lse {lerr:.3e} (tol {ATTN_TOL[w.dtype]})")
    assert np.all(np.isfinite(got))
    assert err <= ATTN_TOL[w.dtype] and lerr <= ATTN_TOL[w.dtype]
    # an empty cache gives a zero output and lse = -inf
    assert np.all(got[~live] == 0.0) and np.all(np.isneginf(glse[~live]))
    return got, glse, ro, rl, eff


def small(**kw):
    return dataclasses.replace(wl.CACHE_CONFIGS["decode-small"], **kw)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f16", 128), ("bf16", 64), ("f16", 64)])
def test_decode_small(dtype, D):
    run_decode(wl.generate_cache(small(dtype=dtype, head_dim=D)))


@pytest.mark.parametrize("hq,hkv", [(2, 2), (32, 1), (40, 1), (64, 2), (12, 4)])
def test_decode_gqa_groups(hq, hkv):
    # group sizes 1, 32, 40 (two column groups, the second partly empty), 32 and 3
    run_decode(wl.generate_cache(small(hq=hq, hkv=hkv, seed=3200 + hq)), label=f"g={hq // hkv}")


@pytest.mark.parametrize("num_splits", [1, 3, 7, 256])
def test_decode_splits(num_splits):
    # 256 splits leave most of them empty for these lengths
    run_decode(wl.generate_cache(small(seed=3300 + num_splits)), num_splits=num_splits)


def test_decode_lengths_edges():
    ci = wl.generate_cache(small(seed=3400))
    # 1 token, one tile exactly, one past, two tiles, and the cache capacity
    run_decode(ci, lens=[1, 32, 33, 64, 304], label="edge lengths")


def test_decode_empty_and_clamped_lengths():
    ci = wl.generate_cache(small(seed=3401))
    lens = (ci.ctx + 1).astype(np.int32)
    lens[1] = 0                      # nothing cached: zero output, lse -inf
    lens[2] = -5
    cap = int(lens.max())
    lens[3] = cap + 7                # above max_seqlen: clamped to it
    run_decode(ci, lens=lens, max_seqlen=cap, label="empty+clamped")


def test_decode_without_rotation_and_layouts():
    ci = wl.generate_cache(small(seed=3402))
    run_decode(ci, rotate=False, label="no rope")
    run_decode(ci, layout="BNSD", label="BNSD cache")
    ci2 = wl.generate_cache(small(seed=3403, block_size=304))
    run_decode(ci2, contiguous=True, label="contiguous")
    run_decode(ci2, contiguous=True, layout="BNSD", label="contiguous BNSD")


def test_decode_strided_query():
    ci = wl.generate_cache(small(seed=3404))
    B, Hq, D = ci.q.shape
    big = torch.zeros((B, Hq + 4, D), dtype=ci.q.dtype)
    big[:, 2:2 + Hq] = ci.q
    run_decode(ci, q=big.to(device())[:, 2:2 + Hq], label="strided q")


def test_decode_long_cache():
    # three sequences with 12001..20000 cached tokens, paged blocks of 64
    w = small(batch=3, hq=16, hkv=4, ctx_range=(12000, 19999), block_size=64, max_len=20032, seed=3405)
    run_decode(wl.generate_cache(w), label="long")


def test_decode_full_size():
    """The benchmarked decode step: 32 sequences, 1024..8192 cached tokens, Hq 64 / Hkv 8."""
    run_decode(wl.generate_cache(wl.CACHE_CONFIGS["decode"]), label="full")


def test_decode_deterministic_and_split_invariant():
    ci = wl.generate_cache(small(seed=3406))
    a, al, *_ = run_decode(ci, num_splits=4, check=False)
    b, bl, *_ = run_decode(ci, num_splits=4, check=False)
    assert np.array_equal(a, b) and np.array_equal(al, bl)
    c, cl, *_ = run_decode(ci, num_splits=1, check=False)
    assert np.abs(a - c).max() <= ATTN_TOL["bf16"]


def test_decode_step_end_to_end():
    """Tables, cache write of the new token and attention all on the GPU, against the oracle."""
    ci = wl.generate_cache(small(seed=3407))
    w = ci.workload
    dev = device()
    nb, bs, H, D = ci.k_cache.shape
    # GPU: tables for the new positions, the cache step, then decode attention
    f = torch.from_numpy(rfa.inv_freq(w.base, D)).to(dev)
    sin, cos = rfa.rope_tables(torch.from_numpy(ci.pos).to(dev), f, [ci.ntokens], D, 1.0, w.torch_dtype)
    kc, vc = ci.k_cache.to(dev), ci.v_cache.to(dev)
    rfa.rope_kv_rms_norm_rope_cache(ci.k.to(dev), ci.v.to(dev), cos, sin, torch.from_numpy(ci.slots).to(dev), kc, vc,
                                    gamma=ci.gamma.to(dev))
    lens = (ci.ctx + 1).astype(np.int32)
    o = rfa.rope_decode_attn_fwd(ci.q.to(dev), kc, vc, torch.from_numpy(lens).to(dev), cos, sin,
                                 max_seqlen=int(lens.max()), block_table=torch.from_numpy(
                                     ci.block_table.astype(np.int32)).to(dev))
    torch.cuda.synchronize()
    # oracle: its own tables (unrounded), cache step and decode attention
    fo = orc.inv_freq(w.base, D)[None, :]
    s64, c64 = orc.rope_tables(ci.pos, fo, [ci.ntokens], 1.0)
    kc64, vc64 = orc.kv_rms_norm_rope_cache(f64(ci.k), f64(ci.v), ci.gamma.double().numpy(), 1e-6, c64, s64, ci.slots,
                                            f64(ci.k_cache).reshape(nb * bs, H, D),
                                            f64(ci.v_cache).reshape(nb * bs, H, D))
    ro, _ = orc.decode_attention(f64(ci.q), c64, s64, kc64, vc64, ci.block_table, lens, bs, 1.0 / D ** 0.5)
    err = np.abs(f64(o) - ro).max()
    say(f"decode step end to end: max-abs {err:.3e}")
    assert err <= ATTN_TOL[w.dtype]


def test_decode_matches_prefill_last_row():
    """A cache written from a prefill's keys: decode of the last query equals the prefill's last row."""
    dev = device()
    w = wl.SMALL[3]                                     # GQA 8/2, D 128, bf16, S 333
    inp = wl.generate(w)
    S, D = w.seqlen, w.head_dim
    f = torch.from_numpy(rfa.inv_freq(w.base, D, [S])).to(dev)
    sin, cos = rfa.rope_tables(torch.arange(S, dtype=torch.int32, device=dev), f, [S], D, 1.0, w.torch_dtype)
    q, k, v = (x.to(dev) for x in (inp.q, inp.k, inp.v))   # BNSD, batch 1
    o = rfa.rope_flash_attn_fwd(q, k, v, cos, sin, causal=True, softmax_scale=w.softmax_scale)
    bs = 16
    nb = (S + bs - 1) // bs
    kc = torch.zeros((nb, bs, w.hkv, D), dtype=w.torch_dtype, device=dev)
    vc = torch.zeros_like(kc)
    kt, vt = k[0].transpose(0, 1).contiguous(), v[0].transpose(0, 1).contiguous()   # [S, Hkv, D]
    rfa.rope_kv_rms_norm_rope_cache(kt, vt, cos, sin, torch.arange(S, dtype=torch.int64, device=dev), kc, vc)
    qd = q[0, :, S - 1].unsqueeze(0).contiguous()     # [1, Hq, D]
    od = rfa.rope_decode_attn_fwd(qd, kc, vc, torch.tensor([S], dtype=torch.int32, device=dev),
                                  cos[S - 1:S].contiguous(), sin[S - 1:S].contiguous(), max_seqlen=S,
                                  softmax_scale=w.softmax_scale)
    torch.cuda.synchronize()
    err = (od[0].float() - o[0, :, S - 1].float()).abs().max().item()
    say(f"decode vs prefill last row: max-abs {err:.3e}")
    assert err <= ATTN_TOL[w.dtype]


@pytest.mark.parametrize("batch", [200, 1030])
def test_decode_many_sequences(batch):
    # 200 sequences: the partial kernel's list of non-empty (sequence, unit, split) items is
    # found by a prefix sum over four blocks of 64 lengths; 1030 (above 1024) takes the grid of
    # all (split, unit, sequence) triples.  Some lengths are zero or clamped.
    w = small(batch=batch, hq=4, hkv=2, head_dim=64, ctx_range=(0, 90), max_len=96, seed=3500 + batch)
    ci = wl.generate_cache(w)
    lens = (ci.ctx + 1).astype(np.int32)
    lens[::7] = 0
    lens[3::11] = 96 + 5
    run_decode(ci, lens=lens, max_seqlen=96, num_splits=3, label=f"{batch} sequences")
