"""GPU parity of the fused RMSNorm + RoPE + KV-cache write (rope_kv_rms_norm_rope_cache).

The HIP path (through the C ABI) against the fp64 oracle on the same seeded inputs.  The
tables are the oracle's, rounded to the cache dtype and handed to both sides, so the test
isolates the kernel's own arithmetic.  Bars: V and every untouched cache slot bit-exact;
rotated K within 1 ulp of the output dtype plus a float32 arithmetic floor of
4e-6 * (|y_i| + |y_partner|), y the normalised row (the sum of squares, the reciprocal
square root and the rotation are float32; the result is rounded once).
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle as orc
import rope_flashattention_amd as rfa
from rope_flashattention_amd import workloads as wl
from gpu_common import device

pytestmark = pytest.mark.gpu

EPS = 1e-6


def say(*a):
    print(*a, flush=True)


def oracle_tables(ci, dtype):
    w = ci.workload
    f = orc.inv_freq(w.base, w.head_dim)[None, :]
    s, c = orc.rope_tables(ci.pos, f, [ci.ntokens], 1.0)
    return orc.round_rne(s, dtype), orc.round_rne(c, dtype)


def f64(t):
    return t.to(torch.float64).cpu().numpy()


def run_case(ci, *, gamma=True, layout="BSND", slots=None, with_v=True, k=None, v=None, eps=EPS, label=""):
    """Run both sides; check V and untouched slots bit-exact and K within tolerance."""
    w = ci.workload
    dev = device()
    dt = w.dtype
    T, H, D = ci.k.shape
    s64, c64 = oracle_tables(ci, dt)
    slots = ci.slots if slots is None else slots
    k = ci.k if k is None else k
    v = ci.v if v is None else v
    kc0, vc0 = ci.k_cache, ci.v_cache                      # [nb, bs, H, D]
    nb, bs = kc0.shape[0], kc0.shape[1]
    g64 = ci.gamma.to(torch.float64).numpy() if gamma else None

    kc_ref, vc_ref = orc.kv_rms_norm_rope_cache(f64(k), f64(v), g64, eps, c64, s64, slots,
                                                f64(kc0).reshape(nb * bs, H, D), f64(vc0).reshape(nb * bs, H, D))

    def to_layout(c):
        c = c.to(dev)
        return c.permute(0, 2, 1, 3).contiguous() if layout == "BNSD" else c

    kc, vc = to_layout(kc0), to_layout(vc0)
    tdt = w.torch_dtype
    cos = torch.from_numpy(c64).to(tdt).to(dev)
    sin = torch.from_numpy(s64).to(tdt).to(dev)
    say(f"kv-cache {label} {w.name} {dt} T={T} H={H} D={D} layout={layout} gamma={gamma} v={with_v}")
    rfa.rope_kv_rms_norm_rope_cache(k.to(dev), v.to(dev) if with_v else None, cos, sin,
                                    torch.from_numpy(np.asarray(slots)).to(dev), kc, vc if with_v else None,
                                    gamma=ci.gamma.to(dev) if gamma else None, eps=eps, cache_layout=layout)
    torch.cuda.synchronize()
    if layout == "BNSD":
        kc, vc = kc.permute(0, 2, 1, 3), vc.permute(0, 2, 1, 3)
    got_k = f64(kc).reshape(nb * bs, H, D)
    got_v = f64(vc).reshape(nb * bs, H, D)
    if with_v:
        assert np.array_equal(got_v, vc_ref)
    else:
        assert np.array_equal(got_v, f64(vc0).reshape(nb * bs, H, D))
    sl = np.asarray(slots)
    written = np.unique(sl[(sl >= 0) & (sl < nb * bs)])
    untouched = np.setdiff1d(np.arange(nb * bs), written)
    assert np.array_equal(got_k[untouched], kc_ref[untouched])
    # tolerance from the normalised rows of the tokens that were written
    kk = f64(k)
    y = kk if g64 is None else orc.rms_norm(kk, g64, eps)
    partner = np.concatenate([y[..., D // 2:], y[..., :D // 2]], axis=-1)
    floor = 4e-6 * (np.abs(y) + np.abs(partner))
    t_of = np.full(nb * bs, -1)
    for t, s_ in enumerate(sl.tolist()):
        if 0 <= s_ < nb * bs:
            t_of[s_] = t
    ref = kc_ref[written]
    tol = orc.ulp(ref, dt) + floor[t_of[written]]
    err = np.abs(got_k[written] - ref)
    say(f"  K max err/tol {np.max(err / tol) if err.size else 0:.3f} over {written.size} slots")
    assert np.all(np.isfinite(got_k[written]))
    assert np.all(err <= tol)


def small(**kw):
    return dataclasses.replace(wl.CACHE_CONFIGS["small"], **kw)


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_kv_cache_small_paged(dtype):
    run_case(wl.generate_cache(small(dtype=dtype)))


def test_kv_cache_bnsd_contiguous_cache():
    # one block per sequence: a contiguous [B, hkv, S_max, D] cache
    ci = wl.generate_cache(small(block_size=144, max_len=144, seed=3003))
    run_case(ci, layout="BNSD")


def test_kv_cache_without_gamma_and_without_v():
    ci = wl.generate_cache(small(seed=3004))
    run_case(ci, gamma=False, label="no-gamma")
    run_case(ci, with_v=False, label="K only")


def test_kv_cache_skipped_slots():
    ci = wl.generate_cache(small(seed=3005))
    slots = ci.slots.copy()
    nslots = ci.k_cache.shape[0] * ci.k_cache.shape[1]
    slots[::5] = -1                     # padding tokens
    slots[3] = nslots                   # past the cache
    slots[7] = np.iinfo(np.int64).max
    slots[8] = np.iinfo(np.int64).min
    run_case(ci, slots=slots, label="skips")


@pytest.mark.parametrize("D", [32, 64, 96, 256, 1024, 2048])
def test_kv_cache_head_dims(D):
    ci = wl.generate_cache(small(head_dim=D, seed=3100 + D))
    run_case(ci, label=f"D{D}")


def test_kv_cache_strided_qkv_views():
    # k and v as views into one fused [T, hq + 2*hkv, D] projection output
    ci = wl.generate_cache(small(seed=3006))
    T, H, D = ci.k.shape
    hq = 4 * H
    dev = device()
    qkv = torch.zeros((T, hq + 2 * H, D), dtype=ci.k.dtype, device=dev)
    qkv[:, hq:hq + H] = ci.k.to(dev)
    qkv[:, hq + H:] = ci.v.to(dev)
    k, v = qkv[:, hq:hq + H], qkv[:, hq + H:]
    assert not k.is_contiguous()
    run_case(ci, k=k, v=v, label="qkv views")


def test_kv_cache_zero_row_and_empty():
    ci = wl.generate_cache(small(seed=3007))
    k = ci.k.clone()
    k[4, 1] = 0                         # a zero row normalises to zero (eps > 0)
    run_case(ci, k=k, label="zero row")
    # no new tokens: nothing is written
    dev = device()
    kc, vc = ci.k_cache.to(dev), ci.v_cache.to(dev)
    e = torch.empty((0, 2, 128), dtype=ci.k.dtype, device=dev)
    tab = torch.empty((0, 128), dtype=ci.k.dtype, device=dev)
    rfa.rope_kv_rms_norm_rope_cache(e, e, tab, tab, torch.empty(0, dtype=torch.int64, device=dev), kc, vc,
                                    gamma=ci.gamma.to(dev))
    torch.cuda.synchronize()
    assert torch.equal(kc.cpu(), ci.k_cache) and torch.equal(vc.cpu(), ci.v_cache)


def test_kv_cache_full_size_prefill():
    """The benchmarked size: 16 x 4096 new tokens, 8 kv heads, paged cache, every element."""
    ci = wl.generate_cache(wl.CACHE_CONFIGS["prefill"])
    run_case(ci, label="full")


def test_kv_cache_deterministic_and_repeatable():
    ci = wl.generate_cache(small(seed=3008))
    dev = device()
    outs = []
    for _ in range(2):
        kc, vc = ci.k_cache.to(dev), ci.v_cache.to(dev)
        s64, c64 = oracle_tables(ci, ci.workload.dtype)
        rfa.rope_kv_rms_norm_rope_cache(ci.k.to(dev), ci.v.to(dev), torch.from_numpy(c64).to(ci.k.dtype).to(dev),
                                        torch.from_numpy(s64).to(ci.k.dtype).to(dev),
                                        torch.from_numpy(ci.slots).to(dev), kc, vc, gamma=ci.gamma.to(dev))
        outs.append(kc.cpu())
    assert torch.equal(outs[0], outs[1])
