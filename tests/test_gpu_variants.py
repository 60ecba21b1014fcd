"""GPU parity of the RoPE variants: interleaved pairing, tables formed inside the kernels,
and the exact-angle table mode.

Bars: tables within the ulp bounds of the table tests (exact-angle mode: 1 ulp of the
output type against the float64 oracle); rope_qk and the KV-cache step within the rope_qk
bars; attention and decode within the attention tolerances; every "tables formed in the
kernel" result bit-identical to the same call given the tables rope_tables_ex writes.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle as orc
import rope_flashattention_amd as rfa
from rope_flashattention_amd import workloads as wl
from gpu_common import ATTN_TOL, device, packed_out, to_dev

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def f64(t):
    return t.to(torch.float64).cpu().numpy()


def ulp_err(got, ref, dtype):
    return np.abs(np.asarray(got, dtype=np.float64) - ref) / orc.ulp(ref, dtype)


def gpu_tables_for(inp, pairing, per_token=False, dtype=None, angle_mode="f32"):
    """Tables from rope_tables_ex, and the (pos, inv_freq) that produced them."""
    w = inp.workload
    dev = device()
    D = w.head_dim
    dtype = dtype or w.torch_dtype
    if not w.varlen and not per_token:
        f = torch.from_numpy(rfa.inv_freq(w.base, D, [w.seqlen], w.trained_len)).to(dev)
        pos = torch.from_numpy(inp.pos[: w.seqlen]).to(dev)
        s, c = rfa.rope_tables(pos, f, [w.seqlen], D, w.pos_scale, dtype, pairing=pairing, angle_mode=angle_mode)
        return s, c, pos, f, 0
    f = torch.from_numpy(rfa.inv_freq(w.base, D, inp.seq_lens, w.trained_len)).to(dev)
    pos = torch.from_numpy(inp.pos).to(dev)
    s, c = rfa.rope_tables(pos, f, inp.seq_lens, D, w.pos_scale, dtype, pairing=pairing, angle_mode=angle_mode)
    return s, c, pos, f, (0 if w.varlen else w.seqlen)


def oracle_tables_for(inp, pairing, dtype=None, mode="fp32"):
    w = inp.workload
    f = orc.inv_freq_per_sequence(w.base, inp.seq_lens, w.head_dim, w.trained_len)
    s, c = orc.rope_tables(inp.pos, f, inp.seq_lens, w.pos_scale, mode, pairing)
    if dtype:
        s, c = orc.round_rne(s, dtype), orc.round_rne(c, dtype)
    return s, c


def attn_kwargs(inp, layout="BNSD"):
    w = inp.workload
    dev = device()
    if w.varlen:
        return dict(layout="TND", cu_seqlens=torch.from_numpy(wl.cu_seqlens(inp.seq_lens)).to(dev),
                    max_seqlen=int(inp.seq_lens.max()))
    return dict(layout=layout)


# --------------------------------------------------------------------------- tables
@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
def test_tables_interleaved(cfg):
    w = wl.CONFIGS[cfg]
    inp = wl.generate(w)
    si, ci, *_ = gpu_tables_for(inp, "interleaved", per_token=True)
    sh, ch, *_ = gpu_tables_for(inp, "half", per_token=True)
    D = w.head_dim
    # the same values, in the interleaved columns
    assert torch.equal(si[:, 0::2], sh[:, :D // 2]) and torch.equal(si[:, 1::2], sh[:, :D // 2])
    assert torch.equal(ci[:, 0::2], ch[:, :D // 2]) and torch.equal(ci[:, 1::2], ch[:, :D // 2])
    rs, rc = oracle_tables_for(inp, "interleaved")
    es, ec = ulp_err(f64(si), rs, w.dtype).max(), ulp_err(f64(ci), rc, w.dtype).max()
    say(f"interleaved tables {w.name}: sin {es:.3f} ulp, cos {ec:.3f} ulp")
    assert es <= 2.0 and ec <= 2.0


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_tables_exact_angle(dtype, pairing):
    # long positions (where float32 angles lose precision) up to the op's 256000-token limit
    w = dataclasses.replace(wl.CONFIGS[5], dtype=dtype)
    dev = device()
    rng = np.random.default_rng(77)
    lens = np.array([4000, 4000], dtype=np.int32)
    pos = np.concatenate([rng.integers(0, 256000, 4000), rng.integers(200000, 256000, 4000)]).astype(np.int32)
    D = 128
    f = rfa.inv_freq(1e6, D, lens)
    s, c = rfa.rope_tables(torch.from_numpy(pos).to(dev), torch.from_numpy(f).to(dev), lens, D, 2.0,
                           w.torch_dtype, pairing=pairing, angle_mode="exact")
    rs, rc = orc.rope_tables(pos, f, lens, 2.0, "exact", pairing)
    es, ec = ulp_err(f64(s), rs, dtype).max(), ulp_err(f64(c), rc, dtype).max()
    say(f"exact-angle tables {dtype} {pairing}: sin {es:.3f} ulp, cos {ec:.3f} ulp")
    assert es <= 1.0 and ec <= 1.0
    # float32 angles drift from the exact ones at these positions; the exact mode does not
    s32, c32 = rfa.rope_tables(torch.from_numpy(pos).to(dev), torch.from_numpy(f).to(dev), lens, D, 2.0,
                               w.torch_dtype, pairing=pairing)
    assert np.abs(f64(s32) - rs).max() >= np.abs(f64(s) - rs).max()


# --------------------------------------------------------------------------- rope_qk
@pytest.mark.parametrize("cfg", [1, 2, 4, 5])
def test_rope_qk_interleaved(cfg):
    inp = wl.generate(wl.SMALL[cfg])
    w = inp.workload
    D = w.head_dim
    q, k, _ = to_dev(inp, "TND" if w.varlen else "BNSD")
    s, c, pos, f, tsr = gpu_tables_for(inp, "interleaved")
    kw = attn_kwargs(inp)
    oq, ok = rfa.rope_qk(q, k, c, s, table_seq_rows=tsr, pairing="interleaved", **kw)
    rs, rc = oracle_tables_for(inp, "interleaved", w.dtype)
    qn, kn, _ = inp.packed()
    for x, o in ((qn, oq), (kn, ok)):
        ref = orc.rotate_tokens(x, rc, rs, pairing="interleaved")
        got = packed_out(inp, o, "TND" if w.varlen else "BNSD")
        partner = x[..., np.arange(D) ^ 1]
        tol = 2 * orc.ulp(ref, w.dtype) + 1e-6 * (np.abs(x) + np.abs(partner)) \
            + 2 * (np.abs(x) * orc.ulp(rc, w.dtype)[:, None, :] + np.abs(partner) * orc.ulp(rs, w.dtype)[:, None, :])
        err = np.abs(got - ref)
        say(f"rope_qk interleaved {w.name}: max err/tol {np.max(err / tol):.3f}")
        assert np.all(err <= tol)


@pytest.mark.parametrize("cfg", [1, 3, 4, 5])
@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_rope_qk_formed_tables_bit_exact(cfg, pairing):
    inp = wl.generate(wl.SMALL[cfg])
    w = inp.workload
    q, k, _ = to_dev(inp, "TND" if w.varlen else "BNSD")
    s, c, pos, f, tsr = gpu_tables_for(inp, pairing)
    kw = attn_kwargs(inp)
    tq, tk = rfa.rope_qk(q, k, c, s, table_seq_rows=tsr, pairing=pairing, **kw)
    gq, gk = rfa.rope_qk(q, k, None, None, table_seq_rows=tsr, pairing=pairing, pos=pos, inv_freq=f,
                         pos_scale=w.pos_scale, **kw)
    torch.cuda.synchronize()
    say(f"rope_qk formed tables {w.name} {pairing}: equal={torch.equal(tq, gq) and torch.equal(tk, gk)}")
    assert torch.equal(tq, gq) and torch.equal(tk, gk)


# --------------------------------------------------------------------------- fused attention
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_attention_interleaved(cfg):
    inp = wl.generate(wl.SMALL[cfg])
    w = inp.workload
    q, k, v = to_dev(inp, "TND" if w.varlen else "BNSD")
    s, c, pos, f, tsr = gpu_tables_for(inp, "interleaved")
    o, lse = rfa.rope_flash_attn_fwd(q, k, v, c, s, causal=w.causal, softmax_scale=w.softmax_scale,
                                     table_seq_rows=tsr, return_lse=True, pairing="interleaved", **attn_kwargs(inp))
    qn, kn, vn = inp.packed()
    rs, rc = oracle_tables_for(inp, "interleaved", w.dtype)
    ro, rl = orc.rope_attention(qn, kn, vn, rc, rs, inp.seq_lens, w.softmax_scale, w.causal, "interleaved")
    got = packed_out(inp, o, "TND" if w.varlen else "BNSD")
    err = np.abs(got - ro).max()
    lerr = np.abs(lse.cpu().numpy().astype(np.float64) - rl).max()
    say(f"attention interleaved {w.name}: max-abs {err:.3e} lse {lerr:.3e} (tol {ATTN_TOL[w.dtype]})")
    assert err <= ATTN_TOL[w.dtype] and lerr <= ATTN_TOL[w.dtype]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_attention_formed_tables_bit_exact(cfg, pairing):
    inp = wl.generate(wl.SMALL[cfg])
    w = inp.workload
    q, k, v = to_dev(inp, "TND" if w.varlen else "BNSD")
    s, c, pos, f, tsr = gpu_tables_for(inp, pairing)
    kw = dict(causal=w.causal, softmax_scale=w.softmax_scale, table_seq_rows=tsr, return_lse=True,
              pairing=pairing, **attn_kwargs(inp))
    to, tl = rfa.rope_flash_attn_fwd(q, k, v, c, s, **kw)
    go, gl = rfa.rope_flash_attn_fwd(q, k, v, None, None, pos=pos, inv_freq=f, pos_scale=w.pos_scale, **kw)
    torch.cuda.synchronize()
    same = torch.equal(to, go) and torch.equal(tl, gl)
    say(f"attention formed tables {w.name} {pairing}: equal={same}")
    assert same


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_attention_head_dim_64_variants(dtype, pairing):
    """head_dim 64 (the unsliced kernel path) with either pairing, GQA 16/2 (8 q heads per
    workgroup) and a ragged length: tables read against the oracle, and tables formed in
    the kernel bit-identical to them."""
    w = wl.Workload(f"D64 GQA {dtype}", dtype, 2, 16, 2, 64, seqlen=301, base=1e4, seed=5300)
    inp = wl.generate(w)
    q, k, v = to_dev(inp)
    s, c, pos, f, tsr = gpu_tables_for(inp, pairing)
    kw = dict(causal=True, softmax_scale=w.softmax_scale, table_seq_rows=tsr, return_lse=True, pairing=pairing)
    to, tl = rfa.rope_flash_attn_fwd(q, k, v, c, s, **kw)
    go, gl = rfa.rope_flash_attn_fwd(q, k, v, None, None, pos=pos, inv_freq=f, pos_scale=w.pos_scale, **kw)
    torch.cuda.synchronize()
    same = torch.equal(to, go) and torch.equal(tl, gl)
    qn, kn, vn = inp.packed()
    rs, rc = oracle_tables_for(inp, pairing, w.dtype)
    ro, rl = orc.rope_attention(qn, kn, vn, rc, rs, inp.seq_lens, w.softmax_scale, True, pairing)
    err = np.abs(packed_out(inp, to, "BNSD") - ro).max()
    lerr = np.abs(tl.cpu().numpy().astype(np.float64) - rl).max()
    say(f"attention D64 {dtype} {pairing}: formed equal={same} max-abs {err:.3e} lse {lerr:.3e}")
    assert same and err <= ATTN_TOL[w.dtype] and lerr <= ATTN_TOL[w.dtype]


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_attention_formed_tables_large_positions(pairing):
    """Positions near 3e6 (scaled by 1/2: angles up to 1.5e6 rad, past the 2^20 limit of the
    sine/cosine fast path): the kernel forming its tables takes its fallback for those
    angles and still equals the call given the tables rope_tables_ex writes for the same
    positions; both within the attention bar of the oracle."""
    inp = wl.generate(wl.SMALL[5])                      # GQA 16/2, D 128, bf16, S 520, s = 2
    w = inp.workload
    dev = device()
    D, S = w.head_dim, w.seqlen
    q, k, v = to_dev(inp)
    pos_np = (inp.pos[:S].astype(np.int64) + 3_000_000).astype(np.int32)
    pos = torch.from_numpy(pos_np).to(dev)
    f = torch.from_numpy(rfa.inv_freq(w.base, D, [S], w.trained_len)).to(dev)
    s, c = rfa.rope_tables(pos, f, [S], D, w.pos_scale, w.torch_dtype, pairing=pairing)
    kw = dict(causal=True, softmax_scale=w.softmax_scale, return_lse=True, pairing=pairing)
    to, tl = rfa.rope_flash_attn_fwd(q, k, v, c, s, **kw)
    go, gl = rfa.rope_flash_attn_fwd(q, k, v, None, None, pos=pos, inv_freq=f, pos_scale=w.pos_scale, **kw)
    torch.cuda.synchronize()
    same = torch.equal(to, go) and torch.equal(tl, gl)
    fo = orc.inv_freq_per_sequence(w.base, inp.seq_lens, D, w.trained_len)
    rs, rc = orc.rope_tables(pos_np, fo, inp.seq_lens, w.pos_scale, "fp32", pairing)
    rs, rc = orc.round_rne(rs, w.dtype), orc.round_rne(rc, w.dtype)
    qn, kn, vn = inp.packed()
    ro, rl = orc.rope_attention(qn, kn, vn, rc, rs, inp.seq_lens, w.softmax_scale, True, pairing)
    err = np.abs(packed_out(inp, go, "BNSD") - ro).max()
    say(f"attention formed tables, positions ~3e6, {pairing}: equal={same} max-abs {err:.3e}")
    assert same and err <= ATTN_TOL[w.dtype]


@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_attention_formed_tables_full_size(pairing):
    """The benchmarked workload (qwen7b-like, S 2048) with tables formed in the kernel."""
    inp = wl.generate(wl.CONFIGS[2])
    w = inp.workload
    q, k, v = to_dev(inp)
    s, c, pos, f, tsr = gpu_tables_for(inp, pairing)
    kw = dict(causal=True, softmax_scale=w.softmax_scale, pairing=pairing)
    to = rfa.rope_flash_attn_fwd(q, k, v, c, s, **kw)
    go = rfa.rope_flash_attn_fwd(q, k, v, None, None, pos=pos, inv_freq=f, **kw)
    torch.cuda.synchronize()
    assert torch.equal(to, go)
    # sampled rows against the oracle
    qn, kn, vn = inp.packed()
    rs, rc = oracle_tables_for(inp, pairing, w.dtype)
    rng = np.random.default_rng(9)
    samples = [(int(t), int(h)) for t, h in zip(rng.integers(0, inp.ntokens, 24), rng.integers(0, w.hq, 24))]
    ro, _ = orc.rope_attention_rows(qn, kn, vn, rc, rs, inp.seq_lens, w.softmax_scale, True, samples, pairing)
    got = packed_out(inp, go)
    err = max(np.abs(got[t, h] - ro[i]).max() for i, (t, h) in enumerate(samples))
    say(f"attention formed tables full size {pairing}: sampled max-abs {err:.3e}")
    assert err <= ATTN_TOL[w.dtype]


# --------------------------------------------------------------------------- KV cache and decode
def test_kv_cache_interleaved():
    ci = wl.generate_cache(wl.CACHE_CONFIGS["small"])
    w = ci.workload
    dev = device()
    T, H, D = ci.k.shape
    f = orc.inv_freq(w.base, D)[None, :]
    rs, rc = orc.rope_tables(ci.pos, f, [T], 1.0, "fp32", "interleaved")
    rs, rc = orc.round_rne(rs, w.dtype), orc.round_rne(rc, w.dtype)
    nb, bs = ci.k_cache.shape[:2]
    kc_ref, vc_ref = orc.kv_rms_norm_rope_cache(f64(ci.k), f64(ci.v), ci.gamma.double().numpy(), 1e-6, rc, rs,
                                                ci.slots, f64(ci.k_cache).reshape(nb * bs, H, D),
                                                f64(ci.v_cache).reshape(nb * bs, H, D), "interleaved")
    kc, vc = ci.k_cache.to(dev), ci.v_cache.to(dev)
    rfa.rope_kv_rms_norm_rope_cache(ci.k.to(dev), ci.v.to(dev), torch.from_numpy(rc).to(ci.k.dtype).to(dev),
                                    torch.from_numpy(rs).to(ci.k.dtype).to(dev), torch.from_numpy(ci.slots).to(dev),
                                    kc, vc, gamma=ci.gamma.to(dev), pairing="interleaved")
    torch.cuda.synchronize()
    got_k = f64(kc).reshape(nb * bs, H, D)
    assert np.array_equal(f64(vc).reshape(nb * bs, H, D), vc_ref)
    sl = ci.slots
    y = orc.rms_norm(f64(ci.k), ci.gamma.double().numpy(), 1e-6)
    partner = y[..., np.arange(D) ^ 1]
    tol = orc.ulp(kc_ref[sl], w.dtype) + 4e-6 * (np.abs(y) + np.abs(partner))
    err = np.abs(got_k[sl] - kc_ref[sl])
    say(f"kv cache interleaved: max err/tol {np.max(err / tol):.3f}")
    assert np.all(err <= tol)
    untouched = np.setdiff1d(np.arange(nb * bs), sl)
    assert np.array_equal(got_k[untouched], kc_ref[untouched])


def test_decode_interleaved_end_to_end():
    """Tables, cache write and decode with interleaved pairs on the GPU, against the oracle."""
    ci = wl.generate_cache(wl.CACHE_CONFIGS["decode-small"])
    w = ci.workload
    dev = device()
    nb, bs, H, D = ci.k_cache.shape
    f = torch.from_numpy(rfa.inv_freq(w.base, D)).to(dev)
    sin, cos = rfa.rope_tables(torch.from_numpy(ci.pos).to(dev), f, [ci.ntokens], D, 1.0, w.torch_dtype,
                               pairing="interleaved")
    kc, vc = ci.k_cache.to(dev), ci.v_cache.to(dev)
    rfa.rope_kv_rms_norm_rope_cache(ci.k.to(dev), ci.v.to(dev), cos, sin, torch.from_numpy(ci.slots).to(dev), kc, vc,
                                    gamma=ci.gamma.to(dev), pairing="interleaved")
    lens = (ci.ctx + 1).astype(np.int32)
    o = rfa.rope_decode_attn_fwd(ci.q.to(dev), kc, vc, torch.from_numpy(lens).to(dev), cos, sin,
                                 max_seqlen=int(lens.max()),
                                 block_table=torch.from_numpy(ci.block_table.astype(np.int32)).to(dev),
                                 pairing="interleaved")
    torch.cuda.synchronize()
    fo = orc.inv_freq(w.base, D)[None, :]
    s64, c64 = orc.rope_tables(ci.pos, fo, [ci.ntokens], 1.0, "fp32", "interleaved")
    kc64, vc64 = orc.kv_rms_norm_rope_cache(f64(ci.k), f64(ci.v), ci.gamma.double().numpy(), 1e-6, c64, s64,
                                            ci.slots, f64(ci.k_cache).reshape(nb * bs, H, D),
                                            f64(ci.v_cache).reshape(nb * bs, H, D), "interleaved")
    ro, _ = orc.decode_attention(f64(ci.q), c64, s64, kc64, vc64, ci.block_table, lens, bs, 1.0 / D ** 0.5,
                                 "interleaved")
    err = np.abs(f64(o) - ro).max()
    say(f"decode interleaved end to end: max-abs {err:.3e}")
    assert err <= ATTN_TOL[w.dtype]
