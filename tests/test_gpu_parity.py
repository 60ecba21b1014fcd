"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Tolerances (the method's stated bars): attention max-abs 1e-4 (fp32), 5e-3 (fp16),
2e-2 (bf16); tables within 2 ulp of the output dtype; indexing bit-exact.
"""

import math

import numpy as np
import pytest
import torch

import oracle as orc
import rope_flashattention_amd as rfa
from rope_flashattention_amd import workloads as wl
from gpu_common import (ATTN_TOL, device, gpu_attention, gpu_tables, oracle_attention, oracle_tables, packed_out,
                        to_dev)

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def ulp_err(got, ref, dtype):
    return np.abs(np.asarray(got, dtype=np.float64) - ref) / orc.ulp(ref, dtype)


# --------------------------------------------------------------------------- tables
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_tables_parity_full_size(cfg):
    """rope_tables at each workload's full size and output dtype, every element."""
    w = wl.CONFIGS[cfg]
    inp = wl.generate(w)
    # the host inverse frequencies equal the oracle's bit for bit
    assert np.array_equal(rfa.inv_freq(w.base, w.head_dim, inp.seq_lens, w.trained_len),
                          orc.inv_freq_per_sequence(w.base, inp.seq_lens, w.head_dim, w.trained_len))
    s, c, _ = gpu_tables(inp, shared=False)
    rs, rc = oracle_tables(inp)
    es = ulp_err(s.to(torch.float64).cpu().numpy(), rs, w.dtype)
    ec = ulp_err(c.to(torch.float64).cpu().numpy(), rc, w.dtype)
    say(f"cfg{cfg} tables: T={inp.ntokens} max ulp sin {es.max():.3f} cos {ec.max():.3f}")
    assert es.max() <= 2.0 and ec.max() <= 2.0


@pytest.mark.parametrize("D,dtype", [(128, torch.float16), (512, torch.bfloat16), (2048, torch.float16),
                                     (2048, torch.bfloat16), (128, torch.float32)])
def test_tables_parity_page_limits(D, dtype):
    """batch 16, ntokens 256000 (the op's limits), sampled rows against the oracle."""
    dev = device()
    rng = np.random.default_rng(77)
    lens = rng.multinomial(256000 - 16, np.ones(16) / 16) + 1
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    f = rfa.inv_freq(1e4, D, lens, 4096)
    s, c = rfa.rope_tables(torch.from_numpy(pos).to(dev), torch.from_numpy(f).to(dev), lens, D, 1.0, dtype)
    rows = np.unique(np.concatenate([rng.integers(0, 256000, 400), np.cumsum(lens)[:-1], np.cumsum(lens) - 1]))
    seg = orc.segment_ids(lens)[rows]
    # oracle on the sampled rows: each row is its own one-token sequence with its batch's frequencies
    fo = orc.inv_freq_per_sequence(1e4, lens, D, 4096)[seg]
    rs, rc = orc.rope_tables(pos[rows], fo, np.ones(rows.size, dtype=np.int64), 1.0)
    dname = {torch.float16: "f16", torch.bfloat16: "bf16", torch.float32: "f32"}[dtype]
    es = ulp_err(s[torch.from_numpy(rows).to(dev)].to(torch.float64).cpu().numpy(), rs, dname)
    ec = ulp_err(c[torch.from_numpy(rows).to(dev)].to(torch.float64).cpu().numpy(), rc, dname)
    say(f"tables D={D} {dname}: max ulp sin {es.max():.3f} cos {ec.max():.3f}")
    assert es.max() <= 2.0 and ec.max() <= 2.0


@pytest.mark.parametrize("D", [32, 96, 160])
@pytest.mark.parametrize("pairing", ["half", "interleaved"])
def test_tables_piece_mapping_odd_sizes(D, pairing):
    """Every dtype and pairing at head sizes whose rows hold an odd number of 16-byte pieces
    and token counts that end inside a wavefront's run of pieces: all elements, 2 ulp."""
    dev = device()
    for T in (1, 5, 37, 301):
        lens = np.array([T], dtype=np.int32) if T < 37 else np.array([T - 20, 20], dtype=np.int32)
        pos = np.concatenate([np.arange(L, dtype=np.int32) * 7 for L in lens])
        f = rfa.inv_freq(1e4, D, lens)
        for dtype, dn in ((torch.float16, "f16"), (torch.bfloat16, "bf16"), (torch.float32, "f32")):
            s, c = rfa.rope_tables(torch.from_numpy(pos).to(dev), torch.from_numpy(f).to(dev), lens, D, 1.0, dtype,
                                   pairing=pairing)
            rs, rc = orc.rope_tables(pos, f, lens, 1.0, "fp32", pairing)
            es = ulp_err(s.to(torch.float64).cpu().numpy(), rs, dn).max()
            ec = ulp_err(c.to(torch.float64).cpu().numpy(), rc, dn).max()
            assert es <= 2.0 and ec <= 2.0, (T, dn, es, ec)
    say(f"tables D={D} {pairing}: T in (1, 5, 37, 301), f16/bf16/f32 within 2 ulp")


def test_tables_segment_index_probe():
    """Exact angles with a different frequency per sequence: recover b(t) from every row."""
    dev = device()
    lens = np.array([5, 1, 64, 3, 100, 7, 2, 9, 33, 1, 1, 40, 8, 6, 11, 4], dtype=np.int32)
    pos = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    D = 32
    f = np.stack([np.full(D // 2, 2.0 ** -(3 + b), dtype=np.float32) for b in range(16)])
    s, _ = rfa.rope_tables(torch.from_numpy(pos).to(dev), torch.from_numpy(f).to(dev), lens, D, 1.0, torch.float32)
    s = s.cpu().numpy().astype(np.float64)[:, 0]
    cand = np.sin(pos[:, None].astype(np.float64) * 2.0 ** -(3 + np.arange(16))[None, :])
    seg = orc.segment_ids(lens)
    for t in range(pos.size):
        if pos[t] == 0:
            assert s[t] == 0.0
            continue
        assert int(np.argmin(np.abs(cand[t] - s[t]))) == seg[t], t
        assert abs(s[t] - cand[t, seg[t]]) <= 2 * orc.ulp(cand[t, seg[t]], "f32")


def test_tables_scaling_negative_positions_and_subnormals():
    dev = device()
    pos = np.array([0, 1, 2, 3, 1, -5, -10000, 255999], dtype=np.int32)
    lens = np.array([4, 4], dtype=np.int32)
    f = np.stack([rfa.inv_freq(1e4, 128)[0], rfa.inv_freq(1e6, 128)[0]])
    for scale in (1.0, 2.0, 4.0):
        for dtype, dn in ((torch.float16, "f16"), (torch.bfloat16, "bf16"), (torch.float32, "f32")):
            s, c = rfa.rope_tables(torch.from_numpy(pos).to(dev), torch.from_numpy(f).to(dev), lens, 128, scale, dtype)
            rs, rc = orc.rope_tables(pos, f, lens, scale)
            es = ulp_err(s.to(torch.float64).cpu().numpy(), rs, dn)
            ec = ulp_err(c.to(torch.float64).cpu().numpy(), rc, dn)
            assert es.max() <= 2.0 and ec.max() <= 2.0, (scale, dn, es.max(), ec.max())
    # fp16 keeps subnormal sines (position 1, smallest frequencies of base 1e6)
    s, _ = rfa.rope_tables(torch.from_numpy(pos).to(dev), torch.from_numpy(f).to(dev), lens, 128, 1.0, torch.float16)
    sub = s[4, 60:64].to(torch.float32).cpu().numpy()
    assert np.all(sub > 0) and np.all(sub < 6.1e-5)


# --------------------------------------------------------------------------- rope_qk
def _rope_qk_check(inp, layout, tables):
    w = inp.workload
    dev = device()
    q, k, _ = to_dev(inp, "TND" if w.varlen else layout)
    T, D = inp.ntokens, w.head_dim
    if tables == "random":
        rng = np.random.default_rng(5)
        cos = torch.from_numpy(rng.uniform(-1, 1, (T, D)).astype(np.float32)).to(w.torch_dtype)
        sin = torch.from_numpy(rng.uniform(-1, 1, (T, D)).astype(np.float32)).to(w.torch_dtype)
        cs, ss, tsr = cos.to(dev), sin.to(dev), (0 if w.varlen else w.seqlen)
        c64, s64 = cos.to(torch.float64).numpy(), sin.to(torch.float64).numpy()
        extra = 0.0
    else:
        ss, cs, tsr = gpu_tables(inp, shared=False)
        s64, c64 = oracle_tables(inp, w.dtype)
        extra = 1.0
    kw = dict(layout="TND", cu_seqlens=torch.from_numpy(wl.cu_seqlens(inp.seq_lens)).to(dev),
              max_seqlen=int(inp.seq_lens.max())) if w.varlen else dict(layout=layout)
    oq, ok = rfa.rope_qk(q, k, cs, ss, table_seq_rows=tsr, **kw)
    qn, kn, _ = inp.packed()
    for x, o in ((qn, oq), (kn, ok)):
        ref = orc.rotate_tokens(x, c64, s64)
        got = packed_out(inp, o, "TND" if w.varlen else layout)
        half = D // 2
        partner = np.concatenate([x[..., half:], x[..., :half]], axis=-1)
        # 2 ulp of the output + float32 arithmetic floor; end to end the GPU's own tables may
        # differ from the oracle's rounded ones by up to 2 table ulp per factor
        tol = 2 * orc.ulp(ref, w.dtype) + 1e-6 * (np.abs(x) + np.abs(partner))
        if extra:
            tol = tol + 2 * (np.abs(x) * orc.ulp(c64, w.dtype)[:, None, :]
                             + np.abs(partner) * orc.ulp(s64, w.dtype)[:, None, :])
        err = np.abs(got - ref)
        say(f"rope_qk {w.name} {layout} {tables}: max err/tol {np.max(err / tol):.3f}")
        assert np.all(err <= tol)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
@pytest.mark.parametrize("tables", ["random", "rope_tables"])
def test_rope_qk_parity_small(cfg, tables):
    _rope_qk_check(wl.generate(wl.SMALL[cfg]), "BNSD", tables)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_rope_qk_parity_full_size(cfg):
    _rope_qk_check(wl.generate(wl.CONFIGS[cfg]), "BNSD", "rope_tables")


def test_rope_qk_bsnd_and_in_place():
    inp = wl.generate(wl.SMALL[3])
    _rope_qk_check(inp, "BSND", "random")
    q, k, _ = to_dev(inp)
    s, c, tsr = gpu_tables(inp)
    oq, ok = rfa.rope_qk(q, k, c, s, table_seq_rows=tsr)
    q2, k2 = q.clone(), k.clone()
    rfa.rope_qk(q2, k2, c, s, table_seq_rows=tsr, out_q=q2, out_k=k2)
    assert torch.equal(q2, oq) and torch.equal(k2, ok)


@pytest.mark.parametrize("case", ["bsnd", "varlen", "long_streaming"])
def test_rope_qk_in_place_every_thread_mapping(case):
    """In place equals out of place on each of rope_qk's paths: heads inner (BSND, packed
    TND), and the streaming path of calls larger than twice the last-level cache (the long
    GQA workload at full size, 612 MB)."""
    w = {"bsnd": wl.SMALL[2], "varlen": wl.SMALL[4], "long_streaming": wl.CONFIGS[5]}[case]
    inp = wl.generate(w)
    dev = device()
    lay = "TND" if w.varlen else ("BSND" if case == "bsnd" else "BNSD")
    q, k, _ = to_dev(inp, lay)
    s, c, tsr = gpu_tables(inp, shared=False)
    kw = dict(layout="TND", cu_seqlens=torch.from_numpy(wl.cu_seqlens(inp.seq_lens)).to(dev),
              max_seqlen=int(inp.seq_lens.max())) if w.varlen else dict(layout=lay)
    oq, ok = rfa.rope_qk(q, k, c, s, table_seq_rows=tsr, **kw)
    rfa.rope_qk(q, k, c, s, table_seq_rows=tsr, out_q=q, out_k=k, **kw)
    assert torch.equal(q, oq) and torch.equal(k, ok)


# --------------------------------------------------------------------------- attention, full output
def _attn_check(inp, layout="BNSD", shared_table=True):
    w = inp.workload
    o, lse = gpu_attention(inp, layout, shared_table, return_lse=True)
    ro, rlse = oracle_attention(inp)
    got = packed_out(inp, o, "TND" if w.varlen else layout)
    err = np.abs(got - ro).max()
    lerr = np.abs(lse.cpu().numpy().astype(np.float64) - rlse).max()
    say(f"attention {w.name} {layout}: max-abs {err:.3e} (tol {ATTN_TOL[w.dtype]}), lse max-abs {lerr:.3e}")
    assert np.all(np.isfinite(got))
    assert err <= ATTN_TOL[w.dtype]
    assert lerr <= ATTN_TOL[w.dtype]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_attention_parity_small(cfg):
    _attn_check(wl.generate(wl.SMALL[cfg]))


def test_attention_parity_config1_full():
    # config 1 at its full size (it is small): fp32 inputs on the float32 matrix cores
    _attn_check(wl.generate(wl.CONFIGS[1]))


@pytest.mark.parametrize("S", [1, 2, 31, 63, 64, 65, 127, 128, 129, 191, 257])
def test_attention_edge_lengths(S):
    w = wl.Workload(f"edge S{S}", "bf16", 1, 4, 2, 128, seqlen=S, base=1e4, seed=3000 + S)
    _attn_check(wl.generate(w))


@pytest.mark.parametrize("lens", [[1], [1, 1, 1], [64, 1, 65, 128], [200, 3, 129, 64, 1, 77]])
def test_attention_varlen_edges(lens):
    import dataclasses
    w = wl.Workload("varlen edges", "f16", len(lens), 4, 4, 128, varlen=True, len_range=(1, 1), base=1e4,
                    trained_len=64, seed=4000 + len(lens))
    inp = wl.generate(w)
    inp = dataclasses.replace(inp, seq_lens=np.asarray(lens, dtype=np.int32))
    T = int(sum(lens))
    g = torch.Generator().manual_seed(9)
    inp.q = torch.randn(T, 4, 128, generator=g).to(torch.float16)
    inp.k = torch.randn(T, 4, 128, generator=g).to(torch.float16)
    inp.v = torch.randn(T, 4, 128, generator=g).to(torch.float16)
    inp.pos = np.concatenate([np.arange(L, dtype=np.int32) for L in lens])
    _attn_check(inp)


@pytest.mark.parametrize("dtype,D", [("bf16", 64), ("f16", 64), ("f16", 128), ("f32", 64)])
def test_attention_dtypes_and_head_dims(dtype, D):
    w = wl.Workload(f"{dtype} D{D}", dtype, 2, 4, 2, D, seqlen=150, base=1e4, seed=5000 + D)
    _attn_check(wl.generate(w))


def test_attention_non_causal():
    w = wl.Workload("non-causal", "bf16", 2, 4, 4, 128, seqlen=200, base=1e4, causal=False, seed=5100)
    _attn_check(wl.generate(w))


def test_attention_bsnd_layout_and_per_sequence_tables():
    inp = wl.generate(wl.SMALL[2])
    _attn_check(inp, "BSND")
    _attn_check(inp, "BNSD", shared_table=False)


# --------------------------------------------------------------------------- attention, full sizes, sampled rows
def _sample_rows(inp, rng, n_pairs=3, per_pair=12):
    w = inp.workload
    starts = orc.segment_starts(inp.seq_lens)
    samples = []
    g = w.hq // w.hkv
    for _ in range(n_pairs):
        b = int(rng.integers(0, w.batch))
        kvh = int(rng.integers(0, w.hkv))
        s0, L = int(starts[b]), int(inp.seq_lens[b])
        rows = {0, L - 1, min(L - 1, 63), min(L - 1, 64), min(L - 1, 127), min(L - 1, 128)}
        rows |= set(int(x) for x in rng.integers(0, L, per_pair - len(rows)))
        for i in sorted(rows):
            samples.append((s0 + i, kvh * g + int(rng.integers(0, g))))
    return samples


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_attention_parity_full_size_sampled(cfg):
    w = wl.CONFIGS[cfg]
    inp = wl.generate(w)
    say(f"cfg{cfg}: {w.name}, T={inp.ntokens}, lens={inp.seq_lens.tolist() if w.varlen else w.seqlen}")
    o, lse = gpu_attention(inp, return_lse=True)
    torch.cuda.synchronize()
    got = packed_out(inp, o)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(cfg)
    samples = _sample_rows(inp, rng)
    q, k, v = inp.packed()
    s, c = oracle_tables(inp, w.dtype)
    rows, lses = orc.rope_attention_rows(q, k, v, c, s, inp.seq_lens, w.softmax_scale, w.causal, samples)
    lse_np = lse.cpu().numpy()
    err = max(np.abs(got[t, h] - r).max() for (t, h), r in zip(samples, rows))
    lerr = max(abs(float(lse_np[h, t]) - l) for (t, h), l in zip(samples, lses))
    say(f"cfg{cfg} full size: {len(samples)} sampled rows, max-abs {err:.3e} (tol {ATTN_TOL[w.dtype]}), lse {lerr:.3e}")
    assert err <= ATTN_TOL[w.dtype] and lerr <= ATTN_TOL[w.dtype]


# --------------------------------------------------------------------------- equivalences and hygiene
def test_fused_equals_unfused():
    """rope_qk then attention without rotation matches the fused call."""
    inp = wl.generate(wl.SMALL[3])
    w = inp.workload
    fused = gpu_attention(inp)
    q, k, v = to_dev(inp)
    s, c, tsr = gpu_tables(inp)
    oq, ok = rfa.rope_qk(q, k, c, s, table_seq_rows=tsr)
    unfused = rfa.rope_flash_attn_fwd(oq, ok, v, None, None, softmax_scale=w.softmax_scale)
    err = (fused.float() - unfused.float()).abs().max().item()
    say(f"fused vs unfused max-abs {err:.3e}")
    assert err <= ATTN_TOL[w.dtype]


def test_gqa_equals_repeated_kv():
    inp = wl.generate(wl.SMALL[5])
    w = inp.workload
    g = w.hq // w.hkv
    o_gqa = gpu_attention(inp)
    q, k, v = to_dev(inp)
    s, c, tsr = gpu_tables(inp)
    k2 = k.repeat_interleave(g, dim=1).contiguous()
    v2 = v.repeat_interleave(g, dim=1).contiguous()
    o_mha = rfa.rope_flash_attn_fwd(q, k2, v2, c, s, softmax_scale=w.softmax_scale)
    assert torch.equal(o_gqa, o_mha)


def test_varlen_equals_per_sequence_dense():
    inp = wl.generate(wl.SMALL[4])
    w = inp.workload
    dev = device()
    o = gpu_attention(inp)
    s, c, _ = gpu_tables(inp)
    starts = orc.segment_starts(inp.seq_lens)
    for b, L in enumerate(inp.seq_lens.tolist()):
        sl = slice(int(starts[b]), int(starts[b]) + L)
        qd, kd, vd = (x[sl].to(dev).transpose(0, 1).unsqueeze(0).contiguous() for x in (inp.q, inp.k, inp.v))
        od = rfa.rope_flash_attn_fwd(qd, kd, vd, c[sl].contiguous(), s[sl].contiguous(), softmax_scale=w.softmax_scale)
        assert torch.equal(od[0].transpose(0, 1), o[sl]), b


def test_deterministic():
    inp = wl.generate(wl.SMALL[2])
    a = gpu_attention(inp)
    b = gpu_attention(inp)
    assert torch.equal(a, b)


def test_every_output_written_and_guard_bands_untouched():
    inp = wl.generate(wl.SMALL[3])
    w = inp.workload
    dev = device()
    q, k, v = to_dev(inp)
    s, c, tsr = gpu_tables(inp)
    n = q.numel()
    buf = torch.full((n + 4096,), float("nan"), dtype=q.dtype, device=dev)
    out = buf[2048:2048 + n].view(q.shape)
    rfa.rope_flash_attn_fwd(q, k, v, c, s, softmax_scale=w.softmax_scale, out=out)
    assert not torch.isnan(out).any()
    assert torch.isnan(buf[:2048]).all() and torch.isnan(buf[2048 + n:]).all()
    # rope_qk: same canary check
    bq = torch.full((q.numel() + 4096,), float("nan"), dtype=q.dtype, device=dev)
    bk = torch.full((k.numel() + 4096,), float("nan"), dtype=q.dtype, device=dev)
    oq = bq[2048:2048 + q.numel()].view(q.shape)
    ok = bk[2048:2048 + k.numel()].view(k.shape)
    rfa.rope_qk(q, k, c, s, table_seq_rows=tsr, out_q=oq, out_k=ok)
    assert not torch.isnan(oq).any() and not torch.isnan(ok).any()
    assert torch.isnan(bq[:2048]).all() and torch.isnan(bq[2048 + q.numel():]).all()
    assert torch.isnan(bk[:2048]).all() and torch.isnan(bk[2048 + k.numel():]).all()


def test_position_shift_invariance():
    """Shifting every position by the same offset leaves attention unchanged (exactly in
    exact arithmetic; here within the tolerance, since table values change)."""
    inp = wl.generate(wl.SMALL[2])
    w = inp.workload
    dev = device()
    q, k, v = to_dev(inp)
    f = torch.from_numpy(rfa.inv_freq(w.base, w.head_dim)).to(dev)
    outs = []
    for shift in (0, 1000):
        pos = torch.arange(shift, shift + w.seqlen, dtype=torch.int32, device=dev)
        s, c = rfa.rope_tables(pos, f, [w.seqlen], w.head_dim, 1.0, torch.float32)
        s, c = s.to(w.torch_dtype), c.to(w.torch_dtype)
        outs.append(rfa.rope_flash_attn_fwd(q, k, v, c, s, softmax_scale=w.softmax_scale).float())
    err = (outs[0] - outs[1]).abs().max().item()
    say(f"position shift max-abs {err:.3e}")
    assert err <= ATTN_TOL[w.dtype]
