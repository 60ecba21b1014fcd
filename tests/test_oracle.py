"""Pins for the CPU oracle: closed forms, invariants, special cases, brute force.

Each check_* function takes the oracle function(s) it checks as arguments, so the
same check runs against the oracle (must pass) and against planted mistakes
(must fail; see the mutation tests at the end).  No GPU is used here.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc

mpmath = pytest.importorskip("mpmath")


def rng(seed=0):
    return np.random.default_rng(seed)


# --------------------------------------------------------------------------- inv_freq (a1)
def check_inv_freq(inv_freq):
    # closed form at small D: 10000^(-0) = 1, 10000^(-2/4) = 0.01
    f = inv_freq(10000.0, 4)
    assert f.dtype == np.float32 and f.shape == (2,)
    assert f[0] == np.float32(1.0) and f[1] == np.float32(0.01)
    # correctly rounded to float32 against a 40-digit reference, several bases/sizes
    mpmath.mp.dps = 40
    for base, D in [(1e4, 64), (1e4, 128), (5e5, 128), (1e6, 128), (1e4, 2048)]:
        f = inv_freq(base, D)
        assert f.shape == (D // 2,)
        for i in range(0, D // 2, max(1, D // 64)):
            exact = mpmath.power(mpmath.mpf(base), -mpmath.mpf(2 * i) / D)
            err = abs(mpmath.mpf(float(f[i])) - exact)
            half_ulp = mpmath.mpf(float(orc.ulp(float(exact), "f32"))) / 2
            assert err <= half_ulp * (1 + mpmath.mpf("1e-6")), (base, D, i)
        assert np.all(np.diff(f.astype(np.float64)) < 0)


def test_inv_freq_closed_form():
    check_inv_freq(orc.inv_freq)


def test_ntk_base_properties():
    # Parity unpinned: only the properties the DynamicNTKOperation page states hold.
    assert orc.ntk_base(1e4, 4096, 4096, 128) == 1e4
    assert orc.ntk_base(1e4, 512, 4096, 128) == 1e4
    b = orc.ntk_base(1e4, 8192, 4096, 128)
    assert b > 1e4
    assert orc.ntk_base(1e4, 8000, 4096, 128) < b   # enlarges with length
    f = orc.inv_freq_per_sequence(1e4, [1000, 8192], 128, 4096)
    assert f.shape == (2, 64) and f.dtype == np.float32
    assert np.array_equal(f[0], orc.inv_freq(1e4, 128))
    assert np.all(f[1] <= f[0]) and np.all(f[1] > 0) and np.all(f <= 1)


def test_ntk_base_reading_stretches_longest_wavelength_by_length_ratio():
    # The enlargement law is a reading (the page lost it), so this pins the reading's defining
    # property, not the page: NTK-aware scaling divides the lowest inverse frequency by exactly
    # the length ratio L / L_train (the longest wavelength then spans the longer context) and
    # leaves the highest (i = 0, f = 1) unchanged.  A wrong exponent ((D-2)/D for D/(D-2), or
    # D/2 for D) moves the lowest frequency by a different factor and fails.
    for D in (64, 128, 256):
        f0 = orc.inv_freq(1e4, D).astype(np.float64)
        for L, Lt in ((8192, 4096), (10000, 4096), (32768, 2048), (4097, 4096)):
            f = orc.inv_freq(orc.ntk_base(1e4, L, Lt, D), D).astype(np.float64)
            assert f[0] == 1.0
            ratio = f0[-1] / f[-1]
            assert abs(ratio / (L / Lt) - 1.0) < 4 * 2.0 ** -24, (D, L, Lt, ratio)
            # every other frequency is divided by less than the ratio (high frequencies extrapolate)
            assert np.all(f0[1:-1] / f[1:-1] < L / Lt) and np.all(f0[1:] / f[1:] > 1.0)


# --------------------------------------------------------------------------- segments and angles
def test_segment_ids_hand():
    assert orc.segment_ids([2, 3, 1]).tolist() == [0, 0, 1, 1, 1, 2]
    assert orc.segment_starts([2, 3, 1]).tolist() == [0, 2, 5]


def check_tables_golden(rope_tables, golden):
    mpmath.mp.dps = 50
    for case in golden["cases"]:
        pos = np.array(case["positionIds"], dtype=np.int32)
        f = np.array(case["invFreq"], dtype=np.float32)
        s, c = rope_tables(pos, f, case["seqLens"], case["scale"])
        emb = np.array(case["emb"], dtype=np.float64)
        for t in range(emb.shape[0]):
            for j in range(emb.shape[1]):
                assert abs(s[t, j] - float(mpmath.sin(mpmath.mpf(emb[t, j])))) <= 1e-16, (case["name"], t, j)
                assert abs(c[t, j] - float(mpmath.cos(mpmath.mpf(emb[t, j])))) <= 1e-16, (case["name"], t, j)


def test_tables_golden(golden_dir):
    with open(os.path.join(golden_dir, "dynamic_ntk_tiny.json")) as fh:
        golden = json.load(fh)
    check_tables_golden(orc.rope_tables, golden)


def check_angles_fp32(angles):
    r = rng(1)
    seq_lens = [5, 9, 3]
    pos = np.concatenate([np.arange(L) for L in seq_lens]).astype(np.int32) * 977
    f = r.uniform(0.0, 1.0, size=(3, 8)).astype(np.float32)
    seg = orc.segment_ids(seq_lens)
    for scale in (1.0, 2.0, 3.0):
        got = angles(pos, f, seq_lens, scale, "fp32")
        # independent path: exact float64 quotient/product, each rounded once to float32
        t = (pos.astype(np.float64) / scale).astype(np.float32).astype(np.float64)
        want = (t[:, None] * f[seg].astype(np.float64)).astype(np.float32).astype(np.float64)
        assert np.array_equal(got, want)


def test_angles_fp32_rounding():
    check_angles_fp32(orc.angles)


def test_angles_exact_mode_error_bound():
    # exact mode: (p / s) * f in float64, within 2 float64 rounding errors of the real product
    mpmath.mp.dps = 40
    r = rng(13)
    pos = np.array([0, 1, 4095, 65535, 1 << 20, (1 << 24) - 3, 250000], dtype=np.int32)
    f = r.uniform(1e-6, 1.0, size=(1, 6)).astype(np.float32)
    for scale in (1.0, 2.0, 3.0):
        got = orc.angles(pos, f, [pos.size], scale, "exact")
        for t in range(pos.size):
            for i in range(f.shape[1]):
                exact = mpmath.mpf(int(pos[t])) / mpmath.mpf(scale) * mpmath.mpf(float(f[0, i]))
                assert abs(mpmath.mpf(float(got[t, i])) - exact) <= 2 * 2.0 ** -53 * abs(exact) + 1e-300
        # and the float32 mode differs from it by at most the two float32 roundings
        g32 = orc.angles(pos, f, [pos.size], scale, "fp32")
        assert np.all(np.abs(g32 - got) <= 2 * 2.0 ** -24 * np.abs(got) + 1e-30)


def check_table_structure(rope_tables):
    r = rng(2)
    seq_lens = [7, 4]
    pos = np.concatenate([np.arange(L) for L in seq_lens]).astype(np.int32)
    f = np.stack([orc.inv_freq(1e4, 64), orc.inv_freq(5e5, 64)])
    s, c = rope_tables(pos, f, seq_lens, 1.0)
    assert s.shape == (11, 64) and c.shape == (11, 64)
    # position 0 of every sequence: cos = 1, sin = 0 exactly
    for t in (0, 7):
        assert np.all(c[t] == 1.0) and np.all(s[t] == 0.0)
    # rotate-half form: column j equals column j + D/2 bit for bit
    assert np.array_equal(s[:, :32], s[:, 32:]) and np.array_equal(c[:, :32], c[:, 32:])
    assert np.max(np.abs(s * s + c * c - 1.0)) < 1e-15
    # each row uses its own sequence's inverse frequencies: t=8 is position 1 of batch 1
    assert np.allclose(s[8, :32], np.sin(f[1].astype(np.float64)), rtol=0, atol=1e-16)
    assert np.allclose(s[1, :32], np.sin(f[0].astype(np.float64)), rtol=0, atol=1e-16)


def test_table_structure():
    check_table_structure(orc.rope_tables)


# --------------------------------------------------------------------------- rotation
def check_rotation(rotation_matrix, rope_op_matrix, rotate_tokens):
    r = rng(3)
    D = 16
    theta = r.uniform(-50, 50, size=D // 2)
    R = rotation_matrix(theta)
    assert np.array_equal(rotation_matrix(np.zeros(D // 2)), np.eye(D))
    assert np.max(np.abs(R @ rotation_matrix(-theta) - np.eye(D))) < 1e-14
    q = r.standard_normal(D)
    assert abs(np.linalg.norm(R @ q) - np.linalg.norm(q)) <= 1e-12 * np.linalg.norm(q)
    # pair i is (i, i + D/2) rotated by theta_i: a single-angle check by hand
    e0 = np.zeros(D)
    e0[0] = 1.0
    th = np.zeros(D // 2)
    th[0] = 0.3
    got = rotation_matrix(th) @ e0
    want = np.zeros(D)
    want[0], want[D // 2] = math.cos(0.3), math.sin(0.3)
    assert np.max(np.abs(got - want)) < 1e-16
    # the Rope op on cat(freq, freq) tables is the same rotation
    emb = np.concatenate([theta, theta])
    assert np.max(np.abs(rope_op_matrix(np.cos(emb), np.sin(emb)) - R)) < 1e-15
    # second formulation: x*cos + rotate_half(x)*sin, rotate_half(x) = cat(-x2, x1)
    x = r.standard_normal((3, 2, D))
    cos = r.uniform(-1, 1, size=(3, D))
    sin = r.uniform(-1, 1, size=(3, D))
    rh = np.concatenate([-x[..., D // 2:], x[..., :D // 2]], axis=-1)
    want = x * cos[:, None, :] + rh * sin[:, None, :]
    assert np.max(np.abs(rotate_tokens(x, cos, sin) - want)) < 1e-14


def test_rotation():
    check_rotation(orc.rotation_matrix, orc.rope_op_matrix, orc.rotate_tokens)


def check_relative_position(rope_tables, rotate_tokens):
    # [RoPE/GQA tutorial, section 五]: the rotated score depends only on m - n.
    r = rng(4)
    D = 64
    f = orc.inv_freq(1e4, D)[None, :]
    q = r.standard_normal((1, 1, D))
    k = r.standard_normal((1, 1, D))
    pos = np.arange(0, 1025, dtype=np.int32)
    s, c = rope_tables(pos, f, [pos.size], 1.0, "exact")

    def score(m, n):
        qm = rotate_tokens(q, c[m:m + 1], s[m:m + 1])[0, 0]
        kn = rotate_tokens(k, c[n:n + 1], s[n:n + 1])[0, 0]
        return qm @ kn

    for m, n, shift in [(5, 2, 100), (300, 17, 700), (0, 0, 1024), (9, 40, 900)]:
        a, b = score(m, n), score(m + shift, n + shift)
        assert abs(a - b) <= 1e-12 * max(1.0, abs(a)), (m, n, shift, a, b)
    # and it does depend on the offset
    assert abs(score(5, 2) - score(5, 3)) > 1e-3


def test_relative_position():
    check_relative_position(orc.rope_tables, orc.rotate_tokens)


# --------------------------------------------------------------------------- interleaved pairing
def _even_odd_perm(D):
    """Indices that gather the rotate-half layout from the interleaved one: x_half = x_int[perm]."""
    return np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])


def check_interleaved(rotation_matrix, rope_op_matrix, rotate_tokens, rope_tables):
    r = rng(11)
    D = 16
    theta = r.uniform(-20, 20, size=D // 2)
    Ri = rotation_matrix(theta, "interleaved")
    # by hand: pair 0 is (x_0, x_1), pair 3 is (x_6, x_7)
    for i in (0, 3):
        e = np.zeros(D)
        e[2 * i] = 1.0
        want = np.zeros(D)
        want[2 * i], want[2 * i + 1] = math.cos(theta[i]), math.sin(theta[i])
        assert np.max(np.abs(Ri @ e - want)) < 1e-15
        e = np.zeros(D)
        e[2 * i + 1] = 1.0
        want = np.zeros(D)
        want[2 * i], want[2 * i + 1] = -math.sin(theta[i]), math.cos(theta[i])
        assert np.max(np.abs(Ri @ e - want)) < 1e-15
    # the same rotation as rotate-half, seen through the even/odd permutation
    perm = _even_odd_perm(D)
    P = np.eye(D)[perm]                                   # x_half = P x_int
    assert np.max(np.abs(Ri - P.T @ rotation_matrix(theta, "half") @ P)) < 1e-15
    # tables: both columns of a pair hold its angle; a column permutation of the half tables
    seq = [9]
    pos = np.arange(9, dtype=np.int32) * 37
    f = orc.inv_freq(1e4, D)[None, :]
    si, ci = rope_tables(pos, f, seq, 1.0, "fp32", "interleaved")
    sh, ch = rope_tables(pos, f, seq, 1.0, "fp32", "half")
    assert np.array_equal(si[:, 0::2], si[:, 1::2]) and np.array_equal(ci[:, 0::2], ci[:, 1::2])
    assert np.array_equal(si[:, 0::2], sh[:, :D // 2]) and np.array_equal(ci[:, 0::2], ch[:, :D // 2])
    # the Rope op on interleaved tables is the interleaved rotation
    emb = np.repeat(theta, 2)
    assert np.max(np.abs(rope_op_matrix(np.cos(emb), np.sin(emb), "interleaved") - Ri)) < 1e-15
    # second formulation: x*cos + rotate_every_two(x)*sin, rotate_every_two(x) = (-x1, x0, -x3, x2, ...)
    x = r.standard_normal((4, 3, D))
    cos = r.uniform(-1, 1, size=(4, D))
    sin = r.uniform(-1, 1, size=(4, D))
    rt = np.empty_like(x)
    rt[..., 0::2] = -x[..., 1::2]
    rt[..., 1::2] = x[..., 0::2]
    want = x * cos[:, None, :] + rt * sin[:, None, :]
    assert np.max(np.abs(rotate_tokens(x, cos, sin, pairing="interleaved") - want)) < 1e-14


def test_interleaved_pairing():
    check_interleaved(orc.rotation_matrix, orc.rope_op_matrix, orc.rotate_tokens, orc.rope_tables)


def test_interleaved_relative_position_and_attention():
    r = rng(12)
    D = 32
    f = orc.inv_freq(1e4, D)[None, :]
    pos = np.arange(0, 700, dtype=np.int32)
    s, c = orc.rope_tables(pos, f, [pos.size], 1.0, "exact", "interleaved")
    q = r.standard_normal((1, 1, D))
    k = r.standard_normal((1, 1, D))

    def score(m, n):
        return (orc.rotate_tokens(q, c[m:m + 1], s[m:m + 1], pairing="interleaved")[0, 0]
                @ orc.rotate_tokens(k, c[n:n + 1], s[n:n + 1], pairing="interleaved")[0, 0])

    for m, n, shift in [(5, 2, 100), (300, 17, 380), (9, 40, 600)]:
        assert abs(score(m, n) - score(m + shift, n + shift)) <= 1e-12 * max(1.0, abs(score(m, n)))
    # attention with interleaved pairs = rotate-half attention on even/odd-permuted q and k
    L, Hq, Hkv = 23, 4, 2
    qs = r.standard_normal((L, Hq, D))
    ks = r.standard_normal((L, Hkv, D))
    vs = r.standard_normal((L, Hkv, D))
    si, ci = orc.rope_tables(np.arange(L, dtype=np.int32), f, [L], 1.0, "fp32", "interleaved")
    sh, ch = orc.rope_tables(np.arange(L, dtype=np.int32), f, [L], 1.0, "fp32", "half")
    perm = _even_odd_perm(D)
    oi, li = orc.rope_attention(qs, ks, vs, ci, si, [L], 0.3, True, "interleaved")
    oh, lh = orc.rope_attention(qs[..., perm], ks[..., perm], vs, ch, sh, [L], 0.3, True, "half")
    assert np.max(np.abs(oi - oh)) < 1e-12 and np.max(np.abs(li - lh)) < 1e-12


# --------------------------------------------------------------------------- attention
def brute_force_attention(q, k, v, scale, causal):
    """Scalar loops, independent of the oracle's matrix form."""
    n, d = len(q), len(q[0])
    out = []
    for i in range(n):
        keys = range(i + 1) if causal else range(len(k))
        sc = []
        for j in keys:
            acc = 0.0
            for e in range(d):
                acc += q[i][e] * k[j][e]
            sc.append(acc * scale)
        m = max(sc)
        w = [math.exp(x - m) for x in sc]
        tot = sum(w)
        row = []
        for e in range(d):
            acc = 0.0
            for jj, j in enumerate(keys):
                acc += w[jj] * v[j][e]
            row.append(acc / tot)
        out.append(row)
    return np.array(out)


def check_attention(attention):
    r = rng(5)
    for n, d, causal in [(1, 4, True), (17, 8, True), (64, 16, True), (23, 8, False)]:
        q, k, v = (r.standard_normal((n, d)) for _ in range(3))
        scale = 1.0 / math.sqrt(d)
        o, lse = attention(q, k, v, scale, causal)
        bf = brute_force_attention(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        assert np.max(np.abs(o - bf)) < 1e-12, (n, d, causal)
        # lse = log sum exp of the kept scores (row 0 of a causal problem: one score)
        if causal:
            assert abs(lse[0] - (q[0] @ k[0]) * scale) < 1e-12
    n, d = 40, 8
    q, k, v = (r.standard_normal((n, d)) for _ in range(3))
    # rows of P sum to 1 (V = ones gives ones), P >= 0 (convex combination bounds)
    o, _ = attention(q, k, np.ones((n, d)), 0.3, True)
    assert np.max(np.abs(o - 1.0)) < 1e-14
    o, _ = attention(q, k, v, 0.3, True)
    for i in range(n):
        assert np.all(o[i] <= v[:i + 1].max(axis=0) + 1e-12) and np.all(o[i] >= v[:i + 1].min(axis=0) - 1e-12)
    # causal row 0 is V[0]; a later key never leaks into an earlier row
    assert np.max(np.abs(o[0] - v[0])) < 1e-15
    v2 = v.copy()
    v2[30:] = 1e6
    o2, _ = attention(q, k, v2, 0.3, True)
    assert np.max(np.abs(o2[:30] - o[:30])) < 1e-12
    # Q = 0: uniform weights over the kept keys -> running mean of V
    o, _ = attention(np.zeros((n, d)), k, v, 0.7, True)
    cm = np.cumsum(v, axis=0) / np.arange(1, n + 1)[:, None]
    assert np.max(np.abs(o - cm)) < 1e-13
    # one dominant logit picks its V row
    kk = np.zeros((n, d))
    kk[11, 0] = 1.0
    qq = np.zeros((n, d))
    qq[:, 0] = 1e4
    o, _ = attention(qq, kk, v, 1.0, True)
    assert np.max(np.abs(o[11:] - v[11])) < 1e-12


def test_attention():
    check_attention(orc.attention)


def _packed_problem(r, seq_lens, hq, hkv, d):
    T = int(np.sum(seq_lens))
    q = r.standard_normal((T, hq, d))
    k = r.standard_normal((T, hkv, d))
    v = r.standard_normal((T, hkv, d))
    pos = np.concatenate([np.arange(L) for L in seq_lens]).astype(np.int32)
    f = orc.inv_freq_per_sequence(1e4, seq_lens, d, None)
    s, c = orc.rope_tables(pos, f, seq_lens, 1.0)
    return q, k, v, s, c


def check_rope_attention(rope_attention, rope_attention_rows):
    r = rng(6)
    d = 16
    scale = 1.0 / math.sqrt(d)
    # GQA reduces to MHA with each kv head repeated g times (contiguous groups)
    seq_lens = [19]
    q, k, v, s, c = _packed_problem(r, seq_lens, 8, 2, d)
    o_gqa, lse_gqa = rope_attention(q, k, v, c, s, seq_lens, scale, True)
    o_mha, lse_mha = rope_attention(q, np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1), c, s, seq_lens, scale, True)
    assert np.max(np.abs(o_gqa - o_mha)) < 1e-14 and np.max(np.abs(lse_gqa - lse_mha)) < 1e-14
    # varlen: packed output = each sequence run on its own
    seq_lens = [5, 12, 1, 9]
    q, k, v, s, c = _packed_problem(r, seq_lens, 4, 2, d)
    o, lse = rope_attention(q, k, v, c, s, seq_lens, scale, True)
    for s0, L in zip(orc.segment_starts(seq_lens), seq_lens):
        sl = slice(s0, s0 + L)
        oi, li = rope_attention(q[sl], k[sl], v[sl], c[sl], s[sl], [L], scale, True)
        assert np.max(np.abs(o[sl] - oi)) < 1e-14 and np.max(np.abs(lse[:, sl] - li)) < 1e-14
    # segment probe: Q = 0, V column 0 = segment id -> output column 0 = segment id
    vv = v.copy()
    vv[:, :, 0] = orc.segment_ids(seq_lens)[:, None]
    o0, _ = rope_attention(np.zeros_like(q), k, vv, c, s, seq_lens, scale, True)
    assert np.max(np.abs(o0[:, :, 0] - orc.segment_ids(seq_lens)[:, None])) < 1e-14
    # zero angles reduce to plain attention on the unrotated inputs
    z = np.zeros_like(s)
    o_z, _ = rope_attention(q, k, v, np.ones_like(c), z, seq_lens, scale, True)
    s0, L = 5, 12
    o_p, _ = orc.attention(q[s0:s0 + L, 3], k[s0:s0 + L, 1], v[s0:s0 + L, 1], scale, True)
    assert np.max(np.abs(o_z[s0:s0 + L, 3] - o_p)) < 1e-14
    # sampled rows equal the full result
    samples = [(0, 0), (4, 3), (5, 1), (16, 2), (17, 0), (26, 3)]
    rows, lses = rope_attention_rows(q, k, v, c, s, seq_lens, scale, True, samples)
    for (t, h), row, l in zip(samples, rows, lses):
        assert np.max(np.abs(row - o[t, h])) < 1e-13 and abs(l - lse[h, t]) < 1e-13


def test_rope_attention():
    check_rope_attention(orc.rope_attention, orc.rope_attention_rows)


# --------------------------------------------------------------------------- rounding helpers
def test_round_rne_matches_library_casts():
    r = rng(7)
    x32 = np.concatenate([
        r.standard_normal(20000).astype(np.float32),
        (r.standard_normal(4000) * 1e-38).astype(np.float32),        # bf16 subnormal range
        np.array([1.0 + 2**-8, 1.0 + 3 * 2**-8, -(1.0 + 2**-8), 2**-130, 0.0], dtype=np.float32),  # ties
    ])
    want = torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(orc.round_rne(x32.astype(np.float64), "bf16"), want)
    x64 = np.concatenate([r.standard_normal(20000), r.standard_normal(4000) * 1e-5,
                          np.array([1 + 2**-11, 1 + 3 * 2**-11, 2**-25, 3 * 2**-25, 0.0])])
    assert np.array_equal(orc.round_rne(x64, "f16"), x64.astype(np.float16).astype(np.float64))
    assert np.array_equal(orc.round_rne(x64, "f32"), x64.astype(np.float32).astype(np.float64))


def test_ulp_values():
    assert orc.ulp(1.0, "bf16") == 2**-7
    assert orc.ulp(1.0, "f16") == 2**-10
    assert orc.ulp(1.5, "f32") == 2**-23
    assert orc.ulp(0.0, "f16") == 2**-24
    assert orc.ulp(5.8e-5, "f16") == 2**-24      # subnormal range of fp16
    assert orc.ulp(-0.75, "bf16") == 2**-8


# --------------------------------------------------------------------------- RMSNorm + RoPE + cache write
def check_rms_norm(rms_norm):
    r = rng(8)
    # constant vector: |c| is its root mean square
    g = r.uniform(0.5, 2.0, size=16)
    y = rms_norm(np.full(16, -3.0), g, 0.0)
    assert np.max(np.abs(y + g)) < 1e-15
    # unit weights, no epsilon: the output has root mean square 1 and the input's direction
    x = r.standard_normal((5, 64))
    y = rms_norm(x, np.ones(64), 0.0)
    assert np.max(np.abs(np.sqrt(np.mean(y * y, axis=-1)) - 1.0)) < 1e-14
    assert np.max(np.abs(y / np.linalg.norm(y, axis=-1, keepdims=True) - x / np.linalg.norm(x, axis=-1, keepdims=True))) < 1e-14
    # scalar loops, independent of the vectorised form, with epsilon
    gg = r.uniform(0.5, 2.0, 64)
    xs = x[2].tolist()
    ms = sum(v * v for v in xs) / len(xs)
    want = [gi * v / math.sqrt(ms + 1e-3) for gi, v in zip(gg.tolist(), xs)]
    assert np.max(np.abs(rms_norm(x[2], gg, 1e-3) - np.array(want))) < 1e-14
    # rows are independent: a batch gives the rows one by one
    xb = r.standard_normal((3, 4, 64))
    yb = rms_norm(xb, gg, 1e-5)
    assert np.max(np.abs(yb[1, 2] - rms_norm(xb[1, 2], gg, 1e-5))) == 0.0


def test_rms_norm():
    check_rms_norm(orc.rms_norm)


def check_kv_cache(kv_rms_norm_rope_cache):
    r = rng(9)
    T, H, D, S = 6, 2, 16, 10
    k = r.standard_normal((T, H, D))
    v = r.standard_normal((T, H, D))
    g = r.uniform(0.5, 2.0, D)
    theta = r.uniform(-3, 3, size=(T, D // 2))
    emb = np.concatenate([theta, theta], axis=-1)
    cos, sin = np.cos(emb), np.sin(emb)
    slots = np.array([3, 7, -1, 0, 9, 5, 10])
    k = np.concatenate([k, r.standard_normal((1, H, D))])
    v = np.concatenate([v, r.standard_normal((1, H, D))])
    theta = np.concatenate([theta, r.uniform(-3, 3, size=(1, D // 2))])
    emb = np.concatenate([theta, theta], axis=-1)
    cos, sin = np.cos(emb), np.sin(emb)
    kc0 = r.standard_normal((S, H, D))
    vc0 = r.standard_normal((S, H, D))
    kc, vc = kv_rms_norm_rope_cache(k, v, g, 1e-6, cos, sin, slots, kc0, vc0)
    # slot 10 is past the cache: skipped like -1
    untouched = [s for s in range(S) if s not in slots.tolist()]
    assert len(untouched) == 5
    assert np.array_equal(kc[untouched], kc0[untouched]) and np.array_equal(vc[untouched], vc0[untouched])
    # without gamma: pure rotation of the raw row, pair by pair
    kc2, _ = kv_rms_norm_rope_cache(k, v, None, 1e-6, cos, sin, slots, kc0, vc0)
    for t, slot in ((0, 3), (5, 5)):
        for i in range(D // 2):
            c, s_ = math.cos(theta[t, i]), math.sin(theta[t, i])
            assert abs(kc2[slot, 1, i] - (c * k[t, 1, i] - s_ * k[t, 1, i + D // 2])) < 1e-12
            assert abs(kc2[slot, 1, i + D // 2] - (s_ * k[t, 1, i] + c * k[t, 1, i + D // 2])) < 1e-12
    for t, slot in enumerate(slots.tolist()):
        if slot < 0 or slot >= S:
            continue
        assert np.array_equal(vc[slot], v[t])
        for h in range(H):
            # rotation keeps the normalised row's length: sqrt(sum((g*x/rms)^2))
            n = np.linalg.norm(g * k[t, h] / math.sqrt(np.mean(k[t, h] ** 2) + 1e-6))
            assert abs(np.linalg.norm(kc[slot, h]) - n) < 1e-12 * n
            # and each pair (i, i+D/2) is the normalised pair turned by theta_i
            y = g * k[t, h] / math.sqrt(np.mean(k[t, h] ** 2) + 1e-6)
            for i in range(D // 2):
                c, s_ = math.cos(theta[t, i]), math.sin(theta[t, i])
                assert abs(kc[slot, h, i] - (c * y[i] - s_ * y[i + D // 2])) < 1e-12
                assert abs(kc[slot, h, i + D // 2] - (s_ * y[i] + c * y[i + D // 2])) < 1e-12


def test_kv_rms_norm_rope_cache():
    check_kv_cache(orc.kv_rms_norm_rope_cache)


# --------------------------------------------------------------------------- decode over a paged cache
def check_cache_slots(cache_slots):
    # hand-worked: blocks of 4, logical blocks 0, 1 -> physical 5, 2
    assert cache_slots([5, 2], 6, 4).tolist() == [20, 21, 22, 23, 8, 9]
    assert cache_slots([3], 0, 4).tolist() == []
    assert cache_slots([7, 1, 4], 9, 3).tolist() == [21, 22, 23, 3, 4, 5, 12, 13, 14]


def test_cache_slots():
    check_cache_slots(orc.cache_slots)


def _decode_brute(q, cos, sin, kc, vc, table, lens, bs, scale):
    """Scalar loops: rotate the query pair by pair, then exp-weighted sums over the cache."""
    B, Hq, D = q.shape
    Hkv = kc.shape[1]
    h2 = D // 2
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        for h in range(Hq):
            qr = [0.0] * D
            for i in range(h2):
                qr[i] = q[b, h, i] * cos[b, i] - q[b, h, i + h2] * sin[b, i]
                qr[i + h2] = q[b, h, i + h2] * cos[b, i + h2] + q[b, h, i] * sin[b, i + h2]
            kv = h // (Hq // Hkv)
            scores = []
            for j in range(lens[b]):
                slot = table[b][j // bs] * bs + j % bs
                scores.append(scale * sum(qr[d] * kc[slot, kv, d] for d in range(D)))
            m = max(scores)
            w = [math.exp(x - m) for x in scores]
            tot = sum(w)
            for j in range(lens[b]):
                slot = table[b][j // bs] * bs + j % bs
                for d in range(D):
                    out[b, h, d] += w[j] / tot * vc[slot, kv, d]
            lse[b, h] = m + math.log(tot)
    return out, lse


def check_decode(decode_attention, cache_slots):
    r = rng(10)
    # brute force on a tiny paged cache with GQA and two lengths
    B, Hq, Hkv, D, bs = 2, 4, 2, 8, 2
    lens = [3, 5]
    table = [[4, 0, 7], [1, 6, 3]]
    kc = r.standard_normal((16, Hkv, D))
    vc = r.standard_normal((16, Hkv, D))
    q = r.standard_normal((B, Hq, D))
    cos = r.uniform(-1, 1, (B, D))
    sin = r.uniform(-1, 1, (B, D))
    o, l = decode_attention(q, cos, sin, kc, vc, table, lens, bs, 0.7)
    ob, lb = _decode_brute(q, cos, sin, kc, vc, table, lens, bs, 0.7)
    assert np.max(np.abs(o - ob)) < 1e-12 and np.max(np.abs(l - lb)) < 1e-12
    # a single cached token: the output is its V, the lse its score
    o1, l1 = decode_attention(q[:1], cos[:1], sin[:1], kc, vc, [[5]], [1], 3, 1.0)
    assert np.max(np.abs(o1[0] - vc[15, np.arange(Hq) // 2])) < 1e-15
    # the last row of causal prefill attention: cache built from the prefill's keys,
    # written through a shuffled paged block table
    L, Hq, Hkv, D, bs = 37, 4, 2, 16, 8
    qs = r.standard_normal((L, Hq, D))
    ks = r.standard_normal((L, Hkv, D))
    vs = r.standard_normal((L, Hkv, D))
    f = orc.inv_freq(1e4, D)[None, :]
    sn, cs = orc.rope_tables(np.arange(L, dtype=np.int32), f, [L], 1.0)
    nblk = 6
    table = r.permutation(nblk)[None, :]
    slots = cache_slots(table[0], L, bs)
    kc, vc = orc.kv_rms_norm_rope_cache(ks, vs, None, 0.0, cs, sn, slots, np.zeros((nblk * bs, Hkv, D)),
                                        np.zeros((nblk * bs, Hkv, D)))
    o, l = decode_attention(qs[L - 1:], cs[L - 1:], sn[L - 1:], kc, vc, table, [L], bs, 0.25)
    po, pl = orc.rope_attention(qs, ks, vs, cs, sn, [L], 0.25, True)
    assert np.max(np.abs(o[0] - po[L - 1])) < 1e-12
    assert np.max(np.abs(l[0] - pl[:, L - 1])) < 1e-12


def test_decode_attention():
    check_decode(orc.decode_attention, orc.cache_slots)


# --------------------------------------------------------------------------- backward
def _fd_loss(q, k, v, dout, cos, sin, seq_lens, scale, causal, pairing):
    o, _ = orc.rope_attention(q, k, v, cos, sin, seq_lens, scale, causal, pairing)
    return float(np.sum(o * dout))


def check_backward(rope_attention_bwd):
    """Directional derivatives of the (pinned) forward by central differences."""
    r = rng(14)
    for seq_lens, Hq, Hkv, causal, pairing, tables in (([7], 2, 1, True, "half", "rotation"),
                                                       ([4, 5], 4, 2, True, "interleaved", "rotation"),
                                                       ([6], 2, 2, False, "half", "random")):
        T, D = sum(seq_lens), 8
        q = r.standard_normal((T, Hq, D))
        k = r.standard_normal((T, Hkv, D))
        v = r.standard_normal((T, Hkv, D))
        dout = r.standard_normal((T, Hq, D))
        if tables == "rotation":
            theta = r.uniform(-3, 3, size=(T, D // 2))
            cols = orc.pair_partner(D, pairing)[2]
            cos, sin = np.cos(theta[:, cols]), np.sin(theta[:, cols])
        else:   # arbitrary table values: the Rope op is then a general linear map
            cos, sin = r.uniform(-1, 1, (T, D)), r.uniform(-1, 1, (T, D))
        scale = 0.6
        dq, dk, dv = rope_attention_bwd(q, k, v, dout, cos, sin, seq_lens, scale, causal, pairing)
        eps = 1e-5
        for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
            u = r.standard_normal(x.shape)
            args = dict(q=q, k=k, v=v)
            args[name] = x + eps * u
            lp = _fd_loss(args["q"], args["k"], args["v"], dout, cos, sin, seq_lens, scale, causal, pairing)
            args[name] = x - eps * u
            lm = _fd_loss(args["q"], args["k"], args["v"], dout, cos, sin, seq_lens, scale, causal, pairing)
            fd = (lp - lm) / (2 * eps)
            an = float(np.sum(grad * u))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, seq_lens, pairing, tables, fd, an)


def test_backward_finite_differences():
    check_backward(orc.rope_attention_bwd)


def test_backward_segments_do_not_mix():
    # the gradient of one sequence's keys ignores another sequence's output gradient
    r = rng(15)
    T, H, D = 9, 2, 8
    q, k, v = (r.standard_normal((T, H, D)) for _ in range(3))
    theta = r.uniform(-3, 3, size=(T, D // 2))
    cos, sin = np.cos(np.concatenate([theta, theta], 1)), np.sin(np.concatenate([theta, theta], 1))
    dout = r.standard_normal((T, H, D))
    dout2 = dout.copy()
    dout2[:4] = r.standard_normal((4, H, D))   # change the first sequence only
    a = orc.rope_attention_bwd(q, k, v, dout, cos, sin, [4, 5], 0.5)
    b = orc.rope_attention_bwd(q, k, v, dout2, cos, sin, [4, 5], 0.5)
    for x, y in zip(a, b):
        assert np.array_equal(x[4:], y[4:]) and not np.array_equal(x[:4], y[:4])


# --------------------------------------------------------------------------- planted mistakes
# Each mutant is one plausible slip; at least one pin above must reject it.

def _mut_inv_freq_off_by_one(base, D):
    exps = np.arange(1, D + 1, 2, dtype=np.float64) / float(D)
    return (1.0 / (float(base) ** exps)).astype(np.float32)


def _mut_tables_no_concat(pos, f, seq_lens, scale=1.0, mode="fp32"):
    freq = orc.angles(pos, f, seq_lens, scale, mode)
    emb = np.repeat(freq, 2, axis=-1)      # interleaved instead of cat(freq, freq)
    return np.sin(emb), np.cos(emb)


def _mut_tables_wrong_batch(pos, f, seq_lens, scale=1.0, mode="fp32"):
    # every token uses batch 0's inverse frequencies
    f0 = np.repeat(np.asarray(f)[:1], len(seq_lens), axis=0)
    return orc.rope_tables(pos, f0, seq_lens, scale, mode)


def _mut_tables_scale_times(pos, f, seq_lens, scale=1.0, mode="fp32"):
    return orc.rope_tables(pos, f, seq_lens, 1.0 / scale, mode)


def _mut_angles_fp64(pos, f, seq_lens, scale=1.0, mode="fp32"):
    return orc.angles(pos, f, seq_lens, scale, "exact")


def _mut_rotation_adjacent(theta):
    D = 2 * len(theta)
    R = np.zeros((D, D))
    for i, th in enumerate(theta):
        c, s = math.cos(th), math.sin(th)
        R[2 * i, 2 * i], R[2 * i, 2 * i + 1], R[2 * i + 1, 2 * i], R[2 * i + 1, 2 * i + 1] = c, -s, s, c
    return R


def _mut_rotate_tokens_sign(x, cos, sin, chunk=512):
    return orc.rotate_tokens(x, cos, -np.asarray(sin))


def _mut_rotate_tokens_no_cos(x, cos, sin, chunk=512):
    return orc.rotate_tokens(x, np.ones_like(cos), sin)


def _mut_attention_no_scale(q, k, v, scale, causal=True):
    return orc.attention(q, k, v, 1.0, causal)


def _mut_attention_mask_offset(q, k, v, scale, causal=True):
    q = np.asarray(q, dtype=np.float64)
    n = q.shape[0]
    S = (q @ np.asarray(k).T) * scale
    if causal:
        S = np.where(np.tril(np.ones((n, n), dtype=bool), -1) | (n == 1), S, -np.inf)
        S[0, 0] = (q[0] @ np.asarray(k)[0]) * scale
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    return (E / l) @ np.asarray(v), m[:, 0] + np.log(l[:, 0])


def _mut_attention_transposed(q, k, v, scale, causal=True):
    o, lse = orc.attention(q, k, v, scale, causal)
    P = np.asarray(q) @ np.asarray(k).T * scale
    n = P.shape[0]
    if causal:
        P = np.where(np.tril(np.ones((n, n), dtype=bool)), P, -np.inf)
    P = np.exp(P - P.max(axis=0, keepdims=True))   # normalised over the wrong axis
    P = P / P.sum(axis=0, keepdims=True)
    return P @ np.asarray(v), lse


def _mut_rms_norm_no_mean(x, gamma, eps):
    x = np.asarray(x, dtype=np.float64)
    return np.asarray(gamma) * x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)


def _mut_kv_cache_norm_after_rope(k, v, gamma, eps, cos, sin, slots, k_cache, v_cache):
    # gamma applied after the rotation instead of before it
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    kn = k if gamma is None else orc.rms_norm(k, np.ones_like(gamma), eps)
    kr = orc.rotate_tokens(kn, cos, sin) * (1.0 if gamma is None else np.asarray(gamma))
    for t, slot in enumerate(np.asarray(slots).tolist()):
        if 0 <= slot < kc.shape[0]:
            kc[slot] = kr[t]
            vc[slot] = v[t]
    return kc, vc


def _mut_cache_slots_swapped(table_row, length, block_size):
    j = np.arange(int(length), dtype=np.int64)
    t = np.asarray(table_row, dtype=np.int64)
    return t[(j % block_size) % t.size] * block_size + j // block_size


def _mut_decode_gqa_modulo(q, cos, sin, k_cache, v_cache, block_table, cache_lens, block_size, scale):
    B, Hq, D = np.asarray(q).shape
    Hkv = np.asarray(k_cache).shape[1]
    qr = orc.rotate_tokens(np.asarray(q, dtype=np.float64), cos, sin)
    out, lse = np.zeros((B, Hq, D)), np.zeros((B, Hq))
    for b in range(B):
        sl = orc.cache_slots(block_table[b], int(cache_lens[b]), block_size)
        for h in range(Hq):
            o, l = orc.attention(qr[b, h][None], np.asarray(k_cache)[sl][:, h % Hkv],
                                 np.asarray(v_cache)[sl][:, h % Hkv], scale, causal=False)
            out[b, h], lse[b, h] = o[0], l[0]
    return out, lse


def _mut_decode_drops_last(q, cos, sin, k_cache, v_cache, block_table, cache_lens, block_size, scale):
    lens = [max(1, int(x) - 1) for x in cache_lens]
    return orc.decode_attention(q, cos, sin, k_cache, v_cache, block_table, lens, block_size, scale)


def _mut_rotation_interleaved_sign(theta_row, pairing="half"):
    return orc.rotation_matrix(-np.asarray(theta_row), pairing) if pairing == "interleaved" \
        else orc.rotation_matrix(theta_row, pairing)


def _mut_tables_interleaved_as_half(pos, inv_freq_b, seq_lens, pos_scale=1.0, mode="fp32", pairing="half"):
    return orc.rope_tables(pos, inv_freq_b, seq_lens, pos_scale, mode, "half")


def _mut_rotate_tokens_interleaved_swapped(x, cos, sin, chunk=512, pairing="half"):
    # partner taken two dims away instead of the adjacent one
    if pairing != "interleaved":
        return orc.rotate_tokens(x, cos, sin, chunk, pairing)
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    j = np.arange(D)
    partner = (j + 2) % D
    sign = np.where(j % 2 == 0, -1.0, 1.0)
    return x * np.asarray(cos)[:, None, :] + sign * x[..., partner] * np.asarray(sin)[:, None, :]


def _mut_bwd_no_transpose(q, k, v, dout, cos, sin, seq_lens, scale, causal=True, pairing="half"):
    # rotates the gradients forward instead of applying M^T
    dq, dk, dv = orc.rope_attention_bwd(q, k, v, dout, cos, sin, seq_lens, scale, causal, pairing)
    back = lambda g: orc.rotate_tokens(orc.rotate_tokens(g, cos, sin, pairing=pairing), cos, sin, pairing=pairing)
    return back(dq), back(dk), dv


def _mut_bwd_no_rowsum(q, k, v, dout, cos, sin, seq_lens, scale, causal=True, pairing="half"):
    T, Hq, D = np.asarray(q).shape
    Hkv = np.asarray(k).shape[1]
    qr = orc.rotate_tokens(q, cos, sin, pairing=pairing)
    kr = orc.rotate_tokens(k, cos, sin, pairing=pairing)
    dq, dk, dv = orc.rope_attention_bwd(q, k, v, dout, cos, sin, seq_lens, scale, causal, pairing)
    # recompute dq without the rowsum term
    g = Hq // Hkv
    dqr = np.zeros((T, Hq, D))
    for s0, L in zip(orc.segment_starts(seq_lens).tolist(), list(seq_lens)):
        sl = slice(s0, s0 + L)
        for h in range(Hq):
            S = (qr[sl, h] @ kr[sl, h // g].T) * scale
            if causal:
                S = np.where(np.tril(np.ones((L, L), dtype=bool)), S, -np.inf)
            P = np.exp(S - S.max(1, keepdims=True))
            P /= P.sum(1, keepdims=True)
            dS = P * (np.asarray(dout)[sl, h] @ np.asarray(v)[sl, h // g].T)
            dqr[sl, h] = scale * dS @ kr[sl, h // g]
    return orc.rotate_tokens_transpose(dqr, cos, sin, pairing), dk, dv


def _mut_bwd_gqa_first_head(q, k, v, dout, cos, sin, seq_lens, scale, causal=True, pairing="half"):
    # dk, dv from the first q head of each group only
    q = np.asarray(q)
    Hq, Hkv = q.shape[1], np.asarray(k).shape[1]
    g = Hq // Hkv
    dq, dk, dv = orc.rope_attention_bwd(q, k, v, dout, cos, sin, seq_lens, scale, causal, pairing)
    if g == 1:
        return dq, dk, dv
    d2 = np.array(dout, dtype=np.float64)
    for h in range(Hq):
        if h % g:
            d2[:, h] = 0.0
    _, dk1, dv1 = orc.rope_attention_bwd(q, k, v, d2, cos, sin, seq_lens, scale, causal, pairing)
    return dq, dk1, dv1


def _mut_rope_attention_gqa_strided(q, k, v, cos, sin, seq_lens, scale, causal=True):
    hq, hkv = q.shape[1], k.shape[1]
    idx = np.arange(hq) % hkv                      # strided instead of contiguous groups
    return orc.rope_attention(q, np.asarray(k)[:, idx], np.asarray(v)[:, idx], cos, sin, seq_lens, scale, causal)


def _mut_rope_attention_no_segments(q, k, v, cos, sin, seq_lens, scale, causal=True):
    return orc.rope_attention(q, k, v, cos, sin, [int(np.sum(seq_lens))], scale, causal)


@pytest.mark.parametrize("name,run", [
    ("inv_freq off by one", lambda g: check_inv_freq(_mut_inv_freq_off_by_one)),
    ("tables interleaved", lambda g: check_table_structure(_mut_tables_no_concat)),
    ("tables interleaved (golden)", lambda g: check_tables_golden(_mut_tables_no_concat, g)),
    ("tables wrong batch row", lambda g: check_tables_golden(_mut_tables_wrong_batch, g)),
    ("scaling multiplies", lambda g: check_tables_golden(_mut_tables_scale_times, g)),
    ("angles not rounded to fp32", lambda g: check_angles_fp32(_mut_angles_fp64)),
    ("adjacent pairs", lambda g: check_rotation(_mut_rotation_adjacent, orc.rope_op_matrix, orc.rotate_tokens)),
    ("rotation sign", lambda g: check_rotation(orc.rotation_matrix, orc.rope_op_matrix, _mut_rotate_tokens_sign)),
    ("rotation drops cos", lambda g: check_rotation(orc.rotation_matrix, orc.rope_op_matrix, _mut_rotate_tokens_no_cos)),
    ("relative position, no cos", lambda g: check_relative_position(orc.rope_tables, _mut_rotate_tokens_no_cos)),
    ("attention drops scale", lambda g: check_attention(_mut_attention_no_scale)),
    ("causal mask off by one", lambda g: check_attention(_mut_attention_mask_offset)),
    ("softmax over wrong axis", lambda g: check_attention(_mut_attention_transposed)),
    ("GQA strided groups", lambda g: check_rope_attention(_mut_rope_attention_gqa_strided, orc.rope_attention_rows)),
    ("segments ignored", lambda g: check_rope_attention(_mut_rope_attention_no_segments, orc.rope_attention_rows)),
    ("RMS without the mean", lambda g: check_rms_norm(_mut_rms_norm_no_mean)),
    ("gamma after the rotation", lambda g: check_kv_cache(_mut_kv_cache_norm_after_rope)),
    ("block and offset swapped", lambda g: check_cache_slots(_mut_cache_slots_swapped)),
    ("decode block and offset swapped", lambda g: check_decode(orc.decode_attention, _mut_cache_slots_swapped)),
    ("decode GQA by modulo", lambda g: check_decode(_mut_decode_gqa_modulo, orc.cache_slots)),
    ("decode drops the newest key", lambda g: check_decode(_mut_decode_drops_last, orc.cache_slots)),
    ("interleaved rotation sign", lambda g: check_interleaved(_mut_rotation_interleaved_sign, orc.rope_op_matrix,
                                                              orc.rotate_tokens, orc.rope_tables)),
    ("interleaved tables in half layout", lambda g: check_interleaved(orc.rotation_matrix, orc.rope_op_matrix,
                                                                      orc.rotate_tokens,
                                                                      _mut_tables_interleaved_as_half)),
    ("interleaved partner two away", lambda g: check_interleaved(orc.rotation_matrix, orc.rope_op_matrix,
                                                                 _mut_rotate_tokens_interleaved_swapped,
                                                                 orc.rope_tables)),
    ("backward without the transpose", lambda g: check_backward(_mut_bwd_no_transpose)),
    ("backward without the rowsum", lambda g: check_backward(_mut_bwd_no_rowsum)),
    ("backward GQA from one head", lambda g: check_backward(_mut_bwd_gqa_first_head)),
])
def test_pins_reject_planted_mistakes(name, run, golden_dir):
    with open(os.path.join(golden_dir, "dynamic_ntk_tiny.json")) as fh:
        golden = json.load(fh)
    with pytest.raises(AssertionError):
        run(golden)
