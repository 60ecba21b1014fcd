"""CPU oracle for rotary position embedding (RoPE) fused into a FlashAttention forward pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  The product
path (the HIP library and its Python binding) never imports it, and this module
imports nothing from the product package.

Everything here is plain numpy in float64 and follows the definitions on the
source pages, with no blocking, fusion or reordering beyond what the definitions
state.  Page key used in the citations:

* [RoPE-fusion blog]  devpress.csdn.net/awstech/6a91ac403bda720d4b352e13 — RoPE
  fused into FlashAttention in ops-transformer (sections 1.2, 5.3).
* [FlashAttention blog]  hwcomputing.csdn.net/6a0d3f5c662f9a54cb75d0b0 — the
  attention formula and its three steps ("Attention 的显存坑在哪"), online softmax.
* [DynamicNTKOperation]  hiascend.com API page ascendtb_01_0140 — sections
  功能说明 (function), 算子功能分析 (formula), 输入/输出 (inputs/outputs),
  约束说明 (constraints).
* [RoPE/GQA tutorial]  smarter.xin/posts/3494b8a4 — section 五 (relative
  position), 六 (rotation geometry), 八 (RMSNorm), 十一/十二 (MQA/GQA).

Readings taken where the pages are silent (also listed in the design notes):
rotate-half pairing by default (dims i and i+D/2 share frequency i, from emb =
cat(freq, freq)); the interleaved pairing of [RoPE/GQA tutorial, section 六]
((x_1, x_2), (x_3, x_4), ...: dims 2i and 2i+1 share frequency i, tables hold each
pair's angle in both of its columns) as the ``pairing="interleaved"`` variant;
rotation sign R = [[cos, -sin], [sin, cos]] on each pair;
angles formed in float32 (int32 positions, float32 inverse frequencies);
contiguous GQA grouping (kv head = q head // group); softmax scale passed in.

Parity status: every function below is pinned by tests/test_oracle.py except
``ntk_base``, whose formula is not on the pages (parity unpinned against the pages;
pinned are the page's "no change at or below the trained length" and the reading's
defining property: the lowest inverse frequency divided by exactly L / L_train, the
highest unchanged).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "inv_freq",
    "ntk_base",
    "inv_freq_per_sequence",
    "segment_ids",
    "segment_starts",
    "angles",
    "rope_tables",
    "rotation_matrix",
    "rope_op_matrix",
    "rotate_tokens",
    "attention",
    "rope_attention",
    "rope_attention_rows",
    "round_rne",
    "ulp",
    "DTYPE_FORMATS",
    "rms_norm",
    "kv_rms_norm_rope_cache",
    "cache_slots",
    "decode_attention",
    "pair_partner",
    "PAIRINGS",
    "rotate_tokens_transpose",
    "rope_attention_bwd",
]

PAIRINGS = ("half", "interleaved")

# (precision p incl. the implicit bit, minimum normal exponent emin)
DTYPE_FORMATS = {"f16": (11, -14), "bf16": (8, -126), "f32": (24, -126)}


# --------------------------------------------------------------------------- a1
def inv_freq(base: float, head_size: int) -> np.ndarray:
    """Inverse frequencies f_i = base^(-2i/D) for i < D/2, as float32.

    [RoPE-fusion blog, section 1.2]: frequency i is the reciprocal of base raised to the
    power 2i/D, for the even dimension indices 2i < D.
    Formed in float64 and rounded once to float32, since the table op takes its
    inverse frequencies as a float32 input ([DynamicNTKOperation, 输入 table]).
    """
    if head_size <= 0 or head_size % 2:
        raise ValueError("head_size must be a positive even number")
    exps = np.arange(0, head_size, 2, dtype=np.float64) / float(head_size)
    return (1.0 / (float(base) ** exps)).astype(np.float32)


def ntk_base(base: float, seq_len: int, trained_len: int, head_size: int) -> float:
    """Dynamic-NTK base for one sequence.  PARITY UNPINNED (formula not on the pages).

    [DynamicNTKOperation, 功能说明]: no interpolation when the inference length is at
    most the trained length; above it the base is enlarged.  The enlargement law is
    lost from the page (its InvFreqs formula did not survive); the reading used is
    base * (L / L_train) ** (D / (D - 2)).
    """
    if seq_len <= trained_len:
        return float(base)
    return float(base) * (float(seq_len) / float(trained_len)) ** (float(head_size) / float(head_size - 2))


def inv_freq_per_sequence(base: float, seq_lens, head_size: int, trained_len: int | None) -> np.ndarray:
    """[batch, D/2] float32 inverse frequencies, one row per sequence.

    [DynamicNTKOperation, 输入]: InvFreqs has shape [batch, headSize/2].  With
    ``trained_len=None`` every row uses ``base`` (no NTK scaling).
    """
    rows = []
    for L in np.asarray(seq_lens).tolist():
        b = float(base) if trained_len is None else ntk_base(base, int(L), int(trained_len), head_size)
        rows.append(inv_freq(b, head_size))
    return np.stack(rows, axis=0)


# --------------------------------------------------------------------------- segments
def segment_ids(seq_lens) -> np.ndarray:
    """b(t) for every packed token t: tokens are laid out sequence after sequence.

    [DynamicNTKOperation, 算子功能分析]: each batch's positionIds are taken out by its
    seqLen; positionIds is the concatenation [0..L_0-1, 0..L_1-1, ...] ([输入]).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    return np.repeat(np.arange(seq_lens.size, dtype=np.int64), seq_lens)


def segment_starts(seq_lens) -> np.ndarray:
    """First packed token index of every sequence (exclusive prefix sum of seqLens)."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(seq_lens)[:-1]]).astype(np.int64)


# --------------------------------------------------------------------------- a2
def angles(pos, inv_freq_b, seq_lens, pos_scale: float = 1.0, mode: str = "fp32") -> np.ndarray:
    """freq[t, i] = (pos[t] / s) * f[b(t), i], the outer product per sequence.

    [DynamicNTKOperation, 算子功能分析]: for each batch, the outer product of that batch's
    position ids with its row of inverse frequencies.  The linear ``rope_scaling_factor`` s of [RoPE-fusion blog,
    section 5.3] divides positions before the outer product.

    mode "fp32": the division and the product are each rounded to float32, as they
    are when int32 positions meet float32 inverse frequencies (the parity mode).
    mode "exact": float64 throughout (used for the relative-position invariant).
    Returns float64 [T, D/2] holding the (float32-representable in fp32 mode) angles.
    """
    pos = np.asarray(pos)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    inv_freq_b = np.asarray(inv_freq_b)
    if int(seq_lens.sum()) != pos.shape[0]:
        raise ValueError("sum(seq_lens) must equal ntokens")
    out = np.empty((pos.shape[0], inv_freq_b.shape[1]), dtype=np.float64)
    start = 0
    for b, L in enumerate(seq_lens.tolist()):
        p = pos[start:start + L]
        if mode == "fp32":
            t = p.astype(np.float32) / np.float32(pos_scale)          # fl32(p / s)
            freq = np.einsum("i,j->ij", t, inv_freq_b[b].astype(np.float32))  # fl32 products
            out[start:start + L] = freq.astype(np.float64)
        elif mode == "exact":
            t = p.astype(np.float64) / float(pos_scale)
            out[start:start + L] = np.einsum("i,j->ij", t, inv_freq_b[b].astype(np.float64))
        else:
            raise ValueError(mode)
        start += L
    return out


def pair_partner(D: int, pairing: str = "half"):
    """(partner, sign, freq_index) of every dimension j < D for the given pairing.

    Rotating pair (a, b) by theta gives a' = a cos - b sin, b' = b cos + a sin, so
    x'_j = x_j cos_j + sign_j * x_partner(j) * sin_j with sign -1 on the first member of
    the pair.  "half": pair i = (i, i + D/2) (emb = cat(freq, freq)); "interleaved":
    pair i = (2i, 2i + 1) ([RoPE/GQA tutorial, section 六], adjacent 2-D blocks).
    freq_index[j] is the frequency (table angle) that dimension j uses.
    """
    j = np.arange(D)
    if pairing == "half":
        h = D // 2
        return np.where(j < h, j + h, j - h), np.where(j < h, -1.0, 1.0), j % h
    if pairing == "interleaved":
        return j ^ 1, np.where(j % 2 == 0, -1.0, 1.0), j // 2
    raise ValueError(pairing)


def rope_tables(pos, inv_freq_b, seq_lens, pos_scale: float = 1.0, mode: str = "fp32", pairing: str = "half"):
    """(sin, cos), each float64 [ntokens, D].

    [DynamicNTKOperation, 算子功能分析]: the sine and the cosine of the angle matrix placed
    twice side by side along the last axis (column j and column j + D/2 hold angle j).
    Output shape [ntokens, headSize] ([输出]).  With
    pairing="interleaved" column j holds the angle of frequency j // 2 instead.
    """
    freq = angles(pos, inv_freq_b, seq_lens, pos_scale, mode)
    D = 2 * freq.shape[1]
    emb = np.ascontiguousarray(freq[:, pair_partner(D, pairing)[2]])
    return np.sin(emb), np.cos(emb)


# --------------------------------------------------------------------------- rotation
def rotation_matrix(theta_row, pairing: str = "half") -> np.ndarray:
    """Explicit D x D rotation for one token, from its D/2 angles.

    [RoPE/GQA tutorial, section 六]: the vector is split into 2-D pairs and each pair is
    rotated by a position-dependent angle; [RoPE-fusion blog, section 一]: each token is
    multiplied by a position-dependent rotation matrix.  "half": pair i is
    (x_i, x_{i+D/2}) (the layout of emb = cat(freq, freq)); "interleaved": pair i is
    (x_{2i}, x_{2i+1}).  Angle theta_i either way.
    """
    theta_row = np.asarray(theta_row, dtype=np.float64)
    half = theta_row.shape[0]
    D = 2 * half
    R = np.zeros((D, D), dtype=np.float64)
    for i in range(half):
        a, b = (i, i + half) if pairing == "half" else (2 * i, 2 * i + 1)
        if pairing not in PAIRINGS:
            raise ValueError(pairing)
        c, s = np.cos(theta_row[i]), np.sin(theta_row[i])
        R[a, a] = c
        R[a, b] = -s
        R[b, a] = s
        R[b, b] = c
    return R


def rope_op_matrix(cos_row, sin_row, pairing: str = "half") -> np.ndarray:
    """Explicit D x D matrix of the Rope op for one token, from its table rows.

    [DynamicNTKOperation, 算子上下文]: q, k, sin, cos enter the Rope op, which outputs the
    rotated q, k.  Written out per element: x'_j = x_j cos_j + rh(x)_j sin_j with
    rh(x) = cat(-x[D/2:], x[:D/2]) for "half" and rh(x)_{2i} = -x_{2i+1},
    rh(x)_{2i+1} = x_{2i} for "interleaved".  For tables in the matching form this is
    the rotation of ``rotation_matrix``; for arbitrary table values it is the same map.
    """
    cos_row = np.asarray(cos_row, dtype=np.float64)
    sin_row = np.asarray(sin_row, dtype=np.float64)
    D = cos_row.shape[0]
    partner, sign, _ = pair_partner(D, pairing)
    M = np.zeros((D, D), dtype=np.float64)
    for j in range(D):
        M[j, j] = cos_row[j]
        M[j, partner[j]] = sign[j] * sin_row[j]
    return M


def rotate_tokens(x, cos, sin, chunk: int = 512, pairing: str = "half") -> np.ndarray:
    """Apply each token's explicit Rope-op matrix to x [T, H, D] (float64 out).

    Token t uses rope_op_matrix(cos[t], sin[t], pairing); every head of the token shares
    it.  Matrices are built in token chunks to bound memory.
    """
    x = np.asarray(x, dtype=np.float64)
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    T, H, D = x.shape
    out = np.empty_like(x)
    idx = np.arange(D)
    partner, sign, _ = pair_partner(D, pairing)
    for t0 in range(0, T, chunk):
        t1 = min(T, t0 + chunk)
        n = t1 - t0
        M = np.zeros((n, D, D), dtype=np.float64)
        M[:, idx, idx] = cos[t0:t1]
        M[:, idx, partner] = sign[None, :] * sin[t0:t1]
        out[t0:t1] = np.einsum("tij,thj->thi", M, x[t0:t1])
    return out


# --------------------------------------------------------------------------- attention
def attention(q, k, v, scale: float, causal: bool = True):
    """Softmax(Q K^T * scale) V for one head with the full N x N score matrix.

    [FlashAttention blog, "Attention 的显存坑在哪"]: Attention(Q,K,V) = Softmax(QK^T/sqrt(d))V
    computed in three steps: the (N, N) scores, the row softmax, the product with V.
    Causal: key j > query i is excluded.  Returns (O [N, D], lse [N]) with
    lse = log(sum_j exp(score_ij)) over the kept keys.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    S = (q @ k.T) * float(scale)
    if causal:
        S = np.where(np.tril(np.ones((n, k.shape[0]), dtype=bool)), S, -np.inf)
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    l = E.sum(axis=1, keepdims=True)
    P = E / l
    return P @ v, (m[:, 0] + np.log(l[:, 0]))


def _check_packed(q, k, v, seq_lens):
    T, Hq, D = q.shape
    if k.shape[0] != T or v.shape[0] != T or k.shape[2] != D or v.shape[2] != D:
        raise ValueError("q, k, v must be packed [T, H, D] with the same T and D")
    Hkv = k.shape[1]
    if v.shape[1] != Hkv or Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv and k, v must share Hkv")
    if int(np.sum(seq_lens)) != T:
        raise ValueError("sum(seq_lens) must equal T")
    return T, Hq, Hkv, D


def rope_attention(q, k, v, cos, sin, seq_lens, scale: float, causal: bool = True, pairing: str = "half"):
    """Full oracle: rotate Q and K with their tokens' tables, then attention per
    (sequence, q head).  Packed layout: q [T, Hq, D], k/v [T, Hkv, D], tables [T, D].

    GQA ([RoPE/GQA tutorial, section 十二]): q heads are split into Hkv groups of
    g = Hq / Hkv contiguous heads; group j shares kv head j.
    Returns (O [T, Hq, D], lse [Hq, T]) in float64.
    """
    T, Hq, Hkv, D = _check_packed(q, k, v, seq_lens)
    g = Hq // Hkv
    qr = rotate_tokens(q, cos, sin, pairing=pairing)
    kr = rotate_tokens(k, cos, sin, pairing=pairing)
    v = np.asarray(v, dtype=np.float64)
    O = np.empty((T, Hq, D), dtype=np.float64)
    lse = np.empty((Hq, T), dtype=np.float64)
    for s0, L in zip(segment_starts(seq_lens).tolist(), np.asarray(seq_lens).tolist()):
        for h in range(Hq):
            kvh = h // g
            o, l = attention(qr[s0:s0 + L, h], kr[s0:s0 + L, kvh], v[s0:s0 + L, kvh], scale, causal)
            O[s0:s0 + L, h] = o
            lse[h, s0:s0 + L] = l
    return O, lse


def rope_attention_rows(q, k, v, cos, sin, seq_lens, scale: float, causal: bool, samples, pairing: str = "half"):
    """Oracle output rows O[t, h, :] (and lse) for a list of (t, h) samples only.

    The same definition as ``rope_attention`` evaluated one query row at a time, so
    that full-size problems can be checked on sampled outputs.  Rotated keys of a
    (sequence, kv head) are formed once and reused across samples.
    """
    T, Hq, Hkv, D = _check_packed(q, k, v, seq_lens)
    g = Hq // Hkv
    seg = segment_ids(seq_lens)
    starts = segment_starts(seq_lens)
    lens = np.asarray(seq_lens, dtype=np.int64)
    cache = {}
    outs, lses = [], []
    for t, h in samples:
        b = int(seg[t])
        s0, L = int(starts[b]), int(lens[b])
        kvh = h // g
        key = (b, kvh)
        if key not in cache:
            kr = rotate_tokens(np.asarray(k[s0:s0 + L, kvh:kvh + 1]), cos[s0:s0 + L], sin[s0:s0 + L],
                               pairing=pairing)[:, 0]
            cache[key] = (kr, np.asarray(v[s0:s0 + L, kvh], dtype=np.float64))
        kr, vv = cache[key]
        qr = rotate_tokens(np.asarray(q[t:t + 1, h:h + 1]), cos[t:t + 1], sin[t:t + 1], pairing=pairing)[0, 0]
        i = t - s0
        n_keys = i + 1 if causal else L
        s = (kr[:n_keys] @ qr) * float(scale)
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        outs.append((e / l) @ vv[:n_keys])
        lses.append(m + np.log(l))
    return np.stack(outs), np.asarray(lses)


# --------------------------------------------------------------------------- backward
def rotate_tokens_transpose(g, cos, sin, pairing: str = "half") -> np.ndarray:
    """Apply the transpose of each token's Rope-op matrix to g [T, H, D] (float64 out).

    The forward maps x to M_t x (``rope_op_matrix``); the gradient with respect to x of a
    function of M_t x is M_t^T times its gradient with respect to M_t x.
    """
    g = np.asarray(g, dtype=np.float64)
    cos = np.asarray(cos, dtype=np.float64)
    sin = np.asarray(sin, dtype=np.float64)
    out = np.empty_like(g)
    for t in range(g.shape[0]):
        M = rope_op_matrix(cos[t], sin[t], pairing)
        out[t] = g[t] @ M          # row vectors: (M^T g^T)^T = g M
    return out


def rope_attention_bwd(q, k, v, dout, cos, sin, seq_lens, scale: float, causal: bool = True,
                       pairing: str = "half"):
    """Gradients (dq, dk, dv) of sum(O * dout) for O = rope_attention(q, k, v, ...).

    The pages say the operator serves training ([FlashAttention blog]) without writing the
    backward out; these are the derivatives of the forward definition, in the usual
    three-matrix form per (sequence, q head): with P the row softmax of S = scale * q' k'^T,
      dV = P^T dO,   dP = dO V^T,   dS = P * (dP - rowsum(dP * P)),
      dq' = scale * dS k',   dk' = scale * dS^T q',
    then dq = M^T dq' and dk = M^T dk' through each token's Rope-op matrix M.  GQA: the
    gradients of a kv head sum over the q heads of its group.  Float64 throughout.
    """
    T, Hq, Hkv, D = _check_packed(q, k, v, seq_lens)
    g = Hq // Hkv
    dout = np.asarray(dout, dtype=np.float64)
    qr = rotate_tokens(q, cos, sin, pairing=pairing)
    kr = rotate_tokens(k, cos, sin, pairing=pairing)
    v = np.asarray(v, dtype=np.float64)
    dqr = np.zeros((T, Hq, D))
    dkr = np.zeros((T, Hkv, D))
    dv = np.zeros((T, Hkv, D))
    for s0, L in zip(segment_starts(seq_lens).tolist(), np.asarray(seq_lens).tolist()):
        sl = slice(s0, s0 + L)
        for h in range(Hq):
            kvh = h // g
            S = (qr[sl, h] @ kr[sl, kvh].T) * float(scale)
            if causal:
                S = np.where(np.tril(np.ones((L, L), dtype=bool)), S, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            dO = dout[sl, h]
            dv[sl, kvh] += P.T @ dO
            dP = dO @ v[sl, kvh].T
            dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
            dqr[sl, h] = float(scale) * dS @ kr[sl, kvh]
            dkr[sl, kvh] += float(scale) * dS.T @ qr[sl, h]
    dq = rotate_tokens_transpose(dqr, cos, sin, pairing)
    dk = rotate_tokens_transpose(dkr, cos, sin, pairing)
    return dq, dk, dv


# --------------------------------------------------------------------------- KV-cache step
def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """RMSNorm over the last axis: gamma * x / sqrt(mean(x^2) + eps).

    [RoPE/GQA tutorial, section 八]: scale by the root mean square, no mean subtraction.
    """
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * x / np.sqrt(ms + float(eps))


def kv_rms_norm_rope_cache(k, v, gamma, eps, cos, sin, slots, k_cache, v_cache, pairing: str = "half"):
    """The fused "RMSNorm, RoPE, write to the KV cache" step for new tokens.

    The [RoPE-fusion blog] (section 五) names this step (kv_rms_norm_rope_cache) without
    defining it; the reading taken: for every new token t and kv head h,
      k_cache[slots[t], h] = rope(rms_norm(k[t, h], gamma, eps), cos[t], sin[t])
      v_cache[slots[t], h] = v[t, h]
    with rope the Rope-op matrix of ``rope_op_matrix`` and tokens whose slot is negative
    or past the cache skipped.  ``gamma=None`` leaves out the normalisation (RoPE and the
    cache write only).  k, v: [T, H, D]; caches: [num_slots, H, D]; returns new float64
    caches.
    """
    k = np.asarray(k, dtype=np.float64)
    kc = np.array(k_cache, dtype=np.float64, copy=True)
    vc = np.array(v_cache, dtype=np.float64, copy=True)
    kn = k if gamma is None else rms_norm(k, gamma, eps)
    kr = rotate_tokens(kn, cos, sin, pairing=pairing)
    for t, slot in enumerate(np.asarray(slots).tolist()):
        if slot < 0 or slot >= kc.shape[0]:
            continue
        kc[slot] = kr[t]
        vc[slot] = np.asarray(v[t], dtype=np.float64)
    return kc, vc


def cache_slots(block_table_row, length: int, block_size: int) -> np.ndarray:
    """Cache slots of logical token positions 0..length-1 of one sequence.

    Token j lives in logical block j // block_size at offset j % block_size; the block
    table maps the logical block to a physical one (paged KV cache, [FlashAttention blog],
    KV-cache pitfall), so the slot is table[j // block_size] * block_size + j % block_size.
    """
    j = np.arange(int(length), dtype=np.int64)
    table = np.asarray(block_table_row, dtype=np.int64)
    return table[j // block_size] * block_size + j % block_size


def decode_attention(q, cos, sin, k_cache, v_cache, block_table, cache_lens, block_size: int, scale: float,
                     pairing: str = "half"):
    """One decode step: each sequence's new query attends to every token in its cache.

    The query q[b, h] (one new token per sequence) is rotated with its table row
    (cos[b], sin[b]; the Rope-op matrix of ``rope_op_matrix``); the cached keys are used as
    stored (they were rotated when written, see ``kv_rms_norm_rope_cache``).  For q head h
    and kv head h // (Hq / Hkv) ([RoPE/GQA tutorial], sections 十一/十二):
      out[b, h] = softmax_j(scale * q'[b, h] . K[b, j]) @ V[b, j],  j < cache_lens[b]
    ([FlashAttention blog]: Softmax(QK^T / sqrt(d)) V).  All keys of the cache precede the
    query, so nothing is masked.  q: [B, Hq, D]; cos, sin: [B, D]; caches: [num_slots, Hkv, D];
    block_table: [B, max_blocks].  Returns (out [B, Hq, D], lse [B, Hq]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    kc = np.asarray(k_cache, dtype=np.float64)
    vc = np.asarray(v_cache, dtype=np.float64)
    B, Hq, D = q.shape
    Hkv = kc.shape[1]
    g = Hq // Hkv
    qr = rotate_tokens(q, cos, sin, pairing=pairing)
    out = np.zeros((B, Hq, D))
    lse = np.zeros((B, Hq))
    for b in range(B):
        sl = cache_slots(block_table[b], int(cache_lens[b]), block_size)
        K, V = kc[sl], vc[sl]                       # [L, Hkv, D]
        for h in range(Hq):
            o, l = attention(qr[b, h][None, :], K[:, h // g], V[:, h // g], scale, causal=False)
            out[b, h], lse[b, h] = o[0], l[0]
    return out, lse


# --------------------------------------------------------------------------- numerics helpers
def round_rne(x, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest value of a binary format (ties to even),
    keeping subnormals (no flush).  dtype in {"f16", "bf16", "f32"}; returns float64.

    Used to model the rounding of inputs and tables to their storage type.  Values
    beyond the format's largest finite number are not expected here (inputs are
    N(0,1) and tables lie in [-1, 1]).
    """
    p, emin = DTYPE_FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    mant, exp = np.frexp(x[nz])              # x = mant * 2**exp, 0.5 <= |mant| < 1
    e = np.maximum(exp - 1, emin)            # exponent of the leading bit, clamped at emin
    quantum = np.ldexp(1.0, e - (p - 1))     # spacing of representable values there
    out[nz] = np.rint(x[nz] / quantum) * quantum   # np.rint rounds half to even
    out[~np.isfinite(x)] = x[~np.isfinite(x)]
    return out


def ulp(x, dtype: str) -> np.ndarray:
    """Unit in the last place of the format at |x|: 2^(max(floor(log2|x|), emin) - p + 1).

    At x = 0 this is the smallest subnormal of the format.
    """
    p, emin = DTYPE_FORMATS[dtype]
    x = np.abs(np.asarray(x, dtype=np.float64))
    e = np.full(x.shape, emin, dtype=np.int64)
    nz = x > 0
    _, ex = np.frexp(x[nz])
    e[nz] = np.maximum(ex - 1, emin)
    return np.ldexp(1.0, (e - (p - 1)).astype(np.int64))
