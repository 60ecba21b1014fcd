"""The per-element bar of the backward parity tests, and the rounding model it rests on.

Test infrastructure (CPU, float64).  The backward kernels round the rotated rows q', k',
the probabilities P and dS = P o (dP - Delta) to the input type for the matrix cores, read
the forward's output O (stored in the input type), accumulate in float32 and store the
gradients in the input type.  Each gradient element is a sum over a sequence's rows of
products that carry these roundings, so its error is a sum of many small terms of either
sign: a part relative to the element itself (the stored rounding, coherent rounding of its
largest terms) and a part on the scale of the gradient's typical element (the random walk
of the rounding errors of all its terms).  The bar, per element, is

    |got - ref| <= u * (BAR_REL * |ref| + BAR_ABS * rms(ref)) + FLOOR

with u the unit roundoff of the input type (2^-8 bf16, 2^-11 fp16), rms over the
gradient tensor, and FLOOR = 2^-16 for gradients that vanish exactly (a one-token sequence
has dS = 0: dP - Delta cancels, and the kernels' float32 sums leave a residue near 2^-24
times a few units).  ``emulated_backward`` applies exactly those roundings to the exact
derivative's computation in float64; tests/test_bwd_bar.py checks that its errors stay
within half the bar on reduced workloads and at a full sequence length of 4096 (where the
random walk of the rounding errors is longest), so the constants are set by the rounding
model, not by the kernels.
"""

import numpy as np

import oracle as orc

UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
BAR_REL = 8.0      # the part relative to the element
BAR_ABS = 64.0     # the part on the scale of the gradient's typical element
FLOOR = 2.0 ** -16


def backward_bar(ref, dtype):
    """Per-element bound for a gradient tensor whose exact value is ref."""
    ref = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    return UNIT_ROUNDOFF[dtype] * (BAR_REL * np.abs(ref) + BAR_ABS * rms) + FLOOR


def emulated_backward(q, k, v, dout, cos, sin, seq_lens, scale, causal, dtype, pairing="half"):
    """(dq, dk, dv) of the oracle's definition with the kernels' rounding points applied:
    q' = M q and k' = M k rounded to dtype, P rounded to dtype (from the exact scores of the
    rounded rows), O = P V rounded to dtype (the forward output Delta reads), dS rounded to
    dtype, and dq = M^T dq', dk = M^T dk', dv rounded to dtype.  Everything else float64."""
    def rnd(x):
        return orc.round_rne(x, dtype)
    T, Hq, D = np.asarray(q).shape
    Hkv = np.asarray(k).shape[1]
    g = Hq // Hkv
    qr = rnd(orc.rotate_tokens(q, cos, sin, pairing=pairing))
    kr = rnd(orc.rotate_tokens(k, cos, sin, pairing=pairing))
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    dqr = np.zeros((T, Hq, D))
    dkr = np.zeros((T, Hkv, D))
    dv = np.zeros((T, Hkv, D))
    for s0, L in zip(orc.segment_starts(seq_lens).tolist(), np.asarray(seq_lens).tolist()):
        sl = slice(s0, s0 + L)
        keep = np.tril(np.ones((L, L), dtype=bool)) if causal else np.ones((L, L), dtype=bool)
        for h in range(Hq):
            j = h // g
            Q, K, V, dO = qr[sl, h], kr[sl, j], v[sl, j], dout[sl, h]
            S = np.where(keep, (Q @ K.T) * scale, -np.inf)
            P = np.exp(S - S.max(axis=1, keepdims=True))
            P /= P.sum(axis=1, keepdims=True)
            O = rnd(P @ V)
            Pr = rnd(P)
            dv[sl, j] += Pr.T @ dO
            dS = rnd(Pr * (dO @ V.T - np.sum(dO * O, axis=1, keepdims=True)))
            dqr[sl, h] = scale * (dS @ K)
            dkr[sl, j] += scale * (dS.T @ Q)
    dq = rnd(orc.rotate_tokens_transpose(dqr, cos, sin, pairing))
    dk = rnd(orc.rotate_tokens_transpose(dkr, cos, sin, pairing))
    return dq, dk, rnd(dv)
