"""CPU check of the backward parity bar: the rounding model of tests/bwd_bar.py stays within
half the bar on reduced workloads of both 16-bit types, GQA and MHA, causal or not, both
pairings; and the bar rejects a gradient with one element off by the model's whole error
budget (a bar too loose to notice a wrong element would fail this)."""

import dataclasses

import numpy as np
import pytest

import oracle as orc
from rope_flashattention_amd import workloads as wl
from bwd_bar import backward_bar, emulated_backward, UNIT_ROUNDOFF


def _case(cfg, dtype, causal, pairing, seed):
    w = dataclasses.replace(wl.SMALL[cfg], dtype=dtype, seed=seed)
    inp = wl.generate(w)
    q, k, v = inp.packed()
    f = orc.inv_freq_per_sequence(w.base, inp.seq_lens, w.head_dim, w.trained_len)
    s, c = orc.rope_tables(inp.pos, f, inp.seq_lens, w.pos_scale, "fp32", pairing)
    s, c = orc.round_rne(s, dtype), orc.round_rne(c, dtype)
    dout = orc.round_rne(np.random.default_rng(seed).standard_normal(q.shape), dtype)
    ref = orc.rope_attention_bwd(q, k, v, dout, c, s, inp.seq_lens, w.softmax_scale, causal, pairing)
    emu = emulated_backward(q, k, v, dout, c, s, inp.seq_lens, w.softmax_scale, causal, dtype, pairing)
    return ref, emu


@pytest.mark.parametrize("cfg,dtype,causal,pairing", [
    (3, "bf16", True, "half"), (3, "f16", True, "half"), (2, "bf16", False, "half"),
    (4, "f16", True, "half"), (5, "bf16", True, "interleaved"),
])
def test_rounding_model_within_half_the_bar(cfg, dtype, causal, pairing):
    ref, emu = _case(cfg, dtype, causal, pairing, 6100 + cfg)
    for name, r, e in zip(("dq", "dk", "dv"), ref, emu):
        ratio = float((np.abs(e - r) / backward_bar(r, dtype)).max())
        print(f"{name}: rounding model error / bar, max over elements: {ratio:.3f}")
        assert ratio <= 0.5, name


def test_rounding_model_within_half_the_bar_at_full_length():
    """One sequence of 4096 tokens, 8 q heads over 2 kv heads (the GQA workload's length)."""
    w = dataclasses.replace(wl.CONFIGS[3], batch=1, hq=8, hkv=2, seed=6300)
    inp = wl.generate(w)
    q, k, v = inp.packed()
    f = orc.inv_freq_per_sequence(w.base, inp.seq_lens, w.head_dim, w.trained_len)
    s, c = orc.rope_tables(inp.pos, f, inp.seq_lens, w.pos_scale)
    s, c = orc.round_rne(s, "bf16"), orc.round_rne(c, "bf16")
    dout = orc.round_rne(np.random.default_rng(6300).standard_normal(q.shape), "bf16")
    ref = orc.rope_attention_bwd(q, k, v, dout, c, s, inp.seq_lens, w.softmax_scale, True)
    emu = emulated_backward(q, k, v, dout, c, s, inp.seq_lens, w.softmax_scale, True, "bf16")
    for name, r, e in zip(("dq", "dk", "dv"), ref, emu):
        ratio = float((np.abs(e - r) / backward_bar(r, "bf16")).max())
        print(f"{name}: rounding model error / bar at S=4096, max over elements: {ratio:.3f}")
        assert ratio <= 0.5, name


def test_bar_rejects_one_wrong_element():
    ref, emu = _case(3, "bf16", True, "half", 6200)
    r = ref[2]
    bad = emu[2].copy()
    i = np.unravel_index(np.argmin(np.abs(r)), r.shape)
    rms = float(np.sqrt(np.mean(r * r)))
    bad[i] = r[i] + 80 * UNIT_ROUNDOFF["bf16"] * rms        # beyond u (8 |r| + 64 rms) at |r| ~ 0
    assert not np.all(np.abs(bad - r) <= backward_bar(r, "bf16"))
