"""CPU-only tests of the C ABI: symbols, struct layout, host validation, host inv_freq.

Every call here is rejected by host validation before any HIP call, or is host-only
(rope_inv_freq, rope_status_str, ...), so nothing touches a GPU.  Device pointers
passed here are dummies that the library never dereferences on these paths.
"""

import ctypes
import math
import os
import re

import numpy as np
import pytest

import oracle as orc
import rope_flashattention_amd as rfa
from rope_flashattention_amd import RopeAttnBwdParams, RopeAttnParams, RopeDecodeParams, RopeKvCacheParams

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rope_fa.h")
FAKE = 0x10000  # 16-byte aligned dummy device address, never dereferenced here

# Dummy device pointers are only ever handed to the library where no GPU exists, so a
# validation slip can never turn into a launch on a real device.
import torch  # noqa: E402
no_gpu_only = pytest.mark.skipif(torch.cuda.device_count() > 0, reason="dummy device pointers: CPU-only test")

ST = {v: k for k, v in rfa.STATUS.items()}


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(rope_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol(ropelib):
    names = declared_functions()
    assert {"rope_tables", "rope_qk", "rope_flash_attn_fwd", "rope_inv_freq",
            "rope_kv_rms_norm_rope_cache", "rope_decode_attn_fwd", "rope_decode_workspace_size",
            "rope_flash_attn_bwd", "rope_flash_attn_bwd_workspace_size", "rope_tables_ex"} <= set(names)
    for n in names:
        assert hasattr(ropelib, n), n


def test_abi_version_and_struct_size(ropelib):
    assert ropelib.rope_abi_version() == 3
    assert ropelib.rope_attn_params_size() == ctypes.sizeof(RopeAttnParams)
    assert ropelib.rope_kv_cache_params_size() == ctypes.sizeof(RopeKvCacheParams)
    assert ropelib.rope_decode_params_size() == ctypes.sizeof(RopeDecodeParams)
    assert ropelib.rope_attn_bwd_params_size() == ctypes.sizeof(RopeAttnBwdParams)
    for s, name in rfa.STATUS.items():
        assert ropelib.rope_status_str(s).decode() == name


# --------------------------------------------------------------------------- rope_inv_freq
@pytest.mark.parametrize("base,D", [(1e4, 64), (1e4, 128), (5e5, 128), (1e6, 128), (1e4, 2048)])
def test_inv_freq_matches_oracle_bitwise(ropelib, base, D):
    got = rfa.inv_freq(base, D)
    want = orc.inv_freq(base, D)
    assert got.dtype == np.float32 and np.array_equal(got[0], want)


def test_inv_freq_ntk_matches_oracle_bitwise(ropelib):
    seq_lens = [512, 4096, 4097, 8192, 6000, 1]
    got = rfa.inv_freq(1e4, 128, seq_lens, trained_len=4096)
    want = orc.inv_freq_per_sequence(1e4, seq_lens, 128, 4096)
    assert np.array_equal(got, want)


def test_inv_freq_errors(ropelib):
    L = ropelib
    out = np.empty(64, dtype=np.float32)
    sl = np.array([10], dtype=np.int32)
    assert L.rope_inv_freq(1e4, 128, None, 1, 0, None) == ST["ROPE_ERR_NULL"]
    assert L.rope_inv_freq(1e4, 128, None, 1, 100, out.ctypes.data) == ST["ROPE_ERR_NULL"]
    assert L.rope_inv_freq(-1.0, 128, None, 1, 0, out.ctypes.data) == ST["ROPE_ERR_SHAPE"]
    assert L.rope_inv_freq(float("inf"), 128, None, 1, 0, out.ctypes.data) == ST["ROPE_ERR_SHAPE"]
    assert L.rope_inv_freq(1e4, 127, None, 1, 0, out.ctypes.data) == ST["ROPE_ERR_SHAPE"]
    assert L.rope_inv_freq(1e4, 4096, None, 1, 0, out.ctypes.data) == ST["ROPE_ERR_LIMIT"]
    assert L.rope_inv_freq(1e4, 128, None, 17, 0, out.ctypes.data) == ST["ROPE_ERR_LIMIT"]
    bad = np.array([0], dtype=np.int32)
    assert L.rope_inv_freq(1e4, 128, bad.ctypes.data, 1, 100, out.ctypes.data) == ST["ROPE_ERR_SHAPE"]
    assert L.rope_inv_freq(1e4, 128, sl.ctypes.data, 1, 100, out.ctypes.data) == 0


# --------------------------------------------------------------------------- rope_tables validation
def call_tables(L, pos=FAKE, f=FAKE, seq_lens=(4, 4), batch=None, ntokens=8, head_size=128, scale=1.0,
                dt=2, so=FAKE, co=FAKE):
    sl = np.asarray(seq_lens if seq_lens is not None else (4, 4), dtype=np.int32)
    batch = sl.size if batch is None else batch
    return L.rope_tables(pos, f, sl.ctypes.data if seq_lens is not None else None, batch, ntokens, head_size,
                         scale, dt, so, co, None)


@no_gpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(pos=None), "ROPE_ERR_NULL"),
    (dict(f=None), "ROPE_ERR_NULL"),
    (dict(seq_lens=None), "ROPE_ERR_NULL"),
    (dict(so=None), "ROPE_ERR_NULL"),
    (dict(co=None), "ROPE_ERR_NULL"),
    (dict(dt=0), "ROPE_ERR_DTYPE"),                      # UNDEFINED is unusable
    (dict(dt=9), "ROPE_ERR_DTYPE"),
    (dict(head_size=100), "ROPE_ERR_LIMIT"),             # not a multiple of 32
    (dict(head_size=2080), "ROPE_ERR_LIMIT"),            # > 2048
    (dict(head_size=0), "ROPE_ERR_SHAPE"),
    (dict(seq_lens=[1] * 17, ntokens=17), "ROPE_ERR_LIMIT"),    # batch > 16
    (dict(seq_lens=[128000, 128001], ntokens=256001), "ROPE_ERR_LIMIT"),
    (dict(ntokens=9), "ROPE_ERR_SHAPE"),                 # sum(seq_lens) != ntokens
    (dict(seq_lens=[8, 0], ntokens=8), "ROPE_ERR_SHAPE"),
    (dict(seq_lens=[9, -1], ntokens=8), "ROPE_ERR_SHAPE"),
    (dict(batch=0), "ROPE_ERR_SHAPE"),
    (dict(scale=0.0), "ROPE_ERR_SHAPE"),
    (dict(scale=float("nan")), "ROPE_ERR_SHAPE"),
    (dict(so=FAKE + 8), "ROPE_ERR_UNSUPPORTED"),         # misaligned output
    (dict(f=FAKE + 4), "ROPE_ERR_UNSUPPORTED"),
    (dict(pos=FAKE + 2), "ROPE_ERR_UNSUPPORTED"),
])
def test_rope_tables_rejects(ropelib, kw, status):
    assert call_tables(ropelib, **kw) == ST[status]


# --------------------------------------------------------------------------- rope_qk / attention validation
def valid_params(attention=True, dtype=2, D=128, hq=8, hkv=2, B=2, S=100):
    p = RopeAttnParams()
    p.struct_size = ctypes.sizeof(RopeAttnParams)
    p.dtype = dtype
    p.q = p.k = p.v = p.out = p.out_q = p.out_k = FAKE
    p.batch, p.hq, p.hkv, p.head_dim, p.seqlen, p.ntokens = B, hq, hkv, D, S, B * S
    p.causal = 1
    for name, H in (("q_stride", hq), ("k_stride", hkv), ("v_stride", hkv), ("o_stride", hq)):
        getattr(p, name)[:] = (H * S * D, D, S * D, 1)   # BNSD
    p.cos = p.sin = FAKE
    p.table_dtype = dtype
    p.softmax_scale = 1.0 / math.sqrt(D)
    return p


def mutate(p, **kw):
    for k, v in kw.items():
        if k.endswith("_stride"):
            getattr(p, k)[:] = v
        elif k == "rsv":
            p.rsv[3] = v
        else:
            setattr(p, k, v)
    return p


BAD_COMMON = [
    (dict(struct_size=8), "ROPE_ERR_ABI"),
    (dict(rsv=1), "ROPE_ERR_ABI"),
    (dict(dtype=0), "ROPE_ERR_DTYPE"),
    (dict(dtype=7), "ROPE_ERR_DTYPE"),
    (dict(q=None), "ROPE_ERR_NULL"),
    (dict(k=None), "ROPE_ERR_NULL"),
    (dict(sin=None), "ROPE_ERR_NULL"),
    (dict(hq=6, hkv=4), "ROPE_ERR_SHAPE"),          # hq % hkv != 0
    (dict(hq=0), "ROPE_ERR_SHAPE"),
    (dict(batch=0), "ROPE_ERR_SHAPE"),
    (dict(seqlen=0), "ROPE_ERR_SHAPE"),
    (dict(ntokens=7), "ROPE_ERR_SHAPE"),
    (dict(table_seq_rows=50), "ROPE_ERR_SHAPE"),    # fewer rows than seqlen
    (dict(table_dtype=1), "ROPE_ERR_DTYPE"),        # table dtype differs from q
    (dict(q_stride=(8 * 100 * 128, 128, 100 * 128, 2)), "ROPE_ERR_UNSUPPORTED"),   # head_dim stride != 1
    (dict(k_stride=(2 * 100 * 128, 131, 100 * 128, 1)), "ROPE_ERR_UNSUPPORTED"),   # 16-byte rows
    (dict(q=FAKE + 2), "ROPE_ERR_UNSUPPORTED"),
    (dict(cos=FAKE + 4), "ROPE_ERR_UNSUPPORTED"),
]


@no_gpu_only
@pytest.mark.parametrize("kw,status", BAD_COMMON + [
    (dict(v=None), "ROPE_ERR_NULL"),
    (dict(out=None), "ROPE_ERR_NULL"),
    (dict(head_dim=96), "ROPE_ERR_UNSUPPORTED"),    # attention serves 64 and 128 only
    (dict(head_dim=256), "ROPE_ERR_UNSUPPORTED"),
    (dict(causal=2), "ROPE_ERR_SHAPE"),
    (dict(softmax_scale=0.0), "ROPE_ERR_SHAPE"),
    (dict(softmax_scale=float("inf")), "ROPE_ERR_SHAPE"),
    (dict(o_stride=(8 * 100 * 128, 128, 100 * 128, 3)), "ROPE_ERR_UNSUPPORTED"),
    # key tiles are addressed with 32-bit per-lane offsets: token strides below 2^26 bytes
    (dict(k_stride=(0, 1 << 25, 128, 1)), "ROPE_ERR_LIMIT"),
    (dict(v_stride=(0, 1 << 25, 128, 1)), "ROPE_ERR_LIMIT"),
    (dict(out=FAKE + 8), "ROPE_ERR_UNSUPPORTED"),
    (dict(lse=FAKE + 2), "ROPE_ERR_UNSUPPORTED"),
    (dict(cu_seqlens=FAKE, max_seqlen=0), "ROPE_ERR_SHAPE"),
    (dict(cu_seqlens=FAKE, max_seqlen=300, ntokens=200), "ROPE_ERR_SHAPE"),
])
def test_rope_flash_attn_fwd_rejects(ropelib, kw, status):
    p = mutate(valid_params(), **kw)
    assert ropelib.rope_flash_attn_fwd(ctypes.byref(p), None) == ST[status]


def fwd_ws_size(ropelib, p):
    return ropelib.rope_flash_attn_fwd_workspace_size(ctypes.byref(p))


def test_fwd_workspace_size(ropelib):
    """k' pre-pass plan: a workspace of rows x hkv x head_dim 16-bit values (256-byte multiple)
    once a key would be rotated by at least 8 (query tile, head group) workgroups in-loop."""
    # GQA 8:1 (8 heads per workgroup, 32 query rows): S448 -> 14 query tiles, 7.5 rotations
    assert fwd_ws_size(ropelib, valid_params(hq=16, hkv=2, S=448)) == 0
    # S480 -> 15 query tiles, 8 rotations per key on average (causal)
    assert fwd_ws_size(ropelib, valid_params(hq=16, hkv=2, S=480)) == 2 * 480 * 2 * 128 * 2
    # without the mask every query tile reaches every key: S224 -> 7, S250 -> 8
    assert fwd_ws_size(ropelib, mutate(valid_params(hq=16, hkv=2, S=224), causal=0)) == 0
    assert fwd_ws_size(ropelib, mutate(valid_params(hq=16, hkv=2, S=250), causal=0)) == \
        (2 * 250 * 2 * 128 * 2 + 255) // 256 * 256
    # MHA: one head and 256 query rows per workgroup; S3584 -> 14 tiles, 7.5; S3840 -> 8
    assert fwd_ws_size(ropelib, valid_params(hq=4, hkv=4, S=3584)) == 0
    assert fwd_ws_size(ropelib, valid_params(hq=4, hkv=4, S=3840)) == 2 * 3840 * 4 * 128 * 2
    big = valid_params(hq=64, hkv=8, B=1, S=16384)
    assert fwd_ws_size(ropelib, big) == 16384 * 8 * 128 * 2
    assert fwd_ws_size(ropelib, mutate(valid_params(hq=64, hkv=8, B=1, S=16384), cos=None, sin=None)) == 0
    assert fwd_ws_size(ropelib, mutate(valid_params(hq=64, hkv=8, B=1, S=16384, dtype=3, D=64))) == 0
    assert fwd_ws_size(ropelib, mutate(valid_params(hq=64, hkv=8, B=1, S=16384), hq=6)) == 0   # invalid
    # formed tables: pre-pass too, except varlen with per-sequence inverse frequencies
    gen = mutate(valid_params(hq=64, hkv=8, B=1, S=16384), cos=None, sin=None, pos=FAKE, inv_freq=FAKE,
                 inv_freq_rows=1, pos_scale=1.0)
    assert fwd_ws_size(ropelib, gen) == 16384 * 8 * 128 * 2
    vl = mutate(valid_params(hq=64, hkv=8, B=2, S=0), seqlen=0, cu_seqlens=FAKE, max_seqlen=8000, ntokens=16000,
                cos=None, sin=None, pos=FAKE, inv_freq=FAKE, inv_freq_rows=1, pos_scale=1.0)
    for name, H in (("q_stride", 64), ("k_stride", 8), ("v_stride", 8), ("o_stride", 64)):
        getattr(vl, name)[:] = (0, H * 128, 128, 1)   # packed TND
    assert fwd_ws_size(ropelib, vl) == 16000 * 8 * 128 * 2
    vl.inv_freq_rows = 2
    assert fwd_ws_size(ropelib, vl) == 0


@no_gpu_only
@pytest.mark.parametrize("ws,nbytes", [(None, 1 << 30), (FAKE + 128, 1 << 30), (FAKE, 16384 * 8 * 128 * 2 - 1)])
def test_fwd_ws_rejects_workspace(ropelib, ws, nbytes):
    p = valid_params(hq=64, hkv=8, B=1, S=16384)
    assert ropelib.rope_flash_attn_fwd_ws(ctypes.byref(p), ws, nbytes, None) == ST["ROPE_ERR_WORKSPACE"]


@no_gpu_only
@pytest.mark.parametrize("kw,status", BAD_COMMON[:8])
def test_fwd_ws_validates_params_first(ropelib, kw, status):
    p = mutate(valid_params(hq=64, hkv=8, B=1, S=16384), **kw)
    assert ropelib.rope_flash_attn_fwd_ws(ctypes.byref(p), None, 0, None) == ST[status]


@no_gpu_only
def test_fp32_attention_head_dim(ropelib):
    p = valid_params(dtype=3, D=128)
    assert ropelib.rope_flash_attn_fwd(ctypes.byref(p), None) == ST["ROPE_ERR_UNSUPPORTED"]


@no_gpu_only
@pytest.mark.parametrize("kw,status", BAD_COMMON + [
    (dict(out_q=None), "ROPE_ERR_NULL"),
    (dict(out_k=None), "ROPE_ERR_NULL"),
    (dict(cos=None, sin=None), "ROPE_ERR_NULL"),    # the Rope op needs its tables
    (dict(head_dim=48), "ROPE_ERR_UNSUPPORTED"),
    (dict(head_dim=4096), "ROPE_ERR_LIMIT"),
    (dict(out_k=FAKE + 8), "ROPE_ERR_UNSUPPORTED"),
])
def test_rope_qk_rejects(ropelib, kw, status):
    p = mutate(valid_params(attention=False), **kw)
    assert ropelib.rope_qk(ctypes.byref(p), None) == ST[status]


@no_gpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(pairing=2), "ROPE_ERR_UNSUPPORTED"),
    (dict(cos=None, sin=None, pos=FAKE), "ROPE_ERR_NULL"),                       # formed tables need inv_freq
    (dict(cos=None, sin=None, pos=FAKE, inv_freq=FAKE, inv_freq_rows=1, pos_scale=0.0), "ROPE_ERR_SHAPE"),
    (dict(cos=None, sin=None, pos=FAKE, inv_freq=FAKE, inv_freq_rows=3, pos_scale=1.0), "ROPE_ERR_SHAPE"),
    (dict(cos=None, sin=None, pos=FAKE + 2, inv_freq=FAKE, inv_freq_rows=1, pos_scale=1.0), "ROPE_ERR_UNSUPPORTED"),
    (dict(cos=None, sin=None, pos=FAKE, inv_freq=FAKE + 2, inv_freq_rows=1, pos_scale=1.0),
     "ROPE_ERR_UNSUPPORTED"),
])
def test_formed_tables_and_pairing_rejects(ropelib, kw, status):
    for attention in (True, False):
        p = mutate(valid_params(attention=attention), **kw)
        fn = ropelib.rope_flash_attn_fwd if attention else ropelib.rope_qk
        assert fn(ctypes.byref(p), None) == ST[status]


@no_gpu_only
def test_rope_qk_varlen_per_sequence_freqs_limit(ropelib):
    # rope_qk finds a packed token's sequence among at most ROPE_MAX_BATCH entries
    p = mutate(valid_params(attention=False, B=17), cos=None, sin=None, pos=FAKE, inv_freq=FAKE, inv_freq_rows=17,
               pos_scale=1.0, cu_seqlens=FAKE, max_seqlen=100, ntokens=1700)
    p.q_stride[:] = p.k_stride[:] = (0, 8 * 128, 128, 1)
    assert ropelib.rope_qk(ctypes.byref(p), None) == ST["ROPE_ERR_LIMIT"]


@no_gpu_only
def test_tables_ex_rejects(ropelib):
    lens = np.array([4, 4], dtype=np.int32)
    def call(pairing, mode):
        return ropelib.rope_tables_ex(FAKE, FAKE, lens.ctypes.data, 2, 8, 128, 1.0, 2, pairing, mode, FAKE, FAKE,
                                      None)
    assert call(2, 0) == ST["ROPE_ERR_UNSUPPORTED"]
    assert call(0, 2) == ST["ROPE_ERR_UNSUPPORTED"]
    assert call(-1, 0) == ST["ROPE_ERR_UNSUPPORTED"]
    # the other checks are rope_tables' own
    assert ropelib.rope_tables_ex(FAKE, FAKE, lens.ctypes.data, 2, 9, 128, 1.0, 2, 1, 1, FAKE, FAKE, None) == \
        ST["ROPE_ERR_SHAPE"]


@no_gpu_only
def test_cache_and_decode_pairing_rejects(ropelib):
    p = mutate(valid_cache_params(), pairing=2)
    assert ropelib.rope_kv_rms_norm_rope_cache(ctypes.byref(p), None) == ST["ROPE_ERR_UNSUPPORTED"]
    p = mutate(valid_decode_params(), pairing=5)
    assert ropelib.rope_decode_attn_fwd(ctypes.byref(p), None) == ST["ROPE_ERR_UNSUPPORTED"]


# --------------------------------------------------------------------------- backward validation
def valid_bwd_params(**fwd_kw):
    p = RopeAttnBwdParams()
    p.struct_size = ctypes.sizeof(RopeAttnBwdParams)
    p.fwd = valid_params(**fwd_kw)
    p.fwd.lse = FAKE
    p.dout = p.dq = p.dk = p.dv = FAKE
    p.do_stride[:] = p.dq_stride[:] = tuple(p.fwd.q_stride)
    p.dk_stride[:] = p.dv_stride[:] = tuple(p.fwd.k_stride)
    p.workspace = 0x100000
    p.workspace_bytes = 1 << 30
    return p


def test_bwd_workspace_size(ropelib):
    p = valid_bwd_params()
    # B2 x S100 rows: delta (one float per row and q head), then q' (8 heads) and k' (2 kv
    # heads) in the dtype (2 bytes), each region on a 256-byte boundary
    rows = 2 * 100
    delta = (rows * 8 * 4 + 255) // 256 * 256
    assert ropelib.rope_flash_attn_bwd_workspace_size(ctypes.byref(p)) == delta + rows * 8 * 128 * 2 + rows * 2 * 128 * 2
    p.fwd.lse = None
    assert ropelib.rope_flash_attn_bwd_workspace_size(ctypes.byref(p)) == 0


@no_gpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), "ROPE_ERR_ABI"),
    (dict(rsv=1), "ROPE_ERR_ABI"),
    (dict(dout=None), "ROPE_ERR_NULL"),
    (dict(dq=None), "ROPE_ERR_NULL"),
    (dict(dk=None), "ROPE_ERR_NULL"),
    (dict(dv=None), "ROPE_ERR_NULL"),
    (dict(dk=FAKE + 8), "ROPE_ERR_UNSUPPORTED"),
    (dict(dq_stride=(8 * 100 * 128, 128, 100 * 128, 2)), "ROPE_ERR_UNSUPPORTED"),
    (dict(workspace=None), "ROPE_ERR_WORKSPACE"),
    (dict(workspace=0x100000 + 64), "ROPE_ERR_WORKSPACE"),
    (dict(workspace_bytes=100), "ROPE_ERR_WORKSPACE"),
])
def test_bwd_rejects(ropelib, kw, status):
    p = mutate(valid_bwd_params(), **kw)
    assert ropelib.rope_flash_attn_bwd(ctypes.byref(p), None) == ST[status]


@no_gpu_only
def test_bwd_rejects_forward_fields(ropelib):
    p = valid_bwd_params()
    p.fwd.lse = None
    assert ropelib.rope_flash_attn_bwd(ctypes.byref(p), None) == ST["ROPE_ERR_NULL"]
    p = valid_bwd_params(dtype=3, D=64)
    assert ropelib.rope_flash_attn_bwd(ctypes.byref(p), None) == ST["ROPE_ERR_UNSUPPORTED"]
    p = valid_bwd_params()
    p.fwd.cos = p.fwd.sin = None
    p.fwd.pos, p.fwd.inv_freq, p.fwd.inv_freq_rows, p.fwd.pos_scale = FAKE, FAKE, 1, 1.0
    assert ropelib.rope_flash_attn_bwd(ctypes.byref(p), None) == ST["ROPE_ERR_UNSUPPORTED"]
    p = valid_bwd_params()
    p.fwd.struct_size = 4
    assert ropelib.rope_flash_attn_bwd(ctypes.byref(p), None) == ST["ROPE_ERR_ABI"]
    p = valid_bwd_params(D=96)
    assert ropelib.rope_flash_attn_bwd(ctypes.byref(p), None) == ST["ROPE_ERR_UNSUPPORTED"]
    p = valid_bwd_params()
    p.fwd.v_stride[1] = 1 << 25  # a V token stride of 2^26 bytes (bf16)
    assert ropelib.rope_flash_attn_bwd(ctypes.byref(p), None) == ST["ROPE_ERR_LIMIT"]
    assert ropelib.rope_flash_attn_bwd(None, None) == ST["ROPE_ERR_NULL"]


@no_gpu_only
def test_null_params(ropelib):
    assert ropelib.rope_qk(None, None) == ST["ROPE_ERR_NULL"]
    assert ropelib.rope_flash_attn_fwd(None, None) == ST["ROPE_ERR_NULL"]


# --------------------------------------------------------------------------- KV-cache step validation
def valid_cache_params(dtype=2, D=128, H=8, T=16, blocks=4, bs=64):
    p = RopeKvCacheParams()
    p.struct_size = ctypes.sizeof(RopeKvCacheParams)
    p.dtype = dtype
    p.k = p.v = p.gamma = p.cos = p.sin = p.slots = p.k_cache = p.v_cache = FAKE
    p.ntokens, p.hkv, p.head_dim, p.block_size, p.num_blocks = T, H, D, bs, blocks
    p.eps = 1e-6
    p.k_stride[:] = p.v_stride[:] = (H * D, D)
    p.kc_stride[:] = p.vc_stride[:] = (bs * H * D, H * D, D)
    return p


@no_gpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), "ROPE_ERR_ABI"),
    (dict(rsv=1), "ROPE_ERR_ABI"),
    (dict(dtype=0), "ROPE_ERR_DTYPE"),
    (dict(k=None), "ROPE_ERR_NULL"),
    (dict(cos=None), "ROPE_ERR_NULL"),
    (dict(slots=None), "ROPE_ERR_NULL"),
    (dict(k_cache=None), "ROPE_ERR_NULL"),
    (dict(v=None), "ROPE_ERR_NULL"),                 # v without v_cache
    (dict(v_cache=None), "ROPE_ERR_NULL"),
    (dict(ntokens=-1), "ROPE_ERR_SHAPE"),
    (dict(hkv=0), "ROPE_ERR_SHAPE"),
    (dict(block_size=0), "ROPE_ERR_SHAPE"),
    (dict(num_blocks=0), "ROPE_ERR_SHAPE"),
    (dict(eps=-1e-6), "ROPE_ERR_SHAPE"),
    (dict(eps=float("nan")), "ROPE_ERR_SHAPE"),
    (dict(head_dim=48), "ROPE_ERR_UNSUPPORTED"),
    (dict(head_dim=4096), "ROPE_ERR_LIMIT"),
    (dict(ntokens=2**28, hkv=16), "ROPE_ERR_LIMIT"),
    (dict(k_stride=(8 * 128, 127)), "ROPE_ERR_UNSUPPORTED"),
    (dict(kc_stride=(64 * 8 * 128, 8 * 128, -128)), "ROPE_ERR_SHAPE"),
    (dict(vc_stride=(64 * 8 * 128, 8 * 128 + 4, 128)), "ROPE_ERR_UNSUPPORTED"),
    (dict(k=FAKE + 8), "ROPE_ERR_UNSUPPORTED"),
    (dict(gamma=FAKE + 4), "ROPE_ERR_UNSUPPORTED"),
    (dict(slots=FAKE + 4), "ROPE_ERR_UNSUPPORTED"),
    (dict(v_cache=FAKE + 2), "ROPE_ERR_UNSUPPORTED"),
])
def test_kv_cache_rejects(ropelib, kw, status):
    p = mutate(valid_cache_params(), **kw)
    assert ropelib.rope_kv_rms_norm_rope_cache(ctypes.byref(p), None) == ST[status]


@no_gpu_only
def test_kv_cache_empty_and_null(ropelib):
    assert ropelib.rope_kv_rms_norm_rope_cache(None, None) == ST["ROPE_ERR_NULL"]
    # no new tokens: accepted, nothing enqueued
    assert ropelib.rope_kv_rms_norm_rope_cache(ctypes.byref(valid_cache_params(T=0)), None) == 0
    # K only (v and v_cache both NULL) passes validation too: checked here with no tokens
    p = mutate(valid_cache_params(T=0), v=None, v_cache=None)
    assert ropelib.rope_kv_rms_norm_rope_cache(ctypes.byref(p), None) == 0
    # with no tokens the token arrays may be NULL (empty allocations); the cache may not
    p = mutate(valid_cache_params(T=0), k=None, v=None, cos=None, sin=None, slots=None)
    assert ropelib.rope_kv_rms_norm_rope_cache(ctypes.byref(p), None) == 0
    p = mutate(valid_cache_params(T=0), k_cache=None)
    assert ropelib.rope_kv_rms_norm_rope_cache(ctypes.byref(p), None) == ST["ROPE_ERR_NULL"]


# --------------------------------------------------------------------------- decode validation
def valid_decode_params(dtype=2, D=128, B=4, hq=16, hkv=4, bs=16, mb=64, L=1000, ws=None):
    p = RopeDecodeParams()
    p.struct_size = ctypes.sizeof(RopeDecodeParams)
    p.dtype = dtype
    p.q = p.cos = p.sin = p.k_cache = p.v_cache = p.block_table = p.cache_seqlens = p.out = FAKE
    p.batch, p.hq, p.hkv, p.head_dim = B, hq, hkv, D
    p.block_size, p.max_blocks_per_seq, p.num_blocks, p.max_seqlen = bs, mb, B * mb, L
    p.softmax_scale = 1.0 / math.sqrt(D)
    p.q_stride[:] = p.o_stride[:] = (hq * D, D)
    p.kc_stride[:] = p.vc_stride[:] = (bs * hkv * D, hkv * D, D)
    p.workspace = 0x100000
    p.workspace_bytes = ropelib_ws(p) if ws is None else ws
    return p


def ropelib_ws(p):
    return rfa.lib().rope_decode_workspace_size(ctypes.byref(p))


def test_decode_workspace_size(ropelib):
    p = valid_decode_params()
    need = ropelib.rope_decode_workspace_size(ctypes.byref(p))
    # partial O (head_dim floats) plus m and l per (sequence, q head, split)
    assert need > 0 and need % (4 * 16 * (128 + 2)) == 0
    splits = need // (4 * 16 * (128 + 2))
    assert 1 <= splits <= 256
    p.num_splits = 5
    assert ropelib.rope_decode_workspace_size(ctypes.byref(p)) == 4 * 16 * 5 * 130 * 4
    p.num_splits = 300
    assert ropelib.rope_decode_workspace_size(ctypes.byref(p)) == 0
    assert ropelib.rope_decode_workspace_size(None) == 0
    # the automatic split never gives a split fewer than 128 keys
    p = valid_decode_params(B=1, hq=8, hkv=8, L=300)
    assert ropelib.rope_decode_workspace_size(ctypes.byref(p)) == 8 * 3 * 130 * 4


@no_gpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), "ROPE_ERR_ABI"),
    (dict(rsv=1), "ROPE_ERR_ABI"),
    (dict(dtype=0), "ROPE_ERR_DTYPE"),
    (dict(dtype=3), "ROPE_ERR_UNSUPPORTED"),          # no float32 decode kernel
    (dict(q=None), "ROPE_ERR_NULL"),
    (dict(k_cache=None), "ROPE_ERR_NULL"),
    (dict(cache_seqlens=None), "ROPE_ERR_NULL"),
    (dict(out=None), "ROPE_ERR_NULL"),
    (dict(sin=None), "ROPE_ERR_NULL"),
    (dict(hq=6), "ROPE_ERR_SHAPE"),
    (dict(batch=0), "ROPE_ERR_SHAPE"),
    (dict(block_size=0), "ROPE_ERR_SHAPE"),
    (dict(max_seqlen=0), "ROPE_ERR_SHAPE"),
    (dict(max_seqlen=64 * 16 + 1), "ROPE_ERR_SHAPE"),  # beyond the block table's reach
    (dict(num_splits=-1), "ROPE_ERR_SHAPE"),
    (dict(num_splits=257), "ROPE_ERR_LIMIT"),
    (dict(softmax_scale=0.0), "ROPE_ERR_SHAPE"),
    (dict(head_dim=96), "ROPE_ERR_UNSUPPORTED"),
    (dict(q_stride=(16 * 128, 130)), "ROPE_ERR_UNSUPPORTED"),
    (dict(kc_stride=(16 * 4 * 128, -4 * 128, 128)), "ROPE_ERR_SHAPE"),
    (dict(out=FAKE + 8), "ROPE_ERR_UNSUPPORTED"),
    (dict(block_table=FAKE + 2), "ROPE_ERR_UNSUPPORTED"),
    (dict(workspace=None), "ROPE_ERR_WORKSPACE"),
    (dict(workspace=0x100000 + 128), "ROPE_ERR_WORKSPACE"),
    (dict(workspace_bytes=1024), "ROPE_ERR_WORKSPACE"),
])
def test_decode_rejects(ropelib, kw, status):
    p = mutate(valid_decode_params(), **kw)
    assert ropelib.rope_decode_attn_fwd(ctypes.byref(p), None) == ST[status]


@no_gpu_only
@pytest.mark.parametrize("kw,status", [
    (dict(struct_size=8), "ROPE_ERR_ABI"),
    (dict(dtype=0), "ROPE_ERR_DTYPE"),
    (dict(q=None), "ROPE_ERR_NULL"),
    (dict(out=None), "ROPE_ERR_NULL"),
    (dict(hq=6), "ROPE_ERR_SHAPE"),
    (dict(head_dim=96), "ROPE_ERR_UNSUPPORTED"),
    (dict(num_splits=257), "ROPE_ERR_LIMIT"),
    # beyond the 16 MiB scratch: 64 x 64 heads x 256 splits x (128 + 2) floats
    (dict(batch=64, hq=64, hkv=8, num_blocks=64 * 64, num_splits=256), "ROPE_ERR_LIMIT"),
])
def test_decode_noalloc_rejects(ropelib, kw, status):
    """The allocation-free decode entry validates like the workspace one (its workspace
    fields are ignored) and rejects a call that needs more than its scratch, all on the host."""
    p = mutate(valid_decode_params(), workspace=None, workspace_bytes=0, **kw)
    assert ropelib.rope_decode_attn_fwd_noalloc(ctypes.byref(p), None) == ST[status]


def test_decode_noalloc_scratch_limit_is_16_mib():
    text = open(HEADER).read()
    assert "#define ROPE_DECODE_NOALLOC_MAX_BYTES ((uint64_t)16 << 20)" in text


def test_binding_refuses_cpu_tensors(ropelib):
    import torch
    q = torch.zeros(1, 4, 8, 64)
    with pytest.raises(ValueError):
        rfa.rope_flash_attn_fwd(q, q, q)


# --------------------------------------------------------------------------- sin/cos constants
def test_sincos_constants_derive_from_pi():
    mpmath = pytest.importorskip("mpmath")
    mpmath.mp.dps = 60
    src = open(os.path.join(ROOT, "rope_flashattention_amd", "csrc", "common.h")).read()

    def const(name):
        m = re.search(r"constexpr float %s = ([-0-9a-fx.p+]+)f;" % name, src)
        return float.fromhex(m.group(1))

    f32 = lambda x: float(np.float32(float(x)))
    hi = f32(mpmath.pi / 2)
    mid = f32(mpmath.pi / 2 - hi)
    lo = f32(mpmath.pi / 2 - hi - mid)
    assert const("kHalfPiHi") == hi
    assert const("kHalfPiMid") == mid
    assert const("kHalfPiLo") == lo
    assert const("kTwoOverPi") == f32(2 / mpmath.pi)
