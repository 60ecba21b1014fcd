"""Python binding of librope_fa.so: fused RoPE + FlashAttention forward on MI355X.

The functions here only marshal torch tensors into the C ABI of ``include/rope_fa.h``
(pointers, sizes, strides, the current HIP stream); every step of the computation runs
in the library's HIP kernels.  There is no fallback: if the library is missing or a
call is rejected, an exception is raised.

Names follow the C ABI: ``inv_freq`` (rope_inv_freq), ``rope_tables``, ``rope_qk``,
``rope_flash_attn_fwd``, ``rope_flash_attn_bwd``, ``rope_kv_rms_norm_rope_cache``,
``rope_decode_attn_fwd``.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np
import torch

__all__ = [
    "RopeError",
    "lib",
    "inv_freq",
    "rope_tables",
    "rope_qk",
    "rope_flash_attn_fwd",
    "flash_attn_fwd_workspace_size",
    "rope_flash_attn_bwd",
    "rope_kv_rms_norm_rope_cache",
    "rope_decode_attn_fwd",
    "decode_workspace_size",
    "RopeAttnParams",
    "RopeKvCacheParams",
    "RopeDecodeParams",
    "RopeAttnBwdParams",
    "STATUS",
    "DTYPE",
    "PAIRING",
    "ANGLE_MODE",
    "LIB_PATH",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "librope_fa.so")

STATUS = {0: "ROPE_OK", 1: "ROPE_ERR_NULL", 2: "ROPE_ERR_SHAPE", 3: "ROPE_ERR_DTYPE", 4: "ROPE_ERR_LIMIT",
          5: "ROPE_ERR_UNSUPPORTED", 6: "ROPE_ERR_ABI", 7: "ROPE_ERR_HIP", 8: "ROPE_ERR_WORKSPACE"}
DTYPE = {None: 0, torch.float16: 1, torch.bfloat16: 2, torch.float32: 3}
PAIRING = {"half": 0, "interleaved": 1}
ANGLE_MODE = {"f32": 0, "exact": 1}
ABI_VERSION = 3


class RopeError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        self.name = STATUS.get(status, f"status {status}")
        super().__init__(f"{func} failed: {self.name}")


class RopeAttnParams(ctypes.Structure):
    """Mirror of ``rope_attn_params`` in include/rope_fa.h (checked against the library's size)."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("out_q", ctypes.c_void_p),
        ("out_k", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("batch", ctypes.c_int32),
        ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("seqlen", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("ntokens", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("cu_seqlens", ctypes.c_void_p),
        ("q_stride", ctypes.c_int64 * 4),
        ("k_stride", ctypes.c_int64 * 4),
        ("v_stride", ctypes.c_int64 * 4),
        ("o_stride", ctypes.c_int64 * 4),
        ("cos", ctypes.c_void_p),
        ("sin", ctypes.c_void_p),
        ("table_dtype", ctypes.c_int),
        ("table_seq_rows", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("pairing", ctypes.c_int),
        ("pos", ctypes.c_void_p),
        ("inv_freq", ctypes.c_void_p),
        ("inv_freq_rows", ctypes.c_int32),
        ("pos_scale", ctypes.c_float),
        ("rsv", ctypes.c_uint8 * 16),
    ]


class RopeAttnBwdParams(ctypes.Structure):
    """Mirror of ``rope_attn_bwd_params`` in include/rope_fa.h (checked against the library's size)."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("fwd", RopeAttnParams),
        ("dout", ctypes.c_void_p),
        ("dq", ctypes.c_void_p),
        ("dk", ctypes.c_void_p),
        ("dv", ctypes.c_void_p),
        ("do_stride", ctypes.c_int64 * 4),
        ("dq_stride", ctypes.c_int64 * 4),
        ("dk_stride", ctypes.c_int64 * 4),
        ("dv_stride", ctypes.c_int64 * 4),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_uint64),
        ("rsv", ctypes.c_uint8 * 16),
    ]


class RopeKvCacheParams(ctypes.Structure):
    """Mirror of ``rope_kv_cache_params`` in include/rope_fa.h (checked against the library's size)."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("gamma", ctypes.c_void_p),
        ("cos", ctypes.c_void_p),
        ("sin", ctypes.c_void_p),
        ("slots", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("ntokens", ctypes.c_int32),
        ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("k_stride", ctypes.c_int64 * 2),
        ("v_stride", ctypes.c_int64 * 2),
        ("kc_stride", ctypes.c_int64 * 3),
        ("vc_stride", ctypes.c_int64 * 3),
        ("pairing", ctypes.c_int),
        ("rsv", ctypes.c_uint8 * 12),
    ]


class RopeDecodeParams(ctypes.Structure):
    """Mirror of ``rope_decode_params`` in include/rope_fa.h (checked against the library's size)."""

    _fields_ = [
        ("struct_size", ctypes.c_uint32),
        ("dtype", ctypes.c_int),
        ("q", ctypes.c_void_p),
        ("cos", ctypes.c_void_p),
        ("sin", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("block_table", ctypes.c_void_p),
        ("cache_seqlens", ctypes.c_void_p),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_uint64),
        ("batch", ctypes.c_int32),
        ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_blocks", ctypes.c_int32),
        ("max_seqlen", ctypes.c_int32),
        ("num_splits", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("q_stride", ctypes.c_int64 * 2),
        ("o_stride", ctypes.c_int64 * 2),
        ("kc_stride", ctypes.c_int64 * 3),
        ("vc_stride", ctypes.c_int64 * 3),
        ("pairing", ctypes.c_int),
        ("rsv", ctypes.c_uint8 * 12),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """Load librope_fa.so once, declare the prototypes, check the ABI."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built (python -m rope_flashattention_amd.build)")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
    L.rope_inv_freq.argtypes = [ctypes.c_double, i32, vp, i32, i32, vp]
    L.rope_inv_freq.restype = st
    L.rope_tables.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_float, ctypes.c_int, vp, vp, vp]
    L.rope_tables.restype = st
    L.rope_tables_ex.argtypes = [vp, vp, vp, i32, i32, i32, ctypes.c_float, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                 vp, vp, vp]
    L.rope_tables_ex.restype = st
    L.rope_qk.argtypes = [ctypes.POINTER(RopeAttnParams), vp]
    L.rope_qk.restype = st
    L.rope_flash_attn_fwd.argtypes = [ctypes.POINTER(RopeAttnParams), vp]
    L.rope_flash_attn_fwd.restype = st
    L.rope_flash_attn_fwd_ws.argtypes = [ctypes.POINTER(RopeAttnParams), vp, ctypes.c_uint64, vp]
    L.rope_flash_attn_fwd_ws.restype = st
    L.rope_flash_attn_fwd_workspace_size.argtypes = [ctypes.POINTER(RopeAttnParams)]
    L.rope_flash_attn_fwd_workspace_size.restype = ctypes.c_uint64
    L.rope_kv_rms_norm_rope_cache.argtypes = [ctypes.POINTER(RopeKvCacheParams), vp]
    L.rope_kv_rms_norm_rope_cache.restype = st
    L.rope_kv_cache_params_size.restype = ctypes.c_uint32
    L.rope_decode_attn_fwd.argtypes = [ctypes.POINTER(RopeDecodeParams), vp]
    L.rope_decode_attn_fwd.restype = st
    L.rope_decode_attn_fwd_noalloc.argtypes = [ctypes.POINTER(RopeDecodeParams), vp]
    L.rope_decode_attn_fwd_noalloc.restype = st
    L.rope_decode_workspace_size.argtypes = [ctypes.POINTER(RopeDecodeParams)]
    L.rope_decode_workspace_size.restype = ctypes.c_uint64
    L.rope_decode_params_size.restype = ctypes.c_uint32
    L.rope_flash_attn_bwd.argtypes = [ctypes.POINTER(RopeAttnBwdParams), vp]
    L.rope_flash_attn_bwd.restype = st
    L.rope_flash_attn_bwd_workspace_size.argtypes = [ctypes.POINTER(RopeAttnBwdParams)]
    L.rope_flash_attn_bwd_workspace_size.restype = ctypes.c_uint64
    L.rope_attn_bwd_params_size.restype = ctypes.c_uint32
    L.rope_status_str.argtypes = [ctypes.c_int]
    L.rope_status_str.restype = ctypes.c_char_p
    L.rope_abi_version.restype = i32
    L.rope_attn_params_size.restype = ctypes.c_uint32
    if L.rope_abi_version() != ABI_VERSION:
        raise RuntimeError("librope_fa ABI version mismatch")
    if L.rope_attn_params_size() != ctypes.sizeof(RopeAttnParams):
        raise RuntimeError("rope_attn_params layout mismatch between binding and library")
    if L.rope_kv_cache_params_size() != ctypes.sizeof(RopeKvCacheParams):
        raise RuntimeError("rope_kv_cache_params layout mismatch between binding and library")
    if L.rope_decode_params_size() != ctypes.sizeof(RopeDecodeParams):
        raise RuntimeError("rope_decode_params layout mismatch between binding and library")
    if L.rope_attn_bwd_params_size() != ctypes.sizeof(RopeAttnBwdParams):
        raise RuntimeError("rope_attn_bwd_params layout mismatch between binding and library")
    _lib = L
    return L


def _check(func: str, status: int):
    if status != 0:
        raise RopeError(func, status)


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")


def _i32_host(seq_lens: Sequence[int]) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(seq_lens, dtype=np.int32))


# --------------------------------------------------------------------------- rope_inv_freq
def inv_freq(base: float, head_size: int, seq_lens: Optional[Sequence[int]] = None,
             trained_len: Optional[int] = None, batch: int = 1) -> np.ndarray:
    """Host inverse frequencies [batch, head_size/2] float32 (rope_inv_freq)."""
    sl = None if seq_lens is None else _i32_host(seq_lens)
    nb = batch if sl is None else int(sl.size)
    out = np.empty((nb, head_size // 2), dtype=np.float32)
    st = lib().rope_inv_freq(float(base), int(head_size), None if sl is None else sl.ctypes.data, nb,
                             int(trained_len or 0), out.ctypes.data)
    _check("rope_inv_freq", st)
    return out


# --------------------------------------------------------------------------- rope_tables
def rope_tables(pos: torch.Tensor, inv_freq_dev: torch.Tensor, seq_lens: Sequence[int], head_size: int,
                pos_scale: float = 1.0, out_dtype=torch.bfloat16, sin_out: Optional[torch.Tensor] = None,
                cos_out: Optional[torch.Tensor] = None, *, pairing: str = "half", angle_mode: str = "f32"):
    """(sin, cos) tables [ntokens, head_size] on the GPU (rope_tables; rope_tables_ex for a
    pairing or angle mode other than the defaults)."""
    _need_cuda(pos, inv_freq_dev, sin_out, cos_out)
    if pos.dtype != torch.int32 or inv_freq_dev.dtype != torch.float32:
        raise ValueError("pos must be int32 and inv_freq float32")
    if not (pos.is_contiguous() and inv_freq_dev.is_contiguous()):
        raise ValueError("pos and inv_freq must be contiguous")
    sl = _i32_host(seq_lens)
    n = pos.numel()
    if inv_freq_dev.numel() != sl.size * (head_size // 2):
        raise ValueError("inv_freq must be [batch, head_size/2]")
    if sin_out is None:
        sin_out = torch.empty((n, head_size), dtype=out_dtype, device=pos.device)
    if cos_out is None:
        cos_out = torch.empty((n, head_size), dtype=out_dtype, device=pos.device)
    for t in (sin_out, cos_out):
        if t.shape != (n, head_size) or not t.is_contiguous() or t.dtype != out_dtype:
            raise ValueError("sin_out/cos_out must be contiguous [ntokens, head_size] of out_dtype")
    if pairing == "half" and angle_mode == "f32":
        st = lib().rope_tables(pos.data_ptr(), inv_freq_dev.data_ptr(), sl.ctypes.data, int(sl.size), n,
                               int(head_size), float(pos_scale), DTYPE.get(out_dtype, -1), sin_out.data_ptr(),
                               cos_out.data_ptr(), _stream(pos))
        _check("rope_tables", st)
    else:
        st = lib().rope_tables_ex(pos.data_ptr(), inv_freq_dev.data_ptr(), sl.ctypes.data, int(sl.size), n,
                                  int(head_size), float(pos_scale), DTYPE.get(out_dtype, -1), PAIRING[pairing],
                                  ANGLE_MODE[angle_mode], sin_out.data_ptr(), cos_out.data_ptr(), _stream(pos))
        _check("rope_tables_ex", st)
    return sin_out, cos_out


# --------------------------------------------------------------------------- shared marshalling
def _strides(t: torch.Tensor, layout: str):
    """{batch, token, head, dim} element strides for a BNSD / BSND / packed TND tensor."""
    if layout == "BNSD":
        return (t.stride(0), t.stride(2), t.stride(1), t.stride(3))
    if layout == "BSND":
        return (t.stride(0), t.stride(1), t.stride(2), t.stride(3))
    if layout == "TND":
        return (0, t.stride(0), t.stride(1), t.stride(2))
    raise ValueError(f"unknown layout {layout}")


def _dims(t: torch.Tensor, layout: str):
    """(batch, seq, heads, head_dim) of a tensor in the given layout (batch=1, seq=T for TND)."""
    if layout == "BNSD":
        return t.shape[0], t.shape[2], t.shape[1], t.shape[3]
    if layout == "BSND":
        return t.shape[0], t.shape[1], t.shape[2], t.shape[3]
    if layout == "TND":
        return 1, t.shape[0], t.shape[1], t.shape[2]
    raise ValueError(f"unknown layout {layout}")


def _gen_tables(p, pos, inv_freq, pos_scale, D):
    """Fill the in-kernel table fields (positions + inverse frequencies)."""
    if pos.dtype != torch.int32 or not pos.is_contiguous():
        raise ValueError("pos must be contiguous int32")
    if inv_freq is None or inv_freq.dtype != torch.float32 or not inv_freq.is_contiguous() \
            or inv_freq.shape[-1] != D // 2:
        raise ValueError("inv_freq must be contiguous float32 [rows, head_dim/2]")
    p.pos, p.inv_freq = pos.data_ptr(), inv_freq.data_ptr()
    p.inv_freq_rows = inv_freq.numel() // (D // 2)
    p.pos_scale = float(pos_scale)


def _params(q, k, layout, cos, sin, cu_seqlens, max_seqlen, table_seq_rows, batch=None):
    if (cu_seqlens is None) != (layout != "TND"):
        raise ValueError("packed TND layout goes with cu_seqlens, dense layouts without")
    p = RopeAttnParams()
    p.struct_size = ctypes.sizeof(RopeAttnParams)
    p.dtype = DTYPE.get(q.dtype, -1)
    p.q, p.k = q.data_ptr(), k.data_ptr()
    B, S, Hq, D = _dims(q, layout)
    Bk, Sk, Hkv, Dk = _dims(k, layout)
    if (Bk, Sk, Dk) != (B, S, D) or k.dtype != q.dtype:
        raise ValueError("q and k must agree in batch, tokens, head_dim and dtype")
    p.hq, p.hkv, p.head_dim = Hq, Hkv, D
    if cu_seqlens is not None:
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous int32")
        if max_seqlen is None:
            raise ValueError("max_seqlen is required with cu_seqlens")
        p.batch = cu_seqlens.numel() - 1
        p.cu_seqlens = cu_seqlens.data_ptr()
        p.max_seqlen = int(max_seqlen)
        p.ntokens = S
        p.seqlen = 0
    else:
        p.batch, p.seqlen, p.ntokens = B, S, B * S
    p.q_stride[:] = _strides(q, layout)
    p.k_stride[:] = _strides(k, layout)
    if cos is not None or sin is not None:
        if cos is None or sin is None:
            raise ValueError("cos and sin go together")
        if not (cos.is_contiguous() and sin.is_contiguous()) or cos.shape != sin.shape or cos.shape[-1] != D:
            raise ValueError("tables must be contiguous [rows, head_dim]")
        p.cos, p.sin = cos.data_ptr(), sin.data_ptr()
        p.table_dtype = DTYPE.get(cos.dtype, -1)
        if sin.dtype != cos.dtype:
            raise ValueError("cos and sin must share a dtype")
        rows_needed = (S if cu_seqlens is not None else
                       (S if table_seq_rows == 0 else B * table_seq_rows))
        if cos.shape[0] < rows_needed:
            raise ValueError(f"tables have {cos.shape[0]} rows, {rows_needed} needed")
    p.table_seq_rows = int(table_seq_rows)
    return p


# --------------------------------------------------------------------------- rope_qk
def rope_qk(q: torch.Tensor, k: torch.Tensor, cos: Optional[torch.Tensor], sin: Optional[torch.Tensor], *,
            layout: str = "BNSD", cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
            table_seq_rows: int = 0, out_q: Optional[torch.Tensor] = None, out_k: Optional[torch.Tensor] = None,
            pairing: str = "half", pos: Optional[torch.Tensor] = None, inv_freq: Optional[torch.Tensor] = None,
            pos_scale: float = 1.0):
    """Rotated (q', k') written to out_q / out_k (new tensors like q / k by default).

    With cos = sin = None and pos / inv_freq given, the kernel forms the table values itself.
    """
    _need_cuda(q, k, cos, sin, cu_seqlens, out_q, out_k, pos, inv_freq)
    p = _params(q, k, layout, cos, sin, cu_seqlens, max_seqlen, table_seq_rows)
    p.pairing = PAIRING[pairing]
    if cos is None and pos is not None:
        _gen_tables(p, pos, inv_freq, pos_scale, p.head_dim)
    out_q = torch.empty_like(q) if out_q is None else out_q
    out_k = torch.empty_like(k) if out_k is None else out_k
    if out_q.shape != q.shape or out_k.shape != k.shape or _strides(out_q, layout) != _strides(q, layout) \
            or _strides(out_k, layout) != _strides(k, layout):
        raise ValueError("out_q/out_k must have the shapes and strides of q/k")
    p.out_q, p.out_k = out_q.data_ptr(), out_k.data_ptr()
    _check("rope_qk", lib().rope_qk(ctypes.byref(p), _stream(q)))
    return out_q, out_k


# --------------------------------------------------------------------------- rope_flash_attn_fwd
def rope_flash_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cos: Optional[torch.Tensor] = None,
                        sin: Optional[torch.Tensor] = None, *, causal: bool = True,
                        softmax_scale: Optional[float] = None, layout: str = "BNSD",
                        cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                        table_seq_rows: int = 0, return_lse: bool = False, out: Optional[torch.Tensor] = None,
                        pairing: str = "half", pos: Optional[torch.Tensor] = None,
                        inv_freq: Optional[torch.Tensor] = None, pos_scale: float = 1.0,
                        workspace="auto"):
    """Attention output (and lse [hq, ntokens] float32 if asked).

    cos = sin = None: no rotation, unless pos / inv_freq are given, in which case the kernel
    forms the table values itself.  workspace: "auto" calls rope_flash_attn_fwd_ws with a
    workspace of the size the library asks for (none when it rotates K in-loop), a uint8
    device tensor calls it with that buffer, None calls rope_flash_attn_fwd (K rotated in
    every workgroup that stages it).  All three give the same bits.
    """
    _need_cuda(q, k, v, cos, sin, cu_seqlens, out, pos, inv_freq)
    p = _params(q, k, layout, cos, sin, cu_seqlens, max_seqlen, table_seq_rows)
    p.pairing = PAIRING[pairing]
    if cos is None and pos is not None:
        _gen_tables(p, pos, inv_freq, pos_scale, p.head_dim)
    if v.shape != k.shape or v.dtype != q.dtype:
        raise ValueError("v must match k")
    out = torch.empty_like(q) if out is None else out
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q")
    p.v, p.out = v.data_ptr(), out.data_ptr()
    p.v_stride[:] = _strides(v, layout)
    p.o_stride[:] = _strides(out, layout)
    p.causal = 1 if causal else 0
    p.softmax_scale = float(softmax_scale if softmax_scale is not None else 1.0 / q.shape[-1] ** 0.5)
    lse = None
    if return_lse:
        lse = torch.empty((p.hq, p.ntokens), dtype=torch.float32, device=q.device)
        p.lse = lse.data_ptr()
    if workspace is None:
        _check("rope_flash_attn_fwd", lib().rope_flash_attn_fwd(ctypes.byref(p), _stream(q)))
        return (out, lse) if return_lse else out
    if isinstance(workspace, str):
        if workspace != "auto":
            raise ValueError("workspace must be 'auto', a device tensor or None")
        need = int(lib().rope_flash_attn_fwd_workspace_size(ctypes.byref(p)))
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device) if need else None
    elif workspace.device != q.device:
        raise ValueError("workspace must be on q's device")
    ptr = workspace.data_ptr() if workspace is not None else None
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("rope_flash_attn_fwd_ws", lib().rope_flash_attn_fwd_ws(ctypes.byref(p), ptr, nbytes, _stream(q)))
    return (out, lse) if return_lse else out


def flash_attn_fwd_workspace_size(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                                  cos: Optional[torch.Tensor] = None, sin: Optional[torch.Tensor] = None, *,
                                  causal: bool = True, layout: str = "BNSD", cu_seqlens: Optional[torch.Tensor] = None,
                                  max_seqlen: Optional[int] = None, table_seq_rows: int = 0, pairing: str = "half",
                                  pos: Optional[torch.Tensor] = None, inv_freq: Optional[torch.Tensor] = None,
                                  pos_scale: float = 1.0) -> int:
    """Bytes rope_flash_attn_fwd_ws would use for this call (0: K rotated in-loop)."""
    p = _params(q, k, layout, cos, sin, cu_seqlens, max_seqlen, table_seq_rows)
    p.pairing = PAIRING[pairing]
    if cos is None and pos is not None:
        _gen_tables(p, pos, inv_freq, pos_scale, p.head_dim)
    p.v = v.data_ptr()
    p.out = q.data_ptr()  # a stand-in: the size depends on the shapes only
    p.v_stride[:] = _strides(v, layout)
    p.o_stride[:] = _strides(q, layout)
    p.causal = 1 if causal else 0
    p.softmax_scale = 1.0 / q.shape[-1] ** 0.5
    return int(lib().rope_flash_attn_fwd_workspace_size(ctypes.byref(p)))


# --------------------------------------------------------------------------- rope_flash_attn_bwd
def rope_flash_attn_bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, out: torch.Tensor, lse: torch.Tensor,
                        dout: torch.Tensor, cos: Optional[torch.Tensor] = None, sin: Optional[torch.Tensor] = None, *,
                        causal: bool = True, softmax_scale: Optional[float] = None, layout: str = "BNSD",
                        cu_seqlens: Optional[torch.Tensor] = None, max_seqlen: Optional[int] = None,
                        table_seq_rows: int = 0, pairing: str = "half", dq: Optional[torch.Tensor] = None,
                        dk: Optional[torch.Tensor] = None, dv: Optional[torch.Tensor] = None,
                        workspace: Optional[torch.Tensor] = None):
    """(dq, dk, dv) for the forward call with the same arguments, given its out and lse."""
    _need_cuda(q, k, v, out, lse, dout, cos, sin, cu_seqlens, dq, dk, dv, workspace)
    f = _params(q, k, layout, cos, sin, cu_seqlens, max_seqlen, table_seq_rows)
    f.pairing = PAIRING[pairing]
    if v.shape != k.shape or v.dtype != q.dtype or out.shape != q.shape or dout.shape != q.shape \
            or dout.dtype != q.dtype or out.dtype != q.dtype:
        raise ValueError("v must match k; out and dout must match q")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != f.hq * f.ntokens:
        raise ValueError("lse must be the forward's contiguous float32 [hq, ntokens]")
    f.v, f.out, f.lse = v.data_ptr(), out.data_ptr(), lse.data_ptr()
    f.v_stride[:] = _strides(v, layout)
    f.o_stride[:] = _strides(out, layout)
    f.causal = 1 if causal else 0
    f.softmax_scale = float(softmax_scale if softmax_scale is not None else 1.0 / q.shape[-1] ** 0.5)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for g, x in ((dq, q), (dk, k), (dv, v)):
        if g.shape != x.shape or g.dtype != x.dtype:
            raise ValueError("gradients must match their inputs")
    p = RopeAttnBwdParams()
    p.struct_size = ctypes.sizeof(RopeAttnBwdParams)
    p.fwd = f
    p.dout, p.dq, p.dk, p.dv = dout.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    p.do_stride[:] = _strides(dout, layout)
    p.dq_stride[:] = _strides(dq, layout)
    p.dk_stride[:] = _strides(dk, layout)
    p.dv_stride[:] = _strides(dv, layout)
    need = int(lib().rope_flash_attn_bwd_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    _check("rope_flash_attn_bwd", lib().rope_flash_attn_bwd(ctypes.byref(p), _stream(q)))
    return dq, dk, dv


# --------------------------------------------------------------------------- rope_kv_rms_norm_rope_cache
def _cache_strides(c: torch.Tensor, cache_layout: str):
    """{block, offset in block, head} strides and (num_blocks, block_size, heads, head_dim)."""
    if c.dim() != 4 or c.stride(3) != 1:
        raise ValueError("caches must be 4-D with a unit head_dim stride")
    if cache_layout == "BSND":   # [num_blocks, block_size, hkv, D]
        return (c.stride(0), c.stride(1), c.stride(2)), (c.shape[0], c.shape[1], c.shape[2], c.shape[3])
    if cache_layout == "BNSD":   # [num_blocks, hkv, block_size, D]
        return (c.stride(0), c.stride(2), c.stride(1)), (c.shape[0], c.shape[2], c.shape[1], c.shape[3])
    raise ValueError(f"unknown cache layout {cache_layout}")


def rope_kv_rms_norm_rope_cache(k: torch.Tensor, v: Optional[torch.Tensor], cos: torch.Tensor, sin: torch.Tensor,
                                slots: torch.Tensor, k_cache: torch.Tensor, v_cache: Optional[torch.Tensor], *,
                                gamma: Optional[torch.Tensor] = None, eps: float = 1e-6,
                                cache_layout: str = "BSND", pairing: str = "half"):
    """RMSNorm (if gamma is given) + RoPE of k [T, hkv, D], written with v into the caches at ``slots``.

    Caches are [num_blocks, block_size, hkv, D] ("BSND") or [num_blocks, hkv, block_size, D]
    ("BNSD"); slot s is block s // block_size, offset s % block_size.  Updates the caches in
    place and returns them.
    """
    _need_cuda(k, v, cos, sin, slots, k_cache, v_cache, gamma)
    if (v is None) != (v_cache is None):
        raise ValueError("v and v_cache go together")
    if k.dim() != 3 or k.stride(2) != 1:
        raise ValueError("k must be [ntokens, hkv, head_dim] with a unit head_dim stride")
    T, H, D = k.shape
    kcs, kshape = _cache_strides(k_cache, cache_layout)
    if kshape[2:] != (H, D) or k_cache.dtype != k.dtype:
        raise ValueError("k_cache must hold hkv heads of head_dim and k's dtype")
    p = RopeKvCacheParams()
    p.struct_size = ctypes.sizeof(RopeKvCacheParams)
    p.dtype = DTYPE.get(k.dtype, -1)
    p.pairing = PAIRING[pairing]
    p.k, p.k_cache = k.data_ptr(), k_cache.data_ptr()
    p.k_stride[:] = (k.stride(0), k.stride(1))
    p.kc_stride[:] = kcs
    if v is not None:
        vcs, vshape = _cache_strides(v_cache, cache_layout)
        if v.shape != k.shape or v.stride(2) != 1 or v.dtype != k.dtype or vshape != kshape \
                or v_cache.dtype != k.dtype:
            raise ValueError("v and v_cache must match k and k_cache")
        p.v, p.v_cache = v.data_ptr(), v_cache.data_ptr()
        p.v_stride[:] = (v.stride(0), v.stride(1))
        p.vc_stride[:] = vcs
    for t in (cos, sin):
        if t.dtype != k.dtype or not t.is_contiguous() or t.dim() != 2 or t.shape[1] != D or t.shape[0] < T:
            raise ValueError("tables must be contiguous [>= ntokens, head_dim] of k's dtype")
    p.cos, p.sin = cos.data_ptr(), sin.data_ptr()
    if slots.dtype != torch.int64 or not slots.is_contiguous() or slots.numel() != T:
        raise ValueError("slots must be contiguous int64 [ntokens]")
    p.slots = slots.data_ptr()
    if gamma is not None:
        if gamma.dtype != torch.float32 or not gamma.is_contiguous() or gamma.numel() != D:
            raise ValueError("gamma must be contiguous float32 [head_dim]")
        p.gamma = gamma.data_ptr()
    p.ntokens, p.hkv, p.head_dim = T, H, D
    p.num_blocks, p.block_size = kshape[0], kshape[1]
    p.eps = float(eps)
    _check("rope_kv_rms_norm_rope_cache", lib().rope_kv_rms_norm_rope_cache(ctypes.byref(p), _stream(k)))
    return k_cache, v_cache


# --------------------------------------------------------------------------- rope_decode_attn_fwd
def _decode_params(q, k_cache, v_cache, cache_seqlens, cos, sin, block_table, max_seqlen, softmax_scale,
                   cache_layout, num_splits, pairing="half"):
    if q.dim() != 3 or q.stride(2) != 1:
        raise ValueError("q must be [batch, hq, head_dim] with a unit head_dim stride")
    B, Hq, D = q.shape
    kcs, kshape = _cache_strides(k_cache, cache_layout)
    vcs, vshape = _cache_strides(v_cache, cache_layout)
    if kshape != vshape or kshape[3] != D or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("k_cache and v_cache must match each other, q's head_dim and q's dtype")
    nblk, bs, Hkv = kshape[0], kshape[1], kshape[2]
    p = RopeDecodeParams()
    p.struct_size = ctypes.sizeof(RopeDecodeParams)
    p.dtype = DTYPE.get(q.dtype, -1)
    p.pairing = PAIRING[pairing]
    p.q, p.k_cache, p.v_cache = q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr()
    if cache_seqlens.dtype != torch.int32 or not cache_seqlens.is_contiguous() or cache_seqlens.numel() != B:
        raise ValueError("cache_seqlens must be contiguous int32 [batch]")
    p.cache_seqlens = cache_seqlens.data_ptr()
    if block_table is not None:
        if block_table.dtype != torch.int32 or not block_table.is_contiguous() or block_table.dim() != 2 \
                or block_table.shape[0] != B:
            raise ValueError("block_table must be contiguous int32 [batch, max_blocks_per_seq]")
        p.block_table = block_table.data_ptr()
        p.max_blocks_per_seq = block_table.shape[1]
    else:
        p.max_blocks_per_seq = nblk // B
    if cos is not None or sin is not None:
        for t in (cos, sin):
            if t is None or t.dtype != q.dtype or not t.is_contiguous() or tuple(t.shape) != (B, D):
                raise ValueError("cos and sin go together, contiguous [batch, head_dim] of q's dtype")
        p.cos, p.sin = cos.data_ptr(), sin.data_ptr()
    p.batch, p.hq, p.hkv, p.head_dim = B, Hq, Hkv, D
    p.block_size, p.num_blocks = bs, nblk
    p.max_seqlen = int(max_seqlen)
    p.num_splits = int(num_splits)
    p.softmax_scale = float(softmax_scale if softmax_scale is not None else 1.0 / D ** 0.5)
    p.q_stride[:] = (q.stride(0), q.stride(1))
    p.kc_stride[:] = kcs
    p.vc_stride[:] = vcs
    return p


def decode_workspace_size(q, k_cache, v_cache, cache_seqlens, *, max_seqlen: int, block_table=None,
                          cache_layout: str = "BSND", num_splits: int = 0) -> int:
    """Workspace bytes rope_decode_attn_fwd needs for these shapes (rope_decode_workspace_size)."""
    p = _decode_params(q, k_cache, v_cache, cache_seqlens, None, None, block_table, max_seqlen, None,
                       cache_layout, num_splits)
    return int(lib().rope_decode_workspace_size(ctypes.byref(p)))


def rope_decode_attn_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor, cache_seqlens: torch.Tensor,
                         cos: Optional[torch.Tensor] = None, sin: Optional[torch.Tensor] = None, *,
                         max_seqlen: int, block_table: Optional[torch.Tensor] = None,
                         softmax_scale: Optional[float] = None, cache_layout: str = "BSND", num_splits: int = 0,
                         return_lse: bool = False, out: Optional[torch.Tensor] = None,
                         workspace: Optional[torch.Tensor] = None, pairing: str = "half"):
    """Decode-step attention of q [batch, hq, D] (rotated with cos/sin [batch, D]) over the caches.

    Caches as in ``rope_kv_rms_norm_rope_cache``; block_table int32 [batch, max_blocks] or None
    (sequence b owns blocks b*max_blocks .. , max_blocks = num_blocks // batch).  The workspace
    (a byte tensor) is allocated here when not given.
    """
    _need_cuda(q, k_cache, v_cache, cache_seqlens, cos, sin, block_table, out, workspace)
    p = _decode_params(q, k_cache, v_cache, cache_seqlens, cos, sin, block_table, max_seqlen, softmax_scale,
                       cache_layout, num_splits, pairing)
    need = int(lib().rope_decode_workspace_size(ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    p.workspace, p.workspace_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    out = torch.empty_like(q) if out is None else out
    if out.shape != q.shape or out.dtype != q.dtype or out.stride(2) != 1:
        raise ValueError("out must match q")
    p.out = out.data_ptr()
    p.o_stride[:] = (out.stride(0), out.stride(1))
    lse = None
    if return_lse:
        lse = torch.empty((q.shape[0], q.shape[1]), dtype=torch.float32, device=q.device)
        p.lse = lse.data_ptr()
    _check("rope_decode_attn_fwd", lib().rope_decode_attn_fwd(ctypes.byref(p), _stream(q)))
    return (out, lse) if return_lse else out


def rope_decode_attn_fwd_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                 cache_seqlens: torch.Tensor, cos: Optional[torch.Tensor] = None,
                                 sin: Optional[torch.Tensor] = None, *, max_seqlen: int, out: torch.Tensor,
                                 lse: Optional[torch.Tensor] = None, block_table: Optional[torch.Tensor] = None,
                                 softmax_scale: Optional[float] = None, cache_layout: str = "BSND",
                                 num_splits: int = 0, pairing: str = "half") -> torch.Tensor:
    """rope_decode_attn_fwd through the allocation-free entry point: nothing is allocated,
    here or in the library (the split partials use the library's per-GPU scratch).  The
    caller passes out (like q) and, if wanted, lse (contiguous float32 [batch, hq])."""
    _need_cuda(q, k_cache, v_cache, cache_seqlens, cos, sin, block_table, out, lse)
    p = _decode_params(q, k_cache, v_cache, cache_seqlens, cos, sin, block_table, max_seqlen, softmax_scale,
                       cache_layout, num_splits, pairing)
    if out.shape != q.shape or out.dtype != q.dtype or out.stride(2) != 1:
        raise ValueError("out must match q")
    p.out = out.data_ptr()
    p.o_stride[:] = (out.stride(0), out.stride(1))
    if lse is not None:
        if lse.dtype != torch.float32 or not lse.is_contiguous() or tuple(lse.shape) != tuple(q.shape[:2]):
            raise ValueError("lse must be contiguous float32 [batch, hq]")
        p.lse = lse.data_ptr()
    _check("rope_decode_attn_fwd_noalloc", lib().rope_decode_attn_fwd_noalloc(ctypes.byref(p), _stream(q)))
    return out
