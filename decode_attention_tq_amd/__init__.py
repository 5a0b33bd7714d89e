"""Python binding of libtq (TurboQuant compressed-KV encode and attention on
MI355X / gfx950).

Argument marshalling only: every step of the method runs in the HIP kernels of
``libtq.so`` behind the C ABI declared in ``include/tq.h``.  PyTorch provides
device memory and the current HIP stream.  Importing this package fails
loudly when the library has not been built; there is no CPU fallback.

The functions carry the C names (``tq_codebook_init``, ``tq_encode_kv``,
``tq_decode_attention``, ...).
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libtq.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libtq.so not found at {LIB_PATH}; build it with "
        "`python decode_attention_tq_amd/build_lib.py` (hipcc, gfx950)")

_lib = ctypes.CDLL(LIB_PATH)

TQ_OK = 0
TQ_ERR_INVALID_ARGUMENT = -1
TQ_ERR_UNSUPPORTED = -2
TQ_ERR_WORKSPACE_TOO_SMALL = -3
TQ_ERR_NOT_INITIALIZED = -4
TQ_ERR_HIP = -5
TQ_F32, TQ_F16, TQ_BF16 = 0, 1, 2
HEAD_DIM = 128
QJL_DIM = 128
BLOCK = 16
K_PAGE_BYTES = 1088   # page sizes of 3-bit codes; tq_k_page_bytes / tq_v_page_bytes give any width
V_PAGE_BYTES = 800

EXPORTED = [
    "tq_codebook_compute", "tq_qjl_matrix", "tq_codebook_device_bytes", "tq_codebook_init",
    "tq_k_page_bytes", "tq_v_page_bytes", "tq_encode_kv", "tq_decode_workspace_bytes",
    "tq_decode_attention", "tq_decode_hot_workspace_bytes", "tq_decode_attention_hot",
    "tq_decode_noalloc_scratch_bytes", "tq_decode_attention_noalloc",
    "tq_decode_window_workspace_bytes", "tq_decode_attention_window",
    "tq_decode_step_workspace_bytes", "tq_decode_step", "tq_last_error",
]


class tq_codebook_t(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_int32), ("bits", ctypes.c_int32),
                ("qjl_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("qjl_seed", ctypes.c_uint64), ("centroids", ctypes.c_float * 16),
                ("thresholds", ctypes.c_float * 15), ("qjl_scale", ctypes.c_float),
                ("d_tables", ctypes.c_void_p), ("magic", ctypes.c_uint32),
                ("reserved", ctypes.c_uint32)]


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_CB = ctypes.POINTER(tq_codebook_t)

_lib.tq_last_error.restype = ctypes.c_char_p
_lib.tq_last_error.argtypes = []
_lib.tq_codebook_compute.restype = _I
_lib.tq_codebook_compute.argtypes = [_I, _I, _P, _P]
_lib.tq_qjl_matrix.restype = _I
_lib.tq_qjl_matrix.argtypes = [ctypes.c_uint64, _I, _I, _P]
_lib.tq_codebook_device_bytes.restype = _SZ
_lib.tq_codebook_device_bytes.argtypes = [_I, _I]
_lib.tq_codebook_init.restype = _I
_lib.tq_codebook_init.argtypes = [_CB, _I, _I, ctypes.c_uint64, _P, _P, _P]
_lib.tq_k_page_bytes.restype = _SZ
_lib.tq_k_page_bytes.argtypes = [_CB]
_lib.tq_v_page_bytes.restype = _SZ
_lib.tq_v_page_bytes.argtypes = [_CB]
_lib.tq_encode_kv.restype = _I
_lib.tq_encode_kv.argtypes = [_CB, _P, _P, _I, _I64, _I, _I64, _I64, _P, _P, _P, _P, _P]
_lib.tq_decode_workspace_bytes.restype = _SZ
_lib.tq_decode_workspace_bytes.argtypes = [_CB, _I, _I, _I, _I, _I, _I]
_lib.tq_decode_attention.restype = _I
_lib.tq_decode_attention.argtypes = [_CB, _P, _I, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I,
                                     ctypes.c_float, _P, _I, _I, _P, _SZ, _P]
_lib.tq_decode_noalloc_scratch_bytes.restype = _SZ
_lib.tq_decode_noalloc_scratch_bytes.argtypes = []
_lib.tq_decode_attention_noalloc.restype = _I
_lib.tq_decode_attention_noalloc.argtypes = [_CB, _P, _I, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I,
                                             ctypes.c_float, _P, _I, _I, _P]
_lib.tq_decode_window_workspace_bytes.restype = _SZ
_lib.tq_decode_window_workspace_bytes.argtypes = [_CB, _I, _I, _I, _I, _I, _I, _I]
_lib.tq_decode_attention_window.restype = _I
_lib.tq_decode_attention_window.argtypes = [_CB, _P, _I, _P, _P, _P, _I, _P, _I, _I, _I, _I, _I, _I,
                                            ctypes.c_float, _P, _I, _I, _P, _SZ, _P]
_lib.tq_decode_hot_workspace_bytes.restype = _SZ
_lib.tq_decode_hot_workspace_bytes.argtypes = [_CB, _I, _I, _I, _I, _I, _I]
_lib.tq_decode_attention_hot.restype = _I
_lib.tq_decode_attention_hot.argtypes = [_CB, _P, _I, _P, _P, _P, _I, _P, _I, _I, _I, _I,
                                         _P, _P, _I, _P, _I, ctypes.c_float, _P, _I, _I, _P,
                                         _SZ, _P]


class TQError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"libtq status {status}: {message}")
        self.status = status


def tq_last_error() -> str:
    return _lib.tq_last_error().decode()


def _check(status: int) -> None:
    if status != TQ_OK:
        raise TQError(status, tq_last_error())


def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    m = {torch.float32: TQ_F32, torch.float16: TQ_F16, torch.bfloat16: TQ_BF16}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream, device=None):
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _check_pools(cb, k_cache, v_cache, num_kv_heads: int) -> None:
    """The C ABI takes the pools as bare pointers with no size: their shape is
    checked here, so that a pool built for another head count or page size
    (bit width) is rejected before any kernel reads or writes it."""
    torch = _torch()
    kpage, vpage = int(_lib.tq_k_page_bytes(cb.ref)), int(_lib.tq_v_page_bytes(cb.ref))
    for name, pool, page in (("k_cache", k_cache, kpage), ("v_cache", v_cache, vpage)):
        if not isinstance(pool, torch.Tensor):
            raise TypeError(f"{name} must be a torch tensor")
        if pool.dtype != torch.uint8 or not pool.is_contiguous():
            raise ValueError(f"{name} must be a contiguous uint8 tensor")
        if pool.dim() != 3 or pool.shape[1] != num_kv_heads or pool.shape[2] != page:
            raise ValueError(f"{name} must be [num_blocks][{num_kv_heads}][{page}], got {tuple(pool.shape)}")
    if k_cache.shape[0] != v_cache.shape[0]:
        raise ValueError("k_cache and v_cache must hold the same number of blocks")


def _check_seq_tables(block_tables, context_lens, num_seqs: int) -> None:
    if block_tables.dim() != 2 or block_tables.shape[0] != num_seqs:
        raise ValueError(f"block_tables must be [{num_seqs}][max_blocks]")
    if context_lens.dim() != 1 or context_lens.shape[0] != num_seqs:
        raise ValueError(f"context_lens must have one entry per sequence ({num_seqs})")


# ---- host-only helpers ------------------------------------------------------

def tq_codebook_compute(head_dim: int = HEAD_DIM, bits: int = 3):
    c = np.zeros(1 << bits, dtype=np.float32)
    t = np.zeros((1 << bits) - 1, dtype=np.float32)
    _check(_lib.tq_codebook_compute(head_dim, bits, c.ctypes.data, t.ctypes.data))
    return c, t


def tq_qjl_matrix(seed: int, rows: int = QJL_DIM, cols: int = HEAD_DIM) -> np.ndarray:
    out = np.zeros((rows, cols), dtype=np.float32)
    _check(_lib.tq_qjl_matrix(seed, rows, cols, out.ctypes.data))
    return out


def tq_codebook_device_bytes(head_dim: int = HEAD_DIM, qjl_dim: int = QJL_DIM) -> int:
    return int(_lib.tq_codebook_device_bytes(head_dim, qjl_dim))


# ---- context ------------------------------------------------------------------

class Codebook:
    """Owns the C struct and the device table buffer it points at."""

    def __init__(self, struct: tq_codebook_t, tables):
        self.struct = struct
        self.tables = tables

    @property
    def ref(self):
        return ctypes.byref(self.struct)

    @property
    def bits(self) -> int:
        return int(self.struct.bits)

    @property
    def centroids(self) -> np.ndarray:
        return np.array(self.struct.centroids[:1 << self.bits], dtype=np.float32)

    @property
    def thresholds(self) -> np.ndarray:
        return np.array(self.struct.thresholds[:(1 << self.bits) - 1], dtype=np.float32)


def tq_codebook_init(head_dim: int = HEAD_DIM, bits: int = 3, qjl_seed: int = 42,
                     qjl_host: np.ndarray | None = None, device=None, stream=None) -> Codebook:
    torch = _torch()
    device = torch.device("cuda") if device is None else torch.device(device)
    nbytes = tq_codebook_device_bytes(head_dim, QJL_DIM)
    tables = torch.empty(max(nbytes, 4), dtype=torch.uint8, device=device)
    s = tq_codebook_t()
    host = None
    if qjl_host is not None:
        host = np.ascontiguousarray(qjl_host, dtype=np.float32)
        if host.shape != (QJL_DIM, head_dim):
            raise ValueError(f"qjl_host must be {QJL_DIM}x{head_dim}")
    _check(_lib.tq_codebook_init(ctypes.byref(s), head_dim, bits, qjl_seed,
                                 None if host is None else host.ctypes.data,
                                 tables.data_ptr(), _stream(stream, device)))
    return Codebook(s, tables)


def tq_k_page_bytes(cb: Codebook) -> int:
    return int(_lib.tq_k_page_bytes(cb.ref))


def tq_v_page_bytes(cb: Codebook) -> int:
    return int(_lib.tq_v_page_bytes(cb.ref))

_lib.tq_decode_step_workspace_bytes.restype = _SZ
_lib.tq_decode_step_workspace_bytes.argtypes = [_CB, _I, _I, _I, _I, _I]
_lib.tq_decode_step.restype = _I
_lib.tq_decode_step.argtypes = [_CB, _P, _P, _I, _I64, _I64, _P, _P, _I, _P, _P, _P, _I, _P, _I, _I,
                                _I, _I, ctypes.c_float, _P, _I, _I, _P, _SZ, _P]


# ---- encode -------------------------------------------------------------------

def tq_encode_kv(cb: Codebook, k, v, slot_mapping, k_cache, v_cache, norms_out=None,
                 stream=None) -> None:
    """k, v: [T][Hkv][128] device tensors (last dim contiguous, same strides);
    slot_mapping: int64 [T]; k_cache/v_cache: uint8 pools."""
    torch = _torch()
    if k.shape != v.shape or k.stride() != v.stride() or k.dtype != v.dtype:
        raise ValueError("k and v must share shape, strides and dtype")
    if k.dim() != 3 or k.shape[2] != HEAD_DIM or k.stride(2) != 1:
        raise ValueError("k must be [T][Hkv][128] with a contiguous last dimension")
    if slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous():
        raise ValueError("slot_mapping must be contiguous int64")
    T, H = k.shape[0], k.shape[1]
    if slot_mapping.dim() != 1 or slot_mapping.shape[0] != T:
        raise ValueError(f"slot_mapping must have one entry per token ({T})")
    _check_pools(cb, k_cache, v_cache, H)
    if norms_out is not None and (norms_out.dtype != torch.float32 or not norms_out.is_contiguous()
                                  or tuple(norms_out.shape) != (T, H, 3)):
        raise ValueError(f"norms_out must be a contiguous float32 [{T}][{H}][3] tensor")
    _check(_lib.tq_encode_kv(cb.ref, _ptr(k), _ptr(v), _dtype_code(k), T, H, k.stride(0),
                             k.stride(1), _ptr(slot_mapping), _ptr(k_cache), _ptr(v_cache),
                             _ptr(norms_out), _stream(stream, k.device)))


# ---- attention ------------------------------------------------------------------

def tq_decode_workspace_bytes(cb: Codebook, num_seqs: int, q_len: int, num_q_heads: int,
                              num_kv_heads: int, max_context_len: int,
                              tokens_per_split: int = 0) -> int:
    return int(_lib.tq_decode_workspace_bytes(cb.ref, num_seqs, q_len, num_q_heads,
                                              num_kv_heads, max_context_len, tokens_per_split))


def tq_decode_attention(cb: Codebook, q, k_cache, v_cache, block_tables, context_lens,
                        max_context_len: int, num_kv_heads: int, out=None,
                        softmax_scale: float = 0.0, tokens_per_split: int = 0,
                        workspace=None, out_dtype=None, stream=None):
    """q: [B][q_len][Hq][128]; block_tables int32 [B][max_blocks]; context_lens
    int32 [B].  Returns ``out`` ([B][q_len][Hq][128], fp32 unless given)."""
    torch = _torch()
    if q.dim() != 4 or q.shape[3] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][q_len][Hq][128] tensor")
    if block_tables.dtype != torch.int32 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32")
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32")
    B, q_len, Hq, _ = q.shape
    _check_pools(cb, k_cache, v_cache, num_kv_heads)
    _check_seq_tables(block_tables, context_lens, B)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape:
        raise ValueError("out must be contiguous with q's shape")
    need = tq_decode_workspace_bytes(cb, B, q_len, Hq, num_kv_heads, max_context_len,
                                     tokens_per_split)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    _check(_lib.tq_decode_attention(
        cb.ref, _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), B, q_len, Hq, num_kv_heads,
        max_context_len, float(softmax_scale), _ptr(out), _dtype_code(out), tokens_per_split,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q.device)))
    return out


# ---- one decode step: append, then attend ------------------------------------------

def tq_decode_step_workspace_bytes(cb: Codebook, num_seqs: int, num_q_heads: int, num_kv_heads: int,
                                   max_context_len: int, tokens_per_split: int = 0) -> int:
    return int(_lib.tq_decode_step_workspace_bytes(cb.ref, num_seqs, num_q_heads, num_kv_heads,
                                                   max_context_len, tokens_per_split))


def tq_decode_step(cb: Codebook, k_new, v_new, slot_mapping, q, k_cache, v_cache, block_tables,
                   context_lens, max_context_len: int, out=None, softmax_scale: float = 0.0,
                   tokens_per_split: int = 0, workspace=None, out_dtype=None, stream=None):
    """One new token per sequence: k_new, v_new [B][Hkv][128] (last dim
    contiguous, same strides), slot_mapping int64 [B], q [B][1][Hq][128].
    Appends the new keys and values, then attends; returns ``out``."""
    torch = _torch()
    if k_new.shape != v_new.shape or k_new.stride() != v_new.stride() or k_new.dtype != v_new.dtype:
        raise ValueError("k_new and v_new must share shape, strides and dtype")
    if k_new.dim() != 3 or k_new.shape[2] != HEAD_DIM or k_new.stride(2) != 1:
        raise ValueError("k_new must be [B][Hkv][128] with a contiguous last dimension")
    if q.dim() != 4 or q.shape[1] != 1 or q.shape[3] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][1][Hq][128] tensor")
    B, Hq = q.shape[0], q.shape[2]
    H = k_new.shape[1]
    if k_new.shape[0] != B:
        raise ValueError(f"k_new must hold one token per sequence ({B})")
    if (slot_mapping.dtype != torch.int64 or not slot_mapping.is_contiguous()
            or slot_mapping.dim() != 1 or slot_mapping.shape[0] != B):
        raise ValueError(f"slot_mapping must be a contiguous int64 [{B}] tensor")
    if block_tables.dtype != torch.int32 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32")
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32")
    _check_pools(cb, k_cache, v_cache, H)
    _check_seq_tables(block_tables, context_lens, B)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape:
        raise ValueError("out must be contiguous with q's shape")
    need = tq_decode_step_workspace_bytes(cb, B, Hq, H, max_context_len, tokens_per_split)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    _check(_lib.tq_decode_step(
        cb.ref, _ptr(k_new), _ptr(v_new), _dtype_code(k_new), k_new.stride(0), k_new.stride(1),
        _ptr(slot_mapping), _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), B, Hq, H, max_context_len, float(softmax_scale),
        _ptr(out), _dtype_code(out), tokens_per_split, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(stream, q.device)))
    return out


def tq_decode_noalloc_scratch_bytes() -> int:
    return int(_lib.tq_decode_noalloc_scratch_bytes())


def tq_decode_attention_noalloc(cb: Codebook, q, k_cache, v_cache, block_tables, context_lens,
                                max_context_len: int, num_kv_heads: int, out,
                                softmax_scale: float = 0.0, tokens_per_split: int = 0, stream=None):
    """tq_decode_attention without a workspace: the library's device scratch
    holds the partial records, and ``out`` (allocated by the caller) is
    filled.  Allocates nothing."""
    torch = _torch()
    if q.dim() != 4 or q.shape[3] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][q_len][Hq][128] tensor")
    if block_tables.dtype != torch.int32 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32")
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32")
    B, q_len, Hq, _ = q.shape
    _check_pools(cb, k_cache, v_cache, num_kv_heads)
    _check_seq_tables(block_tables, context_lens, B)
    if out is None or not out.is_contiguous() or out.shape != q.shape:
        raise ValueError("out must be a contiguous tensor with q's shape")
    _check(_lib.tq_decode_attention_noalloc(
        cb.ref, _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), B, q_len, Hq, num_kv_heads,
        max_context_len, float(softmax_scale), _ptr(out), _dtype_code(out), tokens_per_split,
        _stream(stream, q.device)))
    return out


def tq_decode_window_workspace_bytes(cb: Codebook, num_seqs: int, q_len: int, num_q_heads: int,
                                     num_kv_heads: int, max_context_len: int, window: int,
                                     tokens_per_split: int = 0) -> int:
    return int(_lib.tq_decode_window_workspace_bytes(cb.ref, num_seqs, q_len, num_q_heads, num_kv_heads,
                                                     max_context_len, window, tokens_per_split))


def tq_decode_attention_window(cb: Codebook, q, k_cache, v_cache, block_tables, context_lens,
                               max_context_len: int, num_kv_heads: int, window: int, out=None,
                               softmax_scale: float = 0.0, tokens_per_split: int = 0,
                               workspace=None, out_dtype=None, stream=None):
    """Sliding-window decode over a rotating cache: query t of sequence b sees
    the last ``window`` positions up to its own; ``block_tables`` row b
    (int32 [B][ring_blocks]) is a ring, position j in page
    ``block_tables[b][(j // 16) % ring_blocks]``.  Returns ``out``."""
    torch = _torch()
    if q.dim() != 4 or q.shape[3] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][q_len][Hq][128] tensor")
    if block_tables.dtype != torch.int32 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32")
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32")
    B, q_len, Hq, _ = q.shape
    _check_pools(cb, k_cache, v_cache, num_kv_heads)
    _check_seq_tables(block_tables, context_lens, B)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape:
        raise ValueError("out must be contiguous with q's shape")
    need = tq_decode_window_workspace_bytes(cb, B, q_len, Hq, num_kv_heads, max_context_len, window,
                                            tokens_per_split)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    _check(_lib.tq_decode_attention_window(
        cb.ref, _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), B, q_len, Hq, num_kv_heads, max_context_len, int(window),
        float(softmax_scale), _ptr(out), _dtype_code(out), tokens_per_split,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q.device)))
    return out


def tq_decode_hot_workspace_bytes(cb: Codebook, num_seqs: int, num_q_heads: int,
                                  num_kv_heads: int, max_context_len: int, hot_max: int,
                                  tokens_per_split: int = 0) -> int:
    return int(_lib.tq_decode_hot_workspace_bytes(cb.ref, num_seqs, num_q_heads, num_kv_heads,
                                                  max_context_len, hot_max, tokens_per_split))


def tq_decode_attention_hot(cb: Codebook, q, k_cache, v_cache, block_tables, context_lens,
                            max_context_len: int, num_kv_heads: int, hot_k, hot_v, hot_lens,
                            out=None, softmax_scale: float = 0.0, tokens_per_split: int = 0,
                            workspace=None, out_dtype=None, stream=None):
    """Decode attention (q: [B][1][Hq][128]) over the compressed history of
    context_lens[b] tokens followed by hot_lens[b] exact tokens of
    hot_k / hot_v ([B][hot_max][Hkv][128], f32 / f16 / bf16).  Returns ``out``."""
    torch = _torch()
    if q.dim() != 4 or q.shape[1] != 1 or q.shape[3] != HEAD_DIM or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B][1][Hq][128] tensor")
    if block_tables.dtype != torch.int32 or not block_tables.is_contiguous():
        raise ValueError("block_tables must be contiguous int32")
    if context_lens.dtype != torch.int32 or not context_lens.is_contiguous():
        raise ValueError("context_lens must be contiguous int32")
    if hot_lens.dtype != torch.int32 or not hot_lens.is_contiguous():
        raise ValueError("hot_lens must be contiguous int32")
    B, _, Hq, _ = q.shape
    _check_pools(cb, k_cache, v_cache, num_kv_heads)
    _check_seq_tables(block_tables, context_lens, B)
    if hot_lens.dim() != 1 or hot_lens.shape[0] != B:
        raise ValueError(f"hot_lens must have one entry per sequence ({B})")
    if (hot_k.dim() != 4 or hot_k.shape[0] != B or hot_k.shape[2] != num_kv_heads
            or hot_k.shape[3] != HEAD_DIM or not hot_k.is_contiguous()):
        raise ValueError("hot_k must be a contiguous [B][hot_max][Hkv][128] tensor")
    if hot_v.shape != hot_k.shape or hot_v.dtype != hot_k.dtype or not hot_v.is_contiguous():
        raise ValueError("hot_v must match hot_k")
    hot_max = hot_k.shape[1]
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype or torch.float32, device=q.device)
    if not out.is_contiguous() or out.shape != q.shape:
        raise ValueError("out must be contiguous with q's shape")
    need = tq_decode_hot_workspace_bytes(cb, B, Hq, num_kv_heads, max_context_len, hot_max,
                                         tokens_per_split)
    if workspace is None:
        workspace = torch.empty(max(need, 4), dtype=torch.uint8, device=q.device)
    _check(_lib.tq_decode_attention_hot(
        cb.ref, _ptr(q), _dtype_code(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_tables),
        block_tables.shape[1], _ptr(context_lens), B, Hq, num_kv_heads, max_context_len,
        _ptr(hot_k), _ptr(hot_v), _dtype_code(hot_k), _ptr(hot_lens), hot_max,
        float(softmax_scale), _ptr(out), _dtype_code(out), tokens_per_split,
        _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(stream, q.device)))
    return out
