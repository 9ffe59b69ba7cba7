"""Python binding of libmla.so (argument marshalling only).

Every function here checks its tensors, passes their device pointers and the
current HIP stream to the C ABI declared in include/mla.h, and raises
RuntimeError on a non-zero status. All arithmetic runs in the library's HIP
kernels; there is no fallback path. PyTorch supplies device memory and streams.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla.so")
_lib = None

MLA_FP32 = 0
MLA_BF16 = 1
_TORCH_DTYPE = {MLA_FP32: torch.float32, MLA_BF16: torch.bfloat16}


class MLADims(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("H", ctypes.c_int32), ("d_h", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("d_c", ctypes.c_int32), ("d_R", ctypes.c_int32),
                ("d_cq", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("rope_theta", ctypes.c_float), ("norm_eps", ctypes.c_float),
                ("dtype", ctypes.c_int32)]

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]


class MLACache(ctypes.Structure):
    _fields_ = [("data", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("capacity", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("max_blocks", ctypes.c_int32), ("n_blocks", ctypes.c_int32)]


_SIGS = {
    "mla_compress_append": (ctypes.c_int, [ctypes.POINTER(MLADims), ctypes.c_int32] + [ctypes.c_void_p] * 5
                            + [ctypes.POINTER(MLACache), ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_absorb_q": (ctypes.c_int, [ctypes.POINTER(MLADims), ctypes.c_int32] + [ctypes.c_void_p] * 8
                     + [ctypes.c_size_t, ctypes.c_void_p]),
    "mla_decode_attn": (ctypes.c_int, [ctypes.POINTER(MLADims), ctypes.c_int32, ctypes.c_void_p,
                                       ctypes.POINTER(MLACache), ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_size_t, ctypes.c_void_p]),
    "mla_decode_attn_noalloc": (ctypes.c_int, [ctypes.POINTER(MLADims), ctypes.c_int32, ctypes.c_void_p,
                                               ctypes.POINTER(MLACache), ctypes.c_void_p, ctypes.c_int32,
                                               ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "mla_decode_attn_sparse": (ctypes.c_int, [ctypes.POINTER(MLADims), ctypes.c_int32, ctypes.c_void_p,
                                              ctypes.POINTER(MLACache), ctypes.c_void_p, ctypes.c_int32,
                                              ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_out_proj": (ctypes.c_int, [ctypes.POINTER(MLADims), ctypes.c_int32] + [ctypes.c_void_p] * 6
                     + [ctypes.c_size_t, ctypes.c_void_p]),
    "mla_precompose": (ctypes.c_int, [ctypes.POINTER(MLADims)] + [ctypes.c_void_p] * 7),
    "mla_absorb_q_precomposed": (ctypes.c_int, [ctypes.POINTER(MLADims), ctypes.c_int32] + [ctypes.c_void_p] * 7
                                 + [ctypes.c_size_t, ctypes.c_void_p]),
    "mla_out_proj_precomposed": (ctypes.c_int, [ctypes.POINTER(MLADims), ctypes.c_int32] + [ctypes.c_void_p] * 4
                                 + [ctypes.c_size_t, ctypes.c_void_p]),
    "mla_prefill_attn": (ctypes.c_int, [ctypes.POINTER(MLADims), ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.POINTER(MLACache), ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "mla_prefill_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MLADims), ctypes.c_int32, ctypes.c_int32,
                                                      ctypes.c_int32, ctypes.POINTER(MLACache), ctypes.c_int32]),
    "mla_prefill_choose": (ctypes.c_int32, [ctypes.POINTER(MLADims), ctypes.c_int32, ctypes.c_int32,
                                             ctypes.c_int32, ctypes.POINTER(MLACache)]),
    "mla_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(MLADims), ctypes.c_int32, ctypes.c_int32,
                                              ctypes.c_int32]),
    "mla_decode_num_splits": (ctypes.c_int32, [ctypes.POINTER(MLADims), ctypes.c_int32, ctypes.c_int32,
                                               ctypes.c_int32]),
    "mla_cache_row_bytes": (ctypes.c_size_t, [ctypes.POINTER(MLADims)]),
    "mla_decode_kernel": (ctypes.c_int32, [ctypes.POINTER(MLADims)]),
    "mla_check_indices": (ctypes.c_int, [ctypes.POINTER(MLADims), ctypes.c_int32, ctypes.POINTER(MLACache)]
                          + [ctypes.c_void_p] * 2 + [ctypes.c_int32] + [ctypes.c_void_p] * 2 + [ctypes.c_int32]
                          + [ctypes.c_void_p]),
    "mla_time_next_attn": (ctypes.c_int, [ctypes.c_void_p] * 3),
    "mla_status_str": (ctypes.c_char_p, [ctypes.c_int32]),
    "mla_last_error": (ctypes.c_char_p, []),
}
EXPORTED = tuple(_SIGS)


def library_path() -> str:
    return _LIB_PATH


def lib():
    """The loaded libmla.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it first (__graft_entry__.build())")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status: int, what: str) -> None:
    if status != 0:
        L = lib()
        raise RuntimeError(f"{what}: {L.mla_status_str(status).decode()} ({L.mla_last_error().decode()})")


def make_dims(d, H, d_h, d_v, d_c, d_R, d_cq, dtype, softmax_scale=0.0, rope_theta=10000.0,
              norm_eps=0.0) -> MLADims:
    dt = {"fp32": MLA_FP32, "bf16": MLA_BF16}.get(dtype, dtype)
    return MLADims(d, H, d_h, d_v, d_c, d_R, d_cq, softmax_scale, rope_theta, norm_eps, dt)


def make_cache(data: torch.Tensor, block_table: Optional[torch.Tensor] = None) -> MLACache:
    """Describe a contiguous [B][capacity][D] cache, or a paged pool
    [n_blocks][block_size][D] with an int32 block table [B][max_blocks]."""
    if block_table is None:
        assert data.dim() == 3
        return MLACache(data.data_ptr(), None, data.shape[1], 0, 0, 0)
    assert data.dim() == 3 and block_table.dim() == 2 and block_table.dtype == torch.int32
    return MLACache(data.data_ptr(), block_table.data_ptr(), 0, data.shape[1], block_table.shape[1],
                    data.shape[0])


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor"):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def workspace_bytes(dims: MLADims, B: int, max_seq_len: int, num_splits: int = 0) -> int:
    return lib().mla_workspace_bytes(ctypes.byref(dims), B, max_seq_len, num_splits)


def decode_num_splits(dims: MLADims, B: int, max_seq_len: int, num_splits: int = 0) -> int:
    return lib().mla_decode_num_splits(ctypes.byref(dims), B, max_seq_len, num_splits)


def cache_row_bytes(dims: MLADims) -> int:
    return lib().mla_cache_row_bytes(ctypes.byref(dims))


def decode_kernel(dims: MLADims) -> int:
    return lib().mla_decode_kernel(ctypes.byref(dims))


def _host_i32(a, name):
    """Host int32 array (numpy or CPU tensor) -> (keep-alive object, pointer)."""
    if a is None:
        return None, None
    import numpy as np
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise ValueError(f"{name} must be a host array (copy it back first)")
        a = a.numpy()
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data


def mla_check_indices(dims, B: int, cache: MLACache, pos=None, seq_lens=None, max_seq_len: int = 0,
                      block_table=None, indices=None, counts=None) -> None:
    """Check host copies of the positions, lengths, block table and top-k lists
    the kernels read unchecked (see mla_check_indices in mla.h); raises
    RuntimeError naming the first violation."""
    keep = [_host_i32(a, n) for a, n in ((pos, "pos"), (seq_lens, "seq_lens"), (block_table, "block_table"),
                                          (indices, "indices"), (counts, "counts"))]
    topk = 0 if indices is None else int(keep[3][0].shape[-1])
    _check(lib().mla_check_indices(ctypes.byref(dims), int(B), ctypes.byref(cache), keep[0][1], keep[1][1],
                                   int(max_seq_len), keep[2][1], keep[3][1], topk, keep[4][1]),
           "mla_check_indices")


def mla_compress_append(dims, h_t, W_DKV, W_KR, gamma_kv, pos, cache: MLACache, ws, stream=None):
    dt = dims.torch_dtype
    B = h_t.shape[0]
    _check(lib().mla_compress_append(
        ctypes.byref(dims), B, _ptr(h_t, dt, "h_t"), _ptr(W_DKV, dt, "W_DKV"), _ptr(W_KR, dt, "W_KR"),
        _ptr(gamma_kv, dt, "gamma_kv"), _ptr(pos, torch.int32, "pos"), ctypes.byref(cache),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)), "mla_compress_append")


def mla_absorb_q(dims, h_t, W_DQ, W_UQ, W_QR, W_UK, pos, q, ws, stream=None):
    dt = dims.torch_dtype
    B = h_t.shape[0]
    _check(lib().mla_absorb_q(
        ctypes.byref(dims), B, _ptr(h_t, dt, "h_t"), _ptr(W_DQ, dt, "W_DQ"), _ptr(W_UQ, dt, "W_UQ"),
        _ptr(W_QR, dt, "W_QR"), _ptr(W_UK, dt, "W_UK"), _ptr(pos, torch.int32, "pos"),
        _ptr(q, dt, "q"), _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)),
        "mla_absorb_q")


def mla_decode_attn(dims, q, cache: MLACache, seq_lens, max_seq_len: int, o_lat, lse=None, ws=None,
                    num_splits: int = 0, stream=None):
    dt = dims.torch_dtype
    B = q.shape[0]
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().mla_decode_attn(
        ctypes.byref(dims), B, _ptr(q, dt, "q"), ctypes.byref(cache), _ptr(seq_lens, torch.int32, "seq_lens"),
        int(max_seq_len), int(num_splits), _ptr(o_lat, torch.float32, "o_lat"),
        _ptr(lse, torch.float32, "lse"), _ptr(ws, None, "ws"), wsz, _stream(stream)), "mla_decode_attn")


def mla_decode_attn_noalloc(dims, q, cache: MLACache, seq_lens, max_seq_len: int, o_lat, lse=None,
                            num_splits: int = 0, stream=None):
    """mla_decode_attn with the library's static per-device scratch (no workspace)."""
    dt = dims.torch_dtype
    B = q.shape[0]
    _check(lib().mla_decode_attn_noalloc(
        ctypes.byref(dims), B, _ptr(q, dt, "q"), ctypes.byref(cache), _ptr(seq_lens, torch.int32, "seq_lens"),
        int(max_seq_len), int(num_splits), _ptr(o_lat, torch.float32, "o_lat"),
        _ptr(lse, torch.float32, "lse"), _stream(stream)), "mla_decode_attn_noalloc")


def mla_decode_attn_sparse(dims, q, cache: MLACache, indices, counts, o_lat, lse=None, ws=None,
                           num_splits: int = 0, stream=None):
    """indices [B][topk] int32, counts [B] int32 (entries used per sequence)."""
    dt = dims.torch_dtype
    B = q.shape[0]
    topk = int(indices.shape[1])
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().mla_decode_attn_sparse(
        ctypes.byref(dims), B, _ptr(q, dt, "q"), ctypes.byref(cache), _ptr(indices, torch.int32, "indices"),
        topk, _ptr(counts, torch.int32, "counts"), int(num_splits), _ptr(o_lat, torch.float32, "o_lat"),
        _ptr(lse, torch.float32, "lse"), _ptr(ws, None, "ws"), wsz, _stream(stream)), "mla_decode_attn_sparse")


def mla_time_next_attn(kernel_start=None, kernel_end=None, call_end=None):
    """Stamp hipEvent_t handles (ints, or None to leave one out) with the next
    attention call's kernel start, kernel end and call end on this thread."""
    conv = lambda e: None if e is None else ctypes.c_void_p(int(e))
    _check(lib().mla_time_next_attn(conv(kernel_start), conv(kernel_end), conv(call_end)), "mla_time_next_attn")


def mla_out_proj(dims, o_lat, W_UV, W_O, o_heads, out, ws, stream=None):
    dt = dims.torch_dtype
    B = o_lat.shape[0]
    _check(lib().mla_out_proj(
        ctypes.byref(dims), B, _ptr(o_lat, torch.float32, "o_lat"), _ptr(W_UV, dt, "W_UV"),
        _ptr(W_O, dt, "W_O"), _ptr(o_heads, dt, "o_heads"), _ptr(out, dt, "out"),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)), "mla_out_proj")


def mla_precompose(dims, W_UQ, W_UK, W_QK, W_UV=None, W_O=None, W_OV=None, stream=None):
    """W_QK(i) = W_UK(i)^T W_UQ(i); W_OV = W_O blockdiag(W_UV(i)) when W_UV, W_O, W_OV are given."""
    dt = dims.torch_dtype
    _check(lib().mla_precompose(
        ctypes.byref(dims), _ptr(W_UQ, dt, "W_UQ"), _ptr(W_UK, dt, "W_UK"), _ptr(W_UV, dt, "W_UV"),
        _ptr(W_O, dt, "W_O"), _ptr(W_QK, dt, "W_QK"), _ptr(W_OV, dt, "W_OV"), _stream(stream)), "mla_precompose")


def mla_absorb_q_precomposed(dims, h_t, W_DQ, W_QK, W_QR, pos, q, ws, stream=None):
    dt = dims.torch_dtype
    B = h_t.shape[0]
    _check(lib().mla_absorb_q_precomposed(
        ctypes.byref(dims), B, _ptr(h_t, dt, "h_t"), _ptr(W_DQ, dt, "W_DQ"), _ptr(W_QK, dt, "W_QK"),
        _ptr(W_QR, dt, "W_QR"), _ptr(pos, torch.int32, "pos"), _ptr(q, dt, "q"), _ptr(ws, None, "ws"),
        ws.numel() * ws.element_size(), _stream(stream)), "mla_absorb_q_precomposed")


def mla_out_proj_precomposed(dims, o_lat, W_OV, out, ws, stream=None):
    dt = dims.torch_dtype
    B = o_lat.shape[0]
    _check(lib().mla_out_proj_precomposed(
        ctypes.byref(dims), B, _ptr(o_lat, torch.float32, "o_lat"), _ptr(W_OV, dt, "W_OV"), _ptr(out, dt, "out"),
        _ptr(ws, None, "ws"), ws.numel() * ws.element_size(), _stream(stream)), "mla_out_proj_precomposed")


PREFILL_MATERIALIZED, PREFILL_ABSORBED, PREFILL_AUTO = 0, 1, 2


def prefill_choose(dims: MLADims, B: int, T: int, max_seq_len: int, cache: MLACache) -> int:
    """The form PREFILL_AUTO runs for these sizes (-1 on bad arguments)."""
    return lib().mla_prefill_choose(ctypes.byref(dims), B, T, max_seq_len, ctypes.byref(cache))


def prefill_workspace_bytes(dims: MLADims, B: int, T: int, max_seq_len: int, cache: MLACache, algo: int) -> int:
    return lib().mla_prefill_workspace_bytes(ctypes.byref(dims), B, T, max_seq_len, ctypes.byref(cache), algo)


def mla_prefill_attn(dims, q, cache: MLACache, seq_lens, max_seq_len: int, W_UK, W_UV, algo: int, o, lse=None,
                     ws=None, stream=None):
    """q [B][T][H][d_h + d_R] -> o [B][T][H][d_v] (+ lse [B][T][H]); causal over each sequence's rows."""
    dt = dims.torch_dtype
    B, T = int(q.shape[0]), int(q.shape[1])
    wsz = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().mla_prefill_attn(
        ctypes.byref(dims), B, T, _ptr(q, dt, "q"), ctypes.byref(cache), _ptr(seq_lens, torch.int32, "seq_lens"),
        int(max_seq_len), _ptr(W_UK, dt, "W_UK"), _ptr(W_UV, dt, "W_UV"), int(algo), _ptr(o, dt, "o"),
        _ptr(lse, torch.float32, "lse"), _ptr(ws, None, "ws"), wsz, _stream(stream)), "mla_prefill_attn")
