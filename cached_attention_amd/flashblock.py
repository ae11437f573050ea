"""ctypes binding of libflashblock.so (include/flashblock.h), argument marshalling only.

Every entry point keeps the C name and argument order.  Tensor arguments may be
torch tensors (their data pointer is passed) or plain integer addresses; the
stream defaults to torch's current stream on the current device.  A non-zero
status raises ``FlashBlockError`` carrying fb_last_error().  Nothing here
computes attention: every step runs in the HIP library, and importing a
function from here fails loudly if the library has not been built.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import numpy as np

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libflashblock.so")

FB_ABI_VERSION = 1
FB_OK, FB_ERR_NULL, FB_ERR_SHAPE, FB_ERR_ALIGN, FB_ERR_WORKSPACE, FB_ERR_UNSUPPORTED, FB_ERR_ARG, FB_ERR_HIP = range(8)
FB_F32, FB_BF16 = 0, 1
FB_MODE_CACHED, FB_MODE_FULL = 0, 1
FB_CHUNKS_SELECTED, FB_CHUNKS_COMPLEMENT = 1, 2

EXPORTS = ("fb_workspace_size", "fb_prefix_attn", "fb_prefix_partials", "fb_prefix_combine",
           "fb_block_attn", "fb_merge", "fb_step", "fb_step_noalloc", "fb_refresh_mask_tau",
           "fb_refresh_mask_gamma",
           "fb_step_masked", "fb_append_block", "fb_select_chunks_ws", "fb_select_chunks",
           "fb_pool_chunk_keys", "fb_select_chunks_pooled",
           "fb_status_string", "fb_last_error", "fb_abi_version")


class FlashBlockError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        super().__init__(f"{where}: status {status}: {detail}")
        self.status = status


class fb_desc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("hq", ctypes.c_int32),
        ("hkv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_len", ctypes.c_int32),
        ("softmax_scale", ctypes.c_float),
        ("prefix_offsets_host", ctypes.POINTER(ctypes.c_int64)),
        ("prefix_offsets_dev", ctypes.c_void_p),
        ("q_stride_b", ctypes.c_int64), ("q_stride_t", ctypes.c_int64), ("q_stride_h", ctypes.c_int64),
        ("kv_stride_b", ctypes.c_int64), ("kv_stride_t", ctypes.c_int64), ("kv_stride_h", ctypes.c_int64),
        ("pre_stride_t", ctypes.c_int64), ("pre_stride_h", ctypes.c_int64),
    ]


class fb_sparse(ctypes.Structure):
    _fields_ = [
        ("chunk_idx_dev", ctypes.c_void_p),
        ("k", ctypes.c_int32),
        ("chunk_len", ctypes.c_int32),
        ("mode", ctypes.c_int32),
    ]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it is not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m cached_attention_amd.build`")
        l = ctypes.CDLL(_LIB_PATH)
        P, D, S = ctypes.c_void_p, ctypes.POINTER(fb_desc), ctypes.POINTER(fb_sparse)
        i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
        l.fb_workspace_size.argtypes = [D, S]
        l.fb_workspace_size.restype = sz
        l.fb_prefix_attn.argtypes = [D, P, P, P, S, P, P, P, sz, P]
        l.fb_prefix_attn.restype = i32
        l.fb_prefix_partials.argtypes = [D, P, P, P, S, P, sz, P]
        l.fb_prefix_partials.restype = i32
        l.fb_prefix_combine.argtypes = [D, S, P, P, P, P, P, sz, P]
        l.fb_prefix_combine.restype = i32
        l.fb_block_attn.argtypes = [D, P, P, P, P, P, P, P, P]
        l.fb_block_attn.restype = i32
        l.fb_merge.argtypes = [i64, i32, P, P, P, P, P, P, P]
        l.fb_merge.restype = i32
        l.fb_step.argtypes = [D, P, P, P, P, P, S, P, P, P, P, P, P, i32, i32, i32, i32,
                              ctypes.POINTER(i32), P, sz, P]
        l.fb_step.restype = i32
        l.fb_step_noalloc.argtypes = [D, P, P, P, P, P, S, P, P, P, P, P, P, i32, i32, i32, i32,
                                      ctypes.POINTER(i32), P]
        l.fb_step_noalloc.restype = i32
        f32 = ctypes.c_float
        l.fb_refresh_mask_tau.argtypes = [D, P, P, P, P, f32, i32, i32, P, P, P, sz, P]
        l.fb_refresh_mask_tau.restype = i32
        l.fb_refresh_mask_gamma.argtypes = [D, P, P, f32, i32, P, P, P]
        l.fb_refresh_mask_gamma.restype = i32
        l.fb_step_masked.argtypes = [D, P, P, P, P, P, P, P, P, P, P, P, sz, P]
        l.fb_step_masked.restype = i32
        l.fb_append_block.argtypes = [D, P, P, P, P, P, P]
        l.fb_append_block.restype = i32
        l.fb_select_chunks_ws.argtypes = [D, i32]
        l.fb_select_chunks_ws.restype = sz
        l.fb_select_chunks.argtypes = [D, P, P, i32, i32, P, P, sz, P]
        l.fb_select_chunks.restype = i32
        l.fb_pool_chunk_keys.argtypes = [D, P, i32, i32, i32, P, P]
        l.fb_pool_chunk_keys.restype = i32
        l.fb_select_chunks_pooled.argtypes = [D, P, P, i32, i32, i32, P, P, P]
        l.fb_select_chunks_pooled.restype = i32
        l.fb_status_string.argtypes = [i32]
        l.fb_status_string.restype = ctypes.c_char_p
        l.fb_last_error.argtypes = []
        l.fb_last_error.restype = ctypes.c_char_p
        l.fb_abi_version.argtypes = []
        l.fb_abi_version.restype = i32
        if l.fb_abi_version() != FB_ABI_VERSION:
            raise ImportError(f"libflashblock ABI {l.fb_abi_version()} != binding ABI {FB_ABI_VERSION}")
        _lib = l
    return _lib


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check(status: int, where: str) -> None:
    if status != FB_OK:
        raise FlashBlockError(status, where, lib().fb_last_error().decode())


class Desc:
    """Owns an fb_desc plus the host offsets array it points to."""

    def __init__(self, dtype: int, batch: int, hq: int, hkv: int, head_dim: int, block_len: int,
                 prefix_offsets_host: Sequence[int], prefix_offsets_dev=None, softmax_scale: float = 0.0,
                 q_strides: Optional[Sequence[int]] = None, kv_strides: Optional[Sequence[int]] = None,
                 pre_strides: Optional[Sequence[int]] = None):
        self._off = np.ascontiguousarray(np.asarray(prefix_offsets_host, dtype=np.int64))
        self._off_dev = prefix_offsets_dev      # keeps a tensor alive
        d = fb_desc()
        d.abi_version = FB_ABI_VERSION
        d.dtype, d.batch, d.hq, d.hkv = dtype, batch, hq, hkv
        d.head_dim, d.block_len, d.softmax_scale = head_dim, block_len, softmax_scale
        d.prefix_offsets_host = self._off.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
        d.prefix_offsets_dev = _ptr(prefix_offsets_dev)
        qs = q_strides or (block_len * hq * head_dim, hq * head_dim, head_dim)
        ks = kv_strides or (block_len * hkv * head_dim, hkv * head_dim, head_dim)
        ps = pre_strides or (hkv * head_dim, head_dim)
        d.q_stride_b, d.q_stride_t, d.q_stride_h = qs
        d.kv_stride_b, d.kv_stride_t, d.kv_stride_h = ks
        d.pre_stride_t, d.pre_stride_h = ps
        self.c = d

    @property
    def ref(self):
        return ctypes.byref(self.c)


class Sparse:
    def __init__(self, chunk_idx_dev, k: int, chunk_len: int = 64, mode: int = FB_CHUNKS_SELECTED):
        self._idx = chunk_idx_dev
        s = fb_sparse()
        s.chunk_idx_dev = _ptr(chunk_idx_dev)
        s.k, s.chunk_len, s.mode = k, chunk_len, mode
        self.c = s

    @property
    def ref(self):
        return ctypes.byref(self.c)


def _sref(sparse):
    return None if sparse is None else sparse.ref


def fb_workspace_size(desc: Desc, sparse: Optional[Sparse] = None) -> int:
    n = lib().fb_workspace_size(desc.ref, _sref(sparse))
    if n == 0:
        raise FlashBlockError(FB_ERR_ARG, "fb_workspace_size", lib().fb_last_error().decode())
    return n


def fb_prefix_attn(desc: Desc, q_blk, k_pre, v_pre, sparse: Optional[Sparse], o_ext, lse_ext, ws,
                   ws_bytes: int, stream=None) -> None:
    _check(lib().fb_prefix_attn(desc.ref, _ptr(q_blk), _ptr(k_pre), _ptr(v_pre), _sref(sparse), _ptr(o_ext),
                                _ptr(lse_ext), _ptr(ws), ws_bytes, _stream(stream)), "fb_prefix_attn")


def fb_prefix_partials(desc: Desc, q_blk, k_pre, v_pre, sparse: Optional[Sparse], ws, ws_bytes: int,
                       stream=None) -> None:
    _check(lib().fb_prefix_partials(desc.ref, _ptr(q_blk), _ptr(k_pre), _ptr(v_pre), _sref(sparse), _ptr(ws),
                                    ws_bytes, _stream(stream)), "fb_prefix_partials")


def fb_prefix_combine(desc: Desc, sparse: Optional[Sparse], extra_o, extra_lse, o_ext, lse_ext, ws,
                      ws_bytes: int, stream=None) -> None:
    _check(lib().fb_prefix_combine(desc.ref, _sref(sparse), _ptr(extra_o), _ptr(extra_lse), _ptr(o_ext),
                                   _ptr(lse_ext), _ptr(ws), ws_bytes, _stream(stream)), "fb_prefix_combine")


def fb_block_attn(desc: Desc, q_blk, k_blk, v_blk, o_ext, lse_ext, o, lse_out=None, stream=None) -> None:
    _check(lib().fb_block_attn(desc.ref, _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(o_ext), _ptr(lse_ext),
                               _ptr(o), _ptr(lse_out), _stream(stream)), "fb_block_attn")


def fb_merge(rows: int, head_dim: int, o_a, lse_a, o_b, lse_b, o, lse, stream=None) -> None:
    _check(lib().fb_merge(rows, head_dim, _ptr(o_a), _ptr(lse_a), _ptr(o_b), _ptr(lse_b), _ptr(o), _ptr(lse),
                          _stream(stream)), "fb_merge")


def fb_step(desc: Desc, q_blk, k_blk, v_blk, k_pre, v_pre, sparse: Optional[Sparse], o_ext_cache,
            lse_ext_cache, o_res_cache, lse_res_cache, o, lse_out, step: int, refresh_period: int,
            mode: int, force_refresh: bool, ws, ws_bytes: int, stream=None) -> bool:
    """Returns True if this step refreshed the block-external cache."""
    refreshed = ctypes.c_int32(0)
    _check(lib().fb_step(desc.ref, _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_pre), _ptr(v_pre),
                         _sref(sparse), _ptr(o_ext_cache), _ptr(lse_ext_cache), _ptr(o_res_cache),
                         _ptr(lse_res_cache), _ptr(o), _ptr(lse_out), step, refresh_period, mode,
                         int(bool(force_refresh)), ctypes.byref(refreshed), _ptr(ws), ws_bytes,
                         _stream(stream)), "fb_step")
    return bool(refreshed.value)


FB_NOALLOC_SCRATCH_BYTES = 64 << 20


def fb_step_noalloc(desc: Desc, q_blk, k_blk, v_blk, k_pre, v_pre, sparse: Optional[Sparse], o_ext_cache,
                    lse_ext_cache, o_res_cache, lse_res_cache, o, lse_out, step: int, refresh_period: int,
                    mode: int, force_refresh: bool, stream=None) -> bool:
    """fb_step with the library's per-GPU scratch instead of a workspace; returns
    True if this step refreshed the block-external cache."""
    refreshed = ctypes.c_int32(0)
    _check(lib().fb_step_noalloc(desc.ref, _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_pre), _ptr(v_pre),
                                 _sref(sparse), _ptr(o_ext_cache), _ptr(lse_ext_cache), _ptr(o_res_cache),
                                 _ptr(lse_res_cache), _ptr(o), _ptr(lse_out), step, refresh_period, mode,
                                 int(bool(force_refresh)), ctypes.byref(refreshed), _stream(stream)),
           "fb_step_noalloc")
    return bool(refreshed.value)


def fb_refresh_mask_tau(desc: Desc, k_prev, v_prev, k_cur, v_cur, eps: float, tau: int, step: int, count_out,
                        mask_out, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().fb_refresh_mask_tau(desc.ref, _ptr(k_prev), _ptr(v_prev), _ptr(k_cur), _ptr(v_cur), eps, tau,
                                     step, _ptr(count_out), _ptr(mask_out), _ptr(ws), ws_bytes, _stream(stream)),
           "fb_refresh_mask_tau")


def fb_refresh_mask_gamma(desc: Desc, q_cur, q_ref, gamma: float, step: int, sim_out, mask_out,
                          stream=None) -> None:
    _check(lib().fb_refresh_mask_gamma(desc.ref, _ptr(q_cur), _ptr(q_ref), gamma, step, _ptr(sim_out),
                                       _ptr(mask_out), _stream(stream)), "fb_refresh_mask_gamma")


def fb_step_masked(desc: Desc, q_blk, k_blk, v_blk, k_pre, v_pre, mask, o_ext_cache, lse_ext_cache, o,
                   lse_out, ws, ws_bytes: int, stream=None) -> None:
    _check(lib().fb_step_masked(desc.ref, _ptr(q_blk), _ptr(k_blk), _ptr(v_blk), _ptr(k_pre), _ptr(v_pre),
                                _ptr(mask), _ptr(o_ext_cache), _ptr(lse_ext_cache), _ptr(o), _ptr(lse_out),
                                _ptr(ws), ws_bytes, _stream(stream)), "fb_step_masked")


def fb_append_block(desc: Desc, k_blk, v_blk, k_pre, v_pre, dst_rows_dev, stream=None) -> None:
    _check(lib().fb_append_block(desc.ref, _ptr(k_blk), _ptr(v_blk), _ptr(k_pre), _ptr(v_pre), _ptr(dst_rows_dev),
                                 _stream(stream)), "fb_append_block")


def fb_select_chunks_ws(desc: Desc, chunk_len: int = 64) -> int:
    n = lib().fb_select_chunks_ws(desc.ref, chunk_len)
    if n == 0:
        raise FlashBlockError(FB_ERR_ARG, "fb_select_chunks_ws", lib().fb_last_error().decode())
    return n


def fb_select_chunks(desc: Desc, q_blk, k_pre, chunk_len: int, k: int, chunk_idx_out, ws, ws_bytes: int,
                     stream=None) -> None:
    _check(lib().fb_select_chunks(desc.ref, _ptr(q_blk), _ptr(k_pre), chunk_len, k, _ptr(chunk_idx_out), _ptr(ws),
                                  ws_bytes, _stream(stream)), "fb_select_chunks")


def fb_pool_chunk_keys(desc: Desc, k_pre, chunk_len: int, chunk_cap: int, first_chunk: int, pooled,
                       stream=None) -> None:
    _check(lib().fb_pool_chunk_keys(desc.ref, _ptr(k_pre), chunk_len, chunk_cap, first_chunk, _ptr(pooled),
                                    _stream(stream)), "fb_pool_chunk_keys")


def fb_select_chunks_pooled(desc: Desc, q_blk, pooled, chunk_len: int, chunk_cap: int, k: int, scores,
                            chunk_idx_out, stream=None) -> None:
    _check(lib().fb_select_chunks_pooled(desc.ref, _ptr(q_blk), _ptr(pooled), chunk_len, chunk_cap, k, _ptr(scores),
                                         _ptr(chunk_idx_out), _stream(stream)), "fb_select_chunks_pooled")


def fb_status_string(status: int) -> str:
    return lib().fb_status_string(status).decode()


def fb_last_error() -> str:
    return lib().fb_last_error().decode()


def fb_abi_version() -> int:
    return lib().fb_abi_version()
