"""Thin ctypes binding of libmoe (include/libmoe.h).

Argument marshalling only: tensors become raw device pointers, the stream
defaults to torch's current stream, and a non-OK status raises MoeError with
the library's error text.  Every step of the layer runs in libmoe's HIP
kernels; PyTorch only provides device memory and streams.  There is no CPU
fallback: if the library is not built, loading fails loudly.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

MOE_OK, MOE_ERR_ARG, MOE_ERR_ALIGN, MOE_ERR_UNSUPPORTED, MOE_ERR_HIP, MOE_ERR_STATE, MOE_ERR_CAPACITY = range(7)
MOE_PREC_FP32, MOE_PREC_BF16_MFMA, MOE_PREC_F16_MFMA, MOE_PREC_F16_MFMA_DIRECT = 0, 1, 2, 3
MOE_CALL_ROUTE, MOE_CALL_PERMUTE, MOE_CALL_GATEUP, MOE_CALL_DOWN_COMBINE, MOE_CALL_DECODE_LAYERS = range(5)


class MoeError(RuntimeError):
    def __init__(self, status: int, text: str):
        super().__init__(f"libmoe status {status}: {text}")
        self.status = status


class moe_dims(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("f", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32)]


class moe_stage_stats(ctypes.Structure):
    _fields_ = [("hits", ctypes.c_int64), ("misses", ctypes.c_int64), ("bytes_staged", ctypes.c_int64)]


def dims(d: int, f: int, n_experts: int, top_k: int) -> moe_dims:
    return moe_dims(d, f, n_experts, top_k)


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float

_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_expert_blob_bytes": (_I64, [moe_dims]),
    "moe_expert_blob_offsets": (ctypes.c_int, [moe_dims, ctypes.POINTER(_I64)]),
    "moe_workspace_size": (_SZ, [ctypes.c_int, _I32, moe_dims, ctypes.c_int]),
    "moe_act_bytes": (_SZ, [_I32, moe_dims, ctypes.c_int]),
    "moe_route": (ctypes.c_int, [_P, _P, _F, _P, _P, _I32, moe_dims, _P, _P, _P, _P, _SZ, _P]),
    "moe_route_noalloc": (ctypes.c_int, [_P, _P, _F, _P, _P, _I32, moe_dims, _P, _P, _P, _P]),
    "moe_permute": (ctypes.c_int, [_P, _I32, moe_dims, _P, _P, _P, _P, _P, _SZ, _P]),
    "moe_expert_q4_gateup": (ctypes.c_int, [_P, _P, _P, _I32, _P, _I64, _P, _P, _P, _I32, _I32, moe_dims,
                                            ctypes.c_int, _P, _P, _SZ, _P]),
    "moe_expert_q4_down_combine": (ctypes.c_int, [_P, _P, _P, _P, _I32, _P, _I64, _P, _P, _P, _P, _I32,
                                                  moe_dims, ctypes.c_int, _P, _P, _SZ, _P]),
    "moe_cache_create": (ctypes.c_int, [_I32, _I32, _I32, _I32, _P, _I64, _P, _I64, _P, ctypes.POINTER(_P)]),
    "moe_cache_destroy": (ctypes.c_int, [_P]),
    "moe_slot_stage": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P, _P, _P, ctypes.POINTER(moe_stage_stats)]),
    "moe_cache_wait": (ctypes.c_int, [_P, _I32, _P]),
    "moe_cache_wait_expert": (ctypes.c_int, [_P, _I32, _I32, _P]),
    "moe_cache_slot_table": (ctypes.c_int, [_P, _I32, _P]),
    "moe_cache_export": (ctypes.c_int, [_P, _P, _P]),
    "moe_cache_import": (ctypes.c_int, [_P, _P, _P]),
    "moe_cache_set_policy": (ctypes.c_int, [_P, _I32, _I32]),
    "moe_cache_set_staging": (ctypes.c_int, [_P, _I32, _I32]),
    "moe_cache_enable_device": (ctypes.c_int, [_P]),
    "moe_slot_stage_device": (ctypes.c_int, [_P, _I32, _I32, _P, _P, _P, _P]),
    "moe_cache_stats": (ctypes.c_int, [_P, ctypes.POINTER(moe_stage_stats)]),
    "moe_cache_export_usage": (ctypes.c_int, [_P, _P, _P]),
    "moe_cache_import_usage": (ctypes.c_int, [_P, _P, _P]),
    "moe_shared_gemv_bf16": (ctypes.c_int, [_P, _P, _I32, _I32, _I32, _P, _P]),
    "moe_shared_expert_workspace_size": (_SZ, [_I32, _I32]),
    "moe_shared_expert_bf16": (ctypes.c_int, [_P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _SZ, _P]),
    "moe_rms_rescale": (ctypes.c_int, [_P, _I32, _I32, _F, _P, _P]),
    "moe_profile_next_launch": (ctypes.c_int, [ctypes.c_int, _P, _P]),
    "moe_decode_layers": (ctypes.c_int, [_P, _I32, _P, _F, _P, _P, _P, _I32, _P, _I64, _I64, moe_dims, _P, _P, _P,
                                         _P, _SZ, _P]),
    "moe_decode_check": (ctypes.c_int, [_P, _P]),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libmoe.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libmoe is not built ({LIB_PATH} missing): run __graft_entry__.build()")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def exported_symbols() -> list:
    return list(_SIGNATURES)


def _check(status: int) -> None:
    if status != MOE_OK:
        raise MoeError(status, lib().moe_last_error().decode())


def _dev(t, name):
    """Device pointer of a CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _host(t, name):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or t.is_cuda or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous host tensor")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


# ------------------------------------------------------------------ queries

def moe_expert_blob_bytes(dm: moe_dims) -> int:
    return int(lib().moe_expert_blob_bytes(dm))


def moe_expert_blob_offsets(dm: moe_dims) -> list:
    out = (_I64 * 6)()
    _check(lib().moe_expert_blob_offsets(dm, out))
    return list(out)


def moe_workspace_size(call: int, T: int, dm: moe_dims, prec: int = MOE_PREC_FP32) -> int:
    return int(lib().moe_workspace_size(call, T, dm, prec))


def moe_act_bytes(T: int, dm: moe_dims, prec: int) -> int:
    return int(lib().moe_act_bytes(T, dm, prec))


# ------------------------------------------------------------------ compute calls

def moe_route(x, norm_w, eps, router_w, router_bias, T, dm, h_out, topk_idx, topk_w, ws, stream=None):
    _check(lib().moe_route(_dev(x, "x"), _dev(norm_w, "norm_w"), float(eps), _dev(router_w, "router_w"),
                           _dev(router_bias, "router_bias"), int(T), dm, _dev(h_out, "h_out"),
                           _dev(topk_idx, "topk_idx"), _dev(topk_w, "topk_w"), _dev(ws, "ws"),
                           _nbytes(ws), _stream(stream)))


def moe_route_noalloc(x, norm_w, eps, router_w, router_bias, T, dm, h_out, topk_idx, topk_w, stream=None):
    _check(lib().moe_route_noalloc(_dev(x, "x"), _dev(norm_w, "norm_w"), float(eps), _dev(router_w, "router_w"),
                                   _dev(router_bias, "router_bias"), int(T), dm, _dev(h_out, "h_out"),
                                   _dev(topk_idx, "topk_idx"), _dev(topk_w, "topk_w"), _stream(stream)))


def moe_permute(topk_idx, T, dm, counts, offsets, sorted_pair, pair_pos, ws=None, stream=None):
    _check(lib().moe_permute(_dev(topk_idx, "topk_idx"), int(T), dm, _dev(counts, "counts"),
                             _dev(offsets, "offsets"), _dev(sorted_pair, "sorted_pair"),
                             _dev(pair_pos, "pair_pos"), _dev(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_expert_q4_gateup(h, topk_idx, slot_of_expert, n_slots, arena, slot_stride, offsets, sorted_pair,
                         pair_mask, mask_value, T, dm, prec, act, ws, stream=None):
    _check(lib().moe_expert_q4_gateup(_dev(h, "h"), _dev(topk_idx, "topk_idx"),
                                      _dev(slot_of_expert, "slot_of_expert"), int(n_slots),
                                      _dev(arena, "arena"), int(slot_stride), _dev(offsets, "offsets"),
                                      _dev(sorted_pair, "sorted_pair"), _dev(pair_mask, "pair_mask"),
                                      int(mask_value), int(T), dm, int(prec), _dev(act, "act"),
                                      _dev(ws, "ws"), _nbytes(ws), _stream(stream)))


def moe_expert_q4_down_combine(act, topk_idx, topk_w, slot_of_expert, n_slots, arena, slot_stride, offsets,
                               sorted_pair, pair_pos, residual, T, dm, prec, y, ws, stream=None):
    _check(lib().moe_expert_q4_down_combine(_dev(act, "act"), _dev(topk_idx, "topk_idx"),
                                            _dev(topk_w, "topk_w"), _dev(slot_of_expert, "slot_of_expert"),
                                            int(n_slots), _dev(arena, "arena"), int(slot_stride),
                                            _dev(offsets, "offsets"), _dev(sorted_pair, "sorted_pair"),
                                            _dev(pair_pos, "pair_pos"), _dev(residual, "residual"), int(T),
                                            dm, int(prec), _dev(y, "y"), _dev(ws, "ws"), _nbytes(ws),
                                            _stream(stream)))


def moe_shared_gemv_bf16(w, h, T, rows, cols, out, stream=None):
    _check(lib().moe_shared_gemv_bf16(_dev(w, "w"), _dev(h, "h"), int(T), int(rows), int(cols),
                                      _dev(out, "out"), _stream(stream)))


def moe_shared_expert_workspace_size(T, f_sh) -> int:
    return int(lib().moe_shared_expert_workspace_size(int(T), int(f_sh)))


def moe_shared_expert_bf16(w_gu, w_down, h, residual, T, d, f_sh, out, ws, stream=None):
    _check(lib().moe_shared_expert_bf16(_dev(w_gu, "w_gu"), _dev(w_down, "w_down"), _dev(h, "h"),
                                        _dev(residual, "residual"), int(T), int(d), int(f_sh), _dev(out, "out"),
                                        _dev(ws, "ws"), int(ws.numel() * ws.element_size()), _stream(stream)))


def moe_rms_rescale(x, T, d, eps, out, stream=None):
    _check(lib().moe_rms_rescale(_dev(x, "x"), int(T), int(d), float(eps), _dev(out, "out"), _stream(stream)))


def moe_decode_layers(x_io, n_layers, norm_w, eps, router_w, router_bias, slot_tables, n_slots, arena, layer_stride,
                      slot_stride, dm, topk_idx, topk_w, x_next, ws, stream=None):
    _check(lib().moe_decode_layers(_dev(x_io, "x_io"), int(n_layers), _dev(norm_w, "norm_w"), float(eps),
                                   _dev(router_w, "router_w"), _dev(router_bias, "router_bias"),
                                   _dev(slot_tables, "slot_tables"), int(n_slots), _dev(arena, "arena"),
                                   int(layer_stride), int(slot_stride), dm, _dev(topk_idx, "topk_idx"),
                                   _dev(topk_w, "topk_w"), _dev(x_next, "x_next"), _dev(ws, "ws"), _nbytes(ws),
                                   _stream(stream)))


def moe_decode_check(ws, stream=None):
    _check(lib().moe_decode_check(_dev(ws, "ws"), _stream(stream)))


def moe_profile_next_launch(call, start_event, stop_event):
    """Arm torch.cuda.Event(enable_timing=True) pairs for the next launch of `call`."""
    s = None if start_event is None else ctypes.c_void_p(start_event.cuda_event)
    e = None if stop_event is None else ctypes.c_void_p(stop_event.cuda_event)
    _check(lib().moe_profile_next_launch(int(call), s, e))


# ------------------------------------------------------------------ expert cache

class MoeCache:
    """Owner of a moe_cache handle (see moe_cache_create in libmoe.h)."""

    def __init__(self, n_layers, n_experts, n_slots, top_k, host_pool, blob_bytes, arena, slot_stride,
                 slot_tables):
        if not host_pool.is_pinned():
            raise ValueError("host_pool must be pinned host memory")
        self.n_layers, self.n_experts, self.n_slots, self.top_k = n_layers, n_experts, n_slots, top_k
        self._keep = (host_pool, arena, slot_tables)
        handle = ctypes.c_void_p()
        _check(lib().moe_cache_create(n_layers, n_experts, n_slots, top_k, _host(host_pool, "host_pool"),
                                      int(blob_bytes), _dev(arena, "arena"), int(slot_stride),
                                      _dev(slot_tables, "slot_tables"), ctypes.byref(handle)))
        self.handle = handle

    def close(self):
        if self.handle:
            _check(lib().moe_cache_destroy(self.handle))
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def moe_slot_stage(cache: MoeCache, layer, step, sel_host, side, compute, hit_mask_dev, hit_mask_host=None):
    stats = moe_stage_stats()
    _check(lib().moe_slot_stage(cache.handle, int(layer), int(step), _host(sel_host, "sel_host"),
                                _stream(side), _stream(compute), _dev(hit_mask_dev, "hit_mask_dev"),
                                _host(hit_mask_host, "hit_mask_host"), ctypes.byref(stats)))
    return stats


def moe_cache_wait(cache: MoeCache, layer, compute):
    _check(lib().moe_cache_wait(cache.handle, int(layer), _stream(compute)))


def moe_cache_wait_expert(cache: MoeCache, layer, rank, compute):
    _check(lib().moe_cache_wait_expert(cache.handle, int(layer), int(rank), _stream(compute)))


def moe_cache_slot_table(cache: MoeCache, layer, out_host):
    _check(lib().moe_cache_slot_table(cache.handle, int(layer), _host(out_host, "out_host")))


def moe_cache_export(cache: MoeCache, slot_expert_host, stamp_host):
    _check(lib().moe_cache_export(cache.handle, _host(slot_expert_host, "slot_expert"), _host(stamp_host, "stamp")))


def moe_cache_import(cache: MoeCache, slot_expert_host, stamp_host):
    _check(lib().moe_cache_import(cache.handle, _host(slot_expert_host, "slot_expert"), _host(stamp_host, "stamp")))


MOE_CACHE_LRU, MOE_CACHE_LFU, MOE_CACHE_LFU_WINDOW = 0, 1, 2


def moe_cache_set_policy(cache: MoeCache, policy, window=0):
    _check(lib().moe_cache_set_policy(cache.handle, int(policy), int(window)))


MOE_STAGE_COPY, MOE_STAGE_COPY_SPLIT, MOE_STAGE_KERNEL = 0, 1, 2


def moe_cache_set_staging(cache: MoeCache, mode, n_streams=0):
    _check(lib().moe_cache_set_staging(cache.handle, int(mode), int(n_streams)))


def moe_cache_enable_device(cache: MoeCache):
    _check(lib().moe_cache_enable_device(cache.handle))


def moe_slot_stage_device(cache: MoeCache, layer, step, sel_dev, side, compute, hit_mask_dev):
    _check(lib().moe_slot_stage_device(cache.handle, int(layer), int(step), _dev(sel_dev, "sel_dev"), _stream(side),
                                       _stream(compute), _dev(hit_mask_dev, "hit_mask_dev")))


def moe_cache_stats(cache: MoeCache):
    stats = moe_stage_stats()
    _check(lib().moe_cache_stats(cache.handle, ctypes.byref(stats)))
    return stats


def moe_cache_export_usage(cache: MoeCache, counts_host, recent_host=None):
    _check(lib().moe_cache_export_usage(cache.handle, _host(counts_host, "counts"), _host(recent_host, "recent")))


def moe_cache_import_usage(cache: MoeCache, counts_host, recent_host=None):
    _check(lib().moe_cache_import_usage(cache.handle, _host(counts_host, "counts"), _host(recent_host, "recent")))
