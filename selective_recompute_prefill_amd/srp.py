"""ctypes binding of libsrp.so (include/srp.h), with the same entry-point names.

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. torch tensors are accepted for device memory and streams; their data
pointers and the current HIP stream are passed through unchanged. There is no
fallback: if libsrp.so is missing or fails to load, every call raises."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("SRP_LIB", os.path.join(_PKG, "libsrp.so"))

SRP_OK, SRP_E_INVALID, SRP_E_WORKSPACE, SRP_E_UNSUPPORTED, SRP_E_HIP, SRP_E_BATCH = 0, -1, -2, -3, -4, -5
SRP_F32, SRP_BF16 = 0, 1
SRP_SEL_TOPK, SRP_SEL_GIVEN, SRP_SEL_SCORES = 0, 1, 2
SRP_K_ROUND, SRP_K_CEIL = 0, 1
SRP_DEV_KV, SRP_DEV_V = 0, 1

EXPORTS = ("srp_workspace_size", "srp_fuse_layer", "srp_fuse_layer_noalloc", "srp_encode_kv", "srp_rerotate_kv",
           "srp_residual_rmsnorm", "srp_stack_workspace_size", "srp_fuse_stack",
           "srp_controller_ratio", "srp_validate_batch", "srp_profile_begin", "srp_profile_end",
           "srp_profile_stage_name", "srp_last_error", "srp_version")
SRP_N_STAGES = 6


class SrpError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libsrp error {code}: {msg}")
        self.code = code


class Dims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("rope_base", ctypes.c_double), ("dtype", ctypes.c_int32)]


class Batch(ctypes.Structure):
    _fields_ = [("n_req", ctypes.c_int32), ("n_chunks", ctypes.c_int32),
                ("total_rows", ctypes.c_int32), ("max_req_rows", ctypes.c_int32),
                ("max_position", ctypes.c_int32),
                ("req_offsets", ctypes.c_void_p), ("chunk_offsets", ctypes.c_void_p),
                ("chunk_src_pos", ctypes.c_void_p), ("positions", ctypes.c_void_p),
                ("block_rows", ctypes.c_int32), ("seg_block", ctypes.c_void_p),
                ("block_table", ctypes.c_void_p)]


class Select(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("ratio", ctypes.c_double),
                ("window", ctypes.c_int32), ("tau", ctypes.c_int32),
                ("dev_mode", ctypes.c_int32), ("cand", ctypes.c_void_p),
                ("cand_offsets", ctypes.c_void_p), ("k_rule", ctypes.c_int32),
                ("span_max", ctypes.c_int32), ("scores", ctypes.c_void_p),
                ("tau_smooth", ctypes.c_double), ("tau_cover", ctypes.c_double),
                ("cap_ratio", ctypes.c_double), ("fresh_all", ctypes.c_int32)]


class Layer(ctypes.Structure):
    _fields_ = [("w_qkv", ctypes.c_void_p), ("k_cache", ctypes.c_void_p),
                ("v_cache", ctypes.c_void_p), ("k_host", ctypes.c_void_p),
                ("v_host", ctypes.c_void_p), ("ratio", ctypes.c_double), ("mode", ctypes.c_int32)]


_lib: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built (run selective_recompute_prefill_amd.build)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        P = ctypes.POINTER
        L.srp_workspace_size.argtypes = [P(Dims), P(Batch), P(Select), P(sz)]
        L.srp_fuse_layer.argtypes = [P(Dims), P(Batch), P(Select), vp, vp, vp, vp, vp, vp, vp, vp,
                                     vp, sz, vp]
        L.srp_fuse_layer_noalloc.argtypes = [P(Dims), P(Batch), P(Select), vp, vp, vp, vp, vp, vp, vp,
                                             vp, vp]
        L.srp_encode_kv.argtypes = [P(Dims), i32, i32, vp, vp, vp, vp, vp, vp]
        L.srp_rerotate_kv.argtypes = [P(Dims), P(Batch), vp, vp]
        L.srp_residual_rmsnorm.argtypes = [P(Dims), vp, vp, vp, vp, i32, i32, ctypes.c_float, vp]
        L.srp_stack_workspace_size.argtypes = [P(Dims), P(Batch), P(Select), P(sz)]
        L.srp_fuse_stack.argtypes = [P(Dims), P(Batch), P(Select), i32, P(Layer), vp, ctypes.c_float,
                                     vp, vp, vp, vp, sz, vp, vp]
        L.srp_controller_ratio.argtypes = [ctypes.c_double, ctypes.c_double, ctypes.c_double,
                                           P(ctypes.c_double)]
        L.srp_validate_batch.argtypes = [P(Batch), vp]
        L.srp_profile_begin.argtypes = [i32]
        L.srp_profile_end.argtypes = [P(ctypes.c_float), i32, P(i32)]
        L.srp_profile_stage_name.argtypes = [i32]
        L.srp_profile_stage_name.restype = ctypes.c_char_p
        for f in ("srp_workspace_size", "srp_fuse_layer", "srp_fuse_layer_noalloc", "srp_encode_kv", "srp_rerotate_kv",
                  "srp_residual_rmsnorm", "srp_stack_workspace_size", "srp_fuse_stack",
                  "srp_controller_ratio", "srp_validate_batch", "srp_profile_begin",
                  "srp_profile_end"):
            getattr(L, f).restype = ctypes.c_int
        L.srp_last_error.restype = ctypes.c_char_p
        L.srp_version.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(rc: int) -> int:
    if rc != SRP_OK:
        raise SrpError(rc, lib().srp_last_error().decode())
    return rc


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (or None / an int passed through)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_dims(hidden, n_heads, n_kv_heads, head_dim, rope_base=10000.0, dtype=SRP_BF16) -> Dims:
    return Dims(hidden, n_heads, n_kv_heads, head_dim, float(rope_base), dtype)


def make_batch(req_offsets, chunk_offsets, chunk_src_pos, positions, *, total_rows: int,
               max_req_rows: int, max_position: int, block_rows: int = 0, seg_block=None,
               block_table=None) -> Batch:
    """Batch descriptor over int32 device tensors (sizes are host ints). block_rows > 0
    with seg_block / block_table describes a paged cache pool."""
    return Batch(len(req_offsets) - 1, len(chunk_offsets) - 1, int(total_rows), int(max_req_rows),
                 int(max_position), _ptr(req_offsets), _ptr(chunk_offsets), _ptr(chunk_src_pos),
                 _ptr(positions), int(block_rows), _ptr(seg_block), _ptr(block_table))


def make_select(ratio: float, *, mode=SRP_SEL_TOPK, window=0, tau=0, dev_mode=SRP_DEV_KV,
                cand=None, cand_offsets=None, k_rule=SRP_K_ROUND, scores=None, span_max=0,
                tau_smooth=0.0, tau_cover=0.0, cap_ratio=0.0, fresh_all=False) -> Select:
    """Selection descriptor; `scores` (fp32 device tensor [T]) goes with SRP_SEL_SCORES.
    SpecCache's span completion is span_max=16, tau_smooth=0.4, tau_cover=0.7."""
    return Select(mode, float(ratio), int(window), int(tau), dev_mode, _ptr(cand), _ptr(cand_offsets),
                  int(k_rule), int(span_max), _ptr(scores), float(tau_smooth), float(tau_cover),
                  float(cap_ratio), int(bool(fresh_all)))


def srp_workspace_size(dims: Dims, batch: Batch, sel: Select) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().srp_workspace_size(ctypes.byref(dims), ctypes.byref(batch), ctypes.byref(sel),
                                    ctypes.byref(n)))
    return n.value


def srp_fuse_layer(dims: Dims, batch: Batch, sel: Select, hidden, w_qkv, k_cache, v_cache,
                   sel_idx, sel_offsets, attn_out, dev_out, workspace, workspace_bytes: int,
                   stream=None) -> int:
    return _check(lib().srp_fuse_layer(
        ctypes.byref(dims), ctypes.byref(batch), ctypes.byref(sel), _ptr(hidden), _ptr(w_qkv),
        _ptr(k_cache), _ptr(v_cache), _ptr(sel_idx), _ptr(sel_offsets), _ptr(attn_out),
        _ptr(dev_out), _ptr(workspace), int(workspace_bytes), _stream(stream)))


def srp_fuse_layer_noalloc(dims: Dims, batch: Batch, sel: Select, hidden, w_qkv, k_cache, v_cache,
                           sel_idx, sel_offsets, attn_out, dev_out, stream=None) -> int:
    """srp_fuse_layer on the library's static scratch array (no workspace, no
    allocation); calls that overlap on one GPU race."""
    return _check(lib().srp_fuse_layer_noalloc(
        ctypes.byref(dims), ctypes.byref(batch), ctypes.byref(sel), _ptr(hidden), _ptr(w_qkv),
        _ptr(k_cache), _ptr(v_cache), _ptr(sel_idx), _ptr(sel_offsets), _ptr(attn_out),
        _ptr(dev_out), _stream(stream)))


def srp_encode_kv(dims: Dims, n_rows: int, max_position: int, hidden, w_qkv, positions, k_out,
                  v_out, stream=None) -> int:
    return _check(lib().srp_encode_kv(ctypes.byref(dims), int(n_rows), int(max_position),
                                      _ptr(hidden), _ptr(w_qkv), _ptr(positions), _ptr(k_out),
                                      _ptr(v_out), _stream(stream)))


def srp_rerotate_kv(dims: Dims, batch: Batch, k_cache, stream=None) -> int:
    return _check(lib().srp_rerotate_kv(ctypes.byref(dims), ctypes.byref(batch), _ptr(k_cache),
                                        _stream(stream)))


def srp_residual_rmsnorm(dims: Dims, hidden, attn_out, sel_idx, sel_offsets, n_req: int,
                         sel_capacity: int, eps: float = 1e-6, stream=None) -> int:
    return _check(lib().srp_residual_rmsnorm(ctypes.byref(dims), _ptr(hidden), _ptr(attn_out),
                                             _ptr(sel_idx), _ptr(sel_offsets), int(n_req),
                                             int(sel_capacity), float(eps), _stream(stream)))


def make_layer(w_qkv, k_cache, v_cache, ratio: float, k_host=None, v_host=None,
               mode=SRP_SEL_TOPK) -> Layer:
    """Layer descriptor for srp_fuse_stack; k_host / v_host are host tensors in
    page-locked memory (torch pin_memory=True) or None when the device caches are
    already filled; mode (layers after the first): SRP_SEL_TOPK checks the layer,
    SRP_SEL_GIVEN recomputes the previous layer's selection as it is."""
    return Layer(_ptr(w_qkv), _ptr(k_cache), _ptr(v_cache), _ptr(k_host), _ptr(v_host), float(ratio),
                 int(mode))


def srp_stack_workspace_size(dims: Dims, batch: Batch, first: Select) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().srp_stack_workspace_size(ctypes.byref(dims), ctypes.byref(batch), ctypes.byref(first),
                                          ctypes.byref(n)))
    return n.value


def srp_fuse_stack(dims: Dims, batch: Batch, first: Select, layers, hidden, rms_eps: float,
                   sel_idx, sel_offsets, attn_out, workspace, workspace_bytes: int, stream=None,
                   copy_stream=None) -> int:
    """layers: a sequence of Layer. copy_stream None = the compute stream (in line)."""
    arr = (Layer * len(layers))(*layers)
    st = _stream(stream)
    cs = st if copy_stream is None else _stream(copy_stream)
    return _check(lib().srp_fuse_stack(ctypes.byref(dims), ctypes.byref(batch), ctypes.byref(first),
                                       len(layers), arr, _ptr(hidden), float(rms_eps), _ptr(sel_idx),
                                       _ptr(sel_offsets), _ptr(attn_out), _ptr(workspace),
                                       workspace_bytes, st, cs))


def srp_controller_ratio(full_layer_ms: float, load_ms: float, r_floor: float = 0.15) -> float:
    r = ctypes.c_double(0.0)
    _check(lib().srp_controller_ratio(float(full_layer_ms), float(load_ms), float(r_floor), ctypes.byref(r)))
    return r.value


def srp_validate_batch(batch: Batch, stream=None) -> int:
    return _check(lib().srp_validate_batch(ctypes.byref(batch), _stream(stream)))


def srp_profile_begin(max_calls: int) -> int:
    return _check(lib().srp_profile_begin(int(max_calls)))


def srp_profile_end(max_calls: int):
    """Per-call stage times in ms: list of lists [call][stage]."""
    buf = (ctypes.c_float * (max_calls * SRP_N_STAGES))()
    n = ctypes.c_int32(0)
    _check(lib().srp_profile_end(buf, int(max_calls), ctypes.byref(n)))
    return [[buf[c * SRP_N_STAGES + i] for i in range(SRP_N_STAGES)] for c in range(n.value)]


def srp_profile_stage_name(i: int) -> str:
    return lib().srp_profile_stage_name(int(i)).decode()


def srp_version() -> str:
    return lib().srp_version().decode()
