"""ctypes binding of libnsa.so: argument marshalling only.

Every function here has the name of the C entry point it calls (include/nsa.h)
and takes torch tensors where the C function takes device pointers.  Nothing is
computed in Python; a missing library raises instead of falling back.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB: Optional[ctypes.CDLL] = None

NSA_SUCCESS = 0
NSA_ERROR_INVALID_VALUE = 1
NSA_ERROR_UNSUPPORTED = 2
NSA_ERROR_WORKSPACE = 3
NSA_ERROR_HIP = 4


class NSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{status_name(status)}: {message}")
        self.status = status


class nsa_config_t(ctypes.Structure):
    _fields_ = [("l", ctypes.c_int32), ("d", ctypes.c_int32), ("l_sel", ctypes.c_int32),
                ("n_sel", ctypes.c_int32), ("n_local", ctypes.c_int32), ("force_initial", ctypes.c_int32),
                ("w", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class nsa_dims_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32)]


def make_config(l, d, l_sel, n_sel, n_local, force_initial, w, softmax_scale=0.0) -> nsa_config_t:
    return nsa_config_t(l, d, l_sel, n_sel, n_local, force_initial, w, softmax_scale)


class nsa_dsa_dims_t(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32), ("d_qk", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32)]


def make_dsa_dims(batch, num_heads, d_qk, d_v, idx_heads, idx_dim) -> nsa_dsa_dims_t:
    return nsa_dsa_dims_t(int(batch), int(num_heads), int(d_qk), int(d_v), int(idx_heads), int(idx_dim))


def make_dims(batch, num_q_heads, num_kv_heads, d_k, d_v) -> nsa_dims_t:
    return nsa_dims_t(batch, num_q_heads, num_kv_heads, d_k, d_v)


def lib_path() -> str:
    return os.path.join(_HERE, "libnsa.so")


_VP = ctypes.c_void_p
_SIGS = {
    "nsa_compress_kv": [_VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP],
    "nsa_compress_append": [_VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                            ctypes.c_size_t, _VP],
    "nsa_compress_append_workspace_size": [_VP, _VP, ctypes.POINTER(ctypes.c_size_t)],
    "nsa_decode_fwd": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int64, _VP, _VP, _VP, _VP, _VP,
                       _VP, ctypes.c_size_t, _VP],
    "nsa_decode_fwd_noalloc": [_VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int64, _VP, _VP, _VP,
                               _VP, _VP, _VP],
    "nsa_prefill_fwd": [_VP, _VP, ctypes.c_int64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                        _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "nsa_decode_workspace_size": [_VP, _VP, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)],
    "nsa_prefill_workspace_size": [_VP, _VP, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)],
    "nsa_prefill_bwd": [_VP, _VP, ctypes.c_int64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                        _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_size_t, _VP],
    "nsa_prefill_bwd_workspace_size": [_VP, _VP, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)],
    "nsa_compress_bwd": [_VP, _VP, ctypes.c_int64, ctypes.c_int32, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP,
                         ctypes.c_size_t, _VP],
    "nsa_compress_bwd_workspace_size": [_VP, _VP, ctypes.c_int64, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t)],
    "nsa_dsa_decode_fwd": [_VP, ctypes.c_int32, ctypes.c_float, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.c_int64, _VP,
                           _VP, _VP, ctypes.c_size_t, _VP],
    "nsa_dsa_decode_workspace_size": [_VP, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_size_t)],
    "nsa_set_phase_events": [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32],
    "nsa_set_phase_clock": [_VP, ctypes.c_size_t],
    "nsa_status_string": [ctypes.c_int],
    "nsa_last_error": [],
}
EXPORTS = tuple(_SIGS)


def load_library() -> ctypes.CDLL:
    """Load libnsa.so once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        p = lib_path()
        if not os.path.exists(p):
            raise RuntimeError(f"NSA HIP library not found at {p}; build it with "
                               "`python -m long_context_sparse_nsa_amd.build`")
        lib = ctypes.CDLL(p)
        for name, args in _SIGS.items():
            fn = getattr(lib, name)
            fn.argtypes = args
            fn.restype = ctypes.c_char_p if name in ("nsa_status_string", "nsa_last_error") else ctypes.c_int
        _LIB = lib
    return _LIB


def status_name(status: int) -> str:
    return load_library().nsa_status_string(int(status)).decode()


def nsa_status_string(status: int) -> str:
    return status_name(status)


def nsa_last_error() -> str:
    return load_library().nsa_last_error().decode()


def _check(status: int):
    if status != NSA_SUCCESS:
        raise NSAError(status, nsa_last_error())


_ITEM = {torch.bfloat16: 2, torch.int16: 2, torch.uint16: 2, torch.float32: 4, torch.int32: 4, torch.int64: 8,
         torch.uint8: 1, torch.int8: 1}
if hasattr(torch, "float8_e4m3fn"):
    _ITEM[torch.float8_e4m3fn] = 1


def _ptr(t: Optional[torch.Tensor], what: str, itemsize: Optional[int] = None, numel: Optional[int] = None):
    """Device pointer of a contiguous CUDA tensor (None -> NULL)."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what}: expected a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{what}: tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{what}: tensor must be contiguous")
    if itemsize is not None and _ITEM.get(t.dtype) != itemsize:
        raise ValueError(f"{what}: element size must be {itemsize} bytes (got {t.dtype})")
    if numel is not None and t.numel() < numel:
        raise ValueError(f"{what}: needs at least {numel} elements, has {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> Optional[ctypes.c_void_p]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def nsa_decode_workspace_size(dims: nsa_dims_t, cfg: nsa_config_t, max_seq_len: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().nsa_decode_workspace_size(ctypes.byref(dims), ctypes.byref(cfg), int(max_seq_len),
                                                    ctypes.byref(out)))
    return int(out.value)


def nsa_prefill_workspace_size(dims: nsa_dims_t, cfg: nsa_config_t, seq_len: int, compress_in_call: bool) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().nsa_prefill_workspace_size(ctypes.byref(dims), ctypes.byref(cfg), int(seq_len),
                                                     int(bool(compress_in_call)), ctypes.byref(out)))
    return int(out.value)


def nsa_compress_kv(dims, cfg, k, v, cu_seqlens, seq_lens, max_len, w_k, pe_k, w_v, pe_v, k_cmp, v_cmp, cu_cmp,
                    stream=None):
    lib = load_library()
    _check(lib.nsa_compress_kv(ctypes.byref(dims), ctypes.byref(cfg), _ptr(k, "k", 2), _ptr(v, "v", 2),
                               _ptr(cu_seqlens, "cu_seqlens", 8), _ptr(seq_lens, "seq_lens", 4), int(max_len),
                               _ptr(w_k, "w_k", 2), _ptr(pe_k, "pe_k", 2), _ptr(w_v, "w_v", 2), _ptr(pe_v, "pe_v", 2),
                               _ptr(k_cmp, "k_cmp", 2), _ptr(v_cmp, "v_cmp", 2), _ptr(cu_cmp, "cu_cmp", 8),
                               _stream(stream)))


def nsa_compress_append_workspace_size(dims: nsa_dims_t, cfg: nsa_config_t) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().nsa_compress_append_workspace_size(ctypes.byref(dims), ctypes.byref(cfg),
                                                             ctypes.byref(out)))
    return int(out.value)


def nsa_compress_append(dims, cfg, k, v, cu_seqlens, seq_lens, max_len, w_k, pe_k, w_v, pe_v, k_cmp, v_cmp, cu_cmp,
                        workspace, stream=None):
    lib = load_library()
    B = dims.batch
    _check(lib.nsa_compress_append(ctypes.byref(dims), ctypes.byref(cfg), _ptr(k, "k", 2), _ptr(v, "v", 2),
                                   _ptr(cu_seqlens, "cu_seqlens", 8, B + 1), _ptr(seq_lens, "seq_lens", 4, B),
                                   int(max_len), _ptr(w_k, "w_k", 2), _ptr(pe_k, "pe_k", 2), _ptr(w_v, "w_v", 2),
                                   _ptr(pe_v, "pe_v", 2), _ptr(k_cmp, "k_cmp", 2), _ptr(v_cmp, "v_cmp", 2),
                                   _ptr(cu_cmp, "cu_cmp", 8, B + 1), _ptr(workspace, "workspace"),
                                   workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                   _stream(stream)))


def nsa_decode_fwd(dims, cfg, q, k_cache, v_cache, k_cmp_cache, v_cmp_cache, seq_lens, cu_seqlens, cu_cmp,
                   max_seq_len, gates, out, sel_idx_out, workspace, stream=None, w_gate=None, b_gate=None):
    """gates=None with w_gate (and optionally b_gate) selects the in-kernel gate network."""
    lib = load_library()
    B, Hq, H = dims.batch, dims.num_q_heads, dims.num_kv_heads
    _check(lib.nsa_decode_fwd(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q, "q", 2, B * Hq * dims.d_k),
                              _ptr(k_cache, "k_cache", 2), _ptr(v_cache, "v_cache", 2),
                              _ptr(k_cmp_cache, "k_cmp_cache", 2), _ptr(v_cmp_cache, "v_cmp_cache", 2),
                              _ptr(seq_lens, "seq_lens", 4, B), _ptr(cu_seqlens, "cu_seqlens", 8, B + 1),
                              _ptr(cu_cmp, "cu_cmp", 8, B + 1), int(max_seq_len),
                              _ptr(gates, "gates", 4, B * Hq * 3), _ptr(w_gate, "w_gate", 2, Hq * 3 * dims.d_k),
                              _ptr(b_gate, "b_gate", 4, Hq * 3), _ptr(out, "out", 2, B * Hq * dims.d_v),
                              _ptr(sel_idx_out, "sel_idx_out", 4, B * H * cfg.n_sel),
                              _ptr(workspace, "workspace"),
                              workspace.numel() * workspace.element_size() if workspace is not None else 0,
                              _stream(stream)))


def nsa_decode_fwd_noalloc(dims, cfg, q, k_cache, v_cache, k_cmp_cache, v_cmp_cache, seq_lens, cu_seqlens, cu_cmp,
                           max_seq_len, gates, out, sel_idx_out, stream=None, w_gate=None, b_gate=None):
    """nsa_decode_fwd with the library's own device-resident scratch instead of a workspace."""
    lib = load_library()
    B, Hq, H = dims.batch, dims.num_q_heads, dims.num_kv_heads
    _check(lib.nsa_decode_fwd_noalloc(ctypes.byref(dims), ctypes.byref(cfg), _ptr(q, "q", 2, B * Hq * dims.d_k),
                                      _ptr(k_cache, "k_cache", 2), _ptr(v_cache, "v_cache", 2),
                                      _ptr(k_cmp_cache, "k_cmp_cache", 2), _ptr(v_cmp_cache, "v_cmp_cache", 2),
                                      _ptr(seq_lens, "seq_lens", 4, B), _ptr(cu_seqlens, "cu_seqlens", 8, B + 1),
                                      _ptr(cu_cmp, "cu_cmp", 8, B + 1), int(max_seq_len),
                                      _ptr(gates, "gates", 4, B * Hq * 3), _ptr(w_gate, "w_gate", 2, Hq * 3 * dims.d_k),
                                      _ptr(b_gate, "b_gate", 4, Hq * 3), _ptr(out, "out", 2, B * Hq * dims.d_v),
                                      _ptr(sel_idx_out, "sel_idx_out", 4, B * H * cfg.n_sel), _stream(stream)))


def nsa_prefill_fwd(dims, cfg, seq_len, q, k, v, k_cmp, v_cmp, w_k, pe_k, w_v, pe_v, gates, out, sel_idx_out,
                    workspace, stream=None, w_gate=None, b_gate=None, lse_out=None):
    """gates=None with w_gate (and optionally b_gate) selects the in-kernel gate network;
    lse_out (float32 [B, T, Hq, 3]) receives each branch's log-sum-exp."""
    lib = load_library()
    B, Hq, H, T = dims.batch, dims.num_q_heads, dims.num_kv_heads, int(seq_len)
    _check(lib.nsa_prefill_fwd(ctypes.byref(dims), ctypes.byref(cfg), T, _ptr(q, "q", 2, B * T * Hq * dims.d_k),
                               _ptr(k, "k", 2, B * H * T * dims.d_k), _ptr(v, "v", 2, B * H * T * dims.d_v),
                               _ptr(k_cmp, "k_cmp", 2), _ptr(v_cmp, "v_cmp", 2),
                               _ptr(w_k, "w_k", 2), _ptr(pe_k, "pe_k", 2), _ptr(w_v, "w_v", 2), _ptr(pe_v, "pe_v", 2),
                               _ptr(gates, "gates", 4, B * T * Hq * 3), _ptr(w_gate, "w_gate", 2, Hq * 3 * dims.d_k),
                               _ptr(b_gate, "b_gate", 4, Hq * 3), _ptr(out, "out", 2, B * T * Hq * dims.d_v),
                               _ptr(sel_idx_out, "sel_idx_out", 4, B * T * H * cfg.n_sel),
                               _ptr(lse_out, "lse_out", 4, B * T * Hq * 3), _ptr(workspace, "workspace"),
                               workspace.numel() * workspace.element_size() if workspace is not None else 0,
                               _stream(stream)))


def nsa_prefill_bwd_workspace_size(dims: nsa_dims_t, cfg: nsa_config_t, seq_len: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().nsa_prefill_bwd_workspace_size(ctypes.byref(dims), ctypes.byref(cfg), int(seq_len),
                                                         ctypes.byref(out)))
    return int(out.value)


def nsa_prefill_bwd(dims, cfg, seq_len, q, k, v, k_cmp, v_cmp, gates, sel_idx, dout, dq, dk, dv, dk_cmp, dv_cmp,
                    dgates, workspace, stream=None, w_gate=None, b_gate=None, dw_gate=None, db_gate=None, lse=None):
    """Gradients of nsa_prefill_fwd; dq/dk/dv/dk_cmp/dv_cmp/dgates are float32 outputs.
    gates=None with w_gate (and optionally b_gate) differentiates through the gate network
    into dw_gate (float32 [Hq, 3, d_k]) and db_gate (float32 [Hq, 3]); lse is the forward's lse_out."""
    lib = load_library()
    B, Hq, H, T = dims.batch, dims.num_q_heads, dims.num_kv_heads, int(seq_len)
    nc = compressed_count(T, cfg.l, cfg.d)
    _check(lib.nsa_prefill_bwd(ctypes.byref(dims), ctypes.byref(cfg), T, _ptr(q, "q", 2, B * T * Hq * dims.d_k),
                               _ptr(k, "k", 2, B * H * T * dims.d_k), _ptr(v, "v", 2, B * H * T * dims.d_v),
                               _ptr(k_cmp, "k_cmp", 2, B * H * nc * dims.d_k),
                               _ptr(v_cmp, "v_cmp", 2, B * H * nc * dims.d_v),
                               _ptr(gates, "gates", 4, B * T * Hq * 3), _ptr(w_gate, "w_gate", 2, Hq * 3 * dims.d_k),
                               _ptr(b_gate, "b_gate", 4, Hq * 3), _ptr(sel_idx, "sel_idx", 4, B * T * H * cfg.n_sel),
                               _ptr(lse, "lse", 4, B * T * Hq * 3),
                               _ptr(dout, "dout", 2, B * T * Hq * dims.d_v),
                               _ptr(dq, "dq", 4, B * T * Hq * dims.d_k), _ptr(dk, "dk", 4, B * H * T * dims.d_k),
                               _ptr(dv, "dv", 4, B * H * T * dims.d_v),
                               _ptr(dk_cmp, "dk_cmp", 4, B * H * nc * dims.d_k),
                               _ptr(dv_cmp, "dv_cmp", 4, B * H * nc * dims.d_v),
                               _ptr(dgates, "dgates", 4, B * T * Hq * 3), _ptr(dw_gate, "dw_gate", 4, Hq * 3 * dims.d_k),
                               _ptr(db_gate, "db_gate", 4, Hq * 3), _ptr(workspace, "workspace"),
                               workspace.numel() * workspace.element_size() if workspace is not None else 0,
                               _stream(stream)))


def nsa_compress_bwd_workspace_size(dims: nsa_dims_t, cfg: nsa_config_t, seq_len: int, which: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().nsa_compress_bwd_workspace_size(ctypes.byref(dims), ctypes.byref(cfg), int(seq_len),
                                                          int(which), ctypes.byref(out)))
    return int(out.value)


def nsa_compress_bwd(dims, cfg, seq_len, which, x, w, pe, dy, dx, dw, dpe, workspace, stream=None):
    """which = 0: keys (d_k), 1: values (d_v).  dx is accumulated into; dw, dpe are written."""
    lib = load_library()
    B, H, T = dims.batch, dims.num_kv_heads, int(seq_len)
    D = dims.d_k if which == 0 else dims.d_v
    nc = compressed_count(T, cfg.l, cfg.d)
    _check(lib.nsa_compress_bwd(ctypes.byref(dims), ctypes.byref(cfg), T, int(which),
                                _ptr(x, "x", 2, B * H * T * D), _ptr(w, "w", 2, cfg.l * D * D),
                                _ptr(pe, "pe", 2, cfg.l * D), _ptr(dy, "dy", 4, B * H * nc * D),
                                _ptr(dx, "dx", 4, B * H * T * D), _ptr(dw, "dw", 4, cfg.l * D * D),
                                _ptr(dpe, "dpe", 4, cfg.l * D), _ptr(workspace, "workspace"),
                                workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                _stream(stream)))


def nsa_dsa_decode_workspace_size(dims: nsa_dsa_dims_t, top_k: int, cache_len: int) -> int:
    out = ctypes.c_size_t(0)
    _check(load_library().nsa_dsa_decode_workspace_size(ctypes.byref(dims), int(top_k), int(cache_len),
                                                        ctypes.byref(out)))
    return int(out.value)


def nsa_dsa_decode_fwd(dims, top_k, q, q_idx, w_idx, latent, k_idx, seq_lens, cache_len, out, sel_idx_out,
                       workspace, softmax_scale=0.0, stream=None):
    """q_idx / k_idx are uint8 tensors of FP8 E4M3 bit patterns."""
    lib = load_library()
    B, H = dims.batch, dims.num_heads
    _check(lib.nsa_dsa_decode_fwd(ctypes.byref(dims), int(top_k), float(softmax_scale),
                                  _ptr(q, "q", 2, B * H * dims.d_qk), _ptr(q_idx, "q_idx", 1, B * dims.idx_heads * dims.idx_dim),
                                  _ptr(w_idx, "w_idx", 4, B * dims.idx_heads),
                                  _ptr(latent, "latent", 2, B * int(cache_len) * dims.d_qk),
                                  _ptr(k_idx, "k_idx", 1, B * int(cache_len) * dims.idx_dim),
                                  _ptr(seq_lens, "seq_lens", 4, B), int(cache_len),
                                  _ptr(out, "out", 2, B * H * dims.d_v),
                                  _ptr(sel_idx_out, "sel_idx_out", 4, B * int(top_k)),
                                  _ptr(workspace, "workspace"),
                                  workspace.numel() * workspace.element_size() if workspace is not None else 0,
                                  _stream(stream)))


def nsa_set_phase_events(events=None):
    """Record 4 raw hipEvent_t handles (ints or c_void_p) between the kernels of each decode and
    prefill call on this thread; None disables."""
    if not events:
        _check(load_library().nsa_set_phase_events(None, 0))
        return
    arr = (ctypes.c_void_p * len(events))(*[e.value if isinstance(e, ctypes.c_void_p) else int(e) for e in events])
    _check(load_library().nsa_set_phase_events(arr, len(events)))


def nsa_set_phase_clock(buffer=None):
    """Record the decode kernels' per-workgroup phase clock into a device tensor of at
    least 1 MiB (uint64 ticks of the 100 MHz constant clock); None disables."""
    if buffer is None:
        _check(load_library().nsa_set_phase_clock(None, 0))
        return
    _check(load_library().nsa_set_phase_clock(_ptr(buffer, "buffer"), buffer.numel() * buffer.element_size()))


def compressed_count(L: int, l: int, d: int) -> int:
    """Complete compression blocks among L tokens (buffer sizing for callers)."""
    return (L - l) // d + 1 if L >= l else 0


def new_workspace(nbytes: int, device="cuda") -> torch.Tensor:
    """Workspace buffer of at least nbytes (contents on entry do not matter)."""
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)
