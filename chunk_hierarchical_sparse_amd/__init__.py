"""Hierarchical sparse attention (HSA / DHSA) forward pass for MI355X (gfx950).

A thin ctypes binding over libhsa_attn.so, whose C ABI is declared in
include/hsa_attn.h.  Python only marshals arguments: it checks tensors,
allocates outputs and workspaces with torch (device memory) and passes raw
pointers plus torch's current HIP stream.  Every step of the computation runs
in the library's HIP kernels; there is no other code path.  If the library is
not built, every call raises.
"""
import ctypes
import os

import torch  # loaded first: the library binds to the HIP runtime torch has loaded

from . import build as _build

__all__ = [
    "HsaError", "hsa_status_string", "hsa_build_landmarks", "hsa_prefill",
    "hsa_prefill_workspace_size", "hsa_decode", "hsa_decode_workspace_size",
    "hsa_decode_noalloc", "HSA_DECODE_NOALLOC_SCRATCH_BYTES", "hsa_swa_decode", "hsa_swa_prefill",
    "hsa_swa_decode_workspace_size",
    "hsa_prefill_interval", "hsa_prefill_interval_workspace_size", "hsa_prefill_backward",
    "hsa_prefill_backward_workspace_size", "dhsa_prefill",
    "dhsa_prefill_workspace_size", "dhsa_build_chunk_keys", "dhsa_decode",
    "dhsa_decode_workspace_size", "swa_prefill", "swa_decode", "hsa_profile_enable",
    "hsa_profile_read", "lib_path", "load_library", "hsa_device_checks_enabled",
    "hsa_device_checks_selftest",
]

HSA_OK = 0
HSA_ERR_INVALID_ARGUMENT = 1
HSA_ERR_UNSUPPORTED = 2
HSA_ERR_WORKSPACE_TOO_SMALL = 3
HSA_ERR_HIP = 4

DTYPE_F32 = 0
DTYPE_BF16 = 1

# fixed device scratch of hsa_decode_noalloc (include/hsa_attn.h)
HSA_DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20

_P = ctypes.c_void_p
_I = ctypes.c_int
_L = ctypes.c_int64
_Z = ctypes.c_size_t

_lib = None


class HsaError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{hsa_status_string(status)} ({message})")
        self.status = status


def lib_path():
    """The library this process loads: libhsa_attn.so, or the debug library
    with device checks (libhsa_attn_debug.so) when HSA_ATTN_DEBUG=1."""
    return _build.LIB_DEBUG if os.environ.get("HSA_ATTN_DEBUG", "0") == "1" else _build.LIB


def load_library():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    path = lib_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build() "
                           "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    sig = {
        "hsa_status_string": ([_I], ctypes.c_char_p),
        "hsa_last_error_message": ([], ctypes.c_char_p),
        "hsa_build_landmarks": ([_P, _P, _I, _I, _L, _I, _I, _L, _L, _I, _P], _I),
        "hsa_prefill_workspace_size": ([_I, _L, _I, _I, _I, _I, _I, _I], _Z),
        "hsa_prefill": ([_P, _P, _P, _P, _P, _P, _P, _I, _L, _I, _I, _I, _I, _I, _I, _P, _Z,
                         _P], _I),
        "hsa_prefill_interval_workspace_size": ([_I, _L, _I, _I, _I, _I, _I, _I, _I], _Z),
        "hsa_prefill_interval": ([_P, _P, _P, _P, _P, _P, _P, _I, _L, _I, _I, _I, _I, _I, _I,
                                  _I, _P, _Z, _P], _I),
        "hsa_decode_workspace_size": ([_I, _I, _I, _I, _I, _I, _L], _Z),
        "hsa_decode": ([_P, _P, _P, _P, _L, _L, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I, _P, _Z,
                        _P], _I),
        "hsa_decode_noalloc": ([_P, _P, _P, _P, _L, _L, _P, _P, _P, _I, _I, _I, _I, _I, _I, _I,
                                _P], _I),
        "hsa_swa_decode_workspace_size": ([_I, _I, _I, _I, _I, _I, _L, _L], _Z),
        "hsa_swa_prefill": ([_P, _P, _P, _P, _L, _P, _P, _P, _P, _I, _L, _I, _I, _I, _I, _I, _I,
                             _P, _Z, _P], _I),
        "hsa_swa_decode": ([_P, _P, _P, _P, _L, _L, _L, _P, _P, _P, _P, _I, _I, _I, _I, _I, _I,
                            _I, _P, _Z, _P], _I),
        "dhsa_prefill_workspace_size": ([_I, _L, _I, _I, _I, _I], _Z),
        "dhsa_prefill": ([_P, _P, _P, _P, _I, _L, _P, _P, _P, _I, _L, _I, _I, _I, _P, _Z, _P],
                         _I),
        "dhsa_chunk_keys_workspace_size": ([_I], _Z),
        "dhsa_build_chunk_keys": ([_P, _P, _P, _I, _I, _I, _I, _I, _L, _I, _I, _I, _P, _Z, _P],
                                  _I),
        "dhsa_decode_workspace_size": ([_I, _I, _I, _I, _L, _L], _Z),
        "dhsa_decode": ([_P, _I, _P, _P, _L, _P, _I, _P, _I, _L, _P, _P, _I, _I, _I, _I, _P, _Z,
                         _P], _I),
        "hsa_prefill_backward_workspace_size": ([_I, _L, _I, _I, _I, _I, _I, _I], _Z),
        "hsa_prefill_backward": ([_P, _P, _P, _P, _P, _P, _P, _P, _I, _L, _I, _I, _I, _I, _I, _I,
                                  _P, _Z, _P], _I),
        "swa_prefill": ([_P, _P, _P, _P, _I, _L, _I, _I, _I, _L, _I, _P], _I),
        "swa_decode": ([_P, _P, _P, _L, _L, _L, _P, _I, _I, _I, _I, _I, _P], _I),
        "hsa_profile_enable": ([_I], _I),
        "hsa_profile_read": ([_P, _I, _P], _I),
        "hsa_device_checks_enabled": ([], _I),
        "hsa_device_checks_selftest": ([_I, _P], _I),
    }
    for name, (args, res) in sig.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def hsa_status_string(status):
    return load_library().hsa_status_string(status).decode()


def _check(status):
    if status != HSA_OK:
        msg = load_library().hsa_last_error_message().decode()
        raise HsaError(status, msg)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return DTYPE_F32
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _need(t, name, ndim, dtype=None):
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dim() != ndim or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {ndim}-d tensor")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}")


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(t):
    return torch.cuda.current_stream(t.device).cuda_stream


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace too small: need {nbytes} bytes")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def hsa_build_landmarks(K, S, chunk_begin=0, chunk_end=None, lmk=None):
    """Landmarks of K [B,Hkv,L,d]: fp32 [B,Hkv,L//S,d], the sum of each
    chunk's S keys / sqrt(S).  With `lmk` given, only chunks
    chunk_begin..chunk_end-1 are (re)written in place."""
    _need(K, "K", 4)
    B, Hkv, L, d = K.shape
    n = L // S
    if chunk_end is None:
        chunk_end = n
    if lmk is None:
        lmk = torch.empty((B, Hkv, n, d), dtype=torch.float32, device=K.device)
    _need(lmk, "lmk", 4, torch.float32)
    _check(load_library().hsa_build_landmarks(K.data_ptr(), lmk.data_ptr(), B, Hkv, L, d, S,
                                              chunk_begin, chunk_end, _dtype_code(K),
                                              _stream(K)))
    return lmk


def hsa_prefill_workspace_size(B, L, Hq, Hkv, d, S, topk, dtype):
    code = _dtype_code(torch.empty(0, dtype=dtype))
    return load_library().hsa_prefill_workspace_size(B, L, Hq, Hkv, d, S, topk, code)


def hsa_prefill(Q, K, V, S, topk, lmk=None, out=None, return_selection=False, workspace=None):
    """HSA prefill.  Q [B,Hq,L,d], K and V [B,Hkv,L,d] (same dtype).

    Returns O [B,Hq,L,d]; with return_selection also sel_idx int32
    [B,Hkv,L,topk] (-1 padded) and sel_w fp32 [B,Hq,L,topk]."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, Q.dtype)
    _need(V, "V", 4, Q.dtype)
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (B, Hkv, L, d) or V.shape != K.shape:
        raise ValueError("K and V must be [B,Hkv,L,d] matching Q")
    if lmk is not None:
        _need(lmk, "lmk", 4, torch.float32)
    if out is None:
        out = torch.empty_like(Q)
    sel_idx = sel_w = None
    if return_selection:
        sel_idx = torch.empty((B, Hkv, L, topk), dtype=torch.int32, device=Q.device)
        sel_w = torch.empty((B, Hq, L, topk), dtype=torch.float32, device=Q.device)
    lib = load_library()
    code = _dtype_code(Q)
    nbytes = lib.hsa_prefill_workspace_size(B, L, Hq, Hkv, d, S, topk, code)
    ws = _workspace(nbytes, Q.device, workspace) if nbytes else None
    _check(lib.hsa_prefill(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _ptr(lmk), out.data_ptr(),
                           _ptr(sel_idx), _ptr(sel_w), B, L, Hq, Hkv, d, S, topk, code, _ptr(ws),
                           nbytes, _stream(Q)))
    if return_selection:
        return out, sel_idx, sel_w
    return out


def hsa_prefill_interval_workspace_size(B, L, Hq, Hkv, d, S, topk, interval, dtype):
    code = _dtype_code(torch.empty(0, dtype=dtype))
    return load_library().hsa_prefill_interval_workspace_size(B, L, Hq, Hkv, d, S, topk,
                                                              interval, code)


def hsa_prefill_interval(Q, K, V, S, topk, interval, lmk=None, out=None,
                         return_selection=False, workspace=None):
    """HSA prefill with retrieval every `interval` tokens (token t reuses the
    selection made at (t // interval) * interval).

    Returns O [B,Hq,L,d]; with return_selection also sel_idx int32
    [B,Hkv,ceil(L/interval),topk] (one selection per block, -1 padded) and
    sel_w fp32 [B,Hq,L,topk]."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, Q.dtype)
    _need(V, "V", 4, Q.dtype)
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (B, Hkv, L, d) or V.shape != K.shape:
        raise ValueError("K and V must be [B,Hkv,L,d] matching Q")
    if lmk is not None:
        _need(lmk, "lmk", 4, torch.float32)
    if out is None:
        out = torch.empty_like(Q)
    sel_idx = sel_w = None
    if return_selection:
        nq = (L + interval - 1) // interval
        sel_idx = torch.empty((B, Hkv, nq, topk), dtype=torch.int32, device=Q.device)
        sel_w = torch.empty((B, Hq, L, topk), dtype=torch.float32, device=Q.device)
    lib = load_library()
    code = _dtype_code(Q)
    nbytes = lib.hsa_prefill_interval_workspace_size(B, L, Hq, Hkv, d, S, topk, interval, code)
    ws = _workspace(nbytes, Q.device, workspace) if nbytes else None
    _check(lib.hsa_prefill_interval(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _ptr(lmk),
                                    out.data_ptr(), _ptr(sel_idx), _ptr(sel_w), B, L, Hq, Hkv, d,
                                    S, topk, interval, code, _ptr(ws), nbytes, _stream(Q)))
    if return_selection:
        return out, sel_idx, sel_w
    return out


def hsa_decode_workspace_size(B, Hq, Hkv, d, S, topk, n_ctx):
    return load_library().hsa_decode_workspace_size(B, Hq, Hkv, d, S, topk, n_ctx)


def hsa_decode(q, Kc, Vc, lmk, n_ctx, S, topk, out=None, return_selection=False,
               workspace=None):
    """HSA decode.  q [B,Hq,d], caches Kc, Vc [B,Hkv,n_max,d], landmarks
    fp32 [B,Hkv,n_max//S,d]; the query sits at position n_ctx."""
    _need(q, "q", 3)
    _need(Kc, "Kc", 4, q.dtype)
    _need(Vc, "Vc", 4, q.dtype)
    _need(lmk, "lmk", 4, torch.float32)
    B, Hq, d = q.shape
    Hkv, n_max = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, Hkv, n_max, d) or Vc.shape != Kc.shape:
        raise ValueError("Kc and Vc must be [B,Hkv,n_max,d] matching q")
    if lmk.shape != (B, Hkv, n_max // S, d):
        raise ValueError("lmk must be [B,Hkv,n_max//S,d]")
    if out is None:
        out = torch.empty_like(q)
    sel_idx = sel_w = None
    if return_selection:
        sel_idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=q.device)
        sel_w = torch.empty((B, Hq, topk), dtype=torch.float32, device=q.device)
    lib = load_library()
    nbytes = lib.hsa_decode_workspace_size(B, Hq, Hkv, d, S, topk, n_ctx)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    _check(lib.hsa_decode(q.data_ptr(), Kc.data_ptr(), Vc.data_ptr(), lmk.data_ptr(), n_ctx,
                          n_max, out.data_ptr(), _ptr(sel_idx), _ptr(sel_w), B, Hq, Hkv, d, S,
                          topk, _dtype_code(q), _ptr(ws), nbytes, _stream(q)))
    if return_selection:
        return out, sel_idx, sel_w
    return out


def hsa_decode_noalloc(q, Kc, Vc, lmk, n_ctx, S, topk, out, sel_idx=None, sel_w=None):
    """hsa_decode without a workspace: the library's fixed per-device scratch
    array stands in for it, so the call allocates nothing.  The outputs are
    the caller's: out [B,Hq,d] like q, and optionally sel_idx int32
    [B,Hkv,topk] and sel_w fp32 [B,Hq,topk].  Calls that overlap on one GPU
    race on the scratch."""
    _need(q, "q", 3)
    _need(Kc, "Kc", 4, q.dtype)
    _need(Vc, "Vc", 4, q.dtype)
    _need(lmk, "lmk", 4, torch.float32)
    B, Hq, d = q.shape
    Hkv, n_max = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, Hkv, n_max, d) or Vc.shape != Kc.shape:
        raise ValueError("Kc and Vc must be [B,Hkv,n_max,d] matching q")
    if lmk.shape != (B, Hkv, n_max // S, d):
        raise ValueError("lmk must be [B,Hkv,n_max//S,d]")
    _need(out, "out", 3, q.dtype)
    if out.shape != q.shape:
        raise ValueError("out must be [B,Hq,d] like q")
    if sel_idx is not None:
        _need(sel_idx, "sel_idx", 3, torch.int32)
        if sel_idx.shape != (B, Hkv, topk):
            raise ValueError("sel_idx must be [B,Hkv,topk]")
    if sel_w is not None:
        _need(sel_w, "sel_w", 3, torch.float32)
        if sel_w.shape != (B, Hq, topk):
            raise ValueError("sel_w must be [B,Hq,topk]")
    _check(load_library().hsa_decode_noalloc(q.data_ptr(), Kc.data_ptr(), Vc.data_ptr(),
                                             lmk.data_ptr(), n_ctx, n_max, out.data_ptr(),
                                             _ptr(sel_idx), _ptr(sel_w), B, Hq, Hkv, d, S, topk,
                                             _dtype_code(q), _stream(q)))
    return out


def hsa_swa_prefill(Q, K, V, S, topk, window, lmk=None, out_hsa=None, out_swa=None,
                    return_selection=False, workspace=None):
    """HSA prefill and sliding-window prefill of the same Q [B,Hq,L,d], K, V
    [B,Hkv,L,d] in one pass (one attention launch for both when bf16 and
    S <= 64).  Returns (O_hsa, O_swa), plus sel_idx, sel_w with
    return_selection.  The workspace is hsa_prefill's."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, Q.dtype)
    _need(V, "V", 4, Q.dtype)
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (B, Hkv, L, d) or V.shape != K.shape:
        raise ValueError("K and V must be [B,Hkv,L,d] matching Q")
    if lmk is not None:
        _need(lmk, "lmk", 4, torch.float32)
    out_hsa = torch.empty_like(Q) if out_hsa is None else out_hsa
    out_swa = torch.empty_like(Q) if out_swa is None else out_swa
    sel_idx = sel_w = None
    if return_selection:
        sel_idx = torch.empty((B, Hkv, L, topk), dtype=torch.int32, device=Q.device)
        sel_w = torch.empty((B, Hq, L, topk), dtype=torch.float32, device=Q.device)
    lib = load_library()
    code = _dtype_code(Q)
    nbytes = lib.hsa_prefill_workspace_size(B, L, Hq, Hkv, d, S, topk, code)
    ws = _workspace(nbytes, Q.device, workspace) if nbytes else None
    _check(lib.hsa_swa_prefill(Q.data_ptr(), K.data_ptr(), V.data_ptr(), _ptr(lmk), window,
                               out_hsa.data_ptr(), out_swa.data_ptr(), _ptr(sel_idx),
                               _ptr(sel_w), B, L, Hq, Hkv, d, S, topk, code, _ptr(ws), nbytes,
                               _stream(Q)))
    if return_selection:
        return out_hsa, out_swa, sel_idx, sel_w
    return out_hsa, out_swa


def hsa_swa_decode_workspace_size(B, Hq, Hkv, d, S, topk, n_ctx, window):
    return load_library().hsa_swa_decode_workspace_size(B, Hq, Hkv, d, S, topk, n_ctx, window)


def hsa_swa_decode(q, Kc, Vc, lmk, n_ctx, S, topk, window, out_hsa=None, out_swa=None,
                   return_selection=False, workspace=None):
    """HSA decode and sliding-window decode of the same query in one pass.
    q [B,Hq,d] at position n_ctx; caches Kc, Vc [B,Hkv,n_max,d] holding
    tokens 0..n_ctx; landmarks fp32 [B,Hkv,n_max//S,d].  Returns (o_hsa,
    o_swa), plus sel_idx, sel_w with return_selection."""
    _need(q, "q", 3)
    _need(Kc, "Kc", 4, q.dtype)
    _need(Vc, "Vc", 4, q.dtype)
    _need(lmk, "lmk", 4, torch.float32)
    B, Hq, d = q.shape
    Hkv, n_max = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, Hkv, n_max, d) or Vc.shape != Kc.shape:
        raise ValueError("Kc and Vc must be [B,Hkv,n_max,d] matching q")
    if lmk.shape != (B, Hkv, n_max // S, d):
        raise ValueError("lmk must be [B,Hkv,n_max//S,d]")
    out_hsa = torch.empty_like(q) if out_hsa is None else out_hsa
    out_swa = torch.empty_like(q) if out_swa is None else out_swa
    sel_idx = sel_w = None
    if return_selection:
        sel_idx = torch.empty((B, Hkv, topk), dtype=torch.int32, device=q.device)
        sel_w = torch.empty((B, Hq, topk), dtype=torch.float32, device=q.device)
    lib = load_library()
    nbytes = lib.hsa_swa_decode_workspace_size(B, Hq, Hkv, d, S, topk, n_ctx, window)
    ws = _workspace(nbytes, q.device, workspace) if nbytes else None
    _check(lib.hsa_swa_decode(q.data_ptr(), Kc.data_ptr(), Vc.data_ptr(), lmk.data_ptr(), n_ctx,
                              n_max, window, out_hsa.data_ptr(), out_swa.data_ptr(),
                              _ptr(sel_idx), _ptr(sel_w), B, Hq, Hkv, d, S, topk,
                              _dtype_code(q), _ptr(ws), nbytes, _stream(q)))
    if return_selection:
        return out_hsa, out_swa, sel_idx, sel_w
    return out_hsa, out_swa


def dhsa_prefill_workspace_size(B, L, H, d, n_chunks, dtype):
    code = _dtype_code(torch.empty(0, dtype=dtype))
    return load_library().dhsa_prefill_workspace_size(B, L, H, d, n_chunks, code)


def dhsa_prefill(Q, K, V, offsets, budget, out=None, return_mask=False, return_order=False,
                 workspace=None):
    """DHSA prefill.  Q, K, V [B,H,L,d] fp32 or bf16; offsets: host int32 chunk
    boundaries [n+1] (0 .. L); budget N_b.

    Returns O, plus the uint32 mask bits [B,H,L,ceil(L/32)] and/or the chunk
    order int32 [B,H,n,n] when requested."""
    import numpy as np
    _need(Q, "Q", 4)
    _need(K, "K", 4, Q.dtype)
    _need(V, "V", 4, Q.dtype)
    B, H, L, d = Q.shape
    if K.shape != Q.shape or V.shape != Q.shape:
        raise ValueError("Q, K and V must have the same shape")
    offs = np.ascontiguousarray(offsets, dtype=np.int32)
    nc = len(offs) - 1
    if out is None:
        out = torch.empty_like(Q)
    mask = order = None
    if return_mask:
        mask = torch.empty((B, H, L, (L + 31) // 32), dtype=torch.int32, device=Q.device)
    if return_order:
        order = torch.empty((B, H, nc, nc), dtype=torch.int32, device=Q.device)
    lib = load_library()
    code = _dtype_code(Q)
    nbytes = lib.dhsa_prefill_workspace_size(B, L, H, d, nc, code)
    ws = _workspace(nbytes, Q.device, workspace) if nbytes else None
    _check(lib.dhsa_prefill(Q.data_ptr(), K.data_ptr(), V.data_ptr(), offs.ctypes.data, nc,
                            budget, out.data_ptr(), _ptr(mask), _ptr(order), B, L, H, d, code,
                            _ptr(ws), nbytes, _stream(Q)))
    res = [out]
    if return_mask:
        res.append(mask)
    if return_order:
        res.append(order)
    return res[0] if len(res) == 1 else tuple(res)


def dhsa_build_chunk_keys(K, offsets, chunk_begin=0, chunk_end=None, khat=None, n_cap=None):
    """Pooled keys of the complete chunks given by host offsets [n+1]:
    fp32 [B,H,n_cap,d] (default n_cap = n), row k = (sum of chunk k's keys)
    / sqrt|C_k|.  With `khat` given, only chunks chunk_begin..chunk_end-1
    are (re)written in place."""
    import numpy as np
    _need(K, "K", 4)
    B, H, n_max, d = K.shape
    offs = np.ascontiguousarray(offsets, dtype=np.int32)
    n = len(offs) - 1
    if chunk_end is None:
        chunk_end = n
    if khat is None:
        n_cap = n if n_cap is None else n_cap
        khat = torch.zeros((B, H, max(n_cap, 1), d), dtype=torch.float32, device=K.device)
    else:
        _need(khat, "khat", 4, torch.float32)
        n_cap = khat.shape[2]
    lib = load_library()
    nbytes = lib.dhsa_chunk_keys_workspace_size(chunk_end - chunk_begin)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=K.device)
    _check(lib.dhsa_build_chunk_keys(K.data_ptr(), khat.data_ptr(), offs.ctypes.data, n,
                                     chunk_begin, chunk_end, B, H, n_max, d, n_cap,
                                     _dtype_code(K), ws.data_ptr(), nbytes, _stream(K)))
    return khat


def dhsa_decode_workspace_size(B, H, d, n_chunks, budget, n_max):
    return load_library().dhsa_decode_workspace_size(B, H, d, n_chunks, budget, n_max)


def dhsa_decode(q_cur, Kc, Vc, khat, offsets, budget, out=None, return_order=False,
                workspace=None):
    """DHSA decode of the new query at position offsets[-1] + m - 1.
    q_cur [B,H,m,d]: the current chunk's queries (new query last); Kc, Vc
    [B,H,n_max,d] caches; khat fp32 [B,H,n_cap,d] (dhsa_build_chunk_keys);
    offsets: host int32 boundaries [n+1] of the complete chunks; budget N_b.

    Returns o [B,H,d], plus the chunk order int32 [B,H,n+1] when requested."""
    import numpy as np
    _need(q_cur, "q_cur", 4)
    _need(Kc, "Kc", 4, q_cur.dtype)
    _need(Vc, "Vc", 4, q_cur.dtype)
    _need(khat, "khat", 4, torch.float32)
    B, H, m, d = q_cur.shape
    n_max = Kc.shape[2]
    if Kc.shape != (B, H, n_max, d) or Vc.shape != Kc.shape:
        raise ValueError("Kc and Vc must be [B,H,n_max,d] like q_cur")
    offs = np.ascontiguousarray(offsets, dtype=np.int32)
    n = len(offs) - 1
    if out is None:
        out = torch.empty((B, H, d), dtype=q_cur.dtype, device=q_cur.device)
    order = None
    if return_order:
        order = torch.empty((B, H, n + 1), dtype=torch.int32, device=q_cur.device)
    lib = load_library()
    nbytes = lib.dhsa_decode_workspace_size(B, H, d, n, budget, n_max)
    ws = _workspace(nbytes, q_cur.device, workspace) if nbytes else None
    _check(lib.dhsa_decode(q_cur.data_ptr(), m, Kc.data_ptr(), Vc.data_ptr(), n_max,
                           khat.data_ptr(), khat.shape[2], offs.ctypes.data, n, budget,
                           out.data_ptr(), _ptr(order), B, H, d, _dtype_code(q_cur), _ptr(ws),
                           nbytes, _stream(q_cur)))
    return (out, order) if return_order else out


def hsa_prefill_backward_workspace_size(B, L, Hq, Hkv, d, S, topk, dtype):
    code = _dtype_code(torch.empty(0, dtype=dtype))
    return load_library().hsa_prefill_backward_workspace_size(B, L, Hq, Hkv, d, S, topk, code)


def hsa_prefill_backward(Q, K, V, dO, S, topk, lmk=None, workspace=None, grads=None):
    """Gradients (dQ, dK, dV) of sum(dO * hsa_prefill(Q, K, V, S, topk)), the
    top-K selection held fixed.  bf16, S <= 64."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, Q.dtype)
    _need(V, "V", 4, Q.dtype)
    _need(dO, "dO", 4, Q.dtype)
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (B, Hkv, L, d) or V.shape != K.shape or dO.shape != Q.shape:
        raise ValueError("K, V must be [B,Hkv,L,d] and dO [B,Hq,L,d] matching Q")
    if lmk is not None:
        _need(lmk, "lmk", 4, torch.float32)
    if grads is None:
        grads = (torch.empty_like(Q), torch.empty_like(K), torch.empty_like(V))
    dQ, dK, dV = grads
    lib = load_library()
    nbytes = lib.hsa_prefill_backward_workspace_size(B, L, Hq, Hkv, d, S, topk, _dtype_code(Q))
    ws = _workspace(nbytes, Q.device, workspace) if nbytes else None
    _check(lib.hsa_prefill_backward(Q.data_ptr(), K.data_ptr(), V.data_ptr(), dO.data_ptr(),
                                    _ptr(lmk), dQ.data_ptr(), dK.data_ptr(), dV.data_ptr(), B, L,
                                    Hq, Hkv, d, S, topk, _dtype_code(Q), _ptr(ws), nbytes,
                                    _stream(Q)))
    return dQ, dK, dV


def swa_prefill(Q, K, V, window, out=None):
    """Sliding-window attention over a whole sequence: row t attends keys
    max(0, t-window+1) .. t.  Q [B,Hq,L,d], K, V [B,Hkv,L,d]."""
    _need(Q, "Q", 4)
    _need(K, "K", 4, Q.dtype)
    _need(V, "V", 4, Q.dtype)
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    if K.shape != (B, Hkv, L, d) or V.shape != K.shape:
        raise ValueError("K and V must be [B,Hkv,L,d] matching Q")
    if out is None:
        out = torch.empty_like(Q)
    _check(load_library().swa_prefill(Q.data_ptr(), K.data_ptr(), V.data_ptr(), out.data_ptr(),
                                      B, L, Hq, Hkv, d, window, _dtype_code(Q), _stream(Q)))
    return out


def swa_decode(q, Kc, Vc, pos, window, out=None):
    """Sliding-window decode: the query at position pos over cache keys
    max(0, pos-window+1) .. pos.  q [B,Hq,d], Kc, Vc [B,Hkv,n_max,d] holding
    tokens 0..pos."""
    _need(q, "q", 3)
    _need(Kc, "Kc", 4, q.dtype)
    _need(Vc, "Vc", 4, q.dtype)
    B, Hq, d = q.shape
    Hkv, n_max = Kc.shape[1], Kc.shape[2]
    if Kc.shape != (B, Hkv, n_max, d) or Vc.shape != Kc.shape:
        raise ValueError("Kc and Vc must be [B,Hkv,n_max,d] matching q")
    if out is None:
        out = torch.empty_like(q)
    _check(load_library().swa_decode(q.data_ptr(), Kc.data_ptr(), Vc.data_ptr(), pos, n_max,
                                     window, out.data_ptr(), B, Hq, Hkv, d, _dtype_code(q),
                                     _stream(q)))
    return out


def hsa_profile_enable(enable=True):
    """Record per-stage HIP events in every following call on this thread."""
    _check(load_library().hsa_profile_enable(1 if enable else 0))


def hsa_profile_read(max_stages=8):
    """(number of recorded calls, list of summed per-stage milliseconds)."""
    buf = (ctypes.c_double * max_stages)()
    ns = ctypes.c_int(0)
    calls = load_library().hsa_profile_read(buf, max_stages, ctypes.byref(ns))
    return calls, [buf[i] for i in range(min(ns.value, max_stages))]


def hsa_device_checks_enabled():
    """True when the loaded library is the debug build with device checks."""
    return bool(load_library().hsa_device_checks_enabled())


def hsa_device_checks_selftest(fail_check, stream=None):
    """Run the debug library's one-check self-test kernel; returns the status
    (HSA_ERR_HIP when the check was made to fail, HSA_ERR_UNSUPPORTED in the
    release library)."""
    st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    return load_library().hsa_device_checks_selftest(1 if fail_check else 0, st)
