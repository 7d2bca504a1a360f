"""Seeded, counter-based synthetic inputs shared by the oracle and the GPU path.

Holds no attention arithmetic: Philox4x32-10 + Box-Muller normals (synth_core.h),
uniform integer chunk lengths and a needle index.  Element e of tensor `tid`
under `seed` is the same value on the host (numpy) and on the device (filled in
place by a HIP kernel), so very large caches are filled on the GPU while the
host regenerates just the slabs it needs.
"""
import ctypes
import os

import numpy as np

from . import build as _build

# Tensor ids (the third counter word).
TID_Q = 1
TID_K = 2
TID_V = 3
TID_QDEC = 4
TID_LENGTHS = 5
TID_NEEDLE = 6
TID_DO = 7      # output gradients of the backward

F32, BF16, F64 = 0, 1, 2

_host = None
_dev = None


def _host_lib():
    global _host
    if _host is None:
        if not os.path.exists(_build.HOST_LIB):
            _build.build_host()
        lib = ctypes.CDLL(_build.HOST_LIB)
        lib.synth_fill_normal.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                          ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint32,
                                          ctypes.c_double]
        lib.synth_fill_normal.restype = ctypes.c_int
        lib.synth_philox_block.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        lib.synth_philox_block.restype = None
        lib.synth_log_host.argtypes = [ctypes.c_double]
        lib.synth_log_host.restype = ctypes.c_double
        lib.synth_sincos_quarter_host.argtypes = [ctypes.c_double, ctypes.c_void_p,
                                                  ctypes.c_void_p]
        lib.synth_sincos_quarter_host.restype = None
        lib.synth_chunk_offsets.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                            ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64,
                                            ctypes.c_uint32]
        lib.synth_chunk_offsets.restype = ctypes.c_int64
        lib.synth_pick_index.argtypes = [ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32]
        lib.synth_pick_index.restype = ctypes.c_int64
        _host = lib
    return _host


def _device_lib():
    global _dev
    if _dev is None:
        import torch  # noqa: F401  (load torch's HIP runtime first: one runtime per process)
        if not os.path.exists(_build.DEVICE_LIB):
            raise RuntimeError("libsynth_device.so is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(_build.DEVICE_LIB)
        lib.synth_fill_normal_device.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64,
                                                 ctypes.c_uint64, ctypes.c_uint64,
                                                 ctypes.c_uint32, ctypes.c_double,
                                                 ctypes.c_void_p]
        lib.synth_fill_normal_device.restype = ctypes.c_int
        _dev = lib
    return _dev


_NP = {F32: np.float32, BF16: np.uint16, F64: np.float64}


def normal(shape, dtype, seed, tid, scale=1.0, first=0):
    """numpy array of `shape`: elements first.. of tensor `tid`, scale*N(0,1),
    rounded to fp32 (F32), bf16 bits as uint16 (BF16) or kept in double (F64)."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=_NP[dtype])
    rc = _host_lib().synth_fill_normal(out.ctypes.data, dtype, first, n, seed, tid, scale)
    if rc != 0:
        raise ValueError("synth_fill_normal failed")
    return out.reshape(shape)


def normal_device(tensor, seed, tid, scale=1.0, first=0):
    """Fill a contiguous float32 or bfloat16 torch device tensor in place with
    the same values normal() returns for that dtype."""
    import torch
    if not tensor.is_contiguous() or tensor.device.type != "cuda":
        raise ValueError("need a contiguous device tensor")
    dt = {torch.float32: F32, torch.bfloat16: BF16}[tensor.dtype]
    stream = torch.cuda.current_stream(tensor.device).cuda_stream
    rc = _device_lib().synth_fill_normal_device(tensor.data_ptr(), dt, first, tensor.numel(),
                                                seed, tid, scale, stream)
    if rc != 0:
        raise RuntimeError(f"synth_fill_normal_device failed ({rc})")
    return tensor


def philox_block(ctr, key):
    c = (ctypes.c_uint32 * 4)(*ctr)
    k = (ctypes.c_uint32 * 2)(*key)
    o = (ctypes.c_uint32 * 4)()
    _host_lib().synth_philox_block(c, k, o)
    return list(o)


def log_(x):
    return _host_lib().synth_log_host(x)


def sincos_quarter(a):
    s, c = ctypes.c_double(), ctypes.c_double()
    _host_lib().synth_sincos_quarter_host(a, ctypes.byref(s), ctypes.byref(c))
    return s.value, c.value


def chunk_offsets(L, lo, hi, seed, tid=TID_LENGTHS):
    """int32 offsets [n+1] of i.i.d. U{lo..hi} chunk lengths summing to L."""
    max_chunks = L // lo + 2 if lo > 0 else 1
    buf = np.zeros(max_chunks + 1, dtype=np.int32)
    n = _host_lib().synth_chunk_offsets(buf.ctypes.data, max_chunks, L, lo, hi, seed, tid)
    if n < 0:
        raise ValueError("bad chunk length arguments")
    return buf[: n + 1].copy()


def pick_index(n, seed, tid=TID_NEEDLE):
    return int(_host_lib().synth_pick_index(n, seed, tid))


def bf16_to_f32(bits):
    """uint16 bf16 bits -> float32 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def f32_to_bf16(x):
    """float32 -> bf16 bits, round to nearest even (no NaN)."""
    b = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = b + 0x7FFF + ((b >> 16) & 1)
    return (b >> 16).astype(np.uint16)


def needle_key(q_group_bits_or_f32, is_bf16, scale=3.0):
    """The planted needle key for one KV group: scale * u/|u| with u the sum of
    the group's query rows (computed in double), rounded to the input dtype.
    Returns bf16 bits (uint16) or float32."""
    q = bf16_to_f32(q_group_bits_or_f32) if is_bf16 else np.asarray(q_group_bits_or_f32,
                                                                     np.float32)
    u = q.astype(np.float64).sum(axis=0)
    k = (scale * u / np.sqrt((u * u).sum())).astype(np.float32)
    return f32_to_bf16(k) if is_bf16 else k
