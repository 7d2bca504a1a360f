"""CPU oracle for hierarchical sparse attention (HSA) and DHSA.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  A thin ctypes
wrapper over hsa_oracle.c (plain C, double precision); see that file for the
step-by-step definitions and the pages each one follows.

Arrays are numpy: float32, or uint16 holding bfloat16 bits.  Results are
float64 (outputs, weights, margins) and int32 (indices).
"""
import ctypes
import os

import numpy as np

from . import build as _build

_lib = None
_F32, _BF16 = 0, 1

_P = ctypes.c_void_p
_I = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        L = ctypes.CDLL(_build.LIB)
        L.oracle_landmarks.argtypes = [_P, ctypes.c_int, _I, _I, _I, _I, _I, _P]
        L.oracle_hsa_prefill.argtypes = [_P, _P, _P, ctypes.c_int, _I, _I, _I, _I, _I, _I, _I,
                                         _P, _I, ctypes.c_int, _I, _P, _P, _P, _P, _P]
        L.oracle_hsa_decode_select.argtypes = [_P, ctypes.c_int, _P, _I, _I, _I, _I, _I, _I,
                                               _I, _I, _P, _P, _P]
        L.oracle_hsa_decode_attend.argtypes = [_P, _P, _P, ctypes.c_int, _P, _P, _I, _I, _I,
                                               _I, _I, _I, _P, _P]
        L.oracle_dhsa_prefill.argtypes = [_P, _P, _P, ctypes.c_int, _I, _I, _I, _I, _P, _I, _I,
                                          _P, _I, _P, _P, _P, _P, _P]
        L.oracle_dhsa_chunk_keys.argtypes = [_P, ctypes.c_int, _I, _I, _I, _I, _P, _I, _P]
        L.oracle_dhsa_decode.argtypes = [_P, _P, _P, ctypes.c_int, _I, _I, _I, _I, _I, _P, _I,
                                         _I, _P, _P, _P, _P, _P]
        L.oracle_swa_prefill.argtypes = [_P, _P, _P, ctypes.c_int, _I, _I, _I, _I, _I, _I, _P,
                                         _I, _P]
        L.oracle_swa_decode.argtypes = [_P, _P, _P, ctypes.c_int, _I, _I, _I, _I, _I, _I, _I,
                                        _P]
        L.oracle_hsa_prefill_backward.argtypes = [_P, _P, _P, _P, ctypes.c_int, _I, _I, _I, _I,
                                                  _I, _I, _I, _P, _I, _P, _P, _P]
        L.oracle_num_threads.argtypes = []
        for f in (L.oracle_num_threads, L.oracle_landmarks, L.oracle_hsa_prefill, L.oracle_hsa_decode_select,
                  L.oracle_hsa_decode_attend, L.oracle_dhsa_prefill, L.oracle_dhsa_chunk_keys,
                  L.oracle_dhsa_decode, L.oracle_swa_prefill, L.oracle_swa_decode,
                  L.oracle_hsa_prefill_backward):
            f.restype = ctypes.c_int
        _lib = L
    return _lib


def _dt(*arrays):
    kinds = {a.dtype for a in arrays}
    if kinds == {np.dtype(np.float32)}:
        return _F32
    if kinds == {np.dtype(np.uint16)}:
        return _BF16
    raise TypeError(f"inputs must all be float32 or all bf16 bits (uint16), got {kinds}")


def _c(a):
    return np.ascontiguousarray(a)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check(rc, what):
    if rc != 0:
        raise RuntimeError(f"{what} failed with code {rc}")


def num_threads():
    """Threads the oracle's OpenMP loops use."""
    return int(lib().oracle_num_threads())


def landmarks(K, S):
    """K [B,H,L,d] -> landmarks [B,H,L//S,d] float64: chunk key sums / sqrt(S)."""
    K = _c(K)
    B, H, L, d = K.shape
    out = np.zeros((B, H, L // S, d), np.float64)
    _check(lib().oracle_landmarks(K.ctypes.data, _dt(K), B, H, L, d, S, _ptr(out)), "landmarks")
    return out


def hsa_prefill(Q, K, V, S, topk, rows=None, include_current_chunk=False, want_out=True,
                retrieval_interval=1):
    """HSA prefill for query positions `rows` (default: all).  With
    retrieval_interval R > 1, row t reuses the selection made at
    t0 = (t // R) * R (sel, margin and sel_score describe that selection).

    Returns dict(out [B,Hq,R,d], sel [B,Hkv,R,K], w [B,Hq,R,K], margin [B,Hkv,R],
    sel_score [B,Hkv,R,K] group-summed score of each selected chunk)."""
    Q, K, V = _c(Q), _c(K), _c(V)
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    dt = _dt(Q, K, V)
    if rows is None:
        R = L
        rows_a = None
    else:
        rows_a = np.ascontiguousarray(rows, dtype=np.int64)
        R = len(rows_a)
    out = np.zeros((B, Hq, R, d), np.float64) if want_out else None
    sel = np.zeros((B, Hkv, R, topk), np.int32)
    w = np.zeros((B, Hq, R, topk), np.float64)
    margin = np.zeros((B, Hkv, R), np.float64)
    sel_score = np.zeros((B, Hkv, R, topk), np.float64)
    rc = lib().oracle_hsa_prefill(Q.ctypes.data, K.ctypes.data, V.ctypes.data, dt, B, L, Hq,
                                  Hkv, d, S, topk, _ptr(rows_a), R, int(include_current_chunk),
                                  int(retrieval_interval), _ptr(out), _ptr(sel), _ptr(w),
                                  _ptr(margin), _ptr(sel_score))
    _check(rc, "hsa_prefill")
    return dict(out=out, sel=sel, w=w, margin=margin, sel_score=sel_score)


def hsa_decode_select(q, lmk, S, n_ctx, topk, Hkv):
    """q [B,Hq,d]; lmk float32 [B,Hkv,n_lmk,d].  Returns (sel [B,Hkv,K],
    margin [B,Hkv], sel_score [B,Hkv,K])."""
    q = _c(q)
    lmk = np.ascontiguousarray(lmk, dtype=np.float32)
    B, Hq, d = q.shape
    n_lmk = lmk.shape[2]
    sel = np.zeros((B, Hkv, topk), np.int32)
    margin = np.zeros((B, Hkv), np.float64)
    sel_score = np.zeros((B, Hkv, topk), np.float64)
    rc = lib().oracle_hsa_decode_select(q.ctypes.data, _dt(q), lmk.ctypes.data, B, Hq, Hkv, d,
                                        S, n_ctx, n_lmk, topk, sel.ctypes.data,
                                        margin.ctypes.data, sel_score.ctypes.data)
    _check(rc, "hsa_decode_select")
    return sel, margin, sel_score


def hsa_decode_attend(q, Ksel, Vsel, lmk_sel, sel, S):
    """Ksel, Vsel [B,Hkv,K,S,d] selected chunks in selection order, lmk_sel
    float32 [B,Hkv,K,d], sel [B,Hkv,K].  Returns (out [B,Hq,d], w [B,Hq,K])."""
    q, Ksel, Vsel = _c(q), _c(Ksel), _c(Vsel)
    lmk_sel = np.ascontiguousarray(lmk_sel, dtype=np.float32)
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    B, Hq, d = q.shape
    Hkv, topk = sel.shape[1], sel.shape[2]
    out = np.zeros((B, Hq, d), np.float64)
    w = np.zeros((B, Hq, topk), np.float64)
    rc = lib().oracle_hsa_decode_attend(q.ctypes.data, Ksel.ctypes.data, Vsel.ctypes.data,
                                        _dt(q, Ksel, Vsel), lmk_sel.ctypes.data, sel.ctypes.data,
                                        B, Hq, Hkv, d, S, topk, out.ctypes.data, w.ctypes.data)
    _check(rc, "hsa_decode_attend")
    return out, w


def pack_selected(Kc, sel, S):
    """Gather the selected chunks of a full cache Kc [B,Hkv,N,d] into
    [B,Hkv,K,S,d] (zeros for -1 slots)."""
    B, Hkv, N, d = Kc.shape
    topk = sel.shape[2]
    out = np.zeros((B, Hkv, topk, S, d), Kc.dtype)
    for b in range(B):
        for g in range(Hkv):
            for k in range(topk):
                c = sel[b, g, k]
                if c >= 0:
                    out[b, g, k] = Kc[b, g, c * S:(c + 1) * S]
    return out


def hsa_decode(q, Kc, Vc, lmk, S, n_ctx, topk):
    """Full decode on caches small enough to hold on the host."""
    Hkv = Kc.shape[1]
    sel, margin, sel_score = hsa_decode_select(q, lmk, S, n_ctx, topk, Hkv)
    Ks, Vs = pack_selected(Kc, sel, S), pack_selected(Vc, sel, S)
    lmk = np.asarray(lmk, np.float32)
    B, _, _, d = lmk.shape
    lsel = np.zeros((B, Hkv, topk, d), np.float32)
    for b in range(B):
        for g in range(Hkv):
            for k in range(topk):
                if sel[b, g, k] >= 0:
                    lsel[b, g, k] = lmk[b, g, sel[b, g, k]]
    out, w = hsa_decode_attend(q, Ks, Vs, lsel, sel, S)
    return dict(out=out, w=w, sel=sel, margin=margin, sel_score=sel_score)


def dhsa_prefill(Q, K, V, offsets, budget, rows=None, want_sc=False, want_kept=False):
    """DHSA prefill for query positions `rows` (default: all).

    Returns dict(out [B,H,R,d], sc [B,H,nc,nc] or None, n_kept [B,H,R],
    kept [B,H,R,L] uint8 or None, margin [B,H,R])."""
    Q, K, V = _c(Q), _c(K), _c(V)
    B, H, L, d = Q.shape
    offs = np.ascontiguousarray(offsets, dtype=np.int32)
    nc = len(offs) - 1
    if rows is None:
        R, rows_a = L, None
    else:
        rows_a = np.ascontiguousarray(rows, dtype=np.int64)
        R = len(rows_a)
    out = np.zeros((B, H, R, d), np.float64)
    sc = np.zeros((B, H, nc, nc), np.float64) if want_sc else None
    n_kept = np.zeros((B, H, R), np.int32)
    kept = np.zeros((B, H, R, L), np.uint8) if want_kept else None
    margin = np.zeros((B, H, R), np.float64)
    rc = lib().oracle_dhsa_prefill(Q.ctypes.data, K.ctypes.data, V.ctypes.data, _dt(Q, K, V), B,
                                   L, H, d, offs.ctypes.data, nc, budget, _ptr(rows_a), R,
                                   out.ctypes.data, _ptr(sc), n_kept.ctypes.data, _ptr(kept),
                                   margin.ctypes.data)
    _check(rc, "dhsa_prefill")
    return dict(out=out, sc=sc, n_kept=n_kept, kept=kept, margin=margin)


def dhsa_chunk_keys(K, offsets):
    """k_hat [B,H,n,d] (float64) of the n complete chunks given by offsets[0..n]."""
    K = _c(K)
    B, H, N, d = K.shape
    offs = np.ascontiguousarray(offsets, dtype=np.int32)
    n = len(offs) - 1
    khat = np.zeros((B, H, n, d), np.float64)
    rc = lib().oracle_dhsa_chunk_keys(K.ctypes.data, _dt(K), B, H, N, d, offs.ctypes.data, n,
                                      khat.ctypes.data)
    _check(rc, "dhsa_chunk_keys")
    return khat


def dhsa_decode(Qcur, K, V, offsets, budget, want_kept=False):
    """DHSA decode of the new query at pos = offsets[-1] + m - 1, where
    Qcur [B,H,m,d] holds the current chunk's queries (the last row is the new
    query), K/V [B,H,N,d] caches and offsets[0..n] the complete chunks.

    Returns dict(out [B,H,d], sc [B,H,n+1], n_kept [B,H], kept [B,H,pos+1]
    uint8 or None, margin [B,H], pos)."""
    Qcur, K, V = _c(Qcur), _c(K), _c(V)
    B, H, m, d = Qcur.shape
    N = K.shape[2]
    offs = np.ascontiguousarray(offsets, dtype=np.int32)
    n = len(offs) - 1
    pos = int(offs[-1]) + m - 1
    out = np.zeros((B, H, d), np.float64)
    sc = np.zeros((B, H, n + 1), np.float64)
    n_kept = np.zeros((B, H), np.int32)
    kept = np.zeros((B, H, pos + 1), np.uint8) if want_kept else None
    margin = np.zeros((B, H), np.float64)
    rc = lib().oracle_dhsa_decode(Qcur.ctypes.data, K.ctypes.data, V.ctypes.data,
                                  _dt(Qcur, K, V), B, H, d, m, N, offs.ctypes.data, n, budget,
                                  out.ctypes.data, sc.ctypes.data, n_kept.ctypes.data, _ptr(kept),
                                  margin.ctypes.data)
    _check(rc, "dhsa_decode")
    return dict(out=out, sc=sc, n_kept=n_kept, kept=kept, margin=margin, pos=pos)


def swa_prefill(Q, K, V, window, rows=None):
    """Sliding-window causal attention: row t attends keys
    max(0, t-window+1) .. t.  Returns out [B,Hq,R,d] float64."""
    Q, K, V = _c(Q), _c(K), _c(V)
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    if rows is None:
        R, rows_a = L, None
    else:
        rows_a = np.ascontiguousarray(rows, dtype=np.int64)
        R = len(rows_a)
    out = np.zeros((B, Hq, R, d), np.float64)
    rc = lib().oracle_swa_prefill(Q.ctypes.data, K.ctypes.data, V.ctypes.data, _dt(Q, K, V), B,
                                  L, Hq, Hkv, d, window, _ptr(rows_a), R, out.ctypes.data)
    _check(rc, "swa_prefill")
    return out


def swa_decode(q, K, V, pos, window):
    """The query at position pos over cache keys max(0, pos-window+1) .. pos.
    q [B,Hq,d], K/V [B,Hkv,N,d].  Returns out [B,Hq,d] float64."""
    q, K, V = _c(q), _c(K), _c(V)
    B, Hq, d = q.shape
    Hkv, N = K.shape[1], K.shape[2]
    out = np.zeros((B, Hq, d), np.float64)
    rc = lib().oracle_swa_decode(q.ctypes.data, K.ctypes.data, V.ctypes.data, _dt(q, K, V), B,
                                 Hq, Hkv, d, N, pos, window, out.ctypes.data)
    _check(rc, "swa_decode")
    return out


def hsa_prefill_backward(Q, K, V, dO, S, topk, rows=None):
    """Gradients of sum(dO * out) for HSA prefill (per-token retrieval) with
    respect to Q, K, V, the top-K selection held fixed.  dO has Q's shape and
    dtype.  With `rows`, only those query positions' terms are taken (the
    gradient with dO zero elsewhere).  Returns dict(dQ [B,Hq,L,d],
    dK [B,Hkv,L,d], dV [B,Hkv,L,d]) float64."""
    Q, K, V, dO = _c(Q), _c(K), _c(V), _c(dO)
    B, Hq, L, d = Q.shape
    Hkv = K.shape[1]
    if dO.shape != Q.shape:
        raise ValueError("dO must have Q's shape")
    dQ = np.zeros(Q.shape, np.float64)
    dK = np.zeros(K.shape, np.float64)
    dV = np.zeros(V.shape, np.float64)
    rows_a = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    rc = lib().oracle_hsa_prefill_backward(Q.ctypes.data, K.ctypes.data, V.ctypes.data,
                                           dO.ctypes.data, _dt(Q, K, V, dO), B, L, Hq, Hkv, d,
                                           S, topk, _ptr(rows_a),
                                           0 if rows_a is None else len(rows_a),
                                           dQ.ctypes.data, dK.ctypes.data, dV.ctypes.data)
    _check(rc, "hsa_prefill_backward")
    return dict(dQ=dQ, dK=dK, dV=dV)
