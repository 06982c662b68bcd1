"""ctypes front end of the plain CPU oracle (``gmla_oracle.c``).

TEST INFRASTRUCTURE ONLY (tests, smoke check, CPU-baseline leg of the benchmark).

Every array handed to the C code is converted to C-contiguous float64 first: bf16
and fp32 inputs widen to double exactly, so the oracle sees the very values the GPU
library sees.  Nothing here computes attention itself; it only slices heads and
composes the C functions.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gmla_oracle.c")
_LIB = os.path.join(_HERE, "libgmla_oracle.so")

_lock = threading.Lock()
_loaded: dict[str, ctypes.CDLL] = {}

_c_i64 = ctypes.c_int64
_c_dbl_p = ctypes.POINTER(ctypes.c_double)
_c_i64_p = ctypes.POINTER(ctypes.c_int64)


def library_path() -> str:
    return _LIB


def default_threads() -> int:
    """Threads the oracle uses when asked for 0: the CPUs this process may run on,
    at most 16 (a GPU host's share per GPU)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def build(src: str = _SRC, out: str = _LIB, force: bool = True) -> str:
    """Compile the oracle with gcc into a shared library; returns its path.

    Plain optimisation only (-O2, no -ffast-math, no FMA contraction, no -march)
    so that the arithmetic is the C source's, in IEEE double.
    """
    if not force and os.path.exists(out) and os.path.getmtime(out) >= os.path.getmtime(src):
        return out
    tmp = out + f".tmp{os.getpid()}"
    cmd = ["gcc", "-std=c11", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared",
           "-pthread", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load(path: str | None = None) -> ctypes.CDLL:
    """Load (building first if missing or stale) the oracle library at ``path``."""
    path = path or _LIB
    with _lock:
        lib = _loaded.get(path)
        if lib is not None:
            return lib
        if path == _LIB:
            build(force=False)
        lib = ctypes.CDLL(path)
        lib.gmla_oracle_attend_head.restype = ctypes.c_int
        lib.gmla_oracle_attend_head.argtypes = [
            _c_i64, _c_i64, _c_i64, ctypes.c_double, ctypes.c_int,
            _c_dbl_p, _c_i64, _c_dbl_p, _c_i64, _c_dbl_p, _c_i64,
            _c_i64_p, _c_i64, _c_dbl_p, _c_dbl_p, _c_dbl_p, ctypes.c_int]
        lib.gmla_oracle_linear.restype = ctypes.c_int
        lib.gmla_oracle_linear.argtypes = [_c_i64, _c_i64, _c_i64, _c_dbl_p, _c_dbl_p, _c_dbl_p,
                                           ctypes.c_int]
        lib.gmla_oracle_gate.restype = ctypes.c_int
        lib.gmla_oracle_gate.argtypes = [_c_i64, _c_dbl_p, _c_dbl_p, _c_dbl_p]
        _loaded[path] = lib
        return lib


def _f64(a) -> np.ndarray:
    """float64, and C-contiguous along the last axis (row strides may be arbitrary)."""
    a = np.asarray(a, dtype=np.float64)
    if a.ndim == 0 or a.strides[-1] != 8:
        a = np.ascontiguousarray(a)
    return a


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_c_dbl_p)


def attend_head(q, k, v, scale: float, causal: bool, rows=None, want_lse: bool = False,
                want_probs: bool = False, nthreads: int = 0, lib=None):
    """Attention of one head: q [Tq, D] against k, v [Tk, D].

    Query i sits at absolute position i + Tk - Tq.  ``rows`` selects query indices
    (default: all).  Returns out [n, D] and, on request, lse [n] and probs [n, Tk].
    """
    lib = lib or load()
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 2 or k.ndim != 2 or v.ndim != 2:
        raise ValueError("attend_head takes 2-D q, k, v")
    Tq, D = q.shape
    Tk = k.shape[0]
    if k.shape[1] != D or v.shape != (Tk, D):
        raise ValueError("shape mismatch")
    if rows is None:
        rows_arr = None
        n = Tq
    else:
        rows_arr = np.ascontiguousarray(np.asarray(rows, dtype=np.int64))
        n = rows_arr.size
    out = np.empty((n, D), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64) if want_lse else None
    probs = np.empty((n, Tk), dtype=np.float64) if want_probs else None
    nthreads = nthreads or default_threads()
    rc = lib.gmla_oracle_attend_head(
        Tq, Tk, D, float(scale), 1 if causal else 0,
        _ptr(q), q.strides[0] // 8, _ptr(k), k.strides[0] // 8, _ptr(v), v.strides[0] // 8,
        rows_arr.ctypes.data_as(_c_i64_p) if rows_arr is not None else None, n,
        _ptr(out), _ptr(lse) if lse is not None else None,
        _ptr(probs) if probs is not None else None, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle attend_head failed (rc={rc})")
    res = [out]
    if want_lse:
        res.append(lse)
    if want_probs:
        res.append(probs)
    return res[0] if len(res) == 1 else tuple(res)


def attend(Q, K, V, scale: float, causal: bool = True, layout: str = "bthd", rows=None,
           nthreads: int = 0, lib=None) -> np.ndarray:
    """Multi-head attention, every head independent.

    layout "bthd": Q [B, Tq, H, D], K, V [B, Tk, H, D] (heads side by side on each token).
    layout "bhtd": Q [B, H, Tq, D], K, V [B, H, Tk, D].
    Returns O in Q's layout (only the ``rows`` query indices, if given, along the T axis).
    """
    Q, K, V = _f64(Q), _f64(K), _f64(V)
    if layout == "bthd":
        B, Tq, H, D = Q.shape
        n = Tq if rows is None else len(rows)
        out = np.empty((B, n, H, D), dtype=np.float64)
        for b in range(B):
            for h in range(H):
                out[b, :, h, :] = attend_head(Q[b, :, h, :], K[b, :, h, :], V[b, :, h, :], scale,
                                              causal, rows=rows, nthreads=nthreads, lib=lib)
    elif layout == "bhtd":
        B, H, Tq, D = Q.shape
        n = Tq if rows is None else len(rows)
        out = np.empty((B, H, n, D), dtype=np.float64)
        for b in range(B):
            for h in range(H):
                out[b, h] = attend_head(Q[b, h], K[b, h], V[b, h], scale, causal, rows=rows,
                                        nthreads=nthreads, lib=lib)
    else:
        raise ValueError(f"unknown layout {layout!r}")
    return out


def linear(X, W, nthreads: int = 0, lib=None) -> np.ndarray:
    """Y = X W^T with W stored [out, in]; X may have leading batch axes."""
    lib = lib or load()
    X = np.ascontiguousarray(np.asarray(X, dtype=np.float64))
    W = np.ascontiguousarray(np.asarray(W, dtype=np.float64))
    lead = X.shape[:-1]
    K = X.shape[-1]
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("linear: inner widths differ")
    M = int(np.prod(lead)) if lead else 1
    Y = np.empty((M, N), dtype=np.float64)
    nthreads = nthreads or default_threads()
    rc = lib.gmla_oracle_linear(M, N, K, _ptr(X), _ptr(W), _ptr(Y), int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle linear failed (rc={rc})")
    return Y.reshape(*lead, N)


def gate(G, O, lib=None) -> np.ndarray:
    """sigmoid(G) * O, elementwise (channel-wise gate)."""
    lib = lib or load()
    G = np.ascontiguousarray(np.asarray(G, dtype=np.float64))
    O = np.ascontiguousarray(np.asarray(O, dtype=np.float64))
    if G.shape != O.shape:
        raise ValueError("gate: shapes differ")
    out = np.empty_like(O)
    rc = lib.gmla_oracle_gate(O.size, _ptr(G), _ptr(O), _ptr(out))
    if rc != 0:
        raise ValueError("oracle gate failed")
    return out


def sigmoid(x, lib=None) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return gate(x, np.ones_like(x), lib=lib)


def gated_mla_layer(X, Wq, Wc, Wk, Wv, Wg, Wo, num_heads: int, causal: bool = True, rows=None,
                    nthreads: int = 0, lib=None, intermediates: bool = False) -> dict:
    """One Gated MLA layer in the "Gated MLA" page's implementation order.

    X [B, T, d_model].  Queries Q = X Wq^T; latent C = X Wc^T; keys K = C Wk^T and
    values V = C Wv^T; heads of width d_model / num_heads; causal attention with
    scale 1/sqrt(D_h); heads joined back to model width; gate sigmoid(X Wg^T)
    channel-wise; then the output projection Wo^T.  Returns {"output", "latent_cache"}
    (plus the intermediates on request).  ``rows`` restricts Q, the attention rows,
    the gate and the output to those token indices; C, K and V are always computed
    for every token, since any row may read them.
    """
    X = np.asarray(X, dtype=np.float64)
    B, T, dm = X.shape
    if num_heads <= 0 or dm % num_heads:
        raise ValueError("model width must be divisible by the positive head count")
    Dh = dm // num_heads
    Xr = X if rows is None else X[:, list(rows), :]
    C = linear(X, Wc, nthreads, lib)
    K = linear(C, Wk, nthreads, lib)
    V = linear(C, Wv, nthreads, lib)
    Q = linear(Xr, Wq, nthreads, lib)
    G = linear(Xr, Wg, nthreads, lib)
    n = Q.shape[1]
    Ot = np.empty((B, n, dm), dtype=np.float64)
    for b in range(B):
        for h in range(num_heads):
            sl = slice(h * Dh, (h + 1) * Dh)
            if rows is None:
                Ot[b, :, sl] = attend_head(Q[b, :, sl], K[b, :, sl], V[b, :, sl], 1.0 / np.sqrt(Dh),
                                           causal, nthreads=nthreads, lib=lib)
            else:
                # the query array holds only the selected rows; pad to full length so
                # each selected query keeps its absolute position
                qfull = np.zeros((T, Dh))
                qfull[list(rows)] = Q[b, :, sl]
                Ot[b, :, sl] = attend_head(qfull, K[b, :, sl], V[b, :, sl], 1.0 / np.sqrt(Dh),
                                           causal, rows=rows, nthreads=nthreads, lib=lib)
    gated = gate(G, Ot, lib)
    Y = linear(gated, Wo, nthreads, lib)
    res = {"output": Y, "latent_cache": C}
    if intermediates:
        res.update(Q=Q, K=K, V=V, G=G, O_tilde=Ot, gated=gated)
    return res
