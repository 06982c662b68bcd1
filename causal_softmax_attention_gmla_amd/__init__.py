"""Causal softmax attention for Gated MLA layers on one MI355X (gfx950).

Thin binding over libgmla.so (C ABI in include/gmla.h).  These functions check
that tensor shapes agree with the sizes they pass, allocate outputs with PyTorch
(device memory only), and hand raw device pointers plus the current HIP stream to
the library; every arithmetic step runs in the library's HIP kernels.

    attend_prefill(q, k, v, gate=None, scale=None, causal=True)   -> [B, T, H*D]
    attend_chunk(q, k, v, gate=None, scale=None, causal=True)     -> [B, Tq, H*D]
    attend_varlen(q, k, v, cu_q, cu_k, max_q, max_k, gate=None)   -> [total_q, H*D]
    attend_decode(q, k, v, gate=None, scale=None, num_splits=0)   -> [B, H*D]
    attend_decode_varlen(q, k, v, kv_lens, gate=None)             -> [B, H*D]
    attend_decode_latent(q, c, w_k, w_v, gate=None)               -> [B, H*D]
    latent_expand(c, w_k, w_v)                                    -> (K, V)
    gate_out(o_tilde, w_o=None, gate=None)                        -> Y
    linear(x, w)                                                  -> x w^T
    gated_mla(hidden_states, ..., num_heads, causal=True)         -> {"output", "latent_cache"}

Formulas: "Gated MLA" (ai-engineer-exhaustive.pages.dev, research/kimik3/k3-gated-mla),
sections "Start from familiar attention", "Split attention into heads", "The
channel-wise output gate", "Requirements"; "Kimi K3 - Softmax over keys" and "Kimi K2 -
Construct causal mask" (atlas.klimoza.dev).
"""
from __future__ import annotations

import ctypes
import math

import torch

from . import _lib
from ._lib import GMLA_BF16, GMLA_F32, GmlaError, LIB_PATH  # noqa: F401

__all__ = ["attend_prefill", "attend_prefill_latent", "prefill_latent_workspace_bytes", "attend_chunk", "attend_varlen", "attend_decode", "attend_decode_varlen",
           "attend_decode_latent", "latent_expand", "gate_out",
           "linear", "gated_mla", "decode_num_splits", "decode_workspace_bytes",
           "decode_latent_num_splits", "decode_latent_workspace_bytes", "library", "GmlaError"]

_DTYPES = {torch.float32: GMLA_F32, torch.bfloat16: GMLA_BF16}


def library():
    """The loaded ctypes handle of libgmla.so (raises if it is not built)."""
    return _lib.load()


def _dtype(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise TypeError(f"unsupported dtype {t.dtype}: float32 or bfloat16 only") from None


def _dev(*ts):
    dev = None
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("all tensors must be on the GPU")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError("all tensors must be on the same GPU")
    return dev


def _same_dtype(*ts):
    d = None
    for t in ts:
        if t is None:
            continue
        if d is None:
            d = t.dtype
        elif t.dtype != d:
            raise TypeError("all tensors must share one dtype")
    return d


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(dev, stream):
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


def attend_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor | None = None,
                   *, scale: float | None = None, causal: bool = True, out: torch.Tensor | None = None,
                   stream=None) -> torch.Tensor:
    """Attention of every query against keys 0..t (causal) or all keys.

    q, k, v: [B, T, H, D] with identical strides and a contiguous last axis (views
    into [B, T, H*D] projections are fine).  gate: optional [B, T, H*D] logits; the
    output is multiplied by sigmoid(gate) channel-wise.  Returns [B, T, H*D].
    """
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, T, H, D]")
    if k.stride() != q.stride() or v.stride() != q.stride() or q.stride(3) != 1:
        raise ValueError("q, k, v need identical strides and a contiguous last axis")
    if not isinstance(causal, bool):
        raise TypeError("causal must be a bool")
    B, T, H, D = q.shape
    dev = _dev(q, k, v, gate, out)
    _same_dtype(q, k, v, gate, out)
    if gate is not None and (gate.shape != (B, T, H * D) or not gate.is_contiguous()):
        raise ValueError("gate must be a contiguous [B, T, H*D] tensor")
    if out is None:
        out = torch.empty((B, T, H * D), dtype=q.dtype, device=dev)
    elif out.shape != (B, T, H * D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, T, H*D] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    strides = (ctypes.c_int64 * 3)(q.stride(0), q.stride(1), q.stride(2))
    st = _lib.load().gmla_attend_prefill(_dtype(q), B, T, H, D, float(scale), int(causal),
                                         _ptr(q), _ptr(k), _ptr(v), strides, _ptr(gate), _ptr(out),
                                         _stream(dev, stream))
    _lib.check(st, "gmla_attend_prefill")
    return out


def prefill_latent_workspace_bytes(B: int, T: int, H: int, D: int) -> int:
    return _lib.load().gmla_prefill_latent_workspace_bytes(B, T, H, D)


def attend_prefill_latent(q: torch.Tensor, latent: torch.Tensor, key_up_projection: torch.Tensor,
                          value_up_projection: torch.Tensor, gate: torch.Tensor | None = None, *,
                          scale: float | None = None, causal: bool = True,
                          workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                          stream=None) -> torch.Tensor:
    """Prefill whose keys and values are rebuilt from the latent rows when attention runs
    (K = C W_k^T, V = C W_v^T, "Gated MLA", "Start from familiar attention"), in one
    persistent launch; each head's keys and values are formed once, in the workspace.

    q: [B, T, H, D] with a contiguous last axis; latent: contiguous [B, T, d_c];
    up-projections contiguous [H*D, d_c]; gate: optional [B, T, H*D].  Returns
    [B, T, H*D].
    """
    if q.dim() != 4 or latent.dim() != 3:
        raise ValueError("q must be [B, T, H, D] and latent [B, T, d_c]")
    B, T, H, D = q.shape
    if latent.shape[:2] != (B, T):
        raise ValueError("q and latent disagree in batch or sequence length")
    d_c = latent.shape[2]
    for w in (key_up_projection, value_up_projection):
        if w.shape != (H * D, d_c) or not w.is_contiguous():
            raise ValueError("the up-projections must be contiguous [H*D, d_c]")
    if q.stride(3) != 1 or not latent.is_contiguous():
        raise ValueError("q needs a contiguous last axis and latent must be contiguous")
    if not isinstance(causal, bool):
        raise TypeError("causal must be a bool")
    dev = _dev(q, latent, key_up_projection, value_up_projection, gate, out, workspace)
    _same_dtype(q, latent, key_up_projection, value_up_projection, gate, out)
    if gate is not None and (gate.shape != (B, T, H * D) or not gate.is_contiguous()):
        raise ValueError("gate must be a contiguous [B, T, H*D] tensor")
    if out is None:
        out = torch.empty((B, T, H * D), dtype=q.dtype, device=dev)
    elif out.shape != (B, T, H * D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, T, H*D] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _lib.load()
    need = lib.gmla_prefill_latent_workspace_bytes(B, T, H, D)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    strides = (ctypes.c_int64 * 3)(q.stride(0), q.stride(1), q.stride(2))
    st = lib.gmla_attend_prefill_latent(_dtype(q), B, T, H, D, d_c, float(scale), int(causal),
                                        _ptr(q), strides, _ptr(latent), _ptr(key_up_projection),
                                        _ptr(value_up_projection), _ptr(gate), _ptr(out),
                                        _ptr(workspace), workspace.numel() * workspace.element_size(),
                                        _stream(dev, stream))
    _lib.check(st, "gmla_attend_prefill_latent")
    return out


def attend_chunk(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor | None = None,
                 *, scale: float | None = None, causal: bool = True, out: torch.Tensor | None = None,
                 stream=None) -> torch.Tensor:
    """Attention of Tq new queries that follow Tk - Tq cached tokens: query i sits at
    position i + Tk - Tq and (causal) sees keys 0..i + Tk - Tq.

    q: [B, Tq, H, D]; k, v: [B, Tk, H, D] (the cache followed by the chunk) with
    identical strides; every last axis contiguous.  gate: optional [B, Tq, H*D] logits.
    Returns [B, Tq, H*D].
    """
    if q.dim() != 4 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, Tq, H, D] and k, v [B, Tk, H, D]")
    B, Tq, H, D = q.shape
    Tk = k.shape[1]
    if (k.shape[0], k.shape[2], k.shape[3]) != (B, H, D):
        raise ValueError("q and k, v disagree in batch, heads or head width")
    if Tk < Tq:
        raise ValueError("the chunk cannot be longer than the key sequence")
    if k.stride() != v.stride() or k.stride(3) != 1 or q.stride(3) != 1:
        raise ValueError("k, v need identical strides; every last axis must be contiguous")
    if not isinstance(causal, bool):
        raise TypeError("causal must be a bool")
    dev = _dev(q, k, v, gate, out)
    _same_dtype(q, k, v, gate, out)
    if gate is not None and (gate.shape != (B, Tq, H * D) or not gate.is_contiguous()):
        raise ValueError("gate must be a contiguous [B, Tq, H*D] tensor")
    if out is None:
        out = torch.empty((B, Tq, H * D), dtype=q.dtype, device=dev)
    elif out.shape != (B, Tq, H * D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, Tq, H*D] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qs = (ctypes.c_int64 * 3)(q.stride(0), q.stride(1), q.stride(2))
    kvs = (ctypes.c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))
    st = _lib.load().gmla_attend_chunk(_dtype(q), B, Tq, Tk, H, D, float(scale), int(causal),
                                       _ptr(q), qs, _ptr(k), _ptr(v), kvs, _ptr(gate), _ptr(out),
                                       _stream(dev, stream))
    _lib.check(st, "gmla_attend_chunk")
    return out


def attend_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cu_seqlens_q: torch.Tensor,
                  cu_seqlens_k: torch.Tensor, max_seqlen_q: int | None = None,
                  max_seqlen_k: int | None = None, gate: torch.Tensor | None = None, *,
                  scale: float | None = None, causal: bool = True, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """Attention over a packed batch of sequences of different lengths: sequence b owns
    query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and key rows cu_seqlens_k[b] ..
    cu_seqlens_k[b+1]-1, and its query i sits at position i + Tk_b - Tq_b (bottom-right
    causal mask per sequence).  A query that sees no key gets zeros.

    q: [total_q, H, D]; k, v: [total_k, H, D] with identical strides; every last axis
    contiguous.  cu_seqlens_*: int32 device tensors [B + 1].  max_seqlen_q / _k: the
    longest sequences (read back from the offsets, a host sync, when omitted).  gate:
    optional [total_q, H*D].  Returns [total_q, H*D].
    """
    if q.dim() != 3 or k.dim() != 3 or v.shape != k.shape:
        raise ValueError("q must be [total_q, H, D] and k, v [total_k, H, D]")
    total_q, H, D = q.shape
    if (k.shape[1], k.shape[2]) != (H, D):
        raise ValueError("q and k, v disagree in heads or head width")
    if k.stride() != v.stride() or k.stride(2) != 1 or q.stride(2) != 1:
        raise ValueError("k, v need identical strides; every last axis must be contiguous")
    for cu in (cu_seqlens_q, cu_seqlens_k):
        if cu.dtype != torch.int32 or cu.dim() != 1 or not cu.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous 1-D int32 tensors")
    B = cu_seqlens_q.numel() - 1
    if B < 1 or cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    if not isinstance(causal, bool):
        raise TypeError("causal must be a bool")
    dev = _dev(q, k, v, cu_seqlens_q, cu_seqlens_k, gate, out)
    _same_dtype(q, k, v, gate, out)
    if max_seqlen_q is None:
        max_seqlen_q = int((cu_seqlens_q[1:] - cu_seqlens_q[:-1]).max().item())
    if max_seqlen_k is None:
        max_seqlen_k = int((cu_seqlens_k[1:] - cu_seqlens_k[:-1]).max().item())
    if gate is not None and (gate.shape != (total_q, H * D) or not gate.is_contiguous()):
        raise ValueError("gate must be a contiguous [total_q, H*D] tensor")
    if out is None:
        out = torch.empty((total_q, H * D), dtype=q.dtype, device=dev)
    elif out.shape != (total_q, H * D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [total_q, H*D] tensor")
    if max_seqlen_q == 0:
        return out
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    qs = (ctypes.c_int64 * 2)(q.stride(0), q.stride(1))
    kvs = (ctypes.c_int64 * 2)(k.stride(0), k.stride(1))
    st = _lib.load().gmla_attend_varlen(_dtype(q), B, H, D, float(scale), int(causal), _ptr(q), qs,
                                        _ptr(cu_seqlens_q), int(max_seqlen_q), _ptr(k), _ptr(v), kvs,
                                        _ptr(cu_seqlens_k), int(max_seqlen_k), _ptr(gate), _ptr(out),
                                        _stream(dev, stream))
    _lib.check(st, "gmla_attend_varlen")
    return out


def decode_num_splits(B: int, H: int, N: int, D: int) -> int:
    return _lib.load().gmla_decode_num_splits(B, H, N, D)


def decode_workspace_bytes(B: int, H: int, N: int, D: int, num_splits: int = 0) -> int:
    return _lib.load().gmla_decode_workspace_bytes(B, H, N, D, num_splits)


def attend_decode(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, gate: torch.Tensor | None = None,
                  *, scale: float | None = None, num_splits: int = 0,
                  workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                  stream=None) -> torch.Tensor:
    """One query per (batch, head) at position N-1 against N cached keys.

    q: [B, H, D] contiguous; k, v: [B, H, N, D] with identical strides and a
    contiguous last axis; gate: optional [B, H*D].  Returns [B, H*D].
    """
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, H, D] and k, v [B, H, N, D]")
    B, H, N, D = k.shape
    if q.shape != (B, H, D) or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, H, D] tensor")
    if k.stride() != v.stride() or k.stride(3) != 1:
        raise ValueError("k, v need identical strides and a contiguous last axis")
    dev = _dev(q, k, v, gate, out, workspace)
    _same_dtype(q, k, v, gate, out)
    if gate is not None and (gate.shape != (B, H * D) or not gate.is_contiguous()):
        raise ValueError("gate must be a contiguous [B, H*D] tensor")
    if out is None:
        out = torch.empty((B, H * D), dtype=q.dtype, device=dev)
    elif out.shape != (B, H * D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H*D] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _lib.load()
    need = lib.gmla_decode_workspace_bytes(B, H, N, D, num_splits)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    strides = (ctypes.c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))
    st = lib.gmla_attend_decode(_dtype(q), B, H, N, D, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                strides, _ptr(gate), _ptr(out), _ptr(workspace), ws_bytes,
                                int(num_splits), _stream(dev, stream))
    _lib.check(st, "gmla_attend_decode")
    return out


def attend_decode_varlen(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, kv_lens: torch.Tensor,
                         gate: torch.Tensor | None = None, *, scale: float | None = None,
                         num_splits: int = 0, workspace: torch.Tensor | None = None,
                         out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode with a cache length per batch row: row b's query sits at position
    kv_lens[b] - 1 and attends to keys 0 .. kv_lens[b] - 1 of its cache (values clamped to
    [0, N]; an empty row gives zeros).  q: [B, H, D]; k, v: [B, H, N, D] caches of
    capacity N; kv_lens: int32 device tensor [B].  Returns [B, H*D]."""
    if q.dim() != 3 or k.dim() != 4 or v.shape != k.shape:
        raise ValueError("q must be [B, H, D] and k, v [B, H, N, D]")
    B, H, N, D = k.shape
    if q.shape != (B, H, D) or not q.is_contiguous():
        raise ValueError("q must be a contiguous [B, H, D] tensor")
    if k.stride() != v.stride() or k.stride(3) != 1:
        raise ValueError("k, v need identical strides and a contiguous last axis")
    if kv_lens.dtype != torch.int32 or kv_lens.shape != (B,) or not kv_lens.is_contiguous():
        raise ValueError("kv_lens must be a contiguous int32 tensor [B]")
    dev = _dev(q, k, v, kv_lens, gate, out, workspace)
    _same_dtype(q, k, v, gate, out)
    if gate is not None and (gate.shape != (B, H * D) or not gate.is_contiguous()):
        raise ValueError("gate must be a contiguous [B, H*D] tensor")
    if out is None:
        out = torch.empty((B, H * D), dtype=q.dtype, device=dev)
    elif out.shape != (B, H * D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H*D] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _lib.load()
    need = lib.gmla_decode_workspace_bytes(B, H, N, D, num_splits)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    strides = (ctypes.c_int64 * 3)(k.stride(0), k.stride(1), k.stride(2))
    st = lib.gmla_attend_decode_varlen(_dtype(q), B, H, N, D, float(scale), _ptr(q), _ptr(k), _ptr(v),
                                       strides, _ptr(kv_lens), _ptr(gate), _ptr(out), _ptr(workspace),
                                       ws_bytes, int(num_splits), _stream(dev, stream))
    _lib.check(st, "gmla_attend_decode_varlen")
    return out


def decode_latent_num_splits(B: int, H: int, N: int, d_c: int) -> int:
    return _lib.load().gmla_decode_latent_num_splits(B, H, N, d_c)


def decode_latent_workspace_bytes(B: int, H: int, N: int, d_c: int, num_splits: int = 0) -> int:
    return _lib.load().gmla_decode_latent_workspace_bytes(B, H, N, d_c, num_splits)


def attend_decode_latent(q: torch.Tensor, latent_cache: torch.Tensor, key_up_projection: torch.Tensor,
                         value_up_projection: torch.Tensor, gate: torch.Tensor | None = None, *,
                         scale: float | None = None, num_splits: int = 0,
                         workspace: torch.Tensor | None = None, out: torch.Tensor | None = None,
                         kv_lens: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Decode over the latent cache: the cache holds only C [B, N, d_c]; the keys and values
    K_h = C W_k,h^T, V_h = C W_v,h^T are never formed ("Gated MLA", "Start from familiar
    attention" and "Common mistakes to avoid"; "Le Transformer et l'attention", "MLA —
    compresser en un vecteur latent").  One query per head at position N-1 attends to all
    N cached tokens; the library regroups the products exactly (scores against
    W_k,h^T q_h, values as W_v,h times the weighted latent sum).

    q: [B, H, D] contiguous; latent_cache: [B, N, d_c] with a contiguous last axis (row
    strides free); key/value up-projections [H*D, d_c] contiguous; gate: optional
    [B, H*D].  kv_lens (optional int32 device tensor [B]): row b holds only its first
    kv_lens[b] latent rows (clamped to [0, N]; its query sits at position kv_lens[b] - 1;
    an empty row gives zeros).  Returns [B, H*D].
    """
    if q.dim() != 3 or latent_cache.dim() != 3:
        raise ValueError("q must be [B, H, D] and latent_cache [B, N, d_c]")
    B, H, D = q.shape
    if latent_cache.shape[0] != B:
        raise ValueError("q and latent_cache disagree on the batch size")
    N, d_c = latent_cache.shape[1], latent_cache.shape[2]
    for w in (key_up_projection, value_up_projection):
        if w.shape != (H * D, d_c):
            raise ValueError("the up-projections must be [H*D, d_c]")
        if not w.is_contiguous():
            raise ValueError("the up-projections must be contiguous")
    if not q.is_contiguous() or latent_cache.stride(2) != 1:
        raise ValueError("q must be contiguous and the latent cache rows contiguous")
    dev = _dev(q, latent_cache, key_up_projection, value_up_projection, gate, out, workspace)
    _same_dtype(q, latent_cache, key_up_projection, value_up_projection, gate, out)
    if gate is not None and (gate.shape != (B, H * D) or not gate.is_contiguous()):
        raise ValueError("gate must be a contiguous [B, H*D] tensor")
    if out is None:
        out = torch.empty((B, H * D), dtype=q.dtype, device=dev)
    elif out.shape != (B, H * D) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B, H*D] tensor")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    lib = _lib.load()
    need = lib.gmla_decode_latent_workspace_bytes(B, H, N, d_c, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    ws_bytes = workspace.numel() * workspace.element_size()
    strides = (ctypes.c_int64 * 2)(latent_cache.stride(0), latent_cache.stride(1))
    if kv_lens is not None:
        if kv_lens.dtype != torch.int32 or kv_lens.shape != (B,) or not kv_lens.is_contiguous():
            raise ValueError("kv_lens must be a contiguous int32 tensor [B]")
        _dev(q, kv_lens)
        st = lib.gmla_attend_decode_latent_varlen(_dtype(q), B, H, N, D, d_c, float(scale), _ptr(q),
                                                  _ptr(latent_cache), strides, _ptr(kv_lens),
                                                  _ptr(key_up_projection), _ptr(value_up_projection),
                                                  _ptr(gate), _ptr(out), _ptr(workspace), ws_bytes,
                                                  int(num_splits), _stream(dev, stream))
        _lib.check(st, "gmla_attend_decode_latent_varlen")
        return out
    st = lib.gmla_attend_decode_latent(_dtype(q), B, H, N, D, d_c, float(scale), _ptr(q),
                                       _ptr(latent_cache), strides, _ptr(key_up_projection),
                                       _ptr(value_up_projection), _ptr(gate), _ptr(out),
                                       _ptr(workspace), ws_bytes, int(num_splits),
                                       _stream(dev, stream))
    _lib.check(st, "gmla_attend_decode_latent")
    return out


def latent_expand(c: torch.Tensor, w_k: torch.Tensor, w_v: torch.Tensor, *, stream=None):
    """K = C W_k^T and V = C W_v^T in one pass over C [..., d_c]; W_k, W_v [d_model, d_c]."""
    d_c = c.shape[-1]
    d_model = w_k.shape[0]
    if w_k.shape != (d_model, d_c) or w_v.shape != (d_model, d_c):
        raise ValueError("w_k and w_v must be [d_model, d_c]")
    for t in (c, w_k, w_v):
        if not t.is_contiguous():
            raise ValueError("latent_expand takes contiguous tensors")
    dev = _dev(c, w_k, w_v)
    _same_dtype(c, w_k, w_v)
    M = c.numel() // d_c
    K = torch.empty((*c.shape[:-1], d_model), dtype=c.dtype, device=dev)
    V = torch.empty_like(K)
    st = _lib.load().gmla_latent_expand(_dtype(c), M, d_c, d_model, _ptr(c), _ptr(w_k), _ptr(w_v),
                                        _ptr(K), _ptr(V), _stream(dev, stream))
    _lib.check(st, "gmla_latent_expand")
    return K, V


def gate_out(o_tilde: torch.Tensor, w_o: torch.Tensor | None = None, gate: torch.Tensor | None = None,
             *, fused_gate: bool = False, stream=None) -> torch.Tensor:
    """Y = [sigmoid(gate) * O~] W_o^T (gate before the projection); either part optional.

    With both parts in bf16 the gate runs as its own pass into a workspace allocated here
    and the projection on the LDS-pipelined GEMM (gmla_gate_out_ws); fused_gate=True
    applies the gate inside the GEMM's tile staging instead (gmla_gate_out, no workspace,
    about 4x slower at the layer's shape)."""
    d_model = o_tilde.shape[-1]
    if gate is not None and gate.shape != o_tilde.shape:
        raise ValueError("gate must have O~'s shape")
    if w_o is not None and w_o.shape != (d_model, d_model):
        raise ValueError("w_o must be [d_model, d_model]")
    for t in (o_tilde, w_o, gate):
        if t is not None and not t.is_contiguous():
            raise ValueError("gate_out takes contiguous tensors")
    dev = _dev(o_tilde, w_o, gate)
    _same_dtype(o_tilde, w_o, gate)
    M = o_tilde.numel() // d_model
    Y = torch.empty_like(o_tilde)
    lib = _lib.load()
    nws = lib.gmla_gate_out_workspace_bytes(_dtype(o_tilde), M, d_model)
    if gate is not None and w_o is not None and nws and not fused_gate:
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        st = lib.gmla_gate_out_ws(_dtype(o_tilde), M, d_model, _ptr(gate), _ptr(o_tilde), _ptr(w_o),
                                  _ptr(Y), _ptr(ws), nws, _stream(dev, stream))
        _lib.check(st, "gmla_gate_out_ws")
        return Y
    st = lib.gmla_gate_out(_dtype(o_tilde), M, d_model, _ptr(gate), _ptr(o_tilde), _ptr(w_o),
                           _ptr(Y), _stream(dev, stream))
    _lib.check(st, "gmla_gate_out")
    return Y


def linear(x: torch.Tensor, w: torch.Tensor, *, out: torch.Tensor | None = None,
           split_k: bool = True, stream=None) -> torch.Tensor:
    """x [..., K] times w [N, K] transposed -> [..., N].  With split_k (the default), a
    bf16 product with few output tiles and a deep K (the latent down-projection) splits
    its reduction over a workspace allocated here (gmla_linear_ws)."""
    K = x.shape[-1]
    N = w.shape[0]
    if w.dim() != 2 or w.shape[1] != K:
        raise ValueError("w must be [N, K] with K = x.shape[-1]")
    if not x.is_contiguous() or not w.is_contiguous():
        raise ValueError("linear takes contiguous tensors")
    dev = _dev(x, w, out)
    _same_dtype(x, w, out)
    M = x.numel() // K
    if out is None:
        out = torch.empty((*x.shape[:-1], N), dtype=x.dtype, device=dev)
    elif out.shape != (*x.shape[:-1], N) or not out.is_contiguous():
        raise ValueError("out has the wrong shape")
    lib = _lib.load()
    need = lib.gmla_linear_workspace_bytes(M, N, K) if split_k and x.dtype == torch.bfloat16 else 0
    if need:
        ws = torch.empty(need, dtype=torch.uint8, device=dev)
        st = lib.gmla_linear_ws(_dtype(x), M, N, K, _ptr(x), _ptr(w), _ptr(out), _ptr(ws), need,
                                _stream(dev, stream))
        _lib.check(st, "gmla_linear_ws")
        return out
    st = lib.gmla_linear(_dtype(x), M, N, K, _ptr(x), _ptr(w), _ptr(out), _stream(dev, stream))
    _lib.check(st, "gmla_linear")
    return out


def gated_mla(hidden_states: torch.Tensor, query_projection: torch.Tensor,
              latent_down_projection: torch.Tensor, key_up_projection: torch.Tensor,
              value_up_projection: torch.Tensor, output_gate_projection: torch.Tensor,
              output_projection: torch.Tensor, num_heads: int, causal: bool = True,
              *, fused_latent: bool = False, stream=None) -> dict:
    """One Gated MLA layer ("Gated MLA", sections "Implementation order" and
    "Requirements"): returns {"output": Y, "latent_cache": C} with Y shaped like the
    hidden states and C [batch, sequence, latent width]; inputs are not modified.

    Order: Q = X W_q^T, C = X W_c^T, [K | V] = C [W_k | W_v]^T, G = X W_g^T,
    O~ = sigmoid(G) * attention(Q, K, V) (gate fused in the attention epilogue),
    Y = O~ W_o^T.  With fused_latent=True the keys and values are rebuilt from C inside
    the attention launch (attend_prefill_latent) instead of by a separate expansion.
    """
    if not isinstance(causal, bool):
        raise TypeError("causal must be a bool")
    if not isinstance(num_heads, int) or num_heads <= 0:
        raise ValueError("num_heads must be a positive int")
    X = hidden_states
    if X.dim() != 3:
        raise ValueError("hidden_states must be [batch, sequence, model width]")
    B, T, dm = X.shape
    if dm % num_heads:
        raise ValueError("model width must be divisible by the head count")
    ws = (query_projection, latent_down_projection, key_up_projection, value_up_projection,
          output_gate_projection, output_projection)
    _dev(X, *ws)
    _same_dtype(X, *ws)
    d_c = latent_down_projection.shape[0]
    if (query_projection.shape != (dm, dm) or latent_down_projection.shape != (d_c, dm)
            or key_up_projection.shape != (dm, d_c) or value_up_projection.shape != (dm, d_c)
            or output_gate_projection.shape != (dm, dm) or output_projection.shape != (dm, dm)):
        raise ValueError("projection matrices have incompatible widths")
    D = dm // num_heads
    X = X.contiguous()
    Q = linear(X, query_projection, stream=stream)
    C = linear(X, latent_down_projection, stream=stream)
    G = linear(X, output_gate_projection, stream=stream)
    if fused_latent:
        O = attend_prefill_latent(Q.view(B, T, num_heads, D), C, key_up_projection,
                                  value_up_projection, G, causal=causal, stream=stream)
    else:
        K, V = latent_expand(C, key_up_projection, value_up_projection, stream=stream)
        O = attend_prefill(Q.view(B, T, num_heads, D), K.view(B, T, num_heads, D),
                           V.view(B, T, num_heads, D), G, causal=causal, stream=stream)
    Y = gate_out(O, output_projection, stream=stream)
    return {"output": Y, "latent_cache": C}
