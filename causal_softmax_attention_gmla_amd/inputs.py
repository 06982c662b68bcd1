"""Seeded synthetic inputs shaped like the pages' workloads.

Only random-number generation lives here: no step of the attention method.  The
GPU library's tests and benchmark, and the CPU oracle's checks, all draw their
inputs from these functions; the oracle then reads back the exact bytes.

Shapes follow the pages: 96 heads of width 128 and latent width 512 ("Le
Transformer et l'attention", sections "Les têtes multiples" and "MLA"), the decode
at position 1000 with 1001 keys ("Kimi K3 - Softmax over keys"), and the 128K
context of that page's cost table for the long decode.  Values are N(0, 1)
(weights N(0, 1/fan_in)), drawn in float32 and rounded to bfloat16 (round to
nearest even) for the bf16 workloads.
"""
from __future__ import annotations

import math
import zlib
from dataclasses import dataclass, field

import torch

SEED_BASE = 0x474D4C41


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str  # "prefill", "decode" or "layer"
    dtype: torch.dtype
    dims: dict = field(default_factory=dict)
    describe: str = ""


WORKLOADS = {
    "tiny_prefill_f32": Workload(
        "tiny_prefill_f32", "prefill", torch.float32, dict(B=1, T=64, H=4, D=32, gate=True),
        "causal prefill B=1 T=64 H=4 D=32, fp32, scale 1/sqrt(32), gated by sigmoid(G), G [1,64,128]"),
    "decode_b8_n1001": Workload(
        "decode_b8_n1001", "decode", torch.bfloat16, dict(B=8, H=96, N=1001, D=128),
        "decode B=8 H=96, 1 query at position 1000 against 1001 keys, D=128, bf16"),
    "prefill_b2_t4096": Workload(
        "prefill_b2_t4096", "prefill", torch.bfloat16, dict(B=2, T=4096, H=96, D=128, gate=False),
        "causal prefill B=2 T=4096 H=96 D=128, bf16, fp32 softmax"),
    "layer_t2048": Workload(
        "layer_t2048", "layer", torch.bfloat16, dict(B=1, T=2048, d_model=12288, d_c=512, H=96),
        "Gated MLA layer B=1 T=2048 d_model=12288 (96 x 128) d_c=512, bf16"),
    "decode_b4_n131072": Workload(
        "decode_b4_n131072", "decode", torch.bfloat16, dict(B=4, H=96, N=131072, D=128),
        "decode B=4 H=96, 1 query against 131072 keys, D=128, bf16"),
}
ORDER = ["tiny_prefill_f32", "decode_b8_n1001", "prefill_b2_t4096", "layer_t2048",
         "decode_b4_n131072"]


def seed_of(name: str) -> int:
    """Base seed of a named workload: SEED_BASE + 1, + 2, ... in the order of ORDER
    (its tensors use base, base + 1, ... in their fixed order); other names hash to
    a stable seed."""
    if name in ORDER:
        return SEED_BASE + 1 + ORDER.index(name)
    return SEED_BASE + 100 + zlib.crc32(name.encode()) % 1000003


def normal(shape, dtype=torch.float32, device="cpu", seed=0, std=1.0,
           chunk_elems: int = 1 << 27) -> torch.Tensor:
    """N(0, std^2) in float32 from a seeded generator, rounded to ``dtype``.

    Large tensors are drawn in chunks along the first axis so that the float32
    temporary stays small; the result depends only on (shape, seed, std, device
    type, chunking), not on the dtype.
    """
    shape = tuple(int(s) for s in shape)
    out = torch.empty(shape, dtype=dtype, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    if out.numel() == 0:
        return out
    flat = out.view(shape[0], -1) if len(shape) > 1 else out.view(-1, 1)
    rows = flat.shape[0]
    per_row = flat.shape[1]
    step = max(1, chunk_elems // max(per_row, 1))
    for r0 in range(0, rows, step):
        r1 = min(rows, r0 + step)
        x = torch.randn((r1 - r0, per_row), generator=gen, device=device, dtype=torch.float32)
        if std != 1.0:
            x.mul_(std)
        flat[r0:r1].copy_(x)
    return out


def prefill_inputs(B, T, H, D, dtype, device="cpu", seed=SEED_BASE, gate=False):
    """Q, K, V [B, T, H, D] ~ N(0, 1) and optional gate logits G [B, T, H*D] ~ N(0, 1)."""
    q = normal((B, T, H, D), dtype, device, seed + 0)
    k = normal((B, T, H, D), dtype, device, seed + 1)
    v = normal((B, T, H, D), dtype, device, seed + 2)
    g = normal((B, T, H * D), dtype, device, seed + 3) if gate else None
    return q, k, v, g


def decode_inputs(B, H, N, D, dtype, device="cpu", seed=SEED_BASE, gate=False):
    """Q [B, H, D], K, V [B, H, N, D] ~ N(0, 1); optional gate logits [B, H*D]."""
    q = normal((B, H, D), dtype, device, seed + 0)
    k = normal((B, H, N, D), dtype, device, seed + 1)
    v = normal((B, H, N, D), dtype, device, seed + 2)
    g = normal((B, H * D), dtype, device, seed + 3) if gate else None
    return q, k, v, g


def layer_inputs(B, T, d_model, d_c, dtype, device="cpu", seed=SEED_BASE):
    """X ~ N(0, 1) [B, T, d_model]; every weight [out, in] ~ N(0, 1/in)."""
    x = normal((B, T, d_model), dtype, device, seed)
    shapes = dict(Wq=(d_model, d_model), Wc=(d_c, d_model), Wk=(d_model, d_c), Wv=(d_model, d_c),
                  Wg=(d_model, d_model), Wo=(d_model, d_model))
    ws = {}
    for i, (n, s) in enumerate(shapes.items()):
        ws[n] = normal(s, dtype, device, seed + 1 + i, std=1.0 / math.sqrt(s[1]))
    return x, ws


def workload_inputs(name: str, device="cpu"):
    """All inputs of a named workload, in the fixed order Q, K, V, G or X, weights."""
    w = WORKLOADS[name]
    d = w.dims
    seed = seed_of(name)
    if w.kind == "prefill":
        return prefill_inputs(d["B"], d["T"], d["H"], d["D"], w.dtype, device, seed, d["gate"])
    if w.kind == "decode":
        return decode_inputs(d["B"], d["H"], d["N"], d["D"], w.dtype, device, seed)
    return layer_inputs(d["B"], d["T"], d["d_model"], d["d_c"], w.dtype, device, seed)
