"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times, checked on sampled outputs that the CPU oracle computes one by one (rows are
independent), plus closed forms that hold at any size."""
import numpy as np
import pytest
import torch

import causal_softmax_attention_gmla_amd as gm
import oracle
from causal_softmax_attention_gmla_amd import inputs as I
from gpu_helpers import announce, check_rows_rel, host, need_gpu

pytestmark = pytest.mark.gpu


def test_prefill_b2_t4096_sampled():
    """Causal prefill B=2 T=4096 H=96 D=128 bf16: sampled heads and rows (first,
    tile edges, ragged-free interior, last) against the oracle."""
    dev = need_gpu()
    announce("prefill_b2_t4096 full size, sampled rows")
    q, k, v, _ = I.workload_inputs("prefill_b2_t4096", dev)
    B, T, H, D = q.shape
    out = torch.full((B, T, H * D), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.attend_prefill(q, k, v, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "some (head, query block) was never written"
    r = np.random.default_rng(11)
    heads = [(0, 0), (1, H - 1)] + [(int(r.integers(B)), int(r.integers(H))) for _ in range(4)]
    rows = sorted(set([0, 1, 31, 32, 63, 64, 127, 128, 129, 1000, 2047, 2048, 4094, 4095]
                      + [int(x) for x in r.integers(0, T, 10)]))
    for b, h in heads:
        ref = oracle.attend_head(host(q[b, :, h]), host(k[b, :, h]), host(v[b, :, h]),
                                 1 / np.sqrt(D), True, rows=rows)
        got = host(out[b, rows, h * D:(h + 1) * D])
        check_rows_rel(got, ref, D)


@pytest.mark.parametrize("Tq,Tk", [(16384, 16384), (300, 65536)])
def test_prefill_long_sampled(Tq, Tk):
    """Long sequences on the MFMA kernel: a 16384-token causal prefill (the longest of the
    sequence-length sweep) and a 300-query chunk after 65236 cached tokens (key rows past
    2^16, an offset off the 64-key tile grid); every output written, sampled rows of two
    heads against the oracle."""
    dev = need_gpu()
    announce(f"prefill long Tq={Tq} Tk={Tk}, sampled rows")
    H, D = 2, 128
    out = torch.full((1, Tq, H * D), float("nan"), dtype=torch.bfloat16, device=dev)
    if Tq == Tk:  # one packed [T, 3, H, D] buffer: q, k and v share their strides
        qkv = I.normal((1, Tq, 3, H, D), torch.bfloat16, dev, seed=5100 + Tq)
        q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
        gm.attend_prefill(q, k, v, out=out)
    else:
        q = I.normal((1, Tq, H, D), torch.bfloat16, dev, seed=5100 + Tq)
        kv = I.normal((1, Tk, 2, H, D), torch.bfloat16, dev, seed=5101 + Tk)
        k, v = kv[:, :, 0], kv[:, :, 1]
        gm.attend_chunk(q, k, v, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "some (head, query block) was never written"
    rows = sorted(set([0, 1, 63, 64, 127, 128, Tq // 2, Tq - 129, Tq - 2, Tq - 1]))
    for h in range(H):
        ref = oracle.attend_head(host(q[0, :, h]), host(k[0, :, h]), host(v[0, :, h]),
                                 1 / np.sqrt(D), True, rows=rows)
        check_rows_rel(host(out[0, rows, h * D:(h + 1) * D]), ref, D)


def test_prefill_offsets_past_2_31_sampled():
    """Causal prefill B=2 T=65536 H=96 from one packed [B, T, 3, H, D] buffer: the second
    batch's rows start 2.4e9 elements in, past 32-bit element offsets; every output
    written, sampled rows of heads in both batches against the oracle."""
    dev = need_gpu()
    B, T, H, D = 2, 65536, 96, 128
    announce(f"prefill B={B} T={T} H={H}: element offsets past 2^31")
    qkv = I.normal((B * T, 3, H, D), torch.bfloat16, dev, seed=5200).view(B, T, 3, H, D)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    assert q.stride(0) * (B - 1) > 2 ** 31
    out = torch.full((B, T, H * D), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.attend_prefill(q, k, v, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "some (head, query block) was never written"
    rows = [0, 127, 128, 40000, T - 1]
    for b, h in [(0, 5), (1, 0), (1, H - 1)]:
        ref = oracle.attend_head(host(q[b, :, h]), host(k[b, :, h]), host(v[b, :, h]),
                                 1 / np.sqrt(D), True, rows=rows)
        check_rows_rel(host(out[b, rows, h * D:(h + 1) * D]), ref, D)
    del qkv, out


def test_linear_offsets_past_2_31_sampled():
    """Y = X W^T with X [300000, 8192] (2.46e9 elements, past 32-bit element offsets) on
    the 256 x 384-tile kernel; every output written, sampled rows (the last ones beyond
    2^31 elements into X) against the oracle."""
    dev = need_gpu()
    M, N, K = 300000, 384, 8192
    announce(f"linear {M}x{N}x{K}: element offsets past 2^31")
    x = I.normal((M, K), torch.bfloat16, dev, seed=5300)
    w = I.normal((N, K), torch.bfloat16, dev, seed=5301, std=K ** -0.5)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.linear(x, w, out=y)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    rows = [0, 255, 256, 262143, 262144, 299999]
    check_rows_rel(host(y[rows]), oracle.linear(host(x[rows]), host(w)), N)
    del x, y


def test_decode_b4_n131072_sampled():
    """Decode B=4 H=96 against 131072 keys, split-KV with the log-sum-exp merge:
    sampled heads against the oracle, and the Q = 0 closed form (the mean of all
    131072 value rows) on every head of batch 0."""
    dev = need_gpu()
    announce("decode_b4_n131072 full size, sampled heads")
    q, k, v, _ = I.workload_inputs("decode_b4_n131072", dev)
    out = gm.attend_decode(q, k, v)
    torch.cuda.synchronize()
    B, H, N, D = k.shape
    r = np.random.default_rng(12)
    heads = [(0, 0), (B - 1, H - 1)] + [(int(r.integers(B)), int(r.integers(H))) for _ in range(4)]
    for b, h in heads:
        ref = oracle.attend_head(host(q[b, h][None]), host(k[b, h]), host(v[b, h]), 1 / np.sqrt(D),
                                 True)
        check_rows_rel(host(out[b, h * D:(h + 1) * D])[None], ref, D)
    # Q = 0: uniform weights over all keys
    z = gm.attend_decode(torch.zeros_like(q), k, v)
    torch.cuda.synchronize()
    for h in range(0, H, 8):
        mean = host(v[0, h]).mean(axis=0)
        check_rows_rel(host(z[0, h * D:(h + 1) * D])[None], mean[None], D)


def test_layer_t2048_sampled():
    """Full Gated MLA layer B=1 T=2048 d_model=12288 d_c=512 bf16: the latent cache on
    sampled rows, and the output on sampled tokens, against the oracle layer."""
    dev = need_gpu()
    announce("layer_t2048 full size, sampled tokens")
    x, ws = I.workload_inputs("layer_t2048", dev)
    H = I.WORKLOADS["layer_t2048"].dims["H"]
    res = gm.gated_mla(x, ws["Wq"], ws["Wc"], ws["Wk"], ws["Wv"], ws["Wg"], ws["Wo"], H, True)
    torch.cuda.synchronize()
    rows = [0, 1, 777, 2047]
    ref = oracle.gated_mla_layer(host(x), *(host(ws[n]) for n in ("Wq", "Wc", "Wk", "Wv", "Wg", "Wo")),
                                 H, True, rows=rows)
    check_rows_rel(host(res["latent_cache"]), ref["latent_cache"], 512)
    check_rows_rel(host(res["output"][:, rows]), ref["output"], 12288)
