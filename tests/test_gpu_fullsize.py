"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times: every head of the prefill and long-decode workloads element by element against
the CPU oracle, the layer on 64 tokens spread over every GEMM tile, longer and offset
shapes on sampled rows the oracle computes one by one (rows are independent), plus
closed forms that hold at any size."""
import numpy as np
import pytest
import torch

import causal_softmax_attention_gmla_amd as gm
import oracle
from causal_softmax_attention_gmla_amd import inputs as I
from gpu_helpers import announce, check_rows_rel, host, need_gpu

pytestmark = pytest.mark.gpu


def test_prefill_b2_t4096_every_head():
    """Causal prefill B=2 T=4096 H=96 D=128 bf16, the benchmark's workload and launch:
    every element of all 192 (batch, head) pairs against the oracle (all 4096 rows of
    each head; the output starts as NaN, so every element must have been written)."""
    dev = need_gpu()
    announce("prefill_b2_t4096 full size, every head")
    q, k, v, _ = I.workload_inputs("prefill_b2_t4096", dev)
    B, T, H, D = q.shape
    out = torch.full((B, T, H * D), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.attend_prefill(q, k, v, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "some (head, query block) was never written"
    hq, hk, hv = (t.float().cpu().numpy() for t in (q, k, v))
    got = out.float().cpu().numpy().reshape(B, T, H, D)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            ref = oracle.attend_head(hq[b, :, h], hk[b, :, h], hv[b, :, h], 1 / np.sqrt(D), True)
            ratio, _ = check_rows_rel(got[b, :, h].astype(np.float64), ref, D)
            worst = max(worst, ratio)
    print(f"prefill_b2_t4096: 192 heads x 4096 rows, worst row error / row max {worst:.3e}")


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


def test_prefill_query_token_stride_past_lds_load_offsets():
    """Q rows 2^25 + 2^21 elements apart: 31 rows span more than 2^30 elements, past the 32-bit
    byte offsets of the LDS-direct Q row loads, so the kernel loads each lane's query
    row into registers instead (through the chunk entry, whose Q strides are its own);
    every row against the oracle."""
    dev = need_gpu()
    T, D, qst = 40, 128, 2 ** 25 + 2 ** 21
    assert 31 * qst + D >= 2 ** 30
    announce(f"prefill T={T}: query token stride {qst} elements")
    buf = torch.empty((T - 1) * qst + D, dtype=torch.bfloat16, device=dev)
    q = buf.as_strided((1, T, 1, D), (T * qst, qst, D, 1))
    q.copy_(I.normal((1, T, 1, D), torch.bfloat16, dev, seed=5300))
    k = I.normal((1, T, 1, D), torch.bfloat16, dev, seed=5301)
    v = I.normal((1, T, 1, D), torch.bfloat16, dev, seed=5302)
    out = torch.full((1, T, D), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.attend_chunk(q, k, v, out=out)
    torch.cuda.synchronize()
    ref = oracle.attend_head(host(q[0, :, 0]), host(k[0, :, 0]), host(v[0, :, 0]),
                             1 / np.sqrt(D), True)
    check_rows_rel(host(out[0]), ref, D)
    del buf, out


def test_latent_down_projection_split_k_every_row():
    """The layer's latent down-projection C = X W_c^T (2048 x 512 x 12288) on the split-K
    path: every row against the oracle."""
    dev = need_gpu()
    announce("linear split-K 2048x512x12288, every row")
    x, ws = I.workload_inputs("layer_t2048", dev)
    x2 = x.view(-1, x.shape[-1])
    assert gm.library().gmla_linear_workspace_bytes(2048, 512, 12288) > 0
    c = gm.linear(x2, ws["Wc"])
    torch.cuda.synchronize()
    check_rows_rel(host(c), oracle.linear(host(x2), host(ws["Wc"])), 512)


def test_gate_out_t2048_both_routes_sampled():
    """The gated output projection at the layer's shape (M = 2048, d_model = 12288, bf16),
    both routes: gate pass + LDS GEMM and gate in the GEMM's tile staging.  64 rows over
    every 256-row tile against the oracle, and the two routes within the same bound of
    each other everywhere."""
    dev = need_gpu()
    announce("gate_out 2048x12288 both routes, 64 rows")
    M, dm = 2048, 12288
    o = I.normal((M, dm), torch.bfloat16, dev, seed=7201)
    g = I.normal((M, dm), torch.bfloat16, dev, seed=7202)
    w = I.normal((dm, dm), torch.bfloat16, dev, seed=7203, std=dm ** -0.5)
    assert gm.library().gmla_gate_out_workspace_bytes(1, M, dm) == M * dm * 2
    y_ws = gm.gate_out(o, w, g)
    y_fu = gm.gate_out(o, w, g, fused_gate=True)
    torch.cuda.synchronize()
    rows = layer_rows()
    ref = oracle.linear(oracle.gate(host(g[rows]), host(o[rows])), host(w))
    check_rows_rel(host(y_ws[rows]), ref, dm)
    check_rows_rel(host(y_fu[rows]), ref, dm)
    check_rows_rel(host(y_ws), host(y_fu), dm)
    del o, g, w, y_ws, y_fu


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


def test_decode_b4_n131072_every_head():
    """Decode B=4 H=96 against 131072 keys, split-KV with the log-sum-exp merge: all 384
    heads against the oracle (each head's 131072 key and value rows copied to the host in
    groups of eight heads, the oracle run on them in threads), and the Q = 0 closed form
    (the mean of all 131072 value rows) on every head of batch 0."""
    import concurrent.futures as cf

    dev = need_gpu()
    announce("decode_b4_n131072 full size, every head")
    q, k, v, _ = I.workload_inputs("decode_b4_n131072", dev)
    out = gm.attend_decode(q, k, v)
    torch.cuda.synchronize()
    B, H, N, D = k.shape
    got = host(out).reshape(B, H, D)
    hq = host(q)
    G = 8
    worst = 0.0
    with cf.ThreadPoolExecutor(max_workers=G) as ex:
        for b in range(B):
            for h0 in range(0, H, G):
                kh = k[b, h0:h0 + G].float().cpu().numpy()
                vh = v[b, h0:h0 + G].float().cpu().numpy()
                refs = list(ex.map(lambda i: oracle.attend_head(hq[b, h0 + i][None], kh[i], vh[i],
                                                                1 / np.sqrt(D), True, nthreads=1),
                                   range(G)))
                for i, ref in enumerate(refs):
                    ratio, _ = check_rows_rel(got[b, h0 + i][None], ref, D)
                    worst = max(worst, ratio)
                del kh, vh
    print(f"decode_b4_n131072: 384 heads, worst row error / row max {worst:.3e}")
    # Q = 0: uniform weights over all keys
    z = gm.attend_decode(torch.zeros_like(q), k, v)
    torch.cuda.synchronize()
    mean = v[0].float().mean(dim=1).double().cpu().numpy()  # [H, D], summed on the GPU in fp32
    check_rows_rel(host(z).reshape(B, H, D)[0], mean, D)


def test_decode_latent_b8_n1001_every_head():
    """Decode over the latent cache at the pages' decode shape (B=8, H=96, the query at
    position 1000 against 1001 cached tokens, 512-wide latent, bf16): all 768 heads
    against the oracle's composition (keys and values formed from the latent in double)."""
    from test_gpu_parity import latent_inputs, oracle_latent_decode

    dev = need_gpu()
    announce("decode_latent B8 N1001 d_c 512, every head")
    B, N, H, dc = 8, 1001, 96, 512
    q, c, wk, wv, _ = latent_inputs(B, N, H, dc, dev, 7000, False)
    out = gm.attend_decode_latent(q, c, wk, wv)
    torch.cuda.synchronize()
    got = host(out).reshape(B, H, 128)
    hc, hq, hwk, hwv = host(c), host(q), host(wk), host(wv)
    worst = 0.0
    for b in range(B):
        K = oracle.linear(hc[b], hwk)  # [N, H*D]: every head's keys at once
        V = oracle.linear(hc[b], hwv)
        for h in range(H):
            sl = slice(h * 128, (h + 1) * 128)
            ref = oracle.attend_head(hq[b, h][None], K[:, sl], V[:, sl], 1 / np.sqrt(128), True)
            ratio, _ = check_rows_rel(got[b, h][None], ref, 128)
            worst = max(worst, ratio)
    print(f"decode_latent B8 N1001: 768 heads, worst row error / row max {worst:.3e}")


def test_decode_latent_b4_n131072():
    """Decode over a 131072-token latent cache (B=4, H=96, d_c=512): sampled heads against
    the oracle's composition, and on every head the Q = 0 closed form (uniform weights:
    o_h = W_v,h times the mean latent row)."""
    from test_gpu_parity import latent_inputs, oracle_latent_decode

    dev = need_gpu()
    announce("decode_latent B4 N131072 d_c 512")
    B, N, H, dc = 4, 131072, 96, 512
    q, c, wk, wv, _ = latent_inputs(B, N, H, dc, dev, 7100, False)
    out = gm.attend_decode_latent(q, c, wk, wv)
    torch.cuda.synchronize()
    got = host(out).reshape(B, H, 128)
    for (b, h), ref in oracle_latent_decode(q, c, wk, wv, None, [(0, 0), (3, 95), (1, 50)]).items():
        check_rows_rel(got[b, h][None], ref, 128)
    z = gm.attend_decode_latent(torch.zeros_like(q), c, wk, wv)
    torch.cuda.synchronize()
    hz = host(z).reshape(B, H, 128)
    hwv = host(wv)
    for b in range(B):
        mean_c = c[b].float().mean(dim=0).double().cpu().numpy()  # summed on the GPU in fp32
        ref = oracle.linear(mean_c[None], hwv).reshape(H, 128)
        check_rows_rel(hz[b], ref, 128)


def layer_rows():
    """64 tokens of the T=2048 layer: both edges and the middle seam of each of the eight
    256-row GEMM tiles (which are also edges of 128-query attention blocks), plus eight
    seeded interior tokens."""
    rows = set()
    for t0 in range(0, 2048, 256):
        rows.update((t0, t0 + 1, t0 + 127, t0 + 128, t0 + 254, t0 + 255, t0 + 64))
    rng = np.random.default_rng(2048)
    while len(rows) < 64:
        rows.add(int(rng.integers(0, 2048)))
    return sorted(rows)


def test_layer_t2048_tokens():
    """Full Gated MLA layer B=1 T=2048 d_model=12288 d_c=512 bf16: the whole latent cache
    (all 2048 rows) and the output of 64 tokens spread over every GEMM tile and
    query block, against the oracle layer."""
    dev = need_gpu()
    announce("layer_t2048 full size, 64 tokens")
    x, ws = I.workload_inputs("layer_t2048", dev)
    H = I.WORKLOADS["layer_t2048"].dims["H"]
    res = gm.gated_mla(x, ws["Wq"], ws["Wc"], ws["Wk"], ws["Wv"], ws["Wg"], ws["Wo"], H, True)
    torch.cuda.synchronize()
    rows = layer_rows()
    assert len(rows) == 64
    ref = oracle.gated_mla_layer(host(x), *(host(ws[n]) for n in ("Wq", "Wc", "Wk", "Wv", "Wg", "Wo")),
                                 H, True, rows=rows)
    check_rows_rel(host(res["latent_cache"]), ref["latent_cache"], 512)
    check_rows_rel(host(res["output"][:, rows]), ref["output"], 12288)


def test_layer_t2048_fused_latent_tokens():
    """The full layer (B=1, T=2048, d_model=12288, d_c=512) with the keys and values
    rebuilt from the latent inside the attention launch: 64 tokens over every GEMM tile
    against the oracle layer, and the whole output equal to the two-launch layer's."""
    dev = need_gpu()
    announce("layer_t2048 fused latent, 64 tokens")
    x, ws = I.workload_inputs("layer_t2048", dev)
    H = I.WORKLOADS["layer_t2048"].dims["H"]
    args = (x, ws["Wq"], ws["Wc"], ws["Wk"], ws["Wv"], ws["Wg"], ws["Wo"], H, True)
    res = gm.gated_mla(*args, fused_latent=True)
    two = gm.gated_mla(*args)
    torch.cuda.synchronize()
    assert torch.equal(res["output"], two["output"])
    rows = layer_rows()
    ref = oracle.gated_mla_layer(host(x), *(host(ws[n]) for n in ("Wq", "Wc", "Wk", "Wv", "Wg", "Wo")),
                                 H, True, rows=rows)
    check_rows_rel(host(res["output"][:, rows]), ref["output"], 12288)


@pytest.mark.parametrize("B,T,H", [(1, 5120, 40), (1, 3584, 56)])
def test_prefill_partial_last_head_group(B, T, H):
    """More than three query blocks per workgroup slot on each XCD (200 and 196 blocks per
    XCD), so the launch interleaves heads in groups of four, with 5 and 7 heads per XCD:
    the last group of each XCD is partial (1 and 3 heads).  The output starts as NaN;
    every element of every head is checked against the oracle."""
    dev = need_gpu()
    nqb = (T + 127) // 128
    per_xcd = nqb * B * H // 8
    assert per_xcd > 192 and per_xcd % nqb == 0 and (per_xcd // nqb) % 4 != 0
    announce(f"prefill bf16 partial head group B={B} T={T} H={H}")
    q, k, v, _ = I.prefill_inputs(B, T, H, 128, torch.bfloat16, dev, seed=3100 + H)
    out = torch.full((B, T, H * 128), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.attend_prefill(q, k, v, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any(), "some (head, query block) was never written"
    hq, hk, hv = (t.float().cpu().numpy() for t in (q, k, v))
    got = out.float().cpu().numpy().reshape(B, T, H, 128)
    for b in range(B):
        for h in range(H):
            ref = oracle.attend_head(hq[b, :, h], hk[b, :, h], hv[b, :, h], 1 / np.sqrt(128), True)
            check_rows_rel(got[b, :, h].astype(np.float64), ref, 128)
