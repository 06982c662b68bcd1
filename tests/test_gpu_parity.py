"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the same
seeded inputs, at sizes the oracle finishes in seconds that span several tiles and a
ragged tail, plus the edge cases of the method."""
import numpy as np
import pytest
import torch

import causal_softmax_attention_gmla_amd as gm
import oracle
from causal_softmax_attention_gmla_amd import inputs as I
from gpu_helpers import announce, check_f32_abs, check_rows_rel, host, need_gpu

pytestmark = pytest.mark.gpu


def _oracle_prefill(q, k, v, g, causal, scale=None):
    """Oracle output [B, T, H*D] (gated if g is given) from device tensors' bytes."""
    B, T, H, D = q.shape
    scale = scale if scale is not None else 1.0 / np.sqrt(D)
    o = oracle.attend(host(q), host(k), host(v), scale, causal, layout="bthd").reshape(B, T, H * D)
    if g is not None:
        o = oracle.gate(host(g), o)
    return o


# ---------------------------------------------------------------- prefill


def test_tiny_prefill_f32_gated():
    """Causal prefill B=1 T=64 H=4 D=32 fp32, gated, against the oracle at 1e-5."""
    dev = need_gpu()
    announce("tiny_prefill_f32 gated")
    q, k, v, g = I.workload_inputs("tiny_prefill_f32", dev)
    out = gm.attend_prefill(q, k, v, g)
    torch.cuda.synchronize()
    ref = _oracle_prefill(q, k, v, g, True)
    check_f32_abs(host(out), ref)


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("T", [1, 5, 64, 65, 130])
def test_prefill_f32_shapes(T, D):
    dev = need_gpu()
    announce(f"prefill f32 T={T} D={D}")
    q, k, v, g = I.prefill_inputs(2, T, 3, D, torch.float32, dev, seed=1000 + T + D, gate=True)
    for causal in (True, False):
        out = gm.attend_prefill(q, k, v, g, causal=causal)
        torch.cuda.synchronize()
        check_f32_abs(host(out), _oracle_prefill(q, k, v, g, causal))


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 128, 129, 300, 517])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_bf16_mfma_shapes(T, causal):
    """The MFMA kernel (D = 128) across tile boundaries and ragged tails."""
    dev = need_gpu()
    announce(f"prefill bf16 D=128 T={T} causal={causal}")
    q, k, v, g = I.prefill_inputs(2, T, 3, 128, torch.bfloat16, dev, seed=2000 + T, gate=(T % 2 == 1))
    out = gm.attend_prefill(q, k, v, g, causal=causal)
    torch.cuda.synchronize()
    check_rows_rel(host(out), _oracle_prefill(q, k, v, g, causal), 128)


@pytest.mark.parametrize("T", [65, 300])
@pytest.mark.parametrize("causal", [True, False])
def test_prefill_bf16_writes_only_its_output(T, causal):
    """Ragged last query blocks: the output goes to a view inside a larger NaN-filled
    buffer; every output element is written and nothing around it is."""
    dev = need_gpu()
    announce(f"prefill bf16 output bounds T={T} causal={causal}")
    B, H, D = 2, 3, 128
    q, k, v, _ = I.prefill_inputs(B, T, H, D, torch.bfloat16, dev, seed=5000 + T)
    n = B * T * H * D
    buf = torch.full((n + 4096,), float("nan"), dtype=torch.bfloat16, device=dev)
    out = buf[2048:2048 + n].view(B, T, H * D)
    gm.attend_prefill(q, k, v, causal=causal, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    assert torch.isnan(buf[:2048]).all() and torch.isnan(buf[2048 + n:]).all()
    check_rows_rel(host(out), _oracle_prefill(q, k, v, None, causal), 128)


@pytest.mark.parametrize("B,T,H", [(1, 256, 40), (1, 512, 24), (2, 1024, 8), (1, 384, 48)])
def test_prefill_bf16_launch_groups(B, T, H):
    """Shapes whose query blocks split evenly over the 8 XCDs with 5, 3, 2 and 6 heads per
    XCD: the launch order interleaves heads in groups (a partial last group for 5 and 6),
    and every (head, query block) must still be computed exactly once."""
    dev = need_gpu()
    announce(f"prefill bf16 launch groups B={B} T={T} H={H}")
    q, k, v, _ = I.prefill_inputs(B, T, H, 128, torch.bfloat16, dev, seed=3000 + H)
    out = torch.full((B, T, H * 128), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.attend_prefill(q, k, v, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    check_rows_rel(host(out), _oracle_prefill(q, k, v, None, True), 128)


# ---------------------------------------------------------------- chunk after a cache


def _chunk_inputs(B, Tq, Tk, H, D, dtype, dev, seed, gate):
    """Chunk queries [B, Tq, H, D] (contiguous) and keys/values [B, Tk, H, D] as head
    views into one packed [B, Tk, 2, H, D] cache (strides differ from the queries')."""
    q = I.normal((B, Tq, H, D), dtype, dev, seed)
    kv = I.normal((B, Tk, 2, H, D), dtype, dev, seed + 1)
    g = I.normal((B, Tq, H * D), dtype, dev, seed + 2) if gate else None
    return q, kv[:, :, 0], kv[:, :, 1], g


@pytest.mark.parametrize("Tq,Tk", [(1, 1001), (1, 64), (37, 300), (128, 256), (200, 777), (64, 64),
                                   (129, 130), (300, 1000)])
@pytest.mark.parametrize("causal", [True, False])
def test_chunk_bf16_mfma(Tq, Tk, causal):
    """A chunk of Tq queries after Tk - Tq cached tokens (query i at position
    i + Tk - Tq), offsets on and off the 64-key tile grid, on the MFMA kernel."""
    dev = need_gpu()
    announce(f"chunk bf16 D=128 Tq={Tq} Tk={Tk} causal={causal}")
    q, k, v, g = _chunk_inputs(2, Tq, Tk, 3, 128, torch.bfloat16, dev, 2600 + Tq + Tk, Tq % 2 == 1)
    out = gm.attend_chunk(q, k, v, g, causal=causal)
    torch.cuda.synchronize()
    check_rows_rel(host(out), _oracle_prefill(q, k, v, g, causal), 128)


@pytest.mark.parametrize("Tq,Tk,D", [(5, 77, 32), (70, 133, 64), (33, 200, 128)])
def test_chunk_f32_exact(Tq, Tk, D):
    """The float32 kernel with an offset, to the float32 tolerance."""
    dev = need_gpu()
    announce(f"chunk f32 D={D} Tq={Tq} Tk={Tk}")
    q, k, v, g = _chunk_inputs(1, Tq, Tk, 2, D, torch.float32, dev, 2700 + D, True)
    out = gm.attend_chunk(q, k, v, g, causal=True)
    torch.cuda.synchronize()
    check_f32_abs(host(out), _oracle_prefill(q, k, v, g, True))


@pytest.mark.parametrize("D", [32, 64])
def test_prefill_bf16_small_heads(D):
    dev = need_gpu()
    announce(f"prefill bf16 D={D}")
    q, k, v, g = I.prefill_inputs(1, 200, 4, D, torch.bfloat16, dev, seed=2500 + D, gate=True)
    out = gm.attend_prefill(q, k, v, g)
    torch.cuda.synchronize()
    check_rows_rel(host(out), _oracle_prefill(q, k, v, g, True), D)


def test_prefill_bf16_strided_views():
    """Q, K, V as head views into one packed [B, T, 3, H, D] buffer (strides != contiguous)."""
    dev = need_gpu()
    announce("prefill bf16 strided views")
    B, T, H, D = 2, 257, 4, 128
    qkv = I.normal((B, T, 3, H, D), torch.bfloat16, dev, seed=2600)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    out = gm.attend_prefill(q, k, v)
    torch.cuda.synchronize()
    check_rows_rel(host(out), _oracle_prefill(q, k, v, None, True), 128)


def test_prefill_bf16_large_scores():
    """Scores far from N(0,1) (inputs x 4: scaled-score std ~ 16) still follow the
    plain softmax: the lazy rescale must keep the weights exact."""
    dev = need_gpu()
    announce("prefill bf16 large scores")
    q, k, v, _ = I.prefill_inputs(1, 400, 2, 128, torch.bfloat16, dev, seed=2700)
    q = (q.float() * 4).to(torch.bfloat16)
    k = (k.float() * 4).to(torch.bfloat16)
    out = gm.attend_prefill(q, k, v)
    torch.cuda.synchronize()
    check_rows_rel(host(out), _oracle_prefill(q, k, v, None, True), 128)


def test_prefill_three_token_pattern():
    """The three-token example ('Gated MLA', 'A small causal example'): with V the
    identity on the first three channels, output row t reveals A[t, :], which must be
    lower-triangular with A[0] = (1, 0, 0) exactly."""
    dev = need_gpu()
    announce("prefill three-token pattern")
    for dtype, D in ((torch.bfloat16, 128), (torch.float32, 32)):
        q, k, _, _ = I.prefill_inputs(1, 3, 1, D, dtype, dev, seed=2800)
        v = torch.zeros((1, 3, 1, D), dtype=dtype, device=dev)
        for s in range(3):
            v[0, s, 0, s] = 1.0
        A = host(gm.attend_prefill(q, k, v))[0, :, :3]
        assert A[0, 0] == 1.0 and A[0, 1] == 0.0 and A[0, 2] == 0.0
        assert A[1, 2] == 0.0 and A[1, 0] > 0 and A[1, 1] > 0
        assert np.all(A[2] > 0)
        assert np.allclose(A.sum(axis=1), 1.0, atol=1e-2)


# ---------------------------------------------------------------- decode


@pytest.mark.parametrize("splits", [0, 1, 2, 7])
def test_decode_b8_n1001(splits):
    """Decode at the pages' shape (B=8, H=96, 1001 keys, bf16), every head against the oracle."""
    dev = need_gpu()
    announce(f"decode_b8_n1001 splits={splits}")
    q, k, v, _ = I.workload_inputs("decode_b8_n1001", dev)
    out = gm.attend_decode(q, k, v, num_splits=splits)
    torch.cuda.synchronize()
    B, H, N, D = k.shape
    ref = oracle.attend(host(q)[:, :, None, :], host(k), host(v), 1 / np.sqrt(D), True,
                        layout="bhtd").reshape(B, H * D)
    check_rows_rel(host(out), ref, D)


@pytest.mark.parametrize("B,N,H,dc,gate", [(2, 300, 4, 64, True), (8, 1001, 96, 512, False)])
def test_decode_latent_cache(B, N, H, dc, gate):
    """Decode over the latent cache (K, V rebuilt from C when attention runs), against the
    oracle's composition: K_h = C W_k,h^T, V_h = C W_v,h^T in double, then the softmax of
    the last position over all N keys; every head at the small shape, sampled heads at
    the pages' decode shape (B=8, H=96, 1001 keys, 512-wide latent)."""
    dev = need_gpu()
    D = 128
    announce(f"decode over latent cache B={B} N={N} H={H} d_c={dc}")
    q = I.normal((B, H, D), torch.bfloat16, dev, seed=3300 + N)
    c = I.normal((B, N, dc), torch.bfloat16, dev, seed=3301 + N)
    wk = I.normal((H * D, dc), torch.bfloat16, dev, seed=3302 + N, std=dc ** -0.5)
    wv = I.normal((H * D, dc), torch.bfloat16, dev, seed=3303 + N, std=dc ** -0.5)
    g = I.normal((B, H * D), torch.bfloat16, dev, seed=3304 + N) if gate else None
    out = gm.attend_decode_latent(q, c, wk, wv, g)
    torch.cuda.synchronize()
    r = np.random.default_rng(N)
    pairs = ([(b, h) for b in range(B) for h in range(H)] if B * H <= 16 else
             [(0, 0), (B - 1, H - 1)] + [(int(r.integers(B)), int(r.integers(H))) for _ in range(6)])
    hc, hq, hwk, hwv = host(c), host(q), host(wk), host(wv)
    for b, h in pairs:
        kh = oracle.linear(hc[b], hwk[h * D:(h + 1) * D])
        vh = oracle.linear(hc[b], hwv[h * D:(h + 1) * D])
        ref = oracle.attend_head(hq[b, h][None, :], kh, vh, 1 / np.sqrt(D), True)
        if gate:
            ref = oracle.gate(host(g)[b, h * D:(h + 1) * D][None, :], ref)
        check_rows_rel(host(out)[b, h * D:(h + 1) * D][None, :], ref, D)


@pytest.mark.parametrize("N", [1, 2, 17, 64, 255, 256, 257, 1000])
@pytest.mark.parametrize("D,dtype", [(128, torch.bfloat16), (128, torch.float32),
                                     (64, torch.bfloat16), (32, torch.float32)])
def test_decode_shapes(N, D, dtype):
    dev = need_gpu()
    announce(f"decode N={N} D={D} {dtype}")
    q, k, v, g = I.decode_inputs(2, 3, N, D, dtype, dev, seed=3000 + N + D, gate=True)
    ref = oracle.attend(host(q)[:, :, None, :], host(k), host(v), 1 / np.sqrt(D), True,
                        layout="bhtd").reshape(2, 3 * D)
    ref = oracle.gate(host(g), ref)
    for splits in (0, 1, 3):
        out = gm.attend_decode(q, k, v, g, num_splits=splits)
        torch.cuda.synchronize()
        if dtype == torch.float32:
            check_f32_abs(host(out), ref)
        else:
            check_rows_rel(host(out), ref, D)


def test_decode_token_major_cache():
    """K, V stored [B, N, H, D] (token-major) and passed as strided [B, H, N, D] views."""
    dev = need_gpu()
    announce("decode token-major cache")
    B, N, H, D = 2, 333, 4, 128
    kt = I.normal((B, N, H, D), torch.bfloat16, dev, seed=3100)
    vt = I.normal((B, N, H, D), torch.bfloat16, dev, seed=3101)
    q = I.normal((B, H, D), torch.bfloat16, dev, seed=3102)
    k, v = kt.permute(0, 2, 1, 3), vt.permute(0, 2, 1, 3)
    out = gm.attend_decode(q, k, v, num_splits=2)
    torch.cuda.synchronize()
    ref = oracle.attend(host(q)[:, :, None, :], host(k), host(v), 1 / np.sqrt(D), True,
                        layout="bhtd").reshape(B, H * D)
    check_rows_rel(host(out), ref, D)


def test_decode_matches_prefill_last_row():
    """decode(query t against keys 0..t) equals row t of the causal prefill."""
    dev = need_gpu()
    announce("decode vs prefill last row")
    B, T, H, D = 1, 200, 2, 128
    q, k, v, _ = I.prefill_inputs(B, T, H, D, torch.bfloat16, dev, seed=3200)
    pre = host(gm.attend_prefill(q, k, v))[:, -1]
    dec = host(gm.attend_decode(q[:, -1].contiguous(), k.permute(0, 2, 1, 3),
                                v.permute(0, 2, 1, 3)))
    check_rows_rel(dec, pre, D)


# ---------------------------------------------------------------- projections


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("M,N,K", [(1, 8, 8), (77, 200, 64), (130, 256, 136), (256, 384, 512)])
def test_linear(M, N, K, dtype):
    dev = need_gpu()
    announce(f"linear {M}x{N}x{K} {dtype}")
    x = I.normal((M, K), dtype, dev, seed=4000 + M)
    w = I.normal((N, K), dtype, dev, seed=4001 + N, std=K ** -0.5)
    y = gm.linear(x, w)
    torch.cuda.synchronize()
    ref = oracle.linear(host(x), host(w))
    if dtype == torch.float32:
        check_f32_abs(host(y), ref, 1e-4)
    else:
        check_rows_rel(host(y), ref, N)


@pytest.mark.parametrize("offset", [0, 4, 8])
def test_linear_output_alignment(offset):
    """Output buffers 16-, 8- and 16-byte aligned (bf16 element offsets 0, 4, 8 into one
    allocation): the LDS-pipelined kernel stores 16 bytes per lane and takes only
    16-byte-aligned outputs; the others go to the register-staged kernel.  Both match."""
    dev = need_gpu()
    M, N, K = 512, 1024, 256
    announce(f"linear output offset {offset}")
    x = I.normal((M, K), torch.bfloat16, dev, seed=4100)
    w = I.normal((N, K), torch.bfloat16, dev, seed=4101, std=K ** -0.5)
    buf = torch.full((M * N + 16,), float("nan"), dtype=torch.bfloat16, device=dev)
    y = buf[offset:offset + M * N].view(M, N)
    gm.linear(x, w, out=y)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert torch.isnan(buf[:offset]).all() and torch.isnan(buf[offset + M * N:]).all()
    check_rows_rel(host(y), oracle.linear(host(x), host(w)), N)


@pytest.mark.parametrize("M,N,K", [(2000, 8200, 320), (2048, 8192, 64), (1500, 11000, 192)])
def test_linear_mid_ragged(M, N, K):
    """Mid-size bf16 products (too few 256 x 192 tiles for the wide kernel, so the 64 x 64
    four-stage kernel): M and N not multiples of the tile, K one stage or a few; sampled
    output rows."""
    dev = need_gpu()
    announce(f"linear mid {M}x{N}x{K}")
    x = I.normal((M, K), torch.bfloat16, dev, seed=4300 + K)
    w = I.normal((N, K), torch.bfloat16, dev, seed=4301 + K, std=K ** -0.5)
    y = gm.linear(x, w)
    torch.cuda.synchronize()
    rows = sorted(set(list(range(0, M, 97)) + [M - 1, M - 2, 255, 256]))
    ref = oracle.linear(host(x)[rows], host(w))
    check_rows_rel(host(y)[rows], ref, N)


@pytest.mark.parametrize("M,N,K", [(2000, 12200, 320), (2048, 12296, 1024), (1999, 12288, 1088),
                                   (2048, 12288, 1024), (3, 98304, 1024)])
def test_linear_large_tiles_ragged(M, N, K):
    """Products with enough large tiles to fill the CUs: 256 x 192 tiles (the first two: N
    not a multiple of 192, or K deep but N not a multiple of 384) and 256 x 384 tiles (K >=
    1024 and N a multiple of 384; M not a multiple of 256, an odd number of 64-deep
    stages, and three rows in 256-row tiles).  The output starts as NaN: every element is
    written; sampled rows match the oracle across the full width."""
    dev = need_gpu()
    announce(f"linear large tiles {M}x{N}x{K}")
    x = I.normal((M, K), torch.bfloat16, dev, seed=4400 + K)
    w = I.normal((N, K), torch.bfloat16, dev, seed=4401 + K, std=K ** -0.5)
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.linear(x, w, out=y)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    rows = sorted(r for r in set(list(range(0, M, 89)) + [M - 1, M - 2, 255, 256, 1791, 1792])
                  if 0 <= r < M)
    check_rows_rel(host(y)[rows], oracle.linear(host(x)[rows], host(w)), N)


@pytest.mark.parametrize("M,dc,dm", [(2000, 320, 6152), (2048, 1024, 6144)])
def test_latent_expand_large_tiles(M, dc, dm):
    """Both outputs of one launch in the large-tile kernels: 256 x 192 tiles with widths
    not a tile multiple, and 256 x 384 tiles (a 1024-wide latent); sampled rows."""
    dev = need_gpu()
    announce(f"latent_expand large tiles {M}x{dm}x{dc}")
    c = I.normal((M, dc), torch.bfloat16, dev, seed=4120 + dc)
    wk = I.normal((dm, dc), torch.bfloat16, dev, seed=4121 + dc, std=dc ** -0.5)
    wv = I.normal((dm, dc), torch.bfloat16, dev, seed=4122 + dc, std=dc ** -0.5)
    K, V = gm.latent_expand(c, wk, wv)
    torch.cuda.synchronize()
    rows = sorted(set(list(range(0, M, 127)) + [M - 1, 255, 256]))
    for got, w in ((K, wk), (V, wv)):
        assert not torch.isnan(got).any()
        check_rows_rel(host(got)[rows], oracle.linear(host(c)[rows], host(w)), dm)


def test_latent_expand_wide_ragged():
    """Both outputs of one launch in the 64 x 64 four-stage kernel, widths not a tile
    multiple."""
    dev = need_gpu()
    announce("latent_expand wide 2000x4104x320")
    M, dc, dm = 2000, 320, 4104
    c = I.normal((M, dc), torch.bfloat16, dev, seed=4110)
    wk = I.normal((dm, dc), torch.bfloat16, dev, seed=4111, std=dc ** -0.5)
    wv = I.normal((dm, dc), torch.bfloat16, dev, seed=4112, std=dc ** -0.5)
    K, V = gm.latent_expand(c, wk, wv)
    torch.cuda.synchronize()
    rows = sorted(set(list(range(0, M, 131)) + [M - 1, 1999 - 256]))
    for got, w in ((K, wk), (V, wv)):
        check_rows_rel(host(got)[rows], oracle.linear(host(c)[rows], host(w)), dm)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_latent_expand(dtype):
    dev = need_gpu()
    announce(f"latent_expand {dtype}")
    M, dc, dm = 150, 64, 384
    c = I.normal((M, dc), dtype, dev, seed=4100)
    wk = I.normal((dm, dc), dtype, dev, seed=4101, std=dc ** -0.5)
    wv = I.normal((dm, dc), dtype, dev, seed=4102, std=dc ** -0.5)
    K, V = gm.latent_expand(c, wk, wv)
    torch.cuda.synchronize()
    for got, w in ((K, wk), (V, wv)):
        ref = oracle.linear(host(c), host(w))
        if dtype == torch.float32:
            check_f32_abs(host(got), ref, 1e-4)
        else:
            check_rows_rel(host(got), ref, dm)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("with_gate,with_proj", [(True, True), (True, False), (False, True)])
def test_gate_out(dtype, with_gate, with_proj):
    dev = need_gpu()
    announce(f"gate_out {dtype} gate={with_gate} proj={with_proj}")
    M, dm = 96, 256
    o = I.normal((M, dm), dtype, dev, seed=4200)
    g = I.normal((M, dm), dtype, dev, seed=4201) if with_gate else None
    w = I.normal((dm, dm), dtype, dev, seed=4202, std=dm ** -0.5) if with_proj else None
    y = gm.gate_out(o, w, g)
    torch.cuda.synchronize()
    ref = host(o)
    if with_gate:
        ref = oracle.gate(host(g), ref)
    if with_proj:
        ref = oracle.linear(ref, host(w))
    if dtype == torch.float32:
        check_f32_abs(host(y), ref, 1e-4)
    else:
        check_rows_rel(host(y), ref, dm)


def test_gate_example_on_gpu():
    """'Gated MLA', 'A small causal example': 1.6 with gate logit 0 becomes 0.8
    (exact in fp32; in bf16, bf16(1.6)/2 = bf16(0.8))."""
    dev = need_gpu()
    announce("gate example")
    for dtype in (torch.float32, torch.bfloat16):
        o = torch.full((1, 8), 1.6, dtype=dtype, device=dev)
        g = torch.zeros((1, 8), dtype=dtype, device=dev)
        y = gm.gate_out(o, None, g)
        assert torch.all(y == torch.tensor(0.8, dtype=dtype)).item()


# ---------------------------------------------------------------- layer


@pytest.mark.parametrize("dtype,dm,H,dc", [(torch.bfloat16, 256, 2, 64), (torch.float32, 128, 4, 32),
                                           (torch.bfloat16, 384, 3, 128)])
@pytest.mark.parametrize("causal", [True, False])
def test_gated_mla_layer_small(dtype, dm, H, dc, causal):
    dev = need_gpu()
    announce(f"gated_mla {dtype} dm={dm} H={H} dc={dc} causal={causal}")
    B, T = 2, 100
    x, ws = I.layer_inputs(B, T, dm, dc, dtype, dev, seed=5000 + dm)
    saved = {n: w.clone() for n, w in ws.items()}
    xs = x.clone()
    res = gm.gated_mla(x, ws["Wq"], ws["Wc"], ws["Wk"], ws["Wv"], ws["Wg"], ws["Wo"], H, causal)
    torch.cuda.synchronize()
    assert set(res) == {"output", "latent_cache"}
    assert res["output"].shape == x.shape and res["output"].dtype == x.dtype
    assert res["latent_cache"].shape == (B, T, dc)
    assert torch.equal(x, xs) and all(torch.equal(ws[n], saved[n]) for n in ws)
    ref = oracle.gated_mla_layer(host(x), *(host(ws[n]) for n in ("Wq", "Wc", "Wk", "Wv", "Wg", "Wo")),
                                 H, causal)
    if dtype == torch.float32:
        check_f32_abs(host(res["latent_cache"]), ref["latent_cache"], 1e-4)
        check_f32_abs(host(res["output"]), ref["output"], 1e-4)
    else:
        check_rows_rel(host(res["latent_cache"]), ref["latent_cache"], dc)
        check_rows_rel(host(res["output"]), ref["output"], dm)
    other = gm.gated_mla(x, ws["Wq"], ws["Wc"], ws["Wk"], ws["Wv"], ws["Wg"], ws["Wo"], H, not causal)
    assert torch.equal(other["latent_cache"], res["latent_cache"])
