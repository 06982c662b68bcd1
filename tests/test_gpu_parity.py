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
    XCD and at most three blocks per workgroup slot (10 to 18 blocks per XCD): each XCD
    launches all its heads as one group, heaviest blocks first, and every (head, query
    block) must still be computed exactly once.  Groups of four with a partial last group
    are covered at full size (test_prefill_partial_last_head_group)."""
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


def oracle_latent_decode(q, c, wk, wv, g, heads):
    """The oracle's plain composition for decode over a latent cache: per (b, h), the keys
    K_h = C_b W_k,h^T and values V_h = C_b W_v,h^T in double, then the softmax of the
    query at position N-1 over all N keys, then the gate.  Returns {(b, h): [1, D]}."""
    D = q.shape[-1]
    hc, hq, hwk, hwv = host(c), host(q), host(wk), host(wv)
    hg = host(g) if g is not None else None
    out = {}
    for b, h in heads:
        kh = oracle.linear(hc[b], hwk[h * D:(h + 1) * D])
        vh = oracle.linear(hc[b], hwv[h * D:(h + 1) * D])
        ref = oracle.attend_head(hq[b, h][None, :], kh, vh, 1 / np.sqrt(D), True)
        if hg is not None:
            ref = oracle.gate(hg[b, h * D:(h + 1) * D][None, :], ref)
        out[(b, h)] = ref
    return out


def latent_inputs(B, N, H, dc, dev, seed, gate, packed=False):
    D = 128
    q = I.normal((B, H, D), torch.bfloat16, dev, seed=seed)
    if packed:  # latent rows as a strided view: [B, N, 2, d_c] buffer, first half of each row
        c = I.normal((B, N, 2, dc), torch.bfloat16, dev, seed=seed + 1)[:, :, 0]
    else:
        c = I.normal((B, N, dc), torch.bfloat16, dev, seed=seed + 1)
    wk = I.normal((H * D, dc), torch.bfloat16, dev, seed=seed + 2, std=dc ** -0.5)
    wv = I.normal((H * D, dc), torch.bfloat16, dev, seed=seed + 3, std=dc ** -0.5)
    g = I.normal((B, H * D), torch.bfloat16, dev, seed=seed + 4) if gate else None
    return q, c, wk, wv, g


@pytest.mark.parametrize("B,N,H,dc,gate,splits,packed", [
    (2, 300, 4, 128, True, 0, False), (2, 1, 3, 256, False, 0, False), (1, 33, 40, 512, True, 3, False),
    (3, 1000, 8, 512, False, 7, True), (2, 64, 2, 128, False, 2, False), (1, 31, 1, 512, True, 0, False),
    (2, 777, 33, 256, True, 1, True), (1, 4100, 5, 512, False, 0, False),
    (1, 96, 2, 512, False, 1, False), (1, 200, 3, 256, True, 1, False), (2, 190, 2, 128, False, 1, False)])
def test_decode_latent_cache(B, N, H, dc, gate, splits, packed):
    """Decode over the latent cache (keys and values never formed) on every head, against
    the oracle's composition: ragged cache lengths (1, 31, 33 against the 32-row tiles),
    a partial 32-head block (H = 33, 40), one to seven key ranges, latent widths 128, 256
    and 512, strided latent rows, with and without the gate."""
    dev = need_gpu()
    announce(f"decode over latent cache B={B} N={N} H={H} d_c={dc} splits={splits} packed={packed}")
    q, c, wk, wv, g = latent_inputs(B, N, H, dc, dev, 3300 + N + dc, gate, packed)
    out = torch.full((B, H * 128), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.attend_decode_latent(q, c, wk, wv, g, num_splits=splits, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    heads = [(b, h) for b in range(B) for h in range(H)]
    ref = oracle_latent_decode(q, c, wk, wv, g, heads)
    got = host(out).reshape(B, H, 128)
    for (b, h), r in ref.items():
        check_rows_rel(got[b, h][None], r, 128)


@pytest.mark.parametrize("dc,splits,gate", [(512, 0, True), (512, 7, False), (128, 3, True)])
def test_decode_latent_per_row_lengths(dc, splits, gate):
    """Latent-cache decode with a cache length per batch row (0, 1, 31, 33, 700 and the
    full capacity): each row against the oracle's composition over its own rows (an empty
    row is zeros), key ranges past a row's length left empty, and a full-length row equal
    to the fixed-length call bit for bit."""
    dev = need_gpu()
    announce(f"decode over latent cache, per-row lengths, d_c={dc} splits={splits}")
    lens = [0, 1, 31, 33, 700, 1000]
    B, N, H = len(lens), 1000, 5
    q, c, wk, wv, g = latent_inputs(B, N, H, dc, dev, 3970 + dc + splits, gate)
    kv = torch.tensor(lens, dtype=torch.int32, device=dev)
    out = torch.full((B, H * 128), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.attend_decode_latent(q, c, wk, wv, g, num_splits=splits, out=out, kv_lens=kv)
    full = gm.attend_decode_latent(q, c, wk, wv, g, num_splits=splits)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    got = host(out).reshape(B, H, 128)
    assert np.all(got[0] == 0.0)
    assert torch.equal(out[B - 1], full[B - 1])
    hq, hc, hwk, hwv = host(q), host(c), host(wk), host(wv)
    hg = host(g) if g is not None else None
    for b, n in enumerate(lens):
        if n == 0:
            continue
        for h in range(H):
            kh = oracle.linear(hc[b, :n], hwk[h * 128:(h + 1) * 128])
            vh = oracle.linear(hc[b, :n], hwv[h * 128:(h + 1) * 128])
            ref = oracle.attend_head(hq[b, h][None, :], kh, vh, 1 / np.sqrt(128), True)
            if hg is not None:
                ref = oracle.gate(hg[b, h * 128:(h + 1) * 128][None, :], ref)
            check_rows_rel(got[b, h][None], ref, 128)


def test_decode_latent_graph_replay_matches_eager():
    """The latent-cache decode captured in a HIP graph: replayed three times, with new
    queries written eagerly and the stream synchronised between replays, every replay's
    output equals an eager call on the same inputs bit for bit."""
    dev = need_gpu()
    announce("decode latent graph replay")
    B, N, H, dc = 3, 1001, 40, 512
    q, c, wk, wv, g = latent_inputs(B, N, H, dc, dev, 3950, True)
    ws = torch.empty(gm.decode_latent_workspace_bytes(B, H, N, dc), dtype=torch.uint8, device=dev)
    out = torch.empty((B, H * 128), dtype=torch.bfloat16, device=dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        gm.attend_decode_latent(q, c, wk, wv, g, workspace=ws, out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gm.attend_decode_latent(q, c, wk, wv, g, workspace=ws, out=out)
    for rep in range(3):
        q.copy_(I.normal((B, H, 128), torch.bfloat16, dev, seed=3960 + rep))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = out.clone()
        eager = gm.attend_decode_latent(q, c, wk, wv, g)
        torch.cuda.synchronize()
        assert torch.equal(got, eager), f"replay {rep}"
    heads = [(0, 0), (1, 17), (2, 39)]
    ref = oracle_latent_decode(q, c, wk, wv, g, heads)
    hgot = host(got).reshape(B, H, 128)
    for (b, h), r in ref.items():
        check_rows_rel(hgot[b, h][None], r, 128)


def test_decode_latent_matches_direct_decode_on_expanded_cache():
    """The same attention two ways on the GPU: over the latent cache, and the plain decode
    over K = C W_k^T, V = C W_v^T formed by the latent expansion (both against the same
    oracle rows, and within the bf16 rule of each other)."""
    dev = need_gpu()
    announce("decode latent vs direct decode on the expanded cache")
    B, N, H, dc, D = 2, 500, 6, 512, 128
    q, c, wk, wv, _ = latent_inputs(B, N, H, dc, dev, 3900, False)
    lat = host(gm.attend_decode_latent(q, c, wk, wv))
    kf, vf = gm.latent_expand(c, wk, wv)
    k = kf.view(B, N, H, D).permute(0, 2, 1, 3)
    v = vf.view(B, N, H, D).permute(0, 2, 1, 3)
    direct = host(gm.attend_decode(q, k, v))
    torch.cuda.synchronize()
    check_rows_rel(lat, direct, D)


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
        check_f32_abs(host(y), ref)
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
    not a multiple of 192 with K below 512, or K deep but N not a multiple of 384) and
    256 x 384 tiles (K >= 512 and N a multiple of 384; M not a multiple of 256, an odd
    number of 64-deep stages, and three rows in 256-row tiles).  The output starts as NaN:
    every element is written; sampled rows match the oracle across the full width."""
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


@pytest.mark.parametrize("M,dc,dm", [(2000, 320, 6152), (2048, 1024, 6144), (2048, 512, 6144),
                                     (1999, 576, 6144)])
def test_latent_expand_large_tiles(M, dc, dm):
    """Both outputs of one launch in the large-tile kernels: 256 x 192 tiles with widths
    not a tile multiple (a 320-wide latent), and 256 x 384 tiles (latents of 1024, 512 -
    the pages' width, eight 64-deep stages - and 576, nine stages with a ragged last
    row block); sampled rows."""
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
            check_f32_abs(host(got), ref)
        else:
            check_rows_rel(host(got), ref, dm)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("with_gate,with_proj,fused_gate", [(True, True, False), (True, True, True),
                                                            (True, False, False), (False, True, False)])
@pytest.mark.parametrize("M,dm", [(96, 256), (333, 320)])
def test_gate_out(dtype, with_gate, with_proj, fused_gate, M, dm):
    """Both routes of the gated projection (gate pass into a workspace + LDS GEMM, and the
    gate in the GEMM's tile staging), with a row count that leaves a ragged tile."""
    dev = need_gpu()
    announce(f"gate_out {dtype} gate={with_gate} proj={with_proj} fused={fused_gate} M={M} dm={dm}")
    o = I.normal((M, dm), dtype, dev, seed=4200)
    g = I.normal((M, dm), dtype, dev, seed=4201) if with_gate else None
    w = I.normal((dm, dm), dtype, dev, seed=4202, std=dm ** -0.5) if with_proj else None
    y = gm.gate_out(o, w, g, fused_gate=fused_gate)
    torch.cuda.synchronize()
    ref = host(o)
    if with_gate:
        ref = oracle.gate(host(g), ref)
    if with_proj:
        ref = oracle.linear(ref, host(w))
    if dtype == torch.float32:
        check_f32_abs(host(y), ref)
    else:
        check_rows_rel(host(y), ref, dm)


def test_gate_only_unaligned_rows_match_aligned():
    """The bf16 gate pass takes 8 elements per lane when every pointer is 16-byte aligned
    and one element per lane otherwise; both round the same float to bf16."""
    dev = need_gpu()
    announce("gate only, aligned vs 2-byte offset views")
    M, dm = 37, 264
    ob = I.normal((M * dm + 1,), torch.bfloat16, dev, seed=4210)
    gb = I.normal((M * dm + 1,), torch.bfloat16, dev, seed=4211)
    y_al = gm.gate_out(ob[:-1].view(M, dm), None, gb[:-1].view(M, dm))
    o_un, g_un = ob[:-1].clone(), gb[:-1].clone()
    buf_o = torch.empty(M * dm + 1, dtype=torch.bfloat16, device=dev)
    buf_g = torch.empty(M * dm + 1, dtype=torch.bfloat16, device=dev)
    buf_o[1:] = o_un
    buf_g[1:] = g_un
    y_un = gm.gate_out(buf_o[1:].view(M, dm), None, buf_g[1:].view(M, dm))
    torch.cuda.synchronize()
    assert torch.equal(y_al, y_un)
    ref = oracle.gate(host(gb[:-1].view(M, dm)), host(ob[:-1].view(M, dm)))
    check_rows_rel(host(y_al), ref, dm)


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
        check_f32_abs(host(res["latent_cache"]), ref["latent_cache"])
        check_f32_abs(host(res["output"]), ref["output"])
    else:
        check_rows_rel(host(res["latent_cache"]), ref["latent_cache"], dc)
        check_rows_rel(host(res["output"]), ref["output"], dm)
    other = gm.gated_mla(x, ws["Wq"], ws["Wc"], ws["Wk"], ws["Wv"], ws["Wg"], ws["Wo"], H, not causal)
    assert torch.equal(other["latent_cache"], res["latent_cache"])


# ---------------------------------------------------------------- per-sequence lengths


def _packed(lengths, H, D, dtype, dev, seed, kv=False):
    """Rows of several sequences packed along one axis, and their int32 offsets."""
    total = int(sum(lengths))
    t = I.normal((max(total, 1), H, D), dtype, dev, seed)[:total]
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lengths)]), dtype=torch.int32, device=dev)
    return t, cu


def _oracle_varlen(q, k, v, g, tq, tk, causal):
    """Per sequence: query i at position i + Tk_b - Tq_b against that sequence's keys.  A
    query that sees no key (causal with Tq_b > Tk_b, or Tk_b = 0) is the zero row (the
    library's stated reading); the oracle runs on the queries that see at least one."""
    H, D = q.shape[1], q.shape[2]
    hq, hk, hv = host(q), host(k), host(v)
    out = np.zeros((hq.shape[0], H * D))
    q0 = k0 = 0
    for a, b in zip(tq, tk):
        # with Tq_b > Tk_b, queries 0 .. Tq_b - Tk_b - 1 sit before position 0
        skip = (max(0, a - b) if causal else 0) if b > 0 else a
        for h in range(H):
            if a > skip:
                qq = hq[q0 + skip:q0 + a, h]  # the last a - skip queries: positions from 0
                out[q0 + skip:q0 + a, h * D:(h + 1) * D] = oracle.attend_head(
                    qq, hk[k0:k0 + b, h], hv[k0:k0 + b, h], 1 / np.sqrt(D), causal)
        q0 += a
        k0 += b
    if g is not None:
        out = oracle.gate(host(g), out)
    return out


VARLEN_CASES = {
    # (query lengths, key lengths): ragged prefill (Tq = Tk), and chunks after different
    # cached lengths; lengths of 1 and off the 64-key and 128-query grids
    "prefill": ([1, 64, 129, 300, 7, 200], [1, 64, 129, 300, 7, 200]),
    "chunked": ([5, 128, 1, 70, 300], [1005, 200, 64, 70, 301]),
    "single": ([517], [517]),
}


@pytest.mark.parametrize("case", sorted(VARLEN_CASES))
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_bf16_mfma(case, causal):
    """Per-sequence lengths on the MFMA kernel: every sequence's rows against the oracle
    run on that sequence alone; Q, K, V as head views of packed buffers; gated."""
    dev = need_gpu()
    tq, tk = VARLEN_CASES[case]
    announce(f"varlen bf16 {case} causal={causal}")
    H, D = 3, 128
    q, cuq = _packed(tq, H, D, torch.bfloat16, dev, 8100)
    kv, cuk = _packed(tk, 2 * H, D, torch.bfloat16, dev, 8101)
    k, v = kv[:, :H], kv[:, H:]
    g = I.normal((q.shape[0], H * D), torch.bfloat16, dev, seed=8102)
    out = torch.full((q.shape[0], H * D), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.attend_varlen(q, k, v, cuq, cuk, max(tq), max(tk), g, causal=causal, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    check_rows_rel(host(out), _oracle_varlen(q, k, v, g, tq, tk, causal), D)


@pytest.mark.parametrize("D", [32, 64, 128])
def test_varlen_f32_exact(D):
    dev = need_gpu()
    tq, tk = [3, 65, 1, 40], [3, 130, 77, 40]
    announce(f"varlen f32 D={D}")
    H = 2
    q, cuq = _packed(tq, H, D, torch.float32, dev, 8200 + D)
    k, cuk = _packed(tk, H, D, torch.float32, dev, 8201 + D)
    v, _ = _packed(tk, H, D, torch.float32, dev, 8202 + D)
    out = gm.attend_varlen(q, k, v, cuq, cuk, max(tq), max(tk))
    torch.cuda.synchronize()
    check_f32_abs(host(out), _oracle_varlen(q, k, v, None, tq, tk, True))


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_varlen_equal_lengths_match_chunk_bitwise(dtype, D):
    """With every sequence the same length, the per-sequence call computes exactly what the
    fixed-shape chunk call does (same tiles, same order): bitwise equal rows."""
    dev = need_gpu()
    announce(f"varlen vs chunk bitwise {dtype}")
    B, Tq, Tk, H = 3, 130, 333, 2
    q = I.normal((B, Tq, H, D), dtype, dev, seed=8300)
    k = I.normal((B, Tk, H, D), dtype, dev, seed=8301)
    v = I.normal((B, Tk, H, D), dtype, dev, seed=8302)
    ref = gm.attend_chunk(q, k, v)
    cuq = torch.arange(0, (B + 1) * Tq, Tq, dtype=torch.int32, device=dev)
    cuk = torch.arange(0, (B + 1) * Tk, Tk, dtype=torch.int32, device=dev)
    got = gm.attend_varlen(q.reshape(B * Tq, H, D), k.reshape(B * Tk, H, D), v.reshape(B * Tk, H, D),
                           cuq, cuk, Tq, Tk)
    torch.cuda.synchronize()
    assert torch.equal(got.view(B, Tq, H * D), ref)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 32)])
def test_varlen_queries_without_keys_and_empty_sequences(dtype, D):
    """Sequences with more new queries than keys (the first Tq_b - Tk_b queries see no key
    and get zero rows), with no key at all, and with no query (nothing written for it;
    its neighbours' rows are unaffected)."""
    dev = need_gpu()
    announce(f"varlen empty cases {dtype}")
    tq, tk = [5, 0, 4, 3], [3, 10, 0, 3]
    H = 2
    q, cuq = _packed(tq, H, D, dtype, dev, 8400)
    k, cuk = _packed(tk, H, D, dtype, dev, 8401)
    v, _ = _packed(tk, H, D, dtype, dev, 8402)
    out = torch.full((q.shape[0], H * D), float("nan"), dtype=dtype, device=dev)
    gm.attend_varlen(q, k, v, cuq, cuk, max(tq), max(tk), out=out)
    torch.cuda.synchronize()
    got = host(out)
    assert np.all(got[0:2] == 0) and np.all(got[5:9] == 0)  # no visible key: zeros
    ref = _oracle_varlen(q, k, v, None, tq, tk, True)
    if dtype == torch.float32:
        check_f32_abs(got, ref)
    else:
        check_rows_rel(got[[2, 3, 4, 9, 10, 11]], ref[[2, 3, 4, 9, 10, 11]], D)


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_decode_varlen(splits, dtype):
    """Decode with a cache length per batch row (1001-key capacity, lengths 1001, 1, 0,
    500, 777, 64, 65, 1000): each row's query at position len - 1 against its first len
    keys; the empty row gives zeros."""
    dev = need_gpu()
    announce(f"decode varlen splits={splits} {dtype}")
    lens = [1001, 1, 0, 500, 777, 64, 65, 1000]
    B, H, N, D = len(lens), 4, 1001, 128
    q, k, v, g = I.decode_inputs(B, H, N, D, dtype, dev, seed=8500, gate=True)
    kl = torch.tensor(lens, dtype=torch.int32, device=dev)
    out = gm.attend_decode_varlen(q, k, v, kl, g, num_splits=splits)
    torch.cuda.synchronize()
    got = host(out).reshape(B, H, D)
    hq, hk, hv, hg = host(q), host(k), host(v), host(g).reshape(B, H, D)
    for b, n in enumerate(lens):
        for h in range(H):
            if n == 0:
                assert np.all(got[b, h] == 0)
                continue
            ref = oracle.attend_head(hq[b, h][None], hk[b, h, :n], hv[b, h, :n], 1 / np.sqrt(D), True)
            ref = oracle.gate(hg[b, h][None], ref)
            if dtype == torch.float32:
                check_f32_abs(got[b, h][None], ref)
            else:
                check_rows_rel(got[b, h][None], ref, D)


# ---------------------------------------------------------------- latent-fused prefill


def latent_prefill_inputs(B, T, H, dc, dev, seed, gate):
    D = 128
    q = I.normal((B, T, H, D), torch.bfloat16, dev, seed=seed)
    c = I.normal((B, T, dc), torch.bfloat16, dev, seed=seed + 1)
    wk = I.normal((H * D, dc), torch.bfloat16, dev, seed=seed + 2, std=dc ** -0.5)
    wv = I.normal((H * D, dc), torch.bfloat16, dev, seed=seed + 3, std=dc ** -0.5)
    g = I.normal((B, T, H * D), torch.bfloat16, dev, seed=seed + 4) if gate else None
    return q, c, wk, wv, g


def oracle_latent_prefill(q, c, wk, wv, g, causal):
    """The oracle's composition: K = C W_k^T and V = C W_v^T in double for every head,
    then each head's attention, the heads joined, then the gate."""
    B, T, H, D = q.shape
    hq, hc, hwk, hwv = host(q), host(c), host(wk), host(wv)
    out = np.empty((B, T, H * D))
    for b in range(B):
        K = oracle.linear(hc[b], hwk)
        V = oracle.linear(hc[b], hwv)
        for h in range(H):
            sl = slice(h * D, (h + 1) * D)
            out[b, :, sl] = oracle.attend_head(hq[b, :, h], K[:, sl], V[:, sl], 1 / np.sqrt(D), causal)
    if g is not None:
        out = oracle.gate(host(g), out)
    return out


@pytest.mark.parametrize("B,T,H,dc,causal,gate", [
    (2, 300, 3, 64, True, True), (1, 129, 2, 512, True, False), (2, 1, 4, 128, True, True),
    (1, 64, 2, 32, False, False), (1, 517, 5, 512, True, True), (3, 256, 2, 96, False, True)])
def test_prefill_latent(B, T, H, dc, causal, gate):
    """Keys and values rebuilt from the latent inside the attention launch, every element
    against the oracle's composition: ragged lengths (1, 129, 300, 517 against 128-row
    blocks), latent widths 32 to 512, causal and not, gated and not.  The launch's error
    word (set only if a wait for an expansion ran out) stays 0."""
    dev = need_gpu()
    announce(f"prefill latent B={B} T={T} H={H} d_c={dc} causal={causal} gate={gate}")
    q, c, wk, wv, g = latent_prefill_inputs(B, T, H, dc, dev, 9100 + T + dc, gate)
    need = gm.prefill_latent_workspace_bytes(B, T, H, 128)
    ws = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev)
    out = torch.full((B, T, H * 128), float("nan"), dtype=torch.bfloat16, device=dev)
    gm.attend_prefill_latent(q, c, wk, wv, g, causal=causal, workspace=ws, out=out)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any()
    assert int(ws[-4:].view(torch.int32).item()) == 0  # error word (the workspace's last int)
    check_rows_rel(host(out), oracle_latent_prefill(q, c, wk, wv, g, causal), 128)


@pytest.mark.parametrize("dc", [64, 512])
def test_prefill_latent_matches_expand_then_prefill_bitwise(dc):
    """The fused launch forms each key and value with the same products in the same order
    as the latent expansion, and attends with the same kernel code: bitwise equal to
    latent_expand followed by attend_prefill, on two calls in a row (the workspace's
    flags are cleared by each call)."""
    dev = need_gpu()
    announce(f"prefill latent vs expand + prefill d_c={dc}")
    B, T, H = 2, 700, 3
    q, c, wk, wv, g = latent_prefill_inputs(B, T, H, dc, dev, 9200 + dc, True)
    K, V = gm.latent_expand(c, wk, wv)
    ref = gm.attend_prefill(q, K.view(B, T, H, 128), V.view(B, T, H, 128), g)
    ws = torch.empty(gm.prefill_latent_workspace_bytes(B, T, H, 128), dtype=torch.uint8, device=dev)
    for _ in range(2):
        got = gm.attend_prefill_latent(q, c, wk, wv, g, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(got, ref)


@pytest.mark.parametrize("causal", [True, False])
def test_gated_mla_layer_fused_latent(causal):
    """The layer with the keys and values rebuilt inside the attention launch, against
    the oracle layer, and equal to the two-launch layer."""
    dev = need_gpu()
    announce(f"gated_mla fused latent causal={causal}")
    B, T, dm, H, dc = 2, 200, 384, 3, 128
    x, ws = I.layer_inputs(B, T, dm, dc, torch.bfloat16, dev, seed=9300)
    res = gm.gated_mla(x, ws["Wq"], ws["Wc"], ws["Wk"], ws["Wv"], ws["Wg"], ws["Wo"], H, causal,
                       fused_latent=True)
    two = gm.gated_mla(x, ws["Wq"], ws["Wc"], ws["Wk"], ws["Wv"], ws["Wg"], ws["Wo"], H, causal)
    torch.cuda.synchronize()
    ref = oracle.gated_mla_layer(host(x), *(host(ws[n]) for n in ("Wq", "Wc", "Wk", "Wv", "Wg", "Wo")),
                                 H, causal)
    check_rows_rel(host(res["output"]), ref["output"], dm)
    assert torch.equal(res["latent_cache"], two["latent_cache"])
    assert torch.equal(res["output"], two["output"])


# ---------------------------------------------------------------- split-K projection


@pytest.mark.parametrize("M,N,K", [(300, 264, 4096), (1, 8, 8192), (130, 136, 2048), (2000, 520, 6144)])
def test_linear_split_k(M, N, K):
    """Products with few output tiles and a deep K take the split-K path (float partials
    in a workspace, then a summing kernel): every row against the oracle, and the output
    written inside its buffer only (NaN guard band around it)."""
    dev = need_gpu()
    lib = gm.library()
    assert lib.gmla_linear_workspace_bytes(M, N, K) > 0
    announce(f"linear split-K {M}x{N}x{K}")
    x = I.normal((M, K), torch.bfloat16, dev, seed=9400 + K)
    w = I.normal((N, K), torch.bfloat16, dev, seed=9401 + K, std=K ** -0.5)
    buf = torch.full((M * N + 2048,), float("nan"), dtype=torch.bfloat16, device=dev)
    y = buf[1024:1024 + M * N].view(M, N)
    gm.linear(x, w, out=y)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert torch.isnan(buf[:1024]).all() and torch.isnan(buf[1024 + M * N:]).all()
    check_rows_rel(host(y), oracle.linear(host(x), host(w)), N)
    # without the workspace the same call runs the single-pass kernels
    z = gm.linear(x, w, split_k=False)
    torch.cuda.synchronize()
    check_rows_rel(host(z), host(y), N)
