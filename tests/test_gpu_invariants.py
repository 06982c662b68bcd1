"""GPU invariants that need no oracle: facts of the softmax definition that must hold
exactly (or to the output rounding) for any correct kernel."""
import numpy as np
import pytest
import torch

import causal_softmax_attention_gmla_amd as gm
from causal_softmax_attention_gmla_amd import inputs as I
from gpu_helpers import announce, host, need_gpu

pytestmark = pytest.mark.gpu

BF16_ULP = 2.0 ** -8


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_constant_values_give_constant_output(dtype, D):
    """V = c on every key gives O = c: the weights of each row sum to one."""
    dev = need_gpu()
    announce(f"invariant constant V {dtype}")
    q, k, _, _ = I.prefill_inputs(2, 333, 3, D, dtype, dev, seed=6000)
    v = torch.full_like(q, 1.0)
    out = host(gm.attend_prefill(q, k, v))
    assert np.max(np.abs(out - 1.0)) <= (BF16_ULP if dtype == torch.bfloat16 else 1e-6)
    kd = k.permute(0, 2, 1, 3)
    dec = host(gm.attend_decode(q[:, -1].contiguous(), kd, torch.full_like(kd, 1.0), num_splits=3))
    assert np.max(np.abs(dec - 1.0)) <= (BF16_ULP if dtype == torch.bfloat16 else 1e-6)


def test_identity_values_reveal_causal_weights():
    """V rows = unit vectors e_s (T <= 128 = D): output row t is A[t, :], whose upper
    triangle must be exactly zero and whose rows sum to one."""
    dev = need_gpu()
    announce("invariant identity V")
    T, D = 100, 128
    q, k, _, _ = I.prefill_inputs(1, T, 2, D, torch.bfloat16, dev, seed=6100)
    v = torch.zeros_like(q)
    for s in range(T):
        v[0, s, :, s] = 1.0
    A = host(gm.attend_prefill(q, k, v)).reshape(T, 2, D)[:, :, :T]
    for h in range(2):
        assert np.all(np.triu(A[:, h], 1) == 0.0)
        assert np.all(np.tril(A[:, h]) >= 0.0)
        assert np.max(np.abs(A[:, h].sum(axis=1) - 1.0)) <= 2e-2


def test_future_keys_do_not_change_past_rows_bitwise():
    """Changing K and V at positions s > t0 leaves every output row t <= t0 bitwise
    unchanged (keys after the query are removed before normalisation)."""
    dev = need_gpu()
    announce("invariant causal bitwise")
    B, T, H, D = 1, 390, 2, 128
    q, k, v, _ = I.prefill_inputs(B, T, H, D, torch.bfloat16, dev, seed=6200)
    a = gm.attend_prefill(q, k, v).clone()
    t0 = 200
    k2, v2 = k.clone(), v.clone()
    k2[:, t0 + 1:] = (I.normal(k2[:, t0 + 1:].shape, torch.float32, dev, seed=6201) * 8).to(k.dtype)
    v2[:, t0 + 1:] = -5.0
    b = gm.attend_prefill(q, k2, v2)
    assert torch.equal(a[:, : t0 + 1], b[:, : t0 + 1])
    assert not torch.equal(a[:, t0 + 1:], b[:, t0 + 1:])


@pytest.mark.parametrize("off", [0, 64, 100, 191])
@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 64)])
def test_chunk_rows_equal_full_prefill_rows(off, dtype, D):
    """Positions continue from the cached length ('Kimi K2 - Construct causal mask'): the
    attention of the last T - off queries as a chunk over all T keys is, row for row,
    the causal prefill of the whole sequence.  Each row sees the same keys in the same
    tile order, and the extra tiles a chunk block may visit are fully masked for its
    rows (zero weights), so the rows agree bitwise."""
    dev = need_gpu()
    announce(f"invariant chunk == prefill rows off={off} {dtype}")
    B, T, H = 2, 333, 2
    q, k, v, g = I.prefill_inputs(B, T, H, D, dtype, dev, seed=6300 + off, gate=True)
    full = gm.attend_prefill(q, k, v, g)
    part = gm.attend_chunk(q[:, off:], k, v, g[:, off:].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(full[:, off:], part)


@pytest.mark.parametrize("dtype,D", [(torch.bfloat16, 128), (torch.float32, 32)])
def test_first_row_is_first_value_bitwise(dtype, D):
    """Query 0 sees only key 0: its weight is exactly 1 and the output is V[0]."""
    dev = need_gpu()
    announce(f"invariant first row {dtype}")
    q, k, v, _ = I.prefill_inputs(2, 77, 3, D, dtype, dev, seed=6300)
    out = gm.attend_prefill(q, k, v)
    assert torch.equal(out[:, 0], v[:, 0].reshape(2, 3 * D))
    one = gm.attend_prefill(q[:, :1].contiguous(), k[:, :1].contiguous(), v[:, :1].contiguous())
    assert torch.equal(one[:, 0], v[:, 0].reshape(2, 3 * D))


def test_zero_query_gives_prefix_mean():
    """Q = 0: equal scores, uniform weights, output = causal prefix mean of V."""
    dev = need_gpu()
    announce("invariant zero query")
    B, T, H, D = 1, 300, 2, 128
    _, k, v, _ = I.prefill_inputs(B, T, H, D, torch.bfloat16, dev, seed=6400)
    q = torch.zeros_like(k)
    out = host(gm.attend_prefill(q, k, v)).reshape(B, T, H, D)
    vh = host(v)
    ref = np.cumsum(vh, axis=1) / np.arange(1, T + 1)[None, :, None, None]
    err = np.abs(out - ref).max(axis=-1) / np.abs(ref).max(axis=-1)
    assert np.max(err) <= 2e-2


def test_decode_split_counts_agree():
    """The log-sum-exp merge is an exact regrouping: any split count gives the same
    result up to float32 rounding (checked in fp32)."""
    dev = need_gpu()
    announce("invariant decode splits")
    q, k, v, _ = I.decode_inputs(2, 4, 3000, 128, torch.float32, dev, seed=6500)
    outs = [host(gm.attend_decode(q, k, v, num_splits=s)) for s in (1, 2, 5, 16, 0)]
    for o in outs[1:]:
        assert np.max(np.abs(o - outs[0])) <= 1e-6


def test_repeated_runs_bitwise_identical():
    dev = need_gpu()
    announce("invariant determinism")
    q, k, v, g = I.prefill_inputs(2, 600, 4, 128, torch.bfloat16, dev, seed=6600, gate=True)
    a = gm.attend_prefill(q, k, v, g).clone()
    for _ in range(3):
        assert torch.equal(gm.attend_prefill(q, k, v, g), a)
    qd, kd, vd, _ = I.decode_inputs(4, 8, 5000, 128, torch.bfloat16, dev, seed=6601)
    d = gm.attend_decode(qd, kd, vd).clone()
    for _ in range(3):
        assert torch.equal(gm.attend_decode(qd, kd, vd), d)


def test_repeated_runs_bitwise_identical_projections_and_latent_forms():
    """Run-to-run bitwise repeatability of the other kernels (a race on LDS stages, a
    counter or a split-K partial would show as differing bits): the 256 x 384-tile GEMM
    (loads issued among its MFMAs) and its dual-output latent expansion, the split-K
    down-projection with its reduce, the gated output projection through the gate pass,
    the decode over the latent cache and the latent-fused prefill."""
    dev = need_gpu()
    announce("invariant determinism: projections and latent forms")
    x = I.normal((2048, 1024), torch.bfloat16, dev, seed=6900)
    w = I.normal((12288, 1024), torch.bfloat16, dev, seed=6901, std=1024 ** -0.5)
    c = I.normal((2048, 512), torch.bfloat16, dev, seed=6902)
    wk = I.normal((6144, 512), torch.bfloat16, dev, seed=6903, std=512 ** -0.5)
    wv = I.normal((6144, 512), torch.bfloat16, dev, seed=6904, std=512 ** -0.5)
    xc = I.normal((2048, 6144), torch.bfloat16, dev, seed=6905)
    wc = I.normal((512, 6144), torch.bfloat16, dev, seed=6906, std=6144 ** -0.5)
    g = I.normal((2048, 6144), torch.bfloat16, dev, seed=6907)
    wo = I.normal((6144, 6144), torch.bfloat16, dev, seed=6908, std=6144 ** -0.5)
    q, lc, lwk, lwv, lg = (I.normal((4, 16, 128), torch.bfloat16, dev, seed=6909),
                           I.normal((4, 1001, 512), torch.bfloat16, dev, seed=6910),
                           I.normal((16 * 128, 512), torch.bfloat16, dev, seed=6911, std=512 ** -0.5),
                           I.normal((16 * 128, 512), torch.bfloat16, dev, seed=6912, std=512 ** -0.5),
                           I.normal((4, 16 * 128), torch.bfloat16, dev, seed=6913))
    qp = I.normal((1, 640, 8, 128), torch.bfloat16, dev, seed=6914)
    cp = I.normal((1, 640, 512), torch.bfloat16, dev, seed=6915)
    runs = {
        "linear 256x384 tiles": lambda: gm.linear(x, w),
        "latent expansion": lambda: torch.cat(gm.latent_expand(c, wk, wv), dim=1),
        "split-K down-projection": lambda: gm.linear(xc, wc),
        "gated output projection": lambda: gm.gate_out(xc, wo, g),
        "latent-cache decode": lambda: gm.attend_decode_latent(q, lc, lwk, lwv, lg),
        "latent-fused prefill": lambda: gm.attend_prefill_latent(qp, cp, lwk[:1024], lwv[:1024]),
    }
    for name, fn in runs.items():
        first = fn().clone()
        for _ in range(2):
            assert torch.equal(fn(), first), name


def test_inputs_not_mutated():
    """'Gated MLA', 'Requirements': no input tensor is modified."""
    dev = need_gpu()
    announce("invariant inputs unchanged")
    q, k, v, g = I.prefill_inputs(1, 130, 2, 128, torch.bfloat16, dev, seed=6700, gate=True)
    saved = [t.clone() for t in (q, k, v, g)]
    gm.attend_prefill(q, k, v, g)
    qd, kd, vd, gd = I.decode_inputs(1, 2, 700, 128, torch.bfloat16, dev, seed=6701, gate=True)
    saved_d = [t.clone() for t in (qd, kd, vd, gd)]
    gm.attend_decode(qd, kd, vd, gd, num_splits=3)
    torch.cuda.synchronize()
    assert all(torch.equal(a, b) for a, b in zip((q, k, v, g), saved))
    assert all(torch.equal(a, b) for a, b in zip((qd, kd, vd, gd), saved_d))


def _saturating_logits(shape, dtype, dev):
    """Gate logits cycling over the channels through values far in both tails, where the
    sigmoid is exactly 0 or 1 in float32, and zero (one half)."""
    vals = torch.tensor([-float("inf"), -1e4, -200.0, -100.0, 0.0, 30.0, 100.0, 200.0, 1e4,
                         float("inf")], dtype=torch.float32)
    n = shape[-1]
    row = vals[torch.arange(n) % len(vals)]
    return row.expand(*shape).contiguous().to(dtype).to(dev), row


def _check_saturation(gated, plain, row):
    """Channels with logit <= -100 must come out exactly 0 (1 / (1 + e^100) is below the
    float32 range), those with logit >= 30 exactly the ungated value (the sigmoid rounds
    to 1), those with logit 0 half of it to the output rounding; nothing non-finite."""
    g = gated.reshape(-1, row.numel())
    p = plain.reshape(-1, row.numel())
    assert np.all(np.isfinite(g))
    lo, hi, mid = (row <= -100).numpy(), (row >= 30).numpy(), (row == 0).numpy()
    assert np.all(g[:, lo] == 0.0)
    assert np.array_equal(g[:, hi], p[:, hi])
    assert np.max(np.abs(g[:, mid] - 0.5 * p[:, mid])) <= BF16_ULP * np.max(np.abs(p)) + 1e-7


def test_gate_saturation_every_gated_path():
    """The sigmoid gate at its extremes ('Gated MLA', 'The channel-wise output gate':
    the gate scales each channel by a number in (0, 1)): the prefill epilogue (logits
    staged through LDS), the decode epilogue, and the gate pass of the output projection
    (bf16 and float32) give exact zeros, exact pass-through and a clean half."""
    dev = need_gpu()
    announce("invariant gate saturation")
    q, k, v, _ = I.prefill_inputs(2, 200, 3, 128, torch.bfloat16, dev, seed=6800)
    g, row = _saturating_logits((2, 200, 3 * 128), torch.bfloat16, dev)
    _check_saturation(host(gm.attend_prefill(q, k, v, g)), host(gm.attend_prefill(q, k, v)), row)
    qd, kd, vd, _ = I.decode_inputs(2, 3, 700, 128, torch.bfloat16, dev, seed=6801)
    gd, row = _saturating_logits((2, 3 * 128), torch.bfloat16, dev)
    _check_saturation(host(gm.attend_decode(qd, kd, vd, gd)), host(gm.attend_decode(qd, kd, vd)), row)
    for dtype in (torch.bfloat16, torch.float32):
        o = I.normal((64, 640), dtype, dev, seed=6802)
        go, row = _saturating_logits((64, 640), dtype, dev)
        _check_saturation(host(gm.gate_out(o, None, go)), host(o), row)
