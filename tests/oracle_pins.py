"""Pins for the CPU oracle: facts the pages and plain mathematics fix, independent of
the oracle's own code.

Each ``pin_*`` function takes an oracle object ``orc`` (the ``oracle`` package, or a
deliberately broken copy of it in the mutant tests) and raises AssertionError when
the oracle disagrees with the fact.  None of them re-types the oracle's formula:
they use values the pages print, closed forms (prefix means, constants, one-hot
limits, a two-key logistic), invariants (row sums, causality, permutations) and
hand-computed small products.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- softmax


def pin_rows_sum_to_one(orc):
    """Kimi K3 - Softmax over keys: weights over a query's keys sum to one."""
    r = _rng(1)
    for causal in (True, False):
        q, k, v = r.standard_normal((37, 8)), r.standard_normal((37, 8)), r.standard_normal((37, 8))
        _, A = orc.attend_head(q, k, v, 0.35, causal, want_probs=True)
        assert np.all(np.abs(A.sum(axis=1) - 1.0) <= 1e-12), "attention rows do not sum to 1"
        assert np.all(A >= 0.0)


def pin_causal_zero_upper(orc):
    """Kimi K2 - Construct causal mask: M = -inf for s > t, so A[t,s] = 0 there."""
    r = _rng(2)
    T = 29
    q, k, v = r.standard_normal((T, 6)), r.standard_normal((T, 6)), r.standard_normal((T, 6))
    _, A = orc.attend_head(q, k, v, 0.4, True, want_probs=True)
    upper = np.triu(np.ones((T, T), bool), 1)
    assert np.all(A[upper] == 0.0), "weight on a future key"
    assert np.all(A[~upper] > 0.0), "a visible key got zero weight"


def pin_visible_pair_count(orc):
    """Le Transformer et l'attention, 'Le coût quadratique': causal attention computes
    about T^2/2 dot products -- exactly T(T+1)/2 visible (query, key) pairs, each with a
    positive weight; without the mask all T^2."""
    r = _rng(13)
    for T in (1, 2, 7, 64, 100):
        q, k, v = r.standard_normal((T, 4)), r.standard_normal((T, 4)), r.standard_normal((T, 4))
        _, A = orc.attend_head(q, k, v, 0.5, True, want_probs=True)
        assert int(np.count_nonzero(A)) == T * (T + 1) // 2
        _, A = orc.attend_head(q, k, v, 0.5, False, want_probs=True)
        assert int(np.count_nonzero(A)) == T * T


def pin_three_token_example(orc):
    """Gated MLA, 'A small causal example': the lower-triangular pattern at T = 3,
    and every key visible in non-causal mode."""
    g = _golden("three_token_example.json")
    T = g["T"]
    r = _rng(3)
    q, k, v = r.standard_normal((T, 4)), r.standard_normal((T, 4)), r.standard_normal((T, 4))
    _, A = orc.attend_head(q, k, v, 0.5, True, want_probs=True)
    vis = np.array(g["visible"], bool)
    assert np.array_equal(A > 0, vis), f"pattern {A > 0} != {vis}"
    assert A[0, 0] == 1.0 and A[0, 1] == 0.0 and A[0, 2] == 0.0
    _, An = orc.attend_head(q, k, v, 0.5, False, want_probs=True)
    assert np.array_equal(An > 0, np.array(g["noncausal_visible"], bool))


def pin_single_key_gives_value(orc):
    """One visible key: its weight is exactly 1, so the output is that value row."""
    r = _rng(4)
    q, k, v = r.standard_normal((1, 16)), r.standard_normal((1, 16)), r.standard_normal((1, 16))
    out = orc.attend_head(q, k, v, 0.25, True)
    assert np.array_equal(out, v)
    # the first query of any causal prefill sees only key 0
    T = 11
    q, k, v = r.standard_normal((T, 16)), r.standard_normal((T, 16)), r.standard_normal((T, 16))
    out = orc.attend_head(q, k, v, 0.25, True)
    assert np.array_equal(out[0], v[0])


def pin_zero_query_prefix_mean(orc):
    """Q = 0 makes every visible score equal, so the weights are uniform and the
    output is the causal prefix mean of V (cumulative sum / count); lse = log(t+1)."""
    r = _rng(5)
    T, D = 40, 12
    q = np.zeros((T, D))
    k, v = r.standard_normal((T, D)), r.standard_normal((T, D))
    out, lse = orc.attend_head(q, k, v, 0.3, True, want_lse=True)
    ref = np.cumsum(v, axis=0) / np.arange(1, T + 1)[:, None]
    assert np.max(np.abs(out - ref)) <= 1e-13
    assert np.max(np.abs(lse - np.log(np.arange(1, T + 1)))) <= 1e-13
    # non-causal: the mean of all rows
    out = orc.attend_head(q, k, v, 0.3, False)
    assert np.max(np.abs(out - v.mean(axis=0))) <= 1e-13


def pin_constant_values(orc):
    """V = c on every key gives O = c whatever the weights."""
    r = _rng(6)
    T, D = 23, 5
    q, k = r.standard_normal((T, D)), r.standard_normal((T, D))
    c = r.standard_normal(D)
    v = np.tile(c, (T, 1))
    out = orc.attend_head(q, k, v, 0.7, True)
    assert np.max(np.abs(out - c)) <= 1e-14


def pin_hard_attention_limit(orc):
    """A key aligned with the query at a huge scale takes all the weight, so the
    output tends to that key's value row."""
    r = _rng(7)
    T, D = 9, 8
    q, k, v = r.standard_normal((T, D)), r.standard_normal((T, D)), r.standard_normal((T, D))
    t, j = 7, 3
    q[t] = np.zeros(D)
    q[t, 0] = 1.0
    k[:, 0] = 0.0
    k[j, 0] = 1.0  # score of (t, j) = scale, all other visible scores of row t = 0
    out = orc.attend_head(q, k, v, 200.0, True)
    assert np.max(np.abs(out[t] - v[j])) <= 1e-12
    # the same key beyond the query (j > t) is masked and takes no weight
    k[:, 0] = 0.0
    k[8, 0] = 1.0
    out = orc.attend_head(q, k, v, 200.0, True)
    ref = v[: t + 1].mean(axis=0)
    assert np.max(np.abs(out[t] - ref)) <= 1e-13


def pin_two_key_logistic(orc):
    """Two keys whose scaled scores are 0 and scale*a*b: the second weight is the
    logistic function of that score difference (softmax of two scores)."""
    D = 4
    for scale, a, b in ((0.125, 1.5, -2.0), (1 / np.sqrt(128), 3.0, 4.0), (0.5, -1.0, 0.25)):
        q = np.zeros((1, D))
        q[0, 1] = a
        k = np.zeros((2, D))
        k[1, 1] = b
        v = np.array([[0.0] * D, [1.0] * D])
        out, lse = orc.attend_head(q, k, v, scale, True, want_lse=True)
        ref = 1.0 / (1.0 + np.exp(-scale * a * b))
        assert abs(out[0, 0] - ref) <= 1e-15, (out[0, 0], ref)
        # log-sum-exp of the two scores 0 and scale*a*b
        assert abs(lse[0] - np.log1p(np.exp(scale * a * b))) <= 1e-14, lse


def pin_noncausal_permutation(orc):
    """Le Transformer et l'attention, 'L'encodage de position': without positions,
    attention is permutation-invariant -- jointly permuting the key/value rows leaves
    each non-causal output unchanged."""
    r = _rng(8)
    T, D = 17, 6
    q, k, v = r.standard_normal((T, D)), r.standard_normal((T, D)), r.standard_normal((T, D))
    p = r.permutation(T)
    a = orc.attend_head(q, k, v, 0.4, False)
    b = orc.attend_head(q, k[p], v[p], 0.4, False)
    assert np.max(np.abs(a - b)) <= 1e-13


def pin_causal_prefix_dependence(orc):
    """Row t depends only on keys/values 0..t: changing later rows leaves it
    bitwise unchanged."""
    r = _rng(9)
    T, D = 21, 7
    q, k, v = r.standard_normal((T, D)), r.standard_normal((T, D)), r.standard_normal((T, D))
    a = orc.attend_head(q, k, v, 0.4, True)
    t = 12
    k2, v2 = k.copy(), v.copy()
    k2[t + 1:] = 5.0 * r.standard_normal((T - t - 1, D))
    v2[t + 1:] = -3.0
    b = orc.attend_head(q, k2, v2, 0.4, True)
    assert np.array_equal(a[: t + 1], b[: t + 1])
    assert not np.array_equal(a[t + 1:], b[t + 1:])


def pin_decode_alignment(orc):
    """Kimi K3 - Softmax over keys at p = 1000: one query against 1001 keys sees all
    of them.  It equals the non-causal result and row 1000 of a causal prefill."""
    g = _golden("k3_shapes.json")
    N = g["decode_keys"]["value"]
    p = g["decode_position"]["value"]
    assert N == p + 1
    r = _rng(10)
    D = 16
    k, v = r.standard_normal((N, D)), r.standard_normal((N, D))
    qall = r.standard_normal((N, D))
    dec, A = orc.attend_head(qall[p:], k, v, 0.25, True, want_probs=True)
    assert np.all(A > 0.0), "decode query at the last position must see every key"
    full = orc.attend_head(qall[p:], k, v, 0.25, False)
    assert np.array_equal(dec, full)
    pre = orc.attend_head(qall, k, v, 0.25, True, rows=[p])
    assert np.max(np.abs(dec - pre)) <= 1e-14
    # a query two rows short of the end sits at position N - 2: the last key is masked
    _, A2 = orc.attend_head(qall[p - 1:], k, v, 0.25, True, want_probs=True)
    assert A2[0, -1] == 0.0 and np.all(A2[0, :-1] > 0) and np.all(A2[1] > 0)


def pin_chunk_alignment(orc):
    """Kimi K2 - Construct causal mask: positions continue from the cached length, so
    a chunk of Tq queries after Tk - Tq cached tokens puts query i at position
    i + Tk - Tq.  With Q = 0 the weights are uniform over the visible keys, so row i is
    the mean of V rows 0 .. i + Tk - Tq (a closed form that fixes the alignment); the
    chunk's rows are the last Tq rows of the square causal attention over all Tk
    tokens; without the mask every query sees all Tk keys."""
    r = _rng(12)
    Tk, Tq, D = 70, 23, 8
    off = Tk - Tq
    k, v = r.standard_normal((Tk, D)), r.standard_normal((Tk, D))
    out = orc.attend_head(np.zeros((Tq, D)), k, v, 0.5, True)
    counts = np.arange(off + 1, Tk + 1)
    ref = np.cumsum(v, axis=0)[off:] / counts[:, None]
    assert np.max(np.abs(out - ref)) <= 1e-13
    q_full = r.standard_normal((Tk, D))
    chunk = orc.attend_head(q_full[off:], k, v, 0.5, True)
    square = orc.attend_head(q_full, k, v, 0.5, True)
    assert np.max(np.abs(chunk - square[off:])) <= 1e-14
    _, A = orc.attend_head(q_full[off:], k, v, 0.5, False, want_probs=True)
    assert np.all(A > 0.0)
    _, A = orc.attend_head(q_full[off:], k, v, 0.5, True, want_probs=True)
    for i in range(Tq):
        assert np.all(A[i, : off + i + 1] > 0.0) and np.all(A[i, off + i + 1:] == 0.0)


def pin_scaled_score_variance(orc):
    """Le Transformer et l'attention, 'Vérification de compréhension': with unit
    variance q and k, q.k / sqrt(d_k) has variance 1.  The spread of the log-weights
    over keys of one query is the spread of its scores, so its average over many
    queries must be close to 1 at scale 1/sqrt(D)."""
    g = _golden("k3_shapes.json")
    D = g["head_dim"]["value"]
    r = _rng(11)
    nq, nk = 64, 800
    q, k, v = r.standard_normal((nq, D)), r.standard_normal((nk, D)), r.standard_normal((nk, D))
    _, A = orc.attend_head(q, k, v, 1.0 / np.sqrt(D), False, want_probs=True)
    var = np.log(A).var(axis=1).mean()
    assert abs(var - g["scaled_score_variance"]["value"]) < 0.08, var


# ---------------------------------------------------------------- gate


def pin_gate_example(orc):
    """Gated MLA, 'A small causal example': channel 1.6 with gate logit 0 becomes 0.8;
    a gate near one passes the channel, near zero suppresses it."""
    g = _golden("three_token_example.json")["gate_example"]
    out = orc.gate(np.array([g["gate_logit"]]), np.array([g["context_channel"]]))
    assert abs(out[0] - g["gated"]) <= 1e-15
    o = np.array([1.6, -2.0, 3.0])
    assert np.max(np.abs(orc.gate(np.full(3, 60.0), o) - o)) <= 1e-15
    assert np.max(np.abs(orc.gate(np.full(3, -60.0), o))) <= 1e-25
    x = np.linspace(-8, 8, 33)
    s = orc.sigmoid(x)
    assert np.max(np.abs(s + orc.sigmoid(-x) - 1.0)) <= 1e-15
    assert orc.sigmoid(np.array([0.0]))[0] == 0.5
    assert np.all(np.diff(s) > 0)


# ---------------------------------------------------------------- linear


def pin_linear_convention(orc):
    """Y = X W^T with W stored [out, in] (Gated MLA: C = X W_c^T): identity inputs
    expose the transpose, and a hand-computed product fixes the arithmetic."""
    r = _rng(12)
    W = r.standard_normal((5, 3))
    assert np.array_equal(orc.linear(np.eye(3), W), W.T)
    X = r.standard_normal((4, 3))
    assert np.array_equal(orc.linear(X, np.eye(3)), X)
    # [1 2] . rows (3 4), (5 6), (7 8) = 11, 17, 23
    Y = orc.linear(np.array([[1.0, 2.0]]), np.array([[3.0, 4.0], [5.0, 6.0], [7.0, 8.0]]))
    assert np.array_equal(Y, np.array([[11.0, 17.0, 23.0]]))
    # batch axes pass through
    Xb = r.standard_normal((2, 3, 3))
    assert np.array_equal(orc.linear(Xb, np.eye(3)), Xb)


# ---------------------------------------------------------------- layer


def _layer_weights(dm, dc, r):
    return dict(Wq=r.standard_normal((dm, dm)), Wc=r.standard_normal((dc, dm)),
                Wk=r.standard_normal((dm, dc)), Wv=r.standard_normal((dm, dc)),
                Wg=r.standard_normal((dm, dm)), Wo=r.standard_normal((dm, dm)))


def pin_layer_contract(orc):
    """Gated MLA, 'Requirements' and 'A small causal example': a dict of exactly
    output and latent_cache; output shaped like X; cache (batch, sequence, latent
    width) and identical in causal and non-causal mode; inputs not mutated."""
    r = _rng(13)
    B, T, dm, dc, H = 2, 5, 8, 3, 2
    X = r.standard_normal((B, T, dm))
    W = _layer_weights(dm, dc, r)
    saved = {n: a.copy() for n, a in W.items()}
    Xs = X.copy()
    a = orc.gated_mla_layer(X, W["Wq"], W["Wc"], W["Wk"], W["Wv"], W["Wg"], W["Wo"], H, True)
    b = orc.gated_mla_layer(X, W["Wq"], W["Wc"], W["Wk"], W["Wv"], W["Wg"], W["Wo"], H, False)
    assert set(a) == {"output", "latent_cache"}
    assert a["output"].shape == X.shape
    assert a["latent_cache"].shape == (B, T, dc)
    assert np.array_equal(a["latent_cache"], b["latent_cache"])
    # the cache is the latent itself, X W_c^T (identity-free check: row 0 by hand)
    assert np.max(np.abs(a["latent_cache"][0, 0] - W["Wc"] @ X[0, 0])) <= 1e-12
    assert not np.array_equal(a["output"], b["output"])
    assert np.array_equal(X, Xs) and all(np.array_equal(W[n], saved[n]) for n in W)


def pin_layer_zero_query_closed_form(orc):
    """W_q = 0 gives uniform causal weights, so the joined context is the prefix
    mean of V = X W_c^T W_v^T.  The gate sigmoid(X W_g^T) multiplies it channel by
    channel BEFORE the output projection (Gated MLA, 'The channel-wise output gate');
    with W_o a channel permutation, gating after the projection would differ."""
    r = _rng(14)
    B, T, dm, dc, H = 1, 6, 6, 4, 3
    X = r.standard_normal((B, T, dm))
    Wc, Wv, Wk = r.standard_normal((dc, dm)), r.standard_normal((dm, dc)), r.standard_normal((dm, dc))
    Wq = np.zeros((dm, dm))
    Wg = 3.0 * np.eye(dm)
    perm = np.array([2, 0, 1, 5, 3, 4])
    Wo = np.eye(dm)[perm]  # Y[:, c] = gated[:, perm[c]]
    res = orc.gated_mla_layer(X, Wq, Wc, Wk, Wv, Wg, Wo, H, True)
    V = X[0] @ Wc.T @ Wv.T
    ctx = np.cumsum(V, axis=0) / np.arange(1, T + 1)[:, None]
    gate = 1.0 / (1.0 + np.exp(-3.0 * X[0]))
    ref = (gate * ctx)[:, perm]
    assert np.max(np.abs(res["output"][0] - ref)) <= 1e-12


def pin_layer_head_split(orc):
    """Gated MLA, 'Split attention into heads': head h owns the contiguous channels
    h*D_h .. (h+1)*D_h - 1 of Q, K and V, and attends on its own.  With W_q a huge
    multiple of the identity and W_c = W_k = I, each head's query takes (in the
    limit) the value of the visible key with the largest dot product within that
    head's channels of X; the values are X with channels permuted (W_v), so keys and
    values must come from their own up-projections."""
    r = _rng(15)
    T, dm, H = 7, 6, 3
    Dh = dm // H
    X = r.standard_normal((1, T, dm))
    I = np.eye(dm)
    P = I[[3, 5, 0, 4, 1, 2]]  # V = X P^T: value channel c is X channel perm[c]
    lam = 4000.0
    res = orc.gated_mla_layer(X, lam * I, I, I, P, np.zeros((dm, dm)), I, H, True)
    V = X[0] @ P.T
    ref = np.empty((T, dm))
    for h in range(H):
        xs = X[0, :, h * Dh:(h + 1) * Dh]
        for t in range(T):
            dots = xs[: t + 1] @ xs[t]
            ref[t, h * Dh:(h + 1) * Dh] = V[int(np.argmax(dots)), h * Dh:(h + 1) * Dh]
    # gate logit 0 halves every channel
    assert np.max(np.abs(res["output"][0] - 0.5 * ref)) <= 1e-9


def pin_layer_rows_subset(orc):
    """Rows are independent: computing a subset of tokens gives the same rows."""
    r = _rng(16)
    B, T, dm, dc, H = 1, 9, 4, 2, 2
    X = r.standard_normal((B, T, dm))
    W = _layer_weights(dm, dc, r)
    full = orc.gated_mla_layer(X, W["Wq"], W["Wc"], W["Wk"], W["Wv"], W["Wg"], W["Wo"], H, True)
    rows = [0, 4, 8]
    part = orc.gated_mla_layer(X, W["Wq"], W["Wc"], W["Wk"], W["Wv"], W["Wg"], W["Wo"], H, True,
                               rows=rows)
    assert np.max(np.abs(part["output"][0] - full["output"][0, rows])) <= 1e-13


ALL_PINS = [v for n, v in sorted(globals().items()) if n.startswith("pin_")]
