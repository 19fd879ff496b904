"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test pins one part of the definition so that a plausible slip in the oracle (an
off-by-one window, a flipped bias sign, a swapped rotation pair, a wrong frequency, a
mis-indexed ring slot, a missing normaliser) fails at least one of them:

  selection      - band-mask counts 58 / 136 and reach 4, 7, 10, 13 (glossary example),
                   receptive field 255 / 1,525 (SWAT walkthrough), exact bit readout;
  weights        - softmax worked example and sigmoid values (SWAT page);
  bias           - closed form with q = 0, and the direction of the two head halves;
  rotation       - the d=2 closed form sin(m - n) per frequency, relative-position property;
  library cases  - torch's scaled_dot_product_attention with a float mask, causal attention
                   when the window covers the sequence, w = 1;
  cache          - ring slot closed form, append order, decode == prefill row by row;
  two oracles    - the C windowed loop equals the numpy dense masked computation.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import dense

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def readout_matrix(N, w, s, d=None):
    """Selection matrix of the C oracle: q = k = 0 makes every weight sigmoid(0) = 1/2, and
    one-hot values v_j = e_j put that weight in column j of row i."""
    d = d or N
    q = np.zeros((1, N, 1, d))
    k = np.zeros((1, N, 1, d))
    v = np.zeros((1, N, 1, d))
    for j in range(N):
        v[0, j, 0, j] = 1.0
    o = oracle.prefill(q, k, v, w=w, s=s, mode=oracle.SIGMOID)
    return o[0, :, 0, :N]


# ----------------------------------------------------------------------------- selection

def test_band_mask_counts_match_page():
    g = golden("band_mask_counts.json")
    N, w = g["seq_len"], g["window"]
    mask = dense.band_mask(N, w)
    pos = np.arange(N)
    causal = (pos[:, None] - pos[None, :]) >= 0
    assert int(mask.sum()) == g["window_scores"]
    assert int(causal.sum()) == g["causal_scores"]
    # the C loop's key sets: each selected key contributes exactly 1/2 under q = k = 0
    sel = readout_matrix(N, w, 0)
    assert set(np.unique(sel).tolist()) <= {0.0, 0.5}
    assert int((sel * 2).sum()) == g["window_scores"]
    assert np.array_equal(sel > 0, mask)


def test_reach_by_mask_composition_matches_page():
    g = golden("band_mask_counts.json")
    N, w = g["seq_len"], g["window"]
    mask = (readout_matrix(N, w, 0) > 0).astype(np.int64)
    reach = mask.copy()
    got = []
    for _ in range(4):
        got.append(int(reach[-1].sum()))
        reach = ((mask @ reach) > 0).astype(np.int64)
    assert got == g["last_token_reach_per_layer"]


def test_receptive_field_matches_walkthrough():
    g = golden("receptive_field.json")
    for case in g["cases"]:
        w, L = case["window"], case["layers"]
        N = case["reach"] + 64
        mask = dense.band_mask(N, w).astype(np.float32)
        # last row of mask^L, by left-multiplying a row vector L times (boolean semiring)
        r = mask[-1].copy()
        for _ in range(L - 1):
            r = ((r @ mask) > 0).astype(np.float32)
        assert int(r.sum()) == case["reach"]
        assert 1 + (w - 1) * L == case["reach"]
    for case in g["approximate"]:
        reach = 1 + (case["window"] - 1) * case["layers"]
        assert round(reach / 1000) == case["reach_thousands"]


@pytest.mark.parametrize("N,w,s", [(40, 5, 0), (40, 5, 3), (40, 1, 2), (30, 40, 0), (33, 7, 9)])
def test_selection_bit_readout(N, w, s):
    """q = k = 0 and v_j[c] = bit c of j: o_i[c] = 1/2 * #{j in K(i) with bit c set}. The
    key set is compared with the definition written as a brute-force predicate, and its
    size with the closed form min(i+1, w+s)."""
    bits = max(1, int(N - 1).bit_length())
    d = bits + (bits % 2)
    q = np.zeros((1, N, 1, d))
    k = np.zeros((1, N, 1, d))
    v = np.zeros((1, N, 1, d))
    for j in range(N):
        for c in range(bits):
            v[0, j, 0, c] = float((j >> c) & 1)
    o = oracle.prefill(q, k, v, w=w, s=s, mode=oracle.SIGMOID)[0, :, 0, :]
    ones = oracle.prefill(q, k, np.ones_like(v), w=w, s=s, mode=oracle.SIGMOID)[0, :, 0, 0]
    for i in range(N):
        keys = [j for j in range(N) if j <= i and (i - j < w or j < s)]
        assert len(keys) == min(i + 1, w + s)
        assert ones[i] == 0.5 * len(keys)
        for c in range(bits):
            assert o[i, c] == 0.5 * sum((j >> c) & 1 for j in keys)


# ----------------------------------------------------------------------------- weights

def test_softmax_worked_example():
    g = golden("softmax_example.json")
    x = g["scores"]
    n, d = len(x), 8
    q = np.zeros((1, n, 1, d))
    k = np.zeros((1, n, 1, d))
    v = np.zeros((1, n, 1, d))
    q[0, n - 1, 0, 0] = math.sqrt(d)          # scale 1/sqrt(d) cancels: score = x_j
    for j in range(n):
        k[0, j, 0, 0] = x[j]
        v[0, j, 0, j] = 1.0
    for impl in (oracle.prefill, dense.prefill_dense):
        o = impl(q, k, v, w=n, mode=oracle.SOFTMAX)
        row = o[0, n - 1, 0, :n]
        assert abs(row.sum() - 1.0) < 1e-12
        assert [round(float(t), g["decimals"]) for t in row] == g["weights"]


def test_sigmoid_values():
    g = golden("sigmoid_values.json")
    xs = [e["score"] for e in g["values"]]
    n, d = len(xs), 4
    q = np.zeros((1, n, 1, d))
    k = np.zeros((1, n, 1, d))
    v = np.zeros((1, n, 1, d))
    q[0, n - 1, 0, 0] = math.sqrt(d)
    for j in range(n):
        k[0, j, 0, 0] = xs[j]
        v[0, j, 0, j] = 1.0
    for impl in (oracle.prefill, dense.prefill_dense):
        row = impl(q, k, v, w=n, mode=oracle.SIGMOID)[0, n - 1, 0, :n]
        for j, e in enumerate(g["values"]):
            assert round(float(row[j]), e["decimals"]) == e["weight"]
        # unnormalised: the weights do not sum to one
        assert row.sum() > 2.0


def test_sigmoid_is_overflow_safe():
    """Scores far below zero give weight 0, far above give 1, never NaN."""
    N, d = 6, 6
    q = np.zeros((1, N, 1, d))
    k = np.zeros((1, N, 1, d))
    v = np.eye(N)[None, :, None, :]
    o = oracle.prefill(q, k, v, w=N, mode=oracle.SIGMOID, slopes=[-2000.0])
    assert np.all(np.isfinite(o))
    assert o[0, 5, 0, 5] == 0.5 and o[0, 5, 0, 0] == 0.0
    o = oracle.prefill(q, k, v, w=N, mode=oracle.SIGMOID, slopes=[2000.0])
    assert o[0, 5, 0, 0] == 1.0


# ----------------------------------------------------------------------------- bias

@pytest.mark.parametrize("mode", [oracle.SIGMOID, oracle.SOFTMAX])
def test_alibi_closed_form_and_direction(mode):
    """q = 0 leaves only the bias: x_ij = slope_h * (i - j). Heads with a negative slope
    weight recent keys more, positive slopes weight distant keys more (SWAT page,
    'Balanced ALiBi')."""
    N, w = 24, 9
    slopes = [-0.5, -0.125, 0.25, 0.0625]
    rng = np.random.default_rng(0)
    q = np.zeros((1, N, 4, N))
    k = rng.standard_normal((1, N, 4, N))
    v = np.tile(np.eye(N)[None, :, None, :], (1, 1, 4, 1))
    o = oracle.prefill(q, k, v, w=w, mode=mode, slopes=slopes)
    for h, m in enumerate(slopes):
        for i in range(N):
            keys = list(range(max(0, i - w + 1), i + 1))
            x = np.array([m * (i - j) for j in keys])
            if mode == oracle.SIGMOID:
                want = np.array([1.0 / (1.0 + math.exp(-t)) for t in x])
            else:
                e = np.exp(x - x.max())
                want = e / e.sum()
            np.testing.assert_allclose(o[0, i, h, keys], want, rtol=1e-13, atol=1e-15)
        row = o[0, N - 1, h, N - w:N]          # keys from oldest to newest
        if m < 0:
            assert np.all(np.diff(row) > 0)     # newer keys weigh more
        else:
            assert np.all(np.diff(row) < 0)     # older keys weigh more


# ----------------------------------------------------------------------------- rotation

@pytest.mark.parametrize("pair,theta", [(0, 1e4), (3, 1e4), (5, 1e6)])
def test_rope_closed_form(pair, theta):
    """With q = e_{2t} and k = e_{2t+1}, (R(m) q) . (R(n) k) = sin((m - n) * theta^(-2t/d))
    (RoFormer rotation, interleaved pairs). Read back through the sigmoid with scale 1."""
    N = d = 16
    q = np.zeros((1, N, 1, d))
    k = np.zeros((1, N, 1, d))
    q[0, :, 0, 2 * pair] = 1.0
    k[0, :, 0, 2 * pair + 1] = 1.0
    v = np.eye(N)[None, :, None, :]
    o = oracle.prefill(q, k, v, w=N, mode=oracle.SIGMOID, scale=1.0, rope_theta=theta)
    freq = theta ** (-2.0 * pair / d)
    for m in range(N):
        for n in range(m + 1):
            p = o[0, m, 0, n]
            x = math.log(p / (1.0 - p))
            assert abs(x - math.sin((m - n) * freq)) < 1e-12


def test_rope_relative_position_property():
    """Scores depend on positions only through m - n: copies of the same q, k pair shifted
    by D positions give the same score (SWAT page, 'RoPE')."""
    rng = np.random.default_rng(1)
    N, d, D = 40, 64, 17
    q = rng.standard_normal((1, N, 1, d))
    k = rng.standard_normal((1, N, 1, d))
    for (m, n) in [(5, 2), (9, 9), (12, 0)]:
        q[0, m + D] = q[0, m]
        k[0, n + D] = k[0, n]
    v = np.zeros((1, N, 1, d))
    v[0, :, 0, :N] = np.eye(N)
    o = oracle.prefill(q, k, v, w=N, mode=oracle.SIGMOID, scale=1.0, rope_theta=1e4)
    logit = lambda p: math.log(p / (1.0 - p))
    for (m, n) in [(5, 2), (9, 9), (12, 0)]:
        a, b = logit(o[0, m, 0, n]), logit(o[0, m + D, 0, n + D])
        assert abs(a - b) < 1e-9 * max(1.0, abs(a))
    # and the rotation is not the identity
    o0 = oracle.prefill(q, k, v, w=N, mode=oracle.SIGMOID, scale=1.0)
    assert abs(logit(o0[0, 12, 0, 0]) - logit(o[0, 12, 0, 0])) > 1e-3


# ----------------------------------------------------------------------------- library cases

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("w,s,theta,alibi", [(5, 0, 0.0, False), (7, 3, 1e4, True),
                                             (64, 0, 1e6, True)])
def test_softmax_equals_torch_sdpa_with_float_mask(w, s, theta, alibi):
    """Softmax mode equals torch's scaled_dot_product_attention (CPU, float64) given the
    pre-rotated q, k and a float mask holding -inf outside the key set plus the bias
    (Sliding Window Attention glossary: the mask can be passed as attn_mask)."""
    B, N, Hq, Hkv, d = 2, 37, 4, 2, 16
    q, k, v = _rand((B, N, Hq, d), 1), _rand((B, N, Hkv, d), 2), _rand((B, N, Hkv, d), 3)
    slopes = [-0.5, -0.25, 0.5, 0.25] if alibi else None
    ref = oracle.prefill(q, k, v, w=w, s=s, mode=oracle.SOFTMAX, slopes=slopes, rope_theta=theta)
    qr = dense.rope_dense(q, theta) if theta > 0 else q
    kr = dense.rope_dense(k, theta) if theta > 0 else k
    g = Hq // Hkv
    tq = torch.from_numpy(qr).permute(0, 2, 1, 3)
    tk = torch.from_numpy(np.repeat(kr, g, axis=2)).permute(0, 2, 1, 3).contiguous()
    tv = torch.from_numpy(np.repeat(v, g, axis=2)).permute(0, 2, 1, 3).contiguous()
    mask = torch.from_numpy(dense.band_mask(N, w, s))
    pos = torch.arange(N, dtype=torch.float64)
    dist = pos[:, None] - pos[None, :]
    bias = torch.zeros(Hq, N, N, dtype=torch.float64)
    if slopes is not None:
        bias = torch.tensor(slopes, dtype=torch.float64)[:, None, None] * dist[None]
    fm = torch.where(mask[None], bias, torch.tensor(-math.inf, dtype=torch.float64))
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=fm[None])
    out = out.permute(0, 2, 1, 3).numpy()
    np.testing.assert_allclose(ref, out, rtol=1e-10, atol=1e-12)


def test_window_covering_sequence_is_causal_attention():
    """w >= N, no sinks, softmax, no bias: standard causal attention (SWAT page: window
    longer than the sequence is global attention)."""
    B, N, H, d = 1, 29, 3, 8
    q, k, v = _rand((B, N, H, d), 4), _rand((B, N, H, d), 5), _rand((B, N, H, d), 6)
    ref = oracle.prefill(q, k, v, w=N + 5, mode=oracle.SOFTMAX)
    t = lambda a: torch.from_numpy(a).permute(0, 2, 1, 3).contiguous()
    out = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True)
    np.testing.assert_allclose(ref, out.permute(0, 2, 1, 3).numpy(), rtol=1e-10, atol=1e-12)


def test_window_of_one():
    B, N, H, d = 1, 11, 2, 6
    q, k, v = _rand((B, N, H, d), 7), _rand((B, N, H, d), 8), _rand((B, N, H, d), 9)
    o = oracle.prefill(q, k, v, w=1, mode=oracle.SOFTMAX)
    np.testing.assert_array_equal(o, v)
    o = oracle.prefill(q, k, v, w=1, mode=oracle.SIGMOID)
    x = (q * k).sum(-1, keepdims=True) / math.sqrt(d)
    np.testing.assert_allclose(o, v / (1.0 + np.exp(-x)), rtol=1e-13)


# ----------------------------------------------------------------------------- two oracles

@pytest.mark.parametrize("mode", [oracle.SIGMOID, oracle.SOFTMAX])
@pytest.mark.parametrize("w,s,Hq,Hkv,theta,alibi", [
    (4, 0, 2, 2, 0.0, False), (6, 2, 4, 2, 1e4, True), (13, 5, 4, 1, 1e6, True),
    (50, 0, 2, 1, 1e4, False), (1, 3, 2, 2, 1e4, True)])
def test_windowed_loop_equals_dense_masked(mode, w, s, Hq, Hkv, theta, alibi):
    B, N, d = 2, 31, 8
    q, k, v = _rand((B, N, Hq, d), 10), _rand((B, N, Hkv, d), 11), _rand((B, N, Hkv, d), 12)
    slopes = list(np.linspace(-0.7, 0.7, Hq)) if alibi else None
    a = oracle.prefill(q, k, v, w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta)
    b = dense.prefill_dense(q, k, v, w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta)
    np.testing.assert_allclose(a, b, rtol=1e-11, atol=1e-12)
    rows = [0, 3, N - 1, 17]
    c = oracle.prefill(q, k, v, w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta, rows=rows)
    np.testing.assert_array_equal(c, a[:, rows])


# ----------------------------------------------------------------------------- cache

@pytest.mark.parametrize("w", [1, 4, 7, 64])
def test_ring_slot_closed_form(w):
    """After appending positions 0..p in order, slot t holds p - ((p - t) mod w) when that is
    non-negative (ring of w slots, position i in slot i mod w, oldest overwritten)."""
    for p in range(0, 3 * w + 5):
        got = oracle.ring_fill_positions(p, w)
        for t in range(w):
            held = p - ((p - t) % w)
            assert got[t] == (held if held >= 0 else -1)


def test_cache_ratio_closed_form():
    g = golden("cache_ratio.json")
    assert g["seq_len"] // g["window"] == g["ratio"]


def test_append_of_many_tokens_keeps_last_writer():
    rng = np.random.default_rng(3)
    S, Hkv, w, s, d, n_new = 2, 2, 5, 2, 4, 13
    kn, vn = rng.standard_normal((S, n_new, Hkv, d)), rng.standard_normal((S, n_new, Hkv, d))
    pos0 = np.array([0, 7])
    a = oracle.Ring(S, Hkv, w, s, d)
    a.append(kn, vn, pos0, rope_theta=1e4)
    b = oracle.Ring(S, Hkv, w, s, d)
    for n in range(n_new):
        b.append(kn[:, n:n + 1], vn[:, n:n + 1], pos0 + n, rope_theta=1e4)
    for x, y in [(a.k, b.k), (a.v, b.v), (a.pos, b.pos), (a.k_sink, b.k_sink)]:
        np.testing.assert_array_equal(x, y)
    # sequence 0 started at position 0: positions 0, 1 are in the sink store
    np.testing.assert_array_equal(a.v_sink[0, :, :2], np.transpose(vn[0, :2], (1, 0, 2)))
    # sequence 1 started at 7 > s: its sink store was never written
    assert np.all(a.v_sink[1] == 0)


@pytest.mark.parametrize("mode", [oracle.SIGMOID, oracle.SOFTMAX])
@pytest.mark.parametrize("w,s", [(5, 0), (5, 2), (8, 3), (30, 1)])
def test_decode_equals_prefill_row_by_row(mode, w, s):
    """Appending tokens 0..N-1 one at a time and decoding each reproduces every prefill row."""
    S, N, Hq, Hkv, d, theta = 2, 24, 4, 2, 8, 1e4
    q, k, v = _rand((S, N, Hq, d), 20), _rand((S, N, Hkv, d), 21), _rand((S, N, Hkv, d), 22)
    slopes = [-0.3, -0.1, 0.3, 0.1]
    ref = oracle.prefill(q, k, v, w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta)
    ring = oracle.Ring(S, Hkv, w, s, d)
    for p in range(N):
        pos = np.full(S, p)
        ring.append(k[:, p:p + 1], v[:, p:p + 1], pos, rope_theta=theta)
        o = ring.decode(q[:, p], pos, H_q=Hq, mode=mode, slopes=slopes, rope_theta=theta)
        np.testing.assert_allclose(o, ref[:, p], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("w", [1, 3, 8])
def test_append_writes_position_mod_w(w):
    """Appending token p writes slot p mod w: after positions 0..p the recorded positions
    follow the closed form p - ((p - t) mod w), and slot t holds the value of that token."""
    S, Hkv, s, d = 1, 1, 0, 2
    ring = oracle.Ring(S, Hkv, w, s, d)
    for p in range(3 * w + 2):
        kv = np.full((S, 1, Hkv, d), float(p))
        ring.append(kv, kv, np.array([p]))
        for t in range(w):
            held = p - ((p - t) % w)
            assert ring.pos[0, t] == (held if held >= 0 else -1)
            if held >= 0:
                assert ring.v[0, 0, t, 0] == float(held)


# ----------------------------------------------------------------------------- chunked prefill

def _chunk_schedule(S, N, seed):
    """Ragged split points per sequence: round r hands sequence q the tokens
    [cuts[q][r], cuts[q][r+1]) (possibly none)."""
    rng = np.random.default_rng(seed)
    cuts = []
    for _ in range(S):
        inner = np.sort(rng.choice(np.arange(1, N), size=3, replace=False))
        cuts.append([0] + inner.tolist() + [N])
    return cuts


@pytest.mark.parametrize("mode", [oracle.SIGMOID, oracle.SOFTMAX])
@pytest.mark.parametrize("w,s", [(5, 0), (6, 2), (9, 4), (40, 1), (3, 7)])
def test_chunked_prefill_equals_whole_prefill(mode, w, s):
    """Feeding each sequence in ragged chunks (packed rows, different chunk lengths per
    sequence in one call, empty chunks included), each chunk reading its history from the
    ring and then appended, reproduces the whole-sequence prefill row for row: the ring keeps
    exactly the history a window needs (Sliding Window Attention glossary, ring buffer)."""
    S, N, Hq, Hkv, d, theta = 3, 26, 4, 2, 8, 1e4
    q, k, v = _rand((S, N, Hq, d), 30), _rand((S, N, Hkv, d), 31), _rand((S, N, Hkv, d), 32)
    slopes = [-0.3, -0.1, 0.3, 0.1]
    ref = oracle.prefill(q, k, v, w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta)
    cuts = _chunk_schedule(S, N, seed=w * 10 + s)
    ring = oracle.Ring(S, Hkv, w, s, d)
    got = np.full_like(ref, np.nan)
    for r in range(4):
        lens = [cuts[sq][r + 1] - cuts[sq][r] for sq in range(S)]
        cu = np.concatenate([[0], np.cumsum(lens)])
        pos0 = np.array([cuts[sq][r] for sq in range(S)])
        rows = lambda a: np.concatenate([a[sq, cuts[sq][r]:cuts[sq][r + 1]] for sq in range(S)])
        o = ring.chunk(rows(q), rows(k), rows(v), cu, pos0, H_q=Hq, mode=mode, slopes=slopes,
                       rope_theta=theta)
        for sq in range(S):
            got[sq, cuts[sq][r]:cuts[sq][r + 1]] = o[cu[sq]:cu[sq + 1]]
    np.testing.assert_allclose(got, ref, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("mode", [oracle.SIGMOID, oracle.SOFTMAX])
def test_chunk_of_one_token_equals_decode(mode):
    """A one-token chunk is a decode step: same output as appending it and calling decode."""
    S, Hq, Hkv, d, w, s, theta = 2, 4, 2, 8, 6, 2, 1e4
    hist = 11
    k, v = _rand((S, hist + 1, Hkv, d), 40), _rand((S, hist + 1, Hkv, d), 41)
    qn = _rand((S, Hq, d), 42)
    a, b = oracle.Ring(S, Hkv, w, s, d), oracle.Ring(S, Hkv, w, s, d)
    for ring in (a, b):
        ring.append(k[:, :hist], v[:, :hist], np.zeros(S, dtype=np.int64), rope_theta=theta)
    pos = np.full(S, hist)
    o_chunk = a.chunk(qn, k[:, hist], v[:, hist], np.arange(S + 1), pos, H_q=Hq, mode=mode,
                      rope_theta=theta)
    b.append(k[:, hist:], v[:, hist:], pos, rope_theta=theta)
    o_dec = b.decode(qn, pos, H_q=Hq, mode=mode, rope_theta=theta)
    np.testing.assert_allclose(o_chunk, o_dec, rtol=1e-12, atol=1e-13)
    for x, y in [(a.k, b.k), (a.v, b.v), (a.pos, b.pos), (a.k_sink, b.k_sink)]:
        np.testing.assert_array_equal(x, y)


def test_chunk_without_history_is_rejected():
    """A chunk that starts past position 0 needs its window's history in the ring."""
    ring = oracle.Ring(1, 1, 4, 0, 2)
    with pytest.raises(ValueError, match="does not hold"):
        ring.chunk(np.ones((2, 1, 2)), np.ones((2, 1, 2)), np.ones((2, 1, 2)), [0, 2], [5],
                   H_q=1, mode=oracle.SOFTMAX)


def test_chunk_rows_subset_equals_full():
    """Computing a subset of packed rows gives those rows of the full result."""
    S, Hq, Hkv, d, w, s, theta = 2, 2, 1, 8, 5, 1, 1e4
    T = 9
    q, k, v = _rand((T, Hq, d), 50), _rand((T, Hkv, d), 51), _rand((T, Hkv, d), 52)
    cu, pos0 = np.array([0, 4, 9]), np.array([0, 0])
    full = oracle.Ring(S, Hkv, w, s, d).chunk(q, k, v, cu, pos0, H_q=Hq, mode=oracle.SOFTMAX,
                                             rope_theta=theta)
    rows = [8, 0, 5, 3]
    part = oracle.Ring(S, Hkv, w, s, d).chunk(q, k, v, cu, pos0, H_q=Hq, mode=oracle.SOFTMAX,
                                             rope_theta=theta, rows=rows)
    np.testing.assert_array_equal(part, full[rows])


# ----------------------------------------------------------------------------- backward

@pytest.mark.parametrize("mode", [oracle.SIGMOID, oracle.SOFTMAX])
@pytest.mark.parametrize("w,s,theta,alibi", [(3, 0, 0.0, False), (4, 2, 1e4, True),
                                             (20, 0, 1e4, True), (1, 1, 1e2, False)])
def test_backward_matches_finite_differences(mode, w, s, theta, alibi):
    """The gradients of L = sum(dout * o) equal central differences of the (pinned) forward
    oracle, element by element, for q, k and v, with grouped heads, sinks, bias and rotation."""
    B, N, Hq, Hkv, d = 1, 9, 2, 1, 4
    q, k, v = _rand((B, N, Hq, d), 60), _rand((B, N, Hkv, d), 61), _rand((B, N, Hkv, d), 62)
    g = _rand((B, N, Hq, d), 63)
    slopes = [-0.4, 0.3] if alibi else None
    kw = dict(w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta)
    dq, dk, dv = oracle.backward(q, k, v, g, **kw)
    loss = lambda q_, k_, v_: float(np.sum(g * oracle.prefill(q_, k_, v_, **kw)))
    eps = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if n == name else y for n, y in (("q", q), ("k", k), ("v", v))]
            args_m = [xm if n == name else y for n, y in (("q", q), ("k", k), ("v", v))]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("mode", [oracle.SIGMOID, oracle.SOFTMAX])
def test_backward_equals_torch_autograd(mode):
    """Library case: torch autograd (float64, CPU) through a dense masked form of the layer
    (rotation, scaled scores plus bias, -inf outside the key set, sigmoid or softmax) gives
    the same gradients."""
    B, N, Hq, Hkv, d, w, s, theta = 2, 33, 4, 2, 8, 7, 2, 1e4
    q, k, v = _rand((B, N, Hq, d), 70), _rand((B, N, Hkv, d), 71), _rand((B, N, Hkv, d), 72)
    g = _rand((B, N, Hq, d), 73)
    slopes = [-0.5, -0.25, 0.5, 0.25]
    dq, dk, dv = oracle.backward(q, k, v, g, w=w, s=s, mode=mode, slopes=slopes,
                                 rope_theta=theta)
    tq, tk, tv = (torch.tensor(a, requires_grad=True) for a in (q, k, v))
    pos = torch.arange(N, dtype=torch.float64)
    freq = theta ** (-2.0 * torch.arange(d // 2, dtype=torch.float64) / d)
    ang = pos[:, None] * freq[None, :]
    c, sn = torch.cos(ang)[None, :, None, :], torch.sin(ang)[None, :, None, :]

    def rot(x):
        a, b = x[..., 0::2], x[..., 1::2]
        return torch.stack((a * c - b * sn, a * sn + b * c), dim=-1).flatten(-2)
    qr, kr = rot(tq), rot(tk)
    kr = kr.repeat_interleave(Hq // Hkv, dim=2)
    vr = tv.repeat_interleave(Hq // Hkv, dim=2)
    x = torch.einsum("bihd,bjhd->bhij", qr, kr) / np.sqrt(d)
    i, j = torch.arange(N)[:, None], torch.arange(N)[None, :]
    x = x + torch.tensor(slopes, dtype=torch.float64)[None, :, None, None] * (i - j)
    keep = (j <= i) & ((i - j < w) | (j < s))
    if mode == oracle.SOFTMAX:
        p = torch.softmax(x.masked_fill(~keep, float("-inf")), dim=-1)
    else:
        p = torch.sigmoid(x) * keep
    o = torch.einsum("bhij,bjhd->bihd", p, vr)
    (o * torch.tensor(g)).sum().backward()
    for got, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        np.testing.assert_allclose(got, ref.numpy(), rtol=1e-10, atol=1e-12)


def test_backward_window_of_one_closed_form():
    """w = 1, sigmoid, no rotation or bias: o_i = sigmoid(scale q_i.k_i) v_i, so
    dv_i = sigmoid(scale q_i.k_i) dout_i and dq_i = scale sigma(1 - sigma) (dout_i.v_i) k_i."""
    B, N, H, d = 1, 6, 1, 4
    q, k, v, g = (_rand((B, N, H, d), 80 + t) for t in range(4))
    dq, dk, dv = oracle.backward(q, k, v, g, w=1, mode=oracle.SIGMOID)
    sc = 1 / np.sqrt(d)
    sig = 1 / (1 + np.exp(-sc * np.sum(q * k, axis=-1, keepdims=True)))
    np.testing.assert_allclose(dv, sig * g, rtol=1e-12)
    dp = np.sum(g * v, axis=-1, keepdims=True)
    np.testing.assert_allclose(dq, sc * sig * (1 - sig) * dp * k, rtol=1e-12)
    np.testing.assert_allclose(dk, sc * sig * (1 - sig) * dp * q, rtol=1e-12)


# ----------------------------------------------------------------------------- dilated windows

@pytest.mark.parametrize("N,w,s,r", [(40, 5, 0, 2), (41, 4, 3, 3), (33, 7, 9, 4), (20, 1, 2, 2),
                                     (30, 40, 0, 2)])
def test_dilated_selection_readout(N, w, s, r):
    """q = k = 0 and one-hot values: row i of the output selects, with weight 1/2 each, exactly
    the keys of the dilated definition written as a brute-force predicate: w keys i, i - r,
    ..., i - r (w - 1) that exist, plus every sink j < s at or before i."""
    q = np.zeros((1, N, 1, N))
    k = np.zeros((1, N, 1, N))
    v = np.zeros((1, N, 1, N))
    for j in range(N):
        v[0, j, 0, j] = 1.0
    sel = oracle.prefill(q, k, v, w=w, s=s, mode=oracle.SIGMOID, dilation=r)[0, :, 0, :]
    for i in range(N):
        keys = {i - r * m for m in range(w) if i - r * m >= 0} | {j for j in range(min(s, i + 1))}
        want = np.zeros(N)
        want[sorted(keys)] = 0.5
        assert np.array_equal(sel[i], want), i


@pytest.mark.parametrize("mode", [oracle.SIGMOID, oracle.SOFTMAX])
@pytest.mark.parametrize("r", [2, 3])
def test_dilated_is_plain_window_per_residue_class(mode, r):
    """Without sinks, a dilated window is the plain window over each residue class of
    positions: class c (positions c, c + r, ...) as its own sequence, with q and k rotated at
    their true positions beforehand and the slopes scaled by r (the true distance is r times
    the distance inside the class), gives the same rows."""
    B, N, Hq, Hkv, d, w, theta = 1, 29, 2, 1, 8, 4, 1e4
    q, k, v = _rand((B, N, Hq, d), 90), _rand((B, N, Hkv, d), 91), _rand((B, N, Hkv, d), 92)
    slopes = [-0.3, 0.2]
    full = oracle.prefill(q, k, v, w=w, mode=mode, slopes=slopes, rope_theta=theta, dilation=r)
    qr, kr = dense.rope_dense(q, theta), dense.rope_dense(k, theta)
    for c in range(r):
        sub = oracle.prefill(qr[:, c::r], kr[:, c::r], v[:, c::r], w=w, mode=mode,
                             slopes=[x * r for x in slopes])
        np.testing.assert_allclose(full[:, c::r], sub, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("mode", [oracle.SIGMOID, oracle.SOFTMAX])
@pytest.mark.parametrize("w,s,r,theta,alibi", [(3, 0, 2, 1e4, True), (2, 2, 3, 0.0, False),
                                               (4, 1, 2, 1e2, True)])
def test_dilated_backward_matches_finite_differences(mode, w, s, r, theta, alibi):
    """The dilated backward's gradients of L = sum(dout * o) equal central differences of the
    (pinned) dilated forward oracle, element by element."""
    B, N, Hq, Hkv, d = 1, 11, 2, 1, 4
    q, k, v = _rand((B, N, Hq, d), 64), _rand((B, N, Hkv, d), 65), _rand((B, N, Hkv, d), 66)
    g = _rand((B, N, Hq, d), 67)
    slopes = [0.35, -0.2] if alibi else None
    kw = dict(w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta, dilation=r)
    dq, dk, dv = oracle.backward(q, k, v, g, **kw)
    loss = lambda q_, k_, v_: float(np.sum(g * oracle.prefill(q_, k_, v_, **kw)))
    eps = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = [xp if n == name else y for n, y in (("q", q), ("k", k), ("v", v))]
            args_m = [xm if n == name else y for n, y in (("q", q), ("k", k), ("v", v))]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        np.testing.assert_allclose(grad, num, rtol=1e-6, atol=1e-8, err_msg=name)


@pytest.mark.parametrize("mode", [oracle.SIGMOID, oracle.SOFTMAX])
def test_dilated_backward_is_plain_backward_per_residue_class(mode):
    """Without sinks or rotation the residue classes of a dilated window are independent plain
    windows (slopes scaled by r): their gradients are the plain backward's, class by class."""
    B, N, Hq, Hkv, d, w, r = 1, 26, 2, 1, 6, 4, 3
    q, k, v = _rand((B, N, Hq, d), 96), _rand((B, N, Hkv, d), 97), _rand((B, N, Hkv, d), 98)
    g = _rand((B, N, Hq, d), 99)
    slopes = [-0.3, 0.2]
    full = oracle.backward(q, k, v, g, w=w, mode=mode, slopes=slopes, dilation=r)
    for c in range(r):
        sub = oracle.backward(q[:, c::r], k[:, c::r], v[:, c::r], g[:, c::r], w=w, mode=mode,
                              slopes=[x * r for x in slopes])
        for a, b in zip(full, sub):
            np.testing.assert_allclose(a[:, c::r], b, rtol=1e-12, atol=1e-13)


def test_dilation_one_is_the_plain_window():
    B, N, Hq, Hkv, d = 1, 25, 2, 2, 8
    q, k, v = _rand((B, N, Hq, d), 93), _rand((B, N, Hkv, d), 94), _rand((B, N, Hkv, d), 95)
    a = oracle.prefill(q, k, v, w=6, s=2, mode=oracle.SOFTMAX, rope_theta=1e4)
    lib = oracle._load()
    out = np.zeros_like(a)
    qq, kk, vv = (np.ascontiguousarray(x) for x in (q, k, v))
    rc = lib.swa_oracle_prefill_dilated(B, Hq, Hkv, N, d, 6, 2, 1, oracle.SOFTMAX, 0.0, None, 1e4,
                                        oracle._ptr(qq), oracle._ptr(kk), oracle._ptr(vv), None, 0,
                                        oracle._ptr(out))
    assert rc == 0
    np.testing.assert_array_equal(out, a)
