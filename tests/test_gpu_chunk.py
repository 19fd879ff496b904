"""GPU parity of chunked prefill over the ring cache (swa_prefill_chunk) with the oracle.

Each case builds the same history in the library's cache (swa_kv_append) and in the
oracle's ring, then feeds every sequence a ragged chunk in one packed call: sequences
without history, with a history shorter than the window and with one that has wrapped the
ring, chunks of one row, of a few rows and of several tiles, and an empty chunk. Outputs are
compared element by element with the oracle; a second round checks that the first call
appended its chunk correctly, and the cache it leaves is compared bit for bit with the cache
swa_kv_append builds from the same tokens.
"""
import numpy as np
import pytest
import torch

import oracle
import sliding_window_attention_prefill_amd as swa
import swa_workloads as wl
from tests.helpers import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _randn(g, *shape):
    return torch.randn(shape, generator=g).to(torch.bfloat16)


def fill_history(caches, ring, hist, g, table, theta, tail_only=False):
    """Append positions 0..hist[q]-1 of every sequence q (random keys and values) to each
    library cache and to the oracle ring. tail_only appends just the sinks and the last w
    positions, which leaves the same ring and sink contents."""
    S, Hkv, d, w, s = ring.S, ring.H_kv, ring.d, ring.w, ring.s
    segs = []
    for q_ in range(S):
        n0 = int(hist[q_])
        start = max(0, n0 - w) if tail_only else 0
        if tail_only and start > 0 and s > 0:
            segs.append((q_, 0, min(s, start)))
        if n0 > start:
            segs.append((q_, start, n0))
    for q_, a, b in segs:
        n = b - a
        kh, vh = _randn(g, S, n, Hkv, d), _randn(g, S, n, Hkv, d)
        pos = torch.full((S,), -1, dtype=torch.int32)
        pos[q_] = a
        for c in caches:
            swa.swa_kv_append(c, kh.to(DEV), vh.to(DEV), pos.to(DEV), rope_table=table)
        ring.append(kh, vh, pos, rope_theta=theta)


def packed_chunk(g, lens, Hq, Hkv, d):
    T = int(sum(lens))
    cu = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32)
    return _randn(g, T, Hq, d), _randn(g, T, Hkv, d), _randn(g, T, Hkv, d), cu


def append_packed(cache, k, v, cu, pos0, table):
    """The same tokens through swa_kv_append, one sequence at a time."""
    S = cache.S
    for q_ in range(S):
        a, b = int(cu[q_]), int(cu[q_ + 1])
        if b == a or int(pos0[q_]) < 0:
            continue
        kp = torch.zeros((S, b - a, cache.H_kv, cache.d), dtype=k.dtype)
        vp = torch.zeros_like(kp)
        kp[q_], vp[q_] = k[a:b], v[a:b]
        pos = torch.full((S,), -1, dtype=torch.int32)
        pos[q_] = int(pos0[q_])
        swa.swa_kv_append(cache, kp.to(DEV), vp.to(DEV), pos.to(DEV), rope_table=table)


def assert_caches_equal(a, b):
    assert torch.equal(a.k_ring, b.k_ring) and torch.equal(a.v_ring, b.v_ring)
    if a.s > 0:
        assert torch.equal(a.k_sink, b.k_sink) and torch.equal(a.v_sink, b.v_sink)


CASES = [  # d, G, H_kv, mode, alibi, w, s, theta
    (64, 1, 2, wl.SIGMOID, True, 50, 0, 1e4),
    (64, 4, 2, wl.SOFTMAX, True, 200, 4, 1e4),
    (128, 4, 2, wl.SOFTMAX, False, 100, 3, 1e6),
    (128, 2, 1, wl.SIGMOID, True, 64, 2, 0.0),
    (64, 8, 1, wl.SOFTMAX, True, 1, 1, 1e4),
    (128, 1, 2, wl.SIGMOID, False, 700, 70, 1e4),
    (64, 3, 2, wl.SOFTMAX, True, 130, 65, 1e4),
    (128, 8, 1, wl.SIGMOID, True, 97, 0, 1e4),
]


def _random_cases(n, seed):
    """Seeded draws: 1-5 sequences with histories from empty to several times the window
    (wrapped rings), two rounds of ragged chunks (empty, one row, tile edges, several tiles),
    both head sizes and modes, 1-8 query heads per kv head, sinks, ALiBi, RoPE."""
    rs = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        d = int(rs.choice([64, 128]))
        G = int(rs.choice([1, 2, 3, 4, 8]))
        Hkv = int(rs.choice([1, 2]))
        mode = wl.SIGMOID if rs.rand() < 0.5 else wl.SOFTMAX
        alibi = bool(rs.rand() < 0.5)
        w = int(rs.choice([1, int(rs.randint(2, 100)), int(rs.randint(2, 100)),
                           int(rs.randint(100, 500)), int(rs.randint(100, 500))]))
        s = int(rs.choice([0, 0, 1, int(rs.randint(1, 70))]))
        theta = float(rs.choice([0.0, 1e4, 1e6]))
        S = int(rs.randint(1, 6))
        hist = [int(rs.choice([0, int(rs.randint(1, w + 2)), int(rs.randint(w, 4 * w + 10))]))
                for _ in range(S)]
        rounds = [[int(rs.choice([0, 1, 63, 64, 65, int(rs.randint(1, 260))])) for _ in range(S)]
                  for _ in range(2)]
        cases.append((d, G, Hkv, mode, alibi, w, s, theta, tuple(hist),
                      tuple(tuple(r) for r in rounds)))
    return cases


@pytest.mark.parametrize("case", CASES + _random_cases(12, 20261206),
                         ids=lambda c: "d%d_G%d_Hkv%d_m%d_a%d_w%d_s%d" % c[:7])
def test_chunk_matches_oracle(case):
    d, G, Hkv, mode, alibi, w, s, theta = case[:8]
    Hq = G * Hkv
    if len(case) > 8:
        hist, rounds = list(case[8]), [list(r) for r in case[9]]
    else:
        hist = [0, w // 2 + 5, 3 * w + 17, 2 * w + 1]
        rounds = [[70, 1, 130, 0], [0, 64, 33, 200]]
    S = len(hist)
    g = torch.Generator().manual_seed(w * 31 + d + G + (0 if len(case) == 8 else 1000 + 7 * S))
    for r in rounds:
        if max(r) == 0:
            r[0] = 1   # at least one row per call
    max_pos = max(hist) + sum(max(r) for r in rounds) + 1
    table = swa.swa_rope_table(max_pos, d, theta) if theta > 0 else None
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    twin = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)   # built by swa_kv_append
    ring = oracle.Ring(S, Hkv, w, s, d)
    fill_history([cache, twin], ring, hist, g, table, theta)
    assert_caches_equal(cache, twin)
    slopes = tuple(np.linspace(-0.5, 0.5, Hq).tolist()) if alibi else None
    sl = torch.tensor(slopes, dtype=torch.float32, device=DEV) if alibi else None
    pos0 = torch.tensor(hist, dtype=torch.int32)
    for r, lens in enumerate(rounds):
        q, k, v, cu = packed_chunk(g, lens, Hq, Hkv, d)
        out = swa.swa_prefill_chunk(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), pos0.to(DEV),
                                    cache, max_seqlen=max(lens), mode=mode, alibi_slopes=sl,
                                    rope_table=table, out_dtype=torch.float32)
        ref = ring.chunk(q, k, v, cu, pos0, H_q=Hq, mode=mode, slopes=slopes, rope_theta=theta)
        append_packed(twin, k, v, cu, pos0, table)
        torch.cuda.synchronize()
        assert_parity(out, ref, "bf16", "round %d" % r)
        assert_caches_equal(cache, twin)
        pos0 = pos0 + torch.tensor(lens, dtype=torch.int32)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", [wl.SIGMOID, wl.SOFTMAX])
def test_chunk_from_empty_cache_equals_prefill(d, mode):
    """Whole sequences as one chunk each over an empty cache: the same tiles in the same
    order as swa_prefill, so the outputs agree bit for bit, and the cache afterwards is the
    one swa_kv_append builds."""
    B, N, Hq, Hkv, w, s, theta = 2, 300, 8, 2, 120, 5, 1e4
    cfg = wl.PrefillConfig("chunk_vs_prefill", "bf16", B, Hq, Hkv, N, d, w, s, mode, theta,
                           tuple(np.linspace(-0.4, 0.4, Hq).tolist()), seed=77 + d + mode)
    q, k, v = wl.prefill_inputs(cfg, device=DEV)
    sl = wl.slopes_tensor(cfg.slopes, device=DEV)
    table = swa.swa_rope_table(N, d, theta)
    ref = swa.swa_prefill(q, k, v, w=w, s=s, mode=mode, alibi_slopes=sl, rope_table=table,
                          out_dtype=torch.float32)
    cache = swa.SwaCache.empty(B, Hkv, w, s, d, torch.bfloat16)
    cu = torch.tensor([0, N, 2 * N], dtype=torch.int32, device=DEV)
    pos0 = torch.zeros(B, dtype=torch.int32, device=DEV)
    out = swa.swa_prefill_chunk(q.reshape(B * N, Hq, d), k.reshape(B * N, Hkv, d),
                                v.reshape(B * N, Hkv, d), cu, pos0, cache, max_seqlen=N,
                                mode=mode, alibi_slopes=sl, rope_table=table,
                                out_dtype=torch.float32)
    twin = swa.SwaCache.empty(B, Hkv, w, s, d, torch.bfloat16)
    swa.swa_kv_append(twin, k, v, pos0, rope_table=table)
    torch.cuda.synchronize()
    assert torch.equal(out.reshape(B, N, Hq, d), ref)
    assert_caches_equal(cache, twin)


def test_chunk_bf16_output():
    d, Hq, Hkv, w, s, theta = 128, 8, 2, 90, 2, 1e4
    S = 2
    g = torch.Generator().manual_seed(5)
    table = swa.swa_rope_table(600, d, theta)
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
    hist = [150, 31]
    fill_history([cache], ring, hist, g, table, theta)
    lens = [77, 140]
    q, k, v, cu = packed_chunk(g, lens, Hq, Hkv, d)
    pos0 = torch.tensor(hist, dtype=torch.int32)
    out = swa.swa_prefill_chunk(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), pos0.to(DEV), cache,
                                max_seqlen=140, mode=wl.SOFTMAX, rope_table=table,
                                out_dtype=torch.bfloat16)
    ref = ring.chunk(q, k, v, cu, pos0, H_q=Hq, mode=wl.SOFTMAX, rope_theta=theta)
    ref_r = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    torch.cuda.synchronize()
    assert out.dtype == torch.bfloat16
    assert_parity(out, ref_r, "bf16", "bf16 out")


def test_chunk_invalid_sequences_get_nan_and_keep_their_cache():
    """A negative start, a chunk longer than max_seqlen and positions past the rotation table
    give NaN rows and leave that sequence's cache as it was; the valid sequences of the same
    call are answered and appended."""
    d, Hq, Hkv, w, s, theta = 64, 4, 2, 40, 2, 1e4
    S = 4
    g = torch.Generator().manual_seed(9)
    table = swa.swa_rope_table(200, d, theta)
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
    hist = [60, 10, 60, 190]
    fill_history([cache], ring, hist, g, table, theta)
    before = [t.clone() for t in (cache.k_ring, cache.v_ring, cache.k_sink, cache.v_sink)]
    lens = [20, 9, 30, 20]          # sequence 2 exceeds max_seqlen = 25; 3 runs past row 200
    q, k, v, cu = packed_chunk(g, lens, Hq, Hkv, d)
    pos0 = torch.tensor([hist[0], -1, hist[2], hist[3]], dtype=torch.int32)
    out = swa.swa_prefill_chunk(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), pos0.to(DEV), cache,
                                max_seqlen=25, mode=wl.SOFTMAX, rope_table=table,
                                out_dtype=torch.float32)
    torch.cuda.synchronize()
    rows0 = slice(0, 20)
    ring0 = oracle.Ring(1, Hkv, w, s, d)
    ring0.k[0], ring0.v[0], ring0.pos[0] = ring.k[0], ring.v[0], ring.pos[0]
    ring0.k_sink[0], ring0.v_sink[0] = ring.k_sink[0], ring.v_sink[0]
    ref0 = ring0.chunk(q[rows0], k[rows0], v[rows0], [0, 20], [hist[0]], H_q=Hq,
                       mode=wl.SOFTMAX, rope_theta=theta)
    assert_parity(out[rows0], ref0, "bf16", "valid sequence")
    assert torch.isnan(out[20:]).all()
    after = (cache.k_ring, cache.v_ring, cache.k_sink, cache.v_sink)
    for x, y in zip(before, after):
        assert torch.equal(x[1:], y[1:])             # sequences 1..3 untouched
    assert not torch.equal(before[0][0], after[0][0])  # sequence 0 appended


def test_chunk_full_size_sampled_rows():
    """A serving step at full size: 4 sequences, H_q 32 / H_kv 8, d 128, a 4096-token
    window (histories 0 .. 20000 tokens, chunks of 777 .. 2048 rows), softmax, RoPE
    theta 1e6; sampled rows of every sequence against the oracle, and the cache the call
    leaves bit for bit against swa_kv_append of the same tokens (at H_kv 8, d 128 the append
    spreads each 64-row tile over all eight of its workgroups)."""
    d, Hq, Hkv, w, s, theta = 128, 32, 8, 4096, 0, 1e6
    S = 4
    g = torch.Generator().manual_seed(2024)
    hist = [0, 3000, 9000, 20000]
    lens = [2048, 1500, 2048, 777]
    table = swa.swa_rope_table(max(h + n for h, n in zip(hist, lens)), d, theta)
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
    fill_history([cache], ring, hist, g, table, theta, tail_only=True)
    twin = swa.SwaCache(cache.k_ring.clone(), cache.v_ring.clone())
    q, k, v, cu = packed_chunk(g, lens, Hq, Hkv, d)
    pos0 = torch.tensor(hist, dtype=torch.int32)
    out = swa.swa_prefill_chunk(q.to(DEV), k.to(DEV), v.to(DEV), cu.to(DEV), pos0.to(DEV), cache,
                                max_seqlen=max(lens), mode=wl.SOFTMAX, rope_table=table,
                                out_dtype=torch.float32)
    append_packed(twin, k, v, cu, pos0, table)
    torch.cuda.synchronize()
    assert_caches_equal(cache, twin)
    rows = []
    for q_ in range(S):
        a, n = int(cu[q_]), lens[q_]
        rows += [a, a + 1, a + 63, a + 64, a + n // 2, a + n - 1]
    ref = ring.chunk(q, k, v, cu, pos0, H_q=Hq, mode=wl.SOFTMAX, rope_theta=theta, rows=rows,
                     append=False)
    torch.cuda.synchronize()
    assert_parity(out[rows], ref, "bf16", "sampled rows")
