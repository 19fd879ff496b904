"""GPU parity: the HIP path through the C ABI against the CPU oracle on seeded inputs.

Covers small shapes that span several tiles with a ragged tail (full outputs), the five
workloads at full size (whole outputs, in the launch configuration the bench times), exact
key-selection readouts, the ring buffer's slot mapping, output guard bands and run-to-run
determinism.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import sliding_window_attention_prefill_amd as swa
import swa_workloads as wl
from tests.helpers import (TOL_BF16_MAX, TOL_BF16_SUM, assert_parity, errors,
                           errors_blocked)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _device_inputs(cfg):
    q, k, v = wl.prefill_inputs(cfg, device=DEV)
    slopes = wl.slopes_tensor(cfg.slopes, device=DEV)
    table = swa.swa_rope_table(cfg.N, cfg.d, cfg.rope_theta) if cfg.rope_theta > 0 else None
    return q, k, v, slopes, table


def _run(cfg, out_dtype=torch.float32):
    q, k, v, slopes, table = _device_inputs(cfg)
    out = torch.full((cfg.B, cfg.N, cfg.H_q, cfg.d), float("nan"), dtype=out_dtype, device=DEV)
    swa.swa_prefill(q, k, v, w=cfg.w, s=cfg.s, mode=cfg.mode, alibi_slopes=slopes,
                    rope_table=table, out=out)
    torch.cuda.synchronize()
    return q, k, v, out


def _oracle(cfg, q, k, v, rows=None):
    return oracle.prefill(q, k, v, w=cfg.w, s=cfg.s, mode=cfg.mode, slopes=cfg.slopes,
                          rope_theta=cfg.rope_theta, rows=rows)


def test_c1_tiny_swat_f32_full():
    cfg = wl.C1
    q, k, v, out = _run(cfg)
    ref = _oracle(cfg, q, k, v)
    max_rel, _ = assert_parity(out, ref, "f32", cfg.name)
    print("C1 max_rel %.2e" % max_rel)


SMALL = [
    # dtype, B, Hq, Hkv, N, d, w, s, mode, alibi, theta
    ("bf16", 2, 4, 4, 700, 64, 128, 0, wl.SIGMOID, True, 1e4),
    ("bf16", 1, 8, 2, 600, 128, 200, 4, wl.SOFTMAX, False, 1e6),
    ("bf16", 1, 4, 2, 333, 128, 64, 0, wl.SIGMOID, True, 1e4),
    ("bf16", 1, 4, 1, 515, 64, 77, 9, wl.SOFTMAX, True, 1e4),
    ("bf16", 1, 2, 2, 300, 64, 1000, 0, wl.SOFTMAX, False, 0.0),
    ("bf16", 1, 2, 2, 130, 128, 1, 3, wl.SIGMOID, True, 1e4),
    ("bf16", 1, 16, 2, 260, 128, 96, 2, wl.SOFTMAX, True, 1e4),
    ("bf16", 1, 6, 3, 190, 64, 40, 1, wl.SIGMOID, False, 1e4),
    ("f32", 1, 4, 2, 400, 128, 50, 2, wl.SOFTMAX, True, 1e4),
    ("f32", 1, 2, 1, 97, 32, 20, 0, wl.SIGMOID, True, 1e4),
    ("bf16", 1, 2, 1, 150, 96, 33, 5, wl.SOFTMAX, True, 1e4),
    # one query head per kv head with a long window: keys packed by the pre-pass
    ("bf16", 1, 2, 2, 2600, 64, 1100, 3, wl.SIGMOID, True, 1e4),
    ("bf16", 1, 2, 2, 1500, 128, 1030, 0, wl.SIGMOID, False, 0.0),
    # keys rotated on the way into LDS, d = 128, no rotation table
    ("bf16", 2, 2, 2, 450, 128, 100, 2, wl.SIGMOID, True, 0.0),
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "%s_Hq%d_Hkv%d_N%d_d%d_w%d_s%d_m%d" % (
    c[0], c[2], c[3], c[4], c[5], c[6], c[7], c[8]))
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16], ids=["o32", "o16"])
def test_small_shapes_full_output(case, out_dtype):
    dt, B, Hq, Hkv, N, d, w, s, mode, alibi, theta = case
    slopes = tuple(np.linspace(-0.6, 0.6, Hq).tolist()) if alibi else None
    cfg = wl.PrefillConfig("small", dt, B, Hq, Hkv, N, d, w, s, mode, theta, slopes,
                           seed=100 + N)
    q, k, v, out = _run(cfg, out_dtype)
    ref = _oracle(cfg, q, k, v)
    if out_dtype == torch.bfloat16:
        # the stored output is rounded once more: widen by half an ulp of each element
        ref_t = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
        max_rel, sum_rel = errors(out, ref_t)
        assert max_rel <= 2e-2 and sum_rel <= 2e-3, (max_rel, sum_rel)
    else:
        assert_parity(out, ref, dt, cfg.name)


def _readout_inputs(B, N, Hq, Hkv, d, bits):
    q = torch.zeros((B, N, Hq, d), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, N, Hkv, d), dtype=torch.bfloat16, device=DEV)
    j = torch.arange(N, device=DEV)
    vb = torch.stack([((j >> c) & 1).to(torch.float32) for c in range(bits)], dim=-1)
    v = torch.zeros((B, N, Hkv, d), dtype=torch.float32, device=DEV)
    v[:, :, :, :bits] = vb[None, :, None, :]
    return q, k, v.to(torch.bfloat16)


@pytest.mark.parametrize("N,w,s,Hq,Hkv,d", [(300, 64, 0, 2, 2, 64), (517, 128, 5, 4, 2, 128),
                                             (260, 1, 3, 2, 1, 64), (200, 300, 0, 4, 4, 128),
                                             (1030, 512, 7, 8, 2, 128), (900, 100, 130, 2, 2, 64),
                                             (2100, 1100, 4, 2, 2, 64), (700, 200, 3, 4, 1, 64)])
def test_selection_is_bit_exact(N, w, s, Hq, Hkv, d):
    """q = k = 0 makes every weight exactly 1/2; with v_j[c] = bit c of j the float32 output
    is 1/2 * #{j in K(i) with bit c set}: exact small integers that identify the key set."""
    bits = int(N - 1).bit_length()
    q, k, v = _readout_inputs(1, N, Hq, Hkv, d, bits)
    table = swa.swa_rope_table(N, d, 1e4)
    out = swa.swa_prefill(q, k, v, w=w, s=s, mode=swa.SWA_SIGMOID, rope_table=table,
                          out_dtype=torch.float32)
    got = out[0].cpu().numpy()
    want = np.zeros((N, bits))
    for i in range(N):
        keys = np.array([j for j in range(i + 1) if i - j < w or j < s])
        for c in range(bits):
            want[i, c] = 0.5 * ((keys >> c) & 1).sum()
    for h in range(Hq):
        np.testing.assert_array_equal(got[:, h, :bits], want)
        assert np.all(got[:, h, bits:] == 0.0)


@pytest.mark.parametrize("cfg", [wl.C2, wl.C3, wl.C5], ids=lambda c: c.name)
def test_full_size_whole_output(cfg):
    """The full workload in the bench's launch configuration (float32 output), every output
    element against the oracle: max|err|/max|ref| and sum|err|/sum|ref| over the whole
    output."""
    q, k, v, out = _run(cfg)
    ref = _oracle(cfg, q, k, v)
    max_rel, sum_rel = errors_blocked(out, ref)
    print("%s whole output: max_rel %.2e sum_rel %.2e" % (cfg.name, max_rel, sum_rel))
    assert max_rel <= TOL_BF16_MAX and sum_rel <= TOL_BF16_SUM, (max_rel, sum_rel)


@pytest.mark.parametrize("cfg", [wl.C2, wl.C5], ids=lambda c: c.name)
def test_full_size_bf16_output(cfg):
    """The same with bf16 output (the bench's second output leg): the oracle's output is
    rounded once to bf16 like the stored one."""
    q, k, v, out = _run(cfg, torch.bfloat16)
    ref = _oracle(cfg, q, k, v)
    ref = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
    max_rel, sum_rel = errors_blocked(out, ref)
    print("%s whole output, bf16: max_rel %.2e sum_rel %.2e" % (cfg.name, max_rel, sum_rel))
    assert max_rel <= TOL_BF16_MAX and sum_rel <= TOL_BF16_SUM, (max_rel, sum_rel)


def test_outputs_fully_written_and_guard_bands_intact():
    cfg = wl.PrefillConfig("guard", "bf16", 1, 4, 2, 389, 128, 100, 3, wl.SOFTMAX, 1e4, None,
                           seed=9)
    q, k, v, slopes, table = _device_inputs(cfg)
    n = cfg.B * cfg.N * cfg.H_q * cfg.d
    guard = 4096
    buf = torch.full((n + 2 * guard,), float("nan"), dtype=torch.float32, device=DEV)
    buf[:guard] = 12345.0
    buf[-guard:] = -12345.0
    out = buf[guard:guard + n].view(cfg.B, cfg.N, cfg.H_q, cfg.d)
    swa.swa_prefill(q, k, v, w=cfg.w, s=cfg.s, mode=cfg.mode, rope_table=table, out=out)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert (buf[:guard] == 12345.0).all() and (buf[-guard:] == -12345.0).all()


def test_prefill_is_deterministic():
    cfg = wl.C2.with_(B=2, N=1500)
    q, k, v, slopes, table = _device_inputs(cfg)
    a = swa.swa_prefill(q, k, v, w=cfg.w, mode=cfg.mode, alibi_slopes=slopes, rope_table=table,
                        out_dtype=torch.float32)
    b = swa.swa_prefill(q, k, v, w=cfg.w, mode=cfg.mode, alibi_slopes=slopes, rope_table=table,
                        out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# ----------------------------------------------------------------------------- rotation

def test_rope_table_matches_float64():
    n, d, theta = 131072, 128, 1e4
    t = swa.swa_rope_table(n, d, theta).cpu().double().numpy()
    rows = np.array([0, 1, 7, 4095, 32767, 99999, 131071])
    i = np.arange(d // 2)
    ang = rows[:, None] * theta ** (-2.0 * i / d)
    np.testing.assert_allclose(t[rows, :, 0], np.cos(ang), atol=1.2e-7, rtol=0)
    np.testing.assert_allclose(t[rows, :, 1], np.sin(ang), atol=1.2e-7, rtol=0)


def test_rope_apply_matches_oracle_rotation():
    from oracle import dense
    B, N, H, d = 2, 300, 3, 64
    x = torch.randn((B, N, H, d), generator=torch.Generator().manual_seed(3)).to(DEV)
    pos0 = torch.tensor([0, 1000], dtype=torch.int32, device=DEV)
    table = swa.swa_rope_table(2000, d, 1e4)
    y = swa.swa_rope_apply(x.clone(), pos0, table).cpu().double().numpy()
    xx = x.cpu().double().numpy()
    for b, p0 in enumerate([0, 1000]):
        full = np.zeros((1, p0 + N, H, d))
        full[0, p0:] = xx[b]
        ref = dense.rope_dense(full, 1e4)[0, p0:]
        np.testing.assert_allclose(y[b], ref, atol=2e-5, rtol=1e-5)
    # a position outside the table gives NaN rows
    bad = torch.tensor([0, 1900], dtype=torch.int32, device=DEV)
    z = swa.swa_rope_apply(x.clone(), bad, table).cpu()
    assert torch.isfinite(z[0]).all() and torch.isnan(z[1, 100:]).all()
    assert torch.isfinite(z[1, :100]).all()


# ----------------------------------------------------------------------------- decode

def _gpu_cache_from(ring_o, dtype=torch.bfloat16):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dtype).to(DEV)
    ks = t(ring_o.k_sink) if ring_o.s > 0 else None
    vs = t(ring_o.v_sink) if ring_o.s > 0 else None
    return swa.SwaCache(t(ring_o.k), t(ring_o.v), ks, vs)


@pytest.mark.parametrize("mode", [wl.SIGMOID, wl.SOFTMAX])
@pytest.mark.parametrize("S,Hq,Hkv,d,w,s", [(5, 8, 2, 128, 16, 3), (3, 4, 4, 64, 7, 0),
                                             (4, 32, 8, 128, 64, 4), (2, 2, 1, 96, 33, 40)])
def test_decode_steps_match_oracle(mode, S, Hq, Hkv, d, w, s):
    """Starting from an empty cache at mixed positions, append + decode for several steps;
    every step's output matches the oracle ring, and the value ring matches slot for slot."""
    g = torch.Generator().manual_seed(S * 100 + w)
    steps = 24
    start = torch.randint(0, 3 * w, (S,), generator=g)
    start[0] = 0
    slopes = tuple(np.linspace(-0.5, 0.5, Hq).tolist())
    theta = 1e4
    table = swa.swa_rope_table(int(start.max()) + steps + 1, d, theta)
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
    sl = torch.tensor(slopes, dtype=torch.float32, device=DEV)
    # history: positions 0..start-1 of each sequence in one call per sequence (the other
    # sequences get a negative start and are skipped); n_new may exceed w
    for q_ in range(S):
        n0 = int(start[q_])
        if n0 == 0:
            continue
        pos_all = torch.full((S,), -1, dtype=torch.int32)
        pos_all[q_] = 0
        kh = torch.randn((S, n0, Hkv, d), generator=g).to(torch.bfloat16)
        vh = torch.randn((S, n0, Hkv, d), generator=g).to(torch.bfloat16)
        swa.swa_kv_append(cache, kh.to(DEV), vh.to(DEV), pos_all.to(DEV), rope_table=table)
        ring.append(kh, vh, pos_all, rope_theta=theta)
    for step in range(steps):
        pos = (start + step).to(torch.int32)
        kn = torch.randn((S, 1, Hkv, d), generator=g).to(torch.bfloat16)
        vn = torch.randn((S, 1, Hkv, d), generator=g).to(torch.bfloat16)
        qn = torch.randn((S, Hq, d), generator=g).to(torch.bfloat16)
        swa.swa_kv_append(cache, kn.to(DEV), vn.to(DEV), pos.to(DEV), rope_table=table)
        ring.append(kn, vn, pos, rope_theta=theta)
        out = swa.swa_decode(qn.to(DEV), pos.to(DEV), cache, mode=mode, alibi_slopes=sl,
                             rope_table=table, out_dtype=torch.float32)
        ref = ring.decode(qn, pos, H_q=Hq, mode=mode, slopes=slopes, rope_theta=theta)
        torch.cuda.synchronize()
        assert_parity(out, ref, "bf16", "decode step %d" % step)
    # slots hold exactly the oracle's values (values are stored without rotation)
    vr = cache.v_ring.cpu().double().numpy()
    for q_ in range(S):
        for t in range(w):
            if ring.pos[q_, t] >= 0:
                np.testing.assert_array_equal(vr[q_, :, t], ring.v[q_, :, t])


def test_decode_selection_is_bit_exact():
    """q = k = 0, sigmoid, v = bits of the position: the decode output identifies the key
    set exactly, through ring wrap-around and the sink store."""
    S, Hq, Hkv, d, w, s = 3, 4, 2, 16, 8, 3
    bits = 7
    steps = 40
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    table = swa.swa_rope_table(200, d, 1e4)
    start = torch.tensor([0, 5, 60], dtype=torch.int32)
    # sequences 1 and 2 first receive their earlier tokens in one call each
    for q_ in (1, 2):
        n0 = int(start[q_])
        pos_all = torch.zeros(S, dtype=torch.int32)
        kn = torch.zeros((S, n0, Hkv, d), dtype=torch.bfloat16)
        vn = torch.zeros((S, n0, Hkv, d), dtype=torch.float32)
        for j in range(n0):
            for c in range(bits):
                vn[q_, j, :, c] = float((j >> c) & 1)
        # only sequence q_ is meant to receive these; others get writes at negative positions
        pos_all[:] = -1
        pos_all[q_] = 0
        swa.swa_kv_append(cache, kn.to(DEV), vn.to(torch.bfloat16).to(DEV), pos_all.to(DEV),
                          rope_table=table)
    for step in range(steps):
        pos = start + step
        kn = torch.zeros((S, 1, Hkv, d), dtype=torch.bfloat16)
        vn = torch.zeros((S, 1, Hkv, d), dtype=torch.float32)
        for q_ in range(S):
            for c in range(bits):
                vn[q_, 0, :, c] = float((int(pos[q_]) >> c) & 1)
        swa.swa_kv_append(cache, kn.to(DEV), vn.to(torch.bfloat16).to(DEV), pos.to(DEV),
                          rope_table=table)
        qz = torch.zeros((S, Hq, d), dtype=torch.bfloat16, device=DEV)
        out = swa.swa_decode(qz, pos.to(DEV), cache, mode=swa.SWA_SIGMOID, rope_table=table,
                             out_dtype=torch.float32).cpu().numpy()
        for q_ in range(S):
            p = int(pos[q_])
            keys = np.array([j for j in range(p + 1) if p - j < w or j < s])
            for c in range(bits):
                assert np.all(out[q_, :, c] == 0.5 * ((keys >> c) & 1).sum()), (step, q_, c)


@pytest.mark.parametrize("fused", [False, True], ids=["append_then_decode", "fused"])
def test_decode_c4_full_workload(fused):
    """SWA(64, 4) decode: 64 sequences at lengths in [2048, 16384], 256 steps of append +
    decode (as two launches, and as the fused launch the bench replays); every step's
    output checked against the oracle ring."""
    cfg = wl.C4
    st = wl.decode_inputs(cfg, device="cpu")
    S, T = cfg.num_seqs, cfg.steps
    cache = swa.SwaCache(st.k_ring.to(DEV), st.v_ring.to(DEV), st.k_sink.to(DEV),
                         st.v_sink.to(DEV))
    ring = oracle.Ring.from_state(st.k_ring, st.v_ring, st.k_sink, st.v_sink, st.lengths - 1)
    table = swa.swa_rope_table(cfg.len_hi + T + 1, cfg.d, cfg.rope_theta)
    q_dev, k_dev, v_dev = st.q_steps.to(DEV), st.k_steps.to(DEV), st.v_steps.to(DEV)
    worst = (0.0, 0.0)
    for t in range(T):
        pos = (st.lengths + t).to(torch.int32)
        pos_d = pos.to(DEV)
        if fused:
            out = swa.swa_decode_append(q_dev[t], k_dev[t, :, 0].contiguous(),
                                        v_dev[t, :, 0].contiguous(), pos_d, cache,
                                        mode=cfg.mode, rope_table=table,
                                        out_dtype=torch.float32)
        else:
            swa.swa_kv_append(cache, k_dev[t], v_dev[t], pos_d, rope_table=table)
            out = swa.swa_decode(q_dev[t], pos_d, cache, mode=cfg.mode, rope_table=table,
                                 out_dtype=torch.float32)
        ring.append(st.k_steps[t], st.v_steps[t], pos, rope_theta=cfg.rope_theta)
        ref = ring.decode(st.q_steps[t], pos, H_q=cfg.H_q, mode=cfg.mode,
                          rope_theta=cfg.rope_theta)
        mr, sr = assert_parity(out, ref, "bf16", "C4 step %d" % t)
        worst = (max(worst[0], mr), max(worst[1], sr))
    # the ring ends bit-identical in its values to the oracle's
    vr = cache.v_ring.cpu().double().numpy()
    for q_ in range(S):
        for t_ in range(cfg.w):
            if ring.pos[q_, t_] >= 0:
                np.testing.assert_array_equal(vr[q_, :, t_], ring.v[q_, :, t_])
    print("C4 worst max_rel %.2e sum_rel %.2e" % worst)


@pytest.mark.parametrize("mode", [wl.SIGMOID, wl.SOFTMAX])
@pytest.mark.parametrize("S,Hq,Hkv,d,w,s", [(5, 8, 2, 128, 16, 3), (3, 4, 4, 64, 7, 0),
                                             (4, 32, 8, 128, 64, 4), (3, 16, 2, 128, 200, 2),
                                             (2, 2, 1, 96, 33, 40), (3, 8, 1, 64, 20, 1),
                                             (4, 8, 1, 64, 150, 40), (3, 4, 2, 128, 100, 70)])
def test_fused_append_decode_matches_oracle(mode, S, Hq, Hkv, d, w, s):
    """swa_decode_append (one launch: append the step's token, then answer its query) equals
    the oracle ring step by step, and leaves the same cache contents as the oracle."""
    g = torch.Generator().manual_seed(S * 7 + w + d)
    steps = 20
    start = torch.randint(0, 3 * w, (S,), generator=g)
    start[0] = 0
    slopes = tuple(np.linspace(-0.4, 0.6, Hq).tolist())
    theta = 1e4
    table = swa.swa_rope_table(int(start.max()) + steps + 1, d, theta)
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
    sl = torch.tensor(slopes, dtype=torch.float32, device=DEV)
    for q_ in range(S):
        n0 = int(start[q_])
        if n0 == 0:
            continue
        pos_all = torch.full((S,), -1, dtype=torch.int32)
        pos_all[q_] = 0
        kh = torch.randn((S, n0, Hkv, d), generator=g).to(torch.bfloat16)
        vh = torch.randn((S, n0, Hkv, d), generator=g).to(torch.bfloat16)
        swa.swa_kv_append(cache, kh.to(DEV), vh.to(DEV), pos_all.to(DEV), rope_table=table)
        ring.append(kh, vh, pos_all, rope_theta=theta)
    for step in range(steps):
        pos = (start + step).to(torch.int32)
        kn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16)
        vn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16)
        qn = torch.randn((S, Hq, d), generator=g).to(torch.bfloat16)
        out = swa.swa_decode_append(qn.to(DEV), kn.to(DEV), vn.to(DEV), pos.to(DEV), cache,
                                    mode=mode, alibi_slopes=sl, rope_table=table,
                                    out_dtype=torch.float32)
        ring.append(kn[:, None], vn[:, None], pos, rope_theta=theta)
        ref = ring.decode(qn, pos, H_q=Hq, mode=mode, slopes=slopes, rope_theta=theta)
        torch.cuda.synchronize()
        assert_parity(out, ref, "bf16", "fused step %d" % step)
    vr = cache.v_ring.cpu().double().numpy()
    kr = cache.k_ring.cpu().double().numpy()
    for q_ in range(S):
        for t in range(w):
            if ring.pos[q_, t] >= 0:
                np.testing.assert_array_equal(vr[q_, :, t], ring.v[q_, :, t])
                np.testing.assert_allclose(kr[q_, :, t], ring.k[q_, :, t], rtol=1e-2, atol=1e-2)


def test_fused_append_decode_selection_is_bit_exact():
    """q = k = 0, sigmoid, v = bits of the position, through the fused step: the output
    identifies the key set exactly, across ring wrap-around and the sink store."""
    S, Hq, Hkv, d, w, s = 2, 8, 2, 128, 16, 4
    bits = 7
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    table = swa.swa_rope_table(200, d, 1e4)
    for step in range(70):
        pos = torch.tensor([step, step + 30], dtype=torch.int32)
        if step == 0:
            # sequence 1 receives positions 0..29 first
            pos_all = torch.tensor([-1, 0], dtype=torch.int32)
            vh = torch.zeros((S, 30, Hkv, d))
            for j in range(30):
                for c in range(bits):
                    vh[1, j, :, c] = float((j >> c) & 1)
            swa.swa_kv_append(cache, torch.zeros((S, 30, Hkv, d), dtype=torch.bfloat16, device=DEV),
                              vh.to(torch.bfloat16).to(DEV), pos_all.to(DEV), rope_table=table)
        vn = torch.zeros((S, Hkv, d))
        for q_ in range(S):
            for c in range(bits):
                vn[q_, :, c] = float((int(pos[q_]) >> c) & 1)
        out = swa.swa_decode_append(torch.zeros((S, Hq, d), dtype=torch.bfloat16, device=DEV),
                                    torch.zeros((S, Hkv, d), dtype=torch.bfloat16, device=DEV),
                                    vn.to(torch.bfloat16).to(DEV), pos.to(DEV), cache,
                                    mode=swa.SWA_SIGMOID, rope_table=table,
                                    out_dtype=torch.float32).cpu().numpy()
        for q_ in range(S):
            p = int(pos[q_])
            keys = np.array([j for j in range(p + 1) if p - j < w or j < s])
            for c in range(bits):
                assert np.all(out[q_, :, c] == 0.5 * ((keys >> c) & 1).sum()), (step, q_, c)
