"""GPU parity over a seeded sweep of random shapes and options.

Every case draws its shape (batch, heads, grouping, length, head size, window, sinks) and its
options (mode, ALiBi, RoPE, dtypes) from a fixed seed, runs the library through the C ABI and
compares every output element with the CPU oracle on the same inputs. The hand-picked cases
elsewhere pin particular paths; this sweep covers the combinations between them (short and
ragged sequences, windows longer than the sequence, sinks beyond the window, one to eight
query heads per kv head, both head sizes of the matrix-core path and odd ones of the general
path).
"""
import numpy as np
import pytest
import torch

import oracle
import sliding_window_attention_prefill_amd as swa
import swa_workloads as wl
from tests.helpers import assert_parity, errors

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _prefill_cases(n, seed):
    rs = np.random.RandomState(seed)
    cases = []
    for idx in range(n):
        dtype = "f32" if rs.rand() < 0.15 else "bf16"
        d = int(rs.choice([64, 128, 64, 128, 32, 96])) if dtype == "bf16" else int(rs.choice([32, 64, 128]))
        H_kv = int(rs.choice([1, 2, 4]))
        G = int(rs.choice([1, 2, 3, 4, 8]))
        B = int(rs.choice([1, 2]))
        N = int(rs.choice([1, 2, 63, 64, 65, int(rs.randint(3, 700))]))
        w = int(rs.choice([1, 2, int(rs.randint(1, 300)), int(rs.randint(300, 900))]))
        s = int(rs.choice([0, 0, 1, int(rs.randint(1, 80))]))
        mode = wl.SIGMOID if rs.rand() < 0.5 else wl.SOFTMAX
        alibi = rs.rand() < 0.6
        theta = float(rs.choice([0.0, 1e4, 1e6]))
        out_bf16 = rs.rand() < 0.3
        cases.append((idx, dtype, B, H_kv * G, H_kv, N, d, w, s, mode, alibi, theta, out_bf16))
    return cases


@pytest.mark.parametrize("case", _prefill_cases(28, 20261203),
                         ids=lambda c: "c%02d_%s_B%d_Hq%d_Hkv%d_N%d_d%d_w%d_s%d_m%d" % c[:10])
def test_prefill_random_shapes(case):
    idx, dtype, B, Hq, Hkv, N, d, w, s, mode, alibi, theta, out_bf16 = case
    rs = np.random.RandomState(1000 + idx)
    slopes = tuple((rs.uniform(-0.7, 0.7, Hq)).tolist()) if alibi else None
    cfg = wl.PrefillConfig("sweep", dtype, B, Hq, Hkv, N, d, w, s, mode, theta, slopes,
                           seed=5000 + idx)
    q, k, v = wl.prefill_inputs(cfg, device=DEV)
    sl = wl.slopes_tensor(cfg.slopes, device=DEV)
    table = swa.swa_rope_table(N, d, theta) if theta > 0 else None
    out_dtype = torch.bfloat16 if out_bf16 else torch.float32
    out = torch.full((B, N, Hq, d), float("nan"), dtype=out_dtype, device=DEV)
    swa.swa_prefill(q, k, v, w=w, s=s, mode=mode, alibi_slopes=sl, rope_table=table, out=out)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, k, v, w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta)
    if out_bf16:
        # the stored output is rounded once more: compare against the rounded reference
        ref_r = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
        max_rel, sum_rel = errors(out, ref_r)
        assert max_rel <= 2e-2 and sum_rel <= 2e-3, (max_rel, sum_rel)
    else:
        assert_parity(out, ref, dtype, "sweep case %d" % idx)


def _decode_cases(n, seed):
    rs = np.random.RandomState(seed)
    cases = []
    for idx in range(n):
        d = int(rs.choice([64, 128, 64, 128, 96]))
        H_kv = int(rs.choice([1, 2, 4, 8]))
        G = int(rs.choice([1, 2, 4, 8]))
        S = int(rs.randint(1, 7))
        w = int(rs.choice([1, 3, int(rs.randint(4, 64)), int(rs.randint(64, 300))]))
        s = int(rs.choice([0, 0, 2, int(rs.randint(1, 20))]))
        mode = wl.SIGMOID if rs.rand() < 0.5 else wl.SOFTMAX
        alibi = rs.rand() < 0.5
        cases.append((idx, S, H_kv * G, H_kv, d, w, s, mode, alibi))
    return cases


@pytest.mark.parametrize("case", _decode_cases(12, 7331),
                         ids=lambda c: "c%02d_S%d_Hq%d_Hkv%d_d%d_w%d_s%d_m%d" % c[:8])
def test_fused_decode_random_shapes(case):
    """History appended in one call per sequence, then several fused append + decode steps;
    every step is compared with the oracle ring."""
    idx, S, Hq, Hkv, d, w, s, mode, alibi = case
    g = torch.Generator().manual_seed(900 + idx)
    steps = 6
    start = torch.randint(0, 2 * w + s + 3, (S,), generator=g)
    slopes = tuple(np.linspace(-0.6, 0.6, Hq).tolist()) if alibi else None
    theta = 1e4
    table = swa.swa_rope_table(int(start.max()) + steps + 1, d, theta)
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
    sl = torch.tensor(slopes, dtype=torch.float32, device=DEV) if alibi else None
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
    ws = torch.empty(max(swa.swa_decode_workspace_bytes(cache, Hq, mode=mode,
                                                        out_dtype=torch.float32), 1),
                     dtype=torch.uint8, device=DEV)
    for step in range(steps):
        pos = (start + step).to(torch.int32)
        kn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16)
        vn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16)
        qn = torch.randn((S, Hq, d), generator=g).to(torch.bfloat16)
        out = swa.swa_decode_append(qn.to(DEV), kn.to(DEV), vn.to(DEV), pos.to(DEV), cache,
                                    mode=mode, alibi_slopes=sl, rope_table=table,
                                    out_dtype=torch.float32, workspace=ws)
        ring.append(kn[:, None], vn[:, None], pos, rope_theta=theta)
        ref = ring.decode(qn, pos, H_q=Hq, mode=mode, slopes=slopes, rope_theta=theta)
        torch.cuda.synchronize()
        assert_parity(out, ref, "bf16", "decode sweep case %d step %d" % (idx, step))


@pytest.mark.parametrize("S,Hq,Hkv,d,w,s,mode", [
    (1, 8, 2, 128, 3000, 0, wl.SOFTMAX), (2, 4, 4, 64, 2500, 4, wl.SIGMOID),
    (1, 32, 8, 128, 4096, 0, wl.SOFTMAX), (3, 2, 1, 64, 1100, 7, wl.SOFTMAX),
    (1, 8, 2, 128, 5000, 0, wl.SIGMOID), (2, 8, 8, 128, 1400, 3, wl.SOFTMAX),
    # several sink tiles ahead of the window tiles, eight query heads per kv head
    (2, 8, 1, 64, 1500, 70, wl.SOFTMAX), (2, 16, 2, 128, 1200, 45, wl.SIGMOID)])
@pytest.mark.parametrize("fused", [False, True], ids=["decode", "fused"])
def test_split_kv_decode_long_windows(S, Hq, Hkv, d, w, s, mode, fused):
    """Long windows with few sequences run split over several blocks per (sequence, kv
    head) and merged by the combine kernel; outputs match the oracle ring at positions
    inside the first window and after it has wrapped."""
    g = torch.Generator().manual_seed(S * 7 + w)
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
    # history: sequence q_ has start[q_] tokens (some shorter than w, some past it)
    start = torch.tensor([(w // 3) if q_ % 2 == 0 else (w + 57 + 31 * q_) for q_ in range(S)])
    theta = 1e4
    steps = 3
    table = swa.swa_rope_table(int(start.max()) + steps + 1, d, theta)
    for q_ in range(S):
        n0 = int(start[q_])
        pos_all = torch.full((S,), -1, dtype=torch.int32)
        pos_all[q_] = 0
        kh = torch.randn((S, n0, Hkv, d), generator=g).to(torch.bfloat16)
        vh = torch.randn((S, n0, Hkv, d), generator=g).to(torch.bfloat16)
        swa.swa_kv_append(cache, kh.to(DEV), vh.to(DEV), pos_all.to(DEV), rope_table=table)
        ring.append(kh, vh, pos_all, rope_theta=theta)
    need = swa.swa_decode_workspace_bytes(cache, Hq, mode=mode, out_dtype=torch.float32)
    assert need > 0  # these shapes take the split path
    slopes = tuple(np.linspace(-0.3, 0.3, Hq).tolist())
    sl = torch.tensor(slopes, dtype=torch.float32, device=DEV)
    for step in range(steps):
        pos = (start + step).to(torch.int32)
        kn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16)
        vn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16)
        qn = torch.randn((S, Hq, d), generator=g).to(torch.bfloat16)
        if fused:
            out = swa.swa_decode_append(qn.to(DEV), kn.to(DEV), vn.to(DEV), pos.to(DEV), cache,
                                        mode=mode, alibi_slopes=sl, rope_table=table,
                                        out_dtype=torch.float32)
        else:
            swa.swa_kv_append(cache, kn[:, None].to(DEV), vn[:, None].to(DEV), pos.to(DEV),
                              rope_table=table)
            out = swa.swa_decode(qn.to(DEV), pos.to(DEV), cache, mode=mode, alibi_slopes=sl,
                                 rope_table=table, out_dtype=torch.float32)
        ring.append(kn[:, None], vn[:, None], pos, rope_theta=theta)
        ref = ring.decode(qn, pos, H_q=Hq, mode=mode, slopes=slopes, rope_theta=theta)
        torch.cuda.synchronize()
        assert_parity(out, ref, "bf16", "split decode step %d" % step)
    # an invalid position gives NaN rows on the split path too
    bad = torch.full((S,), -3, dtype=torch.int32, device=DEV)
    qn = torch.randn((S, Hq, d), generator=g).to(torch.bfloat16).to(DEV)
    out = swa.swa_decode(qn, bad, cache, mode=mode, rope_table=table, out_dtype=torch.float32)
    assert torch.isnan(out).all()


@pytest.mark.parametrize("S,Hq,Hkv,d,w,s,mode", [
    (2, 8, 2, 128, 2000, 3, wl.SOFTMAX), (3, 4, 1, 64, 300, 5, wl.SIGMOID)])
def test_long_window_decode_bf16_output(S, Hq, Hkv, d, w, s, mode):
    """Fused append + decode with bf16 outputs on windows past 128 keys (the first shape runs
    split over several key ranges): every step against the oracle ring, rounded once to bf16
    like the stored output."""
    g = torch.Generator().manual_seed(17 * S + w)
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
    start = torch.tensor([(w // 2) if q_ % 2 == 0 else (w + 40 + 13 * q_) for q_ in range(S)])
    theta = 1e4
    steps = 3
    table = swa.swa_rope_table(int(start.max()) + steps + 1, d, theta)
    for q_ in range(S):
        n0 = int(start[q_])
        pos_all = torch.full((S,), -1, dtype=torch.int32)
        pos_all[q_] = 0
        kh = torch.randn((S, n0, Hkv, d), generator=g).to(torch.bfloat16)
        vh = torch.randn((S, n0, Hkv, d), generator=g).to(torch.bfloat16)
        swa.swa_kv_append(cache, kh.to(DEV), vh.to(DEV), pos_all.to(DEV), rope_table=table)
        ring.append(kh, vh, pos_all, rope_theta=theta)
    slopes = tuple(np.linspace(-0.3, 0.3, Hq).tolist())
    sl = torch.tensor(slopes, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(swa.swa_decode_workspace_bytes(cache, Hq, mode=mode,
                                                        out_dtype=torch.bfloat16), 1),
                     dtype=torch.uint8, device=DEV)
    for step in range(steps):
        pos = (start + step).to(torch.int32)
        kn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16)
        vn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16)
        qn = torch.randn((S, Hq, d), generator=g).to(torch.bfloat16)
        out = swa.swa_decode_append(qn.to(DEV), kn.to(DEV), vn.to(DEV), pos.to(DEV), cache,
                                    mode=mode, alibi_slopes=sl, rope_table=table,
                                    out_dtype=torch.bfloat16, workspace=ws)
        assert out.dtype == torch.bfloat16
        ring.append(kn[:, None], vn[:, None], pos, rope_theta=theta)
        ref = ring.decode(qn, pos, H_q=Hq, mode=mode, slopes=slopes, rope_theta=theta)
        torch.cuda.synchronize()
        ref_r = torch.from_numpy(np.asarray(ref)).to(torch.bfloat16).to(torch.float64).numpy()
        max_rel, sum_rel = errors(out.float().cpu().double().numpy(), ref_r)
        assert max_rel <= 2e-2 and sum_rel <= 2e-3, (step, max_rel, sum_rel)
