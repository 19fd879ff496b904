"""GPU parity of the whole-window decode at d = 128 with four or eight query heads per kv head
(the matrix-core form that serves SWA(64, 4)) against the oracle ring.

Shapes cover one live 32-row tile (w + s = 32), exactly 128 rows (four tiles), a window of one
key, sinks past a tile boundary, and eight query heads per kv head (two head groups, of which
only the first writes the appended token). Each case runs from a partly filled ring at mixed
positions, appended separately or fused, with and without rotation, with and without ALiBi,
float32 and bf16 output.
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

# (S, H_kv, G, w, s, theta, alibi, out_dtype)
CASES = [
    (3, 2, 8, 64, 4, 1e4, True, torch.float32),
    (2, 2, 4, 124, 4, 1e6, False, torch.bfloat16),
    (3, 1, 4, 32, 0, 1e4, True, torch.float32),
    (4, 2, 8, 96, 32, 0.0, True, torch.bfloat16),
    (2, 3, 4, 1, 0, 1e4, False, torch.float32),
    (3, 2, 4, 40, 30, 0.0, False, torch.float32),
]


@pytest.mark.parametrize("mode", [wl.SIGMOID, wl.SOFTMAX])
@pytest.mark.parametrize("fused", [False, True], ids=["append_then_decode", "fused"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "S%d_Hkv%d_G%d_w%d_s%d" % c[:5])
def test_window_decode_matches_oracle(case, fused, mode):
    S, Hkv, G, w, s, theta, alibi, out_dtype = case
    d, Hq = 128, Hkv * G
    g = torch.Generator().manual_seed(S * 31 + w + G + s)
    steps = 8
    # positions from an empty ring to past several wraps; the first sequence starts at 0
    start = torch.randint(0, 3 * w + 40, (S,), generator=g)
    start[0] = 0
    table = swa.swa_rope_table(int(start.max()) + steps + 1, d, theta) if theta > 0 else None
    slopes = tuple(np.linspace(-0.5, 0.7, Hq).tolist()) if alibi else None
    sl = torch.tensor(slopes, dtype=torch.float32, device=DEV) if alibi else None
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
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
        print("case", case, "fused", fused, "mode", mode, "step", step, flush=True)
        if fused:
            out = swa.swa_decode_append(qn.to(DEV), kn.to(DEV), vn.to(DEV), pos.to(DEV), cache,
                                        mode=mode, alibi_slopes=sl, rope_table=table,
                                        out_dtype=out_dtype)
        else:
            swa.swa_kv_append(cache, kn[:, None].to(DEV), vn[:, None].to(DEV), pos.to(DEV),
                              rope_table=table)
            out = swa.swa_decode(qn.to(DEV), pos.to(DEV), cache, mode=mode, alibi_slopes=sl,
                                 rope_table=table, out_dtype=out_dtype)
        ring.append(kn[:, None], vn[:, None], pos, rope_theta=theta)
        ref = ring.decode(qn, pos, H_q=Hq, mode=mode, slopes=slopes, rope_theta=theta)
        torch.cuda.synchronize()
        if out_dtype == torch.bfloat16:
            # the stored output is rounded once more: compare against the rounded reference
            ref_r = torch.from_numpy(ref).to(torch.bfloat16).to(torch.float64).numpy()
            max_rel, sum_rel = errors(out, ref_r)
            assert max_rel <= 2e-2 and sum_rel <= 2e-3, (step, max_rel, sum_rel)
        else:
            assert_parity(out, ref, "bf16", "window decode step %d" % step)
    # the cache the launches leave: values bit for bit, keys to the bf16 rounding of the
    # rotation
    vr = cache.v_ring.cpu().double().numpy()
    kr = cache.k_ring.cpu().double().numpy()
    for q_ in range(S):
        for t in range(w):
            if ring.pos[q_, t] >= 0:
                np.testing.assert_array_equal(vr[q_, :, t], ring.v[q_, :, t])
                np.testing.assert_allclose(kr[q_, :, t], ring.k[q_, :, t], rtol=1e-2, atol=1e-2)
    if s > 0:
        vs = cache.v_sink.cpu().double().numpy()
        np.testing.assert_array_equal(vs, ring.v_sink)
