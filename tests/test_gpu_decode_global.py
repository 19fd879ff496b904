"""GPU parity of decode for the global layers of a local/global stack, and of decode calls
whose tensors sit off a 16-byte boundary.

Global layers (Sliding Window Attention glossary, "interleaving local and global layers":
the global layers attend over the whole context) are served by a cache whose ring holds the
whole context, w >= every position, so that each key set is the whole history. With few
(sequence, kv head) pairs the matrix-core decode cuts that history into as many as 64 key
ranges, merged by the combine kernel; these cases reach that cap, positions where most
ranges are empty, two sequences at once, and a ring that has wrapped. Every step is
checked against the oracle ring, both as append + decode and as the fused launch.
"""
import numpy as np
import pytest
import torch

import oracle
import sliding_window_attention_prefill_amd as swa
import swa_workloads as wl
from tests.helpers import assert_parity, misaligned

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _history(S, Hkv, w, s, d, start, theta, g):
    """A cache and the oracle ring after appending positions 0..start[q]-1 of each
    sequence (one call per sequence; the others get a negative start and are skipped)."""
    cache = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
    table = swa.swa_rope_table(int(max(start)) + 8, d, theta)
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
    return cache, ring, table


def _key_ranges(cache, Hq, mode):
    """Key ranges per (sequence, kv head) of the split decode, from the workspace size
    (S * H_kv * ranges * G * (d + 2) floats)."""
    need = swa.swa_decode_workspace_bytes(cache, Hq, mode=mode, out_dtype=torch.float32)
    S, Hkv, d = cache.k_ring.shape[0], cache.k_ring.shape[1], cache.k_ring.shape[3]
    G = Hq // Hkv
    return need // (4 * S * Hkv * G * (d + 2))


GLOBAL = [
    # S, Hq, Hkv, d, w, s, mode, history per sequence, expected key ranges
    (1, 32, 8, 128, 40000, 0, wl.SOFTMAX, [30000], 64),        # inside the first window
    (1, 32, 8, 128, 40000, 0, wl.SOFTMAX, [40123], 64),        # the ring has wrapped
    (1, 16, 8, 128, 40000, 4, wl.SIGMOID, [700], 64),          # 22 tiles: most ranges empty
    (1, 8, 8, 64, 36000, 0, wl.SOFTMAX, [35000], 64),          # d = 64, one head per kv head
    (2, 16, 8, 128, 33000, 0, wl.SOFTMAX, [20000, 33050], 32), # two sequences
]


@pytest.mark.parametrize("case", GLOBAL, ids=lambda c: "S%d_Hq%d_d%d_w%d_hist%s" % (
    c[0], c[1], c[3], c[4], "-".join(str(x) for x in c[7])))
@pytest.mark.parametrize("fused", [False, True], ids=["decode", "fused"])
def test_global_layer_decode(case, fused):
    S, Hq, Hkv, d, w, s, mode, hist, ranges = case
    g = torch.Generator().manual_seed(w + hist[0] + d)
    theta = 1e6
    start = torch.tensor(hist)
    cache, ring, table = _history(S, Hkv, w, s, d, start, theta, g)
    assert _key_ranges(cache, Hq, mode) == ranges
    slopes = tuple(np.linspace(-0.02, 0.02, Hq).tolist()) if mode == wl.SIGMOID else None
    sl = None if slopes is None else torch.tensor(slopes, dtype=torch.float32, device=DEV)
    for step in range(3):
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
        mr, sr = assert_parity(out, ref, "bf16", "global decode step %d" % step)
        print("step %d max_rel %.2e sum_rel %.2e" % (step, mr, sr))


def test_global_128k_workload_first_steps():
    """The Gemma-3-style global layer of the bench (two sequences, a 131,072-token cache,
    positions below it): its first four fused steps against the oracle ring."""
    cfg = wl.DECODE_GLOBAL_128K
    st = wl.decode_inputs(cfg, device="cpu", steps=4)
    cache = swa.SwaCache(st.k_ring.to(DEV), st.v_ring.to(DEV), None, None)
    ring = oracle.Ring.from_state(st.k_ring, st.v_ring, None, None, st.lengths - 1)
    table = swa.swa_rope_table(cfg.len_hi + 8, cfg.d, cfg.rope_theta)
    assert int(st.lengths.max()) + 4 <= cfg.w
    for t in range(4):
        pos = (st.lengths + t).to(torch.int32)
        out = swa.swa_decode_append(st.q_steps[t].to(DEV), st.k_steps[t, :, 0].contiguous().to(DEV),
                                    st.v_steps[t, :, 0].contiguous().to(DEV), pos.to(DEV), cache,
                                    mode=cfg.mode, rope_table=table, out_dtype=torch.float32)
        ring.append(st.k_steps[t], st.v_steps[t], pos, rope_theta=cfg.rope_theta)
        ref = ring.decode(st.q_steps[t], pos, H_q=cfg.H_q, mode=cfg.mode,
                          rope_theta=cfg.rope_theta)
        torch.cuda.synchronize()
        assert_parity(out, ref, "bf16", "global 128K step %d" % t)


# ------------------------------------------------------------------------ misaligned tensors

@pytest.mark.parametrize("w,s,G", [(64, 4, 4), (700, 2, 4), (300, 0, 8)])
@pytest.mark.parametrize("fused", [False, True], ids=["decode", "fused"])
def test_decode_misaligned_tensors(w, s, G, fused):
    """Tensors 4 bytes off a 16-byte boundary (query, output, cache, new token) take the
    general kernel: the result matches the oracle, and the aligned call on the same data."""
    S, Hkv, d = 3, 2, 128
    Hq = G * Hkv
    theta = 1e4
    g = torch.Generator().manual_seed(w + G)
    start = torch.tensor([w // 2, w + 17, 3 * w + 5])
    cache_a, ring, table = _history(S, Hkv, w, s, d, start, theta, g)
    cache_m = swa.SwaCache(misaligned(cache_a.k_ring), misaligned(cache_a.v_ring),
                           None if s == 0 else misaligned(cache_a.k_sink),
                           None if s == 0 else misaligned(cache_a.v_sink))
    for step in range(3):
        pos = (start + step).to(torch.int32).to(DEV)
        kn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16).to(DEV)
        vn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16).to(DEV)
        qn = torch.randn((S, Hq, d), generator=g).to(torch.bfloat16).to(DEV)
        outs = []
        for cache, mis in ((cache_a, False), (cache_m, True)):
            o = torch.empty((S, Hq, d), dtype=torch.float32, device=DEV)
            o = misaligned(o) if mis else o
            qq = misaligned(qn) if mis else qn
            if fused:
                k_ = misaligned(kn) if mis else kn
                v_ = misaligned(vn) if mis else vn
                swa.swa_decode_append(qq, k_, v_, pos, cache, mode=wl.SOFTMAX,
                                      rope_table=table, out=o)
            else:
                swa.swa_kv_append(cache, kn[:, None].contiguous(), vn[:, None].contiguous(), pos,
                                  rope_table=table)
                swa.swa_decode(qq, pos, cache, mode=wl.SOFTMAX, rope_table=table, out=o)
            outs.append(o)
        ring.append(kn[:, None].cpu(), vn[:, None].cpu(), pos.cpu(), rope_theta=theta)
        ref = ring.decode(qn.cpu(), pos.cpu(), H_q=Hq, mode=wl.SOFTMAX, rope_theta=theta)
        torch.cuda.synchronize()
        for o in outs:
            assert_parity(o, ref, "bf16", "misaligned decode step %d" % step)
    # both caches hold the same appended tokens (values bit for bit)
    assert torch.equal(cache_a.v_ring.cpu(), cache_m.v_ring.cpu())
    assert torch.allclose(cache_a.k_ring.float().cpu(), cache_m.k_ring.float().cpu(),
                          atol=1e-2, rtol=1e-2)
