"""swa_decode_append_static, the decode entry point that allocates nothing (its split
partials live in the library's own device scratch array), against swa_decode_append with a
caller workspace: the same outputs and cache contents on two calls in a row, the second on a
smaller problem, and the oracle ring at the usual bar."""
import numpy as np
import pytest
import torch

import oracle
import sliding_window_attention_prefill_amd as swa
import swa_workloads as wl
from tests.helpers import assert_parity

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _twin_caches(S, Hkv, w, s, d, start, theta, g):
    """Two identical caches and the oracle ring after positions 0..start[q]-1."""
    a = swa.SwaCache.empty(S, Hkv, w, s, d, torch.bfloat16)
    ring = oracle.Ring(S, Hkv, w, s, d)
    table = swa.swa_rope_table(int(max(start)) + 8, d, theta)
    for q_ in range(S):
        pos_all = torch.full((S,), -1, dtype=torch.int32)
        pos_all[q_] = 0
        n0 = int(start[q_])
        kh = torch.randn((S, n0, Hkv, d), generator=g).to(torch.bfloat16)
        vh = torch.randn((S, n0, Hkv, d), generator=g).to(torch.bfloat16)
        swa.swa_kv_append(a, kh.to(DEV), vh.to(DEV), pos_all.to(DEV), rope_table=table)
        ring.append(kh, vh, pos_all, rope_theta=theta)
    clone = lambda t: None if t is None else t.clone()
    b = swa.SwaCache(clone(a.k_ring), clone(a.v_ring), clone(a.k_sink), clone(a.v_sink))
    return a, b, ring, table


# the first problem splits each history into 64 key ranges (about 1 MB of partials); the
# second is smaller (5 ranges over 4 (sequence, kv head) pairs)
PROBLEMS = [(1, 32, 8, 128, 40000, 0, wl.SOFTMAX, [30000]),
            (2, 8, 2, 64, 3000, 3, wl.SIGMOID, [2000, 3100])]


def test_static_decode_matches_workspace_decode_two_calls():
    theta = 1e4
    for idx, (S, Hq, Hkv, d, w, s, mode, hist) in enumerate(PROBLEMS):
        g = torch.Generator().manual_seed(100 + idx)
        start = torch.tensor(hist)
        ca, cb, ring, table = _twin_caches(S, Hkv, w, s, d, start, theta, g)
        need = swa.swa_decode_workspace_bytes(ca, Hq, mode=mode, out_dtype=torch.float32)
        assert 0 < need <= 4 << 20
        pos = start.to(torch.int32)
        kn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16)
        vn = torch.randn((S, Hkv, d), generator=g).to(torch.bfloat16)
        qn = torch.randn((S, Hq, d), generator=g).to(torch.bfloat16)
        args = (qn.to(DEV), kn.to(DEV), vn.to(DEV), pos.to(DEV))
        ref_o = swa.swa_decode_append(*args, ca, mode=mode, rope_table=table,
                                      out_dtype=torch.float32)
        out = torch.full((S, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
        swa.swa_decode_append_static(*args, cb, out, mode=mode, rope_table=table)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o), "call %d differs from the workspace entry point" % idx
        for x, y in ((ca.k_ring, cb.k_ring), (ca.v_ring, cb.v_ring)):
            assert torch.equal(x, y)
        ring.append(kn[:, None], vn[:, None], pos, rope_theta=theta)
        ref = ring.decode(qn, pos, H_q=Hq, mode=mode, rope_theta=theta)
        assert_parity(out, ref, "bf16", "static decode call %d" % idx)
