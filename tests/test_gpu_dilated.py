"""GPU parity of dilated windows (swa_prefill with dilation r > 1) with the oracle.

The window keeps every r-th position: keys i, i - r, ..., i - r (w - 1) plus the sinks. On
the matrix cores, a dilation without sinks (r up to 64, any r) runs as the plain window on
each residue class of positions (strided rows, true positions for the rotation, slopes times
r); with sinks a power-of-two dilation runs through the in-kernel stride test. Both head
sizes, both modes, grouped heads, ALiBi and RoPE, sinks, classes of one or two positions and
windows wider than a class; other dilations with sinks and float32 inputs run on the general
kernel. Dilation 1 must reproduce the plain window bit for bit.
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

CASES = [  # dtype, B, Hq, Hkv, N, d, w, s, r, mode, alibi, theta
    ("bf16", 2, 4, 2, 300, 64, 20, 0, 2, wl.SIGMOID, True, 1e4),
    ("bf16", 1, 8, 2, 517, 128, 40, 3, 4, wl.SOFTMAX, True, 1e6),
    ("bf16", 1, 2, 1, 400, 128, 16, 70, 8, wl.SIGMOID, False, 1e4),
    ("bf16", 2, 2, 2, 129, 64, 100, 0, 2, wl.SOFTMAX, False, 0.0),
    ("bf16", 1, 3, 1, 260, 64, 9, 2, 3, wl.SOFTMAX, True, 1e4),     # r = 3: general kernel
    ("f32", 1, 2, 2, 150, 32, 12, 1, 2, wl.SIGMOID, True, 1e4),     # float32: general kernel
    ("bf16", 1, 4, 4, 200, 96, 10, 0, 4, wl.SOFTMAX, False, 1e4),   # d 96: general kernel
    # residue classes (no sinks): r not a power of two, N not a multiple of r, GQA, ALiBi
    ("bf16", 2, 4, 2, 301, 64, 20, 0, 3, wl.SIGMOID, True, 1e4),
    ("bf16", 1, 8, 2, 517, 128, 40, 0, 5, wl.SOFTMAX, True, 1e6),
    ("bf16", 1, 4, 1, 700, 128, 300, 0, 2, wl.SIGMOID, False, 1e4),  # window wider than a class
    ("bf16", 1, 2, 2, 90, 64, 5, 0, 64, wl.SOFTMAX, True, 1e4),      # classes of 1 or 2 rows
    ("bf16", 1, 2, 2, 90, 64, 5, 0, 100, wl.SOFTMAX, False, 1e4),    # r > 64 with no power of two: general kernel
]


def _random_cases(n, seed):
    """Seeded draws: dilations 2-70 (residue classes without sinks, the stride test with sinks
    and a power of two, the general kernel otherwise), lengths that are not multiples of r,
    windows narrower and wider than a class, both head sizes and modes, GQA, ALiBi, RoPE."""
    rs = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        r = int(rs.choice([2, 3, 4, 6, 7, 8, 16, int(rs.randint(2, 70))]))
        d = int(rs.choice([64, 128]))
        Hkv = int(rs.choice([1, 2]))
        G = int(rs.choice([1, 2, 4]))
        N = int(rs.choice([int(rs.randint(1, 80)), int(rs.randint(80, 600))]))
        w = int(rs.choice([1, int(rs.randint(2, 40)), int(rs.randint(2, 40)), int(rs.randint(40, 300))]))
        s = int(rs.choice([0, 0, 0, int(rs.randint(1, 40))]))
        mode = wl.SIGMOID if rs.rand() < 0.5 else wl.SOFTMAX
        alibi = bool(rs.rand() < 0.5)
        theta = float(rs.choice([0.0, 1e4]))
        cases.append(("bf16", int(rs.choice([1, 2])), Hkv * G, Hkv, N, d, w, s, r, mode, alibi, theta))
    return cases


@pytest.mark.parametrize("case", CASES + _random_cases(14, 20261205),
                         ids=lambda c: "%s_N%d_d%d_w%d_s%d_r%d_m%d" % ((c[0],) + c[4:10]))
def test_dilated_matches_oracle(case):
    dtype, B, Hq, Hkv, N, d, w, s, r, mode, alibi, theta = case
    slopes = tuple(np.linspace(-0.4, 0.4, Hq).tolist()) if alibi else None
    cfg = wl.PrefillConfig("dil", dtype, B, Hq, Hkv, N, d, w, s, mode, theta, slopes,
                           seed=N + r + d)
    q, k, v = wl.prefill_inputs(cfg, device=DEV)
    table = swa.swa_rope_table(N, d, theta) if theta > 0 else None
    out = swa.swa_prefill(q, k, v, w=w, s=s, mode=mode, alibi_slopes=wl.slopes_tensor(slopes, DEV),
                          rope_table=table, out_dtype=torch.float32, dilation=r)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, k, v, w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta,
                         dilation=r)
    assert_parity(out, ref, dtype, "dilated")


def test_dilation_one_is_the_plain_window():
    cfg = wl.PrefillConfig("dil1", "bf16", 1, 4, 2, 333, 128, 50, 2, wl.SOFTMAX, 1e4, None, seed=3)
    q, k, v = wl.prefill_inputs(cfg, device=DEV)
    table = swa.swa_rope_table(cfg.N, cfg.d, 1e4)
    a = swa.swa_prefill(q, k, v, w=50, s=2, mode=wl.SOFTMAX, rope_table=table,
                        out_dtype=torch.float32)
    b = swa.swa_prefill(q, k, v, w=50, s=2, mode=wl.SOFTMAX, rope_table=table,
                        out_dtype=torch.float32, dilation=1)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_dilated_swat340m_layer_sampled_rows():
    """The SWAT-340M layer shape with dilation 2 (window of 512 keys over 1023 positions):
    sampled rows of every sequence and head against the oracle, in the full launch."""
    cfg = wl.C2
    q, k, v = wl.prefill_inputs(cfg, device=DEV)
    table = swa.swa_rope_table(cfg.N, cfg.d, cfg.rope_theta)
    out = swa.swa_prefill(q, k, v, w=cfg.w, s=cfg.s, mode=cfg.mode,
                          alibi_slopes=wl.slopes_tensor(cfg.slopes, DEV), rope_table=table,
                          out_dtype=torch.float32, dilation=2)
    rows = wl.sample_rows(cfg.N, 24, seed=21, must=(0, 1, 63, 64, 1021, 1022, 1023, 1024))
    ref = oracle.prefill(q, k, v, w=cfg.w, s=cfg.s, mode=cfg.mode, slopes=cfg.slopes,
                         rope_theta=cfg.rope_theta, rows=rows, dilation=2)
    torch.cuda.synchronize()
    assert_parity(out[:, rows], ref, "bf16", "dilated C2 rows")
