"""GPU parity of the matrix-core prefill over the whole range of ALiBi slopes.

The score product carries the bias through float16 operand splits (the key offset times a
two-term split of the slope; for sigmoid also the query offset i - j0 through a scaled
two-term split). These cases drive both with slopes from 2e-6 to 200 in both signs, zero on
one head, and sink tiles whose query offset reaches the sequence length, against the
float64 oracle at the bf16 bar.
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

SLOPES = (-40.0, -3.0, -1e-3, 0.0, 2e-6, 0.7, 17.0, 200.0)


@pytest.mark.parametrize("mode", [wl.SIGMOID, wl.SOFTMAX])
@pytest.mark.parametrize("B,Hq,Hkv,N,d,w,s", [(1, 8, 2, 700, 64, 100, 40),
                                              (1, 8, 8, 1500, 128, 300, 70),
                                              (2, 8, 1, 333, 64, 64, 130)])
def test_prefill_alibi_slope_range(B, Hq, Hkv, N, d, w, s, mode):
    g = torch.Generator().manual_seed(N + d + s)
    mk = lambda *sh: (torch.randn(sh, generator=g) * 0.5).to(torch.bfloat16)
    q, k, v = mk(B, N, Hq, d), mk(B, N, Hkv, d), mk(B, N, Hkv, d)
    theta = 1e4
    table = swa.swa_rope_table(N, d, theta)
    sl = torch.tensor(SLOPES, dtype=torch.float32, device=DEV)
    o = swa.swa_prefill(q.to(DEV), k.to(DEV), v.to(DEV), w=w, s=s, mode=mode, alibi_slopes=sl,
                        rope_table=table, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref = oracle.prefill(q, k, v, w=w, s=s, mode=mode, slopes=SLOPES, rope_theta=theta)
    assert_parity(o, ref, "bf16", "o")
    # per head too, so that a large-slope head cannot hide a small-slope one
    for h in range(Hq):
        assert_parity(o[:, :, h], ref[:, :, h], "bf16", "head %d" % h)
