"""GPU behaviour at and past the float16 range of the matrix-core operands.

The matrix-core prefill takes the rotated keys, the rotated queries and (softmax) the values
as float16 operands; each saturates at +-65504, the largest finite float16, instead of
overflowing to infinity. So inputs past that range give the attention of the saturated
operands, with finite outputs. These tests put a few key rows (and, for softmax, value and
query rows) at magnitudes 65280 (the largest bf16 value inside the float16 range), 65536 (the
smallest one past it), 1e6 and 1e30, spaced more than a window apart so that each query sees
at most one of them, and compare with the oracle run on the inputs saturated the same way.
Rows that see no such key are compared on their own at the usual bar, so a large value
cannot hide their errors.
"""
import numpy as np
import pytest
import torch

import oracle
import sliding_window_attention_prefill_amd as swa
import swa_workloads as wl
from tests.helpers import errors

pytestmark = pytest.mark.gpu
DEV = "cuda"
F16_MAX = 65504.0


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mode", [wl.SIGMOID, wl.SOFTMAX])
@pytest.mark.parametrize("mag", [65280.0, 65536.0, 1.0e6, 1.0e30])
def test_operands_saturate_at_float16_max(mag, mode, d):
    B, Hq, Hkv, N, w = 1, 2, 1, 700, 100
    g = torch.Generator().manual_seed(int(d + mode))
    q = torch.randn((B, N, Hq, d), generator=g)
    k = torch.randn((B, N, Hkv, d), generator=g)
    v = torch.randn((B, N, Hkv, d), generator=g)
    heavy_k = list(range(10, N, 150))          # more than w apart
    sign = lambda: torch.where(torch.rand((d,), generator=g) < 0.5, -1.0, 1.0)
    for j in heavy_k:
        k[0, j, 0] = sign() * mag
        if mode == wl.SOFTMAX:
            v[0, j, 0] = sign() * mag
    heavy_q = [75, 380] if mode == wl.SOFTMAX else []
    for i in heavy_q:
        q[0, i, 0] = sign() * mag
    q, k, v = (t.to(torch.bfloat16) for t in (q, k, v))
    out = swa.swa_prefill(q.to(DEV), k.to(DEV), v.to(DEV), w=w, mode=mode,
                          out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = out.cpu().double().numpy()
    assert np.all(np.isfinite(got))

    # the oracle on the saturated operands (the values of sigmoid enter as bf16, unclamped)
    clamp = lambda t: torch.clamp(t.double(), -F16_MAX, F16_MAX)
    qs, ks = clamp(q), clamp(k)
    vs = clamp(v) if mode == wl.SOFTMAX else v.double()
    ref = oracle.prefill(qs, ks, vs, w=w, mode=mode)

    sees = np.zeros(N, dtype=bool)
    for j in heavy_k:
        sees[j:j + w] = True
    for i in heavy_q:
        sees[i] = True
    for mask, label in ((~sees, "plain rows"), (sees, "rows that see a saturated operand")):
        mr, sr = errors(got[:, mask], ref[:, mask])
        assert mr <= 2e-2 and sr <= 2e-3, (label, mr, sr)
