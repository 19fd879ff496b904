"""GPU parity of the training pair on the general vector kernels with the oracle.

Shapes outside the matrix-core path train on the general kernels: float32 inputs (the tiny
SWAT layer in float32), head sizes other than 64 and 128, dilated windows, and tensors that
are not 16-byte aligned. Every case compares o, lse (softmax) and dq, dk, dv element by
element with the float64 oracle on the same rounded inputs, at the float32 bar for float32
inputs and the bfloat16 bar otherwise.
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


def _inputs(B, Hq, Hkv, N, d, seed, dtype):
    g = torch.Generator().manual_seed(seed)
    mk = lambda *s: torch.randn(s, generator=g).to(dtype)
    return mk(B, N, Hq, d), mk(B, N, Hkv, d), mk(B, N, Hkv, d), mk(B, N, Hq, d)


def _dense_lse(q, k, w, s, r, slopes, theta):
    """log sum_{j in K(i)} exp(x_ij) in float64 from a dense masked score matrix (dilated K)."""
    B, N, Hq, d = q.shape
    Hkv = k.shape[2]
    qq, kk = q.double().numpy(), k.double().numpy()
    if theta > 0:
        from oracle import dense
        qq, kk = dense.rope_dense(qq, theta), dense.rope_dense(kk, theta)
    kk = np.repeat(kk, Hq // Hkv, axis=2)
    x = np.einsum("bihd,bjhd->bhij", qq, kk) / np.sqrt(d)
    i, j = np.arange(N)[:, None], np.arange(N)[None, :]
    if slopes is not None:
        x = x + np.asarray(slopes)[None, :, None, None] * (i - j)
    keep = (j <= i) & ((((i - j) % r == 0) & ((i - j) // r < w)) | (j < s))
    x = np.where(keep, x, -np.inf)
    m = x.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True)))[..., 0]


def _misalign(t):
    """The same values in a tensor whose data pointer is 4 bytes past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    off = 4 // t.element_size()
    out = flat[off:off + t.numel()].view(t.shape)
    out.copy_(t)
    assert out.data_ptr() % 16 != 0
    return out


def _check(case, misalign=False):
    B, Hq, Hkv, N, d, w, s, r, mode, alibi, theta, dt, out_dt = case
    q, k, v, dout = _inputs(B, Hq, Hkv, N, d, seed=N + d + w + r, dtype=dt)
    slopes = tuple(np.linspace(-0.3, 0.3, Hq).tolist()) if alibi else None
    table = swa.swa_rope_table(N, d, theta) if theta > 0 else None
    sl = torch.tensor(slopes, dtype=torch.float32, device=DEV) if slopes is not None else None
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    g = dout.to(DEV).to(out_dt)
    if misalign:
        qd, kd, vd, g = (_misalign(x) for x in (qd, kd, vd, g))
    o, lse = swa.swa_prefill_train(qd, kd, vd, w=w, s=s, mode=mode, alibi_slopes=sl,
                                   rope_table=table, out_dtype=out_dt, dilation=r)
    dq, dk, dv = swa.swa_prefill_backward(qd, kd, vd, o, lse, g, w=w, s=s, mode=mode,
                                          alibi_slopes=sl, rope_table=table, dilation=r)
    torch.cuda.synchronize()
    bar = "f32" if dt == torch.float32 and out_dt == torch.float32 else "bf16"
    kw = dict(w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta, dilation=r)
    ref_o = oracle.prefill(q, k, v, **kw)
    if out_dt == torch.bfloat16:
        ref_o = torch.from_numpy(ref_o).to(torch.bfloat16).double().numpy()
    assert_parity(o, ref_o, bar, "o")
    ref = oracle.backward(q, k, v, g.cpu(), **kw)
    for name, got, rr in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        if out_dt == torch.bfloat16:
            rr = torch.from_numpy(rr).to(torch.bfloat16).double().numpy()
        assert_parity(got, rr, bar, name)
    if mode == wl.SOFTMAX:
        np.testing.assert_allclose(lse.cpu().double().numpy(),
                                   _dense_lse(q, k, w, s, r, slopes, theta), rtol=0, atol=1e-4)


F32, BF16 = torch.float32, torch.bfloat16
CASES = [  # B, Hq, Hkv, N, d, w, s, r, mode, alibi, theta, in dtype, out dtype
    (1, 4, 4, 256, 64, 16, 0, 1, wl.SIGMOID, True, 1e4, F32, F32),
    (2, 4, 2, 190, 32, 24, 2, 1, wl.SOFTMAX, True, 1e4, F32, F32),
    (1, 6, 2, 150, 96, 40, 0, 1, wl.SIGMOID, False, 1e4, BF16, F32),
    (1, 2, 1, 130, 256, 33, 3, 1, wl.SOFTMAX, True, 1e6, BF16, F32),
    (1, 2, 2, 97, 2, 5, 1, 1, wl.SOFTMAX, False, 1e2, F32, F32),
    (2, 4, 2, 300, 64, 20, 0, 2, wl.SIGMOID, True, 1e4, BF16, F32),
    (1, 4, 1, 257, 128, 16, 4, 4, wl.SOFTMAX, True, 1e6, BF16, F32),
    (1, 3, 1, 200, 48, 9, 2, 3, wl.SOFTMAX, True, 1e4, F32, F32),
    (1, 2, 2, 120, 80, 500, 0, 5, wl.SIGMOID, False, 0.0, F32, F32),
    (1, 2, 1, 140, 64, 30, 1, 1, wl.SOFTMAX, True, 1e4, F32, BF16),
    (1, 2, 2, 1, 64, 4, 0, 1, wl.SIGMOID, True, 1e4, F32, F32),
]


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: "B%d_Hq%d_Hkv%d_N%d_d%d_w%d_s%d_r%d_m%d" % c[:9])
def test_general_training_matches_oracle(case):
    _check(case)


@pytest.mark.parametrize("mode", [wl.SIGMOID, wl.SOFTMAX])
def test_unaligned_bf16_tensors_train_on_the_general_kernels(mode):
    """bf16, d 64, contiguous window, but q, k, v and dout 4 bytes off a 16-byte boundary:
    the matrix-core path does not take them; the general kernels give the oracle's answer."""
    _check((1, 4, 2, 210, 64, 30, 2, 1, mode, True, 1e4, BF16, F32), misalign=True)


def test_tiny_swat_layer_f32():
    """The tiny SWAT layer in float32 (B 1, H 4, N 256, d 64, w 16, sigmoid, balanced ALiBi,
    RoPE) with its workload generator's inputs."""
    cfg = wl.C1
    q, k, v = wl.prefill_inputs(cfg, device="cpu")
    g = torch.Generator().manual_seed(98)
    dout = torch.randn(q.shape, generator=g)
    table = swa.swa_rope_table(cfg.N, cfg.d, cfg.rope_theta)
    sl = torch.tensor(cfg.slopes, dtype=torch.float32, device=DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = swa.swa_prefill_train(qd, kd, vd, w=cfg.w, s=cfg.s, mode=cfg.mode, alibi_slopes=sl,
                                   rope_table=table)
    dq, dk, dv = swa.swa_prefill_backward(qd, kd, vd, o, lse, dout.to(DEV), w=cfg.w, s=cfg.s,
                                          mode=cfg.mode, alibi_slopes=sl, rope_table=table)
    torch.cuda.synchronize()
    assert lse is None and dq.dtype == torch.float32
    ref = oracle.backward(q, k, v, dout, w=cfg.w, s=cfg.s, mode=cfg.mode, slopes=cfg.slopes,
                          rope_theta=cfg.rope_theta)
    for name, got, rr in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        assert_parity(got, rr, "f32", name)


def test_general_backward_deterministic():
    case = (1, 4, 2, 333, 96, 50, 3, 2, wl.SOFTMAX, True, 1e4, BF16, F32)
    B, Hq, Hkv, N, d, w, s, r, mode, alibi, theta, dt, out_dt = case
    q, k, v, dout = (x.to(DEV) for x in _inputs(B, Hq, Hkv, N, d, seed=3, dtype=dt))
    table = swa.swa_rope_table(N, d, theta)
    runs = []
    for _ in range(2):
        o, lse = swa.swa_prefill_train(q, k, v, w=w, s=s, mode=mode, rope_table=table,
                                       out_dtype=out_dt, dilation=r)
        runs.append(swa.swa_prefill_backward(q, k, v, o, lse, dout.to(out_dt), w=w, s=s,
                                             mode=mode, rope_table=table, dilation=r))
    torch.cuda.synchronize()
    for a, b in zip(*runs):
        assert torch.equal(a, b)
