"""GPU parity of the training pair (swa_prefill_train, swa_prefill_backward) with the oracle.

The forward for training must equal swa_prefill bit for bit and return the softmax row
log-normalisers; the backward's dq, dk and dv are compared element by element with the
float64 oracle backward on the same rounded inputs, over head sizes 64 and 128, grouped
heads (1 to 8 query heads per kv head), both modes, with and without ALiBi and RoPE, sinks
(including sinks that only the sink rule reaches, taken by the extra sink workgroups),
windows of 1 and windows longer than the sequence, ragged lengths, and at the SWAT-340M layer
size on one sequence of the batch.
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


def _inputs(B, Hq, Hkv, N, d, seed, scale=1.0):
    g = torch.Generator().manual_seed(seed)
    mk = lambda *s: (torch.randn(s, generator=g) * scale).to(torch.bfloat16)
    return mk(B, N, Hq, d), mk(B, N, Hkv, d), mk(B, N, Hkv, d), mk(B, N, Hq, d)


def _run(q, k, v, dout, w, s, mode, slopes, theta, out_dtype=torch.float32):
    B, N, Hq, d = q.shape
    table = swa.swa_rope_table(N, d, theta) if theta > 0 else None
    sl = torch.tensor(slopes, dtype=torch.float32, device=DEV) if slopes is not None else None
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    o, lse = swa.swa_prefill_train(qd, kd, vd, w=w, s=s, mode=mode, alibi_slopes=sl,
                                   rope_table=table, out_dtype=out_dtype)
    g = dout.to(DEV).to(out_dtype)
    dq, dk, dv = swa.swa_prefill_backward(qd, kd, vd, o, lse, g, w=w, s=s, mode=mode,
                                          alibi_slopes=sl, rope_table=table)
    torch.cuda.synchronize()
    return o, lse, dq, dk, dv, g


def _dense_lse(q, k, w, s, slopes, theta):
    """log sum_{j in K(i)} exp(x_ij) in float64 from a dense masked score matrix."""
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
    keep = (j <= i) & ((i - j < w) | (j < s))
    x = np.where(keep, x, -np.inf)
    m = x.max(axis=-1, keepdims=True)
    return (m + np.log(np.exp(x - m).sum(axis=-1, keepdims=True)))[..., 0]


CASES = [  # B, Hq, Hkv, N, d, w, s, mode, alibi, theta
    (2, 2, 2, 300, 64, 40, 0, wl.SIGMOID, True, 1e4),
    (1, 4, 1, 333, 64, 100, 3, wl.SOFTMAX, True, 1e4),
    (2, 8, 2, 260, 128, 64, 0, wl.SOFTMAX, False, 1e6),
    (1, 2, 1, 450, 128, 90, 5, wl.SIGMOID, False, 0.0),
    (1, 3, 1, 200, 64, 1, 1, wl.SOFTMAX, True, 1e4),
    (1, 8, 1, 129, 128, 500, 0, wl.SIGMOID, True, 1e4),
    (2, 4, 2, 700, 64, 150, 130, wl.SOFTMAX, True, 1e4),
    (1, 2, 2, 1500, 128, 64, 2, wl.SIGMOID, True, 1e4),
    (1, 4, 4, 63, 64, 16, 0, wl.SIGMOID, False, 1e4),
    (1, 2, 1, 1, 128, 4, 0, wl.SOFTMAX, True, 1e4),
]


def _random_cases(n, seed):
    """Seeded draws over the matrix-core backward's options: head size, 1-8 query heads per
    kv head, ragged lengths (including one row and tile edges), windows from 1 to past the
    sequence, sinks (some past the window, which the extra sink workgroups take), both modes,
    ALiBi and RoPE."""
    rs = np.random.RandomState(seed)
    cases = []
    for _ in range(n):
        d = int(rs.choice([64, 128]))
        Hkv = int(rs.choice([1, 2]))
        G = int(rs.choice([1, 2, 4, 8]))
        B = int(rs.choice([1, 2]))
        N = int(rs.choice([1, 63, 64, 65, int(rs.randint(2, 600)), int(rs.randint(2, 600))]))
        w = int(rs.choice([1, int(rs.randint(1, 200)), int(rs.randint(200, 700))]))
        s = int(rs.choice([0, 0, 1, int(rs.randint(1, 100))]))
        mode = wl.SIGMOID if rs.rand() < 0.5 else wl.SOFTMAX
        alibi = bool(rs.rand() < 0.5)
        theta = float(rs.choice([0.0, 1e4, 1e6]))
        cases.append((B, Hkv * G, Hkv, N, d, w, s, mode, alibi, theta))
    return cases


@pytest.mark.parametrize("case", CASES + _random_cases(16, 20261204),
                         ids=lambda c: "B%d_Hq%d_Hkv%d_N%d_d%d_w%d_s%d_m%d" % c[:8])
def test_backward_matches_oracle(case):
    B, Hq, Hkv, N, d, w, s, mode, alibi, theta = case
    q, k, v, dout = _inputs(B, Hq, Hkv, N, d, seed=N + d + w)
    slopes = tuple(np.linspace(-0.3, 0.3, Hq).tolist()) if alibi else None
    o, lse, dq, dk, dv, g = _run(q, k, v, dout, w, s, mode, slopes, theta)
    ref = oracle.backward(q, k, v, g.cpu(), w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta)
    for name, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        if np.abs(r).max() == 0.0:
            # softmax over a single key (N = 1): dq and dk vanish exactly; the GPU's dP - dout.o
            # leaves only rounding residue
            assert got.abs().max().item() <= 1e-4, name
        else:
            assert_parity(got, r, "bf16", name)
    if mode == wl.SOFTMAX:
        np.testing.assert_allclose(lse.cpu().double().numpy(), _dense_lse(q, k, w, s, slopes, theta),
                                   rtol=0, atol=2e-3)


@pytest.mark.parametrize("mode", [wl.SIGMOID, wl.SOFTMAX])
def test_train_forward_equals_prefill(mode):
    """The forward for training is the same kernel: bit-identical output."""
    B, Hq, Hkv, N, d, w, s, theta = 2, 8, 2, 500, 128, 120, 4, 1e4
    q, k, v, _ = _inputs(B, Hq, Hkv, N, d, seed=5)
    table = swa.swa_rope_table(N, d, theta)
    sl = torch.linspace(-0.2, 0.2, Hq, device=DEV)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    ref = swa.swa_prefill(qd, kd, vd, w=w, s=s, mode=mode, alibi_slopes=sl, rope_table=table,
                          out_dtype=torch.float32)
    o, lse = swa.swa_prefill_train(qd, kd, vd, w=w, s=s, mode=mode, alibi_slopes=sl,
                                   rope_table=table, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o, ref)
    assert (lse is None) == (mode == wl.SIGMOID)


@pytest.mark.parametrize("B,Hq,Hkv,N,d,w,s", [(1, 4, 2, 400, 64, 70, 2), (1, 2, 1, 140, 64, 30, 1),
                                              (1, 4, 2, 300, 128, 24, 0)])
def test_backward_bf16_gradients(B, Hq, Hkv, N, d, w, s):
    """bf16 output and gradients: o reaches the softmax row term rounded to bf16."""
    mode, theta = wl.SOFTMAX, 1e4
    q, k, v, dout = _inputs(B, Hq, Hkv, N, d, seed=11 + N)
    slopes = tuple(np.linspace(-0.2, 0.2, Hq).tolist())
    o, lse, dq, dk, dv, g = _run(q, k, v, dout, w, s, mode, slopes, theta, out_dtype=torch.bfloat16)
    assert dq.dtype == torch.bfloat16
    ref = oracle.backward(q, k, v, g.cpu(), w=w, s=s, mode=mode, slopes=slopes, rope_theta=theta)
    for name, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        r = torch.from_numpy(r).to(torch.bfloat16).double().numpy()
        assert_parity(got, r, "bf16", name)


def test_backward_deterministic():
    B, Hq, Hkv, N, d, w, s, mode, theta = 1, 4, 1, 900, 128, 200, 3, wl.SIGMOID, 1e4
    q, k, v, dout = _inputs(B, Hq, Hkv, N, d, seed=12)
    r1 = _run(q, k, v, dout, w, s, mode, None, theta)
    r2 = _run(q, k, v, dout, w, s, mode, None, theta)
    for a, b in zip(r1[2:5], r2[2:5]):
        assert torch.equal(a, b)


@pytest.mark.parametrize("d,mode", [(64, wl.SIGMOID), (128, wl.SOFTMAX), (128, wl.SIGMOID)])
def test_backward_deterministic_several_sink_splits(d, mode):
    """Sinks that only the sink rule reaches over a long sequence: the extra workgroups split
    the queries past the window into 1024-query pieces (N - (127 + w) = 4,809 gives 5
    splits). Each split keeps its own partial and the block sums them in split order, so two
    runs give bit-identical gradients, which also match the oracle."""
    B, Hq, Hkv, N, w, s, theta = 1, 4, 2, 5000, 64, 5, 1e4
    q, k, v, dout = _inputs(B, Hq, Hkv, N, d, seed=21 + d, scale=0.8)
    r1 = _run(q, k, v, dout, w, s, mode, None, theta)
    r2 = _run(q, k, v, dout, w, s, mode, None, theta)
    for a, b in zip(r1[2:5], r2[2:5]):
        assert torch.equal(a, b)
    ref = oracle.backward(q, k, v, r1[5].cpu(), w=w, s=s, mode=mode, rope_theta=theta)
    for name, got, r in (("dq", r1[2], ref[0]), ("dk", r1[3], ref[1]), ("dv", r1[4], ref[2])):
        assert_parity(got, r, "bf16", name)


def test_backward_swat340m_layer_one_sequence():
    """The SWAT-340M layer (B 8, H 16, N 4096, d 64, w 512, sigmoid + balanced ALiBi + RoPE)
    in the full launch; every gradient of sequence 0 against the oracle."""
    cfg = wl.C2
    q, k, v = wl.prefill_inputs(cfg, device="cpu")
    g = torch.Generator().manual_seed(99)
    dout = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    o, lse, dq, dk, dv, gd = _run(q, k, v, dout, cfg.w, cfg.s, cfg.mode, cfg.slopes, cfg.rope_theta)
    ref = oracle.backward(q[:1], k[:1], v[:1], gd[:1].cpu(), w=cfg.w, s=cfg.s, mode=cfg.mode,
                          slopes=cfg.slopes, rope_theta=cfg.rope_theta)
    for name, got, r in (("dq", dq[:1], ref[0]), ("dk", dk[:1], ref[1]), ("dv", dv[:1], ref[2])):
        assert_parity(got, r, "bf16", name)


def test_backward_long_window_softmax_gqa():
    """Softmax, d 128, four query heads per kv head, a 1024-token window over 4096 rows."""
    B, Hq, Hkv, N, d, w, s, theta = 1, 8, 2, 4096, 128, 1024, 0, 1e6
    q, k, v, dout = _inputs(B, Hq, Hkv, N, d, seed=13, scale=0.7)
    o, lse, dq, dk, dv, g = _run(q, k, v, dout, w, s, wl.SOFTMAX, None, theta)
    ref = oracle.backward(q, k, v, g.cpu(), w=w, s=s, mode=wl.SOFTMAX, rope_theta=theta)
    for name, got, r in (("dq", dq, ref[0]), ("dk", dk, ref[1]), ("dv", dv, ref[2])):
        assert_parity(got, r, "bf16", name)
