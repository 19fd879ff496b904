"""GPU parity of the standalone rotation (swa_rope_apply) and ring append (swa_kv_append) on
both of their code paths.

Head sizes that are a multiple of 8 with 16-byte aligned tensors take 16-byte vector
kernels; other head sizes and misaligned tensors take the per-pair kernels. Each case is
checked against the oracle (the rotation in float64, the ring from the oracle append), and
the two paths against each other bit for bit on the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
import sliding_window_attention_prefill_amd as swa

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _misaligned(t):
    """The same values at a data pointer 4 bytes past a 16-byte boundary."""
    flat = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
    off = 4 // t.element_size()
    out = flat[off:off + t.numel()].view(t.shape)
    out.copy_(t)
    assert out.data_ptr() % 16 != 0
    return out


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d", [10, 64, 128])
def test_rope_apply_paths_match_oracle(dtype, d):
    from oracle import dense
    B, N, H = 2, 257, 3
    theta = 1e4
    x = torch.randn((B, N, H, d), generator=torch.Generator().manual_seed(d)).to(dtype)
    p0s = [5, 900]
    pos0 = torch.tensor(p0s, dtype=torch.int32, device=DEV)
    table = swa.swa_rope_table(1200, d, theta)
    fast = swa.swa_rope_apply(x.to(DEV), pos0, table)
    slow = swa.swa_rope_apply(_misaligned(x.to(DEV)), pos0, table)
    torch.cuda.synchronize()
    assert torch.equal(fast.cpu(), slow.cpu())
    xx = x.double().numpy()
    tol = dict(atol=2e-5, rtol=1e-5) if dtype == torch.float32 else dict(atol=1e-2, rtol=8e-3)
    for b, p0 in enumerate(p0s):
        full = np.zeros((1, p0 + N, H, d))
        full[0, p0:] = xx[b]
        ref = dense.rope_dense(full, theta)[0, p0:]
        np.testing.assert_allclose(fast[b].cpu().double().numpy(), ref, **tol)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("d,w,s,n_new", [(64, 16, 3, 40), (128, 64, 4, 5), (10, 8, 2, 11)])
def test_kv_append_paths_match_oracle(dtype, d, w, s, n_new):
    S, Hkv, theta = 3, 2, 1e4
    g = torch.Generator().manual_seed(d + w + n_new)
    k = torch.randn((S, n_new, Hkv, d), generator=g).to(dtype)
    v = torch.randn((S, n_new, Hkv, d), generator=g).to(dtype)
    p0s = [0, 7, 100]
    pos0 = torch.tensor(p0s, dtype=torch.int32, device=DEV)
    table = swa.swa_rope_table(200, d, theta)

    def fresh():
        z = lambda *sh: torch.zeros(sh, dtype=dtype, device=DEV)
        return swa.SwaCache(z(S, Hkv, w, d), z(S, Hkv, w, d), z(S, Hkv, s, d), z(S, Hkv, s, d))

    a, b = fresh(), fresh()
    swa.swa_kv_append(a, k.to(DEV), v.to(DEV), pos0, rope_table=table)
    swa.swa_kv_append(b, _misaligned(k.to(DEV)), _misaligned(v.to(DEV)), pos0, rope_table=table)
    torch.cuda.synchronize()
    for x, y in ((a.k_ring, b.k_ring), (a.v_ring, b.v_ring), (a.k_sink, b.k_sink),
                 (a.v_sink, b.v_sink)):
        assert torch.equal(x.cpu(), y.cpu())
    ring = oracle.Ring(S, Hkv, w, s, d)
    ring.append(k, v, np.array(p0s), rope_theta=theta)
    tol = dict(atol=2e-5, rtol=1e-5) if dtype == torch.float32 else dict(atol=1e-2, rtol=8e-3)
    np.testing.assert_allclose(a.k_ring.cpu().double().numpy(), ring.k, **tol)
    np.testing.assert_allclose(a.v_ring.cpu().double().numpy(), ring.v, **tol)
    np.testing.assert_allclose(a.k_sink.cpu().double().numpy(), ring.k_sink[:, :, :s], **tol)
    np.testing.assert_allclose(a.v_sink.cpu().double().numpy(), ring.v_sink[:, :, :s], **tol)
