"""The multi-head attention layer (QKV projection -> fused attention ->
output projection) against an fp64 reference built from the same weights:
numpy projections around the oracle's attention forward and backward.

The layer rounds three intermediates to the half type (qkv, the attention
output, the result) and its GEMMs accumulate in fp32, so the reference
(fp64 throughout) differs by a few half-type roundings carried through the
projections.  Tolerance: max-abs <= 2e-2 * max|reference| for the output and
5e-2 * max|reference| for every gradient, the attention gradients' own
bound.
"""

import sys

import numpy as np
import pytest
import torch

import io_aware_exact_02_amd as fa
from oracle import attention as oa

Y_TOL = 2e-2
G_TOL = 5e-2


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def test_module_argument_checks():
    with pytest.raises(fa.FaArgError):
        fa.FlashMHA(100, 3)
    with pytest.raises(fa.FaArgError):
        fa.FlashMHA(96, 3)          # head_dim 32
    m = fa.FlashMHA(256, 4)
    assert (m.head_dim, m.Wqkv.out_features, m.out_proj.in_features) == (64, 768, 256)
    with pytest.raises(fa.FaArgError):
        m(torch.zeros(1, 8, 128))


def _layer_reference(x, Wqkv, bqkv, Wo, bo, H, causal, dy):
    """fp64 forward and backward of y = out_proj(attn(x Wqkv^T + bqkv))."""
    B, N, E = x.shape
    D = E // H
    qkv = (x @ Wqkv.T + bqkv).reshape(B, N, 3, H, D)
    q, k, v = qkv[:, :, 0], qkv[:, :, 1], qkv[:, :, 2]
    O, _ = oa.attention_forward(q, k, v, causal=causal)
    o = O.reshape(B, N, E)
    y = o @ Wo.T + bo
    # Backward: out_proj, then the oracle's attention backward, then Wqkv.
    do = (dy @ Wo).reshape(B, N, H, D)
    dWo = np.einsum("bni,bnj->ij", dy, o)
    dbo = dy.sum(axis=(0, 1))
    dq, dk, dv = oa.attention_backward(q, k, v, do, causal=causal)
    dqkv = np.stack([dq, dk, dv], axis=2).reshape(B, N, 3 * E)
    dx = dqkv @ Wqkv
    dWqkv = np.einsum("bni,bnj->ij", dqkv, x)
    dbqkv = dqkv.sum(axis=(0, 1))
    return y, {"x": dx, "Wqkv": dWqkv, "bqkv": dbqkv, "Wo": dWo, "bo": dbo}


def _rel_err(got, ref):
    mag = np.max(np.abs(ref))
    return np.max(np.abs(got - ref)) / mag


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("E,H,N", [(768, 12, 200), (1024, 8, 333)])
def test_module_matches_reference(E, H, N, causal, dtype):
    B = 2
    dt = {"bf16": torch.bfloat16, "f16": torch.float16}[dtype]
    _say(f"case FlashMHA E={E} H={H} N={N} causal={causal} {dtype}")
    torch.manual_seed(7000 + E + N)
    m = fa.FlashMHA(E, H, causal=causal, dtype=dt)          # random init on the CPU
    gen = torch.Generator("cpu").manual_seed(7100 + N)
    x = torch.randn((B, N, E), generator=gen).to(dt)
    dy = torch.randn((B, N, E), generator=gen).to(dt)
    f64 = lambda t: t.detach().to(torch.float64).numpy()
    ref_y, ref_g = _layer_reference(f64(x), f64(m.Wqkv.weight), f64(m.Wqkv.bias),
                                    f64(m.out_proj.weight), f64(m.out_proj.bias), H, causal, f64(dy))

    m = m.to("cuda")
    xg = x.to("cuda").requires_grad_(True)
    y = m(xg)
    y.backward(dy.to("cuda"))
    torch.cuda.synchronize()
    got = {"x": xg.grad, "Wqkv": m.Wqkv.weight.grad, "bqkv": m.Wqkv.bias.grad,
           "Wo": m.out_proj.weight.grad, "bo": m.out_proj.bias.grad}
    ey = _rel_err(f64(y.cpu()), ref_y)
    assert np.all(np.isfinite(f64(y.cpu())))
    assert ey <= Y_TOL, f"y rel max-abs {ey:.3e}"
    for name, ref in ref_g.items():
        g = f64(got[name].cpu())
        assert np.all(np.isfinite(g)), name
        e = _rel_err(g, ref)
        assert e <= G_TOL, f"d{name} rel max-abs {e:.3e}"


@pytest.mark.parametrize("causal", [False, True])
def test_layer_reference_against_autograd(causal):
    """The reference's chain of gradients (projections around the oracle's
    attention backward) equals torch autograd of the same layer written with
    plain fp64 ops on a small case."""
    B, N, E, H = 2, 9, 128, 2
    D = E // H
    g = torch.Generator("cpu").manual_seed(71)
    x, dy = torch.randn(B, N, E, generator=g, dtype=torch.float64), torch.randn(
        B, N, E, generator=g, dtype=torch.float64)
    Wqkv = torch.randn(3 * E, E, generator=g, dtype=torch.float64) / E ** 0.5
    bqkv = torch.randn(3 * E, generator=g, dtype=torch.float64)
    Wo = torch.randn(E, E, generator=g, dtype=torch.float64) / E ** 0.5
    bo = torch.randn(E, generator=g, dtype=torch.float64)
    params = [t.clone().requires_grad_(True) for t in (x, Wqkv, bqkv, Wo, bo)]
    px, pW, pb, pWo, pbo = params
    qkv = (px @ pW.T + pb).reshape(B, N, 3, H, D).permute(2, 0, 3, 1, 4)
    s = qkv[0] @ qkv[1].transpose(-1, -2) / D ** 0.5
    if causal:
        s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
    o = (torch.softmax(s, -1) @ qkv[2]).permute(0, 2, 1, 3).reshape(B, N, E)
    y = o @ pWo.T + pbo
    y.backward(dy)
    ref_y, ref_g = _layer_reference(x.numpy(), Wqkv.numpy(), bqkv.numpy(), Wo.numpy(),
                                    bo.numpy(), H, causal, dy.numpy())
    np.testing.assert_allclose(ref_y, y.detach().numpy(), rtol=0, atol=1e-12)
    for name, p in zip(("x", "Wqkv", "bqkv", "Wo", "bo"), params):
        np.testing.assert_allclose(ref_g[name], p.grad.numpy(), rtol=0, atol=1e-11, err_msg=name)
