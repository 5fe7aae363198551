"""The decoder block's fused kernels (csrc/layer_ops.hip) against plain PyTorch
fp32 of the same operations, on the device: outputs rounded to bf16 may differ
from the rounded reference by one bf16 step (2^-8 relative), fp32 outputs by
fp32 summation order."""
import pytest
import torch

import paged_sparse_attention_amd as P

pytestmark = pytest.mark.gpu

BF16_STEP = 2.0 ** -8


def _gen(seed):
    return torch.Generator(device="cuda").manual_seed(seed)


def _close_bf16(got, ref):
    ref32 = ref.float()
    err = (got.float() - ref32).abs()
    assert bool((err <= BF16_STEP * ref32.abs() + 1e-6).all()), float((err / (ref32.abs() + 1e-6)).max())


@pytest.mark.parametrize("rows,hidden", [(5, 256), (37, 3584), (3, 8192)])
def test_rmsnorm_forward_and_backward(rows, hidden):
    g = _gen(rows)
    x = torch.randn(rows, hidden, device="cuda", generator=g) * 2.0
    gain = (1.0 + 0.1 * torch.randn(hidden, device="cuda", generator=g)).to(torch.bfloat16)
    dh = torch.randn(rows, hidden, device="cuda", generator=g).to(torch.bfloat16)
    dres = torch.randn(rows, hidden, device="cuda", generator=g)
    eps = 1e-6
    h = torch.empty(rows, hidden, dtype=torch.bfloat16, device="cuda")
    rstd = torch.empty(rows, device="cuda")
    P.oomb_rmsnorm_fwd(x, gain, eps, h, rstd)
    xr = x.clone().requires_grad_(True)
    gr = gain.float().clone().requires_grad_(True)
    ref = xr * torch.rsqrt(xr.pow(2).mean(-1, keepdim=True) + eps) * gr
    _close_bf16(h, ref.detach())
    assert torch.allclose(rstd, torch.rsqrt(x.pow(2).mean(-1) + eps), rtol=1e-5)
    ref.backward(dh.float())
    dx = torch.empty_like(x)
    P.oomb_rmsnorm_bwd(x, gain, rstd, dh, dres, dx)
    assert torch.allclose(dx, xr.grad + dres, rtol=1e-4, atol=1e-5)
    P.oomb_rmsnorm_bwd(x, gain, rstd, dh, None, dx)
    assert torch.allclose(dx, xr.grad, rtol=1e-4, atol=1e-5)
    partial = torch.empty(min(4, rows), hidden, device="cuda")
    P.oomb_rmsnorm_gain_grad(x, rstd, dh, partial)
    assert torch.allclose(partial.sum(0), gr.grad, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_rotary_and_its_inverse(dtype):
    g = _gen(7)
    rows, heads, d, first = 48, 3, 128, 100
    half = d // 2
    inv = 1.0e6 ** (-torch.arange(half, dtype=torch.float64) * 2.0 / d)
    ang = torch.arange(first + rows, dtype=torch.float64)[:, None] * inv[None, :]
    cos, sin = torch.cos(ang).float().cuda(), torch.sin(ang).float().cuda()
    x = torch.randn(rows, heads, d, device="cuda", generator=g).to(dtype)
    out = torch.empty(rows, heads, d, dtype=torch.bfloat16, device="cuda")
    P.oomb_rotary(x, out, cos, sin, first)
    c, s = cos[first:, None, :], sin[first:, None, :]
    a, b = x.float()[..., :half], x.float()[..., half:]
    ref = torch.cat([a * c - b * s, b * c + a * s], -1)
    assert torch.allclose(out.float(), ref, rtol=BF16_STEP, atol=1e-2 * BF16_STEP)
    back = torch.empty_like(out)
    P.oomb_rotary(ref.contiguous(), back, cos, sin, first, inverse=True)
    assert torch.allclose(back.float(), x.float(), rtol=BF16_STEP, atol=1e-2 * BF16_STEP)


def test_swiglu_forward_and_backward():
    g = _gen(9)
    n = 4096 * 3
    gate = (torch.randn(n, device="cuda", generator=g) * 3.0).to(torch.bfloat16)
    up = torch.randn(n, device="cuda", generator=g).to(torch.bfloat16)
    dout = torch.randn(n, device="cuda", generator=g).to(torch.bfloat16)
    out = torch.empty_like(gate)
    P.oomb_swiglu_fwd(gate, up, out)
    gr, ur = gate.float().requires_grad_(True), up.float().requires_grad_(True)
    ref = torch.nn.functional.silu(gr) * ur
    _close_bf16(out, ref.detach())
    ref.backward(dout.float())
    dg, du = torch.empty_like(gate), torch.empty_like(up)
    P.oomb_swiglu_bwd(gate, up, dout, dg, du)
    _close_bf16(dg, gr.grad)
    _close_bf16(du, ur.grad)
