"""Pins for the oracle's NVFP4 QAD linear ("nvfp4_qad.py": nvfp4_gemm, _NVFP4STE, the
calibrating path of NVFP4QADLinearMethod.apply), CPU only.

  * the forward equals float64 torch.nn.functional.linear on operands quantized by the pinned
    standalone fake quantization (the weight under the pinned static scale of the weight, the
    activation under the unit or a given static scale) plus the bias;
  * with a weight whose blocks are exact NVFP4 values and a unit activation scale on exact NVFP4
    activations, the quantizers change nothing and the forward is the plain linear;
  * the backward equals float64 autograd of the plain linear on the unquantized operands (the
    straight-through estimator's full-precision gradients);
  * calibration folds the running maximum of |x| exactly.
"""
import numpy as np
import torch

import oracle


def bits(t):
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def f64(u16):
    return torch.from_numpy(oracle.bf16_bits_to_f32(u16).astype(np.float64))


def rand(shape, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    return bits(torch.randn(*shape, generator=g) * mult)


def test_forward_composes_the_standalone_fake_quant():
    M, N, K = 37, 29, 96
    x, w, b = rand((M, K), 1, 3.0), rand((N, K), 2, 0.05), rand((N,), 3)
    for gx in (1.0, 448.0 * 6.0 / 11.5):
        y = oracle.linear_fwd(x, w, b, gx=gx)
        xq = oracle.fq_bf16(x, -1, g=gx)
        wq = oracle.fq_bf16(w, -1, g=oracle.static_scale_bf16(w))
        ref = torch.nn.functional.linear(f64(xq), f64(wq), f64(b)).numpy()
        assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)
    y0 = oracle.linear_fwd(x, w, None)
    ref0 = torch.nn.functional.linear(f64(oracle.fq_bf16(x, -1)), f64(oracle.fq_bf16(w, -1, g=oracle.static_scale_bf16(w)))).numpy()
    assert np.allclose(y0, ref0, rtol=1e-12, atol=1e-12)


def test_exact_operands_pass_through():
    # Activations that are E2M1 values times 0.25 with 6 * 0.25 in every block: the unit-scale
    # block scale is then E4M3(1.5 / 6) = 0.25 exactly and every value is on the grid.  Weights are
    # E2M1 values times 0.125 with every block's maximum equal to the tensor's: g_w = 2688 / 0.75,
    # each block's s = E4M3(0.125 * g_w) = 448 and S = 448 / g_w = 0.125, again exact.
    g = torch.Generator().manual_seed(4)
    grid = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    M, N, K = 8, 6, 32

    def exact(rows):
        v = grid[torch.randint(0, 8, (rows, K), generator=g)] * torch.where(
            torch.rand(rows, K, generator=g) < 0.5, -1.0, 1.0)
        v[:, ::16] = 6.0  # every block holds its scale's maximum
        return v

    x = exact(M) * 0.25
    w = exact(N) * 0.125
    y = oracle.linear_fwd(bits(x), bits(w), None)
    ref = (x.double() @ w.double().T).numpy()
    assert np.array_equal(y, ref)


def test_backward_is_full_precision_autograd():
    M, N, K = 23, 19, 48
    x, w, g = rand((M, K), 5), rand((N, K), 6), rand((M, N), 7)
    r = oracle.linear_bwd(g, x, w)
    X, W, B = f64(x).requires_grad_(), f64(w).requires_grad_(), torch.zeros(N, dtype=torch.float64, requires_grad=True)
    torch.nn.functional.linear(X, W, B).backward(f64(g))
    assert np.allclose(r["gx"], X.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(r["gw"], W.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(r["gb"], B.grad.numpy(), rtol=1e-12, atol=1e-12)


def test_calibration_is_a_running_max():
    a, b = rand((50, 16), 8, 2.0), rand((70, 16), 9, 5.0)
    m1 = oracle.observe_amax(a)
    assert m1 == np.abs(oracle.bf16_bits_to_f32(a)).max()
    m2 = oracle.observe_amax(b, m1)
    assert m2 == max(m1, np.abs(oracle.bf16_bits_to_f32(b)).max())
    assert oracle.observe_amax(a, 1e9) == np.float32(1e9)
