"""GPU parity of the NVFP4 QAD linear ("nvfp4_qad.py": nvfp4_gemm, _NVFP4STE, max calibration)
against the oracle, within the stated tolerance (tests/parity.py): forward with and without bias
under the unit and a static activation scale on shapes with ragged rows and several 256 x 256
tiles; the straight-through backward; the autograd path; the calibration's running maximum and the
layer helper; sampled rows of the Wan2.1 FFN shape (25088 tokens, 1536 -> 8960)."""
import numpy as np
import pytest
import torch

import oracle
from tests.parity import assert_close, bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def m():
    import quantization_aware_attention_nvfp4_amd as m
    return m


def rand(shape, seed, mult=1.0):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(*shape, generator=g) * mult).to(torch.bfloat16)


def vals(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("M,N,K", [(300, 320, 256), (77, 64, 64), (600, 640, 192)])
@pytest.mark.parametrize("static", [False, True])
def test_forward(m, M, N, K, static):
    x, w, b = rand((M, K), M + 1, 2.0), rand((N, K), N + 2, 0.05), rand((N,), K + 3)
    gx = 448.0 * 6.0 / 7.5 if static else 1.0
    sf = torch.tensor(gx, dtype=torch.float32, device="cuda") if static else None
    y = m.qad_linear_fwd(x.cuda(), w.cuda(), b.cuda(), sf)
    y0 = m.qad_linear_fwd(x.cuda(), w.cuda(), None, sf)
    torch.cuda.synchronize()
    gx32 = float(np.float32(gx))
    assert_close(vals(y), oracle.linear_fwd(bits(x), bits(w), bits(b), gx=gx32), f"y {M}x{N}x{K}")
    assert_close(vals(y0), oracle.linear_fwd(bits(x), bits(w), None, gx=gx32), f"y no bias {M}x{N}x{K}")


def test_backward(m):
    M, N, K = 300, 192, 128
    x, w, g = rand((M, K), 11), rand((N, K), 12, 0.1), rand((M, N), 13)
    gx, gw, gb = m.qad_linear_bwd(g.cuda(), x.cuda(), w.cuda())
    torch.cuda.synchronize()
    r = oracle.linear_bwd(bits(g), bits(x), bits(w))
    assert_close(vals(gx), r["gx"], "grad_x")
    assert_close(vals(gw), r["gw"], "grad_w")
    assert_close(vals(gb), r["gb"], "grad_b")


def test_backward_partial_outputs(m):
    # The C entry point computes only the gradients it is given: grad_b alone takes the column-sum
    # pass without the transpose and matches the fused one bit for bit; grad_x alone and grad_w alone
    # match the full call.
    from quantization_aware_attention_nvfp4_amd._lib import load
    M, N, K = 333, 256, 192
    x, w, g = rand((M, K), 31).cuda(), rand((N, K), 32, 0.1).cuda(), rand((M, N), 33).cuda()
    gx, gw, gb = m.qad_linear_bwd(g, x, w)
    lib = load()
    ws = torch.empty(lib.qad_linear_workspace_size(1, M, N, K), dtype=torch.uint8, device="cuda")
    st = torch.cuda.current_stream().cuda_stream
    outs = {"gx": torch.zeros_like(gx), "gw": torch.zeros_like(gw), "gb": torch.zeros_like(gb)}
    for name in ("gb", "gx", "gw"):
        ptr = {k: (v.data_ptr() if k == name else None) for k, v in outs.items()}
        rc = lib.qad_linear_bwd(g.data_ptr(), x.data_ptr(), w.data_ptr(), ptr["gx"], ptr["gw"], ptr["gb"], M, N, K,
                                ws.data_ptr(), ws.numel(), st)
        assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(outs["gb"], gb) and torch.equal(outs["gx"], gx) and torch.equal(outs["gw"], gw)
    r = oracle.linear_bwd(bits(g.cpu()), bits(x.cpu()), bits(w.cpu()))
    assert_close(vals(outs["gb"]), r["gb"], "grad_b alone")


def test_autograd_matches_explicit_calls(m):
    M, N, K = 130, 128, 64
    x, w, b, g = rand((2, M // 2, K), 14), rand((N, K), 15, 0.1), rand((N,), 16), rand((2, M // 2, N), 17)
    xg, wg, bg = (t.cuda().requires_grad_() for t in (x, w, b))
    y = m.qad_linear(xg, wg, bg)
    y.backward(g.cuda())
    torch.cuda.synchronize()
    assert y.shape == (2, M // 2, N)
    assert torch.equal(y.detach(), m.qad_linear_fwd(x.cuda(), w.cuda(), b.cuda()))
    gx, gw, gb = m.qad_linear_bwd(g.cuda(), x.cuda(), w.cuda())
    assert torch.equal(xg.grad, gx) and torch.equal(wg.grad, gw) and torch.equal(bg.grad, gb)


def test_calibration_and_layer(m):
    x1, x2 = rand((100, 64), 18, 3.0), rand((50, 64), 19, 9.0)
    w = rand((64, 64), 20, 0.1)
    layer = m.QADLinear(w.cuda(), None, act_scale="static")
    layer.calibrating = True
    layer(x1.cuda())
    layer(x2.cuda())
    layer.finish_calibration()
    want = oracle.observe_amax(bits(x2), oracle.observe_amax(bits(x1)))
    assert layer.input_amax == want
    # the library's input_global_sf of the observed maximum is the oracle's static scale of the
    # calibration data (whose abs-max is that maximum), bit for bit
    gx = oracle.static_scale_bf16(np.concatenate([bits(x1).ravel(), bits(x2).ravel()]))
    got = layer.input_sf.cpu().numpy()
    assert got.view(np.uint32)[0] == np.float32(gx).view(np.uint32), (got[0], gx)
    y = layer(x1.cuda())
    torch.cuda.synchronize()
    assert_close(vals(y), oracle.linear_fwd(bits(x1), bits(w), None, gx=gx), "static layer")


def test_input_global_sf_matches_oracle(m):
    # every observed maximum the calibration can hold (bf16 magnitudes from 2^-133 to 2^127, and 0)
    # against the oracle's static-scale arithmetic on a tensor with that abs-max
    mags = np.arange(0, 0x7F80, 97, dtype=np.uint16)
    amax = torch.from_numpy(oracle.bf16_bits_to_f32(mags).copy()).cuda()
    got = torch.stack([m.input_global_sf(amax[i:i + 1]) for i in range(amax.numel())]).cpu().numpy().ravel()
    want = np.array([oracle.static_scale_bf16(np.array([mg, 0x8000 | mg], np.uint16)) for mg in mags], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_wan_ffn_sampled_rows(m):
    M, N, K = 25088, 8960, 1536
    x, w, b = rand((M, K), 21), rand((N, K), 22, 0.03), rand((N,), 23)
    y = m.qad_linear_fwd(x.cuda(), w.cuda(), b.cuda())
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(24).choice(M, 24, replace=False))
    rows[-1] = M - 1
    ref = oracle.linear_fwd(bits(x[torch.as_tensor(rows)]), bits(w), bits(b))
    assert_close(vals(y[torch.as_tensor(rows)]), ref, "ffn rows")


def test_wan_ffn_backward_sampled(m):
    # The straight-through backward at the full FFN shape, in the launch configuration the benchmark
    # times: sampled rows of grad_x, sampled rows of grad_w and the matching grad_b entries, each
    # from an oracle call on the sub-problem that defines exactly those outputs.
    import synth
    x, w, b, g = synth.wan_ffn()
    M, N = g.shape
    gx, gw, gb = m.qad_linear_bwd(g.cuda(), x.cuda(), w.cuda())
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(25).choice(M, 24, replace=False))
    rows[-1] = M - 1
    r = oracle.linear_bwd(bits(g[torch.as_tensor(rows)]), bits(x[torch.as_tensor(rows)]), bits(w))
    assert_close(vals(gx[torch.as_tensor(rows)]), r["gx"], "ffn grad_x rows")
    cols = np.sort(np.random.default_rng(26).choice(N, 16, replace=False))
    cols[-1] = N - 1
    ci = torch.as_tensor(cols)
    r = oracle.linear_bwd(bits(g[:, ci].contiguous()), bits(x), bits(w[ci].contiguous()))
    assert_close(vals(gw[ci]), r["gw"], "ffn grad_w rows")
    assert_close(vals(gb[ci]), r["gb"], "ffn grad_b entries")
