"""GPU parity of the fake-quant training support: the straight-through backward (gradient
clamp), the moving-average tensor scale and the autograd wrapper around them, against the
CPU oracle bit for bit (fp32 bits; bf16 bits of the oracle value rounded to nearest-even)."""
import numpy as np
import pytest
import torch

from scale_search_weights_amd import nvfp4, ste, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
INF = float("inf")


def case(msg):
    print(f"[case] {msg}", flush=True)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def assert_same(gpu: torch.Tensor, ref: np.ndarray, orc):
    ref = np.asarray(ref, np.float32)
    if gpu.dtype == torch.bfloat16:
        got = gpu.cpu().view(torch.int16).numpy().view(np.uint16).ravel()
        want = orc.bf16_rne_array(ref).ravel()
    else:
        got = gpu.cpu().numpy().view(np.uint32).ravel()
        want = ref.view(np.uint32).ravel()
    nan = np.isnan(ref.ravel())
    assert np.array_equal(np.isnan(f32(gpu).ravel()), nan)
    bad = np.flatnonzero((got != want) & ~nan)
    assert bad.size == 0, f"{bad.size} mismatches, first at {bad[:3].tolist()}"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("clip", [INF, 1.0, 0.37, 1e-30])
def test_ste_backward(orc, dtype, clip):
    n = 3 * 65536 + 8 * 37                              # several grid strides + a ragged tail
    case(f"ste_backward n={n} {dtype} clip={clip}")
    rng = np.random.default_rng(5)
    g = (rng.standard_t(3, n) * 0.5).astype(np.float32)
    g[:12] = [0.0, -0.0, np.nan, np.inf, -np.inf, 1e-40, -1e-42, 3e38, -3e38, 1.0, -1.0, 0.37]
    gt = torch.from_numpy(g).to(dtype)
    out = nvfp4.ste_backward(gt.to(DEV), clip)
    assert out.dtype == dtype
    assert_same(out, orc.ste_backward(f32(gt), clip), orc)


def test_ste_backward_in_place_and_empty(orc):
    case("ste_backward in place, and n=0")
    g = torch.from_numpy((np.random.default_rng(6).standard_normal(4096) * 3).astype(np.float32))
    gd = g.to(DEV)
    nvfp4.ste_backward(gd, 2.0, out=gd)
    assert_same(gd, orc.ste_backward(g.numpy(), 2.0), orc)
    e = torch.empty(0, device=DEV)
    assert nvfp4.ste_backward(e, 1.0).numel() == 0


@pytest.mark.parametrize("batch", [1, 3, 1000])
@pytest.mark.parametrize("m", [0.0, 0.9, 0.99, 1.0])
def test_scale_ema(orc, batch, m):
    case(f"scale_ema batch={batch} m={m}")
    rng = np.random.default_rng(batch)
    prev = rng.uniform(1e-5, 1e-1, batch).astype(np.float32)
    cur = (prev * rng.uniform(0.5, 2.0, batch)).astype(np.float32)
    S = torch.from_numpy(prev).to(DEV)
    nvfp4.scale_ema(S, torch.from_numpy(cur).to(DEV), m)
    assert np.array_equal(S.cpu().numpy().view(np.uint32),
                          orc.scale_ema(prev, cur, m).view(np.uint32))


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_autograd_forward_backward(orc, dtype):
    case(f"FakeQuantSTE forward/backward 96x512 {dtype}")
    x = synth.activation(11, 96, 512).to(dtype)
    xn = f32(x)
    S = orc.tensor_scale(xn)
    xd = x.to(DEV).requires_grad_(True)
    Sd = torch.tensor([S], device=DEV)
    y = ste.fake_quant_ste(xd, Sd, None, 0.25)
    dq, _, _ = orc.fakequant(xn, S)
    assert_same(y.detach(), dq, orc)
    gy = synth.activation(12, 96, 512).to(dtype)
    y.backward(gy.to(DEV))
    assert xd.grad.dtype == dtype
    assert_same(xd.grad, orc.ste_backward(f32(gy), 0.25), orc)


def test_autograd_mse_scales_and_plain_ste(orc):
    case("FakeQuantSTE with given MSE bytes, unclamped gradient")
    w = synth.projection(2, rows=64, cols=256, tokens=16)[0]
    wn = f32(w)
    S = orc.tensor_scale(wn)
    wd = w.to(DEV).requires_grad_(True)
    Sd = torch.tensor([S], device=DEV)
    sc = nvfp4.scale_search_mse(wd.detach(), Sd)
    y = ste.fake_quant_ste(wd, Sd, sc)
    (y.float() * 3.0).sum().backward()
    dq, _, _ = orc.fakequant(wn, S, orc.scales_mse(wn, S))
    assert_same(y.detach(), dq, orc)
    assert_same(wd.grad, np.full(wn.shape, 3.0, np.float32), orc)


def test_module_running_scale(orc):
    case("NVFP4FakeQuant: three training batches, then eval")
    mod = ste.NVFP4FakeQuant(momentum=0.9, clip=4.0).to(DEV)
    xs = [synth.activation(20 + i, 64, 1024) * (1.0 + i) for i in range(3)]
    S_ref = None
    for x in xs:
        xn = f32(x)
        sb = np.float32(orc.tensor_scale(xn))
        S_ref = np.array([sb], np.float32) if S_ref is None else orc.scale_ema(S_ref, sb, 0.9)
        xd = x.to(DEV).requires_grad_(True)
        y = mod(xd)
        assert mod.scale.cpu().numpy().view(np.uint32)[0] == S_ref.view(np.uint32)[0]
        assert_same(y.detach(), orc.fakequant(xn, S_ref[0])[0], orc)
        gy = torch.full_like(xd, 5.0)
        y.backward(gy)
        assert_same(xd.grad, np.full(xn.shape, 4.0, np.float32), orc)
    mod.eval()
    x = xs[0]
    y = mod(x.to(DEV))
    assert mod.scale.cpu().numpy().view(np.uint32)[0] == S_ref.view(np.uint32)[0]
    assert_same(y, orc.fakequant(f32(x), S_ref[0])[0], orc)


def test_module_mse_selector(orc):
    case("NVFP4FakeQuant with the MSE selector, eval mode on a fixed scale")
    mod = ste.NVFP4FakeQuant(selector="mse").to(DEV)
    w = synth.projection(3, rows=32, cols=256, tokens=16)[0]
    wn = f32(w)
    S = orc.tensor_scale(wn)
    mod.scale.fill_(float(S))
    mod.initialised.fill_(True)
    mod.eval()
    y = mod(w.to(DEV))
    assert mod.scale.item() == S
    assert_same(y, orc.fakequant(wn, S, orc.scales_mse(wn, S))[0], orc)
