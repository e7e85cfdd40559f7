"""GPU parity: every entry point through the C ABI against the CPU oracle on seeded
inputs, at sizes the oracle finishes in seconds (several tiles and ragged tails).

Bar: bit-exact for block bytes, packed codes, dequantised values (fp32 bits; bf16 bits of
the oracle value rounded to nearest-even), MSE objectives, routing lists and the
Local-Hessian bytes and fp64 objectives; block Hessians within 1e-4 relative Frobenius
error per block (fp32 accumulation against the oracle's fp64 sums).
"""
import json
import os

import numpy as np
import pytest
import torch

from scale_search_weights_amd import nvfp4, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def case(msg):
    print(f"[case] {msg}", flush=True)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def dev_S(*vals):
    return torch.tensor(np.array(vals, np.float32), device=DEV)


def assert_bits(gpu_y: torch.Tensor, dq_ref: np.ndarray, orc):
    if gpu_y.dtype == torch.bfloat16:
        got = gpu_y.cpu().view(torch.int16).numpy().view(np.uint16)
        want = orc.bf16_rne_array(dq_ref)
    else:
        got = gpu_y.cpu().numpy().view(np.uint32)
        want = dq_ref.view(np.uint32)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[:3].tolist()}"


def rel_frob(Hg: np.ndarray, Href: np.ndarray) -> float:
    Hg = Hg.reshape(-1, 256).astype(np.float64)
    Hr = Href.reshape(-1, 256)
    num = np.linalg.norm(Hg - Hr, axis=1)
    den = np.linalg.norm(Hr, axis=1)
    r = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    return float(r.max())


@pytest.fixture(scope="module")
def tiny():
    w, x = synth.tiny(0)
    return w, x


# ------------------------------------------------------------------ tensor scale

def test_global_scale(orc, tiny):
    w, _ = tiny
    case("global_scale tiny fp32")
    assert nvfp4.global_scale(w.to(DEV)).item() == orc.tensor_scale(w.numpy())
    case("global_scale activation bf16 256x4096")
    a = synth.activation(1, 256, 4096)
    assert nvfp4.global_scale(a.to(DEV)).item() == orc.tensor_scale(f32(a))
    case("global_scale zero tensor -> 1")
    assert nvfp4.global_scale(torch.zeros(8, 32, device=DEV)).item() == 1.0
    case("global_scale batch of 5 experts")
    e = synth.moe(2, experts=5, rows=64, cols=128, tokens=16, topk=2)[0]
    e[3] *= 0
    S = nvfp4.global_scale(e.to(DEV)).cpu().numpy()
    for b in range(5):
        assert S[b] == orc.tensor_scale(f32(e[b])), b


def test_global_scale_workspace_form(orc, tiny):
    """The workspace form against the oracle, one workspace reused across calls of
    different sizes and first filled with 0xFF (its contents must not matter): 1024
    workgroups, a ragged last round, a batch of experts with an all-zero entry, and the
    maximum in the very last vector of the tensor."""
    ws = torch.full((1 << 20,), 0xFF, dtype=torch.uint8, device=DEV)
    w, _ = tiny
    case("global_scale_ws tiny fp32")
    assert nvfp4.global_scale(w.to(DEV), workspace=ws).item() == orc.tensor_scale(w.numpy())
    for rows, cols, seed in ((8192, 4096, 1), (1000, 1040, 2), (4096, 4096, 3), (3, 16, 4)):
        case(f"global_scale_ws activation bf16 {rows}x{cols}")
        a = synth.activation(seed, rows, cols)
        if seed == 3:
            a[-1, -1] = 1e4  # the largest value in the last vector
        assert nvfp4.global_scale_workspace_size(1, rows * cols) <= ws.numel()
        assert nvfp4.global_scale(a.to(DEV), workspace=ws).item() == orc.tensor_scale(f32(a))
    case("global_scale_ws batch of 7 experts, one all-zero")
    e = synth.moe(3, experts=7, rows=512, cols=256, tokens=16, topk=2)[0]
    e[5] *= 0
    S = nvfp4.global_scale(e.to(DEV), workspace=ws).cpu().numpy()
    for b in range(7):
        assert S[b] == orc.tensor_scale(f32(e[b])), b


# ------------------------------------------------------------------ max scaling / fake-quant

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(64, 256), (333, 1024), (8, 16)])
def test_fakequant_max_scaling(orc, dtype, shape):
    case(f"fakequant max {shape} {dtype}")
    x = synth.activation(3, *shape).to(dtype)
    xn = f32(x)
    S = orc.tensor_scale(xn)
    y, codes, scales = nvfp4.fakequant(x.to(DEV), dev_S(S), return_codes=True)
    dq, codes_ref, sc_ref = orc.fakequant(xn, S)
    assert np.array_equal(scales.cpu().numpy(), sc_ref)
    assert np.array_equal(codes.cpu().numpy(), codes_ref)
    assert_bits(y, dq, orc)
    # the separate entry points agree with the fused one
    assert np.array_equal(nvfp4.scale_search_max(x.to(DEV), dev_S(S)).cpu().numpy(), sc_ref)
    c2, s2 = nvfp4.quantize(x.to(DEV), dev_S(S))
    assert np.array_equal(c2.cpu().numpy(), codes_ref) and np.array_equal(s2.cpu().numpy(), sc_ref)
    y2 = nvfp4.dequantize(c2, s2, dev_S(S), out_dtype=dtype)
    assert_bits(y2, dq, orc)


def test_fakequant_batched_per_entry_scale(orc):
    case("fakequant batch 3 x 40 x 256 bf16, per-entry S")
    x = synth.moe(4, experts=3, rows=40, cols=256, tokens=8, topk=1)[0]
    x[1] *= 1000.0
    xd = x.to(DEV)
    S = nvfp4.global_scale(xd)
    y, codes, sc = nvfp4.fakequant(xd, S, return_codes=True)
    Sn = np.array([orc.tensor_scale(f32(x[b])) for b in range(3)], np.float32)
    assert np.array_equal(S.cpu().numpy(), Sn)
    for b in range(3):
        dq, cr, sr = orc.fakequant(f32(x[b]), Sn[b])
        assert np.array_equal(sc[b].cpu().numpy(), sr)
        assert np.array_equal(codes[b].cpu().numpy(), cr)
        assert_bits(y[b], dq, orc)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_quantize_with_given_scales_all_bytes(orc, dtype):
    case(f"quantize with every byte 1..126, {dtype}")
    rng = np.random.default_rng(5)
    rows, cols = 126, 64
    S = np.float32(3.0e-3)
    sc = np.repeat(np.arange(1, 127, dtype=np.uint8)[:, None], cols // 16, axis=1)
    sval = np.array([orc.e4m3_value(b) for b in range(1, 127)], np.float64)[:, None]
    x = (rng.uniform(-7, 7, (rows, cols)) * sval * float(S)).astype(np.float32)
    xt = torch.from_numpy(x).to(dtype)
    xn = f32(xt)
    codes, _ = nvfp4.quantize(xt.to(DEV), dev_S(S), torch.from_numpy(sc).to(DEV))
    assert np.array_equal(codes.cpu().numpy(), orc.quantize(xn, S, sc))
    y = nvfp4.fakequant(xt.to(DEV), dev_S(S), torch.from_numpy(sc).to(DEV))
    dq, _, _ = orc.fakequant(xn, S, sc)
    assert_bits(y, dq, orc)


def test_given_bytes_outside_the_candidates(orc):
    """Every byte value as a given block scale: a byte acts as its E4M3FN magnitude (sign
    bit ignored), and 0x7F (NaN) codes its block as zeros like 0x00; quantise, fake-quant,
    dequantise and GPTQ agree with the oracle on all 256 values."""
    case("given block bytes 0x00..0xFF: quantize, fakequant, dequantize, gptq")
    rng = np.random.default_rng(11)
    rows, cols = 256, 64
    S = np.float32(3.0e-3)
    sc = np.repeat(np.arange(256, dtype=np.uint8)[:, None], cols // 16, axis=1)
    mag = np.array([orc.e4m3_value(b & 0x7F) if (b & 0x7F) not in (0, 0x7F) else 1.0
                    for b in range(256)], np.float64)[:, None]
    x = (rng.uniform(-7, 7, (rows, cols)) * mag * float(S)).astype(np.float32)
    x[0x80:] = x[:0x80]  # bytes b and b | 0x80 see the same values
    xd, Sd, scd = torch.from_numpy(x).to(DEV), dev_S(S), torch.from_numpy(sc).to(DEV)
    codes, _ = nvfp4.quantize(xd, Sd, scd)
    want = orc.quantize(x, S, sc)
    assert np.array_equal(codes.cpu().numpy(), want)
    # bytes b and b | 0x80 give the same codes; 0x00, 0x7F, 0x80 and 0xFF give zeros
    assert np.array_equal(want[0x01:0x7F], want[0x81:0xFF])
    assert not want[[0x00, 0x7F, 0x80, 0xFF]].any()
    y = nvfp4.fakequant(xd, Sd, scd)
    dq, _, _ = orc.fakequant(x, S, sc)
    assert_bits(y, dq, orc)
    yd = nvfp4.dequantize(torch.from_numpy(want).to(DEV), scd, Sd)
    assert_bits(yd, orc.dequantize(want, sc, S, rows, cols), orc)
    # GPTQ at the same bytes (U of a random well-conditioned H from the oracle)
    a = rng.standard_normal((4 * cols, cols))
    U = orc.gptq_factor(a.T @ a, 0.01)
    g = nvfp4.gptq(xd, Sd, scd, torch.from_numpy(U).to(DEV)).cpu().numpy()
    assert np.array_equal(g, orc.gptq(x, S, sc, U=U))


def test_exact_ties_and_edges(orc):
    case("ties on midpoints, zero blocks, -0, saturation, denormal inputs")
    blocks = []
    # element ties at unit scale: multiples of 1/16 in [-8, 8]; block max 8 -> byte for 8/6
    v = synth.on_grid_block_values(7, 64 * 16).reshape(64, 16)
    blocks.append(v)
    # all-zero and negative-zero blocks
    z = np.zeros((2, 16), np.float32)
    z[1] = -0.0
    blocks.append(z)
    # block max exactly on an E4M3 midpoint times 6 (S = 1): ties to the even byte
    mids = []
    for b in range(1, 126):
        m = (orc.e4m3_value(b) + orc.e4m3_value(b + 1)) / 2 * 6.0
        if np.float32(m) == m:
            row = np.full(16, np.float32(m) / 3, np.float32)
            row[0] = np.float32(m)
            mids.append(row)
    blocks.append(np.array(mids, np.float32))
    # denormal fp32 inputs next to normal ones
    d = np.full((1, 16), 1e-40, np.float32)
    d[0, 3] = 1.0
    blocks.append(d)
    x = np.concatenate(blocks, axis=0)
    S = np.float32(1.0)
    xt = torch.from_numpy(x)
    y, codes, sc = nvfp4.fakequant(xt.to(DEV), dev_S(S), return_codes=True)
    dq, cr, sr = orc.fakequant(x, S)
    assert np.array_equal(sc.cpu().numpy(), sr)
    assert np.array_equal(codes.cpu().numpy(), cr)
    assert_bits(y, dq, orc)
    # saturation: values far beyond 6 * 448 * S with a caller-supplied small S
    big = (np.random.default_rng(8).standard_normal((32, 32)) * 1e6).astype(np.float32)
    S2 = np.float32(1e-3)
    y, codes, sc = nvfp4.fakequant(torch.from_numpy(big).to(DEV), dev_S(S2), return_codes=True)
    dq, cr, sr = orc.fakequant(big, S2)
    assert np.all(sr == 0x7E)
    assert np.array_equal(codes.cpu().numpy(), cr)
    assert_bits(y, dq, orc)
    # tiny values with the smallest normal tensor scale (subnormal block scales)
    tiny_x = (np.random.default_rng(9).standard_normal((16, 64)) * 1e-36).astype(np.float32)
    S3 = orc.tensor_scale(tiny_x)
    y, codes, sc = nvfp4.fakequant(torch.from_numpy(tiny_x).to(DEV), dev_S(S3), return_codes=True)
    dq, cr, sr = orc.fakequant(tiny_x, S3)
    assert np.array_equal(sc.cpu().numpy(), sr)
    assert np.array_equal(codes.cpu().numpy(), cr)
    assert_bits(y, dq, orc)


@pytest.mark.parametrize("S", [1.0, 0.8123457, 3.0517578e-05])
def test_values_on_and_beside_every_midpoint(orc, S):
    """Given bytes, values exactly on every E2M1 midpoint / grid point (times s S, rounded to
    fp32) and one and two ulps either side: exercises the exact fallback of the fast path."""
    case(f"midpoint neighbourhoods, S={S}")
    S = np.float32(S)
    rng = np.random.default_rng(11)
    bytes_ = [0x01, 0x07, 0x08, 0x30, 0x38, 0x3B, 0x56, 0x6F, 0x7E]
    pts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0, 6.5]
    rows, scs = [], []
    for b in bytes_:
        sS = orc.e4m3_value(b) * float(S)
        vals = []
        for p in pts:
            c = np.float32(p * sS)
            for k in (-2, -1, 0, 1, 2):
                v = c
                for _ in range(abs(k)):
                    v = np.nextafter(v, np.float32(np.inf if k > 0 else 0))
                vals.append(v)
        vals = np.array(vals, np.float32)
        vals *= np.where(rng.random(vals.size) < 0.5, -1, 1).astype(np.float32)
        pad = (-vals.size) % 16
        vals = np.concatenate([vals, np.zeros(pad, np.float32)]).reshape(-1, 16)
        rows.append(vals)
        scs.append(np.full((vals.shape[0], 1), b, np.uint8))
    x = np.concatenate(rows)
    sc = np.concatenate(scs)
    xd = torch.from_numpy(x).to(DEV)
    y = nvfp4.fakequant(xd, dev_S(S), torch.from_numpy(sc).to(DEV))
    codes, _ = nvfp4.quantize(xd, dev_S(S), torch.from_numpy(sc).to(DEV))
    dq, cr, _ = orc.fakequant(x, S, sc)
    assert np.array_equal(codes.cpu().numpy(), cr)
    assert_bits(y, dq, orc)
    y2 = nvfp4.dequantize(codes, torch.from_numpy(sc).to(DEV), dev_S(S))
    assert_bits(y2, dq, orc)


def test_worked_example_on_gpu(orc):
    case("worked example block: 84 -> scale 14")
    with open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")) as f:
        g = json.load(f)
    x = torch.tensor([g["block"]], dtype=torch.float32, device=DEV)
    y, codes, sc = nvfp4.fakequant(x, dev_S(1.0), return_codes=True)
    assert orc.e4m3_value(int(sc.item())) == g["scale"]
    yn = y.cpu().numpy()[0]
    assert set(np.abs(yn).tolist()) <= set(g["magnitudes"]) and yn[0] == 84.0
    assert np.all(yn[np.abs(np.array(g["block"])) < g["zero_below"]] == 0)
    assert nvfp4.scale_search_mse(x, dev_S(1.0)).item() == 0x56


# ------------------------------------------------------------------ MSE search

@pytest.mark.parametrize("which", ["tiny_fp32", "mlp_bf16", "mlp_bf16_ragged"])
def test_mse_search(orc, tiny, which):
    if which == "tiny_fp32":
        w = tiny[0]
    elif which == "mlp_bf16":
        w = synth.mlp_weight(1, 256, 1024)
    else:
        w = synth.mlp_weight(2, 37, 48)
    case(f"mse {which} {tuple(w.shape)}")
    wn = f32(w)
    S = orc.tensor_scale(wn)
    sc, obj = nvfp4.scale_search_mse(w.to(DEV), dev_S(S), return_obj=True)
    sr, orf = orc.scales_mse(wn, S, with_obj=True)
    assert np.array_equal(sc.cpu().numpy(), sr)
    assert np.array_equal(obj.cpu().numpy().view(np.uint32), orf.view(np.uint32))


@pytest.mark.parametrize("S", [None, 1e-9, 1e-3, 1.0, 50.0])
def test_mse_pruning_edges(orc, S):
    """Blocks that put the window edges in odd places: everything saturating (tiny S),
    everything rounding to zero for most bytes (huge S), single non-zero values, constant
    blocks, on-grid blocks and exact ties."""
    case(f"mse pruning edges S={S}")
    rng = np.random.default_rng(21)
    blocks = [rng.standard_normal((64, 16)).astype(np.float32) * np.float32(0.02)]
    one = np.zeros((16, 16), np.float32)
    one[np.arange(16), np.arange(16)] = rng.uniform(0.001, 1.0, 16).astype(np.float32)
    blocks.append(one)
    blocks.append(np.repeat(rng.uniform(-1, 1, (16, 1)).astype(np.float32), 16, axis=1))
    blocks.append(synth.on_grid_block_values(3, 32 * 16).reshape(32, 16) * np.float32(0.125))
    with open(os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")) as f:
        blocks.append(np.array([json.load(f)["block"]], np.float32))
    x = np.concatenate(blocks).reshape(-1, 16)
    Sv = orc.tensor_scale(x) if S is None else np.float32(S)
    sc, obj = nvfp4.scale_search_mse(torch.from_numpy(x).to(DEV), dev_S(Sv), return_obj=True)
    sr, orf = orc.scales_mse(x, Sv, with_obj=True)
    assert np.array_equal(sc.cpu().numpy(), sr), np.argwhere(sc.cpu().numpy() != sr)[:5]
    assert np.array_equal(obj.cpu().numpy().view(np.uint32), orf.view(np.uint32))


def test_mse_optimum_far_above_max_byte(orc):
    """Blocks whose MSE byte lies 4 or more above the max-scaling byte (normal and Laplace
    values): the upward walk must reach them before its zero-term bound stops it."""
    case("mse: optimum at least 4 bytes above the max-scaling byte")
    rng = np.random.default_rng(77)
    pool = np.concatenate([rng.standard_normal((6000, 16)), rng.laplace(size=(6000, 16))])
    pool = pool.astype(np.float32)
    S = orc.tensor_scale(pool)
    up = orc.scales_mse(pool, S).astype(int).ravel() - orc.scales_max(pool, S).astype(int).ravel()
    x = np.ascontiguousarray(pool[up >= 4])
    assert len(x) >= 100, len(x)
    sc, obj = nvfp4.scale_search_mse(torch.from_numpy(x).to(DEV), dev_S(S), return_obj=True)
    sr, orf = orc.scales_mse(x, S, with_obj=True)
    assert np.array_equal(sc.cpu().numpy(), sr)
    assert np.array_equal(obj.cpu().numpy().view(np.uint32), orf.view(np.uint32))


def test_mse_batched_and_zero_blocks(orc):
    case("mse batch 4 x 32 x 128 with zero blocks")
    w = synth.moe(3, experts=4, rows=32, cols=128, tokens=8, topk=1)[0]
    w[2, 5, 16:32] = 0
    wd = w.to(DEV)
    S = nvfp4.global_scale(wd)
    sc, obj = nvfp4.scale_search_mse(wd, S, return_obj=True)
    Sn = np.array([orc.tensor_scale(f32(w[b])) for b in range(4)], np.float32)
    assert np.array_equal(S.cpu().numpy(), Sn)
    for b in range(4):
        sr, orf = orc.scales_mse(f32(w[b]), Sn[b], with_obj=True)
        assert np.array_equal(sc[b].cpu().numpy(), sr)
        assert np.array_equal(obj[b].cpu().numpy(), orf)
    assert sc[2, 5, 1].item() == 0


# ------------------------------------------------------------------ Four Over Six

def _fos_check(orc, w, S):
    x = w if isinstance(w, torch.Tensor) else torch.from_numpy(w)
    sc, obj = nvfp4.scale_search_four_over_six(x.to(DEV), dev_S(S), return_obj=True)
    sr, orf = orc.scales_four_over_six(f32(x), S, with_obj=True)
    g = sc.cpu().numpy()
    assert np.array_equal(g, sr), (np.sum(g != sr), np.argwhere(g != sr)[:5])
    assert np.array_equal(obj.cpu().numpy().view(np.uint32), orf.view(np.uint32))
    return g


@pytest.mark.parametrize("which", ["tiny_fp32", "ragged_bf16", "proj_bf16"])
def test_four_over_six(orc, tiny, which):
    case(f"four over six {which}")
    if which == "tiny_fp32":
        w = tiny[0]
    elif which == "ragged_bf16":
        w = synth.mlp_weight(4, 77, 272)           # 17 blocks per row, odd rows
    else:
        w = synth.projection(12, rows=96, cols=512, tokens=16)[0]
    S = orc.tensor_scale(f32(w))
    g = _fos_check(orc, w, S)
    # the choice is one of the two candidates and never worse than max scaling
    mx = orc.scales_max(f32(w), S)
    assert np.mean(g == mx) > 0.2 and np.mean(g != mx) > 0.05


@pytest.mark.parametrize("S", [None, 1.0, 2.0 ** -20, 1e30])
def test_four_over_six_edges(orc, S):
    """Lone exact values 24*2^j (tie: both candidates exact), blocks on the k = 4 grid,
    constant and zero blocks, denormal inputs, midpoint values, and S that saturates every
    byte (tiny S) or pushes the scales to subnormal E4M3 (huge S)."""
    case(f"four over six edges S={S}")
    rng = np.random.default_rng(31)
    blocks = [rng.standard_normal((64, 16)).astype(np.float32) * np.float32(0.02)]
    lone = np.zeros((6, 16), np.float32)
    for i, j in enumerate((-6, -3, 0, 1, 2, 4)):
        lone[i, (5 * i) % 16] = np.float32(24.0 * 2.0 ** j) * (1 if i % 2 else -1)
    blocks.append(lone)
    g4 = np.array([4, -3, 2, 1.5, -1, 0.5, 0, 3, -4, 2, 1, -0.5, 1.5, 0, 4, -2], np.float32)
    blocks.append(np.stack([g4 * np.float32(2.0 ** k) for k in range(-8, 8)]))
    blocks.append(np.repeat(rng.uniform(-1, 1, (8, 1)).astype(np.float32), 16, axis=1))
    blocks.append(np.zeros((2, 16), np.float32))
    blocks.append((rng.standard_normal((4, 16)) * 1e-39).astype(np.float32))  # denormals
    blocks.append(synth.on_grid_block_values(5, 16 * 16).reshape(16, 16) * np.float32(0.375))
    x = np.concatenate(blocks).reshape(-1, 16)
    Sv = orc.tensor_scale(x) if S is None else np.float32(S)
    _fos_check(orc, x, Sv)


def test_four_over_six_batched(orc):
    case("four over six batch of 3 experts with per-entry S and a zero block")
    w = synth.moe(13, experts=3, rows=24, cols=96, tokens=8, topk=1)[0]
    w[1, 4, 32:48] = 0
    wd = w.to(DEV)
    S = nvfp4.global_scale(wd)
    sc, obj = nvfp4.scale_search_four_over_six(wd, S, return_obj=True)
    Sn = np.array([orc.tensor_scale(f32(w[b])) for b in range(3)], np.float32)
    assert np.array_equal(S.cpu().numpy(), Sn)
    for b in range(3):
        sr, orf = orc.scales_four_over_six(f32(w[b]), Sn[b], with_obj=True)
        assert np.array_equal(sc[b].cpu().numpy(), sr)
        assert np.array_equal(obj[b].cpu().numpy().view(np.uint32), orf.view(np.uint32))
    assert sc[1, 4, 2].item() == 0


# ------------------------------------------------------------------ calibration

@pytest.mark.parametrize("which", ["act_bf16", "fp32", "ragged_bf16", "tiny", "zeros_denormals"])
def test_calib_histogram_and_scale(orc, which):
    case(f"calibration histogram and scale: {which}")
    rng = np.random.default_rng(41)
    if which == "act_bf16":
        x = synth.activation(3, tokens=300, hidden=512)                   # 153,600 values
    elif which == "fp32":
        x = torch.from_numpy((rng.standard_t(3, 70_000) * 2).astype(np.float32))
    elif which == "ragged_bf16":
        x = synth.activation(4, tokens=3, hidden=32768 + 8)               # chunks + a tail
    elif which == "tiny":
        x = torch.tensor([0.5, -1.5, 3.0, 0.0, -0.0, 2.0, 1e-3, -7.0])
    else:
        x = torch.tensor([0.0, -0.0, 1e-40, -3e-41, 0.0, 0.0, 2e-39, -0.0] * 5)
    xd = x.to(DEV).contiguous().view(-1)
    h = nvfp4.calib_histogram(xd)
    href = orc.calib_histogram(f32(x).ravel())
    assert np.array_equal(h.cpu().numpy().view(np.uint64), href)
    for frac in (0.5, 0.99, 0.9999, 1.0):
        S = nvfp4.calib_scale(h, frac)
        assert S.item() == orc.calib_scale(href, frac), frac


def test_calib_scale_empty_histogram(orc):
    case("calibration scale of an empty histogram")
    h = torch.zeros(nvfp4.CALIB_BINS, dtype=torch.int64, device=DEV)
    for frac in (0.5, 1.0):
        assert nvfp4.calib_scale(h, frac).item() == orc.calib_scale(np.zeros(nvfp4.CALIB_BINS, np.uint64), frac)


@pytest.mark.parametrize("layout", ["single_bins", "boundaries", "sparse_random", "dense_random", "huge_counts"])
def test_calib_scale_synthetic_histograms(orc, layout):
    """The clip scale from histograms built directly (seeded), with the crossing bin at the
    first and last bin, at 64-bin row and 2048-bin group edges, and with counts above 2^32."""
    case(f"calibration scale of synthetic histograms: {layout}")
    rng = np.random.default_rng(97)
    B = nvfp4.CALIB_BINS
    hists = []
    if layout == "single_bins":
        for b in (0, 1, 63, 64, 2047, 2048, 16383, 30000, B - 1):
            h = np.zeros(B, np.uint64)
            h[b] = 5
            hists.append(h)
    elif layout == "boundaries":
        for edge in (64, 2048, 4096, 30720):
            h = np.zeros(B, np.uint64)
            h[edge - 1] = 3
            h[edge] = 4
            h[edge + 1] = 1
            hists.append(h)
    elif layout == "sparse_random":
        for _ in range(6):
            h = np.zeros(B, np.uint64)
            idx = rng.choice(B, size=40, replace=False)
            h[idx] = rng.integers(1, 1000, size=40).astype(np.uint64)
            hists.append(h)
    elif layout == "dense_random":
        for _ in range(3):
            hists.append(rng.integers(0, 50, size=B).astype(np.uint64))
    else:
        h = np.zeros(B, np.uint64)
        h[[100, 16000, 16001, 32000]] = np.array([3 << 33, 1 << 34, 7, 5 << 32], np.uint64)
        hists.append(h)
    for h in hists:
        hd = torch.from_numpy(h.view(np.int64).copy()).to(DEV)
        for frac in (1e-9, 0.25, 0.5, 0.75, 0.99, 0.9999, 1.0):
            got, want = np.float32(nvfp4.calib_scale(hd, frac).item()), orc.calib_scale(h, frac)
            # the top bins hold inf / NaN magnitudes: their clip scale is NaN on both sides
            assert got == want or (np.isnan(got) and np.isnan(want)), (layout, frac, got, want)


def test_calib_accumulates_over_batches(orc):
    case("calibration histogram over three batches")
    xs = [synth.activation(s, tokens=64, hidden=1024) for s in (7, 8, 9)]
    h = None
    href = None
    for x in xs:
        h = nvfp4.calib_histogram(x.to(DEV).view(-1), h)
        href = orc.calib_histogram(f32(x).ravel(), href)
    assert np.array_equal(h.cpu().numpy().view(np.uint64), href)
    assert nvfp4.calib_scale(h, 0.999).item() == orc.calib_scale(href, 0.999)


# ------------------------------------------------------------------ block Hessian

@pytest.mark.parametrize("which", ["tiny_fp32", "proj_bf16", "ragged_bf16", "narrow_bf16"])
def test_block_hessian_dense(orc, tiny, which):
    if which == "tiny_fp32":
        x = tiny[1]
    elif which == "proj_bf16":
        x = synth.projection(1, rows=16, cols=512, tokens=4096)[1]
    elif which == "ragged_bf16":
        x = synth.projection(2, rows=16, cols=256, tokens=1000)[1]
    else:
        x = synth.projection(3, rows=16, cols=48, tokens=777)[1]
    case(f"hessian dense {which} {tuple(x.shape)}")
    xd = x.to(DEV)
    H = nvfp4.block_hessian(xd)
    Href = orc.block_hessian(f32(x))
    assert rel_frob(H.cpu().numpy(), Href) <= 1e-4
    H2 = nvfp4.block_hessian(xd)
    assert torch.equal(H, H2), "not bitwise reproducible"


def test_block_hessian_accumulate(orc):
    case("hessian accumulate over two batches")
    x = synth.projection(4, rows=16, cols=256, tokens=3000)[1]
    a, b = x[:1200].contiguous(), x[1200:].contiguous()
    H = nvfp4.block_hessian(a.to(DEV))
    H = nvfp4.block_hessian(b.to(DEV), H=H, accumulate=True)
    Href = orc.block_hessian(f32(x))
    assert rel_frob(H.cpu().numpy(), Href) <= 1e-4


def test_route_groups_and_grouped_hessian(orc):
    case("route groups 3000 tokens top-4 over 16 experts + grouped hessian")
    _, x, ids = synth.moe(5, experts=16, rows=16, cols=256, tokens=3000, topk=4)
    ids_np = ids.numpy()
    off, tok = nvfp4.route_groups(ids.to(DEV), 16)
    off_ref, tok_ref = orc.route_groups(ids_np, 16)
    assert np.array_equal(off.cpu().numpy(), off_ref)
    assert np.array_equal(tok.cpu().numpy(), tok_ref)
    H = nvfp4.block_hessian(x.to(DEV), group_offsets=off, token_ids=tok)
    Hn = H.cpu().numpy()
    xn = f32(x)
    for e in range(16):
        Href = orc.block_hessian(xn, tok_ref[off_ref[e]:off_ref[e + 1]])
        assert rel_frob(Hn[e], Href) <= 1e-4, e


@pytest.mark.parametrize("tokens,topk,experts,lo,hi", [
    (5000, 3, 7, -2, 9),        # repeats within a token and out-of-range ids
    (4000, 8, 3000, 0, 3000),   # several expert blocks in the scan
    (700, 2, 16384, -1, 16385), # the largest expert count
    (1234, 5, 1, 0, 1),         # one expert: every pair, in order
    (0, 4, 5, 0, 5),            # no tokens
])
def test_route_groups_repeats_and_invalid_ids(orc, tokens, topk, experts, lo, hi):
    case(f"route groups tokens={tokens} topk={topk} experts={experts} ids in [{lo},{hi})")
    rng = np.random.default_rng(tokens + experts)
    ids = rng.integers(lo, hi, size=(tokens, topk)).astype(np.int32)
    off, tok = nvfp4.route_groups(torch.from_numpy(ids).to(DEV), experts)
    # expected: the stable sort of the valid pairs; invalid ids go to an extra last expert
    dump = np.where((ids >= 0) & (ids < experts), ids, experts).astype(np.int32)
    off_ref, tok_ref = orc.route_groups(dump, experts + 1)
    n = int(off_ref[experts])
    assert np.array_equal(off.cpu().numpy(), off_ref[:experts + 1])
    assert np.array_equal(tok.cpu().numpy()[:n], tok_ref[:n])


def test_grouped_hessian_with_empty_group(orc):
    case("grouped hessian with an empty expert")
    _, x, _ = synth.moe(6, experts=4, rows=16, cols=64, tokens=700, topk=2)
    ids = np.array([[0, 2]] * 400 + [[2, 3]] * 300, np.int32)
    off, tok = nvfp4.route_groups(torch.from_numpy(ids).to(DEV), 4)
    off_ref, tok_ref = orc.route_groups(ids, 4)
    assert np.array_equal(off.cpu().numpy(), off_ref)
    H = nvfp4.block_hessian(x.to(DEV), group_offsets=off, token_ids=tok).cpu().numpy()
    assert np.all(H[1] == 0)
    for e in (0, 2, 3):
        assert rel_frob(H[e], orc.block_hessian(f32(x), tok_ref[off_ref[e]:off_ref[e + 1]])) <= 1e-4


@pytest.mark.parametrize("cols", [256, 208])
def test_grouped_hessian_accumulate_multi_piece(orc, cols):
    """Grouped bf16 Hessians accumulated over two batches. Expert 0 takes every token
    (its list is cut into several pieces whose partial sums are reduced), the others a
    few hundred each (one piece, written straight into H); 208 channels leave a ragged
    last 64-channel chunk."""
    case(f"grouped hessian accumulate, multi-piece expert 0, cols={cols}")
    tokens, E = 9000, 5
    x = synth.projection(11, rows=16, cols=cols, tokens=tokens)[1]
    rng = np.random.default_rng(12)
    second = rng.integers(1, E, size=tokens)
    ids = np.stack([np.zeros(tokens, np.int64), second], 1).astype(np.int32)
    xn = f32(x)
    halves = (slice(0, 4000), slice(4000, tokens))
    H = None
    for sl in halves:
        xb = x[sl].contiguous()
        off, tok = nvfp4.route_groups(torch.from_numpy(ids[sl].copy()).to(DEV), E)
        H = nvfp4.block_hessian(xb.to(DEV), group_offsets=off, token_ids=tok, H=H,
                                accumulate=H is not None)
    off_ref, tok_ref = orc.route_groups(ids, E)
    assert int(off_ref[1]) == tokens  # expert 0: every token
    Hn = H.cpu().numpy()
    for e in range(E):
        Href = orc.block_hessian(xn, tok_ref[off_ref[e]:off_ref[e + 1]])
        assert rel_frob(Hn[e], Href) <= 1e-4, e


# ------------------------------------------------------------------ Local-Hessian search

def _lh_check(orc, w, S, H, stats_out=None):
    """H: fp32 numpy [cols/16, 16, 16], made by the oracle or in closed form; both sides
    search with it. The search also runs without objectives and with its counters on (a
    separate instantiation); all give the same bytes. The counters go to stats_out."""
    H = np.ascontiguousarray(H, dtype=np.float32)
    wd, Sd, Hd = w.to(DEV), dev_S(S), torch.from_numpy(H).to(DEV)
    sc, obj = nvfp4.scale_search_local_hessian(wd, Sd, Hd, return_obj=True)
    sr, orf = orc.scales_local_hessian(f32(w), S, H, with_obj=True)
    g = sc.cpu().numpy()
    assert np.array_equal(g, sr), f"{np.sum(g != sr)} bytes differ"
    assert np.array_equal(obj.cpu().numpy(), orf)
    assert torch.equal(nvfp4.scale_search_local_hessian(wd, Sd, Hd), sc)
    nvfp4.search_stats_read()
    nvfp4.search_stats_enable(True)
    try:
        sc_st = nvfp4.scale_search_local_hessian(wd, Sd, Hd)
        st = nvfp4.search_stats_read()
    finally:
        nvfp4.search_stats_enable(False)
    assert torch.equal(sc_st, sc)
    nz = int((np.abs(f32(w)).reshape(-1, 16).max(1) > 0).sum())
    assert st["lh_pairs"] + st["lh_zero_h"] == nz
    if stats_out is not None:
        stats_out.update(st)
    return g


def test_local_hessian_tiny(orc, tiny):
    w, x = tiny
    case("local hessian tiny fp32")
    S = orc.tensor_scale(w.numpy())
    _lh_check(orc, w, S, orc.block_hessian(f32(x)))


def test_local_hessian_bf16_projection(orc):
    case("local hessian bf16 96x512, H from 4096 t4 tokens")
    w, x = synth.projection(7, rows=96, cols=512, tokens=4096)
    S = orc.tensor_scale(f32(w))
    _lh_check(orc, w, S, orc.block_hessian(f32(x)))


def test_local_hessian_special_hessians(orc):
    case("local hessian with H = I (equals MSE up to fp32/fp64 near-ties) and a zero H block")
    w = synth.mlp_weight(8, 64, 128)
    wn = f32(w)
    S = orc.tensor_scale(wn)
    eye = np.repeat(np.eye(16, dtype=np.float32)[None], 8, axis=0)
    eye[2] = 0.0
    st = {}
    g = _lh_check(orc, w, S, eye, st)
    assert st["lh_zero_h"] == 64  # block column 2's 64 rows took the MSE choice
    mse = orc.scales_mse(wn, S)
    assert np.array_equal(g[:, 2], mse[:, 2])
    assert np.mean(g == mse) > 0.99
    case("local hessian with a rank-1 H (one token)")
    x1 = torch.randn(1, 128, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    _lh_check(orc, w, S, orc.block_hessian(f32(x1)))


def _dominant_h(delta: float) -> np.ndarray:
    """(16 + delta) I - 11^T: PSD, g_i = delta, kappa ~ 30 / delta."""
    return ((16.0 + delta) * np.eye(16) - np.ones((16, 16))).astype(np.float32)


def test_local_hessian_magnitude_regimes(orc):
    w0, x = synth.projection(11, rows=64, cols=256, tokens=2048)
    H0 = orc.block_hessian(f32(x)).astype(np.float32)
    nb = H0.shape[0]
    regimes = [
        ("large weights (x1e4)", 1e4, H0),
        ("tiny weights (x1e-15)", 1e-15, H0),
        ("H in the fp32 denormal range (x1e-44)", 1.0, H0 * np.float32(1e-44)),
        ("huge H (x1e30): fp32 screen would overflow", 1.0, H0 * np.float32(1e30)),
        ("large weights and large H (x1e3, x1e20)", 1e3, H0 * np.float32(1e20)),
        ("diagonally dominant H, kappa ~3e4 (absolute screen bound)", 1.0,
         np.repeat(_dominant_h(1e-3)[None], nb, axis=0)),
        ("nearly singular H, kappa ~3e9 (no pruning)", 1.0,
         np.repeat(_dominant_h(1e-8)[None], nb, axis=0)),
    ]
    seen = {}
    for name, ws, H in regimes:
        case(f"local hessian, {name}")
        w = (w0.float() * ws).to(torch.bfloat16)
        S = orc.tensor_scale(f32(w))
        st = {}
        _lh_check(orc, w, S, H, st)
        print("[info] " + ", ".join(f"{k} {v}" for k, v in st.items() if k.startswith("lh_")), flush=True)
        seen[name] = st
    # each of the kernel's paths is taken, and agrees with the oracle, in some regime
    assert seen["large weights (x1e4)"]["lh_rel"] > 0 and seen["large weights (x1e4)"]["lh_two"] > 0
    assert seen["diagonally dominant H, kappa ~3e4 (absolute screen bound)"]["lh_abs"] > 0
    assert seen["nearly singular H, kappa ~3e9 (no pruning)"]["lh_noprune"] > 0
    assert seen["huge H (x1e30): fp32 screen would overflow"]["lh_rescan"] == 1024
    assert seen["H in the fp32 denormal range (x1e-44)"]["lh_rescan"] == 1024


def test_local_hessian_batched_experts(orc):
    case("local hessian batch of 4 experts with per-expert S and H")
    w, x, ids = synth.moe(9, experts=4, rows=40, cols=128, tokens=600, topk=2)
    off_ref, tok_ref = orc.route_groups(ids.numpy(), 4)
    Href = np.stack([orc.block_hessian(f32(x), tok_ref[off_ref[e]:off_ref[e + 1]])
                     for e in range(4)]).astype(np.float32)
    Sn = np.array([orc.tensor_scale(f32(w[e])) for e in range(4)], np.float32)
    # the GPU's routing, grouped Hessian and scales against the oracle's
    off, tok = nvfp4.route_groups(ids.to(DEV), 4)
    assert np.array_equal(off.cpu().numpy(), off_ref)
    H = nvfp4.block_hessian(x.to(DEV), group_offsets=off, token_ids=tok)
    for e in range(4):
        assert rel_frob(H[e].cpu().numpy(), Href[e].astype(np.float64)) <= 1e-4
    wd = w.to(DEV)
    assert np.array_equal(nvfp4.global_scale(wd).cpu().numpy(), Sn)
    # the batched search, both sides on the oracle's S and H
    S = torch.from_numpy(Sn).to(DEV)
    sc, obj = nvfp4.scale_search_local_hessian(wd, S, torch.from_numpy(Href).to(DEV), return_obj=True)
    srs = []
    for e in range(4):
        sr, orf = orc.scales_local_hessian(f32(w[e]), Sn[e], Href[e], with_obj=True)
        assert np.array_equal(sc[e].cpu().numpy(), sr)
        assert np.array_equal(obj[e].cpu().numpy(), orf)
        srs.append(sr)
    # final quantisation with the chosen bytes (the oracle's, equal to the GPU's)
    codes, _ = nvfp4.quantize(wd, S, torch.from_numpy(np.stack(srs)).to(DEV))
    for e in range(4):
        assert np.array_equal(codes[e].cpu().numpy(), orc.quantize(f32(w[e]), Sn[e], srs[e]))


# ------------------------------------------------------------------ debug input checks

def test_debug_nonfinite_flag(monkeypatch):
    case("NVFP4_DEBUG_CHECKS=1: non-finite inputs raise the device flag")
    monkeypatch.setenv("NVFP4_DEBUG_CHECKS", "1")
    nvfp4.debug_nonfinite()  # start clean
    x = synth.activation(30, 64, 256).to(DEV)
    S = nvfp4.global_scale(x)
    nvfp4.fakequant(x, S)
    assert nvfp4.debug_nonfinite() is False
    x[3, 17] = float("nan")
    nvfp4.fakequant(x, S)
    assert nvfp4.debug_nonfinite() is True
    assert nvfp4.debug_nonfinite() is False          # read clears it
    g = torch.zeros(4096, device=DEV)
    g[100] = float("-inf")
    nvfp4.ste_backward(g, 1.0)
    assert nvfp4.debug_nonfinite() is True
    xh = synth.projection(31, rows=16, cols=64, tokens=100)[1].to(DEV)
    nvfp4.block_hessian(xh)
    assert nvfp4.debug_nonfinite() is False
    xh[50, 7] = float("inf")
    nvfp4.block_hessian(xh)
    assert nvfp4.debug_nonfinite() is True
    xq = synth.activation(32, 16, 64).to(DEV)
    nvfp4.quantize(xq, dev_S(0.0))                    # a non-positive tensor scale
    assert nvfp4.debug_nonfinite() is True
    nvfp4.quantize(xq, dev_S(1e-3))
    assert nvfp4.debug_nonfinite() is False
    monkeypatch.delenv("NVFP4_DEBUG_CHECKS")
    with pytest.raises(nvfp4.NVFP4Error):
        nvfp4.debug_nonfinite()
