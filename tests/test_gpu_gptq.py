"""GPU parity of the full Gram matrix and of GPTQ rounding (factor and column loop) against
the CPU oracle.

Bar: H within 1e-4 relative Frobenius error per 16x16 block (fp32 accumulation against the
oracle's fp64 sums), exactly symmetric and bitwise reproducible; the factor U within 1e-8
of the oracle's (both in double; relative to max |U|); GPTQ codes identical to the oracle's
when both start from the same fp32 H, checked on every column of every row
(tests/gptq_check.py): a row may take the other rounding only at a value within 1e-9 of a
rounding midpoint (relative to the block scale), after which the oracle follows the same
rounding; the end-to-end case (GPU H against the oracle's fp64 H) allows 1e-4 there.
"""
import numpy as np
import pytest
import torch

from gptq_check import check_rows
from scale_search_weights_amd import nvfp4, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def case(msg):
    print(f"[case] {msg}", flush=True)


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy()


def block_rel_frob(Hg: np.ndarray, Hr: np.ndarray) -> float:
    n = Hr.shape[0]
    a = Hg.astype(np.float64).reshape(n // 16, 16, n // 16, 16).transpose(0, 2, 1, 3)
    b = Hr.reshape(n // 16, 16, n // 16, 16).transpose(0, 2, 1, 3)
    num = np.linalg.norm((a - b).reshape(-1, 256), axis=1)
    den = np.linalg.norm(b.reshape(-1, 256), axis=1)
    return float(np.where(den > 0, num / np.where(den > 0, den, 1), num).max())


# ------------------------------------------------------------------ full Gram matrix

@pytest.mark.parametrize("which", ["bf16_ragged", "bf16_proj", "fp32", "bf16_narrow"])
def test_full_hessian(orc, which):
    if which == "bf16_ragged":
        x = synth.projection(5, rows=16, cols=272, tokens=1000)[1]        # 2 tiles + 16 cols
    elif which == "bf16_proj":
        x = synth.projection(6, rows=16, cols=512, tokens=4096)[1]
    elif which == "fp32":
        x = torch.from_numpy((np.random.default_rng(7).standard_t(4, (700, 144))).astype(np.float32))
    else:
        x = synth.projection(8, rows=16, cols=32, tokens=77)[1]
    case(f"full hessian {which} {tuple(x.shape)} {x.dtype}")
    xd = x.to(DEV)
    H = nvfp4.full_hessian(xd)
    Hn = H.cpu().numpy()
    ref = orc.full_hessian(f32(x))
    assert block_rel_frob(Hn, ref) <= 1e-4
    assert np.array_equal(Hn, Hn.T)
    assert np.array_equal(nvfp4.full_hessian(xd).cpu().numpy(), Hn)       # reproducible
    Hb = nvfp4.block_hessian(xd).cpu().numpy()
    for b in range(Hn.shape[0] // 16):
        blk = Hn[16 * b:16 * b + 16, 16 * b:16 * b + 16]
        assert np.abs(blk - Hb[b]).max() <= 1e-5 * np.abs(Hb[b]).max() + 1e-30


def test_full_hessian_long_input_per_xcd_chunks(orc):
    """Enough tokens for the per-XCD chunk layout (8 chunks), with a ragged tile edge."""
    case("full hessian 20000 tokens x 272 bf16 (8 token chunks)")
    x = synth.projection(17, rows=16, cols=272, tokens=20000)[1]
    Hn = nvfp4.full_hessian(x.to(DEV)).cpu().numpy()
    assert block_rel_frob(Hn, orc.full_hessian_blas(f32(x))) <= 1e-4
    assert np.array_equal(Hn, Hn.T)


@pytest.mark.parametrize("tokens,cols", [(1, 16), (33, 48), (20001, 272), (3000, 528)])
def test_full_hessian_bf16_partial_stages(orc, tokens, cols):
    """bf16 inputs whose last 32-token stage is partial (rows past the end must read as
    zero), with channel counts off the 256-channel tile grid; 20001 tokens also takes the
    per-XCD chunk layout with an empty tail chunk."""
    case(f"full hessian bf16 {tokens} tokens x {cols}")
    x = synth.projection(tokens % 97 + cols, rows=16, cols=cols, tokens=tokens)[1]
    assert x.dtype == torch.bfloat16
    Hn = nvfp4.full_hessian(x.to(DEV)).cpu().numpy()
    assert block_rel_frob(Hn, orc.full_hessian_blas(f32(x))) <= 1e-4
    assert np.array_equal(Hn, Hn.T)


def test_full_hessian_wide_unsplit_tokens(orc):
    """16384 channels: 2080 tiles, enough workgroups without splitting the tokens (the
    partial-tile workspace then holds one chunk); ragged token count."""
    case("full hessian bf16 300 tokens x 16384 (no token chunks)")
    x = synth.projection(23, rows=16, cols=16384, tokens=300)[1]
    ws_one = nvfp4.lib().nvfp4_full_hessian_workspace_size(300, 16384)
    assert ws_one <= 2080 * 256 * 256 * 4
    Hn = nvfp4.full_hessian(x.to(DEV)).cpu().numpy()
    assert block_rel_frob(Hn, orc.full_hessian_blas(f32(x))) <= 1e-4
    assert np.array_equal(Hn, Hn.T)


def test_full_hessian_accumulate_and_empty(orc):
    case("full hessian: two batches accumulated, and zero tokens")
    xs = [synth.projection(s, rows=16, cols=256, tokens=600)[1] for s in (9, 10)]
    H = nvfp4.full_hessian(xs[0].to(DEV))
    nvfp4.full_hessian(xs[1].to(DEV), H=H, accumulate=True)
    ref = orc.full_hessian(np.concatenate([f32(x) for x in xs]))
    assert block_rel_frob(H.cpu().numpy(), ref) <= 1e-4
    assert not nvfp4.full_hessian(torch.empty(0, 64, dtype=torch.bfloat16, device=DEV)).cpu().numpy().any()
    e = torch.empty(0, 256, dtype=torch.bfloat16, device=DEV)
    H2 = H.clone()
    nvfp4.full_hessian(e, H=H2, accumulate=True)
    assert torch.equal(H2, H)


# ------------------------------------------------------------------ factor

def _h_problem(orc, seed, n, corr=1.0):
    """fp32 H = X^T X of 2n correlated tokens (condition number about 10 n)."""
    rng = np.random.default_rng(seed)
    X = (corr * rng.standard_normal((2 * n, 1)) + rng.standard_normal((2 * n, n))).astype(np.float32)
    return orc.full_hessian(X).astype(np.float32)


@pytest.mark.parametrize("n", [48, 208, 512, 1040])
def test_gptq_factor(orc, n):
    case(f"gptq factor n={n}")
    H = _h_problem(orc, n, n)
    U, status = nvfp4.gptq_factor(torch.from_numpy(H).to(DEV), 0.01)
    assert status.item() == 0
    Ug = U.cpu().numpy()
    Ur = orc.gptq_factor(H.astype(np.float64), 0.01)
    # backward-stable fp64 factorisations: error ~ n eps kappa, kappa ~ 10 n here
    assert np.abs(Ug - Ur).max() <= 1e-8 * np.abs(Ur).max()
    assert not np.tril(Ug, -1).any()


def test_gptq_factor_wide_and_narrow_updates(orc):
    """n = 3072: the first Cholesky trailing updates have 24 * 25 / 2 = 300 tiles of 128 x 128
    (the wide form), the later ones fewer than the compute units (the 64 x 64 form). A weakly
    correlated H (condition number about 400) keeps the fp64 error far below the bound."""
    n = 3072
    case(f"gptq factor n={n}: wide and 64x64 trailing updates")
    rng = np.random.default_rng(31)
    X = 0.1 * rng.standard_normal((2 * n, 1)) + rng.standard_normal((2 * n, n))
    H = (X.T @ X).astype(np.float32)  # any SPD fp32 matrix serves; a BLAS product is quick
    U, status = nvfp4.gptq_factor(torch.from_numpy(H).to(DEV), 0.01)
    assert status.item() == 0
    Ug = U.cpu().numpy()
    Ur = orc.gptq_factor(H.astype(np.float64), 0.01)
    assert np.abs(Ug - Ur).max() <= 1e-8 * np.abs(Ur).max()
    assert not np.tril(Ug, -1).any()


def test_gptq_factor_degenerate(orc):
    case("gptq factor: zero H gives I; an indefinite H is reported")
    U, status = nvfp4.gptq_factor(torch.zeros(64, 64, device=DEV), 0.01)
    assert status.item() == 0 and torch.equal(U.cpu(), torch.eye(64, dtype=torch.float64))
    H = np.eye(96, dtype=np.float32)
    H[40, 40] = -3.0
    _, status = nvfp4.gptq_factor(torch.from_numpy(H).to(DEV), 0.0)
    assert status.item() != 0


@pytest.mark.parametrize("n", [208, 1040])
def test_gptq_factor_workspace_contents_unread(orc, n):
    """The factor writes every part of its workspace that it reads (the inverse's blocks
    below the diagonal are written before use, those above are zeroed): a workspace filled
    with NaN gives the same U, bit for bit, as a zeroed one."""
    case(f"gptq factor n={n}: NaN-filled workspace")
    H = torch.from_numpy(_h_problem(orc, 7, n)).to(DEV)
    need = int(nvfp4.lib().nvfp4_gptq_factor_workspace_size(n))
    ws0 = torch.zeros(need, dtype=torch.uint8, device=DEV)
    wsn = torch.full((need // 8,), float("nan"), dtype=torch.float64, device=DEV).view(torch.uint8)
    U0, s0 = nvfp4.gptq_factor(H, 0.01, workspace=ws0)
    Un, sn = nvfp4.gptq_factor(H, 0.01, workspace=wsn)
    assert s0.item() == 0 and sn.item() == 0
    assert torch.equal(U0, Un)


def _exact_any_order(diag_f32):
    """True when every partial sum of these fp32 values, in any order, is exact in double:
    each is an integer multiple of 2^qlo (its lowest set bit) below 2^(qhi + 1), so partial
    sums stay below n 2^(qhi + 1) in units of the smallest 2^qlo."""
    u = diag_f32.view(np.uint32) & np.uint32(0x7FFFFFFF)
    u = u[u != 0]
    if u.size == 0:
        return True
    E = (u >> np.uint32(23)).astype(np.int64)
    m = np.where(E > 0, (u & np.uint32(0x7FFFFF)) | np.uint32(0x800000), u).astype(np.int64)
    e0 = np.maximum(E, 1) - 150
    lo = np.array([int(x & -x).bit_length() - 1 for x in m]) + e0
    hi = np.array([int(x).bit_length() - 1 for x in m]) + e0
    n = diag_f32.size
    return (n - 1).bit_length() + int(hi.max()) + 1 - int(lo.min()) <= 53


@pytest.mark.parametrize("spread", [False, True])
def test_gptq_factor_damping_in_index_order(orc, spread):
    """lambda = damp * (sum of diag H in index order) / n, bit for bit, read from the first
    word of the factor's workspace (where the factor keeps it). A diagonal within a narrow
    exponent range takes a tree sum (every partial sum exact); a diagonal spread over 2^-80 to
    2^26 takes the index-order chain. Both must give the index-order sum's bits."""
    n = 1040
    case(f"gptq factor n={n}: damping sum, {'wide' if spread else 'narrow'} diagonal range")
    rng = np.random.default_rng(8)
    X = rng.standard_normal((2 * n, n))
    H = X.T @ X / (2 * n)
    if spread:
        d = np.logspace(-12, 4, n)
        H = d[:, None] * H * d[None, :]
    H = H.astype(np.float32)
    diag = np.ascontiguousarray(np.diagonal(H))
    assert _exact_any_order(diag) != spread
    need = int(nvfp4.lib().nvfp4_gptq_factor_workspace_size(n))
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    _, status = nvfp4.gptq_factor(torch.from_numpy(H).to(DEV), 0.01, workspace=ws)
    assert status.item() == 0
    tr = 0.0
    for v in diag.tolist():  # index order, in double
        tr += v
    assert ws[:8].view(torch.float64).item() == 0.01 * (tr / n)


def test_gptq_factor_bitwise_repeatable():
    """The Cholesky step's waves hand the diagonal block's columns to the panel waves through
    an LDS counter; a missed handoff would read a column before it is written and show up as
    run-to-run differences. Sixteen factors of the same H (n = 1040: 17 steps, from 16 panel
    blocks down to none, the last step without a partner) must agree bit for bit."""
    n = 1040
    case(f"gptq factor n={n}: 16 repeated runs, bit for bit")
    rng = np.random.default_rng(5)
    X = rng.standard_normal((2 * n, 1)) + rng.standard_normal((2 * n, n))
    H = torch.from_numpy((X.T @ X).astype(np.float32)).to(DEV)
    U0, s0 = nvfp4.gptq_factor(H, 0.01)
    assert s0.item() == 0
    for _ in range(15):
        U, st = nvfp4.gptq_factor(H, 0.01)
        assert st.item() == 0 and torch.equal(U, U0)


# ------------------------------------------------------------------ GPTQ rows

def test_gptq_factor_more_workgroups_than_fit():
    """n = 20480: a Cholesky step launches 320 workgroups, more than run at once, so some
    start after workgroup 0 has factored the diagonal block; they must still read A_kk.
    Checked through U (H + lambda I) U^T z = z (U^T U = (H + lambda I)^-1), for H = G G^T + 20 I
    (condition number about 10^3)."""
    n, damp = 20480, 0.01
    case(f"gptq factor n={n}: property U M U^T = I on random vectors")
    g = torch.Generator(device="cpu").manual_seed(123)
    G = torch.randn(n, 64, generator=g).to(DEV)
    H = G @ G.T
    H.diagonal().add_(20.0)
    del G
    U, status = nvfp4.gptq_factor(H, damp)
    assert status == 0
    M = H.double()
    lam = damp * M.diagonal().sum().item() / n
    M.diagonal().add_(lam)
    del H
    Z = torch.randn(n, 4, generator=g, dtype=torch.float64).to(DEV)
    R = U @ (M @ (U.T @ Z))
    rel = ((R - Z).norm(dim=0) / Z.norm(dim=0)).max().item()
    assert rel <= 1e-8, rel
    assert torch.all(torch.diagonal(U) > 0)


@pytest.mark.parametrize("which", ["bf16_lh", "fp32_ragged", "zero_blocks", "wide"])
def test_gptq_rows_same_factor(orc, which):
    """The oracle's own U feeds both sides: only the column loop is compared."""
    rng = np.random.default_rng(11)
    if which == "bf16_lh":
        w, x = synth.projection(12, rows=64, cols=208, tokens=600)
    elif which == "fp32_ragged":
        w = torch.from_numpy((rng.standard_normal((100, 512)) * 0.02).astype(np.float32))
        x = synth.projection(13, rows=16, cols=512, tokens=1500)[1]
    elif which == "wide":                                   # 17 column blocks: 4 outer + 1
        w, x = synth.projection(16, rows=40, cols=1040, tokens=2500)
    else:
        w, x = synth.projection(14, rows=70, cols=128, tokens=400)
        w = w.clone()
        w[3, :48] = 0
        w[:, 64:80] = 0
    case(f"gptq rows {which} {tuple(w.shape)} {w.dtype}")
    wn = f32(w)
    S = orc.tensor_scale(wn)
    H = orc.full_hessian(f32(x)).astype(np.float32)
    sc = orc.scales_local_hessian(wn, S, orc.block_hessian(f32(x)))
    Ur = orc.gptq_factor(H.astype(np.float64), 0.01)
    got = nvfp4.gptq(w.to(DEV), torch.tensor([S], device=DEV), torch.from_numpy(sc).to(DEV),
                     torch.from_numpy(Ur).to(DEV))
    ties = check_rows(got.cpu().numpy(), wn, S, sc, Ur, orc, tie_tol=1e-9)
    print(f"[info] near-ties followed: {ties}", flush=True)


def test_gptq_rows_wide_and_narrow_outer_updates(orc):
    """4096 x 1280: the first outer update has 32 x 8 = 256 tiles of 128 x 128 (the wide form,
    which reads its output tile beside the products), the later ones fewer (the 64 x 64 form).
    The oracle's own U and max-scaling bytes feed both sides."""
    case("gptq rows 4096x1280 bf16: wide and 64x64 outer updates")
    w, x = synth.projection(18, rows=4096, cols=1280, tokens=3000)
    wn = f32(w)
    S = orc.tensor_scale(wn)
    sc = orc.scales_max(wn, S)
    Ur = orc.gptq_factor(orc.full_hessian(f32(x)).astype(np.float32).astype(np.float64), 0.01)
    got = nvfp4.gptq(w.to(DEV), torch.tensor([S], device=DEV), torch.from_numpy(sc).to(DEV),
                     torch.from_numpy(Ur).to(DEV))
    ties = check_rows(got.cpu().numpy(), wn, S, sc, Ur, orc, tie_tol=1e-9)
    print(f"[info] near-ties followed: {ties}", flush=True)


def test_gptq_rows_workspace_contents_unread(orc):
    """GPTQ rounding writes every part of its workspace that it reads (the working copy of W,
    padding included, and each outer block's errors): a NaN-filled workspace gives the same
    codes as a zeroed one. 100 x 1040: padded rows and columns, 4 full outer blocks + 1."""
    case("gptq rows 100x1040: NaN-filled workspace")
    w, x = synth.projection(17, rows=100, cols=1040, tokens=2500)
    wn = f32(w)
    S = orc.tensor_scale(wn)
    sc = orc.scales_local_hessian(wn, S, orc.block_hessian(f32(x)))
    U, status = nvfp4.gptq_factor(torch.from_numpy(orc.full_hessian(f32(x)).astype(np.float32)).to(DEV), 0.01)
    assert status.item() == 0
    need = int(nvfp4.lib().nvfp4_gptq_workspace_size(100, 1040))
    ws0 = torch.zeros(need, dtype=torch.uint8, device=DEV)
    wsn = torch.full((need // 8,), float("nan"), dtype=torch.float64, device=DEV).view(torch.uint8)
    args = (w.to(DEV), torch.tensor([S], device=DEV), torch.from_numpy(sc).to(DEV), U)
    c0 = nvfp4.gptq(*args, workspace=ws0)
    cn = nvfp4.gptq(*args, workspace=wsn)
    assert torch.equal(c0, cn)


def test_gptq_end_to_end(orc):
    """GPU H -> GPU factor -> GPU GPTQ against the oracle's chain from the same X."""
    case("gptq end to end 128x512 bf16")
    w, x = synth.projection(15, rows=128, cols=512, tokens=2048)
    wn, xn = f32(w), f32(x)
    S = orc.tensor_scale(wn)
    sc = orc.scales_local_hessian(wn, S, orc.block_hessian(xn))
    Href = orc.full_hessian(xn)
    Uref = orc.gptq_factor(Href, 0.01)
    Hd = nvfp4.full_hessian(x.to(DEV))
    U, status = nvfp4.gptq_factor(Hd, 0.01)
    assert status.item() == 0
    got = nvfp4.gptq(w.to(DEV), torch.tensor([S], device=DEV), torch.from_numpy(sc).to(DEV), U)
    # the GPU's H (fp32 sums) and factor differ from the oracle's fp64 chain in the last
    # bits, so near-ties are looser here (1e-4 s S); every column of every row is checked
    ties = check_rows(got.cpu().numpy(), wn, S, sc, Uref, orc, tie_tol=1e-4)
    print(f"[info] near-ties followed: {ties}", flush=True)
    # GPTQ lowers the layer-output error against plain rounding at the same bytes
    rows, cols = wn.shape
    deq = lambda c: orc.dequantize(c, sc, S, rows, cols).astype(np.float64) - wn
    err = lambda c: np.einsum("ri,ij,rj->", deq(c), Href, deq(c))
    assert err(got.cpu().numpy()) < 0.95 * err(orc.quantize(wn, S, sc))


@pytest.mark.parametrize("scale", [1e-20, 1e20])
def test_gptq_rows_extreme_magnitudes(orc, scale):
    """Everything stays in double: tiny and huge weights round the same way on both sides."""
    case(f"gptq rows with weights x{scale:g}")
    w0, x = synth.projection(18, rows=32, cols=128, tokens=500)
    wn = (f32(w0).astype(np.float64) * scale).astype(np.float32)
    S = orc.tensor_scale(wn)
    H = orc.full_hessian(f32(x)).astype(np.float32)
    sc = orc.scales_mse(wn, S)
    Ur = orc.gptq_factor(H.astype(np.float64), 0.01)
    got = nvfp4.gptq(torch.from_numpy(wn).to(DEV), torch.tensor([S], device=DEV),
                     torch.from_numpy(sc).to(DEV), torch.from_numpy(Ur).to(DEV))
    check_rows(got.cpu().numpy(), wn, S, sc, Ur, orc, tie_tol=1e-9)


def test_full_hessian_smallest_shapes(orc):
    case("full hessian: one token, 16 channels; 3 tokens, 48 channels")
    for tokens, cols in ((1, 16), (3, 48)):
        x = torch.from_numpy(np.random.default_rng(cols).standard_normal((tokens, cols)).astype(np.float32))
        Hn = nvfp4.full_hessian(x.to(DEV)).cpu().numpy()
        assert block_rel_frob(Hn, orc.full_hessian(f32(x))) <= 1e-6
