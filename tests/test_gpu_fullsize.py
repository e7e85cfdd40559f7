"""GPU parity at the full workload sizes, in the launch configuration the benchmark uses.
The oracle recomputes sampled rows / experts, or all of them where it takes seconds (each is
independent of the rest once S and H are fixed), bit-exact except the Hessian (1e-4 relative
Frobenius). The Local-Hessian searches run on the oracle's Hessians built from every
calibration token, the same data the benchmark's Hessians come from."""
import numpy as np
import pytest
import torch

from gptq_check import check_rows
from scale_search_weights_amd import nvfp4, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def case(msg):
    print(f"[case] {msg}", flush=True)


def f32(t):
    return t.detach().float().cpu().numpy()


def rel_frob(Hg, Href):
    Hg = np.asarray(Hg, np.float64).reshape(-1, 256)
    Hr = Href.reshape(-1, 256)
    return float((np.linalg.norm(Hg - Hr, axis=1) / np.linalg.norm(Hr, axis=1)).max())


def test_activation_fakequant_8192x4096(orc):
    case("activation fake-quant bf16 8192x4096 (max scaling)")
    x = synth.activation(0)
    xd = x.to(DEV)
    S = nvfp4.global_scale(xd)
    xn = f32(x)
    S_ref = orc.tensor_scale(xn)
    assert S.item() == S_ref
    y, codes, sc = nvfp4.fakequant(xd, S, return_codes=True)
    rows = np.random.default_rng(0).choice(x.shape[0], 192, replace=False)
    rows = np.concatenate([rows, [0, x.shape[0] - 1]])
    dq, cr, sr = orc.fakequant(xn[rows], S_ref)
    assert np.array_equal(sc.cpu().numpy()[rows], sr)
    assert np.array_equal(codes.cpu().numpy()[rows], cr)
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)[rows]
    assert np.array_equal(got, orc.bf16_rne_array(dq))


def test_activation_calibration_8192x4096(orc):
    case("calibration histogram and scale over the bf16 8192x4096 activation")
    x = synth.activation(0)
    xd = x.to(DEV)
    h = nvfp4.calib_histogram(xd.view(-1))
    href = orc.calib_histogram(f32(x).ravel())
    assert np.array_equal(h.cpu().numpy().view(np.uint64), href)
    for frac in (0.999, 0.9999, 1.0):
        assert nvfp4.calib_scale(h, frac).item() == orc.calib_scale(href, frac)
    # the whole range reproduces the max calibration
    assert nvfp4.calib_scale(h, 1.0).item() == nvfp4.global_scale(xd).item()


def test_mlp_weight_mse_12288x4096(orc):
    case("MSE search bf16 12288x4096 (3.1M blocks)")
    w = synth.mlp_weight(0)
    wd = w.to(DEV)
    S = nvfp4.global_scale(wd)
    wn = f32(w)
    S_ref = orc.tensor_scale(wn)
    assert S.item() == S_ref
    sc, obj = nvfp4.scale_search_mse(wd, S, return_obj=True)
    rows = np.random.default_rng(1).choice(w.shape[0], 24, replace=False)
    sr, orf = orc.scales_mse(wn[rows], S_ref, with_obj=True)
    assert np.array_equal(sc.cpu().numpy()[rows], sr)
    assert np.array_equal(obj.cpu().numpy()[rows], orf)
    # whole-tensor property: every block's MSE objective is at most its max-scaling error
    # (errors taken against the fp32 dequantised values, as the objective defines them)
    mx = nvfp4.scale_search_max(wd, S)
    codes_max, _ = nvfp4.quantize(wd, S, mx)
    y_max = nvfp4.dequantize(codes_max, mx, S, out_dtype=torch.float32)
    e_max = ((y_max - wd.float()) ** 2).view(-1, 16).sum(1)
    assert torch.all(obj.view(-1) <= e_max * (1 + 1e-5) + 1e-30)


def test_mlp_weight_four_over_six_12288x4096(orc):
    case("Four Over Six bf16 12288x4096 (3.1M blocks)")
    w = synth.mlp_weight(0)
    wd = w.to(DEV)
    S = nvfp4.global_scale(wd)
    wn = f32(w)
    S_ref = orc.tensor_scale(wn)
    assert S.item() == S_ref
    sc, obj = nvfp4.scale_search_four_over_six(wd, S, return_obj=True)
    rows = np.random.default_rng(2).choice(w.shape[0], 24, replace=False)
    sr, orf = orc.scales_four_over_six(wn[rows], S_ref, with_obj=True)
    assert np.array_equal(sc.cpu().numpy()[rows], sr)
    assert np.array_equal(obj.cpu().numpy()[rows], orf)
    # whole tensor: the exhaustive MSE objective is a lower bound (same fp32 objective over a
    # superset of candidates), the max-scaling error an upper bound
    _, obj_mse = nvfp4.scale_search_mse(wd, S, return_obj=True)
    assert torch.all(obj_mse <= obj)
    mx = nvfp4.scale_search_max(wd, S)
    codes_max, _ = nvfp4.quantize(wd, S, mx)
    y_max = nvfp4.dequantize(codes_max, mx, S, out_dtype=torch.float32)
    e_max = ((y_max - wd.float()) ** 2).view(-1, 16).sum(1)
    assert torch.all(obj.view(-1) <= e_max * (1 + 1e-5) + 1e-30)


def _search_three_ways(wd, S, Hd):
    """Local-Hessian bytes as the benchmark runs the search (no objectives, no counters),
    bytes and objectives, and the counters of a third, counting run."""
    sc_bench = nvfp4.scale_search_local_hessian(wd, S, Hd)
    sc, obj = nvfp4.scale_search_local_hessian(wd, S, Hd, return_obj=True)
    nvfp4.search_stats_read()  # clear
    nvfp4.search_stats_enable(True)
    try:
        sc_st = nvfp4.scale_search_local_hessian(wd, S, Hd)
        stats = nvfp4.search_stats_read()
    finally:
        nvfp4.search_stats_enable(False)
    assert torch.equal(sc_bench, sc) and torch.equal(sc_st, sc)
    return sc.cpu().numpy(), obj.cpu().numpy(), stats


def _report(stats, n_blocks):
    print("[info] Local-Hessian paths: " + ", ".join(f"{k} {v}" for k, v in stats.items()
                                                      if k.startswith("lh_")), flush=True)
    assert stats["lh_pairs"] + stats["lh_zero_h"] == n_blocks
    assert stats["lh_rel"] + stats["lh_abs"] <= stats["lh_pairs"]
    assert stats["lh_rescan"] <= stats["lh_pairs"]


def test_projection_hessian_and_local_hessian_full(orc):
    case("block Hessian of 131072x4096 bf16 t4 tokens + Local-Hessian on 4096x4096, "
         "both sides on the oracle's H from all 131072 tokens, every row")
    w, x = synth.projection(0)
    xd, wd = x.to(DEV), w.to(DEV)
    H = nvfp4.block_hessian(xd)
    torch.cuda.synchronize()
    Hn = H.cpu().numpy()
    del xd, H
    Href = orc.block_hessian(f32(x))  # fp64, all tokens
    assert rel_frob(Hn, Href) <= 1e-4
    del Hn
    Href = Href.astype(np.float32)
    wn = f32(w)
    S_ref = orc.tensor_scale(wn)
    S = nvfp4.global_scale(wd)
    assert S.item() == S_ref
    sc, obj, stats = _search_three_ways(wd, torch.tensor([S_ref], device=DEV),
                                        torch.from_numpy(Href).to(DEV))
    sr, orf = orc.scales_local_hessian(wn, S_ref, Href, with_obj=True)
    assert np.array_equal(sc, sr)
    assert np.array_equal(obj, orf)
    _report(stats, int((np.abs(wn).reshape(-1, 16).max(1) > 0).sum()))


def test_projection_full_hessian_and_gptq(orc):
    case("full Gram matrix of 131072x4096 bf16 (sampled); GPTQ factor and rows on 4096x4096")
    w, x = synth.projection(0)
    xd = x.to(DEV)
    H = nvfp4.full_hessian(xd)
    torch.cuda.synchronize()
    del xd
    Hn = H.cpu().numpy()
    del H
    rng = np.random.default_rng(3)
    idx = np.concatenate([[0, 4095], np.sort(rng.choice(np.arange(1, 4095), 46, replace=False))])
    sub = orc.full_hessian_blas(f32(x[:, idx]))
    d = np.sqrt(np.diag(sub))
    assert (np.abs(Hn[np.ix_(idx, idx)] - sub) <= 1e-4 * np.outer(d, d)).all()
    assert np.array_equal(Hn, Hn.T)
    del Hn
    # GPTQ on the 4096-channel layer, with H from 8192 tokens (an H the oracle forms here)
    x8 = f32(x[:8192])
    H8 = orc.full_hessian_blas(x8).astype(np.float32)
    U, status = nvfp4.gptq_factor(torch.from_numpy(H8).to(DEV), 0.01)
    Ur = orc.gptq_factor(H8.astype(np.float64), 0.01)
    assert status.item() == 0
    diff = float(np.abs(U.cpu().numpy() - Ur).max() / np.abs(Ur).max())
    print(f"[info] factor max relative difference {diff:.3g}", flush=True)
    assert diff <= 1e-7  # n eps kappa with n = 4096 and kappa <= 1 + 100 n (damping)
    del U
    wn = f32(w)
    S = orc.tensor_scale(wn)
    sc = orc.scales_max(wn, S)
    codes = nvfp4.gptq(w.to(DEV), torch.tensor([S], device=DEV), torch.from_numpy(sc).to(DEV),
                       torch.from_numpy(Ur).to(DEV)).cpu().numpy()
    rows = np.concatenate([[0, 4095], rng.choice(np.arange(1, 4095), 30, replace=False)])
    ties = check_rows(codes[rows], wn[rows], S, sc[rows], Ur, orc, tie_tol=1e-9)
    print(f"[info] near-ties followed: {ties}", flush=True)


def test_moe_routing_hessian_local_hessian_full(orc):
    case("MoE: 128 experts 512x2048, 65536 tokens top-8 Zipf(1.1); both searches on the "
         "oracle's H from every routed token; every row of 16 experts")
    w, x, ids = synth.moe(0)
    off, tok = nvfp4.route_groups(ids.to(DEV), 128)
    off_ref, tok_ref = orc.route_groups(ids.numpy(), 128)
    assert np.array_equal(off.cpu().numpy(), off_ref)
    assert np.array_equal(tok.cpu().numpy(), tok_ref)
    counts = np.diff(off_ref)
    print(f"[case] tokens per expert: min {counts.min()} median {int(np.median(counts))} max {counts.max()}",
          flush=True)
    H = nvfp4.block_hessian(x.to(DEV), group_offsets=off, token_ids=tok)
    Hn = H.cpu().numpy()
    del H
    xn = f32(x)
    Href = np.stack([orc.block_hessian(xn, tok_ref[off_ref[e]:off_ref[e + 1]]) for e in range(128)])
    assert rel_frob(Hn, Href) <= 1e-4  # every expert, every block
    del Hn
    Href = Href.astype(np.float32)
    wd = w.to(DEV)
    wn = f32(w)
    Sn = np.array([orc.tensor_scale(wn[e]) for e in range(128)], np.float32)
    assert np.array_equal(nvfp4.global_scale(wd).cpu().numpy(), Sn)
    sc, obj, stats = _search_three_ways(wd, torch.from_numpy(Sn).to(DEV), torch.from_numpy(Href).to(DEV))
    _report(stats, int((np.abs(wn).reshape(-1, 16).max(1) > 0).sum()))
    order = np.argsort(counts, kind="stable")
    picks = [int(order[-1]), int(order[64]), int(order[0])]
    rest = [e for e in np.random.default_rng(7).permutation(128) if e not in picks]
    for e in picks + [int(e) for e in rest[:13]]:
        sr, orf = orc.scales_local_hessian(wn[e], Sn[e], Href[e], with_obj=True)
        assert np.array_equal(sc[e], sr), e
        assert np.array_equal(obj[e], orf), e
