"""The allocation-free block Hessian (nvfp4_block_hessian_noalloc) against the workspace
entry point (nvfp4_block_hessian), both called through the C ABI: the same kernels on the
same inputs, so the Hessians must be identical bit for bit (the parity bar for the block
Hessian is 1e-4 relative Frobenius error against the oracle; here both sides are the GPU).
Calls come in a row on the shared static scratch, the later ones smaller, so each sees the
contents the previous call left there."""
import ctypes

import numpy as np
import pytest
import torch

from scale_search_weights_amd import nvfp4, synth

pytestmark = pytest.mark.gpu
DEV = "cuda"


def case(msg):
    print(f"[case] {msg}", flush=True)


def P(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _both(x, offsets=None, ids=None, groups=1, H0=None):
    """H from the workspace entry point and from the allocation-free one (same accumulate
    start H0 when given)."""
    L = nvfp4.lib()
    tokens, cols = x.shape
    n_ids = ids.numel() if ids is not None else 0
    shape = (groups, cols // 16, 16, 16) if offsets is not None else (cols // 16, 16, 16)
    acc = 0 if H0 is None else 1
    Ha = torch.empty(shape, dtype=torch.float32, device=DEV) if H0 is None else H0.clone()
    Hb = torch.full(shape, float("nan"), dtype=torch.float32, device=DEV) if H0 is None else H0.clone()
    need = L.nvfp4_block_hessian_workspace_size(tokens, cols, groups, n_ids)
    assert need <= nvfp4.STATIC_SCRATCH_BYTES
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=DEV)
    st = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    dt = nvfp4.DTYPE_BF16 if x.dtype == torch.bfloat16 else nvfp4.DTYPE_F32
    rc = L.nvfp4_block_hessian(P(x), dt, tokens, cols, groups, P(offsets), P(ids), n_ids, P(Ha),
                               acc, P(ws), ws.numel(), st)
    assert rc == 0, nvfp4.status_string(rc)
    rc = L.nvfp4_block_hessian_noalloc(P(x), dt, tokens, cols, groups, P(offsets), P(ids), n_ids,
                                       P(Hb), acc, st)
    assert rc == 0, nvfp4.status_string(rc)
    torch.cuda.synchronize()
    return Ha, Hb


def test_noalloc_block_hessian_matches_workspace_form():
    # 1. grouped (MoE-shaped: 32 experts, 8192 tokens top-4, Zipf routing), the largest call
    case("no-alloc block Hessian: grouped, 32 experts, 8192 tokens x 1024, top-4")
    _, x, ids = synth.moe(3, experts=32, rows=16, cols=1024, tokens=8192, topk=4)
    off, tok = nvfp4.route_groups(ids.to(DEV), 32)
    Ha, Hb = _both(x.to(DEV), off, tok, groups=32)
    assert torch.equal(Ha, Hb)
    # 2. dense bf16, smaller
    case("no-alloc block Hessian: dense bf16, 3000 tokens x 512")
    xd = synth.projection(5, rows=16, cols=512, tokens=3000)[1].to(DEV)
    Ha, Hb = _both(xd)
    assert torch.equal(Ha, Hb)
    # 3. accumulate onto that H with another, still smaller fp32 batch
    case("no-alloc block Hessian: dense fp32 accumulate, 700 tokens x 512")
    x2 = torch.from_numpy(np.random.default_rng(8).standard_normal((700, 512)).astype(np.float32)).to(DEV)
    Ha2, Hb2 = _both(x2, H0=Ha)
    assert torch.equal(Ha2, Hb2)
    assert not torch.equal(Ha2, Ha)


def test_noalloc_block_hessian_rejects_oversize():
    case("no-alloc block Hessian: a call needing more than the static scratch")
    L = nvfp4.lib()
    tokens, cols = 1 << 20, 16384
    assert L.nvfp4_block_hessian_workspace_size(tokens, cols, 1, 0) > nvfp4.STATIC_SCRATCH_BYTES
    x = torch.empty(16, dtype=torch.bfloat16, device=DEV)   # never read: rejected first
    H = torch.empty(16, dtype=torch.float32, device=DEV)
    rc = L.nvfp4_block_hessian_noalloc(P(x), nvfp4.DTYPE_BF16, tokens, cols, 1, None, None, 0,
                                       P(H), 0, None)
    assert rc == 5  # NVFP4_ERR_WORKSPACE
