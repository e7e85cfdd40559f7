"""Seeded synthetic inputs for the NVFP4 engine and for its CPU oracle.

This module only draws random numbers and shapes them into tensors; it contains none of
the quantisation arithmetic, so the HIP path and the oracle can both be fed from it
without sharing any of the method.

The workloads stand in for one layer of the models the pages quantise (no checkpoints or
datasets are used):

* ``tiny``        W 64x256 fp32 ~N(0, 0.02) with 1% of entries x20; calibration
                  activations X [512 tokens x 256 channels] ~N(0, 1) with 4 channels x10.
* ``activation``  bf16 activations [8192 tokens x 4096], Student-t (nu=3) scaled to unit
                  variance, 8 fixed outlier channels x30.
* ``mlp_weight``  bf16 weight [12288 x 4096] ~N(0, 0.015) with 0.1% of entries x25.
* ``projection``  bf16 weight [4096 x 4096] ~N(0, 0.02) and bf16 calibration activations
                  [131072 tokens x 4096], Student-t (nu=4), 16 outlier channels x20.
* ``moe``         128 bf16 expert weights [512 x 2048] ~N(0, 0.02), bf16 tokens
                  [65536 x 2048] ~N(0, 1), each token routed to 8 distinct experts drawn
                  with probability proportional to (e+1)^-1.1 (Gumbel top-k).

Every generator takes the sizes as arguments so tests can draw smaller tensors with the
same distributions. Draws are made in fp32 in fixed 4M-element chunks, each from its own
PCG64 stream spawned from the seed, so the result does not depend on the thread count.
bf16 tensors are the fp32 draws rounded to nearest-even by torch.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

_CHUNK = 1 << 22


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _chunked(seed_seq: np.random.SeedSequence, n: int, fill) -> np.ndarray:
    """Fill an fp32 vector of length n chunk by chunk, chunk i from spawned stream i."""
    out = np.empty(n, dtype=np.float32)
    nchunks = (n + _CHUNK - 1) // _CHUNK
    seqs = seed_seq.spawn(nchunks)

    def work(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        out[lo:hi] = fill(np.random.default_rng(seqs[i]), hi - lo)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def _normal(seed_seq, n, sigma):
    return _chunked(seed_seq, n, lambda g, m: g.standard_normal(m, dtype=np.float32) * np.float32(sigma))


def _student_t(seed_seq, n, nu):
    """Student-t with nu degrees of freedom: Z / sqrt(V / nu), V ~ chi^2_nu = 2 Gamma(nu/2)."""
    def fill(g, m):
        z = g.standard_normal(m, dtype=np.float32)
        v = g.standard_gamma(nu / 2.0, size=m, dtype=np.float32) * np.float32(2.0 / nu)
        return z / np.sqrt(v)
    return _chunked(seed_seq, n, fill)


def _streams(seed: int, k: int):
    return np.random.SeedSequence(seed).spawn(k)


def _bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(a).to(torch.bfloat16)


def tiny(seed: int = 0, rows: int = 64, cols: int = 256, tokens: int = 512):
    """Returns (W fp32 [rows, cols], X fp32 [tokens, cols])."""
    s = _streams(seed, 4)
    w = _normal(s[0], rows * cols, 0.02)
    n_out = int(round(0.01 * rows * cols))
    idx = np.random.default_rng(s[1]).choice(rows * cols, size=n_out, replace=False)
    w[idx] *= np.float32(20.0)
    x = _normal(s[2], tokens * cols, 1.0).reshape(tokens, cols)
    ch = np.random.default_rng(s[3]).choice(cols, size=min(4, cols), replace=False)
    x[:, ch] *= np.float32(10.0)
    return torch.from_numpy(w.reshape(rows, cols)), torch.from_numpy(x)


def activation(seed: int = 0, tokens: int = 8192, hidden: int = 4096) -> torch.Tensor:
    """bf16 [tokens, hidden]: Student-t(3)/sqrt(3) (unit variance), 8 channels x30."""
    s = _streams(seed, 2)
    a = _student_t(s[0], tokens * hidden, 3.0) * np.float32(1.0 / np.sqrt(3.0))
    a = a.reshape(tokens, hidden)
    ch = np.random.default_rng(s[1]).choice(hidden, size=min(8, hidden), replace=False)
    a[:, ch] *= np.float32(30.0)
    return _bf16(a)


def mlp_weight(seed: int = 0, rows: int = 12288, cols: int = 4096) -> torch.Tensor:
    """bf16 [rows, cols] ~N(0, 0.015) with 0.1% of the entries x25."""
    s = _streams(seed, 2)
    w = _normal(s[0], rows * cols, 0.015)
    n_out = int(round(0.001 * rows * cols))
    idx = np.random.default_rng(s[1]).choice(rows * cols, size=n_out, replace=False)
    w[idx] *= np.float32(25.0)
    return _bf16(w.reshape(rows, cols))


def projection(seed: int = 0, rows: int = 4096, cols: int = 4096, tokens: int = 131072):
    """Returns (W bf16 [rows, cols] ~N(0, 0.02), X bf16 [tokens, cols] Student-t(4), 16 ch x20)."""
    s = _streams(seed, 3)
    w = _normal(s[0], rows * cols, 0.02).reshape(rows, cols)
    x = _student_t(s[1], tokens * cols, 4.0).reshape(tokens, cols)
    ch = np.random.default_rng(s[2]).choice(cols, size=min(16, cols), replace=False)
    x[:, ch] *= np.float32(20.0)
    return _bf16(w), _bf16(x)


def moe(seed: int = 0, experts: int = 128, rows: int = 512, cols: int = 2048,
        tokens: int = 65536, topk: int = 8, zipf: float = 1.1):
    """Returns (W bf16 [experts, rows, cols], X bf16 [tokens, cols], expert_ids int32 [tokens, topk]).

    Each token picks ``topk`` distinct experts; expert e is drawn with probability
    proportional to (e+1)^-zipf, sampled without replacement by Gumbel top-k.
    """
    s = _streams(seed, 3)
    w = _normal(s[0], experts * rows * cols, 0.02).reshape(experts, rows, cols)
    x = _normal(s[1], tokens * cols, 1.0).reshape(tokens, cols)
    g = np.random.default_rng(s[2])
    logits = -zipf * np.log(np.arange(1, experts + 1, dtype=np.float64))
    ids = np.empty((tokens, topk), dtype=np.int32)
    step = 8192
    for lo in range(0, tokens, step):
        hi = min(tokens, lo + step)
        u = g.random((hi - lo, experts))
        score = logits[None, :] - np.log(-np.log(u))
        top = np.argpartition(-score, topk - 1, axis=1)[:, :topk]
        order = np.argsort(-np.take_along_axis(score, top, axis=1), axis=1, kind="stable")
        ids[lo:hi] = np.take_along_axis(top, order, axis=1)
    return _bf16(w), _bf16(x), torch.from_numpy(ids)


def on_grid_block_values(seed: int, n: int) -> np.ndarray:
    """fp32 values that are small dyadic rationals (multiples of 1/16 in [-8, 8]).

    With tensor scale 1 and block scale 1.0 many of them sit exactly on E2M1 grid points
    or on the midpoints between them, which exercises the round-half-to-even rule.
    """
    g = np.random.default_rng(seed)
    return (g.integers(-128, 129, size=n).astype(np.float32) / np.float32(16.0))
