#!/usr/bin/env python3
"""Writes the stored oracle results that the full-size GPU tests compare
against.  Calls only ``oracle`` (and the seeded input generator
``synthetic``); nothing here touches the HIP library.

    python tests/golden/make_golden.py c2     # GPT-2 124M fp32, 10 steps on one batch
    python tests/golden/make_golden.py c4     # GPT-2 124M bf16-init, step 1 at B=8 T=1024
    python tests/golden/make_golden.py c5     # GPT-2 1558M bf16-init, one micro-step at B=1 T=64

Sequences of a batch are independent in the forward pass, and the batch
gradient is the sum of per-sequence gradients, so each sequence runs in its
own worker process (``--jobs``); gradients are summed in sequence order.

Stored per case (numpy .npz, plain arrays): the mean losses, the per-position
losses, per-tensor gradient L2 norms, the gradients and the AdamW-updated
parameters at seeded sample indices per tensor (key-bias elements of qkvb
excluded: their exact gradient is zero and both sides carry only round-off).

Samples: the 124M fp32 case takes 1024 seeded indices per tensor.  The
124M bf16 benchmark step and the 1558M micro-step take tile-covering samples
(tile_samples):
every element of tensors up to 65536 elements; for larger ones one element
in every 64 x 64 block of each layer's matrix (finer than any output tile of
the weight-gradient products), for wte one element in every row whose token
occurs in the step's batches, topped up with seeded random elements to at
least 65536 per tensor.  Their gradients are stored as float32.
"""

from __future__ import annotations

import argparse
import multiprocessing as mp
import os
import sys
import time

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import synthetic as S  # noqa: E402

SAMPLES = 1024
SAMPLE_SEED = 2024

_W = {}


def sample_indices(cfg):
    """Per tensor (in parameter order) sorted flat indices into that tensor."""
    shapes = S.param_shapes(cfg)
    rng = np.random.default_rng(SAMPLE_SEED)
    out = {}
    for name in S.PARAM_NAMES:
        n = int(np.prod(shapes[name]))
        allowed = np.arange(n)
        if name == "qkvb":
            L, C = cfg.num_layers, cfg.channels
            allowed = allowed[(allowed % (3 * C) < C) | (allowed % (3 * C) >= 2 * C)]
        k = min(SAMPLES, allowed.size)
        out[name] = np.sort(rng.choice(allowed, k, replace=False)).astype(np.int64)
    return out


FULL_MAX = 65536  # tensors up to this size are stored whole
BLOCK = 64        # one sample per BLOCK x BLOCK block of a layer's matrix


def tile_samples(cfg, tokens):
    """Per tensor (in parameter order) sorted flat int32 indices: see the
    module docstring.  tokens: every token id of the step's batches."""
    shapes = S.param_shapes(cfg)
    rng = np.random.default_rng(SAMPLE_SEED + 1)
    L, C = cfg.num_layers, cfg.channels
    out = {}
    for name in S.PARAM_NAMES:
        shape = shapes[name]
        n = int(np.prod(shape))
        allowed = None
        if name == "qkvb":
            a = np.arange(n)
            allowed = (a % (3 * C) < C) | (a % (3 * C) >= 2 * C)
        if n <= FULL_MAX:
            idx = np.arange(n) if allowed is None else np.nonzero(allowed)[0]
            out[name] = idx.astype(np.int32)
            continue
        rows, cols = int(np.prod(shape[:-1])), shape[-1]
        sel = set()
        # one element per BLOCK x BLOCK block (layers are stacked along rows;
        # every per-layer row count here is a multiple of BLOCK)
        for r0 in range(0, rows, BLOCK):
            nr = min(BLOCK, rows - r0)
            for c0 in range(0, cols, BLOCK):
                nc = min(BLOCK, cols - c0)
                sel.add((r0 + int(rng.integers(nr))) * cols + c0 + int(rng.integers(nc)))
        if name == "wte":
            for t in np.unique(tokens):
                sel.add(int(t) * cols + int(rng.integers(cols)))
        while len(sel) < FULL_MAX:
            sel.update(int(x) for x in rng.integers(0, n, FULL_MAX - len(sel)))
        out[name] = np.array(sorted(sel), np.int32)
    return out


def _init_worker(cfg, flat):
    _W["cfg"], _W["flat"] = cfg, flat


def _seq_job(job):
    x, y, dloss, want_grads = job
    r = oracle.gpt2_step(_W["cfg"], _W["flat"], x[None, :], y[None, :], dloss=dloss, want_grads=want_grads)
    return r["losses"][0], r["grads"]


def run_batch(pool, batch, dloss, want_grads, grads=None):
    """Per-sequence oracle calls; returns (losses [B,T], grads summed in order)."""
    x, y = batch
    jobs = [(x[b], y[b], dloss, want_grads) for b in range(x.shape[0])]
    losses = []
    for lo, g in pool.imap(_seq_job, jobs, chunksize=1):
        losses.append(lo)
        if want_grads:
            if grads is None:
                grads = g
            else:
                grads += g
        print(f"  sequence {len(losses)}/{len(jobs)} done", flush=True)
    return np.stack(losses), grads


def norms_and_samples(cfg, flat, idx, dtype=np.float64):
    off, cnt, _ = oracle.param_layout(cfg)
    norms, samp = [], []
    for i, name in enumerate(S.PARAM_NAMES):
        t = flat[off[i]:off[i] + cnt[i]]
        norms.append(np.linalg.norm(t))
        samp.append(t[idx[name]].astype(dtype))
    return np.array(norms), np.concatenate(samp)


def case_c2(jobs):
    """10 AdamW steps (lr 1e-4, wd 0) on one fixed batch, B=4 T=64, fp32 init."""
    cfg, B, T, steps = S.GPT2_124M, 4, 64, 10
    params = S.init_params(cfg)
    flat = oracle.pack_params(cfg, params)
    stream = S.token_stream(B * T + 1, cfg.vocab_size, dist="zipf")
    batch = S.batch(stream, 0, B, T)
    idx = sample_indices(cfg)
    m = np.zeros_like(flat); v = np.zeros_like(flat)
    means, losses, gnorms, gsamp, psamp = [], [], [], [], []
    for s in range(steps):
        t0 = time.time()
        with mp.get_context("fork").Pool(jobs, initializer=_init_worker, initargs=(cfg, flat)) as pool:
            lo, g = run_batch(pool, batch, 1.0 / (B * T), True)
        means.append(lo.mean()); losses.append(lo)
        n, smp = norms_and_samples(cfg, g, idx)
        gnorms.append(n); gsamp.append(smp)
        flat, m, v = oracle.adamw(flat, g, m, v, 1e-4, 0.9, 0.999, 1e-8, 0.0, s + 1)
        psamp.append(norms_and_samples(cfg, flat, idx)[1])
        print(f"c2 step {s + 1}: loss {means[-1]:.6f} ({time.time() - t0:.0f} s)", flush=True)
    np.savez_compressed(os.path.join(HERE, "gpt2_124m_fp32_overfit10.npz"),
                        mean_loss=np.array(means), losses=np.stack(losses), grad_norms=np.stack(gnorms),
                        grad_samples=np.stack(gsamp), param_samples=np.stack(psamp),
                        **{f"idx_{k}": v_ for k, v_ in idx.items()})


def case_c4(jobs):
    """Step 1 of the bf16 benchmark workload: 2 micro-steps of B=8 T=1024
    (dloss = 1/(2 B T)) from the bf16-rounded init, then AdamW (lr 6e-4,
    wd 0.1, t = 1) on the fp32 master copy."""
    cfg, B, T, accum = S.GPT2_124M, 8, 1024, 2
    params = {k: S.round_to_bf16(v_) for k, v_ in S.init_params(cfg).items()}
    flat = oracle.pack_params(cfg, params)
    stream = S.token_stream(accum * B * T + 1, cfg.vocab_size, dist="zipf")
    idx = tile_samples(cfg, stream[:accum * B * T])
    print("c4 samples per tensor:", {k: int(v.size) for k, v in idx.items()}, flush=True)
    grads, means, losses = None, [], []
    with mp.get_context("fork").Pool(jobs, initializer=_init_worker, initargs=(cfg, flat)) as pool:
        for a in range(accum):
            lo, grads = run_batch(pool, S.batch(stream, a, B, T), 1.0 / (accum * B * T), True, grads)
            means.append(lo.mean()); losses.append(lo)
            print(f"c4 micro-step {a + 1}: loss {means[-1]:.6f}", flush=True)
    # gradients as float32 (far finer than the bf16 step's accuracy); updated
    # and initial parameters as float64 (the update is a small difference)
    gn, gs = norms_and_samples(cfg, grads, idx, np.float32)
    newp, _, _ = oracle.adamw(flat, grads, np.zeros_like(flat), np.zeros_like(flat), 6e-4, 0.9, 0.999, 1e-8, 0.1, 1)
    ps = norms_and_samples(cfg, newp, idx)[1]
    p0 = norms_and_samples(cfg, flat, idx)[1]
    np.savez_compressed(os.path.join(HERE, "gpt2_124m_bf16_step1.npz"),
                        mean_loss=np.array(means), losses=np.stack(losses), grad_norms=gn, grad_samples=gs,
                        param_samples=ps, init_samples=p0, **{f"idx_{k}": v_ for k, v_ in idx.items()})


def case_c5(jobs):
    """GPT-2 1558M from the bf16-rounded init, one micro-step at B=1 T=64:
    forward losses, gradient norms and sampled gradients."""
    cfg, B, T = S.GPT2_1558M, 1, 64
    params = {k: S.round_to_bf16(v_) for k, v_ in S.init_params(cfg).items()}
    flat = oracle.pack_params(cfg, params)
    del params
    stream = S.token_stream(B * T + 1, cfg.vocab_size, dist="zipf")
    x, y = S.batch(stream, 0, B, T)
    idx = tile_samples(cfg, x.ravel())
    print("c5 samples per tensor:", {k: int(v.size) for k, v in idx.items()}, flush=True)
    r = oracle.gpt2_step(cfg, flat, x, y, dloss=1.0 / (B * T))
    gn, gs = norms_and_samples(cfg, r["grads"], idx, np.float32)
    print(f"c5 loss {r['mean_loss']:.6f}", flush=True)
    np.savez_compressed(os.path.join(HERE, "gpt2_1558m_bf16_b1t64.npz"),
                        mean_loss=np.array([r["mean_loss"]]), losses=r["losses"], grad_norms=gn, grad_samples=gs,
                        **{f"idx_{k}": v_ for k, v_ in idx.items()})


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("case", choices=("c2", "c4", "c5"))
    ap.add_argument("--jobs", type=int, default=4)
    a = ap.parse_args()
    oracle.build()
    {"c2": case_c2, "c4": case_c4, "c5": case_c5}[a.case](a.jobs)


if __name__ == "__main__":
    main()
