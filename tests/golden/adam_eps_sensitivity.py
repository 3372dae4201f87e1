#!/usr/bin/env python3
"""How sensitive is the second step's gradient of the GPT-2 124M fp32 run
(B=4, T=64, one batch, AdamW lr 1e-4, wd 0) to fp32-level noise in the first
step's gradient?  Calls only the oracle.

At step 1 AdamW's bias-corrected moments are m = g and v = g^2, so an
element's update is lr * g / (|g| + eps): for |g| of the order of eps (1e-8)
it moves with g itself, so an absolute gradient error of fp32 size (1e-6 of a
tensor's RMS) changes the update of such elements by up to lr.  This script
perturbs the step-1 gradient by exactly that (seeded Gaussian noise, 1e-6 x
each tensor's RMS), applies AdamW, and reports how far the step-2 gradients
move -- the part of a GPU-vs-oracle trajectory difference that no kernel
accuracy can remove.

    python tests/golden/adam_eps_sensitivity.py [--jobs 4]
"""
import argparse
import multiprocessing as mp
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import synthetic as S  # noqa: E402
import make_golden as G  # noqa: E402


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    jobs = ap.parse_args().jobs
    oracle.build()
    cfg, B, T = S.GPT2_124M, 4, 64
    flat0 = oracle.pack_params(cfg, S.init_params(cfg))
    batch = S.batch(S.token_stream(B * T + 1, cfg.vocab_size, dist="zipf"), 0, B, T)
    idx = G.sample_indices(cfg)
    off, cnt, _ = oracle.param_layout(cfg)

    def grads_at(flat):
        with mp.get_context("fork").Pool(jobs, initializer=G._init_worker, initargs=(cfg, flat)) as pool:
            return G.run_batch(pool, batch, 1.0 / (B * T), True)[1]

    g1 = grads_at(flat0)
    rng = np.random.default_rng(1)
    g1n = g1.copy()
    for i in range(16):
        t = g1[off[i]:off[i] + cnt[i]]
        g1n[off[i]:off[i] + cnt[i]] = t + 1e-6 * np.sqrt(np.mean(t * t)) * rng.standard_normal(t.size)
    z = np.zeros_like(flat0)
    p1, _, _ = oracle.adamw(flat0, g1, z, z, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1)
    p1n, _, _ = oracle.adamw(flat0, g1n, z, z, 1e-4, 0.9, 0.999, 1e-8, 0.0, 1)
    d = np.abs(p1 - p1n)
    print(f"step-1 updates changed by > 1e-7: {int((d > 1e-7).sum())} of {d.size}; largest {d.max():.2e}")
    g2, g2n = grads_at(p1), grads_at(p1n)
    for i, n in enumerate(S.PARAM_NAMES):
        a, b = g2[off[i]:off[i] + cnt[i]][idx[n]], g2n[off[i]:off[i] + cnt[i]][idx[n]]
        print(f"{n:9s} step-2 sampled gradient rel-L2 change: {np.linalg.norm(a - b) / np.linalg.norm(a):.2e}")


if __name__ == "__main__":
    main()
