"""How far two GPT-2 124M fp32 trajectories (B=4, T=64, one batch, AdamW
lr 1e-4, wd 0) drift apart after step 1 from fp32-sized gradient differences
alone -- the reading that sets the tolerance of the ten-step GPU test on
steps 3-10 (tests/test_gpu_full_size.py).  Calls only the oracle (CPU).

At step 1 AdamW's bias-corrected moments are m = g and v = g^2, so an
element's update is lr * g / (|g| + eps): for |g| of the order of eps (1e-8)
the update follows g itself, and an absolute gradient error of fp32 size
moves it by up to lr.  The test perturbs the step-1 gradient by seeded
Gaussian noise of 1e-6 x each tensor's RMS (the size of an fp32 kernel's
error), applies AdamW to both, and measures the step-2 gradient change on the
sampled elements the GPU test compares: it must be visible (> 1e-6: the
trajectories really diverge) and at most 1e-4, a third of the 3e-4 the GPU
test allows on its trajectory gradients.
"""

import multiprocessing as mp
import os
import sys

import numpy as np
import pytest

import synthetic as S

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))

pytestmark = pytest.mark.slow


def test_step2_gradient_drift_from_fp32_noise_is_bounded():
    import oracle
    import make_golden as G

    cfg, B, T = S.GPT2_124M, 4, 64
    flat0 = oracle.pack_params(cfg, S.init_params(cfg))
    batch = S.batch(S.token_stream(B * T + 1, cfg.vocab_size, dist="zipf"), 0, B, T)
    idx = G.sample_indices(cfg)
    off, cnt, _ = oracle.param_layout(cfg)

    def grads_at(flat):
        with mp.get_context("fork").Pool(4, initializer=G._init_worker, initargs=(cfg, flat)) as pool:
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
    g2, g2n = grads_at(p1), grads_at(p1n)
    worst = 0.0
    for i, n in enumerate(S.PARAM_NAMES):
        if n == "qkvb":
            continue  # key-bias gradient is round-off on both sides
        a, b = g2[off[i]:off[i] + cnt[i]][idx[n]], g2n[off[i]:off[i] + cnt[i]][idx[n]]
        e = np.linalg.norm(a - b) / np.linalg.norm(a)
        print(f"{n:9s} step-2 sampled gradient rel-L2 change {e:.2e}")
        worst = max(worst, e)
    assert 1e-6 < worst <= 1e-4, worst
