"""GPU checks at the full GPT-2 sizes, through the C ABI, against stored oracle
results (tests/golden/*.npz, written by tests/golden/make_golden.py, which
calls only the oracle), plus size-independent properties.

* GPT-2 124M fp32, B=4 T=64, 10 AdamW steps overfitting one batch (lr 1e-4,
  wd 0): per-step mean loss rel <= 1e-5; step-1 gradients (norms and samples)
  rel <= 1e-4; step-2 gradients rel-L2 <= 1e-4 per full tensor against the
  oracle evaluated at the GPU's own parameters; trajectory gradients of steps
  2..10 rel <= 3e-4 (AdamW's eps-region sensitivity, see the test); final
  sampled parameters rel-L2 <= 1e-4; the loss falls.
* GPT-2 124M bf16, B=8 T=1024, step 1 of the benchmark workload (2
  micro-steps, AdamW lr 6e-4 wd 0.1): micro-step mean losses abs <= 2e-2;
  gradient cosine >= 0.995 per tensor on tile-covering samples (every element
  of the small tensors, one per 64 x 64 block and per present token row of
  the large ones, at least 65536 per tensor); gradient norms within 1e-2;
  update cosine >= 0.95 and update signs agreeing on >= 99.8% of the
  elements whose gradient exceeds 5% of the tensor's RMS.
* GPT-2 1558M bf16, B=1 T=64 micro-step: loss abs <= 2e-2; gradient cosine
  >= 0.995 per tensor on tile-covering samples and gradient norms within
  1e-2; at B=8 T=1024 the loss at init is near
  ln V + C * 0.02^2 / 2 and falls over three small steps on one batch.
"""

import math
import os

import numpy as np
import pytest

import synthetic as S
from helpers import cosine, rel_l2, say

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    p = os.path.join(GOLDEN, name)
    if not os.path.exists(p):
        pytest.skip(f"{name} not generated (tests/golden/make_golden.py)")
    return np.load(p, allow_pickle=False)


def _samples(model, flat, g):
    out = {}
    for i, name in enumerate(S.PARAM_NAMES):
        t = flat[model.offsets[i]: model.offsets[i] + model.counts[i]]
        out[name] = t[g[f"idx_{name}"]]
    return out


def _split(cfg, g, arr):
    out, pos = {}, 0
    for name in S.PARAM_NAMES:
        n = g[f"idx_{name}"].size
        out[name] = arr[pos: pos + n]
        pos += n
    return out


def _norms(model, flat):
    return np.array([np.linalg.norm(flat[model.offsets[i]: model.offsets[i] + model.counts[i]].astype(np.float64))
                     for i in range(16)])


def _tokens(cfg, n, dev):
    import torch
    return torch.from_numpy(S.token_stream(n, cfg.vocab_size, dist="zipf")).to(dev)


def test_gpt2_124m_fp32_ten_steps_one_batch():
    import torch
    import oracle
    from transformer_lm_step_amd.model import GPT2

    g = _golden("gpt2_124m_fp32_overfit10.npz")
    cfg, B, T = S.GPT2_124M, 4, 64
    model = GPT2(cfg, 0, B, T)
    model.init(model.pack(S.init_params(cfg)))
    dev = model.device
    stream = S.token_stream(B * T + 1, cfg.vocab_size, dist="zipf")
    xb, yb = S.batch(stream, 0, B, T)
    x = torch.from_numpy(xb.reshape(-1)).to(dev)
    y = torch.from_numpy(yb.reshape(-1)).to(dev)
    mean = torch.zeros(1, dtype=torch.float32, device=dev)
    for s in range(10):
        p_before = model.params().cpu().numpy().astype(np.float64) if s == 1 else None
        model.zero_grad()
        model.forward(x, y, None, mean)
        model.backward(1.0 / (B * T))
        grads = model.grads().cpu().numpy()
        model.update(1e-4, 0.9, 0.999, 1e-8, 0.0, s + 1)
        torch.cuda.synchronize()
        lo = float(mean.cpu())
        ref = float(g["mean_loss"][s])
        say(f"124M fp32 step {s + 1}: loss {lo:.6f} oracle {ref:.6f}")
        assert abs(lo - ref) / abs(ref) < 1e-5, (s, lo, ref)
        gs = _samples(model, grads, g)
        ref_s = _split(cfg, g, g["grad_samples"][s])
        # step 1 starts from identical parameters: the kernels' own accuracy.
        # Later steps follow two trajectories (fp32 on the GPU, fp64 in the
        # oracle) whose AdamW updates differ wherever |g| is near eps;
        # tests/test_adam_sensitivity.py bounds the step-2 gradient change
        # from fp32-sized gradient noise alone by 1e-4 (measured 2-3e-5; the
        # largest drift seen here over steps 3-10 is 7.6e-5).
        tol = 1e-4 if s == 0 else 3e-4
        gn = _norms(model, grads)
        assert np.all(np.abs(gn - g["grad_norms"][s]) <= tol * g["grad_norms"][s] + 1e-30), s
        for name in S.PARAM_NAMES:
            if np.linalg.norm(ref_s[name]) == 0:
                assert np.all(gs[name] == 0), (s, name)
            else:
                assert rel_l2(gs[name], ref_s[name]) < tol, (s, name)
        if s == 1:
            # step 2 against the oracle evaluated at the GPU's own parameters
            r = oracle.gpt2_step(cfg, p_before, xb, yb, dloss=1.0 / (B * T))
            worst = 0.0
            for i, name in enumerate(S.PARAM_NAMES):
                a = grads[model.offsets[i]: model.offsets[i] + model.counts[i]]
                b = r["grads"][model.offsets[i]: model.offsets[i] + model.counts[i]]
                if name == "qkvb":
                    keep = (np.arange(a.size) % (3 * cfg.channels) < cfg.channels) | \
                           (np.arange(a.size) % (3 * cfg.channels) >= 2 * cfg.channels)
                    a, b = a[keep], b[keep]
                e = rel_l2(a, b)
                worst = max(worst, e)
                assert e < 1e-4, (name, e)
            say(f"124M fp32 step 2 at the GPU's parameters: worst full-tensor gradient rel-L2 {worst:.2e}")
    assert model.check() == 0
    ps = _samples(model, model.params().cpu().numpy(), g)
    ref_p = _split(cfg, g, g["param_samples"][-1])
    worst = max(rel_l2(ps[n], ref_p[n]) for n in S.PARAM_NAMES)
    say(f"124M fp32 final sampled params worst rel-L2 {worst:.2e}")
    assert worst < 1e-4
    assert g["mean_loss"][-1] < g["mean_loss"][0] - 0.5
    model.close()


def test_gpt2_124m_bf16_benchmark_step1():
    import torch
    from transformer_lm_step_amd.model import GPT2

    g = _golden("gpt2_124m_bf16_step1.npz")
    cfg, B, T, accum = S.GPT2_124M, 8, 1024, 2
    model = GPT2(cfg, 1, B, T)
    model.init(model.pack({k: S.round_to_bf16(v) for k, v in S.init_params(cfg).items()}))
    dev = model.device
    toks = _tokens(cfg, accum * B * T + 1, dev)
    BT = B * T
    mean = torch.zeros(accum, dtype=torch.float32, device=dev)
    model.zero_grad()
    for a in range(accum):
        model.forward(toks[a * BT:(a + 1) * BT].clone(), toks[a * BT + 1:(a + 1) * BT + 1].clone(),
                      None, mean[a:a + 1])
        model.backward(1.0 / (accum * BT))
    grads = model.grads().cpu().numpy()
    p0 = model.master().cpu().numpy().copy()
    model.update(6e-4, 0.9, 0.999, 1e-8, 0.1, 1)
    torch.cuda.synchronize()
    assert model.check() == 0
    lo = mean.cpu().numpy()
    say(f"124M bf16 step 1: micro-step losses {lo} oracle {g['mean_loss']}")
    assert np.all(np.abs(lo - g["mean_loss"]) <= 2e-2)
    gs = _samples(model, grads, g)
    ref = _split(cfg, g, g["grad_samples"])
    cos = {n: cosine(gs[n], ref[n]) for n in S.PARAM_NAMES}
    say("124M bf16 per-tensor gradient cosines (tile-covering samples)", {k: round(v, 5) for k, v in cos.items()})
    for n, c in cos.items():
        assert c >= 0.995, (n, c)
    gn = _norms(model, grads)
    ratio = gn / g["grad_norms"]
    say("124M bf16 gradient norm ratios", np.round(ratio, 5).tolist())
    assert np.all(np.abs(ratio - 1) <= 1e-2), ratio
    # The AdamW step-1 update is lr * (g / (|g| + eps) + wd * p): essentially
    # lr * sign(g), so it can differ only where the bf16 gradient error flips
    # a sign.  Where |g| > 5% of the tensor's RMS that takes an error of
    # several times the error's own RMS (the 0.995 cosine bounds it at 10% of
    # the gradient's RMS): at least 99.8% of those signs agree; over all
    # elements the update directions keep a cosine of at least 0.95 (a few
    # percent of sign flips among the smallest gradients).
    p1 = model.master().cpu().numpy()
    d_gpu = _samples(model, p1, g)
    d_p0 = _samples(model, p0, g)
    ref_p = _split(cfg, g, g["param_samples"])
    ref_p0 = _split(cfg, g, g["init_samples"])
    for n in S.PARAM_NAMES:
        assert np.array_equal(d_p0[n].astype(np.float64), ref_p0[n]), n  # same bf16-exact start
        du, dr = d_gpu[n] - d_p0[n], ref_p[n] - ref_p0[n]
        c = cosine(du, dr)
        r = ref[n].astype(np.float64)
        big = np.abs(r) > 0.05 * np.sqrt(np.mean(r * r))
        agree = float(np.mean(np.sign(du[big]) == np.sign(dr[big]))) if big.any() else 1.0
        assert c >= 0.95, (n, c)
        assert agree >= 0.998, (n, agree)
    model.close()


def test_gpt2_1558m_bf16_micro_step_b1t64():
    import torch
    from transformer_lm_step_amd.model import GPT2

    g = _golden("gpt2_1558m_bf16_b1t64.npz")
    cfg, B, T = S.GPT2_1558M, 1, 64
    model = GPT2(cfg, 1, B, T)
    model.init(model.pack({k: S.round_to_bf16(v) for k, v in S.init_params(cfg).items()}))
    dev = model.device
    toks = _tokens(cfg, B * T + 1, dev)
    mean = torch.zeros(1, dtype=torch.float32, device=dev)
    losses = torch.zeros(B * T, dtype=torch.float32, device=dev)
    model.zero_grad()
    model.forward(toks[:B * T].clone(), toks[1:].clone(), losses, mean)
    model.backward(1.0 / (B * T))
    torch.cuda.synchronize()
    assert model.check() == 0
    lo = float(mean.cpu())
    say(f"1558M bf16 B=1 T=64 loss {lo:.5f} oracle {float(g['mean_loss'][0]):.5f}")
    assert abs(lo - float(g["mean_loss"][0])) <= 2e-2
    assert np.max(np.abs(losses.cpu().numpy() - g["losses"].ravel())) < 0.1
    grads = model.grads().cpu().numpy()
    gs = _samples(model, grads, g)
    ref = _split(cfg, g, g["grad_samples"])
    cos = {n: cosine(gs[n], ref[n]) for n in S.PARAM_NAMES}
    say("1558M bf16 per-tensor gradient cosines (tile-covering samples)", {k: round(v, 5) for k, v in cos.items()})
    for n, c in cos.items():
        assert c >= 0.995, (n, c)
    ratio = _norms(model, grads) / g["grad_norms"]
    say("1558M bf16 gradient norm ratios", np.round(ratio, 5).tolist())
    assert np.all(np.abs(ratio - 1) <= 1e-2), ratio
    model.close()


def test_gpt2_1558m_bf16_full_size_steps():
    """All activations resident at B=8 T=1024: loss at init, and its descent
    over three small AdamW steps (lr 1e-5) on one batch."""
    import torch
    from transformer_lm_step_amd.model import GPT2

    cfg, B, T = S.GPT2_1558M, 8, 1024
    model = GPT2(cfg, 1, B, T)
    model.init(model.pack({k: S.round_to_bf16(v) for k, v in S.init_params(cfg).items()}))
    dev = model.device
    toks = _tokens(cfg, B * T + 1, dev)
    x, y = toks[:B * T].clone(), toks[1:].clone()
    mean = torch.zeros(4, dtype=torch.float32, device=dev)
    for s in range(3):
        model.zero_grad()
        model.forward(x, y, None, mean[s:s + 1])
        model.backward(0.0)
        model.update(1e-5, 0.9, 0.999, 1e-8, 0.0, s + 1)
    model.forward(x, y, None, mean[3:4])
    torch.cuda.synchronize()
    assert model.check() == 0
    lo = mean.cpu().numpy()
    expect = math.log(cfg.vocab_size) + cfg.channels * 0.02 ** 2 / 2
    say(f"1558M bf16 losses {lo} (init expectation {expect:.3f})")
    assert np.all(np.isfinite(lo))
    assert abs(lo[0] - expect) < 0.2
    assert lo[3] < lo[0] - 0.01
    model.close()
