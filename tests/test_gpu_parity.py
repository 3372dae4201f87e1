"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on the
same seeded inputs.

Bars (fp32): loss rel <= 1e-5; every gradient tensor rel-L2 <= 1e-4; every
updated parameter tensor and AdamW moment rel-L2 <= 1e-4.
Bars (bf16): loss abs <= 2e-2; gradient cosine >= 0.995 per tensor.
Token gather / causal mask / padded vocabulary: bit-exact (see test_gpu_exact).
"""

import math

import numpy as np
import pytest

import synthetic as S
from helpers import PARAM_NAMES, cosine, gpu_step, make_inputs, oracle_step, rel_l2, say

pytestmark = pytest.mark.gpu

# several tiles and ragged tails: BT = 300 (128-row tiles), T = 150 (64-row
# attention blocks), Vp = 1000 (128-column tiles), head size 64 and 32
RAGGED64 = S.Config(max_seq_len=160, vocab_size=997, padded_vocab_size=1000, num_layers=2, num_heads=3, channels=192)
RAGGED32 = S.Config(max_seq_len=160, vocab_size=997, padded_vocab_size=1000, num_layers=1, num_heads=6, channels=192)
# T a multiple of 64 with several full key blocks before the diagonal one
BLOCKS64 = S.Config(max_seq_len=256, vocab_size=500, padded_vocab_size=512, num_layers=1, num_heads=2, channels=128)

# B*T = 8192 rows with C = 800: the qkv (N = 2400) and fc (N = 3200) forward
# products and the N = 800 projections run on 256x192 tiles whose last column
# tile is ragged (bias, bias + GELU and bias + residual epilogues)
WIDE = S.Config(max_seq_len=1024, vocab_size=997, padded_vocab_size=1000, num_layers=1, num_heads=25, channels=800)
# C = 576 at B*T = 8192: the fc product (8192 x 2304, with its GELU
# epilogue) runs on the 256 x 288 tile
WIDE576 = S.Config(max_seq_len=1024, vocab_size=997, padded_vocab_size=1000, num_layers=1, num_heads=9, channels=576)

# 64 layers: 129 LayerNorm backwards, more than one launch of their
# parameter-gradient reduction takes (128)
DEEP = S.Config(max_seq_len=16, vocab_size=128, padded_vocab_size=128, num_layers=64, num_heads=2, channels=64)

FP32_CASES = [
    ("tiny", S.TINY, 4, 64, False),
    ("tiny-perturbed", S.TINY, 4, 64, True),
    ("ragged-hs64", RAGGED64, 2, 150, True),
    ("ragged-hs32", RAGGED32, 3, 100, True),
    ("blocks-hs64", BLOCKS64, 2, 256, True),
    ("deep-l64", DEEP, 2, 16, True),
]


def key_bias_mask(cfg):
    """Elements of qkvb that are key biases.  Their gradient is exactly zero in
    exact arithmetic: adding the same q.b_k to every score of a softmax row
    changes nothing.  Adam divides by the gradient's magnitude, so the update
    of those elements is set by round-off on both sides and is compared only
    for being bounded by the learning rate."""
    L, C = cfg.num_layers, cfg.channels
    m = np.zeros((L, 3 * C), bool)
    m[:, C:2 * C] = True
    return m.ravel()


def _check_key_bias(cfg, o, g, lr):
    kb = key_bias_mask(cfg)
    go, gg = o["grads"]["qkvb"].ravel(), g["grads"]["qkvb"].ravel()
    scale = np.abs(go[~kb]).max()
    assert np.abs(go[kb]).max() <= 1e-12 * max(scale, 1.0)
    assert np.abs(gg[kb]).max() <= 1e-5 * scale
    return kb


def _compare_fp32(name, o, g, n_micro=1, cfg=None, lr=1e-4, p0=None):
    kb = _check_key_bias(cfg, o, g, lr)
    d = g["params"]["qkvb"].ravel()[kb] - p0["qkvb"].astype(np.float64).ravel()[kb]
    assert np.all(np.abs(d) <= lr * 1.001 + 1e-12)
    for i in range(n_micro):
        lo, lg = np.asarray(o["losses"][i]), g["losses"][i]
        assert np.max(np.abs(lg - lo) / np.abs(lo)) < 1e-5, (name, "per-position loss")
        assert abs(g["means"][i] - o["means"][i]) / abs(o["means"][i]) < 1e-5, (name, "mean loss")
    worst = {}
    for key in ("grads", "params", "m", "v"):
        for p in PARAM_NAMES:
            a, b = np.ravel(g[key][p]), np.ravel(o[key][p])
            if p == "qkvb" and key != "grads":
                a, b = a[~kb], b[~kb]
            e = rel_l2(a, b)
            worst[f"{key}.{p}"] = e
            assert e < 1e-4, (name, key, p, e)
    say(name, "worst rel-L2", max(worst.items(), key=lambda kv: kv[1]))


@pytest.mark.parametrize("name,cfg,B,T,perturb", FP32_CASES, ids=[c[0] for c in FP32_CASES])
def test_fp32_step_matches_oracle(name, cfg, B, T, perturb):
    say("case", name, "fp32", B, T)
    params, batches = make_inputs(cfg, B, T, perturb=perturb)
    o = oracle_step(cfg, params, batches, lr=1e-4)
    g = gpu_step(cfg, 0, params, batches, lr=1e-4)
    assert g["code"] == 0
    _compare_fp32(name, o, g, cfg=cfg, lr=1e-4, p0=params)
    # padded vocabulary rows: zero gradient, unchanged (zero) parameters
    V = cfg.vocab_size
    assert np.all(g["grads"]["wte"].reshape(cfg.padded_vocab_size, -1)[V:] == 0.0)
    assert np.all(g["params"]["wte"].reshape(cfg.padded_vocab_size, -1)[V:] == 0.0)


def test_fp32_grad_accumulation_and_weight_decay():
    cfg = RAGGED64
    say("case fp32 accumulation", cfg)
    params, batches = make_inputs(cfg, 2, 96, n_micro=2, perturb=True)
    dloss = 1.0 / (2 * 2 * 96)
    o = oracle_step(cfg, params, batches, dloss=dloss, lr=6e-4, wd=0.1)
    g = gpu_step(cfg, 0, params, batches, dloss=dloss, lr=6e-4, wd=0.1)
    _compare_fp32("accum", o, g, n_micro=2, cfg=cfg, lr=6e-4, p0=params)


@pytest.mark.parametrize("name,cfg,B,T,perturb", FP32_CASES[1:3], ids=[c[0] for c in FP32_CASES[1:3]])
def test_bf16_step_matches_oracle(name, cfg, B, T, perturb):
    say("case", name, "bf16", B, T)
    params, batches = make_inputs(cfg, B, T, perturb=perturb, bf16=True)
    o = oracle_step(cfg, params, batches, lr=1e-4)
    g = gpu_step(cfg, 1, params, batches, lr=1e-4)
    assert g["code"] == 0
    assert abs(g["means"][0] - o["means"][0]) <= 2e-2
    assert np.max(np.abs(g["losses"][0] - o["losses"][0])) <= 2e-2 * 4
    cos = {p: cosine(g["grads"][p], o["grads"][p]) for p in PARAM_NAMES}
    say(name, "min grad cosine", min(cos.items(), key=lambda kv: kv[1]))
    for p, c in cos.items():
        assert c >= 0.995, (p, c)
    # the AdamW update direction: cosine of (p1 - p0) per tensor
    p0 = params
    kb = key_bias_mask(cfg)
    for p in PARAM_NAMES:
        dg = np.ravel(g["params"][p]) - p0[p].astype(np.float64).ravel()
        do = np.ravel(o["params"][p]) - p0[p].astype(np.float64).ravel()
        if p == "qkvb":
            dg, do = dg[~kb], do[~kb]
        c = cosine(dg, do)
        assert c >= 0.9, (p, c)


def test_bf16_accumulation_matches_oracle():
    cfg = RAGGED64
    say("case bf16 accumulation")
    params, batches = make_inputs(cfg, 2, 128, n_micro=2, perturb=True, bf16=True)
    dloss = 1.0 / (2 * 2 * 128)
    o = oracle_step(cfg, params, batches, dloss=dloss, lr=6e-4, wd=0.1)
    g = gpu_step(cfg, 1, params, batches, dloss=dloss, lr=6e-4, wd=0.1)
    for i in range(2):
        assert abs(g["means"][i] - o["means"][i]) <= 2e-2
    for p in PARAM_NAMES:
        c = cosine(g["grads"][p], o["grads"][p])
        assert c >= 0.995, (p, c)


def test_deterministic_bitwise():
    cfg = RAGGED64
    say("case determinism bf16")
    params, batches = make_inputs(cfg, 2, 150, perturb=True, bf16=True)
    a = gpu_step(cfg, 1, params, batches)
    b = gpu_step(cfg, 1, params, batches)
    for p in PARAM_NAMES:
        assert np.array_equal(a["grads"][p], b["grads"][p]), p
        assert np.array_equal(a["params"][p], b["params"][p]), p
    assert np.array_equal(a["losses"][0], b["losses"][0])


def test_loss_at_init_near_log_v():
    cfg = S.TINY
    params, batches = make_inputs(cfg, 4, 64)
    g = gpu_step(cfg, 0, params, batches)
    expect = math.log(cfg.vocab_size) + cfg.channels * 0.02 ** 2 / 2
    assert abs(g["means"][0] - expect) < 0.02


# token patterns for the sorted, chunked token-embedding gradient: one id
# everywhere (a single run over every 16-entry chunk), runs of 37 equal ids
# (runs starting mid-chunk and crossing chunk boundaries), all ids distinct
TOKEN_PATTERNS = ["one-id", "runs-37", "distinct"]


@pytest.mark.parametrize("pattern", TOKEN_PATTERNS)
def test_fp32_token_embedding_gradient_runs(pattern):
    cfg, B, T = RAGGED64, 2, 150
    say("case token runs", pattern)
    params, [(x, y)] = make_inputs(cfg, B, T, perturb=True)
    n = B * T
    if pattern == "one-id":
        ids = np.full(n, 5)
    elif pattern == "runs-37":
        ids = (np.arange(n) // 37 * 11) % cfg.vocab_size
    else:
        ids = np.random.default_rng(3).permutation(cfg.vocab_size)[:n]
    x = ids.reshape(B, T).astype(np.int32)
    o = oracle_step(cfg, params, [(x, y)], lr=1e-4)
    g = gpu_step(cfg, 0, params, [(x, y)], lr=1e-4)
    assert g["code"] == 0
    for p in ("wte", "wpe"):
        e = rel_l2(g["grads"][p], o["grads"][p])
        say(pattern, p, "gradient rel-L2", e)
        assert e < 1e-4, (pattern, p, e)


def test_caller_stream_without_host_syncs_matches_bitwise():
    """Two accumulated micro-steps and the update enqueued back to back on a
    non-default caller stream (the backward forks its weight-gradient products
    onto the context's own stream and joins them back), with no host
    synchronisation until the end: bit-identical to the synchronised run."""
    import torch
    from transformer_lm_step_amd.model import GPT2
    cfg, B, T = RAGGED64, 2, 150
    say("case caller stream bf16")
    params, batches = make_inputs(cfg, B, T, n_micro=2, perturb=True, bf16=True)
    ref = gpu_step(cfg, 1, params, batches, dloss=1.0 / (2 * B * T), wd=0.1, t=1)
    model = GPT2(cfg, 1, B, T)
    model.init(model.pack(params))
    torch.cuda.synchronize()
    dev = model.device
    xs = [torch.from_numpy(x.reshape(-1)).to(dev) for x, _ in batches]
    ys = [torch.from_numpy(y.reshape(-1)).to(dev) for _, y in batches]
    torch.cuda.synchronize()
    s = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(s):
        model.zero_grad()
        for xi, yi in zip(xs, ys):
            model.forward(xi, yi, None, None)
            model.backward(1.0 / (2 * B * T))
        grads = model.grads().clone()
        model.update(1e-4, 0.9, 0.999, 1e-8, 0.1, 1)
        newp = model.master().clone()
    s.synchronize()
    assert model.check() == 0
    g = model.unpack(grads.cpu().numpy().astype(np.float64))
    p_ = model.unpack(newp.cpu().numpy().astype(np.float64))
    model.close()
    for p in PARAM_NAMES:
        assert np.array_equal(g[p], ref["grads"][p]), p
        assert np.array_equal(p_[p], ref["params"][p]), p


def test_fp32_token_embedding_gradient_two_position_blocks():
    """B*T = 16448 positions: the token-embedding gradient runs over two
    blocks of positions (16384, then 64), each block's sums added in block
    order; Zipf tokens put the frequent ids in both blocks."""
    cfg, B, T = S.TINY, 257, 64
    say("case token blocks", B * T)
    params, batches = make_inputs(cfg, B, T, perturb=True, dist="zipf")
    o = oracle_step(cfg, params, batches, lr=1e-4)
    g = gpu_step(cfg, 0, params, batches, lr=1e-4)
    assert g["code"] == 0
    assert abs(g["means"][0] - o["means"][0]) / abs(o["means"][0]) < 1e-5
    for p in ("wte", "wpe"):
        e = rel_l2(g["grads"][p], o["grads"][p])
        say("two blocks", p, "gradient rel-L2", e)
        assert e < 1e-4, (p, e)


@pytest.mark.parametrize("cfg", [WIDE, WIDE576], ids=["c800", "c576"])
def test_bf16_wide_forward_ragged_tiles(cfg):
    """The logits of the last sequence of a B=8, T=1024, C=800 (or 576) forward against
    the oracle's forward of that sequence (fp64 from the same bf16-exact
    parameters): rel-L2 <= 2e-2 over the real vocabulary columns.  The MLP and
    attention branches dominate the one-layer residual stream at this init,
    so wrong values in one ragged column tile of a product move the logits
    far past the bar."""
    import oracle
    import torch
    from transformer_lm_step_amd import binding as Bnd
    from transformer_lm_step_amd.model import GPT2
    B, T = 8, 1024
    say("case wide forward", B, T, cfg.channels)
    params, [(x, y)] = make_inputs(cfg, B, T, perturb=True, bf16=True)
    m = GPT2(cfg, 1, B, T)
    m.init(m.pack(params))
    m.forward(torch.from_numpy(np.ascontiguousarray(x).reshape(-1)).cuda())
    torch.cuda.synchronize()
    assert m.check() == 0
    got = m.act(Bnd.GPT2_T_LOGITS).float().cpu().numpy().reshape(B, T, -1)
    m.close()
    b = B - 1
    ref = oracle.gpt2_step(cfg, oracle.pack_params(cfg, params), x[b:b + 1], want_grads=False,
                           want_logits=True)["logits"][0]
    V = cfg.vocab_size
    e = rel_l2(got[b, :, :V], ref[:, :V])
    say("wide forward logits rel-L2", e)
    assert e <= 2e-2, e

