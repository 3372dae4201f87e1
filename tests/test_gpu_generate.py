"""Inference and sampling (train_gpt2.cu, sample_softmax and the generation
loop) through the C ABI: gpt2_sample on the device against the oracle's
sampler on the same logits (same inputs, so the same token unless the draw
sits within fp64 round-off of a CDF step, which the check allows and
verifies), and gpt2_generate against the oracle's generation loop (fp32) or
against a replay of its own draws (bf16)."""

import numpy as np
import pytest

import oracle
import synthetic as S
from helpers import say

pytestmark = pytest.mark.gpu

# GPT-2's vocabulary (V = 50257, Vp = 50304) on a one-layer model
WIDEV = S.Config(max_seq_len=64, vocab_size=50257, padded_vocab_size=50304, num_layers=1, num_heads=2, channels=128)


def _draw_ok(row, V, coin, got):
    """got is the oracle's draw, or the draw sits within fp64 round-off of
    the CDF step between the two."""
    want = oracle.sample_softmax(row, V, coin)
    if got == want:
        return True
    z = np.asarray(row, np.float64)[:V]
    cdf = np.cumsum(np.exp(z - z.max()))
    step = cdf[min(got, want)]
    return 0 <= got < V and abs(coin * cdf[-1] - step) <= 1e-12 * cdf[-1]


def _model(cfg, prec, B, T, seed):
    from transformer_lm_step_amd.model import GPT2
    params = S.init_params(cfg, seed=seed, perturb=True)
    if prec == 1:
        params = {k: S.round_to_bf16(v) for k, v in params.items()}
    m = GPT2(cfg, prec, B, T)
    m.init(m.pack(params))
    return m, params


@pytest.mark.parametrize("prec", [0, 1], ids=["fp32", "bf16"])
@pytest.mark.parametrize("cfg", [S.TINY, WIDEV], ids=["tiny", "gpt2-vocab"])
def test_sample_matches_oracle_on_device_logits(cfg, prec):
    import torch
    from transformer_lm_step_amd import binding as B

    Bn, T = 3, 16
    say("case sample", cfg.vocab_size, prec)
    m, _ = _model(cfg, prec, Bn, T, seed=21)
    rng = np.random.default_rng(8)
    tok = torch.from_numpy(rng.integers(0, cfg.vocab_size, (Bn, T)).astype(np.int32)).to(m.device)
    m.forward(tok.view(-1))
    torch.cuda.synchronize()
    logits = m.act(B.GPT2_T_LOGITS).float().cpu().numpy().reshape(Bn, T, -1)
    for t in (1, 7, T - 1):
        coins = rng.random(Bn).astype(np.float32)
        m.sample(torch.from_numpy(coins).to(m.device), tok, t)
        torch.cuda.synchronize()
        got = tok.cpu().numpy()
        for b in range(Bn):
            assert _draw_ok(logits[b, t - 1], cfg.vocab_size, float(coins[b]), int(got[b, t])), (t, b)
    # extreme coins: 0 draws the first token with positive probability,
    # 1 - 2^-24 the last one reached
    for coin in (0.0, 1.0 - 2.0 ** -24):
        coins = np.full(Bn, coin, np.float32)
        m.sample(torch.from_numpy(coins).to(m.device), tok, 2)
        torch.cuda.synchronize()
        got = tok.cpu().numpy()
        for b in range(Bn):
            assert _draw_ok(logits[b, 1], cfg.vocab_size, float(coin), int(got[b, 2]))
    m.close()


def test_generate_matches_oracle_fp32():
    import torch

    cfg, Bn, T, t0, t1 = S.TINY, 2, 24, 4, 24
    m, params = _model(cfg, 0, Bn, T, seed=33)
    rng = np.random.default_rng(9)
    start = rng.integers(0, cfg.vocab_size, (Bn, T)).astype(np.int32)
    coins = rng.random((t1 - t0, Bn)).astype(np.float32)
    tok = torch.from_numpy(start.copy()).to(m.device)
    m.generate(tok, torch.from_numpy(coins).to(m.device), t0, t1)
    torch.cuda.synchronize()
    got = tok.cpu().numpy()
    want = oracle.generate(cfg, oracle.pack_params(cfg, params), start, coins.astype(np.float64), t0, t1)
    say("generated", got[0, t0:t1].tolist())
    assert np.array_equal(got[:, :t0], start[:, :t0])
    assert np.array_equal(got, want)
    m.close()


def test_generate_bf16_replays_its_own_draws():
    """Each draw at t used the logits at t - 1 of a forward over tokens that
    were final up to t - 1; causality makes one more forward over the final
    tokens reproduce those logits exactly, so every draw can be re-checked."""
    import torch
    from transformer_lm_step_amd import binding as B

    cfg, Bn, T, t0, t1 = WIDEV, 2, 32, 3, 32
    m, _ = _model(cfg, 1, Bn, T, seed=44)
    rng = np.random.default_rng(10)
    start = rng.integers(0, cfg.vocab_size, (Bn, T)).astype(np.int32)
    coins = rng.random((t1 - t0, Bn)).astype(np.float32)
    tok = torch.from_numpy(start.copy()).to(m.device)
    m.generate(tok, torch.from_numpy(coins).to(m.device), t0, t1)
    m.forward(tok.view(-1))
    torch.cuda.synchronize()
    logits = m.act(B.GPT2_T_LOGITS).float().cpu().numpy().reshape(Bn, T, -1)
    got = tok.cpu().numpy()
    assert np.array_equal(got[:, :t0], start[:, :t0])
    for t in range(t0, t1):
        for b in range(Bn):
            assert _draw_ok(logits[b, t - 1], cfg.vocab_size, float(coins[t - t0, b]), int(got[b, t])), (t, b)
    m.close()


def test_sample_state_and_argument_errors():
    import torch
    from transformer_lm_step_amd import binding as B

    cfg, Bn, T = S.TINY, 2, 8
    m, _ = _model(cfg, 0, Bn, T, seed=1)
    tok = torch.zeros(Bn * T, dtype=torch.int32, device=m.device)
    tgt = torch.zeros(Bn * T, dtype=torch.int32, device=m.device)
    coins = torch.zeros(Bn, dtype=torch.float32, device=m.device)
    lo = torch.empty(Bn * T, dtype=torch.float32, device=m.device)
    with pytest.raises(B.GPT2Error) as e:  # no forward yet
        m.sample(coins, tok, 1)
    assert e.value.code == B.GPT2_E_STATE
    m.forward(tok, tgt, lo)
    with pytest.raises(B.GPT2Error) as e:  # logits replaced by softmax - onehot
        m.sample(coins, tok, 1)
    assert e.value.code == B.GPT2_E_STATE
    m.forward(tok)
    for t in (0, T):
        with pytest.raises(B.GPT2Error) as e:
            m.sample(coins, tok, t)
        assert e.value.code == B.GPT2_E_ARG
    with pytest.raises(B.GPT2Error) as e:
        m.generate(tok, coins, 3, 2)
    assert e.value.code == B.GPT2_E_ARG
    torch.cuda.synchronize()
    m.close()
