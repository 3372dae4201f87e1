"""A model built from a model file (gpt2_checkpoint_read + gpt2_init) steps
exactly like the oracle started from the oracle's reading of the same file:
fp32 file into fp32 mode (bars of the fp32 parity tests) and bf16 file into
bf16 mode (bars of the bf16 parity tests)."""

import numpy as np
import pytest

import oracle
import synthetic as S
from helpers import cosine, gpu_step, oracle_step, rel_l2, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("version", [3, 5])
def test_step_from_model_file(tmp_path, version):
    from transformer_lm_step_amd.model import GPT2

    cfg = S.TINY
    params = S.init_params(cfg, seed=11, perturb=True)
    if version == 5:
        params = {k: S.round_to_bf16(v) for k, v in params.items()}
    path = str(tmp_path / "model.bin")
    S.write_checkpoint(path, cfg, oracle.pack_params(cfg, params).astype(np.float32), version)
    _, prec, flat = oracle.read_checkpoint(path)
    shapes = S.param_shapes(cfg)
    p0 = oracle.unpack(cfg, flat, shapes)
    B, T = 4, 64
    stream = S.token_stream(B * T + 1, cfg.vocab_size, seed=5)
    batches = [S.batch(stream, 0, B, T)]
    say("case model file version", version)
    model = GPT2.from_checkpoint(path, prec, B, T)
    g = gpu_step(cfg, prec, None, batches, lr=1e-4, model=model)
    o = oracle_step(cfg, p0, batches, lr=1e-4)
    if prec == 0:
        assert abs(g["means"][0] - o["means"][0]) / abs(o["means"][0]) < 1e-5
        # key-bias gradients are exactly zero in exact arithmetic (round-off on
        # both sides): compared only outside that slice of qkvb
        kb = np.zeros((cfg.num_layers, 3 * cfg.channels), bool)
        kb[:, cfg.channels:2 * cfg.channels] = True
        for p in S.PARAM_NAMES:
            a, b = np.ravel(g["grads"][p]), np.ravel(o["grads"][p])
            if p == "qkvb":
                a, b = a[~kb.ravel()], b[~kb.ravel()]
            assert rel_l2(a, b) < 1e-4, p
    else:
        assert abs(g["means"][0] - o["means"][0]) <= 2e-2
        for p in S.PARAM_NAMES:
            assert cosine(g["grads"][p], o["grads"][p]) >= 0.995, p
