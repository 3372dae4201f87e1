"""GPU checks that must hold bit-exactly: the token/position gather, the causal
mask (future positions cannot change past outputs), the zero padded-vocabulary
gradient, the softmax - onehot rows, the device-side token check and the call
order rules."""

import numpy as np
import pytest
import torch

import oracle
import synthetic as S
from helpers import make_inputs, say

pytestmark = pytest.mark.gpu

RAG = S.Config(max_seq_len=160, vocab_size=997, padded_vocab_size=1000, num_layers=2, num_heads=3, channels=192)


def _model(cfg, prec, B, T, params):
    from transformer_lm_step_amd.model import GPT2
    m = GPT2(cfg, prec, B, T)
    m.init(m.pack(params))
    return m


@pytest.mark.parametrize("prec", [0, 1], ids=["fp32", "bf16"])
def test_encoder_bit_exact(prec):
    say("case encoder exact", prec)
    cfg = RAG
    params, [(x, y)] = make_inputs(cfg, 2, 150, perturb=True, bf16=prec == 1)
    m = _model(cfg, prec, 2, 150, params)
    xi = torch.from_numpy(x.reshape(-1)).cuda()
    m.forward(xi)
    torch.cuda.synchronize()
    got = m.act(4).float().cpu().numpy().reshape(2, 150, -1)
    ref = oracle.encoder_forward(x, params["wte"].reshape(cfg.padded_vocab_size, -1), params["wpe"])
    ref32 = ref.astype(np.float32)  # the sum of two fp32 (or bf16) values, rounded once to fp32
    if prec == 1:
        ref32 = S.round_to_bf16(ref32)
    assert np.array_equal(got, ref32)
    m.close()


@pytest.mark.parametrize("prec", [0, 1], ids=["fp32", "bf16"])
def test_causal_future_perturbation(prec):
    say("case causality", prec)
    cfg = RAG
    params, [(x, y)] = make_inputs(cfg, 2, 150, perturb=True, bf16=prec == 1)
    m = _model(cfg, prec, 2, 150, params)
    outs = []
    for xx in (x, np.where(np.arange(150)[None, :] >= 77, (x + 3) % cfg.vocab_size, x).astype(np.int32)):
        m.forward(torch.from_numpy(np.ascontiguousarray(xx).reshape(-1)).cuda())
        torch.cuda.synchronize()
        outs.append(m.act(0).float().cpu().numpy().reshape(2, 150, -1).copy())
    assert np.array_equal(outs[0][:, :77], outs[1][:, :77])
    assert not np.array_equal(outs[0][:, 77:], outs[1][:, 77:])
    m.close()


def test_softmax_rows_and_padded_zero():
    say("case softmax rows")
    cfg = RAG
    params, [(x, y)] = make_inputs(cfg, 2, 150, perturb=True)
    m = _model(cfg, 0, 2, 150, params)
    m.forward(torch.from_numpy(x.reshape(-1)).cuda(), torch.from_numpy(y.reshape(-1)).cuda())
    torch.cuda.synchronize()
    d = m.act(0).cpu().numpy().reshape(300, cfg.padded_vocab_size).astype(np.float64)
    assert np.all(d[:, cfg.vocab_size:] == 0.0)
    assert np.allclose(d.sum(1), 0.0, atol=1e-5)  # softmax sums to 1, minus the onehot
    p = d.copy()
    p[np.arange(300), y.reshape(-1)] += 1.0
    assert p.min() >= -1e-7 and np.allclose(p.sum(1), 1.0, atol=1e-5)
    m.close()


def test_bad_token_raises_flag_and_state_rules():
    from transformer_lm_step_amd import binding as B
    say("case token flag")
    cfg = S.TINY
    params, [(x, y)] = make_inputs(cfg, 4, 64)
    m = _model(cfg, 0, 4, 64, params)
    with pytest.raises(B.GPT2Error) as e:
        m.backward()  # no forward yet
    assert e.value.code == B.GPT2_E_STATE
    xb = x.copy().reshape(-1)
    xb[5] = cfg.vocab_size + 7
    m.forward(torch.from_numpy(xb).cuda())
    assert m.check() == B.GPT2_E_TOKEN
    assert m.check() == B.GPT2_OK  # cleared
    with pytest.raises(B.GPT2Error) as e:
        m.backward()  # forward had no targets
    assert e.value.code == B.GPT2_E_STATE
    yb = y.copy().reshape(-1)
    yb[3] = -1
    m.forward(torch.from_numpy(x.reshape(-1)).cuda(), torch.from_numpy(yb).cuda())
    assert m.check() == B.GPT2_E_TOKEN
    m.close()


def test_classifier_event_hook():
    """The timing hook records a start/end event pair around the classifier
    product of each forward, cycling through the slots; n = 0 removes it."""
    import ctypes
    from transformer_lm_step_amd import binding as B
    rt = ctypes.CDLL("libamdhip64.so")
    rt.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
    rt.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
    rt.hipEventDestroy.argtypes = [ctypes.c_void_p]
    evs = []
    for _ in range(4):
        e = ctypes.c_void_p()
        assert rt.hipEventCreate(ctypes.byref(e)) == 0
        evs.append(e.value)
    cfg = RAG
    params, [(x, y)] = make_inputs(cfg, 2, 150, perturb=True)
    m = _model(cfg, 0, 2, 150, params)
    hook = B.gpt2_set_classifier_events(m.ctx, evs[:2], evs[2:])
    xi = torch.from_numpy(x.reshape(-1)).cuda()
    for _ in range(3):
        m.forward(xi)
    torch.cuda.synchronize()
    for a, b in zip(evs[:2], evs[2:]):
        t = ctypes.c_float()
        assert rt.hipEventElapsedTime(ctypes.byref(t), a, b) == 0
        assert 0.0 < t.value < 1000.0
    B.gpt2_set_classifier_events(m.ctx, [], [])
    del hook
    with pytest.raises(B.GPT2Error):
        B.lib()  # the raw entry point rejects a negative count
        rc = B.lib().gpt2_set_classifier_events(m.ctx, None, None, -1)
        if rc != 0:
            raise B.GPT2Error(rc, "gpt2_set_classifier_events")
    m.forward(xi)
    torch.cuda.synchronize()
    m.close()
    for e in evs:
        rt.hipEventDestroy(e)
