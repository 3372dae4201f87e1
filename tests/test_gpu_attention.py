"""GPU parity of causal attention (gpt2_attention_forward /
gpt2_attention_backward, the launches the step makes) against the oracle's
attention_forward / attention_backward in fp64 on the same bf16-exact inputs.

Cases: head sizes 64 (the GPT-2 sizes), 32, 128 and 16; T ragged against the
64-row blocks, T < 64, T = 1, T a multiple of 64 with many blocks, and the
full GPT-2 124M layer shape (T = 1024, 12 heads) at B = 2; score scales 1
and 3 (peakier softmax rows).

Bars.  fp32: rel-L2 <= 1e-5 for out and each third of dqkv.  bf16 (P and dS
enter their products rounded to bf16, outputs are bf16): rel-L2 <= 1e-2 and
max |error| <= 2^-5 max(max|ref|, 1e-3) per output tensor.  lse, against log2 of the
softmax denominator summed in fp64 from the same q and k: |error| <= 1e-5
(fp32); bf16 <= 2^-8: the head-size-64 kernel sums the fp32 weights, the
others sum the bf16-rounded probabilities that also weight V (each within
2^-9 relative, so the sum is too and its log2 within log2(1 + 2^-9) =
0.0028).  Every output element is written (NaN-filled
beforehand).
"""

import numpy as np
import pytest

import synthetic as S
from helpers import rel_l2, say

pytestmark = pytest.mark.gpu

# (B, T, C, NH, score scale)
CASES = [
    (2, 150, 192, 3, 1.0),
    (1, 256, 128, 2, 3.0),
    (3, 40, 128, 2, 1.0),
    (2, 1, 128, 2, 1.0),
    (1, 65, 128, 2, 3.0),
    (2, 100, 192, 6, 1.0),
    (1, 130, 256, 2, 1.0),
    (2, 1024, 768, 12, 1.0),
    # head size 16 (its key dimension padded to 32 inside the kernels), ragged T
    (2, 100, 64, 4, 1.0),
    (1, 130, 64, 4, 3.0),
]


def _lse_ref(qkv, NH):
    B, T, C3 = qkv.shape
    C = C3 // 3
    hs = C // NH
    q = qkv[:, :, :C].astype(np.float64).reshape(B, T, NH, hs).transpose(0, 2, 1, 3)
    k = qkv[:, :, C:2 * C].astype(np.float64).reshape(B, T, NH, hs).transpose(0, 2, 1, 3)
    s = q @ k.transpose(0, 1, 3, 2) / np.sqrt(hs)
    s = np.where(np.tril(np.ones((T, T), bool)), s, -np.inf)
    m = s.max(axis=-1, keepdims=True)
    return (m[..., 0] + np.log(np.exp(s - m).sum(axis=-1))) / np.log(2.0)


def _check(name, got, ref, prec):
    e = rel_l2(got, ref)
    say(name, "rel-L2", e)
    assert np.all(np.isfinite(got)), name
    if prec == 1:
        assert e <= 1e-2, (name, e)
        # magnitude floor 1e-3: with T = 1 (one visible key) dq is exactly 0
        assert np.max(np.abs(got - ref)) <= 2.0 ** -5 * max(np.max(np.abs(ref)), 1e-3), name
    else:
        assert e <= 1e-5, (name, e)


@pytest.mark.parametrize("prec", [1, 0], ids=["bf16", "fp32"])
@pytest.mark.parametrize("B,T,C,NH,scale", CASES)
def test_attention_matches_oracle(B, T, C, NH, scale, prec):
    import torch

    import oracle
    from transformer_lm_step_amd import binding as Bnd

    say("case attention", B, T, C, NH, scale, "bf16" if prec else "fp32")
    qkv, dout = S.attention_inputs(B, T, C, scale)
    out_ref, att = oracle.attention_forward(qkv, NH)
    dqkv_ref = oracle.attention_backward(dout, qkv, att, NH)
    del att
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if prec else torch.float32
    qkv_d = torch.from_numpy(qkv).to(dev).to(dt)
    dout_d = torch.from_numpy(dout).to(dev).to(dt)
    out_d = torch.full((B, T, C), float("nan"), dtype=dt, device=dev)
    lse_d = torch.full((B, NH, T), float("nan"), dtype=torch.float32, device=dev)
    dqkv_d = torch.full((B, T, 3 * C), float("nan"), dtype=dt, device=dev)
    delta_d = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    Bnd.gpt2_attention_forward(prec, qkv_d.data_ptr(), out_d.data_ptr(), lse_d.data_ptr(), B, T, C, NH, s)
    Bnd.gpt2_attention_backward(prec, dout_d.data_ptr(), qkv_d.data_ptr(), out_d.data_ptr(), lse_d.data_ptr(),
                                dqkv_d.data_ptr(), delta_d.data_ptr(), B, T, C, NH, s)
    torch.cuda.synchronize()
    out = out_d.float().cpu().numpy()
    lse = lse_d.cpu().numpy()
    dqkv = dqkv_d.float().cpu().numpy()
    _check("out", out, out_ref, prec)
    lse_err = float(np.max(np.abs(lse - _lse_ref(qkv, NH))))
    say("lse max error", lse_err)
    assert lse_err <= (2.0 ** -8 if prec else 1e-5)
    for i, part in enumerate("qkv"):
        _check("d" + part, dqkv[:, :, i * C:(i + 1) * C], dqkv_ref[:, :, i * C:(i + 1) * C], prec)


def test_attention_argument_errors():
    from transformer_lm_step_amd import binding as Bnd

    with pytest.raises(Bnd.GPT2Error):
        Bnd.gpt2_attention_forward(1, 256, 256, 256, 1, 16, 96, 2, 0)  # HS = 48
    with pytest.raises(Bnd.GPT2Error):
        Bnd.gpt2_attention_forward(2, 256, 256, 256, 1, 16, 128, 2, 0)  # precision
    with pytest.raises(Bnd.GPT2Error):
        Bnd.gpt2_attention_backward(1, 256, 256, 256, 256, 256, 0, 1, 16, 128, 2, 0)  # NULL workspace
