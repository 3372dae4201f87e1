"""The allocation-free attention backward (gpt2_attention_backward_noalloc)
against the workspace entry point (gpt2_attention_backward) on the same
inputs: both launch the same kernels in a fixed summation order (no atomics),
so dqkv must match bit for bit.  Two calls in a row per precision, the second
on a smaller, ragged shape (the library's scratch array keeps the first call's
contents), then the size limit of the scratch array."""

import pytest

import synthetic as S
from helpers import say

pytestmark = pytest.mark.gpu

# (B, T, C, NH, score scale): the GPT-2 124M layer shape, then a smaller ragged one
SHAPES = [(2, 1024, 768, 12, 1.0), (1, 130, 192, 3, 3.0)]


def _run(Bnd, torch, prec, B, T, C, NH, scale):
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if prec else torch.float32
    qkv, dout = S.attention_inputs(B, T, C, scale)
    qkv_d = torch.from_numpy(qkv).to(dev).to(dt)
    dout_d = torch.from_numpy(dout).to(dev).to(dt)
    out_d = torch.empty((B, T, C), dtype=dt, device=dev)
    lse_d = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    ref_d = torch.full((B, T, 3 * C), float("nan"), dtype=dt, device=dev)
    got_d = torch.full((B, T, 3 * C), float("nan"), dtype=dt, device=dev)
    delta_d = torch.empty((B, NH, T), dtype=torch.float32, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    Bnd.gpt2_attention_forward(prec, qkv_d.data_ptr(), out_d.data_ptr(), lse_d.data_ptr(), B, T, C, NH, s)
    Bnd.gpt2_attention_backward(prec, dout_d.data_ptr(), qkv_d.data_ptr(), out_d.data_ptr(), lse_d.data_ptr(),
                                ref_d.data_ptr(), delta_d.data_ptr(), B, T, C, NH, s)
    Bnd.gpt2_attention_backward_noalloc(prec, dout_d.data_ptr(), qkv_d.data_ptr(), out_d.data_ptr(),
                                        lse_d.data_ptr(), got_d.data_ptr(), B, T, C, NH, s)
    torch.cuda.synchronize()
    return ref_d, got_d


@pytest.mark.parametrize("prec", [1, 0], ids=["bf16", "fp32"])
def test_noalloc_attention_backward_matches_workspace_entry(prec):
    import torch

    from transformer_lm_step_amd import binding as Bnd

    for B, T, C, NH, scale in SHAPES:
        say("case noalloc attention backward", B, T, C, NH, scale, "bf16" if prec else "fp32")
        ref, got = _run(Bnd, torch, prec, B, T, C, NH, scale)
        assert bool(torch.isfinite(ref.float()).all())
        n_diff = int((got.view(torch.int16 if prec else torch.int32) !=
                      ref.view(torch.int16 if prec else torch.int32)).sum())
        say("elements differing:", n_diff)
        assert n_diff == 0


def test_noalloc_rejects_sizes_beyond_scratch():
    from transformer_lm_step_amd import binding as Bnd

    # B*NH*T = 1048577 > 1048576 delta rows: rejected before any device work
    with pytest.raises(Bnd.GPT2Error):
        Bnd.gpt2_attention_backward_noalloc(1, 256, 256, 256, 256, 256, 1, 1048577, 64, 1, 0)
