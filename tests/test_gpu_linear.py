"""GPU parity of the bf16 Linear products (gpt2_linear_forward /
gpt2_linear_backward, the launches the step makes) against the oracle, at
sizes with more output tiles than the GPU holds at once (the persistent tile
loop) and ragged against every tile shape and the 64-deep contraction stages.

The oracle runs in fp64 on the same bf16-exact operands, on sampled output
rows (forward, input gradient: rows are independent) and sampled output rows
of the weight gradient (each a full contraction over M).  Bars: bf16 outputs
within 2^-8 relative per element (one bf16 rounding of an fp32 sum of exact
products) plus 1e-5 of the row's largest magnitude; fp32 weight and bias
gradients rel-L2 <= 1e-5.  Every output element is written (NaN-filled
beforehand).
"""

import numpy as np
import pytest

import synthetic as S
from helpers import rel_l2, say

pytestmark = pytest.mark.gpu

# (M, K, N): ragged layer-sized products, and a classifier-shaped one
SHAPES = [(8232, 776, 3120), (8200, 3080, 776), (4104, 768, 50304), (8232, 776, 1000)]


def _rows(M, n, seed):
    rng = np.random.default_rng(seed)
    r = set(rng.choice(M, n, replace=False).tolist())
    r.update([0, M - 1, M - 2, (M // 256) * 256, (M // 128) * 128 - 1])
    return np.array(sorted(x for x in r if 0 <= x < M))


def _bf16_close(got, ref):
    tol = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max(axis=-1, keepdims=True)
    return float(np.max(np.abs(got - ref) - tol))


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_linear_forward_bias(M, K, N):
    import torch
    import oracle
    from transformer_lm_step_amd import binding as B

    dev = torch.device("cuda:0")
    x, w, bias, _, _, _ = S.linear_inputs(M, K, N)
    bf = torch.bfloat16
    xd = torch.from_numpy(x).to(dev).to(bf)
    wd = torch.from_numpy(w).to(dev).to(bf)
    bd = torch.from_numpy(bias).to(dev).to(bf)
    y = torch.full((M, N), float("nan"), dtype=bf, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    B.gpt2_linear_forward(B.GPT2_BF16, xd.data_ptr(), wd.data_ptr(), bd.data_ptr(), y.data_ptr(), M, N, K, s)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(y).any()), "unwritten output elements"
    rows = _rows(M, 24, 7)
    got = y[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
    ref = oracle.matmul_forward(x[rows], w, bias)
    excess = _bf16_close(got, ref)
    say(f"forward {M}x{K}x{N}: {rows.size} rows, worst excess over the bound {excess:.2e}")
    assert excess <= 0.0


# plus the qkv layer's exact shape (input gradient N = 768: fewer tiles than CUs)
@pytest.mark.parametrize("M,K,N", SHAPES[:2] + [(8192, 768, 2304)])
def test_linear_backward(M, K, N):
    import torch
    import oracle
    from transformer_lm_step_amd import binding as B

    dev = torch.device("cuda:0")
    x, w, _, dy, dw0, db0 = S.linear_inputs(M, K, N, seed=S.DATA_SEED + 1)
    bf = torch.bfloat16
    xd = torch.from_numpy(x).to(dev).to(bf)
    wd = torch.from_numpy(w).to(dev).to(bf)
    dyd = torch.from_numpy(dy).to(dev).to(bf)
    dx = torch.full((M, K), float("nan"), dtype=bf, device=dev)
    dw = torch.from_numpy(dw0).to(dev)
    db = torch.from_numpy(db0).to(dev)
    alpha = 0.5
    wsz = B.gpt2_linear_backward_workspace(B.GPT2_BF16, M, N, K)
    ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)
    s = torch.cuda.current_stream().cuda_stream
    B.gpt2_linear_backward(B.GPT2_BF16, dyd.data_ptr(), xd.data_ptr(), wd.data_ptr(), dx.data_ptr(),
                           dw.data_ptr(), db.data_ptr(), M, N, K, alpha, ws.data_ptr(), wsz, s)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(dx).any()), "unwritten input-gradient elements"
    rows = _rows(M, 24, 8)
    got = dx[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
    ref_dx, _, _ = oracle.matmul_backward(alpha * dy[rows], x[rows], w)  # dx = alpha dy w
    excess = _bf16_close(got, ref_dx)
    say(f"input gradient {M}x{K} from N={N}: worst excess over the bound {excess:.2e}")
    assert excess <= 0.0
    # weight / bias gradient rows: full contractions over M, accumulated onto dw0 / db0
    ocs = _rows(N, 12, 9)
    _, ref_dw, ref_db = oracle.matmul_backward(alpha * dy[:, ocs], x, w[ocs])
    got_dw = dw.cpu().numpy()[ocs].astype(np.float64)
    got_db = db.cpu().numpy()[ocs].astype(np.float64)
    e_w = rel_l2(got_dw - dw0[ocs], ref_dw)
    e_b = rel_l2(got_db - db0[ocs], ref_db)
    say(f"weight gradient rows {ocs.size}: rel-L2 {e_w:.2e}, bias {e_b:.2e}")
    assert e_w <= 1e-5 and e_b <= 1e-5
