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
# products taken by the 256 x 288 tile: the qkv layer's exact shape (one
# tile per CU), ragged in M, N and K within one round, and ragged with three
# tiles per workgroup (the persistent loop, next tile's stages issued before
# the epilogue)
SHAPES_288 = [(8192, 768, 2304), (8100, 776, 2296), (8200, 1608, 6392)]
# products taken by the depth-sliced 128 x 192 tile (N <= 768, K >= 1536):
# the MLP projection's shape, and ragged in M, N and K
SHAPES_SLICED = [(8192, 3072, 768), (8100, 3080, 760)]


def _rows(M, n, seed):
    rng = np.random.default_rng(seed)
    r = set(rng.choice(M, n, replace=False).tolist())
    r.update([0, M - 1, M - 2, (M // 256) * 256, (M // 128) * 128 - 1])
    return np.array(sorted(x for x in r if 0 <= x < M))


def _bf16_close(got, ref):
    tol = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.abs(ref).max(axis=-1, keepdims=True)
    return float(np.max(np.abs(got - ref) - tol))


@pytest.mark.parametrize("M,K,N", SHAPES + SHAPES_288 + SHAPES_SLICED)
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


def _tile_rows(n, seed, tile=256):
    """One seeded row in every `tile`-row block of n (and the last row): every
    row tile of an output is checked."""
    rng = np.random.default_rng(seed)
    r = {min(n - 1, b + int(rng.integers(tile))) for b in range(0, n, tile)}
    r.add(n - 1)
    return np.array(sorted(r))


# plus the qkv layer's exact shape (input gradient N = 768: fewer tiles than
# CUs) and the tied classifier's (8192 x 768 from N = 50304: the K-split input
# gradient, and a weight gradient of 197 x 3 tiles), and an input gradient
# ragged in M, N and K on 256 x 192 tiles (the 12-unit k-strided slab), and
# input gradients on the depth-sliced 128 x 192 tile (the fc layer's shape,
# and ragged)
@pytest.mark.parametrize("M,K,N", SHAPES[:2] + [(8192, 768, 2304), (8192, 768, 50304), (8100, 3064, 776),
                                               (8192, 768, 3072), (8100, 760, 3080)])
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
    # weight / bias gradient rows (one in every 256-row tile, all columns):
    # full contractions over M, accumulated onto dw0 / db0
    ocs = _tile_rows(N, 9)
    _, ref_dw, ref_db = oracle.matmul_backward(alpha * dy[:, ocs], x, w[ocs])
    got_dw = dw.cpu().numpy()[ocs].astype(np.float64)
    got_db = db.cpu().numpy()[ocs].astype(np.float64)
    e_w = rel_l2(got_dw - dw0[ocs], ref_dw)
    e_b = rel_l2(got_db - db0[ocs], ref_db)
    say(f"weight gradient rows {ocs.size}: rel-L2 {e_w:.2e}, bias {e_b:.2e}")
    assert e_w <= 1e-5 and e_b <= 1e-5


def test_linear_backward_beyond_4gib():
    """The classifier's backward products with B*T = 44000 rows: dlogits
    [44000, 50304] bf16 is 4.4 GB, so tile ranges past 2 GiB from a tile's
    origin are clamped.  Operands come from torch's seeded generator on the
    device; the oracle checks one input-gradient row per 256-row tile range
    sampled and one weight-gradient row in every 256-row tile (full
    contractions over the 44000 rows)."""
    import torch
    import oracle
    from transformer_lm_step_amd import binding as B

    M, K, N = 44000, 768, 50304
    dev = torch.device("cuda:0")
    gen = torch.Generator(device=dev)
    gen.manual_seed(S.DATA_SEED + 7)
    bf = torch.bfloat16
    x = torch.randn(M, K, generator=gen, device=dev).to(bf)
    w = (0.02 * torch.randn(N, K, generator=gen, device=dev)).to(bf)
    dy = (torch.randn(M, N, generator=gen, device=dev) * 1e-3).to(bf)
    dx = torch.full((M, K), float("nan"), dtype=bf, device=dev)
    dw = torch.zeros(N, K, dtype=torch.float32, device=dev)
    db = torch.zeros(N, dtype=torch.float32, device=dev)
    alpha = 0.25
    wsz = B.gpt2_linear_backward_workspace(B.GPT2_BF16, M, N, K)
    ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)
    say(f"backward beyond 4 GiB: dy {M}x{N} bf16 = {M * N * 2 / 1e9:.1f} GB, workspace {wsz} bytes")
    B.gpt2_linear_backward(B.GPT2_BF16, dy.data_ptr(), x.data_ptr(), w.data_ptr(), dx.data_ptr(), dw.data_ptr(),
                           db.data_ptr(), M, N, K, alpha, ws.data_ptr(), wsz, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert not bool(torch.isnan(dx).any()), "unwritten input-gradient elements"
    w64 = w.float().cpu().numpy().astype(np.float64)
    rows = np.array(sorted(set(_rows(M, 16, 10).tolist()) | {M - 1, M - 300, 43008}))
    got = dx[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
    dyr = dy[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
    ref_dx = alpha * dyr @ w64
    excess = _bf16_close(got, ref_dx)
    say(f"input gradient rows {rows.size}: worst excess over the bound {excess:.2e}")
    assert excess <= 0.0
    ocs = _tile_rows(N, 11)
    dyc = dy[:, torch.from_numpy(ocs).to(dev)].float().cpu().numpy().astype(np.float64)
    x64 = x.float().cpu().numpy().astype(np.float64)
    ref_dw = alpha * dyc.T @ x64
    ref_db = alpha * dyc.sum(axis=0)
    got_dw = dw.cpu().numpy()[ocs].astype(np.float64)
    got_db = db.cpu().numpy()[ocs].astype(np.float64)
    e_w, e_b = rel_l2(got_dw, ref_dw), rel_l2(got_db, ref_db)
    say(f"weight gradient rows {ocs.size}: rel-L2 {e_w:.2e}, bias {e_b:.2e}")
    assert e_w <= 1e-5 and e_b <= 1e-5
