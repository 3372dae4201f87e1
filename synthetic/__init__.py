"""Seeded synthetic inputs for the GPT-2 training step.

This module is shared by the CPU oracle's tests and the HIP path's tests and
benchmark.  It only draws random numbers and arranges them into the shapes a
GPT-2 step consumes (parameters, token streams, the standalone fused-op
operands).  It holds none of the step's arithmetic: no layer, loss, gradient or
optimizer formula lives here, and it imports neither ``oracle`` nor the HIP
package.

Recipe (all draws from numpy's PCG64 generator, ``numpy.random.default_rng``):

* parameters follow GPT-2's initialisation as the configs state it: token and
  position embeddings and the qkv / fc weights N(0, 0.02); the two residual
  projections (attproj, fcproj) N(0, 0.02/sqrt(2L)); all biases 0; LayerNorm
  weight 1 and bias 0; the padded vocabulary rows V..Vp-1 of the token
  embedding are exactly 0.  ``perturb=True`` additionally gives every bias and
  LayerNorm parameter random values so that an indexing mistake in a bias or
  LayerNorm path cannot hide behind zeros and ones.
* token streams are uniform over [0, V) or Zipf(s) over [0, V): id r-1 is drawn
  with probability proportional to r**-s, by inverse CDF.
* a batch takes B*T+1 consecutive stream tokens; targets are the inputs shifted
  by one over the flat B*T block (the data loader of the train_gpt2.cu page).
"""

from __future__ import annotations

import dataclasses
import math

import numpy as np

DATA_SEED = 1337
INIT_SEED = 13371337

PARAM_NAMES = (
    "wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
    "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb",
)


@dataclasses.dataclass(frozen=True)
class Config:
    max_seq_len: int
    vocab_size: int
    padded_vocab_size: int
    num_layers: int
    num_heads: int
    channels: int

    def as_tuple(self):
        return (self.max_seq_len, self.vocab_size, self.padded_vocab_size,
                self.num_layers, self.num_heads, self.channels)


TINY = Config(max_seq_len=64, vocab_size=512, padded_vocab_size=512,
              num_layers=2, num_heads=4, channels=64)
GPT2_124M = Config(max_seq_len=1024, vocab_size=50257, padded_vocab_size=50304,
                   num_layers=12, num_heads=12, channels=768)
GPT2_1558M = Config(max_seq_len=1024, vocab_size=50257, padded_vocab_size=50304,
                    num_layers=48, num_heads=25, channels=1600)


def param_shapes(cfg: Config):
    """Shapes of the 16 parameter tensors, in the order the pages store them."""
    Vp, C, maxT, L = cfg.padded_vocab_size, cfg.channels, cfg.max_seq_len, cfg.num_layers
    return {
        "wte": (Vp, C), "wpe": (maxT, C),
        "ln1w": (L, C), "ln1b": (L, C),
        "qkvw": (L, 3 * C, C), "qkvb": (L, 3 * C),
        "attprojw": (L, C, C), "attprojb": (L, C),
        "ln2w": (L, C), "ln2b": (L, C),
        "fcw": (L, 4 * C, C), "fcb": (L, 4 * C),
        "fcprojw": (L, C, 4 * C), "fcprojb": (L, C),
        "lnfw": (C,), "lnfb": (C,),
    }


def init_params(cfg: Config, seed: int = INIT_SEED, perturb: bool = False):
    """GPT-2 initial parameters as a dict of float32 arrays (see module doc)."""
    rng = np.random.default_rng(seed)
    shapes = param_shapes(cfg)
    std = 0.02
    proj_std = 0.02 / math.sqrt(2 * cfg.num_layers)
    out = {}
    for name in PARAM_NAMES:
        shape = shapes[name]
        if name == "wte":
            a = np.zeros(shape, np.float32)
            a[: cfg.vocab_size] = rng.normal(0.0, std, (cfg.vocab_size, shape[1]))
        elif name in ("wpe", "qkvw", "fcw"):
            a = rng.normal(0.0, std, shape).astype(np.float32)
        elif name in ("attprojw", "fcprojw"):
            a = rng.normal(0.0, proj_std, shape).astype(np.float32)
        elif name.endswith("w"):  # LayerNorm weights
            a = np.ones(shape, np.float32)
            if perturb:
                a += rng.normal(0.0, 0.1, shape).astype(np.float32)
        else:  # biases and LayerNorm biases
            a = np.zeros(shape, np.float32)
            if perturb:
                a = rng.normal(0.0, 0.02, shape).astype(np.float32)
        out[name] = np.ascontiguousarray(a, dtype=np.float32)
    return out


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), returned as
    float32.  Used to hand both sides identical, bf16-exact starting values."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return (r.astype(np.uint32)).view(np.float32).reshape(np.shape(x))


def token_stream(n: int, vocab_size: int, seed: int = DATA_SEED,
                 dist: str = "uniform", zipf_s: float = 1.1) -> np.ndarray:
    """A stream of ``n`` int32 token ids in [0, vocab_size)."""
    rng = np.random.default_rng(seed)
    if dist == "uniform":
        return rng.integers(0, vocab_size, size=n, dtype=np.int64).astype(np.int32)
    if dist == "zipf":
        ranks = np.arange(1, vocab_size + 1, dtype=np.float64)
        p = ranks ** (-zipf_s)
        cdf = np.cumsum(p)
        cdf /= cdf[-1]
        u = rng.random(n)
        ids = np.searchsorted(cdf, u, side="right")
        return np.minimum(ids, vocab_size - 1).astype(np.int32)
    raise ValueError(f"unknown token distribution {dist!r}")


def batch(stream: np.ndarray, index: int, B: int, T: int):
    """Micro-batch ``index`` of a stream: (inputs [B,T], targets [B,T]) int32."""
    n = B * T
    start = index * n
    chunk = stream[start: start + n + 1]
    if chunk.shape[0] != n + 1:
        raise ValueError("token stream too short for this batch")
    return (chunk[:n].reshape(B, T).copy(), chunk[1:].reshape(B, T).copy())


def fused_op_inputs(M: int, K: int, N: int, seed: int = DATA_SEED):
    """Operands of the standalone Linear -> GELU -> row-softmax op.

    X ~ N(0, 1) [M,K]; W [N,K] with variance 1/K (so X W^T has unit variance);
    b ~ N(0, 0.02) [N].
    """
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K), dtype=np.float32)
    W = (rng.standard_normal((N, K), dtype=np.float32) * np.float32(1.0 / math.sqrt(K)))
    b = rng.normal(0.0, 0.02, N).astype(np.float32)
    return X, W.astype(np.float32), b


def linear_inputs(M: int, K: int, N: int, seed: int = DATA_SEED):
    """Operands of one Linear layer, all bf16-exact (float32 arrays).

    x ~ N(0, 1) [M,K]; w ~ N(0, 0.02) [N,K] (the GPT-2 init scale);
    bias ~ N(0, 0.02) [N]; dy ~ N(0, 1) [M,N]; dw0 ~ N(0, 0.01) [N,K] and
    db0 ~ N(0, 0.01) [N] as gradients already accumulated (fp32).
    """
    rng = np.random.default_rng(seed)
    x = round_to_bf16(rng.standard_normal((M, K), dtype=np.float32))
    w = round_to_bf16(rng.normal(0.0, 0.02, (N, K)).astype(np.float32))
    bias = round_to_bf16(rng.normal(0.0, 0.02, N).astype(np.float32))
    dy = round_to_bf16(rng.standard_normal((M, N), dtype=np.float32))
    dw0 = rng.normal(0.0, 0.01, (N, K)).astype(np.float32)
    db0 = rng.normal(0.0, 0.01, N).astype(np.float32)
    return x, w, bias, dy, dw0, db0


def attention_inputs(B: int, T: int, C: int, score_scale: float = 1.0, seed: int = DATA_SEED):
    """Operands of one causal attention layer, all bf16-exact (float32 arrays).

    qkv [B,T,3C]: q ~ N(0, score_scale), k ~ N(0, 1), v ~ N(0, 1), so a
    score q.k / sqrt(HS) is about N(0, score_scale^2); dout ~ N(0, 1) [B,T,C].
    """
    rng = np.random.default_rng(seed)
    q = rng.normal(0.0, score_scale, (B, T, C))
    kv = rng.standard_normal((B, T, 2 * C))
    qkv = round_to_bf16(np.concatenate([q, kv], axis=2).astype(np.float32))
    dout = round_to_bf16(rng.standard_normal((B, T, C), dtype=np.float32))
    return qkv, dout


def write_checkpoint(path: str, cfg: Config, flat_params: np.ndarray, version: int, header_extra=None):
    """Writes a model file in the layout train_gpt2.cu's gpt2_build_from_checkpoint
    reads: 256 little-endian int32 (magic 20240326, version, max_seq_len,
    vocab_size, num_layers, num_heads, channels, padded_vocab_size, zeros),
    then flat_params as float32 (version 3) or as bf16 (version 5: the upper
    16 bits of each float32, so the values should already be bf16-exact).
    header_extra: {index: value} overrides, for malformed-file tests."""
    head = np.zeros(256, "<i4")
    head[:8] = [20240326, version, cfg.max_seq_len, cfg.vocab_size, cfg.num_layers, cfg.num_heads,
                cfg.channels, cfg.padded_vocab_size]
    for k, v in (header_extra or {}).items():
        head[k] = v
    vals = np.ascontiguousarray(flat_params, dtype="<f4")
    with open(path, "wb") as f:
        f.write(head.tobytes())
        if version == 5:
            f.write((vals.view("<u4") >> 16).astype("<u2").tobytes())
        else:
            f.write(vals.tobytes())
