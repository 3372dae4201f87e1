"""CPU oracle for the GPT-2 training step -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product path (the HIP library and its
binding) never does.

The arithmetic lives in ``gpt2_oracle.c`` (plain single-threaded C, double
precision).  This module only builds it, loads it and marshals numpy arrays,
plus one piece of byte work written here in numpy: reading a model file
(``read_checkpoint``).
Parity pins for every function are in ``tests/test_oracle_*.py``.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gpt2_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
# -O2, no fast-math, no threads, no vector ISA beyond the x86-64 baseline.
GCC_CMD = ["gcc", "-O2", "-std=gnu11", "-fPIC", "-shared", "-o", _LIB_PATH, _SRC, "-lm"]

PARAM_NAMES = (
    "wte", "wpe", "ln1w", "ln1b", "qkvw", "qkvb", "attprojw", "attprojb",
    "ln2w", "ln2b", "fcw", "fcb", "fcprojw", "fcprojb", "lnfw", "lnfb",
)


def build() -> str:
    subprocess.run(GCC_CMD, check=True)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = ctypes.CDLL(_LIB_PATH)
        _declare(_lib)
    return _lib


class OrcConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "max_seq_len", "vocab_size", "padded_vocab_size", "num_layers", "num_heads", "channels")]


_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int)
_sp = ctypes.POINTER(ctypes.c_size_t)
_i = ctypes.c_int
_z = ctypes.c_size_t
_d = ctypes.c_double


def _declare(L):
    sig = {
        "orc_param_layout": (_z, [ctypes.POINTER(OrcConfig), _sp, _sp]),
        "orc_encoder_forward": (None, [_dp, _ip, _dp, _dp, _i, _i, _i]),
        "orc_encoder_backward": (None, [_dp, _dp, _dp, _ip, _i, _i, _i]),
        "orc_layernorm_forward": (None, [_dp, _dp, _dp, _dp, _dp, _dp, _i, _i]),
        "orc_layernorm_backward": (None, [_dp, _dp, _dp, _dp, _dp, _dp, _dp, _dp, _i, _i]),
        "orc_matmul_forward": (None, [_dp, _dp, _dp, _dp, _i, _i, _i]),
        "orc_matmul_backward": (None, [_dp, _dp, _dp, _dp, _dp, _dp, _i, _i, _i]),
        "orc_attention_forward": (None, [_dp, _dp, _dp, _i, _i, _i, _i]),
        "orc_attention_backward": (None, [_dp, _dp, _dp, _dp, _i, _i, _i, _i]),
        "orc_gelu_forward": (None, [_dp, _dp, _z]),
        "orc_gelu_backward": (None, [_dp, _dp, _dp, _z]),
        "orc_residual_forward": (None, [_dp, _dp, _dp, _z]),
        "orc_crossentropy_forward": (_d, [_dp, _dp, _dp, _ip, _i, _i, _i]),
        "orc_crossentropy_backward": (None, [_dp, _dp, _ip, _d, _i, _i, _i]),
        "orc_adamw": (None, [_dp, _dp, _dp, _dp, _z, _d, _d, _d, _d, _d, _i]),
        "orc_adamw_sr": (None, [ctypes.POINTER(ctypes.c_uint16), ctypes.POINTER(ctypes.c_float),
                                ctypes.POINTER(ctypes.c_float), ctypes.POINTER(ctypes.c_float), _z,
                                ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float, _i,
                                ctypes.c_uint32]),
        "orc_xorshift_u32": (ctypes.c_uint32, [ctypes.POINTER(ctypes.c_uint64)]),
        "orc_noise2d": (ctypes.c_uint32, [_i, _i, ctypes.c_uint32]),
        "orc_sr_bf16": (ctypes.c_uint16, [ctypes.c_float, ctypes.c_uint32]),
        "orc_gpt2_step": (_d, [ctypes.POINTER(OrcConfig), _dp, _ip, _ip, _i, _i, _d, _dp, _dp, _dp]),
        "orc_fused_linear_gelu_softmax": (None, [_dp, _dp, _dp, _dp, _i, _i, _i, _ip, _i]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _p(a):
    if a is None:
        return None
    if a.dtype == np.float64:
        return a.ctypes.data_as(_dp)
    if a.dtype == np.int32:
        return a.ctypes.data_as(_ip)
    raise TypeError(a.dtype)


def config(cfg) -> OrcConfig:
    """Accepts anything with the six GPT2Config fields."""
    return OrcConfig(cfg.max_seq_len, cfg.vocab_size, cfg.padded_vocab_size,
                     cfg.num_layers, cfg.num_heads, cfg.channels)


def param_layout(cfg):
    off = (ctypes.c_size_t * 16)()
    cnt = (ctypes.c_size_t * 16)()
    c = config(cfg)
    total = lib().orc_param_layout(ctypes.byref(c), off, cnt)
    return list(off), list(cnt), int(total)


def pack_params(cfg, tensors: dict) -> np.ndarray:
    off, cnt, total = param_layout(cfg)
    flat = np.zeros(total, np.float64)
    for i, name in enumerate(PARAM_NAMES):
        a = np.asarray(tensors[name], dtype=np.float64).reshape(-1)
        if a.size != cnt[i]:
            raise ValueError(f"{name}: {a.size} elements, layout wants {cnt[i]}")
        flat[off[i]: off[i] + cnt[i]] = a
    return flat


def unpack(cfg, flat: np.ndarray, shapes: dict) -> dict:
    off, cnt, _ = param_layout(cfg)
    return {name: flat[off[i]: off[i] + cnt[i]].reshape(shapes[name])
            for i, name in enumerate(PARAM_NAMES)}


class _Cfg:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def read_checkpoint(path):
    """train_gpt2.cu, gpt2_build_from_checkpoint: a header of 256 int32 (magic
    20240326; version 3 = fp32 parameters, 5 = bf16 parameters; then
    max_seq_len, vocab_size, num_layers, num_heads, channels,
    padded_vocab_size), then all parameters of that config in ParameterTensors
    order.  Returns (config fields as a dict, 0 for fp32 / 1 for bf16, the
    parameters as float64).  bf16 values are widened exactly (a bf16 is the
    upper half of the fp32 with the same value).  Raises ValueError for a bad
    magic or version or a short file."""
    with open(path, "rb") as f:
        head = np.frombuffer(f.read(256 * 4), dtype="<i4")
        if head.size != 256 or head[0] != 20240326 or head[1] not in (3, 5):
            raise ValueError("not a model file")
        names = ("max_seq_len", "vocab_size", "num_layers", "num_heads", "channels", "padded_vocab_size")
        cfg = {n: int(head[2 + i]) for i, n in enumerate(names)}
        _, _, P = param_layout(_Cfg(**cfg))
        if head[1] == 3:
            vals = np.frombuffer(f.read(4 * P), dtype="<f4")
        else:
            raw = np.frombuffer(f.read(2 * P), dtype="<u2")
            vals = (raw.astype(np.uint32) << 16).view(np.float32)
        if vals.size != P:
            raise ValueError("model file shorter than its parameters")
    return cfg, (0 if head[1] == 3 else 1), vals.astype(np.float64)


# ---- per-definition entry points ------------------------------------------------

def encoder_forward(tok, wte, wpe):
    tok = _i32(tok); B, T = tok.shape
    wte = _f64(wte); wpe = _f64(wpe); C = wte.shape[1]
    out = np.empty((B, T, C))
    lib().orc_encoder_forward(_p(out), _p(tok), _p(wte), _p(wpe), B, T, C)
    return out


def encoder_backward(dwte, dwpe, dout, tok):
    """Adds into (copies of) dwte and dwpe and returns them."""
    tok = _i32(tok); B, T = tok.shape
    dwte = _f64(dwte).copy(); dwpe = _f64(dwpe).copy(); dout = _f64(dout)
    C = dwte.shape[1]
    lib().orc_encoder_backward(_p(dwte), _p(dwpe), _p(dout), _p(tok), B, T, C)
    return dwte, dwpe


def layernorm_forward(x, w, b):
    x = _f64(x); N, C = x.shape
    out = np.empty_like(x); mean = np.empty(N); rstd = np.empty(N)
    lib().orc_layernorm_forward(_p(out), _p(mean), _p(rstd), _p(x), _p(_f64(w)), _p(_f64(b)), N, C)
    return out, mean, rstd


def layernorm_backward(dx, dw, db, dout, x, w, mean, rstd):
    x = _f64(x); N, C = x.shape
    dx = _f64(dx).copy(); dw = _f64(dw).copy(); db = _f64(db).copy()
    lib().orc_layernorm_backward(_p(dx), _p(dw), _p(db), _p(_f64(dout)), _p(x), _p(_f64(w)),
                                 _p(_f64(mean)), _p(_f64(rstd)), N, C)
    return dx, dw, db


def matmul_forward(x, w, bias=None):
    x = _f64(x); w = _f64(w); N, K = x.shape; OC = w.shape[0]
    out = np.empty((N, OC))
    lib().orc_matmul_forward(_p(out), _p(x), _p(w), _p(None if bias is None else _f64(bias)), N, K, OC)
    return out


def matmul_backward(dout, x, w, dw=None, db=None):
    """Returns (dx, dw + dW, db + dB); dw/db default to zeros."""
    dout = _f64(dout); x = _f64(x); w = _f64(w)
    N, K = x.shape; OC = w.shape[0]
    dx = np.empty((N, K))
    dw = np.zeros((OC, K)) if dw is None else _f64(dw).copy()
    db = np.zeros(OC) if db is None else _f64(db).copy()
    lib().orc_matmul_backward(_p(dx), _p(dw), _p(db), _p(dout), _p(x), _p(w), N, K, OC)
    return dx, dw, db


def attention_forward(qkv, NH):
    qkv = _f64(qkv); B, T, C3 = qkv.shape; C = C3 // 3
    out = np.empty((B, T, C)); att = np.empty((B, NH, T, T))
    lib().orc_attention_forward(_p(out), _p(att), _p(qkv), B, T, C, NH)
    return out, att


def attention_backward(dout, qkv, att, NH):
    qkv = _f64(qkv); B, T, C3 = qkv.shape; C = C3 // 3
    dqkv = np.empty_like(qkv)
    lib().orc_attention_backward(_p(dqkv), _p(_f64(dout)), _p(qkv), _p(_f64(att)), B, T, C, NH)
    return dqkv


def gelu_forward(x):
    x = _f64(x); out = np.empty_like(x)
    lib().orc_gelu_forward(_p(out), _p(x), x.size)
    return out


def gelu_backward(x, dout):
    x = _f64(x); dx = np.empty_like(x)
    lib().orc_gelu_backward(_p(dx), _p(x), _p(_f64(dout)), x.size)
    return dx


def residual_forward(a, b):
    a = _f64(a); out = np.empty_like(a)
    lib().orc_residual_forward(_p(out), _p(a), _p(_f64(b)), a.size)
    return out


def crossentropy_forward(logits, targets, V):
    logits = _f64(logits); N, Vp = logits.shape
    losses = np.empty(N); probs = np.empty_like(logits)
    mean = lib().orc_crossentropy_forward(_p(losses), _p(probs), _p(logits), _p(_i32(targets)), N, V, Vp)
    return losses, probs, mean


def crossentropy_backward(probs, targets, dloss, V):
    probs = _f64(probs); N, Vp = probs.shape
    d = np.empty_like(probs)
    lib().orc_crossentropy_backward(_p(d), _p(probs), _p(_i32(targets)), float(dloss), N, V, Vp)
    return d


def adamw(params, grads, m, v, lr, beta1, beta2, eps, wd, t):
    """Returns updated (params, m, v) copies."""
    p = _f64(params).copy(); m = _f64(m).copy(); v = _f64(v).copy(); g = _f64(grads)
    lib().orc_adamw(_p(p), _p(g), _p(m), _p(v), p.size, lr, beta1, beta2, eps, wd, int(t))
    return p, m, v


def gpt2_step(cfg, flat_params, inputs, targets=None, dloss=0.0, want_grads=True,
              want_logits=False, grads=None):
    """One micro-step.  Returns dict(mean_loss, losses, logits, grads)."""
    c = config(cfg)
    flat_params = _f64(flat_params)
    inputs = _i32(inputs); B, T = inputs.shape
    tg = None if targets is None else _i32(targets)
    BT = B * T
    losses = np.empty(BT)
    logits = np.empty((BT, cfg.padded_vocab_size)) if want_logits else None
    g = None
    if want_grads and tg is not None:
        g = np.zeros_like(flat_params) if grads is None else _f64(grads).copy()
    mean = lib().orc_gpt2_step(ctypes.byref(c), _p(flat_params), _p(inputs), _p(tg), B, T,
                               float(dloss), _p(losses), _p(logits), _p(g))
    if mean == -2.0:
        raise ValueError("oracle rejected the arguments")
    return {"mean_loss": mean, "losses": losses.reshape(B, T) if tg is not None else None,
            "logits": None if logits is None else logits.reshape(B, T, -1), "grads": g}


def adamw_sr(params_bf16, grads, m, v, lr, beta1, beta2, eps, wd, t, seed):
    """train_gpt2.cu, adamw_kernel3 without master weights, in fp32 with the
    page's stochastic rounding (see gpt2_oracle.c).  params_bf16: uint16 bf16
    bit patterns; grads, m, v: float32.  Returns new (params, m, v)."""
    p = np.array(params_bf16, dtype=np.uint16)
    g = np.ascontiguousarray(grads, dtype=np.float32)
    m2 = np.array(m, dtype=np.float32)
    v2 = np.array(v, dtype=np.float32)
    f32p = ctypes.POINTER(ctypes.c_float)
    lib().orc_adamw_sr(p.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), g.ctypes.data_as(f32p),
                       m2.ctypes.data_as(f32p), v2.ctypes.data_as(f32p), p.size, lr, beta1, beta2, eps, wd, int(t),
                       int(seed))
    return p, m2, v2


def xorshift_u32(state):
    """train_gpt2.cu, random_u32.  Returns (value, new state)."""
    s = ctypes.c_uint64(int(state))
    r = lib().orc_xorshift_u32(ctypes.byref(s))
    return int(r), int(s.value)


def noise2d(x, y, seed):
    """train_gpt2.cu, Get2dNoiseUint."""
    return int(lib().orc_noise2d(int(x), int(y), int(seed)))


def sr_bf16(x, r):
    """train_gpt2.cu, stochastic_rounding of the fp32 value x with threshold r
    (0 <= r < 2^16); returns the bf16 bit pattern."""
    return int(lib().orc_sr_bf16(float(np.float32(x)), int(r)))


def sample_softmax(logits, V, coin):
    """train_gpt2.cu, sample_softmax: the index drawn from softmax(logits[:V])
    by inverse CDF with coin in [0, 1): the smallest i with
    coin * sum_j p_j < p_0 + ... + p_i (p_j = exp(z_j - max z); the maximum
    cancels in exact arithmetic), V - 1 if none.  fp64, sums in index order."""
    z = np.asarray(logits, np.float64)[:V]
    cdf = np.cumsum(np.exp(z - z.max()))
    i = int(np.searchsorted(cdf, float(coin) * cdf[-1], side="right"))
    return min(i, V - 1)


def generate(cfg, flat_params, tokens, coins, t_begin, t_end):
    """train_gpt2.cu, the generation loop: for t = t_begin .. t_end - 1, a full
    forward without targets over tokens [B,T], then every row b draws its
    token at t from the logits at t - 1 with coin coins[t - t_begin][b].
    Returns the updated tokens (int32 [B,T])."""
    tokens = np.array(tokens, np.int32)
    for t in range(t_begin, t_end):
        z = gpt2_step(cfg, flat_params, tokens, want_grads=False, want_logits=True)["logits"]
        for b in range(tokens.shape[0]):
            tokens[b, t] = sample_softmax(z[b, t - 1], cfg.vocab_size, coins[t - t_begin][b])
    return tokens


def fused_linear_gelu_softmax(X, W, b, rows=None):
    X = _f64(X); W = _f64(W); b = _f64(b)
    M, K = X.shape; N = W.shape[0]
    r = None if rows is None else _i32(rows)
    R = M if r is None else r.size
    Y = np.empty((R, N))
    lib().orc_fused_linear_gelu_softmax(_p(Y), _p(X), _p(W), _p(b), M, K, N, _p(r), 0 if r is None else R)
    return Y
