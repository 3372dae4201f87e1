"""Shared test helpers: run one GPT-2 micro-step through the HIP library (C ABI)
and through the oracle on identical seeded inputs."""

from __future__ import annotations

import sys

import numpy as np

import synthetic as S

PARAM_NAMES = S.PARAM_NAMES


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def cosine(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def make_inputs(cfg, B, T, n_micro=1, dist="uniform", data_seed=S.DATA_SEED, init_seed=S.INIT_SEED,
                perturb=False, bf16=False):
    params = S.init_params(cfg, seed=init_seed, perturb=perturb)
    if bf16:
        params = {k: S.round_to_bf16(v) for k, v in params.items()}
    stream = S.token_stream(n_micro * B * T + 1, cfg.vocab_size, seed=data_seed, dist=dist)
    batches = [S.batch(stream, i, B, T) for i in range(n_micro)]
    return params, batches


def oracle_step(cfg, params, batches, dloss=0.0, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0, t=1):
    """Oracle micro-steps (accumulating grads) + one AdamW update."""
    import oracle
    flat = oracle.pack_params(cfg, params)
    grads = np.zeros_like(flat)
    losses, means = [], []
    for x, y in batches:
        r = oracle.gpt2_step(cfg, flat, x, y, dloss=dloss, grads=grads)
        grads = r["grads"]
        losses.append(r["losses"])
        means.append(r["mean_loss"])
    newp, m, v = oracle.adamw(flat, grads, np.zeros_like(flat), np.zeros_like(flat), lr, beta1, beta2, eps, wd, t)
    shapes = S.param_shapes(cfg)
    return {"losses": losses, "means": means,
            "grads": oracle.unpack(cfg, grads, shapes), "params": oracle.unpack(cfg, newp, shapes),
            "m": oracle.unpack(cfg, m, shapes), "v": oracle.unpack(cfg, v, shapes)}


def gpu_step(cfg, precision, params, batches, dloss=0.0, lr=1e-4, beta1=0.9, beta2=0.999, eps=1e-8, wd=0.0,
             t=1, model=None, keep=False):
    """HIP micro-steps + one AdamW update, through the C ABI."""
    import torch
    from transformer_lm_step_amd.model import GPT2
    B, T = batches[0][0].shape
    if model is None:
        model = GPT2(cfg, precision, B, T)
        model.init(model.pack(params))
    dev = model.device
    model.zero_grad()
    losses, means = [], []
    for x, y in batches:
        xi = torch.from_numpy(x.reshape(-1)).to(dev)
        yi = torch.from_numpy(y.reshape(-1)).to(dev)
        lo = torch.empty(B * T, dtype=torch.float32, device=dev)
        mn = torch.empty(1, dtype=torch.float32, device=dev)
        model.forward(xi, yi, lo, mn)
        model.backward(dloss)
        torch.cuda.synchronize()
        losses.append(lo.cpu().numpy().reshape(B, T).astype(np.float64))
        means.append(float(mn.cpu()))
    grads = model.grads().cpu().numpy().astype(np.float64)
    model.update(lr, beta1, beta2, eps, wd, t)
    torch.cuda.synchronize()
    if model.precision == 1:
        newp = model.master().cpu().numpy().astype(np.float64)
    else:
        newp = model.params().float().cpu().numpy().astype(np.float64)
    res = {"losses": losses, "means": means, "grads": model.unpack(grads), "params": model.unpack(newp),
           "m": model.unpack(model.adam_m().cpu().numpy().astype(np.float64)),
           "v": model.unpack(model.adam_v().cpu().numpy().astype(np.float64)),
           "code": model.check()}
    if keep:
        res["model"] = model
    else:
        model.close()
    return res
