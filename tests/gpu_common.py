"""Helpers shared by the GPU parity tests: building a library handle for a workload,
running the CPU oracle on the same seeded inputs, and the comparison metrics.

Comparison metrics (fixed per tensor):
* ``rel_max``: max |gpu - ref| / max |ref| over the tensor (fp32 check mode, bar 1e-4);
* ``cosine``: cosine similarity of the flattened tensors, in float64 (bf16 mode, bar 0.999).
"""
from __future__ import annotations

import functools
import sys

import numpy as np

import synthetic
from oracle import gpt2_oracle as O


def note(msg: str) -> None:
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def rel_max(a, ref) -> float:
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    return float(np.abs(a - ref).max() / (den if den > 0 else 1.0))


def cosine(a, b) -> float:
    a = np.asarray(a, np.float64).reshape(-1)
    b = np.asarray(b, np.float64).reshape(-1)
    na, nb = np.linalg.norm(a), np.linalg.norm(b)
    if na == 0 and nb == 0:
        return 1.0
    return float(a @ b / (na * nb))


def config_for(w, dtype, max_batch=None):
    import transformer_lm_step_amd as G
    return G.make_config(w.n_layer, w.n_head, w.n_embd, w.block_size, w.vocab_size, w.padded_vocab_size,
                         w.batch if max_batch is None else max_batch, dtype)


def make_step(w, dtype, max_batch=None, seed=0):
    import transformer_lm_step_amd as G
    return G.GPT2Step(config_for(w, dtype, max_batch), seed=seed)


def f64(params):
    return {k: v.astype(np.float64) for k, v in params.items()}


@functools.lru_cache(maxsize=8)
def oracle_step(name: str, overrides: tuple, batch: int, k: int, randomize: bool, want_logits: bool):
    """Oracle loss / grads / logits (float64) on the workload's seeded params and batches."""
    w = synthetic.workload(name, **dict(overrides))
    params = synthetic.init_params(w, randomize_affine=randomize)
    batches = synthetic.micro_batches(w, k, batch=batch)
    p64 = f64(params)
    if k == 1:
        x, y = batches[0]
        out = O.forward(p64, w.n_layer, w.n_head, x, y, want_logits=want_logits)
        g = O.backward(p64, w.n_layer, w.n_head, out["cache"], 1.0)
        return params, batches, float(out["loss"]), g, out.get("logits")
    loss, g = O.train_step(p64, w.n_layer, w.n_head, batches)
    return params, batches, loss, g, None
