"""Seeded synthetic inputs for the GPT-2 training step.

This module is shared by the CPU oracle, the HIP path's tests, ``bench.py`` and the smoke
run. It only *draws* inputs: token streams, initial parameter tensors and the workload
table. It holds none of the step's arithmetic (no LayerNorm, attention, loss, gradient or
optimizer math), so neither side of a parity check can inherit a mistake from the other
through it.

Workloads (sizes of the GPT-2 family as the lecture notes describe it, "Karpathy's Zero to
Hero, Lecture 9" notes, chapter 0:02-3:36 and the "Code you'll write" GPTConfig; the 1558M
row uses the 48-layer, 1600-wide shape from the same chapter and the 25 heads named in
chapter 2:06:39):

* ``tiny``        L=2,  H=2,  C=64,   T=64,   B=4,  V=Vp=256,          fp32
* ``gpt2_fwd``    L=12, H=12, C=768,  T=1024, B=4,  V=50257, Vp=50304, forward only
* ``gpt2_step``   L=12, H=12, C=768,  T=1024, B=16, V=50257, Vp=50304, full step
* ``gpt2_accum``  as gpt2_step, 32 micro-steps per optimizer step (2**19 tokens)
* ``gpt2_xl``     L=48, H=25, C=1600, T=1024, B=4,  V=50257, Vp=50304, full step
* ``gpt2_ctx2048`` the 124M widths at GPT-3's context: block_size = T = 2048, B=32 per
  micro-step, 8 micro-steps per optimizer step (2**19 tokens, about half a million), the
  setting chapter 3:43:45-3:59:10 names for matching GPT-3 (and chapter 2:14:58: GPT-3 mainly
  doubles GPT-2's context)

Token streams: the lecture's data (Tiny Shakespeare, FineWeb-Edu) is not available, so a
seeded finite Zipf(1.1) law over the real vocabulary stands in for natural-language token
frequency: P(id = k) is proportional to (k+1)**-1.1 for k in [0, V). Ids are drawn by
inverse-CDF lookup of ``numpy.random.default_rng(seed).random()``. Each micro-batch takes
B*T+1 consecutive ids; inputs are the first B*T and targets the last B*T (the "B*T+1" trick
of chapter 41:44-52:38).

Parameters: drawn per the initialization the notes give in chapter 1:13:27-1:22:16 and the
``_init_weights`` excerpt: N(0, 0.02) for every Linear weight and both embedding tables,
std scaled by (2*n_layer)**-0.5 for the two residual projections (``attn.c_proj`` and
``mlp.c_proj``), zero biases, LayerNorm gain 1 and bias 0. ``randomize_affine=True`` also
gives the biases and LayerNorm parameters random values so that a parity check exercises
every term of the step, not only the ones that survive a zero bias.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "param_spec", "init_params", "zipf_cdf",
    "draw_tokens", "token_batch", "micro_batches", "count_params",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    n_layer: int
    n_head: int
    n_embd: int
    block_size: int
    vocab_size: int          # V: ids are drawn from [0, V)
    padded_vocab_size: int   # Vp: rows of wte and width of the softmax
    batch: int               # B per micro-step
    seq_len: int             # T
    dtype: str               # "fp32" or "bf16"
    tokens: str              # "uniform" or "zipf"
    micro_steps: int = 1
    lr: float = 6e-4
    seed_base: int = 0       # weights use seed_base+1000, tokens seed_base+2000

    @property
    def mlp_hidden(self) -> int:
        return 4 * self.n_embd

    @property
    def head_dim(self) -> int:
        return self.n_embd // self.n_head

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS: Dict[str, Workload] = {
    "tiny": Workload("tiny", 2, 2, 64, 64, 256, 256, 4, 64, "fp32", "uniform", seed_base=1),
    "gpt2_fwd": Workload("gpt2_fwd", 12, 12, 768, 1024, 50257, 50304, 4, 1024, "bf16", "zipf",
                         seed_base=2),
    "gpt2_step": Workload("gpt2_step", 12, 12, 768, 1024, 50257, 50304, 16, 1024, "bf16", "zipf",
                          seed_base=3),
    # learning rate of the cosine schedule at step 100 (still in the 715-step warmup)
    "gpt2_accum": Workload("gpt2_accum", 12, 12, 768, 1024, 50257, 50304, 16, 1024, "bf16", "zipf",
                           micro_steps=32, lr=6e-4 * 101 / 715, seed_base=4),
    "gpt2_xl": Workload("gpt2_xl", 48, 25, 1600, 1024, 50257, 50304, 4, 1024, "bf16", "zipf",
                        seed_base=5),
    "gpt2_ctx2048": Workload("gpt2_ctx2048", 12, 12, 768, 2048, 50257, 50304, 32, 2048, "bf16", "zipf",
                             micro_steps=8, lr=6e-4 * 101 / 715, seed_base=6),
}


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.replace(**overrides) if overrides else w


def param_spec(w: Workload) -> List[Tuple[str, Tuple[int, ...], str]]:
    """(name, shape, init kind) for every parameter tensor, in Hugging Face naming.

    Linear weights are [out, in]. ``lm_head`` has no tensor of its own: it is ``wte``.
    Init kinds: "normal", "normal_resid", "zeros", "ones".
    """
    C, F, L = w.n_embd, w.mlp_hidden, w.n_layer
    spec = [("wte", (w.padded_vocab_size, C), "normal"), ("wpe", (w.block_size, C), "normal")]
    for i in range(L):
        p = f"h.{i}."
        spec += [
            (p + "ln_1.weight", (C,), "ones"), (p + "ln_1.bias", (C,), "zeros"),
            (p + "attn.c_attn.weight", (3 * C, C), "normal"), (p + "attn.c_attn.bias", (3 * C,), "zeros"),
            (p + "attn.c_proj.weight", (C, C), "normal_resid"), (p + "attn.c_proj.bias", (C,), "zeros"),
            (p + "ln_2.weight", (C,), "ones"), (p + "ln_2.bias", (C,), "zeros"),
            (p + "mlp.c_fc.weight", (F, C), "normal"), (p + "mlp.c_fc.bias", (F,), "zeros"),
            (p + "mlp.c_proj.weight", (C, F), "normal_resid"), (p + "mlp.c_proj.bias", (C,), "zeros"),
        ]
    spec += [("ln_f.weight", (C,), "ones"), ("ln_f.bias", (C,), "zeros")]
    return spec


def init_params(w: Workload, seed: int | None = None, dtype=np.float32,
                randomize_affine: bool = False) -> Dict[str, np.ndarray]:
    """Draw the initial parameters of workload ``w`` (see module docstring)."""
    rng = np.random.default_rng(w.seed_base + 1000 if seed is None else seed)
    std = 0.02
    resid_std = std * (2 * w.n_layer) ** -0.5
    out: Dict[str, np.ndarray] = {}
    for name, shape, kind in param_spec(w):
        if kind == "normal" or kind == "normal_resid":
            s = std if kind == "normal" else resid_std
            a = rng.standard_normal(shape, dtype=np.float32)
            a *= np.float32(s)
        elif kind == "zeros":
            a = (rng.standard_normal(shape, dtype=np.float32) * np.float32(0.02)
                 if randomize_affine else np.zeros(shape, np.float32))
        else:  # ones
            a = (np.float32(1.0) + rng.standard_normal(shape, dtype=np.float32) * np.float32(0.1)
                 if randomize_affine else np.ones(shape, np.float32))
        out[name] = a.astype(dtype, copy=False)
    return out


_CDF_CACHE: Dict[Tuple[int, float], np.ndarray] = {}


def zipf_cdf(V: int, s: float = 1.1) -> np.ndarray:
    key = (V, s)
    if key not in _CDF_CACHE:
        wts = np.arange(1, V + 1, dtype=np.float64) ** (-s)
        cdf = np.cumsum(wts)
        cdf /= cdf[-1]
        _CDF_CACHE[key] = cdf
    return _CDF_CACHE[key]


def draw_tokens(rng: np.random.Generator, n: int, V: int, kind: str) -> np.ndarray:
    """``n`` token ids in [0, V) as int32."""
    if kind == "uniform":
        return rng.integers(0, V, size=n, dtype=np.int64).astype(np.int32)
    if kind == "zipf":
        u = rng.random(n)
        ids = np.searchsorted(zipf_cdf(V), u, side="right")
        return np.minimum(ids, V - 1).astype(np.int32)
    raise ValueError(kind)


def token_batch(w: Workload, rng: np.random.Generator, batch: int | None = None
                ) -> Tuple[np.ndarray, np.ndarray]:
    """One micro-batch (x, y), each int32 [B, T], from B*T+1 consecutive ids."""
    B = w.batch if batch is None else batch
    T = w.seq_len
    buf = draw_tokens(rng, B * T + 1, w.vocab_size, w.tokens)
    return buf[:-1].reshape(B, T).copy(), buf[1:].reshape(B, T).copy()


def micro_batches(w: Workload, k: int | None = None, batch: int | None = None,
                  seed: int | None = None) -> List[Tuple[np.ndarray, np.ndarray]]:
    """``k`` micro-batches drawn sequentially from one generator seeded for ``w``."""
    rng = np.random.default_rng(w.seed_base + 2000 if seed is None else seed)
    k = w.micro_steps if k is None else k
    return [token_batch(w, rng, batch) for _ in range(k)]


def count_params(w: Workload, vocab_rows: int | None = None) -> Tuple[int, int, int, int]:
    """(decayed tensors, decayed params, other tensors, other params); wte counted once."""
    nd = pd = no = po = 0
    for name, shape, _ in param_spec(w):
        n = math.prod(shape)
        if name == "wte" and vocab_rows is not None:
            n = vocab_rows * shape[1]
        if len(shape) >= 2:
            nd += 1
            pd += n
        else:
            no += 1
            po += n
    return nd, pd, no, po
