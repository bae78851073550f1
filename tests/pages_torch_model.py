"""A second, independent description of the step, in PyTorch library routines (CPU, float64).

It follows the model the lecture notes print ("Karpathy's Zero to Hero, Lecture 9" notes,
section "Code you'll write": MLP, Block, causal self-attention via
``F.scaled_dot_product_attention(is_causal=True)``, the GPT skeleton with ``nn.LayerNorm``,
``nn.GELU(approximate='tanh')``, tied lm_head, ``F.cross_entropy``; the optimizer step with
``clip_grad_norm_`` and ``torch.optim.AdamW`` in two groups, chapter 2:25:57-2:34:49).
Gradients come from autograd. It is used only to pin the numpy oracle's hand-written
forward, backward and optimizer: it never sees the HIP library.
"""
from __future__ import annotations

import torch
import torch.nn as nn
import torch.nn.functional as F


class MLP(nn.Module):
    def __init__(self, C):
        super().__init__()
        self.c_fc = nn.Linear(C, 4 * C)
        self.gelu = nn.GELU(approximate="tanh")
        self.c_proj = nn.Linear(4 * C, C)

    def forward(self, x):
        return self.c_proj(self.gelu(self.c_fc(x)))


class Attn(nn.Module):
    def __init__(self, C, H):
        super().__init__()
        self.H = H
        self.c_attn = nn.Linear(C, 3 * C)
        self.c_proj = nn.Linear(C, C)

    def forward(self, x):
        B, T, C = x.size()
        q, k, v = self.c_attn(x).split(C, dim=2)
        q, k, v = (t.view(B, T, self.H, C // self.H).transpose(1, 2) for t in (q, k, v))
        y = F.scaled_dot_product_attention(q, k, v, is_causal=True)
        return self.c_proj(y.transpose(1, 2).contiguous().view(B, T, C))


class Block(nn.Module):
    def __init__(self, C, H):
        super().__init__()
        self.ln_1 = nn.LayerNorm(C)
        self.attn = Attn(C, H)
        self.ln_2 = nn.LayerNorm(C)
        self.mlp = MLP(C)

    def forward(self, x):
        x = x + self.attn(self.ln_1(x))
        return x + self.mlp(self.ln_2(x))


class GPT(nn.Module):
    def __init__(self, L, H, C, block_size, vocab):
        super().__init__()
        self.transformer = nn.ModuleDict(dict(
            wte=nn.Embedding(vocab, C), wpe=nn.Embedding(block_size, C),
            h=nn.ModuleList([Block(C, H) for _ in range(L)]), ln_f=nn.LayerNorm(C)))
        self.lm_head = nn.Linear(C, vocab, bias=False)
        self.transformer.wte.weight = self.lm_head.weight

    def forward(self, idx, targets=None):
        B, T = idx.size()
        pos = torch.arange(0, T, dtype=torch.long)
        x = self.transformer.wte(idx) + self.transformer.wpe(pos)
        for blk in self.transformer.h:
            x = blk(x)
        logits = self.lm_head(self.transformer.ln_f(x))
        loss = None
        if targets is not None:
            loss = F.cross_entropy(logits.view(-1, logits.size(-1)), targets.view(-1))
        return logits, loss


def _torch_name(name: str) -> str:
    if name in ("wte", "wpe"):
        return f"transformer.{name}.weight"
    return "transformer." + name


def build(params, L, H):
    """GPT in float64 holding the given numpy parameters (names as in ``synthetic``)."""
    Vp, C = params["wte"].shape
    model = GPT(L, H, C, params["wpe"].shape[0], Vp).double()
    sd = model.state_dict()
    with torch.no_grad():
        for k, v in params.items():
            sd[_torch_name(k)].copy_(torch.from_numpy(v.astype("float64")))
    return model


def grads_of(model, params):
    named = dict(model.named_parameters())
    return {k: named[_torch_name(k)].grad.detach().numpy().copy() for k in params}


def params_of(model, params):
    named = dict(model.named_parameters())
    return {k: named[_torch_name(k)].detach().numpy().copy() for k in params}


def optimizer(model, lr, betas=(0.9, 0.95), eps=1e-8, weight_decay=0.1):
    """Two groups by tensor dimension, as configure_optimizers does."""
    ps = [p for p in model.parameters() if p.requires_grad]
    decay = [p for p in ps if p.dim() >= 2]
    nodecay = [p for p in ps if p.dim() < 2]
    return torch.optim.AdamW([{"params": decay, "weight_decay": weight_decay},
                              {"params": nodecay, "weight_decay": 0.0}],
                             lr=lr, betas=betas, eps=eps, foreach=False)
