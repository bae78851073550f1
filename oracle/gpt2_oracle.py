"""CPU oracle for one GPT-2 training step.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or execute this
module: only the tests, the smoke check and the benchmark's CPU-baseline leg use it. It
shares no code with the HIP library: it receives the same seeded inputs (from the
``synthetic`` module) and computes the step from the plain definitions, in numpy, in the
floating-point type of its inputs (float64 for parity checks unless a caller asks otherwise).

Sources. The step is the one described across five web pages about reproducing GPT-2
(124M). Citations below name the page and the section:

* [LVN] "Karpathy's Zero to Hero, Lecture 9: Reproduce GPT-2 (124M) -- notes, code and
  timestamps" (longvideonotes.com): chapter headings are quoted by their time range, and
  "Code you'll write" is the section of short code excerpts.
* [R4]  "reproduce-gpt2" README: sections "Architecture", "Implementation details".
* [L10] "Lecture 10: Reproducing GPT-2 (124M) from Scratch": section "Key ideas".

What is computed (each function cites the passage it follows):

    x    = wte[idx] + wpe[0..T)
    per block:  x = x + attn(ln_1(x));  x = x + mlp(ln_2(x))        (pre-LayerNorm)
    attn: qkv = h Wqkv^T + b, split q|k|v, heads as batch, causal softmax(q k^T/sqrt(hs)) v,
          heads re-assembled, output projection c_proj
    mlp:  c_fc (C -> 4C), GELU tanh approximation, c_proj (4C -> C)
    hf   = ln_f(x);  z = hf wte^T  (tied lm_head, all Vp columns);  loss = mean CE
    backward: the chain rule written out for every op, gradients of the two uses of wte add
    clip: global L2 norm over all gradients, coefficient min(1, max_norm/(norm+1e-6))
    AdamW: decoupled weight decay on tensors with >= 2 dims, bias-corrected moments
    evaluation: per-position losses reduced per row over a mask (masked_row_losses)
    sampling: softmax, the k most probable tokens, an inverse-CDF draw (topk_sample)

Readings where the pages leave a detail open:

* LayerNorm is ``nn.LayerNorm(n_embd)`` with its defaults: eps 1e-5, biased variance.
* The attention scale is the library default 1/sqrt(head_dim) (no scale is passed).
* The softmax runs over all padded vocabulary columns: the padded rows of wte become extra
  logits ([LVN] chapter 2:06:39-2:14:58).
* AdamW is PyTorch's: p <- p(1 - lr*wd) first, then m, v, bias correction, eps added after
  the square root ([LVN] chapters 52:38-1:06:18 and 2:25:57-2:34:49; [R4] "decoupled").
* The clip coefficient and returned norm follow ``clip_grad_norm_`` (pre-clip norm returned).

Memory: attention is evaluated one batch element at a time and the probabilities are
recomputed in the backward pass, and the lm_head/cross-entropy rows are processed in row
chunks. Every row's arithmetic is unchanged by this; only when results are summed over
rows (the lm_head weight gradient) does the chunking fix a summation order.
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Tuple

import numpy as np

LN_EPS = 1e-5
GELU_C = math.sqrt(2.0 / math.pi)
GELU_A = 0.044715
CE_ROW_CHUNK = 2048


# ----------------------------------------------------------------------------- pieces
def layernorm_forward(x: np.ndarray, w: np.ndarray, b: np.ndarray, eps: float = LN_EPS):
    """nn.LayerNorm over the last axis ([LVN] "Code you'll write", Block; defaults: eps 1e-5,
    biased variance). Returns (out, xhat, rstd)."""
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    xhat = (x - mean) * rstd
    return xhat * w + b, xhat, rstd


def layernorm_backward(dout: np.ndarray, xhat: np.ndarray, rstd: np.ndarray, w: np.ndarray):
    """Chain rule through y = xhat*w + b with xhat = (x - mean)*rstd (per row).
    Returns (dx, dw, db)."""
    dxhat = dout * w
    m1 = dxhat.mean(axis=-1, keepdims=True)
    m2 = (dxhat * xhat).mean(axis=-1, keepdims=True)
    dx = rstd * (dxhat - m1 - xhat * m2)
    rows = dout.reshape(-1, dout.shape[-1])
    xh = xhat.reshape(-1, xhat.shape[-1])
    return dx, (rows * xh).sum(axis=0), rows.sum(axis=0)


def gelu_tanh(u: np.ndarray) -> np.ndarray:
    """GELU, tanh approximation ([LVN] chapter 13:34-28:07 and "Code you'll write", MLP):
    0.5 u (1 + tanh(sqrt(2/pi) (u + 0.044715 u^3)))."""
    return 0.5 * u * (1.0 + np.tanh(GELU_C * (u + GELU_A * u ** 3)))


def gelu_tanh_grad(u: np.ndarray) -> np.ndarray:
    """d gelu_tanh / du, differentiated by hand."""
    w = GELU_C * (u + GELU_A * u ** 3)
    t = np.tanh(w)
    return 0.5 * (1.0 + t) + 0.5 * u * (1.0 - t * t) * GELU_C * (1.0 + 3.0 * GELU_A * u * u)


def split_heads(qkv: np.ndarray, n_head: int):
    """qkv [T, 3C] -> q, k, v each [H, T, hs]: split by n_embd in q, k, v order, then view as
    (T, H, hs) and move heads to the front ([LVN] "Code you'll write", attention forward)."""
    T, C3 = qkv.shape
    C = C3 // 3
    hs = C // n_head
    q, k, v = qkv[:, :C], qkv[:, C:2 * C], qkv[:, 2 * C:]
    return tuple(a.reshape(T, n_head, hs).transpose(1, 0, 2) for a in (q, k, v))


def causal_probs(q: np.ndarray, k: np.ndarray) -> np.ndarray:
    """The attention matrix of the plain four-step definition ([LVN] chapter 13:34-28:07):
    scores q k^T / sqrt(hs), future positions masked, softmax over each row (max, exponent,
    sum, normalize). q, k: [H, T, hs] -> P [H, T, T]."""
    hs = q.shape[-1]
    T = q.shape[-2]
    s = np.matmul(q, k.transpose(0, 2, 1)) / math.sqrt(hs)
    future = np.triu(np.ones((T, T), dtype=bool), k=1)
    s = np.where(future, -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    e = np.exp(s)
    return e / e.sum(axis=-1, keepdims=True)


def attention_forward(qkv: np.ndarray, n_head: int) -> np.ndarray:
    """Causal multi-head self-attention on one sequence: qkv [T, 3C] -> y [T, C] (heads
    re-assembled side by side, [LVN] "Code you'll write", attention forward)."""
    q, k, v = split_heads(qkv, n_head)
    y = np.matmul(causal_probs(q, k), v)             # [H, T, hs]
    T = qkv.shape[0]
    return y.transpose(1, 0, 2).reshape(T, -1)


def attention_backward(dy: np.ndarray, qkv: np.ndarray, n_head: int) -> np.ndarray:
    """Gradient of attention_forward w.r.t. qkv for one sequence (P recomputed).
    With S = q k^T/sqrt(hs), P = softmax(S), Y = P V:
    dV = P^T dY, dP = dY V^T, dS = P * (dP - rowsum(P * dP)), dQ = dS K/sqrt(hs),
    dK = dS^T Q/sqrt(hs)."""
    T, C3 = qkv.shape
    C = C3 // 3
    hs = C // n_head
    q, k, v = split_heads(qkv, n_head)
    P = causal_probs(q, k)
    dyh = dy.reshape(T, n_head, hs).transpose(1, 0, 2)
    dv = np.matmul(P.transpose(0, 2, 1), dyh)
    dP = np.matmul(dyh, v.transpose(0, 2, 1))
    dS = P * (dP - (P * dP).sum(axis=-1, keepdims=True))
    dq = np.matmul(dS, k) / math.sqrt(hs)
    dk = np.matmul(dS.transpose(0, 2, 1), q) / math.sqrt(hs)
    out = np.empty_like(qkv)
    for j, g in enumerate((dq, dk, dv)):
        out[:, j * C:(j + 1) * C] = g.transpose(1, 0, 2).reshape(T, C)
    return out


def cross_entropy_rows(z: np.ndarray, y: np.ndarray):
    """Per-row cross-entropy of logits z [n, Vp] against targets y [n] (F.cross_entropy on
    the flattened logits, [LVN] "Code you'll write", forward with loss). All Vp columns,
    padded ones included, are in the softmax. Returns (loss per row, softmax)."""
    mx = z.max(axis=-1, keepdims=True)
    e = np.exp(z - mx)
    se = e.sum(axis=-1, keepdims=True)
    lse = (mx + np.log(se))[:, 0]
    loss = lse - z[np.arange(z.shape[0]), y]
    return loss, e / se


# ----------------------------------------------------------------------------- model
def _p(params, name):
    return params[name]


def forward(params: Dict[str, np.ndarray], n_layer: int, n_head: int,
            idx: np.ndarray, targets: Optional[np.ndarray] = None,
            want_logits: bool = True, want_cache: bool = True):
    """The model forward ([LVN] "Code you'll write", forward with loss; [L10] "Key ideas" on
    the pre-normalization residual stream; [R4] "Architecture").

    idx, targets: int [B, T]. Returns dict with ``loss`` (mean CE, or None), ``logits``
    [B, T, Vp] (if asked) and ``cache`` (activations for ``backward``)."""
    wte, wpe = params["wte"], params["wpe"]
    B, T = idx.shape
    assert T <= wpe.shape[0], "sequence longer than block_size"
    x = wte[idx] + wpe[:T][None, :, :]                      # [B, T, C]
    C = x.shape[-1]
    cache = {"idx": idx, "layers": []}
    for l in range(n_layer):
        p = f"h.{l}."
        c = {"x_in": x}
        h1, c["xhat1"], c["rstd1"] = layernorm_forward(x, params[p + "ln_1.weight"], params[p + "ln_1.bias"])
        qkv = h1 @ params[p + "attn.c_attn.weight"].T + params[p + "attn.c_attn.bias"]
        yatt = np.stack([attention_forward(qkv[b], n_head) for b in range(B)])
        x = x + yatt @ params[p + "attn.c_proj.weight"].T + params[p + "attn.c_proj.bias"]
        c["x_mid"] = x
        h2, c["xhat2"], c["rstd2"] = layernorm_forward(x, params[p + "ln_2.weight"], params[p + "ln_2.bias"])
        u = h2 @ params[p + "mlp.c_fc.weight"].T + params[p + "mlp.c_fc.bias"]
        a = gelu_tanh(u)
        x = x + a @ params[p + "mlp.c_proj.weight"].T + params[p + "mlp.c_proj.bias"]
        c.update(h1=h1, qkv=qkv, yatt=yatt, h2=h2, u=u, a=a)
        if want_cache:
            cache["layers"].append(c)
    hf, xhatf, rstdf = layernorm_forward(x, params["ln_f.weight"], params["ln_f.bias"])
    cache.update(hf=hf, xhatf=xhatf, rstdf=rstdf)
    n = B * T
    hf2 = hf.reshape(n, C)
    logits = np.empty((n, wte.shape[0]), dtype=hf.dtype) if want_logits else None
    loss = None
    if targets is not None:
        tf = targets.reshape(n)
        losses = np.empty(n, dtype=hf.dtype)
        probs = []
    for r0 in range(0, n, CE_ROW_CHUNK):
        r1 = min(n, r0 + CE_ROW_CHUNK)
        z = hf2[r0:r1] @ wte.T                               # tied lm_head, no bias
        if want_logits:
            logits[r0:r1] = z
        if targets is not None:
            lrow, pr = cross_entropy_rows(z, tf[r0:r1])
            losses[r0:r1] = lrow
            if want_cache:
                probs.append(pr)
    if targets is not None:
        loss = losses.mean()
        cache["targets"] = targets
        if want_cache:
            cache["probs"] = probs
    out = {"loss": loss, "cache": cache if want_cache else None}
    if targets is not None:
        out["losses"] = losses.reshape(B, T)
    if want_logits:
        out["logits"] = logits.reshape(B, T, -1)
    return out


def masked_row_losses(losses: np.ndarray, mask: Optional[np.ndarray] = None):
    """Forward-only scores ([LVN] chapter 3:22:33-3:28:16, the validation loss: the mean loss
    with no backward pass; chapter 3:28:16-3:41:50, completion scoring: a row's score is the
    mean cross-entropy over the tokens its mask marks, the lowest score wins).

    losses: per-position cross-entropy [B, T] (``forward(...)["losses"]``); mask: [B, T],
    nonzero selects (None: all). Returns (row_sum [B], row_mean [B], mean over every selected
    position of the batch); a row with nothing selected has mean 0, as does an empty batch."""
    sel = np.ones(losses.shape, dtype=bool) if mask is None else np.asarray(mask) != 0
    row_sum = np.where(sel, losses, 0.0).sum(axis=-1)
    count = sel.sum(axis=-1)
    row_mean = np.where(count > 0, row_sum / np.maximum(count, 1), 0.0)
    total = row_sum.sum() / count.sum() if count.sum() > 0 else 0.0
    return row_sum, row_mean, total


def topk_sample(logits: np.ndarray, k: int, u: float):
    """One draw of the sampling loop ([LVN] chapter 0:28:07-0:41:44 and the sampling code of
    chapter 3:22:33-3:28:16): softmax over every column of the last position's logits, keep
    the k most probable tokens, draw one in proportion to its probability.

    Readings: equal probabilities are ordered by lower token id; the draw is the inverse CDF
    of the uniform number u in [0, 1) over the k kept tokens in that order (the first whose
    cumulative renormalized probability exceeds u). Returns (token, kept ids, their
    renormalized probabilities)."""
    z = np.asarray(logits, dtype=np.float64)
    p = np.exp(z - z.max())
    p /= p.sum()
    order = np.lexsort((np.arange(z.size), -p))        # larger probability first, then lower id
    ids = order[:k]
    kept = p[ids] / p[ids].sum()
    cdf = np.cumsum(kept)
    i = int(np.searchsorted(cdf, u, side="right"))
    return int(ids[min(i, k - 1)]), ids, kept


def backward(params: Dict[str, np.ndarray], n_layer: int, n_head: int, cache, grad_scale: float = 1.0):
    """Gradients of ``grad_scale * loss`` w.r.t. every parameter, by the chain rule.

    ``grad_scale`` is the 1/micro_steps factor of gradient accumulation ([LVN] chapter
    2:34:49-2:46:43 and the optimizer-step excerpt: the loss is divided by the number of
    micro-steps before backward). The two uses of the tied wte add into one gradient
    ([LVN] chapter 1:06:18-1:13:27)."""
    idx, targets = cache["idx"], cache["targets"]
    B, T = idx.shape
    n = B * T
    wte = params["wte"]
    C = wte.shape[1]
    grads = {k: np.zeros_like(v) for k, v in params.items()}
    # cross-entropy + lm_head
    tf = targets.reshape(n)
    hf2 = cache["hf"].reshape(n, C)
    dhf = np.empty_like(hf2)
    for ci, r0 in enumerate(range(0, n, CE_ROW_CHUNK)):
        r1 = min(n, r0 + CE_ROW_CHUNK)
        dz = cache["probs"][ci].copy()
        dz[np.arange(r1 - r0), tf[r0:r1]] -= 1.0
        dz *= grad_scale / n
        dhf[r0:r1] = dz @ wte
        grads["wte"] += dz.T @ hf2[r0:r1]
    dx, grads["ln_f.weight"], grads["ln_f.bias"] = layernorm_backward(
        dhf.reshape(B, T, C), cache["xhatf"], cache["rstdf"], params["ln_f.weight"])
    for l in reversed(range(n_layer)):
        p = f"h.{l}."
        c = cache["layers"][l]
        # x_out = x_mid + a Wpr^T + bpr
        grads[p + "mlp.c_proj.bias"] = dx.reshape(n, C).sum(axis=0)
        grads[p + "mlp.c_proj.weight"] = dx.reshape(n, C).T @ c["a"].reshape(n, -1)
        da = dx @ params[p + "mlp.c_proj.weight"]
        du = da * gelu_tanh_grad(c["u"])
        grads[p + "mlp.c_fc.bias"] = du.reshape(n, -1).sum(axis=0)
        grads[p + "mlp.c_fc.weight"] = du.reshape(n, -1).T @ c["h2"].reshape(n, C)
        dh2 = du @ params[p + "mlp.c_fc.weight"]
        dln, grads[p + "ln_2.weight"], grads[p + "ln_2.bias"] = layernorm_backward(
            dh2, c["xhat2"], c["rstd2"], params[p + "ln_2.weight"])
        dx = dx + dln
        # x_mid = x_in + y Wo^T + bo
        grads[p + "attn.c_proj.bias"] = dx.reshape(n, C).sum(axis=0)
        grads[p + "attn.c_proj.weight"] = dx.reshape(n, C).T @ c["yatt"].reshape(n, C)
        dyatt = dx @ params[p + "attn.c_proj.weight"]
        dqkv = np.stack([attention_backward(dyatt[b], c["qkv"][b], n_head) for b in range(B)])
        grads[p + "attn.c_attn.bias"] = dqkv.reshape(n, -1).sum(axis=0)
        grads[p + "attn.c_attn.weight"] = dqkv.reshape(n, -1).T @ c["h1"].reshape(n, C)
        dh1 = dqkv @ params[p + "attn.c_attn.weight"]
        dln, grads[p + "ln_1.weight"], grads[p + "ln_1.bias"] = layernorm_backward(
            dh1, c["xhat1"], c["rstd1"], params[p + "ln_1.weight"])
        dx = dx + dln
    # embeddings: position rows sum over the batch, token rows scatter-add (ids repeat)
    grads["wpe"][:T] += dx.sum(axis=0)
    np.add.at(grads["wte"], idx.reshape(n), dx.reshape(n, C))
    return grads


def grad_norm(grads: Dict[str, np.ndarray]) -> float:
    """Global L2 norm over all gradient tensors: square everything, sum, square root
    ([LVN] chapter 2:14:58-2:25:57). wte is one tensor and is counted once."""
    return math.sqrt(sum(float(np.sum(np.asarray(g, np.float64) ** 2)) for g in grads.values()))


def clip_coefficient(norm: float, max_norm: float) -> float:
    """clip_grad_norm_: scale = max_norm/(norm + 1e-6), capped at 1."""
    return min(1.0, max_norm / (norm + 1e-6))


def decays(name: str, p: np.ndarray) -> bool:
    """Weight decay applies to tensors with two or more dimensions only ([LVN] chapter
    2:25:57-2:34:49; [R4] "Implementation details")."""
    return p.ndim >= 2


def adamw_update(p, g, m, v, t: int, lr: float, beta1: float, beta2: float, eps: float,
                 weight_decay: float):
    """One AdamW update of one tensor, in place (PyTorch's AdamW as shown in [LVN] chapter
    52:38-1:06:18): decoupled decay p *= 1 - lr*wd, then m = b1 m + (1-b1) g,
    v = b2 v + (1-b2) g^2, p -= lr * (m/(1-b1^t)) / (sqrt(v/(1-b2^t)) + eps)."""
    p *= (1.0 - lr * weight_decay)
    m *= beta1
    m += (1.0 - beta1) * g
    v *= beta2
    v += (1.0 - beta2) * g * g
    mhat = m / (1.0 - beta1 ** t)
    vhat = v / (1.0 - beta2 ** t)
    p -= lr * mhat / (np.sqrt(vhat) + eps)


def optimizer_step(params, grads, m, v, t: int, lr: float, beta1=0.9, beta2=0.95, eps=1e-8,
                   weight_decay=0.1, max_grad_norm=1.0) -> float:
    """Clip by the global norm, then AdamW on every tensor (in place). Returns the pre-clip
    norm ([LVN] "Code you'll write", one optimizer step)."""
    norm = grad_norm(grads)
    c = clip_coefficient(norm, max_grad_norm)
    for k in params:
        wd = weight_decay if decays(k, params[k]) else 0.0
        adamw_update(params[k], grads[k] * c, m[k], v[k], t, lr, beta1, beta2, eps, wd)
    return norm


def get_lr(it: int, max_lr: float = 6e-4, min_lr: float = 6e-5, warmup_steps: int = 715,
           max_steps: int = 19073) -> float:
    """Linear warmup then cosine decay to min_lr ([LVN] "Code you'll write", cosine
    learning-rate schedule with warmup; chapter 2:14:58-2:25:57)."""
    if it < warmup_steps:
        return max_lr * (it + 1) / warmup_steps
    if it > max_steps:
        return min_lr
    ratio = (it - warmup_steps) / (max_steps - warmup_steps)
    return min_lr + 0.5 * (1.0 + math.cos(math.pi * ratio)) * (max_lr - min_lr)


def train_step(params, n_layer, n_head, batches, grad_scale=None):
    """Forward+backward over micro-batches with the loss scaled by 1/k, gradients summed.
    Returns (sum of scaled losses, grads)."""
    k = len(batches)
    s = 1.0 / k if grad_scale is None else grad_scale
    total = None
    loss_accum = 0.0
    for x, y in batches:
        out = forward(params, n_layer, n_head, x, y, want_logits=False)
        loss_accum += float(out["loss"]) * s
        g = backward(params, n_layer, n_head, out["cache"], s)
        if total is None:
            total = g
        else:
            for kk in total:
                total[kk] += g[kk]
    return loss_accum, total
