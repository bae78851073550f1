"""Pins of the CPU oracle to things other than itself (no GPU needed).

* values the pages print (tests/golden/pages_values.json, each entry with its citation);
* an independent float64 PyTorch model written from the pages' code excerpts
  (tests/pages_torch_model.py): loss, logits, every gradient and the post-AdamW parameters;
* central finite differences of the loss on a very small model (every parameter tensor);
* closed forms and invariants: exact cross-entropy at wte = 0, causality, accumulation
  equivalence, the AdamW first step, LayerNorm / softmax / attention gradient identities.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import synthetic
from oracle import gpt2_oracle as O
from tests import pages_torch_model as PT

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_values.json")))


def _tiny(**kw):
    return synthetic.workload("tiny", **kw)


def _mini():
    # very small model for finite differences
    return synthetic.Workload("mini", 1, 2, 16, 8, 32, 32, 2, 8, "fp32", "uniform", seed_base=7)


def _f64(params):
    return {k: v.astype(np.float64) for k, v in params.items()}


# ----------------------------------------------------------------- values printed on the pages
def test_parameter_inventory_matches_pages():
    w = synthetic.workload("gpt2_step")
    nd, pd, no, po = synthetic.count_params(w)
    assert (nd, pd, no, po) == (GOLDEN["decayed_tensors"]["value"], GOLDEN["decayed_params"]["value"],
                                GOLDEN["nodecay_tensors"]["value"], GOLDEN["nodecay_params"]["value"])
    _, pd50257, _, po50257 = synthetic.count_params(w, vocab_rows=50257)
    assert pd50257 + po50257 == GOLDEN["params_total_vocab_50257"]["value"]
    assert w.padded_vocab_size == GOLDEN["padded_vocab"]["value"]
    assert w.padded_vocab_size % GOLDEN["padded_vocab"]["multiple_of"] == 0
    # the oracle's decay rule picks exactly the pages' 50 tensors
    params = {n: np.zeros(s, np.float32) for n, s, _ in synthetic.param_spec(w)}
    assert sum(O.decays(k, v) for k, v in params.items()) == 50


def test_uniform_guess_loss_value():
    g = GOLDEN["uniform_guess_loss"]
    assert abs(-math.log(1.0 / 50257) - g["value"]) <= g["abs_tol"]


def test_lr_schedule_pins():
    g = GOLDEN["lr_schedule"]
    kw = dict(max_lr=g["max_lr"], min_lr=g["min_lr"], warmup_steps=g["warmup_steps"], max_steps=g["max_steps"])
    assert O.get_lr(0, **kw) == pytest.approx(6e-4 / 715, rel=1e-12)
    assert O.get_lr(100, **kw) == pytest.approx(8.475524475524476e-05, rel=1e-12)
    assert O.get_lr(714, **kw) == pytest.approx(6e-4, rel=1e-12)
    assert O.get_lr(715, **kw) == pytest.approx(6e-4, rel=1e-12)
    assert O.get_lr(19073, **kw) == pytest.approx(6e-5, rel=1e-12)
    assert O.get_lr(30000, **kw) == 6e-5
    mid = (715 + 19073) // 2
    assert O.get_lr(mid, **kw) == pytest.approx(6e-5 + 0.5 * (1 + math.cos(math.pi * (mid - 715) / (19073 - 715))) * 5.4e-4)
    assert synthetic.workload("gpt2_accum").lr == pytest.approx(O.get_lr(100, **kw), rel=1e-12)


def test_tokens_per_optimizer_step():
    g = GOLDEN["tokens_per_opt_step"]
    w = synthetic.workload("gpt2_accum")
    assert w.batch * w.seq_len * w.micro_steps == g["value"] == 2 ** 19
    assert (w.batch, w.seq_len, w.micro_steps) == (g["micro_B"], g["T"], g["micro_steps"])


# ----------------------------------------------------------------- independent torch model
def _torch_step(params, w, x, y, lr):
    model = PT.build(params, w.n_layer, w.n_head)
    opt = PT.optimizer(model, lr)
    logits, loss = model(torch.from_numpy(x).long(), torch.from_numpy(y).long())
    loss.backward()
    g = PT.grads_of(model, params)
    norm = torch.nn.utils.clip_grad_norm_(model.parameters(), 1.0).item()
    opt.step()
    return logits.detach().numpy(), loss.item(), g, norm, PT.params_of(model, params)


@pytest.mark.parametrize("randomize", [False, True])
def test_oracle_matches_torch_float64(randomize):
    w = _tiny()
    params = _f64(synthetic.init_params(w, randomize_affine=randomize))
    (x, y), = synthetic.micro_batches(w, 1)
    t_logits, t_loss, t_grads, t_norm, t_after = _torch_step(params, w, x, y, lr=6e-4)

    out = O.forward(params, w.n_layer, w.n_head, x, y)
    np.testing.assert_allclose(out["logits"], t_logits, rtol=0, atol=1e-12)
    assert abs(out["loss"] - t_loss) <= 1e-12
    grads = O.backward(params, w.n_layer, w.n_head, out["cache"], 1.0)
    for k in params:
        scale = max(np.abs(t_grads[k]).max(), 1e-30)
        assert np.abs(grads[k] - t_grads[k]).max() / scale <= 1e-10, k
    p2 = {k: v.copy() for k, v in params.items()}
    m = {k: np.zeros_like(v) for k, v in params.items()}
    v = {k: np.zeros_like(v) for k, v in params.items()}
    norm = O.optimizer_step(p2, grads, m, v, 1, 6e-4)
    assert norm == pytest.approx(t_norm, rel=1e-12)
    for k in params:
        np.testing.assert_allclose(p2[k], t_after[k], rtol=0, atol=1e-12, err_msg=k)


def test_oracle_matches_torch_two_steps_with_clipping():
    """Second AdamW step (t=2, non-trivial moments) and a clip that actually scales."""
    w = _tiny()
    params = _f64(synthetic.init_params(w, randomize_affine=True))
    b1, b2 = synthetic.micro_batches(w, 2)
    model = PT.build(params, w.n_layer, w.n_head)
    opt = PT.optimizer(model, 1e-3)
    p = {k: v.copy() for k, v in params.items()}
    m = {k: np.zeros_like(v) for k, v in params.items()}
    v = {k: np.zeros_like(v) for k, v in params.items()}
    for t, (x, y) in enumerate((b1, b2), start=1):
        opt.zero_grad()
        _, loss = model(torch.from_numpy(x).long(), torch.from_numpy(y).long())
        (loss * 40.0).backward()           # large gradients so the clip coefficient < 1
        tn = torch.nn.utils.clip_grad_norm_(model.parameters(), 1.0).item()
        opt.step()
        out = O.forward(p, w.n_layer, w.n_head, x, y)
        g = O.backward(p, w.n_layer, w.n_head, out["cache"], 40.0)
        n = O.optimizer_step(p, g, m, v, t, 1e-3)
        assert n > 1.0 and n == pytest.approx(tn, rel=1e-12)
    after = PT.params_of(model, params)
    for k in params:
        np.testing.assert_allclose(p[k], after[k], rtol=0, atol=1e-12, err_msg=k)


# ----------------------------------------------------------------- finite differences
def test_finite_differences_every_tensor():
    w = _mini()
    params = _f64(synthetic.init_params(w, randomize_affine=True))
    (x, y), = synthetic.micro_batches(w, 1)
    out = O.forward(params, w.n_layer, w.n_head, x, y)
    grads = O.backward(params, w.n_layer, w.n_head, out["cache"], 1.0)
    rng = np.random.default_rng(0)
    h = 1e-6

    def loss_at(pp):
        return O.forward(pp, w.n_layer, w.n_head, x, y, want_logits=False, want_cache=False)["loss"]

    for k, p in params.items():
        flat = p.reshape(-1)
        picks = rng.choice(flat.size, size=min(12, flat.size), replace=False)
        # include the largest-gradient entry of each tensor
        picks = np.unique(np.append(picks, np.argmax(np.abs(grads[k].reshape(-1)))))
        gmax = np.abs(grads[k]).max()
        for i in picks:
            old = flat[i]
            flat[i] = old + h
            lp = loss_at(params)
            flat[i] = old - h
            lm = loss_at(params)
            flat[i] = old
            fd = (lp - lm) / (2 * h)
            an = grads[k].reshape(-1)[i]
            assert abs(fd - an) <= 1e-6 * max(gmax, 1e-3), (k, i, fd, an)


def test_finite_differences_components():
    rng = np.random.default_rng(3)
    h = 1e-6
    # LayerNorm
    x = rng.standard_normal((3, 10))
    wv = rng.standard_normal(10)
    bv = rng.standard_normal(10)
    dout = rng.standard_normal((3, 10))
    _, xhat, rstd = O.layernorm_forward(x, wv, bv)
    dx, dw, db = O.layernorm_backward(dout, xhat, rstd, wv)
    for i in range(3):
        for j in range(10):
            xp = x.copy(); xp[i, j] += h
            xm = x.copy(); xm[i, j] -= h
            fd = (np.sum(O.layernorm_forward(xp, wv, bv)[0] * dout) - np.sum(O.layernorm_forward(xm, wv, bv)[0] * dout)) / (2 * h)
            assert abs(fd - dx[i, j]) < 1e-7
    # GELU derivative
    u = np.linspace(-6, 6, 101)
    fd = (O.gelu_tanh(u + h) - O.gelu_tanh(u - h)) / (2 * h)
    np.testing.assert_allclose(O.gelu_tanh_grad(u), fd, atol=1e-8)
    # attention on one sequence
    T, C, H = 6, 8, 2
    qkv = rng.standard_normal((T, 3 * C))
    dy = rng.standard_normal((T, C))
    g = O.attention_backward(dy, qkv, H)
    for i in range(T):
        for j in range(3 * C):
            qp = qkv.copy(); qp[i, j] += h
            qm = qkv.copy(); qm[i, j] -= h
            fd = (np.sum(O.attention_forward(qp, H) * dy) - np.sum(O.attention_forward(qm, H) * dy)) / (2 * h)
            assert abs(fd - g[i, j]) < 1e-7


# ----------------------------------------------------------------- closed forms and invariants
def test_exact_cross_entropy_at_zero_wte():
    """wte = 0 makes every logit 0: loss = ln Vp exactly, dz = (1/Vp - onehot)/BT."""
    w = synthetic.workload("gpt2_step", n_layer=1, batch=1, seq_len=32)
    params = _f64(synthetic.init_params(w, randomize_affine=True))
    params["wte"][:] = 0.0
    (x, y), = synthetic.micro_batches(w, 1)
    out = O.forward(params, w.n_layer, w.n_head, x, y)
    assert abs(out["loss"] - math.log(50304)) <= 1e-12
    assert abs(out["loss"] - 10.825839875788878) <= 1e-12   # ln 50304, not ln 50257
    assert np.all(out["logits"] == 0.0)
    g = O.backward(params, w.n_layer, w.n_head, out["cache"], 1.0)
    # with wte = 0 the lm_head gradient is sum_n dz_n^T hf_n; padded rows only get 1/Vp terms
    hf = out["cache"]["hf"].reshape(-1, w.n_embd)
    n = hf.shape[0]
    pad_rows = g["wte"][50257:]
    np.testing.assert_allclose(pad_rows, np.broadcast_to(hf.sum(0) / (50304 * n), pad_rows.shape), atol=1e-15)


def test_masked_row_losses_hand_values():
    """Completion scores on a hand-checked case: row 0 selects positions 1 and 2 (losses 2, 3:
    sum 5, mean 2.5), row 1 selects nothing (0, 0), row 2 everything (sum 26, mean 6.5); the
    batch mean is over the 6 selected positions: 31 / 6."""
    losses = np.array([[1.0, 2.0, 3.0, 4.0], [5.0, 6.0, 7.0, 8.0], [5.0, 6.0, 7.0, 8.0]])
    mask = np.array([[0, 1, 1, 0], [0, 0, 0, 0], [1, 1, 1, 1]], dtype=np.uint8)
    row_sum, row_mean, total = O.masked_row_losses(losses, mask)
    assert row_sum.tolist() == [5.0, 0.0, 26.0]
    assert row_mean.tolist() == [2.5, 0.0, 6.5]
    assert total == 31.0 / 6.0
    assert int(np.argmin(row_mean[[0, 2]])) == 0
    _, row_mean, total = O.masked_row_losses(losses)
    assert row_mean.tolist() == [2.5, 6.5, 6.5] and total == losses.mean()
    assert O.masked_row_losses(losses, np.zeros_like(mask))[2] == 0.0


def test_eval_losses_zero_wte_and_no_mask():
    """wte = 0: every position's loss is ln 50304, so every non-empty row mean is exactly that
    and a row sum is its count times it; without a mask the batch mean is the forward's loss."""
    w = synthetic.workload("gpt2_step", n_layer=1, batch=2, seq_len=16)
    params = _f64(synthetic.init_params(w, randomize_affine=True))
    (x, y), = synthetic.micro_batches(w, 1)
    p0 = dict(params, wte=np.zeros_like(params["wte"]))
    out = O.forward(p0, w.n_layer, w.n_head, x, y, want_cache=False)
    mask = np.zeros((2, 16), dtype=np.uint8)
    mask[0, 3:9] = 1
    row_sum, row_mean, total = O.masked_row_losses(out["losses"], mask)
    assert abs(row_mean[0] - math.log(50304)) <= 1e-12 and row_mean[1] == 0.0
    assert abs(row_sum[0] - 6 * math.log(50304)) <= 1e-11 and abs(total - math.log(50304)) <= 1e-12
    out = O.forward(params, w.n_layer, w.n_head, x, y, want_cache=False)
    assert abs(O.masked_row_losses(out["losses"])[2] - out["loss"]) <= 1e-12 * out["loss"]


def test_eval_losses_equal_prefix_forwards():
    """Brute force: the loss at position t of a row equals the loss of a forward over that
    row's first t + 1 tokens alone, scored at its last position (only the prefix matters)."""
    w = _tiny()
    params = _f64(synthetic.init_params(w, randomize_affine=True))
    (x, y), = synthetic.micro_batches(w, 1)
    full = O.forward(params, w.n_layer, w.n_head, x, y, want_cache=False)["losses"]
    b = 2
    for t in range(0, x.shape[1], 7):
        one = O.forward(params, w.n_layer, w.n_head, x[b:b + 1, :t + 1], y[b:b + 1, :t + 1], want_cache=False)
        assert abs(one["losses"][0, t] - full[b, t]) <= 1e-12


def test_initial_loss_tiny_and_124m():
    for name, lo, hi in (("tiny", None, None), ("gpt2_step", None, None)):
        w = synthetic.workload(name, batch=1, seq_len=64) if name != "tiny" else _tiny()
        params = _f64(synthetic.init_params(w))
        (x, y), = synthetic.micro_batches(w, 1)
        out = O.forward(params, w.n_layer, w.n_head, x, y)
        z = out["logits"].reshape(-1, w.padded_vocab_size)
        row_var = z.var(axis=-1).mean()
        closed = math.log(w.padded_vocab_size) + row_var / 2
        assert abs(out["loss"] - closed) <= 0.05, (name, out["loss"], closed)
        assert abs(out["loss"] - math.log(w.vocab_size)) <= 0.5


def test_causality_bitwise():
    w = _tiny()
    params = _f64(synthetic.init_params(w, randomize_affine=True))
    (x, y), = synthetic.micro_batches(w, 1)
    base = O.forward(params, w.n_layer, w.n_head, x, y)["logits"]
    for t in (0, 17, 62):
        x2 = x.copy()
        x2[1, t + 1] = (x2[1, t + 1] + 1) % w.vocab_size
        other = O.forward(params, w.n_layer, w.n_head, x2, y)["logits"]
        assert np.array_equal(base[1, :t + 1], other[1, :t + 1])
        assert not np.array_equal(base[1, t + 1:], other[1, t + 1:])
        assert np.array_equal(base[0], other[0])


def test_accumulation_equals_big_batch():
    w = _tiny()
    params = _f64(synthetic.init_params(w, randomize_affine=True))
    (x, y), = synthetic.micro_batches(w, 1, batch=8)
    _, big = O.train_step(params, w.n_layer, w.n_head, [(x, y)])
    parts = [(x[2 * i:2 * i + 2], y[2 * i:2 * i + 2]) for i in range(4)]
    _, acc = O.train_step(params, w.n_layer, w.n_head, parts)
    for k in params:
        assert np.abs(acc[k] - big[k]).max() <= 1e-12 * max(np.abs(big[k]).max(), 1e-30), k


def test_adamw_first_step_closed_form():
    rng = np.random.default_rng(5)
    p0 = rng.standard_normal((4, 5))
    g = rng.standard_normal((4, 5))
    p = p0.copy()
    m = np.zeros_like(p)
    v = np.zeros_like(p)
    lr, wd, eps = 1e-3, 0.1, 1e-8
    O.adamw_update(p, g, m, v, 1, lr, 0.9, 0.95, eps, wd)
    np.testing.assert_allclose(m, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v, 0.05 * g * g, rtol=1e-14)
    np.testing.assert_allclose(p, p0 * (1 - lr * wd) - lr * g / (np.abs(g) + eps), rtol=0, atol=1e-15)


def test_gradient_identities():
    rng = np.random.default_rng(11)
    # LayerNorm: each row of dx sums to 0 and, at eps = 0 (where sum(xhat^2) = C exactly),
    # is orthogonal to xhat
    x = rng.standard_normal((5, 12))
    _, xhat, rstd = O.layernorm_forward(x, np.ones(12), np.zeros(12), eps=0.0)
    dx, _, _ = O.layernorm_backward(rng.standard_normal((5, 12)), xhat, rstd, np.ones(12))
    assert np.abs(dx.sum(-1)).max() < 1e-12
    assert np.abs((dx * xhat).sum(-1)).max() < 1e-12
    # softmax-CE: each row of softmax - onehot sums to 0
    z = rng.standard_normal((7, 30))
    yy = rng.integers(0, 30, 7)
    _, pr = O.cross_entropy_rows(z, yy)
    dz = pr.copy(); dz[np.arange(7), yy] -= 1
    assert np.abs(dz.sum(-1)).max() < 1e-14
    # attention: position 0 attends only to itself; dK sums to 0 over positions per head;
    # the key bias receives no gradient (softmax is shift invariant per query row)
    T, C, H = 9, 8, 2
    qkv = rng.standard_normal((T, 3 * C))
    y0 = O.attention_forward(qkv, H)
    np.testing.assert_array_equal(y0[0], qkv[0, 2 * C:])
    g = O.attention_backward(rng.standard_normal((T, C)), qkv, H)
    assert np.abs(g[:, C:2 * C].sum(0)).max() < 1e-12
    # GELU
    assert O.gelu_tanh(np.array(0.0)) == 0.0
    assert O.gelu_tanh_grad(np.array(0.0)) == 0.5


# ----------------------------------------------------------------- planted mistakes are caught
@pytest.mark.parametrize("mistake", ["ln_drop_mean", "gelu_sign", "attn_scale", "adam_eps_inside"])
def test_pins_catch_planted_mistakes(mistake, monkeypatch):
    """Plant a plausible mistake in the oracle and check that a pin above rejects it."""
    w = _mini()
    params = _f64(synthetic.init_params(w, randomize_affine=True))
    (x, y), = synthetic.micro_batches(w, 1)
    if mistake == "ln_drop_mean":
        def bad(dout, xhat, rstd, wv):
            dxhat = dout * wv
            dx = rstd * (dxhat - xhat * (dxhat * xhat).mean(-1, keepdims=True))
            r = dout.reshape(-1, dout.shape[-1])
            return dx, (r * xhat.reshape(r.shape)).sum(0), r.sum(0)
        monkeypatch.setattr(O, "layernorm_backward", bad)
    elif mistake == "gelu_sign":
        monkeypatch.setattr(O, "gelu_tanh_grad", lambda u: 0.5 * (1 + np.tanh(O.GELU_C * (u + O.GELU_A * u ** 3))))
    elif mistake == "attn_scale":
        def bad_probs(q, k):  # scores not divided by sqrt(head_dim)
            T = q.shape[-2]
            sc = np.matmul(q, k.transpose(0, 2, 1))
            sc = np.where(np.triu(np.ones((T, T), dtype=bool), k=1), -np.inf, sc)
            e = np.exp(sc - sc.max(-1, keepdims=True))
            return e / e.sum(-1, keepdims=True)
        monkeypatch.setattr(O, "causal_probs", bad_probs)
    elif mistake == "adam_eps_inside":
        def bad_adam(p, g, m, v, t, lr, b1, b2, eps, wd):
            p *= (1 - lr * wd)
            m *= b1; m += (1 - b1) * g
            v *= b2; v += (1 - b2) * g * g
            p -= lr * (m / (1 - b1 ** t)) / np.sqrt(v / (1 - b2 ** t) + eps)
        monkeypatch.setattr(O, "adamw_update", bad_adam)
    caught = False
    try:
        if mistake == "adam_eps_inside":
            test_adamw_first_step_closed_form()
        elif mistake == "attn_scale":
            t_logits = _torch_step(params, w, x, y, 6e-4)[0]
            out = O.forward(params, w.n_layer, w.n_head, x, y)
            np.testing.assert_allclose(out["logits"], t_logits, rtol=0, atol=1e-12)
        else:
            out = O.forward(params, w.n_layer, w.n_head, x, y)
            g = O.backward(params, w.n_layer, w.n_head, out["cache"], 1.0)
            k = "h.0.mlp.c_fc.weight"
            flat = params[k].reshape(-1)
            i = int(np.argmax(np.abs(g[k])))
            old = flat[i]
            flat[i] = old + 1e-6
            lp = O.forward(params, w.n_layer, w.n_head, x, y, want_logits=False, want_cache=False)["loss"]
            flat[i] = old - 1e-6
            lm = O.forward(params, w.n_layer, w.n_head, x, y, want_logits=False, want_cache=False)["loss"]
            flat[i] = old
            k2 = "h.0.ln_1.weight"
            j = int(np.argmax(np.abs(g[k2])))
            f2 = params[k2].reshape(-1)
            o2 = f2[j]
            f2[j] = o2 + 1e-6
            lp2 = O.forward(params, w.n_layer, w.n_head, x, y, want_logits=False, want_cache=False)["loss"]
            f2[j] = o2 - 1e-6
            lm2 = O.forward(params, w.n_layer, w.n_head, x, y, want_logits=False, want_cache=False)["loss"]
            f2[j] = o2
            ok1 = abs((lp - lm) / 2e-6 - g[k].reshape(-1)[i]) <= 1e-6 * np.abs(g[k]).max()
            ok2 = abs((lp2 - lm2) / 2e-6 - g[k2].reshape(-1)[j]) <= 1e-6 * np.abs(g[k2]).max()
            assert ok1 and ok2
    except AssertionError:
        caught = True
    assert caught, mistake


@pytest.mark.parametrize("mistake", ["count_all_positions", "mask_shifted"])
def test_eval_pins_catch_planted_mistakes(mistake, monkeypatch):
    """Plant a plausible mistake in the completion scores and check the hand-checked pin
    rejects it: dividing by every position instead of the selected ones, or a mask applied one
    position late (the shift between a token and the logits that predict it done twice)."""
    good = O.masked_row_losses

    def bad(losses, mask=None):
        if mask is None:
            return good(losses)
        if mistake == "mask_shifted":
            return good(losses, np.roll(np.asarray(mask), 1, axis=-1))
        row_sum, _, _ = good(losses, mask)
        return row_sum, row_sum / losses.shape[-1], row_sum.sum() / losses.size

    monkeypatch.setattr(O, "masked_row_losses", bad)
    with pytest.raises(AssertionError):
        test_masked_row_losses_hand_values()


# ----------------------------------------------------------------- sampling
def test_topk_sample_hand_values():
    """z = [1, 3, 3, 2, 0], k = 2: the kept tokens are 1 and 2 (equal, lower id first), each
    with probability 1/2; u < 1/2 draws token 1, u >= 1/2 token 2; k = 1 is the argmax for any
    u (the lowest id among equal maxima)."""
    z = np.array([1.0, 3.0, 3.0, 2.0, 0.0])
    tok, ids, kept = O.topk_sample(z, 2, 0.0)
    assert ids.tolist() == [1, 2] and tok == 1
    np.testing.assert_allclose(kept, [0.5, 0.5], rtol=0, atol=1e-15)
    assert O.topk_sample(z, 2, 0.4999)[0] == 1
    assert O.topk_sample(z, 2, 0.5)[0] == 2
    assert O.topk_sample(z, 2, 0.9999999)[0] == 2
    for u in (0.0, 0.3, 0.999):
        assert O.topk_sample(z, 1, u)[0] == 1
    # k = 3 keeps token 3 as well: probabilities e^3 : e^3 : e^2
    _, ids, kept = O.topk_sample(z, 3, 0.0)
    e = np.exp([3.0, 3.0, 2.0])
    assert ids.tolist() == [1, 2, 3]
    np.testing.assert_allclose(kept, e / e.sum(), rtol=1e-15)


def test_topk_sample_matches_softmax_topk_renormalized():
    """The kept probabilities are the k largest entries of the full softmax, renormalized, as
    the pages compute them (softmax over all columns, top-k, then a draw proportional to the
    kept probabilities); and over a fine grid of uniform numbers each kept token is drawn with
    its probability."""
    rng = np.random.default_rng(7)
    z = rng.standard_normal(300) * 2.0
    k = 50
    tok, ids, kept = O.topk_sample(z, k, 0.5)
    full = np.exp(z - z.max())
    full /= full.sum()
    top = np.sort(full)[::-1][:k]
    np.testing.assert_allclose(kept, top / top.sum(), rtol=1e-12)
    assert set(ids.tolist()) == set(np.argsort(-full)[:k].tolist())
    n = 100000
    counts = np.zeros(z.size)
    for u in (np.arange(n) + 0.5) / n:
        counts[O.topk_sample(z, k, u)[0]] += 1
    np.testing.assert_allclose(counts[ids] / n, kept, atol=2.0 / n)
    assert counts.sum() == counts[ids].sum()


@pytest.mark.parametrize("mistake", ["ties_by_higher_id", "no_renormalization"])
def test_sampling_pins_catch_planted_mistakes(mistake, monkeypatch):
    good = O.topk_sample

    def bad(logits, k, u):
        z = np.asarray(logits, dtype=np.float64)
        p = np.exp(z - z.max())
        p /= p.sum()
        if mistake == "ties_by_higher_id":
            order = np.lexsort((-np.arange(z.size), -p))
            ids = order[:k]
            kept = p[ids] / p[ids].sum()
        else:
            ids = np.lexsort((np.arange(z.size), -p))[:k]
            kept = p[ids]
        cdf = np.cumsum(kept)
        i = int(np.searchsorted(cdf, u, side="right"))
        return int(ids[min(i, k - 1)]), ids, kept

    monkeypatch.setattr(O, "topk_sample", bad)
    with pytest.raises(AssertionError):
        test_topk_sample_hand_values()
    monkeypatch.setattr(O, "topk_sample", good)

