"""Parity of the HIP path (through the C ABI) with the CPU oracle on the same seeded inputs.

Bars: fp32 check mode, per-tensor max|d|/max|ref| <= 1e-4 for logits, loss and gradients;
bf16 modes, |loss - ref| <= 2e-2 and per-tensor gradient cosine >= 0.999 (float64 metrics).
"bf16" is the autocast recipe (fp32 residual stream and gradient); "bf16_res16" also stores
the residual stream and its gradient in bf16.
The oracle runs in float64. Sizes span several tiles and ragged tails; the 124M, 1558M-shaped
and accumulation workloads run at their real widths, with fewer layers or sequences where the
oracle would otherwise take minutes (the kernels and launch shapes per layer are the same).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synthetic
from oracle import gpt2_oracle as O
from tests.gpu_common import config_for, cosine, f64, make_step, note, oracle_step, rel_max

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import transformer_lm_step_amd as G  # noqa: E402


def _grads_fp32_check(st, ref_grads, tol=1e-4):
    g = st.grads()
    worst = max((rel_max(g[k], ref_grads[k]), k) for k in ref_grads)
    assert worst[0] <= tol, worst
    return g


def _grads_cosine(st, ref_grads, bar=0.999):
    g = st.grads()
    for k in ref_grads:
        if k.endswith("attn.c_attn.bias"):
            C = ref_grads[k].shape[0] // 3
            # The key bias has zero gradient (softmax is shift invariant per query row), so
            # its cosine compares two noise vectors. Compare the query and value parts, and
            # bound the key part: in bf16 it is the sum over B*T positions of bf16-rounded
            # dK rows, each off by up to 2^-8 relative, which stays below 1e-2 of the
            # tensor's largest entry at these sizes.
            assert np.abs(g[k][C:2 * C]).max() <= 1e-2 * max(np.abs(g[k]).max(), 1e-30), k
            for sl in (slice(0, C), slice(2 * C, 3 * C)):
                assert cosine(g[k][sl], ref_grads[k][sl]) >= bar, k
            continue
        c = cosine(g[k], ref_grads[k])
        assert c >= bar, (k, c)
    return g


# ------------------------------------------------------------------ tiny, fp32 check mode
@pytest.mark.parametrize("randomize", [False, True])
def test_tiny_fp32_forward_backward(randomize):
    note(f"tiny fp32 randomize={randomize}")
    params, batches, ref_loss, ref_g, ref_logits = oracle_step("tiny", (), 4, 1, randomize, True)
    w = synthetic.workload("tiny")
    st = make_step(w, "fp32")
    st.set_params(params)
    x, y = batches[0]
    loss, logits = st.forward(x, y, want_logits=True)
    assert abs(loss - ref_loss) / abs(ref_loss) <= 1e-4, (loss, ref_loss)
    assert rel_max(logits.cpu().numpy(), ref_logits) <= 1e-4
    st.backward(1.0, False)
    _grads_fp32_check(st, ref_g)


@pytest.mark.parametrize("B,T", [(3, 50), (1, 1), (2, 8), (2, 64), (4, 17)])
def test_tiny_fp32_ragged(B, T):
    note(f"tiny fp32 ragged B={B} T={T}")
    w = synthetic.workload("tiny")
    params = synthetic.init_params(w, randomize_affine=True)
    rng = np.random.default_rng(100 + T)
    buf = synthetic.draw_tokens(rng, B * T + 1, w.vocab_size, w.tokens)
    x, y = buf[:-1].reshape(B, T), buf[1:].reshape(B, T)
    p64 = f64(params)
    out = O.forward(p64, w.n_layer, w.n_head, x, y)
    ref_g = O.backward(p64, w.n_layer, w.n_head, out["cache"], 0.5)
    st = make_step(w, "fp32")
    st.set_params(params)
    loss, logits = st.forward(x, y, want_logits=True)
    assert abs(loss - out["loss"]) / abs(out["loss"]) <= 1e-4
    assert rel_max(logits.cpu().numpy(), out["logits"]) <= 1e-4
    st.backward(0.5, False)
    _grads_fp32_check(st, ref_g)


def test_tiny_fp32_accumulate_flag():
    """accumulate=1 adds to the gradients already there; accumulate=0 overwrites them."""
    note("tiny fp32 accumulate flag")
    params, batches, _, _, _ = oracle_step("tiny", (), 4, 1, True, False)
    w = synthetic.workload("tiny")
    st = make_step(w, "fp32")
    st.set_params(params)
    x, y = batches[0]
    parts = [(x[i:i + 1], y[i:i + 1]) for i in range(4)]
    _, ref_g = O.train_step(f64(params), w.n_layer, w.n_head, parts)
    st.forward(*parts[3], want_loss=True)
    st.backward(1.0, False)      # garbage to be overwritten
    for i, (xi, yi) in enumerate(parts):
        st.forward(xi, yi)
        st.backward(0.25, i > 0)
    _grads_fp32_check(st, ref_g)


BF16_MODES = ["bf16", "bf16_res16"]


@pytest.mark.parametrize("mode", BF16_MODES)
def test_tiny_bf16_matches_oracle(mode):
    note(f"tiny {mode}")
    params, batches, ref_loss, ref_g, _ = oracle_step("tiny", (), 4, 1, True, False)
    w = synthetic.workload("tiny")
    st = make_step(w, mode)
    st.set_params(params)
    x, y = batches[0]
    loss, _ = st.forward(x, y)
    assert abs(loss - ref_loss) <= 2e-2
    st.backward(1.0, False)
    _grads_cosine(st, ref_g)


# ------------------------------------------------------------------ GPT-2 124M
def test_124m_forward_fp32_check_mode():
    """Forward logits and loss of the 124M model in fp32 check mode (one sequence of 1024)."""
    note("124M fp32 forward B=1")
    params, batches, ref_loss, _, ref_logits = oracle_step("gpt2_fwd", (), 1, 1, True, True)
    w = synthetic.workload("gpt2_fwd")
    st = make_step(w, "fp32", max_batch=1)
    st.set_params(params)
    x, y = batches[0]
    loss, logits = st.forward(x, y, want_logits=True)
    assert abs(loss - ref_loss) / abs(ref_loss) <= 1e-4, (loss, ref_loss)
    assert rel_max(logits.cpu().numpy(), ref_logits) <= 1e-4


def test_124m_forward_bf16_loss_b4():
    """The 124M forward at B=4 (4,096 rows: the N = 768 products take the few-row 128x64
    tiles): loss against the oracle, and the logits of the last sequence at every position
    (the oracle's forward of that sequence alone) by cosine."""
    note("124M bf16 forward B=4")
    w = synthetic.workload("gpt2_fwd")
    params = synthetic.init_params(w)
    (x, y), = synthetic.micro_batches(w, 1)
    p64 = f64(params)
    out = O.forward(p64, w.n_layer, w.n_head, x, y, want_logits=False, want_cache=False)
    st = make_step(w, "bf16")
    st.set_params(params)
    loss, logits = st.forward(x, y, want_logits=True)
    assert abs(loss - float(out["loss"])) <= 2e-2, (loss, out["loss"])
    b = x.shape[0] - 1
    ref = O.forward(p64, w.n_layer, w.n_head, x[b:b + 1], y[b:b + 1], want_cache=False)["logits"][0]
    lg = logits[b].float().cpu().numpy()
    for t in range(0, x.shape[1]):
        assert cosine(lg[t], ref[t]) >= 0.999, t


@pytest.mark.parametrize("mode", BF16_MODES)
def test_124m_step_bf16_gradients_b2(mode):
    note(f"124M {mode} step B=2")
    params, batches, ref_loss, ref_g, _ = oracle_step("gpt2_step", (), 2, 1, True, False)
    w = synthetic.workload("gpt2_step")
    st = make_step(w, mode, max_batch=2)
    st.set_params(params)
    loss, _ = st.forward(*batches[0])
    assert abs(loss - ref_loss) <= 2e-2
    st.backward(1.0, False)
    _grads_cosine(st, ref_g)


def test_accumulation_matches_big_batch_oracle():
    """Four micro-steps of B=1 with loss scale 1/4 against the oracle's single batch of B=4
    on the same rows (the accumulation workload, reduced B)."""
    note("124M bf16 accumulation 4 x B=1")
    w = synthetic.workload("gpt2_accum")
    params, batches, ref_loss, ref_g, _ = oracle_step("gpt2_accum", (), 4, 1, True, False)
    x, y = batches[0]
    st = make_step(w, "bf16", max_batch=1)
    st.set_params(params)
    acc_loss = 0.0
    for i in range(4):
        loss, _ = st.forward(x[i:i + 1], y[i:i + 1])
        acc_loss += loss / 4
        st.backward(0.25, i > 0)
    assert abs(acc_loss - ref_loss) <= 2e-2
    _grads_cosine(st, ref_g)


@pytest.mark.parametrize("T", [100, 37])
def test_ragged_context_two_layers_bf16(T):
    """124M widths (head size 64, the LDS-streamed attention kernels) with 2 layers and a
    context that is not a multiple of 64: the last query and key blocks have waves wholly past
    the sequence end, which run the masked computation and store nothing."""
    note(f"124M ragged T={T} L=2 bf16 B=2")
    ov = (("n_layer", 2), ("seq_len", T))
    params, batches, ref_loss, ref_g, _ = oracle_step("gpt2_step", ov, 2, 1, True, False)
    w = synthetic.workload("gpt2_step", **dict(ov))
    st = make_step(w, "bf16", max_batch=2)
    st.set_params(params)
    loss, _ = st.forward(*batches[0])
    assert abs(loss - ref_loss) <= 2e-2
    st.backward(1.0, False)
    _grads_cosine(st, ref_g)


def test_sharp_attention_bf16():
    """124M widths, 2 layers, one sequence of 1024, with the query and key rows of c_attn scaled
    by 3.5 (scores about 12x wider): the running maximum of a wave's queries then grows by more
    than 2^8 after the first key chunk in several hundred of layer 0's 6,528 wave-chunks, which
    runs the forward's lazy rescale with the shift of the chunk's scores, and the backward's
    log-sum-exp offsets are larger. (Much sharper attention leaves the bf16 bar: at a factor 6
    the gradient cosines fall to about 0.99 with or without the scale folded into the queries.)"""
    note("124M sharp attention L=2 bf16 B=1")
    w = synthetic.workload("gpt2_step", n_layer=2)
    params = synthetic.init_params(w, randomize_affine=True)
    C = w.n_embd
    for l in range(w.n_layer):
        k = f"h.{l}.attn.c_attn.weight"
        params[k] = params[k].copy()
        params[k][:2 * C] *= 3.5
    x, y = synthetic.micro_batches(w, 1, batch=1)[0]
    p64 = f64(params)
    out = O.forward(p64, w.n_layer, w.n_head, x, y)
    ref_g = O.backward(p64, w.n_layer, w.n_head, out["cache"], 1.0)
    st = make_step(w, "bf16", max_batch=1)
    st.set_params(params)
    loss, _ = st.forward(x, y)
    assert abs(loss - float(out["loss"])) <= 2e-2
    st.backward(1.0, False)
    _grads_cosine(st, ref_g)


@pytest.mark.parametrize("mode", BF16_MODES)
def test_xl_shape_two_layers_bf16(mode):
    """1558M widths (C=1600, 25 heads, MLP 6400) with 2 layers, one sequence of 1024."""
    note(f"xl-shape L=2 {mode} B=1")
    params, batches, ref_loss, ref_g, _ = oracle_step("gpt2_xl", (("n_layer", 2),), 1, 1, True, False)
    w = synthetic.workload("gpt2_xl", n_layer=2)
    st = make_step(w, mode, max_batch=1)
    st.set_params(params)
    loss, _ = st.forward(*batches[0])
    assert abs(loss - ref_loss) <= 2e-2
    st.backward(1.0, False)
    _grads_cosine(st, ref_g)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", BF16_MODES)
def test_step_b16_two_layers_full_gradients(mode):
    """The benchmark's launch shapes against the oracle: B=16, T=1024 (16,384 rows) at the
    124M widths with 2 layers. At this row count every N=768 product (the projections'
    forwards, every input-gradient product with N=768, the lm_head input gradient) and the
    vocabulary product take 128x192 tiles, as in the timed step. Loss and every gradient."""
    note(f"124M {mode} B=16 L=2 full gradients")
    ov = (("n_layer", 2),)
    params, batches, ref_loss, ref_g, _ = oracle_step("gpt2_step", ov, 16, 1, True, False)
    w = synthetic.workload("gpt2_step", n_layer=2)
    st = make_step(w, mode)
    st.set_params(params)
    loss, _ = st.forward(*batches[0])
    assert abs(loss - ref_loss) <= 2e-2, (loss, ref_loss)
    st.backward(1.0, False)
    _grads_cosine(st, ref_g)
    st.close()


def test_class_timing_same_results():
    """Per-class timing switched on: every product that is one kernel then launches through
    hipExtLaunchKernel with its class's event pair (the live roofline figure of the benchmark).
    The loss and every gradient must be the same bit for bit as with timing off, and every
    class the step runs must report its launches and a positive time."""
    note("124M bf16 B=16 L=2 class timing")
    w = synthetic.workload("gpt2_step", n_layer=2)
    params = synthetic.init_params(w, randomize_affine=True)
    x, y = synthetic.micro_batches(w, 1, batch=16)[0]
    st = make_step(w, "bf16")
    st.set_params(params)
    loss0, _ = st.forward(x, y)
    st.backward(1.0, False)
    g0 = st.grads()
    G.gpt2_timing_begin(st.h)
    loss1, _ = st.forward(x, y)
    st.backward(1.0, False)
    G.gpt2_timing_end(st.h)
    g1 = st.grads()
    assert loss1 == loss0
    for k in g0:
        assert np.array_equal(g0[k], g1[k]), k
    L = w.n_layer
    expect = {"gemm_qkv": L, "gemm_attn_proj": L, "gemm_fc": L, "gemm_mlp_proj": L, "gemm_lm_head": 1,
              "gemm_lm_head_dx": 1, "gemm_lm_head_dw": 1, "gemm_dx": 4 * L, "gemm_dw": 1, "attn_fwd": L,
              "attn_bwd": L, "cross_entropy": 1, "layernorm_bwd": 2 * L + 1}
    for cls, n in expect.items():
        ms, launches = G.gpt2_timing_get(st.h, cls)
        assert launches == n and ms > 0.0, (cls, launches, ms)
    st.close()


@pytest.mark.parametrize("mode,T", [("fp32", 2048), ("bf16_res16", 2048), ("fp32", 1900)])
def test_embedding_backward_chunked(mode, T):
    """More rows than one sort chunk of the embedding backward (9 sequences of T tokens:
    more than 16,384 rows, so the ids are sorted in two chunks and the second chunk's sums add
    onto the first's): tiny widths with block_size T, every gradient against the oracle
    (fp32 check mode 1e-4; the bf16 residual-gradient mode by cosine)."""
    note(f"chunked embedding backward {mode} B=9 T={T}")
    w = synthetic.workload("tiny", block_size=T, seq_len=T, batch=9)
    params = synthetic.init_params(w, randomize_affine=True)
    (x, y), = synthetic.micro_batches(w, 1)
    p64 = f64(params)
    out = O.forward(p64, w.n_layer, w.n_head, x, y, want_logits=False)
    ref_g = O.backward(p64, w.n_layer, w.n_head, out["cache"], 1.0)
    st = make_step(w, mode)
    st.set_params(params)
    loss, _ = st.forward(x, y)
    st.backward(1.0, False)
    if mode == "fp32":
        assert abs(loss - out["loss"]) <= 1e-4 * abs(out["loss"])
        _grads_fp32_check(st, ref_g)
    else:
        assert abs(loss - out["loss"]) <= 2e-2
        _grads_cosine(st, ref_g)


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
@pytest.mark.parametrize("C,H", [(1280, 20), (1408, 22)])
def test_wide_rows(C, H, mode):
    """Widths whose LayerNorm rows take 5 and 6 float4 per lane (C = 1280, the GPT-2 large
    width, and C = 1408): one layer, B=2, T=64, loss and every gradient against the oracle
    (fp32 check mode at 1e-4; bf16 at the bf16 bars), 64-wide heads, a 256-token vocabulary."""
    note(f"wide rows {mode} C={C}")
    w = synthetic.workload("tiny", n_layer=1, n_head=H, n_embd=C, batch=2)
    params = synthetic.init_params(w, randomize_affine=True)
    (x, y), = synthetic.micro_batches(w, 1)
    p64 = f64(params)
    out = O.forward(p64, w.n_layer, w.n_head, x, y, want_logits=False)
    ref_g = O.backward(p64, w.n_layer, w.n_head, out["cache"], 1.0)
    st = make_step(w, mode)
    st.set_params(params)
    loss, _ = st.forward(x, y)
    st.backward(1.0, False)
    if mode == "fp32":
        assert abs(loss - out["loss"]) <= 1e-4 * abs(out["loss"])
        _grads_fp32_check(st, ref_g)
    else:
        assert abs(loss - out["loss"]) <= 2e-2
        _grads_cosine(st, ref_g)


def test_layernorm_backward_partials_sized_for_every_batch():
    """The LayerNorm backward takes 2 rows per wave for batches of at most 8192 rows and 4
    above, so a smaller batch can need more blocks (and partial-sum slots) than the largest
    one: a handle with room for 130 sequences of 64 tokens (8320 rows) runs 128 of them (8192
    rows, twice the blocks); every gradient against the oracle (fp32 check mode, 1e-4)."""
    note("LayerNorm backward partial sets, max batch 130, B=128 T=64 fp32")
    w = synthetic.workload("tiny", batch=128)
    params = synthetic.init_params(w, randomize_affine=True)
    (x, y), = synthetic.micro_batches(w, 1)
    assert x.shape == (128, 64)
    p64 = f64(params)
    out = O.forward(p64, w.n_layer, w.n_head, x, y, want_logits=False)
    ref_g = O.backward(p64, w.n_layer, w.n_head, out["cache"], 1.0)
    st = make_step(w, "fp32", max_batch=130)
    st.set_params(params)
    loss, _ = st.forward(x, y)
    st.backward(1.0, False)
    assert abs(loss - out["loss"]) <= 1e-4 * abs(out["loss"])
    _grads_fp32_check(st, ref_g)


# ------------------------------------------------------------------ full-size invariants
def test_full_step_b16_invariants():
    """The timed workload itself (B=16, T=1024, bf16): per-sequence logits against the oracle
    for a sampled sequence, initial-loss closed form, bitwise determinism, bitwise causality."""
    note("124M bf16 full B=16")
    w = synthetic.workload("gpt2_step")
    params = synthetic.init_params(w)
    (x, y), = synthetic.micro_batches(w, 1)
    st = make_step(w, "bf16")
    st.set_params(params)
    loss, logits = st.forward(x, y, want_logits=True)
    assert math.isfinite(loss)
    b = 5
    ref = O.forward(f64(params), w.n_layer, w.n_head, x[b:b + 1], y[b:b + 1], want_cache=False)
    lg = logits[b].cpu().numpy()
    worst = min(cosine(lg[t], ref["logits"][0, t]) for t in range(w.seq_len))
    assert worst >= 0.999, worst
    z = ref["logits"][0]
    closed = math.log(w.padded_vocab_size) + z.var(axis=-1).mean() / 2
    assert abs(loss - closed) <= 0.05
    st.backward(1.0, False)
    g1 = torch.empty(st.n_params, dtype=torch.float32, device="cuda")
    G.gpt2_get_grads(st.h, g1.data_ptr(), 1)
    st.forward(x, y)
    st.backward(1.0, False)
    g2 = torch.empty_like(g1)
    G.gpt2_get_grads(st.h, g2.data_ptr(), 1)
    assert torch.equal(g1, g2), "backward is not bitwise deterministic"
    x2 = x.copy()
    t = 600
    x2[b, t + 1] = (x2[b, t + 1] + 7) % w.vocab_size
    _, logits2 = st.forward(x2, y, want_logits=True, want_loss=False)
    assert torch.equal(logits[b, :t + 1], logits2[b, :t + 1])
    assert not torch.equal(logits[b, t + 1:], logits2[b, t + 1:])
    assert torch.equal(logits[:b], logits2[:b])


def test_ctx2048_two_layers_bf16():
    """GPT-3's context (block_size = T = 2048) at the 124M widths, 2 layers, one sequence:
    loss and every gradient against the oracle."""
    note("ctx2048 L=2 bf16 B=1")
    params, batches, ref_loss, ref_g, _ = oracle_step("gpt2_ctx2048", (("n_layer", 2),), 1, 1, True, False)
    w = synthetic.workload("gpt2_ctx2048", n_layer=2)
    st = make_step(w, "bf16", max_batch=1)
    st.set_params(params)
    loss, _ = st.forward(*batches[0])
    assert abs(loss - ref_loss) <= 2e-2
    st.backward(1.0, False)
    _grads_cosine(st, ref_g)


def test_full_ctx2048_b32_invariants():
    """The 2048-context micro-step at its real size (B=32, T=2048: 65,536 rows, so the logits
    hold more than 2^31 elements): a sampled sequence's logits against the oracle, the
    initial-loss closed form, bitwise determinism of backward, bitwise causality at t=1500."""
    note("124M bf16 ctx2048 full B=32")
    w = synthetic.workload("gpt2_ctx2048")
    params = synthetic.init_params(w)
    (x, y), = synthetic.micro_batches(w, 1)
    st = make_step(w, "bf16")
    st.set_params(params)
    loss, logits = st.forward(x, y, want_logits=True)
    assert math.isfinite(loss)
    b = 29
    ref = O.forward(f64(params), w.n_layer, w.n_head, x[b:b + 1], y[b:b + 1], want_cache=False)
    assert cosine(logits[b].cpu().numpy(), ref["logits"][0]) >= 0.999
    z = ref["logits"][0]
    closed = math.log(w.padded_vocab_size) + z.var(axis=-1).mean() / 2
    assert abs(loss - closed) <= 0.05
    st.backward(1.0, False)
    g1 = torch.empty(st.n_params, dtype=torch.float32, device="cuda")
    G.gpt2_get_grads(st.h, g1.data_ptr(), 1)
    assert torch.isfinite(g1).all()
    st.forward(x, y)
    st.backward(1.0, False)
    g2 = torch.empty_like(g1)
    G.gpt2_get_grads(st.h, g2.data_ptr(), 1)
    assert torch.equal(g1, g2), "backward is not bitwise deterministic"
    del g1, g2
    x2 = x.copy()
    t = 1500
    x2[b, t + 1] = (x2[b, t + 1] + 7) % w.vocab_size
    lb = logits[b].clone()
    lrest = logits[b + 1:].clone()
    del logits
    _, logits2 = st.forward(x2, y, want_logits=True, want_loss=False)
    assert torch.equal(lb[:t + 1], logits2[b, :t + 1])
    assert not torch.equal(lb[t + 1:], logits2[b, t + 1:])
    assert torch.equal(lrest, logits2[b + 1:])


@pytest.mark.timeout(900)
def test_xl_full_size_invariants():
    """The 1558M-shaped micro-step at its real size (48 layers, 25 heads, C=1600, B=4,
    T=1024, bf16): every position of a sampled sequence's logits against the oracle, that
    sequence's mean loss against the oracle's, the batch loss within 0.5 of ln(V), bitwise
    determinism of the backward, bitwise causality.

    The Gaussian-logit closed form ln(Vp) + var(z)/2 that the 124M tests use is not a gate
    here: it assumes each target's logit has mean zero, but with Zipf-distributed tokens the
    48 layers carry a component along the embeddings of frequent tokens (which are also
    frequent targets), so the target logit has a positive mean (+0.16 on the sampled sequence in the
    oracle, whose log-sum-exp does follow the closed form) and the loss sits 0.1-0.2 below it."""
    note("xl bf16 full L=48 B=4")
    w = synthetic.workload("gpt2_xl")
    params = synthetic.init_params(w)
    (x, y), = synthetic.micro_batches(w, 1)
    st = make_step(w, "bf16")
    st.set_params(params)
    loss, logits = st.forward(x, y, want_logits=True)
    assert math.isfinite(loss)
    b = 2
    note("xl oracle forward of one sequence")
    ref = O.forward(f64(params), w.n_layer, w.n_head, x[b:b + 1], y[b:b + 1], want_cache=False)
    del params
    lg = logits[b].cpu().numpy()
    z = ref["logits"][0]
    worst = min(cosine(lg[t], z[t]) for t in range(w.seq_len))
    assert worst >= 0.999, worst
    assert abs(loss - math.log(w.vocab_size)) <= 0.5, loss
    _, row_mean, tot = st.evaluate(x, y)
    assert tot == loss
    assert abs(row_mean[b] - float(ref["loss"])) <= 2e-2, (row_mean[b], ref["loss"])
    note("xl backward determinism")
    st.forward(x, y)
    st.backward(1.0, False)
    g1 = torch.empty(st.n_params, dtype=torch.float32, device="cuda")
    G.gpt2_get_grads(st.h, g1.data_ptr(), 1)
    assert torch.isfinite(g1).all()
    st.forward(x, y)
    st.backward(1.0, False)
    g2 = torch.empty_like(g1)
    G.gpt2_get_grads(st.h, g2.data_ptr(), 1)
    assert torch.equal(g1, g2), "backward is not bitwise deterministic"
    del g1, g2
    note("xl causality")
    x2 = x.copy()
    t = 700
    x2[b, t + 1] = (x2[b, t + 1] + 7) % w.vocab_size
    _, logits2 = st.forward(x2, y, want_logits=True, want_loss=False)
    assert torch.equal(logits[b, :t + 1], logits2[b, :t + 1])
    assert not torch.equal(logits[b, t + 1:], logits2[b, t + 1:])
    assert torch.equal(logits[:b], logits2[:b])
    del logits, logits2
    st.close()


def _state(st):
    p = torch.empty(st.n_params, dtype=torch.float32, device="cuda")
    m, v = torch.empty_like(p), torch.empty_like(p)
    G.gpt2_get_params(st.h, p.data_ptr(), 1)
    G.gpt2_get_moments(st.h, m.data_ptr(), v.data_ptr(), 1)
    torch.cuda.synchronize()
    return p, m, v


def test_checkpoint_resume_bitwise(tmp_path):
    """Full-state checkpoint and resume: 4 optimizer steps of 2 micro-steps each without a
    break, against 2 steps, a saved state, the handle destroyed, a fresh handle with another
    device initialization, the state loaded and the last 2 steps: parameters and both AdamW
    moments bitwise equal. Restoring the parameters without the moments must not match (the
    check has teeth), and a state does not load into a handle of another model shape."""
    from transformer_lm_step_amd import checkpoint as ck
    note("checkpoint resume 124M widths L=4 B=2")
    w = synthetic.workload("gpt2_step", n_layer=4, batch=2)
    params = synthetic.init_params(w, randomize_affine=True)
    batches = synthetic.micro_batches(w, 8)

    def run(st, s0, s1, pos):
        for s in range(s0, s1):
            for i in range(2):
                x, y = batches[pos]
                pos += 1
                st.forward(x, y)
                st.backward(0.5, i > 0)
            st.adamw_step(G.gpt2_cosine_lr(s, 6e-4, 6e-5, 2, 10), t=s + 1)
        return pos

    a = make_step(w, "bf16")
    a.set_params(params)
    run(a, 0, 4, 0)
    pa, ma, va = _state(a)
    a.close()

    b = make_step(w, "bf16")
    b.set_params(params)
    pos = run(b, 0, 2, 0)
    p2, _, _ = _state(b)
    path = str(tmp_path / "state.npz")
    ck.save(b, path, adam_t=2, data_pos=pos, extra={"note": "after 2 steps"})
    b.close()
    del b

    c = make_step(w, "bf16", seed=77)
    got = ck.load(c, path)
    assert got == {"adam_t": 2, "data_pos": 4, "extra": {"note": "after 2 steps"}}
    run(c, got["adam_t"], 4, got["data_pos"])
    pc, mc, vc = _state(c)
    assert not torch.equal(pc, p2), "the last two steps changed nothing"
    assert torch.equal(pa, pc) and torch.equal(ma, mc) and torch.equal(va, vc)
    c.close()

    d = make_step(w, "bf16", seed=78)
    d.set_params(d.unpack(ck.read_state(path)["params"]))
    run(d, 2, 4, 4)
    pd, _, _ = _state(d)
    assert not torch.equal(pa, pd), "moments made no difference to the resumed steps"
    d.close()

    e = make_step(synthetic.workload("tiny"), "fp32")
    with pytest.raises(ValueError):
        ck.load(e, path)
    e.close()


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_checkpoint_resume_matches_oracle_adamw(tmp_path, mode):
    """The oracle's leg of a resume: a state saved after two optimizer steps is read back with
    allow_pickle=False into the oracle's tensors; both sides take the same gradients (set into
    the resumed handle) and one more step at t = saved t + 1 from the restored params, m and v.
    Parameters, both moments and the norm agree at the AdamW bar, so a convention that save
    and load share (the step count, the order of the moments, the decayed prefix) cannot hide."""
    from transformer_lm_step_amd import checkpoint as ck
    note(f"checkpoint resume vs oracle AdamW {mode}")
    w = synthetic.workload("tiny")
    params = synthetic.init_params(w, randomize_affine=True)
    batches = synthetic.micro_batches(w, 2)
    a = make_step(w, mode)
    a.set_params(params)
    for s_ in range(2):
        a.forward(*batches[s_])
        a.backward(1.0, False)
        a.adamw_step(1e-3 * (s_ + 1), t=s_ + 1)
    path = str(tmp_path / "state.npz")
    ck.save(a, path, adam_t=2, data_pos=2)
    a.close()

    b = make_step(w, mode, seed=5)
    got = ck.load(b, path)
    assert got["adam_t"] == 2
    rng = np.random.default_rng(17)
    grads = {k: (rng.standard_normal(v.shape) * 0.5).astype(np.float32) for k, v in params.items()}
    gt = torch.from_numpy(b.pack(grads)).cuda()
    G.gpt2_set_grads(b.h, gt.data_ptr(), 1)
    t = got["adam_t"] + 1
    lr = 2.5e-3
    norm = b.adamw_step(lr, t=t)

    state = ck.read_state(path)
    p = f64(b.unpack(state["params"]))
    m = f64(b.unpack(state["m"]))
    v = f64(b.unpack(state["v"]))
    assert any(np.abs(m[k]).max() > 0 for k in m), "saved moments are empty"
    ref_norm = O.optimizer_step(p, f64(grads), m, v, t, lr)
    assert norm == pytest.approx(ref_norm, rel=1e-5)
    gp = b.params()
    mm = torch.empty(b.n_params, dtype=torch.float32, device="cuda")
    vv = torch.empty_like(mm)
    G.gpt2_get_moments(b.h, mm.data_ptr(), vv.data_ptr(), 1)
    gm, gv = b.unpack(mm.cpu().numpy()), b.unpack(vv.cpu().numpy())
    for k in p:
        assert np.abs(gp[k] - p[k]).max() <= 1e-6 * max(np.abs(p[k]).max(), 1e-3), k
        assert rel_max(gm[k], m[k]) <= 1e-5 and rel_max(gv[k], v[k]) <= 1e-5, k
    b.close()


def test_hip_graph_replay_matches_eager():
    """A forward + backward captured in a HIP graph (the library's launches recorded on the
    capture stream) and replayed three times, with eager work on other inputs and
    synchronizations between the replays: every replay's loss and gradients equal the eager
    pass on the captured inputs bit for bit. The step enqueues kernels and device-to-device
    copies only (no memset)."""
    note("hip graph replay")
    w = synthetic.workload("gpt2_step", n_layer=2, batch=2, seq_len=256, block_size=256)
    params = synthetic.init_params(w, randomize_affine=True)
    st = make_step(w, "bf16")
    st.set_params(params)
    (x, y), (x2, y2) = synthetic.micro_batches(w, 2)
    B, T = x.shape
    xd, yd = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
    xd2, yd2 = torch.from_numpy(x2).cuda(), torch.from_numpy(y2).cuda()
    d_loss = torch.zeros(1, dtype=torch.float32, device="cuda")

    def fb(a, b):
        G.gpt2_forward(st.h, a.data_ptr(), b.data_ptr(), B, T, None, d_loss.data_ptr())
        G.gpt2_backward(st.h, 1.0, 0)

    def grads():
        g = torch.empty(st.n_params, dtype=torch.float32, device="cuda")
        G.gpt2_get_grads(st.h, g.data_ptr(), 1)
        torch.cuda.synchronize()
        return g

    fb(xd, yd)
    torch.cuda.synchronize()
    ref_loss, ref_g = d_loss.clone(), grads()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        G.gpt2_set_stream(st.h, torch.cuda.current_stream().cuda_stream)
        fb(xd, yd)
    G.gpt2_set_stream(st.h, st.stream)
    for rep in range(3):
        fb(xd2, yd2)                      # eager work in between, on other inputs
        torch.cuda.synchronize()
        assert not torch.equal(d_loss, ref_loss)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(d_loss, ref_loss), rep
        assert torch.equal(grads(), ref_g), rep
    del graph
    st.close()


def test_hip_graph_evaluate_replay_matches_eager():
    """A forward-only scoring pass (gpt2_evaluate: the same forward, per-position losses and the
    per-sequence reduction) captured in a HIP graph and replayed three times, with eager passes
    on other inputs and synchronizations between the replays: every replay's mean loss and
    per-sequence sums equal the eager pass on the captured inputs bit for bit."""
    note("hip graph replay of gpt2_evaluate")
    w = synthetic.workload("gpt2_step", n_layer=2, batch=4, seq_len=256, block_size=256)
    params = synthetic.init_params(w, randomize_affine=True)
    st = make_step(w, "bf16")
    st.set_params(params)
    (x, y), (x2, y2) = synthetic.micro_batches(w, 2)
    B, T = x.shape
    xd, yd = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
    xd2, yd2 = torch.from_numpy(x2).cuda(), torch.from_numpy(y2).cuda()
    d_loss = torch.zeros(1, dtype=torch.float32, device="cuda")
    d_sum = torch.zeros(B, dtype=torch.float32, device="cuda")

    def ev(a, b):
        G.gpt2_evaluate(st.h, a.data_ptr(), b.data_ptr(), None, B, T, d_sum.data_ptr(), None, d_loss.data_ptr())

    ev(xd, yd)
    torch.cuda.synchronize()
    ref_loss, ref_sum = d_loss.clone(), d_sum.clone()
    graph = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        G.gpt2_set_stream(st.h, torch.cuda.current_stream().cuda_stream)
        ev(xd, yd)
    G.gpt2_set_stream(st.h, st.stream)
    for rep in range(3):
        ev(xd2, yd2)                      # eager work in between, on other inputs
        torch.cuda.synchronize()
        assert not torch.equal(d_loss, ref_loss)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(d_loss, ref_loss), rep
        assert torch.equal(d_sum, ref_sum), rep
    del graph
    st.close()


def test_evaluate_tiny_fp32_matches_oracle():
    """Forward-only scores in fp32 check mode: per-row sums and means over a ragged mask (one
    row selects nothing, one row everything) and the masked batch mean against the oracle
    (1e-4 relative); without a mask the batch mean is bitwise the loss gpt2_forward reports."""
    note("evaluate tiny fp32")
    w = synthetic.workload("tiny")
    params = synthetic.init_params(w, randomize_affine=True)
    (x, y), = synthetic.micro_batches(w, 1)
    B, T = x.shape
    mask = (np.random.default_rng(11).random((B, T)) < 0.3).astype(np.uint8)
    mask[1] = 0
    mask[2] = 1
    ref = O.forward(f64(params), w.n_layer, w.n_head, x, y, want_cache=False)
    r_sum, r_mean, r_tot = O.masked_row_losses(ref["losses"], mask)
    st = make_step(w, "fp32")
    st.set_params(params)
    s, m, tot = st.evaluate(x, y, mask)
    assert rel_max(s, r_sum) <= 1e-4 and rel_max(m, r_mean) <= 1e-4
    assert s[1] == 0.0 and m[1] == 0.0
    assert abs(tot - r_tot) <= 1e-4 * abs(r_tot)
    _, _, tot_all = st.evaluate(x, y)
    loss, _ = st.forward(x, y)
    assert tot_all == loss


def test_evaluate_completion_rows_bf16():
    """Completion-style scoring at the 124M widths (2 layers, bf16): four rows share a 60-token
    context and end in 5 to 20 different tokens, zero-padded to T = 96, the mask on the
    positions whose targets are the ending's tokens. Row means against the oracle within the
    bf16 loss bar, and the same lowest row wherever the oracle's margin exceeds twice that bar.
    Gradients are untouched and a backward after the call is refused."""
    note("evaluate completion rows bf16")
    w = synthetic.workload("gpt2_step", n_layer=2, batch=4, seq_len=96)
    params = synthetic.init_params(w, randomize_affine=True)
    rng = np.random.default_rng(5)
    ctx = rng.integers(0, w.vocab_size, 60)
    rows = np.zeros((4, 97), dtype=np.int64)
    mask = np.zeros((4, 96), dtype=np.uint8)
    for r, n_end in enumerate((5, 12, 20, 9)):
        toks = np.concatenate([ctx, rng.integers(0, w.vocab_size, n_end)])
        rows[r, :toks.size] = toks
        mask[r, ctx.size - 1:toks.size - 1] = 1
    x, y = rows[:, :96].astype(np.int32), rows[:, 1:].astype(np.int32)
    ref = O.forward(f64(params), w.n_layer, w.n_head, x, y, want_cache=False)
    _, r_mean, r_tot = O.masked_row_losses(ref["losses"], mask)
    st = make_step(w, "bf16")
    st.set_params(params)
    st.forward(x, y)
    st.backward(1.0, False)
    g0 = torch.empty(st.n_params, dtype=torch.float32, device="cuda")
    G.gpt2_get_grads(st.h, g0.data_ptr(), 1)
    _, m, tot = st.evaluate(x, y, mask)
    assert np.abs(m - r_mean).max() <= 2e-2, (m, r_mean)
    assert abs(tot - r_tot) <= 2e-2
    order = np.sort(r_mean)
    if order[1] - order[0] > 4e-2:
        assert int(np.argmin(m)) == int(np.argmin(r_mean))
    g1 = torch.empty_like(g0)
    G.gpt2_get_grads(st.h, g1.data_ptr(), 1)
    assert torch.equal(g0, g1)
    with pytest.raises(G.GPT2Error):
        st.backward(1.0, False)


def test_evaluate_full_b16():
    """Forward-only scoring at the benchmarked size (B=16, T=1024, bf16), half the positions
    masked at random: a sampled sequence's masked mean against the oracle; without a mask the
    batch mean is bitwise the loss of the training forward."""
    note("evaluate 124M bf16 full B=16")
    w = synthetic.workload("gpt2_step")
    params = synthetic.init_params(w)
    (x, y), = synthetic.micro_batches(w, 1)
    mask = (np.random.default_rng(3).random(x.shape) < 0.5).astype(np.uint8)
    st = make_step(w, "bf16")
    st.set_params(params)
    s, m, _ = st.evaluate(x, y, mask)
    b = 11
    ref = O.forward(f64(params), w.n_layer, w.n_head, x[b:b + 1], y[b:b + 1], want_cache=False)
    _, r_mean, _ = O.masked_row_losses(ref["losses"], mask[b:b + 1])
    assert abs(m[b] - r_mean[0]) <= 2e-2
    assert np.all(np.isfinite(s)) and np.all(s > 0)
    _, _, tot_all = st.evaluate(x, y)
    loss, _ = st.forward(x, y)
    assert tot_all == loss


def _decode(st, params, w, prompt, total, k, rng, check_logits):
    """Feed the prompt [B, P] one token per step, then draw until `total` tokens. At every
    step: check_logits(step logits [B, Vp] host, oracle-free), and the sampler against the
    oracle's on the step's own logits (ids exact, probabilities 1e-5, the drawn token wherever
    u is more than 1e-5 from a cumulative boundary). Returns the final tokens [B, total]."""
    B, P = prompt.shape
    seq = np.zeros((B, total), dtype=np.int64)
    seq[:, :P] = prompt
    st.decode_reset(B)
    assert G.gpt2_decode_position(st.h) == 0
    for t in range(total - 1):
        u = rng.random(B).astype(np.float32)
        logits, nxt, ids, probs = st.decode_step(seq[:, t].astype(np.int32), uniform=u, top_k=k)
        lg = logits.cpu().numpy()
        check_logits(t, seq[:, :t + 1], lg)
        nxt, ids, probs = nxt.cpu().numpy(), ids.cpu().numpy(), probs.cpu().numpy()
        for b in range(B):
            tok, rids, rkept = O.topk_sample(lg[b], k, float(u[b]))
            assert np.array_equal(ids[b], rids), (t, b)
            np.testing.assert_allclose(probs[b], rkept, rtol=0, atol=1e-5)
            if np.abs(np.cumsum(rkept) - u[b]).min() > 1e-5:
                assert nxt[b] == tok, (t, b)
        if t + 1 >= P:
            seq[:, t + 1] = nxt
    assert G.gpt2_decode_position(st.h) == total - 1
    return seq


@pytest.mark.parametrize("mode", BF16_MODES)
def test_few_rows_bf16_forward(mode):
    """A forward of only 16 rows (B=2, T=8) at the 124M widths with 2 layers, bf16: the
    products take the few-row path (every forward epilogue: bias, residual, GELU, and the
    50304-column lm_head); logits (cosine >= 0.999) and loss (bf16 bar) against the oracle."""
    note(f"few rows {mode} B=2 T=8")
    w = synthetic.workload("gpt2_step", n_layer=2, batch=2, seq_len=8)
    params = synthetic.init_params(w, randomize_affine=True)
    (x, y), = synthetic.micro_batches(w, 1)
    ref = O.forward(f64(params), w.n_layer, w.n_head, x, y, want_cache=False)
    st = make_step(w, mode)
    st.set_params(params)
    loss, logits = st.forward(x, y, want_logits=True)
    assert abs(loss - ref["loss"]) <= 2e-2
    lg = logits.cpu().numpy()
    for b in range(2):
        for t in range(8):
            assert cosine(lg[b, t], ref["logits"][b, t]) >= 0.999, (b, t)


def test_decode_tiny_fp32_matches_oracle():
    """Key/value-cache decoding in fp32 check mode, 3 sequences, a 6-token prompt continued to
    the full block of 64 positions with top-50 sampling: every step's logits against the
    oracle's forward over the whole prefix (1e-4 relative), and the sampler as in _decode."""
    note("decode tiny fp32")
    w = synthetic.workload("tiny")
    params = synthetic.init_params(w, randomize_affine=True)
    p64 = f64(params)
    st = make_step(w, "fp32", max_batch=3)
    st.set_params(params)
    rng = np.random.default_rng(21)
    prompt = rng.integers(0, w.vocab_size, (3, 6))

    def check(t, prefix, lg):
        ref = O.forward(p64, w.n_layer, w.n_head, prefix, None, want_cache=False)["logits"][:, -1]
        assert rel_max(lg, ref) <= 1e-4, t

    seq = _decode(st, params, w, prompt, w.block_size, 50, rng, check)
    # the last position of the block still fits; the cache then holds block_size positions
    lg, _, _, _ = st.decode_step(seq[:, -1].astype(np.int32), uniform=np.zeros(3, np.float32))
    check(w.block_size - 1, seq, lg.cpu().numpy())
    with pytest.raises(G.GPT2Error):
        st.decode_step(np.zeros(3, np.int32), uniform=np.zeros(3, np.float32))


def test_decode_124m_bf16_five_sequences():
    """The pages' sampling setup at the 124M size in bf16: 5 sequences, an 8-token prompt
    continued to 30 tokens with top-50 sampling. Every step's logits against the oracle's
    forward over the prefix (cosine >= 0.999 per sequence), the sampler as in _decode, and
    the cached path against the library's full forward over the final tokens (cosine >=
    0.9999 at every position)."""
    note("decode 124M bf16 B=5")
    w = synthetic.workload("gpt2_step")
    params = synthetic.init_params(w)
    p64 = f64(params)
    st = make_step(w, "bf16", max_batch=5)
    st.set_params(params)
    rng = np.random.default_rng(8)
    prompt = rng.integers(0, w.vocab_size, (5, 8))
    steps = []

    def check(t, prefix, lg):
        ref = O.forward(p64, w.n_layer, w.n_head, prefix, None, want_cache=False)["logits"][:, -1]
        for b in range(lg.shape[0]):
            assert cosine(lg[b], ref[b]) >= 0.999, (t, b)
        steps.append(lg)

    seq = _decode(st, params, w, prompt, 30, 50, rng, check)
    _, full = st.forward(seq[:, :29].astype(np.int32), None, want_logits=True)
    full = full.cpu().numpy()
    for t, lg in enumerate(steps):
        for b in range(5):
            assert cosine(lg[b], full[b, t]) >= 0.9999, (t, b)
    assert G.gpt2_decode_position(st.h) == -1   # the forward overwrote the cache


@pytest.mark.parametrize("k", [1, 50, 64])
def test_decode_all_logits_equal(k):
    """Ties everywhere: with wte = 0 every logit of the tied lm_head is exactly 0 (bf16, the
    124M widths, 2 layers, 4 sequences), so the k most probable tokens are the k lowest ids,
    each with probability 1/k, and the draw is the oracle sampler's on the same row."""
    note(f"decode all-equal logits k={k}")
    w = synthetic.workload("gpt2_step", n_layer=2)
    params = synthetic.init_params(w)
    params["wte"][:] = 0.0
    st = make_step(w, "bf16", max_batch=4)
    st.set_params(params)
    st.decode_reset(4)
    u = np.array([0.0, 0.31, 0.71, 0.999], np.float32)   # no multiple of 1/k: no cumulative boundary
    logits, nxt, ids, probs = st.decode_step(np.array([3, 50000, 0, 17], np.int32), uniform=u, top_k=k)
    lg = logits.cpu().numpy()
    assert np.all(lg == 0.0)
    nxt, ids, probs = nxt.cpu().numpy(), ids.cpu().numpy(), probs.cpu().numpy()
    for b in range(4):
        assert np.array_equal(ids[b], np.arange(k)), b
        np.testing.assert_allclose(probs[b], np.full(k, 1.0 / k), rtol=0, atol=1e-7)
        tok, rids, _ = O.topk_sample(lg[b], k, float(u[b]))
        assert np.array_equal(rids, np.arange(k))
        assert nxt[b] == tok, b


@pytest.mark.parametrize("mode", ["fp32", "bf16"])
def test_decode_device_position_graph_matches_eager(mode):
    """gpt2_decode_step_device captured once in a HIP graph and replayed: the position comes
    from device memory and the step advances it there, the drawn token feeds the next step
    through the same buffer, a fresh uniform row is copied in before each replay. After a
    6-token prompt fed eagerly, 12 replayed steps give the same logits and drawn tokens, bit for
    bit, as 12 eager gpt2_decode_step calls on a second handle with the same weights; the
    device position ends at 18. fp32 check mode (the register-staged products take the row
    offset) and bf16 (the few-row products), 2 layers at the 124M widths, 3 sequences."""
    note(f"decode graph replay {mode}")
    w = synthetic.workload("gpt2_step", n_layer=2, block_size=64, seq_len=64)
    params = synthetic.init_params(w, randomize_affine=True)
    B, n_prompt, n_gen = 3, 6, 12
    rng = np.random.default_rng(11)
    prompt = torch.from_numpy(rng.integers(0, w.vocab_size, (B, n_prompt)).astype(np.int32)).cuda()
    uni = torch.from_numpy(rng.random((n_gen, B)).astype(np.float32)).cuda()
    Vp = w.padded_vocab_size

    def start():
        st = make_step(w, mode, max_batch=B)
        st.set_params(params)
        G.gpt2_decode_reset(st.h, B)
        for t in range(n_prompt - 1):
            G.gpt2_decode_step(st.h, prompt[:, t].contiguous().data_ptr())
        return st

    # eager, host position
    ea = start()
    tok = prompt[:, n_prompt - 1].contiguous()
    lg_e, nx_e = [], []
    for i in range(n_gen):
        lg = torch.empty((B, Vp), dtype=torch.float32, device="cuda")
        nxt = torch.empty(B, dtype=torch.int32, device="cuda")
        G.gpt2_decode_step(ea.h, tok.data_ptr(), lg.data_ptr(), 50, uni[i].contiguous().data_ptr(), nxt.data_ptr())
        torch.cuda.synchronize()
        lg_e.append(lg.clone())
        nx_e.append(nxt.clone())
        tok = nxt
    ea.close()

    # captured once, replayed
    gb = start()
    d_pos = torch.tensor([n_prompt - 1], dtype=torch.int32, device="cuda")
    buf = prompt[:, n_prompt - 1].contiguous().clone()
    u_in = torch.empty(B, dtype=torch.float32, device="cuda")
    lg_g = torch.empty((B, Vp), dtype=torch.float32, device="cuda")
    u_in.copy_(uni[0])
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    saved_pos = d_pos.clone()
    saved_buf = buf.clone()
    with torch.cuda.graph(graph):
        G.gpt2_set_stream(gb.h, torch.cuda.current_stream().cuda_stream)
        G.gpt2_decode_step_device(gb.h, buf.data_ptr(), d_pos.data_ptr(), lg_g.data_ptr(), 50, u_in.data_ptr(),
                                  buf.data_ptr())
    G.gpt2_set_stream(gb.h, gb.stream)
    torch.cuda.synchronize()
    d_pos.copy_(saved_pos)   # capture enqueues nothing, but restore in case it ran
    buf.copy_(saved_buf)
    for i in range(n_gen):
        u_in.copy_(uni[i])
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(lg_g, lg_e[i]), i
        assert torch.equal(buf, nx_e[i]), i
    assert int(d_pos.item()) == n_prompt - 1 + n_gen
    del graph
    gb.close()


def test_decode_state_and_errors():
    """Decoding needs a reset; B is bounded by max_batch; top_k by 1..64 and the vocabulary;
    drawing needs the uniform numbers; k = 1 draws the argmax (lowest id among equal maxima)."""
    note("decode errors")
    w = synthetic.workload("tiny")
    st = make_step(w, "fp32", max_batch=2)
    st.set_params(synthetic.init_params(w))
    tok = np.array([3, 5], dtype=np.int32)
    with pytest.raises(G.GPT2Error):
        st.decode_step(tok)
    with pytest.raises(G.GPT2Error):
        G.gpt2_decode_reset(st.h, 3)
    st.decode_reset(2)
    for bad_k in (0, 65):
        with pytest.raises(G.GPT2Error):
            st.decode_step(tok, uniform=np.zeros(2, np.float32), top_k=bad_k)
    st.decode_reset(2)
    d_tok = torch.from_numpy(tok).cuda()
    d_next = torch.empty(2, dtype=torch.int32, device="cuda")
    with pytest.raises(G.GPT2Error):
        G.gpt2_decode_step(st.h, d_tok.data_ptr(), None, 50, None, d_next.data_ptr())
    st.decode_reset(2)
    logits, nxt, ids, _ = st.decode_step(tok, uniform=np.array([0.99, 0.5], np.float32), top_k=1)
    lg = logits.cpu().numpy()
    assert nxt.cpu().numpy().tolist() == [int(np.argmax(lg[0])), int(np.argmax(lg[1]))]
    assert ids.cpu().numpy()[:, 0].tolist() == nxt.cpu().numpy().tolist()


def test_zero_wte_exact_cross_entropy():
    """wte = 0: every logit is 0, so the loss is ln(50304) up to fp32 rounding."""
    note("zero wte exact CE")
    w = synthetic.workload("gpt2_fwd", n_layer=1)
    params = synthetic.init_params(w, randomize_affine=True)
    params["wte"][:] = 0.0
    (x, y), = synthetic.micro_batches(w, 1, batch=2)
    for dtype in ("bf16", "fp32"):
        st = make_step(w, dtype, max_batch=2)
        st.set_params(params)
        loss, logits = st.forward(x, y, want_logits=True)
        assert abs(loss - math.log(50304)) <= 2e-6 * math.log(50304), (dtype, loss)
        assert float(logits.abs().max()) == 0.0
        dz = st.debug_tensor("dz").cpu().numpy().reshape(x.size, -1)
        n = x.size
        expect = np.full_like(dz, 1.0 / (50304 * n))
        expect[np.arange(n), y.reshape(-1)] -= 1.0 / n
        assert rel_max(dz, expect) <= (1e-2 if dtype == "bf16" else 1e-5)


# ------------------------------------------------------------------ optimizer in isolation
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_adamw_matches_oracle(dtype):
    """Same fp32 grads and moments on both sides; two steps (t=1 with clipping, t=2)."""
    note(f"adamw {dtype}")
    w = synthetic.workload("tiny")
    st = make_step(w, dtype)
    params = synthetic.init_params(w, randomize_affine=True)
    st.set_params(params)
    rng = np.random.default_rng(9)
    p = f64(params)
    m = {k: np.zeros_like(v) for k, v in p.items()}
    v = {k: np.zeros_like(x) for k, x in p.items()}
    for t, scale in ((1, 3.0), (2, 0.01)):
        grads = {k: (rng.standard_normal(a.shape) * scale).astype(np.float32) for k, a in params.items()}
        gt = torch.from_numpy(st.pack(grads)).cuda()
        G.gpt2_set_grads(st.h, gt.data_ptr(), 1)
        lr = 1e-3 * t
        norm = st.adamw_step(lr, t=t)
        ref_norm = O.optimizer_step(p, f64(grads), m, v, t, lr)
        assert norm == pytest.approx(ref_norm, rel=1e-5)
        got = st.params()
        for k in p:
            assert np.abs(got[k] - p[k]).max() <= 1e-6 * max(np.abs(p[k]).max(), 1e-3), (t, k)
    mm = torch.empty(st.n_params, dtype=torch.float32, device="cuda")
    vv = torch.empty_like(mm)
    G.gpt2_get_moments(st.h, mm.data_ptr(), vv.data_ptr(), 1)
    mg, vg = st.unpack(mm.cpu().numpy()), st.unpack(vv.cpu().numpy())
    for k in p:
        assert rel_max(mg[k], m[k]) <= 1e-5 and rel_max(vg[k], v[k]) <= 1e-5, k


def test_device_schedule_and_adamw_match_host_path():
    """gpt2_schedule_step_device + gpt2_adamw_step_device against the host-scalar path on two
    handles holding the same state, over warmup, cosine and the tail of the schedule: the
    device learning rate equals gpt2_cosine_lr rounded to float, and parameters and moments
    agree to the last bits the bias corrections may differ in (double pow on the two sides)."""
    note("device schedule + adamw")
    w = synthetic.workload("tiny")
    params = synthetic.init_params(w, randomize_affine=True)
    a, b = make_step(w, "bf16"), make_step(w, "bf16")
    a.set_params(params)
    b.set_params(params)
    rng = np.random.default_rng(11)
    sched = dict(max_lr=6e-4, min_lr=6e-5, warmup_steps=3, max_steps=6)
    step0 = 1
    d_step = torch.tensor([step0], dtype=torch.int32, device="cuda")
    d_lr = torch.zeros(1, dtype=torch.float32, device="cuda")
    d_t = torch.zeros(1, dtype=torch.int32, device="cuda")
    for it in range(step0, step0 + 7):   # warmup, cosine, past max_steps
        grads = {k: (rng.standard_normal(x.shape) * 0.5).astype(np.float32) for k, x in params.items()}
        gt = torch.from_numpy(a.pack(grads)).cuda()
        G.gpt2_set_grads(a.h, gt.data_ptr(), 1)
        G.gpt2_set_grads(b.h, gt.data_ptr(), 1)
        lr = G.gpt2_cosine_lr(it, **sched)
        a.adamw_step(lr, t=it + 1)
        G.gpt2_schedule_step_device(b.h, d_step.data_ptr(), d_lr.data_ptr(), d_t.data_ptr(), **sched)
        G.gpt2_adamw_step_device(b.h, d_lr.data_ptr(), d_t.data_ptr())
        torch.cuda.synchronize()
        assert int(d_step.item()) == it + 1 and int(d_t.item()) == it + 1
        assert float(d_lr.item()) == float(np.float32(lr)), (it, float(d_lr.item()), lr)
    pa, pb = a.params(), b.params()
    for k in pa:
        assert rel_max(pb[k], pa[k]) <= 1e-6, k
    ma = torch.empty(a.n_params, dtype=torch.float32, device="cuda")
    va, mb, vb = torch.empty_like(ma), torch.empty_like(ma), torch.empty_like(ma)
    G.gpt2_get_moments(a.h, ma.data_ptr(), va.data_ptr(), 1)
    G.gpt2_get_moments(b.h, mb.data_ptr(), vb.data_ptr(), 1)
    assert torch.equal(ma, mb) and torch.equal(va, vb)   # the moments do not see the bias corrections
    a.close()
    b.close()


def test_hip_graph_full_training_step():
    """A whole training step -- schedule, forward, backward, AdamW with its scalars in device
    memory -- captured once in a HIP graph and replayed three times, against the same calls made
    eagerly on a second handle from the same state: every step's loss and the final parameters
    and moments agree bit for bit, and the schedule advanced three steps."""
    note("hip graph full training step")
    w = synthetic.workload("gpt2_step", n_layer=2, batch=2, seq_len=256, block_size=256)
    params = synthetic.init_params(w, randomize_affine=True)
    (x, y), = synthetic.micro_batches(w, 1)
    B, T = x.shape
    xd, yd = torch.from_numpy(x).cuda(), torch.from_numpy(y).cuda()
    sched = dict(max_lr=6e-4, min_lr=6e-5, warmup_steps=2, max_steps=10)

    def make():
        st = make_step(w, "bf16")
        st.set_params(params)
        bufs = dict(step=torch.zeros(1, dtype=torch.int32, device="cuda"),
                    lr=torch.zeros(1, dtype=torch.float32, device="cuda"),
                    t=torch.zeros(1, dtype=torch.int32, device="cuda"),
                    loss=torch.zeros(1, dtype=torch.float32, device="cuda"))
        return st, bufs

    def step(st, b):
        G.gpt2_schedule_step_device(st.h, b["step"].data_ptr(), b["lr"].data_ptr(), b["t"].data_ptr(), **sched)
        G.gpt2_forward(st.h, xd.data_ptr(), yd.data_ptr(), B, T, None, b["loss"].data_ptr())
        G.gpt2_backward(st.h, 1.0, 0)
        G.gpt2_adamw_step_device(st.h, b["lr"].data_ptr(), b["t"].data_ptr())

    eager, be = make()
    losses = []
    for _ in range(3):
        step(eager, be)
        torch.cuda.synchronize()
        losses.append(be["loss"].clone())
    graphed, bg = make()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        G.gpt2_set_stream(graphed.h, torch.cuda.current_stream().cuda_stream)
        step(graphed, bg)
    G.gpt2_set_stream(graphed.h, graphed.stream)
    torch.cuda.synchronize()
    assert int(bg["step"].item()) == 0        # capturing ran nothing
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(bg["loss"], losses[rep]), rep
    assert int(bg["step"].item()) == 3 and int(bg["t"].item()) == 3
    for get in (G.gpt2_get_params, G.gpt2_get_grads):
        u = torch.empty(eager.n_params, dtype=torch.float32, device="cuda")
        v = torch.empty_like(u)
        get(eager.h, u.data_ptr(), 1)
        get(graphed.h, v.data_ptr(), 1)
        assert torch.equal(u, v)
    m1, v1, m2, v2 = (torch.empty(eager.n_params, dtype=torch.float32, device="cuda") for _ in range(4))
    G.gpt2_get_moments(eager.h, m1.data_ptr(), v1.data_ptr(), 1)
    G.gpt2_get_moments(graphed.h, m2.data_ptr(), v2.data_ptr(), 1)
    assert torch.equal(m1, m2) and torch.equal(v1, v2)
    del graph
    eager.close()
    graphed.close()


def test_full_training_step_runs_and_decreases_loss():
    """Forward, backward, AdamW on the tiny model: loss goes down over a few steps on one batch
    (the overfit-a-batch sanity loop of chapter 52:38-1:06:18)."""
    note("tiny overfit")
    w = synthetic.workload("tiny")
    params = synthetic.init_params(w)
    (x, y), = synthetic.micro_batches(w, 1)
    st = make_step(w, "bf16")
    st.set_params(params)
    losses = []
    for t in range(1, 31):
        loss, _ = st.forward(x, y)
        losses.append(loss)
        st.backward(1.0, False)
        st.adamw_step(3e-3, t=t)
    assert losses[-1] < losses[0] - 1.0, losses


# ------------------------------------------------------------------ init and error paths
def test_device_init_statistics():
    note("device init")
    w = synthetic.workload("gpt2_step", n_layer=2)
    st = make_step(w, "bf16", max_batch=1, seed=1234)
    got = st.params()
    resid = 0.02 / math.sqrt(2 * w.n_layer)
    for name, shape, kind in synthetic.param_spec(w):
        a = got[name]
        if kind == "zeros":
            assert np.all(a == 0), name
        elif kind == "ones":
            assert np.all(a == 1), name
        else:
            s = 0.02 if kind == "normal" else resid
            assert abs(a.std() / s - 1) <= 0.01, (name, a.std())
            assert abs(a.mean()) <= 0.05 * s, name


def test_error_paths():
    note("error paths")
    w = synthetic.workload("tiny")
    st = make_step(w, "fp32")
    with pytest.raises(G.GPT2Error) as e:
        st.backward(1.0, False)
    assert e.value.code == G.GPT2_ESTATE
    x = np.zeros((5, 8), np.int32)
    with pytest.raises(G.GPT2Error) as e:
        st.forward(x, x)
    assert e.value.code == G.GPT2_EINVAL
    x = np.zeros((1, 65), np.int32)
    with pytest.raises(G.GPT2Error) as e:
        st.forward(x, x)
    assert e.value.code == G.GPT2_EINVAL
    with pytest.raises(G.GPT2Error):
        G.gpt2_forward(st.h, 0, 0, 0, 8)
