"""The C-ABI library loads and exports what include/gpt2.h declares; its host-only logic
(sizes, canonical layout, learning-rate schedule, argument validation) is checked without a
GPU. No kernel is launched here."""
import os
import re

import numpy as np
import pytest

import synthetic
import transformer_lm_step_amd as G
from oracle import gpt2_oracle as O

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "gpt2.h")


def _cfg(w, dtype="bf16", vocab_rows=None):
    return G.make_config(w.n_layer, w.n_head, w.n_embd, w.block_size, w.vocab_size,
                         w.padded_vocab_size if vocab_rows is None else vocab_rows, w.batch, dtype)


def test_every_declared_symbol_is_exported():
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(gpt2_[a-z_0-9]+)\s*\(", text))
    assert len(declared) >= 20
    lib = G._lib
    for name in declared:
        assert hasattr(lib, name), name
    assert declared == set(G.EXPORTED)


def test_param_counts_and_decay_prefix():
    w = synthetic.workload("gpt2_step")
    assert G.gpt2_num_params(_cfg(w, vocab_rows=50257)) == 124439808
    cfg = _cfg(w)
    assert G.gpt2_num_params(cfg) == 124475904
    assert G.gpt2_num_tensors(cfg) == 148
    assert G.gpt2_num_decay_tensors(cfg) == 50
    assert G.gpt2_decay_end(cfg) == 124354560
    xl = synthetic.workload("gpt2_xl")
    assert G.gpt2_num_params(_cfg(xl)) == 1557686400
    assert G.gpt2_num_params(_cfg(xl, vocab_rows=50257)) == 1557611200
    assert G.gpt2_num_params(_cfg(synthetic.workload("tiny"), "fp32")) == 120576


@pytest.mark.parametrize("name", ["tiny", "gpt2_step", "gpt2_xl"])
def test_layout_matches_named_shapes(name):
    w = synthetic.workload(name)
    cfg = _cfg(w)
    spec = {n: s for n, s, _ in synthetic.param_spec(w)}
    infos = [G.gpt2_param_info(cfg, i) for i in range(G.gpt2_num_tensors(cfg))]
    assert {n for n, _, _ in infos} == set(spec)
    end = 0
    decay_end = G.gpt2_decay_end(cfg)
    for n, off, shape in infos:
        assert tuple(shape) == spec[n], n
        assert off == end, n                       # contiguous, in order
        end += int(np.prod(shape))
        assert (len(shape) == 2) == (off < decay_end), n
    assert end == G.gpt2_num_params(cfg)


def test_cosine_lr_matches_oracle_and_pages():
    for it in (0, 1, 100, 714, 715, 716, 5000, 19072, 19073, 19074, 25000):
        assert G.gpt2_cosine_lr(it) == pytest.approx(O.get_lr(it), rel=1e-13, abs=0)
    assert G.gpt2_cosine_lr(100) == pytest.approx(8.475524475524476e-05, rel=1e-12)


def test_workspace_and_validation():
    w = synthetic.workload("gpt2_step")
    n = G.gpt2_workspace_bytes(_cfg(w))
    assert n > 4 * 4 * 124475904
    bad = _cfg(w)
    bad.n_head = 7
    with pytest.raises(G.GPT2Error):
        G.gpt2_workspace_bytes(bad)
    assert "n_head" in G.gpt2_last_error()
    bad = _cfg(w)
    bad.padded_vocab_size = 50000
    with pytest.raises(G.GPT2Error):
        G.gpt2_num_params(bad)
    with pytest.raises(G.GPT2Error):
        G.gpt2_param_info(_cfg(w), 148)


def test_kernel_classes_listed():
    cls = G.kernel_classes()
    for c in ("gemm_lm_head", "attn_fwd", "attn_bwd", "adamw", "cross_entropy", "layernorm_fwd"):
        assert c in cls
