"""The allocation-free evaluation entry point (gpt2_evaluate_noalloc, scratch in a fixed device
array of the library) against gpt2_evaluate (scratch in the handle's workspace), through the C
ABI: per-sequence sums and means and the batch mean on two calls in a row, the second with
fewer sequences and positions (so the shared array still holds the first call's values), and
the size limit. Both entry points run the same kernels in the same order, so the results must
agree bit for bit."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import synthetic
from tests.gpu_common import make_step, note

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import transformer_lm_step_amd as G  # noqa: E402


def _scores(st, fn, x, y, mask):
    B, T = x.shape
    xd = torch.from_numpy(x).cuda().contiguous()
    yd = torch.from_numpy(y).cuda().contiguous()
    md = torch.from_numpy(mask.astype(np.uint8)).cuda().contiguous() if mask is not None else None
    out = torch.full((2 * B + 1,), float("nan"), dtype=torch.float32, device="cuda")
    p = out.data_ptr()
    fn(st.h, xd.data_ptr(), yd.data_ptr(), md.data_ptr() if md is not None else None, B, T, p, p + 4 * B, p + 8 * B)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("mode", ["bf16", "fp32"])
def test_evaluate_noalloc_matches_evaluate(mode):
    note(f"evaluate_noalloc {mode}")
    w = synthetic.workload("gpt2_step", n_layer=2, batch=4, seq_len=256, block_size=256)
    params = synthetic.init_params(w, randomize_affine=True)
    st = make_step(w, mode)
    st.set_params(params)
    (x, y), = synthetic.micro_batches(w, 1)
    rng = np.random.default_rng(4)
    mask = rng.random(x.shape) < 0.4
    mask[1] = False
    first = None
    # two calls in a row, the second smaller; then the second shape without a mask
    for (B, T, m) in ((4, 256, mask), (2, 100, mask[:2, :100]), (2, 100, None)):
        xs, ys = np.ascontiguousarray(x[:B, :T]), np.ascontiguousarray(y[:B, :T])
        got = _scores(st, G.gpt2_evaluate_noalloc, xs, ys, m)
        ref = _scores(st, G.gpt2_evaluate, xs, ys, m)
        assert np.all(np.isfinite(ref)), (B, T)
        assert np.array_equal(got, ref), (B, T, got, ref)
        if first is None:
            first = got
    assert first[1] == 0.0 and first[4 + 1] == 0.0     # the sequence with nothing selected
    st.close()


def test_evaluate_noalloc_size_limit():
    note("evaluate_noalloc size limit")
    w = synthetic.workload("tiny", block_size=1, seq_len=1, batch=G.GPT2_NOALLOC_MAX_SEQ + 1)
    st = make_step(w, "fp32")
    st.set_params(synthetic.init_params(w))
    B = G.GPT2_NOALLOC_MAX_SEQ + 1
    x = np.zeros((B, 1), np.int32)
    with pytest.raises(G.GPT2Error) as e:
        _scores(st, G.gpt2_evaluate_noalloc, x, x, None)
    assert e.value.code == G.GPT2_EINVAL and "allocation-free" in str(e.value)
    # within the limit the same handle works
    got = _scores(st, G.gpt2_evaluate_noalloc, x[:G.GPT2_NOALLOC_MAX_SEQ], x[:G.GPT2_NOALLOC_MAX_SEQ], None)
    ref = _scores(st, G.gpt2_evaluate, x[:G.GPT2_NOALLOC_MAX_SEQ], x[:G.GPT2_NOALLOC_MAX_SEQ], None)
    assert np.array_equal(got, ref)
    st.close()
    # more positions than the array holds (257 sequences of 1024: 263,168 > 262,144)
    w = synthetic.workload("tiny", block_size=1024, seq_len=1024, batch=257)
    st = make_step(w, "fp32")
    x = np.zeros((257, 1024), np.int32)
    with pytest.raises(G.GPT2Error) as e:
        _scores(st, G.gpt2_evaluate_noalloc, x, x, None)
    assert e.value.code == G.GPT2_EINVAL and "positions" in str(e.value)
    st.close()
