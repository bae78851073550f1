"""Python binding of the MI355X GPT-2 training-step library (``libgpt2_step.so``).

The functions here carry the C ABI's names and do argument marshalling only: every step of
the computation runs in the library's HIP kernels. PyTorch is used by callers for device
memory and streams; :class:`GPT2Step` is a convenience holder that allocates the workspace
as a torch tensor and passes raw pointers.

Importing this package loads the library and raises if it has not been built
(``python transformer_lm_step_amd/build.py``). There is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build, or another build of the same library named by GPT2_STEP_LIB
LIB_PATH = os.environ.get("GPT2_STEP_LIB") or os.path.join(_HERE, "libgpt2_step.so")

GPT2_OK, GPT2_EINVAL, GPT2_ESTATE, GPT2_EHIP = 0, -1, -2, -3
GPT2_FP32, GPT2_BF16, GPT2_BF16_RES16 = 0, 1, 2
GPT2_NOALLOC_MAX_SEQ, GPT2_NOALLOC_MAX_ROWS = 4096, 262144
# dtype names accepted by make_config: the C ABI's three arithmetic modes
DTYPES = {"fp32": GPT2_FP32, "bf16": GPT2_BF16, "bf16_res16": GPT2_BF16_RES16}


class gpt2_config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "n_layer", "n_head", "n_embd", "mlp_hidden", "block_size", "vocab_size",
        "padded_vocab_size", "max_batch", "dtype")]


class GPT2Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gpt2 error {code}: {msg}")
        self.code = code


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python transformer_lm_step_amd/build.py`")
# torch ships its own HIP runtime with the same soname as the system one. Loading torch first
# makes the library bind to that already-loaded runtime, so one process never holds two.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

_P = ctypes.c_void_p
_CFG = ctypes.POINTER(gpt2_config)
_SIGS = {
    "gpt2_workspace_bytes": (ctypes.c_size_t, [_CFG]),
    "gpt2_num_params": (ctypes.c_int64, [_CFG]),
    "gpt2_num_tensors": (ctypes.c_int32, [_CFG]),
    "gpt2_num_decay_tensors": (ctypes.c_int32, [_CFG]),
    "gpt2_param_info": (ctypes.c_int, [_CFG, ctypes.c_int32, ctypes.POINTER(ctypes.c_char_p),
                                       ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]),
    "gpt2_decay_end": (ctypes.c_int64, [_CFG]),
    "gpt2_create": (ctypes.c_int, [_CFG, _P, ctypes.c_size_t, ctypes.c_uint64, _P, ctypes.POINTER(_P)]),
    "gpt2_destroy": (ctypes.c_int, [_P]),
    "gpt2_set_stream": (ctypes.c_int, [_P, _P]),
    "gpt2_set_params": (ctypes.c_int, [_P, _P, ctypes.c_int]),
    "gpt2_get_params": (ctypes.c_int, [_P, _P, ctypes.c_int]),
    "gpt2_get_grads": (ctypes.c_int, [_P, _P, ctypes.c_int]),
    "gpt2_set_grads": (ctypes.c_int, [_P, _P, ctypes.c_int]),
    "gpt2_get_moments": (ctypes.c_int, [_P, _P, _P, ctypes.c_int]),
    "gpt2_evaluate": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "gpt2_evaluate_noalloc": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]),
    "gpt2_decode_reset": (ctypes.c_int, [_P, ctypes.c_int32]),
    "gpt2_decode_step": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, _P, _P, _P, _P]),
    "gpt2_decode_step_device": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_int32, _P, _P, _P, _P]),
    "gpt2_decode_position": (ctypes.c_int32, [_P]),
    "gpt2_set_moments": (ctypes.c_int, [_P, _P, _P, ctypes.c_int]),
    "gpt2_params_device": (_P, [_P]),
    "gpt2_grads_device": (_P, [_P]),
    "gpt2_forward": (ctypes.c_int, [_P, _P, _P, ctypes.c_int32, ctypes.c_int32, _P, _P,
                                    ctypes.POINTER(ctypes.c_float)]),
    "gpt2_backward": (ctypes.c_int, [_P, ctypes.c_float, ctypes.c_int32]),
    "gpt2_adamw_step": (ctypes.c_int, [_P, ctypes.c_float, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_float, ctypes.c_int32, _P,
                                       ctypes.POINTER(ctypes.c_float)]),
    "gpt2_adamw_step_device": (ctypes.c_int, [_P, _P, _P, ctypes.c_float, ctypes.c_float, ctypes.c_float,
                                              ctypes.c_float, ctypes.c_float, _P]),
    "gpt2_schedule_step_device": (ctypes.c_int, [_P, _P, _P, _P, ctypes.c_double, ctypes.c_double,
                                                 ctypes.c_int64, ctypes.c_int64]),
    "gpt2_cosine_lr": (ctypes.c_double, [ctypes.c_int64, ctypes.c_double, ctypes.c_double, ctypes.c_int64,
                                         ctypes.c_int64]),
    "gpt2_last_error": (ctypes.c_char_p, []),
    "gpt2_timing_begin": (ctypes.c_int, [_P, ctypes.c_char_p]),
    "gpt2_timing_end": (ctypes.c_int, [_P]),
    "gpt2_timing_get": (ctypes.c_int, [_P, ctypes.c_char_p, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64)]),
    "gpt2_kernel_class": (ctypes.c_char_p, [ctypes.c_int32]),
    "gpt2_debug_tensor": (ctypes.c_int, [_P, ctypes.c_char_p, ctypes.c_int32, _P, ctypes.POINTER(ctypes.c_int64)]),
}
for _name, (_res, _args) in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args

EXPORTED = tuple(_SIGS)


def gpt2_last_error() -> str:
    return (_lib.gpt2_last_error() or b"").decode()


def _check(rc: int) -> int:
    if rc != GPT2_OK:
        raise GPT2Error(rc, gpt2_last_error())
    return rc


def make_config(n_layer, n_head, n_embd, block_size, vocab_size, padded_vocab_size, max_batch,
                dtype="bf16", mlp_hidden=None) -> gpt2_config:
    return gpt2_config(n_layer, n_head, n_embd, 4 * n_embd if mlp_hidden is None else mlp_hidden,
                       block_size, vocab_size, padded_vocab_size, max_batch,
                       dtype if isinstance(dtype, int) else DTYPES[dtype])


# ---------------------------------------------------------------- C ABI, same names
def gpt2_workspace_bytes(cfg: gpt2_config) -> int:
    n = _lib.gpt2_workspace_bytes(ctypes.byref(cfg))
    if n == 0:
        raise GPT2Error(GPT2_EINVAL, gpt2_last_error())
    return n


def gpt2_num_params(cfg: gpt2_config) -> int:
    n = _lib.gpt2_num_params(ctypes.byref(cfg))
    if n < 0:
        raise GPT2Error(GPT2_EINVAL, gpt2_last_error())
    return n


def gpt2_num_tensors(cfg: gpt2_config) -> int:
    return _lib.gpt2_num_tensors(ctypes.byref(cfg))


def gpt2_num_decay_tensors(cfg: gpt2_config) -> int:
    return _lib.gpt2_num_decay_tensors(ctypes.byref(cfg))


def gpt2_decay_end(cfg: gpt2_config) -> int:
    return _lib.gpt2_decay_end(ctypes.byref(cfg))


def gpt2_param_info(cfg: gpt2_config, i: int):
    name = ctypes.c_char_p()
    off = ctypes.c_int64()
    shape = (ctypes.c_int64 * 2)()
    _check(_lib.gpt2_param_info(ctypes.byref(cfg), i, ctypes.byref(name), ctypes.byref(off), shape))
    shp = (shape[0], shape[1]) if shape[1] else (shape[0],)
    return name.value.decode(), off.value, shp


def gpt2_create(cfg: gpt2_config, d_ws: int, ws_bytes: int, seed: int, stream: int) -> int:
    h = _P()
    _check(_lib.gpt2_create(ctypes.byref(cfg), d_ws, ws_bytes, seed, stream, ctypes.byref(h)))
    return h.value


def gpt2_destroy(h: int) -> None:
    _check(_lib.gpt2_destroy(h))


def gpt2_set_stream(h: int, stream: int) -> None:
    _check(_lib.gpt2_set_stream(h, stream))


def gpt2_set_params(h, src_ptr, on_device=1):
    _check(_lib.gpt2_set_params(h, src_ptr, on_device))


def gpt2_get_params(h, dst_ptr, on_device=1):
    _check(_lib.gpt2_get_params(h, dst_ptr, on_device))


def gpt2_get_grads(h, dst_ptr, on_device=1):
    _check(_lib.gpt2_get_grads(h, dst_ptr, on_device))


def gpt2_set_grads(h, src_ptr, on_device=1):
    _check(_lib.gpt2_set_grads(h, src_ptr, on_device))


def gpt2_get_moments(h, m_ptr, v_ptr, on_device=1):
    _check(_lib.gpt2_get_moments(h, m_ptr, v_ptr, on_device))


def gpt2_set_moments(h, m_ptr, v_ptr, on_device=1):
    _check(_lib.gpt2_set_moments(h, m_ptr, v_ptr, on_device))


def gpt2_params_device(h) -> int:
    return _lib.gpt2_params_device(h)


def gpt2_grads_device(h) -> int:
    return _lib.gpt2_grads_device(h)


def gpt2_forward(h, d_idx, d_targets, B, T, d_logits=None, d_loss=None, want_host_loss=False) -> Optional[float]:
    hl = ctypes.c_float()
    _check(_lib.gpt2_forward(h, d_idx, d_targets, B, T, d_logits, d_loss,
                             ctypes.byref(hl) if want_host_loss else None))
    return hl.value if want_host_loss else None


def gpt2_evaluate(h, d_idx, d_targets, d_mask, B, T, d_row_sum=None, d_row_mean=None, d_loss=None) -> None:
    _check(_lib.gpt2_evaluate(h, d_idx, d_targets, d_mask, B, T, d_row_sum, d_row_mean, d_loss))


def gpt2_evaluate_noalloc(h, d_idx, d_targets, d_mask, B, T, d_row_sum=None, d_row_mean=None,
                          d_loss=None) -> None:
    _check(_lib.gpt2_evaluate_noalloc(h, d_idx, d_targets, d_mask, B, T, d_row_sum, d_row_mean, d_loss))


def gpt2_decode_reset(h, B: int) -> None:
    _check(_lib.gpt2_decode_reset(h, B))


def gpt2_decode_step(h, d_tokens, d_logits=None, top_k=50, d_uniform=None, d_next=None, d_topk_idx=None,
                     d_topk_prob=None) -> None:
    _check(_lib.gpt2_decode_step(h, d_tokens, d_logits, top_k, d_uniform, d_next, d_topk_idx, d_topk_prob))


def gpt2_decode_step_device(h, d_tokens, d_pos, d_logits=None, top_k=50, d_uniform=None, d_next=None,
                            d_topk_idx=None, d_topk_prob=None) -> None:
    _check(_lib.gpt2_decode_step_device(h, d_tokens, d_pos, d_logits, top_k, d_uniform, d_next, d_topk_idx,
                                        d_topk_prob))


def gpt2_decode_position(h) -> int:
    return _lib.gpt2_decode_position(h)


def gpt2_backward(h, grad_scale: float, accumulate: int) -> None:
    _check(_lib.gpt2_backward(h, grad_scale, accumulate))


def gpt2_adamw_step(h, lr, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_grad_norm=1.0, t=1,
                    d_grad_norm=None, want_host_norm=False) -> Optional[float]:
    hn = ctypes.c_float()
    _check(_lib.gpt2_adamw_step(h, lr, beta1, beta2, eps, weight_decay, max_grad_norm, t, d_grad_norm,
                                ctypes.byref(hn) if want_host_norm else None))
    return hn.value if want_host_norm else None


def gpt2_cosine_lr(it, max_lr=6e-4, min_lr=6e-5, warmup_steps=715, max_steps=19073) -> float:
    return _lib.gpt2_cosine_lr(it, max_lr, min_lr, warmup_steps, max_steps)


def gpt2_adamw_step_device(h, d_lr, d_t, beta1=0.9, beta2=0.95, eps=1e-8, weight_decay=0.1, max_grad_norm=1.0,
                           d_grad_norm=None) -> None:
    _check(_lib.gpt2_adamw_step_device(h, d_lr, d_t, beta1, beta2, eps, weight_decay, max_grad_norm, d_grad_norm))


def gpt2_schedule_step_device(h, d_step, d_lr, d_t, max_lr=6e-4, min_lr=6e-5, warmup_steps=715,
                              max_steps=19073) -> None:
    _check(_lib.gpt2_schedule_step_device(h, d_step, d_lr, d_t, max_lr, min_lr, warmup_steps, max_steps))


def gpt2_timing_begin(h, name: Optional[str] = None) -> None:
    _check(_lib.gpt2_timing_begin(h, name.encode() if name else None))


def gpt2_timing_end(h) -> None:
    _check(_lib.gpt2_timing_end(h))


def gpt2_timing_get(h, name: str):
    ms = ctypes.c_double()
    n = ctypes.c_int64()
    _check(_lib.gpt2_timing_get(h, name.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def gpt2_kernel_class(i: int) -> Optional[str]:
    r = _lib.gpt2_kernel_class(i)
    return r.decode() if r else None


def gpt2_debug_tensor(h, which: str, layer: int, d_dst=None) -> int:
    n = ctypes.c_int64()
    _check(_lib.gpt2_debug_tensor(h, which.encode(), layer, d_dst, ctypes.byref(n)))
    return n.value


def kernel_classes():
    out, i = [], 0
    while True:
        c = gpt2_kernel_class(i)
        if c is None:
            return out
        out.append(c)
        i += 1


# ---------------------------------------------------------------- convenience holder
class GPT2Step:
    """Owns a torch-allocated workspace and a library handle on the current CUDA/HIP stream."""

    def __init__(self, cfg: gpt2_config, seed: int = 0, device: str = "cuda:0"):
        import torch
        self.torch = torch
        self.cfg = cfg
        self.device = torch.device(device)
        self.ws_bytes = gpt2_workspace_bytes(cfg)
        self.ws = torch.empty(self.ws_bytes + 256, dtype=torch.uint8, device=self.device)
        base = self.ws.data_ptr()
        self.ws_ptr = (base + 255) & ~255
        self.stream = torch.cuda.current_stream(self.device).cuda_stream
        self.h = gpt2_create(cfg, self.ws_ptr, self.ws_bytes, seed, self.stream)
        self.n_params = gpt2_num_params(cfg)
        self.tensors = [gpt2_param_info(cfg, i) for i in range(gpt2_num_tensors(cfg))]

    def close(self):
        if getattr(self, "h", None):
            gpt2_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # arena <-> named tensors (host numpy)
    def pack(self, named):
        import numpy as np
        arena = np.zeros(self.n_params, dtype=np.float32)
        for name, off, shape in self.tensors:
            a = np.asarray(named[name], dtype=np.float32)
            assert a.shape == tuple(shape), (name, a.shape, shape)
            arena[off:off + a.size] = a.reshape(-1)
        return arena

    def unpack(self, arena):
        return {name: arena[off:off + int(__import__("math").prod(shape))].reshape(shape)
                for name, off, shape in self.tensors}

    def set_params(self, named):
        t = self.torch.from_numpy(self.pack(named)).to(self.device)
        gpt2_set_params(self.h, t.data_ptr(), 1)
        self.torch.cuda.synchronize(self.device)

    def _arena(self, getter):
        t = self.torch.empty(self.n_params, dtype=self.torch.float32, device=self.device)
        getter(self.h, t.data_ptr(), 1)
        return t

    def params(self):
        return self.unpack(self._arena(gpt2_get_params).cpu().numpy())

    def grads(self):
        return self.unpack(self._arena(gpt2_get_grads).cpu().numpy())

    def forward(self, idx, targets=None, want_logits=False, want_loss=True):
        torch = self.torch
        B, T = idx.shape
        idx_d = idx if isinstance(idx, torch.Tensor) else torch.from_numpy(idx)
        idx_d = idx_d.to(self.device, torch.int32).contiguous()
        tgt_d = None
        if targets is not None:
            tgt_d = targets if isinstance(targets, torch.Tensor) else torch.from_numpy(targets)
            tgt_d = tgt_d.to(self.device, torch.int32).contiguous()
        logits = None
        if want_logits:
            logits = torch.empty((B, T, self.cfg.padded_vocab_size), dtype=torch.float32, device=self.device)
        loss = gpt2_forward(self.h, idx_d.data_ptr(), tgt_d.data_ptr() if tgt_d is not None else None, B, T,
                            logits.data_ptr() if logits is not None else None, None,
                            want_host_loss=(targets is not None and want_loss))
        self._keep = (idx_d, tgt_d)
        return loss, logits

    def evaluate(self, idx, targets, mask=None):
        """Forward-only scoring: (row_sum [B], row_mean [B], loss) as host numpy values, with
        the mask (bool/uint8 [B, T]) selecting the scored positions (None: all)."""
        torch = self.torch
        B, T = idx.shape

        def dev(a, dt):
            t = a if isinstance(a, torch.Tensor) else torch.from_numpy(a)
            return t.to(self.device, dt).contiguous()

        idx_d, tgt_d = dev(idx, torch.int32), dev(targets, torch.int32)
        mask_d = dev(mask, torch.uint8) if mask is not None else None
        out = torch.empty(2 * B + 1, dtype=torch.float32, device=self.device)
        p = out.data_ptr()
        gpt2_evaluate(self.h, idx_d.data_ptr(), tgt_d.data_ptr(), mask_d.data_ptr() if mask_d is not None else None,
                      B, T, p, p + 4 * B, p + 8 * B)
        o = out.cpu().numpy()
        return o[:B].copy(), o[B:2 * B].copy(), float(o[2 * B])

    def decode_reset(self, B):
        gpt2_decode_reset(self.h, B)

    def decode_step(self, tokens, uniform=None, top_k=50, want_logits=True):
        """One decoding step for every cached sequence: returns (logits [B, Vp] fp32 tensor or
        None, next [B] int32 tensor or None, topk ids [B, k], topk probs [B, k]) on the device;
        sampling outputs only when ``uniform`` ([B] in [0, 1)) is given."""
        torch = self.torch
        tok = tokens if isinstance(tokens, torch.Tensor) else torch.from_numpy(tokens)
        tok = tok.to(self.device, torch.int32).contiguous()
        B = tok.numel()
        logits = torch.empty((B, self.cfg.padded_vocab_size), dtype=torch.float32, device=self.device) \
            if want_logits else None
        nxt = ids = probs = u = None
        if uniform is not None:
            u = uniform if isinstance(uniform, torch.Tensor) else torch.from_numpy(uniform)
            u = u.to(self.device, torch.float32).contiguous()
            nxt = torch.empty(B, dtype=torch.int32, device=self.device)
            ids = torch.empty((B, top_k), dtype=torch.int32, device=self.device)
            probs = torch.empty((B, top_k), dtype=torch.float32, device=self.device)
        gpt2_decode_step(self.h, tok.data_ptr(), logits.data_ptr() if logits is not None else None, top_k,
                         u.data_ptr() if u is not None else None, nxt.data_ptr() if nxt is not None else None,
                         ids.data_ptr() if ids is not None else None, probs.data_ptr() if probs is not None else None)
        self._keep = (tok, u)
        return logits, nxt, ids, probs

    def backward(self, grad_scale=1.0, accumulate=False):
        gpt2_backward(self.h, grad_scale, 1 if accumulate else 0)

    def adamw_step(self, lr, t=1, **kw):
        return gpt2_adamw_step(self.h, lr, t=t, want_host_norm=True, **kw)

    def debug_tensor(self, which, layer=0):
        n = gpt2_debug_tensor(self.h, which, layer)
        out = self.torch.empty(n, dtype=self.torch.float32, device=self.device)
        gpt2_debug_tensor(self.h, which, layer, out.data_ptr())
        return out
