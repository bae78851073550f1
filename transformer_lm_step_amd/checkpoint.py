"""Full training-state checkpoints for the GPT-2 step library.

The lecture notes ("Karpathy's Zero to Hero, Lecture 9", chapter 3:43:45-3:59:10) save the
model's state dict, its config, the step and the validation loss, and point out that resuming
exactly also needs the optimizer state and the data position; the reproduce-gpt2 README ("The
GPT-2 run") restarts a run from its last checkpoint after a failure. A state here is exactly
what the next optimizer step reads:

* the canonical fp32 parameter arena (``gpt2_get_params``; the bf16 weight copies are rebuilt
  from it by ``gpt2_set_params``),
* the AdamW first and second moments (``gpt2_get_moments``),
* the AdamW step count t of the last update (bias corrections use t + 1 next),
* the data position (the index of the next micro-batch of the caller's token stream),
* the model config, checked on load.

Gradients are not state: every optimizer step starts with a backward pass that overwrites them.
With these restored, a resumed run repeats the uninterrupted one bit for bit (the step is
deterministic).

File format: an uncompressed ``.npz`` (no pickled objects; loaded with ``allow_pickle=False``)
holding ``params``, ``m``, ``v`` (float32, one element per parameter) and ``meta`` (the UTF-8
bytes of a JSON object). Writes go to a temporary file in the same directory, which is flushed
to disk and then renamed over the target, so a process killed while saving leaves the previous
checkpoint intact.
"""
from __future__ import annotations

import io
import json
import os
from typing import Any, Dict, Optional

import numpy as np

FORMAT = "gpt2-step-state/1"
CONFIG_KEYS = ("n_layer", "n_head", "n_embd", "mlp_hidden", "block_size", "vocab_size", "padded_vocab_size")


def config_dict(cfg) -> Dict[str, int]:
    """The model-shape fields of a ``gpt2_config`` (batch capacity and dtype are not part of
    the model: a state saved in one mode or capacity loads into another)."""
    return {k: int(getattr(cfg, k)) for k in CONFIG_KEYS}


def write_state(path: str, params: np.ndarray, m: np.ndarray, v: np.ndarray, adam_t: int, data_pos: int,
                config: Dict[str, int], extra: Optional[Dict[str, Any]] = None) -> None:
    """Atomically write one state file (see the module docstring)."""
    params = np.ascontiguousarray(params, dtype=np.float32).reshape(-1)
    m = np.ascontiguousarray(m, dtype=np.float32).reshape(-1)
    v = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
    if not (params.size == m.size == v.size):
        raise ValueError("params, m and v must have the same number of elements")
    if adam_t < 0 or data_pos < 0:
        raise ValueError("adam_t and data_pos must be non-negative")
    meta = {"format": FORMAT, "config": {k: int(config[k]) for k in CONFIG_KEYS}, "n_params": int(params.size),
            "adam_t": int(adam_t), "data_pos": int(data_pos), "extra": extra or {}}
    buf = io.BytesIO()
    np.savez(buf, params=params, m=m, v=v, meta=np.frombuffer(json.dumps(meta).encode(), dtype=np.uint8))
    d = os.path.dirname(os.path.abspath(path))
    tmp = os.path.join(d, f".{os.path.basename(path)}.{os.getpid()}.tmp")
    try:
        with open(tmp, "wb") as f:
            f.write(buf.getbuffer())
            f.flush()
            os.fsync(f.fileno())
        os.replace(tmp, path)
    finally:
        if os.path.exists(tmp):
            os.unlink(tmp)
    try:  # make the rename itself durable
        fd = os.open(d, os.O_RDONLY)
        try:
            os.fsync(fd)
        finally:
            os.close(fd)
    except OSError:
        pass


def read_state(path: str) -> Dict[str, Any]:
    """Read a state file: dict with params, m, v (float32 arrays), adam_t, data_pos, config, extra."""
    with np.load(path, allow_pickle=False) as z:
        meta = json.loads(bytes(z["meta"]).decode())
        if meta.get("format") != FORMAT:
            raise ValueError(f"{path}: not a {FORMAT} file")
        out = {"params": z["params"], "m": z["m"], "v": z["v"]}
    n = meta["n_params"]
    for k in ("params", "m", "v"):
        if out[k].dtype != np.float32 or out[k].shape != (n,):
            raise ValueError(f"{path}: array {k} has dtype {out[k].dtype} and shape {out[k].shape}, expected float32 ({n},)")
    out.update(adam_t=int(meta["adam_t"]), data_pos=int(meta["data_pos"]), config=meta["config"],
               extra=meta.get("extra", {}))
    return out


def save(step, path: str, adam_t: int, data_pos: int, extra: Optional[Dict[str, Any]] = None) -> None:
    """Save the state of a ``GPT2Step`` (device arenas copied to the host)."""
    from . import gpt2_get_moments, gpt2_get_params
    torch = step.torch
    p = torch.empty(step.n_params, dtype=torch.float32, device=step.device)
    m = torch.empty_like(p)
    v = torch.empty_like(p)
    gpt2_get_params(step.h, p.data_ptr(), 1)
    gpt2_get_moments(step.h, m.data_ptr(), v.data_ptr(), 1)
    torch.cuda.synchronize(step.device)
    write_state(path, p.cpu().numpy(), m.cpu().numpy(), v.cpu().numpy(), adam_t, data_pos,
                config_dict(step.cfg), extra)


def load(step, path: str) -> Dict[str, Any]:
    """Restore a state into a ``GPT2Step`` of the same model shape; returns the state's
    adam_t, data_pos and extra. Raises ValueError on a shape or size mismatch."""
    from . import gpt2_set_moments, gpt2_set_params
    st = read_state(path)
    want = config_dict(step.cfg)
    if st["config"] != want:
        raise ValueError(f"{path}: saved for config {st['config']}, this handle has {want}")
    if st["params"].size != step.n_params:
        raise ValueError(f"{path}: {st['params'].size} parameters, this handle has {step.n_params}")
    torch = step.torch
    p = torch.from_numpy(st["params"]).to(step.device)
    m = torch.from_numpy(st["m"]).to(step.device)
    v = torch.from_numpy(st["v"]).to(step.device)
    gpt2_set_params(step.h, p.data_ptr(), 1)
    gpt2_set_moments(step.h, m.data_ptr(), v.data_ptr(), 1)
    torch.cuda.synchronize(step.device)
    return {"adam_t": st["adam_t"], "data_pos": st["data_pos"], "extra": st["extra"]}
