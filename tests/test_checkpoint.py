"""Checkpoint files of the full training state (host side, no GPU): bitwise round trip,
rejection of foreign or inconsistent files, and a writer killed while saving.

The resume itself (a fresh handle continuing bit for bit) is ``test_checkpoint_resume_bitwise``
in the GPU tests."""
import os
import signal
import subprocess
import sys
import time

import numpy as np
import pytest

from transformer_lm_step_amd import checkpoint as ck

CFG = {"n_layer": 2, "n_head": 2, "n_embd": 64, "mlp_hidden": 256, "block_size": 64, "vocab_size": 256,
       "padded_vocab_size": 256}


def _arrays(n, seed):
    rng = np.random.default_rng(seed)
    p = rng.standard_normal(n, dtype=np.float32)
    m = rng.standard_normal(n, dtype=np.float32) * np.float32(1e-3)
    v = np.abs(rng.standard_normal(n, dtype=np.float32)) * np.float32(1e-6)
    return p, m, v


def test_round_trip_bitwise(tmp_path):
    p, m, v = _arrays(10001, 0)
    p[3] = np.float32(-0.0)
    p[7] = np.float32(1e-45)   # a subnormal survives as is
    path = str(tmp_path / "s.npz")
    ck.write_state(path, p, m, v, adam_t=17, data_pos=35, config=CFG, extra={"val_loss": 3.25})
    st = ck.read_state(path)
    assert st["adam_t"] == 17 and st["data_pos"] == 35 and st["config"] == CFG
    assert st["extra"] == {"val_loss": 3.25}
    for k, a in (("params", p), ("m", m), ("v", v)):
        assert st[k].dtype == np.float32
        assert st[k].tobytes() == a.tobytes(), k
    assert [f for f in os.listdir(tmp_path) if f.endswith(".tmp")] == []


def test_overwrite_keeps_one_complete_file(tmp_path):
    path = str(tmp_path / "s.npz")
    for i in range(3):
        p, m, v = _arrays(257, i)
        ck.write_state(path, p, m, v, adam_t=i, data_pos=2 * i, config=CFG)
    st = ck.read_state(path)
    p, m, v = _arrays(257, 2)
    assert st["adam_t"] == 2 and st["params"].tobytes() == p.tobytes()


def test_rejects_bad_inputs_and_files(tmp_path):
    p, m, v = _arrays(100, 1)
    with pytest.raises(ValueError):
        ck.write_state(str(tmp_path / "a.npz"), p, m[:99], v, 1, 0, CFG)
    with pytest.raises(ValueError):
        ck.write_state(str(tmp_path / "a.npz"), p, m, v, -1, 0, CFG)
    # an npz without the format tag
    path = str(tmp_path / "foreign.npz")
    np.savez(path, params=p, m=m, v=v, meta=np.frombuffer(b'{"format": "other"}', dtype=np.uint8))
    with pytest.raises(ValueError):
        ck.read_state(path)
    # arrays that do not match the recorded parameter count
    good = str(tmp_path / "good.npz")
    ck.write_state(good, p, m, v, 1, 0, CFG)
    with np.load(good, allow_pickle=False) as z:
        meta = bytes(z["meta"])
    bad = str(tmp_path / "bad.npz")
    np.savez(bad, params=p, m=m[:50], v=v, meta=np.frombuffer(meta, dtype=np.uint8))
    with pytest.raises(ValueError):
        ck.read_state(bad)


_WRITER = r"""
import sys, numpy as np
sys.path.insert(0, {root!r})
from transformer_lm_step_amd import checkpoint as ck
path, n = sys.argv[1], 1 << 20
cfg = {cfg!r}
i = 0
while True:
    a = np.full(n, np.float32(i), dtype=np.float32)
    ck.write_state(path, a, a * np.float32(2), a * np.float32(3), adam_t=i, data_pos=10 * i, config=cfg)
    print(i, flush=True)
    i += 1
"""


def test_writer_killed_while_saving(tmp_path):
    """A process that keeps overwriting its checkpoint (4 MiB arrays) is killed with SIGKILL at
    an arbitrary moment after its first complete save: the file still reads as one complete,
    self-consistent state."""
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    path = str(tmp_path / "run.npz")
    code = _WRITER.format(root=root, cfg=CFG)
    for delay in (0.05, 0.3, 0.7):
        proc = subprocess.Popen([sys.executable, "-c", code, path], stdout=subprocess.PIPE, text=True)
        try:
            first = proc.stdout.readline()
            assert first.strip() == "0"
            time.sleep(delay)
            proc.send_signal(signal.SIGKILL)
            proc.wait(timeout=30)
        finally:
            if proc.poll() is None:
                proc.kill()
                proc.wait()
        st = ck.read_state(path)
        i = st["adam_t"]
        assert st["data_pos"] == 10 * i
        assert np.all(st["params"] == np.float32(i))
        assert np.all(st["m"] == np.float32(2 * i)) and np.all(st["v"] == np.float32(3 * i))
