"""Benchmark of the GPT-2 training step on one MI355X.

One timed step = forward with loss + backward + clip/AdamW of GPT-2 124M at B=16, T=1024 in
bf16 mode (the "gpt2_step" workload; other workloads with --workload). Inputs are seeded
synthetic Zipf(1.1) token batches already resident in device memory; parameters follow the
GPT-2 initialization. Prints one JSON line.

  value       tokens/s of the whole job (one GPU)
  mfu         tokens/s * (6N + 6*L*T*C) / dense bf16 MFMA peak (2.5166e15 FLOP/s)
  roofline    the kernel class with the largest share of step time, timed live with HIP
              events on the library's stream during the timed steps: algorithmic FLOPs or
              bytes per launch / mean launch time, against the MI355X peak
  kernels     ms per step of every kernel class (same live timing)
  cpu_baseline  the CPU oracle (float32 numpy) on one sequence of the same
              model, forward + backward + AdamW, on this host's cores
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 256 * 2.4e9 * 4096      # dense bf16 MFMA FLOP/s (2.5166 PFLOP/s)
PEAK_FP32 = 157.3e12
PEAK_HBM = 8.0e12                    # bytes/s


def model_flops_per_token(w, n_params, mode="train"):
    f = 6 * n_params + 6 * w.n_layer * w.seq_len * w.n_embd
    return f // 3 if mode in ("eval", "decode") else f     # forward only: 2N + 2LTC


def class_costs(w, B, n_params, n_decay, mode="train"):
    """Algorithmic cost of each kernel class per step: ('flop', total) or ('byte', total).
    A step is w.micro_steps forward/backward passes of B sequences and one optimizer update
    (mode "eval": one forward-only scoring pass, whose cross-entropy reads the logits once)."""
    BT, C, F, Vp, L, T, H = B * w.seq_len, w.n_embd, w.mlp_hidden, w.padded_vocab_size, w.n_layer, w.seq_len, w.n_head
    es = 2  # bf16 storage
    k = w.micro_steps
    attn_fwd = 2 * 2 * B * H * (T * (T + 1) / 2) * (C // H)            # QK^T and PV, causal half
    per_micro = {
        "gemm_qkv": ("flop", 2 * BT * 3 * C * C * L),
        "gemm_attn_proj": ("flop", 2 * BT * C * C * L),
        "gemm_fc": ("flop", 2 * BT * F * C * L),
        "gemm_mlp_proj": ("flop", 2 * BT * C * F * L),
        "gemm_lm_head": ("flop", 2 * BT * Vp * C),
        "gemm_lm_head_dx": ("flop", 2 * BT * Vp * C),
        "gemm_lm_head_dw": ("flop", 2 * BT * Vp * C),
        "gemm_dx": ("flop", 2 * BT * C * (3 * C + C + F + F) * L),
        "gemm_dw": ("flop", 2 * BT * C * (3 * C + C + F + F) * L),
        "attn_fwd": ("flop", attn_fwd * L),
        "attn_bwd": ("flop", 2.5 * attn_fwd * L),   # dV, dP, dK, dQ plus the S recompute
        # the residual stream and the LayerNorm output in the storage type, mean and rstd
        "layernorm_fwd": ("byte", (2 * L + 1) * (2 * BT * C * es + 8 * BT)),
        # x, dh and the residual gradient written (storage type), mean and rstd; all but the
        # final LayerNorm's also read the incoming residual gradient
        "layernorm_bwd": ("byte", (2 * L + 1) * (3 * BT * C * es + 8 * BT) + 2 * L * BT * C * es),
        # the per-row, per-192-column-tile softmax statistics the logits product stores; training
        # also reads the logits once and writes their gradient over them
        "cross_entropy": ("byte", BT * (Vp // 192) * 8 + (0 if mode == "eval" else 2 * BT * Vp * es)),
        "embed_fwd": ("byte", BT * C * (4 + 4 + es)),   # fp32 wte and wpe rows, x in the storage type
    }
    if mode == "decode":
        # one new position per sequence: the products stream their bf16 weights (B rows are
        # far too few to reuse them), the sampler reads each logits row in 5 passes
        return {
            "gemm_qkv": ("byte", 3 * C * C * es * L), "gemm_attn_proj": ("byte", C * C * es * L),
            "gemm_fc": ("byte", F * C * es * L), "gemm_mlp_proj": ("byte", C * F * es * L),
            "gemm_lm_head": ("byte", Vp * C * es), "topk_sample": ("byte", 5 * B * Vp * es),
        }
    if mode == "eval":
        k = 1
    costs = {c: (kind, total * k) for c, (kind, total) in per_micro.items()}
    costs["adamw"] = ("byte", n_params * 28 + n_decay * 2)
    costs["grad_norm"] = ("byte", n_params * 4)
    return costs


def cpu_baseline(w, mode="train"):
    """Time the CPU oracle (float32) on one sequence of the workload: forward, backward, AdamW
    (mode "eval": the forward with its per-position losses only)."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 0) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    import synthetic
    from oracle import gpt2_oracle as O
    params = synthetic.init_params(w)
    (x, y), = synthetic.micro_batches(w, 1, batch=1)
    m = {k: np.zeros_like(v) for k, v in params.items()}
    v = {k: np.zeros_like(a) for k, a in params.items()}
    t0 = time.perf_counter()
    steps = 0
    if mode == "decode":
        # the plain sampling loop: a forward over the whole prefix per new token, top-50 draw
        rng = np.random.default_rng(0)
        seq = list(x[0, :8])
        while True:
            z = O.forward(params, w.n_layer, w.n_head, np.array([seq]), None, want_cache=False)["logits"][0, -1]
            seq.append(O.topk_sample(z, 50, rng.random())[0])
            steps += 1
            el = time.perf_counter() - t0
            if el >= 10.0 or steps >= 32:
                break
        return {"value": steps / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
                "sample": f"{steps} tokens of 1 sequence after an 8-token prompt (a float32 numpy forward over "
                          f"the prefix per token, top-50 draw), {el:.1f} s"}
    while True:
        if mode == "eval":
            O.forward(params, w.n_layer, w.n_head, x, y, want_logits=False, want_cache=False)
        else:
            out = O.forward(params, w.n_layer, w.n_head, x, y, want_logits=False)
            g = O.backward(params, w.n_layer, w.n_head, out["cache"], 1.0)
            O.optimizer_step(params, g, m, v, steps + 1, 6e-4)
        steps += 1
        el = time.perf_counter() - t0
        if el >= 10.0 or steps >= 3:
            break
    return {"value": steps * x.size / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{steps} x (1 sequence of {x.size} tokens: "
                      + ("forward with per-position losses" if mode == "eval" else "forward + backward + AdamW")
                      + f", float32 numpy), {el:.1f} s"}


def sources_sha256():
    h = hashlib.sha256()
    d = os.path.join(ROOT, "transformer_lm_step_amd", "csrc")
    for f in sorted(os.listdir(d)):
        h.update(open(os.path.join(d, f), "rb").read())
    return h.hexdigest()


def traffic_for(kernel_class):
    """HBM bytes per launch measured by rocprofv3 counters, if taken on the current sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("source_sha256") != sources_sha256():
            return None
        c = rec["classes"].get(kernel_class)
        return c["bytes_per_launch"] if c else None
    except Exception:
        return None


# Kernel classes whose kernel can be told apart in a counter trace by name (and, for the
# kernel of the qkv product, by the smallest grid among its launches).
TRAFFIC_CLASSES = {
    "gemm_fc": ("gemm_mm_kernel<0, 0, 2,", None),
    "gemm_lm_head": ("gemm_mm_kernel<0, 0, 6,", None),
    "gemm_qkv": ("gemm_mm_kernel<0, 0, 0,", "min"),
    "gemm_lm_head_dw": ("gemm_mm_kernel<1, 1, 4,", None),
    "cross_entropy": ("cross_entropy_tiled_kernel", None),
    "adamw": ("adamw_kernel", None),
    "attn_fwd": ("attn_fwd_ts_kernel", None),
    "layernorm_fwd": ("layernorm_forward_half_kernel", None),
}
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def traffic_from(fetch_csv, write_csv, copy_bytes, out_path):
    """Turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per dispatch) into HBM bytes
    per launch for the classes above. Each counter is scaled by what it reads for the device
    copy of copy_bytes bytes (which reads and writes exactly copy_bytes)."""
    import csv
    from collections import defaultdict

    def load(path, counter):
        per = defaultdict(float)
        meta = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            d = int(r["Dispatch_Id"])
            per[d] += float(r["Counter_Value"])
            meta[d] = (r["Kernel_Name"], int(r["Grid_Size"]))
        return per, meta

    fetch, fmeta = load(fetch_csv, "FETCH_SIZE")
    write, wmeta = load(write_csv, "WRITE_SIZE")

    def copies(per, meta):
        v = [per[d] for d in per if COPY_KERNEL in meta[d][0]]
        v.sort()
        return v[-1] if v else None  # the calibration copies are the largest copy dispatches

    cf, cw = copies(fetch, fmeta), copies(write, wmeta)
    if not cf or not cw:
        raise SystemExit("no calibration copy found in the counter traces")
    sf, sw = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)

    def select(per, meta, name, grid_rule):
        ds = [d for d in per if name in meta[d][0]]
        if grid_rule and ds:
            grids = sorted({meta[d][1] for d in ds})
            g = grids[-1] if grid_rule == "max" else grids[0]
            ds = [d for d in ds if meta[d][1] == g]
        return ds

    classes = {}
    for cls, (name, rule) in TRAFFIC_CLASSES.items():
        fd, wd = select(fetch, fmeta, name, rule), select(write, wmeta, name, rule)
        if not fd or not wd:
            continue
        fb = sum(fetch[d] for d in fd) / len(fd) * 1024.0 * sf
        wb = sum(write[d] for d in wd) / len(wd) * 1024.0 * sw
        classes[cls] = {"bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                        "dispatches": len(fd)}
    rec = {"_about": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each "
                     "scaled by the ratio of a device copy's known bytes to what the counter read for it",
           "source_sha256": sources_sha256(), "copy_bytes": copy_bytes,
           "copy_scale": {"fetch": round(sf, 4), "write": round(sw, 4)}, "classes": classes}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2_step")
    ap.add_argument("--mode", choices=("train", "eval", "decode"), default="train",
                    help="eval: time forward-only scoring (gpt2_evaluate, the validation-loss form) of "
                         "one micro-batch instead of the training step; decode: time key/value-cache "
                         "decoding steps with top-50 sampling of the workload's B sequences after an "
                         "8-token prompt (one step = one new token per sequence)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="BYTES",
                    help="after timing, run device copies of BYTES bytes (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="build profiles/traffic.json from two rocprofv3 --pmc counter traces and exit")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.copy_bytes,
                     os.path.join(ROOT, "profiles", "traffic.json"))
        return
    if args.gpus != 1:
        print(f"bench.py: the GPT-2 step library runs on one GPU; --gpus {args.gpus} is not supported "
              "(data-parallel sharding over several GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synthetic
    import transformer_lm_step_amd as G

    w = synthetic.workload(args.workload)
    B, T = w.batch, w.seq_len
    cfg = G.make_config(w.n_layer, w.n_head, w.n_embd, w.block_size, w.vocab_size, w.padded_vocab_size, B,
                        w.dtype)
    st = G.GPT2Step(cfg, seed=w.seed_base + 1000)
    n_params = st.n_params
    n_decay = G.gpt2_decay_end(cfg)
    k = w.micro_steps
    nb = max(2, k)
    batches = synthetic.micro_batches(w, nb)
    dev = torch.device("cuda:0")
    xs = [torch.from_numpy(b[0]).to(dev) for b in batches]
    ys = [torch.from_numpy(b[1]).to(dev) for b in batches]
    d_loss = torch.zeros(k, dtype=torch.float32, device=dev)
    d_norm = torch.zeros(1, dtype=torch.float32, device=dev)
    h = st.h
    step_no = [0]

    if args.mode == "decode":
        prompt_len = 8
        n_dec = args.warmup + max(1, min(5, args.steps)) + args.steps
        if prompt_len + n_dec > T:
            raise SystemExit(f"bench.py: {prompt_len} + {n_dec} decoding positions exceed block_size {T}")
        gen = torch.Generator().manual_seed(w.seed_base + 3000)
        uni = torch.rand((n_dec, B), generator=gen).to(dev)
        toks = [xs[0][:, t].contiguous() for t in range(prompt_len)]
        G.gpt2_decode_reset(h, B)
        for t in range(prompt_len - 1):
            G.gpt2_decode_step(h, toks[t].data_ptr())
        bufs = [toks[prompt_len - 1], torch.empty(B, dtype=torch.int32, device=dev)]

    def step():
        if args.mode == "decode":
            i = step_no[0]
            cur, nxt = bufs[i % 2], bufs[(i + 1) % 2]
            G.gpt2_decode_step(h, cur.data_ptr(), None, 50, uni[i].data_ptr(), nxt.data_ptr())
            step_no[0] += 1
            return
        if args.mode == "eval":
            j = step_no[0] % nb
            G.gpt2_evaluate(h, xs[j].data_ptr(), ys[j].data_ptr(), None, B, T, None, None, d_loss.data_ptr())
            step_no[0] += 1
            return
        for i in range(k):
            j = (step_no[0] * k + i) % nb
            G.gpt2_forward(h, xs[j].data_ptr(), ys[j].data_ptr(), B, T, None, d_loss.data_ptr() + 4 * i)
            G.gpt2_backward(h, 1.0 / k, 1 if i > 0 else 0)
        step_no[0] += 1
        G.gpt2_adamw_step(h, w.lr, 0.9, 0.95, 1e-8, 0.1, 1.0, step_no[0], d_norm.data_ptr())

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # per-class live timing over a separate pass to find the dominant class
    kernels = {}
    if not args.no_kernel_timing:
        G.gpt2_timing_begin(h, None)
        for _ in range(max(1, min(5, args.steps))):
            step()
        G.gpt2_timing_end(h)
        nrep = max(1, min(5, args.steps))
        for c in G.kernel_classes():
            ms, n = G.gpt2_timing_get(h, c)
            if n:
                kernels[c] = {"ms_per_step": ms / nrep, "launches_per_step": n / nrep}
    costs = class_costs(w, B, n_params, n_decay, args.mode)
    single = [c for c in ("gemm_lm_head", "gemm_lm_head_dx", "gemm_lm_head_dw", "gemm_fc", "gemm_qkv",
                          "gemm_attn_proj", "gemm_mlp_proj", "attn_fwd", "cross_entropy", "adamw",
                          "layernorm_fwd", "topk_sample") if c in kernels and c in costs]
    dominant = max(single, key=lambda c: kernels[c]["ms_per_step"]) if single else None

    # timed region: the dominant class keeps its HIP events (on the library's stream)
    if dominant:
        G.gpt2_timing_begin(h, dominant)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    roofline = None
    if dominant:
        G.gpt2_timing_end(h)
        ms, n = G.gpt2_timing_get(h, dominant)
        kind, total = costs[dominant]
        per_launch = total / (n / args.steps) if n else 0
        avg_s = ms / 1e3 / n
        if kind == "flop":
            achieved, peak, unit, bound = per_launch / avg_s / 1e12, PEAK_BF16 / 1e12, "TFLOP/s", "mfma"
        else:
            achieved, peak, unit, bound = per_launch / avg_s / 1e9, PEAK_HBM / 1e9, "GB/s", "hbm"
        roofline = {"kernel": dominant, "bound": bound, "achieved": round(achieved, 2), "peak": round(peak, 1),
                    "unit": unit, "frac": round(achieved / peak, 4), "traffic": traffic_for(dominant),
                    "launch_ms": round(ms / n, 4), "per_launch": per_launch,
                    "per_launch_unit": "FLOP" if kind == "flop" else "bytes"}
    if args.mode != "train":
        k = 1
    loss = float(d_loss[:k].sum().item()) / k if args.mode != "decode" else None
    ms_step = el / args.steps * 1e3
    tokens = B * T * k if args.mode != "decode" else B
    value = tokens / (el / args.steps)
    fpt = model_flops_per_token(w, n_params, args.mode)
    mfu = value * fpt / PEAK_BF16
    for c, d in kernels.items():
        if c in costs:
            kind, total = costs[c]
            rate = total / (d["ms_per_step"] / 1e3)
            d["achieved"] = round(rate / (1e12 if kind == "flop" else 1e9), 2)
            d["unit"] = "TFLOP/s" if kind == "flop" else "GB/s"
    out = {
        "metric": ("training tokens/sec and MFU, GPT-2 124M B=16 T=1024 bf16, 1 MI355X"
                   if args.workload == "gpt2_step" else f"training tokens/sec, {args.workload}")
        if args.mode == "train" else (f"evaluation tokens/sec (forward-only scoring), {args.workload}"
                                      if args.mode == "eval" else
                                      f"decoded tokens/sec (key/value cache, top-50 sampling), {args.workload}"),
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32", "data": "synthetic",
        "config": {"workload": f"{w.name}: GPT-2 L={w.n_layer} H={w.n_head} C={w.n_embd}, B={B}, T={T}, "
                               f"vocab {w.vocab_size} padded to {w.padded_vocab_size}, "
                               + (f"{k} micro-step(s) + AdamW per step" if args.mode == "train"
                                  else "one forward-only scoring pass (no backward, no update) per step"
                                  if args.mode == "eval" else
                                  f"one decoding step (one new token for each of B sequences, positions "
                                  f"8..{8 + args.warmup + max(1, min(5, args.steps)) + args.steps - 1}) per step"),
                   "global_batch": B * k, "seq_len": T, "parallelism": "single GPU"},
        "mfu": round(mfu, 4), "model_flops_per_token": fpt, "peak_flops": PEAK_BF16,
        "loss": round(loss, 5) if loss is not None else None, "roofline": roofline, "kernels": kernels,
        "device": torch.cuda.get_device_name(0),
        "cus": torch.cuda.get_device_properties(0).multi_processor_count,
    }
    if args.copy_calib:
        src = torch.empty(args.copy_calib, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.mode)
    print(json.dumps(out))
    st.close()


if __name__ == "__main__":
    main()
