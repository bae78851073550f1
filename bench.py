"""Benchmark of the GPT-2 training step on one MI355X.

One timed step = forward with loss + backward + clip/AdamW of GPT-2 124M at B=16, T=1024 in
bf16 mode (the "gpt2_step" workload; other workloads with --workload). bf16 mode is the
autocast recipe: bf16 product and attention operands, an fp32 residual stream and gradient
(--dtype bf16_res16 times the variant that stores those in bf16 too; the default run also
times it briefly and reports it under "variant_bf16_res16", never as `value`). Inputs are
seeded synthetic Zipf(1.1) token batches already resident in device memory; parameters
follow the GPT-2 initialization. Prints one JSON line.

  value       tokens/s of the whole job (one GPU): training steps timed as replays of the
              whole step captured once in a HIP graph (schedule on the device, forward,
              backward, AdamW with device-side scalars; the next batch copied in before each
              replay; --mode eval: one forward-only scoring pass captured the same way), or as
              separate launches with --no-graph or where capture fails
  timing      which of the two `value` is, and the separate-launch figure ("eager")
  mfu         tokens/s * (6N + 6*L*T*C) / dense bf16 MFMA peak (2.5166e15 FLOP/s)
  roofline    the kernel class with the largest share of step time (every class, single- or
              multi-shape), timed live with HIP events on the library's stream during the
              eager timed steps (a product that is one kernel records them at its own start
              and end): algorithmic FLOPs or bytes per launch (the class's total per step over
              its launches per step) / mean launch time, against the MI355X peak
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


def class_costs(w, B, n_params, n_decay, mode="train", res16=False):
    """Algorithmic cost of each kernel class per step: ('flop', total) or ('byte', total).
    A step is w.micro_steps forward/backward passes of B sequences and one optimizer update
    (mode "eval": one forward-only scoring pass, whose cross-entropy reads the logits once).
    res16: the residual stream and its gradient are bf16 (else fp32, with a bf16 copy of the
    gradient written for the products)."""
    BT, C, F, Vp, L, T, H = B * w.seq_len, w.n_embd, w.mlp_hidden, w.padded_vocab_size, w.n_layer, w.seq_len, w.n_head
    es = 2  # bf16 storage of operands and activations
    er = 2 if res16 else 4  # residual stream and its gradient
    cp = 0 if res16 else 2  # bf16 copy of an fp32 residual gradient
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
        # the first LayerNorm reads the residual stream and writes its bf16 output; the other 2L
        # add the projection output (bf16) to the stream first: the old stream and y read, the
        # new stream and the bf16 output written; mean and rstd
        "layernorm_fwd": ("byte", BT * C * (er + es) + 2 * L * BT * C * (2 * er + 2 * es) + (2 * L + 1) * 8 * BT),
        # dh (bf16) and x read, the residual gradient (and its bf16 copy) written, mean and rstd;
        # all but the final LayerNorm's also read the incoming residual gradient
        "layernorm_bwd": ("byte", (2 * L + 1) * (BT * C * (es + 2 * er + cp) + 8 * BT) + 2 * L * BT * C * er),
        # the per-row, per-192-column-tile softmax statistics the logits product stores; training
        # also reads the logits once and writes their gradient over them
        "cross_entropy": ("byte", BT * (Vp // 192) * 8 + (0 if mode == "eval" else 2 * BT * Vp * es)),
        "embed_fwd": ("byte", BT * C * (4 + 4 + er)),   # fp32 wte and wpe rows, x in the residual type
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


def traffic_for(kernel_class, workload, mode):
    """HBM bytes per launch measured by rocprofv3 counters, if taken on the current sources and
    on this workload (the counters are taken on the default training workload)."""
    if mode != "train":
        return None
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        if rec.get("source_sha256") != sources_sha256() or rec.get("workload", "gpt2_step") != workload:
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
    "gemm_qkv": ("gemm_mm_kernel<0, 0, 0,", "max"),
    "gemm_lm_head_dw": ("gemm_mm_kernel<1, 1, 4,", None),
    "gemm_dw": ("gemm_mm_group_kernel", None),
    "cross_entropy": (("ce_rows_kernel", "ce_grad_kernel"), "sum"),   # its row pass + gradient pass
    "adamw": ("adamw_kernel", None),
    "attn_fwd": ("attn_fwd_ts_kernel", None),
    "layernorm_fwd": ("add_layernorm_forward_kernel", None),
    "layernorm_bwd": ("layernorm_backward_kernel", None),
    # the block input gradients: every GELU-derivative launch and every plain input-gradient
    # launch except the lm_head's (the first one after each cross-entropy launch)
    "gemm_dx": (("gemm_mm_kernel<0, 1, 3,", "gemm_mm_kernel<0, 1, 0,"), "dx_blocks"),
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
        if grid_rule == "dx_blocks":
            out, after_ce = [], False
            for d in sorted(per):
                k = meta[d][0]
                if "ce_grad_kernel" in k:
                    after_ce = True
                elif name[1] in k:
                    if after_ce:
                        after_ce = False   # the lm_head input gradient
                    else:
                        out.append(d)
                elif name[0] in k:
                    out.append(d)
            return out
        ds = [d for d in per if name in meta[d][0]]
        if grid_rule and ds:
            grids = sorted({meta[d][1] for d in ds})
            g = grids[-1] if grid_rule == "max" else grids[0]
            ds = [d for d in ds if meta[d][1] == g]
        return ds

    classes = {}
    for cls, (name, rule) in TRAFFIC_CLASSES.items():
        if rule == "sum":   # a class of several kernels, one launch of each per class launch
            parts = [(select(fetch, fmeta, n, None), select(write, wmeta, n, None)) for n in name]
            if not all(fd and wd for fd, wd in parts):
                continue
            fb = sum(sum(fetch[d] for d in fd) / len(fd) for fd, _ in parts) * 1024.0 * sf
            wb = sum(sum(write[d] for d in wd) / len(wd) for _, wd in parts) * 1024.0 * sw
            classes[cls] = {"bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                            "dispatches": len(parts[-1][0])}
            continue
        fd, wd = select(fetch, fmeta, name, rule), select(write, wmeta, name, rule)
        if not fd or not wd:
            continue
        fb = sum(fetch[d] for d in fd) / len(fd) * 1024.0 * sf
        wb = sum(write[d] for d in wd) / len(wd) * 1024.0 * sw
        classes[cls] = {"bytes_per_launch": round(fb + wb), "fetch_bytes": round(fb), "write_bytes": round(wb),
                        "dispatches": len(fd)}
    rec = {"_about": "HBM bytes per launch from rocprofv3 FETCH_SIZE and WRITE_SIZE (KiB per dispatch), each "
                     "scaled by the ratio of a device copy's known bytes to what the counter read for it",
           "source_sha256": sources_sha256(), "workload": "gpt2_step", "copy_bytes": copy_bytes,
           "copy_scale": {"fetch": round(sf, 4), "write": round(sw, 4)}, "classes": classes}
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def symbol_costs(w, B, n_params, n_decay):
    """Algorithmic work per step of each kernel symbol of the bf16 training step (fp32 residual
    stream) at shapes where every product takes the LDS-streamed path: (name pattern, what it
    runs, 'flop' or 'byte', total per step). Products sharing one instantiation are summed."""
    BT, C, F, Vp, L, T, H = B * w.seq_len, w.n_embd, w.mlp_hidden, w.padded_vocab_size, w.n_layer, w.seq_len, w.n_head
    af = 2 * 2 * B * H * (T * (T + 1) / 2) * (C // H) * L           # attention forward, causal half
    cc = class_costs(w, B, n_params, n_decay)
    return [
        ("gemm_mm_group_kernel", "weight gradients of every block (grouped)", "flop",
         2 * BT * C * (3 * C + C + F + F) * L),
        ("gemm_mm_kernel<0, 1, 0,", "input gradients: lm_head, c_fc, attn c_proj, c_attn", "flop",
         2 * BT * C * Vp + 2 * BT * C * (F + C + 3 * C) * L),
        ("gemm_mm_kernel<0, 1, 3,", "mlp c_proj input gradient with GELU'", "flop", 2 * BT * F * C * L),
        ("gemm_mm_kernel<0, 0, 0,", "forward: c_attn, attn c_proj, mlp c_proj", "flop", 2 * BT * C * (3 * C + C + F) * L),
        ("gemm_mm_kernel<0, 0, 2,", "forward: c_fc with GELU", "flop", 2 * BT * F * C * L),
        ("gemm_mm_kernel<0, 0, 6,", "lm_head logits + softmax statistics", "flop", 2 * BT * Vp * C),
        ("gemm_mm_kernel<1, 1, 4,", "lm_head weight gradient", "flop", 2 * BT * Vp * C),
        ("attn_fwd_ts_kernel", "attention forward", "flop", af),
        # the backward's algorithmic work (dP, dV, dK, dQ and one recompute of S: 2.5x the forward),
        # split as the two kernels divide it (each also recomputes S and dP, not counted twice)
        ("attn_bwd_dkv_ts_kernel", "attention dK, dV", "flop", 1.5 * af),
        ("attn_bwd_dq_ts_kernel", "attention dQ", "flop", 1.0 * af),
        ("add_layernorm_forward_kernel", "residual add + LayerNorm forward (2L calls)", "byte",
         2 * L * (BT * C * (2 * 4 + 2 * 2) + 8 * BT)),
        ("layernorm_forward_kernel", "first LayerNorm forward", "byte", BT * C * (4 + 2) + 8 * BT),
        ("layernorm_backward_kernel", "LayerNorm backward", "byte", cc["layernorm_bwd"][1]),
        ("ce_rows_kernel", "cross-entropy row pass (log-sum-exp, loss)", "byte", BT * (Vp // 192) * 8),
        ("ce_grad_kernel", "cross-entropy gradient over the logits", "byte", cc["cross_entropy"][1] - BT * (Vp // 192) * 8),
        ("adamw_kernel", "AdamW", "byte", cc["adamw"][1]),
        ("norm_partial_kernel", "grad norm", "byte", cc["grad_norm"][1]),
        ("embed_forward_kernel", "embedding forward", "byte", cc["embed_fwd"][1]),
    ]


def profile_table(stats_csv, steps):
    """Markdown table of a rocprofv3 --stats kernel summary of `bench.py` (default workload): per
    kernel symbol its time per step and, where its algorithmic work is known, its rate and
    fraction of the MI355X peak (FLOP: dense bf16 MFMA; bytes: HBM)."""
    import csv

    import synthetic
    w = synthetic.workload("gpt2_step")
    n_params = 124475904
    n_decay = 124354560
    costs = symbol_costs(w, w.batch, n_params, n_decay)
    rows = list(csv.DictReader(open(stats_csv)))
    total = sum(float(r["TotalDurationNs"]) for r in rows) / 1e6 / steps
    print(f"| kernel symbol | what it runs | calls | avg us | ms/step | % of kernel time | work/step | rate | "
          f"frac of peak |")
    print("|---|---|---|---|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        ms = float(r["TotalDurationNs"]) / 1e6 / steps
        if ms < 0.004:
            continue
        name = r["Name"]
        what, work, rate, frac = "", "", "", ""
        for pat, desc, kind, tot in costs:
            if pat in name:
                what = desc
                if kind == "flop":
                    rt = tot / (ms / 1e3)
                    work, rate, frac = f"{tot / 1e12:.3f} TFLOP", f"{rt / 1e12:.0f} TFLOP/s", f"{rt / PEAK_BF16:.3f}"
                else:
                    rt = tot / (ms / 1e3)
                    work, rate, frac = f"{tot / 1e9:.3f} GB", f"{rt / 1e9:.0f} GB/s", f"{rt / PEAK_HBM:.3f}"
                break
        short = name if len(name) <= 70 else name[:67] + "..."
        print(f"| `{short}` | {what} | {int(r['Calls'])} | {float(r['AverageNs']) / 1e3:.1f} | {ms:.3f} | "
              f"{100 * ms / total:.1f} | {work} | {rate} | {frac} |")
    print(f"\nTotal kernel time per step: {total:.2f} ms ({steps} steps in the trace).")


def run_workload(args, w, dtype, steps, warmup, kernel_timing=True, roofline=True, graph_steps=0):
    """Create a handle for workload w in `dtype`, run `warmup` untimed steps, a per-class timing
    pass, then `steps` timed steps (the dominant class keeps its HIP events). Returns a dict of
    the measurements; the handle is destroyed before returning."""
    import torch

    import synthetic
    import transformer_lm_step_amd as G

    B, T = w.batch, w.seq_len
    res16 = dtype == "bf16_res16"
    cfg = G.make_config(w.n_layer, w.n_head, w.n_embd, w.block_size, w.vocab_size, w.padded_vocab_size, B,
                        dtype if w.dtype == "bf16" else w.dtype)
    st = G.GPT2Step(cfg, seed=w.seed_base + 1000)
    n_params = st.n_params
    n_decay = G.gpt2_decay_end(cfg)
    k = w.micro_steps
    nb = max(8, k)   # distinct token batches cycled through (the loss then does not just memorize one)
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
        n_dec = warmup + max(1, min(5, steps)) + steps
        n_graph = graph_steps + 2 if graph_steps else 0
        if prompt_len + n_dec + n_graph > T:
            raise SystemExit(f"bench.py: {prompt_len} + {n_dec + n_graph} decoding positions exceed block_size {T}")
        gen = torch.Generator().manual_seed(w.seed_base + 3000)
        uni = torch.rand((n_dec + n_graph, B), generator=gen).to(dev)
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

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()

    # per-class live timing over a separate pass to find the dominant class
    kernels = {}
    if kernel_timing:
        nrep = max(1, min(5, steps))
        G.gpt2_timing_begin(h, None)
        for _ in range(nrep):
            step()
        G.gpt2_timing_end(h)
        for c in G.kernel_classes():
            ms, n = G.gpt2_timing_get(h, c)
            if n:
                kernels[c] = {"ms_per_step": ms / nrep, "launches_per_step": n / nrep}
    costs = class_costs(w, B, n_params, n_decay, args.mode, res16)
    cands = [c for c in kernels if c in costs]
    dominant = max(cands, key=lambda c: kernels[c]["ms_per_step"]) if (cands and roofline) else None

    # timed region: the dominant class keeps its HIP events (on the library's stream)
    if dominant:
        G.gpt2_timing_begin(h, dominant)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    roof = None
    if dominant:
        G.gpt2_timing_end(h)
        ms, n = G.gpt2_timing_get(h, dominant)
        kind, total = costs[dominant]
        per_launch = total / (n / steps) if n else 0
        avg_s = ms / 1e3 / n
        if kind == "flop":
            achieved, peak, unit, bound = per_launch / avg_s / 1e12, PEAK_BF16 / 1e12, "TFLOP/s", "mfma"
        else:
            achieved, peak, unit, bound = per_launch / avg_s / 1e9, PEAK_HBM / 1e9, "GB/s", "hbm"
        roof = {"kernel": dominant, "bound": bound, "achieved": round(achieved, 2), "peak": round(peak, 1),
                "unit": unit, "frac": round(achieved / peak, 4),
                "traffic": traffic_for(dominant, w.name, args.mode) if not res16 else None,
                "launch_ms": round(ms / n, 4), "launches_per_step": n / steps, "per_launch": per_launch,
                "per_launch_unit": "FLOP" if kind == "flop" else "bytes"}
    graph = None
    if graph_steps and args.mode == "decode":
        # one decoding step captured once in a HIP graph (gpt2_decode_step_device: the position
        # in device memory, advanced by the step; the drawn token written over the input token)
        # and replayed at the following positions, a fresh uniform row copied in before each
        try:
            orig = st.stream
            i0 = step_no[0]
            d_pos = torch.tensor([G.gpt2_decode_position(h)], dtype=torch.int32, device=dev)
            buf = bufs[i0 % 2].clone()
            u_in = uni[i0].clone()
            g = torch.cuda.CUDAGraph()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                G.gpt2_set_stream(h, torch.cuda.current_stream().cuda_stream)
                G.gpt2_decode_step_device(h, buf.data_ptr(), d_pos.data_ptr(), None, 50, u_in.data_ptr(),
                                          buf.data_ptr())
            G.gpt2_set_stream(h, orig)
            for j in range(2):
                u_in.copy_(uni[i0 + j])
                g.replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for j in range(graph_steps):
                u_in.copy_(uni[i0 + 2 + j])
                g.replay()
            torch.cuda.synchronize()
            ge = time.perf_counter() - t1
            graph = {"ms_per_step": ge / graph_steps * 1e3, "steps": graph_steps, "value": B / (ge / graph_steps),
                     "positions": [int(G.gpt2_decode_position(h)), int(d_pos.item())]}
            del g
        except Exception as e:
            G.gpt2_set_stream(h, st.stream)
            torch.cuda.synchronize()
            print(f"bench.py: HIP graph leg skipped ({e})", file=sys.stderr)
            graph = None
    if graph_steps and args.mode == "eval":
        # one forward-only scoring pass captured once in a HIP graph and replayed, the next batch
        # copied into the captured input buffers before each replay (as for the training step)
        try:
            orig = st.stream
            gx, gy = torch.empty_like(xs[0]), torch.empty_like(ys[0])
            gno = [step_no[0]]

            def load_next():
                j = gno[0] % nb
                gx.copy_(xs[j])
                gy.copy_(ys[j])
                gno[0] += 1

            g = torch.cuda.CUDAGraph()
            load_next()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                G.gpt2_set_stream(h, torch.cuda.current_stream().cuda_stream)
                G.gpt2_evaluate(h, gx.data_ptr(), gy.data_ptr(), None, B, T, None, None, d_loss.data_ptr())
            G.gpt2_set_stream(h, orig)
            for _ in range(2):
                load_next()
                g.replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for _ in range(graph_steps):
                load_next()
                g.replay()
            torch.cuda.synchronize()
            ge = time.perf_counter() - t1
            graph = {"ms_per_step": ge / graph_steps * 1e3, "steps": graph_steps, "value": B * T / (ge / graph_steps)}
            del g
        except Exception as e:
            G.gpt2_set_stream(h, st.stream)
            torch.cuda.synchronize()
            print(f"bench.py: HIP graph leg skipped ({e})", file=sys.stderr)
            graph = None
    if graph_steps and args.mode == "train":
        # The whole training step -- the learning-rate schedule advanced on the device, the k
        # micro-steps, AdamW with its scalars read from device memory -- captured once in a HIP
        # graph and replayed; before each replay the next micro-batches are copied into the
        # buffers the graph reads (device to device, ordered on the same stream).
        try:
            orig = st.stream
            gx = [torch.empty_like(xs[0]) for _ in range(k)]
            gy = [torch.empty_like(ys[0]) for _ in range(k)]
            g_step = torch.tensor([step_no[0]], dtype=torch.int32, device=dev)
            g_lr = torch.zeros(1, dtype=torch.float32, device=dev)
            g_t = torch.zeros(1, dtype=torch.int32, device=dev)
            sched = dict(max_lr=w.lr, min_lr=0.1 * w.lr, warmup_steps=10, max_steps=100000)
            gno = [step_no[0]]

            def load_next():
                for i in range(k):
                    j = (gno[0] * k + i) % nb
                    gx[i].copy_(xs[j])
                    gy[i].copy_(ys[j])
                gno[0] += 1

            def captured_step():
                G.gpt2_schedule_step_device(h, g_step.data_ptr(), g_lr.data_ptr(), g_t.data_ptr(), **sched)
                for i in range(k):
                    G.gpt2_forward(h, gx[i].data_ptr(), gy[i].data_ptr(), B, T, None, d_loss.data_ptr() + 4 * i)
                    G.gpt2_backward(h, 1.0 / k, 1 if i > 0 else 0)
                G.gpt2_adamw_step_device(h, g_lr.data_ptr(), g_t.data_ptr(), 0.9, 0.95, 1e-8, 0.1, 1.0,
                                         d_norm.data_ptr())

            g = torch.cuda.CUDAGraph()
            load_next()
            torch.cuda.synchronize()
            with torch.cuda.graph(g):
                G.gpt2_set_stream(h, torch.cuda.current_stream().cuda_stream)
                captured_step()
            G.gpt2_set_stream(h, orig)
            for _ in range(2):
                load_next()
                g.replay()
            torch.cuda.synchronize()
            t1 = time.perf_counter()
            for _ in range(graph_steps):
                load_next()
                g.replay()
            torch.cuda.synchronize()
            ge = time.perf_counter() - t1
            graph = {"ms_per_step": ge / graph_steps * 1e3, "steps": graph_steps,
                     "value": B * T * k / (ge / graph_steps)}
            del g
        except Exception as e:   # keep the eager figure if this platform cannot capture the step
            G.gpt2_set_stream(h, st.stream)
            torch.cuda.synchronize()
            print(f"bench.py: HIP graph leg skipped ({e})", file=sys.stderr)
            graph = None
    kk = k if args.mode == "train" else 1
    loss = float(d_loss[:kk].sum().item()) / kk if args.mode != "decode" else None
    tokens = B * T * kk if args.mode != "decode" else B
    for c, d in kernels.items():
        if c in costs:
            kind, total = costs[c]
            rate = total / (d["ms_per_step"] / 1e3)
            d["achieved"] = round(rate / (1e12 if kind == "flop" else 1e9), 2)
            d["unit"] = "TFLOP/s" if kind == "flop" else "GB/s"
    st.close()
    del st
    torch.cuda.synchronize()
    return {"el": el, "ms_step": el / steps * 1e3, "value": tokens / (el / steps), "loss": loss,
            "roofline": roof, "kernels": kernels, "n_params": n_params, "k": kk, "graph": graph}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="gpt2_step")
    ap.add_argument("--dtype", choices=("bf16", "bf16_res16"), default="bf16",
                    help="bf16: the autocast recipe (fp32 residual stream and gradient), timed for `value`; "
                         "bf16_res16: the variant with a bf16 residual stream and gradient")
    ap.add_argument("--no-variant", action="store_true",
                    help="skip the short timing of the bf16_res16 variant after the main measurement")
    ap.add_argument("--mode", choices=("train", "eval", "decode"), default="train",
                    help="eval: time forward-only scoring (gpt2_evaluate, the validation-loss form) of "
                         "one micro-batch instead of the training step; decode: time key/value-cache "
                         "decoding steps with top-50 sampling of the workload's B sequences after an "
                         "8-token prompt (one step = one new token per sequence)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip the short timing of the same step captured in a HIP graph and replayed")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--copy-calib", type=int, default=0, metavar="BYTES",
                    help="after timing, run device copies of BYTES bytes (counter calibration)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="build profiles/traffic.json from two rocprofv3 --pmc counter traces and exit")
    ap.add_argument("--copy-bytes", type=int, default=1 << 30)
    ap.add_argument("--profile-table", nargs=2, metavar=("STATS_CSV", "STEPS"),
                    help="print the per-symbol roofline table of a rocprofv3 --stats kernel summary of the "
                         "default benchmark (STEPS: training steps in the trace) and exit")
    args = ap.parse_args()
    if args.profile_table:
        profile_table(args.profile_table[0], int(args.profile_table[1]))
        return
    if args.traffic_from:
        traffic_from(args.traffic_from[0], args.traffic_from[1], args.copy_bytes,
                     os.path.join(ROOT, "profiles", "traffic.json"))
        return
    if args.gpus != 1:
        print(f"bench.py: the GPT-2 step library runs on one GPU; --gpus {args.gpus} is not supported "
              "(data-parallel sharding over several GPUs is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synthetic

    w = synthetic.workload(args.workload)
    B, T = w.batch, w.seq_len
    r = run_workload(args, w, args.dtype, args.steps, args.warmup, kernel_timing=not args.no_kernel_timing,
                     graph_steps=0 if args.no_graph else args.steps)
    k = r["k"]
    # `value`: the training step (or scoring pass) as a HIP-graph replay when the capture
    # succeeded (the same kernels and bytes as the eager launch sequence, without the per-launch
    # gaps), else eager
    g = r["graph"]
    value, ms_step = (g["value"], g["ms_per_step"]) if g else (r["value"], r["ms_step"])
    fpt = model_flops_per_token(w, r["n_params"], args.mode)
    mfu = value * fpt / PEAK_BF16
    dtype_name = {"bf16": "bf16", "bf16_res16": "bf16 (bf16 residual stream)"}[args.dtype] \
        if w.dtype == "bf16" else "f32"
    out = {
        "metric": ("training tokens/sec and MFU, GPT-2 124M B=16 T=1024 bf16, 1 MI355X"
                   if args.workload == "gpt2_step" else f"training tokens/sec, {args.workload}")
        if args.mode == "train" else (f"evaluation tokens/sec (forward-only scoring), {args.workload}"
                                      if args.mode == "eval" else
                                      f"decoded tokens/sec (key/value cache, top-50 sampling), {args.workload}"),
        "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": dtype_name, "data": "synthetic",
        "config": {"workload": f"{w.name}: GPT-2 L={w.n_layer} H={w.n_head} C={w.n_embd}, B={B}, T={T}, "
                               f"vocab {w.vocab_size} padded to {w.padded_vocab_size}, "
                               + (f"{k} micro-step(s) + AdamW per step" if args.mode == "train"
                                  else "one forward-only scoring pass (no backward, no update) per step"
                                  if args.mode == "eval" else
                                  "one decoding step (one new token for each of B sequences, after an "
                                  "8-token prompt; positions in `timing`) per step")
                               + ("; residual stream and its gradient fp32, product operands bf16"
                                  if args.dtype == "bf16" and w.dtype == "bf16" else
                                  "; residual stream and its gradient bf16" if w.dtype == "bf16" else ""),
                   "global_batch": B * k, "seq_len": T, "parallelism": "single GPU"},
        "mfu": round(mfu, 4), "model_flops_per_token": fpt, "peak_flops": PEAK_BF16,
        "loss": round(r["loss"], 5) if r["loss"] is not None else None, "roofline": r["roofline"],
        "kernels": r["kernels"],
        "device": torch.cuda.get_device_name(0),
        "cus": torch.cuda.get_device_properties(0).multi_processor_count,
    }
    if args.mode == "decode":
        out["timing"] = {
            "timed": "hip_graph" if g else "eager",
            "eager": {"ms_per_step": round(r["ms_step"], 3), "value": round(r["value"], 1), "steps": args.steps},
            "note": ("one decoding step (gpt2_decode_step_device: position in device memory) captured once in a "
                     "HIP graph and replayed at the following positions, the drawn tokens fed back through the "
                     "captured token buffer. `eager` times gpt2_decode_step as separate launches"
                     f" (positions 8..{8 + args.warmup + max(1, min(5, args.steps)) + args.steps - 1}; the "
                     f"graph's timed steps at positions {g['positions'][0] + 2}..{g['positions'][1] - 1})" if g else
                     "the steps as separate launches (no HIP-graph leg: --no-graph or capture unavailable)")}
    if args.mode == "eval":
        out["timing"] = {
            "timed": "hip_graph" if g else "eager",
            "eager": {"ms_per_step": round(r["ms_step"], 3), "value": round(r["value"], 1), "steps": args.steps},
            "note": ("one forward-only scoring pass captured once in a HIP graph; each timed pass copies the "
                     "next batch into the captured input buffers and replays it. `eager` times the same "
                     "passes as separate launches" if g else
                     "the pass as separate launches (no HIP-graph leg: --no-graph or capture unavailable)")}
    if args.mode == "train":
        out["timing"] = {
            "timed": "hip_graph" if g else "eager",
            "eager": {"ms_per_step": round(r["ms_step"], 3), "value": round(r["value"], 1), "steps": args.steps},
            "note": ("the whole training step (learning-rate schedule advanced on the device, the micro-steps' "
                     "forward and backward, AdamW with its scalars read from device memory) captured once in "
                     "a HIP graph; each timed step copies the next micro-batches into the captured input "
                     "buffers and replays it. `eager` times the same steps as separate launches (its per-launch "
                     "events give `roofline`)" if g else
                     "the step as separate launches (no HIP-graph leg: --no-graph or capture unavailable)")}
    if (args.mode == "train" and args.dtype == "bf16" and w.dtype == "bf16" and not args.no_variant):
        # the narrower-storage variant, timed briefly on a handle of its own (never `value`)
        v = run_workload(args, w, "bf16_res16", max(5, args.steps // 2), 2, kernel_timing=False, roofline=False)
        out["variant_bf16_res16"] = {
            "dtype": "bf16 (bf16 residual stream)", "value": round(v["value"], 1), "unit": "tokens/s",
            "ms_per_step": round(v["ms_step"], 3), "mfu": round(v["value"] * fpt / PEAK_BF16, 4),
            "steps": max(5, args.steps // 2), "warmup": 2,
            "note": "residual stream and its gradient stored in bf16: narrower than the autocast recipe; "
                    "timed as separate launches (compare with timing.eager)"}
    if args.copy_calib:
        dev = torch.device("cuda:0")
        src = torch.empty(args.copy_calib, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.mode)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
