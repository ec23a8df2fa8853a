"""Benchmark of the NVFP4 routed-expert layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 1] [--no-cpu-baseline]

Prints ONE JSON line.  A step is one call of the whole layer (router logits,
softmax/top-k, permutation, expert gate/up + SwiGLU + down, combine) on one
batch of seeded synthetic tokens with every expert resident in HBM.

Default workload: one decode-step layer, W4A16, 512 experts, top-10,
H=3072, I=512, T=1.  value = weight GB/s: algorithmic bytes per step (the
packed codes + block scales of every expert the step touches, plus the bf16
router matrix) over the measured step time.  To keep the 256 MB Infinity
Cache from serving the weights, the steps cycle over 8 independently seeded
copies of the layer and 64 seeded token batches.

roofline: the kernel that streams the expert weights, timed with HIP events on
the stream it runs on.  When the layer call is a single kernel (16-bit
activations, up to 64 token-expert pairs) that kernel is the whole step:
bytes = the step's algorithmic bytes, time = the timed pass above; the
two-launch split of the same work (routing kernel, experts + combine kernel)
is reported beside it.  Otherwise, up to 8 tokens, it is the experts + combine
kernel (bytes: the touched experts' packed codes + scales), timed in a second
pass as (routing + experts) minus routing alone over back-to-back launches;
for wider calls the gate/up + SwiGLU kernel (bytes: the touched experts'
gate/up codes + scales).

cpu_baseline: the oracle (oracle/, double precision numpy, one BLAS thread)
on a bounded sample of the same workload, on this machine's host CPU.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
METRIC = "NVFP4 MoE layer: weight GB/s (% HBM peak), tokens/s at T=1/8/1024"


# --------------------------------------------------------------------------- GPU workload
def build_layer(w, layer, device, mode="A16", gen_buffers=None, fmt="nvfp4"):
    """One seeded layer on the GPU: (Experts, router bf16 [E, H], bias fp32 [E] or None).

    Expert weights are drawn on the GPU by the seeded generator (bit-identical
    to its host build) as fp32 and packed by the library: NVFP4, or with
    fmt="q4" q4_g64_fp16.
    """
    import torch
    import nvfp4_block_scaled_softmax_amd as moe
    E, H, I = w.E, w.H, w.I
    f32 = dict(dtype=torch.float32, device=device)
    if gen_buffers is None:
        gen_buffers = (torch.empty(E, 2, I * H, **f32), torch.empty(E, I * H, **f32),
                       torch.empty(E, H * I, **f32))
    gu, tmp, dn = gen_buffers
    for m in (synth.MAT_GATE, synth.MAT_UP):
        synth.gpu_normal_(tmp, w.seed, synth.TAG_EXPERT, layer=layer, expert=0, matrix=m,
                          sigma=synth.SIGMA_W, n_expert=E)
        gu[:, m].copy_(tmp)
    synth.gpu_normal_(dn, w.seed, synth.TAG_EXPERT, layer=layer, expert=0, matrix=synth.MAT_DOWN,
                      sigma=synth.SIGMA_W, n_expert=E)
    gu_in = dn_in = None
    if mode == "A4":
        g, d = synth.load_input_scales(w)
        gu_in = torch.from_numpy(g).to(device)
        dn_in = torch.from_numpy(d).to(device)
    if fmt == "q4":
        ex = moe.pack_experts_q4(gu.view(E, 2 * I, H), dn.view(E, H, I))
    else:
        ex = moe.pack_experts(gu.view(E, 2 * I, H), dn.view(E, H, I), gu_in, dn_in)
    router = torch.empty(E, H, dtype=torch.bfloat16, device=device)
    synth.gpu_normal_(router, w.seed, synth.TAG_ROUTER, layer=layer, sigma=synth.SIGMA_W)
    bias = synth.zipf_bias(w)
    bias = None if bias is None else torch.from_numpy(bias).to(device)
    return ex, router, bias


def token_batch(w, batch, device, T=None):
    import torch
    x = synth.tokens(w, batch=batch, T=T)
    return torch.from_numpy(x.view(np.int16)).to(device).view(torch.bfloat16)


def touched_bytes(w, ids):
    """Algorithmic bytes of one layer call: packed bytes of each distinct expert + router."""
    n = len(np.unique(ids))
    return n, n * w.expert_bytes + w.E * w.H * 2


# --------------------------------------------------------------------------- timing
def run_gpu(w, mode, steps, warmup, n_layers, n_batches):
    import torch
    import nvfp4_block_scaled_softmax_amd as moe
    dev = torch.device("cuda:0")
    E, H, I, T, k = w.E, w.H, w.I, w.T, w.k
    f32 = dict(dtype=torch.float32, device=dev)
    bufs = (torch.empty(E, 2, I * H, **f32), torch.empty(E, I * H, **f32), torch.empty(E, H * I, **f32))
    layers = [build_layer(w, l, dev, mode, bufs) for l in range(n_layers)]
    del bufs
    torch.cuda.empty_cache()
    xs = [token_batch(w, b, dev) for b in range(n_batches)]
    ws = torch.zeros(moe.layer_workspace_bytes(mode, T, k, E, H, I), dtype=torch.uint8, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    combos = n_layers * n_batches // np.gcd(n_layers, n_batches)

    def step(s):
        ex, router, bias = layers[s % n_layers]
        moe.moe_layer_forward(ex, mode, xs[s % n_batches], router, k, bias=bias, ws=ws, out=out)

    # untimed pass: the experts each (layer, batch) combination touches
    combo_bytes, combo_n = [], []
    views = moe.workspace_views(ws, mode, T, k, E, H, I)
    for s in range(combos):
        step(s)
        ids = views["topk_ids"].cpu().numpy()
        n, b = touched_bytes(w, ids)
        combo_bytes.append(b)
        combo_n.append(n)
    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    # timed pass A: whole-layer calls back to back
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for s in range(steps):
        step(s)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / steps
    total_bytes = sum(combo_bytes[s % combos] for s in range(steps))

    # timed pass B: the step's largest weight stream alone, launched back to back
    # (the queue stays full, so the HIP events bracket GPU time only), cycling
    # over the layer copies so its weights come from HBM.
    fused = bool(moe.lib().moe_layer_is_fused(T, H, I))
    launches = moe.layer_launches(mode, T, k, H, I)
    gu_bytes_e = 2 * I * H // 2 + 2 * I * H // 16        # one expert's gate/up codes + scales
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    split = None
    if fused:
        # Up to 8 tokens the layer is two kernels: routing (stage 0) and the experts
        # with the combine (stage 1, the weight stream).  Stage 1 needs its stage 0
        # first, so it is timed as (stage 0 + stage 1) minus stage 0 alone.
        def half(s, stages):
            ex, router, bias = layers[s % n_layers]
            for st_ in stages:
                moe.moe_layer_forward_stage(ex, mode, st_, xs[s % n_batches], router, k, bias, None, ws, out)
        for s in range(warmup):
            half(s, (0, 1))
        torch.cuda.synchronize()
        ev[0].record()
        for s in range(steps):
            half(s, (0,))
        ev[1].record()
        torch.cuda.synchronize()
        ev[2].record()
        for s in range(steps):
            half(s, (0, 1))
        ev[3].record()
        torch.cuda.synchronize()
        route_us = ev[0].elapsed_time(ev[1]) / steps * 1e3
        kern_us = ev[2].elapsed_time(ev[3]) / steps * 1e3 - route_us
        n_e = float(np.mean([combo_n[s % combos] for s in range(steps)]))
        kern_bytes = n_e * w.expert_bytes
        kernel = "k_experts_decode (gate/up + SwiGLU + down + combine, fused)"
        if launches == 1:
            # moe_layer_forward is one kernel here: pass A timed exactly that kernel,
            # back to back.  The two-launch split of the same work is kept as context.
            split = {"routing_kernel_us": round(route_us, 2), "experts_kernel_us": round(kern_us, 2),
                     "experts_kernel_gbs": round(kern_bytes / (kern_us * 1e-6) / 1e9, 1)}
            kern_us = ms * 1e3
            kern_bytes = total_bytes / steps
            kernel = "k_layer_decode (router, top-k, permutation, experts, combine: one launch)"
    else:
        L = moe.layer_workspace_layout(mode, T, k, E, H, I)
        per_layer = []
        for l in range(n_layers):
            step(l)                            # layer l with token batch l
            v = moe.workspace_views(ws, mode, T, k, E, H, I)
            fws = torch.empty(moe.ffn_workspace_bytes(mode, T, k, H, I), dtype=torch.uint8, device=dev)
            moe.nvfp4_expert_ffn_stage(layers[l][0], mode, 0, xs[l % n_batches], k, v["expert_offsets"],
                                       v["sorted_pairs"], v["y_pairs"], fws)
            n_e = len(np.unique(v["topk_ids"].cpu().numpy()))
            per_layer.append((v["expert_offsets"].clone(), v["sorted_pairs"].clone(), fws, n_e))
        y = torch.empty(T * k, H, dtype=torch.float32, device=dev)

        def gate_up(s):
            l = s % n_layers
            off, sp, fws, _ = per_layer[l]
            moe.nvfp4_expert_ffn_stage(layers[l][0], mode, 1, xs[l % n_batches], k, off, sp, y, fws)

        for s in range(warmup):
            gate_up(s)
        torch.cuda.synchronize()
        ev[0].record()
        for s in range(steps):
            gate_up(s)
        ev[1].record()
        torch.cuda.synchronize()
        route_us = None
        kern_us = ev[0].elapsed_time(ev[1]) / steps * 1e3
        kern_bytes = float(np.mean([per_layer[s % n_layers][3] for s in range(steps)])) * gu_bytes_e
        kernel = ("k_gateup_wide_a4" if (mode == "A4" and T > 8) else "k_gateup_narrow") + " (gate/up + SwiGLU)"
    achieved = kern_bytes / (kern_us * 1e-6) / 1e9
    stack = None
    if w.index == 3:
        stack = stack_step(w, mode, layers, xs[0], ws, steps=max(5, steps // 20), warmup=2)
    return {
        "stack_step": stack,
        "ms_per_step": ms,
        "gbs": total_bytes / steps / (ms * 1e-3) / 1e9,
        "bytes_per_step": total_bytes / steps,
        "kernel": kernel,
        "kern_achieved_gbs": achieved,
        "kern_bytes_per_launch": kern_bytes,
        "kern_us": kern_us,
        "route_us": None if split else route_us,
        "split": split,
    }


def stack_step(w, mode, layers, x0, ws, steps, warmup, depth=48):
    """One decode step through `depth` stacked layers (the layer copies cycled),
    each layer's output plus its input feeding the next, timed eagerly and as a
    replayed HIP graph of the whole step (the layer calls are single-launch
    kernels in both; each is one node of the captured graph)."""
    import torch
    import nvfp4_block_scaled_softmax_amd as moe
    bufs = [torch.empty_like(x0) for _ in range(2)]
    x_in = x0.clone()

    def calls():
        cur = x_in
        for l in range(depth):
            ex, router, bias = layers[l % len(layers)]
            moe.moe_layer_forward(ex, mode, cur, router, w.k, bias=bias, residual=cur, ws=ws, out=bufs[l % 2])
            cur = bufs[l % 2]
        return cur

    for _ in range(warmup):
        calls()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for _ in range(steps):
        calls()
    ev1.record()
    torch.cuda.synchronize()
    eager_us = ev0.elapsed_time(ev1) / steps * 1e3
    eager_out = calls().clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    ev0.record()
    for _ in range(steps):
        g.replay()
    ev1.record()
    torch.cuda.synchronize()
    graph_us = ev0.elapsed_time(ev1) / steps * 1e3
    same = bool(torch.equal(bufs[(depth - 1) % 2].view(torch.int16), eager_out.view(torch.int16)))
    return {"layers": depth, "T": w.T, "eager_us": round(eager_us, 1), "graph_us": round(graph_us, 1),
            "tokens_per_s_graph": round(w.T / (graph_us * 1e-6), 1), "graph_equals_eager": same}


# --------------------------------------------------------------------------- CPU baseline
def _pack_one(args):
    w, e = args
    from oracle import layer as OL
    return e, OL.pack_expert(*(synth.expert_matrix(w, 0, e, m) for m in range(3)))


def cpu_baseline(w, mode, budget_s=20.0, max_tokens=12):
    """The oracle on a bounded sample of the workload: whole-layer calls on single
    tokens of layer 0.  Runs before the GPU is touched; the experts the sample
    needs are packed first (checkpoint preparation, not timed) in a process pool."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    from oracle import layer as OL
    wr = synth.router_weight(w, 0)
    bias = synth.zipf_bias(w)
    xs = [synth.tokens(w, batch=b) for b in range(max_tokens)]
    need = sorted(set(int(e) for x in xs for e in OL.route(x, wr, w.k, bias).ids.reshape(-1)))
    # spawn, not fork: the host generator's OpenMP pool is already running here
    with mp.get_context("spawn").Pool(max(1, min(8, (os.cpu_count() or 2) - 1))) as pool:
        cache = dict(pool.map(_pack_one, [(w, e) for e in need]))
    done, t_total, bytes_total = 0, 0.0, 0
    with threadpool_limits(limits=1):
        for x in xs:
            t0 = time.perf_counter()
            res = OL.moe_layer(x, wr, w.k, cache.__getitem__, mode, bias)
            t_total += time.perf_counter() - t0
            bytes_total += touched_bytes(w, res.route.ids)[1]
            done += 1
            if t_total >= budget_s:
                break
    return {"value": bytes_total / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} single-token layer calls (layer 0, token batches 0..{done - 1}), "
                      f"{t_total:.1f} s of oracle compute on one core, expert packing excluded",
            "tokens_per_s": done * w.T / t_total}


# --------------------------------------------------------------------------- traffic
COPY_BYTES = 256 << 20


def copy_calibration():
    """Five device-to-device copies of COPY_BYTES (torch's copy kernel): each reads
    and writes exactly COPY_BYTES, the reference for the HBM byte counters."""
    import torch
    a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "copies": 5}), flush=True)
    return 0


def kernel_sources_digest():
    """SHA-1 over the library's kernel sources (csrc/*.hip, *.hpp, sorted): a stored
    counter measurement is reported only while the kernels it measured are unchanged."""
    import glob
    import hashlib
    h = hashlib.sha1()
    csrc = os.path.join(ROOT, "nvfp4_block_scaled_softmax_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.hpp"))):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def stored_traffic(workload_index):
    """HBM bytes per launch of the roofline kernel from profiles/traffic_w<i>.json
    (written from rocprofv3 FETCH_SIZE and WRITE_SIZE runs, scaled by the copy
    calibration), or None when absent or taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_w{workload_index}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("sources_sha1") != kernel_sources_digest():
        return None
    return t.get("bytes_per_launch")


# --------------------------------------------------------------------------- main
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1, help="index of the workload (default 1: decode)")
    ap.add_argument("--layers", type=int, default=8, help="seeded layer copies cycled through")
    ap.add_argument("--batches", type=int, default=64, help="seeded token batches cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 256 MiB device copy (x5): the known-size reference that "
                         "scales the FETCH_SIZE / WRITE_SIZE counters of the traffic measurement")
    args = ap.parse_args(argv)
    if args.copy_calibration:
        return copy_calibration()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer runs whole on one MI355X).", file=sys.stderr)
        return 2
    w = synth.CONFIGS[args.workload]
    mode = w.modes[0]
    cpu = None
    if not args.no_cpu_baseline:      # host-only, before anything touches the GPU
        print(f"[bench] cpu baseline: oracle on workload {w.index}", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, mode)
        print(f"[bench] cpu baseline done: {cpu['value']:.3f} GB/s", file=sys.stderr, flush=True)
    print(f"[bench] workload {w.index} ({w.name}) mode {mode}: building {args.layers} layers",
          file=sys.stderr, flush=True)
    r = run_gpu(w, mode, args.steps, args.warmup, args.layers, args.batches)
    print(f"[bench] gpu done: {r['ms_per_step'] * 1e3:.1f} us/step, {r['gbs']:.0f} GB/s",
          file=sys.stderr, flush=True)
    line = {
        "metric": METRIC,
        "value": round(r["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e2m1xbf16" if mode == "A16" else ("e2m1xe4m3" if mode == "A8" else "e2m1xe2m1"),
        "data": "synthetic",
        "config": {"workload": f"{w.name}: one routed-expert layer, E={w.E} top-{w.k}, "
                               f"H={w.H}, I={w.I}, T={w.T}",
                   "E": w.E, "k": w.k, "H": w.H, "I": w.I, "T": w.T, "mode": mode,
                   "layer_copies": args.layers, "token_batches": args.batches},
        "tokens_per_s": round(w.T / (r["ms_per_step"] * 1e-3), 1),
        "pct_hbm_peak": round(100.0 * r["gbs"] / HBM_PEAK_GBS, 2),
        "bytes_per_step": int(r["bytes_per_step"]),
        "roofline": {"kernel": r["kernel"], "bound": "hbm",
                     "achieved": round(r["kern_achieved_gbs"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(r["kern_achieved_gbs"] / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": int(r["kern_bytes_per_launch"]),
                     "us_per_launch": round(r["kern_us"], 2),
                     "routing_us_per_launch": None if r["route_us"] is None else round(r["route_us"], 2),
                     "two_launch_split": r["split"],
                     "traffic": stored_traffic(w.index)},
        "cpu_baseline": cpu,
    }
    if r["stack_step"] is not None:
        line["stack_step"] = r["stack_step"]
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
