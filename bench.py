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

roofline: the gate/up + SwiGLU kernel (the largest weight stream of the step),
timed per launch with HIP events recorded on the stream it runs on, in a
second timed pass that runs the layer stage by stage; its algorithmic bytes
are the touched experts' gate/up codes + scales.

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
def build_layer(w, layer, device, mode="A16", gen_buffers=None):
    """One seeded layer on the GPU: (Experts, router bf16 [E, H], bias fp32 [E] or None).

    Expert weights are drawn on the GPU by the seeded generator (bit-identical
    to its host build) as fp32 and NVFP4-packed by the library.
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
    ws = torch.empty(moe.layer_workspace_bytes(mode, T, k, E, H, I), dtype=torch.uint8, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    combos = n_layers * n_batches // np.gcd(n_layers, n_batches)

    def step(s):
        ex, router, bias = layers[s % n_layers]
        moe.moe_layer_forward(ex, mode, xs[s % n_batches], router, k, bias=bias, ws=ws, out=out)

    # untimed pass: the experts each (layer, batch) combination touches
    combo_bytes, combo_gu_bytes = [], []
    views = moe.workspace_views(ws, mode, T, k, E, H, I)
    for s in range(combos):
        step(s)
        ids = views["topk_ids"].cpu().numpy()
        n, b = touched_bytes(w, ids)
        combo_bytes.append(b)
        combo_gu_bytes.append(n * (2 * I * H // 2 + 2 * I * H // 16))
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

    # timed pass B: stage by stage, HIP events around the gate/up kernel
    L = moe.layer_workspace_layout(mode, T, k, E, H, I)
    ffn_ws = ws[L["ffn"]:]
    ids, tw = views["topk_ids"], views["topk_w"]
    offs, sp, pr, y = views["expert_offsets"], views["sorted_pairs"], views["pair_row"], views["y_pairs"]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    stage_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(6)] for _ in range(steps)]

    route_ws = torch.empty(moe.lib().moe_route_workspace_bytes(T, E), dtype=torch.uint8, device=dev)
    out2 = torch.empty(T, H, dtype=torch.bfloat16, device=dev)

    def staged(s, e_pair=None, marks=None):
        ex, router, bias = layers[s % n_layers]
        x = xs[s % n_batches]
        if marks: marks[0].record()
        moe.moe_route_topk(x, router, k, bias, ids=ids, w=tw, ws=route_ws)
        if marks: marks[1].record()
        moe.moe_permute(ids, E, offs, sp, pr)
        if marks: marks[2].record()
        moe.nvfp4_expert_ffn_stage(ex, mode, 0, x, k, offs, sp, y, ffn_ws)
        if e_pair: e_pair[0].record()
        moe.nvfp4_expert_ffn_stage(ex, mode, 1, x, k, offs, sp, y, ffn_ws)
        if e_pair: e_pair[1].record()
        moe.nvfp4_expert_ffn_stage(ex, mode, 2, x, k, offs, sp, y, ffn_ws)
        if marks: marks[3].record()
        moe.moe_combine(y, pr, tw, out=out2)
        if marks: marks[4].record()

    for s in range(warmup):
        staged(s)
    torch.cuda.synchronize()
    for s in range(steps):
        staged(s, evs[s], stage_ev[s])
    torch.cuda.synchronize()
    gu_ms = np.array([a.elapsed_time(b) for a, b in evs])
    gu_bytes = np.array([combo_gu_bytes[s % combos] for s in range(steps)], np.float64)
    achieved = float(np.mean(gu_bytes) / (np.mean(gu_ms) * 1e-3) / 1e9)
    stage_names = ("route", "permute", "experts", "combine")
    stages = {n: float(np.mean([m[i].elapsed_time(m[i + 1]) for m in stage_ev]) * 1e3)
              for i, n in enumerate(stage_names)}
    stages["gate_up_kernel"] = float(np.mean(gu_ms) * 1e3)
    return {
        "ms_per_step": ms,
        "gbs": total_bytes / steps / (ms * 1e-3) / 1e9,
        "bytes_per_step": total_bytes / steps,
        "gu_achieved_gbs": achieved,
        "gu_bytes_per_launch": float(np.mean(gu_bytes)),
        "gu_us": float(np.mean(gu_ms) * 1e3),
        "stages_us": stages,
    }


# --------------------------------------------------------------------------- CPU baseline
def cpu_baseline(w, mode, budget_s=20.0, max_tokens=16):
    """The oracle on a bounded sample of the workload: whole-layer calls on single tokens."""
    from threadpoolctl import threadpool_limits
    from oracle import layer as OL
    wr = synth.router_weight(w, 0)
    bias = synth.zipf_bias(w)
    cache = {}

    def get(e):
        if e not in cache:
            cache[e] = OL.pack_expert(*(synth.expert_matrix(w, 0, e, m) for m in range(3)))
        return cache[e]

    done, t_total, bytes_total = 0, 0.0, 0
    with threadpool_limits(limits=1):
        for b in range(max_tokens):
            x = synth.tokens(w, batch=b)
            r = OL.route(x, wr, w.k, bias)
            for e in np.unique(r.ids):        # packing is checkpoint preparation: not timed
                get(int(e))
            t0 = time.perf_counter()
            res = OL.moe_layer(x, wr, w.k, get, mode, bias)
            t_total += time.perf_counter() - t0
            bytes_total += touched_bytes(w, res.route.ids)[1]
            done += 1
            if t_total >= budget_s:
                break
    return {"value": bytes_total / t_total / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} single-token layer calls (layer 0, token batches 0..{done - 1}), "
                      f"{t_total:.1f} s of oracle compute, expert packing excluded",
            "tokens_per_s": done * w.T / t_total}


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
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the layer runs whole on one MI355X).", file=sys.stderr)
        return 2
    w = synth.CONFIGS[args.workload]
    mode = w.modes[0]
    print(f"[bench] workload {w.index} ({w.name}) mode {mode}: building {args.layers} layers",
          file=sys.stderr, flush=True)
    r = run_gpu(w, mode, args.steps, args.warmup, args.layers, args.batches)
    print(f"[bench] gpu done: {r['ms_per_step'] * 1e3:.1f} us/step, {r['gbs']:.0f} GB/s",
          file=sys.stderr, flush=True)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, mode)
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
        "stages_us": {k2: round(v, 2) for k2, v in r["stages_us"].items()},
        "roofline": {"kernel": "k_gateup_narrow (gate/up + SwiGLU)", "bound": "hbm",
                     "achieved": round(r["gu_achieved_gbs"], 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(r["gu_achieved_gbs"] / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": int(r["gu_bytes_per_launch"]),
                     "us_per_launch": round(r["gu_us"], 2), "traffic": None},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
