"""Benchmark of the NVFP4 routed-expert layer on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 1] [--no-cpu-baseline]
                    [--no-subrecords] [--only KEY]

Prints ONE JSON line.  A step is one call of the whole layer (router logits,
softmax/top-k, permutation, expert gate/up + SwiGLU + down, combine) on one
batch of seeded synthetic tokens with every expert resident in HBM.

Headline workload: one decode-step layer, W4A16, 512 experts, top-10,
H=3072, I=512, T=1.  value = weight GB/s: algorithmic bytes per step (the
packed codes + block scales of every expert the step touches, plus the bf16
router matrix) over the measured step time.  To keep the 256 MB Infinity
Cache from serving the weights, the steps cycle over 8 independently seeded
copies of the layer and 64 seeded token batches, and the timed pass starts
after the combinations the warmup used.

roofline: the kernel that streams the expert weights, timed with HIP events on
the stream it runs on.  When the layer call is a single kernel (16-bit
activations, up to 64 token-expert pairs) that kernel is the whole step:
bytes = the step's algorithmic bytes, time = the timed pass above; the
two-launch split of the same work (routing kernel, experts + combine kernel)
is reported beside it.  Otherwise, up to 8 tokens, it is the experts + combine
kernel (bytes: the touched experts' packed codes + scales), timed as (routing +
experts) minus routing alone over back-to-back launches; for wider calls the
gate/up + SwiGLU kernel.  measured_read_gbs: torch's sum over 4 GiB, a
streaming-read reference beside the 8 TB/s specification.

subrecords: the same measurement on the verification call (T=8, 4-bit), one
layer of the 48-layer stack (T=2, 16- and 8-bit; the whole 48-layer step eager
and as a replayed graph), the 1024-token prefill chunk in each activation mode
(gate/up and down kernels timed apart, MFMA TFLOP/s against the f16/bf16 and
FP4 peaks), the decode layer with its BF16 shared expert, and the decode layer
with q4_g64_fp16 experts.

cpu_baseline: the oracle (oracle/, double precision numpy) on a bounded sample
of the headline workload, on this machine's host CPU, one core and all cores.
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
MFMA_F16_PEAK_TFLOPS = 2500.0      # dense f16 / bf16
MFMA_FP4_PEAK_TFLOPS = 10100.0     # dense fp4
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
def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def shared_on_gpu(w, layer, device):
    """The layer's seeded BF16 shared expert on the GPU (moe.SharedExpert)."""
    import torch
    import nvfp4_block_scaled_softmax_amd as moe
    gu, dn, gate = synth.shared_expert_weights(w, layer)
    b = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return moe.SharedExpert(b(gu), b(dn), b(gate))


def expert_bytes(w, fmt):
    """Packed bytes of one expert: codes + scales (NVFP4: E4M3 per 16; q4: fp16 per 64)."""
    n = 3 * w.I * w.H
    return n // 2 + (n // 16 if fmt == "nvfp4" else n // 32)


def run_gpu(w, mode, steps, warmup, n_layers, n_batches, fmt="nvfp4", shared=False, split=True, stack=False,
            layout="canonical"):
    """Timed whole-layer calls of one workload; returns a dict of measurements.

    The steps cycle over n_layers seeded layer copies and n_batches token batches;
    the timed pass starts at the combination after the last warmup one, so the
    warmup does not leave the first timed steps' weights in the Infinity Cache."""
    import torch
    import nvfp4_block_scaled_softmax_amd as moe
    dev = torch.device("cuda:0")
    E, H, I, T, k = w.E, w.H, w.I, w.T, w.k
    f32 = dict(dtype=torch.float32, device=dev)
    bufs = (torch.empty(E, 2, I * H, **f32), torch.empty(E, I * H, **f32), torch.empty(E, H * I, **f32))
    layers = [build_layer(w, l, dev, mode, bufs, fmt) for l in range(n_layers)]
    if layout == "tiled":   # the experts' scales in the tiled layout (moe_nvfp4_repack), codes shared
        layers = [(moe.moe_nvfp4_repack(ex), router, bias) for ex, router, bias in layers]
        torch.cuda.synchronize()
    shareds = [shared_on_gpu(w, l, dev) for l in range(n_layers)] if shared else None
    del bufs
    torch.cuda.empty_cache()
    xs = [token_batch(w, b, dev) for b in range(n_batches)]
    if shared:
        ws = torch.zeros(moe.block_workspace_bytes(mode, T, k, E, H, I, w.Is), dtype=torch.uint8, device=dev)
    else:
        ws = torch.zeros(moe.layer_workspace_bytes(mode, T, k, E, H, I), dtype=torch.uint8, device=dev)
    out = torch.empty(T, H, dtype=torch.bfloat16, device=dev)
    combos = n_layers * n_batches // np.gcd(n_layers, n_batches)
    eb = expert_bytes(w, fmt)
    sh_bytes = (3 * w.Is * H + H) * 2 if shared else 0

    def step(s):
        ex, router, bias = layers[s % n_layers]
        if shared:
            moe.moe_block_forward(ex, shareds[s % n_layers], mode, xs[s % n_batches], router, k, bias=bias, ws=ws,
                                  out=out)
        else:
            moe.moe_layer_forward(ex, mode, xs[s % n_batches], router, k, bias=bias, ws=ws, out=out)

    # untimed pass: the experts each (layer, batch) combination touches
    combo_bytes, combo_n, combo_pairs = [], [], []
    views = moe.workspace_views(ws, mode, T, k, E, H, I)
    for s in range(combos):
        step(s)
        ids = views["topk_ids"].cpu().numpy()
        n = len(np.unique(ids))
        combo_bytes.append(n * eb + E * H * 2 + sh_bytes)
        combo_n.append(n)
    moe.moe_layer_status(ws)
    for s in range(warmup):
        step(s)
    torch.cuda.synchronize()
    ev = _events(2)
    ev[0].record()
    for s in range(warmup, warmup + steps):
        step(s)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / steps
    total_bytes = sum(combo_bytes[s % combos] for s in range(warmup, warmup + steps))
    n_e = float(np.mean([combo_n[s % combos] for s in range(warmup, warmup + steps)]))
    launches = moe.block_launches(mode, T, k, H, I, w.Is) if shared else moe.layer_launches(mode, T, k, H, I)
    if fmt == "q4" and launches == 1:
        launches = 2   # q4_g64_fp16 experts take the two-launch form
    rec = {"ms_per_step": ms, "bytes_per_step": total_bytes / steps, "gbs": total_bytes / steps / (ms * 1e-3) / 1e9,
           "experts_per_step": n_e, "launches": launches}
    if shared:
        rec["shared_bytes"] = sh_bytes
    fused = bool(moe.lib().moe_layer_is_fused(T, H, I))
    if split and fused and not shared:
        # Up to 8 tokens the layer runs fused; its two-launch form (routing, experts
        # + combine) is timed as (stage 0 + stage 1) minus stage 0 alone.
        def half(s, stages):
            ex, router, bias = layers[s % n_layers]
            for st_ in stages:
                moe.moe_layer_forward_stage(ex, mode, st_, xs[s % n_batches], router, k, bias, None, ws, out)
        for s in range(warmup):
            half(s, (0, 1))
        torch.cuda.synchronize()
        ev = _events(4)
        ev[0].record()
        for s in range(warmup, warmup + steps):
            half(s, (0,))
        ev[1].record()
        torch.cuda.synchronize()
        ev[2].record()
        for s in range(warmup, warmup + steps):
            half(s, (0, 1))
        ev[3].record()
        torch.cuda.synchronize()
        route_us = ev[0].elapsed_time(ev[1]) / steps * 1e3
        kern_us = ev[2].elapsed_time(ev[3]) / steps * 1e3 - route_us
        rec["two_launch"] = {"routing_kernel_us": route_us, "experts_kernel_us": kern_us,
                             "experts_kernel_bytes": n_e * eb,
                             "experts_kernel_gbs": n_e * eb / (kern_us * 1e-6) / 1e9}
    elif split and not fused:
        # wider calls: gate/up + SwiGLU and down, each launched back to back on the
        # permutations of the layer copies (stage 1, then stage 2)
        per_layer = []
        for l in range(n_layers):
            step(l)
            v = moe.workspace_views(ws, mode, T, k, E, H, I)
            fws = torch.empty(moe.ffn_workspace_bytes(mode, T, k, H, I), dtype=torch.uint8, device=dev)
            moe.nvfp4_expert_ffn_stage(layers[l][0], mode, 0, xs[l % n_batches], k, v["expert_offsets"],
                                       v["sorted_pairs"], v["y_pairs"], fws)
            ids = v["topk_ids"].cpu().numpy()
            per_layer.append((v["expert_offsets"].clone(), v["sorted_pairs"].clone(), fws, len(np.unique(ids)),
                              int((ids >= 0).sum())))
        y = torch.empty(T * k, H, dtype=torch.float32, device=dev)

        def stage(s, st_):
            l = s % n_layers
            off, sp, fws, _, _ = per_layer[l]
            moe.nvfp4_expert_ffn_stage(layers[l][0], mode, st_, xs[l % n_batches], k, off, sp, y, fws)

        times = {}
        for st_ in (1, 2):
            for s in range(warmup):
                stage(s, st_)
            torch.cuda.synchronize()
            ev = _events(2)
            ev[0].record()
            for s in range(warmup, warmup + steps):
                stage(s, st_)
            ev[1].record()
            torch.cuda.synchronize()
            times[st_] = ev[0].elapsed_time(ev[1]) / steps * 1e3
        n_gu = float(np.mean([per_layer[s % n_layers][3] for s in range(warmup, warmup + steps)]))
        pairs = float(np.mean([per_layer[s % n_layers][4] for s in range(warmup, warmup + steps)]))
        gu_b = 2 * I * H // 2 + (2 * I * H // 16 if fmt == "nvfp4" else 2 * I * H // 32)
        dn_b = eb - gu_b
        flops = pairs * 6.0 * I * H
        rec["expert_kernels"] = {"gateup_us": times[1], "down_us": times[2],
                                 "gateup_bytes": n_gu * gu_b, "down_bytes": n_gu * dn_b,
                                 "gateup_gbs": n_gu * gu_b / (times[1] * 1e-6) / 1e9,
                                 "down_gbs": n_gu * dn_b / (times[2] * 1e-6) / 1e9,
                                 "flop": flops,
                                 "mfma_tflops": flops / ((times[1] + times[2]) * 1e-6) / 1e12}
    if stack:
        rec["stack_step"] = stack_step(w, mode, layers, xs[0], ws, steps=max(5, steps // 20), warmup=2)
    del layers, shareds, xs, ws
    torch.cuda.empty_cache()
    return rec


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


def _cpu_facts():
    model = None
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return {"cpu_model": model, "nproc": affinity}


def cpu_baseline(w, mode, budget_s=20.0, max_tokens=12):
    """The oracle on a bounded sample of the workload: whole-layer calls on single
    tokens of layer 0, on one core and on all cores (BLAS threads).  Runs before
    the GPU is touched; the experts the sample needs are packed first (checkpoint
    preparation, not timed) in a process pool."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    from oracle import layer as OL
    wr = synth.router_weight(w, 0)
    bias = synth.zipf_bias(w)
    xs = [synth.tokens(w, batch=b) for b in range(max_tokens)]
    need = sorted(set(int(e) for x in xs for e in OL.route(x, wr, w.k, bias).ids.reshape(-1)))
    facts = _cpu_facts()
    # spawn, not fork: the host generator's OpenMP pool is already running here
    with mp.get_context("spawn").Pool(max(1, min(8, (facts["nproc"] or 2) - 1))) as pool:
        cache = dict(pool.map(_pack_one, [(w, e) for e in need]))

    def timed(threads):
        done, t_total, bytes_total = 0, 0.0, 0
        with threadpool_limits(limits=threads):
            for x in xs:
                t0 = time.perf_counter()
                res = OL.moe_layer(x, wr, w.k, cache.__getitem__, mode, bias)
                t_total += time.perf_counter() - t0
                bytes_total += touched_bytes(w, res.route.ids)[1]
                done += 1
                if t_total >= budget_s / 2:
                    break
        return done, t_total, bytes_total

    d1, t1, b1 = timed(1)
    dn, tn, bn = timed(facts["nproc"])
    return {"value": b1 / t1 / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{d1} single-token layer calls (layer 0, token batches 0..{d1 - 1}), "
                      f"{t1:.1f} s of oracle compute on one core, expert packing excluded",
            "tokens_per_s": d1 * w.T / t1,
            "all_cores": {"value": bn / tn / 1e9, "unit": "GB/s", "cores": facts["nproc"],
                          "tokens_per_s": dn * w.T / tn, "sample": f"{dn} calls, {tn:.1f} s"},
            **facts}


def achievable_read_gbs(gib=4, reps=10):
    """A measured streaming-read reference beside the 8 TB/s specification: torch's
    row sums of a 4 GiB fp32 tensor viewed as rows of 64 Ki values (a library
    reduction kernel that reads every byte once; of torch's reductions, the
    fastest reader measured on MI355X), best of `reps` launches timed with HIP
    events."""
    import torch
    t = torch.ones(gib << 28, dtype=torch.float32, device="cuda:0")
    v = t.view(-1, 1 << 16)
    best = 0.0
    for _ in range(reps):
        ev = _events(2)
        ev[0].record()
        v.sum(1)
        ev[1].record()
        torch.cuda.synchronize()
        best = max(best, t.numel() * 4 / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9)
    del t
    torch.cuda.empty_cache()
    return best


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
# Sub-records of the default run: (key, workload index, mode, weight format,
# shared expert, steps, layer copies, token batches, extra).  The metric is
# quoted at T = 1 / 8 / 1024 on the decode, verification and prefill workloads;
# the 48-layer stack, the 16/8-bit prefill paths, the shared expert and the
# q4_g64_fp16 experts are measured beside them.
SUBRECORDS = (
    ("verify_w4a4_T8", 2, "A4", "nvfp4", False, 100, 8, 64, {}),
    ("stack_layer_w4a16_T2", 3, "A16", "nvfp4", False, 100, 8, 64, {"stack": True}),
    ("stack_layer_w4a8_T2", 3, "A8", "nvfp4", False, 60, 8, 64, {}),
    ("prefill_w4a4_T1024", 4, "A4", "nvfp4", False, 20, 2, 4, {}),
    ("prefill_w4a16_T1024", 4, "A16", "nvfp4", False, 20, 2, 4, {}),
    ("prefill_w4a8_T1024", 4, "A8", "nvfp4", False, 20, 2, 4, {}),
    ("prefill_w4a4_T1024_tiled", 4, "A4", "nvfp4", False, 20, 2, 4, {"layout": "tiled"}),
    ("prefill_w4a16_T1024_tiled", 4, "A16", "nvfp4", False, 20, 2, 4, {"layout": "tiled"}),
    ("decode_w4a16_T1_shared_expert", 1, "A16", "nvfp4", True, 100, 8, 64, {}),
    ("decode_q4g64_T1", 1, "A16", "q4", False, 100, 8, 64, {}),
)


def _summary(w, mode, fmt, rec):
    peak = HBM_PEAK_GBS
    out = {"workload": f"{w.name}: E={w.E} top-{w.k}, H={w.H}, I={w.I}, T={w.T}" +
                       (f", shared expert Is={w.Is}" if w.Is else "") + (", q4_g64_fp16 experts" if fmt == "q4" else ""),
           "mode": mode, "T": w.T, "us_per_step": round(rec["ms_per_step"] * 1e3, 2),
           "tokens_per_s": round(w.T / (rec["ms_per_step"] * 1e-3), 1),
           "bytes_per_step": int(rec["bytes_per_step"]), "weight_gbs": round(rec["gbs"], 1),
           "frac_hbm_peak": round(rec["gbs"] / peak, 4), "experts_per_step": round(rec["experts_per_step"], 2),
           "launches": rec["launches"]}
    if "two_launch" in rec:
        t = rec["two_launch"]
        out["experts_kernel"] = {"us": round(t["experts_kernel_us"], 2), "bytes": int(t["experts_kernel_bytes"]),
                                 "gbs": round(t["experts_kernel_gbs"], 1),
                                 "frac_hbm_peak": round(t["experts_kernel_gbs"] / peak, 4),
                                 "routing_kernel_us": round(t["routing_kernel_us"], 2)}
    if "expert_kernels" in rec:
        e = rec["expert_kernels"]
        out["expert_kernels"] = {"gateup_us": round(e["gateup_us"], 1), "down_us": round(e["down_us"], 1),
                                 "gateup_gbs": round(e["gateup_gbs"], 1), "down_gbs": round(e["down_gbs"], 1),
                                 "gateup_frac_hbm_peak": round(e["gateup_gbs"] / peak, 4),
                                 "mfma_tflops": round(e["mfma_tflops"], 1),
                                 "mfma_frac_f16_bf16_peak": round(e["mfma_tflops"] / MFMA_F16_PEAK_TFLOPS, 4),
                                 "mfma_frac_fp4_peak": round(e["mfma_tflops"] / MFMA_FP4_PEAK_TFLOPS, 4)}
    if "stack_step" in rec:
        out["stack_step"] = rec["stack_step"]
    return out


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=1, help="index of the headline workload (default 1: decode)")
    ap.add_argument("--layers", type=int, default=8, help="seeded layer copies cycled through")
    ap.add_argument("--batches", type=int, default=64, help="seeded token batches cycled through")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-subrecords", action="store_true", help="time the headline workload only")
    ap.add_argument("--only", default=None, help="time only this sub-record (by key), no headline")
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
    if args.only is not None:
        rows = [r for r in SUBRECORDS if r[0] == args.only]
        if not rows:
            print(f"no sub-record {args.only}", file=sys.stderr)
            return 2
        key, wi, mode, fmt, shared, steps, nl, nb, extra = rows[0]
        w = synth.CONFIGS[wi] if not shared else synth.with_shared_expert(synth.CONFIGS[wi])
        rec = run_gpu(w, mode, min(steps, args.steps), args.warmup, nl, nb, fmt, shared, **extra)
        summ = _summary(w, mode, fmt, rec)
        if "layout" in extra:
            summ["layout"] = extra["layout"]
        print(json.dumps({key: summ}), flush=True)
        return 0
    w = synth.CONFIGS[args.workload]
    mode = w.modes[0]
    cpu = None
    if not args.no_cpu_baseline:      # host-only, before anything touches the GPU
        print(f"[bench] cpu baseline: oracle on workload {w.index}", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, mode)
        print(f"[bench] cpu baseline done: {cpu['value']:.3f} GB/s (1 core), "
              f"{cpu['all_cores']['value']:.3f} GB/s ({cpu['all_cores']['cores']} cores)", file=sys.stderr, flush=True)
    print(f"[bench] workload {w.index} ({w.name}) mode {mode}: building {args.layers} layers",
          file=sys.stderr, flush=True)
    r = run_gpu(w, mode, args.steps, args.warmup, args.layers, args.batches)
    print(f"[bench] gpu done: {r['ms_per_step'] * 1e3:.1f} us/step, {r['gbs']:.0f} GB/s",
          file=sys.stderr, flush=True)
    if r["launches"] == 1:
        # the layer call is one kernel: the timed pass above timed exactly it
        kernel = "k_layer_decode (router, top-k, permutation, experts, combine: one launch)"
        kern_us, kern_bytes = r["ms_per_step"] * 1e3, r["bytes_per_step"]
    elif "two_launch" in r:
        kernel = "k_experts_decode (gate/up + SwiGLU + down + combine, fused)"
        kern_us, kern_bytes = r["two_launch"]["experts_kernel_us"], r["two_launch"]["experts_kernel_bytes"]
    else:
        kernel = "k_gateup_wide (gate/up + SwiGLU)"
        kern_us, kern_bytes = r["expert_kernels"]["gateup_us"], r["expert_kernels"]["gateup_bytes"]
    achieved = kern_bytes / (kern_us * 1e-6) / 1e9
    read_ref = achievable_read_gbs()
    print(f"[bench] streaming-read reference: {read_ref:.0f} GB/s", file=sys.stderr, flush=True)
    subs = {}
    if not args.no_subrecords:
        for key, wi, smode, fmt, shared, steps, nl, nb, extra in SUBRECORDS:
            sw = synth.CONFIGS[wi] if not shared else synth.with_shared_expert(synth.CONFIGS[wi])
            print(f"[bench] sub-record {key}", file=sys.stderr, flush=True)
            rec = run_gpu(sw, smode, min(steps, args.steps), min(args.warmup, 10), nl, nb, fmt, shared, **extra)
            subs[key] = _summary(sw, smode, fmt, rec)
            if "layout" in extra:
                subs[key]["layout"] = extra["layout"]
            print(f"[bench]   {subs[key]['us_per_step']} us/step, {subs[key]['weight_gbs']} GB/s",
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
        "measured_read_gbs": round(read_ref, 1),
        "pct_measured_read": round(100.0 * r["gbs"] / read_ref, 2),
        "roofline": {"kernel": kernel, "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "frac_of_measured_read": round(achieved / read_ref, 4),
                     "bytes_per_launch": int(kern_bytes),
                     "us_per_launch": round(kern_us, 2),
                     "two_launch_split": r.get("two_launch"),
                     "traffic": stored_traffic(w.index)},
        "cpu_baseline": cpu,
        "subrecords": subs,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
