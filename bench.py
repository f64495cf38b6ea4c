"""Benchmark: DeepSeek-V3-shape MoE-layer forward on one MI355X.

One step = the whole hot path over one batch: 1x128 quantisation of x, routing
(sigmoid affinities, bias, group limit, top-k, gates, load), permutation, routed FP8
SwiGLU experts, shared expert, combine, bias update. Inputs and weights are seeded
synthetic values already resident in HBM when the timed region starts.

Prints one JSON line. Per-stage HIP events are recorded on the launch stream inside
the timed region; the roofline entry is for the dominant kernel, the gate/up half of the
grouped FFN (routed and shared experts in one launch).
Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload v3_prefill]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/s at V3 shape (T=4096); FP8 TFLOP/s as % MFMA peak"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def ffn_algorithmic_bytes(cfg, counts):
    """Minimum HBM bytes of the two grouped-FFN launches (routed + shared experts in one
    grouped call). Per expert that received a row: its codes and 128x128 scales, read once.
    Per token: its 1x128 codes and scales, read once. Per permuted row: the 1x128 FP8
    intermediate written by gate/up and read by down, and the bf16 output row written by
    down. Returns {"gate_up": bytes, "down": bytes, "experts": n}."""
    H, I, S = cfg.hidden_size, cfg.moe_intermediate_size, cfg.num_shared_experts
    T, k = cfg.tokens, cfg.num_experts_per_tok
    rows = T * (k + S)
    experts = int((counts > 0).sum()) + S
    mat = I * H + (I // 128) * (H // 128) * 4          # one weight matrix + its scales
    act = T * (H + (H // 128) * 4)
    inter = rows * (I + (I // 128) * 4)
    return {"gate_up": experts * 2 * mat + act + inter,
            "down": experts * mat + inter + rows * H * 2,
            "experts": experts}


COUNTER_FILE = os.path.join(ROOT, "profiles", "moe_step_v3_prefill_counters.txt")
KERNEL_SOURCES = [os.path.join(ROOT, "deepseekmoe_routing_fp8_amd", "csrc", f)
                  for f in ("ffn.hip", "common.h")]


def measured_traffic():
    """HBM bytes per gate/up launch from the committed counter summary, or None once the
    kernel sources differ from the ones the counters were taken on."""
    import hashlib
    if not os.path.exists(COUNTER_FILE):
        return None
    kv = {}
    for line in open(COUNTER_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            key, val = line.split("=", 1)
            kv[key.strip()] = val.strip()
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    if kv.get("kernel_sources_sha256") != h.hexdigest():
        return None
    try:
        return int(float(kv["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def _blas_threads() -> int:
    try:
        import numpy as np
        from threadpoolctl import threadpool_info
        np.ones((64, 64)) @ np.ones((64, 64))   # loads the BLAS library
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"] or [1])
    except Exception:  # pragma: no cover
        return 1


def oracle_step_timed(x, wr, b, cfg, routed, shared):
    """The oracle's layer forward (the calls of oracle.layer_forward, in its order) with a
    wall-clock time per stage; returns (out, {stage: seconds})."""
    import numpy as np

    import oracle
    t, c = {}, time.perf_counter()

    def lap(name):
        nonlocal c
        now = time.perf_counter()
        t[name] = t.get(name, 0.0) + now - c
        c = now
    xq, xs = oracle.quantize_1x128(x)
    lap("quantize")
    r = oracle.route(x, wr, b, cfg.num_experts_per_tok, cfg.n_group, cfg.topk_group,
                     cfg.group_score_topn, cfg.routed_scaling_factor)
    lap("route")
    offsets, row_token, row_of = oracle.permute(r["idx"], cfg.num_experts)
    lap("permute")
    y_rows = np.zeros((row_token.shape[0], x.shape[1]), dtype=np.float64)
    for e in range(cfg.num_experts):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi > lo:
            y_rows[lo:hi] = oracle.expert_ffn(xq[row_token[lo:hi]], xs[row_token[lo:hi]], *routed(e))[0]
    lap("ffn_routed")
    y_shared = [oracle.expert_ffn(xq, xs, *shared(s))[0] for s in range(cfg.num_shared_experts)]
    lap("ffn_shared")
    out = oracle.combine(y_rows, row_of, r["gate"], y_shared)
    lap("combine")
    oracle.bias_update(b, r["counts"], x.shape[0], cfg.num_experts_per_tok, cfg.expert_bias_update_rate)
    lap("bias_update")
    return out, t


def cpu_baseline(cfg, n_tokens: int, full=("tiny", "reduced")):
    """Times the CPU oracle: a bounded sample of the headline workload (its first n_tokens
    tokens, all BLAS threads), then the small workloads in full at 1 BLAS thread and at
    all of them. Weight quantisation is input preparation and is not timed."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import oracle
    import synth

    def q3(w):
        return (*oracle.quantize_128x128(w[0]), *oracle.quantize_128x128(w[1]),
                *oracle.quantize_128x128(w[2]))

    def prepare(c, x):
        r = oracle.route(x, synth.router_weight(c), synth.expert_bias(c), c.num_experts_per_tok,
                         c.n_group, c.topk_group, c.group_score_topn, c.routed_scaling_factor)
        cache, sh = {}, {}
        synth.map_experts(c, lambda e, w: cache.__setitem__(e, q3(w)), sorted(set(r["idx"].ravel().tolist())))
        synth.map_experts(c, lambda s, w: sh.__setitem__(s, q3(w)), range(c.num_shared_experts), shared=True)
        return cache, sh

    affinity = len(os.sched_getaffinity(0))
    blas = _blas_threads()
    x = synth.hidden_states(cfg)[:n_tokens]
    log(f"[bench] cpu baseline: quantising the experts of {n_tokens} {cfg.name} tokens on the host")
    cache, sh = prepare(cfg, x)
    log(f"[bench] cpu baseline: oracle on {n_tokens} tokens, {blas} BLAS threads")
    t0 = time.perf_counter()
    _, st = oracle_step_timed(x, synth.router_weight(cfg), synth.expert_bias(cfg), cfg,
                              lambda e: cache[e], lambda s: sh[s])
    dt = time.perf_counter() - t0
    res = {"value": n_tokens / dt, "unit": "tokens/s", "cores": min(blas, affinity), "kind": "oracle",
           "sample": (f"the first {n_tokens} tokens of {cfg.name} through the FP64 oracle layer forward "
                      f"(1x128 quantisation, routing against all {cfg.num_experts} experts, "
                      f"{len(cache)} routed + {cfg.num_shared_experts} shared expert FFNs, combine, "
                      f"bias update), {blas} BLAS threads; weight quantisation excluded; {dt:.1f} s"),
           "seconds": round(dt, 3), "affinity_cores": affinity, "blas_threads": blas,
           "stages_s": {k: round(v, 4) for k, v in st.items()}, "full_workloads": {}}
    for name in full:
        c = synth.PRESETS[name]
        xf = synth.hidden_states(c)
        log(f"[bench] cpu baseline: {name} in full at 1 and {blas} BLAS threads")
        cache_f, sh_f = prepare(c, xf)
        runs = {}
        for label, n in (("1_thread", 1), ("all_threads", blas)):
            with threadpool_limits(limits=n, user_api="blas"):
                t0 = time.perf_counter()
                out, st = oracle_step_timed(xf, synth.router_weight(c), synth.expert_bias(c), c,
                                            lambda e: cache_f[e], lambda s: sh_f[s])
                dt = time.perf_counter() - t0
            runs[label] = {"threads": n, "seconds": round(dt, 3), "tokens_per_s": round(c.tokens / dt, 1),
                           "stages_s": {k: round(v, 4) for k, v in st.items()}}
        res["full_workloads"][name] = runs
    return res


def measure(layer, cfg, xs, steps: int, warmup: int, reset_bias: bool = True):
    """Times ``steps`` forward steps of ``layer`` (bias update included) over the device
    batches ``xs`` (step i uses xs[i % len(xs)]); stage spans from HIP events on the
    launch stream. ``reset_bias``: every step starts from the layer's current bias (a
    1 KB device copy before each step), so that repeating one batch times the configured
    workload rather than a bias drifted by earlier repetitions; otherwise the bias
    follows its trajectory, and the per-step loads and bias range are recorded."""
    import numpy as np
    import torch

    from deepseekmoe_routing_fp8_amd import MoELayer
    b0 = layer.bias.clone()
    for i in range(warmup):
        layer.forward(xs[i % len(xs)])
        layer.bias.copy_(b0)
    torch.cuda.synchronize()
    nst = len(MoELayer.STAGES)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(steps)]
    N = cfg.num_experts
    loads = torch.empty((steps, N), dtype=torch.int32, device=layer.bias.device)
    biases = torch.empty((steps, N), dtype=torch.float32, device=layer.bias.device)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        if reset_bias:
            layer.bias.copy_(b0)
        layer.forward(xs[i % len(xs)], events=evs[i])
        if not reset_bias:
            loads[i].copy_(layer.counts)
            biases[i].copy_(layer.bias)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    stage_ms = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(nst)]
                         for i in range(steps)])
    st = {s: float(stage_ms[:, j].mean()) for j, s in enumerate(MoELayer.STAGES)}
    ab = ffn_algorithmic_bytes(cfg, layer.counts.cpu().numpy())
    H, I, T = cfg.hidden_size, cfg.moe_intermediate_size, cfg.tokens
    k, S = cfg.num_experts_per_tok, cfg.num_shared_experts
    ms = wall * 1e3 / steps
    ffn_ms = st["ffn_gate_up"] + st["ffn_down"]
    tflops = 6.0 * H * I * T * (k + S) / (ms * 1e-3) / 1e12
    gbs = (ab["gate_up"] + ab["down"]) / (ffn_ms * 1e-3) / 1e9
    out = {"workload": cfg.name, "tokens": T, "steps": steps,
           "ms_per_step": round(ms, 4), "tokens_per_s": round(T * steps / wall, 1),
           "tflops_fp8": round(tflops, 1), "frac_fp8_mfma_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
           "experts_touched": ab["experts"], "ffn_algorithmic_bytes": ab["gate_up"] + ab["down"],
           "ffn_ms": round(ffn_ms, 4), "ffn_gbs": round(gbs, 1),
           "ffn_frac_hbm": round(gbs / HBM_PEAK_GBS, 4),
           "gate_up_gbs": round(ab["gate_up"] / (st["ffn_gate_up"] * 1e-3) / 1e9, 1),
           "down_gbs": round(ab["down"] / (st["ffn_down"] * 1e-3) / 1e9, 1),
           "ffn_tflops_fp8": round(6.0 * H * I * T * (k + S) / (ffn_ms * 1e-3) / 1e12, 1),
           "stage_ms": {s: round(v, 4) for s, v in st.items()},
           "bias": "reset to the configured value before every step" if reset_bias else
                   "updated every step from the step's own loads (trajectory from the configured value)"}
    if not reset_bias:
        c = loads.float()
        ratio = (c.max(dim=1).values / c.mean(dim=1)).cpu().numpy()
        out["max_over_mean_load_per_step"] = [round(float(v), 3) for v in ratio]
        b = biases.cpu().numpy()
        out["bias_min_per_step"] = [round(float(v), 4) for v in b.min(axis=1)]
        out["bias_max_per_step"] = [round(float(v), 4) for v in b.max(axis=1)]
    return out


def measure_graph(layer, x, steps: int, warmup: int):
    """The same step (bias update included) captured once into a HIP graph and replayed
    ``steps`` times: the launches' host overhead leaves the timed region. As in the eager
    loop, the configured bias is restored (a 1 KB device copy) before every replay, so both
    route the same workload."""
    import torch
    b0 = layer.bias.clone()
    layer.capture(x, update_bias=True)
    for _ in range(warmup):
        layer.bias.copy_(b0)
        layer.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.bias.copy_(b0)
        layer.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    layer._graph = None
    layer.bias.copy_(b0)
    T = x.shape[0]
    return {"ms_per_step": round(wall * 1e3 / steps, 4), "tokens_per_s": round(T * steps / wall, 1),
            "steps": steps, "note": "MoELayer.capture / replay: one HIP graph per step (bias update "
                                    "inside the graph; the configured bias restored before each "
                                    "replay, as in the eager loop)"}


def device_batches(cfg, n: int):
    """n seeded batches on the device (n = 1: the preset's own batch; otherwise the fresh
    batches of steps 0..n-1), generated on a host thread pool outside any timed region."""
    import torch
    from concurrent.futures import ThreadPoolExecutor

    import synth
    dt = torch.bfloat16 if cfg.x_dtype == "bf16" else torch.float32
    if n == 1:
        return [torch.from_numpy(synth.hidden_states(cfg)).to(dt).cuda()]
    out = []
    with ThreadPoolExecutor(min(16, len(os.sched_getaffinity(0)))) as ex:
        for x in ex.map(lambda i: synth.hidden_states(cfg, step=i), range(n)):
            out.append(torch.from_numpy(x).to(dt).cuda())
    return out


def measure_backward(layer, cfg, x, steps: int, warmup: int):
    """Times ``steps`` training steps (forward, then the FP8 backward of a seeded bf16
    upstream gradient; weight gradients in FP32) on one device batch; per-stage spans of
    the backward from HIP events on the launch stream."""
    import numpy as np
    import torch

    from deepseekmoe_routing_fp8_amd import MoELayer
    T, H, I = cfg.tokens, cfg.hidden_size, cfg.moe_intermediate_size
    k, S, N = cfg.num_experts_per_tok, cfg.num_shared_experts, cfg.num_experts
    g = torch.Generator(device="cpu").manual_seed(1234)
    dout = torch.randn((T, H), generator=g).to(torch.bfloat16).cuda()
    for _ in range(warmup):
        layer.forward(x, update_bias=False)
        layer.backward(dout)
    torch.cuda.synchronize()
    nb = len(MoELayer.BWD_STAGES)
    fe = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    be = [[torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        fe[i][0].record()
        layer.forward(x, update_bias=False)
        fe[i][1].record()
        layer.backward(dout, events=be[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    fwd = float(np.mean([a.elapsed_time(b) for a, b in fe]))
    bwd = float(np.mean([e[0].elapsed_time(e[-1]) for e in be]))
    st = {s_: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in be]))
          for j, s_ in enumerate(MoELayer.BWD_STAGES)}
    rows = T * (k + S)
    # FP8 GEMM work of the backward: dh, dx over K = 2I, three wgrads, and the recompute of a
    # and b unless the forward kept them
    flops = (12.0 if layer.keep_ab else 16.0) * rows * H * I
    dw_bytes = 3 * (N + S) * H * I * layer.dw_dtype.itemsize
    return {"tokens": T, "steps": steps, "train_step_ms": round(wall * 1e3 / steps, 4),
            "train_tokens_per_s": round(T * steps / wall, 1), "forward_ms": round(fwd, 4),
            "backward_ms": round(bwd, 4), "backward_stage_ms": {k_: round(v, 4) for k_, v in st.items()},
            "backward_fp8_tflops": round(flops / (bwd * 1e-3) / 1e12, 1),
            "ffn_backward_fp8_tflops": round(flops / (st["ffn_bwd"] * 1e-3) / 1e12, 1),
            "weight_grad_bytes": dw_bytes, "weight_grad_dtype": str(layer.dw_dtype).replace("torch.", ""),
            "swiglu_inputs": ("kept by the forward (FP32 a, b); the backward recomputes h" if layer.keep_ab
                              else "recomputed in the backward by the gate/up GEMMs"),
            "note": ("forward + FP8 backward (dgrad and wgrad in E4M3); no optimizer")}


def time_seq_balance(layer, cfg, seq_len: int, calls: int = 20):
    """Time moe_seq_balance on the layer's last routing (sequences of seq_len tokens)."""
    import numpy as np
    import torch
    for _ in range(3):
        layer.seq_balance(seq_len)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(calls):
        loss, ent = layer.seq_balance(seq_len)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / calls
    nbytes = cfg.tokens * (cfg.num_experts + cfg.num_experts_per_tok) * 4
    return {"tokens": cfg.tokens, "seq_len": seq_len, "us_per_call": round(us, 2),
            "algorithmic_bytes": nbytes, "achieved_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
            "loss": [round(float(v), 8) for v in loss.cpu()],
            "entropy_nats": [round(float(v), 4) for v in ent.cpu()],
            "max_entropy_nats": round(float(np.log(cfg.num_experts)), 4)}


def other_configs(layer, warmup: int, decode_steps: int, args_skewed_steps: int = 100):
    """The other workloads of the same method, outside the headline number: the T=128
    decode step and the skewed T=16384 step on the same V3 layer, and the reduced layer
    (its own weights)."""
    import numpy as np
    import torch

    import synth
    from deepseekmoe_routing_fp8_amd import MoELayer
    res = {}
    if decode_steps > 0:
        cfg = synth.PRESETS["v3_decode"]
        log(f"[bench] decode: T={cfg.tokens}, {decode_steps} steps")
        xd = device_batches(cfg, 1)
        res["decode"] = measure(layer, cfg, xd, decode_steps, warmup)
        res["decode"]["graph"] = measure_graph(layer, xd[0], decode_steps, warmup)
        cfg = synth.PRESETS["v3_skewed"]
        xs_p2 = []
        if args_skewed_steps > 0:
            log(f"[bench] skewed: T={cfg.tokens}, generating {args_skewed_steps} fresh clustered batches")
            xs = device_batches(cfg, args_skewed_steps)
            log(f"[bench] skewed: {args_skewed_steps} steps, bias from 0, updated every step")
            layer.bias.zero_()
            res["skewed"] = measure(layer, cfg, xs, args_skewed_steps, 0, reset_bias=False)
            xs_p2 = xs[:20]   # the power-of-two variant is compared on the first 20 batches
            del xs
            layer.bias.zero_()
            skewed_default_20 = measure(layer, cfg, xs_p2, len(xs_p2), 0, reset_bias=False)
            # per-sequence balance loss / allocation entropy of the last skewed step's routing
            # (4 sequences of 4096 tokens); timed on its own, it is not part of the forward step
            res["seq_balance"] = time_seq_balance(layer, cfg, 4096)
        cfg = synth.PRESETS["reduced"]
        log("[bench] reduced layer: weights on the device")
        small = MoELayer(cfg)
        small.load_from_synth()
        res["reduced"] = measure(small, cfg, device_batches(cfg, 1), 30, warmup)
        del small
        # the opt-in power-of-two scale variant on the headline workload (its own weights)
        cfg = synth.PRESETS["v3_prefill"]
        log("[bench] power-of-two scale variant: weights on the device")
        p2 = MoELayer(cfg, scale_mode=1)
        p2.load_from_synth()
        res["pow2_scales"] = measure(p2, cfg, device_batches(cfg, 1), 30, warmup)
        res["pow2_scales"]["note"] = ("opt-in variant (scale_mode 1): power-of-two 1x128 / 128x128 "
                                      "scales applied by the MFMA, FP32 accumulation across K")
        # the same variant where compute matters: the skewed T=16384 step, 20 fresh batches
        # from bias 0, beside the default path on the same batches
        cs = synth.PRESETS["v3_skewed"]
        if xs_p2:
            p2.bias.zero_()
            r2 = measure(p2, cs, xs_p2, len(xs_p2), 0, reset_bias=False)
            res["pow2_scales_skewed"] = {
                "steps": len(xs_p2), "pow2_ms_per_step": r2["ms_per_step"],
                "default_ms_per_step": skewed_default_20["ms_per_step"],
                "pow2_ffn_ms": r2["ffn_ms"], "default_ffn_ms": skewed_default_20["ffn_ms"],
                "pow2_tflops_fp8": r2["tflops_fp8"], "default_tflops_fp8": skewed_default_20["tflops_fp8"],
                "note": f"first {len(xs_p2)} fresh skewed batches, bias from 0 updated every step, both paths"}
        del p2, xs_p2
        # forward + FP8 backward on the headline workload (its own layer with the dgrad
        # operands and FP32 weight-gradient buffers)
        log("[bench] backward: weights and transposed dgrad operands on the device")
        bl = MoELayer(cfg, backward=True)
        bl.load_from_synth()
        res["backward"] = measure_backward(bl, cfg, device_batches(cfg, 1)[0], 10, 2)
        del bl
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="v3_prefill")
    ap.add_argument("--cpu-sample-tokens", type=int, default=24)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--backward-only", action="store_true",
                    help="time forward + backward of the workload instead of the forward line "
                         "(for profiling the backward kernels)")
    ap.add_argument("--dw-dtype", default="f32", choices=("f32", "bf16"),
                    help="weight-gradient dtype of the backward measurement")
    ap.add_argument("--seq-len", type=int, default=0,
                    help="also time the per-sequence balance statistic on the last step's "
                         "routing, over sequences of this many tokens (0: only in the extras)")
    ap.add_argument("--decode-steps", type=int, default=50,
                    help="steps of the T=128 decode workload timed after the main one; the "
                         "skewed and reduced workloads follow it (0: skip all three)")
    ap.add_argument("--skewed-steps", type=int, default=100,
                    help="forward + bias-update steps of the skewed T=16384 workload, each on a "
                         "fresh clustered batch generated before the timed region (0: skip it)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the multi-GPU (expert-parallel) path is not "
              "built; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import __graft_entry__
    b = __graft_entry__._builder()
    if not os.path.exists(b.LIB):
        b.build()
    from deepseekmoe_routing_fp8_amd import MoELayer

    cfg = synth.PRESETS[args.workload]
    T, H, I, k, S = (cfg.tokens, cfg.hidden_size, cfg.moe_intermediate_size,
                     cfg.num_experts_per_tok, cfg.num_shared_experts)
    log(f"[bench] {cfg.name}: generating and quantising weights on the device")
    t0 = time.time()
    layer = MoELayer(cfg, backward=args.backward_only,
                     dw_dtype=torch.bfloat16 if args.dw_dtype == "bf16" else torch.float32)
    layer.load_from_synth()
    x = torch.from_numpy(synth.hidden_states(cfg)).to(
        torch.bfloat16 if cfg.x_dtype == "bf16" else torch.float32).cuda()
    log(f"[bench] weights ready in {time.time() - t0:.1f} s; warmup {args.warmup}")
    if args.backward_only:
        r = measure_backward(layer, cfg, x, args.steps, args.warmup)
        r.update({"workload": cfg.name, "dtype": "fp8-e4m3 GEMMs, fp32 accumulation"})
        print(json.dumps(r), flush=True)
        return
    # every step runs the configured workload: the bias update of a step is part of the
    # timed work, and a 1 KB device copy restores the configured bias before the next one
    b0 = layer.bias.clone()
    for _ in range(args.warmup):
        layer.forward(x)
        layer.bias.copy_(b0)
    torch.cuda.synchronize()

    nst = len(MoELayer.STAGES)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nst + 1)] for _ in range(args.steps)]
    log(f"[bench] timing {args.steps} steps")
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for i in range(args.steps):
        layer.bias.copy_(b0)
        layer.forward(x, events=evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    stage_ms = np.array([[evs[i][j].elapsed_time(evs[i][j + 1]) for j in range(nst)]
                         for i in range(args.steps)])
    step_ms = np.array([evs[i][0].elapsed_time(evs[i][nst]) for i in range(args.steps)])
    ms_per_step = wall * 1e3 / args.steps
    value = T * args.steps / wall

    counts = layer.counts.cpu().numpy()
    flops_layer = 6.0 * H * I * T * (k + S)
    tflops = flops_layer / (ms_per_step * 1e-3) / 1e12
    st = {s: float(stage_ms[:, j].mean()) for j, s in enumerate(MoELayer.STAGES)}
    ab = ffn_algorithmic_bytes(cfg, counts)
    gu_ms, dn_ms = st["ffn_gate_up"], st["ffn_down"]
    achieved = ab["gate_up"] / (gu_ms * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": "synthetic (seeded N(0,1) hidden states, N(0,1/fan_in) weights quantised to E4M3 128x128)",
        "config": {"workload": cfg.name, "tokens": T, "hidden": H, "routed_experts": cfg.num_experts,
                   "shared_experts": S, "top_k": k, "expert_intermediate": I,
                   "groups": f"{cfg.n_group}x{cfg.num_experts // cfg.n_group} keep {cfg.topk_group} "
                             f"(top-{cfg.group_score_topn} sum)" if cfg.n_group > 1 else "none",
                   "parallelism": "single GPU"},
        "tflops_fp8": round(tflops, 1),
        "frac_fp8_mfma_peak": round(tflops / FP8_PEAK_TFLOPS, 4),
        "roofline": {
            "kernel": "ffn_kernel<1> (moe_grouped_ffn_fp8_gate_up: routed + shared experts, "
                      "gate/up GEMMs, SwiGLU, 1x128 re-quantisation; includes the tile-plan and scale-gather launch)",
            "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": measured_traffic(),
            "algorithmic_bytes": ab["gate_up"], "experts_touched": ab["experts"],
            "avg_ms": round(gu_ms, 4),
            "mfma_tflops": round(4.0 * H * I * T * (k + S) / (gu_ms * 1e-3) / 1e12, 1),
        },
        "down_kernel": {
            "avg_ms": round(dn_ms, 4), "algorithmic_bytes": ab["down"],
            "achieved_gbs": round(ab["down"] / (dn_ms * 1e-3) / 1e9, 1),
            "mfma_tflops": round(2.0 * H * I * T * (k + S) / (dn_ms * 1e-3) / 1e12, 1),
        },
        "stage_ms": {s: round(v, 4) for s, v in st.items()},
        "event_ms_per_step": round(float(step_ms.mean()), 4),
        "max_over_mean_load": round(float(counts.max() / counts.mean()), 3),
    }
    log(f"[bench] graph replay: {args.steps} steps")
    res["graph"] = measure_graph(layer, x, args.steps, args.warmup)
    if args.seq_len > 0:
        res["seq_balance"] = time_seq_balance(layer, cfg, args.seq_len)
    if args.workload == "v3_prefill":
        layer.bias.copy_(b0)
        res.update(other_configs(layer, args.warmup, args.decode_steps, args.skewed_steps))
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: oracle on {args.cpu_sample_tokens} tokens")
        res["cpu_baseline"] = cpu_baseline(cfg, args.cpu_sample_tokens)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
