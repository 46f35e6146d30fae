#!/usr/bin/env python3
"""Benchmark of the span-commit forward on one MI355X.

Workload (default): a Qwen2.5-1.5B-shaped decoder layer + LM head in bf16, KV cache of 2048
positions built from random tokens, copy spans of N in {8, 16, 32, 64, 128, 256, 512} known
tokens taken from a random document.  One step = one copy-span commit per N (cad_span_forward
with CAD_COMMIT_ALL: a copy span is accepted by construction), each over a cache of exactly
2048 positions.  Committed tokens/s = sum(N) / step time.

Prints ONE JSON line.  Also reported: per-N time and roofline fractions, the autoregressive
baseline (N single-token forwards), per-kernel times from the library's event profiler, the
roofline of the dominant kernel (LM head + argmax), and the CPU oracle's throughput on the
host cores as a reference baseline.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "committed tokens/s vs N (8–512) per span forward; % HBM / MFMA roofline"
ROOF_N = 32            # span length whose LM-head kernel is reported as the dominant-kernel roofline
TRIALS = 25            # separately timed replays behind each median and interquartile range


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--spans", type=str, default="8,16,32,64,128,256,512")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=20.0)
    ap.add_argument("--ar-steps", type=int, default=64)
    ap.add_argument("--no-pld", action="store_true", help="skip the batched PLD round measurement")
    ap.add_argument("--no-stack", action="store_true",
                    help="skip the full-depth (28-layer) span-forward curve on the 1.5B and 7B shapes")
    ap.add_argument("--no-block", action="store_true", help="skip the block-triangular verify measurement")
    ap.add_argument("--no-program", action="store_true",
                    help="skip the Copy-as-Decode program measurement (op-boundary steps, 7B-shaped layer)")
    ap.add_argument("--pmc-pass", action="store_true",
                    help="no timing: a few N = ROOF_N forwards and plain copies of a known size, for a "
                         "hardware-counter run that calibrates and measures the LM head's HBM traffic")
    ap.add_argument("--part", choices=("program", "stack", "pld", "block"), default=None,
                    help="run one secondary workload alone and print its JSON object (for a profiler run); "
                         "no headline line")
    return ap.parse_args()


def main():
    a = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only: --gpus {a.gpus} / WORLD_SIZE {world} is not supported "
              "(the span forward of a sequence batch runs on one GPU and is not sharded across GPUs)",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    from spec_verify_cad_amd import cad, synth
    from spec_verify_cad_amd import roofline as R
    from spec_verify_cad_amd.configs import CONFIGS, copy_sweep_inputs

    if a.part in ("program", "stack", "block"):
        dev = torch.device("cuda:0")
        torch.cuda.set_device(dev)
        cad.lib()
        if a.part == "program":
            out = cad_program(a, dev)
        elif a.part == "block":
            out = block_verify(a, dev)
        else:
            out = [stack_curve(a, dev, "qwen15_span"), stack_curve(a, dev, "qwen7_cad_program", program=True)]
            stack_cost_model(out)
        print(json.dumps(out), flush=True)
        return

    wl = CONFIGS["qwen15_span"]
    shp = wl.shape
    spans = [int(x) for x in a.spans.split(",")]
    L0 = wl.cache_len
    cap = L0 + max(spans) + a.ar_steps + 8
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cad.lib()

    t0 = time.time()
    w = synth.layer_weights(shp, wl.seed)
    log(f"weights generated in {time.time() - t0:.1f}s")
    lay0 = cad.DeviceLayer(shp, w)
    # second copy of every streamed matrix (not the embedding, which is only gathered): forwards
    # alternate between copies so none finds the previous forward's weights in the last-level cache
    lay1 = cad.DeviceLayer.__new__(cad.DeviceLayer)
    lay1.shape = shp
    lay1.t = {k: (v if k == "embed" else v.clone()) for k, v in lay0.t.items()}
    lay1.desc = lay1.make_desc()
    layers = [lay0, lay1]

    doc, prefix, span_toks = copy_sweep_inputs(wl, spans)
    if a.pmc_pass:
        pmc_pass(a, shp, layers, prefix, span_toks, spans, L0, cap, dev)
        return
    if a.part == "pld":
        print(json.dumps(pld_rounds(a, lay0, dev)), flush=True)
        return

    # one cache per N; their lengths are views of one tensor so a single fill restores them all
    lens = torch.zeros(len(spans), dtype=torch.int32, device=dev)
    caches = [cad.DeviceCache(shp, 1, cap, len_tensor=lens[i:i + 1]) for i in range(len(spans))]
    ptoks = torch.from_numpy(prefix[None].astype(np.int32)).to(dev)
    cad.span_forward(lay0, caches[0], ptoks, L0, flags=cad.KV_ONLY | cad.COMMIT_ALL)
    for c in caches[1:]:
        c.k.copy_(caches[0].k)
        c.v.copy_(caches[0].v)
    torch.cuda.synchronize()
    assert int(lens[0]) == L0

    toks = [torch.from_numpy(t[None].astype(np.int32)).to(dev) for t in span_toks]
    outs = [torch.empty((1, N), dtype=torch.int32, device=dev) for N in spans]
    wss = [cad.alloc_workspace(cad.span_forward_workspace(lay0, 1, N, cad.MASK_CAUSAL, 1, 1, cap, cad.COMMIT_ALL))
           for N in spans]
    ar_tok = torch.from_numpy(doc[L0:L0 + a.ar_steps].astype(np.int32).reshape(-1, 1)).to(dev)
    ar_out = torch.empty((1, 1), dtype=torch.int32, device=dev)
    ar_ws = cad.alloc_workspace(cad.span_forward_workspace(lay0, 1, 1, cad.MASK_CAUSAL, 1, 1, cap, cad.COMMIT_ALL))

    outs_last = [torch.empty((1,), dtype=torch.int32, device=dev) for _ in spans]

    def forward(j, copy, stream, last=False):
        """One copy-span commit of spans[j] from a cache of exactly L0 positions (last: copy-commit
        mode, the LM head only for the span's last row)."""
        lens[j:j + 1].fill_(L0)
        cad.span_forward(layers[copy], caches[j], toks[j], spans[j],
                         flags=cad.COMMIT_ALL | (cad.LOGITS_LAST if last else 0),
                         argmax_out=outs_last[j] if last else outs[j], workspace=wss[j], stream=stream)

    def ar_run(stream, copy0=0):
        lens[0:1].fill_(L0)
        for i in range(a.ar_steps):
            cad.span_forward(layers[(copy0 + i) & 1], caches[0], ar_tok[i:i + 1], 1, flags=cad.COMMIT_ALL,
                             argmax_out=ar_out, workspace=ar_ws, stream=stream)

    # eager warm-up of every launch configuration (first calls query occupancy), then capture:
    # the forwards are replayed from HIP graphs, so the timing is of the GPU work, not of the
    # host's launch rate.  Every replay runs every kernel of the forward.
    for _ in range(2):
        for j in range(len(spans)):
            forward(j, j & 1, torch.cuda.current_stream())
            forward(j, j & 1, torch.cuda.current_stream(), last=True)
        ar_run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(torch.cuda.current_stream())

    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            fn(torch.cuda.current_stream())
        return g

    # sweep step graphs: one commit of every N, weight copies alternating forward to forward
    step_graphs = [capture(lambda st, c=c: [forward(j, (j + c) & 1, st) for j in range(len(spans))]) for c in (0, 1)]
    per_n_graphs = [[capture(lambda st, j=j, c=c: forward(j, c, st)) for c in (0, 1)] for j in range(len(spans))]
    ar_graphs = [capture(lambda st, c=c: ar_run(st, c)) for c in (0, 1)]
    last_step_graphs = [capture(lambda st, c=c: [forward(j, (j + c) & 1, st, last=True) for j in range(len(spans))])
                        for c in (0, 1)]
    last_graphs = [[capture(lambda st, j=j, c=c: forward(j, c, st, last=True)) for c in (0, 1)]
                   for j in range(len(spans))]
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()

    def timed(graphs, reps):
        for i in range(3):
            graphs[i & 1].replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(reps):
            graphs[i & 1].replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps        # ms per replay

    def trials(graphs, n=TRIALS):
        """Median and interquartile range (us) of n separately timed replays (an event pair around
        each replay, the replays back to back on one stream)."""
        for i in range(3):
            graphs[i & 1].replay()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        for i, (b, e) in enumerate(ev):
            b.record(stream)
            graphs[i & 1].replay()
            e.record(stream)
        torch.cuda.synchronize()
        return R.med_iqr([b.elapsed_time(e) * 1e3 for b, e in ev])

    # ---- timed region: K steps of the whole sweep
    for i in range(a.warmup):
        step_graphs[i & 1].replay()
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ms_step = timed(step_graphs, a.steps)
    wall = time.perf_counter() - wall0
    tokens_step = sum(spans)
    value = tokens_step / (ms_step * 1e-3)
    step_trials = trials(step_graphs)
    log(f"sweep step {ms_step * 1e3:.1f} us -> {value:.0f} committed tok/s (wall {wall * 1e3 / a.steps:.1f} us/step)")
    # check: the replayed commits left the caches at L0 + N and produced argmax ids
    assert all(int(lens[j]) == L0 + N for j, N in enumerate(spans))

    # ---- per-N: forward time (length restore included), and per-kernel times from the profiler
    per_n = []
    for j, N in enumerate(spans):
        us = timed(per_n_graphs[j], a.steps) * 1e3
        tr = trials(per_n_graphs[j])
        cad.profile_enable(True)
        for i in range(a.steps):
            forward(j, i & 1, stream)
        torch.cuda.synchronize()
        prof = cad.profile_read()
        cad.profile_enable(False)
        kern = {k: round(v[0] * 1e3 / v[1], 2) for k, v in prof.items()}
        nb = R.forward_bytes(shp, 1, N, L0)
        fl = R.forward_flops(shp, 1, N, L0)
        floor, bound = R.floor_us(nb, fl)
        lm_us = kern.get("lm_head_argmax")
        per_n.append({
            "N": N, "us": round(us, 2), "committed_tok_s": round(N / (us * 1e-6), 1),
            "trials_us": tr,
            "alg_bytes": int(nb), "alg_flops": int(fl), "bound": bound, "floor_us": round(floor, 2),
            "frac_of_roofline": round(floor / us, 4),
            "hbm_frac": round(nb / (us * 1e-6) / (R.HBM_PEAK_GBS * 1e9), 4),
            "mfma_frac": round(fl / (us * 1e-6) / (R.MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
            "lm_head_us": lm_us,
            "lm_head_hbm_frac": round(R.lm_head_bytes(shp, N) / (lm_us * 1e-6) / (R.HBM_PEAK_GBS * 1e9), 4),
            "lm_head_mfma_frac": round(R.lm_head_flops(shp, N) / (lm_us * 1e-6) / (R.MFMA_BF16_PEAK_TFLOPS * 1e12), 4),
            "kernel_us": kern,
        })
        log(f"N={N}: {us:.1f} us, {N / (us * 1e-6):.0f} tok/s, {bound} floor {floor:.1f} us "
            f"({floor / us * 100:.1f}%), lm_head {lm_us} us")

    # ---- copy-commit mode (CAD_LOGITS_LAST): inside a copy span only the prediction after the
    # span is consumed, so the LM head runs for the last row only
    ms_last = timed(last_step_graphs, a.steps)
    last_per_n = []
    for j, N in enumerate(spans):
        us = timed(last_graphs[j], a.steps) * 1e3
        last_per_n.append({"N": N, "us": round(us, 2), "committed_tok_s": round(N / (us * 1e-6), 1),
                           "speedup_vs_full": round(per_n[j]["us"] / us, 3)})
        log(f"copy-commit N={N}: {us:.1f} us, {N / (us * 1e-6):.0f} tok/s")
    copy_commit = {"flag": "CAD_LOGITS_LAST", "value": round(tokens_step / (ms_last * 1e-3), 1),
                   "unit": "committed tokens/s", "ms_per_step": round(ms_last, 4), "per_n": last_per_n}
    log(f"copy-commit sweep {ms_last * 1e3:.1f} us -> {copy_commit['value']:.0f} committed tok/s")

    # ---- the tiny fp32 layer (one copy span of 8 over a 128-position cache, and 8 decode steps)
    tiny = tiny_config(a, dev, trials)

    # ---- batched PLD rounds (lookup -> verify forward -> accept, no host sync inside)
    pld = None if a.no_pld else pld_rounds(a, lay0, dev)

    # ---- full-depth stacks: the pages' kernel table (parallel forward vs autoregression) at 28 layers
    stack = None if a.no_stack else [stack_curve(a, dev, "qwen15_span"),
                                     stack_curve(a, dev, "qwen7_cad_program", program=not a.no_program)]
    if stack:
        stack_cost_model(stack)

    # ---- block-triangular multi-candidate verify (7B-shaped layer)
    block = None if a.no_block else block_verify(a, dev)

    # ---- a whole Copy-as-Decode program with its op-boundary steps (7B-shaped layer)
    program = None if a.no_program else cad_program(a, dev)

    # ---- autoregressive baseline: single-token teacher-forced forwards
    ar_us = timed(ar_graphs, max(2, a.steps // 4)) * 1e3 / a.ar_steps
    for r in per_n:
        r["speedup_vs_ar"] = round(r["N"] * ar_us / r["us"], 2)
    ar_floor, _ = R.floor_us(R.forward_bytes(shp, 1, 1, L0), R.forward_flops(shp, 1, 1, L0))
    log(f"AR: {ar_us:.1f} us/token ({1e6 / ar_us:.0f} tok/s), floor {ar_floor:.1f} us")

    # ---- dominant kernel roofline: LM head + argmax at N = ROOF_N (HBM-bound)
    rn = next(r for r in per_n if r["N"] == ROOF_N) if ROOF_N in spans else per_n[0]
    lm_bytes = R.lm_head_bytes(shp, rn["N"])
    achieved = lm_bytes / (rn["lm_head_us"] * 1e-6) / 1e9
    roof = {"kernel": "lm_head_argmax (k_skinny, EPI_ARGMAX)", "N": rn["N"], "bound": "hbm",
            "achieved": round(achieved, 1), "peak": R.HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / R.HBM_PEAK_GBS, 4), "traffic": lm_traffic() if rn["N"] == 32 else None,
            "frac_scope": "the dominant kernel alone (LM head + argmax partials at N = 32); the whole span "
                          "forward's fractions are in forward_frac",
            "alg_bytes_per_launch": int(lm_bytes), "avg_launch_us": rn["lm_head_us"],
            "timing": "HIP events around the kernel on its launch stream, eager forwards after the timed graph replays",
            # the whole forward (every kernel of one commit) against its own floor: HBM at N <= 256,
            # MFMA at N = 512 (targets: >= 0.60 of HBM at N <= 32, >= 0.50 of bf16 MFMA at N = 512)
            "forward_frac": {str(r["N"]): {"bound": r["bound"], "frac": r["frac_of_roofline"],
                                           "hbm_frac": r["hbm_frac"], "mfma_frac": r["mfma_frac"]} for r in per_n}}
    big = next((r for r in per_n if r["N"] == 512), None)
    if big:
        roof["mfma_at_N512"] = {"achieved_tflops": round(R.lm_head_flops(shp, 512) / (big["lm_head_us"] * 1e-6) / 1e12, 1),
                                "peak": R.MFMA_BF16_PEAK_TFLOPS, "frac": big["lm_head_mfma_frac"]}

    # ---- CPU oracle baseline on the host cores (bounded sample of the same sweep)
    cpu = None
    if not a.no_cpu_baseline:
        cpu = cpu_baseline(shp, w, prefix, span_toks, spans, cap, a.cpu_budget_s)

    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "committed tokens/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(ms_step, 4),
        "step_trials_us": step_trials, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "copy-span commit sweep: Qwen2.5-1.5B-shaped layer (hidden 1536, 12/2 heads x 128, "
                               "SwiGLU 8960) + LM head 151936, bf16 weights N(0,0.02), KV cache 2048, one "
                               "commit of each N per step, weights rotated over 2 copies",
                   "spans": spans, "cache_len": L0, "tokens_per_step": tokens_step, "batch": 1},
        "per_n": per_n,
        "ar_baseline": {"us_per_token": round(ar_us, 2), "tok_s": round(1e6 / ar_us, 1), "floor_us": round(ar_floor, 2)},
        "roofline": roof,
        "copy_commit_mode": copy_commit,
        "tiny_f32": tiny,
        "pld_rounds": pld,
        "block_verify": block,
        "cad_program": program,
        "full_depth_stacks": stack,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def tiny_config(a, dev, trials):
    """The tiny fp32 layer (hidden 256, 4 heads x 64, FFN 1024, vocab 1024): one copy span of
    N = 8 committed over a 128-position cache, against 8 single-token forwards.  Everything is
    cache-resident and launch-bound at this size, so no roofline is given; the cache rows come
    from a K/V-only prefill of 128 random tokens (their values do not change the timing)."""
    import numpy as np
    import torch

    from spec_verify_cad_amd import cad, synth
    from spec_verify_cad_amd.configs import CONFIGS

    wl = CONFIGS["tiny_f32"]
    shp, L0, N = wl.shape, wl.cache_len, wl.spans[0]
    lay = cad.DeviceLayer(shp, synth.layer_weights(shp, wl.seed))
    cache = cad.DeviceCache(shp, 1, L0 + 2 * N)
    pre = torch.from_numpy(synth.uniform_tokens(wl.seed, L0, shp.vocab)[None].astype(np.int32)).to(dev)
    cad.span_forward(lay, cache, pre, L0, flags=cad.KV_ONLY | cad.COMMIT_ALL)
    span = torch.from_numpy(synth.uniform_tokens(wl.seed, N, shp.vocab, stream=1)[None].astype(np.int32)).to(dev)
    out = torch.empty((1, N), dtype=torch.int32, device=dev)
    ws = cad.alloc_workspace(cad.span_forward_workspace(lay, 1, N, cad.MASK_CAUSAL, 1, 1, cache.cap, 0))

    def span_fwd(st):
        cache.len.fill_(L0)
        cad.span_forward(lay, cache, span, N, flags=cad.COMMIT_ALL, argmax_out=out, workspace=ws, stream=st)

    def steps(st):
        cache.len.fill_(L0)
        for i in range(N):
            cad.span_forward(lay, cache, span[:, i:i + 1], 1, flags=cad.COMMIT_ALL, argmax_out=out[:, i:i + 1],
                             workspace=ws, stream=st)

    span_fwd(torch.cuda.current_stream())
    steps(torch.cuda.current_stream())
    torch.cuda.synchronize()
    cs = torch.cuda.Stream()
    cs.wait_stream(torch.cuda.current_stream())
    gs = []
    for fn in (span_fwd, steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cs):
            fn(torch.cuda.current_stream())
        gs.append(g)
    torch.cuda.synchronize()
    t_span, t_ar = trials([gs[0], gs[0]]), trials([gs[1], gs[1]])
    log(f"tiny fp32: span of {N} {t_span['median']} us, {N} decode steps {t_ar['median']} us")
    return {"workload": f"tiny fp32 layer, copy span of {N} over a {L0}-position cache (graph replays)",
            "span_us": t_span, "ar_steps_us": t_ar,
            "committed_tok_s": round(N / (t_span["median"] * 1e-6), 1),
            "ar_tok_s": round(N / (t_ar["median"] * 1e-6), 1),
            "speedup_vs_ar": round(t_ar["median"] / t_span["median"], 2),
            "roofline": None, "note": "cache-resident and launch-bound: no roofline"}


def cad_program(a, dev):
    """A whole Copy-as-Decode program on the 7B-shaped layer: after a 4096-token document, 4096
    output tokens as copy splices and <gen> bodies, with every op-boundary step of the grammar
    (masked decisions over at most 11 ids, forced-template prefills), enqueued without a host
    sync and replayed from one HIP graph.  Beside it: the same 4096 output tokens as one-token
    forwards (autoregressive regeneration, eager), and per-step costs of a masked decision, a
    free decision and a 3-token forced prefill at the program's mid-point context.  The layer's
    weights are drawn on the device, N(0, 0.02), bf16 (timing does not depend on their values)."""
    import numpy as np
    import torch

    from spec_verify_cad_amd import cad, synth
    from spec_verify_cad_amd.configs import CONFIGS, cad_program_inputs
    from spec_verify_cad_amd.program import DeviceProgram

    wl = CONFIGS["qwen7_cad_program"]
    shp = wl.shape
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    t = {}
    for name, sh in synth.weight_shapes(shp).items():
        t[name] = (torch.randn(sh, generator=gen, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
    lay = cad.DeviceLayer.from_tensors(shp, t)
    doc, ops = cad_program_inputs(wl)
    fwds = synth.cad_program_forwards(ops)
    Ld, T = len(doc), wl.extra["total_out"]
    fed = sum(f.n for f in fwds)
    cap = ((Ld + max(fed, T) + 64 + 3) // 4) * 4
    cache = cad.DeviceCache(shp, 1, cap)
    dt = torch.from_numpy(doc[None].astype(np.int32)).to(dev)
    cad.span_forward(lay, cache, dt, Ld, flags=cad.KV_ONLY | cad.COMMIT_ALL)
    torch.cuda.synchronize()
    assert int(cache.len[0]) == Ld
    prog = DeviceProgram(lay, cache, doc, fwds, dev)

    def run(st):
        cache.len.fill_(Ld)
        prog.enqueue(st)

    stream = torch.cuda.current_stream()
    run(stream)
    torch.cuda.synchronize()
    assert int(cache.len[0]) == Ld + fed
    # eager, one event after every forward: the time of each forward role
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(fwds) + 1)]
    cache.len.fill_(Ld)
    evs[0].record(stream)
    for f in range(len(fwds)):
        prog.enqueue_one(f, stream)
        evs[f + 1].record(stream)
    torch.cuda.synchronize()
    eager_ms = evs[0].elapsed_time(evs[-1])
    by_role = {}
    for f, pf in enumerate(fwds):
        by_role[pf.role] = by_role.get(pf.role, 0.0) + evs[f].elapsed_time(evs[f + 1])
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cap_stream = torch.cuda.Stream()
    cap_stream.wait_stream(stream)
    t0 = time.time()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap_stream):
        run(torch.cuda.current_stream())
    torch.cuda.synchronize()
    log(f"program graph of {len(fwds)} forwards captured in {time.time() - t0:.1f}s")
    g.replay()
    torch.cuda.synchronize()
    reps = 3
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    assert int(cache.len[0]) == Ld + fed

    # autoregressive regeneration of the same output (copied and generated tokens), one token
    # per forward with the full LM head
    stream_toks = prog.fed_tokens(doc)
    content, pos = [], 0
    for f in fwds:
        if f.role == "splice":
            content += list(stream_toks[pos + len(f.lits):pos + f.n])
        elif f.role == "gen_body":
            content.append(stream_toks[pos])
        pos += f.n
    assert len(content) == T
    ar_tok = torch.from_numpy(np.asarray(content, dtype=np.int32).reshape(-1, 1)).to(dev)
    ar_out = torch.empty((1, 1), dtype=torch.int32, device=dev)
    ws1 = cad.alloc_workspace(cad.span_forward_workspace(lay, 1, 1, cad.MASK_CAUSAL, 1, 1, cap, cad.COMMIT_ALL))

    def ar(st):
        cache.len.fill_(Ld)
        for i in range(T):
            cad.span_forward(lay, cache, ar_tok[i:i + 1], 1, flags=cad.COMMIT_ALL, argmax_out=ar_out, workspace=ws1,
                             stream=st)

    ar(stream)
    torch.cuda.synchronize()
    e0.record(stream)
    ar(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ar_ms = e0.elapsed_time(e1)

    # per-step costs at the program's mid-point context: 32 steps of each kind from one graph
    mid = Ld + fed // 2
    one = torch.full((1, 1), synth.CAD_TOK["LT"], dtype=torch.int32, device=dev)
    three = torch.tensor([[synth.CAD_TOK["COPY"], synth.CAD_TOK["SPACE_LINES"], synth.CAD_TOK["EQ_QUOTE"]]],
                         dtype=torch.int32, device=dev)
    al2 = torch.tensor([[synth.CAD_TOK["COPY"], synth.CAD_TOK["GEN"]]], dtype=torch.int32, device=dev)
    al10 = torch.tensor([list(synth.CAD_DIGITS)], dtype=torch.int32, device=dev)
    o1 = torch.empty(1, dtype=torch.int32, device=dev)
    wsx = cad.alloc_workspace(max(cad.span_forward_workspace(lay, 1, n, cad.MASK_CAUSAL, 1, 1, cap, fl)
                                  for n, fl in ((1, cad.COMMIT_ALL), (3, cad.COMMIT_ALL | cad.LOGITS_LAST))))
    kinds = {
        "masked_step": lambda st: cad.span_forward_allowed(lay, cache, one, 1, al2, 2, flags=cad.COMMIT_ALL,
                                                           argmax_out=o1, workspace=wsx, stream=st),
        "free_step": lambda st: cad.span_forward(lay, cache, one, 1, flags=cad.COMMIT_ALL, argmax_out=o1,
                                                 workspace=wsx, stream=st),
        "forced_prefill_L3": lambda st: cad.span_forward_allowed(lay, cache, three, 3, al10, 10,
                                                                 flags=cad.COMMIT_ALL | cad.LOGITS_LAST,
                                                                 argmax_out=o1, workspace=wsx, stream=st),
    }
    per_step = {}
    for name, fn in kinds.items():
        def body(st, fn=fn):
            cache.len.fill_(mid)
            for _ in range(32):
                fn(st)
        body(stream)
        torch.cuda.synchronize()
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk, stream=cap_stream):
            body(torch.cuda.current_stream())
        gk.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(4):
            gk.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        per_step[name] = round(e0.elapsed_time(e1) * 1e3 / (4 * 32), 2)
    # this layer's own s(N) at the document's length, the page's way (one parallel forward of N
    # against N one-token forwards), for the splice forwards as the program runs them (the
    # decision after the last row masked), and Eq. (2)'s terms from it against the measured roles
    from spec_verify_cad_amd import costmodel as C
    spans_n = [n for n in STACK_SPANS if n >= 2] + [514]
    toks = torch.randint(0, shp.vocab, (1, max(spans_n)), generator=gen, device=dev, dtype=torch.int32)
    wsc = cad.alloc_workspace(max(cad.span_forward_workspace(lay, 1, n, cad.MASK_CAUSAL, 1, 1, cap,
                                                             cad.COMMIT_ALL | cad.LOGITS_LAST) for n in spans_n))
    pp = {}
    for n in spans_n:
        def body(st, n=n):
            cache.len.fill_(Ld)
            cad.span_forward_allowed(lay, cache, toks[:, :n], n, al2, 2, flags=cad.COMMIT_ALL | cad.LOGITS_LAST,
                                     argmax_out=o1, workspace=wsc, stream=st)
        body(stream)
        torch.cuda.synchronize()
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk, stream=cap_stream):
            body(torch.cuda.current_stream())
        gk.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(4):
            gk.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        pp[n] = e0.elapsed_time(e1) / 4
        del gk
    tau = per_step["free_step"] / 1e3
    splice_curve = {n: n * tau / pp[n] for n in spans_n}
    spans = [o[2] for o in ops if o[0] == "copy"]
    T_gen = sum(o[1] for o in ops if o[0] == "gen")
    eq2 = {"gen_decode": round(tau * T_gen, 2),
           "copy_splices": round(sum((n + 2) * tau / C.interp_s(splice_curve, n + 2) for n in spans), 2)}
    measured = {"gen_body": round(by_role.get("gen_body", 0.0), 2), "splices": round(by_role.get("splice", 0.0), 2),
                "fixed_per_op": round(eager_ms - by_role.get("gen_body", 0.0) - by_role.get("splice", 0.0), 2)}
    roles = {}
    for f in fwds:
        roles[f.role] = roles.get(f.role, 0) + 1
    res = {"workload": f"Copy-as-Decode program: Qwen2.5-7B-shaped layer + LM head 152064, {Ld}-token document, "
                       f"{T} output tokens in {len(ops)} ops ({sum(1 for o in ops if o[0] == 'copy')} copy splices), "
                       f"{len(fwds)} forwards feeding {fed} tokens incl. the grammar's structural tokens",
           "ms": round(ms, 3), "eager_ms": round(eager_ms, 3), "output_tok_s": round(T / (ms * 1e-3), 1),
           "ar_ms": round(ar_ms, 3), "ar_tok_s": round(T / (ar_ms * 1e-3), 1),
           "speedup_vs_ar": round(ar_ms / ms, 3), "forwards": roles,
           "masked_forwards": sum(1 for f in fwds if f.allowed is not None),
           "per_step_us": per_step,
           # the page's c_mask is the extra cost of masking a decode step; here a masked step
           # reads A LM-head rows instead of the vocabulary, so both step costs are reported
           "masked_step_us": round(per_step["masked_step"], 2),
           "free_step_us": round(per_step["free_step"], 2),
           "host_syncs_per_op": 0,
           "ms_by_role": {k: round(v, 2) for k, v in by_role.items()},
           "splice_s_curve": {n: round(v, 2) for n, v in splice_curve.items()},
           "ar_ms_eq1": round(tau * T, 2), "eq2_terms_ms": eq2, "measured_ms": measured,
           "realized_speedup_eq1": round(tau * T / ms, 3)}
    log(f"cad program: {ms:.1f} ms (eager {eager_ms:.1f}), AR {ar_ms:.1f} ms -> {ar_ms / ms:.2f}x; "
        f"steps {per_step}")
    del g
    return res


SAMPLE_SEED = 0x5EED_CAD0
STACK_LAYERS = 28
STACK_PREFIX = 1024
STACK_SPANS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512)


def stack_curve(a, dev, shape_key: str, program: bool = False):
    """The span forward through a whole 28-layer stack of the given shape (random weights drawn
    on the device, N(0, 0.02), bf16) after a 1024-token prefix, for N = 1 .. 512: one parallel
    forward of N tokens (full LM head, and copy-commit mode with the LM head for the last row
    only) against N autoregressive one-token forwards from the same prefix; s = AR / parallel.
    Every forward is replayed from a HIP graph.  The autoregressive times are cumulative over
    one run of 512 steps whose context grows from 1024, read at each N."""
    import numpy as np
    import torch

    from spec_verify_cad_amd import cad, synth
    from spec_verify_cad_amd import roofline as R
    from spec_verify_cad_amd.configs import CONFIGS

    shp = CONFIGS[shape_key].shape
    nl, L0 = STACK_LAYERS, STACK_PREFIX
    cap = L0 + max(STACK_SPANS) + 8
    gen = torch.Generator(device=dev)
    gen.manual_seed(4242)
    layers = []
    for l in range(nl):
        t = {}
        for name, sh in synth.weight_shapes(shp).items():
            if (name == "embed" and l > 0) or (name == "w_lm" and l < nl - 1):
                continue
            t[name] = (torch.randn(sh, generator=gen, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
        layers.append(cad.DeviceLayer.from_tensors(shp, t))
    st = cad.DeviceStack(layers)
    sc = cad.StackCache(shp, nl, 1, cap, device=dev)
    pre = torch.randint(0, shp.vocab, (1, L0), generator=gen, device=dev, dtype=torch.int32)
    cad.stack_span_forward(st, sc, pre, L0, flags=cad.KV_ONLY | cad.COMMIT_ALL)
    torch.cuda.synchronize()
    assert int(sc.len[0]) == L0
    toks = torch.randint(0, shp.vocab, (1, max(STACK_SPANS)), generator=gen, device=dev, dtype=torch.int32)
    out = torch.empty(max(STACK_SPANS), dtype=torch.int32, device=dev)
    ws = cad.alloc_workspace(max(cad.stack_span_forward_workspace(st, 1, N, cad.MASK_CAUSAL, 1, 1, cap, cad.COMMIT_ALL)
                                 for N in STACK_SPANS), device=dev)
    stream = torch.cuda.current_stream()
    cap_stream = torch.cuda.Stream()

    def graph_of(fn):
        sc.len.fill_(L0)
        fn(stream)                                         # eager warm-up of the launch shapes
        torch.cuda.synchronize()
        cap_stream.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap_stream):
            fn(torch.cuda.current_stream())
        torch.cuda.synchronize()
        return g

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        return e

    def pp(N, last, st_):
        sc.len.fill_(L0)
        cad.stack_span_forward(st, sc, toks[:, :N], N, flags=cad.COMMIT_ALL | (cad.LOGITS_LAST if last else 0),
                               argmax_out=out[:1] if last else out[:N], workspace=ws, stream=st_)

    rows = []
    for N in STACK_SPANS:
        r = {"N": N}
        for last in (False, True):
            g = graph_of(lambda s_, N=N, last=last: pp(N, last, s_))
            g.replay()
            e0 = ev()
            for _ in range(3):
                g.replay()
            e1 = ev()
            torch.cuda.synchronize()
            r["pp_last_ms" if last else "pp_ms"] = round(e0.elapsed_time(e1) / 3, 4)
            del g
        rows.append(r)
    # autoregressive: one-token forwards, 8 per graph replay, from the prefix onwards
    one = toks[:, :1]

    def steps(k, s_):
        for _ in range(k):
            cad.stack_span_forward(st, sc, one, 1, flags=cad.COMMIT_ALL, argmax_out=out[:1], workspace=ws, stream=s_)

    g1 = graph_of(lambda s_: steps(1, s_))
    g8 = graph_of(lambda s_: steps(8, s_))
    ar = {}
    sc.len.fill_(L0)
    g1.replay()                                            # warm
    sc.len.fill_(L0)
    e = [ev()]
    for _ in range(4):
        g1.replay()
        e.append(ev())
    torch.cuda.synchronize()
    for N in (1, 2, 4):
        ar[N] = e[0].elapsed_time(e[N])
    sc.len.fill_(L0)
    e = [ev()]
    for _ in range(max(STACK_SPANS) // 8):
        g8.replay()
        e.append(ev())
    torch.cuda.synchronize()
    assert int(sc.len[0]) == L0 + max(STACK_SPANS)
    for N in STACK_SPANS:
        if N >= 8:
            ar[N] = e[0].elapsed_time(e[N // 8])
    for r in rows:
        N = r["N"]
        r["ar_ms"] = round(ar[N], 4)
        r["s"] = round(ar[N] / r["pp_ms"], 2)
        r["s_copy_commit"] = round(ar[N] / r["pp_last_ms"], 2)
        nb = R.stack_forward_bytes(shp, nl, 1, N, L0)
        fl = R.stack_forward_flops(shp, nl, 1, N, L0)
        floor, bound = R.floor_us(nb, fl)
        r["floor_ms"] = round(floor / 1e3, 4)
        r["bound"] = bound
        r["frac_of_roofline"] = round(floor / 1e3 / r["pp_ms"], 4)
    log(f"{STACK_LAYERS}-layer {shape_key}: " + ", ".join(f"N={r['N']}: parallel {r['pp_ms']:.3f} ms, AR "
                                                          f"{r['ar_ms']:.2f} ms, s={r['s']}x" for r in rows))
    del g1, g8, sc
    out = {"layers": nl, "prefix": L0, "shape": shape_key, "rows": rows}
    if shape_key == "qwen7_cad_program" and program:
        out["cad_program"] = stack_program(st, dev, rows)
    del st, layers
    torch.cuda.empty_cache()
    return out


def stack_program(st, dev, rows):
    """The Copy-as-Decode program workload through the whole 28-layer 7B-shaped stack, eager
    (one stack call per forward), with an event after every forward so the time splits into
    copy splices, free generation and the grammar's structural forwards.  Beside it, the page's
    cost model on the measured curve: autoregressive regeneration L_AR = tau * T (Eq. (1)), the
    fixed-cost-free bound (Eq. (3)) and the realised speedup."""
    import numpy as np
    import torch

    from spec_verify_cad_amd import cad, synth
    from spec_verify_cad_amd import costmodel as C
    from spec_verify_cad_amd.configs import CONFIGS, cad_program_inputs
    from spec_verify_cad_amd.program import DeviceProgram

    wl = CONFIGS["qwen7_cad_program"]
    doc, ops = cad_program_inputs(wl)
    fwds = synth.cad_program_forwards(ops)
    Ld, T = len(doc), wl.extra["total_out"]
    fed = sum(f.n for f in fwds)
    cap = ((Ld + fed + 8 + 3) // 4) * 4
    sc = cad.StackCache(st.shape, st.n, 1, cap, device=dev)
    dt = torch.from_numpy(doc[None].astype(np.int32)).to(dev)
    for s0 in range(0, Ld, 2048):
        cad.stack_span_forward(st, sc, dt[:, s0:s0 + 2048], min(2048, Ld - s0), flags=cad.KV_ONLY | cad.COMMIT_ALL)
    torch.cuda.synchronize()
    prog = DeviceProgram(st, sc, doc, fwds, dev)
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(len(fwds) + 1)]
    sc.len.fill_(Ld)
    prog.enqueue(stream)                                 # warm-up run
    torch.cuda.synchronize()
    sc.len.fill_(Ld)
    evs[0].record(stream)
    for f in range(len(fwds)):                           # the same forwards, one event after each
        prog.enqueue_one(f, stream)
        evs[f + 1].record(stream)
    torch.cuda.synchronize()
    assert int(sc.len[0]) == Ld + fed
    per = [evs[f].elapsed_time(evs[f + 1]) for f in range(len(fwds))]
    total = evs[0].elapsed_time(evs[-1])
    by_role = {}
    for f, pf in enumerate(fwds):
        by_role[pf.role] = by_role.get(pf.role, 0.0) + per[f]
    cur = {r["N"]: r["s"] for r in rows}
    tau = next(r["ar_ms"] for r in rows if r["N"] == 1)
    spans = [o[2] for o in ops if o[0] == "copy"]
    b = C.bounds(spans, T, cur, m=8)
    splice_pred = tau * sum(n / C.interp_s(cur, n) for n in spans)
    res = {"workload": f"{len(ops)} ops, {len(fwds)} forwards, {fed} fed tokens through {st.n} layers",
           "ms": round(total, 2), "ms_by_role": {k: round(v, 2) for k, v in by_role.items()},
           "tau_ms": tau, "ar_ms_eq1": round(tau * T, 2), "realized_speedup": round(tau * T / total, 3),
           "bnd_exact_eq3": round(b["bnd_exact"], 3),
           "eq2_terms_ms": {"gen_decode": round(tau * b["T_gen"], 2), "copy_splices": round(splice_pred, 2),
                            "fixed_per_op_measured": round(total - by_role.get("gen_body", 0.0)
                                                           - by_role.get("splice", 0.0), 2)},
           "measured_ms": {"gen_body": round(by_role.get("gen_body", 0.0), 2),
                           "splices": round(by_role.get("splice", 0.0), 2)}}
    log(f"full-depth cad program: {res}")
    del sc, prog
    return res


def block_verify(a, dev):
    """The block-triangular multi-candidate verify on the 7B-shaped layer (random weights drawn on
    the device): a 4096-token context with planted repeats, the kappa = 5 lookup of W = 4
    recency-ranked candidates of D = 8 tokens, one 32-row block-triangular verify forward and the
    block accept scan (longest validated candidate, K/V compaction), replayed from a HIP graph.
    Reported per verify, and the forward alone against its HBM floor."""
    import numpy as np
    import torch

    from spec_verify_cad_amd import cad, synth
    from spec_verify_cad_amd import roofline as R
    from spec_verify_cad_amd.configs import CONFIGS, block_verify_context

    wl = CONFIGS["qwen7_block_verify"]
    shp, e = wl.shape, wl.extra
    W, D, n = e["W"], e["D"], e["kappa"]
    gen = torch.Generator(device=dev)
    gen.manual_seed(wl.seed)
    t = {}
    for name, sh in synth.weight_shapes(shp).items():
        t[name] = (torch.randn(sh, generator=gen, device=dev) * 0.02).to(torch.bfloat16).view(torch.int16)
    lay = cad.DeviceLayer.from_tensors(shp, t)
    ctx = block_verify_context(wl)
    Lc = len(ctx)
    cap = ((Lc + W * D + 32 + 3) // 4) * 4
    cache = cad.DeviceCache(shp, 1, cap)
    ct = torch.from_numpy(ctx[None].astype(np.int32)).to(dev)
    cad.span_forward(lay, cache, ct[:, :Lc - 1], Lc - 1, flags=cad.KV_ONLY | cad.COMMIT_ALL)
    anchor = torch.zeros(1, dtype=torch.int32, device=dev)
    cad.span_forward(lay, cache, ct[:, Lc - 1:], 1, flags=cad.COMMIT_ALL, argmax_out=anchor)
    torch.cuda.synchronize()
    assert int(cache.len[0]) == Lc
    hlen = torch.tensor([Lc], dtype=torch.int32, device=dev)
    draft = torch.zeros((1, W * D), dtype=torch.int32, device=dev)
    dlen = torch.zeros((1, W), dtype=torch.int32, device=dev)
    pred = torch.zeros(W * D, dtype=torch.int32, device=dev)
    acc, bw, ne = (torch.zeros(1, dtype=torch.int32, device=dev) for _ in range(3))
    em = torch.zeros((1, D + 1), dtype=torch.int32, device=dev)
    ws = cad.alloc_workspace(cad.span_forward_workspace(lay, 1, W * D, cad.MASK_BLOCK, W, D, cap, 0), device=dev)

    def forward(st):
        cad.span_forward(lay, cache, draft, W * D, cad.MASK_BLOCK, W, D, 0, argmax_out=pred, workspace=ws, stream=st)

    def verify(st):
        cache.len.fill_(Lc)
        cad.ngram_lookup(ct, hlen, n, W, D, 0, draft, dlen, stream=st)
        forward(st)
        cad.accept_scan(draft, 0, dlen, pred, anchor, 1, W, D, cad.MASK_BLOCK, acc, bw, em, ne, cache=cache,
                        stream=st)

    stream = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    out = {}
    for name, fn in (("verify", verify), ("forward", forward)):
        fn(stream)
        torch.cuda.synchronize()
        side.wait_stream(stream)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            for _ in range(8):
                fn(torch.cuda.current_stream())
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) * 1e3 / 40
        del g
    assert int((dlen > 0).sum()) == W
    nb = R.forward_bytes(shp, 1, W * D, Lc)
    floor, bound = R.floor_us(nb, R.forward_flops(shp, 1, W * D, Lc))
    res = {"workload": f"block-triangular verify, 7B-shaped layer: {Lc}-token context with planted repeats, "
                       f"kappa = {n} lookup of W = {W} candidates x D = {D}, one {W * D}-row verify forward and "
                       f"the block accept (K/V compaction), graph-replayed",
           "us_per_verify": round(out["verify"], 2), "forward_us": round(out["forward"], 2),
           "verified_positions_per_s": round(W * D / (out["verify"] * 1e-6), 1),
           "committed_per_verify": int(ne.item()), "alg_bytes": int(nb), "bound": bound,
           "floor_us": round(floor, 2), "forward_frac_of_roofline": round(floor / out["forward"], 4)}
    log(f"block verify: {res}")
    del cache, lay, t
    torch.cuda.empty_cache()
    return res


def stack_cost_model(stack):
    """The Copy-as-Decode cost model on the measured full-depth curves: tau = one autoregressive
    step, m* (Appendix J) with c = 0 (no host synchronisation per op, and a masked decision costs
    less than a free one), and the Eq. (3) bounds of the Copy-as-Decode program workload's copy
    spans on the 7B-shaped stack, with the full LM head and in copy-commit mode."""
    from spec_verify_cad_amd import costmodel as C
    from spec_verify_cad_amd.configs import CONFIGS, cad_program_inputs

    for sc in stack:
        rows = sc["rows"]
        tau = next(r["ar_ms"] for r in rows if r["N"] == 1)
        for key, col in (("full_lm_head", "s"), ("copy_commit", "s_copy_commit")):
            cur = {r["N"]: r[col] for r in rows}
            sc.setdefault("cost_model", {})[key] = {"tau_ms": tau, "m_star": C.m_star(cur, tau, 0.0),
                                                     "m_safe": C.m_safe(cur)}
        if sc["shape"] == "qwen7_cad_program":
            wl = CONFIGS["qwen7_cad_program"]
            _, ops = cad_program_inputs(wl)
            spans = [o[2] for o in ops if o[0] == "copy"]
            T = wl.extra["total_out"]
            for key, col in (("full_lm_head", "s"), ("copy_commit", "s_copy_commit")):
                b = C.bounds(spans, T, {r["N"]: r[col] for r in rows}, m=8)
                sc["cost_model"][key]["program_bounds"] = {k: round(v, 4) if isinstance(v, float) else v
                                                           for k, v in b.items()}
        log(f"cost model {sc['shape']}: {sc['cost_model']}")


def pld_rounds(a, layer, dev):
    """Batched prompt-lookup decoding on the 1.5B-shaped layer: 64 sequences with 32768-token
    histories (planted copies + Zipf background), 32 rounds of n-gram lookup (n = 3, one
    candidate of k = 10), an 11-row verify forward over each sequence's cache, and the accept
    scan that appends a + 1 tokens to the history and commits the cache, all enqueued without
    a host sync and replayed from a HIP graph.  Reported per round and per second."""
    import numpy as np
    import torch

    from spec_verify_cad_amd import cad
    from spec_verify_cad_amd import roofline as R
    from spec_verify_cad_amd.configs import CONFIGS, pld_contexts

    wl = CONFIGS["qwen15_pld_batch"]
    e = wl.extra
    B, Lc, n, k, rounds = e["B"], e["ctx_len"], e["n"], e["k"], e["rounds"]
    t0 = time.time()
    ctxs = pld_contexts(wl)
    stride = Lc + rounds * (k + 1) + 8
    hist_np = np.zeros((B, stride), dtype=np.int32)
    hist_np[:, :Lc] = ctxs
    hist = torch.from_numpy(hist_np).to(dev)
    hlen = torch.full((B,), Lc, dtype=torch.int32, device=dev)
    cache = cad.DeviceCache(wl.shape, B, stride)
    pre = torch.from_numpy(np.ascontiguousarray(ctxs[:, :Lc - 1])).to(dev)
    for s0 in range(0, Lc - 1, 2048):
        blk = pre[:, s0:s0 + 2048].contiguous()
        cad.span_forward(layer, cache, blk, blk.shape[1], flags=cad.KV_ONLY | cad.COMMIT_ALL)
    torch.cuda.synchronize()
    log(f"pld: contexts and 64 x {Lc - 1} prefill in {time.time() - t0:.1f}s")
    rows = torch.zeros((B, 1 + k), dtype=torch.int32, device=dev)
    dlen = torch.zeros((B, 1), dtype=torch.int32, device=dev)
    am = torch.zeros((B, 1 + k), dtype=torch.int32, device=dev)
    acc, ne = (torch.zeros(B, dtype=torch.int32, device=dev) for _ in range(2))
    em = torch.zeros((B, k + 1), dtype=torch.int32, device=dev)
    ws = cad.alloc_workspace(cad.span_forward_workspace(layer, B, 1 + k, cad.MASK_CAUSAL, 1, 1, stride, 0))

    def reset(st):
        hlen.fill_(Lc)
        cache.len.fill_(Lc - 1)

    def run(st, temperature=None):
        for _ in range(rounds):
            cad.ngram_lookup(hist, hlen, n, 1, k, 1, rows, dlen, stream=st)
            if temperature is None:
                cad.span_forward(layer, cache, rows, 1 + k, argmax_out=am, workspace=ws, stream=st)
            else:                                        # stochastic verification of the drafts
                cad.span_forward_sampled(layer, cache, rows, 1 + k, temperature, SAMPLE_SEED, draft_len=dlen,
                                         pred_out=am, workspace=ws, stream=st)
            cad.accept_scan(rows, 1, dlen, am, None, B, 1, k, cad.MASK_CAUSAL, acc, None, em, ne, ctx=hist,
                            ctx_len=hlen, ctx_cap=stride, cache=cache, stream=st)

    st = torch.cuda.current_stream()
    side = torch.cuda.Stream()

    def timed(temperature):
        reset(st)
        run(st, temperature)                             # eager warm-up
        torch.cuda.synchronize()
        side.wait_stream(st)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=side):
            run(torch.cuda.current_stream(), temperature)
        reps, total_ms, committed = 3, 0.0, 0
        for i in range(reps + 1):
            reset(st)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            g.replay()
            e1.record(st)
            torch.cuda.synchronize()
            if i:                                        # the first replay is a warm-up
                total_ms += e0.elapsed_time(e1)
                committed += int((hlen - Lc).sum())
        assert int((cache.len - (hlen - 1)).abs().max()) == 0
        del g
        return total_ms, committed, reps

    # stochastic verification at temperature 1 (the random-weight target is nearly flat, so the
    # drafts are rarely kept: this measures the cost of the sampled LM head and decision)
    s_ms, s_committed, s_reps = timed(1.0)
    sampled = {"temperature": 1.0, "us_per_round": round(s_ms * 1e3 / (s_reps * rounds), 2),
               "mean_accepted_per_round": round(s_committed / (s_reps * rounds * B) - 1, 4)}
    total_ms, committed, reps = timed(None)
    round_us = total_ms * 1e3 / (reps * rounds)
    Lmid = Lc + rounds * (k + 1) // 2                    # mean cache length over the rounds (a ~ 0)
    nb = R.pld_round_bytes(wl.shape, B, k, Lmid, Lc)
    fl = R.pld_round_flops(wl.shape, B, k, Lmid)
    floor, bound = R.floor_us(nb, fl)
    res = {"workload": f"batched PLD, 1.5B-shaped layer: {B} sequences x {Lc}-token histories, n = {n}, k = {k}, "
                       f"{rounds} rounds per replay (lookup + {1 + k}-row verify + accept, no host sync)",
           "us_per_round": round(round_us, 2),
           "verified_positions_per_s": round(B * (1 + k) / (round_us * 1e-6), 1),
           "committed_tokens_per_s": round(committed / (total_ms * 1e-3), 1),
           "mean_accepted_per_round": round(committed / (reps * rounds * B) - 1, 4),
           "alg_bytes_per_round": int(nb), "bound": bound, "floor_us": round(floor, 2),
           "frac_of_roofline": round(floor / round_us, 4),
           "sampled_verify": sampled}
    log(f"pld sampled verify: {sampled}")
    log(f"pld: {round_us:.1f} us/round, {res['verified_positions_per_s']:.0f} verified positions/s, "
        f"{bound} floor {floor:.1f} us ({floor / round_us * 100:.1f}%)")
    return res


COPY_BYTES = 1 << 29     # plain copy of the counter calibration: reads and writes 512 MiB
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "lm_head_argmax_n32_traffic.md")


def lm_traffic():
    """HBM bytes per launch of the N = 32 LM-head kernel from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE of two `--pmc-pass` runs, each scaled by a 512 MiB copy), or None
    when the kernel's sources have changed since the counters were taken."""
    import hashlib
    try:
        line = next(l for l in open(TRAFFIC_FILE) if l.startswith("traffic_record:"))
        rec = json.loads(line.split(":", 1)[1])
        h = hashlib.sha256(b"".join(open(os.path.join(ROOT, f), "rb").read() for f in rec["sources"])).hexdigest()
    except (OSError, StopIteration, ValueError, KeyError):
        return None
    return int(rec["traffic_bytes_per_launch"]) if h == rec["source_sha256"] else None


def pmc_pass(a, shp, layers, prefix, span_toks, spans, L0, cap, dev):
    """Work for a counter run (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE): four N = ROOF_N
    commits from the L0-position cache, eager, alternating weight copies, then four device copies
    of COPY_BYTES.  The copies read and write a known byte count, which scales the counters to bytes."""
    import numpy as np
    import torch

    from spec_verify_cad_amd import cad
    j = spans.index(ROOF_N) if ROOF_N in spans else 0
    N = spans[j]
    cache = cad.DeviceCache(shp, 1, cap)
    ptoks = torch.from_numpy(prefix[None].astype(np.int32)).to(dev)
    cad.span_forward(layers[0], cache, ptoks, L0, flags=cad.KV_ONLY | cad.COMMIT_ALL)
    tok = torch.from_numpy(span_toks[j][None].astype(np.int32)).to(dev)
    out = torch.empty((1, N), dtype=torch.int32, device=dev)
    for i in range(4):
        cache.len.fill_(L0)
        cad.span_forward(layers[i & 1], cache, tok, N, flags=cad.COMMIT_ALL, argmax_out=out)
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"pmc pass: 4 forwards of N={N}, 4 copies of {COPY_BYTES} bytes")


def cpu_baseline(shp, w, prefix, span_toks, spans, cap, budget_s):
    """The oracle as it stands on the host cores: copy-span commits of the sweep's spans from
    the same 2048-position cache, smallest N first, until the time budget is used."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max(int(i.get("num_threads", 1)) for i in threadpool_info()) if threadpool_info() else 1
    except Exception:  # pragma: no cover
        threads = os.cpu_count() or 1
    t0 = time.time()
    OL = O.make_layer(shp.hidden, shp.n_q_heads, shp.n_kv_heads, shp.head_dim, shp.ffn, shp.vocab, w,
                      precision=shp.dtype, rope_base=shp.rope_base, eps=shp.rms_eps)
    base = O.cache_from_tokens(OL, prefix, cap)
    log(f"oracle set-up {time.time() - t0:.1f}s")
    done, toks, secs, sweeps = [], 0, 0.0, 0
    while secs < budget_s / 2 and sweeps < 40:         # whole sweeps, at least half the budget
        for N, t in zip(spans, span_toks):
            c = base.copy()
            s = time.perf_counter()
            O.span_forward(OL, c, t)
            dt = time.perf_counter() - s
            done.append(N)
            toks += N
            secs += dt
            log(f"oracle N={N}: {dt:.2f}s")
            if secs > budget_s:
                break
        sweeps += 1
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), model)
    except OSError:  # pragma: no cover
        pass
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return {"value": round(toks / secs, 2), "unit": "committed tokens/s", "cores": threads, "kind": "oracle",
            "cpu_model": model, "nproc": avail, "host_cpus": os.cpu_count(),
            "sample": f"{len(done)} copy-span commits (N = {done}) over the 2048-position cache "
                      f"({toks} tokens, {secs:.1f}s, numpy fp64 with {threads} BLAS threads)"}


if __name__ == "__main__":
    main()
