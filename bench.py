"""Benchmark: one Medusa decoding step on one MI355X.

Workload (default): Vicuna-7B-shaped single step, bf16 -- hidden 4096, vocab
32000, 5 Medusa heads (W1 4096x4096 + bias, W2 32000x4096), sparse 64-node
tree, one attention layer of 32 heads x 128 over a 2048-token KV cache,
greedy acceptance and accepted-path compaction.  Synthetic seeded inputs,
resident in HBM before timing starts.

A step = medusa_resid_silu + medusa_vocab_topk (the heads) -> medusa_build_tree
-> tree_attention_verify -> medusa_base_greedy -> medusa_accept.

--config 5 times the step of the 32-layer Llama-7B-shaped workload instead:
the heads and the tree as above, then the tree-verify pass through all 32
decoder layers (medusa_decoder_verify, 4096-token caches), greedy acceptance
and compaction of the accepted branch across the 32 layer caches.

Prints one JSON line: metric, value (steps/s), timing, the roofline of the
dominant kernel (algorithmic bytes per launch / measured launch time, HBM
peak 8 TB/s, counter-measured traffic when known) and the float64 oracle's
throughput on the host cores (cpu_baseline).
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth

# HBM bytes per launch of the vocabulary projection (the dominant kernel),
# from rocprofv3 FETCH_SIZE / WRITE_SIZE counters scaled by a plain-copy
# calibration (profiles/medusa_step_hbm_counters__vicuna7b_sparse64.txt).
# Valid only for the kernel sources they were taken on (sha256 prefix of
# heads.hip + common.hpp); reported as null after any change to them.
VOCAB_TRAFFIC = {"sources_sha256_16": "7571114b7ffd3c93", "read_bytes": 1311530849, "write_bytes": 128027}
# the same for the packed vocabulary projection of 8 sequences (5 heads x
# 128256 rows over 4096, the 16 bf16 head/remainder node rows per head)
# (heads.hip + skinny_mfma.hpp + common.hpp)
VOCAB_PACKED_TRAFFIC = {"sources_sha256_16": "7501fdf35a183e01", "read_bytes": 5397545134, "write_bytes": 1286601}
# the same for the gate|up projection of the 32-layer workload (one layer's
# launch: 64 x 4096 node rows against 22016 packed weight rows, unsplit, the
# SwiGLU product written in bf16)
GATE_UP_TRAFFIC = {"sources_sha256_16": "94c592ef53006fda", "read_bytes": 185374649, "write_bytes": 1409024}


def _traffic_bytes(rec, sources):
    """Counter-measured bytes of a kernel, or None once its sources changed."""
    import hashlib
    csrc = os.path.join(ROOT, "speculative_decoding_medusa_amd", "csrc")
    data = b"".join(open(os.path.join(csrc, f), "rb").read() for f in sources)
    if hashlib.sha256(data).hexdigest()[:16] != rec["sources_sha256_16"]:
        return None
    return rec["read_bytes"] + rec["write_bytes"]


def vocab_traffic_bytes():
    return _traffic_bytes(VOCAB_TRAFFIC, ("heads.hip", "common.hpp"))


def vocab_packed_traffic_bytes():
    return _traffic_bytes(VOCAB_PACKED_TRAFFIC, ("heads.hip", "skinny_mfma.hpp", "common.hpp"))


def gate_up_traffic_bytes():
    return _traffic_bytes(GATE_UP_TRAFFIC, ("skinny_mfma.hpp", "decoder.hip", "common.hpp"))
METRIC = "Medusa steps/sec + tree-verify tokens/sec (64-node tree, 7B shape), % of HBM roofline"


def tree_prior_tokens(parent, rank, alpha=0.8):
    """Tokens per step if the heads' guesses were right with the synthetic
    rank prior of the tree spec (rank r right with probability
    alpha (1 - alpha)^r at any depth, independently): the root's bonus token
    plus, for every candidate, the probability that its whole path is right."""
    import medusa_inputs as mi
    prob = [1.0] * len(parent)
    for i in range(1, len(parent)):
        prob[i] = prob[parent[i]] * mi.rank_prior(alpha, int(rank[i]))
    return 1.0 + sum(prob[1:])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=2,
                    help="workload index (2: 7B sparse-64, 3: dense-256, 4: batched, 5: 32-layer decoder verify)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true", help="replay the step as a captured HIP graph")
    ap.add_argument("--typical", action="store_true",
                    help="sampling mode: the base greedy stage also writes the node rows' scores and "
                         "medusa_typical_accept (temperature 0.7, eps 0.09, delta 0.3) replaces medusa_accept")
    ap.add_argument("--prefill-tokens", type=int, default=1024, metavar="T",
                    help="with --loop: also time the prefill of a T-token prompt (0: skip)")
    ap.add_argument("--dynamic", type=int, default=0, metavar="T",
                    help="with --config 5 --loop R: the tree topology study -- static sparse tree vs one re-chosen "
                         "every T rounds from measured acceptance (needs --planted-depths)")
    ap.add_argument("--planted-depths", type=str, default="0.8,0.7,0.6,0.5,0.4", metavar="A1,A2,..",
                    help="per-depth alphas of the planted truth for --dynamic")
    ap.add_argument("--planted", type=float, default=None, metavar="ALPHA",
                    help="with --loop: plant the base model's choices from the rank prior ALPHA (1-ALPHA)^r")
    ap.add_argument("--loop", type=int, default=0, metavar="ROUNDS",
                    help="with --config 5: time ROUNDS rounds of the device-resident generate loop (MedusaLoop), "
                         "eager and as one captured graph, and print that line instead")
    ap.add_argument("--specsample", type=int, default=0, metavar="GAMMA",
                    help="time the speculative-sampling rule alone (8 chains of GAMMA drafts over a "
                         "32000-token vocabulary) and print that line instead")
    ap.add_argument("--probes", action="store_true",
                    help="only measure the memory path and the matrix cores (per-CU read rates from an "
                         "L2-resident window, from HBM and mixed; the wide lm_head's matrix loop on constant "
                         "and random operands) and print that line instead")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device-to-device copies of MIB MiB (scale for HBM byte counters)")
    return ap.parse_args()


def read_ceiling(gib: int = 1, reps: int = 10):
    """The achievable HBM read rate for the weight streams' access pattern:
    medusa_stream_read (16-byte non-temporal loads, 4 in flight per thread,
    16,384 workgroups) over `gib` GiB, timed with HIP events on the launch
    stream."""
    import torch

    import speculative_decoding_medusa_amd as M
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda")
    buf.fill_(3)
    sink = torch.empty(16384, dtype=torch.int32, device="cuda")
    for _ in range(2):
        M.medusa_stream_read(buf, sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        M.medusa_stream_read(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = n * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    return {"GBs": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4), "kernel": "stream_read",
            "bytes": n, "workgroups": 16384, "reps": reps}


def copy_calibration(mib: int):
    """Three plain copies of a known size: the HBM byte counters of these
    dispatches convert counter units into bytes."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n, "copies": 3}), flush=True)


def probes():
    """Per-CU read rates and the matrix loop's rate, one workgroup per CU
    (256 workgroups), each timed over 5 launches with HIP events.

    Reads: a 2 MiB window every workgroup shares (plain loads: it stays in
    L2), a private 4 MiB slice of a 1 GiB buffer per workgroup (non-temporal
    loads from HBM), and 2 : 1 mixes of the two in the same waves with 6 and
    12 loads in flight per thread (the wide lm_head's node-row to weight
    bytes).  Matrix loop: 2000 iterations of 32 products of 32 x 32 x 16 per
    wave with the node fragments read from LDS, constant against random bf16
    operands."""
    import torch

    import speculative_decoding_medusa_amd as M
    n_wg = 256
    win = torch.empty(2 << 20, dtype=torch.uint8, device="cuda")
    win.fill_(1)
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    src.fill_(2)
    sink = torch.empty(n_wg, dtype=torch.int32, device="cuda")

    def timed(fn, reps=5):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps  # us per launch

    reads = {}
    for name, (wp, sp, rounds) in {"l2_window": (8, 0, 256), "hbm_slice": (0, 8, 128),
                                   "mix_2to1_6_in_flight": (4, 2, 512), "mix_2to1_12_in_flight": (8, 4, 256)}.items():
        us = timed(lambda: M.medusa_read_mix(win if wp else None, src if sp else None, wp, sp, rounds, sink, n_wg))
        per_wg = rounds * (wp + sp) * 4096
        reads[name] = {"us": round(us, 1), "GBs_per_cu": round(per_wg / (us * 1e3), 1),
                       "TBs_total": round(per_wg * n_wg / (us * 1e6), 2),
                       "hbm_TBs": round(rounds * sp * 4096 * n_wg / (us * 1e6), 2)}
    del src, win
    out = torch.empty(n_wg * 256, device="cuda")
    iters = 2000
    flops = n_wg * 4 * iters * 32 * 32768.0
    mfma = {}
    for name, rnd in (("constant_operands", False), ("random_operands", True)):
        us = timed(lambda: M.medusa_mfma_rate(rnd, iters, out, n_wg))
        mfma[name] = {"us": round(us, 1), "TFLOPs": round(flops / (us * 1e-6) / 1e12, 1),
                      "ns_per_32_products": round(us * 1e3 / iters, 1)}
    print(json.dumps({"metric": "memory path and matrix-core probes, one workgroup per CU", "n_wg": n_wg,
                      "read_ceiling": read_ceiling(), "reads": reads, "mfma_32x32x16_lds_loop": mfma,
                      "mfma_peak_TFLOPs": 2500.0}), flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Medusa step is a single-GPU path here (sharding it "
              "by vocabulary rows and attention heads is a design, not a measured mode); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.probes:
        probes()
        return
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return

    import medusa_inputs as mi
    import speculative_decoding_medusa_amd as M

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.specsample:
        return bench_specsample(args)
    cfg = mi.config(args.config)
    if args.loop:
        assert cfg.layers, "--loop runs the decoder workload (--config 5)"
        return bench_topology(args, cfg) if args.dynamic else bench_loop(args, cfg)
    if cfg.layers:
        return bench_decoder(args, cfg)
    dt_str = cfg.dtype
    t0 = time.time()
    heads = mi.gen_heads(cfg)
    att = mi.gen_attention(cfg)
    root = mi.gen_root_tokens(cfg)
    gen_s = time.time() - t0

    def dev(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.cuda()

    d = {k: dev(v) for k, v in {**heads, **att}.items()}
    root_d = dev(root)
    B, K, H, V, N, topk = cfg.B, cfg.K, cfg.H, cfg.V, cfg.N, cfg.topk
    parent, rank = cfg.tree.arrays()
    tree = M.Tree(parent, rank, K, topk)
    wdt = M.BF16 if dt_str == "bf16" else M.F32
    z = torch.empty(B, K, H, device="cuda")
    ti = torch.empty(B, K, topk, dtype=torch.int32, device="cuda")
    tv = torch.empty(B, K, topk, device="cuda")
    # from 4 sequences on, W1 and W2 in the packed layout of the MFMA head
    # products (packed once, like a weight load); fewer sequences stream the
    # row-major weights through the vector-ALU GEMVs
    w2_layout = M.PACKED if B >= 4 and wdt == M.BF16 and H % 128 == 0 else M.ROW_MAJOR
    w1 = M.pack_heads(d.pop("W1")) if w2_layout == M.PACKED else d["W1"]
    w2 = M.pack_heads(d.pop("W2")) if w2_layout == M.PACKED else d["W2"]
    ws_h = torch.empty(M.heads_workspace_size(B, H, V, K, topk, wdt, w2_layout), dtype=torch.uint8,
                       device="cuda")
    tok = torch.empty(B, N, dtype=torch.int32, device="cuda")
    pos = torch.empty_like(tok)
    o = torch.empty_like(d["q"])
    ws_a = torch.empty(M.tree_attention_workspace_size(tree, B, cfg.nH, cfg.D, max(cfg.P), wdt), dtype=torch.uint8,
                       device="cuda")
    g = torch.empty(B * N, dtype=torch.int32, device="cuda")
    # bf16 lm_head in the MFMA product's packed layout (packed once, like a
    # weight load; the float32 workload keeps the row-major GEMV)
    lm_layout = M.PACKED if wdt == M.BF16 and H % 64 == 0 else M.ROW_MAJOR
    lm = M.pack(d.pop("lm_head")) if lm_layout == M.PACKED else d["lm_head"]
    ws_g = torch.empty(M.base_greedy_workspace_size(B * N, H, V, wdt, lm_layout), dtype=torch.uint8, device="cuda")
    al = torch.empty(B, dtype=torch.int32, device="cuda")
    an = torch.empty(B, tree.max_depth + 1, dtype=torch.int32, device="cuda")
    ot = torch.empty_like(an)
    ncl = torch.empty(B, dtype=torch.int32, device="cuda")
    maxP = max(cfg.P)
    if args.typical:
        lg = torch.empty(B * N, V, device="cuda")
        u = dev(mi.uniform01((B,), cfg.seed, mi.S_TEST + 41).astype(np.float32))
        ws_t = torch.empty(M._lib.medusa_typical_accept_workspace_size(tree.handle, B), dtype=torch.uint8,
                           device="cuda")

    def step():
        M.medusa_heads_forward_tree(d["h"], w1, d["b1"], w2, topk, ti, tv, tree, root_d, d["cache_len"], tok, pos,
                                    ws=ws_h)
        M.tree_attention_verify(d["q"], d["k_tree"], d["v_tree"], d["k_cache"], d["v_cache"], d["cache_len"], maxP,
                                tree, o, ws=ws_a)
        if args.typical:
            M.medusa_base_greedy(o, lm, g, logits=lg, ws=ws_g)
            M.medusa_typical_accept(tree, tok, lg.view(B, N, V), u, al, an, ot, d["cache_len"], ncl, temperature=0.7,
                                    epsilon=0.09, delta=0.3, k_cache=d["k_cache"], v_cache=d["v_cache"], ws=ws_t)
        else:
            M.medusa_base_greedy(o, lm, g, ws=ws_g)
            M.medusa_accept(tree, tok, g.view(B, N), al, an, ot, d["cache_len"], ncl, k_cache=d["k_cache"],
                            v_cache=d["v_cache"])

    run = step
    graph = None
    if args.graph:
        graph = capture_graph(step)
        run = graph.replay

    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()

    # timed region: K steps between two synchronisations
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps

    # the other mode of the same step (one captured graph when the timed run
    # was eager, eager otherwise), K steps between two synchronisations, and
    # the median of per-step times over max(K, 100) eager steps
    other = graph.replay if graph is not None else capture_graph(step).replay
    for _ in range(args.warmup):
        other()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        other()
    e1.record()
    torch.cuda.synchronize()
    ms_other = e0.elapsed_time(e1) / args.steps
    if graph is not None:
        ms_graph, ms_eager = ms_step, None
        for _ in range(args.warmup):
            step()
        e0.record()
        for _ in range(args.steps):
            step()
        e1.record()
        torch.cuda.synchronize()
        ms_eager = e0.elapsed_time(e1) / args.steps
    else:
        ms_graph, ms_eager = ms_other, ms_step
    n_med = max(args.steps, 100)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n_med + 1)]
    ev[0].record()
    for i in range(n_med):
        step()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per_step = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(n_med))
    modes = {"eager_ms_per_step": round(ms_eager, 4), "graph_ms_per_step": round(ms_graph, 4),
             "graph_steps_per_s": round(1000.0 / ms_graph, 2),
             "eager_median_ms_per_step": round(per_step[n_med // 2], 4),
             "eager_p90_ms_per_step": round(per_step[(9 * n_med) // 10], 4), "median_over": n_med}

    # per-kernel durations: the same K steps again, every launch bracketed by
    # HIP events on the stream it runs on
    M.profiler_reset()
    M.profiler_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = M.profiler_collect()
    M.profiler_enable(False)
    kern_us = {k: 1e3 * ms / n for k, (n, ms) in prof.items()}

    def stage(*names):
        return sum(kern_us.get(n, 0.0) for n in names)

    st = {
        "heads_resid_silu": stage("resid_silu_gemv", "resid_silu_mfma"),
        "heads_vocab_topk": stage("vocab_proj_topk", "split_rows", "vocab_proj_topk_mfma", "topk_merge", "topk_tree"),
        "build_tree": stage("build_tree"),
        "tree_attention": stage("tree_attn_split", "tree_attn_mfma", "tree_attn_merge"),
        "base_greedy": stage("rmsnorm_rows", "lm_head_argmax", "argmax_merge") +
        prof.get("lm_head_gemv", (0, 0.0))[1] * 1e3 / max(args.steps, 1) +
        prof.get("lm_head_gemv_merge", (0, 0.0))[1] * 1e3 / max(args.steps, 1),
        "accept_compact": stage("accept_compact", "row_softmax_stats", "typical_accept_compact", "draw_extra"),
    }

    # roofline of the dominant kernel: the vocabulary projection of the heads
    itemsize = 2 if dt_str == "bf16" else 4
    w2_bytes = K * V * H * itemsize
    z_bytes = B * K * H * 4
    algo_bytes = w2_bytes + z_bytes + B * K * topk * 8
    # (the GEMV over row-major W2, or the MFMA product over packed W2 from 4
    # sequences on; the stored counter traffic is the GEMV's)
    vt_name = "vocab_proj_topk" if w2_layout == M.ROW_MAJOR else "vocab_proj_topk_mfma"
    vt_us = kern_us[vt_name]
    achieved = algo_bytes / (vt_us * 1e-6) / 1e9
    ceiling = read_ceiling()
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": vocab_traffic_bytes() if w2_layout == M.ROW_MAJOR else vocab_packed_traffic_bytes(),
                "kernel": vt_name,
                "bytes_per_launch": algo_bytes, "avg_us": round(vt_us, 2),
                "frac_of_read_ceiling": round(achieved / ceiling["GBs"], 4)}

    t_verify_us = st["tree_attention"]
    prior_tokens = tree_prior_tokens(*cfg.tree.arrays())
    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms_step, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dt_str,
        "data": "synthetic (seeded Philox inputs, random-init weights)",
        "config": {"workload": cfg.name, "batch": B, "hidden": H, "vocab": V, "medusa_heads": K, "topk": topk,
                   "tree_nodes": N, "attn_heads": cfg.nH, "head_dim": cfg.D, "kv_cache_len": list(cfg.P),
                   "graph": bool(args.graph), "acceptance": "typical" if args.typical else "greedy"},
        "tree_verify_tokens_per_s": round(B * N / (t_verify_us * 1e-6), 1) if t_verify_us > 0 else None,
        "tokens_per_step_under_tree_prior": round(prior_tokens, 3),
        "tokens_per_s_under_tree_prior": round(B * prior_tokens * 1000.0 / ms_step, 1),
        "stages_us": {k: round(v, 2) for k, v in st.items()},
        "kernels_us": {k: round(v, 2) for k, v in kern_us.items()},
        "stages_timing": "second pass, every launch between two HIP events: each time includes its launch's "
                         "dispatch (about 2 us more than the kernel trace for the short kernels), which the "
                         "unbracketed step overlaps with the previous kernel, so the stages sum above ms_per_step; "
                         "the tree is built by the heads' top-k merge workgroups (topk_tree, counted under "
                         "heads_vocab_topk)",
        "wall_ms_per_step": round(1e3 * wall / args.steps, 4),
        "step_modes": modes,
        "roofline": roofline,
        "hbm_read_ceiling": ceiling,
        "input_gen_s": round(gen_s, 2),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(cfg, heads, att, root)
    print(json.dumps(result), flush=True)


def capture_graph(fn):
    """fn() captured as one HIP graph (after three eager calls on the capture
    stream, which set up every lazily created library state)."""
    import torch

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    graph = torch.cuda.CUDAGraph()
    gc.collect()
    gc.disable()  # no finalizer may free device memory while the graph is captured
    try:
        with torch.cuda.graph(graph):
            fn()
    finally:
        gc.enable()
    return graph


def _cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "unknown"."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, heads, att, root):
    """The float64 oracle on the host cores, on a bounded sample of the same
    step, scaled to steps/s: one of the K heads (x K), 4 of the attention
    heads (x nH/4), 8 of the B*N greedy rows (lm_head is widened once; the
    per-row product is scaled x B*N/8)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    dt = cfg.dtype
    t = {}
    t0 = time.perf_counter()
    h = oracle.widen(heads["h"], dt)
    W1 = oracle.widen(heads["W1"][:1], dt)
    b1 = oracle.widen(heads["b1"][:1], dt)
    W2 = oracle.widen(heads["W2"][:1], dt)
    logits, _ = oracle.medusa_heads(h, W1, b1, W2)
    oracle.topk(logits, cfg.topk)
    t["heads"] = (time.perf_counter() - t0) * cfg.K
    del W1, W2
    nh = min(4, cfg.nH)
    parent, rank = cfg.tree.arrays()
    t0 = time.perf_counter()
    w = {k: oracle.widen(att[k], dt) for k in ("q", "k_tree", "v_tree", "k_cache", "v_cache")}
    kv_sel = slice(0, max(1, nh * cfg.nKV // cfg.nH))
    o = oracle.tree_attention(w["q"][:, :, :nh], w["k_tree"][:, :, kv_sel], w["v_tree"][:, :, kv_sel],
                              w["k_cache"][:, kv_sel], w["v_cache"][:, kv_sel], att["cache_len"], parent,
                              1.0 / np.sqrt(cfg.D))
    t["attention"] = (time.perf_counter() - t0) * cfg.nH / nh
    t0 = time.perf_counter()
    lm = oracle.widen(heads["lm_head"], dt)
    t_widen = time.perf_counter() - t0
    rows = np.random.default_rng(0).normal(0, 1, (8, cfg.H))
    t0 = time.perf_counter()
    oracle.base_greedy(rows, lm, 1e-6)
    t["base_greedy"] = t_widen + (time.perf_counter() - t0) * cfg.B * cfg.N / 8
    del lm
    tok = np.zeros((cfg.B, cfg.N), dtype=np.int32)
    t0 = time.perf_counter()
    for b in range(cfg.B):
        L, path, _ = oracle.accept(parent, tok[b], np.ones(cfg.N, dtype=np.int32))
    t["accept"] = time.perf_counter() - t0
    total = sum(t.values())
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    # the whole heads stage (every head, nothing scaled) on one thread: the
    # bf16 -> float64 widening, the residual-SiLU block, the projection and
    # the per-head top-k, one head at a time so one head's weights are resident
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        h = oracle.widen(heads["h"], dt)
        for k in range(cfg.K):
            lg, _ = oracle.medusa_heads(h, oracle.widen(heads["W1"][k:k + 1], dt),
                                        oracle.widen(heads["b1"][k:k + 1], dt), oracle.widen(heads["W2"][k:k + 1], dt))
            oracle.topk(lg, cfg.topk)
        heads_1t = time.perf_counter() - t0
    return {"value": round(1.0 / total, 5), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"estimate: float64 NumPy oracle on {int(threads)} threads over 1 of {cfg.K} heads, {nh} of "
                      f"{cfg.nH} attention heads and 8 of {cfg.B * cfg.N} greedy rows, each stage timed and scaled "
                      f"linearly to the full step",
            "stage_s": {k: round(v, 3) for k, v in t.items()},
            "heads_stage_single_thread": {"s": round(heads_1t, 3), "cores": 1, "scaled": False,
                                          "what": f"all {cfg.K} heads: widening, residual-SiLU, projection, top-k"},
            "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": _cpu_model()}


def bench_decoder(args, cfg):
    """The 32-layer workload: heads -> top-k -> tree -> decoder verify ->
    accept with compaction across every layer cache."""
    import numpy as np
    import torch

    import medusa_inputs as mi
    import speculative_decoding_medusa_amd as M

    def dev(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.cuda()

    t0 = time.time()
    B, K, H, V, N, topk, L = cfg.B, cfg.K, cfg.H, cfg.V, cfg.N, cfg.topk, cfg.layers
    heads = mi.gen_heads(cfg)
    d = {k: dev(v) for k, v in heads.items()}
    layers = []
    k_cache = torch.empty(L, B, cfg.nKV, cfg.Lmax, cfg.D, dtype=torch.bfloat16, device="cuda")
    v_cache = torch.empty_like(k_cache)
    for l in range(L):
        W = mi.gen_layer(cfg, l)
        layers.append(M.pack_layer({m: dev(W[m]) for m in W}))
        del W
        kc, vc = mi.gen_layer_cache(cfg, l)
        k_cache[l].copy_(dev(kc))
        v_cache[l].copy_(dev(vc))
        del kc, vc
    emb = dev(mi.gen_embedding(cfg))
    lm_head = M.pack(d.pop("lm_head"))
    root = dev(mi.gen_root_tokens(cfg))
    cache_len = dev(np.asarray(cfg.P, dtype=np.int32))
    gen_s = time.time() - t0

    parent, rank = cfg.tree.arrays()
    tree = M.Tree(parent, rank, K, topk)
    wdt = M.BF16
    z = torch.empty(B, K, H, device="cuda")
    ti = torch.empty(B, K, topk, dtype=torch.int32, device="cuda")
    tv = torch.empty(B, K, topk, device="cuda")
    ws_h = torch.empty(M.heads_workspace_size(B, H, V, K, topk, wdt), dtype=torch.uint8, device="cuda")
    tok = torch.empty(B, N, dtype=torch.int32, device="cuda")
    pos = torch.empty_like(tok)
    maxP = max(cfg.P)
    ws_d = torch.empty(M.decoder_workspace_size(tree, B, H, cfg.nH, cfg.nKV, cfg.D, cfg.ffn, V, maxP),
                       dtype=torch.uint8, device="cuda")
    g = torch.empty(B, N, dtype=torch.int32, device="cuda")
    al = torch.empty(B, dtype=torch.int32, device="cuda")
    an = torch.empty(B, tree.max_depth + 1, dtype=torch.int32, device="cuda")
    ot = torch.empty_like(an)
    ncl = torch.empty(B, dtype=torch.int32, device="cuda")

    def step():
        M.medusa_heads_forward_tree(d["h"], d["W1"], d["b1"], d["W2"], topk, ti, tv, tree, root, cache_len, tok, pos,
                                    ws=ws_h)
        M.medusa_decoder_verify(layers, emb, lm_head, tree, tok, pos, cache_len, maxP, k_cache, v_cache, cfg.nH, g,
                                ws=ws_d)
        M.medusa_accept(tree, tok, g, al, an, ot, cache_len, ncl, k_cache=k_cache, v_cache=v_cache)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    w0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_step = e0.elapsed_time(e1) / args.steps

    # the same step replayed as one captured HIP graph: the step's ~300
    # launches (9 or so per layer) cost the host more than the GPU takes to
    # run them on a slow host, so the replay is the step's reported time
    replay = capture_graph(step).replay
    for _ in range(args.warmup):
        replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        replay()
    e1.record()
    torch.cuda.synchronize()
    ms_graph = e0.elapsed_time(e1) / args.steps

    M.profiler_reset()
    M.profiler_enable(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    prof = M.profiler_collect()
    M.profiler_enable(False)
    per_launch_us = {k: 1e3 * ms / n for k, (n, ms) in prof.items()}
    per_step_us = {k: 1e3 * ms / args.steps for k, (n, ms) in prof.items()}

    # dominant kernel: the gate|up projection (the largest weight stream per
    # launch): packed weights + node rows in, the bf16 SwiGLU product out
    R = B * N
    gu_bytes = 2 * cfg.ffn * H * 2 + R * H * 2 + R * cfg.ffn * 2
    gu_us = per_launch_us["dec_gemm_gate_up"]
    achieved = gu_bytes / (gu_us * 1e-6) / 1e9
    w_layer = sum(int(np.prod(s)) for s in mi.layer_shapes(cfg).values()) * 2
    gemm_us = sum(per_step_us.get(k, 0.0) for k in ("dec_gemm_qkv", "dec_gemm_o", "dec_gemm_gate_up", "dec_gemm_down"))
    kv_bytes = L * B * cfg.nKV * (2 * maxP * cfg.D * 2)
    verify_bytes = L * w_layer + kv_bytes + V * H * 2
    verify_us = sum(v for k, v in per_step_us.items() if k not in ("resid_silu_gemv", "vocab_proj_topk", "topk_merge",
                                                                    "topk_tree", "build_tree", "accept_compact"))
    result = {
        "metric": METRIC,
        "value": round(1000.0 / ms_graph, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_graph, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded Philox inputs, random-init weights)",
        "config": {"workload": cfg.name, "batch": B, "hidden": H, "vocab": V, "medusa_heads": K, "topk": topk,
                   "tree_nodes": N, "attn_heads": cfg.nH, "head_dim": cfg.D, "kv_cache_len": list(cfg.P),
                   "decoder_layers": L, "ffn": cfg.ffn, "graph": True},
        "tree_verify_tokens_per_s": round(B * N / (verify_us * 1e-6), 1),
        "verify_us": round(verify_us, 1),
        "verify_hbm_GBs": round(verify_bytes / (verify_us * 1e-6) / 1e9, 1),
        "verify_algorithmic_bytes": verify_bytes,
        "decoder_gemm_us_per_step": round(gemm_us, 1),
        "decoder_gemm_GBs": round(L * w_layer / (gemm_us * 1e-6) / 1e9, 1),
        "kernels_us_per_step": {k: round(v, 2) for k, v in sorted(per_step_us.items(), key=lambda kv: -kv[1])},
        "step_modes": {"eager_ms_per_step": round(ms_step, 4), "eager_wall_ms_per_step": round(1e3 * wall / args.steps, 4),
                       "graph_ms_per_step": round(ms_graph, 4), "eager_steps_per_s": round(1000.0 / ms_step, 2)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": gate_up_traffic_bytes(),
                     "kernel": "dec_gemm_gate_up",
                     "bytes_per_launch": gu_bytes, "avg_us": round(gu_us, 2)},
        "input_gen_s": round(gen_s, 2),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_decoder(cfg, heads)
    print(json.dumps(result), flush=True)


def _loop_state(args, cfg, R, planted=None):
    """Weights, caches and a MedusaLoop for R rounds of the 32-layer workload,
    starting (Dmax + 1) R tokens before its prefix length; restore() puts the
    caches and the loop's state back to that start."""
    import numpy as np
    import torch

    import medusa_inputs as mi
    import speculative_decoding_medusa_amd as M

    def dev(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.cuda()

    B, K, H, N, topk, L = cfg.B, cfg.K, cfg.H, cfg.N, cfg.topk, cfg.layers
    parent, rank = cfg.tree.arrays()
    tree = M.Tree(parent, rank, K, topk)
    P0 = np.asarray(cfg.P, dtype=np.int32) - (tree.max_depth + 1) * R
    assert P0.min() >= 0, "too many rounds for the workload's prefix"
    heads = mi.gen_heads(cfg)
    d = {k: dev(v) for k, v in heads.items()}
    layers = []
    k_cache = torch.empty(L, B, cfg.nKV, cfg.Lmax, cfg.D, dtype=torch.bfloat16, device="cuda")
    v_cache = torch.empty_like(k_cache)
    for l in range(L):
        W = mi.gen_layer(cfg, l)
        layers.append(M.pack_layer({m: dev(W[m]) for m in W}))
        del W
        kc, vc = mi.gen_layer_cache(cfg, l)
        k_cache[l].copy_(dev(kc))
        v_cache[l].copy_(dev(vc))
        del kc, vc
    emb = dev(mi.gen_embedding(cfg))
    lm_head = M.pack(d.pop("lm_head"))
    state = dict(cache_len=dev(P0), h=d["h"].clone(), root_tok=dev(mi.gen_root_tokens(cfg)))
    loop = M.MedusaLoop({"w1": d["W1"], "b1": d["b1"], "w2": d["W2"]}, layers, emb, lm_head, tree, topk, k_cache,
                        v_cache, cfg.nH, state["cache_len"].clone(), state["h"].clone(), state["root_tok"].clone(),
                        max_cache_len=int(max(cfg.P)), cap=(tree.max_depth + 1) * R, planted=args.planted if planted is None else planted,
                        plant_seed=2024)
    # only the slots [P0, max P + N) change: keep them to restore the initial state
    lo, hi = int(P0.min()), int(max(cfg.P)) + N
    keep_k, keep_v = k_cache[..., lo:hi, :].clone(), v_cache[..., lo:hi, :].clone()

    def restore():
        k_cache[..., lo:hi, :].copy_(keep_k)
        v_cache[..., lo:hi, :].copy_(keep_v)
        loop.cache_len.copy_(state["cache_len"])
        loop.h.copy_(state["h"])
        loop.root_tok.copy_(state["root_tok"])
        loop.n_tokens.zero_()
        loop.restart(int(P0.max()))

    return tree, loop, layers, emb, lm_head, k_cache, v_cache, P0, restore


def bench_loop(args, cfg):
    """ROUNDS rounds of the generate loop on the 32-layer workload: heads ->
    tree -> decoder verify -> [planted choices] -> accept with compaction ->
    hand-off, nothing waiting for the host.  The caches are the workload's;
    the rounds start (Dmax + 1) * ROUNDS tokens before the workload's prefix
    length, so every round fits the caches.  Timed eagerly and as one captured
    graph of all ROUNDS rounds, each from the same initial state.

    With --planted ALPHA the base model's choices are replaced after every
    verify pass by a continuation drawn from the rank prior ALPHA (1 - ALPHA)^r
    (medusa_plant_greedy), so the random-weight model accepts candidates the
    way a trained one would: rounds accept deep branches and compact them in
    all 32 layer caches, and the tokens per round are measured, not modelled.

    The cost reading (the speculative-decoding e-book's accounting: a round
    costs the drafting plus the verify pass, in units of one plain decoding
    step, and yields E tokens): each stage of a round is timed with HIP events
    in an eager pass, and a plain decoding step -- the same decoder pass over
    a one-node tree, the root alone, plus its greedy choice -- is timed the
    same way.  c_draft = heads / plain step, c_verify = verify / plain step,
    c_rest = (tree + accept + hand-off) / plain step; modelled speedup =
    E / (c_draft + c_verify + c_rest) with E the tokens per round, against the
    measured speedup = tokens per round x plain step / round time."""
    import numpy as np
    import torch

    import medusa_inputs as mi
    import speculative_decoding_medusa_amd as M

    def dev(a):
        a = np.ascontiguousarray(a)
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16) if a.dtype == np.uint16 else torch.from_numpy(a)
        return t.cuda()

    R = args.loop
    B, K, H, N, topk, L = cfg.B, cfg.K, cfg.H, cfg.N, cfg.topk, cfg.layers
    parent, rank = cfg.tree.arrays()
    tree, loop, layers, emb, lm_head, k_cache, v_cache, P0, restore = _loop_state(args, cfg, R)
    loop.run(min(R, 2))       # warm the launch paths
    restore()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    loop.run(R)
    e1.record()
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1)
    n_eager = loop.n_tokens.cpu().numpy().copy()
    tokens_eager = loop.tokens.cpu().numpy().copy()

    restore()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    gc.collect()
    gc.disable()  # no finalizer may free device memory while the graph is captured
    try:
        with torch.cuda.graph(graph, stream=s):
            loop.run(R)
    finally:
        gc.enable()
    torch.cuda.synchronize()
    restore()
    torch.cuda.synchronize()
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    graph_ms = e0.elapsed_time(e1)
    n_graph = loop.n_tokens.cpu().numpy()
    same = bool(np.array_equal(n_graph, n_eager) and np.array_equal(loop.tokens.cpu().numpy(), tokens_eager))
    status = tree.status()

    # --- the cost reading: every stage of a round timed with events (eager)
    restore()
    torch.cuda.synchronize()
    stages = ("heads", "tree", "verify", "plant", "accept", "handoff")
    acc_ms = dict.fromkeys(stages, 0.0)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(len(stages) + 1)]
    hd = loop.heads
    for _ in range(R):
        ev[0].record()
        M.medusa_heads_forward(loop.h, hd.get("w1"), hd.get("b1"), hd["w2"], loop.topk, loop.topk_idx, loop.topk_val,
                               ws=loop.ws_heads)
        ev[1].record()
        M.medusa_build_tree(tree, loop.topk_idx, loop.root_tok, loop.cache_len, loop.node_tok, loop.node_pos)
        ev[2].record()
        M.medusa_decoder_verify(layers, emb, lm_head, tree, loop.node_tok, loop.node_pos, loop.cache_len,
                                loop.max_cache_len, k_cache, v_cache, cfg.nH, loop.greedy, hidden=loop.hidden,
                                ws=loop.ws_dec)
        ev[3].record()
        if args.planted is not None:
            M.medusa_plant_greedy(tree, loop.topk_idx, loop.cache_len, loop.greedy, cfg.V, args.planted, 2024)
        ev[4].record()
        M.medusa_accept(tree, loop.node_tok, loop.greedy, loop.accept_len, loop.accept_nodes, loop.out_tokens,
                        loop.cache_len, loop.new_cache_len, k_cache=k_cache, v_cache=v_cache)
        ev[5].record()
        M.medusa_advance(tree, loop.accept_len, loop.accept_nodes, loop.out_tokens, loop.hidden, loop.root_tok, loop.h,
                         tokens=loop.tokens, n_tokens=loop.n_tokens, new_cache_len=loop.new_cache_len,
                         cache_len=loop.cache_len)
        ev[6].record()
        torch.cuda.synchronize()
        for j, st in enumerate(stages):
            acc_ms[st] += ev[j].elapsed_time(ev[j + 1])
    stage_us = {k: round(v * 1e3 / R, 2) for k, v in acc_ms.items()}

    # --- a plain decoding step: the root alone through the same decoder, its greedy choice
    restore()
    one = M.Tree(np.array([-1], dtype=np.int32), np.array([0], dtype=np.int32), K, topk)
    tok1 = loop.root_tok.view(B, 1).clone()
    pos1 = loop.cache_len.view(B, 1).clone()
    g1 = torch.empty(B, 1, dtype=torch.int32, device="cuda")
    ws1 = M._ws(M.decoder_workspace_size(one, B, H, cfg.nH, cfg.nKV, cfg.D, cfg.ffn, cfg.V, loop.max_cache_len),
                "cuda", None)
    for _ in range(3):
        M.medusa_decoder_verify(layers, emb, lm_head, one, tok1, pos1, loop.cache_len, loop.max_cache_len, k_cache,
                                v_cache, cfg.nH, g1, ws=ws1)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(R):
        M.medusa_decoder_verify(layers, emb, lm_head, one, tok1, pos1, loop.cache_len, loop.max_cache_len, k_cache,
                                v_cache, cfg.nH, g1, ws=ws1)
    e1.record()
    torch.cuda.synchronize()
    plain_us = e0.elapsed_time(e1) * 1e3 / R
    restore()
    torch.cuda.synchronize()

    # --- prefill: a TP-token prompt through the 32 layers in chain passes of
    # 256 // B tokens, ending where the rounds start (slots below P0 are
    # overwritten: this runs last)
    TP = args.prefill_tokens
    pf = {}
    if TP > 0 and int(P0.min()) >= TP:
        prompt = torch.from_numpy(mi.uniform_int((B, TP), cfg.seed, mi.S_TEST + 77, 0, cfg.V - 1).astype(np.int32)).cuda()
        start = torch.from_numpy((P0 - TP).astype(np.int32)).cuda()
        C = max(1, min(256 // B, TP))
        chain = M.chain_tree(C)
        ws_pf = M._ws(M._lib.medusa_prefill_workspace_size(chain.handle, B, H, cfg.nH, cfg.nKV, cfg.D, cfg.ffn, cfg.V,
                                                           TP, int(P0.max()) - TP), "cuda", None)
        nt = torch.empty(B, dtype=torch.int32, device="cuda")
        hpf = torch.empty(B, H, dtype=torch.bfloat16, device="cuda")
        times = []
        for rep_ in range(4):
            loop.cache_len.copy_(start)
            torch.cuda.synchronize()
            e0.record()
            M.medusa_prefill(layers, emb, lm_head, chain, prompt, loop.cache_len, int(P0.max()) - TP, k_cache, v_cache,
                             cfg.nH, nt, hpf, ws=ws_pf)
            e1.record()
            torch.cuda.synchronize()
            if rep_ > 0:
                times.append(e0.elapsed_time(e1))
        ok = bool(np.array_equal(loop.cache_len.cpu().numpy(), P0))
        ms = sum(times) / len(times)
        pf = {"prompt_tokens": TP, "tokens_per_pass": C, "passes": -(-TP // C), "ms": round(ms, 3),
              "tokens_per_s": round(B * TP / (ms * 1e-3), 1), "cache_len_advanced": ok}

    expected = tree_prior_tokens(parent, rank)
    rounds_s = R / (graph_ms * 1e-3)
    tpr = float(n_graph.sum()) / (B * R)
    round_us = graph_ms * 1e3 / R
    c_draft = stage_us["heads"] / plain_us
    c_verify = stage_us["verify"] / plain_us
    c_rest = (stage_us["tree"] + stage_us["accept"] + stage_us["handoff"]) / plain_us
    result = {
        "metric": "Medusa generate rounds/sec (32-layer Llama-7B-shaped decoder, device-resident loop)",
        "value": round(rounds_s, 2),
        "unit": "rounds/s",
        "n_gpus": 1,
        "rounds": R,
        "higher_is_better": True,
        "dtype": "bf16",
        "data": "synthetic (seeded Philox inputs, random-init weights)" +
                (f"; base-model choices planted from the rank prior alpha={args.planted}" if args.planted is not None
                 else ""),
        "config": {"workload": cfg.name + "_loop", "batch": B, "tree_nodes": N, "decoder_layers": L,
                   "start_prefix": P0.tolist(), "max_prefix": [int(p) for p in cfg.P],
                   "acceptance": "planted" if args.planted is not None else "model"},
        "ms_per_round_graph": round(graph_ms / R, 4),
        "ms_per_round_eager": round(eager_ms / R, 4),
        "graph_replay_matches_eager": same,
        "tree_status_word": status,
        "tokens_per_round_measured": round(tpr, 3),
        "tokens_per_s_measured": round(float(n_graph.sum()) / (graph_ms * 1e-3), 1),
        "tokens_per_round_under_tree_prior": round(expected, 3),
        "prefill": pf,
        "cost_reading": {
            "stage_us": stage_us,
            "plain_decode_step_us": round(plain_us, 2),
            "plain_decode_tokens_per_s": round(B * 1e6 / plain_us, 1),
            "c_draft": round(c_draft, 4), "c_verify": round(c_verify, 4), "c_rest": round(c_rest, 4),
            "speedup_modelled": round(tpr / (c_draft + c_verify + c_rest), 3),
            "speedup_modelled_prior": round(expected / (c_draft + c_verify + c_rest), 3),
            "speedup_measured": round(tpr * plain_us / round_us, 3),
        },
    }
    print(json.dumps(result), flush=True)


def bench_topology(args, cfg):
    """The tree topology study, dynamic variant: the same 32-layer loop on the
    same planted truth -- base-model choices drawn with per-depth alphas that
    fall with depth (the e-book's caveat: once a guess slips, later positions
    slip more) -- run twice from the same state, R rounds each: with the
    static sparse 64-node tree (chosen for 0.8 at every depth), and with a
    64-node tree re-chosen every T rounds from the acceptance counts the
    rounds gathered so far (medusa_accept_stats -> per-depth rank estimates ->
    medusa_tree_select).  Reports tokens per round and tokens/s of both (wall
    time including the re-selections), and the expected tokens per round of
    the static tree, the final dynamic tree and the best 64-node tree under
    the true prior."""
    import numpy as np
    import torch

    import medusa_inputs as mi
    import speculative_decoding_medusa_amd as M

    R, T = args.loop, args.dynamic
    alphas = [float(a) for a in args.planted_depths.split(",")]
    B, K, topk, N = cfg.B, cfg.K, cfg.topk, cfg.N
    tree, loop, layers, emb, lm_head, k_cache, v_cache, P0, restore = _loop_state(args, cfg, R, planted=alphas)
    static = tree

    def prior_matrix(al):
        return np.array([[mi.rank_prior(al[min(d, len(al) - 1)], r) for r in range(topk)] for d in range(K)])

    def expected(parent, rank, acc):
        e = 1.0
        depth = np.zeros(len(parent), int)
        prod = np.ones(len(parent))
        for i in range(1, len(parent)):
            depth[i] = depth[parent[i]] + 1
            prod[i] = prod[parent[i]] * acc[depth[i] - 1][rank[i]]
            e += prod[i]
        return e

    truth = prior_matrix(alphas)
    assumed = prior_matrix([0.8])
    best = M.tree_select(truth, N)

    def run(dynamic):
        restore()
        loop.set_tree(static)
        loop.stats = torch.zeros(K, topk + 1, dtype=torch.int32, device="cuda") if dynamic else None
        loop.run(2)                       # warm the launch paths
        restore()
        if dynamic:
            loop.stats.zero_()
        torch.cuda.synchronize()
        trees, history = [static], []
        t0 = time.perf_counter()
        done = 0
        while done < R:
            n = min(T if dynamic else R, R - done)
            loop.run(n)
            done += n
            if dynamic and done < R:
                c = loop.stats.cpu().numpy().astype(np.float64)        # waits for the rounds
                a0 = 4.0                                               # pseudo-observations of the assumed prior
                tot = c.sum(axis=1, keepdims=True)
                acc = (c[:, :topk] + a0 * assumed) / (tot + a0)
                parent, rank = M.tree_select(acc, N)
                nt = M.Tree(parent, rank, K, topk)
                loop.set_tree(nt)
                trees.append(nt)
                history.append(round(expected(parent, rank, truth), 3))
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ntok = int(loop.n_tokens.sum().item())
        last = trees[-1]
        res = {"tokens_per_round": round(ntok / (B * R), 3), "tokens_per_s": round(ntok / wall, 1),
               "ms_per_round_wall": round(wall * 1e3 / R, 4), "tree_status_word": last.status(),
               "expected_tokens_final_tree": None}
        if dynamic:
            res["reselections"] = len(history)
            res["expected_tokens_per_reselection"] = history
        return res, trees

    # alternate the two (static, dynamic, static, dynamic) so both see the same
    # warm state; the figures are the means of the two runs of each
    runs = {False: [], True: []}
    trees = None
    for dynamic in (False, True, False, True):
        res, tr = run(dynamic)
        runs[dynamic].append(res)
        if dynamic:
            trees = tr

    def mean_of(rs):
        out = dict(rs[-1])
        for k in ("tokens_per_round", "tokens_per_s", "ms_per_round_wall"):
            out[k] = round(sum(r[k] for r in rs) / len(rs), 4)
        out["runs_tokens_per_s"] = [r["tokens_per_s"] for r in rs]
        return out

    st, dy = mean_of(runs[False]), mean_of(runs[True])
    restore()
    loop.set_tree(static)
    sp, sr = cfg.tree.arrays()
    st["expected_tokens_final_tree"] = round(expected(sp, sr, truth), 3)
    if len(trees) > 1:
        dy["expected_tokens_final_tree"] = dy["expected_tokens_per_reselection"][-1]
    result = {
        "metric": "tree topology study: tokens/s of the 32-layer loop, static sparse 64-node tree vs a 64-node tree "
                  "re-chosen from measured acceptance",
        "value": dy["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "rounds": R, "reselect_every": T,
        "higher_is_better": True, "dtype": "bf16",
        "data": f"synthetic; base-model choices planted with per-depth alphas {alphas}",
        "config": {"workload": cfg.name + "_topology", "batch": B, "tree_nodes": N, "decoder_layers": cfg.layers},
        "static_sparse64": st, "dynamic": dy,
        "expected_tokens_static_tree_under_truth": st["expected_tokens_final_tree"],
        "expected_tokens_best_tree_under_truth": round(expected(best[0], best[1], truth), 3),
        "expected_tokens_static_tree_as_assumed": round(expected(sp, sr, assumed), 3),
        "dynamic_over_static_tokens_per_s": round(dy["tokens_per_s"] / st["tokens_per_s"], 4),
    }
    print(json.dumps(result), flush=True)


def bench_specsample(args):
    """The speculative-sampling rule alone: 8 chains of GAMMA drafts over a
    32000-token vocabulary (seeded target/draft rows, drafts and uniforms),
    timed with HIP events over K calls; the bytes are the rows a call must
    read at least (the draft tests' values and the stopping row's p and q)."""
    import numpy as np
    import torch

    import medusa_inputs as mi
    import speculative_decoding_medusa_amd as M
    B, G, V, seed = 8, args.specsample, 32000, 905
    lp = mi.normal((B, G + 1, V), seed, mi.S_TEST + 61, 1.5, "f32")
    lq = lp[:, :G] + mi.normal((B, G, V), seed, mi.S_TEST + 62, 0.7, "f32")
    sm = lambda x: np.exp(x - x.max(-1, keepdims=True)) / np.exp(x - x.max(-1, keepdims=True)).sum(-1, keepdims=True)
    p = torch.from_numpy(sm(lp).astype(np.float32)).cuda()
    q = torch.from_numpy(sm(lq).astype(np.float32)).cuda()
    drafts = torch.from_numpy(mi.uniform_int((B, G), seed, mi.S_TEST + 63, 0, V - 1).astype(np.int32)).cuda()
    ua = torch.from_numpy(mi.uniform01((B, G), seed, mi.S_TEST + 64)).cuda()
    ur = torch.from_numpy(mi.uniform01((B, G + 1), seed, mi.S_TEST + 65)).cuda()
    n = torch.empty(B, dtype=torch.int32, device="cuda")
    out = torch.empty(B, G + 1, dtype=torch.int32, device="cuda")
    for _ in range(args.warmup):
        M.medusa_speculative_sample(p, q, drafts, ua, ur, n, out)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(args.steps):
        M.medusa_speculative_sample(p, q, drafts, ua, ur, n, out)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / args.steps
    nn = n.cpu().numpy()
    row_bytes = int(sum(V * 4 * (2 if k < G else 1) for k in nn))
    print(json.dumps({"metric": "speculative-sampling rule, us per call (8 chains, 32000-token rows)",
                      "value": round(us, 2), "unit": "us", "higher_is_better": False, "gamma": G, "batch": B,
                      "vocab": V, "accepted": nn.tolist(), "row_GBs": round(row_bytes / (us * 1e-6) / 1e9, 1),
                      "data": "synthetic (seeded Philox rows, drafts and uniforms)"}), flush=True)


def cpu_baseline_decoder(cfg, heads):
    """The float64 oracle on the host cores over a bounded sample of the
    32-layer step, scaled to steps/s: one of the K heads (x K); one decoder
    layer at full width over the 64 tree tokens with 4 of the 32 attention
    heads computed exactly (x 8 for attention, the layer x 32); lm_head over 8
    of the 64 rows (x 8)."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import medusa_inputs as mi
    import oracle
    t = {}
    dt = cfg.dtype
    t0 = time.perf_counter()
    h = oracle.widen(heads["h"], dt)
    logits, _ = oracle.medusa_heads(h, oracle.widen(heads["W1"][:1], dt), oracle.widen(heads["b1"][:1], dt),
                                    oracle.widen(heads["W2"][:1], dt))
    oracle.topk(logits, cfg.topk)
    t["heads"] = (time.perf_counter() - t0) * cfg.K
    parent, _ = cfg.tree.arrays()
    W = mi.gen_layer(cfg, 0)
    kc, vc = mi.gen_layer_cache(cfg, 0)
    t0 = time.perf_counter()
    Wl = {m: oracle.widen(W[m], dt) for m in W}
    r = np.random.default_rng(0)
    x = r.normal(0, 1, (cfg.B, cfg.N, cfg.H))
    n = oracle.round_bf16(oracle.rmsnorm(x, 1e-6))
    mats = [n @ Wl[m].T for m in ("wq", "wk", "wv")]
    o = x @ Wl["wo"].T
    a = oracle.round_bf16(oracle.silu(n @ Wl["w_gate"].T) * (n @ Wl["w_up"].T))
    x = x + a @ Wl["w_down"].T
    t_lin = time.perf_counter() - t0
    nh = 4
    D = cfg.D
    q = mats[0].reshape(cfg.B, cfg.N, cfg.nH, D)[:, :, :nh]
    k = mats[1].reshape(cfg.B, cfg.N, cfg.nKV, D)[:, :, :nh]
    v = mats[2].reshape(cfg.B, cfg.N, cfg.nKV, D)[:, :, :nh]
    t0 = time.perf_counter()
    oracle.tree_attention(q, k, v, oracle.widen(kc[:, :nh], dt), oracle.widen(vc[:, :nh], dt),
                          np.asarray(cfg.P), parent, 1.0 / np.sqrt(D))
    t_att = (time.perf_counter() - t0) * cfg.nH / nh
    t["decoder_layers"] = (t_lin + t_att) * cfg.layers
    del Wl, W, kc, vc
    t0 = time.perf_counter()
    lm = oracle.widen(heads["lm_head"], dt)
    oracle.base_greedy(r.normal(0, 1, (8, cfg.H)), lm, 1e-6)
    t["lm_head"] = (time.perf_counter() - t0) * cfg.B * cfg.N / 8
    total = sum(t.values())
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    return {"value": round(1.0 / total, 6), "unit": "steps/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 NumPy oracle: 1 of {cfg.K} heads; one full-width decoder layer (4 of {cfg.nH} "
                      f"attention heads exact) scaled to {cfg.layers} layers; 8 of {cfg.B * cfg.N} lm_head rows; "
                      "each part timed and scaled linearly",
            "stage_s": {k: round(v, 3) for k, v in t.items()}, "host_cpus": len(os.sched_getaffinity(0)),
            "cpu_model": _cpu_model()}


if __name__ == "__main__":
    main()
