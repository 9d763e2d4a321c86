"""Benchmark of the EAGLE verification hot path on one MI355X.

One step = one verification of one draft tree for one target layer at the
LLaMA-3.1-8B / 8K-prefix shape: tree attention (B=1, 32 q heads / 8 KV heads,
D=128, prefix 8192, 61 tree rows) followed by multi-round speculative
sampling over a 128256-token vocabulary.  Inputs are seeded synthetic data
of that shape, resident in HBM before timing starts; eight independent input
sets (over 256 MiB together) are rotated so that the 256 MiB Infinity Cache
cannot serve a step from the previous one.

Prints ONE JSON line on stdout; details go to stderr.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MODEL_LAYERS = 32   # decoder layers of the 8B model whose caches one commit call covers
METRIC = "verified tree nodes/s per layer (attn+accept) at 8B/8K shape; % of HBM peak"


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--sets", type=int, default=8, help="rotated input sets (Infinity Cache defeat)")
    ap.add_argument("--workload", default="llama31_8b_8k",
                    help="synthetic workload by name (the headline is llama31_8b_8k; serving_b32 is the "
                         "32-sequence serving batch)")
    ap.add_argument("--temperature", type=float, default=None,
                    help="override the workload's temperature (0 = greedy verification)")
    ap.add_argument("--page-size", type=int, default=0,
                    help="paged K/V: rows per page (a multiple of 64; pages at random slots of one pool); "
                         "0 = contiguous")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-commit", action="store_true",
                    help="skip timing the calls beside the step (KV commit, tree expansion)")
    ap.add_argument("--cpu-budget", type=float, default=20.0, help="seconds of oracle work to sample")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 256 MiB device copy (HBM counter calibration)")
    return ap.parse_args()


def workload_bytes(spec, T, parents):
    """Algorithmic bytes of one step (see the design notes for the formulas)."""
    B, Hq, Hkv, D, V = spec.batch, spec.q_heads, spec.kv_heads, spec.head_dim, spec.vocab
    esz = 2 if spec.dtype == "bf16" else 4
    lsz = 2 if spec.ldtype == "bf16" else 4
    L = sum(spec.prefix_lens)
    prefix_kv = 2 * L * Hkv * D * esz
    tree_kv = 2 * B * T * Hkv * D * esz
    q = B * T * Hq * D * esz
    out = B * T * Hq * D * 4
    logits = 2 * B * T * V * lsz
    internal = sum(1 for b in range(B) for n in range(T) if (parents[b] == n).any())
    # target rows + draft rows with children; greedy decoding reads no draft row
    logits_read = B * T * V * lsz + (internal * V * lsz if spec.temperature > 0 else 0)
    return {
        "metric_bytes": prefix_kv + logits,                 # prefix KV + logits read once
        "attention_bytes": prefix_kv + tree_kv + q + out,   # one tree-attention launch
        "accept_bytes": logits_read,                        # one acceptance call, leaf draft rows skipped
        "compulsory_bytes": prefix_kv + tree_kv + q + out + logits_read,
    }


def roofline(kernel, nbytes, seconds):
    """HBM roofline of one call: algorithmic bytes over its mean duration."""
    gbs = nbytes / seconds / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gbs / HBM_PEAK_GBS, "traffic": None, "algorithmic_bytes_per_launch": nbytes,
            "us_mean": seconds * 1e6}


def recorded_traffic(call, workload):
    """HBM bytes per launch measured with rocprofv3 counters (FETCH_SIZE + WRITE_SIZE,
    calibrated on a plain copy), as recorded in profiles/; None when no record exists
    or the kernel sources changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{call}_{workload}.txt")
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                rec[k.strip()] = v.strip()
    src = os.path.join(ROOT, "eagle_draft_tree_attention_amd", "csrc", rec.get("source", ""))
    if not os.path.isfile(src):
        return None
    with open(src, "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != rec.get("source_sha256"):
            return None
    try:
        return float(rec["bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, spec, budget_s):
    """The oracle, untuned, on a bounded sample of the same workload.

    The sample: `n` whole nodes (every query head) of tree attention from
    each sequence of the batch, and one acceptance call over the whole batch
    at offset 0.  It is timed best of 3 with the BLAS pool limited to one
    thread, then best of 3 with the BLAS pool's own thread count; the faster
    leg is the reported value and its thread count the reported cores.  The
    step time is extrapolated to all T nodes of every sequence.  The
    acceptance walk is scalar Python either way."""
    import numpy as np
    from oracle import accept as oacc
    from oracle import attention as oatt
    from synth import inputs as si
    from threadpoolctl import threadpool_info, threadpool_limits
    affinity = len(os.sched_getaffinity(0))
    T, Hq, Hkv, B = inp.T, spec.q_heads, spec.kv_heads, spec.batch
    g = Hq // Hkv
    scale = 1.0 / np.sqrt(spec.head_dim)
    q64 = inp.q64()
    t0 = time.perf_counter()
    kv = {(b, h): tuple(si.as_f64(x, spec.dtype) for x in si.kv_head_block(spec, T, b, h))
          for b in range(B) for h in range(Hkv)}
    tgt64, drf64 = inp.target64(), (None if spec.temperature == 0 else inp.draft64())
    setup = time.perf_counter() - t0

    def attn_nodes(b, nodes):
        for i in nodes:
            for h in range(Hq):
                k64, v64 = kv[(b, h // g)]
                oatt.node_head_output(q64[b, i, h], k64, v64, spec.prefix_lens[b], inp.parents[b], i, scale)

    def accept():
        oacc.spec_accept(tgt64, drf64, inp.parents, inp.tokens, spec.temperature, 0x5EED0000, 0)

    # calibration: one node of each sequence and one acceptance call decide
    # how many nodes per sequence fit the budget (6 timed runs share it)
    t0 = time.perf_counter()
    attn_nodes_t = []
    for b in range(B):
        t1 = time.perf_counter()
        attn_nodes(b, [T - 1])
        attn_nodes_t.append(time.perf_counter() - t1)
    t1 = time.perf_counter()
    accept()
    t_acc0 = time.perf_counter() - t1
    per_run = budget_s / 6.0
    n = int(max(1, min(T, (per_run - t_acc0) / max(sum(attn_nodes_t), 1e-9))))
    sample_nodes = [T - 1 - (j * T) // n for j in range(n)]       # spread over the tree

    def run_once():
        ta = []
        for b in range(B):
            t1 = time.perf_counter()
            attn_nodes(b, sample_nodes)
            ta.append((time.perf_counter() - t1) / n)
        t1 = time.perf_counter()
        accept()
        return sum(ta) * T + (time.perf_counter() - t1)     # one whole step, extrapolated

    # all cores: the BLAS pool as the process starts it (OMP_NUM_THREADS, the
    # host's share of cores for this GPU, when set)
    legs = {}
    for label, threads in (("one_thread", 1), ("all_cores", None)):
        with threadpool_limits(limits=threads):
            used = max([int(p.get("num_threads", 1)) for p in threadpool_info()] or [1])
            best = min(run_once() for _ in range(3))
        legs[label] = {"step_s": best, "value": (B * (T - 1)) / best, "blas_threads": used}
    # the faster leg is the baseline (small per-head products can run slower
    # on a multi-threaded BLAS pool than on one thread)
    best_leg = max(legs, key=lambda k: legs[k]["value"])
    return {
        "value": legs[best_leg]["value"],
        "unit": "nodes/s",
        "cores": legs[best_leg]["blas_threads"],
        "kind": "oracle",
        "affinity_cores": affinity,
        "legs": {k: {"value": v["value"], "blas_threads": v["blas_threads"], "step_s": v["step_s"]}
                 for k, v in legs.items()},
        "sample": (f"fp64 oracle on the host: tree attention for {n} of {T} nodes x {Hq} heads of each of "
                   f"{B} sequence(s) (extrapolated to all {T} nodes) plus one acceptance call over the batch; "
                   f"best of 3 with 1 BLAS thread and with {legs['all_cores']['blas_threads']} "
                   f"(affinity {affinity} cores), the faster leg reported; K/V setup {setup:.1f} s excluded"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import eagle_draft_tree_attention_amd as ev
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    by_name = {sp.name: i for i, sp in synth.CONFIGS.items()}
    if args.workload not in by_name:
        raise SystemExit(f"unknown workload {args.workload!r}; one of {sorted(by_name)}")
    spec = synth.config_spec(by_name[args.workload], temperature=args.temperature)
    eprint(f"[bench] generating {spec.name} inputs")
    inp = synth.make_inputs(spec)
    T = inp.T
    B, Hq, Hkv, D, V = spec.batch, spec.q_heads, spec.kv_heads, spec.head_dim, spec.vocab

    def to_dev(a, dt=None):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    kv_k, kv_v, table = inp.k, inp.v, None
    if args.page_size:
        from synth.paging import to_paged
        kv_k, kv_v, table = to_paged(inp.k, inp.v, inp.kv_indptr, inp.prefix_lens, T, args.page_size,
                                     np.random.default_rng(spec.seed))
        table = torch.from_numpy(table).cuda()
    base = {
        "q": to_dev(inp.q, spec.dtype), "k": to_dev(kv_k, spec.dtype), "v": to_dev(kv_v, spec.dtype),
        "tgt": to_dev(inp.target, spec.ldtype), "drf": to_dev(inp.draft, spec.ldtype),
    }
    sets = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(args.sets - 1)]
    indptr = to_dev(inp.kv_indptr)
    parents = to_dev(inp.parents)
    tokens = to_dev(inp.tokens)
    set_bytes = sum(t.numel() * t.element_size() for t in base.values())
    eprint(f"[bench] {args.sets} input sets x {set_bytes / 2**20:.1f} MiB resident")

    ver = ev.Verifier(B, Hq, Hkv, D, T, V, kv_dtype=spec.dtype, logits_dtype=spec.ldtype)
    scale = 1.0 / np.sqrt(D)
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
    aflags = torch.empty((B,), dtype=torch.int32, device="cuda")
    outs = {k: torch.empty(s, dtype=torch.int32, device="cuda") for k, s in
            (("accept_len", (B,)), ("accepted_nodes", (B, T)), ("out_tokens", (B, T)), ("flags", (B,)),
             ("near_ties", (B,)))}
    stream = torch.cuda.current_stream()

    # argument blocks are built once per input set, so the host stays far ahead
    # of the GPU and back-to-back launches leave no gaps
    handle = ver.handle
    sptr = int(stream.cuda_stream)
    attn_args, acc_args, keep = [], [], []
    for s in sets:
        a, lens = ev.verify.tree_attention_args(s["q"], s["k"], s["v"], indptr, inp.prefix_lens, parents, scale,
                                                out, aflags, table, args.page_size)
        attn_args.append(a)
        keep.append(lens)
        c = ev.SpecAcceptArgs()
        c.batch, c.tree_rows = B, T
        c.target_logits, c.draft_logits = s["tgt"].data_ptr(), s["drf"].data_ptr()
        c.parents, c.tokens = parents.data_ptr(), tokens.data_ptr()
        c.temperature = float(spec.temperature)
        c.seed, c.offset = 0x5EED0002, 0
        c.accept_len = outs["accept_len"].data_ptr()
        c.accepted_nodes = outs["accepted_nodes"].data_ptr()
        c.out_tokens = outs["out_tokens"].data_ptr()
        c.flags = outs["flags"].data_ptr()
        c.near_ties = outs["near_ties"].data_ptr()
        acc_args.append(c)
    call_attn = ev.verify.eagle_verify_tree_attention
    call_acc = ev.verify.eagle_verify_spec_accept

    def step(i, ev_pairs=None):
        j = i % len(sets)
        if ev_pairs is not None:
            ev_pairs[0][0].record(stream)
        call_attn(handle, attn_args[j], sptr)
        if ev_pairs is not None:
            ev_pairs[0][1].record(stream)
            ev_pairs[1][0].record(stream)
        acc_args[j].offset = i
        call_acc(handle, acc_args[j], sptr)
        if ev_pairs is not None:
            ev_pairs[1][1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # timed region 1: whole steps, back to back
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    t1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # timed region 2: same steps with events around each call (per-kernel durations)
    pairs = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(2)]
             for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(args.warmup + i, pairs[i])
    torch.cuda.synchronize()
    attn_ms = np.array([p[0][0].elapsed_time(p[0][1]) for p in pairs])
    acc_ms = np.array([p[1][0].elapsed_time(p[1][1]) for p in pairs])

    # timed region 3 (reported beside the step, not part of it): committing an
    # accepted path into the K/V caches of every layer of the model (one call,
    # in place; the caches' contents do not matter for the timing, so they are
    # left uninitialised).  The path is fixed, not the last step's outcome: the
    # root path of each sequence's deepest node whose index is not its depth,
    # so that rows do move.
    commit_ms = None
    if not args.no_commit:
        layers = MODEL_LAYERS
        fixed_len = np.zeros(B, dtype=np.int32)
        fixed_nodes = np.full((B, T), -1, dtype=np.int32)
        for b in range(B):
            par = inp.parents[b]
            depth = np.zeros(T, dtype=int)
            for i in range(1, T):
                depth[i] = depth[par[i]] + 1
            leaf = max((i for i in range(1, T) if i != depth[i]), key=lambda i: (depth[i], -i), default=0)
            path = []
            while leaf > 0:
                path.append(leaf)
                leaf = int(par[leaf])
            fixed_len[b] = len(path)
            fixed_nodes[b, :len(path)] = path[::-1]
        c_len = torch.from_numpy(fixed_len).cuda()
        c_nodes = torch.from_numpy(fixed_nodes).cuda()
        kv_shape = (layers,) + tuple(sets[0]["k"].shape)
        kl = torch.empty(kv_shape, dtype=sets[0]["k"].dtype, device="cuda")
        vl = torch.empty(kv_shape, dtype=sets[0]["v"].dtype, device="cuda")
        new_lens = torch.empty((B,), dtype=torch.int32, device="cuda")
        cflags = torch.empty((B,), dtype=torch.int32, device="cuda")
        ca, ckeep = ev.verify.kv_commit_args(kl, vl, indptr, inp.prefix_lens, c_len, c_nodes, new_lens, cflags,
                                             table, args.page_size)
        call_commit = ev.verify.eagle_verify_kv_commit
        for _ in range(5):
            call_commit(handle, ca, sptr)
        torch.cuda.synchronize()
        cpairs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            cpairs[i][0].record(stream)
            call_commit(handle, ca, sptr)
            cpairs[i][1].record(stream)
        torch.cuda.synchronize()
        commit_ms = np.array([p[0].elapsed_time(p[1]) for p in cpairs])
        alens, nodes_acc = fixed_len, fixed_nodes
        moved = sum(1 for b in range(B) for i, node in enumerate(nodes_acc[b][:max(int(alens[b]), 0)], start=1)
                    if node != i)
        assert moved > 0
        esz = 2 if spec.dtype == "bf16" else 4
        commit_bytes = layers * 2 * moved * Hkv * D * esz * 2   # K and V slices, read once and written once
        del kl, vl

    # timed region 4 (beside the step): one draft-tree expansion step at the
    # workload's vocabulary, an 8-node frontier with 4 children each, 8 kept
    # (the draft's next-token rows are the synthetic draft logits of input
    # set 0, whose first 8 rows stand in for the frontier)
    expand_ms = None
    if not args.no_commit:
        F, K_EXP, M_EXP = 8, 4, 8
        xl = sets[0]["drf"][:, :F].contiguous()
        fr = torch.zeros((B, F), dtype=torch.float32, device="cuda")
        eouts = None
        for _ in range(5):
            eouts = ver.tree_expand(xl, fr, 1.0, K_EXP, M_EXP, outputs=eouts)
        torch.cuda.synchronize()
        epairs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
        for i in range(args.steps):
            epairs[i][0].record(stream)
            ver.tree_expand(xl, fr, 1.0, K_EXP, M_EXP, outputs=eouts, stream=stream)
            epairs[i][1].record(stream)
        torch.cuda.synchronize()
        expand_ms = np.array([p[0].elapsed_time(p[1]) for p in epairs])
        expand_bytes = B * F * V * (2 if spec.ldtype == "bf16" else 4)   # the frontier's logit rows, read once

    if args.copy_probe:
        src = torch.empty(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1.0)
        torch.cuda.synchronize()
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        eprint("[bench] copy probe: 5 x 256 MiB device-to-device copies")

    nb = workload_bytes(spec, T, inp.parents)
    tree_depth = 0
    for b in range(B):
        dep = np.zeros(T, dtype=int)
        for i in range(1, T):
            dep[i] = dep[inp.parents[b][i]] + 1
        tree_depth = max(tree_depth, int(dep.max()))
    nodes = B * (T - 1)
    step_s = ms_per_step * 1e-3
    attn_us = float(np.median(attn_ms) * 1e3)
    acc_us = float(np.median(acc_ms) * 1e3)
    aplan = ver.last_attention_plan()
    attn_kernels = "tree_attn_mfma" if aplan.path == 1 else "tree_attn_fma"
    if aplan.merge_in_kernel:
        attn_kernels += " with its split merge inside"
    elif aplan.merge_workgroups > 0:
        attn_kernels += " + tree_attn_merge"
    apaths = ver.last_accept_paths()
    acc_kernels = " + ".join(name for bit, name in ((ev.ACCEPT_PATH_NODE_PARALLEL, "sa_node + sa_finish"),
                                                    (ev.ACCEPT_PATH_FUSED, "sa_fused"),
                                                    (ev.ACCEPT_PATH_THREE_KERNEL, "sa_stats + sa_pass + sa_final"))
                             if apaths & bit)
    rooflines = {
        "tree_attention": roofline(f"{attn_kernels} (one tree_attention call)",
                                   nb["attention_bytes"], float(attn_ms.mean()) * 1e-3),
        "spec_accept": roofline(f"{acc_kernels} (one spec_accept call)", nb["accept_bytes"],
                                float(acc_ms.mean()) * 1e-3),
    }
    if expand_ms is not None:
        rooflines["tree_expand"] = roofline(f"te_chunk + te_select (one tree_expand call: {F}-node frontier, "
                                            f"top-{K_EXP} each, {M_EXP} kept)", expand_bytes,
                                            float(expand_ms.mean()) * 1e-3)
    if commit_ms is not None:
        rooflines["kv_commit"] = roofline(f"kv_commit_rows (one kv_commit call over {layers} layers, "
                                          f"{moved} of {int(np.maximum(alens, 0).sum())} accepted rows move over {B} sequences)",
                                          commit_bytes, float(commit_ms.mean()) * 1e-3)
    dominant = "spec_accept" if acc_ms.mean() > attn_ms.mean() else "tree_attention"
    main_roof = dict(rooflines[dominant])
    main_roof["traffic"] = recorded_traffic(dominant, spec.name)
    result = {
        "metric": METRIC,
        "value": nodes / step_s,
        "unit": "nodes/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{spec.name}: B={B} Hq={Hq} Hkv={Hkv} D={D} "
                        f"prefix={spec.prefix_lens[0] if B == 1 else f'{min(spec.prefix_lens)}..{max(spec.prefix_lens)}'} "
                        f"tree_rows={T} ({T - 1} draft nodes, depth {tree_depth}) vocab={V} "
                        f"temperature={spec.temperature}",
            "global_batch": B,
            "seq_len": max(spec.prefix_lens),
            "parallelism": "single GPU",
            "input_sets_rotated": args.sets,
            "kv_layout": f"paged, {args.page_size} rows per page" if args.page_size else "contiguous",
        },
        "hbm_frac_metric_bytes": nb["metric_bytes"] / step_s / (HBM_PEAK_GBS * 1e9),
        "hbm_frac_compulsory_bytes": nb["compulsory_bytes"] / step_s / (HBM_PEAK_GBS * 1e9),
        "attention_us_median": attn_us,
        "attention_us_p10_p90": [float(np.percentile(attn_ms, 10) * 1e3), float(np.percentile(attn_ms, 90) * 1e3)],
        "accept_us_median": acc_us,
        "accept_us_p10_p90": [float(np.percentile(acc_ms, 10) * 1e3), float(np.percentile(acc_ms, 90) * 1e3)],
        "kv_commit_us_median": float(np.median(commit_ms) * 1e3) if commit_ms is not None else None,
        "tree_expand_us_median": float(np.median(expand_ms) * 1e3) if expand_ms is not None else None,
        "roofline": main_roof,
        "roofline_per_call": rooflines,
    }
    eprint(f"[bench] step {ms_per_step * 1e3:.1f} us  attention {attn_us:.1f} us  accept {acc_us:.1f} us")
    if not args.no_cpu_baseline:
        eprint("[bench] timing the oracle on the host (bounded sample)")
        result["cpu_baseline"] = cpu_baseline(inp, spec, args.cpu_budget)
    ver.close()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
