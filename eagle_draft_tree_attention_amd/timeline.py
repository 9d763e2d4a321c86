"""Phase timeline of the two step kernels on a benchmark workload (diagnostic).

    python -m eagle_draft_tree_attention_amd.timeline --workload llama31_8b_8k

Runs the workload's tree_attention and spec_accept calls (seeded synthetic
inputs, input sets rotated as in the benchmark) with the library's timeline
buffer set (eagle_verify_set_timeline), one call at a time, and prints for
every phase mark the distribution over workgroups of its time since the
first workgroup of the launch started, pooled over the calls, plus the
derived per-workgroup phase durations.  The marks come from the device's
constant-rate real-time counter; its rate is read from the device.
"""
import argparse
import ctypes
import sys

import numpy as np

ATTN_MARKS = {0: "start", 1: "parents and query rows landed", 2: "ancestor words built",
              3: "tile loop done", 4: "partial rows stored", 5: "row statistics published",
              6: "every split of its merge rows arrived", 7: "merged rows written"}
CHUNK_MARKS = {0: "start", 1: "chunk maximum", 2: "statistics and the waves' lists", 3: "record written"}
SEL_MARKS = {0: "start", 1: "row 0: records in", 2: "row 0: normaliser", 3: "row 0 merged", 4: "rows merged",
             5: "ranked", 6: "outputs written"}
NODE_MARKS = {0: "start", 1: "target row in, its maximum", 2: "row statistics", 3: "tests and rounds done"}
FINISH_MARKS = {0: "start", 1: "outputs written"}
ACC_MARKS = {0: "start", 1: "chunk in LDS", 2: "chunk statistics", 3: "row statistics combined",
             4: "first decision", 17: "node decided", 18: "terminal preparation starts",
             19: "terminal chunk known", 20: "walk ends here", 21: "outputs written"}
SLOTS = 32


def _tick_us():
    """Microseconds per tick of the device's wall clock (hipDeviceAttributeWallClockRate, kHz)."""
    import torch
    lib = ctypes.CDLL("libamdhip64.so")
    rate = ctypes.c_int(0)
    if lib.hipDeviceGetAttribute(ctypes.byref(rate), 10017, torch.cuda.current_device()) != 0 or rate.value <= 0:
        raise RuntimeError("hipDeviceGetAttribute(hipDeviceAttributeWallClockRate) failed")
    return 1e3 / rate.value


def _stats(x):
    x = np.asarray(x, dtype=np.float64)
    if x.size == 0:
        return "n=     0"
    return (f"n={x.size:6d}  p10 {np.percentile(x, 10):7.2f}  med {np.median(x):7.2f}  "
            f"p90 {np.percentile(x, 90):7.2f}  max {x.max():7.2f}")


def _node_parallel_section(acc_rows, B, T, tick):
    print(f"\n## sa_node: {B * T} workgroups (one per node: {B} sequences x {T} nodes), "
          f"then sa_finish: {B} workgroups (one per sequence)")
    marks = {k: [] for k in NODE_MARKS}
    fmarks = {k: [] for k in FINISH_MARKS}
    durs = {"load + maximum": (0, 1), "statistics": (1, 2), "tests and rounds": (2, 3)}
    dv = {k: [] for k in durs}
    fin, ends = [], []
    kinds = {}
    for w in acc_rows:
        n, f = w[:B * T], w[B * T:B * T + B]
        t0 = n[:, 0][n[:, 0] > 0].min()
        ends.append((max(n[:, :4].max(), f[:, :2].max()) - t0) * tick)
        for k in NODE_MARKS:
            sel = n[:, k] > 0
            marks[k].extend(((n[sel, k] - t0) * tick).tolist())
        for k in FINISH_MARKS:
            sel = f[:, k] > 0
            fmarks[k].extend(((f[sel, k] - t0) * tick).tolist())
        for name, (x, y) in durs.items():
            sel = (n[:, x] > 0) & (n[:, y] > 0)
            dv[name].extend(((n[sel, y] - n[sel, x]) * tick).tolist())
        sel = (f[:, 0] > 0) & (f[:, 1] > 0)
        fin.extend(((f[sel, 1] - f[sel, 0]) * tick).tolist())
        for kd in n[n[:, 3] > 0, 30]:
            kinds[int(kd)] = kinds.get(int(kd), 0) + 1
    for k, name in NODE_MARKS.items():
        print(f"  sa_node   mark {k} {name:32s} {_stats(marks[k])}")
    for k, name in FINISH_MARKS.items():
        print(f"  sa_finish mark {k} {name:32s} {_stats(fmarks[k])}")
    print("  per-workgroup phase durations:")
    for name in durs:
        print(f"    sa_node {name:30s}     {_stats(dv[name])}")
    print(f"    sa_finish walk and sample              {_stats(fin)}")
    print(f"  last mark of the launches                     {_stats(ends)}")
    # consecutive workgroups on one compute unit (placement word: XCD index high, hardware id low;
    # the CU is the hardware id's bits 8..15, shader engine and CU number)
    gaps, per_cu = [], []
    for w in acc_rows:
        n = w[:B * T]
        live = (n[:, 0] > 0) & (n[:, 3] > 0)
        cu = (n[:, 29] >> 32) * 256 + ((n[:, 29] >> 8) & 0xFF)
        for c in np.unique(cu[live]):
            sel = np.where(live & (cu == c))[0]
            order = sel[np.argsort(n[sel, 0])]
            per_cu.append(len(order))
            for x, y in zip(order[:-1], order[1:]):
                gaps.append((n[y, 0] - n[x, 3]) * tick)
    if per_cu:
        print(f"  sa_node workgroups per compute unit            {_stats(per_cu)}")
        print(f"  sa_node gap, one workgroup's last mark to the next one's start on that unit {_stats(gaps)}")
    names = {0: "leaf", 1: "accepted", 2: "rejected"}
    print("  decided nodes by kind: " + ", ".join(f"{names.get(k, k)}: {c}" for k, c in sorted(kinds.items())))


def _fused_section(acc_rows, B, T, V, tick):
    NC = (V + 8191) // 8192
    print(f"\n## sa_fused: {B * T * NC} workgroups ({B} sequences x {T} nodes x {NC} vocabulary chunks)")
    marks = {k: [] for k in ACC_MARKS}
    rounds_hist = {}
    round_durs, first_round, terminal, sample_tail, ends = [], [], [], [], []
    for w in acc_rows:
        t0 = w[:, 0][w[:, 0] > 0].min()
        ends.append((w[:, :22].max() - t0) * tick)
        for k in ACC_MARKS:
            sel = w[:, k] > 0
            marks[k].extend(((w[sel, k] - t0) * tick).tolist())
        live = w[:, 0] > 0
        nr = w[:, 30]
        for r in np.unique(nr[live & (w[:, 17] > 0)]):
            rounds_hist[int(r)] = rounds_hist.get(int(r), 0) + int(((nr == r) & live & (w[:, 17] > 0)).sum())
        for i in range(12):
            prev = 4 + i if i > 0 else 4
            sel = (w[:, 5 + i] > 0) & (w[:, prev] > 0)
            d = (w[sel, 5 + i] - w[sel, prev]) * tick
            (first_round if i == 0 else round_durs).extend(d.tolist())
        sel = (w[:, 18] > 0) & (w[:, 19] > 0)
        terminal.extend(((w[sel, 19] - w[sel, 18]) * tick).tolist())
        sel = (w[:, 20] > 0) & (w[:, 21] > 0)
        sample_tail.extend(((w[sel, 21] - w[sel, 20]) * tick).tolist())
    for k, name in ACC_MARKS.items():
        print(f"  mark {k:2d} {name:39s} {_stats(marks[k])}")
    print("  per-workgroup phase durations:")
    print(f"    first residual round                      {_stats(first_round)}")
    print(f"    later residual rounds                     {_stats(round_durs)}")
    print(f"    terminal preparation (18 -> 19)           {_stats(terminal)}")
    print(f"    terminal sample and outputs (20 -> 21)    {_stats(sample_tail)}")
    print(f"  last mark of the launch                       {_stats(ends)}")
    print("  workgroups by residual rounds of their node: " +
          ", ".join(f"{r}: {c}" for r, c in sorted(rounds_hist.items())))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--workload", default="llama31_8b_8k")
    ap.add_argument("--temperature", type=float, default=None)
    ap.add_argument("--calls", type=int, default=40)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--sets", type=int, default=8)
    ap.add_argument("--expand", action="store_true",
                    help="also the expansion step (8-node frontier, top 4, 8 kept, draft rows of set 0)")
    args = ap.parse_args(argv)

    import torch

    import synth
    from . import Verifier, verify

    assert torch.cuda.is_available(), "the timeline needs a GPU"
    torch.cuda.set_device(0)
    by_name = {sp.name: i for i, sp in synth.CONFIGS.items()}
    spec = synth.config_spec(by_name[args.workload], temperature=args.temperature)
    inp = synth.make_inputs(spec)
    T = inp.T
    B, Hq, Hkv, D, V = spec.batch, spec.q_heads, spec.kv_heads, spec.head_dim, spec.vocab

    def to_dev(a, dt=None):
        a = np.ascontiguousarray(a)
        if dt == "bf16":
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(a).cuda()

    base = {"q": to_dev(inp.q, spec.dtype), "k": to_dev(inp.k, spec.dtype), "v": to_dev(inp.v, spec.dtype),
            "tgt": to_dev(inp.target, spec.ldtype), "drf": to_dev(inp.draft, spec.ldtype)}
    sets = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(args.sets - 1)]
    indptr, parents, tokens = to_dev(inp.kv_indptr), to_dev(inp.parents), to_dev(inp.tokens)
    ver = Verifier(B, Hq, Hkv, D, T, V, kv_dtype=spec.dtype, logits_dtype=spec.ldtype)
    out = torch.empty((B, T, Hq, D), dtype=torch.float32, device="cuda")
    aflags = torch.empty((B,), dtype=torch.int32, device="cuda")
    scale = 1.0 / np.sqrt(D)
    stream = torch.cuda.current_stream()
    sptr = int(stream.cuda_stream)
    attn_args, acc_args, keep = [], [], []
    outs = {k: torch.empty(s, dtype=torch.int32, device="cuda") for k, s in
            (("accept_len", (B,)), ("accepted_nodes", (B, T)), ("out_tokens", (B, T)), ("flags", (B,)),
             ("near_ties", (B,)))}
    for s in sets:
        a, lens = verify.tree_attention_args(s["q"], s["k"], s["v"], indptr, inp.prefix_lens, parents, scale, out,
                                             aflags)
        attn_args.append(a)
        keep.append(lens)
        c = verify.SpecAcceptArgs()
        c.batch, c.tree_rows = B, T
        c.target_logits, c.draft_logits = s["tgt"].data_ptr(), s["drf"].data_ptr()
        c.parents, c.tokens = parents.data_ptr(), tokens.data_ptr()
        c.temperature = float(spec.temperature)
        c.seed, c.offset = 0x5EED0002, 0
        for k in outs:
            setattr(c, k, outs[k].data_ptr())
        acc_args.append(c)

    words = torch.zeros(1 << 21, dtype=torch.int64, device="cuda")   # 65536 workgroups
    tick = _tick_us()
    for i in range(args.warmup):
        verify.eagle_verify_tree_attention(ver.handle, attn_args[i % len(sets)], sptr)
        acc_args[i % len(sets)].offset = i
        verify.eagle_verify_spec_accept(ver.handle, acc_args[i % len(sets)], sptr)
    torch.cuda.synchronize()
    plan = ver.last_attention_plan()

    ver.set_timeline(words)
    attn_rows, acc_rows = [], []
    for i in range(args.calls):
        j = i % len(sets)
        words.zero_()
        verify.eagle_verify_tree_attention(ver.handle, attn_args[j], sptr)
        torch.cuda.synchronize()
        attn_rows.append(words[: plan.workgroups * SLOTS].view(-1, SLOTS).cpu().numpy().copy())
        words.zero_()
        acc_args[j].offset = args.warmup + i
        verify.eagle_verify_spec_accept(ver.handle, acc_args[j], sptr)
        torch.cuda.synchronize()
        nwg = B * T * ((V + 8191) // 8192)
        acc_rows.append(words[: max(nwg, B * T + B) * SLOTS].view(-1, SLOTS).cpu().numpy().copy())
    exp_rows = []
    if args.expand:
        F, KE, ME = 8, 4, 8
        xl = sets[0]["drf"][:, :F].contiguous()
        fr = torch.zeros((B, F), dtype=torch.float32, device="cuda")
        eo = None
        for _ in range(args.warmup):
            eo = ver.tree_expand(xl, fr, 1.0, KE, ME, outputs=eo, stream=stream)
        chunk = 2048 if V <= 64 * 2048 else (4096 if V <= 64 * 4096 else 8192)
        nc_e = (V + chunk - 1) // chunk
        nslots = B * F * nc_e + B
        for i in range(args.calls):
            words.zero_()
            ver.tree_expand(xl, fr, 1.0, KE, ME, outputs=eo, stream=stream)
            torch.cuda.synchronize()
            exp_rows.append(words[: nslots * SLOTS].view(-1, SLOTS).cpu().numpy().copy())
    ver.set_timeline(None)
    ver.close()

    print(f"# workload {spec.name}: B={B} Hq={Hq} Hkv={Hkv} D={D} prefix {max(spec.prefix_lens)} tree rows {T} "
          f"vocab {V} temperature {spec.temperature}; {args.calls} calls of each kernel, one at a time, "
          f"input sets rotated ({args.sets}); clock tick {tick * 1e3:.1f} ns")
    print(f"# times in microseconds since the first workgroup of the launch started; n = workgroups that "
          f"reached the mark (over all calls)")

    # ---- tree attention
    print(f"\n## tree_attn_mfma: {plan.workgroups} workgroups, {plan.total_splits} key splits x "
          f"{plan.row_tiles} row tiles, {plan.chunk_keys} keys per split, merge inside: {plan.merge_in_kernel}")
    marks = {k: [] for k in ATTN_MARKS}
    durs = {"parents and query rows": (0, 1), "ancestors": (1, 2),
            "tile loop (from the first tile's wait)": (2, 3), "epilogue": (3, 4),
            "publish": (4, 5), "merge wait": (5, 6), "merge": (6, 7)}
    dvals = {k: [] for k in durs}
    ends, tiles = [], []
    for w in attn_rows:
        t0 = w[:, 0][w[:, 0] > 0].min()
        ends.append((w[:, :12].max() - t0) * tick)
        for k in ATTN_MARKS:
            sel = w[:, k] > 0
            marks[k].extend(((w[sel, k] - t0) * tick).tolist())
        for name, (x, y) in durs.items():
            sel = (w[:, x] > 0) & (w[:, y] > 0)
            dvals[name].extend(((w[sel, y] - w[sel, x]) * tick).tolist())
        tiles.extend(w[:, 30][w[:, 0] > 0].tolist())
    for k, name in ATTN_MARKS.items():
        print(f"  mark {k} {name:40s} {_stats(marks[k])}")
    print("  per-workgroup phase durations:")
    for name in durs:
        print(f"    {name:38s}     {_stats(dvals[name])}")
    print(f"  last mark of the launch                       {_stats(ends)}")
    print(f"  tiles per workgroup: min {min(tiles)} max {max(tiles)}")

    # ---- acceptance: node-parallel kernels (one workgroup per node, then one per sequence) or
    # the fused kernel (which marks 17, "node decided", in every workgroup; sa_node never does)
    node_parallel = (acc_rows[0][:, 17] == 0).all() and (acc_rows[0][:B * T, 3] > 0).any()
    if node_parallel:
        _node_parallel_section(acc_rows, B, T, tick)
    else:
        _fused_section(acc_rows, B, T, V, tick)
    if exp_rows:
        nwg = exp_rows[0].shape[0] - B
        print(f"\n## te_chunk + te_select: {nwg} chunk workgroups ({B} sequences x 8 frontier rows x "
              f"{nwg // (8 * B)} vocabulary chunks), then {B} selection workgroup(s); top 4, 8 kept; "
              f"times since the first chunk workgroup started")
        cm = {k: [] for k in CHUNK_MARKS}
        sm = {k: [] for k in SEL_MARKS}
        ends = []
        for w in exp_rows:
            t0 = w[:nwg, 0][w[:nwg, 0] > 0].min()
            ends.append((w[:, :8].max() - t0) * tick)
            for k in CHUNK_MARKS:
                sel = w[:nwg, k] > 0
                cm[k].extend(((w[:nwg][sel, k] - t0) * tick).tolist())
            for k in SEL_MARKS:
                sel = w[nwg:, k] > 0
                sm[k].extend(((w[nwg:][sel, k] - t0) * tick).tolist())
        for k, name in CHUNK_MARKS.items():
            print(f"  te_chunk  mark {k} {name:32s} {_stats(cm[k])}")
        for k, name in SEL_MARKS.items():
            print(f"  te_select mark {k} {name:32s} {_stats(sm[k])}")
        print(f"  last mark                                         {_stats(ends)}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
