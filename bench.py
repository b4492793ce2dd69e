#!/usr/bin/env python3
"""Benchmark of the Token Recycling step hot path on one MI355X.

One step = tr_tree_attn (tree attention of the merged sequence against the
prefix cache, one layer) + tr_step (top-k of every node's logits,
verification, update of M, commit of the accepted path, retrieval of the
next tree).  Default workload: the large-vocabulary batch (32 independent
sequences, V=128256, k=8, 81-node depth-6 trees, GQA 32/8 x d=128 bf16,
prefixes uniform in [1024, 4096], 128 steps), the largest configuration
that fits one GPU; `--workload` picks another.

Protocol: a record pass runs the whole trajectory once and keeps every
step's synthetic inputs (queries, tree keys/values, logits with the planted
continuation of that step's tree) in HBM.  The state is then reset to the
start and the same trajectory is replayed: `--warmup` steps untimed, then
`--steps` steps timed.  Passes over the same steps:
  * stream replay: launched one by one from Python between two device
    synchronisations, HIP events around every call (per-call figures);
  * graph replay (the headline `value`): the timed steps captured once into
    a HIP graph and replayed between two synchronisations;
  * warm kernel timing: the library's launch profiling on (two HIP events
    around every kernel, on the stream it runs on);
  * cold kernel timing: the same, with a 1 GiB scrub buffer written before
    every library call, so no kernel finds its inputs in the 256 MB
    Infinity Cache or the L2s; the roofline is taken from this pass.
Every replay must end in the record pass's state (checked).  Also measured:
the achievable streaming-read bandwidth (tr_read_probe over 2 GiB, a sanity
denominator), and the CPU oracle on the same trajectory (cpu_baseline).
Prints one JSON line.
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TR steps/sec (retrieve+tree-attn+verify+top-k update); achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}     # dense matrix-core peaks
SCRUB_BYTES = 1 << 30                                  # cold pass: written before every call
PROBE_BYTES = 2 << 30                                  # read probe buffer


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: the workload's)")
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", default="largevocab")
    ap.add_argument("--temperature", type=float, default=0.0,
                    help="0: greedy verification (tr_step); above 0: verification by sampling "
                         "at this temperature (tr_step_sample, seeded uniforms)")
    ap.add_argument("--page-size", type=int, default=0,
                    help="0: contiguous prefix cache; else a paged cache with pages of this many "
                         "rows in shuffled order (tr_tree_attn_paged, tr_step_paged)")
    ap.add_argument("--lmhead", type=int, default=0, metavar="H",
                    help="0: the step takes logits; else it takes hidden states [B][T][H] and a "
                         "seeded output embedding [V][H] through the fused LM head "
                         "(tr_step_lmhead); the unfused product + tr_step is timed beside it")
    ap.add_argument("--launch", choices=("graph", "stream"), default="graph",
                    help="graph: the timed steps are captured once into a HIP graph and replayed "
                         "(value); stream: launched one by one from Python.  Both are timed; "
                         "per-call figures come from the stream pass")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache kernel timing")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="budget of the CPU oracle baseline, split between a 1-thread and an "
                         "all-threads run (0 disables it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB five times (reference for "
                         "the FETCH_SIZE / WRITE_SIZE counters) and exit")
    return ap.parse_args()


# Kernels of the library (profiling names), the kernel name prefix they
# carry in counter records, and the sources they are built from: a counter
# record taken on other sources of a kernel is stale for that kernel.
KERNEL_SOURCES = {
    "attn_prefix": ("attn_prefix", ["k_attn.hip", "dev_common.h", "tr_internal.h"]),
    "attn_combine": ("attn_merge", ["k_attn.hip", "dev_common.h", "tr_internal.h"]),
    "topk": ("topk_kernel", ["k_topk.hip", "select.h", "tail.h", "sample.h", "dev_common.h",
                             "tr_internal.h"]),
    "step": ("step_kernel", ["k_step.hip", "select.h", "tail.h", "dev_common.h", "tr_internal.h"]),
}
STEP_MAX_V = 32768          # the few-row step kernel: fewer than 256 rows of at most this many logits


def record_kernel(w, kernel):
    """The counter-record name of timed kernel `kernel` on workload w: the
    step's top-k launch is the few-row step kernel when B*T < 256 and
    V <= 32768 (greedy verification), the general top-k kernel otherwise."""
    if kernel == "topk" and w.B * w.T < 256 and w.V <= STEP_MAX_V:
        return "step"
    return kernel


def kernel_sources_sha256(kernel):
    """Hash of the HIP sources `kernel` is built from."""
    import hashlib
    d = os.path.join(ROOT, "draft_tree_retrieval_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(KERNEL_SOURCES[kernel][1]):
        with open(os.path.join(d, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def counter_record(kind, workload, kernel):
    """The committed counter record `profiles/<kind>_<workload>.json` entry
    of `kernel`, or None when there is none or the kernel's sources changed
    since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}.json")
    if kernel not in KERNEL_SOURCES or not os.path.exists(path):
        return None, None
    with open(path) as f:
        rec = json.load(f)
    prefix = KERNEL_SOURCES[kernel][0]
    if rec.get("sources_sha256", {}).get(prefix) != kernel_sources_sha256(kernel):
        return None, rec
    return rec.get("per_kernel", {}).get(prefix), rec


def measured_traffic(workload, kernel):
    """HBM bytes per launch of `kernel` from the committed counter record of
    this workload (a FETCH_SIZE run and a WRITE_SIZE run, each scaled by what
    it reads for a plain copy of known size), or None when there is no
    record or the kernel changed since it was taken."""
    k, rec = counter_record("traffic", workload, kernel)
    if not k:
        return None
    cal = rec.get("copy_calibration", {})
    if not cal:
        return None
    return int(round((k["FETCH_SIZE"] * cal["fetch_scale"] + k["WRITE_SIZE"] * cal["write_scale"]) * 1024))


def measured_mfma(workload, kernel):
    """Matrix-core figures of `kernel` from the committed counter record:
    busy fraction = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE x SIMDs) and
    the matrix-core work per launch (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512
    flops), or None."""
    k, rec = counter_record("mfma", workload, kernel)
    if not k:
        return None
    return {"busy_frac": k["busy_frac"], "mops_flops": k["mops_flops"]}


def copy_calibration(mib):
    """A plain copy kernel of known size: each launch reads and writes
    exactly mib MiB, so HBM counters read on it give their scale."""
    import torch
    src = torch.ones(mib << 18, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_per_launch": mib << 20, "launches": 5}), flush=True)


def read_probe(tr):
    """Achievable streaming-read bandwidth: the median of five
    tr_read_probe launches over 2 GiB (GB/s)."""
    import torch
    src = torch.ones(PROBE_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    tr.tr_read_probe(src, sink)
    torch.cuda.synchronize()
    tr.tr_profile_enable(True)
    for _ in range(5):
        tr.tr_read_probe(src, sink)
    ms = sorted(m for n, m in tr.tr_profile_read() if n == "read_probe")
    tr.tr_profile_enable(False)
    del src
    return round(PROBE_BYTES / (ms[len(ms) // 2] * 1e-3) / 1e9, 1)


def cpu_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count()
    return model, os.cpu_count(), affinity


def _oracle_run(w, inputs, init_host, seconds, temperature, threads):
    """The CPU oracle, as it stands, stepping sequence 0 of the trajectory
    with `threads` BLAS threads (None: the pool's default) for about
    `seconds`: per-phase seconds and the steps done."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import tr_oracle as O
    phases = ["attention", "topk", "verify", "update", "commit", "retrieve"]
    acc = {p: 0.0 for p in phases}
    with threadpool_limits(limits=threads):
        used = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        t = O.template_from_levels(w.levels)
        b = 0
        M = init_host.M[b].numpy().astype(np.int64).copy()
        kc = init_host.k_cache[b].float().numpy().copy()
        vc = init_host.v_cache[b].float().numpy().copy()
        P = int(init_host.prefix_len[b])
        tok = O.retrieve(t, M, int(init_host.root[b]))
        done, elapsed = 0, 0.0
        for (q, kt, vt, z, U) in inputs:
            if elapsed >= seconds:
                break
            qh, kth, vth, zh = (x[b].float().cpu().numpy() for x in (q, kt, vt, z))
            uh = U[b].double().cpu().numpy() if U is not None else None
            c0 = time.perf_counter()
            O.tree_attention(t, qh, kth, vth, kc, vc, P)
            c1 = time.perf_counter()
            top = O.topk_rows(zh, w.k)
            c2 = time.perf_counter()
            v = (O.verify_sample(t, tok, zh, temperature, uh) if temperature > 0
                 else O.verify(t, tok, top[:, 0]))
            c3 = time.perf_counter()
            O.update(M, tok, top)
            c4 = time.perf_counter()
            P = O.commit(kc, vc, kth, vth, P, v.path)
            c5 = time.perf_counter()
            tok = O.retrieve(t, M, v.bonus)
            c6 = time.perf_counter()
            for p, dt in zip(phases, (c1 - c0, c2 - c1, c3 - c2, c4 - c3, c5 - c4, c6 - c5)):
                acc[p] += dt
            elapsed += c6 - c0
            done += 1
    return acc, done, elapsed, used


def cpu_baseline(w, inputs, init_host, seconds, temperature=0.0):
    """The CPU oracle (float64 numpy, as it stands) on the first steps of
    the same trajectory, sequence 0, once with one BLAS thread and once with
    the pool's default thread count; a step of the batch is B sequences'
    work, so each rate is the sequence rate divided by B."""
    model, nproc, affinity = cpu_info()
    runs = {}
    for name, threads in (("one_thread", 1), ("all_threads", None)):
        acc, done, elapsed, used = _oracle_run(w, inputs, init_host, seconds / 2, temperature, threads)
        runs[name] = {"value": round(done / elapsed / w.B, 4) if elapsed else None, "threads": used,
                      "steps": done, "seconds": round(elapsed, 2),
                      "per_phase_ms": {p: round(s * 1e3 / max(done, 1), 3) for p, s in acc.items()}}
    best = runs["all_threads"]
    return {"value": best["value"], "unit": "steps/s", "cores": best["threads"], "kind": "oracle",
            "sample": f"first {best['steps']} steps of the same trajectory, sequence 0 of {w.B} "
                      f"(tree attention + top-k + verify + update + commit + retrieve, float64 "
                      f"numpy), {best['seconds']} s of CPU time; value = that rate / {w.B} "
                      f"(steps of the whole batch)",
            "one_thread": runs["one_thread"], "all_threads": runs["all_threads"],
            "nproc": nproc, "affinity_cpus": affinity, "cpu_model": model}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(sequences shard across GPUs with no exchange; see the design notes).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from draft_tree_retrieval_amd import tr
    from draft_tree_retrieval_amd.loop import TRDecoder
    from synth import workloads as W

    tr.load()
    w = W.WORKLOADS[args.workload]
    steps = args.steps if args.steps is not None else w.steps
    total = args.warmup + steps
    dev = "cuda"
    cap = w.cap(total)
    if args.page_size:
        cap = -(-cap // args.page_size) * args.page_size
    init = W.initial_state(w, dev, cap=cap)
    init_host = init.to("cpu")
    tree = tr.Tree.from_levels(w.levels, w.k)

    temp = args.temperature
    Hl = args.lmhead
    if Hl:
        gw = torch.Generator(device=dev).manual_seed(w.seed + 91)
        W_out = (torch.randn((w.V, Hl), generator=gw, device=dev) / Hl ** 0.5).to(torch.bfloat16)
        lm_ws = {}

    def step(dec, z, kt, vt, U):
        if temp > 0:
            dec.step_sample(z, kt, vt, temp, U)
        elif Hl:
            key = id(dec)
            if key not in lm_ws:
                lm_ws[key] = tr.new_lmhead_workspace(w.B * w.T, w.V, w.k)
            tr.tr_step_lmhead(tree, z, W_out, dec.M, dec.tree_tok, dec.root_tok, dec.accept_len,
                              dec.accept_path, dec.emitted, lm_ws[key], kt, vt, dec.k_cache,
                              dec.v_cache, dec.prefix_len, dec.topk, dec.update)
        else:
            dec.step(z, kt, vt)

    def fresh_decoder():
        st = init.clone()
        return TRDecoder(tree, st.M, st.k_cache, st.v_cache, st.prefix_len, st.root, Hq=w.Hq,
                         page_size=args.page_size or None)

    # ---- record pass: the trajectory's inputs, kept in HBM
    t0 = time.time()
    dec = fresh_decoder()
    out = torch.empty((w.B, w.T, w.Hq, w.d), dtype=w.kv_dtype, device=dev)
    ug = torch.Generator(device=dev).manual_seed(w.seed + 77)
    inputs, prefix_hist, accepted = [], [], []
    for s in range(total):
        q, kt, vt = W.step_qkv(w, s, dev)
        if Hl:
            z = torch.randn((w.B, w.T, Hl), generator=ug, device=dev).to(torch.bfloat16)
        else:
            z = W.step_logits(w, s, dec.tree_tok, dev)
        U = torch.rand((w.B, w.T, 2), generator=ug, device=dev) if temp > 0 else None
        prefix_hist.append(dec.prefix_len.clone())
        dec.attend(q, kt, vt, out)
        step(dec, z, kt, vt, U)
        accepted.append(dec.accept_len.clone())
        inputs.append((q, kt, vt, z, U))
    torch.cuda.synchronize()
    rec_tok, rec_M = dec.tree_tok.clone(), dec.M.clone()
    assert dec.device_flags() == 0
    prefix_hist = torch.stack(prefix_hist).cpu()          # [total, B]
    accepted = torch.stack(accepted).cpu()
    log(f"record pass: {total} steps in {time.time() - t0:.1f} s")

    def warmed():
        d = fresh_decoder()
        for s in range(args.warmup):
            q, kt, vt, z, U = inputs[s]
            d.attend(q, kt, vt, out)
            step(d, z, kt, vt, U)
        torch.cuda.synchronize()
        return d

    # ---- stream replay: warmup, then the timed region
    dec = warmed()
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    t_start = time.perf_counter()
    for i in range(steps):
        q, kt, vt, z, U = inputs[args.warmup + i]
        ev[i][0].record(stream)
        dec.attend(q, kt, vt, out)
        ev[i][1].record(stream)
        step(dec, z, kt, vt, U)
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    same = torch.equal(dec.tree_tok, rec_tok) and torch.equal(dec.M, rec_M)
    assert same, "replay diverged from the record pass"
    assert dec.device_flags() == 0

    attn_ms = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    step_ms = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    stream_wall = wall
    log(f"stream launches: {steps / wall:.1f} steps/s")

    # ---- graph replay: the timed steps captured once (every library call
    # launches its kernels on the capturing stream, so each becomes a kernel
    # node with its arguments fixed) and replayed from the post-warmup state;
    # the replay must end in the record pass's state as well
    if args.launch == "graph":
        dec = warmed()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(steps):
                q, kt, vt, z, U = inputs[args.warmup + i]
                dec.attend(q, kt, vt, out)
                step(dec, z, kt, vt, U)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        graph.replay()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        same = torch.equal(dec.tree_tok, rec_tok) and torch.equal(dec.M, rec_M)
        assert same, "graph replay diverged from the record pass"
        assert dec.device_flags() == 0
        del graph
        log(f"graph replay: {steps / wall:.1f} steps/s")
    ms_per_step = wall * 1e3 / steps

    # ---- kernel timing: the same steps again, every launch between two HIP
    # events on its stream; warm, then cold (a 1 GiB scrub written before
    # every library call, outside the events)
    def kernel_pass(cold):
        d = warmed()
        scrub = torch.empty(SCRUB_BYTES // 4, dtype=torch.int32, device=dev) if cold else None
        tr.tr_profile_enable(True)
        for i in range(steps):
            q, kt, vt, z, U = inputs[args.warmup + i]
            if cold:
                scrub.fill_(2 * i)
            d.attend(q, kt, vt, out)
            if cold:
                scrub.fill_(2 * i + 1)
            step(d, z, kt, vt, U)
        launches = tr.tr_profile_read()
        tr.tr_profile_enable(False)
        assert torch.equal(d.tree_tok, rec_tok), "profiled replay diverged from the record pass"
        ks = {}
        for name, ms in launches:
            ks.setdefault(name, []).append(ms)
        return {k: sum(v) / len(v) for k, v in ks.items() if len(v) == steps}

    kernel_ms = kernel_pass(False)
    cold_ms = kernel_pass(True) if not args.no_cold else None

    # ---- algorithmic bytes per call (what the method must move)
    esz = torch.tensor([], dtype=w.kv_dtype).element_size()
    lsz = torch.tensor([], dtype=w.logit_dtype).element_size()
    timed = slice(args.warmup, total)
    P_sum = prefix_hist[timed].double().sum(dim=1)        # prefix positions per step, all sequences
    kv_bytes = (P_sum * w.Hkv * w.d * 2 * esz).mean().item()
    qo_bytes = 2 * w.B * w.T * w.Hq * w.d * esz
    tkv_bytes = 2 * w.B * w.T * w.Hkv * w.d * esz
    attn_bytes = kv_bytes + qo_bytes + tkv_bytes
    L_mean = accepted[timed].double().mean().item()
    commit_bytes = 2 * 2 * (L_mean + 1) * w.Hkv * w.d * esz * w.B   # K and V rows, read + write
    logits_bytes = w.B * w.T * w.V * lsz
    m_bytes = w.B * w.T * w.k * 4 * 2                              # rows written + read back
    step_bytes = logits_bytes + commit_bytes + m_bytes
    if Hl:
        # the step reads h and the output embedding instead of logits; the
        # slice keys (8 per row and 128-id slice) are written and read back
        lm_bytes = w.V * Hl * 2 + w.B * w.T * Hl * 2
        part_bytes = w.B * w.T * ((w.V + 127) // 128) * 8 * 8
        step_bytes = lm_bytes + 2 * part_bytes + commit_bytes + m_bytes
    calls = {
        "tr_tree_attn": (attn_ms, attn_bytes),
        "tr_step": (step_ms, step_bytes),
    }
    detail = {c: {"avg_us": round(ms * 1e3, 2), "bytes": int(b),
                  "GB_s": round(b / (ms * 1e-3) / 1e9, 1)} for c, (ms, b) in calls.items()}
    log("per call:", json.dumps(detail))
    # per kernel: in the bf16 path the prefix pass reads the cache, the tree
    # keys/values and the queries and writes the output of every (sequence,
    # kv head) that one block finishes; the merge writes the rest, so the
    # output bytes are booked to the merge (its upper bound).  In the fp32
    # path the combine reads the tree keys/values and writes the output.
    if w.kv_dtype == torch.bfloat16:
        kbytes = {"attn_prefix": kv_bytes + tkv_bytes + qo_bytes / 2, "attn_combine": qo_bytes / 2,
                  "topk": step_bytes}
    else:
        kbytes = {"attn_prefix": kv_bytes + qo_bytes / 2, "attn_combine": tkv_bytes + qo_bytes / 2,
                  "topk": step_bytes}
    if Hl:
        kbytes["lmhead"] = lm_bytes + part_bytes
        kbytes["lmhead_merge"] = part_bytes + commit_bytes + m_bytes

    def per_kernel(ms_map):
        return {k: {"avg_us": round(ms * 1e3, 2), "bytes": int(kbytes[k]),
                    "GB_s": round(kbytes[k] / (ms * 1e-3) / 1e9, 1)} for k, ms in ms_map.items()}

    kdetail = per_kernel(kernel_ms)
    log("per kernel (warm):", json.dumps(kdetail))
    cdetail = per_kernel(cold_ms) if cold_ms else None
    if cdetail:
        log("per kernel (cold):", json.dumps(cdetail))
    # matrix-core work of the prefix pass: two products of rows x keys x d
    attn_flops = 4.0 * w.T * w.Hq * w.d * (P_sum.mean().item())
    dtype = "bf16" if w.kv_dtype == torch.bfloat16 else "f32"
    kflops = {"attn_prefix": attn_flops}
    if Hl:
        kflops["lmhead"] = 2.0 * w.B * w.T * w.V * Hl
    # the roofline of the dominant kernel, from the cold pass when there is
    # one: its binding roof is whichever takes longer at peak
    roof_ms = cold_ms or kernel_ms
    dom = max(roof_ms, key=roof_ms.get)
    dms, dbytes = roof_ms[dom], kbytes[dom]
    t_hbm = dbytes / (HBM_PEAK_GBS * 1e9)
    t_mfma = kflops.get(dom, 0.0) / (MFMA_PEAK_TFLOPS[dtype] * 1e12)
    if t_mfma > t_hbm:
        achieved = kflops[dom] / (dms * 1e-3) / 1e12
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 1),
                "peak": MFMA_PEAK_TFLOPS[dtype], "unit": "TFLOP/s",
                "frac": round(achieved / MFMA_PEAK_TFLOPS[dtype], 4)}
    else:
        achieved = dbytes / (dms * 1e-3) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(args.workload, record_kernel(w, dom))
    roof["timing"] = "cold (1 GiB scrub before every call)" if cold_ms else "warm"
    # both roofs of the dominant kernel, and its matrix-core counters
    roof["hbm_GB_s"] = round(dbytes / (dms * 1e-3) / 1e9, 1)
    if dom in kflops:
        roof["mfma_TFLOP_s"] = round(kflops[dom] / (dms * 1e-3) / 1e12, 1)
    roof["mfma_counters"] = measured_mfma(args.workload, record_kernel(w, dom))
    probe = read_probe(tr)
    roof["achievable_read_GB_s"] = probe
    log(f"read probe: {probe} GB/s; mean accepted drafts {L_mean:.3f}, emitted/step {L_mean + 1:.3f}")

    unfused = None
    if Hl:
        # the same steps with the product unfused: one bf16 GEMM writing the
        # logits, then tr_step on them
        dec = fresh_decoder()
        logits = torch.empty((w.B, w.T, w.V), dtype=torch.bfloat16, device=dev)
        W_t = W_out.t()

        def unfused_step(i):
            q, kt, vt, h, _ = inputs[i]
            dec.attend(q, kt, vt, out)
            torch.matmul(h.view(-1, Hl), W_t, out=logits.view(-1, w.V))
            dec.step(logits, kt, vt)

        for i in range(args.warmup):
            unfused_step(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            unfused_step(args.warmup + i)
        torch.cuda.synchronize()
        unfused = {"steps_per_s": round(steps / (time.perf_counter() - t0), 2),
                   "what": "attention + bf16 GEMM writing the logits (torch.matmul) + tr_step"}
        if args.launch == "graph":
            # the same steps captured once and replayed, as the fused value is
            # (its trajectory differs from the fused one where the bf16
            # logits round a ranking differently, so only the time is kept)
            dec = fresh_decoder()
            for i in range(args.warmup):
                unfused_step(i)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                for i in range(steps):
                    unfused_step(args.warmup + i)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            graph.replay()
            torch.cuda.synchronize()
            unfused["graph_steps_per_s"] = round(steps / (time.perf_counter() - t0), 2)
            assert dec.device_flags() == 0
            del graph
        log("unfused:", json.dumps(unfused))

    cpu = None
    if args.cpu_seconds > 0 and not Hl:
        cpu = cpu_baseline(w, inputs, init_host, args.cpu_seconds, temp)

    res = {
        "metric": METRIC,
        "value": round(steps / wall, 2),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype,
        "data": "synthetic",
        "config": {"workload": w.description, "V": w.V, "k": w.k, "sequences": w.B,
                   "tree_nodes": w.T, "tree_depth": w.depth, "Hq": w.Hq, "Hkv": w.Hkv,
                   "head_dim": w.d, "prefix": list(w.prefix), "M_dtype": str(w.m_dtype)[6:],
                   "verification": f"sampling, temperature {temp}" if temp > 0 else "greedy",
                   "cache": f"paged, {args.page_size} rows per page" if args.page_size else "contiguous",
                   "launch": "one HIP graph of the timed steps" if args.launch == "graph"
                             else "stream launches"},
        "roofline": roof,
        "stream_launch_steps_per_s": round(steps / stream_wall, 2),
        "per_call": detail,
        "per_kernel": kdetail,
        "per_kernel_cold": cdetail,
        "kernel_sum_steps_per_s": {"warm": round(1e3 / sum(kernel_ms.values()), 2),
                                   "cold": round(1e3 / sum(cold_ms.values()), 2) if cold_ms else None},
        "emitted_per_step": round(L_mean + 1, 3),
        "cpu_baseline": cpu,
    }
    if Hl:
        res["config"]["lm_head"] = f"fused, H={Hl}, W [V][H] bf16 seeded"
        res["unfused"] = unfused
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
