"""CSA2 decode benchmark on one MI355X.

One step = one decode token for every sequence of the batch through every layer of the
workload.  The headline workload is the largest single-GPU decode configuration: the
16-layer stack, batch 64, 131,072 FP4 entries per sequence, four sharing groups in modes
Full, Reindex, Reuse, Reuse, top-k 2048, 16 bf16 heads of dim 128, window 128, bf16 index
keys 4 x 64.  Inputs are seeded synthetic N(0,1) data already resident in HBM when timing
starts.

Prints one JSON line with:
  * tokens/s over exactly --steps timed steps (after --warmup), and the median, p10 and p90
    of the per-step times (HIP events around every step);
  * the roofline of the dominant kernel, the exact index-score stream, from its launches
    inside the timed steps (HIP events that the library records around each Full/Reindex
    layer's scoring on the same stream); its algorithmic bytes are the index keys plus the
    index queries, and the score spill is reported beside them;
  * the HBM traffic of that kernel from the committed rocprofv3 counter summary (null when
    the kernel source has changed since);
  * legs: the 4-layer batch-32 group, the long-context fp8 decode, the draft-block verify,
    FP4 index keys, hierarchical search, the host tier, and the prefill chunk (4,096 queries
    against 131,072 causal entries, e4m3 index keys on MFMA) with its index stage's MFMA
    utilisation;
  * the CPU oracle on a bounded sample of the headline workload: one host thread, and all
    the host's threads.

`--traffic-probe` runs only three 1 GiB device copies and two steps of the workload, for
`rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs.
"""
from __future__ import annotations

import argparse
import concurrent.futures
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E
FP8_PEAK_TFLOPS = 5000.0  # MI355X dense fp8 MFMA
HEADLINE = 5  # the 16-layer, batch-64 decode stack
TRAFFIC_SUMMARY = {5: os.path.join(ROOT, "profiles", "score_exact_w5_hbm_traffic.md"),
                   7: os.path.join(ROOT, "profiles", "score_fp4_mfma_w7_hbm_traffic.md")}
SCORE_SOURCE = os.path.join(ROOT, "compressed_kv_cache_03_amd", "csrc", "score.hip")


def measured_traffic(wid):
    """HBM bytes per launch of the workload's dominant kernel (FETCH_SIZE + WRITE_SIZE, scaled by
    the copy calibration) from the committed counter summary, or None when there is none or it was
    taken on another version of the kernel source."""
    if wid not in TRAFFIC_SUMMARY:
        return None
    try:
        text = open(TRAFFIC_SUMMARY[wid]).read()
        src = hashlib.sha256(open(SCORE_SOURCE, "rb").read()).hexdigest()
    except OSError:
        return None
    fields = {}
    for line in text.splitlines():
        if ":" in line and line.startswith("- "):
            key, val = line[2:].split(":", 1)
            fields[key.strip()] = val.strip().strip("`")
    if fields.get("score.hip sha256") != src:
        return None
    try:
        return int(fields["traffic bytes per launch"])
    except (KeyError, ValueError):
        return None


def _dev(a, device):
    import torch

    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(device)


def _key_bytes(wl):
    """(bytes per stored index key, per index query row, per new key written by Full)."""
    K = wl.H_I * wl.d_I
    if wl.idx_dtype == "fp4":
        return K // 2 + K // 32 * 4, K * 2, K * 4 + K // 2 + K // 32 * 4
    eb = 2 if wl.idx_dtype == "bf16" else 1
    return K * eb, K * eb, K * eb * 2


def algorithmic_bytes(wl):
    """Bytes the method must move per step.  Every layer reads its selection, the selected FP4
    records, its window rows and query and writes its output; a selecting layer also streams
    every index key and reads its index query (the dominant kernel's bytes), and writes its
    selection; a Full layer also packs and stores its new entry and index key.  The fp32
    scores a selecting layer spills between its scan and its top-k are an intermediate,
    counted separately."""
    B, N, D, k, W, Hq, Qs = wl.B, wl.N, wl.D, wl.k, wl.W, wl.Hq, wl.Qs
    key_b, q_b, new_key_b = _key_bytes(wl)
    per_layer_attend = B * Qs * (k * (D // 2 + D // 32 * 4) + 2 * (Qs + W - 1) * D * 2 // Qs
                                 + Hq * D * 2 + Hq * D * 4 + Hq * 4)
    scan = B * (N * key_b + Qs * q_b)  # index keys + index queries
    spill = B * Qs * N * 4             # score write
    select = B * Qs * k * 4            # selection written
    full_write = B * Qs * (D * 4 + D // 2 + D // 32 * 4 + new_key_b)
    total = 0
    for mode in wl.pattern * wl.groups:
        total += per_layer_attend + B * Qs * k * 4  # every mode reads its selection
        if mode in ("F", "Ri"):
            total += scan + select
        if mode == "F":
            total += full_write
    return {"step": total, "score_launch": scan, "score_spill": spill}


def _pct(xs, q):
    return float(np.percentile(np.asarray(xs, dtype=np.float64), q))


def _summary(ms_list):
    return {"median": round(_pct(ms_list, 50), 4), "p10": round(_pct(ms_list, 10), 4),
            "p90": round(_pct(ms_list, 90), 4)}


def setup_decode(wl, device):
    import torch

    import compressed_kv_cache_03_amd as csa2
    from synth.inputs import make_inputs

    t0 = time.time()
    inp = make_inputs(wl)
    B, N = wl.B, wl.N
    groups = []
    for g in range(wl.groups):
        gc, gs = csa2.fp4_pack(_dev(inp.cache_x[g], device))
        keys, kscales = _dev(inp.ikeys[g], device), None
        if wl.idx_dtype == "fp4":
            K = wl.H_I * wl.d_I
            kc, kscales = csa2.fp4_pack(keys.reshape(B * N, K))
            keys, kscales = kc.reshape(B, N, wl.H_I, wl.d_I // 2), kscales.reshape(B, N, K // 32)
        groups.append(csa2.Group(gc, gs, keys, _dev(inp.n_valid, device), wl.idx_dtype, wl.k,
                                 sel_rows=B * wl.Qs, ikey_scales=kscales, pool_blocks=wl.pool_blocks))
        torch.cuda.synchronize()
    layers = []
    for L in inp.layers:
        d = {k: (_dev(v, device) if isinstance(v, np.ndarray) else v) for k, v in L.items()}
        d["out"] = torch.empty(B, wl.Qs, wl.Hq, wl.D, dtype=torch.float32, device=device)
        d["lse"] = torch.empty(B, wl.Qs, wl.Hq, dtype=torch.float32, device=device)
        layers.append(d)
    for grp in groups:
        grp.workspace(wl.Qs, wl.Hq, wl.W)
    torch.cuda.synchronize()
    print(f"# {wl.name}: inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)
    return inp, groups, layers


def run_decode(wl, steps, warmup, device, state=None):
    """Warm up, then time exactly `steps` decode steps.  Returns per-step times and the
    durations of every index-score launch inside the timed steps."""
    import torch

    inp, groups, layers = state if state is not None else setup_decode(wl, device)
    stream = torch.cuda.current_stream()
    selecting = [li for li, d in enumerate(layers) if d["mode"] in ("F", "Ri")]

    def new_event():
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)  # creates the event, so the library can record it by handle
        return e

    score_ev = [[(new_event(), new_event()) for _ in selecting] for _ in range(steps)]
    step_ev = [new_event() for _ in range(steps + 1)]
    torch.cuda.synchronize()

    def step(t=None):
        j = 0
        for d in layers:
            grp = groups[d["group"]]
            kw = dict(q=d["q"], wk=d["wk"], wv=d["wv"], W=wl.W, sm_scale=wl.sm_scale,
                      out=d["out"], lse=d["lse"])
            if d["iq"] is not None:
                kw["iq"] = d["iq"]
                if t is not None:
                    kw["index_events"] = score_ev[t][j]
                    j += 1
            if d["new_entry"] is not None:
                kw["new_entry"] = d["new_entry"]
                kw["new_ikey"] = d["new_ikey"]
            grp.layer_step(d["mode"], **kw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    step_ev[0].record(stream)
    for t in range(steps):
        step(t)
        step_ev[t + 1].record(stream)
    torch.cuda.synchronize()
    per_step = [step_ev[t].elapsed_time(step_ev[t + 1]) for t in range(steps)]
    total = step_ev[0].elapsed_time(step_ev[-1])
    score_ms = [a.elapsed_time(b) for row in score_ev for a, b in row]
    return {"ms_mean": total / steps, "per_step": per_step, "score_ms": score_ms,
            "state": (inp, groups, layers)}


def decode_leg(wl, steps, warmup, device, extra=None):
    r = run_decode(wl, steps, warmup, device)
    ab = algorithmic_bytes(wl)
    res = {"workload": wl.name, "steps": steps, "ms_per_step": round(r["ms_mean"], 4),
           "ms_per_step_pct": _summary(r["per_step"]),
           "tokens_per_s": round(wl.B * wl.Qs / (r["ms_mean"] * 1e-3), 1),
           "step_GBps": round(ab["step"] / (r["ms_mean"] * 1e-3) / 1e9, 1)}
    if r["score_ms"]:
        us = float(np.mean(r["score_ms"])) * 1e3
        res["score_launch_us"] = round(us, 2)
        res["score_GBps"] = round(ab["score_launch"] / (us * 1e-6) / 1e9, 1)
    res.update(extra or {})
    return res, r


def host_tier(grp, reps=3):
    """Save a group to a pinned host image and restore it: GB/s each way."""
    import torch

    image = grp.save()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record(stream)
    for _ in range(reps):
        grp.save(image)
    e[1].record(stream)
    for _ in range(reps):
        grp.restore(image)
    e[2].record(stream)
    torch.cuda.synchronize()
    n = image.numel()
    ms_save, ms_restore = e[0].elapsed_time(e[1]) / reps, e[1].elapsed_time(e[2]) / reps
    return {"image_bytes": n, "save_GBps": round(n / (ms_save * 1e-3) / 1e9, 1),
            "restore_GBps": round(n / (ms_restore * 1e-3) / 1e9, 1),
            "note": "pinned host image of the batch-32 group (FP4 codes, scales, index keys, "
                    "selection); device <-> host copies, restored bits checked by the GPU tests"}


def copy_bandwidth(device, reps=5):
    """Device-to-device copy of 1 GiB: bytes read plus bytes written per second."""
    import torch

    src = torch.ones(1 << 30, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    dst.copy_(src)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    return round(2 * src.numel() * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)


def read_bandwidth(device, reps=5):
    """Bytes per second read by torch's own sum over 4 GiB of fp32 (one pass, nothing written but
    the result): what a library reduction reads on this device, beside the score kernel's rate."""
    import torch

    x = torch.ones(1 << 30, dtype=torch.float32, device=device)
    torch.sum(x)
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        torch.sum(x)
    e1.record(stream)
    torch.cuda.synchronize()
    gbps = round(x.numel() * 4 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    del x
    return gbps


def cache_accounting(wl):
    """Stored cache bytes of the workload's layers with entries and index keys shared inside each
    group, against every layer keeping its own (entries x numbers x copies x bits / 8 per array,
    computed by the library's accounting entry point)."""
    import compressed_kv_cache_03_amd as csa2

    entries = wl.B * wl.N
    K = wl.H_I * wl.d_I
    arrays = {"fp4_codes": (wl.D, 4), "fp4_scales": (wl.D // 32, 32)}
    if wl.idx_dtype == "fp4":
        arrays.update({"index_keys": (K, 4), "index_key_scales": (K // 32, 32)})
    else:
        arrays["index_keys"] = (K, 16 if wl.idx_dtype == "bf16" else 8)
    layers = len(wl.pattern) * wl.groups
    shared = {n: csa2.cache_bytes(entries, num, wl.groups, bits) for n, (num, bits) in arrays.items()}
    unshared = {n: csa2.cache_bytes(entries, num, layers, bits) for n, (num, bits) in arrays.items()}
    return {"layers": layers, "stored_copies": wl.groups, "shared_bytes": shared,
            "unshared_bytes": unshared, "shared_total": sum(shared.values()),
            "unshared_total": sum(unshared.values()),
            "ratio": round(sum(unshared.values()) / sum(shared.values()), 3)}


def traffic_probe(wl, device):
    """Three plain 1 GiB device copies (the counter calibration), then two decode steps of the
    workload (every Full/Reindex layer launches the dominant kernel once), nothing else."""
    import torch

    src = torch.ones(1 << 30, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    run_decode(wl, 2, 0, device)
    print(f"traffic probe: 3 copies of 1073741824 B, 2 steps of {wl.name}", flush=True)


def run_prefill(wl, steps, warmup, device):
    """One Full layer over a prefill chunk; returns ms per chunk and the index stage's (threshold
    sample GEMM through the MFMA filter GEMM) ms per chunk, both from HIP events."""
    import torch

    import compressed_kv_cache_03_amd as csa2
    from synth.inputs import make_inputs

    inp = make_inputs(wl)
    gc, gs = csa2.fp4_pack(_dev(inp.cache_x[0], device))
    grp = csa2.Group(gc, gs, _dev(inp.ikeys[0], device), _dev(inp.n_valid, device), wl.idx_dtype, wl.k,
                     sel_rows=wl.B * wl.Qs)
    L = inp.layers[0]
    kw = dict(q=_dev(L["q"], device), iq=_dev(L["iq"], device), wk=_dev(L["wk"], device),
              wv=_dev(L["wv"], device), W=wl.W, sm_scale=wl.sm_scale,
              new_entry=_dev(L["new_entry"], device), new_ikey=_dev(L["new_ikey"], device))
    grp.workspace(wl.Qs, wl.Hq, wl.W)
    for _ in range(warmup):
        grp.layer_step("F", **kw)
    stream = torch.cuda.current_stream()
    ev = []
    for _ in range(steps + 1):
        e = torch.cuda.Event(enable_timing=True)
        e.record(stream)
        ev.append(e)
    idx_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for a, b in idx_ev:
        a.record(stream)
        b.record(stream)
    torch.cuda.synchronize()
    ev[0].record(stream)
    for t in range(steps):
        grp.layer_step("F", index_events=idx_ev[t], **kw)
        ev[t + 1].record(stream)
    torch.cuda.synchronize()
    chunk = [ev[t].elapsed_time(ev[t + 1]) for t in range(steps)]
    index = [a.elapsed_time(b) for a, b in idx_ev]
    return chunk, index


def prefill_index_flops(wl):
    """Useful MFMA work of the causal index scoring: 2 K flops per visible (query, entry)."""
    K = wl.H_I * wl.d_I
    visible = sum(wl.N - wl.Qs + i + 1 for i in range(wl.Qs)) * wl.B
    return 2 * K * visible


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _host_threads():
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    omp = os.environ.get("OMP_NUM_THREADS")
    return max(1, min(avail, int(omp))) if omp and omp.isdigit() else avail


def cpu_baseline(wl, inp, one_seqs=2, all_seqs=16, target_seconds=8.0, max_reps=20):
    """The oracle, as it stands, on a bounded sample of the workload: whole decode steps through
    every layer, first for `one_seqs` sequences on one host thread, then for `all_seqs`
    sequences on every host thread (OpenMP over query rows).  Cache packing is untimed setup
    (spread over host threads; the oracle's own packing routine)."""
    import oracle

    gomp = ctypes.CDLL("libgomp.so.1")  # the OpenMP runtime the oracle is linked against
    threads = _host_threads()
    bs = min(wl.B, max(all_seqs, one_seqs))
    B, N, D = wl.B, wl.N, wl.D
    t0 = time.time()

    def pack(g, b):
        return oracle.fp4_pack(inp.cache_x[g][b].reshape(N, D))

    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        packed = {(g, b): ex.submit(pack, g, b) for g in range(wl.groups) for b in range(bs)}
        packed = {key: f.result() for key, f in packed.items()}
    t_setup = time.time() - t0

    def make_groups(n):
        groups = []
        for g in range(wl.groups):
            oc = np.stack([packed[(g, b)][0] for b in range(n)])
            os_ = np.stack([packed[(g, b)][1] for b in range(n)])
            groups.append(oracle.Group(oc, os_, inp.ikeys[g][:n].copy(), inp.n_valid[:n].astype(np.int64),
                                       wl.idx_dtype, wl.k, max_rows=n * wl.Qs))
        return groups

    def timed(n, nthreads):
        gomp.omp_set_num_threads(nthreads)
        groups = make_groups(n)
        reps = 0
        t0 = time.time()
        while True:
            for L in inp.layers:
                kw = dict(q=L["q"][:n], wk=L["wk"][:n], wv=L["wv"][:n], W=wl.W,
                          sm_scale=np.float32(wl.sm_scale))
                if L["iq"] is not None:
                    kw["iq"] = L["iq"][:n]
                if L["new_entry"] is not None:
                    kw["new_entry"] = L["new_entry"][:n]
                    kw["new_ikey"] = L["new_ikey"][:n]
                rc, _, _ = groups[L["group"]].layer_step(L["mode"], **kw)
                assert rc == 0
            reps += 1
            if time.time() - t0 >= target_seconds or reps >= max_reps:
                break
        return reps, time.time() - t0

    r1, t1 = timed(min(one_seqs, bs), 1)
    ra, ta = timed(bs, threads)
    gomp.omp_set_num_threads(threads)
    n1 = min(one_seqs, bs)
    return {"value": round(ra * bs * wl.Qs / ta, 4), "unit": "tokens/s", "cores": min(threads, bs),
            "kind": "oracle",
            "single_thread_tokens_per_s": round(r1 * n1 * wl.Qs / t1, 4),
            "single_thread_s": round(t1, 2), "all_core_s": round(ta, 2),
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "threads_available": threads,
            "sample": f"{wl.name}: whole decode steps through all {len(inp.layers)} layers; "
                      f"{r1} step(s) of {n1} of {B} sequences on 1 thread ({t1:.1f}s), then {ra} "
                      f"step(s) of {bs} sequences on {min(threads, bs)} threads ({ta:.1f}s); cache "
                      f"packing untimed ({t_setup:.1f}s)"}


def prefill_section(device):
    """The prefill chunk (one Full layer over 4,096 queries) timed with HIP events."""
    from synth.workloads import ALL

    pw = ALL[4]
    chunk, index = run_prefill(pw, 10, 2, device)
    flops = prefill_index_flops(pw)
    idx_ms = float(np.mean(index))
    return {
        "workload": pw.name, "ms_per_chunk": round(float(np.mean(chunk)), 4),
        "ms_per_chunk_pct": _summary(chunk),
        "tokens_per_s": round(pw.Qs / (float(np.mean(chunk)) * 1e-3), 1),
        "index_flops": flops,
        "index_stage_us": round(idx_ms * 1e3, 2),
        "index_stage_mfma_util": round(flops / (idx_ms * 1e-3) / (FP8_PEAK_TFLOPS * 1e12), 4),
        "note": "index stage = sampled-threshold GEMM, key norms, threshold selection and the "
                "MFMA filter GEMM (HIP events around them inside the chunk); mfma_util = useful "
                "index flops / (index stage time x 5.0 PFLOP/s fp8)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", type=int, default=HEADLINE, choices=[1, 2, 3, 5, 6, 7, 8],
                    help="decode workload timed as the main line (the default is the headline stack)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-legs", action="store_true", help="headline workload only")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill chunk and print its section (for profiling runs)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this implementation runs on one GPU; --gpus {args.gpus} is not supported "
              "(sequences are independent, so the path would shard by sequence with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from synth.workloads import ALL

    wl = ALL[args.workload]
    device = "cuda:0"
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.traffic_probe:
        traffic_probe(wl, device)
        return
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_section(device)}), flush=True)
        return
    r = run_decode(wl, args.steps, args.warmup, device)
    inp = r["state"][0]
    ab = algorithmic_bytes(wl)
    ms = r["ms_mean"]
    score_us = float(np.mean(r["score_ms"])) * 1e3
    achieved = ab["score_launch"] / (score_us * 1e-6) / 1e9
    res = {
        "metric": "CSA2 decode tokens/s + achieved HBM GB/s (frac. of peak) at 1 MI355X",
        "value": round(wl.B * wl.Qs / (ms * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_pct": _summary(r["per_step"]),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "dtype_detail": "exact index scores accumulated in f64 from bf16/e4m3 keys; attention in "
                        "f32 over FP4 e2m1 entries and bf16 window rows",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "entries": wl.N,
                   "layers": list(wl.pattern) * wl.groups, "index": f"{wl.H_I}x{wl.d_I} {wl.idx_dtype}",
                   "k": wl.k, "heads": wl.Hq, "head_dim": wl.D, "window": wl.W},
        "step_hbm": {"algorithmic_bytes": ab["step"],
                     "GBps": round(ab["step"] / (ms * 1e-3) / 1e9, 1),
                     "frac": round(ab["step"] / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "roofline": {"kernel": ("score_fp4_mfma_kernel (FP4-key index scores on the matrix cores, inside "
                                "the timed steps)" if wl.idx_dtype == "fp4" else
                                "score_exact_kernel (exact index-score stream, inside the timed steps)"),
                     "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(wl.wid),
                     "bytes_per_launch": ab["score_launch"], "score_spill_bytes_per_launch": ab["score_spill"],
                     "launches": len(r["score_ms"]), "avg_launch_us": round(score_us, 2),
                     "launch_us_pct": _summary([x * 1e3 for x in r["score_ms"]])},
        "hbm_copy_GBps": copy_bandwidth(device),
        "hbm_read_GBps": read_bandwidth(device),
        "cache": cache_accounting(wl),
    }
    del r
    torch.cuda.empty_cache()
    if not args.no_legs:
        legs = {}
        for wid, extra in ((2, None), (3, None),
                           (6, {"note": "draft block of 5 queries per sequence; tokens/s counts the 5 "
                                        "verified positions of each sequence"}),
                           (7, {"note": "FP4 e2m1 index keys (fp32 block-32 scales, bf16 index queries); "
                                        "scores still exact"}),
                           (8, {"pool": "2048 blocks x 8 = 16384 candidates per row",
                                "note": "Full scores all entries and keeps the pool; Reindex scores and "
                                        "ranks only the pool's entries"})):
            lw = ALL[wid]
            leg, lr = decode_leg(lw, max(args.steps // 2, 10), 3, device, extra)
            if wid == 2:
                res["host_tier"] = host_tier(lr["state"][1][0])
            legs[lw.name] = leg
            del lr
            torch.cuda.empty_cache()
        res["legs"] = legs
    if not args.no_prefill:
        res["prefill"] = prefill_section(device)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, inp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
