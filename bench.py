"""CSA2 decode benchmark on one MI355X.

One step = one decode token for every sequence of the batch through every layer of
the workload (default: batch 32, 65,536 FP4 entries per sequence, one sharing group in
modes Full, Reindex, Reuse, Reuse, top-k 2048, 16 bf16 heads of dim 128, window 128).
Inputs are seeded synthetic N(0,1) data already resident in HBM when timing starts.

Prints one JSON line with tokens/s, the roofline of the dominant kernel (the exact
index-score stream) measured with HIP events, the HBM traffic of that kernel from the
committed rocprofv3 counter summary (null when the kernel source has changed since),
a prefill-chunk leg (4,096 queries against 131,072 causal entries, e4m3 index keys on
MFMA), and the CPU oracle timed on a bounded sample of the same workload on this
host's cores.

`--traffic-probe` runs only a 1 GiB device copy and five launches of the dominant
kernel, for `rocprofv3 --pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs.
"""
from __future__ import annotations

import argparse
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
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "score_exact_w2_hbm_traffic.md")
SCORE_SOURCE = os.path.join(ROOT, "compressed_kv_cache_03_amd", "csrc", "score.hip")


TRAFFIC_WORKLOAD = "decode_b32_n65536_group_F_Ri_Ru_Ru"  # the workload the summary's counters cover


def measured_traffic():
    """Bytes per launch of the dominant kernel from the committed counter summary, or None
    when the summary is missing or was taken on another version of the kernel source."""
    try:
        text = open(TRAFFIC_SUMMARY).read()
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


def algorithmic_bytes(wl):
    """Bytes the method must move per step: every layer reads its selection, the selected FP4
    records, its window rows and query and writes its output; a selecting layer also streams every
    index key, reads its index query, writes a score per entry and its selection; a Full layer
    also packs and stores its new entry and index key.  Returns (total, bytes of one score launch)."""
    B, N, D, K, k, W, Hq, Qs = wl.B, wl.N, wl.D, wl.H_I * wl.d_I, wl.k, wl.W, wl.Hq, wl.Qs
    if wl.idx_dtype == "fp4":
        key_b, q_b, new_key_b = K // 2 + K // 32 * 4, K * 2, K * 4 + K // 2 + K // 32 * 4
    else:
        eb = 2 if wl.idx_dtype == "bf16" else 1
        key_b, q_b, new_key_b = K * eb, K * eb, K * eb * 2
    per_layer_attend = B * Qs * (k * (D // 2 + D // 32 * 4) + 2 * (Qs + W - 1) * D * 2 // Qs
                                 + Hq * D * 2 + Hq * D * 4 + Hq * 4)
    scan = B * (N * key_b + Qs * q_b + Qs * N * 4)  # keys + index query + score write
    select = B * Qs * k * 4                         # selection written
    full_write = B * Qs * (D * 4 + D // 2 + D // 32 * 4 + new_key_b)
    total = 0
    for mode in wl.pattern * wl.groups:
        total += per_layer_attend + B * Qs * k * 4  # every mode reads its selection
        if mode in ("F", "Ri"):
            total += scan + select
        if mode == "F":
            total += full_write
    return total, scan


def run_gpu(wl, steps, warmup, device, scan_loop=True):
    import torch

    import compressed_kv_cache_03_amd as csa2
    from synth.inputs import make_inputs

    t0 = time.time()
    inp = make_inputs(wl)
    B, N, D = wl.B, wl.N, wl.D
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
    layers = []
    for L in inp.layers:
        d = {k: (_dev(v, device) if isinstance(v, np.ndarray) else v) for k, v in L.items()}
        d["out"] = torch.empty(B, wl.Qs, wl.Hq, D, dtype=torch.float32, device=device)
        d["lse"] = torch.empty(B, wl.Qs, wl.Hq, dtype=torch.float32, device=device)
        layers.append(d)
    for grp in groups:
        grp.workspace(wl.Qs, wl.Hq, wl.W)
    torch.cuda.synchronize()
    print(f"# inputs ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def step():
        for d in layers:
            grp = groups[d["group"]]
            kw = dict(q=d["q"], wk=d["wk"], wv=d["wv"], W=wl.W, sm_scale=wl.sm_scale,
                      out=d["out"], lse=d["lse"])
            if d["iq"] is not None:
                kw["iq"] = d["iq"]
            if d["new_entry"] is not None:
                kw["new_entry"] = d["new_entry"]
                kw["new_ikey"] = d["new_ikey"]
            grp.layer_step(d["mode"], **kw)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    if not scan_loop:
        return ms_step, None, inp, groups

    # dominant kernel: the exact index-score stream over one group's keys (same kernel the
    # Full/Reindex layers launch), timed over its own loop on the same stream
    first = next(d for d in layers if d["mode"] == "F")
    grp = groups[first["group"]]
    scores = torch.empty(B, wl.Qs, N, dtype=torch.float32, device=device)
    reps = max(steps, 5)
    for _ in range(2):
        csa2.index_score(first["iq"], grp.ikeys, wl.idx_dtype, out=scores, ik_scales=grp.ikey_scales)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        csa2.index_score(first["iq"], grp.ikeys, wl.idx_dtype, out=scores, ik_scales=grp.ikey_scales)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_scan = e0.elapsed_time(e1) / reps
    return ms_step, ms_scan, inp, groups


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
            "note": "pinned host image of the workload's first sharing group (FP4 codes, scales, index "
                    "keys, selection); device <-> host copies, restored bits checked by the GPU tests"}


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
    """A plain 1 GiB device copy (the counter calibration) and five launches of the
    dominant kernel on one group of the workload, nothing else."""
    import torch

    import compressed_kv_cache_03_amd as csa2
    from synth.inputs import make_inputs

    inp = make_inputs(wl)
    src = torch.ones(1 << 30, dtype=torch.uint8, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    first = next(L for L in inp.layers if L["mode"] == "F")
    iq = _dev(first["iq"], device)
    keys = _dev(inp.ikeys[first["group"]], device)
    scores = torch.empty(wl.B, wl.Qs, wl.N, dtype=torch.float32, device=device)
    for _ in range(5):
        csa2.index_score(iq, keys, wl.idx_dtype, out=scores)
    torch.cuda.synchronize()
    print("traffic probe: 3 copies of 1073741824 B, 5 index-score launches", flush=True)


def run_prefill(wl, steps, warmup, device):
    """One Full layer over a prefill chunk; returns ms per chunk."""
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
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        grp.layer_step("F", **kw)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def prefill_index_flops(wl):
    """Useful MFMA work of the causal index scoring: 2 K flops per visible (query, entry)."""
    K = wl.H_I * wl.d_I
    visible = sum(wl.N - wl.Qs + i + 1 for i in range(wl.Qs)) * wl.B
    return 2 * K * visible


def cpu_baseline(wl, inp, target_seconds=12.0, max_reps=50):
    """The oracle, as it stands, on a bounded sample of the same workload: whole decode steps
    over (up to) 32 sequences, repeated until about target_seconds of host time have run."""
    import oracle

    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    threads = max(1, min(threads, os.cpu_count() or 1))
    bs = min(wl.B, 32)
    B, N, D = wl.B, wl.N, wl.D
    t0 = time.time()
    groups = []
    for g in range(wl.groups):
        x = inp.cache_x[g][:bs]
        oc, os_ = oracle.fp4_pack(x.reshape(bs * N, D))
        groups.append(oracle.Group(oc.reshape(bs, N, D // 2), os_.reshape(bs, N, D // 32),
                                   inp.ikeys[g][:bs].copy(), inp.n_valid[:bs].astype(np.int64),
                                   wl.idx_dtype, wl.k, max_rows=bs * wl.Qs))
    t_setup = time.time() - t0
    reps = 0
    t0 = time.time()
    while True:
        for L in inp.layers:
            kw = dict(q=L["q"][:bs], wk=L["wk"][:bs], wv=L["wv"][:bs], W=wl.W,
                      sm_scale=np.float32(wl.sm_scale))
            if L["iq"] is not None:
                kw["iq"] = L["iq"][:bs]
            if L["new_entry"] is not None:
                kw["new_entry"] = L["new_entry"][:bs]
                kw["new_ikey"] = L["new_ikey"][:bs]
            rc, _, _ = groups[L["group"]].layer_step(L["mode"], **kw)
            assert rc == 0
        reps += 1
        if time.time() - t0 >= target_seconds or reps >= max_reps:
            break
    t_step = time.time() - t0
    return {"value": round(reps * bs * wl.Qs / t_step, 4), "unit": "tokens/s",
            "cores": min(threads, bs), "kind": "oracle",
            "sample": f"{reps} decode step(s) of {bs} of {B} sequences through all "
                      f"{len(inp.layers)} layers, {t_step:.1f}s on {min(threads, bs)} host threads "
                      f"(OpenMP over sequences; cache packing untimed, {t_setup:.1f}s)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=2, choices=[1, 2, 3, 5])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-fp4-index", action="store_true")
    ap.add_argument("--no-hier", action="store_true")
    ap.add_argument("--traffic-probe", action="store_true")
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
    ms_step, ms_scan, inp, groups = run_gpu(wl, args.steps, args.warmup, device)
    total_bytes, scan_bytes = algorithmic_bytes(wl)
    achieved = scan_bytes / (ms_scan * 1e-3) / 1e9
    tokens = wl.B * wl.Qs
    res = {
        "metric": "CSA2 decode tokens/s + achieved HBM GB/s (frac. of peak) at 1 MI355X",
        "value": round(tokens / (ms_step * 1e-3), 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64",
        "dtype_detail": "exact index scores accumulated in f64 from bf16/e4m3 keys; attention in "
                        "f32 over FP4 e2m1 entries and bf16 window rows",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": wl.B, "entries": wl.N, "layers": list(wl.pattern) * wl.groups,
                   "index": f"{wl.H_I}x{wl.d_I} {wl.idx_dtype}", "k": wl.k, "heads": wl.Hq,
                   "head_dim": wl.D, "window": wl.W},
        "step_hbm": {"algorithmic_bytes": total_bytes,
                     "GBps": round(total_bytes / (ms_step * 1e-3) / 1e9, 1),
                     "frac": round(total_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)},
        "roofline": {"kernel": "score_exact_kernel (exact index-score stream)", "bound": "hbm",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic() if wl.name == TRAFFIC_WORKLOAD else None,
                     "bytes_per_launch": scan_bytes, "avg_launch_us": round(ms_scan * 1e3, 2)},
    }
    res["cache"] = cache_accounting(wl)
    res["host_tier"] = host_tier(groups[0])
    del groups
    if not args.no_verify:
        vw = ALL[6]
        ms_v, _, _, _ = run_gpu(vw, max(args.steps // 2, 3), 2, device, scan_loop=False)
        res["verify5"] = {
            "workload": vw.name, "ms_per_step": round(ms_v, 4),
            "tokens_per_s": round(vw.B * vw.Qs / (ms_v * 1e-3), 1),
            "note": "draft block of 5 queries per sequence through the same 4-layer group; tokens/s "
                    "counts the 5 verified positions of each of the 32 sequences per step"}
    if not args.no_fp4_index:
        fw = ALL[7]
        ms_f, ms_fscan, _, _ = run_gpu(fw, max(args.steps // 2, 3), 2, device)
        _, f_scan_bytes = algorithmic_bytes(fw)
        res["fp4_index"] = {
            "workload": fw.name, "ms_per_step": round(ms_f, 4),
            "tokens_per_s": round(fw.B * fw.Qs / (ms_f * 1e-3), 1),
            "score_us": round(ms_fscan * 1e3, 2),
            "score_GBps": round(f_scan_bytes / (ms_fscan * 1e-3) / 1e9, 1),
            "note": "the w2 step with FP4 e2m1 index keys (fp32 block-32 scales, bf16 index queries); "
                    "scores still exact"}
    if not args.no_hier:
        hw = ALL[8]
        ms_h, _, _, _ = run_gpu(hw, max(args.steps // 2, 3), 2, device, scan_loop=False)
        res["hierarchical"] = {
            "workload": hw.name, "ms_per_step": round(ms_h, 4),
            "tokens_per_s": round(hw.B * hw.Qs / (ms_h * 1e-3), 1),
            "pool": f"{hw.pool_blocks} blocks x 8 = {hw.pool_blocks * 8} candidates per row",
            "note": "the w2 step with hierarchical search: Full scores all entries and keeps the pool, "
                    "Reindex scores and ranks only the pool's entries"}
    if not args.no_prefill:
        pw = ALL[4]
        ms_chunk = run_prefill(pw, 5, 2, device)
        flops = prefill_index_flops(pw)
        res["prefill"] = {
            "workload": pw.name, "ms_per_chunk": round(ms_chunk, 4),
            "tokens_per_s": round(pw.Qs / (ms_chunk * 1e-3), 1),
            "index_flops": flops,
            "index_tflops_over_whole_chunk": round(flops / (ms_chunk * 1e-3) / 1e12, 1),
            "note": "whole Full layer (sampled threshold, MFMA score filter, exact band selection, "
                    "attention); per-kernel MFMA figures are in profiles/"}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, inp)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
