#!/usr/bin/env python3
"""Decode-step benchmark of the PN-Mix key-cache path on one MI355X.

One step = one generation step of every layer through the library: one fused call per layer
places the new key/value rows and attends over sinks + packed pages + fp16 residual
(pnmix_append_decode_attn), and -- whenever a residual buffer reaches N tokens -- it is
quantized into a page (pnmix_quantize_kv_pages, pnmix_commit_page).  The caches are built
before timing from seeded synthetic inputs (prefill score of the first P tokens, bulk page
quantization); W warm-up steps run eagerly, then the K timed steps are captured once in a HIP
graph and replayed between device synchronisations, so host launch overhead stays out of the
timed region.  A workload with fewer than `--min-layers` layers is run over that many distinct
copies of its layer (different seeds), so that the caches touched per step exceed the on-die
last-level cache and every step reads HBM.

Prints ONE JSON line: throughput in KV token-heads per second (sum over steps and layers of
B * cached tokens * H_kv / elapsed), the decode call's roofline (algorithmic bytes per call /
event-timed duration of the call: median, p10 and p90 over >= 20 replays), a plain device copy's
bandwidth beside it, page-quantization and prefill-score sub-measurements, and the CPU oracle
timed on a bounded sample of the same workload.  The default workload is the largest one that
fits one GPU: Qwen3-32B shape, 64 layers, B = 32, 32K cached tokens (46 GB of packed cache).
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

HBM_PEAK_GBS = 8000.0
DEFAULT_WORKLOAD = "qwen3-32b-64L-b32-32k"


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def decode_bytes(cfg, lens, B, kpb, vpb):
    """Algorithmic bytes of one decode call: packed pages, fp16 sink/residual rows, mask,
    queries and fp32 outputs, over the B sequences and their KV heads."""
    s, n_p, r = lens
    ng = cfg.H_q // cfg.H_kv
    words = (cfg.d // 2 + 31) // 32
    per_head = n_p * (kpb + vpb) + (s + r) * cfg.d * 2 * 2 + words * 4 + ng * cfg.d * (2 + 4)
    return B * (per_head * cfg.H_kv + 16)


ROOT = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(ROOT, "decode_attention_pnmix_amd", "csrc")
DECODE_SRCS = [os.path.join(CSRC, f) for f in ("decode.hip", "decode_args.h", "common.h")]
PROFILES = os.path.join(ROOT, "profiles")
COPY_MB = 256  # plain device copy that calibrates the HBM byte counters


def _sha(paths):
    import hashlib
    h = hashlib.sha256()
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload, call_bytes):
    """HBM bytes per decode call from the committed counter summary of this workload, scaled by
    the ratio of algorithmic bytes (the call measured here may hold a few more or fewer tokens
    than the profiled one), or None when there is no summary or the decode kernels changed
    since the counters were taken."""
    path = os.path.join(PROFILES, f"decode_attn_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("decode_src_sha256_16") != _sha(DECODE_SRCS) or not t.get("algorithmic_bytes"):
        return None
    return t["hbm_bytes_per_call"] * call_bytes / t["algorithmic_bytes"]


def _csv_rows(d, suffix):
    import csv
    import glob
    out = []
    for fn in glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True):
        with open(fn) as f:
            out += list(csv.DictReader(f))
    return out


def pmc_summary(fetch_dir, write_dir, workload, lens, call_bytes):
    """Summarise two rocprofv3 --pmc runs of this script (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch), each scaled by the ratio of the known bytes of the calibration copy to what the
    same counter reads for it: the decode call at the last decode of the run (split + merge
    kernel, the roofline call), and for every pnmix kernel its bytes per workgroup over all its
    dispatches (a page for the quantizers, a 64-token chunk of one head for the score)."""
    res, per_kernel = {}, {}
    for name, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rs = [r for r in _csv_rows(d, "counter_collection.csv") if r["Counter_Name"] == name]
        rs.sort(key=lambda r: int(r["Dispatch_Id"]))
        # the calibration copy is the first copy dispatched after the last decode call (the run
        # makes it right there with --copy-calibration; input generation makes larger copies)
        last = max(i for i, r in enumerate(rs) if "decode_merge_kernel" in r["Kernel_Name"])
        copy = [float(r["Counter_Value"]) for r in rs[last + 1:]
                if "copybuffer" in r["Kernel_Name"].lower() or "copy" in r["Kernel_Name"].lower()]
        big = copy[0] * 1024.0
        factor = COPY_MB * 2**20 / big
        dec = [r for r in rs if "decode_kernel" in r["Kernel_Name"]]
        mrg = [r for r in rs if "decode_merge_kernel" in r["Kernel_Name"]]
        k = float(dec[-1]["Counter_Value"]) * 1024.0 * factor
        m = float(mrg[-1]["Counter_Value"]) * 1024.0 * factor
        res[name] = {"copy_counter_bytes": big, "copy_factor": factor,
                     "decode_kernel_bytes": k, "merge_kernel_bytes": m,
                     "decode_kernel_name": dec[-1]["Kernel_Name"]}
        for r in rs:
            kn = r["Kernel_Name"]
            if "pnmix::" not in kn:
                continue
            short = kn.split("(")[0].replace("void ", "")
            wgs = max(1, int(r["Grid_Size"]) // max(1, int(r["Workgroup_Size"])))
            s = per_kernel.setdefault(short, {}).setdefault(name, {"dispatches": 0,
                                                                   "bytes": 0.0, "wgs": 0})
            s["dispatches"] += 1
            s["bytes"] += float(r["Counter_Value"]) * 1024.0 * factor
            s["wgs"] += wgs
    for kn, ss in per_kernel.items():
        for name, s in ss.items():
            s["bytes_per_workgroup"] = s["bytes"] / max(1, s["wgs"])
    total = sum(res[n]["decode_kernel_bytes"] + res[n]["merge_kernel_bytes"] for n in res)
    return {"workload": workload, "lens": list(lens), "counters": res,
            "algorithmic_bytes": call_bytes, "hbm_bytes_per_call": total,
            "hbm_over_algorithmic": total / call_bytes if call_bytes else None,
            "per_kernel": per_kernel, "decode_src_sha256_16": _sha(DECODE_SRCS)}


def kt_summary(kt_dir):
    """Text table of a rocprofv3 --kernel-trace --stats run (its kernel_stats.csv): the 16
    kernels with the most time, then every other pnmix kernel."""
    rows = _csv_rows(kt_dir, "kernel_stats.csv")
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    rows = rows[:16] + [r for r in rows[16:] if "pnmix::" in r["Name"]]
    lines = [f"{'kernel':72s} {'calls':>7s} {'avg us':>9s} {'min us':>9s} {'max us':>9s} "
             f"{'time %':>7s}"]
    for r in rows:
        lines.append(f"{r['Name'][:72]:72s} {int(r['Calls']):7d} "
                     f"{float(r['AverageNs']) / 1e3:9.2f} {float(r['MinNs']) / 1e3:9.2f} "
                     f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):7.2f}")
    return "\n".join(lines)


SQ_PER_WAVE = ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS", "SQ_ACTIVE_INST_VMEM",
               "SQ_ACTIVE_INST_ANY", "SQ_WAIT_INST_LDS", "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY")
SQ_INSTS = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_INSTS_VMEM")


def sq_summary(dirs):
    """Text table of rocprofv3 --pmc runs of this script (SQ_ and TA_ counters) for every pnmix
    kernel, summed over its dispatches: the per-wave counters (quad-cycles) as fractions of the
    waves' lifetime SQ_WAVE_CYCLES, instructions per wave, LDS bank-conflict cycles per active
    LDS cycle, MFMA-busy cycles per SQ-busy cycle, and the raw sums."""
    sums, meta = {}, {}
    for d in dirs:
        for r in _csv_rows(d, "counter_collection.csv"):
            kn = r["Kernel_Name"]
            if "pnmix::" not in kn:
                continue
            short = kn.split("(")[0].replace("void ", "").replace("pnmix::", "")
            s = sums.setdefault(short, {})
            s[r["Counter_Name"]] = s.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
            m = meta.setdefault(short, {"dispatches": {}, "lds": r.get("LDS_Block_Size", "?")})
            m["dispatches"].setdefault(d, set()).add(r["Dispatch_Id"])
    lines = []
    for kn in sorted(sums, key=lambda k: -sums[k].get("SQ_WAVE_CYCLES", 0.0)):
        s, m = sums[kn], meta[kn]
        lines.append(f"{kn}")
        nd = max(len(x) for x in m["dispatches"].values())
        lines.append(f"  dispatches per run {nd}  static lds {m['lds']}")
        wc = s.get("SQ_WAVE_CYCLES")
        if wc:
            lines.append("  per-wave fraction of lifetime: " + "  ".join(
                f"{c[3:].lower()} {s[c] / wc:.3f}" for c in SQ_PER_WAVE if c in s))
        nw = s.get("SQ_WAVES")
        if nw:
            lines.append("  instructions per wave: " + "  ".join(
                f"{c[9:].lower()} {s[c] / nw:.1f}" for c in SQ_INSTS if c in s))
        if s.get("SQ_ACTIVE_INST_LDS") and "SQ_LDS_BANK_CONFLICT" in s:
            lines.append(f"  lds bank-conflict cycles / active lds cycles: "
                         f"{s['SQ_LDS_BANK_CONFLICT'] / s['SQ_ACTIVE_INST_LDS']:.3f}")
        if s.get("SQ_BUSY_CYCLES") and "SQ_VALU_MFMA_BUSY_CYCLES" in s:
            lines.append(f"  mfma busy cycles / sq busy cycles: "
                         f"{s['SQ_VALU_MFMA_BUSY_CYCLES'] / s['SQ_BUSY_CYCLES']:.3f}")
        lines.append("  sums: " + "  ".join(f"{c} {v:.4g}" for c, v in sorted(s.items())))
    return "\n".join(lines)


def build_layer(w, cfg, layer, B, T0, max_pages, steps, dev, P, synth, torch):
    """Cache of one layer holding tokens [0, T0) and the inputs of `steps` decode steps."""
    npairs = w.d // 2
    sq = synth.pair_scales(w.H_q, npairs, w.sigma_ln, dev, w.name, layer, "q")
    sk = synth.pair_scales(w.H_kv, npairs, w.sigma_ln, dev, w.name, layer, "k")
    k = synth.rope_tokens(sk, B, torch.arange(T0 + steps, device=dev), w.d, w.pairing,
                          w.rope_base, dev, w.name, layer, "k")
    v = synth.values(B, w.H_kv, T0 + steps, w.d, dev, w.name, layer)
    qp = synth.rope_tokens(sq, B, torch.arange(w.P, device=dev), w.d, w.pairing, w.rope_base,
                           dev, w.name, layer, "qpre")
    qs = synth.rope_tokens(sq, B, torch.arange(T0, T0 + steps, device=dev), w.d, w.pairing,
                           w.rope_base, dev, w.name, layer, "qdec")
    c = P.PNMixLayerCache(cfg, B, max_pages, dev)
    c.prefill(qp, k[:, :, :w.P].contiguous(), v[:, :, :w.P].contiguous())
    s = min(T0, w.N_s)
    n_pages = (T0 - s) // w.N
    if n_pages:
        kj, _ = c.page_jobs(k, s, 0, n_pages)
        _, vj = c.page_jobs(v, s, 0, n_pages)
        P.pnmix_quantize_kv_pages(cfg, kj, vj, c.mask)
    a = s + n_pages * w.N
    rest = T0 - a
    c.k_res[:, :, :rest] = k[:, :, a:T0]
    c.v_res[:, :, :rest] = v[:, :, a:T0]
    c.sink_len, c.n_pages, c.res_len = s, n_pages, rest
    c._sync_lens()
    # per-step inputs [steps][B][H][d], contiguous per step
    q_steps = qs.permute(2, 0, 1, 3).contiguous()
    k_steps = k[:, :, T0:T0 + steps].permute(2, 0, 1, 3).contiguous()
    v_steps = v[:, :, T0:T0 + steps].permute(2, 0, 1, 3).contiguous()
    torch.cuda.synchronize()
    return c, q_steps, k_steps, v_steps, (k, v, qp, qs)


def cpu_baseline(w, sample, seconds, threads):
    """Time the oracle's float64 decode attention on sampled sequences of the workload."""
    import numpy as np
    import oracle
    oracle.build(force=False)
    oc = oracle.Cfg(w.H_q, w.H_kv, w.d, w.pairing, w.n_hi_pairs, G=w.G, b_H=w.b_H, b_L=w.b_L,
                    b_V=w.b_V, g_V=w.g_V,
                    N_s=w.N_s, N=w.N)
    sm = float(np.float32(1.0 / math.sqrt(w.d)))
    prepared = []
    t_score = t_quant = 0.0
    score_bytes = quant_bytes = 0
    for (qp_b, k_b, v_b, qd_b, T) in sample:
        t0 = time.perf_counter()
        _, _, _, mask = oracle.score_prefill(oc, qp_b, k_b[:, :w.P])
        t_score += time.perf_counter() - t0
        score_bytes += (w.H_q + w.H_kv) * w.P * w.d * 2
        s = min(T, w.N_s)
        n_pages = (T - s) // w.N
        kp = np.zeros((w.H_kv, max(n_pages, 1), oracle.k_page_bytes(oc)), np.uint8)
        vp = np.zeros((w.H_kv, max(n_pages, 1), oracle.v_page_bytes(oc)), np.uint8)
        jobs = [(h, p) for h in range(w.H_kv) for p in range(n_pages)]

        def qj(j, k_b=k_b, v_b=v_b, mask=mask, kp=kp, vp=vp, s=s):
            h, p = j
            kp[h, p] = oracle.quantize_k_page(oc, k_b[h, s + p * w.N:s + (p + 1) * w.N], mask[h])
            vp[h, p] = oracle.quantize_v_page(oc, v_b[h, s + p * w.N:s + (p + 1) * w.N])

        t0 = time.perf_counter()
        oracle.parallel_map(qj, jobs, threads)
        t_quant += time.perf_counter() - t0
        quant_bytes += len(jobs) * (2 * w.N * w.d * 2 + oracle.k_page_bytes(oc) +
                                    oracle.v_page_bytes(oc))
        a = s + n_pages * w.N
        ks = np.zeros((w.H_kv, w.N_s, w.d), np.uint16)
        vs = np.zeros_like(ks)
        ks[:, :s], vs[:, :s] = k_b[:, :s], v_b[:, :s]
        kr = np.zeros((w.H_kv, w.N, w.d), np.uint16)
        vr = np.zeros_like(kr)
        kr[:, :T - a], vr[:, :T - a] = k_b[:, a:T], v_b[:, a:T]
        prepared.append((qd_b, ks, vs, kp, vp, kr, vr, mask, s, n_pages, T - a, T))

    def run(i):
        qd_b, ks, vs, kp, vp, kr, vr, mask, s, n_p, r, T = prepared[i % len(prepared)]
        oracle.decode_attn_f64(oc, qd_b, ks, vs, kp, vp, kr, vr, mask, s, n_p, r, sm)
        return T * w.H_kv

    t0 = time.perf_counter()
    run(0)
    t_one = time.perf_counter() - t0
    n_items = max(threads, int(seconds * threads / max(t_one, 1e-3)))
    n_items = (n_items + threads - 1) // threads * threads
    t0 = time.perf_counter()
    work = sum(oracle.parallel_map(run, range(n_items), threads))
    el = time.perf_counter() - t0
    n_pg = quant_bytes // (2 * w.N * w.d * 2 + oracle.k_page_bytes(oc) + oracle.v_page_bytes(oc))
    return {"value": work / el, "unit": "KV token-heads/s", "cores": threads, "kind": "oracle",
            "sample": (f"float64 decode attention (the oracle's dequantize-then-softmax) of "
                       f"{n_items} sequence-layers drawn from {len(prepared)} sampled sequences "
                       f"(T={sample[0][4]}, {w.H_kv} KV heads, {w.H_q} query heads), "
                       f"{el:.1f} s wall on {threads} threads; page quantization and prefill "
                       f"score timed separately below"),
            "page_quant": {"value": quant_bytes / max(t_quant, 1e-9) / 1e9, "unit": "GB/s",
                           "cores": threads, "kind": "oracle",
                           "sample": f"{n_pg} K+V page pairs of the sampled sequences, "
                                     f"{t_quant:.2f} s wall"},
            "prefill_score": {"value": score_bytes / max(t_score, 1e-9) / 1e9, "unit": "GB/s",
                              "cores": 1, "kind": "oracle",
                              "sample": f"P={w.P} prompt, {len(prepared)} sequence(s), "
                                        f"{t_score:.3f} s wall (single-threaded)"}}


def prefill_timing(w, cfg, P, synth, torch, np, reps=6):
    """The prompt of one layer, scored and its full pages quantized: score then one launch of key
    and value pages (pnmix_score_prefill + pnmix_quantize_kv_pages) against the one-pass
    pnmix_prefill_fused; median of `reps` event-timed runs each, for the workload's prompt at
    its batch and its long prompt at B = 1 if it has one.  The fused entry point packs the
    (b_H, b_L, b_V) = (3, 1, 2) widths only; other widths time the two-step sequence alone."""
    dev = "cuda"
    out = {}
    fused = (w.b_H, w.b_L, w.b_V) == (3, 1, 2)
    for (Bs, Ps) in ([(w.B, w.P)] + ([(1, w.prefill_score_P)] if w.prefill_score_P else [])):
        sq = synth.pair_scales(w.H_q, w.d // 2, w.sigma_ln, dev, w.name, 0, "q")
        sk = synth.pair_scales(w.H_kv, w.d // 2, w.sigma_ln, dev, w.name, 0, "k")
        qpp = synth.rope_tokens(sq, Bs, torch.arange(Ps, device=dev), w.d, w.pairing,
                                w.rope_base, dev, w.name, "prefill", "q")
        kpp = synth.rope_tokens(sk, Bs, torch.arange(Ps, device=dev), w.d, w.pairing,
                                w.rope_base, dev, w.name, "prefill", "k")
        vpp = synth.values(Bs, w.H_kv, Ps, w.d, dev, w.name, "prefill")
        n_full = max(0, (Ps - w.N_s) // w.N)
        c = P.PNMixLayerCache(cfg, Bs, max(n_full, 1), dev)
        kj = vj = None
        if n_full:
            kj, _ = c.page_jobs(kpp, w.N_s, 0, n_full)
            _, vj = c.page_jobs(vpp, w.N_s, 0, n_full)
        ws_s = torch.empty(P.pnmix_score_workspace_bytes(cfg, Bs, Ps), dtype=torch.uint8,
                           device=dev)
        ws_f = torch.empty(P.pnmix_prefill_fused_workspace_bytes(cfg, Bs, Ps) if fused else 256,
                           dtype=torch.uint8, device=dev)
        tu, tf = [], []
        for rep in range(reps + 1):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            _, m = P.pnmix_score_prefill(cfg, qpp, kpp, ws=ws_s, want_sigma=False)
            if n_full:
                c.mask.copy_(m)
                P.pnmix_quantize_kv_pages(cfg, kj, vj, c.mask)
            e[1].record()
            if fused:
                P.pnmix_prefill_fused(cfg, qpp, kpp, vpp, c.k_pages, c.v_pages, mask=c.mask,
                                      ws=ws_f, want_sigma=False)
            e[2].record()
            torch.cuda.synchronize()
            if rep:
                tu.append(e[0].elapsed_time(e[1]) * 1e3)
                tf.append(e[1].elapsed_time(e[2]) * 1e3)
        nb_read = Bs * Ps * (w.H_q + 2 * w.H_kv) * w.d * 2
        out[f"B{Bs}_P{Ps}"] = {"pages_per_kv_head": n_full,
                               "score_then_quantize_us": float(np.median(tu))}
        if fused:
            out[f"B{Bs}_P{Ps}"].update({"fused_us": float(np.median(tf)),
                                        "fused_GBps_of_qkv_read":
                                            nb_read / float(np.median(tf)) / 1e3})
        del qpp, kpp, vpp, c
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--min-layers", type=int, default=16,
                    help="run a workload with fewer layers over this many distinct layer copies")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--roofline-reps", type=int, default=24,
                    help="timed replays of the per-layer decode calls (p10 / median / p90)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help=f"run one plain {COPY_MB} MiB device copy (HBM counter calibration)")
    ap.add_argument("--profile-step", action="store_true",
                    help="stop after the decode-call timing (short runs under a profiler)")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs of this script and exit (no GPU)")
    ap.add_argument("--lens", type=int, nargs=3, metavar=("SINK", "PAGES", "RES"),
                    help="with --pmc-summary: the cache lengths of the profiled decode call")
    ap.add_argument("--call-bytes", type=int,
                    help="with --pmc-summary: algorithmic bytes of the profiled decode call")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time the prompt's scoring and page quantization (fused and unfused) "
                         "for the workload's prompts and exit")
    ap.add_argument("--kt-summary", metavar="KT_DIR",
                    help="print the kernel table of a rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--bits", type=int, nargs=3, metavar=("B_H", "B_L", "B_V"),
                    help="run the workload with these key and value bit widths (the sweep of the "
                         "PN-Mix paper's bit-width appendix; any width but (3, 1, 2) takes the "
                         "generic decode kernel)")
    ap.add_argument("--gv", type=int, help="value group size g_V for --bits (default: the workload's)")
    ap.add_argument("--sq-summary", nargs="+", metavar="PMC_DIR",
                    help="print the SQ/TA counter table of rocprofv3 --pmc runs and exit")
    args = ap.parse_args()
    if args.kt_summary:
        print(kt_summary(args.kt_summary))
        return
    if args.sq_summary:
        print(sq_summary(args.sq_summary))
        return
    if args.pmc_summary:
        print(json.dumps(pmc_summary(args.pmc_summary[0], args.pmc_summary[1], args.workload,
                                     args.lens, args.call_bytes), indent=1))
        return
    if args.gpus != 1:
        print(f"bench.py: the benchmark runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by sequence and KV head with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import decode_attention_pnmix_amd as P
    import synth

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = "cuda"
    w = synth.WORKLOADS[args.workload]
    if args.bits or args.gv:
        import dataclasses
        bh, bl, bv = args.bits or (w.b_H, w.b_L, w.b_V)
        gv = args.gv or w.g_V
        w = dataclasses.replace(w, name=f"{w.name}-h{bh}l{bl}v{bv}g{gv}", b_H=bh, b_L=bl, b_V=bv,
                                g_V=gv)
    cfg = P.make_cfg(w.H_q, w.H_kv, w.d, w.pairing, w.n_hi_pairs, G=w.G, b_H=w.b_H, b_L=w.b_L,
                     b_V=w.b_V, g_V=w.g_V, N_s=w.N_s, N=w.N)
    if args.prefill_only:
        print(json.dumps({"workload": w.name, "prefill": prefill_timing(w, cfg, P, synth, torch,
                                                                        np)}), flush=True)
        return
    kpb, vpb = P.pnmix_k_page_bytes(cfg), P.pnmix_v_page_bytes(cfg)
    W, K = args.warmup, args.steps
    layers = max(w.layers, args.min_layers)
    # the first timed step attends over exactly w.T tokens
    T0 = w.T - W - 1
    max_pages = (T0 + W + K - w.N_s) // w.N + 1
    _say(f"[bench] workload={w.name} layers={w.layers} (run over {layers}) B={w.B} T0={T0} "
         f"steps={K} warmup={W} max_pages={max_pages}")

    caches, inputs, sample = [], [], []
    n_sample = 4
    t_build = time.perf_counter()
    for layer in range(layers):
        c, qst, kst, vst, raw = build_layer(w, cfg, layer, w.B, T0, max_pages, W + K, dev, P,
                                            synth, torch)
        caches.append(c)
        inputs.append((qst, kst, vst))
        if layer == 0 and not args.no_cpu_baseline:
            k, v, qp, qs = raw
            u16 = lambda t: t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
            for b in range(min(n_sample, w.B)):
                sample.append((u16(qp[b]), u16(k[b, :, :T0]), u16(v[b, :, :T0]),
                               u16(qs[b, :, 0]), T0))
        del raw
        for s in range(c.n_pages, max_pages):  # page jobs of every flush slot, built up front
            c.flush_jobs(s)
        if layer % 8 == 7:
            _say(f"[bench] {layer + 1} layers built ({time.perf_counter() - t_build:.1f} s)")
    torch.cuda.synchronize()
    _say(f"[bench] caches built in {time.perf_counter() - t_build:.1f} s")

    outs = [torch.empty(w.B, w.H_q, w.d, dtype=torch.float32, device=dev) for _ in caches]

    def run_step(i, lens_log=None):
        for layer, c in enumerate(caches):
            qst, kst, vst = inputs[layer]
            c.step(qst[i], kst[i], vst[i], outs[layer])  # append + attend, then flush if full
            if lens_log is not None and layer == 0:
                lens_log.append((c.sink_len, c.n_pages, c.res_len))

    for i in range(W):
        run_step(i)
    torch.cuda.synchronize()

    # ---- capture the K timed steps once, then replay them from the same starting state
    saved_lens = [c.lens.clone() for c in caches]
    saved_host = [(c.sink_len, c.n_pages, c.res_len) for c in caches]
    # a step reads one lengths buffer and writes the other; the graph's first step reads these
    saved_bufs = [(c.lens, c._lens_next) for c in caches]
    lens_log = []
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(W, W + K):
            run_step(i, lens_log)

    def restore():
        for c, sl, sh, bufs in zip(caches, saved_lens, saved_host, saved_bufs):
            c.lens, c._lens_next = bufs
            c.lens.copy_(sl)
            c.sink_len, c.n_pages, c.res_len = sh
        torch.cuda.synchronize()

    restore()
    graph.replay()  # untimed pass over the captured steps
    restore()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    graph.replay()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tokheads = sum(layers * w.B * (s + n_p * w.N + r) * w.H_kv for (s, n_p, r) in lens_log)
    value = tokheads / elapsed
    _say(f"[bench] {K} steps x {layers} layers in {elapsed * 1e3:.2f} ms "
         f"({elapsed / K * 1e3:.3f} ms/step)")

    # ---- decode-call roofline: every layer's call timed with HIP events on torch's stream
    # (the stream the library launches on), state after the timed steps
    restore()
    for i in range(W, W + K):  # replay eagerly to the end state so lens match the host
        run_step(i)
    torch.cuda.synchronize()
    lens_now = (caches[0].sink_len, caches[0].n_pages, caches[0].res_len)
    qlast = [inputs[l][0][W + K - 1] for l in range(layers)]
    # the layers' calls are captured once in a HIP graph and replayed back to back between one
    # pair of events on the launch stream, so host launch overhead stays out of the per-call
    # time; the first replay is a warm-up
    call_graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(call_graph):
        for layer, c in enumerate(caches):
            c.attend(qlast[layer], outs[layer])
    torch.cuda.synchronize()
    durs = []
    for rep in range(args.roofline_reps + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call_graph.replay()
        e1.record()
        torch.cuda.synchronize()
        if rep:
            durs.append(e0.elapsed_time(e1) * 1e-3 / layers)
    call_s = float(np.median(durs))
    call_p10, call_p90 = float(np.percentile(durs, 10)), float(np.percentile(durs, 90))
    call_bytes = decode_bytes(cfg, lens_now, w.B, kpb, vpb)
    achieved = call_bytes / call_s / 1e9
    _say(f"[bench] decode call: {call_bytes / 1e6:.2f} MB in {call_s * 1e6:.2f} us median "
         f"(p10 {call_p10 * 1e6:.2f}, p90 {call_p90 * 1e6:.2f}) -> {achieved:.0f} GB/s")
    traffic = measured_traffic(w.name, call_bytes)
    _say(f"[bench] decode call lens (sink, pages, residual) = {lens_now}, "
         f"algorithmic bytes {call_bytes}")
    if args.copy_calibration:
        src = torch.empty(COPY_MB * 2**20 // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.profile_step:
        print(json.dumps({"profile_step": True, "workload": w.name, "lens": lens_now,
                          "call_bytes": call_bytes, "call_us": call_s * 1e6}), flush=True)
        return

    # ---- a plain device-to-device copy of 1 GiB: the HBM rate this machine reaches
    cp_src = torch.empty(2**28, dtype=torch.float32, device=dev).fill_(1.0)
    cp_dst = torch.empty_like(cp_src)
    cts = []
    for rep in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        cp_dst.copy_(cp_src)
        e1.record()
        torch.cuda.synchronize()
        if rep:
            cts.append(e0.elapsed_time(e1) * 1e-3)
    copy_GBps = 2 * cp_src.numel() * 4 / float(np.median(cts)) / 1e9
    del cp_src, cp_dst
    _say(f"[bench] device copy: {copy_GBps:.0f} GB/s (read + write)")

    # ---- page quantization: one fill event of every layer's residual buffers, key and value
    # pages in one launch (and, for reference, as two launches)
    n_jobs = layers * w.B * w.H_kv
    scratch_k = torch.empty(n_jobs, kpb, dtype=torch.uint8, device=dev)
    scratch_v = torch.empty(n_jobs, vpb, dtype=torch.uint8, device=dev)
    srcs_k, srcs_v, dk, dv, rows = [], [], [], [], []
    masks = torch.cat([c.mask.reshape(-1, c.mask.shape[-1]) for c in caches]).contiguous()
    for layer, c in enumerate(caches):
        for bh in range(w.B * w.H_kv):
            j = layer * w.B * w.H_kv + bh
            srcs_k.append(c.k_res.data_ptr() + bh * w.N * w.d * 2)
            srcs_v.append(c.v_res.data_ptr() + bh * w.N * w.d * 2)
            dk.append(scratch_k.data_ptr() + j * kpb)
            dv.append(scratch_v.data_ptr() + j * vpb)
            rows.append(j)
    kj = P.page_jobs(srcs_k, w.d, dk, rows, dev)
    vj = P.page_jobs(srcs_v, w.d, dv, rows, dev)
    qkv_t, qk_t, qv_t = [], [], []
    for rep in range(8):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        P.pnmix_quantize_kv_pages(cfg, kj, vj, masks)
        e[1].record()
        P.pnmix_quantize_k_page(cfg, kj, masks)
        e[2].record()
        P.pnmix_quantize_v_page(cfg, vj)
        e[3].record()
        torch.cuda.synchronize()
        if rep:
            qkv_t.append(e[0].elapsed_time(e[1]) * 1e-3)
            qk_t.append(e[1].elapsed_time(e[2]) * 1e-3)
            qv_t.append(e[2].elapsed_time(e[3]) * 1e-3)
    tkv, tk, tv = (float(np.median(x)) for x in (qkv_t, qk_t, qv_t))
    kbytes = n_jobs * (w.N * w.d * 2 + kpb)
    vbytes = n_jobs * (w.N * w.d * 2 + vpb)
    qkern = ("quantize_kv_kernel" if (w.b_H, w.b_L, w.b_V) == (3, 1, 2)
             else "quantize_kv_generic_kernel")
    quant = {"pages_per_launch": 2 * n_jobs, "kernel": f"{qkern} (K and V pages in one launch)",
             "kv_us": tkv * 1e6, "kv_us_p10": float(np.percentile(qkv_t, 10)) * 1e6,
             "kv_us_p90": float(np.percentile(qkv_t, 90)) * 1e6,
             "kv_GBps": (kbytes + vbytes) / tkv / 1e9,
             "kv_frac_of_peak": (kbytes + vbytes) / tkv / 1e9 / HBM_PEAK_GBS,
             "separate_launches": {"k_us": tk * 1e6, "v_us": tv * 1e6,
                                   "k_GBps": kbytes / tk / 1e9, "v_GBps": vbytes / tv / 1e9}}
    _say(f"[bench] page quant, {2 * n_jobs} pages in one launch: {tkv * 1e6:.1f} us, "
         f"{quant['kv_GBps']:.0f} GB/s ({quant['kv_frac_of_peak'] * 100:.1f}%)")
    del scratch_k, scratch_v

    # ---- prefill score of one layer's prompt batch (and the long prefill if the workload has one)
    prefill = prefill_timing(w, cfg, P, synth, torch, np)
    score = {}
    for (Bs, Ps) in ([(w.B, w.P)] + ([(1, w.prefill_score_P)] if w.prefill_score_P else [])):
        sq = synth.pair_scales(w.H_q, w.d // 2, w.sigma_ln, dev, w.name, 0, "q")
        sk = synth.pair_scales(w.H_kv, w.d // 2, w.sigma_ln, dev, w.name, 0, "k")
        qpp = synth.rope_tokens(sq, Bs, torch.arange(Ps, device=dev), w.d, w.pairing,
                                w.rope_base, dev, w.name, "score", "q")
        kpp = synth.rope_tokens(sk, Bs, torch.arange(Ps, device=dev), w.d, w.pairing,
                                w.rope_base, dev, w.name, "score", "k")
        ws = torch.empty(P.pnmix_score_workspace_bytes(cfg, Bs, Ps), dtype=torch.uint8,
                         device=dev)
        ts = []
        for rep in range(6):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            P.pnmix_score_prefill(cfg, qpp, kpp, ws=ws, want_sigma=False)
            e1.record()
            torch.cuda.synchronize()
            if rep:
                ts.append(e0.elapsed_time(e1) * 1e-3)
        t = float(np.median(ts))
        nb = Bs * Ps * (w.H_q + w.H_kv) * w.d * 2
        score[f"B{Bs}_P{Ps}"] = {"us": t * 1e6, "GBps": nb / t / 1e9}

    cpu = None
    if not args.no_cpu_baseline and sample:
        host_cpus = os.cpu_count() or 1
        try:
            affinity = len(os.sched_getaffinity(0))
        except AttributeError:
            affinity = host_cpus
        # the machine's CPU share for one GPU caps the pool (OMP_NUM_THREADS states it there)
        share = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or affinity
        threads = max(1, min(affinity, share))
        cpu = cpu_baseline(w, sample, args.cpu_seconds, threads)
        cpu["host_cpus"] = host_cpus
        cpu["affinity_cpus"] = affinity

    line = {
        "metric": "decode-attn KV tokens·heads/s & % of HBM peak; K/V page-quant GB/s",
        "value": value,
        "unit": "KV token-heads/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": elapsed / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp16 in / packed u8 cache / fp32 attention",
        "data": "synthetic (seeded; log-normal persistent pair outliers, RoPE, V ~ N(0,1))",
        "config": {"workload": w.name, "layers": w.layers, "layer_copies_per_step": layers,
                   "global_batch": w.B, "kv_tokens_at_first_timed_step": w.T, "H_q": w.H_q,
                   "H_kv": w.H_kv, "head_dim": w.d, "r": w.r, "G": w.G, "b_H": w.b_H,
                   "b_L": w.b_L, "b_V": w.b_V, "g_V": w.g_V, "N_s": w.N_s, "N": w.N,
                   "parallelism": "single GPU", "timed": "one HIP graph of K steps"},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": ("pnmix_decode_attn = decode_kernel (page and fp16 splits) + "
                                "decode_merge_kernel, one call per layer"
                                if (w.b_H, w.b_L, w.b_V) == (3, 1, 2) and w.g_V >= 32 else
                                "pnmix_decode_attn = decode_generic_kernel (vector ALU, every "
                                "chunk of 128 tokens) + decode_merge_kernel, one call per layer"),
                     "bytes_per_call": call_bytes, "avg_call_us": call_s * 1e6,
                     "call_us_p10": call_p10 * 1e6, "call_us_p90": call_p90 * 1e6,
                     "timed_replays": len(durs), "lens": list(lens_now),
                     "device_copy_GBps": copy_GBps,
                     "frac_of_device_copy": achieved / copy_GBps},
        "page_quant": quant,
        "prefill_score": score,
        "prefill": prefill,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
