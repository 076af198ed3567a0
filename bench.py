#!/usr/bin/env python3
"""Benchmark of the quantised-base LoRA hot path on one MI355X.

A step is the fused dequant-GEMM + LoRA forward and fast backward of the
dense Q4_0 linear layer (T 2048 tokens, 2048 -> 6144, rank 4, alpha 8):
gq_linear_lora_fwd + gq_linear_lora_bwd on inputs already resident in HBM.
`value` is its algorithmic TFLOP/s.  The same JSON line also carries the
routed MoE layer (Q4_0, 2048 tokens, hidden 2048, 128 experts top-8,
intermediate 768, rank 4) train tokens/s, the roofline of the dominant MMQ
kernel (timed with HIP events that the kernel dispatch itself stamps, in a
pass of the same steps beside the timed one) and the fp64 oracle timed on the
host cores.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]

The default run also times every other workload on its own line entry:
the Q8_0 linear layer (T 128), the 2-bit Zipf MoE layer (T 4096, 256
experts), the LM head with chunked cross entropy (T 2048, V 151936), the
small-token sweep (grouped layer T 16-512, LM-head forward T 16-128),
RMSNorm and the 8-bit AdamW step, each against its roofline.  Every GPU
time is the median of 5 repeats of K back-to-back steps (spread reported).
--quick keeps only the headline linear step and the Q4_0 MoE layer.

HBM traffic of the two MMQ launches: run the step under two rocprofv3
counter passes with a plain device copy of known size in the same process,

    rocprofv3 --pmc FETCH_SIZE -d F -o run --output-format csv -- \\
        python3 bench.py --eager --copy-probe --no-cpu --steps 2 --warmup 1 --repeats 1
    rocprofv3 --pmc WRITE_SIZE -d W -o run --output-format csv -- (same)

then `python bench.py --traffic-from F/run_counter_collection.csv
W/run_counter_collection.csv "<the bench arguments of those runs>"` (no GPU
needed) scales each counter by what it reads for the copy and writes
profiles/mmq_traffic.json and its summary.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import shlex
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def linear_flops(T, K, N, r):
    # fwd: 2TNK + 2TKr + 2TNr ; bwd: dX 2TNK + 2TNr + 2TKr, dB 2TNr, dA 2TKr
    return 4 * T * N * K + 6 * T * r * (N + K)


def moe_flops(T, H, I, k, r):
    return T * k * (12 * H * I + 18 * r * (H + I))


def gemm_source_hash():
    """Hash of the MMQ kernel source with comments and blank lines dropped,
    so that counters stay attributed to the kernel until its code changes."""
    h = hashlib.sha256()
    for f in ("gq_gemm_impl.h", "gq_wide_impl.h", "gq_wide_nn_impl.h", "gq_skinny_impl.h", "gq_dev.h"):
        with open(os.path.join(ROOT, "quantized_base_lora_amd", "csrc", f)) as fh:
            for line in fh:
                code = line.split("//", 1)[0].strip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def load_traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    the counters were taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "mmq_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    ent = d.get(kernel_key)
    if not ent or ent.get("source_hash") != gemm_source_hash():
        return None
    return ent.get("hbm_bytes_per_launch")


COPY_BYTES = 256 << 20
# the two MMQ launches of the linear step: kernel name fragment, threads per
# launch (tiles x workgroup size), key in mmq_traffic.json
MMQ_LAUNCHES = (
    ("wide::wide_kernel<1, 0>", 256 * 512, "mmq_nt_lin_q4_0_t2048_2048x6144"),
    ("gemm_kernel<1, 4, 128, 128, 2>", 256 * 512, "mmq_nn_lin_bwd_q4_0_t2048_2048x6144"),
)
# kernels whose counters are kept in profiles/mmq_counters.json
MMQ_KERNEL_TAGS = ("gemm_kernel", "skinny", "wide_kernel", "wide_nn_kernel", "ce_bwd_dh_kernel")


def moe_layer_bytes(T, H, I, E, k, r, qtype_bytes, active):
    """Algorithmic HBM bytes of one routed-MoE layer fwd+bwd: the blocks of
    the active experts read once per pass (gate, up, down; forward and
    backward), token activations in and out (x, dY read; y, dx written), all
    experts' adapters read and their gradients written."""
    per_expert = (2 * I * (H // 32) + H * (I // 32)) * qtype_bytes
    weights = 2 * active * per_expert
    acts = 4 * T * H * 2
    adapters = 2 * E * 4 * r * (2 * H + I + 2 * I + H)
    return weights + acts + adapters


def write_kernel_summary(csv_dir, out_md, title):
    """rocprofv3's own --stats table, plus the same trace broken out by launch
    size (kernels of one name run at several grid sizes)."""
    import csv
    import re
    import statistics

    def short(n):
        n = n.replace("void ", "").replace("gq::(anonymous namespace)::", "").replace("gq::", "")
        return re.sub(r"\(.*", "", n)

    stats = list(csv.DictReader(open(os.path.join(csv_dir, "run_kernel_stats.csv"))))
    trace = list(csv.DictReader(open(os.path.join(csv_dir, "run_kernel_trace.csv"))))
    by = {}
    for r in trace:
        key = (short(r["Kernel_Name"]), int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"]))
        by.setdefault(key, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    total = sum(sum(v) for v in by.values())
    with open(out_md, "w") as fh:
        fh.write(f"# rocprofv3 kernel summary: {title}\n\n")
        fh.write("Command (repo root on the GPU box, TMPDIR=/tmp, run from /tmp):\n\n")
        fh.write("    rocprofv3 --kernel-trace --stats --output-format csv -d <repo>/gpurun_out/<dir> -o run -- "
                 f"python3 <repo>/bench.py {title}\n\n")
        fh.write("gemm_kernel<qtype, epilogue, BM, BN, k-groups>: qtype 0 Q8_0, 1 Q4_0, 2 2-bit; epilogue 0 linear, "
                 "1 SwiGLU, 2 CE logits, 3 CE gradient, 4 linear backward (dX), 5 SwiGLU backward, "
                 "6 gate/up backward, 7 dh accumulate; wide::wide_kernel<qtype, epilogue>: the 256 x 192 tile "
                 "(epilogue 0 linear, 2 CE logits, 3 CE gradient over up to six vocabulary chunks); "
                 "wnn::wide_nn_kernel<qtype, 7, ragged>: the LM head's dh on 256 x 128 tiles, two reduction "
                 "ranges per tile; ce_bwd_dh_kernel<qtype>: one vocabulary chunk's CE-gradient tiles with the "
                 "previous chunk's dh tiles.\n\n")
        fh.write("## rocprofv3 --stats (run_kernel_stats.csv)\n\n| kernel | calls | avg us | min us | max us | % |\n"
                 "|---|---|---|---|---|---|\n")
        for r in stats[:30]:
            fh.write(f"| {short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                     f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | {float(r['Percentage']):.1f} |\n")
        fh.write("\n## Same trace by launch size (run_kernel_trace.csv)\n\n| kernel | threads per launch | calls | "
                 "avg us | median us | % of GPU time |\n|---|---|---|---|---|---|\n")
        for (name, grid), v in sorted(by.items(), key=lambda kv: -sum(kv[1]))[:40]:
            fh.write(f"| {name} | {grid} | {len(v)} | {sum(v) / len(v):.1f} | {statistics.median(v):.1f} | "
                     f"{100 * sum(v) / total:.1f} |\n")
    log(f"wrote {out_md}")


def write_traffic(fetch_csv, write_csv, run_args, cmdline):
    """Bytes per launch of the MMQ kernels from FETCH_SIZE / WRITE_SIZE (KiB
    per dispatch), each scaled so that the reference copy reads and writes
    exactly its size."""
    import csv
    import statistics

    def per_kernel(path, counter):
        rows = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            rows.setdefault((r["Kernel_Name"], int(r["Grid_Size"])), []).append(float(r["Counter_Value"]))
        return rows

    out, lines = {}, []
    scale = {}
    for path, counter in ((fetch_csv, "FETCH_SIZE"), (write_csv, "WRITE_SIZE")):
        rows = per_kernel(path, counter)
        copy = [v for (n, g), vs in rows.items() if "copy" in n.lower() for v in vs
                if v * 1024 > 0.5 * COPY_BYTES]
        if not copy:
            raise SystemExit(f"no reference copy of {COPY_BYTES} bytes found in {path}")
        scale[counter] = statistics.median(copy) * 1024 / COPY_BYTES
        lines.append(f"| reference copy ({COPY_BYTES >> 20} MiB) | {counter} | "
                     f"{statistics.median(copy):.0f} KiB | factor {scale[counter]:.4f} |")
        for frag, grid, key in MMQ_LAUNCHES:
            vals = [v for (n, g), vs in rows.items() if frag in n and g == grid for v in vs]
            if not vals:
                raise SystemExit(f"no dispatch of {frag} (grid {grid}) in {path}")
            med = statistics.median(vals)
            bytes_ = med * 1024 / scale[counter]
            e = out.setdefault(key, {"source_hash": gemm_source_hash(), "kernel": frag})
            e["fetch_bytes" if counter == "FETCH_SIZE" else "write_bytes"] = round(bytes_)
            lines.append(f"| {frag} (grid {grid}) | {counter} | {med:.0f} KiB x {len(vals)} | "
                         f"{bytes_ / 1e6:.2f} MB per launch |")
    for e in out.values():
        e["hbm_bytes_per_launch"] = e["fetch_bytes"] + e["write_bytes"]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", "mmq_traffic.json"), "w") as fh:
        json.dump(out, fh, indent=1)
    with open(os.path.join(ROOT, "profiles", "mmq_traffic_linear_q4_0_t2048_2048x6144.md"), "w") as fh:
        fh.write("# HBM traffic of the two MMQ launches of the dense Q4_0 linear step "
                 "(T 2048, 2048 -> 6144, rank 4)\n\n")
        fh.write("Counter passes (repo root on the GPU box, TMPDIR=/tmp, run from /tmp):\n\n")
        fh.write("    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <repo>/gpurun_out/pmc_fetch -o run -- "
                 f"python3 <repo>/bench.py {run_args}\n")
        fh.write("    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <repo>/gpurun_out/pmc_write -o run -- "
                 f"python3 <repo>/bench.py {run_args}\n\n")
        fh.write(f"Summary written by: `{cmdline}`\n\n")
        fh.write("Each counter (KiB per dispatch, median over dispatches) is divided by what the same "
                 "counter reads for a plain device copy of known size in the same process.\n\n")
        fh.write("| kernel | counter | raw | scaled |\n|---|---|---|---|\n")
        fh.write("\n".join(lines) + "\n\n")
        for key, e in out.items():
            fh.write(f"- {key}: fetch {e['fetch_bytes'] / 1e6:.2f} MB + write {e['write_bytes'] / 1e6:.2f} MB"
                     f" = {e['hbm_bytes_per_launch'] / 1e6:.2f} MB per launch (source hash {e['source_hash']})\n")
    log(json.dumps(out))


def write_counters(sq_csv, fetch_csv, write_csv, out_md, title, cmdline):
    """Per-kernel counter summary of one run of the bench under three
    rocprofv3 --pmc passes (SQ counters + GRBM_GUI_ACTIVE, FETCH_SIZE,
    WRITE_SIZE): MFMA busy (the MfmaUtil formula: MFMA-busy cycles of all
    SIMDs over GUI-active cycles x SIMD count), VALU and LDS instructions per
    MFMA, LDS bank-conflict cycles per CU cycle, HBM bytes (each counter
    scaled by what it reads for the plain device copy of known size in the
    same run).  Also merges the MMQ kernels into profiles/mmq_counters.json
    under the current kernel source hash."""
    import csv
    import re
    import statistics

    def short(n):
        n = n.replace("void ", "").replace("gq::(anonymous namespace)::", "").replace("gq::", "")
        return re.sub(r"\(.*", "", n)

    SIMDS, CUS, XCDS = 1024, 256, 8
    rows = {}
    for path in (sq_csv, fetch_csv, write_csv):
        for r in csv.DictReader(open(path)):
            key = (short(r["Kernel_Name"]), int(r["Grid_Size"]))
            ent = rows.setdefault(key, {})
            ent.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if r["Counter_Name"] == "GRBM_GUI_ACTIVE":
                ent.setdefault("_dur", []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    scale = {}
    for cn in ("FETCH_SIZE", "WRITE_SIZE"):
        copy = [v for (n, g), e in rows.items() if "copy" in n.lower() for v in e.get(cn, [])
                if v * 1024 > 0.5 * COPY_BYTES]
        if not copy:
            raise SystemExit(f"no reference copy of {COPY_BYTES} bytes for {cn}")
        scale[cn] = statistics.median(copy) * 1024 / COPY_BYTES
    med = lambda e, n: statistics.median(e[n]) if n in e else float("nan")
    table = []
    for (name, grid), e in rows.items():
        if "GRBM_GUI_ACTIVE" not in e or "copy" in name.lower():
            continue
        gui = med(e, "GRBM_GUI_ACTIVE") / XCDS
        mf = med(e, "SQ_INSTS_MFMA")
        table.append({
            "kernel": name, "grid": grid, "calls": len(e["GRBM_GUI_ACTIVE"]),
            "us": statistics.median(e["_dur"]),
            "mfma_busy": med(e, "SQ_VALU_MFMA_BUSY_CYCLES") / (gui * SIMDS),
            "valu_per_mfma": med(e, "SQ_INSTS_VALU") / mf if mf else float("nan"),
            "lds_per_mfma": med(e, "SQ_INSTS_LDS") / mf if mf else float("nan"),
            "lds_conflict": med(e, "SQ_LDS_BANK_CONFLICT") / (gui * CUS),
            "fetch_mb": med(e, "FETCH_SIZE") * 1024 / scale["FETCH_SIZE"] / 1e6,
            "write_mb": med(e, "WRITE_SIZE") * 1024 / scale["WRITE_SIZE"] / 1e6,
        })
    table.sort(key=lambda t: -t["us"] * t["calls"])
    with open(out_md, "w") as fh:
        fh.write(f"# Hardware counters per kernel: {title}\n\n")
        fh.write("Three counter passes over the same run (repo root on the GPU box, TMPDIR=/tmp, run from /tmp):\n\n")
        fh.write("    rocprofv3 --pmc SQ_WAVES SQ_BUSY_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
                 "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_ACTIVE_INST_VALU GRBM_GUI_ACTIVE --output-format csv "
                 f"-d <repo>/gpurun_out/pmc_sq -o run -- python3 <repo>/bench.py {title}\n")
        fh.write("    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <repo>/gpurun_out/pmc_fetch -o run -- "
                 f"python3 <repo>/bench.py {title}\n")
        fh.write("    rocprofv3 --pmc WRITE_SIZE --output-format csv -d <repo>/gpurun_out/pmc_write -o run -- "
                 f"python3 <repo>/bench.py {title}\n\n")
        fh.write(f"Summary written by: `{cmdline}`\n\n")
        fh.write("MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCD x 1024 SIMDs) (rocprofv3's MfmaUtil); "
                 "LDS conflict = SQ_LDS_BANK_CONFLICT / (GUI-active cycles x 256 CUs); HBM MB = FETCH_SIZE / WRITE_SIZE "
                 f"divided by the factor the same counter reads for a {COPY_BYTES >> 20} MiB device copy "
                 f"(FETCH {scale['FETCH_SIZE']:.4f}, WRITE {scale['WRITE_SIZE']:.4f}).  Durations are under the "
                 "profiler (kernels serialised).  Kernel template arguments: gemm_kernel<qtype, epilogue, BM, BN, "
                 "k-groups> (qtype 0 Q8_0, 1 Q4_0, 2 2-bit; epilogue 0 linear, 1 SwiGLU, 2 CE logits, 3 CE gradient, "
                 "4 linear backward (dX), 5 SwiGLU backward, 6 gate/up backward, 7 dh accumulate); "
                 "wide::wide_kernel<qtype, epilogue> the 256 x 192 tile (epilogue 0, 2 or 3); "
                 "wnn::wide_nn_kernel<qtype, 7, ragged> the LM head's dh on 256 x 128 tiles; ce_bwd_dh_kernel<qtype> one "
                 "vocabulary chunk's CE-gradient tiles with the previous chunk's dh tiles.\n\n")
        fh.write("| kernel | threads | calls | us | MFMA busy | VALU/MFMA | LDS/MFMA | LDS conflict | HBM fetch MB | "
                 "HBM write MB |\n|---|---|---|---|---|---|---|---|---|---|\n")
        for t in table[:40]:
            fh.write(f"| {t['kernel']} | {t['grid']} | {t['calls']} | {t['us']:.1f} | {t['mfma_busy']:.3f} | "
                     f"{t['valu_per_mfma']:.2f} | {t['lds_per_mfma']:.2f} | {t['lds_conflict']:.3f} | "
                     f"{t['fetch_mb']:.1f} | {t['write_mb']:.1f} |\n")
    jpath = os.path.join(ROOT, "profiles", "mmq_counters.json")
    js = json.load(open(jpath)) if os.path.exists(jpath) else {}
    for t in table:
        if any(tag in t["kernel"] for tag in MMQ_KERNEL_TAGS):
            js[f"{t['kernel']}|{t['grid']}"] = dict(t, source_hash=gemm_source_hash())
    with open(jpath, "w") as fh:
        json.dump(js, fh, indent=1, sort_keys=True)
    log(f"wrote {out_md} and {jpath}")


def load_counters(kernel_name, grid):
    """MFMA-busy fraction etc. of one MMQ launch from the committed counter
    summary, if it was taken on the current kernel source."""
    p = os.path.join(ROOT, "profiles", "mmq_counters.json")
    if not os.path.exists(p):
        return None
    try:
        ent = json.load(open(p)).get(f"{kernel_name}|{grid}")
    except Exception:
        return None
    if not ent or ent.get("source_hash") != gemm_source_hash():
        return None
    return ent


EXPERT_FETCH_MD = "moe_expert_fetch_q4_0_t2048_h2048_e128k8_i768.md"
EXPERT_FETCH_REPS = 3


def write_expert_fetch(fetch_csv, cmdline):
    """Summary of the --expert-fetch run under rocprofv3 --pmc FETCH_SIZE:
    bytes fetched by the grouped gate/up (SwiGLU) and down launches when all
    128 experts own rows and when only 8 do (same 16384 rows)."""
    import csv
    import statistics
    rows = [r for r in csv.DictReader(open(fetch_csv)) if r["Counter_Name"] == "FETCH_SIZE"]
    rows.sort(key=lambda r: int(r["Dispatch_Id"]))
    copy = [float(r["Counter_Value"]) for r in rows if "copy" in r["Kernel_Name"].lower()
            and float(r["Counter_Value"]) * 1024 > 0.5 * COPY_BYTES]
    if not copy:
        raise SystemExit(f"no reference copy of {COPY_BYTES} bytes found in {fetch_csv}")
    scale = statistics.median(copy) * 1024 / COPY_BYTES
    mmq = [r for r in rows if "gemm_kernel" in r["Kernel_Name"] or "skinny" in r["Kernel_Name"]
           or "wide" in r["Kernel_Name"]]
    # dispatch order: per case, EXPERT_FETCH_REPS x (gate/up launch, down launch)
    want = 2 * 2 * EXPERT_FETCH_REPS
    if len(mmq) != want:
        raise SystemExit(f"expected {want} MMQ dispatches, found {len(mmq)}")
    res = {}
    for ci, case in enumerate(("all 128 experts active", "8 experts active")):
        part = mmq[ci * 2 * EXPERT_FETCH_REPS:(ci + 1) * 2 * EXPERT_FETCH_REPS]
        for li, launch in enumerate(("gate/up + SwiGLU", "down")):
            vals = [float(r["Counter_Value"]) * 1024 / scale for r in part[li::2]]
            res[(case, launch)] = (statistics.median(vals), part[li]["Kernel_Name"])
    bs = 18  # Q4_0 block bytes
    wbytes = {"gate/up + SwiGLU": 2 * 768 * (2048 // 32) * bs, "down": 2048 * (768 // 32) * bs}
    path = os.path.join(ROOT, "profiles", EXPERT_FETCH_MD)
    with open(path, "w") as fh:
        fh.write("# Idle experts' blocks are not fetched: grouped MMQ launches of the Q4_0 MoE layer\n\n")
        fh.write("T 2048, H 2048, I 768, 128 experts, top-8: 16384 routed rows in both cases.  Case A: every "
                 "expert owns 128 rows.  Case B: experts 0, 16, ..., 112 own 2048 rows each, the other 120 "
                 "experts none.  The weights, activations and rows are the same; only the offsets differ.\n\n")
        fh.write("Counter pass (repo root on the GPU box, TMPDIR=/tmp, run from /tmp):\n\n")
        fh.write("    rocprofv3 --pmc FETCH_SIZE --output-format csv -d <repo>/gpurun_out/pmc_experts -o run -- "
                 "python3 <repo>/bench.py --expert-fetch\n\n")
        fh.write(f"Summary written by: `{cmdline}`\n\n")
        fh.write(f"FETCH_SIZE (KiB per dispatch) scaled by a {COPY_BYTES >> 20} MiB device copy in the same "
                 f"process (factor {scale:.4f}); median of {EXPERT_FETCH_REPS} dispatches.\n\n")
        fh.write("| case | launch | kernel | fetched MB | weight bytes of the active experts (MB) |\n"
                 "|---|---|---|---|---|\n")
        for (case, launch), (v, kname) in res.items():
            nact = 128 if case.startswith("all") else 8
            fh.write(f"| {case} | {launch} | `{kname}` | {v / 1e6:.1f} | {nact * wbytes[launch] / 1e6:.1f} |\n")
        for launch in ("gate/up + SwiGLU", "down"):
            a = res[("all 128 experts active", launch)][0]
            b = res[("8 experts active", launch)][0]
            fh.write(f"\n- {launch}: case B fetches {b / 1e6:.1f} MB in all, less than the "
                     f"{128 * wbytes[launch] / 1e6:.1f} MB that the blocks of all 128 experts occupy, so the "
                     f"blocks of its 120 idle experts ({120 * wbytes[launch] / 1e6:.1f} MB) are not fetched; "
                     f"case A fetches {(a - b) / 1e6:.1f} MB more than case B (not exactly the idle weights: the "
                     f"activation reads differ too, each expert of case B gathering every token).")
        fh.write("\n")
    log(open(path).read())


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-moe", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--all", action="store_true", help="(default) time every workload")
    ap.add_argument("--quick", action="store_true",
                    help="only the headline linear step and the Q4_0 MoE layer")
    ap.add_argument("--sweep", action="store_true", help="small-token sweep (part of the default run)")
    ap.add_argument("--repeats", type=int, default=5, help="timing repeats (median reported)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--eager", action="store_true", help="no HIP-graph replay (counter runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="first run a %d MiB device copy (counter scale reference)" % (COPY_BYTES >> 20))
    ap.add_argument("--kernel-summary", nargs=3, metavar=("CSV_DIR", "OUT_MD", "TITLE"),
                    help="write a kernel-time summary from a rocprofv3 --kernel-trace --stats "
                         "--output-format csv run (files run_kernel_stats.csv, run_kernel_trace.csv)")
    ap.add_argument("--counters-from", nargs=5, metavar=("SQ_CSV", "FETCH_CSV", "WRITE_CSV", "OUT_MD", "TITLE"),
                    help="write a per-kernel counter summary from three rocprofv3 --pmc runs and exit")
    ap.add_argument("--expert-fetch", action="store_true",
                    help="run the grouped Q4_0 MoE launches with all / 8 experts active and exit "
                         "(for a rocprofv3 --pmc FETCH_SIZE pass)")
    ap.add_argument("--expert-fetch-from", metavar="FETCH_CSV",
                    help="write the idle-expert fetch summary from that counter pass and exit")
    ap.add_argument("--traffic-from", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "RUN_ARGS"),
                    help="write profiles/mmq_traffic.json from two rocprofv3 counter CSVs and exit")
    args = ap.parse_args()
    if not args.quick:
        args.all = True
    if args.traffic_from:
        write_traffic(*args.traffic_from, shlex.join(sys.argv))
        return
    if args.expert_fetch_from:
        write_expert_fetch(args.expert_fetch_from, shlex.join(sys.argv))
        return
    if args.counters_from:
        write_counters(*args.counters_from, shlex.join(sys.argv))
        return
    if args.kernel_summary:
        write_kernel_summary(*args.kernel_summary)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path: each GPU would run these kernels on its share of the "
              "tokens with the adapter gradients all-reduced, which is not built)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import quantized_base_lora_amd as gq
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def f32(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(dev)

    def u8(a):
        return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).to(dev)

    def ev():
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        return e

    lib = gq.lib()
    if args.copy_probe:
        src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if args.expert_fetch:
        if not args.copy_probe:
            src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
            torch.empty_like(src).copy_(src)
            del src
        mc = synth.MOE_Q4_0_T2048
        minp = synth.make_moe(mc)
        E, H, I, s = mc.E, mc.H, mc.I, float(minp["scale"])
        mk = lambda w, a, b, no, ni: gq.Proj(mc.qtype, no, ni, u8(w), f32(a), f32(b), s, E)
        gate, up = mk(minp["wg"], minp["ag"], minp["bg"], I, H), mk(minp["wu"], minp["au"], minp["bu"], I, H)
        down = mk(minp["wd"], minp["ad"], minp["bd"], H, I)
        x = bf(minp["x"])
        M = mc.T * mc.k
        gather = torch.arange(M, dtype=torch.int32, device=dev) % mc.T * mc.k  # token t's rows, k-major
        for case, counts in (("all", np.full(E, M // E)),
                             ("eight", np.where(np.arange(E) % 16 == 0, M // 8, 0))):
            offs = torch.from_numpy(np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)).to(dev)
            log(f"[bench] expert fetch: case {case}, active experts {int((counts > 0).sum())}")
            for _ in range(EXPERT_FETCH_REPS):
                h, _, _, _ = gq.grouped_mmq_lora_fwd([gate, up], gq.EPI_SWIGLU, x, gather, mc.k, offs, M)
                gq.grouped_mmq_lora_fwd([down], gq.EPI_NONE, h, None, 1, offs, M)
            torch.cuda.synchronize()
        log("[bench] expert fetch: done")
        return

    spreads = {}

    def time_steps(fn, steps, warmup, graph_too=True, key=None):
        """(eager ms, graph ms) per step: `steps` calls issued from Python
        (the median of `--repeats` such runs; their spread is kept under
        `key`), then the same step captured once in a HIP graph and replayed
        `steps` times (no host launch work between kernels; every kernel
        still runs)."""
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a, b = ev(), torch.cuda.Event(enable_timing=True)
        runs = []
        for _ in range(max(1, args.repeats)):
            a.record()
            for _ in range(steps):
                fn()
            b.record()
            torch.cuda.synchronize()
            runs.append(a.elapsed_time(b) / steps)
        eager = float(np.median(runs))
        if key:
            spreads[key] = {"repeats": len(runs), "median_ms": round(eager, 4),
                            "min_ms": round(min(runs), 4), "max_ms": round(max(runs), 4)}
        if args.eager or not graph_too:
            return eager, eager
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            fn()
        graph.replay()
        torch.cuda.synchronize()
        a.record()
        for _ in range(steps):
            graph.replay()
        b.record()
        torch.cuda.synchronize()
        replayed = a.elapsed_time(b) / steps
        del graph
        return eager, replayed

    def batched_ms(fn, n, reps=5):
        """ms per call of fn: n calls captured in one HIP graph, replayed."""
        fn()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a, b = ev(), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / (reps * n)

    # The Q4_0 MoE layer and then the headline linear step are timed after the
    # other workloads, with their inputs made up front: the timed work before
    # them brings the GPU to its sustained clocks (a kernel trace of this run
    # shows the dX MMQ going from 82 to 69.5 us per launch over the first
    # ~30 ms of sustained work), so their W warm-up steps and K timed steps
    # run at the clocks a training loop runs at, not at the ramp.  Every
    # workload keeps its own W untimed warm-up steps.
    K = args.steps
    result = {}

    # inputs of the headline linear step, resident in HBM from here on (made
    # before the other workloads so that no host work idles the GPU between
    # them and its timed steps)
    cfg = synth.LINEAR_Q4_0_T2048
    t0 = time.time()
    inp = synth.make_linear(cfg)
    log(f"[bench] inputs {cfg.name} generated in {time.time() - t0:.1f}s")
    p = gq.Proj(cfg.qtype, cfg.N, cfg.K, u8(inp["blocks"]), f32(inp["A"]), f32(inp["B"]),
                float(inp["scale"]))
    x, dy = bf(inp["x"]), bf(inp["dy"])
    ws = torch.empty(lib.gq_linear_lora_bwd_workspace_size(gq.C.byref(p.c()), cfg.T),
                     dtype=torch.uint8, device=dev)

    # inputs of the Q4_0 MoE layer, resident from here on (timed below, after
    # the other workloads, like the headline step)
    if not args.no_moe:
        mc = synth.MOE_Q4_0_T2048
        t0 = time.time()
        minp = synth.make_moe(mc)
        log(f"[bench] inputs {mc.name} generated in {time.time() - t0:.1f}s")
        E, H, I, s = mc.E, mc.H, mc.I, float(minp["scale"])
        mk = lambda w, a, b, no, ni: gq.Proj(mc.qtype, no, ni, u8(w), f32(a), f32(b), s, E)
        wts = gq.MoEWeights(mk(minp["wg"], minp["ag"], minp["bg"], I, H),
                            mk(minp["wu"], minp["au"], minp["bu"], I, H),
                            mk(minp["wd"], minp["ad"], minp["bd"], H, I))
        mx, mdy, mlg = bf(minp["x"]), bf(minp["dy"]), f32(minp["logits"])
        del minp

    # ------------------------------------------------------- other workloads
    if args.all:
        extra = {}

        def timed(fn, steps, key):
            return time_steps(fn, steps, 2, key=key)[0]

        c1 = synth.LINEAR_Q8_0_T128
        i1 = synth.make_linear(c1)
        p1 = gq.Proj(c1.qtype, c1.N, c1.K, u8(i1["blocks"]), f32(i1["A"]), f32(i1["B"]),
                     float(i1["scale"]))
        x1, dy1 = bf(i1["x"]), bf(i1["dy"])

        def s1():
            yy, xa1 = gq.linear_lora_fwd(p1, x1)
            return gq.linear_lora_bwd(p1, x1, xa1, dy1)

        m1, m1g = time_steps(s1, K, 2, key=c1.name)
        f1 = linear_flops(c1.T, c1.K, c1.N, c1.rank)
        # algorithmic bytes: W blocks once per pass (fwd, bwd), x, dY read,
        # y, dX written, adapters read, adapter gradients written
        b1 = (2 * i1["blocks"].nbytes + 2 * 2 * c1.T * (c1.K + c1.N) +
              2 * 4 * c1.rank * (c1.K + c1.N))
        extra[c1.name] = {"ms_per_step": round(m1, 4), "ms_per_step_hip_graph": round(m1g, 4),
                          "tflops": round(f1 / (m1 * 1e-3) / 1e12, 2),
                          "algorithmic_bytes": int(b1),
                          "frac_hbm": round(b1 / (m1 * 1e-3) / 1e9 / PEAK_HBM_GBS, 5),
                          "frac_bf16_peak": round(f1 / (m1 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 5),
                          "bound": "hbm; in practice launch latency (7 dependent launches)",
                          "launches": 7}
        log(f"[bench] {c1.name}: {m1 * 1e3:.1f} us/step ({m1g * 1e3:.1f} us replayed from a HIP graph)")

        c4 = synth.MOE_Q2DM_T4096_ZIPF
        t0 = time.time()
        i4 = synth.make_moe(c4)
        log(f"[bench] inputs {c4.name} generated in {time.time() - t0:.1f}s")
        s4 = float(i4["scale"])
        mk4 = lambda w, a, b, no, ni: gq.Proj(c4.qtype, no, ni, u8(w), f32(a), f32(b), s4, c4.E)
        w4 = gq.MoEWeights(mk4(i4["wg"], i4["ag"], i4["bg"], c4.I, c4.H),
                           mk4(i4["wu"], i4["au"], i4["bu"], c4.I, c4.H),
                           mk4(i4["wd"], i4["ad"], i4["bd"], c4.H, c4.I))
        x4, dy4, lg4 = bf(i4["x"]), bf(i4["dy"]), f32(i4["logits"])
        del i4

        def st4():
            yy, sv = gq.moe_ffn_fwd(w4, x4, lg4, c4.k)
            return gq.moe_ffn_bwd(w4, x4, dy4, sv, c4.k, c4.E)

        m4 = timed(st4, max(3, K // 4), c4.name)
        f4 = moe_flops(c4.T, c4.H, c4.I, c4.k, c4.rank)
        cnt4 = np.diff(gq.moe_route(lg4, c4.k)[3].cpu().numpy().astype(np.int64))
        act4 = cnt4[cnt4 > 0]
        extra[c4.name] = {"ms_per_step": round(m4, 4), "tokens_per_s": round(c4.T / (m4 * 1e-3), 1),
                          "tflops": round(f4 / (m4 * 1e-3) / 1e12, 2),
                          "frac_bf16_peak": round(f4 / (m4 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                          "route_rows_per_expert": {"active_experts": int(act4.size),
                                                    "max_rows": int(cnt4.max()),
                                                    "median_rows": float(np.median(cnt4)),
                                                    "min_active_rows": int(act4.min())}}
        log(f"[bench] {c4.name}: {m4:.3f} ms/step")
        del w4, x4, dy4, lg4

        c5 = synth.LMHEAD_Q8_0_T2048
        t0 = time.time()
        i5 = synth.make_head(c5)
        log(f"[bench] inputs {c5.name} generated in {time.time() - t0:.1f}s")
        hd = gq.Proj(c5.qtype, c5.V, c5.H, u8(i5["blocks"]), f32(i5["A"]), f32(i5["B"]),
                     float(i5["scale"]))
        h5 = bf(i5["h"])
        lab5 = torch.from_numpy(i5["labels"]).to(dev)
        ws5 = [None]

        def st5():
            out = gq.lmhead_chunked_ce(hd, h5, lab5, chunk_rows=c5.chunk, ws=ws5[0])
            ws5[0] = out["ws"]
            return out

        m5 = timed(st5, max(3, K // 4), c5.name)
        f5 = 6 * c5.T * c5.V * c5.H + 8 * c5.T * c5.V * c5.rank + 6 * c5.T * c5.rank * c5.H
        extra[c5.name] = {"ms_per_step": round(m5, 4), "tokens_per_s": round(c5.T / (m5 * 1e-3), 1),
                          "tflops": round(f5 / (m5 * 1e-3) / 1e12, 2),
                          "frac_bf16_peak": round(f5 / (m5 * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
        log(f"[bench] {c5.name}: {m5:.3f} ms/step")
        result["other_workloads"] = extra

        # RMS normalisation ahead of the linear layers (hidden 2048 and 4096,
        # 2048 tokens): HBM-bound, against the HBM roofline; the fp64 oracle
        # on the same inputs beside it (host cores)
        rng = np.random.default_rng(0)
        norm = []
        for Tn, Hn in ((2048, 2048), (2048, 4096)):
            xnb = synth.f32_to_bf16_bits(rng.standard_normal((Tn, Hn)).astype(np.float32))
            dynb = synth.f32_to_bf16_bits(rng.standard_normal((Tn, Hn)).astype(np.float32))
            wn_h = rng.uniform(0.5, 1.5, Hn).astype(np.float32)
            xn, dyn, wn = bf(xnb), bf(dynb), f32(wn_h)
            # launches of a few us: 50 launches captured in one HIP graph and
            # the graph replayed, so neither host launch work nor the graph
            # launch hides the kernels
            fms = batched_ms(lambda: gq.rmsnorm_fwd(xn, wn), 50)
            _, rs = gq.rmsnorm_fwd(xn, wn)
            bms = batched_ms(lambda: gq.rmsnorm_bwd(dyn, xn, wn, rs), 50)
            fbytes = 2 * Tn * Hn * 2 + Hn * 4 + Tn * 4
            bbytes = 3 * Tn * Hn * 2 + Hn * 4 + Tn * 4
            ent = {"workload": f"rmsnorm_t{Tn}_h{Hn}", "fwd_us": round(fms * 1e3, 2),
                   "bwd_us": round(bms * 1e3, 2),
                   "fwd_GB_per_s": round(fbytes / (fms * 1e-3) / 1e9, 1),
                   "bwd_GB_per_s": round(bbytes / (bms * 1e-3) / 1e9, 1),
                   "fwd_frac_hbm": round(fbytes / (fms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                   "bwd_frac_hbm": round(bbytes / (bms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
            if not args.no_cpu:
                from oracle import rmsnorm as orms
                xo = synth.bf16_bits_to_f32(xnb).astype(np.float64)
                dyo = synth.bf16_bits_to_f32(dynb).astype(np.float64)
                reps, spent = 0, 0.0
                while spent < 1.0:
                    t0 = time.perf_counter()
                    orms.forward(xo, wn_h, 1e-6)
                    orms.backward(xo, wn_h, dyo, 1e-6)
                    spent += time.perf_counter() - t0
                    reps += 1
                ent["cpu_baseline_fwd_bwd_ms"] = round(1e3 * spent / reps, 2)
            norm.append(ent)
            log(f"[bench] rmsnorm T {Tn} H {Hn}: fwd {fms * 1e3:.1f} us ({ent['fwd_GB_per_s']:.0f} GB/s), "
                f"bwd {bms * 1e3:.1f} us ({ent['bwd_GB_per_s']:.0f} GB/s)")
        result["rmsnorm"] = norm

        # 8-bit AdamW step over the adapters of the Q4_0 MoE layer (gate, up,
        # down of 128 experts, rank 4: 4.3 M parameters), against HBM
        # bandwidth: p read and written, g read, both code arrays read and
        # written, scales
        mc = synth.MOE_Q4_0_T2048
        na = mc.E * (2 * (mc.rank * mc.H + mc.I * mc.rank) + mc.rank * mc.I + mc.H * mc.rank)
        pa = torch.from_numpy(rng.standard_normal(na).astype(np.float32)).to(dev)
        ga = torch.from_numpy((1e-3 * rng.standard_normal(na)).astype(np.float32)).to(dev)
        sta = gq.AdamW8bitState(na, pa.device)
        for _ in range(3):
            gq.adamw8bit_step(pa, ga, sta, 1e-4)
        ams = batched_ms(lambda: gq.adamw8bit_step(pa, ga, sta, 1e-4), 20)
        abytes = na * (4 + 4 + 4 + 1 + 1 + 1 + 1) + 4 * 4 * ((na + 255) // 256)
        ent = {"workload": f"adamw8bit_moe_adapters_{na}", "params": na, "us": round(ams * 1e3, 2),
               "GB_per_s": round(abytes / (ams * 1e-3) / 1e9, 1),
               "frac_hbm": round(abytes / (ams * 1e-3) / 1e9 / PEAK_HBM_GBS, 4)}
        if not args.no_cpu:
            from oracle import adamw8bit as oa
            ph = pa.cpu().numpy()
            gh = ga.cpu().numpy()
            z8 = np.zeros(na, np.uint8)
            zs = np.zeros((na + 255) // 256, np.float32)
            t0 = time.perf_counter()
            oa.step(ph, gh, z8, z8, zs, zs, 1, 1e-4, 0.9, 0.999, 1e-8, 0.0)
            ent["cpu_baseline_ms"] = round(1e3 * (time.perf_counter() - t0), 1)
        result["adamw8bit"] = ent
        log(f"[bench] adamw8bit {na} params: {ams * 1e3:.1f} us ({ent['GB_per_s']:.0f} GB/s)")

    # ------------------------------------------------- small-token sweep
    if args.sweep or args.all:
        sweep = []
        sc = synth.MOE_Q4_0_T2048
        t0 = time.time()
        winp = synth.make_moe(sc)  # expert weights are per-expert streams: shared by every T
        log(f"[bench] sweep weights {sc.name} generated in {time.time() - t0:.1f}s")
        mk = lambda w, a, b, no, ni: gq.Proj(sc.qtype, no, ni, u8(w), f32(a), f32(b),
                                             float(winp["scale"]), sc.E)
        swts = gq.MoEWeights(mk(winp["wg"], winp["ag"], winp["bg"], sc.I, sc.H),
                             mk(winp["wu"], winp["au"], winp["bu"], sc.I, sc.H),
                             mk(winp["wd"], winp["ad"], winp["bd"], sc.H, sc.I))
        del winp
        bs = {0: 34, 1: 18, 2: 12}[sc.qtype]
        for T in (16, 64, 128, 256, 512):
            tc = synth.MoECfg(f"moe_q4_0_t{T}_h2048_e128k8_i768_r4", T=T, H=sc.H, I=sc.I, E=sc.E,
                              k=sc.k, qtype=sc.qtype, rank=sc.rank, alpha=sc.alpha, seed=sc.seed)
            tinp = synth.make_moe(tc, experts=[])  # token draws only
            tx, tdy, tlg = bf(tinp["x"]), bf(tinp["dy"]), f32(tinp["logits"])

            def tstep():
                yy, sv = gq.moe_ffn_fwd(swts, tx, tlg, tc.k)
                return gq.moe_ffn_bwd(swts, tx, tdy, sv, tc.k, tc.E)

            tms_e, tms_g = time_steps(tstep, max(10, K), 3, key=tc.name)
            # small steps are host-launch bound when issued from Python: the
            # HIP-graph replay (every kernel still runs) gives the GPU rate
            tms = min(tms_e, tms_g)
            _, sv = gq.moe_ffn_fwd(swts, tx, tlg, tc.k)
            active = int((sv["offsets"][1:] - sv["offsets"][:-1] > 0).sum().item())
            nbytes = moe_layer_bytes(T, sc.H, sc.I, sc.E, sc.k, sc.rank, bs, active)
            gbs = nbytes / (tms * 1e-3) / 1e9
            sweep.append({"workload": tc.name, "op": "moe layer fwd+bwd", "ms": round(tms, 4),
                          "ms_eager": round(tms_e, 4), "ms_hip_graph": round(tms_g, 4),
                          "active_experts": active, "algorithmic_bytes": nbytes,
                          "GB_per_s": round(gbs, 1), "frac_hbm": round(gbs / PEAK_HBM_GBS, 4),
                          "tokens_per_s": round(T / (tms * 1e-3), 1)})
            log(f"[bench] sweep {tc.name}: {tms:.3f} ms (eager {tms_e:.3f}, graph {tms_g:.3f}), {active} experts, "
                f"{gbs:.0f} GB/s ({100 * gbs / PEAK_HBM_GBS:.1f}% HBM)")
        del swts
        hc = synth.LMHEAD_Q8_0_T2048
        for T in (16, 64, 128):
            cfgT = synth.HeadCfg(f"lmhead_fwd_q8_0_t{T}_h2048_v151936_r4", T=T, H=hc.H, V=hc.V,
                                 qtype=hc.qtype, rank=hc.rank, alpha=hc.alpha, chunk=hc.chunk,
                                 seed=hc.seed)
            hinp = synth.make_head(cfgT)
            hd = gq.Proj(cfgT.qtype, cfgT.V, cfgT.H, u8(hinp["blocks"]), f32(hinp["A"]),
                         f32(hinp["B"]), float(hinp["scale"]))
            hh = bf(hinp["h"])
            hl = torch.from_numpy(hinp["labels"]).to(dev)
            del hinp
            hws = [None]

            def hstep():
                out = gq.lmhead_chunked_ce(hd, hh, hl, chunk_rows=cfgT.chunk, want_grad=False, ws=hws[0])
                hws[0] = out["ws"]
                return out

            hms_e, hms_g = time_steps(hstep, max(10, K), 3, key=cfgT.name)
            hms = min(hms_e, hms_g)
            nbytes = cfgT.V * (cfgT.H // 32) * 34 + T * cfgT.H * 2 + cfgT.V * cfgT.rank * 4 + cfgT.rank * cfgT.H * 4
            gbs = nbytes / (hms * 1e-3) / 1e9
            sweep.append({"workload": cfgT.name, "op": "LM head forward (loss, lse)", "ms": round(hms, 4),
                          "ms_eager": round(hms_e, 4), "ms_hip_graph": round(hms_g, 4),
                          "algorithmic_bytes": nbytes, "GB_per_s": round(gbs, 1),
                          "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)})
            log(f"[bench] sweep {cfgT.name}: {hms:.3f} ms (eager {hms_e:.3f}, graph {hms_g:.3f}), {gbs:.0f} GB/s "
                f"({100 * gbs / PEAK_HBM_GBS:.1f}% HBM)")
            del hd
        result["small_token_sweep"] = sweep

    # --------------------------------------------------------------- MoE layer
    if not args.no_moe:
        def mstep():
            yy, saved = gq.moe_ffn_fwd(wts, mx, mlg, mc.k)
            return gq.moe_ffn_bwd(wts, mx, mdy, saved, mc.k, E)

        mms, mms_graph = time_steps(mstep, K, max(2, args.warmup), key=mc.name)
        mfl = moe_flops(mc.T, H, I, mc.k, mc.rank)
        # rows routed to each expert (one routing call outside the timed steps)
        counts = np.diff(gq.moe_route(mlg, mc.k)[3].cpu().numpy().astype(np.int64))
        act = counts[counts > 0]
        route_hist = {"active_experts": int(act.size), "max_rows": int(counts.max()),
                      "median_rows": float(np.median(counts)), "min_active_rows": int(act.min())}
        result["moe_layer"] = {"workload": mc.name, "tokens_per_s": round(mc.T / (mms * 1e-3), 1),
                               "ms_per_step": round(mms, 4), "ms_per_step_hip_graph": round(mms_graph, 4),
                               "tflops": round(mfl / (mms * 1e-3) / 1e12, 2),
                               "frac_bf16_peak": round(mfl / (mms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                               "route_rows_per_expert": route_hist}
        log(f"[bench] moe layer {mms:.3f} ms/step, {mc.T / (mms * 1e-3):.0f} tok/s")

    # ------------------------------------------------------------ linear step (timed below)
    def step(prof=None):
        if prof:
            lib.gq_profile_mmq_events(prof[0].cuda_event, prof[1].cuda_event)
        y, xa = gq.linear_lora_fwd(p, x)
        if prof:
            lib.gq_profile_mmq_events(prof[2].cuda_event, prof[3].cuda_event)
        out = gq.linear_lora_bwd(p, x, xa, dy, ws=ws)
        if prof:
            lib.gq_profile_mmq_events(None, None)
        return y, out

    # timed steps: nothing but the step itself on the stream
    ms, ms_graph = time_steps(step, K, args.warmup, key=cfg.name)
    # a second pass of K steps with events on the two MMQ launches (stamped
    # by the kernel dispatch itself on the stream they are launched on)
    # gives the per-launch durations, outside the timed steps
    prof = [[ev() for _ in range(4)] for _ in range(K)]
    torch.cuda.synchronize()
    for i in range(K):
        step(prof[i])
    torch.cuda.synchronize()
    fwd_ms = sum(pp[0].elapsed_time(pp[1]) for pp in prof) / K
    bwd_ms = sum(pp[2].elapsed_time(pp[3]) for pp in prof) / K
    flops = linear_flops(cfg.T, cfg.K, cfg.N, cfg.rank)
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"[bench] linear step {ms:.3f} ms ({tflops:.1f} TFLOP/s), {ms_graph:.3f} ms replayed from a "
        f"HIP graph; MMQ fwd {fwd_ms*1e3:.1f} us, MMQ dX {bwd_ms*1e3:.1f} us")

    # dominant kernel: the slower of the two MMQ launches of the step
    gemm_flops = 2 * cfg.T * cfg.N * cfg.K + 2 * cfg.T * cfg.N * cfg.rank
    if bwd_ms >= fwd_ms:
        kname, kms, kkey = "mmq_nn_dx_q4_0_t2048_2048x6144", bwd_ms, "mmq_nn_lin_bwd_q4_0_t2048_2048x6144"
    else:
        kname, kms, kkey = "mmq_nt_fwd_q4_0_t2048_2048x6144", fwd_ms, "mmq_nt_lin_q4_0_t2048_2048x6144"
    achieved = gemm_flops / (kms * 1e-3) / 1e12
    roofline = {"kernel": kname, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic(kkey), "launch_us": round(kms * 1e3, 2),
                "other_mmq_us": round((fwd_ms if kms == bwd_ms else bwd_ms) * 1e3, 2),
                "algorithmic_flops_per_launch": gemm_flops}
    # MFMA-busy fraction of the same launch from the committed counter summary
    frag, grid = {k: (f, g) for f, g, k in MMQ_LAUNCHES}[kkey]
    cnt = load_counters(frag, grid)
    roofline["mfma_busy_counter"] = round(cnt["mfma_busy"], 4) if cnt else None

    # cold operands: the same step rotating over copies of W, x and dY that
    # together exceed the 256 MB Infinity Cache, so every step streams its
    # operands from HBM (the timed numbers above have them cache-resident)
    set_bytes = inp["blocks"].nbytes + 2 * cfg.T * (cfg.K + cfg.N)
    ncopy = max(2, -(-(512 << 20) // set_bytes))
    copies = [(gq.Proj(cfg.qtype, cfg.N, cfg.K, p.blocks.clone(), p.A, p.B, float(inp["scale"])),
               x.clone(), dy.clone()) for _ in range(ncopy)]
    rot = [0]

    def cold_step():
        pc, xc, dyc = copies[rot[0] % ncopy]
        rot[0] += 1
        yc, xac = gq.linear_lora_fwd(pc, xc)
        return gq.linear_lora_bwd(pc, xc, xac, dyc, ws=ws)

    ms_cold = time_steps(cold_step, max(K, 2 * ncopy), ncopy, graph_too=False, key=cfg.name + "_cold")[0]
    del copies
    log(f"[bench] linear step, cold operands ({ncopy} copies, {ncopy * set_bytes / 1e6:.0f} MB): "
        f"{ms_cold:.3f} ms ({flops / (ms_cold * 1e-3) / 1e12:.1f} TFLOP/s)")

    head = {
        "metric": "fused dequant-GEMM+LoRA fwd+bwd TFLOP/s & MoE-layer train tokens/s, % roofline",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_hip_graph": round(ms_graph, 4),
        "ms_per_step_cold_operands": round(ms_cold, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "tokens": cfg.T, "n_in": cfg.K, "n_out": cfg.N,
                   "qtype": "q4_0", "rank": cfg.rank, "alpha": cfg.alpha, "seed": cfg.seed,
                   "parallelism": "single-gpu"},
        "roofline": roofline,
    }
    result = {**head, **result}  # headline fields first

    # ------------------------------------------------------------ CPU oracle
    if not args.no_cpu:
        from threadpoolctl import threadpool_info, threadpool_limits

        from oracle import linear as ol

        # every host core this process may run on, set explicitly for the BLAS
        ncpu = os.cpu_count() or 1
        try:
            n_affinity = len(os.sched_getaffinity(0))
        except AttributeError:
            n_affinity = ncpu
        want = max(1, min(n_affinity, int(os.environ.get("OMP_NUM_THREADS", n_affinity))))
        cpu_model = "unknown"
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
        reps, spent = 0, 0.0
        ref = None
        with threadpool_limits(limits=want, user_api="blas"):
            blas = [i for i in threadpool_info() if i.get("user_api") == "blas"]
            threads = max([i.get("num_threads", 1) for i in blas] or [1])
            while spent < args.cpu_seconds and reps < 500:
                t0 = time.perf_counter()
                ref = ol.run(inp)
                spent += time.perf_counter() - t0
                reps += 1
        # parity of the timed step against the oracle on the same inputs
        # (relative Frobenius error per output)
        yg, (dxg, dAg, dBg) = step()
        torch.cuda.synchronize()

        def rel(got, key):
            g = got.float().cpu().numpy().astype(np.float64)
            r = np.asarray(ref[key], np.float64)
            return float(np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300))

        result["parity_rel_frobenius"] = {k: f"{rel(t, k):.2e}" for k, t in
                                          (("y", yg), ("dx", dxg), ("dA", dAg), ("dB", dBg))}
        blas_desc = ", ".join(f"{b.get('internal_api')} {b.get('version')} ({b.get('threading_layer')})"
                              for b in blas) or "none found"
        result["cpu_baseline"] = {"value": round(flops * reps / spent / 1e12, 5), "unit": "TFLOP/s",
                                  "cores": threads, "kind": "oracle",
                                  "sample": f"{reps} full fwd+bwd passes of {cfg.name} in fp64 numpy, "
                                            f"{spent:.1f}s",
                                  "os_cpu_count": ncpu, "affinity_cpus": n_affinity,
                                  "cpu_model": cpu_model, "blas": blas_desc,
                                  "blas_threads_set": want,
                                  "tokens_per_s": round(cfg.T * reps / spent, 1),
                                  "gflops_fp64": round(flops * reps / spent / 1e9, 1)}
        log(f"[bench] cpu oracle {reps} reps in {spent:.1f}s on {threads} BLAS threads "
            f"({cpu_model}, os.cpu_count {ncpu}, affinity {n_affinity}, {blas_desc})")

    result["timing_spread"] = spreads

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
