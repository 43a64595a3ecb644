"""Summaries of rocprofv3 kernel traces for the profiles/ notes.

``python -m weight_streaming_gemv_amd.profsum decode <run_kernel_trace.csv>``
    per-kernel median durations of a decode run and the per-token sum;
``python -m weight_streaming_gemv_amd.profsum instances <run_kernel_trace.csv>``
    the same per template instance (row count, weight storage and launch
    shape are template arguments), with workgroups per launch;
``python -m weight_streaming_gemv_amd.profsum sweep <run_kernel_trace.csv>``
    kernel-only GB/s of every cold-sweep configuration (bench.py --sweep-only),
    matched to its launch by kernel template arguments and grid size;
``python -m weight_streaming_gemv_amd.profsum phases <run_kernel_trace.csv> <kernel> <run> <phases>``
    the dispatches of one kernel (name containing <kernel>) in start order,
    dispatch i counted in phase (i // run) % phases: median duration per phase
    (e.g. the prefill attention of each chunk: 27 launches per chunk, 4 chunks);
``python -m weight_streaming_gemv_amd.profsum counters <run_counter_collection.csv>``
    per template instance and grid size (threads): dispatches, then the median
    per dispatch and the total over all dispatches of every collected counter
    (a ``rocprofv3 --pmc`` run).

Durations are the trace's begin/end timestamps (device time of each dispatch,
no launch gaps).
"""
from __future__ import annotations

import csv
import re
import statistics
import sys
from collections import defaultdict

HBM_PEAK_GBPS = 8000.0


def load(path):
    groups = defaultdict(list)
    with open(path) as f:
        for r in csv.DictReader(f):
            d = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
            blocks = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            groups[(r["Kernel_Name"], blocks, int(r["Grid_Size_Y"]))].append(d)
    return groups


def short(name):
    m = re.match(r"(?:void )?(?:wsg::)?(?:\(anonymous namespace\)::)?([\w:]+)(<[^(]*>)?", name)
    return (m.group(1) + (m.group(2) or "")) if m else name[:60]


def decode_table(path):
    g = load(path)
    by_name = defaultdict(list)
    for (name, blocks, gy), ds in g.items():
        by_name[short(name).split("<")[0]].extend(ds)
    rows = sorted(((sum(ds), n, ds) for n, ds in by_name.items()), reverse=True)
    print("| kernel | calls | median us | mean us | total ms | share |")
    print("|---|---|---|---|---|---|")
    tot = sum(r[0] for r in rows)
    for s, n, ds in rows:
        print(f"| {n} | {len(ds)} | {statistics.median(ds) / 1e3:.2f} | {statistics.fmean(ds) / 1e3:.2f} | "
              f"{s / 1e6:.2f} | {100 * s / tot:.1f}% |")


def instance_table(path):
    g = load(path)
    by_inst = defaultdict(list)
    for (name, blocks, gy), ds in g.items():
        by_inst[(short(name), blocks * gy)].extend(ds)
    rows = sorted(((sum(ds), k, ds) for k, ds in by_inst.items()), reverse=True)
    print("| kernel instance | workgroups | calls | median us | mean us | total ms |")
    print("|---|---|---|---|---|---|")
    for s, (n, wg), ds in rows:
        print(f"| `{n}` | {wg} | {len(ds)} | {statistics.median(ds) / 1e3:.2f} | "
              f"{statistics.fmean(ds) / 1e3:.2f} | {s / 1e6:.2f} |")


def phase_table(path, kernel, run, phases):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if kernel in r["Kernel_Name"]:
                rows.append((int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    by = defaultdict(list)
    for i, (_, d) in enumerate(rows):
        by[(i // run) % phases].append(d)
    print(f"| phase | dispatches | median us | mean us |")
    print("|---|---|---|---|")
    for ph in range(phases):
        ds = by[ph]
        if ds:
            print(f"| {ph} | {len(ds)} | {statistics.median(ds) / 1e3:.2f} | {statistics.fmean(ds) / 1e3:.2f} |")


def counter_table(path):
    vals = defaultdict(lambda: defaultdict(list))
    names = []
    with open(path) as f:
        for r in csv.DictReader(f):
            c = r["Counter_Name"]
            if c not in names:
                names.append(c)
            vals[(short(r["Kernel_Name"]), int(r["Grid_Size"]))][c].append(float(r["Counter_Value"]))
    rows = sorted(vals.items(), key=lambda kv: -sum(kv[1][names[0]]))
    print("| kernel instance | grid | dispatches | " + " | ".join(f"{c} median | {c} total" for c in names) + " |")
    print("|---|---|---|" + "---|---|" * len(names))
    for (n, grid), cs in rows:
        cells = " | ".join(f"{statistics.median(cs[c]):.6g} | {sum(cs[c]):.6g}" if cs[c] else "- | -"
                           for c in names)
        print(f"| `{n}` | {grid} | {len(cs[names[0]])} | {cells} |")


def _ceil(a, b):
    return -(-a // b)


def sweep_table(path):
    from synth import GEMV_SHAPES, Q4_SHAPES
    g = load(path)
    idx = defaultdict(list)
    for (name, blocks, gy), ds in g.items():
        idx[(short(name), blocks)].extend(ds)
    print("| kernel | M x K | T | R | NT | blocks | calls | median us | GB/s | % of 8 TB/s |")
    print("|---|---|---|---|---|---|---|---|---|---|")
    best = {}
    # A (kernel instance, grid) pair that two shapes both launch pools their
    # dispatches in the trace: it is shown for the first shape only (whose
    # dispatches dominate it) and left out for the later ones.
    owner = {}
    pooled = []
    for dt, es, kname in (("f32", 4, "k_gemv_f32"), ("f16", 2, "k_gemv_f16"), ("q4g64", None, "k_gemv_q4")):
        shapes = Q4_SHAPES if dt == "q4g64" else GEMV_SHAPES
        for (M, K) in shapes:
            nbytes = M * K // 2 + M * (K // 64) * 2 if dt == "q4g64" else M * K * es
            for T in (1, 2):
                # "1s": one FP32 row over two waves (k_gemv_f32_split2, one workgroup per row pair)
                split_ok = dt == "f32" and K in (1024, 2048, 3072)
                for R in (1, 2, 4, 8) + (("1s",) if split_ok else ()):
                    for nt in ("false", "true"):   # ordinary / non-temporal weight loads
                        seen = set()
                        grids = (0, 256, 512) if dt == "q4g64" else ((0, 1280, 2048, 4096) if M > 100000 else (0,))
                        # int4 rows of 14336 run 16-wave workgroups, every other shape 4-wave ones
                        wv = ({1: 16, 2: 8}.get(R, 4)) if dt == "q4g64" and K == 14336 else 4
                        for G in grids:
                            one = _ceil(M, 2) if R == "1s" else _ceil(_ceil(M, R), wv)
                            blocks = one if G == 0 or G >= one else G
                            if blocks in seen:
                                continue
                            seen.add(blocks)
                            if R == "1s":
                                key = (f"k_gemv_f32_split2<{K}, {T}, {nt}>", blocks)
                            else:
                                tmpl = f"{K}, {R}, {T}, {nt}, {wv}" if dt == "q4g64" else f"{K}, {R}, {T}, {nt}"
                                key = (f"{kname}<{tmpl}>", blocks)
                            ds = idx.get(key)
                            if not ds:
                                continue
                            if owner.setdefault(key, (M, K)) != (M, K):
                                pooled.append(f"{key[0]} on {key[1]} blocks: {M}x{K} pooled with "
                                              f"{owner[key][0]}x{owner[key][1]}")
                                continue
                            us = statistics.median(ds) / 1e3
                            gbps = nbytes / us / 1e3
                            print(f"| {kname} | {M}x{K} | {T} | {R} | {'y' if nt == 'true' else 'n'} | {blocks} | "
                                  f"{len(ds)} | {us:.2f} | {gbps:.0f} | {100 * gbps / HBM_PEAK_GBPS:.1f} |")
                            k = (dt, M, K, T)
                            if k not in best or us < best[k][0]:
                                best[k] = (us, R, blocks, gbps)
    if pooled:
        print()
        print("Left out (launches of the same kernel instance and grid by two shapes; the row above "
              "belongs to the first): " + "; ".join(pooled) + ".")
    print()
    print("Best per shape (kernel-only):")
    print()
    print("| dtype | M x K | T | R | blocks | median us | GB/s | % of peak |")
    print("|---|---|---|---|---|---|---|---|")
    for (dt, M, K, T), (us, R, b, gbps) in sorted(best.items()):
        print(f"| {dt} | {M}x{K} | {T} | {R} | {b} | {us:.2f} | {gbps:.0f} | {100 * gbps / HBM_PEAK_GBPS:.1f} |")
    for dt, es in (("f32", 4), ("f16", 2)):
        names = [(4096, 1024), (1024, 2048), (6144, 1024), (1024, 3072), (151936, 1024)]
        if all((dt, M, K, 1) in best for M, K in names):
            w = [28, 28, 28, 28, 1]
            b = sum(wi * M * K * es for wi, (M, K) in zip(w, names))
            t = sum(wi * best[(dt, M, K, 1)][0] for wi, (M, K) in zip(w, names))
            print(f"\nDecode-mix aggregate {dt} (28 x [QKV, O, gate/up, down] + vocab, T=1, best R): "
                  f"{b / t / 1e3:.0f} GB/s = {100 * b / t / 1e3 / HBM_PEAK_GBPS:.1f}% of 8 TB/s")


if __name__ == "__main__":
    import os
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    mode, path = sys.argv[1], sys.argv[2]
    if mode == "phases":
        phase_table(path, sys.argv[3], int(sys.argv[4]), int(sys.argv[5]))
    else:
        {"decode": decode_table, "instances": instance_table, "sweep": sweep_table,
         "counters": counter_table}[mode](path)
