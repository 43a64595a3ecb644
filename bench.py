#!/usr/bin/env python3
"""Decode benchmark on one MI355X: 28-layer FP32 Qwen3-0.6B-shaped decoder.

One step = the four short greedy generations of the pages' GPU-wide study
(prompt/output 8/8, 8/16, 32/8, 32/16; Megakernels, "GPU-wide end-to-end
generation"), each timed from before the cache reset to the last token id
on the host.  The decode steps of a generation go through ``wsg_generate``
(enqueued back to back, one wait at the end: the token is chosen on the GPU
and the history stays there); the same generations with one waiting
``wsg_step`` per token are reported as ``step_loop``.  ``value`` is the
post-first-token decode rate: generated
tokens after the first, divided by the time after the first token
(Benchmark methodology, "What the measurements mean" and "Long-document
chunked prefill").  Timings are published only after the GPU's greedy
tokens, logits and KV matched the CPU oracle on the same inputs; every timed
generation must reproduce the validated token ids.

Also reported: every decode stage against the HBM roofline, the one with
the largest share of per-token stage time as ``roofline`` (its time per
launch inside the step: the step's layer graph with and without the stage,
replayed between HIP events after the timed region), the whole step's weight
bytes per token times tokens/s
(``step_roofline``), the head timed with HIP events in the step-loop pass
after the timed region, the oracle timed
on the host cores, provenance (hashes, versions, device, launch shapes), and
(``--sweep``) the cold-cache GEMV sweep.  A validation failure anywhere
publishes nothing (exit status 3).
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
COMBOS = [(8, 8), (8, 16), (32, 8), (32, 16)]
STAGES = {"qkv": 0, "attn": 1, "o": 2, "gateup": 3, "down": 4, "head": 5}
# Kernel of each stage kind at the short-prompt contexts (attention fused with the output
# projection up to 128 keys).
STAGE_KERNEL = {"qkv": "k_qkv", "attn": "k_attn_o", "o": "k_gemv_residual", "gateup": "k_gateup",
                "down": "k_gemv_residual", "head": "k_head"}


# HBM bytes per launch of decode kernels from rocprofv3 FETCH_SIZE and WRITE_SIZE
# runs, each scaled by what the same counter reads for a plain copy of known size
# (FETCH x 2.0, WRITE x 1.0); valid only for the decode kernel sources they were
# measured on (their hash below), else reported as null.
DECODE_TRAFFIC = {"sha256_16": "247485dc258d7d4a",
                  "bytes": {"k_gateup": 25_539_434, "k_attn_o": 9_014_883, "k_qkv": 16_915_703,
                            "k_gemv_residual": 12_763_573, "k_head": 623_631_400}}


def decode_source_hash():
    """sha256 (16 hex digits) of the decode kernels' sources and their default launch shapes
    (decode.hip, common.hpp, decode.hpp and the shape defaults in model.hip)."""
    import hashlib
    import re
    csrc = os.path.join(ROOT, "weight_streaming_gemv_amd", "csrc")
    try:
        parts = [open(os.path.join(csrc, f)).read() for f in ("decode.hip", "common.hpp", "decode.hpp")]
        mod = open(os.path.join(csrc, "model.hip")).read()
    except OSError:
        return None
    m = re.search(r"  DecodeShape& sh = m->shape;.*?\n  std::vector<float> cs, sn;", mod, re.S)
    if not m:
        return None
    return hashlib.sha256(("".join(parts) + m.group(0)).encode()).hexdigest()[:16]


def recorded_traffic(kernel):
    """Recorded HBM bytes per launch of `kernel`, or None if the sources changed since."""
    h = decode_source_hash()
    if h is None or h != DECODE_TRAFFIC["sha256_16"]:
        return None
    return DECODE_TRAFFIC["bytes"].get(kernel)


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_threads():
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return max(n)
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def generate(model, prompt, n_out, pipelined=True):
    """One timed greedy generation: (tokens, ttft_s, decode_s, total_s).  Pipelined: the
    decode steps through ``wsg_generate`` (enqueued back to back, one wait); else one
    ``wsg_step`` per token, each waiting for its token."""
    t0 = time.perf_counter()
    model.reset()
    toks = [model.prefill(prompt)]
    t1 = time.perf_counter()
    if pipelined:
        toks += model.generate(n_out - 1)
    else:
        for _ in range(n_out - 1):
            toks.append(model.step())
    t2 = time.perf_counter()
    return toks, t1 - t0, t2 - t1, t2 - t0


class ValidationError(RuntimeError):
    """The GPU disagreed with the oracle: every timing of the run is discarded."""


def check_close(got, ref, what, tol=1e-3):
    """|got - ref| <= tol + tol |ref| elementwise in float64 (ref = the oracle's values);
    a NaN or Inf fails.  ``got`` is a torch tensor (any device), ``ref`` array-like.
    Returns the largest absolute error."""
    g = got.float().cpu().numpy().astype(np.float64)
    r = np.asarray(ref, dtype=np.float64)
    err = np.abs(g - r)
    if not np.all(err <= tol + tol * np.abs(r)):   # NaN compares false
        raise ValidationError(f"validation failed: {what} off by {np.nanmax(err) if err.size else 0:.3e}")
    return float(err.max()) if err.size else 0.0


def check_close_big(got, ref, what, tol=1e-3):
    """check_close for large cache prefixes: the oracle's values are copied to the
    tensor's device and compared there, in float64, with the same inequality."""
    import torch
    r = torch.from_numpy(np.ascontiguousarray(ref)).to(got.device).double()
    err = (got.double() - r).abs()
    ok = bool((err <= tol + tol * r.abs()).all())
    if not ok:
        raise ValidationError(f"validation failed: {what} off by {float(torch.nan_to_num(err, nan=float('inf')).max()):.3e}")
    return float(err.max()) if err.numel() else 0.0


def check_prefix(model, orc, n, what, big=False):
    """Every valid K/V entry [0, n) of every layer against the oracle; returns the largest error."""
    mk = 0.0
    cmp = check_close_big if big else check_close
    for l in range(orc.shape.n_layers):
        k, v, _ = model.kv(l)
        mk = max(mk, cmp(k[:, :n], orc.k_cache[l][:, :n], f"{what} K layer {l}"))
        mk = max(mk, cmp(v[:, :n], orc.v_cache[l][:, :n], f"{what} V layer {l}"))
    return mk


def check_slot(model, orc, p, what):
    """The K/V slot p of every layer (one copy per layer and tensor) against the oracle."""
    mk = 0.0
    for l in range(orc.shape.n_layers):
        k, v, _ = model.kv(l)
        mk = max(mk, check_close(k[:, p:p + 1], orc.k_cache[l][:, p:p + 1], f"K layer {l} {what}"))
        mk = max(mk, check_close(v[:, p:p + 1], orc.v_cache[l][:, p:p + 1], f"V layer {l} {what}"))
    return mk


def validate(model, orc, prompt, n_out):
    """Lockstep check of logits, tokens and KV; returns (tokens, max errors, oracle decode seconds)."""
    import oracle
    model.reset()
    orc.reset()
    tok = model.prefill(prompt)
    ref = orc.forward_rows(prompt)
    toks, rtoks = [tok], [oracle.argmax_lowest(ref)]
    max_l = max_kv = 0.0
    t_dec = 0.0
    cmp = check_close

    max_l = max(max_l, cmp(model.logits(), ref, "logits at the first output"))
    for s in range(1, n_out):
        if toks[-1] != rtoks[-1]:
            raise ValidationError(f"validation failed: token {toks[-1]} != oracle {rtoks[-1]} "
                                  f"(oracle margin {orc.logits_margin(ref):.3e})")
        p = orc.pos
        toks.append(model.step())
        t = time.perf_counter()
        ref = orc.forward_rows([rtoks[-1]])
        t_dec += time.perf_counter() - t
        rtoks.append(oracle.argmax_lowest(ref))
        max_l = max(max_l, cmp(model.logits(), ref, f"logits at step {s}"))
        for l in range(orc.shape.n_layers):
            k, v, _ = model.kv(l)
            max_kv = max(max_kv, cmp(k[:, p:p + 1], orc.k_cache[l][:, p:p + 1], f"K layer {l} step {s}"))
            max_kv = max(max_kv, cmp(v[:, p:p + 1], orc.v_cache[l][:, p:p + 1], f"V layer {l} step {s}"))
    if toks != rtoks:
        raise ValidationError(f"validation failed: tokens {toks} != oracle {rtoks}")
    n = orc.pos
    for l in range(orc.shape.n_layers):
        k, v, _ = model.kv(l)
        max_kv = max(max_kv, cmp(k[:, :n], orc.k_cache[l][:, :n], f"K prefix layer {l}"))
        max_kv = max(max_kv, cmp(v[:, :n], orc.v_cache[l][:, :n], f"V prefix layer {l}"))
    return toks, max_l, max_kv, t_dec


def gemv_sweep(rounds=15, kind="full"):
    """Cold-cache GEMV sweep: each shape cycles >= 1 GiB of distinct matrices.

    Our Kernel Benchmark Was Measuring the System Cache ("The fix"): one reused
    matrix sits in the system cache, so the working set must exceed it (here
    the 256 MiB Infinity Cache; every cycle reads >= 1 GiB).  The launches of
    one cycle are captured into a graph and replayed; per-dispatch time =
    cycle time / copies (dispatch-inclusive), median over rounds; rows per
    wave interleaved within each round (A/B/A, "Two neighboring traps").
    Effective GB/s = weight bytes / that time (Benchmark methodology, "What the
    measurements mean").  A warm figure (one matrix reused) is given for T=1.
    ``kind``: "full" (every shape), "quick" (the first FP32/FP16 shape), "int4" (the int4
    shapes only, e.g. for counter runs).
    """
    import torch
    import weight_streaming_gemv_amd as wsg
    from synth import GEMV_SHAPES, Q4_SHAPES

    GiB = 1 << 30
    # blocks: 0 = one row group per wave; capped grids only where they cannot
    # coincide with another configuration's launch (the kernel trace tells
    # configurations apart by kernel name and grid size)
    GRIDS = (0, 1280, 2048, 4096)
    # weights are streamed with non-temporal loads, as in the decode path
    # (a read-only stream runs ~9 % faster that way on this part)
    NT = wsg.WSG_GEMV_NONTEMPORAL
    s = torch.cuda.Stream()
    gen = torch.Generator(device="cuda")
    gen.manual_seed(100)
    out = {}

    sink = torch.empty(1, dtype=torch.float32, device="cuda")

    def ceiling_read(buf):
        # read-only streaming reference over the same copies (16-byte non-temporal loads)
        return lambda: wsg.stream_read(buf, out=sink, stream=s)

    def time_graph(fn_list):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for fn in fn_list:
                fn()
        return g

    def run(label, bytes_per, n, make_launch, Rs, Ts, grids=(0,)):
        res = {}
        graphs = {}
        for T in Ts:
            for R in Rs:
                for G in grids:
                    graphs[(T, R, G)] = time_graph([make_launch(c, T, R, G) for c in range(n)])
        times = {k: [] for k in graphs}
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(s):          # replay() runs on the current stream
            for g in graphs.values():
                g.replay()                   # warm-up: one full cycle each
            torch.cuda.synchronize()
            for _ in range(rounds):
                for k, g in graphs.items():
                    e0.record(s)
                    g.replay()
                    e1.record(s)
                    e1.synchronize()
                    times[k].append(e0.elapsed_time(e1) * 1e3 / n)
        for (T, R, G), t in times.items():
            us = statistics.median(t)
            res[f"T{T}_R{R}_G{G}"] = {"us": round(us, 3), "gbps": round(bytes_per / us / 1e3, 1)}
        del graphs
        return res

    shapes = {"full": GEMV_SHAPES, "quick": GEMV_SHAPES[:1], "int4": []}[kind]
    for dt_name, tdt, es in (("f32", torch.float32, 4), ("f16", torch.float16, 2)):
        for (M, K) in shapes:
            bytes_per = M * K * es
            n = -(-GiB // bytes_per)
            W = (torch.randn((n, M, K), device="cuda", generator=gen, dtype=torch.float32) * 0.02).to(tdt)
            X = torch.randn((2, K), device="cuda", generator=gen, dtype=torch.float32).to(tdt)
            Y = torch.empty((2, M), device="cuda", dtype=torch.float32)

            def make(c, T, R, G, W=W, X=X, Y=Y):
                if R == "1s":   # each row over two waves of a workgroup
                    return lambda: wsg.gemv(W[c], X[:T], rows_per_wave=1, Y=Y, stream=s, grid_blocks=G,
                                            flags=NT | wsg.WSG_GEMV_SPLIT2)
                return lambda: wsg.gemv(W[c], X[:T], rows_per_wave=R, Y=Y, stream=s, grid_blocks=G, flags=NT)
            log(f"sweep {dt_name} {M}x{K}: {n} copies")
            Rs = (1, 2, 4, 8) + (("1s",) if dt_name == "f32" and K in (1024, 2048, 3072) else ())
            r = run(f"{dt_name}", bytes_per, n, make, Rs, (1, 2), GRIDS if M > 100000 else (0,))
            # warm: one matrix, reused n times
            r["warm_T1"] = run("warm", bytes_per, n, lambda c, T, R, G: make(0, T, R, G), (1,), (1,))["T1_R1_G0"]
            r["ceiling"] = run("ceiling", bytes_per, n, lambda c, T, R, G: ceiling_read(W[c]), (1,), (1,))["T1_R1_G0"]
            out[f"{dt_name}_{M}x{K}"] = {"bytes": bytes_per, "copies": n, **r}
            del W, X, Y
            torch.cuda.empty_cache()
    for (M, K) in (Q4_SHAPES if kind in ("full", "int4") else []):
        bytes_per = M * K // 2 + M * (K // 64) * 2
        n = -(-GiB // bytes_per)
        Wq = torch.randint(-2 ** 31, 2 ** 31 - 1, (n, M, K // 8), device="cuda", generator=gen, dtype=torch.int32)
        S = (torch.randn((n, M, K // 64), device="cuda", generator=gen).abs() * 0.01).half()
        X = torch.randn((2, K), device="cuda", generator=gen).half()
        Y = torch.empty((2, M), device="cuda", dtype=torch.float32)

        def make(c, T, R, G, Wq=Wq, S=S, X=X, Y=Y):
            return lambda: wsg.gemv_q4g64(Wq[c], S[c], X[:T], rows_per_wave=R, Y=Y, stream=s, grid_blocks=G,
                                          flags=NT)
        log(f"sweep q4g64 {M}x{K}: {n} copies")
        r = run("q4", bytes_per, n, make, (1, 2, 4, 8), (1, 2), (0, 256, 512))
        r["warm_T1"] = run("warm", bytes_per, n, lambda c, T, R, G: make(0, T, R, G), (1,), (1,))["T1_R1_G0"]
        # the int4 ceiling reads the packed words (the scales add 1/32 of their bytes)
        r["ceiling"] = run("ceiling", M * K // 2, n, lambda c, T, R, G: ceiling_read(Wq[c]), (1,), (1,))["T1_R1_G0"]
        out[f"q4g64_{M}x{K}"] = {"bytes": bytes_per, "copies": n, **r}
        del Wq, S, X, Y
        torch.cuda.empty_cache()
    return out


def cpu_gemv_rates(copies=2):
    """The oracle's GEMVs on the host cores: one call on each of `copies` host-generated
    matrices (T=1), effective GB/s = weight bytes / median call time.  A bounded sample: the
    four per-layer shapes in FP32 and FP16 and the smallest int4 shape (the vocabulary and the
    two large int4 shapes would add minutes of CPU time at the same rates); one untimed call
    first pages in the BLAS library."""
    import oracle
    from synth import GEMV_SHAPES, Q4_SHAPES, gemv_inputs, q4g64_inputs
    W, X = gemv_inputs(256, 256, 1, seed=5)
    oracle.gemv(W, X)
    res = {}
    for dt_name, dt, es in (("f32", np.float32, 4), ("f16", np.float16, 2)):
        for (M, K) in GEMV_SHAPES[:4]:
            ts = []
            for c in range(copies):
                W, X = gemv_inputs(M, K, 1, seed=5, copy=c, dtype=dt)
                t = time.perf_counter()
                oracle.gemv(W, X)
                ts.append(time.perf_counter() - t)
            res[f"{dt_name}_{M}x{K}"] = round(M * K * es / statistics.median(ts) / 1e9, 3)
    M, K = Q4_SHAPES[0]
    ts = []
    for c in range(copies):
        _, words, scales, X = q4g64_inputs(M, K, 1, seed=5, copy=c)
        t = time.perf_counter()
        oracle.gemv_q4g64(words, scales, X, K)
        ts.append(time.perf_counter() - t)
    res[f"q4g64_{M}x{K}"] = round((M * K // 2 + M * (K // 64) * 2) / statistics.median(ts) / 1e9, 4)
    return {"gbps": res, "cores": cpu_threads(), "kind": "oracle", "copies": copies,
            "sample": "per-layer shapes (FP32, FP16) and int4 4096x4096, T=1"}


def host_info():
    """The host cores the CPU figures ran on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"affinity_cpus": len(os.sched_getaffinity(0)), "cpu_count": os.cpu_count(), "cpu_model": model,
            "blas_threads": cpu_threads()}


def provenance(model=None):
    """What produced the figures (Benchmark methodology, "Long-document chunked prefill":
    reports keep hashes, versions and kernel fingerprints): source and library hashes, the
    git commit when a checkout is present, torch / HIP / ROCm versions, the device, and the
    model's launch shapes."""
    import hashlib
    import subprocess
    import torch

    def sha(paths):
        h = hashlib.sha256()
        for p in paths:
            try:
                with open(p, "rb") as f:
                    h.update(f.read())
            except OSError:
                h.update(b"<missing>")
        return h.hexdigest()[:16]

    csrc = os.path.join(ROOT, "weight_streaming_gemv_amd", "csrc")
    srcs = sorted(os.path.join(csrc, f) for f in os.listdir(csrc))
    srcs += [os.path.join(ROOT, "include", "wsg.h"), os.path.abspath(__file__)]
    srcs += sorted(os.path.join(ROOT, "oracle", f) for f in os.listdir(os.path.join(ROOT, "oracle"))
                   if f.endswith(".py"))
    git = None
    try:
        r = subprocess.run(["git", "-C", ROOT, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        git = r.stdout.strip() or None
    except Exception:
        pass
    rocm = None
    try:
        with open("/opt/rocm/.info/version") as f:
            rocm = f.read().strip()
    except OSError:
        pass
    props = torch.cuda.get_device_properties(0)
    dev = {"name": props.name, "arch": getattr(props, "gcnArchName", None),
           "compute_units": props.multi_processor_count, "memory_bytes": props.total_memory}
    for attr in ("clock_rate", "memory_clock_rate", "L2_cache_size"):
        if hasattr(props, attr):
            dev[attr] = getattr(props, attr)
    out = {"sources_sha256_16": sha(srcs), "decode_kernels_sha256_16": decode_source_hash(),
           "libwsg_sha256_16": sha([os.path.join(ROOT, "weight_streaming_gemv_amd", "libwsg.so")]),
           "git_head": git, "torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
           "rocm": rocm, "device": dev}
    if model is not None:
        out["launch_shapes"] = model.describe()
    return out


def sweep_summary(sw):
    """Best rows-per-wave per shape and the bytes-weighted decode-mix aggregate."""
    from synth import QWEN3_0_6B
    best = {}
    for key, r in sw.items():
        for T in (1, 2):
            cands = [(v["us"], k) for k, v in r.items() if k.startswith(f"T{T}_")]
            if cands:
                us, k = min(cands)
                rk = k.split("_R")[1].split("_")[0]   # "1s": one row per two waves (WSG_GEMV_SPLIT2)
                best[f"{key}_T{T}"] = {"R": int(rk.rstrip("s")), "waves_per_row": 2 if rk.endswith("s") else 1,
                                       "grid": int(k.split("_G")[1]), "us": us,
                                       "gbps": round(r["bytes"] / us / 1e3, 1),
                                       "frac": round(r["bytes"] / us / 1e3 / HBM_PEAK_GBPS, 4)}
                if "ceiling" in r:
                    best[f"{key}_T{T}"]["frac_of_stream_ceiling"] = round(r["bytes"] / us / 1e3 / r["ceiling"]["gbps"], 4)
    agg = {}
    for dt in ("f32", "f16"):
        names = ["4096x1024", "1024x2048", "6144x1024", "1024x3072", "151936x1024"]
        if all(f"{dt}_{n}_T1" in best for n in names):
            L = QWEN3_0_6B.n_layers
            w = [L, L, L, L, 1]
            b = sum(wi * sw[f"{dt}_{n}"]["bytes"] for wi, n in zip(w, names))
            t = sum(wi * best[f"{dt}_{n}_T1"]["us"] for wi, n in zip(w, names))
            agg[dt] = {"gbps": round(b / t / 1e3, 1), "frac": round(b / t / 1e3 / HBM_PEAK_GBPS, 4),
                       "us_per_token": round(t, 1)}
            if all("ceiling" in sw[f"{dt}_{n}"] for n in names):
                tc = sum(wi * sw[f"{dt}_{n}"]["ceiling"]["us"] for wi, n in zip(w, names))
                agg[dt]["stream_ceiling_gbps"] = round(b / tc / 1e3, 1)
                agg[dt]["frac_of_stream_ceiling"] = round(tc / t, 4)
    return best, agg


def fixed_context(torch, wsg, shape, w, contexts=(0, 16, 64), trials=9, reps=50):
    """Single-forward latency at fixed contexts (Megakernels, "Fixed-context methodology"):
    per context c, three autoregressive forwards (slots c, c+1, c+2) are checked against the
    oracle (full-vocabulary logits, every valid K/V entry, exact greedy tokens) before
    timing; a trial then repeats the forward of one token at slot c `reps` times (rewind to
    c, step, read the token id: the same token every time).  Median and minimum over trials
    of the time per forward, including the rewind's one-word device update and the 4-byte
    token read."""
    import oracle
    from synth import prompt_ids
    cap = max(contexts) + 4
    model = wsg.Model(shape, w, max_context=cap, prefill_chunk=64)
    orc = oracle.OracleModel(shape, w, cap)
    res, errs = {}, []
    for c in contexts:
        prefix = prompt_ids(50 + c, c + 1, shape.vocab)
        toks, ml, mkv, _ = validate(model, orc, prefix, 3)
        errs.append((ml, mkv))
        model.reset()
        tok = model.prefill(prefix)
        per = []
        for t in range(trials + 1):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                model.rewind(c)
                if model.step() != toks[0]:
                    raise ValidationError(f"fixed context {c}: repeated forward changed its token")
            if t > 0:                      # the first trial warms up
                per.append((time.perf_counter() - t0) / reps * 1e6)
        assert tok == toks[0]
        res[str(c)] = {"us_median": round(statistics.median(per), 2), "us_min": round(min(per), 2)}
    model.close()
    res["validation"] = {"max_abs_logit_err": max(e[0] for e in errs), "max_abs_kv_err": max(e[1] for e in errs),
                         "forwards_checked_per_context": 3}
    res["workload"] = (f"28-layer FP32; contexts {list(contexts)}; {trials} trials x {reps} repeats of one "
                       "token's forward at the fixed slot (graph replay + head + argmax + token read)")
    return res


def lossless_bf16(torch, wsg, shape, steps=5, warmup=2):
    """The short-prompt workload on BF16-representable FP32 weights (the synthetic weights
    rounded to BF16), decode weights packed losslessly (Megakernels, "Lossless decode-weight
    storage"): the packed model is validated against the oracle on the same weights, must
    give the unpacked model's tokens, and both are timed the same way."""
    import oracle
    from synth import PROMPT_SEEDS, model_weights_bf16, prompt_ids
    cap = 48
    w = model_weights_bf16(shape, seed=0)
    prompt32 = prompt_ids(PROMPT_SEEDS["short"], 32, shape.vocab)
    prompts = {8: prompt32[:8], 32: prompt32}
    packed = wsg.Model(shape, w, max_context=cap, prefill_chunk=32, lossless_pack=True)
    plain = wsg.Model(shape, w, max_context=cap, prefill_chunk=32)
    orc = oracle.OracleModel(shape, w, cap)
    expected, errs = {}, []
    for n_p in (8, 32):
        toks, ml, mkv, _ = validate(packed, orc, prompts[n_p], 16)
        errs.append((ml, mkv))
        for n_o in (8, 16):
            expected[(n_p, n_o)] = toks[:n_o]
    del orc, w
    res = {}
    for name, model in (("packed", packed), ("unpacked", plain)):
        rec = []
        for i in range(warmup + steps):
            for (n_p, n_o) in COMBOS:
                toks, ttft, dec, tot = generate(model, prompts[n_p], n_o)
                if toks != expected[(n_p, n_o)]:
                    raise ValidationError(f"lossless {name} {n_p}/{n_o}: tokens differ from the validated packed run")
                if i >= warmup:
                    rec.append((n_o, dec))
        st = model.storage()
        res[name] = {"decode_tok_s": round(sum(n - 1 for n, _ in rec) / sum(d for _, d in rec), 2),
                     "decode_weight_bytes": st["decode_weight_bytes"],
                     "packed_matrices": f"{st['packed_matrices']}/{st['decode_matrices']}"}
        model.close()
    res["speedup"] = round(res["packed"]["decode_tok_s"] / res["unpacked"]["decode_tok_s"], 3)
    res["validation"] = {"max_abs_logit_err": max(e[0] for e in errs), "max_abs_kv_err": max(e[1] for e in errs),
                         "unpacked_tokens_identical": True}
    res["workload"] = ("28-layer FP32 model with BF16-representable weights (seed-0 draws rounded to BF16); "
                       "prompt/output 8/8, 8/16, 32/8, 32/16; decode projections and the head read the "
                       "packed copies, prefill the FP32 matrices")
    return res


def two_token(torch, wsg, shape, w, context=16, trials=9, reps=50, n_prompt=32, n_out=33):
    """Two-token step (the verify pass of greedy speculative decoding; "Our Kernel Benchmark
    Was Measuring the System Cache", "Why it mattered, concretely"): each weight matrix is
    streamed once for the last token and a draft of the next.  Validated first against the
    oracle (both rows' full-vocabulary logits, exact greedy tokens, both new K/V slots of
    every layer, one accepted and one rejected draft per pair of steps); then (a) the
    latency of one two-token forward at a fixed slot beside one single-token forward
    (rewind, forward, token read, as in the fixed-context harness), with HIP events around
    the two-row head launch; (b) decode throughput of speculative generation with drafts
    taken from a previous greedy run (all accepted: the decoder-side ceiling of speculative
    decoding) and with every other draft corrupted, each checked to emit exactly the greedy
    stream."""
    import oracle
    from synth import prompt_ids
    cap = n_prompt + n_out + 4
    model = wsg.Model(shape, w, max_context=cap, prefill_chunk=32)
    orc = oracle.OracleModel(shape, w, cap)
    prompt = prompt_ids(60, n_prompt, shape.vocab)

    def cmp(got, ref_, what):
        g = got.float().cpu().numpy().astype(np.float64)
        r = np.asarray(ref_, dtype=np.float64)
        err = np.abs(g - r)
        if not np.all(err <= 1e-3 + 1e-3 * np.abs(r)):
            raise ValidationError(f"two-token validation failed: {what} off by {err.max():.3e}")
        return float(err.max())

    # ---- validation: 4 steps, drafts accepted / rejected alternately
    tok = model.prefill(prompt)
    ref = orc.forward_rows(prompt)
    if tok != oracle.argmax_lowest(ref):
        raise ValidationError("two-token validation failed: first token")
    last, max_l, max_kv = tok, 0.0, 0.0
    for s in range(4):
        p = orc.pos
        ref0 = orc.forward_rows([last])
        g0 = oracle.argmax_lowest(ref0)
        draft = g0 if s % 2 == 0 else (g0 + 1) % shape.vocab
        (t0, t1), n = model.step2(draft)
        ref1 = orc.forward_rows([draft])
        lg = model.logits()
        max_l = max(max_l, cmp(lg[0], ref0, f"row 0 logits step {s}"), cmp(lg[1], ref1, f"row 1 logits step {s}"))
        for l in range(shape.n_layers):
            k, v, _ = model.kv(l)
            max_kv = max(max_kv, cmp(k[:, p:p + 2], orc.k_cache[l][:, p:p + 2], f"K layer {l} step {s}"),
                         cmp(v[:, p:p + 2], orc.v_cache[l][:, p:p + 2], f"V layer {l} step {s}"))
        if t0 != g0 or (n == 2 and t1 != oracle.argmax_lowest(ref1)) or n != (2 if s % 2 == 0 else 1):
            raise ValidationError(f"two-token validation failed: tokens {t0},{t1} n={n} at step {s}")
        if n == 1:
            orc.pos = p + 1
        last = t1 if n == 2 else t0
        if model.position != orc.pos:
            raise ValidationError("two-token validation failed: position")
    del orc

    # ---- (a) fixed-slot latency: one two-token forward vs one single-token forward
    model.reset()
    model.prefill(prompt[:context])          # its output token sits at slot `context`
    nxt = model.step()                       # greedy token after slot `context`
    after = model.step()                     # greedy token after slot `context + 1`
    model.set_option(wsg._abi.WSG_OPT_TIMED_STAGE, STAGES["head"])
    res = {}
    for name in ("step", "step2"):
        per = []
        for t in range(trials + 1):
            model.stage_time()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(reps):
                model.rewind(context)
                if name == "step":
                    ok = model.step() == nxt
                else:
                    (a, b), n = model.step2(nxt)
                    ok = (a, b, n) == (nxt, after, 2)
                if not ok:
                    raise ValidationError(f"two-token fixed slot: repeated {name} changed its tokens")
            if t > 0:
                per.append((time.perf_counter() - t0) / reps * 1e6)
        ms, nl, by = model.stage_time()
        res[name] = {"us_median": round(statistics.median(per), 2), "us_min": round(min(per), 2),
                     "head_us": round(ms / max(nl, 1) * 1e3, 2),
                     "head_weight_gbps": round(by / max(nl, 1) / (ms / max(nl, 1) * 1e-3) / 1e9, 1)}
    model.set_option(wsg._abi.WSG_OPT_TIMED_STAGE, -1)
    res["step2_over_step"] = round(res["step2"]["us_median"] / res["step"]["us_median"], 3)
    res["tokens_per_s_at_slot"] = {"step": round(1e6 / res["step"]["us_median"], 1),
                                   "step2_both_emitted": round(2e6 / res["step2"]["us_median"], 1)}

    # ---- (b) speculative generation with drafts from a greedy run
    greedy, _, _, _ = generate(model, prompt, n_out)
    gen = {}
    for name, bad_every in (("all_accepted", 0), ("every_other_rejected", 2)):
        rates = []
        for t in range(trials + 1):
            model.reset()
            out = [model.prefill(prompt)]
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            k = 0
            while len(out) < n_out:
                d = greedy[len(out)]
                if bad_every and k % bad_every == 1:
                    d = (d + 1) % shape.vocab
                k += 1
                (a, b), n = model.step2(d)
                out += [a, b][:n]
            dt = time.perf_counter() - t0
            if out[:n_out] != greedy:
                raise ValidationError(f"speculative generation ({name}) differs from the greedy stream")
            if t > 0:
                rates.append((len(out) - 1) / dt)
        gen[name] = {"decode_tok_s": round(statistics.median(rates), 1), "two_token_steps": k}
    for name, pipelined in (("greedy_step_only", False), ("greedy_generate", True)):
        g_rates = []
        for t in range(trials + 1):
            toks, _, dec, _ = generate(model, prompt, n_out, pipelined)
            if toks != greedy:
                raise ValidationError(f"greedy generation ({name}) not repeatable")
            if t > 0:
                g_rates.append((n_out - 1) / dec)
        gen[name] = {"decode_tok_s": round(statistics.median(g_rates), 1)}
    model.close()
    res["speculative_generation"] = gen
    res["validation"] = {"max_abs_logit_err": max_l, "max_abs_kv_err": max_kv, "steps_checked": 4,
                         "drafts": "accepted, rejected, accepted, rejected"}
    res["workload"] = (f"28-layer FP32; fixed slot {context} ({trials} trials x {reps} repeats, rewind + forward "
                       f"+ token read); generation: {n_prompt}-id prompt, {n_out} outputs, drafts from the "
                       "greedy stream (every other one corrupted in the second run)")
    return res


def f16_storage_decoder(torch, wsg, shape, fmt, steps=5, warmup=2, n_check=8):
    """The short-prompt workload on a model of the same shape with 16-bit storage:
    ``fmt`` "int4": every decode matrix and the tied embedding int4 in groups of 64 with
    FP16 scales (the int4 GEMV workload's distributions: q uniform in [-8, 7], scales
    |N(0, 0.01)|; "Our Kernel Benchmark Was Measuring the System Cache", "Summary": 4-bit
    decode); "fp16": the FP32 model's weights rounded to FP16 (the FP16 storage
    configuration whose validation Megakernels, "GPU-wide end-to-end generation", reports).  FP16 activations, KV cache and logits, FP32
    accumulation.  Validated first against the oracle, which computes from the same stored
    values on the CPU: teacher-forced (both sides consume the oracle's tokens), every logit
    and new K/V slot within the FP16 tolerance rtol=atol=2e-2; the share of greedy tokens
    that agree is reported.  Prompt rows run through the decode forward, two per forward
    (chunked prefill needs FP32 storage).
    HIP events time the head launches."""
    import oracle
    from synth import PROMPT_SEEDS, model_weights, model_weights_q4, prompt_ids
    t = time.perf_counter()
    w = model_weights_q4(shape, seed=0) if fmt == "int4" else model_weights(shape, seed=0, dtype=np.float16)
    log(f"{fmt} weights generated in {time.perf_counter() - t:.1f} s")
    cap = 48
    model = wsg.Model(shape, w, max_context=cap, dtype=wsg.WSG_F16)
    orc = oracle.OracleModel(shape, w, cap)
    del w
    prompt32 = prompt_ids(PROMPT_SEEDS["short"], 32, shape.vocab)
    prompts = {8: prompt32[:8], 32: prompt32}
    tol = 2e-2

    def cmp(got, ref_, what):
        g = got.float().cpu().numpy().astype(np.float64)
        r = np.asarray(ref_, dtype=np.float64)
        err = np.abs(g - r)
        if not np.all(err <= tol + tol * np.abs(r)):
            raise ValidationError(f"{fmt} validation failed: {what} off by {err.max():.3e}")
        return float(err.max())

    max_l = max_kv = 0.0
    agree = total = 0
    tok = model.prefill(prompts[8])
    ref = orc.forward_rows(prompts[8])
    max_l = max(max_l, cmp(model.logits(), ref, "prefill logits"))
    for s in range(n_check):
        rtok = oracle.argmax_lowest(ref)
        agree += int(tok == rtok)
        total += 1
        p = orc.pos
        tok = model.step(rtok)
        ref = orc.forward_rows([rtok])
        max_l = max(max_l, cmp(model.logits(), ref, f"logits step {s}"))
        for l in range(shape.n_layers):
            k, v, _ = model.kv(l)
            max_kv = max(max_kv, cmp(k[:, p:p + 1], orc.k_cache[l][:, p:p + 1], f"K layer {l}"),
                         cmp(v[:, p:p + 1], orc.v_cache[l][:, p:p + 1], f"V layer {l}"))
    n = orc.pos
    for l in range(shape.n_layers):
        k, v, _ = model.kv(l)
        max_kv = max(max_kv, cmp(k[:, :n], orc.k_cache[l][:, :n], f"K prefix {l}"),
                     cmp(v[:, :n], orc.v_cache[l][:, :n], f"V prefix {l}"))
    del orc
    # timed generations (tokens must repeat exactly run to run), then one pass of
    # step-by-step generations with HIP events around the head
    expected, rec = {}, []
    for i in range(warmup + steps):
        for (n_p, n_o) in COMBOS:
            toks, ttft, dec, tot = generate(model, prompts[n_p], n_o)
            if expected.setdefault((n_p, n_o), toks) != toks:
                raise ValidationError(f"{fmt} generation {n_p}/{n_o} not repeatable")
            if i >= warmup:
                rec.append((n_p, n_o, ttft, dec))
    model.set_option(wsg._abi.WSG_OPT_TIMED_STAGE, STAGES["head"])
    model.stage_time()
    for (n_p, n_o) in COMBOS:
        if generate(model, prompts[n_p], n_o, pipelined=False)[0] != expected[(n_p, n_o)]:
            raise ValidationError(f"{fmt} step-by-step generation {n_p}/{n_o} differs")
    ms, nl, by = model.stage_time()
    model.set_option(wsg._abi.WSG_OPT_TIMED_STAGE, -1)
    st = model.storage()
    model.close()
    value = sum(n_o - 1 for _, n_o, _, _ in rec) / sum(r[3] for r in rec)
    head_us = ms / max(nl, 1) * 1e3
    return {"decode_tok_s": round(value, 2),
            "decode_weight_bytes": st["decode_weight_bytes"],
            "decode_weight_gbps": round(st["decode_weight_bytes"] * value / 1e9, 1),
            "ttft_ms_median": {str(n_p): round(statistics.median(r[2] for r in rec if r[0] == n_p) * 1e3, 3)
                               for n_p in (8, 32)},
            "head": {"us": round(head_us, 2), "bytes_per_launch": by // max(nl, 1),
                     "gbps": round(by / max(nl, 1) / (head_us * 1e-6) / 1e9, 1) if nl else None},
            "validation": {"max_abs_logit_err": max_l, "max_abs_kv_err": max_kv, "rtol": tol, "atol": tol,
                           "teacher_forced_steps": n_check, "greedy_token_agreement": f"{agree}/{total}"},
            "workload": ("28-layer Qwen3-0.6B-shaped decoder, " +
                         ("int4 group-64 weights with FP16 scales for every decode matrix and the tied embedding"
                          if fmt == "int4" else "FP16 weights (the FP32 draws rounded to nearest)") +
                         ", FP16 activations/KV/logits; prompt/output 8/8, 8/16, 32/8, 32/16, prompt rows two "
                         "per decode forward")}


def prefill_only(torch, wsg, shape, w, chunk=1024, trials=3):
    """The held-out 4096-id prompt's chunked prefill alone (the prefill half of the
    long-document workload, Benchmark methodology, "Long-document chunked prefill"),
    for counter runs: one warm-up and ``trials`` timed prefills, no decode.  The
    matrix work per prefill is the four projections' 2*rows*N*K flops per chunk
    plus the causal attention's score and value products."""
    from synth import PROMPT_SEEDS, prompt_ids
    held = prompt_ids(PROMPT_SEEDS["heldout"], 4096, shape.vocab)
    model = wsg.Model(shape, w, max_context=len(held) + 1, prefill_chunk=chunk)
    times = []
    for i in range(1 + trials):
        model.reset()
        torch.cuda.synchronize()
        t = time.perf_counter()
        model.prefill(held)
        torch.cuda.synchronize()
        if i:
            times.append(time.perf_counter() - t)
    H, I, D = shape.hidden, shape.intermediate, shape.head_dim
    M = (shape.n_q_heads + 2 * shape.n_kv_heads) * D
    n = len(held)
    proj = 2 * n * shape.n_layers * (M * H + H * shape.n_q_heads * D + 2 * I * H + H * I)
    attn = 2 * 2 * shape.n_layers * shape.n_q_heads * D * (n * (n + 1) // 2)
    model.close()
    return {"prompt": n, "chunk": chunk, "prefill_ms_median": round(statistics.median(times) * 1e3, 2),
            "projection_flop": proj, "attention_flop": attn}


def long_context(torch, wsg, shape, w, trials=5, warmup=2, tune_len=2048, held_len=4096, n_out=1024,
                 chunks=(128, 256, 512, 1024), prefix_every=64, make_model=None):
    """Long-document workload (Benchmark methodology, "Long-document chunked prefill").

    Chunk selection: a ``tune_len``-id prompt with 8 outputs at each candidate chunk size;
    every candidate is validated first (whole-prefix KV of every layer, first-output logits,
    greedy tokens against the oracle); 2 warm-ups and 5 timed trials each; the smallest
    median TTFT wins, ties to the smaller chunk.

    Held-out: a different ``held_len``-id prompt with ``n_out`` outputs at the chosen chunk,
    validated before it is timed: the prompt is prefilled one chunk per call, and after each
    chunk the whole K/V prefix of every layer is checked against the oracle (run chunk by
    chunk too); then every one of the ``n_out`` outputs is checked in lockstep (full
    logits, exact token, the new K/V slot of every layer), and the whole prefix again at
    every ``prefix_every``-th output and at the last.  Timed runs prefill the prompt in one
    call; each must reproduce every validated token, and the last one's whole cache (valid
    length ``held_len + n_out - 1``) is checked against the oracle once more.  Any failure
    raises ValidationError, which discards every timing of the run.

    ``make_model(cap, chunk)`` builds the model (default: the HIP library's).
    """
    import oracle
    from synth import PROMPT_SEEDS, prompt_ids
    cap = held_len + n_out
    tune = prompt_ids(PROMPT_SEEDS["tuning"], tune_len, shape.vocab)
    held = prompt_ids(PROMPT_SEEDS["heldout"], held_len, shape.vocab)
    assert not np.array_equal(tune[:min(tune_len, held_len)], held[:min(tune_len, held_len)])
    if make_model is None:
        def make_model(cap_, chunk_):
            return wsg.Model(shape, w, max_context=cap_, prefill_chunk=chunk_)
    model = make_model(cap, max(chunks))
    orc = oracle.OracleModel(shape, w, cap)

    # oracle reference for the tuning prompt (chunk-independent): 8 outputs
    t = time.perf_counter()
    orc.reset()
    ref_logits = [orc.forward_rows(tune)]
    ref_toks = [oracle.argmax_lowest(ref_logits[0])]
    for _ in range(7):
        ref_logits.append(orc.forward_rows([ref_toks[-1]]))
        ref_toks.append(oracle.argmax_lowest(ref_logits[-1]))
    log(f"long: oracle tuning reference in {time.perf_counter() - t:.1f} s")
    # orc now holds the KV of tune_len + 7 positions
    max_kv = max_logit = 0.0
    sweep = {}
    for chunk in chunks:
        # every candidate in lockstep: the prompt's K/V prefix, then each output's logits,
        # token and new K/V slot, and the whole prefix at the end
        model.set_prefill_chunk(chunk)
        model.reset()
        toks = [model.prefill(tune)]
        max_kv = max(max_kv, check_prefix(model, orc, tune_len, f"chunk {chunk} prompt", big=True))
        for i in range(8):
            if i:
                p = model.position
                toks.append(model.step())
                max_kv = max(max_kv, check_slot(model, orc, p, f"chunk {chunk} output {i + 1}"))
            max_logit = max(max_logit, check_close(model.logits(), ref_logits[i], f"chunk {chunk} logits at output {i + 1}"))
            if toks[-1] != ref_toks[i]:
                raise ValidationError(f"long-context validation failed: chunk {chunk} output {i + 1} token "
                                      f"{toks[-1]} != oracle {ref_toks[i]}")
        max_kv = max(max_kv, check_prefix(model, orc, tune_len + 7, f"chunk {chunk} prefix after 8 outputs", big=True))
        rec = []
        for i in range(warmup + trials):
            tk, ttft, dec, tot = generate(model, tune, 8)
            if tk != ref_toks:
                raise ValidationError(f"chunk {chunk}: timed tokens differ from the validated ones")
            if i >= warmup:
                rec.append((ttft, dec, tot))
        sweep[chunk] = {"ttft_ms": round(statistics.median(r[0] for r in rec) * 1e3, 2),
                        "total_ms": round(statistics.median(r[2] for r in rec) * 1e3, 2)}
        log(f"long: chunk {chunk}: {sweep[chunk]}")
    best = min(sweep, key=lambda c: (sweep[c]["ttft_ms"], c))

    del ref_logits
    # ---- held-out validation: chunk by chunk, then every output in lockstep
    model.set_prefill_chunk(best)
    model.reset()
    orc.reset()
    t = time.perf_counter()
    t_or_prefill = 0.0
    boundaries = []
    for r0 in range(0, held_len, best):
        part = held[r0:r0 + best]
        t0 = time.perf_counter()
        ref_logits = orc.forward_rows(part, want_logits=r0 + len(part) == held_len)
        t_or_prefill += time.perf_counter() - t0
        tok = model.prefill(part)
        n = r0 + len(part)
        if model.position != n:
            raise ValidationError(f"held-out prefill: position {model.position} after {n} rows")
        max_kv = max(max_kv, check_prefix(model, orc, n, f"held-out chunk boundary {n}", big=True))
        boundaries.append(n)
    max_logit = max(max_logit, check_close(model.logits(), ref_logits, "held-out first logits"))
    toks = [tok]
    rtok = oracle.argmax_lowest(ref_logits)
    if tok != rtok:
        raise ValidationError(f"held-out first token {tok} != oracle {rtok} "
                              f"(margin {orc.logits_margin(ref_logits):.3e})")
    log(f"long: held-out prefill validated at {len(boundaries)} chunk boundaries "
        f"(oracle {t_or_prefill:.1f} s)")
    t_or = 0.0
    prefix_checks = [held_len]
    for s_ in range(1, n_out):
        p = model.position
        toks.append(model.step())
        t0 = time.perf_counter()
        ref = orc.forward_rows([toks[-2]])
        t_or += time.perf_counter() - t0
        rtok = oracle.argmax_lowest(ref)
        max_logit = max(max_logit, check_close(model.logits(), ref, f"held-out logits at output {s_ + 1}"))
        max_kv = max(max_kv, check_slot(model, orc, p, f"held-out output {s_ + 1}"))
        if toks[-1] != rtok:
            raise ValidationError(f"held-out output {s_ + 1}: token {toks[-1]} != oracle {rtok} "
                                  f"(margin {orc.logits_margin(ref):.3e})")
        if (s_ + 1) % prefix_every == 0 or s_ == n_out - 1:
            n = model.position
            max_kv = max(max_kv, check_prefix(model, orc, n, f"held-out prefix at output {s_ + 1}", big=True))
            prefix_checks.append(n)
        if (s_ + 1) % 128 == 0:
            log(f"long: held-out output {s_ + 1}/{n_out} validated (oracle {t_or:.1f} s)")
    if model.position != held_len + n_out - 1:
        raise ValidationError(f"held-out valid length is {model.position}, not {held_len + n_out - 1}")
    log(f"long: held-out generation validated in {time.perf_counter() - t:.1f} s")

    # ---- timed: one prefill call per run, every token reproduced
    rec = []
    for i in range(warmup + trials):
        tk, ttft, dec, tot = generate(model, held, n_out)
        if tk != toks:
            raise ValidationError("held-out timed tokens differ from the validated sequence")
        if i >= warmup:
            rec.append((ttft, dec, tot))
    # the single-call prefill and its generation leave the validated cache
    max_kv = max(max_kv, check_prefix(model, orc, held_len + n_out - 1, "held-out timed run's cache", big=True))
    model.close()
    return {
        "workload": f"28-layer FP32; chunk selection on a {tune_len}-id prompt / 8 outputs, held-out "
                    f"{held_len}-id prompt / {n_out} outputs ({held_len + n_out - 1} valid KV entries at the end)",
        "chunk_sweep": sweep, "selected_chunk": best,
        "heldout_median": {"ttft_ms": round(statistics.median(r[0] for r in rec) * 1e3, 2),
                           "decode_tok_s": round(statistics.median((n_out - 1) / r[1] for r in rec), 1),
                           "total_s": round(statistics.median(r[2] for r in rec), 3)},
        "heldout_prefill_mfma": prefill_mfma(shape, held_len, statistics.median(r[0] for r in rec)),
        "validation": {"max_abs_logit_err": max_logit, "max_abs_kv_err": max_kv, "rtol": 1e-3, "atol": 1e-3,
                       "oracle_checked_outputs": n_out, "chunk_boundary_prefix_checks": boundaries,
                       "whole_prefix_checks": prefix_checks, "timed_runs_token_exact": True,
                       "timed_run_cache_checked": held_len + n_out - 1},
        "cpu_oracle_decode_tok_s_at_4k": round((n_out - 1) / t_or, 3) if t_or else None,
    }


def stage_pass(wsg, model, head, reps=20):
    """Per-stage HBM rooflines of the decode step.  Each per-layer stage is timed with
    ``wsg_time_stage``: the next step's layer body (one graph of all stages of all layers)
    and the same body without that stage are replayed alternately ``reps`` times, each
    replay between two HIP events on the model stream; the difference of the mean replay
    times over the layer count is the stage's time per launch inside the step.  (An event
    pair around one launch would add its own dispatch cost to kernels of 4-7 us, so the
    events bracket whole replays.)  The head comes from the timed region (``head``: HIP
    events around each of its launches, a single 90-us kernel).  Per stage: time per
    launch, algorithmic bytes per launch (weights; the attention launch's cached keys and
    values plus, fused, its output-projection weights), achieved GB/s, and the stage's
    share of the per-token time of all stages (n_layers launches per token for the layer
    stages, one for the head)."""
    L = model.shape.n_layers
    res = {}
    for name in ("qkv", "attn", "gateup", "down"):
        us, b = model.time_stage(STAGES[name], reps)
        res[name] = {"kernel": STAGE_KERNEL[name], "launches": reps * L,
                     "us_per_launch": round(us, 3), "bytes_per_launch": b, "gbps": round(b / (us * 1e-6) / 1e9, 1),
                     "ms_per_token": round(us * L / 1e3, 4)}
    if head:
        res["head"] = {"kernel": head["kernel"], "launches": head["launches_timed"],
                       "us_per_launch": head["avg_launch_us"], "bytes_per_launch": head["bytes_per_launch"],
                       "gbps": head["achieved"], "ms_per_token": round(head["avg_launch_us"] / 1e3, 4)}
    tot = sum(r["ms_per_token"] for r in res.values())
    for r in res.values():
        r["share"] = round(r["ms_per_token"] / tot, 4) if tot else None
        r["frac"] = round(r["gbps"] / HBM_PEAK_GBPS, 4)
    return res


def launch_floor(torch, launches, reps=20):
    """Cost per node of a chain of ``launches`` dependent one-element kernels (torch's
    in-place add) replayed as one HIP graph, median over ``reps`` replays between HIP
    events: the dispatch floor that each of the decode step's launches pays besides its own
    kernel time (completion, the cache write-back and invalidation between dependent
    launches, the next dispatch).  An upper bound: the add itself runs well under 1 us."""
    t = torch.zeros(1, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(3):
            t.add_(1.0)
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(launches):
            t.add_(1.0)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per_node = []
    for _ in range(reps):
        e0.record()
        g.replay()
        e1.record()
        e1.synchronize()
        per_node.append(e0.elapsed_time(e1) * 1e3 / launches)
    del g
    return statistics.median(per_node)


MFMA_FP32_PEAK_TFLOPS = 157.3   # MI355X dense FP32 matrix peak


def prefill_mfma(shape, n, ttft_s):
    """Effective FP32 matrix throughput of a timed prefill: chunked-prefill flops / TTFT (a
    lower bound: TTFT also holds the last row's decode forward and the head)."""
    f = prefill_flops(shape, n)
    tf = f / ttft_s / 1e12
    return {"flops": f, "tflops": round(tf, 1), "peak_tflops": MFMA_FP32_PEAK_TFLOPS,
            "frac": round(tf / MFMA_FP32_PEAK_TFLOPS, 3)}


def prefill_flops(shape, n):
    """FP32 flops of the chunked part of a prefill of n ids (rows 0..n-2; the last row runs
    the decode path): 2 per weight per row for the projections (the last layer runs only its
    QKV projection, its K/V being the only output with a consumer), and 4*head_dim per
    (query head, visible key) pair for QK^T and PV in the layers before the last."""
    rows = n - 1
    h, i, q, kv, nl = shape.hidden, shape.intermediate, shape.q_width, shape.kv_width, shape.n_layers
    per_layer = (q + 2 * kv) * h + h * q + 2 * i * h + h * i
    proj = 2 * rows * (per_layer * (nl - 1) + (q + 2 * kv) * h)
    pairs = rows * (rows + 1) // 2
    attn = 4 * shape.head_dim * shape.n_q_heads * pairs * (nl - 1)
    return proj + attn


def main(argv=None):
    """Run the benchmark; a validation failure discards every timing (exit 3, nothing on
    stdout: Benchmark methodology, "Long-document chunked prefill")."""
    try:
        return _main(argv)
    except ValidationError as e:
        log(f"{e}: no timing is published")
        return 3


def _main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--timed-stage", default="head", choices=sorted(STAGES),
                    help="stage kind bracketed by HIP events (graph mode: head only)")
    ap.add_argument("--no-graph", action="store_true", help="launch every kernel directly")
    ap.add_argument("--roofline-reps", type=int, default=20,
                    help="replays of each per-layer stage's graph for the stage rooflines (0: none)")
    ap.add_argument("--sweep", choices=["full", "quick", "int4", "none"], default="full",
                    help="cold-cache GEMV sweep after the decode timing")
    ap.add_argument("--sweep-only", action="store_true", help="run only the cold-cache GEMV sweep")
    ap.add_argument("--sweep-json", default=None, help="also write every sweep configuration's row to this file")
    ap.add_argument("--sweep-rounds", type=int, default=15, help="timed rounds per sweep configuration")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a 512 MiB device copy (reference for the HBM traffic counters)")
    ap.add_argument("--long", choices=["on", "off", "only"], default="on",
                    help="long-document workload (2048-id chunk selection, 4096 -> 1024 held-out)")
    ap.add_argument("--fixed", choices=["on", "off", "only"], default="on",
                    help="single-forward latency at contexts 0/16/64 (fixed cache slot)")
    ap.add_argument("--lossless", choices=["on", "off", "only"], default="on",
                    help="short-prompt workload on BF16-representable weights, packed vs unpacked decode")
    ap.add_argument("--two-token", choices=["on", "off", "only"], default="on",
                    help="two-token step (speculative verify pass): fixed-slot latency and generation")
    ap.add_argument("--int4", choices=["on", "off", "only"], default="on",
                    help="short-prompt workload on an int4 (group-64) model of the same shape")
    ap.add_argument("--fp16", choices=["on", "off", "only"], default="on",
                    help="short-prompt workload on the same model with FP16 storage")
    ap.add_argument("--prefill-only", action="store_true",
                    help="only the held-out 4096-id prompt's chunk-1024 prefill, 1 warm-up + 3 timed "
                         "(profiling runs: MFMA counters; no value is published)")
    ap.add_argument("--no-oracle", action="store_true",
                    help="skip validation and the CPU baseline (profiling runs only; no value is published)")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one MI355X: the library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        return 2

    import torch
    import weight_streaming_gemv_amd as wsg
    from synth import PROMPT_SEEDS, QWEN3_0_6B, model_weights, prompt_ids

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.copy_calibration:
        # a plain device copy of known size, for scaling the FETCH_SIZE /
        # WRITE_SIZE counters of the profiled kernels
        n = 1 << 27                                   # 128 Mi floats = 512 MiB each way
        src = torch.randn(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4}), flush=True)
        return 0
    if args.sweep_only:
        sw = gemv_sweep(rounds=args.sweep_rounds, kind=args.sweep)
        best, agg = sweep_summary(sw)
        if args.sweep_json:
            with open(args.sweep_json, "w") as f:
                json.dump(sw, f, indent=1)
        print(json.dumps({"gemv_cold": {"best": best, "decode_mix": agg}}), flush=True)
        return 0
    shape = QWEN3_0_6B
    cap = 48
    t = time.perf_counter()
    w = model_weights(shape, seed=0)
    log(f"weights generated in {time.perf_counter() - t:.1f} s")
    if args.prefill_only:
        print(json.dumps({"prefill_only": prefill_only(torch, wsg, shape, w)}), flush=True)
        return 0
    prompt32 = prompt_ids(PROMPT_SEEDS["short"], 32, shape.vocab)
    prompts = {8: prompt32[:8], 32: prompt32}
    model = wsg.Model(shape, w, max_context=cap, prefill_chunk=32)
    if args.no_graph:
        model.set_option(wsg._abi.WSG_OPT_USE_GRAPH, 0)

    # ---- correctness gate and CPU baseline (oracle on the host cores)
    expected = {}
    cpu = None
    errs = {}
    if not args.no_oracle:
        import oracle
        t = time.perf_counter()
        orc = oracle.OracleModel(shape, w, cap)
        log(f"oracle set up in {time.perf_counter() - t:.1f} s")
        for n_p in (8, 32):
            toks, ml, mkv, t_dec = validate(model, orc, prompts[n_p], 16)
            for n_o in (8, 16):
                expected[(n_p, n_o)] = toks[:n_o]
            errs[n_p] = (ml, mkv)
            if n_p == 8:
                cpu = {"value": round(15 / t_dec, 3), "unit": "tokens/s", "cores": cpu_threads(), "kind": "oracle",
                       "sample": "15 post-first-token decode forwards of the 8/16 generation (28 layers, "
                                 "float64 reductions), same weights and prompt"}
        log(f"validation passed: max |dlogit| {max(e[0] for e in errs.values()):.2e}, "
            f"max |dkv| {max(e[1] for e in errs.values()):.2e}")

    if args.lossless == "only":
        print(json.dumps({"lossless_bf16": lossless_bf16(torch, wsg, shape)}), flush=True)
        return 0
    if args.int4 == "only":
        del w, model
        torch.cuda.empty_cache()
        print(json.dumps({"int4_decoder": f16_storage_decoder(torch, wsg, shape, "int4")}), flush=True)
        return 0
    if args.fp16 == "only":
        del w, model
        torch.cuda.empty_cache()
        print(json.dumps({"fp16_decoder": f16_storage_decoder(torch, wsg, shape, "fp16")}), flush=True)
        return 0
    fixed_res = None
    if args.fixed != "off" and not args.no_oracle:
        fixed_res = fixed_context(torch, wsg, shape, w)
        if args.fixed == "only":
            print(json.dumps({"fixed_context": fixed_res}), flush=True)
            return 0
    two_res = None
    if args.two_token != "off" and not args.no_oracle:
        t = time.perf_counter()
        two_res = two_token(torch, wsg, shape, w)
        log(f"two-token section in {time.perf_counter() - t:.1f} s")
        if args.two_token == "only":
            print(json.dumps({"two_token": two_res}), flush=True)
            return 0
    long_res = None
    if args.long != "off" and not args.no_oracle:
        long_res = long_context(torch, wsg, shape, w)
        if args.long == "only":
            print(json.dumps({"long_context": long_res}), flush=True)
            return 0
    del w
    stage = STAGES[args.timed_stage]
    model.set_option(wsg._abi.WSG_OPT_TIMED_STAGE, -1)

    def run_step(rec, pipelined=True):
        for (n_p, n_o) in COMBOS:
            toks, ttft, dec, tot = generate(model, prompts[n_p], n_o, pipelined)
            if expected and toks != expected[(n_p, n_o)]:
                raise ValidationError(f"timed generation {n_p}/{n_o} returned {toks}, validated "
                                      f"{expected[(n_p, n_o)]}")
            if rec is not None:
                rec.append((n_p, n_o, ttft, dec, tot))

    for _ in range(args.warmup):
        run_step(None)
    rec = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run_step(rec)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    # After the timed region: the same generations one wsg_step per token, with HIP
    # events around the timed stage's launches (no events inside the timed region).
    model.set_option(wsg._abi.WSG_OPT_TIMED_STAGE, stage)
    run_step(None, pipelined=False)
    model.stage_time()   # reset the event accumulators
    step_rec = []
    for _ in range(args.steps):
        run_step(step_rec, pipelined=False)
    st_ms, st_n, st_bytes = model.stage_time()
    model.set_option(wsg._abi.WSG_OPT_TIMED_STAGE, -1)
    step_loop = {"decode_tok_s": round(sum(n_o - 1 for (_, n_o, _, _, _) in step_rec) / sum(r[3] for r in step_rec), 2),
                 "note": "the same generations with one wsg_step call per token (each waits for its token), "
                         "HIP events around the timed stage's launches; after the timed region"}

    dec_tokens = sum(n_o - 1 for (_, n_o, _, _, _) in rec)
    dec_time = sum(r[3] for r in rec)
    value = dec_tokens / dec_time
    per_combo = {}
    for (n_p, n_o) in COMBOS:
        rows = [r for r in rec if r[0] == n_p and r[1] == n_o]
        per_combo[f"{n_p}/{n_o}"] = {
            "ttft_ms": round(statistics.median(r[2] for r in rows) * 1e3, 3),
            "decode_tok_s": round(statistics.median((n_o - 1) / r[3] for r in rows), 1),
            "total_ms": round(statistics.median(r[4] for r in rows) * 1e3, 3)}
    weight_bytes = shape.weight_bytes_per_token(4)
    avg_launch_ms = st_ms / max(st_n, 1)
    achieved = (st_bytes / max(st_n, 1)) / (avg_launch_ms * 1e-3) / 1e9 if st_n else None
    timed_stage = {"kernel": STAGE_KERNEL[args.timed_stage], "bound": "hbm",
                   "achieved": round(achieved, 1) if achieved else None, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                   "frac": round(achieved / HBM_PEAK_GBPS, 4) if achieved else None,
                   "traffic": recorded_traffic(STAGE_KERNEL[args.timed_stage]),
                   "bytes_per_launch": st_bytes // max(st_n, 1), "avg_launch_us": round(avg_launch_ms * 1e3, 3),
                   "launches_timed": st_n, "timing": "HIP events on the model stream around each launch, "
                                                    "in the step-loop pass after the timed region (graph replay; "
                                                    "the head is a direct launch)"}
    stages = {}
    if args.roofline_reps:
        # at the context of the first short prompt's first step (its prefill done)
        model.reset()
        model.prefill(prompts[8])
        stages = stage_pass(wsg, model, timed_stage if args.timed_stage == "head" else None,
                            reps=args.roofline_reps)
    if stages:
        dom = max(stages, key=lambda k: stages[k]["ms_per_token"])
        d = stages[dom]
        roofline = {"bound": "hbm", "kernel": d["kernel"], "stage": dom, "achieved": d["gbps"],
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(d["gbps"] / HBM_PEAK_GBPS, 4),
                    "traffic": recorded_traffic(d["kernel"]), "bytes_per_launch": d["bytes_per_launch"],
                    "avg_launch_us": d["us_per_launch"], "launches_timed": d["launches"],
                    "share_of_stage_time": d["share"],
                    "timing": "stage with the largest share of per-token stage time; time per launch = "
                              "(step body graph - the same graph without the stage) / layers, HIP events around "
                              "whole replays on the model stream, alternated 20 times each, after the timed "
                              "region, at the context of the short prompt's first step"}
    else:
        roofline = timed_stage
    # the dispatch floor of the step's launches: 4 per layer, the head and the argmax
    n_launch = 4 * shape.n_layers + 2
    try:
        floor_us = launch_floor(torch, n_launch)
        floor = {"us_per_dependent_launch": round(floor_us, 3), "launches_per_token": n_launch,
                 "us_per_token": round(floor_us * n_launch, 1),
                 "share_of_token_time": round(floor_us * n_launch * value / 1e6, 4) if value else None,
                 "note": "a chain of dependent one-element kernels replayed as one HIP graph (median per node of "
                         "20 replays): the cost each launch pays besides its kernel time, an upper bound"}
    except Exception as e:   # a context measurement: its failure must not cost the bench line
        floor = {"us_per_dependent_launch": None, "error": f"{type(e).__name__}: {e}"}
    out = {
        "metric": "decode tokens/s + cold-cache effective weight GB/s (% of HBM peak), 1 MI355X",
        "value": None if args.no_oracle else round(value, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(elapsed / args.steps * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (random-init N(0,0.02) weights, uniform-random token ids)",
        "config": {"workload": "Qwen3-0.6B-shaped decoder, 28 layers, FP32 weights/activations/KV, batch 1, "
                               "greedy; prompt/output 8/8, 8/16, 32/8, 32/16 per step",
                   "global_batch": 1, "seq_len": 48, "parallelism": "single-gpu"},
        "decode_weight_gbps": round(weight_bytes * value / 1e9, 1),
        "decode_weight_frac_of_hbm_peak": round(weight_bytes * value / 1e9 / HBM_PEAK_GBPS, 4),
        "step_roofline": {"bound": "hbm", "bytes_per_token": weight_bytes,
                          "achieved": round(weight_bytes * value / 1e9, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                          "frac": round(weight_bytes * value / 1e9 / HBM_PEAK_GBPS, 4),
                          "note": "decode weight bytes per token x post-first-token tokens/s"},
        "per_combo_median": per_combo,
        "decode_loop": "wsg_generate: the decode steps of a generation enqueued back to back, one wait",
        "step_loop": step_loop,
        "roofline": roofline,
        "stage_rooflines": stages,
        "launch_floor": floor,
        ("roofline_" + args.timed_stage): timed_stage,
        "cpu_baseline": cpu,
        "validation": ({"status": "passed", "max_abs_logit_err": max(e[0] for e in errs.values()),
                        "max_abs_kv_err": max(e[1] for e in errs.values()), "rtol": 1e-3, "atol": 1e-3}
                       if errs else {"status": "skipped"}),
        "graphs": not args.no_graph,
        "host": host_info(),
        "provenance": provenance(model),
        "long_context": long_res,
        "fixed_context": fixed_res,
        "two_token": two_res,
    }
    model.close()
    del model
    torch.cuda.empty_cache()
    if args.lossless == "on" and not args.no_oracle:
        t = time.perf_counter()
        out["lossless_bf16"] = lossless_bf16(torch, wsg, shape)
        log(f"lossless BF16-in-FP32 section in {time.perf_counter() - t:.1f} s")
        torch.cuda.empty_cache()
    if args.int4 == "on" and not args.no_oracle:
        t = time.perf_counter()
        out["int4_decoder"] = f16_storage_decoder(torch, wsg, shape, "int4")
        log(f"int4 decoder section in {time.perf_counter() - t:.1f} s")
        torch.cuda.empty_cache()
    if args.fp16 == "on" and not args.no_oracle:
        t = time.perf_counter()
        out["fp16_decoder"] = f16_storage_decoder(torch, wsg, shape, "fp16")
        log(f"fp16 decoder section in {time.perf_counter() - t:.1f} s")
        torch.cuda.empty_cache()
    if args.sweep != "none":
        sw = gemv_sweep(rounds=args.sweep_rounds, kind=args.sweep)
        best, agg = sweep_summary(sw)
        out["gemv_cold"] = {"best": best, "decode_mix": agg, "note": "dispatch-inclusive (graph replay) per-dispatch "
                            "time over >= 1 GiB of distinct matrices per shape; median of 15 rounds; stream ceiling "
                            "= a read-only 16-byte-load kernel over the same copies"}
        if not args.no_oracle:
            t = time.perf_counter()
            out["gemv_cold"]["cpu_oracle"] = cpu_gemv_rates()
            log(f"oracle GEMVs on the host in {time.perf_counter() - t:.1f} s")
        if args.sweep_json:
            with open(args.sweep_json, "w") as f:
                json.dump(sw, f, indent=1)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
