#!/usr/bin/env python3
"""Decode-step benchmark of the quantized KV cache on one MI355X.

A step is one pass of the whole hot path over one batch: quantize-append of
the new token of every sequence (folding the fp16 window into the quantized
cache when a block fills) followed by split-K decode attention over all cached
tokens (pass 1 + merge), issued as one kvq_decode_step call (one launch pair
unless a fold is due).  Inputs are synthetic, seeded, and resident in HBM
before the timed region.

Prints one JSON line.  ``value`` is algorithmic bytes per step / step time
(GB/s); ``roofline`` prices the decode-attention launches (pass 1 + merge)
against MI355X's 8 TB/s HBM peak with their durations measured by HIP events
on the launch stream; ``cpu_baseline`` times the CPU oracle (dequantize from
codes + fp64 attention) on a bounded sample of (sequence, kv head) pairs.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# cache format of each workload: (k spec, v spec, residual, pre-RoPE, calibrate)
FORMATS = {
    "c3_fp8_e4m3_gqa_8k": ((3, 8, 0, 0), (3, 8, 0, 0), 0, False, True),
    "c3_fp8_e5m2_gqa_8k": ((4, 8, 0, 0), (4, 8, 0, 0), 0, False, False),
    "c4_int4_llama70b_128k": ((1, 4, 1, 128), (1, 4, 2, 0), 128, False, False),
    "c5_int2_kivi_prerope_32k": ((1, 2, 1, 32), (1, 2, 2, 32), 32, True, False),
}
# what bounds each workload's attention launch, from the measurements recorded
# with the profiles (SQ busy counters, context / batch sweeps, ablations)
LIMITER = {
    "c3_fp8_e4m3_gqa_8k": "hbm streaming (~6.7 TB/s marginal) plus ~8.6 us fixed per-launch cost",
    "c3_fp8_e5m2_gqa_8k": "hbm streaming plus fixed per-launch cost, as the E4M3 cache",
    "c4_int4_llama70b_128k": "~11 us fixed per-launch cost at batch 1 (two kernels, start-up) over ~5.1 TB/s streaming, latency-bound 32-token steps at two wavefronts per SIMD",
    "c5_int2_kivi_prerope_32k": "vector-ALU issue (~634 VALU instructions per 32-token step, ~67% of SIMD cycles: pre-RoPE dequantize, rotation and fp16 split per key pair) and the step's dependent chain at two wavefronts per SIMD (a variant with the rotation on the matrix unit, 455 per step, ran in equal time)",
}
DESCR = {
    "c3_fp8_e4m3_gqa_8k": "FP8 E4M3 K/V, per-kv-head calibrated scales",
    "c3_fp8_e5m2_gqa_8k": "FP8 E5M2 K/V, no scales",
    "c4_int4_llama70b_128k": "INT4 K per-channel G128 + INT4 V per-token, fp16 window 128",
    "c5_int2_kivi_prerope_32k": "INT2 K per-channel G32 (pre-RoPE) + INT2 V per-token G32, fp16 window 32",
}


def code_bits(spec):
    scheme, bits = spec[0], spec[1]
    return bits if scheme in (0, 1) else 8


def algorithmic_bytes(w, fmt, T, meta_bytes=4, lens=None):
    """Bytes one decode attention over T tokens must move: every packed code, its
    scale/zero (fp32, or fp16 with meta_bytes=2) and the fp16 window read once,
    q (bf16) read, out (fp32) written.  lens: per-sequence lengths of a ragged
    batch (T is then ignored); returns (bytes, Tq of the last length)."""
    kspec, vspec, R, _, _ = fmt
    B, Hq, Hkv, D = w["B"], w["Hq"], w["Hkv"], w["D"]
    G = kspec[3] if (kspec[0] in (1, 2) and kspec[2] == 1 and kspec[3] > 0) else 1

    def per_seq(T):
        Tq = G * (max(T - R, 0) // G) if (R > 0 or G > 1) else T
        per = 0.0
        per += Tq * D * code_bits(kspec) / 8 + Tq * D * code_bits(vspec) / 8
        for spec in (kspec, vspec):
            nmeta = 2 if spec[0] == 1 else 1
            if spec[0] in (1, 2):
                if spec[2] == 1:
                    per += (Tq // spec[3] if spec[3] else 1) * D * meta_bytes * nmeta
                elif spec[2] == 2:
                    per += Tq * (D // (spec[3] or D)) * meta_bytes * nmeta
                else:
                    per += meta_bytes * nmeta
        per += (T - Tq) * D * 2 * 2
        return per, Tq

    if lens is None:
        lens = [T] * B
    total, Tq = 0.0, 0
    for t in lens:
        per, Tq = per_seq(int(t))
        total += per * Hkv
    fp8_scales = 8 * Hkv if kspec[0] in (3, 4) else 0
    return total + fp8_scales + B * Hq * D * 2 + B * Hq * D * 4, Tq


def cpu_baseline(name, w, fmt, T, bytes_per_step, budget_s=12.0, meta16=False):
    """The oracle as it stands, on host cores: per sampled (sequence, kv head),
    dequantize the cache from its codes and run fp64 attention for its query
    heads; scaled to the whole step."""
    import numpy as np
    import workloads as W
    from oracle import attention as OA
    from oracle import cache as OC

    kspec, vspec, R, pre_rope, calibrate = fmt
    n_rep = w["Hq"] // w["Hkv"]
    sub = OC.Cfg(1, n_rep, 1, w["D"], OC.Spec(*kspec, meta16=meta16), OC.Spec(*vspec, meta16=meta16), R, pre_rope,
                 w.get("rope_base", 1e4))
    q = W.bf16_bits_to_f32(W.query(name))
    sm = 1.0 / math.sqrt(w["D"])
    done, spent = 0, 0.0
    pairs = [(b, h) for b in range(w["B"]) for h in range(w["Hkv"])]
    for (b, h) in pairs:
        kb, vb = W.kv_chunk(name, b, h, "k"), W.kv_chunk(name, b, h, "v")
        if w.get("n_new", 0):
            kb = np.concatenate([kb, W.new_token_chunk(name, b, h, "k")])
            vb = np.concatenate([vb, W.new_token_chunk(name, b, h, "v")])
        Kf, Vf = W.bf16_bits_to_f32(kb)[None, None], W.bf16_bits_to_f32(vb)[None, None]
        st = OC.quantize_cache(sub, Kf, Vf, T, k_scale=np.ones(1, np.float32), v_scale=np.ones(1, np.float32))
        Tq = st["Tq"]
        t0 = time.perf_counter()
        kh = np.concatenate([OC.dequantize_part(st["k"], sub.k), Kf[:, :, Tq:T].astype(np.float16).astype(np.float32)
                             if OC.has_window(sub) else Kf[:, :, Tq:T]], axis=2)
        vh = np.concatenate([OC.dequantize_part(st["v"], sub.v), Vf[:, :, Tq:T].astype(np.float16).astype(np.float32)
                             if OC.has_window(sub) else Vf[:, :, Tq:T]], axis=2)
        OA.decode_attention(q[b:b + 1, h * n_rep:(h + 1) * n_rep], kh, vh, sm,
                            pre_rope_base=sub.rope_base if pre_rope else None)
        spent += time.perf_counter() - t0
        done += 1
        if spent >= budget_s:
            break
    per_pair = spent / done
    step_s = per_pair * len(pairs)
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = 1
    return {
        "value": round(bytes_per_step / step_s / 1e9, 4),
        "unit": "GB/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": f"{done} of {len(pairs)} (sequence, kv head) pairs: numpy dequantize from codes + fp64 "
                  f"attention ({'with RoPE, ' if pre_rope else ''}{n_rep} query heads each), "
                  f"{per_pair:.3f} s/pair, scaled to the full step ({step_s:.1f} s/step, "
                  f"{1.0 / step_s:.4f} steps/s); host os.cpu_count()={os.cpu_count()}",
        "seconds_per_step": round(step_s, 3),
    }


ATTN_SOURCES = ("quantized_decode_attention_05_amd/csrc/kvq_attn_mfma.hip",
                "quantized_decode_attention_05_amd/csrc/kvq_attn.hip")


def attention_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name):
    """HBM bytes per attention launch (pass 1 + merge) from the committed
    hardware-counter summary of this workload, when it was taken on the
    current attention sources; None otherwise."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("attention_source_hash") != attention_source_hash():
        return None
    return {"bytes_per_launch": t["traffic_bytes_per_launch"],
            "source": f"profiles/traffic_{name}.json (FETCH_SIZE + WRITE_SIZE, copy-calibrated)"}


def summarize_counters(workload, fetch_dir, write_dir, copy_bytes, command):
    """Write profiles/traffic_<workload>.json and .md from two rocprofv3 --pmc
    runs of this script with --copy-probe (FETCH_SIZE, then WRITE_SIZE, KiB per
    dispatch).  The copy kernel moves copy_bytes each way and calibrates both
    counters; traffic = calibrated FETCH + WRITE of one attention launch
    (pass 1 + merge), averaged over its dispatches."""
    import csv
    import glob

    def per_dispatch(d, counter):
        acc = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            for r in csv.DictReader(open(f)):
                if r["Counter_Name"] != counter:
                    continue
                key = (r["Kernel_Name"], int(r.get("Dispatch_Id") or 0))
                acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
        return acc

    def mean_of(table, needle, after=-1):
        vals = [(k, v) for (k, i), v in table.items() if needle in k and i > after]
        if not vals:
            raise SystemExit(f"no dispatch of a kernel matching {needle!r}")
        return vals[0][0], sum(v for _, v in vals) / len(vals)

    def probe(table):
        # the copy probe runs after the timed region: only copies issued after
        # the last attention launch count (set-up copies, such as the arena
        # copies of a rotating-arena run, are excluded)
        last = max(i for (k, i) in table if "attn_mfma" in k)
        return mean_of(table, "copyBuffer", after=last)[1]

    fetch, write = per_dispatch(fetch_dir, "FETCH_SIZE"), per_dispatch(write_dir, "WRITE_SIZE")
    f_copy, w_copy = probe(fetch), probe(write)
    k1, f_attn = mean_of(fetch, "attn_mfma")
    _, f_merge = mean_of(fetch, "attn_merge")
    _, w_attn = mean_of(write, "attn_mfma")
    _, w_merge = mean_of(write, "attn_merge")
    cf, cw = copy_bytes / (f_copy * 1024.0), copy_bytes / (w_copy * 1024.0)
    fetched = (f_attn + f_merge) * 1024.0 * cf
    written = (w_attn + w_merge) * 1024.0 * cw
    out = {
        "workload": workload,
        "attention_source_hash": attention_source_hash(),
        "traffic_bytes_per_launch": round(fetched + written),
        "fetch_bytes_per_launch": round(fetched),
        "write_bytes_per_launch": round(written),
        "fetch_kib_per_dispatch": {"pass1": f_attn, "merge": f_merge, "copy": f_copy},
        "write_kib_per_dispatch": {"pass1": w_attn, "merge": w_merge, "copy": w_copy},
        "copy_bytes": copy_bytes,
        "calibration": {"fetch": cf, "write": cw},
        "pass1_kernel": k1,
        "command": command,
    }
    base = os.path.join(ROOT, "profiles", f"traffic_{workload}")
    with open(base + ".json", "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def timed_window(qtok, T0, warmup, steps, period):
    """Untimed positioning steps to run after the warm-up so that the timed
    decode steps hold a fold of the fp16 window, as a long decode run does once
    every ``period`` steps (the key group).  qtok(T) is the number of quantized
    tokens of a cache holding T tokens; step i appends at T0 + i.  Returns
    (extra, folds): the extra steps, and the offsets inside the timed window of
    the steps that fold.  Caches without a window (period <= 1) fold never."""
    if period <= 1:
        return 0, []

    def folds_at(i):
        return qtok(T0 + i + 1) > qtok(T0 + i)

    first = next((i for i in range(2 * period + 1) if folds_at(i)), None)
    if first is None:
        return 0, []
    f = first
    while f < warmup + steps // 2:
        f += period
    extra = f - steps // 2 - warmup
    start = warmup + extra
    return extra, [i - start for i in range(start, start + steps) if folds_at(i)]


def gpu_clock_record():
    """Clock and power of the GPU as rocm-smi reports them (sampled while
    attention launches are queued), or the reason there is none."""
    import subprocess
    # under a profiler the tool's preloaded library would initialise the GPU in
    # rocm-smi's own process too, which then re-executes its interpreter
    if "rocprof" in os.environ.get("LD_PRELOAD", "") or any(k.startswith("ROCPROF") for k in os.environ):
        return {"error": "not sampled under a profiler"}
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--showpower", "--json"], capture_output=True,
                           text=True, timeout=20)
        data = json.loads(r.stdout)
    except Exception as e:  # noqa: BLE001  (a record, never a failure)
        return {"error": f"{type(e).__name__}: {e}"[:200]}
    card = next((v for k, v in sorted(data.items()) if k.startswith("card")), {})
    keep = {k.strip(): v for k, v in card.items()
            if any(x in k.lower() for x in ("sclk", "mclk", "fclk", "power"))}
    return keep or {"raw": str(data)[:300]}


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--summarize-counters":
        # bench.py --summarize-counters WORKLOAD FETCH_DIR WRITE_DIR COPY_MIB "COMMAND"
        summarize_counters(sys.argv[2], sys.argv[3], sys.argv[4], int(sys.argv[5]) << 20, sys.argv[6])
        return
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5_int2_kivi_prerope_32k", choices=list(FORMATS))
    ap.add_argument("--kernel", type=int, default=0, help="0 auto, 1 generic, 2 MFMA")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--spinup", type=float, default=1.0,
                    help="seconds of untimed attention launches before the warm-up steps")
    ap.add_argument("--arena-copies", type=int, default=0,
                    help="identical arenas the attention launches rotate through (0: 4 when the "
                         "workload appends nothing and its arena is under 1 GiB, else 1), so that "
                         "a cache small enough for MI355X's 256 MB Infinity Cache is not re-read "
                         "from it")
    ap.add_argument("--context", type=int, default=0, metavar="T",
                    help="prefill context length in place of the workload's own (same format, seeds "
                         "and value recipe; a measurement of the format at another size, reported "
                         "under a derived workload name)")
    ap.add_argument("--meta-f16", action="store_true",
                    help="store the INT sides' scales and zero-points in fp16 (reported under a "
                         "derived workload name)")
    ap.add_argument("--batch", type=int, default=0, metavar="B",
                    help="number of sequences in place of the workload's own (as --context)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="size of the device-to-device copy that measures the copy ceiling (default "
                         "2048 MiB); the same copy kernel calibrates hardware byte counters")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the attention-only timings of the other serving-shaped workloads")
    ap.add_argument("--paged", type=int, default=0, metavar="P",
                    help="a paged cache of P-token pages handed out in a shuffled order (block tables; "
                         "reported under a derived workload name)")
    ap.add_argument("--ragged", action="store_true",
                    help="with --paged: sequence b holds T - (1021 b mod 8192) tokens instead of T")
    a = ap.parse_args()
    if a.gpus != 1:
        print(f"bench.py: runs on one GPU; --gpus {a.gpus} is not supported "
              f"(the path shards over (sequence, kv head) pairs without communication)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import quantized_decode_attention_05_amd as K
    import workloads as W

    base = a.workload
    name = base
    w = W.WORKLOADS[base]
    if a.context or a.batch:
        # the same cache format and inputs recipe at another context / batch size
        w = dict(w, T=a.context or w["T"], B=a.batch or w["B"])
        name = f"{base}@B{w['B']}_T{w['T']}"
        W.WORKLOADS[name] = w
    if a.meta_f16:
        name = f"{name}+meta16"
        W.WORKLOADS[name] = w
    if a.ragged and not a.paged:
        raise SystemExit("bench.py: --ragged needs --paged")
    if a.paged:
        name = f"{name}+paged{a.paged}" + ("+ragged" if a.ragged else "")
        W.WORKLOADS[name] = w
    meta_bytes = 2 if a.meta_f16 else 4
    fmt = FORMATS[base]
    kspec, vspec, R, pre_rope, calibrate = fmt
    B, Hq, Hkv, D, T0 = w["B"], w["Hq"], w["Hkv"], w["D"], w["T"]
    n_new = w.get("n_new", 0)
    dev = torch.device("cuda:0")

    def make_cfg(cap, paged=False):
        P = a.paged if paged else 0
        pages = B * (-(-cap // P)) + 8 if paged else 0
        return K.make_config(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, max_tokens=cap,
                             k=kspec, v=vspec, in_dtype=K.BF16, out_dtype=K.F32, residual=R,
                             pre_rope_k=pre_rope, rope_base=w.get("rope_base", 10000.0),
                             meta_dtype=K.F16 if a.meta_f16 else K.F32, page_tokens=P, num_pages=pages)

    # positioning: the timed steps hold a fold of the fp16 window (one every
    # `period` steps), and a whole fold period is timed on its own afterwards
    probe = make_cfg(T0 + 4096)
    lay = K.kvq_arena_layout(probe)
    period = lay.token_group if (n_new == 1 and lay.ring_slots > 0) else 1
    extra, folds_in_window = timed_window(lambda T: K.kvq_quantized_tokens(probe, T), T0, a.warmup, a.steps,
                                          period)
    steps_total = a.warmup + extra + a.steps + (period if period > 1 else 0)
    cap = T0 + n_new * (steps_total + 1) + 64
    cfg = make_cfg(cap, paged=a.paged > 0)
    # paged caches: lengths lens0[b] + s after s decode steps (s = T - T0 for
    # the uniform-length bookkeeping below), one device array per s prepared
    # up front so the timed steps launch nothing else
    lens0 = np.array([T0 - (1021 * b) % 8192 for b in range(B)] if a.ragged else [T0] * B, dtype=np.int64)
    if a.paged:
        pages = K.kvq_arena_layout(cfg).pages
        nblk = -(-cap // a.paged)
        perm = np.random.default_rng(1234).permutation(pages)[:B * nblk].astype(np.int32)
        bt = torch.from_numpy(perm.reshape(B, nblk)).to(dev)
        lens_dev = [torch.from_numpy((lens0 + i).astype(np.int32)).to(dev) for i in range(steps_total + 3)]

    def lens_at(T):
        return lens0 + (T - T0)
    print(f"[bench] {name}: generating inputs", file=sys.stderr, flush=True)
    kp = torch.from_numpy(W.full_prefill(name, "k").view(np.int16)).view(torch.bfloat16).to(dev)
    vp = torch.from_numpy(W.full_prefill(name, "v").view(np.int16)).view(torch.bfloat16).to(dev)
    q = torch.from_numpy(W.query(name).view(np.int16)).view(torch.bfloat16).to(dev)
    if n_new:
        kn = torch.from_numpy(W.full_new_tokens(name, "k").view(np.int16)).view(torch.bfloat16).to(dev)
        vn = torch.from_numpy(W.full_new_tokens(name, "v").view(np.int16)).view(torch.bfloat16).to(dev)
    arena = torch.empty(K.kvq_arena_bytes(cfg), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.zeros(K.kvq_workspace_bytes(cfg, cap, a.kernel, a.splits), dtype=torch.uint8, device=dev)
    sm = 1.0 / math.sqrt(D)
    print(f"[bench] prefill T={T0}", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream(dev)

    def prefill(kin, vin, lens):
        """Quantize-append every sequence's first tokens from position 0."""
        if a.paged:
            zero = torch.zeros(B, dtype=torch.int32, device=dev)
            K.kvq_paged_quantize_append(cfg, arena, bt, zero, kin, vin, lens,
                                        flags=K.INIT | (K.CALIBRATE if calibrate else 0))
        else:
            K.kvq_quantize_append(cfg, arena, 0, kin, vin, flags=K.CALIBRATE if calibrate else 0)

    # an untimed append of the first 32 tokens loads the kernels; the timed
    # prefill then rewrites the cache from position 0
    n_w = min(32, T0)
    prefill(kp[:, :, :n_w].contiguous(), vp[:, :, :n_w].contiguous(),
            torch.full((B,), n_w, dtype=torch.int32, device=dev) if a.paged else None)
    torch.cuda.synchronize()
    pe0, pe1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    pe0.record(stream)
    prefill(kp, vp, lens_dev[0] if a.paged else None)
    pe1.record(stream)
    torch.cuda.synchronize()
    prefill_ms = pe0.elapsed_time(pe1)
    prefill_tokens = int(lens0.sum()) if a.paged else B * T0
    prefill_in_bytes = 2 * prefill_tokens * Hkv * D * kp.element_size()
    del kp, vp
    torch.cuda.synchronize()
    T = T0
    copies = a.arena_copies or (4 if (n_new == 0 and arena.numel() < (1 << 30)) else 1)
    if copies > 1 and n_new:
        raise SystemExit("bench.py: --arena-copies > 1 needs a workload without appends")
    arenas = [arena] + [arena.clone() for _ in range(copies - 1)]
    torch.cuda.synchronize()

    def attend(arena_i, T):
        """Decode attention over T tokens (paged: the lengths after T - T0 steps)."""
        if a.paged:
            K.kvq_paged_decode_attention(cfg, arena_i, bt, lens_dev[T - T0], int(lens_at(T).max()), q, out, sm, ws,
                                         a.kernel, a.splits)
        else:
            K.kvq_decode_attention(cfg, arena_i, T, q, out, sm, ws, a.kernel, a.splits)

    def step(T):
        """One decode step: append the new token of every sequence at T, attend
        over T + 1 (kvq_decode_step: one launch unless a fold is due)."""
        if n_new == 1 and a.paged:
            K.kvq_paged_decode_step(cfg, arena, bt, lens_dev[T - T0], int(lens_at(T).max()) + 1, kn, vn, q, out, sm,
                                    ws, a.kernel, a.splits)
            return T + 1
        if n_new == 1:
            K.kvq_decode_step(cfg, arena, T, kn, vn, q, out, sm, ws, a.kernel, a.splits)
            return T + 1
        if n_new:
            K.kvq_quantize_append(cfg, arena, T, kn, vn)
            T += n_new
        K.kvq_decode_attention(cfg, arena, T, q, out, sm, ws, a.kernel, a.splits)
        return T

    def timed(fn, n):
        """Mean ms of fn(i) over n back-to-back calls, between two HIP events
        recorded on the launch stream."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(n):
            fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # Clock spin-up (untimed, leaves the cache unchanged): the GPU raises its
    # clocks only under sustained load, so attention at the starting context is
    # launched for a.spinup seconds before the warm-up steps.
    spin_end = time.perf_counter() + a.spinup
    clocks = None
    while time.perf_counter() < spin_end or clocks is None:
        for i in range(10):
            attend(arenas[i % copies], T)
        if clocks is None:
            for i in range(40):   # keep the GPU busy while rocm-smi samples it
                attend(arenas[i % copies], T)
            clocks = gpu_clock_record()
        torch.cuda.synchronize()
    for _ in range(a.warmup + extra):
        T = step(T)
    torch.cuda.synchronize()
    T_first = T + n_new
    wall0 = time.perf_counter()
    if n_new:
        box = [T]

        def one(i):
            box[0] = step(box[0])
        ms_per_step = timed(one, a.steps)
        T = box[0]
    else:
        ms_per_step = timed(lambda i: attend(arenas[i % copies], T), a.steps)
    wall = time.perf_counter() - wall0
    if n_new:
        # decode attention alone (pass 1 + merge) at the final context, for the
        # roofline (the steps above also appended)
        attn_us = 1000.0 * timed(lambda i: attend(arena, T), a.steps)
    else:
        attn_us = 1000.0 * ms_per_step
    fold_period = None
    if period > 1:
        # a whole fold period of decode steps: exactly one of them folds
        T_p0 = T
        box = [T]

        def one(i):
            box[0] = step(box[0])
        ms_p = timed(one, period)
        T = box[0]
        fold_period = {"steps": period, "context_start": T_p0 + 1, "context_end": T,
                       "ms_per_step": round(ms_p, 5), "decode_steps_per_s": round(1000.0 / ms_p, 2),
                       "note": "fold-amortized rate: the fp16 window folds once in these steps"}
    warm_us = None
    if copies > 1:
        # the same launches on one arena only (cache-warm), reported separately
        warm_us = 1000.0 * timed(lambda i: attend(arena, T), a.steps)
    T_last = T_first + a.steps - 1 if n_new else T
    T_mid = (T_first + T_last) // 2
    rag = (lambda T: lens_at(T)) if a.paged else (lambda T: None)
    bytes_step, Tq = algorithmic_bytes(w, fmt, T_mid, meta_bytes, lens=rag(T_mid))
    T_attn = T
    bytes_attn = algorithmic_bytes(w, fmt, T_attn, meta_bytes, lens=rag(T_attn))[0]
    achieved = bytes_attn / (attn_us * 1e-6) / 1e9
    value = bytes_step / (ms_per_step * 1e-3) / 1e9
    used_kernel = a.kernel
    if used_kernel == 0:
        try:
            K.kvq_workspace_bytes(cfg, T, K.KERNEL_MFMA)
            used_kernel = 2
        except K.KvqError:
            used_kernel = 1
    # copy ceiling: a plain device-to-device copy (HIP's copy kernel) of a
    # 2 GiB buffer, reads + writes over time; the same copy calibrates counters
    del arenas
    copy_bytes = (a.copy_probe or 2048) << 20
    src = torch.empty(copy_bytes, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    copy_ms = timed(lambda i: dst.copy_(src), 5)
    copy_gbs = 2.0 * copy_bytes / (copy_ms * 1e-3) / 1e9
    del src, dst
    res = {
        "metric": "quantized decode-attention HBM GB/s (% of peak) + decode steps/s at 32K ctx",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2+fp32" if kspec[1] == 2 else ({3: "fp8e4m3+fp32", 4: "fp8e5m2+fp32"}.get(kspec[0], "int4+fp32")),
        "data": "synthetic (seeded Gaussian K/V with fixed outlier key channels, bf16)",
        "config": {
            "workload": name, "format": DESCR[base], "batch": B, "q_heads": Hq, "kv_heads": Hkv,
            "head_dim": D, "context_start": T_first, "context_end": T_last, "append_tokens_per_step": n_new,
            "attention_kernel": {1: "generic", 2: "mfma"}[used_kernel],
            "arena_copies": copies,
            "scale_zero_dtype": "f16" if a.meta_f16 else "f32",
            "untimed_positioning_steps": extra,
            "folds_in_timed_steps": len(folds_in_window),
            "layout": (f"paged, {a.paged}-token pages in a shuffled order" if a.paged else "contiguous"),
            "lengths": ("ragged " + f"{int(lens0.min())}..{int(lens0.max())} at the start" if a.ragged
                        else "uniform"),
        },
        "decode_steps_per_s": round(1000.0 / ms_per_step, 2),
        "attention_us": round(attn_us, 3),
        "attention_pct_of_hbm_peak": round(100.0 * achieved / HBM_PEAK_GBS, 2),
        "algorithmic_bytes_per_step": int(bytes_step),
        "wall_s_timed": round(wall, 4),
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None,
            "copy_gbs": round(copy_gbs, 1),
            "frac_of_copy": round(achieved / copy_gbs, 4),
            "copy": f"device-to-device copy of {copy_bytes >> 20} MiB (HIP copy kernel), reads + writes / time, "
                    f"mean of 5 between HIP events",
            "kernel": "decode attention launch: pass 1 (split-K) + merge; mean of back-to-back launches between two HIP events on the launch stream",
            "limiter": LIMITER[base] if name in (base, base + "+meta16") else "not recorded for this size",
        },
        "gpu_clocks": clocks,
    }
    res["prefill"] = {
        "tokens": prefill_tokens, "ms": round(prefill_ms, 4),
        "input_gb_per_s": round(prefill_in_bytes / (prefill_ms * 1e-3) / 1e9, 1),
        "note": "one quantize-append of every sequence's context from position 0 (codes, scales / zero-points, "
                "window; FP8 calibration included), between two HIP events on the launch stream, after an untimed "
                "32-token append that loads the kernels",
    }
    if fold_period is not None:
        res["fold_period"] = fold_period
    if warm_us is not None:
        res["attention_us_one_arena_warm"] = round(warm_us, 3)
    traffic = measured_traffic(name) if name in (base, base + "+meta16") else None
    if traffic is not None:
        res["roofline"]["traffic"] = traffic["bytes_per_launch"]
        res["roofline"]["traffic_source"] = traffic["source"]
    if a.copy_probe > 0:
        res["copy_probe_bytes"] = copy_bytes
    del arena, ws
    torch.cuda.empty_cache()
    if not a.no_secondary and name == base:
        res["secondary"] = {}
        for other in SECONDARY:
            if other == base:
                continue
            print(f"[bench] secondary: {other} attention only", file=sys.stderr, flush=True)
            res["secondary"][other] = attention_only(K, W, torch, other, a.steps, min(a.spinup, 0.5))
    if not a.no_cpu:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(name, w, fmt, T_first, algorithmic_bytes(w, fmt, T_first, meta_bytes)[0],
                                           a.cpu_budget, meta16=a.meta_f16)
    print(json.dumps(res), flush=True)


# the other serving-shaped workloads, timed (attention only) in the same run
SECONDARY = ("c3_fp8_e4m3_gqa_8k", "c4_int4_llama70b_128k", "c5_int2_kivi_prerope_32k")


def attention_only(K, W, torch, name, steps, spinup):
    """Decode attention (pass 1 + merge) of a workload's full-size cache after
    its prefill and, where the workload appends, its first new token: mean of
    `steps` back-to-back launches rotated over identical arenas (4 when the
    arena is under 1 GiB, so the 256 MB Infinity Cache cannot hold them)."""
    import numpy as np
    w = W.WORKLOADS[name]
    kspec, vspec, R, pre_rope, calibrate = FORMATS[name]
    B, Hq, Hkv, D = w["B"], w["Hq"], w["Hkv"], w["D"]
    n_new = w.get("n_new", 0)
    T = w["T"] + n_new
    dev = torch.device("cuda:0")
    cfg = K.make_config(batch=B, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, max_tokens=T, k=kspec, v=vspec,
                        in_dtype=K.BF16, out_dtype=K.F32, residual=R, pre_rope_k=pre_rope,
                        rope_base=w.get("rope_base", 10000.0))

    def up(x):
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).to(dev)

    arena = torch.empty(K.kvq_arena_bytes(cfg), dtype=torch.uint8, device=dev)
    kp, vp = up(W.full_prefill(name, "k")), up(W.full_prefill(name, "v"))
    K.kvq_quantize_append(cfg, arena, 0, kp, vp, flags=K.CALIBRATE if calibrate else 0)
    del kp, vp
    if n_new:
        K.kvq_quantize_append(cfg, arena, w["T"], up(W.full_new_tokens(name, "k")), up(W.full_new_tokens(name, "v")))
    q = up(W.query(name))
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    ws = torch.zeros(K.kvq_workspace_bytes(cfg, T), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    copies = 4 if arena.numel() < (1 << 30) else 1
    arenas = [arena] + [arena.clone() for _ in range(copies - 1)]
    sm = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream(dev)
    end = time.perf_counter() + spinup
    while time.perf_counter() < end:
        for i in range(10):
            K.kvq_decode_attention(cfg, arenas[i % copies], T, q, out, sm, ws)
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(steps):
        K.kvq_decode_attention(cfg, arenas[i % copies], T, q, out, sm, ws)
    e1.record(stream)
    torch.cuda.synchronize()
    us = 1000.0 * e0.elapsed_time(e1) / steps
    nbytes = algorithmic_bytes(w, FORMATS[name], T)[0]
    gbs = nbytes / (us * 1e-6) / 1e9
    del arenas, arena, ws
    torch.cuda.empty_cache()
    return {"attention_us": round(us, 3), "achieved_gbs": round(gbs, 1),
            "pct_of_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
            "attention_launches_per_s": round(1e6 / us, 1), "context": T, "arena_copies": copies,
            "algorithmic_bytes": int(nbytes)}


if __name__ == "__main__":
    main()
