"""Benchmark of the compressed-domain KV-cache decode hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]

Workload (default, ``c4``): batch 8, 32 query heads / 8 KV heads (GQA 4:1),
d = 128, 4-bit PQ4 keys and values, context 65,536 per sequence: 65,535
tokens prefilled, then every step quantizes one new fp16 token per sequence
and KV head into position 65,535, rotates the 256 queries and runs the fused
split-K decode attention over the compressed bytes.  Inputs are the seeded
synthetic rows of ``synth`` (Gaussian, 1% of channels scaled by 8), already
resident in HBM when timing starts.

One step = append (K and V) + query rotation + decode partial, in one launch
of the decode kernel (tq_decode_step), then the combine of the split records.
Two launches measured faster than the one-launch step that merges the splits
in each stream's last workgroup (``--one-launch``).  Two cache copies (1.14 GB
together) alternate between steps so that the 256 MB Infinity Cache cannot
hold the bytes a step reads.  The default 200 warm-up steps (about 20 ms of
decode) let the GPU clock settle before the 200 timed steps; a 10-step
warm-up measures the kernel about 10% slower.

Output: one JSON line.  ``value`` is compressed-KV tokens attended per second
(batch * context / host-clock step time).  ``roofline`` reports the dominant
kernel, decode_partial: algorithmic K+V bytes per launch over its mean
duration, measured with HIP events that the runtime attaches to the kernel's
own dispatch on every 8th timed step (events on every step add about 4 us to
each step they are on).  ``decode_attention_gbs`` divides the same bytes by
the whole host-clock step (append, rotation, partial, combine and the gaps
between launches).
``cpu_baseline`` times the float64 CPU oracle on a bounded sample of the same
step.  ``--copy-calibration`` additionally runs a plain 1 GiB elementwise
copy, the reference kernel for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
COUNTERS_FILE = os.path.join(ROOT, "profiles", "decode_partial_pq4_c4_counters.txt")
# the sources the decode_partial kernels are compiled from
DECODE_SRCS = [os.path.join(ROOT, "compressed_domain_attention_kv_amd", "csrc", f)
               for f in ("tq_decode.hip", "tq_device.h", "tq_internal.h", "tq_pq4.h")]


def _log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def decode_source_hash():
    h = hashlib.sha256()
    for path in DECODE_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode_partial launch from the committed counter summary,
    or None when the kernel source changed since the counters were taken."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    vals = {}
    for ln in open(COUNTERS_FILE):
        if ":" in ln and not ln.startswith("#"):
            k, v = ln.split(":", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_source_sha256") != decode_source_hash():
        return None
    try:
        return int(float(vals["traffic_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def gen_rows(w, tensor, count, threads=16):
    """fp16 [B, count, Hkv, d] rows of every sequence, generated in parallel."""
    import numpy as np
    from concurrent.futures import ThreadPoolExecutor

    import synth
    with ThreadPoolExecutor(threads) as ex:
        rows = list(ex.map(lambda b: synth.batch_rows(w, tensor, b, 0, count), range(w.batch)))
    return np.stack(rows)


def cpu_baseline(w, target_seconds):
    """Time the oracle on whole (b, kv-head) streams of one decode step."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import synth
    from oracle import attention as oatt
    from oracle import codebook as ocb
    from oracle import formats as ofmt
    from oracle import prng as oprng

    d, N, G = w.head_dim, w.context, w.group
    tk, tv = ocb.tables(d, w.k_bits, w.k_kind), ocb.tables(d, w.v_bits, w.v_kind)
    sk, sv = oprng.rotation_signs(w.rot_seed_k, d), oprng.rotation_signs(w.rot_seed_v, d)
    q = synth.queries(w, step=0)
    done, elapsed = 0, 0.0
    streams = [(b, h) for b in range(w.batch) for h in range(w.n_kv_heads)]
    for b, h in streams:
        # cache bytes the oracle writes itself (setup, not timed)
        kb = ofmt.encode_rotated(synth.stream(w, synth.K_TENSOR, b, h, 0, N - 1), ofmt.PQ4, tk, sk).blocks
        vb = ofmt.encode_rotated(synth.stream(w, synth.V_TENSOR, b, h, 0, N - 1), ofmt.PQ4, tv, sv).blocks
        t0 = time.perf_counter()
        kn = ofmt.encode_rotated(synth.appended(w, synth.K_TENSOR, b, h, 0)[None], ofmt.PQ4, tk, sk).blocks
        vn = ofmt.encode_rotated(synth.appended(w, synth.V_TENSOR, b, h, 0)[None], ofmt.PQ4, tv, sv).blocks
        kdq = ofmt.dequant(np.concatenate([kb, kn]), ofmt.PQ4, d, tk, sk)
        vdq = ofmt.dequant(np.concatenate([vb, vn]), ofmt.PQ4, d, tv, sv)
        for g in range(h * G, (h + 1) * G):
            oatt.softmax_attention(q[b, g], kdq, vdq)
        elapsed += time.perf_counter() - t0
        done += 1
        if elapsed >= target_seconds:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": done * N / elapsed,
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{done} of {len(streams)} (sequence, KV head) streams of one decode step: encode the appended "
                   f"K/V token, dequantize {N} K and V blocks, softmax attention for {G} query heads; "
                   f"{elapsed:.1f} s of float64 NumPy; host cpu_count {os.cpu_count()}, affinity "
                   f"{len(os.sched_getaffinity(0))}, BLAS threads {threads}"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="c4")
    ap.add_argument("--split-tokens", type=int, default=0)
    ap.add_argument("--copies", type=int, default=2, help="cache copies rotated between steps")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--hybrid", action="store_true",
                    help="measure the capture-ring mode instead: exact ring + batched flush + hybrid read")
    ap.add_argument("--sweep", action="store_true",
                    help="kernel times of the other workloads at full size (c5 bulk prefill, c1/c2/c3/c5 decode), "
                         "one JSON line each; not the headline line")
    ap.add_argument("--one-launch", action="store_true",
                    help="time the one-launch step (the decode kernel merges the splits; no combine launch)")
    ap.add_argument("--ring-cap", type=int, default=128)
    ap.add_argument("--flush", type=int, default=64)
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the decode path runs on a single MI355X and the library has no "
              "multi-GPU path; rerun with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import compressed_domain_attention_kv_amd as tq
    import synth

    if args.workload != "c4":
        raise SystemExit("the bench line is the c4 decode workload; other workloads are parity tests")
    if args.hybrid:
        return bench_hybrid(args)
    if args.sweep:
        return bench_sweep(args)
    w = synth.C4
    B, Hq, Hkv, d, cap, N = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.capacity, w.context
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    L = tq.Layout(B, Hq, Hkv, d, cap, tq.FMT_PQ4, tq.FMT_PQ4)
    cbk, _ = tq.build_codebook(d, w.k_bits, w.k_kind, w.rot_seed_k, w.qjl_seed)
    cbv, _ = tq.build_codebook(d, w.v_bits, w.v_kind, w.rot_seed_v, w.qjl_seed + 1)

    # ---- prefill: 65,535 tokens of every sequence, written by the HIP encoder
    kbytes, vbytes = tq.cache_bytes(L)
    caches = [(torch.empty(kbytes, dtype=torch.uint8, device=dev), torch.empty(vbytes, dtype=torch.uint8, device=dev))
              for _ in range(args.copies)]
    t0 = time.time()
    k_rows = gen_rows(w, synth.K_TENSOR, w.prefill)
    v_rows = gen_rows(w, synth.V_TENSOR, w.prefill)
    _log(f"generated {2 * k_rows.nbytes / 2**30:.2f} GiB of fp16 rows in {time.time() - t0:.1f}s")
    kc, vc = caches[0]
    for b in range(B):
        dst = torch.arange(b * cap, b * cap + w.prefill, dtype=torch.int32, device=dev)
        tq.quantize_append(L, cbk, cbv, None, torch.from_numpy(k_rows[b]).to(dev), torch.from_numpy(v_rows[b]).to(dev),
                           dst, kc, vc)
    del k_rows, v_rows
    torch.cuda.synchronize()
    for kc, vc in caches[1:]:
        kc.copy_(caches[0][0])
        vc.copy_(caches[0][1])
    torch.cuda.synchronize()
    _log(f"prefill {B}x{Hkv} streams x {w.prefill} tokens in {time.time() - t0:.1f}s")

    # ---- per-step inputs, resident before timing
    total = args.warmup + args.steps
    kn = np.stack([np.stack([np.stack([synth.appended(w, synth.K_TENSOR, b, h, s) for h in range(Hkv)])
                             for b in range(B)]) for s in range(total)])
    vn = np.stack([np.stack([np.stack([synth.appended(w, synth.V_TENSOR, b, h, s) for h in range(Hkv)])
                             for b in range(B)]) for s in range(total)])
    k_new = torch.from_numpy(kn).to(dev)  # [steps, B, Hkv, d]: token t = sequence b
    v_new = torch.from_numpy(vn).to(dev)
    qs = torch.from_numpy(np.stack([synth.queries(w, step=s) for s in range(total)])).to(dev)
    new_pos = torch.full((B,), N - 1, dtype=torch.int32, device=dev)  # the appended token of each sequence
    seq_lens = torch.full((B,), N, dtype=torch.int32, device=dev)
    q_rot = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)  # scratch; the c4 kernel rotates in place
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws = tq.decode_workspace(L, args.split_tokens)
    splits = tq.decode_splits(L, args.split_tokens)

    # The decode kernel (tq_decode_step) appends the step's token and rotates the query in its
    # prologue; the combine follows (or, with --one-launch, the kernel merges the splits itself).
    # On every EVERY-th timed step the runtime records two events on the decode kernel's own
    # dispatch, so their interval is that kernel alone.
    EVERY = 8
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(total)]
    for e in ev:  # create the HIP events now (torch creates them on first record)
        e[0].record()
        e[1].record()
    torch.cuda.synchronize()

    def step(s):
        kc, vc = caches[s % args.copies]
        evs = (ev[s][0].cuda_event, ev[s][1].cuda_event) if s % EVERY == 0 else None
        if args.one_launch:
            tq.decode_step(L, cbk, cbv, k_new[s], v_new[s], new_pos, qs[s], q_rot, kc, vc, seq_lens, ws, out=out,
                           split_tokens=args.split_tokens, events=evs)
        else:
            tq.decode_step(L, cbk, cbv, k_new[s], v_new[s], new_pos, qs[s], q_rot, kc, vc, seq_lens, ws,
                           split_tokens=args.split_tokens, events=evs)
            tq.decode_combine(L, cbv, ws, out, split_tokens=args.split_tokens)

    for s in range(args.warmup):
        step(s)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.warmup, total):
        step(s)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start

    timed_steps = [s for s in range(args.warmup, total) if s % EVERY == 0]
    kern = np.array([ev[s][0].elapsed_time(ev[s][1]) for s in timed_steps])
    kernel_ms = float(np.mean(kern))
    ms_step = t_total / args.steps * 1e3
    alg_bytes = B * Hkv * N * (tq.vector_bytes(tq.FMT_PQ4, d) * 2)
    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9

    if args.copy_calibration:
        src = torch.ones(1 << 28, dtype=torch.float32, device=dev)  # 1 GiB
        dstc = torch.empty_like(src)
        for _ in range(3):
            torch.mul(src, 1.0, out=dstc)
        torch.cuda.synchronize()
        _log("copy calibration: 3 x torch.mul over 1 GiB in, 1 GiB out")

    cpu = None
    if not args.no_cpu:
        _log("timing the CPU oracle")
        cpu = cpu_baseline(w, args.cpu_seconds)

    res = {
        "metric": "compressed-KV decode-attention tokens/s; achieved HBM GB/s as % of peak",
        "value": B * N / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16x2",
        "data": "synthetic",
        "config": {
            "workload": "c4: batch 8, 32 query / 8 KV heads, d 128, context 65536 (65535 prefilled + 1 appended "
                        "per step), PQ4 4-bit K and V (68-byte blocks), seeded Gaussian K/V with 1% outlier channels",
            "global_batch": B,
            "seq_len": N,
            "parallelism": "single GPU; split-K over context",
            "splits": splits,
            "cache_copies": args.copies,
        },
        "step_breakdown_ms": {"decode_kernel": kernel_ms, "decode_kernel_median": float(np.median(kern)),
                              "rest_of_step": ms_step - kernel_ms},
        "step_breakdown_note": (f"decode_kernel: token append and query rotation in its prologue, then the "
                                f"partial{' and the merge of the splits' if args.one_launch else ''}; HIP events on "
                                f"the kernel's own dispatch on {len(timed_steps)} of the {args.steps} timed steps "
                                f"(every {EVERY}th); rest_of_step: host-clock step time minus that kernel "
                                f"({'launch gaps' if args.one_launch else 'the combine and the launch gaps'})"),
        "decode_attention_gbs": alg_bytes / (ms_step * 1e-3) / 1e9,
        "decode_attention_gbs_note": "algorithmic K+V bytes over the whole host-clock step",
        "roofline": {
            "kernel": "decode_partial_sparse_kernel<4, false>" + (" (with the merge)" if args.one_launch else ""),
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(),
            "algorithmic_bytes_per_launch": alg_bytes,
        },
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def bench_hybrid(args):
    """c4 shapes in the capture-ring mode: each step appends one exact fp16 token per
    sequence and KV head to the ring, flushes the oldest `flush` ring tokens into the
    compressed cache whenever a ring is full, rotates the queries and runs the hybrid read
    over the compressed tokens and the ring.  Contexts start at 65,536 (65,472 compressed +
    64 in the ring) and grow by one token per step; the cache has room for the growth."""
    import numpy as np
    import torch

    import compressed_domain_attention_kv_amd as tq
    import synth

    w = synth.C4
    B, Hq, Hkv, d, N = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.context
    R, F = args.ring_cap, args.flush
    total = args.warmup + args.steps
    cap = N + ((total + 255) // 256) * 256
    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    L = tq.Layout(B, Hq, Hkv, d, cap, tq.FMT_PQ4, tq.FMT_PQ4)
    cbk, _ = tq.build_codebook(d, w.k_bits, w.k_kind, w.rot_seed_k, w.qjl_seed)
    cbv, _ = tq.build_codebook(d, w.v_bits, w.v_kind, w.rot_seed_v, w.qjl_seed + 1)
    comp0, ring0 = N - 64, 64
    kbytes, vbytes = tq.cache_bytes(L)
    kc = torch.empty(kbytes, dtype=torch.uint8, device=dev)
    vc = torch.empty(vbytes, dtype=torch.uint8, device=dev)
    t0 = time.time()
    k_rows = gen_rows(w, synth.K_TENSOR, comp0)
    v_rows = gen_rows(w, synth.V_TENSOR, comp0)
    for b in range(B):
        dst = torch.arange(b * cap, b * cap + comp0, dtype=torch.int32, device=dev)
        tq.quantize_append(L, cbk, cbv, None, torch.from_numpy(k_rows[b]).to(dev), torch.from_numpy(v_rows[b]).to(dev),
                           dst, kc, vc)
    del k_rows, v_rows
    kr = torch.empty(tq.ring_bytes(L, R) // 2, dtype=torch.float16, device=dev)
    vr = torch.empty_like(kr)
    # the ring's first tokens and the per-step new tokens, resident before timing
    pre_k = torch.from_numpy(np.stack([synth.batch_rows(w, synth.K_TENSOR, b, comp0, ring0) for b in range(B)])).to(dev)
    pre_v = torch.from_numpy(np.stack([synth.batch_rows(w, synth.V_TENSOR, b, comp0, ring0) for b in range(B)])).to(dev)
    for i in range(ring0):
        pos = torch.full((B,), comp0 + i, dtype=torch.int32, device=dev)
        tq.ring_append(L, R, pre_k[:, i].contiguous(), pre_v[:, i].contiguous(), pos, kr, vr)
    kn = torch.from_numpy(np.stack([np.stack([np.stack([synth.appended(w, synth.K_TENSOR, b, h, s) for h in range(Hkv)])
                                              for b in range(B)]) for s in range(total)])).to(dev)
    vn = torch.from_numpy(np.stack([np.stack([np.stack([synth.appended(w, synth.V_TENSOR, b, h, s) for h in range(Hkv)])
                                              for b in range(B)]) for s in range(total)])).to(dev)
    qs = torch.from_numpy(np.stack([synth.queries(w, step=s) for s in range(total)])).to(dev)
    torch.cuda.synchronize()
    _log(f"hybrid prefill: {B}x{Hkv} streams, {comp0} compressed + {ring0} ring tokens, {time.time() - t0:.1f}s")

    # host-side schedule of lengths (every sequence advances together), device copies per step
    comp, n = comp0, ring0
    sched = []
    for s in range(total):
        pos = comp + n
        n += 1
        flush = n == R
        sched.append((pos, flush, comp))
        if flush:
            comp += F
            n -= F
        sched[-1] = sched[-1] + (comp, n)
    pos_t = torch.tensor([[x[0]] * B for x in sched], dtype=torch.int32, device=dev)
    first_t = torch.tensor([[x[2]] * B for x in sched], dtype=torch.int32, device=dev)
    comp_t = torch.tensor([[x[3]] * B for x in sched], dtype=torch.int32, device=dev)
    ring_t = torch.tensor([[x[4]] * B for x in sched], dtype=torch.int32, device=dev)
    q_rot = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.decode_hybrid_workspace_bytes(L, args.split_tokens), dtype=torch.uint8, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(total)]
    # the breakdown comes from every 8th timed step (events between the calls), as in the
    # headline line: no warm-up or first-launch step enters it
    probe = [s for s in range(args.warmup, total) if (s - args.warmup) % 8 == 0]
    probe_set = set(probe)

    def step(s, marks):
        e = ev[s]
        if marks:
            e[0].record()
        tq.ring_append(L, R, kn[s], vn[s], pos_t[s], kr, vr)
        if marks:
            e[1].record()
        if sched[s][1]:
            tq.ring_flush(L, cbk, cbv, None, R, kr, vr, first_t[s], F, kc, vc)
        if marks:
            e[2].record()
        tq.rotate_sketch_query(L, cbk, None, qs[s], q_rot, None)
        if marks:
            e[3].record()
        tq.decode_attention_hybrid(L, cbk, cbv, q_rot, None, kc, vc, comp_t[s], R, kr, vr, ring_t[s], out, ws,
                                   split_tokens=args.split_tokens)
        if marks:
            e[4].record()

    for s in range(args.warmup):
        step(s, False)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for s in range(args.warmup, total):
        step(s, s in probe_set)
    torch.cuda.synchronize()
    t_total = time.perf_counter() - t_start
    ms_step = t_total / args.steps * 1e3
    attended = float(np.mean([sched[s][3] + sched[s][4] for s in range(args.warmup, total)]))

    def mean_ms(i, j, steps):
        return float(np.mean([ev[s][i].elapsed_time(ev[s][j]) for s in steps])) if len(steps) else None

    flush_steps = [s for s in probe if sched[s][1]]
    res = {
        "metric": "compressed-KV decode-attention tokens/s; achieved HBM GB/s as % of peak",
        "mode": "hybrid (capture ring of exact recent tokens + compressed history)",
        "value": B * attended / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16x2",
        "data": "synthetic",
        "config": {"workload": f"c4 shapes in ring mode: ring of {R} exact fp16 tokens per stream, flush of {F} "
                               "when full, contexts from 65,536 growing by one per step",
                   "global_batch": B, "mean_context": attended, "ring_cap": R, "flush": F,
                   "flushes_in_timed_steps": sum(1 for s in range(args.warmup, total) if sched[s][1])},
        "step_breakdown_ms": {"ring_append": mean_ms(0, 1, probe), "rotate_query": mean_ms(2, 3, probe),
                              "decode_attention_hybrid": mean_ms(3, 4, probe),
                              "ring_flush_when_it_runs": mean_ms(1, 2, flush_steps)},
        "step_breakdown_note": f"{len(probe)} sampled timed steps (every 8th), events between the calls",
        "roofline": None,
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


SWEEP_NOTE = ("per-kernel times of a workload other than the headline one, on a cold cache: before every timed "
              "call a 512 MiB buffer is overwritten (twice the 256 MB Infinity Cache), so the call reads its bytes "
              "from HBM; decode_partial from HIP events on its own dispatch, median over the calls; the write "
              "path from events around the call; the combine (a few microseconds on records the partial just "
              "wrote) as the mean over a replayed HIP graph of repeated calls; algorithmic bytes as in the "
              "roofline of the headline line; useful flops count the method's arithmetic only (2 G d FMA per "
              "token and KV head, plus G d for the QJL term of TQ3K keys)")


def bench_sweep(args):
    """The write path at its bulk sizes (c5 prefill: 131,072 tokens x 4 KV heads at d 256; c3
    prefill: 30,000 tokens x 8 KV heads, TQ3K keys and GQ2V values) and the
    decode of every other workload at full size -- c1, c2, c3, c5, c3's shapes with GQ4V values,
    c2's and c4's shapes with PQ3 keys (and PQ4 or PQ3 values) -- each timed alone on a cold cache,
    plus sparse V against the plain decode at c3 and c5; one JSON line per item."""
    import numpy as np
    import torch

    import compressed_domain_attention_kv_amd as tq
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda", 0)
    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def cold_ms(fn, reps, attached):
        """Median time of `reps` calls, each after the scrub.  attached: fn takes (start, stop)
        raw events recorded on the kernel's own dispatch; else events are recorded around fn."""
        times = []
        for r in range(reps + 2):
            scrub.fill_(r & 0xFF)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            if attached:
                e0.record()  # creates the HIP events before their handles are passed on
                e1.record()
                fn((e0.cuda_event, e1.cuda_event))
            else:
                e0.record()
                fn(None)
                e1.record()
            torch.cuda.synchronize()
            if r >= 2:  # two untimed calls first
                times.append(e0.elapsed_time(e1))
        return float(np.median(times))

    def per_call_ms(fn, reps):
        """Mean time per call of `reps` calls captured in one HIP graph and replayed, so the
        host's launch rate does not set the time of microsecond kernels."""
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                fn()
        g.replay()
        torch.cuda.synchronize()
        best = None
        for _ in range(3):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) / reps
            best = t if best is None else min(best, t)
        del g
        return best

    def emit(item, **kv):
        print(json.dumps({"sweep": item, "note": SWEEP_NOTE, **kv}), flush=True)

    def codebooks(w):
        tq3k = w.k_format == synth.TQ3K
        cbk, S = tq.build_codebook(w.head_dim, w.k_bits, w.k_kind, w.rot_seed_k, w.qjl_seed, want_qjl_matrix=tq3k)
        cbv, _ = tq.build_codebook(w.head_dim, w.v_bits, w.v_kind, w.rot_seed_v, w.qjl_seed + 1)
        return cbk, cbv, (torch.from_numpy(S).to(dev) if tq3k else None)

    # ---- write path: c5 bulk prefill in one call (fp16 rows in, blocks out)
    w5 = synth.C5
    T, Hp, d = w5.extra["prefill_tokens"], w5.extra["prefill_kv_heads"], w5.head_dim
    wp = synth.scaled(w5, batch=1, n_q_heads=Hp, n_kv_heads=Hp, capacity=T, context=T, prefill=T)
    cbk5, cbv5, _ = codebooks(w5)
    Lp = tq.Layout(1, Hp, Hp, d, T, w5.k_format, w5.v_format)
    kb5, vb5 = tq.cache_bytes(Lp)
    kc5 = torch.empty(kb5, dtype=torch.uint8, device=dev)
    vc5 = torch.empty(vb5, dtype=torch.uint8, device=dev)
    t0 = time.time()
    k_rows = torch.from_numpy(synth.batch_rows(wp, synth.K_TENSOR, 0, 0, T)).to(dev)
    v_rows = torch.from_numpy(synth.batch_rows(wp, synth.V_TENSOR, 0, 0, T)).to(dev)
    dst = torch.arange(T, dtype=torch.int32, device=dev)
    _log(f"sweep: c5 prefill rows generated in {time.time() - t0:.1f}s")
    ms = cold_ms(lambda ev: tq.quantize_append(Lp, cbk5, cbv5, None, k_rows, v_rows, dst, kc5, vc5), 10, False)
    nbytes = 2 * T * Hp * d * 2 + kb5 + vb5
    emit("c5 bulk prefill (write path: norm, rotate, quantize, pack K and V)", kernel="quantize_pq4_kernel<256>",
         workload=f"{T} tokens x {Hp} KV heads, d {d}, PQ4 K and V", us=ms * 1e3, bytes=nbytes,
         roofline={"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
    del k_rows, v_rows
    torch.cuda.synchronize()

    # ---- write path: c3 prefill (TQ3K keys with their QJL sketch, GQ2V values) in one call
    w3 = synth.C3
    L3 = tq.Layout(1, w3.n_q_heads, w3.n_kv_heads, w3.head_dim, w3.capacity, w3.k_format, w3.v_format)
    cbk3, cbv3, S3 = codebooks(w3)
    kb3, vb3 = tq.cache_bytes(L3)
    kc3 = torch.empty(kb3, dtype=torch.uint8, device=dev)
    vc3 = torch.empty(vb3, dtype=torch.uint8, device=dev)
    k3 = torch.from_numpy(synth.batch_rows(w3, synth.K_TENSOR, 0, 0, w3.prefill)).to(dev)
    v3 = torch.from_numpy(synth.batch_rows(w3, synth.V_TENSOR, 0, 0, w3.prefill)).to(dev)
    dst3 = torch.arange(w3.prefill, dtype=torch.int32, device=dev)
    ms = cold_ms(lambda ev: tq.quantize_append(L3, cbk3, cbv3, S3, k3, v3, dst3, kc3, vc3), 10, False)
    nbytes = 2 * w3.prefill * w3.n_kv_heads * w3.head_dim * 2 + w3.prefill * w3.n_kv_heads * (
        tq.vector_bytes(w3.k_format, w3.head_dim) + tq.vector_bytes(w3.v_format, w3.head_dim))
    emit("c3 prefill (write path: TQ3K keys with the QJL sketch, GQ2V values)",
         kernel="quantize_tq3k_mfma_kernel + quantize_kernel<GQ2V>",
         workload=f"{w3.prefill} tokens x {w3.n_kv_heads} KV heads, d {w3.head_dim}", us=ms * 1e3, bytes=nbytes,
         roofline={"bound": "hbm", "achieved": nbytes / (ms * 1e-3) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                   "frac": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS})
    del k3, v3, kc3, vc3
    torch.cuda.synchronize()

    # ---- decode of the other workloads (c5 reads the prefill bytes as [32][2][8192])
    c2_asym = synth.scaled(synth.C2, name="c2 with PQ3 keys and PQ4 values", v_format=synth.PQ4, v_bits=4)
    c3_gq4v = synth.scaled(synth.C3, name="c3 with GQ4V values", v_format=synth.GQ4V, v_bits=4)
    c4_pq3 = synth.scaled(synth.C4, name="c4 shapes with PQ3 keys and values", k_format=synth.PQ3,
                          v_format=synth.PQ3, k_bits=3, v_bits=3, prefill=synth.C4.context)
    c4_asym = synth.scaled(c4_pq3, name="c4 shapes with PQ3 keys and PQ4 values", v_format=synth.PQ4, v_bits=4)
    # eight query heads per KV head at d 128 (64 query / 8 KV heads, grouped-query models of that shape)
    c4_g8 = synth.scaled(synth.C4, name="c4 shapes with 64 query heads (G = 8)", n_q_heads=64,
                         prefill=synth.C4.context)
    for w in (synth.C1, synth.C2, c2_asym, synth.C3, c3_gq4v, synth.C5, c4_pq3, c4_asym, c4_g8):
        B, Hq, Hkv, d, N = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.context
        L = tq.Layout(B, Hq, Hkv, d, w.capacity, w.k_format, w.v_format)
        if w is synth.C5:
            cbk, cbv, S = cbk5, cbv5, None
            kc, vc = kc5, vc5
        else:
            cbk, cbv, S = codebooks(w)
            kbytes, vbytes = tq.cache_bytes(L)
            kc = torch.zeros(kbytes, dtype=torch.uint8, device=dev)
            vc = torch.zeros(vbytes, dtype=torch.uint8, device=dev)
            for b in range(B):
                krows = torch.from_numpy(synth.batch_rows(w, synth.K_TENSOR, b, 0, w.prefill)).to(dev)
                vrows = torch.from_numpy(synth.batch_rows(w, synth.V_TENSOR, b, 0, w.prefill)).to(dev)
                dst = torch.arange(b * w.capacity, b * w.capacity + w.prefill, dtype=torch.int32, device=dev)
                tq.quantize_append(L, cbk, cbv, S, krows, vrows, dst, kc, vc)
                del krows, vrows
        q = torch.from_numpy(synth.queries(w)).to(dev)
        q_rot = torch.empty_like(q)
        q_sk = torch.empty_like(q) if S is not None else None
        out = torch.empty_like(q)
        seq = torch.full((B,), N, dtype=torch.int32, device=dev)
        ws = torch.empty(tq.decode_workspace_bytes(L), dtype=torch.uint8, device=dev)
        reps = 30
        rot_ms = per_call_ms(lambda: tq.rotate_sketch_query(L, cbk, S, q, q_rot, q_sk), 100)
        part_ms = cold_ms(lambda ev: tq.decode_partial(L, cbk, cbv, q_rot, q_sk, kc, vc, seq, ws, events=ev), reps,
                          True)
        comb_ms = per_call_ms(lambda: tq.decode_combine(L, cbv, ws, out), 100)
        alg = B * Hkv * N * (tq.vector_bytes(w.k_format, d) + tq.vector_bytes(w.v_format, d))
        fma = B * Hkv * N * w.group * d * (3 if w.k_format == synth.TQ3K else 2)
        gbs = alg / (part_ms * 1e-3) / 1e9
        emit(f"{w.name} decode", kernel="decode_partial + decode_combine",
             workload=f"batch {B}, {Hq} query / {Hkv} KV heads, d {d}, context {N}, formats K {w.k_format} V "
                      f"{w.v_format} (1 PQ4, 2 PQ3, 3 TQ3K, 4 GQ2V, 5 GQ4V)",
             splits=tq.decode_splits(L), us={"rotate_query": rot_ms * 1e3, "decode_partial": part_ms * 1e3,
                                             "decode_combine": comb_ms * 1e3},
             bytes=alg, useful_tflops=2 * fma / (part_ms * 1e-3) / 1e12,
             roofline={"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                       "frac": gbs / HBM_PEAK_GBS})
        if w is synth.C3 or w is synth.C5:
            # sparse V against the plain call on the same cache, with queries four times as sharp
            # (logit spread about 8): most tokens then sit far below their wavefront's running
            # maximum, the case the threshold is for (warm: a replayed graph of each call)
            qs = q * 4.0
            qs_rot = torch.empty_like(qs)
            qs_sk = torch.empty_like(qs) if S is not None else None
            tq.rotate_sketch_query(L, cbk, S, qs, qs_rot, qs_sk)
            tau = 1e-3
            plain_ms = per_call_ms(lambda: tq.decode_partial(L, cbk, cbv, qs_rot, qs_sk, kc, vc, seq, ws), 50)
            sv_ms = per_call_ms(lambda: tq.decode_partial_sparse_v(L, cbk, cbv, qs_rot, qs_sk, kc, vc, seq, ws, tau),
                                50)
            emit(f"{w.name} decode, sparse V", kernel="decode_partial vs decode_partial_sparse_v",
                 workload=f"as the {w.name} decode line, queries scaled by 4; warm (replayed graph)", threshold=tau,
                 us={"decode_partial": plain_ms * 1e3, "decode_partial_sparse_v": sv_ms * 1e3},
                 speedup=plain_ms / sv_ms)
        del kc, vc
        torch.cuda.synchronize()


if __name__ == "__main__":
    main()
