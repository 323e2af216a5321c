"""Benchmark: RHT 4-bit quantize + dequantize of a KV-cache block on one MI355X.

Workload: K and V, each 32 layers x 8 KV heads x 32768 tokens x d = 128 fp16
(n = 8,388,608 vectors each; N(0,1) with one seeded outlier channel x20 and
per-vector log-normal(0, 0.5) norms), randomized Hadamard transform + 4-bit
N(0,1) Lloyd-Max codes + one fp32 norm per vector, then decode back to fp16.
One step = quantize K, quantize V, dequantize K, dequantize V; inputs are
resident in HBM before timing starts.

Prints one JSON line.  `value` is vectors per second through the whole step
(every vector is encoded and decoded once per step).  `roofline` is for the
slower of the two kernels, from HIP events on the stream the kernels run on;
algorithmic bytes are 256 B in + 64 B codes + 4 B norm per vector for the
encoder and the same 324 B for the decoder.  `shape_ceiling` times trivial
streaming kernels with each direction's exact traffic (the achievable
ceiling of these shapes); the two 4-bit scoring rows carry the same for
their own traffic (`other_workloads.score.shape_ceiling`,
`other_workloads.score_large.shape_ceiling`).  `cpu_baseline` times the oracle on every host
thread over the whole K tensor (and on one thread over a bounded sample).
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BYTES_PER_VECTOR = 128 * 2 + 64 + 4  # fp16 row + 4-bit codes + fp32 norm
COPY_BYTES = 8388608 * BYTES_PER_VECTOR // 2  # plain copy moving one launch's bytes


def source_digest():
    h = hashlib.sha256()
    # the sources the timed d = 128 kernels are compiled from
    for f in ("rht_kv128.hip", "rht_device.h"):
        with open(os.path.join(ROOT, "rotation_vector_quantization_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel):
    """HBM bytes per launch from committed rocprofv3 PMC summaries, only if
    they were taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic_c2_kv.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes_per_launch")


def traffic_from(fetch_dir, write_dir):
    """Build profiles/traffic_c2_kv.json from two rocprofv3 --pmc runs of this
    script (FETCH_SIZE, then WRITE_SIZE; csv output).  Counters are KiB per
    dispatch; each is scaled by the factor that maps the plain copy kernel's
    reading to its known byte count (COPY_BYTES read and written)."""
    import csv
    import glob

    def per_kernel(d, counter):
        vals = {}
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for row in csv.DictReader(fh):
                    if row.get("Counter_Name") != counter:
                        continue
                    name = row.get("Kernel_Name", "")
                    vals.setdefault(name, []).append(float(row["Counter_Value"]))
        return vals

    fetch, write = per_kernel(fetch_dir, "FETCH_SIZE"), per_kernel(write_dir, "WRITE_SIZE")

    def pick(vals, key):
        hits = [v for k, v in vals.items() if key in k]
        if not hits:
            raise SystemExit("no %s dispatches in the counter files" % key)
        allv = [x for h in hits for x in h]
        return sum(allv) / len(allv)

    def pick_copy(vals):
        # torch's copy_ between contiguous device tensors runs __amd_rocclr_copyBuffer; the
        # copy of known size is the largest of them (host -> device uploads use it too)
        allv = [x for k, v in vals.items() if "copyBuffer" in k for x in v]
        if not allv:
            raise SystemExit("no copyBuffer dispatches in the counter files")
        big = [x for x in allv if x > 0.9 * max(allv)]
        return sum(big) / len(big)

    f_copy, w_copy = pick_copy(fetch) * 1024, pick_copy(write) * 1024
    kf, kw = COPY_BYTES / f_copy, COPY_BYTES / w_copy
    rec = {"source_digest": source_digest(), "copy_bytes_each_way": COPY_BYTES,
           "fetch_scale": kf, "write_scale": kw, "kernels": {}}
    for key in ("k_quantize", "k_dequantize"):
        fb, wb = pick(fetch, key) * 1024 * kf, pick(write, key) * 1024 * kw
        rec["kernels"][key] = {"fetch_bytes": fb, "write_bytes": wb, "hbm_bytes_per_launch": fb + wb,
                               "algorithmic_bytes_per_launch": 8388608 * BYTES_PER_VECTOR}
    out = os.path.join(ROOT, "profiles", "traffic_c2_kv.json")
    with open(out, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec, indent=1))


def time_launches(torch, stream, fn, sets, iters=20, warm_ms=100.0):
    """Per-launch times (ms) of fn(set_index), cycling through `sets` buffer
    sets, from HIP events recorded on `stream` between launches.  The kernel
    first runs untimed for at least warm_ms of GPU time, so clocks that dropped
    during host-side set-up have ramped up again.  Kernels shorter than 0.1 ms
    are timed in groups of 8 launches per event interval (each value is the
    group's mean): with an event after every launch the host's submission
    rate, not the GPU, would set the interval.

    The first launch of a kernel also loads its code object, so it is left out
    of the launch-time estimate, and the warm-up is measured rather than
    counted: batches of launches run until their event-timed total reaches
    warm_ms.  A heavy kernel's time drifts for tens of milliseconds after it
    starts (the clock settles under the new load), so a warm-up sized from a
    slow first launch would leave the timed launches inside that drift."""
    fn(0)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(3):
        fn(i % sets)
    e1.record(stream)
    torch.cuda.synchronize()
    est = max(e0.elapsed_time(e1) / 3, 1e-3)
    batch = max(1, min(int(5.0 / est), 1000))  # about 5 ms of launches per batch
    warmed, k = 0.0, 0
    while warmed < warm_ms and k < 20000:
        e0.record(stream)
        for _ in range(batch):
            fn(k % sets)
            k += 1
        e1.record(stream)
        torch.cuda.synchronize()
        warmed += e0.elapsed_time(e1)
    group = 8 if est < 0.1 else 1
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    k = 0
    for i in range(iters):
        for _ in range(group):
            fn(k % sets)
            k += 1
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([ev[i].elapsed_time(ev[i + 1]) / group for i in range(iters)])


def stats(ms):
    """mean / median / min / max of per-launch times in ms."""
    return {"ms_per_launch": float(np.mean(ms)), "ms_median": float(np.median(ms)),
            "ms_min": float(np.min(ms)), "ms_max": float(np.max(ms))}


def other_workloads(torch, rht, dev, stream, with_ceiling=True):
    """The other hot-path rows, each at its full workload size: DRIVE 1-bit
    (65536 x 1024 fp32, both scales), the residual chain (2^20 x 256 fp16,
    2+1 bits) and rotated-domain scoring (131072 4-bit keys x 64 queries).
    Working sets under 512 MB are rotated over several buffer sets so the
    256 MB Infinity Cache cannot serve repeats."""
    import testdata

    sh = stream.cuda_stream
    out = {}

    def hbm(name, units, unit, bytes_per_unit, times):
        st = stats(times)
        ms = st["ms_median"]
        gbs = units * bytes_per_unit / (ms / 1e3) / 1e9
        return dict(st, **{unit + "_per_s": units / (ms / 1e3), "bytes_per_" + unit: bytes_per_unit,
                           "GB_per_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS, "bound": "hbm"})

    # DRIVE, C3: two input sets (2 x 256 MiB)
    w3 = testdata.WORKLOADS["c3"]
    xs = [torch.from_numpy(testdata.generate(w3)).to(dev)]
    xs.append(torch.roll(xs[0], 1, 0))
    n3, d3 = w3.n, w3.d
    b3 = [torch.empty((n3, d3 // 8), dtype=torch.uint8, device=dev) for _ in range(2)]
    s3 = [torch.empty((n3,), dtype=torch.float32, device=dev) for _ in range(2)]
    y3 = [torch.empty((n3, d3), dtype=torch.float32, device=dev) for _ in range(2)]
    per3 = d3 * 4 + d3 // 8 + 4
    for mode, tag in ((rht.SCALE_SIGN_BIASED, "biased"), (rht.SCALE_SIGN_UNBIASED, "unbiased")):
        qms = time_launches(torch, stream, lambda i: rht.rht_quantize(
            xs[i].data_ptr(), rht.F32, n3, d3, 1, mode, w3.rot_seed, b3[i].data_ptr(), s3[i].data_ptr(), sh), 2)
        dms = time_launches(torch, stream, lambda i: rht.rht_dequantize(
            b3[i].data_ptr(), s3[i].data_ptr(), n3, d3, 1, mode, w3.rot_seed, y3[i].data_ptr(), rht.F32, sh), 2)
        out["drive_" + tag] = {"workload": "65536 x 1024 fp32 Student-t, 1-bit signs + S, decode to fp32",
                               "quantize": hbm("q", n3, "chunk", per3, qms),
                               "dequantize": hbm("d", n3, "chunk", per3, dms)}
    del xs, b3, s3, y3

    # residual chain, C4: 512 MiB input, one set suffices
    w4 = testdata.WORKLOADS["c4"]
    x4 = torch.from_numpy(testdata.generate(w4)).to(dev)
    n4, d4, bt = w4.n, w4.d, w4.bits
    c4 = torch.empty((n4, (bt - 1) * d4 // 8), dtype=torch.uint8, device=dev)
    g4 = torch.empty((n4, d4 // 8), dtype=torch.uint8, device=dev)
    nr4 = torch.empty((n4,), dtype=torch.float32, device=dev)
    r4 = torch.empty_like(nr4)
    y4 = torch.empty((n4, d4), dtype=torch.float16, device=dev)
    per4 = d4 * 2 + (bt - 1) * d4 // 8 + d4 // 8 + 8
    qms = time_launches(torch, stream, lambda i: rht.rht_residual_quantize(
        x4.data_ptr(), rht.F16, n4, d4, bt, w4.rot_seed, c4.data_ptr(), g4.data_ptr(), nr4.data_ptr(),
        r4.data_ptr(), sh), 1)
    dms = time_launches(torch, stream, lambda i: rht.rht_residual_dequantize(
        c4.data_ptr(), g4.data_ptr(), nr4.data_ptr(), r4.data_ptr(), n4, d4, bt, w4.rot_seed, y4.data_ptr(),
        rht.F16, sh), 1)
    out["residual"] = {"workload": "16 x 65536 x 256 fp16, 5 outlier channels x30, 2-bit + 1-bit residual sign",
                       "quantize": hbm("q", n4, "vector", per4, qms), "dequantize": hbm("d", n4, "vector", per4, dms)}
    del x4, c4, g4, nr4, r4, y4

    # scoring, C5: 16 key/logit sets (16 x 42.5 MB) rotated
    wk, wq = testdata.WORKLOADS["c5k"], testdata.WORKLOADS["c5q"]
    keys = torch.from_numpy(testdata.generate(wk)).to(dev)
    q = torch.from_numpy(testdata.generate(wq)).to(dev)
    nk, d5, b5, m = wk.n, wk.d, wk.bits, wq.n
    c5, n5 = rht.quantize(keys, b5, wk.rot_seed)
    sets = 16
    cs = [c5.clone() for _ in range(sets)]
    ns = [n5.clone() for _ in range(sets)]
    ls = [torch.empty((m, nk), dtype=torch.float32, device=dev) for _ in range(sets)]
    sms = time_launches(torch, stream, lambda i: rht.rht_score(
        q.data_ptr(), m, cs[i].data_ptr(), ns[i].data_ptr(), nk, d5, b5, wk.rot_seed, ls[i].data_ptr(), sh), sets)
    flops = 2.0 * m * nk * d5
    sbytes = nk * (d5 * b5 // 8 + 4) + m * d5 * 4 + m * nk * 4
    st = stats(sms)
    sms = st["ms_median"]
    tfs = flops / (sms / 1e3) / 1e12
    # the contraction runs on fp16 matrix cores (hi/lo operand splits, 3 products per
    # 16 coordinates), far from their peak; the logits and codes in HBM bound it
    gbs = sbytes / (sms / 1e3) / 1e9
    out["score"] = dict(st, **{"workload": "131072 keys d=128 4-bit codes + norms, 64 fp32 queries, fp32 logits",
                               "keys_per_s": nk / (sms / 1e3), "TFLOP_per_s": tfs,
                               "algorithmic_bytes": sbytes, "GB_per_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
                               "bound": "hbm"})
    if with_ceiling:
        out["score"]["shape_ceiling"] = score_ceiling(torch, stream, cs, ns, ls, nk, m)
    del cs, ns, ls

    # the same keys as 1-bit sign codes (unbiased scale) and as a 2+1-bit residual chain
    bsg, ssg = rht.quantize(keys, 1, wk.rot_seed, mode=rht.SCALE_SIGN_UNBIASED)
    rc, rg, rn, rr = rht.residual_quantize(keys, 3, wk.rot_seed)
    sets_b = [(bsg.clone(), ssg.clone()) for _ in range(sets)]
    sets_r = [(rc.clone(), rg.clone(), rn.clone(), rr.clone()) for _ in range(sets)]
    ls = [torch.empty((m, nk), dtype=torch.float32, device=dev) for _ in range(sets)]
    for name, fn, key_bytes in (
            ("score_sign", lambda i: rht.rht_score_sign(q.data_ptr(), m, sets_b[i][0].data_ptr(),
                                                        sets_b[i][1].data_ptr(), nk, d5, wk.rot_seed,
                                                        ls[i].data_ptr(), sh), d5 // 8 + 4),
            ("score_residual", lambda i: rht.rht_residual_score(
                q.data_ptr(), m, sets_r[i][0].data_ptr(), sets_r[i][1].data_ptr(), sets_r[i][2].data_ptr(),
                sets_r[i][3].data_ptr(), nk, d5, 3, wk.rot_seed, ls[i].data_ptr(), sh), 3 * d5 // 8 + 8)):
        st = stats(time_launches(torch, stream, fn, sets))
        ms = st["ms_median"]
        tfs = flops / (ms / 1e3) / 1e12
        alg = nk * key_bytes + m * d5 * 4 + m * nk * 4
        gbs = alg / (ms / 1e3) / 1e9
        out[name] = dict(st, **{"workload": "131072 keys d=128 %s, 64 fp32 queries, fp32 logits" % (
                                    "1-bit sign codes + S" if name == "score_sign" else "2-bit codes + sign plane + 2 scales"),
                                "keys_per_s": nk / (ms / 1e3), "TFLOP_per_s": tfs,
                                "algorithmic_bytes": alg, "GB_per_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
                                "bound": "hbm"})
    del sets_b, sets_r, ls, bsg, ssg, rc, rg, rn, rr

    # MSE scoring at 2^21 keys (673 MB per launch): at 131072 keys a launch
    # takes 15-17 us and its fixed part (the launch and each block's query
    # rotation) is a large share.  The keys are the 131072 encoded ones, 16 times.
    nl = nk * 16
    cl, nlr = c5.repeat(16, 1), n5.repeat(16)
    ll = torch.empty((m, nl), dtype=torch.float32, device=dev)
    st = stats(time_launches(torch, stream, lambda i: rht.rht_score(
        q.data_ptr(), m, cl.data_ptr(), nlr.data_ptr(), nl, d5, b5, wk.rot_seed, ll.data_ptr(), sh), 1))
    ms = st["ms_median"]
    alg = nl * (d5 * b5 // 8 + 4) + m * d5 * 4 + m * nl * 4
    gbs = alg / (ms / 1e3) / 1e9
    out["score_large"] = dict(st, **{"workload": "2097152 keys d=128 4-bit codes + norms, 64 fp32 queries, fp32 logits",
                                     "keys_per_s": nl / (ms / 1e3), "TFLOP_per_s": 2.0 * m * nl * d5 / (ms / 1e3) / 1e12,
                                     "algorithmic_bytes": alg, "GB_per_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
                                     "bound": "hbm"})
    if with_ceiling:
        out["score_large"]["shape_ceiling"] = score_ceiling(torch, stream, [cl], [nlr], [ll], nl, m)
    del cl, nlr, ll
    return out


def attention_workload(torch, rht, dev, stream, ck, nk, cv, nv, n_vec, d, k_bits=4, v_bits=4):
    """Decode attention over the KV block just encoded: 32 layers x 8 KV heads
    = 256 heads of 32768 tokens, 4 queries per KV head (grouped-query), scale
    1/sqrt(d), logits and value sums in the rotated domains (rht_attention);
    k_bits / v_bits are the widths of the key and value codes."""
    heads, m = 256, 4
    n = n_vec // heads
    g = torch.Generator(device=dev)
    g.manual_seed(1010)
    q = torch.randn((heads, m, d), generator=g, device=dev, dtype=torch.float32)
    out = torch.empty((heads, m, d), dtype=torch.float32, device=dev)
    need = rht.rht_attention_workspace_bytes(heads, m, n, d)
    ws = torch.empty((need,), dtype=torch.uint8, device=dev)
    sh = stream.cuda_stream
    scale = 1.0 / math.sqrt(d)
    times = time_launches(torch, stream, lambda i: rht.rht_attention(
        q.data_ptr(), m, ck.data_ptr(), nk.data_ptr(), cv.data_ptr(), nv.data_ptr(), heads, n, d, k_bits,
        v_bits, 42, 43, scale, out.data_ptr(), ws.data_ptr(), need, sh), 1)
    st = stats(times)
    ms = st["ms_median"]
    # codes and norms of K and V, the queries and the outputs
    alg = n_vec * (d * k_bits // 8 + 4 + d * v_bits // 8 + 4) + 2 * heads * m * d * 4
    gbs = alg / (ms / 1e3) / 1e9
    flops = 2.0 * 2 * heads * m * n * d  # logits and value sums, counted once
    return dict(st, **{"workload": "decode attention over the KV block: 256 heads x 32768 tokens, "
                                   "%d-bit K and %d-bit V, 4 queries per head, d=128" % (k_bits, v_bits),
                       "algorithmic_bytes": alg, "GB_per_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
                       "bound": "hbm", "tokens_per_s": heads * n / (ms / 1e3),
                       "algorithmic_TFLOP_per_s": flops / (ms / 1e3) / 1e12,
                       "workspace_bytes": need})


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads():
    """Worker threads for the all-cores oracle leg: the CPUs this process may
    run on, at most 16 (one GPU's share of a GPU host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(x_host, rows_single):
    """The oracle (plain fp64 C, unchanged) on the K tensor of the KV block:
    quantize + dequantize to fp16.  One thread on the first `rows_single`
    rows, then every host thread on the whole tensor, the rows split into
    equal contiguous shards (each vector is independent; the ctypes calls
    release the GIL, so the shards run in parallel)."""
    import concurrent.futures

    import oracle
    import testdata

    w = testdata.WORKLOADS["c2k"]

    def run(lo, hi):
        codes, norms = oracle.quantize(x_host[lo:hi], w.bits, w.rot_seed)
        oracle.dequantize(codes, norms, w.d, w.bits, w.rot_seed, np.float16)

    t0 = time.perf_counter()
    run(0, rows_single)
    dt1 = time.perf_counter() - t0
    threads = host_threads()
    rows = x_host.shape[0]
    edges = np.linspace(0, rows, 4 * threads + 1).astype(np.int64)
    t0 = time.perf_counter()
    with concurrent.futures.ThreadPoolExecutor(threads) as ex:
        list(ex.map(lambda i: run(int(edges[i]), int(edges[i + 1])), range(len(edges) - 1)))
    dtn = time.perf_counter() - t0
    return {"value": rows / dtn, "unit": "vectors/s", "cores": threads, "kind": "oracle",
            "cpu_model": cpu_model(),
            "sample": "all %d K vectors of the KV-cache block, quantize + dequantize to fp16, fp64 oracle "
                      "on %d threads over %d equal row shards (%.1f s)" % (rows, threads, len(edges) - 1, dtn),
            "single_thread": {"value": rows_single / dt1, "unit": "vectors/s", "cores": 1,
                              "sample": "first %d K vectors, same work, one thread (%.1f s)" % (rows_single, dt1)}}


def ceiling(torch, dev, stream, xk, ck, nk, yk, n):
    """Trivial streaming kernels with each direction's exact traffic (encode
    shape: 256 B in, 64 + 4 B out per vector; decode shape: the reverse), on
    the same buffers, at 1-8 blocks of 256 threads per CU.  The fastest
    occupancy is each shape's achievable ceiling."""
    import ctypes

    import rotation_vector_quantization_amd.build as rb

    if not os.path.exists(rb.CEIL_LIB):
        return None
    L = ctypes.CDLL(rb.CEIL_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    L.ceiling_encode_shape.argtypes = [vp, vp, vp, i64, i32, vp]
    L.ceiling_decode_shape.argtypes = [vp, vp, vp, i64, i32, vp]
    sh = stream.cuda_stream
    c2 = torch.empty_like(ck)
    n2 = torch.empty_like(nk)
    out = {}
    per_launch = n * BYTES_PER_VECTOR
    for shape, fn in (("encode_shape", lambda bpc: L.ceiling_encode_shape(xk.data_ptr(), c2.data_ptr(),
                                                                           n2.data_ptr(), n, bpc, sh)),
                      ("decode_shape", lambda bpc: L.ceiling_decode_shape(ck.data_ptr(), nk.data_ptr(),
                                                                           yk.data_ptr(), n, bpc, sh))):
        sweep = {}
        for bpc in (1, 2, 3, 4, 6, 8):
            if fn(bpc) != 0:
                raise RuntimeError("ceiling kernel %s failed to launch" % shape)
            ms = float(np.median(time_launches(torch, stream, lambda i: fn(bpc), 1)))
            sweep[bpc] = ms
        best = min(sweep, key=sweep.get)
        gbs = per_launch / (sweep[best] / 1e3) / 1e9
        out[shape] = {"ms_median_by_blocks_per_cu": sweep, "best_blocks_per_cu": best,
                      "ms_median": sweep[best], "GB_per_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS,
                      "bytes_per_launch": per_launch}
    del c2, n2
    return out


def score_ceiling(torch, stream, codes, norms, logits, n, m):
    """The trivial kernel with the 4-bit scorer's traffic (68 B read and m fp32
    logits written per key) on the scorer's own buffer sets, at 1-4 blocks of
    256 threads per CU; the fastest is the achievable ceiling of that shape."""
    import ctypes

    import rotation_vector_quantization_amd.build as rb

    if not os.path.exists(rb.CEIL_LIB):
        return None
    L = ctypes.CDLL(rb.CEIL_LIB)
    vp = ctypes.c_void_p
    L.ceiling_score_shape.argtypes = [vp, vp, vp, ctypes.c_int64, ctypes.c_int, ctypes.c_int, vp]
    sh = stream.cuda_stream
    sweep = {}
    for bpc in (1, 2, 3, 4):
        fn = lambda i: L.ceiling_score_shape(codes[i].data_ptr(), norms[i].data_ptr(), logits[i].data_ptr(), n, m,
                                             bpc, sh)
        if fn(0) != 0:
            raise RuntimeError("score-shape ceiling kernel failed to launch")
        sweep[bpc] = float(np.median(time_launches(torch, stream, fn, len(codes))))
    best = min(sweep, key=sweep.get)
    per_launch = n * 68 + m * n * 4
    gbs = per_launch / (sweep[best] / 1e3) / 1e9
    return {"ms_median_by_blocks_per_cu": sweep, "best_blocks_per_cu": best, "ms_median": sweep[best],
            "GB_per_s": gbs, "frac_of_peak": gbs / HBM_PEAK_GBS, "bytes_per_launch": per_launch}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--cpu-rows", type=int, default=1 << 20,
                    help="rows of the single-thread oracle leg (the all-cores leg takes every K row)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip timing the DRIVE, residual and scoring workloads")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip timing the streaming ceiling kernels (shorter profiled runs)")
    ap.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_c2_kv.json from rocprofv3 PMC runs and exit")
    args = ap.parse_args()
    if args.traffic_from:
        traffic_from(*args.traffic_from)
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: every vector is independent, and the multi-GPU "
              "split (shard the vectors, replicate seed and codebook) is not built; use --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import rotation_vector_quantization_amd as rht
    import testdata

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    rht.load()

    wk, wv = testdata.WORKLOADS["c2k"], testdata.WORKLOADS["c2v"]
    n, d, bits = wk.n, wk.d, wk.bits
    print("generating K and V (%d x %d fp16 each)" % (n, d), file=sys.stderr, flush=True)
    xk_host = testdata.generate(wk)
    xk = torch.from_numpy(xk_host).to(dev)
    xv = torch.from_numpy(testdata.generate(wv)).to(dev)
    ck = torch.empty((n, d * bits // 8), dtype=torch.uint8, device=dev)
    cv = torch.empty_like(ck)
    nk = torch.empty((n,), dtype=torch.float32, device=dev)
    nv = torch.empty_like(nk)
    yk = torch.empty((n, d), dtype=torch.float16, device=dev)
    yv = torch.empty_like(yk)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def q(x, c, nr, w):
        rht.rht_quantize(x.data_ptr(), rht.F16, n, d, bits, rht.SCALE_NORM, w.rot_seed,
                         c.data_ptr(), nr.data_ptr(), sh)

    def dq(c, nr, y, w):
        rht.rht_dequantize(c.data_ptr(), nr.data_ptr(), n, d, bits, rht.SCALE_NORM, w.rot_seed,
                           y.data_ptr(), rht.F16, sh)

    def step(ev=None):
        calls = (lambda: q(xk, ck, nk, wk), lambda: q(xv, cv, nv, wv),
                 lambda: dq(ck, nk, yk, wk), lambda: dq(cv, nv, yv, wv))
        if ev is not None:
            ev[0].record(stream)
        for i, call in enumerate(calls):
            call()
            if ev is not None:
                ev[i + 1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        step(evs[i])
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = start.elapsed_time(end) / args.steps
    # per launch: [quantize K, quantize V, dequantize K, dequantize V] of every step
    per = np.array([[e[i].elapsed_time(e[i + 1]) for i in range(4)] for e in evs])
    q_ms = per[:, 0:2].ravel()
    dq_ms = per[:, 2:4].ravel()
    # practical ceiling: a plain device copy moving the same bytes as one launch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    src.fill_(1)
    for _ in range(3):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_ms = c0.elapsed_time(c1) / 10
    copy_gbs = 2 * COPY_BYTES / (copy_ms / 1e3) / 1e9
    del src, dst

    def direction(ms):
        st = stats(ms)
        gbs = per_launch_bytes / (st["ms_per_launch"] / 1e3) / 1e9
        return dict(st, vectors_per_s=n / (st["ms_per_launch"] / 1e3), GB_per_s=gbs,
                    frac_of_peak=gbs / HBM_PEAK_GBS)

    vectors_per_step = 2 * n
    value = vectors_per_step / (ms_step / 1e3)

    per_launch_bytes = n * BYTES_PER_VECTOR
    kern = {"quantize": float(q_ms.mean()), "dequantize": float(dq_ms.mean())}
    dom = max(kern, key=kern.get)
    achieved = per_launch_bytes / (kern[dom] / 1e3) / 1e9
    kname = {"quantize": "k_quantize", "dequantize": "k_dequantize"}[dom]
    traffic = load_traffic(kname)
    # the kernel the library dispatches for d = 128 fp16 (the generic one if
    # RHT_HADAMARD=valu moves the transform off MFMA)
    kfull = kname + ("<128, ...> (generic)" if os.environ.get("RHT_HADAMARD") == "valu" else "_mfma128")

    out = {
        "metric": "vectors/s + achieved HBM GB/s (% of peak), RHT 4-bit quant/dequant d=128",
        "value": value,
        "unit": "vectors/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "KV-cache block: K and V, each 32 layers x 8 heads x 32768 tokens x d=128 "
                        "fp16; RHT + 4-bit Lloyd-Max quantize, then dequantize to fp16",
            "vectors_per_tensor": n, "d": d, "bits": bits, "io_dtype": "f16",
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "hbm", "kernel": kfull, "achieved": achieved, "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic,
        },
        "per_direction": {k: direction(v) for k, v in (("quantize", q_ms), ("dequantize", dq_ms))},
        "per_tensor": {k: direction(per[:, i]) for i, k in enumerate(
            ("quantize_K", "quantize_V", "dequantize_K", "dequantize_V"))},
        "copy_ceiling": {"GB_per_s": copy_gbs, "frac_of_peak": copy_gbs / HBM_PEAK_GBS,
                         "bytes": 2 * COPY_BYTES, "kernel": "torch device copy"},
        "shape_ceiling": None,
        "wall_s_timed_region": wall,
        "cpu_baseline": None,
    }
    attn = None
    if not args.no_other_workloads:
        print("timing attention over the KV block", file=sys.stderr, flush=True)
        attn = attention_workload(torch, rht, dev, stream, ck, nk, cv, nv, n, d)
        # the pages' KV-cache pairing: the same values coded with 3 bits
        cv3, nv3 = rht.quantize(xv, 3, wv.rot_seed)
        attn_k4v3 = attention_workload(torch, rht, dev, stream, ck, nk, cv3, nv3, n, d, 4, 3)
        del cv3, nv3
    if not args.no_ceiling:
        print("timing the streaming ceiling kernels", file=sys.stderr, flush=True)
        out["shape_ceiling"] = ceiling(torch, dev, stream, xk, ck, nk, yk, n)
    if not args.no_other_workloads:
        del xk, xv, ck, cv, nk, nv, yk, yv
        torch.cuda.empty_cache()
        print("timing the DRIVE, residual and scoring workloads", file=sys.stderr, flush=True)
        out["other_workloads"] = other_workloads(torch, rht, dev, stream, not args.no_ceiling)
        out["other_workloads"]["attention"] = attn
        out["other_workloads"]["attention_k4v3"] = attn_k4v3
    if not args.no_cpu_baseline:
        print("timing the CPU oracle on %d vectors" % args.cpu_rows, file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(xk_host, min(args.cpu_rows, n))
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
