"""Benchmark of the paged KV decode path on one MI355X.

One step = the whole hot path over one batch: append each sequence's new K/V
row into its paged slot, the split-K partition pass of decode attention, and
the log-sum-exp merge, all through the C ABI on torch's current stream.  The
timed step is the fused call (paged_kv_append_attention_decode_ws: two kernels
under the flat schedule); the same step as separate calls (append, partition
pass, merge) is timed beside it, and its per-kernel HIP events give the
roofline of the partition kernel.

Default workload: one Llama-2-7B-shaped layer (32 query / 32 KV heads,
head_dim 128, fp16, block size 16, a pool of 5,120 blocks), 64 sequences with
context lengths uniform in [128, 2048], physical blocks in seeded shuffled
order, synthetic N(0,1)/sqrt(128) data.

Printed (one JSON line): KV-read GB/s over the whole step (value), tokens/s,
the partition kernel's roofline (algorithmic KV bytes per launch / its mean
duration from HIP events, against the 8 TB/s HBM peak), the oracle on the host
cores as a CPU baseline, and context figures (merge and append times, a
streaming-read probe, shuffled vs in-order block tables).  The default run
also measures the other decode configurations (GQA-8B, the copied and the
shared prefix, long context at 512-token partitions and under the library's
own schedule), each kernel after a cache flush, in a "configs" object.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]
                    [--no-cpu-baseline] [--no-extras] [--side-iters N]
    python bench.py --summarize-pmc DIR     # condense rocprofv3 --pmc output
"""
import argparse
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged-attn decode: KV-read GB/s (% of HBM peak), tokens/s at Llama-2-7B shape"
KERNEL_SOURCES = ["paged_kv_cache_227_amd/csrc/decode.hip", "paged_kv_cache_227_amd/csrc/pkv_device.h",
                  "paged_kv_cache_227_amd/csrc/pkv_mfma.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_{config}.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


COPY_KERNEL_SOURCES = ["paged_kv_cache_227_amd/csrc/copy_blocks.hip"]


def code_tokens(text):
    """C++ source with its comments removed and each run of whitespace made one
    space: an edit to comments or layout leaves it unchanged, any change to the
    code does not."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_hash(sources=None):
    """Hash of the kernel sources' code (comments and layout excluded), which keys
    the stored counter summaries to the code they were taken on."""
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), encoding="utf-8") as f:
            h.update(code_tokens(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(config, n_bytes, sources=None):
    """HBM traffic of the measured kernel from committed counter summaries,
    or None when absent or taken on different kernel sources."""
    path = TRAFFIC_FILE.format(config=config)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_hash") != kernel_hash(sources):
        return None
    return t


def make_workload(name):
    from paged_kv_cache_227_amd import workloads as W
    return W.CONFIGS[name]()


def decode_kernel_name(w, part):
    """The partition-pass kernel that runs for this workload: the flat schedule,
    or fixed partitions (persistent workgroups for the matrix-core shapes whose
    KV heads form teams of four)."""
    if part == 0:
        return "decode_flat_kernel"
    g = w.n_q_heads // w.n_kv_heads
    if w.dtype in ("f16", "bf16") and g >= 4 and w.n_kv_heads % 4 == 0:
        return "decode_partition_persistent_kernel"
    return "decode_partition_kernel"


def with_schedule(w, schedule):
    """The workload as given ("workload": its own partition length, if it fixes
    one), or under the library's default schedule ("default"), then named
    <workload>_default_schedule for its traffic and profile files."""
    if schedule == "default" and w.part_tokens:
        w.part_tokens = 0
        w.name = w.name + "_default_schedule"
    return w


def run_gpu(w, steps, warmup, extras, graph=False):
    import torch
    import paged_kv_cache_227_amd as P
    from paged_kv_cache_227_amd import workloads as W

    dev = torch.device("cuda:0")
    T = W.to_torch(w, dev)
    q, kc, vc, bt, lens = T["q"], T["k_cache"], T["v_cache"], T["block_tables"], T["context_lens"]
    out = torch.empty_like(q)
    layout = P.layout_of(kc)
    part = w.part_tokens or P.partition_tokens_for(w.num_seqs, w.n_q_heads, w.max_blocks_per_seq, layout)
    ws = P.alloc_workspace(q, kc, bt, part)

    def fused_step():
        P.paged_kv_append_attention_decode(T["k_new"], T["v_new"], T["positions"], q, kc, vc, bt, lens, w.scale,
                                           out, part_tokens=part, workspace=ws)

    def step(ev=None):
        if ev:
            ev[0].record()
        P.paged_kv_append(T["k_new"], T["v_new"], kc, vc, bt, T["positions"])
        if ev:
            ev[1].record()
        P.paged_attention_partitions(q, kc, vc, bt, lens, w.scale, out, part, ws)
        if ev:
            ev[2].record()
        P.paged_attention_merge(kc, bt, lens, out, part, ws)
        if ev:
            ev[3].record()

    for _ in range(warmup):
        step()
        fused_step()
    torch.cuda.synchronize()
    res_graph = {}
    if graph:
        # the whole step as one HIP graph, replayed
        g = torch.cuda.CUDAGraph()
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            fused_step()
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            fused_step()
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            g.replay()
        torch.cuda.synchronize()
        res_graph["graph_ms_per_step"] = (time.perf_counter() - t0) * 1e3 / steps
    # The timed region: exactly `steps` steps between two synchronisations,
    # nothing else on the stream.
    # the same step as separate calls, for comparison (not the reported value);
    # timed first, since the first timed region of a run measures slightly slow
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    res_graph["two_calls_ms_per_step"] = (time.perf_counter() - t0) * 1e3 / steps
    t0 = time.perf_counter()
    for i in range(steps):
        fused_step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    # Right after it, the same steps with HIP events around every kernel (on
    # torch's current stream, where the library launches): per-kernel durations.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        step(events[i])
    torch.cuda.synchronize()
    t_app = [e[0].elapsed_time(e[1]) for e in events]
    t_part = [e[1].elapsed_time(e[2]) for e in events]
    t_merge = [e[2].elapsed_time(e[3]) for e in events]
    res = dict(ms_per_step=ms_step, part_tokens=part, **res_graph, kernel=decode_kernel_name(w, part),
               partition_ms_mean=statistics.fmean(t_part), partition_ms_median=statistics.median(t_part),
               partition_ms_p10=sorted(t_part)[len(t_part) // 10],
               partition_ms_p90=sorted(t_part)[(len(t_part) * 9) // 10],
               merge_ms_mean=statistics.fmean(t_merge), append_ms_mean=statistics.fmean(t_app))

    if extras:
        # a streaming read of 4 GiB: the HBM read rate a plain streaming kernel reaches
        buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
        buf.fill_(1)
        sink = torch.empty(4096, dtype=torch.float32, device=dev)
        for _ in range(3):
            P.probe_read(buf, sink)
        s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s0.record()
        for _ in range(10):
            P.probe_read(buf, sink)
        s1.record()
        torch.cuda.synchronize()
        res["probe_read_gbs"] = buf.numel() * 10 / (s0.elapsed_time(s1) * 1e-3) / 1e9
        # the decode kernel after a flush: a 2 GiB copy (8x the 256 MB last-level
        # cache) before each launch, so no K/V byte can be served from cache
        src, dst = buf[:1 << 30], buf[1 << 30:2 << 30]
        t_fl = []
        for _ in range(10):
            P.probe_copy(src, dst)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            P.paged_attention_partitions(q, kc, vc, bt, lens, w.scale, out, part, ws)
            e1.record()
            P.paged_attention_merge(kc, bt, lens, out, part, ws)
            torch.cuda.synchronize()
            t_fl.append(e0.elapsed_time(e1))
        res["partition_ms_flushed_median"] = statistics.median(t_fl)
        del buf, sink, src, dst
    del T, q, kc, vc, out, ws
    torch.cuda.empty_cache()
    return res


def time_partitions_only(w, iters=30):
    """Mean partition-pass time (ms) for a workload, e.g. in-order block tables."""
    import torch
    import paged_kv_cache_227_amd as P
    from paged_kv_cache_227_amd import workloads as W
    T = W.to_torch(w, "cuda:0")
    out = torch.empty_like(T["q"])
    layout = P.layout_of(T["k_cache"])
    part = w.part_tokens or P.partition_tokens_for(w.num_seqs, w.n_q_heads, w.max_blocks_per_seq, layout)
    ws = P.alloc_workspace(T["q"], T["k_cache"], T["block_tables"], part)
    args = (T["q"], T["k_cache"], T["v_cache"], T["block_tables"], T["context_lens"], w.scale, out, part, ws)
    for _ in range(5):
        P.paged_attention_partitions(*args)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(iters):
        P.paged_attention_partitions(*args)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters


# The other decode configurations, each on its own layer, measured in the same
# run: (key, workload, partition length: None = the library's choice, label).
# "graded" rows count against the HBM peak; the shared-prefix layout reads its
# 64 prompt blocks 128 times, from cache after the first, so its rate is an
# effective one (logical K/V bytes / time) and is not graded against HBM.
SIDE_CONFIGS = [
    ("gqa_8b", "gqa_8b", None, "graded"),
    ("prefix_copied", "prefix_copied", None, "graded"),
    ("prefix_shared", "prefix_shared", None, "effective"),
    ("long_context", "long_context", 512, "graded"),
    ("long_context_default_schedule", "long_context", None, "graded"),
]


def profile_for(key, kernel):
    """The committed rocprofv3 kernel-trace summary of this kernel on this workload, if any."""
    path = os.path.join("profiles", "%s_%s.md" % (kernel, key))
    return path if os.path.exists(os.path.join(ROOT, path)) else None


def measure_side_configs(iters, flush_bytes=2 << 30):
    """Decode kernel of each SIDE_CONFIGS workload: `iters` launches, each after
    a copy of flush_bytes (8x the 256 MB last-level cache) so that no K/V byte
    is left in cache from the launch before, with HIP events around the
    partition pass; plus the fused step (append + decode + merge) timed over
    `iters` back-to-back calls."""
    import torch
    import paged_kv_cache_227_amd as P
    from paged_kv_cache_227_amd import workloads as W
    dev = torch.device("cuda:0")
    buf = torch.empty(flush_bytes, dtype=torch.uint8, device=dev)
    buf.fill_(1)
    src, dst = buf[:flush_bytes // 2], buf[flush_bytes // 2:]
    out_rows = {}
    cache = {}
    for key, name, part_req, label in SIDE_CONFIGS:
        t_gen = time.perf_counter()
        if name not in cache:
            cache.clear()
            cache[name] = make_workload(name)
        w = cache[name]
        T = W.to_torch(w, dev)
        q, kc, vc, bt, lens = T["q"], T["k_cache"], T["v_cache"], T["block_tables"], T["context_lens"]
        out = torch.empty_like(q)
        layout = P.layout_of(kc)
        part = part_req if part_req is not None else P.partition_tokens_for(w.num_seqs, w.n_q_heads,
                                                                          w.max_blocks_per_seq, layout)
        ws = P.alloc_workspace(q, kc, bt, part)
        t_gen = time.perf_counter() - t_gen

        def fused():
            P.paged_kv_append_attention_decode(T["k_new"], T["v_new"], T["positions"], q, kc, vc, bt, lens,
                                               w.scale, out, part_tokens=part, workspace=ws)
        for _ in range(3):
            fused()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(iters):
            fused()
        torch.cuda.synchronize()
        ms_step = (time.perf_counter() - t0) * 1e3 / iters
        t_k, t_m = [], []
        for _ in range(iters):
            P.probe_copy(src, dst)
            e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
            e[0].record()
            P.paged_attention_partitions(q, kc, vc, bt, lens, w.scale, out, part, ws)
            e[1].record()
            P.paged_attention_merge(kc, bt, lens, out, part, ws)
            e[2].record()
            torch.cuda.synchronize()
            t_k.append(e[0].elapsed_time(e[1]))
            t_m.append(e[1].elapsed_time(e[2]))
        kv = w.kv_read_bytes()
        kms = statistics.fmean(t_k)
        gbs = kv / (kms * 1e-3) / 1e9
        kernel = decode_kernel_name(w, part)
        row = {"label": label, "workload": name, "kernel": kernel, "partition_tokens": part, "dtype": w.dtype,
               "num_seqs": w.num_seqs, "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads,
               "kv_read_bytes": kv, "mean_launch_ms": round(kms, 5),
               "median_launch_ms": round(statistics.median(t_k), 5), "merge_ms_mean": round(statistics.fmean(t_m), 5),
               "fused_step_ms": round(ms_step, 5), "fused_step_gbs": round(kv / (ms_step * 1e-3) / 1e9, 1),
               "timing": "HIP events around each of %d launches, each after a %d GiB cache flush" % (
                   iters, flush_bytes >> 30)}
        if label == "graded":
            row["kernel_gbs"] = round(gbs, 1)
            row["frac"] = round(gbs / HBM_PEAK_GBS, 4)
            t = load_traffic(key, kv)
            row["traffic"] = None if t is None else round(t["hbm_bytes_per_launch"])
            row["hbm_read_over_algorithmic"] = None if t is None else round(t["read_over_algorithmic"], 4)
        else:
            row["kernel_gbs_effective"] = round(gbs, 1)
            row["unique_kv_bytes"] = int(w.used_blocks()) * w.block_size * w.n_kv_heads * 2 * w.head_dim * (
                4 if w.dtype == "f32" else 2)
        row["profile"] = profile_for(key, kernel)
        out_rows[key] = row
        log("config %s: %s, kernel %.4f ms (%.0f GB/s%s), fused step %.4f ms (setup %.1f s)" % (
            key, kernel, kms, gbs, "" if label == "graded" else ", effective", ms_step, t_gen))
        del T, q, kc, vc, bt, lens, out, ws
        torch.cuda.empty_cache()
    del buf, src, dst
    cache.clear()
    torch.cuda.empty_cache()
    return out_rows


def cpu_baseline(w, budget_s=15.0, min_s=10.0):
    """The oracle (append + decode, fp64) on a bounded sample of the workload's
    sequences, on every host core it may use: batches of sequences until
    budget_s is spent; when the whole workload takes less than min_s, whole
    passes repeat until min_s has elapsed."""
    import numpy as np
    from oracle import ref
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    orc = ref.default()
    threads = orc.num_threads()
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    t0 = time.perf_counter()
    orc.append(w.k_new, w.v_new, kc, vc, w.block_tables, w.positions, w.dtype_code)
    t_append = time.perf_counter() - t0
    done, elapsed, tokens, passes = 0, 0.0, 0, 0
    batch = max(1, w.num_seqs // 16)
    while elapsed < budget_s:
        order = list(range(w.num_seqs))
        while order and elapsed < budget_s:
            ids, order = order[:batch], order[batch:]
            t0 = time.perf_counter()
            orc.attention_decode(w.q, kc, vc, w.block_tables, w.context_lens, w.scale, w.dtype_code, seq_ids=ids)
            elapsed += time.perf_counter() - t0
            done += len(ids)
            tokens += int(np.sum(w.context_lens[ids]))
        passes += not order
        if order or elapsed >= min_s:
            break
    kv_bytes = tokens * w.n_kv_heads * 2 * w.head_dim * (4 if w.dtype == "f32" else 2)
    sample = ("%d sequence decodes: %d whole pass(es) over the %d sequences%s (%d tokens, %.1f s of decode)"
              % (done, passes, w.num_seqs, " and part of another" if done > passes * w.num_seqs else "",
                 tokens, elapsed))
    return {"value": kv_bytes / elapsed / 1e9, "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": sample + ", append of all %d sequences %.3f s" % (w.num_seqs, t_append),
            "tokens_per_s": done / elapsed}


def run_copy_probe(n_bytes):
    """One launch of the plain copy kernel over n_bytes: a dispatch of known
    traffic for calibrating hardware counters in the same profiled run."""
    import torch
    import paged_kv_cache_227_amd as P
    n = n_bytes // 16 * 16
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    P.probe_copy(src, dst)
    torch.cuda.synchronize()
    del src, dst
    torch.cuda.empty_cache()


def run_copy(cw, steps, warmup):
    """Time paged_kv_copy_blocks on the copy workload: `steps` calls between two
    synchronisations, then the same calls with HIP events around each launch."""
    import torch
    import paged_kv_cache_227_amd as P
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[cw.dtype]
    shape = (cw.num_blocks, cw.block_size, cw.n_kv_heads, cw.head_dim)
    kc = torch.zeros(shape, dtype=tdt, device="cuda:0")
    vc = torch.zeros_like(kc)
    src, dst, rows = (torch.from_numpy(x).to("cuda:0") for x in (cw.src, cw.dst, cw.rows))

    def step():
        P.paged_kv_copy_blocks(kc, vc, src, dst, rows)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    # per-launch HIP events, each launch after a 2 GiB copy: a small copy workload's
    # rows would otherwise stay in the L2s from the call before, and the rate
    # would not be an HBM one
    buf = torch.empty(2 << 30, dtype=torch.uint8, device="cuda:0")
    buf.fill_(1)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e in ev:
        P.probe_copy(buf[:1 << 30], buf[1 << 30:])
        e[0].record()
        step()
        e[1].record()
    torch.cuda.synchronize()
    t = [a.elapsed_time(b) for a, b in ev]
    del kc, vc, buf
    torch.cuda.empty_cache()
    return dict(ms_per_step=ms_step, kernel_ms_mean=statistics.fmean(t), kernel_ms_median=statistics.median(t))


def cpu_baseline_copy(cw, min_s=3.0):
    """The oracle's block copy on host copies of the caches, repeated until
    min_s has elapsed."""
    import numpy as np
    from oracle import ref
    orc = ref.default()
    st = np.float32 if cw.dtype == "f32" else np.uint16
    shape = (cw.num_blocks, cw.block_size, cw.n_kv_heads, cw.head_dim)
    kc, vc = np.zeros(shape, st), np.zeros(shape, st)
    code = {"f32": 0, "f16": 1, "bf16": 2}[cw.dtype]
    n, elapsed = 0, 0.0
    while elapsed < min_s:
        t0 = time.perf_counter()
        orc.copy_blocks(kc, vc, cw.src, cw.dst, cw.rows, code)
        elapsed += time.perf_counter() - t0
        n += 1
    return {"value": 2 * cw.moved_bytes() * n / elapsed / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d whole calls (%d copies each), %.1f s" % (n, len(cw.src), elapsed)}


def main_copy(a):
    from paged_kv_cache_227_amd import workloads as W
    if a.config not in W.COPY_CONFIGS:
        raise SystemExit("copy workloads: %s" % ", ".join(W.COPY_CONFIGS))
    name = a.config
    cw = W.COPY_CONFIGS[name]()
    moved = 2 * cw.moved_bytes()  # read + written
    log("copy workload %s: %d copies, %d rows, %.1f MB read and written" % (
        name, len(cw.src), int(cw.rows.sum()), moved / 1e6))
    g = run_copy(cw, a.steps, a.warmup)
    log("gpu: %.4f ms/call, kernel %.4f ms" % (g["ms_per_step"], g["kernel_ms_mean"]))
    achieved = moved / (g["kernel_ms_mean"] * 1e-3) / 1e9
    value = moved / (g["ms_per_step"] * 1e-3) / 1e9
    t = load_traffic(name, moved, COPY_KERNEL_SOURCES)
    traffic = None if t is None else int(round(t["hbm_bytes_per_launch"]))
    res = {
        "metric": "paged KV block copy (copy-on-write): bytes read + written per second", "value": round(value, 1),
        "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(g["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cw.dtype, "data": "synthetic",
        "config": {"workload": name, "n_copies": int(len(cw.src)), "rows_copied": int(cw.rows.sum()),
                   "num_blocks": cw.num_blocks, "n_kv_heads": cw.n_kv_heads, "head_dim": cw.head_dim,
                   "block_size": cw.block_size, "bytes_read_and_written": moved, "seed": cw.seed,
                   "notes": cw.notes},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": "copy_blocks_kernel",
                     "algorithmic_bytes_per_launch": moved,
                     "timing": "HIP events around each of %d launches right after the timed region, each after "
                               "a 2 GiB cache-evicting copy" % a.steps,
                     "mean_launch_ms": round(g["kernel_ms_mean"], 5)},
        "us_per_call": round(g["ms_per_step"] * 1e3, 2),
    }
    if a.copy_probe_bytes:
        run_copy_probe(a.copy_probe_bytes)
        res["copy_probe_bytes"] = a.copy_probe_bytes // 16 * 16
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_copy(cw)
    print(json.dumps(res), flush=True)
    return 0


MFMA_PEAK_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}


def run_prefill(w, steps, warmup):
    """Time the chunked-prefill step (n-token append, then attention) on the
    workload: `steps` steps between two synchronisations, then the same steps
    with HIP events around each kernel."""
    import numpy as np
    import torch
    import paged_kv_cache_227_amd as P
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).to("cuda:0")

    def i32(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to("cuda:0")

    kc, vc, q, kn, vn = (dev(a) for a in (w.k_cache, w.v_cache, w.q, w.k_new, w.v_new))
    bt, cu, lens, sp = i32(w.block_tables), i32(w.cu_q), i32(w.context_lens), i32(w.start_pos)
    out = torch.empty_like(q)

    def step(ev=None):
        if ev:
            ev[0].record()
        P.paged_kv_append_tokens(kn, vn, kc, vc, bt, cu, sp)
        if ev:
            ev[1].record()
        P.paged_attention_prefill(q, kc, vc, bt, cu, lens, w.scale, out, w.max_q_len)
        if ev:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        step(e)
    torch.cuda.synchronize()
    t_app = [e[0].elapsed_time(e[1]) for e in ev]
    t_att = [e[1].elapsed_time(e[2]) for e in ev]
    del kc, vc, q, kn, vn, out
    torch.cuda.empty_cache()
    return dict(ms_per_step=ms_step, prefill_ms_mean=statistics.fmean(t_att),
                prefill_ms_median=statistics.median(t_att), append_ms_mean=statistics.fmean(t_app))


def cpu_baseline_prefill(w, budget_s=10.0):
    """The oracle's prefill attention on query rows in a fixed random order
    (whole passes over the step's rows repeated) until budget_s is spent;
    flops per second of the rows computed."""
    import numpy as np
    from oracle import ref
    cores = len(os.sched_getaffinity(0))
    os.environ.setdefault("OMP_NUM_THREADS", str(cores))
    orc = ref.default()
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    orc.append_tokens(w.k_new, w.v_new, kc, vc, w.block_tables, w.cu_q, w.start_pos, w.dtype_code)
    total = int(w.cu_q[-1])
    order = np.random.default_rng(0).permutation(total)
    seq_of = np.searchsorted(w.cu_q, np.arange(total), side="right") - 1
    pos = w.start_pos[seq_of] + (np.arange(total) - w.cu_q[seq_of])
    if total == 0:
        return None
    done, flops, elapsed = 0, 0, 0.0
    batch = 64
    while elapsed < budget_s:
        start = done % total
        ids = np.sort(order[start:start + batch])
        t0 = time.perf_counter()
        orc.attention_prefill(w.q, kc, vc, w.block_tables, w.cu_q, w.context_lens, w.scale, w.dtype_code,
                              row_ids=ids)
        elapsed += time.perf_counter() - t0
        flops += int(np.sum(pos[ids] + 1)) * 4 * w.head_dim * w.n_q_heads
        done += len(ids)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": orc.num_threads(), "kind": "oracle",
            "sample": "%d query rows (all heads): %.2f passes over the step's %d rows, %.1f s" % (
                done, done / total, total, elapsed)}


def main_prefill(a):
    from paged_kv_cache_227_amd import workloads as W
    if a.config not in W.PREFILL_CONFIGS:
        raise SystemExit("prefill workloads: %s" % ", ".join(W.PREFILL_CONFIGS))
    w = W.PREFILL_CONFIGS[a.config]()
    flops = w.attention_flops()
    log("prefill workload %s: %d sequences, chunks %s, contexts %s, %.2f GFLOP" % (
        w.name, w.num_seqs, list(w.chunk_lens), list(w.context_lens), flops / 1e9))
    g = run_prefill(w, a.steps, a.warmup)
    log("gpu: %.4f ms/step, prefill %.4f ms, append %.4f ms" % (g["ms_per_step"], g["prefill_ms_mean"],
                                                                 g["append_ms_mean"]))
    value = flops / (g["ms_per_step"] * 1e-3) / 1e12
    achieved = flops / (g["prefill_ms_mean"] * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    res = {
        "metric": "chunked prefill: attention TFLOP/s (causal flops of the step's chunks)", "value": round(value, 2),
        "unit": "TFLOP/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(g["ms_per_step"], 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "chunk_lens": [int(x) for x in w.chunk_lens],
                   "context_lens": [int(x) for x in w.context_lens], "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "attention_flops": flops, "seed": w.seed, "notes": w.notes},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": None, "kernel": "prefill_kernel",
                     "algorithmic_flops_per_launch": flops,
                     "timing": "HIP events around each launch, %d steps right after the timed region" % a.steps,
                     "mean_launch_ms": round(g["prefill_ms_mean"], 5)},
        "kernel_ms": {k: round(g[k], 5) for k in ("prefill_ms_mean", "prefill_ms_median", "append_ms_mean")},
        "tokens_per_s": round(int(w.cu_q[-1]) / (g["ms_per_step"] * 1e-3), 1),
        "kv_read_gbs": round(w.kv_bytes() / (g["prefill_ms_mean"] * 1e-3) / 1e9, 1),
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prefill(w)
    print(json.dumps(res), flush=True)
    return 0


HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, each direction


def run_swap(cw, steps, warmup):
    """Time the swap round trip (swap-out, then swap-in) of the workload's
    blocks: `steps` round trips between two synchronisations, then each call
    again with HIP events; also a contiguous DMA copy of the same bytes
    (hipMemcpyAsync through torch) each way, for reference."""
    import torch
    import paged_kv_cache_227_amd as P
    shape = (cw.num_blocks, cw.block_size, cw.n_kv_heads, cw.head_dim)
    kc = torch.zeros(shape, dtype=torch.float16, device="cuda:0")
    vc = torch.zeros_like(kc)
    blocks = torch.from_numpy(cw.src).to("cuda:0")
    hk = torch.empty((len(cw.src),) + shape[1:], dtype=torch.float16, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)

    def step(ev=None):
        if ev:
            ev[0].record()
        P.paged_kv_swap_out(kc, vc, blocks, hk, hv)
        if ev:
            ev[1].record()
        P.paged_kv_swap_in(kc, vc, blocks, hk, hv)
        if ev:
            ev[2].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        step(e)
    torch.cuda.synchronize()
    t_out = statistics.fmean(e[0].elapsed_time(e[1]) for e in ev)
    t_in = statistics.fmean(e[1].elapsed_time(e[2]) for e in ev)
    # reference: one contiguous buffer of the same size, each way, on the DMA engine
    dev = torch.empty(2 * hk.numel(), dtype=torch.float16, device="cuda:0")
    host = torch.empty(2 * hk.numel(), dtype=torch.float16, pin_memory=True)
    for _ in range(2):
        host.copy_(dev, non_blocking=True)
        dev.copy_(host, non_blocking=True)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    host.copy_(dev, non_blocking=True)
    e[1].record()
    dev.copy_(host, non_blocking=True)
    e[2].record()
    torch.cuda.synchronize()
    dma_out, dma_in = e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])
    del kc, vc, hk, hv, dev, host
    torch.cuda.empty_cache()
    return dict(ms_per_step=ms_step, out_ms=t_out, in_ms=t_in, dma_out_ms=dma_out, dma_in_ms=dma_in)


def cpu_baseline_swap(cw, min_s=3.0):
    """The oracle's swap (out, then in) on host copies of the caches."""
    import numpy as np
    from oracle import ref
    orc = ref.default()
    shape = (cw.num_blocks, cw.block_size, cw.n_kv_heads, cw.head_dim)
    kc, vc = np.zeros(shape, np.uint16), np.zeros(shape, np.uint16)
    n, elapsed = 0, 0.0
    while elapsed < min_s:
        t0 = time.perf_counter()
        hk, hv = orc.swap_out(kc, vc, cw.src, 1)
        orc.swap_in(kc, vc, cw.dst, hk, hv, 1)
        elapsed += time.perf_counter() - t0
        n += 1
    return {"value": 2 * 2 * cw.moved_bytes() * n / elapsed / 1e9, "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%d round trips of %d blocks, %.1f s" % (n, len(cw.src), elapsed)}


def main_swap(a):
    from paged_kv_cache_227_amd import workloads as W
    if a.config not in W.SWAP_CONFIGS:
        raise SystemExit("swap workloads: %s" % ", ".join(W.SWAP_CONFIGS))
    cw = W.SWAP_CONFIGS[a.config]()
    each_way = cw.moved_bytes()  # both caches' blocks, one direction
    log("swap workload %s: %d blocks, %.1f MB each way" % (cw.name, len(cw.src), each_way / 1e6))
    g = run_swap(cw, a.steps, a.warmup)
    gbs = lambda ms: each_way / (ms * 1e-3) / 1e9
    log("gpu: %.3f ms per round trip; out %.3f ms (%.1f GB/s), in %.3f ms (%.1f GB/s); DMA %.1f / %.1f GB/s"
        % (g["ms_per_step"], g["out_ms"], gbs(g["out_ms"]), g["in_ms"], gbs(g["in_ms"]), gbs(g["dma_out_ms"]),
           gbs(g["dma_in_ms"])))
    achieved = 2 * each_way / ((g["out_ms"] + g["in_ms"]) * 1e-3) / 1e9  # per direction, over both launches
    res = {
        "metric": "paged KV swap (preemption): bytes moved per second over the host link, out + in",
        "value": round(2 * each_way / (g["ms_per_step"] * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": a.steps, "warmup": a.warmup, "ms_per_step": round(g["ms_per_step"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": cw.dtype, "data": "synthetic",
        "config": {"workload": cw.name, "n_blocks": int(len(cw.src)), "bytes_each_way": each_way,
                   "num_blocks": cw.num_blocks, "n_kv_heads": cw.n_kv_heads, "head_dim": cw.head_dim,
                   "block_size": cw.block_size, "seed": cw.seed, "notes": cw.notes},
        "roofline": {"bound": "host_link", "achieved": round(achieved, 2), "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HOST_LINK_PEAK_GBS, 4), "traffic": None, "kernel": "swap_kernel",
                     "algorithmic_bytes_per_launch": each_way,
                     "timing": "HIP events around each launch, %d round trips after the timed region" % a.steps,
                     "mean_launch_ms": {"out": round(g["out_ms"], 4), "in": round(g["in_ms"], 4)}},
        "swap_out_gbs": round(gbs(g["out_ms"]), 2), "swap_in_gbs": round(gbs(g["in_ms"]), 2),
        "dma_reference_gbs": {"out": round(gbs(g["dma_out_ms"]), 2), "in": round(gbs(g["dma_in_ms"]), 2),
                              "what": "one contiguous buffer of the same size, hipMemcpyAsync"},
    }
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_swap(cw)
    print(json.dumps(res), flush=True)
    return 0


def summarize_pmc(d):
    """Mean FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel from rocprofv3
    --pmc CSV output under directory d."""
    import csv
    rows = {}
    for path in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r.get("Kernel_Name", "")
                key = (name, r.get("Counter_Name", ""))
                rows.setdefault(key, []).append(float(r.get("Counter_Value", 0)))
    out = {}
    for (name, ctr), vals in rows.items():
        out.setdefault(name, {})[ctr] = {"mean": statistics.fmean(vals), "dispatches": len(vals)}
    return out


def write_traffic(fetch_dir, write_dir, config, kv_bytes, copy_bytes, out_path, kernel_key="decode_flat_kernel",
                  sources=None):
    """HBM traffic per launch of the decode kernel from two rocprofv3 --pmc runs
    (FETCH_SIZE, then WRITE_SIZE; KiB per dispatch), each scaled by what the same
    counter reads for the plain copy kernel of known size in the same run."""
    f, w = summarize_pmc(fetch_dir), summarize_pmc(write_dir)

    def pick(d, key):
        names = [n for n in d if key in n]
        if len(names) > 1:  # the flat kernel with and without a fused append: the plain one
            names = [n for n in names if ">, false, " in n]
        if len(names) != 1:
            raise SystemExit("expected one kernel matching %r, found %r" % (key, names))
        return d[names[0]], names[0]

    copy_f, _ = pick(f, "probe_copy_kernel")
    copy_w, _ = pick(w, "probe_copy_kernel")
    dec_f, name = pick(f, kernel_key)
    dec_w, _ = pick(w, kernel_key)
    copy_kib = copy_bytes / 1024.0
    f_scale = copy_kib / copy_f["FETCH_SIZE"]["mean"]
    w_scale = copy_kib / copy_w["WRITE_SIZE"]["mean"]
    read_b = dec_f["FETCH_SIZE"]["mean"] * f_scale * 1024
    write_b = dec_w["WRITE_SIZE"]["mean"] * w_scale * 1024
    t = {"config": config, "kernel": name, "kernel_hash": kernel_hash(sources),
         "fetch_size_kib_raw": dec_f["FETCH_SIZE"]["mean"], "write_size_kib_raw": dec_w["WRITE_SIZE"]["mean"],
         "dispatches": dec_f["FETCH_SIZE"]["dispatches"],
         "copy_probe_bytes": copy_bytes, "copy_fetch_kib_raw": copy_f["FETCH_SIZE"]["mean"],
         "copy_write_kib_raw": copy_w["WRITE_SIZE"]["mean"], "fetch_scale": f_scale, "write_scale": w_scale,
         "hbm_read_bytes_per_launch": read_b, "hbm_write_bytes_per_launch": write_b,
         "hbm_bytes_per_launch": read_b + write_b, "algorithmic_kv_bytes": kv_bytes,
         "read_over_algorithmic": read_b / kv_bytes}
    with open(out_path, "w") as fh:
        json.dump(t, fh, indent=1)
        fh.write("\n")
    return t


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--op", default="decode", choices=["decode", "copy_blocks", "prefill", "swap"],
                    help="decode: the append + decode step (default); copy_blocks: the copy-on-write block "
                         "copy; prefill: the chunked-prefill step (n-token append + attention); swap: a "
                         "preempted sequence's blocks out to pinned host memory and back")
    ap.add_argument("--config", default=None,
                    help="workload (default llama2_7b for decode, copy_whole_llama2_7b for copy_blocks)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--summarize-pmc", metavar="DIR")
    ap.add_argument("--write-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic_<config>.json from two rocprofv3 --pmc runs of this bench "
                         "made with --copy-probe-bytes (pass the same size)")
    ap.add_argument("--graph", action="store_true", help="also time the step as a replayed HIP graph")
    ap.add_argument("--schedule", default="workload", choices=["workload", "default"],
                    help="decode: the workload's own partition length (long_context: 512 tokens), or the "
                         "library's default schedule")
    ap.add_argument("--side-iters", type=int, default=20,
                    help="flushed launches per configuration in the 'configs' object of the default run")
    ap.add_argument("--copy-probe-bytes", type=int, default=0,
                    help="after the steps, run the plain copy kernel once over this many bytes "
                         "(a launch of known traffic for calibrating hardware counters)")
    a = ap.parse_args()
    if a.config is None:
        a.config = {"decode": "llama2_7b", "copy_blocks": "copy_whole_llama2_7b",
                    "prefill": "prefill_llama2_7b", "swap": "swap_llama2_7b"}[a.op]

    if a.summarize_pmc:
        print(json.dumps(summarize_pmc(a.summarize_pmc), indent=1))
        return 0
    if a.write_traffic:
        if not a.copy_probe_bytes:
            raise SystemExit("--write-traffic needs --copy-probe-bytes (the size the counter runs used)")
        if a.op == "copy_blocks":
            from paged_kv_cache_227_amd import workloads as W
            cw = W.COPY_CONFIGS[a.config]()
            # algorithmic reads: the bytes copied (the writes are as many)
            t = write_traffic(a.write_traffic[0], a.write_traffic[1], a.config, cw.moved_bytes(),
                              a.copy_probe_bytes // 16 * 16, TRAFFIC_FILE.format(config=a.config),
                              "copy_blocks_kernel", COPY_KERNEL_SOURCES)
        else:
            w = with_schedule(make_workload(a.config), a.schedule)
            t = write_traffic(a.write_traffic[0], a.write_traffic[1], w.name, w.kv_read_bytes(),
                              a.copy_probe_bytes // 16 * 16, TRAFFIC_FILE.format(config=w.name),
                              decode_kernel_name(w, w.part_tokens))
        print(json.dumps(t, indent=1))
        return 0
    if a.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (use --gpus 1)", file=sys.stderr)
        return 2

    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if a.op == "copy_blocks":
        return main_copy(a)
    if a.op == "prefill":
        return main_prefill(a)
    if a.op == "swap":
        return main_swap(a)

    t = time.perf_counter()
    w = with_schedule(make_workload(a.config), a.schedule)
    log("workload %s: %d sequences, %d tokens, KV bytes %.3f GB (generated in %.1f s)"
        % (w.name, w.num_seqs, int(w.context_lens.sum()), w.kv_read_bytes() / 1e9, time.perf_counter() - t))
    kv = w.kv_read_bytes()
    g = run_gpu(w, a.steps, a.warmup, not a.no_extras, graph=a.graph)
    log("gpu: %.4f ms/step, partition %.4f ms, merge %.4f ms, append %.4f ms"
        % (g["ms_per_step"], g["partition_ms_mean"], g["merge_ms_mean"], g["append_ms_mean"]))

    achieved = kv / (g["partition_ms_mean"] * 1e-3) / 1e9
    traffic = load_traffic(w.name, kv)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": None if traffic is None else round(traffic["hbm_bytes_per_launch"]),
                "kernel": g["kernel"], "algorithmic_bytes_per_launch": kv,
                "timing": "HIP events around each launch, %d steps right after the timed region" % a.steps,
                "mean_launch_ms": round(g["partition_ms_mean"], 5)}
    value = kv / (g["ms_per_step"] * 1e-3) / 1e9
    res = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": a.steps,
        "warmup": a.warmup, "ms_per_step": round(g["ms_per_step"], 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": w.num_seqs, "n_q_heads": w.n_q_heads,
                   "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "block_size": w.block_size,
                   "num_blocks": w.num_blocks, "total_context_tokens": int(w.context_lens.sum()),
                   "kv_read_bytes": kv, "partition_tokens": g["part_tokens"], "seed": w.seed},
        "roofline": roofline,
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "tokens_per_s": round(w.num_seqs / (g["ms_per_step"] * 1e-3), 1),
        "tokens_per_s_32_layers": round(w.num_seqs / (32 * g["ms_per_step"] * 1e-3), 1),
        "kernel_ms": {k: round(g[k], 5) for k in ("partition_ms_mean", "partition_ms_median",
                                                  "partition_ms_p10", "partition_ms_p90",
                                                  "merge_ms_mean", "append_ms_mean")},
        "step_ms_variants": {k: round(g[k], 5) for k in ("graph_ms_per_step", "two_calls_ms_per_step") if k in g},
    }
    if not a.no_extras:
        from paged_kv_cache_227_amd import workloads as W
        res["probe_read_gbs"] = round(g["probe_read_gbs"], 1)
        res["decode_kernel_gbs_after_flush"] = round(kv / (g["partition_ms_flushed_median"] * 1e-3) / 1e9, 1)
        # the decode kernel against the streaming-read probe (the practical HBM read ceiling)
        res["decode_kernel_vs_probe_read"] = round(res["roofline"]["achieved"] / g["probe_read_gbs"], 4)
        if a.config == "llama2_7b":
            import math
            lens = w.context_lens
            seq = W.build("llama2_7b_in_order", lens, w.n_q_heads, w.n_kv_heads, w.head_dim, w.dtype, w.seed,
                          num_blocks=w.num_blocks, data_mult=1.0 / math.sqrt(128.0), shuffle=False)
            t_seq = time_partitions_only(seq)
            res["shuffled_vs_in_order_throughput"] = round(t_seq / g["partition_ms_mean"], 4)
            del seq
    if a.copy_probe_bytes:
        run_copy_probe(a.copy_probe_bytes)
        res["copy_probe_bytes"] = a.copy_probe_bytes // 16 * 16
    if not a.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(w, a.cpu_budget)
    if not a.no_extras and a.config == "llama2_7b":
        del w
        res["configs"] = measure_side_configs(a.side_iters)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
