"""Benchmark of the compressed-KV hot path on one MI355X.

Workload (default): Llama-3-8B-shaped attention, 32 layers, batch 32, context
lengths uniform in [3072, 4096], 32 query / 8 KV heads, head_dim 128, TQ4 keys
(4-bit Lloyd-Max + 1-bit QJL) and values (4-bit), 16-token pages with random
non-contiguous block tables. The decode split count is the library's choice
(one split per (sequence, KV head) at this shape: the whole decode is one
launch; --splits 4 runs the pages' 4-way split instead). Every layer has its own
compressed cache (5.2 GB in all, far beyond the 256 MB last-level cache), filled
by compressing the whole synthetic context before timing.

One step = one decode step of the whole 32-layer stack: per layer, the newest
token's K and V compressed into its slot and the attention of the 32 sequences
over their compressed pages: fq_decode_step, one launch per layer at this shape.
--split-step enqueues its two halves instead (fq_step_prepare: append + query
preparation; fq_step_attend: the attention), --separate runs fq_compress +
fq_decode_attention per layer. value = batch / step time (decode tokens/s).
Inputs are resident in HBM before the timed region.

Also reported: the prefill compress rate (Mvectors/s) measured while filling
the caches, the roofline of the dominant kernel (the attention launch) and the
CPU oracle timed on a bounded sample of the same work.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--layers 32] [--splits S]
                    [--split-step | --separate] [--no-cpu]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "compressed-KV decode tokens/s & HBM GB/s (8B-shape, 4K ctx); compress Mvec/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_call_traffic.json")
DECODE_SRC = os.path.join(ROOT, "kv_cache_vector_tq4_amd", "csrc", "fq_decode.hip")


def measured_traffic(mode):
    """HBM bytes per timed launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE
    summary, or None when the decode source has changed since it was measured or it
    was measured for another step form."""
    import hashlib

    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
        with open(DECODE_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("decode_source_sha256") != sha or rec.get("bench_mode") != mode:
        return None
    return rec.get("bytes_per_launch")
HBM_PEAK_GBS = 8000.0
MFMA_FILE = os.path.join(ROOT, "profiles", "compress_mfma_util.json")
COMPRESS_SRC = os.path.join(ROOT, "kv_cache_vector_tq4_amd", "csrc", "fq_compress.hip")


def measured_mfma_util():
    """Matrix-core utilisation of the prefill compress kernels from the committed
    rocprofv3 counter summary, or None when the compress source has changed since."""
    import hashlib

    try:
        with open(MFMA_FILE) as f:
            rec = json.load(f)
        with open(COMPRESS_SRC, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("compress_source_sha256") != sha:
        return None
    return rec.get("kernels")


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=3)
    p.add_argument("--layers", type=int, default=32)
    p.add_argument("--splits", type=int, default=0,
                   help="decode splits per (sequence, KV head); 0 = the library's choice")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--no-graph", action="store_true", help="time eager launches instead of a HIP graph")
    p.add_argument("--separate", action="store_true",
                   help="per layer fq_compress of the newest tokens, then fq_decode_attention")
    p.add_argument("--split-step", action="store_true",
                   help="per layer fq_step_prepare, then fq_step_attend (the two halves of fq_decode_step)")
    p.add_argument("--no-extra", action="store_true", help="skip the other workloads' measurements")
    p.add_argument("--only", choices=ONLY, default=None,
                   help="measure one workload alone (for profiling its kernels); prints {only, result}")
    p.add_argument("--calibrate-copy", type=int, default=0, metavar="BYTES",
                   help="only run a plain device-to-device copy of BYTES (for scaling HBM byte counters)")
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(w, layer_seed, budget_s):
    """The oracle (unchanged) on a bounded sample: whole sequences of one layer, each
    one compress of the new token + decode over the oracle's own compressed pages."""
    import threadpoolctl

    from kv_cache_vector_tq4_amd import synth
    from oracle import attention, paged, pipeline

    oq = pipeline.build(4, 128)
    inp = synth.layer_inputs(synth.Workload("cpu-sample", 1, w.num_q_heads, w.num_kv_heads, 128,
                                            [w.seq_lens[0]], w.capacity_tokens), data_seed=layer_seed)
    L = int(inp["seq_lens"][0])
    cache = paged.empty_cache(inp["num_blocks"], w.num_kv_heads, 128, 4, qjl_dim=128)
    pipeline.compress(cache, inp["k"][0, :L], inp["v"][0, :L], inp["slot_mapping"][:L], oq)
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] + [1])

    def decode_rate(budget):
        n = 0
        t0 = time.perf_counter()
        while True:
            pipeline.compress(cache, inp["k"][0, L - 1:L], inp["v"][0, L - 1:L], inp["slot_mapping"][L - 1:L], oq)
            attention.decode_rotated(inp["q"], cache, inp["block_tables"], inp["seq_lens"], oq["levels"],
                                     oq["pi"], oq["s"], 4)
            n += 1
            if time.perf_counter() - t0 >= budget:
                break
        return n, time.perf_counter() - t0

    def compress_rate(budget):
        # whole-sequence compress of the sample's K and V (L tokens x 8 heads each)
        n = 0
        t0 = time.perf_counter()
        while True:
            pipeline.compress(cache, inp["k"][0, :L], inp["v"][0, :L], inp["slot_mapping"][:L], oq)
            n += 1
            if time.perf_counter() - t0 >= budget:
                break
        return n * 2 * L * w.num_kv_heads, time.perf_counter() - t0

    n, dt = decode_rate(budget_s * 0.6)
    nv, dtc = compress_rate(budget_s * 0.25)
    with threadpoolctl.threadpool_limits(limits=1):
        n1, dt1 = decode_rate(budget_s * 0.15)
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    per_seq_layer = dt / n
    return {
        "value": 1.0 / (per_seq_layer * w.layers),
        "unit": "tokens/s",
        "cores": cores,
        "kind": "oracle",
        "sample": "%d x (compress 1 new token + decode 1 sequence of %d tokens, 32 q / 8 kv heads, one layer) "
                  "in %.1f s; tokens/s = 1 / (seconds per sequence-layer x %d layers)" % (n, L, dt, w.layers),
        "single_thread_tokens_per_s": 1.0 / (dt1 / n1 * w.layers),
        "single_thread_sample": "%d decode samples in %.1f s with the BLAS pool limited to 1 thread" % (n1, dt1),
        "compress_mvec_per_s": nv / dtc / 1e6,
        "compress_sample": "%d K + V vectors (whole %d-token sequences x 8 heads) in %.1f s" % (nv, L, dtc),
        "cpu_model": model,
        "os_cpu_count": os.cpu_count(),
        "blas": [{k: i.get(k) for k in ("internal_api", "num_threads")} for i in info],
    }


GB = 1 << 30
MIN_SAMPLES = 50  # timed repetitions behind every median


def stats_ms(samples):
    """Median and p10 / p90 (ms) of per-call durations."""
    x = np.asarray(samples, np.float64)
    return {"median_ms": float(np.median(x)), "p10_ms": float(np.percentile(x, 10)),
            "p90_ms": float(np.percentile(x, 90)), "samples": int(x.size)}


def _events_samples(fn, reps, stream, per=1):
    """Durations (ms) of reps calls of fn() from HIP events recorded on the library's
    stream, each divided by per (the number of calls fn() enqueues)."""
    import torch

    out = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn()
        e1.record(stream)
        out.append((e0, e1))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) / per for a, b in out]


def _events_ms(fn, reps, stream):
    """Median duration (ms) of fn() from HIP events recorded on the library's stream."""
    return float(np.median(_events_samples(fn, reps, stream)))


def _capture(calls):
    """A HIP graph holding the given calls (captured on a side stream, replayed once)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for c in calls:
                c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    return g


EAGER = False  # --no-graph: time the call sequences eagerly (e.g. under a counter profiler)


def graph_stats(calls, stream, reps=MIN_SAMPLES):
    """Per-call device time: HIP events around reps replays of a graph holding the calls,
    each replay's time divided by the number of calls; median, p10, p90. With --no-graph
    the same sequence of calls is launched eagerly instead."""
    if EAGER:
        def seq():
            for c in calls:
                c()
        seq()
        return stats_ms(_events_samples(seq, reps, stream, per=len(calls)))
    g = _capture(calls)
    return stats_ms(_events_samples(g.replay, reps, stream, per=len(calls)))


def decode_layer_measure(index, bits, rot, stream, key_bits=None):
    """One decode layer of a workload, rotating through distinct cache replicas so that
    the reads come from HBM: at least 1 GiB of caches (4x the 256 MB last-level cache)."""
    import torch

    from kv_cache_vector_tq4_amd import fq, synth

    w = synth.workload(index, bits=bits)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    lens = np.asarray(w.seq_lens, np.int32)
    bt_np, nblocks = synth.block_tables(77 + index, w.seq_lens, w.capacity_tokens)
    slots = torch.from_numpy(np.concatenate([synth.slot_mapping_for(bt_np[b], int(lens[b]))
                                             for b in range(B)])).cuda()
    qz = fq.Quantizer(bits, d, rot, 1, 2, 128, key_bits=key_bits)
    per_cache = fq.PagedCache(1, Hkv, d, bits, 128, key_bits=key_bits).bytes_per_token_head() * int(lens.sum()) * Hkv
    replicas = int(min(256, max(2, math.ceil(GB / per_cache))))
    caches = []
    k, v = synth.kv_device(6000 + 17 * index, int(lens.sum()), Hkv, d)
    for r in range(replicas):
        c = fq.PagedCache(nblocks, Hkv, d, bits, 128, key_bits=key_bits)
        fq.compress(qz, c, k, v, slots)
        caches.append(c)
    del k, v
    bt = torch.from_numpy(bt_np).cuda()
    lt = torch.from_numpy(lens).cuda()
    q = torch.randn((B, Hq, d), device="cuda").to(torch.bfloat16)
    ws = torch.empty(fq.workspace_bytes(B, Hq, Hkv, d, 128, int(lens.max())), dtype=torch.uint8, device="cuda")
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    it = iter(range(10 ** 9))

    def call():
        fq.decode(qz, caches[next(it) % replicas], q, bt, lt, int(lens.max()), workspace=ws, out=out)

    for _ in range(3):
        call()
    ms_eager = _events_ms(call, MIN_SAMPLES, stream)
    # device time of a call: HIP events around replays of a graph holding one call per
    # replica (as for the stack's decode roofline; eager calls add host launch gaps)
    st = graph_stats([lambda c=c: fq.decode(qz, c, q, bt, lt, int(lens.max()), workspace=ws, out=out)
                      for c in caches], stream)
    ms = st["median_ms"]
    nbytes = int(lens.sum()) * Hkv * caches[0].bytes_per_token_head()
    return {"workload": w.name, "bits": bits, "key_bits": caches[0].key_bits, "rotation": "wht" if rot else "haar",
            "splits": fq.auto_splits(B, Hkv, int(lens.max())), "decode_ms": ms, "decode_ms_eager": ms_eager,
            "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"], "samples": st["samples"],
            "timing": "HIP events around graph replays of one call per cache replica (median over replays)",
            "achieved_gbs": nbytes / (ms * 1e-3) / 1e9, "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": nbytes, "cache_replicas": replicas,
            "rotated_bytes": replicas * nbytes}


def compress_layer_measure(index, rot, stream, bits=4, key_bits=None):
    """Prefill compress of one layer's whole context (K and V) of a workload; inputs and
    output caches rotate over at least 1 GiB so that neither sits in the last-level cache."""
    import torch

    from kv_cache_vector_tq4_amd import fq, synth

    w = synth.workload(index)
    Hkv, d = w.num_kv_heads, w.head_dim
    T = int(np.sum(w.seq_lens))
    qz = fq.Quantizer(bits, d, rot, 1, 2, 128, key_bits=key_bits)
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    nvec = 2 * T * Hkv
    probe = fq.PagedCache(1, Hkv, d, bits, 128, key_bits=key_bits)
    nbytes = nvec * d * 2 + T * 8 + T * Hkv * probe.bytes_per_token_head()
    reps = int(min(64, max(2, math.ceil(GB / nbytes))))
    pool = []
    for r in range(reps):
        k, v = synth.kv_device(8000 + index + 101 * r, T, Hkv, d)
        pool.append((k, v, fq.PagedCache((T + 15) // 16, Hkv, d, bits, 128, key_bits=key_bits)))
    st = graph_stats([lambda x=x: fq.compress(qz, x[2], x[0], x[1], slots) for x in pool], stream)
    ms = st["median_ms"]
    return {"workload": w.name, "rotation": "wht" if rot else "haar", "bits": bits, "key_bits": probe.key_bits,
            "vectors": nvec, "ms": ms, "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"], "samples": st["samples"],
            "timing": "HIP events around graph replays of one call per input / cache replica (median)",
            "replicas": reps, "rotated_bytes": reps * nbytes,
            "mvec_per_s": nvec / (ms * 1e-3) / 1e6, "achieved_gbs": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_bytes": nbytes}


def decompress_measure(qz, caches, slots, stream):
    """fq_decompress of a layer's stored tokens (K and V, bf16 out): one call per layer
    cache (each 144 MB of input) into three rotating output pairs (474 MB each), so the
    reads and writes of a call are not in the last-level cache; graph replays."""
    import torch

    from kv_cache_vector_tq4_amd import fq

    T, Hkv, d = slots.numel(), caches[0].num_kv_heads, caches[0].head_dim
    outs = [(torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=slots.device),
             torch.empty((T, Hkv, d), dtype=torch.bfloat16, device=slots.device)) for _ in range(3)]
    calls = [lambda i=i, c=c: fq.decompress(qz, c, slots, k_out=outs[i % 3][0], v_out=outs[i % 3][1])
             for i, c in enumerate(caches)]
    st = graph_stats(calls, stream, reps=max(2, MIN_SAMPLES // 8))
    ms = st["median_ms"]
    cache = caches[0]
    nvec = 2 * int((slots >= 0).sum().item()) * Hkv
    nbytes = nvec * (d * cache.bits // 8 + 4 + 2 * d) + 8 * T
    del outs
    return {"what": "fq_decompress of one layer's stored tokens, K and V, bf16 out (MSE reconstruction n Pi^T c)",
            "vectors": nvec, "ms": ms, "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"],
            "samples": st["samples"] * len(caches),
            "timing": "HIP events around graph replays of one call per layer cache (%d calls, median of replays)"
                      % len(caches),
            "mvec_per_s": nvec / (ms * 1e-3) / 1e6,
            "algorithmic_bytes": nbytes, "achieved_gbs": nbytes / (ms * 1e-3) / 1e9,
            "frac_hbm": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "bytes_per_vector": "codes %d + norm 4 in, %d out" % (d * cache.bits // 8, 2 * d)}


def window_measure(qz, cache, q, bt, lens, slots_np, W, reps, stream):
    """One decode step per layer with a W-token full-precision window (timed with events):
    fq_window_append of each sequence's newest token (the token W positions back goes
    from the ring into the compressed cache), then fq_decode_attention_window over the
    compressed tokens and the ring. Runs on a copy of the cache (the append writes it)."""
    import torch

    from kv_cache_vector_tq4_amd import fq

    B, Hq, d = q.shape
    Hkv = cache.num_kv_heads
    dev = q.device
    cw = fq.PagedCache(cache.num_blocks, Hkv, d, cache.bits, cache.qjl_dim, device=dev)
    for name, t in cache.fields().items():
        cw.fields()[name].copy_(t)
    g = torch.Generator(device=dev).manual_seed(4242)
    wk = torch.randn((B, W, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    wv = torch.randn((B, W, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    kn = torch.randn((B, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    vn = torch.randn((B, Hkv, d), generator=g, device=dev).to(torch.bfloat16)
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    pos = torch.from_numpy((lens - 1).astype(np.int64)).to(dev)
    ev = torch.from_numpy(np.array([slots_np[offs[b] + lens[b] - 1 - W] for b in range(B)], np.int64)).to(dev)
    lens_c = torch.from_numpy((lens - W).astype(np.int32)).to(dev)
    win_lens = torch.full((B,), W, dtype=torch.int32, device=dev)
    max_len = int(lens.max())
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    wsa = torch.empty(1 << 20, dtype=torch.uint8, device=dev)
    app = lambda: fq.window_append(qz, cw, kn, vn, pos, ev, wk, wv, workspace=wsa)
    def graph_us(fn, n=8):
        """Median GPU time (us) of fn() over replays of a HIP graph of n calls (no host gaps)."""
        fn()
        return graph_stats([fn] * n, stream)["median_ms"] * 1e3

    per_split = {}
    for sp in (1, 2, 4):
        ws = torch.empty(fq.workspace_bytes(B, Hq, Hkv, d, qz.qjl_dim, max_len, sp), dtype=torch.uint8, device=dev)
        per_split[sp] = graph_us(lambda: fq.decode_window(qz, cw, q, bt, lens_c, max_len, wk, wv, win_lens,
                                                          num_splits=sp, workspace=ws, out=out))
    ws1 = torch.empty(fq.workspace_bytes(B, Hq, Hkv, d, qz.qjl_dim, max_len, 1), dtype=torch.uint8, device=dev)
    no_win = torch.zeros((B,), dtype=torch.int32, device=dev)
    empty_us = graph_us(lambda: fq.decode_window(qz, cw, q, bt, lens_c, max_len, wk, wv, no_win, num_splits=1,
                                                 workspace=ws1, out=out))
    plain_us = graph_us(lambda: fq.decode(qz, cw, q, bt, lens_c, max_len, num_splits=1, workspace=ws1, out=out))
    append_us = graph_us(app)
    # the window step: the append and the one-split decode in one call (one launch)
    step_us = graph_us(lambda: fq.decode_step_window(qz, cw, kn, vn, pos, ev, wk, wv, win_lens, q, bt, lens_c,
                                                     max_len, num_splits=1, workspace=ws1, out=out))
    del cw
    return {"what": "per layer, batch 32: fq_window_append + fq_decode_attention_window, %d-token bf16 window, "
                    "the rest of each context compressed; step_us: both as one fq_decode_step_window call" % W,
            "timing": "HIP-graph replays (8 calls per graph; median of %d replays)" % MIN_SAMPLES,
            "window": W, "append_us": append_us, "decode_us_by_splits": per_split,
            "step_us": step_us, "append_plus_decode_us": append_us + per_split[1],
            "decode_us_empty_window_1_split": empty_us, "plain_decode_us_same_lengths": plain_us}


def prefill_measure(qz, cache, bt, lens, reps, stream):
    """Causal prefill attention of sequence 0 of the layer over its own cached tokens:
    one query token per position (q_lens = position + 1), fq_prefill_attention,
    timed with events around HIP-graph replays."""
    import torch

    from kv_cache_vector_tq4_amd import fq

    Hkv, d = cache.num_kv_heads, cache.head_dim
    Hq = 4 * Hkv
    L = int(lens[0])
    dev = bt.device
    g = torch.Generator(device=dev).manual_seed(777)
    q = torch.randn((L, Hq, d), generator=g, device=dev).to(torch.bfloat16)
    q_seq = torch.zeros(L, dtype=torch.int32, device=dev)
    q_lens = torch.arange(1, L + 1, dtype=torch.int32, device=dev)
    ws = torch.empty(fq.workspace_bytes(L, Hq, Hkv, d, qz.qjl_dim, L, 0), dtype=torch.uint8, device=dev)
    out = torch.empty((L, Hq, d), dtype=torch.float32, device=dev)
    fn = lambda: fq.prefill(qz, cache, q, q_seq, q_lens, bt, L, workspace=ws, out=out)
    fn()
    st = graph_stats([fn], stream, reps=reps)
    ms = st["median_ms"]
    attended = L * (L + 1) // 2
    return {"what": "causal prefill attention of one %d-token sequence over its compressed cache "
                    "(fq_prefill_attention, tiled: a wave per 16 query-head rows shares each page of its rows' "
                    "prefixes; query and output rotations as row GEMMs on the matrix cores)" % L,
            "queries": L, "q_heads": Hq, "ms": ms, "p10_ms": st["p10_ms"], "p90_ms": st["p90_ms"],
            "samples": st["samples"], "queries_per_s": L / (ms * 1e-3),
            "attended_token_heads_per_s": attended * Hkv / (ms * 1e-3),
            "cache_bytes_read_per_query_sum": attended * Hkv * cache.bytes_per_token_head()}


def attention_cosines(q, k, v, lens, kv_rows, out, seqs):
    """Cosine of the decode outputs against exact softmax attention over the
    uncompressed (bf16) K and V, per (sequence, query head), for sampled sequences.
    Reference arithmetic in fp32 with torch (measurement only)."""
    import torch

    Hq, d = q.shape[1], q.shape[2]
    Hkv = k.shape[1]
    G = Hq // Hkv
    cos = []
    for b in seqs:
        kb, vb = kv_rows(b)  # [len][Hkv][d] float32
        qb = q[b].float().view(Hkv, G, d)
        s = torch.matmul(qb, kb.permute(1, 2, 0).contiguous()) / np.sqrt(d)  # [Hkv][G][len]
        o = torch.matmul(torch.softmax(s, dim=-1), vb.permute(1, 0, 2).contiguous())  # [Hkv][G][d]
        ref = o.reshape(Hq, d)
        got = out[b]
        cos.append(torch.nn.functional.cosine_similarity(ref, got, dim=-1).cpu().numpy())
    c = np.concatenate(cos)
    return {"mean": float(c.mean()), "min": float(c.min()), "pairs": int(c.size)}


def variants_measure(stream):
    """The codebook variants on the batch-32 8B-shaped layer: 3-bit keys (+ QJL) and values,
    and the Prod budget at 4 bits (3-bit keys + QJL, 4-bit values): decode (the library's
    split choice) and prefill compress, each rotating over >= 1 GiB."""
    from kv_cache_vector_tq4_amd import fq

    out = {}
    for name, bits, kb in (("bits3", 3, 3), ("prod", 4, 3)):
        out[name] = {"decode": decode_layer_measure(2, bits, fq.ROT_HAAR, stream, key_bits=kb),
                     "compress": compress_layer_measure(2, fq.ROT_HAAR, stream, bits=bits, key_bits=kb)}
    return out


def stream_compress_measure(bits, layers, stream):
    """The 80-layer 70B-shaped prefill stream: every layer's 32768 tokens x 8 KV heads of K
    and V (bf16, generated on the device beforehand) compressed with that layer's
    quantizer. Inputs come from a pool of 8 layers' K/V (1.07 GB) and outputs go to a
    ring of caches of at least 1 GiB, both cycled, so that no layer finds its inputs or
    its outputs in the last-level cache; the 80 calls are one graph."""
    import torch

    from kv_cache_vector_tq4_amd import fq, synth

    T, Hkv, d = 32768, 8, 128
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    pool = [synth.kv_device(7000 + i, T, Hkv, d) for i in range(8)]
    per_out = fq.PagedCache(1, Hkv, d, bits, 128).bytes_per_token_head() * T * Hkv
    nc = int(math.ceil(GB / per_out))
    caches = [fq.PagedCache(T // 16, Hkv, d, bits, 128) for _ in range(nc)]
    quants = [fq.Quantizer(bits, d, fq.ROT_HAAR, 1 + layer, 2 + layer, 128) for layer in range(layers)]
    calls = [lambda l=l: fq.compress(quants[l], caches[l % nc], pool[l % 8][0], pool[l % 8][1], slots)
             for l in range(layers)]
    if EAGER:
        def run_all():
            for c in calls:
                c()
        run_all()
        tot = _events_samples(run_all, 5, stream)
    else:
        g = _capture(calls)
        tot = _events_samples(g.replay, 5, stream)
    total_ms = float(np.median(tot))
    nvec = 2 * layers * T * Hkv
    out_b = caches[0].bytes_per_token_head() * T * Hkv * layers
    in_b = 2 * layers * T * Hkv * d * 2 + layers * T * 8
    del pool, caches
    return {"layers": layers, "bits": bits, "vectors": nvec, "ms": total_ms,
            "ms_per_layer": total_ms / layers, "replays": len(tot),
            "p10_ms": float(np.percentile(tot, 10)), "p90_ms": float(np.percentile(tot, 90)),
            "timing": "HIP events around replays of a graph of the %d layers' fq_compress calls (median)" % layers,
            "mvec_per_s": nvec / (total_ms * 1e-3) / 1e6,
            "achieved_gbs": (in_b + out_b) / (total_ms * 1e-3) / 1e9,
            "frac_hbm": (in_b + out_b) / (total_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes": in_b + out_b}


ONLY = ("step", "step4", "c2", "c4_haar", "c4_wht", "c4_compress_haar", "c4_compress_wht", "c5_decode",
        "stream4", "stream2", "decompress", "window", "prefill", "bits3", "prod")


def main():
    args = parse()
    global EAGER
    EAGER = args.no_graph
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from kv_cache_vector_tq4_amd import fq, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda"
    if args.calibrate_copy:
        n = args.calibrate_copy // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_read": 4 * n, "calibrate_copy_bytes_written": 4 * n, "launches": 3}))
        return
    stream = torch.cuda.current_stream()
    if args.only and args.only not in ("step", "step4", "decompress", "window", "prefill"):
        # one other workload alone (for profiling its kernels)
        log("measuring %s alone..." % args.only)
        f = {"c2": lambda: decode_layer_measure(1, 4, fq.ROT_HAAR, stream),
             "c4_haar": lambda: decode_layer_measure(3, 4, fq.ROT_HAAR, stream),
             "c4_wht": lambda: decode_layer_measure(3, 4, fq.ROT_WHT, stream),
             "c4_compress_haar": lambda: compress_layer_measure(3, fq.ROT_HAAR, stream),
             "c4_compress_wht": lambda: compress_layer_measure(3, fq.ROT_WHT, stream),
             "c5_decode": lambda: decode_layer_measure(4, 2, fq.ROT_HAAR, stream),
             "stream4": lambda: stream_compress_measure(4, 80, stream),
             "stream2": lambda: stream_compress_measure(2, 80, stream),
             "bits3": lambda: variants_measure(stream)["bits3"],
             "prod": lambda: variants_measure(stream)["prod"]}[args.only]
        print(json.dumps({"only": args.only, "result": f()}), flush=True)
        return

    w = synth.workload(2)
    w.layers = args.layers
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    lens = np.asarray(w.seq_lens, np.int32)
    max_len = int(lens.max())
    splits = args.splits if args.splits > 0 else fq.auto_splits(B, Hkv, max_len)
    if args.only == "step4":
        splits = 4

    qz = fq.Quantizer(4, d, fq.ROT_HAAR, 1, 2, 128, device=dev)
    bt_np, nblocks = synth.block_tables(1234, w.seq_lens, w.capacity_tokens)
    bt = torch.from_numpy(bt_np).to(dev)
    lens_t = torch.from_numpy(lens).to(dev)
    slots_np = np.concatenate([synth.slot_mapping_for(bt_np[b], int(lens[b])) for b in range(B)])
    slots_all = torch.from_numpy(slots_np).to(dev)
    new_slots = torch.from_numpy(np.array([synth.slot_mapping_for(bt_np[b], int(lens[b]))[-1]
                                           for b in range(B)], np.int64)).to(dev)
    ntok = int(lens.sum())

    caches, qs, knew, vnew = [], [], [], []
    comp_ms = []
    log("filling %d layer caches (%d tokens x %d heads each)..." % (w.layers, ntok, Hkv))
    for layer in range(w.layers):
        cache = fq.PagedCache(nblocks, Hkv, d, 4, 128, device=dev)
        k, v = synth.kv_device(5000 + layer, ntok, Hkv, d, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fq.compress(qz, cache, k, v, slots_all)
        e1.record(stream)
        torch.cuda.synchronize()
        comp_ms.append(e0.elapsed_time(e1))
        g = torch.Generator(device=dev)
        g.manual_seed(9000 + layer)
        qs.append(torch.randn((B, Hq, d), generator=g, device=dev).to(torch.bfloat16))
        knew.append(k[-B:].contiguous())
        vnew.append(v[-B:].contiguous())
        caches.append(cache)
        del k, v
    torch.cuda.synchronize()
    if args.only in ("decompress", "window", "prefill"):
        log("measuring %s alone..." % args.only)
        f = {"decompress": lambda: decompress_measure(qz, caches, slots_all[slots_all >= 0].contiguous(), stream),
             "window": lambda: window_measure(qz, caches[0], qs[0], bt, lens, slots_np, 128, MIN_SAMPLES, stream),
             "prefill": lambda: prefill_measure(qz, caches[0], bt, lens, 10, stream)}[args.only]
        print(json.dumps({"only": args.only, "result": f()}), flush=True)
        return
    measure_parts = not args.only
    if measure_parts:
        log("decompress, residual window, prefill...")
        decomp = decompress_measure(qz, caches, slots_all[slots_all >= 0].contiguous(), stream)
        win = window_measure(qz, caches[0], qs[0], bt, lens, slots_np, 128, MIN_SAMPLES, stream)
        pre = prefill_measure(qz, caches[0], bt, lens, 10, stream)
    ws_bytes = fq.workspace_bytes(B, Hq, Hkv, d, 128, max_len, splits)
    # one workspace per layer: each keeps its layer's prepared queries, so the
    # attention launches can also be replayed on their own
    wss = [torch.empty(ws_bytes, dtype=torch.uint8, device=dev) for _ in range(w.layers)]
    outs = [torch.empty((B, Hq, d), dtype=torch.float32, device=dev) for _ in range(w.layers)]

    ev = []  # (start, end) events around each timed call (the attention part) in the timed steps
    mode = "separate" if args.separate else "split" if args.split_step else "step"

    def attend(layer, sp=None):
        sp = splits if sp is None else sp
        if mode == "separate":
            fq.decode(qz, caches[layer], qs[layer], bt, lens_t, max_len, num_splits=sp, workspace=wss[layer],
                      out=outs[layer])
        elif mode == "split":
            fq.step_attend(qz, caches[layer], B, Hq, bt, lens_t, max_len, wss[layer], num_splits=sp,
                           out=outs[layer])
        else:
            fq.decode_step(qz, caches[layer], knew[layer], vnew[layer], new_slots, qs[layer], bt, lens_t, max_len,
                           num_splits=sp, workspace=wss[layer], out=outs[layer])

    def prepare(layer):
        if mode == "separate":
            fq.compress(qz, caches[layer], knew[layer], vnew[layer], new_slots)
        elif mode == "split":
            fq.step_prepare(qz, caches[layer], knew[layer], vnew[layer], new_slots, qs[layer], max_len,
                            wss[layer], num_splits=splits)

    def step(record):
        for layer in range(w.layers):
            prepare(layer)
            if record:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
            attend(layer)
            if record:
                e1.record(stream)
                ev.append((e0, e1))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()

    graph = None
    graph_check = None
    if not args.no_graph:
        # The step is launch-bound (one or two launches per layer): capture it once, replay it.
        ref = [o.clone() for o in outs]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            with torch.cuda.graph(graph, stream=side):
                step(False)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        for _ in range(3):  # replays with eager work and syncs between them match eager output
            for o in outs:
                o.zero_()
            graph.replay()
            torch.cuda.synchronize()
            graph_check = max(float((o - r).abs().max()) for o, r in zip(outs, ref))
            assert graph_check == 0.0, "graph replay differs from eager: %g" % graph_check

    log("timing %d steps (%s)..." % (args.steps, "graph replay" if graph else "eager"))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step(False)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1000.0 / args.steps

    # per-launch durations of the dominant call: HIP events around each decode call,
    # on the stream the library launches on, over K eager steps (includes the host's
    # launch gaps between the call's kernels) ...
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    ms_eager = (time.perf_counter() - t1) * 1000.0 / args.steps
    dec_ms_eager = float(np.median([a.elapsed_time(b) for a, b in ev]))
    # ... and from HIP events around >= 50 replays of a graph holding only the layers'
    # attention launches (device time of the launch as the stack runs it; median and
    # p10 / p90 over replays), and one holding only the preparation launches
    dec_ms = dec_ms_eager
    dec_stats = None
    prep_ms = None
    if graph is not None:
        ref = [o.clone() for o in outs]
        dec_stats = graph_stats([lambda l=l: attend(l) for l in range(w.layers)], stream)
        dec_ms = dec_stats["median_ms"]
        assert all(torch.equal(o, r) for o, r in zip(outs, ref)), "attention replays differ from the step"
        if mode != "step":
            prep_ms = graph_stats([lambda l=l: prepare(l) for l in range(w.layers)], stream)["median_ms"]
    four = None
    if mode == "step" and splits != 4 and graph is not None and measure_parts:
        # the batch-32 configuration's own 4-way split, next to the library's choice
        ws4 = [torch.empty(fq.workspace_bytes(B, Hq, Hkv, d, 128, max_len, 4), dtype=torch.uint8, device=dev)
               for _ in range(w.layers)]
        o4 = [torch.empty_like(o) for o in outs]
        st4 = graph_stats([lambda l=l: fq.decode_step(qz, caches[l], knew[l], vnew[l], new_slots, qs[l], bt, lens_t,
                                                      max_len, num_splits=4, workspace=ws4[l], out=o4[l])
                           for l in range(w.layers)], stream)
        diff4 = max(float((a - b).abs().max()) for a, b in zip(o4, outs))
        lb4 = ntok * Hkv * caches[0].bytes_per_token_head() + B * Hkv * (2 * d * 2 + caches[0].bytes_per_token_head())
        four = dict(st4, what="fq_decode_step at 4 splits (prepare_queries + packed split attention + merge), "
                              "per layer", tokens_per_s=B / (w.layers * st4["median_ms"] * 1e-3),
                    achieved_gbs=lb4 / (st4["median_ms"] * 1e-3) / 1e9,
                    frac_hbm=lb4 / (st4["median_ms"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
                    max_abs_vs_one_split=diff4)
        del ws4, o4

    # accuracy: layer 0's outputs against exact attention over its uncompressed K / V
    # (the newest token of sequence b holds knew[0][b] / vnew[0][b], written by the step)
    k0, v0 = synth.kv_device(5000, ntok, Hkv, d, device=dev)
    offs = np.concatenate([[0], np.cumsum(lens)])

    def kv_rows(b):
        kb = k0[offs[b]:offs[b + 1]].float().clone()
        vb = v0[offs[b]:offs[b + 1]].float().clone()
        kb[-1] = knew[0][b].float()
        vb[-1] = vnew[0][b].float()
        return kb, vb

    accuracy = attention_cosines(qs[0], k0, v0, lens, kv_rows, outs[0], [0, 7, 15, 31])
    del k0, v0

    bpt = caches[0].bytes_per_token_head()  # 156 B at 4 bits with QJL keys
    dec_bytes = ntok * Hkv * bpt
    # the timed launch reads the layer's cache; in the one-launch step it also reads
    # the newest bf16 K and V (2 x 256 B per sequence and KV head) and writes their
    # records (bpt bytes each)
    launch_bytes = dec_bytes + (B * Hkv * (2 * d * 2 + bpt) if mode == "step" else 0)
    achieved = launch_bytes / (dec_ms * 1e-3) / 1e9
    comp_vec = 2 * ntok * Hkv
    comp_med_ms = float(np.median(comp_ms[1:] if len(comp_ms) > 1 else comp_ms))
    comp_bytes = ntok * Hkv * (2 * d * 2) + ntok * 8 + ntok * Hkv * bpt
    result = {
        "metric": METRIC,
        "value": B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "timing": {"mode": "hip graph replay" if graph is not None else "eager", "ms_per_step_eager": ms_eager,
                   "graph_vs_eager_max_abs": graph_check},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": "llama3-8b-shape attention stack: %d layers x (compress new token + decode: %s), batch %d, "
                        "ctx U[3072,4096] (sum %d), 32 q / 8 kv heads, d 128, TQ4 K(MSE+QJL)+V, 16-token pages, "
                        "%d splits" % (w.layers, {"separate": "fq_compress, fq_decode_attention",
                                                  "split": "fq_step_prepare, fq_step_attend",
                                                  "step": "fq_decode_step"}[mode], B, ntok, splits),
            "layers": w.layers, "batch": B, "context_tokens": ntok, "num_splits": splits,
            "cache_bytes_per_layer": dec_bytes, "bytes_per_token_head": bpt,
        },
        "roofline": {
            "kernel": {
                ("separate", True): "fq_decode_attention (one launch: packed_decode_kernel, query preparation and "
                                    "output rotation in-kernel)",
                ("separate", False): "fq_decode_attention (prepare_queries + packed split attention + merge_unrotate)",
                ("split", True): "fq_step_attend (one launch: packed_decode_kernel, queries prepared by "
                                 "fq_step_prepare, output rotation in-kernel)",
                ("split", False): "fq_step_attend (packed split attention + merge_unrotate)",
                ("step", True): "fq_decode_step (one launch: packed_decode_kernel appending the newest K/V token, "
                                "preparing the queries and rotating the output in-kernel)",
                ("step", False): "fq_decode_step (prepare_queries with the append + packed split attention + "
                                 "merge_unrotate)"}[(mode, splits == 1)],
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": measured_traffic(mode),
            "algorithmic_bytes_per_launch": launch_bytes,
            "avg_launch_ms": dec_ms,
            "launch_ms_p10": dec_stats["p10_ms"] if dec_stats else None,
            "launch_ms_p90": dec_stats["p90_ms"] if dec_stats else None,
            "launch_samples": dec_stats["samples"] if dec_stats else None,
            "timing": "median over %d replays of a graph of the %d layers' %s calls, HIP events on the library's "
                      "stream, per call" % (MIN_SAMPLES, w.layers, "fq_decode_step" if mode == "step" else "attention")
                      if graph is not None else "HIP events around eager calls (median)",
            "avg_launch_ms_eager": dec_ms_eager,
        },
        "step_4_splits": four,
        "step_parts": None if mode == "step" else {
            "prepare_ms": prep_ms,
            "prepare": ("fq_compress of the newest 32 x 8 K and V" if mode == "separate" else
                        "fq_step_prepare: newest 32 x 8 K and V compressed + queries prepared (one launch)"),
            "attend_ms": dec_ms,
            "timing": "HIP events around graph replays of the %d layers' calls of each part" % w.layers,
        },
        "compress": {
            "mvec_per_s": comp_vec / (comp_med_ms * 1e-3) / 1e6,
            "vectors_per_launch": comp_vec,
            "avg_launch_ms": comp_med_ms,
            "timing": "HIP events around each layer's fill (median of the layers after the first)",
            "achieved_gbs": comp_bytes / (comp_med_ms * 1e-3) / 1e9,
            "frac_hbm": comp_bytes / (comp_med_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes_per_launch": comp_bytes,
            "mfma_util": measured_mfma_util(),
        },
        "accuracy": dict(accuracy, what="cosine of decode outputs vs exact fp32 softmax attention over the "
                         "uncompressed bf16 K/V, layer 0, sequences 0 / 7 / 15 / 31, all 32 query heads"),
    }
    if measure_parts:
        result.update(decompress=decomp, residual_window=win, prefill=pre)
    if not args.no_extra and not args.only:
        del caches, knew, vnew, qs, outs, wss
        torch.cuda.empty_cache()
        log("other workloads: 70B-shape 32K decode and compress, 80-layer compress stream, batch-4 2-bit "
            "decode, batch-1 8B decode, 3-bit and Prod variants...")
        extra = {}
        extra["llama70b_b1_ctx32k_haar"] = decode_layer_measure(3, 4, fq.ROT_HAAR, stream)
        extra["llama70b_b1_ctx32k_wht"] = decode_layer_measure(3, 4, fq.ROT_WHT, stream)
        extra["stream_80layer_compress_4bit"] = stream_compress_measure(4, 80, stream)
        extra["stream_80layer_compress_2bit"] = stream_compress_measure(2, 80, stream)
        extra["b4_ctx32k_decode_2bit"] = decode_layer_measure(4, 2, fq.ROT_HAAR, stream)
        extra["llama8b_b1_ctx4k"] = decode_layer_measure(1, 4, fq.ROT_HAAR, stream)
        extra["llama70b_b1_ctx32k_compress_haar"] = compress_layer_measure(3, fq.ROT_HAAR, stream)
        extra["llama70b_b1_ctx32k_compress_wht"] = compress_layer_measure(3, fq.ROT_WHT, stream)
        extra.update(variants_measure(stream))
        result["other_workloads"] = extra
    if not args.no_cpu and not args.only:
        log("timing the CPU oracle (~%.0f s)..." % args.cpu_seconds)
        result["cpu_baseline"] = cpu_baseline(w, 77, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
