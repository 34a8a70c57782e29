"""Benchmark of the GQA attention library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--only-main]
                    [--no-cpu-baseline] [--graph]

A step is one attn_decode call (split kernel + combine kernel) over the whole
gqa_decode_ragged_bf16 workload (B=16, h_q=64, n_kv=8, d_h=128, ragged
L_b in [1024, 4096]).  With inputs resident in HBM, K steps are
launched back to back and timed by the host clock between two device
synchronisations; HIP events recorded on the launch stream at the two ends of
the same region give the device-side time.  The KV cache is held in several
copies that the steps rotate through, so the 256 MB Infinity Cache cannot
serve one step's reads from the previous step.  Before the W warmup steps of
each workload the GPU runs dense matrix products for 0.3 s, so the timed
steps do not start from the idle clock state.

value    = KV bytes per step / step time  (KV bytes = 2 * b * n_kv * d_h * sum L_b)
roofline = the split kernel, which reads the cache: KV bytes / its mean launch
           duration (event time of a region of K split launches / K), against
           the 8 TB/s HBM peak.
Also reported (same JSON line, "workloads"): the other decode workloads and
the causal prefill (TFLOP/s against the 2.5 PFLOP/s bf16 matrix peak), each
with its own roofline, and the fp64 CPU oracle timed on the host cores.
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from transformer_attention_gqa_amd import binding, inputs, roofline  # noqa: E402

METRIC = "GQA decode achieved HBM GB/s (% peak) + causal prefill TFLOP/s (% MFMA peak)"
MAIN = "gqa_decode_ragged_bf16"
MALL_BYTES = 256 << 20
COUNTERS = os.path.join(ROOT, "profiles", "counters.json")


def source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "transformer_attention_gqa_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel_key):
    """HBM bytes per launch from the committed counter runs, or None if absent
    or taken on a different kernel source."""
    try:
        data = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return None
    ent = data.get("kernels", {}).get(kernel_key)
    if not ent or ent.get("source_digest") != source_digest():
        return None
    return ent.get("hbm_bytes_per_launch")


def measured_mfma(kernel_key):
    """Matrix-core counters of a prefill kernel from the committed counter run
    (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES, SQ_BUSY_CYCLES, GRBM_GUI_ACTIVE), or
    nulls if absent or taken on a different kernel source."""
    none = {"mfma_busy": None, "clock_GHz": None}
    try:
        data = json.load(open(COUNTERS))
    except (OSError, ValueError):
        return none
    ent = data.get("kernels", {}).get(kernel_key)
    if not ent or ent.get("source_digest") != source_digest() or ent.get("mfma_busy") is None:
        return none
    return {"mfma_busy": ent["mfma_busy"], "clock_GHz": ent.get("clock_GHz")}


def precondition_gpu(seconds=0.3):
    """Run dense bf16 matrix products for about `seconds` so the GPU has left
    its idle clock state before the first warmup step (a few warmup steps of
    a 40 us decode would not get it there)."""
    a = torch.randn(4096, 4096, device="cuda", dtype=torch.bfloat16)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            torch.mm(a, a)
        torch.cuda.synchronize()
    del a


def measure_ceilings():
    """Reference rates measured on this GPU in the same run (context for the
    roofline fractions, which are taken against the vendor peaks): the
    library's read-only stream over 2 GiB (gqa_stream_read: every byte read
    once with the decode kernels' 128-bit non-temporal loads, nothing
    written), median of 10 timed passes, and an 8192^3 bf16 matrix product
    through the vendor BLAS."""
    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record()
        for i in range(reps):
            fn()
            ev[i + 1].record()
        torch.cuda.synchronize()
        ts = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e-3 for i in range(reps))
        return ts[len(ts) // 2], ts[0]
    nbytes = 2 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    t_read, t_read_min = timed(lambda: binding.gqa_stream_read(buf, sink), 10)
    del buf
    a = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    bm = torch.randn(8192, 8192, dtype=torch.bfloat16, device="cuda")
    t_mm, _ = timed(lambda: torch.mm(a, bm), 20)
    del a, bm
    torch.cuda.empty_cache()
    return {"stream_read_GBps": nbytes / t_read / 1e9,
            "stream_read_GBps_best": nbytes / t_read_min / 1e9,
            "bf16_gemm_TFLOPs": 2 * 8192 ** 3 / t_mm / 1e12,
            "note": "gqa_stream_read over 2 GiB (read-only, median and best of 10) and an 8192^3 bf16 "
                    "torch.mm (median of 20), same run"}


def step_distribution(step_fn, steps):
    """Per-step device times (ms) of `steps` back-to-back steps: HIP events
    recorded on the launch stream between consecutive steps, in a region of
    its own after the timed one.  Returns median, min and max."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(steps):
        step_fn(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ts = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    return {"median": ts[len(ts) // 2] if len(ts) % 2 else 0.5 * (ts[len(ts) // 2 - 1] + ts[len(ts) // 2]),
            "min": ts[0], "max": ts[-1], "n": steps}


def time_steps(step_fn, steps, warmup, use_graph=False):
    """Run `warmup` untimed steps, then time exactly `steps` steps.

    Returns (ms per step by the host clock between two device
    synchronisations, ms per step by HIP events recorded on the launch stream
    at the two ends of the same region).  With use_graph the steps are
    captured once into a HIP graph and the timed region is one replay."""
    for i in range(warmup):
        step_fn(i)
    torch.cuda.synchronize()
    if use_graph:
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                for i in range(steps):
                    step_fn(i)
        torch.cuda.synchronize()
        g.replay()  # untimed replay
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    if use_graph:
        g.replay()
    else:
        for i in range(steps):
            step_fn(i)
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) * 1e3 / steps, e0.elapsed_time(e1) / steps


def bench_decode(wl, steps, warmup, use_graph=False, n_split=0):
    dev = torch.device("cuda")
    x = inputs.make_decode_inputs(wl, device=dev)
    lens = x.seq_lens.cpu().tolist()
    kv_bytes = roofline.decode_kv_bytes(wl.kv_dtype, wl.n_kv, wl.d_h, lens)
    cache_bytes = x.k.numel() * x.k.element_size() * 2
    ncopies = min(16, max(2, math.ceil(4 * MALL_BYTES / cache_bytes) + 1))
    ks, vs = [x.k], [x.v]
    kss, vss = [x.k_scale], [x.v_scale]
    for _ in range(ncopies - 1):
        ks.append(x.k.clone())
        vs.append(x.v.clone())
        kss.append(None if x.k_scale is None else x.k_scale.clone())
        vss.append(None if x.v_scale is None else x.v_scale.clone())
    desc = binding.decode_desc(x.q, x.k, n_split)
    n_split_req = n_split
    n_split = binding.attn_decode_num_splits(desc)
    ws = torch.empty(binding.attn_decode_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x.q)

    # arguments checked and packed once per cache copy: a step is one ctypes call
    calls = [binding.prepare_decode(x.q, ks[c], vs[c], x.seq_lens, wl.scale, out, ws, k_scale=kss[c],
                                    v_scale=vss[c], n_split=n_split_req) for c in range(ncopies)]
    part_calls = [binding.prepare_decode_partials(x.q, ks[c], vs[c], x.seq_lens, wl.scale, ws, k_scale=kss[c],
                                                  v_scale=vss[c], n_split=n_split_req) for c in range(ncopies)]

    def step(i):
        calls[i % ncopies]()

    def partials(i):
        part_calls[i % ncopies]()

    ms_step, ev_ms = time_steps(step, steps, warmup, use_graph)
    dist = step_distribution(step, steps)
    # the split kernel (the one that reads the cache) over a region of its own
    _, kernel_ms = time_steps(partials, steps, 2, use_graph)

    key = f"decode_split_{wl.kv_dtype}:{wl.name}"
    achieved = kv_bytes / (kernel_ms * 1e-3) / 1e9
    traffic = measured_traffic(key)
    return {
        "workload": wl.name,
        "value": kv_bytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "ms_per_step": ms_step,
        "pct_hbm_peak": 100.0 * kv_bytes / (ms_step * 1e-3) / 1e9 / roofline.HBM_PEAK_GBPS,
        "kv_bytes": kv_bytes,
        "scale_bytes": roofline.decode_scale_bytes(wl.kv_dtype, wl.n_kv, lens),
        "sum_L": int(sum(lens)),
        "n_split": n_split,
        "kv_copies_rotated": ncopies,
        "event_ms_per_step": ev_ms,
        "step_ms": dist,
        "split_kernel_ms": kernel_ms,
        "combine_ms_approx": ev_ms - kernel_ms,
        "roofline": {"bound": "hbm", "kernel": "gqa_decode_split_mfma" if wl.kv_dtype != "f32"
                     else "gqa_decode_split_f32",
                     "achieved": achieved, "peak": roofline.HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / roofline.HBM_PEAK_GBPS, "traffic": traffic},
        "dtype": wl.kv_dtype,
        "config": {"workload": wl.name, "B": wl.B, "h_q": wl.h_q, "n_kv": wl.n_kv, "d_h": wl.d_h,
                   "S_max": wl.S_max, "q_dtype": wl.q_dtype, "kv_dtype": wl.kv_dtype, "seed": wl.seed},
    }


def bench_decode_paged(pwl, steps, warmup, use_graph=False):
    """attn_decode_paged over a decode workload whose cache is scattered over a
    page pool in a seeded random order.  Algorithmic bytes are those of the
    contiguous workload (the visible K/V rows); the block-table reads (4 bytes
    per page per (sequence, kv-head) range) are not counted."""
    wl = pwl.base
    dev = torch.device("cuda")
    x = inputs.make_paged_decode_inputs(wl, pwl.page_size, device=dev, keep_base=False)
    b = x.base
    lens = b.seq_lens.cpu().tolist()
    kv_bytes = roofline.decode_kv_bytes(wl.kv_dtype, wl.n_kv, wl.d_h, lens)
    pool_bytes = x.k_pages.numel() * x.k_pages.element_size() * 2
    ncopies = min(16, max(2, math.ceil(4 * MALL_BYTES / pool_bytes) + 1))
    kps, vps = [x.k_pages], [x.v_pages]
    for _ in range(ncopies - 1):
        kps.append(x.k_pages.clone())
        vps.append(x.v_pages.clone())
    desc = binding.paged_desc(b.q, x.k_pages, x.block_table)
    n_split = binding.attn_decode_paged_num_splits(desc)
    ws = torch.empty(binding.attn_decode_paged_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    out = torch.empty_like(b.q)
    calls = [binding.prepare_decode_paged(b.q, kps[c], vps[c], x.block_table, b.seq_lens, wl.scale, out, ws)
             for c in range(ncopies)]

    def step(i):
        calls[i % ncopies]()

    ms_step, ev_ms = time_steps(step, steps, warmup, use_graph)
    dist = step_distribution(step, steps)
    key = f"decode_split_paged_{wl.kv_dtype}:{pwl.name}"
    # a step is split + combine; the combine's share is taken from the
    # contiguous workload's launches of the same grid in the kernel trace
    achieved_step = kv_bytes / (ev_ms * 1e-3) / 1e9
    return {
        "workload": pwl.name,
        "value": kv_bytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "ms_per_step": ms_step,
        "pct_hbm_peak": 100.0 * kv_bytes / (ms_step * 1e-3) / 1e9 / roofline.HBM_PEAK_GBPS,
        "kv_bytes": kv_bytes,
        "sum_L": int(sum(lens)),
        "page_size": pwl.page_size,
        "num_pages": int(x.k_pages.shape[0]),
        "n_split": n_split,
        "kv_copies_rotated": ncopies,
        "event_ms_per_step": ev_ms,
        "step_ms": dist,
        "roofline": {"bound": "hbm", "kernel": "gqa_decode_split_mfma (paged) + gqa_decode_combine",
                     "achieved": achieved_step, "peak": roofline.HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": achieved_step / roofline.HBM_PEAK_GBPS, "traffic": measured_traffic(key)},
        "dtype": wl.kv_dtype,
        "config": {"workload": pwl.name, "B": wl.B, "h_q": wl.h_q, "n_kv": wl.n_kv, "d_h": wl.d_h,
                   "S_max": wl.S_max, "page_size": pwl.page_size, "q_dtype": wl.q_dtype,
                   "kv_dtype": wl.kv_dtype, "seed": wl.seed},
    }


def bench_decode_mla(wl, steps, warmup, use_graph=False):
    """attn_decode_mla (absorbed latent attention): a step reads the visible
    latent rows once (they are the keys and the values of every head)."""
    dev = torch.device("cuda")
    x = inputs.make_mla_inputs(wl, device=dev)
    lens = x.seq_lens.cpu().tolist()
    nbytes = roofline.mla_latent_bytes(wl.d_c, lens)
    cache_bytes = x.c_kv.numel() * x.c_kv.element_size()
    ncopies = min(16, max(2, math.ceil(4 * MALL_BYTES / cache_bytes) + 1))
    cs = [x.c_kv] + [x.c_kv.clone() for _ in range(ncopies - 1)]
    desc = binding.mla_desc(x.q, x.c_kv)
    ws = torch.empty(binding.attn_decode_mla_workspace_bytes(desc), dtype=torch.uint8, device=dev)
    out = torch.empty_like(x.q)
    calls = [binding.prepare_decode_mla(x.q, cs[c], x.seq_lens, wl.scale, out, ws) for c in range(ncopies)]
    part_calls = [binding.prepare_decode_mla_partials(x.q, cs[c], x.seq_lens, wl.scale, ws) for c in range(ncopies)]

    def step(i):
        calls[i % ncopies]()

    def partials(i):
        part_calls[i % ncopies]()

    ms_step, ev_ms = time_steps(step, steps, warmup, use_graph)
    dist = step_distribution(step, steps)
    _, kernel_ms = time_steps(partials, steps, 2, use_graph)
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    flops = roofline.mla_flops(wl.h_q, wl.d_c, lens)
    return {
        "workload": wl.name,
        "value": nbytes / (ms_step * 1e-3) / 1e9,
        "unit": "GB/s",
        "ms_per_step": ms_step,
        "pct_hbm_peak": 100.0 * nbytes / (ms_step * 1e-3) / 1e9 / roofline.HBM_PEAK_GBPS,
        "latent_bytes": nbytes,
        "sum_L": int(sum(lens)),
        "n_split": binding.attn_decode_mla_num_splits(desc),
        "kv_copies_rotated": ncopies,
        "event_ms_per_step": ev_ms,
        "step_ms": dist,
        "split_kernel_ms": kernel_ms,
        "combine_ms_approx": ev_ms - kernel_ms,
        "split_kernel_tflops": flops / (kernel_ms * 1e-3) / 1e12,
        "roofline": {"bound": "hbm", "kernel": "gqa_mla_decode_split", "achieved": achieved,
                     "peak": roofline.HBM_PEAK_GBPS, "unit": "GB/s", "frac": achieved / roofline.HBM_PEAK_GBPS,
                     "traffic": measured_traffic(f"mla_decode_split:{wl.name}")},
        "dtype": "bf16",
        "config": {"workload": wl.name, "B": wl.B, "h_q": wl.h_q, "d_c": wl.d_c, "S_max": wl.S_max,
                   "seed": wl.seed},
    }


def bench_prefill(wl, steps, warmup, use_graph=False):
    dev = torch.device("cuda")
    x = inputs.make_prefill_inputs(wl, device=dev)
    out = torch.empty_like(x.q)
    flops = roofline.prefill_causal_flops(wl.B, wl.S, wl.h_q, wl.d_h)

    call = binding.prepare_prefill_causal(x.q, x.k, x.v, wl.scale, out)

    def step(i):
        call()

    ms_step, k_ms = time_steps(step, steps, warmup, use_graph)  # one launch per step
    dist = step_distribution(step, steps)
    achieved = flops / (k_ms * 1e-3) / 1e12
    peak = roofline.MFMA_PEAK_TFLOPS["bf16"]
    ckey = f"prefill_causal:{wl.name}"
    return {
        "workload": wl.name,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "ms_per_step": ms_step,
        "pct_mfma_peak": 100.0 * flops / (ms_step * 1e-3) / 1e12 / peak,
        "causal_flops": flops,
        "io_bytes": roofline.prefill_io_bytes(wl.B, wl.S, wl.h_q, wl.n_kv, wl.d_h),
        "kernel_ms": k_ms,
        "step_ms": dist,
        "roofline": {"bound": "mfma", "kernel": "gqa_prefill_causal_kernel", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": measured_traffic(ckey),
                     **measured_mfma(ckey)},
        "dtype": "bf16",
        "config": {"workload": wl.name, "B": wl.B, "S": wl.S, "h_q": wl.h_q, "n_kv": wl.n_kv, "d_h": wl.d_h,
                   "seed": wl.seed},
    }


def bench_prefill_masked(wl, steps, warmup, use_graph=False):
    """attn_prefill with general masks; flops count only the visible (query,
    key) pairs (causal rule, key lengths and mask combined)."""
    dev = torch.device("cuda")
    x = inputs.make_masked_prefill_inputs(wl, device=dev)
    pairs = roofline.visible_pairs(wl.B, wl.S_q, wl.S_k, wl.causal, None if x.kv_lens is None else x.kv_lens.cpu(),
                                   None if x.mask is None else x.mask.cpu())
    flops = roofline.prefill_masked_flops(wl.h_q, wl.d_h, pairs)
    out = torch.empty(x.q.shape, dtype=torch.bfloat16, device=dev)
    ws = None
    if x.mask is not None:  # the key-tile bitmaps of the pass over the mask
        desc = binding._attn_desc(x.q, x.k, x.v, out, wl.causal, x.kv_lens, x.mask)
        ws = torch.empty(max(binding.attn_prefill_workspace_bytes(desc), 16), dtype=torch.uint8, device=dev)
    call = binding.prepare_prefill(x.q, x.k, x.v, wl.scale, out, causal=wl.causal, kv_lens=x.kv_lens, mask=x.mask,
                                   q_descale=x.q_descale, k_descale=x.k_descale, v_descale=x.v_descale,
                                   workspace=ws)

    def step(i):
        call()

    ms_step, k_ms = time_steps(step, steps, warmup, use_graph)
    dist = step_distribution(step, steps)
    achieved = flops / (k_ms * 1e-3) / 1e12
    peak = roofline.MFMA_PEAK_TFLOPS[wl.dtype]  # a contraction takes its own dtype's peak
    ckey = f"prefill_masked:{wl.name}"
    return {
        "workload": wl.name,
        "value": flops / (ms_step * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "ms_per_step": ms_step,
        "pct_mfma_peak": 100.0 * flops / (ms_step * 1e-3) / 1e12 / peak,
        "visible_pairs": pairs,
        "visible_flops": flops,
        "kernel_ms": k_ms,
        "step_ms": dist,
        "roofline": {"bound": "mfma", "kernel": ("gqa_prefill_fp8_kernel" if wl.dtype == "fp8"
                                                 else "gqa_prefill_masked_kernel")
                     + (" + gqa_mask_tiles_kernel" if x.mask is not None else ""), "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": measured_traffic(ckey),
                     **measured_mfma(ckey)},
        "dtype": wl.dtype,
        "config": {"workload": wl.name, "B": wl.B, "S_q": wl.S_q, "S_k": wl.S_k, "h_q": wl.h_q, "n_kv": wl.n_kv,
                   "d_h": wl.d_h, "causal": wl.causal, "kv_lens": wl.kv_lens, "mask": wl.mask, "dtype": wl.dtype,
                   "seed": wl.seed},
    }


def copy_calibration(nbytes=1 << 30, reps=3):
    """A plain elementwise kernel of known traffic (reads nbytes, writes nbytes)
    for scaling hardware byte counters: dst = -src over float32."""
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    return {"bytes_read": nbytes, "bytes_written": nbytes, "reps": reps}


def cpu_baseline(wl, budget_s=12.0):
    """The fp64 oracle, as it stands, on the host cores: full passes over the
    decode workload (stored-value decoding included), repeated until about
    `budget_s` seconds have elapsed; mean seconds per pass."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits

    cores = len(os.sched_getaffinity(0))
    x = inputs.make_decode_inputs(wl, device="cpu")
    lens = x.seq_lens.tolist()
    kv_bytes = roofline.decode_kv_bytes(wl.kv_dtype, wl.n_kv, wl.d_h, lens)
    with threadpool_limits(limits=cores):
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        passes, t0 = 0, time.perf_counter()
        while True:
            q = oracle.bf16_bits_to_f64(inputs.stored_numpy(x.q))
            k = oracle.bf16_bits_to_f64(inputs.stored_numpy(x.k))
            v = oracle.bf16_bits_to_f64(inputs.stored_numpy(x.v))
            oracle.decode(q, k, v, lens, wl.scale)
            passes += 1
            el = time.perf_counter() - t0
            if el >= budget_s or passes >= 50:
                break
    sec = el / passes
    return {"value": kv_bytes / sec / 1e9, "unit": "GB/s", "cores": blas_threads, "kind": "oracle",
            "sample": f"whole {wl.name} workload (B={wl.B}, h_q={wl.h_q}, sum L={sum(lens)}), bf16->fp64 "
                      f"decoding included; {passes} pass(es), {sec:.3f} s/pass; host cores available: {cores}",
            "seconds_per_pass": sec}


# ----------------------------------------------------------------------------
# rocprofv3 output -> profiles/
# ----------------------------------------------------------------------------
PROFILE_COMMANDS = {
    "trace": "rocprofv3 --kernel-trace --stats -d <out>/prof_trace -o run --output-format csv -- "
             "python3 bench.py --steps 20 --warmup 2 --no-cpu-baseline",
    "fetch": "rocprofv3 --pmc FETCH_SIZE --kernel-trace -d <out>/prof_fetch -o run --output-format csv -- "
             "python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --copy-calibration",
    "write": "rocprofv3 --pmc WRITE_SIZE --kernel-trace -d <out>/prof_write -o run --output-format csv -- "
             "python3 bench.py --steps 5 --warmup 1 --no-cpu-baseline --copy-calibration",
    "mfma": "rocprofv3 --pmc SQ_VALU_MFMA_BUSY_CYCLES SQ_BUSY_CYCLES GRBM_GUI_ACTIVE --kernel-trace "
            "-d <out>/prof_mfma -o run --output-format csv -- python3 bench.py --steps 5 --warmup 1 "
            "--no-cpu-baseline",
}
MFMA_COUNTERS = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE")
CALIB_GRID = (1 << 30) // 16  # threads of the calibration kernel (4 floats per thread)


def kernel_identity(name):
    """'void gqa::k<128, 1, false, 8>(gqa::Args)' -> ('k', ('128', '1', 'false', '8'))."""
    name = name.strip().replace("(anonymous namespace)::", "")
    if name.startswith("void "):
        name = name[5:]
    name = name.split("(")[0]
    base, _, targs = name.partition("<")
    targs = tuple(t.strip() for t in targs.rstrip(">").split(",")) if targs else ()
    return base.split("::")[-1].strip(), targs


PREFILL_PERSISTENT_WGS = 256  # the prefill kernels without a dense mask launch one workgroup per CU of an MI355X


def _workload_launches():
    """[((kernel, template args, grid threads), (counter key, workload, algorithmic bytes or flops, unit))].

    Mirrors the library's launch plan: the decode split kernel runs W
    workgroups of 512 threads (matrix-core paths) or 256 (float32 path); the
    combine kernel a grid of (slabs, ceil(heads_per_chunk * d / 4 / 256))
    workgroups of 256.  Two workloads can launch the same kernel with the same
    grid (the combine kernel of the ragged GQA and the long MQA decode); such
    launches are told apart by the workload whose unambiguous kernel ran last."""
    out = []
    kvf = {"bf16": "0", "fp8": "1", "int8": "2", "int4": "3"}  # template code of the cache format
    for wl in list(inputs.DECODE_WORKLOADS.values()) + list(inputs.QUANT_DECODE_WORKLOADS.values()):
        qd = torch.empty((wl.B, wl.h_q, wl.d_h), dtype={"f32": torch.float32, "bf16": torch.bfloat16}[wl.q_dtype],
                         device="meta")
        shape, cdt = inputs.code_shape(wl.kv_dtype, (wl.B, wl.n_kv, wl.S_max, wl.d_h)) \
            if wl.kv_dtype in inputs.QUANTIZED else ((wl.B, wl.n_kv, wl.S_max, wl.d_h),
                                                     {"f32": torch.float32, "bf16": torch.bfloat16}[wl.kv_dtype])
        kd = torch.empty(shape, device="meta", dtype=cdt)
        ns = binding.attn_decode_num_splits(binding.decode_desc(qd, kd))
        G = wl.h_q // wl.n_kv
        lens = inputs.draw_lengths(wl.B, *wl.lens, wl.seed).tolist()
        kv = roofline.decode_kv_bytes(wl.kv_dtype, wl.n_kv, wl.d_h, lens)
        key = f"decode_split_{wl.kv_dtype}:{wl.name}"
        hpc = 16 if (wl.kv_dtype == "f32" or G <= 16) else 32
        if wl.kv_dtype == "f32":
            out.append((("gqa_decode_split_f32", (str(wl.d_h), "false"), ns * 256), (key, wl.name, kv, "bytes")))
        else:
            targs = (str(wl.d_h), str(hpc // 16), kvf[wl.kv_dtype], "8", "false")
            out.append((("gqa_decode_split_mfma", targs, ns * 512), (key, wl.name, kv, "bytes")))
        n_slabs = wl.B * wl.n_kv * -(-G // hpc)
        grid = n_slabs * -(-(min(hpc, G) * wl.d_h // 4) // 256) * 256
        targs = (str(wl.d_h), "false" if wl.q_dtype == "f32" else "true")
        out.append((("gqa_decode_combine", targs, grid), (f"decode_combine:{wl.name}", wl.name, None, None)))
    for pwl in inputs.PAGED_WORKLOADS.values():
        wl = pwl.base
        G = wl.h_q // wl.n_kv
        hpc = 16 if G <= 16 else 32
        qd = torch.empty((wl.B, wl.h_q, wl.d_h), dtype=torch.bfloat16, device="meta")
        kd = torch.empty((wl.B, wl.n_kv, wl.S_max, wl.d_h), dtype=torch.bfloat16, device="meta")
        ns = binding.attn_decode_num_splits(binding.decode_desc(qd, kd))
        lens = inputs.draw_lengths(wl.B, *wl.lens, wl.seed).tolist()
        kv = roofline.decode_kv_bytes(wl.kv_dtype, wl.n_kv, wl.d_h, lens)
        targs = (str(wl.d_h), str(hpc // 16), kvf[wl.kv_dtype], "8", "true")
        out.append((("gqa_decode_split_mfma", targs, ns * 512),
                    (f"decode_split_paged_{wl.kv_dtype}:{pwl.name}", pwl.name, kv, "bytes")))
        n_slabs = wl.B * wl.n_kv * -(-G // hpc)
        grid = n_slabs * -(-(min(hpc, G) * wl.d_h // 4) // 256) * 256
        out.append((("gqa_decode_combine", (str(wl.d_h), "true"), grid),
                    (f"decode_combine:{pwl.name}", pwl.name, None, None)))
    for wl in inputs.MLA_WORKLOADS.values():
        qd = torch.empty((wl.B, wl.h_q, wl.d_c), dtype=torch.bfloat16, device="meta")
        cd = torch.empty((wl.B, wl.S_max, wl.d_c), dtype=torch.bfloat16, device="meta")
        ns = binding.attn_decode_mla_num_splits(binding.mla_desc(qd, cd))
        hpc = 64 if wl.h_q > 32 else 32
        lens = inputs.draw_lengths(wl.B, *wl.lens, wl.seed).tolist()
        out.append((("gqa_mla_decode_split", (str(wl.d_c), str(hpc // 32)), ns * 512),
                    (f"mla_decode_split:{wl.name}", wl.name, roofline.mla_latent_bytes(wl.d_c, lens), "bytes")))
        n_slabs = wl.B * -(-wl.h_q // hpc)
        grid = n_slabs * -(-(hpc * wl.d_c // 4) // 256) * 256
        out.append((("gqa_decode_combine", (str(wl.d_c), "true"), grid),
                    (f"decode_combine:{wl.name}", wl.name, None, None)))
    for wl in inputs.PREFILL_WORKLOADS.values():
        G = wl.h_q // wl.n_kv
        hc = math.gcd(G, 8)
        bm = 32 * (8 // hc)
        n_wg = wl.B * wl.n_kv * (G // hc) * (-(-wl.S // bm))
        grid = min(-(-n_wg // 8) * 8, PREFILL_PERSISTENT_WGS) * 512  # one workgroup per CU, looping over row blocks
        out.append((("gqa_prefill_causal_kernel", (str(wl.d_h), str(hc)), grid),
                    (f"prefill_causal:{wl.name}", wl.name, roofline.prefill_causal_flops(wl.B, wl.S, wl.h_q, wl.d_h),
                     "flops")))
    for wl in inputs.MASKED_PREFILL_WORKLOADS.values():
        G = wl.h_q // wl.n_kv
        hc = math.gcd(G, 8)
        bm = 32 * (8 // hc)
        n_wg = wl.B * wl.n_kv * (G // hc) * (-(-wl.S_q // bm))
        grid = -(-n_wg // 8) * 8  # with a dense mask one workgroup per row block, else one per CU
        grid = (grid if wl.mask else min(grid, PREFILL_PERSISTENT_WGS)) * 512
        lens = inputs.draw_lengths(wl.B, *wl.kv_lens, wl.seed) if wl.kv_lens else None
        mask = inputs.draw_mask(wl.mask, wl.B, wl.S_q, wl.S_k, wl.seed, wl.doc_lens) if wl.mask else None
        pairs = roofline.visible_pairs(wl.B, wl.S_q, wl.S_k, wl.causal, lens, mask)
        has_mask = "true" if wl.mask else "false"  # dense-mask instantiation of the kernel
        kname, targs = (("gqa_prefill_fp8_kernel", (str(wl.d_h), str(hc), has_mask)) if wl.dtype == "fp8"
                        else ("gqa_prefill_masked_kernel", (str(wl.d_h), str(hc), has_mask)))
        out.append(((kname, targs, grid),
                    (f"prefill_masked:{wl.name}", wl.name, roofline.prefill_masked_flops(wl.h_q, wl.d_h, pairs),
                     "flops")))
        if wl.mask:  # the pass over the mask: one workgroup of 512 per (row block, batch entry, bitmap word)
            words = min(-(-wl.S_k // (64 * 32)), 256)
            out.append((("gqa_mask_tiles_kernel", (str(bm),), -(-wl.S_q // bm) * wl.B * words * 512),
                        (f"mask_tiles:{wl.name}", wl.name, None, None)))
    return out


def mfma_utilisation(busy, gui_active, duration_ns, n_cu):
    """Matrix-core busy fraction and clock of one dispatch from rocprofv3
    counters.  GRBM_GUI_ACTIVE counts the GPU's busy cycles once per XCD
    (8 on MI355X), so per-XCD cycles are GRBM_GUI_ACTIVE / 8 and the clock is
    that over the kernel's duration; SQ_VALU_MFMA_BUSY_CYCLES sums the busy
    cycles of every SIMD's matrix core (4 per compute unit), so the busy
    fraction is it over 4 * n_cu * per-XCD cycles."""
    cycles = gui_active / 8.0
    return busy / (4.0 * n_cu * cycles), cycles / duration_ns


def _counter_rows(d):
    """rocprofv3 counter rows of a run -> {dispatch id: (kernel name, grid size, {counter: value})}."""
    import csv
    out = {}
    for f in os.listdir(d):
        if f.endswith("counter_collection.csv"):
            for r in csv.DictReader(open(os.path.join(d, f))):
                ent = out.setdefault(int(r["Dispatch_Id"]), (r["Kernel_Name"], int(r["Grid_Size"]), {}))
                ent[2][r["Counter_Name"]] = ent[2].get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return out


def summarize_profiles(trace_dir, fetch_dir, write_dir, dest, mfma_dir=None, n_cu=256):
    import csv
    import statistics

    def rows(d, suffix):
        for f in os.listdir(d):
            if f.endswith(suffix):
                return list(csv.DictReader(open(os.path.join(d, f))))
        raise FileNotFoundError(f"no *{suffix} in {d}")

    launches = _workload_launches()
    by_key = {}
    for key, ent in launches:
        by_key.setdefault(key, []).append(ent)
    info = {ent[0]: (key, ent) for key, ent in launches}  # counter key -> (launch key, entry)

    order = run_order(MAIN)

    def resolve(stream):
        """(launch key, row) in dispatch order -> (counter key, row) for our kernels.

        The default run times the workloads one after another in run_order(),
        each preceded by warm-up matrix products and its own input set-up, so
        the k-th unbroken run of library launches belongs to the k-th
        workload; that settles launches two workloads share (same kernel and
        grid)."""
        seg, in_ours = -1, False
        for key, r in stream:
            ents = by_key.get(key)
            if not ents:
                in_ours = False
                continue
            if not in_ours:
                seg, in_ours = seg + 1, True
            wname = order[seg] if seg < len(order) else None
            match = [e for e in ents if e[1] == wname]
            if match:
                yield match[0][0], r

    def ordered(rs):
        return sorted(rs, key=lambda r: int(r["Dispatch_Id"]))

    dur = {}
    trace = ordered(rows(trace_dir, "kernel_trace.csv"))
    for ckey, r in resolve(((*kernel_identity(r["Kernel_Name"]),
                             int(r["Grid_Size_X"]) * int(r["Grid_Size_Y"]) * int(r["Grid_Size_Z"])), r) for r in trace):
        dur.setdefault(ckey, []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    counters = {}
    for kind, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        calib = []
        crow = ordered(rows(d, "counter_collection.csv"))
        for r in crow:
            key = (*kernel_identity(r["Kernel_Name"]), int(r["Grid_Size"]))
            if key[0] == "vectorized_elementwise_kernel" and key[2] == CALIB_GRID and float(r["Counter_Value"]) > 1024:
                calib.append(float(r["Counter_Value"]))
        for ckey, r in resolve(((*kernel_identity(r["Kernel_Name"]), int(r["Grid_Size"])), r) for r in crow):
            counters.setdefault((kind, ckey), []).append(float(r["Counter_Value"]))
        counters[(kind, "scale")] = (1 << 20) / statistics.median(calib)  # KiB expected / KiB counted
    # matrix-core counters: per dispatch, joined with the same run's kernel trace for the duration
    mfma = {}
    gemm_check = None
    if mfma_dir:
        crows = _counter_rows(mfma_dir)
        trows = {int(r["Dispatch_Id"]): r for r in rows(mfma_dir, "kernel_trace.csv")}
        stream = []
        for did in sorted(crows):
            kname, grid, vals = crows[did]
            if did not in trows or any(c not in vals for c in MFMA_COUNTERS):
                continue
            t = trows[did]
            dt = int(t["End_Timestamp"]) - int(t["Start_Timestamp"])
            stream.append(((*kernel_identity(kname), grid), (vals, dt, kname)))
        for ckey, (vals, dt, _) in resolve(stream):
            mfma.setdefault(ckey, []).append((vals, dt))
        # the warm-up products (torch.mm of two 4096 x 4096 bf16 matrices) are a kernel of known
        # work: their counter-derived busy fraction against their timed flop rate checks the formula
        g = [(vals, dur) for (_, (vals, dur, kname)) in stream if kname.startswith("Cijk_") and dur > 0]
        if g:
            busy = statistics.median(mfma_utilisation(v["SQ_VALU_MFMA_BUSY_CYCLES"], v["GRBM_GUI_ACTIVE"], d,
                                                      n_cu)[0] for v, d in g)
            clk = statistics.median(mfma_utilisation(v["SQ_VALU_MFMA_BUSY_CYCLES"], v["GRBM_GUI_ACTIVE"], d,
                                                     n_cu)[1] for v, d in g)
            tfl = statistics.median(2 * 4096 ** 3 / (d * 1e-9) / 1e12 for v, d in g)
            gemm_check = {"kernel": "torch.mm 4096^3 bf16 (warm-up)", "dispatches": len(g), "mfma_busy": busy,
                          "clock_GHz": clk, "TFLOPs": tfl,
                          "TFLOPs_implied_by_busy": busy * roofline.MFMA_PEAK_TFLOPS["bf16"] * clk / 2.4}
    digest = source_digest()
    summary = {"source_digest": digest, "fetch_scale": counters[("FETCH_SIZE", "scale")],
               "write_scale": counters[("WRITE_SIZE", "scale")], "n_cu": n_cu, "mfma_counter_check": gemm_check,
               "kernels": {}}
    os.makedirs(dest, exist_ok=True)
    for ckey in sorted(info):
        key, (_, wname, algo, algo_unit) = info[ckey]
        if ckey not in dur:
            continue
        d = sorted(dur[ckey])
        fetch = counters.get(("FETCH_SIZE", ckey))
        write = counters.get(("WRITE_SIZE", ckey))
        fb = statistics.median(fetch) * 1024 * summary["fetch_scale"] if fetch else None
        wb = statistics.median(write) * 1024 * summary["write_scale"] if write else None
        ent = {"kernel": key[0], "template_args": list(key[1]), "workload": wname, "grid_threads": key[2],
               "launches": len(d),
               "mean_us": statistics.mean(d), "median_us": statistics.median(d), "min_us": d[0], "max_us": d[-1],
               "fetch_bytes_per_launch": fb, "write_bytes_per_launch": wb,
               "hbm_bytes_per_launch": (fb + wb) if fb is not None and wb is not None else None,
               "source_digest": digest}
        if algo_unit == "bytes":
            ent["algorithmic_bytes"] = algo
            ent["achieved_GBps_at_mean"] = algo / (ent["mean_us"] * 1e-6) / 1e9
            if fb:
                ent["fetch_over_algorithmic"] = fb / algo
        elif algo_unit == "flops":
            ent["algorithmic_flops"] = algo
            ent["achieved_TFLOPs_at_mean"] = algo / (ent["mean_us"] * 1e-6) / 1e12
        ent["mfma_busy"] = ent["clock_GHz"] = None
        if mfma.get(ckey):
            util = [mfma_utilisation(v["SQ_VALU_MFMA_BUSY_CYCLES"], v["GRBM_GUI_ACTIVE"], d, n_cu) for v, d in mfma[ckey]]
            ent["mfma_busy"] = statistics.median(u[0] for u in util)
            ent["clock_GHz"] = statistics.median(u[1] for u in util)
            ent["mfma_counters_median"] = {c: statistics.median(v[c] for v, _ in mfma[ckey]) for c in MFMA_COUNTERS}
            ent["mfma_run_duration_us_median"] = statistics.median(d for _, d in mfma[ckey]) * 1e-3
        summary["kernels"][ckey] = ent
        fname = os.path.join(dest, f"{key[0]}__{wname}.txt")
        with open(fname, "w") as f:
            f.write(f"kernel: {key[0]}<{', '.join(key[1])}>   workload: {wname}   grid threads: {key[2]}\n")
            f.write("commands (run from the repository root on one MI355X; <out> = output directory):\n")
            for k in ("trace", "fetch", "write"):
                f.write(f"  {PROFILE_COMMANDS[k]}\n")
            if mfma_dir:
                f.write(f"  {PROFILE_COMMANDS['mfma']}\n")
            f.write(f"kernel source digest: {digest}\n\n")
            f.write(f"kernel-trace: {len(d)} launches, mean {ent['mean_us']:.2f} us, median {ent['median_us']:.2f} us, "
                    f"min {ent['min_us']:.2f} us, max {ent['max_us']:.2f} us\n")
            if fb is not None:
                f.write(f"FETCH_SIZE: median {statistics.median(fetch):.0f} KiB/launch x scale "
                        f"{summary['fetch_scale']:.4f} = {fb / 1e6:.2f} MB\n")
            if wb is not None:
                f.write(f"WRITE_SIZE: median {statistics.median(write):.0f} KiB/launch x scale "
                        f"{summary['write_scale']:.4f} = {wb / 1e6:.2f} MB\n")
            f.write("(scales: a 1 GiB-read / 1 GiB-write elementwise kernel in the same runs, expected KiB / counted "
                    "KiB)\n")
            if algo_unit == "bytes":
                f.write(f"algorithmic KV bytes: {algo / 1e6:.2f} MB -> {ent['achieved_GBps_at_mean']:.0f} GB/s at the "
                        f"mean duration ({ent['achieved_GBps_at_mean'] / roofline.HBM_PEAK_GBPS * 100:.1f}% of 8 TB/s)\n")
                if fb:
                    f.write(f"fetched / algorithmic bytes: {fb / algo:.4f}\n")
            elif algo_unit == "flops":
                pk, pname = (5000.0, "5.0 PFLOP/s fp8") if "fp8" in key[0] else (2500.0, "2.5 PFLOP/s bf16")
                f.write(f"flops of the visible pairs: {algo:.4e} -> {ent['achieved_TFLOPs_at_mean']:.0f} TFLOP/s at "
                        f"the mean duration ({ent['achieved_TFLOPs_at_mean'] / pk * 100:.1f}% of {pname})\n")
            if ent["mfma_busy"] is not None:
                mc = ent["mfma_counters_median"]
                f.write(f"matrix cores busy: {ent['mfma_busy'] * 100:.1f}% of SIMD cycles at {ent['clock_GHz']:.2f} GHz "
                        f"(median over {len(mfma[ckey])} dispatches: SQ_VALU_MFMA_BUSY_CYCLES {mc['SQ_VALU_MFMA_BUSY_CYCLES']:.4g}"
                        f", GRBM_GUI_ACTIVE {mc['GRBM_GUI_ACTIVE']:.4g}, SQ_BUSY_CYCLES {mc['SQ_BUSY_CYCLES']:.4g}, "
                        f"{ent['mfma_run_duration_us_median']:.1f} us in that run; busy = MFMA cycles / "
                        f"(4 SIMDs x {n_cu} CUs x GRBM_GUI_ACTIVE / 8 XCDs))\n")
                if gemm_check:
                    f.write(f"counter check on the same run's torch.mm 4096^3 bf16: busy {gemm_check['mfma_busy'] * 100:.1f}% "
                            f"at {gemm_check['clock_GHz']:.2f} GHz implies {gemm_check['TFLOPs_implied_by_busy']:.0f} "
                            f"TFLOP/s; timed {gemm_check['TFLOPs']:.0f} TFLOP/s\n")
    json.dump(summary, open(os.path.join(dest, "counters.json"), "w"), indent=1)
    with open(os.path.join(dest, "all_kernels__bench_default_run.txt"), "w") as f:
        f.write(f"rocprofv3 --stats kernel summary of: {PROFILE_COMMANDS['trace']}\n")
        f.write("(all workloads of the default bench run, plus the dense matrix products that warm the GPU up "
                "before each workload; per-workload figures are in the <kernel>__<workload>.txt files)\n")
        f.write(f"kernel source digest: {digest}\n")
        f.write(f"{'calls':>6} {'total_ms':>10} {'mean_us':>10} {'min_us':>9} {'max_us':>9} {'pct':>6}  kernel\n")
        for r in rows(trace_dir, "kernel_stats.csv"):
            name = r["Name"] if len(r["Name"]) <= 110 else r["Name"][:107] + "..."
            f.write(f"{int(r['Calls']):6d} {float(r['TotalDurationNs']) / 1e6:10.3f} "
                    f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:9.2f} "
                    f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}  {name}\n")
    return summary


def all_workloads():
    return (list(inputs.DECODE_WORKLOADS) + list(inputs.QUANT_DECODE_WORKLOADS) + list(inputs.PAGED_WORKLOADS)
            + list(inputs.MLA_WORKLOADS) + list(inputs.PREFILL_WORKLOADS) + list(inputs.MASKED_PREFILL_WORKLOADS))


def run_order(main_name):
    """Workloads in the order one default run times them."""
    return [main_name] + [n for n in all_workloads() if n != main_name]


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=MAIN, choices=sorted(inputs.DECODE_WORKLOADS) + sorted(
        inputs.QUANT_DECODE_WORKLOADS) + sorted(inputs.PAGED_WORKLOADS) + sorted(inputs.MLA_WORKLOADS) + sorted(
        inputs.PREFILL_WORKLOADS) + sorted(inputs.MASKED_PREFILL_WORKLOADS))
    ap.add_argument("--only-main", action="store_true", help="skip the other workloads")
    ap.add_argument("--n-split", type=int, default=0, help="decode: force the number of key ranges (0 = library)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the copy / GEMM reference rates")
    ap.add_argument("--graph", action="store_true", help="time one HIP-graph replay of the K steps instead of "
                    "K eager launches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a 1 GiB read + 1 GiB write elementwise kernel (counter calibration)")
    ap.add_argument("--summarize", nargs="+", metavar="DIR",
                    help="TRACE_DIR FETCH_DIR WRITE_DIR [MFMA_DIR]: turn rocprofv3 output directories into "
                         "profiles/ summaries and exit")
    args = ap.parse_args(argv)
    if args.summarize:
        if len(args.summarize) not in (3, 4):
            ap.error("--summarize takes 3 or 4 directories")
        s = summarize_profiles(*args.summarize[:3], dest=os.path.join(ROOT, "profiles"),
                               mfma_dir=args.summarize[3] if len(args.summarize) == 4 else None)
        print(json.dumps({k: {kk: vv for kk, vv in v.items() if kk in ("mean_us", "hbm_bytes_per_launch")}
                          for k, v in s["kernels"].items()}, indent=1))
        return 0

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this library has no multi-GPU path (each GPU would run its own "
              "share of sequences/heads independently); run with --gpus 1", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    binding.load_library()
    props = torch.cuda.get_device_properties(0)
    use_graph = args.graph
    if args.copy_calibration:
        print(f"[bench] copy calibration {copy_calibration()}", file=sys.stderr, flush=True)

    def run(name, steps, warmup):
        print(f"[bench] {name} steps={steps} warmup={warmup}", file=sys.stderr, flush=True)
        precondition_gpu()
        if name in inputs.PREFILL_WORKLOADS:
            return bench_prefill(inputs.PREFILL_WORKLOADS[name], steps, warmup, use_graph)
        if name in inputs.PAGED_WORKLOADS:
            return bench_decode_paged(inputs.PAGED_WORKLOADS[name], steps, warmup, use_graph)
        if name in inputs.MLA_WORKLOADS:
            return bench_decode_mla(inputs.MLA_WORKLOADS[name], steps, warmup, use_graph)
        if name in inputs.MASKED_PREFILL_WORKLOADS:
            return bench_prefill_masked(inputs.MASKED_PREFILL_WORKLOADS[name], steps, warmup, use_graph)
        wl = {**inputs.DECODE_WORKLOADS, **inputs.QUANT_DECODE_WORKLOADS}[name]
        return bench_decode(wl, steps, warmup, use_graph, args.n_split)

    ceilings = None
    if not args.no_ceilings:
        print("[bench] measured ceilings", file=sys.stderr, flush=True)
        ceilings = measure_ceilings()

    def vs_ceiling(res):
        # decode: the step's and the split kernel's bytes/s as a share of the read-only stream in this run
        if ceilings and res.get("unit") == "GB/s":
            res["pct_of_measured_read_ceiling"] = 100.0 * res["value"] / ceilings["stream_read_GBps"]
            res["roofline"]["frac_of_measured_read_ceiling"] = res["roofline"]["achieved"] / ceilings[
                "stream_read_GBps"]
        if ceilings and res.get("unit") == "TFLOP/s" and res.get("dtype") == "bf16":
            res["pct_of_measured_gemm"] = 100.0 * res["value"] / ceilings["bf16_gemm_TFLOPs"]
        return res

    main_res = vs_ceiling(run(args.workload, args.steps, args.warmup))
    others = {}
    if not args.only_main:
        for name in run_order(args.workload)[1:]:
            others[name] = vs_ceiling(run(name, max(5, min(args.steps, 20)), 2))
            torch.cuda.empty_cache()

    line = {
        "metric": METRIC,
        "value": main_res["value"],
        "unit": main_res["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_res["dtype"],
        "data": "synthetic",
        "config": main_res["config"],
        "roofline": main_res["roofline"],
        "timing": "one hip-graph replay of K steps" if use_graph else "K eager launches",
        "device": {"name": props.name, "gcn_arch": getattr(props, "gcnArchName", ""),
                   "cus": props.multi_processor_count},
        "main": {k: v for k, v in main_res.items() if k not in ("config", "roofline")},
        "workloads": others,
    }
    if ceilings:
        line["measured_ceilings"] = ceilings
    if not args.no_cpu_baseline and args.workload in inputs.DECODE_WORKLOADS:
        print("[bench] cpu baseline (fp64 oracle)", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(inputs.DECODE_WORKLOADS[args.workload])
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
