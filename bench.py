"""Throughput of the block-paged KV cache hot path on one MI355X.

A step is one pass of the whole path over one synthetic batch (one layer):
slot mapping of the new tokens, store of their K/V rows into the page pools,
then paged decode attention of every sequence (partition + reduce kernels).
A plain decode step (one new token per sequence, stored at ctx-1) runs as the
fused hpkv_paged_attention_decode_step, which stores the row inside the decode
launch; --unfused times the three separate calls instead.
Default workload: the Llama-2-7B-shaped layer (Hq = Hkv = 32, d = 128,
16-token pages, 64 sequences with ctx ~ U{512..4096}, bf16, u32 tables), one
new token per sequence stored at position ctx-1 before decoding.

Timing protocol (cold caches): before every timed call a 1 GiB scratch
buffer is written, outside the timed interval, so no K/V byte can be served
from the L2s or the 256 MB Infinity Cache; each call is bracketed by its own
pair of HIP events on the launch stream, and the median over the calls is
reported (mean, min and max beside it). --warm times back-to-back calls
without the scratch writes instead; the warm back-to-back figure is printed
beside the cold one in any case.

Printed: ONE JSON line with
  value        KV bytes the decode must read per step (sum ctx * 2 * Hkv * d * b)
               divided by the median step time, in GB/s (1e9 B/s);
  roofline     the partition pass alone (the dominant work: a one-workgroup
               ordering kernel of a few microseconds, then the partition
               kernel), timed per launch as above: algorithmic bytes per
               launch (KV + q + out + block-table entries + lengths) over its
               median duration, against the 8 TB/s HBM peak;
  ceilings     the library's read-ceiling kernel (hpkv_read_ceiling) on a
               buffer the size of the step's K/V: a plain streaming read and
               the decode's row patterns (one head's 256-byte rows and two
               heads' 512-byte rows at an 8 KiB and a 2 KiB stride), each
               timed like the kernels;
  cpu_baseline the CPU oracle (double precision, plain loops) running the same
               step on host copies of the same inputs, repeated for about ten
               seconds and timed on the host (median per step).
Inputs are resident in HBM before timing starts; nothing is skipped inside the
timed region.

--path prefill times causal chunked-prefill attention instead (default
workload: the prefix-sharing batch, 512 sequences whose tails are written in
three chunks): a step is, per chunk, slot mapping + store of the chunk's K/V
rows + hpkv_paged_attention_prefill of its queries. value is the causal
attention flops of the step (4 * d * Hq * (p + 1) per query position p) over
the step time in TFLOP/s; roofline is the prefill kernel alone against the
dense 16-bit matrix-core peak; cpu_baseline runs the oracle on sampled rows.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0
MFMA16_PEAK_TFLOPS = 2500.0  # dense bf16 / f16 matrix-core peak
PREFILL_METRIC = "paged chunked-prefill attention: achieved TFLOP/s (causal flops)"
METRIC = "paged decode: achieved KV HBM GB/s (% of peak) + sequences/s per layer"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_traffic.json")
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_hpkv_amd", "csrc", "hpkv_decode.hip")
QUANT_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_quant_traffic.json")
PREFILL_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_traffic.json")
PREFILL_SRC = os.path.join(ROOT, "paged_kv_cache_hpkv_amd", "csrc", "hpkv_prefill.hip")

WORKLOAD_TEXT = {
    "llama7b": "Llama-2-7B-shaped layer decode step: Hq=Hkv=32, d=128, bs=16, 64 seqs, "
               "ctx~U{512..4096}",
    "gqa": "GQA layer decode step: Hq=32, Hkv=8, d=128, bs=16, 256 seqs, ctx log-U[128,8192]",
    "qwen3": "Qwen3-0.6B-shaped layer decode step: Hq=16, Hkv=8, d=128, bs=256, 128 seqs, "
             "ctx~U{1..16384}, 5% dropped slots",
    "prefix": "prefix-sharing layer: 32 groups x 16 seqs share 2048-token prefixes, chunked "
              "prefill of U{64..1024}-token tails, then decode",
    "tiny": "tiny fp32 step: bs=4, Hq=4, Hkv=2, d=8, ctx [1,4,11]",
}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--path", default="decode", choices=["decode", "prefill"])
    p.add_argument("--workload", default=None, choices=sorted(workloads.WORKLOADS))
    p.add_argument("--dtype", default=None, choices=["bf16", "f16", "f32"])
    p.add_argument("--index", default=None, choices=["u32", "u64"])
    p.add_argument("--roofline-launches", type=int, default=50)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--unfused", action="store_true",
                   help="run slot mapping, store and decode as separate calls")
    p.add_argument("--shared", action="store_true",
                   help="decode with hpkv_paged_attention_decode_shared (a full partition that "
                        "consecutive sequences alias is read once for all of them); the "
                        "roofline then times that whole call")
    p.add_argument("--kv", default=None, choices=["i8", "fp8"],
                   help="decode over quantized pools (per page-slot, per KV head scales)")
    p.add_argument("--graph", action="store_true",
                   help="decode path: time the step as a HIP graph replay (captured once "
                        "after the warmup; the roofline leg stays a direct call)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (for HBM counter calibration)")
    p.add_argument("--warm", action="store_true",
                   help="time back-to-back calls without clearing the caches in between")
    p.add_argument("--no-ceiling", action="store_true",
                   help="skip the read-ceiling measurement")
    p.add_argument("--ceiling", action="store_true",
                   help="only measure the read ceilings (streaming and the decode's row "
                        "pattern) on a buffer of the workload's K/V size")
    p.add_argument("--cpu-seconds", type=float, default=10.0,
                   help="host time the cpu_baseline repeats the oracle for")
    return p.parse_args()


SCRATCH_BYTES = 1 << 30


class Timer:
    """Per-call HIP-event timing on one stream. With cold=True a 1 GiB scratch buffer is
    written before every call, outside its events, evicting the L2s and the 256 MB
    Infinity Cache."""

    def __init__(self, dev, stream, cold=True):
        self.stream = stream
        self.cold = cold
        self.scratch = torch.empty(SCRATCH_BYTES, dtype=torch.uint8, device=dev) if cold else None
        self.k = 0

    def flush(self):
        if self.scratch is not None:
            self.k ^= 1
            self.scratch.fill_(self.k)

    def time(self, fn, n):
        """Times n calls of fn; returns per-call statistics in ms and the wall time."""
        starts = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        ends = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            self.flush()
            starts[i].record(self.stream)
            fn()
            ends[i].record(self.stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        d = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)], dtype=np.float64)
        return dict(median_ms=float(np.median(d)), mean_ms=float(d.mean()),
                    min_ms=float(d.min()), max_ms=float(d.max()), wall_s=wall, n=n)

    def warm(self, fn, n):
        """Mean ms per call of n back-to-back calls (no cache clearing), one event pair."""
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(self.stream)
        for _ in range(n):
            fn()
        e1.record(self.stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    def protocol(self):
        if self.cold:
            return ("cold caches: 1 GiB scratch write before each call, outside its HIP event "
                    "pair; median over the calls")
        return "warm: back-to-back calls, each with its own HIP event pair; median"


def ceilings(dev, timer, nbytes, launches=20):
    """HBM read ceilings on a buffer of about nbytes (hpkv_read_ceiling), GB/s (median):
    a plain streaming read; one head row (256 B at d=128 bf16) of every token at the
    8 KiB and 2 KiB token strides of 32 and 8 KV heads; and two adjacent heads' 512 B,
    the rows the two-head decode workgroups read."""
    import paged_kv_cache_hpkv_amd as hpkv
    stride_max = 8192
    nbytes = max(stride_max, nbytes // stride_max * stride_max)
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(3)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    out = {}
    for name, row, stride, rows_per_wg in (("stream", 4096, 4096, 64),
                                          ("rows256_stride8k", 256, 8192, 512),
                                          ("rows256_stride2k", 256, 2048, 512),
                                          ("rows512_stride8k", 512, 8192, 512),
                                          ("rows512_stride2k", 512, 2048, 512)):
        def fn():
            hpkv.hpkv_read_ceiling(buf, row, stride, rows_per_wg, sink)
        fn()
        st = timer.time(fn, launches)
        read = nbytes // stride * stride
        out[name] = dict(gbs=round(read / (st["median_ms"] * 1e-3) / 1e9, 1),
                         median_ms=round(st["median_ms"], 5), bytes=read,
                         row_bytes=row, stride_bytes=stride, rows_per_workgroup=rows_per_wg)
    del buf
    out["launches_each"] = launches
    out["protocol"] = timer.protocol()
    return out


def make_workload(args):
    name = args.workload or ("prefix" if args.path == "prefill" else "llama7b")
    w = workloads.WORKLOADS[name]()
    if args.dtype:
        w = w.with_dtype(args.dtype)
    if args.index:
        w = w.with_index(args.index)
    return w


def is_decode_step(w):
    """One new token per sequence at position ctx-1 and no dropped slots."""
    if len(w.chunks) != 1 or w.drop_mask is not None:
        return False
    start, cu = w.chunks[0]
    return bool(np.all(w.context_lens > 0) and np.array_equal(cu, np.arange(w.num_seqs + 1))
                and np.array_equal(start, w.context_lens - 1))


class Step:
    """Pre-allocated device state for repeated steps of one workload.

    A decode step (one new token per sequence at ctx-1) runs as the fused
    hpkv_paged_attention_decode_step; any other step (chunked prefill, dropped
    slots) or --unfused runs hpkv_slot_mapping, hpkv_store_kvcache and
    hpkv_paged_attention_decode.
    """

    def __init__(self, w, t, fused, shared=False):
        import paged_kv_cache_hpkv_amd as hpkv
        self.hpkv, self.w, self.t = hpkv, w, t
        self.fused = fused and not shared
        self.shared = shared
        dev = t.q.device
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.sp = torch.from_numpy(w.seq_ptr).to(dev)
        self.ctx = torch.from_numpy(w.context_lens).to(dev)
        self.chunks = [(torch.from_numpy(s).to(dev), torch.from_numpy(c).to(dev),
                        torch.empty(int(c[-1]), dtype=torch.int64, device=dev))
                       for s, c in w.chunks]
        self.drop = None if w.drop_mask is None else torch.from_numpy(w.drop_mask).to(dev)
        self.out = torch.empty_like(t.q)
        self.ws = hpkv.alloc_workspace(t.q, t.k_cache, w.max_context_len)

    def __call__(self):
        h, w, t = self.hpkv, self.w, self.t
        if self.fused:
            h.hpkv_paged_attention_decode_step(
                t.q, t.new_keys[0], t.new_values[0], t.k_cache, t.v_cache, self.bt, self.sp,
                self.ctx, w.scale, w.max_context_len, self.ws, self.out,
                slots_out=self.chunks[0][2])
            return
        for c, (start, cu, slots) in enumerate(self.chunks):
            h.hpkv_slot_mapping(self.bt, self.sp, w.page_size, w.num_pages, start, cu, slots)
            if self.drop is not None and c == 0:
                slots.masked_fill_(self.drop, -1)
            h.hpkv_store_kvcache(t.new_keys[c], t.new_values[c], t.k_cache, t.v_cache, slots)
        decode = (h.hpkv_paged_attention_decode_shared if self.shared
                  else h.hpkv_paged_attention_decode)
        decode(t.q, t.k_cache, t.v_cache, self.bt, self.sp, self.ctx, w.scale,
               w.max_context_len, self.ws, self.out)

    def partitions_only(self):
        w, t = self.w, self.t
        if self.shared:  # the detection, ordering, partition and reduce kernels
            self.hpkv.hpkv_paged_attention_decode_shared(
                t.q, t.k_cache, t.v_cache, self.bt, self.sp, self.ctx, w.scale,
                w.max_context_len, self.ws, self.out)
            return
        self.hpkv.hpkv_paged_attention_decode_partitions(
            t.q, t.k_cache, t.v_cache, self.bt, self.sp, self.ctx, w.scale, w.max_context_len,
            self.ws, self.out)


def algorithmic_decode_bytes(w):
    """Bytes the partition kernel must move from HBM: KV rows, q, out, table entries,
    lengths. A pool row that several sequences alias (shared prefix pages) has to come from
    HBM only once, so the KV term counts distinct rows; without aliasing that is the
    logical sum(ctx) * 2 * Hkv * d * b."""
    b = torch.tensor([], dtype=w.torch_dtype).element_size()
    idx = w.block_table.dtype.itemsize
    ctx = w.context_lens.astype(np.int64)
    pages = -(-ctx // w.page_size)
    per_seq = 2 * w.num_q_heads * w.head_dim * b + 4 + 2 * idx
    return int(w.kv_bytes_unique_rows() + pages.sum() * idx + per_seq * w.num_seqs)


def recorded_traffic(w, traffic_file=TRAFFIC_FILE, src=DECODE_SRC, variant=""):
    """HBM bytes per launch of the dominant kernel from committed counter runs, if the
    kernel source has not changed since they were taken (variant: "/shared" for the
    shared decode's record)."""
    try:
        with open(traffic_file) as f:
            rec = json.load(f)
        with open(src, "rb") as f:
            src_hash = hashlib.sha256(f.read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != src_hash:
        return None  # the kernel changed since the counters were taken
    return rec.get("workloads", {}).get(f"{w.name}/{w.dtype}/{w.index}{variant}")


def host_description():
    """CPU model and the core counts the host reports."""
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}; nproc {len(os.sched_getaffinity(0))}, os.cpu_count {os.cpu_count()}"


def cpu_baseline(w, t, out_gpu, seconds):
    """The oracle on the same step (host copies), repeated for about `seconds`."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from paths import decode_errors, host_bits, host_threads, oracle_step  # noqa: E402
    # host copies of the step's inputs (the store already ran on the GPU, so
    # the pools hold the post-store state; the oracle's store rewrites the
    # same rows with the same bits)
    h = dict(q=host_bits(t.q), k_cache=host_bits(t.k_cache), v_cache=host_bits(t.v_cache),
             new_keys=[host_bits(x) for x in t.new_keys],
             new_values=[host_bits(x) for x in t.new_values])
    threads = host_threads()
    runs = []
    t_start = time.perf_counter()
    while not runs or (time.perf_counter() - t_start < seconds and len(runs) < 200):
        t0 = time.perf_counter()
        _, _, out64 = oracle_step(w, h, threads)
        runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    max_err, ratio, finite = decode_errors(w.dtype, host_bits(out_gpu), out64)
    return dict(value=round(w.kv_bytes_logical() / dt / 1e9, 4), unit="GB/s", cores=threads,
                kind="oracle",
                sample=f"the full timed step (slot mapping, store, decode of all {w.num_seqs} "
                       f"sequences), double precision, {threads} host threads, repeated "
                       f"{len(runs)} times in {sum(runs):.1f} s, median {dt:.3f} s per step "
                       f"({host_description()})"), \
        dict(max_abs_err=max_err, within_tolerance=ratio <= 1.0 and finite)


class QuantStep:
    """A decode step over quantized pools: slot mapping, the quantizing store of the new
    rows, then decode (partition + reduce)."""

    def __init__(self, w, t, qt, kv):
        import paged_kv_cache_hpkv_amd as hpkv
        self.hpkv, self.w, self.t, self.qt, self.kv = hpkv, w, t, qt, kv
        dev = t.q.device
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.sp = torch.from_numpy(w.seq_ptr).to(dev)
        self.ctx = torch.from_numpy(w.context_lens).to(dev)
        self.chunks = [(torch.from_numpy(s).to(dev), torch.from_numpy(c).to(dev),
                        torch.empty(int(c[-1]), dtype=torch.int64, device=dev))
                       for s, c in w.chunks]
        self.drop = None if w.drop_mask is None else torch.from_numpy(w.drop_mask).to(dev)
        self.out = torch.empty_like(t.q)
        self.ws = hpkv.alloc_workspace(t.q, qt.k_codes, w.max_context_len)

    def decode(self):
        w, t, q = self.w, self.t, self.qt
        self.hpkv.hpkv_paged_attention_decode_quant(
            self.kv, t.q, q.k_codes, q.v_codes, q.k_scale, q.k_zero, q.v_scale, q.v_zero,
            self.bt, self.sp, self.ctx, w.scale, w.max_context_len, self.ws, self.out)

    def __call__(self):
        h, w, t, q = self.hpkv, self.w, self.t, self.qt
        for c, (start, cu, slots) in enumerate(self.chunks):
            h.hpkv_slot_mapping(self.bt, self.sp, w.page_size, w.num_pages, start, cu, slots)
            if self.drop is not None and c == 0:
                slots.masked_fill_(self.drop, -1)
            h.hpkv_store_kvcache_quant(self.kv, t.new_keys[c], t.new_values[c], q.k_codes,
                                       q.v_codes, q.k_scale, q.k_zero, q.v_scale, q.v_zero,
                                       slots)
        self.decode()


def quant_cpu_baseline(w, t, qt, kv, out_gpu, seconds):
    """The oracle on the quantized step (slot mapping, quantizing store, decode over the
    codes), on host copies of the same inputs, repeated for about `seconds`."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle  # noqa: E402
    from paths import decode_errors, host_bits, host_threads  # noqa: E402
    h = {n: getattr(qt, n).cpu().numpy().copy() for n in
         ("k_codes", "v_codes", "k_scale", "k_zero", "v_scale", "v_zero")}
    q = host_bits(t.q)
    nk = [host_bits(x) for x in t.new_keys]
    nv = [host_bits(x) for x in t.new_values]
    threads = host_threads()
    runs = []
    t_start = time.perf_counter()
    while not runs or (time.perf_counter() - t_start < seconds and len(runs) < 200):
        t0 = time.perf_counter()
        for c, (start, cu) in enumerate(w.chunks):
            slots = oracle.slot_mapping(w.block_table, w.seq_ptr, w.page_size, w.num_pages,
                                        start, cu)
            if w.drop_mask is not None and c == 0:
                slots[w.drop_mask] = -1
            oracle.store_kvcache_quant(w.dtype, kv, nk[c], nv[c], h["k_codes"], h["v_codes"],
                                       h["k_scale"], h["k_zero"], h["v_scale"], h["v_zero"],
                                       slots)
        _, ref = oracle.paged_attention_decode_quant(
            w.dtype, kv, q, h["k_codes"], h["v_codes"], h["k_scale"], h["k_zero"], h["v_scale"],
            h["v_zero"], w.block_table, w.seq_ptr, w.context_lens, w.scale, threads)
        runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    max_err, ratio, finite = decode_errors(w.dtype, host_bits(out_gpu), ref)
    return dict(value=round(quant_kv_bytes(w) / dt / 1e9, 4), unit="GB/s", cores=threads,
                kind="oracle",
                sample=f"the full timed step (slot mapping, quantizing store, decode of all "
                       f"{w.num_seqs} sequences over {kv} codes), double precision, {threads} "
                       f"host threads, repeated {len(runs)} times in {sum(runs):.1f} s, median "
                       f"{dt:.3f} s per step ({host_description()})"), \
        dict(max_abs_err=max_err, within_tolerance=ratio <= 1.0 and finite)


def quant_kv_bytes(w):
    """K+V bytes of one-byte codes a decode pass must read: sum(ctx) * 2 * Hkv * d."""
    return int(w.context_lens.astype(np.int64).sum()) * 2 * w.num_kv_heads * w.head_dim


def algorithmic_quant_bytes(w):
    """Codes, q, out, table entries, lengths and the (scale, zero) pairs of K and V of
    every page a sequence reads (16 B per page and KV head)."""
    b = torch.tensor([], dtype=w.torch_dtype).element_size()
    idx = w.block_table.dtype.itemsize
    pages = -(-w.context_lens.astype(np.int64) // w.page_size)
    per_seq = 2 * w.num_q_heads * w.head_dim * b + 4 + 2 * idx
    return int(quant_kv_bytes(w) + pages.sum() * (idx + 16 * w.num_kv_heads)
               + per_seq * w.num_seqs)


def quant_partition_kernel(w):
    """The library's quantized partition kernel for this shape: the matrix-core one for
    16-bit q, head_dim 32/64/128 and GQA groups of 4 or more, else the VALU one."""
    mfma = (w.dtype != "f32" and w.head_dim in (32, 64, 128)
            and (w.num_q_heads // w.num_kv_heads) % 4 == 0)
    return "decode_partition_mfma_quant_kernel" if mfma else "decode_partition_quant_kernel"


def main_quant(args, dev):
    w = make_workload(args)
    t = workloads.make_tensors(w, dev)
    qt = workloads.make_quant_tensors(w, args.kv, dev)
    step = QuantStep(w, t, qt, args.kv)
    stream = torch.cuda.current_stream(dev)
    timer = Timer(dev, stream, cold=not args.warm)
    for _ in range(args.warmup):
        timer.flush()
        step()
    torch.cuda.synchronize()
    st = timer.time(step, args.steps)
    ms_per_step = st["median_ms"]
    t_wall = st["wall_s"]
    warm_ms = timer.warm(step, args.steps)
    rt = timer.time(step.decode, args.roofline_launches)
    dec_ms = rt["median_ms"]
    alg = algorithmic_quant_bytes(w)
    achieved = alg / (dec_ms * 1e-3) / 1e9
    kv = quant_kv_bytes(w)
    value = kv / (ms_per_step * 1e-3) / 1e9
    rec = recorded_traffic(w, QUANT_TRAFFIC_FILE, variant=f"/{args.kv}")
    line = {
        "metric": METRIC + " (quantized pools)",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype + "/" + args.kv,
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_TEXT.get(w.name, w.name) + f", {args.kv} KV pools",
            "global_batch": w.num_seqs,
            "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "page_size": w.page_size, "index": w.index,
            "sum_ctx_tokens": int(w.context_lens.astype(np.int64).sum()),
            "kv_bytes_per_step": kv,
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "sequences_per_s_per_layer": round(w.num_seqs / (ms_per_step * 1e-3), 1),
            "step": "slot mapping + quantizing store + quantized decode (separate launches)",
        },
        "timing": {
            "protocol": timer.protocol(),
            "step_ms": {k: round(v, 5) for k, v in st.items() if k.endswith("_ms")},
            "wall_s_timed_region": round(t_wall, 4),
            "warm_back_to_back_ms_per_step": round(warm_ms, 5),
        },
        "roofline": {
            "kernel": f"decode_order_kernel + {quant_partition_kernel(w)} + decode_reduce_kernel",
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if rec is None else rec.get("hbm_bytes_per_launch"),
            "algorithmic_bytes_per_launch": alg,
            "median_launch_ms": round(dec_ms, 5),
            "mean_launch_ms": round(rt["mean_ms"], 5),
            "launches": args.roofline_launches,
        },
    }
    if rec is not None:
        line["roofline"]["traffic_unit"] = ("HBM bytes per launch of the partition kernel "
                                            "(rocprofv3 FETCH_SIZE + WRITE_SIZE)")
    if args.copy_calibration:
        calibration_copy(dev)
    if not args.no_cpu_baseline:
        step()  # leave `out` holding a full decode for the parity check
        torch.cuda.synchronize()
        cb, parity = quant_cpu_baseline(w, t, qt, args.kv, step.out, args.cpu_seconds)
        line["cpu_baseline"] = cb
        line["parity_vs_oracle"] = parity
    print(json.dumps(line), flush=True)


def calibration_copy(dev):
    """A plain 1 GiB device copy, whose counter readings scale the kernels' HBM bytes."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def prefill_flops(w, chunk):
    """Causal attention flops of one chunk: 4 * d * Hq * (p + 1) summed over its positions."""
    start, cu = chunk
    n = np.diff(cu).astype(np.int64)
    st = start.astype(np.int64)
    keys = n * st + n * (n + 1) // 2  # sum over p in [start, start+n) of (p + 1)
    return 4 * w.head_dim * w.num_q_heads * int(keys.sum())


class PrefillStep:
    """Per chunk: slot mapping + store of its K/V rows, then causal prefill attention."""

    def __init__(self, w, t, queries):
        import paged_kv_cache_hpkv_amd as hpkv
        self.hpkv, self.w, self.t, self.q = hpkv, w, t, queries
        dev = t.k_cache.device
        self.bt = torch.from_numpy(w.block_table).to(dev)
        self.sp = torch.from_numpy(w.seq_ptr).to(dev)
        self.chunks = [(torch.from_numpy(s).to(dev), torch.from_numpy(c).to(dev),
                        torch.empty(int(c[-1]), dtype=torch.int64, device=dev),
                        max(1, int(np.diff(c).max())))
                       for s, c in w.chunks]
        self.out = [torch.empty_like(q) for q in queries]

    def attention(self, c):
        w, t = self.w, self.t
        start, cu, _, mq = self.chunks[c]
        self.hpkv.hpkv_paged_attention_prefill(self.q[c], t.k_cache, t.v_cache, self.bt, self.sp,
                                               start, cu, w.scale, mq, self.out[c])

    def __call__(self):
        h, w, t = self.hpkv, self.w, self.t
        for c, (start, cu, slots, _) in enumerate(self.chunks):
            h.hpkv_slot_mapping(self.bt, self.sp, w.page_size, w.num_pages, start, cu, slots)
            h.hpkv_store_kvcache(t.new_keys[c], t.new_values[c], t.k_cache, t.v_cache, slots)
            self.attention(c)


def prefill_cpu_baseline(w, t, step, seconds, rows_per_chunk=8):
    """The oracle's prefill on sampled query rows of every chunk, on host copies of the
    pools after the step (a row at position p only reads keys 0..p, which hold the same
    bits at any point after their chunk was stored); rounds of rows_per_chunk random rows
    per chunk are added until about `seconds` of oracle time."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from paths import decode_errors, host_bits, oracle_prefill_rows  # noqa: E402
    h = dict(k_cache=host_bits(t.k_cache), v_cache=host_bits(t.v_cache))
    q_bits = [host_bits(q) for q in step.q]
    outs = [host_bits(o) for o in step.out]
    rng = np.random.default_rng(0)
    flops, secs, worst, ok, nrows = 0, 0.0, 0.0, True, 0
    while nrows == 0 or (secs < seconds and nrows < 4096):
        for c, (start, cu) in enumerate(w.chunks):
            rows = np.sort(rng.choice(int(cu[-1]), rows_per_chunk, replace=False))
            seq_of = np.searchsorted(cu, rows, side="right") - 1
            pos = start[seq_of].astype(np.int64) + rows - cu[seq_of]
            t0 = time.perf_counter()
            ref = oracle_prefill_rows(w, h, q_bits[c], start, cu, rows)
            secs += time.perf_counter() - t0
            flops += 4 * w.head_dim * w.num_q_heads * int((pos + 1).sum())
            nrows += len(rows)
            err, ratio, finite = decode_errors(w.dtype, outs[c][rows], ref)
            worst = max(worst, err)
            ok = ok and finite and ratio <= 1.0
    return dict(value=round(flops / secs / 1e12, 6), unit="TFLOP/s", cores=1, kind="oracle",
                sample=f"{nrows} random query rows (all heads; {rows_per_chunk} per chunk per "
                       f"round over the {len(w.chunks)} chunks), double precision, 1 host "
                       f"thread, {secs:.2f} s ({host_description()})"), \
        dict(max_abs_err=worst, within_tolerance=ok)


def main_prefill(args, dev):
    w = make_workload(args)
    t = workloads.make_tensors(w, dev)
    queries = workloads.make_prefill_queries(w, dev)
    step = PrefillStep(w, t, queries)
    stream = torch.cuda.current_stream(dev)
    timer = Timer(dev, stream, cold=not args.warm)
    for _ in range(args.warmup):
        timer.flush()
        step()
    torch.cuda.synchronize()
    st = timer.time(step, args.steps)
    ms_per_step = st["median_ms"]
    t_wall = st["wall_s"]
    warm_ms = timer.warm(step, args.steps)

    # the prefill kernel alone, per chunk: per-launch HIP events, same protocol
    nl = max(1, args.roofline_launches // len(w.chunks))
    per = [timer.time(lambda c=c: step.attention(c), nl) for c in range(len(w.chunks))]
    med_ms = [x["median_ms"] for x in per]
    mean_ms = [x["mean_ms"] for x in per]
    flops = [prefill_flops(w, ch) for ch in w.chunks]
    achieved = sum(flops) / (sum(med_ms) * 1e-3) / 1e12
    value = sum(flops) / (ms_per_step * 1e-3) / 1e12
    prec = recorded_traffic(w, PREFILL_TRAFFIC_FILE, PREFILL_SRC)
    line = {
        "metric": PREFILL_METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_TEXT.get(w.name, w.name) + " (prefill attention of each chunk)",
            "global_batch": w.num_seqs,
            "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "page_size": w.page_size, "index": w.index,
            "query_rows_per_chunk": [int(cu[-1]) for _, cu in w.chunks],
            "flops_per_step": sum(flops),
            "step": "per chunk: slot mapping + store + prefill attention (separate launches)",
        },
        "timing": {
            "protocol": timer.protocol(),
            "step_ms": {k: round(v, 5) for k, v in st.items() if k.endswith("_ms")},
            "wall_s_timed_region": round(t_wall, 4),
            "warm_back_to_back_ms_per_step": round(warm_ms, 5),
        },
        "roofline": {
            "kernel": "prefill_mfma_kernel",
            "bound": "mfma",
            "achieved": round(achieved, 2),
            "peak": MFMA16_PEAK_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / MFMA16_PEAK_TFLOPS, 4),
            "traffic": None if prec is None else prec.get("hbm_bytes_per_launch"),
            "algorithmic_flops_per_launch": flops,
            "median_launch_ms": [round(x, 5) for x in med_ms],
            "mean_launch_ms": [round(x, 5) for x in mean_ms],
            "launches": nl * len(w.chunks),
        },
    }
    if prec is not None:
        line["roofline"]["traffic_unit"] = ("HBM bytes per launch, one entry per chunk "
                                            "(rocprofv3 FETCH_SIZE + WRITE_SIZE)")
    if args.copy_calibration:
        calibration_copy(dev)
    if not args.no_cpu_baseline:
        cb, parity = prefill_cpu_baseline(w, t, step, args.cpu_seconds)
        line["cpu_baseline"] = cb
        line["parity_vs_oracle"] = parity
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has "
              "no multi-GPU path", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.path == "prefill":
        main_prefill(args, dev)
        return
    if args.kv:
        main_quant(args, dev)
        return
    w = make_workload(args)
    stream = torch.cuda.current_stream(dev)
    timer = Timer(dev, stream, cold=not args.warm)
    if args.ceiling:
        line = {"metric": "HBM read ceiling (hpkv_read_ceiling)", "unit": "GB/s",
                "config": {"workload": WORKLOAD_TEXT.get(w.name, w.name),
                           "buffer_bytes": w.kv_bytes_logical()},
                "ceilings": ceilings(dev, timer, w.kv_bytes_logical())}
        print(json.dumps(line), flush=True)
        return
    t = workloads.make_tensors(w, dev)
    step = Step(w, t, fused=is_decode_step(w) and not args.unfused, shared=args.shared)

    if args.copy_calibration:
        calibration_copy(dev)

    for _ in range(args.warmup):
        timer.flush()
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # capture one step (every argument is a device address fixed at capture) and
        # replay it; the cache-clearing writes stay outside the graph
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            step()
        stream.wait_stream(side)
        with torch.cuda.graph(graph):
            step()
        torch.cuda.synchronize()
        run = graph.replay
    st = timer.time(run, args.steps)             # the K timed steps
    ms_per_step = st["median_ms"]
    warm_ms = timer.warm(run, args.steps)
    # dominant work alone (ordering + partition kernels), same protocol
    rt = timer.time(step.partitions_only, args.roofline_launches)
    part_ms = rt["median_ms"]
    alg = algorithmic_decode_bytes(w)
    achieved = alg / (part_ms * 1e-3) / 1e9
    step()  # leave `out` holding a full decode for the parity check below
    torch.cuda.synchronize()

    kv = w.kv_bytes_logical()
    value = kv / (ms_per_step * 1e-3) / 1e9
    rec = recorded_traffic(w, variant="/shared" if args.shared else "")
    b = torch.tensor([], dtype=w.torch_dtype).element_size()
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_TEXT.get(w.name, w.name),
            "global_batch": w.num_seqs,
            "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "page_size": w.page_size, "index": w.index,
            "sum_ctx_tokens": int(w.context_lens.astype(np.int64).sum()),
            "kv_bytes_per_step": kv,
            "kv_bytes_unique_rows": w.kv_bytes_unique_rows(),
            "bytes_per_elem": b,
            "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
            "sequences_per_s_per_layer": round(w.num_seqs / (ms_per_step * 1e-3), 1),
            "step": ("fused decode step (store of the ctx-1 row inside the decode launch)"
                     if step.fused else "slot mapping + store + decode (separate launches)")
                    + (", decode by hpkv_paged_attention_decode_shared" if step.shared else "")
                    + (", replayed from a HIP graph" if args.graph else ""),
        },
        "timing": {
            "protocol": timer.protocol(),
            "step_ms": {k: round(v, 5) for k, v in st.items() if k.endswith("_ms")},
            "wall_s_timed_region": round(st["wall_s"], 4),
            "warm_back_to_back_ms_per_step": round(warm_ms, 5),
            "warm_back_to_back_GBs": round(kv / (warm_ms * 1e-3) / 1e9, 2),
        },
        "roofline": {
            "kernel": ("decode_share_kernel + decode_order_kernel + decode_partition_mfma_kernel"
                       " + decode_reduce_kernel (the whole shared decode call)" if step.shared
                       else "decode_order_kernel + decode_partition[_mfma]_kernel "
                            "(the partition pass)"),
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": None if rec is None else rec.get("hbm_bytes_per_launch"),
            "algorithmic_bytes_per_launch": alg,
            "median_launch_ms": round(part_ms, 5),
            "mean_launch_ms": round(rt["mean_ms"], 5),
            "launches": args.roofline_launches,
        },
    }
    if rec is not None:
        line["roofline"]["traffic_unit"] = "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE)"
    if not args.no_ceiling:
        line["ceilings"] = ceilings(dev, timer, kv)
    if not args.no_cpu_baseline:
        cb, parity = cpu_baseline(w, t, step.out, args.cpu_seconds)
        line["cpu_baseline"] = cb
        line["parity_vs_oracle"] = parity
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
