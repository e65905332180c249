"""Benchmark of the block-sparse masked attention forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-configs] [--no-cpu-baseline]

One step is one pass of the whole hot path over one batch of synthetic input already resident
in HBM: the BlockMask build (for masked workloads) followed by the forward pass; for the
quantized form, quantize + quantized forward. Prints ONE JSON line.

Default: the headline is the largest single-GPU configuration, dense self-attention B=1, H=32,
S=24576, head dim 128, bf16 (`value`, `roofline`, `cpu_baseline`), and the same line carries a
`configs` array with every configuration (the 68-token fp32 grouped variate case, 4096 packed
groups, causal document packing, sliding-window GQA with soft-cap, the dense case in bf16 and in
the int8/fp8 form): forward time, roofline bound and fraction, HBM traffic from the committed
counters, a flushed-cache time for the two HBM-bound cases, and a bounded oracle sample timed on
the host cores. --workload NAME measures one workload alone (the profiling runs use this).

Metric: effective TFLOP/s counted on unmasked FLOPs (4 * D per allowed (query, key) pair per
query head: Q.K^T and P.V), plus algorithmic HBM GB/s (Q, K, V, document ids and the BlockMask
lists read once; O and LSE written once). Roofline entries are for the forward kernel alone,
timed with HIP events on the stream it is launched on.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-sparse attn fwd effective TFLOP/s (unmasked FLOPs) + HBM GB/s, 1 GPU"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2516.6
FP32_PEAK_TFLOPS = 157.3
INT8_FP8_PEAK_TOPS = 5033.2  # dense int8 / fp8 MFMA (2x bf16)
KERNEL_SOURCES = ["block_sparse_masked_blockmask_amd/csrc/fwd.hip",
                  "block_sparse_masked_blockmask_amd/csrc/fwd_dense.hip",
                  "block_sparse_masked_blockmask_amd/csrc/fwd_pipe.hip",
                  "block_sparse_masked_blockmask_amd/csrc/work_order.h",
                  "block_sparse_masked_blockmask_amd/csrc/quant.hip",
                  "block_sparse_masked_blockmask_amd/csrc/device_common.h",
                  "block_sparse_masked_blockmask_amd/csrc/tile_class.h"]

# The configurations, in the order of the target: (label, workload, quantized form).
CONFIGS = [
    ("cfg1", "grouped_variate_4x17_f32", False),
    ("cfg2", "grouped_variate_4096g_bf16", False),
    ("cfg3", "doc_causal_b4h16t8192_bf16", False),
    ("cfg4", "swa1024_gqa32x8_softcap50_t16384_bf16", False),
    ("cfg5", "dense_b1h32s24576_bf16", False),
    ("cfg5q", "dense_b1h32s24576_bf16", True),
]
HEADLINE = "cfg5"
# HBM-bound workloads whose working set (> 256 MB) meets the MALL: also timed after a 1 GiB flush.
FLUSHED = ("grouped_variate_4096g_bf16", "doc_causal_b4h16t8192_bf16")
FLUSH_BYTES = 1 << 30
CPU_BUDGET_S = {"headline": 12.0, "config": 3.0}


def launch_config(w, quantized: bool = False) -> dict:
    """How each workload is launched, here and in the full-size parity tests: BlockMask block
    sizes, the optional cost-ordered schedule (row_order) and whether a BlockMask is built at all
    (an unmasked workload runs with bm = NULL, every tile full)."""
    if quantized:
        return dict(q_block=128, kv_block=128, row_order=False, block_mask=False)
    masked = bool(w.doc or w.causal or w.window is not None or w.prefix_len is not None)
    if w.dtype == "f32":
        return dict(q_block=128, kv_block=128, row_order=False, block_mask=masked)
    return dict(q_block=128, kv_block=64, row_order=bool(w.doc and w.causal), block_mask=masked)


def mask_kind(fa, w) -> int:
    return (fa.FA_MASK_DOC if w.doc else 0) | (fa.FA_MASK_CAUSAL if w.causal else 0) \
        | (fa.FA_MASK_WINDOW if w.window is not None else 0) | (fa.FA_MASK_PREFIX_LM if w.prefix_len is not None else 0)


def score_kind(fa, w) -> int:
    return (fa.FA_SCORE_ALIBI if w.alibi_slopes is not None else 0) | (fa.FA_SCORE_SOFTCAP if w.softcap else 0)


def allowed_pairs(w) -> int:
    """Exact number of allowed (query, key) pairs per query head, from the mask structure."""
    total = 0
    for b in range(w.B):
        if w.doc and not w.causal and w.window is None and w.prefix_len is None:
            qa = np.unique(w.q_doc[b], return_counts=True)
            ka = dict(zip(*np.unique(w.kv_doc[b], return_counts=True)))
            total += int(sum(int(c) * int(ka.get(d, 0)) for d, c in zip(*qa)))
        elif w.doc and w.causal and w.window is None and w.prefix_len is None and w.Lq == w.Lkv \
                and np.array_equal(w.q_doc[b], w.kv_doc[b]) and np.all(np.diff(w.q_doc[b]) >= 0):
            _, c = np.unique(w.q_doc[b], return_counts=True)
            total += int(sum(int(n) * (int(n) + 1) // 2 for n in c))
        elif not w.doc and w.causal and w.prefix_len is None and w.Lq == w.Lkv:
            i = np.arange(w.Lq, dtype=np.int64)
            per_row = i + 1 if w.window is None else np.minimum(i + 1, w.window)
            total += int(per_row.sum())
        elif not (w.doc or w.causal or w.window is not None or w.prefix_len is not None):
            total += w.Lq * w.Lkv
        else:
            raise NotImplementedError("pair count for this mask combination")
    return total


def algorithmic_bytes(w, bm, quantized=False) -> int:
    """Bytes the forward must move once: Q, K, V (and scales), document ids and BlockMask lists
    read; O and LSE written."""
    if quantized:
        qkvo = (w.B * w.Hq * w.Lq + 2 * w.B * w.Hkv * w.Lkv) * w.D + w.B * w.Hq * w.Lq * w.D * 2
        scales = 4 * (w.B * w.Hq * -(-w.Lq // 128) + w.B * w.Hkv * -(-w.Lkv // 128) + w.B * w.Hkv * w.D)
        return qkvo + scales + w.B * w.Hq * w.Lq * 4
    el = 2 if w.dtype == "bf16" else 4
    qkvo = (2 * w.B * w.Hq * w.Lq + 2 * w.B * w.Hkv * w.Lkv) * w.D * el
    lse = w.B * w.Hq * w.Lq * 4
    docs = (w.B * (w.Lq + w.Lkv) * 4) if w.doc else 0
    lists = 0
    if bm is not None:
        counts = 2 * bm.kv_num_blocks.numel() * 4
        live = int(bm.kv_num_blocks.sum().item() + bm.full_kv_num_blocks.sum().item())
        lists = counts + live * 4
    return qkvo + lse + docs + lists


def source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _counters_json(workload: str, tag: str):
    """The `<tag>-json:` record of profiles/fwd_<workload>_counters.md when its kernel-source hash
    matches the current sources, else None (counters of other kernels are not reported)."""
    path = os.path.join(ROOT, "profiles", f"fwd_{workload}_counters.md")
    if not os.path.exists(path):
        return None
    m = re.search(rf"^{tag}-json: (\{{.*\}})\s*$", open(path).read(), re.M)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("source_sha") != source_hash():
        return None
    return d


def read_traffic(workload: str):
    """HBM traffic per forward launch from the committed rocprofv3 counter summary, scaled by the
    copy-kernel calibration it records; None if absent or taken on other kernel sources."""
    d = _counters_json(workload, "traffic")
    return None if d is None else int(d["hbm_bytes_per_launch"])


def rows_allowed(w, b, rows) -> int:
    """Allowed (query, key) pairs of the given query rows (metric bookkeeping)."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(w.Lkv, dtype=np.int64)[None, :]
    ok = np.ones((i.shape[0], w.Lkv), dtype=bool)
    if w.doc:
        ok &= w.q_doc[b][i] == w.kv_doc[b][j]
    if w.causal:
        ok &= i >= j
    if w.window is not None:
        ok &= (i - j) < w.window
    if w.prefix_len is not None:
        ok &= (j < w.prefix_len) | (i >= j)
    return int(ok.sum())


def spec_of(w) -> dict:
    return dict(doc=w.doc, causal=w.causal, window=w.window, prefix_len=w.prefix_len, q_doc=w.q_doc,
                kv_doc=w.kv_doc, alibi_slopes=w.alibi_slopes, softcap=w.softcap)


def cpu_baseline(w, quantized: bool, budget_s: float):
    """The oracle as it stands, on the host cores, on a bounded sample of the same workload:
    whole 128-row query blocks of random (batch, query head) pairs, all keys each, until the
    budget is spent. The quantized form's oracle is attention on the oracle's own int8 / E4M3
    dequantized inputs with P coded through E4M3 (its quantizers run on the sampled heads)."""
    from oracle import attention as ref_attn
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    qf, kf, vf = w.qkv_f32()
    rng = np.random.default_rng(0)
    nqb = -(-w.Lq // 128)
    spec = spec_of(w)
    n_pairs = n_rows = n_blocks = 0
    qcache = {}
    t0 = time.perf_counter()
    while True:
        b, hq, qb = int(rng.integers(w.B)), int(rng.integers(w.Hq)), int(rng.integers(nqb))
        rows = np.arange(qb * 128, min(w.Lq, qb * 128 + 128))
        if quantized:
            from oracle import quant as ref_q
            hk = hq // (w.Hq // w.Hkv)
            if (b, hq) not in qcache:
                q8, sq = ref_q.quantize_int8_blocks(qf[b:b + 1, hq:hq + 1])
                k8, sk = ref_q.quantize_int8_blocks(kf[b:b + 1, hk:hk + 1])
                v8, sv = ref_q.quantize_fp8_channels(vf[b:b + 1, hk:hk + 1])
                qcache[(b, hq)] = (q8, sq, k8, sk, v8, sv)
            ref_q.attention_dequantized(*qcache[(b, hq)], rows, 0, 0, round_p=True)
        else:
            ref_attn.attention_rows(qf, kf, vf, spec, b, hq, rows)
        n_rows += len(rows)
        n_blocks += 1
        n_pairs += rows_allowed(w, b, rows)
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    flops = 4.0 * w.D * n_pairs
    what = "fp64 dequantized-input attention (int8 Q/K, E4M3 V and P)" if quantized else "numpy fp64 dense rows"
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{n_rows} query rows ({n_blocks} random 128-row query blocks of random (batch, head) pairs), "
                      f"all {w.Lkv} keys each, {what}; {dt:.1f} s; rate on the sample's allowed pairs"}


def achievable_peaks(torch, dev):
    """What this machine reaches outside the method: a 1 GiB device copy (HBM read + write bytes per
    second) and an 8192^3 bf16 GEMM through the vendor BLAS (TFLOP/s); best of 5 after warm-up."""
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    m = 8192
    x = torch.randn(m, m, device=dev).bfloat16()
    y = torch.randn(m, m, device=dev).bfloat16()

    def best(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(5):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e-3)
        return min(ts)

    t_copy = best(lambda: b.copy_(a))
    t_gemm = best(lambda: torch.matmul(x, y))
    res = {"hbm_copy_gbs": 2 * n / t_copy / 1e9, "bf16_gemm_tflops": 2.0 * m ** 3 / t_gemm / 1e12}
    del a, b, x, y
    torch.cuda.empty_cache()
    return res


class Case:
    """One workload on the device in its launch configuration: inputs, outputs, BlockMask and
    workspaces allocated once; step() and fwd() only enqueue kernels."""

    def __init__(self, fa, torch, dev, w, quantized=False, refined=False, launch=None):
        self.fa, self.torch, self.w = fa, torch, w
        self.quantized, self.refined = quantized, refined
        self.launch = dict(launch or launch_config(w, quantized))
        self.mk, self.sk = mask_kind(fa, w), score_kind(fa, w)
        if quantized and (self.mk or self.sk or w.dtype != "bf16"):
            raise ValueError("the quantized form serves unmasked bf16 workloads only")

        def dev_tensor(x):
            if w.dtype == "bf16":
                return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
            return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

        self.q, self.k, self.v = dev_tensor(w.q), dev_tensor(w.k), dev_tensor(w.v)
        self.qd = torch.from_numpy(w.q_doc).to(dev) if w.doc else None
        # Self-attention packing passes one id array for both sides (the ABI allows the alias).
        self.kd = (self.qd if w.kv_doc is w.q_doc else torch.from_numpy(w.kv_doc).to(dev)) if w.doc else None
        self.sl = torch.from_numpy(w.alibi_slopes).to(dev) if w.alibi_slopes is not None else None
        self.out = torch.empty(self.q.shape, dtype=torch.bfloat16 if quantized else self.q.dtype, device=dev)
        self.lse = torch.empty(self.q.shape[:3], dtype=torch.float32, device=dev)
        self.stream = torch.cuda.current_stream()
        L = self.launch
        self.bm = self.ws = None
        if L["block_mask"] and not quantized:
            self.bm = fa.BlockMask(w.B if w.doc else 1, 1, w.Lq, w.Lkv, L["q_block"], L["kv_block"], dev,
                                   row_order=L["row_order"])
            ws_bytes = fa.flexattn_block_mask_workspace_bytes(self.mk, w.B, w.Lq, w.Lkv, L["q_block"], L["kv_block"])
            self.ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
        if quantized:
            if refined:
                self.qbufs = fa.flexattn_quantize_qkv_ex(self.q, self.k, self.v, qk_block=32, center_k=True)
                self.qws = torch.empty(max(1, fa.flexattn_quantize_qkv_ex_workspace_bytes(w.B, w.Hkv, w.Lkv)),
                                       dtype=torch.uint8, device=dev)
            else:
                self.qbufs = fa.flexattn_quantize_qkv(self.q, self.k, self.v)
        torch.cuda.synchronize()

    def prep(self):
        """The part of the step before the forward: BlockMask build, or quantization."""
        fa, w, s = self.fa, self.w, self.stream
        if self.quantized:
            if self.refined:
                fa.flexattn_quantize_qkv_ex(self.q, self.k, self.v, qk_block=32, center_k=True, out=self.qbufs,
                                            workspace=self.qws, stream=s)
            else:
                fa.flexattn_quantize_qkv(self.q, self.k, self.v, out=self.qbufs, stream=s)
        elif self.bm is not None:
            L = self.launch
            fa.flexattn_block_mask_build(self.mk, w.B, w.Lq, w.Lkv, L["q_block"], L["kv_block"], q_doc=self.qd,
                                         kv_doc=self.kd, window=w.window or 0, prefix_len=w.prefix_len or 0,
                                         out=self.bm, workspace=self.ws, stream=s)

    def fwd(self):
        fa, w, s = self.fa, self.w, self.stream
        if self.quantized:
            if self.refined:
                fa.flexattn_fwd_quant(self.qbufs, out=self.out, lse=self.lse, stream=s)
            else:
                qb = self.qbufs
                fa.flexattn_fwd(qb["q8"], qb["k8"], qb["v8"], q_scale=qb["q_scale"], k_scale=qb["k_scale"],
                                v_scale=qb["v_scale"], out=self.out, lse=self.lse, stream=s)
        else:
            fa.flexattn_fwd(self.q, self.k, self.v, self.bm, self.mk, self.sk, window=w.window or 0,
                            prefix_len=w.prefix_len or 0, softcap=w.softcap or 0.0, alibi_slopes=self.sl,
                            q_doc=self.qd, kv_doc=self.kd, out=self.out, lse=self.lse, stream=s)

    def step(self, ev=None):
        self.prep()
        if ev is not None:
            ev[0].record(self.stream)
        self.fwd()
        if ev is not None:
            ev[1].record(self.stream)

    def kernel_name(self) -> str:
        if self.quantized:
            return "fwd_quant_kernel"
        if self.w.dtype != "bf16":
            return "fwd_f32_kernel"
        # bf16 without a BlockMask runs the software-pipelined every-tile-full kernel; with a
        # BlockMask of 128-query blocks and a mask without document ids, the software-pipelined
        # block-sparse kernel.
        if self.bm is None:
            return "fwd_bf16_dense_kernel"
        if self.launch["q_block"] == 128 and not self.w.doc:
            return "fwd_bf16_pipe_kernel"
        return "fwd_bf16_kernel"

    def flops(self) -> float:
        return 4.0 * self.w.D * allowed_pairs(self.w) * self.w.Hq

    def abytes(self) -> int:
        return algorithmic_bytes(self.w, self.bm, self.quantized)


def warm_up(case, torch, min_steps=3, min_s=0.2, max_steps=20000):
    """The clocks take tens of milliseconds of sustained load to settle (forward durations drift by
    up to 12% over the first 30 ms), so warm up for a fixed time, not a count; returns the count."""
    n, t_w = 0, time.perf_counter()
    while n < min_steps or (time.perf_counter() - t_w < min_s and n < max_steps):
        case.step()
        torch.cuda.synchronize()
        n += 1
    return n


def sample_fwd(case, torch, inner, reps=7, flush=None):
    """Median over reps - 2 samples (two warm-up samples dropped) of the forward's duration, each
    sample the mean of `inner` back-to-back forwards between two HIP events on the launch stream.
    With `flush` (a 1 GiB device buffer), every sample first overwrites it (untimed), so the
    forward starts with cold caches, and times one forward."""
    samples = []
    for rep in range(reps):
        if flush is not None:
            flush.fill_(rep & 0xFF)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(case.stream)
        for _ in range(inner):
            case.fwd()
        e1.record(case.stream)
        torch.cuda.synchronize()
        if rep >= 2:
            samples.append(e0.elapsed_time(e1) / inner * 1e3)
    return float(np.median(samples))


def roofline_of(case, fwd_us):
    """Roofline entry of the forward kernel: the bound follows the arithmetic intensity of the
    algorithmic work against the dtype's MFMA peak and HBM peak."""
    flops, abytes = case.flops(), case.abytes()
    tflops = flops / (fwd_us * 1e-6) / 1e12
    gbs = abytes / (fwd_us * 1e-6) / 1e9
    peak = INT8_FP8_PEAK_TOPS if case.quantized else (BF16_PEAK_TFLOPS if case.w.dtype == "bf16" else FP32_PEAK_TFLOPS)
    hbm_bound = (flops / abytes) < (peak * 1e12 / (HBM_PEAK_GBS * 1e9))
    if hbm_bound:
        roof = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": tflops, "peak": peak, "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    wl = case.w.name + ("_quantized" if case.quantized else "")
    roof["traffic"] = None if case.refined else read_traffic(wl)
    roof["kernel"] = case.kernel_name()
    roof["algorithmic_bytes"] = abytes
    roof["unmasked_flops"] = flops
    roof["avg_launch_ms"] = fwd_us * 1e-3
    roof["mfma_frac"] = tflops / peak
    roof["hbm_frac"] = gbs / HBM_PEAK_GBS
    util = None if case.refined else _counters_json(wl, "util")
    if util is not None:
        roof["counters"] = {k: util[k] for k in ("mfma_busy_frac", "valu_busy_frac") if k in util}
    return roof


def measure_config(label, name, quantized, fa, torch, dev, make_workload, flush_buf, cpu_budget, cache):
    """One entry of the `configs` array."""
    if name not in cache:
        cache.clear()
        cache[name] = make_workload(name)
    w = cache[name]
    case = Case(fa, torch, dev, w, quantized=quantized)
    warm_up(case, torch, min_s=0.1)
    # Back-to-back forwards per sample: enough for about 2 ms of work (at least 1).
    t1 = sample_fwd(case, torch, inner=1, reps=4)
    inner = int(min(200, max(1, 2000.0 / max(t1, 1.0))))
    fwd_us = sample_fwd(case, torch, inner=inner)
    # The whole step (prep + forward), back to back, between two events.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(case.stream)
    for _ in range(inner):
        case.step()
    e1.record(case.stream)
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) / inner * 1e3
    rec = {"label": label, "workload": name, "dtype": "i8/fp8e4m3->bf16" if quantized else w.dtype,
           "launch": case.launch, "fwd_us": fwd_us, "fwd_samples_of": inner, "step_us": step_us,
           "tflops": case.flops() / (fwd_us * 1e-6) / 1e12, "gbs": case.abytes() / (fwd_us * 1e-6) / 1e9,
           "roofline": roofline_of(case, fwd_us)}
    if name in FLUSHED and not quantized:
        single = sample_fwd(case, torch, inner=1)
        flushed = sample_fwd(case, torch, inner=1, flush=flush_buf)
        rec["fwd_us_single"] = single
        rec["fwd_us_flushed"] = flushed
        rec["roofline_flushed"] = {k: v for k, v in roofline_of(case, flushed).items()
                                   if k in ("bound", "achieved", "peak", "unit", "frac", "mfma_frac", "hbm_frac")}
    del case
    torch.cuda.empty_cache()
    if cpu_budget > 0:
        rec["cpu_baseline"] = cpu_baseline(w, quantized, cpu_budget)
    return rec


def run_decode(args, fa, torch, dev):
    """Decoding shape through flexattn_fwd (one workgroup per (batch, query head)) and
    flexattn_fwd_splitkv. Each sample is the mean of 20 back-to-back calls between two HIP
    events; median of 5 after 2 warm-up samples. Bytes: Q, K, V read once, O and lse written."""
    from workloads import decode_workload
    w = decode_workload()
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    q, k, v = bf(w.q), bf(w.k), bf(w.v)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    flops = 4.0 * w.D * w.Lq * w.Lkv * w.Hq * w.B
    abytes = (q.numel() + k.numel() + v.numel() + out.numel()) * 2 + lse.numel() * 4

    def time_call(call):
        samples = []
        for rep in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(20):
                call()
            e1.record()
            torch.cuda.synchronize()
            if rep >= 2:
                samples.append(e0.elapsed_time(e1) / 20 * 1e3)
        return float(np.median(samples))

    for n in (1, 2, 4, 8, 16, 32):
        ws = None
        if n > 1:
            ws = torch.empty(fa.flexattn_fwd_splitkv_workspace_bytes(w.B, w.Hq, w.Lq, n), dtype=torch.uint8, device=dev)
        call = (lambda: fa.flexattn_fwd(q, k, v, None, out=out, lse=lse, stream=stream)) if n == 1 else \
               (lambda ws=ws, n=n: fa.flexattn_fwd_splitkv(q, k, v, None, n_splits=n, workspace=ws, out=out, lse=lse,
                                                         stream=stream))
        us = time_call(call)
        print(json.dumps({"decode": w.name, "entry": "flexattn_fwd" if n == 1 else "flexattn_fwd_splitkv",
                          "n_splits": n, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lq": w.Lq, "Lkv": w.Lkv,
                          "us": us, "tflops": flops / (us * 1e-6) / 1e12,
                          "gbs": abytes / (us * 1e-6) / 1e9, "hbm_frac": abytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS}),
              flush=True)


BWD_WORKLOADS = ["grouped_variate_4096g_bf16", "doc_causal_b4h16t8192_bf16",
                 "swa1024_gqa32x8_softcap50_t16384_bf16", "dense_b1h32s24576_bf16"]


def run_backward(args, fa, torch, dev):
    """Backward pass (flexattn_bwd) on the bf16 workloads, BlockMask tiles 128 x 128. Each sample
    is the mean of 5 back-to-back backward calls between two HIP events; median of 5 after 2
    warm-up samples. The transposed BlockMask is built once beforehand (timed on its own, as a
    BlockMask's column lists are built with it). FLOPs: 10 * D per allowed pair per query head
    (S, dP, dV, dQ, dK products); bytes: Q, K, V, O, dO, lse, document ids and both BlockMask
    views read once, dQ, dK, dV written once."""
    from workloads import grad_output, make_workload
    names = [args.workload] if args.workload else BWD_WORKLOADS
    bf = lambda x: torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
    stream = torch.cuda.current_stream()

    def time_call(call, inner):
        samples = []
        for rep in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(inner):
                call()
            e1.record()
            torch.cuda.synchronize()
            if rep >= 2:
                samples.append(e0.elapsed_time(e1) / inner * 1e3)
        return float(np.median(samples))

    for name in names:
        w = make_workload(name)
        q, k, v, do = bf(w.q), bf(w.k), bf(w.v), bf(grad_output(w, 900))
        mk, sk = mask_kind(fa, w), score_kind(fa, w)
        qd = kd = sl = None
        if w.doc:
            qd = torch.from_numpy(np.ascontiguousarray(w.q_doc)).to(dev)
            kd = qd if w.kv_doc is w.q_doc else torch.from_numpy(np.ascontiguousarray(w.kv_doc)).to(dev)
        if w.alibi_slopes is not None:
            sl = torch.from_numpy(w.alibi_slopes).to(dev)
        kw = dict(window=w.window or 0, prefix_len=w.prefix_len or 0, softcap=w.softcap or 0.0, alibi_slopes=sl,
                  q_doc=qd, kv_doc=kd)
        # The schedule (query blocks by decreasing cost) where row costs vary: causal document masks.
        order = args.row_order == "on" if args.row_order else bool(w.doc and w.causal)
        bm = fa.flexattn_block_mask_build(mk, w.B, w.Lq, w.Lkv, 128, 128, q_doc=qd, kv_doc=kd,
                                          window=w.window or 0, prefix_len=w.prefix_len or 0, device=dev,
                                          row_order=order)
        bmt = fa.flexattn_block_mask_transpose(bm, col_order=order)
        out, lse = fa.flexattn_fwd(q, k, v, bm, mk, sk, **kw)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        ds = torch.empty(w.Hq, dtype=torch.float32, device=dev) if sl is not None else None
        ws = torch.empty(max(1, fa.flexattn_bwd_workspace_bytes(w.B, w.Hq, w.Lq)), dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        inner = 5
        t_us = time_call(lambda: fa.flexattn_bwd(q, k, v, out, do, lse, bm, bmt, mk, sk, dq=dq, dk=dk, dv=dv,
                                                 dslopes=ds, slope_grad=ds is not None, workspace=ws, stream=stream,
                                                 **kw), inner)
        tr_us = time_call(lambda: fa.flexattn_block_mask_transpose(bm, out=bmt, stream=stream), inner)
        pairs = allowed_pairs(w) * w.Hq
        flops = 10.0 * w.D * pairs
        el = 2
        abytes = (4 * w.B * w.Hq * w.Lq + 4 * w.B * w.Hkv * w.Lkv) * w.D * el + w.B * w.Hq * w.Lq * 4
        abytes += (w.B * (w.Lq + w.Lkv) * 4) if w.doc else 0
        live = int(bm.kv_num_blocks.sum().item() + bm.full_kv_num_blocks.sum().item())
        abytes += 2 * (bm.kv_num_blocks.numel() + bmt.q_num_blocks.numel()) * 4 + 2 * live * 4
        tf = flops / (t_us * 1e-6) / 1e12
        gb = abytes / (t_us * 1e-6) / 1e9
        print(json.dumps({"backward": name, "us": t_us, "transpose_us": tr_us, "tflops": tf, "gbs": gb,
                          "mfma_frac": tf / BF16_PEAK_TFLOPS, "hbm_frac": gb / HBM_PEAK_GBS,
                          "live_tiles": live, "algorithmic_bytes": abytes, "flops": flops}), flush=True)
        del q, k, v, do, out, lse, dq, dk, dv, ws, bm, bmt
        torch.cuda.empty_cache()


def run_sweep(args, fa, torch, dev):
    """Group-count sweep of the grouped variate workload. Each sample is the mean of 100
    back-to-back forward launches between two HIP events (the forwards run for microseconds);
    the median of 5 samples is reported, after 2 warm-up samples."""
    from workloads import SWEEP_GROUPS, grouped_sweep

    def time_fwd(call):
        samples = []
        for rep in range(7):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(100):
                call()
            e1.record()
            torch.cuda.synchronize()
            if rep >= 2:
                samples.append(e0.elapsed_time(e1) / 100 * 1e3)
        return float(np.median(samples))

    for dtype in ("f32", "bf16"):
        for n in SWEEP_GROUPS:
            w = grouped_sweep(n, dtype)
            if dtype == "bf16":
                q, k, v = (torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(dev)
                           for x in (w.q, w.k, w.v))
            else:
                q, k, v = (torch.from_numpy(np.ascontiguousarray(x)).to(dev) for x in (w.q, w.k, w.v))
            qd = torch.from_numpy(w.q_doc).to(dev)
            kv_block = 64 if dtype == "bf16" else 128
            out = torch.empty_like(q)
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=dev)
            sparse = fa.flexattn_block_mask_build(fa.FA_MASK_DOC, 1, w.Lq, w.Lkv, 128, kv_block, q_doc=qd, kv_doc=qd)
            dense = fa.block_mask_all_partial(1, 1, w.Lq, w.Lkv, 128, kv_block, device=dev)
            stream = torch.cuda.current_stream()
            t = {}
            for name, bm in (("sparse", sparse), ("all_live", dense)):
                t[name] = time_fwd(lambda bm=bm: fa.flexattn_fwd(q, k, v, bm, fa.FA_MASK_DOC, q_doc=qd, kv_doc=qd,
                                                                 out=out, lse=lse, stream=stream))
            tiles = int(sparse.kv_num_blocks.sum() + sparse.full_kv_num_blocks.sum())
            flops = 4.0 * w.D * w.Hq * 17 * 17 * n
            print(json.dumps({"sweep": "grouped_variate", "groups": n, "variates_per_group": 17, "dtype": dtype,
                              "L": w.Lq, "H": w.Hq, "D": w.D, "kv_block": kv_block,
                              "tiles_sparse": tiles, "tiles_all_live": dense.n_qb * dense.n_kvb,
                              "fwd_us_sparse": t["sparse"], "fwd_us_all_live": t["all_live"],
                              "speedup_sparse": t["all_live"] / t["sparse"],
                              "tflops_sparse": flops / (t["sparse"] * 1e-6) / 1e12}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default: at least 3 steps and 200 ms of completed steps, "
                         "so that the GPU clocks have settled; the count run is reported)")
    ap.add_argument("--workload", default=None,
                    help="measure this workload alone (default: the dense headline plus the configs array; "
                         "with --backward: all bf16 workloads)")
    ap.add_argument("--kv-block", type=int, default=None, help="override the BlockMask kv block")
    ap.add_argument("--q-block", type=int, default=None, help="override the BlockMask q block")
    ap.add_argument("--block-mask", choices=("on", "off"), default=None,
                    help="override whether an unmasked workload builds an all-full BlockMask (off: bm = NULL)")
    ap.add_argument("--quantized", action="store_true",
                    help="int8-QK / fp8-PV form (unmasked workloads): step = quantize + quantized forward")
    ap.add_argument("--refined", action="store_true",
                    help="with --quantized: 32-token Q/K scales and K centring (flexattn_quantize_qkv_ex + "
                         "flexattn_fwd_quant)")
    ap.add_argument("--row-order", choices=("on", "off"), default=None,
                    help="override building the BlockMask's schedule array (query blocks by decreasing cost) "
                         "inside the step (default: on for causal document masks, off otherwise)")
    ap.add_argument("--no-configs", action="store_true", help="skip the per-configuration array")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-peaks", action="store_true", help="skip the achievable-peak measurements")
    ap.add_argument("--sweep", action="store_true",
                    help="group-count sweep (8/32/64/128 groups x 17 variates, fp32 and bf16): block-sparse "
                         "BlockMask against an all-live BlockMask through the same kernel, one JSON line each")
    ap.add_argument("--decode", action="store_true",
                    help="decoding shape (B=8, GQA 32/8, 16 queries x 32768 keys): flexattn_fwd and "
                         "flexattn_fwd_splitkv over split counts, one JSON line each")
    ap.add_argument("--backward", action="store_true",
                    help="backward pass on the bf16 workloads (or --workload NAME), one JSON line each")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run only a plain 1 GiB device copy (HBM counter calibration for rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark measures one GPU; runs on several GPUs are not part of "
                                   "this build (the path shards by heads or groups with no exchange)"}))
        sys.exit(2)

    import torch
    dev = torch.device("cuda", 0)
    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n}))
        return

    import block_sparse_masked_blockmask_amd as fa
    from workloads import make_workload
    if args.sweep:
        run_sweep(args, fa, torch, dev)
        return
    if args.decode:
        run_decode(args, fa, torch, dev)
        return
    if args.backward:
        run_backward(args, fa, torch, dev)
        return

    single = args.workload is not None
    if single:
        label, name, quant = "single", args.workload, args.quantized
    else:
        label, name, quant = next(c for c in CONFIGS if c[0] == HEADLINE)

    t_gen = time.perf_counter()
    w = make_workload(name)
    launch = launch_config(w, quant)
    if args.q_block is not None:
        launch["q_block"] = args.q_block
    if args.kv_block is not None:
        launch["kv_block"] = args.kv_block
    if args.row_order is not None:
        launch["row_order"] = args.row_order == "on"
    if args.block_mask is not None and not quant:
        launch["block_mask"] = args.block_mask == "on" or mask_kind(fa, w) != 0
    case = Case(fa, torch, dev, w, quantized=quant, refined=args.refined and quant, launch=launch)
    gen_s = time.perf_counter() - t_gen

    if args.warmup is None:
        args.warmup = warm_up(case, torch)
    else:
        for _ in range(args.warmup):
            case.step()
    torch.cuda.synchronize()
    # Timed region: exactly K steps, bracketed by device synchronisation. It records no events: on
    # this platform each timing event costs about 10 us of the step (measured), so the forward's
    # own duration is taken in a second pass of K identical steps with HIP events around every
    # forward launch, on the stream the kernels are launched on.
    t0 = time.perf_counter()
    for _ in range(args.steps):
        case.step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    events = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        case.step(events[i])
    torch.cuda.synchronize()
    fwd_avg_ms = float(np.mean([a.elapsed_time(b) for a, b in events]))
    ms_per_step = wall * 1e3 / args.steps

    flops, abytes = case.flops(), case.abytes()
    roof = roofline_of(case, fwd_avg_ms * 1e3)
    step_desc = ("quantize_qkv_ex (32-token Q/K scales, K centring) + fwd_quant (int8 QK, fp8 PV)"
                 if case.refined else "quantize_qkv + fwd (int8 QK, fp8 PV)") if quant else \
        ("block_mask_build + fwd" if case.bm is not None else "fwd (bm = NULL: every tile full)")
    rec = {
        "metric": METRIC, "value": flops / (ms_per_step * 1e-3) / 1e12, "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "i8/fp8e4m3->bf16" if quant else w.dtype,
        "data": "synthetic (seeded numpy PCG64)",
        "config": {"workload": name, "label": label, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "Lq": w.Lq, "Lkv": w.Lkv,
                   "D": w.D, "mask": case.mk, "score": case.sk, "launch": case.launch, "step": step_desc},
        "hbm_gbs": abytes / (ms_per_step * 1e-3) / 1e9,
        "fwd_only": {"ms": fwd_avg_ms, "tflops": flops / (fwd_avg_ms * 1e-3) / 1e12,
                     "gbs": abytes / (fwd_avg_ms * 1e-3) / 1e9},
        "roofline": roof,
        "input_gen_s": gen_s,
    }
    del case
    torch.cuda.empty_cache()
    if not args.no_peaks and not quant and w.dtype == "bf16":
        ach = achievable_peaks(torch, dev)
        ref = ach["hbm_copy_gbs"] if roof["unit"] == "GB/s" else ach["bf16_gemm_tflops"]
        ach["frac_of_achievable"] = roof["achieved"] / ref
        rec["achievable"] = ach
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(w, quant, CPU_BUDGET_S["headline"])
    if not single and not args.no_configs:
        flush_buf = torch.empty(FLUSH_BYTES, dtype=torch.uint8, device=dev)
        cache = {name: w}
        # The headline's workload is already generated: measure its entries first.
        todo = sorted(CONFIGS, key=lambda c: c[1] != name)
        got = {}
        for lab, nm, qz in todo:
            print(f"# config {lab} {nm}{' quantized' if qz else ''}", file=sys.stderr, flush=True)
            got[lab] = measure_config(lab, nm, qz, fa, torch, dev, make_workload, flush_buf,
                                      0.0 if args.no_cpu_baseline else CPU_BUDGET_S["config"], cache)
        rec["configs"] = [got[lab] for lab, _, _ in CONFIGS]
        del flush_buf
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
