#!/usr/bin/env python3
"""Benchmark of the OScaR INT2 decode path on one MI355X.

Headline workload: Qwen3-8B-shaped single-sequence decode at 128K context --
batch 1, 32 query heads / 8 KV heads, head dim 128, bf16 inputs, 131072
tokens after the first step (130944 INT2 + 128 fp16).  The cache is
prefilled with 131071 synthetic tokens, then every timed step runs, for each
of L distinct layer caches, the whole decode hot path:
  append_kv   -- FHT + Omni-Token Scaling of the new Key, residual-window
                 bookkeeping, INT2 flush of a 32-token block when due
  decode_attn -- query FHT, split-K attention over the INT2 blocks and the
                 fp16 window, cross-split log-sum-exp merge (one launch).
L copies (8 at 128K, 806 MB) are cycled so that the 256 MB Infinity Cache
cannot serve a layer from a previous visit.

The same JSON line also carries the other workloads of the metric, each with
its own roofline: `llama_32k` (Llama-3.1-8B shape, 32K, 32 layers cycled),
`multimodal_64k` (Qwen3-VL-8B-like token-norm mix, 64K: bulk prefill
throughput, then decode, 16 layers) and `batch48` (48 ragged sequences of
8K..32K tokens, 36 resident layer caches).  `--headline-only` skips them.

Output: one JSON line.  value = context tokens attended per second in the
headline's timed region (whole job), plus per-layer microseconds, the
roofline of the attention kernel and the CPU oracle timed on a bounded sample
of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak
# batch-1 decode workloads: option name -> (synthetic workload id, description,
# layer caches cycled so that they exceed 3x the 256 MB Infinity Cache,
# profile summary holding the decode-step kernel's byte counters)
WORKLOADS = {
    "llama-32k": (1, "llama-3.1-8b-shape decode, 32K ctx, batch 1", 32,
                  "decode_step_llama-3.1-8b-32k.md"),
    "qwen3-128k": (2, "qwen3-8b-shape decode, 128K ctx, batch 1", 8,
                   "decode_step_qwen3-8b-128k.md"),
    "multimodal-64k": (4, "qwen3-vl-8b-shape multimodal prefill + decode, 64K ctx, batch 1", 16,
                       "decode_step_multimodal-64k.md"),
}
BATCH48_PROFILE = "decode_step_qwen3-8b-batch48.md"
# the decode-attention kernel and the headers it compiles from
ATTN_SRC = [os.path.join(ROOT, "int2_kv_cache_amd", "csrc", f)
            for f in ("oscar_attn.hip", "oscar_device.hpp", "oscar_host.hpp", "oscar_quant.hpp")]


def attn_src_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in ATTN_SRC:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def counter_traffic(profile: str):
    """HBM bytes of one attention launch from the committed rocprofv3 counters
    in profiles/<profile> (FETCH_SIZE / WRITE_SIZE, scaled by the same
    counters on a plain copy), or None when the attention sources (kernel
    file and the headers it includes) have changed since they were taken."""
    try:
        src = attn_src_hash()
        line = [l for l in open(os.path.join(ROOT, "profiles", profile))
                if l.startswith("counters:")][0]
    except (OSError, IndexError):
        return None
    kv = dict(tok.split("=") for tok in line.split()[1:])
    if kv.get("src") != src:
        return None
    kib = float(kv["fetch_kib"]) * float(kv["fetch_factor"]) + \
        float(kv["write_kib"]) * float(kv["write_factor"])
    return kib * 1024.0


def algorithmic_bytes(n: int, Q: int, hq: int, hkv: int, head_norm: bool = False) -> int:
    """Bytes one decode_attn launch must move for one sequence: each INT2
    (block, KV head) record (3072 B) + the block's token norms (64 B, or 64 B
    per KV head in HEAD scope), each fp16 window token (256 B K + 256 B V per
    KV head + 2 B norm, per KV head in HEAD scope), the bf16 query and the
    fp32 output."""
    nb = Q // 32
    r = n - Q
    nh = hkv if head_norm else 1
    return nb * (hkv * 3072 + 64 * nh) + r * (hkv * 512 + 2 * nh) + hq * 128 * 2 + hq * 128 * 4


def quantized(n: int, flush128: bool = False) -> int:
    """Q(n): tokens quantized after n appends (one-block or 128-token flushes)."""
    if flush128:
        return 128 * ((n - 1) // 128) if n > 128 else 0
    return 32 * ((max(0, n - 128) + 31) // 32)


def append_bytes(batch: int, hkv: int, head_norm: bool) -> int:
    """Algorithmic bytes of one append per sequence: the new token's Keys and
    Values in (bf16), its window rows out (fp16 Key row and Value column
    entries), its norm(s) and the state."""
    return batch * (hkv * 128 * 2 * 2 + hkv * 128 * 2 * 2 + (hkv if head_norm else 1) * 2 + 8)


def kernel_desc(args) -> str:
    if args.variant == 1:
        return ("decode_attn (VALU attention + LSE reduce)" if args.unfused else
                "append_kv + decode_attn (VALU attention + LSE reduce)")
    if args.unfused:
        return "decode_attn (one launch: split-K attention and the cross-split merge)"
    return ("decode_step (one launch: the append, split-K attention and the cross-split "
            "merge)")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3-128k", choices=sorted(WORKLOADS),
                    help="the workload of the top-level line: qwen3-128k (default), "
                         "llama-32k or multimodal-64k")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other workloads' sub-objects")
    ap.add_argument("--layers", type=int, default=0,
                    help="layer caches cycled (0: enough to exceed 3x the 256 MB Infinity Cache)")
    ap.add_argument("--ctx", type=int, default=0, help="context at the first step (0: the workload's)")
    ap.add_argument("--variant", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--hw-rsqrt", action="store_true",
                    help="Key scaling factor from the hardware rsqrt (OSCAR_SCALE_HW_RSQ)")
    ap.add_argument("--no-bf16", action="store_true",
                    help="skip the bf16 (unquantized) decode-attention baselines")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="query heads of the one-thread oracle sample (scaled to all heads)")
    ap.add_argument("--head-norm", action="store_true",
                    help="HEAD norm scope (a norm per token and KV head) instead of TOKEN")
    ap.add_argument("--flush128", action="store_true",
                    help="quantize the full 128-token window at once (four blocks) instead "
                         "of one block per flush")
    ap.add_argument("--q-standalone", action="store_true",
                    help="rotate the query with its own oscar_rotate_scale launch and pass "
                         "q' as fp32, instead of the rotation inside decode attention")
    ap.add_argument("--unfused", action="store_true",
                    help="run each layer's step as two launches (oscar_append_kv, then "
                         "oscar_decode_attn) instead of one oscar_decode_step")
    ap.add_argument("--batch48", action="store_true",
                    help="only the batched workload (48 ragged sequences of 8K..32K tokens, "
                         "36 resident layer caches), on a JSON line of its own")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device copy of this many MiB (5 times) and "
                         "exit: the reference for scaling HBM byte counters")
    return ap.parse_args()


def copy_ceiling_gbs(mib: int = 2048) -> float:
    """Bandwidth of a plain device copy (reads + writes) of `mib` MiB: a
    measured HBM ceiling to set the attention's rate beside the 8 TB/s peak."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.ones(n, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)
    ev[1].record()
    torch.cuda.synchronize()
    gbs = 5 * 2 * n * 4 / (ev[0].elapsed_time(ev[1]) * 1e-3) / 1e9
    del src, dst
    return gbs


def copy_probe(mib: int):
    """A plain device-to-device copy of known size, for calibrating the
    FETCH_SIZE / WRITE_SIZE counters against the attention kernel's."""
    import torch
    n = mib * 1024 * 1024 // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        torch.mul(src, 1.0, out=dst)   # elementwise kernel: reads and writes n*4 bytes
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes_each_way": n * 4, "calls": 5}), flush=True)


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), else the machine type."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def cpu_decode_baseline(wl, k, v, step0, args):
    """The oracle as it stands on a bounded sample of the same workload: its
    append of one step's token, then decode attention for every query head
    over the full context, the heads spread over the host's threads (the
    oracle's C code runs outside the interpreter lock and is re-entrant);
    median of 3 runs.  Also one thread on `cpu_heads` heads, scaled to all
    heads."""
    import concurrent.futures as cf

    import oracle
    cfg = wl.cfg
    mb = (wl.ctx_lens[0] + 4096) // 32
    orc = oracle.OracleCache(1, cfg.hq, cfg.hkv, mb, mb,
                             norm_scope=oracle.NORM_HEAD if args.head_norm else oracle.NORM_TOKEN,
                             flush_tokens=128 if args.flush128 else 32)
    orc.prefill(0, k, v, cfg.dtype)
    kn, vn, q = step0
    t0 = time.perf_counter()
    orc.append(kn, vn, cfg.dtype)
    t_append = time.perf_counter() - t0
    qr = oracle.rotate_query(q, cfg.dtype)
    n = orc.n(0)
    hq = cfg.hq
    heads = list(range(0, hq, max(1, hq // args.cpu_heads)))[: args.cpu_heads]
    t0 = time.perf_counter()
    for i in heads:
        orc.decode_attn_one(qr, 0, i)
    t1 = t_append + (time.perf_counter() - t0) * hq / len(heads)
    threads = host_threads()
    runs = []
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        for _ in range(3):
            t0 = time.perf_counter()
            list(ex.map(lambda i: orc.decode_attn_one(qr, 0, i), range(hq)))
            runs.append(time.perf_counter() - t0)
    tn = t_append + float(np.median(runs))
    return {"value": n / tn, "unit": "ctx tokens/s", "cores": threads, "kind": "oracle",
            "sample": "one decode step of one layer at n=%d: append (%.3f s) + attention for all "
                      "%d query heads on %d threads (median of 3: %.2f s)"
                      % (n, t_append, hq, threads, tn - t_append),
            "single_core_value": n / t1,
            "single_core_sample": "append + %d of %d heads on one thread, scaled to all heads "
                                  "(%.2f s per step)" % (len(heads), hq, t1),
            "cpu": cpu_model(), "host_threads": os.cpu_count()}


def cpu_prefill_baseline(wl, k, v, n_sample: int = 8192):
    """The oracle's prefill (n appends) of the first n_sample tokens of the
    same sequence, one thread (the oracle is sequential), median of 3."""
    import oracle
    cfg = wl.cfg
    mb = (n_sample + 4096) // 32
    runs = []
    for _ in range(3):
        orc = oracle.OracleCache(1, cfg.hq, cfg.hkv, mb, mb)
        t0 = time.perf_counter()
        orc.prefill(0, k[:n_sample], v[:n_sample], cfg.dtype)
        runs.append(time.perf_counter() - t0)
    t = float(np.median(runs))
    return {"value": n_sample / t, "unit": "prefill tokens/s", "cores": 1, "kind": "oracle",
            "sample": "oracle prefill of the first %d of the workload's tokens (median of 3: %.2f s)"
                      % (n_sample, t), "cpu": cpu_model()}


def stateless_calls(ok, torch, cfg, k, v, reps: int = 5):
    """The two stateless entry points on the prefill's tokens, outside the
    timed decode steps: oscar_rotate_scale (KEY) over all of them, then
    oscar_quant_pack over their whole 32-token blocks (fp16 Values converted
    by torch beforehand).  Median of `reps` calls, HIP events on the stream
    they run on."""
    T, hkv = k.shape[0], k.shape[1]
    nb = T // 32
    kd = torch.from_numpy(np.ascontiguousarray(k).view(np.int16)).cuda()
    khat = torch.empty_like(kd)
    knorm = torch.empty(T, dtype=torch.int16, device="cuda")
    v16 = torch.from_numpy(np.ascontiguousarray(v).view(np.int16)).cuda()
    if cfg.dtype == ok.BF16:
        v16 = v16.view(torch.bfloat16).to(torch.float16).view(torch.int16)
    rec = torch.empty(nb, hkv, ok.RECORD_BYTES, dtype=torch.uint8, device="cuda")
    nrm = torch.empty(nb, 32, dtype=torch.int16, device="cuda")

    def timed(fn):
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return float(np.median(ms)) * 1000.0

    rot_us = timed(lambda: ok.rotate_scale(kd, cfg.dtype, ok.ROT_KEY, khat_out=khat, norm_out=knorm))
    qp_us = timed(lambda: ok.quant_pack(khat[:32 * nb], knorm[:32 * nb], v16[:32 * nb], rec, nrm))
    rot_bytes = T * hkv * 128 * 2 * 2 + T * 2                     # k in, k_hat out, norms
    qp_bytes = nb * (32 * hkv * 128 * 2 * 2 + 64) + nb * (hkv * 3072 + 64)
    return {"rotate_scale_key": {"tokens": T, "us": rot_us, "algorithmic_bytes": rot_bytes,
                                 "achieved_gbs": rot_bytes / (rot_us * 1e-6) / 1e9},
            "quant_pack": {"blocks": nb, "us": qp_us, "algorithmic_bytes": qp_bytes,
                           "achieved_gbs": qp_bytes / (qp_us * 1e-6) / 1e9}}


def dense_bytes(ctxs, hq: int, hkv: int) -> int:
    """Algorithmic bytes of one bf16 baseline call: every token's bf16 Key and
    Value rows, the bf16 queries in and the fp32 outputs."""
    return sum(int(n) * hkv * 128 * 2 * 2 for n in ctxs) + len(ctxs) * hq * 128 * (2 + 4)


class DenseLeg:
    """The BF16 baseline at the same shape: n_layers distinct bf16 caches
    (written by oscar_dense_write_kv), then timed decode attention calls,
    one event pair per call, cycling the layers."""

    def __init__(self, ok, torch, geom, table, ctxs, n_layers):
        self.ok, self.torch, self.geom = ok, torch, geom
        self.ctxs = [int(n) for n in ctxs]
        self.caches = [ok.DenseCache(geom, block_table=table) for _ in range(n_layers)]
        for c in self.caches:
            c.ctx_lens.copy_(torch.tensor(self.ctxs, dtype=torch.int32))

    def write(self, b, k_dev, v_dev):
        self.ok.dense_write_kv(self.caches[0], b, 0, k_dev, v_dev)

    def replicate(self):
        for c in self.caches[1:]:
            c.k_pool.copy_(self.caches[0].k_pool)
            c.v_pool.copy_(self.caches[0].v_pool)
        self.torch.cuda.synchronize()

    def time(self, q_list, calls, warm, splits, int2_attn_us):
        ok, torch = self.ok, self.torch
        g = self.geom
        max_ctx = max(self.ctxs)
        S, nbytes = ok.dense_workspace_bytes(g, max_ctx, splits)
        ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        out = torch.empty(g.batch, g.num_q_heads, 128, dtype=torch.float32, device="cuda")
        lse = torch.empty(g.batch, g.num_q_heads, dtype=torch.float32, device="cuda")
        L = len(self.caches)
        for i in range(warm):
            ok.dense_decode_attn(self.caches[i % L], q_list[i % len(q_list)], out, lse, ws, max_ctx, S)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(calls)]
        torch.cuda.synchronize()
        for i in range(calls):
            ev[i][0].record()
            ok.dense_decode_attn(self.caches[i % L], q_list[i % len(q_list)], out, lse, ws, max_ctx, S)
            ev[i][1].record()
        torch.cuda.synchronize()
        for c in self.caches:
            assert int(c.error_flag.item()) == 0
        us = float(np.mean([e[0].elapsed_time(e[1]) for e in ev])) * 1000.0
        nb = dense_bytes(self.ctxs, g.num_q_heads, g.num_kv_heads)
        ach = nb / (us * 1e-6) / 1e9
        return {"kernel": "dense_decode_attn (bf16 split-K attention + LSE reduce)",
                "attn_us": us, "algorithmic_bytes": nb, "achieved_gbs": ach,
                "frac": ach / HBM_PEAK_GBS, "splits": S, "layers_cycled": L, "calls": calls,
                "ctx": self.ctxs[0] if len(self.ctxs) == 1 else float(np.mean(self.ctxs)),
                "int2_speedup": us / int2_attn_us}


def event_us(pairs) -> float:
    return float(np.mean([e[0].elapsed_time(e[1]) for e in pairs])) * 1000.0


def hot_attn_us(torch, call, reps: int = 20) -> float:
    """decode_attn on one layer cache called back to back (MALL-resident after
    the first call when the layer fits the 256 MB Infinity Cache)."""
    call()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record()
        call()
        e[1].record()
    torch.cuda.synchronize()
    return event_us(ev)


def decode_workload(ok, torch, synth, args, wname: str, steps: int, warmup: int,
                    bf16: bool, cpu: bool, stateless: bool, layers: int = 0, ctx: int = 0,
                    prefill_cpu: bool = False):
    """One batch-1 decode workload: L layer caches prefilled (each prefill
    timed), then `steps` timed steps of append_kv + decode_attn on every
    layer.  Event pairs, on the stream the calls run on (torch's current
    stream, which the binding passes), bracket one decode_attn call and one
    append_kv call per step (a pair around every call would cost the whole
    step ~5 us per layer)."""
    wid, wdesc, default_layers, profile = WORKLOADS[wname]
    wl = synth.workload(wid, ctx=ctx) if ctx else synth.workload(wid)
    n_ctx = wl.ctx_lens[0]
    cfg = wl.cfg
    L = layers or default_layers
    n_steps_total = warmup + steps
    max_ctx = n_ctx + n_steps_total + 64
    mb = (max_ctx + 31) // 32
    geom = ok.make_geom(1, cfg.hq, cfg.hkv, mb, mb,
                        norm_scope=ok.NORM_HEAD if args.head_norm else ok.NORM_TOKEN,
                        flush_tokens=128 if args.flush128 else 32,
                        key_scale=ok.SCALE_HW_RSQ if args.hw_rsqrt else ok.SCALE_IEEE)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    t0 = time.perf_counter()
    k, v = wl.prefill(0)
    kd, vd = dev(k), dev(v)
    dense = None
    if bf16:
        # the bf16 baseline's caches: the same prefilled tokens, at least two
        # layers and enough to exceed 3x the 256 MB Infinity Cache
        dgeom = ok.make_geom(1, cfg.hq, cfg.hkv, mb, mb)
        dense = DenseLeg(ok, torch, dgeom, None, [n_ctx - 1], max(2, -(-3 * 256 * 2**20 // (
            (n_ctx - 1) * cfg.hkv * 512))))
        dense.write(0, kd, vd)
        dense.replicate()
    caches = []
    pre_ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    pre_ms = []
    for _ in range(L):
        c = ok.DeviceCache(geom)
        pre_ev[0].record()
        ok.prefill_quantize(c, 0, kd, vd, cfg.dtype)
        pre_ev[1].record()
        torch.cuda.synchronize()
        pre_ms.append(pre_ev[0].elapsed_time(pre_ev[1]))
        caches.append(c)
    del kd, vd
    stp = list(wl.steps(n_steps_total))
    kn_d = [dev(s[0]) for s in stp]
    vn_d = [dev(s[1]) for s in stp]
    q_d = [dev(s[2]) for s in stp]
    S, nbytes = ok.decode_workspace_bytes(geom, max_ctx, args.splits)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(1, cfg.hq, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(1, cfg.hq, dtype=torch.float32, device="cuda")
    qrot = torch.empty(1, cfg.hq, 128, dtype=torch.float32, device="cuda")
    setup_s = time.perf_counter() - t0

    def attend(c, i):
        if args.q_standalone:
            ok.rotate_scale(q_d[i], cfg.dtype, ok.ROT_QUERY, q_out=qrot)
            ok.decode_attn(c, qrot, ok.FP32, out, lse, ws, max_ctx, S, args.variant)
        else:
            ok.decode_attn(c, q_d[i], cfg.dtype, out, lse, ws, max_ctx, S, args.variant)

    # the timed steps' calls, marshalled once (a call through the binding's
    # convenience wrappers costs several microseconds of host time, which at
    # short contexts is more than the GPU spends on a layer)
    def fused_standalone(c, i):
        ok.rotate_scale(q_d[i], cfg.dtype, ok.ROT_QUERY, q_out=qrot)
        ok.decode_step(c, kn_d[i], vn_d[i], cfg.dtype, qrot, ok.FP32, out, lse, ws, max_ctx, S,
                       args.variant)

    stream = torch.cuda.current_stream()
    calls = []
    for i in range(n_steps_total):
        row = []
        for c in caches:
            if args.unfused:
                app = ok.prepare_append_kv(c, kn_d[i], vn_d[i], cfg.dtype, stream=stream)
                if args.q_standalone:
                    att = (lambda c=c, i=i: attend(c, i))
                else:
                    att = ok.prepare_decode_attn(c, q_d[i], cfg.dtype, out, lse, ws, max_ctx, S,
                                                 args.variant, stream=stream)
            else:
                # one launch: the append and attention (oscar_decode_step)
                app = None
                if args.q_standalone:
                    att = (lambda c=c, i=i: fused_standalone(c, i))
                else:
                    att = ok.prepare_decode_step(c, kn_d[i], vn_d[i], cfg.dtype, q_d[i],
                                                 cfg.dtype, out, lse, ws, max_ctx, S,
                                                 args.variant, stream=stream)
            row.append((app, att))
        calls.append(row)
    # attention alone on the last layer's cache, for the Infinity-Cache probe
    hot_call = ok.prepare_decode_attn(caches[-1], q_d[-1], cfg.dtype, out, lse, ws, max_ctx, S,
                                      args.variant, stream=stream)

    def step(i, ev=None, ev_layer=-1, ap=None, ap_layer=-1):
        for li, (app, att) in enumerate(calls[i]):
            if app is not None:
                if li == ap_layer:
                    ap[0].record()
                app()
                if li == ap_layer:
                    ap[1].record()
            if li == ev_layer:
                ev[0].record()
            att()
            if li == ev_layer:
                ev[1].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    n0 = int(caches[0].seq_state[0, 0].item())

    # timed region: whole steps; in step s the decode_attn call of layer
    # s mod L and the append_kv call of layer (s + 1) mod L are bracketed
    attn_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    app_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t_beg, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_beg.record()
    for s_i in range(steps):
        step(warmup + s_i, attn_ev[s_i], s_i % L, app_ev[s_i], (s_i + 1) % L)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_beg.elapsed_time(t_end)
    st = caches[0].seq_state.cpu().numpy()[0]
    flag = int(caches[0].error_flag.item())
    assert flag == 0, "cache error flag %d" % flag
    n1, Q1 = int(st[0]), int(st[1])
    attn_us_pair = event_us(attn_ev)
    append_us = event_us(app_ev) if args.unfused else None
    hot_us = hot_attn_us(torch, hot_call)

    ms_per_step = total_ms / steps
    us_per_layer = ms_per_step * 1000.0 / L
    # With one launch per layer step (decode_step), that kernel's average
    # duration is the timed region, bracketed by HIP events on its stream,
    # over the launches; an event pair around a single call also times the
    # pair itself.  Two launches per step: the pair around decode_attn.
    one_launch = not args.unfused and args.variant != 1
    attn_us = us_per_layer if one_launch else attn_us_pair
    ctx_tokens = sum(n0 + 1 + s for s in range(steps)) * L
    n_mid = n0 + 1 + steps // 2
    bytes_attn = algorithmic_bytes(n_mid, quantized(n_mid, args.flush128), cfg.hq, cfg.hkv,
                                   args.head_norm)
    if not args.unfused:
        bytes_attn += append_bytes(1, cfg.hkv, args.head_norm)
    achieved = bytes_attn / (attn_us * 1e-6) / 1e9
    plain = not (args.head_norm or args.flush128 or args.q_standalone or args.hw_rsqrt
                 or args.variant == 1 or args.splits or args.unfused)
    res = {
        "workload": wdesc,
        "value": ctx_tokens / (total_ms / 1000.0),
        "unit": "ctx tokens/s",
        "steps": steps, "warmup": warmup, "ms_per_step": ms_per_step,
        "config": {"workload": wdesc, "batch": 1, "num_q_heads": cfg.hq,
                   "num_kv_heads": cfg.hkv, "head_dim": 128, "ctx_first_step": n_ctx,
                   "layers_cycled": L, "splits": S, "variant": args.variant,
                   "norm_scope": "head" if args.head_norm else "token",
                   "flush_tokens": 128 if args.flush128 else 32,
                   "query_rotation": "standalone" if args.q_standalone else "fused",
                   "key_scale": "hw_rsq" if args.hw_rsqrt else "ieee"},
        "us_per_layer_step": us_per_layer,
        "step_launches": 2 if args.unfused or args.variant == 1 else 1,
        "attn_us": attn_us,
        "attn_us_is": ("decode_step, one launch per layer step: timed region / launches"
                       if one_launch else "decode_attn between events"),
        "attn_us_event_pair": attn_us_pair,
        "attn_us_hot_mall_resident": hot_us,
        "append_us": append_us,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": counter_traffic(profile) if plain else None,
                     "kernel": kernel_desc(args),
                     "algorithmic_bytes": bytes_attn},
        "prefill_ms_per_layer": float(np.median(pre_ms)),
        "prefill_tokens_per_s": (n_ctx - 1) / (float(np.median(pre_ms)) / 1000.0),
        "final_state": [n1, Q1],
        "setup_s": setup_s,
    }
    if stateless:
        res["stateless"] = stateless_calls(ok, torch, cfg, k, v)
    if dense is not None:
        res["bf16_baseline"] = dense.time(q_d, steps, warmup, 0, attn_us_pair)
    del caches, dense, ws, calls
    torch.cuda.empty_cache()
    if cpu:
        res["cpu_baseline"] = cpu_decode_baseline(wl, k, v, stp[0], args)
    if prefill_cpu:
        res["prefill_cpu_baseline"] = cpu_prefill_baseline(wl, k, v)
    return res


def batch48_workload(ok, torch, synth, args, steps: int, warmup: int, bf16: bool):
    """The batched decode workload: 48 sequences with contexts drawn from
    8K..32K (block-table indexed, blocks packed per sequence), 32/8 heads,
    bf16; one layer's cache is prefilled and copied to all 36 layers, which
    stay resident.  A step appends one token to every sequence and runs
    decode attention, layer by layer.  Reports decode tokens/s (48 per step)
    and the attention's algorithmic bandwidth."""
    wl = synth.workload(3)
    cfg = wl.cfg
    L = 36
    B = cfg.batch
    n_total = steps + warmup
    cap = [(n + n_total + 64 + 31) // 32 for n in wl.ctx_lens]
    mb = max(cap)
    nphys = sum(cap)
    table = np.full((B, mb), -1, np.int32)
    off = 0
    for b, c in enumerate(cap):
        table[b, :c] = np.arange(off, off + c)
        off += c
    geom = ok.make_geom(B, cfg.hq, cfg.hkv, mb, nphys)

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()

    t0 = time.perf_counter()
    c0 = ok.DeviceCache(geom, block_table=table)
    dense = None
    if bf16:
        dgeom = ok.make_geom(B, cfg.hq, cfg.hkv, mb, nphys)
        dense = DenseLeg(ok, torch, dgeom, table, [n - 1 for n in wl.ctx_lens], 4)
    for b in range(B):
        k, v = wl.prefill(b)
        kd, vd = dev(k), dev(v)
        ok.prefill_quantize(c0, b, kd, vd, cfg.dtype)
        if dense is not None:
            dense.write(b, kd, vd)
    torch.cuda.synchronize()
    print("batch48: prefilled %d sequences (%.1f s)" % (B, time.perf_counter() - t0),
          file=sys.stderr, flush=True)
    caches = [c0]
    for _ in range(L - 1):
        c = ok.DeviceCache(geom, block_table=table)
        for name in ("pool", "pool_norm", "res_k", "res_v", "res_norm", "seq_state"):
            getattr(c, name).copy_(getattr(c0, name))
        caches.append(c)
    torch.cuda.synchronize()
    print("batch48: %d layer caches resident (%.1f s)" % (L, time.perf_counter() - t0),
          file=sys.stderr, flush=True)
    stp = list(wl.steps(n_total))
    kn_d = [dev(x[0]) for x in stp]
    vn_d = [dev(x[1]) for x in stp]
    q_d = [dev(x[2]) for x in stp]
    max_ctx = max(wl.ctx_lens) + n_total + 64
    S, nbytes = ok.decode_workspace_bytes(geom, max_ctx, args.splits)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(B, cfg.hq, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, cfg.hq, dtype=torch.float32, device="cuda")
    setup_s = time.perf_counter() - t0

    stream = torch.cuda.current_stream()
    if args.unfused:
        calls = [[(ok.prepare_append_kv(c, kn_d[i], vn_d[i], cfg.dtype, stream=stream),
                   ok.prepare_decode_attn(c, q_d[i], cfg.dtype, out, lse, ws, max_ctx, S,
                                          args.variant, stream=stream))
                  for c in caches] for i in range(n_total)]
    else:
        calls = [[(None, ok.prepare_decode_step(c, kn_d[i], vn_d[i], cfg.dtype, q_d[i],
                                                 cfg.dtype, out, lse, ws, max_ctx, S,
                                                 args.variant, stream=stream))
                  for c in caches] for i in range(n_total)]

    def step(i, ev=None, ev_layer=-1, ap=None, ap_layer=-1):
        for li, (app, att) in enumerate(calls[i]):
            if app is not None:
                if li == ap_layer:
                    ap[0].record()
                app()
                if li == ap_layer:
                    ap[1].record()
            if li == ev_layer:
                ev[0].record()
            att()
            if li == ev_layer:
                ev[1].record()

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    n0 = caches[0].seq_state.cpu().numpy()[:, 0].astype(np.int64)
    attn_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    app_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t_beg, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_beg.record()
    for s_i in range(steps):
        step(warmup + s_i, attn_ev[s_i], (7 * s_i) % L, app_ev[s_i], (7 * s_i + 3) % L)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_beg.elapsed_time(t_end)
    attn_us_pair = event_us(attn_ev)
    append_us = event_us(app_ev) if args.unfused else None
    # (as for the single-sequence workloads: one launch per layer step is
    # timed by the region over the launches)
    one_launch = not args.unfused and args.variant != 1
    attn_us = total_ms * 1000.0 / (steps * L) if one_launch else attn_us_pair
    assert int(caches[0].error_flag.item()) == 0
    n_mid = n0 + 1 + steps // 2
    bytes_attn = sum(algorithmic_bytes(int(n), quantized(int(n)), cfg.hq, cfg.hkv) for n in n_mid)
    if not args.unfused:
        bytes_attn += append_bytes(B, cfg.hkv, False)
    achieved = bytes_attn / (attn_us * 1e-6) / 1e9
    int2_bytes = sum(int(n) // 32 * (cfg.hkv * 3072 + 64) + 128 * (cfg.hkv * 512 + 2)
                     for n in n0) * L
    bf16_bytes = int(np.sum(n0)) * cfg.hkv * 128 * 2 * 2 * L
    wdesc = "qwen3-8b-shape decode, batch 48, contexts 8K..32K, 36 layers"
    res = {
        "workload": wdesc,
        "value": B * steps / (total_ms / 1000.0),
        "unit": "decode tokens/s",
        "steps": steps, "warmup": warmup, "ms_per_step": total_ms / steps,
        "config": {"workload": wdesc, "batch": B, "num_q_heads": cfg.hq,
                   "num_kv_heads": cfg.hkv, "head_dim": 128, "mean_ctx": float(np.mean(n0)),
                   "layers": L, "splits": S},
        "ctx_tokens_per_s": float(np.sum(n0 + 1 + (steps - 1) / 2.0)) * L / (total_ms / 1000.0),
        "us_per_layer_step": total_ms * 1000.0 / (steps * L),
        "step_launches": 2 if args.unfused or args.variant == 1 else 1,
        "attn_us_per_layer": attn_us,
        "attn_us_is": ("decode_step, one launch per layer step: timed region / launches"
                       if one_launch else "decode_attn between events"),
        "attn_us_event_pair": attn_us_pair,
        "append_us_per_layer": append_us,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (counter_traffic(BATCH48_PROFILE)
                                 if args.variant != 1 and not args.splits and not args.unfused
                                 else None),
                     "kernel": kernel_desc(args),
                     "algorithmic_bytes": bytes_attn},
        "cache_bytes_int2_36_layers": int2_bytes,
        "cache_bytes_bf16_36_layers": bf16_bytes,
        "setup_s": setup_s,
    }
    del caches, c0, ws, calls
    torch.cuda.empty_cache()
    if dense is not None:
        dense.replicate()
        res["bf16_baseline"] = dense.time(q_d, 20, 4, 0, attn_us_pair)
    return res


def main():
    args = parse()
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode (it would "
              "shard by KV head, sequence or context, each GPU running these kernels on its "
              "share)", file=sys.stderr)
        sys.exit(2)
    import torch

    import int2_kv_cache_amd as ok
    from int2_kv_cache_amd import synth

    torch.cuda.set_device(0)
    common = {"n_gpus": 1, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
              "dtype": "fp32" if args.variant == 1 else "fp16",
              "dtype_detail": ("INT2 cache; fp32 vector math" if args.variant == 1 else
                               "INT2 cache; fp16 MFMA operands, fp32 accumulate"),
              "data": "synthetic (seeded; K outliers/sinks/log-normal norms, V and q N(0,1))"}
    if args.batch48:
        steps = args.steps if args.steps != 100 else 10
        warm = args.warmup if args.warmup != 5 else 2
        r = batch48_workload(ok, torch, synth, args, steps, warm, not args.no_bf16)
        r["metric"] = "decode tokens/s, batch 48 ragged 8K..32K, 36 layers resident"
        r.update(common)
        print(json.dumps(r), flush=True)
        return

    head = decode_workload(ok, torch, synth, args, args.workload, args.steps, args.warmup,
                           bf16=not args.no_bf16, cpu=not args.no_cpu, stateless=True,
                           layers=args.layers, ctx=args.ctx,
                           prefill_cpu=not args.no_cpu and args.workload == "multimodal-64k")
    print("headline done: attn %.2f us" % head["attn_us"], file=sys.stderr, flush=True)
    res = {"metric": "INT2 decode-attn µs/step, ctx tokens/s & % HBM peak; 128K ctx bs1, 16K bs48",
           "value": head.pop("value"), "unit": head.pop("unit"), "n_gpus": 1,
           "steps": head.pop("steps"), "warmup": head.pop("warmup"),
           "ms_per_step": head.pop("ms_per_step")}
    res.update(common)
    head.pop("workload")
    res.update(head)
    res["roofline"]["measured_copy_gbs"] = copy_ceiling_gbs()
    res["roofline"]["frac_of_measured_copy"] = (res["roofline"]["achieved"] /
                                                res["roofline"]["measured_copy_gbs"])
    if not args.headline_only and not args.ctx:
        for w in ("llama-32k", "multimodal-64k"):
            if w == args.workload:
                continue
            key = w.replace("-", "_")
            res[key] = decode_workload(ok, torch, synth, args, w, min(args.steps, 50),
                                       args.warmup, bf16=not args.no_bf16, cpu=not args.no_cpu,
                                       stateless=False,
                                       prefill_cpu=not args.no_cpu and w == "multimodal-64k")
            print("%s done: attn %.2f us" % (w, res[key]["attn_us"]), file=sys.stderr, flush=True)
        res["batch48"] = batch48_workload(ok, torch, synth, args, 10, 2, not args.no_bf16)
        print("batch48 done: attn %.2f us per layer" % res["batch48"]["attn_us_per_layer"],
              file=sys.stderr, flush=True)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
