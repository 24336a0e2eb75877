#!/usr/bin/env python3
"""Benchmark of the OScaR INT2 decode path on one MI355X.

Workload (the headline configuration): Qwen3-8B-shaped single-sequence decode
at 128K context -- batch 1, 32 query heads / 8 KV heads, head dim 128, bf16
inputs, 131072 tokens after the first step (130944 INT2 + 128 fp16).  The
cache is prefilled with 131071 synthetic tokens, then every timed step runs,
for each of L distinct layer caches, the whole decode hot path:
  append_kv   -- FHT + Omni-Token Scaling of the new Key, residual-window
                 bookkeeping, INT2 flush of a 32-token block when due
  decode_attn -- query FHT, split-K attention over the INT2 blocks and the
                 fp16 window, cross-split LSE reduce.
L copies (default 8, 806 MB) are cycled so the 256 MB Infinity Cache cannot
serve a layer from a previous visit.  `--workload llama-32k` (Llama-3.1-8B
shape, 32K, 32 layers) and `--workload multimodal-64k` (bulk prefill
throughput, then decode, 16 layers) run the other single-sequence workloads
the same way.

Output: one JSON line.  value = context tokens attended per second (whole job),
plus the per-layer microseconds, the roofline of the attention kernels and
the CPU oracle timed on a bounded sample of the same workload.
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
# layer caches cycled so that they exceed 3x the 256 MB Infinity Cache)
WORKLOADS = {
    "llama-32k": (1, "llama-3.1-8b-shape decode, 32K ctx, batch 1", 32),
    "qwen3-128k": (2, "qwen3-8b-shape decode, 128K ctx, batch 1", 8),
    "multimodal-64k": (4, "qwen3-vl-8b-shape multimodal prefill + decode, 64K ctx, batch 1", 16),
}
# the decode-attention kernels and the headers they compile from
ATTN_SRC = [os.path.join(ROOT, "int2_kv_cache_amd", "csrc", f)
            for f in ("oscar_attn.hip", "oscar_device.hpp", "oscar_host.hpp")]
PROFILE = os.path.join(ROOT, "profiles", "decode_attn_qwen3-8b-128k.md")


def counter_traffic():
    """HBM bytes of one attention launch from the committed rocprofv3 counters
    (FETCH_SIZE / WRITE_SIZE, scaled by the same counters on a plain copy),
    or None when the attention sources (kernel file and the headers it
    includes) have changed since they were taken."""
    import hashlib
    try:
        h = hashlib.sha256()
        for f in ATTN_SRC:
            h.update(open(f, "rb").read())
        src = h.hexdigest()[:16]
        line = [l for l in open(PROFILE) if l.startswith("counters:")][0]
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3-128k", choices=sorted(WORKLOADS),
                    help="qwen3-128k: Qwen3-8B shape at 128K (default); llama-32k: "
                         "Llama-3.1-8B shape at 32K; multimodal-64k: Qwen3-VL-8B-like "
                         "multimodal 64K (prefill + decode)")
    ap.add_argument("--layers", type=int, default=0,
                    help="layer caches cycled (0: enough to exceed 3x the 256 MB Infinity Cache)")
    ap.add_argument("--ctx", type=int, default=0, help="context at the first step (0: the workload's)")
    ap.add_argument("--variant", type=int, default=0, help="0 auto, 1 VALU, 2 MFMA")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--hw-rsqrt", action="store_true",
                    help="Key scaling factor from the hardware rsqrt (OSCAR_SCALE_HW_RSQ)")
    ap.add_argument("--no-bf16", action="store_true",
                    help="skip the bf16 (unquantized) decode-attention baseline")
    ap.add_argument("--cpu-heads", type=int, default=8,
                    help="query heads of the oracle sample (scaled to all heads)")
    ap.add_argument("--head-norm", action="store_true",
                    help="HEAD norm scope (a norm per token and KV head) instead of TOKEN")
    ap.add_argument("--flush128", action="store_true",
                    help="quantize the full 128-token window at once (four blocks) instead "
                         "of one block per flush")
    ap.add_argument("--q-standalone", action="store_true",
                    help="rotate the query with its own oscar_rotate_scale launch and pass "
                         "q' as fp32, instead of the rotation inside decode attention")
    ap.add_argument("--batch48", action="store_true",
                    help="instead of the headline run: the batched workload (48 ragged "
                         "sequences of 8K..32K tokens, every one of 36 layer caches resident), "
                         "one JSON line of its own")
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


def cpu_baseline(wl, k, v, steps, hq, args):
    """The oracle as it stands on a bounded sample of the same workload: its
    append of one step's token, then decode attention for every query head
    over the full context, the heads spread over host threads (the oracle's
    C code runs outside the interpreter lock and is re-entrant).  Also timed
    on one thread for `cpu_heads` heads, scaled to all heads."""
    import concurrent.futures as cf

    import oracle
    cfg = wl.cfg
    mb = (wl.ctx_lens[0] + 4096) // 32
    orc = oracle.OracleCache(1, cfg.hq, cfg.hkv, mb, mb,
                             norm_scope=oracle.NORM_HEAD if args.head_norm else oracle.NORM_TOKEN,
                             flush_tokens=128 if args.flush128 else 32)
    orc.prefill(0, k, v, cfg.dtype)
    kn, vn, q = steps[0]
    t0 = time.perf_counter()
    orc.append(kn, vn, cfg.dtype)
    t_append = time.perf_counter() - t0
    qr = oracle.rotate_query(q, cfg.dtype)
    n = orc.n(0)
    # one thread, a sample of the heads
    heads = list(range(0, hq, max(1, hq // args.cpu_heads)))[: args.cpu_heads]
    t0 = time.perf_counter()
    for i in heads:
        orc.decode_attn_one(qr, 0, i)
    t1 = t_append + (time.perf_counter() - t0) * hq / len(heads)
    # all heads over the host's threads (at most 16)
    threads = max(1, min(16, os.cpu_count() or 1))
    t0 = time.perf_counter()
    with cf.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(lambda i: orc.decode_attn_one(qr, 0, i), range(hq)))
    tn = t_append + (time.perf_counter() - t0)
    return {"value": n / tn, "unit": "ctx tokens/s", "cores": threads, "kind": "oracle",
            "sample": "one decode step of one layer at n=%d: append (%.3f s) + attention for all "
                      "%d query heads on %d threads (%.2f s)" % (n, t_append, hq, threads, tn - t_append),
            "single_core_value": n / t1,
            "single_core_sample": "append + %d of %d heads on one thread, scaled to all heads "
                                  "(%.2f s per step)" % (len(heads), hq, t1),
            "cpu": cpu_model(), "host_threads": os.cpu_count()}


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), else the machine type."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


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
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
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


def batch48(args):
    """The batched decode workload: 48 sequences with contexts drawn from
    8K..32K (block-table indexed, blocks packed per sequence), 32/8 heads,
    bf16; one layer's cache is prefilled and copied to all 36 layers, which
    stay resident.  A step appends one token to every sequence and runs
    decode attention, layer by layer.  Reports decode tokens/s (48 per step)
    and the attention's algorithmic bandwidth."""
    import torch

    import int2_kv_cache_amd as ok
    from int2_kv_cache_amd import synth

    torch.cuda.set_device(0)
    wl = synth.workload(3)
    cfg = wl.cfg
    L = 36
    B = cfg.batch
    steps = args.steps if args.steps != 100 else 10
    warm = args.warmup if args.warmup != 5 else 2
    n_total = steps + warm
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
    if not args.no_bf16:
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
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(B, cfg.hq, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(B, cfg.hq, dtype=torch.float32, device="cuda")
    setup_s = time.perf_counter() - t0

    def step(i, ev=None, ev_layer=-1):
        for li, c in enumerate(caches):
            ok.append_kv(c, kn_d[i], vn_d[i], cfg.dtype)
            if li == ev_layer:
                ev[0].record()
            ok.decode_attn(c, q_d[i], cfg.dtype, out, lse, ws, max_ctx, S, args.variant)
            if li == ev_layer:
                ev[1].record()

    for i in range(warm):
        step(i)
    torch.cuda.synchronize()
    n0 = caches[0].seq_state.cpu().numpy()[:, 0].astype(np.int64)
    attn_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t_beg, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_beg.record()
    for s_i in range(steps):
        step(warm + s_i, attn_ev[s_i], (7 * s_i) % L)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_beg.elapsed_time(t_end)
    attn_us = float(np.mean([e[0].elapsed_time(e[1]) for e in attn_ev])) * 1000.0
    assert int(caches[0].error_flag.item()) == 0
    n_mid = n0 + 1 + steps // 2
    q_mid = 32 * ((np.maximum(0, n_mid - 128) + 31) // 32)
    bytes_attn = sum(algorithmic_bytes(int(n), int(q), cfg.hq, cfg.hkv) for n, q in zip(n_mid, q_mid))
    achieved = bytes_attn / (attn_us * 1e-6) / 1e9
    int2_bytes = sum(int(n) // 32 * (cfg.hkv * 3072 + 64) + 128 * (cfg.hkv * 512 + 2)
                     for n in n0) * L
    bf16_bytes = int(np.sum(n0)) * cfg.hkv * 128 * 2 * 2 * L
    res = {
        "metric": "decode tokens/s, batch 48 ragged 8K..32K, 36 layers resident",
        "value": B * steps / (total_ms / 1000.0),
        "unit": "decode tokens/s",
        "n_gpus": 1, "steps": steps, "warmup": warm,
        "ms_per_step": total_ms / steps,
        "higher_is_better": True,
        "dtype": "fp16",
        "dtype_detail": "INT2 cache; fp16 MFMA operands, fp32 accumulate",
        "data": "synthetic (seeded; K outliers/sinks/log-normal norms, V and q N(0,1))",
        "config": {"workload": "qwen3-8b-shape decode, batch 48, contexts 8K..32K, 36 layers",
                   "batch": B, "num_q_heads": cfg.hq, "num_kv_heads": cfg.hkv,
                   "head_dim": 128, "mean_ctx": float(np.mean(n0)), "layers": L, "splits": S},
        "ctx_tokens_per_s": float(np.sum(n0 + 1 + (steps - 1) / 2.0)) * L / (total_ms / 1000.0),
        "us_per_layer_step": total_ms * 1000.0 / (steps * L),
        "attn_us_per_layer": attn_us,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": "decode_attn (split-K attention + LSE reduce, timed together)",
                     "algorithmic_bytes": bytes_attn},
        "cache_bytes_int2_36_layers": int2_bytes,
        "cache_bytes_bf16_36_layers": bf16_bytes,
        "setup_s": setup_s,
    }
    if dense is not None:
        del caches, c0
        dense.replicate()
        res["bf16_baseline"] = dense.time(q_d, 20, 4, 0, attn_us)
    print(json.dumps(res), flush=True)


def main():
    args = parse()
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.batch48:
        if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
            print("bench.py runs on one GPU only", file=sys.stderr)
            sys.exit(2)
        batch48(args)
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
    wid, wname, default_layers = WORKLOADS[args.workload]
    wl = synth.workload(wid, ctx=args.ctx) if args.ctx else synth.workload(wid)
    ctx = wl.ctx_lens[0]
    cfg = wl.cfg
    L = args.layers or default_layers
    n_steps_total = args.warmup + args.steps
    max_ctx = ctx + n_steps_total + 64
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
    if not args.no_bf16:
        # the bf16 baseline's caches: the same prefilled tokens, at least two
        # layers and enough to exceed 3x the 256 MB Infinity Cache (two at 128K)
        dgeom = ok.make_geom(1, cfg.hq, cfg.hkv, mb, mb)
        dense = DenseLeg(ok, torch, dgeom, None, [ctx - 1], max(2, -(-3 * 256 * 2**20 // (
            (ctx - 1) * cfg.hkv * 512))))
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
    steps = list(wl.steps(n_steps_total))
    kn_d = [dev(s[0]) for s in steps]
    vn_d = [dev(s[1]) for s in steps]
    q_d = [dev(s[2]) for s in steps]
    S, nbytes = ok.decode_workspace_bytes(geom, max_ctx, args.splits)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
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

    def step(i, ev=None, ev_layer=-1):
        for li, c in enumerate(caches):
            ok.append_kv(c, kn_d[i], vn_d[i], cfg.dtype)
            if li == ev_layer:
                ev[0].record()
            attend(c, i)
            if li == ev_layer:
                ev[1].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    n0 = int(caches[0].seq_state[0, 0].item())

    # timed region: whole steps.  In step s the decode_attn call of layer
    # s mod L is bracketed by a pair of events on the stream it runs on
    # (torch's current stream, which the binding passes): one pair per step,
    # since an event pair around every call costs the whole step ~5 us per
    # layer on this GPU.
    attn_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    t_beg, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_beg.record()
    for s_i in range(args.steps):
        step(args.warmup + s_i, attn_ev[s_i], s_i % L)
    t_end.record()
    torch.cuda.synchronize()
    total_ms = t_beg.elapsed_time(t_end)
    attn_ms = [ev[0].elapsed_time(ev[1]) for ev in attn_ev]
    st = caches[0].seq_state.cpu().numpy()[0]
    flag = int(caches[0].error_flag.item())
    assert flag == 0, "cache error flag %d" % flag
    n1, Q1 = int(st[0]), int(st[1])

    copy_gbs = copy_ceiling_gbs()   # after the timed region
    ms_per_step = total_ms / args.steps
    us_per_layer = ms_per_step * 1000.0 / L
    # context tokens attended in the timed region (every layer, every step)
    ctx_tokens = sum(n0 + 1 + s for s in range(args.steps)) * L
    value = ctx_tokens / (total_ms / 1000.0)
    attn_us = float(np.mean(attn_ms)) * 1000.0
    n_mid = n0 + 1 + args.steps // 2
    if args.flush128:
        q_mid = 128 * ((n_mid - 1) // 128) if n_mid > 128 else 0
    else:
        q_mid = 32 * ((max(0, n_mid - 128) + 31) // 32)
    bytes_attn = algorithmic_bytes(n_mid, q_mid, cfg.hq, cfg.hkv, args.head_norm)
    achieved = bytes_attn / (attn_us * 1e-6) / 1e9
    res = {
        "metric": "INT2 decode-attn µs/step, ctx tokens/s & % HBM peak; 128K ctx bs1, 16K bs48",
        "value": value,
        "unit": "ctx tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32" if args.variant == 1 else "fp16",
        "dtype_detail": ("INT2 cache; fp32 vector math" if args.variant == 1 else
                         "INT2 cache; fp16 MFMA operands, fp32 accumulate"),
        "data": "synthetic (seeded; K outliers/sinks/log-normal norms, V and q N(0,1))",
        "config": {"workload": wname,
                   "batch": 1, "num_q_heads": cfg.hq, "num_kv_heads": cfg.hkv,
                   "head_dim": 128, "ctx_first_step": ctx, "layers_cycled": L,
                   "splits": S, "variant": args.variant,
                   "norm_scope": "head" if args.head_norm else "token",
                   "flush_tokens": 128 if args.flush128 else 32,
                   "query_rotation": "standalone" if args.q_standalone else "fused",
                   "key_scale": "hw_rsq" if args.hw_rsqrt else "ieee"},
        "us_per_layer_step": us_per_layer,
        "attn_us": attn_us,
        "append_plus_gaps_us": us_per_layer - attn_us,
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": None if (args.head_norm or args.flush128 or args.q_standalone
                                         or args.hw_rsqrt)
                     else counter_traffic(),
                     "kernel": "decode_attn (split-K attention + LSE reduce, timed together)",
                     "algorithmic_bytes": bytes_attn,
                     "measured_copy_gbs": copy_gbs,
                     "frac_of_measured_copy": achieved / copy_gbs},
        "prefill_ms_per_layer": float(np.median(pre_ms)),
        "prefill_tokens_per_s": (ctx - 1) / (float(np.median(pre_ms)) / 1000.0),
        "final_state": [n1, Q1],
        "setup_s": setup_s,
    }
    res["stateless"] = stateless_calls(ok, torch, cfg, k, v)
    if dense is not None:
        res["bf16_baseline"] = dense.time(q_d, args.steps, args.warmup, 0, attn_us)
    if not args.no_cpu:
        res["cpu_baseline"] = cpu_baseline(wl, k, v, steps, cfg.hq, args)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
