"""Seeded synthetic inputs shaped like the pages' workloads.

This module holds none of the method's arithmetic: it only draws random
numbers and casts them to the 16-bit input formats.  It serves the CPU
oracle's tests, the GPU parity tests, the smoke check and the benchmark alike.

Recipe (the shapes and distributions of the five workloads):
  * Keys   K[t, h, :] = m_t * g, g ~ N(0, 1)^128, except on each KV head's
           outlier channels, where g_c <- 20 g_c + 5.  The outlier channel set
           is fixed per KV head (4 channels, or a count drawn from U{4..8}).
  * Token multipliers m_t: 0.05 for the first 4 tokens (attention-sink-like
           low-norm tokens), otherwise exp(sigma * N(0, 1)); in the multimodal
           workload a segment pattern (text x1 for 2048 tokens, vision x5 for
           8192, audio x0.3 for 4096, repeating) plus 0.1% of the tokens at x30.
           m_t is shared by all heads of token t.
  * Optional flat sinks (Workload.flat_sinks): the sink tokens' g is instead an
           isotropic N(0, 1) vector rescaled to the norm the outlier-bearing g
           of that token had -- low-norm tokens whose energy is spread evenly
           over the channels, the shape the pages give for attention sinks (an
           extra draw after the multipliers; off by default, which leaves every
           other stream unchanged).
  * Values V ~ N(0, 1).  The pages rotate V offline by a Hadamard matrix; an
           orthonormal rotation of an i.i.d. standard normal vector is again
           i.i.d. standard normal, so drawing N(0, 1) directly gives exactly the
           distribution of a rotated V without doing any rotation here.
  * Queries q ~ N(0, 1).
  * Cast to fp16 or bf16 with round-to-nearest-even.
Random streams: numpy PCG64.  One stream (seed) draws the context lengths and
the outlier channel sets; stream (seed, 1, b) draws sequence b's prefill keys,
multipliers and values in that order; stream (seed, 2) draws the decode steps.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FP16, BF16 = 0, 1
D = 128


@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    hq: int
    hkv: int
    ctx: int | None            # context after the first decode step (None: ragged)
    dtype: int
    sigma: float | None        # log-normal sigma of the token multipliers
    outliers: tuple            # (min, max) outlier channels per KV head
    steps: int
    ragged: tuple | None = None   # (lo, hi) per-sequence contexts
    multimodal: bool = False
    layers: int = 1


CONFIGS = {
    0: Config("tiny-gqa4-1k", 1, 4, 1, 1024, FP16, 0.3, (4, 4), 1),
    1: Config("llama3.1-8b-32k", 1, 32, 8, 32768, BF16, 0.3, (4, 4), 100),
    2: Config("qwen3-8b-128k", 1, 32, 8, 131072, BF16, 0.4, (4, 8), 100),
    3: Config("qwen3-8b-b48-ragged", 48, 32, 8, None, BF16, 0.4, (4, 8), 10,
              ragged=(8192, 32768), layers=36),
    4: Config("qwen3-vl-8b-64k-mm", 1, 32, 8, 65536, BF16, None, (4, 8), 100,
              multimodal=True),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))
    return (r >> np.uint32(16)).astype(np.uint16)


def to_fp16_bits(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def cast_bits(x: np.ndarray, dtype: int) -> np.ndarray:
    return to_bf16_bits(x) if dtype == BF16 else to_fp16_bits(x)


def bits_to_f32(bits: np.ndarray, dtype: int) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)
    return bits.view(np.float16).astype(np.float32)


def segment_multiplier(t: np.ndarray) -> np.ndarray:
    """text 2048 (x1), vision 8192 (x5), audio 4096 (x0.3), repeating."""
    pos = np.asarray(t) % (2048 + 8192 + 4096)
    return np.where(pos < 2048, 1.0, np.where(pos < 2048 + 8192, 5.0, 0.3)).astype(np.float32)


@dataclass
class Workload:
    cfg: Config
    seed: int
    ctx_lens: list = field(default_factory=list)   # tokens attended at step 1
    outlier_idx: list = field(default_factory=list)  # per KV head: channel ids
    flat_sinks: bool = False   # sink tokens isotropic instead of outlier-shaped

    @property
    def batch(self):
        return self.cfg.batch

    def _keys(self, rng, T, t0, mult_fn):
        g = rng.standard_normal((T, self.cfg.hkv, D), dtype=np.float32)
        for h, idx in enumerate(self.outlier_idx):
            g[:, h, idx] = 20.0 * g[:, h, idx] + 5.0
        m = mult_fn(rng, np.arange(t0, t0 + T))
        if self.flat_sinks:
            sinks = np.arange(t0, t0 + T) < 4
            if sinks.any():
                iso = rng.standard_normal((int(sinks.sum()), self.cfg.hkv, D), dtype=np.float32)
                scale = np.linalg.norm(g[sinks].reshape(len(iso), -1), axis=1) / \
                    np.linalg.norm(iso.reshape(len(iso), -1), axis=1)
                g[sinks] = iso * scale[:, None, None]
        return g * m[:, None, None]

    def _mult_prefill(self, rng, t):
        cfg = self.cfg
        if cfg.multimodal:
            m = segment_multiplier(t)
            pool = t[t >= 4]
            k = int(round(0.001 * (len(t) + 1)))
            if k > 0 and len(pool) > 0:
                hi = rng.choice(pool, size=min(k, len(pool)), replace=False)
                m[hi - t[0]] = 30.0
        else:
            m = np.exp(cfg.sigma * rng.standard_normal(len(t))).astype(np.float32)
        m[t < 4] = 0.05
        return m.astype(np.float32)

    def _mult_step(self, rng, t):
        cfg = self.cfg
        if cfg.multimodal:
            m = segment_multiplier(t)
        else:
            m = np.exp(cfg.sigma * rng.standard_normal(len(t))).astype(np.float32)
        m[t < 4] = 0.05
        return m.astype(np.float32)

    def prefill(self, b: int, n_tokens: int | None = None):
        """Sequence b's first ctx-1 tokens: (K bits, V bits), [T, Hkv, 128]."""
        T = self.ctx_lens[b] - 1 if n_tokens is None else n_tokens
        rng = np.random.Generator(np.random.PCG64([self.seed, 1, b]))
        k = self._keys(rng, T, 0, self._mult_prefill)
        v = rng.standard_normal((T, self.cfg.hkv, D), dtype=np.float32)
        return cast_bits(k, self.cfg.dtype), cast_bits(v, self.cfg.dtype)

    def steps(self, n_steps: int):
        """Yields (k_new [B,Hkv,128], v_new [B,Hkv,128], q [B,Hq,128]) bits."""
        rng = np.random.Generator(np.random.PCG64([self.seed, 2]))
        cfg = self.cfg
        for s in range(n_steps):
            pos = np.array([L - 1 + s for L in self.ctx_lens])
            g = rng.standard_normal((cfg.batch, cfg.hkv, D), dtype=np.float32)
            for h, idx in enumerate(self.outlier_idx):
                g[:, h, idx] = 20.0 * g[:, h, idx] + 5.0
            m = self._mult_step(rng, pos)
            k = g * m[:, None, None]
            v = rng.standard_normal((cfg.batch, cfg.hkv, D), dtype=np.float32)
            q = rng.standard_normal((cfg.batch, cfg.hq, D), dtype=np.float32)
            yield (cast_bits(k, cfg.dtype), cast_bits(v, cfg.dtype),
                   cast_bits(q, cfg.dtype))


def rope_table(max_pos: int, theta: float = 1.0e6) -> np.ndarray:
    """The model's rotary-position table, an input like its weights:
    [max_pos][64] (cos, sin) pairs in fp32 for the angles pos * theta^(-i/64)
    of channel pairs (i, i + 64), computed in fp64 and rounded once.  theta
    1e6 is Qwen3's base (Llama-3.1 uses 5e5)."""
    inv = theta ** (-np.arange(64, dtype=np.float64) / 64.0)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return np.stack([np.cos(ang), np.sin(ang)], axis=-1).astype(np.float32)


def workload(cfg_id: int, *, ctx: int | None = None, batch: int | None = None,
             seed: int | None = None) -> Workload:
    """Build workload cfg_id; ctx/batch override the sizes for small cases."""
    cfg = CONFIGS[cfg_id]
    if batch is not None or ctx is not None:
        cfg = Config(cfg.name, batch if batch is not None else cfg.batch, cfg.hq,
                     cfg.hkv, ctx if ctx is not None else cfg.ctx, cfg.dtype,
                     cfg.sigma, cfg.outliers, cfg.steps,
                     None if ctx is not None else cfg.ragged, cfg.multimodal,
                     cfg.layers)
    seed = 1000 + cfg_id if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    if cfg.ragged is not None:
        lo, hi = cfg.ragged
        ctx_lens = [int(x) for x in rng.integers(lo, hi + 1, size=cfg.batch)]
    else:
        ctx_lens = [cfg.ctx] * cfg.batch
    lo, hi = cfg.outliers
    outl = []
    for _ in range(cfg.hkv):
        cnt = lo if lo == hi else int(rng.integers(lo, hi + 1))
        outl.append(np.sort(rng.choice(D, size=cnt, replace=False)))
    return Workload(cfg, seed, ctx_lens, outl)
