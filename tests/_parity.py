"""Shared helpers of the GPU parity tests: run the same seeded inputs through
the HIP library (via the C ABI) and through the CPU oracle, and compare."""
from __future__ import annotations

import numpy as np
import torch

import int2_kv_cache_amd as ok
import oracle
from int2_kv_cache_amd import synth

ATOL = 2e-3   # max-abs tolerance on attention outputs (fp32 accumulation)


def fp32_score_tol(lse: float, v_range: float) -> float:
    """Tolerance for inputs whose scores are large: ATOL plus what rounding
    the scores to fp32 alone can do.  A score s (natural log units, about
    |lse| for the tokens that carry weight) is held to a relative 2^-24, so
    each weight can move by ~2^-24 |s| relative, and the output by that times
    the range of the Values; 2^-20 leaves a factor 16 for the dot products'
    own rounding.  For unit-scale inputs (|lse| ~ 20, range ~ 10) this adds
    ~2e-4; for Values x1000 with scores ~ 1e3 it is ~10."""
    return ATOL + 2.0 ** -20 * abs(lse) * v_range


def dev_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint16).view(np.int16)).cuda()


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def assert_same_bits(got: np.ndarray, want: np.ndarray, what: str = ""):
    """Bit-exact comparison with a short report (count, first positions and
    the largest difference in units of the last place)."""
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    if np.array_equal(got, want):
        return
    bad = np.argwhere(got != want)
    gi = got.astype(np.int64)[tuple(bad.T)]
    wi = want.astype(np.int64)[tuple(bad.T)]
    raise AssertionError("%s: %d of %d differ; first at %s got %s want %s; max |diff| %d"
                         % (what, len(bad), got.size, bad[:4].tolist(), gi[:4].tolist(),
                            wi[:4].tolist(), int(np.abs(gi - wi).max())))


def oracle_outputs(orc: "oracle.OracleCache", qr: np.ndarray, pairs):
    """The oracle's (out, lse) for every (sequence, query head) in `pairs`,
    spread over the host's threads (at most 16): the oracle's C code runs
    outside the interpreter lock and is re-entrant."""
    import concurrent.futures as cf
    import os
    pairs = list(pairs)
    with cf.ThreadPoolExecutor(max_workers=max(1, min(16, os.cpu_count() or 1))) as ex:
        res = list(ex.map(lambda bi: orc.decode_attn_one(qr, bi[0], bi[1]), pairs))
    return dict(zip(pairs, res))


def blocks_needed(ctx: int) -> int:
    return (max(0, ctx - 128) + 31) // 32 + 1


def shuffled_table(batch: int, max_blocks: int, seed: int = 99) -> np.ndarray:
    """A non-trivial block table: a random permutation of physical blocks."""
    rng = np.random.default_rng(seed)
    return rng.permutation(batch * max_blocks).astype(np.int32).reshape(batch, max_blocks)


def compare_cache(g: "ok.DeviceCache", o: "oracle.OracleCache", table: np.ndarray):
    """Bit-exact comparison of a GPU cache's valid region (state, flags,
    the records and norms of its quantized blocks, its window slots) with the
    oracle's."""
    torch.cuda.synchronize()
    st = g.seq_state.cpu().numpy()
    assert np.array_equal(st, o.seq_state), (st, o.seq_state)
    assert int(g.error_flag.cpu()[0]) == int(o.error_flag[0])
    pool = g.pool.cpu().numpy()
    pnorm = host_u16(g.pool_norm)
    rk, rv, rn = host_u16(g.res_k), host_u16(g.res_v), host_u16(g.res_norm)
    for b in range(g.geom.batch):
        n, Q = o.n(b), o.q(b)
        phys = table[b, :Q // 32]
        for j, p in enumerate(phys):
            assert_same_bits(pool[p], o.pool[p], "seq %d block %d record" % (b, j))
            assert_same_bits(pnorm[p], o.pool_norm[p], "seq %d block %d norms" % (b, j))
        slots = np.array([t % 128 for t in range(Q, n)], dtype=np.int64)
        if len(slots):
            assert_same_bits(rk[b][:, slots, :], o.res_k[b][:, slots, :], "res_k seq %d" % b)
            assert_same_bits(rv[b][:, :, slots], o.res_v[b][:, :, slots], "res_v seq %d" % b)
            assert_same_bits(rn[b][..., slots], o.res_norm[b][..., slots], "res_norm seq %d" % b)


class Pair:
    """The same cache on the GPU and in the oracle."""

    def __init__(self, wl: synth.Workload, max_ctx: int | None = None, table=None,
                 norm_scope: int = ok.NORM_TOKEN, flush_tokens: int = 32,
                 rope_table: np.ndarray | None = None):
        cfg = wl.cfg
        self.wl = wl
        mctx = max_ctx or (max(wl.ctx_lens) + 8)
        self.max_blocks = blocks_needed(mctx)
        self.table = table if table is not None else shuffled_table(cfg.batch, self.max_blocks)
        nphys = cfg.batch * self.max_blocks
        self.geom = ok.make_geom(cfg.batch, cfg.hq, cfg.hkv, self.max_blocks, nphys,
                                 norm_scope=norm_scope, flush_tokens=flush_tokens,
                                 rope_max_pos=0 if rope_table is None else len(rope_table))
        self.gpu = ok.DeviceCache(self.geom, block_table=torch.from_numpy(self.table),
                                  rope_table=rope_table)
        self.rope_table = rope_table
        self.orc = oracle.OracleCache(cfg.batch, cfg.hq, cfg.hkv, self.max_blocks, nphys,
                                      block_table=self.table, norm_scope=norm_scope,
                                      flush_tokens=flush_tokens, rope_table=rope_table)
        self.dtype = cfg.dtype

    def prefill(self, b: int, k: np.ndarray, v: np.ndarray, gpu_bulk: bool = True):
        self.orc.prefill(b, k, v, self.dtype)
        if len(k) == 0:
            return
        if gpu_bulk:
            ok.prefill_quantize(self.gpu, b, dev_u16(k), dev_u16(v), self.dtype)
        else:
            raise NotImplementedError

    def append(self, kn: np.ndarray, vn: np.ndarray):
        self.orc.append(kn, vn, self.dtype)
        ok.append_kv(self.gpu, dev_u16(kn), dev_u16(vn), self.dtype)

    def compare_state(self, gpu=None):
        """Bit-exact comparison of the valid cache region of `gpu` (default:
        this pair's own GPU cache) with the oracle's."""
        compare_cache(self.gpu if gpu is None else gpu, self.orc, self.table)

    def attend(self, q: np.ndarray, variant=ok.ATTN_AUTO, splits=0, max_ctx=None,
               q_dtype=None, ws=None):
        """GPU decode attention -> (out, lse) numpy.  `ws`: a workspace to
        reuse, else a fresh one."""
        cfg = self.wl.cfg
        mctx = max_ctx or (max(o for o in [self.orc.n(b) for b in range(cfg.batch)]) + 1)
        S, nbytes = ok.decode_workspace_bytes(self.geom, mctx, splits)
        if ws is None:
            ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        assert ws.numel() >= nbytes
        out = torch.empty(cfg.batch, cfg.hq, 128, dtype=torch.float32, device="cuda")
        lse = torch.empty(cfg.batch, cfg.hq, dtype=torch.float32, device="cuda")
        if q_dtype == ok.FP32:
            qt = torch.from_numpy(np.ascontiguousarray(q, np.float32)).cuda()
        else:
            qt = dev_u16(q)
        ok.decode_attn(self.gpu, qt, self.dtype if q_dtype is None else q_dtype, out, lse, ws,
                       mctx, splits, variant)
        torch.cuda.synchronize()
        return out.cpu().numpy(), lse.cpu().numpy()
