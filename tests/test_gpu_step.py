"""The fused decode step (oscar_decode_step) against an append followed by
decode attention on a second cache: the same out and lse bit for bit at every
step, and the same cache bytes and flags as the oracle's, through window
flushes, ragged batches, both norm scopes, 128-token flushes, RoPE, the
hardware-rsqrt scaling, many splits, the vector-ALU variant, and the
append's error paths (a full block table, a position past the RoPE table, a
corrupt state).
"""
import numpy as np
import pytest
import torch

import int2_kv_cache_amd as ok
from int2_kv_cache_amd import synth
from tests._parity import Pair, assert_same_bits, compare_cache, dev_u16, oracle_outputs, ATOL

pytestmark = pytest.mark.gpu


def _twin(pr: Pair, geom=None) -> ok.DeviceCache:
    """A second GPU cache with the pair's geometry and block table."""
    return ok.DeviceCache(geom or pr.geom, block_table=torch.from_numpy(pr.table),
                          rope_table=pr.rope_table)


def _run(pr: Pair, twin: ok.DeviceCache, n_steps: int, splits: int = 0,
         variant: int = ok.ATTN_AUTO, check_every: int = 8, v_steps=None):
    """n_steps decode steps: the pair's GPU cache (and the oracle) by append
    + attention, the twin by decode_step; outputs compared every step, the
    twin's cache with the oracle's every `check_every` steps and at the end."""
    cfg = pr.wl.cfg
    ws_a = ws_b = None
    steps = list(pr.wl.steps(n_steps)) if v_steps is None else v_steps
    for i, (kn, vn, q) in enumerate(steps):
        pr.append(kn, vn)
        mctx = max(pr.orc.n(b) for b in range(cfg.batch)) + 1
        S, nbytes = ok.decode_workspace_bytes(pr.geom, mctx, splits)
        if ws_a is None or ws_a.numel() < nbytes:
            ws_a = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
            ws_b = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        want, wlse = pr.attend(q, variant=variant, splits=splits, max_ctx=mctx, ws=ws_a)
        out = torch.empty(cfg.batch, cfg.hq, 128, dtype=torch.float32, device="cuda")
        lse = torch.empty(cfg.batch, cfg.hq, dtype=torch.float32, device="cuda")
        ok.decode_step(twin, dev_u16(kn), dev_u16(vn), cfg.dtype, dev_u16(q), cfg.dtype, out, lse,
                       ws_b, mctx, splits, variant)
        torch.cuda.synchronize()
        assert_same_bits(out.cpu().numpy().view(np.uint32), want.view(np.uint32), "out step %d" % i)
        assert_same_bits(lse.cpu().numpy().view(np.uint32), wlse.view(np.uint32), "lse step %d" % i)
        if (i + 1) % check_every == 0:
            compare_cache(twin, pr.orc, pr.table)
    compare_cache(twin, pr.orc, pr.table)
    pr.compare_state()
    return pr


def _prefilled(wl, lens, **kw):
    pr = Pair(wl, **kw)
    twin = _twin(pr)
    for b, n0 in enumerate(lens):
        k, v = wl.prefill(b, n0)
        pr.prefill(b, k, v)
        if n0:
            ok.prefill_quantize(twin, b, dev_u16(k), dev_u16(v), wl.cfg.dtype)
    return pr, twin


@pytest.mark.parametrize("cfg,n0,steps", [(0, 120, 80), (1, 1990, 70), (2, 4000, 40)])
def test_step_equals_append_then_attention(cfg, n0, steps):
    wl = synth.workload(cfg, ctx=n0 + steps + 4)
    pr, twin = _prefilled(wl, [n0])
    _run(pr, twin, steps)


def test_step_from_an_empty_sequence():
    """The first tokens of a sequence: n = 0 .. 140, through the first flush."""
    wl = synth.workload(0, ctx=150)
    pr, twin = _prefilled(wl, [0])
    _run(pr, twin, 140, check_every=20)


def test_step_ragged_batch():
    """Sequences at different places of their window: one flushes at a step
    where the others do not; one starts empty."""
    cfg = synth.CONFIGS[2]
    lens = [127, 300, 0, 1000]
    c = synth.Config("ragged4", len(lens), cfg.hq, cfg.hkv, None, cfg.dtype, cfg.sigma,
                     cfg.outliers, 1)
    wl = synth.Workload(c, 5, [L + 60 for L in lens], synth.workload(2, ctx=64).outlier_idx)
    pr, twin = _prefilled(wl, lens)
    _run(pr, twin, 40, check_every=10)


@pytest.mark.parametrize("scope,flush", [(ok.NORM_HEAD, 32), (ok.NORM_TOKEN, 128),
                                         (ok.NORM_HEAD, 128)])
def test_step_norm_scopes_and_flush128(scope, flush):
    wl = synth.workload(1, ctx=700)
    pr, twin = _prefilled(wl, [560], norm_scope=scope, flush_tokens=flush)
    _run(pr, twin, 140, check_every=35)


def test_step_with_rope():
    wl = synth.workload(1, ctx=600)
    tab = synth.rope_table(700)
    pr, twin = _prefilled(wl, [520], rope_table=tab)
    _run(pr, twin, 60, check_every=15)


@pytest.mark.parametrize("splits", [1, 7, 64])
def test_step_split_counts(splits):
    """One split (no cross-split merge) and many (the append's last arrival
    among hundreds of workgroups)."""
    wl = synth.workload(1, ctx=3000)
    pr, twin = _prefilled(wl, [2900])
    _run(pr, twin, 35, splits=splits, check_every=35)


def test_step_many_pairs():
    """Enough (sequence, KV head) pairs for 4-wave workgroups (the flush
    staging then has the least room)."""
    cfg = synth.CONFIGS[2]
    lens = [120 + 11 * b for b in range(16)]
    c = synth.Config("b16", 16, cfg.hq, cfg.hkv, None, cfg.dtype, cfg.sigma, cfg.outliers, 1)
    wl = synth.Workload(c, 9, [L + 40 for L in lens], synth.workload(2, ctx=64).outlier_idx)
    pr, twin = _prefilled(wl, lens)
    _run(pr, twin, 36, check_every=12)


def test_step_batch_in_two_rounds():
    """48 ragged sequences in four splits each: 1536 workgroups, more than the
    chip holds at once, so the launch runs in two rounds while the first
    round's appenders already rewrite their sequences' states.  The launch
    order (longest first) comes from a snapshot taken before the launch;
    every step must still equal append + attention bit for bit."""
    cfg = synth.CONFIGS[2]
    rng = np.random.default_rng(48)
    lens = [int(x) for x in rng.integers(0, 2600, 48)]
    lens[5], lens[17] = 0, 127   # an empty sequence, one about to flush
    c = synth.Config("b48r", 48, cfg.hq, cfg.hkv, None, cfg.dtype, cfg.sigma, cfg.outliers, 1)
    wl = synth.Workload(c, 48, [L + 40 for L in lens], synth.workload(2, ctx=64).outlier_idx)
    pr, twin = _prefilled(wl, lens)
    _run(pr, twin, 34, splits=4, check_every=17)


@pytest.mark.parametrize("grp", [1, 2, 8])
def test_step_group_sizes(grp):
    wl = synth.workload(1, ctx=700)
    hkv = 8 if grp <= 2 else 2
    cfg = synth.Config("grp", 1, hkv * grp, hkv, 700, synth.BF16, 0.3, (4, 4), 1)
    wl2 = synth.Workload(cfg, 77, [700], wl.outlier_idx[:hkv])
    pr, twin = _prefilled(wl2, [600])
    _run(pr, twin, 40, check_every=40)


def test_step_valu_variant():
    wl = synth.workload(1, ctx=400)
    pr, twin = _prefilled(wl, [300])
    _run(pr, twin, 40, variant=ok.ATTN_VALU, check_every=40)


def test_step_hw_rsqrt_scaling():
    """The hardware-rsqrt scaling (no oracle counterpart): the fused step's
    cache and outputs equal the append + attention path's bit for bit."""
    wl = synth.workload(1, ctx=500)
    cfg = wl.cfg
    geom = ok.make_geom(1, cfg.hq, cfg.hkv, 20, 20, key_scale=ok.SCALE_HW_RSQ)
    a = ok.DeviceCache(geom)
    b = ok.DeviceCache(geom)
    k, v = wl.prefill(0, 400)
    for c in (a, b):
        ok.prefill_quantize(c, 0, dev_u16(k), dev_u16(v), cfg.dtype)
    S, nbytes = ok.decode_workspace_bytes(geom, 500)
    wa = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    wb = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = [torch.empty(1, cfg.hq, 128, device="cuda") for _ in range(2)]
    lses = [torch.empty(1, cfg.hq, device="cuda") for _ in range(2)]
    for kn, vn, q in wl.steps(40):
        ok.append_kv(a, dev_u16(kn), dev_u16(vn), cfg.dtype)
        ok.decode_attn(a, dev_u16(q), cfg.dtype, outs[0], lses[0], wa, 500)
        ok.decode_step(b, dev_u16(kn), dev_u16(vn), cfg.dtype, dev_u16(q), cfg.dtype, outs[1],
                       lses[1], wb, 500)
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.int32), outs[1].view(torch.int32))
        assert torch.equal(lses[0].view(torch.int32), lses[1].view(torch.int32))
    for name in ("seq_state", "error_flag", "pool", "pool_norm", "res_k", "res_v", "res_norm"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name


def test_step_against_oracle_outputs():
    """The fused step's outputs against the oracle's attention within the
    attention tolerance, across a flush."""
    wl = synth.workload(0, ctx=300)
    pr, twin = _prefilled(wl, [250])
    cfg = wl.cfg
    ws = None
    for i, (kn, vn, q) in enumerate(wl.steps(12)):
        pr.orc.append(kn, vn, cfg.dtype)
        mctx = pr.orc.n(0) + 1
        S, nbytes = ok.decode_workspace_bytes(pr.geom, mctx)
        ws = ws if ws is not None and ws.numel() >= nbytes else torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
        out = torch.empty(1, cfg.hq, 128, device="cuda")
        lse = torch.empty(1, cfg.hq, device="cuda")
        ok.decode_step(twin, dev_u16(kn), dev_u16(vn), cfg.dtype, dev_u16(q), cfg.dtype, out, lse,
                       ws, mctx)
        torch.cuda.synchronize()
        from oracle import rotate_query
        want = oracle_outputs(pr.orc, rotate_query(q, cfg.dtype), [(0, h) for h in range(cfg.hq)])
        got = out.cpu().numpy()
        for h in range(cfg.hq):
            assert np.abs(got[0, h] - want[(0, h)][0]).max() <= ATOL, (i, h)
    compare_cache(twin, pr.orc, pr.table)


# ------------------------------------------------------------ the append's errors

def test_step_full_block_table_drops_the_append():
    """A table without room for the next flush: OSCAR_FLAG_CAPACITY, the token
    is dropped, attention covers the unchanged cache -- as append + attention."""
    wl = synth.workload(0, ctx=400)
    pr, twin = _prefilled(wl, [200], max_ctx=200)
    _run(pr, twin, 60, check_every=20)
    assert int(twin.error_flag.cpu()[0]) & ok.FLAG_CAPACITY


def test_step_position_past_rope_table():
    wl = synth.workload(0, ctx=300)
    tab = synth.rope_table(230)
    pr, twin = _prefilled(wl, [225], rope_table=tab)
    _run(pr, twin, 10, check_every=10)
    assert int(twin.error_flag.cpu()[0]) & ok.FLAG_POSITION


def test_step_corrupt_state():
    """{n, Q} that no append leaves: BADSTATE, nothing appended, zeros out."""
    wl = synth.workload(0, ctx=300)
    pr, twin = _prefilled(wl, [200])
    twin.seq_state.copy_(torch.tensor([[150, 7]], dtype=torch.int32))
    cfg = wl.cfg
    kn, vn, q = next(wl.steps(1))
    S, nbytes = ok.decode_workspace_bytes(pr.geom, 300)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((1, cfg.hq, 128), 7.0, device="cuda")
    lse = torch.empty(1, cfg.hq, device="cuda")
    ok.decode_step(twin, dev_u16(kn), dev_u16(vn), cfg.dtype, dev_u16(q), cfg.dtype, out, lse,
                   ws, 300)
    torch.cuda.synchronize()
    assert int(twin.error_flag.cpu()[0]) & ok.FLAG_BADSTATE
    assert np.array_equal(twin.seq_state.cpu().numpy(), [[150, 7]])
    assert float(out.abs().max()) == 0.0
    assert int(twin.append_sync.abs().max()) == 0
