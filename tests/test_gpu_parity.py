"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact for the rotation, the norms, the INT2 codes, the packed records,
the residual window and the sequence state; max-abs <= 2e-3 for attention.
"""
import numpy as np
import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]

if gpu_available():
    import torch
    import int2_kv_cache_amd as ok
    import oracle
    from int2_kv_cache_amd import synth
    from _parity import ATOL, Pair, assert_same_bits, dev_u16, fp32_score_tol, host_u16


@pytest.mark.parametrize("dtype", [0, 1])
def test_rotate_query_bit_exact(dtype):
    wl = synth.workload(1, ctx=64)
    qs = [q for _, _, q in wl.steps(3)]
    q = np.concatenate(qs)                       # [3, 32, 128]
    if dtype == 0:
        q = synth.to_fp16_bits(synth.bits_to_f32(q, 1))
    out = torch.empty(q.shape, dtype=torch.float32, device="cuda")
    ok.rotate_scale(dev_u16(q), dtype, ok.ROT_QUERY, q_out=out)
    torch.cuda.synchronize()
    want = oracle.rotate_query(q, dtype)
    assert_same_bits(out.cpu().numpy().view(np.uint32), want.view(np.uint32), "q'")


@pytest.mark.parametrize("cfg,hkv", [(0, None), (2, None), (2, 5), (4, None)])
def test_rotate_scale_key_bit_exact(cfg, hkv):
    wl = synth.workload(cfg, ctx=300)
    k, _ = wl.prefill(0, 200)
    if hkv is not None:
        k = np.ascontiguousarray(k[:, :hkv])
    dt = wl.cfg.dtype
    khat = torch.empty(k.shape, dtype=torch.int16, device="cuda")
    norm = torch.empty(k.shape[0], dtype=torch.int16, device="cuda")
    ok.rotate_scale(dev_u16(k), dt, ok.ROT_KEY, khat_out=khat, norm_out=norm)
    torch.cuda.synchronize()
    wk, wn = oracle.rotate_scale_key(k, dt)
    assert_same_bits(host_u16(norm), wn, "norm")
    assert_same_bits(host_u16(khat), wk, "k_hat")


def test_rotate_scale_zero_token():
    k = np.zeros((2, 8, 128), np.uint16)
    khat = torch.ones(k.shape, dtype=torch.int16, device="cuda")
    norm = torch.ones(2, dtype=torch.int16, device="cuda")
    ok.rotate_scale(dev_u16(k), 1, ok.ROT_KEY, khat_out=khat, norm_out=norm)
    torch.cuda.synchronize()
    assert not khat.cpu().numpy().any() and not norm.cpu().numpy().any()


@pytest.mark.parametrize("nb,hkv", [(1, 1), (5, 8), (3, 3)])
def test_quant_pack_bit_exact(nb, hkv):
    rng = np.random.default_rng(nb * 10 + hkv)
    wl = synth.workload(2, ctx=32 * nb + 10)
    k, v = wl.prefill(0, 32 * nb)
    k, v = np.ascontiguousarray(k[:, :hkv]), np.ascontiguousarray(v[:, :hkv])
    khat, knorm = oracle.rotate_scale_key(k, synth.BF16)
    v16 = oracle.in_to_f16(v, synth.BF16)
    # a few constant channels and exact ties
    khat[:, 0, 5] = khat[0, 0, 5]
    v16[:, 0, :32] = synth.to_fp16_bits(rng.integers(-2, 2, (32 * nb, 32)) * 0.5)
    rec = torch.zeros(nb, hkv, 3072, dtype=torch.uint8, device="cuda")
    nrm = torch.zeros(nb, 32, dtype=torch.int16, device="cuda")
    ok.quant_pack(dev_u16(khat), dev_u16(knorm), dev_u16(v16), rec, nrm)
    torch.cuda.synchronize()
    wr, wn = oracle.quant_pack(khat, knorm, v16)
    assert_same_bits(rec.cpu().numpy(), wr, "records")
    assert_same_bits(host_u16(nrm), wn, "norms")


def _tie_groups(rng, shape):
    """Values whose quantization quotients (x - min) / delta are exact half
    integers under a delta that is not a power of two: per 32-value group
    min = -r d/2, max = min + 3 d, the rest min + q d/2 (q = 0..6), with
    d = m 2^e, m odd <= 15, so every value is exact in bf16 and fp16 and the
    correctly rounded 1/delta is inexact.  shape[-1] is a multiple of 32."""
    *lead, c = shape
    g = int(np.prod(lead)) * (c // 32)
    m = rng.choice(np.arange(3, 16, 2), g)
    e = rng.integers(-9, -2, g)
    d = (m * np.exp2(e)).astype(np.float64)
    r = rng.integers(0, 7, g)
    q = rng.integers(0, 7, (g, 32))
    q[:, 0], q[:, 1] = 0, 6
    x = (q - r[:, None]) * (d[:, None] / 2)
    return x.reshape(*lead, c).astype(np.float32)


def test_quant_pack_exact_ties():
    """Keys and Values whose every second quotient is a tie: the reciprocal
    fast path must hand each of them to the exact division."""
    rng = np.random.default_rng(7)
    nb, hkv = 4, 2
    wl = synth.workload(2, ctx=32 * nb + 10)
    k, v = wl.prefill(0, 32 * nb)
    khat, knorm = oracle.rotate_scale_key(np.ascontiguousarray(k[:, :hkv]), synth.BF16)
    # Key ties run along the tokens of a channel: groups of 32 tokens
    kt = _tie_groups(rng, (nb, hkv, 128, 32)).transpose(0, 3, 1, 2).reshape(32 * nb, hkv, 128)
    khat[:, :, 64:] = synth.to_fp16_bits(kt[:, :, 64:])
    v16 = synth.to_fp16_bits(_tie_groups(rng, (32 * nb, hkv, 128)))
    rec = torch.zeros(nb, hkv, 3072, dtype=torch.uint8, device="cuda")
    nrm = torch.zeros(nb, 32, dtype=torch.int16, device="cuda")
    ok.quant_pack(dev_u16(khat), dev_u16(knorm), dev_u16(v16), rec, nrm)
    torch.cuda.synchronize()
    wr, wn = oracle.quant_pack(khat, knorm, v16)
    assert_same_bits(rec.cpu().numpy(), wr, "records")


def test_prefill_and_flush_value_ties():
    """bf16 Values with exact-tie quotients through bulk prefill and through
    appends that flush blocks."""
    rng = np.random.default_rng(11)
    wl = synth.workload(1, ctx=32 * 6 + 150 + 40)
    pr = Pair(wl)
    n0 = 32 * 6 + 150
    k, _ = wl.prefill(0, n0)
    v = synth.to_bf16_bits(_tie_groups(rng, (n0, wl.cfg.hkv, 128)))
    pr.prefill(0, k, v)
    pr.compare_state()
    for kn, _, _ in wl.steps(40):
        vn = synth.to_bf16_bits(_tie_groups(rng, (1, wl.cfg.hkv, 128)))
        pr.append(kn, vn)
    pr.compare_state()


def _tiny_values(rng, shape, dtype):
    """Values whose 32-channel groups run from ordinary to far below fp16's
    smallest normal (2^-14): bf16 inputs there round to fp16's subnormal grid
    (2^-24) when stored.  Some groups hold one repeated tiny value, some
    exact zeros of either sign."""
    x = rng.standard_normal(shape).astype(np.float32)
    g = x.reshape(-1, 32)
    scale = np.float32([1.0, 1e-3, 2e-5, 3e-6, 4e-7, 6e-8, 2e-8])
    g *= scale[rng.integers(0, scale.size, size=(g.shape[0], 1))]
    rep = rng.random(g.shape[0]) < 0.05
    g[rep] = g[rep, :1] * np.float32(1e-6)
    g.ravel()[rng.integers(0, g.size, size=g.size // 50)] = 0.0
    g.ravel()[rng.integers(0, g.size, size=g.size // 50)] = -0.0
    return synth.cast_bits(x, dtype)


@pytest.mark.parametrize("cfg", [0, 2])
def test_prefill_tiny_values(cfg):
    """Values below fp16's normal range through bulk prefill and appends that
    flush: bit-exact with the oracle, which rounds every Value to fp16 before
    its range and codes."""
    rng = np.random.default_rng(41 + cfg)
    n0 = 32 * 7 + 133
    wl = synth.workload(cfg, ctx=n0 + 50)
    pr = Pair(wl)
    k, _ = wl.prefill(0, n0)
    pr.prefill(0, k, _tiny_values(rng, (n0, wl.cfg.hkv, 128), wl.cfg.dtype))
    pr.compare_state()
    for kn, _, _ in wl.steps(50):
        pr.append(kn, _tiny_values(rng, (1, wl.cfg.hkv, 128), wl.cfg.dtype))
    pr.compare_state()


@pytest.mark.parametrize("cfg,batch,steps", [(0, 1, 300), (1, 2, 200)])
def test_append_sequence_bit_exact(cfg, batch, steps):
    """Appends from an empty cache cross several window flushes."""
    wl = synth.workload(cfg, ctx=steps + 1, batch=batch)
    pr = Pair(wl, max_ctx=steps + 8)
    for i, (kn, vn, _) in enumerate(wl.steps(steps)):
        pr.append(kn, vn)
        if i in (0, 127, 128, 129, 160, steps - 1):
            pr.compare_state()


@pytest.mark.parametrize("n", [1, 31, 32, 127, 128, 129, 160, 161, 1000, 1023])
def test_prefill_equals_appends(n):
    """Bulk prefill gives the bytes n oracle appends give."""
    wl = synth.workload(1, ctx=n + 1)
    pr = Pair(wl)
    k, v = wl.prefill(0, n)
    pr.prefill(0, k, v)
    pr.compare_state()


@pytest.mark.parametrize("hkv", [1, 3, 5, 16])
def test_prefill_kv_head_counts(hkv):
    """Bulk prefill with KV-head counts that are not the workloads' 8 (the
    rotation tree pads the heads to 16; 16 heads take two lane rounds)."""
    base = synth.workload(2, ctx=300)
    cfg = synth.Config("hkv", 1, hkv, hkv, 300, synth.BF16, 0.4, (4, 8), 1)
    outl = (base.outlier_idx * 4)[:hkv]
    wl = synth.Workload(cfg, 55, [300], outl)
    pr = Pair(wl)
    k, v = wl.prefill(0, 299)
    pr.prefill(0, k, v)
    pr.compare_state()


def test_prefill_then_appends_and_ragged_batch():
    wl = synth.workload(2, ctx=None, batch=3)
    wl.ctx_lens = [300, 1000, 161]
    pr = Pair(wl)
    for b in range(3):
        k, v = wl.prefill(b)
        pr.prefill(b, k, v)
    pr.compare_state()
    for kn, vn, _ in wl.steps(40):
        pr.append(kn, vn)
    pr.compare_state()


def test_prefill_nonempty_flag_and_capacity():
    wl = synth.workload(0, ctx=400)
    pr = Pair(wl, max_ctx=200)       # capacity: blocks for 200 tokens
    k, v = wl.prefill(0, 150)
    pr.prefill(0, k, v)
    ok.prefill_quantize(pr.gpu, 0, dev_u16(k), dev_u16(v), wl.cfg.dtype)
    torch.cuda.synchronize()
    assert int(pr.gpu.error_flag.cpu()[0]) == ok.FLAG_NONEMPTY
    assert pr.gpu.seq_state.cpu().numpy()[0].tolist() == [150, 32]
    pr.gpu.error_flag.zero_()
    # too many blocks for the table: rejected on the host
    with pytest.raises(ok.OscarError):
        big_k, big_v = wl.prefill(0, 399)
        ok.prefill_quantize(pr.gpu, 0, dev_u16(big_k), dev_u16(big_v), wl.cfg.dtype)
    # appends past capacity set the flag and are dropped, as in the oracle
    for kn, vn, _ in wl.steps(120):
        pr.append(kn, vn)
    pr.compare_state()
    assert int(pr.gpu.error_flag.cpu()[0]) == ok.FLAG_CAPACITY


def _attn_case(wl, splits_list, variants, steps=1):
    pr = Pair(wl)
    for b in range(wl.cfg.batch):
        k, v = wl.prefill(b)
        pr.prefill(b, k, v)
    worst = 0.0
    for kn, vn, q in wl.steps(steps):
        pr.append(kn, vn)
        want, wlse = pr.orc.decode_attn(oracle.rotate_query(q, wl.cfg.dtype))
        for var in variants:
            for S in splits_list:
                got, glse = pr.attend(q, variant=var, splits=S)
                err = np.abs(got - want).max()
                worst = max(worst, err)
                assert err <= ATOL, (var, S, err)
                assert np.abs(glse - wlse).max() <= 1e-3 * max(1.0, np.abs(wlse).max())
    return worst


VARIANTS = [1, 2]   # VALU, MFMA


@pytest.mark.parametrize("variant", VARIANTS)
def test_attention_tiny_config(variant):
    wl = synth.workload(0)
    _attn_case(wl, [0, 1, 2, 7], [variant], steps=2)


@pytest.mark.parametrize("variant", VARIANTS)
@pytest.mark.parametrize("ctx", [1, 33, 129, 161, 2000])
def test_attention_llama_shape_small(variant, ctx):
    wl = synth.workload(1, ctx=ctx)
    _attn_case(wl, [0, 3], [variant])


@pytest.mark.parametrize("variant", VARIANTS)
def test_attention_ragged_batch(variant):
    wl = synth.workload(3, batch=4, ctx=None)
    wl.ctx_lens = [4000, 129, 1500, 8200]
    _attn_case(wl, [0, 5], [variant])


@pytest.mark.parametrize("grp", [1, 2, 8])
@pytest.mark.parametrize("variant", VARIANTS)
def test_attention_group_sizes(variant, grp):
    """GQA groups of 1, 2 and 8 query heads per KV head (the workloads use 4)."""
    wl = synth.workload(1, ctx=700)
    hkv = 8 if grp <= 2 else 2
    cfg = synth.Config("grp", 1, hkv * grp, hkv, 700, synth.BF16, 0.3, (4, 4), 1)
    wl2 = synth.Workload(cfg, 77, [700], wl.outlier_idx[:hkv])
    _attn_case(wl2, [0, 3], [variant], steps=1)


def test_attention_prerotated_query():
    wl = synth.workload(1, ctx=700)
    pr = Pair(wl)
    k, v = wl.prefill(0)
    pr.prefill(0, k, v)
    kn, vn, q = next(wl.steps(1))
    pr.append(kn, vn)
    qr = oracle.rotate_query(q, wl.cfg.dtype)
    want, _ = pr.orc.decode_attn(qr)
    got, _ = pr.attend(qr, q_dtype=ok.FP32, variant=1)
    assert np.abs(got - want).max() <= ATOL


COUNTER_BYTES = 256 * 1024   # the workspace's arrival counters (zeroed once)


def test_attention_workspace_reuse():
    """One workspace, its counter region zeroed once and its partials region
    full of garbage, serves calls with different split counts and kernels:
    no call depends on partials an earlier one left, and every call leaves
    the counters zero for the next."""
    wl = synth.workload(3, batch=3, ctx=None)
    wl.ctx_lens = [3000, 700, 129]
    pr = Pair(wl)
    for b in range(3):
        k, v = wl.prefill(b)
        pr.prefill(b, k, v)
    kn, vn, q = next(wl.steps(1))
    pr.append(kn, vn)
    want, _ = pr.orc.decode_attn(oracle.rotate_query(q, wl.cfg.dtype))
    _, nbytes = ok.decode_workspace_bytes(pr.geom, 3001, 64)
    ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device="cuda")
    ws[:COUNTER_BYTES] = 0
    for S, var in [(64, 2), (5, 2), (1, 1), (0, 2), (64, 1), (3, 2), (1, 2), (2, 2)]:
        got, _ = pr.attend(q, variant=var, splits=S, max_ctx=3001, ws=ws)
        assert np.abs(got - want).max() <= ATOL, (S, var)
        assert not ws[:COUNTER_BYTES].any().item(), (S, var)


def test_attention_workspace_shared_by_geometries():
    """A workspace zeroed once serves two different caches (batch 3 and
    batch 1, other head counts) in alternation."""
    wa = synth.workload(3, batch=3, ctx=None)
    wa.ctx_lens = [2100, 900, 300]
    wb = synth.workload(0, ctx=1500)
    pa, pb = Pair(wa), Pair(wb)
    for pr, wl in ((pa, wa), (pb, wb)):
        for b in range(wl.cfg.batch):
            k, v = wl.prefill(b)
            pr.prefill(b, k, v)
    qa = next(wa.steps(1))[2]
    qb = next(wb.steps(1))[2]
    want_a, _ = pa.orc.decode_attn(oracle.rotate_query(qa, wa.cfg.dtype))
    want_b, _ = pb.orc.decode_attn(oracle.rotate_query(qb, wb.cfg.dtype))
    na = ok.decode_workspace_bytes(pa.geom, 2200, 0)[1]
    nb = ok.decode_workspace_bytes(pb.geom, 1600, 0)[1]
    ws = torch.zeros(max(na, nb), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        got, _ = pa.attend(qa, max_ctx=2200, ws=ws)
        assert np.abs(got - want_a).max() <= ATOL
        got, _ = pb.attend(qb, max_ctx=1600, ws=ws)
        assert np.abs(got - want_b).max() <= ATOL
    assert not ws[:COUNTER_BYTES].any().item()


def test_abi_rejects_bad_arguments():
    g = ok.make_geom(1, 4, 1, 4, 4, head_dim=64)
    with pytest.raises(ok.OscarError) as e:
        ok.cache_layout(g)
    assert e.value.status == ok.EINVAL
    g = ok.make_geom(1, 6, 4, 4, 4)
    with pytest.raises(ok.OscarError):
        ok.cache_layout(g)
    wl = synth.workload(0, ctx=100)
    pr = Pair(wl)
    S, nbytes = ok.decode_workspace_bytes(pr.geom, 100, 0)
    small = torch.empty(nbytes // 2, dtype=torch.uint8, device="cuda")
    out = torch.empty(1, 4, 128, dtype=torch.float32, device="cuda")
    q = torch.zeros(1, 4, 128, dtype=torch.int16, device="cuda")
    with pytest.raises(ok.OscarError) as e:
        ok.decode_attn(pr.gpu, q, 0, out, None, small, 100, 0)
    assert e.value.status == ok.EWORKSPACE


# ---------------------------------------------------------------- HEAD scope
# One norm per (token, KV head) instead of one per token.

@pytest.mark.parametrize("hkv", [3, 8])
def test_head_scope_rotate_scale_key(hkv):
    wl = synth.workload(2, ctx=300)
    k, _ = wl.prefill(0, 150)
    k = np.ascontiguousarray(k[:, :hkv])
    khat = torch.empty(k.shape, dtype=torch.int16, device="cuda")
    norm = torch.empty(k.shape[0], hkv, dtype=torch.int16, device="cuda")
    ok.rotate_scale(dev_u16(k), wl.cfg.dtype, ok.ROT_KEY, norm_scope=ok.NORM_HEAD,
                    khat_out=khat, norm_out=norm)
    torch.cuda.synchronize()
    wk, wn = oracle.rotate_scale_key(k, wl.cfg.dtype, oracle.NORM_HEAD)
    assert_same_bits(host_u16(norm), wn, "norm")
    assert_same_bits(host_u16(khat), wk, "k_hat")


def test_head_scope_quant_pack():
    nb, hkv = 3, 8
    wl = synth.workload(2, ctx=32 * nb + 10)
    k, v = wl.prefill(0, 32 * nb)
    khat, knorm = oracle.rotate_scale_key(k, synth.BF16, oracle.NORM_HEAD)
    v16 = oracle.in_to_f16(v, synth.BF16)
    rec = torch.zeros(nb, hkv, 3072, dtype=torch.uint8, device="cuda")
    nrm = torch.zeros(nb, hkv, 32, dtype=torch.int16, device="cuda")
    ok.quant_pack(dev_u16(khat), dev_u16(knorm), dev_u16(v16), rec, nrm, norm_scope=ok.NORM_HEAD)
    torch.cuda.synchronize()
    wr, wn = oracle.quant_pack(khat, knorm, v16, norm_scope=oracle.NORM_HEAD)
    assert_same_bits(rec.cpu().numpy(), wr, "records")
    assert_same_bits(host_u16(nrm), wn, "norms")


@pytest.mark.parametrize("hkv", [8, 16])
def test_head_scope_cache_and_attention(hkv):
    """Bulk prefill, appends across block flushes and decode attention (both
    kernels) in HEAD scope; 16 KV heads take the 1024-thread prefill."""
    base = synth.workload(1, ctx=700)
    if hkv == 8:
        wl = base
    else:
        cfg = synth.Config("hkv16", 1, 32, 16, 700, synth.BF16, 0.3, (4, 4), 1)
        wl = synth.Workload(cfg, 57, [700], (base.outlier_idx * 2)[:16])
    pr = Pair(wl, max_ctx=760, norm_scope=ok.NORM_HEAD)
    k, v = wl.prefill(0, 640)
    pr.prefill(0, k, v)
    pr.compare_state()
    for kn, vn, q in wl.steps(45):
        pr.append(kn, vn)
    pr.compare_state()
    want, wlse = pr.orc.decode_attn(oracle.rotate_query(q, wl.cfg.dtype))
    for var in VARIANTS:
        got, glse = pr.attend(q, variant=var, splits=3)
        assert np.abs(got - want).max() <= ATOL, var
        assert np.abs(glse - wlse).max() <= 1e-3 * max(1.0, np.abs(wlse).max())


# ---------------------------------------------------------------- 128-token flush
# A full window is quantized as four blocks at once.

@pytest.mark.parametrize("n", [1, 128, 129, 300, 385])
def test_flush128_prefill_equals_appends(n):
    wl = synth.workload(1, ctx=n + 1)
    pr = Pair(wl, max_ctx=n + 160, flush_tokens=128)   # room for whole 128-token flushes
    k, v = wl.prefill(0, n)
    pr.prefill(0, k, v)
    pr.compare_state()


def test_flush128_appends_and_attention():
    """Prefill, then appends across a four-block flush; both attention kernels."""
    wl = synth.workload(1, ctx=400, batch=2)
    pr = Pair(wl, max_ctx=560, flush_tokens=128)
    for b, n in enumerate((300, 350)):
        k, v = wl.prefill(b, n)
        pr.prefill(b, k, v)
    pr.compare_state()
    for i, (kn, vn, q) in enumerate(wl.steps(140)):
        pr.append(kn, vn)
        if i in (83, 84, 139):
            pr.compare_state()
    want, _ = pr.orc.decode_attn(oracle.rotate_query(q, wl.cfg.dtype))
    for var in VARIANTS:
        got, _ = pr.attend(q, variant=var, splits=4)
        assert np.abs(got - want).max() <= ATOL, var


def test_flush128_capacity_drops_whole_flush():
    """A block table with room for the prefill's four blocks and no more: the
    next four-block flush sets the capacity flag and the append is dropped,
    as in the oracle."""
    wl = synth.workload(0, ctx=300)
    pr = Pair(wl, max_ctx=130 + 64, flush_tokens=128)   # 4 blocks of room
    k, v = wl.prefill(0, 256)
    pr.prefill(0, k, v)
    for kn, vn, _ in wl.steps(3):
        pr.append(kn, vn)
    pr.compare_state()
    assert int(pr.gpu.error_flag.cpu()[0]) == ok.FLAG_CAPACITY


def _scaled_bits(bits, dtype, factor):
    return synth.cast_bits(synth.bits_to_f32(bits, dtype) * np.float32(factor), dtype)


def _saturating_inputs(wl, huge_keys: bool, seed: int = 17):
    """Prefill tokens and 12 decode steps whose bf16 Values include entries
    beyond fp16's range (1e5, -2e5, +-3e38, +-inf) and NaN; with huge_keys,
    some Keys scaled so that their token norm exceeds 65504."""
    cfg = wl.cfg
    k, v = wl.prefill(0, 290)
    rng = np.random.default_rng(seed)
    odd = np.float32([1e5, -2e5, 7e4, 3e38, -3e38, np.inf, -np.inf, np.nan])
    vf = synth.bits_to_f32(v, cfg.dtype).copy()
    idx = rng.integers(0, vf.size, size=600)
    vf.ravel()[idx] = odd[rng.integers(0, odd.size, size=idx.size)]
    kf = synth.bits_to_f32(k, cfg.dtype).copy()
    if huge_keys:
        kf[[3, 100, 250, 280]] *= 5000.0
    steps = []
    for s_, (kn, vn, q) in enumerate(wl.steps(12)):
        if huge_keys and s_ % 5 == 0:
            kn = _scaled_bits(kn, cfg.dtype, 5000.0)
        vnf = synth.bits_to_f32(vn, cfg.dtype).copy()
        vnf.ravel()[rng.integers(0, vnf.size, size=40)] = odd[rng.integers(0, odd.size, size=40)]
        steps.append((kn, synth.to_bf16_bits(vnf), q))
    return synth.to_bf16_bits(kf), synth.to_bf16_bits(vf), steps


def test_values_and_norms_beyond_fp16_range_saturate():
    """bf16 Values beyond fp16's range and NaN, and Keys whose token norm
    exceeds 65504, through prefill and appends (with a flush): the cache is
    bit-exact with the oracle's saturating reading and attention stays
    finite.  (The scores of tokens with norm 65504 reach ~6e3 and their dot
    products cancel heavily; no fp32 attention matches an fp64 one to 2e-3
    on them, so their outputs are checked for finiteness only.)"""
    wl = synth.workload(2, ctx=330)
    pr = Pair(wl)
    k, v, steps = _saturating_inputs(wl, huge_keys=True)
    pr.prefill(0, k, v)
    for kn, vn, q in steps:
        pr.append(kn, vn)
    pr.compare_state()
    got, glse = pr.attend(q)
    assert np.isfinite(got).all() and np.isfinite(glse).all()


def test_saturated_values_attention():
    """Saturated Values (entries +-65504) with ordinary Keys: bit-exact cache,
    and every head within 2e-3 plus what fp32 rounding of Values this large
    allows (fp32_score_tol)."""
    wl = synth.workload(2, ctx=330)
    cfg = wl.cfg
    pr = Pair(wl)
    k, v, steps = _saturating_inputs(wl, huge_keys=False, seed=23)
    pr.prefill(0, k, v)
    for kn, vn, q in steps:
        pr.append(kn, vn)
    pr.compare_state()
    got, _ = pr.attend(q)
    want, wlse = pr.orc.decode_attn(oracle.rotate_query(q, cfg.dtype))
    for i in range(cfg.hq):
        tol = fp32_score_tol(float(wlse[0, i]), 2 * 65504.0)
        assert float(np.abs(got[0, i] - want[0, i]).max()) <= tol, i


def test_zero_key_tokens_through_prefill_and_append():
    """Zero Keys (norm 0: k_hat = 0, norm = 0) in a quantized block, in the
    window and as an appended token: bit-exact cache, every head within 2e-3."""
    wl = synth.workload(2, ctx=320)
    pr = Pair(wl)
    k, v = wl.prefill(0, 290)
    k = k.copy()
    k[[0, 5, 31, 200, 280]] = 0
    pr.prefill(0, k, v)
    for s, (kn, vn, q) in enumerate(wl.steps(6)):
        pr.append(np.zeros_like(kn) if s in (1, 4) else kn, vn)
    pr.compare_state()
    got, glse = pr.attend(q)
    want, wlse = pr.orc.decode_attn(oracle.rotate_query(q, wl.cfg.dtype))
    assert float(np.abs(got - want).max()) <= ATOL
    assert np.allclose(glse, wlse, rtol=1e-4, atol=1e-4)


@pytest.mark.parametrize("scope,flush,hkv,batch", [
    (0, 32, 16, 3), (1, 32, 16, 2), (0, 128, 5, 4), (1, 128, 3, 2), (0, 32, 1, 5)])
def test_append_workgroup_per_head(scope, flush, hkv, batch):
    """append_kv runs one workgroup per (sequence, KV head): every head count
    (1, odd, 16 = four heads per wave), both norm scopes and both flush sizes
    give the oracle's bytes over appends that cross flushes in ragged
    sequences, and the per-sequence arrival counters are zero after every
    call."""
    base = synth.workload(2, ctx=600)
    cfg = synth.Config("appendw", batch, 2 * hkv, hkv, None, synth.BF16, 0.4, (4, 8), 1)
    wl = synth.Workload(cfg, 61 + hkv, [300 + 57 * b for b in range(batch)],
                        (base.outlier_idx * 2)[:hkv])
    pr = Pair(wl, max_ctx=max(wl.ctx_lens) + 150, norm_scope=scope, flush_tokens=flush)
    for b in range(batch):
        k, v = wl.prefill(b)
        pr.prefill(b, k, v)
    for i, (kn, vn, q) in enumerate(wl.steps(140)):
        pr.append(kn, vn)
        if i % 35 == 34:
            pr.compare_state()
            assert not pr.gpu.append_sync.any().item()
    pr.compare_state()
    want, _ = pr.orc.decode_attn(oracle.rotate_query(q, wl.cfg.dtype))
    got, _ = pr.attend(q)
    assert np.abs(got - want).max() <= ATOL
