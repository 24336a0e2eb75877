"""Rotary position embedding on the GPU path, through the C ABI.

With a RoPE table in the cache, prefill and append rotate each Key by its
position before the online FHT, and decode attention rotates a raw query by
the position of the step's own token (n - 1) before its FHT.  The cache bytes
equal the oracle's bit for bit; attention equals the oracle's attention on
the oracle's RoPE'd + rotated query; a pre-rotated fp32 query (the caller
applied RoPE and the FHT) gives the same outputs; a position past the table
is refused (prefill) or flagged and dropped (append).

The offline absorption of the Value rotation into W_v and W_o gives the
oracle's weights bit for bit, and a decode step whose Values come from the
absorbed W_v, followed by the absorbed W_o, gives the layer output of the
original weights."""
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
    from _parity import ATOL, Pair, dev_u16


def _roped_pair(wl, tab, scope=0, flush=32, extra=200):
    pr = Pair(wl, max_ctx=max(wl.ctx_lens) + extra, norm_scope=scope, flush_tokens=flush,
              rope_table=tab)
    for b in range(wl.cfg.batch):
        k, v = wl.prefill(b)
        pr.prefill(b, k, v)
    return pr


def _oracle_attn(pr, q, tab):
    """The oracle's attention with each sequence's query RoPE'd at n - 1."""
    dt = pr.wl.cfg.dtype
    qr = np.stack([oracle.rotate_query_pos(q[b:b + 1], dt, tab[pr.orc.n(b) - 1])[0]
                   for b in range(pr.wl.cfg.batch)])
    return pr.orc.decode_attn(qr), qr


@pytest.mark.parametrize("wid,scope,flush", [(0, 0, 32), (2, 0, 32), (2, 1, 32), (1, 0, 128)])
def test_roped_cache_and_attention(wid, scope, flush):
    """Ragged batch, appends across flushes: bit-exact cache, attention within
    the fp32 tolerance, every query head."""
    base = synth.workload(wid, ctx=700)
    cfg = synth.Config("rope", 3, base.cfg.hq, base.cfg.hkv, None, base.cfg.dtype, 0.4,
                       (4, 8), 1)
    wl = synth.Workload(cfg, 70 + wid, [650, 333, 129], base.outlier_idx)
    tab = synth.rope_table(1024)
    pr = _roped_pair(wl, tab, scope, flush)
    pr.compare_state()
    q = None
    for i, (kn, vn, q) in enumerate(wl.steps(90)):
        pr.append(kn, vn)
        if i % 45 == 44:
            pr.compare_state()
    (want, wlse), qr = _oracle_attn(pr, q, tab)
    got, glse = pr.attend(q)
    assert float(np.abs(got - want).max()) <= ATOL
    assert np.allclose(glse, wlse, rtol=1e-4, atol=1e-4)
    # the caller may apply RoPE + FHT itself and hand over fp32 q'
    got2, _ = pr.attend(qr, q_dtype=ok.FP32)
    assert float(np.abs(got2 - want).max()) <= ATOL


def test_rope_changes_the_cache():
    """The same inputs with and without a table give different Key bytes
    (beyond position 0) and the same Value bytes."""
    wl = synth.workload(2, ctx=300, batch=1)
    tab = synth.rope_table(512)
    a = _roped_pair(wl, tab)
    p = Pair(wl, max_ctx=500)
    k, v = wl.prefill(0)
    p.prefill(0, k, v)
    torch.cuda.synchronize()
    assert not torch.equal(a.gpu.pool, p.gpu.pool)
    assert torch.equal(a.gpu.res_v, p.gpu.res_v)


def test_rope_position_limit():
    """rope_max_pos bounds the sequence: a prefill longer than the table is
    refused, an append at position rope_max_pos sets OSCAR_FLAG_POSITION and
    leaves the sequence unchanged (as the oracle does)."""
    wl = synth.workload(2, ctx=200, batch=1)
    tab = synth.rope_table(160)
    pr = Pair(wl, max_ctx=300, rope_table=tab)
    k, v = wl.prefill(0, 200)
    with pytest.raises(RuntimeError):
        ok.prefill_quantize(pr.gpu, 0, dev_u16(k), dev_u16(v), wl.cfg.dtype)
    torch.cuda.synchronize()
    assert int(pr.gpu.seq_state[0, 0].item()) == 0
    pr.prefill(0, k[:158], v[:158])
    steps = list(wl.steps(3))
    for kn, vn, _ in steps:
        pr.append(kn, vn)
    pr.compare_state()
    assert pr.orc.n(0) == 160 and int(pr.orc.error_flag[0]) == ok.FLAG_POSITION
    q = steps[-1][2]
    (want, _), _ = _oracle_attn(pr, q, tab)
    got, _ = pr.attend(q)
    assert float(np.abs(got - want).max()) <= ATOL


# ---------------------------------------------------------------- absorption
@pytest.mark.parametrize("rows,cols,axis", [
    (1024, 4096, 0),     # W_v of 8 KV heads, d_model 4096, nn.Linear layout
    (4096, 4096, 1),     # W_o of 32 query heads
    (256, 37, 0), (3, 384, 1), (1, 1024, 1), (128, 1, 0)])
def test_absorb_value_rotation_bit_exact(rows, cols, axis):
    rng = np.random.default_rng(rows * 7 + cols + axis)
    w = (rng.standard_normal((rows, cols)) *
         10.0 ** rng.uniform(-3, 3, size=(rows, 1))).astype(np.float32)
    want = oracle.absorb_value_rotation(w, axis)
    wt = torch.from_numpy(w).cuda()
    got = ok.absorb_value_rotation(wt, axis)
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy().view(np.uint32), want.view(np.uint32))
    # in place gives the same bytes; a second application gives w back
    ok.absorb_value_rotation(wt, axis, out=wt)
    ok.absorb_value_rotation(wt, axis, out=wt)
    torch.cuda.synchronize()
    back = wt.cpu().numpy().astype(np.float64)
    assert np.abs(back - w).max() <= 1e-6 * np.abs(w).max()


def test_absorbed_weights_through_the_cache():
    """A layer whose Values come from W_v' = H W_v and whose output goes
    through W_o' = W_o H: the GPU cache holds V' (all 100 tokens in the fp16
    window), GPU attention returns H o per query head, and W_o' maps it to
    the original layer's output (fp64 attention with W_v, W_o), up to the
    fp16 storage of k_hat and V'."""
    wl = synth.workload(2, ctx=100, batch=1)
    cfg = wl.cfg
    rng = np.random.default_rng(12)
    dm = 256
    X = rng.standard_normal((100, dm))
    Wv = (rng.standard_normal((cfg.hkv * 128, dm)) / np.sqrt(dm)).astype(np.float32)
    Wo = (rng.standard_normal((dm, cfg.hq * 128)) / np.sqrt(cfg.hq * 128)).astype(np.float32)
    Wv2 = ok.absorb_value_rotation(torch.from_numpy(Wv).cuda(), 0).cpu().numpy()
    Wo2 = ok.absorb_value_rotation(torch.from_numpy(Wo).cuda(), 1).cpu().numpy()
    V2 = (X @ Wv2.astype(np.float64).T).reshape(100, cfg.hkv, 128)
    k, _ = wl.prefill(0, 99)
    kn, _, q = next(wl.steps(1))
    pr = Pair(wl, max_ctx=200)
    vbits = synth.cast_bits(V2.astype(np.float32), cfg.dtype)
    pr.prefill(0, k, vbits[:99])
    pr.append(kn, vbits[99:100])
    pr.compare_state()
    got, _ = pr.attend(q)                                  # [1][Hq][128], rotated basis
    y = Wo2.astype(np.float64) @ got[0].reshape(-1).astype(np.float64)
    # the original layer in fp64: unrotated Keys and query, V = X W_v^T, W_o
    K = synth.bits_to_f32(np.concatenate([k, kn]), cfg.dtype).astype(np.float64)
    V = (X @ Wv.astype(np.float64).T).reshape(100, cfg.hkv, 128)
    qf = synth.bits_to_f32(q, cfg.dtype)[0].astype(np.float64)
    g = cfg.hq // cfg.hkv
    o = np.zeros((cfg.hq, 128))
    for i in range(cfg.hq):
        s = K[:, i // g, :] @ qf[i] / np.sqrt(128.0)
        p = np.exp(s - s.max())
        o[i] = (p / p.sum()) @ V[:, i // g, :]
    ref = Wo.astype(np.float64) @ o.reshape(-1)
    assert np.abs(y - ref).max() <= 1e-2 * np.abs(ref).max()
