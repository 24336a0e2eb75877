"""GPU checks of the hardware reciprocal-square-root scaling variant
(OSCAR_SCALE_HW_RSQ / OSCAR_ROT_KEY_HW_RSQ), through the C ABI.

The oracle computes the scaling factor as 1/sqrt(ss) in IEEE fp32; the
hardware instruction is accurate to about one ulp, so the variant is held to:
  - norms bit-exact (the stored norm is still the correctly rounded root);
  - k_hat within one fp16 step of the oracle's;
  - stage-wise bit-exactness after the scaling: the cache that append and
    prefill build equals, byte for byte, what the oracle's stateless
    quantizer and ring bookkeeping make from the GPU's own variant k_hat
    (the quantizer and the state machine do not depend on how r was formed);
  - decode attention within the 2e-3 tolerance of the IEEE oracle."""
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
    from _parity import ATOL, Pair, assert_same_bits, dev_u16, host_u16


def _gpu_khat_hw(k, dt, norm_scope=0):
    khat = torch.empty(k.shape, dtype=torch.int16, device="cuda")
    nshape = (k.shape[0],) if norm_scope == ok.NORM_TOKEN else (k.shape[0], k.shape[1])
    norm = torch.empty(nshape, dtype=torch.int16, device="cuda")
    ok.rotate_scale(dev_u16(k), dt, ok.ROT_KEY_HW_RSQ, norm_scope, khat_out=khat, norm_out=norm)
    torch.cuda.synchronize()
    return host_u16(khat), host_u16(norm)


@pytest.mark.parametrize("cfg,norm_scope", [(0, 0), (2, 0), (2, 1), (4, 0)])
def test_hw_rsq_khat_within_one_fp16_step(cfg, norm_scope):
    wl = synth.workload(cfg, ctx=600)
    k, _ = wl.prefill(0, 512)
    dt = wl.cfg.dtype
    gk, gn = _gpu_khat_hw(k, dt, norm_scope)
    wk, wn = oracle.rotate_scale_key(k, dt, norm_scope)
    assert_same_bits(gn, wn, "norm")
    d = np.abs(gk.view(np.int16).astype(np.int32) - wk.view(np.int16).astype(np.int32))
    assert d.max() <= 1, d.max()


@pytest.mark.parametrize("n_prefill,n_append", [(1000, 0), (700, 45), (129, 40)])
def test_hw_rsq_cache_stagewise_and_attention(n_prefill, n_append):
    wl = synth.workload(2, ctx=n_prefill + n_append + 1, batch=1)
    dt = wl.cfg.dtype
    pr = Pair(wl, max_ctx=n_prefill + n_append + 8)
    hw_geom = ok.make_geom(1, wl.cfg.hq, wl.cfg.hkv, pr.max_blocks, pr.geom.num_physical_blocks,
                           key_scale=ok.SCALE_HW_RSQ)
    gpu = ok.DeviceCache(hw_geom, block_table=torch.from_numpy(pr.table))
    k, v = wl.prefill(0, n_prefill)
    pr.orc.prefill(0, k, v, dt)
    ok.prefill_quantize(gpu, 0, dev_u16(k), dev_u16(v), dt)
    ks, vs = [k], [v]
    q = None
    for kn, vn, q in wl.steps(n_append):
        pr.orc.append(kn, vn, dt)
        ok.append_kv(gpu, dev_u16(kn), dev_u16(vn), dt)
        ks.append(kn)
        vs.append(vn)
    torch.cuda.synchronize()
    K, V = np.concatenate(ks), np.concatenate(vs)
    n, Q = pr.orc.n(0), pr.orc.q(0)
    assert np.array_equal(gpu.seq_state.cpu().numpy()[0], [n, Q])
    assert int(gpu.error_flag.item()) == 0
    khat, knorm = _gpu_khat_hw(K, dt)
    v16 = oracle.in_to_f16(V, dt)
    pool, pnorm = gpu.pool.cpu().numpy(), host_u16(gpu.pool_norm)
    if Q:
        rec, nrm = oracle.quant_pack(khat[:Q], knorm[:Q], v16[:Q])
        for j in range(Q // 32):
            p = pr.table[0, j]
            assert_same_bits(pool[p], rec[j], "block %d record" % j)
            assert_same_bits(pnorm[p], nrm[j], "block %d norms" % j)
    slots = np.array([t % 128 for t in range(Q, n)])
    rk, rv, rn = host_u16(gpu.res_k)[0], host_u16(gpu.res_v)[0], host_u16(gpu.res_norm)[0]
    assert_same_bits(rk[:, slots, :], khat[Q:n].transpose(1, 0, 2), "ring k_hat")
    assert_same_bits(rv[:, :, slots], v16[Q:n].transpose(1, 2, 0), "ring v")
    assert_same_bits(rn[slots], knorm[Q:n], "ring norms")
    # attention over the variant cache vs the IEEE oracle
    if q is None:
        q = next(wl.steps(1))[2]
    S, nbytes = ok.decode_workspace_bytes(hw_geom, n + 1)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(1, wl.cfg.hq, 128, dtype=torch.float32, device="cuda")
    ok.decode_attn(gpu, dev_u16(q), dt, out, None, ws, n + 1)
    torch.cuda.synchronize()
    want, _ = pr.orc.decode_attn(oracle.rotate_query(q, dt))
    err = float(np.abs(out.cpu().numpy() - want).max())
    assert err <= ATOL, err
