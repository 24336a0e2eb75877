"""Determinism and checkpoint/resume of the GPU path, through the C ABI.

Every reduction order is fixed, so the same inputs give the same bytes:
two caches built by the same prefill and appends are byte-identical, and two
decode calls on one cache give identical outputs (INT2 and bf16 baseline).
The cache is plain device arrays plus {n, Q}: copying every buffer to the host
and back into fresh allocations (a checkpoint) and then continuing the decode
gives the same bytes as never having stopped."""
import numpy as np
import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]

if gpu_available():
    import torch
    import int2_kv_cache_amd as ok
    from int2_kv_cache_amd import synth
    from _parity import dev_u16, shuffled_table

BUFS = ("pool", "pool_norm", "res_k", "res_v", "res_norm", "block_table", "seq_state",
        "error_flag")


def _state(c):
    torch.cuda.synchronize()
    return {name: getattr(c, name).cpu().numpy().copy() for name in BUFS}


def _same(a, b):
    for name in BUFS:
        assert np.array_equal(a[name], b[name]), name


def _setup(batch=2, ctx=900, steps=40):
    wl = synth.workload(2, ctx=ctx, batch=batch)
    mb = (ctx + steps + 64) // 32
    geom = ok.make_geom(batch, wl.cfg.hq, wl.cfg.hkv, mb, batch * mb)
    return wl, geom, shuffled_table(batch, mb, seed=5)


def _decode(c, q, dt, geom, max_ctx):
    S, nbytes = ok.decode_workspace_bytes(geom, max_ctx)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.empty(geom.batch, geom.num_q_heads, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(geom.batch, geom.num_q_heads, dtype=torch.float32, device="cuda")
    ok.decode_attn(c, dev_u16(q), dt, out, lse, ws, max_ctx)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def test_int2_path_is_deterministic():
    wl, geom, table = _setup()
    dt = wl.cfg.dtype
    caches = [ok.DeviceCache(geom, block_table=torch.from_numpy(table)) for _ in range(2)]
    for b in range(geom.batch):
        k, v = wl.prefill(b, 700 + 31 * b)
        for c in caches:
            ok.prefill_quantize(c, b, dev_u16(k), dev_u16(v), dt)
    q = None
    for kn, vn, q in wl.steps(40):
        for c in caches:
            ok.append_kv(c, dev_u16(kn), dev_u16(vn), dt)
    _same(_state(caches[0]), _state(caches[1]))
    o1, l1 = _decode(caches[0], q, dt, geom, 1000)
    o2, l2 = _decode(caches[0], q, dt, geom, 1000)
    o3, l3 = _decode(caches[1], q, dt, geom, 1000)
    assert np.array_equal(o1.view(np.uint32), o2.view(np.uint32))
    assert np.array_equal(o1.view(np.uint32), o3.view(np.uint32))
    assert np.array_equal(l1.view(np.uint32), l2.view(np.uint32))


def test_bf16_baseline_is_deterministic():
    wl = synth.workload(2, ctx=3000, batch=1)
    k, v = wl.prefill(0, 2999)
    geom = ok.make_geom(1, wl.cfg.hq, wl.cfg.hkv, 94, 94)
    c = ok.DenseCache(geom)
    ok.dense_write_kv(c, 0, 0, dev_u16(k), dev_u16(v))
    c.ctx_lens.fill_(2999)
    q = dev_u16(next(wl.steps(1))[2])
    S, nbytes = ok.dense_workspace_bytes(geom, 2999)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        out = torch.empty(1, wl.cfg.hq, 128, dtype=torch.float32, device="cuda")
        ok.dense_decode_attn(c, q, out, None, ws, 2999)
        torch.cuda.synchronize()
        outs.append(out.cpu().numpy())
    assert np.array_equal(outs[0].view(np.uint32), outs[1].view(np.uint32))


def test_checkpoint_and_resume():
    """Dump every cache buffer to the host after prefill and 10 appends, load
    the dump into a fresh cache, continue both for 40 appends (crossing
    flushes) and a decode step: identical bytes."""
    wl, geom, table = _setup()
    dt = wl.cfg.dtype
    a = ok.DeviceCache(geom, block_table=torch.from_numpy(table))
    for b in range(geom.batch):
        k, v = wl.prefill(b, 650 + 45 * b)
        ok.prefill_quantize(a, b, dev_u16(k), dev_u16(v), dt)
    steps = list(wl.steps(50))
    for kn, vn, _ in steps[:10]:
        ok.append_kv(a, dev_u16(kn), dev_u16(vn), dt)
    dump = _state(a)
    r = ok.DeviceCache(geom, block_table=torch.from_numpy(dump["block_table"]))
    for name in BUFS:
        getattr(r, name).copy_(torch.from_numpy(dump[name]))
    _same(dump, _state(r))
    for kn, vn, _ in steps[10:]:
        for c in (a, r):
            ok.append_kv(c, dev_u16(kn), dev_u16(vn), dt)
    _same(_state(a), _state(r))
    q = steps[-1][2]
    oa, la = _decode(a, q, dt, geom, 1000)
    orr, lr = _decode(r, q, dt, geom, 1000)
    assert np.array_equal(oa.view(np.uint32), orr.view(np.uint32))
    assert np.array_equal(la.view(np.uint32), lr.view(np.uint32))
