"""oscar_decode_attn_noalloc -- decode attention with the library's own
static workspace, for callers that cannot allocate -- through the C ABI,
against oscar_decode_attn with a caller workspace: two calls in a row, the
second with a smaller input, must give identical outputs (the same kernels,
split count and merge order), within 2e-3 of the oracle; a call needing more
than the static workspace is refused."""
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


def _noalloc(pr, q, max_ctx, splits=0, variant=0):
    cfg = pr.wl.cfg
    out = torch.full((cfg.batch, cfg.hq, 128), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((cfg.batch, cfg.hq), float("nan"), dtype=torch.float32, device="cuda")
    ok.decode_attn_noalloc(pr.gpu, dev_u16(q), pr.dtype, out, lse, max_ctx, splits, variant)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _case(wl, max_ctx, variant=0):
    pr = Pair(wl)
    for b in range(wl.cfg.batch):
        k, v = wl.prefill(b)
        pr.prefill(b, k, v)
    kn, vn, q = next(wl.steps(1))
    pr.append(kn, vn)
    return pr, q


@pytest.mark.parametrize("variant", [ok.ATTN_AUTO, ok.ATTN_VALU] if gpu_available() else [0])
def test_noalloc_equals_workspace_entry_point_twice(variant):
    """First a larger call (2 ragged sequences, Qwen3-8B shape, 5000 and
    1700 tokens), then a smaller one (1 sequence, 4/1 heads, 700 tokens):
    each equals
    oscar_decode_attn bit for bit and the oracle within 2e-3."""
    b48 = synth.workload(3)
    cfg = synth.Config("noalloc-big", 2, b48.cfg.hq, b48.cfg.hkv, None, b48.cfg.dtype,
                       b48.cfg.sigma, b48.cfg.outliers, 1)
    big = synth.Workload(cfg, 404, [5000, 1700], b48.outlier_idx)
    small = synth.workload(0, ctx=700)
    for wl, mctx in ((big, 5100), (small, 760)):
        pr, q = _case(wl, mctx)
        got, glse = _noalloc(pr, q, mctx, variant=variant)
        ref, rlse = pr.attend(q, max_ctx=mctx, variant=variant)
        assert np.array_equal(got, ref) and np.array_equal(glse, rlse)
        want, _ = pr.orc.decode_attn(oracle.rotate_query(q, wl.cfg.dtype))
        assert np.abs(got - want).max() <= ATOL


def test_noalloc_refuses_more_than_its_workspace():
    """48 sequences at 32K with 1024 splits need ~100 MB of partials: the
    call is refused with OSCAR_EWORKSPACE before anything is enqueued."""
    geom = ok.make_geom(48, 32, 8, 1100, 48 * 1100)
    need = ok.decode_workspace_bytes(geom, 35000, 1024)[1]
    assert need > ok.STATIC_WORKSPACE_BYTES
    cache = ok.DeviceCache(geom)
    q = torch.zeros(48, 32, 128, dtype=torch.int16, device="cuda")
    out = torch.zeros(48, 32, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(ok.OscarError) as e:
        ok.decode_attn_noalloc(cache, q, ok.BF16, out, None, 35000, 1024)
    assert e.value.status == ok.EWORKSPACE
    torch.cuda.synchronize()
    assert not out.any().item()
