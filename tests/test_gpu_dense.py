"""GPU parity of the BF16 baseline (unquantized paged bf16 decode attention)
against the oracle's fp64 attention, through the C ABI: several tiles and
ragged tails, every GQA group size, forced split counts, shuffled block
tables, chunked writes, empty sequences, the error flags, and the
benchmark's full sizes (128K batch 1 and a ragged 8K..32K batch)."""
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
    from _parity import ATOL, dev_u16


def _bf16(bits, dtype):
    return synth.to_bf16_bits(synth.bits_to_f32(bits, dtype))


def _run(wl, ctxs, grp=None, splits=0, max_ctx=None, chunks=1, seed=0, heads=None):
    """Write each sequence's first ctxs[b] tokens of workload wl into the bf16
    pool (shuffled physical blocks), attend with one bf16 query per head and
    compare every (or the listed) query heads with the oracle."""
    cfg = wl.cfg
    B, hkv = len(ctxs), cfg.hkv
    hq = cfg.hq if grp is None else grp * hkv
    mb = max(1, (max(ctxs) + 31) // 32)
    P = B * mb + 3
    rng = np.random.default_rng(seed)
    table = rng.permutation(P)[:B * mb].reshape(B, mb).astype(np.int32)
    geom = ok.make_geom(B, hq, hkv, mb, P)
    cache = ok.DenseCache(geom, block_table=torch.from_numpy(table))
    kv = []
    for b, n in enumerate(ctxs):
        if n == 0:
            kv.append((np.zeros((0, hkv, 128), np.uint16),) * 2)
            continue
        k, v = wl.prefill(b % wl.cfg.batch, n)
        k, v = _bf16(k, cfg.dtype), _bf16(v, cfg.dtype)
        kv.append((k, v))
        edges = np.linspace(0, n, chunks + 1).astype(int)
        for a, e in zip(edges[:-1], edges[1:]):
            if e > a:
                ok.dense_write_kv(cache, b, int(a), dev_u16(k[a:e]), dev_u16(v[a:e]))
    cache.ctx_lens.copy_(torch.tensor(ctxs, dtype=torch.int32))
    q = synth.to_bf16_bits(rng.standard_normal((B, hq, 128)))
    mc = max(ctxs) if max_ctx is None else max_ctx
    s, nbytes = ok.dense_workspace_bytes(geom, mc, splits)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((B, hq, 128), float("nan"), device="cuda")
    lse = torch.full((B, hq), float("nan"), device="cuda")
    ok.dense_decode_attn(cache, dev_u16(q), out, lse, ws, mc, splits)
    torch.cuda.synchronize()
    assert int(cache.error_flag.item()) == 0
    got, glse = out.cpu().numpy(), lse.cpu().numpy()
    worst = 0.0
    for b in range(B):
        k, v = kv[b]
        want, wlse = oracle.dense_attn(oracle.bf16_bits_to_f32(q[b]), oracle.bf16_bits_to_f32(k),
                                       oracle.bf16_bits_to_f32(v))
        hs = range(hq) if heads is None else heads
        for i in hs:
            err = float(np.abs(got[b, i] - want[i]).max())
            assert err <= ATOL, (b, i, ctxs[b], err)
            worst = max(worst, err)
            if ctxs[b] == 0:
                assert np.isneginf(glse[b, i])
            else:
                assert abs(float(glse[b, i]) - float(wlse[i])) <= 1e-3 * max(1.0, abs(float(wlse[i])))
    return worst, s


@pytest.mark.parametrize("grp", [1, 2, 4, 8])
def test_dense_group_sizes_ragged(grp):
    wl = synth.workload(2, ctx=3000, batch=3)
    _run(wl, [1, 33, 2049], grp=grp, seed=grp)


@pytest.mark.parametrize("ctx", [1, 31, 32, 33, 64, 95, 1000, 4097])
def test_dense_tails(ctx):
    wl = synth.workload(1, ctx=ctx + 1, batch=1)
    _run(wl, [ctx], seed=ctx)


@pytest.mark.parametrize("splits", [1, 3, 7, 64])
def test_dense_forced_splits(splits):
    """More splits than blocks leaves empty splits (m = -inf partials)."""
    wl = synth.workload(2, ctx=1500, batch=2)
    _run(wl, [1500, 77], splits=splits, seed=splits)


def test_dense_empty_sequences_and_chunked_writes():
    wl = synth.workload(0, ctx=700, batch=3)
    _run(wl, [0, 700, 0], chunks=5, seed=4)


def test_dense_multimodal_norm_mix():
    """x30 tokens and x5 / x0.3 segments: very peaked softmax rows."""
    wl = synth.workload(4, ctx=12000, batch=1)
    _run(wl, [12000], seed=9)


def test_dense_flags():
    geom = ok.make_geom(1, 4, 1, 2, 2)
    table = torch.tensor([[0, 5]], dtype=torch.int32)  # block id 5 is outside the pool
    cache = ok.DenseCache(geom, block_table=table)
    k = dev_u16(np.zeros((64, 1, 128), np.uint16))
    ok.dense_write_kv(cache, 0, 0, k, k)
    torch.cuda.synchronize()
    assert int(cache.error_flag.item()) == ok.FLAG_BADSTATE
    with pytest.raises(ok.OscarError):
        ok.dense_write_kv(cache, 0, 60, k, k)  # past 32 * max_blocks
    cache.error_flag.zero_()
    cache.ctx_lens.fill_(65)  # above the table's capacity: attends to nothing
    s, nbytes = ok.dense_workspace_bytes(geom, 64)
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    out = torch.full((1, 4, 128), float("nan"), device="cuda")
    ok.dense_decode_attn(cache, dev_u16(np.zeros((1, 4, 128), np.uint16)), out, None, ws, 64)
    torch.cuda.synchronize()
    assert int(cache.error_flag.item()) == ok.FLAG_BADSTATE
    assert not out.isnan().any() and not out.any()


def test_dense_qwen3_8b_128k_bench_configuration():
    """Batch 1, 32 / 8 heads, 131072 tokens, the bench's split count."""
    wl = synth.workload(2)
    worst, s = _run(wl, [131072], max_ctx=131072 + 105 + 64, seed=1)
    assert s > 1


def test_dense_ragged_batch_8k_32k():
    wl = synth.workload(3, batch=6)
    _run(wl, wl.ctx_lens[:6], seed=2, heads=[0, 9, 18, 31])


def test_dense_ragged_batch_48_full():
    """The whole 48-sequence batch (8K..32K) in one launch, in the split count
    the bench uses; sampled (sequence, head) outputs against the oracle."""
    wl = synth.workload(3)
    assert wl.cfg.batch == 48
    ctxs = [n - 1 for n in wl.ctx_lens]
    _run(wl, ctxs, seed=3, heads=[7])
