"""Pins of the oracle's unquantized decode attention (the BF16 baseline).

Against torch's scaled_dot_product_attention in fp64 (a library routine) on
the workloads' bf16 Keys and Values, the one-token and identical-key closed
forms, the contiguous GQA mapping, the empty sequence, and agreement with the
INT2 path's own attention where that path stores nothing in INT2 (n <= 128:
every token sits in the fp16 window, so its Keys are exactly norm * k_hat).
"""
import numpy as np
import pytest
import torch

from int2_kv_cache_amd import synth


def _sdpa64(q, K, V):
    """q [Hq][128], K, V [Hq][n][128] (already expanded per query head)."""
    out = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None, None, :].double(),
        torch.from_numpy(K)[:, None].double(), torch.from_numpy(V)[:, None].double())
    return out[:, 0, 0].numpy()


def _bf16_case(seed, n, hq, hkv):
    wl = synth.workload(2, ctx=max(n, 1) + 1)
    rng = np.random.default_rng(seed)
    if n:
        k, v = wl.prefill(0, n)
        k = synth.to_bf16_bits(synth.bits_to_f32(k, wl.cfg.dtype)[:, :hkv])
        v = synth.to_bf16_bits(synth.bits_to_f32(v, wl.cfg.dtype)[:, :hkv])
    else:
        k = v = np.zeros((0, hkv, 128), np.uint16)
    q = synth.to_bf16_bits(rng.standard_normal((hq, 128)))
    return q, k, v


@pytest.mark.parametrize("n,hq,hkv", [(1, 4, 1), (31, 4, 1), (33, 8, 2), (200, 8, 8), (1000, 32, 8)])
def test_dense_equals_library_sdpa(orc, n, hq, hkv):
    q, k, v = _bf16_case(11 + n, n, hq, hkv)
    qf, kf, vf = orc.bf16_bits_to_f32(q), orc.bf16_bits_to_f32(k), orc.bf16_bits_to_f32(v)
    out, lse = orc.dense_attn(qf, kf, vf)
    g = hq // hkv
    K = np.stack([kf[:, i // g].astype(np.float64) for i in range(hq)])
    V = np.stack([vf[:, i // g].astype(np.float64) for i in range(hq)])
    ref = _sdpa64(qf.astype(np.float64), K, V)
    assert np.abs(out - ref).max() <= 1e-6 * max(1.0, np.abs(ref).max())
    s = np.einsum("hc,htc->ht", qf.astype(np.float64), K) / np.sqrt(128.0)
    assert np.allclose(lse, np.log(np.exp(s - s.max(1, keepdims=True)).sum(1)) + s.max(1), rtol=1e-6)


def test_dense_one_token_returns_its_value(orc):
    q, k, v = _bf16_case(3, 1, 8, 2)
    vf = orc.bf16_bits_to_f32(v)
    out, lse = orc.dense_attn(orc.bf16_bits_to_f32(q), orc.bf16_bits_to_f32(k), vf)
    assert np.array_equal(out, np.repeat(vf[0], 4, axis=0))
    s = (orc.bf16_bits_to_f32(q).astype(np.float64).reshape(2, 4, 128)
         * orc.bf16_bits_to_f32(k)[0].astype(np.float64)[:, None, :]).sum(-1).reshape(8) / np.sqrt(128)
    assert np.allclose(lse, s, rtol=1e-6)


def test_dense_identical_keys_give_mean_of_values(orc):
    rng = np.random.default_rng(7)
    k1 = synth.to_bf16_bits(rng.standard_normal((1, 1, 128)))
    k = np.repeat(k1, 77, axis=0)
    v = synth.to_bf16_bits(rng.standard_normal((77, 1, 128)))
    q = synth.to_bf16_bits(3.0 * rng.standard_normal((4, 128)))
    vf = orc.bf16_bits_to_f32(v).astype(np.float64)
    out, _ = orc.dense_attn(orc.bf16_bits_to_f32(q), orc.bf16_bits_to_f32(k), orc.bf16_bits_to_f32(v))
    assert np.abs(out - vf[:, 0].mean(0)[None]).max() < 1e-6


def test_dense_gqa_mapping_contiguous(orc):
    rng = np.random.default_rng(8)
    k = synth.to_bf16_bits(rng.standard_normal((50, 2, 128)))
    v = np.zeros((50, 2, 128), np.float32)
    v[:, 0] = -3.0
    v[:, 1] = 7.0
    out, _ = orc.dense_attn(orc.bf16_bits_to_f32(synth.to_bf16_bits(rng.standard_normal((4, 128)))),
                            orc.bf16_bits_to_f32(k), v)
    assert np.all(out[:2] == -3.0) and np.all(out[2:] == 7.0)


def test_dense_empty_sequence(orc):
    out, lse = orc.dense_attn(np.ones((4, 128), np.float32), np.zeros((0, 1, 128), np.float32),
                              np.zeros((0, 1, 128), np.float32))
    assert not out.any() and np.all(np.isneginf(lse))


@pytest.mark.parametrize("n", [1, 57, 128])
def test_dense_equals_int2_path_on_the_fp16_window(orc, n):
    """n <= 128: the INT2 path's attention over its window (Keys norm * k_hat,
    Values fp16) equals the unquantized attention over those same rows."""
    wl = synth.workload(1, ctx=n)
    hq, hkv, dt = wl.cfg.hq, wl.cfg.hkv, wl.cfg.dtype
    c = orc.OracleCache(1, hq, hkv, 8)
    k, v = wl.prefill(0)
    if n > 1:
        c.prefill(0, k, v, dt)
    kn, vn, q = next(wl.steps(1))
    c.append(kn, vn, dt)
    assert (c.n(0), c.q(0)) == (n, 0)
    qr = orc.rotate_query(q, dt)
    out, lse = c.decode_attn(qr)
    K = np.stack([np.stack([c.key_row(0, h, t) for h in range(hkv)]) for t in range(n)])
    V = np.stack([np.stack([c.value_row(0, h, t) for h in range(hkv)]) for t in range(n)])
    assert np.array_equal(K.astype(np.float32).astype(np.float64), K)  # exact in fp32
    ref, rlse = orc.dense_attn(qr[0], K.astype(np.float32), V.astype(np.float32))
    assert np.abs(out[0] - ref).max() < 1e-6
    assert np.allclose(lse[0], rlse, rtol=1e-6)
