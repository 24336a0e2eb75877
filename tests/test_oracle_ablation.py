"""The Key-path ablation (oracle/ablation.py): its reconstructions agree with
the oracle cache, and per-token scaling does what it is for -- it bounds every
token's relative error, which the shared per-channel ranges of unscaled Keys
do not (sink tokens at 0.05x the norm)."""
import numpy as np

from int2_kv_cache_amd import synth


def test_oscar_reconstruction_matches_oracle_cache(orc):
    from oracle import ablation
    wl = synth.workload(2, ctx=300)
    k, v = wl.prefill(0, 256)
    ref, rec = ablation.reconstruct(k, wl.cfg.dtype, "oscar")
    c = orc.OracleCache(1, wl.cfg.hq, wl.cfg.hkv, 16)
    c.prefill(0, k, v, wl.cfg.dtype)
    for t in (0, 5, 77, 127):                 # quantized tokens (Q = 128)
        for h in (0, 3, 7):
            assert np.allclose(c.key_row(0, h, t), rec[t, h], rtol=0, atol=1e-12)


def test_scaling_bounds_every_tokens_relative_error(orc):
    from oracle import ablation
    r = ablation.run(synth.workload(0), 1024)
    for var in ablation.VARIANTS:
        assert all(np.isfinite(list(r[var].values())))
    # sinks (x0.05) and log-normal norms: unscaled tails, scaled tails bounded
    assert r["kivi"]["rel_p99"] > 1.0 and r["rotation"]["rel_p99"] > 1.0
    assert r["scaling"]["rel_p99"] < 0.6 and r["oscar"]["rel_p99"] < 0.6
    assert r["oscar"]["rel_mean"] < r["kivi"]["rel_mean"]


def test_scaling_without_rotation_inflates_blocks_with_flat_sinks(orc):
    """The Scaling-Induced Outlier Artifact (popular-science article, 二; reading
    notes, §II Step One): with flat low-norm sinks, per-token scaling alone
    stretches the ranges of the sinks' block, and rotating first removes it.
    With outlier-shaped sinks there is nothing to remove."""
    from oracle import ablation
    plain = synth.workload(2, ctx=2049)
    flat = synth.workload(2, ctx=2049)
    flat.flat_sinks = True
    rp, rf = ablation.run(plain, 2048), ablation.run(flat, 2048)
    sb = "sink_block_rel_mean"
    assert rf["scaling"][sb] > 1.08 * rf["oscar"][sb]
    assert rp["scaling"][sb] < 1.04 * rp["oscar"][sb]
    assert abs(rf["oscar"][sb] - rp["oscar"][sb]) < 0.02 * rp["oscar"][sb]
    # only the sinks' block moves: the whole-sequence means stay put
    assert abs(rf["scaling"]["rel_mean"] - rp["scaling"]["rel_mean"]) < 0.01


def test_flat_sinks_change_only_the_sink_tokens():
    """The generator option redraws the first four tokens only (isotropic, at
    the same norm as the outlier-shaped draw) and leaves every later token and
    the default stream untouched."""
    a = synth.workload(2, ctx=300)
    b = synth.workload(2, ctx=300)
    b.flat_sinks = True
    ka, va = a.prefill(0, 200)
    kb, vb = b.prefill(0, 200)
    assert np.array_equal(ka[4:], kb[4:])
    assert not np.array_equal(ka[:4], kb[:4])
    fa = synth.bits_to_f32(ka[:4], a.cfg.dtype).reshape(4, -1)
    fb = synth.bits_to_f32(kb[:4], b.cfg.dtype).reshape(4, -1)
    assert np.allclose(np.linalg.norm(fa, axis=1), np.linalg.norm(fb, axis=1), rtol=0.02)
    # energy share of each sink's 32 largest channels (of 1024): the outlier
    # channels hold ~90 % of an outlier-shaped sink's energy, ~20 % of a flat one's
    def top32(f):
        e = f ** 2
        return np.sort(e, axis=1)[:, -32:].sum(axis=1) / e.sum(axis=1)
    assert top32(fa).min() > 0.8 and top32(fb).max() < 0.3
