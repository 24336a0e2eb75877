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
