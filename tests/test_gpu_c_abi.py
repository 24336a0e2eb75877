"""The C ABI from plain C: tests/c_abi_demo (built by __graft_entry__.build()
from tests/c_abi_demo.c with gcc, linked against liboscar.so and the HIP
runtime only) runs layout, prefill, one append and decode attention on inputs
this test writes, and its outputs match the oracle."""
import os
import subprocess

import numpy as np
import pytest

from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a gfx950 GPU")]

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
EXE = os.path.join(ROOT, "tests", "c_abi_demo")

if gpu_available():
    import oracle
    from int2_kv_cache_amd import synth
    from _parity import ATOL


@pytest.mark.parametrize("cfg,ctx", [(0, 1024), (1, 700), (2, 97)])
def test_plain_c_caller_matches_oracle(tmp_path, cfg, ctx):
    assert os.path.exists(EXE), "tests/c_abi_demo is built by __graft_entry__.build()"
    wl = synth.workload(cfg, ctx=ctx)
    c = wl.cfg
    n = ctx - 1
    k, v = wl.prefill(0, n)
    kn, vn, q = next(wl.steps(1))
    src = tmp_path / "in.bin"
    with open(src, "wb") as f:
        f.write(np.array([c.hq, c.hkv, n, c.dtype], np.int32).tobytes())
        for a in (k, v, kn[0], vn[0], q[0]):
            f.write(np.ascontiguousarray(a, np.uint16).tobytes())
    dst = tmp_path / "out.bin"
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    raw = np.fromfile(dst, np.uint8)
    out = raw[:c.hq * 128 * 4].view(np.float32).reshape(c.hq, 128)
    lse = raw[c.hq * 128 * 4:c.hq * 129 * 4].view(np.float32)
    st = raw[c.hq * 129 * 4:].view(np.int32)
    orc = oracle.OracleCache(1, c.hq, c.hkv, ctx // 32 + 1)
    if n:
        orc.prefill(0, k, v, c.dtype)
    orc.append(kn, vn, c.dtype)
    want, wlse = orc.decode_attn(oracle.rotate_query(q, c.dtype))
    assert st.tolist() == [orc.n(0), orc.q(0), 0]
    assert np.abs(out - want[0]).max() <= ATOL
    assert np.allclose(lse, wlse[0], rtol=1e-3, atol=1e-3)
