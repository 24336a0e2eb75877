"""CPU checks of the C-ABI library: it loads, exports every symbol the
header declares, and its host-only calls behave (no GPU compute here)."""
import ctypes
import os
import re

import pytest

import int2_kv_cache_amd as ok

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "oscar.h")).read()
    return sorted(set(re.findall(r"\b(oscar_[a-z_]+)\s*\(", src)))


def test_header_declares_the_api():
    assert set(_declared()) == set(ok.API)


def test_library_exports_every_declared_symbol():
    lib = ok.lib()
    for name in _declared():
        assert hasattr(lib, name), name


def test_cache_layout_sizes():
    g = ok.make_geom(2, 32, 8, 100, 200)
    s = ok.cache_layout(g)
    assert s.pool == 200 * 8 * 3072
    assert s.pool_norm == 200 * 32 * 2
    assert s.res_k == s.res_v == 2 * 8 * 128 * 128 * 2
    assert s.res_norm == 2 * 128 * 2
    assert s.block_table == 2 * 100 * 4
    assert s.seq_state == 2 * 2 * 4
    assert s.error_flag == 4 and s.append_sync == 2 * 4


@pytest.mark.parametrize("bad", [
    dict(head_dim=64), dict(num_q_heads=6, num_kv_heads=4), dict(num_kv_heads=17, num_q_heads=34),
    dict(batch=0), dict(num_q_heads=24, num_kv_heads=8), dict(max_blocks_per_seq=0),
    dict(block_tokens=64), dict(block_tokens=0), dict(residual_tokens=256),
    dict(residual_tokens=0), dict(v_group=128), dict(v_group=0), dict(flush_tokens=64)])
def test_cache_layout_rejects(bad):
    args = dict(batch=1, num_q_heads=4, num_kv_heads=1, max_blocks_per_seq=4,
                num_physical_blocks=4)
    args.update(bad)
    with pytest.raises(ok.OscarError) as e:
        ok.cache_layout(ok.make_geom(**args))
    assert e.value.status == ok.EINVAL


def test_cache_layout_norm_scopes():
    """TOKEN scope keeps one norm per token, HEAD one per (token, KV head);
    any other scope value is rejected."""
    t = ok.cache_layout(ok.make_geom(3, 16, 4, 10, 25))
    h = ok.cache_layout(ok.make_geom(3, 16, 4, 10, 25, norm_scope=ok.NORM_HEAD))
    assert (t.pool_norm, t.res_norm) == (25 * 32 * 2, 3 * 128 * 2)
    assert (h.pool_norm, h.res_norm) == (25 * 4 * 32 * 2, 3 * 4 * 128 * 2)
    assert (t.pool, t.res_k, t.res_v) == (h.pool, h.res_k, h.res_v)
    with pytest.raises(ok.OscarError) as e:
        ok.cache_layout(ok.make_geom(1, 4, 1, 4, 4, norm_scope=7))
    assert e.value.status == ok.EINVAL


def test_cache_layout_key_scale():
    """The scaling factor's two forms are accepted, nothing else; the sizes do
    not depend on it."""
    a = ok.cache_layout(ok.make_geom(1, 8, 2, 6, 6))
    b = ok.cache_layout(ok.make_geom(1, 8, 2, 6, 6, key_scale=ok.SCALE_HW_RSQ))
    assert (a.pool, a.pool_norm, a.res_k) == (b.pool, b.pool_norm, b.res_k)
    with pytest.raises(ok.OscarError) as e:
        ok.cache_layout(ok.make_geom(1, 8, 2, 6, 6, key_scale=2))
    assert e.value.status == ok.EINVAL


def _dense_call(fn, *args):
    return getattr(ok.lib(), fn)(*args)


def test_dense_workspace_query_and_rejects():
    """Host-only: the bf16 baseline's workspace query sizes the same partials
    as the INT2 path; bad arguments are rejected before anything runs."""
    g = ok.make_geom(1, 32, 8, 4200, 4200)
    s, nbytes = ok.dense_workspace_bytes(g, 131072)
    assert 1 <= s <= 1024
    assert nbytes >= 32 * s * (8 + 512)
    for bad in [dict(max_ctx=-1), dict(num_splits=1025)]:
        args = dict(max_ctx=100, num_splits=0)
        args.update(bad)
        with pytest.raises(ok.OscarError) as e:
            ok.dense_workspace_bytes(g, **args)
        assert e.value.status == ok.EINVAL


def test_dense_calls_validate_before_touching_memory():
    """Null, misaligned or undersized arguments return a status and enqueue
    nothing (the fake addresses below are never dereferenced)."""
    g = ok.make_geom(1, 4, 1, 4, 4)
    vp = ctypes.c_void_p
    A = vp(0x100000)          # 256-byte aligned stand-ins
    odd = vp(0x100002)
    gr = ctypes.byref(g)
    _, need = ok.dense_workspace_bytes(g, 128, 0)
    common = lambda k, ws, nbytes: (gr, k, A, A, A, A, A, None, ws, nbytes, 0, 128, A, None)
    assert _dense_call("oscar_dense_decode_attn", *common(None, A, need)) == ok.EINVAL
    assert _dense_call("oscar_dense_decode_attn", *common(A, odd, need)) == ok.EINVAL
    assert _dense_call("oscar_dense_decode_attn", *common(A, A, need - 1)) == ok.EWORKSPACE
    # writes: sequence out of range, past the block table's capacity, misaligned input
    assert _dense_call("oscar_dense_write_kv", gr, A, A, A, 1, 0, A, A, 8, A, None) == ok.EINVAL
    assert _dense_call("oscar_dense_write_kv", gr, A, A, A, 0, 120, A, A, 9, A, None) == ok.EINVAL
    assert _dense_call("oscar_dense_write_kv", gr, A, A, A, 0, 0, odd, A, 8, A, None) == ok.EINVAL


def test_absorb_value_rotation_validates_before_launch():
    """Shapes the transform cannot take are refused on the host (the fake
    addresses are never dereferenced)."""
    L = ok.lib()
    A = ctypes.c_void_p(0x100000)
    for w, o, rows, cols, axis in [(None, A, 128, 4, 0), (A, None, 128, 4, 0),
                                   (A, A, 100, 4, 0), (A, A, 4, 100, 1), (A, A, 128, 128, 2),
                                   (A, A, -128, 4, 0), (A, A, 128, -1, 0),
                                   (A, A, 1 << 40, 1 << 40, 1)]:
        assert L.oscar_absorb_value_rotation(w, o, rows, cols, axis, None) == ok.EINVAL


def test_noalloc_refuses_a_workspace_beyond_its_array():
    """Host-only: a call whose partials need more than the 8 MiB static
    workspace returns OSCAR_EWORKSPACE before touching the device (the fake
    addresses are never dereferenced)."""
    g = ok.make_geom(48, 32, 8, 1100, 48 * 1100)
    assert ok.decode_workspace_bytes(g, 35000, 1024)[1] > ok.STATIC_WORKSPACE_BYTES
    A = ctypes.c_void_p(0x100000)
    bufs = ok.CacheBufs(*([0x100000] * len(ok.CacheBufs._fields_)))
    st = ok.lib().oscar_decode_attn_noalloc(ctypes.byref(g), ctypes.byref(bufs), A, ok.BF16, A,
                                            None, 1024, 35000, ok.ATTN_AUTO, None)
    assert st == ok.EWORKSPACE


def test_status_strings():
    assert ok.status_str(ok.OK) == "ok"
    assert "workspace" in ok.status_str(ok.EWORKSPACE)
