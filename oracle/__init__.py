"""CPU oracle of the OScaR INT2 KV-cache hot path (ctypes binding).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``.  The GPU package never imports it.

The arithmetic lives in ``oscar_oracle.c`` (plain C, built with
``-O2 -ffp-contract=off``).  This module only marshals numpy arrays.
Every function cites the page passage it follows in the C source.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oscar_oracle.c")
LIB = os.path.join(HERE, "liboscar_oracle.so")

D, G, R, VG, REC_BYTES = 128, 32, 128, 32, 3072
FP16, BF16 = 0, 1
NORM_TOKEN, NORM_HEAD = 0, 1


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no FMA contraction, no fast-math)."""
    if not force and os.path.exists(LIB):
        return LIB
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-Wall", "-Wextra", "-shared", "-fPIC", SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


class Cache(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("norm_scope", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("num_physical_blocks", ctypes.c_int32), ("flush_tokens", ctypes.c_int32),
        ("pool", ctypes.c_void_p), ("pool_norm", ctypes.c_void_p),
        ("res_k", ctypes.c_void_p), ("res_v", ctypes.c_void_p),
        ("res_norm", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
        ("seq_state", ctypes.c_void_p), ("error_flag", ctypes.c_void_p),
        ("rope", ctypes.c_void_p), ("rope_max_pos", ctypes.c_int32),
    ]


def lib():
    global _lib
    if _lib is None:
        src_time = max(os.path.getmtime(SRC), os.path.getmtime(os.path.join(HERE, "oscar_oracle.h")))
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < src_time:
            build()
        L = ctypes.CDLL(LIB)
        vp, i32, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        sig = {
            "orc_f32_to_f16": (ctypes.c_uint16, [f32]),
            "orc_f32_to_f16_sat": (ctypes.c_uint16, [f32]),
            "orc_f16_to_f32": (f32, [ctypes.c_uint16]),
            "orc_bf16_to_f32": (f32, [ctypes.c_uint16]),
            "orc_to_f16": (None, [vp, i32, sz, vp]),
            "orc_fht_scale": (f32, []),
            "orc_fht128": (None, [vp]),
            "orc_rotate_query": (None, [vp, i32, sz, vp]),
            "orc_tree_sumsq": (f32, [vp, i32]),
            "orc_rotate_scale_key": (None, [vp, i32, i32, i32, i32, vp, vp]),
            "orc_rotate_scale_key_pos": (None, [vp, i32, i32, i32, i32, vp, i32, vp, vp]),
            "orc_rope": (None, [vp, vp]),
            "orc_rotate_query_pos": (None, [vp, i32, sz, vp, vp]),
            "orc_absorb_value_rotation": (None, [vp, vp, i32, i32, i32]),
            "orc_quant_group32": (None, [vp, sz, vp, vp, vp]),
            "orc_kcode_byte": (sz, [i32, i32]),
            "orc_kcode_shift": (i32, [i32, i32]),
            "orc_vcode_byte": (sz, [i32, i32]),
            "orc_vcode_shift": (i32, [i32, i32]),
            "orc_quant_pack": (None, [vp, vp, vp, i32, i32, i32, vp, vp]),
            "orc_append": (None, [vp, vp, vp, i32]),
            "orc_append_one": (None, [vp, i32, vp, vp, i32]),
            "orc_prefill": (i32, [vp, i32, vp, vp, i32, i32]),
            "orc_key_row": (None, [vp, i32, i32, i32, vp]),
            "orc_value_row": (None, [vp, i32, i32, i32, vp]),
            "orc_decode_attn": (None, [vp, vp, vp, vp]),
            "orc_decode_attn_one": (None, [vp, vp, i32, i32, vp, vp]),
            "orc_decode_attn_partial": (None, [vp, vp, i32, i32, i32, i32, vp, vp, vp]),
            "orc_lse_merge": (None, [i32, vp, vp, vp, vp, vp]),
            "orc_dense_attn": (None, [vp, vp, vp, i32, i32, i32, vp, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def bf16_bits_to_f32(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> the fp32 values they denote (exact)."""
    return (np.asarray(x, np.uint16).astype(np.uint32) << 16).view(np.float32)


def dense_attn(q: np.ndarray, k: np.ndarray, v: np.ndarray):
    """Unquantized fp64 decode attention of one sequence (the BF16 baseline).

    q [Hq][128], k and v [n][Hkv][128], fp32 values (bf16 inputs converted
    exactly with ``bf16_bits_to_f32``).  Returns out [Hq][128] fp32 and
    lse [Hq] fp32.  The arithmetic is ``orc_dense_attn`` in oscar_oracle.c.
    """
    q = np.ascontiguousarray(q, np.float32)
    k = np.ascontiguousarray(k, np.float32)
    v = np.ascontiguousarray(v, np.float32)
    hq = q.shape[0]
    n, hkv = k.shape[0], k.shape[1]
    assert q.shape == (hq, D) and k.shape == (n, hkv, D) and v.shape == k.shape
    assert hq % hkv == 0
    out = np.zeros((hq, D), np.float32)
    lse = np.zeros(hq, np.float32)
    lib().orc_dense_attn(_p(q), _p(k), _p(v), n, hq, hkv, _p(out), _p(lse))
    return out, lse


def _p(a: np.ndarray | None):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data


# ---------------------------------------------------------------- numbers
def f32_to_f16(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32).ravel()
    L = lib()
    return np.array([L.orc_f32_to_f16(float(v)) for v in x], dtype=np.uint16)


def f32_to_f16_sat(x) -> np.ndarray:
    """fp32 -> fp16 bits of a stored value: clamped to +-65504, then RNE."""
    x = np.asarray(x, dtype=np.float32).ravel()
    L = lib()
    return np.array([L.orc_f32_to_f16_sat(float(v)) for v in x], dtype=np.uint16)


def lse_merge(m: np.ndarray, l: np.ndarray, o: np.ndarray):
    """Merge split-K partials of one query head: m, l [S] (natural log), o
    [S][128] (unnormalised).  Returns out [128] fp32 and lse fp32."""
    m = np.ascontiguousarray(m, np.float64)
    l = np.ascontiguousarray(l, np.float64)
    o = np.ascontiguousarray(o, np.float64)
    assert m.shape == l.shape and o.shape == (m.size, D)
    out = np.zeros(D, np.float32)
    lse = np.zeros(1, np.float32)
    lib().orc_lse_merge(m.size, _p(m), _p(l), _p(o), _p(out), _p(lse))
    return out, lse[0]


def in_to_f16(x: np.ndarray, dtype: int) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.empty_like(x)
    lib().orc_to_f16(_p(x), dtype, x.size, _p(out))
    return out


# ---------------------------------------------------------------- rotation
def fht128(x: np.ndarray) -> np.ndarray:
    """FHT of each 128-vector along the last axis (fp32 in, fp32 out)."""
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    flat = y.reshape(-1, D)
    L = lib()
    for r in range(flat.shape[0]):
        L.orc_fht128(flat[r].ctypes.data)
    return y


def rotate_query(q: np.ndarray, dtype: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint16)
    out = np.empty(q.shape, dtype=np.float32)
    lib().orc_rotate_query(_p(q), dtype, q.size // D, _p(out))
    return out


def rope(x: np.ndarray, cs: np.ndarray) -> np.ndarray:
    """RoPE of one 128-vector (fp32) with a (cos, sin) row cs [64][2]."""
    y = np.ascontiguousarray(x, dtype=np.float32).copy()
    cs = np.ascontiguousarray(cs, dtype=np.float32)
    assert y.shape == (D,) and cs.shape == (D // 2, 2)
    lib().orc_rope(_p(y), _p(cs))
    return y


def rotate_query_pos(q: np.ndarray, dtype: int, cs) -> np.ndarray:
    """RoPE (every vector at the position of the (cos, sin) row cs, or none
    when cs is None) then the FHT, fp32 out."""
    q = np.ascontiguousarray(q, dtype=np.uint16)
    out = np.empty(q.shape, dtype=np.float32)
    csp = None
    if cs is not None:
        cs = np.ascontiguousarray(cs, dtype=np.float32)
        assert cs.shape == (D // 2, 2)
        csp = _p(cs)
    lib().orc_rotate_query_pos(_p(q), dtype, q.size // D, csp, _p(out))
    return out


def absorb_value_rotation(w: np.ndarray, axis: int) -> np.ndarray:
    """W_v' = H W_v per 128-row block (axis 0) or W_o' = W_o H per 128-column
    block (axis 1), fp32."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    rows, cols = w.shape
    assert (rows if axis == 0 else cols) % D == 0
    out = np.empty_like(w)
    lib().orc_absorb_value_rotation(_p(w), _p(out), rows, cols, axis)
    return out


def tree_sumsq(y: np.ndarray) -> np.float32:
    y = np.ascontiguousarray(y, dtype=np.float32)
    return np.float32(lib().orc_tree_sumsq(_p(y), y.size))


def rotate_scale_key(k: np.ndarray, dtype: int, norm_scope: int = NORM_TOKEN,
                     rope_table=None, pos0: int = 0):
    """k: [T, Hkv, 128] raw bits -> (khat fp16 bits [T,Hkv,128], norm fp16 bits).
    With rope_table ([positions][64][2] fp32), token t is first rotated by
    position pos0 + t."""
    k = np.ascontiguousarray(k, dtype=np.uint16)
    T, hkv, _ = k.shape
    khat = np.empty_like(k)
    norm = np.empty((T,) if norm_scope == NORM_TOKEN else (T, hkv), dtype=np.uint16)
    rp = None
    if rope_table is not None:
        rope_table = np.ascontiguousarray(rope_table, dtype=np.float32)
        assert rope_table.shape[0] >= pos0 + T
        rp = _p(rope_table)
    lib().orc_rotate_scale_key_pos(_p(k), dtype, T, hkv, norm_scope, rp, pos0, _p(khat),
                                   _p(norm))
    return khat, norm


# ---------------------------------------------------------------- quantizer
def quant_group32(x16: np.ndarray):
    """32 fp16 bit patterns -> (delta fp32, zero fp32, codes uint8[32])."""
    x16 = np.ascontiguousarray(x16, dtype=np.uint16)
    assert x16.size == 32
    d = np.zeros(1, np.float32)
    z = np.zeros(1, np.float32)
    codes = np.zeros(32, np.uint8)
    lib().orc_quant_group32(_p(x16), 1, _p(d), _p(z), _p(codes))
    return d[0], z[0], codes


def quant_pack(khat: np.ndarray, knorm: np.ndarray, v16: np.ndarray,
               norm_scope: int = NORM_TOKEN):
    """khat, v16: [32*nb, Hkv, 128] fp16 bits -> (records [nb,Hkv,3072], norms)."""
    khat = np.ascontiguousarray(khat, dtype=np.uint16)
    v16 = np.ascontiguousarray(v16, dtype=np.uint16)
    knorm = np.ascontiguousarray(knorm, dtype=np.uint16)
    T, hkv, _ = khat.shape
    assert T % G == 0
    nb = T // G
    rec = np.zeros((nb, hkv, REC_BYTES), np.uint8)
    norm = np.zeros((nb, G) if norm_scope == NORM_TOKEN else (nb, hkv, G), np.uint16)
    lib().orc_quant_pack(_p(khat), _p(knorm), _p(v16), nb, hkv, norm_scope,
                         _p(rec), _p(norm))
    return rec, norm


def kcode_get(rec: np.ndarray, t: int, c: int) -> int:
    L = lib()
    return (int(rec[L.orc_kcode_byte(t, c)]) >> L.orc_kcode_shift(t, c)) & 3


def vcode_get(rec: np.ndarray, t: int, c: int) -> int:
    L = lib()
    return (int(rec[L.orc_vcode_byte(t, c)]) >> L.orc_vcode_shift(t, c)) & 3


# ---------------------------------------------------------------- cache
class OracleCache:
    """Numpy-backed cache in the canonical byte layout (see oscar_oracle.c)."""

    def __init__(self, batch: int, hq: int, hkv: int, max_blocks: int,
                 num_phys: int | None = None, norm_scope: int = NORM_TOKEN,
                 block_table: np.ndarray | None = None, flush_tokens: int = 32,
                 rope_table: np.ndarray | None = None):
        self.batch, self.hq, self.hkv = batch, hq, hkv
        self.norm_scope = norm_scope
        self.max_blocks = max_blocks
        self.num_phys = num_phys if num_phys is not None else batch * max_blocks
        self.pool = np.zeros((self.num_phys, hkv, REC_BYTES), np.uint8)
        if norm_scope == NORM_TOKEN:
            self.pool_norm = np.zeros((self.num_phys, G), np.uint16)
            self.res_norm = np.zeros((batch, R), np.uint16)
        else:
            self.pool_norm = np.zeros((self.num_phys, hkv, G), np.uint16)
            self.res_norm = np.zeros((batch, hkv, R), np.uint16)
        self.res_k = np.zeros((batch, hkv, R, D), np.uint16)
        self.res_v = np.zeros((batch, hkv, D, R), np.uint16)
        if block_table is None:
            block_table = np.arange(batch * max_blocks, dtype=np.int32).reshape(batch, max_blocks)
        self.block_table = np.ascontiguousarray(block_table, dtype=np.int32)
        self.seq_state = np.zeros((batch, 2), np.int32)
        self.error_flag = np.zeros(1, np.int32)
        assert flush_tokens in (32, 128)
        self.flush_tokens = flush_tokens
        self.rope_table = None
        if rope_table is not None:
            self.rope_table = np.ascontiguousarray(rope_table, dtype=np.float32)
            assert self.rope_table.shape[1:] == (D // 2, 2)
        self._s = Cache(batch, hq, hkv, norm_scope, max_blocks, self.num_phys, flush_tokens,
                        _p(self.pool), _p(self.pool_norm), _p(self.res_k),
                        _p(self.res_v), _p(self.res_norm), _p(self.block_table),
                        _p(self.seq_state), _p(self.error_flag),
                        _p(self.rope_table) if self.rope_table is not None else None,
                        self.rope_table.shape[0] if self.rope_table is not None else 0)

    @property
    def ref(self):
        return ctypes.byref(self._s)

    def append(self, k_new: np.ndarray, v_new: np.ndarray, dtype: int):
        k_new = np.ascontiguousarray(k_new, dtype=np.uint16)
        v_new = np.ascontiguousarray(v_new, dtype=np.uint16)
        assert k_new.shape == (self.batch, self.hkv, D) == v_new.shape
        lib().orc_append(self.ref, _p(k_new), _p(v_new), dtype)

    def prefill(self, b: int, k: np.ndarray, v: np.ndarray, dtype: int):
        k = np.ascontiguousarray(k, dtype=np.uint16)
        v = np.ascontiguousarray(v, dtype=np.uint16)
        assert k.shape == v.shape and k.shape[1:] == (self.hkv, D)
        rc = lib().orc_prefill(self.ref, b, _p(k), _p(v), k.shape[0], dtype)
        if rc != 0:
            raise ValueError("prefill into a non-empty sequence")

    def key_row(self, b: int, h: int, t: int) -> np.ndarray:
        out = np.zeros(D, np.float64)
        lib().orc_key_row(self.ref, b, h, t, _p(out))
        return out

    def value_row(self, b: int, h: int, t: int) -> np.ndarray:
        out = np.zeros(D, np.float64)
        lib().orc_value_row(self.ref, b, h, t, _p(out))
        return out

    def decode_attn(self, qrot: np.ndarray):
        qrot = np.ascontiguousarray(qrot, dtype=np.float32)
        assert qrot.shape == (self.batch, self.hq, D)
        out = np.zeros_like(qrot)
        lse = np.zeros((self.batch, self.hq), np.float32)
        lib().orc_decode_attn(self.ref, _p(qrot), _p(out), _p(lse))
        return out, lse

    def decode_attn_one(self, qrot: np.ndarray, b: int, i: int):
        qrot = np.ascontiguousarray(qrot, dtype=np.float32)
        out = np.zeros(D, np.float32)
        lse = np.zeros(1, np.float32)
        lib().orc_decode_attn_one(self.ref, _p(qrot), b, i, _p(out), _p(lse))
        return out, lse[0]

    def decode_attn_partial(self, qrot: np.ndarray, b: int, i: int, t0: int, t1: int):
        """Split-K partial over tokens [t0, t1): (m, l, o[128]), fp64."""
        qrot = np.ascontiguousarray(qrot, dtype=np.float32)
        m = np.zeros(1, np.float64)
        l = np.zeros(1, np.float64)
        o = np.zeros(D, np.float64)
        lib().orc_decode_attn_partial(self.ref, _p(qrot), b, i, t0, t1, _p(m), _p(l), _p(o))
        return m[0], l[0], o

    # views of the valid state (what parity compares)
    def n(self, b: int) -> int:
        return int(self.seq_state[b, 0])

    def q(self, b: int) -> int:
        return int(self.seq_state[b, 1])
