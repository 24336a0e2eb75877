"""Python binding of liboscar.so, the gfx950 OScaR INT2 KV-cache library.

Argument marshalling only: every step of the path runs in the HIP kernels
behind the C ABI declared in ``include/oscar.h``.  torch supplies device
memory and the current stream.  There is no CPU fallback: if the library is
not built, or the device is not gfx950, calls raise.

The functions keep the C names without the ``oscar_`` prefix:
``cache_layout``, ``rotate_scale``, ``quant_pack``, ``append_kv``,
``prefill_quantize``, ``decode_workspace_bytes``, ``decode_attn``.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liboscar.so")

OK, EINVAL, EUNSUPPORTED, ELAUNCH, EWORKSPACE = 0, 1, 2, 3, 4
FP16, BF16, FP32 = 0, 1, 2
NORM_TOKEN, NORM_HEAD = 0, 1
ROT_QUERY, ROT_KEY, ROT_KEY_HW_RSQ = 0, 1, 2
SCALE_IEEE, SCALE_HW_RSQ = 0, 1
ATTN_AUTO, ATTN_VALU, ATTN_MFMA = 0, 1, 2
FLAG_CAPACITY, FLAG_NONEMPTY, FLAG_BADSTATE, FLAG_POSITION = 1, 2, 4, 8
HEAD_DIM, BLOCK_TOKENS, RESIDUAL_TOKENS, V_GROUP, RECORD_BYTES = 128, 32, 128, 32, 3072

API = ("oscar_cache_layout", "oscar_rotate_scale", "oscar_quant_pack", "oscar_append_kv",
       "oscar_prefill_quantize", "oscar_decode_workspace_bytes", "oscar_decode_attn",
       "oscar_dense_write_kv", "oscar_dense_workspace_bytes", "oscar_dense_decode_attn",
       "oscar_absorb_value_rotation", "oscar_decode_attn_noalloc", "oscar_decode_step",
       "oscar_status_str")


class OscarError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (%d)" % (fn, status_str(status), status))
        self.status = status


class Geom(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_tokens", ctypes.c_int32), ("residual_tokens", ctypes.c_int32),
                ("v_group", ctypes.c_int32),
                ("norm_scope", ctypes.c_int32), ("max_blocks_per_seq", ctypes.c_int32),
                ("num_physical_blocks", ctypes.c_int32), ("flush_tokens", ctypes.c_int32),
                ("key_scale", ctypes.c_int32), ("rope_max_pos", ctypes.c_int32)]


class CacheBufs(ctypes.Structure):
    _fields_ = [("pool", ctypes.c_void_p), ("pool_norm", ctypes.c_void_p),
                ("res_k", ctypes.c_void_p), ("res_v", ctypes.c_void_p),
                ("res_norm", ctypes.c_void_p), ("block_table", ctypes.c_void_p),
                ("seq_state", ctypes.c_void_p), ("error_flag", ctypes.c_void_p),
                ("append_sync", ctypes.c_void_p), ("rope", ctypes.c_void_p)]


class CacheSizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("pool", "pool_norm", "res_k", "res_v", "res_norm", "block_table",
                 "seq_state", "error_flag", "append_sync")]


_lib = None


def lib() -> ctypes.CDLL:
    """Load liboscar.so; raise if it is not built (no fallback exists)."""
    global _lib
    if _lib is None:
        # torch first: its bundled HIP runtime must be the one liboscar.so binds
        # to (same soname), so tensors and kernels share one runtime.
        import torch  # noqa: F401
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("liboscar.so is not built: run __graft_entry__.build() "
                               "(the HIP library is the only implementation)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, st = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int
        P = ctypes.POINTER
        L.oscar_cache_layout.argtypes = [P(Geom), P(CacheSizes)]
        L.oscar_rotate_scale.argtypes = [vp, st, i32, i32, st, st, vp, vp, vp, vp]
        L.oscar_quant_pack.argtypes = [vp, vp, vp, i32, i32, st, vp, vp, vp]
        L.oscar_append_kv.argtypes = [P(Geom), P(CacheBufs), vp, vp, st, vp]
        L.oscar_prefill_quantize.argtypes = [P(Geom), P(CacheBufs), i32, vp, vp, i32, st, vp]
        L.oscar_decode_workspace_bytes.argtypes = [P(Geom), i32, i32, P(ctypes.c_int32),
                                                   P(ctypes.c_size_t)]
        L.oscar_decode_attn.argtypes = [P(Geom), P(CacheBufs), vp, st, vp, vp, vp,
                                        ctypes.c_size_t, i32, i32, st, vp]
        L.oscar_decode_step.argtypes = [P(Geom), P(CacheBufs), vp, vp, st, vp, st, vp, vp, vp,
                                        ctypes.c_size_t, i32, i32, st, vp]
        L.oscar_dense_write_kv.argtypes = [P(Geom), vp, vp, vp, i32, i32, vp, vp, i32, vp, vp]
        L.oscar_dense_workspace_bytes.argtypes = [P(Geom), i32, i32, P(ctypes.c_int32),
                                                  P(ctypes.c_size_t)]
        L.oscar_dense_decode_attn.argtypes = [P(Geom), vp, vp, vp, vp, vp, vp, vp, vp,
                                              ctypes.c_size_t, i32, i32, vp, vp]
        L.oscar_decode_attn_noalloc.argtypes = [P(Geom), P(CacheBufs), vp, st, vp, vp, i32, i32,
                                                st, vp]
        L.oscar_absorb_value_rotation.argtypes = [vp, vp, ctypes.c_int64, ctypes.c_int64, i32,
                                                  vp]
        for name in API:
            getattr(L, name).restype = ctypes.c_int
        L.oscar_status_str.restype = ctypes.c_char_p
        L.oscar_status_str.argtypes = [ctypes.c_int]
        _lib = L
    return _lib


def status_str(s: int) -> str:
    return lib().oscar_status_str(s).decode()


def _check(fn: str, s: int):
    if s != OK:
        raise OscarError(fn, s)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def make_geom(batch, num_q_heads, num_kv_heads, max_blocks_per_seq, num_physical_blocks,
              norm_scope=NORM_TOKEN, head_dim=HEAD_DIM, flush_tokens=32,
              key_scale=SCALE_IEEE, block_tokens=BLOCK_TOKENS,
              residual_tokens=RESIDUAL_TOKENS, v_group=V_GROUP, rope_max_pos=0) -> Geom:
    return Geom(batch, num_q_heads, num_kv_heads, head_dim, block_tokens, residual_tokens,
                v_group, norm_scope, max_blocks_per_seq, num_physical_blocks, flush_tokens,
                key_scale, rope_max_pos)


def cache_layout(geom: Geom) -> CacheSizes:
    out = CacheSizes()
    _check("oscar_cache_layout", lib().oscar_cache_layout(ctypes.byref(geom), ctypes.byref(out)))
    return out


class DeviceCache:
    """Cache buffers as torch tensors on the current device, sized by
    oscar_cache_layout and zero-initialised (torch is the allocator)."""

    def __init__(self, geom: Geom, block_table=None, device="cuda", rope_table=None):
        """rope_table: [geom.rope_max_pos][64][2] fp32 (cos, sin), required
        when geom.rope_max_pos > 0."""
        import torch
        self.geom = geom
        sz = cache_layout(geom)
        B, H = geom.batch, geom.num_kv_heads

        def u8(n):
            return torch.zeros(n, dtype=torch.uint8, device=device)

        self.pool = u8(sz.pool).view(geom.num_physical_blocks, H, RECORD_BYTES)
        nh = (H,) if geom.norm_scope == NORM_HEAD else ()   # norms per (token, KV head)
        self.pool_norm = torch.zeros(geom.num_physical_blocks, *nh, 32, dtype=torch.int16,
                                     device=device)
        self.res_k = torch.zeros(B, H, 128, 128, dtype=torch.int16, device=device)
        self.res_v = torch.zeros(B, H, 128, 128, dtype=torch.int16, device=device)
        self.res_norm = torch.zeros(B, *nh, 128, dtype=torch.int16, device=device)
        assert self.pool_norm.numel() * 2 == sz.pool_norm and self.res_norm.numel() * 2 == sz.res_norm
        if block_table is None:
            block_table = torch.arange(B * geom.max_blocks_per_seq, dtype=torch.int32)
            block_table = block_table.view(B, geom.max_blocks_per_seq) % geom.num_physical_blocks
        self.block_table = torch.as_tensor(block_table, dtype=torch.int32).to(device).contiguous()
        self.seq_state = torch.zeros(B, 2, dtype=torch.int32, device=device)
        self.error_flag = torch.zeros(1, dtype=torch.int32, device=device)
        self.append_sync = torch.zeros(B, dtype=torch.int32, device=device)
        self.rope = None
        if rope_table is not None:
            self.rope = torch.as_tensor(rope_table, dtype=torch.float32).to(device).contiguous()
            assert tuple(self.rope.shape) == (geom.rope_max_pos, 64, 2)
        self.bufs = CacheBufs(*(t.data_ptr() for t in (
            self.pool, self.pool_norm, self.res_k, self.res_v, self.res_norm,
            self.block_table, self.seq_state, self.error_flag, self.append_sync)),
            self.rope.data_ptr() if self.rope is not None else None)


def rotate_scale(x, dtype: int, mode: int, norm_scope: int = NORM_TOKEN, q_out=None,
                 khat_out=None, norm_out=None, stream=None):
    """x: [n_tokens, n_heads, 128] 16-bit tensor (bit patterns of dtype)."""
    n_tokens, n_heads = x.shape[0], x.shape[1]
    _check("oscar_rotate_scale", lib().oscar_rotate_scale(
        _ptr(x), dtype, n_tokens, n_heads, mode, norm_scope, _ptr(q_out), _ptr(khat_out),
        _ptr(norm_out), _stream(stream)))


def absorb_value_rotation(w, axis: int, out=None, stream=None):
    """w: 2-D contiguous fp32 device tensor.  axis 0: H times every 128-row
    block (W_v' = H W_v); axis 1: every 128-column block times H
    (W_o' = W_o H).  Returns `out` (a new tensor unless given; may be w)."""
    assert w.dtype.is_floating_point and w.element_size() == 4 and w.dim() == 2
    assert w.is_contiguous()
    if out is None:
        import torch
        out = torch.empty_like(w)
    _check("oscar_absorb_value_rotation", lib().oscar_absorb_value_rotation(
        _ptr(w), _ptr(out), w.shape[0], w.shape[1], axis, _stream(stream)))
    return out


def quant_pack(khat16, knorm16, v16, rec_out, norm_out, norm_scope=NORM_TOKEN, stream=None):
    n_blocks, hkv = khat16.shape[0] // BLOCK_TOKENS, khat16.shape[1]
    _check("oscar_quant_pack", lib().oscar_quant_pack(
        _ptr(khat16), _ptr(knorm16), _ptr(v16), n_blocks, hkv, norm_scope, _ptr(rec_out),
        _ptr(norm_out), _stream(stream)))


def append_kv(cache: DeviceCache, k_new, v_new, dtype: int, stream=None):
    _check("oscar_append_kv", lib().oscar_append_kv(
        ctypes.byref(cache.geom), ctypes.byref(cache.bufs), _ptr(k_new), _ptr(v_new), dtype,
        _stream(stream)))


def prefill_quantize(cache: DeviceCache, seq: int, k, v, dtype: int, stream=None):
    _check("oscar_prefill_quantize", lib().oscar_prefill_quantize(
        ctypes.byref(cache.geom), ctypes.byref(cache.bufs), seq, _ptr(k), _ptr(v), k.shape[0],
        dtype, _stream(stream)))


def decode_workspace_bytes(geom: Geom, max_ctx: int, num_splits: int = 0):
    s = ctypes.c_int32(0)
    nbytes = ctypes.c_size_t(0)
    _check("oscar_decode_workspace_bytes", lib().oscar_decode_workspace_bytes(
        ctypes.byref(geom), max_ctx, num_splits, ctypes.byref(s), ctypes.byref(nbytes)))
    return s.value, nbytes.value


def decode_attn(cache: DeviceCache, q, q_dtype: int, out, lse, workspace, max_ctx: int,
                num_splits: int = 0, variant: int = ATTN_AUTO, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    _check("oscar_decode_attn", lib().oscar_decode_attn(
        ctypes.byref(cache.geom), ctypes.byref(cache.bufs), _ptr(q), q_dtype, _ptr(out),
        _ptr(lse), _ptr(workspace), nbytes, num_splits, max_ctx, variant, _stream(stream)))


def decode_step(cache: DeviceCache, k_new, v_new, kv_dtype: int, q, q_dtype: int, out, lse,
                workspace, max_ctx: int, num_splits: int = 0, variant: int = ATTN_AUTO,
                stream=None):
    """oscar_decode_step: append_kv(k_new, v_new) then decode_attn(q), in one
    launch (two with ATTN_VALU)."""
    nbytes = workspace.numel() * workspace.element_size()
    _check("oscar_decode_step", lib().oscar_decode_step(
        ctypes.byref(cache.geom), ctypes.byref(cache.bufs), _ptr(k_new), _ptr(v_new), kv_dtype,
        _ptr(q), q_dtype, _ptr(out), _ptr(lse), _ptr(workspace), nbytes, num_splits, max_ctx,
        variant, _stream(stream)))


STATIC_WORKSPACE_BYTES = 8 << 20   # OSCAR_STATIC_WORKSPACE_BYTES


def decode_attn_noalloc(cache: DeviceCache, q, q_dtype: int, out, lse, max_ctx: int,
                        num_splits: int = 0, variant: int = ATTN_AUTO, stream=None):
    """oscar_decode_attn_noalloc: decode attention with the library's own
    per-GPU workspace, for callers that cannot allocate."""
    _check("oscar_decode_attn_noalloc", lib().oscar_decode_attn_noalloc(
        ctypes.byref(cache.geom), ctypes.byref(cache.bufs), _ptr(q), q_dtype, _ptr(out),
        _ptr(lse), num_splits, max_ctx, variant, _stream(stream)))


# ---------------------------------------------------------------- prepared calls

class PreparedCall:
    """One C-ABI call whose arguments were marshalled once: calling it only
    crosses into the library.  The tensors it was prepared with must stay
    alive and in place (their device addresses are baked in), and the
    stream is fixed at preparation."""
    __slots__ = ("fn", "name", "args")

    def __init__(self, name: str, args: tuple):
        self.fn = getattr(lib(), name)
        self.name = name
        self.args = args

    def __call__(self):
        s = self.fn(*self.args)
        if s != OK:
            raise OscarError(self.name, s)


def prepare_append_kv(cache: DeviceCache, k_new, v_new, dtype: int, stream=None) -> PreparedCall:
    return PreparedCall("oscar_append_kv", (
        ctypes.byref(cache.geom), ctypes.byref(cache.bufs), _ptr(k_new), _ptr(v_new), dtype,
        _stream(stream)))


def prepare_decode_attn(cache: DeviceCache, q, q_dtype: int, out, lse, workspace, max_ctx: int,
                        num_splits: int = 0, variant: int = ATTN_AUTO,
                        stream=None) -> PreparedCall:
    nbytes = workspace.numel() * workspace.element_size()
    return PreparedCall("oscar_decode_attn", (
        ctypes.byref(cache.geom), ctypes.byref(cache.bufs), _ptr(q), q_dtype, _ptr(out),
        _ptr(lse), _ptr(workspace), ctypes.c_size_t(nbytes), num_splits, max_ctx, variant,
        _stream(stream)))


def prepare_decode_step(cache: DeviceCache, k_new, v_new, kv_dtype: int, q, q_dtype: int, out,
                        lse, workspace, max_ctx: int, num_splits: int = 0,
                        variant: int = ATTN_AUTO, stream=None) -> PreparedCall:
    nbytes = workspace.numel() * workspace.element_size()
    return PreparedCall("oscar_decode_step", (
        ctypes.byref(cache.geom), ctypes.byref(cache.bufs), _ptr(k_new), _ptr(v_new), kv_dtype,
        _ptr(q), q_dtype, _ptr(out), _ptr(lse), _ptr(workspace), ctypes.c_size_t(nbytes),
        num_splits, max_ctx, variant, _stream(stream)))


# ---------------------------------------------------------------- bf16 baseline

class DenseCache:
    """Paged bf16 cache of the baseline kernel as torch tensors on the current
    device: k_pool [P][Hkv][32][128], v_pool [P][Hkv][128][32] (bf16 bit
    patterns as int16), block_table [B][max_blocks], ctx_lens [B], error_flag."""

    def __init__(self, geom: Geom, block_table=None, device="cuda"):
        import torch
        self.geom = geom
        P, H, B = geom.num_physical_blocks, geom.num_kv_heads, geom.batch
        self.k_pool = torch.zeros(P, H, BLOCK_TOKENS, HEAD_DIM, dtype=torch.int16, device=device)
        self.v_pool = torch.zeros(P, H, HEAD_DIM, BLOCK_TOKENS, dtype=torch.int16, device=device)
        if block_table is None:
            block_table = torch.arange(B * geom.max_blocks_per_seq, dtype=torch.int32)
            block_table = block_table.view(B, geom.max_blocks_per_seq) % P
        self.block_table = torch.as_tensor(block_table, dtype=torch.int32).to(device).contiguous()
        self.ctx_lens = torch.zeros(B, dtype=torch.int32, device=device)
        self.error_flag = torch.zeros(1, dtype=torch.int32, device=device)


def dense_write_kv(cache: DenseCache, seq: int, start: int, k, v, stream=None):
    """k, v: [n_tokens, Hkv, 128] bf16 bit patterns (int16/uint16 tensor)."""
    _check("oscar_dense_write_kv", lib().oscar_dense_write_kv(
        ctypes.byref(cache.geom), _ptr(cache.k_pool), _ptr(cache.v_pool), _ptr(cache.block_table),
        seq, start, _ptr(k), _ptr(v), k.shape[0], _ptr(cache.error_flag), _stream(stream)))


def dense_workspace_bytes(geom: Geom, max_ctx: int, num_splits: int = 0):
    s = ctypes.c_int32(0)
    nbytes = ctypes.c_size_t(0)
    _check("oscar_dense_workspace_bytes", lib().oscar_dense_workspace_bytes(
        ctypes.byref(geom), max_ctx, num_splits, ctypes.byref(s), ctypes.byref(nbytes)))
    return s.value, nbytes.value


def dense_decode_attn(cache: DenseCache, q, out, lse, workspace, max_ctx: int,
                      num_splits: int = 0, stream=None):
    """q: [B, Hq, 128] bf16 bit patterns; out [B, Hq, 128] fp32; lse [B, Hq] or None."""
    nbytes = workspace.numel() * workspace.element_size()
    _check("oscar_dense_decode_attn", lib().oscar_dense_decode_attn(
        ctypes.byref(cache.geom), _ptr(cache.k_pool), _ptr(cache.v_pool), _ptr(cache.block_table),
        _ptr(cache.ctx_lens), _ptr(q), _ptr(out), _ptr(lse), _ptr(workspace), nbytes, num_splits,
        max_ctx, _ptr(cache.error_flag), _stream(stream)))
