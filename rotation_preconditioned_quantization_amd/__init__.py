"""Python binding of liboctox.so, the OCTOPUS key-codec library for MI355X.

Argument marshalling only: every step of the codec runs in the HIP kernels
behind the C ABI declared in include/octo.h.  The functions below carry the
same names as the C entry points; torch tensors are used only as device
memory and torch's current stream as the launch stream.  The library must be
built first (``python -m rotation_preconditioned_quantization_amd.build``);
importing works without it, but every call then raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboctox.so")

OCTO_OK, OCTO_ERR_INVALID_ARG, OCTO_ERR_UNSUPPORTED, OCTO_ERR_HIP, OCTO_ERR_NOMEM, OCTO_ERR_WORKSPACE = range(6)
OCTO_F32, OCTO_BF16, OCTO_F16 = 0, 1, 2
STAGE_ROTATE, STAGE_MAIN, STAGE_COMBINE, STAGE_ALL = 1, 2, 4, 7
TILE = 64


class OctoError(RuntimeError):
    def __init__(self, status: int, what: str, msg: str):
        super().__init__(f"{what}: status {status} ({msg})")
        self.status = status


class octo_params(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int), ("b", ctypes.c_int), ("seed", ctypes.c_uint64),
                ("cb_seed", ctypes.c_uint64), ("b_xi", ctypes.c_int), ("b_eta", ctypes.c_int),
                ("b_rho", ctypes.c_int), ("qjl", ctypes.c_int), ("mc_vectors", ctypes.c_int),
                ("device", ctypes.c_int)]


class octo_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int) for n in (
        "d", "n_triplets", "pad_dim", "b_xi", "b_eta", "b_rho", "bits_per_triplet",
        "bits_per_key", "words_per_key", "tile_keys", "qjl", "qjl_words_per_key")] + \
        [("packed_bytes_per_key_alloc", ctypes.c_size_t)]


class octo_lds_copy(ctypes.Structure):
    _fields_ = [("kernel", ctypes.c_char_p), ("d", ctypes.c_int), ("b", ctypes.c_int),
                ("qjl", ctypes.c_int), ("table", ctypes.c_int), ("lds_slots", ctypes.c_int64),
                ("slots_written", ctypes.c_int64), ("entries_read", ctypes.c_int64),
                ("copied", ctypes.c_int64), ("threads", ctypes.c_int), ("masked", ctypes.c_int)]


TABLES = ("dir", "trip", "rho", "qx", "qe", "qr2", "s16")   # octo_table order

_lib = None

_P, _I, _I64, _SZ, _F = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float
_SIGS = {
    "octo_codebook_build": (_I, [ctypes.POINTER(octo_params), ctypes.POINTER(_P)]),
    "octo_codebook_free": (_I, [_P]),
    "octo_codebook_layout": (_I, [_P, ctypes.POINTER(octo_layout)]),
    "octo_codebook_export": (_I, [_P, _P, _P, _P, _P, _P]),
    "octo_packed_bytes": (_SZ, [_P, _I64, _I64]),
    "octo_qjl_bits_bytes": (_SZ, [_P, _I64, _I64]),
    "octo_encode": (_I, [_P, _P, _I, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "octo_encode_joint": (_I, [_P, _P, _I, _I64, _I64, _I64, _I64, _I64, _I64, _P, _P, _P, _P, _P]),
    "octo_decode_attn_append": (_I, [_P, _P, _I, _I64, _P, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I,
                                     _I64, _I64, _F, _P, _P, _SZ, _P]),
    "octo_decode_workspace_bytes": (_SZ, [_P, _I, _I, _I, _I, _I, _I64]),
    "octo_decode_logits": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _I64, _I64, _P, _P, _SZ, _P]),
    "octo_decode_attn": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _I64, _I64, _F,
                              _P, _P, _SZ, _P]),
    "octo_decode_attn_static": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _I64, _I64, _F,
                                     _P, _P]),
    "octo_decode_logits_stages": (_I, [_P, _P, _I, _I, _I, _I, _P, _P, _P, _P, _I64, _I64, _P, _P, _SZ,
                                       _P, _I]),
    "octo_decode_attn_stages": (_I, [_P, _P, _I, _I, _I, _I, _I, _P, _P, _P, _P, _P, _I, _I64, _I64,
                                     _F, _P, _P, _SZ, _P, _I]),
    "octo_debug_reconstruct": (_I, [_P, _P, _P, _I64, _I64, _I64, _P, _P]),
    "octo_debug_copy": (_I, [_P, _P, _SZ, _P]),
    "octo_codebook_table_entries": (_I64, [_P, _I]),
    "octo_debug_lds_copy": (_I, [_I, _P]),
    "octo_debug_bucket_index": (_I, [_P, _I, _P, _I64, _P]),
    "octo_status_str": (ctypes.c_char_p, [_I]),
    "octo_last_error": (ctypes.c_char_p, []),
}


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run "
                               "`python -m rotation_preconditioned_quantization_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return sorted(_SIGS)


def _check(status: int, what: str):
    if status != OCTO_OK:
        raise OctoError(status, what, lib().octo_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _dtype_code(t):
    import torch
    return {torch.float32: OCTO_F32, torch.bfloat16: OCTO_BF16, torch.float16: OCTO_F16}[t.dtype]


def _stream(stream=None):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _need(cond: bool, msg: str):
    if not cond:
        raise ValueError(msg)


def _need_cuda(**tensors):
    """Checked last, after the shapes: every tensor a kernel reads or writes
    must be device memory (the C ABI receives bare pointers)."""
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise ValueError(f"{name} must be a CUDA tensor")


def _need_dtype(t, name: str):
    import torch
    _need(t.dtype in (torch.float32, torch.bfloat16, torch.float16),
          f"{name} must be float32, bfloat16 or float16, not {t.dtype}")


def _need_out(t, shape, name: str):
    import torch
    _need(tuple(t.shape) == tuple(shape), f"{name} must have shape {tuple(shape)}, not {tuple(t.shape)}")
    _need(t.dtype == torch.float32 and t.is_contiguous(), f"{name} must be contiguous float32")


def _need_cache(cb, cache, n_seq: int, what: str):
    _need(cache.cb is cb or cache.packed.numel() == cb.packed_words(cache.n_seq, cache.cap),
          "the cache was laid out for another codebook")
    _need(n_seq == cache.n_seq, f"{what} ({n_seq}) must equal cache.n_seq ({cache.n_seq})")


@dataclass
class Layout:
    d: int
    n_triplets: int
    pad_dim: int
    b_xi: int
    b_eta: int
    b_rho: int
    bits_per_triplet: int
    bits_per_key: int
    words_per_key: int
    tile_keys: int
    qjl: int
    qjl_words_per_key: int


class Codebook:
    """Owns an octo_codebook handle (octo_codebook_build / octo_codebook_free)."""

    def __init__(self, d: int, b: int, seed: int = 0, cb_seed: int = 0, alloc=None,
                 qjl: bool = False, mc_vectors: int = 0, device: int | None = 0):
        p = octo_params()
        p.d, p.b, p.seed, p.cb_seed = d, b, seed, cb_seed
        p.b_xi, p.b_eta, p.b_rho = alloc if alloc is not None else (-1, -1, -1)
        p.qjl, p.mc_vectors = int(bool(qjl)), mc_vectors
        p.device = -1 if device is None else device
        h = ctypes.c_void_p()
        _check(lib().octo_codebook_build(ctypes.byref(p), ctypes.byref(h)), "octo_codebook_build")
        self.handle = h
        lay = octo_layout()
        _check(lib().octo_codebook_layout(h, ctypes.byref(lay)), "octo_codebook_layout")
        self.layout = Layout(*[getattr(lay, f) for f, _ in octo_layout._fields_[:-1]])
        self.d, self.b, self.seed, self.cb_seed, self.qjl = d, b, seed, cb_seed, bool(qjl)

    def close(self):
        if getattr(self, "handle", None) is not None:
            lib().octo_codebook_free(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def export(self):
        """Host copies of the tables: (c_xi, c_eta, c_rho, signs, S or None) as numpy."""
        import numpy as np
        lay = self.layout
        cx = np.zeros(1 << lay.b_xi)
        ce = np.zeros(1 << lay.b_eta)
        cr = np.zeros(1 << lay.b_rho)
        sg = np.zeros(self.d, dtype=np.int8)
        S = np.zeros((self.d, self.d), dtype=np.float32) if self.qjl else None
        _check(lib().octo_codebook_export(self.handle, cx.ctypes.data, ce.ctypes.data, cr.ctypes.data,
                                          sg.ctypes.data, S.ctypes.data if S is not None else None),
               "octo_codebook_export")
        return cx, ce, cr, sg, S

    def table_entries(self, table: int) -> int:
        """Entries of codebook table `table` (index into TABLES)."""
        return lib().octo_codebook_table_entries(self.handle, table)

    # sizes ---------------------------------------------------------------
    def packed_words(self, n_seq: int, cap: int) -> int:
        return lib().octo_packed_bytes(self.handle, n_seq, cap) // 4

    def qjl_words(self, n_seq: int, cap: int) -> int:
        return lib().octo_qjl_bits_bytes(self.handle, n_seq, cap) // 4

    def workspace_bytes(self, mode: int, B: int, Hq: int, Hkv: int, n_q: int, n_keys: int) -> int:
        return lib().octo_decode_workspace_bytes(self.handle, mode, B, Hq, Hkv, n_q, n_keys)


class Cache:
    """Caller-owned device buffers of one compressed K cache (torch tensors)."""

    def __init__(self, cb: Codebook, n_seq: int, cap: int, device="cuda", qjl: bool | None = None):
        import torch
        if cap % TILE:
            raise ValueError("cap must be a multiple of 64")
        self.cb, self.n_seq, self.cap = cb, n_seq, cap
        self.packed = torch.zeros(cb.packed_words(n_seq, cap), dtype=torch.int32, device=device)
        self.gamma = torch.zeros(n_seq * cap, dtype=torch.float32, device=device)
        use_qjl = cb.qjl if qjl is None else qjl
        self.qjl_bits = (torch.zeros(cb.qjl_words(n_seq, cap), dtype=torch.int32, device=device)
                         if use_qjl else None)
        self.qjl_norm = (torch.zeros(n_seq * cap, dtype=torch.int16, device=device)
                         if use_qjl else None)


def _encode(fn, name, cb: Codebook, keys, cache: Cache, pos0: int, stream):
    _need(keys.dim() == 3, "keys must be [n_seq, n_new, d]")
    n_seq, n_new, d = keys.shape
    _need(d == cb.d and keys.stride(2) == 1, "keys must be [n_seq, n_new, d] with a contiguous last dim")
    _need_dtype(keys, "keys")
    _need_cache(cb, cache, n_seq, "keys.shape[0]")
    _need(0 <= pos0 and pos0 + n_new <= cache.cap,
          f"positions {pos0}..{pos0 + n_new - 1} exceed the cache capacity {cache.cap}")
    _need_cuda(keys=keys, packed=cache.packed, gamma=cache.gamma, qjl_bits=cache.qjl_bits,
               qjl_norm=cache.qjl_norm)
    _check(fn(cb.handle, _ptr(keys), _dtype_code(keys), n_seq, n_new, keys.stride(0),
              keys.stride(1), pos0, cache.cap, _ptr(cache.packed), _ptr(cache.gamma),
              _ptr(cache.qjl_bits), _ptr(cache.qjl_norm), _stream(stream)), name)


def octo_encode(cb: Codebook, keys, cache: Cache, pos0: int = 0, stream=None):
    """keys: device tensor [n_seq, n_new, d] (f32/bf16/f16, last dim contiguous)."""
    _encode(lib().octo_encode, "octo_encode", cb, keys, cache, pos0, stream)


def octo_encode_joint(cb: Codebook, keys, cache: Cache, pos0: int = 0, stream=None):
    """octo_encode with joint 3x3 rounding of every triplet."""
    _encode(lib().octo_encode_joint, "octo_encode_joint", cb, keys, cache, pos0, stream)


def _workspace(cb, mode, B, Hq, Hkv, n_q, n_keys, workspace, device):
    import torch
    need = cb.workspace_bytes(mode, B, Hq, Hkv, n_q, n_keys)
    if workspace is None:
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=device)
    _need(workspace.dtype == torch.uint8 and workspace.is_contiguous(),
          "workspace must be a contiguous uint8 tensor")
    _need(workspace.numel() >= need, f"workspace holds {workspace.numel()} bytes, {need} needed")
    return workspace, need


def _need_decode(cb, q, cache, B, Hq, Hkv, n_keys, qjl):
    _need(q.shape[-1] == cb.d, f"q's last dim ({q.shape[-1]}) must be the head dim {cb.d}")
    _need_dtype(q, "q")
    _need(q.is_contiguous(), "q must be contiguous")
    _need(Hkv > 0 and Hq % Hkv == 0, f"Hq ({Hq}) must be a multiple of Hkv ({Hkv})")
    _need_cache(cb, cache, B * Hkv, "B * Hkv")
    _need(0 <= n_keys <= cache.cap, f"n_keys ({n_keys}) must lie in [0, cache.cap = {cache.cap}]")
    if qjl:
        _need(cb.qjl and cache.qjl_bits is not None and cache.qjl_norm is not None,
              "the QJL term needs a QJL codebook and a cache with QJL buffers")


def _need_values(v, cache, d):
    import torch
    _need(v is not None and tuple(v.shape) == (cache.n_seq, cache.cap, d),
          f"v must have shape (n_seq, cap, d) = {(cache.n_seq, cache.cap, d)}")
    _need(v.dtype == torch.bfloat16 and v.is_contiguous(), "v must be contiguous bfloat16")


def octo_decode_logits(cb: Codebook, q, cache: Cache, n_keys: int, Hkv: int, logits=None,
                       workspace=None, use_qjl: bool | None = None, stream=None,
                       stages: int = STAGE_ALL):
    """q: [B, Hq, d]; returns fp32 logits [B, Hq, n_keys] (raw <q, k^>)."""
    import torch
    _need(q.dim() == 3, "q must be [B, Hq, d]")
    B, Hq, d = q.shape
    qjl = cache.qjl_bits is not None if use_qjl is None else use_qjl
    _need_decode(cb, q, cache, B, Hq, Hkv, n_keys, qjl)
    if logits is None:
        logits = torch.empty((B, Hq, n_keys), dtype=torch.float32, device=q.device)
    _need_out(logits, (B, Hq, n_keys), "logits")
    workspace, _ = _workspace(cb, 0, B, Hq, Hkv, 1, n_keys, workspace, q.device)
    _need_cuda(q=q, logits=logits, packed=cache.packed, workspace=workspace)
    _check(lib().octo_decode_logits_stages(cb.handle, _ptr(q), _dtype_code(q), B, Hq, Hkv,
                                           _ptr(cache.packed), _ptr(cache.gamma),
                                           _ptr(cache.qjl_bits) if qjl else None,
                                           _ptr(cache.qjl_norm) if qjl else None, n_keys, cache.cap,
                                           _ptr(logits), _ptr(workspace), workspace.numel(),
                                           _stream(stream), stages),
           "octo_decode_logits")
    return logits


def octo_decode_attn(cb: Codebook, q, cache: Cache, v, n_keys: int, Hkv: int, out=None,
                     scale: float = 0.0, workspace=None, use_qjl: bool | None = None, stream=None,
                     stages: int = STAGE_ALL):
    """q: [B, Hq, n_q, d]; v: [B*Hkv, cap, d] bf16; returns fp32 [B, Hq, n_q, d].

    ``stages`` selects a subset of the launches (octo_decode_attn_stages)."""
    import torch
    _need(q.dim() == 4, "q must be [B, Hq, n_q, d]")
    B, Hq, n_q, d = q.shape
    qjl = cache.qjl_bits is not None if use_qjl is None else use_qjl
    _need_decode(cb, q, cache, B, Hq, Hkv, n_keys, qjl)
    _need_values(v, cache, d)
    if out is None:
        out = torch.empty((B, Hq, n_q, d), dtype=torch.float32, device=q.device)
    _need_out(out, (B, Hq, n_q, d), "out")
    workspace, _ = _workspace(cb, 1, B, Hq, Hkv, n_q, n_keys, workspace, q.device)
    _need_cuda(q=q, v=v, out=out, packed=cache.packed, workspace=workspace)
    _check(lib().octo_decode_attn_stages(cb.handle, _ptr(q), _dtype_code(q), B, Hq, Hkv, n_q,
                                         _ptr(cache.packed), _ptr(cache.gamma),
                                         _ptr(cache.qjl_bits) if qjl else None,
                                         _ptr(cache.qjl_norm) if qjl else None, _ptr(v),
                                         _dtype_code(v), n_keys, cache.cap, scale, _ptr(out),
                                         _ptr(workspace), workspace.numel(), _stream(stream), stages),
           "octo_decode_attn")
    return out


def octo_decode_attn_static(cb: Codebook, q, cache: Cache, v, n_keys: int, Hkv: int, out=None,
                            scale: float = 0.0, use_qjl: bool | None = None, stream=None):
    """octo_decode_attn with the library's static device scratch instead of
    a workspace: allocates nothing on the device when `out` is given (calls
    on one GPU must not overlap in time)."""
    import torch
    _need(q.dim() == 4, "q must be [B, Hq, n_q, d]")
    B, Hq, n_q, d = q.shape
    qjl = cache.qjl_bits is not None if use_qjl is None else use_qjl
    _need_decode(cb, q, cache, B, Hq, Hkv, n_keys, qjl)
    _need_values(v, cache, d)
    if out is None:
        out = torch.empty((B, Hq, n_q, d), dtype=torch.float32, device=q.device)
    _need_out(out, (B, Hq, n_q, d), "out")
    _need_cuda(q=q, v=v, out=out, packed=cache.packed)
    _check(lib().octo_decode_attn_static(cb.handle, _ptr(q), _dtype_code(q), B, Hq, Hkv, n_q,
                                         _ptr(cache.packed), _ptr(cache.gamma),
                                         _ptr(cache.qjl_bits) if qjl else None,
                                         _ptr(cache.qjl_norm) if qjl else None, _ptr(v),
                                         _dtype_code(v), n_keys, cache.cap, scale, _ptr(out),
                                         _stream(stream)),
           "octo_decode_attn_static")
    return out


def octo_decode_attn_append(cb: Codebook, new_keys, q, cache: Cache, v, n_keys: int, Hkv: int,
                            out=None, scale: float = 0.0, workspace=None,
                            use_qjl: bool | None = None, stream=None):
    """One decode step: encode new_keys [B*Hkv, d] (or [B*Hkv, 1, d]) at cache
    position n_keys - 1, then attend q [B, Hq, 1, d] over the n_keys keys."""
    import torch
    _need(q.dim() == 4, "q must be [B, Hq, 1, d]")
    B, Hq, n_q, d = q.shape
    _need(n_q == 1, "one query token per head")
    qjl = cache.qjl_bits is not None if use_qjl is None else use_qjl
    _need_decode(cb, q, cache, B, Hq, Hkv, n_keys, qjl)
    _need(n_keys >= 1, "the step appends at position n_keys - 1: n_keys >= 1")
    _need(new_keys.numel() == B * Hkv * d and new_keys.shape[0] == B * Hkv and new_keys.shape[-1] == d,
          f"new_keys must be [B * Hkv, d] = [{B * Hkv}, {d}] (or [B * Hkv, 1, d])")
    _need_dtype(new_keys, "new_keys")
    nk = new_keys.reshape(new_keys.shape[0], d)
    _need(nk.stride(1) == 1, "new_keys must have a contiguous last dim")
    _need_values(v, cache, d)
    if out is None:
        out = torch.empty((B, Hq, 1, d), dtype=torch.float32, device=q.device)
    _need_out(out, (B, Hq, 1, d), "out")
    workspace, _ = _workspace(cb, 1, B, Hq, Hkv, 1, n_keys, workspace, q.device)
    _need_cuda(new_keys=nk, q=q, v=v, out=out, packed=cache.packed, workspace=workspace)
    _check(lib().octo_decode_attn_append(cb.handle, _ptr(nk), _dtype_code(nk), nk.stride(0),
                                         _ptr(q), _dtype_code(q), B, Hq, Hkv, _ptr(cache.packed),
                                         _ptr(cache.gamma), _ptr(cache.qjl_bits) if qjl else None,
                                         _ptr(cache.qjl_norm) if qjl else None, _ptr(v),
                                         _dtype_code(v), n_keys, cache.cap, scale, _ptr(out),
                                         _ptr(workspace), workspace.numel(), _stream(stream)),
           "octo_decode_attn_append")
    return out


def octo_debug_lds_copies():
    """Every copy of a codebook table into LDS by a kernel instantiation
    (octo_debug_lds_copy), as a list of dicts."""
    out, i = [], 0
    rec = octo_lds_copy()
    while lib().octo_debug_lds_copy(i, ctypes.byref(rec)) == OCTO_OK:
        out.append({f: getattr(rec, f) for f, _ in octo_lds_copy._fields_})
        out[-1]["kernel"] = rec.kernel.decode()
        i += 1
    return out


def octo_debug_bucket_index(cb: Codebook, table: int, x):
    """The encoder kernels' nearest-centroid index of each value of x for xi
    (table TABLES.index("qx")) or eta ("qe"), by their own lookup formula on
    the host (octo_debug_bucket_index); numpy float32 in, uint32 out."""
    import numpy as np
    xs = np.ascontiguousarray(x, dtype=np.float32)
    out = np.zeros(xs.shape, dtype=np.uint32)
    _check(lib().octo_debug_bucket_index(cb.handle, table, xs.ctypes.data, xs.size, out.ctypes.data),
           "octo_debug_bucket_index")
    return out


def octo_debug_copy(dst, src, stream=None):
    """Plain 16-byte-access device copy of src into dst (same byte size)."""
    nbytes = src.numel() * src.element_size()
    _need(dst.numel() * dst.element_size() == nbytes, "dst and src differ in size")
    _need(src.is_contiguous() and dst.is_contiguous(), "dst and src must be contiguous")
    _need_cuda(dst=dst, src=src)
    _check(lib().octo_debug_copy(_ptr(dst), _ptr(src), nbytes, _stream(stream)), "octo_debug_copy")


def octo_debug_reconstruct(cb: Codebook, cache: Cache, n_keys: int, out=None, stream=None):
    import torch
    _need_cache(cb, cache, cache.n_seq, "cache.n_seq")
    _need(0 <= n_keys <= cache.cap, f"n_keys ({n_keys}) must lie in [0, cache.cap = {cache.cap}]")
    if out is None:
        out = torch.empty((cache.n_seq, n_keys, cb.d), dtype=torch.float32, device=cache.packed.device)
    _need_out(out, (cache.n_seq, n_keys, cb.d), "out")
    _need_cuda(out=out, packed=cache.packed)
    _check(lib().octo_debug_reconstruct(cb.handle, _ptr(cache.packed), _ptr(cache.gamma), cache.n_seq,
                                        n_keys, cache.cap, _ptr(out), _stream(stream)),
           "octo_debug_reconstruct")
    return out

