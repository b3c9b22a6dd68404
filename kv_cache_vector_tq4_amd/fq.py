"""Python binding of libfq (ctypes): argument marshalling only.

Every step of the method runs inside libfq (host builder or HIP kernels).
PyTorch supplies device memory and the stream. The binding refuses to run
without the built library: there is no fallback path.
"""
import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfq.so")

FQ_OK, FQ_ERR_INVALID_ARG, FQ_ERR_UNSUPPORTED, FQ_ERR_WORKSPACE, FQ_ERR_HIP, FQ_ERR_SCRATCH = range(6)
ROT_HAAR, ROT_WHT = 0, 1
F32, BF16 = 0, 1
CB_GAUSSIAN, CB_SPHERE = 0, 1
BLOCK = 16

_lib = None


class FQError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s failed: %s" % (what, status_string(status)))


class QuantizerT(ctypes.Structure):
    _fields_ = [
        ("bits", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("rotation", ctypes.c_int32),
        ("qjl_dim", ctypes.c_int32),
        ("levels", ctypes.c_void_p),
        ("boundaries", ctypes.c_void_p),
        ("rotation_matrix", ctypes.c_void_p),
        ("rotation_t", ctypes.c_void_p),
        ("wht_signs", ctypes.c_void_p),
        ("qjl_matrix", ctypes.c_void_p),
        ("qjl_matrix_t", ctypes.c_void_p),
        ("mfma_operands", ctypes.c_void_p),
        ("key_bits", ctypes.c_int32),
        ("key_levels", ctypes.c_void_p),
        ("key_boundaries", ctypes.c_void_p),
    ]


MFMA_OPERAND_BYTES = 131072


class CacheT(ctypes.Structure):
    _fields_ = [
        ("num_blocks", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("bits", ctypes.c_int32),
        ("qjl_dim", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p),
        ("k_norm", ctypes.c_void_p),
        ("k_qjl", ctypes.c_void_p),
        ("k_gamma", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("v_norm", ctypes.c_void_p),
        ("key_bits", ctypes.c_int32),
    ]


EXPORTS = {
    "fq_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "fq_version": (ctypes.c_int, []),
    "fq_build_codebook": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_uint64,
                                         ctypes.c_uint64, ctypes.c_int] + [ctypes.c_void_p] * 7),
    "fq_build_levels": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]),
    "fq_window_workspace_size": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)]),
    "fq_prefill_attention": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT), ctypes.POINTER(CacheT),
                                            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                            ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                            ctypes.c_size_t, ctypes.c_void_p]),
    "fq_window_append": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT), ctypes.POINTER(CacheT),
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t]),
    "fq_decode_attention_window": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT),
                                                  ctypes.POINTER(CacheT), ctypes.c_void_p, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                                  ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                                  ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                                  ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                                  ctypes.c_void_p]),
    "fq_decode_step_window": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT), ctypes.POINTER(CacheT),
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                             ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                             ctypes.c_size_t, ctypes.c_void_p]),
    "fq_compress": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT), ctypes.POINTER(CacheT),
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                   ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p]),
    "fq_pack_mfma_operands": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                             ctypes.c_size_t]),
    "fq_decode_auto_splits": (ctypes.c_int, [ctypes.c_int, ctypes.c_int, ctypes.c_int]),
    "fq_decode_attention_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT),
                                                   ctypes.POINTER(CacheT), ctypes.c_void_p, ctypes.c_int,
                                                   ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                                   ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                                   ctypes.c_void_p]),
    "fq_validate_indices": (ctypes.c_int, [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int64)]),
    "fq_decode_workspace_size": (ctypes.c_int, [ctypes.c_int] * 7 + [ctypes.POINTER(ctypes.c_size_t)]),
    "fq_decode_attention": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT), ctypes.POINTER(CacheT),
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t,
                                           ctypes.c_void_p]),
    "fq_decode_step": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT), ctypes.POINTER(CacheT),
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                      ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "fq_decompress": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT), ctypes.POINTER(CacheT),
                                     ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_int64, ctypes.c_int64]),
    "fq_step_prepare": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT), ctypes.POINTER(CacheT),
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_float,
                                       ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p]),
    "fq_step_attend": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(QuantizerT), ctypes.POINTER(CacheT),
                                      ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_float, ctypes.c_void_p,
                                      ctypes.c_size_t, ctypes.c_void_p]),
}


def lib():
    """The loaded libfq; raises if the HIP library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfq.so is not built (run `python -m kv_cache_vector_tq4_amd.build`)")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _lib = h
    return _lib


def status_string(status):
    return lib().fq_status_string(int(status)).decode()


def _check(status, what):
    if status != FQ_OK:
        raise FQError(status, what)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch

    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def build_codebook(bits=4, head_dim=128, rotation=ROT_HAAR, rot_seed=1, qjl_seed=2, qjl_dim=128):
    """Host arrays of one layer's quantizer, built by libfq (fq_build_codebook)."""
    L = 1 << bits
    out = {
        "levels": np.zeros(L, np.float32),
        "boundaries": np.zeros(L - 1, np.float32),
        "rotation_matrix": np.zeros((head_dim, head_dim), np.float32),
        "rotation_t": np.zeros((head_dim, head_dim), np.float32),
        "wht_signs": np.zeros(head_dim, np.float32),
        "qjl_matrix": np.zeros((max(qjl_dim, 1), head_dim), np.float32),
        "qjl_matrix_t": np.zeros((head_dim, max(qjl_dim, 1)), np.float32),
    }
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    st = lib().fq_build_codebook(bits, head_dim, rotation, rot_seed, qjl_seed, qjl_dim,
                                 p(out["levels"]), p(out["boundaries"]), p(out["rotation_matrix"]),
                                 p(out["rotation_t"]), p(out["wht_signs"]),
                                 p(out["qjl_matrix"]) if qjl_dim else None,
                                 p(out["qjl_matrix_t"]) if qjl_dim else None)
    _check(st, "fq_build_codebook")
    out.update(bits=bits, head_dim=head_dim, rotation=rotation, qjl_dim=qjl_dim)
    return out


def build_levels(bits=4, head_dim=128, kind=None):
    """Host (levels, boundaries) fp32 of a scalar codebook (fq_build_levels); kind
    CB_GAUSSIAN (default) or CB_SPHERE."""
    kind = CB_GAUSSIAN if kind is None else kind
    L = 1 << bits
    lev, bnd = np.zeros(L, np.float32), np.zeros(L - 1, np.float32)
    st = lib().fq_build_levels(bits, head_dim, kind, lev.ctypes.data_as(ctypes.c_void_p),
                               bnd.ctypes.data_as(ctypes.c_void_p))
    _check(st, "fq_build_levels")
    return lev, bnd


def pack_mfma_operands(rotation_matrix, qjl_matrix=None):
    """Host bytes of the prepared matrix-core operands (fq_pack_mfma_operands)."""
    out = np.zeros(MFMA_OPERAND_BYTES, np.uint8)
    r = np.ascontiguousarray(rotation_matrix, np.float32)
    sq = None if qjl_matrix is None else np.ascontiguousarray(qjl_matrix, np.float32)
    st = lib().fq_pack_mfma_operands(r.ctypes.data_as(ctypes.c_void_p),
                                     None if sq is None else sq.ctypes.data_as(ctypes.c_void_p),
                                     r.shape[0], out.ctypes.data_as(ctypes.c_void_p), out.nbytes)
    _check(st, "fq_pack_mfma_operands")
    return out


class Quantizer:
    """Device copy of a layer's quantizer parameters plus the C struct pointing at them.

    prepared=True also uploads the packed matrix-core operands (fq_pack_mfma_operands);
    with prepared=False the kernels derive them from the fp32 matrices themselves.
    codebook: CB_GAUSSIAN (fq_build_codebook's) or CB_SPHERE (fq_build_levels' exact
    spherical marginal, replacing the levels and boundaries).
    key_bits: width of the keys' MSE codes when it differs from bits (their codebook is
    then that width's); key_bits = bits - 1 with QJL keys is the Prod budget.
    """

    def __init__(self, bits=4, head_dim=128, rotation=ROT_HAAR, rot_seed=1, qjl_seed=2, qjl_dim=128,
                 device="cuda", prepared=True, codebook=CB_GAUSSIAN, key_bits=None):
        import torch

        self.host = build_codebook(bits, head_dim, rotation, rot_seed, qjl_seed, qjl_dim)
        if codebook != CB_GAUSSIAN:
            self.host["levels"], self.host["boundaries"] = build_levels(bits, head_dim, codebook)
        self.key_bits = bits if key_bits is None else key_bits
        if self.key_bits != bits:
            self.host["key_levels"], self.host["key_boundaries"] = build_levels(self.key_bits, head_dim, codebook)
        self.bits, self.head_dim, self.rotation, self.qjl_dim = bits, head_dim, rotation, qjl_dim
        self.codebook = codebook
        keys = ("levels", "boundaries", "rotation_matrix", "rotation_t", "wht_signs", "qjl_matrix",
                "qjl_matrix_t") + (("key_levels", "key_boundaries") if self.key_bits != bits else ())
        self.dev = {k: torch.from_numpy(np.ascontiguousarray(self.host[k])).to(device) for k in keys}
        if prepared:
            ops = pack_mfma_operands(self.host["rotation_matrix"], self.host["qjl_matrix"] if qjl_dim else None)
            self.dev["mfma_operands"] = torch.from_numpy(ops).to(device)
        d = self.dev
        self.struct = QuantizerT(bits, head_dim, rotation, qjl_dim, d["levels"].data_ptr(),
                                 d["boundaries"].data_ptr(), d["rotation_matrix"].data_ptr(),
                                 d["rotation_t"].data_ptr(), d["wht_signs"].data_ptr(),
                                 d["qjl_matrix"].data_ptr() if qjl_dim else None,
                                 d["qjl_matrix_t"].data_ptr() if qjl_dim else None,
                                 d["mfma_operands"].data_ptr() if prepared else None,
                                 0 if self.key_bits == bits else self.key_bits,
                                 d["key_levels"].data_ptr() if self.key_bits != bits else None,
                                 d["key_boundaries"].data_ptr() if self.key_bits != bits else None)


class PagedCache:
    """A layer's paged compressed cache in device memory (torch tensors) plus its C struct."""

    def __init__(self, num_blocks, num_kv_heads, head_dim=128, bits=4, qjl_dim=128, device="cuda", key_bits=None):
        import torch

        cb = head_dim * bits // 8
        self.key_bits = bits if key_bits is None else key_bits
        self.num_blocks, self.num_kv_heads, self.head_dim = num_blocks, num_kv_heads, head_dim
        self.bits, self.qjl_dim = bits, qjl_dim
        z = lambda *shape, dt: torch.zeros(shape, dtype=dt, device=device)
        self.k_codes = z(num_blocks, num_kv_heads, BLOCK, head_dim * self.key_bits // 8, dt=torch.uint8)
        self.k_norm = z(num_blocks, num_kv_heads, BLOCK, dt=torch.float32)
        self.v_codes = z(num_blocks, num_kv_heads, BLOCK, cb, dt=torch.uint8)
        self.v_norm = z(num_blocks, num_kv_heads, BLOCK, dt=torch.float32)
        if qjl_dim:
            self.k_qjl = z(num_blocks, num_kv_heads, BLOCK, qjl_dim // 8, dt=torch.uint8)
            self.k_gamma = z(num_blocks, num_kv_heads, BLOCK, dt=torch.float32)
        else:
            self.k_qjl = self.k_gamma = None
        self.struct = CacheT(num_blocks, BLOCK, num_kv_heads, head_dim, bits, qjl_dim,
                             self.k_codes.data_ptr(), self.k_norm.data_ptr(),
                             self.k_qjl.data_ptr() if qjl_dim else None,
                             self.k_gamma.data_ptr() if qjl_dim else None,
                             self.v_codes.data_ptr(), self.v_norm.data_ptr(),
                             0 if self.key_bits == bits else self.key_bits)

    def fields(self):
        out = {"k_codes": self.k_codes, "k_norm": self.k_norm, "v_codes": self.v_codes, "v_norm": self.v_norm}
        if self.qjl_dim:
            out.update(k_qjl=self.k_qjl, k_gamma=self.k_gamma)
        return out

    def bytes_per_token_head(self):
        cb = self.head_dim * self.bits // 8
        kcb = self.head_dim * self.key_bits // 8
        return (kcb + 4) + (cb + 4) + ((self.qjl_dim // 8 + 4) if self.qjl_dim else 0)


def _dtype_code(t):
    import torch

    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("K/V/q must be float32 or bfloat16, got %s" % t.dtype)


def compress(quant, cache, k, v, slot_mapping, debug=False, stream=None):
    """fq_compress: K, V [T, Hkv, d] (innermost contiguous), slot_mapping int64 [T].

    Returns (debug_y [2, T, Hkv, d], debug_p [T, Hkv, m]) when debug, else None.
    """
    import torch

    src = k if k is not None else v
    T = src.shape[0]
    for x in (k, v):
        if x is not None:
            assert x.shape[1:] == (cache.num_kv_heads, cache.head_dim) and x.stride(2) == 1
            assert x.dtype == src.dtype and x.stride() == src.stride()
    assert slot_mapping.dtype == torch.int64 and slot_mapping.numel() == T and slot_mapping.is_contiguous()
    dy = dp = None
    if debug:
        dy = torch.zeros((2, T, cache.num_kv_heads, cache.head_dim), dtype=torch.float32, device=src.device)
        dp = torch.zeros((T, cache.num_kv_heads, max(quant.qjl_dim, 1)), dtype=torch.float32, device=src.device)
    st = lib().fq_compress(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct),
                           _ptr(k), _ptr(v), _dtype_code(src), T, src.stride(0), src.stride(1),
                           _ptr(slot_mapping), _ptr(dy), _ptr(dp))
    _check(st, "fq_compress")
    return (dy, dp) if debug else None


def _host_array(x, dtype):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray(x, dtype=dtype)


def validate_indices(num_blocks, slot_mapping=None, block_tables=None, seq_lens=None, max_seq_len=None):
    """fq_validate_indices on host copies of a slot mapping and / or block tables with their
    lengths. Returns None when every index is in range; raises FQError (with .what and
    .where: 1 slot, 2 length, 3 table entry, and its flat index) otherwise."""
    sm = _host_array(slot_mapping, np.int64)
    bt = _host_array(block_tables, np.int32)
    sl = _host_array(seq_lens, np.int32)
    p = lambda a: None if a is None else a.ctypes.data_as(ctypes.c_void_p)
    batch = 0 if bt is None else bt.shape[0]
    width = 0 if bt is None else bt.shape[1]
    if max_seq_len is None:
        max_seq_len = 0 if sl is None or sl.size == 0 else int(sl.max())
    what, where = ctypes.c_int(0), ctypes.c_int64(0)
    st = lib().fq_validate_indices(int(num_blocks), p(sm), 0 if sm is None else sm.size, p(bt), batch, width,
                                   p(sl), int(max_seq_len), ctypes.byref(what), ctypes.byref(where))
    if st != FQ_OK:
        err = FQError(st, "fq_validate_indices")
        err.what, err.where = what.value, where.value
        raise err


def auto_splits(batch, num_kv_heads, max_seq_len):
    return int(lib().fq_decode_auto_splits(batch, num_kv_heads, max_seq_len))


def workspace_bytes(batch, num_q_heads, num_kv_heads, head_dim, qjl_dim, max_seq_len, num_splits=0):
    n = ctypes.c_size_t(0)
    st = lib().fq_decode_workspace_size(batch, num_q_heads, num_kv_heads, head_dim, qjl_dim, max_seq_len,
                                        num_splits, ctypes.byref(n))
    _check(st, "fq_decode_workspace_size")
    return int(n.value)


def decode(quant, cache, q, block_tables, seq_lens, max_seq_len, num_splits=0, scale=None, workspace=None,
           out=None, stream=None):
    """fq_decode_attention: q [B, Hq, d] -> out fp32 [B, Hq, d]."""
    import torch

    B, Hq, d = q.shape
    assert q.is_contiguous() and block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_tables.is_contiguous() and seq_lens.is_contiguous()
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    need = workspace_bytes(B, Hq, cache.num_kv_heads, d, quant.qjl_dim, max_seq_len, num_splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    st = lib().fq_decode_attention(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct),
                                   _ptr(q), _dtype_code(q), B, Hq, _ptr(block_tables), block_tables.shape[1],
                                   _ptr(seq_lens), int(max_seq_len), int(num_splits), float(scale),
                                   _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out))
    _check(st, "fq_decode_attention")
    return out


STATIC_SCRATCH_BYTES = 8 << 20


def decode_noalloc(quant, cache, q, block_tables, seq_lens, max_seq_len, out, num_splits=0, scale=None,
                   stream=None):
    """fq_decode_attention_noalloc: fq_decode_attention with the library's static scratch as its
    workspace; the caller passes the output (fp32 [B, Hq, d]); nothing is allocated."""
    B, Hq, d = q.shape
    assert q.is_contiguous() and block_tables.is_contiguous() and seq_lens.is_contiguous()
    assert out.shape == (B, Hq, d) and out.is_contiguous()
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    st = lib().fq_decode_attention_noalloc(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct),
                                           _ptr(q), _dtype_code(q), B, Hq, _ptr(block_tables), block_tables.shape[1],
                                           _ptr(seq_lens), int(max_seq_len), int(num_splits), float(scale), _ptr(out))
    _check(st, "fq_decode_attention_noalloc")
    return out


def decode_window(quant, cache, q, block_tables, seq_lens, max_seq_len, win_k, win_v, win_lens, num_splits=0,
                  scale=None, workspace=None, out=None, stream=None):
    """fq_decode_attention_window: decode over the compressed tokens [0, seq_lens[b]) and the
    window ring win_k / win_v (bf16 [B, W, Hkv, d]) slots < win_lens[b] (int32 [B])."""
    import torch

    B, Hq, d = q.shape
    assert q.is_contiguous() and block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_tables.is_contiguous() and seq_lens.is_contiguous()
    for x in (win_k, win_v):
        assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape == win_k.shape
        assert x.shape[0] == B and x.shape[2:] == (cache.num_kv_heads, d)
    assert win_lens.dtype == torch.int32 and win_lens.is_contiguous() and win_lens.numel() == B
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    need = workspace_bytes(B, Hq, cache.num_kv_heads, d, quant.qjl_dim, max_seq_len, num_splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    st = lib().fq_decode_attention_window(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct),
                                          _ptr(q), _dtype_code(q), B, Hq, _ptr(block_tables), block_tables.shape[1],
                                          _ptr(seq_lens), int(max_seq_len), int(num_splits), float(scale),
                                          _ptr(workspace), workspace.numel() * workspace.element_size(),
                                          _ptr(win_k), _ptr(win_v), win_k.shape[1], _ptr(win_lens), _ptr(out))
    _check(st, "fq_decode_attention_window")
    return out


def prefill(quant, cache, q, q_seq, q_lens, block_tables, max_seq_len, num_splits=0, scale=None, workspace=None,
            out=None, stream=None):
    """fq_prefill_attention: query tokens q [T, Hq, d] of sequences q_seq [T] (int32) attend to
    their sequence's cached tokens [0, q_lens[t]) -> out fp32 [T, Hq, d]."""
    import torch

    T, Hq, d = q.shape
    assert q.is_contiguous() and block_tables.dtype == torch.int32 and block_tables.is_contiguous()
    for x in (q_seq, q_lens):
        assert x.dtype == torch.int32 and x.is_contiguous() and x.numel() == T
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    need = workspace_bytes(T, Hq, cache.num_kv_heads, d, quant.qjl_dim, max_seq_len, num_splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((T, Hq, d), dtype=torch.float32, device=q.device)
    st = lib().fq_prefill_attention(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct),
                                    _ptr(q), _dtype_code(q), T, Hq, _ptr(q_seq), _ptr(q_lens), _ptr(block_tables),
                                    block_tables.shape[1], int(max_seq_len), int(num_splits), float(scale),
                                    _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out))
    _check(st, "fq_prefill_attention")
    return out


def window_append(quant, cache, k_new, v_new, positions, evict_slots, win_k, win_v, workspace=None, stream=None):
    """fq_window_append: k_new / v_new [B, Hkv, d] (contiguous, bf16 or fp32) into ring slot
    positions[b] % W of win_k / win_v (bf16 [B, W, Hkv, d]) after compressing the token there
    into the cache at evict_slots[b] (int64 [B]; < 0 drops it)."""
    import torch

    B = k_new.shape[0]
    for x in (k_new, v_new):
        assert x.is_contiguous() and x.shape == (B, cache.num_kv_heads, cache.head_dim) and x.dtype == k_new.dtype
    for x in (positions, evict_slots):
        assert x.dtype == torch.int64 and x.is_contiguous() and x.numel() == B
    for x in (win_k, win_v):
        assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape == win_k.shape and x.shape[0] == B
    need = ctypes.c_size_t(0)
    _check(lib().fq_window_workspace_size(B, cache.num_kv_heads, ctypes.byref(need)), "fq_window_workspace_size")
    if workspace is None:
        workspace = torch.empty(max(need.value, 1), dtype=torch.uint8, device=k_new.device)
    st = lib().fq_window_append(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct),
                                _ptr(k_new), _ptr(v_new), _dtype_code(k_new), B, _ptr(positions),
                                _ptr(evict_slots), _ptr(win_k), _ptr(win_v), win_k.shape[1], _ptr(workspace),
                                workspace.numel() * workspace.element_size())
    _check(st, "fq_window_append")


def decode_step_window(quant, cache, k_new, v_new, positions, evict_slots, win_k, win_v, win_lens, q, block_tables,
                       seq_lens, max_seq_len, num_splits=0, scale=None, workspace=None, out=None, stream=None):
    """fq_decode_step_window: window_append(k_new, v_new, positions, evict_slots, win_k, win_v)
    then decode_window(q, ...) over the updated cache and ring, as one call (seq_lens and
    win_lens (int32 [B]) describe the state after the append)."""
    import torch

    B, Hq, d = q.shape
    assert q.is_contiguous() and block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_tables.is_contiguous() and seq_lens.is_contiguous()
    for x in (k_new, v_new):
        assert x.is_contiguous() and x.shape == (B, cache.num_kv_heads, d) and x.dtype == k_new.dtype
    for x in (positions, evict_slots):
        assert x.dtype == torch.int64 and x.is_contiguous() and x.numel() == B
    for x in (win_k, win_v):
        assert x.dtype == torch.bfloat16 and x.is_contiguous() and x.shape == win_k.shape
        assert x.shape[0] == B and x.shape[2:] == (cache.num_kv_heads, d)
    assert win_lens.dtype == torch.int32 and win_lens.is_contiguous() and win_lens.numel() == B
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    need = workspace_bytes(B, Hq, cache.num_kv_heads, d, quant.qjl_dim, max_seq_len, num_splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    st = lib().fq_decode_step_window(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct),
                                     _ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(positions),
                                     _ptr(evict_slots), _ptr(win_k), _ptr(win_v), win_k.shape[1], _ptr(win_lens),
                                     _ptr(q), _dtype_code(q), B, Hq, _ptr(block_tables), block_tables.shape[1],
                                     _ptr(seq_lens), int(max_seq_len), int(num_splits), float(scale),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(), _ptr(out))
    _check(st, "fq_decode_step_window")
    return out


def decode_step(quant, cache, k_new, v_new, slot_mapping, q, block_tables, seq_lens, max_seq_len, num_splits=0,
                scale=None, workspace=None, out=None, debug=False, stream=None):
    """fq_decode_step: compress k_new / v_new [B, Hkv, d] into slot_mapping [B], then decode q [B, Hq, d].

    Returns out fp32 [B, Hq, d], or (out, debug_y [2, B, Hkv, d], debug_p [B, Hkv, m]) when debug.
    """
    import torch

    B, Hq, d = q.shape
    assert q.is_contiguous() and block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_tables.is_contiguous() and seq_lens.is_contiguous()
    for x in (k_new, v_new):
        assert x.shape == (B, cache.num_kv_heads, d) and x.stride(2) == 1
        assert x.dtype == k_new.dtype and x.stride() == k_new.stride()
    assert slot_mapping.dtype == torch.int64 and slot_mapping.numel() == B and slot_mapping.is_contiguous()
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    need = workspace_bytes(B, Hq, cache.num_kv_heads, d, quant.qjl_dim, max_seq_len, num_splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    dy = dp = None
    if debug:
        dy = torch.zeros((2, B, cache.num_kv_heads, d), dtype=torch.float32, device=q.device)
        dp = torch.zeros((B, cache.num_kv_heads, max(quant.qjl_dim, 1)), dtype=torch.float32, device=q.device)
    st = lib().fq_decode_step(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct),
                              _ptr(k_new), _ptr(v_new), _dtype_code(k_new), k_new.stride(0), k_new.stride(1),
                              _ptr(slot_mapping), _ptr(q), _dtype_code(q), B, Hq, _ptr(block_tables),
                              block_tables.shape[1], _ptr(seq_lens), int(max_seq_len), int(num_splits),
                              float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(),
                              _ptr(out), _ptr(dy), _ptr(dp))
    _check(st, "fq_decode_step")
    return (out, dy, dp) if debug else out


def step_prepare(quant, cache, k_new, v_new, slot_mapping, q, max_seq_len, workspace, num_splits=0, scale=None,
                 debug=False, stream=None):
    """fq_step_prepare: append k_new / v_new [B, Hkv, d] at slot_mapping [B] and prepare q [B, Hq, d] into
    workspace. Returns (debug_y, debug_p) when debug, else None."""
    import torch

    B, Hq, d = q.shape
    assert q.is_contiguous()
    for x in (k_new, v_new):
        assert x.shape == (B, cache.num_kv_heads, d) and x.stride(2) == 1
        assert x.dtype == k_new.dtype and x.stride() == k_new.stride()
    assert slot_mapping.dtype == torch.int64 and slot_mapping.numel() == B and slot_mapping.is_contiguous()
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    dy = dp = None
    if debug:
        dy = torch.zeros((2, B, cache.num_kv_heads, d), dtype=torch.float32, device=q.device)
        dp = torch.zeros((B, cache.num_kv_heads, max(quant.qjl_dim, 1)), dtype=torch.float32, device=q.device)
    st = lib().fq_step_prepare(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct),
                               _ptr(k_new), _ptr(v_new), _dtype_code(k_new), k_new.stride(0), k_new.stride(1),
                               _ptr(slot_mapping), _ptr(q), _dtype_code(q), B, Hq, int(max_seq_len),
                               int(num_splits), float(scale), _ptr(workspace),
                               workspace.numel() * workspace.element_size(), _ptr(dy), _ptr(dp))
    _check(st, "fq_step_prepare")
    return (dy, dp) if debug else None


def step_attend(quant, cache, batch, num_q_heads, block_tables, seq_lens, max_seq_len, workspace, num_splits=0,
                scale=None, out=None, stream=None):
    """fq_step_attend: the attention from a workspace prepared by step_prepare -> out fp32 [B, Hq, d]."""
    import torch

    d = cache.head_dim
    assert block_tables.dtype == torch.int32 and seq_lens.dtype == torch.int32
    assert block_tables.is_contiguous() and seq_lens.is_contiguous()
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty((batch, num_q_heads, d), dtype=torch.float32, device=block_tables.device)
    st = lib().fq_step_attend(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct), batch,
                              num_q_heads, _ptr(block_tables), block_tables.shape[1], _ptr(seq_lens),
                              int(max_seq_len), int(num_splits), float(scale), _ptr(workspace),
                              workspace.numel() * workspace.element_size(), _ptr(out))
    _check(st, "fq_step_attend")
    return out


def decompress(quant, cache, slot_mapping, dtype=None, k_out=None, v_out=None, which="kv", stream=None):
    """fq_decompress: the MSE reconstructions of the tokens at slot_mapping [T] as [T, Hkv, d] tensors.

    Returns (k_hat, v_hat); a side not in `which` is None. dtype: torch.float32 (default) or bfloat16.
    """
    import torch

    T = slot_mapping.numel()
    assert slot_mapping.dtype == torch.int64 and slot_mapping.is_contiguous()
    dtype = torch.float32 if dtype is None else dtype
    shape = (T, cache.num_kv_heads, cache.head_dim)
    if "k" in which and k_out is None:
        k_out = torch.empty(shape, dtype=dtype, device=slot_mapping.device)
    if "v" in which and v_out is None:
        v_out = torch.empty(shape, dtype=dtype, device=slot_mapping.device)
    ref = k_out if k_out is not None else v_out
    for x in (k_out, v_out):
        if x is not None:
            assert x.shape == shape and x.stride(2) == 1 and x.dtype == ref.dtype and x.stride() == ref.stride()
    st = lib().fq_decompress(_stream(stream), ctypes.byref(quant.struct), ctypes.byref(cache.struct),
                             _ptr(slot_mapping), T, _dtype_code(ref), _ptr(k_out), _ptr(v_out), ref.stride(0),
                             ref.stride(1))
    _check(st, "fq_decompress")
    return k_out, v_out
