"""CPU tests of the C-ABI library: it loads, exports every declared entry point,
its host-side builder matches the oracle, and argument checks return their
status codes without touching a device."""
import ctypes
import os
import re

import numpy as np
import pytest

from kv_cache_vector_tq4_amd import fq
from oracle import pipeline

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names |= set(re.findall(r"\b(fq_[a-z0-9_]+)\s*\(", text))
    return names


def test_library_exports_every_declared_symbol():
    lib = fq.lib()
    declared = _declared()
    assert {"fq_build_codebook", "fq_compress", "fq_decode_attention"} <= declared
    for name in declared:
        assert hasattr(lib, name), name
    assert set(fq.EXPORTS) == declared


def test_status_strings():
    assert fq.status_string(0) == "FQ_OK"
    assert fq.status_string(3) == "FQ_ERR_WORKSPACE"
    assert fq.status_string(99) == "FQ_ERR_UNKNOWN"


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("rot", [fq.ROT_HAAR, fq.ROT_WHT])
def test_builder_matches_oracle(bits, rot):
    lib_cb = fq.build_codebook(bits, 128, rot, rot_seed=11, qjl_seed=12, qjl_dim=128)
    ora = pipeline.build(bits, 128, rot=rot, rot_seed=11, qjl_seed=12)
    assert np.array_equal(lib_cb["levels"], ora["levels"])
    assert np.array_equal(lib_cb["boundaries"], ora["boundaries"])
    pi = lib_cb["rotation_matrix"].astype(np.float64)
    assert np.max(np.abs(pi - ora["pi"])) <= 1e-6
    assert np.array_equal(lib_cb["rotation_t"], lib_cb["rotation_matrix"].T)
    assert np.array_equal(lib_cb["qjl_matrix"].astype(np.float64), ora["s"])
    assert np.array_equal(lib_cb["qjl_matrix_t"], lib_cb["qjl_matrix"].T)
    if rot == fq.ROT_WHT:
        assert np.array_equal(lib_cb["wht_signs"].astype(np.float64), ora["signs"])
        assert np.array_equal(pi, ora["pi"])


def test_builder_haar_matches_oracle_bitwise_mostly():
    """Householder in C++ vs LAPACK: after rounding to fp32 nearly every entry is equal."""
    lib_cb = fq.build_codebook(4, 128, fq.ROT_HAAR, rot_seed=1, qjl_seed=2)
    ora = pipeline.build(4, 128)
    diff = lib_cb["rotation_matrix"] != ora["pi"].astype(np.float32)
    assert diff.mean() < 1e-3


def test_builder_errors():
    L = fq.lib()
    buf = np.zeros(128 * 128, np.float32)
    p = buf.ctypes.data_as(ctypes.c_void_p)
    assert L.fq_build_codebook(5, 128, 0, 1, 2, 128, p, p, None, None, None, None, None) == fq.FQ_ERR_UNSUPPORTED
    assert L.fq_build_codebook(1, 128, 0, 1, 2, 128, p, p, None, None, None, None, None) == fq.FQ_ERR_UNSUPPORTED
    assert L.fq_build_codebook(4, 64, 0, 1, 2, 128, p, p, None, None, None, None, None) == fq.FQ_ERR_UNSUPPORTED
    assert L.fq_build_codebook(4, 128, 5, 1, 2, 128, p, p, None, None, None, None, None) == fq.FQ_ERR_INVALID_ARG
    assert L.fq_build_codebook(4, 128, 0, 1, 2, 128, None, p, None, None, None, None, None) == fq.FQ_ERR_INVALID_ARG
    assert L.fq_build_codebook(4, 128, 0, 1, 2, 64, p, p, None, None, None, None, None) == fq.FQ_ERR_UNSUPPORTED


def _fake_structs(bits=4, qjl=128, hkv=2):
    """Structs whose pointers are aligned host addresses: only argument checks may see them."""
    store = np.zeros(1 << 16, np.float32)
    base = (store.ctypes.data + 255) & ~255
    qz = fq.QuantizerT(bits, 128, fq.ROT_HAAR, qjl, base, base, base, base, base, base, base, None)
    cz = fq.CacheT(4, 16, hkv, 128, bits, qjl, base, base, base, base, base, base)
    return store, base, qz, cz


def test_compress_argument_checks():
    L = fq.lib()
    store, base, qz, cz = _fake_structs()
    call = lambda q, c, **kw: L.fq_compress(None, ctypes.byref(q) if q else None, ctypes.byref(c) if c else None,
                                            kw.get("k", base), kw.get("v", base), kw.get("dt", fq.BF16),
                                            kw.get("n", 4), kw.get("ts", 256), kw.get("hs", 128),
                                            kw.get("slots", base), None, None)
    assert call(None, cz) == fq.FQ_ERR_INVALID_ARG
    assert call(qz, None) == fq.FQ_ERR_INVALID_ARG
    assert call(qz, cz, dt=7) == fq.FQ_ERR_INVALID_ARG
    assert call(qz, cz, n=-1) == fq.FQ_ERR_INVALID_ARG
    assert call(qz, cz, n=0) == fq.FQ_OK                      # empty input is a no-op
    assert call(qz, cz, k=None, v=None) == fq.FQ_OK
    assert call(qz, cz, slots=None) == fq.FQ_ERR_INVALID_ARG
    assert call(qz, cz, k=base + 2) == fq.FQ_ERR_INVALID_ARG  # vectors must be 16-byte aligned
    assert call(qz, cz, hs=4) == fq.FQ_ERR_INVALID_ARG        # 8-byte head stride
    qb = fq.QuantizerT(5, 128, 0, 128, base, base, base, base, base, base, base, None)
    assert call(qb, cz) == fq.FQ_ERR_UNSUPPORTED
    # keys of their own width: 2..4 bits, with their own codebook, matching the cache's
    qk = fq.QuantizerT(4, 128, 0, 128, base, base, base, base, base, base, base, None, 5, base, base)
    assert call(qk, cz) == fq.FQ_ERR_UNSUPPORTED
    qk = fq.QuantizerT(4, 128, 0, 128, base, base, base, base, base, base, base, None, 3, None, base)
    assert call(qk, cz) == fq.FQ_ERR_INVALID_ARG              # key codebook required
    qk = fq.QuantizerT(4, 128, 0, 128, base, base, base, base, base, base, base, None, 3, base, base)
    assert call(qk, cz) == fq.FQ_ERR_INVALID_ARG              # the cache's keys are 4-bit
    ck = fq.CacheT(4, 16, 2, 128, 4, 128, base, base, base, base, base, base, 3)
    assert call(qk, ck, n=0) == fq.FQ_OK
    assert call(qz, ck) == fq.FQ_ERR_INVALID_ARG              # 3-bit keys in the cache, 4-bit quantizer
    qk4 = fq.QuantizerT(4, 128, 0, 128, base, base, base, base, base, base, base, None, 4, None, None)
    assert call(qk4, cz, n=0) == fq.FQ_OK                     # key_bits = bits: the shared codebook
    cb = fq.CacheT(4, 8, 2, 128, 4, 128, base, base, base, base, base, base)
    assert call(qz, cb) == fq.FQ_ERR_UNSUPPORTED              # block size must be 16
    cm = fq.CacheT(4, 16, 2, 128, 2, 128, base, base, base, base, base, base)
    assert call(qz, cm) == fq.FQ_ERR_INVALID_ARG              # bits differ from the quantizer's
    cn = fq.CacheT(4, 16, 2, 128, 4, 128, base, base, None, base, base, base)
    assert call(qz, cn) == fq.FQ_ERR_INVALID_ARG              # QJL keys need k_qjl
    qn = fq.QuantizerT(4, 128, 0, 128, base, base, base, None, base, base, base, None)
    assert call(qn, cz) == fq.FQ_ERR_INVALID_ARG              # Pi^T required
    qt = fq.QuantizerT(4, 128, 0, 128, base, base, base, base, base, base, None, None)
    assert call(qt, cz) == fq.FQ_ERR_INVALID_ARG              # S^T required with QJL
    qm = fq.QuantizerT(4, 128, 0, 128, base, base, base, base, base, base, base, base + 8)
    assert call(qm, cz) == fq.FQ_ERR_INVALID_ARG              # operand buffer must be 16-byte aligned


def test_decode_argument_checks_and_workspace():
    L = fq.lib()
    store, base, qz, cz = _fake_structs(hkv=2)
    n = fq.workspace_bytes(3, 8, 2, 128, 128, 1000, 4)
    assert n >= 3 * 8 * 128 * 4 * 2 + 3 * 8 * 4 * (128 + 2) * 4
    assert fq.workspace_bytes(3, 8, 2, 128, 128, 1000, 0) == fq.workspace_bytes(
        3, 8, 2, 128, 128, 1000, fq.auto_splits(3, 2, 1000))

    def call(**kw):
        return L.fq_decode_attention(None, ctypes.byref(qz), ctypes.byref(cz), kw.get("q", base), fq.F32,
                                     kw.get("B", 3), kw.get("hq", 8), base, kw.get("mb", 63), base,
                                     kw.get("ms", 1000), kw.get("ns", 4), 0.088, kw.get("ws", base),
                                     kw.get("wb", n), kw.get("out", base))
    assert call(hq=7) == fq.FQ_ERR_INVALID_ARG       # Hq not a multiple of Hkv
    assert call(hq=2 * 17) == fq.FQ_ERR_UNSUPPORTED  # group of 17 query heads
    assert call(ns=65) == fq.FQ_ERR_UNSUPPORTED
    assert call(ms=63 * 16 + 1) == fq.FQ_ERR_INVALID_ARG
    assert call(out=None) == fq.FQ_ERR_INVALID_ARG
    assert call(wb=n - 1) == fq.FQ_ERR_WORKSPACE
    assert call(ws=None) == fq.FQ_ERR_WORKSPACE
    assert call(ws=base + 16) == fq.FQ_ERR_WORKSPACE  # 256-byte alignment
    assert call(B=0) == fq.FQ_OK


def test_step_window_argument_checks():
    """fq_decode_step_window: the append's arguments are checked before anything is launched."""
    L = fq.lib()
    store, base, qz, cz = _fake_structs(hkv=2)
    n = fq.workspace_bytes(3, 8, 2, 128, 128, 1000, 1)

    def call(**kw):
        return L.fq_decode_step_window(None, ctypes.byref(qz), ctypes.byref(cz), kw.get("kn", base),
                                       kw.get("vn", base), kw.get("kdt", fq.BF16), kw.get("pos", base),
                                       kw.get("ev", base), kw.get("wk", base), kw.get("wv", base),
                                       kw.get("cap", 16), base, base, fq.F32, kw.get("B", 3), 8, base, 63, base,
                                       1000, 1, 0.088, base, n, base)
    assert call(pos=None) == fq.FQ_ERR_INVALID_ARG
    assert call(ev=None) == fq.FQ_ERR_INVALID_ARG
    assert call(kn=None) == fq.FQ_ERR_INVALID_ARG
    assert call(kdt=7) == fq.FQ_ERR_INVALID_ARG
    assert call(kn=base + 4) == fq.FQ_ERR_INVALID_ARG   # new rows 8-byte aligned
    assert call(pos=base + 4) == fq.FQ_ERR_INVALID_ARG  # int64 positions
    assert call(wk=None) == fq.FQ_ERR_INVALID_ARG
    assert call(cap=0) == fq.FQ_ERR_INVALID_ARG
    assert call(cap=4097) == fq.FQ_ERR_INVALID_ARG
    assert call(B=0) == fq.FQ_OK


def test_auto_splits():
    assert fq.auto_splits(1, 8, 4096) == 32
    assert fq.auto_splits(1, 8, 32768) == 32
    assert fq.auto_splits(4, 8, 32768) == 16
    assert fq.auto_splits(1, 8, 1000) == 7
    assert fq.auto_splits(32, 8, 4096) == 1
    assert fq.auto_splits(16, 8, 4096) == 4
    assert fq.auto_splits(64, 8, 4096) == 1
    assert fq.auto_splits(1, 1, 100) == 1


def _perm_row(T, r):
    return 64 * ((r >> 2) & 1) + 16 * T + 4 * (r >> 3) + (r & 3)


def test_pack_mfma_operands_layout():
    """The packed operands are Pi in bf16 hi + lo and S in fp16 hi + lo (round to nearest
    even), in the fragment order documented in the header; checked entry by entry."""
    cb = fq.build_codebook(4, 128, fq.ROT_HAAR, 1, 2, 128)
    pi, sm = cb["rotation_matrix"], cb["qjl_matrix"]
    raw = fq.pack_mfma_operands(pi, sm).view(np.uint16).reshape(4, 32, 64, 8)

    def bf16_rne(x):
        u = np.asarray(x, np.float32).view(np.uint32).astype(np.uint64)
        return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) & 0xFFFF).astype(np.uint16)

    def bf16_val(b):
        return (b.astype(np.uint32) << 16).view(np.float32)

    for f in (0, 7, 13, 31):
        T, s = f >> 3, f & 7
        for l in (0, 5, 31, 32, 63):
            row = _perm_row(T, l & 31)
            col = 64 * (l >> 5) + 8 * s
            x = pi[row, col:col + 8]
            hi = bf16_rne(x)
            lo = bf16_rne(x - bf16_val(hi))
            assert np.array_equal(raw[0, f, l], hi) and np.array_equal(raw[1, f, l], lo)
            y = sm[row, col:col + 8]
            yh = y.astype(np.float16)
            yl = (y - yh.astype(np.float32)).astype(np.float16)
            assert np.array_equal(raw[2, f, l], yh.view(np.uint16))
            assert np.array_equal(raw[3, f, l], yl.view(np.uint16))
    # every coordinate appears exactly once per fragment column set
    rows = sorted(_perm_row(T, r) for T in range(4) for r in range(32) if (r >> 2) & 1 == 0)
    assert rows == list(range(64))
    assert fq.lib().fq_pack_mfma_operands(None, None, 128, None, 0) == fq.FQ_ERR_INVALID_ARG


def test_validate_indices_reports_every_error():
    """The host-side bounds check on slot ids, lengths and block-table entries
    (FlashQuant page, section 关键工程改进: index bounds checks on packing)."""
    nb = 10
    ok_slots = np.array([0, 5, -1, nb * 16 - 1], np.int64)
    fq.validate_indices(nb, slot_mapping=ok_slots)
    fq.validate_indices(nb, slot_mapping=np.zeros(0, np.int64))
    with pytest.raises(fq.FQError) as e:
        fq.validate_indices(nb, slot_mapping=np.array([3, nb * 16, 2], np.int64))
    assert (e.value.what, e.value.where, e.value.status) == (1, 1, fq.FQ_ERR_INVALID_ARG)
    bt = np.array([[0, 9, 3, -5], [7, 8, 12, 42]], np.int32)  # entries past each length are not read
    lens = np.array([48, 32], np.int32)
    fq.validate_indices(nb, block_tables=bt, seq_lens=lens, max_seq_len=64)
    fq.validate_indices(nb, slot_mapping=ok_slots, block_tables=bt, seq_lens=lens)
    with pytest.raises(fq.FQError) as e:  # block 12 is the 3rd block of sequence 1 (length 33)
        fq.validate_indices(nb, block_tables=bt, seq_lens=np.array([48, 33], np.int32), max_seq_len=64)
    assert (e.value.what, e.value.where) == (3, 1 * 4 + 2)
    with pytest.raises(fq.FQError) as e:  # negative entry within the length
        fq.validate_indices(nb, block_tables=bt, seq_lens=np.array([64, 0], np.int32), max_seq_len=64)
    assert (e.value.what, e.value.where) == (3, 3)
    with pytest.raises(fq.FQError) as e:  # length above max_seq_len
        fq.validate_indices(nb, block_tables=bt, seq_lens=np.array([16, 50], np.int32), max_seq_len=49)
    assert (e.value.what, e.value.where) == (2, 1)
    with pytest.raises(fq.FQError) as e:  # negative length
        fq.validate_indices(nb, block_tables=bt, seq_lens=np.array([-1, 0], np.int32), max_seq_len=64)
    assert (e.value.what, e.value.where) == (2, 0)
    with pytest.raises(fq.FQError) as e:  # max_seq_len wider than the table
        fq.validate_indices(nb, block_tables=bt, seq_lens=lens, max_seq_len=65)
    assert e.value.what == 0
    L = fq.lib()
    assert L.fq_validate_indices(-1, None, 0, None, 0, 0, None, 0, None, None) == fq.FQ_ERR_INVALID_ARG
    assert L.fq_validate_indices(nb, None, 3, None, 0, 0, None, 0, None, None) == fq.FQ_ERR_INVALID_ARG
    assert L.fq_validate_indices(nb, None, 0, ok_slots.ctypes.data_as(ctypes.c_void_p), 1, 4, None, 0,
                                 None, None) == fq.FQ_ERR_INVALID_ARG  # table without lengths
    assert fq.status_string(fq.FQ_ERR_SCRATCH) == "FQ_ERR_SCRATCH"
