"""GPU parity of the codebook variants with 3-bit codes and the Prod key budget
("TurboQuant" blog, section on the mathematical intuition: 3-bit TurboQuant;
"FlashQuant" page, "架构设计": the quantizer's MSE / Prod modes), through the C ABI.

* 3 bits everywhere (keys 3-bit MSE + the QJL bit, values 3-bit): 48 bytes of codes
  per vector, coordinate j at bits 3j .. 3j+2 of the vector's bit stream;
* Prod budget at b = 4 (keys 3-bit MSE + QJL, values 4-bit) and b = 3 (keys 2-bit
  MSE + QJL, values 3-bit).
Compress under the fed protocol (both compress kernels: the many-tile one without
prepared operands, the small-input one with them), decode of the oracle's bytes
(one and three splits, groups 4 / 8 / 16, Haar and WHT; the matrix-core kernel at
one split against the vector-ALU one for groups 1 to 8), the decode step (the
newest token appended by the GPU), and decompress (fp32 within 1e-5 n of the
oracle's reconstruction; bf16 within the bf16 rounding of it plus 1e-3 n)."""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq
from oracle import quantize
from tests import parity
from tests.test_gpu_step import _step_case

pytestmark = pytest.mark.gpu

# (value bits, key bits)
WIDTHS = [(3, 3), (4, 3), (3, 2)]


def _cache(inp, w, kb, qjl=128):
    return fq.PagedCache(inp["num_blocks"], w.num_kv_heads, 128, w.bits, qjl, key_bits=kb)


@pytest.mark.parametrize("prepared", [False, True])
@pytest.mark.parametrize("rot", [fq.ROT_HAAR, fq.ROT_WHT])
@pytest.mark.parametrize("vb,kb", WIDTHS)
def test_compress(gpu_lib, vb, kb, rot, prepared):
    w, inp = parity.small_workload(2, 8, 4, [300, 77], 304, bits=vb, seed=300 + 10 * vb + kb)
    t = parity.torch_inputs(inp, w.dtype)
    qz = fq.Quantizer(vb, 128, rot, 1, 2, 128, prepared=prepared, key_bits=kb)
    oq = parity.oracle_quantizer(vb, rot=rot, key_bits=kb)
    cache = _cache(inp, w, kb)
    assert cache.k_codes.shape[-1] == 16 * kb and cache.v_codes.shape[-1] == 16 * vb
    dy, dp = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)
    torch.cuda.synchronize()
    print("near-tie mismatches", parity.check_compress(inp, oq, cache, dy, dp))


def test_compress_tiny_f32_three_bits(gpu_lib):
    from kv_cache_vector_tq4_amd import synth

    w = synth.workload(0, bits=3)
    inp = synth.layer_inputs(w)
    t = parity.torch_inputs(inp, w.dtype)
    qz = fq.Quantizer(3, 128, fq.ROT_HAAR, 1, 2, 128)
    cache = _cache(inp, w, 3)
    dy, dp = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)
    torch.cuda.synchronize()
    print("near-tie mismatches", parity.check_compress(inp, parity.oracle_quantizer(3), cache, dy, dp))


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("G", [4, 8, 16])
@pytest.mark.parametrize("vb,kb", WIDTHS)
def test_decode(gpu_lib, vb, kb, G, splits):
    w, inp = parity.small_workload(3, 2 * G, 2, [5, 333, 1000], 1008, bits=vb, seed=310 + G + vb + kb)
    t = parity.torch_inputs(inp, w.dtype)
    oq = parity.oracle_quantizer(vb, key_bits=kb)
    qz = fq.Quantizer(vb, 128, fq.ROT_HAAR, 1, 2, 128, key_bits=kb)
    host = parity.oracle_cache(inp, oq)
    cache = _cache(inp, w, kb)
    parity.upload_cache(host, cache)
    out = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 1000, num_splits=splits).cpu().numpy()
    ref = parity.oracle_decode(inp, host, oq)
    err = float(np.max(np.abs(out - ref)))
    print("max-abs", err, "cos vs exact", parity.cosine(out, parity.exact(inp)))
    assert err <= parity.DECODE_TOL


@pytest.mark.parametrize("G", [1, 2, 4, 8])
@pytest.mark.parametrize("vb,kb", WIDTHS)
def test_decode_matrix_core_matches_vector_alu(gpu_lib, monkeypatch, vb, kb, G):
    """3-bit keys (with 3- or 4-bit values) and 2-bit keys with 3-bit values decode on
    the matrix cores at G <= 8 (the codes widened to the 4-bit kernel's layouts); the vector-ALU kernel
    (FQ_DECODE_KERNEL=valu) computes the same function. Both against the oracle and
    within 1e-4 of each other, on ragged lengths over many pages."""
    w, inp = parity.small_workload(3, 2 * G, 2, [1, 600, 1500], 1504, bits=vb, seed=350 + G + vb)
    t = parity.torch_inputs(inp, w.dtype)
    oq = parity.oracle_quantizer(vb, key_bits=kb)
    qz = fq.Quantizer(vb, 128, fq.ROT_HAAR, 1, 2, 128, key_bits=kb)
    host = parity.oracle_cache(inp, oq)
    cache = _cache(inp, w, kb)
    parity.upload_cache(host, cache)
    out_m = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 1500, num_splits=1).cpu().numpy()
    monkeypatch.setenv("FQ_DECODE_KERNEL", "valu")
    out_v = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 1500, num_splits=1).cpu().numpy()
    monkeypatch.delenv("FQ_DECODE_KERNEL")
    ref = parity.oracle_decode(inp, host, oq)
    assert np.max(np.abs(out_m - ref)) <= parity.DECODE_TOL
    assert np.max(np.abs(out_v - ref)) <= parity.DECODE_TOL
    assert np.max(np.abs(out_m - out_v)) <= 1e-4


@pytest.mark.parametrize("vb,kb", WIDTHS)
def test_window_and_prefill(gpu_lib, vb, kb):
    """The residual window's decode (a 32-token bf16 window) and a causal prefill (every
    query token a decode of its prefix: 3-bit codes take the per-query path) on 3-bit
    keys, against oracle/window.py and oracle/prefill.py."""
    from oracle import prefill, window
    w, inp = parity.small_workload(2, 8, 2, [300, 77], 304, bits=vb, seed=360 + vb)
    t = parity.torch_inputs(inp, w.dtype)
    oq = parity.oracle_quantizer(vb, key_bits=kb)
    qz = fq.Quantizer(vb, 128, fq.ROT_HAAR, 1, 2, 128, key_bits=kb)
    host = parity.oracle_cache(inp, oq)
    cache = _cache(inp, w, kb)
    parity.upload_cache(host, cache)
    g = torch.Generator(device="cuda").manual_seed(vb)
    wk = torch.randn((2, 32, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
    wv = torch.randn((2, 32, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
    wl = [32, 9]
    out = fq.decode_window(qz, cache, t["q"], t["bt"], t["lens"], 300, wk, wv,
                           torch.tensor(wl, dtype=torch.int32, device="cuda")).cpu().numpy()
    ref = window.decode_with_window(inp["q"], host, inp["block_tables"], inp["seq_lens"], oq["levels"], oq["pi"],
                                    oq["s"], vb, wk.float().cpu().numpy(), wv.float().cpu().numpy(), wl,
                                    key_levels32=oq["key_levels"], key_bits=kb)
    assert np.max(np.abs(out - ref)) <= parity.DECODE_TOL
    L = 300
    q = torch.randn((L, 8, 128), generator=g, device="cuda").to(torch.bfloat16)
    seq, lens = [0] * L, list(range(1, L + 1))
    outp = fq.prefill(qz, cache, q, torch.tensor(seq, dtype=torch.int32, device="cuda"),
                      torch.tensor(lens, dtype=torch.int32, device="cuda"), t["bt"], L).cpu().numpy()
    refp = prefill.prefill_rotated(q.float().cpu().numpy(), seq, lens, host, inp["block_tables"], oq["levels"],
                                   oq["pi"], oq["s"], vb, key_levels32=oq["key_levels"], key_bits=kb)
    assert np.max(np.abs(outp - refp)) <= parity.DECODE_TOL


@pytest.mark.parametrize("vb,kb", WIDTHS)
def test_decode_wht_and_mse_only_keys(gpu_lib, vb, kb):
    w, inp = parity.small_workload(2, 8, 2, [700, 64], 704, bits=vb, seed=330 + vb + kb)
    t = parity.torch_inputs(inp, w.dtype)
    for rot, qjl in ((fq.ROT_WHT, True), (fq.ROT_HAAR, False)):
        oq = parity.oracle_quantizer(vb, rot=rot, key_bits=kb)
        qz = fq.Quantizer(vb, 128, rot, 1, 2, 128, key_bits=kb)
        host = parity.oracle_cache(inp, oq, with_qjl=qjl)
        cache = _cache(inp, w, kb, 128 if qjl else 0)
        parity.upload_cache(host, cache)
        out = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 704).cpu().numpy()
        ref = parity.oracle_decode(inp, host, oq, with_qjl=qjl)
        assert np.max(np.abs(out - ref)) <= parity.DECODE_TOL, (rot, qjl)


@pytest.mark.parametrize("splits", [1, 2])
@pytest.mark.parametrize("vb,kb", WIDTHS)
def test_decode_step(gpu_lib, vb, kb, splits):
    w, inp = parity.small_workload(3, 8, 2, [1, 17, 333], 336, bits=vb, seed=340 + vb + kb)
    _step_case(w, inp, num_splits=splits, key_bits=kb)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("vb,kb", WIDTHS)
def test_decompress(gpu_lib, vb, kb, out_dtype):
    w, inp = parity.small_workload(2, 8, 2, [300, 77], 304, bits=vb, seed=350 + vb + kb)
    oq = parity.oracle_quantizer(vb, key_bits=kb)
    qz = fq.Quantizer(vb, 128, fq.ROT_HAAR, 1, 2, 128, key_bits=kb)
    host = parity.oracle_cache(inp, oq)
    cache = _cache(inp, w, kb)
    parity.upload_cache(host, cache)
    slots = inp["slot_mapping"]
    k_hat, v_hat = fq.decompress(qz, cache, torch.from_numpy(slots).cuda(), dtype=out_dtype)
    torch.cuda.synchronize()
    live = slots >= 0
    for name, g, bits, lev in (("k", k_hat, kb, oq["key_levels"]), ("v", v_hat, vb, oq["levels"])):
        gg = g.float().cpu().numpy()[live].astype(np.float64)
        s = slots[live]
        blk, off = s // 16, s % 16
        worst = 0.0
        for h in range(2):
            idx = quantize.unpack_codes(host[name + "_codes"][blk, h, off], bits, 128)
            nrm = host[name + "_norm"][blk, h, off]
            ref = quantize.reconstruct(nrm, idx, lev, oq["pi"])
            n64 = np.asarray(nrm, np.float64)[:, None]
            if out_dtype == torch.float32:
                tol = 1e-5 * n64
            else:  # fp16 operands (2^-11 relative per term) + the bf16 rounding of the result
                tol = 1e-3 * n64 + np.abs(ref) * 2.0 ** -8
            worst = max(worst, float(np.max(np.abs(gg[:, h] - ref) / tol)))
        print(name, "worst error / tolerance", worst)
        assert worst <= 1.0, (name, worst)
