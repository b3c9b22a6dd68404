"""GPU parity with the spherical-marginal codebook (fq_build_levels, FQ_CB_SPHERE):
the kernels take the levels and boundaries the quantizer holds, so compress, decode
and decompress are checked against the oracle built with the same codebook, to the
tolerances of the Gaussian-codebook tests (through the C ABI)."""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq
from oracle import pipeline, quantize
from tests import parity

pytestmark = pytest.mark.gpu


def _quantizers(bits, rot=fq.ROT_HAAR):
    qz = fq.Quantizer(bits, 128, rot, 1, 2, 128, codebook=fq.CB_SPHERE)
    oq = parity.oracle_quantizer(bits, rot=rot, law=pipeline.SPHERE)
    assert np.array_equal(qz.host["levels"], oq["levels"])
    assert np.array_equal(qz.host["boundaries"], oq["boundaries"])
    g = parity.oracle_quantizer(bits, rot=rot)
    assert not np.array_equal(g["levels"], oq["levels"])
    return qz, oq


@pytest.mark.parametrize("bits", [4, 2])
def test_compress_with_sphere_codebook(gpu_lib, bits):
    w, inp = parity.small_workload(3, 8, 4, [1, 77, 300], 320, bits=bits, seed=41)
    t = parity.torch_inputs(inp, w.dtype)
    qz, oq = _quantizers(bits)
    cache = fq.PagedCache(inp["num_blocks"], w.num_kv_heads, 128, bits, 128)
    dy, dp = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)
    print("near-tie mismatches", parity.check_compress(inp, oq, cache, dy, dp))


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("rot", [fq.ROT_HAAR, fq.ROT_WHT])
def test_decode_with_sphere_codebook(gpu_lib, bits, splits, rot):
    w, inp = parity.small_workload(3, 8, 2, [5, 333, 1000], 1008, bits=bits, seed=43)
    t = parity.torch_inputs(inp, w.dtype)
    qz, oq = _quantizers(bits, rot)
    host = parity.oracle_cache(inp, oq)
    cache = fq.PagedCache(inp["num_blocks"], w.num_kv_heads, 128, bits, 128)
    parity.upload_cache(host, cache)
    out = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], max(w.seq_lens), num_splits=splits)
    torch.cuda.synchronize()
    ref = parity.oracle_decode(inp, host, oq)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    print("max-abs", err)
    assert err <= parity.DECODE_TOL


def test_decompress_with_sphere_codebook(gpu_lib):
    w, inp = parity.small_workload(2, 8, 2, [77, 200], 208, seed=47)
    qz, oq = _quantizers(4)
    host = parity.oracle_cache(inp, oq)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, 4, 128)
    parity.upload_cache(host, cache)
    slots = inp["slot_mapping"]
    k_hat, v_hat = fq.decompress(qz, cache, torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    for name, g in (("k", k_hat), ("v", v_hat)):
        gg = g.cpu().numpy()  # rows of skipped slots are never written: only stored rows are read
        for t_, s in enumerate(slots):
            if s < 0:
                continue
            blk, off = s // 16, s % 16
            idx = quantize.unpack_codes(host[name + "_codes"][blk, :, off], 4, 128)
            nrm = host[name + "_norm"][blk, :, off]
            ref = quantize.reconstruct(nrm, idx, oq["levels"], oq["pi"])
            assert np.all(np.abs(gg[t_].astype(np.float64) - ref) <= 1e-5 * np.asarray(nrm, np.float64)[:, None]), (name, t_)
