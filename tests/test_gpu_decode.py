"""GPU parity of fq_decode_attention against the oracle (through the C ABI).

The GPU decodes the oracle's own compressed bytes, so the comparison isolates
the decode arithmetic; tolerance 1e-3 max-abs on the fp32 outputs."""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq, synth
from tests import parity

pytestmark = pytest.mark.gpu


def _decode_case(w, inp, rot=fq.ROT_HAAR, with_qjl=True, num_splits=0, seqs=None):
    t = parity.torch_inputs(inp, w.dtype)
    oq = parity.oracle_quantizer(w.bits, rot=rot)
    qz = fq.Quantizer(w.bits, 128, rot, 1, 2, 128)
    host = parity.oracle_cache(inp, oq, with_qjl=with_qjl, seqs=seqs)
    cache = fq.PagedCache(inp["num_blocks"], w.num_kv_heads, 128, w.bits, 128 if with_qjl else 0)
    parity.upload_cache(host, cache)
    out = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], max(w.seq_lens), num_splits=num_splits)
    torch.cuda.synchronize()
    ref = parity.oracle_decode(inp, host, oq, with_qjl=with_qjl, seqs=seqs)
    return out.cpu().numpy(), ref, (qz, cache, t, oq, host)


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("rot", [fq.ROT_HAAR, fq.ROT_WHT])
def test_decode_tiny(gpu_lib, bits, rot):
    w = synth.workload(0, bits=bits)
    inp = synth.layer_inputs(w)
    out, ref, _ = _decode_case(w, inp, rot=rot)
    err = np.max(np.abs(out - ref))
    print("max-abs", err, "cos vs exact", parity.cosine(out, parity.exact(inp)))
    assert err <= parity.DECODE_TOL


@pytest.mark.parametrize("splits", [3, 1])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("G", [1, 4, 8, 16])
def test_decode_groups_ragged(gpu_lib, G, bits, splits):
    w, inp = parity.small_workload(3, 2 * G, 2, [5, 333, 1000], 1008, bits=bits, seed=G)
    out, ref, _ = _decode_case(w, inp, num_splits=splits)
    assert np.max(np.abs(out - ref)) <= parity.DECODE_TOL


@pytest.mark.parametrize("splits", [0, 1])
@pytest.mark.parametrize("bits", [4, 2])
def test_decode_mse_only_keys(gpu_lib, bits, splits):
    w, inp = parity.small_workload(2, 8, 2, [700, 64], 704, bits=bits, seed=41)
    out, ref, _ = _decode_case(w, inp, with_qjl=False, num_splits=splits)
    assert np.max(np.abs(out - ref)) <= parity.DECODE_TOL


@pytest.mark.parametrize("splits", [2, 1])
def test_decode_empty_and_single_token(gpu_lib, splits):
    w, inp = parity.small_workload(3, 4, 2, [0, 1, 17], 32, seed=43)
    out, ref, _ = _decode_case(w, inp, num_splits=splits)
    assert np.all(out[0] == 0)
    assert np.max(np.abs(out - ref)) <= parity.DECODE_TOL


def test_decode_split_invariance_and_determinism(gpu_lib):
    w, inp = parity.small_workload(2, 16, 4, [1500, 999], 1504, seed=47)
    base, ref, (qz, cache, t, oq, host) = _decode_case(w, inp, num_splits=1)
    assert np.max(np.abs(base - ref)) <= parity.DECODE_TOL
    for s in (2, 4, 7, 64, 0):
        o = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 1500, num_splits=s).cpu().numpy()
        assert np.max(np.abs(o - base)) <= 1e-5, s
        o2 = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 1500, num_splits=s).cpu().numpy()
        assert np.array_equal(o, o2), s


def test_decode_block_permutation_is_bit_identical(gpu_lib):
    w, inp = parity.small_workload(1, 8, 2, [400], 400, seed=53)
    out, ref, (qz, cache, t, oq, host) = _decode_case(w, inp, num_splits=4)
    nb = inp["num_blocks"]
    perm = np.random.default_rng(1).permutation(nb)
    moved = {n: np.empty_like(a) for n, a in host.items()}
    for n, a in host.items():
        moved[n][perm] = a
    cache2 = fq.PagedCache(nb, 2, 128, 4, 128)
    parity.upload_cache(moved, cache2)
    bt2 = torch.from_numpy(perm[inp["block_tables"]].astype(np.int32)).cuda()
    o2 = fq.decode(qz, cache2, t["q"], bt2, t["lens"], 400, num_splits=4).cpu().numpy()
    assert np.array_equal(out, o2)


@pytest.mark.parametrize("splits", [0, 4])
def test_decode_full_size_b32_sampled(gpu_lib, splits):
    """The batch-32 8B-shaped layer (lengths 3072..4096) in the launch configuration the
    benchmark times (the library's split choice: one split, single launch) and with the
    4-way split; the oracle writes and checks three of the 32 sequences."""
    w = synth.workload(2)
    inp = synth.layer_inputs(w)
    seqs = [0, 13, 31]
    t = parity.torch_inputs(inp, "bf16")
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    cache = fq.PagedCache(inp["num_blocks"], 8, 128, 4, 128)
    dy, dp = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)  # many-tile LDS path
    rs = np.random.default_rng(3)
    tok = np.sort(rs.choice(parity.valid_tokens(inp)[0], size=192, replace=False))
    print("compress near-tie mismatches", parity.check_compress(inp, oq, cache, dy, dp, tokens=tok))
    del dy, dp
    host = parity.oracle_cache(inp, oq, seqs=seqs)
    blocks = np.concatenate([inp["block_tables"][b] for b in seqs])
    parity.upload_cache(host, cache, blocks=blocks)
    assert fq.auto_splits(32, 8, 4096) == 1
    out = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 4096, num_splits=splits).cpu().numpy()
    ref = parity.oracle_decode(inp, host, oq, seqs=seqs)
    err = np.max(np.abs(out[seqs] - ref))
    print("max-abs", err, "cos vs exact", parity.cosine(out[seqs], parity.exact(inp, seqs)))
    assert err <= parity.DECODE_TOL


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("G", [4, 8])
def test_decode_vector_alu_kernel_matches_matrix_core_kernel(gpu_lib, monkeypatch, bits, G):
    """The decode has matrix-core split kernels (default) and a vector-ALU one
    (FQ_DECODE_KERNEL=valu); both must match the oracle."""
    w, inp = parity.small_workload(2, 8 * G, 8, [2000, 777], 2000, bits=bits, seed=59)
    out_m, ref, (qz, cache, t, oq, host) = _decode_case(w, inp, num_splits=3)
    monkeypatch.setenv("FQ_DECODE_KERNEL", "valu")
    out_v = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 2000, num_splits=3).cpu().numpy()
    monkeypatch.delenv("FQ_DECODE_KERNEL")
    assert np.max(np.abs(out_m - ref)) <= parity.DECODE_TOL
    assert np.max(np.abs(out_v - ref)) <= parity.DECODE_TOL
    assert np.max(np.abs(out_m - out_v)) <= 1e-4


@pytest.mark.parametrize("rot", [fq.ROT_HAAR, fq.ROT_WHT])
def test_llama70b_layer_ctx32k_full_size(gpu_lib, rot):
    """70B-shaped layer, one sequence of 32768 tokens, 64 query / 8 KV heads (GQA 8),
    automatic split count; dense Haar and randomized Walsh-Hadamard rotations. The oracle
    compresses the whole context (the GPU decodes the oracle's bytes); 256 sampled
    tokens of the GPU's own compression of the same context are checked too."""
    w = synth.workload(3)
    inp = synth.layer_inputs(w)
    t = parity.torch_inputs(inp, "bf16")
    oq = parity.oracle_quantizer(4, rot=rot)
    qz = fq.Quantizer(4, 128, rot, 1, 2, 128)
    cache = fq.PagedCache(inp["num_blocks"], 8, 128, 4, 128)
    dy, dp = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)
    tok = np.sort(np.random.default_rng(5).choice(32768, size=256, replace=False))
    print("compress near-tie mismatches", parity.check_compress(inp, oq, cache, dy, dp, tokens=tok))
    del dy, dp
    host = parity.oracle_cache(inp, oq)
    parity.upload_cache(host, cache)
    splits = fq.auto_splits(1, 8, 32768)
    out = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 32768).cpu().numpy()
    ref = parity.oracle_decode(inp, host, oq)
    err = np.max(np.abs(out - ref))
    print("splits", splits, "max-abs", err, "cos vs exact", parity.cosine(out, parity.exact(inp)))
    assert splits == 32
    assert err <= parity.DECODE_TOL
    out64 = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 32768, num_splits=64).cpu().numpy()
    err64 = np.max(np.abs(out64 - ref))
    print("splits 64 max-abs", err64)
    assert err64 <= parity.DECODE_TOL


@pytest.mark.parametrize("vscale", [100.0, 1e4])
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("G", [4, 8, 16])
def test_decode_large_value_norms(gpu_lib, G, bits, splits, vscale):
    """Values scaled x100 and x1e4 (norms ~1.1e3 and ~1.1e5): the fp16 operand of the
    value product is kept in range by a power-of-two exponent that follows the value
    norms; the output matches the oracle within 1e-3 of the value scale."""
    w, inp = parity.small_workload(2, 2 * G, 2, [900, 333], 912, bits=bits, seed=200 + G)
    inp = dict(inp)
    inp["v"] = inp["v"] * np.float32(vscale)
    out, ref, _ = _decode_case(w, inp, num_splits=splits)
    assert np.all(np.isfinite(out))
    err = np.max(np.abs(out - ref)) / vscale
    print("max-abs / scale", err)
    assert err <= parity.DECODE_TOL
