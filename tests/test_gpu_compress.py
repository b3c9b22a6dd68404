"""GPU parity of fq_compress against the oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq, synth
from tests import parity

pytestmark = pytest.mark.gpu


def _run(w, inp, rot=fq.ROT_HAAR, qjl=128, rot_seed=1, qjl_seed=2, prepared=True):
    t = parity.torch_inputs(inp, w.dtype)
    qz = fq.Quantizer(w.bits, 128, rot, rot_seed, qjl_seed, 128, prepared=prepared)
    cache = fq.PagedCache(inp["num_blocks"], w.num_kv_heads, 128, w.bits, qjl)
    dy, dp = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)
    oq = parity.oracle_quantizer(w.bits, rot=rot, rot_seed=rot_seed, qjl_seed=qjl_seed)
    return qz, cache, dy, dp, oq, t


@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("rot", [fq.ROT_HAAR, fq.ROT_WHT])
def test_compress_tiny_f32(gpu_lib, bits, rot):
    w = synth.workload(0, bits=bits)
    inp = synth.layer_inputs(w)
    qz, cache, dy, dp, oq, _ = _run(w, inp, rot=rot)
    c = parity.check_compress(inp, oq, cache, dy, dp)
    print("near-tie mismatches", c)


@pytest.mark.parametrize("bits", [4, 2])
def test_compress_ragged_bf16_several_tiles(gpu_lib, bits):
    """Ragged lengths (not multiples of 16 or 64), skipped slots, GQA shapes, bf16."""
    w, inp = parity.small_workload(3, 8, 4, [1, 77, 300], 320, bits=bits, seed=31)
    qz, cache, dy, dp, oq, _ = _run(w, inp)
    c = parity.check_compress(inp, oq, cache, dy, dp)
    print("near-tie mismatches", c)
    # slots of tokens past each sequence's length were never written
    host = parity.cache_to_host(cache)
    used = np.zeros(inp["num_blocks"] * 16, bool)
    used[inp["slot_mapping"][inp["slot_mapping"] >= 0]] = True
    unused = ~used.reshape(-1, 16)
    assert np.all(host["k_norm"].transpose(0, 2, 1)[unused] == 0)
    assert np.all(host["v_codes"].transpose(0, 2, 1, 3)[unused] == 0)


def test_compress_mse_only_keys(gpu_lib):
    w, inp = parity.small_workload(1, 4, 2, [100], 112, seed=3)
    qz, cache, dy, dp, oq, _ = _run(w, inp, qjl=0)
    assert cache.k_qjl is None
    parity.check_compress(inp, oq, cache, dy, None)


@pytest.mark.parametrize("prepared", [True, False])
def test_compress_zero_and_extreme_vectors(gpu_lib, prepared):
    """n = 0 gives y = 0 (all codes = #{boundaries < 0}); a huge-norm and a one-hot vector;
    through the small-input kernel (prepared operands) and the large-input one."""
    import torch

    w, inp = parity.small_workload(1, 2, 2, [16], 16, dtype="f32", seed=5)
    inp["k"][0, 0, 0] = 0.0
    inp["v"][0, 1, 1] = 0.0
    inp["k"][0, 2, 1] = 0.0
    inp["k"][0, 2, 1, 5] = 3.0
    inp["v"][0, 3, 0] *= 1e6
    qz, cache, dy, dp, oq, _ = _run(w, inp, prepared=prepared)
    parity.check_compress(inp, oq, cache, dy, dp)
    host = parity.cache_to_host(cache)
    s0 = inp["slot_mapping"][0]
    assert host["k_norm"][s0 // 16, 0, s0 % 16] == 0
    assert np.all(host["k_codes"][s0 // 16, 0, s0 % 16] == 0x77)
    assert host["k_gamma"][s0 // 16, 0, s0 % 16] == 0


def test_compress_strided_input(gpu_lib):
    """K and V may be views with token / head strides (e.g. slices of a fused QKV buffer)."""
    import torch

    w, inp = parity.small_workload(1, 8, 2, [50], 64, seed=9)
    t = parity.torch_inputs(inp, "bf16")
    fused = torch.zeros((t["k"].shape[0], 3, 2, 128), dtype=torch.bfloat16, device="cuda")
    fused[:, 1] = t["k"]
    fused[:, 2] = t["v"]
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, 4, 128)
    dy, dp = fq.compress(qz, cache, fused[:, 1], fused[:, 2], t["slots"], debug=True)
    oq = parity.oracle_quantizer(4)
    parity.check_compress(inp, oq, cache, dy, dp)


def test_compress_is_deterministic(gpu_lib):
    w, inp = parity.small_workload(2, 8, 2, [200, 130], 208, seed=13)
    outs = []
    for _ in range(2):
        qz, cache, dy, dp, oq, _ = _run(w, inp)
        outs.append(parity.cache_to_host(cache))
    for name in outs[0]:
        assert np.array_equal(outs[0][name], outs[1][name]), name


def test_compress_full_size_8b_layer_sampled(gpu_lib):
    """Whole 4096-token context of the 8B-shaped layer (8 KV heads, bf16) in one launch;
    sampled tokens of every head compared with the oracle."""
    w = synth.workload(1)
    inp = synth.layer_inputs(w)
    qz, cache, dy, dp, oq, _ = _run(w, inp)
    rs = np.random.default_rng(0)
    tok = np.sort(rs.choice(4096, size=256, replace=False))
    c = parity.check_compress(inp, oq, cache, dy, dp, tokens=tok)
    print("near-tie mismatches", c)


def test_compress_lane_kernel_matches_matrix_core_kernel(gpu_lib, monkeypatch):
    """fq_compress has a matrix-core tile kernel (default) and a lane-per-vector kernel
    (FQ_COMPRESS_KERNEL=lane); both must meet the parity bar on the same inputs."""
    w, inp = parity.small_workload(2, 8, 4, [300, 45], 304, seed=61)
    for impl in ("lane", None):
        if impl:
            monkeypatch.setenv("FQ_COMPRESS_KERNEL", impl)
        else:
            monkeypatch.delenv("FQ_COMPRESS_KERNEL", raising=False)
        qz, cache, dy, dp, oq, _ = _run(w, inp)
        parity.check_compress(inp, oq, cache, dy, dp)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("bits", [4, 2])
def test_compress_kernels_derive_operands_without_prepared_buffer(gpu_lib, bits, dtype):
    """Without the packed operand buffer the multi-tile kernel (the one large inputs use)
    builds the fragments in LDS; bf16 and fp32 inputs."""
    w, inp = parity.small_workload(2, 8, 4, [300, 45], 304, dtype=dtype, bits=bits, seed=67)
    qz, cache, dy, dp, oq, _ = _run(w, inp, prepared=False)
    parity.check_compress(inp, oq, cache, dy, dp)


@pytest.mark.parametrize("prepared", [False, True])
def test_compress_quantizer_without_qjl_matrix(gpu_lib, prepared):
    """A quantizer with no QJL matrix at all (qjl_dim 0) and an MSE-only cache, with
    and without the prepared matrix-core operands: keys use the MSE encoding only,
    checked against the oracle under the fed protocol."""
    w, inp = parity.small_workload(2, 4, 2, [300, 77], 304, seed=91)
    t = parity.torch_inputs(inp, w.dtype)
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 0, prepared=prepared)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, 4, 0)
    dy, _ = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)
    torch.cuda.synchronize()
    print("near-tie mismatches", parity.check_compress(inp, oq, cache, dy, None))


@pytest.mark.parametrize("impl", [None, "tile32"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("vb,kb", [(4, 4), (3, 3), (2, 2), (4, 3), (3, 2)])
def test_compress_many_tile_kernels(gpu_lib, monkeypatch, vb, kb, dtype, impl):
    """The kernels of large inputs (the path without the prepared operand buffer):
    16-vector tiles on 16x16x32 matrix-core products, two waves per SIMD (default),
    and 32-vector tiles (FQ_COMPRESS_KERNEL=tile32), on every width pair, bf16 and
    fp32 inputs, Haar and WHT, ragged lengths spanning several tiles and work-groups,
    against the oracle."""
    if impl:
        monkeypatch.setenv("FQ_COMPRESS_KERNEL", impl)
    else:
        monkeypatch.delenv("FQ_COMPRESS_KERNEL", raising=False)
    w, inp = parity.small_workload(3, 8, 4, [300, 45, 1], 304, dtype=dtype, bits=vb, seed=400 + 10 * vb + kb)
    t = parity.torch_inputs(inp, w.dtype)
    for rot in (fq.ROT_HAAR, fq.ROT_WHT):
        qz = fq.Quantizer(vb, 128, rot, 1, 2, 128, key_bits=kb, prepared=False)
        oq = parity.oracle_quantizer(vb, rot=rot, key_bits=kb)
        cache = fq.PagedCache(inp["num_blocks"], 4, 128, vb, 128, key_bits=kb)
        dy, dp = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)
        torch.cuda.synchronize()
        print(rot, "near-tie mismatches", parity.check_compress(inp, oq, cache, dy, dp))


@pytest.mark.parametrize("impl", [None, "tile32"])
def test_compress_many_tile_kernels_mse_only_and_full_size(gpu_lib, monkeypatch, impl):
    """The same kernels without QJL fields, and on the whole 4096-token 8B-shaped
    layer (32768 vectors per kind; sampled tokens of every head)."""
    if impl:
        monkeypatch.setenv("FQ_COMPRESS_KERNEL", impl)
    else:
        monkeypatch.delenv("FQ_COMPRESS_KERNEL", raising=False)
    w, inp = parity.small_workload(2, 4, 2, [300, 77], 304, seed=93)
    t = parity.torch_inputs(inp, w.dtype)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 0, prepared=False)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, 4, 0)
    dy, _ = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)
    torch.cuda.synchronize()
    parity.check_compress(inp, parity.oracle_quantizer(4), cache, dy, None)
    w = synth.workload(1)
    inp = synth.layer_inputs(w)
    qz, cache, dy, dp, oq, _ = _run(w, inp, prepared=False)
    tok = np.sort(np.random.default_rng(1).choice(4096, size=256, replace=False))
    print("near-tie mismatches", parity.check_compress(inp, oq, cache, dy, dp, tokens=tok))


@pytest.mark.parametrize("case", range(4))
def test_compress_many_tile_random_shapes(gpu_lib, case):
    """The large-input kernel on seeded random shapes: 1, 2, 3 or 8 KV heads, ragged
    lengths (tiles straddle tokens and sequences), K and V as strided views of one
    fused buffer, tokens past each length skipped, every width pair, bf16 or fp32."""
    rs = np.random.default_rng(700 + case)
    hkv = [1, 2, 3, 8][case]
    B = int(rs.integers(1, 4))
    lens = [int(x) for x in rs.integers(1, 200, size=B)]
    cap = (max(lens) + 15) // 16 * 16 + 16
    vb, kb = [(4, 4), (3, 3), (2, 2), (4, 3), (3, 2)][int(rs.integers(0, 5))]
    dtype = ["bf16", "f32"][case % 2]
    w, inp = parity.small_workload(B, 2 * hkv, hkv, lens, cap, dtype=dtype, bits=vb, seed=710 + case)
    t = parity.torch_inputs(inp, dtype)
    fused = torch.zeros((t["k"].shape[0], 3, hkv, 128), dtype=t["k"].dtype, device="cuda")
    fused[:, 0] = t["k"]
    fused[:, 2] = t["v"]
    qz = fq.Quantizer(vb, 128, fq.ROT_HAAR, 1, 2, 128, key_bits=kb, prepared=False)
    oq = parity.oracle_quantizer(vb, key_bits=kb)
    cache = fq.PagedCache(inp["num_blocks"], hkv, 128, vb, 128, key_bits=kb)
    dy, dp = fq.compress(qz, cache, fused[:, 0], fused[:, 2], t["slots"], debug=True)
    torch.cuda.synchronize()
    print(hkv, B, lens, vb, kb, dtype, "near-tie mismatches", parity.check_compress(inp, oq, cache, dy, dp))


@pytest.mark.parametrize("vb,kb,qjl", [(4, 4, 128), (4, 3, 128), (2, 2, 0)])
def test_compress_large_prepared_equals_derived(gpu_lib, vb, kb, qjl):
    """Past 1024 tiles of 32 vectors the 16-vector kernel takes its fragments from the
    prepared operand buffer (a gather) or derives them from the fp32 matrices: both
    must write the same bytes, and sampled tokens match the oracle. 4200 tokens x 8
    KV heads (33 600 vectors per kind)."""
    w, inp = parity.small_workload(1, 32, 8, [4200], 4208, bits=vb, seed=800 + vb + kb)
    t = parity.torch_inputs(inp, w.dtype)
    hosts = []
    for prepared in (True, False):
        qz = fq.Quantizer(vb, 128, fq.ROT_HAAR, 1, 2, qjl, key_bits=kb, prepared=prepared)
        cache = fq.PagedCache(inp["num_blocks"], 8, 128, vb, qjl, key_bits=kb)
        dy, dp = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)
        torch.cuda.synchronize()
        hosts.append(parity.cache_to_host(cache))
    for name in hosts[0]:
        assert np.array_equal(hosts[0][name], hosts[1][name]), name
    oq = parity.oracle_quantizer(vb, key_bits=kb)
    tok = np.sort(np.random.default_rng(3).choice(4200, size=128, replace=False))
    print("near-tie mismatches", parity.check_compress(inp, oq, cache, dy, dp if qjl else None, tokens=tok))
