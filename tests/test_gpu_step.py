"""GPU parity of fq_decode_step: the newest token of every sequence is compressed
into its slot, then the attention reads the cache (through the C ABI).

The oracle compresses every token but the newest of each sequence; the GPU appends
the newest ones itself. Checked:
* the appended records under the fed protocol (codes and QJL bits bit-exact given
  the GPU's y and p; y, p, norms and gamma to the compress tolerances);
* every other record of the cache untouched;
* the output against the oracle's decode of the GPU-written cache bytes (1e-3
  max-abs) and, bit for bit, against fq_decode_attention over the same cache.
"""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq, synth
from tests import parity

pytestmark = pytest.mark.gpu

GARBAGE = {"k_codes": 0xA5, "v_codes": 0x5A, "k_qjl": 0x3C}


def _newest(inp):
    """Flat index (into B*cap) and slot of each sequence's newest token (-1: none)."""
    B, cap = inp["k"].shape[:2]
    lens = inp["seq_lens"].astype(np.int64)
    flat = np.arange(B) * cap + np.maximum(lens - 1, 0)
    slots = np.where(lens > 0, inp["slot_mapping"][flat], -1)
    return flat, slots


def _without_newest(inp):
    prev = dict(inp)
    prev["seq_lens"] = np.maximum(inp["seq_lens"] - 1, 0).astype(inp["seq_lens"].dtype)
    return prev


def _fill_garbage(cache, slots):
    """Non-zero bytes / norms in the records the step must overwrite."""
    f = cache.fields()
    for s in slots[slots >= 0]:
        blk, off = int(s) // 16, int(s) % 16
        for name, t in f.items():
            if name in GARBAGE:
                t[blk, :, off] = GARBAGE[name]
            else:
                t[blk, :, off] = 0.75


def _flat_debug(dy, dp, flat, B, cap):
    Hkv, d = dy.shape[2], dy.shape[3]
    dyf = torch.zeros((2, B * cap, Hkv, d), dtype=torch.float32)
    dpf = torch.zeros((B * cap, Hkv, dp.shape[2]), dtype=torch.float32)
    dyf[:, flat] = dy.cpu()
    dpf[flat] = dp.cpu()
    return dyf, dpf


def _strip(host, slots):
    """The cache with the given records zeroed (for comparing everything else)."""
    out = {n: a.copy() for n, a in host.items()}
    for s in slots[slots >= 0]:
        for a in out.values():
            a[int(s) // 16, :, int(s) % 16] = 0
    return out


def _step_case(w, inp, rot=fq.ROT_HAAR, with_qjl=True, num_splits=0, kv_dtype=None, skip=(), key_bits=None):
    kvd = w.dtype if kv_dtype is None else kv_dtype
    t = parity.torch_inputs(inp, kvd)
    q = parity.torch_inputs(inp, w.dtype)["q"]
    oq = parity.oracle_quantizer(w.bits, rot=rot, key_bits=key_bits)
    qz = fq.Quantizer(w.bits, 128, rot, 1, 2, 128, key_bits=key_bits)
    B, cap, Hkv, d = inp["k"].shape
    flat, slots = _newest(inp)
    slots = slots.copy()
    for b in skip:
        slots[b] = -1
    host0 = parity.oracle_cache(_without_newest(inp), oq, with_qjl=with_qjl)
    cache = fq.PagedCache(inp["num_blocks"], Hkv, 128, w.bits, 128 if with_qjl else 0, key_bits=key_bits)
    parity.upload_cache(host0, cache)
    _fill_garbage(cache, slots)
    host_g = parity.cache_to_host(cache)
    k_new, v_new = t["k"][flat].contiguous(), t["v"][flat].contiguous()
    st = torch.from_numpy(slots).cuda()
    max_len = int(max(inp["seq_lens"].max(), 1))
    out, dy, dp = fq.decode_step(qz, cache, k_new, v_new, st, q, t["bt"], t["lens"], max_len,
                                 num_splits=num_splits, debug=True)
    torch.cuda.synchronize()
    host = parity.cache_to_host(cache)
    written = slots >= 0
    # records other than the appended ones are untouched (skipped slots keep their bytes)
    for n in host:
        assert np.array_equal(_strip(host, slots)[n], _strip(host_g, slots)[n]), n
    for b in np.nonzero(~written)[0]:
        s = _newest(inp)[1][b]
        if s >= 0:
            for n in host:
                assert np.array_equal(host[n][s // 16, :, s % 16], host_g[n][s // 16, :, s % 16]), (n, b)
    if written.any():
        dyf, dpf = _flat_debug(dy, dp, flat, B, cap)
        counts = parity.check_compress(inp, oq, cache, dyf, dpf if with_qjl else None, tokens=flat[written])
        print("near-tie mismatches", counts)
    ref = parity.oracle_decode(inp, host, oq, with_qjl=with_qjl)
    o = out.cpu().numpy()
    err = np.max(np.abs(o - ref))
    print("max-abs", err)
    assert err <= parity.DECODE_TOL
    plain = fq.decode(qz, cache, q, t["bt"], t["lens"], max_len, num_splits=num_splits).cpu().numpy()
    assert np.array_equal(o, plain)
    # the two halves, enqueued separately, are the step; the attention repeats exactly
    Hq = q.shape[1]
    ws = torch.empty(fq.workspace_bytes(B, Hq, Hkv, d, qz.qjl_dim, max_len, num_splits),
                     dtype=torch.uint8, device="cuda")
    fq.step_prepare(qz, cache, k_new, v_new, st, q, max_len, ws, num_splits=num_splits)
    for _ in range(2):
        o2 = fq.step_attend(qz, cache, B, Hq, t["bt"], t["lens"], max_len, ws, num_splits=num_splits)
        assert np.array_equal(o2.cpu().numpy(), o)
    again = parity.cache_to_host(cache)
    for n in host:
        assert np.array_equal(again[n], host[n]), n
    return o


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("bits", [4, 2])
@pytest.mark.parametrize("G", [4, 8, 16])
def test_step_groups_ragged(gpu_lib, G, bits, splits):
    w, inp = parity.small_workload(3, 2 * G, 2, [5, 333, 1000], 1008, bits=bits, seed=100 + G)
    _step_case(w, inp, num_splits=splits)


@pytest.mark.parametrize("kv", ["f32", "bf16"])
@pytest.mark.parametrize("rot", [fq.ROT_HAAR, fq.ROT_WHT])
def test_step_input_dtypes_and_rotations(gpu_lib, kv, rot):
    w, inp = parity.small_workload(2, 8, 2, [17, 300], 304, dtype="bf16", seed=71)
    _step_case(w, inp, rot=rot, num_splits=1, kv_dtype=kv)


@pytest.mark.parametrize("splits", [1, 2])
def test_step_mse_only_keys(gpu_lib, splits):
    w, inp = parity.small_workload(2, 8, 2, [700, 64], 704, seed=73)
    _step_case(w, inp, with_qjl=False, num_splits=splits)


@pytest.mark.parametrize("splits", [1, 2])
def test_step_empty_single_token_and_skipped_slot(gpu_lib, splits):
    """Length 0 (no token, zero output), length 1 (the new token is the whole
    context), and a sequence whose newest token is not stored (negative slot)."""
    w, inp = parity.small_workload(4, 4, 2, [0, 1, 17, 40], 48, seed=79)
    o = _step_case(w, inp, num_splits=splits, skip=(3,))
    assert np.all(o[0] == 0)


def test_step_full_size_b32(gpu_lib):
    """The batch-32 8B-shaped layer (lengths 3072..4096) in the launch configuration
    the benchmark times: the context but the newest tokens compressed by fq_compress,
    the newest 32 x 8 appended by the step; all appended records under the fed
    protocol, three sequences' outputs against the oracle's decode of the GPU bytes."""
    w = synth.workload(2)
    inp = synth.layer_inputs(w)
    t = parity.torch_inputs(inp, "bf16")
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    B, cap, Hkv, d = inp["k"].shape
    cache = fq.PagedCache(inp["num_blocks"], Hkv, 128, 4, 128)
    flat, slots = _newest(inp)
    ctx_slots = t["slots"].clone()
    ctx_slots[torch.from_numpy(flat).cuda()] = -1
    fq.compress(qz, cache, t["k"], t["v"], ctx_slots)
    _fill_garbage(cache, slots)
    k_new, v_new = t["k"][flat].contiguous(), t["v"][flat].contiguous()
    st = torch.from_numpy(slots).cuda()
    assert fq.auto_splits(B, Hkv, 4096) == 1
    out, dy, dp = fq.decode_step(qz, cache, k_new, v_new, st, t["q"], t["bt"], t["lens"], 4096, debug=True)
    torch.cuda.synchronize()
    dyf, dpf = _flat_debug(dy, dp, flat, B, cap)
    print("near-tie mismatches", parity.check_compress(inp, oq, cache, dyf, dpf, tokens=flat))
    host = parity.cache_to_host(cache)
    seqs = [0, 13, 31]
    ref = parity.oracle_decode(inp, host, oq, seqs=seqs)
    o = out.cpu().numpy()
    err = np.max(np.abs(o[seqs] - ref))
    print("max-abs", err)
    assert err <= parity.DECODE_TOL
    plain = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 4096).cpu().numpy()
    assert np.array_equal(o, plain)
