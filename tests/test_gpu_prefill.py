"""GPU parity of fq_prefill_attention (many query tokens per sequence, each attending
to its sequence's cached tokens [0, q_lens[t])) against oracle/prefill.py, through the
C ABI: causal prefill of whole sequences, a chunk of queries at the end of a long
context, full-attention queries (equal to fq_decode_attention's output for the same
queries), MSE-only keys; tolerance 1e-3 max-abs as for the decode.

With num_splits 0 or 1 (4-bit codes, groups dividing 16) the call takes the tiled path
(a wave per 16 query-head rows shares every page of its rows' prefixes); with a split
count it runs every query token as a decode of its prefix. Both are checked against
the oracle, and against each other."""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq
from oracle import prefill
from tests import parity

pytestmark = pytest.mark.gpu


def _case(G, with_qjl=True, seed=301):
    w, inp = parity.small_workload(2, 2 * G, 2, [300, 1000], 1008, seed=seed)
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    host = parity.oracle_cache(inp, oq, with_qjl=with_qjl)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, 4, 128 if with_qjl else 0)
    parity.upload_cache(host, cache)
    return inp, oq, qz, host, cache


def _check(inp, oq, qz, host, cache, seq, lens, G, splits=0, with_qjl=True, dtype=torch.bfloat16):
    T = len(seq)
    g = torch.Generator(device="cuda").manual_seed(T + G)
    q = torch.randn((T, 2 * G, 128), generator=g, device="cuda").to(dtype)
    st = torch.tensor(seq, dtype=torch.int32, device="cuda")
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    bt = torch.from_numpy(inp["block_tables"]).cuda()
    out = fq.prefill(qz, cache, q, st, lt, bt, int(max(lens)), num_splits=splits)
    torch.cuda.synchronize()
    ref = prefill.prefill_rotated(q.float().cpu().numpy(), seq, lens, host, inp["block_tables"], oq["levels"],
                                  oq["pi"], oq["s"] if with_qjl else None, 4)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    print("queries", T, "max-abs", err)
    assert err <= parity.DECODE_TOL
    return q, out


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("G", [4, 8, 16])
def test_causal_prefill_of_a_sequence(gpu_lib, G, splits):
    inp, oq, qz, host, cache = _case(G)
    L = int(inp["seq_lens"][0])
    _check(inp, oq, qz, host, cache, [0] * L, list(range(1, L + 1)), G, splits)


def test_chunk_at_the_end_of_a_long_context_and_mixed_sequences(gpu_lib):
    inp, oq, qz, host, cache = _case(4, seed=303)
    L1 = int(inp["seq_lens"][1])
    seq = [1] * 64 + [0] * 5
    lens = list(range(L1 - 63, L1 + 1)) + [1, 2, 150, 299, 300]
    _check(inp, oq, qz, host, cache, seq, lens, 4)


def test_full_attention_queries_equal_the_decode(gpu_lib):
    """Per-query path (a split count): bit-identical to fq_decode_attention; tiled path:
    within 1e-4 of it (its query rotation and value product round differently)."""
    inp, oq, qz, host, cache = _case(8, seed=305)
    seq, lens = [0, 1], [int(inp["seq_lens"][0]), int(inp["seq_lens"][1])]
    dec = None
    for splits in (2, 1):
        q, out = _check(inp, oq, qz, host, cache, seq, lens, 8, splits=splits)
        if dec is None:
            dec = fq.decode(qz, cache, q, torch.from_numpy(inp["block_tables"]).cuda(),
                            torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens), num_splits=2)
            assert torch.equal(dec, out)
        else:
            assert float((dec - out).abs().max()) <= 1e-4


def test_mse_only_keys(gpu_lib):
    inp, oq, qz, host, cache = _case(4, with_qjl=False, seed=307)
    L = int(inp["seq_lens"][0])
    _check(inp, oq, qz, host, cache, [0] * 40, list(range(L - 39, L + 1)), 4, with_qjl=False)


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
def test_tiled_rows_mixed_sequences_and_edges(gpu_lib, G):
    """Waves whose 16 rows mix two sequences, zero-length queries, a query count that
    leaves dead rows in the last tile, fp32 queries, and a prefix longer than 64 pages
    (1100 tokens: the block table is read in two chunks)."""
    w, inp = parity.small_workload(2, 2 * G, 2, [300, 1100], 1104, seed=320 + G)
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    host = parity.oracle_cache(inp, oq)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, 4, 128)
    parity.upload_cache(host, cache)
    rs = np.random.default_rng(G)
    seq = [int(x) for x in rs.integers(0, 2, size=37)]
    lens = [0 if i % 11 == 5 else int(rs.integers(1, int(inp["seq_lens"][s]) + 1)) for i, s in enumerate(seq)]
    lens[3], seq[3] = 1100, 1
    _check(inp, oq, qz, host, cache, seq, lens, G, dtype=torch.float32)


def test_tiled_and_per_query_paths_agree(gpu_lib, monkeypatch):
    inp, oq, qz, host, cache = _case(4, seed=331)
    L = int(inp["seq_lens"][1])
    seq, lens = [1] * L, list(range(1, L + 1))
    q, tiled = _check(inp, oq, qz, host, cache, seq, lens, 4)
    monkeypatch.setenv("FQ_PREFILL_UNTILED", "1")
    _, per_query = _check(inp, oq, qz, host, cache, seq, lens, 4)
    monkeypatch.delenv("FQ_PREFILL_UNTILED")
    assert float((tiled - per_query).abs().max()) <= 1e-4


@pytest.mark.parametrize("vscale", [100.0, 1e4])
def test_tiled_large_value_norms(gpu_lib, vscale):
    w, inp = parity.small_workload(1, 8, 2, [500], 512, seed=341)
    inp = dict(inp)
    inp["v"] = inp["v"] * np.float32(vscale)
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    host = parity.oracle_cache(inp, oq)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, 4, 128)
    parity.upload_cache(host, cache)
    L = 500
    q = torch.randn((L, 8, 128), generator=torch.Generator(device="cuda").manual_seed(5), device="cuda")
    st = torch.zeros(L, dtype=torch.int32, device="cuda")
    lt = torch.arange(1, L + 1, dtype=torch.int32, device="cuda")
    out = fq.prefill(qz, cache, q, st, lt, torch.from_numpy(inp["block_tables"]).cuda(), L)
    ref = prefill.prefill_rotated(q.cpu().numpy(), [0] * L, list(range(1, L + 1)), host, inp["block_tables"],
                                  oq["levels"], oq["pi"], oq["s"], 4)
    o = out.cpu().numpy()
    assert np.all(np.isfinite(o))
    assert float(np.max(np.abs(o - ref))) / vscale <= parity.DECODE_TOL


def test_tiled_full_size_causal_prefill_sampled(gpu_lib):
    """Causal prefill of one whole sequence of the batch-32 8B-shaped layer (3691 tokens,
    32 query / 8 KV heads) in the launch configuration the benchmark times; the oracle
    checks 48 sampled query tokens (all 32 heads each)."""
    from kv_cache_vector_tq4_amd import synth

    w = synth.workload(2)
    inp = synth.layer_inputs(w)
    b = 0
    L = int(inp["seq_lens"][b])
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    host = parity.oracle_cache(inp, oq, seqs=[b])
    cache = fq.PagedCache(inp["num_blocks"], 8, 128, 4, 128)
    parity.upload_cache(host, cache, blocks=inp["block_tables"][b])
    q = torch.randn((L, 32, 128), generator=torch.Generator(device="cuda").manual_seed(9), device="cuda")
    q = q.to(torch.bfloat16)
    st = torch.full((L,), b, dtype=torch.int32, device="cuda")
    lt = torch.arange(1, L + 1, dtype=torch.int32, device="cuda")
    out = fq.prefill(qz, cache, q, st, lt, torch.from_numpy(inp["block_tables"]).cuda(), 4096).cpu().numpy()
    pick = np.sort(np.random.default_rng(13).choice(L, size=48, replace=False))
    ref = prefill.prefill_rotated(q.float().cpu().numpy()[pick], [b] * len(pick), (pick + 1).tolist(), host,
                                  inp["block_tables"], oq["levels"], oq["pi"], oq["s"], 4)
    err = float(np.max(np.abs(out[pick] - ref)))
    print("max-abs over %d sampled queries" % len(pick), err)
    assert err <= parity.DECODE_TOL
