"""GPU parity of fq_prefill_attention (many query tokens per sequence, each attending
to its sequence's cached tokens [0, q_lens[t])) against oracle/prefill.py, through the
C ABI: causal prefill of whole sequences, a chunk of queries at the end of a long
context, full-attention queries (equal to fq_decode_attention's output for the same
queries), MSE-only keys; tolerance 1e-3 max-abs as for the decode."""
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


def _check(inp, oq, qz, host, cache, seq, lens, G, splits=0, with_qjl=True):
    T = len(seq)
    g = torch.Generator(device="cuda").manual_seed(T + G)
    q = torch.randn((T, 2 * G, 128), generator=g, device="cuda").to(torch.bfloat16)
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
    inp, oq, qz, host, cache = _case(8, seed=305)
    seq, lens = [0, 1], [int(inp["seq_lens"][0]), int(inp["seq_lens"][1])]
    q, out = _check(inp, oq, qz, host, cache, seq, lens, 8, splits=1)
    dec = fq.decode(qz, cache, q, torch.from_numpy(inp["block_tables"]).cuda(),
                    torch.tensor(lens, dtype=torch.int32, device="cuda"), max(lens), num_splits=1)
    assert torch.equal(dec, out)


def test_mse_only_keys(gpu_lib):
    inp, oq, qz, host, cache = _case(4, with_qjl=False, seed=307)
    L = int(inp["seq_lens"][0])
    _check(inp, oq, qz, host, cache, [0] * 40, list(range(L - 39, L + 1)), 4, with_qjl=False)
