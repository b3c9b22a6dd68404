"""The Llama-3-8B-shaped layer at batch 1 with a 4096-token context (32 query / 8 KV
heads, GQA 4, bf16 K/V, 16-token pages with a shuffled block table), end to end on
the GPU through the C ABI ("FlashQuant" page, section 性能数据: the batch-1, 4K-context
case).

* The GPU compresses the whole context: 256 sampled tokens under the fed protocol,
  and the cache written without the debug outputs is byte-identical to the one
  written with them (the benchmark runs without them).
* The oracle writes its own bytes; fq_decode_attention in the library's split
  choice for this shape (32 splits: the packed split kernel and the merge), at 16
  and at one split, against oracle.attention.decode_rotated within 1e-3 max-abs.
* fq_decode_step (the newest token appended by the GPU, 32 splits): the appended
  records under the fed protocol, the output against the oracle's decode of the
  GPU-written bytes within 1e-3.
"""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq, synth
from tests import parity
from tests.test_gpu_step import _step_case

pytestmark = pytest.mark.gpu


def test_compress_full_context_and_debug_off_bytes(gpu_lib):
    w = synth.workload(1)
    inp = synth.layer_inputs(w)
    t = parity.torch_inputs(inp, "bf16")
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    cache = fq.PagedCache(inp["num_blocks"], 8, 128, 4, 128)
    dy, dp = fq.compress(qz, cache, t["k"], t["v"], t["slots"], debug=True)
    tok = np.sort(np.random.default_rng(11).choice(4096, size=256, replace=False))
    print("near-tie mismatches", parity.check_compress(inp, oq, cache, dy, dp, tokens=tok))
    plain = fq.PagedCache(inp["num_blocks"], 8, 128, 4, 128)
    fq.compress(qz, plain, t["k"], t["v"], t["slots"])
    torch.cuda.synchronize()
    for name, a in cache.fields().items():
        assert torch.equal(a, plain.fields()[name]), name


@pytest.mark.parametrize("splits", [0, 1, 16])
def test_decode_against_oracle(gpu_lib, splits):
    w = synth.workload(1)
    inp = synth.layer_inputs(w)
    t = parity.torch_inputs(inp, "bf16")
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    host = parity.oracle_cache(inp, oq)
    cache = fq.PagedCache(inp["num_blocks"], 8, 128, 4, 128)
    parity.upload_cache(host, cache)
    assert fq.auto_splits(1, 8, 4096) == 32
    out = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 4096, num_splits=splits).cpu().numpy()
    ref = parity.oracle_decode(inp, host, oq)
    err = float(np.max(np.abs(out - ref)))
    print("splits", splits or 32, "max-abs", err, "cos vs exact", parity.cosine(out, parity.exact(inp)))
    assert err <= parity.DECODE_TOL


def test_decode_step_against_oracle(gpu_lib):
    w = synth.workload(1)
    inp = synth.layer_inputs(w)
    o = _step_case(w, inp, num_splits=0)
    assert o.shape == (1, 32, 128)
