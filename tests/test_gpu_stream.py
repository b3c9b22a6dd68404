"""The compression-bound prefill stream of a 70B-shaped model: 80 layers x 8 KV heads x
32768 tokens (bf16 K and V, 10.7 GB in), compressed at 4 bits and at 2 bits with the
dense Haar rotation, then batch-4 decode at 32K context on the 2-bit cache. Sampled
outputs are compared with the oracle."""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq, synth
from tests import parity

pytestmark = pytest.mark.gpu

LAYERS, HKV, T = 80, 8, 32768


@pytest.mark.parametrize("bits", [4, 2])
def test_eighty_layer_stream_compress(gpu_lib, bits):
    """All 80 layers compressed in one launch each (one quantizer per layer: rotation seed
    1 + layer, QJL seed 2 + layer); two layers are checked on sampled tokens."""
    slots = torch.arange(T, dtype=torch.int64, device="cuda")
    checked = {0: None, 79: None}
    for layer in range(LAYERS):
        qz = fq.Quantizer(bits, 128, fq.ROT_HAAR, 1 + layer, 2 + layer, 128)
        cache = fq.PagedCache(T // 16, HKV, 128, bits, 128)
        if layer in checked:
            w = synth.Workload("stream-layer", 1, 64, HKV, 128, [T], T, bits=bits)
            inp = synth.layer_inputs(w, data_seed=3000 + layer)
            inp["slot_mapping"] = np.arange(T, dtype=np.int64)  # identity pages
            tt = parity.torch_inputs(inp, "bf16")
            dy, dp = fq.compress(qz, cache, tt["k"], tt["v"], slots, debug=True)
            oq = parity.oracle_quantizer(bits, rot_seed=1 + layer, qjl_seed=2 + layer)
            tok = np.sort(np.random.default_rng(layer).choice(T, size=128, replace=False))
            checked[layer] = parity.check_compress(inp, oq, cache, dy, dp, tokens=tok)
            del dy, dp, tt
        else:
            k, v = synth.kv_device(4000 + layer, T, HKV, 128)
            fq.compress(qz, cache, k, v, slots)
            del k, v
        del cache
    torch.cuda.synchronize()
    print("near-tie mismatches", checked)


def test_batch4_decode_ctx32k_on_2bit_cache(gpu_lib):
    """Batch 4 x 32768 tokens, 64 query / 8 KV heads, 2-bit K (MSE + QJL) and V: the GPU
    compresses all four sequences, the oracle rewrites two of them with its own bytes and
    checks those outputs."""
    w = synth.workload(4, bits=2, layers=1)
    inp = synth.layer_inputs(w)
    t = parity.torch_inputs(inp, "bf16")
    oq = parity.oracle_quantizer(2)
    qz = fq.Quantizer(2, 128, fq.ROT_HAAR, 1, 2, 128)
    cache = fq.PagedCache(inp["num_blocks"], 8, 128, 2, 128)
    fq.compress(qz, cache, t["k"], t["v"], t["slots"])
    del t["k"], t["v"]
    seqs = [0, 3]
    host = parity.oracle_cache(inp, oq, seqs=seqs)
    blocks = np.concatenate([inp["block_tables"][b] for b in seqs])
    parity.upload_cache(host, cache, blocks=blocks)
    out = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 32768).cpu().numpy()
    ref = parity.oracle_decode(inp, host, oq, seqs=seqs)
    err = np.max(np.abs(out[seqs] - ref))
    print("max-abs", err)
    assert err <= parity.DECODE_TOL
