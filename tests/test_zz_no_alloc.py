"""fq_decode_attention_noalloc (the decode with the library's static scratch as its
workspace) against fq_decode_attention on the same inputs, through the C ABI: two
calls in a row, the second with a smaller input, each bit-identical to the
workspace entry point (same kernels) and within 1e-3 of the oracle; a call whose
workspace would exceed the static scratch is refused and launches nothing."""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq
from tests import parity

pytestmark = pytest.mark.gpu


def _case(B, G, lens, cap, seed, splits):
    w, inp = parity.small_workload(B, 2 * G, 2, lens, cap, seed=seed)
    t = parity.torch_inputs(inp, w.dtype)
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    host = parity.oracle_cache(inp, oq)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, 4, 128)
    parity.upload_cache(host, cache)
    ref = parity.oracle_decode(inp, host, oq)
    return qz, cache, t, max(lens), ref


def test_noalloc_matches_workspace_entry_point(gpu_lib):
    big = _case(3, 8, [5, 700, 1000], 1008, 301, 3)
    small = _case(1, 4, [260], 272, 302, 0)
    for (qz, cache, t, ml, ref), splits in ((big, 3), (small, 0), (big, 1)):
        B, Hq, d = t["q"].shape
        out = torch.full((B, Hq, d), float("nan"), dtype=torch.float32, device="cuda")
        fq.decode_noalloc(qz, cache, t["q"], t["bt"], t["lens"], ml, out, num_splits=splits)
        want = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], ml, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out, want), splits
        assert np.max(np.abs(out.cpu().numpy() - ref)) <= parity.DECODE_TOL


def test_noalloc_refuses_oversized_workspace(gpu_lib):
    qz, cache, t, ml, _ = _case(1, 4, [260], 272, 303, 0)
    # 4096 sequences x 8 query heads at one split needs > 8 MiB of workspace
    B = 4096
    assert fq.workspace_bytes(B, 8, 2, 128, 128, 272, 1) > fq.STATIC_SCRATCH_BYTES
    q = torch.zeros((B, 8, 128), dtype=torch.bfloat16, device="cuda")
    bt = t["bt"][:1].repeat(B, 1).contiguous()
    lens = t["lens"][:1].repeat(B).contiguous()
    out = torch.full((B, 8, 128), 7.0, dtype=torch.float32, device="cuda")
    with pytest.raises(fq.FQError) as e:
        fq.decode_noalloc(qz, cache, q, bt, lens, 272, out, num_splits=1)
    assert e.value.status == fq.FQ_ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
