"""GPU parity of the residual full-precision window (fq_decode_attention_window,
fq_window_append) against oracle/window.py (through the C ABI).

* Decode: the oracle's compressed bytes plus a bf16 window; one softmax over both,
  against the oracle to the decode tolerance (1e-3 max-abs), through the split
  kernels and the merge (1, 3 and automatic splits; groups 4, 8 and 16), with empty
  windows, windows only, and empty sequences; a 300-slot ring in the single launch
  (several 16-token rounds per wave, 4- and 2-bit codes, groups 4 and 8).
* Append: a run of decode steps. The ring after each append holds exactly the bf16
  of the tokens of the last W positions; the records the append compresses are
  bit-identical to fq_decode_step's append of the same bf16 tokens into a mirror
  cache (the same single-vector arithmetic, itself checked against the oracle in
  the step tests), and match the oracle's encoding of those tokens directly (codes
  and QJL bits up to near-ties, norms and gamma to rounding); nothing else in the
  cache changes; the final decode of the GPU-written cache and ring matches the
  oracle.
"""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq
from oracle import pipeline, quantize, window
from tests import parity

pytestmark = pytest.mark.gpu


def _oracle(inp, host, oq, wk, wv, wl, seq_lens=None):
    sl = inp["seq_lens"] if seq_lens is None else seq_lens
    return window.decode_with_window(inp["q"], host, inp["block_tables"], sl, oq["levels"], oq["pi"], oq["s"],
                                     oq["bits"], wk.float().cpu().numpy(), wv.float().cpu().numpy(), wl)


@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("G", [4, 8, 16])
def test_decode_with_window_matches_oracle(gpu_lib, G, splits):
    w, inp = parity.small_workload(4, 2 * G, 2, [5, 333, 1000, 0], 1008, seed=200 + G)
    t = parity.torch_inputs(inp, w.dtype)
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    host = parity.oracle_cache(inp, oq)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, 4, 128)
    parity.upload_cache(host, cache)
    W = 32
    g = torch.Generator(device="cuda").manual_seed(7 + G)
    wk = torch.randn((4, W, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
    wv = torch.randn((4, W, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
    for wl in ([32, 7, 0, 5], [0, 0, 0, 0], [1, 32, 32, 0]):
        wlt = torch.tensor(wl, dtype=torch.int32, device="cuda")
        out = fq.decode_window(qz, cache, t["q"], t["bt"], t["lens"], 1000, wk, wv, wlt, num_splits=splits)
        torch.cuda.synchronize()
        ref = _oracle(inp, host, oq, wk, wv, wl)
        err = float(np.max(np.abs(out.cpu().numpy() - ref)))
        print("window", wl, "max-abs", err)
        assert err <= parity.DECODE_TOL
        if wl == [0, 0, 0, 0]:  # no window: the plain decode's value
            plain = fq.decode(qz, cache, t["q"], t["bt"], t["lens"], 1000, num_splits=max(splits, 1))
            assert float((plain - out).abs().max()) <= 1e-5
        assert np.all(out.cpu().numpy()[3] == 0) == (wl[3] == 0)


def test_window_only_sequences(gpu_lib):
    """Nothing compressed (seq_lens 0): plain attention over the window tokens."""
    w, inp = parity.small_workload(2, 8, 2, [40, 17], 48, seed=211)
    t = parity.torch_inputs(inp, w.dtype)
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, 4, 128)
    g = torch.Generator(device="cuda").manual_seed(3)
    wk = torch.randn((2, 16, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
    wv = torch.randn((2, 16, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
    zero = torch.zeros(2, dtype=torch.int32, device="cuda")
    wl = [16, 3]
    out = fq.decode_window(qz, cache, t["q"], t["bt"], zero, 16, wk, wv,
                           torch.tensor(wl, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    host = parity.cache_to_host(cache)
    ref = _oracle(inp, host, oq, wk, wv, wl, seq_lens=np.zeros(2, np.int32))
    assert float(np.max(np.abs(out.cpu().numpy() - ref))) <= 1e-5


def _check_evicted(host, evicted, bk, bv, oq):
    """The records of the evicted tokens against the oracle's encoding of their bf16
    rows: codes differ only where the oracle's y is within rounding of a boundary,
    QJL bits only where its projection is within rounding of 0 or a code changed,
    norms to fp32 rounding, gamma to rounding where no code changed."""
    for h in range(bk.shape[2]):
        blk = np.array([s // 16 for _, _, s in evicted])
        off = np.array([s % 16 for _, _, s in evicted])
        for name, src in (("k", bk), ("v", bv)):
            x = np.stack([src[b, p, h].float().cpu().numpy() for b, p, _ in evicted]).astype(np.float64)
            e = pipeline.encode_keys(x, oq) if name == "k" else pipeline.encode_values(x, oq)
            bits = oq["key_bits"] if name == "k" else oq["bits"]
            bnd = oq["key_boundaries"] if name == "k" else oq["boundaries"]
            idx = quantize.unpack_codes(host[name + "_codes"][blk, h, off], bits, 128)
            diff = idx != e["idx"]
            if diff.any():
                gap = np.min(np.abs(e["y"][diff][:, None] - bnd.astype(np.float64)[None]), axis=1)
                assert np.all(gap <= parity.Y_TOL), (name, h, gap.max())
            assert np.allclose(host[name + "_norm"][blk, h, off], e["n"], rtol=1e-6, atol=0), (name, h)
            if name == "k":
                sig = quantize.unpack_bits(host["k_qjl"][blk, h, off], 128)
                sc = np.linalg.norm(oq["s"], axis=1)[None] * np.linalg.norm(e["r"], axis=1)[:, None]
                allowed = (np.abs(e["p"]) <= 2 * parity.Y_TOL * sc) | diff.any(axis=1)[:, None]
                assert np.all(allowed[sig != e["sig"]]), ("bits", h)
                same = ~diff.any(axis=1)
                assert np.allclose(host["k_gamma"][blk, h, off][same], e["gamma"][same], rtol=1e-5, atol=1e-30)


@pytest.mark.parametrize("kv", ["bf16", "f32"])
def test_append_steps_then_decode(gpu_lib, kv):
    B, Hkv, G, W, steps = 3, 2, 4, 16, 21
    n0 = np.array([5, 40, 70])
    cap = int(n0.max()) + steps
    rng = np.random.default_rng(17)
    nblk = (cap + 15) // 16
    bt = np.ascontiguousarray(np.arange(B * nblk, dtype=np.int32).reshape(B, nblk)[:, rng.permutation(nblk)])
    slot = lambda b, p: int(bt[b, p // 16]) * 16 + p % 16
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    oq = parity.oracle_quantizer(4)
    cache = fq.PagedCache(B * nblk, Hkv, 128, 4, 128)
    mirror = fq.PagedCache(B * nblk, Hkv, 128, 4, 128)
    # the mirror's appends go through fq_decode_step, whose decode part has nothing to read
    q0 = torch.zeros((B, Hkv * G, 128), dtype=torch.bfloat16, device="cuda")
    bt_t = torch.from_numpy(bt).cuda()
    no_len = torch.zeros(B, dtype=torch.int32, device="cuda")
    evicted = []  # (b, position, slot) of every record the append compressed
    dt = torch.bfloat16 if kv == "bf16" else torch.float32
    toks_k = torch.randn((B, cap, Hkv, 128), device="cuda").to(dt)
    toks_v = torch.randn((B, cap, Hkv, 128), device="cuda").to(dt)
    bk, bv = toks_k.to(torch.bfloat16), toks_v.to(torch.bfloat16)
    # initial state: positions < n - W compressed, the rest in the ring
    wk = torch.zeros((B, W, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    wv = torch.zeros_like(wk)
    for b in range(B):
        n = int(n0[b])
        c_end = max(0, n - W)
        if c_end:
            sl = torch.tensor([slot(b, p) for p in range(c_end)], dtype=torch.int64, device="cuda")
            for cc in (cache, mirror):
                fq.compress(qz, cc, bk[b, :c_end].contiguous(), bv[b, :c_end].contiguous(), sl)
        for p in range(c_end, n):
            wk[b, p % W] = bk[b, p]
            wv[b, p % W] = bv[b, p]
    n = n0.copy()
    for _ in range(steps):
        pos = torch.tensor(n, dtype=torch.int64, device="cuda")
        ev = [slot(b, int(n[b]) - W) if n[b] >= W else -1 for b in range(B)]
        evt = torch.tensor(ev, dtype=torch.int64, device="cuda")
        # mirror: the step's append of the same bf16 tokens
        ek = torch.stack([bk[b, max(int(n[b]) - W, 0)] for b in range(B)]).contiguous()
        evv = torch.stack([bv[b, max(int(n[b]) - W, 0)] for b in range(B)]).contiguous()
        fq.decode_step(qz, mirror, ek, evv, evt, q0, bt_t, no_len, 1)
        evicted += [(b, int(n[b]) - W, ev[b]) for b in range(B) if ev[b] >= 0]
        kn = torch.stack([toks_k[b, int(n[b])] for b in range(B)]).contiguous()
        vn = torch.stack([toks_v[b, int(n[b])] for b in range(B)]).contiguous()
        fq.window_append(qz, cache, kn, vn, pos, evt, wk, wv)
        n += 1
        torch.cuda.synchronize()
        for b in range(B):  # the ring holds the bf16 of the last min(n, W) tokens
            for p in range(max(0, int(n[b]) - W), int(n[b])):
                assert torch.equal(wk[b, p % W], bk[b, p]) and torch.equal(wv[b, p % W], bv[b, p])
    got, want = parity.cache_to_host(cache), parity.cache_to_host(mirror)
    for name in got:
        assert np.array_equal(got[name], want[name]), name
    assert len(evicted) > 0
    _check_evicted(got, evicted, bk, bv, oq)
    # final decode over the GPU-written cache and ring
    q = torch.randn((B, Hkv * G, 128), device="cuda").to(torch.bfloat16)
    seq_lens = np.maximum(n - W, 0).astype(np.int32)
    wl = np.minimum(n, W).astype(np.int32)
    out = fq.decode_window(qz, cache, q, torch.from_numpy(bt).cuda(), torch.from_numpy(seq_lens).cuda(), cap,
                           wk, wv, torch.from_numpy(wl).cuda())
    torch.cuda.synchronize()
    inp = {"q": q.float().cpu().numpy(), "block_tables": bt, "seq_lens": seq_lens}
    ref = _oracle(inp, got, oq, wk, wv, wl)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    print("max-abs", err)
    assert err <= parity.DECODE_TOL


@pytest.mark.parametrize("G,bits", [(4, 4), (8, 4), (4, 2), (8, 2)])
def test_long_window_single_launch(gpu_lib, G, bits):
    """A 300-slot ring at one split: several 16-token rounds per wave in the single launch
    (8 waves at 4-bit, 12 at 2-bit), windows of 300, 129, 17 and 0 tokens."""
    w, inp = parity.small_workload(4, 2 * G, 2, [40, 333, 7, 100], 352, bits=bits, seed=230 + G + bits)
    t = parity.torch_inputs(inp, w.dtype)
    oq = parity.oracle_quantizer(bits)
    qz = fq.Quantizer(bits, 128, fq.ROT_HAAR, 1, 2, 128)
    host = parity.oracle_cache(inp, oq)
    cache = fq.PagedCache(inp["num_blocks"], 2, 128, bits, 128)
    parity.upload_cache(host, cache)
    W = 300
    g = torch.Generator(device="cuda").manual_seed(19 + G)
    wk = torch.randn((4, W, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
    wv = torch.randn((4, W, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
    wl = [300, 129, 17, 0]
    out = fq.decode_window(qz, cache, t["q"], t["bt"], t["lens"], 352, wk, wv,
                           torch.tensor(wl, dtype=torch.int32, device="cuda"), num_splits=1)
    torch.cuda.synchronize()
    ref = _oracle(inp, host, oq, wk, wv, wl)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    print("max-abs", err)
    assert err <= parity.DECODE_TOL
