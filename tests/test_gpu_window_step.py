"""GPU parity of the window step (fq_decode_step_window): the residual window's
append and the decode over the compressed cache plus the window in one call.

* Small shapes, several steps in a row (rings not yet full, exactly full and
  wrapping; a sequence with no new token in some steps), groups 4 / 8 / 16, 4- and
  2-bit codes, bf16 and fp32 new rows, one split (the single launch), the automatic
  split count and 3 splits (the append's own launch, then the split path): every
  step's output, the cache bytes and the ring are bit-identical to fq_window_append
  followed by fq_decode_attention_window on a mirror copy; the last step's output
  matches oracle/window.py's decode over the GPU-written cache and ring to the
  decode tolerance (1e-3 max-abs).
* The batch-32 8B-shaped layer with a 128-token window in the launch configuration
  the benchmark times (one split): bit-identical to the two calls, three sequences
  against the oracle.
* A 300-slot ring at one split, the new token's slot in a wave's first 16-token round
  (rows requested before the append) or in a later one (requested after it).
"""
import numpy as np
import pytest
import torch

from kv_cache_vector_tq4_amd import fq, synth
from oracle import window
from tests import parity

pytestmark = pytest.mark.gpu


def _clone_cache(cache):
    c = fq.PagedCache(cache.num_blocks, cache.num_kv_heads, cache.head_dim, cache.bits, cache.qjl_dim)
    for name, t in cache.fields().items():
        c.fields()[name].copy_(t)
    return c


def _same_cache(a, b):
    ha, hb = parity.cache_to_host(a), parity.cache_to_host(b)
    for name in ha:
        assert np.array_equal(ha[name], hb[name]), name


def _oracle(q, host, oq, bt, seq_lens, wk, wv, wl):
    return window.decode_with_window(q.float().cpu().numpy(), host, bt, seq_lens, oq["levels"], oq["pi"], oq["s"],
                                     oq["bits"], wk.float().cpu().numpy(), wv.float().cpu().numpy(), wl)


@pytest.mark.parametrize("G,bits,splits,kv", [(4, 4, 1, "bf16"), (8, 4, 1, "f32"), (4, 2, 1, "bf16"),
                                              (8, 2, 1, "bf16"), (4, 4, 0, "bf16"), (8, 4, 3, "f32"),
                                              (16, 4, 1, "bf16")])
def test_step_window_matches_append_then_decode(gpu_lib, G, bits, splits, kv):
    B, Hkv, W, steps = 4, 2, 16, 5
    n0 = np.array([5, 14, 40, 70])  # ring filling, filling up during the steps, full, full
    cap = int(n0.max()) + steps
    rng = np.random.default_rng(300 + G + bits)
    nblk = (cap + 15) // 16
    bt = np.ascontiguousarray(np.arange(B * nblk, dtype=np.int32).reshape(B, nblk)[:, rng.permutation(nblk)])
    slot = lambda b, p: int(bt[b, p // 16]) * 16 + p % 16
    qz = fq.Quantizer(bits, 128, fq.ROT_HAAR, 1, 2, 128)
    oq = parity.oracle_quantizer(bits)
    cache = fq.PagedCache(B * nblk, Hkv, 128, bits, 128)
    g = torch.Generator(device="cuda").manual_seed(41 + G)
    dt = torch.bfloat16 if kv == "bf16" else torch.float32
    toks_k = torch.randn((B, cap, Hkv, 128), generator=g, device="cuda").to(dt)
    toks_v = torch.randn((B, cap, Hkv, 128), generator=g, device="cuda").to(dt)
    bk, bv = toks_k.to(torch.bfloat16), toks_v.to(torch.bfloat16)
    wk = torch.zeros((B, W, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    wv = torch.zeros_like(wk)
    for b in range(B):  # positions < n - W compressed, the rest in the ring
        n = int(n0[b])
        c_end = max(0, n - W)
        if c_end:
            sl = torch.tensor([slot(b, p) for p in range(c_end)], dtype=torch.int64, device="cuda")
            fq.compress(qz, cache, bk[b, :c_end].contiguous(), bv[b, :c_end].contiguous(), sl)
        for p in range(c_end, n):
            wk[b, p % W] = bk[b, p]
            wv[b, p % W] = bv[b, p]
    mirror, mk, mv = _clone_cache(cache), wk.clone(), wv.clone()
    bt_t = torch.from_numpy(bt).cuda()
    n = n0.copy()
    for step in range(steps):
        idle = step == 2  # sequence 1 gets no new token in this step
        pos_np = np.array([-1 if (idle and b == 1) else int(n[b]) for b in range(B)], np.int64)
        ev = [slot(b, int(n[b]) - W) if pos_np[b] >= 0 and n[b] >= W else -1 for b in range(B)]
        pos = torch.from_numpy(pos_np).cuda()
        evt = torch.tensor(ev, dtype=torch.int64, device="cuda")
        kn = torch.stack([toks_k[b, min(int(n[b]), cap - 1)] for b in range(B)]).contiguous()
        vn = torch.stack([toks_v[b, min(int(n[b]), cap - 1)] for b in range(B)]).contiguous()
        n_after = n + (pos_np >= 0)
        seq_lens = np.maximum(n_after - W, 0).astype(np.int32)
        wl = np.minimum(n_after, W).astype(np.int32)
        sl_t, wl_t = torch.from_numpy(seq_lens).cuda(), torch.from_numpy(wl).cuda()
        q = torch.randn((B, Hkv * G, 128), generator=g, device="cuda").to(torch.bfloat16)
        out = fq.decode_step_window(qz, cache, kn, vn, pos, evt, wk, wv, wl_t, q, bt_t, sl_t, cap, num_splits=splits)
        fq.window_append(qz, mirror, kn, vn, pos, evt, mk, mv)
        ref = fq.decode_window(qz, mirror, q, bt_t, sl_t, cap, mk, mv, wl_t, num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (step, float((out - ref).abs().max()))
        assert torch.equal(wk, mk) and torch.equal(wv, mv), step
        n = n_after
    _same_cache(cache, mirror)
    host = parity.cache_to_host(cache)
    want = _oracle(q, host, oq, bt, seq_lens, wk, wv, wl)
    err = float(np.max(np.abs(out.cpu().numpy() - want)))
    print("max-abs vs oracle", err)
    assert err <= parity.DECODE_TOL


def test_step_window_full_size_b32(gpu_lib):
    """The batch-32 8B-shaped layer (lengths 3072..4096, 32 q / 8 kv heads), a 128-token
    window: each sequence's newest token enters the ring, the one 128 positions back goes
    to the compressed cache; one split (the benchmark's launch)."""
    w = synth.workload(2)
    inp = synth.layer_inputs(w)
    t = parity.torch_inputs(inp, "bf16")
    oq = parity.oracle_quantizer(4)
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    B, cap, Hkv, d = inp["k"].shape
    W = 128
    lens = inp["seq_lens"].astype(np.int64)
    bt = inp["block_tables"]
    slot = lambda b, p: int(bt[b, p // 16]) * 16 + p % 16
    # before the step: tokens < n - 1 - W compressed, the W tokens before the newest in the ring
    ctx = t["slots"].clone().view(B, cap)
    for b in range(B):
        ctx[b, int(lens[b]) - 1 - W:] = -1
    cache = fq.PagedCache(inp["num_blocks"], Hkv, 128, 4, 128)
    fq.compress(qz, cache, t["k"], t["v"], ctx.reshape(-1).contiguous())
    wk = torch.zeros((B, W, Hkv, d), dtype=torch.bfloat16, device="cuda")
    wv = torch.zeros_like(wk)
    kb, vb = t["k"].view(B, cap, Hkv, d), t["v"].view(B, cap, Hkv, d)
    for b in range(B):
        for p in range(int(lens[b]) - 1 - W, int(lens[b]) - 1):
            wk[b, p % W] = kb[b, p]
            wv[b, p % W] = vb[b, p]
    mirror, mk, mv = _clone_cache(cache), wk.clone(), wv.clone()
    pos = torch.from_numpy(lens - 1).cuda()
    evt = torch.tensor([slot(b, int(lens[b]) - 1 - W) for b in range(B)], dtype=torch.int64, device="cuda")
    kn = torch.stack([kb[b, int(lens[b]) - 1] for b in range(B)]).contiguous()
    vn = torch.stack([vb[b, int(lens[b]) - 1] for b in range(B)]).contiguous()
    sl_t = torch.from_numpy((lens - W).astype(np.int32)).cuda()
    wl_t = torch.full((B,), W, dtype=torch.int32, device="cuda")
    assert fq.auto_splits(B, Hkv, cap) == 1
    out = fq.decode_step_window(qz, cache, kn, vn, pos, evt, wk, wv, wl_t, t["q"], t["bt"], sl_t, cap)
    fq.window_append(qz, mirror, kn, vn, pos, evt, mk, mv)
    ref = fq.decode_window(qz, mirror, t["q"], t["bt"], sl_t, cap, mk, mv, wl_t)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), float((out - ref).abs().max())
    assert torch.equal(wk, mk) and torch.equal(wv, mv)
    _same_cache(cache, mirror)
    seqs = [0, 13, 31]
    host = parity.cache_to_host(cache)
    want = _oracle(t["q"][seqs], host, oq, bt[seqs], (lens - W).astype(np.int32)[seqs], wk[seqs], wv[seqs],
                   np.full(len(seqs), W, np.int32))
    err = float(np.max(np.abs(out.cpu().numpy()[seqs] - want)))
    print("max-abs vs oracle", err)
    assert err <= parity.DECODE_TOL


def test_step_window_long_ring(gpu_lib):
    """A 300-slot ring, one split: the new token's slot lies in a later 16-token round of
    its wave (rows requested after the append), bit-identical to the two calls."""
    B, Hkv, G, W = 2, 2, 4, 300
    n0 = np.array([310, 290])  # full ring; filling ring
    cap = int(n0.max()) + 1
    rng = np.random.default_rng(77)
    nblk = (cap + 15) // 16
    bt = np.ascontiguousarray(np.arange(B * nblk, dtype=np.int32).reshape(B, nblk)[:, rng.permutation(nblk)])
    slot = lambda b, p: int(bt[b, p // 16]) * 16 + p % 16
    qz = fq.Quantizer(4, 128, fq.ROT_HAAR, 1, 2, 128)
    oq = parity.oracle_quantizer(4)
    cache = fq.PagedCache(B * nblk, Hkv, 128, 4, 128)
    g = torch.Generator(device="cuda").manual_seed(5)
    toks_k = torch.randn((B, cap, Hkv, 128), generator=g, device="cuda").to(torch.bfloat16)
    toks_v = torch.randn((B, cap, Hkv, 128), generator=g, device="cuda").to(torch.bfloat16)
    wk = torch.zeros((B, W, Hkv, 128), dtype=torch.bfloat16, device="cuda")
    wv = torch.zeros_like(wk)
    for b in range(B):
        n = int(n0[b])
        c_end = max(0, n - W)
        if c_end:
            sl = torch.tensor([slot(b, p) for p in range(c_end)], dtype=torch.int64, device="cuda")
            fq.compress(qz, cache, toks_k[b, :c_end].contiguous(), toks_v[b, :c_end].contiguous(), sl)
        for p in range(c_end, n):
            wk[b, p % W] = toks_k[b, p]
            wv[b, p % W] = toks_v[b, p]
    mirror, mk, mv = _clone_cache(cache), wk.clone(), wv.clone()
    pos = torch.from_numpy(n0.astype(np.int64)).cuda()
    evt = torch.tensor([slot(b, int(n0[b]) - W) if n0[b] >= W else -1 for b in range(B)], dtype=torch.int64,
                       device="cuda")
    kn = torch.stack([toks_k[b, int(n0[b])] for b in range(B)]).contiguous()
    vn = torch.stack([toks_v[b, int(n0[b])] for b in range(B)]).contiguous()
    n1 = n0 + 1
    sl_t = torch.from_numpy(np.maximum(n1 - W, 0).astype(np.int32)).cuda()
    wl = np.minimum(n1, W).astype(np.int32)
    wl_t = torch.from_numpy(wl).cuda()
    bt_t = torch.from_numpy(bt).cuda()
    q = torch.randn((B, Hkv * G, 128), generator=g, device="cuda").to(torch.bfloat16)
    out = fq.decode_step_window(qz, cache, kn, vn, pos, evt, wk, wv, wl_t, q, bt_t, sl_t, cap, num_splits=1)
    fq.window_append(qz, mirror, kn, vn, pos, evt, mk, mv)
    ref = fq.decode_window(qz, mirror, q, bt_t, sl_t, cap, mk, mv, wl_t, num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), float((out - ref).abs().max())
    assert torch.equal(wk, mk) and torch.equal(wv, mv)
    _same_cache(cache, mirror)
    want = _oracle(q, parity.cache_to_host(cache), oq, bt, np.maximum(n1 - W, 0).astype(np.int32), wk, wv, wl)
    err = float(np.max(np.abs(out.cpu().numpy() - want)))
    print("max-abs vs oracle", err)
    assert err <= parity.DECODE_TOL
