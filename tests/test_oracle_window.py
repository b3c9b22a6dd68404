"""CPU pins of the residual-window attention oracle (oracle/window.py): it reduces to
the compressed decode when the window is empty and to plain attention when nothing is
compressed; with MSE-only keys it equals plain attention over the reconstructed keys
and values followed by the window's; the ring order of the window does not matter."""
import numpy as np

from kv_cache_vector_tq4_amd import synth
from oracle import attention, window
from tests import parity


def _case(seed, lens, with_qjl=True, W=24):
    w, inp = parity.small_workload(3, 8, 2, lens, 64, seed=seed)
    oq = parity.oracle_quantizer(4)
    host = parity.oracle_cache(inp, oq, with_qjl=with_qjl)
    rng = np.random.default_rng(seed)
    B, Hkv = 3, 2
    wk = rng.standard_normal((B, W, Hkv, 128)).astype(np.float32)
    wv = rng.standard_normal((B, W, Hkv, 128)).astype(np.float32)
    return inp, oq, host, wk, wv


def _run(inp, oq, host, wk, wv, wl, with_qjl=True):
    return window.decode_with_window(inp["q"], host, inp["block_tables"], inp["seq_lens"], oq["levels"], oq["pi"],
                                     oq["s"] if with_qjl else None, 4, wk, wv, wl)


def test_empty_window_is_the_compressed_decode():
    inp, oq, host, wk, wv = _case(3, [5, 40, 17])
    out = _run(inp, oq, host, wk, wv, [0, 0, 0])
    ref = attention.decode_rotated(inp["q"], host, inp["block_tables"], inp["seq_lens"], oq["levels"], oq["pi"],
                                   oq["s"], 4)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_nothing_compressed_is_plain_attention_over_the_window():
    inp, oq, host, wk, wv = _case(5, [5, 40, 17])
    inp = dict(inp)
    inp["seq_lens"] = np.zeros(3, np.int32)
    wl = np.array([24, 1, 9])
    out = _run(inp, oq, host, wk, wv, wl)
    ref = attention.exact_attention(inp["q"], wk, wv, wl)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_mse_only_keys_equal_plain_attention_over_reconstructions_then_window():
    inp, oq, host, wk, wv = _case(7, [5, 40, 17], with_qjl=False)
    wl = np.array([3, 24, 0])
    out = _run(inp, oq, host, wk, wv, wl, with_qjl=False)
    B, W, Hkv, d = wk.shape
    T = 64 + W
    k = np.zeros((B, T, Hkv, d))
    v = np.zeros((B, T, Hkv, d))
    lens = np.zeros(B, int)
    c = np.asarray(oq["levels"], dtype=np.float64)
    for b in range(B):
        L = int(inp["seq_lens"][b])
        for h in range(Hkv):
            r = attention.head_records(host, inp["block_tables"][b], L, h, 4, d, 0)
            k[b, :L, h] = r["k_n"][:, None] * (c[r["k_idx"]] @ oq["pi"])
            v[b, :L, h] = r["v_n"][:, None] * (c[r["v_idx"]] @ oq["pi"])
            k[b, L:L + wl[b], h] = wk[b, :wl[b], h]
            v[b, L:L + wl[b], h] = wv[b, :wl[b], h]
        lens[b] = L + wl[b]
    ref = attention.exact_attention(inp["q"], k, v, lens)
    assert np.max(np.abs(out - ref)) < 1e-12


def test_ring_order_does_not_matter():
    inp, oq, host, wk, wv = _case(9, [5, 40, 17])
    wl = np.array([24, 24, 24])
    out = _run(inp, oq, host, wk, wv, wl)
    perm = np.random.default_rng(1).permutation(24)
    out2 = _run(inp, oq, host, wk[:, perm], wv[:, perm], wl)
    assert np.max(np.abs(out - out2)) < 1e-12
