"""Decode attention with a full-precision residual window (oracle; test infrastructure).

"TurboQuant" blog, "Couche 5" (the residual window) and "Couche 7" (a window of 128
tokens in its cache interface), and the KIVI page (its configuration's 128-token
residual length; "Limitations", item 4: the most recent tokens stay in 16-bit
floats): the newest tokens of a sequence stay in a small full-precision buffer and
only older ones are compressed. Readings: the window holds up to W tokens per
sequence in bf16 (the 16-bit type of this build's K/V inputs), in a
ring (token position pos lives in ring slot pos mod W, so the valid slots are the
first min(n, W) as a set); the attention of a query is one softmax over the
compressed tokens (scored as in ``attention.decode_rotated``, values reconstructed)
and the window tokens (exact scores and values); scale 1/sqrt(d).
"""
import numpy as np

from . import attention


def decode_with_window(q, cache, block_tables, seq_lens, levels32, pi, s, bits, win_k, win_v, win_lens,
                       scale=None, key_levels32=None, key_bits=None):
    """q: [B, Hq, d]; compressed tokens [0, seq_lens[b]) in the paged cache; window
    K/V win_k, win_v: [B, W, Hkv, d] with the first win_lens[b] ring slots valid.
    Returns out [B, Hq, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = cache["k_norm"].shape[1]
    G = Hq // Hkv
    c = np.asarray(levels32, dtype=np.float64)
    ck = c if key_levels32 is None else np.asarray(key_levels32, dtype=np.float64)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    m = s.shape[0] if s is not None else 0
    wk = np.asarray(win_k, dtype=np.float64)
    wv = np.asarray(win_v, dtype=np.float64)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L, w = int(seq_lens[b]), int(win_lens[b])
        for kvh in range(Hkv):
            if L > 0:
                r = attention.head_records(cache, block_tables[b], L, kvh, bits, d, m, key_bits)
                kc = ck[r["k_idx"]]
                v_hat = r["v_n"][:, None] * (c[r["v_idx"]] @ pi)
            for g in range(G):
                h = kvh * G + g
                sc, vals = [], []
                if L > 0:
                    sc.append(scale * attention.key_scores(pi @ q[b, h], kc, r, s))
                    vals.append(v_hat)
                if w > 0:
                    sc.append(scale * (wk[b, :w, kvh] @ q[b, h]))
                    vals.append(wv[b, :w, kvh])
                if not sc:
                    continue
                p = attention._softmax(np.concatenate(sc))
                out[b, h] = p @ np.concatenate(vals)
    return out
