"""Decode attention over the compressed, paged cache (oracle).

"FlashQuant" page: "架构设计" (paged decode reads the compressed cache) and
"QJL" (the corrected inner product <q,k> ~ <q,k_mse> + gamma sqrt(pi/2)/d
<Sq, sign(Sr)>). Readings: softmax scale 1/sqrt(d); output in float (the
oracle keeps float64); the QJL term uses m = d rows.

Two independent forms are given:
* ``decode_rotated``: rotate the query once (q~ = Pi q, q_s = S q~), score every
  token from its codes in the rotated frame, accumulate values in the rotated
  frame and un-rotate the weighted sum once (o = Pi^T o_rot);
* ``decode_reconstructed``: rebuild every k_hat and v_hat in the original frame
  and run a plain softmax attention over them, with the QJL term added.
They are algebraically equal, so they must agree to float64 rounding.
"""
import numpy as np

from . import paged
from .quantize import unpack_bits, unpack_codes, qjl_inner_product


def _softmax(s):
    s = np.asarray(s, dtype=np.float64)
    e = np.exp(s - np.max(s, axis=-1, keepdims=True))
    return e / np.sum(e, axis=-1, keepdims=True)


def head_records(cache, bt_row, seq_len, kvh, bits, d, m, key_bits=None):
    rec = paged.read(cache, bt_row, seq_len, kvh)
    out = {
        "k_idx": unpack_codes(rec["k_codes"], bits if key_bits is None else key_bits, d),
        "k_n": rec["k_norm"].astype(np.float64),
        "v_idx": unpack_codes(rec["v_codes"], bits, d),
        "v_n": rec["v_norm"].astype(np.float64),
    }
    if "k_qjl" in rec:
        out["sig"] = unpack_bits(rec["k_qjl"], m)
        out["gamma"] = rec["k_gamma"].astype(np.float64)
    return out


def key_scores(q_rot, k_levels, rec, s):
    """Unscaled scores of one rotated query against a sequence's keys.

    n_t <q~, c[idx_t]> plus, when the keys carry QJL fields, the QJL estimate of
    <q, k_t - k_mse_t>. k_levels: c[idx] per token [T, d].
    """
    sc = rec["k_n"] * (k_levels @ q_rot)
    if s is not None and "sig" in rec:
        sc = sc + qjl_inner_product(q_rot, rec["sig"], rec["gamma"], s)
    return sc


def decode_rotated(q, cache, block_tables, seq_lens, levels32, pi, s, bits, scale=None, key_levels32=None,
                   key_bits=None):
    """Form 1. q: [B, Hq, d]; returns out [B, Hq, d] float64.

    pi, s: the stored fp32 operators promoted to float64; s may be None for
    MSE-only keys (no QJL fields in the cache). key_levels32 / key_bits: the keys'
    codebook and width when they differ from the values' (levels32, bits).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = cache["k_norm"].shape[1]
    G = Hq // Hkv
    c = np.asarray(levels32, dtype=np.float64)
    ck = c if key_levels32 is None else np.asarray(key_levels32, dtype=np.float64)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    m = s.shape[0] if s is not None else 0
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for kvh in range(Hkv):
            r = head_records(cache, block_tables[b], L, kvh, bits, d, m, key_bits)
            kc = ck[r["k_idx"]]
            vc = c[r["v_idx"]]
            for g in range(G):
                h = kvh * G + g
                qr = pi @ q[b, h]
                p = _softmax(scale * key_scores(qr, kc, r, s))
                o_rot = (p * r["v_n"]) @ vc
                out[b, h] = pi.T @ o_rot
    return out


def decode_reconstructed(q, cache, block_tables, seq_lens, levels32, pi, s, bits, scale=None, key_levels32=None,
                         key_bits=None):
    """Form 2: reconstruct k_hat, v_hat in the original frame, then plain attention."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = cache["k_norm"].shape[1]
    G = Hq // Hkv
    c = np.asarray(levels32, dtype=np.float64)
    ck = c if key_levels32 is None else np.asarray(key_levels32, dtype=np.float64)
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    m = s.shape[0] if s is not None else 0
    s_orig = s @ pi if s is not None else None
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for kvh in range(Hkv):
            r = head_records(cache, block_tables[b], L, kvh, bits, d, m, key_bits)
            k_hat = r["k_n"][:, None] * (ck[r["k_idx"]] @ pi)
            v_hat = r["v_n"][:, None] * (c[r["v_idx"]] @ pi)
            for g in range(G):
                h = kvh * G + g
                sc = k_hat @ q[b, h]
                if s is not None and "sig" in r:
                    pm = 2.0 * r["sig"] - 1.0
                    sc = sc + r["gamma"] * np.sqrt(np.pi / 2.0) / m * (pm @ (s_orig @ q[b, h]))
                p = _softmax(scale * sc)
                out[b, h] = p @ v_hat
    return out


def exact_attention(q, k, v, seq_lens, scale=None):
    """Uncompressed attention. q: [B, Hq, d]; k, v: [B, T, Hkv, d] (float64)."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k.shape[2]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(d) if scale is None else scale
    out = np.zeros((B, Hq, d))
    for b in range(B):
        L = int(seq_lens[b])
        if L == 0:
            continue
        for h in range(Hq):
            kk = np.asarray(k[b, :L, h // G], dtype=np.float64)
            vv = np.asarray(v[b, :L, h // G], dtype=np.float64)
            p = _softmax(scale * (kk @ q[b, h]))
            out[b, h] = p @ vv
    return out
