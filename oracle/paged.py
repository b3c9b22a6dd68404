"""Paged compressed-cache layout (oracle).

The "FlashQuant" page ("架构设计") decodes straight from a paged cache
("Paged Decode", split-K over pages); the French FlashQuant page gives the
16-token block size. The field layout is this library's choice and is stated
here as the format both sides write:

  k_codes [num_blocks][Hkv][16][d*kbits/8] uint8   (kbits = key bits, = bits
                                                    unless keys use their own width)
  k_norm  [num_blocks][Hkv][16]            fp32
  k_qjl   [num_blocks][Hkv][16][m/8]       uint8   (keys with QJL only)
  k_gamma [num_blocks][Hkv][16]            fp32    (keys with QJL only)
  v_codes [num_blocks][Hkv][16][d*bits/8]  uint8
  v_norm  [num_blocks][Hkv][16]            fp32

A token goes to slot = block * 16 + offset. Token t of sequence b lives in
block block_table[b][t // 16] at offset t % 16.
"""
import numpy as np

BLOCK = 16


def empty_cache(num_blocks, num_kv_heads, head_dim, bits, qjl_dim=None, key_bits=None):
    cb = head_dim * bits // 8
    kcb = head_dim * (bits if key_bits is None else key_bits) // 8
    c = {
        "k_codes": np.zeros((num_blocks, num_kv_heads, BLOCK, kcb), np.uint8),
        "k_norm": np.zeros((num_blocks, num_kv_heads, BLOCK), np.float32),
        "v_codes": np.zeros((num_blocks, num_kv_heads, BLOCK, cb), np.uint8),
        "v_norm": np.zeros((num_blocks, num_kv_heads, BLOCK), np.float32),
    }
    if qjl_dim:
        c["k_qjl"] = np.zeros((num_blocks, num_kv_heads, BLOCK, qjl_dim // 8), np.uint8)
        c["k_gamma"] = np.zeros((num_blocks, num_kv_heads, BLOCK), np.float32)
    return c


def write(cache, slots, head, k_enc=None, v_enc=None):
    """Store encoded vectors of one KV head at the given slots (slot < 0 is skipped)."""
    slots = np.asarray(slots, dtype=np.int64)
    keep = slots >= 0
    blk = slots[keep] // BLOCK
    off = slots[keep] % BLOCK
    if k_enc is not None:
        cache["k_codes"][blk, head, off] = k_enc["codes"][keep]
        cache["k_norm"][blk, head, off] = k_enc["n"][keep]
        if "qjl" in k_enc and "k_qjl" in cache:
            cache["k_qjl"][blk, head, off] = k_enc["qjl"][keep]
            cache["k_gamma"][blk, head, off] = k_enc["gamma"][keep]
    if v_enc is not None:
        cache["v_codes"][blk, head, off] = v_enc["codes"][keep]
        cache["v_norm"][blk, head, off] = v_enc["n"][keep]


def token_locations(block_table_row, seq_len):
    """(block, offset) of tokens 0..seq_len-1 of one sequence."""
    t = np.arange(seq_len)
    return np.asarray(block_table_row, dtype=np.int64)[t // BLOCK], t % BLOCK


def read(cache, block_table_row, seq_len, head):
    """The records of one sequence and KV head, in token order."""
    blk, off = token_locations(block_table_row, seq_len)
    rec = {name: arr[blk, head, off] for name, arr in cache.items()}
    return rec
