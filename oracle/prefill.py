"""Attention of many query tokens over the compressed, paged cache (oracle; test
infrastructure).

"FlashQuant" page, "架构设计": the fused attention with inline decompression serves
prefill, i.e. many queries per sequence. Reading: query token t of sequence s
attends to s's cached tokens [0, L_t) (L_t = position + 1 under the causal mask),
with the scores, QJL term and softmax of the decode (``attention.decode_rotated``)
- each query token is a decode of its own prefix.
"""
import numpy as np

from . import attention


def prefill_rotated(q, q_seq, q_lens, cache, block_tables, levels32, pi, s, bits, scale=None, key_levels32=None,
                    key_bits=None):
    """q: [T, Hq, d]; q_seq, q_lens: [T]; returns out [T, Hq, d] float64."""
    q = np.asarray(q, dtype=np.float64)
    bt = np.asarray(block_tables)[np.asarray(q_seq)]
    return attention.decode_rotated(q, cache, bt, np.asarray(q_lens), levels32, pi, s, bits, scale=scale,
                                    key_levels32=key_levels32, key_bits=key_bits)
