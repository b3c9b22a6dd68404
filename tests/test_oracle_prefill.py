"""CPU pins of the many-query (prefill) attention oracle (oracle/prefill.py): a query
that sees one token returns that token's value; tokens a query does not see can
change without changing its output; with MSE-only keys it equals causal softmax
attention written as one masked score matrix over the reconstructed keys and values."""
import numpy as np

from oracle import attention, prefill
from tests import parity


def _setup(with_qjl=True, seed=21):
    w, inp = parity.small_workload(2, 8, 2, [40, 23], 48, seed=seed)
    oq = parity.oracle_quantizer(4)
    host = parity.oracle_cache(inp, oq, with_qjl=with_qjl)
    return inp, oq, host


def _recon(host, bt_row, L, h, oq):
    c = np.asarray(oq["levels"], dtype=np.float64)
    r = attention.head_records(host, bt_row, L, h, 4, 128, 128)
    return r["k_n"][:, None] * (c[r["k_idx"]] @ oq["pi"]), r["v_n"][:, None] * (c[r["v_idx"]] @ oq["pi"])


def test_one_visible_token_gives_its_value():
    inp, oq, host = _setup()
    rng = np.random.default_rng(1)
    q = rng.standard_normal((3, 8, 128))
    out = prefill.prefill_rotated(q, [0, 1, 1], [1, 1, 1], host, inp["block_tables"], oq["levels"], oq["pi"],
                                  oq["s"], 4)
    for t, b in enumerate([0, 1, 1]):
        for h in range(8):
            _, v = _recon(host, inp["block_tables"][b], 1, h // 4, oq)
            assert np.max(np.abs(out[t, h] - v[0])) < 1e-12


def test_unseen_tokens_do_not_matter():
    inp, oq, host = _setup()
    rng = np.random.default_rng(2)
    q = rng.standard_normal((4, 8, 128))
    seq, lens = [0, 0, 1, 1], [5, 17, 3, 23]
    a = prefill.prefill_rotated(q, seq, lens, host, inp["block_tables"], oq["levels"], oq["pi"], oq["s"], 4)
    # scramble every record past position 17 of sequence 0 and past 3 of sequence 1 ...
    h2 = {k: v.copy() for k, v in host.items()}
    for b, start in ((0, 17), (1, 23)):
        for p in range(start, int(inp["seq_lens"][b])):
            blk, off = int(inp["block_tables"][b][p // 16]), p % 16
            for k in h2:
                h2[k][blk, :, off] = np.roll(h2[k][blk, :, off], 1, axis=-1) if h2[k].ndim == 4 else h2[k][blk, :, off] * 1.5
    b2 = prefill.prefill_rotated(q, seq, lens, h2, inp["block_tables"], oq["levels"], oq["pi"], oq["s"], 4)
    assert np.max(np.abs(a - b2)) < 1e-12


def test_mse_only_keys_equal_masked_score_matrix_attention():
    inp, oq, host = _setup(with_qjl=False, seed=23)
    rng = np.random.default_rng(3)
    L = int(inp["seq_lens"][0])
    q = rng.standard_normal((L, 8, 128))
    out = prefill.prefill_rotated(q, [0] * L, np.arange(1, L + 1), host, inp["block_tables"], oq["levels"],
                                  oq["pi"], None, 4)
    scale = 1.0 / np.sqrt(128)
    mask = np.tril(np.ones((L, L), bool))
    for h in range(8):
        k, v = _recon(host, inp["block_tables"][0], L, h // 4, oq)
        s = scale * (q[:, h] @ k.T)
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - s.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        assert np.max(np.abs(out[:, h] - p @ v)) < 1e-12
