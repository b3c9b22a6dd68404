"""Pins of the oracle's per-vector encoding and QJL estimator.

Sources: byte counts ("FlashQuant" page, "TurboQuant" step 4 and "性能数据":
64 B of 4-bit codes + 4 B fp32 norm = 68 B per 128-d vector; "TurboQuant"
blog, "Couche 3": two indices per byte at 4 bits, four at 2 bits; "QJL":
one extra bit per dimension), the MSE bound of the "TurboQuant" section,
the QJL properties (unbiased, O(1/d) variance) of the "QJL" section, the
cosine >= 0.95 of the standalone 4-bit quantizer ("使用方式"), and closed
forms derived from them.
"""
import numpy as np
import pytest

from kv_cache_vector_tq4_amd import synth
from oracle import codebook, pipeline, quantize, rotation


@pytest.fixture(scope="module")
def q4():
    return pipeline.build(4, 128)


@pytest.fixture(scope="module")
def q2():
    return pipeline.build(2, 128)


def test_record_sizes(q4, q2):
    x = np.random.default_rng(0).standard_normal((3, 128))
    e4 = pipeline.encode_keys(x, q4)
    assert e4["codes"].shape == (3, 64) and e4["n"].dtype == np.float32
    assert e4["codes"].shape[1] + e4["n"].itemsize == 68
    assert e4["qjl"].shape == (3, 16) and e4["gamma"].dtype == np.float32
    e2 = pipeline.encode_values(x, q2)
    assert e2["codes"].shape == (3, 32)
    # 3 bits: 48 B of codes; the Prod key record at a 4-bit budget (3-bit MSE codes +
    # 16 B of QJL signs + norm + gamma) is 72 B, the 4-bit value record 68 B
    qp = pipeline.build_prod(4, 128)
    ek, ev = pipeline.encode_keys(x, qp), pipeline.encode_values(x, qp)
    assert ek["codes"].shape == (3, 48) and ev["codes"].shape == (3, 64)
    assert ek["codes"].shape[1] + ek["qjl"].shape[1] + 4 + 4 == 72
    assert ek["idx"].max() < 8 and ev["idx"].max() < 16


def test_packing_layout_by_hand():
    idx = np.array([[1, 2, 15, 0, 7, 8, 3, 12]])
    assert list(quantize.pack_codes(idx, 4)[0]) == [0x21, 0x0F, 0x87, 0xC3]
    idx2 = np.array([[1, 2, 3, 0, 0, 3, 2, 1]])
    assert list(quantize.pack_codes(idx2, 2)[0]) == [0b00111001, 0b01101100]
    # 3 bits: sum_j idx_j << 3j = 0x1F58D1, little-endian bytes; coordinates 2 and 5
    # straddle a byte boundary
    idx3 = np.array([[1, 2, 3, 4, 5, 6, 7, 0]])
    assert list(quantize.pack_codes(idx3, 3)[0]) == [0xD1, 0x58, 0x1F]
    sig = np.array([[1, 0, 0, 0, 0, 0, 0, 1, 0, 1, 0, 0, 0, 0, 0, 0]])
    assert list(quantize.pack_bits(sig)[0]) == [0x81, 0x02]


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_roundtrip(bits):
    rs = np.random.default_rng(bits)
    idx = rs.integers(0, 1 << bits, size=(20, 128))
    assert np.array_equal(quantize.unpack_codes(quantize.pack_codes(idx, bits), bits, 128), idx)
    sig = rs.integers(0, 2, size=(20, 128))
    assert np.array_equal(quantize.unpack_bits(quantize.pack_bits(sig), 128), sig)


def test_quantize_is_nearest_level(q4):
    """Boundaries at level midpoints make the cell decision a nearest-level search."""
    y = np.random.default_rng(1).standard_normal(20000) * 0.2
    idx = quantize.quantize_indices(y, q4["boundaries"])
    lev = q4["levels"].astype(np.float64)
    brute = np.argmin(np.abs(y[:, None].astype(np.float32).astype(np.float64) - lev[None]), axis=1)
    bnd = q4["boundaries"].astype(np.float64)
    far = np.min(np.abs(y[:, None] - bnd[None]), axis=1) > 1e-6
    assert np.array_equal(idx[far], brute[far])
    # ties go to the lower cell; levels reproduce themselves
    assert np.array_equal(quantize.quantize_indices(q4["boundaries"], q4["boundaries"]), np.arange(15))
    assert np.array_equal(quantize.quantize_indices(q4["levels"], q4["boundaries"]), np.arange(16))


def test_zero_vector(q4):
    e = pipeline.encode_keys(np.zeros((1, 128)), q4)
    assert e["n"][0] == 0 and np.all(e["y"] == 0)
    assert np.all(e["idx"] == 7) and np.all(e["codes"] == 0x77)
    assert e["gamma"][0] == 0


@pytest.mark.parametrize("bits,rtol", [(4, 0.03), (3, 0.03), (2, 0.03)])
def test_mse_bound_on_random_unit_vectors(bits, rtol):
    """Mean ||u - u_hat||^2 over 10^4 random unit vectors is below the page's
    bound (sqrt(3) pi / 2) / 4^b and close to the Gaussian Lloyd-Max MSE."""
    q = pipeline.build(bits, 128)
    x = np.random.default_rng(10 + bits).standard_normal((10000, 128))
    u = x / np.linalg.norm(x, axis=1, keepdims=True)
    e = pipeline.encode_values(u, q)
    uh = quantize.reconstruct(e["n"], e["idx"], q["levels"], q["pi"])
    mse = float(np.mean(np.sum((u - uh) ** 2, axis=1)))
    assert mse <= np.sqrt(3) * np.pi / 2 / 4 ** bits
    lev, bnd, _, _ = codebook.lloyd_max_gaussian(bits)
    assert abs(mse / codebook.gaussian_mse(lev, bnd) - 1) < rtol


def test_reconstruction_cosine_on_outlier_keys(q4):
    """The standalone 4-bit quantizer keeps cosine >= 0.95 on Llama-like keys."""
    k, v = synth.kv_tensors(3, 2000, 1, 128)
    for x in (k[:, 0], v[:, 0]):
        e = pipeline.encode_values(x, q4)
        xh = quantize.reconstruct(e["n"], e["idx"], q4["levels"], q4["pi"])
        cos = np.sum(x * xh, 1) / np.linalg.norm(x, axis=1) / np.linalg.norm(xh, axis=1)
        assert cos.min() >= 0.95 and cos.mean() > 0.98


def test_gamma_is_residual_norm_in_original_frame(q4):
    x = np.random.default_rng(4).standard_normal((50, 128)) * 3
    e = pipeline.encode_keys(x, q4)
    xh = quantize.reconstruct(e["n"].astype(np.float64), e["idx"], q4["levels"], q4["pi"])
    # n is rounded to fp32 in storage; compare with the float64 residual norm
    n64 = np.linalg.norm(x, axis=1)
    xh64 = n64[:, None] * (q4["levels"].astype(np.float64)[e["idx"]] @ q4["pi"])
    r = x - xh64
    assert np.allclose(e["gamma"], np.linalg.norm(r, axis=1), rtol=2e-6)
    assert np.allclose(xh, xh64, rtol=1e-6)


def test_on_grid_residual_vanishes(q4):
    idx = np.random.default_rng(6).integers(0, 16, size=(5, 128))
    y = q4["levels"].astype(np.float64)[idx]
    assert np.array_equal(quantize.quantize_indices(y, q4["boundaries"]), idx)
    r = quantize.qjl_residual(y, idx, q4["levels"])
    assert np.all(r == 0)
    sig = np.random.default_rng(7).integers(0, 2, size=(5, 128))
    est = quantize.qjl_inner_product(np.ones(128), sig, np.zeros(5, np.float32), q4["s"])
    assert np.all(est == 0)


def test_qjl_unbiased_with_closed_form_variance():
    """E over Gaussian S of gamma sqrt(pi/2)/m <S q, sign(S r)> equals <q, r>; its
    variance is (pi/2 ||q||^2 ||r||^2 - <q,r>^2) / m (derived from
    E[<s,q> sign(<s,r>)] = sqrt(2/pi) <q,r>/||r|| for s ~ N(0, I))."""
    d = m = 128
    rs = np.random.default_rng(11)
    q = rs.standard_normal(d)
    r = 0.3 * q / np.linalg.norm(q) * 2 + rs.standard_normal(d) * 0.05
    gamma = np.float32(np.linalg.norm(r))
    N = 20000
    est = np.empty(N)
    for i in range(N):
        s = rs.standard_normal((m, d))
        sig = (s @ r >= 0).astype(np.int64)[None]
        est[i] = quantize.qjl_inner_product(q, sig, np.array([gamma]), s)[0]
    truth = float(q @ r) * float(gamma) / np.linalg.norm(r)
    se = est.std() / np.sqrt(N)
    assert abs(est.mean() - truth) < 4 * se
    var = (np.pi / 2 * (q @ q) * float(gamma) ** 2 - truth ** 2) / m
    assert abs(est.var() / var - 1) < 0.05


def test_keys_reuse_value_codes(q4):
    """A key's MSE part is exactly the value encoding of the same vector."""
    x = np.random.default_rng(8).standard_normal((30, 128))
    ek, ev = pipeline.encode_keys(x, q4), pipeline.encode_values(x, q4)
    assert np.array_equal(ek["codes"], ev["codes"]) and np.array_equal(ek["n"], ev["n"])


def test_wht_variant_encodes_with_the_dense_operator():
    q = pipeline.build(4, 128, rot=pipeline.WHT, rot_seed=9)
    x = np.random.default_rng(9).standard_normal((40, 128))
    n, y = quantize.rotate_unit(x, q["pi"])
    yf = rotation.fwht_rotate(x / np.linalg.norm(x, axis=1, keepdims=True), q["signs"])
    assert np.allclose(y, yf, atol=1e-7)  # fp32 storage of +-1/sqrt(d) entries
