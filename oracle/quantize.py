"""Per-vector TurboQuant encoding and the QJL residual signs (oracle).

Follows the four steps of the "FlashQuant" page, section "TurboQuant":
(1) split x into its L2 norm and unit direction, (2) rotate, (3) Lloyd-Max
scalar quantization of every rotated coordinate, (4) pack the 4-bit indices two
per byte and keep the norm in fp32. Packing at 2 bits (four per byte) and the
fp32 norm side channel follow the "TurboQuant" blog, "Couche 3" and
"Couche 4". The QJL step for keys follows the "FlashQuant" page, section
"QJL": r = k - k_mse, gamma = ||r||, one sign bit per projection of r.

Readings (the pages fix none of these):
* n = 0 gives u = 0 (so y = 0);
* idx_j = #{i : boundary_i < y_j}, the decision taken on fp32(y_j) against the
  fp32 boundaries (a value equal to a boundary goes to the lower cell);
* the indices of a vector form one little-endian bit stream: coordinate j takes
  bits b*j .. b*j + b-1 of it, bit 8k+i of the stream being bit i of byte k. At 4
  bits that is coordinate 2k in the low nibble of byte k and 2k+1 in the high
  nibble; at 2 bits coordinate 4k+i in bits 2i..2i+1 of byte k; at 3 bits (the
  codebook variant of the "TurboQuant" blog's 3-bit remark) eight coordinates fill
  three bytes, some indices straddling two bytes;
* QJL works in the rotated frame: r~ = y - c[idx] (unit scale), gamma = n ||r~||
  (equal to ||k - k_mse|| because the rotation is orthogonal), p = S r~ with m = d
  Gaussian rows, sigma_i = [p_i >= 0] (sign(0) = +1), bit i of byte j = sigma_{8j+i}.
"""
import numpy as np


def norms(x: np.ndarray) -> np.ndarray:
    """||x|| per row, float64."""
    x = np.asarray(x, dtype=np.float64)
    return np.sqrt(np.sum(x * x, axis=-1))


def rotate_unit(x: np.ndarray, pi: np.ndarray):
    """Steps 1-2: n = ||x||, u = x / n (0 when n = 0), y = Pi u. Returns (n, y), float64."""
    x = np.asarray(x, dtype=np.float64)
    n = norms(x)
    safe = np.where(n > 0, n, 1.0)
    u = np.where((n > 0)[:, None], x / safe[:, None], 0.0)
    y = u @ pi.T
    return n, y


def quantize_indices(y: np.ndarray, boundaries32: np.ndarray) -> np.ndarray:
    """Step 3: index of the cell of each coordinate, decided in fp32.

    idx = number of boundaries strictly below fp32(y).
    """
    y32 = np.asarray(y, dtype=np.float32)
    b32 = np.asarray(boundaries32, dtype=np.float32)
    return np.searchsorted(b32, y32, side="left").astype(np.int64)


def pack_codes(idx: np.ndarray, bits: int) -> np.ndarray:
    """Step 4: pack [N, d] indices into [N, d * bits / 8] bytes: the little-endian bit
    stream in which coordinate j occupies bits bits*j .. bits*j + bits - 1."""
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    stream = np.zeros((n, d * bits), dtype=np.int64)  # one entry per bit of the stream
    for i in range(bits):
        stream[:, i::bits] = (idx >> i) & 1
    grp = stream.reshape(n, d * bits // 8, 8)
    out = np.zeros((n, d * bits // 8), dtype=np.int64)
    for i in range(8):
        out |= grp[:, :, i] << i
    return out.astype(np.uint8)


def unpack_codes(codes: np.ndarray, bits: int, d: int) -> np.ndarray:
    """Inverse of pack_codes: bytes [N, d*bits/8] -> indices [N, d]."""
    codes = np.asarray(codes, dtype=np.int64)
    n = codes.shape[0]
    stream = np.stack([(codes >> i) & 1 for i in range(8)], axis=-1).reshape(n, d * bits)
    idx = np.zeros((n, d), dtype=np.int64)
    for i in range(bits):
        idx |= stream[:, i::bits] << i
    return idx


def pack_bits(sig: np.ndarray) -> np.ndarray:
    """[N, m] booleans -> [N, m/8] bytes, bit i of byte j = sig[8j + i]."""
    sig = np.asarray(sig, dtype=np.int64)
    n, m = sig.shape
    grp = sig.reshape(n, m // 8, 8)
    out = np.zeros((n, m // 8), dtype=np.int64)
    for i in range(8):
        out |= grp[:, :, i] << i
    return out.astype(np.uint8)


def unpack_bits(packed: np.ndarray, m: int) -> np.ndarray:
    """Inverse of pack_bits: [N, m/8] bytes -> [N, m] in {0, 1}."""
    packed = np.asarray(packed, dtype=np.int64)
    parts = [(packed >> i) & 1 for i in range(8)]
    return np.stack(parts, axis=-1).reshape(packed.shape[0], m)


def qjl_residual(y: np.ndarray, idx: np.ndarray, levels32: np.ndarray):
    """r~ = y - c[idx] in the rotated unit frame (float64)."""
    return np.asarray(y, dtype=np.float64) - np.asarray(levels32, dtype=np.float64)[idx]


def qjl_signs(p: np.ndarray) -> np.ndarray:
    """sigma = [p >= 0], decided on fp32(p)."""
    return (np.asarray(p, dtype=np.float32) >= 0).astype(np.int64)


def encode(x, pi, levels32, boundaries32, bits, s=None):
    """Full per-vector encoding of the rows of x (float64 math, fp32 storage).

    Returns a dict with n (fp32), y (float64 rotated unit coordinates), idx,
    codes (packed bytes); and when the QJL matrix s is given (keys): r (float64),
    gamma (fp32), p (float64 projections), sig (0/1), qjl (packed bytes).
    """
    n, y = rotate_unit(x, pi)
    idx = quantize_indices(y, boundaries32)
    out = {
        "n": n.astype(np.float32),
        "y": y,
        "idx": idx,
        "codes": pack_codes(idx, bits),
    }
    if s is not None:
        r = qjl_residual(y, idx, levels32)
        gamma = n * norms(r)
        p = r @ s.T
        sig = qjl_signs(p)
        out.update(r=r, gamma=gamma.astype(np.float32), p=p, sig=sig, qjl=pack_bits(sig))
    return out


def reconstruct(n32, idx, levels32, pi):
    """x_hat = n * Pi^T c[idx] (float64): the MSE reconstruction in the original frame."""
    c = np.asarray(levels32, dtype=np.float64)[idx]
    return np.asarray(n32, dtype=np.float64)[:, None] * (c @ pi)


def qjl_inner_product(q_rot, sig, gamma32, s):
    """QJL estimate of <q, k - k_mse> ("FlashQuant" page, section "QJL").

    gamma * sqrt(pi/2) / m * <S q~, 2 sigma - 1>, with q~ the rotated query and
    m the number of rows of S. q_rot: [d] or [Q, d]; sig: [T, m]; returns [..., T].
    """
    m = s.shape[0]
    qs = np.asarray(q_rot, dtype=np.float64) @ s.T
    pm = 2.0 * np.asarray(sig, dtype=np.float64) - 1.0
    return np.asarray(gamma32, dtype=np.float64) * np.sqrt(np.pi / 2.0) / m * (qs @ pm.T)
