"""Oracle end-to-end helpers: build the quantizer from seeds, compress into a paged cache.

Composition only; the arithmetic lives in codebook, rotation, quantize and
attention. Keys get MSE codes plus QJL signs, values MSE codes only
("FlashQuant" page, "使用方式": MSE mode for values, inner-product mode for
keys). K and V of one layer share the rotation (a reading: the pages do not
say).
"""
import numpy as np

from . import codebook, paged, quantize, rotation

HAAR = 0
WHT = 1


GAUSSIAN, SPHERE = "gaussian", "sphere"


def build(bits, head_dim, rot=HAAR, rot_seed=1, qjl_seed=2, qjl_dim=None, law=GAUSSIAN, key_bits=None):
    """All stored parameters of one layer's quantizer.

    Returns levels32, boundaries32, pi (fp32 operator as float64), signs (WHT
    only, else None), s (fp32 QJL matrix as float64, m x d). law: the codebook's
    model of a rotated coordinate, GAUSSIAN (N(0, 1/d)) or SPHERE (the exact
    spherical marginal). key_bits: the width of the keys' MSE codes when it differs
    from the values' (key_levels / key_boundaries are then that width's codebook;
    otherwise they are the values' own).
    """
    def book(b):
        if law == GAUSSIAN:
            return codebook.scaled_codebook(b, head_dim)
        if law == SPHERE:
            return codebook.sphere_codebook(b, head_dim)
        raise ValueError(law)

    lev, bnd = book(bits)
    kb = bits if key_bits is None else key_bits
    klev, kbnd = (lev, bnd) if kb == bits else book(kb)
    m = head_dim if qjl_dim is None else qjl_dim
    if rot == HAAR:
        pi = rotation.stored(rotation.haar_rotation(rot_seed, head_dim))
        sg = None
    else:
        sg = rotation.wht_signs(rot_seed, head_dim)
        pi = rotation.stored(rotation.wht_matrix(sg))
    s = rotation.stored(rotation.qjl_matrix(qjl_seed, m, head_dim))
    return {"bits": bits, "d": head_dim, "rot": rot, "levels": lev, "boundaries": bnd,
            "key_bits": kb, "key_levels": klev, "key_boundaries": kbnd,
            "pi": pi, "signs": sg, "s": s, "m": m, "law": law}


def build_prod(bits, head_dim, **kw):
    """The inner-product ("Prod") mode of the quantizer at a budget of `bits` bits per
    key coordinate ("FlashQuant" page, "架构设计": the quantizer's MSE / Prod modes):
    keys get (bits - 1)-bit MSE codes plus the 1-bit QJL signs of their residual,
    values keep bits-bit MSE codes. (The pages name the mode; the (b - 1) + 1 split of
    the budget is TurboQuant's definition of its inner-product quantizer.)"""
    return build(bits, head_dim, key_bits=bits - 1, **kw)


def encode_keys(x, q):
    return quantize.encode(x, q["pi"], q["key_levels"], q["key_boundaries"], q["key_bits"], s=q["s"])


def encode_keys_mse(x, q):
    """Keys without QJL fields: the MSE encoding at the keys' width."""
    return quantize.encode(x, q["pi"], q["key_levels"], q["key_boundaries"], q["key_bits"])


def encode_values(x, q):
    return quantize.encode(x, q["pi"], q["levels"], q["boundaries"], q["bits"])


def compress(cache, k, v, slot_mapping, q, with_qjl=True):
    """Encode k, v ([T, Hkv, d]) and store them at slot_mapping ([T]).

    Returns the per-head encodings (list over heads of (k_enc, v_enc)) so that
    tests can look at y, p and the codes directly.
    """
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    T, Hkv, d = k.shape
    encs = []
    for h in range(Hkv):
        ke = encode_keys(k[:, h], q) if with_qjl else encode_keys_mse(k[:, h], q)
        ve = encode_values(v[:, h], q)
        paged.write(cache, slot_mapping, h, ke, ve)
        encs.append((ke, ve))
    return encs
