"""Pins for the oracle's block codec (CPU only).

The checks do not re-type the oracle's formulas: reconstructions are rebuilt
here from the Kronecker form of H, codes are checked by brute force over every
code vector on d = 4 / 8 blocks, and the statistics are compared with the
Lloyd-Max distortion.
"""

import itertools
import math

import numpy as np
import pytest

from oracle import codec, lloyd_max, hadamard
from oracle.numerics import round_fp16


def _kron_H(d):
    H = np.array([[1.0]])
    while H.shape[0] < d:
        H = np.block([[H, H], [H, -H]])
    return H


def _recon(codes, n, D, bits):
    """x_hat = n R^T c / sqrt(d) with R = H diag(D)/sqrt(d), built independently."""
    d = codes.shape[-1]
    c, _, _ = lloyd_max.codebook(bits)
    R = _kron_H(d) * D[None, :] / math.sqrt(d)
    return n * (c[codes] @ R) / math.sqrt(d)


@pytest.mark.parametrize("d,bits", [(4, 1), (4, 2), (4, 3), (8, 1), (8, 2)])
def test_brute_force_nearest_reconstruction(d, bits):
    rng = np.random.default_rng(100 + d * 10 + bits)
    L = 1 << bits
    all_codes = np.array(list(itertools.product(range(L), repeat=d)), dtype=np.int64)
    for trial in range(12):
        D = rng.choice([-1.0, 1.0], size=d)
        x = rng.standard_normal(d)
        x /= np.linalg.norm(x)            # norm 1: exactly representable in fp16, n16 = n
        q = codec.quantize(x[None, :], bits, D)
        assert q["n16"][0] == 1.0
        recons = _recon(all_codes, 1.0, D, bits)
        err = np.sum((recons - x[None, :]) ** 2, axis=1)
        best = all_codes[np.argmin(err)]
        assert np.array_equal(q["codes"][0].astype(np.int64), best)
        # dequantize agrees with the independent reconstruction
        assert np.allclose(codec.dequantize(q["codes"], q["n16"], bits, D)[0],
                           _recon(q["codes"][0].astype(np.int64), 1.0, D, bits), atol=1e-14)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 8])
def test_codes_are_per_coordinate_nearest_centroid(bits):
    d = 64
    rng = np.random.default_rng(bits)
    D = rng.choice([-1.0, 1.0], size=d)
    x = rng.standard_normal((200, d)) * 0.02
    q = codec.quantize(x, bits, D)
    c, _, _ = lloyd_max.codebook(bits)
    dist = np.abs(q["y"][..., None] - c[None, None, :])
    nearest = np.argmin(dist, axis=-1)
    near_b, _ = codec.boundary_distance(q["y"], bits)
    ok = near_b > 1e-9     # a decision within fp32 rounding of a boundary may go either way
    assert np.array_equal(q["codes"][ok], nearest[ok])
    # y is sqrt(d) R x / ||x||
    R = _kron_H(d) * D[None, :] / math.sqrt(d)
    y_ref = math.sqrt(d) * (x @ R.T) / np.linalg.norm(x, axis=1, keepdims=True)
    assert np.allclose(q["y"], y_ref, atol=1e-12)


@pytest.mark.parametrize("bits,d", [(2, 128), (3, 128), (4, 128), (5, 128), (4, 64), (3, 256)])
def test_round_trip_distortion_matches_lloyd_max(bits, d):
    rng = np.random.default_rng(bits * 1000 + d)
    D = rng.choice([-1.0, 1.0], size=d)
    x = rng.standard_normal((3000, d))
    q = codec.quantize(x, bits, D)
    rel = codec.mse_per_coordinate(x, q["codes"], q["n16"], bits, D)
    _, _, mse = lloyd_max.codebook(bits)
    assert abs(np.mean(rel) - mse) < 0.04 * mse


def test_norms_are_fp16_of_l2_norm():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((100, 128)) * 10.0 ** rng.integers(-3, 3, (100, 1))
    D = np.ones(128)
    q = codec.quantize(x, 4, D)
    assert np.array_equal(q["n16"], np.linalg.norm(x, axis=1).astype(np.float16).astype(np.float64))


@pytest.mark.parametrize("bits", [1, 2, 3, 5])
def test_zero_block(bits):
    d = 128
    D = np.random.default_rng(0).choice([-1.0, 1.0], size=d)
    G = np.random.default_rng(1).standard_normal((64, d))
    x = np.zeros((1, d))
    q = codec.quantize(x, bits, D)
    assert q["n16"][0] == 0.0
    assert np.all(q["codes"] == (1 << (bits - 1)) - 1)
    assert np.all(codec.dequantize(q["codes"], q["n16"], bits, D) == 0.0)
    r = codec.qjl_residual(x, q["codes"], q["n16"], bits, D, G)
    assert r["rnorm16"][0] == 0.0 and np.all(r["bits"] == 0)


def test_one_hot_block_maps_to_unit_coordinates():
    d, bits = 128, 4
    rng = np.random.default_rng(9)
    D = rng.choice([-1.0, 1.0], size=d)
    j = 17
    x = np.zeros((1, d))
    x[0, j] = -3.0
    q = codec.quantize(x, bits, D)
    # y_i = H_ij D_j sign(x_j): every coordinate is +-1
    expect_y = _kron_H(d)[:, j] * D[j] * -1.0
    assert np.allclose(q["y"][0], expect_y, atol=1e-14)
    _, beta, _ = lloyd_max.codebook(bits)
    code_pos, code_neg = int(np.sum(1.0 > beta)), int(np.sum(-1.0 > beta))
    assert np.array_equal(q["codes"][0], np.where(expect_y > 0, code_pos, code_neg).astype(np.uint8))


def test_power_of_two_scaling_keeps_codes():
    rng = np.random.default_rng(12)
    d, bits = 128, 5
    D = rng.choice([-1.0, 1.0], size=d)
    x = rng.standard_normal((50, d))
    a = codec.quantize(x, bits, D)
    b = codec.quantize(x * 8.0, bits, D)
    assert np.array_equal(a["codes"], b["codes"])
    assert np.array_equal(a["n16"] * 8.0, b["n16"])


def test_idempotent_away_from_boundaries():
    rng = np.random.default_rng(13)
    d, bits = 128, 4
    D = rng.choice([-1.0, 1.0], size=d)
    x = rng.standard_normal((200, d))
    a = codec.quantize(x, bits, D)
    xhat = codec.dequantize(a["codes"], a["n16"], bits, D)
    b = codec.quantize(xhat, bits, D)
    dist, _ = codec.boundary_distance(b["y"], bits)
    ok = dist > 1e-6
    assert ok.mean() > 0.999
    assert np.array_equal(a["codes"][ok], b["codes"][ok])


def test_residual_projection_identities():
    rng = np.random.default_rng(14)
    d, bits, m = 128, 3, 64
    D = rng.choice([-1.0, 1.0], size=d)
    G = rng.standard_normal((m, d))
    x = rng.standard_normal((20, d))
    q = codec.quantize(x, bits, D)
    out = codec.qjl_residual(x, q["codes"], q["n16"], bits, D, G)
    # r is x minus the independent reconstruction
    r_ref = x - _recon(q["codes"].astype(np.int64), q["n16"][:, None], D, bits)
    assert np.allclose(out["r"], r_ref, atol=1e-13)
    assert np.allclose(out["rnorm"], np.linalg.norm(r_ref, axis=1), rtol=1e-13)
    assert np.array_equal(out["rnorm16"], round_fp16(out["rnorm"]))
    # p is G applied to r itself, one dot product per row of G
    for i in (0, 7, m - 1):
        for b in (0, 19):
            assert abs(out["p"][b, i] - sum(G[i, e] * r_ref[b, e] for e in range(d))) < 1e-12
    # and it is not G applied to the rotated residual R r
    R = _kron_H(d) * D[None, :] / math.sqrt(d)
    assert not np.allclose(out["p"], (r_ref @ R.T) @ G.T, atol=1e-3)
    bits_unpacked = (out["bits"][:, :, None] >> np.arange(8)) & 1
    assert np.array_equal(bits_unpacked.reshape(20, m).astype(bool), out["p"] > 0)


def test_storage_accounting():
    # codes-only payload: 1 byte per coordinate + fp16 norm per block
    assert codec.storage_bytes_per_block(128) == 130
    assert codec.storage_bytes_per_block(128, m=64) == 130 + 8 + 2


# --- packed codes ---------------------------------------------------------------------
# eliza quantization README, TurboQuant, "Algorithm in one paragraph", step 4: indices are
# bit-packed into bytes, two per byte at 4 bits, four per byte at 2 bits.

def test_pack_codes_hand_fixture():
    """Bytes worked out by hand from the stated bit order (first index, lowest bits)."""
    four = codec.pack_codes(np.array([[1, 2, 3, 15, 0, 7, 8, 9]]), 4)
    assert four.tolist() == [[0x21, 0xF3, 0x70, 0x98]]
    two = codec.pack_codes(np.array([[0, 1, 2, 3, 3, 2, 1, 0]]), 2)
    assert two.tolist() == [[0xE4, 0x1B]]
    three = codec.pack_codes(np.array([[5, 6, 7, 1, 0, 2, 4, 3]]), 3)
    assert three.tolist() == [[0xF5, 0x03, 0x71]]
    one = codec.pack_codes(np.array([[1, 0, 0, 1, 1, 1, 0, 1]]), 1)
    assert one.tolist() == [[0xB9]]


@pytest.mark.parametrize("bits", range(1, 9))
@pytest.mark.parametrize("d", [8, 64, 128, 512])
def test_pack_codes_against_numpy_packbits(bits, d):
    """The packed stream equals numpy's little-endian packbits of the explicit bit matrix;
    the size is d * bits / 8 bytes (d / 2 at 4 bits, d / 4 at 2 bits); unpack inverts."""
    rng = np.random.default_rng(bits * 1000 + d)
    codes = rng.integers(0, 1 << bits, size=(37, d))
    bitmat = ((codes[:, :, None] >> np.arange(bits)) & 1).reshape(37, d * bits).astype(np.uint8)
    ref = np.packbits(bitmat, axis=1, bitorder="little")
    got = codec.pack_codes(codes, bits)
    assert got.shape == (37, d * bits // 8)
    assert np.array_equal(got, ref)
    assert np.array_equal(codec.unpack_codes(got, bits, d), codes.astype(np.uint8))


def test_pack_codes_rejects_bad_input():
    with pytest.raises(ValueError):
        codec.pack_codes(np.array([[16, 0]]), 4)
    with pytest.raises(ValueError):
        codec.pack_codes(np.zeros((1, 3)), 3)


# ---- block sizes that are not powers of two (block-diagonal rotation) ------------------------

@pytest.mark.parametrize("d,bits", [(192, 4), (320, 3), (96, 2), (576, 5)])
def test_block_diagonal_codec_matches_per_block_rotation(d, bits):
    """y = sqrt(d) R x / ||x|| with R the block-diagonal rotation, each block rotated by its own
    power-of-two H (the pinned single-block rotation); dequantize = n16 R^T c / sqrt(d)."""
    from oracle import hadamard, lloyd_max
    rng = np.random.default_rng(d * 3 + bits)
    D = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    x = rng.standard_normal((5, d)) * np.exp(rng.standard_normal((5, 1)))
    q = codec.quantize(x, bits, D)
    o = 0
    y = np.zeros_like(x)
    for s in hadamard.block_sizes(d):
        y[:, o:o + s] = math.sqrt(d) * (x[:, o:o + s] @ hadamard.rotation(s, D[o:o + s]).T) / q["norm"][:, None]
        o += s
    np.testing.assert_allclose(q["y"], y, atol=1e-12)
    c = lloyd_max.codebook(bits)[0][q["codes"].astype(np.int64)]
    ref = np.zeros_like(x)
    o = 0
    for s in hadamard.block_sizes(d):
        ref[:, o:o + s] = (c[:, o:o + s] @ hadamard.rotation(s, D[o:o + s])) * q["n16"][:, None] / math.sqrt(d)
        o += s
    np.testing.assert_allclose(codec.dequantize(q["codes"], q["n16"], bits, D), ref, atol=1e-12)


def test_block_diagonal_round_trip_mse_near_table():
    """Isotropic Gaussian blocks of d = 192: the rotated coordinates are close to N(0, 1), so
    the per-coordinate error of a 4-bit round trip is close to the Lloyd-Max table MSE."""
    from oracle import lloyd_max
    d, bits = 192, 4
    rng = np.random.default_rng(11)
    D = np.where(rng.random(d) < 0.5, -1.0, 1.0)
    x = rng.standard_normal((4000, d))
    q = codec.quantize(x, bits, D)
    xhat = codec.dequantize(q["codes"], q["n16"], bits, D)
    mse = np.mean(np.sum((x - xhat) ** 2, axis=1) / np.sum(x ** 2, axis=1))
    table = lloyd_max.codebook(bits)[2]
    assert abs(mse - table) < 0.05 * table


# ------------------------------------------------------------------ decision precision pins

def _brute_boundary(y, beta):
    """Nearest boundary by a scan over every boundary, and the code across it."""
    dist = np.full(y.shape, np.inf)
    other = np.zeros(y.shape, dtype=np.int64)
    for idx, v in np.ndenumerate(y):
        code = sum(1 for b in beta if v > b)          # strict >: a coordinate on a boundary is below it
        best, bj = np.inf, -1
        for j, b in enumerate(beta):
            if abs(v - b) < best:
                best, bj = abs(v - b), j
        dist[idx] = best
        other[idx] = code + 1 if v <= beta[bj] else code - 1
    return dist, other


@pytest.mark.parametrize("bits", [1, 2, 3, 5, 8])
def test_boundary_distance_against_a_scan(bits):
    """Distance and far-side code of ``boundary_distance`` equal a scan over every boundary, for
    random coordinates, coordinates exactly on a boundary and one fp32 ulp to either side."""
    _, beta, _ = lloyd_max.codebook(bits)
    rng = np.random.default_rng(50 + bits)
    ys = [rng.standard_normal(400) * 1.5, beta.copy()]
    b32 = beta.astype(np.float32)
    ys.append(np.nextafter(b32, np.float32(np.inf)).astype(np.float64))
    ys.append(np.nextafter(b32, np.float32(-np.inf)).astype(np.float64))
    ys.append(np.array([-50.0, 50.0, 0.0]))
    y = np.concatenate(ys)
    dist, other = codec.boundary_distance(y, bits)
    bdist, bother = _brute_boundary(y, beta)
    np.testing.assert_array_equal(dist, bdist)
    np.testing.assert_array_equal(other.astype(np.int64), bother)
    # on a boundary: distance 0, the far side is the upper code
    nb = len(beta)
    d_on, o_on = codec.boundary_distance(beta, bits)
    assert np.all(d_on == 0.0) and np.array_equal(o_on.astype(np.int64), np.arange(1, nb + 1))


def test_codes_decided_in_float64():
    """Coordinates 1e-9 above or below a boundary -- far below fp32 resolution -- take the code of
    their float64 side.  The block is built backwards from a target t with ||t||^2 = d:
    x = D * (H t) / d gives H (D * x) = t and ||x|| = ||t|| / sqrt(d), so y = t up to float64
    rounding (~1e-15)."""
    bits, d = 3, 32
    _, beta, _ = lloyd_max.codebook(bits)
    rng = np.random.default_rng(7)
    for trial in range(20):
        D = rng.choice([-1.0, 1.0], size=d)
        j = rng.integers(0, len(beta), size=8)
        delta = rng.choice([-1e-9, 1e-9], size=8)
        t = np.empty(d)
        t[:8] = beta[j] + delta
        t[8:d - 1] = rng.choice([-0.3, 0.25, -0.2], size=d - 9)     # away from every boundary
        rest = d - np.sum(t[:d - 1] ** 2)
        assert rest > 0
        t[d - 1] = math.sqrt(rest)
        assert np.min(np.abs(t[d - 1] - beta)) > 1e-3
        H = _kron_H(d)
        x = D * (H @ t) / d
        q = codec.quantize(x[None, :], bits, D)
        assert np.max(np.abs(q["y"][0] - t)) < 1e-13
        expect = np.where(delta > 0, j + 1, j)
        np.testing.assert_array_equal(q["codes"][0, :8].astype(np.int64), expect)
        # fp32 cannot separate these coordinates from their boundary
        assert np.all(np.abs(np.float32(t[:8]).astype(np.float64) - beta[j]) < 2e-7)
