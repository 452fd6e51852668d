"""Pins of the CPU oracle against facts fixed by the pages and by mathematics (no GPU).

Each test is chosen so that a plausible mistake in the oracle (a dropped term, a wrong sign or
index, a transposed operand, a wrong normalisation) fails at least one of them. None of them
re-types the oracle's own formula: they use closed forms, numerical integration, library
routines (scipy's Hadamard matrix, brute-force argmin), invariants and printed values.
"""
import math
import os

import numpy as np
import pytest
import scipy.integrate
import scipy.linalg
import scipy.stats
import torch

import oracle
from kv_cache_compression_vector_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_rows(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _bf16(a):
    return synth.bf16_bits(torch.as_tensor(np.asarray(a, np.float32)).to(torch.bfloat16))


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------------------------
# Lloyd-Max table


@pytest.mark.parametrize("row", _golden_rows("lloyd_max_gaussian.txt"), ids=lambda r: f"b{r[0]}")
def test_gaussian_table_matches_printed_values(row):
    bits, tol, mse = int(row[0]), float(row[1]), float(row[2])
    pos = np.array([float(v) for v in row[3:]])
    c64, c32 = oracle.gaussian_table(bits)
    L = 1 << bits
    assert np.all(np.diff(c64) > 0)
    np.testing.assert_allclose(c64[L // 2:], pos, atol=tol)
    np.testing.assert_array_equal(c32, -c32[::-1])  # exact antisymmetry of the stored table


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_gaussian_table_satisfies_lloyd_conditions_by_quadrature(bits):
    """Centroid = conditional mean of its cell, computed by numerical integration (scipy)."""
    c64, _ = oracle.gaussian_table(bits)
    L = 1 << bits
    edges = np.concatenate([[-np.inf], 0.5 * (c64[:-1] + c64[1:]), [np.inf]])
    pdf = scipy.stats.norm.pdf
    for k in range(L):
        num = scipy.integrate.quad(lambda x: x * pdf(x), edges[k], edges[k + 1], epsabs=1e-13)[0]
        den = scipy.integrate.quad(pdf, edges[k], edges[k + 1], epsabs=1e-13)[0]
        assert abs(num / den - c64[k]) < 1e-8


@pytest.mark.parametrize("row", _golden_rows("lloyd_max_gaussian.txt"), ids=lambda r: f"b{r[0]}")
def test_gaussian_table_mse_by_quadrature(row):
    bits, mse_printed = int(row[0]), float(row[2])
    c64, _ = oracle.gaussian_table(bits)
    edges = np.concatenate([[-np.inf], 0.5 * (c64[:-1] + c64[1:]), [np.inf]])
    mse = sum(scipy.integrate.quad(lambda x, c=c: (x - c) ** 2 * scipy.stats.norm.pdf(x),
                                   edges[k], edges[k + 1], epsabs=1e-13)[0]
              for k, c in enumerate(c64))
    assert mse == pytest.approx(mse_printed, rel=2e-3)
    if bits == 1:
        assert c64[1] == pytest.approx(math.sqrt(2 / math.pi), abs=1e-12)
        assert mse == pytest.approx(1 - 2 / math.pi, abs=1e-9)


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_thresholds_reproduce_brute_force_nearest_centroid(bits):
    """code = #{t_k < z} must equal argmin_k |z - c_k| (ties to the lower index) wherever z is
    not within 1e-6 of a threshold."""
    _, c32 = oracle.gaussian_table(bits)
    t = oracle.thresholds(c32)
    rng = np.random.default_rng(bits)
    z = np.concatenate([rng.normal(size=20000) * 1.5, rng.uniform(-4, 4, 20000)])
    by_count = (z[:, None] > t[None, :].astype(np.float64)).sum(1)
    dist = np.abs(z[:, None] - c32[None, :].astype(np.float64))
    by_argmin = np.argmin(dist, axis=1)  # first minimum = lower index on ties
    far = np.min(np.abs(z[:, None] - t[None, :]), axis=1) > 1e-6
    np.testing.assert_array_equal(by_count[far], by_argmin[far])


# ---------------------------------------------------------------------------------------------
# Signs


def test_signs_follow_splitmix64_published_outputs():
    """SplitMix64 from seed 0 emits 0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F
    (the reference splitmix64.c stream); the sign is the top bit of each output."""
    raw = oracle.splitmix64(0, 3)
    np.testing.assert_array_equal(raw, np.array([0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4,
                                                 0x06C45D188009454F], np.uint64))
    s = oracle.signs(0, 3)
    np.testing.assert_array_equal(s, [-1, 1, 1])


def test_signs_balanced_and_seed_dependent():
    a = oracle.signs(42, 4096)
    b = oracle.signs(43, 4096)
    assert set(np.unique(a)) == {-1, 1}
    assert abs(int(a.sum())) < 4 * math.sqrt(4096)
    assert (a != b).mean() > 0.4
    np.testing.assert_array_equal(oracle.signs(42, 100), a[:100])  # prefix-stable stream


# ---------------------------------------------------------------------------------------------
# Hadamard rotation


@pytest.mark.parametrize("m", [32, 64, 128, 256, 512])
def test_fwht_equals_sylvester_matrix(m):
    """Butterfly on the identity rows gives scipy's Sylvester Hadamard matrix; H H^T = m I."""
    H = oracle.fwht_rows(np.eye(m))
    np.testing.assert_array_equal(H, scipy.linalg.hadamard(m).astype(np.float64))
    np.testing.assert_array_equal(H @ H.T, m * np.eye(m))


def test_fwht_preserves_norm_up_to_m():
    rng = np.random.default_rng(0)
    v = rng.normal(size=(16, 128))
    u = oracle.fwht_rows(v)
    np.testing.assert_allclose((u * u).sum(1), 128 * (v * v).sum(1), rtol=1e-12)


# ---------------------------------------------------------------------------------------------
# Encode: independent formulation (explicit matrix, brute-force argmin)


def _independent_codes(x_bits, D, bits, seed, c32):
    v = _bf16_to_f64(x_bits)
    s = oracle.signs(seed, D).astype(np.float64)
    u = (scipy.linalg.hadamard(D) @ (s[None, :] * v).T).T
    n = np.sqrt((v * v).sum(1))
    z = u / n[:, None]
    codes = np.argmin(np.abs(z[..., None] - c32.astype(np.float64)), axis=-1)
    return codes, n, z


@pytest.mark.parametrize("D,bits", [(64, 1), (128, 2), (128, 3), (256, 4), (512, 4), (512, 2)])
def test_encode_matches_matrix_hadamard_and_argmin(D, bits):
    x = _bf16(np.random.default_rng(D + bits).normal(size=(64, D)))
    cd = oracle.Codec(D, bits, seed=42)
    out = oracle.encode(cd, x)
    codes, n, z = _independent_codes(x, D, bits, 42, cd.centroids)
    ok = out["flags"] == 0
    np.testing.assert_array_equal(out["codes"][ok], codes[ok])
    np.testing.assert_allclose(out["norms"], n, rtol=1e-14)
    np.testing.assert_allclose(out["z"], z, atol=1e-12)
    # the stored norm is the f32 of the norm
    for row in range(4):
        _, nrm32 = oracle.unpack_codes(cd.m, bits, out["records"][row])
        assert nrm32 == np.float32(n[row])


def test_encode_scale_by_power_of_two_is_exact():
    x = np.random.default_rng(1).normal(size=(32, 128)).astype(np.float32)
    cd = oracle.Codec(128, 3, seed=7)
    a = oracle.encode(cd, _bf16(x))
    b = oracle.encode(cd, _bf16(x * 8.0))
    np.testing.assert_array_equal(a["codes"], b["codes"])
    np.testing.assert_array_equal(b["norms"], 8.0 * a["norms"])


def test_encode_sign_mirror():
    x = np.random.default_rng(2).normal(size=(32, 128)).astype(np.float32)
    cd = oracle.Codec(128, 3, seed=7)
    a = oracle.encode(cd, _bf16(x))
    b = oracle.encode(cd, _bf16(-x))
    ok = (a["flags"] == 0) & (b["flags"] == 0)
    np.testing.assert_array_equal(b["codes"][ok], 7 - a["codes"][ok])


def test_code_frequencies_match_gaussian_cell_masses():
    """On iid Gaussian rows the rotated, normalised coordinates are ~N(0,1), so code k must
    occur with the N(0,1) mass of cell k."""
    x = np.random.default_rng(3).normal(size=(4000, 128)).astype(np.float32)
    cd = oracle.Codec(128, 3, seed=11)
    out = oracle.encode(cd, _bf16(x))
    freq = np.bincount(out["codes"].ravel(), minlength=8) / out["codes"].size
    edges = np.concatenate([[-np.inf], oracle.thresholds(cd.centroids), [np.inf]])
    mass = np.diff(scipy.stats.norm.cdf(edges))
    np.testing.assert_allclose(freq, mass, atol=4e-3)


def test_zero_vector_codes_and_decode():
    cd = oracle.Codec(128, 3, seed=5)
    out = oracle.encode(cd, np.zeros((2, 128), np.uint16))
    assert np.all(out["codes"] == 3)          # z = 0 sits in the cell just below t = 0
    assert np.all(out["norms"] == 0)
    np.testing.assert_array_equal(oracle.decode(cd, out["records"]), 0.0)


# ---------------------------------------------------------------------------------------------
# Packing and record size


@pytest.mark.parametrize("row", _golden_rows("record_bytes.txt"), ids=lambda r: f"m{r[0]}b{r[1]}")
def test_record_bytes_match_pages(row):
    m, bits, nbytes = int(row[0]), int(row[1]), int(row[2])
    assert oracle.record_bytes(m, bits) == nbytes
    x = _bf16(np.random.default_rng(m).normal(size=(3, m)))
    assert oracle.encode(oracle.Codec(m, bits, seed=1), x)["records"].shape == (3, nbytes)


@pytest.mark.parametrize("m", [32, 64, 128, 256, 512])
def test_plane_positions_are_a_permutation(m):
    pos = sorted(oracle.plane_position(i, m) for i in range(m))
    assert pos == list(range(m))


@pytest.mark.parametrize("m,bits", [(32, 4), (64, 3), (128, 3), (128, 2), (512, 4), (256, 1)])
def test_unpack_inverts_pack(m, bits):
    x = _bf16(np.random.default_rng(m * bits).normal(size=(20, m)))
    out = oracle.encode(oracle.Codec(m, bits, seed=3), x)
    for row in range(20):
        codes, nrm = oracle.unpack_codes(m, bits, out["records"][row])
        np.testing.assert_array_equal(codes, out["codes"][row])
        assert nrm == np.float32(out["norms"][row])


def test_pack_places_bits_per_format():
    """A single coordinate with code 2^p lands on one bit of word g*b + p (format v1)."""
    m, bits = 128, 3
    rng = np.random.default_rng(9)
    x = _bf16(rng.normal(size=(8, m)))
    out = oracle.encode(oracle.Codec(m, bits, seed=3), x)
    rec = out["records"][0]
    words = rec[: m * bits // 8].view("<u4")
    codes = out["codes"][0]
    for i in [0, 1, 7, 8, 9, 63, 64, 127]:
        pos = (i % 8) * (m // 8) + i // 8
        for p in range(bits):
            assert ((int(words[(pos // 32) * bits + p]) >> (pos % 32)) & 1) == ((int(codes[i]) >> p) & 1)


# ---------------------------------------------------------------------------------------------
# Decode


def test_decode_of_constant_code_record_is_closed_form():
    """All codes k: z^ = c_k * 1, H 1 = m e_0, so x^ = n c_k s_0 e_0."""
    m, bits, seed = 128, 3, 21
    cd = oracle.Codec(m, bits, seed=seed)
    for k in range(8):
        codes = np.full(m, k, np.uint8)
        words = np.zeros((m // 32) * bits, np.uint32)
        for i in range(m):
            pos = (i % 8) * (m // 8) + i // 8
            for p in range(bits):
                if (k >> p) & 1:
                    words[(pos // 32) * bits + p] |= np.uint32(1 << (pos % 32))
        rec = np.concatenate([words.view(np.uint8), np.array([2.5], np.float32).view(np.uint8)])
        y = oracle.decode(cd, rec[None, :])[0]
        expect = np.zeros(m)
        expect[0] = 2.5 * cd.centroids[k] * oracle.signs(seed, m)[0]
        np.testing.assert_allclose(y, expect, atol=1e-12)
        np.testing.assert_array_equal(oracle.unpack_codes(m, bits, rec)[0], codes)


@pytest.mark.parametrize("D,bits", [(128, 2), (128, 3), (512, 4)])
def test_decode_error_equals_coordinate_error(D, bits):
    """Parseval: ||x - x^||^2 / ||x||^2 = (1/m) sum (z_i - z^_i)^2 (up to the f32 norm)."""
    x = _bf16(np.random.default_rng(D).normal(size=(50, D)))
    cd = oracle.Codec(D, bits, seed=4)
    out = oracle.encode(cd, x)
    y = oracle.decode(cd, out["records"])
    xv = _bf16_to_f64(x)
    lhs = ((xv - y) ** 2).sum(1) / (xv * xv).sum(1)
    zhat = cd.centroids.astype(np.float64)[out["codes"]]
    rhs = ((out["z"] - zhat) ** 2).mean(1)
    np.testing.assert_allclose(lhs, rhs, rtol=1e-6)


@pytest.mark.parametrize("bits,expect", [(2, 0.1159), (3, 0.0340)])
def test_decode_mse_on_gaussian_rows(bits, expect):
    x = _bf16(np.random.default_rng(bits).normal(size=(3000, 128)))
    cd = oracle.Codec(128, bits, seed=4)
    out = oracle.encode(cd, x)
    y = oracle.decode(cd, out["records"])
    xv = _bf16_to_f64(x)
    rel = ((xv - y) ** 2).sum(1) / (xv * xv).sum(1)
    assert rel.mean() == pytest.approx(expect, rel=0.03)


# ---------------------------------------------------------------------------------------------
# Outliers


def test_outliers_infinite_threshold_is_the_plain_path():
    x = _bf16(np.random.default_rng(5).normal(size=(40, 128)))
    plain = oracle.encode(oracle.Codec(128, 2, seed=8), x)
    big = oracle.encode(oracle.Codec(128, 2, seed=8, T=1e9), x)
    assert big["total"] == 0
    np.testing.assert_array_equal(plain["records"], big["records"])
    np.testing.assert_array_equal(
        oracle.decode(oracle.Codec(128, 2, seed=8), plain["records"]),
        oracle.decode(oracle.Codec(128, 2, seed=8, T=1e9), big["records"], big["offsets"],
                      big["idx"], big["val"]))


@pytest.mark.parametrize("D", [64, 128, 256, 512])
def test_outliers_tiny_threshold_reconstructs_input(D):
    """T -> 0+: every nonzero coordinate is listed with its bf16 value, so decode returns x
    up to bf16 rounding of z (relative 2^-8 per coordinate)."""
    x = _bf16(np.random.default_rng(D).normal(size=(30, D)))
    cd = oracle.Codec(D, 2, seed=9, T=1e-30)
    out = oracle.encode(cd, x)
    assert out["total"] == 30 * D
    y = oracle.decode(cd, out["records"], out["offsets"], out["idx"], out["val"])
    xv = _bf16_to_f64(x)
    err = np.linalg.norm(xv - y, axis=1) / np.linalg.norm(xv, axis=1)
    assert err.max() < 2 ** -8


def test_outlier_rate_on_gaussian_rows_and_csr_order():
    x = _bf16(np.random.default_rng(6).normal(size=(2000, 128)))
    cd = oracle.Codec(128, 2, seed=10, T=2.0)
    out = oracle.encode(cd, x)
    rate = out["total"] / x.size
    assert rate == pytest.approx(2 * scipy.stats.norm.sf(2.0), abs=0.002)
    off = out["offsets"]
    assert off[0] == 0 and off[-1] == out["total"] and np.all(np.diff(off.astype(np.int64)) >= 0)
    for row in range(50):
        ix = out["idx"][off[row]:off[row + 1]]
        assert np.all(np.diff(ix.astype(int)) > 0)
        np.testing.assert_array_equal(ix, np.nonzero(np.abs(out["z"][row]) > 2.0)[0])


def test_outlier_lists_at_head_dim_512_use_two_byte_indices():
    """m = 512 (the V4-Flash geometry): indices reach 511, so the list holds u16 indices
    [kakeyaturbo PR #15, calibrated Lloyd-Max + outlier commit: (u16 idx, f16 val)]; the entries
    are exactly the coordinates with |z| > T in ascending order, the Gaussian tail rate holds,
    and decoding with the list moves the listed coordinates to their bf16 values."""
    x = _bf16(np.random.default_rng(8).normal(size=(400, 512)))
    cd = oracle.Codec(512, 4, seed=11, T=2.0)
    out = oracle.encode(cd, x)
    assert out["idx"].dtype == np.uint16 and out["idx"].max() > 255
    assert out["total"] / x.size == pytest.approx(2 * scipy.stats.norm.sf(2.0), abs=0.003)
    off = out["offsets"]
    for row in range(0, 400, 7):
        ix = out["idx"][off[row]:off[row + 1]]
        np.testing.assert_array_equal(ix, np.nonzero(np.abs(out["z"][row]) > 2.0)[0])
    plain = oracle.decode(oracle.Codec(512, 4, seed=11), out["records"])
    withl = oracle.decode(cd, out["records"], out["offsets"], out["idx"], out["val"])
    xv = _bf16_to_f64(x)
    e_plain = np.linalg.norm(xv - plain, axis=1) / np.linalg.norm(xv, axis=1)
    e_list = np.linalg.norm(xv - withl, axis=1) / np.linalg.norm(xv, axis=1)
    assert e_list.mean() < e_plain.mean()


def test_outlier_capacity_truncates_entries_not_offsets():
    x = _bf16(np.random.default_rng(7).normal(size=(100, 128)))
    cd = oracle.Codec(128, 2, seed=10, T=2.0)
    full = oracle.encode(cd, x)
    cut = oracle.encode(cd, x, ol_cap=10)
    np.testing.assert_array_equal(full["offsets"], cut["offsets"])
    np.testing.assert_array_equal(full["idx"][:10], cut["idx"])


# ---------------------------------------------------------------------------------------------
# Score


@pytest.mark.parametrize("D,bits", [(128, 3), (64, 2), (512, 4)])
def test_score_equals_rotated_domain_identity(D, bits):
    """q . decode(rec) = (n/m) sum_i q'_i z^_i with q' = H (s .* q), H from scipy."""
    rng = np.random.default_rng(D * bits)
    k = _bf16(rng.normal(size=(40, D)))
    q = _bf16(rng.normal(size=(40, D)))
    cd = oracle.Codec(D, bits, seed=12)
    out = oracle.encode(cd, k)
    got = oracle.score(cd, q, out["records"])
    s = oracle.signs(12, D).astype(np.float64)
    qp = (scipy.linalg.hadamard(D) @ (s[None, :] * _bf16_to_f64(q)).T).T
    zhat = cd.centroids.astype(np.float64)[out["codes"]]
    nrm = np.array([oracle.unpack_codes(D, bits, r)[1] for r in out["records"]], np.float64)
    np.testing.assert_allclose(got, nrm / D * (qp * zhat).sum(1), rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------------------------------------
# Stored-scale rules (matched norm, inner-product preserving, least squares)


@pytest.mark.parametrize("D,bits", [(64, 1), (128, 2), (128, 3), (512, 4)])
def test_scale_rules_meet_their_defining_identities(D, bits):
    """Decoded x^ of each rule: ||x^|| = ||x|| (matched), <x^, x> = ||x||^2 (inner product),
    <x - x^, x^> = 0 (least squares); the codes are those of the plain rule."""
    rng = np.random.default_rng(D + bits)
    x = _bf16(rng.normal(size=(40, D)) * rng.lognormal(0.0, 1.0, size=(40, 1)))
    xf = _bf16_to_f64(x)
    plain = oracle.Codec(D, bits, seed=21)
    base = oracle.encode(plain, x)
    for rule in (1, 2, 3):
        cd = oracle.Codec(D, bits, seed=21, scale_rule=rule)
        out = oracle.encode(cd, x)
        np.testing.assert_array_equal(out["codes"], base["codes"])
        y = oracle.decode(cd, out["records"])
        nx2 = (xf * xf).sum(1)
        if rule == 1:
            np.testing.assert_allclose(np.sqrt((y * y).sum(1)), np.sqrt(nx2), rtol=2e-7)
        elif rule == 2:
            np.testing.assert_allclose((y * xf).sum(1), nx2, rtol=2e-7)
        else:
            resid = ((xf - y) * y).sum(1)
            assert np.all(np.abs(resid) <= 2e-7 * np.sqrt(nx2 * (y * y).sum(1)))


def test_least_squares_rule_minimises_the_error_among_the_rules():
    rng = np.random.default_rng(7)
    x = _bf16(rng.normal(size=(64, 128)))
    xf = _bf16_to_f64(x)
    errs = []
    for rule in (0, 1, 2, 3):
        cd = oracle.Codec(128, 2, seed=3, scale_rule=rule)
        y = oracle.decode(cd, oracle.encode(cd, x)["records"])
        errs.append(((xf - y) ** 2).sum(1))
    errs = np.array(errs)
    assert np.all(errs[3] <= errs.min(axis=0) * (1 + 1e-6))
    # the plain norm is not the per-vector optimum, so least squares is strictly better on average
    assert errs[3].mean() < errs[0].mean()


# ---------------------------------------------------------------------------------------------
# Decode attention over packed K and V


def _attn_case(T, D=64, kb=3, vb=2, G=3, seed=0):
    rng = np.random.default_rng(seed)
    kc, vc = oracle.Codec(D, kb, seed=5), oracle.Codec(D, vb, seed=6)
    krec = oracle.encode_records(kc, _bf16(rng.normal(size=(T, D))))
    vrec = oracle.encode_records(vc, _bf16(rng.normal(size=(T, D))))
    q = _bf16(rng.normal(size=(G, D)))
    return kc, vc, q, krec, vrec


def test_attend_single_token_returns_its_decoded_value():
    kc, vc, q, krec, vrec = _attn_case(1)
    got = oracle.attend(kc, vc, q, krec, vrec, 0.125)
    want = oracle.decode(vc, vrec)[0]
    np.testing.assert_allclose(got, np.repeat(want[None], q.shape[0], 0), rtol=0, atol=1e-15)


def test_attend_zero_query_averages_the_values():
    kc, vc, q, krec, vrec = _attn_case(37)
    got = oracle.attend(kc, vc, np.zeros_like(q), krec, vrec, 0.125)
    want = oracle.decode(vc, vrec).mean(axis=0)
    np.testing.assert_allclose(got, np.repeat(want[None], q.shape[0], 0), rtol=1e-13, atol=1e-14)


def test_attend_two_tokens_is_the_logistic_mix():
    """T = 2: weights are sigma(l0 - l1) and sigma(l1 - l0), logits from the oracle's C score."""
    kc, vc, q, krec, vrec = _attn_case(2, G=4, seed=3)
    scale = 0.3
    got = oracle.attend(kc, vc, q, krec, vrec, scale)
    v = oracle.decode(vc, vrec)
    for g in range(q.shape[0]):
        l = scale * oracle.score(kc, np.repeat(q[g][None], 2, 0), krec)
        w0 = 1.0 / (1.0 + math.exp(-(l[0] - l[1])))
        np.testing.assert_allclose(got[g], w0 * v[0] + (1.0 - w0) * v[1], rtol=1e-12, atol=1e-13)


def test_attend_sharp_limit_selects_the_top_scoring_token():
    kc, vc, q, krec, vrec = _attn_case(29, G=2, seed=4)
    v = oracle.decode(vc, vrec)
    got = oracle.attend(kc, vc, q, krec, vrec, 1e6)
    for g in range(q.shape[0]):
        top = np.argmax(oracle.score(kc, np.repeat(q[g][None], 29, 0), krec))
        np.testing.assert_allclose(got[g], v[top], rtol=0, atol=1e-9)


def test_attend_ignores_token_order():
    kc, vc, q, krec, vrec = _attn_case(50, seed=5)
    perm = np.random.default_rng(1).permutation(50)
    a = oracle.attend(kc, vc, q, krec, vrec, 0.2)
    b = oracle.attend(kc, vc, q, krec[perm], vrec[perm], 0.2)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-13)


def test_attend_softcap_limits():
    """A huge cap changes nothing; a tiny cap flattens every logit towards 0 (uniform mean)."""
    kc, vc, q, krec, vrec = _attn_case(41, seed=6)
    plain = oracle.attend(kc, vc, q, krec, vrec, 0.5)
    np.testing.assert_allclose(oracle.attend(kc, vc, q, krec, vrec, 0.5, softcap=1e9), plain,
                               rtol=1e-9, atol=1e-12)
    flat = oracle.attend(kc, vc, q, krec, vrec, 0.5, softcap=1e-7)
    mean = oracle.decode(vc, vrec).mean(axis=0)
    np.testing.assert_allclose(flat, np.repeat(mean[None], q.shape[0], 0), rtol=1e-5, atol=1e-6)


# ---------------------------------------------------------------------------------------------
# PCA path


def test_pca_identity_basis_equals_plain_path():
    D = 128
    x = _bf16(np.random.default_rng(13).normal(size=(20, D)))
    eye = synth.bf16_bits(torch.eye(D).to(torch.bfloat16))
    pca = oracle.encode(oracle.Codec(D, 3, seed=2, r=D, basis_bf16=eye), x)
    plain = oracle.encode(oracle.Codec(D, 3, seed=2), x)
    np.testing.assert_array_equal(pca["records"], plain["records"])


def test_pca_tiny_threshold_reconstructs_projection():
    """With every coordinate listed as an outlier, decode returns mu + B B^T (x - mu)."""
    D, r = 128, 64
    k = synth.qwen2_1p5b_cache(layers=1, batch=1, kv_heads=1, tokens=600, seed=77)[0][0, 0, 0]
    mu, basis = synth.pca_basis_from_calibration(k[:512], r)
    bbits = synth.bf16_bits(basis)
    cd = oracle.Codec(D, 3, seed=2, r=r, T=1e-30, basis_bf16=bbits, mean=mu)
    x = synth.bf16_bits(k[512:])
    out = oracle.encode(cd, x)
    y = oracle.decode(cd, out["records"], out["offsets"], out["idx"], out["val"])
    B = _bf16_to_f64(bbits).reshape(D, r)
    xv = _bf16_to_f64(x)
    proj = mu + ((xv - mu) @ B) @ B.T
    err = np.linalg.norm(y - proj, axis=1) / np.linalg.norm(proj - mu, axis=1)
    assert err.max() < 2 ** -8


def test_pca_fit_residual_equals_discarded_eigenvalues():
    """Calibration input recipe: on the calibration slice, the mean squared projection residual
    equals the sum of the discarded covariance eigenvalues (f64 basis)."""
    k = synth.qwen2_1p5b_cache(layers=1, batch=1, kv_heads=1, tokens=512, seed=78)[0][0, 0, 0]
    x = k.float().double().numpy()
    mu = x.mean(0)
    cov = (x - mu).T @ (x - mu) / (x.shape[0] - 1)
    w, v = np.linalg.eigh(cov)
    order = np.argsort(w)[::-1]
    B = v[:, order[:64]]
    resid = (x - mu) - ((x - mu) @ B) @ B.T
    assert (resid ** 2).sum() / (x.shape[0] - 1) == pytest.approx(w[order[64:]].sum(), rel=1e-9)
    mu32, basis = synth.pca_basis_from_calibration(k, 64)
    np.testing.assert_allclose(np.abs(basis.float().numpy()), np.abs(B), atol=2 ** -8)


# ---------------------------------------------------------------------------------------------
# Q-preconditioning: the projection pair (basis L B_w, decode basis L^-T B_w, mean L^-T mu_w)


def _exact_whitening_factor(D, seed):
    """A lower-triangular factor L whose inverse is exact in bf16: unit diagonal, subdiagonal
    +-1/2, so (L^-1)[i][j] = prod_{k=j+1..i} (-a_k), a signed power of two (>= 2^-127)."""
    a = np.random.default_rng(seed).choice([-0.5, 0.5], size=D - 1)
    L = np.eye(D)
    L[np.arange(1, D), np.arange(D - 1)] = a
    Linv = np.eye(D)
    for i in range(D):
        for j in range(i):
            Linv[i, j] = np.prod(-a[j:i])
    assert np.array_equal(L @ Linv, np.eye(D))
    return L, Linv


def _bf16_exact(a):
    bits = _bf16(a)
    assert np.array_equal(_bf16_to_f64(bits).reshape(np.shape(a)), a)
    return bits


@pytest.mark.parametrize("D,bits", [(64, 2), (128, 3)])
def test_q_preconditioning_error_in_the_query_metric(D, bits):
    """Sigma_q = L L^T; whitening by L before the codec and by L^-T after it makes the
    query-metric error (x - x^)^T Sigma_q (x - x^) equal the codec's own error on the whitened
    vector, (1/m) ||n z - n32 z^||^2 (n32 the stored f32 scale). A transposed or swapped factor
    on either side breaks the identity, as L is not symmetric."""
    L, Linv = _exact_whitening_factor(D, seed=D + bits)
    cd = oracle.Codec(D, bits, seed=6, r=D, basis_bf16=_bf16_exact(L),
                      unbasis_bf16=_bf16_exact(Linv.T))
    x = _bf16(np.random.default_rng(7).normal(size=(40, D)))
    out = oracle.encode(cd, x)
    y = oracle.decode(cd, out["records"])
    e = _bf16_to_f64(x) - y
    lhs = np.einsum("nd,de,ne->n", e, L @ L.T, e)
    n32 = np.array([oracle.unpack_codes(D, bits, r)[1] for r in out["records"]], np.float64)
    zhat = cd.centroids.astype(np.float64)[out["codes"]]
    rhs = ((out["norms"][:, None] * out["z"] - n32[:, None] * zhat) ** 2).sum(1) / D
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9)
    # the whitened norm is what the record scales by
    np.testing.assert_allclose(out["norms"], np.linalg.norm(_bf16_to_f64(x) @ L, axis=1), rtol=1e-12)


def test_q_preconditioning_with_projection_and_mean():
    """Whitened-domain projection B_w (r of the D coordinates) and mean mu_w: the query-metric
    error splits into the discarded whitened energy plus the codec's error on the r kept
    coordinates, ||(I - B_w B_w^T) L^T (x - mu)||^2 + (1/r) ||n z - n32 z^||^2."""
    D, r, bits = 128, 64, 3
    L, Linv = _exact_whitening_factor(D, seed=21)
    keep = np.sort(np.random.default_rng(22).choice(D, size=r, replace=False))
    Bw = np.eye(D)[:, keep]
    mu_w = np.random.default_rng(23).normal(size=D)
    mu = (Linv.T @ mu_w).astype(np.float32)
    cd = oracle.Codec(D, bits, seed=8, r=r, basis_bf16=_bf16_exact(L @ Bw),
                      unbasis_bf16=_bf16_exact(Linv.T @ Bw), mean=mu)
    x = _bf16(np.random.default_rng(24).normal(size=(30, D)) * 2.0)
    out = oracle.encode(cd, x)
    y = oracle.decode(cd, out["records"])
    xc = _bf16_to_f64(x) - mu.astype(np.float64)
    e = _bf16_to_f64(x) - y
    lhs = np.einsum("nd,de,ne->n", e, L @ L.T, e)
    w = xc @ L                                   # whitened, centred rows (L^T (x - mu))
    dropped = (w ** 2).sum(1) - (w[:, keep] ** 2).sum(1)
    n32 = np.array([oracle.unpack_codes(r, bits, rec)[1] for rec in out["records"]], np.float64)
    zhat = cd.centroids.astype(np.float64)[out["codes"]]
    rhs = dropped + ((out["norms"][:, None] * out["z"] - n32[:, None] * zhat) ** 2).sum(1) / r
    np.testing.assert_allclose(lhs, rhs, rtol=1e-9)


def test_q_preconditioning_score_is_the_whitened_dot_product():
    """q . x^ = (L^-1 q) . (L^T x^): the score of a preconditioned record equals the score of
    the whitened query against the plain record of the whitened row when L is a signed
    permutation times powers of two (every product exact, so the two codecs see the same
    vector)."""
    D, bits = 64, 3
    rng = np.random.default_rng(31)
    P = np.eye(D)[rng.permutation(D)] * rng.choice([-1.0, 1.0], size=D)
    L = P * (2.0 ** rng.integers(-2, 3, size=D))[None, :]
    Linv = np.linalg.inv(L)
    qp = oracle.Codec(D, bits, seed=9, r=D, basis_bf16=_bf16_exact(L),
                      unbasis_bf16=_bf16_exact(Linv.T))
    plain = oracle.Codec(D, bits, seed=9)
    x = _bf16(rng.normal(size=(25, D)))
    q = _bf16(rng.normal(size=(25, D)))
    xw = _bf16_exact(_bf16_to_f64(x) @ L)
    rec = oracle.encode(qp, x)["records"]
    np.testing.assert_array_equal(rec, oracle.encode(plain, xw)["records"])
    qw = _bf16_exact(_bf16_to_f64(q) @ Linv.T)
    np.testing.assert_allclose(oracle.score(qp, q, rec), oracle.score(plain, qw, rec), rtol=1e-12)


# ---------------------------------------------------------------------------------------------
# Two-region cache model


def test_cache_model_invariants():
    D, window, margin = 128, 64, 16
    cd = oracle.Codec(D, 3, seed=3)
    model = oracle.CacheModel(cd, window, margin)
    rng = np.random.default_rng(14)
    rows_all = []
    for t_new in [300, 1, 1, 5, 0, 128, 1, 0, 40, 1]:
        rows = _bf16(rng.normal(size=(t_new, D)))
        rows_all.extend(list(rows))
        model.append_evict(rows)
        floor = oracle.retention_floor(window, t_new, margin)
        if len(model.tail) >= floor:
            assert floor <= len(model.tail) < floor + oracle.EVICT_CHUNK
        # the reachable span (last t_new + window - 1 rows) is always dense
        assert len(model.tail) >= min(len(rows_all), t_new + window - 1)
        n_packed = len(model.packed)
        assert n_packed % oracle.EVICT_CHUNK == 0
        np.testing.assert_array_equal(np.stack(model.tail), np.stack(rows_all[n_packed:]))
        if n_packed:
            np.testing.assert_array_equal(np.stack(model.packed),
                                          oracle.encode_records(cd, np.stack(rows_all[:n_packed])))


def test_retention_floor_terms_each_bind():
    """Each term of the floor binds somewhere (the pages' mutation table: dropping the margin,
    the t_new term or the max() must change the result)."""
    assert oracle.retention_floor(1024, 1, 16) == 1040       # margin binds
    assert oracle.retention_floor(1024, 100, 16) == 1123     # t_new - 1 binds
    assert oracle.retention_floor(1024, 0, 16) == 1040       # flush: window + margin
    assert oracle.retention_floor(1024, 17, 16) == 1040      # max() ties


# --- Rollback / truncation of the two-region cache [arc PR #98, "What landed": truncation maps
# onto both time bases; "Mutation runs": the rollback margin]. The pins compare the model with the
# plain append history (an independent list) and with the encode of its prefix.

def _cache_with_history(D, window, margin, t_news, seed):
    cd = oracle.Codec(D, 3, seed=3)
    model = oracle.CacheModel(cd, window, margin)
    rng = np.random.default_rng(seed)
    hist = []
    for t_new in t_news:
        rows = _bf16(rng.normal(size=(t_new, D)))
        hist.extend(list(rows))
        model.append_evict(rows)
    return cd, model, hist, rng


def test_truncate_inside_the_dense_tail_drops_the_newest_rows():
    D, window, margin = 64, 48, 16
    cd, model, hist, _ = _cache_with_history(D, window, margin, [400, 1, 1, 7], seed=21)
    n_packed, L = len(model.packed), len(model)
    assert L == len(hist) and len(model.tail) > 20
    packed_before = [r.copy() for r in model.packed]
    model.truncate(L - 13)
    assert len(model) == L - 13 and len(model.packed) == n_packed
    np.testing.assert_array_equal(np.stack(model.tail), np.stack(hist[n_packed:L - 13]))
    np.testing.assert_array_equal(np.stack(model.packed), np.stack(packed_before))
    model.truncate(L - 13)   # idempotent at the current length
    assert len(model) == L - 13
    model.truncate(n_packed)  # exactly the packed length: the tail empties, nothing packed goes
    assert len(model.tail) == 0 and len(model.packed) == n_packed


def test_truncate_into_the_packed_region_keeps_the_encoded_prefix():
    D, window, margin = 64, 48, 16
    cd, model, hist, _ = _cache_with_history(D, window, margin, [700, 0], seed=22)
    assert len(model.packed) >= 3 * oracle.EVICT_CHUNK
    new_len = len(model.packed) - 150          # not a chunk boundary
    model.truncate(new_len)
    assert len(model) == new_len and len(model.tail) == 0
    np.testing.assert_array_equal(np.stack(model.packed), oracle.encode_records(cd, np.stack(hist[:new_len])))
    model.truncate(0)
    assert len(model) == 0
    with pytest.raises(ValueError):
        model.truncate(1)


def test_reappend_after_rollback_keeps_the_reachable_span_dense():
    """Rollbacks of at most margin + 1 tokens between appends: after every append the span a
    query can reach (its t_new rows and the window - 1 before them) lies in the dense tail, the
    tail equals the history past the packed region, and the packed region is the encode of the
    history's prefix."""
    D, window, margin = 32, 40, 16
    cd = oracle.Codec(D, 2, seed=9)
    model = oracle.CacheModel(cd, window, margin)
    rng = np.random.default_rng(23)
    hist = []
    for step in range(300):
        t_new = int(rng.choice([1, 1, 1, 2, 5, 33]))
        rows = _bf16(rng.normal(size=(t_new, D)))
        hist.extend(list(rows))
        model.append_evict(rows)
        assert len(model.tail) >= min(len(hist), t_new + window - 1)
        n_packed = len(model.packed)
        np.testing.assert_array_equal(np.stack(model.tail), np.stack(hist[n_packed:]))
        if step % 3 == 2:  # speculative tokens rejected
            r = int(rng.integers(0, min(margin + 1, len(model.tail)) + 1))
            model.truncate(len(model) - r)
            del hist[len(hist) - r:]
            assert len(model.packed) == n_packed  # a shallow rollback never reaches the records
    np.testing.assert_array_equal(np.stack(model.packed),
                                  oracle.encode_records(cd, np.stack(hist[:len(model.packed)])))


def test_a_rollback_past_the_margin_can_leave_the_window_short():
    """The margin term binds: from a tail at exactly window + margin rows, rolling back
    margin + 2 tokens and appending one token leaves fewer dense rows than the window reaches."""
    D, window, margin = 32, 40, 16
    cd = oracle.Codec(D, 2, seed=9)
    model = oracle.CacheModel(cd, window, margin)
    rng = np.random.default_rng(24)
    model.append_evict(_bf16(rng.normal(size=(window + margin + 128, D))))
    model.append_evict(np.zeros((0, D), np.uint16))          # flush: exactly the floor remains
    assert len(model.tail) == window + margin
    safe = oracle.CacheModel(cd, window, margin)
    safe.packed, safe.tail = list(model.packed), list(model.tail)
    safe.truncate(len(safe) - (margin + 1))
    safe.append_evict(_bf16(rng.normal(size=(1, D))))
    assert len(safe.tail) >= window                           # still dense
    model.truncate(len(model) - (margin + 2))
    model.append_evict(_bf16(rng.normal(size=(1, D))))
    assert len(model.tail) == window - 1                      # one reachable row is packed


# --- Lloyd-Max refit on a sample [kakeyaturbo PR #15, calibration-artefacts commit]. Pinned by
# the population optimum it must approach on Gaussian samples, by the monotone-distortion
# property of Lloyd's iteration, by a direct numpy evaluation of the sample MSE, and by the
# heavy-tailed case whose refit must beat the Gaussian table.

def _np_table_mse(z, c32):
    t = np.array([np.float32(0.5 * (float(c32[k]) + float(c32[k + 1]))) for k in range(len(c32) - 1)],
                 np.float64)
    code = np.searchsorted(t, z, side="left")  # #{k : z > t_k}
    return float(np.mean((z - c32.astype(np.float64)[code]) ** 2))


@pytest.mark.parametrize("bits", [2, 3])
def test_refit_on_gaussian_samples_reproduces_the_gaussian_table(bits):
    rng = np.random.default_rng(30 + bits)
    z = rng.normal(size=1 << 20)
    gauss = oracle.gaussian_table(bits)[1]
    start = np.linspace(-2.5, 2.5, 1 << bits).astype(np.float32)   # far from the optimum
    fit = oracle.lloyd_fit(z, start, 200)
    assert np.all(np.diff(fit) > 0)
    np.testing.assert_allclose(fit, gauss, atol=0.012)          # sampling error ~1/sqrt(cell size)
    assert abs(oracle.table_mse(z, fit) - oracle.table_mse(z, gauss)) < 2e-4


def test_table_mse_matches_a_direct_evaluation():
    rng = np.random.default_rng(35)
    z = np.concatenate([rng.standard_t(3, size=5000), [0.0, -0.5006, 1.05]])
    c = oracle.gaussian_table(3)[1]
    assert abs(oracle.table_mse(z, c) - _np_table_mse(z, c)) < 1e-12


def test_refit_never_increases_the_sample_mse_and_beats_gaussian_on_heavy_tails():
    """Student-t(3) rows with 3 channels of 128 scaled x16 (the heavy-tailed V workload),
    rotated by the codec: each Lloyd pass does not raise the sample MSE, and the refit ends
    below the Gaussian table's MSE."""
    D, bits = 128, 2
    rng = np.random.default_rng(36)
    x = rng.standard_t(3, size=(4096, D))
    x[:, rng.choice(D, 3, replace=False)] *= 16
    cd = oracle.Codec(D, bits, seed=43)
    z = oracle.encode(cd, _bf16(x))["z"].reshape(-1)
    c = oracle.gaussian_table(bits)[1]
    mse = [oracle.table_mse(z, c)]
    for _ in range(15):
        c = oracle.lloyd_fit(z, c, 1)
        mse.append(oracle.table_mse(z, c))
    assert all(b <= a + 1e-12 for a, b in zip(mse, mse[1:])), mse
    assert mse[-1] < 0.98 * mse[0]
    np.testing.assert_array_equal(oracle.fit_table(cd, _bf16(x), 15), c)
