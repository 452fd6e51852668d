"""Shared comparison helpers of the GPU parity tests (the oracle is the reference)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from kv_cache_compression_vector_amd import synth

CODE_MISMATCH_BAR = 1e-4   # mismatching codes, as a fraction of coordinates (flagged only)
NORM_RTOL = 1e-5
DECODE_ATOL_REL = 1e-3     # times the vector's norm
SCORE_RTOL = 1e-3          # times max(|s|, sum of |terms|)


def say(*args):
    print("[gpu]", *args, flush=True)
    sys.stdout.flush()


def unpack_records(rec: np.ndarray, m: int, bits: int):
    """Vectorised unpack of format-v1 records -> (codes [n, m] u8, norms [n] f32)."""
    rec = np.ascontiguousarray(rec, np.uint8)
    n = rec.shape[0]
    nw = (m // 32) * bits
    words = rec[:, : 4 * nw].copy().view("<u4").reshape(n, m // 32, bits)
    i = np.arange(m)
    pos = (i % 8) * (m // 8) + i // 8
    g, j = pos // 32, pos % 32
    codes = np.zeros((n, m), np.uint8)
    for p in range(bits):
        codes |= (((words[:, g, p] >> j[None, :].astype(np.uint32)) & 1).astype(np.uint8) << p)
    norms = rec[:, 4 * nw: 4 * nw + 4].copy().view("<f4").reshape(n)
    return codes, norms


def compare_codes(gpu_rec: np.ndarray, ref: dict, m: int, bits: int, what: str):
    """Codes bit-exact except at coordinates within 1e-5 of a decision boundary t_k; there the
    GPU's code must be one of the two cells the boundary separates (k or k + 1, k the boundary
    nearest to the oracle's z), and such mismatches must stay under CODE_MISMATCH_BAR of the
    coordinates. Norms within NORM_RTOL. Returns (mismatches, flagged)."""
    gc, gn = unpack_records(gpu_rec, m, bits)
    rc, rn = unpack_records(ref["records"], m, bits)
    mism = gc != rc
    flagged = (ref["flags"] & oracle.FLAG_NEAR_BOUNDARY) != 0
    bad = mism & ~flagged
    assert not bad.any(), (f"{what}: {int(bad.sum())} unflagged code mismatches, first at "
                           f"{np.argwhere(bad)[:5].tolist()}")
    if mism.any():
        t = np.asarray(ref["thresholds"], np.float64)
        z = ref["z"][mism]
        k = np.abs(z[:, None] - t[None, :]).argmin(axis=1)  # the boundary the coordinate is near
        g = gc[mism].astype(np.int64)
        off = ~((g == k) | (g == k + 1))
        assert not off.any(), (f"{what}: {int(off.sum())} flagged coordinates coded outside the two "
                               f"cells of their nearby boundary, first at "
                               f"{np.argwhere(mism)[np.nonzero(off)[0][:5]].tolist()}")
    n_coords = max(mism.size, 1)
    assert mism.sum() <= CODE_MISMATCH_BAR * n_coords + 0, (
        f"{what}: {int(mism.sum())} flagged mismatches > {CODE_MISMATCH_BAR} of {n_coords}")
    ok = rn > 0
    np.testing.assert_allclose(gn[ok], rn[ok], rtol=NORM_RTOL, err_msg=f"{what}: norms")
    assert np.all(gn[~ok] == 0), f"{what}: zero vectors must have norm 0"
    return int(mism.sum()), int(flagged.sum())


def compare_decoded(gpu_y: np.ndarray, ref_y: np.ndarray, norms: np.ndarray, what: str,
                    extra_ulp_bf16: bool = False):
    err = np.abs(gpu_y.astype(np.float64) - ref_y)
    tol = DECODE_ATOL_REL * norms.astype(np.float64)[:, None]
    if extra_ulp_bf16:
        tol = tol + np.abs(ref_y) * 2.0 ** -8
    worst = (err - tol).max() if err.size else -1
    assert worst <= 0, f"{what}: decode error exceeds 1e-3*||x|| (worst excess {worst:.3g})"
    return float((err / np.maximum(norms[:, None], 1e-30)).max()) if err.size else 0.0


def bf16_host(t: torch.Tensor) -> np.ndarray:
    return synth.bf16_bits(t)


def oracle_codec_like(codec, basis_host=None, mean_host=None) -> oracle.Codec:
    # the oracle builds its own Gaussian table; a custom table is an input given to both sides
    return oracle.Codec(codec.head_dim, codec.bits, seed=codec.seed, r=codec.proj_rank,
                        T=codec.outlier_T, centroids=codec._centroids, basis_bf16=basis_host,
                        mean=mean_host, scale_rule=codec.flags & 3)


def compare_outlier_lists(off, idx, val, ref, rows=None, what="outliers"):
    """Every vector's CSR entries against the oracle's. off/idx/val: the GPU's list (offsets
    [n+1], entries); ref: oracle.encode of the vectors `rows` (all vectors when None), in
    order. Per vector the index sets must be equal except at coordinates the oracle flags as
    within 1e-5 of T (where either membership is valid), and the values of common entries must
    agree to one bf16 ulp. Returns the number of vectors whose lists differ (near-T only)."""
    off = np.asarray(off).astype(np.int64)
    roff = np.asarray(ref["offsets"]).astype(np.int64)
    rows = np.arange(len(roff) - 1) if rows is None else np.asarray(rows)
    near_t = (ref["flags"] & oracle.FLAG_NEAR_T) != 0
    differing = 0
    for k, v in enumerate(rows):
        gi = np.asarray(idx[off[v]:off[v + 1]]).astype(np.int64)
        gv = np.asarray(val[off[v]:off[v + 1]]).astype(np.int64)
        ri = np.asarray(ref["idx"][roff[k]:roff[k + 1]]).astype(np.int64)
        rv = np.asarray(ref["val"][roff[k]:roff[k + 1]]).astype(np.int64)
        assert np.all(np.diff(gi) > 0), f"{what}: vector {v} entries not in ascending order"
        sym = np.setxor1d(gi, ri)
        if sym.size:
            differing += 1
            assert np.all(near_t[k, sym]), (f"{what}: vector {v} lists differ at coordinates "
                                            f"{sym[~near_t[k, sym]][:5].tolist()} not within 1e-5 of T")
        common, gpos, rpos = np.intersect1d(gi, ri, return_indices=True)
        assert np.all(np.abs(gv[gpos] - rv[rpos]) <= 1), f"{what}: vector {v} values beyond 1 bf16 ulp"
    return differing


def _f64_of_bf16(bits_u16):
    return (np.asarray(bits_u16, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def score_scale(oc: oracle.Codec, q_bits: np.ndarray, recs: np.ndarray) -> np.ndarray:
    """Normwise scale of the packed score of each (query, record) pair, the sum of the absolute
    terms the score adds: (n/m) sum_i |q'_i z^_i| with q' = H_m(s (.) q); for a projection codec
    q' = H_r(s (.) C^T q) (C the decode basis) plus |q . mu|."""
    q = _f64_of_bf16(q_bits).reshape(-1, oc.D)
    qmu = np.zeros(q.shape[0])
    if oc.r > 0:
        C = _f64_of_bf16(oc.unbasis if oc.unbasis is not None else oc.basis).reshape(oc.D, oc.r)
        if oc.mean is not None:
            qmu = np.abs(q @ oc.mean.astype(np.float64))
        q = q @ C
    qp = oracle.fwht_rows(q * oracle.signs(oc.seed, oc.m).astype(np.float64))
    codes, norms = unpack_records(recs, oc.m, oc.bits)
    zh = oc.centroids.astype(np.float64)[codes]
    return norms.astype(np.float64) / oc.m * np.abs(qp * zh).sum(axis=1) + qmu


def check_scores(got, sref, scale, what):
    """|got - ref| <= SCORE_RTOL * max(|ref|, scale) element by element."""
    got = np.asarray(got, np.float64).reshape(-1)
    sref = np.asarray(sref, np.float64).reshape(-1)
    bound = SCORE_RTOL * np.maximum(np.abs(sref), np.asarray(scale, np.float64).reshape(-1))
    err = np.abs(got - sref)
    assert np.all(err <= bound), (f"{what}: score error exceeds the normwise bar at "
                                  f"{int((err > bound).sum())} pairs (worst err/bound "
                                  f"{float(np.max(err / np.maximum(bound, 1e-300))):.3g})")
    return float(np.max(err / np.maximum(bound, 1e-300))) if err.size else 0.0
