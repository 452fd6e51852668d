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
    """Codes bit-exact except at flagged coordinates (|z - t| < 1e-5), whose mismatches must stay
    under CODE_MISMATCH_BAR; norms within NORM_RTOL. Returns (mismatches, flagged)."""
    gc, gn = unpack_records(gpu_rec, m, bits)
    rc, rn = unpack_records(ref["records"], m, bits)
    mism = gc != rc
    flagged = ref["flags"] != 0
    bad = mism & ~flagged
    assert not bad.any(), (f"{what}: {int(bad.sum())} unflagged code mismatches, first at "
                           f"{np.argwhere(bad)[:5].tolist()}")
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
