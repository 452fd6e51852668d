"""Seeded synthetic K/V inputs shaped like the workloads the pages measure.

This module holds no codec arithmetic: it draws random numbers, shapes them like the caches of
the models the pages use, and rounds them to bf16. Both the GPU path and the CPU oracle take
their inputs from here (the oracle via host copies), so neither side generates data for the
other. Every draw comes from a torch.Generator seeded from the workload's own seed, on the
device the data will live on. Recipes:

  kv_pair_outlier_channels   iid N(0,1) K and V with two channels of every head scaled x8
                             (single layer, 8 KV heads x 2048 tokens x head_dim 128)
  qwen2_1p5b_cache           [layers, batch, kv_heads, tokens, head_dim] values N(0,1) times a
                             per-channel lognormal(0, 0.5) scale drawn once per (layer, kv head,
                             stream, channel)
  iid_normal                 iid N(0,1) rows (DeepSeek-V4-Flash-shaped MQA cache, head_dim 512)
  student_t_heavy            Student-t (3 degrees of freedom) with round(0.02 * head_dim) channels
                             per (layer, head), drawn without replacement, scaled x16
  pca_basis_from_calibration top-r eigenvectors of the centred covariance of a calibration slice
                             (the frozen, one-time fit the codec is given as an input)
  query_covariance           synthetic Sigma_q = U diag(lambda) U^T: U Haar-random orthogonal,
                             lambda log-spaced over [1, cond] (the pages report a median condition
                             number of 4506 for real pre-RoPE query covariances), trace = D
  q_precondition_codec_inputs  the one-time host calibration of Q-preconditioning: the Cholesky
                             factor L of Sigma_q, optionally a PCA fit on whitened calibration rows,
                             folded into the projection pair (basis, decode basis, mean) that the
                             codec is given as inputs
"""
from __future__ import annotations

import numpy as np
import torch


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def iid_normal(shape, seed: int, device="cpu") -> torch.Tensor:
    """iid N(0,1), rounded to bf16."""
    g = _gen(seed, device)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32).to(torch.bfloat16)


def kv_pair_outlier_channels(heads=8, tokens=2048, head_dim=128, channels=(7, 93), factor=8.0,
                             seed=1001, device="cpu"):
    """K and V [1, heads, tokens, head_dim] bf16: iid N(0,1) with `channels` of every head
    multiplied by `factor`."""
    g = _gen(seed, device)
    out = []
    for _ in range(2):
        x = torch.randn(1, heads, tokens, head_dim, generator=g, device=device)
        for ch in channels:
            x[..., ch] *= factor
        out.append(x.to(torch.bfloat16))
    return out[0], out[1]


def qwen2_1p5b_cache(layers=28, batch=4, kv_heads=2, tokens=2048, head_dim=128, sigma=0.5,
                     seed=1002, device="cpu"):
    """K and V [layers, batch, kv_heads, tokens, head_dim] bf16: N(0,1) * scale[channel], with
    scale ~ lognormal(0, sigma) drawn per (layer, kv head, stream, channel)."""
    g = _gen(seed, device)
    out = []
    for _ in range(2):
        scale = torch.exp(sigma * torch.randn(layers, 1, kv_heads, 1, head_dim, generator=g,
                                              device=device))
        x = torch.randn(layers, batch, kv_heads, tokens, head_dim, generator=g, device=device)
        out.append((x * scale).to(torch.bfloat16))
    return out[0], out[1]


def student_t_heavy(layers=28, heads=8, tokens=8192, head_dim=128, df=3, frac=0.02,
                    factor=16.0, seed=1004, device="cpu"):
    """[layers, heads, tokens, head_dim] bf16 Student-t(df) values; round(frac * head_dim)
    channels per (layer, head), chosen without replacement, multiplied by `factor`.
    Student-t is drawn as N / sqrt(chi2_df / df), chi2_df a sum of df squared normals.
    Built one layer at a time to bound temporary memory."""
    g = _gen(seed, device)
    k = int(round(frac * head_dim))
    out = torch.empty(layers, heads, tokens, head_dim, dtype=torch.bfloat16, device=device)
    for l in range(layers):
        z = torch.randn(heads, tokens, head_dim, generator=g, device=device)
        chi2 = torch.zeros_like(z)
        for _ in range(df):
            e = torch.randn(heads, tokens, head_dim, generator=g, device=device)
            chi2 += e * e
        t = z / torch.sqrt(chi2 / df)
        for h in range(heads):
            ch = torch.randperm(head_dim, generator=g, device=device)[:k]
            t[h][:, ch] *= factor
        out[l] = t.to(torch.bfloat16)
    return out


def v4_flash_layers(layers=43, tokens=65536, head_dim=512, seed=1003, device="cpu"):
    """DeepSeek-V4-Flash-shaped K rows (one KV head per layer): yields one bf16
    [tokens, head_dim] iid N(0,1) tensor per layer from a single seeded stream."""
    g = _gen(seed, device)
    for _ in range(layers):
        yield torch.randn(tokens, head_dim, generator=g, device=device).to(torch.bfloat16)


def long_context_keys(batch=8, kv_heads=8, tokens=131072, head_dim=128, heads_q=32,
                      seed=1005, device="cpu"):
    """Keys [batch, kv_heads, tokens, head_dim] and decode-step queries [batch, heads_q,
    head_dim], both iid N(0,1) rounded to bf16 (keys drawn one batch row at a time)."""
    g = _gen(seed, device)
    k = torch.empty(batch, kv_heads, tokens, head_dim, dtype=torch.bfloat16, device=device)
    for b in range(batch):
        k[b] = torch.randn(kv_heads, tokens, head_dim, generator=g, device=device).to(torch.bfloat16)
    q = torch.randn(batch, heads_q, head_dim, generator=g, device=device).to(torch.bfloat16)
    return k, q


def pca_basis_from_calibration(calib_bf16: torch.Tensor, rank: int):
    """Frozen PCA fit on a calibration slice [tokens, D] (bf16): the mean (f32 [D]) and the
    top-`rank` eigenvectors of the centred covariance, in descending eigenvalue order, each
    column signed so its largest-magnitude entry is positive, rounded to bf16 ([D][rank]).
    This is the one-time host fit; the codec receives its result as an input."""
    x = calib_bf16.float().cpu().double().numpy()
    mu = x.mean(axis=0)
    xc = x - mu
    cov = xc.T @ xc / max(x.shape[0] - 1, 1)
    w, v = np.linalg.eigh(cov)
    order = np.argsort(w)[::-1][:rank]
    basis = v[:, order]
    for j in range(rank):
        if basis[np.argmax(np.abs(basis[:, j])), j] < 0:
            basis[:, j] = -basis[:, j]
    basis_bf16 = torch.from_numpy(basis.astype(np.float32)).to(torch.bfloat16)
    return mu.astype(np.float32), basis_bf16


def query_covariance(head_dim: int, cond: float, seed: int) -> np.ndarray:
    """Synthetic query covariance Sigma_q [D][D] (f64): Haar-random eigenvectors (QR of a
    Gaussian matrix, column signs fixed by R's diagonal), eigenvalues log-spaced over [1, cond]
    and scaled to trace D."""
    rng = np.random.default_rng(seed)
    z = rng.normal(size=(head_dim, head_dim))
    q, r = np.linalg.qr(z)
    q = q * np.sign(np.diag(r))[None, :]
    lam = np.exp(np.linspace(0.0, np.log(cond), head_dim))
    lam *= head_dim / lam.sum()
    return (q * lam) @ q.T


def q_precondition_codec_inputs(sigma_q: np.ndarray, calib_bf16: torch.Tensor | None = None,
                                rank: int = 0):
    """Projection pair for a Q-preconditioned codec, from Sigma_q = L L^T (L lower Cholesky).

    Whitening alone (rank 0): basis = L, decode basis = L^-T, no mean (coded length D).
    With a calibration slice and rank r: (mu_w, B_w) = the PCA fit of the whitened rows
    (calib @ L), then basis = L B_w, decode basis = L^-T B_w, mean = L^-T mu_w.
    Returns (basis bf16 [D][r], decode basis bf16 [D][r], mean f32 [D] or None)."""
    L = np.linalg.cholesky(sigma_q)
    Lit = np.linalg.inv(L).T
    if rank == 0:
        enc, dec, mean = L, Lit, None
    else:
        x = calib_bf16.float().cpu().double().numpy() @ L
        mu_w, bw = pca_basis_from_calibration(torch.from_numpy(x).to(torch.bfloat16), rank)
        bw = bw.float().double().numpy()
        enc, dec, mean = L @ bw, Lit @ bw, (Lit @ mu_w.astype(np.float64)).astype(np.float32)
    as_bf16 = lambda a: torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16)
    return as_bf16(enc), as_bf16(dec), mean


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    """Host uint16 view of a bf16 tensor (the oracle's input form)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view(np.uint16)
