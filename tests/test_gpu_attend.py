"""GPU parity of the decode-attention kernels (kvq_attend_packed) against the oracle's plain
softmax(scale * q . k^) . v^ on identical packed K and V records.

Bar: |out - out_ref| <= 1e-3 * max_t ||v^_t|| per element. A logit error d changes every weight
by a factor within e^{+-2d}; the kernels' logits and weighted sums carry ~2^-16 relative error
(bf16 hi + lo products, f32 sums), far inside the bar.
"""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_vector_amd import kvq, synth
from tests.gpu_helpers import bf16_host, oracle_codec_like, say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
ATTN_ATOL_REL = 1e-3


def _records(codec, B, Hkv, T, seed, scale=1.0):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    x = (scale * torch.randn(B * Hkv * T, codec.head_dim, generator=g, device=DEV)).to(torch.bfloat16)
    return kvq.encode(codec, x)


def _check(kc, vc, q, krec, vrec, B, Hkv, T, scale, softcap, out, okc, ovc, heads=None):
    Hq, D = q.shape[1], q.shape[2]
    G = Hq // Hkv
    kr = krec.cpu().numpy().reshape(B, Hkv, T, -1)
    vr = vrec.cpu().numpy().reshape(B, Hkv, T, -1)
    qh = bf16_host(q).reshape(B, Hq, D)
    got = out.cpu().numpy()
    worst = 0.0
    for b in range(B):
        for kv in range(Hkv):
            if heads is not None and (b, kv) not in heads:
                continue
            ref = oracle.attend(okc, ovc, qh[b, kv * G:(kv + 1) * G], kr[b, kv], vr[b, kv],
                                scale, softcap)
            vmax = np.linalg.norm(oracle.decode(ovc, vr[b, kv]), axis=1).max()
            err = np.abs(got[b, kv * G:(kv + 1) * G] - ref).max()
            assert err <= ATTN_ATOL_REL * vmax, f"(b={b}, kv={kv}): error {err:.3g} vs bar {ATTN_ATOL_REL * vmax:.3g}"
            worst = max(worst, err / vmax)
    return worst


@pytest.mark.parametrize("D,kb,vb,G,T", [(128, 3, 2, 4, 1), (128, 3, 2, 4, 17), (128, 3, 2, 6, 300),
                                         (128, 2, 3, 8, 1000), (64, 4, 1, 1, 777),
                                         (64, 1, 3, 2, 2049), (128, 4, 3, 8, 65), (128, 1, 1, 4, 333)])
def test_attend_parity_hadamard(D, kb, vb, G, T):
    B, Hkv = 2, 2
    kc, vc = kvq.Codec(D, kb, seed=31), kvq.Codec(D, vb, seed=32)
    krec = _records(kc, B, Hkv, T, seed=T + D)
    vrec = _records(vc, B, Hkv, T, seed=T + D + 1)
    q = synth.iid_normal((B, Hkv * G, D), seed=T * 7 + D, device=DEV)
    scale = 1.0 / np.sqrt(D)
    say(f"attend D={D} K b={kb} V b={vb} G={G} T={T}")
    out = kvq.attend_packed(kc, vc, q, krec, vrec, Hkv, T, rec_sb=Hkv * T, rec_sh=T, softmax_scale=scale)
    torch.cuda.synchronize()
    worst = _check(kc, vc, q, krec, vrec, B, Hkv, T, scale, 0.0, out, oracle_codec_like(kc),
                   oracle_codec_like(vc))
    say(f"  worst error / max||v^|| = {worst:.3g}")


def test_attend_softcap_and_sharp_scale():
    D, B, Hkv, G, T = 128, 1, 2, 3, 600
    kc, vc = kvq.Codec(D, 3, seed=41), kvq.Codec(D, 2, seed=42)
    krec = _records(kc, B, Hkv, T, seed=5)
    vrec = _records(vc, B, Hkv, T, seed=6)
    q = synth.iid_normal((B, Hkv * G, D), seed=7, device=DEV)
    for scale, cap in ((0.5, 0.0), (0.5, 5.0), (0.02, 30.0)):
        say(f"attend softcap={cap} scale={scale}")
        out = kvq.attend_packed(kc, vc, q, krec, vrec, Hkv, T, rec_sb=Hkv * T, rec_sh=T,
                                softmax_scale=scale, softcap=cap)
        torch.cuda.synchronize()
        _check(kc, vc, q, krec, vrec, B, Hkv, T, scale, cap, out, oracle_codec_like(kc),
               oracle_codec_like(vc))


def test_attend_projected_keys_several_bases():
    """K through the PCA codec (one basis per (batch, KV head) block of 512 rows), V Hadamard."""
    D, r, B, Hkv, G, T = 128, 64, 2, 2, 6, 512
    K = synth.qwen2_1p5b_cache(layers=1, batch=B, kv_heads=Hkv, tokens=T, head_dim=D, seed=77,
                               device=DEV)[0][0]       # [B, Hkv, T, D]
    mus, bases = [], []
    for h in range(Hkv):
        mu, basis = synth.pca_basis_from_calibration(K[0, h, :256], r)
        mus.append(mu)
        bases.append(basis)
    basis_t = torch.stack(bases).to(DEV).contiguous()
    mean_t = torch.from_numpy(np.stack(mus)).to(DEV).contiguous()
    index = (torch.arange(B * Hkv, dtype=torch.int32) % Hkv).to(DEV)
    kc = kvq.Codec(D, 3, seed=42, proj_rank=r, basis=basis_t, mean=mean_t, basis_index=index,
                   basis_block_rows=T)
    vc = kvq.Codec(D, 2, seed=43)
    krec = kvq.encode(kc, K.reshape(-1, D))
    vrec = _records(vc, B, Hkv, T, seed=78)
    q = synth.iid_normal((B, Hkv * G, D), seed=79, device=DEV)
    scale = 1.0 / np.sqrt(D)
    say(f"attend PCA K r={r}, {Hkv} bases")
    out = kvq.attend_packed(kc, vc, q, krec, vrec, Hkv, T, rec_sb=Hkv * T, rec_sh=T, softmax_scale=scale)
    torch.cuda.synchronize()
    bh = synth.bf16_bits(basis_t)
    for b in range(B):
        for kv in range(Hkv):
            okc = oracle.Codec(D, 3, seed=42, r=r, basis_bf16=bh[kv], mean=mus[kv])
            _check(kc, vc, q, krec, vrec, B, Hkv, T, scale, 0.0, out, okc, oracle_codec_like(vc),
                   heads={(b, kv)})


def test_attend_long_context_sampled():
    """One batch row at 65,536 tokens (the block split puts many blocks on each KV head);
    two (batch, KV head) pairs are checked in full against the oracle."""
    D, B, Hkv, G, T = 128, 2, 4, 4, 65536
    kc, vc = kvq.Codec(D, 3, seed=51), kvq.Codec(D, 2, seed=52)
    krec = _records(kc, B, Hkv, T, seed=53)
    vrec = _records(vc, B, Hkv, T, seed=54)
    q = synth.iid_normal((B, Hkv * G, D), seed=55, device=DEV)
    say(f"attend long context T={T} B={B} Hkv={Hkv} G={G}")
    out = kvq.attend_packed(kc, vc, q, krec, vrec, Hkv, T, rec_sb=Hkv * T, rec_sh=T,
                            softmax_scale=1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    _check(kc, vc, q, krec, vrec, B, Hkv, T, 1.0 / np.sqrt(D), 0.0, out, oracle_codec_like(kc),
           oracle_codec_like(vc), heads={(0, 0), (1, 3)})


def test_attend_strided_query_and_output():
    """Query rows and output rows inside wider buffers; the padding stays untouched."""
    D, B, Hkv, G, T = 64, 3, 1, 5, 333
    kc, vc = kvq.Codec(D, 2, seed=61), kvq.Codec(D, 2, seed=62)
    krec = _records(kc, B, Hkv, T, seed=63)
    vrec = _records(vc, B, Hkv, T, seed=64)
    qbig = synth.iid_normal((B, G, D + 16), seed=65, device=DEV)
    q = qbig[:, :, :D]
    outbig = torch.full((B, G + 1, D + 8), 7.0, dtype=torch.float32, device=DEV)
    out = outbig[:, :G, :D]
    kvq.attend_packed(kc, vc, q, krec, vrec, Hkv, T, rec_sb=Hkv * T, rec_sh=T, softmax_scale=0.125,
                      out=out)
    torch.cuda.synchronize()
    assert torch.all(outbig[:, G:, :] == 7.0) and torch.all(outbig[:, :, D:] == 7.0)
    _check(kc, vc, q.contiguous(), krec, vrec, B, Hkv, T, 0.125, 0.0, out, oracle_codec_like(kc),
           oracle_codec_like(vc))
