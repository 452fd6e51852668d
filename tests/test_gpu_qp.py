"""GPU parity of Q-preconditioned codecs: the whitening factor L of a synthetic query covariance
folded into the projection pair (basis L B_w, decode basis L^-T B_w, mean L^-T mu_w), through
encode, decode, the packed score and decode attention, against the oracle on the same bf16
pair. Whitening alone is the square case r = D."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_vector_amd import kvq, synth
from tests.gpu_helpers import (bf16_host, check_scores, compare_codes, compare_decoded,
                               oracle_codec_like, say, score_scale)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _pair(D, r, count, seed, cond=4506.0):
    """count (Sigma_q, calibration) draws -> stacked device pair and host copies."""
    K = synth.qwen2_1p5b_cache(layers=count, batch=1, kv_heads=1, tokens=512, head_dim=D,
                               seed=seed)[0]
    enc, dec, mus = [], [], []
    for k in range(count):
        sig = synth.query_covariance(D, cond, seed=seed + 17 * k)
        e, d, mu = synth.q_precondition_codec_inputs(sig, K[k, 0, 0] if r < D else None,
                                                     0 if r == D else r)
        enc.append(e)
        dec.append(d)
        mus.append(np.zeros(D, np.float32) if mu is None else mu)
    enc_t = torch.stack(enc).to(DEV).contiguous()
    dec_t = torch.stack(dec).to(DEV).contiguous()
    mean_t = torch.from_numpy(np.stack(mus)).to(DEV).contiguous() if r < D else None
    return enc_t, dec_t, mean_t, synth.bf16_bits(enc_t), synth.bf16_bits(dec_t), np.stack(mus)


def _oracle(D, r, bits, seed, eb, db, mu):
    return oracle.Codec(D, bits, seed=seed, r=r, basis_bf16=eb, unbasis_bf16=db,
                        mean=mu if r < D else None)


@pytest.mark.parametrize("D,r,bits", [(64, 64, 2), (64, 64, 3), (128, 128, 3), (128, 128, 2),
                                      (128, 64, 3), (128, 32, 2), (64, 32, 4), (256, 64, 3)])
def test_qp_encode_decode_score(D, r, bits):
    enc, dec, mean, eb, db, mu = _pair(D, r, 1, seed=D + r + bits)
    codec = kvq.Codec(D, bits, seed=42, proj_rank=r, basis=enc[0], mean=None if mean is None else mean[0],
                      unbasis=dec[0])
    oc = _oracle(D, r, bits, 42, eb[0], db[0], mu[0])
    n = 700 + 13
    x = synth.qwen2_1p5b_cache(layers=1, batch=1, kv_heads=1, tokens=n, head_dim=D,
                               seed=D * r + bits, device=DEV)[0].reshape(n, D)
    say(f"qp encode D={D} r={r} b={bits} n={n}")
    rec = kvq.encode(codec, x)
    torch.cuda.synchronize()
    ref = oracle.encode(oc, bf16_host(x))
    recn = rec.cpu().numpy()
    mism, flagged = compare_codes(recn, ref, r, bits, f"qp D={D} r={r} b={bits}")
    say(f"  mismatches {mism} flagged {flagged}")
    yref = oracle.decode(oc, recn)
    nrm = np.linalg.norm(yref, axis=1)
    for dt, ulp in ((torch.float32, False), (torch.bfloat16, True)):
        y = kvq.decode(codec, rec, dtype=dt)
        compare_decoded(y.float().cpu().numpy(), yref, nrm, f"qp decode {dt}", extra_ulp_bf16=ulp)
    # packed score: one batch row, one KV head, 3 query heads over the n records
    q = synth.iid_normal((1, 3, D), seed=n + D, device=DEV)
    s = kvq.score_packed(codec, q, rec, Hkv=1, T=n, rec_sb=n, rec_sh=n)
    torch.cuda.synchronize()
    qh = bf16_host(q).reshape(3, D)
    for h in range(3):
        qq = np.repeat(qh[h][None], n, 0)
        sref = oracle.score(oc, qq, recn)
        check_scores(s[0, h].cpu().numpy(), sref, score_scale(oc, qq, recn), f"score head {h}")


def test_qp_several_bases_and_attention():
    """One (Sigma_q, whitened PCA) pair per KV head over [batch, heads, tokens] blocks; K through
    the preconditioned codec, V Hadamard; attention against the oracle."""
    D, r, bits, B, H, T, G = 128, 64, 3, 2, 2, 512, 6
    enc, dec, mean, eb, db, mu = _pair(D, r, H, seed=91)
    index = (torch.arange(B * H, dtype=torch.int32) % H).to(DEV)
    kc = kvq.Codec(D, bits, seed=42, proj_rank=r, basis=enc, mean=mean, unbasis=dec,
                   basis_index=index, basis_block_rows=T)
    vc = kvq.Codec(D, 2, seed=43)
    K, V = synth.qwen2_1p5b_cache(layers=1, batch=B, kv_heads=H, tokens=T, head_dim=D, seed=92,
                                  device=DEV)
    say(f"qp several bases B={B} H={H} T={T}")
    krec = kvq.encode(kc, K[0].reshape(-1, D))
    vrec = kvq.encode(vc, V[0].reshape(-1, D))
    q = synth.iid_normal((B, H * G, D), seed=93, device=DEV)
    out = kvq.attend_packed(kc, vc, q, krec, vrec, H, T, rec_sb=H * T, rec_sh=T,
                            softmax_scale=1.0 / np.sqrt(D))
    torch.cuda.synchronize()
    kr = krec.cpu().numpy().reshape(B, H, T, -1)
    vr = vrec.cpu().numpy().reshape(B, H, T, -1)
    xh = bf16_host(K[0].reshape(-1, D)).reshape(B, H, T, D)
    qh = bf16_host(q).reshape(B, H * G, D)
    got = out.cpu().numpy()
    ovc = oracle_codec_like(vc)
    for h in range(H):
        oc = _oracle(D, r, bits, 42, eb[h], db[h], mu[h])
        for b in range(B):
            compare_codes(kr[b, h], oracle.encode(oc, xh[b, h]), r, bits, f"K b={b} h={h}")
            ref = oracle.attend(oc, ovc, qh[b, h * G:(h + 1) * G], kr[b, h], vr[b, h], 1.0 / np.sqrt(D))
            vmax = np.linalg.norm(oracle.decode(ovc, vr[b, h]), axis=1).max()
            err = np.abs(got[b, h * G:(h + 1) * G] - ref).max()
            assert err <= 1e-3 * vmax, f"attention b={b} h={h}: {err:.3g}"


@pytest.mark.parametrize("D", [64, 128])
def test_qp_whitening_alone_attention(D):
    """Square whitening (r = D) for K: the attention kernel's projected-query path at m = D."""
    B, H, G, T = 1, 2, 4, 700
    enc, dec, _, eb, db, mu = _pair(D, D, 1, seed=D + 5)
    kc = kvq.Codec(D, 3, seed=44, proj_rank=D, basis=enc[0], unbasis=dec[0])
    vc = kvq.Codec(D, 2, seed=45)
    K, V = synth.qwen2_1p5b_cache(layers=1, batch=B, kv_heads=H, tokens=T, head_dim=D, seed=D,
                                  device=DEV)
    say(f"qp whitening attention D={D} T={T}")
    krec = kvq.encode(kc, K[0].reshape(-1, D))
    vrec = kvq.encode(vc, V[0].reshape(-1, D))
    q = synth.iid_normal((B, H * G, D), seed=D + 1, device=DEV)
    out = kvq.attend_packed(kc, vc, q, krec, vrec, H, T, rec_sb=H * T, rec_sh=T, softmax_scale=0.1,
                            softcap=20.0)
    torch.cuda.synchronize()
    oc = _oracle(D, D, 3, 44, eb[0], db[0], mu[0])
    ovc = oracle_codec_like(vc)
    kr = krec.cpu().numpy().reshape(B, H, T, -1)
    vr = vrec.cpu().numpy().reshape(B, H, T, -1)
    qh = bf16_host(q).reshape(B, H * G, D)
    got = out.cpu().numpy()
    for h in range(H):
        ref = oracle.attend(oc, ovc, qh[0, h * G:(h + 1) * G], kr[0, h], vr[0, h], 0.1, 20.0)
        vmax = np.linalg.norm(oracle.decode(ovc, vr[0, h]), axis=1).max()
        err = np.abs(got[0, h * G:(h + 1) * G] - ref).max()
        assert err <= 1e-3 * vmax, f"attention h={h}: {err:.3g}"
