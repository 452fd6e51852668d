"""GPU parity of the projection (PCA) codec: MFMA projection + Hadamard over r coordinates,
MFMA unprojection, and the packed score with a projected query; one or several bases."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_vector_amd import kvq, synth
from tests.gpu_helpers import (bf16_host, check_scores, compare_codes, compare_decoded, say,
                               score_scale, unpack_records)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _bases(D, r, count, seed):
    """count frozen PCA fits, each on its own 512-row calibration slice."""
    K = synth.qwen2_1p5b_cache(layers=count, batch=1, kv_heads=1, tokens=512, head_dim=D,
                               seed=seed)[0]
    mus, bs = [], []
    for k in range(count):
        mu, basis = synth.pca_basis_from_calibration(K[k, 0, 0], r)
        mus.append(mu)
        bs.append(synth.bf16_bits(basis))
    return np.stack(mus), np.stack(bs)


def _oracle_codec(D, r, bits, seed, mu, b):
    return oracle.Codec(D, bits, seed=seed, r=r, basis_bf16=b, mean=mu)


@pytest.mark.parametrize("D,r,bits", [(128, 64, 3), (128, 32, 2), (256, 64, 4), (256, 128, 3),
                                      (64, 32, 1), (512, 64, 4), (256, 32, 3), (128, 64, 2)])
def test_pca_single_basis_encode_decode(D, r, bits):
    mu, b = _bases(D, r, 1, seed=D + r)
    basis = torch.from_numpy(b[0].view(np.int16)).view(torch.bfloat16).to(DEV).contiguous()
    mean = torch.from_numpy(mu[0]).to(DEV)
    codec = kvq.Codec(D, bits, seed=42, proj_rank=r, basis=basis, mean=mean)
    n = 700 + 13
    x = synth.qwen2_1p5b_cache(layers=1, batch=1, kv_heads=1, tokens=n, head_dim=D,
                               seed=D * r + bits, device=DEV)[0].reshape(n, D)
    say(f"pca encode D={D} r={r} b={bits} n={n}")
    rec = kvq.encode(codec, x)
    torch.cuda.synchronize()
    oc = _oracle_codec(D, r, bits, 42, mu[0], b[0])
    ref = oracle.encode(oc, bf16_host(x))
    recn = rec.cpu().numpy()
    mism, flagged = compare_codes(recn, ref, r, bits, f"pca D={D} r={r} b={bits}")
    say(f"  mismatches {mism} flagged {flagged}")
    for dt, ulp in ((torch.float32, False), (torch.bfloat16, True)):
        y = kvq.decode(codec, rec, dtype=dt)
        yref = oracle.decode(oc, recn)
        nrm = np.linalg.norm(yref, axis=1)
        compare_decoded(y.float().cpu().numpy(), yref, nrm, f"pca decode {dt}", extra_ulp_bf16=ulp)


def test_pca_many_bases_and_score():
    """Config-2 layout in miniature: [layers, batch, heads, tokens, D] with one basis per
    (layer, kv head), rows in blocks of `tokens`."""
    D, r, bits, L, B, H, T, G = 128, 64, 3, 3, 2, 2, 256, 6
    mu, b = _bases(D, r, L * H, seed=5)
    basis = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV).contiguous()
    mean = torch.from_numpy(mu).to(DEV).contiguous()
    blocks = torch.arange(L * B * H, dtype=torch.int32)
    index = ((blocks // (B * H)) * H + blocks % H).to(torch.int32).to(DEV)   # layer*H + head
    codec = kvq.Codec(D, bits, seed=42, proj_rank=r, basis=basis, mean=mean,
                      basis_index=index, basis_block_rows=T)
    K = synth.qwen2_1p5b_cache(layers=L, batch=B, kv_heads=H, tokens=T, seed=9, device=DEV)[0]
    x = K.reshape(-1, D)
    say(f"pca multi-basis L={L} B={B} H={H} T={T}")
    rec = kvq.encode(codec, x)
    y = kvq.decode(codec, rec)
    q = synth.iid_normal((L * B, H * G, D), seed=3, device=DEV)
    s = kvq.score_packed(codec, q, rec, Hkv=H, T=T, rec_sb=H * T, rec_sh=T)
    torch.cuda.synchronize()
    recn, yn, sn = rec.cpu().numpy(), y.cpu().numpy(), s.cpu().numpy()
    xh = bf16_host(x).reshape(L, B, H, T, D)
    qh = bf16_host(q).reshape(L, B, H * G, D)
    rh = recn.reshape(L, B, H, T, -1)
    for l in range(L):
        for h in range(H):
            k = l * H + h
            oc = _oracle_codec(D, r, bits, 42, mu[k], b[k])
            rows = xh[l, :, h].reshape(-1, D)
            ref = oracle.encode(oc, rows)
            got = rh[l, :, h].reshape(-1, recn.shape[1])
            compare_codes(got, ref, r, bits, f"layer {l} head {h}")
            yref = oracle.decode(oc, got)
            compare_decoded(yn.reshape(L, B, H, T, D)[l, :, h].reshape(-1, D), yref,
                            np.linalg.norm(yref, axis=1), f"decode layer {l} head {h}")
            for bb in range(B):
                for g in range(G):
                    hq = h * G + g
                    qq = np.repeat(qh[l, bb, hq][None], T, 0)
                    sref = oracle.score(oc, qq, rh[l, bb, h])
                    check_scores(sn[l * B + bb, hq], sref, score_scale(oc, qq, rh[l, bb, h]),
                                 f"score l={l} h={h} b={bb} g={g}")


def test_pca_score_bases_change_inside_a_block_run():
    """Bases change every 256 rows, inside the token run that one score block takes: with 128
    (batch, KV head) pairs of 2048 tokens each block takes at least two 256-token segments, so
    the block prepares its queries again for every new basis."""
    D, r, bits, B, H, T, G, NB = 128, 64, 3, 64, 2, 2048, 6, 5
    mu, b = _bases(D, r, NB, seed=11)
    basis = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(DEV).contiguous()
    mean = torch.from_numpy(mu).to(DEV).contiguous()
    index_h = (np.arange(B * H * T // 256) * 3 % NB).astype(np.int32)  # neighbours differ
    codec = kvq.Codec(D, bits, seed=42, proj_rank=r, basis=basis, mean=mean,
                      basis_index=torch.from_numpy(index_h).to(DEV), basis_block_rows=256)
    x = synth.iid_normal((B * H * T, D), seed=21, device=DEV)
    say(f"pca score, bases every 256 rows: B={B} H={H} T={T} G={G}")
    rec = kvq.encode(codec, x)
    q = synth.iid_normal((B, H * G, D), seed=22, device=DEV)
    s = kvq.score_packed(codec, q, rec, Hkv=H, T=T, rec_sb=H * T, rec_sh=T)
    torch.cuda.synchronize()
    recn, sn, qh = rec.cpu().numpy(), s.cpu().numpy(), bf16_host(q)
    for bb, h in [(0, 0), (31, 1), (63, 1)]:
        for blk in range(T // 256):
            row0 = (bb * H + h) * T + 256 * blk
            k = int(index_h[row0 // 256])
            oc = _oracle_codec(D, r, bits, 42, mu[k], b[k])
            recs = recn[row0: row0 + 256]
            for g in range(G):
                hq = h * G + g
                qq = np.repeat(qh[bb, hq][None], 256, 0)
                sref = oracle.score(oc, qq, recs)
                got = sn[bb, hq, 256 * blk: 256 * (blk + 1)]
                check_scores(got, sref, score_scale(oc, qq, recs), f"b={bb} h={h} block {blk} g={g}")


def test_pca_refusals():
    D, r = 128, 64
    basis = torch.zeros(D, r, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kvq.KvqError) as e:
        kvq.encode(kvq.Codec(D, 3, proj_rank=r, basis=basis, outlier_T=2.0),
                   torch.zeros(4, D, dtype=torch.bfloat16, device=DEV))
    assert e.value.name == "KVQ_E_OUTLIER"
    with pytest.raises(kvq.KvqError) as e:
        kvq.encode(kvq.Codec(512, 3, proj_rank=128, basis=torch.zeros(512, 128, dtype=torch.bfloat16, device=DEV)),
                   torch.zeros(4, 512, dtype=torch.bfloat16, device=DEV))
    assert e.value.name == "KVQ_E_DIM"
