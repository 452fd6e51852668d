"""GPU parity at the full sizes of the larger workloads. Each test makes one library call over
the whole tensor, launched as a caller (and bench.py) would. It compares outputs at sampled
positions against the oracle, computed one by one, and checks properties that hold at any size
(CSR monotonicity, cache lengths, bit-identical tail rows)."""
import time

import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_vector_amd import kvq, synth
from tests.gpu_helpers import (bf16_host, check_scores, compare_codes, compare_decoded,
                               compare_outlier_lists, oracle_codec_like, say, score_scale,
                               unpack_records)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _sample(n, k, seed):
    """k distinct random positions in [0, n), plus both ends (ragged last tiles)."""
    rng = np.random.default_rng(seed)
    s = rng.choice(n, size=min(k, n), replace=False)
    return np.unique(np.concatenate([s, [0, n - 1]])).astype(np.int64)


def _take(t, rows):
    return t[torch.from_numpy(rows).to(t.device)]


def _f64(bits_u16):
    return (bits_u16.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_v4_flash_cache_bulk_flush_then_steady_appends():
    """43 layers x 1 KV head x 65,536 rows x head_dim 512, 4 bits, window 1024, margin 16:
    a bulk flush evicts 503 chunks per layer; then 1,024 single-row appends."""
    L, T0, D, bits, window, margin, steps = 43, 65536, 512, 4, 1024, 16, 1024
    codec = kvq.Codec(D, bits, seed=42)
    oc = oracle_codec_like(codec)
    say(f"v4-flash cache: {L} layers x {T0} x {D}, b={bits}")
    layers = list(synth.v4_flash_layers(L, T0, D, device=DEV))
    steady = synth.iid_normal((L, steps, D), seed=1103, device=DEV)
    caches = [kvq.Cache(codec, packed_cap=T0 + steps, tail_cap=T0 + 1, window=window,
                        margin=margin, device=DEV) for _ in range(L)]
    assert kvq.append_evict_chunk(codec, caches, layers, T0) == [0] * L
    floor = oracle.retention_floor(window, 0, margin)
    k0 = (T0 - floor) // 128
    assert k0 == 503
    t0 = time.perf_counter()
    assert kvq.append_evict_chunk(codec, caches, None, 0) == [k0] * L
    torch.cuda.synchronize()
    say(f"  bulk flush of {L * k0 * 128} rows: {1e3 * (time.perf_counter() - t0):.2f} ms host-inclusive")
    tail, packed = T0 - 128 * k0, 128 * k0
    assert all(c.packed_len == packed and c.tail_len == tail for c in caches)
    floor1 = oracle.retention_floor(window, 1, margin)
    t0 = time.perf_counter()
    for i in range(steps):
        ev = kvq.append_evict_chunk(codec, caches, [steady[l, i:i + 1] for l in range(L)], 1)
        tail += 1
        k = (tail - floor1) // 128 if tail >= floor1 + 128 else 0
        assert ev == [k] * L, f"step {i}"
        tail -= 128 * k
        packed += 128 * k
        assert floor1 <= tail < floor1 + 128
    torch.cuda.synchronize()
    say(f"  steady state: {1e6 * (time.perf_counter() - t0) / steps:.1f} us/step host-inclusive "
        f"({L} caches per call)")
    for l in (0, 21, 42):
        c = caches[l]
        assert c.packed_len == packed and c.tail_len == tail
        allrows = torch.cat([layers[l], steady[l]])
        np.testing.assert_array_equal(bf16_host(c.tail_rows()), bf16_host(allrows[packed:packed + tail]))
        rows = _sample(packed, 1500, seed=l)
        got = _take(c.packed, rows).cpu().numpy()
        ref = oracle.encode(oc, bf16_host(_take(allrows, rows)))
        mism, flagged = compare_codes(got, ref, D, bits, f"layer {l} packed rows")
        say(f"  layer {l}: {len(rows)} sampled records, mismatches {mism} flagged {flagged}")


def test_heavy_tailed_v_with_outliers_full_size():
    """[28, 8, 8192, 128] Student-t(3) with 3 channels per (layer, head) x16; b=2, T=2.0."""
    D, bits, T_ = 128, 2, 2.0
    X = synth.student_t_heavy(device=DEV)
    x = X.reshape(-1, D)
    n = x.shape[0]
    codec = kvq.Codec(D, bits, seed=43, outlier_T=T_)
    oc = oracle_codec_like(codec)
    ol = kvq.Outliers(codec, n, capacity=n * D // 16, device=DEV)
    say(f"heavy-tailed V: n={n}, b={bits}, T={T_}")
    rec, total = kvq.encode(codec, x, outliers=ol, want_total=True)
    rate = total / (n * D)
    say(f"  outliers {total} ({100 * rate:.2f} % of coordinates)")
    assert 0.01 < rate < 0.05
    off = ol.offsets.cpu().numpy().view(np.uint32).astype(np.int64)
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[-1] == total
    rows = _sample(n, 4000, seed=4)
    xs = bf16_host(_take(x, rows))
    ref = oracle.encode(oc, xs)
    got = _take(rec, rows).cpu().numpy()
    mism, flagged = compare_codes(got, ref, D, bits, "heavy-tailed codes")
    idx = ol.idx[:total].cpu().numpy()
    val = ol.val[:total].cpu().numpy().view(np.uint16)
    differing = compare_outlier_lists(off, idx, val, ref, rows, "heavy-tailed outliers")
    say(f"  {len(rows)} sampled vectors' lists: {differing} differ, each only at near-T coordinates")
    sub_off, sub_idx, sub_val = [0], [np.zeros(0, np.uint8)], [np.zeros(0, np.uint16)]
    for k, v in enumerate(rows):
        gi, gv = idx[off[v]:off[v + 1]], val[off[v]:off[v + 1]]
        sub_idx.append(gi)
        sub_val.append(gv)
        sub_off.append(sub_off[-1] + len(gi))
    y = kvq.decode(codec, rec, outliers=ol)
    ys = _take(y, rows).cpu().numpy()
    yref = oracle.decode(oc, got, np.array(sub_off, np.uint32), np.concatenate(sub_idx),
                         np.concatenate(sub_val))
    worst = compare_decoded(ys, yref, unpack_records(got, D, bits)[1], "heavy-tailed decode")
    y0 = _take(kvq.decode(codec, rec), rows).cpu().numpy()
    xf = _f64(xs)
    nx = np.linalg.norm(xf, axis=1)
    e_with = float(np.mean(np.linalg.norm(ys - xf, axis=1) / nx))
    e_without = float(np.mean(np.linalg.norm(y0 - xf, axis=1) / nx))
    say(f"  codes: mismatches {mism} flagged {flagged}; decode worst err/||x|| {worst:.2e}; "
        f"L2-rel error {e_with:.3f} with the side list, {e_without:.3f} without")
    assert e_with < e_without


def test_v4_flash_geometry_outlier_lists_full_size():
    """One V4-Flash-shaped layer (65,536 rows of head_dim 512, iid N(0,1)), 4 bits, T = 2.0: the
    outlier lists carry u16 indices; sampled vectors' codes and lists against the oracle, CSR
    monotone, decode with the list against the oracle on the GPU's own records and list."""
    D, bits, T_ = 512, 4, 2.0
    x = synth.iid_normal((65536, D), seed=1003, device=DEV)
    n = x.shape[0]
    codec = kvq.Codec(D, bits, seed=42, outlier_T=T_)
    oc = oracle_codec_like(codec)
    ol = kvq.Outliers(codec, n, capacity=n * D // 8, device=DEV)
    say(f"v4-flash geometry outliers: n={n}, D={D}, b={bits}, T={T_}")
    rec, total = kvq.encode(codec, x, outliers=ol, want_total=True)
    rate = total / (n * D)
    say(f"  outliers {total} ({100 * rate:.2f} % of coordinates)")
    assert 0.04 < rate < 0.05
    off = ol.offsets.cpu().numpy().view(np.uint32).astype(np.int64)
    assert off[0] == 0 and np.all(np.diff(off) >= 0) and off[-1] == total
    idx = ol.idx[:total].cpu().numpy().view(np.uint16)
    val = ol.val[:total].cpu().numpy().view(np.uint16)
    assert idx.max() > 255
    rows = _sample(n, 1500, seed=9)
    ref = oracle.encode(oc, bf16_host(_take(x, rows)))
    got = _take(rec, rows).cpu().numpy()
    compare_codes(got, ref, D, bits, "v4-flash geometry codes")
    compare_outlier_lists(off, idx, val, ref, rows, "v4-flash geometry outliers")
    sub_off, sub_idx, sub_val = [0], [], []
    for v in rows:
        sub_idx.append(idx[off[v]:off[v + 1]])
        sub_val.append(val[off[v]:off[v + 1]])
        sub_off.append(sub_off[-1] + off[v + 1] - off[v])
    y = kvq.decode(codec, rec, outliers=ol)
    yref = oracle.decode(oc, got, np.array(sub_off, np.uint32), np.concatenate(sub_idx),
                         np.concatenate(sub_val))
    compare_decoded(_take(y, rows).cpu().numpy(), yref, unpack_records(got, D, bits)[1],
                    "v4-flash geometry decode")


def test_long_context_score_full_size():
    """K [8, 8, 131072, 128] iid N(0,1) at 3 bits; q [8, 32, 128]; GQA 4:1."""
    B, Hkv, T, D, Hq, bits = 8, 8, 131072, 128, 32, 3
    K, q = synth.long_context_keys(device=DEV)
    x = K.reshape(-1, D)
    n = x.shape[0]
    codec = kvq.Codec(D, bits, seed=42)
    oc = oracle_codec_like(codec)
    say(f"long-context score: {n} keys, q {tuple(q.shape)}")
    rec = kvq.encode(codec, x)
    s = kvq.score_packed(codec, q, rec, Hkv, T, rec_sb=Hkv * T, rec_sh=T)
    torch.cuda.synchronize()
    assert torch.isfinite(s).all()
    rows = _sample(n, 3000, seed=5)
    ref = oracle.encode(oc, bf16_host(_take(x, rows)))
    compare_codes(_take(rec, rows).cpu().numpy(), ref, D, bits, "long-context codes")
    rng = np.random.default_rng(6)
    m = 4000
    bs = np.concatenate([rng.integers(0, B, m), [0, B - 1]])
    hs = np.concatenate([rng.integers(0, Hq, m), [0, Hq - 1]])
    ts = np.concatenate([rng.integers(0, T, m), [0, T - 1]])
    kv = hs * Hkv // Hq
    recs = _take(rec, bs * Hkv * T + kv * T + ts).cpu().numpy()
    qh = bf16_host(q)[bs, hs]
    sref = oracle.score(oc, qh, recs)
    sg = s[torch.from_numpy(bs).to(DEV), torch.from_numpy(hs).to(DEV),
           torch.from_numpy(ts).to(DEV)].cpu().numpy().astype(np.float64)
    worst = check_scores(sg, sref, score_scale(oc, qh, recs), "long-context scores")
    say(f"  {len(bs)} sampled scores, worst err/bound {worst:.3f}")


def test_qwen2_shaped_cache_full_size():
    """[28, 4, 2, 2048, 128] with per-channel lognormal scales, 22 coded layers. K: PCA r=64 per
    (layer, KV head) + 3 bits; V: 2 bits; decode both to bf16; score 12 query heads."""
    L, B, H, T, D, R, HQ = 28, 4, 2, 2048, 128, 64, 12
    lo, hi = 3, 25
    lc = hi - lo
    K, V = synth.qwen2_1p5b_cache(layers=L, batch=B, kv_heads=H, tokens=T, head_dim=D,
                                  seed=1002, device=DEV)
    Kc, Vc = K[lo:hi].contiguous(), V[lo:hi].contiguous()
    del K, V
    mus, bases = [], []
    for li in range(lc):
        for h in range(H):
            mu, basis = synth.pca_basis_from_calibration(Kc[li, 0, h, :512], R)
            mus.append(mu)
            bases.append(basis)
    basis = torch.stack(bases).to(DEV).contiguous()
    mean = torch.from_numpy(np.stack(mus)).to(DEV).contiguous()
    blocks = torch.arange(lc * B * H, dtype=torch.int32)
    index = ((blocks // (B * H)) * H + blocks % H).to(torch.int32)
    ck = kvq.Codec(D, 3, seed=42, proj_rank=R, basis=basis, mean=mean,
                   basis_index=index.to(DEV), basis_block_rows=T)
    cv = kvq.Codec(D, 2, seed=43)
    xk, xv = Kc.reshape(-1, D), Vc.reshape(-1, D)
    n = xk.shape[0]
    say(f"qwen2-shaped cache: {n} K and {n} V rows")
    rk, rv = kvq.encode(ck, xk), kvq.encode(cv, xv)
    yk = kvq.decode(ck, rk, dtype=torch.bfloat16)
    yv = kvq.decode(cv, rv, dtype=torch.bfloat16)
    q = synth.iid_normal((lc * B, HQ, D), seed=1102, device=DEV)
    s = kvq.score_packed(ck, q, rk, H, T, rec_sb=H * T, rec_sh=T)
    torch.cuda.synchronize()
    rows = _sample(n, 3000, seed=7)
    # V: Hadamard path
    ocv = oracle_codec_like(cv)
    gv = _take(rv, rows).cpu().numpy()
    compare_codes(gv, oracle.encode(ocv, bf16_host(_take(xv, rows))), D, 2, "V codes")
    yref = oracle.decode(ocv, gv)
    compare_decoded(_f64(bf16_host(_take(yv, rows))), yref, unpack_records(gv, D, 2)[1],
                    "V decode (bf16)", extra_ulp_bf16=True)
    # K: PCA path, grouped by basis
    bhost = synth.bf16_bits(basis)
    mhost = mean.cpu().numpy()
    bidx = index.numpy()[rows // T]
    gk = _take(rk, rows).cpu().numpy()
    xs = bf16_host(_take(xk, rows))
    yks = _f64(bf16_host(_take(yk, rows)))
    for k in np.unique(bidx):
        sel = bidx == k
        ock = oracle_codec_like(ck, basis_host=bhost[k], mean_host=mhost[k])
        compare_codes(gk[sel], oracle.encode(ock, xs[sel]), R, 3, f"K codes basis {k}")
        yr = oracle.decode(ock, gk[sel])
        compare_decoded(yks[sel], yr, np.linalg.norm(yr, axis=1), f"K decode basis {k}",
                        extra_ulp_bf16=True)
    # scores at sampled (layer*batch, query head, token)
    rng = np.random.default_rng(8)
    m = 3000
    bb = np.concatenate([rng.integers(0, lc * B, m), [0, lc * B - 1]])
    hq = np.concatenate([rng.integers(0, HQ, m), [0, HQ - 1]])
    tt = np.concatenate([rng.integers(0, T, m), [0, T - 1]])
    kvh = hq * H // HQ
    ridx = bb * H * T + kvh * T + tt
    recs = _take(rk, ridx).cpu().numpy()
    qh = bf16_host(q)[bb, hq]
    sg = s[torch.from_numpy(bb).to(DEV), torch.from_numpy(hq).to(DEV),
           torch.from_numpy(tt).to(DEV)].cpu().numpy().astype(np.float64)
    kb = index.numpy()[ridx // T]
    for k in np.unique(kb):
        sel = kb == k
        ock = oracle_codec_like(ck, basis_host=bhost[k], mean_host=mhost[k])
        sref = oracle.score(ock, qh[sel], recs[sel])
        check_scores(sg[sel], sref, score_scale(ock, qh[sel], recs[sel]), f"scores, basis {k}")
    say(f"  {len(rows)} sampled rows per stream and {len(bb)} sampled scores agree")
