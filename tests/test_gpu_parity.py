"""GPU parity of the HIP codec against the CPU oracle, through the C ABI.

Bars: codes bit-exact except coordinates within 1e-5 of a decision boundary (those mismatches
<= 1e-4 of coordinates); norms within 1e-5 relative; decode (f32, same records) within
1e-3*||x||; scores within 1e-3 of max(|s|, sum of |terms|) on the same records.
"""
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


def _rows(n, D, seed, scale=1.0, ld=None):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    ld = ld or D
    x = torch.zeros(n, ld, dtype=torch.bfloat16, device=DEV)
    x[:, :D] = (scale * torch.randn(n, D, generator=g, device=DEV)).to(torch.bfloat16)
    return x


def _encode_both(codec, x, D):
    say(f"encode D={D} b={codec.bits} n={x.shape[0]} ld={x.stride(0)} seed={codec.seed}")
    rec = kvq.encode(codec, x)
    torch.cuda.synchronize()
    ref = oracle.encode(oracle_codec_like(codec), bf16_host(x[:, :D]))
    return rec.cpu().numpy(), ref


@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_encode_decode_parity_hadamard(D, bits):
    n = 1000 + 37 * bits + D // 64  # not a multiple of any tile
    x = _rows(n, D, seed=D * 10 + bits, ld=D + 8 * (bits % 2))
    codec = kvq.Codec(D, bits, seed=42 + bits)
    rec, ref = _encode_both(codec, x, D)
    mism, flagged = compare_codes(rec, ref, D, bits, f"D={D} b={bits}")
    say(f"  code mismatches {mism}, flagged {flagged}")
    # decode of the GPU records: GPU vs oracle, f32 and bf16
    recd = torch.from_numpy(rec).to(DEV)
    y32 = kvq.decode(codec, recd, dtype=torch.float32)
    y16 = kvq.decode(codec, recd, dtype=torch.bfloat16)
    torch.cuda.synchronize()
    yref = oracle.decode(oracle_codec_like(codec), rec)
    _, norms = unpack_records(rec, D, bits)
    compare_decoded(y32.cpu().numpy(), yref, norms, f"decode f32 D={D} b={bits}")
    compare_decoded(y16.float().cpu().numpy(), yref, norms, f"decode bf16 D={D} b={bits}",
                    extra_ulp_bf16=True)


@pytest.mark.parametrize("D,bits", [(128, 2), (128, 3), (512, 4)])
def test_custom_asymmetric_table(D, bits):
    L = 1 << bits
    c = oracle.gaussian_table(bits)[1].astype(np.float64)
    c = (c * (1.0 + 0.05 * np.sin(np.arange(L))) + 0.03).astype(np.float32)  # still ascending
    assert np.all(np.diff(c) > 0) and not np.array_equal(c, -c[::-1])
    codec = kvq.Codec(D, bits, seed=9, centroids=c)
    x = _rows(700, D, seed=5)
    rec, ref = _encode_both(codec, x, D)
    compare_codes(rec, ref, D, bits, "custom table")
    y = kvq.decode(codec, torch.from_numpy(rec).to(DEV))
    yref = oracle.decode(oracle_codec_like(codec), rec)
    compare_decoded(y.cpu().numpy(), yref, unpack_records(rec, D, bits)[1], "custom decode")


def test_edge_vectors_zero_single_and_scaled():
    D, bits = 128, 3
    codec = kvq.Codec(D, bits, seed=3)
    x = _rows(67, D, seed=11)
    x[5] = 0
    x[6, :] = 0
    x[6, 17] = 1.0   # one nonzero coordinate
    x[7] = x[8] * 64  # power-of-two scale
    rec, ref = _encode_both(codec, x, D)
    compare_codes(rec, ref, D, bits, "edge")
    codes, norms = unpack_records(rec, D, bits)
    assert norms[5] == 0 and np.all(codes[5] == 3)
    # n = 1 and n = 0
    one = kvq.encode(codec, x[:1].contiguous())
    np.testing.assert_array_equal(one.cpu().numpy()[0], rec[0])
    empty = kvq.encode(codec, x[:0])
    assert empty.shape[0] == 0


@pytest.mark.parametrize("D,bits", [(128, 2), (64, 3), (128, 1), (256, 3), (512, 4), (512, 1)])
@pytest.mark.parametrize("n", [1, 17, 255, 257, 4099])
def test_decode_strided_output_and_ragged_n(D, bits, n):
    """Decode into rows wider than D (ld = D + 24): the columns past D stay untouched; vector
    counts below, at and past the block tile (256) and a ragged large count."""
    codec = kvq.Codec(D, bits, seed=21)
    x = _rows(n, D, seed=n + D + bits)
    rec = kvq.encode(codec, x)
    for dt in (torch.float32, torch.bfloat16):
        big = torch.full((n, D + 24), 7.0, dtype=dt, device=DEV)
        kvq.decode(codec, rec, out=big[:, :D])
        torch.cuda.synchronize()
        recn = rec.cpu().numpy()
        yref = oracle.decode(oracle_codec_like(codec), recn)
        _, norms = unpack_records(recn, D, bits)
        compare_decoded(big[:, :D].float().cpu().numpy(), yref, norms, f"strided decode {dt} n={n}",
                        extra_ulp_bf16=dt == torch.bfloat16)
        assert torch.all(big[:, D:] == 7.0), "decode wrote past the row's D columns"


def test_scale_invariance_on_gpu():
    D, bits = 256, 4
    codec = kvq.Codec(D, bits, seed=13)
    x = _rows(512, D, seed=17)
    a = kvq.encode(codec, x).cpu().numpy()
    b = kvq.encode(codec, (x.float() * 4).to(torch.bfloat16)).cpu().numpy()
    ca, na = unpack_records(a, D, bits)
    cb, nb = unpack_records(b, D, bits)
    np.testing.assert_array_equal(ca, cb)
    np.testing.assert_array_equal(nb, na * 4)


@pytest.mark.parametrize("D,bits,G", [(128, 3, 4), (64, 2, 1), (256, 4, 2), (512, 4, 8), (128, 1, 4)])
def test_score_packed_parity(D, bits, G):
    B, Hkv, T = 2, 2, 300
    Hq = Hkv * G
    codec = kvq.Codec(D, bits, seed=21)
    k = _rows(B * Hkv * T, D, seed=31)
    rec = kvq.encode(codec, k)
    q = _rows(B * Hq, D, seed=41).view(B, Hq, D)
    say(f"score D={D} b={bits} G={G} B={B} Hkv={Hkv} T={T}")
    s = kvq.score_packed(codec, q, rec, Hkv, T, rec_sb=Hkv * T, rec_sh=T)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    rec_h = rec.cpu().numpy().reshape(B, Hkv, T, -1)
    q_h = bf16_host(q)
    oc = oracle_codec_like(codec)
    qq = np.repeat(q_h[:, :, None, :], T, axis=2)                       # [B, Hq, T, D]
    rr = rec_h[:, np.arange(Hq) // G]                                   # [B, Hq, T, rb]
    ref = oracle.score(oc, qq.reshape(-1, D), rr.reshape(-1, rr.shape[-1])).reshape(B, Hq, T)
    # normwise scale: (n/D) sum_i |q'_i z^_i|
    sgn = oracle.signs(codec.seed, D).astype(np.float64)
    qv = (q_h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qp = oracle.fwht_rows(qv * sgn)                                    # [B, Hq, D]
    codes, norms = unpack_records(rr.reshape(-1, rr.shape[-1]), D, bits)
    zh = oc.centroids.astype(np.float64)[codes].reshape(B, Hq, T, D)
    scale = norms.reshape(B, Hq, T) / D * np.abs(qp[:, :, None, :] * zh).sum(-1)
    err = np.abs(s - ref)
    bound = 1e-3 * np.maximum(np.abs(ref), scale)
    assert np.all(err <= bound), f"score error {err.max():.3g} (bound min {bound.min():.3g})"


@pytest.mark.parametrize("T", [1, 15, 16, 63, 64, 255, 256, 257, 1000])
def test_score_packed_ragged_lengths_and_strides(T):
    """Every context length against the kernel's 16-token tiles, 64-token wave steps and
    256-token segments, with padded record and score layouts (rec_sh = T + 5, rec_sb with 7
    spare records; s_sh = T + 9, s_sb with 3 spare floats): scores within the normwise bar of the
    oracle, and no score slot outside [0, T) of each row written."""
    D, bits, G, B, Hkv = 128, 3, 2, 2, 3
    Hq = Hkv * G
    codec = kvq.Codec(D, bits, seed=23)
    rec_sh, rec_sb = T + 5, Hkv * (T + 5) + 7
    s_sh, s_sb = T + 9, Hq * (T + 9) + 3
    k = _rows(B * rec_sb, D, seed=T + 77)
    rec = kvq.encode(codec, k)
    q = _rows(B * Hq, D, seed=T + 78).view(B, Hq, D)
    say(f"score ragged T={T} B={B} Hkv={Hkv} G={G}")
    SENT = 12345.0
    buf = torch.full((B * s_sb,), SENT, dtype=torch.float32, device=DEV)
    out = torch.as_strided(buf, (B, Hq, T), (s_sb, s_sh, 1))
    kvq.score_packed(codec, q, rec, Hkv, T, rec_sb=rec_sb, rec_sh=rec_sh, out=out)
    torch.cuda.synchronize()
    hb = buf.cpu().numpy()
    written = np.zeros(B * s_sb, bool)
    for b_ in range(B):
        for h in range(Hq):
            written[b_ * s_sb + h * s_sh: b_ * s_sb + h * s_sh + T] = True
    assert np.all(hb[~written] == SENT), "a score slot outside [0, T) was written"
    s = out.cpu().numpy()
    rec_h = rec.cpu().numpy()
    oc = oracle_codec_like(codec)
    q_h = bf16_host(q)
    for b_ in range(B):
        for h in range(Hq):
            kv = h // G
            rows = b_ * rec_sb + kv * rec_sh + np.arange(T)
            recs = rec_h[rows]
            ref = oracle.score(oc, np.repeat(q_h[b_, h][None], T, axis=0), recs)
            check_scores(s[b_, h], ref, score_scale(oc, np.repeat(q_h[b_, h][None], T, axis=0), recs),
                         f"score T={T} b={b_} h={h}")


@pytest.mark.parametrize("cscale", [2.0 ** -30, 1.0, 2.0 ** 30])
def test_score_packed_query_and_table_scales(cscale):
    """The score's f16 products hold each query head and the centroid table scaled by powers of
    two: heads 2^40, 2^-40, zero and unit in one GQA group, and tables scaled by 2^-30 .. 2^30,
    stay within the normwise bound of the oracle's score."""
    D, bits, G, B, Hkv, T = 128, 3, 4, 1, 2, 300
    Hq = Hkv * G
    cent = np.array([-2.2, -1.3, -0.7, -0.2, 0.25, 0.8, 1.4, 2.1], np.float64) * cscale
    codec = kvq.Codec(D, bits, seed=23, centroids=cent.astype(np.float32))
    k = _rows(B * Hkv * T, D, seed=33)
    rec = kvq.encode(codec, k)
    q = _rows(B * Hq, D, seed=43).view(B, Hq, D)
    head_scale = torch.tensor([2.0 ** 40, 2.0 ** -40, 0.0, 1.0] * Hkv, device=DEV)
    q = (q.float() * head_scale[None, :, None]).to(torch.bfloat16)
    say(f"score scales D={D} b={bits} G={G} table x{cscale:g}")
    s = kvq.score_packed(codec, q, rec, Hkv, T, rec_sb=Hkv * T, rec_sh=T)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    rec_h = rec.cpu().numpy().reshape(B, Hkv, T, -1)
    q_h = bf16_host(q)
    oc = oracle_codec_like(codec)
    qq = np.repeat(q_h[:, :, None, :], T, axis=2)
    rr = rec_h[:, np.arange(Hq) // G]
    ref = oracle.score(oc, qq.reshape(-1, D), rr.reshape(-1, rr.shape[-1])).reshape(B, Hq, T)
    sgn = oracle.signs(codec.seed, D).astype(np.float64)
    qv = (q_h.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    qp = oracle.fwht_rows(qv * sgn)
    codes, norms = unpack_records(rr.reshape(-1, rr.shape[-1]), D, bits)
    zh = oc.centroids.astype(np.float64)[codes].reshape(B, Hq, T, D)
    scale = norms.reshape(B, Hq, T) / D * np.abs(qp[:, :, None, :] * zh).sum(-1)
    err = np.abs(s - ref)
    bound = 1e-3 * np.maximum(np.abs(ref), scale)
    assert np.all(err <= bound), f"score error {err.max():.3g} (bound min {bound.min():.3g})"
    assert np.all(s[:, 2::G] == 0.0), "a zero query head scores zero"


@pytest.mark.parametrize("D,bits,T_", [(128, 2, 2.0), (64, 3, 1.5), (256, 2, 2.5), (128, 4, 2.0),
                                       (512, 4, 2.0), (512, 2, 1.8), (128, 3, 1.85), (128, 2, 1.3)])
def test_outlier_parity(D, bits, T_):
    """Every vector's CSR entries against the oracle's. At coded length 128 the entries of a
    16-vector tile are staged by the first pass when there are at most 128 of them and copied
    after the scan; T = 1.85 leaves some tiles over that budget (recomputed from the rows), T =
    1.3 all of them."""
    n = 3000 + 13
    x = _rows(n, D, seed=D + bits)
    x[:, 3] *= 16  # heavy channel
    codec = kvq.Codec(D, bits, seed=5, outlier_T=T_)
    ol = kvq.Outliers(codec, n, capacity=n * D // 4, device=DEV)
    say(f"outliers D={D} b={bits} T={T_} n={n}")
    rec, total = kvq.encode(codec, x, outliers=ol, want_total=True)
    ref = oracle.encode(oracle_codec_like(codec), bf16_host(x))
    recn = rec.cpu().numpy()
    compare_codes(recn, ref, D, bits, "outlier codes")
    off = ol.offsets.cpu().numpy().view(np.uint32)
    idx = ol.idx.cpu().numpy()
    idx = idx.view(np.uint16) if D > 256 else idx   # u16 indices above 256 coordinates
    val = ol.val.cpu().numpy().view(np.uint16)
    roff = ref["offsets"]
    near_t = (ref["flags"] & oracle.FLAG_NEAR_T) != 0
    per_vec_ok = np.diff(off.astype(np.int64)) == np.diff(roff.astype(np.int64))
    # counts may differ only for vectors with a coordinate within 1e-5 of T
    bad = ~per_vec_ok & ~near_t.any(1)
    assert not bad.any(), f"outlier counts differ at unflagged vectors {np.nonzero(bad)[0][:5]}"
    assert total == off[-1] and abs(int(off[-1]) - ref["total"]) <= near_t.sum()
    rate = ref["total"] / (n * D)
    say(f"  outliers {total} (oracle {ref['total']}), rate {rate:.4f}")
    differing = compare_outlier_lists(off, idx, val, ref, None, "outlier lists")
    say(f"  lists of all {n} vectors compared: {differing} differ, only at near-T coordinates")
    # decode with the side list: GPU vs oracle on the GPU's own records and list
    y = kvq.decode(codec, rec, outliers=ol)
    yref = oracle.decode(oracle_codec_like(codec), recn, off, idx[:total], val[:total])
    compare_decoded(y.cpu().numpy(), yref, unpack_records(recn, D, bits)[1], "outlier decode")


@pytest.mark.parametrize("D,bits,n", [(128, 2, 1000 + 7), (64, 3, 999), (128, 3, 33)])
def test_outlier_decode_bf16_rows_with_a_ragged_tail(D, bits, n):
    """Decode with side lists to bf16 rows when n is not a multiple of the kernel's 32-vector
    step: the lanes past the end decode the last record again and store its row again, so they
    must apply that record's entries too (the last row must equal the oracle's)."""
    x = _rows(n, D, seed=3 * D + bits + n)
    x[:, 5] *= 12  # heavy channel: many entries per vector, the last included
    codec = kvq.Codec(D, bits, seed=11, outlier_T=1.5)
    ol = kvq.Outliers(codec, n, capacity=n * D // 2, device=DEV)
    say(f"outlier decode bf16 D={D} b={bits} n={n}")
    rec, total = kvq.encode(codec, x, outliers=ol, want_total=True)
    recn = rec.cpu().numpy()
    off = ol.offsets.cpu().numpy().view(np.uint32)
    idx = ol.idx.cpu().numpy()
    val = ol.val.cpu().numpy().view(np.uint16)
    assert off[-1] - off[-2] > 0, "the last vector carries entries"
    y = kvq.decode(codec, rec, outliers=ol, dtype=torch.bfloat16)
    y32 = y.float().cpu().numpy()
    yref = oracle.decode(oracle_codec_like(codec), recn, off, idx[:total], val[:total])
    compare_decoded(y32, yref, unpack_records(recn, D, bits)[1], "outlier decode (bf16)",
                    extra_ulp_bf16=True)


@pytest.mark.parametrize("D,cut", [(128, "none"), (128, "half"), (64, "half"), (256, "half")])
def test_outlier_decode_with_a_list_cut_at_capacity(D, cut):
    """Decode applies exactly the entries below the capacity (none at capacity 0): the vectors
    whose span is cut keep their first entries, those past the cut keep none."""
    bits, n = 2, 1500 + 9
    x = _rows(n, D, seed=D + 61)
    x[:, 9] *= 14
    codec = kvq.Codec(D, bits, seed=13, outlier_T=1.6)
    full = kvq.Outliers(codec, n, capacity=n * D // 2, device=DEV)
    rec, total = kvq.encode(codec, x, outliers=full, want_total=True)
    cap = 0 if cut == "none" else total // 2 + 5
    part = kvq.Outliers(codec, n, capacity=cap, device=DEV)
    say(f"outlier decode with the list cut at {cap} of {total} entries, D={D}")
    rec_p = kvq.encode(codec, x, outliers=part)
    torch.cuda.synchronize()
    assert torch.equal(rec_p, rec)
    recn = rec.cpu().numpy()
    off = part.offsets.cpu().numpy().view(np.uint32)
    idx = part.idx.cpu().numpy()[:cap]
    val = part.val.cpu().numpy().view(np.uint16)[:cap]
    yref = oracle.decode(oracle_codec_like(codec), recn, off, idx, val)
    norms = unpack_records(recn, D, bits)[1]
    for dt in (torch.float32, torch.bfloat16):
        y = kvq.decode(codec, rec_p, outliers=part, dtype=dt)
        compare_decoded(y.float().cpu().numpy(), yref, norms, f"decode cut at {cap} ({dt})",
                        extra_ulp_bf16=dt == torch.bfloat16)


@pytest.mark.parametrize("T_", [2.2, 1.85, 1.3])
def test_outlier_list_cut_at_capacity_is_a_prefix(T_):
    """A list cut short by the capacity holds exactly the first `capacity` entries of the full
    list (staged tiles are copied, tiles over the staging budget recomputed, both clipped)."""
    D, bits, n = 128, 2, 2000 + 5
    codec = kvq.Codec(D, bits, seed=8, outlier_T=T_)
    x = _rows(n, D, seed=41)
    x[:, 7] *= 10
    full = kvq.Outliers(codec, n, capacity=n * D, device=DEV)
    rec_f, total = kvq.encode(codec, x, outliers=full, want_total=True)
    cap = total // 2 + 3
    part = kvq.Outliers(codec, n, capacity=cap, device=DEV)
    say(f"outlier list cut at {cap} of {total} (T={T_})")
    with pytest.raises(kvq.KvqError) as ei:
        kvq.encode(codec, x, outliers=part, want_total=True)
    assert ei.value.name == "KVQ_E_CAPACITY"
    rec_p = kvq.encode(codec, x, outliers=part)
    torch.cuda.synchronize()
    assert torch.equal(rec_p, rec_f)
    assert torch.equal(part.offsets, full.offsets)
    assert torch.equal(part.idx[:cap], full.idx[:cap]) and torch.equal(part.val[:cap], full.val[:cap])


def test_outlier_capacity_overflow_reports_and_truncates():
    D, bits, n = 128, 2, 2000
    codec = kvq.Codec(D, bits, seed=5, outlier_T=1.0)
    x = _rows(n, D, seed=99)
    ol = kvq.Outliers(codec, n, capacity=100, device=DEV)
    with pytest.raises(kvq.KvqError) as ei:
        kvq.encode(codec, x, outliers=ol, want_total=True)
    assert ei.value.name == "KVQ_E_CAPACITY"
    off = ol.offsets.cpu().numpy().view(np.uint32)
    ref = oracle.encode(oracle_codec_like(codec), bf16_host(x), ol_cap=100)
    assert abs(int(off[-1]) - ref["total"]) <= ((ref["flags"] & 2) != 0).sum()
    y = kvq.decode(codec, kvq.encode(codec, x, outliers=ol), outliers=ol)  # decode ignores the tail
    assert torch.isfinite(y).all()


def _append_evict_against_model(window, margin, tail_cap, t_news, n_caches=3, seed=1):
    D, bits = 128, 3
    codec = kvq.Codec(D, bits, seed=77)
    caches = [kvq.Cache(codec, packed_cap=4096, tail_cap=tail_cap, window=window, margin=margin,
                        device=DEV) for _ in range(n_caches)]
    models = [oracle.CacheModel(oracle_codec_like(codec), window, margin) for _ in range(n_caches)]
    appended = [np.zeros((0, D), np.uint16) for _ in range(n_caches)]
    for t_new in t_news:
        rows = [_rows(max(t_new, 1), D, seed=seed + k) for k in range(n_caches)]
        seed += 10
        say(f"append t_new={t_new} (tail_cap={tail_cap}, window={window})")
        ev = kvq.append_evict_chunk(codec, caches, rows if t_new else None, t_new)
        for k in range(n_caches):
            host = bf16_host(rows[k][:t_new]) if t_new else np.zeros((0, D), np.uint16)
            appended[k] = np.concatenate([appended[k], host])
            assert ev[k] == models[k].append_evict(host)
        torch.cuda.synchronize()
        for k in range(n_caches):
            c, mdl = caches[k], models[k]
            assert c.tail_len == len(mdl.tail) and c.packed_len == len(mdl.packed)
            np.testing.assert_array_equal(bf16_host(c.tail_rows()), np.stack(mdl.tail))
            if c.packed_len:
                got = c.packed[: c.packed_len].cpu().numpy()
                ref = oracle.encode(oracle_codec_like(codec), appended[k][: c.packed_len])
                compare_codes(got, ref, D, bits, f"evict cache {k}")
    return caches


def test_append_evict_matches_oracle_model():
    _append_evict_against_model(200, 16, 1500, [700, 1, 1, 129, 0, 1, 300, 5, 0, 1])


def test_append_evict_with_a_cache_set_and_one_row_tensor():
    """The binding's reusable CacheSet with one [n_caches, t, D] row tensor (rows of different
    caches at any stride) drives the same calls as a list of caches and per-cache tensors: the
    packed regions and tails end bit-identical, across evictions."""
    D, bits, L = 128, 3, 3
    codec = kvq.Codec(D, bits, seed=91)
    mk = lambda: [kvq.Cache(codec, packed_cap=2048, tail_cap=700, window=160, margin=16, device=DEV)
                  for _ in range(L)]
    a, b = mk(), mk()
    cs = kvq.CacheSet(b)
    say(f"append/evict through a CacheSet, {L} caches")
    big = _rows(L * 1200, D, seed=5).view(L, 1200, D)
    t = 0
    for t_new in (300, 1, 1, 129, 0, 250, 1, 77):
        rows = big[:, t:t + t_new] if t_new else None
        ev_a = kvq.append_evict_chunk(codec, a, [rows[i] for i in range(L)] if t_new else None, t_new)
        ev_b = kvq.append_evict_chunk(codec, cs, rows, t_new)
        assert ev_a == ev_b
        t += t_new
    torch.cuda.synchronize()
    for ca, cb in zip(a, b):
        assert (ca.packed_len, ca.tail_len, ca.tail_head) == (cb.packed_len, cb.tail_len, cb.tail_head)
        assert ca.packed_len > 0
        assert torch.equal(ca.packed[: ca.packed_len], cb.packed[: cb.packed_len])
        assert torch.equal(ca.tail_rows(), cb.tail_rows())


def test_append_evict_tail_ring_wraps():
    """A 480-row tail ring whose head passes its end several times: the evicted chunks read
    rows across the wrap."""
    t_news = [150, 1, 130, 64, 1, 1, 120, 37, 0, 150, 1, 90, 149, 1, 77, 150, 3, 140, 1, 66]
    caches = _append_evict_against_model(160, 16, 480, t_news, seed=501)
    assert all(c.packed_len > 480 for c in caches)  # more rows left the ring than it holds: it wrapped


def test_config1_full_roundtrip():
    """8 KV heads x 2048 tokens x head_dim 128, channels 7 and 93 x8; K b=3, V b=2."""
    K, V = synth.kv_pair_outlier_channels(device=DEV)
    for name, X, bits in (("K", K, 3), ("V", V, 2)):
        x = X.reshape(-1, 128)
        codec = kvq.Codec(128, bits, seed=42)
        rec, ref = _encode_both(codec, x, 128)
        mism, flagged = compare_codes(rec, ref, 128, bits, f"config1 {name}")
        y = kvq.decode(codec, torch.from_numpy(rec).to(DEV))
        yref = oracle.decode(oracle_codec_like(codec), rec)
        worst = compare_decoded(y.cpu().numpy(), yref, unpack_records(rec, 128, bits)[1], "config1")
        say(f"config1 {name}: mismatches {mism} flagged {flagged} worst decode err/||x|| {worst:.2e}")


def _rule_scale(rule, n, z, zh, m):
    """The stored scale of a rule in f64 from the norm, z and the chosen centroids."""
    zu, zz = float((z * zh).sum()), float((zh * zh).sum())
    if n == 0:
        return 0.0
    if rule == 1 and zz > 0:
        return n * np.sqrt(m / zz)
    if rule == 2 and zu > 0:
        return n * m / zu
    if rule == 3 and zz > 0:
        return n * zu / zz
    return n


@pytest.mark.parametrize("rule", [1, 2, 3])
@pytest.mark.parametrize("D,bits,custom", [(64, 1, False), (128, 2, False), (128, 3, True),
                                           (256, 3, False), (512, 4, False)])
def test_scale_rules_parity(rule, D, bits, custom):
    """Codes equal the plain rule's; the stored scale matches the oracle's (recomputed from the
    GPU's own codes where a boundary-flagged coordinate differs); the decoded vectors meet the
    rule's identity."""
    c = None
    if custom:  # an asymmetric table takes the kernels' general compare path
        c = oracle.gaussian_table(bits)[1].astype(np.float64)
        c = (c * (1.0 + 0.05 * np.sin(np.arange(1 << bits))) + 0.03).astype(np.float32)
    codec = kvq.Codec(D, bits, seed=70 + rule, centroids=c, flags=rule)
    n = 777
    x = _rows(n, D, seed=D + bits + rule, scale=1.5)
    say(f"scale rule {rule} D={D} b={bits} custom={custom}")
    rec = kvq.encode(codec, x)
    torch.cuda.synchronize()
    recn = rec.cpu().numpy()
    ocd = oracle_codec_like(codec)
    ref = oracle.encode(ocd, bf16_host(x))
    gc, gs = unpack_records(recn, D, bits)
    rc, rs = unpack_records(ref["records"], D, bits)
    mism = gc != rc
    assert not (mism & (ref["flags"] == 0)).any(), "unflagged code mismatch"
    cen = ocd.centroids.astype(np.float64)
    for v in range(n):
        want = rs[v] if not mism[v].any() else _rule_scale(rule, ref["norms"][v], ref["z"][v],
                                                           cen[gc[v]], D)
        assert abs(gs[v] - want) <= 1e-5 * abs(want) + 1e-30, f"vector {v}: {gs[v]} vs {want}"
    y = kvq.decode(codec, rec).double().cpu()
    xf = torch.from_numpy((bf16_host(x).astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    if rule == 1:
        torch.testing.assert_close(y.norm(dim=1), xf.norm(dim=1), rtol=1e-4, atol=0)
    elif rule == 2:
        torch.testing.assert_close((y * xf).sum(1), (xf * xf).sum(1), rtol=1e-4, atol=0)
    else:
        r = ((xf - y) * y).sum(1).abs()
        assert torch.all(r <= 1e-4 * xf.norm(dim=1) * y.norm(dim=1))


def test_truncate_and_reappend_match_the_model():
    """Appends, shallow rollbacks (inside the dense tail), a deep rollback into the packed region
    and appends after them, on two caches at once, against the oracle's cache model: lengths,
    evicted chunks, dense rows bit-identical, packed records against the oracle's encode of the
    kept history."""
    D, bits, window, margin = 128, 3, 160, 16
    codec = kvq.Codec(D, bits, seed=77)
    n_caches = 2
    caches = [kvq.Cache(codec, packed_cap=4096, tail_cap=1200, window=window, margin=margin,
                        device=DEV) for _ in range(n_caches)]
    oc = oracle_codec_like(codec)
    models = [oracle.CacheModel(oc, window, margin) for _ in range(n_caches)]
    hist = [np.zeros((0, D), np.uint16) for _ in range(n_caches)]
    ops = [("a", 700), ("t", 5), ("a", 1), ("a", 1), ("t", 17), ("a", 129), ("a", 0),
           ("deep", 200), ("a", 300), ("t", 3), ("a", 1), ("a", 0), ("deep", 1), ("a", 450)]
    seed = 900
    for op, v in ops:
        if op == "a":
            rows = [_rows(max(v, 1), D, seed=seed + k) for k in range(n_caches)]
            seed += 10
            say(f"append t_new={v}")
            ev = kvq.append_evict_chunk(codec, caches, rows if v else None, v)
            for k in range(n_caches):
                host = bf16_host(rows[k][:v]) if v else np.zeros((0, D), np.uint16)
                hist[k] = np.concatenate([hist[k], host])
                assert ev[k] == models[k].append_evict(host)
        else:
            for k in range(n_caches):
                c = caches[k]
                new_len = len(c) - v if op == "t" else c.packed_len - v
                say(f"truncate cache {k} to {new_len} ({op}, packed {c.packed_len}, dense {c.tail_len})")
                c.truncate(new_len)
                models[k].truncate(new_len)
                hist[k] = hist[k][:new_len]
        torch.cuda.synchronize()
        for k in range(n_caches):
            c, mdl = caches[k], models[k]
            assert c.tail_len == len(mdl.tail) and c.packed_len == len(mdl.packed)
            assert len(c) == len(hist[k])
            if c.tail_len:
                np.testing.assert_array_equal(bf16_host(c.tail_rows()), np.stack(mdl.tail))
            if c.packed_len:
                got = c.packed[: c.packed_len].cpu().numpy()
                compare_codes(got, oracle.encode(oc, hist[k][: c.packed_len]), D, bits,
                              f"cache {k} after {op} {v}")
    with pytest.raises(kvq.KvqError) as e:
        caches[0].truncate(len(caches[0]) + 1)
    assert e.value.name == "KVQ_E_ARG"
