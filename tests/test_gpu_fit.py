"""GPU parity of the Lloyd-Max refit (kvq_fit_table) against the oracle's refit of the same rows:
the same number of passes from the same table, cells decided by the f32 thresholds, centroids the
cells' means rounded to f32. The GPU forms z = u/n in f32 and sums it per block in f32; the bar
is 2e-5 absolute on centroids of order 1."""
import numpy as np
import pytest
import torch

import oracle
from kv_cache_compression_vector_amd import kvq, synth
from tests.gpu_helpers import (bf16_host, compare_codes, compare_decoded, oracle_codec_like, say,
                               unpack_records)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
FIT_ATOL = 2e-5


@pytest.mark.parametrize("D,bits,n,iters", [(128, 2, 20000, 8), (128, 3, 20000, 8), (64, 1, 5000, 5),
                                            (256, 3, 7000, 5), (512, 4, 3000, 4)])
def test_fit_matches_the_oracle_on_gaussian_rows(D, bits, n, iters):
    x = synth.iid_normal((n, D), seed=D + bits, device=DEV)
    x[5] = 0  # a zero row: all its coordinates are z = 0
    codec = kvq.Codec(D, bits, seed=42)
    say(f"fit D={D} b={bits} n={n} iters={iters}")
    got = kvq.fit_table(codec, x, iters)
    ref = oracle.fit_table(oracle_codec_like(codec), bf16_host(x), iters)
    np.testing.assert_allclose(got, ref, rtol=0, atol=FIT_ATOL)
    assert np.all(np.diff(got) > 0)


def test_fit_on_heavy_tailed_rows_lowers_the_error():
    """Student-t(3) rows with 3 channels of 128 scaled x16 (the heavy-tailed V workload, 1 layer x
    8 heads x 4096 tokens): the refit equals the oracle's, the codec with the refitted table codes
    the rows as the oracle does, and its decode error is below the Gaussian table's."""
    D, bits, iters = 128, 2, 10
    X = synth.student_t_heavy(layers=1, heads=8, tokens=4096, device=DEV)
    x = X.reshape(-1, D)
    codec = kvq.Codec(D, bits, seed=43)
    say(f"heavy-tailed fit n={x.shape[0]}")
    got = kvq.fit_table(codec, x, iters)
    oc = oracle_codec_like(codec)
    ref = oracle.fit_table(oc, bf16_host(x), iters)
    np.testing.assert_allclose(got, ref, rtol=0, atol=FIT_ATOL)
    fitted = kvq.Codec(D, bits, seed=43, centroids=got)
    rec = kvq.encode(fitted, x)
    torch.cuda.synchronize()
    recn = rec.cpu().numpy()
    ofit = oracle_codec_like(fitted)
    rows = np.arange(0, x.shape[0], 7)
    compare_codes(recn[rows], oracle.encode(ofit, bf16_host(x[torch.from_numpy(rows).to(DEV)])), D,
                  bits, "refitted codes")
    y = kvq.decode(fitted, rec)
    y0 = kvq.decode(codec, kvq.encode(codec, x))
    yref = oracle.decode(ofit, recn[rows])
    compare_decoded(y.cpu().numpy()[rows], yref, unpack_records(recn[rows], D, bits)[1], "refitted decode")
    xf = x.float()
    e_fit = ((xf - y) ** 2).sum().item() / (xf ** 2).sum().item()
    e_gauss = ((xf - y0) ** 2).sum().item() / (xf ** 2).sum().item()
    say(f"  relative squared error: refitted {e_fit:.5f}, Gaussian {e_gauss:.5f}")
    assert e_fit < e_gauss


def test_fit_refusals():
    x = synth.iid_normal((100, 128), seed=1, device=DEV)
    with pytest.raises(kvq.KvqError) as e:
        kvq.fit_table(kvq.Codec(128, 3, seed=1), x[:0], 3)
    assert e.value.name == "KVQ_E_ARG"
    basis = torch.zeros(128, 64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(kvq.KvqError) as e:
        kvq.fit_table(kvq.Codec(128, 3, seed=1, proj_rank=64, basis=basis), x, 3)
    assert e.value.name == "KVQ_E_ARG"
