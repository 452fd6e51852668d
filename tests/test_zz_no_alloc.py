"""The allocation-free decode attention entry point (kvq_attend_packed_static) against
kvq_attend_packed with a caller workspace, through the C ABI: two calls in a row, the second
with a smaller input, must give the same outputs; a size whose partials exceed the static
scratch is refused before any launch."""
import numpy as np
import pytest
import torch

from kv_cache_compression_vector_amd import kvq, synth
from tests.gpu_helpers import say

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _case(B, Hkv, G, T, D, seed, kbits=3, vbits=2):
    kc, vc = kvq.Codec(D, kbits, seed=42), kvq.Codec(D, vbits, seed=43)
    n = B * Hkv * T
    K = synth.iid_normal((n, D), seed=seed, device=DEV)
    V = synth.iid_normal((n, D), seed=seed + 1, device=DEV)
    kr, vr = kvq.encode(kc, K), kvq.encode(vc, V)
    q = synth.iid_normal((B, Hkv * G, D), seed=seed + 2, device=DEV)
    return kc, vc, q, kr, vr


def test_static_attention_matches_workspace_attention_twice():
    # first a larger call, then a smaller one: the second must not see the first's partials
    for B, Hkv, G, T, D, cap in ((4, 8, 4, 5000, 128, 30.0), (2, 2, 6, 700, 64, 0.0)):
        kc, vc, q, kr, vr = _case(B, Hkv, G, T, D, seed=B * 100 + T)
        say(f"static attention B={B} Hkv={Hkv} G={G} T={T} D={D}")
        ref = kvq.attend_packed(kc, vc, q, kr, vr, Hkv, T, rec_sb=Hkv * T, rec_sh=T,
                                softmax_scale=D ** -0.5, softcap=cap)
        out = torch.full_like(ref, float("nan"))
        kvq.attend_packed_static(kc, vc, q, kr, vr, Hkv, T, rec_sb=Hkv * T, rec_sh=T,
                                 softmax_scale=D ** -0.5, softcap=cap, out=out)
        torch.cuda.synchronize()
        assert torch.isfinite(out).all()
        assert torch.equal(out, ref), f"max diff {(out - ref).abs().max().item():.3g}"


def test_static_attention_refuses_what_the_scratch_cannot_hold():
    D = 128
    kc, vc = kvq.Codec(D, 3, seed=42), kvq.Codec(D, 2, seed=43)
    B, Hkv, T = 1000, 1, 256   # 1000 (batch, KV head) pairs of partials > 16 MiB
    need = kvq.attend_workspace_bytes(vc, B, Hkv, T)
    assert need > kvq.STATIC_SCRATCH_BYTES
    q = torch.zeros(B, 4, D, dtype=torch.bfloat16, device=DEV)
    rec = torch.zeros(16, dtype=torch.uint8, device=DEV)
    out = torch.zeros(B, 4, D, dtype=torch.float32, device=DEV)
    with pytest.raises(kvq.KvqError) as e:
        kvq.attend_packed_static(kc, vc, q, rec, rec, Hkv, T, rec_sb=T, rec_sh=T,
                                 softmax_scale=0.1, out=out)
    assert e.value.name == "KVQ_E_CAPACITY"
    assert torch.all(out == 0)
