"""MI355X (gfx950) KV-cache vector codec: Python binding over the C-ABI library libkvq.so.

The binding only marshals arguments; all codec arithmetic runs in the library's HIP kernels.
Seeded synthetic inputs live in `synth` (no codec arithmetic there).
"""
from .kvq import (EVICT_CHUNK, Cache, Codec, KvqError, Outliers, append_evict_chunk, decode,
                  encode, lib, score_packed)

__all__ = ["EVICT_CHUNK", "Cache", "Codec", "KvqError", "Outliers", "append_evict_chunk",
           "decode", "encode", "lib", "score_packed"]
