"""ctypes binding of libkvq.so. Argument marshalling only: PyTorch supplies device memory and
the current HIP stream; every step of the codec runs in the library's kernels.

Functions mirror include/kvq.h: encode, decode, score_packed, cache_init, append_evict_chunk.
The library must have been built (kv_cache_compression_vector_amd/build.py); importing a
missing library raises — there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq.so")

KVQ_OK = 0
STATUS_NAMES = {0: "KVQ_OK", 1: "KVQ_E_NULL", 2: "KVQ_E_DIM", 3: "KVQ_E_BITS",
                4: "KVQ_E_CENTROIDS", 5: "KVQ_E_STRIDE", 6: "KVQ_E_OUTLIER",
                7: "KVQ_E_CAPACITY", 8: "KVQ_E_CACHE", 9: "KVQ_E_DEVICE", 10: "KVQ_E_ARG"}
EVICT_CHUNK = 128


class KvqError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.name = STATUS_NAMES.get(status, str(status))


class _Codec(ctypes.Structure):
    _fields_ = [("head_dim", ctypes.c_uint32), ("bits", ctypes.c_uint32),
                ("proj_rank", ctypes.c_uint32), ("flags", ctypes.c_uint32),
                ("seed", ctypes.c_uint64), ("outlier_T", ctypes.c_float),
                ("reserved0", ctypes.c_uint32), ("centroids_host", ctypes.c_void_p),
                ("basis_dev", ctypes.c_void_p), ("mean_dev", ctypes.c_void_p),
                ("basis_count", ctypes.c_uint32), ("basis_block_rows", ctypes.c_uint32),
                ("basis_index_dev", ctypes.c_void_p), ("unbasis_dev", ctypes.c_void_p)]


class _Outliers(ctypes.Structure):
    _fields_ = [("offsets_dev", ctypes.c_void_p), ("idx_dev", ctypes.c_void_p),
                ("val_dev", ctypes.c_void_p), ("capacity", ctypes.c_int64),
                ("workspace_dev", ctypes.c_void_p), ("workspace_bytes", ctypes.c_int64)]


class _Cache(ctypes.Structure):
    _fields_ = [("magic", ctypes.c_uint64), ("codec_key", ctypes.c_uint64),
                ("packed_dev", ctypes.c_void_p), ("packed_len", ctypes.c_int64),
                ("packed_cap", ctypes.c_int64), ("tail_dev", ctypes.c_void_p),
                ("tail_head", ctypes.c_int64), ("tail_len", ctypes.c_int64),
                ("tail_cap", ctypes.c_int64), ("window", ctypes.c_int32),
                ("margin", ctypes.c_int32)]


_lib = None


def lib() -> ctypes.CDLL:
    """Load libkvq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python kv_cache_compression_vector_amd/build.py`")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
        PC = ctypes.POINTER(_Codec)
        L.kvq_record_bytes.argtypes = [PC]
        L.kvq_record_bytes.restype = ctypes.c_size_t
        L.kvq_encode_workspace_bytes.argtypes = [PC, I64]
        L.kvq_encode_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_codec_tables.argtypes = [PC, P, P, P]
        L.kvq_encode.argtypes = [PC, P, I64, I64, P, ctypes.POINTER(_Outliers),
                                 ctypes.POINTER(ctypes.c_int64), P]
        L.kvq_decode.argtypes = [PC, P, I64, ctypes.POINTER(_Outliers), P, ctypes.c_int, I64, P]
        L.kvq_score_packed.argtypes = [PC, P, I32, I32, I64, I64, P, I32, I64, I64, I64, P,
                                       I64, I64, P]
        L.kvq_cache_init.argtypes = [PC, ctypes.POINTER(_Cache), P, I64, P, I64, I32, I32]
        L.kvq_append_evict_chunk.argtypes = [PC, ctypes.POINTER(ctypes.POINTER(_Cache)), I32,
                                             ctypes.POINTER(ctypes.c_void_p), I64, P,
                                             ctypes.POINTER(ctypes.c_int64)]
        L.kvq_attend_workspace_bytes.argtypes = [PC, I32, I32, I64]
        L.kvq_attend_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_attend_packed.argtypes = [PC, PC, P, I32, I32, I64, I64, P, P, I32, I64, I64, I64,
                                        ctypes.c_float, ctypes.c_float, P, I64, I64, P,
                                        ctypes.c_size_t, P]
        L.kvq_attend_packed_static.argtypes = [PC, PC, P, I32, I32, I64, I64, P, P, I32, I64, I64,
                                               I64, ctypes.c_float, ctypes.c_float, P, I64, I64, P]
        L.kvq_stream_copy.argtypes = [P, P, I64, P]
        L.kvq_stream_read.argtypes = [P, I64, P, P]
        L.kvq_stream_fill.argtypes = [P, I64, ctypes.c_uint32, P]
        L.kvq_cache_truncate.argtypes = [PC, ctypes.POINTER(_Cache), I64]
        L.kvq_fit_workspace_bytes.argtypes = [PC, I64]
        L.kvq_fit_workspace_bytes.restype = ctypes.c_size_t
        L.kvq_fit_table.argtypes = [PC, P, I64, I64, I32, P, P, ctypes.c_size_t, P]
        L.kvq_last_error.restype = ctypes.c_char_p
        L.kvq_abi_version.restype = ctypes.c_int32
        for name in ("kvq_codec_tables", "kvq_encode", "kvq_decode", "kvq_score_packed",
                     "kvq_attend_packed", "kvq_cache_init", "kvq_append_evict_chunk",
                     "kvq_stream_copy", "kvq_attend_packed_static", "kvq_cache_truncate",
                     "kvq_fit_table", "kvq_stream_read", "kvq_stream_fill"):
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(status: int):
    if status != KVQ_OK:
        raise KvqError(status, lib().kvq_last_error().decode())


def _stream(t: torch.Tensor | None = None):
    dev = t.device if t is not None and t.is_cuda else None
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _ptr(t: torch.Tensor | None):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class Codec:
    """Codec descriptor. centroids: host f32 array (or None = Gaussian Lloyd-Max).
    PCA: basis device bf16 [D, r] or [k, D, r]; mean device f32 [D] or [k, D] (optional);
    with k > 1 bases, basis_index (device int32, one per block of basis_block_rows rows);
    unbasis: the decode basis (same shape as basis), or None = basis."""

    def __init__(self, head_dim: int, bits: int, seed: int = 42, proj_rank: int = 0,
                 outlier_T: float = 0.0, centroids=None, basis: torch.Tensor | None = None,
                 mean: torch.Tensor | None = None, flags: int = 0,
                 basis_index: torch.Tensor | None = None, basis_block_rows: int = 0,
                 unbasis: torch.Tensor | None = None):
        self.head_dim, self.bits, self.seed, self.flags = head_dim, bits, seed, flags
        self.proj_rank, self.outlier_T = proj_rank, float(outlier_T)
        self.m = proj_rank if proj_rank else head_dim
        self._centroids = None if centroids is None else np.ascontiguousarray(centroids, np.float32)
        self.basis, self.mean, self.basis_index, self.unbasis = basis, mean, basis_index, unbasis
        count = 0 if basis is None else (basis.shape[0] if basis.dim() == 3 else 1)
        if basis is not None:
            assert basis.dtype == torch.bfloat16 and basis.is_contiguous()
        if mean is not None:
            assert mean.dtype == torch.float32 and mean.is_contiguous()
        if basis_index is not None:
            assert basis_index.dtype == torch.int32 and basis_index.is_contiguous()
        if unbasis is not None:
            assert unbasis.dtype == torch.bfloat16 and unbasis.is_contiguous()
        self._c = _Codec(head_dim, bits, proj_rank, flags, seed, self.outlier_T, 0,
                         None if self._centroids is None else self._centroids.ctypes.data,
                         None if basis is None else basis.data_ptr(),
                         None if mean is None else mean.data_ptr(),
                         count, basis_block_rows,
                         None if basis_index is None else basis_index.data_ptr(),
                         None if unbasis is None else unbasis.data_ptr())

    @property
    def ref(self):
        return ctypes.byref(self._c)

    def record_bytes(self) -> int:
        n = lib().kvq_record_bytes(self.ref)
        if n == 0:  # invalid codec: report the typed status of its validation
            _check(lib().kvq_codec_tables(self.ref, None, None, None))
        return n

    def tables(self):
        L = 1 << self.bits
        c = np.zeros(L, np.float32)
        t = np.zeros(L - 1, np.float32)
        s = np.zeros(self.m, np.int8)
        _check(lib().kvq_codec_tables(self.ref, c.ctypes.data, t.ctypes.data, s.ctypes.data))
        return c, t, s


class Outliers:
    """Device CSR outlier list: offsets [n+1] u32, idx [cap] (u8 for coded length m <= 256, u16
    bits in an int16 tensor above), val [cap] bf16 bits."""

    def __init__(self, codec: Codec, n: int, capacity: int, device):
        self.offsets = torch.zeros(n + 1, dtype=torch.int32, device=device)
        self.idx = torch.zeros(max(capacity, 1), dtype=torch.uint8 if codec.m <= 256 else torch.int16,
                               device=device)
        self.val = torch.zeros(max(capacity, 1), dtype=torch.int16, device=device)
        self.capacity = capacity
        wsb = lib().kvq_encode_workspace_bytes(codec.ref, n)
        self.workspace = torch.empty(max(wsb, 16), dtype=torch.uint8, device=device)
        self._s = _Outliers(self.offsets.data_ptr(), self.idx.data_ptr(), self.val.data_ptr(),
                            capacity, self.workspace.data_ptr(), wsb)

    @property
    def ref(self):
        return ctypes.byref(self._s)


def encode(codec: Codec, x: torch.Tensor, records: torch.Tensor | None = None,
           outliers: Outliers | None = None, want_total: bool = False):
    """x: bf16 [n, >=D] (row stride multiple of 8). Returns records (uint8 [n, rec_bytes]) and,
    with want_total, the outlier total (synchronises)."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    n = x.shape[0]
    rb = codec.record_bytes()
    if records is None:
        records = torch.empty(n, rb, dtype=torch.uint8, device=x.device)
    total = ctypes.c_int64(-1)
    _check(lib().kvq_encode(codec.ref, _ptr(x), n, x.stride(0), _ptr(records),
                            outliers.ref if outliers is not None else None,
                            ctypes.byref(total) if want_total else None, _stream(x)))
    return (records, total.value) if want_total else records


def fit_table(codec: Codec, x: torch.Tensor, iters: int) -> np.ndarray:
    """Lloyd-Max table refitted to the codec's rotated, normalised coordinates of the rows x
    (bf16 [n, >=D]), `iters` passes from the codec's table. Returns f32 [2^bits] (host)."""
    assert x.dtype == torch.bfloat16 and x.dim() == 2 and x.stride(1) == 1
    n = x.shape[0]
    ws = torch.empty(max(int(lib().kvq_fit_workspace_bytes(codec.ref, n)), 16), dtype=torch.uint8,
                     device=x.device)
    out = np.zeros(1 << codec.bits, np.float32)
    _check(lib().kvq_fit_table(codec.ref, _ptr(x), n, x.stride(0), int(iters), out.ctypes.data,
                               _ptr(ws), ws.numel(), _stream(x)))
    return out


def decode(codec: Codec, records: torch.Tensor, n: int | None = None,
           outliers: Outliers | None = None, out: torch.Tensor | None = None,
           dtype=torch.float32) -> torch.Tensor:
    n = records.shape[0] if n is None else n
    if out is None:
        out = torch.empty(n, codec.head_dim, dtype=dtype, device=records.device)
    ydt = 1 if out.dtype == torch.bfloat16 else 0
    _check(lib().kvq_decode(codec.ref, _ptr(records), n,
                            outliers.ref if outliers is not None else None, _ptr(out), ydt,
                            out.stride(0), _stream(records)))
    return out


def score_packed(codec: Codec, q: torch.Tensor, records: torch.Tensor, Hkv: int, T: int,
                 rec_sb: int, rec_sh: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """q: bf16 [B, Hq, D] (last dim contiguous); records: record (b, kv, t) at index
    b*rec_sb + kv*rec_sh + t. Returns f32 scores [B, Hq, T]."""
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty(B, Hq, T, dtype=torch.float32, device=q.device)
    _check(lib().kvq_score_packed(codec.ref, _ptr(q), B, Hq, q.stride(0), q.stride(1),
                                  _ptr(records), Hkv, T, rec_sb, rec_sh, _ptr(out),
                                  out.stride(0), out.stride(1), _stream(q)))
    return out


def attend_workspace_bytes(vcodec: Codec, B: int, Hkv: int, T: int) -> int:
    return int(lib().kvq_attend_workspace_bytes(vcodec.ref, B, Hkv, T))


def attend_packed(kcodec: Codec, vcodec: Codec, q: torch.Tensor, krecords: torch.Tensor,
                  vrecords: torch.Tensor, Hkv: int, T: int, rec_sb: int, rec_sh: int,
                  softmax_scale: float, softcap: float = 0.0, out: torch.Tensor | None = None,
                  workspace: torch.Tensor | None = None) -> torch.Tensor:
    """q: bf16 [B, Hq, D] (last dim contiguous); K and V record (b, kv, t) at index
    b*rec_sb + kv*rec_sh + t of krecords / vrecords. Returns f32 [B, Hq, D]."""
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    need = attend_workspace_bytes(vcodec, B, Hkv, T)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check(lib().kvq_attend_packed(kcodec.ref, vcodec.ref, _ptr(q), B, Hq, q.stride(0),
                                   q.stride(1), _ptr(krecords), _ptr(vrecords), Hkv, T, rec_sb,
                                   rec_sh, softmax_scale, softcap, _ptr(out), out.stride(0),
                                   out.stride(1), _ptr(workspace), workspace.numel(), _stream(q)))
    return out


STATIC_SCRATCH_BYTES = 16 << 20


def attend_packed_static(kcodec: Codec, vcodec: Codec, q: torch.Tensor, krecords: torch.Tensor,
                         vrecords: torch.Tensor, Hkv: int, T: int, rec_sb: int, rec_sh: int,
                         softmax_scale: float, softcap: float = 0.0,
                         out: torch.Tensor | None = None) -> torch.Tensor:
    """attend_packed through the allocation-free entry point (partials in the library's static
    device scratch). Pass `out` to allocate nothing here either."""
    B, Hq, D = q.shape
    if out is None:
        out = torch.empty(B, Hq, D, dtype=torch.float32, device=q.device)
    _check(lib().kvq_attend_packed_static(kcodec.ref, vcodec.ref, _ptr(q), B, Hq, q.stride(0),
                                          q.stride(1), _ptr(krecords), _ptr(vrecords), Hkv, T,
                                          rec_sb, rec_sh, softmax_scale, softcap, _ptr(out),
                                          out.stride(0), out.stride(1), _stream(q)))
    return out


class Cache:
    """Two-region cache over caller (torch) buffers; lengths live on the host."""

    def __init__(self, codec: Codec, packed_cap: int, tail_cap: int, window: int,
                 margin: int = 16, device="cuda"):
        self.codec = codec
        self.packed = torch.zeros(max(packed_cap, 1), codec.record_bytes(), dtype=torch.uint8,
                                  device=device)
        self.tail = torch.zeros(tail_cap, codec.head_dim, dtype=torch.bfloat16, device=device)
        self._s = _Cache()
        _check(lib().kvq_cache_init(codec.ref, ctypes.byref(self._s), _ptr(self.packed),
                                    packed_cap, _ptr(self.tail), tail_cap, window, margin))

    @property
    def packed_len(self):
        return self._s.packed_len

    @property
    def tail_len(self):
        return self._s.tail_len

    @property
    def tail_head(self):
        return self._s.tail_head

    def __len__(self):
        return self._s.packed_len + self._s.tail_len

    def truncate(self, new_len: int) -> None:
        """Roll back to the first new_len tokens (host-side lengths only)."""
        _check(lib().kvq_cache_truncate(self.codec.ref, ctypes.byref(self._s), new_len))

    def tail_rows(self) -> torch.Tensor:
        """Dense rows in order, oldest first (a copy)."""
        cap, h, n = self.tail.shape[0], self._s.tail_head, self._s.tail_len
        idx = (torch.arange(n, device=self.tail.device) + h) % cap
        return self.tail[idx]


class CacheSet:
    """A fixed list of caches with its C pointer array built once, for repeated
    append_evict_chunk calls (a serving loop appends to the same caches every step)."""

    def __init__(self, caches: list[Cache]):
        self.caches = list(caches)
        n = len(self.caches)
        self.arr = (ctypes.POINTER(_Cache) * n)(*[ctypes.pointer(c._s) for c in self.caches])
        self.rows = (ctypes.c_void_p * n)()
        self.ev = (ctypes.c_int64 * n)()

    def __len__(self):
        return len(self.caches)


def append_evict_chunk(codec: Codec, caches, new_rows, t_new: int):
    """Append t_new rows to each cache and evict whole chunks (kvq_append_evict_chunk).

    caches: a list of Cache or a CacheSet. new_rows: None (t_new = 0), a list with one bf16
    tensor of >= t_new contiguous rows per cache, or one bf16 tensor [n_caches, >= t_new, D]
    whose rows are contiguous within each cache (any stride between caches). Returns the
    chunks evicted per cache."""
    cs = caches if isinstance(caches, CacheSet) else CacheSet(caches)
    n = len(cs)
    rows = None
    if t_new > 0:
        assert new_rows is not None
        if isinstance(new_rows, torch.Tensor):
            D = cs.caches[0].codec.head_dim if n else 0
            assert new_rows.dtype == torch.bfloat16 and new_rows.dim() == 3 and new_rows.shape[0] == n
            assert new_rows.shape[1] >= t_new and new_rows.shape[2] == D
            assert new_rows.stride(2) == 1 and new_rows.stride(1) == D
            base, step = new_rows.data_ptr(), new_rows.stride(0) * 2
            for i in range(n):
                cs.rows[i] = base + i * step
        else:
            assert len(new_rows) == n
            for i, r in enumerate(new_rows):
                assert r.dtype == torch.bfloat16 and r.is_contiguous() and r.shape[0] >= t_new
                cs.rows[i] = r.data_ptr()
        rows = cs.rows
    dev = cs.caches[0].tail if n else None
    _check(lib().kvq_append_evict_chunk(codec.ref, cs.arr, n, rows, t_new, _stream(dev), cs.ev))
    return list(cs.ev)


def stream_copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    """The library's streaming copy kernel (a bandwidth control): dst <- src, same byte size."""
    nb = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nb and src.is_contiguous() and dst.is_contiguous()
    _check(lib().kvq_stream_copy(_ptr(dst), _ptr(src), nb, _stream(src)))


def stream_read(src: torch.Tensor, sink: torch.Tensor) -> None:
    """The library's streaming read kernel (a bandwidth control): sink (one int32 on the same
    device) ^= the XOR of every 32-bit word of src."""
    assert src.is_contiguous() and sink.numel() >= 1 and sink.element_size() == 4
    _check(lib().kvq_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                 _stream(src)))


def stream_fill(dst: torch.Tensor, value: int) -> None:
    """The library's streaming fill kernel (a bandwidth control): every 32-bit word of dst <-
    value."""
    assert dst.is_contiguous()
    _check(lib().kvq_stream_fill(_ptr(dst), dst.numel() * dst.element_size(), value & 0xFFFFFFFF,
                                 _stream(dst)))
