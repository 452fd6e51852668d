"""Plain CPU reference ("oracle") of the KV-cache vector codec.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the smoke check and by the CPU-baseline leg of
the benchmark, never by the library. It shares no code with the GPU path; the C source
(kvq_oracle.c) is built here with gcc, single-threaded, -O2 without fast-math.

Functions follow the passages cited in kvq_oracle.c. The two-region cache model at the bottom
follows arc PR #98 ("What landed": dense tail bounded by window + max(t_q - 1, margin) +
EVICT_CHUNK; "Eviction is chunked, on purpose": EVICT_CHUNK = 128; "Mutation runs": margin 16).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvq_oracle.c")
_LIB = os.path.join(_HERE, "libkvq_oracle.so")

FLAG_NEAR_BOUNDARY = 1
FLAG_NEAR_T = 2
EVICT_CHUNK = 128


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no threads, no intrinsics)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.run(["gcc", "-O2", "-std=c11", "-D_GNU_SOURCE", "-fPIC", "-shared",
                        "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"],
                       check=True)
        os.replace(tmp, _LIB)
    return _LIB


class _RefCodec(ctypes.Structure):
    _fields_ = [("D", ctypes.c_int32), ("bits", ctypes.c_int32), ("r", ctypes.c_int32),
                ("scale_rule", ctypes.c_int32), ("seed", ctypes.c_uint64), ("T", ctypes.c_double),
                ("centroids", ctypes.c_void_p), ("basis", ctypes.c_void_p),
                ("mean", ctypes.c_void_p), ("unbasis", ctypes.c_void_p)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = ctypes.CDLL(build())
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        _lib.kvq_ref_lloyd_max_gaussian.argtypes = [ctypes.c_int, P, P]
        _lib.kvq_ref_lloyd_max_gaussian.restype = ctypes.c_int
        _lib.kvq_ref_thresholds.argtypes = [P, ctypes.c_int, P]
        _lib.kvq_ref_signs.argtypes = [ctypes.c_uint64, ctypes.c_int, P]
        _lib.kvq_ref_fwht_rows.argtypes = [P, I64, ctypes.c_int]
        _lib.kvq_ref_splitmix64.argtypes = [ctypes.c_uint64, ctypes.c_int, P]
        _lib.kvq_ref_record_bytes.argtypes = [ctypes.c_int, ctypes.c_int]
        _lib.kvq_ref_plane_position.argtypes = [ctypes.c_int, ctypes.c_int]
        _lib.kvq_ref_unpack_codes.argtypes = [ctypes.c_int, ctypes.c_int, P, P, P]
        _lib.kvq_ref_encode.argtypes = [ctypes.POINTER(_RefCodec), I64, P, I64, P, P, P, P, P,
                                        P, P, P, I64]
        _lib.kvq_ref_encode.restype = I64
        _lib.kvq_ref_decode.argtypes = [ctypes.POINTER(_RefCodec), I64, P, P, P, P, I64, P]
        _lib.kvq_ref_score.argtypes = [ctypes.POINTER(_RefCodec), I64, P, P, P]
        _lib.kvq_ref_lloyd_fit.argtypes = [P, I64, ctypes.c_int, ctypes.c_int, P]
        _lib.kvq_ref_table_mse.argtypes = [P, I64, ctypes.c_int, P]
        _lib.kvq_ref_table_mse.restype = ctypes.c_double
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


# --------------------------------------------------------------------------------------------
# Tables and signs

_TABLES: dict[int, tuple[np.ndarray, np.ndarray]] = {}


def gaussian_table(bits: int) -> tuple[np.ndarray, np.ndarray]:
    """(f64 centroids, f32 centroids) of the N(0,1) Lloyd-Max quantiser with 2^bits cells."""
    if bits not in _TABLES:
        L = 1 << bits
        c64 = np.zeros(L, np.float64)
        c32 = np.zeros(L, np.float32)
        it = lib().kvq_ref_lloyd_max_gaussian(bits, _p(c64), _p(c32))
        if it < 0:
            raise RuntimeError(f"Lloyd-Max iteration failed for bits={bits}")
        _TABLES[bits] = (c64, c32)
    c64, c32 = _TABLES[bits]
    return c64.copy(), c32.copy()


def thresholds(c32: np.ndarray) -> np.ndarray:
    c32 = np.ascontiguousarray(c32, np.float32)
    t = np.zeros(len(c32) - 1, np.float32)
    lib().kvq_ref_thresholds(_p(c32), len(c32), _p(t))
    return t


def signs(seed: int, m: int) -> np.ndarray:
    s = np.zeros(m, np.int8)
    lib().kvq_ref_signs(seed, m, _p(s))
    return s


def splitmix64(seed: int, n: int) -> np.ndarray:
    out = np.zeros(n, np.uint64)
    lib().kvq_ref_splitmix64(seed, n, _p(out))
    return out


def fwht_rows(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a, np.float64).copy()
    n, m = a.reshape(-1, a.shape[-1]).shape
    lib().kvq_ref_fwht_rows(_p(a), n, m)
    return a


def record_bytes(m: int, bits: int) -> int:
    return lib().kvq_ref_record_bytes(m, bits)


def plane_position(i: int, m: int) -> int:
    return lib().kvq_ref_plane_position(i, m)


def unpack_codes(m: int, bits: int, rec: np.ndarray) -> tuple[np.ndarray, float]:
    rec = np.ascontiguousarray(rec, np.uint8)
    codes = np.zeros(m, np.uint8)
    nrm = np.zeros(1, np.float32)
    lib().kvq_ref_unpack_codes(m, bits, _p(rec), _p(codes), _p(nrm))
    return codes, float(nrm[0])


# --------------------------------------------------------------------------------------------
# Codec


class Codec:
    """Parameters of one codec as the oracle sees them (host arrays only)."""

    def __init__(self, D: int, bits: int, seed: int, r: int = 0, T: float = 0.0,
                 centroids: np.ndarray | None = None, basis_bf16: np.ndarray | None = None,
                 mean: np.ndarray | None = None, scale_rule: int = 0,
                 unbasis_bf16: np.ndarray | None = None):
        """scale_rule: the f32 scale a record stores: 0 the norm ||v||; 1 matched norm
        (||x^|| = ||v||); 2 inner-product preserving (<x^, v> = ||v||^2); 3 least-squares
        optimal (<v - x^, x^> = 0).

        unbasis_bf16: projection codecs only, the decode basis C ([D][r] bf16 bits): decode
        returns mu + C v^ instead of mu + B v^ (score and attention follow decode). With
        Sigma_q = L L^T, Q-preconditioning is basis = L B_w, unbasis = L^-T B_w, mean = L^-T mu_w
        [kakeyaturbo PR #15: K_tilde = K @ L before the codec, the inverse factor after it]."""
        self.D, self.bits, self.seed, self.r, self.T = D, bits, seed, r, float(T)
        self.scale_rule = int(scale_rule)
        self.m = r if r > 0 else D
        if centroids is None:
            centroids = gaussian_table(bits)[1]
        self.centroids = np.ascontiguousarray(centroids, np.float32)
        self.basis = None if basis_bf16 is None else np.ascontiguousarray(basis_bf16, np.uint16)
        self.mean = None if mean is None else np.ascontiguousarray(mean, np.float32)
        if r > 0 and (self.basis is None or self.basis.shape != (D, r)):
            raise ValueError("PCA codec needs a bf16 basis of shape [D][r]")
        self.unbasis = None if unbasis_bf16 is None else np.ascontiguousarray(unbasis_bf16, np.uint16)
        if self.unbasis is not None and (r == 0 or self.unbasis.shape != (D, r)):
            raise ValueError("a decode basis needs a projection codec and shape [D][r]")
        self.rec_bytes = record_bytes(self.m, bits)

    def _c(self) -> _RefCodec:
        return _RefCodec(self.D, self.bits, self.r, self.scale_rule, self.seed, self.T,
                         _p(self.centroids), _p(self.basis), _p(self.mean), _p(self.unbasis))


def encode(cd: Codec, x_bf16: np.ndarray, ol_cap: int | None = None) -> dict:
    """Encode rows of x (uint16 bf16 bits, shape [n, D]). Returns a dict with records
    ([n, rec_bytes] u8), codes and flags ([n, m] u8), z ([n, m] f64), norms ([n] f64), the f32
    decision thresholds and, when T > 0, the outlier CSR (offsets [n+1] u32, idx u8 for
    m <= 256 and u16 above, val u16 bf16 bits, total)."""
    x = np.ascontiguousarray(x_bf16, np.uint16).reshape(-1, cd.D)
    n = x.shape[0]
    rec = np.zeros((n, cd.rec_bytes), np.uint8)
    codes = np.zeros((n, cd.m), np.uint8)
    flags = np.zeros((n, cd.m), np.uint8)
    z = np.zeros((n, cd.m), np.float64)
    norms = np.zeros(n, np.float64)
    out = dict(records=rec, codes=codes, flags=flags, z=z, norms=norms,
               thresholds=thresholds(cd.centroids))
    c = cd._c()
    if cd.T > 0:
        cap = n * cd.m if ol_cap is None else ol_cap
        off = np.zeros(n + 1, np.uint32)
        idx = np.zeros(max(cap, 1), np.uint16)
        val = np.zeros(max(cap, 1), np.uint16)
        total = lib().kvq_ref_encode(ctypes.byref(c), n, _p(x), cd.D, _p(rec), _p(codes),
                                     _p(flags), _p(z), _p(norms), _p(off), _p(idx), _p(val), cap)
        idx = idx[:min(total, cap)]
        out.update(offsets=off, idx=idx.astype(np.uint8) if cd.m <= 256 else idx,
                   val=val[:min(total, cap)], total=int(total))
    else:
        lib().kvq_ref_encode(ctypes.byref(c), n, _p(x), cd.D, _p(rec), _p(codes), _p(flags),
                             _p(z), _p(norms), None, None, None, 0)
    return out


def encode_records(cd: Codec, x_bf16: np.ndarray) -> np.ndarray:
    """Records only (no per-coordinate outputs): the form the CPU baseline times."""
    x = np.ascontiguousarray(x_bf16, np.uint16).reshape(-1, cd.D)
    n = x.shape[0]
    rec = np.zeros((n, cd.rec_bytes), np.uint8)
    c = cd._c()
    lib().kvq_ref_encode(ctypes.byref(c), n, _p(x), cd.D, _p(rec), None, None, None, None,
                         None, None, None, 0)
    return rec


def decode(cd: Codec, records: np.ndarray, offsets=None, idx=None, val=None) -> np.ndarray:
    """Decode records ([n, rec_bytes] u8) to f64 [n, D]."""
    rec = np.ascontiguousarray(records, np.uint8).reshape(-1, cd.rec_bytes)
    n = rec.shape[0]
    y = np.zeros((n, cd.D), np.float64)
    c = cd._c()
    if offsets is not None:
        off = np.ascontiguousarray(offsets, np.uint32)
        ix = np.ascontiguousarray(np.asarray(idx).astype(np.uint16))
        vv = np.ascontiguousarray(val, np.uint16)
        lib().kvq_ref_decode(ctypes.byref(c), n, _p(rec), _p(off), _p(ix), _p(vv), len(ix), _p(y))
    else:
        lib().kvq_ref_decode(ctypes.byref(c), n, _p(rec), None, None, None, 0, _p(y))
    return y


def score(cd: Codec, q_bf16: np.ndarray, records: np.ndarray) -> np.ndarray:
    """q . decode(record) for paired rows: q [n, D] bf16 bits, records [n, rec_bytes]."""
    q = np.ascontiguousarray(q_bf16, np.uint16).reshape(-1, cd.D)
    rec = np.ascontiguousarray(records, np.uint8).reshape(-1, cd.rec_bytes)
    assert q.shape[0] == rec.shape[0]
    out = np.zeros(q.shape[0], np.float64)
    lib().kvq_ref_score(ctypes.byref(cd._c()), q.shape[0], _p(q), _p(rec), _p(out))
    return out


def attend(kc: Codec, vc: Codec, q_bf16: np.ndarray, krecs: np.ndarray, vrecs: np.ndarray,
           softmax_scale: float, softcap: float = 0.0) -> np.ndarray:
    """Decode attention of the query heads of one KV head over packed K and V records:
    q [G, D] bf16 bits, krecs [T, kc.rec_bytes], vrecs [T, vc.rec_bytes] -> f64 [G, D].

    Logits l_t = softmax_scale * (q . k^_t); with softcap > 0 they become softcap * tanh(l / softcap),
    after the scale multiply and before the maximum [arc PR #98, "Also: two silently-ignored
    kernel parameters"]; weights w = softmax over t; output sum_t w_t v^_t with k^, v^ the
    decoded records [arc PR #98 / #94 kernel commit: attention reads the packed cache]."""
    K = decode(kc, krecs)                                    # [T, D]
    V = decode(vc, vrecs)                                    # [T, D]
    q = (np.ascontiguousarray(q_bf16, np.uint16).reshape(-1, kc.D).astype(np.uint32) << 16)
    q = q.view(np.float32).astype(np.float64)                # [G, D]
    logits = softmax_scale * (q @ K.T)                       # [G, T]
    if softcap > 0:
        logits = softcap * np.tanh(logits / softcap)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return w @ V


def lloyd_fit(z: np.ndarray, centroids: np.ndarray, iters: int) -> np.ndarray:
    """Lloyd iterations of an f32 table on samples z (f64), from `centroids` (ascending): cells
    by the table's f32 thresholds, centroids replaced by their cells' f64 means rounded to f32.
    Returns the f32 table. [kakeyaturbo PR #15, calibration-artefacts commit]"""
    z = np.ascontiguousarray(z, np.float64).reshape(-1)
    c = np.ascontiguousarray(centroids, np.float32).copy()
    lib().kvq_ref_lloyd_fit(_p(z), z.size, c.size, int(iters), _p(c))
    return c


def table_mse(z: np.ndarray, centroids: np.ndarray) -> float:
    """Mean squared error of samples z under an f32 table (cells by its f32 thresholds)."""
    z = np.ascontiguousarray(z, np.float64).reshape(-1)
    c = np.ascontiguousarray(centroids, np.float32)
    return float(lib().kvq_ref_table_mse(_p(z), z.size, c.size, _p(c)))


def fit_table(cd: Codec, x_bf16: np.ndarray, iters: int) -> np.ndarray:
    """A codec's table refitted to its own rotated, normalised coordinates z of the rows x
    (the samples a calibration pass sees), starting from the codec's table."""
    z = encode(cd, x_bf16)["z"]
    return lloyd_fit(z, cd.centroids, iters)


# --------------------------------------------------------------------------------------------
# Two-region cache model [arc PR #98]: a dense tail (list of bf16 rows) and a packed region.


def retention_floor(window: int, t_new: int, margin: int) -> int:
    """Rows the dense tail must keep after appending t_new rows: the raw span the next t_new
    queries can reach (t_new + window - 1), never less than window + margin."""
    return window + max(t_new - 1, margin)


class CacheModel:
    def __init__(self, cd: Codec, window: int, margin: int = 16):
        self.cd, self.window, self.margin = cd, window, margin
        self.tail: list[np.ndarray] = []       # oldest first, each [D] uint16
        self.packed: list[np.ndarray] = []     # records, oldest first

    def __len__(self) -> int:
        """Length in tokens: packed records plus dense rows [arc PR #98, "What landed"]."""
        return len(self.packed) + len(self.tail)

    def truncate(self, new_len: int) -> None:
        """Roll the cache back to its first new_len tokens. Truncation maps onto both regions
        [arc PR #98, "What landed": the cache reports its length in tokens and maps truncation
        onto both time bases]: a length inside the dense tail drops its newest rows; a length
        inside the packed region drops the records past it and empties the tail (the tokens
        between are gone from both regions; a caller that needs them dense again decodes
        records, the dequantizing path a deep rollback can ask for)."""
        if not 0 <= new_len <= len(self):
            raise ValueError(f"new_len={new_len} outside [0, {len(self)}]")
        if new_len >= len(self.packed):
            del self.tail[new_len - len(self.packed):]
        else:
            del self.packed[new_len:]
            self.tail = []

    def append_evict(self, rows_bf16: np.ndarray) -> int:
        rows = np.ascontiguousarray(rows_bf16, np.uint16).reshape(-1, self.cd.D)
        t_new = rows.shape[0]
        self.tail.extend(list(rows))
        floor = retention_floor(self.window, t_new, self.margin)
        chunks = 0
        while len(self.tail) >= floor + EVICT_CHUNK:
            block = np.stack(self.tail[:EVICT_CHUNK])
            self.packed.extend(list(encode_records(self.cd, block)))
            del self.tail[:EVICT_CHUNK]
            chunks += 1
        return chunks
