"""ctypes wrapper of the float64 CPU oracle (``skv_oracle.c``).

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package. The GPU library never loads it and it shares no code with
the GPU path. Inputs are host numpy arrays holding the exact bytes of the cache (bf16 as uint16
bit patterns). Every function is a thin marshalling layer over the C oracle; the arithmetic
lives in ``skv_oracle.c`` and each C function cites the passage it follows.

Functions with no pin of their own against the pages or mathematics: none. Approximation quality
of the Gaussian threshold against the exact entmax threshold is reported, not pinned (it is
not a property the pages fix).
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "skv_oracle.c")
# SKV_ORACLE_LIB names another build of the same source (the mutation test points it at copies of
# the oracle with planted mistakes)
_LIB = os.environ.get("SKV_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1


GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra"]


def compile_source(src: str, out: str, extra=()) -> str:
    """Compile an oracle source file into a shared library (no fast-math, no FMA contraction)."""
    tmp = out + ".tmp"
    subprocess.check_call(["gcc", *GCC_FLAGS, *extra, "-o", tmp, src, "-lm"])
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile ``skv_oracle.c`` into ``liboracle.so`` with gcc."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _lib = C.CDLL(_LIB)
        _declare(_lib)
    return _lib


class _Cache(C.Structure):
    _fields_ = [("B", C.c_int32), ("Hq", C.c_int32), ("Hkv", C.c_int32), ("d", C.c_int32),
                ("S", C.c_int32), ("maxP", C.c_int32), ("Nphys", C.c_int32), ("dtype", C.c_int32),
                ("k", C.c_void_p), ("v", C.c_void_p), ("q", C.c_void_p),
                ("block_table", C.c_void_p), ("seq_lens", C.c_void_p)]


_P = C.c_void_p
_I = C.c_int32
_D = C.c_double


def _declare(L):
    sig = {
        "orc_round_bf16": (C.c_uint16, [_D]),
        "orc_meta_box": (None, [_P, _P, _P]),
        "orc_meta_gauss": (None, [_P, _P, _P]),
        "orc_meta_proj": (None, [_P, _I, _P, _P]),
        "orc_meta_pool": (None, [_P, _I, _P]),
        "orc_score_pool": (None, [_P, _I, _P, _P]),
        "orc_meta_lsh": (None, [_P, _I, _I, _P, _P, _P]),
        "orc_lsh_tables": (None, [_P, _I, _I, _P, _D, _P]),
        "orc_score_lsh": (None, [_P, _I, _I, _P, _P, _P, _P]),
        "orc_score_box": (None, [_P, _P, _P, _P]),
        "orc_score_gauss": (None, [_P, _P, _P, _D, _I, _P, _P, _P]),
        "orc_Phi_inv": (_D, [_D]),
        "orc_Phi_inv_upper": (_D, [_D]),
        "orc_score_proj": (None, [_P, _I, _P, _P, _P]),
        "orc_select_topk": (_I, [_P, _I, _I, _P]),
        "orc_budget_k": (_I, [_I, _I]),
        "orc_gauss_partial_moment": (_D, [_D, _D, _D, _D]),
        "orc_gauss_partial_moment_quad": (_D, [_D, _D, _D, _D]),
        "orc_trunc_power_moment": (_D, [_D, _D]),
        "orc_tau_hat": (_D, [_P, _P, _P, _I, _D]),
        "orc_select_thresh": (_I, [_P, _P, _I, _I, _D, _D, _P]),
        "orc_select_thresh_box": (_I, [_P, _P, _I, _I, _D, _D, _D, _P]),
        "orc_softmax": (None, [_P, _I, _P]),
        "orc_sparsemax": (_D, [_P, _I, _P]),
        "orc_entmax15": (_D, [_P, _I, _P]),
        "orc_entmax_bisect": (_D, [_P, _I, _D, _P]),
        "orc_entmax": (_D, [_P, _I, _D, _P]),
        "orc_attend_head": (C.c_int64, [_P, _I, _I, _P, _I, _I, _D, _D, _P, _P, _P]),
        "orc_attend_full_head": (C.c_int64, [_P, _I, _I, _D, _D, _P, _P]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args


def _ptr(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(C.c_void_p)


@dataclass
class Cache:
    """Host copy of a paged GQA cache. k, v: [Nphys, Hkv, S, d]; q: [B, Hq, d]; float32 arrays, or
    uint16 arrays holding bf16 bit patterns. block_table [B, maxP] int32, seq_lens [B] int32."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    block_table: np.ndarray
    seq_lens: np.ndarray

    def __post_init__(self):
        for name in ("q", "k", "v"):
            a = np.ascontiguousarray(getattr(self, name))
            assert a.dtype in (np.float32, np.uint16), f"{name}: float32 or uint16 (bf16 bits)"
            setattr(self, name, a)
        assert self.q.dtype == self.k.dtype == self.v.dtype
        self.block_table = np.ascontiguousarray(self.block_table, dtype=np.int32)
        self.seq_lens = np.ascontiguousarray(self.seq_lens, dtype=np.int32)
        self.Nphys, self.Hkv, self.S, self.d = self.k.shape
        self.B, self.Hq, _ = self.q.shape
        self.maxP = self.block_table.shape[1]
        self.G = self.Hq // self.Hkv
        self.dtype = F32 if self.k.dtype == np.float32 else BF16
        self._c = _Cache(self.B, self.Hq, self.Hkv, self.d, self.S, self.maxP, self.Nphys, self.dtype,
                         self.k.ctypes.data, self.v.ctypes.data, self.q.ctypes.data,
                         self.block_table.ctypes.data, self.seq_lens.ctypes.data)

    @property
    def ref(self):
        return C.byref(self._c)

    def length(self, b: int) -> int:
        return int(min(max(int(self.seq_lens[b]), 0), self.maxP * self.S))

    def pages(self, b: int) -> int:
        return (self.length(b) + self.S - 1) // self.S

    def page_tokens(self, b: int, p: int) -> int:
        return min(self.S, self.length(b) - p * self.S)


def round_bf16(x: float) -> int:
    return int(lib().orc_round_bf16(float(x)))


def meta_box(c: Cache):
    kmin = np.full((c.Nphys, c.Hkv, c.d), np.nan)
    kmax = np.full((c.Nphys, c.Hkv, c.d), np.nan)
    lib().orc_meta_box(c.ref, _ptr(kmin), _ptr(kmax))
    return kmin, kmax


def meta_gauss(c: Cache):
    mean = np.full((c.Nphys, c.Hkv, c.d), np.nan)
    var = np.full((c.Nphys, c.Hkv, c.d), np.nan)
    lib().orc_meta_gauss(c.ref, _ptr(mean), _ptr(var))
    return mean, var


def meta_proj(c: Cache, P: np.ndarray):
    P = np.ascontiguousarray(P, dtype=np.float32)
    r = P.shape[0]
    kproj = np.zeros((c.Nphys, c.Hkv, c.S, r), dtype=np.uint16)
    lib().orc_meta_proj(c.ref, r, _ptr(P), _ptr(kproj))
    return kproj


def meta_pool(c: Cache, pb: int):
    """Sub-block mean keys [Nphys, Hkv, S / pb, d] float32 (NaN where not written)."""
    pool = np.full((c.Nphys, c.Hkv, c.S // pb, c.d), np.nan, dtype=np.float32)
    lib().orc_meta_pool(c.ref, int(pb), _ptr(pool))
    return pool


def score_pool(c: Cache, pb: int, pool: np.ndarray):
    key = np.empty((c.B, c.Hkv, c.maxP), dtype=np.float32)
    lib().orc_score_pool(c.ref, int(pb), _ptr(pool), _ptr(key))
    return key


def meta_lsh(c: Cache, planes: np.ndarray):
    """Soft-LSH metadata for hyperplanes planes [L, P, d]: bucket ids [Nphys, Hkv, S, L] uint8 and
    value norms [Nphys, Hkv, S] float32 (NaN / 255 where not written)."""
    planes = np.ascontiguousarray(planes, dtype=np.float32)
    L, P, _ = planes.shape
    bucket = np.full((c.Nphys, c.Hkv, c.S, L), 255, dtype=np.uint8)
    vnorm = np.full((c.Nphys, c.Hkv, c.S), np.nan, dtype=np.float32)
    lib().orc_meta_lsh(c.ref, int(L), int(P), _ptr(planes), _ptr(bucket), _ptr(vnorm))
    return bucket, vnorm


def lsh_tables(c: Cache, planes: np.ndarray, tau: float):
    """Fixed-point bucket masses [B, Hq, L, 2^P] uint32 (2^24 = probability 1). tau is rounded to
    float32 first, the precision in which the C ABI takes it."""
    planes = np.ascontiguousarray(planes, dtype=np.float32)
    L, P, _ = planes.shape
    tab = np.empty((c.B, c.Hq, L, 1 << P), dtype=np.uint32)
    lib().orc_lsh_tables(c.ref, int(L), int(P), _ptr(planes), float(np.float32(tau)), _ptr(tab))
    return tab


def score_lsh(c: Cache, bucket: np.ndarray, vnorm: np.ndarray, tab: np.ndarray):
    """Soft-collision token keys [B, Hkv, maxP * S] float32."""
    L, nb = tab.shape[2], tab.shape[3]
    key = np.empty((c.B, c.Hkv, c.maxP * c.S), dtype=np.float32)
    lib().orc_score_lsh(c.ref, int(L), int(nb).bit_length() - 1, _ptr(bucket), _ptr(vnorm),
                        _ptr(np.ascontiguousarray(tab, dtype=np.uint32)), _ptr(key))
    return key


def score_box(c: Cache, kmin, kmax):
    key = np.empty((c.B, c.Hkv, c.maxP), dtype=np.float32)
    lib().orc_score_box(c.ref, _ptr(kmin), _ptr(kmax), _ptr(key))
    return key


def score_gauss(c: Cache, mean, var, scale: float, quantile: bool = False):
    """quantile: estimated maximum m + s Phi^-1(1 - 1/n) instead of m + s sqrt(2 ln n)."""
    shape = (c.B, c.Hq, c.maxP)
    m, s, shat = np.empty(shape), np.empty(shape), np.empty(shape)
    lib().orc_score_gauss(c.ref, _ptr(mean), _ptr(var), float(scale), int(bool(quantile)), _ptr(m), _ptr(s),
                          _ptr(shat))
    return m, s, shat


def Phi_inv(p: float) -> float:
    return float(lib().orc_Phi_inv(float(p)))


def Phi_inv_upper(q: float) -> float:
    """Phi^-1(1 - q)."""
    return float(lib().orc_Phi_inv_upper(float(q)))


def score_proj(c: Cache, P: np.ndarray, kproj: np.ndarray):
    P = np.ascontiguousarray(P, dtype=np.float32)
    key = np.empty((c.B, c.Hkv, c.maxP * c.S), dtype=np.float32)
    lib().orc_score_proj(c.ref, P.shape[0], _ptr(P), _ptr(kproj), _ptr(key))
    return key


def select_topk(key: np.ndarray, k: int) -> np.ndarray:
    key = np.ascontiguousarray(key, dtype=np.float32)
    out = np.empty(max(min(k, key.size), 1), dtype=np.int32)
    n = lib().orc_select_topk(_ptr(key), key.size, int(k), _ptr(out))
    return out[:n].copy()


def budget_k(P_b: int, pct: int) -> int:
    return int(lib().orc_budget_k(int(P_b), int(pct)))


def gauss_partial_moment(mu: float, sd: float, tau: float, alpha: float) -> float:
    return float(lib().orc_gauss_partial_moment(mu, sd, tau, alpha))


def gauss_partial_moment_quad(mu: float, sd: float, tau: float, alpha: float) -> float:
    """The same expectation by quadrature for every alpha (the closed forms bypassed)."""
    return float(lib().orc_gauss_partial_moment_quad(mu, sd, tau, alpha))


def trunc_power_moment(a: float, k: float) -> float:
    """E[(Z + a)_+^k], Z ~ N(0, 1)."""
    return float(lib().orc_trunc_power_moment(float(a), float(k)))


def tau_hat(m: np.ndarray, s: np.ndarray, n: np.ndarray, alpha: float) -> float:
    m = np.ascontiguousarray(m, dtype=np.float64)
    s = np.ascontiguousarray(s, dtype=np.float64)
    n = np.ascontiguousarray(n, dtype=np.int32)
    return float(lib().orc_tau_hat(_ptr(m), _ptr(s), _ptr(n), m.size, float(alpha)))


def select_thresh_box(key: np.ndarray, tau: np.ndarray, scale: float, alpha: float, delta: float) -> np.ndarray:
    key = np.ascontiguousarray(key, dtype=np.float64)
    tau = np.ascontiguousarray(tau, dtype=np.float64)
    P = key.size
    out = np.empty(max(P, 1), dtype=np.int32)
    n = lib().orc_select_thresh_box(_ptr(key), _ptr(tau), tau.size, P, float(scale), float(alpha), float(delta),
                                    _ptr(out))
    return out[:n].copy()


def select_thresh(shat: np.ndarray, tau: np.ndarray, alpha: float, delta: float) -> np.ndarray:
    shat = np.ascontiguousarray(shat, dtype=np.float64)
    tau = np.ascontiguousarray(tau, dtype=np.float64)
    G, P = shat.shape
    out = np.empty(max(P, 1), dtype=np.int32)
    n = lib().orc_select_thresh(_ptr(shat), _ptr(tau), G, P, float(alpha), float(delta), _ptr(out))
    return out[:n].copy()


def _vec(fname, z, *extra):
    z = np.ascontiguousarray(z, dtype=np.float64)
    p = np.empty_like(z)
    tau = getattr(lib(), fname)(_ptr(z), z.size, *extra, _ptr(p)) if extra else \
        getattr(lib(), fname)(_ptr(z), z.size, _ptr(p))
    return p, tau


def softmax(z):
    return _vec("orc_softmax", z)[0]


def sparsemax(z):
    return _vec("orc_sparsemax", z)


def entmax15(z):
    return _vec("orc_entmax15", z)


def entmax_bisect(z, alpha: float):
    return _vec("orc_entmax_bisect", z, float(alpha))


def entmax(z, alpha: float):
    return _vec("orc_entmax", z, float(alpha))


def attend_head(c: Cache, b: int, h: int, sel: np.ndarray, gran: int, alpha: float, scale: float):
    """Returns (out[d], p[n], tok[n]) for query head h of sequence b over the selection."""
    sel = np.ascontiguousarray(sel, dtype=np.int32)
    cap = max(len(sel) * (1 if gran == 1 else c.S), 1)
    out = np.empty(c.d)
    p = np.empty(cap)
    tok = np.empty(cap, dtype=np.int64)
    n = lib().orc_attend_head(c.ref, b, h, _ptr(sel) if len(sel) else None, len(sel), gran,
                              float(alpha), float(scale), _ptr(out), _ptr(p), _ptr(tok))
    return out, p[:n].copy(), tok[:n].copy()


def attend_full_head(c: Cache, b: int, h: int, alpha: float, scale: float):
    """Returns (out[d], p[L]) over every valid token of sequence b (token order)."""
    out = np.empty(c.d)
    p = np.empty(max(c.length(b), 1))
    n = lib().orc_attend_full_head(c.ref, b, h, float(alpha), float(scale), _ptr(out), _ptr(p))
    return out, p[:n].copy()
