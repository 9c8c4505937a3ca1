"""ctypes binding of libskv.so (include/skv.h): argument marshalling only.

PyTorch supplies device memory and the stream; every step of the decode path runs in the
library's HIP kernels. There is no fallback: if libskv.so is missing or cannot be loaded, the
calls raise. torch is imported before the library is loaded so that the library binds to the
HIP runtime torch already loaded (one runtime per process).
"""
from __future__ import annotations

import ctypes as C
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# SKV_LIB names another build of the same library (the sanitizer test loads one built with
# host-side AddressSanitizer and UndefinedBehaviorSanitizer)
LIB_PATH = os.environ.get("SKV_LIB") or os.path.join(_PKG, "libskv.so")

# status codes
SKV_OK, SKV_ERR_INVALID_ARG, SKV_ERR_UNSUPPORTED, SKV_ERR_CAPACITY, SKV_ERR_WORKSPACE, SKV_ERR_HIP = range(6)
DTYPE_F32, DTYPE_BF16 = 0, 1
META_BOX, META_GAUSS, META_PROJ, META_POOL, META_LSH = 1, 2, 4, 8, 16
SCORE_BOX, SCORE_GAUSS, SCORE_PROJ, SCORE_GAUSS_Q, SCORE_POOL, SCORE_LSH = 0, 1, 2, 3, 4, 5
SEL_TOPK, SEL_BUDGET, SEL_THRESH_GAUSS, SEL_TOKEN_TOPK, SEL_ALL, SEL_THRESH_BOX = range(6)
OP_SCORE, OP_SELECT, OP_ATTN, OP_CANDIDATES = 0, 1, 2, 3

EXPORTS = ("skv_build_page_meta", "skv_append_page_meta", "skv_score_pages", "skv_select_pages",
           "skv_sparse_decode_attn", "skv_sparse_decode_attn_noalloc", "skv_workspace_bytes", "skv_status_str")
NOALLOC_SCRATCH_BYTES = 64 << 20


class SkvError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        super().__init__(f"{what}: {status_str(code)} ({code})")


class Cache(C.Structure):
    _fields_ = [("batch", C.c_int32), ("num_q_heads", C.c_int32), ("num_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("page_size", C.c_int32), ("max_pages", C.c_int32),
                ("num_phys_pages", C.c_int32), ("dtype", C.c_int32),
                ("k", C.c_void_p), ("v", C.c_void_p), ("block_table", C.c_void_p), ("seq_lens", C.c_void_p)]


class Meta(C.Structure):
    _fields_ = [("kinds", C.c_uint32), ("box", C.c_void_p), ("gauss", C.c_void_p), ("proj_rank", C.c_int32),
                ("proj", C.c_void_p), ("kproj", C.c_void_p), ("pool_block", C.c_int32), ("pool", C.c_void_p),
                ("lsh_tables", C.c_int32), ("lsh_bits", C.c_int32), ("lsh_planes", C.c_void_p),
                ("lsh_bucket", C.c_void_p), ("vnorm", C.c_void_p)]


class Scores(C.Structure):
    _fields_ = [("key", C.c_void_p), ("m", C.c_void_p), ("s", C.c_void_p), ("shat", C.c_void_p),
                ("token_k", C.c_int32), ("cand", C.c_void_p), ("token_phase", C.c_int32),
                ("ev_begin", C.c_void_p), ("ev_end", C.c_void_p)]


class SelectParams(C.Structure):
    _fields_ = [("policy", C.c_int32), ("k", C.c_int32), ("budget_pct", C.c_int32), ("alpha", C.c_float),
                ("delta", C.c_float), ("tokens", C.c_int32), ("scale", C.c_float)]


class AttnParams(C.Structure):
    _fields_ = [("alpha", C.c_float), ("sm_scale", C.c_float), ("granularity", C.c_int32), ("split", C.c_int32),
                ("ev_begin", C.c_void_p), ("ev_end", C.c_void_p)]


_lib = None


def lib():
    """The loaded library, with argument types declared. Raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = C.CDLL(LIB_PATH)
        P, I, F, S = C.c_void_p, C.c_int32, C.c_float, C.c_size_t
        L.skv_build_page_meta.argtypes = [P, P, P]
        L.skv_append_page_meta.argtypes = [P, P, I, P]
        L.skv_score_pages.argtypes = [P, P, P, I, F, P, P, S, P]
        L.skv_select_pages.argtypes = [P, P, P, P, P, I, P, P, S, P]
        L.skv_sparse_decode_attn.argtypes = [P, P, P, P, I, P, P, P, S, P]
        L.skv_sparse_decode_attn_noalloc.argtypes = [P, P, P, P, I, P, P, P]
        L.skv_workspace_bytes.argtypes = [P, I, P, I, C.POINTER(C.c_size_t)]
        L.skv_status_str.argtypes = [I]
        L.skv_status_str.restype = C.c_char_p
        for n in EXPORTS[:-1]:
            getattr(L, n).restype = C.c_int
        _lib = L
    return _lib


def event_pair():
    """Two timing events (torch.cuda.Event) that exist on the device, for the `events` argument of
    score_pages and sparse_decode_attn: the library records them right around one kernel launch,
    and start.elapsed_time(end) is then that kernel alone. The caller owns them."""
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()   # torch creates an event on its first record
    b.record()
    return a, b


def _events(events):
    if events is None:
        return None, None
    a, b = events
    return C.c_void_p(a.cuda_event), C.c_void_p(b.cuda_event)


def status_str(code: int) -> str:
    return lib().skv_status_str(int(code)).decode()


def _check(code: int, what: str):
    if code != SKV_OK:
        raise SkvError(code, what)


def _ptr(t):
    return None if t is None else C.c_void_p(t.data_ptr())


def _stream(stream):
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


class PagedCache:
    """A paged GQA KV cache held in torch tensors.

    k, v: [num_phys_pages, num_kv_heads, page_size, head_dim] (float32 or bfloat16)
    block_table: [batch, max_pages] int32; seq_lens: [batch] int32."""

    def __init__(self, k, v, block_table, seq_lens, num_q_heads: int):
        assert k.shape == v.shape and k.dtype == v.dtype and k.is_contiguous() and v.is_contiguous()
        assert k.dtype in (torch.float32, torch.bfloat16)
        assert block_table.dtype == torch.int32 and seq_lens.dtype == torch.int32
        assert block_table.is_contiguous() and seq_lens.is_contiguous()
        self.k, self.v, self.block_table, self.seq_lens = k, v, block_table, seq_lens
        Np, Hkv, S, d = k.shape
        B, maxP = block_table.shape
        self.B, self.Hq, self.Hkv, self.d, self.S, self.maxP, self.Nphys = B, num_q_heads, Hkv, d, S, maxP, Np
        self.G = num_q_heads // Hkv
        self.dtype = k.dtype
        self.c = Cache(B, num_q_heads, Hkv, d, S, maxP, Np, DTYPE_F32 if k.dtype == torch.float32 else DTYPE_BF16,
                       k.data_ptr(), v.data_ptr(), block_table.data_ptr(), seq_lens.data_ptr())

    @property
    def ref(self):
        return C.byref(self.c)

    @property
    def device(self):
        return self.k.device


class PageMeta:
    """Per-page metadata tensors (see skv_meta in include/skv.h)."""

    def __init__(self, cache: PagedCache, kinds=("box",), proj=None, pool_block: int = 0, lsh_planes=None):
        """lsh_planes: [tables, bits, d] float32 hyperplanes of the soft-LSH kind."""
        dev, Np, Hkv, d = cache.device, cache.Nphys, cache.Hkv, cache.d
        self.kinds = 0
        self.box = self.gauss = self.kproj = self.pool = self.lsh_bucket = self.vnorm = None
        self.proj = proj
        self.pool_block = int(pool_block)
        self.lsh_planes = lsh_planes
        if "box" in kinds:
            self.kinds |= META_BOX
            cb = 64 // (2 if cache.dtype == torch.bfloat16 else 4)   # coordinates per 64-byte block
            self.box = torch.empty((Np, Hkv, d // cb, 2, cb), dtype=cache.dtype, device=dev)
        if "gauss" in kinds:
            self.kinds |= META_GAUSS
            # 64-byte blocks of the mean and variance rows alternate
            self.gauss = torch.empty((Np, Hkv, d // 16, 2, 16), dtype=torch.float32, device=dev)
        if "proj" in kinds:
            assert proj is not None and proj.dtype == torch.float32 and proj.is_contiguous()
            self.kinds |= META_PROJ
            self.kproj = torch.zeros((Np, Hkv, cache.S, proj.shape[0]), dtype=torch.int16, device=dev)
        if "pool" in kinds:
            assert self.pool_block > 0 and cache.S % self.pool_block == 0, "pool_block must divide the page size"
            self.kinds |= META_POOL
            self.pool = torch.empty((Np, Hkv, cache.S // self.pool_block, d), dtype=torch.float32, device=dev)
        tables = bits = 0
        if "lsh" in kinds:
            assert lsh_planes is not None and lsh_planes.dtype == torch.float32 and lsh_planes.is_contiguous()
            tables, bits = int(lsh_planes.shape[0]), int(lsh_planes.shape[1])
            self.kinds |= META_LSH
            self.lsh_bucket = torch.zeros((Np, Hkv, cache.S, tables), dtype=torch.uint8, device=dev)
            self.vnorm = torch.zeros((Np, Hkv, cache.S), dtype=torch.float32, device=dev)
        r = proj.shape[0] if proj is not None else 0
        self.m = Meta(self.kinds, self.box.data_ptr() if self.box is not None else None,
                      self.gauss.data_ptr() if self.gauss is not None else None, r,
                      proj.data_ptr() if proj is not None else None,
                      self.kproj.data_ptr() if self.kproj is not None else None,
                      self.pool_block, self.pool.data_ptr() if self.pool is not None else None,
                      tables, bits, lsh_planes.data_ptr() if self.lsh_bucket is not None else None,
                      self.lsh_bucket.data_ptr() if self.lsh_bucket is not None else None,
                      self.vnorm.data_ptr() if self.vnorm is not None else None)

    @property
    def ref(self):
        return C.byref(self.m)


def build_page_meta(cache: PagedCache, kinds=("box",), proj=None, stream=None, pool_block: int = 0,
                    lsh_planes=None) -> PageMeta:
    meta = PageMeta(cache, kinds, proj, pool_block, lsh_planes)
    _check(lib().skv_build_page_meta(cache.ref, meta.ref, _stream(stream)), "skv_build_page_meta")
    return meta


def append_page_meta(cache: PagedCache, meta: PageMeta, n_new: int = 1, stream=None) -> PageMeta:
    """After the last n_new tokens of every sequence were written into the cache (seq_lens counting
    them): bring the metadata of the pages holding them up to date."""
    _check(lib().skv_append_page_meta(cache.ref, meta.ref, int(n_new), _stream(stream)), "skv_append_page_meta")
    return meta


def workspace_bytes(cache: PagedCache, op: int, params, cap: int = 0) -> int:
    n = C.c_size_t(0)
    _check(lib().skv_workspace_bytes(cache.ref, op, C.byref(params), cap, C.byref(n)), "skv_workspace_bytes")
    return n.value


def _workspace(cache, nbytes: int):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=cache.device)


_KIND = {"box": SCORE_BOX, "gauss": SCORE_GAUSS, "proj": SCORE_PROJ, "gauss_q": SCORE_GAUSS_Q, "pool": SCORE_POOL,
         "lsh": SCORE_LSH}


class ScoreBuffers:
    """Output tensors of skv_score_pages for one score kind. For "proj" with token_k > 0 the
    scores are kept as the candidate set of a top-token_k selection instead of dense keys."""

    def __init__(self, cache: PagedCache, kind: str, token_k: int = 0):
        dev, B, Hq, Hkv, maxP, S = cache.device, cache.B, cache.Hq, cache.Hkv, cache.maxP, cache.S
        self.kind = kind
        self.token_k = int(token_k) if kind == "proj" else 0
        self.key = self.m = self.s = self.shat = self.cand = None
        if kind in ("box", "pool"):
            self.key = torch.empty((B, Hkv, maxP), dtype=torch.float32, device=dev)
        elif kind == "proj" and self.token_k > 0:
            n = workspace_bytes(cache, OP_CANDIDATES, C.c_int32(self.token_k))
            self.cand = torch.empty(n, dtype=torch.uint8, device=dev)
        elif kind in ("proj", "lsh"):
            self.key = torch.empty((B, Hkv, maxP * S), dtype=torch.float32, device=dev)
        elif kind in ("gauss", "gauss_q"):
            self.m, self.s, self.shat = (torch.empty((B, Hq, maxP), dtype=torch.float32, device=dev) for _ in range(3))
        else:
            raise ValueError(kind)
        ptrs = [t.data_ptr() if t is not None else None for t in (self.key, self.m, self.s, self.shat)]
        self.sc = Scores(*ptrs, self.token_k, self.cand.data_ptr() if self.cand is not None else None, 0, None, None)
        kind_i = C.c_int32(_KIND[kind])
        self.ws = _workspace(cache, workspace_bytes(cache, OP_SCORE, kind_i))

    @property
    def ref(self):
        return C.byref(self.sc)


TOKEN_PHASE_ALL, TOKEN_PHASE_BOUND, TOKEN_PHASE_FILTER = 0, 1, 2


def score_pages(cache: PagedCache, meta: PageMeta, q, kind: str, sm_scale=None, out: ScoreBuffers | None = None,
                token_k: int = 0, stream=None, phase: int = TOKEN_PHASE_ALL, temperature=None,
                events=None) -> ScoreBuffers:
    """phase (candidate scoring only): TOKEN_PHASE_BOUND / TOKEN_PHASE_FILTER run its two parts
    as separate calls, the bound first. temperature: the soft-LSH temperature ("lsh" only; it
    travels in the scale argument of the C call). events: a pair from event_pair(), recorded right
    around the scoring kernel proper."""
    assert q.dtype == cache.dtype and q.is_contiguous() and tuple(q.shape) == (cache.B, cache.Hq, cache.d)
    out = out or ScoreBuffers(cache, kind, token_k)
    if kind == "lsh":
        assert temperature is not None, "the soft-LSH scores need a temperature"
        scale = float(temperature)
    else:
        scale = float(sm_scale) if sm_scale is not None else 1.0 / math.sqrt(cache.d)
    out.sc.token_phase = int(phase)
    out.sc.ev_begin, out.sc.ev_end = _events(events)
    _check(lib().skv_score_pages(cache.ref, meta.ref, _ptr(q), _KIND[kind], scale, out.ref, _ptr(out.ws),
                                 out.ws.numel(), _stream(stream)), "skv_score_pages")
    return out


_POLICY = {"topk": SEL_TOPK, "budget": SEL_BUDGET, "thresh": SEL_THRESH_GAUSS, "token_topk": SEL_TOKEN_TOPK,
           "all": SEL_ALL, "thresh_box": SEL_THRESH_BOX}


def select_params(policy: str, k=0, budget_pct=0, alpha=1.5, delta=0.0, tokens=0, scale=0.0) -> SelectParams:
    """scale: the logit scale of the Gaussian scores (thresh_box only)."""
    return SelectParams(_POLICY[policy], int(k), int(budget_pct), float(alpha), float(delta), int(tokens),
                        float(scale))


class CombinedScores:
    """One skv_scores holding the BOX key of `box` and the Gaussian m, s, shat of `gauss` (the
    threshold policy with the box key reads both)."""

    def __init__(self, box: "ScoreBuffers", gauss: "ScoreBuffers"):
        self.parts = (box, gauss)
        self.key, self.m, self.s, self.shat = box.key, gauss.m, gauss.s, gauss.shat
        self.sc = Scores(box.key.data_ptr(), gauss.m.data_ptr(), gauss.s.data_ptr(), gauss.shat.data_ptr(), 0,
                         None, 0, None, None)

    @property
    def ref(self):
        return C.byref(self.sc)


def select_cap(cache: PagedCache, p: SelectParams) -> int:
    if p.policy in (SEL_TOPK, SEL_TOKEN_TOPK):
        return max(int(p.k), 1)
    if p.policy == SEL_BUDGET:
        return max(1, (p.budget_pct * cache.maxP + 99) // 100)
    if p.policy == SEL_ALL and p.tokens:
        return cache.maxP * cache.S
    return cache.maxP


class Selection:
    def __init__(self, cache: PagedCache, p: SelectParams, cap: int | None = None):
        dev = cache.device
        self.p = p
        self.cap = int(cap) if cap else select_cap(cache, p)
        self.idx = torch.empty((cache.B, cache.Hkv, self.cap), dtype=torch.int32, device=dev)
        self.count = torch.empty((cache.B, cache.Hkv), dtype=torch.int32, device=dev)
        self.tau_hat = torch.empty((cache.B, cache.Hq), dtype=torch.float32, device=dev)
        self.ws = _workspace(cache, workspace_bytes(cache, OP_SELECT, p, self.cap))
        self.granularity = 1 if (p.policy == SEL_TOKEN_TOPK or (p.policy == SEL_ALL and p.tokens)) else 0


def select_pages(cache: PagedCache, scores, policy: str, k=0, budget_pct=0, alpha=1.5, delta=0.0,
                 tokens=0, cap=None, out: Selection | None = None, stream=None, scale=None) -> Selection:
    """scores: ScoreBuffers, or CombinedScores for the threshold with the box key. scale: the logit
    scale of the Gaussian scores (default 1/sqrt(d))."""
    sc = float(scale) if scale is not None else 1.0 / math.sqrt(cache.d)
    p = out.p if out is not None else select_params(policy, k, budget_pct, alpha, delta, tokens, sc)
    out = out or Selection(cache, p, cap)
    _check(lib().skv_select_pages(cache.ref, scores.ref, C.byref(p), _ptr(out.idx), _ptr(out.count), out.cap,
                                  _ptr(out.tau_hat), _ptr(out.ws), out.ws.numel(), _stream(stream)),
           "skv_select_pages")
    return out


class AttnBuffers:
    def __init__(self, cache: PagedCache, p: AttnParams, cap: int):
        self.p = p
        self.cap = int(cap)
        self.out = torch.empty((cache.B, cache.Hq, cache.d), dtype=torch.float32, device=cache.device)
        self.ws = _workspace(cache, workspace_bytes(cache, OP_ATTN, p, self.cap))


def attn_params(cache: PagedCache, alpha=1.0, sm_scale=None, granularity=0, split=0) -> AttnParams:
    scale = float(sm_scale) if sm_scale is not None else 1.0 / math.sqrt(cache.d)
    return AttnParams(float(alpha), scale, int(granularity), int(split), None, None)


def sparse_decode_attn(cache: PagedCache, q, sel: Selection, alpha=1.0, sm_scale=None, split=0,
                       out: AttnBuffers | None = None, stream=None, events=None):
    """events: a pair from event_pair(), recorded right around the first attention kernel."""
    assert q.dtype == cache.dtype and q.is_contiguous() and tuple(q.shape) == (cache.B, cache.Hq, cache.d)
    out = out or AttnBuffers(cache, attn_params(cache, alpha, sm_scale, sel.granularity, split), sel.cap)
    out.p.ev_begin, out.p.ev_end = _events(events)
    _check(lib().skv_sparse_decode_attn(cache.ref, _ptr(q), _ptr(sel.idx), _ptr(sel.count), sel.cap,
                                        C.byref(out.p), _ptr(out.out), _ptr(out.ws), out.ws.numel(),
                                        _stream(stream)), "skv_sparse_decode_attn")
    return out.out


def sparse_decode_attn_noalloc(cache: PagedCache, q, sel: Selection, out, alpha=1.0, sm_scale=None, split=0,
                               stream=None):
    """skv_sparse_decode_attn_noalloc: the same attention with the library's fixed device scratch as
    its workspace (nothing allocated). `out` is a caller-owned float32 [B, Hq, d] tensor. Calls that
    overlap on one GPU race."""
    assert q.dtype == cache.dtype and q.is_contiguous() and tuple(q.shape) == (cache.B, cache.Hq, cache.d)
    assert out.dtype == torch.float32 and out.is_contiguous() and tuple(out.shape) == (cache.B, cache.Hq, cache.d)
    p = attn_params(cache, alpha, sm_scale, sel.granularity, split)
    _check(lib().skv_sparse_decode_attn_noalloc(cache.ref, _ptr(q), _ptr(sel.idx), _ptr(sel.count), sel.cap,
                                                C.byref(p), _ptr(out), _stream(stream)),
           "skv_sparse_decode_attn_noalloc")
    return out

