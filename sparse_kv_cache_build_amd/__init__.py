"""Query-aware sparse decode attention over a paged GQA KV cache, for AMD MI355X (gfx950).

The compute path is libskv.so (hand-written HIP kernels behind the C ABI of include/skv.h);
this package is its thin ctypes binding. The library loads on first use and the calls raise if
it is missing: there is no CPU fallback.
"""
from ._binding import (TOKEN_PHASE_ALL, TOKEN_PHASE_BOUND, TOKEN_PHASE_FILTER, AttnBuffers, AttnParams,
                       CombinedScores, PagedCache, PageMeta, ScoreBuffers, Selection, SelectParams, SkvError,
                       append_page_meta, attn_params, build_page_meta, event_pair, lib, score_pages, select_cap,
                       select_pages, select_params, sparse_decode_attn, sparse_decode_attn_noalloc, status_str,
                       workspace_bytes)

__all__ = ["TOKEN_PHASE_ALL", "TOKEN_PHASE_BOUND", "TOKEN_PHASE_FILTER", "AttnBuffers", "AttnParams",
           "CombinedScores", "PagedCache", "PageMeta", "ScoreBuffers", "Selection", "SelectParams", "SkvError",
           "append_page_meta", "attn_params", "build_page_meta", "event_pair", "lib", "score_pages", "select_cap",
           "select_pages", "select_params", "sparse_decode_attn", "sparse_decode_attn_noalloc", "status_str",
           "workspace_bytes"]
