"""MI355X (gfx950) implementation of the decode-time hot path of Lookahead
Sparse Attention (LSA, "FlashMemory"): memory-indexer scan, top-k chunk
re-selection every tau = 64 steps, gathered-chunk GQA decode attention, and a
host-tier chunk fetch.

The compute runs in hand-written HIP kernels behind a C ABI (include/lsa.h,
``liblsa.so``); this package binds that ABI with the same names and adds the
decode schedule (``decode.LsaDecoder``).  Importing it fails if the library
has not been built: there is no CPU fallback.
"""
from ._binding import (CHUNK_TOKENS, EXPORTS, LIB_PATH, LsaError, alloc_workspace, load_library,
                       lsa_fetch_chunks, lsa_fetch_chunks_pull, lsa_gather_attend, lsa_gather_attend_default_splits,
                       lsa_gather_attend_tokens, lsa_fetch_chunks_staged, alloc_fetch_staging,
                       lsa_gather_attend_workspace_size, lsa_index_score, lsa_pool_assign, lsa_threshold_chunks,
                       lsa_topk_chunks, lsa_topk_tokens, lsa_topk_tokens_workspace_size,
                       alloc_topk_tokens_workspace, lsa_set_tuning, lsa_get_tuning, tuning, TUNE_KNOBS,
                       lsa_gather_attend_noalloc, NOALLOC_SCRATCH_BYTES, lsa_check_ids)

load_library()

__all__ = ["CHUNK_TOKENS", "EXPORTS", "LIB_PATH", "LsaError", "alloc_workspace", "load_library",
           "lsa_fetch_chunks", "lsa_fetch_chunks_pull", "lsa_gather_attend", "lsa_gather_attend_default_splits",
           "lsa_gather_attend_tokens", "lsa_fetch_chunks_staged", "alloc_fetch_staging",
           "lsa_gather_attend_workspace_size", "lsa_index_score", "lsa_pool_assign", "lsa_threshold_chunks", "lsa_topk_chunks",
           "lsa_topk_tokens", "lsa_topk_tokens_workspace_size", "alloc_topk_tokens_workspace",
           "lsa_set_tuning", "lsa_get_tuning", "tuning", "TUNE_KNOBS", "lsa_gather_attend_noalloc",
           "NOALLOC_SCRATCH_BYTES", "lsa_check_ids"]
