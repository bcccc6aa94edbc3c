"""Decode schedule for one attention layer (or several sharing a selection) on one GPU.

Every tau = 64 decode steps the memory indexer scores all chunks against the
current indexer query and the top-k chunks are re-selected; every step
attends over the selected chunks only (paperlayer.ai summary of
"FlashMemory-DeepSeek-V4", 1 Introduction and 2.1 Architecture: the indexer
runs every tau steps and predicts what the upcoming tau-step window needs;
3 Experiments / Experimental Setup: tau = 64).

Two placements of the K/V:
  * HBM-resident store (lag 0): interval i attends with the selection made at
    its own first step.
  * Host tier (lag 1): the whole K/V lives in pinned host memory; the chunks
    of selection i are copied into an HBM pool on a side stream while interval
    i decodes with selection i-1 (the handbook page's asynchronous prefetch;
    in the summary, chunks not recalled leave GPU memory for the CPU), so the copy
    overlaps attention.  Two pool buffers alternate; the first interval waits
    for its own fetch.  The copy is either a device-side gather that reads
    the selected ids on the GPU (fetch="pull", the default: no host round
    trip, graph-capturable) or DMA copies issued from the host, spread over
    several copy streams (fetch="memcpy": the ids, and the slots, are copied
    to the host first; the copies use no compute unit), or the same DMA
    through a staging buffer (fetch="staged": the host gathers the chunks to
    fetch, which cross the link in large copies and are scattered into the
    pool on the device; the host waits for its copies, so not under graph
    capture).
    With delta=True (the default) one pool of 2k slots replaces the two
    buffers: chunks selected again keep their slot and only new chunks are
    copied, into slots the selection being attended over does not hold.

Two selection rules: a fixed budget of k chunks (selection="topk"), or the
pages' sigmoid gating (selection="threshold": chunks whose score passes 0.5,
i.e. logit > 0, at most k of them; 2.1 Architecture and 2.4 Configuration of
the summary), whose budget varies per request.

A token-level second stage (token_topk=k_tok) keeps, at every step, only
the k_tok best tokens of the recalled chunks by the model's own token scores,
passed to attend() (summary 2.1 Architecture: the native token-level top-k
runs over the recalled subset only; the pages give no scoring formula, so
the scores are an input), and attends over those tokens.

Several layers can share one selection (kv, or host_kv, given as a list of
per-layer stores): each interval runs one indexer scan and selection, then
every step attends over the same chunks in every layer.  On the host tier
every layer has its own HBM pool, filled at the same slots.  Reusing one layer's selection
in the following layers is how the indexer cost is amortised across depth
(the "Daily Papers" listing for the query "lightning indexer": the LongCat
LSA abstract's cross-layer indexing, and the Multi-layer Indexer and
IndexCache abstracts, which reuse a top-k across consecutive layers).

This module only orders calls into liblsa.so on HIP streams and records
events; it computes nothing itself.
"""
from __future__ import annotations

import math

import torch

from ._binding import (CHUNK_TOKENS, alloc_fetch_staging, alloc_topk_tokens_workspace, alloc_workspace,
                       lsa_fetch_chunks, lsa_fetch_chunks_pull, lsa_fetch_chunks_staged, lsa_gather_attend,
                       lsa_index_score, lsa_pool_assign, lsa_threshold_chunks, lsa_topk_chunks, lsa_topk_tokens)

TAU = 64


def selection_for_step(t: int, tau: int = TAU, lag: int = 0) -> int:
    """Re-selection whose chunks step t attends over (interval t//tau, minus lag, at least 0)."""
    return max(t // tau - lag, 0)


class LsaDecoder:
    """Decode state: indexer keys, K/V placement, selection buffers.

    k_idx    device int8 [B][C][d_idx]
    ctx_len  device int32 [B]
    kv       device bf16 [B][C][2][Hkv][64][d]        (HBM-resident store; a list
                                                        of such: one per layer), or
    host_kv  pinned bf16 [B][C][2][Hkv][64][d]        (host tier; a list of such:
                                                        one per layer, one pool each)
    """

    def __init__(self, *, k_idx: torch.Tensor, ctx_len: torch.Tensor, Hq: int, k: int, alpha: float,
                 kv: torch.Tensor | None = None, host_kv: torch.Tensor | None = None, tau: int = TAU,
                 n_split: int = 0, sm_scale: float | None = None, fetch: str = "pull", fetch_grid: int = 0,
                 delta: bool | None = None, selection: str = "topk", logit_threshold: int = 0,
                 seg_kv: torch.Tensor | None = None, seg_len: torch.Tensor | None = None, token_topk: int = 0,
                 stage_chunks: int = 1024, device="cuda"):
        if (kv is None) == (host_kv is None):
            raise ValueError("give exactly one of kv (HBM store) or host_kv (host tier)")
        self.k_idx = k_idx
        self.ctx_len = ctx_len
        self.layers = list(kv) if isinstance(kv, (list, tuple)) else None
        self.host_layers = list(host_kv) if isinstance(host_kv, (list, tuple)) else None
        if self.layers is not None:
            kv = self.layers[0]
        if self.host_layers is not None:
            host_kv = self.host_layers[0]
            self.layers = self.host_layers  # one attention per layer, each on its own pool
        # resident segment: the local window and the decoded tokens, always in
        # HBM and attended with the recalled chunks (ctx_len then bounds only
        # the offloadable history); the caller appends to it and bumps seg_len
        self.seg_kv, self.seg_len = seg_kv, seg_len
        self.kv = kv
        self.host_kv = host_kv
        store = kv if kv is not None else host_kv
        self.B, self.C, _, self.Hkv, self.T, self.d = store.shape
        self.Hq, self.k, self.alpha, self.tau = Hq, k, alpha, tau
        self.d_idx = k_idx.shape[2]
        self.lag = 1 if host_kv is not None else 0
        # The host tier keeps the library's split count too (0).  Measured on
        # the 1M workload with the 16-workgroup pull fetch: with the delta
        # fetch and a stable selection (the steady state) it runs 3,992
        # steps/s against 3,633 with 4x the splits; while the host link is
        # busy all interval (a drifting query, or full re-fetches) 4x the
        # splits balance around the fetch workgroups only 1-2% better.
        self.n_split = n_split
        if fetch not in ("pull", "memcpy", "staged"):
            raise ValueError("fetch must be 'pull', 'memcpy' or 'staged'")
        self.fetch, self.fetch_grid = fetch, fetch_grid
        if selection not in ("topk", "threshold"):
            raise ValueError("selection must be 'topk' or 'threshold'")
        self.selection, self.logit_threshold = selection, int(logit_threshold)
        self.delta = True if delta is None else bool(delta)
        if selection == "threshold" and host_kv is not None and fetch != "pull" and not self.delta:
            # the -1 padding past a request's count is skipped through its slot (-1)
            raise NotImplementedError(f"threshold selection with fetch='{fetch}' on the host tier needs delta=True")
        self.sm_scale = 1.0 / math.sqrt(self.d) if sm_scale is None else sm_scale
        dev = torch.device(device)
        B = self.B
        self.logits = torch.empty((B, 1, self.C), dtype=torch.int32, device=dev)
        self.scores = torch.empty((B, 1, self.C), dtype=torch.float32, device=dev)
        # selection buffers alternate by selection parity so a new selection
        # never overwrites the one the current interval attends with
        self.sel_ids = [torch.empty((B, k), dtype=torch.int32, device=dev) for _ in range(2)]
        self.sel_counts = [torch.empty(B, dtype=torch.int32, device=dev) for _ in range(2)] \
            if selection == "threshold" else [None, None]
        self.k_tok = int(token_topk)
        if self.k_tok:
            self.tok = torch.empty((B, self.k_tok), dtype=torch.int32, device=dev)
            self.tok_counts = torch.empty(B, dtype=torch.int32, device=dev)
            self.tok_workspace = alloc_topk_tokens_workspace(B, k, self.k_tok, device=dev)
            entries = (self.k_tok + CHUNK_TOKENS - 1) // CHUNK_TOKENS
            self.workspace = alloc_workspace(B, Hq, self.Hkv, self.d, entries, n_split, device=dev)
        else:
            self.workspace = alloc_workspace(B, Hq, self.Hkv, self.d, k, n_split, device=dev)
        if self.lag:
            n_pools = len(self.host_layers) if self.host_layers is not None else 1
            self.pools = []  # per layer: the pool buffers of selections 0 and 1
            for _ in range(n_pools):
                if self.delta:
                    one = torch.empty((B, 2 * k, 2, self.Hkv, self.T, self.d), dtype=torch.bfloat16, device=dev)
                    self.pools.append([one, one])  # one pool, indexed through per-selection slots
                else:
                    self.pools.append([torch.empty((B, k, 2, self.Hkv, self.T, self.d), dtype=torch.bfloat16,
                                                   device=dev) for _ in range(2)])
            self.pool = self.pools[0]
            if self.delta:
                self.sel_slots = [torch.empty((B, k), dtype=torch.int32, device=dev) for _ in range(2)]
                self.fetch_slots = [torch.empty((B, k), dtype=torch.int32, device=dev) for _ in range(2)]
            self.slots = torch.arange(k, dtype=torch.int32, device=dev).repeat(B, 1).contiguous()
            self.host_ids = [torch.empty((B, k), dtype=torch.int32).pin_memory() for _ in range(2)]
            self.host_slots = [torch.empty((B, k), dtype=torch.int32).pin_memory() for _ in range(2)] \
                if self.delta and fetch != "pull" else None
            # the staged fetch's buffers (two halves of stage_chunks / 2 chunks
            # each, the size of one copy over the link)
            self.staging = alloc_fetch_staging(host_kv, max(2, min(int(stage_chunks), 2 * B * k)), device=dev) \
                if fetch == "staged" else None
            self.side = torch.cuda.Stream(device=dev)
            self.ev_ids = torch.cuda.Event()
            self.ev_sel = torch.cuda.Event()
            self.fetch_done = [torch.cuda.Event() for _ in range(2)]
            self.attn_done = torch.cuda.Event()
            self._attn_done_valid = False
            # set to a list to record (interval, start, end) timing events
            # around every fetch on the side stream (eager use only, not
            # under graph capture)
            self.fetch_events = None

    # ---- single operations -------------------------------------------------
    def reselect(self, q_idx: torch.Tensor, sel: int, stream=None) -> torch.Tensor:
        """Score every chunk against q_idx (int8 [B][1][d_idx]) and keep the top k
        into selection buffer sel % 2."""
        lsa_index_score(q_idx, self.k_idx, self.alpha, logits=self.logits, scores=self.scores, stream=stream)
        ids = self.sel_ids[sel % 2]
        if self.selection == "threshold":
            lsa_threshold_chunks(self.logits.view(self.B, self.C), self.k, self.logit_threshold, chunk_ids=ids,
                                 counts=self.sel_counts[sel % 2], stream=stream)
        else:
            lsa_topk_chunks(self.logits.view(self.B, self.C), self.k, chunk_ids=ids, stream=stream)
        return ids

    def attend(self, q: torch.Tensor, sel: int, out: torch.Tensor, stream=None, layer: int = 0,
               token_scores: torch.Tensor | None = None) -> torch.Tensor:
        """One decode step's attention with selection `sel` (on the host tier
        with the delta fetch, the selection's pool slots must have been
        assigned, as run_interval does).  With the token stage, token_scores
        (fp32 [B][k*64], the step's scores of the recalled tokens by list
        position) pick the k_tok tokens attended over."""
        ids = self.sel_ids[sel % 2]
        tok = {}
        if self.k_tok:
            if token_scores is None:
                raise ValueError("the token stage needs this step's token_scores")
            lsa_topk_tokens(token_scores, ids, self.ctx_len, self.k_tok, counts=self.sel_counts[sel % 2],
                            tok=self.tok, tok_counts=self.tok_counts, workspace=self.tok_workspace, stream=stream)
            tok = dict(tok=self.tok, tok_counts=self.tok_counts)
        if self.lag:
            slots = self.sel_slots[sel % 2] if self.delta else self.slots
            return lsa_gather_attend(q, self.pools[layer][sel % 2], ids, self.ctx_len, self.sm_scale, slots=slots,
                                     workspace=self.workspace, n_split=self.n_split, out=out,
                                     counts=self.sel_counts[sel % 2], seg_kv=self.seg_kv, seg_len=self.seg_len,
                                     stream=stream, **tok)
        kv = self.layers[layer] if self.layers is not None else self.kv
        return lsa_gather_attend(q, kv, ids, self.ctx_len, self.sm_scale, workspace=self.workspace,
                                 n_split=self.n_split, out=out, counts=self.sel_counts[sel % 2],
                                 seg_kv=self.seg_kv, seg_len=self.seg_len, stream=stream, **tok)

    # ---- one interval ------------------------------------------------------
    def run_interval(self, i: int, q_idx: torch.Tensor, qs, outs, token_scores=None) -> None:
        """Enqueue interval i: its re-selection and len(qs) attention steps.
        qs[j] is the bf16 [B][Hq][d] query of step i*tau + j; outs[j] receives
        its fp32 output (the same tensor may be passed for every step);
        token_scores[j] is step j's token scores when the token stage is on."""
        ts = token_scores if token_scores is not None else [None] * len(qs)
        if not self.lag:
            self.reselect(q_idx, i)
            for q, o, sc in zip(qs, outs, ts):
                if self.layers is None:
                    self.attend(q, i, o, token_scores=sc)
                else:  # q[l] and o[l] per layer; one selection for all layers
                    for layer in range(len(self.layers)):
                        self.attend(q[layer], i, o[layer], layer=layer)
            return
        main = torch.cuda.current_stream()
        self.reselect(q_idx, i)
        if self.delta:
            prev = (self.sel_ids[(i - 1) % 2], self.sel_slots[(i - 1) % 2]) if i >= 1 else (None, None)
            lsa_pool_assign(prev[0], prev[1], self.sel_ids[i % 2], 2 * self.k, new_slots=self.sel_slots[i % 2],
                            fetch_slots=self.fetch_slots[i % 2])
        if self.fetch != "pull":
            self.host_ids[i % 2].copy_(self.sel_ids[i % 2], non_blocking=True)
            if self.delta:
                self.host_slots[i % 2].copy_(self.fetch_slots[i % 2], non_blocking=True)
            self.ev_ids.record(main)
        else:
            self.ev_sel.record(main)
        if i == 0:
            self._fetch(0)
        src = max(i - 1, 0)
        main.wait_event(self.fetch_done[src % 2])
        for q, o, sc in zip(qs, outs, ts):
            if self.layers is None:
                self.attend(q, src, o, token_scores=sc)
            else:  # q[l] and o[l] per layer; one selection, one pool per layer
                for layer in range(len(self.layers)):
                    self.attend(q[layer], src, o[layer], layer=layer)
        if i >= 1:
            self._fetch(i)  # overlaps the steps just enqueued
        self.attn_done.record(main)
        self._attn_done_valid = True

    def _fetch(self, i: int) -> None:
        """Copy selection i's chunks from host into pool buffer i % 2 on the side stream."""
        if self._attn_done_valid:
            # pool buffer i % 2 was last read by the previous interval
            self.side.wait_event(self.attn_done)
        timing = self.fetch_events is not None
        if timing and self.fetch == "pull":
            self.side.wait_event(self.ev_sel)  # start the clock once the copy may begin
        if timing:
            ev0 = torch.cuda.Event(enable_timing=True)
            ev0.record(self.side)
        if self.fetch != "pull":
            self.ev_ids.synchronize()  # the ids (and slots) must be on the host before the copies are issued
            slots = self.host_slots[i % 2] if self.delta else None
            for host, pool in zip(self.host_layers or [self.host_kv], self.pools):
                if self.fetch == "staged":
                    lsa_fetch_chunks_staged(host, self.host_ids[i % 2], pool[i % 2], *self.staging,
                                            host_slots=slots, stream=self.side)
                else:
                    lsa_fetch_chunks(host, self.host_ids[i % 2], pool[i % 2], host_slots=slots, stream=self.side,
                                     done=None)
        else:
            self.side.wait_event(self.ev_sel)  # selection i (and its slots) are on the device
            for host, pool in zip(self.host_layers or [self.host_kv], self.pools):
                lsa_fetch_chunks_pull(host, self.sel_ids[i % 2], pool[i % 2],
                                      slots=self.fetch_slots[i % 2] if self.delta else None, grid=self.fetch_grid,
                                      stream=self.side)
        if timing:
            ev1 = torch.cuda.Event(enable_timing=True)
            ev1.record(self.side)
            self.fetch_events.append((i, ev0, ev1))
        self.fetch_done[i % 2].record(self.side)

    def join(self) -> None:
        """Make the current stream wait for every copy issued so far (needed
        before the end of a graph capture, and before reading the pool)."""
        if self.lag:
            for ev in self.fetch_done:
                torch.cuda.current_stream().wait_event(ev)
