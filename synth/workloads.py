"""The five decode workloads and how their synthetic inputs are assembled.

Shapes follow the pages' DeepSeek-V4 GQA description (64 query heads, 8 KV
heads, head dim 128; sergiiob.dev handbook page, section "Grouped Query
Attention (GQA) vs. Multi-Head Attention (MHA)") and the retention budgets the pages report (13.5% average
footprint, 10% at 500K and 1M; paperlayer.ai summary, Abstract and
"3 Experiments / Main Results").  The evaluation suites the pages measure on
(LongBench-v2, LongMemEval, RULER, MRCR) are not available; these seeded
inputs stand in for them, with the same context lengths and retention.

Recipe (seed 0 unless a test says otherwise):
  * indexer query  q_idx[b][qi][:]  uniform int in [-16, 15]  (one per
    interval when the workload drifts, else one for the whole run);
  * indexer keys   K_idx[b][c][:]   uniform int in [-16, 15];
  * golden chunks  n_golden positions per request (and per interval when the
    workload drifts, disjoint from earlier intervals' sets), uniform without
    replacement; their keys are 8*sign(q_idx) + uniform int in [-4, 4]
    (sign(0) = 0), so they score high against that interval's query;
  * K/V store      kv[b][c][K|V][g][t][i] bf16 N(0,1), chunk-major;
  * query          q[t][b][h][i] bf16 N(0,1), fresh each step.
Churn-controlled indexer (a workload with churn > 0, for the host tier):
every chunk sits at an angle on a ring (theta_c = 2 pi perm(c) / C, perm a
seeded permutation per request, so neighbouring angles are scattered chunk
ids), its key is K[c][i] = round(15 cos(theta_c - pi i / d_idx)), and the
interval-i query is q[i'] = round(15 cos(phi_i - pi i' / d_idx)) with
phi_i = phi_0 + i * churn * 2 pi k / C.  A query then favours the chunks
nearest its angle, an arc of about k chunks, and the arc moves by about
`churn` of its length per interval (the exact fraction is whatever the
selections give; the benchmark measures it).

No value here is computed by the method; the generator is SplitMix64
(see synth.c).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

from . import (TAG_GOLD_NOISE, TAG_GOLD_POS, TAG_KIDX, TAG_KV, TAG_Q, TAG_QIDX, TAG_RING, TAG_RING_PHASE, choose,
               normal_bf16, normal_bf16_into, normal_bf16_runs, raw_u64, stream, uniform_i8)

CHUNK_TOKENS = 64  # tokens per KV chunk (T)
TAU = 64           # decode steps between re-selections


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int            # requests in the batch
    Hq: int           # query heads
    Hkv: int          # KV heads
    d: int            # head dim
    N: int            # context tokens per request
    k: int            # retained chunks per request
    steps: int        # decode steps
    d_idx: int        # indexer dim
    n_golden: int     # planted chunks per request (per interval if drifting)
    drift: bool = False
    host_tier: bool = False
    seed: int = 0
    nq: int = 1
    T: int = CHUNK_TOKENS
    tau: int = TAU
    churn: float = 0.0   # > 0: the ring indexer, moving by about this fraction of k per interval

    @property
    def C(self) -> int:
        return (self.N + self.T - 1) // self.T

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def intervals(self) -> int:
        return (self.steps + self.tau - 1) // self.tau

    @property
    def alpha(self) -> float:
        """Scale applied to the logit before the sigmoid: 1/(16*d_idx), a
        power of two so alpha*logit is exact in fp32."""
        return 1.0 / (16.0 * self.d_idx)

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def lag(self) -> int:
        """Interval i attends with the selection of interval i - lag."""
        return 1 if self.host_tier else 0

    @property
    def tile_bytes(self) -> int:
        """One (chunk, K|V, kv-head) tile of bf16."""
        return self.T * self.d * 2

    @property
    def chunk_bytes(self) -> int:
        """One chunk: K and V for all KV heads."""
        return 2 * self.Hkv * self.tile_bytes

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", B=1, Hq=8, Hkv=1, d=64, N=4096, k=8, steps=64, d_idx=64, n_golden=4),
    "32k": Workload("32k", B=4, Hq=64, Hkv=8, d=128, N=32768, k=32, steps=256, d_idx=128,
                    n_golden=26),
    "128k": Workload("128k", B=16, Hq=64, Hkv=8, d=128, N=131072, k=276, steps=256, d_idx=128,
                     n_golden=102, drift=True),
    "500k": Workload("500k", B=8, Hq=64, Hkv=8, d=128, N=500000, k=782, steps=128, d_idx=128,
                     n_golden=156),
    "1m_host": Workload("1m_host", B=4, Hq=64, Hkv=8, d=128, N=1048576, k=1638, steps=128,
                        d_idx=128, n_golden=164, host_tier=True),
}
WORKLOAD_ORDER = ["tiny", "32k", "128k", "500k", "1m_host"]


def query_interval(w: Workload, interval: int) -> int:
    """Which generated indexer query serves re-selection `interval`."""
    return interval if (w.drift or w.churn) else 0


def _ring_offsets(w: Workload) -> np.ndarray:
    """Angular offsets pi i / d_idx of the indexer dimensions."""
    return np.pi * np.arange(w.d_idx) / w.d_idx


def _ring_int8(angles: np.ndarray, w: Workload) -> np.ndarray:
    """round(15 cos(angle - offset_i)) for every angle and dimension i."""
    v = np.rint(15.0 * np.cos(angles[..., None] - _ring_offsets(w)))
    return v.astype(np.int8)


def ring_angles(w: Workload) -> np.ndarray:
    """float64 [B][C]: the ring angle of every chunk (a seeded permutation of
    C equally spaced angles per request)."""
    out = np.empty((w.B, w.C), dtype=np.float64)
    for b in range(w.B):
        perm = choose(w.C, w.C, w.seed, stream(TAG_RING, b))
        out[b] = 2.0 * np.pi * perm / w.C
    return out


def ring_query_angle(w: Workload, interval: int) -> np.ndarray:
    """float64 [B]: the interval's query angle on the ring."""
    phase = raw_u64(w.B, w.seed, stream(TAG_RING_PHASE)).astype(np.float64) / 2.0 ** 64 * 2.0 * np.pi
    return phase + interval * w.churn * 2.0 * np.pi * w.k / w.C


def indexer_query(w: Workload, interval: int) -> np.ndarray:
    """int8 [B][nq][d_idx]."""
    if w.churn:
        assert w.nq == 1
        return _ring_int8(ring_query_angle(w, interval), w)[:, None, :]
    return uniform_i8((w.B, w.nq, w.d_idx), w.seed, stream(TAG_QIDX, query_interval(w, interval)), -16, 15)


def golden_sets(w: Workload) -> list[np.ndarray]:
    """Per generated query (one per interval if drifting, else one): int32
    [B][nq][n_golden] planted positions.  Drifting sets are disjoint from all
    earlier intervals' sets of the same request."""
    nsets = w.intervals if w.drift else 1
    out = [np.zeros((w.B, w.nq, w.n_golden), dtype=np.int32) for _ in range(nsets)]
    for b in range(w.B):
        used = np.zeros(w.C, dtype=np.uint8)
        for s in range(nsets):
            for qi in range(w.nq):
                pos = choose(w.n_golden, w.C, w.seed,
                             stream(TAG_GOLD_POS, (b << 20) | (s << 8) | qi), used)
                assert pos.size == w.n_golden, "not enough chunks for disjoint golden sets"
                out[s][b, qi] = pos
                used[pos] = 1
    return out


def indexer_keys(w: Workload) -> np.ndarray:
    """int8 [B][C][d_idx]: background uniform keys with golden chunks planted
    against every generated query (frozen for the whole run); for a workload
    with churn, the ring keys."""
    if w.churn:
        return _ring_int8(ring_angles(w), w)
    K = uniform_i8((w.B, w.C, w.d_idx), w.seed, stream(TAG_KIDX), -16, 15)
    noise = uniform_i8((w.B, w.C, w.d_idx), w.seed, stream(TAG_GOLD_NOISE), -4, 4)
    sets = golden_sets(w)
    for s, gs in enumerate(sets):
        q = indexer_query(w, s)  # [B][nq][d_idx]
        for b in range(w.B):
            for qi in range(w.nq):
                sign = np.sign(q[b, qi].astype(np.int32))
                for c in gs[b, qi]:
                    K[b, c] = (8 * sign + noise[b, c].astype(np.int32)).astype(np.int8)
    return K


def kv_elems_per_request(w: Workload, C_store: int | None = None) -> int:
    return (w.C if C_store is None else C_store) * 2 * w.Hkv * w.T * w.d


def kv_fill_request(w: Workload, b: int, out: np.ndarray) -> np.ndarray:
    """Fill the K/V store of request b: uint16 [C][2][Hkv][T][d] (bf16 bits)."""
    n = kv_elems_per_request(w)
    assert out.size == n and out.dtype == np.uint16
    return normal_bf16_into(out, w.seed, stream(TAG_KV), first=b * n)


def kv_store(w: Workload) -> np.ndarray:
    """uint16 [B][C][2][Hkv][T][d].  Only for workloads that fit in host RAM."""
    out = np.empty((w.B, w.C, 2, w.Hkv, w.T, w.d), dtype=np.uint16)
    for b in range(w.B):
        kv_fill_request(w, b, out[b].reshape(-1))
    return out


def kv_chunks(w: Workload, b: int, chunks: np.ndarray) -> np.ndarray:
    """Regenerate chunks `chunks` of request b: uint16 [len][2][Hkv][T][d]."""
    chunks = np.asarray(chunks, dtype=np.int64)
    per_chunk = 2 * w.Hkv * w.T * w.d
    first = b * kv_elems_per_request(w) + chunks * per_chunk
    runs = normal_bf16_runs(first, per_chunk, w.seed, stream(TAG_KV))
    return runs.reshape(len(chunks), 2, w.Hkv, w.T, w.d)


def attn_query(w: Workload, t: int, scale: float = 1.0) -> np.ndarray:
    """uint16 [B][Hq][d] bf16 bits of the step-t query (times `scale`)."""
    return normal_bf16((w.B, w.Hq, w.d), w.seed, stream(TAG_Q, t), scale=scale)


def ctx_lens(w: Workload) -> np.ndarray:
    return np.full(w.B, w.N, dtype=np.int32)


# ---- placing the K/V store (torch is used for memory only) ----------------

def device_kv_store(w: Workload, device="cuda"):
    """The K/V store in device memory: torch bf16 [B][C][2][Hkv][T][d],
    generated request by request on the host and copied over."""
    import torch
    out = torch.empty((w.B, w.C, 2, w.Hkv, w.T, w.d), dtype=torch.bfloat16, device=device)
    n = kv_elems_per_request(w)
    host = torch.empty(n, dtype=torch.int16).pin_memory()
    buf = host.numpy().view(np.uint16)
    for b in range(w.B):
        kv_fill_request(w, b, buf)
        out[b].view(-1).view(torch.int16).copy_(host, non_blocking=False)
    return out


def pinned_kv_store(w: Workload):
    """The K/V store in pinned host memory: torch bf16 [B][C][2][Hkv][T][d]."""
    import torch
    out = torch.empty((w.B, w.C, 2, w.Hkv, w.T, w.d), dtype=torch.bfloat16, pin_memory=True)
    flat = out.view(torch.int16).numpy().view(np.uint16).reshape(w.B, -1)
    for b in range(w.B):
        kv_fill_request(w, b, flat[b])
    return out
