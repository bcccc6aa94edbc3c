"""lsa_check_ids, the opt-in check of a chunk list: the lists the selects
write pass; a list with an id or store position out of range, a value listed
twice or a count out of range is refused, and the message names the first
offending request and entry.  Bad lists are given to the check only, never
to an attention or fetch kernel."""
import numpy as np
import pytest

from conftest import gpu_available
from helpers import to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


@pytest.fixture(scope="module")
def lsa():
    import lookahead_chunk_sparse_amd as m
    return m


def _selection(lsa, synth_lib, B, C, k, seed):
    """Top-k ids of random logits, as the library writes them."""
    logits = synth_lib.uniform_i32((B, C), seed, synth_lib.stream(synth_lib.TAG_MISC, 9500), -1000, 1000)
    return lsa.lsa_topk_chunks(to_dev(logits), k).cpu().numpy()


def test_valid_lists_pass(lsa, synth_lib):
    B, C, k = 3, 2048, 276
    ids = _selection(lsa, synth_lib, B, C, k, seed=1)
    lsa.lsa_check_ids(to_dev(ids), C)
    # with a compact pool's permuted slots
    slots = np.stack([np.random.default_rng(b).permutation(k) for b in range(B)]).astype(np.int32)
    lsa.lsa_check_ids(to_dev(ids), C, C_store=k, slots=to_dev(slots))
    # threshold output: -1 padding past each count is not looked at
    logits = synth_lib.uniform_i32((B, C), 2, synth_lib.stream(synth_lib.TAG_MISC, 9501), -1000, 1000)
    tids, counts = lsa.lsa_threshold_chunks(to_dev(logits), k, 900)
    assert (counts.cpu().numpy() < k).all() and (tids.cpu().numpy() == -1).any()
    lsa.lsa_check_ids(tids, C, counts=counts)
    # the largest list the check takes, and a single entry
    big = np.arange(16384, dtype=np.int32)[None]
    lsa.lsa_check_ids(to_dev(big), 16384)
    lsa.lsa_check_ids(to_dev(np.array([[5]], dtype=np.int32)), 6)


def _expect(lsa, ids, C, match, **kw):
    with pytest.raises(lsa.LsaError, match=match) as e:
        lsa.lsa_check_ids(to_dev(ids), C, **{k: (to_dev(v) if isinstance(v, np.ndarray) else v) for k, v in kw.items()})
    assert e.value.status == 1
    print("  refused:", e.value, flush=True)


def test_bad_lists_are_refused(lsa, synth_lib):
    B, C, k = 3, 2048, 276
    ids = _selection(lsa, synth_lib, B, C, k, seed=3)

    bad = ids.copy()
    bad[1, 5] = C  # one past the context
    _expect(lsa, bad, C, r"request 1 entry 5: chunk id 2048 \(must be in \[0, 2048\)\)")

    bad = ids.copy()
    bad[2, 0] = -7
    _expect(lsa, bad, C, r"request 2 entry 0: chunk id -7")

    bad = ids.copy()
    bad[0, 200] = bad[0, 17]  # listed twice: the later entry is named
    _expect(lsa, bad, C, rf"request 0 entry 200: chunk id {ids[0, 17]} listed twice")

    # errors in two requests: the first one (in request, then entry order) is named
    bad = ids.copy()
    bad[2, 3] = C + 5
    bad[1, 100] = -1
    _expect(lsa, bad, C, r"request 1 entry 100")

    slots = np.tile(np.arange(k, dtype=np.int32), (B, 1))
    sl = slots.copy()
    sl[1, 9] = k  # store position out of a pool of k slots
    _expect(lsa, ids, C, r"request 1 entry 9: .* store position 276 \(must be in \[0, 276\)\)", C_store=k, slots=sl)
    sl = slots.copy()
    sl[2, 50] = sl[2, 40]
    _expect(lsa, ids, C, r"request 2 entry 50: store position 40 listed twice", C_store=k, slots=sl)

    counts = np.array([k, k + 1, 3], dtype=np.int32)
    _expect(lsa, ids, C, r"request 1: count 277 outside \[0, k=276\]", counts=counts)
    counts = np.array([k, 10, -2], dtype=np.int32)
    _expect(lsa, ids, C, r"request 2: count -2", counts=counts)

    # without slots the ids are the store positions: C_store bounds them too
    _expect(lsa, ids, C, r"must be in \[0, 1000\)\)", C_store=1000)


def test_entries_past_the_count_are_not_checked(lsa, synth_lib):
    B, C, k = 2, 500, 40
    ids = _selection(lsa, synth_lib, B, C, k, seed=4)
    counts = np.array([30, 40], dtype=np.int32)
    bad = ids.copy()
    bad[0, 30:] = -1       # padding past the count
    bad[0, 35] = 99999     # garbage past the count
    lsa.lsa_check_ids(to_dev(bad), C, counts=to_dev(counts))
    bad[0, 29] = -1        # inside the count
    _expect(lsa, bad, C, r"request 0 entry 29", counts=counts)
