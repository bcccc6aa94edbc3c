"""Property checks of the C ABI's host-side size queries over the whole int32
argument range (negative, zero, huge, overflowing products): each returns
its documented "invalid" value exactly when include/lsa.h says the
arguments are invalid, and otherwise a size consistent with the split rule
it reports.  These functions make no HIP call, so they run without a GPU."""
import ctypes

import pytest

hypothesis = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

SIZE_INVALID = ctypes.c_size_t(-1).value
I32 = st.one_of(st.integers(-4, 300), st.sampled_from([0, 1, 2, 16, 64, 128, 4096, 2 ** 20, 2 ** 30, 2 ** 31 - 1,
                                                       -1, -(2 ** 31)]))


@pytest.fixture(scope="module")
def lib():
    import lookahead_chunk_sparse_amd as m
    return m.load_library()


def _attend_valid(B, Hq, Hkv, d, k):
    return (B >= 1 and Hq >= 1 and Hkv >= 1 and k >= 1 and Hq % Hkv == 0 and Hq // Hkv <= 16 and d in (64, 128)
            and B * Hq < 2 ** 24 and B * k < 2 ** 31)


@settings(max_examples=400, deadline=None)
@given(B=I32, Hq=st.one_of(I32, st.sampled_from([8, 64])), Hkv=st.one_of(I32, st.sampled_from([1, 8])),
       d=st.one_of(I32, st.sampled_from([64, 128])), k=I32, n_split=I32)
def test_attend_workspace_size(lib, B, Hq, Hkv, d, k, n_split):
    got = lib.lsa_gather_attend_workspace_size(B, Hq, Hkv, d, k, n_split)
    if not _attend_valid(B, Hq, Hkv, d, k) or n_split < 0:
        assert got == SIZE_INVALID
        return
    eff = lib.lsa_gather_attend_default_splits(B, Hkv, k) if n_split == 0 else n_split
    assert 1 <= lib.lsa_gather_attend_default_splits(B, Hkv, k) <= k
    eff = min(eff, k)
    if B * Hkv * eff >= 2 ** 24:  # more split workgroups than one launch may have
        assert got == SIZE_INVALID
        return
    if eff == 1:
        assert got == 0
    else:
        # at least the fp32 partial outputs and the (m, l) pairs of every split
        parts = B * Hkv * eff * (Hq // Hkv)
        assert got >= parts * d * 4 + parts * 2 * 4
        assert got % 4 == 0
    # n_split = 0 means the library's own choice
    if n_split == 0:
        assert got == lib.lsa_gather_attend_workspace_size(B, Hq, Hkv, d, k,
                                                           lib.lsa_gather_attend_default_splits(B, Hkv, k))


@settings(max_examples=300, deadline=None)
@given(B=I32, Hkv=I32, k=I32)
def test_default_splits(lib, B, Hkv, k):
    s = lib.lsa_gather_attend_default_splits(B, Hkv, k)
    if B < 1 or Hkv < 1 or k < 1:
        assert s == -1
    else:
        assert 1 <= s <= k


@settings(max_examples=400, deadline=None)
@given(B=I32, k=I32, k_tok=I32)
def test_topk_tokens_workspace_size(lib, B, k, k_tok):
    got = lib.lsa_topk_tokens_workspace_size(B, k, k_tok)
    if B < 1 or k < 1 or k_tok < 1 or k * 64 > 2 ** 30:
        assert got == SIZE_INVALID
        return
    assert got != SIZE_INVALID
    if got:
        # a split happens only for long rows, and holds a (position, key) pair
        # for each of at least two slices' k_tok candidates per row
        assert k * 64 > 32768
        assert got >= B * 2 * k_tok * 8


def test_attend_workspace_size_never_wraps(lib):
    """Arguments whose partial-output bytes would pass 2^64 are rejected,
    not answered with a wrapped size (B*Hkv*n_split split workgroups must
    stay below 2^24, B*Hq below 2^24)."""
    assert lib.lsa_gather_attend_workspace_size(1, 2 ** 30, 2 ** 30, 128, 2 ** 30, 2 ** 30) == SIZE_INVALID
    big = 2 ** 31 - 1
    assert lib.lsa_gather_attend_workspace_size(1, big, big, 128, big, big) == SIZE_INVALID
    assert lib.lsa_gather_attend_workspace_size(1, 2 ** 20, 2 ** 20, 128, 64, 16) == SIZE_INVALID  # 2^24 groups
    assert lib.lsa_gather_attend_workspace_size(1, 2 ** 20, 2 ** 20, 128, 64, 15) not in (0, SIZE_INVALID)
    assert lib.lsa_gather_attend_workspace_size(2 ** 18, 64, 8, 128, 276, 2) == SIZE_INVALID  # B*Hq = 2^24


BOGUS = 1 << 20  # a non-null, aligned address that no rejected call dereferences


def test_launch_size_limits_are_rejected_before_any_hip_call(lib):
    """Calls whose launch would count more work-items than 32 bits hold are
    rejected by validation (no kernel is launched: these run without a GPU)."""
    # top-k rows: 1024-thread workgroups, fewer than 2^22 of them
    assert lib.lsa_topk_chunks(BOGUS, 1 << 22, 8, 2, BOGUS, None) == 2
    assert b"2^22" in lib.lsa_last_error()
    assert lib.lsa_threshold_chunks(BOGUS, 1 << 22, 8, 0, 2, BOGUS, BOGUS, None) == 2
    # attention: B*Hq below 2^24
    args = [BOGUS, BOGUS, 4, BOGUS, None, None, BOGUS, None, None, 0, 1 << 18, 64, 8, 128, 2, 0.1, BOGUS, 1 << 30, 2,
            BOGUS, None]
    assert lib.lsa_gather_attend(*args) == 2 and b"2^24" in lib.lsa_last_error()
    # pool assignment: one 1024-thread workgroup per request
    assert lib.lsa_pool_assign(None, None, 0, BOGUS, 1 << 22, 4, 8, BOGUS, BOGUS, None) == 2
    # pull fetch: the caller's grid
    assert lib.lsa_fetch_chunks_pull(BOGUS, 4, BOGUS, None, BOGUS, 4, 1, 1, 64, 2, 1 << 24, None) == 1
