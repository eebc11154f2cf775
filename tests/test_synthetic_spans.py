"""Host checks of the image-span input recipe: spans disjoint and within
length bounds, last keys at the image's end for its rows and the own
position elsewhere, and chunk plans that never cut an image (PR #1183 body:
a prompt chunk never cuts through an image; PR #975 commit body: a cut that
would moves before the image, or past it when the chunk starts there)."""
import numpy as np
import pytest

from synthetic.gen import chunk_starts, image_span_last_keys, image_spans


@pytest.mark.parametrize("seed,n", [(1, 8192), (2, 2000), (3, 1700), (4, 32768)])
def test_spans_and_chunks(seed, n):
    spans = image_spans(np.random.default_rng(seed), n)
    assert len(spans) == 6
    prev = -1
    for a, b in spans:
        assert prev < a <= b < n and 64 <= b - a + 1 <= 280
        prev = b
    lk = image_span_last_keys(0, n, spans)
    inside = np.zeros(n, bool)
    for a, b in spans:
        assert np.all(lk[a:b + 1] == b)
        inside[a:b + 1] = True
    assert np.array_equal(lk[~inside], np.arange(n)[~inside])
    for mx in (128, 512):
        st = chunk_starts(n, mx, spans)
        ends = st[1:] + [n]
        assert st[0] == 0 and all(e > s for s, e in zip(st, ends))
        for s, e in zip(st, ends):
            # no image straddles a cut; a chunk is longer than mx only when
            # it starts at an image longer than mx and ends right after it
            for a, b in spans:
                assert not (a < e <= b) and not (a < s <= b)
            if e - s > mx:
                assert any(a == s and b + 1 == e for a, b in spans)


def test_chunk_cut_moves_before_an_image():
    assert chunk_starts(1000, 300, [(250, 400)]) == [0, 250, 550, 850]
    assert chunk_starts(1000, 100, [(100, 299)]) == [0, 100, 300, 400, 500, 600, 700, 800, 900]


def test_last_keys_with_offset():
    lk = image_span_last_keys(10, 8, [(12, 14)])
    assert lk.tolist() == [10, 11, 14, 14, 14, 15, 16, 17]
