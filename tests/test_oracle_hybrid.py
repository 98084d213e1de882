"""Pins of the oracle's hybrid read (compressed history + exact ring tokens).

The hybrid read is softmax attention over the union of the two key sets
("TurboQuant Triton deep dive": capture ring in the write path, hybrid mode
in the limits section).  Pinned here against what holds independently of its
code: where the boundary between the parts falls must not matter, an empty
part must reduce to plain attention, a lone exact token is returned exactly,
and merging the online-softmax records of the compressed splits with the
ring's record (what the GPU path does) gives the same output.
"""

import numpy as np

from oracle import attention as oatt


def _data(seed, n, d=16):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(d) * 2.0, rng.standard_normal((n, d)), rng.standard_normal((n, d))


def test_boundary_between_parts_does_not_matter():
    q, k, v = _data(0, 40)
    ref, _ = oatt.softmax_attention(q, k, v)
    for a in (0, 1, 17, 39, 40):
        o, _ = oatt.hybrid_attention(q, k[:a], v[:a], k[a:], v[a:])
        assert np.allclose(o, ref, rtol=1e-12, atol=1e-12)


def test_empty_parts_reduce_to_plain_attention():
    q, k, v = _data(1, 9)
    ref, _ = oatt.softmax_attention(q, k, v)
    o1, _ = oatt.hybrid_attention(q, k, v, k[:0], v[:0])
    o2, _ = oatt.hybrid_attention(q, k[:0], v[:0], k, v)
    assert np.allclose(o1, ref) and np.allclose(o2, ref)
    o3, _ = oatt.hybrid_attention(q, k[:0], v[:0], k[:0], v[:0])
    assert np.all(o3 == 0.0)


def test_single_exact_token_is_returned_exactly():
    q, k, v = _data(2, 1)
    o, s = oatt.hybrid_attention(q, k[:0], v[:0], k, v)
    assert np.array_equal(o, v[0])
    assert np.isclose(s[0], k[0] @ q / np.sqrt(q.shape[0]))


def test_split_records_plus_ring_record_merge_to_the_hybrid_output():
    q, k, v = _data(3, 70)
    comp, ring = 50, 20
    ref, s = oatt.hybrid_attention(q, k[:comp], v[:comp], k[comp:], v[comp:])
    recs = oatt.split_records(s[:comp], v[:comp], [0, 16, 32, 48, 50, 50])
    recs += oatt.split_records(s[comp:], v[comp:], [0, ring])
    assert np.allclose(oatt.combine_records(recs), ref, rtol=1e-12, atol=1e-12)
