"""Pins of the oracle's dispatch step (expert-contiguous rows padded to BM).

The grouping is the "sort tokens by expert id" of "Mixture of Experts optimiza
Transformers y LLMs", section "Ejecución eficiente: backends de expertos"
(grouped_mm backend) together with the token duplication of the glossary
"MoE (Mixture of Experts - Mezcla de Expertos)", section 3 step 3.  Stability
(ascending assignment index inside each expert) is a reading: the pages leave
the order inside an expert open.
"""
import numpy as np
import pytest

import oracle


def _check(ids, E, BM, shared):
    T, k = ids.shape
    r = oracle.align(ids, E, BM, shared=shared)
    flat = ids.ravel()
    A = T * k
    # brute force: Python's sort of (expert, assignment) pairs
    ref = [a for _, a in sorted((int(flat[a]), a) for a in range(A))]
    assert r["sorted_assign"].tolist() == ref
    counts = np.bincount(flat, minlength=E)
    G = E + (1 if shared else 0)
    exp_counts = np.concatenate([counts, [T]]) if shared else counts
    assert r["counts"].tolist() == exp_counts.tolist()
    assert r["offsets"][0] == 0 and np.array_equal(np.diff(r["offsets"]), exp_counts)
    pad = np.diff(r["padded"])
    assert np.all(pad % BM == 0) and np.all(pad >= exp_counts) and np.all(pad - exp_counts < BM)
    assert r["padded"][G] <= A + G * (BM - 1) + (T if shared else 0)
    assert r["n_tiles"] * BM == r["padded"][G]
    # every segment holds only its own expert, ascending; row_of is consistent
    for e in range(E):
        seg = r["sorted_assign"][r["offsets"][e]:r["offsets"][e + 1]]
        assert np.all(flat[seg] == e) and np.all(np.diff(seg) > 0)
        rows = r["row_of"][seg]
        assert rows.tolist() == list(range(r["padded"][e], r["padded"][e] + len(seg)))
    # row_token: token of each real row, -1 on padding
    rt = r["row_token"]
    assert np.array_equal(rt[r["row_of"]], np.arange(A) // k)
    real = np.zeros(len(rt), bool)
    real[r["row_of"]] = True
    if shared:
        base = r["padded"][E]
        assert np.array_equal(rt[base:base + T], np.arange(T))
        real[base:base + T] = True
    assert np.all(rt[~real] == -1)
    # tile -> group
    for i, g in enumerate(r["tile_group"]):
        assert r["padded"][g] <= i * BM < r["padded"][g + 1]
    return r


@pytest.mark.parametrize("T,k,E,BM", [(64, 2, 8, 16), (300, 4, 32, 32), (1, 4, 32, 16),
                                      (513, 8, 256, 64), (100, 2, 8, 128)])
def test_align_random(T, k, E, BM):
    rng = np.random.default_rng(T + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    _check(ids, E, BM, False)
    _check(ids, E, BM, True)


def test_align_all_to_one_expert_and_empty_experts():
    T, k, E = 77, 2, 8
    ids = np.tile(np.array([[5, 2]], np.int32), (T, 1))
    r = _check(ids, E, 32, False)
    assert r["counts"].tolist() == [0, 0, T, 0, 0, T, 0, 0]


def test_align_zero_tokens():
    ids = np.zeros((0, 2), np.int32)
    r = oracle.align(ids, 8, 16)
    assert r["n_tiles"] == 0 and np.all(r["padded"] == 0)


def test_align_rejects_bad_ids():
    with pytest.raises(ValueError):
        oracle.align(np.array([[0, 9]], np.int32), 8, 16)
