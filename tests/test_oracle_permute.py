"""Pins of the oracle's histogram / scan / scatter against the invariants of
a dropless permutation and a brute-force Python sort."""
import numpy as np
import pytest

import oracle


def _check(ids, E, out):
    T, k = ids.shape
    n = T * k
    flat = ids.reshape(-1)
    # brute force: slots are the pairs q sorted by (expert, q)
    order = sorted(range(n), key=lambda q: (int(flat[q]), q))
    assert list(out["slot_token"]) == [q // k for q in order]
    assert list(out["slot_k"]) == [q % k for q in order]
    counts = np.bincount(flat, minlength=E)
    assert np.array_equal(out["counts"], counts)
    assert out["counts"].sum() == n
    assert out["offsets"][0] == 0 and out["offsets"][-1] == n
    assert np.array_equal(np.diff(out["offsets"]), counts)
    # bijection: token_slot is the inverse of (slot_token, slot_k)
    inv = out["token_slot"]
    assert sorted(inv) == list(range(n))
    q_of_slot = out["slot_token"] * k + out["slot_k"]
    assert np.array_equal(q_of_slot[inv], np.arange(n))
    # each segment holds only its expert, in increasing q (stable)
    for e in range(E):
        seg = q_of_slot[out["offsets"][e]:out["offsets"][e + 1]]
        assert (flat[seg] == e).all()
        assert (np.diff(seg) > 0).all()


@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (7, 2, 5), (64, 8, 256), (333, 3, 7),
                                   (1000, 6, 64)])
def test_permute_random(T, k, E):
    rng = np.random.default_rng(T + k + E)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    _check(ids, E, oracle.permute(ids, E))


def test_permute_all_to_one_expert_and_empty_experts():
    T, k, E = 50, 1, 40
    ids = np.full((T, k), 17, np.int32)
    out = oracle.permute(ids, E)
    _check(ids, E, out)
    assert out["counts"][17] == T and out["counts"].sum() == T


def test_permute_rejects_out_of_range():
    with pytest.raises(ValueError):
        oracle.permute(np.array([[0, 3]], np.int32), 3)
