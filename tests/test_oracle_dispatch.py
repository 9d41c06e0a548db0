"""Pins of the oracle's dispatch plan, capacity rule and permutation."""
import os

import numpy as np
import pytest

from oracle import moe_oracle as O
from workloads import make

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def random_topk(rng, T, E, k):
    return np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)


def test_capacity_worked_example_from_page():
    rows = [l.split() for l in open(os.path.join(GOLDEN, "capacity_worked_example.txt"))
            if l.strip() and not l.startswith("#")]
    assert rows
    for b, s, k, E, want in rows:
        T = int(b) * int(s)
        assert O.capacity(T, int(k), int(E), 1.0) == int(want)


def test_capacity_rounding_and_none():
    assert O.capacity(16384, 2, 128, 1.25) == 320
    assert O.capacity(10, 1, 3, 1.0) == 4           # ceil(10/3)
    assert O.capacity(9, 1, 3, 1.0) == 3            # exact, no spurious round-up
    assert O.capacity(100, 2, 8, 0.1) == 3          # 0.1 taken as the decimal 1/10: ceil(2.5)
    assert O.capacity(100, 2, 8, None) == -1


@pytest.mark.parametrize("T,E,k", [(1, 1, 1), (7, 3, 2), (64, 8, 2), (300, 64, 8), (257, 256, 8)])
def test_uncapped_full_range_is_stable_argsort(T, E, k):
    rng = np.random.default_rng(T + E + k)
    idx = random_topk(rng, T, E, k)
    plan = O.dispatch(idx, E)
    ref = np.argsort(idx.ravel(), kind="stable")
    assert np.array_equal(plan["sorted_pair"], ref)
    bc = np.bincount(idx.ravel(), minlength=E)
    assert np.array_equal(plan["counts"], bc)
    assert np.array_equal(plan["offsets"], np.concatenate([[0], np.cumsum(bc)]))
    assert plan["n_kept"] == T * k


def test_position_is_count_of_earlier_tokens():
    rng = np.random.default_rng(11)
    T, E, k = 40, 6, 3
    idx = random_topk(rng, T, E, k)
    plan = O.dispatch(idx, E)
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            earlier = sum(1 for t2 in range(t) if e in idx[t2])
            assert plan["pos"][t * k + j] == earlier


def test_hand_worked_plan():
    # 4 tokens, E = 3, k = 2, capacity 1, local experts [1, 3)
    idx = np.array([[1, 0], [1, 2], [2, 0], [0, 1]], dtype=np.int32)
    plan = O.dispatch(idx, 3, capacity=1, e_begin=1, e_end=3)
    assert plan["counts"].tolist() == [3, 3, 2]
    # expert 1: pairs 0 (t0), 2 (t1), 7 (t3) -> keep pair 0
    # expert 2: pairs 3 (t1), 4 (t2)         -> keep pair 3
    # expert 0: pairs 1 (t0), 5 (t2), 6 (t3) -> keep pair 1 (remote)
    assert plan["offsets"].tolist() == [0, 1, 2]
    assert plan["sorted_pair"].tolist() == [0, 3]
    assert plan["pair_pos"].tolist() == [0, O.REMOTE, O.DROPPED, 1, O.DROPPED, O.DROPPED,
                                         O.DROPPED, O.DROPPED]
    assert plan["n_kept"] == 2


@pytest.mark.parametrize("cap,e0,e1", [(-1, 0, 16), (5, 0, 16), (5, 4, 9), (0, 0, 16),
                                       (1000, 0, 16), (3, 15, 16)])
def test_plan_invariants(cap, e0, e1):
    rng = np.random.default_rng(abs(cap) + 7 * e0)
    T, E, k = 200, 16, 4
    idx = random_topk(rng, T, E, k)
    plan = O.dispatch(idx, E, cap, e0, e1)
    counts, off, sp, pp = plan["counts"], plan["offsets"], plan["sorted_pair"], plan["pair_pos"]
    assert counts.sum() == T * k
    kept_e = counts if cap < 0 else np.minimum(counts, cap)
    assert np.array_equal(np.diff(off), kept_e[e0:e1])
    assert off[0] == 0 and off[-1] == plan["n_kept"] == len(sp)
    # bijection between local rows and local kept pairs
    rows = pp[pp >= 0]
    assert sorted(rows.tolist()) == list(range(plan["n_kept"]))
    assert np.array_equal(pp[sp], np.arange(plan["n_kept"]))
    # each segment holds only its expert, in ascending token order
    for i in range(e1 - e0):
        seg = sp[off[i]:off[i + 1]]
        assert np.all(idx.ravel()[seg] == e0 + i)
        assert np.all(np.diff(seg // k) > 0)
    # accounting: kept local + dropped + kept remote = T*k
    n_drop = int((pp == O.DROPPED).sum())
    n_remote = int((pp == O.REMOTE).sum())
    assert plan["n_kept"] + n_drop + n_remote == T * k
    assert n_drop == int((counts - kept_e).sum())
    if cap == 0:
        assert plan["n_kept"] == 0 and n_drop == T * k
    if cap >= T:
        assert n_drop == 0


def test_dropped_pairs_are_the_latest_tokens():
    T, E, k = 30, 2, 1
    idx = np.zeros((T, k), dtype=np.int32)     # every token picks expert 0
    plan = O.dispatch(idx, E, capacity=7)
    assert plan["pair_pos"].tolist() == list(range(7)) + [O.DROPPED] * 23


def test_rejects_out_of_range_index():
    with pytest.raises(ValueError):
        O.dispatch(np.array([[0, 3]], dtype=np.int32), 3)
    with pytest.raises(ValueError):
        O.dispatch(np.array([[0, -1]], dtype=np.int32), 3)


def test_permute_is_row_copy():
    x = np.arange(24, dtype=np.uint16).reshape(6, 4)
    sp = np.array([5, 0, 3], dtype=np.int32)   # pairs with k = 2 -> tokens 2, 0, 1
    xp = O.permute(x, sp, 2)
    assert xp.dtype == np.uint16
    assert np.array_equal(xp, x[[2, 0, 1]])


def test_ep_rank_share_plan():
    """The expert-parallel workload: capacity 320 of 128 experts, experts [0, 32) local."""
    wl = make("ep_rank_share")
    C = O.capacity(wl.T, wl.k, wl.E, wl.capacity_factor)
    assert C == 320
    idx, _ = O.route(wl.logits, wl.k, wl.gate)
    plan = O.dispatch(idx, wl.E, C, wl.e_begin, wl.e_end)
    kept = np.minimum(plan["counts"], C)
    assert plan["n_kept"] == int(kept[:32].sum()) <= 32 * C
    assert plan["n_kept"] + (plan["pair_pos"] == O.DROPPED).sum() + \
        (plan["pair_pos"] == O.REMOTE).sum() == wl.T * wl.k
