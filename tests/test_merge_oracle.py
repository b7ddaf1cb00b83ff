"""Pins of the oracle's merge of attention states (the cascade / shared-prefix use of the
log-sum-exp reduction), CPU only.

The merge is tied to something other than itself: the fp64 decode oracle (pinned against
torch's SDPA) over a whole cache must equal the merge of the decodes over disjoint runs of its
keys (a prefix and suffixes cut at page boundaries); closed forms (two equal states, empty
states); and large log-sum-exp values that overflow without the max subtraction. Mutants with a
planted mistake must fail a pin.
"""
import math
import os
import tempfile

import numpy as np
import pytest

import oracle
import workloads


def check_split_keys(lib, seed=1, cuts=(2,), T=1):
    """Decode over all keys = merge of decodes over [0, c1), [c1, c2), ... (cuts in pages)."""
    s = workloads.spec(name="split", batch=3, q_per_seq=T, num_qo_heads=8, num_kv_heads=2,
                       head_dim=64, page_size=16, kv_dtype="f16", lens=("list", (200, 97, 130)))
    prob = workloads.generate(s, seed)
    o_full, l_full = oracle.decode(prob)
    P = 16
    L = prob["kv_len"].astype(np.int64)
    bounds = [0] + [c * P for c in cuts] + [None]
    states_o, states_l = [], []
    for a, b in zip(bounds[:-1], bounds[1:]):
        table = prob["page_table"][:, a // P:]
        kv = np.clip((L if b is None else np.minimum(L, b)) - a, 0, None).astype(np.int32)
        sub = dict(prob, page_table=np.ascontiguousarray(table), kv_len=kv)
        o, l_ = oracle.decode(sub)
        states_o.append(o)
        states_l.append(l_)
    o_m, l_m = oracle.merge_states(np.stack(states_o), np.stack(states_l), lib=lib)
    return np.abs(o_m - o_full).max() <= 1e-12 and np.abs(l_m - l_full).max() <= 1e-12


def check_closed_forms(lib, seed=2):
    rng = np.random.default_rng(seed)
    rows, D = 5, 32
    o1 = rng.standard_normal((rows, D))
    o2 = rng.standard_normal((rows, D))
    l1 = rng.standard_normal(rows)
    # two equal-weight states: mean of o, lse + ln 2
    o, l_ = oracle.merge_states(np.stack([o1, o2]), np.stack([l1, l1]), lib=lib)
    ok = np.allclose(o, (o1 + o2) / 2, atol=1e-14) and np.allclose(l_, l1 + math.log(2), atol=1e-14)
    # an empty state contributes nothing; all empty gives o = 0, lse = -inf
    o, l_ = oracle.merge_states(np.stack([o1, o2]), np.stack([l1, np.full(rows, -np.inf)]), lib=lib)
    ok &= np.array_equal(o, o1) and np.array_equal(l_, l1)
    o, l_ = oracle.merge_states(np.stack([o1, o2]), np.full((2, rows), -np.inf), lib=lib)
    ok &= not o.any() and np.isneginf(l_).all()
    # weights e^(l1 - lse) and e^(l2 - lse) sum to one; order of states is free
    l2 = l1 + rng.uniform(-3, 3, rows)
    o, l_ = oracle.merge_states(np.stack([o1, o2]), np.stack([l1, l2]), lib=lib)
    ob, lb = oracle.merge_states(np.stack([o2, o1]), np.stack([l2, l1]), lib=lib)
    w1, w2 = np.exp(l1 - l_), np.exp(l2 - l_)
    ok &= np.allclose(w1 + w2, 1, atol=1e-14)
    ok &= np.allclose(o, w1[:, None] * o1 + w2[:, None] * o2, atol=1e-13)
    ok &= np.allclose(o, ob, atol=1e-14) and np.allclose(l_, lb, atol=1e-14)
    return bool(ok)


def check_large_lse(lib):
    """lse values near 1e4 (exp overflows without the max subtraction)."""
    o1, o2 = np.ones((1, 8)), 3 * np.ones((1, 8))
    o, l_ = oracle.merge_states(np.stack([o1, o2]), np.array([[1e4], [1e4 + math.log(3)]]), lib=lib)
    return np.allclose(o, 2.5) and np.allclose(l_, 1e4 + math.log(4))


ALL_PINS = [
    ("split_keys_2", check_split_keys),
    ("split_keys_3", lambda lib: check_split_keys(lib, seed=3, cuts=(1, 5))),
    ("closed_forms", check_closed_forms),
    ("large_lse", check_large_lse),
]


@pytest.mark.parametrize("name,fn", ALL_PINS, ids=[n for n, _ in ALL_PINS])
def test_merge_pin(name, fn):
    assert fn(oracle.load())


MUTANTS = {15: "weight sign flipped", 16: "max dropped from lse"}


@pytest.mark.parametrize("mutant", sorted(MUTANTS), ids=[MUTANTS[m] for m in sorted(MUTANTS)])
def test_merge_pins_catch_planted_mistake(mutant):
    with tempfile.TemporaryDirectory() as d:
        lib = oracle.load(oracle.build(os.path.join(d, f"liboracle_m{mutant}.so"), mutant=mutant))
        failed = [n for n, fn in ALL_PINS if not fn(lib)]
        assert failed, f"no pin catches mutant {mutant} ({MUTANTS[mutant]})"
