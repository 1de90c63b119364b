"""CPU pins for the row-softmax oracle and the online normalizer model.

Each test pins the oracle to something other than itself: the article's
worked example, closed forms, brute force with a different formulation,
invariants the mathematics fixes, or a library sort.
"""
import json
import math
import os

import numpy as np
import pytest

from oracle import softmax_ref, topk_ref
from oracle.models import (merge_md, online_normalizer, online_softmax,
                           two_pass_unshifted_softmax)
from online_softmax_fa2_amd.inputs import softmax_rows_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# --- the article's worked example ------------------------------------------------

def test_worked_example_trace():
    g = _load("worked_example.json")
    m, d, trace = online_normalizer(g["x"])
    for (mt, dt), m_exp, d_exp in zip(trace, g["m_trace"], g["d_trace"]):
        assert mt == m_exp
        assert round(dt, g["decimals"]) == pytest.approx(d_exp, abs=1e-12)
    # The rescale when 3 arrives: 1.3679 * exp(2 - 3) = 0.5032.
    assert round(math.exp(2 - 3), 4) == g["rescale_factor_at_element_3"]
    assert round(trace[1][1] * math.exp(2 - 3), 4) == g["rescaled_old_sum_at_element_3"]


def test_worked_example_outputs():
    g = _load("worked_example.json")
    y = softmax_ref(np.array([g["x"]]))[0]
    assert np.round(y, 4).tolist() == g["y"]
    assert np.round(online_softmax(g["x"]), 4).tolist() == g["y"]
    assert abs(y.sum() - 1) < 1e-15


def test_worked_example_merge():
    g = _load("worked_example.json")
    x = g["x"]
    left = online_normalizer(x[:2])[:2]
    right = online_normalizer(x[2:])[:2]
    assert left[0] == g["merge_left"][0] and round(left[1], 4) == g["merge_left"][1]
    assert right[0] == g["merge_right"][0] and round(right[1], 4) == g["merge_right"][1]
    M, D = merge_md(left, right)
    assert M == g["merge_result"][0] and round(D, 4) == g["merge_result"][1]


# --- closed forms and brute force --------------------------------------------------

def test_constant_row_is_uniform():
    for n in (1, 2, 7, 1000):
        y = softmax_ref(np.full((1, n), 3.25))[0]
        assert np.all(y == 1.0 / n) or np.max(np.abs(y - 1.0 / n)) < 1e-16


def test_two_elements_is_logistic():
    rng = np.random.default_rng(11)
    for a, b in rng.normal(size=(50, 2)) * 5:
        y = softmax_ref(np.array([[a, b]]))[0]
        assert y[0] == pytest.approx(1.0 / (1.0 + math.exp(b - a)), rel=1e-14)


@pytest.mark.parametrize("seed", range(20))
def test_brute_force_tiny_rows(seed):
    """Unshifted exp with an exactly rounded sum on tiny, small-magnitude rows."""
    rng = np.random.default_rng([7, seed])
    n = int(rng.integers(1, 7))
    x = rng.uniform(-20, 20, size=n)
    e = [math.exp(float(v)) for v in x]
    z = math.fsum(e)
    want = np.array([v / z for v in e])
    assert np.max(np.abs(softmax_ref(x[None])[0] - want)) < 1e-15


def test_large_gap_is_one_hot():
    x = np.array([[0.0, -800.0, 5.0, -1.0e4]])
    y = softmax_ref(x)[0]
    assert y[2] == pytest.approx(1.0, abs=1e-2)
    assert y[3] == 0.0 and y[1] == 0.0


# --- invariants the pages fix ------------------------------------------------------

def test_rows_sum_to_one():
    x = softmax_rows_inputs(64, 4000, seed=3)
    y = softmax_ref(x)
    assert np.max(np.abs(y.sum(axis=1) - 1.0)) < 1e-14


@pytest.mark.parametrize("c", [1000.0, -1000.0, 0.5])
def test_shift_invariance(c):
    x = softmax_rows_inputs(16, 300, seed=4).astype(np.float64)
    assert np.max(np.abs(softmax_ref(x + c) - softmax_ref(x))) < 1e-14


def test_large_scores_stay_finite_where_unshifted_is_nan():
    """Scores of magnitude 1e4 (page 'Derive online softmax, prove it is exact')."""
    rng = np.random.default_rng(5)
    x = rng.uniform(-1, 1, size=100) * 1e4
    y = softmax_ref(x[None])[0]
    assert np.all(np.isfinite(y)) and abs(y.sum() - 1) < 1e-15
    assert np.isnan(two_pass_unshifted_softmax(x)).any()
    assert np.all(np.isfinite(online_softmax(x)))
    assert np.max(np.abs(online_softmax(x) - y)) <= 1e-15


def test_overflow_thresholds():
    facts = _load("page_facts.json")
    fp16_max = float(np.finfo(np.float16).max)
    fp32_max = float(np.finfo(np.float32).max)
    assert round(math.log(fp16_max), 2) == facts["fp16_exp_overflow_x"]["value"]
    assert round(math.log(fp32_max), 1) == facts["fp32_exp_overflow_x"]["value"]
    with np.errstate(over="ignore"):
        assert np.isinf(np.exp(np.float16(11.1)))
        assert np.isfinite(np.exp(np.float16(11.08)))
        assert np.isinf(np.exp(np.float32(88.75)))
        assert np.isfinite(np.exp(np.float32(88.7)))


def test_bf16_sum_stagnates_past_256():
    import torch
    facts = _load("page_facts.json")
    s = torch.tensor(float(facts["bf16_sum_stagnation"]["value"]), dtype=torch.bfloat16)
    assert (s + torch.tensor(1.0, dtype=torch.bfloat16)).item() == 256.0
    s2 = torch.tensor(255.0, dtype=torch.bfloat16)
    assert (s2 + torch.tensor(1.0, dtype=torch.bfloat16)).item() == 256.0
    s3 = torch.tensor(128.0, dtype=torch.bfloat16)
    assert (s3 + torch.tensor(1.0, dtype=torch.bfloat16)).item() == 129.0


@pytest.mark.parametrize("seed", range(10))
def test_normalizer_bounds(seed):
    """Article 'Online softmax', Step 2: after j elements, 1 <= d <= j."""
    x = np.random.default_rng([8, seed]).normal(size=200) * 30
    _, _, trace = online_normalizer(x)
    for j, (_, d) in enumerate(trace, start=1):
        assert 1.0 <= d <= j


@pytest.mark.parametrize("seed", range(10))
def test_merge_associative_any_grouping(seed):
    """Article 'Online softmax', Step 4: the merge is associative."""
    rng = np.random.default_rng([9, seed])
    x = rng.normal(size=int(rng.integers(2, 65))) * 10
    nblk = int(rng.integers(2, min(len(x), 64) + 1))
    cuts = np.sort(rng.choice(np.arange(1, len(x)), size=nblk - 1, replace=False))
    pairs = [online_normalizer(b)[:2] for b in np.split(x, cuts)]
    whole = online_normalizer(x)[:2]
    # left fold
    acc = pairs[0]
    for p in pairs[1:]:
        acc = merge_md(acc, p)
    # random tree
    work = list(pairs)
    while len(work) > 1:
        i = int(rng.integers(0, len(work) - 1))
        work[i:i + 2] = [merge_md(work[i], work[i + 1])]
    for got in (acc, work[0]):
        assert got[0] == whole[0]
        assert got[1] == pytest.approx(whole[1], rel=1e-14)
    # the empty pair is the identity
    assert merge_md((-math.inf, 0.0), whole) == whole


def test_online_equals_safe_on_1000_vectors():
    """Article 'Online softmax', 'Worked example': 1,000 seeded vectors, < 1e-12."""
    facts = _load("page_facts.json")["exactness_claims"]
    rng = np.random.default_rng(12)
    worst = 0.0
    for _ in range(facts["online_vs_safe_vectors"]):
        x = rng.normal(size=int(rng.integers(1, 40))) * 5
        _, d, _ = online_normalizer(x)
        y_safe = softmax_ref(x[None])[0]
        e = np.exp(x - x.max())
        worst = max(worst, abs(d - e.sum()), float(np.max(np.abs(online_softmax(x) - y_safe))))
    assert worst < facts["online_vs_safe_max_err"]


# --- top-k ---------------------------------------------------------------------------

def test_topk_matches_stable_full_sort():
    x = softmax_rows_inputs(32, 2500, seed=6)
    vals, idx = topk_ref(x, 5)
    y = softmax_ref(x)
    for r in range(x.shape[0]):
        order = np.lexsort((np.arange(x.shape[1]), -x[r].astype(np.float64)))
        assert idx[r].tolist() == order[:5].tolist()
        assert np.all(vals[r] == y[r, order[:5]])
        assert np.all(np.diff(vals[r]) <= 0)


def test_topk_ties_take_lower_index():
    x = np.array([[1.0, 3.0, 3.0, 2.0, 3.0, -1.0],
                  [0.0, 0.0, 0.0, 0.0, 0.0, 0.0]], dtype=np.float32)
    _, idx = topk_ref(x, 4)
    assert idx[0].tolist() == [1, 2, 4, 3]
    assert idx[1].tolist() == [0, 1, 2, 3]


def test_topk_brute_force_small():
    rng = np.random.default_rng(13)
    for _ in range(50):
        n = int(rng.integers(1, 12))
        k = int(rng.integers(1, n + 1))
        x = rng.integers(-3, 4, size=(1, n)).astype(np.float32)  # many ties
        _, idx = topk_ref(x, k)
        # brute force: repeatedly take the first maximal element not yet taken
        left = list(range(n))
        want = []
        for _ in range(k):
            best = left[0]
            for c in left:
                if x[0, c] > x[0, best]:
                    best = c
            want.append(best)
            left.remove(best)
        assert idx[0].tolist() == want


def _first_max_selection(row, k):
    """Brute force without sorting: k times, scan the row left to right and take the first element that is
    maximal among those not yet taken (so equal values go to the lower column first)."""
    taken = set()
    out = []
    for _ in range(k):
        best = None
        for c in range(len(row)):
            if c in taken:
                continue
            if best is None or row[c] > row[best]:
                best = c
        taken.add(best)
        out.append(best)
    return out


@pytest.mark.parametrize("cols,k", [(65, 16), (3000, 16), (25000, 5), (4099, 1)])
def test_topk_wide_rows_with_massive_ties_brute_force(cols, k):
    """Rows wider than 64 columns (the lexsort path of topk_order) with integer values in [-3, 3], so that
    hundreds of columns share each value: the order must be the first-maximal selection."""
    rng = np.random.default_rng([14, cols])
    x = rng.integers(-3, 4, size=(3, cols)).astype(np.float32)
    x[2, :] = 0.0  # one row entirely tied
    x[2, cols // 2] = -1.0
    _, idx = topk_ref(x, k)
    for r in range(x.shape[0]):
        assert idx[r].tolist() == _first_max_selection(x[r].tolist(), k)
