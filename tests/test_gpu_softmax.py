"""GPU parity: online_softmax_rows and online_softmax_topk_rows against the oracle."""
import numpy as np
import pytest
import torch

import online_softmax_fa2_amd as osfa
from online_softmax_fa2_amd.inputs import WORKLOADS, softmax_rows_inputs
from oracle import softmax_ref, topk_ref
from tests.gpu_util import Guarded, assert_f32_rel, upload_f32

pytestmark = pytest.mark.gpu


def _run_rows(x_np):
    x = upload_f32(x_np)
    y = Guarded(x_np.shape, torch.float32)
    osfa.online_softmax_rows(x, out=y.t)
    torch.cuda.synchronize()
    y.check()
    return y.t.cpu().numpy()


@pytest.mark.parametrize("rows,cols", [
    (1, 1), (7, 3), (5, 4), (33, 1000), (17, 1001), (64, 4000), (8, 8192), (3, 8196),
    (4, 8193), (3, 20000), (2, 100003), (300, 63), (2, 1024), (2, 4096), (2, 4097),
    # 4096 rows or more: one wave per row for rows of up to 2048 aligned floats, one wave per two rows
    # (rows g and g + ceil(rows / 2)) up to 4096; odd row counts leave the last wave one row
    (4097, 4), (4099, 1000), (4100, 2000), (4097, 4096), (4099, 2052), (4096, 4100),
])
def test_softmax_rows_parity(rows, cols):
    print(f"softmax_rows rows={rows} cols={cols}", flush=True)
    x = softmax_rows_inputs(rows, cols, seed=rows * 7 + cols)
    y = _run_rows(x)
    assert_f32_rel(y, softmax_ref(x), what=f"softmax {rows}x{cols}")
    assert np.max(np.abs(y.astype(np.float64).sum(axis=1) - 1.0)) <= cols * 2.0 ** -23


def test_softmax_rows_large_magnitude_and_shift():
    """Scores of magnitude 1e4 stay finite; y(x + c) = y(x) for exact shifts."""
    rng = np.random.default_rng(3)
    x = (rng.uniform(-1, 1, size=(16, 777)) * 1e4).astype(np.float32)
    y = _run_rows(x)
    assert np.all(np.isfinite(y))
    assert_f32_rel(y, softmax_ref(x), what="1e4")
    # inputs on a 2^-8 grid so that adding 1024 is exact in float32
    x2 = np.round(softmax_rows_inputs(8, 500, seed=9) * 256) / 256
    y1 = _run_rows(x2)
    y2 = _run_rows(x2 + np.float32(1024.0))
    assert np.array_equal((x2 + np.float32(1024.0)).astype(np.float64), x2.astype(np.float64) + 1024.0)
    assert_f32_rel(y2, softmax_ref(x2.astype(np.float64) + 1024.0), what="shifted")
    assert np.max(np.abs(y1 - y2)) < 1e-5


def test_softmax_rows_constant_and_one_hot():
    x = np.full((4, 300), 2.5, np.float32)
    assert np.allclose(_run_rows(x), 1.0 / 300, rtol=1e-6, atol=0)
    x = np.zeros((3, 100), np.float32)
    x[:, 17] = 200.0
    y = _run_rows(x)
    assert np.all(y[:, 17] == 1.0) and np.all(np.delete(y, 17, axis=1) == 0.0)


def test_softmax_rows_in_place():
    x_np = softmax_rows_inputs(20, 4000, seed=11)
    x = upload_f32(x_np)
    osfa.online_softmax_rows(x, out=x)
    torch.cuda.synchronize()
    assert_f32_rel(x.cpu().numpy(), softmax_ref(x_np), what="in place")


def test_softmax_rows_full_workload():
    w = WORKLOADS["softmax_rows_4096x4000"]
    x_np = softmax_rows_inputs(w["rows"], w["cols"], seed=w["seed"], sigma=w["sigma"])
    print("softmax_rows full 4096x4000", flush=True)
    y = _run_rows(x_np)
    assert_f32_rel(y, softmax_ref(x_np), what="full workload, every row")
    assert np.max(np.abs(y.astype(np.float64).sum(axis=1) - 1.0)) <= w["cols"] * 2.0 ** -23


def _run_topk(x_np, k, with_probs=False):
    x = upload_f32(x_np)
    rows = x_np.shape[0]
    tv = Guarded((rows, k), torch.float32)
    ti = Guarded((rows, k), torch.int32)
    y = Guarded(x_np.shape, torch.float32) if with_probs else None
    lib = osfa.load_library()
    st = lib.online_softmax_topk_rows(x.data_ptr(), y.t.data_ptr() if y else None, tv.t.data_ptr(),
                                      ti.t.data_ptr(), rows, x_np.shape[1], k,
                                      torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.attn_last_error()
    torch.cuda.synchronize()
    tv.check()
    ti.check()
    if y:
        y.check()
    return tv.t.cpu().numpy(), ti.t.cpu().numpy(), (y.t.cpu().numpy() if y else None)


@pytest.mark.parametrize("rows,cols,k", [
    (9, 5, 5), (16, 100, 1), (16, 1000, 5), (8, 25000, 5), (4, 3001, 16), (5, 64, 16),
    (3, 257, 7), (2, 1, 1), (6, 70001, 3), (1, 17, 2),
])
def test_topk_parity(rows, cols, k):
    print(f"topk rows={rows} cols={cols} k={k}", flush=True)
    x = softmax_rows_inputs(rows, cols, seed=rows + cols + k)
    tv, ti, _ = _run_topk(x, k)
    rv, ri = topk_ref(x, k)
    assert np.array_equal(ti, ri), "top-k indices differ"
    assert_f32_rel(tv, rv, what="top-k values")


@pytest.mark.parametrize("order", ["ascending", "descending", "plateau", "random"])
@pytest.mark.parametrize("cols,k", [(5000, 5), (2051, 16), (777, 3)])
def test_topk_structured_rows(order, cols, k):
    """Rows whose order stresses the candidate handling: ascending (every element beats the running
    threshold, so every chunk fills the candidate queue), descending (only the first chunk offers any),
    a plateau of equal maxima spread over the row, and random; aligned and unaligned row lengths."""
    rng = np.random.default_rng(cols + k)
    rows = 6
    if order == "ascending":
        x = np.tile(np.linspace(-5.0, 5.0, cols, dtype=np.float32), (rows, 1))
    elif order == "descending":
        x = np.tile(np.linspace(5.0, -5.0, cols, dtype=np.float32), (rows, 1))
    elif order == "plateau":
        x = rng.normal(0.0, 1.0, (rows, cols)).astype(np.float32)
        x[:, rng.choice(cols, size=min(cols, 3 * k), replace=False)] = 9.0
    else:
        x = rng.normal(0.0, 4.0, (rows, cols)).astype(np.float32)
    print(f"topk structured {order} cols={cols} k={k}", flush=True)
    tv, ti, _ = _run_topk(x, k)
    rv, ri = topk_ref(x, k)
    assert np.array_equal(ti, ri), "top-k indices differ"
    assert_f32_rel(tv, rv, what=f"top-k values ({order})")


def test_topk_ties_take_lower_index():
    rng = np.random.default_rng(5)
    x = rng.integers(-3, 4, size=(32, 3000)).astype(np.float32)  # massive ties
    tv, ti, _ = _run_topk(x, 16)
    rv, ri = topk_ref(x, 16)
    assert np.array_equal(ti, ri)
    assert_f32_rel(tv, rv, what="ties")
    x = np.zeros((4, 600), np.float32)
    tv, ti, _ = _run_topk(x, 5)
    assert np.array_equal(ti, np.tile(np.arange(5), (4, 1)))


def test_topk_with_full_probs():
    x = softmax_rows_inputs(6, 25000, seed=77)
    tv, ti, y = _run_topk(x, 5, with_probs=True)
    assert_f32_rel(y, softmax_ref(x), what="topk y")
    assert np.array_equal(ti, topk_ref(x, 5)[1])


def test_topk_full_workload():
    w = WORKLOADS["softmax_top5_1024x25000"]
    x = softmax_rows_inputs(w["rows"], w["cols"], seed=w["seed"], sigma=w["sigma"])
    print("topk full 1024x25000", flush=True)
    tv, ti, _ = _run_topk(x, w["k"])
    rv, ri = topk_ref(x, w["k"])
    assert np.array_equal(ti, ri)
    assert_f32_rel(tv, rv, what="full top-5")
