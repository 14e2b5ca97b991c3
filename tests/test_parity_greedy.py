"""Greedy-mode parity of the HIP path with the fp64 oracle (GPU): bit-exact."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

from tests.gpu_util import check_greedy_parity, run_greedy  # noqa: E402
from workloads import GREEDY, generate, to_bf16_bits  # noqa: E402


@pytest.mark.parametrize("B,K,V,dtype", [(4, 4, 1000, "f32"), (5, 3, 4099, "f32"),
                                         (6, 8, 16400, "bf16"), (3, 64, 777, "bf16"),
                                         (2, 1, 70000, "f32")])
def test_small_shapes(B, K, V, dtype):
    w = GREEDY.replace(name=f"greedy_B{B}_K{K}_V{V}_{dtype}", B=B, K=K, V=V, dtype=dtype,
                       seed=4000 + B + K + V)
    inp = generate(w)
    check_greedy_parity(w.name, inp.target, dtype, inp.tokens)


def test_ties_take_the_lowest_index_and_partial_matches():
    rng = np.random.default_rng(5)
    B, K, V = 16, 6, 9000
    T = rng.integers(-2, 3, size=(B, K + 1, V)).astype(np.float32)  # heavy ties
    T[:, :, 4321] = 7.0  # a maximum tied at two places in some rows
    T[::2, :, 8999] = 7.0
    T[3, 2, :] = -np.inf  # a row of -inf only: argmax 0
    x = np.argmax(T[:, :K], axis=2).astype(np.int32)
    x[1::3, 2] = 5  # break the match at slot 2 for some requests
    check_greedy_parity("ties", T, "f32", x)
    bits = np.ascontiguousarray(to_bf16_bits(T))
    check_greedy_parity("ties_bf16", bits, "bf16", x)


def test_ragged_num_draft():
    w = GREEDY.replace(name="greedy_ragged", B=11, K=7, V=12000, ragged=True, seed=91)
    inp = generate(w)
    check_greedy_parity(w.name, inp.target, "f32", inp.tokens, inp.num_draft)
    acc, com = run_greedy(inp.target, inp.tokens, inp.num_draft)
    assert np.all(acc <= inp.num_draft)


def test_full_greedy_B512_K8_f32():
    inp = generate(GREEDY)
    check_greedy_parity(GREEDY.name, inp.target, "f32", inp.tokens)
