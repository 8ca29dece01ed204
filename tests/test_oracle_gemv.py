"""Pins of the oracle's matrix-vector products against facts fixed by the
mathematics and by hand-derived cases.

Pages: "Binade" package page (pypi.org/project/binade), intro and "How it
works" (outputs bit-identical because the products are added in one fixed
order; the expert gather follows the matvec's order) and "Verify and
reproduce" (order-sensitive test data that exposes any change of summation
order). The order itself is this library's reading, stated in
oracle/binade_oracle.c; the cases below derive its results by hand.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_gemv_tensor_amd import synth


def bf16(values) -> np.ndarray:
    """float values that are exact in bf16 -> their bit patterns"""
    t = torch.tensor(np.asarray(values, np.float32)).to(torch.bfloat16)
    assert torch.equal(t.float(), torch.tensor(np.asarray(values, np.float32)))
    return t.view(torch.int16).numpy().view(np.uint16)


def f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def rand_bits(rows, cols, sigma, seed):
    spec = synth.TensorSpec("t", rows, cols, sigma, seed, outlier_frac=1e-3,
                            outlier_scale=20.0)
    return synth.bits(synth.normal_bf16(spec)).numpy().view(np.uint16)


# ---------------------------------------------------------------- exactness
@pytest.mark.parametrize("K", [32, 96, 2048, 3072, 4160])
def test_one_hot_input_selects_a_column(K):
    W = rand_bits(37, K, 0.02, K)
    for j in [0, 1, 31, K // 2 + 3, K - 1]:
        x = np.zeros(K, np.float32)
        x[j] = 1.0
        y = oracle.gemv_replay(W, bf16(x))
        assert np.array_equal(y, f32(W[:, j]))


def test_each_chain_step_rounds_once():
    """A chain step is one fused multiply-add: a product that falls between
    two fp32 subnormals is rounded together with the running sum. Slot 0's
    even chain takes 2^-74 * 2^-75 = 2^-149 (the smallest subnormal), then
    2^-75 * 2^-75 = 2^-150: fused, 2^-149 + 2^-150 lies halfway between
    2^-149 and 2^-148 and goes to the even 2^-148. A product rounded on its
    own would be a tie between 0 and 2^-149, go to 0, and leave 2^-149."""
    K = 32
    w = np.zeros(K, np.float32)
    x = np.zeros(K, np.float32)
    w[0], x[0] = 2.0 ** -74, 2.0 ** -75   # columns 0 and 2: the even chain, in order
    w[2], x[2] = 2.0 ** -75, 2.0 ** -75
    y = oracle.gemv_replay(bf16(w).reshape(1, K), bf16(x))
    assert y[0] == np.float32(2.0 ** -148)


@pytest.mark.parametrize("K", [64, 3072, 8192])
def test_small_integers_are_exact_in_any_order(K):
    rng = np.random.default_rng(K)
    Wi = rng.integers(-8, 9, size=(19, K))
    xi = rng.integers(-8, 9, size=K)
    y = oracle.gemv_replay(bf16(Wi), bf16(xi))
    # |partial sums| <= 64 K < 2^24: every fp32 step is exact
    assert np.array_equal(y.astype(np.int64), Wi @ xi)


@pytest.mark.parametrize("shape,sigma", [((64, 1024), 0.02), ((48, 3072), 0.02),
                                         ((16, 15360), 0.015)])
def test_replay_within_1e2_of_f64(shape, sigma):
    W = rand_bits(*shape, sigma, 1)
    x = synth.bits(synth.vector_bf16(shape[1], 2)).numpy().view(np.uint16)
    y = oracle.gemv_replay(W, x).astype(np.float64)
    y64 = oracle.gemv_f64(W, x)
    # the double sum against numpy's own float64 product (library routine)
    ref = f32(W).astype(np.float64) @ f32(x).astype(np.float64)
    assert np.allclose(y64, ref, rtol=1e-12, atol=1e-12)
    scale = np.abs(f32(W).astype(np.float64)) @ np.abs(f32(x).astype(np.float64))
    assert np.all(np.abs(y - y64) <= 1e-2 * scale)
    assert np.linalg.norm(y - y64) <= 1e-2 * np.linalg.norm(y64)


# ---------------------------------------------------------------- the order
# 2^24 + 1 is a tie in fp32 and rounds to 2^24 (even): a large term, a unit
# and the large term's negative give 0 or 1 depending on which adds happen
# first. Each case below gives the value the documented order must produce.
BIG = 4096.0  # 4096 * 4096 = 2^24


def test_order_chain_within_a_slot_is_increasing():
    K = 32
    w = np.zeros(K); x = np.zeros(K)
    w[0], x[0] = BIG, BIG        # a0 += 2^24
    w[2], x[2] = 1.0, 1.0        # a0 += 1   -> 2^24 (tie to even)
    w[4], x[4] = -BIG, BIG       # a0 -= 2^24 -> 0
    y = oracle.gemv_replay(bf16(w).reshape(1, K), bf16(x))
    assert y[0] == 0.0           # exact sum would be 1; reverse order gives 1


def test_order_even_and_odd_columns_use_two_sums():
    K = 32
    w = np.zeros(K); x = np.zeros(K)
    w[1], x[1] = BIG, BIG        # a1 = 2^24
    w[2], x[2] = 1.0, 1.0        # a0 = 1
    w[4], x[4] = -BIG, BIG       # a0 = 1 - 2^24 (exact)
    y = oracle.gemv_replay(bf16(w).reshape(1, K), bf16(x))
    assert y[0] == 1.0           # one running sum in column order gives 0


def test_order_tiles_go_to_slot_j_mod_64():
    K = 32 * 128                  # every slot owns tiles j and j + 64
    w = np.zeros(K); x = np.zeros(K)
    w[0], x[0] = BIG, BIG         # slot 0, tile 0
    w[2048 + 2], x[2048 + 2] = 1.0, 1.0    # slot 0, tile 64
    w[2048 + 4], x[2048 + 4] = -BIG, BIG   # slot 0, tile 64
    y = oracle.gemv_replay(bf16(w).reshape(1, K), bf16(x))
    assert y[0] == 0.0
    # the same terms in slots 0 and 1 (tiles 0 and 1) meet only in the tree:
    w2 = np.zeros(K); x2 = np.zeros(K)
    w2[0], x2[0] = BIG, BIG       # slot 0
    w2[32 + 2], x2[32 + 2] = 1.0, 1.0      # slot 1
    w2[32 + 4], x2[32 + 4] = -BIG, BIG     # slot 1: p1 = 1 - 2^24
    y2 = oracle.gemv_replay(bf16(w2).reshape(1, K), bf16(x2))
    assert y2[0] == 1.0           # p0 + p1 = 2^24 + (1 - 2^24) = 1


def test_order_tree_halves_slots():
    K = 32 * 64
    w = np.zeros(K); x = np.zeros(K)
    w[32 * 0], x[32 * 0] = BIG, BIG        # p0  = 2^24
    w[32 * 32], x[32 * 32] = 1.0, 1.0      # p32 = 1
    w[32 * 16], x[32 * 16] = -BIG, BIG     # p16 = -2^24
    y = oracle.gemv_replay(bf16(w).reshape(1, K), bf16(x))
    # s=32: p0 = 2^24 + 1 -> 2^24; s=16: p0 + p16 = 0. A left-to-right slot
    # sum or a neighbour-pair tree meets p0 and p16 first and gives 1.
    assert y[0] == 0.0


def test_negative_zero_products_give_positive_zero():
    K = 64
    W = bf16(-np.ones((3, K)))
    x = np.zeros(K, np.uint16)             # +0.0
    y = oracle.gemv_replay(W, x)
    assert y.view(np.uint32).tolist() == [0, 0, 0]


def test_order_sensitive_data_differs_from_a_plain_sum():
    """Powers of two spread over 40 binades: the replay is deterministic and
    a different order (numpy's float32 pairwise sum) gives other bits on some
    rows, so these data do expose an order change."""
    rng = np.random.default_rng(3)
    K = 3072
    W = np.ldexp(rng.choice([-1.0, 1.0], size=(64, K)), rng.integers(-20, 21, size=(64, K)))
    x = np.ldexp(1.0, rng.integers(-20, 21, size=K)) * rng.choice([-1.0, 1.0], size=K)
    Wb, xb = bf16(W), bf16(x)
    y = oracle.gemv_replay(Wb, xb)
    assert np.array_equal(y, oracle.gemv_replay(Wb, xb))
    other = (f32(Wb) * f32(xb)).astype(np.float32).sum(axis=1, dtype=np.float32)
    assert np.count_nonzero(y != other) > 0


# ---------------------------------------------------------------- rounding
def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    u = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, size=5000, dtype=np.uint32) << 16) | 0x8000
    u = np.concatenate([u, ties, np.array([0, 0x80000000, 0x7F800000, 0xFF800000,
                                           0x7F7FFFFF, 0x00000001, 0x7FC00000],
                                          np.uint32)])
    f = u.view(np.float32)
    got = oracle.f32_to_bf16(f)
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(f)
    assert np.array_equal(got[~nan], want[~nan])
    assert np.all((got[nan] & 0x7F80) == 0x7F80) and np.all(got[nan] & 0x7F)


# ---------------------------------------------------------------- MoE
def test_moe_rows_are_the_selected_experts_matvec():
    E, N, K = 6, 40, 96
    rng = np.random.default_rng(1)
    experts = rand_bits(E * N, K, 0.02, 4).reshape(E, N, K)
    # expert e's row r scaled so the gather index shows in the output
    idx = np.array([[0, 5, 2], [3, 3 - 3, 4]], np.int32)
    x = synth.bits(synth.vector_bf16(K, 5, count=2)).numpy().view(np.uint16)
    y = oracle.moe_replay(experts, x, idx, x_per_slot=False)
    for t in range(2):
        for j in range(3):
            assert np.array_equal(y[t * 3 + j],
                                  oracle.gemv_replay(experts[idx[t, j]], x[t]))
    xs = synth.bits(synth.vector_bf16(K, 6, count=6)).numpy().view(np.uint16)
    y2 = oracle.moe_replay(experts, xs, idx, x_per_slot=True)
    for p in range(6):
        assert np.array_equal(y2[p], oracle.gemv_replay(experts[idx.reshape(-1)[p]], xs[p]))


def test_moe_gather_picks_expert_by_index():
    E, N, K = 5, 8, 64
    experts = np.stack([bf16(np.full((N, K), float(e + 1))) for e in range(E)])
    x = bf16(np.ones((1, K)))
    idx = np.array([[4, 0, 2]], np.int32)
    y = oracle.moe_replay(experts, x, idx, x_per_slot=False)
    assert y[:, 0].tolist() == [5.0 * K, 1.0 * K, 3.0 * K]
    with pytest.raises(oracle.OracleError):
        oracle.moe_replay(experts, x, np.array([[5, 0, 0]], np.int32), False)


# ---------------------------------------------------------------- GEMM (fp64)
def test_gemm_one_hot_rows_select_columns():
    N, K = 24, 96
    W = rand_bits(N, K, 0.02, 11)
    cols = [0, 5, 31, 32, 95]
    X = np.zeros((len(cols), K), np.float32)
    for m, j in enumerate(cols):
        X[m, j] = 1.0
    Y = oracle.gemm_f64(W, bf16(X))
    assert Y.shape == (len(cols), N)
    for m, j in enumerate(cols):
        assert np.array_equal(Y[m], f32(W[:, j]).astype(np.float64))


def test_gemm_small_integers_equal_integer_matmul():
    # M, N, K all different, so a transposed operand or swapped index fails
    rng = np.random.default_rng(3)
    M, N, K = 5, 7, 64
    Xi = rng.integers(-8, 9, size=(M, K))
    Wi = rng.integers(-8, 9, size=(N, K))
    Y = oracle.gemm_f64(bf16(Wi), bf16(Xi))
    assert np.array_equal(Y.astype(np.int64), Xi @ Wi.T)


def test_gemm_rows_equal_the_matvec_definition():
    W = rand_bits(33, 160, 0.02, 12)
    X = synth.bits(synth.vector_bf16(160, 13, count=4)).numpy().view(np.uint16)
    Y = oracle.gemm_f64(W, X)
    for m in range(4):
        assert np.array_equal(Y[m], oracle.gemv_f64(W, X[m]))
    with pytest.raises(oracle.OracleError):
        oracle.gemm_f64(W[:, :0], X[:, :0])
