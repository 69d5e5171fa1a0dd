"""Pins of the oracle's standalone grouped GEMM (LightMoE "Grouped GEMM": expert-major
rows, B as [E, N, K], m_indptr offsets): a scalar triple loop on small inputs, zero-row
experts, the down projection of the expert MLP written as a grouped GEMM, and MXFP8
operands that the format holds exactly."""
import numpy as np

import oracle.moe_oracle as orc


def _bf16_values(rng, shape, scale=1.0):
    return orc.bf16_round(scale * rng.standard_normal(shape))


def test_matches_scalar_loops():
    rng = np.random.default_rng(0)
    M, N, K = 11, 5, 7
    m_indptr = np.array([0, 3, 3, 9, 11], dtype=np.int32)     # expert 1 has no rows
    A = _bf16_values(rng, (M, K))
    B = _bf16_values(rng, (4, N, K))
    C = orc.grouped_gemm(A, B, m_indptr, exact=True)
    for e in range(4):
        for r in range(m_indptr[e], m_indptr[e + 1]):
            for n in range(N):
                acc = 0.0
                for k in range(K):
                    acc += A[r, k] * B[e, n, k]
                assert abs(C[r, n] - acc) <= 1e-12 * (1 + abs(acc))
    # one rounding of the exact sum
    assert np.array_equal(orc.grouped_gemm(A, B, m_indptr), orc.bf16_round(C))


def test_zero_row_experts_and_rows_outside():
    rng = np.random.default_rng(1)
    A = _bf16_values(rng, (6, 8))
    B = _bf16_values(rng, (3, 4, 8))
    full = orc.grouped_gemm(A, B, np.array([0, 0, 6, 6], np.int32))
    assert np.array_equal(full, orc.bf16_round(A @ B[1].T))
    part = orc.grouped_gemm(A, B, np.array([0, 2, 2, 4], np.int32))      # rows 4-5 belong to no expert
    assert np.all(part[4:] == 0)
    assert np.array_equal(part[:2], orc.bf16_round(A[:2] @ B[0].T))


def test_down_projection_of_the_expert_mlp():
    # O of the expert MLP is the grouped GEMM of h with W_down packed as [E, H, I]
    rng = np.random.default_rng(2)
    T, H, I, E, k = 40, 64, 32, 5, 2
    X = orc.bf16_round(rng.standard_normal((T, H)))
    Wg, Wu = (orc.bf16_round(rng.standard_normal((E, H, I)) / 8) for _ in range(2))
    Wd = orc.bf16_round(rng.standard_normal((E, I, H)) / 6)
    idx, _ = orc.route(rng.standard_normal((T, E)).astype(np.float32), k)
    off, row_token, _, _ = orc.dispatch(idx, E)
    h, O = orc.expert_mlp(X, row_token, off, Wg, Wu, Wd)
    assert np.array_equal(orc.grouped_gemm(h, np.transpose(Wd, (0, 2, 1)), off), O)


def test_mxfp8_exact_operands():
    # operands already on the MXFP8 grid (one scale per block, codes of E4M3): the quantised
    # product equals the plain one
    rng = np.random.default_rng(3)
    M, N, K, E = 9, 6, 64, 2
    A = np.ldexp(rng.integers(-8, 9, (M, K)).astype(np.float64), -3)
    B = np.ldexp(rng.integers(-8, 9, (E, N, K)).astype(np.float64), -4)
    off = np.array([0, 4, 9], np.int32)
    assert np.array_equal(orc.grouped_gemm(A, B, off, mxfp8=True), orc.grouped_gemm(A, B, off))
