"""The CPU oracle against worked examples, library special cases, brute force
and invariants (no GPU)."""
import numpy as np
import pytest

from tests import oracle_pins as P


def test_golden_worked_examples(orc):
    P.check_golden(orc)


def test_single_value_blocks_all_bf16(orc):
    P.check_single_value_blocks(orc)


def test_pair_blocks_every_scale(orc):
    # every bf16 value against every reachable scale byte (about 8.4M pairs)
    P.check_pair_blocks(orc)


def test_float32_input_against_torch_and_ties(orc):
    P.check_f32_input(orc)


def test_gemm_against_numpy_and_closed_forms(orc):
    P.check_gemm(orc)


def test_dequant_decode_tables(orc):
    P.check_dequant_tables(orc)


def test_round_bf16_against_torch(orc):
    P.check_round_bf16(orc)


def test_rmsnorm_closed_forms(orc):
    P.check_rmsnorm(orc)


def test_rmsnorm_over_the_whole_bf16_range(orc):
    P.check_rmsnorm_range(orc)


@pytest.fixture(scope="module")
def xs():
    return P.random_tensors()


def test_error_bound(orc, xs):
    P.check_error_bound(orc, xs)


def test_idempotent(orc, xs):
    P.check_idempotent(orc, xs)


def test_sign_symmetry(orc, xs):
    P.check_sign_symmetry(orc, xs)


def test_power_of_two_shift(orc, xs):
    P.check_pow2_shift(orc, xs)


def test_columnwise_is_rowwise_of_transpose(orc, xs):
    P.check_col_is_row_of_transpose(orc, xs)


def test_transposed_columnwise_is_rowwise_of_transpose(orc, xs):
    P.check_col_t_is_row_of_transpose(orc, xs)


def test_row_and_column_planes_agree(orc, xs):
    P.check_row_col_agree(orc, xs)


def test_rejects_partial_blocks(orc):
    with pytest.raises(ValueError):
        orc.quantize_rowwise(np.zeros((4, 48), np.uint16))
    with pytest.raises(ValueError):
        orc.quantize_colwise(np.zeros((48, 4), np.uint16))


def test_threads_do_not_change_results(orc, xs):
    x = np.concatenate(xs)
    orc.set_threads(1)
    a = orc.quantize_rowwise(x), orc.quantize_colwise(x)
    orc.set_threads(4)
    b = orc.quantize_rowwise(x), orc.quantize_colwise(x)
    for (qa, sa), (qb, sb) in zip(a, b):
        assert (qa == qb).all() and (sa == sb).all()
