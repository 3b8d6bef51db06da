"""Runs the oracle's pins against one oracle build and reports whether they
all hold.  Used by test_oracle_mutants.py to show that deliberately altered
copies of the oracle (planted mistakes, on the CPU only) are caught.

    python -m tests.pin_runner /path/to/liboracle_variant.so   -> exit 0 if every pin holds
"""
import sys

from oracle import oracle
from tests import test_oracle_attention as A
from tests import test_oracle_index as I
from tests import test_oracle_joint_text as J
from tests import test_oracle_perm as P
from tests import test_oracle_ragged as R
from tests import test_oracle_window_options as W
from tests.conftest import read_golden


def checks():
    yield lambda: P.test_golden_small("perm_small.txt")
    yield lambda: P.test_golden_small("perm_asym.txt")
    yield lambda: P.test_bijection_and_tile_contiguity("asym")
    yield lambda: P.test_golden_small("perm_ragged.txt")
    for grid, tile in P.RAGGED:
        yield (lambda a, b: lambda: P.test_ragged_tiles_are_contiguous_and_ordered(a, b))(grid, tile)
    for row in read_golden("window_axis.txt"):
        yield (lambda r: lambda: I.test_window_axis_golden(r))(row)
    yield lambda: I.test_attendee_counts_720p_golden()
    yield lambda: I.test_tiny_fp32_workload_is_dense()
    for case in range(4):
        yield (lambda c: lambda: I.test_list_invariants(c))(case)
        yield (lambda c: lambda: I.test_lists_match_enumerated_token_mask(c))(case)
    yield lambda: I.test_interior_tiles_get_chebyshev_ball()
    yield lambda: I.test_zero_offsets_equal_no_offsets_and_large_offsets_saturate()
    yield lambda: A.test_constant_values_and_zero_queries()
    yield lambda: A.test_whole_grid_window_is_full_attention()
    yield lambda: A.test_unit_window_is_per_tile_attention()
    for seed in (1, 2):
        for off in (False, True):
            yield (lambda s, o: lambda: A.test_forward_backward_match_torch_dense(s, o))(seed, off)
    yield lambda: A.test_lse_bounds()
    yield lambda: A.test_gradient_identities()
    yield lambda: A.test_backward_matches_finite_differences()
    for row in read_golden("window_axis_truncate.txt"):
        yield (lambda r: lambda: W.test_truncate_axis_golden(r))(row)
    for case in range(len(W.CASES)):
        yield (lambda c: lambda: W.test_truncate_lists_match_enumeration_and_transpose(c))(case)
    yield lambda: W.test_truncate_holds_clamped_centre_and_never_exceeds_window()
    yield lambda: W.test_truncate_interior_equals_shift_and_border_is_smaller()
    yield lambda: W.test_truncate_mirror_symmetry_and_wide_window()
    for border in ("shift", "truncate"):
        yield (lambda b: lambda: W.test_head_offsets_reduce_to_shared_and_single_head(b))(border)
        yield (lambda b: lambda: W.test_attention_options_match_torch_dense(b))(border)
        for nt in (1, 7):
            yield (lambda b, n: lambda: J.test_joint_matches_torch_dense(b, n))(border, nt)
    yield lambda: J.test_text_rows_are_unmasked_attention()
    yield lambda: J.test_video_rows_merge_window_and_text_keys()
    yield lambda: J.test_whole_grid_window_with_text_is_full_attention()
    yield lambda: J.test_zero_text_tokens_equal_video_only()
    yield lambda: J.test_text_permutation_equivariance()
    for case in range(len(R.CASES)):
        yield (lambda c: lambda: R.test_ragged_matches_torch_dense(c))(case)
    for case in (0, 1):
        yield (lambda c: lambda: R.test_ragged_equals_padded_grid_with_padding_masked(c))(case)
    yield lambda: R.test_ragged_index_is_that_of_the_tile_grid()
    yield lambda: R.test_ragged_whole_window_is_full_attention()


def main(path):
    oracle.use(path)
    for i, check in enumerate(checks()):
        try:
            check()
        except (AssertionError, ValueError) as e:
            print("pin %d failed: %s" % (i, str(e).splitlines()[0][:200] if str(e) else type(e).__name__))
            return 1
    print("all pins hold")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
