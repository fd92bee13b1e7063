"""The paged and multi-token call forms at batches above 64 sequences (GPU
parity against the fp64 oracle): past 64 the kernels read the lengths while
walking the schedule instead of keeping them in registers, and the schedule's
prefix sums run over several 64-lane chunks. Same checks as the random-form
cases: outputs to the decode parity bar, appended rows, pools and lengths bit
for bit."""
import pytest

from test_random_forms_gpu import test_random_form as _run_form

pytestmark = pytest.mark.gpu

CASES = [
    # (id, form, dtype, b, h, g, d, n, pre-append lengths, block size)
    (0, "paged_step", "bf16", 100, 16, 4, 128, 1, [(13 * s) % 90 for s in range(100)], 32),
    (1, "paged_attention", "f32", 200, 8, 2, 64, 1, [(7 * s) % 70 for s in range(200)], 64),
    (2, "multi", "bf16", 100, 16, 8, 128, 3, [(11 * s) % 80 for s in range(100)], 32),
    (3, "multi", "f32", 80, 8, 2, 32, 4, [(5 * s) % 60 for s in range(80)], 32),
    (4, "multi_paged", "bf16", 130, 32, 4, 128, 2, [(17 * s) % 100 for s in range(130)], 32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[1]}-b{c[3]}")
def test_large_batch_form(gpu_lib, oracle_mod, case):
    _run_form(gpu_lib, oracle_mod, (900 + case[0],) + tuple(case[1:]))
