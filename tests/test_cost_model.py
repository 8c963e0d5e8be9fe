"""The cost accounting used for throughput reporting, pinned to the worked
numbers printed on the Shampoo blog page ("Kronecker factorization",
"The cost dial")."""

import os

import pytest

from workloads import cost

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "cost_model.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        k, v, tol = line.split()
        out[k] = (float(v), float(tol))
    return out


def test_page_numbers():
    g = _golden()

    def close(key, value):
        ref, tol = g[key]
        assert abs(value - ref) <= tol * abs(ref), (key, value, ref)

    close("factor_floats_1024", cost.factor_floats(1024, 1024))
    close("factor_megabytes_1024", cost.factor_floats(1024, 1024) * 4 / 1e6)
    close("overhead_4096_B1e6", cost.page_overhead_ratio(4096, 4096, 1e6))
    close("overhead_2048_B4096", cost.page_overhead_ratio(2048, 2048, 4096))
    close("accumulator_floats_4096x11008", cost.factor_floats(4096, 11008))
    close("adam_floats_4096x11008", 2 * 4096 * 11008)


@pytest.mark.parametrize("m,n", [(64, 32), (1024, 1024), (512, 1024)])
def test_page_step_cost_is_4mn_m_plus_n(m, n):
    assert cost.page_step_flops(m, n) == 4 * m * n * (m + n)
    # overhead ratio is the step cost over 6 B m n
    B = 4096
    assert abs(cost.page_step_flops(m, n) / (6 * B * m * n) - cost.page_overhead_ratio(m, n, B)) < 1e-15


def test_block_step_accounting_components():
    # statistics + sandwich terms reduce to the page's per-step 4mn(m+n) plus
    # the extra two products of the eigen form (2 m^2 n + 2 m n^2)
    m, n = 96, 40
    stats_g = 2 * m * m * n + 2 * n * n * m
    sandwich = cost.precondition_side_flops(m, n) + cost.precondition_side_flops(n, m)
    assert stats_g + sandwich == cost.page_step_flops(m, n) + 2 * m * m * n + 2 * m * n * n
    f1 = cost.block_step_flops(m, n, 1, 1)
    f10 = cost.block_step_flops(m, n, 1, 10)
    assert f10 > f1
    extra = cost.block_step_flops(m, n, 1, 1, cached_root=False) - f1
    assert abs(extra - (cost.bjorck_flops(m, 1) + cost.bjorck_flops(n, 1))) < 1e-6 * extra
