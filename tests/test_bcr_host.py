"""CPU checks of the BCR chunk budget in the C ABI (a host-only call) against
the oracle and the budget column of BCR's Table 8."""
import itertools
import json
import os

import pytest

import cross_context_kv_amd.kvfix as kv
from oracle import kvref as K

pytestmark = pytest.mark.skipif(not os.path.exists(kv._LIB_PATH),
                                reason="libkvfix.so not built (run the build first)")

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_chunk_budget_printed_budget_column():
    g = json.load(open(os.path.join(GOLDEN, "bcr_table8_budget.json")))
    M, (num, den) = g["segment_rows"], g["rho"]
    for unit, pct in zip(g["units"], g["budget_percent_printed"]):
        c = kv.kvfix_chunk_budget(M, unit, num, den, kv.BUDGET_AT_LEAST_ONE)
        assert round(100.0 * c * unit / M, g["printed_decimals"]) == pct


def test_chunk_budget_matches_oracle_on_a_grid():
    rules = {kv.BUDGET_SKIP: "alg1", kv.BUDGET_AT_LEAST_ONE: "table8"}
    for M, B, (num, den), rule in itertools.product(
            [0, 1, 63, 64, 127, 128, 191, 192, 319, 320, 1000, 2048, 2240, 4096, 32768, 100003],
            [1, 16, 64, 100, 1024],
            [(0, 1), (1, 20), (1, 10), (3, 20), (1, 5), (1, 4), (1, 2), (2, 3), (1, 1)],
            rules):
        assert kv.kvfix_chunk_budget(M, B, num, den, rule) == K.chunk_budget(
            M, B, num, den, rules[rule]), (M, B, num, den, rule)


def test_chunk_budget_rejects_bad_arguments():
    L = kv.lib()
    assert L.kvfix_chunk_budget(100, 0, 1, 5, 0) == -1          # chunk < 1
    assert L.kvfix_chunk_budget(-1, 64, 1, 5, 0) == -1          # negative M
    assert L.kvfix_chunk_budget(100, 64, 6, 5, 0) == -1         # rho > 1
    assert L.kvfix_chunk_budget(100, 64, 1, 0, 0) == -1         # rho_den < 1
    assert L.kvfix_chunk_budget(100, 64, 1, 5, 7) == -1         # unknown rule
    assert L.kvfix_chunk_budget(100, 64, 1, (1 << 30) + 1, 0) == -1


def test_layout_calls_validate_before_launch():
    L = kv.lib()
    P = None
    # negative sizes, b > n, NaN tau
    assert L.kvfix_chunk_means(P, -1, 10, 4, P, P) == 1
    assert L.kvfix_chunk_means(P, 1, 10, 0, P, P) == 1
    assert L.kvfix_expand_chunks(P, 1, -1, 10, 4, P, P, P, P) == 1
    assert L.kvfix_select_grow(P, 1, 10, 11, 0.25, P, P, P) == 1
    assert L.kvfix_select_grow(P, 1, 10, 5, float("nan"), P, P, P) == 1
    # null pointers with work to do
    assert L.kvfix_chunk_means(P, 1, 10, 4, P, P) == 1
    assert L.kvfix_expand_chunks(P, 1, 2, 10, 4, P, P, P, P) == 1
    assert L.kvfix_select_grow(P, 1, 10, 5, 0.25, P, P, P) == 1
    # empty work is a no-op
    assert L.kvfix_chunk_means(P, 0, 10, 4, P, P) == 0
    assert L.kvfix_select_grow(P, 0, 10, 5, 0.25, P, P, P) == 0
