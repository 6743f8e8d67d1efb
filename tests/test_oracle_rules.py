"""Argument rules of the oracle against the ranges the pages state
(tests/golden/page_facts.json holds each value with its citation)."""
import json
import os

import pytest

FACTS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")))
KMAX = FACTS["topk_max"]["value"]
EMAX = FACTS["experts_max"]["value"]
HMUL = FACTS["hidden_multiple"]["value"]


def test_capacity_bound(orc):
    assert orc.recv_capacity_bound(4096, 8, 256, 1) == 32768
    assert orc.recv_capacity_bound(32768, 16, 512, 128) == 32768 * 16 + 512 * 127
    assert orc.recv_capacity_bound(0, 4, 8, 4) == 24
    assert orc.recv_capacity_bound(-1, 4, 8, 4) == -1


@pytest.mark.parametrize("T,K,E,R,a,code", [
    (8, 1, 4, 2, 1, 0), (8, KMAX, 4, 2, 1, 0), (8, 0, 4, 2, 1, -1), (8, KMAX + 1, 4, 2, 1, -1),
    (8, 2, EMAX, 8, 1, 0), (8, 2, EMAX + 1, 1, 1, -1), (8, 2, 0, 1, 1, -1),
    (8, 2, 6, 4, 1, -1), (8, 2, 6, 3, 1, 0), (8, 2, 6, 7, 1, -1), (8, 2, 6, 0, 1, -1),
    (8, 2, 6, 3, 0, -1), (-1, 2, 6, 3, 1, -1), (0, 2, 6, 3, 5, 0),
])
def test_layout_rules(orc, T, K, E, R, a, code):
    cap = max(orc.recv_capacity_bound(T, K, max(E, 1), max(a, 1)), 0)
    assert orc.check_layout_args(T, K, E, R, a, cap) == code


def test_layout_capacity_rule(orc):
    bound = orc.recv_capacity_bound(100, 4, 16, 8)
    assert orc.check_layout_args(100, 4, 16, 4, 8, bound) == 0
    assert orc.check_layout_args(100, 4, 16, 4, 8, bound + 1000) == 0
    assert orc.check_layout_args(100, 4, 16, 4, 8, bound - 1) == -2
    assert orc.check_layout_args(2 ** 28, 16, 16, 4, 8, 2 ** 31) == -1   # rows exceed int32


@pytest.mark.parametrize("H,q,code", [
    (HMUL, 0, 0), (7168, 0, 0), (16384, 4, 0), (HMUL // 2, 0, -1), (HMUL + 16, 0, -1),
    (16384 + HMUL, 0, -1), (0, 0, -1), (1024, 1, -1), (1024, 3, -1), (1024, 2, 0), (1024, 4, 0),
    (1024, -1, -1), (1024, 5, -1),
])
def test_rows_rules(orc, H, q, code):
    assert orc.check_rows_args(16, H, 4, 1000, q) == code


def test_rows_rules_topk(orc):
    assert orc.check_rows_args(16, 64, KMAX, 1000, 0) == 0
    assert orc.check_rows_args(16, 64, KMAX + 1, 1000, 0) == -1
    assert orc.check_rows_args(16, 64, 0, 1000, 0) == -1
