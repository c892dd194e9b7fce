"""The pages' worked numbers (tests/golden/pages_numbers.json) against the oracle,
the allocator fixture and the library's host-side arithmetic.

Every fixture entry carries the page title and section it restates.
"""
import json
import math
import os

import numpy as np
import pytest

import kvgen
import oracle

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_token_to_block_examples_through_the_oracle_slot_mapping():
    for case in GOLDEN["token_to_block"]:
        B = case["block_size"]
        pos = case["position"]
        # a table whose entry b holds 1000 + b: the slot names the logical block it went through
        table = (1000 + np.arange(64, dtype=np.int32))[None, :]
        slot = oracle.slot_mapping(table, B, 2000, np.array([0]), np.array([pos]), np.array([1]))[0]
        logical = slot // B - 1000
        assert logical == case["expected_logical_block"]
        if "expected_block_first_token" in case:
            assert logical * B == case["expected_block_first_token"]
            assert (logical + 1) * B - 1 == case["expected_block_last_token"]


def test_slot_formula_examples():
    B = GOLDEN["slot_formula"]["block_size"]
    for c in GOLDEN["slot_formula"]["cases"]:
        n = c["physical_block"] + 1
        table = np.full((1, 1), c["physical_block"], dtype=np.int32)
        s = oracle.slot_mapping(table, B, n, np.array([0]), np.array([c["offset"]]), np.array([1]))[0]
        assert s == c["expected_slot"]


def test_prompt_block_counts_through_the_allocator():
    for c in GOLDEN["prompt_blocks"]:
        B = c["block_size"]
        a = kvgen.BlockAllocator(4096)
        if "expected_blocks" in c:
            # admission allocates ceil(tokens / B) blocks for the prompt
            table = [a.alloc() for _ in range(-(-c["tokens"] // B))]
            assert len(table) == c["expected_blocks"]
        else:
            # prefix sharing covers whole blocks from token 0 only
            assert (c["tokens"] // B) == c["expected_shared_full_blocks"]
            assert (c["tokens"] // B) * B == c["expected_shared_tokens"]


def test_expected_waste_and_gather_iterations():
    g = GOLDEN["expected_waste_300"]
    n = g["tokens"]
    for row in g["rows"]:
        B = row["block_size"]
        # mean waste over uniformly distributed lengths: average of (ceil(L/B)*B - L) over one period
        waste = np.mean([(-(-L // B)) * B - L for L in range(n, n + B)])
        assert waste == pytest.approx(row["expected_waste_tokens"])
        assert round(100 * waste / n, 1) == row["expected_pct"]
        if "expected_gather_iters" in row:
            assert -(-n // B) == row["expected_gather_iters"]


def test_fleet_waste():
    f = GOLDEN["fleet_waste"]
    B = f["block_size"]
    per_seq = np.mean([(-(-L // B)) * B - L for L in range(1, 1 + B)])
    assert f["sequences"] * per_seq == f["expected_total_waste_tokens"]
