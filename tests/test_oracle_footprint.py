"""Pins of oracle.footprint against the numbers the pages print (tests/golden/footprint.json)."""
import json
import math
import os

import pytest

from oracle import footprint as fp

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "footprint.json")))
KiB, MiB, GiB = 1024, 1024 ** 2, 1024 ** 3


@pytest.mark.parametrize("case", GOLD["bytes_per_token"], ids=lambda c: c["cite"][:60])
def test_bytes_per_token(case):
    got = fp.bytes_per_token(case["layers"], case["kv_heads"], case["head_dim"], case["elem_bytes"], case["tp"])
    assert got == case["expect"], case["cite"]


@pytest.mark.parametrize("case", GOLD["aggregate_kib_over_ranks"], ids=lambda c: c["cite"][:60])
def test_aggregate_over_ranks(case):
    for tp, kib in zip(case["tp"], case["expect_kib"]):
        per_rank = fp.bytes_per_token(case["layers"], case["kv_heads"], case["head_dim"], case["elem_bytes"], tp)
        assert per_rank * tp == kib * KiB


def test_trajectories_and_node_capacity():
    (case,) = GOLD["trajectory_gb"]
    m = fp.bytes_per_token(80, 8, 128, 2)
    for S, gb, count in zip(case["tokens"], case["expect_gb_1dp"], case["expect_count"]):
        assert round(S * m / 1e9, 1) == gb
        assert math.floor(case["pool_gb"] * 1e9 / (S * m)) == count


def test_bmax_480_gib():
    (case,) = GOLD["bmax_gib"]
    m = fp.bytes_per_token(80, 8, 128, 2)
    assert m == 320 * KiB
    for S, expect in zip(case["tokens"], case["expect"]):
        assert (case["pool_gib"] * GiB) // (S * m) == expect


def test_napkin_0_3_block_sizing():
    c = GOLD["napkin_0_3"]
    for B, expect in c["block_bytes"].items():
        assert fp.bytes_per_block(c["layers"], c["kv_heads_per_gpu"], c["head_dim"], c["elem_bytes"], int(B)) == expect
    blk16 = fp.bytes_per_block(c["layers"], 1, c["head_dim"], c["elem_bytes"], 16)
    assert (c["pool_kib"] * KiB) // blk16 == c["blocks_at_16"]
    assert c["blocks_at_16"] * 16 == c["tokens_at_16"]
    m_gpu = fp.bytes_per_token(c["layers"], 8, c["head_dim"], c["elem_bytes"], tp=8)
    for B in ("16", "64"):
        waste = c["seqs"] * fp.expected_tail_slots(int(B)) * m_gpu
        assert waste == c["waste_kib"][B] * KiB
        assert waste == c["waste_mib"][B] * MiB
        assert round(100 * waste / (c["pool_mib"] * MiB), 2) == c["waste_pct_2dp"][B]


@pytest.mark.parametrize("case", GOLD["table_entries"], ids=lambda c: c["cite"][:60])
def test_table_entries(case):
    n = fp.blocks_for_tokens(case["tokens"], case["block_size"])
    assert n == case["expect"]
    if "entry_bytes" in case:
        assert n * case["entry_bytes"] == case["expect_bytes"]


def test_gpt2_and_7b_projection():
    g = GOLD["gpt2_cache"]
    m = fp.bytes_per_token(g["layers"], g["kv_heads"], g["head_dim"], g["elem_bytes"])
    assert m * g["tokens"] == g["expect_mib"] * MiB
    s = GOLD["seven_b"]
    m7 = fp.bytes_per_token(32, 32, 128, 2)
    assert m7 * s["tokens"] == s["expect_mib"] * MiB
    assert (s["budget_gib"] * GiB) // (m7 * s["tokens"]) == s["expect_seqs"]


@pytest.mark.parametrize("case", GOLD["expected_tail"], ids=lambda c: str(c["block_size"]))
def test_expected_tail(case):
    assert fp.expected_tail_slots(case["block_size"]) == case["expect"]


def test_expected_tail_is_mean_of_tail_slots_over_residues():
    # Closed form check: averaging Delta_tail over S mod B uniform gives (B - 1) / 2.
    for B in (1, 2, 4, 16, 64, 256):
        mean = sum(fp.tail_slots(S, B) for S in range(1, B + 1)) / B
        assert mean == fp.expected_tail_slots(B)


def test_tail_slots_fill_last_block():
    for B in (1, 3, 16, 32):
        for S in range(0, 200):
            assert fp.blocks_for_tokens(S, B) * B - S == fp.tail_slots(S, B)


def test_waste_table():
    w = GOLD["waste_table"]
    for row in w["rows"]:
        pct = 100 * fp.tail_waste_fraction(row["b"], w["mean_length"])
        assert round(pct, row["dp"]) == row["pct"], row


def test_m_block_equals_b_times_m_token():
    for (L, H, d, b) in [(80, 8, 128, 2), (12, 12, 64, 4), (32, 8, 128, 2)]:
        for B in (1, 16, 64):
            assert fp.bytes_per_block(L, H, d, b, B) == B * fp.bytes_per_token(L, H, d, b)
