"""Pins of the load-statistics / placement oracle (oracle/eplb_oracle.py).

The infra guide's section 5.2 prints the outcome of its simulated workload;
the oracle regenerates that workload and must reproduce every printed number.
Invariants and a brute-force check on tiny cases pin the placement itself."""
import itertools
import json
import os

import pytest

from oracle import eplb_oracle as P

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "p5_eplb_table.json")))


@pytest.fixture(scope="module")
def counts():
    s = GOLD["setup"]
    return P.simulate_counts(s["seed"], s["experts"], s["top_k"], s["tokens"], s["skew"])


def test_workload_matches_printed_extremes(counts):
    g = GOLD["printed"]
    assert max(counts) == g["hottest"] and min(counts) == g["coldest"]
    assert sum(counts) / len(counts) == g["average"]
    assert sum(counts) == GOLD["setup"]["tokens"] * GOLD["setup"]["top_k"]


@pytest.mark.parametrize("row", GOLD["printed"]["rows"], ids=lambda r: f"ep{r['ep']}")
def test_printed_imbalance_table(counts, row):
    ep = row["ep"]
    assert len(counts) // ep == row["experts_per_gpu"]
    assert round(P.imbalance(P.contiguous_loads(counts, ep)), 2) == row["contiguous"]
    _, _, loads0 = P.balanced_placement(counts, ep, 0)
    assert round(P.imbalance(loads0), 2) == row["rebalance"]
    _, _, loads1 = P.balanced_placement(counts, ep, ep)
    assert round(P.imbalance(loads1), 2) == row["redundant_one_per_gpu"]


@pytest.mark.parametrize("ep,red", [(8, 0), (8, 8), (32, 32), (64, 0), (256, 256), (16, 48)])
def test_placement_invariants(counts, ep, red):
    replicas, slots, loads = P.balanced_placement(counts, ep, red)
    n = len(counts)
    assert sum(replicas) == n + red and min(replicas) >= 1
    assert all(len(s) == (n + red) // ep for s in slots)
    held = [0] * n
    for s in slots:
        for e in s:
            held[e] += 1
    assert held == replicas
    # every token's share is somewhere: loads sum to the total count
    assert abs(sum(loads) - sum(counts)) < 1e-6 * sum(counts)
    for g, s in enumerate(slots):
        assert abs(loads[g] - sum(counts[e] / replicas[e] for e in s)) < 1e-9 * max(1.0, loads[g])


def test_replication_goes_to_largest_share():
    # closed form: with equal counts every expert gets one extra replica before
    # any gets two, lowest ids first
    counts = [10] * 6
    assert P.replicate(counts, 4) == [2, 2, 2, 2, 1, 1]
    assert P.replicate([7, 100, 3], 3) == [1, 4, 1]          # 100/4 = 25 > 7
    assert P.replicate([30, 100, 3], 3) == [1, 4, 1]         # 100/3 = 33.3 > 30 takes the third
    assert P.replicate([40, 100, 3], 3) == [2, 3, 1]         # 40 > 100/3 takes the third


def test_greedy_matches_its_own_definition_on_tiny_cases():
    """Brute force: replay the greedy rule by hand-written enumeration order on
    tiny inputs, and check the result never exceeds the contiguous placement's
    maximum when no replicas are added and the slot count is 1 per GPU."""
    for counts in itertools.product([0, 1, 3, 5], repeat=4):
        counts = list(counts)
        if sum(counts) == 0:
            continue
        _, slots, loads = P.balanced_placement(counts, 4, 0)
        assert sorted(e for s in slots for e in s) == [0, 1, 2, 3]
        assert sorted(loads) == sorted(float(c) for c in counts)
        _, slots, loads = P.balanced_placement(counts, 2, 0)
        # longest-processing-time with two bins of two: heaviest two split
        top = sorted(counts, reverse=True)
        assert max(loads) == max(top[0] + top[3], top[1] + top[2])
