"""Plain CPU oracle of expert load statistics and redundant-expert placement.

TEST INFRASTRUCTURE. Only tests/ may import this module. The library's planner
(libmoe.so, moe_eplb_plan) never calls it and shares no code with it.

What it computes follows the infra guide "Data parallelism and expert
parallelism", section 5 (uneven load: the busiest GPU sets the pace):

  imbalance        section 5.1: the busiest GPU's load divided by the mean
                   load over GPUs (1 means perfectly balanced); its inverse,
                   mean / max, is the balancedness of section 5.3.
  contiguous       section 5.2: the default placement, experts dealt to GPUs
                   in contiguous id ranges of E / EP experts each.
  balanced         section 5.2: re-placement from the observed loads. First
                   each redundant slot goes, one at a time, to the expert with
                   the largest load per replica (a token stream split evenly
                   across its replicas); then the replicas, heaviest first,
                   are put one by one on the GPU with the least load so far
                   among those that still have a free slot; every GPU has
                   (E + R) / EP slots.
  simulate_counts  section 5.2: the synthetic workload the section measures:
                   power-law popularity 1 / (rank)^s over E experts with the
                   ranks shuffled, each of T tokens drawing k distinct experts
                   with probability proportional to popularity.

Ties (not specified by the section) go to the lowest expert id and the lowest
GPU index; equal replica loads keep their order of creation (expert id, then
replica), which is what a stable descending sort gives.
"""
import random


def simulate_counts(seed=0, n_experts=256, top_k=8, tokens=4096, skew=0.4):
    """Per-expert token counts of the section 5.2 workload (Python's Mersenne
    Twister, seeded; the popularity list is shuffled once, then each token
    draws experts one at a time, redrawing repeats, until it has top_k)."""
    rng = random.Random(seed)
    popularity = [1.0 / (rank + 1) ** skew for rank in range(n_experts)]
    rng.shuffle(popularity)
    experts = range(n_experts)
    counts = [0] * n_experts
    for _ in range(tokens):
        picked = set()
        while len(picked) < top_k:
            picked.add(rng.choices(experts, weights=popularity)[0])
        for e in picked:
            counts[e] += 1
    return counts


def imbalance(loads):
    """max / mean of per-GPU loads (no load at all counts as balanced, 1)."""
    total = sum(loads)
    return max(loads) / (total / len(loads)) if total > 0 else 1.0


def contiguous_loads(counts, ep):
    """Per-GPU loads when GPU g holds experts [g E/EP, (g+1) E/EP)."""
    per = len(counts) // ep
    return [sum(counts[g * per:(g + 1) * per]) for g in range(ep)]


def replicate(counts, redundant):
    """Replica count per expert after giving out `redundant` extra replicas,
    each to the expert with the largest load per replica (lowest id on ties)."""
    replicas = [1] * len(counts)
    for _ in range(redundant):
        best = 0
        for e in range(1, len(counts)):
            if counts[e] * replicas[best] > counts[best] * replicas[e]:
                best = e
        replicas[best] += 1
    return replicas


def balanced_placement(counts, ep, redundant):
    """Greedy placement of section 5.2.

    Returns (replicas, slots, loads): replicas[e] is the replica count of
    expert e; slots[g] lists the experts whose replicas GPU g holds, in the
    order they were placed; loads[g] is GPU g's load (sum of counts[e] /
    replicas[e] over its replicas)."""
    n = len(counts)
    if (n + redundant) % ep:
        raise ValueError("E + R must divide evenly over the GPUs")
    per_gpu = (n + redundant) // ep
    replicas = replicate(counts, redundant)
    pieces = [(counts[e] / replicas[e], e) for e in range(n) for _ in range(replicas[e])]
    order = sorted(range(len(pieces)), key=lambda i: -pieces[i][0])      # stable: creation order on ties
    loads = [0.0] * ep
    slots = [[] for _ in range(ep)]
    for i in order:
        load, e = pieces[i]
        g = min((g for g in range(ep) if len(slots[g]) < per_gpu), key=lambda g: loads[g])
        loads[g] += load
        slots[g].append(e)
    return replicas, slots, loads
