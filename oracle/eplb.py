"""Redundant experts and load-balanced placement (oracle side).

Sources:
* "6.4 Data parallelism and expert parallelism" (infra-guide), section 5.2: a
  CPU simulation counts tokens per expert under power-law expert popularity
  (seed 0, exponent 0.4, 256 experts, top-8, 4096 tokens) and compares the
  busiest-rank / mean-rank load for contiguous placement, for placement by
  observed load, and for placement with one redundant replica per rank.  The
  balanced placement gives each redundant slot to the expert with the highest
  load per replica, then places replicas heaviest first onto the currently
  lightest rank that still has a free slot.  Section 5.3: with redundancy a
  rank holds (experts + redundant) / EP physical experts.
* "Expert Parallel and All-to-All Backends" (aiinfrainterviews), "Load
  imbalance": redundant replicas split a hot expert's tokens.

The skewed workload's rule for one rank (8 extra replicas for the 8 hottest
local experts, tokens split round-robin) is ``hottest_replica_map``.
"""
from __future__ import annotations

import bisect
import heapq
import itertools
import random
from fractions import Fraction
from typing import List, Sequence, Tuple

import numpy as np


# ---------------------------------------------------- one rank's replicas
def hottest_replica_map(local_counts: Sequence[int], redundant: int):
    """Map for one rank holding ``num_local`` logical experts plus
    ``redundant`` extra physical experts: the ``redundant`` hottest local
    experts (more local pairs first, lower id on ties) get one extra replica
    each; physical id num_local + i is the second replica of the i-th hottest.

    Returns (l2p [num_local, 2] int32 with -1 padding, rep_count [num_local]
    int32, P)."""
    counts = [int(c) for c in local_counts]
    L = len(counts)
    if not 0 <= redundant <= L:
        raise ValueError("redundant must be in [0, num_local]")
    max_rep = 2 if redundant > 0 else 1
    l2p = np.full((L, max_rep), -1, dtype=np.int32)
    l2p[:, 0] = np.arange(L, dtype=np.int32)
    rep = np.ones(L, dtype=np.int32)
    hottest = sorted(range(L), key=lambda e: (-counts[e], e))[:redundant]
    for i, e in enumerate(hottest):
        l2p[e, 1] = L + i
        rep[e] = 2
    return l2p, rep, L + redundant


def replica_share(n: int, R: int) -> List[int]:
    """Closed form of the round-robin split: replica r of an expert with n
    pairs and R replicas receives ceil((n - r) / R) pairs."""
    return [max(0, -(-(n - r) // R)) for r in range(R)]


# ------------------------------------------------ the load simulation (5.2)
def simulate_routing(seed: int = 0, experts: int = 256, top_k: int = 8,
                     tokens: int = 4096, skew: float = 0.4):
    """Per-token expert picks under power-law popularity, and the counts.

    The model of section 5.2: expert i (before shuffling) is popular in
    proportion to 1/(i+1)^skew; the popularity list is shuffled so hot
    experts land on scattered ids; every token then draws experts one at a
    time, with probability proportional to popularity, until it holds
    ``top_k`` distinct ones.

    Sampling contract (the only part kept in step with the page's script,
    because its printed counts can be reproduced in no other way): one
    Python ``random.Random(seed)`` stream, consumed first by the shuffle and
    then by one uniform variate per draw, and a draw maps its variate u to
    the first expert whose cumulative popularity exceeds u * total -- the
    inverse-CDF lookup that ``random.choices`` performs.

    Returns (picks [tokens][top_k] with each token's experts in ascending
    id order, counts [experts])."""
    rng = random.Random(seed)
    pop = [1.0 / (i + 1) ** skew for i in range(experts)]
    rng.shuffle(pop)
    cum = list(itertools.accumulate(pop))
    total = cum[-1] + 0.0
    picks: List[List[int]] = []
    for _ in range(tokens):
        held = set()
        while len(held) < top_k:
            held.add(bisect.bisect(cum, rng.random() * total, 0,
                                   experts - 1))
        picks.append(sorted(held))
    counts = [0] * experts
    for row in picks:
        for e in row:
            counts[e] += 1
    return picks, counts


def simulate_expert_counts(seed: int = 0, experts: int = 256, top_k: int = 8,
                           tokens: int = 4096, skew: float = 0.4) -> List[int]:
    """Token counts per expert of ``simulate_routing``."""
    return simulate_routing(seed, experts, top_k, tokens, skew)[1]


def contiguous_load(counts: Sequence[int], ep: int) -> List[float]:
    """Rank loads when rank g owns experts [g*E/ep, (g+1)*E/ep)."""
    per = len(counts) // ep
    return [float(sum(counts[g * per:(g + 1) * per])) for g in range(ep)]


def plan_replicas(counts: Sequence[int], redundant: int) -> List[int]:
    """Replica count per expert (section 5.2's rule): every redundant slot,
    one at a time, goes to the expert whose load per replica is highest at
    that moment; among equal loads per replica the lower id wins.

    A priority queue holds each expert keyed by its exact load per replica
    (a ``Fraction``, so no rounding decides a tie); the granted expert goes
    back in with its new, lower key."""
    rep = [1] * len(counts)
    queue = [(-Fraction(int(c)), e) for e, c in enumerate(counts)]
    heapq.heapify(queue)
    for _ in range(redundant):
        _, e = heapq.heappop(queue)
        rep[e] += 1
        heapq.heappush(queue, (-Fraction(int(counts[e]), rep[e]), e))
    return rep


def place_replicas(counts: Sequence[int], replicas: Sequence[int], ep: int
                   ) -> Tuple[List[List[Tuple[int, int]]], List[float]]:
    """Placement of every replica (section 5.2's rule): a replica carries
    load counts[e] / replicas[e]; replicas are taken heaviest first and each
    goes to the currently lightest rank that still has a free slot.  Every
    rank has (total replicas) / ep slots (section 5.3's (E + R) / EP).

    Order among equal loads: replicas in (expert, replica) order; among
    equally light ranks the lower rank.  The open ranks sit in a priority
    queue keyed (load, rank); a rank leaves it when its slots are full.
    Returns per rank the list of (expert, replica index) it holds, in
    placement order, and the rank loads (float sums in placement order)."""
    total = sum(replicas)
    if total % ep:
        raise ValueError("total replicas must divide evenly over the ranks")
    slots = total // ep
    order = sorted(((e, r) for e in range(len(counts))
                    for r in range(replicas[e])),
                   key=lambda er: (-Fraction(int(counts[er[0]]),
                                             replicas[er[0]]),) + er)
    load = [0.0] * ep
    held: List[List[Tuple[int, int]]] = [[] for _ in range(ep)]
    open_ranks = [(0.0, g) for g in range(ep)] if slots else []
    for e, r in order:
        _, g = heapq.heappop(open_ranks)
        load[g] += counts[e] / replicas[e]
        held[g].append((e, r))
        if len(held[g]) < slots:
            heapq.heappush(open_ranks, (load[g], g))
    return held, load


def rank_map(held: Sequence[Sequence[Tuple[int, int]]],
             replicas: Sequence[int], rank: int):
    """Dispatch map of one rank under a placement over all ranks.

    The rank's physical experts are its slots ordered by (expert, replica);
    l2p[e, r] is the physical id on this rank of replica r of expert e, or -1
    when that replica is placed on another rank; rep_count[e] is the
    expert's replica count over the whole group, so pair n of e still goes to
    replica n mod R_e.  Returns (l2p [E, max(replicas)], rep_count [E], P)."""
    E = len(replicas)
    slots = sorted(held[rank])
    l2p = np.full((E, max(replicas)), -1, dtype=np.int32)
    for pid, (e, r) in enumerate(slots):
        l2p[e, r] = pid
    return l2p, np.asarray(replicas, dtype=np.int32), len(slots)


def window_load(history: Sequence[Sequence[int]], window: int) -> np.ndarray:
    """Load over the sliding window (section 5.3: the balancer averages the
    recorded per-expert load over the most recent steps): the element-wise
    sum of the last ``window`` recorded count vectors."""
    recent = list(history)[-window:] if window > 0 else []
    if not recent:
        return np.zeros(0, dtype=np.int64)
    return np.sum(np.asarray(recent, dtype=np.int64), axis=0)


def busiest_over_mean(load: Sequence[float]) -> float:
    return max(load) / (sum(load) / len(load))


def mean_over_busiest(load: Sequence[float]) -> float:
    """The balancedness that vLLM's EPLB logs (mean / max, 1 is perfect)."""
    return (sum(load) / len(load)) / max(load)


def imbalance_table(counts: Sequence[int], eps=(8, 32, 64, 256)):
    """busiest/mean per EP degree for contiguous placement, for placement by
    load without redundancy, and with one redundant replica per rank."""
    rows = []
    for ep in eps:
        c = busiest_over_mean(contiguous_load(counts, ep))
        _, l0 = place_replicas(counts, plan_replicas(counts, 0), ep)
        _, l1 = place_replicas(counts, plan_replicas(counts, ep), ep)
        rows.append((ep, len(counts) // ep, c, busiest_over_mean(l0),
                     busiest_over_mean(l1)))
    return rows
