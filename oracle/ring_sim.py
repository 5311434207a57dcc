"""Literal message-passing model of ring AllReduce, for pinning the oracle.

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

This follows the step-by-step description of ring AllReduce in the CMU 11-868
L14-L15 notes ("Ring AllReduce: ReduceScatter, then AllGather"): each of K
workers splits its gradient into K chunks; in the ReduceScatter phase, at
every step each worker sends one chunk to the next worker in the ring, which
adds it to its own matching chunk, and after K-1 steps each worker holds one
fully reduced chunk; in the AllGather phase another K-1 steps pass the
finished chunks on until every worker has all of them. Messages are chopped
into S pieces as in the same notes' section "Why a ring: chop the data so
transfers pipeline".

Schedule used (the reading in which worker c ends up owning chunk c): at
ReduceScatter step t, worker r sends its running partial of chunk
(r - 1 - t) mod K to worker r + 1, which replaces its own copy of that chunk
by (received + own). At AllGather step t, worker r forwards finished chunk
(r - t) mod K to worker r + 1, which stores it.

Nothing here is shared with dp_oracle.c: this module models the workers and
their messages explicitly, while the C oracle evaluates a closed-form fold.
The payload type is pluggable, so the same code runs on numpy float32 arrays
(IEEE arithmetic) and on symbolic term lists (to read off who adds what).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Callable

import numpy as np


def chunk_bounds(n: int, k: int) -> list[tuple[int, int]]:
    """Chunk c of an n-element gradient: [cL, min((c+1)L, n)), L = ceil(n/k)."""
    L = -(-n // k) if n else 0
    return [(min(c * L, n), min((c + 1) * L, n)) for c in range(k)]


def split_messages(lo: int, hi: int, s: int) -> list[tuple[int, int]]:
    """Cut [lo, hi) into s consecutive pieces of ceil(len/s) (the last ones short/empty)."""
    m = -(-(hi - lo) // s) if hi > lo else 0
    return [(min(lo + q * m, hi), min(lo + (q + 1) * m, hi)) for q in range(s)]


@dataclass
class Link:
    """One-way link r -> r+1; counts the messages it carried."""
    messages: int = 0
    log: list = field(default_factory=list)


@dataclass
class Worker:
    rank: int
    chunks: list          # chunk index -> list of S payload pieces


def _make_workers(data, k, s, bounds, take):
    workers = []
    for r in range(k):
        pieces = []
        for (lo, hi) in bounds:
            pieces.append([take(data[r], a, b) for (a, b) in split_messages(lo, hi, s)])
        workers.append(Worker(r, pieces))
    return workers


def reduce_scatter(data, k: int, n: int, s: int = 1,
                   add: Callable = None, take: Callable = None, links=None):
    """Run the ReduceScatter phase; returns the workers (worker c owns chunk c)."""
    add = add or (lambda recv, own: recv + own)
    take = take or (lambda buf, a, b: buf[a:b].copy())
    bounds = chunk_bounds(n, k)
    workers = _make_workers(data, k, s, bounds, take)
    links = links if links is not None else [Link() for _ in range(k)]
    for t in range(k - 1):
        # every worker puts one chunk on its outgoing link at the same time
        sent = []
        for w in workers:
            ch = (w.rank - 1 - t) % k
            sent.append((ch, list(w.chunks[ch])))
            links[w.rank].messages += s
            links[w.rank].log.append(("rs", t, ch))
        for w in workers:
            src = (w.rank - 1) % k
            ch, msgs = sent[src]
            for q in range(s):   # pieces arrive in order; each is added on arrival
                w.chunks[ch][q] = add(msgs[q], w.chunks[ch][q])
    return workers


def all_gather(workers, k: int, links=None):
    """Run the AllGather phase on workers that each own their finished chunk."""
    links = links if links is not None else [Link() for _ in range(k)]
    for t in range(k - 1):
        sent = []
        for w in workers:
            ch = (w.rank - t) % k
            sent.append((ch, list(w.chunks[ch])))
            links[w.rank].messages += len(w.chunks[ch])
            links[w.rank].log.append(("ag", t, ch))
        for w in workers:
            ch, msgs = sent[(w.rank - 1) % k]
            w.chunks[ch] = msgs
    return workers


def flatten(worker) -> np.ndarray:
    return np.concatenate([np.concatenate(p) if p else np.zeros(0, np.float32)
                           for p in worker.chunks])


# ----------------------------------------------------------------- numerics

def rs_f32(xs, s: int = 1, op: str = "sum", weights=None, total=None):
    """Numeric ring ReduceScatter on float32 arrays.

    op 'sum': plain ring sums. op 'avg': the owner divides its finished chunk
    by K. With weights (f32 per rank) each worker first scales its own
    gradient, and the owner divides by `total` at the end.
    Returns K float32 arrays, the finished chunk of each worker (unpadded).
    """
    k, n = len(xs), xs[0].size
    data = [np.asarray(x, np.float32) for x in xs]
    if weights is not None:
        data = [np.float32(weights[r]) * data[r] for r in range(k)]
    workers = reduce_scatter(data, k, n, s)
    out = []
    for c, w in enumerate(workers):
        chunk = np.concatenate(w.chunks[c]).astype(np.float32) if w.chunks[c] else \
            np.zeros(0, np.float32)
        if op == "avg":
            chunk = chunk / np.float32(k)
        elif weights is not None:
            chunk = chunk / np.float32(total)
        out.append(chunk.astype(np.float32))
    return out


def rs_i32(xs, s: int = 1):
    """Ring ReduceScatter with wrap-around int32 addition."""
    k, n = len(xs), xs[0].size
    data = [np.asarray(x, np.int32).astype(np.uint32) for x in xs]
    workers = reduce_scatter(data, k, n, s, add=lambda a, b: (a + b).astype(np.uint32))
    return [np.concatenate(w.chunks[c]).astype(np.uint32).view(np.int32) if w.chunks[c]
            else np.zeros(0, np.int32) for c, w in enumerate(workers)]


def ar_f32(xs, s: int = 1, op: str = "sum"):
    """Ring AllReduce (ReduceScatter then AllGather) on float32 arrays."""
    k, n = len(xs), xs[0].size
    data = [np.asarray(x, np.float32) for x in xs]
    workers = reduce_scatter(data, k, n, s)
    if op == "avg":
        for c, w in enumerate(workers):
            w.chunks[c] = [p / np.float32(k) for p in w.chunks[c]]
    all_gather(workers, k)
    return [flatten(w).astype(np.float32) for w in workers]


# ----------------------------------------------------------------- symbolic

def symbolic_ring(k: int, s: int = 1):
    """Each worker's gradient is K chunks named <letter><index> (a0..a3 on
    worker 0, b0..b3 on worker 1, ...). Returns (after_rs, after_ag), lists
    per worker of the term tuples each chunk holds."""
    letters = "abcdefghijklmnopqrstuvwxyz"
    data = [[(f"{letters[r]}{c}",) for c in range(k)] for r in range(k)]
    take = lambda buf, a, b: buf[a:b]            # one element per chunk
    add = lambda recv, own: [x + y for x, y in zip(recv, own)]
    workers = reduce_scatter(data, k, k, s, add=add, take=take)
    after_rs = [[tuple(t for piece in w.chunks[c] for elem in piece for t in elem)
                 for c in range(k)] for w in workers]
    all_gather(workers, k)
    after_ag = [[tuple(t for piece in w.chunks[c] for elem in piece for t in elem)
                 for c in range(k)] for w in workers]
    return after_rs, after_ag
