"""Whole-shard parity at full size: a shard is streamed through the oracle in chunks on host threads.

Each chunk's inputs and results are downloaded and checked by the caller's ``work(a, b)``; numpy
releases the interpreter lock inside its array operations, so the chunks run in parallel. The
element count covered is returned so a test can assert and report 100% coverage.
"""

from __future__ import annotations

import concurrent.futures
import os
import time

CHUNK = 1 << 24                                   # elements per chunk (16 Mi)
THREADS = max(1, min(12, os.cpu_count() or 1))


def chunks(S: int, chunk: int = CHUNK):
    return [(a, min(S, a + chunk)) for a in range(0, S, chunk)]


def run_chunks(S: int, work, chunk: int = CHUNK, threads: int = THREADS):
    """Run work(a, b) for every chunk [a, b) of [0, S); re-raise the first failure. Returns
    (elements covered, seconds)."""
    t0 = time.perf_counter()
    covered = 0
    ex = concurrent.futures.ThreadPoolExecutor(threads)
    try:
        futs = {ex.submit(work, a, b): (a, b) for a, b in chunks(S, chunk)}
        for f in concurrent.futures.as_completed(futs):
            f.result()
            a, b = futs[f]
            covered += b - a
    finally:
        ex.shutdown(wait=True, cancel_futures=True)
    return covered, time.perf_counter() - t0
