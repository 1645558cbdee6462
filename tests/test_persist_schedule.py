"""Host emulation of the persistent prefill's work schedule (DKV_PREFILL_PERSIST, disabled on the
GPU). One XCD's queue is replayed with W resident workgroups and random item durations: each
workgroup takes the next item index, decodes it into (super-chunk s, query tile) or the producer
slot, waits until the tile's completion counter reaches s, runs, and bumps the counter. The
checks: the queue drains for every W (no wait is ever left without a running item to end it),
every item runs once, the items of a query tile run in super-chunk order and each starts after
its predecessor ended, and the storer shares cover every new row of the pair once.

This is the index arithmetic of attn_persist_kernel and of the host planner that launches it,
restated; it does not run GPU code.
"""
import heapq
import random

import pytest


def _plan(T, G, L, sk, rows_per_tile=256, cus=256):
    Q = (T * G + rows_per_tile - 1) // rows_per_tile
    S = (L + T + sk - 1) // sk
    pre_slot = min(max(1, cus // 8), Q)
    s_store = min(S - 1, (L + sk - 1) // sk)
    return Q, S, pre_slot, s_store


def _decode(item, Q, pre_slot):
    per_sc = Q + 1
    s, r = divmod(item, per_sc)
    if r == pre_slot:
        return s, None, None               # producer item
    ci = r if r < pre_slot else r - 1
    return s, ci, Q - 1 - ci


def _replay(T, G, L, sk, workers, seed):
    Q, S, pre_slot, s_store = _plan(T, G, L, sk)
    n_items = S * (Q + 1)
    n_store = (S - s_store) * Q
    rng = random.Random(seed)
    done = [0] * Q
    next_item = 0
    clock = 0.0
    running = []                           # (end time, worker, item)
    waiting = []                           # (worker, item) blocked on a counter
    finished = {}                          # item -> (start, end)
    stored = []
    idle = list(range(workers))

    def start(w, item, t):
        s, ci, qt = _decode(item, Q, pre_slot)
        if ci is not None and s > 0 and done[qt] < s:
            waiting.append((w, item))
            return
        if ci is not None and s >= s_store:
            k = (s - s_store) * Q + ci
            stored.extend(range(T * k // n_store, T * (k + 1) // n_store))
        end = t + rng.uniform(0.5, 2.0)
        heapq.heappush(running, (end, w, item, t))

    while True:
        while idle:
            w = idle.pop()
            item = next_item
            next_item += 1
            if item < n_items:
                start(w, item, clock)
            # a workgroup that takes an index past the queue exits
        if not running:
            assert not waiting, f"stalled: {len(waiting)} waiting, nothing running"
            break
        end, w, item, t0 = heapq.heappop(running)
        clock = end
        s, ci, qt = _decode(item, Q, pre_slot)
        finished[item] = (t0, end)
        if ci is not None:
            done[qt] += 1
        idle.append(w)
        # waiters whose counter is now reached start at once
        still = []
        for ww, it in waiting:
            s2, c2, q2 = _decode(it, Q, pre_slot)
            if done[q2] >= s2:
                start(ww, it, clock)
            else:
                still.append((ww, it))
        waiting[:] = still
    return Q, S, finished, stored, pre_slot


@pytest.mark.parametrize("T, G, L, sk", [
    (300, 4, 3000, 2048),      # 5 query tiles, 2 super-chunks (the first GPU case)
    (1100, 4, 5000, 2048),     # 18 query tiles, 4 super-chunks
    (2048, 2, 2100, 2048),     # 16 query tiles
    (8192, 4, 24576, 2048),    # 128 query tiles: the producer slot inside the super-chunk
    (64, 4, 0, 2048),          # one super-chunk, nothing past
])
@pytest.mark.parametrize("workers", [1, 2, 7, 32])
def test_persistent_schedule_drains_in_order(T, G, L, sk, workers):
    Q, S, finished, stored, pre_slot = _replay(T, G, L, sk, workers, seed=T + workers)
    assert len(finished) == S * (Q + 1)
    for qt in range(Q):
        ci = Q - 1 - qt
        r = ci if ci < pre_slot else ci + 1
        items = [s * (Q + 1) + r for s in range(S)]
        for a, b in zip(items, items[1:]):
            assert finished[b][0] >= finished[a][1], "a super-chunk started before its predecessor ended"
    assert sorted(stored) == list(range(T)), "storer shares must cover every new row once"
