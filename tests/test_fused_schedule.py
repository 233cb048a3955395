"""The fused decode kernel's ticket protocol, simulated on the CPU.

The kernel (ffn_fused_dma_kernel) hands out tiles from one monotone ticket
counter: tickets [0, n13) are W13 tiles (channel tile y = t // blocks, row
block b = t % blocks), tickets [n13, n13 + n2) are W2 tiles (split z, channel
group dt, block b).  A W13 tile counts itself into done[b][16 y // ksplit]
when its h is written; a W2 tile waits until done[b][z] reaches the number of
16-channel W13 tiles in its K range; after writing its partials it counts one
arrival per real slot on (token, dt), and the arrival that completes k *
splits does that token's combine.  These tests mirror the kernel's integer
arithmetic and check, for many shapes and many random interleavings of a
bounded set of resident workers, that every tile is handed out exactly once,
that every wait depends only on tickets handed out earlier, that no schedule
deadlocks, and that every (token, channel group) is combined exactly once,
after all of its partials.
"""

import random

import numpy as np
import pytest

import oracle


def layout(T, E, k, B, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
    al = oracle.align(ids, E, B)
    return al["sorted_ids"], al["num_padded"] // B


def tiles(nblk, I, d, rn, splits, ksplit):
    n13 = nblk * (I // 16)
    nd = d // (16 * rn)
    n2 = nblk * nd * splits
    out = []
    for t in range(n13 + n2):
        if t < n13:
            y, b = t // nblk, t % nblk
            out.append(("w13", b, y, (16 * y) // ksplit))
        else:
            t2 = t - n13
            z = t2 // (nblk * nd)
            r = t2 - z * nblk * nd
            dt, b = r // nblk, r % nblk
            kb = z * ksplit
            need = (min(I, kb + ksplit) - kb) // 16
            out.append(("w2", b, dt, z, need))
    return out, n13, nd


SHAPES = [
    # T, E, k, B, d, I, rn, splits
    (1, 8, 2, 16, 4096, 14336, 4, 8),
    (8, 8, 2, 16, 4096, 14336, 2, 8),
    (16, 16, 4, 16, 512, 2048, 2, 4),
    (32, 8, 2, 32, 4096, 14336, 2, 4),
    (64, 8, 2, 32, 4096, 14336, 2, 2),
    (64, 8, 2, 32, 512, 768, 2, 3),         # uneven last split: 768 = 2 * 256 + 256
    (40, 4, 1, 32, 256, 512, 2, 1),         # one split; an expert with two blocks
]


@pytest.mark.parametrize("T,E,k,B,d,I,rn,splits", SHAPES)
def test_every_tile_once_and_waits_only_on_earlier_tickets(T, E, k, B, d, I, rn, splits):
    sorted_ids, nblk = layout(T, E, k, B, T * 7 + E)
    ksplit = -(-I // splits)
    ksplit = -(-ksplit // 256) * 256          # a multiple of the K stage (and of 16)
    splits = -(-I // ksplit)
    ts, n13, nd = tiles(nblk, I, d, rn, splits, ksplit)
    w13 = [x for x in ts if x[0] == "w13"]
    w2 = [x for x in ts if x[0] == "w2"]
    assert len(set((b, y) for _, b, y, _ in w13)) == len(w13) == nblk * (I // 16)
    assert len(set((b, dt, z) for _, b, dt, z, _ in w2)) == len(w2) == nblk * nd * splits
    # the W13 tiles counted into done[b][z] are exactly the ones a W2 tile of
    # (b, z) needs, and all of them hold earlier tickets
    for t, x in enumerate(ts):
        if x[0] == "w2":
            _, b, dt, z, need = x
            deps = [u for u, y in enumerate(ts) if y[0] == "w13" and y[1] == b and y[3] == z]
            assert len(deps) == need and need > 0
            assert max(deps) < t


def simulate(T, E, k, B, d, I, rn, splits, workers, seed, w2_first=False):
    sorted_ids, nblk = layout(T, E, k, B, T * 7 + E)
    ksplit = -(-I // splits)
    ksplit = -(-ksplit // 256) * 256
    splits = -(-I // ksplit)
    ts, n13, nd = tiles(nblk, I, d, rn, splits, ksplit)
    if w2_first:             # a wrong order, to show the simulation catches it
        ts = ts[n13:] + ts[:n13]
    A = T * k
    rnd = random.Random(seed)
    ticket = 0
    done = {}
    arrive = {}
    written = set()          # (z, slot, dt) partials written
    combined = {}
    # worker state: None (free), ("run", tile, remaining), ("wait", tile)
    state = [None] * workers
    steps = 0
    while True:
        steps += 1
        assert steps < 10 ** 6, "no progress"
        progressed = False
        order = list(range(workers))
        rnd.shuffle(order)
        for w in order:
            st = state[w]
            if st is None:
                if ticket >= len(ts):
                    continue
                tile = ts[ticket]
                ticket += 1
                state[w] = ("wait", tile) if tile[0] == "w2" else ("run", tile, rnd.randint(1, 5))
                progressed = True
            elif st[0] == "wait":
                _, b, dt, z, need = st[1]
                if done.get((b, z), 0) >= need:
                    state[w] = ("run", st[1], rnd.randint(1, 5))
                    progressed = True
            else:
                _, tile, rem = st
                if rnd.random() < 0.5:
                    continue          # this worker is slow this round
                progressed = True
                if rem > 1:
                    state[w] = ("run", tile, rem - 1)
                    continue
                state[w] = None
                if tile[0] == "w13":
                    _, b, y, z = tile
                    done[(b, z)] = done.get((b, z), 0) + 1
                else:
                    _, b, dt, z, need = tile
                    slots = [int(f) for f in sorted_ids[b * B:(b + 1) * B] if f < A]
                    for f in slots:
                        written.add((z, f, dt))
                    for f in slots:
                        key = (f // k, dt)
                        arrive[key] = arrive.get(key, 0) + 1
                        if arrive[key] == k * splits:
                            tok = f // k
                            assert key not in combined
                            for j in range(k):
                                for zz in range(splits):
                                    assert (zz, tok * k + j, dt) in written
                            combined[key] = True
        if ticket >= len(ts) and all(s is None for s in state):
            break
        # a deadlock: nobody runs, nobody can take a ticket, and no wait can end
        running = any(s is not None and s[0] == "run" for s in state)
        can_take = ticket < len(ts) and any(s is None for s in state)
        can_wake = any(s is not None and s[0] == "wait" and
                       done.get((s[1][1], s[1][3]), 0) >= s[1][4] for s in state)
        assert running or can_take or can_wake or progressed, "deadlock: every worker waits"
    assert len(combined) == T * nd
    assert all(v == k * splits for v in arrive.values())


@pytest.mark.parametrize("T,E,k,B,d,I,rn,splits", SHAPES)
@pytest.mark.parametrize("workers", [1, 3, 64])
def test_no_schedule_deadlocks_and_each_token_is_combined_once(T, E, k, B, d, I, rn, splits,
                                                               workers):
    # d and I scaled down where the tile count would make the simulation slow
    scale = max(1, (I // 16 + d // (16 * rn) * splits) // 256)
    I_s = max(256, (I // scale) // 256 * 256)
    for seed in range(3):
        simulate(T, E, k, B, min(d, 1024), I_s, rn, splits, workers, seed)


def test_simulation_catches_a_wrong_ticket_order():
    # W2 tickets before W13 tickets: a single resident worker waits forever
    with pytest.raises(AssertionError, match="deadlock"):
        simulate(8, 8, 2, 16, 512, 512, 2, 2, workers=1, seed=0, w2_first=True)
