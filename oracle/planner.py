"""Exact block plan by enumeration: tiles, classes, pair counts, PTRR, step maps.

MARBLE, section 03:
  * "Block classification": a (query block, key block) pair is *full* when
    every token pair is legal, *empty* when none is, *partial* otherwise.  The
    page classifies from per-block summaries ("provably" full / empty), which is
    sound but may leave a truly full or empty pair marked partial; the unique
    target fixed here is the exact tri-state over the tile's valid token pairs,
    found by counting the legal pairs with the mask predicate.
  * Ring step submask: at step s rank r pairs its query shard with the key
    shard of rank j = (r - s) mod R.
  * "PTRR": sort query blocks by cost, deal them to ranks in rounds of R with
    every other round reversed, keep each rank's blocks in sequence order.
    Readings (the page fixes none of them): the cost of a block is its exact
    number of legal (query, key) pairs over all keys (the count Libra's Eq. 6
    estimates, and the quantity the FLOP metric counts); the sort is by cost
    descending with ties broken by ascending original block index; round t
    deals sorted positions [tR, (t+1)R), to ranks 0..R-1 when t is even and to
    ranks R-1..0 when t is odd; shards are the ranks' block lists concatenated
    in rank order.
  * Layout transforms: the contiguous layout (no permutation) shards tokens
    into R equal runs; tiles are then `block`-token pieces of each shard, the
    last one ragged when the shard is not a multiple of `block`.

Pinned by: tests/test_oracle_planner.py (brute-force pair enumeration in pure
Python on tiny layouts; causal contiguous shards give 1, 2, 3, 4 non-empty
blocks and zigzag gives 9 per device, as the ring-attention explainer counts
them; closed-form pair totals; the sliding-window tile map in closed form;
PTRR is a bijection with equal block counts per rank).
"""
from __future__ import annotations

from dataclasses import dataclass
import numpy as np

from .mask import legal, take

EMPTY, PARTIAL, FULL = 0, 1, 2


@dataclass
class OraclePlan:
    n: int
    ranks: int
    block: int
    tiles_per_shard: int
    shard_tokens: int
    starts: np.ndarray          # original-order tile starts  [T]
    ends: np.ndarray            # original-order tile ends    [T]
    tiles_new: np.ndarray       # original tile id of new tile position [T]
    owner: np.ndarray           # shard of each original tile [T]
    local: np.ndarray           # index of each original tile within its shard [T]
    cost: np.ndarray            # legal pairs of each original tile's queries [T]
    pairs_k: list               # per original q tile: original k tile ids with count > 0
    pairs_c: list               # per original q tile: counts (int64) matching pairs_k
    perm: np.ndarray            # token permutation, perm[new] = original

    def tile_len(self, t):
        return int(self.ends[t] - self.starts[t])

    def step_map(self, r: int, s: int):
        """map[a][b] (uint8 class) for q tile a of rank r and k tile b of shard (r-s) mod R."""
        j = (r - s) % self.ranks
        t_sh = self.tiles_per_shard
        mp = np.zeros((t_sh, t_sh), np.uint8)
        total = 0
        for a in range(t_sh):
            tq = int(self.tiles_new[r * t_sh + a])
            for tk, c in zip(self.pairs_k[tq], self.pairs_c[tq]):
                if self.owner[tk] != j:
                    continue
                b = int(self.local[tk])
                full = self.tile_len(tq) * self.tile_len(tk)
                mp[a, b] = FULL if c == full else PARTIAL
                total += int(c)
        return mp, total

    def rank_pairs(self):
        """pairs[r][s]: legal pairs between rank r's queries and shard (r-s) mod R."""
        out = np.zeros((self.ranks, self.ranks), np.int64)
        for r in range(self.ranks):
            for s in range(self.ranks):
                out[r, s] = self.step_map(r, s)[1]
        return out

    def busiest_rank(self) -> int:
        """Rank with the most legal pairs (ties: lowest rank)."""
        t_sh = self.tiles_per_shard
        tot = [int(sum(self.cost[self.tiles_new[r * t_sh:(r + 1) * t_sh]]))
               for r in range(self.ranks)]
        return int(np.argmax(tot))


def tile_bounds(n: int, ranks: int, block: int, order: str):
    if order == "contiguous":
        if n % ranks:
            raise ValueError("contiguous layout needs n % ranks == 0")
        s_tok = n // ranks
        per = -(-s_tok // block)
        starts, ends = [], []
        for r in range(ranks):
            for t in range(per):
                a = r * s_tok + t * block
                starts.append(a)
                ends.append(min(a + block, (r + 1) * s_tok))
        return np.asarray(starts, np.int64), np.asarray(ends, np.int64), per
    if n % (block * ranks):
        raise ValueError("block orders need n % (block * ranks) == 0")
    starts = np.arange(0, n, block, dtype=np.int64)
    return starts, starts + block, n // block // ranks


def pair_counts(tracks, window: int, starts, ends):
    """Legal-pair counts of every tile pair whose samples overlap, by enumeration."""
    sample = np.asarray(tracks[0], np.int64)
    n = len(sample)
    tile_of = np.repeat(np.arange(len(starts)), ends - starts)
    change = np.flatnonzero(np.diff(sample)) + 1
    run_start = np.concatenate([[0], change])
    run_end = np.concatenate([change, [n]])
    first = {int(sample[a]): int(a) for a in run_start}
    last = {int(sample[a]): int(b - 1) for a, b in zip(run_start, run_end)}
    ks, cs = [], []
    for t in range(len(starts)):
        a, b = int(starts[t]), int(ends[t])
        ka = first[int(sample[a])]
        kb = last[int(sample[b - 1])] + 1
        allowed = legal(take(tracks, np.arange(a, b)), take(tracks, np.arange(ka, kb)), window)
        per_key = allowed.sum(axis=0)
        tiles = tile_of[ka:kb]
        t0 = tiles.min()
        cnt = np.bincount(tiles - t0, weights=per_key).astype(np.int64)
        nz = np.flatnonzero(cnt)
        ks.append((nz + t0).astype(np.int64))
        cs.append(cnt[nz])
    return ks, cs


def ptrr_owner(cost, ranks: int):
    """PTRR deal: owner rank of each block (see the module header for the readings)."""
    cost = np.asarray(cost, np.int64)
    order = sorted(range(len(cost)), key=lambda t: (-int(cost[t]), t))
    owner = np.empty(len(cost), np.int64)
    for pos, t in enumerate(order):
        rnd, i = divmod(pos, ranks)
        owner[t] = i if rnd % 2 == 0 else ranks - 1 - i
    return owner


def build(tracks, window: int, ranks: int, block: int = 128, order: str = "ptrr",
          explicit_block_perm=None) -> OraclePlan:
    n = len(tracks[0])
    starts, ends, per = tile_bounds(n, ranks, block, order)
    ks, cs = pair_counts(tracks, window, starts, ends)
    cost = np.array([int(c.sum()) for c in cs], np.int64)
    t_all = len(starts)
    if order == "contiguous":
        tiles_new = np.arange(t_all)
    elif order == "ptrr":
        owner = ptrr_owner(cost, ranks)
        tiles_new = np.concatenate([np.flatnonzero(owner == r) for r in range(ranks)])
    elif order == "explicit":
        tiles_new = np.asarray(explicit_block_perm, np.int64)
        if sorted(tiles_new.tolist()) != list(range(t_all)):
            raise ValueError("explicit block order must be a permutation")
    else:
        raise ValueError(order)
    owner = np.empty(t_all, np.int64)
    local = np.empty(t_all, np.int64)
    for pos, t in enumerate(tiles_new):
        owner[t] = pos // per
        local[t] = pos % per
    perm = np.concatenate([np.arange(starts[t], ends[t]) for t in tiles_new]).astype(np.int64)
    return OraclePlan(n=n, ranks=ranks, block=block, tiles_per_shard=per,
                      shard_tokens=n // ranks, starts=starts, ends=ends,
                      tiles_new=np.asarray(tiles_new, np.int64), owner=owner, local=local,
                      cost=cost, pairs_k=ks, pairs_c=cs, perm=perm)

