"""Reference model of the decode-host block cache (TEST INFRASTRUCTURE ONLY).

Pure Python, one request at a time, written from the pages' description:
OasisKV paperpeel v2 text, §3.2.1 (ii) (the decode host fetches, from remote
memory, whole blocks for the union of every KV head's selections, even if only
one head selects a block) and §3.2.3 (a per-request budget of f_Host*P + F
blocks; a periodic pass evicts the least recently used prompt blocks while
protecting generated blocks and the current working set; evicted blocks stay
in remote memory and are fetched again when selected); §3.2.2, union block
mapping (remote block -> decode-host block, per request).

Policy details the pages leave open (readings):
  * the union of a step is the plan's source blocks in (head, entry) order,
    each once;
  * a missing block takes the lowest free slot, else evicts the occupied slot
    with the smallest (last use, slot) among blocks that are neither
    generated, nor in the request's HBM working set after the plan, nor in
    this step's union; with none left the fetch fails (budget too small);
  * every block of the union is stamped with the step (last use);
  * trim(target) evicts by the same order until at most `target` slots hold
    blocks.
"""
from __future__ import annotations

import numpy as np


class HostTierModel:
    def __init__(self, capacity, n_blk, remote=None):
        """capacity [R] slots per request; n_blk blocks per request in remote
        memory; remote [R][n_blk][bytes] (optional: then data moves too)."""
        self.cap = [int(c) for c in capacity]
        self.R = len(self.cap)
        self.n_blk = int(n_blk)
        self.map = -np.ones((self.R, self.n_blk), np.int32)
        self.slot_blk = [[-1] * c for c in self.cap]
        self.last = [[-1] * c for c in self.cap]
        self.generated = [set() for _ in range(self.R)]
        self.remote = remote
        self.cache = None if remote is None else [
            np.zeros((c, remote.shape[2]), remote.dtype) for c in self.cap]
        self.fetched = 0
        self.evicted = 0

    def _victim(self, r, keep):
        best = None
        for s, b in enumerate(self.slot_blk[r]):
            if b < 0 or b in keep or b in self.generated[r]:
                continue
            key = (self.last[r][s], s)
            if best is None or key < best[0]:
                best = (key, s)
        return None if best is None else best[1]

    def _place(self, r, b, keep):
        free = [s for s, x in enumerate(self.slot_blk[r]) if x < 0]
        if free:
            s = free[0]
        else:
            s = self._victim(r, keep)
            if s is None:
                raise RuntimeError("decode-host budget holds no evictable block")
            self.map[r, self.slot_blk[r][s]] = -1
            self.evicted += 1
        self.slot_blk[r][s] = b
        self.map[r, b] = s
        return s

    def fetch(self, step, plan_count, plan_src, slot_block):
        """One layer-step: plan_count [R][H], plan_src [R][H][K], slot_block
        [R][H][K] (the HBM working set after the plan).  Returns the list of
        (r, block, slot) fetched from remote, in order."""
        out = []
        R, H = plan_count.shape
        for r in range(R):
            union = []
            for g in range(H):
                for i in range(int(plan_count[r, g])):
                    b = int(plan_src[r, g, i])
                    if b not in union:
                        union.append(b)
            keep = set(union) | {int(x) for x in slot_block[r].ravel() if x >= 0}
            for b in union:
                if self.map[r, b] < 0:
                    s = self._place(r, b, keep)
                    self.fetched += 1
                    out.append((r, b, s))
                    if self.cache is not None:
                        self.cache[r][s] = self.remote[r, b]
            for b in union:
                self.last[r][self.map[r, b]] = step
        return out

    def add_generated(self, r, b, step, slot_block):
        """A block generated on the decode node joins the cache, protected."""
        keep = {int(x) for x in np.asarray(slot_block[r]).ravel() if x >= 0}
        s = self._place(r, b, keep) if self.map[r, b] < 0 else int(self.map[r, b])
        self.generated[r].add(b)
        self.last[r][s] = step
        return s

    def trim(self, target, slot_block):
        for r in range(self.R):
            keep = {int(x) for x in np.asarray(slot_block[r]).ravel() if x >= 0}
            while sum(1 for b in self.slot_blk[r] if b >= 0) > int(target[r]):
                s = self._victim(r, keep)
                if s is None:
                    break
                self.map[r, self.slot_blk[r][s]] = -1
                self.slot_blk[r][s] = -1
                self.last[r][s] = -1
                self.evicted += 1
