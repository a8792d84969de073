"""Keyed-table model of the oracle -- TEST INFRASTRUCTURE ONLY.

Collisionless int64-keyed embedding table with a frequency filter, after the
Monolith paper, Sec. 2.1 "Hash Table": distinct IDs never share an embedding, and
an ID is admitted only once its occurrence count reaches a tunable threshold.

The model keeps what the method defines and nothing about slot placement:
  key -> (occurrence count, admitted?, row values).
Step rule (batch-level, independent of thread order):
  m_k  = occurrences of valid key k (k >= 1) in the step, repeats included;
  present keys: count += m_k; absent keys: inserted with count = m_k;
  a key without a row whose count reaches the threshold is admitted now and gets
  a fresh row (oracle_init_row); every occurrence of an admitted key returns its
  row, the others return DEFAULT (a zero row that counts in a mean).
  Keys < 1 are dropped.  Prepopulated keys are admitted with count 0.

Lifecycle (Monolith Sec. 2.1 also expires IDs that go unseen for long, so the
table holds only live features):
  every lookup-or-insert is one table step s = 0, 1, 2, ...; a key present after
  step s (found or inserted) records last_seen = s; prepopulated / imported keys
  record the step counter's value at that time;
  evict(min_seen) removes every key with last_seen < min_seen: its count, its
  admission and its row values are gone, and a later occurrence starts it anew;
  a checkpoint is (keys, counts, last_seen, admitted, values, step counter), and
  a table restored from it behaves exactly like the original.

Count-min admission (optional; Monolith Sec. 2.1 filters IDs by frequency, and a
probabilistic filter avoids holding a slot for every rare ID): keys not in the
table are counted in a d x w sketch instead of slots.  Cell j of key k is
h_j(k) = x_j mod w, where x_0, x_1, ... are the outputs of a SplitMix64 generator
seeded with k (x_j = splitmix64(k + j * gamma), gamma = 0x9E3779B97F4A7C15).  A
step adds m_k to the d cells of every absent key, then each absent key whose
estimate min_j C[j, h_j(k)] reaches the threshold enters the table with
count = its estimate and a fresh row; the others read DEFAULT.  Keys in the
table count exactly, as above.
"""
from __future__ import annotations

import numpy as np

from . import ROW_DEFAULT, ROW_DROPPED, init_row, splitmix64

GAMMA = np.uint64(0x9E3779B97F4A7C15)


def count_min_cells(keys, depth: int, width: int) -> np.ndarray:
    """[depth, n] sketch cells of the keys: SplitMix64 output j of seed k, mod width."""
    k = np.asarray(keys, dtype=np.int64).astype(np.uint64)
    with np.errstate(over="ignore"):
        return np.stack([splitmix64(k + np.uint64(j) * GAMMA) % np.uint64(width)
                         for j in range(depth)]).astype(np.int64)


class TableFull(RuntimeError):
    pass


class OracleTable:
    def __init__(self, capacity: int, dim: int, threshold: int, init_std: float,
                 prepop_keys=None, prepop_rows=None):
        """prepop_rows: array-like [n, dim] or a callable idx -> rows (lazy, so a
        large prepopulated pool can stay wherever it lives)."""
        self.capacity, self.dim, self.threshold, self.init_std = capacity, dim, threshold, init_std
        if prepop_keys is None:
            prepop_keys = np.empty(0, dtype=np.int64)
        pk = np.asarray(prepop_keys, dtype=np.int64)
        order = np.argsort(pk, kind="stable")
        self.keys = pk[order]
        if self.keys.size and np.any(self.keys[1:] == self.keys[:-1]):
            raise ValueError("duplicate prepopulated keys")
        self.count = np.zeros(self.keys.size, dtype=np.int64)
        self.admitted = np.ones(self.keys.size, dtype=bool)
        self.step_no = 0
        self.seen = np.zeros(self.keys.size, dtype=np.int64)
        self.sketch = None                                # count-min: int64 [depth, width]
        self.prepop_idx = order.astype(np.int64)         # index into the prepop rows
        self._prepop_rows = prepop_rows
        self.vals = {}                                    # key -> row values (new or updated)
        if self.keys.size > capacity:
            raise TableFull("prepopulation exceeds capacity")

    def use_count_min(self, depth: int, width: int):
        self.sketch = np.zeros((depth, width), dtype=np.int64)

    # ------------------------------------------------------------- queries
    def _find(self, k: np.ndarray):
        i = np.searchsorted(self.keys, k)
        i = np.minimum(i, max(self.keys.size - 1, 0))
        hit = (self.keys.size > 0) & (self.keys[i] == k) if self.keys.size else np.zeros(k.shape, bool)
        return i, hit

    def row_values(self, keys) -> np.ndarray:
        keys = np.asarray(keys, dtype=np.int64)
        out = np.zeros((keys.size, self.dim), dtype=np.float32)
        idx, hit = self._find(keys)
        need = []
        for j, k in enumerate(keys.tolist()):
            if k in self.vals:
                out[j] = self.vals[k]
            elif hit[j] and self.admitted[idx[j]]:
                need.append(j)
        if need:
            src = self.prepop_idx[idx[need]]
            pr = self._prepop_rows
            vals = pr(src) if callable(pr) else np.asarray(pr)[src]
            out[need] = np.asarray(vals, dtype=np.float32)
        return out

    def state(self, keys):
        """(present, count, admitted) for each key."""
        keys = np.asarray(keys, dtype=np.int64)
        idx, hit = self._find(keys)
        cnt = np.where(hit, self.count[idx] if self.keys.size else 0, 0)
        adm = np.where(hit, self.admitted[idx] if self.keys.size else False, False)
        return hit, cnt, adm

    # ---------------------------------------------------------------- step
    def step(self, keys):
        """One lookup-or-insert over a batch of keys.  Returns (uk, admitted_uk):
        the step's distinct valid keys and whether each is admitted after it."""
        keys = np.asarray(keys, dtype=np.int64)
        valid = keys >= 1
        uk, m = np.unique(keys[valid], return_counts=True)
        idx, hit = self._find(uk)
        new_cnt = m[~hit]
        if self.sketch is not None:
            # absent keys: add the step's occurrences to the sketch, then admit
            # those whose estimate reached the threshold
            absent, ma = uk[~hit], m[~hit]
            cells = count_min_cells(absent, *self.sketch.shape)
            for j in range(self.sketch.shape[0]):
                np.add.at(self.sketch[j], cells[j], ma)
            est = (np.min(np.stack([self.sketch[j][cells[j]] for j in range(self.sketch.shape[0])]),
                          axis=0) if absent.size else np.zeros(0, np.int64))
            enter = est >= self.threshold
            hit = hit.copy()
            keep = np.ones(uk.size, dtype=bool)
            keep[np.nonzero(~hit)[0][~enter]] = False       # stay in the sketch only
            new_cnt = est[enter]
            uk, m, idx, hit = uk[keep], m[keep], idx[keep], hit[keep]
        new = uk[~hit]
        if self.keys.size + new.size > self.capacity:
            raise TableFull(f"{new.size} new keys, {self.capacity - self.keys.size} free slots")
        # count the present keys
        if self.keys.size:
            np.add.at(self.count, idx[hit], m[hit])
        # insert the absent keys with their counts
        if new.size:
            keys2 = np.concatenate([self.keys, new])
            cnt2 = np.concatenate([self.count, new_cnt])
            adm2 = np.concatenate([self.admitted, np.zeros(new.size, dtype=bool)])
            pidx2 = np.concatenate([self.prepop_idx, np.full(new.size, -1, dtype=np.int64)])
            seen2 = np.concatenate([self.seen, np.zeros(new.size, dtype=np.int64)])
            order = np.argsort(keys2, kind="stable")
            self.keys, self.count = keys2[order], cnt2[order]
            self.admitted, self.prepop_idx = adm2[order], pidx2[order]
            self.seen = seen2[order]
        # admit whatever reached the threshold and has no row yet
        idx, hit = self._find(uk)
        assert hit.all()
        self.seen[idx] = self.step_no
        self.step_no += 1
        fresh = (~self.admitted[idx]) & (self.count[idx] >= self.threshold)
        for k in uk[fresh].tolist():
            self.vals[k] = init_row(k, self.dim, self.init_std)
        self.admitted[idx[fresh]] = True
        return uk, self.admitted[idx]

    # ------------------------------------------------------------ lifecycle
    def evict(self, min_seen: int) -> int:
        """Removes the keys last seen before step min_seen; returns how many."""
        keep = self.seen >= min_seen
        for k in self.keys[~keep].tolist():
            self.vals.pop(int(k), None)
        n = int((~keep).sum())
        self.keys, self.count, self.admitted = self.keys[keep], self.count[keep], self.admitted[keep]
        self.prepop_idx, self.seen = self.prepop_idx[keep], self.seen[keep]
        return n

    def checkpoint(self):
        """(keys, counts, last_seen, admitted, values [n, dim], step counter), keys ascending;
        values are zero for keys without a row."""
        vals = np.zeros((self.keys.size, self.dim), dtype=np.float32)
        if self.admitted.any():
            vals[self.admitted] = self.row_values(self.keys[self.admitted])
        return (self.keys.copy(), self.count.copy(), self.seen.copy(), self.admitted.copy(), vals,
                self.step_no)

    @classmethod
    def restore(cls, capacity, dim, threshold, init_std, ckpt):
        keys, counts, seen, admitted, vals, step_no = ckpt
        T = cls(capacity, dim, threshold, init_std)
        order = np.argsort(np.asarray(keys, dtype=np.int64), kind="stable")
        T.keys = np.asarray(keys, dtype=np.int64)[order]
        T.count = np.asarray(counts, dtype=np.int64)[order]
        T.seen = np.asarray(seen, dtype=np.int64)[order]
        T.admitted = np.asarray(admitted, dtype=bool)[order]
        T.prepop_idx = np.full(T.keys.size, -1, dtype=np.int64)
        vals = np.asarray(vals, dtype=np.float32)[order]
        for k, a, v in zip(T.keys.tolist(), T.admitted.tolist(), vals):
            if a:
                T.vals[int(k)] = v.copy()
        T.step_no = int(step_no)
        return T

    def resolve(self, keys):
        """Per-position rows into a compact local pool for the oracle's forward:
        returns (keyed_rows int32 [n], pool_keys int64 [P], pool fp32 [P, dim])."""
        keys = np.asarray(keys, dtype=np.int64)
        valid = keys >= 1
        _, _, adm = self.state(keys)
        use = valid & adm
        pool_keys, inv = np.unique(keys[use], return_inverse=True)
        rows = np.full(keys.size, ROW_DROPPED, dtype=np.int32)
        rows[valid & ~adm] = ROW_DEFAULT
        rows[use] = inv.astype(np.int32)
        return rows, pool_keys, self.row_values(pool_keys)

    def store(self, pool_keys, pool_rows):
        """Write updated row values back (after an oracle row update)."""
        for k, r in zip(np.asarray(pool_keys).tolist(), np.asarray(pool_rows)):
            self.vals[int(k)] = np.array(r, dtype=np.float32)
