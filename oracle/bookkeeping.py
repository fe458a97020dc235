"""Model of the KV block manager: free list, per-sequence block tables,
seq_len, append by slice-update and O(1) rollback.

Sources:
* AX Engine page, "Core Technical Architecture & Methods": the KV manager is
  deterministic and synchronous; the cache grows by slice-updates into
  preallocated buffers; a rejected speculation is undone in O(1) by moving the
  sequence-length pointer only.
* mlx-engine blog ("Improving LM Studio's MLX engine for agentic workflows"),
  prompt-caching section: the cache is handled in 256-token blocks.
* same blog, section on current model architectures: a cache must be able to
  rewind to an earlier length before new tokens are appended.

Readings where the pages are silent:
* blocks hold 256 token positions; sequence s owns blocks table[s][0..owned);
  position p lives in block table[s][p // 256], slot p % 256.
* an append of n tokens needs ceil((seq_len + n) / 256) blocks in all; the
  missing ones are popped from the front of the free list, in order.  A
  multi-sequence append is all-or-nothing: if the pool cannot cover every
  sequence in the call, nothing changes and ENOMEM is returned.  Entries are
  validated in call order and the first bad one decides the status (bad id:
  ENOSEQ; repeated id: EINVAL; table overflow: ERANGE); ENOMEM comes last.
* rollback r requires 0 <= r <= seq_len and only moves seq_len; the blocks stay
  owned and the next append overwrites the rolled-back slots.
* freeing a sequence pushes its blocks back onto the front of the free list in
  reverse ownership order, so its first block is the next one handed out.

Ring caches for sliding-window layers (the same blog's 512-token local
layers; the window bounds what a layer can ever read again).  With window W
a sequence keeps only the blocks holding its last W + H positions, H = 8
(the most rows one verify call appends, so the rows just appended can still
be verified and rolled back):
* after an append to length L, blocks wholly below position
  max(0, L - H - W + 1) are released (table entry -1) and pushed onto the
  front of the free list in increasing index order, before the entry's new
  blocks are popped; positions in released blocks are never stored again;
* a rollback to length L' must keep every position a later window can see:
  max(0, L' - W + 1) >= the first kept position, else ERANGE;
* freeing a sequence returns only its kept blocks (same order rule).

The logical store keeps, per sequence, one payload per position (whatever the
caller appended: K/V rows or encoded records), without any paging, so paging
mistakes on the other side show up as mismatches.
"""

import math

from .splitmix import free_list_order

OK = 0
EINVAL = -1
ENOMEM = -2
ERANGE = -3
ENOSEQ = -4

BLOCK = 256
HISTORY = 8  # positions kept beyond the window in a ring cache


class KVModel:
    def __init__(self, num_blocks, max_seqs, max_blocks_per_seq, alloc_seed=0, ring_window=0):
        self.num_blocks = num_blocks
        self.max_seqs = max_seqs
        self.max_blocks_per_seq = max_blocks_per_seq
        self.ring_window = ring_window
        self.free = free_list_order(num_blocks, alloc_seed)
        self.table = [[] for _ in range(max_seqs)]  # -1: released (ring caches)
        self.first = [0] * max_seqs  # index of the first kept block
        self.seq_len = [0] * max_seqs
        self.store = [[] for _ in range(max_seqs)]

    # -- queries ---------------------------------------------------------
    def blocks_needed(self, length):
        return math.ceil(length / BLOCK)

    def live_table(self, s):
        """Table entries of the blocks below seq_len (-1 where a ring cache
        released the block)."""
        return list(self.table[s][: self.blocks_needed(self.seq_len[s])])

    def kept_blocks(self, s):
        return [b for b in self.table[s][self.first[s]:] if b >= 0]

    def first_position(self, s):
        return self.first[s] * BLOCK

    def slot_of(self, s, p):
        """Physical (block, slot) of logical position p of sequence s."""
        return self.table[s][p // BLOCK], p % BLOCK

    def contents(self, s):
        """Logical payloads at positions 0..seq_len-1."""
        return list(self.store[s][: self.seq_len[s]])

    def _keep_from(self, s, length):
        """First block a ring cache must keep at this length."""
        if not self.ring_window:
            return self.first[s]
        return max(self.first[s], max(0, length - HISTORY - self.ring_window + 1) // BLOCK)

    # -- mutations -------------------------------------------------------
    def append(self, seqs, payloads):
        """Append payloads[i] (a list, one entry per new token) to seqs[i]."""
        if len(seqs) != len(payloads):
            return EINVAL
        seen = set()
        for s, items in zip(seqs, payloads):  # entries checked in call order
            if not (0 <= s < self.max_seqs):
                return ENOSEQ
            if s in seen:
                return EINVAL
            seen.add(s)
            if self.blocks_needed(self.seq_len[s] + len(items)) > self.max_blocks_per_seq:
                return ERANGE
        # all or nothing: walk the entries on a copy of the free list first
        free = list(self.free)
        for s, items in zip(seqs, payloads):
            new_len = self.seq_len[s] + len(items)
            keep = self._keep_from(s, new_len)
            for i in range(self.first[s], min(keep, len(self.table[s]))):
                if self.table[s][i] >= 0:
                    free.insert(0, self.table[s][i])
            need = self.blocks_needed(new_len) - max(len(self.table[s]), keep)
            if need > len(free):
                return ENOMEM
            del free[: max(0, need)]
        for s, items in zip(seqs, payloads):
            new_len = self.seq_len[s] + len(items)
            keep = self._keep_from(s, new_len)
            row = self.table[s]
            for i in range(self.first[s], min(keep, len(row))):
                if row[i] >= 0:
                    self.free.insert(0, row[i])
                    row[i] = -1
            while len(row) < keep:
                row.append(-1)  # never held a block
            while len(row) < self.blocks_needed(new_len):
                row.append(self.free.pop(0))
            self.first[s] = keep
            base = self.seq_len[s]
            for i, item in enumerate(items):
                p = base + i
                if p < len(self.store[s]):
                    self.store[s][p] = item
                else:
                    self.store[s].append(item)
            self.seq_len[s] = new_len
        return OK

    def rollback(self, s, r):
        if not (0 <= s < self.max_seqs):
            return ENOSEQ
        if r < 0:
            return EINVAL
        if r > self.seq_len[s]:
            return ERANGE
        if self.ring_window and max(0, self.seq_len[s] - r - self.ring_window + 1) < self.first_position(s):
            return ERANGE  # a later window would reach a released block
        self.seq_len[s] -= r
        return OK

    def free_seq(self, s):
        if not (0 <= s < self.max_seqs):
            return ENOSEQ
        for b in reversed(self.kept_blocks(s)):
            self.free.insert(0, b)
        self.table[s] = []
        self.first[s] = 0
        self.seq_len[s] = 0
        self.store[s] = []
        return OK
