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


class KVModel:
    def __init__(self, num_blocks, max_seqs, max_blocks_per_seq, alloc_seed=0):
        self.num_blocks = num_blocks
        self.max_seqs = max_seqs
        self.max_blocks_per_seq = max_blocks_per_seq
        self.free = free_list_order(num_blocks, alloc_seed)
        self.table = [[] for _ in range(max_seqs)]
        self.seq_len = [0] * max_seqs
        self.store = [[] for _ in range(max_seqs)]

    # -- queries ---------------------------------------------------------
    def blocks_needed(self, length):
        return math.ceil(length / BLOCK)

    def live_table(self, s):
        """Blocks that hold positions below seq_len (the part reads can reach)."""
        return list(self.table[s][: self.blocks_needed(self.seq_len[s])])

    def slot_of(self, s, p):
        """Physical (block, slot) of logical position p of sequence s."""
        return self.table[s][p // BLOCK], p % BLOCK

    def contents(self, s):
        """Logical payloads at positions 0..seq_len-1."""
        return list(self.store[s][: self.seq_len[s]])

    # -- mutations -------------------------------------------------------
    def append(self, seqs, payloads):
        """Append payloads[i] (a list, one entry per new token) to seqs[i]."""
        if len(seqs) != len(payloads):
            return EINVAL
        need = []
        seen = set()
        for s, items in zip(seqs, payloads):  # entries checked in call order
            if not (0 <= s < self.max_seqs):
                return ENOSEQ
            if s in seen:
                return EINVAL
            seen.add(s)
            total = self.blocks_needed(self.seq_len[s] + len(items))
            if total > self.max_blocks_per_seq:
                return ERANGE
            need.append(max(0, total - len(self.table[s])))
        if sum(need) > len(self.free):
            return ENOMEM
        for s, items, k in zip(seqs, payloads, need):
            for _ in range(k):
                self.table[s].append(self.free.pop(0))
            base = self.seq_len[s]
            for i, item in enumerate(items):
                p = base + i
                if p < len(self.store[s]):
                    self.store[s][p] = item
                else:
                    self.store[s].append(item)
            self.seq_len[s] = base + len(items)
        return OK

    def rollback(self, s, r):
        if not (0 <= s < self.max_seqs):
            return ENOSEQ
        if r < 0:
            return EINVAL
        if r > self.seq_len[s]:
            return ERANGE
        self.seq_len[s] -= r
        return OK

    def free_seq(self, s):
        if not (0 <= s < self.max_seqs):
            return ENOSEQ
        for b in reversed(self.table[s]):
            self.free.insert(0, b)
        self.table[s] = []
        self.seq_len[s] = 0
        self.store[s] = []
        return OK
