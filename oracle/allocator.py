"""Block pool, per-sequence block tables and slot mapping (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows the ARTICLE, §2.2 (block manager): the pool starts with every block
id free, in the order ``0 .. num_blocks-1`` unless another order is given;
``allocate(n)`` takes the first ``n`` ids of the free list and fails when
fewer than ``n`` are free (the comparison operator is lost in the printed
text; "fewer than" is the only reading under which the allocation that
follows can succeed); ``free(ids)`` appends the ids to the back of the list in
the order given.

The LESSON ("The Concept: PagedAttention as a virtual memory system") fixes
the rest: a sequence's table maps logical token position p to a physical
block; the token lives in block ``table[p // block_size]`` at offset
``p % block_size``; when a sequence grows past its blocks, one more block is
added; when it finishes, its blocks go back to the pool.

Readings taken where the texts are silent or contradict themselves:
* the ARTICLE raises an error on shortage but its scheduler (§3.1) tests the
  result for emptiness: here every allocation is all-or-nothing and a failed
  call leaves the pool and the table untouched (status ``NO_BLOCKS``);
* the ARTICLE's ``get_block_table`` reads a map that is never defined: here
  the pool keeps one table per sequence id;
* a sequence is created with ``ceil(num_tokens / block_size)`` blocks (the
  ARTICLE's scheduler, §3.1, allocates that many for a prompt at admission);
* release returns the table to the back of the free list in table order.

Prefix sharing (ARTICLE §4.3: requests with the same system-prompt prefix
reuse one set of KV blocks, marked read-only).  Readings taken:
* only FULL blocks are shared: a sequence created from a prefix of another
  takes that sequence's first ``shared_tokens // block_size`` blocks, and the
  rest of its tokens (including the part of the prefix that fills a partial
  block) go to fresh blocks, so no sequence ever writes into a shared block;
* a block is counted once for every table that holds it and returns to the
  back of the free list when the last table holding it is released (in that
  table's order).

Prefix detection (ARTICLE §4.3 names the prefix-match detection as the
scheduler's added work; it gives no algorithm).  Readings taken:
* a block can be found only after the caller declares its K/V computed
  (``seq_register_prefix``); it is found by its content: the block before it
  in the registering sequence's table (none for a first block) and its
  ``block_size`` token ids, so a match of block i implies a match of every
  earlier position;
* a new sequence (``seq_create_prefix``) takes matched blocks from its first
  full block on and stops at the first full block whose content is not
  registered; the rest of its blocks are fresh, exactly as ``seq_share``;
* content already registered for another block is not registered again
  (registration of that sequence stops there); a block leaves the index when
  it returns to the free list.

Prefix retention (an extension, off by default: the pages reuse a prefix
among running requests).  Read as follows: a registered block whose last
holder lets go is retained, still found by its content, instead of joining
the free list (the blocks one release retains enter deepest first, i.e. in
reverse table order, so a chain is evicted from its tail); retained blocks
count as free; fresh blocks are taken from the
free list first and then from the retained blocks, oldest release first,
each leaving the index as it is taken; a lookup that finds a retained block
brings it back into use; the free list as listed is the free list followed
by the retained blocks in that order; turning retention off moves the
retained blocks, oldest first, to the back of the free list and out of the
index.
"""
from __future__ import annotations

from collections import OrderedDict, deque

OK = 0
ERR_INVALID = -1
ERR_NO_BLOCKS = -2
ERR_UNKNOWN_SEQ = -3
ERR_EXISTS = -4


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)


class BlockPool:
    def __init__(self, num_blocks: int, block_size: int, initial_free_order=None):
        if num_blocks < 0 or block_size <= 0:
            raise ValueError("bad pool geometry")
        self.num_blocks = int(num_blocks)
        self.block_size = int(block_size)
        if initial_free_order is None:
            order = list(range(self.num_blocks))
        else:
            order = [int(b) for b in initial_free_order]
            if sorted(order) != list(range(self.num_blocks)):
                raise ValueError("initial free order must be a permutation of the pool")
        self.free = deque(order)
        self.tables: dict[int, list[int]] = {}
        self.lengths: dict[int, int] = {}
        self.refs = [0] * self.num_blocks   # tables holding each block
        self.index: dict = {}               # (previous block, token ids) -> block
        self.content: dict = {}             # block -> its key in the index
        self.retain = False                 # prefix retention
        self.retained = OrderedDict()       # retained blocks, oldest release first

    # -- ARTICLE §2.2: allocate / free ---------------------------------------
    def _unregister(self, b: int):
        key = self.content.pop(b, None)
        if key is not None:
            del self.index[key]

    def _take(self, n: int):
        if self.num_free() < n:
            return None
        ids = []
        for _ in range(n):
            if self.free:
                b = self.free.popleft()
            else:
                b, _ = self.retained.popitem(last=False)
                self._unregister(b)
            ids.append(b)
        for b in ids:
            self.refs[b] = 1
        return ids

    def _give_back(self, ids):
        kept = []
        for b in ids:
            self.refs[b] -= 1
            if self.refs[b] == 0:
                if self.retain and b in self.content:
                    kept.append(b)
                    continue
                self._unregister(b)
                self.free.append(b)
        for b in reversed(kept):      # deepest first: chains are evicted from the tail
            self.retained[b] = None

    def set_prefix_retention(self, on: bool):
        self.retain = bool(on)
        if not self.retain:
            for b in list(self.retained):
                self._unregister(b)
                self.free.append(b)
            self.retained.clear()
        return OK

    def num_retained(self) -> int:
        return len(self.retained)

    # -- sequence-level verbs -------------------------------------------------
    def num_free(self) -> int:
        return len(self.free) + len(self.retained)

    def seq_create(self, seq: int, num_tokens: int) -> int:
        if num_tokens < 0:
            return ERR_INVALID
        if seq in self.tables:
            return ERR_EXISTS
        ids = self._take(ceil_div(num_tokens, self.block_size))
        if ids is None:
            return ERR_NO_BLOCKS
        self.tables[seq] = ids
        self.lengths[seq] = num_tokens
        return OK

    def seq_share(self, seq: int, src: int, shared_tokens: int, num_tokens: int):
        """Create ``seq`` with ``num_tokens`` tokens whose first
        ``shared_tokens`` are those of ``src`` (ARTICLE §4.3): the full blocks
        among them are shared, the rest is fresh.  Returns (status, number of
        leading tokens that live in shared blocks)."""
        if seq in self.tables:
            return ERR_EXISTS, 0
        if src not in self.tables:
            return ERR_UNKNOWN_SEQ, 0
        if not (0 <= shared_tokens <= self.lengths[src]) or num_tokens < shared_tokens:
            return ERR_INVALID, 0
        n_shared = shared_tokens // self.block_size
        fresh = self._take(ceil_div(num_tokens, self.block_size) - n_shared)
        if fresh is None:
            return ERR_NO_BLOCKS, 0
        head = self.tables[src][:n_shared]
        for b in head:
            self.refs[b] += 1
        self.tables[seq] = head + fresh
        self.lengths[seq] = num_tokens
        return OK, n_shared * self.block_size

    # -- ARTICLE §4.3: prefix detection ---------------------------------------
    def seq_register_prefix(self, seq: int, tokens) -> int:
        """Declare the K/V of positions 0 .. len(tokens)-1 of ``seq`` computed,
        holding these token ids: index each full block among them by its
        content."""
        if seq not in self.tables:
            return ERR_UNKNOWN_SEQ
        tokens = [int(t) for t in tokens]
        if len(tokens) > self.lengths[seq]:
            return ERR_INVALID
        table, bs = self.tables[seq], self.block_size
        keys = []
        for i in range(len(tokens) // bs):
            keys.append((table[i - 1] if i else -1, tuple(tokens[i * bs:(i + 1) * bs])))
        for b, key in zip(table, keys):
            if b in self.content and self.content[b] != key:
                return ERR_INVALID
        for b, key in zip(table, keys):
            if key in self.index:
                if self.index[key] == b:
                    continue
                break
            self.index[key] = b
            self.content[b] = key
        return OK

    def seq_create_prefix(self, seq: int, tokens):
        """Create ``seq`` for the prompt ``tokens``, sharing the leading full
        blocks whose content is registered.  Returns (status, tokens that live
        in shared blocks)."""
        tokens = [int(t) for t in tokens]
        if seq in self.tables:
            return ERR_EXISTS, 0
        bs = self.block_size
        matched, parent = [], -1
        for i in range(len(tokens) // bs):
            b = self.index.get((parent, tuple(tokens[i * bs:(i + 1) * bs])))
            if b is None:
                break
            matched.append(b)
            parent = b
        # matched blocks nobody holds (retained) come back into use: they
        # are not available as fresh blocks
        idle = [b for b in matched if self.refs[b] == 0]
        if ceil_div(len(tokens), bs) - len(matched) > self.num_free() - len(idle):
            return ERR_NO_BLOCKS, 0
        for b in idle:
            del self.retained[b]
        fresh = self._take(ceil_div(len(tokens), bs) - len(matched))
        assert fresh is not None
        for b in matched:
            self.refs[b] += 1
        self.tables[seq] = matched + fresh
        self.lengths[seq] = len(tokens)
        return OK, len(matched) * bs

    def match_prefix(self, tokens, with_retained: bool = False):
        """Tokens of the leading full blocks of ``tokens`` whose content is
        registered (the walk of ``seq_create_prefix``, nothing taken)[, and
        how many of those blocks are retained rather than held]."""
        tokens = [int(t) for t in tokens]
        bs = self.block_size
        n, idle, parent = 0, 0, -1
        for i in range(len(tokens) // bs):
            b = self.index.get((parent, tuple(tokens[i * bs:(i + 1) * bs])))
            if b is None:
                break
            n += 1
            idle += self.refs[b] == 0
            parent = b
        return (n * bs, idle) if with_retained else n * bs

    def num_registered(self) -> int:
        return len(self.content)

    def block_refs(self, block: int) -> int:
        return self.refs[block]

    def seq_append(self, seq: int, n_new: int):
        """Grow a sequence by ``n_new`` tokens, taking one block per block
        boundary crossed.  Returns (status, slots of the new tokens)."""
        if n_new < 0:
            return ERR_INVALID, []
        if seq not in self.tables:
            return ERR_UNKNOWN_SEQ, []
        old = self.lengths[seq]
        need = ceil_div(old + n_new, self.block_size) - len(self.tables[seq])
        if need > 0:
            ids = self._take(need)
            if ids is None:
                return ERR_NO_BLOCKS, []
            self.tables[seq].extend(ids)
        self.lengths[seq] = old + n_new
        return OK, self.slots(seq, old, n_new)

    def seq_release(self, seq: int) -> int:
        if seq not in self.tables:
            return ERR_UNKNOWN_SEQ
        self._give_back(self.tables.pop(seq))
        del self.lengths[seq]
        return OK

    def block_table(self, seq: int) -> list[int]:
        return list(self.tables[seq])

    def slots(self, seq: int, start: int, n: int) -> list[int]:
        """Flat slot index ``block * block_size + offset`` of positions
        ``start .. start+n-1``."""
        t = self.tables[seq]
        bs = self.block_size
        return [t[p // bs] * bs + p % bs for p in range(start, start + n)]

    def pack(self, seqs, max_blocks: int):
        """Dense ``[len(seqs), max_blocks]`` table padded with -1, and the
        context length of each sequence."""
        tables = []
        lens = []
        for s in seqs:
            t = self.tables[s]
            if len(t) > max_blocks:
                raise ValueError("table wider than max_blocks")
            tables.append(t + [-1] * (max_blocks - len(t)))
            lens.append(self.lengths[s])
        return tables, lens

    def free_list(self) -> list[int]:
        """The free list, then the retained blocks, oldest release first."""
        return list(self.free) + list(self.retained)
