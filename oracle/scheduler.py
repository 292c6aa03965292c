"""Iteration-level continuous batching with chunked prefill (oracle side).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Policy, from the two texts:
* LESSON, "Continuous batching at the iteration level" and "What the
  scheduler looks like": the scheduler runs once per iteration; sequences
  that reached their end leave RUNNING and release their blocks; waiting
  sequences are admitted in arrival order while the head of the queue fits
  in the free blocks; every RUNNING sequence then contributes either a
  prefill slice or exactly one decode token to one batch.
* LESSON, "Chunked prefill": prefill is cut into fixed-size slices (512
  tokens by default), each scheduled as a unit, interleaved with decodes.
* ARTICLE §3.1 (continuous batching): running sequences that need one more
  block take it first; if none is free the sequence is preempted -- its
  blocks are freed, its computed-token count reset to zero and it goes to the
  back of the waiting queue; admission is capped by a maximum number of
  running sequences and allocates ``ceil(prompt_len / block_size)`` blocks at
  once; a sequence that does not fit goes back to the front of the queue and
  admission stops.
* ARTICLE §3.2: a preempted sequence is recovered by recomputation: it
  prefills again every token it knows (prompt plus the output produced so
  far) before decoding resumes.

Readings taken where the texts leave a step open:
* order inside one iteration: (1) arrivals join the queue, (2) finished
  sequences are released, (3) decode-phase sequences grow by one token each,
  in RUNNING order, preempting on shortage, (4) admission, (5) prefill slices
  are handed out in RUNNING order until the per-iteration prefill budget is
  spent;
* the prefill slice that completes a sequence's known tokens produces its
  next output token; the sequence decodes from the next iteration on; a
  decode step appends the newest output token (its K/V written, context
  grows by one) and produces the next;
* a sequence is finished once it has produced its target number of output
  tokens; it is released at the start of the following iteration.

The other three schedules of the LESSON's simulator ("Use It": one request
at a time; padded static batches; iteration-level admission and release
without chunking), read as follows:
* ``continuous``: as above, except that a prompt is prefilled whole in the
  iteration that admits it, so the head of the queue is admitted only if its
  known tokens fit the budget still unspent in this iteration (or nothing
  has been prefilled in it yet: a prompt longer than the whole budget then
  runs in budget-sized slices);
* ``static``: a new batch is taken only when nothing runs: heads of the
  queue in order, as long as (members x longest known length) stays within
  the budget (the first member always) and that many padded blocks are
  free; each member is padded to the longest (the padding sits before the
  output, in the cache) and the batch is prefilled at once; a member that
  reached its target keeps decoding padding until every member has, and the
  batch leaves together;
* ``naive``: ``static`` with one request per batch.

Prefix caching (ARTICLE §4.3 names prefix sharing and the detection of a
shared prefix, not its mechanics; ``chunked`` only), read as follows: a
request may carry its prompt's token ids; at admission the leading full
blocks of the prompt without its last token are looked up by content (the
allocator's index: the block before and the block's ids), the request fits
if the free list holds the blocks it needs beyond those, it is created
sharing them, and its prefill starts after them (the last prompt token is
always computed: its slice yields the first output token); a re-admitted
request does the same for its prompt and then grows to every token it
knows.  A sequence's full prompt blocks are registered at the start of the
step after the one whose slices complete them (their K/V are then in the
cache).
"""
from __future__ import annotations

from dataclasses import dataclass, field

from .allocator import BlockPool, OK, ERR_NO_BLOCKS, ceil_div


@dataclass
class Seq:
    sid: int
    prompt_len: int
    target: int               # output tokens to produce (>= 1)
    known: int = 0            # tokens to prefill on (re)admission
    prefilled: int = 0        # of ``known``, tokens whose K/V are cached
    decoded: int = 0          # output tokens produced so far
    in_prefill: bool = True
    preemptions: int = 0
    padding: int = 0          # static batches: padding tokens before the output
    ids: list | None = None   # the prompt's token ids (prefix caching)
    reg_blocks: int = 0       # leading blocks of the current table registered

    def cached_len(self) -> int:
        if self.in_prefill:
            return self.prefilled
        return self.prompt_len + self.padding + self.decoded - 1


@dataclass
class Batch:
    decode: list = field(default_factory=list)    # (sid, position, slot)
    prefill: list = field(default_factory=list)   # (sid, start, n, slots)
    emits: list = field(default_factory=list)     # per slice: yields a token
    finished: list = field(default_factory=list)
    admitted: list = field(default_factory=list)
    preempted: list = field(default_factory=list)


class Scheduler:
    MODES = ("chunked", "continuous", "static", "naive")

    def __init__(self, pool: BlockPool, max_running: int = 256, prefill_budget: int = 512,
                 mode: str = "chunked"):
        if mode not in self.MODES:
            raise ValueError(mode)
        self.mode = mode
        self.pool = pool
        self.max_running = max_running
        self.prefill_budget = prefill_budget
        self.waiting: list[Seq] = []
        self.running: list[Seq] = []
        self.done: list[Seq] = []
        self.prefix_hits = 0      # prompt tokens found shared at admission

    def add(self, sid: int, prompt_len: int, target: int):
        if prompt_len < 1 or target < 1:
            raise ValueError("prompt and target must be positive")
        self.waiting.append(Seq(sid, prompt_len, target, known=prompt_len))

    def add_prompt(self, sid: int, prompt_len: int, target: int, ids):
        """A request with its prompt's token ids (prefix caching)."""
        if self.mode != "chunked":
            raise ValueError("prefix caching needs the chunked schedule")
        ids = [int(t) for t in ids]
        if len(ids) != prompt_len:
            raise ValueError("one token id per prompt position")
        self.add(sid, prompt_len, target)
        self.waiting[-1].ids = ids

    def _preempt(self, s: Seq):
        self.pool.seq_release(s.sid)
        s.preemptions += 1
        s.in_prefill = True
        s.prefilled = 0
        s.reg_blocks = 0
        s.known = s.prompt_len + s.padding + s.decoded
        self.waiting.append(s)

    def _prefill(self, out: Batch, seqs, budget: int) -> int:
        """Hands out slices to the prefill-phase sequences of ``seqs`` in
        order; returns the budget left."""
        for s in seqs:
            if not s.in_prefill or budget == 0:
                continue
            n = min(s.known - s.prefilled, budget)
            if n <= 0:
                continue
            slots = self.pool.slots(s.sid, s.prefilled, n)
            out.prefill.append((s.sid, s.prefilled, n, slots))
            s.prefilled += n
            budget -= n
            done = s.prefilled == s.known
            out.emits.append(done)
            if done:
                s.in_prefill = False
                s.decoded += 1
        return budget

    def _admit(self, out: Batch, s: Seq):
        st = self.pool.seq_create(s.sid, s.known)
        assert st == OK
        self.waiting.pop(0)
        self.running.append(s)
        out.admitted.append(s.sid)

    def _admit_prefix(self, out: Batch, s: Seq) -> bool:
        """Admission of a request with token ids; False if it does not fit."""
        bs = self.pool.block_size
        head = s.ids[:s.prompt_len - 1]          # the last prompt token is always computed
        matched, idle = self.pool.match_prefix(head, with_retained=True)
        # matched blocks that are retained rather than held count as free but
        # come back into use: they are not fresh blocks
        if self.pool.num_free() - idle < ceil_div(s.known, bs) - matched // bs:
            return False
        st, shared = self.pool.seq_create_prefix(s.sid, head)
        assert st == OK and shared == matched
        st, _ = self.pool.seq_append(s.sid, s.known - len(head))
        assert st == OK
        s.prefilled = shared
        s.reg_blocks = shared // bs
        self.prefix_hits += shared
        self.waiting.pop(0)
        self.running.append(s)
        out.admitted.append(s.sid)
        return True

    def _register_computed(self):
        """(1') Prompt blocks completed by the last step's slices (their K/V
        are in the cache now) join the allocator's index."""
        bs = self.pool.block_size
        for s in self.running:
            if s.ids is None:
                continue
            nb = min(s.prefilled, s.prompt_len) // bs
            if nb > s.reg_blocks:
                assert self.pool.seq_register_prefix(s.sid, s.ids[:nb * bs]) == OK
                s.reg_blocks = nb

    def step(self) -> Batch:
        out = Batch()
        bs = self.pool.block_size
        static = self.mode in ("static", "naive")
        self._register_computed()
        # (2) release finished sequences; a static batch only all at once
        over = [not s.in_prefill and s.decoded >= s.target for s in self.running]
        if static and not all(over):
            over = [False] * len(self.running)
        keep = []
        for s, f in zip(self.running, over):
            if f:
                self.pool.seq_release(s.sid)
                out.finished.append(s.sid)
                self.done.append(s)
            else:
                keep.append(s)
        self.running = keep
        # (3) one decode token per decode-phase sequence, preempting on shortage
        keep = []
        for s in self.running:
            if s.in_prefill:
                keep.append(s)
                continue
            st, slots = self.pool.seq_append(s.sid, 1)
            if st == ERR_NO_BLOCKS:
                self._preempt(s)
                out.preempted.append(s.sid)
                continue
            assert st == OK
            out.decode.append((s.sid, s.cached_len(), slots[0]))
            s.decoded += 1
            keep.append(s)
        self.running = keep
        # (4) admission and (5) prefill slices within the budget
        budget = self.prefill_budget
        if self.mode == "chunked":
            while self.waiting and len(self.running) < self.max_running:
                s = self.waiting[0]
                if s.ids is not None:
                    if not self._admit_prefix(out, s):
                        break
                    continue
                if self.pool.num_free() < ceil_div(s.known, bs):
                    break
                self._admit(out, s)
            self._prefill(out, self.running, budget)
        elif self.mode == "continuous":
            budget = self._prefill(out, self.running, budget)
            while self.waiting and len(self.running) < self.max_running:
                s = self.waiting[0]
                if self.pool.num_free() < ceil_div(s.known, bs):
                    break
                if s.known > budget and budget < self.prefill_budget:
                    break
                self._admit(out, s)
                budget = self._prefill(out, [s], budget)
        else:
            if not self.running:
                size = 1 if self.mode == "naive" else self.max_running
                members = []
                for s in self.waiting[:size]:
                    width = max([m.known for m in members] + [s.known])
                    n = len(members) + 1
                    if members and n * width > self.prefill_budget:
                        break
                    if n * ceil_div(width, bs) > self.pool.num_free():
                        break
                    members.append(s)
                if members:
                    width = max(m.known for m in members)
                    for s in members:
                        s.padding += width - s.known
                        s.known = width
                        self._admit(out, s)
            self._prefill(out, self.running, budget)
        return out

    # -- accounting -------------------------------------------------------
    def held(self):
        """(blocks held, tokens assigned, reserved-unwritten prompt slots)."""
        blocks = 0
        assigned = 0
        unwritten = 0
        for s in self.running:
            blocks += len(self.pool.tables[s.sid])
            assigned += self.pool.lengths[s.sid]
            if s.in_prefill:
                unwritten += s.known - s.prefilled
        return blocks, assigned, unwritten
