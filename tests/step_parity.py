"""Helpers of the pa_decode_step parity tests: a fixed decode batch held
by the oracle's allocator and cache (oracle/allocator.py, oracle/cache.py)
with a device twin of its cache and block tables, and the pinned metadata
buffer a step reads."""
import numpy as np
import torch

import workloads
from oracle import allocator as oa
from oracle import attention as oat
from oracle import cache as oc
from oracle import codecs
from paged_kv_cache_host_amd.engine import to_device_raw

DEV = "cuda"
KS, VS = 0.03, 0.05      # fp8 per-tensor scales (ignored by a bf16 cache)


def _blocks(n):
    return -(-int(n) // 16)


class StepBatch:
    """A fixed decode batch held by the oracle's allocator and cache, with a
    device twin of the cache and tables.  Sequence s starts with lengths[s]
    cached tokens; each iteration appends one token to every sequence."""

    def __init__(self, seed, lengths, h_q, h_kv, d, cache_dt, steps, extra_blocks=6):
        self.rng = np.random.default_rng(seed)
        self.lengths = np.asarray(lengths, dtype=np.int64)
        self.S, self.h_q, self.h_kv, self.d, self.cache_dt = len(lengths), h_q, h_kv, d, cache_dt
        self.mb = _blocks(self.lengths.max() + steps)
        self.nb = int(sum(_blocks(L + steps) for L in self.lengths)) + extra_blocks
        order = self.rng.permutation(self.nb).astype(np.int32)
        self.pool = oa.BlockPool(self.nb, 16, order.tolist())
        self.kc, self.vc = oc.new_cache(self.nb, h_kv, 16, d, cache_dt)
        for s, L in enumerate(self.lengths.tolist()):
            assert self.pool.seq_create(s, int(L)) == oa.OK
            if L:
                k = workloads.normal_raw(self.rng, (L, h_kv, d), "bf16")
                v = workloads.normal_raw(self.rng, (L, h_kv, d), "bf16")
                oc.cache_write(self.kc, self.vc, k, v, self.pool.slots(s, 0, L), "bf16",
                               cache_dt, KS, VS)
        self.k_dev = to_device_raw(self.kc, cache_dt, DEV)
        self.v_dev = to_device_raw(self.vc, cache_dt, DEV)
        tables, _ = self.pool.pack(range(self.S), self.mb)
        self.tab_dev = torch.from_numpy(np.asarray(tables, dtype=np.int32)).to(DEV)
        self.lens = self.lengths.astype(np.int32).copy()
        self.sm = 1.0 / np.sqrt(d)

    def next_tokens(self):
        """Append one token per sequence (oracle allocator); returns the
        slots and the new tokens' raw K, V, Q."""
        slots = []
        for s in range(self.S):
            st, sl = self.pool.seq_append(s, 1)
            assert st == oa.OK
            slots += sl
        self.lens += 1
        k = workloads.normal_raw(self.rng, (self.S, self.h_kv, self.d), "bf16")
        v = workloads.normal_raw(self.rng, (self.S, self.h_kv, self.d), "bf16")
        q = workloads.normal_raw(self.rng, (self.S, self.h_q, self.d), "bf16")
        return np.asarray(slots, dtype=np.int32), k, v, q

    def oracle_step(self, slots, k, v, q):
        oc.cache_write(self.kc, self.vc, k, v, slots, "bf16", self.cache_dt, KS, VS)
        tables, _ = self.pool.pack(range(self.S), self.mb)
        tables = np.asarray(tables, dtype=np.int32)
        out = oat.decode(codecs.decode(q, "bf16"), self.kc, self.vc, tables, self.lens, self.h_kv,
                         self.sm, self.cache_dt, KS, VS)
        return out, tables


def _meta(S, slots, lens, pad):
    """Pinned metadata buffer: `pad` filler words, the slots, the lengths,
    then filler again (the staged copy must reproduce all of it)."""
    words = pad + 2 * S + 3
    host = torch.empty(words, dtype=torch.int32, pin_memory=True)
    h = host.numpy()
    h[:] = -12345
    h[pad:pad + S] = slots
    h[pad + S:pad + 2 * S] = lens
    return host, 4 * pad, 4 * (pad + S), 4 * words


