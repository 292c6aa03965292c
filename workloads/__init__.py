"""Seeded synthetic inputs for the paged-attention hot path.

This module only draws random inputs and rounds them to their storage
format; it holds none of the attention, allocation or quantisation
arithmetic.  Both sides of every parity check (the HIP library and the CPU
oracle) receive exactly the arrays produced here and nothing else.

The source pages measure a production serving trace on a 70B model; no
dataset is named and none is used.  These generators stand in for it with
the shapes of one attention layer of that model family: 64 query heads, 8 KV
heads, head dimension 128, 16-token blocks.

Draw order inside one workload: lengths, then the pool's initial free-order
permutation, then K, V and Q (each N(0, 1)).  Storage rounding (float32 to
bf16, round to nearest even) uses torch's CPU cast, a library primitive.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

BLOCK = 16

# Lognormal with mean 1500 and standard deviation 600 (the trace of the
# LESSON's fragmentation exercise): sigma^2 = ln(1 + (600/1500)^2),
# mu = ln(1500) - sigma^2 / 2.
LEN_SIGMA = math.sqrt(math.log(1.0 + (600.0 / 1500.0) ** 2))
LEN_MU = math.log(1500.0) - LEN_SIGMA ** 2 / 2.0
LEN_CAP = 8192


def to_bf16_bits(x_f32: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_raw(rng: np.random.Generator, shape, dtype: str, chunk: int = 1 << 24) -> np.ndarray:
    """N(0,1) values in raw storage of ``dtype`` ('f32' or 'bf16'), drawn in
    float32 in bounded chunks."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    for a in range(0, n, chunk):
        b = min(n, a + chunk)
        x = rng.standard_normal(b - a, dtype=np.float32)
        out[a:b] = x if dtype == "f32" else to_bf16_bits(x)
    return out.reshape(shape)


def lognormal_lengths(rng, n: int, mu=LEN_MU, sigma=LEN_SIGMA, cap=LEN_CAP) -> np.ndarray:
    return np.minimum(cap, np.ceil(rng.lognormal(mu, sigma, size=n))).astype(np.int64)


@dataclass
class DecodeWorkload:
    name: str
    lengths: np.ndarray          # [S] context length of each sequence (incl. the query token)
    num_blocks: int
    free_order: np.ndarray       # [num_blocks] int32, initial free-list order
    h_q: int
    h_kv: int
    d: int
    kv_dtype: str                # storage of the new K/V vectors ('f32' | 'bf16')
    cache_dtype: str             # storage of the cache ('f32' | 'bf16' | 'fp8')
    q_dtype: str
    k_tok: np.ndarray            # [sum L, H_kv, D] raw, sequence-major then position
    v_tok: np.ndarray
    q: np.ndarray                # [S, H_q, D] raw
    k_scale: float = 1.0
    v_scale: float = 1.0
    sm_scale: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return len(self.lengths)

    def token_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.lengths)]).astype(np.int64)


def _sm_scale(d: int) -> float:
    return float(np.float32(1.0) / np.float32(math.sqrt(d)))


def _amax_scale(raw_bf16: np.ndarray) -> float:
    """Per-tensor fp8 scale: largest magnitude / 448, in float32."""
    t = torch.from_numpy(raw_bf16.view(np.int16)).view(torch.bfloat16)
    amax = float(t.abs().max().float())
    return float(np.float32(amax) / np.float32(448.0))


def decode_layout(seed, lengths_fn, pool_fn):
    """The first draws of a decode workload: (lengths, pool size, free
    order), identical to those of ``decode_workload`` with the same seed."""
    rng = np.random.default_rng(seed)
    lengths = lengths_fn(rng)
    num_blocks = int(pool_fn(lengths))
    free_order = rng.permutation(num_blocks).astype(np.int32)
    return rng, lengths, num_blocks, free_order


def decode_workload(name, seed, lengths_fn, h_q, h_kv, d, kv_dtype, cache_dtype,
                    pool_fn, q_dtype=None, score_ramp: float = 0.0) -> DecodeWorkload:
    """``score_ramp`` > 0 (bf16 only): each query's scores climb along its
    context by about that many powers of two per 64 keys (the construction
    of ``prefill_workload``)."""
    rng, lengths, num_blocks, free_order = decode_layout(seed, lengths_fn, pool_fn)
    ntok = int(lengths.sum())
    k_tok = normal_raw(rng, (ntok, h_kv, d), kv_dtype)
    v_tok = normal_raw(rng, (ntok, h_kv, d), kv_dtype)
    q_dtype = q_dtype or kv_dtype
    q = normal_raw(rng, (len(lengths), h_q, d), q_dtype)
    if score_ramp > 0:
        assert kv_dtype == "bf16" and cache_dtype == "bf16" and q_dtype == "bf16"
        k_tok, q = _ramped(rng, [int(x) for x in lengths], len(lengths), h_q, h_kv, d,
                           score_ramp)
    w = DecodeWorkload(name, lengths, num_blocks, free_order, h_q, h_kv, d, kv_dtype,
                       cache_dtype, q_dtype, k_tok, v_tok, q, sm_scale=_sm_scale(d))
    if cache_dtype == "fp8":
        w.k_scale = _amax_scale(k_tok)
        w.v_scale = _amax_scale(v_tok)
    return w


def _ramped(rng, lengths, n_q: int, h_q: int, h_kv: int, d: int, ramp: float):
    """Raw bf16 K rows of sequences of ``lengths`` (concatenated) and ``n_q``
    raw bf16 Q rows whose scores climb along each sequence: every query of a
    KV head's group is one direction u (|u|^2 = d) plus noise, the key at
    position p is c(p) u plus noise, c(p) growing by ramp / (sqrt(d) log2 e)
    per 64 positions (about ``ramp`` powers of two per 64 keys once scaled
    by 1/sqrt(d))."""
    u = rng.standard_normal((h_kv, d)).astype(np.float32)
    u *= np.float32(math.sqrt(d)) / np.linalg.norm(u, axis=1, keepdims=True)
    step = ramp / (math.sqrt(d) * math.log2(math.e))
    pos = np.concatenate([np.arange(n) for n in lengths])
    c = (step * (pos // 64)).astype(np.float32)
    kf = c[:, None, None] * u[None] + \
        np.float32(0.1) * rng.standard_normal((len(pos), h_kv, d), dtype=np.float32)
    qf = np.repeat(u, h_q // h_kv, axis=0)[None] + \
        np.float32(0.1) * rng.standard_normal((n_q, h_q, d), dtype=np.float32)
    return to_bf16_bits(kf.astype(np.float32)), to_bf16_bits(qf.astype(np.float32))


def blocks_needed(lengths) -> int:
    return int(np.sum(-(-np.asarray(lengths, dtype=np.int64) // BLOCK)))


# ----------------------------------------------------------- the configs ---

def tiny_decode(seed: int = 1) -> DecodeWorkload:
    """4 sequences, 4 = 4 heads, D 64, fp32, lengths uniform in [1, 200],
    64-block pool in a random order."""
    return decode_workload(
        "tiny-decode-4seq-4h-d64-f32", seed,
        lambda rng: rng.integers(1, 201, size=4).astype(np.int64),
        4, 4, 64, "f32", "f32", lambda L: 64)


def decode_70b_layout(seed: int = 2, num_seqs: int = 128):
    """(lengths, pool size, free order) of ``decode_70b`` without its data."""
    _, lengths, nb, order = decode_layout(seed, lambda rng: lognormal_lengths(rng, num_seqs),
                                          lambda L: math.ceil(1.1 * blocks_needed(L)))
    return lengths, nb, order


def decode_70b(seed: int = 2, num_seqs: int = 128) -> DecodeWorkload:
    """128 sequences, 64/8 heads, D 128, bf16; lognormal lengths (mean 1500,
    sd 600, cap 8192); pool = all sequences' blocks plus 10% free."""
    return decode_workload(
        f"decode-70b-{num_seqs}seq-64q8kv-d128-bf16", seed,
        lambda rng: lognormal_lengths(rng, num_seqs),
        64, 8, 128, "bf16", "bf16", lambda L: math.ceil(1.1 * blocks_needed(L)))


def decode_fp8_long(seed: int = 4, num_seqs: int = 64, length: int = 8192) -> DecodeWorkload:
    """64 sequences x 8192 tokens, 64/8 heads, D 128, bf16 source values
    stored as fp8 e4m3fn with per-tensor scales; pool exactly the blocks
    needed, fully shuffled."""
    return decode_workload(
        f"decode-fp8-{num_seqs}seq-ctx{length}-64q8kv-d128", seed,
        lambda rng: np.full(num_seqs, length, dtype=np.int64),
        64, 8, 128, "bf16", "fp8", lambda L: blocks_needed(L), q_dtype="bf16")


@dataclass
class MixedWorkload:
    """One long prompt cut into prefill slices, interleaved with decodes."""
    name: str
    prompt_len: int
    chunk: int
    decode_lengths: np.ndarray   # [S_dec] context length at the first iteration
    num_blocks: int
    free_order: np.ndarray
    h_q: int
    h_kv: int
    d: int
    dtype: str
    prompt_k: np.ndarray         # [P, H_kv, D] raw
    prompt_v: np.ndarray
    prompt_q: np.ndarray         # [P, H_q, D] raw
    dec_k: np.ndarray            # [sum L0 + iters*S_dec, H_kv, D] decode-sequence K/V
    dec_v: np.ndarray
    dec_q: np.ndarray            # [iters, S_dec, H_q, D]
    sm_scale: float

    @property
    def iters(self) -> int:
        return self.prompt_len // self.chunk


def _mixed_layout(rng, prompt_len, chunk, num_decode):
    lengths = lognormal_lengths(rng, num_decode)
    iters = prompt_len // chunk
    need = prompt_len // BLOCK + blocks_needed(lengths + iters)
    num_blocks = math.ceil(1.1 * need)
    free_order = rng.permutation(num_blocks).astype(np.int32)
    return lengths, num_blocks, free_order


def mixed_prefill_layout(seed: int = 3, prompt_len: int = 32768, chunk: int = 512,
                         num_decode: int = 127):
    """(decode lengths, pool size, free order) of ``mixed_prefill`` without
    its data."""
    return _mixed_layout(np.random.default_rng(seed), prompt_len, chunk, num_decode)


def mixed_prefill(seed: int = 3, prompt_len: int = 32768, chunk: int = 512,
                  num_decode: int = 127) -> MixedWorkload:
    """A 32768-token prompt as 64 causal 512-token slices, each iteration also
    decoding one token for each of 127 sequences (lengths as the 70B decode
    workload, growing by one per iteration)."""
    rng = np.random.default_rng(seed)
    lengths, num_blocks, free_order = _mixed_layout(rng, prompt_len, chunk, num_decode)
    iters = prompt_len // chunk
    h_q, h_kv, d = 64, 8, 128
    prompt_k = normal_raw(rng, (prompt_len, h_kv, d), "bf16")
    prompt_v = normal_raw(rng, (prompt_len, h_kv, d), "bf16")
    n_dec_tok = int(lengths.sum()) + iters * num_decode
    dec_k = normal_raw(rng, (n_dec_tok, h_kv, d), "bf16")
    dec_v = normal_raw(rng, (n_dec_tok, h_kv, d), "bf16")
    prompt_q = normal_raw(rng, (prompt_len, h_q, d), "bf16")
    dec_q = normal_raw(rng, (iters, num_decode, h_q, d), "bf16")
    return MixedWorkload(f"mixed-prefill{prompt_len}-chunk{chunk}-dec{num_decode}-64q8kv-d128-bf16",
                         prompt_len, chunk, lengths, num_blocks, free_order, h_q, h_kv, d, "bf16",
                         prompt_k, prompt_v, prompt_q, dec_k, dec_v, dec_q, _sm_scale(d))


@dataclass
class TraceWorkload:
    """Arrivals of a continuous-batching trace: per iteration, a list of
    (sequence id, prompt length, output length)."""
    name: str
    iters: int
    arrivals: list
    num_blocks: int
    free_order: np.ndarray | None
    max_running: int = 256
    prefill_budget: int = 512


def trace(seed: int = 5, iters: int = 1000, lam: float = 0.5, prompt_median: float = 1000.0,
          prompt_sigma: float = 1.0, prompt_cap: int = 32768, out_mean: float = 256.0,
          num_blocks: int | None = None) -> TraceWorkload:
    """Poisson arrivals (rate ``lam`` per iteration), lognormal prompts
    (median 1000, sigma 1.0, cap 32768), geometric outputs (mean 256).  The
    default pool is 0.9 of 288 GB at 64 KiB per block (16 tokens x K and V x
    8 heads x 128 x bf16)."""
    rng = np.random.default_rng(seed)
    arrivals = []
    sid = 0
    for _ in range(iters):
        k = int(rng.poisson(lam))
        row = []
        for _ in range(k):
            p = int(min(prompt_cap, math.ceil(rng.lognormal(math.log(prompt_median), prompt_sigma))))
            o = int(rng.geometric(1.0 / out_mean))
            row.append((sid, max(1, p), o))
            sid += 1
        arrivals.append(row)
    if num_blocks is None:
        num_blocks = int(0.9 * 288e9) // (BLOCK * 2 * 8 * 128 * 2)
    return TraceWorkload(f"trace-{iters}it-lam{lam}", iters, arrivals, num_blocks, None)


def prefix_trace(seed: int = 9, iters: int = 1000, lam: float = 0.5, n_system: int = 8,
                 system_min: int = 512, system_max: int = 2048, user_median: float = 256.0,
                 user_sigma: float = 1.0, user_cap: int = 8192, out_mean: float = 256.0,
                 num_blocks: int = 200_000):
    """Requests behind shared system prompts: Poisson arrivals (``lam`` per
    iteration); each prompt is one of ``n_system`` system prompts (token
    ids drawn once, lengths uniform in [system_min, system_max]) followed by
    the request's own tokens (lognormal length, median 256, sigma 1.0, cap
    8192, ids drawn apart from the system prompts'); geometric outputs (mean
    256).  Returns (arrivals [[(id, prompt_len, output_len, ids)] per
    iteration], num_blocks)."""
    rng = np.random.default_rng(seed)
    systems = [rng.integers(0, 50000, int(rng.integers(system_min, system_max + 1))).astype(np.int32)
               for _ in range(n_system)]
    arrivals = []
    sid = 0
    for _ in range(iters):
        row = []
        for _ in range(int(rng.poisson(lam))):
            u = int(min(user_cap, math.ceil(rng.lognormal(math.log(user_median), user_sigma))))
            ids = np.concatenate([systems[int(rng.integers(0, n_system))],
                                  rng.integers(50000, 100000, max(1, u)).astype(np.int32)])
            o = int(rng.geometric(1.0 / out_mean))
            row.append((sid, len(ids), o, ids))
            sid += 1
        arrivals.append(row)
    return arrivals, num_blocks


def timed_requests(seed: int = 7, n: int = 256, rate_per_ms: float = 2.0,
                   prompt_median: float = 512.0, prompt_sigma: float = 1.2,
                   prompt_cap: int = 8192, out_mean: float = 64.0, out_cap: int = 512):
    """Requests on a time axis for serving-schedule comparisons: a Poisson
    process (``rate_per_ms`` arrivals per millisecond), lognormal prompts
    (median 512, sigma 1.2, cap 8192), geometric outputs (mean 64, cap 512).
    Returns [(arrival_ms, id, prompt_len, output_len)] in arrival order."""
    rng = np.random.default_rng(seed)
    gaps = rng.exponential(1.0 / rate_per_ms, n)
    t = np.cumsum(gaps) - gaps[0]
    out = []
    for i in range(n):
        p = int(min(prompt_cap, math.ceil(rng.lognormal(math.log(prompt_median), prompt_sigma))))
        o = int(min(out_cap, rng.geometric(1.0 / out_mean)))
        out.append((float(t[i]), i, max(1, p), o))
    return out


@dataclass
class PrefillWorkload:
    """Prompts whose K/V are all written, then attended by prefill slices
    (sequence, start position, length) in one call."""
    name: str
    prompts: np.ndarray          # [n_seq] prompt lengths
    slices: list                 # [(seq, start, n)]
    num_blocks: int
    free_order: np.ndarray
    h_q: int
    h_kv: int
    d: int
    kv_dtype: str
    cache_dtype: str
    q_dtype: str
    k_tok: np.ndarray            # [sum prompts, H_kv, D] raw, sequence-major
    v_tok: np.ndarray
    q_tok: np.ndarray            # [sum prompts, H_q, D] raw
    k_scale: float = 1.0
    v_scale: float = 1.0
    sm_scale: float = 0.0

    def token_offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.prompts)]).astype(np.int64)


def prefill_workload(name: str, seed: int, prompt_len: int | None = None, chunks=None,
                     prompts=None, slices=None, h_q: int = 64, h_kv: int = 8, d: int = 128,
                     dtype: str = "bf16", cache_dtype: str = "bf16",
                     extra_blocks: int = 9, score_ramp: float = 0.0) -> PrefillWorkload:
    """Either one prompt of ``prompt_len`` tokens cut into ``chunks`` (sizes),
    or several ``prompts`` with explicit ``slices``.

    ``score_ramp`` > 0 (bf16 only): scores that climb along each prompt by
    about that many powers of two per 64 keys.  Every query of a KV head's
    group is one direction u (|u|^2 = d) plus noise, the key at position p
    is c(p) u plus noise with c(p) growing by one step per 64 positions, so
    each new tile outweighs the ones before it."""
    if prompts is None:
        prompts = [prompt_len]
        slices = []
        start = 0
        for n in chunks:
            slices.append((0, start, n))
            start += n
        assert start <= prompt_len
    prompts = np.asarray(prompts, dtype=np.int64)
    rng = np.random.default_rng(seed)
    num_blocks = blocks_needed(prompts) + extra_blocks
    free_order = rng.permutation(num_blocks).astype(np.int32)
    ntok = int(prompts.sum())
    kvd = "bf16" if cache_dtype == "fp8" else dtype
    k_tok = normal_raw(rng, (ntok, h_kv, d), kvd)
    v_tok = normal_raw(rng, (ntok, h_kv, d), kvd)
    q_dtype = "bf16" if cache_dtype == "fp8" else dtype
    q_tok = normal_raw(rng, (ntok, h_q, d), q_dtype)
    if score_ramp > 0:
        assert dtype == "bf16" and cache_dtype == "bf16"
        k_tok, q_tok = _ramped(rng, [int(n) for n in prompts], ntok, h_q, h_kv, d, score_ramp)
    w = PrefillWorkload(name, prompts, list(slices), num_blocks, free_order, h_q, h_kv, d, kvd,
                        cache_dtype, q_dtype, k_tok, v_tok, q_tok, sm_scale=_sm_scale(d))
    if cache_dtype == "fp8":
        w.k_scale = _amax_scale(k_tok)
        w.v_scale = _amax_scale(v_tok)
    return w


def seq_token_rows(seed: int, sid: int, length: int, h_q: int, h_kv: int, d: int):
    """K, V (raw bf16 [length, h_kv, d]) and Q (raw bf16 [length, h_q, d]) of
    positions 0..length-1 of sequence ``sid``: per-sequence streams, so that a
    position's data does not depend on when it is scheduled."""
    rng = np.random.default_rng([seed, sid])
    k = normal_raw(rng, (length, h_kv, d), "bf16")
    v = normal_raw(rng, (length, h_kv, d), "bf16")
    q = normal_raw(rng, (length, h_q, d), "bf16")
    return k, v, q


def seq_token_chunk(seed: int, sid: int, chunk: int, rows: int, h_q: int, h_kv: int, d: int):
    """K, V (raw bf16 [rows, h_kv, d]) and Q (raw bf16 [rows, h_q, d]) of
    positions chunk*rows .. chunk*rows+rows-1 of sequence ``sid``, each chunk
    from a stream of its own, so that long sequences are drawn piece by piece
    and a position's data does not depend on when it is scheduled."""
    rng = np.random.default_rng([seed, sid, chunk])
    k = normal_raw(rng, (rows, h_kv, d), "bf16")
    v = normal_raw(rng, (rows, h_kv, d), "bf16")
    q = normal_raw(rng, (rows, h_q, d), "bf16")
    return k, v, q
