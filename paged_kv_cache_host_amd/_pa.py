"""ctypes binding of libpa (include/pa.h), same names as the C ABI.

Argument marshalling only: every step runs in the library (host allocator in
C++, attention and cache writes in HIP kernels).  Device buffers are torch
tensors on a ROCm device (``tensor.data_ptr()``); streams are torch streams
(``stream.cuda_stream``) or raw hipStream_t integers.  Importing this module
fails loudly when libpa.so has not been built.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# PA_LIBRARY selects another build of the same library (the sanitizer build
# of the host code that the CPU tests run under); it must exist as well
LIB_PATH = os.environ.get("PA_LIBRARY") or os.path.join(_HERE, "libpa.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libpa.so is not built ({LIB_PATH}); run `python -m paged_kv_cache_host_amd.build`")
_lib = C.CDLL(LIB_PATH)

PA_OK = 0
PA_ERR_INVALID = -1
PA_ERR_NO_BLOCKS = -2
PA_ERR_UNKNOWN_SEQ = -3
PA_ERR_EXISTS = -4
PA_ERR_DEVICE = -5
PA_ERR_WORKSPACE = -6

PA_F32 = 0
PA_BF16 = 1
PA_FP8_E4M3 = 2

_i32p = C.POINTER(C.c_int32)
_i64p = C.POINTER(C.c_int64)
_vp = C.c_void_p
_i32 = C.c_int32
_i64 = C.c_int64
_f32 = C.c_float
_sz = C.c_size_t

class SchedBatchC(C.Structure):
    """``pa_sched_batch`` of include/pa.h."""
    _fields_ = [("decode_seq", _i64p), ("decode_pos", _i32p), ("decode_slot", _i32p),
                ("decode_cap", _i32),
                ("prefill_seq", _i64p), ("prefill_start", _i32p), ("prefill_len", _i32p),
                ("prefill_emits", _i32p),
                ("prefill_cap", _i32),
                ("prefill_slots", _i32p), ("prefill_slots_cap", _i32),
                ("finished", _i64p), ("admitted", _i64p), ("preempted", _i64p),
                ("event_cap", _i32),
                ("n_decode", _i32), ("n_prefill", _i32), ("n_prefill_tokens", _i32),
                ("n_finished", _i32), ("n_admitted", _i32), ("n_preempted", _i32)]


class SchedAccountingC(C.Structure):
    """``pa_sched_accounting`` of include/pa.h."""
    _fields_ = [("running", _i32), ("waiting", _i32), ("finished", _i64), ("preemptions", _i64),
                ("blocks_held", _i64), ("tokens_held", _i64), ("unwritten", _i64),
                ("prefix_hit_tokens", _i64)]


_SIGS = {
    "pa_version": (_i32, []),
    "pa_last_error": (C.c_char_p, []),
    "pa_pool_create": (_i32, [_i32, _i32, _i32p, C.POINTER(_vp)]),
    "pa_pool_destroy": (None, [_vp]),
    "pa_pool_num_free": (_i32, [_vp]),
    "pa_pool_num_seqs": (_i32, [_vp]),
    "pa_pool_free_list": (_i32, [_vp, _i32p, _i32, _i32p]),
    "pa_seq_create": (_i32, [_vp, _i64, _i32]),
    "pa_seq_append": (_i32, [_vp, _i64, _i32, _i32p]),
    "pa_batch_append": (_i32, [_vp, _i64p, _i32, _i32, _i32p, _i32p]),
    "pa_seq_slots": (_i32, [_vp, _i64, _i32, _i32, _i32p]),
    "pa_seq_release": (_i32, [_vp, _i64]),
    "pa_seq_share": (_i32, [_vp, _i64, _i64, _i32, _i32, _i32p]),
    "pa_pool_block_refs": (_i32, [_vp, _i32, _i32p]),
    "pa_seq_register_prefix": (_i32, [_vp, _i64, _i32p, _i32]),
    "pa_seq_create_prefix": (_i32, [_vp, _i64, _i32p, _i32, _i32p]),
    "pa_pool_match_prefix": (_i32, [_vp, _i32p, _i32, _i32p, _i32p]),
    "pa_pool_set_prefix_retention": (_i32, [_vp, _i32]),
    "pa_pool_num_retained": (_i32, [_vp]),
    "pa_pool_num_registered": (_i32, [_vp]),
    "pa_seq_length": (_i32, [_vp, _i64, _i32p]),
    "pa_seq_block_table": (_i32, [_vp, _i64, _i32p, _i32, _i32p]),
    "pa_pack_batch": (_i32, [_vp, _i64p, _i32, _i32, _i32p, _i32p]),
    "pa_validate_tables": (_i32, [_i32p, _i32p, _i32, _i32, _i32, _i32]),
    "pa_cache_write": (_i32, [_vp, _vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _i32, _i32,
                              _i32, _f32, _f32]),
    "pa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "pa_decode": (_i32, [_vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _i32, _vp, _i32,
                         _i32, _i32, _i32, _i32, _i32, _f32, _f32, _f32, _vp, _sz]),
    "pa_decode_noalloc": (_i32, [_vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _vp, _i32, _i32, _vp,
                                  _i32, _i32, _i32, _i32, _i32, _i32, _f32, _f32, _f32]),
    "pa_sched_create": (_i32, [_vp, _i32, _i32, _i32, C.POINTER(_vp)]),
    "pa_sched_create_mode": (_i32, [_vp, _i32, _i32, _i32, _i32, C.POINTER(_vp)]),
    "pa_sched_destroy": (None, [_vp]),
    "pa_sched_add": (_i32, [_vp, _i64, _i32, _i32]),
    "pa_sched_add_prompt": (_i32, [_vp, _i64, _i32, _i32, _i32p]),
    "pa_sched_step": (_i32, [_vp, C.POINTER(SchedBatchC)]),
    "pa_sched_stats": (_i32, [_vp, C.POINTER(SchedAccountingC)]),
    "pa_stage": (_i32, [_vp, _vp, _vp, _sz]),
    "pa_pinned_alias": (_i32, [_vp, C.POINTER(_vp)]),
    "pa_stage_cache_write": (_i32, [_vp, _vp, _vp, _sz, _sz, _vp, _vp, _i32, _i32, _vp, _vp, _i32,
                                    _i32, _i32, _i32, _i32, _f32, _f32]),
    "pa_stage_decode_append": (_i32, [_vp, _vp, _vp, _sz, _sz, _sz, _vp, _vp, _i32, _i32, _vp,
                                       _vp, _i32, _i32, _i32, _i32, _i32, _f32, _f32, _vp,
                                       _i32]),
    "pa_decode_append": (_i32, [_vp, _vp, _vp, _i32, _vp, _vp, _i32, _vp, _vp, _i32, _i32, _i32,
                                 _i32, _i32, _f32, _f32, _vp, _i32]),
    "pa_decode_step": (_i32, [_vp, _vp, _vp, _sz, _sz, _sz, _vp, _vp, _i32, _vp, _i32, _vp,
                               _i32, _vp, _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32,
                               _i32, _i32, _f32, _f32, _f32, _vp, _sz]),
    "pa_decode_step_set_spin_limit": (_i32, [_i32]),
    "pa_timing_enable": (_i32, [_i32, _i32]),
    "pa_timing_query": (_i32, [C.c_char_p, _i32p, C.POINTER(_f32), C.POINTER(_f32)]),
    "pa_prefill_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_prefill_chunk": (_i32, [_vp, _vp, _i32, _vp, _i32, _vp, _vp, _vp, _vp, _i32, _vp, _i32,
                                _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _f32, _f32, _f32,
                                _vp, _sz]),
    "pa_attend_varlen_counters": (_i64, [_i32, _i32, _i32, _i32, _i32]),
    "pa_attend_varlen_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32]),
    "pa_attend_varlen": (_i32, [_vp, _vp, _i32, _vp, _i32, _vp, _vp, _i32, _i32, _vp, _vp, _i32,
                                _vp, _i32, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _i32, _i32,
                                _i32, _f32, _f32, _f32, _vp, _i64, _vp, _sz]),
}

for _name, (_res, _args) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args

EXPORTED = tuple(_SIGS)


class PaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"libpa status {status}: {msg}")
        self.status = status


def pa_version() -> int:
    return _lib.pa_version()


def pa_last_error() -> str:
    return _lib.pa_last_error().decode()


def check(status: int) -> int:
    """Raise PaError for a non-OK status, else return it."""
    if status != PA_OK:
        raise PaError(status, pa_last_error())
    return status


def _i32_array(a) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(a, dtype=np.int32))


def _ptr_i32(a: np.ndarray):
    return a.ctypes.data_as(_i32p)


# ---------------------------------------------------------------- pool -----

def pa_pool_create(num_blocks: int, block_size: int = 16, initial_free_order=None):
    """Returns (status, pool handle or None)."""
    out = _vp()
    order = None if initial_free_order is None else _i32_array(initial_free_order)
    st = _lib.pa_pool_create(num_blocks, block_size, None if order is None else _ptr_i32(order),
                             C.byref(out))
    return st, (out.value if st == PA_OK else None)


def pa_pool_destroy(pool) -> None:
    _lib.pa_pool_destroy(pool)


def pa_pool_num_free(pool) -> int:
    return _lib.pa_pool_num_free(pool)


def pa_pool_num_seqs(pool) -> int:
    return _lib.pa_pool_num_seqs(pool)


def pa_pool_free_list(pool):
    n = _i32()
    cap = max(0, pa_pool_num_free(pool))
    buf = np.empty(cap, dtype=np.int32)
    st = _lib.pa_pool_free_list(pool, _ptr_i32(buf), cap, C.byref(n))
    return st, buf[: n.value]


def pa_seq_create(pool, seq: int, num_tokens: int) -> int:
    return _lib.pa_seq_create(pool, seq, num_tokens)


def pa_seq_append(pool, seq: int, n_new: int, want_slots: bool = True):
    """Returns (status, slots of the new positions or None)."""
    if want_slots and n_new > 0:
        buf = np.empty(n_new, dtype=np.int32)
        st = _lib.pa_seq_append(pool, seq, n_new, _ptr_i32(buf))
        return st, buf
    return _lib.pa_seq_append(pool, seq, n_new, None), None


def pa_batch_append(pool, seqs, n_new: int = 1, slots_out: np.ndarray | None = None):
    """Returns (status, number of sequences grown, slots [n_seqs, n_new])."""
    s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
    if slots_out is None:
        slots_out = np.empty((len(s), n_new), dtype=np.int32)
    assert slots_out.dtype == np.int32 and slots_out.flags.c_contiguous
    assert slots_out.size >= len(s) * n_new
    done = _i32()
    st = _lib.pa_batch_append(pool, s.ctypes.data_as(_i64p), len(s), n_new, _ptr_i32(slots_out),
                              C.byref(done))
    return st, done.value, slots_out


def pa_seq_slots(pool, seq: int, start: int, n: int, out: np.ndarray | None = None):
    """Returns (status, slots); ``out`` (int32, >= n entries, e.g. a pinned
    tensor's numpy view) is filled in place when given."""
    buf = np.empty(max(n, 0), dtype=np.int32) if out is None else out
    assert buf.dtype == np.int32 and buf.flags.c_contiguous and buf.size >= n
    st = _lib.pa_seq_slots(pool, seq, start, n, _ptr_i32(buf))
    return st, buf


def pa_seq_share(pool, seq: int, src: int, shared_tokens: int, num_tokens: int):
    """Returns (status, tokens that live in shared blocks)."""
    out = _i32(0)
    st = _lib.pa_seq_share(pool, seq, src, shared_tokens, num_tokens, C.byref(out))
    return st, out.value


def pa_seq_register_prefix(pool, seq: int, tokens, n_tokens: int | None = None) -> int:
    """Register the full blocks among the first n_tokens (default: all of
    ``tokens``) positions of ``seq`` under their token ids."""
    t = _i32_array(tokens)
    n = len(t) if n_tokens is None else int(n_tokens)
    if n > len(t):
        raise PaError(PA_ERR_INVALID, "pa_seq_register_prefix: n_tokens exceeds tokens")
    return _lib.pa_seq_register_prefix(pool, seq, _ptr_i32(t) if len(t) else None, n)


def pa_seq_create_prefix(pool, seq: int, tokens):
    """Create ``seq`` for the prompt ``tokens``, sharing every leading full
    block whose content is registered.  Returns (status, tokens that live
    in shared blocks)."""
    t = _i32_array(tokens)
    out = _i32(0)
    st = _lib.pa_seq_create_prefix(pool, seq, _ptr_i32(t) if len(t) else None, len(t),
                                   C.byref(out))
    return st, out.value


def pa_pool_match_prefix(pool, tokens, with_retained: bool = False):
    """Returns (status, tokens of the leading full blocks of ``tokens``
    whose content is registered[, how many of those blocks are retained]);
    changes nothing."""
    t = _i32_array(tokens)
    out, ret = _i32(0), _i32(0)
    st = _lib.pa_pool_match_prefix(pool, _ptr_i32(t) if len(t) else None, len(t), C.byref(out),
                                   C.byref(ret))
    return (st, out.value, ret.value) if with_retained else (st, out.value)


def pa_pool_set_prefix_retention(pool, enable: bool) -> int:
    return _lib.pa_pool_set_prefix_retention(pool, 1 if enable else 0)


def pa_pool_num_retained(pool) -> int:
    return _lib.pa_pool_num_retained(pool)


def pa_pool_num_registered(pool) -> int:
    return _lib.pa_pool_num_registered(pool)


def pa_pool_block_refs(pool, block: int):
    """Returns (status, number of sequences holding the block)."""
    out = _i32(0)
    st = _lib.pa_pool_block_refs(pool, block, C.byref(out))
    return st, out.value


def pa_seq_release(pool, seq: int) -> int:
    return _lib.pa_seq_release(pool, seq)


def pa_seq_length(pool, seq: int):
    n = _i32()
    st = _lib.pa_seq_length(pool, seq, C.byref(n))
    return st, n.value


def pa_seq_block_table(pool, seq: int):
    n = _i32()
    st = _lib.pa_seq_block_table(pool, seq, None, 0, C.byref(n))
    if st == PA_ERR_UNKNOWN_SEQ:
        return st, None
    buf = np.empty(n.value, dtype=np.int32)
    st = _lib.pa_seq_block_table(pool, seq, _ptr_i32(buf), n.value, C.byref(n))
    return st, buf


def pa_pack_batch(pool, seqs, max_blocks: int, block_tables: np.ndarray | None = None,
                  context_lens: np.ndarray | None = None):
    """Returns (status, block_tables [n, max_blocks] int32, context_lens [n] int32).
    Caller-provided output arrays (e.g. pinned host tensors' numpy views) are
    filled in place."""
    s = np.ascontiguousarray(np.asarray(seqs, dtype=np.int64))
    n = len(s)
    if block_tables is None:
        block_tables = np.empty((n, max_blocks), dtype=np.int32)
    if context_lens is None:
        context_lens = np.empty(n, dtype=np.int32)
    assert block_tables.dtype == np.int32 and block_tables.flags.c_contiguous
    assert block_tables.size >= n * max_blocks and context_lens.size >= n
    st = _lib.pa_pack_batch(pool, s.ctypes.data_as(_i64p), n, max_blocks, _ptr_i32(block_tables),
                            _ptr_i32(context_lens))
    return st, block_tables, context_lens


def pa_validate_tables(block_tables, context_lens, max_blocks: int, block_size: int,
                       num_blocks: int) -> int:
    t = _i32_array(block_tables)
    lens = _i32_array(context_lens)
    return _lib.pa_validate_tables(_ptr_i32(t), _ptr_i32(lens), len(lens), max_blocks, block_size,
                                   num_blocks)


# ----------------------------------------------------------- scheduler -----

def pa_sched_create(pool, max_running: int = 256, prefill_budget: int = 512,
                    block_size: int = 16):
    """Returns (status, scheduler handle or None)."""
    out = _vp()
    st = _lib.pa_sched_create(pool, max_running, prefill_budget, block_size, C.byref(out))
    return st, (out.value if st == PA_OK else None)


SCHED_MODES = {"chunked": 0, "continuous": 1, "static": 2, "naive": 3}


def pa_sched_create_mode(pool, mode: str, max_running: int = 256, prefill_budget: int = 512,
                         block_size: int = 16):
    """Returns (status, scheduler handle or None); ``mode`` is one of
    ``SCHED_MODES``."""
    out = _vp()
    st = _lib.pa_sched_create_mode(pool, SCHED_MODES[mode], max_running, prefill_budget,
                                   block_size, C.byref(out))
    return st, (out.value if st == PA_OK else None)


def pa_sched_destroy(sched) -> None:
    _lib.pa_sched_destroy(sched)


def pa_sched_add(sched, seq: int, prompt_len: int, target: int) -> int:
    return _lib.pa_sched_add(sched, seq, prompt_len, target)


def pa_sched_add_prompt(sched, seq: int, target: int, ids) -> int:
    """Queue a request with its prompt's token ids (prefix caching); the
    prompt length is len(ids)."""
    t = _i32_array(ids)
    if len(t) < 1:
        raise PaError(PA_ERR_INVALID, "pa_sched_add_prompt: empty prompt")
    return _lib.pa_sched_add_prompt(sched, seq, len(t), target, _ptr_i32(t))


class SchedBatch:
    """Host arrays of one pa_sched_step (numpy views, reused every step)."""

    def __init__(self, max_running: int, prefill_budget: int):
        R, B = max_running, max(prefill_budget, 1)
        self.decode_seq = np.zeros(R, np.int64)
        self.decode_pos = np.zeros(R, np.int32)
        self.decode_slot = np.zeros(R, np.int32)
        self.prefill_seq = np.zeros(R, np.int64)
        self.prefill_start = np.zeros(R, np.int32)
        self.prefill_len = np.zeros(R, np.int32)
        self.prefill_emits = np.zeros(R, np.int32)
        self.prefill_slots = np.zeros(B, np.int32)
        self.finished = np.zeros(R, np.int64)
        self.admitted = np.zeros(R, np.int64)
        self.preempted = np.zeros(R, np.int64)
        p64 = lambda a: a.ctypes.data_as(_i64p)
        self.c = SchedBatchC(p64(self.decode_seq), _ptr_i32(self.decode_pos),
                             _ptr_i32(self.decode_slot), R, p64(self.prefill_seq),
                             _ptr_i32(self.prefill_start), _ptr_i32(self.prefill_len),
                             _ptr_i32(self.prefill_emits), R,
                             _ptr_i32(self.prefill_slots), B, p64(self.finished),
                             p64(self.admitted), p64(self.preempted), R, 0, 0, 0, 0, 0, 0)

    @property
    def n_decode(self):
        return self.c.n_decode

    @property
    def n_prefill(self):
        return self.c.n_prefill

    @property
    def n_prefill_tokens(self):
        return self.c.n_prefill_tokens

    def decode(self):
        n = self.c.n_decode
        return self.decode_seq[:n], self.decode_pos[:n], self.decode_slot[:n]

    def prefill(self):
        n = self.c.n_prefill
        return self.prefill_seq[:n], self.prefill_start[:n], self.prefill_len[:n]

    def emits(self):
        """Per prefill slice: 1 if it yields the sequence's next output token."""
        return self.prefill_emits[:self.c.n_prefill]

    def slots(self):
        return self.prefill_slots[:self.c.n_prefill_tokens]

    def events(self):
        return (self.finished[:self.c.n_finished].tolist(),
                self.admitted[:self.c.n_admitted].tolist(),
                self.preempted[:self.c.n_preempted].tolist())


def pa_sched_step(sched, batch: SchedBatch) -> int:
    return _lib.pa_sched_step(sched, C.byref(batch.c))


def pa_sched_stats(sched):
    """Returns (status, dict of the accounting fields)."""
    a = SchedAccountingC()
    st = _lib.pa_sched_stats(sched, C.byref(a))
    return st, {k: getattr(a, k) for k, _ in SchedAccountingC._fields_}


# -------------------------------------------------------------- timing -----

TIMING_BITS = {"cache_write": 1, "decode": 2, "decode_merge": 4, "prefill": 8,
               "prefill_merge": 16, "generic": 32, "stage": 64,
               "stage_cache_write": 128, "varlen": 256, "decode_step": 512}


def pa_timing_enable(enable=True, every: int = 1) -> int:
    """``enable``: True (all kernels), False (none), or an iterable of kernel
    names to record; ``every``: time every n-th launch of each (from 0)."""
    if enable is True:
        mask = -1
    elif not enable:
        mask = 0
    else:
        mask = 0
        for name in enable:
            mask |= TIMING_BITS[name]
    return _lib.pa_timing_enable(mask, every)


def pa_timing_query(kernel: str):
    """Returns (status, count, mean_us, total_us) of the recorded launches."""
    n = _i32()
    mean = _f32()
    tot = _f32()
    st = _lib.pa_timing_query(kernel.encode(), C.byref(n), C.byref(mean), C.byref(tot))
    return st, n.value, mean.value, tot.value


# ------------------------------------------------------------- kernels -----

def _stream_handle(stream) -> int | None:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dptr(t) -> int:
    if t is None:
        return None
    if not t.is_cuda:
        raise PaError(PA_ERR_INVALID, "expected a device tensor")
    return t.data_ptr()


def dtype_of(t) -> int:
    import torch
    if t.dtype == torch.float32:
        return PA_F32
    if t.dtype == torch.bfloat16:
        return PA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return PA_FP8_E4M3
    raise PaError(PA_ERR_INVALID, f"unsupported tensor dtype {t.dtype}")


# Argument checks of the kernel wrappers (shapes, dtypes and extents of the
# tensors whose pointers cross the C ABI): a tensor that is too small, of
# the wrong integer width or strided would otherwise be read or written out
# of bounds by a kernel that trusts its sizes.

def _need(ok: bool, who: str, what: str):
    if not ok:
        raise PaError(PA_ERR_INVALID, f"{who}: {what}")


def _check_i32(who: str, name: str, t, n_min: int):
    _need(t is not None and str(t.dtype) == "torch.int32" and t.is_contiguous()
          and t.numel() >= n_min, who,
          f"{name} must be a contiguous int32 tensor of at least {n_min} entries")


def _check_tables(who: str, t, rows: int):
    _need(str(t.dtype) == "torch.int32" and t.is_contiguous() and t.dim() == 2
          and t.shape[0] >= rows and t.shape[1] >= 1, who,
          f"block_tables must be a contiguous int32 [>= {rows}, max_blocks] tensor")


def _check_cache(who: str, k_cache, v_cache, num_blocks: int, H_kv: int, D: int, bs: int):
    need = num_blocks * H_kv * D * bs
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache)):
        _need(t.is_contiguous() and t.numel() >= need, who,
              f"{name} must be contiguous with room for {num_blocks} blocks of {H_kv} x {D} x "
              f"{bs} elements")
    _need(k_cache.dtype == v_cache.dtype, who, "k_cache and v_cache differ in dtype")


def _check_rows(who: str, name: str, t, rows: int, H: int, D: int):
    _need(t.is_contiguous() and t.dim() == 3 and t.shape[0] >= rows and t.shape[1] == H
          and t.shape[2] == D, who, f"{name} must be a contiguous [>= {rows}, {H}, {D}] tensor")


def pa_pinned_alias(src_host) -> tuple[int, int]:
    """Host-only check of a staging source: (status, device alias or 0)."""
    out = _vp()
    st = _lib.pa_pinned_alias(src_host, C.byref(out))
    return st, (out.value or 0)


def pa_cache_write(stream, k_new, v_new, slot_mapping, k_cache, v_cache, num_blocks: int,
                   H_kv: int, D: int, bs: int = 16, k_scale: float = 1.0, v_scale: float = 1.0,
                   n: int | None = None) -> int:
    n = slot_mapping.numel() if n is None else n
    who = "pa_cache_write"
    _check_i32(who, "slot_mapping", slot_mapping, n)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t.is_contiguous() and t.numel() >= n * H_kv * D, who,
              f"{name} must be a contiguous [>= {n}, {H_kv}, {D}] tensor")
    _check_cache(who, k_cache, v_cache, num_blocks, H_kv, D, bs)
    return _lib.pa_cache_write(_stream_handle(stream), _dptr(k_new), _dptr(v_new),
                               dtype_of(k_new), _dptr(slot_mapping), n, _dptr(k_cache),
                               _dptr(v_cache), dtype_of(k_cache), num_blocks, H_kv, D, bs,
                               k_scale, v_scale)


def pa_stage(stream, dst, src_host, nbytes: int | None = None) -> int:
    """Copy ``nbytes`` (default: all of ``src_host``) from a pinned host
    tensor into the device tensor ``dst`` with a kernel on ``stream``."""
    if src_host.is_cuda or not src_host.is_pinned():
        raise PaError(PA_ERR_INVALID, "pa_stage: source must be a pinned host tensor")
    n = src_host.numel() * src_host.element_size() if nbytes is None else int(nbytes)
    if n > src_host.numel() * src_host.element_size() or n > dst.numel() * dst.element_size():
        raise PaError(PA_ERR_INVALID, "pa_stage: nbytes exceeds a buffer")
    return _lib.pa_stage(_stream_handle(stream), _dptr(dst), src_host.data_ptr(), n)


def pa_stage_cache_write(stream, dst, src_host, nbytes: int, slot_offset: int, n: int, k_new,
                         v_new, k_cache, v_cache, num_blocks: int, H_kv: int, D: int,
                         bs: int = 16, k_scale: float = 1.0, v_scale: float = 1.0) -> int:
    """pa_stage of the first ``nbytes`` of the pinned tensor ``src_host`` into
    ``dst`` plus the cache write of ``n`` new tokens whose int32 slots sit at
    byte ``slot_offset`` of that buffer, in one launch."""
    if src_host.is_cuda or not src_host.is_pinned():
        raise PaError(PA_ERR_INVALID, "pa_stage_cache_write: source must be a pinned host tensor")
    if nbytes > src_host.numel() * src_host.element_size() or \
            nbytes > dst.numel() * dst.element_size():
        raise PaError(PA_ERR_INVALID, "pa_stage_cache_write: nbytes exceeds a buffer")
    return _lib.pa_stage_cache_write(_stream_handle(stream), _dptr(dst), src_host.data_ptr(),
                                     nbytes, slot_offset, _dptr(k_new), _dptr(v_new),
                                     dtype_of(k_new), n, _dptr(k_cache), _dptr(v_cache),
                                     dtype_of(k_cache), num_blocks, H_kv, D, bs, k_scale, v_scale)


def pa_stage_decode_append(stream, dst, src_host, nbytes: int, slot_offset: int,
                           lens_offset: int, n: int, k_new, v_new, k_cache, v_cache,
                           num_blocks: int, H_kv: int, D: int, block_tables, bs: int = 16,
                           k_scale: float = 1.0, v_scale: float = 1.0) -> int:
    """pa_stage_cache_write of a decode batch whose device block tables
    (``block_tables`` [n, max_blocks] int32 on the device) are kept up to date
    in the same launch: token i (slot at byte ``slot_offset``, context length
    at byte ``lens_offset`` of the staged buffer) enters its block in row i."""
    if src_host.is_cuda or not src_host.is_pinned():
        raise PaError(PA_ERR_INVALID, "pa_stage_decode_append: source must be a pinned host tensor")
    if nbytes > src_host.numel() * src_host.element_size() or \
            nbytes > dst.numel() * dst.element_size():
        raise PaError(PA_ERR_INVALID, "pa_stage_decode_append: nbytes exceeds a buffer")
    if str(block_tables.dtype) != "torch.int32" or not block_tables.is_contiguous() or \
            block_tables.dim() != 2 or block_tables.shape[0] < n:
        raise PaError(PA_ERR_INVALID, "pa_stage_decode_append: block_tables must be a contiguous "
                      "int32 [n, max_blocks] tensor")
    return _lib.pa_stage_decode_append(_stream_handle(stream), _dptr(dst), src_host.data_ptr(),
                                       nbytes, slot_offset, lens_offset, _dptr(k_new),
                                       _dptr(v_new), dtype_of(k_new), n, _dptr(k_cache),
                                       _dptr(v_cache), dtype_of(k_cache), num_blocks, H_kv, D, bs,
                                       k_scale, v_scale, _dptr(block_tables),
                                       block_tables.shape[1])


def pa_decode_append(stream, slots, lens, n: int, k_new, v_new, k_cache, v_cache,
                     num_blocks: int, H_kv: int, D: int, block_tables, bs: int = 16,
                     k_scale: float = 1.0, v_scale: float = 1.0) -> int:
    """pa_stage_decode_append with the ``n`` slots and context lengths
    already in device int32 tensors (``slots``, ``lens``)."""
    for name, t in (("slots", slots), ("lens", lens)):
        if str(t.dtype) != "torch.int32" or not t.is_contiguous() or t.numel() < n:
            raise PaError(PA_ERR_INVALID, f"pa_decode_append: {name} must be a contiguous int32 "
                          "tensor of at least n entries")
    if str(block_tables.dtype) != "torch.int32" or not block_tables.is_contiguous() or \
            block_tables.dim() != 2 or block_tables.shape[0] < n:
        raise PaError(PA_ERR_INVALID, "pa_decode_append: block_tables must be a contiguous "
                      "int32 [n, max_blocks] tensor")
    return _lib.pa_decode_append(_stream_handle(stream), _dptr(slots), _dptr(lens), n,
                                 _dptr(k_new), _dptr(v_new), dtype_of(k_new), _dptr(k_cache),
                                 _dptr(v_cache), dtype_of(k_cache), num_blocks, H_kv, D, bs,
                                 k_scale, v_scale, _dptr(block_tables), block_tables.shape[1])


def pa_decode_step(stream, dst, src_host, nbytes: int, slot_offset: int, lens_offset: int,
                   k_new, v_new, out, q, k_cache, v_cache, block_tables, num_blocks: int,
                   H_kv: int, max_context_len: int, sm_scale: float, k_scale: float = 1.0,
                   v_scale: float = 1.0, ws=None, bs: int = 16) -> int:
    """One decode iteration in one launch: the S = q.shape[0] new tokens'
    K/V (``k_new``/``v_new`` [S, H_kv, D] bf16) into their slots, their
    blocks into ``block_tables`` (device [S, max_blocks] int32, updated in
    place) and decode attention into ``out``.  The int32 slots and context
    lengths sit at byte ``slot_offset`` / ``lens_offset`` of the metadata
    buffer: ``src_host`` (pinned host tensor), staged into the device tensor
    ``dst`` by the launch, or None when ``dst`` already holds them."""
    S, H_q, D = q.shape
    who = "pa_decode_step"
    if src_host is not None:
        if src_host.is_cuda or not src_host.is_pinned():
            raise PaError(PA_ERR_INVALID, f"{who}: source must be a pinned host tensor")
        if nbytes > src_host.numel() * src_host.element_size():
            raise PaError(PA_ERR_INVALID, f"{who}: nbytes exceeds the source")
    if nbytes > dst.numel() * dst.element_size():
        raise PaError(PA_ERR_INVALID, f"{who}: nbytes exceeds dst")
    _check_rows(who, "q", q, S, H_q, D)
    _check_rows(who, "out", out, S, H_q, D)
    _check_tables(who, block_tables, S)
    _check_cache(who, k_cache, v_cache, num_blocks, H_kv, D, bs)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        _need(t.is_contiguous() and t.numel() >= S * H_kv * D, who,
              f"{name} must be a contiguous [>= {S}, {H_kv}, {D}] tensor")
    return _lib.pa_decode_step(_stream_handle(stream), _dptr(dst),
                               None if src_host is None else src_host.data_ptr(), nbytes,
                               slot_offset, lens_offset, _dptr(k_new), _dptr(v_new),
                               dtype_of(k_new), _dptr(out), dtype_of(out), _dptr(q), dtype_of(q),
                               _dptr(k_cache), _dptr(v_cache), dtype_of(k_cache),
                               _dptr(block_tables), block_tables.shape[1], num_blocks, S, H_q,
                               H_kv, D, bs, max_context_len, sm_scale, k_scale, v_scale,
                               _dptr(ws), 0 if ws is None else ws.numel() * ws.element_size())


def pa_decode_step_set_spin_limit(polls: int) -> int:
    """Testing aid: polls a pa_decode_step work-group makes for the staged
    metadata before it takes no work (default 65536)."""
    return _lib.pa_decode_step_set_spin_limit(polls)


def pa_decode_workspace_bytes(S: int, H_q: int, H_kv: int, D: int, max_context_len: int) -> int:
    return _lib.pa_decode_workspace_bytes(S, H_q, H_kv, D, max_context_len)


def pa_decode(stream, out, q, k_cache, v_cache, block_tables, context_lens, num_blocks: int,
              H_kv: int, max_context_len: int, sm_scale: float, k_scale: float = 1.0,
              v_scale: float = 1.0, ws=None, bs: int = 16) -> int:
    S, H_q, D = q.shape
    who = "pa_decode"
    _check_rows(who, "q", q, S, H_q, D)
    _check_rows(who, "out", out, S, H_q, D)
    _check_tables(who, block_tables, S)
    _check_i32(who, "context_lens", context_lens, S)
    _check_cache(who, k_cache, v_cache, num_blocks, H_kv, D, bs)
    max_blocks = block_tables.shape[1]
    return _lib.pa_decode(_stream_handle(stream), _dptr(out), dtype_of(out), _dptr(q), dtype_of(q),
                          _dptr(k_cache), _dptr(v_cache), dtype_of(k_cache), _dptr(block_tables),
                          max_blocks, num_blocks, _dptr(context_lens), S, H_q, H_kv, D, bs,
                          max_context_len, sm_scale, k_scale, v_scale, _dptr(ws),
                          0 if ws is None else ws.numel() * ws.element_size())


def pa_decode_noalloc(stream, out, q, k_cache, v_cache, block_tables, context_lens,
                      num_blocks: int, H_kv: int, max_context_len: int, sm_scale: float,
                      k_scale: float = 1.0, v_scale: float = 1.0, bs: int = 16) -> int:
    """pa_decode with the library's own per-device scratch array as its
    workspace (no workspace argument, nothing allocated)."""
    S, H_q, D = q.shape
    who = "pa_decode_noalloc"
    _check_rows(who, "q", q, S, H_q, D)
    _check_rows(who, "out", out, S, H_q, D)
    _check_tables(who, block_tables, S)
    _check_i32(who, "context_lens", context_lens, S)
    _check_cache(who, k_cache, v_cache, num_blocks, H_kv, D, bs)
    return _lib.pa_decode_noalloc(_stream_handle(stream), _dptr(out), dtype_of(out), _dptr(q),
                                  dtype_of(q), _dptr(k_cache), _dptr(v_cache), dtype_of(k_cache),
                                  _dptr(block_tables), block_tables.shape[1], num_blocks,
                                  _dptr(context_lens), S, H_q, H_kv, D, bs, max_context_len,
                                  sm_scale, k_scale, v_scale)


def pa_prefill_workspace_bytes(n_chunks: int, max_q_len: int, H_q: int, H_kv: int, D: int,
                               max_context_len: int) -> int:
    return _lib.pa_prefill_workspace_bytes(n_chunks, max_q_len, H_q, H_kv, D, max_context_len)


def pa_prefill_chunk(stream, out, q, cu_q_lens, start_pos, k_cache, v_cache, block_tables,
                     num_blocks: int, H_kv: int, max_q_len: int, max_context_len: int,
                     sm_scale: float, k_scale: float = 1.0, v_scale: float = 1.0, ws=None,
                     bs: int = 16) -> int:
    T, H_q, D = q.shape
    n_chunks = start_pos.numel()
    who = "pa_prefill_chunk"
    _check_rows(who, "q", q, T, H_q, D)
    _check_rows(who, "out", out, T, H_q, D)
    _check_i32(who, "cu_q_lens", cu_q_lens, n_chunks + 1)
    _check_i32(who, "start_pos", start_pos, n_chunks)
    _check_tables(who, block_tables, n_chunks)
    _check_cache(who, k_cache, v_cache, num_blocks, H_kv, D, bs)
    max_blocks = block_tables.shape[1]
    return _lib.pa_prefill_chunk(_stream_handle(stream), _dptr(out), dtype_of(out), _dptr(q),
                                 dtype_of(q), _dptr(cu_q_lens), _dptr(start_pos), _dptr(k_cache),
                                 _dptr(v_cache), dtype_of(k_cache), _dptr(block_tables),
                                 max_blocks, num_blocks, n_chunks, H_q, H_kv, D, bs, max_q_len,
                                 max_context_len, sm_scale, k_scale, v_scale, _dptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size())


def pa_attend_varlen_counters(n_decode: int, n_prefill: int, H_q: int, H_kv: int,
                              max_q_len: int) -> int:
    return _lib.pa_attend_varlen_counters(n_decode, n_prefill, H_q, H_kv, max_q_len)


def pa_attend_varlen_workspace_bytes(n_decode: int, n_prefill: int, H_q: int, H_kv: int, D: int,
                                     max_q_len: int, max_decode_len: int,
                                     max_prefill_len: int) -> int:
    return _lib.pa_attend_varlen_workspace_bytes(n_decode, n_prefill, H_q, H_kv, D, max_q_len,
                                                 max_decode_len, max_prefill_len)


def pa_attend_varlen(stream, out, q, cu_q_lens, seq_lens, n_decode: int, k_cache, v_cache,
                     dec_tables, pf_tables, num_blocks: int, H_kv: int, max_q_len: int,
                     max_decode_len: int, max_prefill_len: int, sm_scale: float,
                     k_scale: float = 1.0, v_scale: float = 1.0, counters=None, ws=None,
                     bs: int = 16) -> int:
    """The decode rows (the first n_decode sequences, one query each, block
    tables ``dec_tables``) and the prefill slices (the rest of seq_lens,
    tables ``pf_tables``) of one iteration in one launch."""
    T, H_q, D = q.shape
    who = "pa_attend_varlen"
    n_seqs = seq_lens.numel()
    n_pf = n_seqs - n_decode
    _need(0 <= n_decode <= n_seqs, who, f"n_decode={n_decode} must lie in [0, {n_seqs}]")
    _need(T >= n_decode, who, f"q has {T} rows, fewer than the {n_decode} decode rows")
    _check_rows(who, "q", q, T, H_q, D)
    _check_rows(who, "out", out, T, H_q, D)
    _check_i32(who, "cu_q_lens", cu_q_lens, n_seqs + 1)
    _check_i32(who, "seq_lens", seq_lens, n_seqs)
    if n_decode:
        _check_tables(who, dec_tables, n_decode)
    if n_pf:
        _check_tables(who, pf_tables, n_pf)
    _check_cache(who, k_cache, v_cache, num_blocks, H_kv, D, bs)
    _need(counters is None or (str(counters.dtype) == "torch.int32" and counters.is_contiguous()),
          who, "counters must be a contiguous int32 tensor")
    dmb = dec_tables.shape[1] if n_decode else 0
    pmb = pf_tables.shape[1] if n_pf else 0
    return _lib.pa_attend_varlen(_stream_handle(stream), _dptr(out), dtype_of(out), _dptr(q),
                                 dtype_of(q), _dptr(cu_q_lens), _dptr(seq_lens), n_decode, n_pf,
                                 _dptr(k_cache), _dptr(v_cache), dtype_of(k_cache),
                                 _dptr(dec_tables) if n_decode else None, dmb,
                                 _dptr(pf_tables) if n_pf else None, pmb, num_blocks, H_q, H_kv,
                                 D, bs, max_q_len, max_decode_len, max_prefill_len, sm_scale,
                                 k_scale, v_scale, _dptr(counters),
                                 0 if counters is None else counters.numel(), _dptr(ws),
                                 0 if ws is None else ws.numel() * ws.element_size())
