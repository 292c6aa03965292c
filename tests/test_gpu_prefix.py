"""GPU parity with prefix sharing (ARTICLE 4.3): sequences created from the
prompt of another with pa_seq_share hold its full blocks read-only; their
decode and a prefill slice over their own tokens read the shared blocks
through their tables.  Tables and block counts are compared bit-exactly with
the oracle's pool, cache bytes bit-exactly, attention within tolerance."""
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_host_amd._pa as pa
import workloads
from oracle import allocator as oa
from oracle import attention as oat
from oracle import cache as oc
from oracle import codecs
from paged_kv_cache_host_amd.engine import (PagedKV, decode_workspace, prefill_workspace,
                                            to_device_raw, to_host_raw)
from tests.parity import assert_close, filled, out_to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
H_Q, H_KV, D, BS = 32, 4, 128, 16


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("cache_dtype", ["bf16", "fp8"])
def test_shared_prefix_decode_and_prefill(cache_dtype):
    rng = np.random.default_rng(700)
    P = 1000                                    # prefix: 62 full blocks + 8 tokens
    suffix = [1, 8, 9, 24, 300, 600, 41]        # sharers' own tokens after the prefix
    S = 1 + len(suffix)
    nb = -(-P // BS) + sum(-(-(P + n) // BS) - P // BS for n in suffix) + 5
    order = rng.permutation(nb).astype(np.int32)
    pk = workloads.normal_raw(rng, (P, H_KV, D), "bf16")
    pv = workloads.normal_raw(rng, (P, H_KV, D), "bf16")
    sk = [workloads.normal_raw(rng, (n, H_KV, D), "bf16") for n in suffix]
    sv = [workloads.normal_raw(rng, (n, H_KV, D), "bf16") for n in suffix]
    q_dec = workloads.normal_raw(rng, (S, H_Q, D), "bf16")
    scale = (4.9 / 448.0) if cache_dtype == "fp8" else 1.0
    sm = float(np.float32(1.0) / np.float32(np.sqrt(D)))
    say(f"[prefix] {cache_dtype}: prefix {P}, sharers {suffix}, pool {nb}")

    kv = PagedKV(nb, H_KV, D, cache_dtype, DEV, order, scale, scale)
    ref = oa.BlockPool(nb, BS, order.tolist())
    kc, vc = oc.new_cache(nb, H_KV, BS, D, cache_dtype)

    def write_both(seq, start, k_raw, v_raw):
        n = k_raw.shape[0]
        if n == 0:
            return
        slots = kv.slots(seq, start, n)
        assert list(slots) == ref.slots(seq, start, n)
        kv.write(to_device_raw(k_raw, "bf16", DEV), to_device_raw(v_raw, "bf16", DEV),
                 torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int32)).to(DEV))
        oc.cache_write(kc, vc, k_raw, v_raw, list(slots), "bf16", cache_dtype, scale, scale)

    assert kv.create(0, P) == 0 and ref.seq_create(0, P) == oa.OK
    write_both(0, 0, pk, pv)
    for i, n in enumerate(suffix):
        st1 = pa.pa_seq_share(kv.pool, i + 1, 0, P, P + n)
        st2 = ref.seq_share(i + 1, 0, P, P + n)
        assert st1 == st2 and st1[0] == 0
        shared = st1[1]
        assert shared == (P // BS) * BS
        # the prefix tail in the sharer's own block, then its own tokens
        write_both(i + 1, shared, pk[shared:], pv[shared:])
        write_both(i + 1, P, sk[i], sv[i])
    for b in range(nb):
        assert pa.pa_pool_block_refs(kv.pool, b)[1] == ref.block_refs(b)
    assert max(ref.refs) == S                   # the full prefix blocks are held by all

    tables, lens = kv.pack(list(range(S)))
    rt, rl = ref.pack(list(range(S)), tables.shape[1])
    assert tables.tolist() == rt and lens.tolist() == rl
    kb = to_host_raw(kv.k, cache_dtype)
    vb = to_host_raw(kv.v, cache_dtype)
    assert np.array_equal(kb, kc) and np.array_equal(vb, vc), "cache bytes differ"

    # decode of every sequence
    t_d = torch.from_numpy(tables).to(DEV)
    l_d = torch.from_numpy(lens).to(DEV)
    qd = to_device_raw(q_dec, "bf16", DEV)
    out = filled((S, H_Q, D), torch.bfloat16, DEV)
    mc = int(lens.max())
    ws = decode_workspace(S, H_Q, H_KV, D, mc, DEV)
    kv.decode(out, qd, t_d, l_d, mc, sm, ws)
    torch.cuda.synchronize()
    got = out_to_f64(to_host_raw(out.cpu(), "bf16"), "bf16")
    want = oat.decode(codecs.decode(q_dec, "bf16"), kc, vc, np.asarray(rt), np.asarray(rl), H_KV,
                      sm, cache_dtype, scale, scale)
    err = assert_close(got, want, cache_dtype, "shared-prefix decode")
    say(f"    decode max|d| = {err:.3g}")

    # the 600-token sharer's own tokens as one prefill slice over the prefix
    k = suffix.index(600)
    seq = k + 1
    n = suffix[k]
    qp = workloads.normal_raw(rng, (n, H_Q, D), "bf16")
    row = tables[seq:seq + 1]
    cu = torch.tensor([0, n], dtype=torch.int32, device=DEV)
    st_ = torch.tensor([P], dtype=torch.int32, device=DEV)
    outp = filled((n, H_Q, D), torch.bfloat16, DEV)
    wsp = prefill_workspace(1, n, H_Q, H_KV, D, P + n, DEV)
    kv.prefill(outp, to_device_raw(qp, "bf16", DEV), cu, st_, torch.from_numpy(row).to(DEV), n,
               P + n, sm, wsp)
    torch.cuda.synchronize()
    gotp = out_to_f64(to_host_raw(outp.cpu(), "bf16"), "bf16")
    wantp = oat.prefill_chunk(codecs.decode(qp, "bf16"), P, kc, vc, np.asarray(rt[seq]), H_KV, sm,
                              cache_dtype, scale, scale)
    err = assert_close(gotp, wantp, cache_dtype, "shared-prefix prefill")
    say(f"    prefill max|d| = {err:.3g}")

    # releasing the owner keeps the shared blocks for the sharers
    assert pa.pa_seq_release(kv.pool, 0) == 0 and ref.seq_release(0) == oa.OK
    assert list(pa.pa_pool_free_list(kv.pool)[1]) == ref.free_list()
    kv.close()


def test_detected_prefix_prefill_and_decode():
    """Prefix detection (ARTICLE 4.3): requests that start with the same
    200-token system prompt find its blocks by content.  Request 0 is
    prefilled and its prompt registered; each later request is created from
    its token ids, takes the matched full blocks, and writes and prefills
    only from the first position past them (its prefill slice starts
    there).  One request diverges inside the system prompt and shares only
    the blocks before the divergence.  Tables, reference counts, the
    registered count and the cache bytes equal the oracle pool's; every
    prefill slice and a decode of all requests pass the gate against the
    oracle.  Same tokens are taken to give the same K/V (the premise of
    reusing them), so the K/V of a position are drawn once per distinct
    token prefix."""
    rng = np.random.default_rng(701)
    sp = rng.integers(1, 50000, size=200).tolist()         # system prompt token ids
    users = [rng.integers(1, 50000, size=n).tolist() for n in (40, 3, 77, 16)]
    prompts = [sp + u for u in users]
    div = sp[:100] + [7] + sp[101:]                          # diverges at position 100
    prompts.append(div + users[0])
    S = len(prompts)
    nb = sum(-(-len(p) // BS) for p in prompts) + 4
    order = rng.permutation(nb).astype(np.int32)
    sm = float(np.float32(1.0) / np.float32(np.sqrt(D)))
    say(f"[prefix detection] {S} requests, system prompt 200 tokens, pool {nb}")

    kv = PagedKV(nb, H_KV, D, "bf16", DEV, order)
    ref = oa.BlockPool(nb, BS, order.tolist())
    kc, vc = oc.new_cache(nb, H_KV, BS, D, "bf16")
    # K/V per distinct token prefix (position p of a prompt is identified by
    # its first p+1 token ids)
    kv_of = {}

    def token_kv(prompt, p):
        key = tuple(prompt[:p + 1])
        if key not in kv_of:
            kv_of[key] = (workloads.normal_raw(rng, (1, H_KV, D), "bf16"),
                          workloads.normal_raw(rng, (1, H_KV, D), "bf16"))
        return kv_of[key]

    written = []
    for i, prompt in enumerate(prompts):
        st1 = pa.pa_seq_create_prefix(kv.pool, i, prompt)
        st2 = ref.seq_create_prefix(i, prompt)
        assert st1 == st2 and st1[0] == pa.PA_OK, (st1, st2)
        shared = st1[1]
        expect = 0 if i == 0 else (96 if i == S - 1 else 192)
        assert shared == expect, (i, shared)
        n = len(prompt) - shared
        k_raw = np.concatenate([token_kv(prompt, p)[0] for p in range(shared, len(prompt))])
        v_raw = np.concatenate([token_kv(prompt, p)[1] for p in range(shared, len(prompt))])
        slots = kv.slots(i, shared, n)
        assert list(slots) == ref.slots(i, shared, n)
        kv.write(to_device_raw(k_raw, "bf16", DEV), to_device_raw(v_raw, "bf16", DEV),
                 torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int32)).to(DEV))
        oc.cache_write(kc, vc, k_raw, v_raw, list(slots), "bf16", "bf16")
        written.append(n)
        # the slice's prefill from the first unshared position
        t_row, _ = kv.pack([i])
        qp = workloads.normal_raw(rng, (n, H_Q, D), "bf16")
        cu = torch.tensor([0, n], dtype=torch.int32, device=DEV)
        st_ = torch.tensor([shared], dtype=torch.int32, device=DEV)
        outp = filled((n, H_Q, D), torch.bfloat16, DEV)
        wsp = prefill_workspace(1, n, H_Q, H_KV, D, len(prompt), DEV)
        kv.prefill(outp, to_device_raw(qp, "bf16", DEV), cu, st_, torch.from_numpy(t_row).to(DEV),
                   n, len(prompt), sm, wsp)
        torch.cuda.synchronize()
        gotp = out_to_f64(to_host_raw(outp.cpu(), "bf16"), "bf16")
        wantp = oat.prefill_chunk(codecs.decode(qp, "bf16"), shared, kc, vc,
                                  np.asarray(ref.block_table(i)), H_KV, sm, "bf16")
        err = assert_close(gotp, wantp, "bf16", f"request {i} prefill from {shared}")
        say(f"    request {i}: shared {shared}, wrote {n}, prefill max|d| = {err:.3g}")
        # its prompt is now computed: register it for the next requests
        assert pa.pa_seq_register_prefix(kv.pool, i, prompt) == ref.seq_register_prefix(i, prompt)
        assert pa.pa_pool_num_registered(kv.pool) == ref.num_registered()

    for b in range(nb):
        assert pa.pa_pool_block_refs(kv.pool, b)[1] == ref.block_refs(b)
    assert sum(written) < sum(len(p) for p in prompts) - 3 * 192
    tables, lens = kv.pack(list(range(S)))
    rt, rl = ref.pack(list(range(S)), tables.shape[1])
    assert tables.tolist() == rt and lens.tolist() == rl
    assert np.array_equal(to_host_raw(kv.k, "bf16"), kc) and \
        np.array_equal(to_host_raw(kv.v, "bf16"), vc), "cache bytes differ"

    q_dec = workloads.normal_raw(rng, (S, H_Q, D), "bf16")
    out = filled((S, H_Q, D), torch.bfloat16, DEV)
    mc = int(lens.max())
    ws = decode_workspace(S, H_Q, H_KV, D, mc, DEV)
    kv.decode(out, to_device_raw(q_dec, "bf16", DEV), torch.from_numpy(tables).to(DEV),
              torch.from_numpy(lens).to(DEV), mc, sm, ws)
    torch.cuda.synchronize()
    got = out_to_f64(to_host_raw(out.cpu(), "bf16"), "bf16")
    want = oat.decode(codecs.decode(q_dec, "bf16"), kc, vc, np.asarray(rt), np.asarray(rl), H_KV,
                      sm, "bf16")
    err = assert_close(got, want, "bf16", "detected-prefix decode")
    say(f"    decode max|d| = {err:.3g}")
    kv.close()
