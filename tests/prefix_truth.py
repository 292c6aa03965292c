"""A content check for prefix sharing, used by the oracle's and the C
allocator's tests: it keeps, for every block, the prompt prefix whose K/V the
block holds, and fails when a sequence is handed a block computed under
another prefix."""
from oracle import allocator as oa

# A block's K/V are those of the tokens that filled it AND of every token
# before them in the sequence that computed it.  The checker below keeps, for
# every block, the prompt prefix its contents were computed under, and fails
# when a sequence is handed a block computed under another prefix, or when a
# key in the index names a parent block that is no longer registered (that
# parent's id can be reused for other content, and the key would then match
# under it).

def run_with_truth(pool, ops, check_index=True):
    truth = {}                       # block -> token prefix its K/V hold
    toks = {}                        # live sequence -> its token ids
    bs = pool.block_size
    for op in ops:
        kind = op[0]
        if kind == "create":
            _, seq, tokens = op
            before = set(pool.free_list())
            st, shared = pool.seq_create_prefix(seq, tokens)
            if st == oa.OK:
                table = pool.block_table(seq)
                for i, b in enumerate(table):
                    if i < shared // bs:
                        assert truth.get(b) == tuple(tokens[:(i + 1) * bs]), \
                            f"seq {seq} shares block {b} computed under another prefix"
                    else:
                        assert b in before
                        truth.pop(b, None)
                toks[seq] = list(tokens)
        elif kind == "append":
            _, seq, new = op
            if seq in toks:
                old = pool.block_table(seq)
                if pool.seq_append(seq, len(new))[0] == oa.OK:
                    for b in pool.block_table(seq)[len(old):]:
                        truth.pop(b, None)
                    toks[seq] += list(new)
        elif kind == "register":
            _, seq, frac = op
            if seq in toks:
                n = len(toks[seq]) * frac // 4
                table = pool.block_table(seq)
                for i in range(n // bs):
                    pre = tuple(toks[seq][:(i + 1) * bs])
                    assert truth.setdefault(table[i], pre) == pre
                assert pool.seq_register_prefix(seq, toks[seq][:n]) == oa.OK
        elif kind == "release":
            _, seq = op
            if seq in toks:
                assert pool.seq_release(seq) == oa.OK
                del toks[seq]
        elif kind == "retention":
            pool.set_prefix_retention(op[1])
        for parent, _ in (pool.index if check_index else ()):
            assert parent == -1 or parent in pool.content, \
                f"a registered block names block {parent}, which is no longer registered"


def random_ops(rng):
    ops = [("retention", True)]
    for _ in range(rng.randint(1, 60)):
        kind = rng.choice(["create", "append", "register", "release", "retention"])
        seq = rng.randint(0, 5)
        if kind == "create":
            ops.append((kind, seq, [rng.randint(0, 1) for _ in range(rng.randint(0, 10))]))
        elif kind == "append":
            ops.append((kind, seq, [rng.randint(0, 1) for _ in range(rng.randint(0, 5))]))
        elif kind == "register":
            ops.append((kind, seq, rng.randint(0, 4)))
        elif kind == "release":
            ops.append((kind, seq))
        else:
            ops.append((kind, rng.random() < 0.5))
    return ops, rng.randint(0, 12)


def seeded_cases(n=6000, seed=20261202):
    """``n`` seeded random (ops, number of blocks) cases."""
    import random

    rng = random.Random(seed)
    return [random_ops(rng) for _ in range(n)]
