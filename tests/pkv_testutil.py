"""Helpers shared by the tests: fixture parsing, independent storage-format
conversions (numpy / torch), a sequential cache writer and NaN poisoning.

Nothing here is used by the product or by the oracle's arithmetic.
"""
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
F32, F16, BF16 = 0, 1, 2
DTYPES = {"f32": F32, "f16": F16, "bf16": BF16}
NAN_BITS = {F16: 0x7E00, BF16: 0x7FC0}


def read_golden(name):
    """key -> list of rows (each a list of tokens); '#' starts a comment."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, *vals = line.split()
            out.setdefault(key, []).append(vals)
    return out


def ints(row):
    return [int(v) for v in row]


def to_storage(x, dtype):
    """float array -> storage form (float32, or uint16 bits), RNE, via numpy/torch."""
    x = np.asarray(x)
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return np.ascontiguousarray(x.astype(np.float16).view(np.uint16))
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return np.ascontiguousarray(t.view(torch.int16).numpy().view(np.uint16))


def from_storage(a, dtype):
    """storage form -> float64, via numpy/torch (independent of the oracle)."""
    if dtype == F32:
        return a.astype(np.float64)
    if dtype == F16:
        return a.view(np.float16).astype(np.float64)
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def sequential_fill(pool, table, rows):
    """Write rows[i] (one token's [Hkv][D] row, i = 0, 1, ...) into `pool`
    ([num_blocks][B][Hkv][D]) the way a growing sequence fills its blocks: the
    next row of the current block, moving to the next listed block when the
    current one is full.  An independent construction of the paged layout."""
    B = pool.shape[1]
    cur, row = -1, B
    for r in rows:
        if row == B:
            cur += 1
            row = 0
        pool[table[cur], row] = r
        row += 1
    return pool


def poison_unused(cache, tables, lens, dtype):
    """Set every slot not holding one of the first lens[s] tokens of some
    sequence to NaN (blocks walked in table order, rows filled front to back)."""
    B = cache.shape[1]
    keep = np.zeros(cache.shape[:2], dtype=bool)
    for s, L in enumerate(lens):
        left = int(L)
        for b in tables[s]:
            if left <= 0 or b < 0:
                break
            n = min(B, left)
            keep[b, :n] = True
            left -= n
    nanv = np.float32(np.nan) if dtype == F32 else np.uint16(NAN_BITS[dtype])
    cache[~keep] = nanv
    return cache


def random_problem(rng, dtype, S, Hq, Hkv, D, B, lens, pool_extra=3, data_mult=1.0):
    """Dense per-sequence K/V/q in float32 plus a shuffled paged layout of them."""
    lens = [int(L) for L in lens]
    need = [-(-L // B) for L in lens]
    nb = sum(need) + pool_extra
    perm = rng.permutation(nb)
    tables, off = [], 0
    for n in need:
        tables.append(perm[off:off + n].astype(np.int32))
        off += n
    width = max(1, max(need))
    bt = np.full((S, width), -1, dtype=np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    q = to_storage(rng.standard_normal((S, Hq, D)) * data_mult, dtype)
    kc = to_storage(rng.standard_normal((nb, B, Hkv, D)) * data_mult, dtype)
    vc = to_storage(rng.standard_normal((nb, B, Hkv, D)) * data_mult, dtype)
    dense_k, dense_v = [], []
    for s in range(S):
        dk = to_storage(rng.standard_normal((lens[s], Hkv, D)) * data_mult, dtype)
        dv = to_storage(rng.standard_normal((lens[s], Hkv, D)) * data_mult, dtype)
        sequential_fill(kc, tables[s], dk)
        sequential_fill(vc, tables[s], dv)
        dense_k.append(dk)
        dense_v.append(dv)
    return dict(q=q, k_cache=kc, v_cache=vc, block_tables=bt, context_lens=np.array(lens, np.int32),
                tables=tables, dense_k=dense_k, dense_v=dense_v, dtype=dtype, B=B)
