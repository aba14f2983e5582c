"""Pins of the CPU oracle: checks against what the pages and the mathematics fix,
never against the oracle itself.

Each ``pin_*`` takes an ``oracle.ref.Oracle`` and raises AssertionError when the
oracle disagrees with:

* values the pages print for worked examples (tests/golden/, each file citing
  its page and section);
* library routines for special cases (numpy's float16 conversions, torch's
  bfloat16 conversions, torch's scaled_dot_product_attention in float64 on the
  contiguous layout);
* closed forms (one token, zero query, equal keys);
* invariants (any permutation of physical blocks, a shared versus a copied
  prefix, split-K versus unsplit, NaN in slots that no sequence owns);
* an independent construction of the paged layout (``sequential_fill``).

test_oracle_pins.py runs every pin on the real oracle; test_oracle_mutants.py
plants plausible mistakes in copies of the oracle's source and checks that some
pin fails for each.
"""
import numpy as np
import torch

from pkv_testutil import (BF16, F16, F32, from_storage, ints, poison_unused, random_problem,
                          read_golden, sequential_fill, to_storage)


def _close(a, b, tol, what):
    err = float(np.max(np.abs(np.asarray(a) - np.asarray(b)))) if np.size(a) else 0.0
    assert np.all(np.isfinite(a)), "%s: non-finite values" % what
    assert err <= tol, "%s: max abs error %.3g > %.3g" % (what, err, tol)


# ---------------------------------------------------------------------------
# Storage formats
# ---------------------------------------------------------------------------

def pin_f16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.to_double(bits, F16)
    want = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "f16 decode: NaN patterns differ"
    assert np.array_equal(got[~nan], want[~nan]), "f16 decode differs from numpy"


def pin_bf16_decode_exhaustive(orc):
    bits = np.arange(65536, dtype=np.uint16)
    got = orc.to_double(bits, BF16)
    want = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(want)
    assert np.array_equal(np.isnan(got), nan), "bf16 decode: NaN patterns differ"
    assert np.array_equal(got[~nan], want[~nan]), "bf16 decode differs from torch"


def _encode_samples(rng):
    mags = np.concatenate([
        rng.uniform(-1, 1, 4000),
        rng.standard_normal(4000) * 2.0 ** rng.integers(-30, 20, 4000),
        rng.uniform(-7e4, 7e4, 1000),                       # around the f16 overflow point
        rng.standard_normal(1000) * 2.0 ** -24,             # f16 subnormals
    ])
    # exact midpoints between neighbouring f16 values (ties go to even)
    h = rng.integers(0, 0x7BFF, 2000).astype(np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    return np.concatenate([mags, (lo + hi) / 2, -(lo + hi) / 2, [0.0, -0.0, 65504.0, 65520.0,
                                                              65519.99, 6e-8, 3e-8, 2.9e-8]])


def pin_f16_encode(orc):
    x = _encode_samples(np.random.default_rng(11))
    got = orc.cast(x, F16)
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, "f16 encode differs from numpy at %r" % (x[bad[:4]],)


def pin_bf16_encode(orc):
    rng = np.random.default_rng(12)
    # values exactly representable in float32: torch's float32 -> bfloat16 is a single rounding
    f = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        (rng.standard_normal(2000) * 2.0 ** rng.integers(-130, 120, 2000)).astype(np.float32),
                        np.array([0, -0.0, 3.3895314e38, 3.39e38, 1e-40, -1e-45], np.float32)])
    got = orc.cast(f.astype(np.float64), BF16)
    want = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, want), "bf16 encode differs from torch"
    # rounding straight from double: 1 + 2^-8 + 2^-30 lies above the midpoint of
    # 1 and 1 + 2^-7, so it rounds up (via binary32 it would tie down to 1.0)
    assert orc.double_to_bf16_bits(1 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81
    assert orc.double_to_bf16_bits(1 + 2.0 ** -8) == 0x3F80          # tie -> even
    assert orc.double_to_bf16_bits(1 + 3 * 2.0 ** -8) == 0x3F82      # tie -> even
    assert orc.double_to_bf16_bits(-2.0 ** 128) == 0xFF80            # overflow -> -inf


def pin_f32_cast(orc):
    x = np.random.default_rng(13).standard_normal(5000) * 1e3
    assert np.array_equal(orc.cast(x, F32), x.astype(np.float32))


# ---------------------------------------------------------------------------
# Address translation and append
# ---------------------------------------------------------------------------

def pin_slots_block_table_example(orc):
    g = read_golden("block_table_b4.txt")
    B = ints(g["block_size"][0])[0]
    table = ints(g["table_after"][-1][1:])
    want = ints(g["slots"][0])
    got = [orc.physical_slot(table, B, i) for i in range(len(want))]
    assert got == want, "slots %r != printed example %r" % (got, want)


def pin_slot_out_of_blocks_example(orc):
    g = read_golden("out_of_blocks_b16.txt")
    B = ints(g["block_size"][0])[0]
    table = ints(g["seq0_table_after_append"][0])
    n = ints(g["seq0_n_tokens_after_append"][0])[0]
    assert orc.physical_slot(table, B, n - 1) == ints(g["slot_token32"][0])[0]


def pin_gather_sequential_fill(orc):
    rng = np.random.default_rng(21)
    for B, Hkv, D, L in [(1, 1, 3, 5), (3, 2, 4, 10), (4, 3, 5, 13), (16, 2, 8, 33), (16, 1, 4, 16)]:
        nb = -(-L // B) + 4
        table = rng.permutation(nb)[: -(-L // B)]
        rows = rng.standard_normal((L, Hkv, D)).astype(np.float32)
        pool = sequential_fill(np.zeros((nb, B, Hkv, D), np.float32), table, rows)
        got = orc.gather(pool, table, L, F32)
        assert np.array_equal(got, rows.transpose(1, 0, 2).astype(np.float64)), \
            "gather != sequential fill (B=%d)" % B


def pin_append_one_token_at_a_time(orc):
    """Appending tokens 0..L-1 one call each builds the sequential-fill layout."""
    rng = np.random.default_rng(22)
    for dtype in (F32, BF16):
        B, Hkv, D, S = 4, 3, 8, 3
        lens = [9, 4, 13]
        need = [-(-L // B) for L in lens]
        nb = sum(need) + 2
        perm = rng.permutation(nb)
        tables, off = [], 0
        for n in need:
            tables.append(perm[off:off + n])
            off += n
        bt = np.full((S, max(need)), -1, np.int32)
        for s, t in enumerate(tables):
            bt[s, :len(t)] = t
        rows = [to_storage(rng.standard_normal((L, Hkv, D)), dtype) for L in lens]
        want_k = np.zeros((nb, B, Hkv, D), rows[0].dtype)
        for s in range(S):
            sequential_fill(want_k, tables[s], rows[s])
        kc = np.zeros_like(want_k)
        vc = np.zeros_like(want_k)
        for i in range(max(lens)):
            active = [s for s in range(S) if i < lens[s]]
            kn = np.ascontiguousarray(np.stack([rows[s][i] for s in active]))
            orc.append(kn, kn.copy(), kc, vc, bt[active], np.full(len(active), i, np.int32), dtype)
        assert np.array_equal(kc, want_k) and np.array_equal(vc, want_k), "append layout"


def pin_append_overwrites_only_its_slot(orc):
    rng = np.random.default_rng(23)
    B, Hkv, D = 16, 2, 8
    p = random_problem(rng, F16, 3, 2, Hkv, D, B, [5, 16, 17])
    kc, vc = p["k_cache"].copy(), p["v_cache"].copy()
    S = 3
    pos = p["context_lens"] - 1
    kn = to_storage(rng.standard_normal((S, Hkv, D)), F16)
    vn = to_storage(rng.standard_normal((S, Hkv, D)), F16)
    orc.append(kn, vn, kc, vc, p["block_tables"], pos, F16)
    for s in range(S):
        rows_k = list(p["dense_k"][s])
        rows_v = list(p["dense_v"][s])
        rows_k[pos[s]] = kn[s]
        rows_v[pos[s]] = vn[s]
        sequential_fill(p["k_cache"], p["tables"][s], rows_k)
        sequential_fill(p["v_cache"], p["tables"][s], rows_v)
    assert np.array_equal(kc, p["k_cache"]) and np.array_equal(vc, p["v_cache"])


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def _sdpa_dense(p, scale, Hq):
    """torch scaled_dot_product_attention (float64, CPU) on the contiguous layout."""
    dtype = p["dtype"]
    out = []
    for s in range(len(p["dense_k"])):
        q = torch.from_numpy(from_storage(p["q"][s], dtype))[None, :, None, :]        # [1,Hq,1,D]
        k = torch.from_numpy(from_storage(p["dense_k"][s], dtype).transpose(1, 0, 2).copy())[None]
        v = torch.from_numpy(from_storage(p["dense_v"][s], dtype).transpose(1, 0, 2).copy())[None]
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale, enable_gqa=True)
        out.append(o[0, :, 0, :].numpy())
    return np.stack(out)


def _oracle(orc, p, scale, **kw):
    return orc.attention_decode(p["q"], p["k_cache"], p["v_cache"], p["block_tables"],
                                p["context_lens"], scale, p["dtype"], **kw)


def pin_attention_matches_sdpa(orc):
    rng = np.random.default_rng(31)
    cases = [(F32, 4, 4, 16, 16, [5, 16, 17, 33]),
             (F16, 8, 2, 8, 4, [1, 4, 5, 9]),
             (BF16, 8, 1, 16, 16, [2, 31, 48]),
             (BF16, 6, 3, 8, 3, [7, 1, 12])]
    for dtype, Hq, Hkv, D, B, lens in cases:
        p = random_problem(rng, dtype, len(lens), Hq, Hkv, D, B, lens)
        scale = 1.0 / np.sqrt(D)
        _close(_oracle(orc, p, scale), _sdpa_dense(p, scale, Hq), 1e-12,
               "oracle vs SDPA (dtype %d, %d/%d heads)" % (dtype, Hq, Hkv))


def pin_closed_forms(orc):
    rng = np.random.default_rng(32)
    # one token: the output is that token's value row, exactly
    p = random_problem(rng, F32, 2, 4, 2, 8, 16, [1, 1])
    got = _oracle(orc, p, 0.3)
    for s in range(2):
        want = np.repeat(p["dense_v"][s][0].astype(np.float64), 2, axis=0)
        assert np.array_equal(got[s], want), "L=1 must return V_0"
    # zero query, or all keys equal: the plain mean of the value rows
    p = random_problem(rng, F32, 2, 2, 2, 8, 4, [7, 13])
    p["q"][:] = 0
    got = _oracle(orc, p, 1.0)
    for s in range(2):
        want = np.repeat(p["dense_v"][s].astype(np.float64).mean(axis=0), 1, axis=0)
        _close(got[s], want, 1e-14, "q = 0 gives the mean of V")
    p = random_problem(rng, F32, 1, 3, 1, 8, 4, [11])
    row = p["dense_k"][0][0].copy()
    sequential_fill(p["k_cache"], p["tables"][0], [row] * 11)
    got = _oracle(orc, p, 0.7)
    want = np.repeat(p["dense_v"][0].astype(np.float64).mean(axis=0), 3, axis=0)
    _close(got[0], want, 1e-14, "equal keys give the mean of V")


def pin_block_permutation_invariance(orc):
    rng = np.random.default_rng(33)
    p = random_problem(rng, BF16, 3, 8, 2, 16, 16, [20, 47, 3])
    base = _oracle(orc, p, 0.25)
    nb = p["k_cache"].shape[0]
    pi = rng.permutation(nb)
    k2 = np.empty_like(p["k_cache"])
    v2 = np.empty_like(p["v_cache"])
    k2[pi] = p["k_cache"]
    v2[pi] = p["v_cache"]
    bt = p["block_tables"].copy()
    bt[bt >= 0] = pi[bt[bt >= 0]]
    q = dict(p, k_cache=k2, v_cache=v2, block_tables=bt)
    assert np.array_equal(_oracle(orc, q, 0.25), base), "output moved with the physical layout"


def pin_shared_vs_copied_prefix(orc):
    rng = np.random.default_rng(34)
    B, Hkv, D, S, pre = 4, 2, 8, 3, 8
    suffix = [3, 5, 1]
    pre_k = to_storage(rng.standard_normal((pre, Hkv, D)), F16)
    pre_v = to_storage(rng.standard_normal((pre, Hkv, D)), F16)
    suf_k = [to_storage(rng.standard_normal((n, Hkv, D)), F16) for n in suffix]
    suf_v = [to_storage(rng.standard_normal((n, Hkv, D)), F16) for n in suffix]
    q = to_storage(rng.standard_normal((S, 4, D)), F16)
    lens = np.array([pre + n for n in suffix], np.int32)
    outs = []
    for shared in (True, False):
        nb = 40
        order = list(rng.permutation(nb))
        kc = np.zeros((nb, B, Hkv, D), np.uint16)
        vc = np.zeros_like(kc)
        pre_blocks = [order.pop() for _ in range(pre // B)]
        bt = np.full((S, 8), -1, np.int32)
        for s in range(S):
            mine = pre_blocks if shared else [order.pop() for _ in range(pre // B)]
            mine = mine + [order.pop() for _ in range(-(-suffix[s] // B))]
            sequential_fill(kc, mine, list(pre_k) + list(suf_k[s]))
            sequential_fill(vc, mine, list(pre_v) + list(suf_v[s]))
            bt[s, :len(mine)] = mine
        outs.append(orc.attention_decode(q, kc, vc, bt, lens, 0.35, F16))
    assert np.array_equal(outs[0], outs[1]), "shared and copied prefix differ"


def pin_split_k_identity(orc):
    rng = np.random.default_rng(35)
    p = random_problem(rng, BF16, 3, 8, 2, 16, 16, [600, 77, 1030])
    whole = _oracle(orc, p, 0.25)
    for P in (1, 5, 16, 64, 512, 2048):
        _close(_oracle(orc, p, 0.25, part_tokens=P), whole, 1e-12, "split-K P=%d" % P)
    # also against the library on the contiguous layout
    _close(_oracle(orc, p, 0.25, part_tokens=64), _sdpa_dense(p, 0.25, 8), 1e-12, "split-K vs SDPA")


def pin_unused_slots_never_read(orc):
    rng = np.random.default_rng(36)
    for dtype in (F32, F16, BF16):
        p = random_problem(rng, dtype, 4, 4, 2, 8, 16, [5, 16, 17, 33], pool_extra=5)
        base = _oracle(orc, p, 0.5)
        poison_unused(p["k_cache"], p["block_tables"], p["context_lens"], dtype)
        poison_unused(p["v_cache"], p["block_tables"], p["context_lens"], dtype)
        got = _oracle(orc, p, 0.5)
        assert np.array_equal(got, base), "a slot past the context changed the output"


def pin_zero_length(orc):
    rng = np.random.default_rng(37)
    p = random_problem(rng, F32, 2, 2, 2, 8, 4, [0, 3])
    got = _oracle(orc, p, 1.0)
    assert np.array_equal(got[0], np.zeros((2, 8))), "L = 0 gives zeros"
    assert np.all(np.isfinite(got[1]))


def pin_sampled_sequences(orc):
    rng = np.random.default_rng(38)
    p = random_problem(rng, F16, 5, 4, 4, 8, 16, [3, 40, 17, 1, 22])
    full = _oracle(orc, p, 0.5)
    part = _oracle(orc, p, 0.5, seq_ids=[3, 1])
    assert np.array_equal(part[[1, 3]], full[[1, 3]])
    assert np.all(np.isnan(part[[0, 2, 4]]))


# ---------------------------------------------------------------------------
# Copy-on-write: the data half
# ---------------------------------------------------------------------------

def _poisoned_pool(shape, dtype):
    """A pool of quiet NaNs whose payload names the block (1 + block index), so
    a row copied from the wrong block, or past the rows asked for, changes bits."""
    b = (np.arange(shape[0]) + 1).reshape((-1,) + (1,) * (len(shape) - 1))
    if dtype == F32:
        return np.ascontiguousarray(np.broadcast_to((0x7FC00000 | b).astype(np.uint32), shape)).view(np.float32)
    quiet = {F16: 0x7E00, BF16: 0x7FC0}[dtype]
    mask = {F16: 0x1FF, BF16: 0x3F}[dtype]
    return np.ascontiguousarray(np.broadcast_to((quiet | (b & mask)).astype(np.uint16), shape))


def _bits(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _fork_example():
    g = read_golden("fork_cow_b16.txt")
    B = ints(g["block_size"][0])[0]
    n_prompt = ints(g["prompt_tokens"][0])[0]
    prompt_table = ints(g["prompt_table"][0])
    samples = [ints(r[1:]) for r in sorted(g["sample_table"], key=lambda r: int(r[0]))]
    return B, n_prompt, prompt_table, samples


def _diverge(orc, rng, dtype, Hkv, D):
    """The printed fork: the prompt's rows in its blocks, then for each sample
    the copy of the shared last block's filled rows into the sample's private
    block, then the sample's first generated token appended at position
    n_prompt.  Unwritten slots hold NaN."""
    B, n_prompt, prompt_table, samples = _fork_example()
    nb = 1 + max(max(t) for t in samples + [prompt_table])
    pk = to_storage(rng.standard_normal((n_prompt, Hkv, D)), dtype)
    pv = to_storage(rng.standard_normal((n_prompt, Hkv, D)), dtype)
    nk = to_storage(rng.standard_normal((len(samples), Hkv, D)), dtype)
    nv = to_storage(rng.standard_normal((len(samples), Hkv, D)), dtype)
    kc, vc = _poisoned_pool((nb, B, Hkv, D), dtype), _poisoned_pool((nb, B, Hkv, D), dtype)
    sequential_fill(kc, prompt_table, pk)
    sequential_fill(vc, prompt_table, pv)
    before_k, before_v = kc.copy(), vc.copy()
    # each sample's table differs from the prompt's in its last entry only
    for t in samples:
        assert t[:-1] == prompt_table[:-1] and t[-1] != prompt_table[-1]
    src = [prompt_table[-1]] * len(samples)
    dst = [t[-1] for t in samples]
    orc.copy_blocks(kc, vc, src, dst, [n_prompt % B] * len(samples), dtype)
    orc.append(nk, nv, kc, vc, np.array(samples, np.int32), np.full(len(samples), n_prompt, np.int32), dtype)
    return dict(B=B, n_prompt=n_prompt, prompt_table=prompt_table, samples=samples, kc=kc, vc=vc,
                before_k=before_k, before_v=before_v, pk=pk, pv=pv, nk=nk, nv=nv)


def pin_fork_diverge_copy(orc):
    """Worked example of "How a serving engine actually works", section
    "Copy-on-write, because you have used fork()", with data: every sample's
    blocks hold exactly the prompt followed by its own token (checked against
    an independent sequential fill, NaN slots included), and the prompt's
    blocks are untouched."""
    rng = np.random.default_rng(41)
    for dtype in (F32, F16, BF16):
        r = _diverge(orc, rng, dtype, 2, 8)
        for i, t in enumerate(r["samples"]):
            for cache, rows, new in ((r["kc"], r["pk"], r["nk"]), (r["vc"], r["pv"], r["nv"])):
                want = _poisoned_pool(cache.shape, dtype)
                sequential_fill(want, t, list(rows) + [new[i]])
                assert np.array_equal(_bits(cache[t]), _bits(want[t])), "sample %d's blocks (dtype %d)" % (i, dtype)
        pt = r["prompt_table"]
        assert np.array_equal(_bits(r["kc"][pt]), _bits(r["before_k"][pt])), "prompt K blocks changed"
        assert np.array_equal(_bits(r["vc"][pt]), _bits(r["before_v"][pt])), "prompt V blocks changed"


def pin_fork_diverge_attention(orc):
    """After the divergence each sample attends to the prompt plus its own token:
    the oracle through the shared tables equals torch SDPA (float64) on the
    dense sequences."""
    rng = np.random.default_rng(42)
    Hkv, D, Hq = 2, 16, 4
    r = _diverge(orc, rng, BF16, Hkv, D)
    S = len(r["samples"])
    L = r["n_prompt"] + 1
    q = to_storage(rng.standard_normal((S, Hq, D)), BF16)
    got = orc.attention_decode(q, r["kc"], r["vc"], np.array(r["samples"], np.int32),
                               np.full(S, L, np.int32), 0.25, BF16)
    for i in range(S):
        k = np.concatenate([from_storage(r["pk"], BF16), from_storage(r["nk"][i:i + 1], BF16)])
        v = np.concatenate([from_storage(r["pv"], BF16), from_storage(r["nv"][i:i + 1], BF16)])
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(from_storage(q[i], BF16))[None, :, None, :],
            torch.from_numpy(k.transpose(1, 0, 2).copy())[None],
            torch.from_numpy(v.transpose(1, 0, 2).copy())[None], scale=0.25, enable_gqa=True)
        _close(got[i], o[0, :, 0, :].numpy(), 1e-12, "sample %d after copy-on-write" % i)


def pin_copy_blocks_whole_and_empty(orc):
    """n_rows = B moves a whole block (a full block's sequence reads the same
    through either block); n_rows = 0 changes nothing; a bad argument rejects
    the call before anything is written."""
    rng = np.random.default_rng(43)
    B, Hkv, D, L = 16, 2, 8, 16
    rows = to_storage(rng.standard_normal((L, Hkv, D)), F16)
    kc, vc = _poisoned_pool((6, B, Hkv, D), F16), _poisoned_pool((6, B, Hkv, D), F16)
    sequential_fill(kc, [2], rows)
    sequential_fill(vc, [2], rows)
    snap = kc.copy()
    orc.copy_blocks(kc, vc, [2], [4], [0], F16)
    assert np.array_equal(_bits(kc), _bits(snap)), "n_rows = 0 wrote something"
    orc.copy_blocks(kc, vc, [2], [4], [B], F16)
    assert np.array_equal(orc.gather(kc, [4], L, F16), orc.gather(kc, [2], L, F16))
    assert np.array_equal(orc.gather(kc, [4], L, F16), from_storage(rows, F16).transpose(1, 0, 2))
    snap = kc.copy()
    for bad in (([2], [6], [1]), ([-1], [4], [1]), ([2], [4], [B + 1]), ([2], [4], [-1])):
        try:
            orc.copy_blocks(kc, vc, *bad, F16)
        except ValueError:
            pass
        else:
            raise AssertionError("copy_blocks accepted %r" % (bad,))
    assert np.array_equal(_bits(kc), _bits(snap)), "a rejected call wrote something"


# ---------------------------------------------------------------------------
# Chunked prefill
# ---------------------------------------------------------------------------

def _prefill_case(rng, dtype, Hq, Hkv, D, B, lens, chunk):
    """A paged problem plus packed queries for each sequence's last chunk[s] tokens."""
    p = random_problem(rng, dtype, len(lens), Hq, Hkv, D, B, lens)
    cu = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    q = to_storage(rng.standard_normal((int(cu[-1]), Hq, D)), dtype)
    return p, q, cu


def _sdpa_prefill(p, q, cu, scale, causal_flag=False):
    """torch SDPA (float64, CPU) on the dense sequences, the chunk's queries being
    the last n positions: query j may see key i iff i <= L - n + j."""
    dtype = p["dtype"]
    out = np.empty(q.shape)
    for s in range(len(p["dense_k"])):
        lo, hi = int(cu[s]), int(cu[s + 1])
        n, L = hi - lo, len(p["dense_k"][s])
        qs = torch.from_numpy(from_storage(q[lo:hi], dtype).transpose(1, 0, 2).copy())[None]   # [1,Hq,n,D]
        k = torch.from_numpy(from_storage(p["dense_k"][s], dtype).transpose(1, 0, 2).copy())[None]
        v = torch.from_numpy(from_storage(p["dense_v"][s], dtype).transpose(1, 0, 2).copy())[None]
        if causal_flag:
            assert n == L
            o = torch.nn.functional.scaled_dot_product_attention(qs, k, v, scale=scale, is_causal=True,
                                                                 enable_gqa=True)
        else:
            mask = torch.from_numpy(np.arange(L)[None, :] <= (L - n + np.arange(n))[:, None])
            o = torch.nn.functional.scaled_dot_product_attention(qs, k, v, attn_mask=mask, scale=scale,
                                                                 enable_gqa=True)
        out[lo:hi] = o[0].numpy().transpose(1, 0, 2)
    return out


def pin_prefill_matches_masked_sdpa(orc):
    rng = np.random.default_rng(51)
    cases = [(F32, 4, 4, 16, 16, [5, 16, 17, 33], [5, 3, 17, 10]),
             (BF16, 8, 2, 16, 4, [9, 20, 7], [4, 20, 1]),
             (F16, 6, 3, 8, 16, [40, 33], [16, 1]),
             (BF16, 8, 1, 16, 16, [70], [35])]
    for dtype, Hq, Hkv, D, B, lens, chunk in cases:
        p, q, cu = _prefill_case(rng, dtype, Hq, Hkv, D, B, lens, chunk)
        got = orc.attention_prefill(q, p["k_cache"], p["v_cache"], p["block_tables"], cu, p["context_lens"],
                                    0.3, dtype)
        _close(got, _sdpa_prefill(p, q, cu, 0.3), 1e-12, "prefill vs masked SDPA (dtype %d)" % dtype)


def pin_prefill_whole_prompt_is_causal(orc):
    rng = np.random.default_rng(52)
    p, q, cu = _prefill_case(rng, BF16, 4, 2, 16, 16, [37], [37])
    got = orc.attention_prefill(q, p["k_cache"], p["v_cache"], p["block_tables"], cu, p["context_lens"], 0.25, BF16)
    _close(got, _sdpa_prefill(p, q, cu, 0.25, causal_flag=True), 1e-12, "whole prompt vs causal SDPA")


def pin_prefill_single_token_is_decode(orc):
    """A one-token chunk is a decode step."""
    rng = np.random.default_rng(53)
    p, q, cu = _prefill_case(rng, F16, 8, 2, 16, 16, [5, 16, 17, 33], [1, 1, 1, 1])
    got = orc.attention_prefill(q, p["k_cache"], p["v_cache"], p["block_tables"], cu, p["context_lens"], 0.4, F16)
    want = orc.attention_decode(q, p["k_cache"], p["v_cache"], p["block_tables"], p["context_lens"], 0.4, F16)
    _close(got, want, 1e-13, "one-token chunk vs decode")


def pin_prefill_chunking_invariance(orc):
    """A prompt prefilled in chunks (the context growing chunk by chunk) gives
    every token the same output as one chunk holding the whole prompt."""
    rng = np.random.default_rng(54)
    L = 45
    p, q, cu = _prefill_case(rng, BF16, 4, 2, 16, 16, [L], [L])
    whole = orc.attention_prefill(q, p["k_cache"], p["v_cache"], p["block_tables"], cu, p["context_lens"],
                                  0.3, BF16)
    start = 0
    for n in (16, 16, 13):
        part = orc.attention_prefill(np.ascontiguousarray(q[start:start + n]), p["k_cache"], p["v_cache"],
                                     p["block_tables"], np.array([0, n], np.int32),
                                     np.array([start + n], np.int32), 0.3, BF16)
        assert np.array_equal(part, whole[start:start + n]), "chunk at %d differs" % start
        start += n


def pin_append_tokens_builds_sequential_fill(orc):
    """Appending each sequence's tokens in chunks of several tokens per call
    builds the sequential-fill layout, and nothing else changes."""
    rng = np.random.default_rng(55)
    B, Hkv, D = 4, 2, 8
    lens = [9, 14, 3]
    need = [-(-L // B) for L in lens]
    nb = sum(need) + 3
    perm = rng.permutation(nb)
    tables, off = [], 0
    for n in need:
        tables.append(perm[off:off + n])
        off += n
    bt = np.full((3, max(need)), -1, np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    rows = [to_storage(rng.standard_normal((L, Hkv, D)), F16) for L in lens]
    want = _poisoned_pool((nb, B, Hkv, D), F16)
    for s in range(3):
        sequential_fill(want, tables[s], rows[s])
    kc, vc = _poisoned_pool((nb, B, Hkv, D), F16), _poisoned_pool((nb, B, Hkv, D), F16)
    done = [0, 0, 0]
    for step in ([4, 5, 1], [5, 9, 2], [0, 0, 0]):
        n = [min(a, L - d) for a, L, d in zip(step, lens, done)]
        cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
        kn = np.ascontiguousarray(np.concatenate([rows[s][done[s]:done[s] + n[s]] for s in range(3)]))
        orc.append_tokens(kn, kn.copy(), kc, vc, bt, cu, np.array(done, np.int32), F16)
        done = [d + k for d, k in zip(done, n)]
    assert done == lens
    assert np.array_equal(_bits(kc), _bits(want)) and np.array_equal(_bits(vc), _bits(want)), "n-token append"


# ---------------------------------------------------------------------------
# Swap (preemption)
# ---------------------------------------------------------------------------

def pin_swap_round_trip_out_of_blocks_example(orc):
    """The pages' full pool ("How a serving engine actually works", section
    "When there are no free blocks left"), with data: 4 sequences x 2 blocks
    fill all 8 blocks; the victim (seq-3) is swapped out, its blocks go back to
    the pool and seq-0's next token lands in one of them; later the victim is
    swapped back into other blocks.  Its gathered cache is its original rows,
    and its attention is bit-identical to before the preemption."""
    g = read_golden("out_of_blocks_b16.txt")
    B = ints(g["block_size"][0])[0]
    n_blocks = ints(g["n_blocks"][0])[0]
    n_seq = ints(g["seqs"][0])[0]
    L = ints(g["tokens_per_seq"][0])[0]
    victim = ints(g["preempt"][0])[0]
    freed = ints(g["free_after_preempt"][0])
    seq0_after = ints(g["seq0_table_after_append"][0])
    rng = np.random.default_rng(61)
    Hkv, D, Hq = 2, 16, 4
    for dtype in (F32, BF16):
        # tables as the pages print them: sequence s holds blocks 2s, 2s + 1
        tables = [[2 * s, 2 * s + 1] for s in range(n_seq)]
        assert tables[victim] == freed
        rows = [to_storage(rng.standard_normal((L, Hkv, D)), dtype) for _ in range(n_seq)]
        kc, vc = _poisoned_pool((n_blocks, B, Hkv, D), dtype), _poisoned_pool((n_blocks, B, Hkv, D), dtype)
        for s in range(n_seq):
            sequential_fill(kc, tables[s], rows[s])
            sequential_fill(vc, tables[s], [r[::-1] for r in rows[s]])
        q = to_storage(rng.standard_normal((1, Hq, D)), dtype)
        bt = np.array([tables[victim]], np.int32)
        before = orc.attention_decode(q, kc, vc, bt, np.array([L], np.int32), 0.3, dtype)
        hk, hv = orc.swap_out(kc, vc, tables[victim], dtype)
        # seq-0 grows into the first freed block (its table as printed) and writes token L there
        assert seq0_after[:2] == tables[0] and seq0_after[2] == freed[0]
        new_k = to_storage(rng.standard_normal((1, Hkv, D)), dtype)
        orc.append(new_k, new_k.copy(), kc, vc, np.array([seq0_after], np.int32), np.array([L], np.int32), dtype)
        # seq-0 and seq-1 finish; the victim comes back into blocks 1 and 2
        back = [1, 2]
        orc.swap_in(kc, vc, back, hk, hv, dtype)
        assert np.array_equal(orc.gather(kc, back, L, dtype), from_storage(rows[victim], dtype).transpose(1, 0, 2))
        after = orc.attention_decode(q, kc, vc, np.array([back], np.int32), np.array([L], np.int32), 0.3, dtype)
        assert np.array_equal(before, after), "attention changed across swap-out / swap-in (dtype %d)" % dtype
        # block 6 now holds seq-0's token in row 0 and the victim's old rows after it, untouched by the swap
        assert np.array_equal(_bits(kc[freed[0], 0]), _bits(new_k[0]))
        assert np.array_equal(_bits(kc[freed[0], 1:]), _bits(hk[0, 1:]))


def pin_swap_rejects_bad_blocks(orc):
    k = _poisoned_pool((4, 4, 2, 8), F16)
    v = k.copy()
    snap = k.copy()
    for bad in ([4], [-1], [0, 9]):
        try:
            orc.swap_out(k, v, bad, F16)
        except ValueError:
            pass
        else:
            raise AssertionError("swap_out accepted %r" % (bad,))
    hk, hv = orc.swap_out(k, v, [1, 3], F16)
    try:
        orc.swap_in(k, v, [1, 7], hk, hv, F16)
    except ValueError:
        pass
    else:
        raise AssertionError("swap_in accepted block 7 of 4")
    assert np.array_equal(_bits(k), _bits(snap)), "a rejected swap wrote something"


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
