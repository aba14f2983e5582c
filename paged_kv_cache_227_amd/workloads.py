"""Seeded synthetic inputs for the paged KV decode path.

This module draws context lengths, assigns physical blocks through the host
allocator (``blocks.BlockAllocator``) and fills buffers with seeded random
numbers.  It holds none of the decode path's arithmetic (no address
translation, no attention); the CPU oracle and the HIP path both take their
inputs from here and from nowhere else.

Every buffer is a numpy array in *storage* form: float32 for fp32 data and the
raw uint16 bit patterns for fp16 / bf16 (numpy has no bfloat16).  Values are
drawn as float32 N(0, 1) and rounded to the storage type with round-to-nearest-
even, so the oracle and the GPU see identical bits.

Random streams: ``numpy.random.SeedSequence(seed).spawn`` gives independent
children for lengths, the block permutation, q, k, v, k_new and v_new; large
fills are split into fixed chunks with a child seed each, so the bits do not
depend on the number of threads used.

The named workloads are the five decode-step configurations: a tiny fp32 step,
a Llama-2-7B-shaped MHA layer, a GQA 8B-shaped layer, a shared system prompt
and a long-context layer.  Where their description leaves a choice open the
reading taken is written next to the code.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import math
import os
from typing import Optional, Sequence as _Seq

import numpy as np

from .blocks import BlockAllocator, Sequence

DTYPE_CODES = {"f32": 0, "f16": 1, "bf16": 2}
ELT_BYTES = {"f32": 4, "f16": 2, "bf16": 2}
BLOCK_SIZE = 16

_CHUNK = 1 << 22  # elements per independently seeded chunk
_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity")
                      else (os.cpu_count() or 1)))


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str                 # "f32" | "f16" | "bf16"
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray   # int32 [S]: tokens attended, the appended one included
    positions: np.ndarray      # int32 [S]: logical index of the appended token
    block_tables: np.ndarray   # int32 [S][max_blocks]; entries past a sequence's blocks are -1
    q: np.ndarray              # [S][Hq][D]
    k_new: np.ndarray          # [S][Hkv][D]
    v_new: np.ndarray          # [S][Hkv][D]
    k_cache: np.ndarray        # [num_blocks][B][Hkv][D]
    v_cache: np.ndarray        # [num_blocks][B][Hkv][D]
    scale: float
    seed: int
    part_tokens: int = 0       # split-K partition length; 0 leaves it to the library
    notes: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def dtype_code(self) -> int:
        return DTYPE_CODES[self.dtype]

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def kv_read_bytes(self) -> int:
        """Algorithmic K+V bytes one decode step reads: sum_s L_s * Hkv * 2 * D * elt."""
        return int(self.context_lens.astype(np.int64).sum()) * self.n_kv_heads * 2 * \
            self.head_dim * ELT_BYTES[self.dtype]

    def used_blocks(self) -> int:
        t = self.block_tables
        return int(np.unique(t[t >= 0]).size)


# --------------------------------------------------------------------------
# Random fills
# --------------------------------------------------------------------------

def _store_dtype(dtype: str):
    return np.float32 if dtype == "f32" else np.uint16


def _round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 -> storage form, round to nearest even."""
    if dtype == "f32":
        return x
    import torch
    t = torch.from_numpy(x)
    t = t.to(torch.float16 if dtype == "f16" else torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_fill(shape, dtype: str, seed_seq: np.random.SeedSequence, mult: float = 1.0) -> np.ndarray:
    """N(0,1) * mult in storage form; chunked so the bits are thread-count independent."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=_store_dtype(dtype))
    n_chunks = max(1, -(-n // _CHUNK))
    seeds = seed_seq.spawn(n_chunks)

    def work(i):
        lo, hi = i * _CHUNK, min(n, (i + 1) * _CHUNK)
        g = np.random.Generator(np.random.PCG64(seeds[i]))
        x = g.standard_normal(hi - lo, dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        out[lo:hi] = _round_to_storage(x, dtype)

    if n_chunks == 1:
        work(0)
    else:
        with _cf.ThreadPoolExecutor(_THREADS) as ex:
            list(ex.map(work, range(n_chunks)))
    return out.reshape(shape)


# --------------------------------------------------------------------------
# Builders
# --------------------------------------------------------------------------

def _tables_from_lists(tables, max_blocks: Optional[int] = None) -> np.ndarray:
    width = max(1, max(len(t) for t in tables)) if max_blocks is None else max_blocks
    bt = np.full((len(tables), width), -1, dtype=np.int32)
    for s, t in enumerate(tables):
        bt[s, :len(t)] = t
    return bt


def build(name: str, context_lens: _Seq[int], n_q_heads: int, n_kv_heads: int, head_dim: int,
          dtype: str, seed: int, num_blocks: Optional[int] = None, pool_factor: float = 1.0,
          block_size: int = BLOCK_SIZE, data_mult: float = 1.0, shuffle: bool = True,
          part_tokens: int = 0, shared_prefix_tokens: int = 0, prefix_layout: str = "shared",
          positions: Optional[_Seq[int]] = None, notes: str = "") -> Workload:
    """A decode step: each sequence s holds context_lens[s] tokens (its new token
    included), its table is grown for all of them, and the new token's position
    is context_lens[s] - 1 unless ``positions`` says otherwise.

    ``shared_prefix_tokens`` > 0 (a multiple of block_size) puts that many
    leading tokens of every sequence in one set of blocks: held once and shared
    by refcount (``prefix_layout="shared"``) or copied bit for bit into private
    blocks of each sequence (``"copied"``).
    """
    if dtype not in DTYPE_CODES:
        raise ValueError("dtype must be one of %s" % sorted(DTYPE_CODES))
    lens = np.asarray(context_lens, dtype=np.int64)
    S = lens.shape[0]
    ss = np.random.SeedSequence(seed)
    c_perm, c_q, c_k, c_v, c_kn, c_vn = ss.spawn(6)

    probe = BlockAllocator(1, block_size)
    need = [probe.blocks_needed(int(L)) for L in lens]
    n_pre = probe.blocks_needed(shared_prefix_tokens) if shared_prefix_tokens else 0
    if shared_prefix_tokens:
        if shared_prefix_tokens % block_size or np.any(lens <= shared_prefix_tokens):
            raise ValueError("the shared prefix must be block aligned and shorter than every sequence")
        if prefix_layout == "shared":
            total = n_pre + sum(n - n_pre for n in need)
        elif prefix_layout == "copied":
            total = sum(need)
        else:
            raise ValueError("prefix_layout must be 'shared' or 'copied'")
    else:
        total = sum(need)
    if num_blocks is None:
        num_blocks = max(1, int(math.ceil(pool_factor * total)))
    if total > num_blocks:
        raise ValueError("pool of %d blocks cannot hold the %d blocks needed" % (num_blocks, total))

    rng_perm = np.random.Generator(np.random.PCG64(c_perm))
    order = rng_perm.permutation(num_blocks) if shuffle else np.arange(num_blocks)
    alloc = BlockAllocator(num_blocks, block_size, free_order=order.tolist())

    # Physical placement through the allocator.
    tables = []
    if shared_prefix_tokens:
        root = Sequence("prefix", alloc)
        if prefix_layout == "shared":
            root.append_tokens(shared_prefix_tokens)
        for s in range(S):
            if prefix_layout == "shared":
                seq = root.fork("seq-%d" % s)
            else:
                seq = Sequence("seq-%d" % s, alloc)
                seq.table = alloc.allocate(n_pre)
            seq.table += alloc.allocate(need[s] - n_pre)
            tables.append(list(seq.table))
        if prefix_layout == "shared":
            # the sequences hold the prompt's blocks; the prompt itself lets go
            for b in root.table:
                alloc.free_block(b)
    else:
        for s in range(S):
            tables.append(alloc.allocate(need[s]))

    # Content is drawn per *logical* block (the prompt's blocks once, then each
    # sequence's own blocks in order) and copied block by block to wherever the
    # allocator put them, so the values do not depend on the placement.
    own = [need[s] - n_pre for s in range(S)]
    n_logical = n_pre + sum(own)
    kv_shape = (num_blocks, block_size, n_kv_heads, head_dim)
    caches = []
    for child in (c_k, c_v):
        logical = normal_fill((n_logical,) + kv_shape[1:], dtype, child, data_mult)
        cache = np.zeros(kv_shape, dtype=_store_dtype(dtype))
        off = n_pre
        for s in range(S):
            t = np.asarray(tables[s], dtype=np.int64)
            if n_pre and (prefix_layout == "copied" or s == 0):
                cache[t[:n_pre]] = logical[:n_pre]
            cache[t[n_pre:]] = logical[off:off + own[s]]
            off += own[s]
        del logical
        caches.append(cache)
    k_cache, v_cache = caches

    bt = _tables_from_lists(tables)
    pos = (lens - 1) if positions is None else np.asarray(positions, dtype=np.int64)
    scale = 1.0 / math.sqrt(head_dim)
    return Workload(
        name=name, dtype=dtype, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
        block_size=block_size, num_blocks=num_blocks,
        context_lens=lens.astype(np.int32), positions=pos.astype(np.int32), block_tables=bt,
        q=normal_fill((S, n_q_heads, head_dim), dtype, c_q, data_mult),
        k_new=normal_fill((S, n_kv_heads, head_dim), dtype, c_kn, data_mult),
        v_new=normal_fill((S, n_kv_heads, head_dim), dtype, c_vn, data_mult),
        k_cache=k_cache, v_cache=v_cache, scale=scale, seed=seed, part_tokens=part_tokens,
        notes=notes)


def _lens_rng(seed: int) -> np.random.Generator:
    # a stream of its own, apart from the ones build() spawns for data
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1])))


# --------------------------------------------------------------------------
# The five decode-step configurations
# --------------------------------------------------------------------------

SEED_BASE = 2270


def tiny(lengths_include_new: bool = True, seed: int = SEED_BASE + 1) -> Workload:
    """4 sequences, lengths {5,16,17,33}, 4 q heads, 4 KV heads, D=64, fp32,
    B=16, pool of 16 blocks in seeded random order.

    Reading: the lengths count the appended token (new token at L-1: mid-block,
    last slot of a block, and two first slots of fresh blocks).  The other
    reading (lengths before the append, attend L+1) is lengths_include_new=False.
    """
    base = np.array([5, 16, 17, 33])
    lens = base if lengths_include_new else base + 1
    return build("tiny" if lengths_include_new else "tiny_pre_append_lengths", lens, 4, 4, 64,
                 "f32", seed, num_blocks=16)


def llama2_7b(seed: int = SEED_BASE + 2) -> Workload:
    """One Llama-2-7B-shaped layer: 32/32 heads, D=128, fp16, pool 5,120 blocks
    (81,920 tokens), 64 sequences with L ~ U{128..2048}; data N(0,1)/sqrt(128).

    Reading: if the draw does not fit the pool, redraw with the next seed
    (the seed actually used is recorded)."""
    lens, s = _llama_lengths_and_seed(seed)
    return build("llama2_7b", lens, 32, 32, 128, "f16", s, num_blocks=5120,
                 data_mult=1.0 / math.sqrt(128.0))


def _llama_lengths_and_seed(seed: int):
    s = seed
    while True:
        lens = _lens_rng(s).integers(128, 2048, size=64, endpoint=True)
        if sum(-(-int(L) // BLOCK_SIZE) for L in lens) <= 5120:
            return lens, s
        s += 1000


def llama2_7b_lengths(seed: int = SEED_BASE + 2) -> np.ndarray:
    """The Llama-2-7B configuration's 64 context lengths (without drawing data)."""
    return _llama_lengths_and_seed(seed)[0]


def gqa_8b(seed: int = SEED_BASE + 3) -> Workload:
    """GQA 8B-shaped layer: 32 q heads, 8 KV heads, D=128, bf16, 256 sequences.

    Reading: prompt = round(lognormal(mu=ln 512, sigma=1)) clipped to
    [16, 4096], plus generated tokens drawn uniformly from {8,16,32,64,128};
    pool = ceil(1.25 * blocks needed), shuffled."""
    r = _lens_rng(seed)
    prompt = np.clip(np.rint(r.lognormal(math.log(512.0), 1.0, size=256)), 16, 4096).astype(np.int64)
    gen = r.choice(np.array([8, 16, 32, 64, 128]), size=256)
    return build("gqa_8b", prompt + gen, 32, 8, 128, "bf16", seed, pool_factor=1.25)


def prefix_sharing(layout: str = "shared", seed: int = SEED_BASE + 4) -> Workload:
    """128 sequences share a 1,024-token prompt (64 blocks), each followed by a
    suffix ~ U{1..512}; 32 q / 8 KV heads, D=128, bf16.

    Reading: the shared layout holds the prompt once at refcount 128 (one
    reference per sequence); the copied layout gives every sequence 64 private
    blocks with bit-identical contents.  Both draw identical lengths and data
    for the prompt, so their outputs must be identical."""
    suffix = _lens_rng(seed).integers(1, 512, size=128, endpoint=True)
    return build("prefix_" + layout, 1024 + suffix, 32, 8, 128, "bf16", seed,
                 shared_prefix_tokens=1024, prefix_layout=layout)


def long_context(seed: int = SEED_BASE + 5, num_seqs: int = 8) -> Workload:
    """8 sequences with L ~ U{32768..131072}; 64 q heads, 8 KV heads, D=128,
    bf16; pool = ceil(1.05 * blocks needed), fully shuffled; 512-token split-K
    partitions merged by log-sum-exp."""
    lens = _lens_rng(seed).integers(32768, 131072, size=num_seqs, endpoint=True)
    return build("long_context", lens, 64, 8, 128, "bf16", seed, pool_factor=1.05, part_tokens=512)


def with_block_size(base: str, B: int) -> Workload:
    """A decode configuration with cache blocks of B tokens instead of 16: the
    same lengths, head shape, dtype and data; the pool holds the same number of
    tokens (or, if the coarser blocks waste more, just enough blocks)."""
    if base == "llama2_7b":
        lens, seed = _llama_lengths_and_seed(SEED_BASE + 2)
        need = sum(-(-int(L) // B) for L in lens)
        return build("llama2_7b_b%d" % B, lens, 32, 32, 128, "f16", seed, num_blocks=max(5120 * 16 // B, need),
                     block_size=B, data_mult=1.0 / math.sqrt(128.0))
    if base == "gqa_8b":
        seed = SEED_BASE + 3
        r = _lens_rng(seed)
        prompt = np.clip(np.rint(r.lognormal(math.log(512.0), 1.0, size=256)), 16, 4096).astype(np.int64)
        gen = r.choice(np.array([8, 16, 32, 64, 128]), size=256)
        return build("gqa_8b_b%d" % B, prompt + gen, 32, 8, 128, "bf16", seed, pool_factor=1.25, block_size=B)
    raise ValueError("block-size variants exist for llama2_7b and gqa_8b")


CONFIGS = {
    "tiny": tiny,
    "llama2_7b": llama2_7b,
    "gqa_8b": gqa_8b,
    "prefix_shared": lambda: prefix_sharing("shared"),
    "prefix_copied": lambda: prefix_sharing("copied"),
    "long_context": long_context,
}
# the block-size sweep: B in {8, 32, 64} next to the 16 of the configurations above
for _base in ("llama2_7b", "gqa_8b"):
    for _B in (8, 32, 64):
        CONFIGS["%s_b%d" % (_base, _B)] = (lambda b=_base, B=_B: with_block_size(b, B))


# --------------------------------------------------------------------------
# Chunked prefill
# --------------------------------------------------------------------------

@dataclasses.dataclass
class PrefillWorkload:
    """One chunked-prefill step.  Sequence s holds context_lens[s] tokens once
    its chunk of n_s = cu_q[s+1] - cu_q[s] tokens is appended (positions
    context_lens[s] - n_s ..); q, k_new and v_new are the packed chunk rows.
    The caches hold data for every position, the chunk's slots included (the
    append overwrites those)."""
    name: str
    dtype: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    context_lens: np.ndarray   # int32 [S]
    cu_q: np.ndarray           # int32 [S + 1]
    block_tables: np.ndarray   # int32 [S][max_blocks]
    q: np.ndarray              # [total][Hq][D]
    k_new: np.ndarray          # [total][Hkv][D]
    v_new: np.ndarray          # [total][Hkv][D]
    k_cache: np.ndarray
    v_cache: np.ndarray
    scale: float
    seed: int
    notes: str = ""

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def chunk_lens(self) -> np.ndarray:
        return np.diff(self.cu_q).astype(np.int32)

    @property
    def start_pos(self) -> np.ndarray:
        return (self.context_lens - self.chunk_lens).astype(np.int32)

    @property
    def max_q_len(self) -> int:
        return int(self.chunk_lens.max()) if self.num_seqs else 0

    @property
    def dtype_code(self) -> int:
        return DTYPE_CODES[self.dtype]

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_tables.shape[1])

    def attention_flops(self) -> int:
        """Algorithmic flops of the attention: 4 * head_dim per (query head, key)
        pair a query sees (QK and PV, a multiply-add counted as two)."""
        n = self.chunk_lens.astype(np.int64)
        ctx = self.start_pos.astype(np.int64)
        pairs = int(np.sum(n * ctx + n * (n + 1) // 2))
        return 4 * self.head_dim * self.n_q_heads * pairs

    def kv_bytes(self) -> int:
        """K and V bytes of all positions the chunk's queries see (each once)."""
        return int(np.sum(self.context_lens, dtype=np.int64)) * 2 * self.n_kv_heads * self.head_dim * \
            ELT_BYTES[self.dtype]


def build_prefill(name: str, context: _Seq[int], chunk: _Seq[int], n_q_heads: int, n_kv_heads: int,
                  head_dim: int, dtype: str, seed: int, pool_factor: float = 1.0, data_mult: float = 1.0,
                  notes: str = "", block_size: int = BLOCK_SIZE) -> PrefillWorkload:
    """Sequence s has context[s] tokens cached and a chunk of chunk[s] new ones.
    Tables, caches and scale come from ``build`` (same seeded streams); the
    chunk's q / k_new / v_new rows come from a stream of their own."""
    context = np.asarray(context, dtype=np.int64)
    chunk = np.asarray(chunk, dtype=np.int64)
    lens = context + chunk
    w = build(name, lens, n_q_heads, n_kv_heads, head_dim, dtype, seed, pool_factor=pool_factor,
              data_mult=data_mult, notes=notes, block_size=block_size)
    c_q, c_kn, c_vn = np.random.SeedSequence([seed, 11]).spawn(3)
    total = int(chunk.sum())
    cu = np.concatenate([[0], np.cumsum(chunk)]).astype(np.int32)
    return PrefillWorkload(
        name=name, dtype=dtype, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim,
        block_size=w.block_size, num_blocks=w.num_blocks, context_lens=lens.astype(np.int32), cu_q=cu,
        block_tables=w.block_tables, q=normal_fill((total, n_q_heads, head_dim), dtype, c_q, data_mult),
        k_new=normal_fill((total, n_kv_heads, head_dim), dtype, c_kn, data_mult),
        v_new=normal_fill((total, n_kv_heads, head_dim), dtype, c_vn, data_mult),
        k_cache=w.k_cache, v_cache=w.v_cache, scale=w.scale, seed=seed, notes=notes)


def _b_suffix(block_size: int) -> str:
    return "" if block_size == BLOCK_SIZE else "_b%d" % block_size


def prefill_llama2_7b(chunk: int = 512, seed: int = SEED_BASE + 7, block_size: int = BLOCK_SIZE) -> PrefillWorkload:
    """Chunked prefill of 2,048-token prompts on the Llama-2-7B layer (32/32
    heads, D=128, fp16; data N(0,1)/sqrt(128)), one step with four prompts at
    the four stages of a 512-token chunking: contexts 0, 512, 1024 and 1536
    tokens cached, each with its next 512-token chunk."""
    stages = 2048 // chunk
    return build_prefill("prefill_llama2_7b" + _b_suffix(block_size), [i * chunk for i in range(stages)],
                         [chunk] * stages, 32, 32, 128, "f16", seed, data_mult=1.0 / math.sqrt(128.0),
                         notes="2048-token prompts in %d-token chunks, one prompt per stage" % chunk,
                         block_size=block_size)


def prefill_gqa_8b(chunk: int = 512, seed: int = SEED_BASE + 8, block_size: int = BLOCK_SIZE) -> PrefillWorkload:
    """The same chunking on the GQA 8B layer (32 q heads, 8 KV heads, D=128, bf16)."""
    stages = 2048 // chunk
    return build_prefill("prefill_gqa_8b" + _b_suffix(block_size), [i * chunk for i in range(stages)],
                         [chunk] * stages, 32, 8, 128, "bf16", seed,
                         notes="2048-token prompts in %d-token chunks, one prompt per stage" % chunk,
                         block_size=block_size)


PREFILL_CONFIGS = {
    "prefill_llama2_7b": prefill_llama2_7b,
    "prefill_gqa_8b": prefill_gqa_8b,
}
# the same steps with the caches in blocks of 8, 32 or 64 tokens (prefill_<layer>_b<B>)
for _base, _fn in list(PREFILL_CONFIGS.items()):
    for _B in (8, 32, 64):
        PREFILL_CONFIGS["%s_b%d" % (_base, _B)] = (lambda f=_fn, B=_B: f(block_size=B))


# --------------------------------------------------------------------------
# Block copies (copy-on-write, whole-block moves)
# --------------------------------------------------------------------------

@dataclasses.dataclass
class CopyWorkload:
    """A batch of block copies on one layer's caches: rows [0, rows[i]) of block
    src[i] to block dst[i], both caches.  Cache contents do not matter for
    timing; tests draw their own."""
    name: str
    dtype: str
    n_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    src: np.ndarray   # int32 [n]
    dst: np.ndarray   # int32 [n]
    rows: np.ndarray  # int32 [n]
    seed: int
    notes: str = ""

    @property
    def row_bytes(self) -> int:
        return self.n_kv_heads * self.head_dim * ELT_BYTES[self.dtype]

    def moved_bytes(self) -> int:
        """Bytes read (= bytes written) by one call: both caches."""
        return 2 * int(np.sum(self.rows, dtype=np.int64)) * self.row_bytes


def cow_llama2_7b(samples: int = 4, seed: int = SEED_BASE + 2) -> CopyWorkload:
    """One fork wave of parallel sampling on the Llama-2-7B layer: each of the
    64 sequences (lengths as in the Llama-2-7B configuration) is forked into
    `samples` samples, and each sample's first generated token copies the
    shared last block's filled rows (L mod 16 of them) into a private block.
    The host block manager decides every block; the pool is 5,120 blocks plus
    one per sample, in seeded shuffled order."""
    base = llama2_7b_lengths(seed)
    n_pool = 5120 + samples * len(base)
    order = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 7]))).permutation(n_pool)
    alloc = BlockAllocator(n_pool, BLOCK_SIZE, free_order=order)
    copies = []
    for L in base:
        prompt = Sequence("p", alloc)
        prompt.append_tokens(int(L))
        for i in range(samples):
            child = prompt.fork("s%d" % i)
            child.append_tokens(1)
            copies += child.take_copies()
    src, dst, rows = (np.array(x, np.int32) for x in zip(*copies))
    return CopyWorkload("cow_llama2_7b", "f16", 32, 128, BLOCK_SIZE, n_pool, src, dst, rows, seed,
                        notes="%d sequences x %d samples; sequences with L mod 16 = 0 need no copy"
                              % (len(base), samples))


def copy_whole_llama2_7b(n: int = 2048, seed: int = SEED_BASE + 6) -> CopyWorkload:
    """`n` whole-block copies (16 rows x 8 KiB per cache) in the Llama-2-7B
    layer's 5,120-block pool: distinct sources and targets in seeded order."""
    perm = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 8]))).permutation(5120)
    return CopyWorkload("copy_whole_llama2_7b", "f16", 32, 128, BLOCK_SIZE, 5120,
                        perm[:n].astype(np.int32), perm[n:2 * n].astype(np.int32),
                        np.full(n, BLOCK_SIZE, np.int32), seed)


def swap_llama2_7b(n_victims: int = 8, seed: int = SEED_BASE + 2) -> CopyWorkload:
    """Preemption by swapping on the Llama-2-7B layer: the `n_victims` longest of
    its 64 sequences are swapped out (all their blocks, in table order) and back.
    src = the blocks swapped out; dst = the blocks swapped back into (the same
    ones here: the pool is otherwise idle); rows = whole blocks."""
    w = llama2_7b(seed)
    order = np.argsort(-w.context_lens, kind="stable")[:n_victims]
    blocks = np.concatenate([w.block_tables[s][w.block_tables[s] >= 0] for s in order]).astype(np.int32)
    return CopyWorkload("swap_llama2_7b", "f16", 32, 128, BLOCK_SIZE, w.num_blocks, blocks, blocks.copy(),
                        np.full(len(blocks), BLOCK_SIZE, np.int32), seed,
                        notes="the %d longest sequences (%d tokens)" % (n_victims, int(w.context_lens[order].sum())))


SWAP_CONFIGS = {"swap_llama2_7b": swap_llama2_7b}


COPY_CONFIGS = {
    "cow_llama2_7b": cow_llama2_7b,
    "copy_whole_llama2_7b": copy_whole_llama2_7b,
}


def small(num_seqs: int, lens, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: str,
          seed: int, **kw) -> Workload:
    """A small ad-hoc workload for tests (same generator, explicit lengths)."""
    lens = np.asarray(lens, dtype=np.int64)
    assert lens.shape[0] == num_seqs
    return build("small", lens, n_q_heads, n_kv_heads, head_dim, dtype, seed, **kw)


def to_torch(w: Workload, device):
    """Torch tensors holding the workload's buffers on ``device`` (memory only)."""
    import torch
    tdt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[w.dtype]

    def t(a):
        x = torch.from_numpy(np.ascontiguousarray(a))
        if w.dtype != "f32":
            x = x.view(torch.int16).view(tdt)
        return x.to(device)

    def i(a):
        return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)

    return dict(q=t(w.q), k_new=t(w.k_new), v_new=t(w.v_new), k_cache=t(w.k_cache),
                v_cache=t(w.v_cache), block_tables=i(w.block_tables),
                context_lens=i(w.context_lens), positions=i(w.positions))
