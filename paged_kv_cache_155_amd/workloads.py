"""Seeded synthetic inputs for paged-attention decode.

This module only draws inputs: random lengths, block tables, fp16 tensors and
the slots a block manager would hand out.  It holds none of the attention
arithmetic and imports neither the GPU binding nor the CPU oracle, so both
sides are fed the very same host bytes.

Shapes follow the pages' models: LLaMA-7B (32 heads of 128, "深入解析LLM推理引擎"
§2.1) and LLaMA-13B (40 heads of 128, "vLLM推理加速深度解读" §2.1); block
sizes 16 and 32 ("vLLM推理加速深度解读" §2.3).  Physical block ids come from a
seeded permutation without replacement, which is what popping a free list in
random order produces ("深入解析LLM推理引擎" §3.3).

Random streams: numpy PCG64.  Lengths, queries and new tokens come from
children of SeedSequence([155, config, variant]); the block table, K/V pools,
outlier picks and free-slot picks from children of SeedSequence([155, config,
variant, block size]).  Every array has its own child stream.  Normals are drawn in
float32 and rounded to fp16 (round to nearest even).
"""
from __future__ import annotations

import dataclasses
import math
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SEED = 155
_CHUNK = 1 << 22  # elements per drawing chunk (bounds the float32 temporary)

DESCRIPTIONS = {
    0: "tiny: 4 seqs ctx {1,17,33,100}, 4 heads x 64, B=16, pool 64 blocks",
    1: "LLaMA-7B layer: 64 seqs ctx U[1,2048], 32 heads x 128, B=16",
    2: "LLaMA-13B layer: 256 seqs ctx 70% U[16,512] / 30% U[512,4096], 40 heads x 128",
    3: "shared prefix: 128 seqs, 32-block (512-token) common prefix + U[1,512] suffix, "
       "32 heads x 128, B=16",
    4: "long context: 8 seqs ctx 32768, 32 heads x 128, B=16, 1% x8 key outliers, P=512",
}


@dataclasses.dataclass
class Workload:
    """One decode step of one layer, as host arrays (fp16 stored as np.float16)."""
    name: str
    config: int
    num_seqs: int
    num_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    max_blocks_per_seq: int
    partition_size: int
    scale: np.float32
    q: np.ndarray             # [S, H, D] fp16
    k_cache: np.ndarray       # [NB, B, H, D] fp16 (before the new tokens are written)
    v_cache: np.ndarray       # [NB, B, H, D] fp16
    block_tables: np.ndarray  # [S, MB] int32 (entries past the context: poison block)
    context_lens: np.ndarray  # [S] int32 (counts the token written this step)
    key: np.ndarray           # [T, H, D] fp16 new keys
    value: np.ndarray         # [T, H, D] fp16 new values
    slot_mapping: np.ndarray  # [T] int64
    poison_block: int         # block id filled with NaN, used to pad the tables
    ref_counts: np.ndarray    # [NB] int32 table references per physical block

    @property
    def num_tokens(self):
        return int(self.slot_mapping.shape[0])

    def kv_bytes(self):
        """K+V bytes the decode must read: sum of context lengths x H x D x 2 x 2."""
        return kv_bytes_per_token(self.num_heads, self.head_dim) * int(self.context_lens.sum())

    def unique_kv_bytes(self):
        """K+V bytes of the distinct (physical block, position) slots read."""
        B = self.block_size
        used = {}  # physical block -> most positions any sequence reads from it
        for s in range(self.num_seqs):
            L = int(self.context_lens[s])
            for j in range((L + B - 1) // B):
                pb = int(self.block_tables[s, j])
                used[pb] = max(used.get(pb, 0), min(B, L - j * B))
        return kv_bytes_per_token(self.num_heads, self.head_dim) * sum(used.values())


def kv_bytes_per_token(num_heads, head_dim, dtype_bytes=2):
    """Bytes of K plus V for one token in one layer: 2 x heads x head_dim x dtype."""
    return 2 * num_heads * head_dim * dtype_bytes


def _threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _normal_f16(seq, shape):
    """N(0,1) fp16 array; chunk c of _CHUNK elements is drawn from the child
    stream SeedSequence(seq.entropy, spawn_key=seq.spawn_key + (c,)), so the
    values do not depend on the thread count."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float16)

    def fill(c):
        g = np.random.Generator(np.random.PCG64(
            np.random.SeedSequence(seq.entropy, spawn_key=tuple(seq.spawn_key) + (c,))))
        i = c * _CHUNK
        out[i:i + min(_CHUNK, n - i)] = g.standard_normal(min(_CHUNK, n - i), dtype=np.float32)

    chunks = range(-(-n // _CHUNK))
    if n > _CHUNK:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, chunks))
    else:
        for c in chunks:
            fill(c)
    return out.reshape(shape)


_SEQ_STREAMS = ["lens", "q", "newk", "newv"]
_POOL_STREAMS = ["table", "k", "v", "outlier", "slots"]


def _streams(config, block_size, variant):
    """Per-sequence draws depend on (config, variant) only, so both block
    sizes of a configuration see the same lengths and queries; pool draws
    also depend on the block size."""
    seq = np.random.SeedSequence([SEED, config, variant])
    pool = np.random.SeedSequence([SEED, config, variant, block_size])
    st = dict(zip(_SEQ_STREAMS, seq.spawn(len(_SEQ_STREAMS))))
    st.update(zip(_POOL_STREAMS, pool.spawn(len(_POOL_STREAMS))))
    return st


def _gen(seq):
    return np.random.Generator(np.random.PCG64(seq))


def _draw_lengths(config, S, rng):
    if config == 0:
        return np.array([1, 17, 33, 100], dtype=np.int64)[:S]
    if config == 1:
        return rng.integers(1, 2048, size=S, endpoint=True)
    if config == 2:
        short = rng.integers(16, 512, size=S, endpoint=True)
        long_ = rng.integers(512, 4096, size=S, endpoint=True)
        pick_short = rng.random(S) < 0.7
        return np.where(pick_short, short, long_)
    if config == 3:
        return 512 + rng.integers(1, 512, size=S, endpoint=True)
    if config == 4:
        return np.full(S, 32768, dtype=np.int64)
    raise ValueError(config)


# config -> (S, H, D, B default, max context, partition size).  The partition
# sizes are the launch configuration the benchmark times: the 32K-context
# case is specified with 512-token partitions; for the others the size was
# picked by measurement on MI355X (0 = no split: one work unit per sequence
# and head, which wins for the shared-prefix batch).
_SHAPES = {
    0: (4, 4, 64, 16, 100, 16),
    1: (64, 32, 128, 16, 2048, 512),
    2: (256, 40, 128, 16, 4096, 1024),
    3: (128, 32, 128, 16, 1024, 0),
    4: (8, 32, 128, 16, 32768, 512),
}


def make_workload(config, block_size=None, num_seqs=None, num_heads=None, variant=0,
                  poison=True, partition_size=None):
    """Draw one configuration.

    num_seqs / num_heads shrink a configuration for quick parity runs while
    keeping its length distribution, block size and table structure.
    poison=True fills every slot that must never be read (positions at or
    past a sequence's context in its last block, the table padding block and
    the slot about to receive the new token) with fp16 NaN.
    """
    S0, H0, D, B0, max_ctx, P0 = _SHAPES[config]
    S = S0 if num_seqs is None else int(num_seqs)
    H = H0 if num_heads is None else int(num_heads)
    B = B0 if block_size is None else int(block_size)
    P = P0 if partition_size is None else int(partition_size)
    st = _streams(config, B, variant)
    MB = -(-max_ctx // B)

    lens = _draw_lengths(config, S, _gen(st["lens"])).astype(np.int64)
    if config == 3:
        n_prefix = 512 // B
        suffix_blocks = [-(-(int(L) - 512) // B) for L in lens]
        needed = n_prefix + sum(suffix_blocks)
    else:
        n_prefix = 0
        needed = sum(-(-int(L) // B) for L in lens)
    NB = 64 if config == 0 else int(math.ceil(1.1 * needed))
    NB = max(NB, needed + 1)  # at least one spare block for the poison padding
    perm = _gen(st["table"]).permutation(NB).astype(np.int64)

    tables = np.empty((S, MB), dtype=np.int32)
    cursor = 0
    prefix_ids = perm[:n_prefix]
    cursor = n_prefix
    owned = []
    for s in range(S):
        L = int(lens[s])
        if config == 3:
            nsuf = -(-(L - 512) // B)
            ids = np.concatenate([prefix_ids, perm[cursor:cursor + nsuf]])
            cursor += nsuf
        else:
            n = -(-L // B)
            ids = perm[cursor:cursor + n]
            cursor += n
        owned.append(ids)
    poison_block = int(perm[cursor])
    cursor += 1
    for s in range(S):
        tables[s, :] = poison_block
        tables[s, :len(owned[s])] = owned[s]

    ref = np.zeros(NB, dtype=np.int32)
    for s in range(S):
        np.add.at(ref, owned[s].astype(np.int64), 1)
    if config == 3:
        assert np.all(ref[prefix_ids] == S), "shared prefix blocks must be referenced by all"

    q = _normal_f16(st["q"], (S, H, D))
    k_cache = _normal_f16(st["k"], (NB, B, H, D))
    v_cache = _normal_f16(st["v"], (NB, B, H, D))
    T = S
    key = _normal_f16(st["newk"], (T, H, D))
    value = _normal_f16(st["newv"], (T, H, D))

    if config == 4:
        # 1% of (physical slot, head) key vectors scaled by 8 (exact in fp16)
        rng = _gen(st["outlier"])
        for arr in (k_cache, key):
            flat = arr.reshape(-1, D)
            sel = rng.random(flat.shape[0]) < 0.01
            flat[sel] = flat[sel] * np.float16(8)

    if config == 0:
        # the new tokens go to random free slots: slots that hold none of the
        # live positions and are not in the poison block
        live = np.zeros(NB * B, dtype=bool)
        for s in range(S):
            for i in range(int(lens[s])):
                live[int(tables[s, i // B]) * B + i % B] = True
        live[poison_block * B:(poison_block + 1) * B] = True
        free = np.flatnonzero(~live)
        T = 4
        key, value = key[:T], value[:T]
        slots = _gen(st["slots"]).choice(free, size=T, replace=False).astype(np.int64)
    else:
        # one new token per sequence at logical position ctx-1: the slot the
        # block manager assigned to that position
        pos = lens - 1
        slots = np.array([int(tables[s, pos[s] // B]) * B + int(pos[s] % B) for s in range(S)],
                         dtype=np.int64)

    if poison:
        nan = np.float16(np.nan)
        k_cache[poison_block] = nan
        v_cache[poison_block] = nan
        for s in range(S):
            L = int(lens[s])
            if L % B:
                last = int(tables[s, (L - 1) // B])
                if config != 3 or (L - 1) // B >= n_prefix:
                    k_cache[last, L % B:] = nan
                    v_cache[last, L % B:] = nan
        if config != 0:
            kf = k_cache.reshape(NB * B, H, D)
            vf = v_cache.reshape(NB * B, H, D)
            kf[slots] = nan
            vf[slots] = nan

    return Workload(
        name=f"config{config}" + (f"_B{B}" if block_size else ""),
        config=config, num_seqs=S, num_heads=H, head_dim=D, block_size=B, num_blocks=NB,
        max_blocks_per_seq=MB, partition_size=P, scale=np.float32(1.0 / math.sqrt(D)),
        q=q, k_cache=k_cache, v_cache=v_cache, block_tables=tables,
        context_lens=lens.astype(np.int32), key=key, value=value, slot_mapping=slots,
        poison_block=poison_block, ref_counts=ref)


def make_random(context_lens, num_heads, head_dim, block_size, seed=0, partition_size=512,
                max_blocks_per_seq=None, spare_blocks=3, poison=True):
    """A custom-shaped workload for edge cases: the given context lengths,
    scattered tables from a seeded permutation, N(0,1) fp16 data, one new
    token per sequence with ctx > 0 (written at position ctx-1; sequences
    with ctx == 0 get slot -1, i.e. no write)."""
    lens = np.asarray(context_lens, dtype=np.int64)
    S, H, D, B = len(lens), int(num_heads), int(head_dim), int(block_size)
    ss = np.random.SeedSequence([SEED, 1000, seed])
    st = dict(zip(["table", "q", "k", "v", "newk", "newv"], ss.spawn(6)))
    nblk = [-(-int(L) // B) for L in lens]
    MB = max(1, max(nblk, default=1)) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    NB = sum(nblk) + 1 + int(spare_blocks)
    perm = _gen(st["table"]).permutation(NB).astype(np.int64)
    poison_block = int(perm[-1])
    tables = np.full((S, MB), poison_block, dtype=np.int32)
    c = 0
    for s, n in enumerate(nblk):
        tables[s, :n] = perm[c:c + n]
        c += n
    ref = np.zeros(NB, dtype=np.int32)
    for s, n in enumerate(nblk):
        np.add.at(ref, tables[s, :n].astype(np.int64), 1)
    q = _normal_f16(st["q"], (S, H, D))
    k_cache = _normal_f16(st["k"], (NB, B, H, D))
    v_cache = _normal_f16(st["v"], (NB, B, H, D))
    key = _normal_f16(st["newk"], (S, H, D))
    value = _normal_f16(st["newv"], (S, H, D))
    slots = np.full(S, -1, dtype=np.int64)
    for s in range(S):
        if lens[s] > 0:
            p = int(lens[s]) - 1
            slots[s] = int(tables[s, p // B]) * B + p % B
    if poison:
        nan = np.float16(np.nan)
        k_cache[poison_block] = nan
        v_cache[poison_block] = nan
        for s in range(S):
            L = int(lens[s])
            if L % B:
                k_cache[tables[s, (L - 1) // B], L % B:] = nan
                v_cache[tables[s, (L - 1) // B], L % B:] = nan
        ok = slots >= 0
        k_cache.reshape(NB * B, H, D)[slots[ok]] = nan
        v_cache.reshape(NB * B, H, D)[slots[ok]] = nan
    return Workload(
        name="random", config=-1, num_seqs=S, num_heads=H, head_dim=D, block_size=B,
        num_blocks=NB, max_blocks_per_seq=MB, partition_size=int(partition_size),
        scale=np.float32(1.0 / math.sqrt(D)), q=q, k_cache=k_cache, v_cache=v_cache,
        block_tables=tables, context_lens=lens.astype(np.int32), key=key, value=value,
        slot_mapping=slots, poison_block=poison_block, ref_counts=ref)


@dataclasses.dataclass
class Fp8Pools:
    """FP8 (OCP E4M3) copies of a workload's K/V pools."""
    k_cache: np.ndarray   # [NB, B, H, D] uint8 codes
    v_cache: np.ndarray
    k_scale: np.float32
    v_scale: np.float32


def fp8_pools(w, headroom=1.0):
    """Quantise a workload's pools for the FP8 cache variant: one scale per
    cache, scale = amax(|pool and new tokens|) / 448 (the largest E4M3 value,
    so nothing saturates), codes from torch's float -> float8_e4m3fn cast of
    x * (1/scale) on the host.  These are *inputs*: any valid codes with a
    realistic spread will do; never-read NaN slots stay NaN codes."""
    import torch

    def scale_of(a, b):
        amax = max(float(np.nanmax(np.abs(a.astype(np.float32)))) if a.size else 0.0,
                   float(np.nanmax(np.abs(b.astype(np.float32)))) if b.size else 0.0)
        return np.float32(max(amax, 1e-6) * headroom / 448.0)

    def quant(a, scale):
        inv = np.float32(1.0 / float(scale))
        t = torch.from_numpy(a.reshape(-1))
        out = torch.empty(t.numel(), dtype=torch.uint8)
        step = 1 << 24
        for i in range(0, t.numel(), step):
            y = t[i:i + step].float() * float(inv)
            out[i:i + step] = y.to(torch.float8_e4m3fn).view(torch.uint8)
        return out.numpy().reshape(a.shape)

    ks = scale_of(w.k_cache, w.key)
    vs = scale_of(w.v_cache, w.value)
    return Fp8Pools(k_cache=quant(w.k_cache, ks), v_cache=quant(w.v_cache, vs), k_scale=ks,
                    v_scale=vs)


def make_multi_query(context_lens, query_lens, num_heads, head_dim, block_size, seed=0,
                     poison=True):
    """Inputs of a multi-query (chunked prefill / mixed) batch: sequence s has
    context_lens[s] positions in the cache, of which the last query_lens[s]
    are this step's new tokens; q holds their rows, query_start the offsets.
    Returns (Workload, q [T, H, D] fp16, query_start [S + 1] int32)."""
    w = make_random(context_lens, num_heads, head_dim, block_size, seed=seed, poison=poison)
    qlen = np.asarray(query_lens, dtype=np.int64)
    assert np.all(qlen <= w.context_lens) and np.all(qlen >= 0)
    qs = np.concatenate([[0], np.cumsum(qlen)]).astype(np.int32)
    ss = np.random.SeedSequence([SEED, 2000, seed])
    q = _normal_f16(ss, (int(qs[-1]), w.num_heads, w.head_dim))
    return w, q, qs


def split_shared_prefix(w, prefix_blocks):
    """For a workload whose tables all start with the same prefix_blocks ids
    (the shared-prefix configuration): the prefix table, its length, and the
    suffix tables / lengths that pa_decode_cascade takes."""
    prefix = w.block_tables[0, :prefix_blocks].copy()
    assert np.all(w.block_tables[:, :prefix_blocks] == prefix)
    B = w.block_size
    suffix_tables = np.ascontiguousarray(w.block_tables[:, prefix_blocks:])
    suffix_lens = (w.context_lens - prefix_blocks * B).astype(np.int32)
    assert np.all(suffix_lens >= 0)
    return prefix.astype(np.int32), prefix_blocks * B, suffix_tables, suffix_lens
