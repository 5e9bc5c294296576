"""Matrix-core paths against the oracle: multi-query (chunked-prefill) paged
attention, and the shared-prefix (cascade) decode, which must equal the
plain decode over the concatenated tables."""
import numpy as np
import pytest

from gpu_util import (DeviceWorkload, assert_close, assert_close_split_rows, log,
                      oracle_after_write, to_dev)

pytestmark = pytest.mark.gpu


def _run_mq(orc, w, q, qs, max_q):
    import torch
    import paged_kv_cache_155_amd as pa
    out = to_dev(np.full(q.shape, np.nan, dtype=np.float16))
    pa.multi_query(out, to_dev(q), to_dev(w.k_cache), to_dev(w.v_cache), to_dev(w.block_tables),
                   to_dev(w.context_lens), to_dev(qs), max_q, float(w.scale))
    torch.cuda.synchronize()
    ref = orc.prefill(q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, qs, float(w.scale))
    return out.cpu().numpy(), ref


def _live(w):
    """Pools without the NaN that make_random puts in the slot of each
    sequence's last position (these tests write no new token)."""
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    ok = w.slot_mapping >= 0
    kc.reshape(-1, w.num_heads, w.head_dim)[w.slot_mapping[ok]] = np.float16(0.25)
    vc.reshape(-1, w.num_heads, w.head_dim)[w.slot_mapping[ok]] = np.float16(-0.5)
    w.k_cache, w.v_cache = kc, vc
    return w


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("B", [16, 32])
def test_multi_query_sweep(orc, D, B):
    from paged_kv_cache_155_amd.workloads import make_multi_query
    ctx = [1, 5, 16, 17, 31, 32, 33, 100, 257, 300, 1000, 64]
    qn = [1, 5, 16, 1, 16, 17, 33, 37, 200, 1, 300, 64]    # last: a whole prompt
    log(f"[mq] multi-query sweep D={D} B={B}")
    w, q, qs = make_multi_query(ctx, qn, 3, D, B, seed=D + B)
    got, ref = _run_mq(orc, _live(w), q, qs, max(qn))
    assert_close(got, ref, f"multi-query D={D} B={B}")


def test_multi_query_single_rows_equal_decode(orc):
    from paged_kv_cache_155_amd.workloads import make_multi_query
    log("[mq] one row per sequence = decode")
    ctx = [1, 40, 700, 2048, 129]
    w, q, qs = make_multi_query(ctx, [1] * 5, 4, 128, 16, seed=7)
    w = _live(w)
    got, ref = _run_mq(orc, w, q, qs, 1)
    dec = orc.decode(q, w.k_cache, w.v_cache, w.block_tables, w.context_lens, float(w.scale))
    assert np.array_equal(ref.view(np.uint64), dec.view(np.uint64))
    assert_close(got, ref, "single-row multi-query")


def test_multi_query_chunked_prefill_batch(orc):
    """A LLaMA-7B-shaped mixed batch: 8 sequences, contexts up to 2048, new
    chunks of 1..256 tokens (1 = a decode step)."""
    from paged_kv_cache_155_amd.workloads import make_multi_query
    rng = np.random.default_rng(31)
    ctx = rng.integers(256, 2049, size=8)
    qn = [1, 256, 64, 1, 200, 17, 128, 1]
    log("[mq] chunked-prefill batch, 8 seqs, 32 heads x 128")
    w, q, qs = make_multi_query(ctx, qn, 32, 128, 16, seed=8)
    got, ref = _run_mq(orc, _live(w), q, qs, 256)
    ea, _ = assert_close(got, ref, "chunked prefill batch")
    log(f"[mq] max abs err {ea:.3e}")


def test_multi_query_empty_chunks_and_loose_bound(orc):
    """Sequences that bring no new rows (first, middle and last of the batch)
    launch only tiles that return at once, and a max_query_len three times
    the longest chunk only adds such tiles: every row that exists is written
    (the output starts as NaN) and matches the oracle."""
    from paged_kv_cache_155_amd.workloads import make_multi_query
    ctx = [40, 300, 1, 129, 700, 64]
    qn = [0, 37, 0, 129, 200, 0]
    log("[mq] empty chunks, max_query_len 3x the longest chunk")
    w, q, qs = make_multi_query(ctx, qn, 4, 128, 16, seed=21)
    got, ref = _run_mq(orc, _live(w), q, qs, 3 * max(qn))
    assert np.isfinite(got).all()
    assert_close(got, ref, "empty chunks")


def test_multi_query_late_outlier_keys(orc):
    """Keys 30x larger at a few late positions (logit jumps of tens of log2
    units after the running maximum has settled), so the kernel moves its
    reference maximum and rescales O in the middle of a stream, while most
    chunks keep a reference below their own maximum."""
    from paged_kv_cache_155_amd.workloads import make_multi_query
    rng = np.random.default_rng(5)
    ctx = [700, 1500, 333, 1024]
    qn = [300, 64, 333, 128]
    log("[mq] late outlier keys, 4 seqs, 4 heads x 128")
    w, q, qs = make_multi_query(ctx, qn, 4, 128, 16, seed=12)
    w = _live(w)
    kc = w.k_cache.copy()
    for s in range(len(ctx)):
        for pos in rng.integers(ctx[s] // 2, ctx[s], size=3):
            blk = w.block_tables[s, pos // 16]
            kc[blk, pos % 16] = (kc[blk, pos % 16].astype(np.float32) * 30).astype(np.float16)
    w.k_cache = kc
    got, ref = _run_mq(orc, w, q, qs, 333)
    ea, _ = assert_close(got, ref, "late outlier keys")
    log(f"[mq] max abs err {ea:.3e}")


@pytest.mark.parametrize("kw,P", [(dict(num_seqs=12, num_heads=2), 512),
                                  (dict(num_seqs=37, num_heads=3), 0), ({}, 512), ({}, 0)],
                         ids=["small_P512", "ragged_P0", "full_P512", "full_P0"])
def test_cascade_matches_plain_decode(orc, kw, P):
    """The shared-prefix workload through pa_decode_cascade: the oracle over
    the full tables decides; the plain decode agrees within the tolerance."""
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import make_workload, split_shared_prefix
    w = make_workload(3, **kw)
    log(f"[cascade] S={w.num_seqs} H={w.num_heads} P={P}")
    d = DeviceWorkload(w)
    d.reshape_and_cache()
    prefix, plen, suf_tables, suf_lens = split_shared_prefix(w, 32)
    out = torch.full_like(d.q, float("nan"))
    pa.decode_cascade(out, d.q, d.k_cache, d.v_cache, to_dev(prefix), plen, to_dev(suf_tables),
                      to_dev(suf_lens), float(w.scale), partition_size=P)
    plain = d.decode(P)
    torch.cuda.synchronize()
    kc, vc, ref = oracle_after_write(orc, w)
    got = out.cpu().numpy()
    ea, _ = assert_close(got, ref, "cascade")
    assert_close(got, plain.cpu().numpy().astype(np.float64), "cascade vs plain decode")
    log(f"[cascade] max abs err {ea:.3e}")


@pytest.mark.parametrize("prefix_blocks,B,D", [(4, 16, 128), (9, 16, 128), (5, 32, 128),
                                                (9, 16, 64), (5, 32, 64)],
                         ids=["prefix64_B16", "prefix144_B16", "prefix160_B32",
                              "prefix144_B16_D64", "prefix160_B32_D64"])
def test_cascade_suffix_edges(orc, prefix_blocks, B, D):
    """Suffixes of length 0 (the whole context is the prefix), 1, and a
    block and a partition boundary; a batch size that is not a multiple of 16;
    prefixes that end inside a 64-token chunk and inside a prefix partition.
    P = 0 puts every suffix in one partition (the partition kernel merges the
    prefix slots), P = 16 and 512 go through the reduce."""
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import make_random
    log(f"[cascade] suffix edges prefix {prefix_blocks} blocks of {B}, head_dim {D}")
    suffix = [0, 1, 15, 16, 17, 511, 512, 513, 0, 40, 3, 100, 64, 65, 2, 1, 0, 300]
    S = len(suffix)
    plen = prefix_blocks * B
    w = make_random([plen + x for x in suffix], 2, D, B, seed=41 + B + D, poison=True)
    w.block_tables[:, :prefix_blocks] = w.block_tables[0, :prefix_blocks]
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    ok = w.slot_mapping >= 0
    kc.reshape(-1, 2, D)[w.slot_mapping[ok]] = np.float16(0.1)   # no new token here
    vc.reshape(-1, 2, D)[w.slot_mapping[ok]] = np.float16(0.2)
    ref = orc.decode(w.q, kc, vc, w.block_tables, w.context_lens, float(w.scale))
    prefix = w.block_tables[0, :prefix_blocks].astype(np.int32)
    st = np.ascontiguousarray(w.block_tables[:, prefix_blocks:])
    sl = np.array(suffix, dtype=np.int32)
    for P in (0, B, 512):
        out = to_dev(np.full((S, 2, D), np.nan, dtype=np.float16))
        pa.decode_cascade(out, to_dev(w.q), to_dev(kc), to_dev(vc), to_dev(prefix),
                          plen, to_dev(st), to_dev(sl), float(w.scale), partition_size=P)
        torch.cuda.synchronize()
        assert_close(out.cpu().numpy(), ref, f"cascade edges P={P}")


@pytest.mark.parametrize("P", [0, 16])
def test_cascade_large_values(orc, P):
    """|v| up to 60000 through the shared-prefix path: the prefix pieces'
    rows are kept in fp16 (a normalised row lies within the range of V, so
    nothing overflows; their rounding widens the tolerance as for the split
    decode), P = 0 merges them in the partition kernel and P = 16 in the
    reduce."""
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import make_random
    log(f"[cascade] large values P={P}")
    prefix_blocks, B, D = 9, 16, 128
    suffix = [0, 1, 17, 300, 512, 40]
    plen = prefix_blocks * B
    w = make_random([plen + x for x in suffix], 2, D, B, seed=77, poison=True)
    w.block_tables[:, :prefix_blocks] = w.block_tables[0, :prefix_blocks]
    kc = w.k_cache.copy()
    vc = (np.clip(w.v_cache.astype(np.float32), -5.0, 5.0) * 12000.0).astype(np.float16)
    ok = w.slot_mapping >= 0  # the step's own slots hold poison until written: fill them
    kc.reshape(-1, 2, D)[w.slot_mapping[ok]] = w.key[ok]
    vc.reshape(-1, 2, D)[w.slot_mapping[ok]] = np.float16(-30000.0)
    ref = orc.decode(w.q, kc, vc, w.block_tables, w.context_lens, float(w.scale))
    st = np.ascontiguousarray(w.block_tables[:, prefix_blocks:])
    out = to_dev(np.full((len(suffix), 2, D), np.nan, dtype=np.float16))
    pa.decode_cascade(out, to_dev(w.q), to_dev(kc), to_dev(vc),
                      to_dev(w.block_tables[0, :prefix_blocks].astype(np.int32)), plen,
                      to_dev(st), to_dev(np.array(suffix, dtype=np.int32)), float(w.scale),
                      partition_size=P)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.isfinite(got).all() and np.abs(ref).max() > 1000.0
    assert_close_split_rows(got, ref, 60000.0, f"cascade large values P={P}")

@pytest.mark.parametrize("P", [0, 512])
def test_cascade_needles_and_late_outliers_full(orc, P):
    """Full config 3 through pa_decode_cascade with keys that stress the
    matrix-core prefix pass (fp16 weights in its P.V product) and the merge:
    needle keys (24 x a unit query of some sequence) at the prefix's chunk
    and piece boundaries, and keys 30x larger at a few late prefix positions
    and late in every suffix long enough.  Elementwise against the oracle."""
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import make_workload, split_shared_prefix
    w = make_workload(3)
    log(f"[cascade] needles + late x30 outliers, full config 3, P={P}")
    B, D = w.block_size, w.head_dim
    kc = w.k_cache.copy()
    pref = w.block_tables[0, :512 // B]
    for j, pos in enumerate([0, 63, 64, 127, 128, 255, 256, 383, 384, 511]):
        s = (7 * j + 3) % w.num_seqs
        qv = w.q[s].astype(np.float32)  # [H, D]
        kc[pref[pos // B], pos % B] = (24.0 * qv / np.linalg.norm(qv, axis=1, keepdims=True)
                                       ).astype(np.float16)
    rng = np.random.default_rng(303)

    def boost(blk, off):
        kc[blk, off] = (kc[blk, off].astype(np.float32) * 30.0).astype(np.float16)
    for pos in rng.integers(400, 512, size=3):
        boost(pref[pos // B], pos % B)
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        lo = 512 + (L - 512) // 2
        if L - 1 > lo:  # never the new token's position L - 1
            for pos in rng.integers(lo, L - 1, size=2):
                boost(w.block_tables[s, pos // B], pos % B)
    w.k_cache = kc
    d = DeviceWorkload(w)
    d.reshape_and_cache()
    prefix, plen, suf_tables, suf_lens = split_shared_prefix(w, 512 // B)
    out = torch.full_like(d.q, float("nan"))
    pa.decode_cascade(out, d.q, d.k_cache, d.v_cache, to_dev(prefix), plen, to_dev(suf_tables),
                      to_dev(suf_lens), float(w.scale), partition_size=P)
    torch.cuda.synchronize()
    _, _, ref = oracle_after_write(orc, w)
    ea, er = assert_close(out.cpu().numpy(), ref, f"cascade needles/outliers P={P}")
    log(f"[cascade] needles/outliers P={P}: max abs err {ea:.3e}, max rel err {er:.3e}")


def test_cascade_repeated_calls_and_determinism(orc):
    """Calls on one workspace must not read the previous call's prefix
    pieces: three calls with different queries, each checked against the
    oracle, then the first queries again, bitwise equal to the first result."""
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import make_workload, split_shared_prefix
    w = make_workload(3)
    log(f"[cascade] repeated calls S={w.num_seqs} H={w.num_heads}")
    d = DeviceWorkload(w)
    d.reshape_and_cache()
    prefix, plen, suf_tables, suf_lens = split_shared_prefix(w, 32)
    kc, vc, _ = oracle_after_write(orc, w)
    ws = torch.empty(pa.decode_cascade_workspace_size(w.num_seqs, w.num_heads, w.head_dim,
                                                      w.block_size, plen, suf_tables.shape[1], 0),
                     dtype=torch.uint8, device="cuda")
    args = (d.k_cache, d.v_cache, to_dev(prefix), plen, to_dev(suf_tables), to_dev(suf_lens))
    rng = np.random.default_rng(77)
    qs = [w.q] + [rng.standard_normal(w.q.shape).astype(np.float16) for _ in range(2)]
    first = None
    for i, qh in enumerate(qs + [w.q]):
        out = torch.full_like(d.q, float("nan"))
        pa.decode_cascade(out, to_dev(qh), *args, float(w.scale), partition_size=0, workspace=ws)
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        if i < len(qs):
            ref = orc.decode(qh, kc, vc, w.block_tables, w.context_lens, float(w.scale))
            assert_close(got, ref, f"cascade call {i}")
        if first is None:
            first = got
    assert np.array_equal(got.view(np.uint16), first.view(np.uint16)), \
        "cascade not bitwise deterministic across calls"


@pytest.mark.parametrize("max_suffix", [600, 1100], ids=["exact_order", "bucketed_order"])
def test_cascade_suffix_order(orc, max_suffix):
    """The prefix pass orders the sequences for the suffix launch (longest
    suffix first).  300 sequences (more than one per thread of the ordering
    workgroup), ties, empty suffixes and the longest possible one: the
    result is the oracle's; the order written after the partials is a
    permutation whose lengths do not increase (exactly when the suffix tables
    cover fewer than 1024 tokens, by buckets of 2 tokens at 1100); and the
    batch with its sequences reversed on the host gives the same rows
    bitwise."""
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import make_random
    S, H, D, B, prefix_blocks = 300, 2, 128, 16, 4
    rng = np.random.default_rng(max_suffix)
    suffix = rng.integers(0, max_suffix + 1, S)
    suffix[:40] = rng.choice([0, 1, 17, 17, 256], 40)  # ties and empty suffixes
    suffix[57] = suffix[58] = max_suffix
    plen = prefix_blocks * B
    log(f"[cascade] suffix order S={S} max suffix {max_suffix}")
    w = make_random([plen + int(x) for x in suffix], H, D, B, seed=max_suffix, poison=True)
    w.block_tables[:, :prefix_blocks] = w.block_tables[0, :prefix_blocks]
    kc, vc = w.k_cache.copy(), w.v_cache.copy()
    ok = w.slot_mapping >= 0
    kc.reshape(-1, H, D)[w.slot_mapping[ok]] = np.float16(0.1)   # no new token here
    vc.reshape(-1, H, D)[w.slot_mapping[ok]] = np.float16(0.2)
    ref = orc.decode(w.q, kc, vc, w.block_tables, w.context_lens, float(w.scale))
    prefix = w.block_tables[0, :prefix_blocks].astype(np.int32)
    st = np.ascontiguousarray(w.block_tables[:, prefix_blocks:])
    max_len = st.shape[1] * B
    assert (max_len < 1024) == (max_suffix < 1024)
    sl = suffix.astype(np.int32)
    need = pa.decode_cascade_workspace_size(S, H, D, B, plen, st.shape[1], 0)
    dk, dv, dp = to_dev(kc), to_dev(vc), to_dev(prefix)

    def run(q, tables, lens):
        ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
        out = to_dev(np.full((S, H, D), np.nan, dtype=np.float16))
        pa.decode_cascade(out, to_dev(q), dk, dv, dp, plen, to_dev(tables), to_dev(lens),
                          float(w.scale), partition_size=0, workspace=ws)
        torch.cuda.synchronize()
        order = ws[need - (S * 8 + 255) // 256 * 256:].cpu().numpy()[:S * 8].view(np.int32)
        return out.cpu().numpy(), order[:S], order[S:]

    got, ids, lens = run(w.q, st, sl)
    assert_close(got, ref, "cascade, ordered suffixes")
    assert sorted(ids.tolist()) == list(range(S)), "the order is not a permutation"
    assert np.array_equal(lens, sl[ids]), "the order's lengths are not the sequences' lengths"
    width = max_len // 1024 + 1
    keys = (max_len - lens) // width
    assert np.all(np.diff(keys) >= 0), "suffix lengths increase along the order"
    if width == 1:
        assert np.all(np.diff(lens) <= 0)
    rev = np.arange(S)[::-1]
    got_rev, _, _ = run(w.q[rev], st[rev], sl[rev])
    assert np.array_equal(got_rev[rev].view(np.uint16), got.view(np.uint16)), \
        "a sequence's rows depend on the batch order"


def test_multi_query_bench_workload_sampled(orc):
    """The launch bench.py --op multi_query times (16 sequences of 2048
    positions, the last 512 new, 32 heads x 128, B = 16, the same seeded
    inputs): every row and head of sequences 0, 7 and 15 against the oracle's
    prefill of those sequences alone (their rows are independent of the
    others')."""
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import make_multi_query
    S, ctx, n = 16, 2048, 512
    log("[mq] bench workload 16 x 2048, last 512 new (sampled)")
    w, q, qs = make_multi_query([ctx] * S, [n] * S, 32, 128, 16, seed=155, poison=False)
    out = to_dev(np.full(q.shape, np.nan, dtype=np.float16))
    pa.multi_query(out, to_dev(q), to_dev(w.k_cache), to_dev(w.v_cache), to_dev(w.block_tables),
                   to_dev(w.context_lens), to_dev(qs), n, float(w.scale))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for s in (0, 7, 15):
        rows = slice(int(qs[s]), int(qs[s + 1]))
        ref = orc.prefill(q[rows], w.k_cache, w.v_cache, w.block_tables[s:s + 1],
                          w.context_lens[s:s + 1], np.array([0, n], dtype=np.int32), float(w.scale))
        ea, _ = assert_close(got[rows], ref, f"bench workload, sequence {s}")
        log(f"[mq] sequence {s}: max abs err {ea:.3e}")
