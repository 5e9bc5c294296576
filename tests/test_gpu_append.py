"""pa_decode_cascade_append: one decode step of a shared-prefix batch (the new
tokens written, then the cascade decode) in the launches of the decode alone.

Against the two-call step on a second upload of the same arrays
(pa_reshape_and_cache, then pa_decode_cascade):
  * output and both entire pools bitwise equal;
and against the oracle (reshape, then decode over the full tables):
  * pools bitwise equal, output within 2e-3 + 1e-2 |oracle|.
The slot each new token goes to holds NaN beforehand (poisoned workloads), so
a decode that ran before the write landed would show NaN.
"""
import numpy as np
import pytest

from gpu_util import DeviceWorkload, assert_close, log, oracle_after_write, to_dev

pytestmark = pytest.mark.gpu


def _pools(d):
    return (d.k_cache.cpu().numpy().view(np.uint16), d.v_cache.cpu().numpy().view(np.uint16))


def _both(w, prefix, plen, st, sl, P):
    """(output, pools) of the two-call step and of the appending call."""
    import torch
    import paged_kv_cache_155_amd as pa
    res = []
    for append in (False, True):
        d = DeviceWorkload(w)
        pt, stt, slt = to_dev(prefix), to_dev(st), to_dev(sl)
        if append:
            pa.decode_cascade_append(d.out, d.q, d.key, d.value, d.k_cache, d.v_cache,
                                     d.slot_mapping, pt, plen, stt, slt, float(w.scale),
                                     partition_size=P)
        else:
            d.reshape_and_cache()
            pa.decode_cascade(d.out, d.q, d.k_cache, d.v_cache, pt, plen, stt, slt,
                              float(w.scale), partition_size=P)
        torch.cuda.synchronize()
        res.append((d.out.cpu().numpy(), _pools(d)))
    return res


def _check(orc, w, prefix, plen, st, sl, P, what):
    (ref, (rk, rv)), (got, (gk, gv)) = _both(w, prefix, plen, st, sl, P)
    assert np.array_equal(got.view(np.uint16), ref.view(np.uint16)), f"{what}: output differs"
    assert np.array_equal(gk, rk) and np.array_equal(gv, rv), f"{what}: pools differ"
    kc, vc, oref = oracle_after_write(orc, w)
    assert np.array_equal(gk, kc.view(np.uint16)), f"{what}: K pool differs from the oracle's"
    assert np.array_equal(gv, vc.view(np.uint16)), f"{what}: V pool differs from the oracle's"
    ea, _ = assert_close(got, oref, what)
    log(f"[append] {what}: bitwise equal to the two-call step; max abs err {ea:.3e}")


@pytest.mark.parametrize("kw,P", [(dict(num_seqs=12, num_heads=2), 0),
                                  (dict(num_seqs=70, num_heads=3), 0),
                                  (dict(num_seqs=12, num_heads=2), 256),
                                  ({}, 0)],
                         ids=["small", "70seqs", "small_split", "full"])
def test_shared_prefix_workload(orc, kw, P):
    """The shared-prefix workload (32 shared blocks, private suffixes of 1..512
    tokens); 70 sequences span two 64-row tiles, P = 256 sends the suffixes
    through the reduce."""
    from paged_kv_cache_155_amd.workloads import make_workload, split_shared_prefix
    w = make_workload(3, **kw)
    prefix, plen, st, sl = split_shared_prefix(w, 32)
    log(f"[append] shared prefix S={w.num_seqs} H={w.num_heads} prefix {plen} P={P}")
    _check(orc, w, prefix, plen, st, sl, P, f"S={w.num_seqs} H={w.num_heads} P={P}")


def _prefixed(lens, prefix_blocks, H, D, B, seed, slots=None):
    """A make_random workload whose first prefix_blocks table entries are
    shared by every sequence (the new token always lands in the suffix)."""
    from paged_kv_cache_155_amd.workloads import make_random, split_shared_prefix
    w = make_random(lens, H, D, B, seed=seed, partition_size=0, poison=False)
    w.block_tables[:, :prefix_blocks] = w.block_tables[0, :prefix_blocks]
    if slots is not None:
        w.slot_mapping = np.asarray(slots, dtype=np.int64)
    return w, split_shared_prefix(w, prefix_blocks)


@pytest.mark.parametrize("D,B", [(64, 16), (128, 32)])
def test_shapes_and_skipped_slots(orc, D, B):
    """Head dims and block sizes; a suffix of one token; a negative and an
    out-of-range slot (written nowhere, read from the cache as it is)."""
    lens = [4 * B + 1, 4 * B + 7, 4 * B + 3 * B, 4 * B + 1, 4 * B + 2 * B + 5]
    w, _ = _prefixed(lens, 4, 3, D, B, seed=D + B)
    slots = w.slot_mapping.copy()
    slots[1] = -1
    slots[3] = w.num_blocks * B + 11
    w, (prefix, plen, st, sl) = _prefixed(lens, 4, 3, D, B, seed=D + B, slots=slots)
    log(f"[append] D={D} B={B} prefix {plen}, skipped slots")
    _check(orc, w, prefix, plen, st, sl, 0, f"D={D} B={B}")


def test_no_prefix_is_the_plain_step(orc):
    """prefix_len = 0: pa_reshape_and_cache then pa_decode."""
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import make_workload
    w = make_workload(1, num_seqs=8, num_heads=4)
    d = DeviceWorkload(w)
    empty = to_dev(np.zeros(1, dtype=np.int32))
    pa.decode_cascade_append(d.out, d.q, d.key, d.value, d.k_cache, d.v_cache, d.slot_mapping,
                             empty, 0, d.block_tables, d.context_lens, float(w.scale),
                             partition_size=512)
    torch.cuda.synchronize()
    kc, vc, oref = oracle_after_write(orc, w)
    gk, gv = _pools(d)
    assert np.array_equal(gk, kc.view(np.uint16)) and np.array_equal(gv, vc.view(np.uint16))
    assert_close(d.out.cpu().numpy(), oref, "no prefix")


def test_graph_capture_replays_match_eager(orc):
    """The appending step enqueues only kernels, so it can be captured in a
    HIP graph: captured once and replayed three times, with the new tokens'
    slots reset to NaN and the workspace filled with 0xFF before each replay
    (eager work and synchronisations in between); every replay writes the
    slots again and is bitwise equal to the eager call."""
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import make_workload, split_shared_prefix
    w = make_workload(3, num_seqs=70, num_heads=4)
    prefix, plen, st, sl = split_shared_prefix(w, 32)
    log(f"[append] graph capture S={w.num_seqs} H={w.num_heads} prefix {plen}")
    d = DeviceWorkload(w)
    pt, stt, slt = to_dev(prefix), to_dev(st), to_dev(sl)
    ws = torch.empty(pa.decode_cascade_workspace_size(w.num_seqs, w.num_heads, w.head_dim,
                                                      w.block_size, plen, st.shape[1], 0),
                     dtype=torch.uint8, device="cuda")
    H, D = w.num_heads, w.head_dim

    def step(out):
        pa.decode_cascade_append(out, d.q, d.key, d.value, d.k_cache, d.v_cache, d.slot_mapping,
                                 pt, plen, stt, slt, float(w.scale), partition_size=0,
                                 workspace=ws)

    def reset_slots():
        d.k_cache.view(-1, H, D)[d.slot_mapping] = float("nan")
        d.v_cache.view(-1, H, D)[d.slot_mapping] = float("nan")

    eager = torch.full_like(d.q, float("nan"))
    step(eager)
    torch.cuda.synchronize()
    kc, vc, ref = oracle_after_write(orc, w)
    assert_close(eager.cpu().numpy(), ref, "eager step before capture")
    pools = _pools(d)
    assert np.array_equal(pools[0], kc.view(np.uint16))
    out = torch.full_like(d.q, float("nan"))
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            step(out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for i in range(3):
        out.fill_(float("nan"))
        ws.fill_(0xFF)
        reset_slots()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy().view(np.uint16), eager.cpu().numpy().view(np.uint16)), \
            f"replay {i}: output differs from the eager call"
        got = _pools(d)
        assert np.array_equal(got[0], pools[0]) and np.array_equal(got[1], pools[1]), \
            f"replay {i}: pools differ from the eager call"


@pytest.mark.parametrize("kw,P", [(dict(num_seqs=70, num_heads=3), 0), ({}, 0),
                                  (dict(num_seqs=12, num_heads=2), 256)],
                         ids=["70seqs", "full", "small_split"])
def test_fp8_one_call_equals_two_calls(orc, kw, P):
    """pa_decode_cascade_append_fp8 against pa_reshape_and_cache_fp8 +
    pa_decode_cascade_fp8: the copy workgroups quantise with the cache
    write's rule, so output and both FP8 pools are bitwise equal; the pools
    also equal the oracle's quantised write, the output its FP8 decode."""
    import torch
    import paged_kv_cache_155_amd as pa
    from paged_kv_cache_155_amd.workloads import fp8_pools, make_workload, split_shared_prefix
    w = make_workload(3, **kw)
    f = fp8_pools(w)
    prefix, plen, st, sl = split_shared_prefix(w, 32)
    log(f"[append] fp8 S={w.num_seqs} H={w.num_heads} P={P}")
    res = []
    for one_call in (False, True):
        kc, vc, q = to_dev(f.k_cache), to_dev(f.v_cache), to_dev(w.q)
        key, val, sm = to_dev(w.key), to_dev(w.value), to_dev(w.slot_mapping)
        pt, stt, slt = to_dev(prefix), to_dev(st), to_dev(sl)
        out = torch.full_like(q, float("nan"))
        if one_call:
            pa.decode_cascade_append_fp8(out, q, key, val, kc, vc, sm, pt, plen, stt, slt,
                                         float(w.scale), f.k_scale, f.v_scale, partition_size=P)
        else:
            pa.reshape_and_cache_fp8(key, val, kc, vc, sm, f.k_scale, f.v_scale)
            pa.decode_cascade_fp8(out, q, kc, vc, pt, plen, stt, slt, float(w.scale), f.k_scale,
                                  f.v_scale, partition_size=P)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy(), kc.cpu().numpy(), vc.cpu().numpy()))
    (o2, k2, v2), (o1, k1, v1) = res
    assert np.array_equal(o1.view(np.uint16), o2.view(np.uint16)), "output differs"
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2), "FP8 pools differ"
    hk, hv = f.k_cache.copy(), f.v_cache.copy()
    orc.reshape_and_cache_fp8(w.key, w.value, hk, hv, w.slot_mapping, f.k_scale, f.v_scale)
    assert np.array_equal(k1, hk) and np.array_equal(v1, hv), "pools differ from the oracle's"
    ref = orc.decode_fp8(w.q, hk, hv, w.block_tables, w.context_lens, float(w.scale), f.k_scale,
                         f.v_scale)
    ea, _ = assert_close(o1, ref, "fp8 one call")
    log(f"[append] fp8 S={w.num_seqs} P={P}: bitwise equal to the two-call step; max abs err {ea:.3e}")
