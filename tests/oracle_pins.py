"""Pins of the CPU oracle against facts that do not come from the oracle.

Each pin takes an `oracle.Oracle` and raises AssertionError on a mismatch.
They are collected by test_oracle.py for the default oracle and run by
test_oracle_mutants.py against deliberately broken copies of the oracle (each
broken copy must fail at least one pin).  Running this file as a script with
`--lib PATH` checks the library at PATH and exits 1 if any pin fails.

What pins what:
  half decode      all 65,536 binary16 patterns vs numpy's float16 -> float64
  gather           the block-table worked example ("深入解析LLM推理引擎：从
                   PagedAttention到调度优化" §3.2), a golden fixture
  attention        torch's scaled_dot_product_attention (CPU, float64) on the
                   contiguous layout; pure-Python brute force (math.exp,
                   math.fsum) on tiny inputs; closed forms (equal keys or a
                   zero query give the mean of V, one token gives v0, two
                   tokens give sigmoid weights, a dominant needle key selects
                   its value)
  paging           bitwise invariance under relabelling of physical blocks
  reshape_and_cache  numpy scatter by slot on sentinel pools, special bit
                   patterns, out-of-range slots, the worked example's slot
  copy / swap      numpy block assignment on random bit patterns; a
                   copy-on-write sequence ("vLLM基础架构" §2.3) seen through
                   the gather; out-of-range pairs
  multi-query      one query per sequence reduces bitwise to the decode;
                   torch SDPA with the causal mask of the last n positions on
                   the contiguous layout (n = ctx is the ordinary causal
                   mask); pure-Python brute force on tiny inputs
  FP8 (OCP E4M3)   all 256 codes vs torch.float8_e4m3fn; the encoder vs
                   torch's float -> float8_e4m3fn cast wherever torch does not
                   overflow (all fp16 values, ties, random floats), closed forms
                   for saturation and NaN; the scaled quantiser vs torch doing
                   the float32 multiply and cast; FP8 decode vs torch SDPA on
                   the dequantised contiguous K/V
"""
import json
import math
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden")


def _f16(a):
    return np.asarray(a, dtype=np.float16)


def _rand_case(rng, S, H, D, B, lens, extra_blocks=3):
    """Random pool with a random scattered table (numpy only)."""
    MB = max(1, max(-(-int(L) // B) for L in lens))
    need = sum(-(-int(L) // B) for L in lens)
    NB = need + extra_blocks
    perm = rng.permutation(NB)
    bt = np.zeros((S, MB), dtype=np.int32)
    c = 0
    for s, L in enumerate(lens):
        n = -(-int(L) // B)
        bt[s, :n] = perm[c:c + n]
        bt[s, n:] = perm[-1]
        c += n
    q = _f16(rng.standard_normal((S, H, D)))
    kc = _f16(rng.standard_normal((NB, B, H, D)))
    vc = _f16(rng.standard_normal((NB, B, H, D)))
    return q, kc, vc, bt, np.asarray(lens, dtype=np.int32)


# --------------------------------------------------------------------------
# binary16 decoding
# --------------------------------------------------------------------------
def pin_half_decode_exhaustive(orc):
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = orc.half_to_double(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan), "NaN classification differs"
    assert np.array_equal(got[~nan], ref[~nan]), "binary16 values differ"
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])), "signed zero differs"


# --------------------------------------------------------------------------
# gather: the pages' worked example
# --------------------------------------------------------------------------
def pin_gather_worked_example(orc):
    ex = json.load(open(os.path.join(GOLDEN, "block_table_worked_example.json")))
    B = ex["block_size"]
    table = ex["block_table"]
    NB = max(table) + 1
    H, D = 2, 2
    # slot (b, o) of head h holds the vector (b + 100 h, o): its provenance
    kc = np.zeros((NB, B, H, D), dtype=np.float16)
    for b in range(NB):
        for o in range(B):
            for h in range(H):
                kc[b, o, h] = (b + 100 * h, o)
    vc = -kc
    L = ex["position_ranges"][-1]["last"] + 1
    bt = np.array([table], dtype=np.int32)
    cl = np.array([L], dtype=np.int32)
    for h in range(H):
        K, V = orc.gather(kc, vc, bt, cl, 0, h)
        assert K.shape == (L, D)
        for r in ex["position_ranges"]:
            for i in range(r["first"], r["last"] + 1):
                assert K[i, 0] == r["physical_block"] + 100 * h, (i, K[i])
                assert K[i, 1] == i % B, (i, K[i])
                assert V[i, 0] == -(r["physical_block"] + 100 * h)
        used = {int(k) for k in K[:, 0] - 100 * h}
        assert ex["unused_physical_block"] not in used


# --------------------------------------------------------------------------
# attention vs an independent library on the contiguous layout
# --------------------------------------------------------------------------
def pin_contiguous_sdpa(orc):
    import torch
    rng = np.random.default_rng(1)
    for (S, H, D, B) in [(3, 2, 64, 16), (2, 3, 128, 32), (2, 1, 8, 4)]:
        lens = rng.integers(1, 3 * B + 2, size=S)
        MB = int(-(-lens.max() // B))
        # identity tables: sequence s owns blocks s*MB .. s*MB+MB-1 in order,
        # so its slice of the pool is its contiguous K / V
        bt = (np.arange(S)[:, None] * MB + np.arange(MB)[None, :]).astype(np.int32)
        NB = S * MB
        q = _f16(rng.standard_normal((S, H, D)))
        kc = _f16(rng.standard_normal((NB, B, H, D)))
        vc = _f16(rng.standard_normal((NB, B, H, D)))
        scale = float(np.float32(1 / math.sqrt(D)))
        got = orc.decode(q, kc, vc, bt, lens.astype(np.int32), scale)
        for s in range(S):
            L = int(lens[s])
            Kc = torch.from_numpy(kc[s * MB:(s + 1) * MB].reshape(MB * B, H, D)[:L].astype(np.float64))
            Vc = torch.from_numpy(vc[s * MB:(s + 1) * MB].reshape(MB * B, H, D)[:L].astype(np.float64))
            Q = torch.from_numpy(q[s].astype(np.float64))
            for h in range(H):
                ref = torch.nn.functional.scaled_dot_product_attention(
                    Q[h].reshape(1, 1, D), Kc[:, h].reshape(1, L, D).contiguous(),
                    Vc[:, h].reshape(1, L, D).contiguous(), scale=scale).reshape(D).numpy()
                assert np.allclose(got[s, h], ref, rtol=1e-11, atol=1e-13), (S, H, D, B, s, h)


def pin_block_permutation_invariance(orc):
    rng = np.random.default_rng(2)
    S, H, D, B = 3, 2, 64, 16
    q, kc, vc, bt, cl = _rand_case(rng, S, H, D, B, [5, 37, 64])
    base = orc.decode(q, kc, vc, bt, cl, 0.125)
    for _ in range(3):
        pi = rng.permutation(kc.shape[0])
        kc2 = np.empty_like(kc)
        vc2 = np.empty_like(vc)
        kc2[pi] = kc
        vc2[pi] = vc
        got = orc.decode(q, kc2, vc2, pi[bt].astype(np.int32), cl, 0.125)
        assert np.array_equal(got.view(np.uint64), base.view(np.uint64))


# --------------------------------------------------------------------------
# brute force in pure Python on tiny inputs
# --------------------------------------------------------------------------
def _brute(q, kc, vc, bt, cl, scale):
    S, H, D = q.shape
    B = kc.shape[1]
    out = np.zeros((S, H, D))
    for s in range(S):
        L = int(cl[s])
        for h in range(H):
            rows = []
            for i in range(L):
                blk = int(bt[s][i // B])
                rows.append((kc[blk][i % B][h].astype(float).tolist(),
                             vc[blk][i % B][h].astype(float).tolist()))
            qq = q[s][h].astype(float).tolist()
            logits = [scale * math.fsum(a * b for a, b in zip(qq, k)) for k, _ in rows]
            if not logits:
                continue
            mx = max(logits)
            e = [math.exp(x - mx) for x in logits]
            z = math.fsum(e)
            for d in range(D):
                out[s, h, d] = math.fsum(w * v[d] for w, (_, v) in zip(e, rows)) / z
    return out


def pin_brute_force_tiny(orc):
    rng = np.random.default_rng(3)
    for B in (2, 4, 16):
        for D in (8, 64):
            lens = list(range(1, 3 * B + 2))
            # three sequences per call, all residues of ctx mod B across calls
            for i in range(0, len(lens), 3):
                chunk = lens[i:i + 3]
                q, kc, vc, bt, cl = _rand_case(rng, len(chunk), 2, D, B, chunk)
                scale = float(np.float32(1 / math.sqrt(D)))
                got = orc.decode(q, kc, vc, bt, cl, scale)
                ref = _brute(q, kc, vc, bt, cl, scale)
                assert np.allclose(got, ref, rtol=1e-11, atol=1e-13), (B, D, chunk)


# --------------------------------------------------------------------------
# closed forms
# --------------------------------------------------------------------------
def pin_closed_forms(orc):
    rng = np.random.default_rng(4)
    S, H, D, B = 2, 2, 64, 16
    q, kc, vc, bt, cl = _rand_case(rng, S, H, D, B, [40, 19])
    # (a) every key of head 0 equal -> uniform weights -> mean of V
    kc_eq = kc.copy()
    kc_eq[:, :, 0, :] = kc[0, 0, 0, :]
    got = orc.decode(q, kc_eq, vc, bt, cl, 0.125)
    for s in range(S):
        _, V = orc.gather(kc, vc, bt, cl, s, 0)
        assert np.allclose(got[s, 0], V.mean(axis=0), rtol=1e-12, atol=1e-14)
    # (b) zero query -> mean of V for every head
    got = orc.decode(np.zeros_like(q), kc, vc, bt, cl, 0.125)
    for s in range(S):
        for h in range(H):
            _, V = orc.gather(kc, vc, bt, cl, s, h)
            assert np.allclose(got[s, h], V.mean(axis=0), rtol=1e-12, atol=1e-14)
    # (c) one token -> exactly its value row
    cl1 = np.ones(S, dtype=np.int32)
    got = orc.decode(q, kc, vc, bt, cl1, 0.125)
    for s in range(S):
        for h in range(H):
            assert np.array_equal(got[s, h], vc[bt[s, 0], 0, h].astype(np.float64))
    # (d) two tokens with logits a, b -> weights sigmoid(a - b), sigmoid(b - a)
    q2 = np.zeros((1, 1, 8), dtype=np.float16)
    q2[0, 0, 0] = 1.0
    kc2 = np.zeros((2, 2, 1, 8), dtype=np.float16)
    vc2 = _f16(rng.standard_normal((2, 2, 1, 8)))
    a, b = 1.5, -0.75
    kc2[1, 0, 0, 0] = a
    kc2[1, 1, 0, 0] = b
    bt2 = np.array([[1]], dtype=np.int32)
    for scale in (1.0, 0.5):
        got = orc.decode(q2, kc2, vc2, bt2, np.array([2], dtype=np.int32), scale)
        w0 = 1.0 / (1.0 + math.exp(-(a - b) * scale))
        ref = w0 * vc2[1, 0, 0].astype(np.float64) + (1 - w0) * vc2[1, 1, 0].astype(np.float64)
        assert np.allclose(got[0, 0], ref, rtol=1e-12, atol=1e-14)
    # (e) context length 0 -> zeros
    got = orc.decode(q, kc, vc, bt, np.zeros(S, dtype=np.int32), 0.125)
    assert np.array_equal(got, np.zeros_like(got))


def pin_needles(orc):
    """A key parallel to the query with a huge logit takes all the weight, at
    every block boundary, partition boundary and the last position."""
    rng = np.random.default_rng(5)
    D, B, H = 64, 16, 1
    L = 1100
    q, kc, vc, bt, cl = _rand_case(rng, 1, H, D, B, [L])
    qn = q[0, 0].astype(np.float64)
    for pos in (0, 15, 16, 17, 511, 512, 1023, 1024, L - 1):
        kcn = kc.copy()
        blk, off = bt[0, pos // B], pos % B
        # logit of the needle ~ 1000 (exp overflows without the max shift)
        kcn[blk, off, 0] = _f16(qn / np.dot(qn, qn) * 1000.0 / 0.125 * 1.0)
        got = orc.decode(q, kcn, vc, bt, cl, 0.125)
        assert np.all(np.isfinite(got)), pos
        assert np.allclose(got[0, 0], vc[blk, off, 0].astype(np.float64), rtol=1e-9, atol=1e-9), pos


# --------------------------------------------------------------------------
# reshape_and_cache
# --------------------------------------------------------------------------
_SPECIAL = np.array([0x0000, 0x8000, 0x0001, 0x83FF, 0x7C00, 0xFC00, 0x7C01, 0x7E00,
                     0xFE01, 0xFFFF, 0x3C00, 0x7BFF], dtype=np.uint16)


def pin_reshape_scatter(orc):
    rng = np.random.default_rng(6)
    for (NB, B, H, D, T) in [(9, 16, 3, 64, 7), (5, 32, 2, 128, 5), (4, 4, 1, 8, 6)]:
        sentinel = np.uint16(0x5A5A)
        kc = np.full((NB, B, H, D), sentinel, dtype=np.uint16)
        vc = np.full((NB, B, H, D), sentinel + 1, dtype=np.uint16)
        key = rng.integers(0, 1 << 16, size=(T, H, D), dtype=np.uint32).astype(np.uint16)
        key.reshape(-1)[:len(_SPECIAL)] = _SPECIAL
        val = rng.integers(0, 1 << 16, size=(T, H, D), dtype=np.uint32).astype(np.uint16)
        slots = rng.choice(NB * B, size=T, replace=False).astype(np.int64)
        slots[0] = -1            # padding token: no write
        slots[1] = NB * B        # one past the pool: no write
        orc.reshape_and_cache(key, val, kc, vc, slots)
        ref_k = np.full((NB * B, H, D), sentinel, dtype=np.uint16)
        ref_v = np.full((NB * B, H, D), sentinel + 1, dtype=np.uint16)
        ok = (slots >= 0) & (slots < NB * B)
        ref_k[slots[ok]] = key[ok]
        ref_v[slots[ok]] = val[ok]
        assert np.array_equal(kc.reshape(NB * B, H, D), ref_k)
        assert np.array_equal(vc.reshape(NB * B, H, D), ref_v)


def pin_reshape_worked_example(orc):
    """Appending logical position 5 with block size 4 and table [0, 1, 3]
    writes slot 1*4 + 1, and the gather then returns the new key there."""
    ex = json.load(open(os.path.join(GOLDEN, "block_table_worked_example.json")))
    B, table = ex["block_size"], ex["block_table"]
    NB = max(table) + 1
    kc = np.zeros((NB, B, 1, 2), dtype=np.float16)
    vc = np.zeros_like(kc)
    pos = 5
    phys = [r["physical_block"] for r in ex["position_ranges"] if r["first"] <= pos <= r["last"]][0]
    slot = phys * B + pos % B
    key = np.array([[[7.0, 8.0]]], dtype=np.float16)
    orc.reshape_and_cache(key, -key, kc, vc, np.array([slot], dtype=np.int64))
    K, V = orc.gather(kc, vc, np.array([table], dtype=np.int32), np.array([pos + 1], dtype=np.int32), 0, 0)
    assert np.array_equal(K[pos], [7.0, 8.0]) and np.array_equal(V[pos], [-7.0, -8.0])
    assert not K[:pos].any()


def _rand_bits(rng, shape):
    a = rng.integers(0, 1 << 16, size=shape, dtype=np.uint32).astype(np.uint16)
    a.reshape(-1)[:len(_SPECIAL)] = _SPECIAL
    return a


def pin_copy_blocks(orc):
    rng = np.random.default_rng(8)
    NB, B, H, D = 12, 16, 3, 64
    kc0 = _rand_bits(rng, (NB, B, H, D))
    vc0 = _rand_bits(rng, (NB, B, H, D))
    perm = rng.permutation(NB)
    mapping = np.stack([perm[:4], perm[4:8]], axis=1).astype(np.int64)  # 4 src -> 4 fresh dst
    bad = np.array([[-1, perm[8]], [perm[0], NB]], dtype=np.int64)       # skipped
    kc, vc = kc0.copy(), vc0.copy()
    orc.copy_blocks(kc, vc, np.concatenate([mapping, bad]))
    rk, rv = kc0.copy(), vc0.copy()
    rk[mapping[:, 1]] = kc0[mapping[:, 0]]
    rv[mapping[:, 1]] = vc0[mapping[:, 0]]
    assert np.array_equal(kc, rk) and np.array_equal(vc, rv)


def pin_copy_on_write(orc):
    """Two sequences share block X; the second must write into it, so X is
    copied to a free block Y, its table points at Y, and the write lands in
    Y: the first sequence still reads the old data, the second the new."""
    B, H, D = 4, 1, 2
    NB = 4
    kc = np.zeros((NB, B, H, D), dtype=np.float16)
    for b in range(NB):
        for o in range(B):
            kc[b, o, 0] = (b, o)
    vc = -kc
    X, Y = 2, 3
    tables = np.array([[0, X], [1, X]], dtype=np.int32)
    orc.copy_blocks(kc, vc, [[X, Y]])
    tables[1, 1] = Y
    pos = 6                       # logical block 1, offset 2
    slot = int(tables[1, pos // B]) * B + pos % B
    orc.reshape_and_cache(np.array([[[50.0, 60.0]]], np.float16),
                          np.array([[[-50.0, -60.0]]], np.float16), kc, vc,
                          np.array([slot], dtype=np.int64))
    lens = np.array([8, 8], dtype=np.int32)
    K0, _ = orc.gather(kc, vc, tables, lens, 0, 0)
    K1, V1 = orc.gather(kc, vc, tables, lens, 1, 0)
    assert np.array_equal(K0[4:8], [[X, 0], [X, 1], [X, 2], [X, 3]])
    assert np.array_equal(K1[4:8], [[X, 0], [X, 1], [50, 60], [X, 3]])
    assert np.array_equal(V1[pos], [-50, -60])


def pin_swap_blocks(orc):
    rng = np.random.default_rng(9)
    shape = (3, 16, 2, 128)
    gpu = _rand_bits(rng, (10,) + shape[1:])
    host = np.zeros((6,) + shape[1:], dtype=np.uint16)
    out_map = np.array([[7, 0], [2, 5], [9, 3]], dtype=np.int64)
    orc.swap_blocks(gpu, host, out_map)
    ref = np.zeros_like(host)
    ref[out_map[:, 1]] = gpu[out_map[:, 0]]
    assert np.array_equal(host, ref)
    back = np.zeros_like(gpu)
    in_map = out_map[:, ::-1].copy()
    in_map[:, 1] = [1, 4, 8]
    orc.swap_blocks(host, back, in_map)
    assert np.array_equal(back[[1, 4, 8]], gpu[[7, 2, 9]])
    try:
        orc.swap_blocks(gpu, host, [[0, 6]])
    except ValueError:
        pass
    else:
        raise AssertionError("out-of-range swap accepted")


def _torch_e4m3_codes(y_f32):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(y_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_decode_exhaustive(orc):
    import torch
    codes = np.arange(256, dtype=np.uint8)
    got = orc.e4m3_to_double(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    # the format's landmarks
    assert got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6 and got[0x38] == 1.0
    assert got[0x7E] == 448.0 and np.isnan(got[0x7F]) and got[0xFE] == -448.0


def pin_e4m3_encode(orc):
    rng = np.random.default_rng(10)
    f16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16)
    ys = [f16.astype(np.float32)[np.isfinite(f16)]]
    # exact midpoints between neighbouring codes (ties) and their neighbours
    vals = orc.e4m3_to_double(np.arange(0x7F, dtype=np.uint8))
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)
    ys += [mids, -mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(1e9))]
    ys += [rng.standard_normal(20000).astype(np.float32) * np.float32(50.0),
           (rng.random(20000) * 2.0 ** -8).astype(np.float32)]
    y = np.concatenate(ys).astype(np.float32)
    got = orc.float_to_e4m3(y)
    small = np.abs(y) < 464.0   # torch's cast is defined (no NaN) only below 464
    assert np.array_equal(got[small], _torch_e4m3_codes(y[small]))
    big = ~small
    assert np.all(got[big] == np.where(np.signbit(y[big]), 0xFE, 0x7E))
    special = np.array([np.inf, -np.inf, np.nan, -np.nan, 1e30, -1e-30, 0.0, -0.0], np.float32)
    assert orc.float_to_e4m3(special).tolist() == [0x7E, 0xFE, 0x7F, 0xFF, 0x7E, 0x80, 0x00, 0x80]


def pin_quantize_scale(orc):
    import torch
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(50000) * 3).astype(np.float16)
    for scale in (1.0, 0.02, 1 / 64.0, 3.7):
        got = orc.quantize_e4m3(x, scale)
        inv = torch.tensor(1.0 / scale, dtype=torch.float64).float()
        y = (torch.from_numpy(x.astype(np.float32)) * inv).numpy()
        ref = np.where(np.abs(y) >= 464.0, np.where(np.signbit(y), 0xFE, 0x7E),
                       _torch_e4m3_codes(np.clip(y, -463.0, 463.0))).astype(np.uint8)
        assert np.array_equal(got, ref), scale


def pin_fp8_decode_sdpa(orc):
    import torch
    rng = np.random.default_rng(12)
    S, H, D, B = 3, 2, 128, 16
    lens = np.array([1, 37, 80])
    MB = 5
    bt = (np.arange(S)[:, None] * MB + np.arange(MB)[None, :]).astype(np.int32)
    NB = S * MB
    q = _f16(rng.standard_normal((S, H, D)))
    kc = rng.integers(0, 256, size=(NB, B, H, D), dtype=np.uint32).astype(np.uint8)
    vc = rng.integers(0, 256, size=(NB, B, H, D), dtype=np.uint32).astype(np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x3C   # no NaN codes in live data
    vc[(vc & 0x7F) == 0x7F] = 0x3C
    ks, vs = 0.01, 0.05
    got = orc.decode_fp8(q, kc, vc, bt, lens.astype(np.int32), 0.0884, ks, vs)
    Kd = torch.from_numpy(kc).view(torch.float8_e4m3fn).double() * float(np.float32(ks))
    Vd = torch.from_numpy(vc).view(torch.float8_e4m3fn).double() * float(np.float32(vs))
    for s in range(S):
        L = int(lens[s])
        Kc = Kd[s * MB:(s + 1) * MB].reshape(MB * B, H, D)[:L]
        Vc = Vd[s * MB:(s + 1) * MB].reshape(MB * B, H, D)[:L]
        for h in range(H):
            ref = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(q[s, h].astype(np.float64)).reshape(1, 1, D),
                Kc[:, h].reshape(1, L, D).contiguous(), Vc[:, h].reshape(1, L, D).contiguous(),
                scale=0.0884).reshape(D).numpy()
            assert np.allclose(got[s, h], ref, rtol=1e-11, atol=1e-13), (s, h)


def pin_fp8_reshape(orc):
    rng = np.random.default_rng(13)
    NB, B, H, D, T = 6, 16, 2, 64, 5
    kc = np.full((NB, B, H, D), 0xA5, dtype=np.uint8)
    vc = np.full((NB, B, H, D), 0x5A, dtype=np.uint8)
    key = _f16(rng.standard_normal((T, H, D)) * 4)
    val = _f16(rng.standard_normal((T, H, D)) * 4)
    slots = rng.choice(NB * B, size=T, replace=False).astype(np.int64)
    slots[0] = -1          # padding token
    slots[1] = NB * B      # one past the pool
    orc.reshape_and_cache_fp8(key, val, kc, vc, slots, 0.05, 0.02)
    rk = np.full((NB * B, H, D), 0xA5, dtype=np.uint8)
    rv = np.full((NB * B, H, D), 0x5A, dtype=np.uint8)
    rk[slots[2:]] = orc.quantize_e4m3(key[2:], 0.05)
    rv[slots[2:]] = orc.quantize_e4m3(val[2:], 0.02)
    assert np.array_equal(kc.reshape(NB * B, H, D), rk) and np.array_equal(vc.reshape(NB * B, H, D), rv)


def _prefill_case(rng, lens, nq, H, D, B, identity=False):
    S = len(lens)
    MB = max(1, max(-(-int(L) // B) for L in lens))
    if identity:
        bt = (np.arange(S)[:, None] * MB + np.arange(MB)[None, :]).astype(np.int32)
        NB = S * MB
    else:
        NB = sum(-(-int(L) // B) for L in lens) + 2
        perm = rng.permutation(NB)
        bt = np.full((S, MB), perm[-1], dtype=np.int32)
        c = 0
        for s_, L in enumerate(lens):
            n = -(-int(L) // B)
            bt[s_, :n] = perm[c:c + n]
            c += n
    qs = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    q = _f16(rng.standard_normal((int(qs[-1]), H, D)))
    kc = _f16(rng.standard_normal((NB, B, H, D)))
    vc = _f16(rng.standard_normal((NB, B, H, D)))
    return q, kc, vc, bt, np.asarray(lens, np.int32), qs, MB


def pin_prefill_single_query_is_decode(orc):
    rng = np.random.default_rng(14)
    q, kc, vc, bt, cl, qs, _ = _prefill_case(rng, [1, 30, 77, 16], [1, 1, 1, 1], 2, 64, 16)
    a = orc.prefill(q, kc, vc, bt, cl, qs, 0.125)
    b = orc.decode(q, kc, vc, bt, cl, 0.125)
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


def pin_prefill_sdpa_causal(orc):
    import torch
    rng = np.random.default_rng(15)
    lens, nq = [37, 64, 5, 50], [37, 9, 1, 16]   # first: a whole prompt; others: chunks
    H, D, B = 2, 64, 16
    q, kc, vc, bt, cl, qs, MB = _prefill_case(rng, lens, nq, H, D, B, identity=True)
    got = orc.prefill(q, kc, vc, bt, cl, qs, 0.125)
    for s in range(len(lens)):
        L, n = lens[s], nq[s]
        Kc = torch.from_numpy(kc[s * MB:(s + 1) * MB].reshape(MB * B, H, D)[:L].astype(np.float64))
        Vc = torch.from_numpy(vc[s * MB:(s + 1) * MB].reshape(MB * B, H, D)[:L].astype(np.float64))
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]].astype(np.float64))
        allowed = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
        for h in range(H):
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[:, h].reshape(1, n, D).contiguous(), Kc[:, h].reshape(1, L, D).contiguous(),
                Vc[:, h].reshape(1, L, D).contiguous(), attn_mask=allowed.reshape(1, n, L),
                scale=0.125).reshape(n, D).numpy()
            assert np.allclose(got[qs[s]:qs[s + 1], h], ref, rtol=1e-11, atol=1e-13), (s, h)
        if n == L:
            causal = torch.nn.functional.scaled_dot_product_attention(
                Q[:, 0].reshape(1, n, D).contiguous(), Kc[:, 0].reshape(1, L, D).contiguous(),
                Vc[:, 0].reshape(1, L, D).contiguous(), is_causal=True, scale=0.125).reshape(n, D)
            assert np.allclose(got[qs[s]:qs[s + 1], 0], causal.numpy(), rtol=1e-11, atol=1e-13)


def pin_prefill_brute_force(orc):
    rng = np.random.default_rng(16)
    for B in (2, 4):
        lens, nq = [3, 9, 6], [3, 4, 1]
        q, kc, vc, bt, cl, qs, _ = _prefill_case(rng, lens, nq, 1, 8, B)
        got = orc.prefill(q, kc, vc, bt, cl, qs, 0.5)
        for s in range(3):
            L, n = lens[s], nq[s]
            for i in range(n):
                p = L - n + i
                rows = [(kc[bt[s][t // B]][t % B][0].astype(float).tolist(),
                         vc[bt[s][t // B]][t % B][0].astype(float).tolist()) for t in range(p + 1)]
                qq = q[qs[s] + i][0].astype(float).tolist()
                lg = [0.5 * math.fsum(a * b for a, b in zip(qq, k)) for k, _ in rows]
                mx = max(lg)
                e = [math.exp(x - mx) for x in lg]
                z = math.fsum(e)
                ref = [math.fsum(w * v[d] for w, (_, v) in zip(e, rows)) / z for d in range(8)]
                assert np.allclose(got[qs[s] + i, 0], ref, rtol=1e-11, atol=1e-13), (B, s, i)


def _fp8_codes(rng, shape):
    c = rng.integers(0, 256, size=shape, dtype=np.uint32).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x3C   # no NaN codes in live data
    return c


def pin_prefill_fp8_sdpa_causal(orc):
    """FP8 prefill against torch's own E4M3 decoding and causal SDPA in fp64,
    through a scattered table."""
    import torch
    rng = np.random.default_rng(17)
    lens, nq = [40, 17, 64], [40, 5, 1]
    H, D, B = 2, 64, 16
    q, _, _, bt, cl, qs, MB = _prefill_case(rng, lens, nq, H, D, B)
    NB = int(bt.max()) + 1
    kc, vc = _fp8_codes(rng, (NB, B, H, D)), _fp8_codes(rng, (NB, B, H, D))
    ks, vs = 0.02, 0.125
    got = orc.prefill_fp8(q, kc, vc, bt, cl, qs, 0.125, ks, vs)
    Kd = torch.from_numpy(kc).view(torch.float8_e4m3fn).double() * float(np.float32(ks))
    Vd = torch.from_numpy(vc).view(torch.float8_e4m3fn).double() * float(np.float32(vs))
    for s in range(len(lens)):
        L, n = lens[s], nq[s]
        idx = [int(bt[s][t // B]) * B + t % B for t in range(L)]
        Kc = Kd.reshape(NB * B, H, D)[idx]
        Vc = Vd.reshape(NB * B, H, D)[idx]
        Q = torch.from_numpy(q[qs[s]:qs[s + 1]].astype(np.float64))
        allowed = torch.arange(L)[None, :] <= (L - n + torch.arange(n))[:, None]
        for h in range(H):
            ref = torch.nn.functional.scaled_dot_product_attention(
                Q[:, h].reshape(1, n, D).contiguous(), Kc[:, h].reshape(1, L, D).contiguous(),
                Vc[:, h].reshape(1, L, D).contiguous(), attn_mask=allowed.reshape(1, n, L),
                scale=0.125).reshape(n, D).numpy()
            assert np.allclose(got[qs[s]:qs[s + 1], h], ref, rtol=1e-11, atol=1e-13), (s, h)


def pin_prefill_fp8_single_query_is_decode(orc):
    rng = np.random.default_rng(18)
    q, _, _, bt, cl, qs, _ = _prefill_case(rng, [1, 30, 77, 16], [1, 1, 1, 1], 2, 64, 16)
    NB = int(bt.max()) + 1
    kc, vc = _fp8_codes(rng, (NB, 16, 2, 64)), _fp8_codes(rng, (NB, 16, 2, 64))
    a = orc.prefill_fp8(q, kc, vc, bt, cl, qs, 0.125, 0.5, 0.03)
    b = orc.decode_fp8(q, kc, vc, bt, cl, 0.125, 0.5, 0.03)
    assert np.array_equal(a.view(np.uint64), b.view(np.uint64))


PINS = [pin_half_decode_exhaustive, pin_gather_worked_example, pin_contiguous_sdpa,
        pin_block_permutation_invariance, pin_brute_force_tiny, pin_closed_forms, pin_needles,
        pin_reshape_scatter, pin_reshape_worked_example, pin_copy_blocks, pin_copy_on_write,
        pin_swap_blocks, pin_e4m3_decode_exhaustive, pin_e4m3_encode, pin_quantize_scale,
        pin_fp8_decode_sdpa, pin_fp8_reshape, pin_prefill_single_query_is_decode,
        pin_prefill_sdpa_causal, pin_prefill_brute_force, pin_prefill_fp8_sdpa_causal,
        pin_prefill_fp8_single_query_is_decode]


def main(argv):
    sys.path.insert(0, os.path.dirname(HERE))
    import oracle
    lib = argv[argv.index("--lib") + 1] if "--lib" in argv else None
    orc = oracle.Oracle(lib)
    failed = []
    for pin in PINS:
        try:
            pin(orc)
        except Exception as e:  # noqa: BLE001 - any failure is a caught mistake
            failed.append(f"{pin.__name__}: {type(e).__name__}: {str(e)[:120]}")
            if "--fail-fast" in argv:
                break
    for f in failed:
        print("FAIL", f)
    print(f"{len(PINS) - len(failed)}/{len(PINS)} pins passed")
    return 1 if failed else 0


if __name__ == "__main__":
    sys.exit(main(sys.argv))
