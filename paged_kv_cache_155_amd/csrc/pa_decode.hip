// Paged-attention decode kernels for gfx950 (MI355X): fp16 or FP8 (OCP E4M3)
// KV cache, fp16 queries, fp32 math.
//
// Sources (web pages), cited by title and section:
//   [10x]  "vLLM推理加速深度解读：PagedAttention如何提升10x吞吐量"
//          §2.1 attention equation; §2.3 paged attention and the gather
//          K_paged[i] = K_physical[BlockTable[i / B]][i mod B];
//          §4.2 kernel strategy (walk the context block by block, keep the
//          block table close, one group of lanes per query head) and the
//          cache layout [num_blocks, block_size, num_heads, head_size];
//          §3.3 FP8 quantisation (format not given; OCP E4M3 with one scale
//          per cache is our reading)
//   [eng]  "深入解析LLM推理引擎：从PagedAttention到调度优化" §3.3 (the
//          gather follows block_table up to the current position)
//
// Design on CDNA4 (decode with one query per head is a batched GEMV: every
// K/V byte is used once, so the bound is HBM bandwidth and MFMA has nothing
// to do):
//   * one workgroup (4 waves) per (sequence, head, context partition).  The
//     logical unit order is sequence fastest, then partition, then head, and
//     the hardware workgroup id is remapped so that each of the 8 XCDs (which
//     receive workgroups round-robin) gets a contiguous range of that order:
//     an XCD works through whole heads, and the long and short partitions of
//     a ragged batch are spread evenly over time.  After a shared-prefix pass
//     the sequences are taken in the order that pass wrote, longest suffix
//     first, so the launch ends on its shortest units;
//   * K/V are streamed with nontemporal loads (read once, so they should not
//     displace other lines in the caches);
//   * every lane loads 16 bytes of a token's row of one head (8 fp16 or 16
//     FP8 values).  For fp16 and head_dim 128 that is 16 lanes per token and
//     4 tokens per global_load_dwordx4; FP8 halves the lanes per token.  A
//     wave walks tiles of 8 loads (32 tokens for fp16 / 128, 64 for FP8 /
//     128) and issues all 8 K and 8 V loads before any arithmetic;
//   * block ids: each wave reads up to 64 table entries with one vector load
//     and pulls the one a load needs with v_readlane (a scalar), so the
//     K/V address of a whole load is scalar base + lane offset;
//   * q.k with v_dot2_f32_f16 (fp16 products, fp32 sum; FP8 codes are first
//     widened exactly to fp16 pairs), then a DPP butterfly over the lanes of
//     a token (quad_perm, row_half_mirror, row_mirror) - no LDS;
//   * online softmax per lane group (running max m, sum l, fp32 row
//     accumulator, rescaled once per tile), merged across lane groups with
//     shuffles and across waves through LDS, in a fixed order;
//   * base-2 exponent: logits are scaled by scale*log2(e) (times the K scale
//     for FP8) and exponentiated with v_exp_f32;
//   * split context: each partition writes (m, l, normalised row) to the
//     workspace - the row in fp16 (half the bytes to write and read back; a
//     normalised row lies within the range of V), m and l in fp32 - and the
//     reduce kernel merges them with the log-sum-exp identity.
//     A single-partition (sequence, head) writes its fp16 row directly - or,
//     behind a shared prefix whose pieces already sit in the first workspace
//     slots, merges those slots itself and writes the row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = 4;
constexpr int kThreads = kWave * kWaves;
constexpr int kLoads = 8;  // K (and V) 16-byte loads per lane per tile
constexpr float kNegInf = -__builtin_inff();

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }

template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), kCtrl, 0xF, 0xF, false));
}

// Sum over aligned groups of kLanes lanes (4, 8 or 16); every lane of a
// group ends with the group sum.  quad_perm [1,0,3,2], quad_perm [2,3,0,1],
// row_half_mirror, row_mirror.
template <int kLanes>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(kLanes == 4 || kLanes == 8 || kLanes == 16, "group of 4, 8 or 16 lanes");
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    if constexpr (kLanes >= 8)
        v += dpp_mov<0x141>(v);
    if constexpr (kLanes == 16)
        v += dpp_mov<0x140>(v);
    return v;
}

// Max over aligned groups of 16 lanes (the same DPP steps as group_sum).
__device__ __forceinline__ float group_max16(float v)
{
    v = fmaxf(v, dpp_mov<0xB1>(v));
    v = fmaxf(v, dpp_mov<0x4E>(v));
    v = fmaxf(v, dpp_mov<0x141>(v));
    return fmaxf(v, dpp_mov<0x140>(v));
}

// Sum / max over the whole wave, every lane ending with the result: the
// 16-lane groups by DPP, then the four groups by exchanging rows with
// v_permlane32_swap and v_permlane16_swap (no LDS round trip).  Each step adds
// a lane's value and its partner's, in either order: the same bits in both.
__device__ __forceinline__ float wave_sum(float v)
{
    v = group_sum<16>(v);
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max(float v)
{
    v = group_max16(v);
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                    false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int readlane(int v, int lane)
{
    return __builtin_amdgcn_readlane(v, lane);
}

// Hardware workgroup i of n lands on XCD i % 8.  Give XCD x the contiguous
// logical range [x*n/8, (x+1)*n/8) (remainder spread over the first XCDs).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t n)
{
    constexpr uint32_t kXcds = 8;
    const uint32_t q = n / kXcds, r = n % kXcds;
    const uint32_t xcd = i % kXcds, k = i / kXcds;
    return xcd < r ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

// ---- cache element types -------------------------------------------------
// Each lane holds 16 bytes of one token's row: kElems values, whose q
// counterparts are kElems/2 fp16 pairs.  dot() is the lane's share of q.k;
// the V update is written out in tile_step (as a called helper the compiler
// stops keeping the accumulators in registers).

struct KvF16 {
    static constexpr int kElemBytes = 2;
    static constexpr int kElems = 8;
    static constexpr bool kScaledOutput = false;
    // partial q.k over this lane's 8 values
    __device__ static __forceinline__ float dot(const u32x4& k, const h2* q)
    {
        float d = __builtin_amdgcn_fdot2(as_h2(k.x), q[0], 0.0f, false);
        d = __builtin_amdgcn_fdot2(as_h2(k.y), q[1], d, false);
        d = __builtin_amdgcn_fdot2(as_h2(k.z), q[2], d, false);
        return __builtin_amdgcn_fdot2(as_h2(k.w), q[3], d, false);
    }
};

struct KvFp8 {
    static constexpr int kElemBytes = 1;
    static constexpr int kElems = 16;
    static constexpr bool kScaledOutput = true;
    // Widen byte pair kHi (low or high half of w) to an exact fp16 pair.
    template <bool kHi>
    __device__ static __forceinline__ h2 widen(uint32_t w)
    {
        return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHi);
    }
    __device__ static __forceinline__ float dot(const u32x4& k, const h2* q)
    {
        const uint32_t w[4] = {k.x, k.y, k.z, k.w};
        float d = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            d = __builtin_amdgcn_fdot2(widen<false>(w[i]), q[2 * i], d, false);
            d = __builtin_amdgcn_fdot2(widen<true>(w[i]), q[2 * i + 1], d, false);
        }
        return d;
    }
};

template <typename KV>
struct LaneState {
    float m;                // running maximum of base-2 logits (group-uniform)
    float l;                // running sum of exp2(logit - m)
    float acc[KV::kElems];  // running sum of exp2(logit - m) * v over this lane's columns
};

template <typename KV, int D, int B>
struct Geometry {
    static constexpr int kLanesPerToken = D / KV::kElems;    // 16 bytes per lane
    static constexpr int kTokensPerLoad = kWave / kLanesPerToken;
    static constexpr int kTile = kLoads * kTokensPerLoad;     // tokens per wave step
    static_assert(kTile % B == 0 || B % kTile == 0, "tile / block mismatch");
    static_assert(B % kTokensPerLoad == 0, "a load must stay in one block");
};

template <typename KV>
struct TileCtx {
    const char* k;
    const char* v;
    int64_t block_bytes;  // B * H * D * element bytes
    int lane_byte;        // ((g * H + h) * D + lt * kElems) * element bytes, in-block offset 0
    int token_stride;     // H * D * element bytes between consecutive in-block offsets
    int group;            // lane / lanes-per-token
    int end;              // first logical position not attended by this partition
    float scale_log2;
    h2 q[KV::kElems / 2];
};

// One tile of kTile tokens starting at logical position t0 (a multiple of
// the tile).  ids holds table entries [chunk0, chunk0 + 64) in lane order.
template <typename KV, int D, int B, bool kMasked>
__device__ __forceinline__ void tile_step(LaneState<KV>& st, const TileCtx<KV>& c, int t0,
                                          int ids, int chunk0)
{
    using G = Geometry<KV, D, B>;
    u32x4 kr[kLoads], vr[kLoads];
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const int tj = t0 + j * G::kTokensPerLoad;  // first token of this load (uniform)
        if (!kMasked || tj < c.end) {
            const int pb = readlane(ids, tj / B - chunk0);
            const int64_t e = (int64_t)pb * c.block_bytes + (int64_t)((tj % B) * c.token_stride) +
                              c.lane_byte;
            kr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c.k + e));
            vr[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c.v + e));
        } else {
            kr[j] = u32x4{0, 0, 0, 0};
            vr[j] = u32x4{0, 0, 0, 0};
        }
    }
    // FP8: all 2 * kLoads loads issued before any arithmetic (the scheduler otherwise starts the
    // K dot products as the first loads land, keeping about half of them in flight); measured
    // 1-2% faster for FP8 and 1% slower for fp16, which keeps the default schedule.
    if constexpr (KV::kElemBytes == 1)
        __builtin_amdgcn_sched_barrier(0);
    float x[kLoads];
    float tmax = kNegInf;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        float d = group_sum<G::kLanesPerToken>(KV::dot(kr[j], c.q)) * c.scale_log2;
        if (kMasked) {
            const bool valid = t0 + j * G::kTokensPerLoad + c.group < c.end;
            d = valid ? d : kNegInf;
            vr[j] = valid ? vr[j] : u32x4{0, 0, 0, 0};
        }
        x[j] = d;
        tmax = fmaxf(tmax, d);
    }
    const float m_new = fmaxf(st.m, tmax);
    const float m_ref = m_new == kNegInf ? 0.0f : m_new;  // all masked so far: keep zeros
    const float alpha = exp2_fast(st.m - m_ref);
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < KV::kElems; ++i)
        st.acc[i] *= alpha;
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
        const float p = exp2_fast(x[j] - m_ref);
        st.l += p;
        const uint32_t w[4] = {vr[j].x, vr[j].y, vr[j].z, vr[j].w};
        if constexpr (KV::kElemBytes == 2) {  // acc += p * v, 8 fp16 values
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const h2 v2 = as_h2(w[i]);
                st.acc[2 * i] = fmaf(p, (float)v2.x, st.acc[2 * i]);
                st.acc[2 * i + 1] = fmaf(p, (float)v2.y, st.acc[2 * i + 1]);
            }
        } else {  // acc += p * v, 16 FP8 codes decoded exactly to fp32
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const f2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
                const f2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
                st.acc[4 * i] = fmaf(p, lo.x, st.acc[4 * i]);
                st.acc[4 * i + 1] = fmaf(p, lo.y, st.acc[4 * i + 1]);
                st.acc[4 * i + 2] = fmaf(p, hi.x, st.acc[4 * i + 2]);
                st.acc[4 * i + 3] = fmaf(p, hi.y, st.acc[4 * i + 3]);
            }
        }
    }
    st.m = m_new;
}

// Merge (m, l, acc) of two partial softmax states with the log-sum-exp rule.
template <typename KV>
__device__ __forceinline__ void merge_into(LaneState<KV>& st, float m_o, float l_o,
                                           const float* acc_o)
{
    const float M = fmaxf(st.m, m_o);
    const float Mr = M == kNegInf ? 0.0f : M;
    const float wa = exp2_fast(st.m - Mr), wb = exp2_fast(m_o - Mr);
    st.l = st.l * wa + l_o * wb;
#pragma unroll
    for (int i = 0; i < KV::kElems; ++i)
        st.acc[i] = st.acc[i] * wa + acc_o[i] * wb;
    st.m = M;
}

// Element d of the partial row in workspace slot u (a partition's or a
// shared-prefix piece's): stored in fp16 before the FP8 V scale, which is
// applied here (v_scale = 1 for fp16 caches).
template <int D>
__device__ __forceinline__ float slot_row(const DecodeParams& P, int64_t u, int d)
{
    return (float)P.ws_o[u * D + d] * P.v_scale;
}

// Column d of a row whose shared-prefix partials sit in workspace slots
// 0 .. slot_base-1 of u0 and whose one suffix partition has (M, L, o):
// the log-sum-exp merge, prefix slots first, then the suffix (L = 0: none).
template <int D>
__device__ float merge_with_prefix(const DecodeParams& P, int64_t u0, int d, float M, float L,
                                   float o)
{
    float Mx = M;
    for (int p = 0; p < P.slot_base; ++p)
        Mx = fmaxf(Mx, P.ws_m[u0 + p]);
    float wsum = 0.0f, acc = 0.0f;
    for (int p = 0; p < P.slot_base; ++p) {
        const float w = P.ws_l[u0 + p] * exp2_fast(P.ws_m[u0 + p] - Mx);
        wsum += w;
        acc = fmaf(w, slot_row<D>(P, u0 + p, d), acc);
    }
    if (L > 0.0f) {
        const float w = L * exp2_fast(M - Mx);
        wsum += w;
        acc = fmaf(w, o, acc);
    }
    return acc / wsum;
}

template <typename KV, int D, int B>
__global__ __launch_bounds__(kThreads) void pa_partition_kernel(DecodeParams P)
{
    using G = Geometry<KV, D, B>;
    constexpr int LPT = G::kLanesPerToken;
    constexpr int TILE = G::kTile;
    constexpr int E = KV::kElems;
    constexpr int EB = KV::kElemBytes;

    const uint32_t logical = xcd_remap(blockIdx.x, P.total_units);
    const uint32_t rank = logical % (uint32_t)P.num_seqs;
    const uint32_t rest = logical / (uint32_t)P.num_seqs;
    const int part = (int)(rest % (uint32_t)P.num_partitions);
    const int h = (int)(rest / (uint32_t)P.num_partitions);
    // the rank-th sequence of the given order; its length is read by rank,
    // so that both loads issue together
    const int32_t* lens = P.seq_order != nullptr ? P.seq_order_len : P.context_lens;
    const int ctx = lens[rank];
    const int s = P.seq_order != nullptr ? P.seq_order[rank] : (int)rank;
    const int p0 = part * P.partition_size;
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int64_t row = ((int64_t)s * P.num_heads + h) * D;

    if (ctx <= 0) {  // empty context: partition 0 writes the row
        if (part == 0 && threadIdx.x < D) {
            if (P.slot_base == 0)
                P.out[row + threadIdx.x] = (_Float16)0.0f;
            else if (P.num_partitions == 1)  // the shared prefix alone
                P.out[row + threadIdx.x] = (_Float16)merge_with_prefix<D>(
                    P, ((int64_t)s * P.num_heads + h) * P.num_slots, threadIdx.x, kNegInf, 0.0f,
                    0.0f);
        }
        return;
    }
    if (p0 >= ctx)
        return;
    const int end = min(p0 + P.partition_size, ctx);
    const int nparts_seq = (ctx + P.partition_size - 1) / P.partition_size;

    TileCtx<KV> c;
    c.k = static_cast<const char*>(P.k_cache);
    c.v = static_cast<const char*>(P.v_cache);
    c.block_bytes = (int64_t)B * P.num_heads * D * EB;
    c.group = lane / LPT;
    c.token_stride = P.num_heads * D * EB;
    c.lane_byte = ((c.group * P.num_heads + h) * D + (lane % LPT) * E) * EB;
    c.end = end;
    c.scale_log2 = P.scale_log2;
#pragma unroll
    for (int i = 0; i < E / 8; ++i) {
        const u32x4 qv = *reinterpret_cast<const u32x4*>(P.q + row + (lane % LPT) * E + 8 * i);
        c.q[4 * i] = as_h2(qv.x);
        c.q[4 * i + 1] = as_h2(qv.y);
        c.q[4 * i + 2] = as_h2(qv.z);
        c.q[4 * i + 3] = as_h2(qv.w);
    }

    LaneState<KV> st;
    st.m = kNegInf;
    st.l = 0.0f;
#pragma unroll
    for (int i = 0; i < E; ++i)
        st.acc[i] = 0.0f;

    const int32_t* table = P.block_tables + (int64_t)s * P.max_blocks_per_seq;
    const int first_blk = p0 / B;
    const int last_blk = (end + B - 1) / B;  // exclusive
    // Chunks of 64 table entries; a chunk spans 64*B tokens = whole tiles.
    for (int chunk0 = first_blk; chunk0 < last_blk; chunk0 += kWave) {
        const int n_ids = min(kWave, last_blk - chunk0);
        const int ids = lane < n_ids ? table[chunk0 + lane] : 0;
        const int tok_lo = chunk0 * B;
        const int tok_hi = min(end, (chunk0 + kWave) * B);
        for (int t0 = tok_lo + wave * TILE; t0 < tok_hi; t0 += kWaves * TILE) {
            if (t0 + TILE <= end)
                tile_step<KV, D, B, false>(st, c, t0, ids, chunk0);
            else
                tile_step<KV, D, B, true>(st, c, t0, ids, chunk0);
        }
    }

    // Merge the lane groups of this wave (lanes l, l^LPT, l^2LPT, ...).
#pragma unroll
    for (int off = LPT; off < kWave; off <<= 1) {
        float acc_o[E];
#pragma unroll
        for (int i = 0; i < E; ++i)
            acc_o[i] = __shfl_xor(st.acc[i], off);
        const float m_o = __shfl_xor(st.m, off);
        const float l_o = __shfl_xor(st.l, off);
        merge_into(st, m_o, l_o, acc_o);
    }

    // Merge the waves through LDS in wave order.
    __shared__ float s_acc[kWaves][D];
    __shared__ float s_m[kWaves], s_l[kWaves];
    if (lane < LPT) {
#pragma unroll
        for (int i = 0; i < E; ++i)
            s_acc[wave][lane * E + i] = st.acc[i];
    }
    if (lane == 0) {
        s_m[wave] = st.m;
        s_l[wave] = st.l;
    }
    __syncthreads();
    if (threadIdx.x < D) {
        const int d = threadIdx.x;
        float M = s_m[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w)
            M = fmaxf(M, s_m[w]);
        float L = 0.0f, o = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float wt = s_m[w] == kNegInf ? 0.0f : exp2_fast(s_m[w] - M);
            L = fmaf(s_l[w], wt, L);
            o = fmaf(s_acc[w][d], wt, o);
        }
        o = o / L;
        const float o_scaled = KV::kScaledOutput ? o * P.v_scale : o;
        if (nparts_seq == 1 && P.slot_base == 0) {
            P.out[row + d] = (_Float16)o_scaled;
        } else if (P.slot_base > 0 && P.num_partitions == 1) {
            P.out[row + d] = (_Float16)merge_with_prefix<D>(
                P, ((int64_t)s * P.num_heads + h) * P.num_slots, d, M, L, o_scaled);
        } else {  // a partial row for the reduce: fp16, before the FP8 V scale
            const int64_t u = ((int64_t)s * P.num_heads + h) * P.num_slots + P.slot_base + part;
            P.ws_o[u * D + d] = (_Float16)o;
            if (d == 0) {
                P.ws_m[u] = M;
                P.ws_l[u] = L;
            }
        }
    }
}

// Merge the partitions of one (sequence, head): M = max m_p,
// w_p = l_p * 2^(m_p - M), out = sum_p w_p o_p / sum_p w_p.  One wave per
// (sequence, head), four per workgroup.  Lane i takes the (m, l) of
// partitions i, i + 64, ...; M and sum_p w_p come from fixed butterflies; each
// lane owns D / 64 output columns and adds w_p o_p over the partitions in
// order p = 0, 1, ... (the weight broadcast from its lane with v_readlane),
// up to sixteen slot loads in flight; the rows are fp16 before any FP8 V
// scale, which is applied once to the merged row.
// A fixed order, so the result is deterministic.
template <int D>
__global__ __launch_bounds__(kThreads) void pa_reduce_kernel(DecodeParams P)
{
    constexpr int CPL = D / kWave;  // output columns per lane
    static_assert(CPL == 1 || CPL == 2, "head_dim 64 or 128");
    const int lane = threadIdx.x % kWave;
    const int sh = blockIdx.x * kWaves + threadIdx.x / kWave;
    if (sh >= P.num_seqs * P.num_heads)
        return;  // no barriers in this kernel
    const int s = sh / P.num_heads;
    const int ctx = P.context_lens[s];
    // slots in use: the shared-prefix slots (if any) + this sequence's partitions
    const int np = P.slot_base + (ctx + P.partition_size - 1) / P.partition_size;
    if (np == 0 || (np == 1 && P.slot_base == 0))
        return;  // nothing to merge (an unsplit sequence wrote its own row)
    const int64_t u0 = (int64_t)sh * P.num_slots;
    const float* m = P.ws_m + u0;
    const float* l = P.ws_l + u0;
    _Float16* orow = P.out + (int64_t)sh * D + lane * CPL;

    constexpr int kFirst = 8;  // partitions the one-round-trip path takes
    if (np <= kFirst) {
        // The usual case, in one round trip after the context length: the
        // (m, l) of partition `lane` and the rows of all np partitions are
        // loaded together (the rows do not depend on the weights), and the
        // wave's max and sum take register exchanges.  The rows are added in
        // partition order, as in the general path below.
        const bool has = lane < np;
        const int lc = min(lane, np - 1);  // a written slot for every lane
        const float m_raw = m[lc], l_raw = l[lc];
        const _Float16* oc = P.ws_o + u0 * D + lane * CPL;
        // Loads of rows past np read row np-1 again (a written slot) and go
        // unused: straight-line loads, all in flight together (a load under
        // a branch would be waited for before the branch joins).
        float ob[kFirst][CPL];
#pragma unroll
        for (int j = 0; j < kFirst; ++j) {
            const int64_t r = min(j, np - 1);
            if constexpr (CPL == 2) {
                const h2 o2 = *reinterpret_cast<const h2*>(oc + r * D);
                ob[j][0] = (float)o2.x;
                ob[j][1] = (float)o2.y;
            } else {
                ob[j][0] = (float)oc[r * D];
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // every load above issued before the first wait
        const float mp = has ? m_raw : kNegInf;
        const float lp = has ? l_raw : 0.0f;
        const float Mx = wave_max(mp);
        const float w = has ? lp * exp2_fast(mp - Mx) : 0.0f;
        const float Lx = wave_sum(w);
        float acc[CPL] = {};
        auto wj = [&](int j) {
            return __builtin_bit_cast(float,
                                      __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
        };
#pragma unroll
        for (int j = 0; j < kFirst; ++j) {
            if (j < np) {
#pragma unroll
                for (int i = 0; i < CPL; ++i)
                    acc[i] = fmaf(wj(j), ob[j][i], acc[i]);
            }
        }
#pragma unroll
        for (int i = 0; i < CPL; ++i)
            orow[i] = (_Float16)(acc[i] / Lx * P.v_scale);  // the FP8 V scale (1 for fp16)
        return;
    }

    float M = kNegInf;
    for (int p = lane; p < np; p += kWave)
        M = fmaxf(M, m[p]);
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1)
        M = fmaxf(M, __shfl_xor(M, off));

    float acc[CPL] = {};
    float L = 0.0f;
    for (int c0 = 0; c0 < np; c0 += kWave) {
        const int p = c0 + lane;
        const float w = p < np ? l[p] * exp2_fast(m[p] - M) : 0.0f;
        float wsum = w;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1)
            wsum += __shfl_xor(wsum, off);
        L += wsum;
        const int n = min(kWave, np - c0);
        const _Float16* oc = P.ws_o + (u0 + c0) * D + lane * CPL;
        auto add = [&](int j) {
            const float wj = __builtin_bit_cast(
                float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, w), j));
            if constexpr (CPL == 2) {
                const h2 o2 = *reinterpret_cast<const h2*>(oc + (int64_t)j * D);
                acc[0] = fmaf(wj, (float)o2.x, acc[0]);
                acc[1] = fmaf(wj, (float)o2.y, acc[1]);
            } else {
                acc[0] = fmaf(wj, (float)oc[(int64_t)j * D], acc[0]);
            }
        };
        int j = 0;
        for (; j + 16 <= n; j += 16) {  // sixteen independent loads in flight
#pragma unroll
            for (int k = 0; k < 16; ++k)
                add(j + k);
        }
        for (; j + 4 <= n; j += 4) {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                add(j + k);
        }
        for (; j < n; ++j)
            add(j);
    }
#pragma unroll
    for (int i = 0; i < CPL; ++i)
        orow[i] = (_Float16)(acc[i] / L * P.v_scale);  // the FP8 V scale (1 for fp16)
}

template <typename KV, int D, int B>
hipError_t launch_partitions(const DecodeParams& P, hipStream_t stream)
{
    hipLaunchKernelGGL((pa_partition_kernel<KV, D, B>), dim3(P.total_units), dim3(kThreads), 0,
                       stream, P);
    return hipGetLastError();
}

template <typename KV>
hipError_t dispatch_partitions(const DecodeParams& P, int head_dim, int block_size,
                               hipStream_t stream)
{
    if (head_dim == 128 && block_size == 16)
        return launch_partitions<KV, 128, 16>(P, stream);
    if (head_dim == 128 && block_size == 32)
        return launch_partitions<KV, 128, 32>(P, stream);
    if (head_dim == 64 && block_size == 16)
        return launch_partitions<KV, 64, 16>(P, stream);
    if (head_dim == 64 && block_size == 32)
        return launch_partitions<KV, 64, 32>(P, stream);
    return hipErrorInvalidValue;
}

template <typename KV>
hipError_t dispatch(const DecodeParams& P, int head_dim, int block_size, hipStream_t stream)
{
    hipError_t e = dispatch_partitions<KV>(P, head_dim, block_size, stream);
    if (e == hipSuccess)
        e = launch_decode_reduce(P, head_dim, stream);
    return e;
}

}  // namespace

hipError_t launch_decode_reduce(const DecodeParams& P, int head_dim, hipStream_t stream)
{
    if (P.num_partitions <= 1)
        return hipSuccess;  // the partition kernel wrote every row
    const dim3 grid((uint32_t)(((int64_t)P.num_seqs * P.num_heads + kWaves - 1) / kWaves));
    if (head_dim == 128)
        hipLaunchKernelGGL((pa_reduce_kernel<128>), grid, dim3(kThreads), 0, stream, P);
    else if (head_dim == 64)
        hipLaunchKernelGGL((pa_reduce_kernel<64>), grid, dim3(kThreads), 0, stream, P);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t launch_decode_partitions(const DecodeParams& P, int head_dim, int block_size,
                                    hipStream_t stream)
{
    return dispatch_partitions<KvF16>(P, head_dim, block_size, stream);
}

hipError_t launch_decode_dispatch(const DecodeParams& P, int head_dim, int block_size,
                                  hipStream_t stream)
{
    return dispatch<KvF16>(P, head_dim, block_size, stream);
}

hipError_t launch_decode_fp8_dispatch(const DecodeParams& P, int head_dim, int block_size,
                                      hipStream_t stream)
{
    return dispatch<KvFp8>(P, head_dim, block_size, stream);
}

}  // namespace pa
