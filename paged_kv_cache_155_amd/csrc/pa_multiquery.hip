// Paged attention for several query rows that share one K/V token stream,
// on the matrix cores of gfx950 (fp16 KV, fp32 accumulation).
//
// Sources (web pages), cited by title and section:
//   [10x]  "vLLM推理加速深度解读：PagedAttention如何提升10x吞吐量" §2.3 (the
//          paged gather), §4.3 (prefill and decode work in one batch), §4.4
//          (requests sharing a prefix reuse its blocks)
//   [eng]  "深入解析LLM推理引擎：从PagedAttention到调度优化" §3.2 (shared
//          prefix blocks), §4.2 (mixed prefill / decode batches)
//
// Two uses of one kernel, each a group of up to 16 query rows per wave:
//   * multi-query (chunked prefill): 16 consecutive new tokens of one
//     sequence; row r at logical position p_r sees positions 0..p_r;
//   * shared prefix (cascade decode): the decode queries of 16 sequences that
//     all list the same prefix blocks first; every row sees the whole prefix,
//     which is therefore read once per 16 sequences instead of once per
//     sequence.  The prefix is cut into partitions of a few blocks (one wave
//     each, so the short stream still fills the chip); each yields a
//     log-sum-exp partial that the decode reduce merges with the partials of
//     the private suffixes.
//
// Per 16-token block of the stream (always inside one physical block, B is
// 16 or 32), with K, V rows of one head loaded as 16-byte vectors:
//   S^T = K Q^T   8 x v_mfma_f32_16x16x16f16 (k runs over the head dim; each
//                 lane group of 16 lanes owns a contiguous quarter of the
//                 dims, so K and Q are read as they lie in memory)
//   online softmax per query row on the S^T tile (lane = query, 4 tokens
//                 per lane), base-2 exponent
//   O^T += V^T P^T  8 x v_mfma_f32_16x16x16f16: the S^T tile is already P^T
//                 in the B-operand layout, and O^T comes out with the query
//                 as the lane's column, like the softmax state, so rescaling
//                 needs no cross-lane traffic.  V goes through LDS in its own
//                 row layout (16-byte stores, rows padded to 136 halves so the
//                 four lane groups use different banks); each lane then reads
//                 its 4 tokens of one column as 2-byte values.
// The K/V loads of the next block are issued before the current block is
// computed (register double buffering), so one block's latency hides behind
// the previous block's math.
// Positions past the stream end get -inf scores and zero V rows (select, not
// multiply), so unread slots may hold anything.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr float kNegInf = -__builtin_inff();

typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ h4 lo_h4(const u32x4& v) { return __builtin_bit_cast(h4, u32x2{v.x, v.y}); }
__device__ __forceinline__ h4 hi_h4(const u32x4& v) { return __builtin_bit_cast(h4, u32x2{v.z, v.w}); }

// Hardware workgroup i of n lands on XCD i % 8; XCD x gets logical range
// [x*n/8, (x+1)*n/8).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t n)
{
    constexpr uint32_t kXcds = 8;
    const uint32_t q = n / kXcds, r = n % kXcds;
    const uint32_t xcd = i % kXcds, k = i / kXcds;
    return xcd < r ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

template <int D, int B, bool kCascade>
__global__ __launch_bounds__(kWave) void pa_mq_kernel(MqParams P)
{
    constexpr int NB = D / 16;     // 16-column blocks of the output
    constexpr int LPR = D / 32;    // 16-byte loads per lane per K (or V) row quarter
    constexpr int VS = D + 8;      // LDS row stride (halves) of the V tile
    static_assert(B % 16 == 0, "16-token blocks must stay inside one physical block");

    const int lane = threadIdx.x;
    const int g = lane / 16;       // lane group: owns dims [g*D/4, (g+1)*D/4)
    const int c = lane % 16;       // this lane's query column of S^T (and token row of K)

    const uint32_t logical = xcd_remap(blockIdx.x, P.total_units);
    const int h = (int)(logical % (uint32_t)P.num_heads);
    const int unit = (int)(logical / (uint32_t)P.num_heads);

    // ---- the 16 query rows of this unit and the token stream they share ----
    int s_first = 0, seq = 0, n_rows = 0, limit = 0, stream_begin = 0, stream_end = 0;
    int part = 0;
    int64_t q_row = 0;
    const int32_t* table;
    if constexpr (kCascade) {
        part = unit % P.prefix_parts;            // prefix tokens [part*len, (part+1)*len)
        s_first = (unit / P.prefix_parts) * 16;  // sequences s_first .. s_first+15
        n_rows = min(16, P.num_seqs - s_first);
        seq = s_first + c;
        q_row = seq;
        stream_begin = part * P.prefix_part_len;
        stream_end = min(stream_begin + P.prefix_part_len, P.prefix_len);
        limit = c < n_rows ? stream_end : 0;
        table = P.prefix_table;
    } else {
        const int chunk = unit % P.max_chunks;   // 16-row chunk of a sequence's new tokens
        seq = unit / P.max_chunks;
        const int q0 = P.query_start[seq];
        const int n = P.query_start[seq + 1] - q0;
        const int r0 = chunk * 16;
        if (r0 >= n)
            return;
        n_rows = min(16, n - r0);
        const int ctx = P.context_lens[seq];
        q_row = q0 + r0 + c;
        limit = c < n_rows ? ctx - n + r0 + c + 1 : 0;
        stream_end = ctx - n + r0 + n_rows;      // the last row's position + 1
        table = P.block_tables + (int64_t)seq * P.max_blocks_per_seq;
    }

    // Q^T as MFMA B operand: lane (query c) holds dims [g*D/4, g*D/4 + D/4).
    u32x4 qf[LPR];
    {
        const bool valid = c < n_rows;
        const u32x4* qp = reinterpret_cast<const u32x4*>(
            P.q + (q_row * P.num_heads + h) * D + g * (D / 4));
#pragma unroll
        for (int i = 0; i < LPR; ++i)
            qf[i] = valid ? qp[i] : u32x4{0, 0, 0, 0};
    }

    f4 o[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        o[nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    float m = kNegInf, lsum = 0.0f;  // softmax state of query c

    __shared__ __attribute__((aligned(16))) _Float16 vt[16 * VS];  // V of one block: [token][dim]

    const int64_t block_elems = (int64_t)B * P.num_heads * D;
    const int token_stride = P.num_heads * D;
    const int lane_elem = h * D + g * (D / 4);
    // K/V of the 16-token block at t (this lane: token t + c, its quarter of the dims)
    auto load_block = [&](int t, u32x4* kd, u32x4* vd) {
        const int pb = table[t / B];
        const int64_t e = (int64_t)pb * block_elems + (int64_t)((t % B) + c) * token_stride +
                          lane_elem;
#pragma unroll
        for (int i = 0; i < LPR; ++i) {
            kd[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(P.k_cache + e) + i);
            vd[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(P.v_cache + e) + i);
        }
    };
    u32x4 kr[LPR], vr[LPR];
    if (stream_begin < stream_end)
        load_block(stream_begin, kr, vr);
    for (int t0 = stream_begin; t0 < stream_end; t0 += 16) {
        const bool live = t0 + c < stream_end;   // this lane's K/V token exists
        u32x4 kn[LPR], vn[LPR];
        if (t0 + 16 < stream_end)
            load_block(t0 + 16, kn, vn);

        // S^T[token 4g+j][query c] over the head dim
        f4 st = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < LPR; ++i) {
            st = __builtin_amdgcn_mfma_f32_16x16x16f16(lo_h4(kr[i]), lo_h4(qf[i]), st, 0, 0, 0);
            st = __builtin_amdgcn_mfma_f32_16x16x16f16(hi_h4(kr[i]), hi_h4(qf[i]), st, 0, 0, 0);
        }

        // online softmax for query c over tokens t0 + 4g + j
        float x[4];
        float bmax = kNegInf;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bool vis = t0 + 4 * g + j < limit;
            x[j] = vis ? st[j] * P.scale_log2 : kNegInf;
            bmax = fmaxf(bmax, x[j]);
        }
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
        const float m_new = fmaxf(m, bmax);
        const float m_ref = m_new == kNegInf ? 0.0f : m_new;
        const float alpha = exp2_fast(m - m_ref);
        h4 pa;
        float psum = 0.0f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float p = exp2_fast(x[j] - m_ref);
            psum += p;
            pa[j] = (_Float16)p;
        }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        lsum = lsum * alpha + psum;
        m = m_new;

        // rescale this query's columns of O^T
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                o[nb][j] *= alpha;

        // V block -> LDS as it lies in memory (rows past the stream end are zero)
        {
            u32x4* row = reinterpret_cast<u32x4*>(&vt[c * VS + g * (D / 4)]);
#pragma unroll
            for (int i = 0; i < LPR; ++i)
                row[i] = live ? vr[i] : u32x4{0, 0, 0, 0};
        }
        __syncthreads();
        // A operand V^T[column 16nb + c][token 4g + j]
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
            h4 va;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                va[j] = vt[(4 * g + j) * VS + nb * 16 + c];
            o[nb] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pa, o[nb], 0, 0, 0);
        }
        __syncthreads();  // the tile is rewritten next iteration
#pragma unroll
        for (int i = 0; i < LPR; ++i) {
            kr[i] = kn[i];
            vr[i] = vn[i];
        }
    }

    // O^T[column 16nb + 4g + j][query c] / l(query c)
    if (c < n_rows) {
        const float inv = lsum > 0.0f ? 1.0f / lsum : 0.0f;
        if constexpr (kCascade) {
            const int64_t u = ((int64_t)seq * P.num_heads + h) * P.num_slots + part;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                f4 r = o[nb] * inv;
                *reinterpret_cast<f4*>(&P.ws_o[u * D + nb * 16 + 4 * g]) = r;
            }
            if (g == 0) {
                P.ws_m[u] = m;
                P.ws_l[u] = lsum;
            }
        } else {
            _Float16* orow = P.out + (q_row * P.num_heads + h) * D;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                h4 r;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    r[j] = (_Float16)(o[nb][j] * inv);
                *reinterpret_cast<h4*>(&orow[nb * 16 + 4 * g]) = r;
            }
        }
    }
}

template <bool kCascade>
hipError_t launch_mq(const MqParams& P, int head_dim, int block_size, hipStream_t stream)
{
    const dim3 grid(P.total_units), block(kWave);
    if (head_dim == 128 && block_size == 16)
        hipLaunchKernelGGL((pa_mq_kernel<128, 16, kCascade>), grid, block, 0, stream, P);
    else if (head_dim == 128 && block_size == 32)
        hipLaunchKernelGGL((pa_mq_kernel<128, 32, kCascade>), grid, block, 0, stream, P);
    else if (head_dim == 64 && block_size == 16)
        hipLaunchKernelGGL((pa_mq_kernel<64, 16, kCascade>), grid, block, 0, stream, P);
    else if (head_dim == 64 && block_size == 32)
        hipLaunchKernelGGL((pa_mq_kernel<64, 32, kCascade>), grid, block, 0, stream, P);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_multiquery(const MqParams& p, int head_dim, int block_size, hipStream_t stream)
{
    return launch_mq<false>(p, head_dim, block_size, stream);
}

hipError_t launch_cascade_prefix(const MqParams& p, int head_dim, int block_size,
                                 hipStream_t stream)
{
    return launch_mq<true>(p, head_dim, block_size, stream);
}

}  // namespace pa
