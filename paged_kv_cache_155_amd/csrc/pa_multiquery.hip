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
// Two uses of one kernel; a workgroup of 4 waves owns a tile of query rows
// (16 * QT per wave) that all read the same token stream:
//   * multi-query (chunked prefill): consecutive new tokens of one sequence;
//     row r at logical position p_r sees positions 0..p_r;
//   * shared prefix (cascade decode): the decode queries of many sequences
//     that all list the same prefix blocks first; every row sees the whole
//     prefix, which is therefore read once per tile of sequences instead of
//     once per sequence.  The prefix is cut into partitions so that the short
//     stream still fills the chip; each yields a log-sum-exp partial that the
//     decode reduce merges with the partials of the private suffixes.  One
//     more workgroup of this launch orders the sequences by suffix length for
//     the suffix launch that follows (longest first).
//
// Per chunk of the stream (32 tokens for fp16 multi-query, 64 otherwise):
//   * the workgroup loads it once into LDS, [token][dim] tiles with unpadded
//     rows whose 16-byte pieces are XOR-swizzled by row (so the operand reads
//     below fall on distinct banks), double buffered so one barrier per chunk
//     suffices; the next chunk is loaded while this one is computed.  fp16
//     caches go straight to LDS (buffer loads with an LDS destination, 1 KiB
//     per wave instruction, one block per wave and chunk); FP8 caches pass
//     through registers, where they are widened to fp16;
//   * each wave, for its 16 * QT rows:
//       S^T = K Q^T      v_mfma_f32_16x16x32_f16 over the head dim (each lane
//                        group owns a contiguous quarter of the dims, so K and
//                        Q are read as they lie)
//       online softmax   per query column (lane = query, 16 tokens per lane),
//                        base-2 exponent against a lazy reference: the scores
//                        are shifted by it, and only when a shifted score in the
//                        wave passes 2^8 (or a reference is unset) are the row
//                        maxima exchanged across the four lane groups (permlane
//                        swaps), the reference moved and O rescaled
//       l += ones P^T    the row sums on the matrix cores: the fp16 weights
//                        that P.V takes, summed in fp32
//       O^T += V^T P^T   v_mfma_f32_16x16x32_f16 over 32 tokens; the S^T
//                        tiles are already P^T in the B-operand layout, and
//                        the V^T operand comes from the transposing LDS read
//                        ds_read_b64_tr_b16 on the [token][dim] V tile
// Positions past a row's limit get -inf scores; K/V rows past the stream end
// are loaded as zeros (select, not multiply), so unread slots may hold
// anything.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_fp8_quant.h"
#include "pa_internal.h"

namespace pa {
namespace {

constexpr int kWave = 64;
constexpr int kWaves = kMqThreads / kWave;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLazyRescale = 8.0f;  // log2 units: weights stay below 256
constexpr int kCopyItems = 4;         // new-row pieces per thread of a copy workgroup
constexpr int kOrderBuckets = 1024;   // suffix-length buckets of the ordering workgroup
// s_waitcnt vmcnt(0), the other counters left alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kWaitVmcnt0 = 0x0F70;
// the last word of a raw buffer resource on gfx9 parts (32-bit data, no swizzle)
constexpr int kBufferFlags = 0x00020000;

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ h8 as_h8(const u32x4& v) { return __builtin_bit_cast(h8, v); }

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

// K/V elements as they lie in the cache: 8 fp16 values (16 bytes), or 8 FP8
// (OCP E4M3) codes (8 bytes) that staging widens exactly to fp16 (every E4M3
// value is an fp16 value; the cache scales are applied outside the tile).
template <bool kFp8> struct Raw8 { typedef u32x4 type; };
template <> struct Raw8<true> { typedef u32x2 type; };

__device__ __forceinline__ u32x4 widen8(const u32x4& v) { return v; }
__device__ __forceinline__ u32x4 widen8(const u32x2& v)
{
    const h2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.x, 1.0f, false);  // bytes 0, 1
    const h2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.x, 1.0f, true);   // bytes 2, 3
    const h2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.y, 1.0f, false);
    const h2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v.y, 1.0f, true);
    return u32x4{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b),
                 __builtin_bit_cast(uint32_t, c), __builtin_bit_cast(uint32_t, d)};
}

typedef short s4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s4 lds_s4;
// ds_read_b64_tr_b16 (transposing LDS read; 8-byte aligned LDS address)
__device__ __forceinline__ s4 ds_read_tr16(const _Float16* p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s4*)(p));
}

// The V^T operand of one MFMA (16 dims x 32 tokens): two transposing reads of
// the tile's token rows 0..15 and 16..31 (rows of D halves) at this lane's
// offset (elements).
template <int D>
__device__ __forceinline__ h8 read_vt(const _Float16* tile, int off)
{
    const s4 lo = ds_read_tr16(&tile[off]);
    const s4 hi = ds_read_tr16(&tile[16 * D + off]);
    return __builtin_bit_cast(h8, u32x4{__builtin_bit_cast(u32x2, lo).x, __builtin_bit_cast(u32x2, lo).y,
                                        __builtin_bit_cast(u32x2, hi).x, __builtin_bit_cast(u32x2, hi).y});
}

// max over the four 16-lane groups (lanes c, c+16, c+32, c+48)
__device__ __forceinline__ float group_max(float x)
{
    auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

}  // namespace

// Workgroups that the appending shared-prefix pass adds for the copy.
int64_t copy_workgroups(const MqParams& P, int head_dim)
{
    if (P.new_k == nullptr)
        return 0;
    const int64_t items = (int64_t)P.num_seqs * P.num_heads * (head_dim / 8);
    const int64_t wgs = (items + (int64_t)kMqThreads * kCopyItems - 1) /
                        ((int64_t)kMqThreads * kCopyItems);
    return (wgs + 7) / 8 * 8;  // whole rounds of the 8 XCDs
}

namespace {

// Hardware workgroup i of n lands on XCD i % 8; XCD x gets logical range
// [x*n/8, (x+1)*n/8).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t i, uint32_t n)
{
    constexpr uint32_t kXcds = 8;
    const uint32_t q = n / kXcds, r = n % kXcds;
    const uint32_t xcd = i % kXcds, k = i / kXcds;
    return xcd < r ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}

// LDS tiles are [token][dim] with unpadded rows; the 16-byte piece p (dims
// 8p .. 8p+7) of row r is stored at piece p ^ swz(r).  With 64 banks of 4
// bytes, a 256-byte span holds 256 / (2 D) rows.  K (read 16 bytes per lane,
// the 16 lanes of a group on 16 consecutive rows): the rows sharing a span
// half get distinct pieces.  V (read with the transposing 8-byte read, the 16
// lanes of a group on 4 consecutive rows x 2 pieces x 2 halves): the shift by
// one bit keeps the piece's low bit free for the two pieces of a row.
// 16 bytes per lane from base + voff into LDS at lds + 16 * lane: a buffer
// load through a resource on base (scalar registers), so the lane offset is
// the only vector operand
__device__ __forceinline__ void load_lds16(const char* base, _Float16* lds, uint32_t voff)
{
    typedef __attribute__((address_space(3))) void lds_void;
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, 0x7fffffff, kBufferFlags);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, 0, 0, 0);
}

template <int D> __device__ __forceinline__ int swz_k(int r) { return (r / (128 / D)) % (D / 8); }
template <int D> __device__ __forceinline__ int swz_v(int r) { return (2 * (r / (128 / D))) % (D / 8); }

// Appending form of the shared-prefix pass: the first workgroups of the grid
// copy this step's new K/V rows (row s of new_k / new_v [S, H, D]) to their
// slots, 16 bytes of K and of V per item, kCopyItems items per thread with
// every load (slot and data alike) issued before the first store.  The slots
// are private suffix slots, so these writes never meet the prefix units'
// reads.  FP8 caches get the codes of the cache-write quantiser.
template <int D, bool kFp8>
__device__ void copy_new_rows(const MqParams& P, uint32_t wg)
{
    constexpr int kPieces = D / 8;  // 16-byte pieces of a head row
    const int64_t items = (int64_t)P.num_seqs * P.num_heads * kPieces;
    const int64_t first = (int64_t)wg * kMqThreads * kCopyItems + threadIdx.x;
    u32x4 kv[kCopyItems], vv[kCopyItems];
    int64_t dst[kCopyItems];
#pragma unroll
    for (int j = 0; j < kCopyItems; ++j) {
        const int64_t i = first + (int64_t)j * kMqThreads;
        dst[j] = -1;
        if (i < items) {
            const int64_t row = i / kPieces;  // sequence * H + head
            const int piece = (int)(i % kPieces);
            const int64_t slot = P.slot_mapping[row / P.num_heads];
            kv[j] = *reinterpret_cast<const u32x4*>(P.new_k + row * D + piece * 8);
            vv[j] = *reinterpret_cast<const u32x4*>(P.new_v + row * D + piece * 8);
            if (slot >= 0 && slot < P.cache_slots)
                dst[j] = (slot * P.num_heads + row % P.num_heads) * D + piece * 8;
        }
    }
#pragma unroll
    for (int j = 0; j < kCopyItems; ++j) {
        if (dst[j] >= 0) {
            if constexpr (kFp8) {  // one byte per element
                *reinterpret_cast<u32x2*>(static_cast<char*>(P.k_store) + dst[j]) =
                    fp8::quantize8(kv[j], P.k_inv);
                *reinterpret_cast<u32x2*>(static_cast<char*>(P.v_store) + dst[j]) =
                    fp8::quantize8(vv[j], P.v_inv);
            } else {
                *reinterpret_cast<u32x4*>(static_cast<_Float16*>(P.k_store) + dst[j]) = kv[j];
                *reinterpret_cast<u32x4*>(static_cast<_Float16*>(P.v_store) + dst[j]) = vv[j];
            }
        }
    }
}

// Shared-prefix pass, workgroup 0: the order in which the suffix launch that
// follows takes the sequences, longest suffix first, so that its long units
// start early and the launch drains on short ones.  A counting sort on the
// suffix length (descending; clamped to [0, order_max_len] and grouped into at
// most kOrderBuckets buckets of equal width): histogram, exclusive scan,
// scatter, with LDS atomics.  Sequences of one bucket come in whatever order
// the atomics give; the order decides only which workgroup computes which
// sequence, never a result.  cnt: kOrderBuckets + kWaves ints of LDS.
__device__ void order_by_suffix_length(const MqParams& P, int* cnt)
{
    constexpr int kPer = kOrderBuckets / kMqThreads;  // buckets per thread in the scan
    static_assert(kOrderBuckets % kMqThreads == 0, "scan geometry");
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int max_len = P.order_max_len;
    const int width = max_len / kOrderBuckets + 1;  // (max_len - 0) / width < kOrderBuckets
    auto bucket = [&](int len) { return (max_len - min(max(len, 0), max_len)) / width; };

    for (int b = tid; b < kOrderBuckets; b += kMqThreads)
        cnt[b] = 0;
    __syncthreads();
    for (int i = tid; i < P.num_seqs; i += kMqThreads)
        atomicAdd(&cnt[bucket(P.suffix_lens[i])], 1);
    __syncthreads();
    // exclusive scan: thread t owns buckets [kPer t, kPer t + kPer)
    int c[kPer], own = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        c[j] = cnt[kPer * tid + j];
        own += c[j];
    }
    int incl = own;  // inclusive scan over the wave
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d)
            incl += y;
    }
    if (lane == kWave - 1)
        cnt[kOrderBuckets + wave] = incl;
    __syncthreads();
    int start = incl - own;
    for (int w = 0; w < wave; ++w)
        start += cnt[kOrderBuckets + w];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {  // this thread's buckets only
        cnt[kPer * tid + j] = start;
        start += c[j];
    }
    __syncthreads();
    for (int i = tid; i < P.num_seqs; i += kMqThreads) {
        const int len = P.suffix_lens[i];
        const int pos = atomicAdd(&cnt[bucket(len)], 1);
        if (pos < P.num_seqs) {  // always, unless the lengths changed between the reads
            P.seq_order[pos] = i;
            P.seq_order_len[pos] = len;
        }
    }
}

// Chunk length and the waves per SIMD asked of the compiler.  The fp16
// multi-query tile takes 32-token chunks: half the score and weight registers
// and half the LDS of 64, so that three workgroups (three waves per SIMD) fit
// -- measured 5.4% faster than 64 tokens at two.  The FP8 form (staging
// registers) and the shared-prefix pass keep 64-token chunks.
template <bool kCascade, bool kFp8> struct MqShape {
    static constexpr int kChunk = (!kCascade && !kFp8) ? 32 : kMqChunk;
    static constexpr int kWavesPerSimd = (!kCascade && !kFp8) ? 3 : 1;
};

template <int D, int B, bool kCascade, int QT, bool kFp8>
__global__ __launch_bounds__(kMqThreads) __attribute__((amdgpu_waves_per_eu(
    MqShape<kCascade, kFp8>::kWavesPerSimd))) void pa_mq_kernel(MqParams P)
{
    constexpr int N = MqShape<kCascade, kFp8>::kChunk;  // tokens per staged chunk
    constexpr int NB = D / 16;            // 16-dim blocks of O^T
    constexpr int KI = D / 32;            // MFMA k-steps over the head dim
    constexpr int WROWS = 16 * QT;        // query rows per wave
    constexpr int ROWS = kWaves * WROWS;  // query rows per workgroup
    constexpr int DG = D / 8;             // 8-dim groups per token row
    constexpr int UNITS = (N / 4) * DG;   // 4-token x 8-dim load units per chunk
    constexpr int WR = N / kWaves;        // rows of a chunk that each wave loads
    constexpr int RPI = 64 / DG;          // rows per direct-to-LDS load (64 lanes x 16 bytes)
    constexpr int DJ = WR / RPI;          // direct loads per wave and tile
    static_assert(N % 32 == 0 && UNITS <= kMqThreads && DG <= 16 && DJ >= 1, "chunk geometry");
    static_assert(B % WR == 0, "a wave's rows of a chunk must stay inside one physical block");
    static_assert(ROWS == (kCascade ? kCascadeTileRows : kMqTileRows), "tile rows");

    __shared__ __attribute__((aligned(16))) _Float16 k_lds[2][N * D];  // [token][dim], swizzled
    __shared__ __attribute__((aligned(16))) _Float16 v_lds[2][N * D];

    uint32_t wg = blockIdx.x;
    if constexpr (kCascade) {
        static_assert(N * D * sizeof(_Float16) >= (kOrderBuckets + kWaves) * sizeof(int),
                      "the ordering workgroup's counters fit in one K tile");
        if (wg == P.copy_units + P.total_units) {  // the ordering workgroup, last
            order_by_suffix_length(P, reinterpret_cast<int*>(&k_lds[0][0]));
            return;
        }
        if (wg < P.copy_units) {  // a copy workgroup (appending form only)
            copy_new_rows<D, kFp8>(P, wg);
            return;  // the whole workgroup, before any barrier
        }
        // A multiple of 8: each prefix unit stays on the XCD whose suffix
        // workgroups (same heads) merge its slots, from that XCD's L2.
        wg -= P.copy_units;
    }

    const int tid = threadIdx.x;
    // the wave index is uniform: taken as a scalar, the row bounds and tests
    // derived from it stay on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
    const int g = lane / 16;  // lane group: owns dims [g*D/4, (g+1)*D/4) of K and Q
    const int c = lane % 16;  // this lane's query column of S^T (and token row of K)

    // ---- the tile of query rows and the token stream they share ----
    const uint32_t logical = xcd_remap(wg, P.total_units);
    const int tile = (int)(logical % (uint32_t)P.row_tiles);
    const uint32_t rest = logical / (uint32_t)P.row_tiles;
    int h, n_rows, stream_begin = 0, stream_end, lim0 = 0, part = 0;
    int64_t row0;  // q row (multi-query) or sequence (shared prefix) of tile row 0
    const int32_t* table;
    if constexpr (kCascade) {
        part = (int)(rest % (uint32_t)P.prefix_parts);  // prefix tokens [part*len, (part+1)*len)
        h = (int)(rest / (uint32_t)P.prefix_parts);
        row0 = (int64_t)tile * ROWS;
        n_rows = min(ROWS, P.num_seqs - (int)row0);
        stream_begin = part * P.prefix_part_len;
        stream_end = min(stream_begin + P.prefix_part_len, P.prefix_len);
        table = P.prefix_table;
    } else {
        h = (int)(rest % (uint32_t)P.num_heads);
        const int seq = (int)(rest / (uint32_t)P.num_heads);
        const int q0 = P.query_start[seq];
        const int n = P.query_start[seq + 1] - q0;
        const int r0 = tile * ROWS;
        if (r0 >= n)
            return;  // the whole workgroup, before any barrier
        n_rows = min(ROWS, n - r0);
        row0 = q0 + r0;
        lim0 = P.context_lens[seq] - n + r0 + 1;  // tile row r sees positions < lim0 + r
        stream_end = lim0 + n_rows - 1;
        table = P.block_tables + (int64_t)seq * P.max_blocks_per_seq;
    }

    // rows of this wave, their visibility limits (wave-uniform bounds)
    const int wr0 = wave * WROWS;
    const int wrows = max(0, min(WROWS, n_rows - wr0));
    const int wave_lo = kCascade ? stream_end : lim0 + wr0;              // smallest limit
    const int wave_hi = kCascade ? stream_end : lim0 + wr0 + wrows - 1;  // largest limit
    int lim[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
        lim[qt] = kCascade ? stream_end : lim0 + wr0 + 16 * qt + c;

    // Q^T as MFMA B operand: lane (query c) holds dims g*D/4 + 8i .. +7 for step i
    u32x4 qf[QT][KI];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int r = wr0 + 16 * qt + c;
        const u32x4* qp =
            reinterpret_cast<const u32x4*>(P.q + ((row0 + r) * P.num_heads + h) * D + g * (D / 4));
#pragma unroll
        for (int i = 0; i < KI; ++i)
            qf[qt][i] = r < n_rows ? qp[i] : u32x4{0, 0, 0, 0};
    }

    // O^T, the row sums (every element of lsum[qt] holds the sum of query c), and
    // the reference the exponentials are taken against (scaled, base 2)
    f4 o[QT][NB], lsum[QT];
    // m: the reference (-inf until a row has a finite score); m_ref: the shift
    // the scores take, m or 0 while m is unset; all_set (wave-uniform): no lane
    // of the wave has an unset reference
    float m[QT], m_ref[QT];
    bool all_set = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        m[qt] = kNegInf;
        m_ref[qt] = 0.0f;
        lsum[qt] = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
            o[qt][nb] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // all-ones A operand: ones * P^T sums the fp16 weights that P.V takes
    const h8 ones = h8{1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16, 1.0f16};

    const int64_t block_elems = (int64_t)B * P.num_heads * D;
    const int token_stride = P.num_heads * D;
    constexpr int EB = kFp8 ? 1 : 2;  // bytes per cache element
    const char* k_bytes = static_cast<const char*>(P.k_cache);
    const char* v_bytes = static_cast<const char*>(P.v_cache);

    // ---- fp16 caches: direct-to-LDS loads.  Wave w fills rows WR w .. WR w +
    // WR-1 of both tiles, RPI rows (1 KiB) per load: lane l of load j takes row
    // r = WR w + RPI j + l / DG and stored piece l % DG, i.e. source piece
    // (l % DG) ^ swz(r).  A chunk starts at a multiple of N tokens, so the rows
    // of a wave lie in one physical block, whose id is read once per wave and
    // chunk (one chunk ahead) and whose lane offsets do not change.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    uint32_t dk[DJ], dv[DJ];  // byte offsets of this lane's sources inside a block
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
        const int r = WR * wave + RPI * j + lane / DG;
        const uint32_t row = (uint32_t)((r % B) * token_stride + h * D) * 2u;
        dk[j] = row + (uint32_t)(((lane % DG) ^ swz_k<D>(r)) * 16);
        dv[j] = row + (uint32_t)(((lane % DG) ^ swz_v<D>(r)) * 16);
    }
    // the block of this wave's rows of the chunk at t0 (clamped into the stream;
    // a wave whose rows all lie past the stream end loads nothing).  A vector
    // read (the direct loads count as clobbers of global memory, so the compiler
    // will not make it a scalar one), issued before a chunk's direct loads and
    // made uniform only after the wait that lands them: taken earlier, it would
    // wait for every load issued before it.
    // (positions and block ids are never negative: unsigned arithmetic is one
    // shift and one 32 x 32 -> 64-bit product on the scalar unit)
    auto wave_block = [&](int t0) {
        return table[(uint32_t)min(t0 + WR * wave_u, stream_end - 1) / (uint32_t)B];
    };
    const uint32_t block_bytes = (uint32_t)block_elems * 2u;  // < 4 GiB: B * H * D * 2
    auto dma_chunk = [&](int t0, int b, int blk) {
        if (t0 + WR * wave_u >= stream_end)
            return;
        const uint64_t off = (uint64_t)(uint32_t)blk * block_bytes;
        const char* kb = k_bytes + off;
        const char* vb = v_bytes + off;
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
            load_lds16(kb, &k_lds[b][(WR * wave_u + RPI * j) * D], dk[j]);
            load_lds16(vb, &v_lds[b][(WR * wave_u + RPI * j) * D], dv[j]);
        }
    };
    // Rows past the stream end (in the last chunk) are zeroed once the direct
    // loads have landed: unread slots may hold anything, and P.V must not see
    // it (those positions are masked, but 0 * NaN is NaN).
    auto zero_tail = [&](int t0, int b) {
        if (t0 + WR * wave_u + WR <= stream_end)
            return;  // wave-uniform
#pragma unroll
        for (int k = 0; k < WR * DG / kWave; ++k) {
            const int piece = k * kWave + lane;  // of the wave's WR rows
            const int r = WR * wave_u + piece / DG;
            if (t0 + r >= stream_end) {
                *reinterpret_cast<u32x4*>(&k_lds[b][r * D + (piece % DG) * 8]) = u32x4{0, 0, 0, 0};
                *reinterpret_cast<u32x4*>(&v_lds[b][r * D + (piece % DG) * 8]) = u32x4{0, 0, 0, 0};
            }
        }
    };

    // ---- FP8 caches: each thread loads 4 tokens (4*lq .. 4*lq+3 of the chunk) x
    // 8 dims (8*lp ..) into registers and widens them to fp16 as it stores them
    const bool loader = UNITS == kMqThreads || tid < UNITS;  // a constant when all threads load
    const int lp = tid % DG, lq = tid / DG;
    typedef typename Raw8<kFp8>::type Raw;
    Raw kr[4], vr[4];  // (unused, and removed, for fp16 caches)
    // The physical block of this thread's four tokens of the chunk at t0 (one
    // block, as 4 divides B).  Loaded a chunk ahead of its K/V loads, so that
    // their addresses never wait on a table read.  The position is clamped
    // into the stream (the entry is then unused), so the read is always inside
    // the table and needs no select: a select would make the compiler drain
    // the loads in flight before overwriting the register.
    auto chunk_block = [&](int t0) {
        const int t = max(0, min(t0 + 4 * lq, stream_end - 1));
        return table[t / B];
    };
    auto load_chunk = [&](int t0, int blk) {
        const int t = t0 + 4 * lq;
        if (!loader)
            return;  // (only when D < 128: these threads stage nothing)
        const int64_t base = t < stream_end ? (int64_t)blk * block_elems +
                                                  (int64_t)(t % B) * token_stride + h * D + 8 * lp
                                            : 0;
        if (t + 4 <= stream_end) {  // all four tokens exist: no selects
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t e = (base + (int64_t)j * token_stride) * EB;
                kr[j] = *reinterpret_cast<const Raw*>(k_bytes + e);
                vr[j] = *reinterpret_cast<const Raw*>(v_bytes + e);
            }
        } else {  // the stream ends inside this group: zeros past the end
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const bool ok = t + j < stream_end;
                const int64_t e = (base + (int64_t)j * token_stride) * EB;
                kr[j] = ok ? *reinterpret_cast<const Raw*>(k_bytes + e) : Raw{};
                vr[j] = ok ? *reinterpret_cast<const Raw*>(v_bytes + e) : Raw{};
            }
        }
    };
    auto store_chunk = [&](int b) {
        if (!loader)
            return;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int r = 4 * lq + j;
            *reinterpret_cast<u32x4*>(&k_lds[b][r * D + (lp ^ swz_k<D>(r)) * 8]) = widen8(kr[j]);
            *reinterpret_cast<u32x4*>(&v_lds[b][r * D + (lp ^ swz_v<D>(r)) * 8]) = widen8(vr[j]);
        }
    };

    int next_blk;
    if constexpr (kFp8) {
        load_chunk(stream_begin, chunk_block(stream_begin));
        next_blk = chunk_block(stream_begin + N);
    } else {
        dma_chunk(stream_begin, 0, __builtin_amdgcn_readfirstlane(wave_block(stream_begin)));
        next_blk = wave_block(stream_begin + N);
    }
    // Wait for q here, once: inside the loop the compiler cannot prove these
    // loads complete on every path and would otherwise drain every load in
    // flight (the next chunk's prefetch included) before the first product.
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int i = 0; i < KI; ++i)
            asm volatile("" ::"v"(qf[qt][i]));

    // this lane's operand addresses in a tile (elements): K row 16s + c, pieces
    // g*KI + i; V^T rows 32kk + 16hh + 4g + c/4, dims 16nb + 4(c%4) .. +3 (the
    // swizzle of those rows does not depend on kk and hh)
    int koff[KI], voff[NB];
#pragma unroll
    for (int i = 0; i < KI; ++i)
        koff[i] = c * D + ((g * KI + i) ^ swz_k<D>(c)) * 8;
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
        voff[nb] = (4 * g + c / 4) * D + ((2 * nb + (c % 4) / 2) ^ swz_v<D>(4 * g + c / 4)) * 8 +
                   4 * (c % 2);

    // One chunk at t0 in LDS buffer b.  Called with a constant b from a loop
    // unrolled by two, so the buffer's base folds into the LDS instructions'
    // immediate offsets.
    auto step = [&](const int t0, const int b) __attribute__((always_inline)) {
        const _Float16* ks = k_lds[b];
        const _Float16* vs = v_lds[b];
        if constexpr (kFp8) {
            store_chunk(b);
            if (t0 + N < stream_end)
                load_chunk(t0 + N, next_blk);  // in flight during this chunk's math
            next_blk = chunk_block(t0 + 2 * N);  // unconditional, so no copy waits on it
        } else {
            __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);  // this wave's direct loads of the chunk landed
            if (t0 + N > stream_end)
                zero_tail(t0, b);
        }
        __syncthreads();
        if constexpr (!kFp8) {
            // the next chunk into the other buffer, which every wave is done with
            const int blk = __builtin_amdgcn_readfirstlane(next_blk);
            next_blk = wave_block(t0 + 2 * N);
            if (t0 + N < stream_end)
                dma_chunk(t0 + N, b ^ 1, blk);
        }

        if (wrows > 0 && t0 < wave_hi) {  // wave-uniform: some row of this wave sees the chunk
            // S^T[token 16s + 4g + j][query c] for the four 16-token subtiles
            f4 st[QT][N / 16];
#pragma unroll
            for (int s = 0; s < N / 16; ++s) {
                u32x4 ka[KI];
#pragma unroll
                for (int i = 0; i < KI; ++i)
                    ka[i] = *reinterpret_cast<const u32x4*>(&ks[16 * s * D + koff[i]]);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) {
                    f4 acc = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int i = 0; i < KI; ++i)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(as_h8(ka[i]), as_h8(qf[qt][i]),
                                                                     acc, 0, 0, 0);
                    st[qt][s] = acc;
                }
            }

            // positions at or past a row's limit: -inf (only in chunks that
            // cross some row's limit; a wave-uniform branch)
            if (t0 + N > wave_lo) {
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) {
                    const int nvis = lim[qt] - t0 - 4 * g;  // visible offsets 16s + j < nvis
#pragma unroll
                    for (int s = 0; s < N / 16; ++s)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            if (16 * s + j >= nvis)
                                st[qt][s][j] = kNegInf;
                }
            }

            // Online softmax per query column, against a lazy reference m (scaled,
            // base 2): the exponentials are taken against m, which moves (and O and
            // the row sums are rescaled) only when a chunk's max passes it by more
            // than kLazyRescale, so every weight stays below 2^kLazyRescale, far
            // inside fp16; the result is the same softmax, since O and l share the
            // reference.  The scores are shifted against the current reference
            // first; only when some shifted score in the wave passes the threshold,
            // or a reference is not yet set, are the row maxima formed and the
            // reference moved (the shift then corrected) -- the same decisions as
            // forming every chunk's max, at none of its cost in the usual chunk.
            float tmax[N / 16];  // partial maxima, independent chains
#pragma unroll
            for (int s = 0; s < N / 16; ++s)
                tmax[s] = kNegInf;
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
                for (int s = 0; s < N / 16; ++s)
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        // scale > 0: the shifted scores keep the order of the raw ones
                        st[qt][s][j] = __builtin_fmaf(st[qt][s][j], P.scale_log2, -m_ref[qt]);
                        tmax[s] = fmaxf(tmax[s], st[qt][s][j]);
                    }
            }
#pragma unroll
            for (int s = 1; s < N / 16; ++s)
                tmax[0] = fmaxf(tmax[0], tmax[s]);
            if (!all_set || __builtin_amdgcn_ballot_w64(tmax[0] > kLazyRescale) != 0) {
                bool moved = false, unset = false;
                float alpha[QT];
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) {
                    float bmax = kNegInf;
#pragma unroll
                    for (int s = 0; s < N / 16; ++s)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            bmax = fmaxf(bmax, st[qt][s][j]);
                    const float cm = group_max(bmax) + m_ref[qt];  // -inf stays -inf
                    const bool up = cm > m[qt] + kLazyRescale;    // any finite cm while m = -inf
                    const float m_new = up ? cm : m[qt];
                    const float ref_new = m_new == kNegInf ? 0.0f : m_new;
                    alpha[qt] = up ? exp2_fast(m[qt] - ref_new) : 1.0f;
                    moved |= up;
                    m[qt] = m_new;
                    unset |= m_new == kNegInf;
                    const float shift = ref_new - m_ref[qt];
                    m_ref[qt] = ref_new;
#pragma unroll
                    for (int s = 0; s < N / 16; ++s)
#pragma unroll
                        for (int j = 0; j < 4; ++j)
                            st[qt][s][j] -= shift;
                }
                all_set = __builtin_amdgcn_ballot_w64(unset) == 0;
                if (__builtin_amdgcn_ballot_w64(moved) != 0) {
#pragma unroll
                    for (int qt = 0; qt < QT; ++qt) {
                        lsum[qt] *= alpha[qt];
#pragma unroll
                        for (int nb = 0; nb < NB; ++nb)
                            o[qt][nb] *= alpha[qt];
                    }
                }
            }
            // The V^T operands of the first kPreV dim blocks (token step 0) are read
            // here, ahead of the exponentials they do not depend on, and the
            // scheduling barrier keeps them here (the scheduler otherwise sinks
            // every operand read to just before its products, where the wave then
            // waits on it): 0.7% on the multi-query workload.
            constexpr int kPreV = NB < 2 ? NB : 2;
            h8 va_pre[kPreV];
#pragma unroll
            for (int nb = 0; nb < kPreV; ++nb)
                va_pre[nb] = read_vt<D>(vs, voff[nb]);
            __builtin_amdgcn_sched_barrier(0);

            // the weights, rounded to fp16 as P^T, the B operand of the next products
            h8 pb[QT][N / 32];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                for (int s = 0; s < N / 16; ++s)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        pb[qt][s / 2][4 * (s % 2) + j] = (_Float16)exp2_fast(st[qt][s][j]);

            // Row sums: ones * P^T over the chunk's tokens, the fp16 weights that
            // P.V takes summed in fp32 (numerator and denominator share them).
#pragma unroll
            for (int kk = 0; kk < N / 32; ++kk)
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    lsum[qt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pb[qt][kk], lsum[qt], 0, 0, 0);

            // O^T[dim 16nb + 4g + j][query c] += V^T P^T over the chunk's 64 tokens.
            // B element 4*(s%2)+j of step kk is token 32kk + 16(s%2) + 4g + j; the
            // A operand takes the same tokens of dim 16nb + c, read with the
            // transposing LDS load: in each 16-lane group, lane i gets element
            // i%4 of the 8 bytes addressed by lane 4e + i/4 as its element e, so
            // lane (c, g) addresses token 32kk + 16h + 4g + c/4, dims
            // 16nb + 4(c%4) .. +3, and receives 4 tokens of dim 16nb + c.
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
                for (int kk = 0; kk < N / 32; ++kk) {
                    const h8 va = kk == 0 && nb < kPreV ? va_pre[nb < kPreV ? nb : 0]
                                                        : read_vt<D>(vs + 32 * kk * D, voff[nb]);
#pragma unroll
                    for (int qt = 0; qt < QT; ++qt)
                        o[qt][nb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb[qt][kk], o[qt][nb],
                                                                           0, 0, 0);
                }
            }
        }
    };
    for (int t0 = stream_begin; t0 < stream_end; t0 += 2 * N) {
        step(t0, 0);
        if (t0 + N < stream_end)
            step(t0 + N, 1);
    }

    // ---- O^T[dim 16nb + 4g + j][query c] / l(query c) ----
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const float l = lsum[qt][0];
        const int r = wr0 + 16 * qt + c;
        if (r >= n_rows)
            continue;
        if constexpr (kCascade) {
            // The normalised row in fp16 (half the bytes of fp32 to write here
            // and to read in the merge), without the FP8 V scale: the readers
            // apply it, so the stored values stay within the cache's code range.
            const float inv = l > 0.0f ? 1.0f / l : 0.0f;
            const int64_t u = ((row0 + r) * P.num_heads + h) * P.num_slots + part;
            _Float16* orow = P.ws_o + u * D;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                typedef _Float16 h4 __attribute__((ext_vector_type(4)));
                h4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = (_Float16)(o[qt][nb][j] * inv);
                *reinterpret_cast<h4*>(&orow[nb * 16 + 4 * g]) = v;
            }
            if (g == 0) {
                P.ws_m[u] = m[qt];
                P.ws_l[u] = l;
            }
        } else {
            // FP8: the V scale (the K scale is in scale_log2)
            const float inv = (l > 0.0f ? 1.0f / l : 0.0f) * (kFp8 ? P.v_scale : 1.0f);
            _Float16* orow = P.out + ((row0 + r) * P.num_heads + h) * D;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
                typedef _Float16 h4 __attribute__((ext_vector_type(4)));
                h4 v;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = (_Float16)(o[qt][nb][j] * inv);
                *reinterpret_cast<h4*>(&orow[nb * 16 + 4 * g]) = v;
            }
        }
    }
}

template <bool kCascade, bool kFp8>
hipError_t launch_mq(const MqParams& P, int head_dim, int block_size, hipStream_t stream)
{
    constexpr int QT = (kCascade ? kCascadeTileRows : kMqTileRows) / (kWaves * 16);
    // shared prefix: the copy workgroups, the prefix units, the ordering workgroup
    const dim3 grid(P.total_units + (kCascade ? 1u + P.copy_units : 0u)), block(kMqThreads);
    if (head_dim == 128 && block_size == 16)
        hipLaunchKernelGGL((pa_mq_kernel<128, 16, kCascade, QT, kFp8>), grid, block, 0, stream, P);
    else if (head_dim == 128 && block_size == 32)
        hipLaunchKernelGGL((pa_mq_kernel<128, 32, kCascade, QT, kFp8>), grid, block, 0, stream, P);
    else if (head_dim == 64 && block_size == 16)
        hipLaunchKernelGGL((pa_mq_kernel<64, 16, kCascade, QT, kFp8>), grid, block, 0, stream, P);
    else if (head_dim == 64 && block_size == 32)
        hipLaunchKernelGGL((pa_mq_kernel<64, 32, kCascade, QT, kFp8>), grid, block, 0, stream, P);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

hipError_t launch_multiquery(const MqParams& p, int head_dim, int block_size, hipStream_t stream)
{
    return launch_mq<false, false>(p, head_dim, block_size, stream);
}

hipError_t launch_multiquery_fp8(const MqParams& p, int head_dim, int block_size,
                                 hipStream_t stream)
{
    return launch_mq<false, true>(p, head_dim, block_size, stream);
}

hipError_t launch_cascade_prefix(const MqParams& p, int head_dim, int block_size,
                                 hipStream_t stream)
{
    return launch_mq<true, false>(p, head_dim, block_size, stream);
}

hipError_t launch_cascade_prefix_fp8(const MqParams& p, int head_dim, int block_size,
                                     hipStream_t stream)
{
    return launch_mq<true, true>(p, head_dim, block_size, stream);
}

}  // namespace pa
