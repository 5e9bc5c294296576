// C ABI of the paged-attention decode library: host-side argument checks,
// workspace sizing and launches on the caller's stream.  The semantics of
// every entry point are documented with its declaration in pa.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>

#include "pa.h"
#include "pa_internal.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// A launch is at most 2^32 - 1 work-items: a grid of `workgroups` workgroups
// of 256 threads fits.
bool grid_fits(int64_t workgroups) { return workgroups <= (int64_t)(UINT32_MAX / 256); }

// The kernels address a token row and a physical block of one cache with
// 32-bit byte offsets: B * H * D * 2 (fp16) must fit.
bool block_fits(int32_t block_size, int32_t num_heads, int32_t head_dim)
{
    return (int64_t)block_size * num_heads * head_dim * 2 <= INT32_MAX;
}

// Number of context partitions the grid covers, or -1 for bad arguments.
int64_t num_partitions(int32_t block_size, int32_t max_blocks_per_seq, int32_t partition_size)
{
    const int64_t max_tokens = (int64_t)max_blocks_per_seq * block_size;
    if (partition_size == 0)
        return 1;
    return (max_tokens + partition_size - 1) / partition_size;
}

bool supported_decode(int32_t head_dim, int32_t block_size)
{
    return (head_dim == 64 || head_dim == 128) && (block_size == 16 || block_size == 32);
}

struct WorkspaceLayout {
    size_t o_bytes, m_bytes, l_bytes, total;
};

size_t round256(size_t b) { return (b + 255) & ~size_t(255); }

WorkspaceLayout layout(int64_t units, int32_t head_dim)
{
    WorkspaceLayout w;
    w.o_bytes = round256((size_t)units * head_dim * sizeof(_Float16));  // fp16 rows
    w.m_bytes = round256((size_t)units * sizeof(float));
    w.l_bytes = round256((size_t)units * sizeof(float));
    w.total = w.o_bytes + w.m_bytes + w.l_bytes;
    return w;
}

}  // namespace

extern "C" {

const char* pa_status_string(int status)
{
    switch (status) {
    case PA_OK: return "PA_OK: success";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_INVALID_DIM: return "PA_ERR_INVALID_DIM: a size is out of range";
    case PA_ERR_UNSUPPORTED:
        return "PA_ERR_UNSUPPORTED: head_dim must be 64 or 128 and block_size 16 or 32";
    case PA_ERR_PARTITION:
        return "PA_ERR_PARTITION: partition_size must be 0 or a positive multiple of block_size";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: a base pointer is not 16-byte aligned";
    case PA_ERR_HIP: return "PA_ERR_HIP: the HIP runtime reported a launch error";
    case PA_ERR_RANGE: return "PA_ERR_RANGE: a block index is outside its cache";
    case PA_ERR_SCRATCH:
        return "PA_ERR_SCRATCH: the split-context partials need more than the "
               "PA_NOALLOC_SCRATCH_BYTES (32 MiB) of pa_decode_noalloc's static scratch";
    default: return "unknown pa status";
    }
}

int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_heads,
                         int32_t head_dim, int32_t num_blocks, int32_t block_size, void* stream)
{
    if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || num_blocks <= 0 || block_size <= 0)
        return PA_ERR_INVALID_DIM;
    if (head_dim % 8 != 0)
        return PA_ERR_UNSUPPORTED;
    if ((int64_t)num_heads * head_dim / 8 > INT32_MAX)
        return PA_ERR_INVALID_DIM;
    if (num_tokens == 0)
        return PA_OK;
    if (!grid_fits(num_tokens))  // one workgroup per token
        return PA_ERR_INVALID_DIM;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping)
        return PA_ERR_NULL;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
        return PA_ERR_ALIGN;
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    const int32_t row_vectors = num_heads * head_dim / 8;
    hipError_t e = pa::launch_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping,
                                                num_tokens, num_slots, row_vectors,
                                                static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t partition_size)
{
    if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
        max_blocks_per_seq <= 0 || partition_size < 0)
        return 0;
    if (partition_size % block_size != 0)
        return 0;
    const int64_t np = num_partitions(block_size, max_blocks_per_seq, partition_size);
    if (np <= 1)
        return 0;
    return layout((int64_t)num_seqs * num_heads * np, head_dim).total;
}

namespace {

// Shared checks and parameter set-up of pa_decode, pa_decode_fp8 and the
// suffix part of pa_decode_cascade (extra_slots = 1 there: slot 0 of every
// (sequence, head) holds the shared-prefix partial).
int prepare_decode(pa::DecodeParams& p, void* out, const void* q, const void* k_cache,
                   const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                   int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                   int32_t block_size, int32_t max_blocks_per_seq, float scale,
                   int32_t partition_size, void* workspace, size_t workspace_bytes,
                   int32_t extra_slots = 0)
{
    if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || num_blocks <= 0 || block_size <= 0 ||
        max_blocks_per_seq <= 0)
        return PA_ERR_INVALID_DIM;
    if (!supported_decode(head_dim, block_size))
        return PA_ERR_UNSUPPORTED;
    if ((int64_t)max_blocks_per_seq * block_size > INT32_MAX || !block_fits(block_size, num_heads, head_dim))
        return PA_ERR_INVALID_DIM;
    if (partition_size < 0 || partition_size % block_size != 0)
        return PA_ERR_PARTITION;
    if (!std::isfinite(scale))
        return PA_ERR_INVALID_DIM;
    if (num_seqs == 0)
        return 1;  // nothing to enqueue
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens)
        return PA_ERR_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
        (reinterpret_cast<uintptr_t>(context_lens) & 3u))
        return PA_ERR_ALIGN;

    const int64_t np = num_partitions(block_size, max_blocks_per_seq, partition_size);
    const int64_t units = (int64_t)num_seqs * num_heads * np;
    const int64_t slots = np + extra_slots;
    if (units > INT32_MAX || (int64_t)num_seqs * num_heads * slots > INT32_MAX)
        return PA_ERR_INVALID_DIM;
    if (!grid_fits(units))
        return PA_ERR_INVALID_DIM;

    p = pa::DecodeParams{};
    p.out = static_cast<_Float16*>(out);
    p.q = static_cast<const _Float16*>(q);
    p.k_cache = k_cache;
    p.v_cache = v_cache;
    p.block_tables = block_tables;
    p.context_lens = context_lens;
    p.num_seqs = num_seqs;
    p.num_heads = num_heads;
    p.max_blocks_per_seq = max_blocks_per_seq;
    p.partition_size = np == 1 ? max_blocks_per_seq * block_size : partition_size;
    p.num_partitions = (int32_t)np;
    p.total_units = (uint32_t)units;
    p.scale_log2 = (float)((double)scale * 1.4426950408889634074);  // log2(e)
    p.v_scale = 1.0f;
    p.slot_base = extra_slots;
    p.num_slots = (int32_t)slots;
    if (slots > 1) {
        const WorkspaceLayout w = layout((int64_t)num_seqs * num_heads * slots, head_dim);
        if (!workspace || workspace_bytes < w.total)
            return PA_ERR_WORKSPACE;
        if (!aligned16(workspace))
            return PA_ERR_ALIGN;
        char* base = static_cast<char*>(workspace);
        p.ws_o = reinterpret_cast<_Float16*>(base);
        p.ws_m = reinterpret_cast<float*>(base + w.o_bytes);
        p.ws_l = reinterpret_cast<float*>(base + w.o_bytes + w.m_bytes);
    }
    return PA_OK;
}

bool valid_scale(float s) { return std::isfinite(s) && s > 0.0f; }

}  // namespace

namespace {
constexpr int32_t kPrefixPartLen = 2 * pa::kMqChunk;  // shared-prefix tokens per workgroup

int32_t prefix_parts(int32_t prefix_len) { return (prefix_len + kPrefixPartLen - 1) / kPrefixPartLen; }

// After the partials: the suffix launch's sequence order, ids then lengths
size_t order_bytes(int32_t num_seqs) { return round256((size_t)num_seqs * 2 * sizeof(int32_t)); }

}  // namespace

size_t pa_decode_cascade_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t block_size, int32_t prefix_len,
                                        int32_t max_blocks_per_seq, int32_t partition_size)
{
    if (num_seqs < 0 || num_heads <= 0 || head_dim <= 0 || block_size <= 0 || prefix_len < 0 ||
        max_blocks_per_seq <= 0 || partition_size < 0 || partition_size % block_size != 0)
        return 0;
    if (prefix_len == 0)
        return pa_decode_workspace_size(num_seqs, num_heads, head_dim, block_size,
                                        max_blocks_per_seq, partition_size);
    const int64_t slots =
        prefix_parts(prefix_len) + num_partitions(block_size, max_blocks_per_seq, partition_size);
    return layout((int64_t)num_seqs * num_heads * slots, head_dim).total + order_bytes(num_seqs);
}

namespace {

// FP8 caches: the dequantisation scales of K and V
struct Fp8Scales {
    float k, v;
};

// pa_decode_cascade; pa_decode_cascade_append when append; the _fp8 forms
// of both when fp8 != nullptr
int cascade(void* out, const void* q, const void* key, const void* value, void* k_cache,
            void* v_cache, const int64_t* slot_mapping, const int32_t* prefix_block_table,
            int32_t prefix_len, const int32_t* block_tables, const int32_t* context_lens,
            int32_t num_seqs, int32_t num_heads, int32_t head_dim, int32_t num_blocks,
            int32_t block_size, int32_t max_blocks_per_seq, float scale, int32_t partition_size,
            void* workspace, size_t workspace_bytes, void* stream, bool append,
            const Fp8Scales* fp8 = nullptr)
{
    if (prefix_len < 0 || (block_size > 0 && prefix_len % block_size != 0))
        return PA_ERR_INVALID_DIM;
    if (!(std::isfinite(scale) && scale > 0.0f))
        return PA_ERR_INVALID_DIM;
    if (fp8 && (!valid_scale(fp8->k) || !valid_scale(fp8->v)))
        return PA_ERR_INVALID_DIM;
    if (append && (!key || !value || !slot_mapping) && num_seqs > 0)
        return PA_ERR_NULL;
    if (append && num_seqs > 0 &&
        (!aligned16(key) || !aligned16(value) || (reinterpret_cast<uintptr_t>(slot_mapping) & 7u)))
        return PA_ERR_ALIGN;
    if (prefix_len == 0) {  // nothing shared: the plain step (its own write, then the decode)
        if (!append)
            return fp8 ? pa_decode_fp8(out, q, k_cache, v_cache, block_tables, context_lens,
                                       num_seqs, num_heads, head_dim, num_blocks, block_size,
                                       max_blocks_per_seq, scale, fp8->k, fp8->v,
                                       partition_size, workspace, workspace_bytes, stream)
                       : pa_decode(out, q, k_cache, v_cache, block_tables, context_lens,
                                   num_seqs, num_heads, head_dim, num_blocks, block_size,
                                   max_blocks_per_seq, scale, partition_size, workspace,
                                   workspace_bytes, stream);
        pa::DecodeParams p;  // every decode check before the write is enqueued
        int rc = prepare_decode(p, out, q, k_cache, v_cache, block_tables, context_lens,
                                num_seqs, num_heads, head_dim, num_blocks, block_size,
                                max_blocks_per_seq, scale, partition_size, workspace,
                                workspace_bytes);
        if (rc != PA_OK)
            return rc == 1 ? PA_OK : rc;
        if (fp8) {
            p.scale_log2 = (float)((double)scale * (double)fp8->k * 1.4426950408889634074);
            p.v_scale = fp8->v;
        }
        rc = fp8 ? pa_reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping,
                                            num_seqs, num_heads, head_dim, num_blocks,
                                            block_size, fp8->k, fp8->v, stream)
                 : pa_reshape_and_cache(key, value, k_cache, v_cache, slot_mapping, num_seqs,
                                        num_heads, head_dim, num_blocks, block_size, stream);
        if (rc != PA_OK)
            return rc;  // its checks fail before it enqueues anything
        hipError_t e = fp8 ? pa::launch_decode_fp8_dispatch(p, head_dim, block_size,
                                                             static_cast<hipStream_t>(stream))
                           : pa::launch_decode_dispatch(p, head_dim, block_size,
                                                        static_cast<hipStream_t>(stream));
        return e == hipSuccess ? PA_OK : PA_ERR_HIP;
    }
    if (head_dim != 64 && head_dim != 128)
        return PA_ERR_UNSUPPORTED;
    pa::DecodeParams p;
    const int32_t parts = prefix_parts(prefix_len);
    int rc = prepare_decode(p, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                            num_heads, head_dim, num_blocks, block_size, max_blocks_per_seq, scale,
                            partition_size, workspace, workspace_bytes, /*extra_slots=*/parts);
    if (rc != PA_OK)
        return rc == 1 ? PA_OK : rc;
    if (!prefix_block_table)
        return PA_ERR_NULL;
    const size_t partial_bytes =
        layout((int64_t)num_seqs * num_heads * p.num_slots, head_dim).total;
    if (workspace_bytes < partial_bytes + order_bytes(num_seqs))
        return PA_ERR_WORKSPACE;
    int32_t* order = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + partial_bytes);
    p.seq_order = order;
    p.seq_order_len = order + num_seqs;
    if (fp8) {  // the K scale folds into the logit scale, the V scale into the rows
        p.scale_log2 = (float)((double)scale * (double)fp8->k * 1.4426950408889634074);
        p.v_scale = fp8->v;
    }
    const int64_t row_tiles = ((int64_t)num_seqs + pa::kCascadeTileRows - 1) / pa::kCascadeTileRows;
    if (row_tiles * num_heads * parts > INT32_MAX || !grid_fits(row_tiles * num_heads * parts + 1))
        return PA_ERR_INVALID_DIM;
    pa::MqParams m{};
    m.ws_o = p.ws_o;
    m.ws_m = p.ws_m;
    m.ws_l = p.ws_l;
    m.q = static_cast<const _Float16*>(q);
    m.k_cache = static_cast<const _Float16*>(k_cache);
    m.v_cache = static_cast<const _Float16*>(v_cache);
    m.prefix_table = prefix_block_table;
    m.num_seqs = num_seqs;
    m.num_heads = num_heads;
    m.prefix_len = prefix_len;
    m.prefix_part_len = kPrefixPartLen;
    m.prefix_parts = parts;
    m.num_slots = p.num_slots;
    m.row_tiles = (int32_t)row_tiles;
    m.total_units = (uint32_t)(row_tiles * parts * num_heads);
    m.scale_log2 = p.scale_log2;
    m.v_scale = p.v_scale;
    m.suffix_lens = context_lens;
    m.order_max_len = max_blocks_per_seq * block_size;  // fits int32 (prepare_decode)
    m.seq_order = order;
    m.seq_order_len = order + num_seqs;
    if (append) {  // the prefix pass also writes the new tokens (into private suffix slots)
        m.new_k = static_cast<const _Float16*>(key);
        m.new_v = static_cast<const _Float16*>(value);
        m.k_store = k_cache;
        m.v_store = v_cache;
        if (fp8) {  // the cache-write quantiser multiplies by 1/scale rounded to float
            m.k_inv = (float)(1.0 / (double)fp8->k);
            m.v_inv = (float)(1.0 / (double)fp8->v);
        }
        m.slot_mapping = slot_mapping;
        m.cache_slots = (int64_t)num_blocks * block_size;
        const int64_t copy_units = pa::copy_workgroups(m, head_dim);
        if (!grid_fits((int64_t)m.total_units + copy_units + 1))
            return PA_ERR_INVALID_DIM;
        m.copy_units = (uint32_t)copy_units;
    }
    // Prefix pass first (slots 0..parts-1, and the order in which the suffix
    // launch takes the sequences), then the suffix partitions; when
    // every suffix fits one partition the partition kernel merges the prefix
    // slots itself and writes the rows, else the reduce merges all slots.
    hipStream_t st = static_cast<hipStream_t>(stream);
    hipError_t e = fp8 ? pa::launch_cascade_prefix_fp8(m, head_dim, block_size, st)
                       : pa::launch_cascade_prefix(m, head_dim, block_size, st);
    if (e == hipSuccess)
        e = fp8 ? pa::launch_decode_fp8_dispatch(p, head_dim, block_size, st)
                : pa::launch_decode_dispatch(p, head_dim, block_size, st);
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

int pa_decode_cascade(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* prefix_block_table, int32_t prefix_len,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                      int32_t max_blocks_per_seq, float scale, int32_t partition_size,
                      void* workspace, size_t workspace_bytes, void* stream)
{
    return cascade(out, q, nullptr, nullptr, const_cast<void*>(k_cache),
                   const_cast<void*>(v_cache), nullptr, prefix_block_table, prefix_len,
                   block_tables, context_lens, num_seqs, num_heads, head_dim, num_blocks,
                   block_size, max_blocks_per_seq, scale, partition_size, workspace,
                   workspace_bytes, stream, /*append=*/false);
}

int pa_decode_cascade_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* prefix_block_table, int32_t prefix_len,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                          int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                          float scale, float k_scale, float v_scale, int32_t partition_size,
                          void* workspace, size_t workspace_bytes, void* stream)
{
    const Fp8Scales sc{k_scale, v_scale};
    return cascade(out, q, nullptr, nullptr, const_cast<void*>(k_cache),
                   const_cast<void*>(v_cache), nullptr, prefix_block_table, prefix_len,
                   block_tables, context_lens, num_seqs, num_heads, head_dim, num_blocks,
                   block_size, max_blocks_per_seq, scale, partition_size, workspace,
                   workspace_bytes, stream, /*append=*/false, &sc);
}

int pa_decode_cascade_append_fp8(void* out, const void* q, const void* key, const void* value,
                                 void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                 const int32_t* prefix_block_table, int32_t prefix_len,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t num_blocks, int32_t block_size,
                                 int32_t max_blocks_per_seq, float scale, float k_scale,
                                 float v_scale, int32_t partition_size, void* workspace,
                                 size_t workspace_bytes, void* stream)
{
    const Fp8Scales sc{k_scale, v_scale};
    return cascade(out, q, key, value, k_cache, v_cache, slot_mapping, prefix_block_table,
                   prefix_len, block_tables, context_lens, num_seqs, num_heads, head_dim,
                   num_blocks, block_size, max_blocks_per_seq, scale, partition_size, workspace,
                   workspace_bytes, stream, /*append=*/true, &sc);
}

int pa_decode_cascade_append(void* out, const void* q, const void* key, const void* value,
                             void* k_cache, void* v_cache, const int64_t* slot_mapping,
                             const int32_t* prefix_block_table, int32_t prefix_len,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                             int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                             float scale, int32_t partition_size, void* workspace,
                             size_t workspace_bytes, void* stream)
{
    return cascade(out, q, key, value, k_cache, v_cache, slot_mapping, prefix_block_table,
                   prefix_len, block_tables, context_lens, num_seqs, num_heads, head_dim,
                   num_blocks, block_size, max_blocks_per_seq, scale, partition_size, workspace,
                   workspace_bytes, stream, /*append=*/true);
}

namespace {

// pa_multi_query; pa_multi_query_fp8 when fp8 != nullptr
int multi_query(void* out, const void* q, const void* k_cache, const void* v_cache,
                const int32_t* block_tables, const int32_t* context_lens,
                const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                int32_t max_query_len, int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                int32_t block_size, int32_t max_blocks_per_seq, float scale, void* stream,
                const Fp8Scales* fp8)
{
    if (fp8 && (!valid_scale(fp8->k) || !valid_scale(fp8->v)))
        return PA_ERR_INVALID_DIM;
    if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || num_heads <= 0 || head_dim <= 0 ||
        num_blocks <= 0 || block_size <= 0 || max_blocks_per_seq <= 0)
        return PA_ERR_INVALID_DIM;
    if (!supported_decode(head_dim, block_size))
        return PA_ERR_UNSUPPORTED;
    if (!(std::isfinite(scale) && scale > 0.0f) ||
        (int64_t)max_blocks_per_seq * block_size > INT32_MAX || !block_fits(block_size, num_heads, head_dim))
        return PA_ERR_INVALID_DIM;
    if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0)
        return PA_OK;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start)
        return PA_ERR_NULL;
    if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(block_tables) & 3u) ||
        (reinterpret_cast<uintptr_t>(context_lens) & 3u) ||
        (reinterpret_cast<uintptr_t>(query_start) & 3u))
        return PA_ERR_ALIGN;
    const int64_t tiles = ((int64_t)max_query_len + pa::kMqTileRows - 1) / pa::kMqTileRows;
    const int64_t units = (int64_t)num_seqs * tiles * num_heads;
    if (units > INT32_MAX || !grid_fits(units))
        return PA_ERR_INVALID_DIM;
    pa::MqParams m{};
    m.out = static_cast<_Float16*>(out);
    m.q = static_cast<const _Float16*>(q);
    m.k_cache = static_cast<const _Float16*>(k_cache);
    m.v_cache = static_cast<const _Float16*>(v_cache);
    m.block_tables = block_tables;
    m.context_lens = context_lens;
    m.query_start = query_start;
    m.num_seqs = num_seqs;
    m.num_heads = num_heads;
    m.max_blocks_per_seq = max_blocks_per_seq;
    m.row_tiles = (int32_t)tiles;
    m.total_units = (uint32_t)units;
    m.scale_log2 = (float)((double)scale * (fp8 ? (double)fp8->k : 1.0) * 1.4426950408889634074);
    m.v_scale = fp8 ? fp8->v : 1.0f;
    hipError_t e = fp8 ? pa::launch_multiquery_fp8(m, head_dim, block_size,
                                                   static_cast<hipStream_t>(stream))
                       : pa::launch_multiquery(m, head_dim, block_size,
                                               static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

int pa_multi_query(void* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* context_lens,
                   const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                   int32_t max_query_len, int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                   int32_t block_size, int32_t max_blocks_per_seq, float scale, void* stream)
{
    return multi_query(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                       num_seqs, num_tokens, max_query_len, num_heads, head_dim, num_blocks,
                       block_size, max_blocks_per_seq, scale, stream, nullptr);
}

int pa_multi_query_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                       int32_t max_query_len, int32_t num_heads, int32_t head_dim,
                       int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                       float scale, float k_scale, float v_scale, void* stream)
{
    const Fp8Scales sc{k_scale, v_scale};
    return multi_query(out, q, k_cache, v_cache, block_tables, context_lens, query_start,
                       num_seqs, num_tokens, max_query_len, num_heads, head_dim, num_blocks,
                       block_size, max_blocks_per_seq, scale, stream, &sc);
}

int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
              int32_t max_blocks_per_seq, float scale, int32_t partition_size, void* workspace,
              size_t workspace_bytes, void* stream)
{
    pa::DecodeParams p;
    int rc = prepare_decode(p, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                            num_heads, head_dim, num_blocks, block_size, max_blocks_per_seq, scale,
                            partition_size, workspace, workspace_bytes);
    if (rc != PA_OK)
        return rc == 1 ? PA_OK : rc;
    hipError_t e = pa::launch_decode_dispatch(p, head_dim, block_size,
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

// ---- pa_decode_noalloc: the split partials in a static device array ----
namespace {

constexpr size_t kScratchBytes = PA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "whole 256-byte pieces");

// The partials of pa_decode_noalloc.  Each GPU holds its own copy of this
// array (from the first call on it until the process ends), at its own
// address: host code uses the address hipGetSymbolAddress returns with that
// device current, never the array's name (a host-side stand-in).
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device id

// Address of the current device's scratch, looked up once per device.
int current_scratch(void** ptr)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return PA_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p)
            return PA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                      int32_t max_blocks_per_seq, float scale, int32_t partition_size,
                      void* stream)
{
    // Every host check first, with no workspace: only the workspace check can
    // then fail, and only when the call splits.
    pa::DecodeParams p;
    int rc = prepare_decode(p, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                            num_heads, head_dim, num_blocks, block_size, max_blocks_per_seq,
                            scale, partition_size, nullptr, 0);
    if (rc == 1)
        return PA_OK;  // nothing to enqueue
    if (rc == PA_ERR_WORKSPACE) {
        const size_t need = pa_decode_workspace_size(num_seqs, num_heads, head_dim, block_size,
                                                     max_blocks_per_seq, partition_size);
        if (need > kScratchBytes)
            return PA_ERR_SCRATCH;
        void* ws = nullptr;
        rc = current_scratch(&ws);
        if (rc != PA_OK)
            return rc;
        rc = prepare_decode(p, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                            num_heads, head_dim, num_blocks, block_size, max_blocks_per_seq,
                            scale, partition_size, ws, kScratchBytes);
    }
    if (rc != PA_OK)
        return rc;
    hipError_t e = pa::launch_decode_dispatch(p, head_dim, block_size,
                                              static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                  int32_t max_blocks_per_seq, float scale, float k_scale, float v_scale,
                  int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream)
{
    if (!valid_scale(k_scale) || !valid_scale(v_scale))
        return PA_ERR_INVALID_DIM;
    pa::DecodeParams p;
    int rc = prepare_decode(p, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                            num_heads, head_dim, num_blocks, block_size, max_blocks_per_seq, scale,
                            partition_size, workspace, workspace_bytes);
    if (rc != PA_OK)
        return rc == 1 ? PA_OK : rc;
    p.scale_log2 = (float)((double)scale * (double)k_scale * 1.4426950408889634074);
    p.v_scale = v_scale;
    hipError_t e = pa::launch_decode_fp8_dispatch(p, head_dim, block_size,
                                                  static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, int32_t num_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t num_blocks, int32_t block_size,
                             float k_scale, float v_scale, void* stream)
{
    if (num_tokens < 0 || num_heads <= 0 || head_dim <= 0 || num_blocks <= 0 || block_size <= 0)
        return PA_ERR_INVALID_DIM;
    if (!valid_scale(k_scale) || !valid_scale(v_scale))
        return PA_ERR_INVALID_DIM;
    if (head_dim % 16 != 0)
        return PA_ERR_UNSUPPORTED;
    if ((int64_t)num_heads * head_dim > INT32_MAX)
        return PA_ERR_INVALID_DIM;
    if (num_tokens == 0)
        return PA_OK;
    if (!grid_fits(num_tokens))  // one workgroup per token
        return PA_ERR_INVALID_DIM;
    if (!key || !value || !k_cache || !v_cache || !slot_mapping)
        return PA_ERR_NULL;
    if (!aligned16(key) || !aligned16(value) || !aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(slot_mapping) & 7u))
        return PA_ERR_ALIGN;
    const int64_t num_slots = (int64_t)num_blocks * block_size;
    // the quantiser multiplies by 1/scale rounded to float
    const float k_inv = (float)(1.0 / (double)k_scale);
    const float v_inv = (float)(1.0 / (double)v_scale);
    hipError_t e = pa::launch_reshape_and_cache_fp8(key, value, k_cache, v_cache, slot_mapping,
                                                    num_tokens, num_slots, num_heads * head_dim,
                                                    k_inv, v_inv,
                                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int32_t num_pairs,
                   int32_t num_blocks, int32_t block_size, int32_t num_heads, int32_t head_dim,
                   void* stream)
{
    if (num_pairs < 0 || num_blocks <= 0 || block_size <= 0 || num_heads <= 0 || head_dim <= 0)
        return PA_ERR_INVALID_DIM;
    if (head_dim % 8 != 0)
        return PA_ERR_UNSUPPORTED;
    if (num_pairs == 0)
        return PA_OK;
    if (!k_cache || !v_cache || !block_mapping)
        return PA_ERR_NULL;
    if (!aligned16(k_cache) || !aligned16(v_cache) ||
        (reinterpret_cast<uintptr_t>(block_mapping) & 7u))
        return PA_ERR_ALIGN;
    const int64_t block_vecs = (int64_t)block_size * num_heads * head_dim / 8;
    const int64_t chunks = (block_vecs + 2047) / 2048;
    if ((int64_t)num_pairs * chunks > INT32_MAX || !grid_fits((int64_t)num_pairs * chunks))
        return PA_ERR_INVALID_DIM;
    hipError_t e = pa::launch_copy_blocks(k_cache, v_cache, block_mapping, num_pairs, num_blocks,
                                          block_vecs, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int pa_swap_blocks(const void* src, void* dst, const int64_t* block_mapping, int32_t num_pairs,
                   int32_t src_num_blocks, int32_t dst_num_blocks, int64_t block_bytes,
                   void* stream)
{
    if (num_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0 || block_bytes <= 0)
        return PA_ERR_INVALID_DIM;
    if (num_pairs == 0)
        return PA_OK;
    if (!src || !dst || !block_mapping)
        return PA_ERR_NULL;
    for (int32_t i = 0; i < num_pairs; ++i) {
        const int64_t a = block_mapping[2 * i], b = block_mapping[2 * i + 1];
        if (a < 0 || a >= src_num_blocks || b < 0 || b >= dst_num_blocks)
            return PA_ERR_RANGE;
    }
    hipError_t e = pa::enqueue_swap_blocks(src, dst, block_mapping, num_pairs, block_bytes,
                                           static_cast<hipStream_t>(stream));
    return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
