// Internal launch interface between the C ABI layer and the kernels.
#ifndef PA_INTERNAL_H_
#define PA_INTERNAL_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

struct DecodeParams {
    _Float16* out;
    const _Float16* q;
    const void* k_cache;     // fp16 or FP8 codes, [NB, B, H, D]
    const void* v_cache;
    const int32_t* block_tables;
    const int32_t* context_lens;
    _Float16* ws_o;  // [S, H, NP, D] normalised partition rows in fp16, before any FP8 V scale
    float* ws_m;  // [S, H, NP] partition maxima (base-2 logits)
    float* ws_l;  // [S, H, NP] partition sums
    int32_t num_seqs;
    int32_t num_heads;
    int32_t max_blocks_per_seq;
    int32_t partition_size;  // tokens per partition (the whole table when not split)
    int32_t num_partitions;  // NP = ceil(max_blocks_per_seq * block_size / partition_size)
    uint32_t total_units;    // num_seqs * num_heads * num_partitions workgroups
    float scale_log2;        // scale * log2(e) (times the K scale for FP8)
    float v_scale;           // FP8: dequantisation scale of V (unused for fp16)
    int32_t slot_base;       // first workspace slot of partition 0 (1 when a shared-prefix
                             // partial occupies slot 0; partials are then always written)
    int32_t num_slots;       // workspace slots per (sequence, head) = slot_base + num_partitions
    // shared-prefix decode: the order in which the workgroups take the
    // sequences (ids by descending suffix length, and those lengths), written
    // by the prefix pass; nullptr: sequence order, lengths from context_lens
    const int32_t* seq_order;
    const int32_t* seq_order_len;
};

// Several query rows against one K/V token stream (multi-query / shared prefix).
constexpr int kMqThreads = 256;       // threads per workgroup (4 waves)
constexpr int kMqChunk = 64;          // tokens staged in LDS per step
constexpr int kMqTileRows = 128;      // multi-query rows per workgroup (32 per wave)
constexpr int kCascadeTileRows = 64;  // shared-prefix sequences per workgroup

struct MqParams {
    _Float16* out;                 // multi-query: final rows [T, H, D]
    _Float16* ws_o;                // shared prefix: partial rows (fp16, before any FP8 V scale)
                                   // in slots 0..parts-1 of each (s, h)
    float* ws_m;
    float* ws_l;
    const _Float16* q;             // multi-query: [T, H, D]; shared prefix: [S, H, D]
    const void* k_cache;           // fp16, or FP8 codes (the _fp8 launches)
    const void* v_cache;
    const int32_t* block_tables;   // multi-query: [S, MB]
    const int32_t* context_lens;   // multi-query: [S] (including the new tokens)
    const int32_t* query_start;    // multi-query: [S + 1]
    const int32_t* prefix_table;   // shared prefix: the prefix's physical blocks
    int32_t num_seqs;
    int32_t num_heads;
    int32_t max_blocks_per_seq;
    int32_t row_tiles;             // tiles of query rows per stream: multi-query
                                   // ceil(max query rows / kMqTileRows), shared prefix
                                   // ceil(num_seqs / kCascadeTileRows)
    int32_t prefix_len;            // shared prefix: tokens in the prefix
    int32_t prefix_part_len;       // shared prefix: tokens per prefix partition (multiple of kMqChunk)
    int32_t prefix_parts;          // shared prefix: partitions = workspace slots 0..parts-1
    int32_t num_slots;             // shared prefix: workspace slots per (s, h)
    uint32_t total_units;          // workgroups of query-row tiles
    float scale_log2;              // scale * log2(e) (times the K scale for FP8)
    float v_scale;                 // FP8: dequantisation scale of V
    uint32_t copy_units;           // shared prefix, appending form: copy workgroups first
    // shared prefix, appending form (new_k == nullptr otherwise): row s of
    // new_k / new_v [S, H, D] (fp16) goes to cache slot slot_mapping[s] when
    // 0 <= slot < cache_slots (a private suffix slot, never a prefix block);
    // FP8 caches get the codes E4M3(x * k_inv) / E4M3(x * v_inv)
    const _Float16* new_k;
    const _Float16* new_v;
    void* k_store;                 // the caches again, written through these
    void* v_store;
    const int64_t* slot_mapping;
    int64_t cache_slots;           // num_blocks * block_size
    float k_inv, v_inv;            // FP8: 1 / scale, rounded to float
    // shared prefix: workgroup 0 orders the sequences for the suffix launch,
    // by descending suffix_lens[s] clamped to [0, order_max_len]
    const int32_t* suffix_lens;
    int32_t order_max_len;         // max_blocks_per_seq * block_size of the suffix tables
    int32_t* seq_order;            // [S] sequence ids
    int32_t* seq_order_len;        // [S] their suffix_lens, as read
};

hipError_t launch_multiquery(const MqParams& p, int head_dim, int block_size, hipStream_t stream);
hipError_t launch_multiquery_fp8(const MqParams& p, int head_dim, int block_size,
                                 hipStream_t stream);
// extra workgroups of the appending shared-prefix pass (0 unless p.new_k)
int64_t copy_workgroups(const MqParams& p, int head_dim);
hipError_t launch_cascade_prefix(const MqParams& p, int head_dim, int block_size,
                                 hipStream_t stream);
hipError_t launch_cascade_prefix_fp8(const MqParams& p, int head_dim, int block_size,
                                     hipStream_t stream);

// partition kernel + (if num_slots > 1) the log-sum-exp reduce
hipError_t launch_decode_dispatch(const DecodeParams& p, int head_dim, int block_size,
                                  hipStream_t stream);
// the two halves of launch_decode_dispatch (fp16 cache), for callers that
// order other work between them
hipError_t launch_decode_partitions(const DecodeParams& p, int head_dim, int block_size,
                                    hipStream_t stream);
hipError_t launch_decode_reduce(const DecodeParams& p, int head_dim, hipStream_t stream);

hipError_t launch_decode_fp8_dispatch(const DecodeParams& p, int head_dim, int block_size,
                                      hipStream_t stream);

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                        void* v_cache, const int64_t* slot_mapping,
                                        int32_t num_tokens, int64_t num_slots, int32_t row_elems,
                                        float k_inv_scale, float v_inv_scale, hipStream_t stream);

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping, int32_t num_tokens,
                                    int64_t num_slots, int32_t row_vectors, hipStream_t stream);

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                              int32_t num_pairs, int64_t num_blocks, int64_t block_vecs,
                              hipStream_t stream);

hipError_t enqueue_swap_blocks(const void* src, void* dst, const int64_t* block_mapping,
                               int32_t num_pairs, int64_t block_bytes, hipStream_t stream);

}  // namespace pa

#endif  // PA_INTERNAL_H_
