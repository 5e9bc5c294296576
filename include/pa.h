/*
 * pa.h — C ABI of the paged-attention decode library for AMD Instinct
 * MI355X (gfx950).
 *
 * Sources (web pages), cited by title and section:
 *   [10x]  "vLLM推理加速深度解读：PagedAttention如何提升10x吞吐量"
 *          §2.1 attention equation; §2.3 paged attention equations and the
 *          gather K_paged[i] = K_physical[BlockTable[i / B]][i mod B];
 *          §4.2 cache layout [num_blocks, block_size, num_heads, head_size];
 *          §3.3 FP8 quantisation (named only); §4.3 prefill and decode work
 *          in one batch; §4.4 requests sharing a prefix reuse its blocks
 *   [eng]  "深入解析LLM推理引擎：从PagedAttention到调度优化"
 *          §3.2 on-demand block filling, the block table, shared prefix
 *          blocks; §3.3 the gather driven by block_table and the current
 *          position; §4.2 batches that mix prefill and decode requests
 *   [arch] "vLLM基础架构：核心组件、PagedAttention原理、KV Cache管理与连续批处理机制"
 *          §2.3 a new block every block_size tokens; shared prefix blocks;
 *          copy-on-write of a shared block before a sequence writes into it
 *   [src]  "【硬核】啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密"
 *          §三 blocks swapped out to host memory and back in
 *
 * Conventions shared by every entry point
 *   - Every array pointer is a DEVICE pointer owned by the caller, except
 *     where an entry point says otherwise (pa_swap_blocks).  The library
 *     never allocates, frees or synchronises; it keeps no state between
 *     calls.  Work is enqueued on `stream` (a hipStream_t passed as
 *     void*, NULL = the null stream) and runs asynchronously in stream order.
 *   - fp16 means IEEE-754 binary16.  All arrays are dense, row-major, and
 *     their base pointers are 16-byte aligned.
 *   - K/V cache layout [num_blocks, block_size, num_heads, head_dim] ([10x]
 *     §4.2), K and V in separate arrays.  A slot is
 *     physical_block * block_size + offset_in_block.
 *   - Return value: PA_OK (0) or a negative PA_ERR_* code.  Arguments are
 *     checked on the host before anything is enqueued; a failed check
 *     enqueues nothing.  Values that live on the device (block ids, context
 *     lengths, slots) are preconditions and are not checked, since checking
 *     them would need a synchronisation.
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    PA_OK = 0,
    PA_ERR_NULL = -1,        /* a required pointer is NULL                          */
    PA_ERR_INVALID_DIM = -2, /* a size is <= 0 (num_tokens/num_seqs < 0) or overflows:
                                the grid, or (decode, cascade, multi-query) a physical
                                block of block_size * num_heads * head_dim * 2 bytes
                                past INT32_MAX                                        */
    PA_ERR_UNSUPPORTED = -3, /* head_dim or block_size not compiled in               */
    PA_ERR_PARTITION = -4,   /* partition_size not 0 and not a positive multiple of block_size */
    PA_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than pa_decode_workspace_size */
    PA_ERR_ALIGN = -6,       /* a base pointer is not 16-byte aligned                */
    PA_ERR_HIP = -7,         /* the HIP runtime reported an error at launch          */
    PA_ERR_RANGE = -8,       /* a host-side block index is outside its cache          */
    PA_ERR_SCRATCH = -9      /* pa_decode_noalloc: partials exceed its static scratch  */
};

/*
 * Write this step's new keys and values into their cache slots.
 *
 * The block manager gives the token at logical position p of a sequence the
 * slot BlockTable[p / block_size] * block_size + p % block_size ([10x] §2.3
 * gather equation read as a write; [eng] §3.2 and [arch] §2.3: a block fills
 * position by position and a new block is taken every block_size tokens).
 *
 *   key, value    fp16 [num_tokens, num_heads, head_dim]        (read)
 *   k_cache,
 *   v_cache       fp16 [num_blocks, block_size, num_heads, head_dim] (written
 *                 at the given slots only)
 *   slot_mapping  int64 [num_tokens]: slot of each token.  A slot outside
 *                 [0, num_blocks * block_size) — e.g. -1 for a padding
 *                 token — is skipped.  Valid slots must be distinct within a
 *                 call (otherwise which token lands there is unspecified).
 *
 * The copy is bit-exact: raw 16-bit patterns (NaN payloads, signed zeros,
 * subnormals included) are moved, never converted.
 * Requires head_dim % 8 == 0 (whole 16-byte vectors per head row).
 * num_tokens == 0 enqueues nothing and returns PA_OK.
 */
int pa_reshape_and_cache(const void* key, const void* value, void* k_cache, void* v_cache,
                         const int64_t* slot_mapping, int32_t num_tokens, int32_t num_heads,
                         int32_t head_dim, int32_t num_blocks, int32_t block_size,
                         void* stream);

/*
 * Bytes of device workspace pa_decode needs for the split-context path:
 * partial results (normalised output row in fp16, running maximum and sum in
 * fp32) for each (sequence, head, context partition).  [src] §六 names a second version of
 * PagedAttention ("v2") without describing it; the split reading here is
 * partitions of partition_size logical tokens starting at multiples of it,
 * each reduced to (max, sum, normalised row) and merged by the exact
 * log-sum-exp identity of the softmax in [10x] §2.1 (the merge is exact in
 * any precision of the rows; the fp16 rows, before any FP8 V scale, add at
 * most 2^-11 relative per element, the size of the output's own rounding).
 * Layout in the workspace: o [num_seqs, num_heads, NP, head_dim] fp16, then
 * m and l [num_seqs, num_heads, NP] fp32, each part starting at a 256-byte
 * boundary,
 * NP = ceil(max_blocks_per_seq * block_size / partition_size).  Returns 0
 * when no split happens (partition_size == 0, or a single partition covers
 * max_blocks_per_seq * block_size tokens) and 0 for invalid arguments (no
 * error code: pa_decode reports those).  Host only; no device call.
 */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                int32_t block_size, int32_t max_blocks_per_seq,
                                int32_t partition_size);

/*
 * Paged-attention decode, one query token per sequence ([10x] §2.3):
 *   out[s,h,:] = softmax(scale * q[s,h,:] . K_paged[s,h,i,:]^T over
 *                i < context_lens[s]) . V_paged[s,h,:,:]
 * with K_paged[s,h,i] = k_cache[block_tables[s, i / block_size],
 * i % block_size, h] and likewise V ([10x] §2.3; [eng] §3.3).  scale is
 * the caller's 1/sqrt(d_k) ([10x] §2.1).  A physical block that several
 * tables list (a shared prefix, [arch] §2.3) is simply read through each.
 *
 *   out           fp16 [num_seqs, num_heads, head_dim]              (written)
 *   q             fp16 [num_seqs, num_heads, head_dim]              (read)
 *   k_cache,
 *   v_cache       fp16 [num_blocks, block_size, num_heads, head_dim] (read)
 *   block_tables  int32 [num_seqs, max_blocks_per_seq]; only the first
 *                 ceil(context_lens[s] / block_size) entries of row s are
 *                 read, and each must lie in [0, num_blocks).
 *   context_lens  int32 [num_seqs]; 0 <= context_lens[s] <=
 *                 max_blocks_per_seq * block_size.  0 gives an all-zero row.
 *                 Cache positions at or past the context are never used in
 *                 arithmetic, whatever they hold.
 *   head_dim      64 or 128;  block_size  16 or 32.
 *   partition_size  0: each (sequence, head) is one work unit.  Otherwise a
 *                 positive multiple of block_size: the context is split into
 *                 partitions of that many tokens, each reduced to (max, sum,
 *                 normalised row), and a second kernel merges them with the
 *                 log-sum-exp identity.
 *   workspace, workspace_bytes  device scratch of at least
 *                 pa_decode_workspace_size(...) bytes (may be NULL when that
 *                 is 0).  Contents on entry do not matter.
 *
 * Arithmetic: fp16 inputs, fp32 products, sums and softmax; the result is
 * rounded to fp16 (nearest even).  For fixed arguments the result is
 * bitwise reproducible, and it does not depend on which physical blocks
 * hold the data.
 */
int pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
              int32_t num_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
              int32_t max_blocks_per_seq, float scale, int32_t partition_size,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same arguments, semantics, result bits and errors as pa_decode, without
 * the workspace arguments.  The split-context partials go to a static device
 * array of PA_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it
 * runs on (from the first call on that GPU until the process ends); the
 * call itself allocates and frees nothing.
 *   - A call whose pa_decode_workspace_size(...) exceeds
 *     PA_NOALLOC_SCRATCH_BYTES returns PA_ERR_SCRATCH and enqueues nothing
 *     (32 MiB holds, e.g., 256 sequences x 40 heads x 8 partitions of
 *     head_dim 128: 21.6 MB).
 *   - The scratch is that of the calling thread's current device; `stream`
 *     must belong to that device.
 *   - Every call on a GPU shares that GPU's array, and nothing in it has to
 *     start at zero (each partition writes its slot before the merge reads
 *     it).  Calls that may overlap in time on one GPU (on different streams
 *     without an ordering between them) race on the array; calls on one
 *     stream are ordered and safe.
 * The first call on a device looks the array's address up
 * (hipGetSymbolAddress); a failure there returns PA_ERR_HIP.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

int pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                      int32_t max_blocks_per_seq, float scale, int32_t partition_size,
                      void* stream);

/*
 * Decode for a batch whose sequences all begin with the same shared prefix
 * ([eng] §3.2, [10x] §4.4: several tables list the same physical blocks).
 * The result equals pa_decode over the tables prefix_block_table ++
 * block_tables[s] with context prefix_len + context_lens[s]; it is computed
 * so that the prefix is read once per 64 sequences and head (a workgroup
 * stages 64-token pieces of the prefix in LDS for the matrix-core products of
 * 64 queries) and each suffix once, all pieces merged with the log-sum-exp
 * identity.  Each 128-token piece of the prefix leaves (max, sum, normalised
 * row) per (sequence, head) in the workspace, the row in fp16 as pa_decode's
 * partition rows.  The same launch writes, in the last round_up(8 * num_seqs,
 * 256) bytes of the pa_decode_cascade_workspace_size(...) it needs, the order
 * in which the suffix launch takes the sequences: num_seqs int32 ids by
 * descending suffix length, then their lengths (a schedule only: every order
 * gives the same bits).
 *
 *   prefix_block_table  int32 [prefix_len / block_size], DEVICE: the prefix's
 *                       physical blocks in logical order
 *   prefix_len          tokens in the prefix, a multiple of block_size
 *                       (0: plain pa_decode)
 *   block_tables,
 *   context_lens        the private suffixes: [num_seqs, max_blocks_per_seq]
 *                       and [num_seqs] (suffix lengths, 0 allowed)
 *   workspace           at least pa_decode_cascade_workspace_size(...) bytes
 * Other arguments, layouts and errors as pa_decode, except that scale must
 * be finite and > 0 (else PA_ERR_INVALID_DIM).  head_dim 64 or 128,
 * block_size 16 or 32.
 */
size_t pa_decode_cascade_workspace_size(int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                        int32_t block_size, int32_t prefix_len,
                                        int32_t max_blocks_per_seq, int32_t partition_size);

int pa_decode_cascade(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* prefix_block_table, int32_t prefix_len,
                      const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                      int32_t num_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                      int32_t max_blocks_per_seq, float scale, int32_t partition_size,
                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * One decode step of a shared-prefix batch in one call: pa_reshape_and_cache
 * of this step's tokens followed by pa_decode_cascade ([10x] §2.3: each new
 * token's K/V go into the slot its block table names, then attention runs
 * over the context that now includes it).  Token s of key / value is the new
 * token of sequence s; it belongs to the private suffix.
 *
 *   key, value     fp16 [num_seqs, num_heads, head_dim] (read)
 *   k_cache,
 *   v_cache        as pa_decode_cascade, and written: row s of key / value
 *                  goes to slot_mapping[s] exactly as pa_reshape_and_cache
 *                  puts it (bit patterns kept; slots outside [0, num_blocks *
 *                  block_size) skipped)
 *   slot_mapping   int64 [num_seqs], DEVICE, 8-byte aligned
 * Other arguments, workspace and errors as pa_decode_cascade; key / value
 * 16-byte aligned.
 *
 * The writes are made by the prefix pass, which reads only the prefix blocks,
 * and the suffix partitions run after it on the stream, so no second launch
 * is needed.  Precondition: no slot_mapping[s] lies in a prefix block (a new
 * token always lands in a private block; [arch] §2.3: a shared block is
 * copied before a sequence writes into it).  Then out and both caches are
 * bitwise what pa_reshape_and_cache (num_tokens = num_seqs) followed by
 * pa_decode_cascade produce.  prefix_len = 0 runs exactly those two steps.
 */
int pa_decode_cascade_append(void* out, const void* q, const void* key, const void* value,
                             void* k_cache, void* v_cache, const int64_t* slot_mapping,
                             const int32_t* prefix_block_table, int32_t prefix_len,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                             int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                             float scale, int32_t partition_size, void* workspace,
                             size_t workspace_bytes, void* stream);

/*
 * Multi-query paged attention: several new tokens per sequence in one batch
 * (chunked prefill, or prefill mixed with decode: [10x] §4.3, [eng] §4.2).
 * Sequence s brings n_s = query_start[s+1] - query_start[s] query rows; they
 * are the last n_s positions of its context (their K/V already written, e.g.
 * by pa_reshape_and_cache), so row i sits at logical position
 * p = context_lens[s] - n_s + i and attends positions 0..p (causal):
 *   out[row, h, :] = softmax(scale * q[row, h, :] . K_paged[s, h, 0..p]^T)
 *                    . V_paged[s, h, 0..p, :]
 * n_s = 1 is the decode step.
 *
 *   q, out         fp16 [num_tokens, num_heads, head_dim]; the rows of
 *                  sequence s are query_start[s] .. query_start[s+1]-1
 *   query_start    int32 [num_seqs + 1], DEVICE, non-decreasing,
 *                  query_start[0] = 0, query_start[num_seqs] = num_tokens
 *   max_query_len  an upper bound of every n_s (sizes the launch)
 *   block_tables, context_lens  as pa_decode; n_s <= context_lens[s]
 *   scale          finite and > 0 (else PA_ERR_INVALID_DIM)
 * head_dim 64 or 128, block_size 16 or 32.  No workspace.  Rows are
 * processed in tiles of 128 per (sequence, head); a K/V chunk of 64 tokens is
 * read once per tile.
 */
int pa_multi_query(void* out, const void* q, const void* k_cache, const void* v_cache,
                   const int32_t* block_tables, const int32_t* context_lens,
                   const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                   int32_t max_query_len, int32_t num_heads, int32_t head_dim, int32_t num_blocks,
                   int32_t block_size, int32_t max_blocks_per_seq, float scale, void* stream);

/*
 * FP8 KV cache.  [10x] §3.3 names FP8 quantisation without fixing a format;
 * the reading used here is OCP FP8 E4M3 (1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits, no infinities, S.1111.111 = NaN, largest value 448)
 * with one float scale per cache: code = E4M3(x * (1/scale)) where the
 * product is rounded to float and then to the nearest E4M3 value (ties to
 * even); finite values beyond +-448 saturate to +-448 and NaN stays NaN.  A
 * code decodes to value(code) * scale.  Caches hold one byte per element in
 * the same [num_blocks, block_size, num_heads, head_dim] layout.
 */

/*
 * pa_reshape_and_cache for FP8 caches: the same slots and skip rule as
 * pa_reshape_and_cache; each fp16 value of key (value) is quantised with
 * k_scale (v_scale).  Scales must be finite and > 0; head_dim % 16 == 0.
 * The codes are bit-exact for the rule above.
 */
int pa_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache, void* v_cache,
                             const int64_t* slot_mapping, int32_t num_tokens, int32_t num_heads,
                             int32_t head_dim, int32_t num_blocks, int32_t block_size,
                             float k_scale, float v_scale, void* stream);

/*
 * pa_decode over FP8 caches: the same arguments, semantics, workspace
 * (pa_decode_workspace_size) and errors as pa_decode, with k_cache / v_cache
 * holding E4M3 codes and K_paged, V_paged replaced by value(code) * k_scale
 * and value(code) * v_scale.  q and out stay fp16; the arithmetic is fp32
 * (codes are widened exactly).  Scales must be finite and > 0.
 */
int pa_decode_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* block_tables, const int32_t* context_lens, int32_t num_seqs,
                  int32_t num_heads, int32_t head_dim, int32_t num_blocks, int32_t block_size,
                  int32_t max_blocks_per_seq, float scale, float k_scale, float v_scale,
                  int32_t partition_size, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_cascade over FP8 caches: the same arguments, semantics,
 * workspace (pa_decode_cascade_workspace_size) and errors as
 * pa_decode_cascade, with k_cache / v_cache holding E4M3 codes dequantised
 * as in pa_decode_fp8 (k_scale, v_scale finite and > 0, else
 * PA_ERR_INVALID_DIM).  The prefix pass widens each staged code exactly to
 * fp16 for the matrix-core products; the K scale is folded into the logit
 * scale and the V scale into the rows (for the prefix pieces' fp16 rows, when
 * they are merged).  prefix_len = 0 is pa_decode_fp8.
 */
int pa_decode_cascade_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* prefix_block_table, int32_t prefix_len,
                          const int32_t* block_tables, const int32_t* context_lens,
                          int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                          int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                          float scale, float k_scale, float v_scale, int32_t partition_size,
                          void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_cascade_append over FP8 caches: the same arguments and
 * semantics, with k_scale / v_scale as in pa_decode_cascade_fp8; the new
 * rows (fp16) are quantised exactly as pa_reshape_and_cache_fp8 quantises
 * them.  Under the same precondition, out and both caches are bitwise what
 * pa_reshape_and_cache_fp8 followed by pa_decode_cascade_fp8 produce.
 */
int pa_decode_cascade_append_fp8(void* out, const void* q, const void* key, const void* value,
                                 void* k_cache, void* v_cache, const int64_t* slot_mapping,
                                 const int32_t* prefix_block_table, int32_t prefix_len,
                                 const int32_t* block_tables, const int32_t* context_lens,
                                 int32_t num_seqs, int32_t num_heads, int32_t head_dim,
                                 int32_t num_blocks, int32_t block_size,
                                 int32_t max_blocks_per_seq, float scale, float k_scale,
                                 float v_scale, int32_t partition_size, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * pa_multi_query over FP8 caches: the same arguments, semantics and errors as
 * pa_multi_query, with k_cache / v_cache holding E4M3 codes dequantised as in
 * pa_decode_fp8 (k_scale, v_scale finite and > 0, else PA_ERR_INVALID_DIM).
 * Staging widens each code exactly to fp16 for the matrix-core products;
 * the K scale is folded into the logit scale and the V scale into the rows.
 */
int pa_multi_query_fp8(void* out, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* query_start, int32_t num_seqs, int32_t num_tokens,
                       int32_t max_query_len, int32_t num_heads, int32_t head_dim,
                       int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                       float scale, float k_scale, float v_scale, void* stream);

/*
 * Copy whole physical blocks inside one cache pair: the copy-on-write step
 * of [arch] §2.3 (a sequence about to write into a block it shares gets a
 * private copy, and its table is then pointed at the copy by the caller).
 * For each pair i, block block_mapping[2i+1] of k_cache and of v_cache
 * becomes a bitwise copy of block block_mapping[2i].
 *
 *   k_cache,
 *   v_cache        fp16 [num_blocks, block_size, num_heads, head_dim]
 *   block_mapping  int64 [num_pairs, 2], DEVICE array of (src, dst) block ids.
 *                  A pair naming a block outside [0, num_blocks) is skipped.
 *                  Destinations must be distinct and no destination may be
 *                  a source in the same call (otherwise the result is
 *                  unspecified).
 * Requires head_dim % 8 == 0.  num_pairs == 0 enqueues nothing.
 */
int pa_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping, int32_t num_pairs,
                   int32_t num_blocks, int32_t block_size, int32_t num_heads, int32_t head_dim,
                   void* stream);

/*
 * Move whole blocks between two caches of the same block shape, one of
 * which may live in host memory: the swap-out / swap-in of [src] §三.  For
 * each pair i, block block_mapping[2i+1] of dst becomes a bitwise copy of
 * block block_mapping[2i] of src.
 *
 *   src, dst        base pointers of two caches ([src_num_blocks, ...] and
 *                   [dst_num_blocks, ...] blocks), device memory or host
 *                   memory.  src and dst must not overlap.
 *   block_mapping   int64 [num_pairs, 2], HOST array of (src, dst) block ids;
 *                   every id is range-checked first (PA_ERR_RANGE, nothing
 *                   enqueued).
 *   block_bytes     bytes of one block (block_size*num_heads*head_dim*2).
 * When both caches are reachable from the GPU (device memory, or pinned host
 * memory from hipHostMalloc, as hipPointerGetAttributes reports), the moves
 * run as kernels on `stream` that read and write across PCIe (the pairs
 * travel in the kernel arguments).  Otherwise they are hipMemcpyAsync copies
 * on `stream`, with runs of pairs whose source and destination ids both
 * increase by one merged into one copy (with pageable host memory these
 * complete before the call returns).
 */
int pa_swap_blocks(const void* src, void* dst, const int64_t* block_mapping, int32_t num_pairs,
                   int32_t src_num_blocks, int32_t dst_num_blocks, int64_t block_bytes,
                   void* stream);

/*
 * Static text of a status code returned by any entry point above (never
 * NULL; an unknown code gives "unknown pa status").  The codes and the
 * conditions behind them are this library's own (the pages define no error
 * interface; [eng] §3.3 only has the block manager raise when no block is
 * free).  The string is owned by the library and must not be freed.
 */
const char* pa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
