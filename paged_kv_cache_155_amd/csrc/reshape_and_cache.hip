// reshape_and_cache for gfx950: copy each new token's K and V rows into
// their cache slots as raw 16-bit patterns.
//
// Source: "vLLM推理加速深度解读：PagedAttention如何提升10x吞吐量" §2.3 (the
// slot of logical position i is BlockTable[i / B] * B + i mod B) and §4.2
// (cache layout [num_blocks, block_size, num_heads, head_size]).  In that
// layout a slot's rows for all heads are num_heads * head_dim contiguous
// values, so the copy of one token is one contiguous run per cache.
//
// One workgroup per token; lanes move 16-byte vectors (no conversion, so
// NaN payloads, signed zeros and subnormals survive).  The whole step moves
// a few MB at most and is launch-latency bound.
//
// The FP8 variant quantises on the way (the E4M3 rule of pa_fp8_quant.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_fp8_quant.h"
#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void reshape_and_cache_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value, u32x4* __restrict__ k_cache,
    u32x4* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int64_t num_slots,
    int32_t row_vectors)
{
    const int64_t t = blockIdx.x;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots)
        return;
    const u32x4* ks = key + t * row_vectors;
    const u32x4* vs = value + t * row_vectors;
    u32x4* kd = k_cache + slot * row_vectors;
    u32x4* vd = v_cache + slot * row_vectors;
    for (int i = threadIdx.x; i < row_vectors; i += kThreads) {
        const u32x4 a = ks[i];
        const u32x4 b = vs[i];
        kd[i] = a;
        vd[i] = b;
    }
}

using fp8::quantize8;
using fp8::u32x2;

__global__ __launch_bounds__(kThreads) void reshape_and_cache_fp8_kernel(
    const u32x4* __restrict__ key, const u32x4* __restrict__ value, u32x2* __restrict__ k_cache,
    u32x2* __restrict__ v_cache, const int64_t* __restrict__ slot_mapping, int64_t num_slots,
    int32_t row_groups, float k_inv, float v_inv)
{
    const int64_t t = blockIdx.x;
    const int64_t slot = slot_mapping[t];
    if (slot < 0 || slot >= num_slots)
        return;
    const u32x4* ks = key + t * row_groups;
    const u32x4* vs = value + t * row_groups;
    u32x2* kd = k_cache + slot * row_groups;
    u32x2* vd = v_cache + slot * row_groups;
    for (int i = threadIdx.x; i < row_groups; i += kThreads) {
        kd[i] = quantize8(ks[i], k_inv);
        vd[i] = quantize8(vs[i], v_inv);
    }
}

}  // namespace

hipError_t launch_reshape_and_cache_fp8(const void* key, const void* value, void* k_cache,
                                        void* v_cache, const int64_t* slot_mapping,
                                        int32_t num_tokens, int64_t num_slots, int32_t row_elems,
                                        float k_inv_scale, float v_inv_scale, hipStream_t stream)
{
    hipLaunchKernelGGL(reshape_and_cache_fp8_kernel, dim3(num_tokens), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(key), static_cast<const u32x4*>(value),
                       static_cast<u32x2*>(k_cache), static_cast<u32x2*>(v_cache), slot_mapping,
                       num_slots, row_elems / 8, k_inv_scale, v_inv_scale);
    return hipGetLastError();
}

hipError_t launch_reshape_and_cache(const void* key, const void* value, void* k_cache,
                                    void* v_cache, const int64_t* slot_mapping, int32_t num_tokens,
                                    int64_t num_slots, int32_t row_vectors, hipStream_t stream)
{
    hipLaunchKernelGGL(reshape_and_cache_kernel, dim3(num_tokens), dim3(kThreads), 0, stream,
                       static_cast<const u32x4*>(key), static_cast<const u32x4*>(value),
                       static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), slot_mapping,
                       num_slots, row_vectors);
    return hipGetLastError();
}

}  // namespace pa
