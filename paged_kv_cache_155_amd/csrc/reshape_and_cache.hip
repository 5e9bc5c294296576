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
// The FP8 variant ("vLLM推理加速深度解读" §3.3 names FP8 quantisation; the
// format is OCP E4M3 with one scale per cache) quantises on the way:
// code = E4M3(x * inv_scale), the product rounded to float, then rounded to
// the nearest E4M3 value with ties to even by v_cvt_pk_fp8_f32.  Finite
// values beyond +-448 saturate to +-448 and NaN maps to the NaN code with the
// input's sign; both are decided here, so the conversion instruction only
// sees values in range.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float saturate_e4m3(float y)
{
    return fminf(fmaxf(y, -448.0f), 448.0f);
}

// Two fp16 values (one dword) -> two E4M3 codes in the low 16 bits.
__device__ __forceinline__ uint32_t quantize_pair(uint32_t w, float inv)
{
    const h2 x = __builtin_bit_cast(h2, w);
    const float y0 = (float)x.x * inv;
    const float y1 = (float)x.y * inv;
    uint32_t c = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(saturate_e4m3(y0), saturate_e4m3(y1),
                                                            0, false) & 0xFFFFu;
    const uint32_t nan0 = 0x7Fu | ((w >> 8) & 0x80u);    // sign of x.x is bit 15
    const uint32_t nan1 = 0x7Fu | ((w >> 24) & 0x80u);   // sign of x.y is bit 31
    if (y0 != y0)
        c = (c & 0xFF00u) | nan0;
    if (y1 != y1)
        c = (c & 0x00FFu) | (nan1 << 8);
    return c;
}

// Eight fp16 values (16 bytes) -> eight codes (8 bytes).
__device__ __forceinline__ u32x2 quantize8(const u32x4& v, float inv)
{
    const uint32_t c0 = quantize_pair(v.x, inv), c1 = quantize_pair(v.y, inv);
    const uint32_t c2 = quantize_pair(v.z, inv), c3 = quantize_pair(v.w, inv);
    return u32x2{c0 | (c1 << 16), c2 | (c3 << 16)};
}

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
