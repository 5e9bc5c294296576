// The FP8 (OCP E4M3) quantiser of the cache writes, shared by
// reshape_and_cache_fp8 and the appending shared-prefix pass so that both
// write the same codes.  "vLLM推理加速深度解读：PagedAttention如何提升10x吞吐量"
// §3.3 names FP8 quantisation without a format; the format is OCP E4M3 with
// one scale per cache: code = E4M3(x * inv_scale), the product rounded to
// float, then rounded to the nearest E4M3 value with ties to even by
// v_cvt_pk_fp8_f32.  Finite values beyond +-448 saturate to +-448 and NaN maps
// to the NaN code with the input's sign; both are decided here, so the
// conversion instruction only sees values in range.
#ifndef PA_FP8_QUANT_H_
#define PA_FP8_QUANT_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {
namespace fp8 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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

}  // namespace fp8
}  // namespace pa

#endif  // PA_FP8_QUANT_H_
