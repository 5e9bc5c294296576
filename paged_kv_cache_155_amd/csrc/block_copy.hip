// Whole-block copies for gfx950: copy-on-write inside a cache pair, and
// swaps between device and host caches.
//
// Sources: "vLLM基础架构：核心组件、PagedAttention原理、KV Cache管理与连续批处理机制"
// §2.3 (a shared block is copied before a sequence writes into it) and
// "【硬核】啃透vLLM源码：从PagedAttention到连续批处理，大模型推理加速24倍的秘密"
// §三 (blocks swapped out to host memory and back in).
//
// copy_blocks: a block is B*H*D fp16 values stored contiguously, so each
// pair is one contiguous run per cache.  The grid has kChunks workgroups per
// pair; a workgroup moves kVecsPerWg 16-byte vectors of K and of V, all of
// a thread's loads in flight before its stores (nontemporal loads: the
// source is read once; plain stores: the copy is read soon after by the
// decode).  Bit-exact,
// no conversion.  Pure HBM copy: 2 * block bytes read and written per pair.
//
// swap_blocks: when both caches are reachable from the GPU (device memory,
// or pinned host memory mapped into the device address space, as reported
// by hipPointerGetAttributes), one kernel moves all the scattered blocks over
// PCIe with 16-byte loads and stores; the pairs travel in the kernel
// arguments (up to kPairsPerLaunch per launch), so nothing is allocated.
// Otherwise the moves go to the DMA engines with hipMemcpyAsync, with runs of
// consecutive pairs merged into longer copies.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_internal.h"

namespace pa {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kThreads = 256;
constexpr int kVecsPerWg = 2048;  // 32 KiB of each cache per workgroup

__global__ __launch_bounds__(kThreads) void copy_blocks_kernel(
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache,
    const int64_t* __restrict__ block_mapping, int64_t num_blocks, int64_t block_vecs,
    int32_t chunks)
{
    const int pair = blockIdx.x / chunks;
    const int chunk = blockIdx.x % chunks;
    const int64_t src = block_mapping[2 * pair];
    const int64_t dst = block_mapping[2 * pair + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks)
        return;
    const int64_t lo = (int64_t)chunk * kVecsPerWg;
    const int64_t hi = min(lo + kVecsPerWg, block_vecs);
    const u32x4* ks = k_cache + src * block_vecs;
    const u32x4* vs = v_cache + src * block_vecs;
    u32x4* kd = k_cache + dst * block_vecs;
    u32x4* vd = v_cache + dst * block_vecs;
    constexpr int kPerThread = kVecsPerWg / kThreads;
    if (hi - lo == kVecsPerWg) {  // a whole chunk: all loads in flight before the stores
        u32x4 a[kPerThread], b[kPerThread];
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t i = lo + threadIdx.x + (int64_t)j * kThreads;
            a[j] = __builtin_nontemporal_load(ks + i);
            b[j] = __builtin_nontemporal_load(vs + i);
        }
#pragma unroll
        for (int j = 0; j < kPerThread; ++j) {
            const int64_t i = lo + threadIdx.x + (int64_t)j * kThreads;
            kd[i] = a[j];
            vd[i] = b[j];
        }
        return;
    }
    for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads) {
        const u32x4 a = __builtin_nontemporal_load(ks + i);
        const u32x4 b = __builtin_nontemporal_load(vs + i);
        kd[i] = a;
        vd[i] = b;
    }
}

constexpr int kPairsPerLaunch = 120;  // 1920 bytes of kernel arguments

struct SwapPairs {
    int64_t src[kPairsPerLaunch];
    int64_t dst[kPairsPerLaunch];
};

__global__ __launch_bounds__(kThreads) void swap_blocks_kernel(
    const u32x4* __restrict__ src, u32x4* __restrict__ dst, int64_t block_vecs, int32_t chunks,
    SwapPairs pairs)
{
    const int pair = blockIdx.x / chunks;
    const int chunk = blockIdx.x % chunks;
    const int64_t a = pairs.src[pair];
    const int64_t b = pairs.dst[pair];
    const int64_t lo = (int64_t)chunk * kVecsPerWg;
    const int64_t hi = min(lo + kVecsPerWg, block_vecs);
    const u32x4* s = src + a * block_vecs;
    u32x4* d = dst + b * block_vecs;
    for (int64_t i = lo + threadIdx.x; i < hi; i += kThreads)
        d[i] = s[i];
}

// Device-side address of ptr if the GPU can reach it (device memory or
// pinned, mapped host memory), else nullptr.
void* reachable(const void* ptr)
{
    hipPointerAttribute_t at{};
    if (hipPointerGetAttributes(&at, ptr) != hipSuccess) {
        (void)hipGetLastError();  // clear the sticky error of an unknown pointer
        return nullptr;
    }
    if (at.type == hipMemoryTypeDevice || at.type == hipMemoryTypeHost)
        return at.devicePointer;
    return nullptr;
}

}  // namespace

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_mapping,
                              int32_t num_pairs, int64_t num_blocks, int64_t block_vecs,
                              hipStream_t stream)
{
    const int32_t chunks = (int32_t)((block_vecs + kVecsPerWg - 1) / kVecsPerWg);
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((uint32_t)num_pairs * chunks), dim3(kThreads), 0,
                       stream, static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache),
                       block_mapping, num_blocks, block_vecs, chunks);
    return hipGetLastError();
}

hipError_t enqueue_swap_blocks(const void* src, void* dst, const int64_t* block_mapping,
                               int32_t num_pairs, int64_t block_bytes, hipStream_t stream)
{
    void* src_dev = reachable(src);
    void* dst_dev = reachable(dst);
    // (the kernel path also needs its grid, kPairsPerLaunch blocks of
    // ceil(block_vecs / kVecsPerWg) workgroups, to stay under 2^32 work-items)
    if (src_dev && dst_dev && block_bytes % 16 == 0 &&
        (reinterpret_cast<uintptr_t>(src_dev) & 15u) == 0 &&
        (reinterpret_cast<uintptr_t>(dst_dev) & 15u) == 0 &&
        (block_bytes / 16 + kVecsPerWg - 1) / kVecsPerWg * kPairsPerLaunch <=
            (int64_t)(UINT32_MAX / kThreads)) {
        const int64_t block_vecs = block_bytes / 16;
        const int32_t chunks = (int32_t)((block_vecs + kVecsPerWg - 1) / kVecsPerWg);
        for (int32_t i0 = 0; i0 < num_pairs; i0 += kPairsPerLaunch) {
            const int32_t n = min(kPairsPerLaunch, num_pairs - i0);
            SwapPairs pairs{};
            for (int32_t j = 0; j < n; ++j) {
                pairs.src[j] = block_mapping[2 * (i0 + j)];
                pairs.dst[j] = block_mapping[2 * (i0 + j) + 1];
            }
            hipLaunchKernelGGL(swap_blocks_kernel, dim3((uint32_t)n * chunks), dim3(kThreads), 0,
                               stream, static_cast<const u32x4*>(src_dev),
                               static_cast<u32x4*>(dst_dev), block_vecs, chunks, pairs);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess)
                return e;
        }
        return hipSuccess;
    }
    const char* s = static_cast<const char*>(src);
    char* d = static_cast<char*>(dst);
    int32_t i = 0;
    while (i < num_pairs) {
        const int64_t a = block_mapping[2 * i], b = block_mapping[2 * i + 1];
        int32_t run = 1;
        while (i + run < num_pairs && block_mapping[2 * (i + run)] == a + run &&
               block_mapping[2 * (i + run) + 1] == b + run)
            ++run;
        hipError_t e = hipMemcpyAsync(d + b * block_bytes, s + a * block_bytes,
                                      (size_t)run * block_bytes, hipMemcpyDefault, stream);
        if (e != hipSuccess)
            return e;
        i += run;
    }
    return hipSuccess;
}

}  // namespace pa
