// Streaming-read and copy bandwidth of this GPU, for bench.py's achievable-peak
// figure: an 8 GiB device buffer read once per launch with 16-byte
// nontemporal loads (plain loads for comparison), and a 2 GiB -> 2 GiB copy.
// Prints one JSON line.  Not part of the library.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdio>
#include <vector>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                       \
    do {                                                                               \
        hipError_t e_ = (x);                                                           \
        if (e_ != hipSuccess) {                                                        \
            fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__); \
            return 1;                                                                  \
        }                                                                              \
    } while (0)

constexpr int kThreads = 256;
constexpr int kUnroll = 16;

// Workgroup w reads the contiguous range [w*per, (w+1)*per) of n16 vectors,
// kUnroll loads in flight per lane; an XOR of the data keeps the loads live.
template <bool kNontemporal>
__global__ __launch_bounds__(kThreads) void read_kernel(const u32x4* __restrict__ p, size_t n16,
                                                        uint32_t* sink)
{
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t begin = (size_t)blockIdx.x * per;
    const size_t end = begin + per < n16 ? begin + per : n16;
    uint32_t acc = 0;
    for (size_t i = begin + threadIdx.x; i < end; i += (size_t)kThreads * kUnroll) {
        u32x4 v[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const size_t j = i + (size_t)u * kThreads;
            v[u] = j < end ? (kNontemporal ? __builtin_nontemporal_load(p + j) : p[j])
                           : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9e3779b9u)  // practically never true: the store only keeps the loads
        sink[blockIdx.x % 1024] = acc;
}

__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src,
                                                        u32x4* __restrict__ dst, size_t n16)
{
    for (size_t i = (size_t)blockIdx.x * kThreads + threadIdx.x; i < n16;
         i += (size_t)gridDim.x * kThreads)
        __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

template <typename F>
int median_ms(F launch, hipEvent_t e0, hipEvent_t e1, float* out)
{
    std::vector<float> ts;
    for (int r = 0; r < 7; ++r) {
        CHECK(hipEventRecord(e0));
        launch();
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(e1));
        CHECK(hipEventSynchronize(e1));
        float ms = 0.0f;
        CHECK(hipEventElapsedTime(&ms, e0, e1));
        ts.push_back(ms);
    }
    std::sort(ts.begin(), ts.end());
    *out = ts[ts.size() / 2];
    return 0;
}

int main()
{
    const size_t bytes = (size_t)8 << 30;
    const size_t n16 = bytes / 16;
    u32x4* a = nullptr;
    uint32_t* sink = nullptr;
    CHECK(hipMalloc(&a, bytes));
    CHECK(hipMalloc(&sink, 4096));
    CHECK(hipMemset(a, 1, bytes));
    CHECK(hipDeviceSynchronize());
    hipEvent_t e0, e1;
    CHECK(hipEventCreate(&e0));
    CHECK(hipEventCreate(&e1));

    printf("{\"probe\": \"read\", \"bytes\": %zu, \"runs\": \"median of 7\", \"read_gbs\": {", bytes);
    float best = 0.0f;
    const int grids[] = {4096, 8192, 16384};
    bool first = true;
    for (int nt = 1; nt >= 0; --nt) {
        for (int g : grids) {
            float ms = 0.0f;
            if (nt) {
                if (median_ms([&] { hipLaunchKernelGGL(read_kernel<true>, dim3(g), dim3(kThreads), 0, 0, a, n16, sink); }, e0, e1, &ms))
                    return 1;
            } else {
                if (median_ms([&] { hipLaunchKernelGGL(read_kernel<false>, dim3(g), dim3(kThreads), 0, 0, a, n16, sink); }, e0, e1, &ms))
                    return 1;
            }
            const float gbs = (float)(bytes / (ms * 1e-3) / 1e9);
            if (nt)
                best = std::max(best, gbs);
            printf("%s\"%s_grid%d\": %.1f", first ? "" : ", ", nt ? "nontemporal" : "plain", g, gbs);
            first = false;
        }
    }
    const size_t half = n16 / 4;  // 2 GiB each way
    float ms = 0.0f;
    if (median_ms([&] { hipLaunchKernelGGL(copy_kernel, dim3(16384), dim3(kThreads), 0, 0, a, a + half * 2, half); }, e0, e1, &ms))
        return 1;
    const float copy = (float)(2.0 * half * 16 / (ms * 1e-3) / 1e9);
    printf("}, \"best_read_gbs\": %.1f, \"copy_read_plus_write_gbs\": %.1f}\n", best, copy);
    CHECK(hipFree(a));
    CHECK(hipFree(sink));
    return 0;
}
