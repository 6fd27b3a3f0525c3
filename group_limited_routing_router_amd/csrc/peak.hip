// peak.hip -- two measurement kernels that anchor the roofline: the streaming
// read bandwidth and the bf16 MFMA rate this GPU sustains (declared in
// include/moe_peak.h).  They compute nothing of the MoE block; the benchmark
// reports the block's kernels against these figures next to the published
// peaks.
#include "common.h"
#include "moe_peak.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace moe {
namespace {

constexpr int kPeakThreads = 256;
constexpr int kReadUnroll = 8;  // independent 16-byte loads in flight per lane

// Every lane reads kReadUnroll 16-byte chunks per step, the chunks of one step
// one grid width (all threads) apart, and the workgroups walk the buffer
// together (grid stride), so each step of the grid covers one contiguous span.  The XOR of everything
// read is stored only if it equals a value it practically never takes, which
// keeps the loads alive without a write stream.
template <bool NT>
__global__ __launch_bounds__(kPeakThreads) void stream_read_kernel(const u32x4* __restrict__ src,
                                                                   int64_t chunks, uint32_t key,
                                                                   uint32_t* __restrict__ sink) {
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kPeakThreads;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kPeakThreads + threadIdx.x;
    const int64_t step = nthreads * kReadUnroll;
    const int64_t full = chunks / step * step;  // chunks covered by whole steps
    auto load = [&](int64_t c) {
        if constexpr (NT)
            return __builtin_nontemporal_load(src + c);
        else
            return src[c];
    };
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int64_t s0 = 0; s0 < full; s0 += step) {
        u32x4 v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) v[u] = load(s0 + u * nthreads + tid);
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u];
    }
    for (int64_t c = full + tid; c < chunks; c += nthreads) acc ^= load(c);
    const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
    if (r == key) sink[0] = r;
}

// Each wave runs `iters` steps of kChains independent 32x32x16 bf16 MFMAs on
// operands held in registers (no memory traffic inside the loop), then stores
// one sum per wave so the chains stay live.  With four waves per SIMD the
// matrix pipe always has an independent MFMA to issue.
constexpr int kChains = 8;

// splitmix64 finalizer (Steele, Lea and Flood, "Fast splittable pseudorandom
// number generators", 2014): a bijective mix of a 64-bit counter.
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z += 0x9e3779b97f4a7c15ull;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

// Two bf16 values from 32 random bits: random sign and 7-bit mantissa,
// exponent 2^-5 .. 2^-2, so magnitudes lie in [2^-5, 2^-1).
__device__ __forceinline__ uint32_t random_bf16_pair(uint32_t r) {
    uint32_t w = 0;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const uint32_t q = r >> (16 * h);
        const uint32_t bits = ((q & 1u) << 15) | ((122u + ((q >> 1) & 3u)) << 7) | ((q >> 3) & 0x7fu);
        w |= bits << (16 * h);
    }
    return w;
}

__global__ __launch_bounds__(kPeakThreads) void mfma_loop_kernel(int64_t iters, int random_operands,
                                                                 float* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const uint64_t tid = static_cast<uint64_t>(blockIdx.x) * kPeakThreads + threadIdx.x;
    bf16x8 a[kChains], b[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c) {
        u32x4 ra, rb;
#pragma unroll
        for (int i = 0; i < 4; i += 2) {
            if (random_operands) {
                // chain c takes its own operands, different on every lane
                const uint64_t za = mix64((tid * kChains + c) * 4 + i / 2);
                const uint64_t zb = mix64((tid * kChains + c) * 4 + 2 + i / 2);
                ra[i] = random_bf16_pair(static_cast<uint32_t>(za));
                ra[i + 1] = random_bf16_pair(static_cast<uint32_t>(za >> 32));
                rb[i] = random_bf16_pair(static_cast<uint32_t>(zb));
                rb[i + 1] = random_bf16_pair(static_cast<uint32_t>(zb >> 32));
            } else {
                // fixed bf16 operands: a = 1 + lane / 128, b about 2^-9, so
                // the sums stay far from overflow over any number of steps
                ra[i] = ra[i + 1] = 0x3f803f80u + static_cast<uint32_t>(lane);
                rb[i] = 0x3b003b00u + static_cast<uint32_t>(i);
                rb[i + 1] = 0x3b003b00u + static_cast<uint32_t>(i + 1);
            }
        }
        a[c] = as_bf16x8(ra);
        b[c] = as_bf16x8(rb);
    }
    f32x16 acc[kChains];
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int c = 0; c < kChains; ++c) acc[c] = mfma32(a[c], b[c], acc[c]);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < kChains; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) s += acc[c][i];
    if (lane == 0)
        sink[static_cast<int64_t>(blockIdx.x) * (kPeakThreads / kWave) + (threadIdx.x >> 6)] = s;
}

}  // namespace
}  // namespace moe

MOE_EXPORT moe_status moe_peak_stream_read(const void* buf, size_t bytes, int nontemporal,
                                           uint32_t* sink, int workgroups, hipStream_t stream) {
    if (!buf || !sink || bytes < 16 || bytes % 16 != 0 ||
        reinterpret_cast<uintptr_t>(buf) % 16 != 0 || workgroups < 1)
        return MOE_ERR_INVALID_ARG;
    const int64_t chunks = static_cast<int64_t>(bytes / 16);
    const auto* src = static_cast<const moe::u32x4*>(buf);
    // 0x9e3779b9: a key the XOR of the buffer almost never equals
    if (nontemporal)
        moe::stream_read_kernel<true><<<dim3(workgroups), dim3(moe::kPeakThreads), 0, stream>>>(
            src, chunks, 0x9e3779b9u, sink);
    else
        moe::stream_read_kernel<false><<<dim3(workgroups), dim3(moe::kPeakThreads), 0, stream>>>(
            src, chunks, 0x9e3779b9u, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_EXPORT moe_status moe_peak_mfma_bf16(int64_t iters, int random_operands, float* sink,
                                         int workgroups, hipStream_t stream) {
    if (!sink || iters < 1 || workgroups < 1) return MOE_ERR_INVALID_ARG;
    moe::mfma_loop_kernel<<<dim3(workgroups), dim3(moe::kPeakThreads), 0, stream>>>(
        iters, random_operands != 0, sink);
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_EXPORT double moe_peak_mfma_bf16_flops(int64_t iters, int workgroups) {
    // waves x steps x chains x (2 * 32 * 32 * 16) FLOP
    return static_cast<double>(workgroups) * (moe::kPeakThreads / moe::kWave) *
           static_cast<double>(iters) * moe::kChains * 2.0 * 32 * 32 * 16;
}
