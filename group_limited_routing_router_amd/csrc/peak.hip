// peak.hip -- measurement kernels that anchor the roofline (declared in
// include/moe_peak.h): the streaming read bandwidth, the bf16 MFMA rate, and
// the MFMA rate beside an HBM stream in a GEMM's proportions that this GPU
// sustains.  They compute nothing of the MoE block; the benchmark reports the
// block's kernels against these figures next to the published peaks.
#include "common.h"
#include "moe_peak.h"

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace moe {
namespace {

constexpr int kPeakThreads = 256;
constexpr int kReadUnroll = 8;  // independent 16-byte loads in flight per lane

// Every lane reads kReadUnroll 16-byte chunks per step, the chunks of one step
// one grid width (all threads) apart, and the workgroups walk the buffer
// together (grid stride), so each step of the grid covers one contiguous
// span.  The XOR of everything read is stored only if it equals a value it
// practically never takes, which keeps the loads alive without a write
// stream.
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
// one sum per wave so the chains stay live.  The eight chains keep the matrix
// pipe issuing back to back: no MFMA waits for the result of the one before
// it.
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

// MFMAs fed from LDS with an HBM stream beside them, in the proportions of a
// GEMM: per step every wave reads four A and four B fragments (16 bytes a
// lane each) from a 16 KB LDS region of its own holding pseudo-random bf16
// values (a window that moves every step, so no read repeats the last one)
// and issues the 16 MFMAs of their 4 x 4 outer product (the per-wave ratio
// of a 128 x 128 wave tile), and every lane issues NL nontemporal
// 16-byte loads from the buffer, consumed kStreamAhead steps later so the
// loads are in flight under the MFMAs.  Thread t reads chunks
// t + (s * NL + j) * nthreads for steps s = 0 .. steps + kStreamAhead - 1, so
// the launch reads one contiguous span of the buffer once.  The XOR of the
// loaded data decides whether a value is added to the sum each wave stores,
// which keeps the loads alive.
constexpr int kStreamAhead = 8;
constexpr int kMixLdsChunks = 4096;  // 64 KB: 1024 16-byte chunks per wave

template <int NL>
__global__ __launch_bounds__(kPeakThreads) void mfma_stream_kernel(const u32x4* __restrict__ src,
                                                                   int64_t steps,
                                                                   float* __restrict__ sink) {
    __shared__ u32x4 s_frag[kMixLdsChunks];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * kPeakThreads;
    const int64_t tid = static_cast<int64_t>(blockIdx.x) * kPeakThreads + threadIdx.x;
    for (int i = threadIdx.x; i < kMixLdsChunks; i += kPeakThreads) {
        const uint64_t z = mix64(static_cast<uint64_t>(blockIdx.x) * kMixLdsChunks + i);
        u32x4 v;
        v[0] = random_bf16_pair(static_cast<uint32_t>(z));
        v[1] = random_bf16_pair(static_cast<uint32_t>(z >> 32));
        const uint64_t z2 = mix64(z);
        v[2] = random_bf16_pair(static_cast<uint32_t>(z2));
        v[3] = random_bf16_pair(static_cast<uint32_t>(z2 >> 32));
        s_frag[i] = v;
    }
    __syncthreads();
    f32x16 acc[16];
#pragma unroll
    for (int c = 0; c < 16; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[c][i] = 0.0f;
    const u32x4* p = src + tid;
    u32x4 x = {0u, 0u, 0u, 0u};
    u32x4 ring[kStreamAhead][NL > 0 ? NL : 1];
#pragma unroll
    for (int d = 0; d < kStreamAhead; ++d)
#pragma unroll
        for (int j = 0; j < NL; ++j)
            ring[d][j] = __builtin_nontemporal_load(p + static_cast<int64_t>(d * NL + j) * nthreads);
    const int base = wave * (kMixLdsChunks / 4) + lane;
    for (int64_t s0 = 0; s0 < steps; s0 += kStreamAhead) {
#pragma unroll
        for (int d = 0; d < kStreamAhead; ++d) {
            const int64_t st = s0 + d;
#pragma unroll
            for (int j = 0; j < NL; ++j) {
                x ^= ring[d][j];
                ring[d][j] = __builtin_nontemporal_load(p + ((st + kStreamAhead) * NL + j) * nthreads);
            }
            // the read window moves by 72 chunks a step (wrapping within the
            // wave's region; not a divisor of the unrolled 8 steps' span), so
            // the reads stay in the loop
            const int off = base + static_cast<int>((st * 72) & 511);
            u32x4 fa[4], fb[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                fa[j] = s_frag[off + j * 64];
                fb[j] = s_frag[off + 256 + j * 64];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i * 4 + j] = mfma32(as_bf16x8(fa[i]), as_bf16x8(fb[j]), acc[i * 4 + j]);
        }
    }
#pragma unroll
    for (int d = 0; d < kStreamAhead; ++d)
#pragma unroll
        for (int j = 0; j < NL; ++j) x ^= ring[d][j];
    float sum = ((x[0] ^ x[1] ^ x[2] ^ x[3]) == 0x9e3779b9u) ? 1.0f : 0.0f;
#pragma unroll
    for (int c = 0; c < 16; ++c)
#pragma unroll
        for (int i = 0; i < 16; ++i) sum += acc[c][i];
    if (lane == 0) sink[static_cast<int64_t>(blockIdx.x) * (kPeakThreads / kWave) + wave] = sum;
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

MOE_EXPORT moe_status moe_peak_mfma_stream(const void* buf, size_t bytes, int loads_per_step,
                                           int64_t steps, float* sink, int workgroups,
                                           hipStream_t stream) {
    if (!sink || workgroups < 1 || steps < moe::kStreamAhead || steps % moe::kStreamAhead != 0)
        return MOE_ERR_INVALID_ARG;
    if (loads_per_step != 0 && loads_per_step != 1 && loads_per_step != 2 && loads_per_step != 4)
        return MOE_ERR_INVALID_ARG;
    if (loads_per_step > 0) {
        // every chunk the launch reads lies inside the buffer
        const double need = static_cast<double>(steps + moe::kStreamAhead) * loads_per_step *
                            workgroups * moe::kPeakThreads * 16.0;
        if (!buf || reinterpret_cast<uintptr_t>(buf) % 16 != 0 || static_cast<double>(bytes) < need)
            return MOE_ERR_INVALID_ARG;
    }
    const auto* src = static_cast<const moe::u32x4*>(buf);
    const dim3 grid(workgroups), block(moe::kPeakThreads);
    switch (loads_per_step) {
        case 0: moe::mfma_stream_kernel<0><<<grid, block, 0, stream>>>(src, steps, sink); break;
        case 1: moe::mfma_stream_kernel<1><<<grid, block, 0, stream>>>(src, steps, sink); break;
        case 2: moe::mfma_stream_kernel<2><<<grid, block, 0, stream>>>(src, steps, sink); break;
        default: moe::mfma_stream_kernel<4><<<grid, block, 0, stream>>>(src, steps, sink); break;
    }
    return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_HIP;
}

MOE_EXPORT double moe_peak_mfma_stream_flops(int64_t steps, int workgroups) {
    // waves x steps x 16 MFMAs x (2 * 32 * 32 * 16) FLOP
    return static_cast<double>(workgroups) * (moe::kPeakThreads / moe::kWave) *
           static_cast<double>(steps) * 16 * 2.0 * 32 * 32 * 16;
}

MOE_EXPORT double moe_peak_mfma_stream_bytes(int64_t steps, int loads_per_step, int workgroups) {
    // bytes consumed by the steps (the last kStreamAhead steps' loads come on top)
    return static_cast<double>(workgroups) * moe::kPeakThreads * static_cast<double>(steps) *
           loads_per_step * 16.0;
}
