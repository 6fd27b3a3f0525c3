// combine.hip -- weighted recombination of the expert outputs.
//
// The k expert outputs of a token are summed with the normalised router
// weights and the sum is multiplied by the block's scale ("Welcome Beam: a
// 501B open model you can own, customize, and scale", section "Mixture of
// Experts": 2.5 for Beam).  Token-major gather: each output element reads its
// k rows of y through pair_rows and sums them in fixed j order in fp32, so
// there are no atomics and the result is deterministic.  HBM-bound: it reads
// T*k*H fp32 and writes T*H outputs; loads are 16 B per lane and the k row
// loads of one column chunk are independent, so k loads are in flight per
// lane.  A token's workgroup takes the fewest passes over the row's float4
// chunks that at most 1024 threads allow, with the fewest whole waves for
// that many passes (two passes of 640 threads for a 5120-wide row: 3% faster
// than five passes of 256 at 8192 tokens, 20% at 128).
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;            // combine + residual with many tokens
constexpr int kCombineMaxThreads = 1024;
constexpr int64_t kWideBelowTokens = 256;  // about one workgroup per compute unit

int combine_threads(int H) {
    const int nv = H / 4;
    const int passes = (nv + kCombineMaxThreads - 1) / kCombineMaxThreads;
    const int per = (nv + passes - 1) / passes;
    return (per + 63) / 64 * 64;
}

// y larger than kStreamBytes streams past the caches (nontemporal loads and
// output stores): at prefill it is far larger than L2 plus the Infinity Cache
// and is read once; at decode it is still cache-resident from the down
// projection.

__device__ __forceinline__ float4 load4(const float* p, bool nt) {
    if (nt) {
        const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        return make_float4(v[0], v[1], v[2], v[3]);
    }
    return *reinterpret_cast<const float4*>(p);
}

template <int K, bool OUT_BF16>
__global__ __launch_bounds__(kCombineMaxThreads) void combine_kernel(int64_t T, int H, float scale,
                                                           const float* __restrict__ y,
                                                           const int32_t* __restrict__ pair_rows,
                                                           const float* __restrict__ weights,
                                                           void* __restrict__ out, bool nt) {
    const int64_t t = blockIdx.x;
    int32_t row[K];
    float w[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        row[j] = pair_rows[t * K + j];
        w[j] = weights[t * K + j];
    }
    const int nv = H >> 2;  // float4 chunks per row
    for (int c = threadIdx.x; c < nv; c += blockDim.x) {
        float4 v[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (row[j] >= 0)
                v[j] = load4(y + static_cast<int64_t>(row[j]) * H + 4 * c, nt);
            else
                v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int j = 0; j < K; ++j) {
            acc.x = acc.x + w[j] * v[j].x;
            acc.y = acc.y + w[j] * v[j].y;
            acc.z = acc.z + w[j] * v[j].z;
            acc.w = acc.w + w[j] * v[j].w;
        }
        acc.x *= scale;
        acc.y *= scale;
        acc.z *= scale;
        acc.w *= scale;
        if constexpr (OUT_BF16) {
            uint2 packed;
            packed.x = static_cast<uint32_t>(f32_to_bf16_rne(acc.x)) |
                       (static_cast<uint32_t>(f32_to_bf16_rne(acc.y)) << 16);
            packed.y = static_cast<uint32_t>(f32_to_bf16_rne(acc.z)) |
                       (static_cast<uint32_t>(f32_to_bf16_rne(acc.w)) << 16);
            reinterpret_cast<uint2*>(static_cast<uint16_t*>(out) + t * H)[c] = packed;
        } else {
            float* o = static_cast<float*>(out) + t * H + 4 * c;
            if (nt)
                __builtin_nontemporal_store(f32x4{acc.x, acc.y, acc.z, acc.w}, reinterpret_cast<f32x4*>(o));
            else
                *reinterpret_cast<float4*>(o) = acc;
        }
    }
}

template <int K>
hipError_t launch_k(const Problem& p, const float* y, const int32_t* pair_rows,
                    const float* weights, void* out, bool out_bf16, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(p.T)), block(combine_threads(p.H));
    const bool nt = p.T * p.k * static_cast<int64_t>(p.H) * 4 > kStreamBytes;
    if (out_bf16)
        combine_kernel<K, true><<<grid, block, 0, s>>>(p.T, p.H, p.scale, y, pair_rows, weights, out, nt);
    else
        combine_kernel<K, false><<<grid, block, 0, s>>>(p.T, p.H, p.scale, y, pair_rows, weights, out, nt);
    return hipGetLastError();
}

// Sublayer epilogue fused into the combine ("Welcome Beam: a 501B open model
// you can own, customize, and scale", section "Residual Stream": every
// sublayer output is normalised; step s of the stream adds it with weight
// 1/sqrt(s) and keeps the stream with weight sqrt((s-1)/s); the norms run in
// FP32).  The norm is RMSNorm with a per-channel gain.  The combined row o
// stays in registers (NC float4 chunks per thread) between the sum of squares
// and the update, so it never goes to memory.  The sum of squares is reduced
// in a fixed order: per thread over its chunks, a shuffle tree in each wave,
// then the waves in index order.  The workgroup is a whole number of waves
// (blockDim.x), each thread holding at most NC chunks.
template <int K, int NC>
__global__ __launch_bounds__(kCombineMaxThreads) void combine_residual_kernel(
    int64_t T, int H, float scale, const float* __restrict__ y,
    const int32_t* __restrict__ pair_rows, const float* __restrict__ weights,
    const float* __restrict__ gain, float eps, float wa, float wb, float* __restrict__ res,
    bool nt) {
    __shared__ float s_part[kCombineMaxThreads / 64];
    const int nth = blockDim.x;
    const int64_t t = blockIdx.x;
    int32_t row[K];
    float w[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        row[j] = pair_rows[t * K + j];
        w[j] = weights[t * K + j];
    }
    const int nv = H >> 2;
    float4 o[NC];
    float ss = 0.0f;
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = threadIdx.x + i * nth;
        o[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (c < nv) {
            float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int j = 0; j < K; ++j) {
                if (row[j] < 0) continue;
                const float4 v = load4(y + static_cast<int64_t>(row[j]) * H + 4 * c, nt);
                acc.x = acc.x + w[j] * v.x;
                acc.y = acc.y + w[j] * v.y;
                acc.z = acc.z + w[j] * v.z;
                acc.w = acc.w + w[j] * v.w;
            }
            acc.x *= scale;
            acc.y *= scale;
            acc.z *= scale;
            acc.w *= scale;
            o[i] = acc;
            ss = ss + acc.x * acc.x;
            ss = ss + acc.y * acc.y;
            ss = ss + acc.z * acc.z;
            ss = ss + acc.w * acc.w;
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss = ss + __shfl_xor(ss, off);
    if ((threadIdx.x & 63) == 0) s_part[threadIdx.x >> 6] = ss;
    __syncthreads();
    float tot = s_part[0];
    for (int i = 1; i < (nth >> 6); ++i) tot = tot + s_part[i];
    const float inv = 1.0f / sqrtf(tot / static_cast<float>(H) + eps);
    float4* r4 = reinterpret_cast<float4*>(res + t * H);
    const float4* g4 = reinterpret_cast<const float4*>(gain);
#pragma unroll
    for (int i = 0; i < NC; ++i) {
        const int c = threadIdx.x + i * nth;
        if (c < nv) {
            const float4 g = g4[c];
            float4 r = r4[c];
            r.x = wa * r.x + wb * ((o[i].x * inv) * g.x);
            r.y = wa * r.y + wb * ((o[i].y * inv) * g.y);
            r.z = wa * r.z + wb * ((o[i].z * inv) * g.z);
            r.w = wa * r.w + wb * ((o[i].w * inv) * g.w);
            r4[c] = r;
        }
    }
}

template <int K>
hipError_t launch_residual_k(const Problem& p, const float* y, const int32_t* pair_rows,
                             const float* weights, const float* gain, float eps, float wa,
                             float wb, float* res, hipStream_t s) {
    // fewer tokens than compute units: the combine's wide workgroups (10.3 ->
    // 6.4 us at 128 tokens); otherwise 256 threads, whose shorter wait at the
    // barrier wins with many tokens (640 were 8% slower at 8192)
    const int threads = p.T < kWideBelowTokens ? combine_threads(p.H) : kThreads;
    const dim3 grid(static_cast<unsigned>(p.T)), block(threads);
    const int chunks = (p.H / 4 + threads - 1) / threads;
    const bool nt = p.T * p.k * static_cast<int64_t>(p.H) * 4 > kStreamBytes;
#define MOE_RES(NC)                                                                       \
    combine_residual_kernel<K, NC><<<grid, block, 0, s>>>(p.T, p.H, p.scale, y, pair_rows, \
                                                          weights, gain, eps, wa, wb, res, nt)
    if (chunks <= 1) MOE_RES(1);
    else if (chunks <= 2) MOE_RES(2);
    else if (chunks <= 4) MOE_RES(4);
    else if (chunks <= 8) MOE_RES(8);
    else if (chunks <= kResidualMaxChunks) MOE_RES(16);
    else return hipErrorInvalidValue;
#undef MOE_RES
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine(const Problem& p, const float* y, const int32_t* pair_rows,
                          const float* weights, void* out, bool out_bf16, hipStream_t s) {
    switch (p.k) {
#define MOE_CASE(K) \
    case K: return launch_k<K>(p, y, pair_rows, weights, out, out_bf16, s);
        MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7)
        MOE_CASE(8) MOE_CASE(9) MOE_CASE(10) MOE_CASE(11) MOE_CASE(12) MOE_CASE(13)
        MOE_CASE(14) MOE_CASE(15) MOE_CASE(16)
#undef MOE_CASE
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_combine_residual(const Problem& p, const float* y, const int32_t* pair_rows,
                                   const float* weights, const float* gain, float eps,
                                   float wa, float wb, float* res, hipStream_t s) {
    switch (p.k) {
#define MOE_CASE(K) \
    case K: return launch_residual_k<K>(p, y, pair_rows, weights, gain, eps, wa, wb, res, s);
        MOE_CASE(1) MOE_CASE(2) MOE_CASE(3) MOE_CASE(4) MOE_CASE(5) MOE_CASE(6) MOE_CASE(7)
        MOE_CASE(8) MOE_CASE(9) MOE_CASE(10) MOE_CASE(11) MOE_CASE(12) MOE_CASE(13)
        MOE_CASE(14) MOE_CASE(15) MOE_CASE(16)
#undef MOE_CASE
        default: return hipErrorInvalidValue;
    }
}

}  // namespace moe
