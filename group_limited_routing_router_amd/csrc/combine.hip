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
// lane.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;

template <int K, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void combine_kernel(int64_t T, int H, float scale,
                                                           const float* __restrict__ y,
                                                           const int32_t* __restrict__ pair_rows,
                                                           const float* __restrict__ weights,
                                                           void* __restrict__ out) {
    const int64_t t = blockIdx.x;
    int32_t row[K];
    float w[K];
#pragma unroll
    for (int j = 0; j < K; ++j) {
        row[j] = pair_rows[t * K + j];
        w[j] = weights[t * K + j];
    }
    const int nv = H >> 2;  // float4 chunks per row
    for (int c = threadIdx.x; c < nv; c += kThreads) {
        float4 v[K];
#pragma unroll
        for (int j = 0; j < K; ++j) {
            if (row[j] >= 0)
                v[j] = reinterpret_cast<const float4*>(y + static_cast<int64_t>(row[j]) * H)[c];
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
            reinterpret_cast<float4*>(static_cast<float*>(out) + t * H)[c] = acc;
        }
    }
}

template <int K>
hipError_t launch_k(const Problem& p, const float* y, const int32_t* pair_rows,
                    const float* weights, void* out, bool out_bf16, hipStream_t s) {
    const dim3 grid(static_cast<unsigned>(p.T)), block(kThreads);
    if (out_bf16)
        combine_kernel<K, true><<<grid, block, 0, s>>>(p.T, p.H, p.scale, y, pair_rows, weights, out);
    else
        combine_kernel<K, false><<<grid, block, 0, s>>>(p.T, p.H, p.scale, y, pair_rows, weights, out);
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

}  // namespace moe
