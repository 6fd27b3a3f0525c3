// kernels.h -- internal launchers behind the C ABI (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct Problem {
    int64_t T;
    int H, I, E, G, TG, k;
    float scale;
};

// Pairs handled by one block of the counting sort.
constexpr int kPermuteChunk = 4096;

inline int64_t permute_blocks(int64_t pairs) {
    return pairs <= 0 ? 1 : (pairs + kPermuteChunk - 1) / kPermuteChunk;
}

hipError_t launch_route(const Problem& p, const uint16_t* x, const uint16_t* w_router,
                        const float* bias, int32_t* ids, float* weights, hipStream_t s);

// The router with device scratch of at least T*E*4 bytes (unused contents):
// for up to 512 tokens the experts are split over workgroups and the scores
// pass through the scratch (the same scores, bit for bit, as launch_route);
// otherwise, or with too little scratch, launch_route.
hipError_t launch_route_scratch(const Problem& p, const uint16_t* x, const uint16_t* w_router,
                                const float* bias, int32_t* ids, float* weights, void* scratch,
                                size_t scratch_bytes, hipStream_t s);

hipError_t launch_permute(const Problem& p, const int32_t* ids, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_rows, int32_t* block_counts,
                          hipStream_t s);

// sorted_pairs = 0 .. T-1 and offsets = {0, T}: the dispatch of one expert
// that takes every token (a dense layer).
hipError_t launch_identity_dispatch(int64_t T, int32_t* offsets, int32_t* sorted_pairs,
                                    hipStream_t s);

hipError_t launch_expert_ffn(const Problem& p, const uint16_t* x, const int32_t* sorted_pairs,
                             const int32_t* offsets, const uint16_t* w_gate,
                             const uint16_t* w_up, const uint16_t* w_down, uint16_t* h, float* y,
                             hipStream_t s);

// The expert FFN with FP8 E4M3 weights and fp32 per-output-channel scales
// (s_gate/s_up [E,I], s_down [E,H]); x, h and y as in launch_expert_ffn.
hipError_t launch_expert_ffn_fp8(const Problem& p, const uint16_t* x, const int32_t* sorted_pairs,
                                 const int32_t* offsets, const uint8_t* w_gate,
                                 const float* s_gate, const uint8_t* w_up, const float* s_up,
                                 const uint8_t* w_down, const float* s_down, uint16_t* h,
                                 float* y, hipStream_t s);

hipError_t launch_gate_up(const Problem& p, const uint16_t* x, const int32_t* sorted_pairs,
                          const int32_t* offsets, const uint16_t* w_gate, const uint16_t* w_up,
                          uint16_t* h, hipStream_t s);

hipError_t launch_down(const Problem& p, const uint16_t* h, const int32_t* offsets,
                       const uint16_t* w_down, float* y, hipStream_t s);

hipError_t launch_combine(const Problem& p, const float* y, const int32_t* pair_rows,
                          const float* weights, void* out, bool out_bf16, hipStream_t s);

// Combine fused with the post-norm and residual update; the combined row is
// held in registers, at most kResidualMaxChunks float4 chunks per thread of
// 256, i.e. H <= 16384.
constexpr int kResidualMaxChunks = 16;
constexpr int kResidualMaxH = kResidualMaxChunks * 4 * 256;

hipError_t launch_combine_residual(const Problem& p, const float* y, const int32_t* pair_rows,
                                   const float* weights, const float* gain, float eps,
                                   float wa, float wb, float* res, hipStream_t s);

}  // namespace moe
