// permute.hip -- dispatch of (token, slot) pairs to experts.
//
// Each token runs on its k chosen experts ("Welcome Beam: a 501B open model
// you can own, customize, and scale", section "Mixture of Experts": only 8
// experts run per token), so the rows bound for one expert are gathered into
// one contiguous segment.  This is a stable counting sort of the pair ids
// p = t*k + j by expert id, in three launches:
//   1. count:   each block of kPermuteChunk pairs builds an LDS histogram;
//   2. scan:    one workgroup turns the per-block counts into the start of
//               every (expert, block) segment and writes expert_offsets;
//   3. scatter: each block walks its pairs in order, 256 at a time; a pair's
//               place inside its expert is found with wave ballots (match on
//               the expert id bits) plus the counts of the waves before it, so
//               the order is the pair order and no atomics touch the outputs.
// Up to kPermuteChunk pairs (decode batches) one workgroup does all three
// steps in LDS in a single launch, with the same scatter.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxE = 256;

__global__ __launch_bounds__(kThreads) void permute_count_kernel(
    int64_t pairs, int E, const int32_t* __restrict__ ids, int32_t* __restrict__ counts) {
    __shared__ int32_t hist[kMaxE];
    for (int e = threadIdx.x; e < E; e += kThreads) hist[e] = 0;
    __syncthreads();
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kPermuteChunk;
    const int64_t p1 = p0 + kPermuteChunk < pairs ? p0 + kPermuteChunk : pairs;
    for (int64_t p = p0 + threadIdx.x; p < p1; p += kThreads) {
        const int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&hist[e], 1);  // LDS counter; the count is exact
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kThreads)
        counts[static_cast<int64_t>(blockIdx.x) * E + e] = hist[e];
}

// Exclusive prefix sum over tot[0..kThreads) in LDS (inclusive Hillis-Steele
// scan, left in tot); thread e gets the sum of tot[0..e).  Every thread of
// the workgroup calls it, after tot is written and the workgroup synchronised.
__device__ __forceinline__ int32_t exclusive_scan(int32_t* tot, int e) {
    for (int d = 1; d < kThreads; d <<= 1) {
        const int32_t v = (e >= d) ? tot[e - d] : 0;
        __syncthreads();
        tot[e] += v;
        __syncthreads();
    }
    return (e == 0) ? 0 : tot[e - 1];
}

// Places the pairs [p0, p1) in pair order: base[e] holds the first free
// sorted position of expert e and is advanced past each 256-pair step;
// wcount must start at zero (it is zero again on return).  Every thread of
// the workgroup calls it.
__device__ void scatter_pairs(int64_t p0, int64_t p1, int E, const int32_t* __restrict__ ids,
                              int32_t* base, int32_t (*wcount)[kMaxE],
                              int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_rows) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int64_t s = p0; s < p1; s += kThreads) {
        const int64_t p = s + tid;
        int e = (p < p1) ? ids[p] : -1;
        const bool ok = e >= 0 && e < E;
        if (!ok) e = -1;
        // lanes of this wave with the same expert id (9 bits: 8 id bits + valid)
        uint64_t same = __ballot(ok);
        if (!ok) same = ~same;
#pragma unroll
        for (int bit = 0; bit < 8; ++bit) {
            const bool on = (e >> bit) & 1;
            const uint64_t bal = __ballot(on);
            same &= on ? bal : ~bal;
        }
        const int rank = __popcll(same & below);
        const bool leader = ok && rank == 0;
        if (leader) wcount[wave][e] = __popcll(same);
        __syncthreads();
        if (ok) {
            int32_t pos = base[e] + rank;
            for (int w = 0; w < wave; ++w) pos += wcount[w][e];
            sorted_pairs[pos] = static_cast<int32_t>(p);
            pair_rows[p] = pos;
        } else if (p < p1) {
            pair_rows[p] = -1;
        }
        __syncthreads();
        if (leader) {
            atomicAdd(&base[e], wcount[wave][e]);  // LDS; a sum, order-free
            wcount[wave][e] = 0;
        }
        __syncthreads();
    }
}

// counts[b][e] becomes the first sorted position of block b's pairs of
// expert e; offsets[e] the first position of expert e.
__global__ __launch_bounds__(kThreads) void permute_scan_kernel(int nblocks, int E,
                                                                int32_t* __restrict__ counts,
                                                                int32_t* __restrict__ offsets) {
    __shared__ int32_t tot[kThreads];
    const int e = threadIdx.x;
    int32_t run = 0;
    if (e < E) {
        for (int b = 0; b < nblocks; ++b) {
            const int32_t c = counts[static_cast<int64_t>(b) * E + e];
            counts[static_cast<int64_t>(b) * E + e] = run;
            run += c;
        }
    }
    tot[e] = (e < E) ? run : 0;
    __syncthreads();
    const int32_t start = exclusive_scan(tot, e);
    if (e < E) {
        offsets[e] = start;
        for (int b = 0; b < nblocks; ++b) counts[static_cast<int64_t>(b) * E + e] += start;
    }
    if (e == E - 1) offsets[E] = tot[e];
}

__global__ __launch_bounds__(kThreads) void permute_scatter_kernel(
    int64_t pairs, int E, const int32_t* __restrict__ ids, const int32_t* __restrict__ counts,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_rows) {
    __shared__ int32_t base[kMaxE];
    __shared__ int32_t wcount[kThreads / kWave][kMaxE];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kThreads) {
        base[e] = counts[static_cast<int64_t>(blockIdx.x) * E + e];
#pragma unroll
        for (int w = 0; w < kThreads / kWave; ++w) wcount[w][e] = 0;
    }
    __syncthreads();
    const int64_t p0 = static_cast<int64_t>(blockIdx.x) * kPermuteChunk;
    const int64_t p1 = p0 + kPermuteChunk < pairs ? p0 + kPermuteChunk : pairs;
    scatter_pairs(p0, p1, E, ids, base, wcount, sorted_pairs, pair_rows);
}

// All three steps for at most kPermuteChunk pairs in one workgroup: the
// histogram, its scan into expert_offsets and the scatter, all in LDS.
__global__ __launch_bounds__(kThreads) void permute_single_kernel(
    int64_t pairs, int E, const int32_t* __restrict__ ids, int32_t* __restrict__ offsets,
    int32_t* __restrict__ sorted_pairs, int32_t* __restrict__ pair_rows) {
    __shared__ int32_t base[kMaxE];
    __shared__ int32_t tot[kThreads];
    __shared__ int32_t wcount[kThreads / kWave][kMaxE];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += kThreads) {
        base[e] = 0;
#pragma unroll
        for (int w = 0; w < kThreads / kWave; ++w) wcount[w][e] = 0;
    }
    __syncthreads();
    for (int64_t p = tid; p < pairs; p += kThreads) {
        const int e = ids[p];
        if (e >= 0 && e < E) atomicAdd(&base[e], 1);  // LDS counter; the count is exact
    }
    __syncthreads();
    tot[tid] = (tid < E) ? base[tid] : 0;
    __syncthreads();
    const int32_t start = exclusive_scan(tot, tid);
    if (tid < E) {
        offsets[tid] = start;
        base[tid] = start;
    }
    if (tid == E - 1) offsets[E] = tot[tid];
    __syncthreads();
    scatter_pairs(0, pairs, E, ids, base, wcount, sorted_pairs, pair_rows);
}

}  // namespace

hipError_t launch_permute(const Problem& p, const int32_t* ids, int32_t* offsets,
                          int32_t* sorted_pairs, int32_t* pair_rows, int32_t* block_counts,
                          hipStream_t s) {
    const int64_t pairs = p.T * p.k;
    const int64_t nb = permute_blocks(pairs);
    if (nb == 1) {
        permute_single_kernel<<<dim3(1), dim3(kThreads), 0, s>>>(pairs, p.E, ids, offsets,
                                                                 sorted_pairs, pair_rows);
        return hipGetLastError();
    }
    permute_count_kernel<<<dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0, s>>>(pairs, p.E, ids,
                                                                                block_counts);
    permute_scan_kernel<<<dim3(1), dim3(kThreads), 0, s>>>(static_cast<int>(nb), p.E, block_counts,
                                                           offsets);
    permute_scatter_kernel<<<dim3(static_cast<unsigned>(nb)), dim3(kThreads), 0, s>>>(
        pairs, p.E, ids, block_counts, sorted_pairs, pair_rows);
    return hipGetLastError();
}

namespace {

// The dispatch of a dense layer: one expert owns every row, row q is token q.
__global__ __launch_bounds__(kThreads) void identity_dispatch_kernel(int64_t T, int32_t* offsets,
                                                                     int32_t* sorted_pairs) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (i < T) sorted_pairs[i] = static_cast<int32_t>(i);
    if (i == 0) {
        offsets[0] = 0;
        offsets[1] = static_cast<int32_t>(T);
    }
}

}  // namespace

hipError_t launch_identity_dispatch(int64_t T, int32_t* offsets, int32_t* sorted_pairs,
                                    hipStream_t s) {
    const int64_t grid = T > 0 ? (T + kThreads - 1) / kThreads : 1;
    identity_dispatch_kernel<<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s>>>(
        T, offsets, sorted_pairs);
    return hipGetLastError();
}

}  // namespace moe
