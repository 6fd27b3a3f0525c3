// route.hip -- router scores and group-limited top-k selection.
//
// Method ("Welcome Beam: a 501B open model you can own, customize, and
// scale", section "Mixture of Experts"): every expert gets a sigmoid score;
// experts form G groups of E/G consecutive indices; a group ranks by the sum
// of its two best scores; the TG best groups are kept; the k best experts of
// the kept groups are chosen and their scores normalised to sum to one.  The
// router runs in FP32 (same page, section "Residual Stream").  Ties go to the
// lower index.
//
// One workgroup of 8 waves owns 16*MB tokens and all E <= 256 experts.  The
// logits x . w_router^T are a small dense contraction with bf16 inputs and
// fp32 accumulation, so they run on 16x16x32 bf16 MFMA: wave w covers the
// expert quarter (w % 4) over half (w / 4) of the hidden dimension, and the
// two halves meet in LDS.  Scores never leave LDS: group ranking and the
// top-k run in the same kernel, one wave per token, with the k picks done as
// k wave-wide arg-max reductions.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRouteThreads = 512;
constexpr int kMaxE = 256;
constexpr int kMaxK = 16;

template <int MB>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    int64_t T, int H, int E, int G, int TG, int k, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ wr, const float* __restrict__ bias, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
    constexpr int TT = 16 * MB;
    __shared__ float s_score[TT][kMaxE + 4];
    __shared__ float s_gscore[TT][kMaxE];      // group score (G <= E <= 256)
    __shared__ unsigned char s_kept[TT][kMaxE];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int eq = wave & 3;      // expert quarter
    const int kh = wave >> 2;     // hidden half
    const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * TT;

    // ---- logits: D[token][expert] over this wave's hidden half ----
    const int nblk = (E + 15) >> 4;  // 16-expert blocks
    f32x4 acc[4][MB];
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int r16 = lane & 15;
    const int q = lane >> 4;  // which 16-element k chunk of a 64-wide step
    const uint16_t* xrow[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        int64_t t = tok0 + m * 16 + r16;
        if (t > T - 1) t = T - 1;  // padded rows read a valid row; results dropped
        xrow[m] = x + t * H;
    }
    const uint16_t* wrow[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        int e = (eq + 4 * b) * 16 + r16;
        if (e > E - 1) e = E - 1;
        wrow[b] = wr + static_cast<int64_t>(e) * H;
    }
    const int half = H >> 1;
    const int k0 = kh * half;
    for (int kk = k0; kk < k0 + half; kk += 64) {
        const int off = kk + q * 16;
        bf16x8 a0[MB], a1[MB];
#pragma unroll
        for (int m = 0; m < MB; ++m) {
            a0[m] = as_bf16x8(ld16(xrow[m] + off));
            a1[m] = as_bf16x8(ld16(xrow[m] + off + 8));
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            if (eq + 4 * b >= nblk) break;
            bf16x8 b0 = as_bf16x8(ld16(wrow[b] + off));
            bf16x8 b1 = as_bf16x8(ld16(wrow[b] + off + 8));
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                acc[b][m] = mfma16(a0[m], b0, acc[b][m]);
                acc[b][m] = mfma16(a1[m], b1, acc[b][m]);
            }
        }
    }

    // ---- meet the two halves in LDS, add bias, sigmoid ----
    if (kh == 1) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int e = (eq + 4 * b) * 16 + r16;
            if (eq + 4 * b >= nblk || e >= E) continue;
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) s_score[m * 16 + q * 4 + i][e] = acc[b][m][i];
        }
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int e = (eq + 4 * b) * 16 + r16;
            if (eq + 4 * b >= nblk || e >= E) continue;
            const float be = bias ? bias[e] : 0.0f;
#pragma unroll
            for (int m = 0; m < MB; ++m)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float& s = s_score[m * 16 + q * 4 + i][e];
                    s = sigmoid_f32((acc[b][m][i] + s) + be);
                }
        }
    }
    __syncthreads();

    // ---- group scores: sum of each group's two best scores ----
    const int gs = E / G;
    for (int item = tid; item < TT * G; item += kRouteThreads) {
        const int tt = item / G, g = item - tt * G;
        const float* s = &s_score[tt][g * gs];
        float t1 = s[0], t2 = -1.0f;
        for (int i = 1; i < gs; ++i) {
            const float v = s[i];
            if (v > t1) {
                t2 = t1;
                t1 = v;
            } else if (v > t2) {
                t2 = v;
            }
        }
        s_gscore[tt][g] = gs == 1 ? t1 : t1 + t2;
    }
    __syncthreads();
    // ---- kept groups: rank under (score desc, index asc) below TG ----
    for (int item = tid; item < TT * G; item += kRouteThreads) {
        const int tt = item / G, g = item - tt * G;
        const float mine = s_gscore[tt][g];
        int rank = 0;
        for (int o = 0; o < G; ++o) {
            const float v = s_gscore[tt][o];
            rank += (v > mine) || (v == mine && o < g);
        }
        s_kept[tt][g] = rank < TG;
    }
    __syncthreads();

    // ---- top-k among kept groups: one wave per token ----
    for (int tt = wave; tt < TT; tt += kRouteThreads / kWave) {
        const int64_t t = tok0 + tt;
        if (t >= T) break;  // wave-uniform; no barrier follows
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int e = lane + 64 * i;
            v[i] = (e < E && s_kept[tt][e / gs]) ? s_score[tt][e] : -1.0f;
        }
        float pick_v[kMaxK];
        int pick_e[kMaxK];
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= k) break;
            float bv = v[0];
            int be = lane;
#pragma unroll
            for (int i = 1; i < 4; ++i)
                if (v[i] > bv) {
                    bv = v[i];
                    be = lane + 64 * i;
                }
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) {
                const float ov = __shfl_xor(bv, off);
                const int oe = __shfl_xor(be, off);
                if (ov > bv || (ov == bv && oe < be)) {
                    bv = ov;
                    be = oe;
                }
            }
            pick_v[j] = bv;
            pick_e[j] = be;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (lane + 64 * i == be) v[i] = -2.0f;
        }
        float sum = 0.0f;
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= k) break;
            sum = sum + pick_v[j];
        }
#pragma unroll
        for (int j = 0; j < kMaxK; ++j) {
            if (j >= k) break;
            if (lane == j) {
                ids[t * k + j] = pick_e[j];
                weights[t * k + j] = pick_v[j] / sum;
            }
        }
    }
}

}  // namespace

hipError_t launch_route(const Problem& p, const uint16_t* x, const uint16_t* w_router,
                        const float* bias, int32_t* ids, float* weights, hipStream_t s) {
    if (p.T >= 4096) {
        const int64_t grid = (p.T + 31) / 32;
        route_kernel<2><<<dim3(static_cast<unsigned>(grid)), dim3(kRouteThreads), 0, s>>>(
            p.T, p.H, p.E, p.G, p.TG, p.k, x, w_router, bias, ids, weights);
    } else {
        const int64_t grid = (p.T + 15) / 16;
        route_kernel<1><<<dim3(static_cast<unsigned>(grid)), dim3(kRouteThreads), 0, s>>>(
            p.T, p.H, p.E, p.G, p.TG, p.k, x, w_router, bias, ids, weights);
    }
    return hipGetLastError();
}

}  // namespace moe
