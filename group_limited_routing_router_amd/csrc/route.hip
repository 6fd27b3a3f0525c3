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
// route_kernel (batches above 512 tokens): one workgroup owns up to 16*MB
// tokens and all E <= 256 experts.  The
// logits x . w_router^T are a small dense contraction with bf16 inputs and
// fp32 accumulation, so they run on 16x16x32 bf16 MFMA.  The hidden dimension
// is walked 64 at a time: the workgroup loads the router-weight tile (256
// experts x 128 bytes) and the token tile with coalesced 16-byte loads, a
// few steps ahead into registers, writes the current step to LDS and every
// wave reads its MFMA operands from there (loading MFMA operands straight
// from memory would give every lane of a quad its own row and cache access).
// Each wave owns a set of 16-expert blocks and accumulates its logits over
// the steps in order.  Scores never leave LDS: group ranking and the top-k
// run in the same kernel, one wave per token, with the k picks done as k
// wave-wide arg-max reductions.
//
// route_small_kernel (up to 512 tokens): one workgroup per token or two,
// logits as per-lane bf16 dot products over register-held token chunks and
// a butterfly sum over the wave (see the kernel); the same selection.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kMaxE = 256;
constexpr int kMaxK = 16;
constexpr int kRowBytes = 128;          // one 64-wide step of a bf16 row
constexpr int kWTile = kMaxE * kRowBytes;  // router-weight tile of one step (32 KB)

// LDS byte offset of 16-byte chunk c of row r in a staged tile: chunks are
// XOR-swizzled so the 16 rows of one MFMA operand read hit distinct banks.
__device__ __forceinline__ int stage_off(int r, int c) {
    return r * kRowBytes + ((c ^ ((r >> 1) & 7)) << 4);
}

// Group-limited top-k of the scores of TT tokens in LDS (rows of s_score; row
// tt is token tok0 + tt, rows at or past tpw or T are ignored): group score =
// sum of the group's two best scores, the TG best groups kept (ties to the
// lower index), then one wave per token picks the k best experts of the kept
// groups as k wave-wide arg-max reductions (ties to the lower index) and
// writes ids and weights (the scores normalised to sum to one).  s_gscore and
// s_kept are LDS scratch; NT threads take part, all of them must call.
template <int TT, int NT>
__device__ __forceinline__ void select_topk(float (*s_score)[kMaxE + 4], float (*s_gscore)[kMaxE],
                                            unsigned char (*s_kept)[kMaxE], int64_t tok0, int tpw,
                                            int64_t T, int E, int G, int TG, int k,
                                            int32_t* __restrict__ ids, float* __restrict__ weights) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // ---- group scores: sum of each group's two best scores ----
    const int gs = E / G;
    for (int item = tid; item < TT * G; item += NT) {
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
    for (int item = tid; item < TT * G; item += NT) {
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
    for (int tt = wave; tt < tpw; tt += NT / kWave) {
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
            // wave arg-max under (score desc, index asc), a total order, so
            // any reduction tree gives the same pick: DPP within each row of
            // 16 lanes (swap neighbours, swap pairs, mirror halves, mirror
            // the row: every lane of a row ends with the row's best), then
            // the four rows combined from one lane each
            auto take = [&](float ov, int oe) {  // branch-free (selects)
                const bool t = (ov > bv) | ((ov == bv) & (oe < be));
                bv = t ? ov : bv;
                be = t ? oe : be;
            };
            auto dpp_step = [&](auto ctrl_c) {
                constexpr int CTRL = decltype(ctrl_c)::value;
                const int ovb = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bv), CTRL, 0xF, 0xF, false);
                const int oe = __builtin_amdgcn_update_dpp(0, be, CTRL, 0xF, 0xF, false);
                take(__builtin_bit_cast(float, ovb), oe);
            };
            dpp_step(std::integral_constant<int, 0xB1>{});   // quad_perm [1, 0, 3, 2]
            dpp_step(std::integral_constant<int, 0x4E>{});   // quad_perm [2, 3, 0, 1]
            dpp_step(std::integral_constant<int, 0x141>{});  // row_half_mirror
            dpp_step(std::integral_constant<int, 0x140>{});  // row_mirror
            float sv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 0));
            int se = __builtin_amdgcn_readlane(be, 0);
#pragma unroll
            for (int r = 1; r < 4; ++r) {
                const float ov = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 16 * r));
                const int oe = __builtin_amdgcn_readlane(be, 16 * r);
                const bool t = (ov > sv) | ((ov == sv) & (oe < se));
                sv = t ? ov : sv;
                se = t ? oe : se;
            }
            bv = sv;
            be = se;
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

// NW waves; a workgroup owns tpw <= TT = 16 * MB tokens (with few tokens a
// workgroup takes fewer than 16 so that more compute units share the work;
// MFMA rows past tpw repeat a valid row and are dropped).  D: steps loaded
// ahead into registers.
template <int MB, int NW, int D>
__global__ __launch_bounds__(64 * NW) void route_kernel(
    int64_t T, int H, int E, int G, int TG, int k, int tpw, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ wr, const float* __restrict__ bias, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
    constexpr int NT = 64 * NW;
    constexpr int TT = 16 * MB;
    constexpr int BPW = kMaxE / 16 / NW;          // 16-expert blocks per wave
    constexpr int XTILE = TT * kRowBytes;
    constexpr int STAGE = kWTile + XTILE;
    constexpr int WL = kWTile / 16 / NT;          // weight loads per thread and step
    constexpr int XL = (TT * 8 + NT - 1) / NT;    // token loads per thread and step
    static_assert(WL * 16 * NT == kWTile, "whole weight tile per step");
    struct Gather {                               // the loads of one step (ring of D)
        u32x4 w[WL];
        u32x4 x[XL];
    };
    __shared__ __attribute__((aligned(16))) unsigned char s_stage[2][STAGE];
    __shared__ float s_score[TT][kMaxE + 4];
    // group scores and kept flags reuse the staging area once the logits are done
    static_assert(TT * kMaxE * 4 + TT * kMaxE <= 2 * STAGE, "selection scratch fits");
    float (*s_gscore)[kMaxE] = reinterpret_cast<float (*)[kMaxE]>(&s_stage[0][0]);
    unsigned char (*s_kept)[kMaxE] =
        reinterpret_cast<unsigned char (*)[kMaxE]>(&s_stage[0][0] + TT * kMaxE * 4);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave
    const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * tpw;

    // ---- coalesced load addressing: eight threads per 128-byte row ----
    const uint16_t* wsrc[WL];
    int wdst[WL];
#pragma unroll
    for (int j = 0; j < WL; ++j) {
        const int q = j * NT + tid;
        const int r = q >> 3, c = q & 7;
        const int e = r < E ? r : E - 1;  // rows past the last expert repeat it; dropped
        wsrc[j] = wr + static_cast<int64_t>(e) * H + c * 8;
        wdst[j] = stage_off(r, c);
    }
    const uint16_t* xsrc[XL];
    int xdst[XL];
#pragma unroll
    for (int j = 0; j < XL; ++j) {
        const int q = j * NT + tid;
        const int r = (q >> 3) < TT ? (q >> 3) : TT - 1;
        const int c = q & 7;
        int64_t t = tok0 + (r < tpw ? r : tpw - 1);
        if (t > T - 1) t = T - 1;  // padded rows read a valid row; results dropped
        xsrc[j] = x + t * H + c * 8;
        xdst[j] = (q >> 3) < TT ? kWTile + stage_off(r, c) : -1;
    }
    const int nsteps = H >> 6;
    auto gather = [&](Gather& g, int st) {
        const int off = (st < nsteps ? st : nsteps - 1) * 64;  // past the end: repeat
#pragma unroll
        for (int j = 0; j < WL; ++j) g.w[j] = ld16(wsrc[j] + off);
#pragma unroll
        for (int j = 0; j < XL; ++j) g.x[j] = ld16(xsrc[j] + off);
    };
    auto put = [&](const Gather& g, int buf) {
        unsigned char* base = &s_stage[buf][0];
#pragma unroll
        for (int j = 0; j < WL; ++j) *reinterpret_cast<u32x4*>(base + wdst[j]) = g.w[j];
#pragma unroll
        for (int j = 0; j < XL; ++j)
            if (xdst[j] >= 0) *reinterpret_cast<u32x4*>(base + xdst[j]) = g.x[j];
    };

    // ---- logits: this wave's expert blocks wave, wave + NW, ... ----
    f32x4 acc[BPW][MB];
#pragma unroll
    for (int b = 0; b < BPW; ++b)
#pragma unroll
        for (int m = 0; m < MB; ++m) acc[b][m] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int r16 = lane & 15;
    const int q = lane >> 4;  // which 8-element k chunk of a 32-wide MFMA step
    auto compute = [&](int buf) {
        const unsigned char* base = &s_stage[buf][0];
#pragma unroll
        for (int h = 0; h < 2; ++h) {  // two 32-wide MFMA steps per 64-wide step
            const int c = h * 4 + q;
            bf16x8 a[MB], b[BPW];
#pragma unroll
            for (int m = 0; m < MB; ++m)
                a[m] = *reinterpret_cast<const bf16x8*>(base + kWTile + stage_off(m * 16 + r16, c));
#pragma unroll
            for (int bb = 0; bb < BPW; ++bb)
                b[bb] = *reinterpret_cast<const bf16x8*>(
                    base + stage_off((wave + NW * bb) * 16 + r16, c));
#pragma unroll
            for (int bb = 0; bb < BPW; ++bb)
#pragma unroll
                for (int m = 0; m < MB; ++m) acc[bb][m] = mfma16(a[m], b[bb], acc[bb][m]);
        }
    };
    {
        Gather ring[D];
#pragma unroll
        for (int d = 0; d < D; ++d) gather(ring[d], d);
        // step st: stage the loads of step st, refill their registers with step
        // st + D, then run the step's MFMAs; two LDS buffers alternate
        for (int st0 = 0; st0 < nsteps; st0 += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                const int st = st0 + d;
                if (st < nsteps) {  // uniform
                    put(ring[d], st & 1);
                    __syncthreads();
                    gather(ring[d], st + D);
                    compute(st & 1);
                }
            }
        }
    }
    __syncthreads();  // staging buffers are reused below

    // ---- bias and sigmoid into s_score ----
#pragma unroll
    for (int bb = 0; bb < BPW; ++bb) {
        const int e = (wave + NW * bb) * 16 + r16;
        if (e >= E) continue;
        const float be = bias ? bias[e] : 0.0f;
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) s_score[m * 16 + q * 4 + i][e] = sigmoid_f32(acc[bb][m][i] + be);
    }
    __syncthreads();

    select_topk<TT, NT>(s_score, s_gscore, s_kept, tok0, tpw, T, E, G, TG, k, ids, weights);
}

// Few tokens (decode batches): no MFMA (one token would fill one of its
// sixteen rows) and no LDS staging.  Lane l of every wave holds the tokens'
// 16-byte hidden chunks l, l + 64, ... (8 values each, XC chunks) in
// registers.  Wave w takes experts e_begin + w, e_begin + w + NW, ...: it
// reads an expert's router row as whole 1-KB pieces (lane l reads chunk l of
// each piece), accumulates the bf16 products of its chunks in fp32 with
// two-wide dot instructions in chunk order, and sums the 64 lane partials
// with a butterfly (every lane ends with the same sum).  Lane 0 hands
// sigmoid(sum + bias) to out(t, e, score).  Every kernel below computes a
// score with this one function, so they agree bit for bit.
template <int TPW, int XC>
__device__ __forceinline__ void load_token_chunks(u32x4 (&xr)[TPW][XC], const uint16_t* __restrict__ x,
                                                  int64_t T, int H, int64_t tok0, int lane) {
    const int nch = H >> 3;
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
        int64_t tok = tok0 + t;
        if (tok > T - 1) tok = T - 1;  // rows past the batch repeat its last token; dropped
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int c = i * 64 + lane;
            xr[t][i] = c < nch ? ld16(x + tok * H + c * 8) : u32x4{0u, 0u, 0u, 0u};
        }
    }
}

template <int NW, int TPW, int XC, typename Out>
__device__ __forceinline__ void small_scores(const u32x4 (&xr)[TPW][XC], const uint16_t* __restrict__ wr,
                                             const float* __restrict__ bias, int H, int e_begin,
                                             int e_end, int lane, int wave, Out out) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const int nch = H >> 3;  // 16-byte chunks per row (<= 64 XC)
    auto dot8 = [&](const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            // elements copied out first: a bit cast of a vector element in
            // place would read element 0
            const uint32_t aj = a[j], bj = b[j];
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, aj),
                                                  __builtin_bit_cast(bf16x2, bj), acc, false);
        }
        return acc;
    };
    // FULL: every lane has all XC chunks (H = 512 XC), no per-lane guards
    auto experts = [&](auto full_c) {
        constexpr bool FULL = decltype(full_c)::value;
#pragma unroll 2
        for (int e = e_begin + wave; e < e_end; e += NW) {
            const uint16_t* row = wr + static_cast<int64_t>(e) * H;
            u32x4 w[XC];
#pragma unroll
            for (int i = 0; i < XC; ++i) {
                const int c = i * 64 + lane;
                w[i] = (FULL || c < nch) ? ld16(row + c * 8) : u32x4{0u, 0u, 0u, 0u};
            }
            float acc[TPW];
#pragma unroll
            for (int t = 0; t < TPW; ++t) {
                acc[t] = 0.0f;
#pragma unroll
                for (int i = 0; i < XC; ++i) acc[t] = dot8(xr[t][i], w[i], acc[t]);
#pragma unroll
                for (int off = 32; off >= 1; off >>= 1) acc[t] = acc[t] + __shfl_xor(acc[t], off);
            }
            if (lane == 0) {
                const float be = bias ? bias[e] : 0.0f;
#pragma unroll
                for (int t = 0; t < TPW; ++t) out(t, e, sigmoid_f32(acc[t] + be));
            }
        }
    };
    if (nch == 64 * XC)
        experts(std::true_type{});
    else
        experts(std::false_type{});
}

// A workgroup owns TPW tokens and all experts; then select_topk.
template <int NW, int TPW, int XC>
__global__ __launch_bounds__(64 * NW) void route_small_kernel(
    int64_t T, int H, int E, int G, int TG, int k, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ wr, const float* __restrict__ bias, int32_t* __restrict__ ids,
    float* __restrict__ weights) {
    __shared__ float s_score[TPW][kMaxE + 4];
    __shared__ float s_gscore[TPW][kMaxE];
    __shared__ unsigned char s_kept[TPW][kMaxE];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * TPW;
    u32x4 xr[TPW][XC];
    load_token_chunks<TPW, XC>(xr, x, T, H, tok0, lane);
    small_scores<NW, TPW, XC>(xr, wr, bias, H, 0, E, lane, wave,
                              [&](int t, int e, float v) { s_score[t][e] = v; });
    __syncthreads();
    select_topk<TPW, 64 * NW>(s_score, s_gscore, s_kept, tok0, TPW, T, E, G, TG, k, ids, weights);
}

// The same scores with the experts split over workgroups (tokens
// [TPW blockIdx.x, +TPW), experts [es blockIdx.y, +es)), written to scores
// [T, E] in memory; route_select_kernel then selects.  Each workgroup reads
// only its slice of the router weight, once for its TPW tokens.
template <int NW, int TPW, int XC>
__global__ __launch_bounds__(64 * NW) void route_scores_kernel(
    int64_t T, int H, int E, int es, const uint16_t* __restrict__ x,
    const uint16_t* __restrict__ wr, const float* __restrict__ bias, float* __restrict__ scores) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * TPW;
    const int e0 = blockIdx.y * es;
    const int e1 = e0 + es < E ? e0 + es : E;
    u32x4 xr[TPW][XC];
    load_token_chunks<TPW, XC>(xr, x, T, H, tok0, lane);
    small_scores<NW, TPW, XC>(xr, wr, bias, H, e0, e1, lane, wave, [&](int t, int e, float v) {
        if (tok0 + t < T) scores[(tok0 + t) * E + e] = v;
    });
}

// select_topk over TT tokens' rows of scores [T, E]; one wave per token.
template <int TT>
__global__ __launch_bounds__(64 * TT) void route_select_kernel(
    int64_t T, int E, int G, int TG, int k, const float* __restrict__ scores,
    int32_t* __restrict__ ids, float* __restrict__ weights) {
    __shared__ float s_score[TT][kMaxE + 4];
    __shared__ float s_gscore[TT][kMaxE];
    __shared__ unsigned char s_kept[TT][kMaxE];
    const int64_t tok0 = static_cast<int64_t>(blockIdx.x) * TT;
    for (int i = threadIdx.x; i < TT * E; i += 64 * TT) {
        const int tt = i / E, e = i - tt * E;
        int64_t t = tok0 + tt;
        if (t > T - 1) t = T - 1;  // rows past the batch: dropped by select_topk
        s_score[tt][e] = scores[t * E + e];
    }
    __syncthreads();
    select_topk<TT, 64 * TT>(s_score, s_gscore, s_kept, tok0, TT, T, E, G, TG, k, ids, weights);
}

template <int XC>
void launch_route_split(const Problem& p, const uint16_t* x, const uint16_t* w_router,
                        const float* bias, int32_t* ids, float* weights, float* scores,
                        hipStream_t s) {
    constexpr int kSlice = 32, kSelTok = 4, kTpw = 4;
    const dim3 grid(static_cast<unsigned>((p.T + kTpw - 1) / kTpw),
                    static_cast<unsigned>((p.E + kSlice - 1) / kSlice));
    route_scores_kernel<8, kTpw, XC><<<grid, dim3(512), 0, s>>>(p.T, p.H, p.E, kSlice, x, w_router,
                                                                bias, scores);
    const int64_t g2 = (p.T + kSelTok - 1) / kSelTok;
    route_select_kernel<kSelTok><<<dim3(static_cast<unsigned>(g2)), dim3(64 * kSelTok), 0, s>>>(
        p.T, p.E, p.G, p.TG, p.k, scores, ids, weights);
}

template <int TPW, int XC>
void launch_route_small(const Problem& p, const uint16_t* x, const uint16_t* w_router,
                        const float* bias, int32_t* ids, float* weights, hipStream_t s) {
    const int64_t grid = (p.T + TPW - 1) / TPW;
    route_small_kernel<8, TPW, XC><<<dim3(static_cast<unsigned>(grid)), dim3(512), 0, s>>>(
        p.T, p.H, p.E, p.G, p.TG, p.k, x, w_router, bias, ids, weights);
}

}  // namespace

hipError_t launch_route(const Problem& p, const uint16_t* x, const uint16_t* w_router,
                        const float* bias, int32_t* ids, float* weights, hipStream_t s) {
    const int xc = (p.H / 8 + 63) / 64;  // hidden chunks per lane of the small-batch kernel
    if (p.T <= 512 && xc <= 16) {
        // few tokens: one or two per workgroup, at most 256 workgroups
        if (p.T <= 256) {
            if (xc <= 1) launch_route_small<1, 1>(p, x, w_router, bias, ids, weights, s);
            else if (xc <= 2) launch_route_small<1, 2>(p, x, w_router, bias, ids, weights, s);
            else if (xc <= 4) launch_route_small<1, 4>(p, x, w_router, bias, ids, weights, s);
            else if (xc <= 10) launch_route_small<1, 10>(p, x, w_router, bias, ids, weights, s);
            else launch_route_small<1, 16>(p, x, w_router, bias, ids, weights, s);
        } else {
            if (xc <= 1) launch_route_small<2, 1>(p, x, w_router, bias, ids, weights, s);
            else if (xc <= 2) launch_route_small<2, 2>(p, x, w_router, bias, ids, weights, s);
            else if (xc <= 4) launch_route_small<2, 4>(p, x, w_router, bias, ids, weights, s);
            else if (xc <= 10) launch_route_small<2, 10>(p, x, w_router, bias, ids, weights, s);
            else launch_route_small<2, 16>(p, x, w_router, bias, ids, weights, s);
        }
    } else if (p.T > 8192) {
        // more tokens than one wave of 256 32-token workgroups: 64-token tiles
        // stream the router weight half as often (30% faster at 65536 tokens)
        const int64_t grid = (p.T + 63) / 64;
        route_kernel<4, 8, 6><<<dim3(static_cast<unsigned>(grid)), dim3(512), 0, s>>>(
            p.T, p.H, p.E, p.G, p.TG, p.k, 64, x, w_router, bias, ids, weights);
    } else if (p.T > 4096) {
        // many tokens: 32-token tiles (the router weight is read once per tile;
        // at most 256 workgroups, one per compute unit, where 64-token tiles
        // would leave half of them idle and take 35% longer; at 4096 tokens
        // 16-token tiles fill all 256 and take 82 us against 94 us cold)
        const int64_t grid = (p.T + 31) / 32;
        route_kernel<2, 8, 6><<<dim3(static_cast<unsigned>(grid)), dim3(512), 0, s>>>(
            p.T, p.H, p.E, p.G, p.TG, p.k, 32, x, w_router, bias, ids, weights);
    } else {
        // few tokens: a workgroup takes only as many tokens (a power of two up
        // to 16) as spread the batch over about 256 compute units
        int tpw = 1;
        while (tpw < 16 && (p.T + tpw - 1) / tpw > 256) tpw *= 2;
        const int64_t grid = (p.T + tpw - 1) / tpw;
        route_kernel<1, 16, 4><<<dim3(static_cast<unsigned>(grid)), dim3(1024), 0, s>>>(
            p.T, p.H, p.E, p.G, p.TG, p.k, tpw, x, w_router, bias, ids, weights);
    }
    return hipGetLastError();
}


hipError_t launch_route_scratch(const Problem& p, const uint16_t* x, const uint16_t* w_router,
                                const float* bias, int32_t* ids, float* weights, void* scratch,
                                size_t scratch_bytes, hipStream_t s) {
    const int xc = (p.H / 8 + 63) / 64;
    const size_t need = static_cast<size_t>(p.T) * static_cast<size_t>(p.E) * 4;
    if (p.T > 512 || xc > 16 || scratch == nullptr || scratch_bytes < need)
        return launch_route(p, x, w_router, bias, ids, weights, s);
    float* scores = static_cast<float*>(scratch);
    if (xc <= 1) launch_route_split<1>(p, x, w_router, bias, ids, weights, scores, s);
    else if (xc <= 2) launch_route_split<2>(p, x, w_router, bias, ids, weights, scores, s);
    else if (xc <= 4) launch_route_split<4>(p, x, w_router, bias, ids, weights, scores, s);
    else if (xc <= 10) launch_route_split<10>(p, x, w_router, bias, ids, weights, scores, s);
    else launch_route_split<16>(p, x, w_router, bias, ids, weights, scores, s);
    return hipGetLastError();
}

}  // namespace moe
