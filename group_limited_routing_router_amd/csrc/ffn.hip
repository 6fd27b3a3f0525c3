// ffn.hip -- the experts: two grouped bf16 MFMA GEMMs over the sorted pairs.
//
// Each expert is a SwiGLU MLP with intermediate size I ("Welcome Beam: a 501B
// open model you can own, customize, and scale", section "Mixture of
// Experts"); the SwiGLU product is computed in FP32 (same page, section
// "Residual Stream") and rounded to bf16 before the down projection.
//
//   gate/up:  for expert e and its rows q in [off[e], off[e+1]):
//             h[q, n] = bf16( silu(X_q . Wg[e,n]) * (X_q . Wu[e,n]) ),
//             X_q = x[sorted_pairs[q] / k]  (rows gathered on the fly)
//   down:     y[q, m] = h[q] . Wd[e,m]      (fp32 out)
//
// One kernel template serves both.  A workgroup (4 waves) computes a BM x BN
// tile of one expert: BM sorted rows by BN weight rows.  For gate/up the BN
// weight rows are BN/2 gate rows and the BN/2 up rows of the same output
// columns, so a lane holds gate and up accumulators of the same (row, col)
// and the SwiGLU epilogue needs no data exchange.  Tiles of 64 along K are
// staged through LDS with two buffers; global loads of tile k+1 are in flight
// while the MFMAs of tile k run.  LDS rows are padded by 16 B so the 16-row
// MFMA operand reads hit distinct banks.
//
// The tile list is data-dependent and never read back by the host: the grid
// is an upper bound, every workgroup rebuilds the per-expert tile prefix sum
// from expert_offsets in LDS and maps itself to a tile, and surplus
// workgroups exit.  The mapping is XCD-aware: workgroup b runs on XCD b % 8,
// and each XCD receives one contiguous run of the tile list (expert-major,
// then column tile, then row tile), so the tiles of one expert share its
// gathered activations and, across row tiles, its weight tiles in that XCD's
// L2.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxE = 256;
constexpr int BK = 64;           // K elements per LDS stage
constexpr int LDS_STRIDE = BK + 8;  // bf16 per LDS row (16 B pad)

struct FfnArgs {
    int64_t P;       // pairs (rows of h and y)
    int64_t T;       // tokens (rows of x)
    int k;           // experts per token
    int E;           // experts
    int K;           // reduction length (H for gate/up, I for down)
    int N;           // output columns (I for gate/up, H for down)
    const uint16_t* a_src;   // x [T,H] (gate/up) or h [P,I] (down)
    const int32_t* sorted_pairs;
    const int32_t* offsets;  // [E+1]
    const uint16_t* b0;      // w_gate [E,I,H] or w_down [E,H,I]
    const uint16_t* b1;      // w_up [E,I,H] (gate/up only)
    void* out;               // h [P,I] bf16 (gate/up) or y [P,H] fp32 (down)
};

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATEUP>
__global__ __launch_bounds__(kThreads) void ffn_gemm_kernel(FfnArgs a) {
    static_assert(WAVES_M * WAVES_N == kWaves, "4 waves");
    constexpr int BN_OUT = GATEUP ? BN / 2 : BN;     // output columns per tile
    constexpr int WM = BM / WAVES_M;                  // rows per wave
    constexpr int MB = WM / 16;
    constexpr int WN_OUT = BN_OUT / WAVES_N;          // output columns per wave
    constexpr int NB = WN_OUT / 16;
    static_assert(MB >= 1 && NB >= 1, "tile too small");
    constexpr int A_CHUNKS = BM * (BK / 8);           // 16-byte chunks per stage
    constexpr int B_CHUNKS = BN * (BK / 8);
    constexpr int A_ITERS = (A_CHUNKS + kThreads - 1) / kThreads;
    constexpr int B_ITERS = B_CHUNKS / kThreads;
    static_assert(B_CHUNKS % kThreads == 0, "B tile");

    __shared__ __attribute__((aligned(16))) uint16_t s_a[2][BM * LDS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t s_b[2][BN * LDS_STRIDE];
    __shared__ int32_t s_off[kMaxE + 1];
    __shared__ int32_t s_tstart[kMaxE + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    // ---- tile schedule from expert_offsets ----
    const int E = a.E;
    for (int e = tid; e <= E; e += kThreads) {
        int64_t o = a.offsets[e];
        o = o < 0 ? 0 : (o > a.P ? a.P : o);
        s_off[e] = static_cast<int32_t>(o);
    }
    __syncthreads();
    {
        int cnt = 0;
        if (tid < E) {
            const int n = s_off[tid + 1] - s_off[tid];
            cnt = n > 0 ? (n + BM - 1) / BM : 0;
        }
        s_tstart[tid] = cnt;  // kThreads == kMaxE
        __syncthreads();
        for (int d = 1; d < kThreads; d <<= 1) {
            const int v = tid >= d ? s_tstart[tid - d] : 0;
            __syncthreads();
            s_tstart[tid] += v;
            __syncthreads();
        }
        // inclusive -> exclusive, s_tstart[E] = total
        const int incl = s_tstart[tid];
        __syncthreads();
        s_tstart[tid + 1] = incl;
        if (tid == 0) s_tstart[0] = 0;
        __syncthreads();
    }
    const int NT = a.N / BN_OUT;
    const int64_t total = static_cast<int64_t>(s_tstart[E]) * NT;
    const int xcd = blockIdx.x % kNumXcd;
    const int64_t local = blockIdx.x / kNumXcd;
    const int64_t per = total / kNumXcd, rem = total % kNumXcd;
    const int64_t cnt = per + (xcd < rem ? 1 : 0);
    if (local >= cnt) return;  // uniform over the workgroup
    const int64_t L = xcd * per + (xcd < rem ? xcd : rem) + local;
    // expert: last e with s_tstart[e] * NT <= L
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(s_tstart[mid]) * NT <= L) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int tiles_e = s_tstart[e + 1] - s_tstart[e];
    const int64_t rel = L - static_cast<int64_t>(s_tstart[e]) * NT;
    const int nt = static_cast<int>(rel / tiles_e);
    const int mt = static_cast<int>(rel - static_cast<int64_t>(nt) * tiles_e);
    const int row0 = s_off[e] + mt * BM;
    const int rows = min(BM, s_off[e + 1] - row0);
    const int n0 = nt * BN_OUT;
    const int K = a.K;

    // ---- loader addressing: chunk c -> (row c/8, 16-byte column c%8) ----
    const uint16_t* a_ptr[A_ITERS];
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
        const int c = tid + i * kThreads;
        const int r = min(c >> 3, rows - 1);
        int64_t src_row;
        if constexpr (GATEUP) {
            int64_t tok = a.sorted_pairs[row0 + r] / a.k;
            tok = tok < 0 ? 0 : (tok >= a.T ? a.T - 1 : tok);
            src_row = tok;
        } else {
            src_row = row0 + r;
        }
        a_ptr[i] = a.a_src + src_row * K + (c & 7) * 8;
    }
    const uint16_t* b_ptr[B_ITERS];
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
        const int c = tid + i * kThreads;
        const int r = c >> 3;
        const uint16_t* base;
        int col;
        if constexpr (GATEUP) {
            base = r < BN_OUT ? a.b0 : a.b1;
            col = n0 + (r < BN_OUT ? r : r - BN_OUT);
        } else {
            base = a.b0;
            col = n0 + r;
        }
        b_ptr[i] = base + (static_cast<int64_t>(e) * a.N + col) * K + (c & 7) * 8;
    }

    u32x4 ra[A_ITERS], rb[B_ITERS];
    auto load_global = [&](int kt) {
        const int koff = kt * BK;
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i)
            if (A_CHUNKS % kThreads == 0 || tid + i * kThreads < A_CHUNKS) ra[i] = ld16(a_ptr[i] + koff);
#pragma unroll
        for (int i = 0; i < B_ITERS; ++i) rb[i] = ld16(b_ptr[i] + koff);
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int c = tid + i * kThreads;
            if (A_CHUNKS % kThreads == 0 || c < A_CHUNKS)
                *reinterpret_cast<u32x4*>(&s_a[buf][(c >> 3) * LDS_STRIDE + (c & 7) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_ITERS; ++i) {
            const int c = tid + i * kThreads;
            *reinterpret_cast<u32x4*>(&s_b[buf][(c >> 3) * LDS_STRIDE + (c & 7) * 8]) = rb[i];
        }
    };

    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int r16 = lane & 15, q = lane >> 4;
    constexpr int NACC = GATEUP ? 2 : 1;
    f32x4 acc[NACC][MB][NB];
#pragma unroll
    for (int g = 0; g < NACC; ++g)
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int n = 0; n < NB; ++n) acc[g][m][n] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int nk = K / BK;
    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_global(kt + 1);
        const uint16_t* sa = s_a[buf];
        const uint16_t* sb = s_b[buf];
#pragma unroll
        for (int ks = 0; ks < BK / 32; ++ks) {
            const int kof = ks * 32 + q * 8;
            bf16x8 af[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m)
                af[m] = *reinterpret_cast<const bf16x8*>(&sa[(wm * WM + m * 16 + r16) * LDS_STRIDE + kof]);
#pragma unroll
            for (int g = 0; g < NACC; ++g) {
#pragma unroll
                for (int n = 0; n < NB; ++n) {
                    const int brow = g * BN_OUT + wn * WN_OUT + n * 16 + r16;
                    const bf16x8 bfr = *reinterpret_cast<const bf16x8*>(&sb[brow * LDS_STRIDE + kof]);
#pragma unroll
                    for (int m = 0; m < MB; ++m) acc[g][m][n] = mfma16(af[m], bfr, acc[g][m][n]);
                }
            }
        }
        if (kt + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
#pragma unroll
    for (int m = 0; m < MB; ++m) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wm * WM + m * 16 + q * 4 + i;
            if (r >= rows) continue;
            const int64_t orow = row0 + r;
#pragma unroll
            for (int n = 0; n < NB; ++n) {
                const int col = n0 + wn * WN_OUT + n * 16 + r16;
                if constexpr (GATEUP) {
                    const float g = acc[0][m][n][i];
                    const float u = acc[1][m][n][i];
                    const float prod = (g * sigmoid_f32(g)) * u;
                    static_cast<uint16_t*>(a.out)[orow * a.N + col] = f32_to_bf16_rne(prod);
                } else {
                    static_cast<float*>(a.out)[orow * a.N + col] = acc[0][m][n][i];
                }
            }
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATEUP>
hipError_t launch_gemm(const FfnArgs& a, hipStream_t s) {
    constexpr int BN_OUT = GATEUP ? BN / 2 : BN;
    const int64_t mtiles = (a.P + BM - 1) / BM + (a.E < a.P ? a.E : a.P);
    const int64_t tiles = mtiles * (a.N / BN_OUT);
    const int64_t grid = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    ffn_gemm_kernel<BM, BN, WAVES_M, WAVES_N, GATEUP>
        <<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expert_ffn(const Problem& p, const uint16_t* x, const int32_t* sorted_pairs,
                             const int32_t* offsets, const uint16_t* w_gate,
                             const uint16_t* w_up, const uint16_t* w_down, uint16_t* h, float* y,
                             hipStream_t s) {
    const int64_t P = p.T * p.k;
    FfnArgs gu{P, p.T, p.k, p.E, p.H, p.I, x, sorted_pairs, offsets, w_gate, w_up, h};
    FfnArgs dn{P, p.T, p.k, p.E, p.I, p.H, h, sorted_pairs, offsets, w_down, nullptr, y};
    const int64_t rows_per_expert = P / p.E;
    hipError_t err;
    if (rows_per_expert <= 24) {
        err = launch_gemm<16, 128, 1, 4, true>(gu, s);
        if (err != hipSuccess) return err;
        return launch_gemm<16, 64, 1, 4, false>(dn, s);
    }
    if (rows_per_expert <= 96) {
        err = launch_gemm<64, 128, 1, 4, true>(gu, s);
        if (err != hipSuccess) return err;
        return launch_gemm<64, 128, 1, 4, false>(dn, s);
    }
    err = launch_gemm<128, 128, 2, 2, true>(gu, s);
    if (err != hipSuccess) return err;
    return launch_gemm<128, 128, 2, 2, false>(dn, s);
}

}  // namespace moe
