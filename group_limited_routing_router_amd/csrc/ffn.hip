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
// Two kernels serve both projections.  A workgroup (4 waves) computes a tile
// of one expert: BM sorted rows by BN weight rows.  For gate/up the BN weight
// rows are BN/2 gate rows and the BN/2 up rows of the same output columns, so
// a lane holds gate and up accumulators of the same (row, col) and the SwiGLU
// epilogue needs no data exchange.
//   ffn_gemm_kernel      16- or 64-row tiles (few rows per expert: decode
//                        and small batches), 16x16x32 MFMA, K staged 64 or
//                        128 at a time through two padded LDS buffers via
//                        registers; with about one row tile per expert the
//                        weights stream past the caches.
//   ffn_gemm_dma_kernel  256 x 256 tiles (many rows per expert: prefill),
//                        32x32x16 MFMA, operands loaded straight into LDS.
//
// The tile list is data-dependent and never read back by the host: the grid
// is an upper bound, every workgroup rebuilds the per-expert tile prefix sum
// from expert_offsets in LDS and maps itself to a tile, and surplus
// workgroups exit.  The mapping is XCD-aware (see find_tile).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxE = 256;
constexpr int BK = 64;           // K elements per LDS stage (large-tile kernel)

// Raw buffer resource over [base, base + bytes): 32-bit offsets from one
// scalar base; loads past `bytes` return zero.  Third dword: gfx9 default.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

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
    const void* b0;          // w_gate [E,I,H] or w_down [E,H,I]: bf16, or FP8 E4M3 codes
    const void* b1;          // w_up [E,I,H] (gate/up only)
    void* out;               // h [P,I] bf16 (gate/up) or y [P,H] fp32 (down)
    const float* s0;         // FP8 weights only: per-channel scales of b0 [E,N]
    const float* s1;         // and of b1
    bool stream_out = false; // large-tile down: y stores stream past the caches
    bool stream_w = false;   // small tiles: every weight is read once (about one row
                             // tile per expert), so it streams past the caches
};

// Map this workgroup to a tile (expert e, column tile nt, row range
// [row0, row0 + rows)).  Every workgroup rebuilds the prefix sum of per-expert
// row tiles from expert_offsets in LDS (no host read-back); an expert with n
// rows gets ceil(n / BM) row tiles.  The tile list is ordered
// by expert position, then column tile, then row tile; workgroup b runs on
// XCD b % 8 and XCD x takes the x-th contiguous run of the list, so the row
// tiles that share a weight tile are neighbours on one XCD.  Expert positions
// interleave the experts (position i holds expert (i % 8) * (E / 8) + i / 8
// when 8 divides E), so each XCD's run draws on every group of consecutive
// experts and a few heavily routed neighbours do not land on one XCD.
// GRAN = 1 splits an expert's rows evenly over its row tiles; GRAN > 1 gives
// every row tile but the last the same multiple of GRAN rows (for the large
// tile, whose two row waves take alternate 32-row blocks: 64-row multiples
// keep them equally busy).  Returns false for surplus workgroups (uniform
// over the workgroup).  s_off holds kMaxE + 1 entries, s_tstart
// kMaxE + 1 + kWaves.
template <int BM, int GRAN = 1>
__device__ bool find_tile(const FfnArgs& a, int ncol_tiles, int32_t* s_off, int32_t* s_tstart,
                          int& e_out, int& nt_out, int& row0_out, int& rows_out) {
    const int tid = threadIdx.x;
    const int E = a.E;
    for (int e = tid; e <= E; e += kThreads) {
        int64_t o = a.offsets[e];
        o = o < 0 ? 0 : (o > a.P ? a.P : o);
        s_off[e] = static_cast<int32_t>(o);
    }
    __syncthreads();
    // expert at list position i
    const bool interleave = E % kNumXcd == 0;
    auto expert_at = [&](int i) { return interleave ? (i % kNumXcd) * (E / kNumXcd) + i / kNumXcd : i; };
    int cnt = 0;
    if (tid < E) {
        const int ex = expert_at(tid);
        const int n = s_off[ex + 1] - s_off[ex];
        cnt = n > 0 ? (n + BM - 1) / BM : 0;
    }
    // inclusive prefix sum over positions (kThreads == kMaxE): within each
    // wave by shuffles, then the totals of the waves before it
    const int lane = tid & (kWave - 1), wave = tid / kWave;
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int v = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += v;
    }
    int32_t* s_wave_total = s_tstart + (kMaxE + 1);
    if (lane == kWave - 1) s_wave_total[wave] = incl;
    __syncthreads();
    for (int w = 0; w < wave; ++w) incl += s_wave_total[w];
    s_tstart[tid + 1] = incl;  // exclusive prefix over positions; s_tstart[E] = total row tiles
    if (tid == 0) s_tstart[0] = 0;
    __syncthreads();
    const int64_t total = static_cast<int64_t>(s_tstart[E]) * ncol_tiles;
    const int xcd = blockIdx.x % kNumXcd;
    const int64_t local = blockIdx.x / kNumXcd;
    const int64_t per = total / kNumXcd, rem = total % kNumXcd;
    if (local >= per + (xcd < rem ? 1 : 0)) return false;
    const int64_t L = xcd * per + (xcd < rem ? xcd : rem) + local;
    int lo = 0, hi = E - 1;  // last position i with s_tstart[i] * ncol_tiles <= L
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (static_cast<int64_t>(s_tstart[mid]) * ncol_tiles <= L) lo = mid; else hi = mid - 1;
    }
    const int pos = lo;
    const int e = expert_at(pos);
    const int tiles_e = s_tstart[pos + 1] - s_tstart[pos];  // >= 1 for the position found
    const int64_t rel = L - static_cast<int64_t>(s_tstart[pos]) * ncol_tiles;
    const int nt = static_cast<int>(rel / tiles_e);
    const int mt = static_cast<int>(rel - static_cast<int64_t>(nt) * tiles_e);
    const int n_e = s_off[e + 1] - s_off[e];
    e_out = e;
    nt_out = nt;
    if constexpr (GRAN == 1) {
        const int base = n_e / tiles_e, extra = n_e % tiles_e;
        row0_out = s_off[e] + mt * base + (mt < extra ? mt : extra);
        rows_out = base + (mt < extra ? 1 : 0);
    } else {
        // per <= BM since GRAN divides BM, so the last tile keeps >= 1 row
        static_assert(BM % GRAN == 0, "granule divides the tile");
        const int per = ((n_e + tiles_e - 1) / tiles_e + GRAN - 1) / GRAN * GRAN;
        row0_out = s_off[e] + mt * per;
        rows_out = min(per, n_e - mt * per);
    }
    return true;
}

// FP8 E4M3 codes -> bf16, eight at a time, two per instruction.  With a unit
// scale the gfx950 conversion is exact (OCP e4m3fn codes; every E4M3 value is
// a bf16 value) and NaN codes stay NaN.
__device__ __forceinline__ bf16x8 e4m3x8_to_bf16x8(uint32_t lo, uint32_t hi) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    u32x4 r;
    r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false));
    r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true));
    r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false));
    r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true));
    return as_bf16x8(r);
}

// FP8 = true: the weights are E4M3 codes with one fp32 scale per output
// channel (FfnArgs::s0/s1).  They are staged in LDS as codes, widened to bf16
// as each MFMA operand is read, and the channel scale multiplies the fp32
// accumulator in the epilogue.  SK is the K extent of an LDS stage: 128 for
// FP8 weights, so that every weight row of a stage is one whole 128-byte line.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATEUP, bool FP8 = false, int SK = 64,
          bool NTW = false>
__global__ __launch_bounds__(kThreads) void ffn_gemm_kernel(FfnArgs a) {
    static_assert(WAVES_M * WAVES_N == kWaves, "4 waves");
    static_assert(SK == 64 || SK == 128, "stage depth");
    constexpr int A_STRIDE = SK + 8;                  // bf16 per LDS activation row (16 B pad)
    constexpr int A_CPR = SK / 8;                     // 16-byte chunks per activation row
    constexpr int BN_OUT = GATEUP ? BN / 2 : BN;     // output columns per tile
    constexpr int WM = BM / WAVES_M;                  // rows per wave
    constexpr int MB = WM / 16;
    constexpr int WN_OUT = BN_OUT / WAVES_N;          // output columns per wave
    constexpr int NB = WN_OUT / 16;
    static_assert(MB >= 1 && NB >= 1, "tile too small");
    constexpr int EB = FP8 ? 1 : 2;                   // bytes per weight
    constexpr int B_ROW = SK * EB;                    // weight bytes per row and stage
    // LDS row pitch of the weight stage.  The pad moves consecutive rows to
    // other banks; FP8 rows are read 8 bytes a lane, for which 8 bytes of pad
    // suffice, and the smaller pitch lets two 256-row FP8 workgroups share a
    // compute unit.
    constexpr int B_STRIDE = B_ROW + (FP8 ? 8 : 16);
    constexpr int B_CPR = B_ROW / 16;                 // 16-byte chunks per weight row
    constexpr int A_CHUNKS = BM * A_CPR;              // 16-byte chunks per stage
    constexpr int B_CHUNKS = BN * B_CPR;
    constexpr int A_ITERS = (A_CHUNKS + kThreads - 1) / kThreads;
    constexpr int B_ITERS = B_CHUNKS / kThreads;
    static_assert(B_CHUNKS % kThreads == 0, "B tile");

    __shared__ __attribute__((aligned(16))) uint16_t s_a[2][BM * A_STRIDE];
    __shared__ __attribute__((aligned(16))) unsigned char s_b[2][BN * B_STRIDE];
    __shared__ int32_t s_off[kMaxE + 1];
    __shared__ int32_t s_tstart[kMaxE + 1 + kWaves];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    int e, nt, row0, rows;
    if (!find_tile<BM>(a, a.N / BN_OUT, s_off, s_tstart, e, nt, row0, rows)) return;
    const int n0 = nt * BN_OUT;
    const int K = a.K;

    // ---- loader addressing: chunk c -> (row c / A_CPR, 16-byte column c % A_CPR) ----
    const uint16_t* a_ptr[A_ITERS];
#pragma unroll
    for (int i = 0; i < A_ITERS; ++i) {
        const int c = tid + i * kThreads;
        const int r = min(c / A_CPR, rows - 1);
        int64_t src_row;
        if constexpr (GATEUP) {
            int64_t tok = a.sorted_pairs[row0 + r] / a.k;
            tok = tok < 0 ? 0 : (tok >= a.T ? a.T - 1 : tok);
            src_row = tok;
        } else {
            src_row = row0 + r;
        }
        a_ptr[i] = a.a_src + src_row * K + (c % A_CPR) * 8;
    }
    const unsigned char* b_ptr[B_ITERS];
#pragma unroll
    for (int i = 0; i < B_ITERS; ++i) {
        const int c = tid + i * kThreads;
        const int r = c / B_CPR;
        const void* base;
        int col;
        if constexpr (GATEUP) {
            base = r < BN_OUT ? a.b0 : a.b1;
            col = n0 + (r < BN_OUT ? r : r - BN_OUT);
        } else {
            base = a.b0;
            col = n0 + r;
        }
        b_ptr[i] = static_cast<const unsigned char*>(base) +
                   ((static_cast<int64_t>(e) * a.N + col) * K) * EB + (c % B_CPR) * 16;
    }

    u32x4 ra[A_ITERS], rb[B_ITERS];
    auto load_global = [&](int kt) {
        const int koff = kt * SK;
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i)
            if (A_CHUNKS % kThreads == 0 || tid + i * kThreads < A_CHUNKS) ra[i] = ld16(a_ptr[i] + koff);
#pragma unroll
        for (int i = 0; i < B_ITERS; ++i) {
            // with about one row tile per expert every weight is read once:
            // streamed past the caches, so it does not evict what is reused
            // (decode 8-12% faster; the weight stream reaches 7.0 TB/s)
            // (a compile-time choice: with a run-time branch the compiler
            // merges the two loads into one plain load)
            if constexpr (NTW)
                rb[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(b_ptr[i] + koff * EB));
            else
                rb[i] = ld16(b_ptr[i] + koff * EB);
        }
    };
    auto store_lds = [&](int buf) {
#pragma unroll
        for (int i = 0; i < A_ITERS; ++i) {
            const int c = tid + i * kThreads;
            if (A_CHUNKS % kThreads == 0 || c < A_CHUNKS)
                *reinterpret_cast<u32x4*>(&s_a[buf][(c / A_CPR) * A_STRIDE + (c % A_CPR) * 8]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < B_ITERS; ++i) {
            const int c = tid + i * kThreads;
            unsigned char* dst = &s_b[buf][(c / B_CPR) * B_STRIDE + (c % B_CPR) * 16];
            if constexpr (B_STRIDE % 16 == 0) {
                *reinterpret_cast<u32x4*>(dst) = rb[i];
            } else {  // an 8-byte aligned row: two 8-byte stores
                typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                reinterpret_cast<u32x2*>(dst)[0] = u32x2{rb[i][0], rb[i][1]};
                reinterpret_cast<u32x2*>(dst)[1] = u32x2{rb[i][2], rb[i][3]};
            }
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

    const int nk = K / SK;
    load_global(0);
    store_lds(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nk) load_global(kt + 1);
        const uint16_t* sa = s_a[buf];
        const unsigned char* sb = s_b[buf];
#pragma unroll
        for (int ks = 0; ks < SK / 32; ++ks) {
            const int kof = ks * 32 + q * 8;
            bf16x8 af[MB];
#pragma unroll
            for (int m = 0; m < MB; ++m)
                af[m] = *reinterpret_cast<const bf16x8*>(&sa[(wm * WM + m * 16 + r16) * A_STRIDE + kof]);
#pragma unroll
            for (int g = 0; g < NACC; ++g) {
#pragma unroll
                for (int n = 0; n < NB; ++n) {
                    const int brow = g * BN_OUT + wn * WN_OUT + n * 16 + r16;
                    bf16x8 bfr;
                    if constexpr (FP8) {
                        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
                        const u32x2 w8 = *reinterpret_cast<const u32x2*>(&sb[brow * B_STRIDE + kof]);
                        bfr = e4m3x8_to_bf16x8(w8[0], w8[1]);
                    } else {
                        bfr = *reinterpret_cast<const bf16x8*>(&sb[brow * B_STRIDE + kof * 2]);
                    }
#pragma unroll
                    for (int m = 0; m < MB; ++m) acc[g][m][n] = mfma16(af[m], bfr, acc[g][m][n]);
                }
            }
        }
        if (kt + 1 < nk) store_lds(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ----
    float sc0[NB], sc1[NB];  // per-channel scales of this lane's columns (FP8)
#pragma unroll
    for (int n = 0; n < NB; ++n) {
        const int64_t ch = static_cast<int64_t>(e) * a.N + n0 + wn * WN_OUT + n * 16 + r16;
        sc0[n] = FP8 ? a.s0[ch] : 1.0f;
        sc1[n] = (FP8 && GATEUP) ? a.s1[ch] : 1.0f;
    }
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
                    float g = acc[0][m][n][i];
                    float u = acc[1][m][n][i];
                    if constexpr (FP8) {
                        g = sc0[n] * g;
                        u = sc1[n] * u;
                    }
                    const float prod = (g * sigmoid_f32(g)) * u;
                    static_cast<uint16_t*>(a.out)[orow * a.N + col] = f32_to_bf16_rne(prod);
                } else {
                    float v = acc[0][m][n][i];
                    if constexpr (FP8) v = sc0[n] * v;
                    static_cast<float*>(a.out)[orow * a.N + col] = v;
                }
            }
        }
    }
}

template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATEUP, bool FP8, int SK, bool NTW>
hipError_t launch_gemm_nt(const FfnArgs& a, hipStream_t s) {
    constexpr int BN_OUT = GATEUP ? BN / 2 : BN;
    const int64_t mtiles = (a.P + BM - 1) / BM + (a.E < a.P ? a.E : a.P);
    const int64_t tiles = mtiles * (a.N / BN_OUT);
    const int64_t grid = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    ffn_gemm_kernel<BM, BN, WAVES_M, WAVES_N, GATEUP, FP8, SK, NTW>
        <<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
}

// The small-tile GEMM with the weight loads streamed past the caches when
// a.stream_w is set.
template <int BM, int BN, int WAVES_M, int WAVES_N, bool GATEUP, bool FP8 = false, int SK = 64>
hipError_t launch_gemm(const FfnArgs& a, hipStream_t s) {
    if (a.stream_w) return launch_gemm_nt<BM, BN, WAVES_M, WAVES_N, GATEUP, FP8, SK, true>(a, s);
    return launch_gemm_nt<BM, BN, WAVES_M, WAVES_N, GATEUP, FP8, SK, false>(a, s);
}

// The large tile reads its operands through buffer resources with 32-bit
// offsets.  A stage row past the tile's last 32-row block gets this offset,
// which lies past the end of any operand the kernel takes (x of at most
// kNoRowOffset bytes, so up to 4 GiB less 1 MiB) and cannot wrap when a
// stage's K offset is added, so its loads fetch nothing.
constexpr uint32_t kNoRowOffset = 0xFFF00000u;

// Large-tile GEMM for experts with many rows (prefill and longer).
//
// 32x32x16 MFMA; a 256-thread workgroup owns a 256 x 256 tile and each of its
// 4 waves a 128 x 128 sub-tile, 256 fp32 accumulators per lane.  Row blocks
// of 32 go to the two M-waves cyclically (block b to wave b % 2) and blocks
// past the tile's last row are skipped, so a partly filled tile costs MFMA
// time in proportion to its rows.  The tile map is find_tile's.
//
// Global data goes straight into LDS with buffer_load_dwordx4 ... lds: no
// staging registers and no LDS store instructions.  Each such load writes one
// wave's 64 x 16 bytes contiguously at M0, so a tile stage (K = 64, 128 bytes
// per row) is laid out row-major without padding, and the 16-byte chunk c of
// row r sits at chunk c ^ ((r >> 1) & 7): the 16 rows read by one MFMA
// operand load then hit all 64 banks once.  The 160 KB of LDS hold two
// activation stages and three weight stages: activations (mostly L2 hits)
// are loaded one stage ahead, weights (the HBM stream) two stages ahead.  The
// compiler does not see these loads, so the kernel itself waits for them
// (vmcnt) before each barrier, and for all of them before it ends.  Results
// are stored straight from the accumulators (see the epilogue).
constexpr int kDmaArena = 163840;  // the whole LDS of a gfx950 workgroup

__device__ __forceinline__ void dma_load16(uint32_t lds_byte_addr, __amdgpu_buffer_rsrc_t rsrc,
                                           uint32_t voffset, uint32_t soffset) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(__builtin_amdgcn_readfirstlane(lds_byte_addr)), "v"(voffset), "s"(rsrc),
          "s"(__builtin_amdgcn_readfirstlane(soffset))
        : "memory", "m0");
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// FP8 = true: the weights are E4M3 codes, widened to bf16 as each MFMA
// operand is read; the per-channel scale multiplies the accumulators before
// the results are stored.  A weight stage then spans two activation stages
// (K = 128 codes, again 128 bytes a row: every weight row of a stage is one
// whole line, laid out and swizzled like an activation row), and its loads
// are spread over those two.
template <bool GATEUP, bool FP8 = false>
__global__ __launch_bounds__(kThreads) void ffn_gemm_dma_kernel(FfnArgs a) {
    constexpr int BM = 256, BN = 256, WAVES_M = 2, WAVES_N = 2;
    constexpr int BN_OUT = GATEUP ? BN / 2 : BN;
    constexpr int MB = BM / 32 / WAVES_M;      // 4 row blocks per wave
    constexpr int WN_OUT = BN_OUT / WAVES_N;
    constexpr int NB = WN_OUT / 32;
    constexpr int NACC = GATEUP ? 2 : 1;
    constexpr int NFB = NACC * NB;             // B fragments per substep (4)
    constexpr int ROW_BYTES = BK * 2;          // 128 (activations)
    constexpr int EB = FP8 ? 1 : 2;            // bytes per weight
    constexpr int SB = FP8 ? 2 : 1;            // activation stages per weight stage
    constexpr int B_ROW = BK * SB * EB;        // 128 bytes of each weight row per weight stage
    static_assert(B_ROW == ROW_BYTES, "weight rows are staged like activation rows");
    constexpr int A_STAGE = BM * ROW_BYTES;    // 32 KB
    constexpr int B_STAGE = BN * B_ROW;        // 32 KB
    constexpr int A_BUFS = 2, B_BUFS = 3;
    constexpr int ARENA = A_BUFS * A_STAGE + B_BUFS * B_STAGE;
    static_assert(ARENA <= kDmaArena, "LDS budget");
    constexpr int DMA_A = BM / kWaves / 8;     // 1-KB activation loads per wave and stage (8)
    constexpr int B_RPL = 1024 / B_ROW;        // weight rows per 1-KB load (8)
    constexpr int B_LPR = B_ROW / 16;          // lanes per weight row (8)
    constexpr int DMA_BS = BN / kWaves / B_RPL; // weight loads per wave and weight stage (8)
    constexpr int DMA_B = DMA_BS / SB;         // ... per activation stage (8, FP8: 4)

    __shared__ __attribute__((aligned(1024))) unsigned char s_arena[ARENA];
    const uint32_t arena = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(s_arena));

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave

    int e, nt, row0, rows;
    {
        int32_t* s_off = reinterpret_cast<int32_t*>(s_arena);
        int32_t* s_tstart = s_off + (kMaxE + 1);
        if (!find_tile<BM, 32 * WAVES_M>(a, a.N / BN_OUT, s_off, s_tstart, e, nt, row0, rows)) return;
        __syncthreads();  // everyone is done with the schedule before DMA reuses the arena
    }
    const int n0 = nt * BN_OUT;
    const int K = a.K;
    const int nblk = (rows + 31) >> 5;

    // ---- DMA addressing: wave w fills rows [64 w, 64 w + 64) of a stage,
    // 8 rows per load; lane L of load j writes row 64 w + 8 j + L / 8, physical
    // chunk L % 8, i.e. logical chunk (L % 8) ^ ((row >> 1) & 7). ----
    __amdgpu_buffer_rsrc_t rsrc_a, rsrc_b;
    uint32_t va[DMA_A], vb[DMA_BS];
    if constexpr (GATEUP)
        rsrc_a = make_rsrc(a.a_src, static_cast<uint32_t>(a.T * K * 2));
    else
        rsrc_a = make_rsrc(a.a_src + static_cast<int64_t>(row0) * K,
                           static_cast<uint32_t>(rows * K * 2));
    {
        const int64_t first = (static_cast<int64_t>(e) * a.N + n0) * K * EB;
        const unsigned char* wbase;
        if constexpr (GATEUP)  // waves 0-1: gate rows, 2-3: up rows
            wbase = static_cast<const unsigned char*>(wave < 2 ? a.b0 : a.b1) + first;
        else
            wbase = static_cast<const unsigned char*>(a.b0) + first;
        rsrc_b = make_rsrc(wbase, static_cast<uint32_t>((GATEUP ? BN_OUT : BN) * K * EB));
    }
#pragma unroll
    for (int j = 0; j < DMA_A; ++j) {
        const int r = wave * 64 + j * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((r >> 1) & 7);
        uint32_t av;
        if (r >= nblk * 32) {
            av = kNoRowOffset;
        } else if constexpr (GATEUP) {
            const int rr = min(r, rows - 1);
            int64_t tok = a.sorted_pairs[row0 + rr] / a.k;
            tok = tok < 0 ? 0 : (tok >= a.T ? a.T - 1 : tok);
            av = static_cast<uint32_t>(tok * K * 2 + c * 16);
        } else {
            av = static_cast<uint32_t>(r * K * 2 + c * 16);
        }
        va[j] = av;
    }
#pragma unroll
    for (int j = 0; j < DMA_BS; ++j) {
        const int r = wave * 64 + j * B_RPL + lane / B_LPR;
        const int c = (lane % B_LPR) ^ ((r >> 1) & 7);
        const int rb = GATEUP ? (r & (BN_OUT - 1)) : r;  // row within the gate / up half
        vb[j] = static_cast<uint32_t>(rb * K * EB + c * 16);
    }
    auto a_buf = [&](int i) { return arena + i * A_STAGE; };
    auto b_buf = [&](int i) { return arena + A_BUFS * A_STAGE + i * B_STAGE; };
    auto dma_a = [&](int j, int buf, int kt) {
        dma_load16(a_buf(buf) + (wave * 64 + j * 8) * ROW_BYTES, rsrc_a, va[j],
                   static_cast<uint32_t>(kt * ROW_BYTES));
    };
    auto dma_b = [&](int j, int buf, int kbs) {  // load j of weight stage kbs
        dma_load16(b_buf(buf) + (wave * 64 + j * B_RPL) * B_ROW, rsrc_b, vb[j],
                   static_cast<uint32_t>(kbs * B_ROW));
    };

    const int wm = wave / WAVES_N, wn = wave % WAVES_N;
    const int r32 = lane & 31, half = lane >> 5;
    int mb_valid = 0;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) mb_valid += (wm + WAVES_M * mb) < nblk;

    f32x16 acc[NACC][MB][NB];
#pragma unroll
    for (int g = 0; g < NACC; ++g)
#pragma unroll
        for (int m = 0; m < MB; ++m)
#pragma unroll
            for (int n = 0; n < NB; ++n)
#pragma unroll
                for (int i = 0; i < 16; ++i) acc[g][m][n][i] = 0.0f;

    // LDS byte offset of the fragment (row r, logical chunk c) of a stage
    auto frag_off = [&](int r, int c) { return r * ROW_BYTES + ((c ^ ((r >> 1) & 7)) << 4); };

    auto k_loop = [&](auto nv_tag) {
        constexpr int NV = decltype(nv_tag)::value;
        constexpr int NA = NV > 0 ? NV : 1;
        constexpr int MF = NV * NFB;  // MFMAs per substep
        // B fragments are held as read: bf16, or E4M3 codes widened to bf16
        // right before the MFMAs that use them (converting at the read would
        // wait out the LDS latency there).
        //
        // FP8: substeps go in pairs (2p, 2p + 1), which cover codes
        // [32 p, 32 p + 32) of the activation stage's half of the weight stage.
        // In the even substep every lane reads one whole 16-byte chunk of codes
        // -- lanes below 32 chunk 2p, the others chunk 2p + 1 -- and the pair's
        // two MFMAs take its first and its second 8 bytes.  The MFMA's k lanes
        // then stand for physical k = 16 (2p + half) + 8 j + (0..7) in substep
        // 2p + j, and the A fragments follow the same mapping (activation
        // chunk 4p + 2 half + j).  Every product is the same; only the order of
        // the fp32 sum changes.  The reads are whole chunks, 16 lanes to 16
        // rows of one chunk, so the swizzle keeps them free of bank conflicts
        // (8-byte half-chunk reads met 2-way conflicts on about 30% of LDS
        // accesses).  The second 8 bytes are widened together with the first
        // (bh), so the raw codes are dead after the even substep and the next
        // pair's chunks load during the odd one.
        typedef typename std::conditional<FP8, u32x4, bf16x8>::type BFrag;
        struct Frags {
            bf16x8 a[NA];
            BFrag b[NFB];
        };
        bf16x8 bh[FP8 ? NFB : 1];  // FP8: codes 8..15 of the pair's chunks, widened
        // fragment pieces of substep ks: A blocks first, then B blocks (none
        // in an odd FP8 substep: the pair's chunks are already held)
        auto pieces = [](int ks) { return NV > 0 ? NV + ((FP8 && (ks & 1)) ? 0 : NFB) : 0; };
        // piece q of substep ks's fragments (FP8: from half hb of the weight stage)
        auto load_piece = [&](Frags& f, int ab, int bb, int ks, int hb, auto qc) {
            constexpr int q = decltype(qc)::value;
            if constexpr (q < NV) {
                const int c = FP8 ? 4 * (ks >> 1) + 2 * half + (ks & 1) : ks * 2 + half;
                const unsigned char* sa = s_arena + (a_buf(ab) - arena);
                f.a[q] = *reinterpret_cast<const bf16x8*>(sa + frag_off((wm + WAVES_M * q) * 32 + r32, c));
            } else if constexpr (NV > 0) {
                constexpr int gn = q - NV;
                constexpr int g = gn / NB, n = gn % NB;
                const unsigned char* sb = s_arena + (b_buf(bb) - arena);
                const int br = g * BN_OUT + wn * WN_OUT + n * 32 + r32;
                if constexpr (FP8) {
                    // 16 codes: chunk 4 hb + ks + half (ks even)
                    f.b[gn] = *reinterpret_cast<const u32x4*>(sb + frag_off(br, hb * 4 + ks + half));
                } else {
                    f.b[gn] = *reinterpret_cast<const bf16x8*>(sb + frag_off(br, ks * 2 + half));
                }
            }
        };
        constexpr int NP = NV > 0 ? NV + NFB : 0;  // most fragment pieces of a substep
        auto load_frags = [&](Frags& f, int ab, int bb, int ks, int hb) {
            static_for<0, NP>([&](auto qc) {
                if (decltype(qc)::value < pieces(ks)) load_piece(f, ab, bb, ks, hb, qc);
            });
        };
        // MFMA i = (g * NB + n) * NV + m of substep ks; bop holds B fragment
        // gn in bf16 (FIRST: MFMA i is the first of a run on it, so it is
        // widened, or for an odd FP8 substep taken from bh, here)
        auto mfma_one = [&](const Frags& f, auto ic, auto ks_c, bf16x8& bop, bool first) {
            constexpr int i = decltype(ic)::value;
            constexpr int KS = decltype(ks_c)::value;
            constexpr int m = i % (NV > 0 ? NV : 1);
            constexpr int gn = i / (NV > 0 ? NV : 1);
            constexpr int g = gn / NB, n = gn % NB;
            if constexpr (NV > 0) {
                if (m == 0 || first) {  // compile-time at every call site
                    if constexpr (FP8 && (KS & 1)) {
                        bop = bh[gn];
                    } else if constexpr (FP8) {
                        bop = e4m3x8_to_bf16x8(f.b[gn][0], f.b[gn][1]);
                        bh[gn] = e4m3x8_to_bf16x8(f.b[gn][2], f.b[gn][3]);
                    } else {
                        bop = f.b[gn];
                    }
                }
                acc[g][m][n] = mfma32(f.a[m], bop, acc[g][m][n]);
            }
        };
        const int nk = K / BK;     // activation stages (a multiple of SB)
        const int nbs = nk / SB;   // weight stages
        // prologue: A(0), B(0), B(1) in flight; wait for the first two
#pragma unroll
        for (int j = 0; j < DMA_A; ++j) dma_a(j, 0, 0);
#pragma unroll
        for (int j = 0; j < DMA_BS; ++j) dma_b(j, 0, 0);
#pragma unroll
        for (int j = 0; j < DMA_BS; ++j) dma_b(j, 1, nbs > 1 ? 1 : 0);
        wait_vmcnt<DMA_BS>();
        __syncthreads();
        int abuf = 0, bbuf = 0;
        Frags f0, f1;
        load_frags(f0, 0, 0, 0, 0);
        // activation stage kt = kt0 + HB is half HB of weight stage kt0 / SB
        for (int kt0 = 0; kt0 < nk; kt0 += SB) static_for<0, SB>([&](auto hb_c) {
            constexpr int HB = decltype(hb_c)::value;
            const int kt = kt0 + HB;
            const int kbs = kt0 / SB;
            const int ka = kt + 1 < nk ? kt + 1 : nk - 1;      // past the end: refill an idle buffer
            const int kb = kbs + 2 < nbs ? kbs + 2 : nbs - 1;  // weight stage loaded two ahead
            const int anext = abuf ^ 1;
            const int bnext = bbuf == 0 ? 2 : bbuf - 1;        // (bbuf + 2) % 3
            // Phases are pinned with scheduling fences (the compiler would
            // otherwise sink fragment reads next to their MFMAs or bunch them):
            // the fragments of the next substep are read one at a time between
            // the MFMAs of this one (A first, then B, in order of first use),
            // and the stage's loads are spread evenly over its MFMAs up to the
            // stage barrier (activations first, they are needed one stage
            // ahead; weights after), so neither the LDS nor the texture unit
            // backs up into the MFMA issue stream.  The stage barrier sits
            // before the last eighth of the last substep's MFMAs: the first
            // fragments of the next stage are read while those run, so the
            // matrix pipe does not wait out a whole LDS round trip at every
            // stage (a later barrier leaves the loads of the next stage more
            // time to land).
            constexpr int LPS = (DMA_A + DMA_B) / 4;  // loads per substep (4, FP8: 3)
            static_assert(LPS * 4 == DMA_A + DMA_B, "loads split evenly over the substeps");
            // MFMAs [LO, HI) of substep SUB with its stage loads spread over them
            // (none for a negative SUB) and, for KN >= 0, the fragments of
            // substep KN read into FN piece by piece between them
            // (KS: the substep whose MFMAs these are, 0..3)
            auto substep = [&](const Frags& f, auto sc, auto ks_c, auto lo_c, auto hi_c, Frags& fn, auto kn_c) {
                constexpr int sub = decltype(sc)::value;
                constexpr int LO = decltype(lo_c)::value, HI = decltype(hi_c)::value;
                constexpr int KN = decltype(kn_c)::value;
                constexpr int NM = HI - LO;
                constexpr int NL = sub >= 0 ? LPS : 0;
                constexpr int NPC = KN >= 0 ? (NV > 0 ? NV + ((FP8 && (KN & 1)) ? 0 : NFB) : 0) : 0;
                constexpr int IT = NM > NL ? (NM > 0 ? NM : 1) : (NL > 0 ? NL : 1);
                bf16x8 bop;
                static_for<0, IT>([&](auto ic) {
                    constexpr int i = decltype(ic)::value;
                    static_for<0, NPC>([&](auto qc) {
                        constexpr int q = decltype(qc)::value;
                        if constexpr (q * IT / (NPC > 0 ? NPC : 1) == i) load_piece(fn, abuf, bbuf, KN, HB, qc);
                    });
                    if constexpr (i < NM) mfma_one(f, std::integral_constant<int, LO + i>{}, ks_c, bop, i == 0);
                    constexpr int step = NM >= NL ? (NL > 0 ? NM / NL : 1) : 1;
                    if constexpr (NL > 0 && i % step == step - 1 && i / step < NL) {
                        constexpr int j = sub * LPS + i / step;
                        if constexpr (j < DMA_A)
                            dma_a(j, anext, ka);
                        else
                            dma_b(HB * DMA_B + j - DMA_A, bnext, kb);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                });
            };
            using C0 = std::integral_constant<int, 0>;
            using CM = std::integral_constant<int, MF>;
            using CH = std::integral_constant<int, MF * 7 / 8>;
            using KNone = std::integral_constant<int, -1>;
            using K0 = std::integral_constant<int, 0>;
            using K1 = std::integral_constant<int, 1>;
            using K2 = std::integral_constant<int, 2>;
            using K3 = std::integral_constant<int, 3>;
            substep(f0, K0{}, K0{}, C0{}, CM{}, f1, K1{});
            substep(f1, K1{}, K1{}, C0{}, CM{}, f0, K2{});
            substep(f0, K2{}, K2{}, C0{}, CM{}, f1, K3{});
            substep(f1, K3{}, K3{}, C0{}, CH{}, f0, KNone{});
            wait_vmcnt<DMA_B>();
            __syncthreads();
            abuf = anext;
            if constexpr (HB == SB - 1) bbuf = bbuf == 2 ? 0 : bbuf + 1;
            load_frags(f0, abuf, bbuf, 0, (HB + 1) % SB);  // after the last stage: read, never used
            __builtin_amdgcn_sched_barrier(0);
            substep(f1, std::integral_constant<int, -1>{}, K3{}, CH{}, CM{}, f0, KNone{});
        });
        wait_vmcnt<0>();
        __syncthreads();
    };
    switch (mb_valid) {
        case 0: k_loop(std::integral_constant<int, 0>{}); break;
        case 1: k_loop(std::integral_constant<int, 1>{}); break;
        case 2: k_loop(std::integral_constant<int, 2>{}); break;
        case 3: k_loop(std::integral_constant<int, 3>{}); break;
        default: k_loop(std::integral_constant<int, 4>{}); break;
    }

    // ---- epilogue ----
    {
        // Straight from the accumulators, one value per lane and store: lane l
        // holds column l % 32, so one store covers two rows of 32 contiguous
        // columns (two full 128-byte lines of y, two half lines of h).  The
        // stores go through a buffer resource over rows [row0, row0 + rows) of
        // the output, whose range check drops the rows past the tile.
        constexpr int OB = GATEUP ? 2 : 4;  // output bytes per element
        const __amdgpu_buffer_rsrc_t rsrc_o = make_rsrc(
            static_cast<unsigned char*>(a.out) + static_cast<int64_t>(row0) * a.N * OB,
            static_cast<uint32_t>(rows * a.N * OB));
        // FP8: per-channel scales of this lane's column of each accumulator
        // block, applied as each accumulator is read
        float sc0[NB], sc1[NB];
#pragma unroll
        for (int n = 0; n < NB; ++n) {
            const int64_t ch = static_cast<int64_t>(e) * a.N + n0 + wn * WN_OUT + n * 32 + r32;
            sc0[n] = FP8 ? a.s0[ch] : 1.0f;
            sc1[n] = (FP8 && GATEUP) ? a.s1[ch] : 1.0f;
        }
        const uint32_t lane_off = static_cast<uint32_t>(((4 * half) * a.N + n0 + wn * WN_OUT + r32) * OB);
        const uint32_t row_bytes = static_cast<uint32_t>(a.N * OB);
        if constexpr (GATEUP) {
#pragma unroll
            for (int m = 0; m < MB; ++m) {
                if (m >= mb_valid) continue;
                const int blk = wm + WAVES_M * m;
#pragma unroll
                for (int n = 0; n < NB; ++n) {
#pragma unroll
                    for (int i = 0; i < 16; i += 2) {
                        // rows blk * 32 + 8 (i / 4) + 4 half + i % 4 and the next,
                        // column n0 + wn WN_OUT + 32 n + l % 32, converted together
                        const uint32_t off = lane_off + (blk * 32 + 8 * (i >> 2) + (i & 3)) * row_bytes + n * 32 * OB;
                        typedef float f32x2 __attribute__((ext_vector_type(2)));
                        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
                        float g0 = acc[0][m][n][i], g1 = acc[0][m][n][i + 1];
                        float u0 = acc[1][m][n][i], u1 = acc[1][m][n][i + 1];
                        if constexpr (FP8) {
                            g0 *= sc0[n];
                            g1 *= sc0[n];
                            u0 *= sc1[n];
                            u1 *= sc1[n];
                        }
                        const float v0 = silu_f32(g0) * u0;
                        const float v1 = silu_f32(g1) * u1;
                        const uint32_t pk = __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{v0, v1}, bf16x2));
                        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pk), rsrc_o, off, 0, 0);
                        __builtin_amdgcn_raw_buffer_store_b16(static_cast<uint16_t>(pk >> 16), rsrc_o, off + row_bytes, 0, 0);
                    }
                }
            }
        } else {
            // y larger than the caches is written nontemporally (cache policy
            // nt): the combine reads it once, long after
            auto store_y = [&](auto nt_c) {
                constexpr int kPolicy = decltype(nt_c)::value ? 2 : 0;
#pragma unroll
                for (int m = 0; m < MB; ++m) {
                    if (m >= mb_valid) continue;
                    const int blk = wm + WAVES_M * m;
#pragma unroll
                    for (int n = 0; n < NB; ++n)
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            // row blk * 32 + 8 (i / 4) + 4 half + i % 4, column n0 + wn WN_OUT + 32 n + l % 32
                            const uint32_t off = lane_off + (blk * 32 + 8 * (i >> 2) + (i & 3)) * row_bytes + n * 32 * OB;
                            // (copied out first: a bit cast of a vector element in
                            // place would read element 0)
                            float v = acc[0][m][n][i];
                            if constexpr (FP8) v *= sc0[n];
                            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rsrc_o, off, 0, kPolicy);
                        }
                }
            };
            if (a.stream_out)
                store_y(std::true_type{});
            else
                store_y(std::false_type{});
        }
    }
}

template <bool GATEUP, bool FP8 = false>
hipError_t launch_gemm_dma(const FfnArgs& a, hipStream_t s) {
    constexpr int BM = 256, BN_OUT = GATEUP ? 128 : 256;
    const int64_t mtiles = (a.P + BM - 1) / BM + (a.E < a.P ? a.E : a.P);
    const int64_t tiles = mtiles * (a.N / BN_OUT);
    const int64_t grid = (tiles + kNumXcd - 1) / kNumXcd * kNumXcd;
    if (grid <= 0) return hipSuccess;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    ffn_gemm_dma_kernel<GATEUP, FP8><<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, s>>>(a);
    return hipGetLastError();
}

}  // namespace

// Tile height from the mean rows per expert (the host does not read the
// counts back).  16-row tiles while nearly every expert fits in one: a mean
// of at most 12 (at 128 tokens the mean is 4 and the busiest expert about
// 12).  Above that the large tile, which streams the weights as fast with few
// rows and takes up to 256 rows in one row tile.  Between the two, 16- or
// 64-row tiles split the busier experts into several row tiles, each of which
// streams that expert's weights again (3072 tokens: 5.8 ms per layer with
// 64-row tiles, 3.9 ms with the large tile).  The 64-row tile remains for
// shapes the large tile does not take.
constexpr int64_t kSmallTileMaxRows = 12;
// bf16 gate/up from there up to a mean of 32 rows per expert: 64-row tiles
// with the weights streamed past the caches (512 tokens: 2.10 against 2.27 ms
// on the large tile, 1024 tokens: 2.20 against 2.31 ms; at 1280 tokens they
// draw level).  The down projection stays on the large tile there (the
// 64-row tile was 2-6% slower for it).
constexpr int64_t kBf16MidTileMaxRows = 32;
// Weights stream past the caches when a 64-row tile covers an average
// expert: each weight is then read about once.
constexpr int64_t kStreamWeightsMaxRows = 64;
// With FP8 weights the large tile streams more slowly at few rows (it widens
// the codes inside its MFMA loop): 64-row tiles up to a mean of 48 rows
// (1536 tokens: 2.29 ms for the expert FFN against 2.44 ms), the large tile
// above (2048 tokens: 2.68 against 2.88 ms).
constexpr int64_t kFp8MidTileMaxRows = 48;

hipError_t launch_gate_up(const Problem& p, const uint16_t* x, const int32_t* sorted_pairs,
                          const int32_t* offsets, const uint16_t* w_gate, const uint16_t* w_up,
                          uint16_t* h, hipStream_t s) {
    const int64_t P = p.T * p.k;
    FfnArgs a{P, p.T, p.k, p.E, p.H, p.I, x, sorted_pairs, offsets, w_gate, w_up, h,
              nullptr, nullptr};
    const int64_t rows_per_expert = P / p.E;
    a.stream_w = rows_per_expert <= kStreamWeightsMaxRows;
    // weight streaming in stages of K = 128 (H % 128 == 0 holds for every
    // accepted problem)
    if (rows_per_expert <= kSmallTileMaxRows)
        return launch_gemm<16, 128, 1, 4, true, false, 128>(a, s);
    // the large-tile kernel addresses x with 32-bit buffer offsets
    const bool x_fits = p.T * static_cast<int64_t>(p.H) * 2 <= static_cast<int64_t>(kNoRowOffset);
    if (rows_per_expert <= kBf16MidTileMaxRows || p.I % 128 != 0 || !x_fits)
        return launch_gemm<64, 128, 1, 4, true>(a, s);
    return launch_gemm_dma<true>(a, s);
}

hipError_t launch_down(const Problem& p, const uint16_t* h, const int32_t* offsets,
                       const uint16_t* w_down, float* y, hipStream_t s) {
    const int64_t P = p.T * p.k;
    FfnArgs a{P, p.T, p.k, p.E, p.I, p.H, h, nullptr, offsets, w_down, nullptr, y, nullptr,
              nullptr};
    a.stream_out = P * static_cast<int64_t>(p.H) * 4 > kStreamBytes;
    const int64_t rows_per_expert = P / p.E;
    a.stream_w = rows_per_expert <= kStreamWeightsMaxRows;
    if (rows_per_expert <= kSmallTileMaxRows) {
        // stages of K = 128 where I allows
        if (p.I % 128 == 0) return launch_gemm<16, 64, 1, 4, false, false, 128>(a, s);
        return launch_gemm<16, 64, 1, 4, false>(a, s);
    }
    if (p.H % 256 != 0 || p.I % 128 != 0) return launch_gemm<64, 128, 1, 4, false>(a, s);
    return launch_gemm_dma<false>(a, s);
}

hipError_t launch_expert_ffn(const Problem& p, const uint16_t* x, const int32_t* sorted_pairs,
                             const int32_t* offsets, const uint16_t* w_gate,
                             const uint16_t* w_up, const uint16_t* w_down, uint16_t* h, float* y,
                             hipStream_t s) {
    const hipError_t err = launch_gate_up(p, x, sorted_pairs, offsets, w_gate, w_up, h, s);
    if (err != hipSuccess) return err;
    return launch_down(p, h, offsets, w_down, y, s);
}

hipError_t launch_expert_ffn_fp8(const Problem& p, const uint16_t* x, const int32_t* sorted_pairs,
                                 const int32_t* offsets, const uint8_t* w_gate,
                                 const float* s_gate, const uint8_t* w_up, const float* s_up,
                                 const uint8_t* w_down, const float* s_down, uint16_t* h,
                                 float* y, hipStream_t s) {
    const int64_t P = p.T * p.k;
    const int64_t rows_per_expert = P / p.E;
    FfnArgs gu{P, p.T, p.k, p.E, p.H, p.I, x, sorted_pairs, offsets, w_gate, w_up, h,
               s_gate, s_up};
    gu.stream_w = rows_per_expert <= kStreamWeightsMaxRows;
    // few rows per expert: the weight stream is the cost; stages of K = 128
    // make every weight row of a stage one whole 128-byte line (gate/up: K = H,
    // and H % 128 == 0 holds for every accepted problem; down: where I allows).
    // 256 weight rows per workgroup where the shape allows: a 32 KB weight
    // stage, the bytes in flight of the bf16 kernel (decode 2% faster, 384
    // tokens 4%, than 128 gate/up and 64 down rows)
    const bool x_fits = p.T * static_cast<int64_t>(p.H) * 2 <= static_cast<int64_t>(kNoRowOffset);
    hipError_t err;
    if (rows_per_expert <= kSmallTileMaxRows && p.I % 128 == 0)
        err = launch_gemm<16, 256, 1, 4, true, true, 128>(gu, s);
    else if (rows_per_expert <= kSmallTileMaxRows)
        err = launch_gemm<16, 128, 1, 4, true, true, 128>(gu, s);
    else if (rows_per_expert <= kFp8MidTileMaxRows || p.I % 128 != 0 || !x_fits)
        err = launch_gemm<64, 128, 1, 4, true, true, 128>(gu, s);
    else
        err = launch_gemm_dma<true, true>(gu, s);
    if (err != hipSuccess) return err;
    FfnArgs dn{P, p.T, p.k, p.E, p.I, p.H, h, nullptr, offsets, w_down, nullptr, y, s_down,
               nullptr};
    dn.stream_out = P * static_cast<int64_t>(p.H) * 4 > kStreamBytes;
    dn.stream_w = rows_per_expert <= kStreamWeightsMaxRows;
    if (rows_per_expert <= kSmallTileMaxRows && p.I % 128 == 0 && p.H % 256 == 0)
        return launch_gemm<16, 256, 1, 4, false, true, 128>(dn, s);
    if (rows_per_expert <= kSmallTileMaxRows && p.I % 128 == 0)
        return launch_gemm<16, 64, 1, 4, false, true, 128>(dn, s);
    if (rows_per_expert <= kFp8MidTileMaxRows || p.H % 256 != 0 || p.I % 128 != 0) {
        if (p.I % 128 == 0) return launch_gemm<64, 128, 1, 4, false, true, 128>(dn, s);
        return launch_gemm<64, 128, 1, 4, false, true>(dn, s);
    }
    return launch_gemm_dma<false, true>(dn, s);
}

}  // namespace moe
