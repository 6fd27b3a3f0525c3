/*
 * moe.h -- C ABI of libmoe.so: forward pass of one Beam-style
 * Mixture-of-Experts block on an AMD Instinct MI355X (gfx950).
 *
 * The operation ("Welcome Beam: a 501B open model you can own, customize, and
 * scale", section "Mixture of Experts"; the same text is in "Reflection
 * Releases Beam: An Open 501B MoE Model with 1M Context", section "Mixture of
 * Experts"): a router gives each of E experts a sigmoid score; the experts
 * form G groups of E/G consecutive indices; each group is ranked by the sum of
 * its two best scores and the TG best groups are kept; the k best experts of
 * the kept groups run on the token; their scores, normalised to sum to one,
 * weight the expert outputs, and the sum is multiplied by a scale (2.5 for
 * Beam).  Each expert is a SwiGLU MLP with intermediate size I.  Section
 * "Residual Stream" of the first page fixes the router and the SwiGLU product
 * in FP32.  Beam: H=5120, E=256, G=8, TG=4, k=8, I=2560, scale=2.5.
 *
 * Conventions for every call:
 *  - All tensor pointers are device memory owned by the caller, contiguous,
 *    row-major and 16-byte aligned.  bf16 tensors are passed as moe_bf16 (the
 *    raw 16-bit pattern).
 *  - The library never allocates, frees or synchronises; each call only
 *    enqueues kernels on `stream` (0 = the null stream).  No call reads
 *    results back to the host or clears memory with a memset, so a call can
 *    be captured into a HIP graph and replayed (the tile schedule of the
 *    expert GEMMs is derived on the device from expert_offsets).
 *  - Every argument is checked on the host before anything is enqueued.  On
 *    any error nothing is enqueued and no output is touched; the call returns
 *    a moe_status and moe_last_error() gives a message (per host thread).
 *    MOE_ERR_HIP means a launch was refused by the HIP runtime; kernels of the
 *    same call that were enqueued before it may have run.
 *  - Routing ties go to the lower index, for groups and for experts.  Scores
 *    are fp32; expert GEMMs multiply bf16 values and accumulate in fp32; the
 *    SwiGLU product is rounded to bf16 (nearest-even) before the down
 *    projection; expert outputs y stay fp32.
 *  - No call uses atomics on its outputs: results are deterministic run to
 *    run.
 *  - Calls that share a workspace or outputs on one stream are ordered by the
 *    stream; calls on different streams that share them race.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef uint16_t moe_bf16; /* bf16 bit pattern */

typedef enum moe_status {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1, /* null pointer, misalignment, inconsistent shape */
    MOE_ERR_UNSUPPORTED = 2, /* valid problem outside the kernels' limits       */
    MOE_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required      */
    MOE_ERR_HIP = 4          /* the HIP runtime refused a launch                */
} moe_status;

typedef enum moe_dtype { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;

/* Problem shape.
 *   T  tokens (>= 0; T = 0 is a no-op that returns MOE_OK)
 *   H  hidden size,        H % 64 == 0 (H % 128 == 0 and H <= 65536 for the
 *      kernels, else MOE_ERR_UNSUPPORTED)
 *   I  expert intermediate size, I % 64 == 0 (I <= 65536 for the kernels)
 *   E  experts, 1 <= E <= 256
 *   G  groups, E % G == 0; group g holds experts [g*E/G, (g+1)*E/G)
 *   TG kept groups, 1 <= TG <= G
 *   k  experts per token, 1 <= k <= TG*E/G and k <= 16
 *   scale  factor applied to the weighted sum (2.5 for Beam)
 * T*k must fit in int32. */
typedef struct moe_problem {
    int64_t T;
    int32_t H, I, E, G, TG, k;
    float scale;
} moe_problem;

/* Bytes of scratch every call below needs in `ws` for problem p (0 if p is
 * invalid).  The largest part is the bf16 SwiGLU product [T*k, I].  One
 * workspace sized by this function serves every call. */
size_t moe_workspace_bytes(const moe_problem* p);

/* Router and group-limited selection for T tokens ("Welcome Beam: a 501B open
 * model you can own, customize, and scale", section "Mixture of Experts": a
 * sigmoid score per expert, groups ranked by their two best scores, the best
 * groups kept, the top k experts of those groups, normalised weights).
 *   x            [T,H] bf16 activations
 *   w_router     [E,H] bf16 router weight
 *   bias         [E] fp32 added to each logit before the sigmoid, or NULL (0)
 *   topk_ids     [T,k] int32 out: chosen experts, best score first
 *   topk_weights [T,k] fp32 out: chosen scores / their sum (sum to 1)
 * Scores are sigmoid(x . w_router[e] + bias[e]) with fp32 accumulation. */
moe_status moe_route(const moe_problem* p, const moe_bf16* x, const moe_bf16* w_router,
                     const float* bias, int32_t* topk_ids, float* topk_weights,
                     hipStream_t stream);

/* Dispatch: stable counting sort of the T*k pairs p = t*k + j by expert (the
 * same section: only the k chosen experts run on a token, so each expert's
 * tokens are gathered into one contiguous run of rows).
 *   topk_ids       [T,k] int32 in: expert of each pair, 0 <= id < E
 *   expert_offsets [E+1] int32 out: first sorted position of each expert;
 *                  expert_offsets[E] = T*k
 *   sorted_pairs   [T*k] int32 out: pair ids grouped by expert, increasing
 *                  pair id inside each expert
 *   pair_rows      [T*k] int32 out: inverse of sorted_pairs
 * Uses the permutation scratch of `ws`.  Ids outside [0,E) are dropped:
 * their pair_rows entry is -1 and expert_offsets[E] counts only kept pairs. */
moe_status moe_permute(const moe_problem* p, const int32_t* topk_ids, int32_t* expert_offsets,
                       int32_t* sorted_pairs, int32_t* pair_rows, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* Expert SwiGLU MLPs over the sorted pairs (the same section: every expert is
 * a SwiGLU MLP; section "Residual Stream": the SwiGLU product in FP32).
 *   x              [T,H] bf16; row of pair q is x[sorted_pairs[q] / k]
 *   sorted_pairs, expert_offsets   as written by moe_permute
 *   w_gate, w_up   [E,I,H] bf16;  w_down [E,H,I] bf16
 *   y              [T*k,H] fp32 out, sorted order: y[q] is the output of the
 *                  expert that owns position q for the token of pair
 *                  sorted_pairs[q]
 * h[q] = bf16(silu(x_q . w_gate[e]^T) * (x_q . w_up[e]^T)) goes to `ws`;
 * y[q] = h[q] . w_down[e]^T.  The tile schedule is derived on the device from
 * expert_offsets, so no host read of device data is needed.  Rows of y past
 * expert_offsets[E] are not written. */
moe_status moe_expert_ffn(const moe_problem* p, const moe_bf16* x, const int32_t* sorted_pairs,
                          const int32_t* expert_offsets, const moe_bf16* w_gate,
                          const moe_bf16* w_up, const moe_bf16* w_down, float* y, void* ws,
                          size_t ws_bytes, hipStream_t stream);

/* The two halves of moe_expert_ffn, for callers that keep h themselves.
 *   moe_expert_gate_up:  h [T*k,I] bf16 out (sorted order),
 *       h[q] = bf16(silu(x_q . w_gate[e]^T) * (x_q . w_up[e]^T)),
 *       x_q = x[sorted_pairs[q] / k], e the expert owning position q.
 *   moe_expert_down:     y [T*k,H] fp32 out, y[q] = h[q] . w_down[e]^T.
 * Same layouts, tile schedule and rounding as moe_expert_ffn, which is
 * exactly these two calls with h in the workspace.  No workspace needed. */
moe_status moe_expert_gate_up(const moe_problem* p, const moe_bf16* x, const int32_t* sorted_pairs,
                              const int32_t* expert_offsets, const moe_bf16* w_gate,
                              const moe_bf16* w_up, moe_bf16* h, hipStream_t stream);

moe_status moe_expert_down(const moe_problem* p, const moe_bf16* h, const int32_t* expert_offsets,
                           const moe_bf16* w_down, float* y, hipStream_t stream);

/* Weighted recombination without atomics (the same section: the expert outputs
 * are summed with the normalised router weights and scaled by 2.5 for Beam).
 *   y            [T*k,H] fp32 in sorted order
 *   pair_rows    [T*k] int32 (from moe_permute); -1 entries contribute 0
 *   topk_weights [T,k] fp32
 *   out          [T,H] fp32 or bf16 (out_dtype):
 *                out[t] = scale * sum_{j=0..k-1} w[t,j] * y[pair_rows[t*k+j]],
 *                summed in j order in fp32; bf16 output is the
 *                round-to-nearest-even cast of that fp32 value. */
moe_status moe_combine(const moe_problem* p, const float* y, const int32_t* pair_rows,
                       const float* topk_weights, void* out, moe_dtype out_dtype,
                       hipStream_t stream);

/* The combine fused with the sublayer epilogue that follows it ("Welcome Beam:
 * a 501B open model you can own, customize, and scale", section "Residual
 * Stream": every sublayer output is normalised; the embedding is step 1 of
 * the residual stream and step s adds the normalised output with weight
 * 1/sqrt(s) while the stream keeps weight sqrt((s-1)/s); the norms compute in
 * FP32).  The norm is RMSNorm with a per-channel gain.
 *   y, pair_rows, topk_weights   as for moe_combine
 *   norm_weight  [H] fp32 gain g
 *   eps          > 0, added to the mean square
 *   step         s >= 1 (s = 1 replaces the stream)
 *   residual     [T,H] fp32, updated in place:
 *                o        = the fp32 row moe_combine would write for token t
 *                res[t,m] = sqrt((s-1)/s) * res[t,m]
 *                           + (1/sqrt(s)) * g[m] * o[m] / sqrt(mean(o^2) + eps)
 * The combined output itself is not written.  H <= 16384 (else
 * MOE_ERR_UNSUPPORTED).  The sum of squares is reduced in a fixed order, so
 * the result is deterministic. */
moe_status moe_combine_residual(const moe_problem* p, const float* y, const int32_t* pair_rows,
                                const float* topk_weights, const float* norm_weight, float eps,
                                int32_t step, float* residual, hipStream_t stream);

/* Dense SwiGLU MLP on the expert kernels ("Welcome Beam: a 501B open model you
 * can own, customize, and scale", section "Mixture of Experts": the first
 * layers use a dense SwiGLU MLP instead of the expert block).
 *   p         E = G = TG = k = 1 (else MOE_ERR_INVALID_ARG); scale unused;
 *             I is the MLP's intermediate size
 *   x         [T,H] bf16
 *   w_gate, w_up  [I,H] bf16;  w_down [H,I] bf16
 *   out       [T,H] fp32: out[t] = bf16(silu(x_t . w_gate^T) * (x_t . w_up^T))
 *             . w_down^T, the same arithmetic as one expert of moe_expert_ffn
 *   ws        moe_workspace_bytes(p) bytes (holds the bf16 product [T,I]) */
moe_status moe_dense_mlp(const moe_problem* p, const moe_bf16* x, const moe_bf16* w_gate,
                         const moe_bf16* w_up, const moe_bf16* w_down, float* out, void* ws,
                         size_t ws_bytes, hipStream_t stream);

/* FP8 expert weights.  The pages give no FP8 scheme for the experts; the one
 * taken: every weight matrix is stored as FP8 E4M3 codes (the OCP e4m3fn
 * encoding: bias 7, no infinities, 0x7f/0xff NaN) with one fp32 scale per
 * output channel, and a channel's dot product is its scale times the dot
 * product with the decoded codes:
 *   g[n] = s_gate[e,n] * (x_q . w_gate[e,n]),  u[n] = s_up[e,n] * (x_q . w_up[e,n])
 *   h[n] = bf16(silu(g[n]) * u[n]),            y[m] = s_down[e,m] * (h . w_down[e,m])
 * Activations, h, y and every accumulation are as in the bf16 calls; the codes
 * are widened to bf16 exactly and multiplied on the bf16 MFMA path.  Halves
 * the bytes of the weight stream.
 *   w_gate, w_up  [E,I,H] uint8 codes;  s_gate, s_up  [E,I] fp32
 *   w_down        [E,H,I] uint8 codes;  s_down        [E,H] fp32
 * Everything else as moe_expert_ffn / moe_forward. */
moe_status moe_expert_ffn_fp8(const moe_problem* p, const moe_bf16* x,
                              const int32_t* sorted_pairs, const int32_t* expert_offsets,
                              const uint8_t* w_gate, const float* s_gate, const uint8_t* w_up,
                              const float* s_up, const uint8_t* w_down, const float* s_down,
                              float* y, void* ws, size_t ws_bytes, hipStream_t stream);

moe_status moe_forward_fp8(const moe_problem* p, const moe_bf16* x, const moe_bf16* w_router,
                           const float* bias, const uint8_t* w_gate, const float* s_gate,
                           const uint8_t* w_up, const float* s_up, const uint8_t* w_down,
                           const float* s_down, void* out, moe_dtype out_dtype,
                           int32_t* topk_ids, float* topk_weights, float* y, void* ws,
                           size_t ws_bytes, hipStream_t stream);

/* The whole block: route, permute, expert FFN, combine ("Welcome Beam: a 501B
 * open model you can own, customize, and scale", section "Mixture of Experts").
 *   topk_ids, topk_weights  optional [T,k] outputs (NULL: kept in `ws`)
 *   y                       [T*k,H] fp32 caller buffer for expert outputs
 *   out                     [T,H] in out_dtype
 * Routing gives the same ids and weights, bit for bit, as moe_route; for up
 * to 512 tokens the scores pass through the part of `ws` that later holds
 * the SwiGLU product. */
moe_status moe_forward(const moe_problem* p, const moe_bf16* x, const moe_bf16* w_router,
                       const float* bias, const moe_bf16* w_gate, const moe_bf16* w_up,
                       const moe_bf16* w_down, void* out, moe_dtype out_dtype, int32_t* topk_ids,
                       float* topk_weights, float* y, void* ws, size_t ws_bytes,
                       hipStream_t stream);

/* moe_forward for callers that cannot allocate (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument.  The workspace is a fixed array of MOE_NOALLOC_SCRATCH_BYTES in
 * device memory inside the library, one copy per GPU, held until the process
 * ends; the call allocates and frees nothing.  Problems that need more
 * (moe_workspace_bytes(p) > MOE_NOALLOC_SCRATCH_BYTES; at Beam's sizes about
 * 1600 tokens) return MOE_ERR_UNSUPPORTED before anything is enqueued.
 * Arguments, outputs and results are those of moe_forward, bit for bit.
 * Every call on one GPU shares that GPU's array: calls that overlap on one
 * GPU (two streams, two host threads) race and give undefined results; calls
 * ordered on one stream are safe.  The first call on a GPU looks the array up
 * (hipGetSymbolAddress); make it outside graph capture. */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)

moe_status moe_forward_noalloc(const moe_problem* p, const moe_bf16* x, const moe_bf16* w_router,
                               const float* bias, const moe_bf16* w_gate, const moe_bf16* w_up,
                               const moe_bf16* w_down, void* out, moe_dtype out_dtype,
                               int32_t* topk_ids, float* topk_weights, float* y,
                               hipStream_t stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status s);

/* Message of the last failed call on this host thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
