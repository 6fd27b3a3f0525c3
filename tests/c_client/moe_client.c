/*
 * moe_client.c -- a plain C11 program that drives libmoe.so through
 * include/moe.h alone: no Python, no torch.  Device memory and the stream come
 * from the HIP runtime's C API; the inputs come from this file's own seeded
 * generator.  It checks the host-side argument errors, runs moe_forward with
 * fp32 and with bf16 output, and writes the inputs and outputs as raw files
 * for tests/test_gpu_c_client.py, which compares them with the oracle.
 *
 *   moe_client OUTDIR T H I E G TG K SCALE SEED
 *
 * Files written to OUTDIR (little-endian, row-major):
 *   x.bin [T,H] u16, w_router.bin [E,H] u16, bias.bin [E] f32,
 *   w_gate.bin [E,I,H] u16, w_up.bin [E,I,H] u16, w_down.bin [E,H,I] u16,
 *   out.bin [T,H] f32, out_bf16.bin [T,H] u16, ids.bin [T,K] i32,
 *   weights.bin [T,K] f32
 * Exit status 0 when every call behaved as documented.
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe.h"

#define CHECK_HIP(call)                                                              \
    do {                                                                             \
        hipError_t e_ = (call);                                                      \
        if (e_ != hipSuccess) {                                                      \
            fprintf(stderr, "%s:%d: %s -> %s\n", __FILE__, __LINE__, #call,          \
                    hipGetErrorString(e_));                                          \
            exit(2);                                                                 \
        }                                                                            \
    } while (0)

#define EXPECT(cond, ...)                           \
    do {                                            \
        if (!(cond)) {                              \
            fprintf(stderr, "FAIL: " __VA_ARGS__);  \
            fprintf(stderr, "\n");                  \
            exit(1);                                \
        }                                           \
    } while (0)

/* splitmix64: a counter-based 64-bit generator (Steele, Lea, Flood 2014) */
static uint64_t g_state;
static uint64_t next_u64(void) {
    uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
/* uniform in (0, 1): 53 random bits, never 0 */
static double next_unit(void) { return ((double)(next_u64() >> 11) + 0.5) * (1.0 / 9007199254740992.0); }
/* standard normal by the Box-Muller transform (one value per pair of draws) */
static double next_normal(void) {
    const double u1 = next_unit(), u2 = next_unit();
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586 * u2);
}
/* nearest-even bf16 of a finite float (inputs only) */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}
static uint16_t* normal_bf16(size_t n, double sd) {
    uint16_t* p = (uint16_t*)malloc(n * 2);
    EXPECT(p != NULL, "host allocation of %zu values", n);
    for (size_t i = 0; i < n; ++i) p[i] = to_bf16((float)(sd * next_normal()));
    return p;
}

static void* to_device(const void* host, size_t bytes) {
    void* d = NULL;
    CHECK_HIP(hipMalloc(&d, bytes > 0 ? bytes : 1));
    if (host != NULL && bytes > 0) CHECK_HIP(hipMemcpy(d, host, bytes, hipMemcpyHostToDevice));
    return d;
}
static void* from_device(const void* dev, size_t bytes) {
    void* h = malloc(bytes > 0 ? bytes : 1);
    EXPECT(h != NULL, "host allocation of %zu bytes", bytes);
    CHECK_HIP(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
    return h;
}
static void write_file(const char* dir, const char* name, const void* p, size_t bytes) {
    char path[4096];
    snprintf(path, sizeof path, "%s/%s", dir, name);
    FILE* f = fopen(path, "wb");
    EXPECT(f != NULL, "cannot open %s", path);
    EXPECT(fwrite(p, 1, bytes, f) == bytes, "short write to %s", path);
    fclose(f);
}

int main(int argc, char** argv) {
    if (argc != 11) {
        fprintf(stderr, "usage: %s OUTDIR T H I E G TG K SCALE SEED\n", argv[0]);
        return 2;
    }
    const char* dir = argv[1];
    moe_problem p;
    p.T = atoll(argv[2]);
    p.H = atoi(argv[3]);
    p.I = atoi(argv[4]);
    p.E = atoi(argv[5]);
    p.G = atoi(argv[6]);
    p.TG = atoi(argv[7]);
    p.k = atoi(argv[8]);
    p.scale = (float)atof(argv[9]);
    g_state = strtoull(argv[10], NULL, 10);
    EXPECT(p.T > 0 && p.H > 0 && p.I > 0 && p.E > 0 && p.k > 0, "positive sizes");

    const size_t T = (size_t)p.T, H = (size_t)p.H, I = (size_t)p.I, E = (size_t)p.E,
                 K = (size_t)p.k;
    /* inputs: x ~ N(0, 1), weights ~ N(0, 0.02), a zero router bias */
    uint16_t* x = normal_bf16(T * H, 1.0);
    uint16_t* wr = normal_bf16(E * H, 0.02);
    uint16_t* wg = normal_bf16(E * I * H, 0.02);
    uint16_t* wu = normal_bf16(E * I * H, 0.02);
    uint16_t* wd = normal_bf16(E * H * I, 0.02);
    float* bias = (float*)calloc(E, sizeof(float));
    EXPECT(bias != NULL, "host allocation");

    CHECK_HIP(hipSetDevice(0));
    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    void* d_x = to_device(x, T * H * 2);
    void* d_wr = to_device(wr, E * H * 2);
    void* d_b = to_device(bias, E * 4);
    void* d_wg = to_device(wg, E * I * H * 2);
    void* d_wu = to_device(wu, E * I * H * 2);
    void* d_wd = to_device(wd, E * H * I * 2);
    void* d_out = to_device(NULL, T * H * 4);
    void* d_out16 = to_device(NULL, T * H * 2);
    void* d_ids = to_device(NULL, T * K * 4);
    void* d_w = to_device(NULL, T * K * 4);
    void* d_y = to_device(NULL, T * K * H * 4);
    const size_t ws_bytes = moe_workspace_bytes(&p);
    EXPECT(ws_bytes > 0, "workspace size for a valid problem");
    void* d_ws = to_device(NULL, ws_bytes);

    /* host-side errors: nothing is enqueued, the status and message say why */
    moe_problem bad = p;
    bad.G = p.E + 1;
    moe_status st = moe_forward(&bad, (const moe_bf16*)d_x, (const moe_bf16*)d_wr, (const float*)d_b,
                                (const moe_bf16*)d_wg, (const moe_bf16*)d_wu,
                                (const moe_bf16*)d_wd, d_out, MOE_DTYPE_F32, (int32_t*)d_ids,
                                (float*)d_w, (float*)d_y, d_ws, ws_bytes, stream);
    EXPECT(st == MOE_ERR_INVALID_ARG, "bad group count gave status %d", (int)st);
    EXPECT(strlen(moe_last_error()) > 0, "an error message after a failed call");
    st = moe_forward(&p, (const moe_bf16*)d_x, (const moe_bf16*)d_wr, (const float*)d_b,
                     (const moe_bf16*)d_wg, (const moe_bf16*)d_wu, (const moe_bf16*)d_wd, d_out,
                     MOE_DTYPE_F32, (int32_t*)d_ids, (float*)d_w, (float*)d_y, d_ws, ws_bytes - 1,
                     stream);
    EXPECT(st == MOE_ERR_WORKSPACE, "short workspace gave status %d", (int)st);
    st = moe_forward(&p, NULL, (const moe_bf16*)d_wr, (const float*)d_b, (const moe_bf16*)d_wg,
                     (const moe_bf16*)d_wu, (const moe_bf16*)d_wd, d_out, MOE_DTYPE_F32,
                     (int32_t*)d_ids, (float*)d_w, (float*)d_y, d_ws, ws_bytes, stream);
    EXPECT(st == MOE_ERR_INVALID_ARG, "null x gave status %d", (int)st);
    EXPECT(strcmp(moe_status_string(MOE_OK), moe_status_string(MOE_ERR_HIP)) != 0,
           "distinct status strings");

    /* the forward pass, fp32 output and then bf16 output */
    st = moe_forward(&p, (const moe_bf16*)d_x, (const moe_bf16*)d_wr, (const float*)d_b,
                     (const moe_bf16*)d_wg, (const moe_bf16*)d_wu, (const moe_bf16*)d_wd, d_out,
                     MOE_DTYPE_F32, (int32_t*)d_ids, (float*)d_w, (float*)d_y, d_ws, ws_bytes,
                     stream);
    EXPECT(st == MOE_OK, "moe_forward: %s (%s)", moe_status_string(st), moe_last_error());
    st = moe_forward(&p, (const moe_bf16*)d_x, (const moe_bf16*)d_wr, (const float*)d_b,
                     (const moe_bf16*)d_wg, (const moe_bf16*)d_wu, (const moe_bf16*)d_wd, d_out16,
                     MOE_DTYPE_BF16, NULL, NULL, (float*)d_y, d_ws, ws_bytes, stream);
    EXPECT(st == MOE_OK, "moe_forward bf16: %s (%s)", moe_status_string(st), moe_last_error());
    CHECK_HIP(hipStreamSynchronize(stream));

    void* out = from_device(d_out, T * H * 4);
    void* out16 = from_device(d_out16, T * H * 2);
    void* ids = from_device(d_ids, T * K * 4);
    void* w = from_device(d_w, T * K * 4);
    write_file(dir, "x.bin", x, T * H * 2);
    write_file(dir, "w_router.bin", wr, E * H * 2);
    write_file(dir, "bias.bin", bias, E * 4);
    write_file(dir, "w_gate.bin", wg, E * I * H * 2);
    write_file(dir, "w_up.bin", wu, E * I * H * 2);
    write_file(dir, "w_down.bin", wd, E * H * I * 2);
    write_file(dir, "out.bin", out, T * H * 4);
    write_file(dir, "out_bf16.bin", out16, T * H * 2);
    write_file(dir, "ids.bin", ids, T * K * 4);
    write_file(dir, "weights.bin", w, T * K * 4);

    void* dev[] = {d_x, d_wr, d_b, d_wg, d_wu, d_wd, d_out, d_out16, d_ids, d_w, d_y, d_ws};
    for (size_t i = 0; i < sizeof dev / sizeof dev[0]; ++i) CHECK_HIP(hipFree(dev[i]));
    CHECK_HIP(hipStreamDestroy(stream));
    void* host[] = {x, wr, wg, wu, wd, bias, out, out16, ids, w};
    for (size_t i = 0; i < sizeof host / sizeof host[0]; ++i) free(host[i]);
    printf("moe_client ok: T=%lld H=%d I=%d E=%d G=%d TG=%d k=%d workspace=%zu bytes\n",
           (long long)p.T, p.H, p.I, p.E, p.G, p.TG, p.k, ws_bytes);
    return 0;
}
