/*
 * Calls libla_decode from plain C through include/la_decode.h: device buffers
 * from the HIP runtime, host context lengths, one la_decode_bf16 call and one
 * la_decode_ex call (kind auto, 4 K/V heads for 8 query heads); then a decode
 * step on a [B, H, S, D] cache with the lengths in device memory, captured
 * into a HIP graph on a stream of its own and replayed STEPS times, the
 * lengths raised by one token between replays. Writes the inputs' bit
 * patterns and all outputs to a file for the test to check against the
 * oracle. Test infrastructure (tests/test_c_abi.py).
 *
 * Usage: decode_from_c OUTFILE. Exit status 0 on success.
 */
#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "la_decode.h"

enum { B = 2, H = 8, HK = 4, D = 128, S = 1024, STEPS = 3 };
static const int32_t kLens[B] = {300, 1000};

/* xorshift64*, mapped to roughly N(0,1) by summing four uniforms */
static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static float draw(void) {
    float s = 0.f;
    for (int i = 0; i < 4; ++i) {
        g_state ^= g_state >> 12;
        g_state ^= g_state << 25;
        g_state ^= g_state >> 27;
        const uint64_t x = g_state * 0x2545F4914F6CDD1Dull;
        s += (float)(x >> 40) / (float)(1ull << 24) - 0.5f;
    }
    return s * 1.7320508f;
}

/* fp32 -> bf16 bits, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

#define CHECK_HIP(x) do { if ((x) != hipSuccess) { fprintf(stderr, "%s failed\n", #x); return 2; } } while (0)
#define CHECK_LA(x) do { la_status s_ = (x); if (s_ != LA_OK) { fprintf(stderr, "%s: %d %s\n", #x, (int)s_, la_last_error()); return 3; } } while (0)

int main(int argc, char** argv) {
    if (argc != 2) return 1;
    int64_t n = 0;
    for (int b = 0; b < B; ++b) n += kLens[b];
    const size_t nq = (size_t)B * H * D, nkv = (size_t)HK * n * D, nkv_mha = (size_t)H * n * D;
    uint16_t* q = malloc(nq * 2);
    uint16_t* k = malloc(nkv_mha * 2);
    uint16_t* v = malloc(nkv_mha * 2);
    float* out1 = malloc(nq * 4);
    float* out2 = malloc(nq * 4);
    if (!q || !k || !v || !out1 || !out2) return 1;
    for (size_t i = 0; i < nq; ++i) q[i] = to_bf16(draw());
    for (size_t i = 0; i < nkv_mha; ++i) k[i] = to_bf16(draw());
    for (size_t i = 0; i < nkv_mha; ++i) v[i] = to_bf16(draw());

    void *dq, *dk, *dv;
    float* dout;
    CHECK_HIP(hipMalloc(&dq, nq * 2));
    CHECK_HIP(hipMalloc(&dk, nkv_mha * 2));
    CHECK_HIP(hipMalloc(&dv, nkv_mha * 2));
    CHECK_HIP(hipMalloc((void**)&dout, nq * 4));
    CHECK_HIP(hipMemcpy(dq, q, nq * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dk, k, nkv_mha * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dv, v, nkv_mha * 2, hipMemcpyHostToDevice));
    const float scale = 0.08838834764831845f;   /* 1/sqrt(128) */

    /* 1: plain multi-head decode with the plain argument list */
    CHECK_LA(la_decode_bf16(dq, dk, dv, kLens, B, H, D, scale, dout, NULL));
    CHECK_LA(la_sync_check(NULL));
    CHECK_HIP(hipMemcpy(out1, dout, nq * 4, hipMemcpyDeviceToHost));

    /* 2: the same q over the first HK * n rows as 4 grouped K/V heads, kind auto */
    la_opts o;
    la_opts_init(&o);
    o.dtype = LA_BF16;
    o.kind = LA_KIND_AUTO;
    o.kv_heads = HK;
    CHECK_LA(la_decode_ex(dq, dk, dv, kLens, B, H, D, scale, dout, NULL, &o));
    CHECK_LA(la_sync_check(NULL));
    CHECK_HIP(hipMemcpy(out2, dout, nq * 4, hipMemcpyDeviceToHost));

    /* 3: lengths on the device, one decode step captured into a graph */
    const size_t ncache = (size_t)B * H * S * D;
    uint16_t* ks = malloc(ncache * 2);
    uint16_t* vs = malloc(ncache * 2);
    float* out3 = malloc(nq * 4 * STEPS);
    if (!ks || !vs || !out3) return 1;
    for (size_t i = 0; i < ncache; ++i) ks[i] = to_bf16(draw());
    for (size_t i = 0; i < ncache; ++i) vs[i] = to_bf16(draw());
    void *dks, *dvs;
    int32_t* dlens;
    CHECK_HIP(hipMalloc(&dks, ncache * 2));
    CHECK_HIP(hipMalloc(&dvs, ncache * 2));
    CHECK_HIP(hipMalloc((void**)&dlens, B * sizeof(int32_t)));
    CHECK_HIP(hipMemcpy(dks, ks, ncache * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dvs, vs, ncache * 2, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dlens, kLens, B * sizeof(int32_t), hipMemcpyHostToDevice));
    hipStream_t st;
    CHECK_HIP(hipStreamCreate(&st));
    la_opts_init(&o);
    o.dtype = LA_BF16;
    o.kv_stride = S;
    o.ctx_lens_device = dlens;
    /* an eager call sizes the stream's workspace; capture needs it */
    CHECK_LA(la_decode_ex(dq, dks, dvs, NULL, B, H, D, scale, dout, st, &o));
    CHECK_LA(la_sync_check(st));
    hipGraph_t graph;
    hipGraphExec_t exec;
    CHECK_HIP(hipStreamBeginCapture(st, hipStreamCaptureModeGlobal));
    const la_status cap = la_decode_ex(dq, dks, dvs, NULL, B, H, D, scale, dout, st, &o);
    CHECK_HIP(hipStreamEndCapture(st, &graph));
    CHECK_LA(cap);
    CHECK_HIP(hipGraphInstantiateWithFlags(&exec, graph, 0));
    for (int i = 0; i < STEPS; ++i) {
        int32_t lens[B];
        for (int b = 0; b < B; ++b) lens[b] = kLens[b] + i + 1;
        CHECK_HIP(hipMemcpy(dlens, lens, sizeof(lens), hipMemcpyHostToDevice));
        CHECK_HIP(hipGraphLaunch(exec, st));
        CHECK_HIP(hipStreamSynchronize(st));
        CHECK_LA(la_sync_check(st));
        CHECK_HIP(hipMemcpy(out3 + (size_t)i * nq, dout, nq * 4, hipMemcpyDeviceToHost));
    }
    CHECK_HIP(hipGraphExecDestroy(exec));
    CHECK_HIP(hipGraphDestroy(graph));

    FILE* f = fopen(argv[1], "wb");
    if (!f) return 1;
    const int32_t hdr[4] = {B, H, HK, D};
    fwrite(hdr, 4, 4, f);
    fwrite(kLens, 4, B, f);
    fwrite(q, 2, nq, f);
    fwrite(k, 2, nkv_mha, f);
    fwrite(v, 2, nkv_mha, f);
    fwrite(out1, 4, nq, f);
    fwrite(out2, 4, nq, f);
    fwrite(ks, 2, ncache, f);
    fwrite(vs, 2, ncache, f);
    fwrite(out3, 4, nq * STEPS, f);
    fclose(f);
    la_shutdown();
    CHECK_HIP(hipStreamDestroy(st));
    (void)nkv;
    return 0;
}
