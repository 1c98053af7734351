// Sanitizer driver for the library's host code (test infrastructure): the
// C-ABI's size queries, argument checks, error messages and mode switches,
// built host-only under AddressSanitizer and UndefinedBehaviorSanitizer.
// Only calls that return before any device work are made; on a machine
// that has a HIP device the calls that would reach one are skipped.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "coli_moe.h"

static int failures = 0;

static void expect(bool ok, const char *what) {
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s (last error: %s)\n", what, coli_moe_last_error());
        ++failures;
    }
}

static coli_moe_dims dims(int H, int I, int E, int K, int ns, int bits, int group, int fmt) {
    coli_moe_dims d;
    std::memset(&d, 0, sizeof d);
    d.hidden = H;
    d.inter = I;
    d.n_experts = E;
    d.top_k = K;
    d.n_shared = ns;
    d.wbits = bits;
    d.routed_scaling_factor = 2.5f;
    d.norm_topk_prob = 1;
    d.group_size = group;
    d.wformat = fmt;
    return d;
}

int main() {
    // valid shapes, including the limits of every field
    const coli_moe_dims good[] = {
        dims(256, 32, 1, 1, 0, 8, 0, 0),        dims(256, 128, 16, 2, 1, 4, 0, 0),
        dims(6144, 2048, 256, 8, 1, 4, 0, 0),   dims(6144, 2048, 256, 8, 1, 4, 64, 0),
        dims(6144, 2048, 256, 8, 1, 4, 0, 1),   dims(16384, 16384, 1024, 32, 1, 8, 0, 0),
        dims(16384, 16384, 1024, 32, 1, 4, 512, 0), dims(16384, 16384, 1024, 32, 1, 4, 0, 1),
        dims(512, 96, 9, 9, 0, 2, 0, 0),
    };
    const int32_t tokens[] = {0, 1, 2, 8, 9, 132, 2048, 4096, 65536};
    for (const auto &d : good) {
        const size_t eb = coli_moe_expert_bytes(&d);
        expect(eb > 0 && eb % 256 == 0, "expert_bytes of a valid shape");
        size_t prev = 0;
        for (int32_t s : tokens) {
            const size_t ws = coli_moe_workspace_bytes(&d, s);
            expect(ws > 0 && ws % 256 == 0 && ws >= prev, "workspace_bytes grows with tokens");
            prev = ws;
        }
        expect(coli_moe_workspace_bytes(&d, -1) == 0, "workspace_bytes(-1)");
        expect(coli_moe_workspace_bytes(&d, INT32_MAX) == 0, "workspace_bytes beyond the token limit");
    }
    // invalid shapes
    const coli_moe_dims bad[] = {
        dims(0, 32, 1, 1, 0, 8, 0, 0),         dims(255, 32, 1, 1, 0, 8, 0, 0),
        dims(16640, 32, 1, 1, 0, 8, 0, 0),     dims(256, 0, 1, 1, 0, 8, 0, 0),
        dims(256, 33, 1, 1, 0, 8, 0, 0),       dims(256, 32, 0, 1, 0, 8, 0, 0),
        dims(256, 32, 1025, 1, 0, 8, 0, 0),    dims(256, 32, 4, 5, 0, 8, 0, 0),
        dims(256, 32, 64, 33, 0, 8, 0, 0),     dims(256, 32, 4, 0, 0, 8, 0, 0),
        dims(256, 32, 4, 1, 2, 8, 0, 0),       dims(256, 32, 4, 1, 0, 3, 0, 0),
        dims(256, 64, 4, 1, 0, 4, 48, 0),      dims(256, 64, 4, 1, 0, 8, 64, 0),
        dims(256, 64, 4, 1, 0, 4, 1024, 0),    dims(256, 128, 4, 1, 0, 4, 0, 2),
        dims(256, 128, 4, 1, 0, 8, 0, 1),      dims(256, 96, 4, 1, 0, 4, 0, 1),
        dims(INT32_MAX - 255, 32, 1, 1, 0, 8, 0, 0), dims(INT32_MIN, INT32_MIN, INT32_MIN, INT32_MIN, 0, 4, 0, 0),
    };
    for (const auto &d : bad) {
        expect(coli_moe_expert_bytes(&d) == 0, "expert_bytes of an invalid shape");
        expect(coli_moe_workspace_bytes(&d, 8) == 0, "workspace_bytes of an invalid shape");
        expect(std::strlen(coli_moe_last_error()) > 0, "invalid shape leaves a message");
    }
    expect(coli_moe_expert_bytes(nullptr) == 0, "expert_bytes(NULL)");

    // argument checks that return before any device work
    const coli_moe_dims d = dims(256, 128, 16, 2, 1, 4, 0, 0);
    alignas(16) static float x[4 * 256], W[16 * 256], out[4 * 256], tw[8];
    alignas(16) static int32_t ti[8];
    alignas(256) static uint8_t ws[1 << 20], blob[65536];
    const void *blobs[16];
    for (auto &b : blobs) b = blob;
    const size_t wsb = coli_moe_workspace_bytes(&d, 4);
    expect(wsb <= sizeof ws, "test workspace big enough");
    expect(coli_moe_route(&d, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == COLI_OK,
           "route of 0 tokens is a no-op");
    expect(coli_moe_route(&d, -1, x, W, nullptr, ti, tw, ws, wsb, nullptr) == COLI_EINVAL, "route n<0");
    expect(coli_moe_route(&d, 4, nullptr, W, nullptr, ti, tw, ws, wsb, nullptr) == COLI_EINVAL, "route NULL x");
    expect(coli_moe_route(&d, 4, x + 1, W, nullptr, ti, tw, ws, wsb, nullptr) == COLI_EINVAL, "route unaligned x");
    expect(coli_moe_route(&d, 4, x, W, nullptr, ti, tw, ws, 64, nullptr) == COLI_EWORKSPACE, "route small ws");
    expect(coli_moe_route(&d, 70000, x, W, nullptr, ti, tw, ws, wsb, nullptr) == COLI_EINVAL,
           "route beyond the token limit");
    expect(coli_moe_forward(&d, 0, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                            0, nullptr) == COLI_OK, "forward of 0 tokens");
    expect(coli_moe_forward(&d, 4, x, ti, tw, blobs, nullptr, nullptr, nullptr, out, ws, wsb, nullptr) ==
               COLI_ENOTRESIDENT, "forward without the shared blob");
    expect(coli_moe_forward(&d, 4, x, ti, tw, blobs, blob + 4, nullptr, nullptr, out, ws, wsb, nullptr) ==
               COLI_EINVAL, "forward unaligned shared blob");
    expect(coli_moe_forward(&d, 4, x, ti, tw, nullptr, blob, nullptr, nullptr, out, ws, wsb, nullptr) == COLI_EINVAL,
           "forward NULL blob array");
    expect(coli_moe_forward(&d, 4, x, ti, tw, blobs, blob, nullptr, nullptr, out, ws, 255, nullptr) ==
               COLI_EWORKSPACE, "forward small ws");
    expect(coli_moe_forward(&d, INT32_MAX, x, ti, tw, blobs, blob, nullptr, nullptr, out, ws, wsb, nullptr) ==
               COLI_EINVAL, "forward beyond the token limit");
    expect(coli_moe_layer(&d, 4, x, W, nullptr, blobs, blob, ti, tw, out, nullptr, wsb, nullptr) == COLI_EINVAL,
           "layer NULL ws");
    expect(coli_moe_layer(&d, 4, x, W, nullptr, blobs, blob, ti, tw, nullptr, ws, wsb, nullptr) == COLI_EINVAL,
           "layer NULL out");
    expect(coli_moe_layer(&d, 4, x, W, nullptr, blobs, blob, ti, tw, out, ws, 100, nullptr) == COLI_EWORKSPACE,
           "layer small ws");
    expect(coli_moe_layer(&d, INT32_MAX, x, W, nullptr, blobs, blob, ti, tw, out, ws, SIZE_MAX, nullptr) ==
               COLI_EINVAL, "layer beyond the token limit");
    const coli_moe_dims glm = dims(6144, 2048, 256, 8, 1, 4, 0, 0);
    expect(coli_moe_layer_noalloc(&glm, 133, x, W, nullptr, blobs, blob, ti, tw, out, nullptr, nullptr) ==
               COLI_EWORKSPACE, "noalloc beyond its scratch");
    expect(coli_moe_layer_noalloc(&glm, -3, x, W, nullptr, blobs, blob, ti, tw, out, nullptr, nullptr) == COLI_EINVAL,
           "noalloc n<0");
    expect(coli_moe_layer_noalloc(&glm, 0, x, W, nullptr, blobs, blob, ti, tw, out, nullptr, nullptr) == COLI_OK,
           "noalloc of 0 tokens");
    expect(coli_moe_stage_experts(-1, nullptr, nullptr, 0, nullptr, nullptr) == COLI_EINVAL, "stage n<0");
    expect(coli_moe_stage_experts(2, nullptr, nullptr, 16, nullptr, nullptr) == COLI_EINVAL, "stage NULL arrays");
    const void *src[2] = {blob, nullptr};
    void *dst[2] = {ws, ws};
    expect(coli_moe_stage_experts(2, src, dst, 16, nullptr, nullptr) == COLI_EINVAL, "stage NULL source");
    expect(coli_moe_stage_experts(0, nullptr, nullptr, 0, nullptr, nullptr) == COLI_OK, "stage nothing");
    expect(coli_moe_status(nullptr, nullptr) == COLI_EINVAL, "status(NULL)");
    expect(coli_moe_debug_force_path(4) == COLI_EINVAL, "force_path 4");
    expect(coli_moe_debug_force_path(-1) == COLI_EINVAL, "force_path -1");
    expect(coli_moe_debug_route_wait(0, 1) == COLI_EINVAL, "route_wait unbounded unreachable");
    expect(coli_moe_debug_route_wait(16, 2) == COLI_EINVAL, "route_wait unreachable 2");
    expect(coli_moe_debug_route_wait(16, 1) == COLI_OK && coli_moe_debug_route_wait(0, 0) == COLI_OK,
           "route_wait set and restore");
    expect(coli_moe_timing_read(99, nullptr, nullptr) == COLI_EINVAL, "timing_read bad kind");
    double ms = -1.0;
    int64_t n = -1;
    expect(coli_moe_timing_enable(1) == COLI_OK && coli_moe_timing_enable(0) == COLI_OK, "timing switch");
    expect(coli_moe_timing_read(2, &ms, &n) == COLI_OK && ms == 0.0 && n == 0, "timing_read with nothing recorded");
    expect(coli_moe_debug_unpack(3, 1, 32, blob, nullptr, nullptr) == COLI_EINVAL, "debug_unpack bad bits");
    expect(coli_moe_debug_unpack(4, INT32_MAX, 1 << 30, blob, reinterpret_cast<int8_t *>(ws), nullptr) ==
               COLI_EINVAL, "debug_unpack too large");
    expect(coli_moe_debug_unpack(4, 0, 32, blob, reinterpret_cast<int8_t *>(ws), nullptr) == COLI_OK,
           "debug_unpack of 0 rows");
    expect(coli_moe_roof_stream_read(blob, 17, nullptr, nullptr) == COLI_EINVAL, "roof_stream_read bad size");
    expect(coli_moe_roof_sink_words() > 0, "roof_sink_words");
    expect(coli_moe_roof_mfma_i8(0, nullptr, nullptr) == COLI_EINVAL, "roof_mfma_i8 iters 0");

    // calls that pass every host check and stop at the device query: only
    // where no device is present
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess) ndev = 0;
    if (ndev == 0) {
        for (int path = 0; path <= 3; ++path) {
            expect(coli_moe_debug_force_path(path) == COLI_OK, "force_path");
            const int rcf = coli_moe_forward(&d, 4, x, ti, tw, blobs, blob, nullptr, nullptr, out, ws, wsb, nullptr);
            expect(rcf == COLI_EHIP || (path == 2 && rcf == COLI_EINVAL), "forward stops at the device query");
            const int rcl = coli_moe_layer(&d, 4, x, W, nullptr, blobs, blob, ti, tw, out, ws, wsb, nullptr);
            expect(rcl == COLI_EHIP, "layer stops at the device query");
            expect(coli_moe_route(&d, 4, x, W, nullptr, ti, tw, ws, wsb, nullptr) == COLI_EHIP,
                   "route stops at the device query");
        }
        expect(coli_moe_debug_force_path(0) == COLI_OK, "force_path 0");
        const coli_moe_dims mx = dims(256, 128, 16, 2, 1, 4, 0, 1);
        expect(coli_moe_layer(&mx, 4, x, W, nullptr, blobs, blob, ti, tw, out, ws, SIZE_MAX, nullptr) == COLI_EHIP,
               "MXFP4 layer stops at the device query");
    } else {
        std::printf("a HIP device is present: device-reaching calls skipped\n");
    }
    if (failures) return 1;
    std::printf("host sanitizer run ok\n");
    return 0;
}
