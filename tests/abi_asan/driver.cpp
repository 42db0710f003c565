// Host-side argument checks of libssmscan.so under AddressSanitizer and
// UndefinedBehaviorSanitizer: every entry point is called with each kind of bad
// argument (null dims or pointers, bad shapes, unknown dtype, unsupported sizes,
// misaligned bases, too-small workspace) and must return its documented status
// before any HIP call; the size queries, status strings and kernel names are
// exercised over their whole ranges.  Pointers are fake, 16-byte aligned device
// addresses that no error path dereferences.  Built host-only (no GPU code is
// compiled, no kernel can run) by tests/test_abi_asan.py.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "ssm_conv1d.h"
#include "ssm_gdn2.h"
#include "ssm_scan.h"

static int fails = 0;
static void expect(ssm_status got, ssm_status want, const char* what) {
    if (got != want) {
        fprintf(stderr, "FAIL %s: got %d, want %d\n", what, (int)got, (int)want);
        ++fails;
    }
}
#define EXPECT(call, want) expect((call), (want), #call)

int main() {
    void* F = (void*)(uintptr_t)(1u << 20);     // aligned fake device address
    void* M = (void*)(uintptr_t)((1u << 20) + 4);  // misaligned
    const float* Ff = (const float*)F;
    float* Fw = (float*)F;

    // status strings and kernel names over their whole ranges
    for (int32_t s = -2; s < 12; ++s)
        if (!ssm_status_str(s) || !ssm_status_str(s)[0]) ++fails;
    if (strcmp(ssm_status_str(SSM_E_ALIGN), ssm_status_str(4)) != 0) ++fails;
    for (int k = -2; k < 64; ++k)
        if (!ssm_kernel_name(k)) ++fails;

    // ---- scan: size queries
    ssm_dims ok{2, 64, 32, 16, SSM_F32}, big{2, 4096, 1536, 16, SSM_F32};  // big: a chunked forward
    ssm_dims bad[] = {{0, 64, 32, 16, SSM_F32}, {2, -1, 32, 16, SSM_F32}, {2, 64, 0, 16, SSM_F32},
                      {2, 64, 32, 8, SSM_F32},  {2, 64, 32, 16, 7},         {70000, 64, 32, 16, SSM_F32}};
    if (ssm_scan_ckpt_bytes(&ok) == 0 || ssm_scan_bwd_workspace_bytes(&ok) == 0) ++fails;
    if (ssm_scan_fwd_workspace_bytes(&big) == 0) ++fails;
    for (auto& b : bad) {
        if (ssm_scan_ckpt_bytes(&b) || ssm_scan_fwd_workspace_bytes(&b) || ssm_scan_bwd_workspace_bytes(&b)) ++fails;
    }
    if (ssm_scan_ckpt_bytes(nullptr) || ssm_scan_fwd_workspace_bytes(nullptr)) ++fails;

    // ---- scan forward
    auto fwd = [&](const ssm_dims* d, const void* x, const void* dt, const void* z, const float* A, void* y,
                   float* ckpt, void* ws, size_t wsb) {
        return ssm_scan_fwd(d, x, dt, F, F, z, A, nullptr, nullptr, nullptr, y, nullptr, ckpt, ws, wsb, nullptr,
                            nullptr);
    };
    EXPECT(fwd(nullptr, F, F, nullptr, Ff, F, nullptr, nullptr, 0), SSM_E_NULLPTR);
    EXPECT(fwd(&bad[0], F, F, nullptr, Ff, F, nullptr, nullptr, 0), SSM_E_SHAPE);
    EXPECT(fwd(&bad[3], F, F, nullptr, Ff, F, nullptr, nullptr, 0), SSM_E_UNSUPPORTED);
    EXPECT(fwd(&bad[4], F, F, nullptr, Ff, F, nullptr, nullptr, 0), SSM_E_DTYPE);
    EXPECT(fwd(&bad[5], F, F, nullptr, Ff, F, nullptr, nullptr, 0), SSM_E_UNSUPPORTED);
    EXPECT(fwd(&ok, nullptr, F, nullptr, Ff, F, nullptr, nullptr, 0), SSM_E_NULLPTR);
    EXPECT(fwd(&ok, F, F, nullptr, nullptr, F, nullptr, nullptr, 0), SSM_E_NULLPTR);
    EXPECT(fwd(&ok, F, F, nullptr, Ff, nullptr, nullptr, nullptr, 0), SSM_E_NULLPTR);
    EXPECT(fwd(&ok, F, M, nullptr, Ff, F, nullptr, nullptr, 0), SSM_E_ALIGN);
    EXPECT(fwd(&ok, F, F, M, Ff, F, nullptr, nullptr, 0), SSM_E_ALIGN);
    const size_t need = ssm_scan_fwd_workspace_bytes(&big);
    EXPECT(fwd(&big, F, F, nullptr, Ff, F, nullptr, nullptr, 0), SSM_E_WORKSPACE);
    EXPECT(fwd(&big, F, F, nullptr, Ff, F, nullptr, F, need - 1), SSM_E_WORKSPACE);

    // ---- scan backward
    auto bwd = [&](const ssm_dims* d, const float* ckpt, const void* dy, void* dx, const void* z, void* dz,
                   void* ws, size_t wsb) {
        return ssm_scan_bwd(d, F, F, F, F, z, Ff, nullptr, nullptr, nullptr, ckpt, dy, dx, F, F, F, dz, Fw, nullptr,
                            Fw, nullptr, ws, wsb, nullptr, nullptr);
    };
    const size_t nb = ssm_scan_bwd_workspace_bytes(&ok);
    EXPECT(bwd(nullptr, Ff, F, F, nullptr, nullptr, F, nb), SSM_E_NULLPTR);
    EXPECT(bwd(&bad[1], Ff, F, F, nullptr, nullptr, F, nb), SSM_E_SHAPE);
    EXPECT(bwd(&ok, nullptr, F, F, nullptr, nullptr, F, nb), SSM_E_NULLPTR);
    EXPECT(bwd(&ok, Ff, nullptr, F, nullptr, nullptr, F, nb), SSM_E_NULLPTR);
    EXPECT(bwd(&ok, Ff, F, M, nullptr, nullptr, F, nb), SSM_E_ALIGN);
    EXPECT(bwd(&ok, Ff, F, F, F, nullptr, F, nb), SSM_E_NULLPTR);  // gated without dz
    EXPECT(bwd(&ok, Ff, F, F, nullptr, nullptr, F, nb - 1), SSM_E_WORKSPACE);
    EXPECT(bwd(&ok, Ff, F, F, nullptr, nullptr, nullptr, 0), SSM_E_WORKSPACE);

    // ---- scan step
    EXPECT(ssm_scan_step(0, 32, 16, SSM_F32, Fw, F, F, F, F, nullptr, Ff, nullptr, nullptr, F, nullptr, nullptr),
           SSM_E_SHAPE);
    EXPECT(ssm_scan_step(2, 32, 8, SSM_F32, Fw, F, F, F, F, nullptr, Ff, nullptr, nullptr, F, nullptr, nullptr),
           SSM_E_UNSUPPORTED);
    EXPECT(ssm_scan_step(2, 32, 16, 9, Fw, F, F, F, F, nullptr, Ff, nullptr, nullptr, F, nullptr, nullptr),
           SSM_E_DTYPE);
    EXPECT(ssm_scan_step(2, 32, 16, SSM_F32, nullptr, F, F, F, F, nullptr, Ff, nullptr, nullptr, F, nullptr,
                         nullptr),
           SSM_E_NULLPTR);
    EXPECT(ssm_scan_step(2, 32, 16, SSM_F32, Fw, M, F, F, F, nullptr, Ff, nullptr, nullptr, F, nullptr, nullptr),
           SSM_E_ALIGN);

    // ---- conv1d
    ssm_conv_dims cok{2, 64, 32, 4, SSM_BF16};
    ssm_conv_dims cbad[] = {{0, 64, 32, 4, SSM_BF16}, {2, 64, 32, 5, SSM_BF16}, {2, 64, 32, 4, 3},
                            {2, -1, 32, 4, SSM_BF16}};
    if (ssm_conv1d_bwd_workspace_bytes(&cok) == 0) ++fails;
    for (auto& b : cbad)
        if (ssm_conv1d_bwd_workspace_bytes(&b)) ++fails;
    EXPECT(ssm_conv1d_fwd(nullptr, F, Ff, nullptr, nullptr, F, nullptr, nullptr, nullptr), SSM_E_NULLPTR);
    EXPECT(ssm_conv1d_fwd(&cbad[0], F, Ff, nullptr, nullptr, F, nullptr, nullptr, nullptr), SSM_E_SHAPE);
    EXPECT(ssm_conv1d_fwd(&cbad[1], F, Ff, nullptr, nullptr, F, nullptr, nullptr, nullptr), SSM_E_UNSUPPORTED);
    EXPECT(ssm_conv1d_fwd(&cbad[2], F, Ff, nullptr, nullptr, F, nullptr, nullptr, nullptr), SSM_E_DTYPE);
    EXPECT(ssm_conv1d_fwd(&cok, F, nullptr, nullptr, nullptr, F, nullptr, nullptr, nullptr), SSM_E_NULLPTR);
    EXPECT(ssm_conv1d_fwd(&cok, M, Ff, nullptr, nullptr, F, nullptr, nullptr, nullptr), SSM_E_ALIGN);
    EXPECT(ssm_conv1d_fwd(&cok, F, Ff, nullptr, Ff, F, Fw, nullptr, nullptr), SSM_E_UNSUPPORTED);  // ring aliasing
    const size_t cw = ssm_conv1d_bwd_workspace_bytes(&cok);
    EXPECT(ssm_conv1d_bwd(&cok, F, Ff, nullptr, nullptr, F, F, Fw, Fw, nullptr, F, cw - 1, nullptr, nullptr),
           SSM_E_WORKSPACE);
    EXPECT(ssm_conv1d_bwd(&cok, F, Ff, nullptr, nullptr, F, F, nullptr, Fw, nullptr, F, cw, nullptr, nullptr),
           SSM_E_NULLPTR);
    EXPECT(ssm_conv1d_bwd(&cok, F, Ff, nullptr, nullptr, M, F, Fw, Fw, nullptr, F, cw, nullptr, nullptr),
           SSM_E_ALIGN);
    ssm_conv_dims chuge{8, 8192, 5120, 4, SSM_BF16};  // partials beyond the static scratch
    EXPECT(ssm_conv1d_bwd_noalloc(&chuge, F, Ff, nullptr, nullptr, F, F, Fw, Fw, nullptr, nullptr, nullptr),
           SSM_E_WORKSPACE);
    EXPECT(ssm_conv1d_step(2, 32, 4, SSM_F32, nullptr, F, Ff, nullptr, F, nullptr, nullptr), SSM_E_NULLPTR);
    EXPECT(ssm_conv1d_step(2, 32, 9, SSM_F32, Fw, F, Ff, nullptr, F, nullptr, nullptr), SSM_E_UNSUPPORTED);

    // ---- GDN2, token recurrence and chunked form
    ssm_gdn2_dims gok{2, 3, 100, 64, 32, SSM_F32};
    ssm_gdn2_dims gbad[] = {{0, 3, 100, 64, 32, SSM_F32}, {2, 3, 100, 48, 32, SSM_F32}, {2, 3, 100, 64, 32, 6},
                            {2, 3, 100, 64, 40, SSM_F32}};
    EXPECT(ssm_gdn2_fwd(nullptr, F, F, F, F, F, F, nullptr, 1.0f, F, nullptr, nullptr, nullptr), SSM_E_NULLPTR);
    EXPECT(ssm_gdn2_fwd(&gbad[0], F, F, F, F, F, F, nullptr, 1.0f, F, nullptr, nullptr, nullptr), SSM_E_SHAPE);
    EXPECT(ssm_gdn2_fwd(&gbad[1], F, F, F, F, F, F, nullptr, 1.0f, F, nullptr, nullptr, nullptr),
           SSM_E_UNSUPPORTED);
    EXPECT(ssm_gdn2_fwd(&gbad[2], F, F, F, F, F, F, nullptr, 1.0f, F, nullptr, nullptr, nullptr), SSM_E_DTYPE);
    EXPECT(ssm_gdn2_fwd(&gok, F, nullptr, F, F, F, F, nullptr, 1.0f, F, nullptr, nullptr, nullptr), SSM_E_NULLPTR);
    EXPECT(ssm_gdn2_fwd(&gok, F, F, M, F, F, F, nullptr, 1.0f, F, nullptr, nullptr, nullptr), SSM_E_ALIGN);
    const size_t gw = ssm_gdn2_chunked_workspace_bytes(&gok);
    if (gw == 0 || ssm_gdn2_chunked_workspace_bytes(&gbad[3]) != 0) ++fails;
    EXPECT(ssm_gdn2_fwd_chunked(&gbad[3], F, F, F, F, F, F, nullptr, 1.0f, F, nullptr, F, gw, nullptr, nullptr),
           SSM_E_UNSUPPORTED);
    EXPECT(ssm_gdn2_fwd_chunked(&gok, F, F, F, F, F, F, nullptr, 1.0f, F, nullptr, F, gw - 1, nullptr, nullptr),
           SSM_E_WORKSPACE);
    EXPECT(ssm_gdn2_fwd_chunked(&gok, F, F, F, F, F, F, nullptr, 1.0f, F, nullptr, nullptr, gw, nullptr, nullptr),
           SSM_E_WORKSPACE);
    EXPECT(ssm_gdn2_fwd_chunked(&gok, F, F, F, F, F, F, Ff, 1.0f, F, Fw, F, gw, nullptr, nullptr),
           SSM_E_UNSUPPORTED);  // S_last aliasing S0
    EXPECT(ssm_gdn2_fwd_chunked(&gok, F, F, F, F, M, F, nullptr, 1.0f, F, nullptr, F, gw, nullptr, nullptr),
           SSM_E_ALIGN);

    if (fails) {
        fprintf(stderr, "%d check(s) failed\n", fails);
        return 1;
    }
    printf("abi sanitizer run: ok\n");
    return 0;
}
