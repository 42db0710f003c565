// block_from_c.cpp -- one Mamba block driven through libssmblock.so's C ABI from
// a host program with no Python or PyTorch in the process (so the block's
// hipBLASLt dependency resolves to the system ROCm library).
//
// usage: block_from_c check <out-file>
//          f32, batch 2 x seqlen 100, d_model 64, d_inner 128, dt_rank 8, d_conv 4:
//          one training forward and one backward; writes int64 batch, seqlen,
//          d_model, d_inner, d_state, dt_rank, d_conv, then float32 X, dY, W_in,
//          conv_w, conv_b, W_x, W_dt, dt_bias, A_log, D, W_out (inputs), Y, dX,
//          dW_in, dconv_w, dconv_b, dW_x, dW_dt, ddt_bias, dA_log, dD, dW_out.
//        block_from_c time <steps> <warmup>
//          bf16, batch 4 x seqlen 8192, d_model 2560, d_inner 5120, dt_rank 160,
//          d_conv 4: prints "ms_per_step <t>" for forward + backward, timed with
//          HIP events on the program's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>
#include <vector>

#include "ssm_block.h"

#define HIP_OK(e)                                                              \
    do {                                                                       \
        hipError_t err_ = (e);                                                 \
        if (err_ != hipSuccess) {                                              \
            fprintf(stderr, "%s: %s\n", #e, hipGetErrorString(err_));          \
            exit(3);                                                           \
        }                                                                      \
    } while (0)
#define SSM_OK_OR_DIE(e)                                                       \
    do {                                                                       \
        ssm_status st_ = (e);                                                  \
        if (st_ != SSM_OK) {                                                   \
            fprintf(stderr, "%s: %s\n", #e, ssm_status_str(st_));              \
            exit(1);                                                           \
        }                                                                      \
    } while (0)

static uint64_t rng_state = 0x9E3779B97F4A7C15ULL;
static float uniform() {  // [-1, 1), 64-bit LCG (Knuth's MMIX constants)
    rng_state = rng_state * 6364136223846793005ULL + 1442695040888963407ULL;
    return (float)((double)(rng_state >> 11) * (1.0 / 9007199254740992.0) * 2.0 - 1.0);
}
static uint16_t to_bf16(float f) {  // round to nearest even
    uint32_t u;
    memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

struct Buf {
    void* p = nullptr;
    size_t bytes = 0;
    explicit Buf(size_t b) : bytes(b) { if (b) HIP_OK(hipMalloc(&p, b)); }
    ~Buf() { if (p) (void)hipFree(p); }
    Buf(const Buf&) = delete;
    Buf& operator=(const Buf&) = delete;
};

struct Host {  // one f32 host array, its device copy in the io dtype
    std::vector<float> h;
    Buf* d = nullptr;
    Host(size_t n, float scale, bool bf16) : h(n) {
        for (auto& v : h) v = scale * uniform();
        upload(bf16);
    }
    void upload(bool bf16) {
        delete d;
        d = new Buf(h.size() * (bf16 ? 2 : 4));
        if (bf16) {
            std::vector<uint16_t> b(h.size());
            for (size_t i = 0; i < h.size(); ++i) {
                b[i] = to_bf16(h[i]);
                uint32_t u = (uint32_t)b[i] << 16;
                memcpy(&h[i], &u, 4);  // host copy holds the rounded value
            }
            HIP_OK(hipMemcpy(d->p, b.data(), b.size() * 2, hipMemcpyHostToDevice));
        } else {
            HIP_OK(hipMemcpy(d->p, h.data(), h.size() * 4, hipMemcpyHostToDevice));
        }
    }
    ~Host() { delete d; }
};

int main(int argc, char** argv) {
    if (argc < 3 || (strcmp(argv[1], "check") && strcmp(argv[1], "time"))) {
        fprintf(stderr, "usage: %s check <out-file> | time <steps> <warmup>\n", argv[0]);
        return 2;
    }
    const bool timing = !strcmp(argv[1], "time");
    const bool bf16 = timing;
    ssm_block_dims d = timing ? ssm_block_dims{4, 8192, 2560, 5120, 16, 160, 4, SSM_BF16}
                              : ssm_block_dims{2, 100, 64, 128, 16, 8, 4, SSM_F32};
    const int64_t T = d.batch * d.seqlen, dm = d.d_model, di = d.d_inner, N = d.d_state, R = d.dt_rank,
                  K = d.d_conv, P = R + 2 * N;
    auto sc = [](int64_t fan_in) { return fminf(1.0f / sqrtf((float)fan_in), 0.5f) * 1.7320508f; };
    Host X((size_t)(T * dm), 1.0f, bf16), dY((size_t)(T * dm), 1.0f, bf16);
    Host W_in((size_t)(2 * di * dm), sc(dm), bf16), W_x((size_t)(P * di), sc(di), bf16),
        W_dt((size_t)(di * R), sc(R), bf16), W_out((size_t)(dm * di), sc(di), bf16);
    Host conv_w((size_t)(di * K), sc(K), false), conv_b((size_t)di, 0.3f, false);
    Host dt_bias((size_t)di, 0.0f, false), A_log((size_t)(di * N), 0.0f, false), Dp((size_t)di, 0.0f, false);
    for (int64_t c = 0; c < di; ++c) {
        dt_bias.h[(size_t)c] = -4.6f + 0.5f * uniform();
        Dp.h[(size_t)c] = 1.0f + 0.1f * uniform();
        for (int64_t n = 0; n < N; ++n) A_log.h[(size_t)(c * N + n)] = logf((float)(n + 1));
    }
    dt_bias.upload(false); Dp.upload(false); A_log.upload(false);

    ssm_block_params p = {W_in.d->p, (const float*)conv_w.d->p, (const float*)conv_b.d->p, W_x.d->p, W_dt.d->p,
                          (const float*)dt_bias.d->p, (const float*)A_log.d->p, (const float*)Dp.d->p,
                          W_out.d->p};
    const size_t esz = bf16 ? 2 : 4;
    Buf Y((size_t)(T * dm) * esz), dX((size_t)(T * dm) * esz);
    Buf gW_in((size_t)(2 * di * dm) * 4), gconv_w((size_t)(di * K) * 4), gconv_b((size_t)di * 4),
        gW_x((size_t)(P * di) * 4), gW_dt((size_t)(di * R) * 4), gdt_bias((size_t)di * 4),
        gA_log((size_t)(di * N) * 4), gD((size_t)di * 4), gW_out((size_t)(dm * di) * 4);
    ssm_block_grads g = {(float*)gW_in.p, (float*)gconv_w.p, (float*)gconv_b.p, (float*)gW_x.p, (float*)gW_dt.p,
                         (float*)gdt_bias.p, (float*)gA_log.p, (float*)gD.p, (float*)gW_out.p};
    Buf saved(ssm_block_saved_bytes(&d)), wsf(ssm_block_fwd_training_workspace_bytes(&d)),
        wsb(ssm_block_bwd_workspace_bytes(&d));
    if (!saved.bytes || !wsf.bytes || !wsb.bytes) {
        fprintf(stderr, "size queries rejected the dims\n");
        return 1;
    }
    ssm_block_ctx* ctx = nullptr;
    SSM_OK_OR_DIE(ssm_block_create(&ctx));
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    auto step = [&]() {
        SSM_OK_OR_DIE(ssm_block_fwd(ctx, &d, X.d->p, &p, Y.p, saved.p, wsf.p, wsf.bytes, s, nullptr));
        SSM_OK_OR_DIE(ssm_block_bwd(ctx, &d, X.d->p, &p, saved.p, dY.d->p, dX.p, &g, wsb.p, wsb.bytes, s,
                                    nullptr));
    };
    if (timing) {
        const int steps = atoi(argv[2]), warm = argc > 3 ? atoi(argv[3]) : 2;
        for (int i = 0; i < warm; ++i) step();
        HIP_OK(hipStreamSynchronize(s));
        hipEvent_t e0, e1;
        HIP_OK(hipEventCreate(&e0));
        HIP_OK(hipEventCreate(&e1));
        HIP_OK(hipEventRecord(e0, s));
        for (int i = 0; i < steps; ++i) step();
        HIP_OK(hipEventRecord(e1, s));
        HIP_OK(hipEventSynchronize(e1));
        float ms = 0.0f;
        HIP_OK(hipEventElapsedTime(&ms, e0, e1));
        printf("ms_per_step %.4f\n", ms / steps);
    } else {
        step();
        HIP_OK(hipStreamSynchronize(s));
        FILE* f = fopen(argv[2], "wb");
        if (!f) {
            perror(argv[2]);
            return 2;
        }
        const int64_t hdr[7] = {d.batch, d.seqlen, dm, di, N, R, K};
        fwrite(hdr, sizeof(hdr), 1, f);
        for (const Host* h : {&X, &dY, &W_in, &conv_w, &conv_b, &W_x, &W_dt, &dt_bias, &A_log, &Dp, &W_out})
            fwrite(h->h.data(), 4, h->h.size(), f);
        auto put = [&](const Buf& b) {
            std::vector<float> h(b.bytes / 4);
            HIP_OK(hipMemcpy(h.data(), b.p, b.bytes, hipMemcpyDeviceToHost));
            fwrite(h.data(), 4, h.size(), f);
        };
        put(Y); put(dX); put(gW_in); put(gconv_w); put(gconv_b); put(gW_x); put(gW_dt); put(gdt_bias);
        put(gA_log); put(gD); put(gW_out);
        fclose(f);
        printf("block_from_c: check written\n");
    }
    HIP_OK(hipStreamDestroy(s));
    ssm_block_destroy(ctx);
    return 0;
}
