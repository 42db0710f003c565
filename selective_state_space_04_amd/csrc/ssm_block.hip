// ssm_block.hip -- one Mamba block around the selective scan, on one MI355X:
// the four projections on hipBLASLt (bf16 or f32 operands, f32 accumulation), the
// conv1d + SiLU and the scan on this project's kernels, everything on the
// caller's stream.  Built as libssmblock.so on top of libssmscan.so.
//
// Operation (rustytorch commit log, page "crates/training/rtx-transformers/tests":
// the real-S6-forward commit and the hand-written VJP commit):
//   xi = X W_in[:di]^T, z = X W_in[di:]^T, xc = silu(conv1d(xi)),
//   (dt_low, B, C) = xc W_x^T, dt = dt_low W_dt^T,
//   y_s = scan(xc, dt, B, C, z; A_log, D, dt_bias), Y = y_s W_out^T,
// and the chain rule back through the same steps.
//
// Activations are token-major [T, features] (T = batch*seqlen), the layout the
// conv and scan kernels read, so every projection is one row-major GEMM with
// no transposes of data; x_proj's output columns are split into dense dt_low,
// B and C arrays (and joined back for the backward) by a small copy kernel.
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>
#include <stdint.h>

#include <algorithm>
#include <deque>
#include <initializer_list>

#include "ssm_block.h"
#include "ssm_common.h"
#include "ssm_conv1d.h"
#include "ssm_scan.h"

// One GEMM configuration: its descriptors and the algorithm hipBLASLt's
// heuristic picked for it, kept for the life of the context.
struct LtPlan {
    int64_t key[11];
    hipblasLtMatmulDesc_t op;
    hipblasLtMatrixLayout_t a, b, c;
    hipblasLtMatmulAlgo_t algo;
    size_t ws;  // workspace bytes the algorithm uses
};

struct ssm_block_ctx {
    hipblasLtHandle_t lt;
    std::deque<LtPlan> plans;  // a deque: adding a plan keeps earlier plans where they are
};

namespace {

using ssm::bf16_t;
using ssm::misaligned;

constexpr int WG = 256;
constexpr int NS = 16;
constexpr size_t GEMM_WS = (size_t)64 << 20;  // workspace offered to each GEMM

struct Plan {
    int64_t Bt, L, T, dm, di, N, R, K, P;
    int io;
    size_t esz;
};

ssm_status check_block(const ssm_block_dims* d) {
    if (!d) return SSM_E_NULLPTR;
    if (d->batch < 1 || d->seqlen < 1 || d->d_model < 1 || d->d_inner < 1 || d->d_state < 1 ||
        d->dt_rank < 1 || d->d_conv < 1)
        return SSM_E_SHAPE;
    if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_E_DTYPE;
    if (d->d_model % 8 || d->d_inner % 8) return SSM_E_SHAPE;  // 16-byte rows for every operand
    if (d->d_state != NS || d->d_conv > 4 || d->batch > 65535) return SSM_E_UNSUPPORTED;
    if (d->batch * d->seqlen >= ((int64_t)1 << 31) || d->d_inner >= ((int64_t)1 << 28) ||
        d->d_model >= ((int64_t)1 << 28) || d->dt_rank >= ((int64_t)1 << 20))
        return SSM_E_UNSUPPORTED;
    return SSM_OK;
}

Plan make_plan(const ssm_block_dims* d) {
    Plan p;
    p.Bt = d->batch;
    p.L = d->seqlen;
    p.T = p.Bt * p.L;
    p.dm = d->d_model;
    p.di = d->d_inner;
    p.N = d->d_state;
    p.R = d->dt_rank;
    p.K = d->d_conv;
    p.P = p.R + 2 * p.N;
    p.io = d->io_dtype;
    p.esz = p.io == SSM_BF16 ? 2 : 4;
    return p;
}

ssm_dims scan_dims(const Plan& p) { return ssm_dims{p.Bt, p.L, p.di, p.N, p.io}; }
ssm_conv_dims conv_dims(const Plan& p) { return ssm_conv_dims{p.Bt, p.L, p.di, p.K, p.io}; }

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

// Sequential 256-byte aligned carve-up of a buffer.
struct Carve {
    size_t off = 0;
    size_t take(size_t bytes) {
        const size_t at = off;
        off = align_up(off + bytes);
        return at;
    }
};

// Activations the backward needs (the forward's intermediates and the scan's
// checkpoints).
struct Saved {
    size_t xi, z, xc, proj, dtl, Bm, Cm, dt, ys, ckpt, total;
};
Saved saved_layout(const Plan& p) {
    Carve c;
    Saved s;
    const size_t act = (size_t)p.T * p.di * p.esz;
    s.xi = c.take(act);
    s.z = c.take(act);
    s.xc = c.take(act);
    s.proj = c.take((size_t)p.T * p.P * p.esz);
    s.dtl = c.take((size_t)p.T * p.R * p.esz);
    s.Bm = c.take((size_t)p.T * p.N * p.esz);
    s.Cm = c.take((size_t)p.T * p.N * p.esz);
    s.dt = c.take(act);
    s.ys = c.take(act);
    const ssm_dims sd = scan_dims(p);
    s.ckpt = c.take(ssm_scan_ckpt_bytes(&sd));
    s.total = c.off;
    return s;
}

// Forward workspace: the GEMMs' workspace, the scan's own workspace, then room
// for the intermediates, which is used only when no `saved` buffer is given
// (inference).
struct FwdWs {
    size_t gemm, scan, act, training, total;
};
FwdWs fwd_ws(const Plan& p) {
    Carve c;
    FwdWs w;
    w.gemm = c.take(GEMM_WS);
    const ssm_dims sd = scan_dims(p);
    w.scan = c.take(ssm_scan_fwd_workspace_bytes(&sd));
    w.training = c.off;
    const Saved s = saved_layout(p);
    w.act = c.take(s.ckpt);  // everything before the checkpoints
    w.total = c.off;
    return w;
}

// Weight gradients sum over all T tokens (the GEMM's K).  Their outputs are
// small next to K, so one GEMM has few output tiles for 256 CUs; the tokens are
// split into S equal chunks computed as one strided-batched GEMM into f32
// partials, which a fixed-order kernel then sums (deterministic).
int64_t wgrad_splits(int64_t m, int64_t n, int64_t T) {
    const int64_t tiles = ((m + 255) / 256) * ((n + 255) / 256);
    int64_t S = 1;
    while (S < 16 && tiles * S < 512 && T % (2 * S) == 0 && T / (2 * S) >= 2048) S *= 2;
    return S;
}

struct BwdWs {
    size_t gemm, dys, dxc, ddt, ddtl, dB, dC, dz, dproj, dxi, conv, scan, part, total;
};
BwdWs bwd_ws(const Plan& p) {
    Carve c;
    BwdWs w;
    w.gemm = c.take(GEMM_WS);
    const size_t act = (size_t)p.T * p.di * p.esz;
    w.dys = c.take(act);
    w.dxc = c.take(act);
    w.ddt = c.take(act);
    w.ddtl = c.take((size_t)p.T * p.R * p.esz);
    w.dB = c.take((size_t)p.T * p.N * p.esz);
    w.dC = c.take((size_t)p.T * p.N * p.esz);
    w.dz = c.take(act);
    w.dproj = c.take((size_t)p.T * p.P * p.esz);
    w.dxi = c.take(act);
    const ssm_conv_dims cd = conv_dims(p);
    w.conv = c.take(ssm_conv1d_bwd_workspace_bytes(&cd));
    const ssm_dims sd = scan_dims(p);
    w.scan = c.take(ssm_scan_bwd_workspace_bytes(&sd));
    // partials of the largest split weight gradient (in_proj halves, out_proj, x_proj, dt_proj)
    size_t part = 0;
    const int64_t shapes[4][2] = {{p.di, p.dm}, {p.dm, p.di}, {p.P, p.di}, {p.di, p.R}};
    for (const auto& mn : shapes) {
        const int64_t S = wgrad_splits(mn[0], mn[1], p.T);
        if (S > 1) part = std::max(part, sizeof(float) * (size_t)(S * mn[0] * mn[1]));
    }
    w.part = c.take(part);
    w.total = c.off;
    return w;
}

// ------------------------------------------------------------------ GEMMs
// Row-major C[m, n] (ldc) = opA(A) opB(B) + beta C, where opA(A) = A [m, k] (lda)
// or, with ta, A^T for A stored [k, m]; opB(B) = B [k, n] (ldb) or, with tb, B^T
// for B stored [n, k].  hipBLASLt is column-major, so this is the column-major
// product C^T = opB(B)^T opA(A)^T with the operands swapped.  `batch` > 1 runs
// that many such products at element strides sA, sB, sC.  Each call may use up
// to GEMM_WS bytes of the caller's workspace.
bool set_batch(hipblasLtMatrixLayout_t l, int32_t batch, int64_t stride) {
    if (batch <= 1) return true;
    return hipblasLtMatrixLayoutSetAttribute(l, HIPBLASLT_MATRIX_LAYOUT_BATCH_COUNT, &batch, sizeof(batch)) ==
               HIPBLAS_STATUS_SUCCESS &&
           hipblasLtMatrixLayoutSetAttribute(l, HIPBLASLT_MATRIX_LAYOUT_STRIDED_BATCH_OFFSET, &stride,
                                             sizeof(stride)) == HIPBLAS_STATUS_SUCCESS;
}

void destroy_plan(LtPlan& e) {
    if (e.a) hipblasLtMatrixLayoutDestroy(e.a);
    if (e.b) hipblasLtMatrixLayoutDestroy(e.b);
    if (e.c) hipblasLtMatrixLayoutDestroy(e.c);
    if (e.op) hipblasLtMatmulDescDestroy(e.op);
}

// The plan for one configuration, created (descriptors + heuristic query) on
// first use.  Returns nullptr if hipBLASLt offers no algorithm for it.
const LtPlan* get_plan(ssm_block_ctx* ctx, bool ta, bool tb, int64_t m, int64_t n, int64_t k, int64_t lda,
                       int64_t ldb, int64_t ldc, hipDataType ab, hipDataType ct, int32_t batch, int64_t sA,
                       int64_t sB, int64_t sC) {
    const int64_t key[11] = {(int64_t)ta | ((int64_t)tb << 1) | ((int64_t)ab << 8) | ((int64_t)ct << 24),
                             m, n, k, lda, ldb, ldc, batch, sA, sB, sC};
    for (const LtPlan& e : ctx->plans)
        if (std::equal(key, key + 11, e.key)) return &e;
    LtPlan e{};
    std::copy(key, key + 11, e.key);
    bool ok = hipblasLtMatmulDescCreate(&e.op, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS;
    const int32_t opa = tb ? HIPBLAS_OP_T : HIPBLAS_OP_N, opb = ta ? HIPBLAS_OP_T : HIPBLAS_OP_N;
    ok = ok &&
         hipblasLtMatmulDescSetAttribute(e.op, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)) ==
             HIPBLAS_STATUS_SUCCESS &&
         hipblasLtMatmulDescSetAttribute(e.op, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)) ==
             HIPBLAS_STATUS_SUCCESS;
    // column-major: a = B viewed [n, k] (stored [k, n] or, with tb, [n, k] = a^T),
    // b = A viewed [k, m], c = C viewed [n, m]
    ok = ok && hipblasLtMatrixLayoutCreate(&e.a, ab, tb ? k : n, tb ? n : k, ldb) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&e.b, ab, ta ? m : k, ta ? k : m, lda) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && hipblasLtMatrixLayoutCreate(&e.c, ct, n, m, ldc) == HIPBLAS_STATUS_SUCCESS;
    ok = ok && set_batch(e.a, batch, sB) && set_batch(e.b, batch, sA) && set_batch(e.c, batch, sC);
    // the heuristic's first choice within the workspace offered
    hipblasLtMatmulPreference_t pref = nullptr;
    ok = ok && hipblasLtMatmulPreferenceCreate(&pref) == HIPBLAS_STATUS_SUCCESS;
    const uint64_t max_ws = GEMM_WS;
    ok = ok && hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &max_ws,
                                                     sizeof(max_ws)) == HIPBLAS_STATUS_SUCCESS;
    constexpr int NREQ = 8;
    hipblasLtMatmulHeuristicResult_t res[NREQ];
    int got = 0;
    ok = ok && hipblasLtMatmulAlgoGetHeuristic(ctx->lt, e.op, e.a, e.b, e.c, e.c, pref, NREQ, res, &got) ==
                   HIPBLAS_STATUS_SUCCESS;
    if (pref) hipblasLtMatmulPreferenceDestroy(pref);
    int pick = -1;
    for (int r = 0; ok && r < got && pick < 0; ++r)
        if (res[r].state == HIPBLAS_STATUS_SUCCESS && res[r].workspaceSize <= GEMM_WS) pick = r;
    if (pick < 0) {
        destroy_plan(e);
        return nullptr;
    }
    e.algo = res[pick].algo;
    e.ws = res[pick].workspaceSize;
    ctx->plans.push_back(e);
    return &ctx->plans.back();
}

// The projections' GEMMs: the caller's stream, GEMM_WS bytes of workspace and
// the caller's optional launch log (each GEMM is logged as SSM_K_BLOCK_GEMM).
struct Gemm {
    ssm_block_ctx* ctx;
    hipDataType ab, io_c;
    hipStream_t s;
    void* ws;  // GEMM_WS bytes
    ssm_timing* tm;
    ssm_status operator()(bool ta, bool tb, int64_t m, int64_t n, int64_t k, const void* A, int64_t lda,
                          const void* B, int64_t ldb, float beta, void* C, int64_t ldc,
                          bool f32_out = false, int32_t batch = 1, int64_t sA = 0, int64_t sB = 0,
                          int64_t sC = 0) const {
        const float alpha = 1.0f;
        const LtPlan* e = get_plan(ctx, ta, tb, m, n, k, lda, ldb, ldc, ab, f32_out ? HIP_R_32F : io_c, batch,
                                   sA, sB, sC);
        if (!e) return SSM_E_UNSUPPORTED;
        const bool rec = tm && tm->events && tm->count < tm->capacity && tm->count < SSM_TIMING_MAX;
        if (rec) (void)hipEventRecord(tm->events[2 * tm->count], s);
        const hipblasStatus_t st = hipblasLtMatmul(ctx->lt, e->op, &alpha, B, e->a, A, e->b, &beta, C, e->c, C,
                                                   e->c, &e->algo, e->ws ? ws : nullptr, e->ws, s);
        if (rec) {
            (void)hipEventRecord(tm->events[2 * tm->count + 1], s);
            tm->kernel_id[tm->count] = SSM_K_BLOCK_GEMM;
            tm->count++;
        }
        return st == HIPBLAS_STATUS_SUCCESS ? SSM_OK : SSM_E_LAUNCH;
    }
};

// C[i] = sum_s part[s][i], s in increasing order.
__global__ __launch_bounds__(WG) void k_sum_parts(const float* __restrict__ part, float* __restrict__ C,
                                                  int64_t mn, int S) {
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (i >= mn) return;
    float acc = part[i];
    for (int s = 1; s < S; ++s) acc += part[(int64_t)s * mn + i];
    C[i] = acc;
}

// Row-major f32 weight gradient C[m, n] = A^T B over T tokens, A [T, m] (lda),
// B [T, n] (ldb), with the tokens split as described at wgrad_splits.
ssm_status wgrad(const Gemm& g, int64_t m, int64_t n, int64_t T, const void* A, int64_t lda, const void* B,
                 int64_t ldb, float* C, float* part) {
    ssm_timing* tm = g.tm;
    const int64_t S = wgrad_splits(m, n, T);
    if (S == 1) return g(true, false, m, n, T, A, lda, B, ldb, 0.0f, C, n, true);
    const int64_t Tc = T / S;
    SSM_TRY(g(true, false, m, n, Tc, A, lda, B, ldb, 0.0f, part, n, true, (int32_t)S, Tc * lda, Tc * ldb, m * n));
    ssm::Launcher launch{g.s, tm};
    const int64_t mn = m * n;
    return launch(SSM_K_BLOCK_SUM, k_sum_parts, dim3((unsigned)((mn + WG - 1) / WG)), dim3(WG),
                  (const float*)part, C, mn, (int)S);
}

// ------------------------------------------------------------------ x_proj columns
// proj [T, R + 2N] -> dt_low [T, R], B [T, N], C [T, N] (forward), and the
// gradients back into dproj (backward).  Dense copies: the dt_proj GEMMs and the
// scan then read unit-stride rows.
template <typename T>
__global__ __launch_bounds__(WG) void k_split_proj(const T* __restrict__ proj, T* __restrict__ dtl,
                                                   T* __restrict__ Bm, T* __restrict__ Cm, int64_t n, int R,
                                                   int N) {
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (i >= n) return;
    const int P = R + 2 * N;
    const int64_t t = i / P;
    const int j = (int)(i % P);
    const T v = proj[i];
    if (j < R) dtl[t * R + j] = v;
    else if (j < R + N) Bm[t * N + (j - R)] = v;
    else Cm[t * N + (j - R - N)] = v;
}

template <typename T>
__global__ __launch_bounds__(WG) void k_join_proj(const T* __restrict__ ddtl, const T* __restrict__ dB,
                                                  const T* __restrict__ dC, T* __restrict__ dproj, int64_t n,
                                                  int R, int N) {
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (i >= n) return;
    const int P = R + 2 * N;
    const int64_t t = i / P;
    const int j = (int)(i % P);
    dproj[i] = j < R ? ddtl[t * R + j] : (j < R + N ? dB[t * N + (j - R)] : dC[t * N + (j - R - N)]);
}

template <typename T>
ssm_status launch_proj_t(const Plan& p, bool split, const void* a, const void* b, const void* c, void* d,
                         hipStream_t s, ssm_timing* tm) {
    ssm::Launcher launch{s, tm};
    const int64_t n = p.T * p.P;
    const dim3 grid((unsigned)((n + WG - 1) / WG));
    if (split)  // a = proj -> b = dt_low, c = B, d = C
        return launch(SSM_K_BLOCK_BC, k_split_proj<T>, grid, dim3(WG), (const T*)a, (T*)b, (T*)c, (T*)d, n,
                      (int)p.R, (int)p.N);
    // a = d dt_low, b = dB, c = dC -> d = dproj
    return launch(SSM_K_BLOCK_BC, k_join_proj<T>, grid, dim3(WG), (const T*)a, (const T*)b, (const T*)c, (T*)d,
                  n, (int)p.R, (int)p.N);
}

ssm_status launch_proj(const Plan& p, bool split, const void* a, const void* b, const void* c, void* d,
                       hipStream_t s, ssm_timing* tm) {
    return p.io == SSM_F32 ? launch_proj_t<float>(p, split, a, b, c, d, s, tm)
                           : launch_proj_t<bf16_t>(p, split, a, b, c, d, s, tm);
}

bool any_misaligned(std::initializer_list<const void*> ptrs) {
    for (const void* q : ptrs)
        if (q && misaligned(q)) return true;
    return false;
}

}  // namespace

extern "C" {

ssm_status ssm_block_create(ssm_block_ctx** ctx) {
    if (!ctx) return SSM_E_NULLPTR;
    *ctx = nullptr;
    hipblasLtHandle_t lt;
    if (hipblasLtCreate(&lt) != HIPBLAS_STATUS_SUCCESS) return SSM_E_LAUNCH;
    *ctx = new ssm_block_ctx{lt, {}};
    return SSM_OK;
}

void ssm_block_destroy(ssm_block_ctx* ctx) {
    if (!ctx) return;
    for (LtPlan& e : ctx->plans) destroy_plan(e);
    hipblasLtDestroy(ctx->lt);
    delete ctx;
}

size_t ssm_block_saved_bytes(const ssm_block_dims* dims) {
    if (check_block(dims) != SSM_OK) return 0;
    return saved_layout(make_plan(dims)).total;
}

size_t ssm_block_fwd_workspace_bytes(const ssm_block_dims* dims) {
    if (check_block(dims) != SSM_OK) return 0;
    return fwd_ws(make_plan(dims)).total;
}

size_t ssm_block_fwd_training_workspace_bytes(const ssm_block_dims* dims) {
    if (check_block(dims) != SSM_OK) return 0;
    return fwd_ws(make_plan(dims)).training;
}

size_t ssm_block_bwd_workspace_bytes(const ssm_block_dims* dims) {
    if (check_block(dims) != SSM_OK) return 0;
    return bwd_ws(make_plan(dims)).total;
}

ssm_status ssm_block_fwd(ssm_block_ctx* ctx, const ssm_block_dims* dims, const void* X,
                         const ssm_block_params* p, void* Y, void* saved, void* ws, size_t ws_bytes,
                         hipStream_t stream, ssm_timing* timing) {
    if (!ctx || !p) return SSM_E_NULLPTR;
    SSM_TRY(check_block(dims));
    const Plan q = make_plan(dims);
    if (!X || !Y || !p->W_in || !p->conv_w || !p->W_x || !p->W_dt || !p->dt_bias || !p->A_log || !p->D ||
        !p->W_out)
        return SSM_E_NULLPTR;
    if (any_misaligned({X, Y, saved, ws, p->W_in, p->conv_w, p->conv_b, p->W_x, p->W_dt, p->dt_bias, p->A_log,
                        p->D, p->W_out}))
        return SSM_E_ALIGN;
    const FwdWs w = fwd_ws(q);
    const size_t need = saved ? w.training : w.total;
    if (!ws || ws_bytes < need) return SSM_E_WORKSPACE;
    (void)hipGetLastError();
    const Saved s = saved_layout(q);
    char* act = saved ? static_cast<char*>(saved) : static_cast<char*>(ws) + w.act;
    void *xi = act + s.xi, *z = act + s.z, *xc = act + s.xc, *proj = act + s.proj, *dtl = act + s.dtl,
         *Bm = act + s.Bm, *Cm = act + s.Cm, *dt = act + s.dt, *ys = act + s.ys;
    float* ckpt = saved ? reinterpret_cast<float*>(act + s.ckpt) : nullptr;
    const hipDataType io_t = q.io == SSM_BF16 ? HIP_R_16BF : HIP_R_32F;
    const Gemm gemm{ctx, io_t, io_t, stream, static_cast<char*>(ws) + w.gemm, timing};
    const char* W_in = static_cast<const char*>(p->W_in);
    const size_t half = (size_t)q.di * q.dm * q.esz;
    SSM_TRY(gemm(false, true, q.T, q.di, q.dm, X, q.dm, W_in, q.dm, 0.0f, xi, q.di));
    SSM_TRY(gemm(false, true, q.T, q.di, q.dm, X, q.dm, W_in + half, q.dm, 0.0f, z, q.di));
    const ssm_conv_dims cd = conv_dims(q);
    SSM_TRY(ssm_conv1d_fwd(&cd, xi, p->conv_w, p->conv_b, nullptr, xc, nullptr, stream, timing));
    SSM_TRY(gemm(false, true, q.T, q.P, q.di, xc, q.di, p->W_x, q.di, 0.0f, proj, q.P));
    SSM_TRY(launch_proj(q, true, proj, dtl, Bm, Cm, stream, timing));
    SSM_TRY(gemm(false, true, q.T, q.di, q.R, dtl, q.R, p->W_dt, q.R, 0.0f, dt, q.di));
    const ssm_dims sd = scan_dims(q);
    SSM_TRY(ssm_scan_fwd(&sd, xc, dt, Bm, Cm, z, p->A_log, p->D, p->dt_bias, nullptr, ys, nullptr, ckpt,
                         static_cast<char*>(ws) + w.scan, w.training - w.scan, stream, timing));
    return gemm(false, true, q.T, q.dm, q.di, ys, q.di, p->W_out, q.di, 0.0f, Y, q.dm);
}

ssm_status ssm_block_bwd(ssm_block_ctx* ctx, const ssm_block_dims* dims, const void* X,
                         const ssm_block_params* p, const void* saved, const void* dY, void* dX,
                         const ssm_block_grads* g, void* ws, size_t ws_bytes, hipStream_t stream,
                         ssm_timing* timing) {
    if (!ctx || !p || !g) return SSM_E_NULLPTR;
    SSM_TRY(check_block(dims));
    const Plan q = make_plan(dims);
    if (!X || !saved || !dY || !dX || !p->W_in || !p->conv_w || !p->W_x || !p->W_dt || !p->dt_bias ||
        !p->A_log || !p->D || !p->W_out)
        return SSM_E_NULLPTR;
    if (!g->dW_in || !g->dconv_w || !g->dconv_b || !g->dW_x || !g->dW_dt || !g->ddt_bias || !g->dA_log ||
        !g->dD || !g->dW_out)
        return SSM_E_NULLPTR;
    if (any_misaligned({X, saved, dY, dX, ws, p->W_in, p->conv_w, p->conv_b, p->W_x, p->W_dt, p->dt_bias,
                        p->A_log, p->D, p->W_out, g->dW_in, g->dconv_w, g->dconv_b, g->dW_x, g->dW_dt,
                        g->ddt_bias, g->dA_log, g->dD, g->dW_out}))
        return SSM_E_ALIGN;
    const BwdWs w = bwd_ws(q);
    if (!ws || ws_bytes < w.total) return SSM_E_WORKSPACE;
    (void)hipGetLastError();
    const Saved s = saved_layout(q);
    const char* act = static_cast<const char*>(saved);
    const void *xi = act + s.xi, *z = act + s.z, *xc = act + s.xc, *dtl = act + s.dtl, *Bm = act + s.Bm,
               *Cm = act + s.Cm, *dt = act + s.dt, *ys = act + s.ys;
    const float* ckpt = reinterpret_cast<const float*>(act + s.ckpt);
    char* wb = static_cast<char*>(ws);
    void *dys = wb + w.dys, *dxc = wb + w.dxc, *ddt = wb + w.ddt, *ddtl = wb + w.ddtl, *dB = wb + w.dB,
         *dC = wb + w.dC, *dz = wb + w.dz, *dproj = wb + w.dproj, *dxi = wb + w.dxi;
    const hipDataType io_t = q.io == SSM_BF16 ? HIP_R_16BF : HIP_R_32F;
    const Gemm gemm{ctx, io_t, io_t, stream, wb + w.gemm, timing};
    // out_proj
    SSM_TRY(gemm(false, false, q.T, q.di, q.dm, dY, q.dm, p->W_out, q.di, 0.0f, dys, q.di));
    float* part = reinterpret_cast<float*>(wb + w.part);
    SSM_TRY(wgrad(gemm, q.dm, q.di, q.T, dY, q.dm, ys, q.di, g->dW_out, part));
    // scan
    const ssm_dims sd = scan_dims(q);
    SSM_TRY(ssm_scan_bwd(&sd, xc, dt, Bm, Cm, z, p->A_log, p->D, p->dt_bias, nullptr, ckpt, dys, dxc, ddt, dB,
                         dC, dz, g->dA_log, g->dD, g->ddt_bias, nullptr, wb + w.scan, w.total - w.scan, stream,
                         timing));
    // dt_proj, then x_proj's gradient rows [d dt_low | dB | dC]
    SSM_TRY(gemm(false, false, q.T, q.R, q.di, ddt, q.di, p->W_dt, q.R, 0.0f, ddtl, q.R));
    SSM_TRY(wgrad(gemm, q.di, q.R, q.T, ddt, q.di, dtl, q.R, g->dW_dt, part));
    SSM_TRY(launch_proj(q, false, ddtl, dB, dC, dproj, stream, timing));
    // x_proj: dxc += dproj W_x
    SSM_TRY(gemm(false, false, q.T, q.di, q.P, dproj, q.P, p->W_x, q.di, 1.0f, dxc, q.di));
    SSM_TRY(wgrad(gemm, q.P, q.di, q.T, dproj, q.P, xc, q.di, g->dW_x, part));
    // conv1d + SiLU
    const ssm_conv_dims cd = conv_dims(q);
    SSM_TRY(ssm_conv1d_bwd(&cd, xi, p->conv_w, p->conv_b, nullptr, dxc, dxi, g->dconv_w, g->dconv_b, nullptr,
                           wb + w.conv, w.scan - w.conv, stream, timing));
    // in_proj
    const char* W_in = static_cast<const char*>(p->W_in);
    const size_t half = (size_t)q.di * q.dm * q.esz;
    SSM_TRY(gemm(false, false, q.T, q.dm, q.di, dxi, q.di, W_in, q.dm, 0.0f, dX, q.dm));
    SSM_TRY(gemm(false, false, q.T, q.dm, q.di, dz, q.di, W_in + half, q.dm, 1.0f, dX, q.dm));
    SSM_TRY(wgrad(gemm, q.di, q.dm, q.T, dxi, q.di, X, q.dm, g->dW_in, part));
    return wgrad(gemm, q.di, q.dm, q.T, dz, q.di, X, q.dm, g->dW_in + (size_t)q.di * q.dm, part);
}

}  // extern "C"
