// ssm_gdn2.hip -- Gated DeltaNet-2 forward for MI355X (gfx950, wave64): the
// gated delta rule with per-key-dimension decay, token by token.
//
// Operation (burn-gdn2 0.1.4, page "src/forward.rs": the recurrence that its
// chunked WY forward regroups, decays kept per key dimension), state S [K, V]:
//   S' = diag(exp(g_t)) S;  vn = w_t * v_t - S'^T (b_t * k_t);
//   S  = S' + k_t vn^T;     o_t = scale * S^T q_t.
//
// Mapping to the hardware
//   * The columns of S evolve independently (every column sees the same key-side
//     vectors q, k, g, b), so a (batch, head) pair splits over V-column blocks.
//   * One column is one 16-lane DPP row: lane r of the row holds key rows
//     R r .. R r + R - 1 (K = 16 R) of that column in VGPRs.  The two sums over
//     the key dimension per token (the erase read and the output) are R
//     in-lane FMAs and four DPP adds across the row, after which every lane of
//     the row holds the total (fixed order: bitwise repeatable).
//   * A wave is 4 columns, a workgroup 16; the column blocks of one (batch,
//     head) pair are numbered to run on one XCD so that its L2 serves their
//     shared key-side reads.  The key-side vectors are staged in
//     chunks of 16 tokens through double-buffered LDS (exp(g) and b * k formed
//     once per element there), loaded while the previous chunk is computed.
//   * No atomics, no MFMA: per token this form is rank-one updates and
//     matrix-vector sums.  The chunked form of the same operation (dense
//     intra-chunk products) is where MFMA would apply.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_common.h"
#include "ssm_gdn2.h"

namespace {

constexpr int WG = 256;
constexpr int ROWS = 16;            // lanes per column (one DPP row)
constexpr int CPB = WG / ROWS;      // columns per workgroup
constexpr int XCDS = 8;             // XCDs of an MI355X (one L2 each)
constexpr float LOG2E = 1.4426950408889634f;

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over the 16 lanes of a DPP row; every lane of the row receives the total.
// IEEE addition is commutative, so the partner lanes of each step compute the
// same bits and the row ends with one value.
__device__ __forceinline__ float row_sum16(float x) {
    x += dpp<0xB1>(x);   // quad_perm [1, 0, 3, 2]: lane ^ 1
    x += dpp<0x4E>(x);   // quad_perm [2, 3, 0, 1]: lane ^ 2
    x += dpp<0x141>(x);  // row_half_mirror: quads 0 <-> 1 within each 8 lanes
    x += dpp<0x140>(x);  // row_mirror: halves of the 16-lane row
    return x;
}

// Four consecutive activations of type T as floats (T = float or bf16 bits).
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const ssm::bf16_t* p) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

// Tokens per chunk staged through LDS: the key-side vectors of a chunk (q, k,
// exp(g) and b * k, K floats each per token) and w * v for the workgroup's
// columns are loaded by the whole workgroup while the previous chunk is being
// computed, and read back per token with wide LDS reads.  One lane of each
// column keeps the output of token r of the chunk and stores it at the end.
constexpr int TC = ROWS;

template <typename TT, int R>
__global__ __launch_bounds__(WG) void k_gdn2_fwd(
    const TT* __restrict__ q, const TT* __restrict__ k, const TT* __restrict__ v,
    const TT* __restrict__ g, const TT* __restrict__ b, const TT* __restrict__ w,
    const float* __restrict__ S0, float scale, TT* __restrict__ o, float* __restrict__ S_last,
    int64_t nbh, int ncb, int T, int V) {
    constexpr int K = ROWS * R;
    constexpr int K4 = K / 4 > 0 ? K / 4 : 1;          // float4 pieces per token row (K >= 16)
    constexpr int NST = (TC * K4 + WG - 1) / WG;       // float4 pieces per thread per vector
    __shared__ float4 sq[2][TC * K4], sk[2][TC * K4], se[2][TC * K4], sbk[2][TC * K4];
    __shared__ float swv[2][TC][CPB];
    const int tid = threadIdx.x;
    const int r = tid & (ROWS - 1);
    const int cl = tid >> 4;                 // column within the workgroup
    // Workgroups go round-robin over the 8 XCDs, each with its own L2.  The ncb
    // column blocks of one (batch, head) pair read the same key-side vectors, so
    // they are numbered to run on one XCD: each run of 8 ncb consecutive
    // workgroups holds 8 pairs, pair (8 g + x) on XCD x.
    const int64_t grp = blockIdx.x / (XCDS * ncb);
    const int within = (int)(blockIdx.x % (XCDS * ncb));
    const int64_t bh = grp * XCDS + within % XCDS;
    if (bh >= nbh) return;  // tail of the last run: the whole workgroup, before any barrier
    const int j0 = (within / XCDS) * CPB;
    const int j = j0 + cl;
    const bool act = j < V;
    const int jc = act ? j : V - 1;
    const TT* qb = q + bh * T * K;
    const TT* kb = k + bh * T * K;
    const TT* gb = g + bh * T * K;
    const TT* bb = b + bh * T * K;
    float S[R];
#pragma unroll
    for (int i = 0; i < R; ++i) S[i] = S0 ? S0[(bh * K + R * r + i) * V + jc] : 0.0f;
    const int nch = (T + TC - 1) / TC;

    // staging registers: this thread's pieces of one chunk
    float4 rq[NST], rk[NST], rg[NST], rb[NST];
    float rwv = 0.0f;
    auto stage_load = [&](int c) {
        const int t0 = c * TC, nt = min(TC, T - t0);
#pragma unroll
        for (int s2 = 0; s2 < NST; ++s2) {
            const int idx = tid + s2 * WG;
            if (idx < nt * K4) {
                const int64_t off = (int64_t)t0 * K + (int64_t)idx * 4;
                rq[s2] = load4(qb + off);
                rk[s2] = load4(kb + off);
                rg[s2] = load4(gb + off);
                rb[s2] = load4(bb + off);
            }
        }
        const int tt = tid / CPB, col = j0 + tid % CPB;
        rwv = 0.0f;
        if (tt < nt && col < V) {
            const int64_t e = (bh * T + t0 + tt) * V + col;
            rwv = ssm::to_f(w[e]) * ssm::to_f(v[e]);
        }
    };
    auto stage_store = [&](int c, int buf) {
        const int nt = min(TC, T - c * TC);
#pragma unroll
        for (int s2 = 0; s2 < NST; ++s2) {
            const int idx = tid + s2 * WG;
            if (idx < nt * K4) {
                const float4 gv = rg[s2], bv = rb[s2], kv = rk[s2];
                sq[buf][idx] = rq[s2];
                sk[buf][idx] = kv;
                se[buf][idx] = make_float4(__builtin_amdgcn_exp2f(gv.x * LOG2E), __builtin_amdgcn_exp2f(gv.y * LOG2E),
                                           __builtin_amdgcn_exp2f(gv.z * LOG2E), __builtin_amdgcn_exp2f(gv.w * LOG2E));
                sbk[buf][idx] = make_float4(bv.x * kv.x, bv.y * kv.y, bv.z * kv.z, bv.w * kv.w);
            }
        }
        swv[buf][tid / CPB][tid % CPB] = rwv;
    };

    if (nch > 0) {
        stage_load(0);
        stage_store(0, 0);
    }
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const int buf = c & 1;
        const int t0 = c * TC, nt = min(TC, T - t0);
        if (c + 1 < nch) stage_load(c + 1);  // in flight during this chunk
        const float* fq = reinterpret_cast<const float*>(sq[buf]) + R * r;
        const float* fk = reinterpret_cast<const float*>(sk[buf]) + R * r;
        const float* fe = reinterpret_cast<const float*>(se[buf]) + R * r;
        const float* fb = reinterpret_cast<const float*>(sbk[buf]) + R * r;
        float mine = 0.0f;  // output of token t0 + r of this column
        // one token: decay, erase read S'^T (b k), write k vn^T, output read S^T q;
        // each key-dimension sum is two in-lane partials (fixed order) and a row sum
        auto token = [&](int tt) {
            float u0 = 0.0f, u1 = 0.0f;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                S[i] *= fe[tt * K + i];
                if (i & 1) u1 = __builtin_fmaf(fb[tt * K + i], S[i], u1);
                else u0 = __builtin_fmaf(fb[tt * K + i], S[i], u0);
            }
            const float vnew = swv[buf][tt][cl] - row_sum16(u0 + u1);
            float o0 = 0.0f, o1 = 0.0f;
#pragma unroll
            for (int i = 0; i < R; ++i) {
                S[i] = __builtin_fmaf(fk[tt * K + i], vnew, S[i]);
                if (i & 1) o1 = __builtin_fmaf(fq[tt * K + i], S[i], o1);
                else o0 = __builtin_fmaf(fq[tt * K + i], S[i], o0);
            }
            const float ot = row_sum16(o0 + o1);
            if (tt == r) mine = ot;
        };
        if (nt == TC) {  // full chunk: unrolled, so LDS reads can run ahead of the chain
#pragma unroll
            for (int tt = 0; tt < TC; ++tt) token(tt);
        } else {
            for (int tt = 0; tt < nt; ++tt) token(tt);
        }
        if (act && r < nt) o[(bh * T + t0 + r) * V + j] = ssm::from_f<TT>(scale * mine);
        if (c + 1 < nch) stage_store(c + 1, buf ^ 1);
        __syncthreads();
    }
    if (S_last && act) {
#pragma unroll
        for (int i = 0; i < R; ++i) S_last[(bh * K + R * r + i) * V + j] = S[i];
    }
}

ssm_status check_gdn2(const ssm_gdn2_dims* d) {
    if (!d) return SSM_E_NULLPTR;
    if (d->batch < 1 || d->heads < 1 || d->seqlen < 0 || d->k_dim < 1 || d->v_dim < 1) return SSM_E_SHAPE;
    if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_E_DTYPE;
    if (d->k_dim != 16 && d->k_dim != 32 && d->k_dim != 64 && d->k_dim != 128) return SSM_E_UNSUPPORTED;
    // one-dimensional grid of at most 2^31 workgroups
    const int64_t ncb = (d->v_dim + 15) / 16, nbh = d->batch * d->heads;
    if (d->batch > 65535 || d->heads > 65535 || d->seqlen > ((int64_t)1 << 30) ||
        d->v_dim > ((int64_t)1 << 30) || (nbh + 7) / 8 * 8 * ncb >= ((int64_t)1 << 31))
        return SSM_E_UNSUPPORTED;
    return SSM_OK;
}

template <typename TT, int R>
ssm_status run(const ssm_gdn2_dims* d, const void* q, const void* k, const void* v, const void* g,
               const void* b, const void* w, const float* S0, float scale, void* o, float* S_last,
               ssm::Launcher& launch) {
    const int64_t nbh = d->batch * d->heads;
    const int ncb = (int)((d->v_dim + CPB - 1) / CPB);
    const int64_t nwg = (nbh + XCDS - 1) / XCDS * XCDS * ncb;
    return launch(SSM_K_GDN2_FWD, k_gdn2_fwd<TT, R>, dim3((unsigned)nwg), dim3(WG), (const TT*)q, (const TT*)k,
                  (const TT*)v, (const TT*)g, (const TT*)b, (const TT*)w, S0, scale, (TT*)o, S_last, nbh, ncb,
                  (int)d->seqlen, (int)d->v_dim);
}

template <typename TT>
ssm_status run_k(const ssm_gdn2_dims* d, const void* q, const void* k, const void* v, const void* g,
                 const void* b, const void* w, const float* S0, float scale, void* o, float* S_last,
                 ssm::Launcher& launch) {
    switch (d->k_dim) {
        case 16: return run<TT, 1>(d, q, k, v, g, b, w, S0, scale, o, S_last, launch);
        case 32: return run<TT, 2>(d, q, k, v, g, b, w, S0, scale, o, S_last, launch);
        case 64: return run<TT, 4>(d, q, k, v, g, b, w, S0, scale, o, S_last, launch);
        default: return run<TT, 8>(d, q, k, v, g, b, w, S0, scale, o, S_last, launch);
    }
}

}  // namespace

extern "C" {

ssm_status ssm_gdn2_fwd(const ssm_gdn2_dims* dims, const void* q, const void* k, const void* v,
                        const void* g, const void* b, const void* w, const float* S0, float scale,
                        void* o, float* S_last, hipStream_t stream, ssm_timing* timing) {
    SSM_TRY(check_gdn2(dims));
    if (dims->seqlen > 0 && (!q || !k || !v || !g || !b || !w || !o)) return SSM_E_NULLPTR;
    if (S_last && S_last == S0) return SSM_E_UNSUPPORTED;
    const void* ptrs[] = {q, k, v, g, b, w, S0, o, S_last};
    for (const void* p : ptrs)
        if (p && ssm::misaligned(p)) return SSM_E_ALIGN;
    if (dims->seqlen == 0 && !S_last) return SSM_OK;
    (void)hipGetLastError();
    ssm::Launcher launch{stream, timing};
    if (dims->io_dtype == SSM_BF16) return run_k<ssm::bf16_t>(dims, q, k, v, g, b, w, S0, scale, o, S_last, launch);
    return run_k<float>(dims, q, k, v, g, b, w, S0, scale, o, S_last, launch);
}

}  // extern "C"
