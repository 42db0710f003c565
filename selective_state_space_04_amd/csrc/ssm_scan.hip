// ssm_scan.hip -- Mamba S6 selective scan for MI355X (gfx950, CDNA4, wave64).
//
// Operation (rustytorch commit log, page "crates/training/rtx-transformers/tests",
// commit replacing the MambaBlock stub with a real S6 forward):
//   delta = softplus(dt + dt_bias), A = -exp(A_log)
//   h_t   = exp(delta*A) * h_{t-1} + delta*B_t*x_t        (per batch, channel, state)
//   y_t   = (sum_n C_t[n] h_t[n] + D x_t) * silu(z_t)
// Backward: the reverse-time adjoint (commit adding the hand-written VJP),
// dA_log = dA * A, parameter gradients summed over batch and time.
// Step: the forward's per-token body on a carried state (commit introducing
// MambaRecurrence::step); it shares scan_token()/finish_y() with the forward so
// that stepping reproduces a single-chunk forward bit for bit.
//
// Mapping to the hardware
//   * One lane owns one (batch, channel) and its 16 states in VGPRs.  A
//     workgroup is 256 consecutive channels of one batch row, so x/dt/z/y are
//     coalesced per token and B_t/C_t (shared by all channels) are
//     wave-uniform loads served by the scalar cache.
//   * Long sequences are cut into K chunks so that batch*d_inner*K lanes fill
//     the 256 CUs.  Forward: (1) each chunk's zero-start end state S and delta
//     sum; (2) a sequential combine h <- exp(A*sum delta)*h + S over chunks
//     gives every chunk's true start; (3) every chunk re-runs from its start and
//     writes y and the checkpoints.  The backward mirrors this with the adjoint
//     (lambda <- exp(A*sum delta)*lambda + G, walking chunks in reverse).
//   * When batch*d_inner alone gives too few lanes but 16x as many would do,
//     or the sequence is short, the forward instead runs one lane per
//     (channel, state) over the whole sequence in one kernel (k_fwd_state, no
//     chunks).
//   * The backward recomputes states from checkpoints taken every TS tokens,
//     keeps the TS+1 states of a block in registers and sweeps it in reverse.
//   * dB/dC (sums over channels) are reduced through LDS per wave, across the
//     4 waves per block, then across workgroups by a fixed-order kernel: no
//     atomics, bitwise deterministic.
//   * exp(delta*A) is one v_exp_f32 of delta*(A*log2 e).  No MFMA: nothing on
//     this path is a dense contraction.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <utility>

#include "ssm_common.h"
#include "ssm_scan.h"

namespace {

using ssm::bf16_t;
using ssm::from_f;
using ssm::misaligned;
using ssm::sigmoid_f;
using ssm::to_f;

constexpr int NS = 16;    // d_state handled by these kernels
constexpr int TS = 8;     // checkpoint stride (tokens)
constexpr int WG = 256;   // threads per workgroup: one channel each
constexpr int NWAVE = WG / 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int64_t TARGET_LANES = 262144;  // 4096 waves = 4 per SIMD
constexpr int64_t MIN_CHUNK = 64;
// From this many batch rows x channels up to TARGET_LANES the forward runs one
// lane per (channel, state) over the whole sequence (k_fwd_state): at least
// 2048 waves, 2 per SIMD.  A forward that writes checkpoints does so only below
// STATE_LANES_CKPT_L tokens: measured at 4 x L x 5120 bf16, its checkpoint
// stores fall behind as the sequence grows (faster than the chunked form up to
// 14336 tokens, even at 16384, 5.1 against 4.4 ms at 32768), while without
// checkpoints it stays ahead at every length.
constexpr int64_t STATE_LANES_MIN = 8192;
constexpr int64_t STATE_LANES_CKPT_L = 16384;
// Below STATE_LANES_MIN the lane-per-state forward is still taken for sequences of
// up to this many tokens, where the chunked form is bound by latency.
constexpr int64_t STATE_LANES_SHORT_L = 512;
constexpr int64_t NUM_CU = 256;
// Resident workgroups of the forward main kernel (6 waves/SIMD: 73-76 VGPRs in
// its gated variants, allocated in steps of 8 out of 512) and of the backward
// main kernel (2 waves/SIMD at 256 VGPRs), chip-wide.
constexpr int64_t FWD_SLOTS = NUM_CU * 6;
constexpr int64_t BWD_SLOTS = NUM_CU * 2;

// ------------------------------------------------------------------ io helpers
// 16 consecutive values (one B_t or C_t row); the address is wave-uniform.
__device__ __forceinline__ void load16(const float* __restrict__ p, float v[NS]) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 f = q[i];
        v[4 * i + 0] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
    }
}
__device__ __forceinline__ void load16(const bf16_t* __restrict__ p, float v[NS]) {
    const uint4* q = reinterpret_cast<const uint4*>(p);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        uint4 u = q[i];
        uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[8 * i + 2 * j + 0] = __uint_as_float(w[j] << 16);
            v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
}

// A 16-value row (B_t or C_t) loaded now and converted to f32 later, so that
// the wait for it can come a token after the load was issued.
template <typename T>
struct RawRow;
template <>
struct RawRow<float> {
    float4 q[4];
    __device__ __forceinline__ void load(const float* __restrict__ p) {
        const float4* s = reinterpret_cast<const float4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = s[i];
    }
    __device__ __forceinline__ void get(float v[NS]) const {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[4 * i + 0] = q[i].x; v[4 * i + 1] = q[i].y; v[4 * i + 2] = q[i].z; v[4 * i + 3] = q[i].w;
        }
    }
};
template <>
struct RawRow<bf16_t> {
    uint4 q[2];
    __device__ __forceinline__ void load(const bf16_t* __restrict__ p) {
        const uint4* s = reinterpret_cast<const uint4*>(p);
        q[0] = s[0];
        q[1] = s[1];
    }
    __device__ __forceinline__ void get(float v[NS]) const {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const uint32_t w[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[8 * i + 2 * j + 0] = __uint_as_float(w[j] << 16);
                v[8 * i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        }
    }
};

__device__ __forceinline__ void load_state(const float* __restrict__ p, float h[NS]) {
    const float4* q = reinterpret_cast<const float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 f = q[i];
        h[4 * i + 0] = f.x; h[4 * i + 1] = f.y; h[4 * i + 2] = f.z; h[4 * i + 3] = f.w;
    }
}
// Grouped state rows: states 4g..4g+3 of channel d at base[(g * D + d) * 4 ..],
// base wave-uniform.  Each of the 4 accesses moves 16 bytes per lane, and the
// lanes of a wave (consecutive channels) cover one dense 1 KB piece.
__device__ __forceinline__ void load_state_g4(const float* __restrict__ base, int64_t D, int64_t d,
                                              float h[NS]) {
#pragma unroll
    for (int g = 0; g < NS / 4; ++g) {
        const float4 f = reinterpret_cast<const float4*>(base)[g * D + d];
        h[4 * g + 0] = f.x; h[4 * g + 1] = f.y; h[4 * g + 2] = f.z; h[4 * g + 3] = f.w;
    }
}
__device__ __forceinline__ void store_state_g4(float* __restrict__ base, int64_t D, int64_t d,
                                               const float h[NS]) {
#pragma unroll
    for (int g = 0; g < NS / 4; ++g)
        reinterpret_cast<float4*>(base)[g * D + d] = make_float4(h[4 * g], h[4 * g + 1], h[4 * g + 2], h[4 * g + 3]);
}
__device__ __forceinline__ void store_state(float* __restrict__ p, const float h[NS]) {
    float4* q = reinterpret_cast<float4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) q[i] = make_float4(h[4 * i], h[4 * i + 1], h[4 * i + 2], h[4 * i + 3]);
}

// ---------------------------------------------------------------- token math
// A2[n] = A[n] * log2(e) with A = -exp(A_log), so exp(delta*A) = exp2(delta*A2).
// exp(A_log) is one v_exp_f32 of A_log*log2(e) (about 2e-7 relative).
__device__ __forceinline__ void load_A2(const float* __restrict__ A_log, int d, float A2[NS]) {
    const float4* p = reinterpret_cast<const float4*>(A_log + (int64_t)d * NS);
#pragma unroll
    for (int i = 0; i < NS / 4; ++i) {
        const float4 v = p[i];
        A2[4 * i + 0] = -__builtin_amdgcn_exp2f(v.x * LOG2E) * LOG2E;
        A2[4 * i + 1] = -__builtin_amdgcn_exp2f(v.y * LOG2E) * LOG2E;
        A2[4 * i + 2] = -__builtin_amdgcn_exp2f(v.z * LOG2E) * LOG2E;
        A2[4 * i + 3] = -__builtin_amdgcn_exp2f(v.w * LOG2E) * LOG2E;
    }
}

// Stable softplus(u) = max(u, 0) + log1p(e), e = exp(-|u|) in (0, 1], and
// sigmoid(u) (its derivative).  log1p(e) comes from one hardware log2 through
// the compensated form log1p(e) = log(w) * e / (w - 1), w = fl(1 + e): the
// rounding of w cancels in the ratio, so the result stays within a few ulp
// even when e is tiny (Goldberg, "What every computer scientist should know
// about floating-point arithmetic", 1991, Theorem 4).
__device__ __forceinline__ float softplus_sig(float u, float& sig) {
    const float e = __builtin_amdgcn_exp2f(-fabsf(u) * LOG2E);
    const float w = 1.0f + e;
    const float wm1 = w - 1.0f;
    const float r = __builtin_amdgcn_rcpf(w);
    sig = u >= 0.0f ? r : e * r;
    const float lp = wm1 == 0.0f
                         ? e
                         : (__builtin_amdgcn_logf(w) * LN2) * (e * __builtin_amdgcn_rcpf(wm1));
    return fmaxf(u, 0.0f) + lp;
}

// One token of the recurrence for one channel: h <- exp2(delta*A2) h + (delta x) B,
// returns sum_n C[n] h[n] (accumulated in state order).
__device__ __forceinline__ float scan_token(float h[NS], const float A2[NS], const float Bv[NS],
                                            const float Cv[NS], float delta, float xv) {
    const float dxv = delta * xv;
    float acc = 0.0f;
#pragma unroll
    for (int n = 0; n < NS; ++n) {
        const float a = __builtin_amdgcn_exp2f(delta * A2[n]);
        h[n] = __builtin_fmaf(a, h[n], dxv * Bv[n]);
        acc = __builtin_fmaf(Cv[n], h[n], acc);
    }
    return acc;
}

template <bool GATE>
__device__ __forceinline__ float finish_y(float acc, float Dd, float xv, float zv) {
    const float ypre = __builtin_fmaf(Dd, xv, acc);
    if (!GATE) return ypre;
    return ypre * (zv * sigmoid_f(zv));
}

// Streaming per-lane loads of one activation column (stride D elements); the
// value of token i+1 is fetched while token i is processed.
template <typename T>
struct Stream {
    const T* p;
    int64_t stride;
    __device__ __forceinline__ float at(int i) const { return to_f(p[(int64_t)i * stride]); }
    __device__ __forceinline__ T raw(int i) const { return p[(int64_t)i * stride]; }
};

// Per-lane loads run PF tokens ahead of use (a ring of raw values; the token
// loop is unrolled PF times so the ring rotation is register renaming).
constexpr int PF = 3;

// ===================================================================== forward

// (1) zero-start end state S and delta sum of chunk k (k = 0 .. K-2).
template <typename T>
__global__ __launch_bounds__(WG) void k_fwd_chunk(
    const T* __restrict__ x, const T* __restrict__ dt, const T* __restrict__ Bm,
    const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    float* __restrict__ wsS, float* __restrict__ wsSum, int L, int D, int Tc, int K) {
    const int d = blockIdx.x * WG + threadIdx.x;
    const int k = blockIdx.y;
    const int b = blockIdx.z;
    const bool act = d < D;
    const int dc = act ? d : D - 1;
    float A2[NS];
    load_A2(A_log, dc, A2);
    const float bias = dt_bias ? dt_bias[dc] : 0.0f;
    float S[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) S[n] = 0.0f;
    float sumd = 0.0f;
    const int t0 = k * Tc, nt = min(Tc, L - t0);
    const int64_t row0 = (int64_t)b * L + t0;
    const Stream<T> xs{x + row0 * D + dc, D}, ds{dt + row0 * D + dc, D};
    const T* bp = Bm + row0 * NS;
    T xq[PF], dq[PF];
#pragma unroll
    for (int q = 0; q < PF; ++q) {
        xq[q] = xs.raw(min(q, nt - 1));
        dq[q] = ds.raw(min(q, nt - 1));
    }
    float Bn[NS];
    load16(bp, Bn);
#pragma unroll PF
    for (int i = 0; i < nt; ++i) {
        const float xv = to_f(xq[0]), dtv = to_f(dq[0]);
#pragma unroll
        for (int q = 0; q + 1 < PF; ++q) {
            xq[q] = xq[q + 1];
            dq[q] = dq[q + 1];
        }
        xq[PF - 1] = xs.raw(min(i + PF, nt - 1));
        dq[PF - 1] = ds.raw(min(i + PF, nt - 1));
        const int ip = min(i + 1, nt - 1);
        float Bv[NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) Bv[n] = Bn[n];
        load16(bp + (int64_t)ip * NS, Bn);  // next token's row (scalar cache)
        float sg;
        const float delta = softplus_sig(dtv + bias, sg);
        const float dxv = delta * xv;
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const float a = __builtin_amdgcn_exp2f(delta * A2[n]);
            S[n] = __builtin_fmaf(a, S[n], dxv * Bv[n]);
        }
        sumd += delta;
    }
    if (act) {
        const int64_t e = (int64_t)b * (K - 1) + k;
        store_state_g4(wsS + e * NS * D, D, d, S);
        wsSum[e * D + d] = sumd;
    }
}

// (2) chunk start states: starts(b, k) for k = 0..K-1, sequential over chunks.
//     One lane per (batch, channel, state): the 16 states of a channel are
//     independent here.  The chunk end states and delta sums are fetched CB
//     chunks at a time, so that many loads are in flight per step of the
//     sequential combine.
constexpr int CB = 8;
__device__ __forceinline__ float a2_of(const float* __restrict__ A_log, int64_t i) {
    return -__builtin_amdgcn_exp2f(A_log[i] * LOG2E) * LOG2E;  // as load_A2
}
__global__ __launch_bounds__(WG) void k_fwd_carry(
    const float* __restrict__ A_log, const float* __restrict__ h0, const float* __restrict__ wsS,
    const float* __restrict__ wsSum, float* __restrict__ starts, int D, int K,
    int64_t start_bs, int64_t start_ks) {
    const int64_t DN = (int64_t)D * NS;
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;  // (state group, channel, state % 4)
    const int b = blockIdx.z;
    if (i >= DN) return;
    const int64_t d = (i / 4) % D, n = 4 * (i / (4 * D)) + i % 4;
    const float A2 = a2_of(A_log, d * NS + n);
    float h = h0 ? h0[(int64_t)b * DN + d * NS + n] : 0.0f;
    const int64_t e0 = (int64_t)b * (K - 1);  // entry of chunk 0 in wsS / wsSum
    for (int k0 = 0; k0 < K - 1; k0 += CB) {
        float Sb[CB], sb[CB];
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            if (k0 + j < K - 1) {
                Sb[j] = wsS[(e0 + k0 + j) * DN + i];
                sb[j] = wsSum[(e0 + k0 + j) * D + d];
            }
        }
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            if (k0 + j < K - 1) {
                starts[((int64_t)b * start_bs + (int64_t)(k0 + j) * start_ks) * DN + i] = h;
                const float P = __builtin_amdgcn_exp2f(A2 * sb[j]);
                h = __builtin_fmaf(P, h, Sb[j]);
            }
        }
    }
    starts[((int64_t)b * start_bs + (int64_t)(K - 1) * start_ks) * DN + i] = h;
}

// (3) recurrence of chunk k from its start; writes y, checkpoints and h_last.
template <typename T, bool GATE>
__global__ __launch_bounds__(WG) void k_fwd_main(
    const T* __restrict__ x, const T* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const T* __restrict__ z, const float* __restrict__ A_log,
    const float* __restrict__ Dp, const float* __restrict__ dt_bias,
    const float* __restrict__ h0, const float* __restrict__ starts, T* __restrict__ y,
    float* __restrict__ h_last, float* __restrict__ ckpt, int L, int D, int Tc, int K,
    int64_t start_bs, int64_t start_ks) {
    const int d = blockIdx.x * WG + threadIdx.x;
    const int k = blockIdx.y;
    const int b = blockIdx.z;
    const bool act = d < D;
    const int dc = act ? d : D - 1;
    float A2[NS];
    load_A2(A_log, dc, A2);
    const float bias = dt_bias ? dt_bias[dc] : 0.0f;
    const float Dd = Dp ? Dp[dc] : 0.0f;
    float h[NS];
    if (k > 0) {
        load_state_g4(starts + ((int64_t)b * start_bs + (int64_t)k * start_ks) * NS * D, D, dc, h);
    } else if (h0) {
        load_state(h0 + ((int64_t)b * D + dc) * NS, h);
    } else {
#pragma unroll
        for (int n = 0; n < NS; ++n) h[n] = 0.0f;
    }
    const int t0 = k * Tc, nt = min(Tc, L - t0);
    const int64_t row0 = (int64_t)b * L + t0;
    const Stream<T> xs{x + row0 * D + dc, D}, ds{dt + row0 * D + dc, D};
    const Stream<T> zs{GATE ? z + row0 * D + dc : nullptr, D};
    const T* bp = Bm + row0 * NS;
    const T* cp = Cm + row0 * NS;
    T* yp = y + row0 * D + d;
    // checkpoints [L/8, batch, 4, D, 4]: the rows of all batch rows for one
    // token block are adjacent
    const int64_t ckstride = (int64_t)gridDim.z * D * NS;
    float* ck = ckpt ? ckpt + ((int64_t)(t0 / TS) * gridDim.z + b) * NS * D : nullptr;
    T xq[PF], dq[PF], zq[PF];
#pragma unroll
    for (int q = 0; q < PF; ++q) {
        xq[q] = xs.raw(min(q, nt - 1));
        dq[q] = ds.raw(min(q, nt - 1));
        zq[q] = GATE ? zs.raw(min(q, nt - 1)) : T(0);
    }
    float Bn[NS], Cn[NS];
    load16(bp, Bn);
    load16(cp, Cn);
    T ypend = T(0);  // output of the previous token, stored one token late
#pragma unroll PF
    for (int i = 0; i < nt; ++i) {
        const float xv = to_f(xq[0]), dtv = to_f(dq[0]), zv = GATE ? to_f(zq[0]) : 0.0f;
#pragma unroll
        for (int q = 0; q + 1 < PF; ++q) {
            xq[q] = xq[q + 1];
            dq[q] = dq[q + 1];
            zq[q] = zq[q + 1];
        }
        xq[PF - 1] = xs.raw(min(i + PF, nt - 1));
        dq[PF - 1] = ds.raw(min(i + PF, nt - 1));
        if (GATE) zq[PF - 1] = zs.raw(min(i + PF, nt - 1));
        // the previous token's output and, every TS tokens, the checkpoint (state
        // before token t0+i; chunk starts k>0 come from the carry kernel) are
        // stored after this token's prefetch loads are issued: a later wait on a
        // load would also wait for every store issued before it
        if (i > 0 && act) yp[(int64_t)(i - 1) * D] = ypend;
        if ((i & (TS - 1)) == 0 && ck && act && (i > 0 || k == 0))
            store_state_g4(ck + (int64_t)(i / TS) * ckstride, D, d, h);
        const int ip = min(i + 1, nt - 1);
        float Bv[NS], Cv[NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            Bv[n] = Bn[n];
            Cv[n] = Cn[n];
        }
        load16(bp + (int64_t)ip * NS, Bn);  // next token's rows (scalar cache)
        load16(cp + (int64_t)ip * NS, Cn);
        float sg;
        const float delta = softplus_sig(dtv + bias, sg);
        const float acc = scan_token(h, A2, Bv, Cv, delta, xv);
        ypend = from_f<T>(finish_y<GATE>(acc, Dd, xv, zv));
    }
    if (nt > 0 && act) yp[(int64_t)(nt - 1) * D] = ypend;
    if (h_last && act && k == K - 1) store_state(h_last + ((int64_t)b * D + d) * NS, h);
}

// (4) The forward in one pass, one lane per (batch, channel, state): used when
//     batch rows x channels give too few lanes at one lane per channel, where
//     the chunked form above would pay a second exp per element in its chunk
//     pass.  Here every lane walks the whole sequence (16x the lanes of the
//     chunked form, so no chunks are needed) and each element's exp is taken
//     once.  A wave holds 4 channels x 16 states, one 16-lane row per channel.
//     Per tile of 16 tokens:
//       * lane n of a row does the per-token channel work (softplus, gate,
//         output) of token t0+n and hands delta and delta*x to its row with DPP
//         row broadcasts folded into the multiplies;
//       * B and C of the tile are staged in LDS as [state][token] f32, so a
//         lane reads its state's 16 values with 4 vector reads;
//       * x, dt, z come in and y goes out through LDS as 16-channel row pieces
//         (one instruction per tensor and tile), checkpoints as 256-byte pieces;
//       * the readout sum over the 16 states is a butterfly over the row
//         (the first two stages as bank-masked DPP adds); after it, lane n
//         holds the sum of token t0+n.
//     The states follow the same operations as scan_token(), bit for bit; the
//     readout sums them in butterfly order instead of state order.
constexpr int LT = 16;       // tokens per tile (= lanes per channel row)
constexpr int LRS = LT + 4;  // LDS row stride in floats: 16-byte rows, conflict-free reads

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}
// one butterfly stage between lanes that differ in bit M of their row index:
// each keeps the M slots of its half and adds the partner's copy of them
template <int M, int CTRL>
__device__ __forceinline__ void bfly(float* v, bool hi) {
#pragma unroll
    for (int j = 0; j < M; ++j) {
        const float keep = hi ? v[j + M] : v[j];
        const float send = hi ? v[j] : v[j + M];
        v[j] = keep + dpp_f<CTRL>(send);
    }
}
template <typename F, int... I>
__device__ __forceinline__ void for_each_i(F&& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
// two consecutive states' values of one B or C row (4 bytes in bf16, 8 in f32)
template <typename T> struct Pair;
template <> struct Pair<float> {
    float2 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float2*>(p); }
    __device__ __forceinline__ float lo() const { return v.x; }
    __device__ __forceinline__ float hi() const { return v.y; }
};
template <> struct Pair<bf16_t> {
    uint32_t v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint32_t*>(p); }
    __device__ __forceinline__ float lo() const { return __uint_as_float(v << 16); }
    __device__ __forceinline__ float hi() const { return __uint_as_float(v & 0xffff0000u); }
};

// 4 consecutive activations of one token row (8 bytes in bf16, 16 in f32)
template <typename T> struct Quad;
template <> struct Quad<float> {
    float4 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const float4*>(p); }
    __device__ __forceinline__ void store(float* p) const { *reinterpret_cast<float4*>(p) = v; }
};
template <> struct Quad<bf16_t> {
    uint2 v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ void store(bf16_t* p) const { *reinterpret_cast<uint2*>(p) = v; }
};

template <typename T, bool GATE, bool CK>
__global__ __launch_bounds__(WG) void k_fwd_state(
    const T* __restrict__ x, const T* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const T* __restrict__ z, const float* __restrict__ A_log,
    const float* __restrict__ Dp, const float* __restrict__ dt_bias,
    const float* __restrict__ h0, T* __restrict__ y, float* __restrict__ h_last,
    float* __restrict__ ckpt, int L, int D, int ncb) {
    __shared__ float bc[2][2][NS * LRS];    // [buffer][B, C][state][token]
    __shared__ T act_s[2][3][LT][16];       // [buffer][x, dt, z][token][channel of the block]
    __shared__ T y_s[2][LT][16];            // [buffer][token][channel of the block]
    __shared__ float4 ck_s[2][2][4][16];     // [buffer][checkpoint][state group][channel of the block]
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int n = lane & 15;
    // channel blocks of 16; the 4 blocks of one 64-channel row segment are
    // numbered onto one XCD (blocks are dealt to the 8 XCDs round robin)
    const int xb = blockIdx.x;
    const int cb = 4 * ((xb & 7) + 8 * (xb >> 5)) + ((xb >> 3) & 3);
    if (cb >= ncb) return;  // uniform over the workgroup
    const int cw = wave * 4 + (lane >> 4);  // channel within the block
    const int d = cb * 16 + cw;             // D is a multiple of 16 on this path
    const int b = blockIdx.y;
    const float A2 = a2_of(A_log, (int64_t)d * NS + n);
    const float bias = dt_bias ? dt_bias[d] : 0.0f;
    const float Dd = Dp ? Dp[d] : 0.0f;
    float h = h0 ? h0[((int64_t)b * D + d) * NS + n] : 0.0f;
    const int64_t row0 = (int64_t)b * L;
    // B and C staging: thread -> (tensor, token, pair of states)
    const int st = threadIdx.x >> 7, sw = threadIdx.x & 127, stok = sw >> 3, sn = 2 * (sw & 7);
    const T* sp = (st ? Cm : Bm) + row0 * NS + sn;
    // activation staging (threads 0..191) and output rows (threads 0..63):
    // thread -> (tensor, token, 4 channels)
    const int aq = threadIdx.x >> 6, atok = (threadIdx.x & 63) >> 2, a4 = 4 * (threadIdx.x & 3);
    const bool astage = threadIdx.x < 3 * 64 && (GATE || aq < 2);
    const T* ap = (aq == 0 ? x : aq == 1 ? dt : z) + row0 * D + cb * 16 + a4;
    T* yrow = y + row0 * D + cb * 16 + a4;
    const int ntile = (L + LT - 1) / LT;
    // checkpoints of the previous tile (states before its tokens 0 and 8),
    // written as 4 x 256-byte pieces per checkpoint: thread -> (checkpoint,
    // state group, channel)
    auto store_ck = [&](int buf, int tp) {
        const int which = threadIdx.x >> 6, g = (threadIdx.x >> 4) & 3, c16 = threadIdx.x & 15;
        if (CK && threadIdx.x < 128 && tp + TS * which < L) {
            const int64_t j = (tp + TS * which) / TS;
            reinterpret_cast<float4*>(ckpt)[((j * gridDim.y + b) * 4 + g) * D + cb * 16 + c16] =
                ck_s[buf][which][g][c16];
        }
    };
    float* ckl = reinterpret_cast<float*>(&ck_s[0][0][n >> 2][cw]) + (n & 3);
    constexpr int CKBUF = 2 * 4 * 16 * 4;  // floats per buffer
    auto stage_load = [&](int t1, Pair<T>& pbc, Quad<T>& pa) {
        pbc.load(sp + (int64_t)min(t1 + stok, L - 1) * NS);
        if (astage) pa.load(ap + (int64_t)min(t1 + atok, L - 1) * D);
    };
    // While the next tile is whole and the previous one was, each thread's rows
    // advance by one tile per step: running pointers instead of clamped 64-bit
    // row arithmetic.  spn/apn: this thread's rows of the tile after the
    // current one; yq: its output row of the previous tile; ckq: its
    // checkpoint piece of the previous tile.
    const T* spn = sp + (int64_t)(LT + stok) * NS;
    const T* apn = ap + (int64_t)(LT + atok) * D;
    T* yq = yrow + (int64_t)atok * D;
    float4* ckq = CK ? reinterpret_cast<float4*>(ckpt) +
                           (((int64_t)(threadIdx.x >> 6) * gridDim.y + b) * 4 + ((threadIdx.x >> 4) & 3)) * D +
                           cb * 16 + (threadIdx.x & 15)
                     : nullptr;
    const int64_t ckstep = (int64_t)(LT / TS) * gridDim.y * 4 * D;
    auto stage_store = [&](int buf, const Pair<T>& pbc, const Quad<T>& pa) {
        bc[buf][st][sn * LRS + stok] = pbc.lo();
        bc[buf][st][(sn + 1) * LRS + stok] = pbc.hi();
        if (astage) pa.store(&act_s[buf][aq][atok][a4]);
    };
    // rows of the previous tile's outputs, one 4-channel piece per thread
    auto store_y = [&](int buf, int tp) {
        if (threadIdx.x < 64 && tp + atok < L) {
            Quad<T> q;
            q.load(&y_s[buf][atok][a4]);
            q.store(yrow + (int64_t)(tp + atok) * D);
        }
    };
    {
        Pair<T> p0;
        Quad<T> a0;
        stage_load(0, p0, a0);
        stage_store(0, p0, a0);
    }
    __syncthreads();
    auto tile = [&](int k, auto full_c, auto next_full_c) {
        constexpr bool FULL = decltype(full_c)::value;
        constexpr bool NEXT_FULL = decltype(next_full_c)::value;
        const int t0 = k * LT;
        const int buf = k & 1;
        Pair<T> pbc;
        Quad<T> pa;
        if (NEXT_FULL) {  // the next tile's loads first
            pbc.load(spn);
            if (astage) pa.load(apn);
        } else {
            stage_load(t0 + LT, pbc, pa);
        }
        spn += LT * NS;
        apn += (int64_t)LT * D;
        __builtin_amdgcn_sched_barrier(0);
        float Bv[LT], Cv[LT];
        {
            const float4* pb = reinterpret_cast<const float4*>(&bc[buf][0][n * LRS]);
            const float4* pc = reinterpret_cast<const float4*>(&bc[buf][1][n * LRS]);
#pragma unroll
            for (int q = 0; q < LT / 4; ++q) {
                const float4 fb = pb[q], fc = pc[q];
                Bv[4 * q + 0] = fb.x; Bv[4 * q + 1] = fb.y; Bv[4 * q + 2] = fb.z; Bv[4 * q + 3] = fb.w;
                Cv[4 * q + 0] = fc.x; Cv[4 * q + 1] = fc.y; Cv[4 * q + 2] = fc.z; Cv[4 * q + 3] = fc.w;
            }
        }
        // this lane's token of the tile
        const float xv = to_f(act_s[buf][0][n][cw]);
        const float zv = GATE ? to_f(act_s[buf][2][n][cw]) : 0.0f;
        float sg;
        const float delta = softplus_sig(to_f(act_s[buf][1][n][cw]) + bias, sg);
        const float dxv = delta * xv;
        if (k > 0) {  // the previous tile is whole: all its rows and checkpoints exist
            if (threadIdx.x < 64) {
                Quad<T> q;
                q.load(&y_s[buf ^ 1][atok][a4]);
                q.store(yq);
            }
            if (CK && threadIdx.x < 128) {
                *ckq = ck_s[buf ^ 1][threadIdx.x >> 6][(threadIdx.x >> 4) & 3][threadIdx.x & 15];
                ckq += ckstep;
            }
            yq += (int64_t)LT * D;
        }
        float yp[LT];
        for_each_i([&](auto ic) {
            constexpr int I = decltype(ic)::value;
            if (FULL || t0 + I < L) {
                if (CK && (I % TS) == 0)  // state before token t0+I
                    ckl[buf * CKBUF + (I / TS) * 4 * 16 * 4] = h;
                const float a = __builtin_amdgcn_exp2f(dpp_f<0x150 + I>(delta) * A2);
                h = __builtin_fmaf(a, h, dpp_f<0x150 + I>(dxv) * Bv[I]);
                yp[I] = Cv[I] * h;
            } else {
                yp[I] = 0.0f;
            }
        }, std::make_integer_sequence<int, LT>{});
        // readout: butterfly over the row's 16 lanes.  Stage 1 pairs lane i with
        // i^8 (row_ror:8): lanes 0-7 (banks 0,1) keep tokens 0-7, lanes 8-15
        // (banks 2,3) tokens 8-15, each adding the partner's copy; stage 2 does
        // the same within each half with row_half_mirror (lane i with 7-i; banks
        // 0,2 keep the lower 4 slots).  A bank-masked DPP add writes only its
        // banks, so each stage is 2 instructions per pair, no selects.  The
        // s_nop covers the DPP read-after-VALU-write hazard inside the asm.
        {
            float o8[8];
#pragma unroll
            for (int j = 0; j < 8; ++j)
                asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_ror:8 row_mask:0xf bank_mask:0x3\n\t"
                    "v_add_f32_dpp %0, %2, %2 row_ror:8 row_mask:0xf bank_mask:0xc"
                    : "=&v"(o8[j]) : "v"(yp[j]), "v"(yp[j + 8]));
#pragma unroll
            for (int j = 0; j < 4; ++j)
                asm("s_nop 1\n\tv_add_f32_dpp %0, %1, %1 row_half_mirror row_mask:0xf bank_mask:0x5\n\t"
                    "v_add_f32_dpp %0, %2, %2 row_half_mirror row_mask:0xf bank_mask:0xa"
                    : "=&v"(yp[j]) : "v"(o8[j]), "v"(o8[j + 4]));
        }
        bfly<2, 0x4E>(yp, (n & 2) != 0);   // quad_perm [2,3,0,1]
        bfly<1, 0xB1>(yp, (n & 1) != 0);   // quad_perm [1,0,3,2]
        y_s[buf][n][cw] = from_f<T>(finish_y<GATE>(yp[0], Dd, xv, zv));
        __builtin_amdgcn_sched_barrier(0);  // the loads are first used here, a tile after their issue
        stage_store(buf ^ 1, pbc, pa);
        __syncthreads();
    };
    const int nfull = L / LT;
    for (int k = 0; k + 1 < nfull; ++k) tile(k, std::true_type{}, std::true_type{});
    if (nfull > 0) tile(nfull - 1, std::true_type{}, std::false_type{});
    if (nfull < ntile) tile(nfull, std::false_type{}, std::false_type{});
    store_y((ntile - 1) & 1, (ntile - 1) * LT);
    store_ck((ntile - 1) & 1, (ntile - 1) * LT);
    if (h_last) h_last[((int64_t)b * D + d) * NS + n] = h;
}

// ==================================================================== backward

// (1) zero-end adjoint G of chunk k (k = 1..K-1) and its delta sum:
//     walking the chunk backwards, lam <- (lam + C_t g_t) * exp(delta_t A).
template <typename T, bool GATE>
__global__ __launch_bounds__(WG) void k_bwd_chunk(
    const T* __restrict__ dt, const T* __restrict__ Cm, const T* __restrict__ z,
    const T* __restrict__ dy, const float* __restrict__ A_log, const float* __restrict__ dt_bias,
    float* __restrict__ wsG, float* __restrict__ wsSum, int L, int D, int Tc, int K) {
    const int d = blockIdx.x * WG + threadIdx.x;
    const int k = blockIdx.y + 1;
    const int b = blockIdx.z;
    const bool act = d < D;
    const int dc = act ? d : D - 1;
    float A2[NS];
    load_A2(A_log, dc, A2);
    const float bias = dt_bias ? dt_bias[dc] : 0.0f;
    float lam[NS];
#pragma unroll
    for (int n = 0; n < NS; ++n) lam[n] = 0.0f;
    float sumd = 0.0f;
    const int t0 = k * Tc, nt = min(Tc, L - t0);
    const int64_t row0 = (int64_t)b * L + t0;
    const Stream<T> ds{dt + row0 * D + dc, D}, gs{dy + row0 * D + dc, D};
    const Stream<T> zs{GATE ? z + row0 * D + dc : nullptr, D};
    const T* cp = Cm + row0 * NS;
    T dq[PF], gq[PF], zq[PF];
#pragma unroll
    for (int q = 0; q < PF; ++q) {
        dq[q] = ds.raw(max(nt - 1 - q, 0));
        gq[q] = gs.raw(max(nt - 1 - q, 0));
        zq[q] = GATE ? zs.raw(max(nt - 1 - q, 0)) : T(0);
    }
    float Cn[NS];
    load16(cp + (int64_t)(nt - 1) * NS, Cn);
#pragma unroll PF
    for (int i = nt - 1; i >= 0; --i) {
        const float dtv = to_f(dq[0]), dyv = to_f(gq[0]), zv = GATE ? to_f(zq[0]) : 0.0f;
#pragma unroll
        for (int q = 0; q + 1 < PF; ++q) {
            dq[q] = dq[q + 1];
            gq[q] = gq[q + 1];
            zq[q] = zq[q + 1];
        }
        dq[PF - 1] = ds.raw(max(i - PF, 0));
        gq[PF - 1] = gs.raw(max(i - PF, 0));
        if (GATE) zq[PF - 1] = zs.raw(max(i - PF, 0));
        const int ip = max(i - 1, 0);
        const float g = GATE ? dyv * (zv * sigmoid_f(zv)) : dyv;
        float Cv[NS];
#pragma unroll
        for (int n = 0; n < NS; ++n) Cv[n] = Cn[n];
        load16(cp + (int64_t)ip * NS, Cn);  // next token's row (scalar cache)
        float sg;
        const float delta = softplus_sig(dtv + bias, sg);
#pragma unroll
        for (int n = 0; n < NS; ++n) {
            const float a = __builtin_amdgcn_exp2f(delta * A2[n]);
            lam[n] = __builtin_fmaf(Cv[n], g, lam[n]) * a;
        }
        sumd += delta;
    }
    if (act) {
        const int64_t e = ((int64_t)b * (K - 1) + (k - 1)) * D + d;
        store_state(wsG + e * NS, lam);
        wsSum[e] = sumd;
    }
}

// (2) adjoint entering each chunk from the right: Xin(b, k) = dL/dh at the
//     chunk's last token from all later tokens; walks chunks in reverse.  One
//     lane per (batch, channel, state); the chunk adjoints and delta sums are
//     fetched CB chunks at a time.
__global__ __launch_bounds__(WG) void k_bwd_carry(
    const float* __restrict__ A_log, const float* __restrict__ wsG,
    const float* __restrict__ wsSum, float* __restrict__ Xin, int D, int K) {
    const int64_t DN = (int64_t)D * NS;
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;  // channel * NS + state
    const int b = blockIdx.z;
    if (i >= DN) return;
    const int64_t d = i / NS;
    const float A2 = a2_of(A_log, i);
    float X = 0.0f;
    const int64_t e0 = (int64_t)b * (K - 1) - 1;  // entry of chunk k is e0 + k (k >= 1)
    for (int k0 = K - 1; k0 > 0; k0 -= CB) {
        float Gb[CB], sb[CB];
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            if (k0 - j > 0) {
                Gb[j] = wsG[(e0 + k0 - j) * DN + i];
                sb[j] = wsSum[(e0 + k0 - j) * D + d];
            }
        }
#pragma unroll
        for (int j = 0; j < CB; ++j) {
            if (k0 - j > 0) {
                Xin[((int64_t)b * K + k0 - j) * DN + i] = X;
                const float P = __builtin_amdgcn_exp2f(A2 * sb[j]);
                X = __builtin_fmaf(P, X, Gb[j]);
            }
        }
    }
    Xin[(int64_t)b * K * DN + i] = X;
}

// (3) per chunk: adjoint sweep in reverse over blocks of TS tokens.  Each block
//     recomputes its TS states (and delta, sigmoid(u)) from the checkpoint,
//     then walks backwards:
//       lam  += C_t g_t                        (g_t = dy_t silu(z_t), lam = dL/dh_t)
//       dx    = delta sum_n lam B + D g        dB[t,n] = sum_d lam delta x
//       dC[t,n] = sum_d g h_t                   ddelta = sum_n lam (A a h_{t-1} + B x)
//       dA[n] += lam a h_{t-1} delta            lam <- lam a
//     dB/dC: each lane writes its 32 products to an LDS row; lane q of the
//     wave sums column (q mod 32) over half of the 64 rows; the 2 halves x 4
//     waves are summed after the block and written as one partial per
//     (token, workgroup).
//     Latency: at 2 waves per SIMD (the TS x NS states take most of the 256
//     VGPRs) little else hides a wait, so a block's x and dt are fetched
//     together with its checkpoint, B_t rows a token ahead of their use, C_t
//     rows touched during the recompute (the reverse sweep then finds them in
//     the scalar cache), dy and z two tokens ahead, and x kept in LDS for the
//     reverse sweep instead of being read again.
template <typename T, bool GATE>
__global__ __launch_bounds__(WG) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_bwd_main(
    const T* __restrict__ x, const T* __restrict__ dt, const T* __restrict__ Bm,
    const T* __restrict__ Cm, const T* __restrict__ z, const T* __restrict__ dy,
    const float* __restrict__ A_log, const float* __restrict__ Dp,
    const float* __restrict__ dt_bias, const float* __restrict__ ckpt,
    const float* __restrict__ Xin, T* __restrict__ dxo, T* __restrict__ ddto,
    T* __restrict__ dzo, float* __restrict__ dh0, float* __restrict__ wsBC,
    float* __restrict__ wsPA, float* __restrict__ wsPD, int L, int D, int Tc, int K,
    int ndb) {
    constexpr int RS = 36;  // LDS row stride in floats: 16-byte aligned rows
    static_assert(TS * 32 <= WG, "one dB/dC partial per thread at the block end");
    __shared__ float rows[NWAVE][64 * RS];
    __shared__ float wres[TS][2 * NWAVE][32];
    __shared__ float2 dsg[NWAVE][TS][64];  // per token: delta, sigmoid(dt + dt_bias)
    __shared__ float xsl[NWAVE][TS][64];   // per token: x
    const int d = blockIdx.x * WG + threadIdx.x;
    const int k = blockIdx.y;
    const int b = blockIdx.z;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool act = d < D;
    const int dc = act ? d : D - 1;
    float A2[NS];
    load_A2(A_log, dc, A2);
    const float bias = dt_bias ? dt_bias[dc] : 0.0f;
    const float Dd = Dp ? Dp[dc] : 0.0f;
    float lam[NS], dA[NS];
    if (Xin && act) load_state(Xin + (((int64_t)b * K + k) * D + d) * NS, lam);
    else {
#pragma unroll
        for (int n = 0; n < NS; ++n) lam[n] = 0.0f;
    }
#pragma unroll
    for (int n = 0; n < NS; ++n) dA[n] = 0.0f;
    float dDacc = 0.0f, ddtbacc = 0.0f;
    float* myrow = rows[wave] + lane * RS;
    const int col = lane & 31, half = lane >> 5;
    const float* colp = rows[wave] + (half * 32) * RS + col;
    const int t0 = k * Tc, t1 = min(t0 + Tc, L);
    const int j0 = t0 / TS, j1 = (t1 + TS - 1) / TS;
    // The outputs of a block's last-swept token (its first) and its dB/dC partial
    // are stored after the next block's first loads have been issued: the memory
    // counter is in order, so waiting for those loads would otherwise also wait
    // for these stores.
    T pdx = T(0), pddt = T(0), pdz = T(0);
    int64_t prow = -1, pbc_at = -1;
    float pbc = 0.0f;
    auto flush = [&]() {
        if (prow >= 0 && act) {
            __builtin_nontemporal_store(pdx, &dxo[prow * D + d]);
            __builtin_nontemporal_store(pddt, &ddto[prow * D + d]);
            if (GATE) __builtin_nontemporal_store(pdz, &dzo[prow * D + d]);
        }
        if (pbc_at >= 0) wsBC[pbc_at] = pbc;
        prow = -1;
        pbc_at = -1;
    };
    for (int j = j1 - 1; j >= j0; --j) {
        const int ts = j * TS;
        const int cnt = min(TS, t1 - ts);
        const int64_t row0 = (int64_t)b * L + ts;
        const float* ckp = ckpt + ((int64_t)j * gridDim.z + b) * NS * D;
        float hc[TS][NS];  // state after token ts+i
        // dy, z of the first RP tokens of the reverse sweep, fetched early
        constexpr int RP = 2;
        T gq[RP], zq[RP];
#pragma unroll
        for (int q = 0; q < RP; ++q) {
            const int64_t rl = (row0 + max(cnt - 1 - q, 0)) * D + dc;
            gq[q] = dy[rl];
            zq[q] = GATE ? z[rl] : T(0);
        }
        {
            float hs[NS];
            load_state_g4(ckp, D, dc, hs);
            T xr[TS], dr[TS];  // the block's x and dt, all fetched at once
#pragma unroll
            for (int i = 0; i < TS; ++i) {
                const int64_t rr = (row0 + min(i, cnt - 1)) * D + dc;
                xr[i] = x[rr];
                dr[i] = dt[rr];
            }
            flush();  // the previous block's deferred stores
            // B_t one token ahead; C_t touched one token ahead (its first word is
            // consumed a token later, so the load is kept but not waited for early)
            // so that the reverse sweep finds the row in the scalar cache.  The
            // next row is clamped into the block rather than skipped: a
            // conditional load would leave a copy that waits for it at once.
            RawRow<T> bn;
            bn.load(Bm + row0 * NS);
            uint32_t cw = *reinterpret_cast<const uint32_t*>(Cm + row0 * NS);
#pragma unroll
            for (int i = 0; i < TS; ++i) {
                if (i < cnt) {
                    const float xv = to_f(xr[i]), dtv = to_f(dr[i]);
                    float Bv[NS];
                    bn.get(Bv);
                    asm volatile("" ::"s"(cw));
                    {
                        const int64_t rn = row0 + min(i + 1, cnt - 1);  // in bounds
                        bn.load(Bm + rn * NS);
                        cw = *reinterpret_cast<const uint32_t*>(Cm + rn * NS);
                    }
                    float sg;
                    const float delta = softplus_sig(dtv + bias, sg);
                    dsg[wave][i][lane] = make_float2(delta, sg);
                    xsl[wave][i][lane] = xv;
                    const float dxv = delta * xv;
#pragma unroll
                    for (int n = 0; n < NS; ++n) {
                        const float a = __builtin_amdgcn_exp2f(delta * A2[n]);
                        hc[i][n] = __builtin_fmaf(a, i ? hc[i - 1][n] : hs[n], dxv * Bv[n]);
                    }
                }
            }
        }
        // dy and z of the token two ahead (earlier in time) are fetched before
        // this token's stores are issued: loads and stores retire in order, so a
        // load issued after a store would also wait for that store.  dy and z are
        // read once and dx, ddt, dz written once: non-temporal, so that this
        // streaming traffic does not push the block's checkpoint (read again at
        // its first token) out of L2.
#pragma unroll
        for (int i = TS - 1; i >= 0; --i) {
            if (i < cnt) {
                const int64_t row = row0 + i;
                const float xv = xsl[wave][i][lane];
                const float dyv = to_f(gq[0]);
                float zv = 0.0f, sz = 0.0f, g = dyv;
                if (GATE) zv = to_f(zq[0]);
#pragma unroll
                for (int q = 0; q + 1 < RP; ++q) {
                    gq[q] = gq[q + 1];
                    zq[q] = zq[q + 1];
                }
                if (i >= RP) {  // token i - RP, RP tokens ahead
                    const int64_t rp = (row - RP) * D + dc;
                    gq[RP - 1] = __builtin_nontemporal_load(&dy[rp]);
                    if (GATE) zq[RP - 1] = __builtin_nontemporal_load(&z[rp]);
                }
                if (GATE) {
                    sz = sigmoid_f(zv);
                    g = dyv * (zv * sz);
                }
                if (!act) g = 0.0f;
                float Bv[NS], Cv[NS];
                load16(Bm + row * NS, Bv);
                load16(Cm + row * NS, Cv);
                const float2 ds = dsg[wave][i][lane];
                const float delta = ds.x, sgu = ds.y;
                const float dxv = delta * xv;
                float hp[NS];
                if (i == 0) {
                    // the same rows again; an opaque zero keeps the compiler from
                    // holding the first load's addresses across the block
                    int64_t z0 = 0;
                    asm volatile("" : "+s"(z0));
                    load_state_g4(ckp + z0, D, dc, hp);
                }
                float s1 = 0.0f, s2 = 0.0f, yacc = 0.0f;
                float4* r4 = reinterpret_cast<float4*>(myrow);
#pragma unroll
                for (int q = 0; q < NS / 4; ++q) {
                    float pb[4], pc[4];
#pragma unroll
                    for (int m = 0; m < 4; ++m) {
                        const int n = 4 * q + m;
                        const float a = __builtin_amdgcn_exp2f(delta * A2[n]);
                        const float hprev = i ? hc[i - 1][n] : hp[n];
                        if (GATE) yacc = __builtin_fmaf(Cv[n], hc[i][n], yacc);
                        lam[n] = __builtin_fmaf(Cv[n], g, lam[n]);
                        s1 = __builtin_fmaf(lam[n], Bv[n], s1);
                        pb[m] = lam[n] * dxv;
                        pc[m] = g * hc[i][n];
                        const float lp = lam[n] * a;
                        const float gg = lp * hprev;
                        s2 = __builtin_fmaf(A2[n], gg, s2);
                        dA[n] = __builtin_fmaf(delta, gg, dA[n]);
                        lam[n] = lp;
                    }
                    r4[q] = make_float4(pb[0], pb[1], pb[2], pb[3]);
                    r4[4 + q] = make_float4(pc[0], pc[1], pc[2], pc[3]);
                }
                // dB / dC partial sums over this wave's 64 channels
                {
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    float sacc = 0.0f;
#pragma unroll
                    for (int r0 = 0; r0 < 32; r0 += 8) {  // 8 reads in flight, then the adds in row order
                        float cv[8];
#pragma unroll
                        for (int r = 0; r < 8; ++r) cv[r] = colp[(r0 + r) * RS];
#pragma unroll
                        for (int r = 0; r < 8; ++r) sacc += cv[r];
                    }
                    wres[i][2 * wave + half][col] = sacc;
                    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                    __builtin_amdgcn_wave_barrier();
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                }
                s2 *= LN2;  // A = A2 * ln 2
                const float dxv_out = __builtin_fmaf(delta, s1, Dd * g);
                const float ddelta = __builtin_fmaf(xv, s1, s2);
                const float ddtv = ddelta * sgu;
                float dzv = 0.0f;
                if (GATE) {
                    const float ypre = __builtin_fmaf(Dd, xv, yacc);
                    dzv = dyv * ypre * sz * (1.0f + zv * (1.0f - sz));
                }
                if (i == 0) {  // stored after the next block's first loads
                    pdx = from_f<T>(dxv_out);
                    pddt = from_f<T>(ddtv);
                    pdz = from_f<T>(dzv);
                    prow = row;
                } else if (act) {
                    __builtin_nontemporal_store(from_f<T>(dxv_out), &dxo[row * D + d]);
                    __builtin_nontemporal_store(from_f<T>(ddtv), &ddto[row * D + d]);
                    if (GATE) __builtin_nontemporal_store(from_f<T>(dzv), &dzo[row * D + d]);
                }
                if (act) {
                    dDacc = __builtin_fmaf(g, xv, dDacc);
                    ddtbacc += ddtv;
                }
            }
        }
        __syncthreads();
        if (threadIdx.x < cnt * 32) {  // one (token, value) per thread: cnt * 32 <= WG
            const int i = threadIdx.x >> 5, v = threadIdx.x & 31;
            float s = wres[i][0][v];
#pragma unroll
            for (int w = 1; w < 2 * NWAVE; ++w) s += wres[i][w][v];
            pbc = s;  // stored after the next block's first loads
            pbc_at = ((row0 + i) * ndb + blockIdx.x) * 32 + v;
        }
        __syncthreads();
    }
    flush();
    if (act) {
        const int64_t e = ((int64_t)b * K + k) * D + d;
        store_state(wsPA + e * NS, dA);
        wsPD[e * 2 + 0] = dDacc;
        wsPD[e * 2 + 1] = ddtbacc;
        if (dh0 && k == 0) store_state(dh0 + ((int64_t)b * D + d) * NS, lam);
    }
}

// dB/dC: fixed-order sum over channel blocks.  One thread per (b, t, value).
template <typename T>
__global__ __launch_bounds__(WG) void k_bwd_reduce_bc(const float* __restrict__ wsBC,
                                                      T* __restrict__ dB, T* __restrict__ dC,
                                                      int64_t rows, int ndb) {
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (i >= rows * 32) return;
    const int64_t row = i >> 5;
    const int v = (int)(i & 31);
    const float* p = wsBC + row * ndb * 32 + v;
    float s = 0.0f;
    for (int b0 = 0; b0 < ndb; b0 += CB) {  // CB loads in flight, then the adds in order
        float q[CB];
#pragma unroll
        for (int j = 0; j < CB; ++j)
            if (b0 + j < ndb) q[j] = p[(b0 + j) * 32];
#pragma unroll
        for (int j = 0; j < CB; ++j)
            if (b0 + j < ndb) s += q[j];
    }
    if (v < NS) dB[row * NS + v] = from_f<T>(s);
    else dC[row * NS + (v - NS)] = from_f<T>(s);
}

// dA_log = A * sum dA, dD, ddt_bias: fixed-order sums over the (batch, chunk)
// partials.  A workgroup takes RO outputs; its RG thread groups each sum a
// contiguous run of the partials in order, and the RG run sums are then added
// in run order (a fixed association, so the result is bitwise reproducible).
// Splitting the runs puts RG times as many loads in flight as one sequential
// sum per output, which at few outputs (small d_inner) was latency-bound.
constexpr int RO = 32, RG = WG / RO;
__global__ __launch_bounds__(WG) void k_bwd_reduce_params(
    const float* __restrict__ A_log, const float* __restrict__ wsPA,
    const float* __restrict__ wsPD, float* __restrict__ dA_log, float* __restrict__ dDo,
    float* __restrict__ ddt_bias, int Bt, int K, int D) {
    __shared__ float2 red[RG][RO];
    const int64_t DN = (int64_t)D * NS;
    const int o = threadIdx.x % RO, g = threadIdx.x / RO;
    const int64_t i = (int64_t)blockIdx.x * RO + o;  // dA outputs [0, DN), then (dD, ddt_bias) [DN, DN + D)
    const int64_t J = (int64_t)Bt * K;               // partials, in (batch, chunk) order
    const int64_t jb = J * g / RG, je = J * (g + 1) / RG;
    float s0 = 0.0f, s1 = 0.0f;
    if (i < DN) {
        for (int64_t j0 = jb; j0 < je; j0 += CB) {  // CB loads in flight, then the adds in order
            float v[CB];
#pragma unroll
            for (int j = 0; j < CB; ++j)
                if (j0 + j < je) v[j] = wsPA[(j0 + j) * DN + i];
#pragma unroll
            for (int j = 0; j < CB; ++j)
                if (j0 + j < je) s0 += v[j];
        }
    } else if (i < DN + D) {
        const int64_t d = i - DN;
        for (int64_t j0 = jb; j0 < je; j0 += CB) {
            float2 v[CB];
#pragma unroll
            for (int j = 0; j < CB; ++j)
                if (j0 + j < je) v[j] = reinterpret_cast<const float2*>(wsPD)[(j0 + j) * D + d];
#pragma unroll
            for (int j = 0; j < CB; ++j)
                if (j0 + j < je) {
                    s0 += v[j].x;
                    s1 += v[j].y;
                }
        }
    }
    red[g][o] = make_float2(s0, s1);
    __syncthreads();
    if (g == 0) {
        float2 t = red[0][o];
#pragma unroll
        for (int r = 1; r < RG; ++r) {
            t.x += red[r][o].x;
            t.y += red[r][o].y;
        }
        if (i < DN) {
            dA_log[i] = t.x * -expf(A_log[i]);
        } else if (i < DN + D) {
            const int64_t d = i - DN;
            if (dDo) dDo[d] = t.x;
            ddt_bias[d] = t.y;
        }
    }
}

// ======================================================================= step
// One token for 256 channels of SR consecutive batch rows.  Each wave's 64
// channels hold 4 KB of contiguous state per row; it is moved between memory and
// registers through LDS so that every global load/store instruction covers 1 KB
// contiguously.  A wave walks its rows in turn: the decay rates are formed once
// for all of them, and the next row's state and activations are loaded while
// the current row is computed.
template <typename T, bool GATE>
__global__ __launch_bounds__(WG) void k_step(
    float* __restrict__ h, const T* __restrict__ x, const T* __restrict__ dt,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const T* __restrict__ z,
    const float* __restrict__ A_log, const float* __restrict__ Dp,
    const float* __restrict__ dt_bias, T* __restrict__ y, int D, int Bt, int SR) {
    constexpr int HS = NS + 4;  // padded LDS row (16-byte aligned, conflict-free)
    __shared__ float hsm[NWAVE][64 * HS];
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int d0 = blockIdx.x * WG + wave * 64;
    const int nvalid = min(64, D - d0);  // channels of this wave (uniform)
    if (nvalid <= 0) return;             // no block-wide barriers below
    const int b0 = blockIdx.z * SR, b1 = min(b0 + SR, Bt);
    const int d = d0 + lane;
    const bool act = lane < nvalid;
    const int dc = act ? d : d0;
    float* sm = hsm[wave];
    float A2[NS];
    load_A2(A_log, dc, A2);
    const float bias = dt_bias ? dt_bias[dc] : 0.0f;
    const float Dd = Dp ? Dp[dc] : 0.0f;
    // a row's state as 16-byte pieces (piece pc: channel pc/4, states 4*(pc%4)..)
    // and its activations
    float4 raw[4];
    T xr, dr, zr = T(0);
    auto fetch = [&](int b) {
        const float4* hb = reinterpret_cast<const float4*>(h + ((int64_t)b * D + d0) * NS);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pc = j * 64 + lane;
            raw[j] = (pc >> 2) < nvalid ? hb[pc] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        const int64_t i = (int64_t)b * D + dc;
        xr = x[i];
        dr = dt[i];
        if (GATE) zr = z[i];
    };
    fetch(b0);
    for (int b = b0; b < b1; ++b) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pc = j * 64 + lane;
            if ((pc >> 2) < nvalid) *reinterpret_cast<float4*>(sm + (pc >> 2) * HS + (pc & 3) * 4) = raw[j];
        }
        const float xv = to_f(xr), dtv = to_f(dr);
        const float zv = GATE ? to_f(zr) : 0.0f;
        float Bv[NS], Cv[NS];
        load16(Bm + (int64_t)b * NS, Bv);
        load16(Cm + (int64_t)b * NS, Cv);
        if (b + 1 < b1) fetch(b + 1);  // the next row, while this one is computed
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float hs[NS];
        load_state(sm + (act ? lane : 0) * HS, hs);
        float sg;
        const float delta = softplus_sig(dtv + bias, sg);
        const float acc = scan_token(hs, A2, Bv, Cv, delta, xv);
        const int64_t i = (int64_t)b * D + dc;
        if (act) {
            y[i] = from_f<T>(finish_y<GATE>(acc, Dd, xv, zv));
            store_state(sm + lane * HS, hs);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        float4* hb = reinterpret_cast<float4*>(h + ((int64_t)b * D + d0) * NS);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int pc = j * 64 + lane;
            if ((pc >> 2) < nvalid) hb[pc] = *reinterpret_cast<const float4*>(sm + (pc >> 2) * HS + (pc & 3) * 4);
        }
    }
}

// Fills used when seqlen == 0: dst[i] = src ? src[i] : 0.
__global__ __launch_bounds__(WG) void k_fill(float* __restrict__ dst, const float* __restrict__ src,
                                             int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

// ================================================================ host side

struct Plan {
    int64_t Bt, L, D;
    int io;
    int64_t Tf, Kf;  // forward chunk length / count
    int64_t Tb, Kb;  // backward chunk length / count
    int64_t nck, ndb;
    bool state_lanes;       // forward without checkpoints by k_fwd_state (one lane per channel and state)
    bool state_lanes_ckpt;  // the same with checkpoints (then Kf = 1: no forward workspace)
};

ssm_status check_dims(const ssm_dims* d) {
    if (!d) return SSM_E_NULLPTR;
    if (d->batch < 1 || d->seqlen < 0 || d->d_inner < 1 || d->d_state < 1) return SSM_E_SHAPE;
    if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_E_DTYPE;
    if (d->d_state != NS) return SSM_E_UNSUPPORTED;
    if (d->batch > 65535) return SSM_E_UNSUPPORTED;
    // kernels index tokens and channels with 32-bit ints
    if (d->seqlen > (int64_t)1 << 30 || d->d_inner > (int64_t)1 << 30) return SSM_E_UNSUPPORTED;
    return SSM_OK;
}

// Chunk length (a multiple of TS) for a kernel launched as one workgroup per
// (channel block, chunk, batch row), `wg_per_chunk` workgroups per chunk, with
// `slots` workgroups resident on the chip at once.  Picks the chunk count that
// fills whole rounds of resident workgroups best (the last round of a launch
// otherwise runs partly empty), among counts that fill the chip at least once;
// ties go to fewer chunks.  Tiny problems take as many chunks as allowed.
int64_t pick_chunk(int64_t L, int64_t wg_per_chunk, int64_t slots, int64_t min_chunk = MIN_CHUNK) {
    if (L < 1) return TS;  // empty sequence: one (empty) chunk
    const int64_t kmax = std::max<int64_t>(1, std::min<int64_t>(L / min_chunk, 4096));
    int64_t best_tc = -1;
    double best_eff = -1.0;
    int64_t prev_k = -1;
    for (int64_t kt = 1; kt <= kmax; ++kt) {
        int64_t tc = (L + kt - 1) / kt;
        tc = (tc + TS - 1) / TS * TS;
        const int64_t k = (L + tc - 1) / tc;
        if (k == prev_k) continue;
        prev_k = k;
        const int64_t w = wg_per_chunk * k;
        if (w < slots && kt < kmax) continue;
        const int64_t rounds = (w + slots - 1) / slots;
        const double eff = (double)w / (double)(rounds * slots);
        if (eff > best_eff + 1e-9) {
            best_eff = eff;
            best_tc = tc;
        }
    }
    if (best_tc < 0) best_tc = (L + TS - 1) / TS * TS;
    return std::max<int64_t>(best_tc, TS);
}

Plan make_plan(const ssm_dims* d) {
    Plan p;
    p.Bt = d->batch;
    p.L = d->seqlen;
    p.D = d->d_inner;
    p.io = d->io_dtype;
    p.nck = (p.L + TS - 1) / TS;
    p.ndb = (p.D + WG - 1) / WG;
    const int64_t Lp = std::max<int64_t>(p.L, 1);
    // Forward: one lane per state (k_fwd_state) at the widths and lengths above;
    // else one chunk (a purely sequential scan, same operation order as the
    // single-token step) when the channels alone fill the chip or the sequence
    // is short; else chunks.  Backward: chunks sized to fill the resident slots;
    // with few workgroups per chunk, chunks down to one 8-token block, so that
    // short sequences are not walked by a handful of waves one token at a time.
    p.state_lanes = p.Bt * p.D < TARGET_LANES && p.Bt <= 65535 && p.D % 16 == 0 &&
                    (p.Bt * p.D >= STATE_LANES_MIN || p.L <= STATE_LANES_SHORT_L);
    p.state_lanes_ckpt = p.state_lanes && p.L < STATE_LANES_CKPT_L;
    if (p.state_lanes_ckpt || p.Bt * p.D >= TARGET_LANES || p.L < 2 * MIN_CHUNK) p.Tf = (Lp + TS - 1) / TS * TS;
    else p.Tf = pick_chunk(p.L, p.Bt * p.ndb, FWD_SLOTS);
    p.Kf = (Lp + p.Tf - 1) / p.Tf;
    if (p.Bt * p.ndb * 8 <= BWD_SLOTS && p.L >= 2 * TS)  // few workgroups per chunk: chunks down to 8 tokens
        p.Tb = pick_chunk(p.L, p.Bt * p.ndb, BWD_SLOTS, TS);
    else
        p.Tb = p.L < 2 * MIN_CHUNK ? (Lp + TS - 1) / TS * TS : pick_chunk(p.L, p.Bt * p.ndb, BWD_SLOTS);
    p.Kb = (Lp + p.Tb - 1) / p.Tb;
    return p;
}

size_t align_up(size_t v) { return (v + 255) & ~(size_t)255; }

struct FwdWs {
    size_t S, sum, starts, total;
};
FwdWs fwd_ws(const Plan& p) {
    FwdWs w{0, 0, 0, 0};
    if (p.Kf > 1) {
        w.S = 0;
        w.sum = w.S + align_up(sizeof(float) * p.Bt * (p.Kf - 1) * p.D * NS);
        w.starts = w.sum + align_up(sizeof(float) * p.Bt * (p.Kf - 1) * p.D);
        w.total = w.starts + align_up(sizeof(float) * p.Bt * p.Kf * p.D * NS);
    }
    return w;
}

struct BwdWs {
    size_t G, sum, X, BC, PA, PD, total;
};
BwdWs bwd_ws(const Plan& p) {
    BwdWs w{};
    size_t off = 0;
    if (p.Kb > 1) {
        w.G = off; off += align_up(sizeof(float) * p.Bt * (p.Kb - 1) * p.D * NS);
        w.sum = off; off += align_up(sizeof(float) * p.Bt * (p.Kb - 1) * p.D);
        w.X = off; off += align_up(sizeof(float) * p.Bt * p.Kb * p.D * NS);
    }
    w.BC = off; off += align_up(sizeof(float) * p.Bt * p.L * p.ndb * 32);
    w.PA = off; off += align_up(sizeof(float) * p.Bt * p.Kb * p.D * NS);
    w.PD = off; off += align_up(sizeof(float) * p.Bt * p.Kb * p.D * 2);
    w.total = off;
    return w;
}

// Every scan kernel runs 256-thread workgroups.
struct Launcher {
    ssm::Launcher l;
    template <typename Kern, typename... Args>
    ssm_status operator()(int kid, Kern kern, dim3 grid, Args... args) {
        return l(kid, kern, grid, dim3(WG), args...);
    }
};

template <typename T, bool GATE>
ssm_status run_fwd(const Plan& p, const void* x, const void* dt, const void* B, const void* C,
                   const void* z, const float* A_log, const float* Dp, const float* dt_bias,
                   const float* h0, void* y, float* h_last, float* ckpt, void* ws,
                   Launcher& launch) {
    const FwdWs w = fwd_ws(p);
    char* wsb = static_cast<char*>(ws);
    float* S = p.Kf > 1 ? reinterpret_cast<float*>(wsb + w.S) : nullptr;
    float* sum = p.Kf > 1 ? reinterpret_cast<float*>(wsb + w.sum) : nullptr;
    float* starts;
    int64_t sb, sk;  // entry of chunk k of batch row b: b * sb + k * sk
    if (ckpt) {          // chunk starts are checkpoints: [L/8, batch, ...]
        starts = ckpt;
        sb = 1;
        sk = p.Tf / TS * p.Bt;
    } else {
        starts = p.Kf > 1 ? reinterpret_cast<float*>(wsb + w.starts) : nullptr;
        sb = p.Kf;
        sk = 1;
    }
    const int L = (int)p.L, D = (int)p.D, Tc = (int)p.Tf, K = (int)p.Kf;
    if (ckpt ? p.state_lanes_ckpt : p.state_lanes) {
        const int ncb = D / 16;
        const dim3 grid((unsigned)((ncb + 31) / 32 * 32), (unsigned)p.Bt);
        if (ckpt)
            return launch(SSM_K_FWD_STATE, k_fwd_state<T, GATE, true>, grid, (const T*)x, (const T*)dt,
                          (const T*)B, (const T*)C, (const T*)z, A_log, Dp, dt_bias, h0, (T*)y, h_last,
                          ckpt, L, D, ncb);
        return launch(SSM_K_FWD_STATE, k_fwd_state<T, GATE, false>, grid, (const T*)x, (const T*)dt,
                      (const T*)B, (const T*)C, (const T*)z, A_log, Dp, dt_bias, h0, (T*)y, h_last, ckpt,
                      L, D, ncb);
    }
    if (p.Kf > 1) {
        SSM_TRY(launch(SSM_K_FWD_CHUNK, k_fwd_chunk<T>, dim3(p.ndb, p.Kf - 1, p.Bt),
                       (const T*)x, (const T*)dt, (const T*)B, A_log, dt_bias, S, sum, L, D, Tc, K));
        SSM_TRY(launch(SSM_K_FWD_CARRY, k_fwd_carry, dim3((unsigned)((p.D * NS + WG - 1) / WG), 1, p.Bt), A_log, h0,
                       (const float*)S, (const float*)sum, starts, D, K, sb, sk));
    }
    return launch(SSM_K_FWD_MAIN, k_fwd_main<T, GATE>, dim3(p.ndb, p.Kf, p.Bt), (const T*)x,
                  (const T*)dt, (const T*)B, (const T*)C, (const T*)z, A_log, Dp, dt_bias, h0,
                  (const float*)starts, (T*)y, h_last, ckpt, L, D, Tc, K, sb, sk);
}

template <typename T, bool GATE>
ssm_status run_bwd(const Plan& p, const void* x, const void* dt, const void* B, const void* C,
                   const void* z, const float* A_log, const float* Dp, const float* dt_bias,
                   const float* ckpt, const void* dy, void* dx, void* ddt, void* dB, void* dC,
                   void* dz, float* dA_log, float* dD, float* ddt_bias, float* dh0, void* ws,
                   Launcher& launch) {
    const BwdWs w = bwd_ws(p);
    char* wsb = static_cast<char*>(ws);
    float* G = p.Kb > 1 ? reinterpret_cast<float*>(wsb + w.G) : nullptr;
    float* sum = p.Kb > 1 ? reinterpret_cast<float*>(wsb + w.sum) : nullptr;
    float* X = p.Kb > 1 ? reinterpret_cast<float*>(wsb + w.X) : nullptr;
    float* BC = reinterpret_cast<float*>(wsb + w.BC);
    float* PA = reinterpret_cast<float*>(wsb + w.PA);
    float* PD = reinterpret_cast<float*>(wsb + w.PD);
    const int L = (int)p.L, D = (int)p.D, Tc = (int)p.Tb, K = (int)p.Kb;
    if (p.Kb > 1) {
        SSM_TRY(launch(SSM_K_BWD_CHUNK, k_bwd_chunk<T, GATE>, dim3(p.ndb, p.Kb - 1, p.Bt),
                       (const T*)dt, (const T*)C, (const T*)z, (const T*)dy, A_log, dt_bias, G,
                       sum, L, D, Tc, K));
        SSM_TRY(launch(SSM_K_BWD_CARRY, k_bwd_carry, dim3((unsigned)((p.D * NS + WG - 1) / WG), 1, p.Bt), A_log,
                       (const float*)G, (const float*)sum, X, D, K));
    }
    SSM_TRY(launch(SSM_K_BWD_MAIN, k_bwd_main<T, GATE>, dim3(p.ndb, p.Kb, p.Bt), (const T*)x,
                   (const T*)dt, (const T*)B, (const T*)C, (const T*)z, (const T*)dy, A_log, Dp,
                   dt_bias, ckpt, (const float*)X, (T*)dx, (T*)ddt, (T*)dz, dh0, BC, PA, PD, L,
                   D, Tc, K, (int)p.ndb));
    const int64_t rows = p.Bt * p.L;
    SSM_TRY(launch(SSM_K_BWD_REDUCE_BC, k_bwd_reduce_bc<T>, dim3((unsigned)((rows * 32 + WG - 1) / WG)),
                   (const float*)BC, (T*)dB, (T*)dC, rows, (int)p.ndb));
    const int64_t np = p.D * NS + p.D;
    return launch(SSM_K_BWD_REDUCE_P, k_bwd_reduce_params, dim3((unsigned)((np + RO - 1) / RO)),
                  A_log, (const float*)PA, (const float*)PD, dA_log, dD, ddt_bias, (int)p.Bt,
                  (int)p.Kb, D);
}

}  // namespace

// ===================================================================== C ABI
extern "C" {

const char* ssm_status_str(int32_t status) {
    switch (status) {
        case SSM_OK: return "ok";
        case SSM_E_NULLPTR: return "required pointer is NULL";
        case SSM_E_SHAPE: return "dimension out of range";
        case SSM_E_DTYPE: return "unknown io dtype";
        case SSM_E_ALIGN: return "pointer not 16-byte aligned";
        case SSM_E_WORKSPACE: return "workspace too small";
        case SSM_E_LAUNCH: return "kernel launch failed";
        case SSM_E_UNSUPPORTED:
            return "unsupported configuration (outside the limits its header states: e.g. d_state 16, "
                   "d_conv 1..4, batch <= 65535, GDN2 k_dim 16/32/64/128)";
    }
    return "unknown status";
}

const char* ssm_kernel_name(int32_t id) {
    switch (id) {
        case SSM_K_FWD_CHUNK: return "k_fwd_chunk";
        case SSM_K_FWD_CARRY: return "k_fwd_carry";
        case SSM_K_FWD_MAIN: return "k_fwd_main";
        case SSM_K_FWD_STATE: return "k_fwd_state";
        case SSM_K_BWD_CHUNK: return "k_bwd_chunk";
        case SSM_K_BWD_CARRY: return "k_bwd_carry";
        case SSM_K_BWD_MAIN: return "k_bwd_main";
        case SSM_K_BWD_REDUCE_BC: return "k_bwd_reduce_bc";
        case SSM_K_BWD_REDUCE_P: return "k_bwd_reduce_params";
        case SSM_K_STEP: return "k_step";
        case SSM_K_FILL: return "k_fill";
        case SSM_K_CONV_FWD: return "k_conv_fwd";
        case SSM_K_CONV_BWD: return "k_conv_bwd";
        case SSM_K_CONV_BWD_REDUCE: return "k_conv_bwd_reduce";
        case SSM_K_CONV_STEP: return "k_conv_step";
        case SSM_K_CONV_RING: return "k_conv_ring";
        case SSM_K_BLOCK_BC: return "k_block_bc";
        case SSM_K_GDN2_FWD: return "k_gdn2_fwd";
        case SSM_K_GDN2_WY: return "k_gdn2_wy";
        case SSM_K_GDN2_STATE: return "k_gdn2_state";
        case SSM_K_BLOCK_GEMM: return "block_gemm";
        case SSM_K_BLOCK_SUM: return "k_sum_parts";
    }
    return "?";
}

size_t ssm_scan_ckpt_bytes(const ssm_dims* dims) {
    if (check_dims(dims) != SSM_OK) return 0;
    const Plan p = make_plan(dims);
    return sizeof(float) * (size_t)(p.Bt * p.nck * p.D * NS);
}

size_t ssm_scan_fwd_workspace_bytes(const ssm_dims* dims) {
    if (check_dims(dims) != SSM_OK) return 0;
    return fwd_ws(make_plan(dims)).total;
}

size_t ssm_scan_bwd_workspace_bytes(const ssm_dims* dims) {
    if (check_dims(dims) != SSM_OK) return 0;
    const Plan p = make_plan(dims);
    if (p.L == 0) return 0;
    return bwd_ws(p).total;
}

ssm_status ssm_scan_fwd(const ssm_dims* dims, const void* x, const void* dt, const void* B,
                        const void* C, const void* z, const float* A_log, const float* D,
                        const float* dt_bias, const float* h0, void* y, float* h_last,
                        float* ckpt, void* ws, size_t ws_bytes, hipStream_t stream,
                        ssm_timing* timing) {
    SSM_TRY(check_dims(dims));
    const Plan p = make_plan(dims);
    if (!A_log) return SSM_E_NULLPTR;
    if (p.L > 0 && (!x || !dt || !B || !C || !y)) return SSM_E_NULLPTR;
    const void* ptrs[] = {x, dt, B, C, z, A_log, D, dt_bias, h0, y, h_last, ckpt, ws};
    for (const void* q : ptrs)
        if (q && misaligned(q)) return SSM_E_ALIGN;
    const size_t need = fwd_ws(p).total;
    if (p.L > 0 && need > 0 && (!ws || ws_bytes < need)) return SSM_E_WORKSPACE;
    (void)hipGetLastError();
    Launcher launch{{stream, timing}};
    if (p.L == 0) {
        if (!h_last) return SSM_OK;
        const int64_t n = p.Bt * p.D * NS;
        return launch(SSM_K_FILL, k_fill, dim3((unsigned)((n + WG - 1) / WG)), h_last, h0, n);
    }
    const bool gate = z != nullptr;
    if (p.io == SSM_F32) {
        return gate ? run_fwd<float, true>(p, x, dt, B, C, z, A_log, D, dt_bias, h0, y, h_last, ckpt, ws, launch)
                    : run_fwd<float, false>(p, x, dt, B, C, z, A_log, D, dt_bias, h0, y, h_last, ckpt, ws, launch);
    }
    return gate ? run_fwd<bf16_t, true>(p, x, dt, B, C, z, A_log, D, dt_bias, h0, y, h_last, ckpt, ws, launch)
                : run_fwd<bf16_t, false>(p, x, dt, B, C, z, A_log, D, dt_bias, h0, y, h_last, ckpt, ws, launch);
}

ssm_status ssm_scan_bwd(const ssm_dims* dims, const void* x, const void* dt, const void* B,
                        const void* C, const void* z, const float* A_log, const float* D,
                        const float* dt_bias, const float* h0, const float* ckpt,
                        const void* dy, void* dx, void* ddt, void* dB, void* dC, void* dz,
                        float* dA_log, float* dD, float* ddt_bias, float* dh0, void* ws,
                        size_t ws_bytes, hipStream_t stream, ssm_timing* timing) {
    (void)h0;  // the checkpoints already hold h0 (entry 0)
    SSM_TRY(check_dims(dims));
    const Plan p = make_plan(dims);
    if (!A_log || !dA_log || !ddt_bias || (D && !dD)) return SSM_E_NULLPTR;
    if (p.L > 0 && (!x || !dt || !B || !C || !ckpt || !dy || !dx || !ddt || !dB || !dC))
        return SSM_E_NULLPTR;
    if (p.L > 0 && z && !dz) return SSM_E_NULLPTR;
    const void* ptrs[] = {x, dt, B, C, z, A_log, D, dt_bias, h0, ckpt, dy, dx, ddt, dB, dC, dz,
                          dA_log, dD, ddt_bias, dh0, ws};
    for (const void* q : ptrs)
        if (q && misaligned(q)) return SSM_E_ALIGN;
    const size_t need = p.L > 0 ? bwd_ws(p).total : 0;
    if (need > 0 && (!ws || ws_bytes < need)) return SSM_E_WORKSPACE;
    (void)hipGetLastError();
    Launcher launch{{stream, timing}};
    if (p.L == 0) {
        const int64_t np = p.D * NS;
        SSM_TRY(launch(SSM_K_FILL, k_fill, dim3((unsigned)((np + WG - 1) / WG)), dA_log,
                       (const float*)nullptr, np));
        SSM_TRY(launch(SSM_K_FILL, k_fill, dim3((unsigned)((p.D + WG - 1) / WG)), ddt_bias,
                       (const float*)nullptr, p.D));
        if (dD)
            SSM_TRY(launch(SSM_K_FILL, k_fill, dim3((unsigned)((p.D + WG - 1) / WG)), dD,
                           (const float*)nullptr, p.D));
        if (dh0) {
            const int64_t n = p.Bt * p.D * NS;
            SSM_TRY(launch(SSM_K_FILL, k_fill, dim3((unsigned)((n + WG - 1) / WG)), dh0,
                           (const float*)nullptr, n));
        }
        return SSM_OK;
    }
    const bool gate = z != nullptr;
    if (p.io == SSM_F32) {
        return gate ? run_bwd<float, true>(p, x, dt, B, C, z, A_log, D, dt_bias, ckpt, dy, dx, ddt, dB, dC, dz, dA_log, dD, ddt_bias, dh0, ws, launch)
                    : run_bwd<float, false>(p, x, dt, B, C, z, A_log, D, dt_bias, ckpt, dy, dx, ddt, dB, dC, dz, dA_log, dD, ddt_bias, dh0, ws, launch);
    }
    return gate ? run_bwd<bf16_t, true>(p, x, dt, B, C, z, A_log, D, dt_bias, ckpt, dy, dx, ddt, dB, dC, dz, dA_log, dD, ddt_bias, dh0, ws, launch)
                : run_bwd<bf16_t, false>(p, x, dt, B, C, z, A_log, D, dt_bias, ckpt, dy, dx, ddt, dB, dC, dz, dA_log, dD, ddt_bias, dh0, ws, launch);
}

ssm_status ssm_scan_step(int64_t batch, int64_t d_inner, int64_t d_state, int32_t io_dtype,
                         float* h, const void* x, const void* dt, const void* B, const void* C,
                         const void* z, const float* A_log, const float* D,
                         const float* dt_bias, void* y, hipStream_t stream, ssm_timing* timing) {
    ssm_dims dims{batch, 1, d_inner, d_state, io_dtype};
    SSM_TRY(check_dims(&dims));
    if (!h || !x || !dt || !B || !C || !A_log || !y) return SSM_E_NULLPTR;
    const void* ptrs[] = {h, x, dt, B, C, z, A_log, D, dt_bias, y};
    for (const void* q : ptrs)
        if (q && misaligned(q)) return SSM_E_ALIGN;
    (void)hipGetLastError();
    Launcher launch{{stream, timing}};
    // batch rows per wave: up to 4, as many as still leave >= 4096 waves (4 per SIMD)
    const int64_t ndb = (d_inner + WG - 1) / WG;
    int SR = 1;
    while (SR < 4 && ndb * NWAVE * ((batch + 2 * SR - 1) / (2 * SR)) >= 4096) SR *= 2;
    const dim3 grid((unsigned)ndb, 1, (unsigned)((batch + SR - 1) / SR));
    const int Dn = (int)d_inner, Bn = (int)batch;
    if (io_dtype == SSM_F32) {
        return z ? launch(SSM_K_STEP, k_step<float, true>, grid, h, (const float*)x, (const float*)dt, (const float*)B, (const float*)C, (const float*)z, A_log, D, dt_bias, (float*)y, Dn, Bn, SR)
                 : launch(SSM_K_STEP, k_step<float, false>, grid, h, (const float*)x, (const float*)dt, (const float*)B, (const float*)C, (const float*)z, A_log, D, dt_bias, (float*)y, Dn, Bn, SR);
    }
    return z ? launch(SSM_K_STEP, k_step<bf16_t, true>, grid, h, (const bf16_t*)x, (const bf16_t*)dt, (const bf16_t*)B, (const bf16_t*)C, (const bf16_t*)z, A_log, D, dt_bias, (bf16_t*)y, Dn, Bn, SR)
             : launch(SSM_K_STEP, k_step<bf16_t, false>, grid, h, (const bf16_t*)x, (const bf16_t*)dt, (const bf16_t*)B, (const bf16_t*)C, (const bf16_t*)z, A_log, D, dt_bias, (bf16_t*)y, Dn, Bn, SR);
}

}  // extern "C"
