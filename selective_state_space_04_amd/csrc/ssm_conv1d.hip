// ssm_conv1d.hip -- causal depthwise conv1d + SiLU in front of the selective scan,
// for MI355X (gfx950, CDNA4, wave64).
//
// Operation (rustytorch commit log, page "crates/training/rtx-transformers/tests":
// the real-S6-forward commit runs a causal depthwise conv1d then SiLU before
// x_proj; the VJP commit returns conv1d_weight / conv1d_bias gradients;
// MambaRecurrence::step carries a conv ring), read as PyTorch's
// Conv1d(groups=d_inner, padding=K-1) truncated to the first L outputs:
//   pre[b,t,d] = bias[d] + sum_k w[d,k] * v[b, t-(K-1)+k, d],   y = silu(pre)
// with v = x at t >= 0 and the caller's ring of the K-1 previous inputs before.
//
// Mapping to the hardware.  The operation is a K-tap stencil along time with no
// reuse across channels: HBM-bound, a few flops per byte.
//   * A lane owns VEC = 4 consecutive channels (8 or 16 contiguous bytes per
//     token), so a wave reads 64 * VEC channels of one token as one coalesced
//     512 B / 1 KB row; rows whose d_inner is not a multiple of 4 use VEC = 1.
//   * A wave streams a run of TT = 64 tokens with a sliding window of the last
//     K inputs in registers, PF = 4 tokens of loads in flight; the 4 waves of a
//     workgroup take 4 consecutive runs, so the K-1 token halo a run re-reads
//     was just read by its neighbour (L2 hit).
//   * Backward: g = dy * silu'(pre) needs the forward's pre, recomputed from the
//     window; dx[t] = sum_k w[k] g[t+K-1-k] needs g K-1 tokens ahead, so a run
//     computes g over TT + K - 1 tokens.  dw/dbias are summed per lane over the
//     run, across the 4 waves through LDS, and across workgroups by a
//     fixed-order kernel: deterministic, no atomics.
//   * The step shares the forward's per-token arithmetic (bias first, taps in
//     increasing k, explicit FMAs), so stepping reproduces the forward exactly.
#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "ssm_common.h"
#include "ssm_conv1d.h"

namespace {

using ssm::bf16_t;
using ssm::from_f;
using ssm::misaligned;
using ssm::to_f;

constexpr int WG = 256;  // 64 lanes (channel groups) x 4 waves (token runs)
constexpr int NWAVE = WG / 64;
constexpr int TT = 64;   // tokens per wave
constexpr int PF = 4;    // tokens fetched ahead
constexpr int KMAX = 4;
// A run is whole groups of PF tokens (but a sequence's ragged last run), and a
// group holds the K-1 token look-ahead and a token more.
static_assert(TT % PF == 0 && PF >= KMAX, "token run must split into groups of PF >= KMAX");

// ---------------------------------------------------------------- VEC channels
template <typename T, int VEC> struct Raw;
template <> struct Raw<float, 4> { typedef float4 type; };
template <> struct Raw<bf16_t, 4> { typedef uint2 type; };
template <> struct Raw<float, 1> { typedef float type; };
template <> struct Raw<bf16_t, 1> { typedef bf16_t type; };

template <typename T, int VEC>
__device__ __forceinline__ typename Raw<T, VEC>::type ld(const T* p) {
    return *reinterpret_cast<const typename Raw<T, VEC>::type*>(p);
}

// Streaming access to the token rows.  Every row of x and dy is read once (but
// the K-1 token halo a neighbouring run re-reads) and every row of y and dx is
// written once, so these loads and stores are non-temporal: they do not
// displace lines that other data would reuse from the caches.
__device__ __forceinline__ uint2 ld_stream(const uint2* p) {
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ float4 ld_stream(const float4* p) {
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    const f32x4 v = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float ld_stream(const float* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ bf16_t ld_stream(const bf16_t* p) { return *p; }
template <typename T, int VEC>
__device__ __forceinline__ typename Raw<T, VEC>::type ld_nt(const T* p) {
    return ld_stream(reinterpret_cast<const typename Raw<T, VEC>::type*>(p));
}

__device__ __forceinline__ void unpack(float4 r, float v[4]) {
    v[0] = r.x; v[1] = r.y; v[2] = r.z; v[3] = r.w;
}
__device__ __forceinline__ void unpack(uint2 r, float v[4]) {
    v[0] = __uint_as_float(r.x << 16);
    v[1] = __uint_as_float(r.x & 0xffff0000u);
    v[2] = __uint_as_float(r.y << 16);
    v[3] = __uint_as_float(r.y & 0xffff0000u);
}
__device__ __forceinline__ void unpack(float r, float v[1]) { v[0] = r; }
__device__ __forceinline__ void unpack(bf16_t r, float v[1]) { v[0] = to_f(r); }

template <typename T, int VEC> __device__ __forceinline__ void st(T* p, const float v[VEC]);
template <> __device__ __forceinline__ void st<float, 4>(float* p, const float v[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
// two floats to two bf16 (round to nearest even) in one packed conversion
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
template <> __device__ __forceinline__ void st<bf16_t, 4>(bf16_t* p, const float v[4]) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}
template <> __device__ __forceinline__ void st<float, 1>(float* p, const float v[1]) { p[0] = v[0]; }
template <> __device__ __forceinline__ void st<bf16_t, 1>(bf16_t* p, const float v[1]) {
    p[0] = from_f<bf16_t>(v[0]);
}

// non-temporal stores of one lane's VEC channels (see ld_nt)
template <typename T, int VEC> __device__ __forceinline__ void st_nt(T* p, const float v[VEC]) {
    if constexpr (VEC == 4 && std::is_same<T, bf16_t>::value) {
        typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 r = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        __builtin_nontemporal_store(r, reinterpret_cast<u32x2*>(p));
    } else if constexpr (VEC == 4) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 r = {v[0], v[1], v[2], v[3]};
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(p));
    } else {
        st<T, VEC>(p, v);
    }
}

// sigmoid(p) = 1 / (1 + exp(-p)) with the hardware exp2 and reciprocal.  No sign
// folding is needed here: for p << 0 the exponential is large and its
// reciprocal stays relatively accurate, and past overflow 1/inf gives 0.
__device__ __forceinline__ float sigmoid_c(float p) {
    return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(p * -1.4426950408889634f));
}

// pre-activation of one channel: bias first, then the taps in increasing k.
template <int K>
__device__ __forceinline__ float conv_pre(float bias, const float w[K], const float v[K]) {
    float acc = bias;
#pragma unroll
    for (int k = 0; k < K; ++k) acc = __builtin_fmaf(w[k], v[k], acc);
    return acc;
}

template <int K, int VEC>
__device__ __forceinline__ void load_params(const float* __restrict__ w, const float* __restrict__ bias,
                                            int c0, float wk[VEC][K], float bs[VEC]) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
#pragma unroll
        for (int k = 0; k < K; ++k) wk[v][k] = w[(int64_t)(c0 + v) * K + k];
        bs[v] = bias ? bias[c0 + v] : 0.0f;
    }
}

// Input of one lane's VEC channels at time tau < L: x for tau >= 0, else the
// caller's ring (zero when absent).
template <typename T, int K, int VEC>
__device__ __forceinline__ void input_at(const T* __restrict__ x, const float* __restrict__ ring0, int b,
                                         int c0, int tau, int L, int D, float out[VEC]) {
    if (tau >= 0) {
        unpack(ld<T, VEC>(x + ((int64_t)b * L + tau) * D + c0), out);
    } else {
#pragma unroll
        for (int v = 0; v < VEC; ++v)
            out[v] = ring0 ? ring0[((int64_t)b * D + c0 + v) * (K - 1) + (tau + K - 1)] : 0.0f;
    }
}

// Drop the oldest of N window entries (the caller then writes entry N-1).
template <int N, int VEC>
__device__ __forceinline__ void shift_window(float win[N][VEC]) {
#pragma unroll
    for (int j = 0; j + 1 < N; ++j)
#pragma unroll
        for (int v = 0; v < VEC; ++v) win[j][v] = win[j + 1][v];
}

// ------------------------------------------------------------------ forward
// One output token from the window of its K inputs (oldest first).
template <typename T, int K, int VEC>
__device__ __forceinline__ void fwd_token(const float wk[VEC][K], const float bs[VEC],
                                          const float win[K][VEC], T* __restrict__ yrow) {
    float out[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        float tap[K];
#pragma unroll
        for (int k = 0; k < K; ++k) tap[k] = win[k][v];
        const float pre = conv_pre<K>(bs[v], wk[v], tap);
        out[v] = pre * sigmoid_c(pre);
    }
    st_nt<T, VEC>(yrow, out);
}

template <typename T, int K, int VEC>
__global__ __launch_bounds__(WG) void k_conv_fwd(const T* __restrict__ x, const float* __restrict__ w,
                                                 const float* __restrict__ bias,
                                                 const float* __restrict__ ring0, T* __restrict__ y,
                                                 float* __restrict__ ring_last, int L, int D) {
    typedef typename Raw<T, VEC>::type R;
    // the wave index is uniform across the wave: say so, so that every token-range
    // test below is a scalar branch instead of an exec-mask region
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c0 = (blockIdx.x * 64 + lane) * VEC;
    const int b = blockIdx.z;
    const int t0 = (blockIdx.y * NWAVE + wave) * TT;
    if (c0 >= D || t0 >= L) return;  // no barrier in this kernel
    const int t1 = min(t0 + TT, L);
    float wk[VEC][K], bs[VEC], win[K][VEC];
    load_params<K, VEC>(w, bias, c0, wk, bs);
#pragma unroll
    for (int j = 0; j < K - 1; ++j) input_at<T, K, VEC>(x, ring0, b, c0, t0 - (K - 1) + j, L, D, win[j]);
    const T* xp = x + (int64_t)b * L * D + c0;
    T* yp = y + (int64_t)b * L * D + c0;
    const int tf = t0 + (t1 - t0) / PF * PF;  // end of the run's whole groups of PF tokens
    if (tf > t0) {
        // whole groups: PF tokens in flight, no range tests in the body, so the
        // window rotates through registers without copies
        R q[PF];
#pragma unroll
        for (int p = 0; p < PF; ++p) q[p] = ld_nt<T, VEC>(xp + (int64_t)(t0 + p) * D);
        // Every group of PF tokens but the last fetches the PF tokens after it, all
        // inside the run: with no per-token fetch test the queue is refilled in
        // place, so no wait on the loads just issued is needed at the loop's end.
        auto group = [&](int u, auto fetch) {
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                unpack(q[p], win[K - 1]);
                if constexpr (decltype(fetch)::value) q[p] = ld_nt<T, VEC>(xp + (int64_t)(u + p + PF) * D);
                fwd_token<T, K, VEC>(wk, bs, win, yp + (int64_t)(u + p) * D);
                shift_window<K, VEC>(win);
            }
        };
        int u = t0;
        for (; u + PF < tf; u += PF) group(u, std::true_type{});
        group(u, std::false_type{});
    }
    for (int u = tf; u < t1; ++u) {  // a ragged last run's remaining tokens
        unpack(ld<T, VEC>(xp + (int64_t)u * D), win[K - 1]);
        fwd_token<T, K, VEC>(wk, bs, win, yp + (int64_t)u * D);
        shift_window<K, VEC>(win);
    }
    // the last K-1 inputs (oldest first) continue the stream
    if (t1 == L && ring_last) {
#pragma unroll
        for (int v = 0; v < VEC; ++v)
#pragma unroll
            for (int j = 0; j < K - 1; ++j)
                ring_last[((int64_t)b * D + c0 + v) * (K - 1) + j] = win[j][v];
    }
}

// ------------------------------------------------------------------ backward
// g = dy * d silu / d pre at one token, from the window of its K inputs.
template <int K, int VEC>
__device__ __forceinline__ void silu_grad(const float wk[VEC][K], const float bs[VEC],
                                          const float (*taps)[VEC], const float dyv[VEC], float g[VEC]) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        float tap[K];
#pragma unroll
        for (int k = 0; k < K; ++k) tap[k] = taps[k][v];
        const float pre = conv_pre<K>(bs[v], wk[v], tap);
        const float s = sigmoid_c(pre);
        g[v] = dyv[v] * (s * __builtin_fmaf(pre, 1.0f - s, 1.0f));  // s (1 + pre (1 - s))
    }
}

// One step of the backward sweep: token u enters (input xn, upstream dyn; HAVE =
// u < L, else its g is 0).  Windows before the step: xw[i] = x[u-K+i] and
// gw[i] = g[u-K+i] (i = 1 .. K-1); after it they end at token u.  Then
//   own token (u inside this run):  dw[k] += g[u] x[u-K+1+k],  dbias += g[u]
//   STORE (tau = u-K+1 inside this run):  dx[tau] = sum_k w[k] g[tau+K-1-k]
template <typename T, int K, int VEC>
__device__ __forceinline__ void bwd_step(const float wk[VEC][K], const float bs[VEC], float xw[K][VEC],
                                         float gw[K][VEC], bool have, bool own, bool store,
                                         const float xn[VEC], const float dyn[VEC], float dwa[K][VEC],
                                         float dba[VEC], T* __restrict__ dxrow) {
    shift_window<K, VEC>(xw);
    shift_window<K, VEC>(gw);
#pragma unroll
    for (int v = 0; v < VEC; ++v) xw[K - 1][v] = xn[v];
    float g[VEC];
    silu_grad<K, VEC>(wk, bs, xw, dyn, g);
#pragma unroll
    for (int v = 0; v < VEC; ++v) gw[K - 1][v] = have ? g[v] : 0.0f;
    if (own) {
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            dba[v] += gw[K - 1][v];
#pragma unroll
            for (int k = 0; k < K; ++k) dwa[k][v] = __builtin_fmaf(gw[K - 1][v], xw[k][v], dwa[k][v]);
        }
    }
    if (store) {
        float o[VEC];
#pragma unroll
        for (int v = 0; v < VEC; ++v) {
            float acc = 0.0f;
#pragma unroll
            for (int k = 0; k < K; ++k) acc = __builtin_fmaf(wk[v][k], gw[K - 1 - k][v], acc);
            o[v] = acc;
        }
        st_nt<T, VEC>(dxrow, o);
    }
}

// part: [Bt * gridDim.y, K+1, D] per-workgroup sums (dw taps, then dbias).
template <typename T, int K, int VEC>
__global__ __launch_bounds__(WG) void k_conv_bwd(const T* __restrict__ x, const float* __restrict__ w,
                                                 const float* __restrict__ bias,
                                                 const float* __restrict__ ring0,
                                                 const T* __restrict__ dy, T* __restrict__ dx,
                                                 float* __restrict__ dring0, float* __restrict__ part,
                                                 int L, int D) {
    typedef typename Raw<T, VEC>::type R;
    constexpr int NP = (K + 1) * VEC;
    __shared__ float red[NWAVE][NP][64];
    const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int c0 = (blockIdx.x * 64 + lane) * VEC;
    const int b = blockIdx.z;
    const int t0 = (blockIdx.y * NWAVE + wave) * TT;
    float dwa[K][VEC], dba[VEC];
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
        dba[v] = 0.0f;
#pragma unroll
        for (int k = 0; k < K; ++k) dwa[k][v] = 0.0f;
    }
    if (c0 < D && t0 < L) {
        const int t1 = min(t0 + TT, L);
        float wk[VEC][K], bs[VEC], xw[K][VEC], gw[K][VEC];
        load_params<K, VEC>(w, bias, c0, wk, bs);
#pragma unroll
        for (int i = 1; i < K; ++i) input_at<T, K, VEC>(x, ring0, b, c0, t0 - K + i, L, D, xw[i]);
#pragma unroll
        for (int i = 0; i < K; ++i)
#pragma unroll
            for (int v = 0; v < VEC; ++v) gw[i][v] = 0.0f;
        const int64_t base = (int64_t)b * L * D + c0;
        const T* xp = x + base;
        const T* gp = dy + base;
        T* dxp = dx + base;
        // ring entry j (input time j-(K-1)) feeds tokens 0..j through tap j-t; it
        // is final once gw[t+1] = g[t] for t = 0 .. K-2 (after token K-2 entered)
        auto ring_grad = [&]() {
#pragma unroll
            for (int v = 0; v < VEC; ++v)
#pragma unroll
                for (int j = 0; j < K - 1; ++j) {
                    float acc = 0.0f;
#pragma unroll
                    for (int t = 0; t <= j; ++t) acc = __builtin_fmaf(wk[v][j - t], gw[t + 1][v], acc);
                    dring0[((int64_t)b * D + c0 + v) * (K - 1) + j] = acc;
                }
        };
        const int uend = t1 + K - 1;  // tokens entering: the run plus the look-ahead
        if (t1 - t0 >= PF) {
            // The first K-1 tokens (no dx yet) and the first PF of the rest are
            // fetched together; the rest stream with PF tokens in flight.  Groups
            // of own tokens need no range test; the last group or two hold the
            // run's last tokens and the K-1 token look-ahead (zero past the
            // sequence end, and a ragged last run is padded to whole groups), with
            // wave-uniform tests only.  Both windows rotate through registers.
            const int ugen = t0 + K - 1;
            const int ulim = min(uend, L);  // entering tokens that exist
            R hx[K > 1 ? K - 1 : 1], hg[K > 1 ? K - 1 : 1], qx[PF], qg[PF];
#pragma unroll
            for (int i = 0; i < K - 1; ++i) {
                hx[i] = ld_nt<T, VEC>(xp + (int64_t)(t0 + i) * D);
                hg[i] = ld_nt<T, VEC>(gp + (int64_t)(t0 + i) * D);
            }
#pragma unroll
            for (int p = 0; p < PF; ++p) {
                if (ugen + p < ulim) {
                    qx[p] = ld_nt<T, VEC>(xp + (int64_t)(ugen + p) * D);
                    qg[p] = ld_nt<T, VEC>(gp + (int64_t)(ugen + p) * D);
                } else {
                    qx[p] = qg[p] = R{};
                }
            }
#pragma unroll
            for (int i = 0; i < K - 1; ++i) {
                float xn[VEC], dyn[VEC];
                unpack(hx[i], xn);
                unpack(hg[i], dyn);
                bwd_step<T, K, VEC>(wk, bs, xw, gw, true, true, false, xn, dyn, dwa, dba, dxp);
            }
            if (t0 == 0 && dring0) ring_grad();
            int u0 = ugen;
            for (; u0 + PF <= t1; u0 += PF) {  // groups of own tokens
#pragma unroll
                for (int p = 0; p < PF; ++p) {
                    const int u = u0 + p;
                    float xn[VEC], dyn[VEC];
                    unpack(qx[p], xn);
                    unpack(qg[p], dyn);
                    if (u + PF < ulim) {
                        qx[p] = ld_nt<T, VEC>(xp + (int64_t)(u + PF) * D);
                        qg[p] = ld_nt<T, VEC>(gp + (int64_t)(u + PF) * D);
                    }
                    bwd_step<T, K, VEC>(wk, bs, xw, gw, true, true, true, xn, dyn, dwa, dba,
                                        dxp + (int64_t)(u - (K - 1)) * D);
                }
            }
            for (; u0 < uend; u0 += PF) {  // the run's last tokens and the look-ahead
#pragma unroll
                for (int p = 0; p < PF; ++p) {
                    const int u = u0 + p;
                    float xn[VEC], dyn[VEC];
                    unpack(qx[p], xn);
                    unpack(qg[p], dyn);
                    if (u + PF < ulim) {
                        qx[p] = ld_nt<T, VEC>(xp + (int64_t)(u + PF) * D);
                        qg[p] = ld_nt<T, VEC>(gp + (int64_t)(u + PF) * D);
                    }
                    bwd_step<T, K, VEC>(wk, bs, xw, gw, u < L, u < t1, u < uend, xn, dyn, dwa, dba,
                                        dxp + (int64_t)(u - (K - 1)) * D);
                }
            }
        } else {
            for (int u = t0; u < uend; ++u) {
                const bool have = u < L;
                float xn[VEC], dyn[VEC];
                if (have) {
                    unpack(ld_nt<T, VEC>(xp + (int64_t)u * D), xn);
                    unpack(ld_nt<T, VEC>(gp + (int64_t)u * D), dyn);
                } else {
#pragma unroll
                    for (int v = 0; v < VEC; ++v) xn[v] = dyn[v] = 0.0f;
                }
                const int tau = u - (K - 1);
                bwd_step<T, K, VEC>(wk, bs, xw, gw, have, u < t1, tau >= t0, xn, dyn, dwa, dba,
                                    dxp + (int64_t)max(tau, 0) * D);
                if (u == K - 2 && t0 == 0 && dring0) ring_grad();
            }
        }
    }
    // dw / dbias: this lane's sums over its run, then over the 4 runs in order
#pragma unroll
    for (int v = 0; v < VEC; ++v) {
#pragma unroll
        for (int k = 0; k < K; ++k) red[wave][k * VEC + v][lane] = dwa[k][v];
        red[wave][K * VEC + v][lane] = dba[v];
    }
    __syncthreads();
    // row k of this workgroup's partials (dw tap k, or dbias at k = K) holds the
    // D channels contiguously, so each lane stores its VEC channels in one piece
    if (c0 < D) {
        float* prow = part + ((int64_t)b * gridDim.y + blockIdx.y) * (K + 1) * D + c0;
        for (int k = wave; k <= K; k += NWAVE) {
            float s[VEC];
#pragma unroll
            for (int v = 0; v < VEC; ++v) {
                const int e = k * VEC + v;
                s[v] = ((red[0][e][lane] + red[1][e][lane]) + red[2][e][lane]) + red[3][e][lane];
            }
            st<float, VEC>(prow + (int64_t)k * D, s);
        }
    }
}

// dw[d,k] / dbias[d] = sum over tiles of the partials, in a fixed order: each of
// the 4 waves sums a contiguous quarter of the tiles for 64 consecutive outputs
// (8 loads in flight per lane), then the quarters are added in order.
__global__ __launch_bounds__(WG) void k_conv_bwd_reduce(const float* __restrict__ part,
                                                        float* __restrict__ dw,
                                                        float* __restrict__ dbias, int64_t ntiles,
                                                        int D, int K) {
    __shared__ float q[NWAVE][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t per = (int64_t)D * (K + 1);
    const int64_t idx = (int64_t)blockIdx.x * 64 + lane;
    const int64_t n0 = ntiles * wave / NWAVE, n1 = ntiles * (wave + 1) / NWAVE;
    float s = 0.0f;
    if (idx < per) {
        int64_t t = n0;
        for (; t + 8 <= n1; t += 8) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = part[(t + j) * per + idx];
#pragma unroll
            for (int j = 0; j < 8; ++j) s += v[j];
        }
        for (; t < n1; ++t) s += part[t * per + idx];
    }
    q[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && idx < per) {
        const float tot = ((q[0][lane] + q[1][lane]) + q[2][lane]) + q[3][lane];
        const int k = (int)(idx / D), d = (int)(idx % D);
        if (k < K) dw[(int64_t)d * K + k] = tot;
        else dbias[d] = tot;
    }
}

// ------------------------------------------------------------------ step
template <typename T, int K>
__global__ __launch_bounds__(WG) void k_conv_step(float* __restrict__ ring, const T* __restrict__ x,
                                                  const float* __restrict__ w,
                                                  const float* __restrict__ bias, T* __restrict__ y,
                                                  int64_t n, int D) {
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (i >= n) return;
    const int d = (int)(i % D);
    const float xv = to_f(x[i]);
    float* r = ring + i * (K - 1);
    float wk[K], tap[K];
#pragma unroll
    for (int k = 0; k < K; ++k) wk[k] = w[(int64_t)d * K + k];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) tap[k] = r[k];
    tap[K - 1] = xv;
    const float pre = conv_pre<K>(bias ? bias[d] : 0.0f, wk, tap);
    y[i] = from_f<T>(pre * sigmoid_c(pre));
#pragma unroll
    for (int j = 0; j < K - 1; ++j) r[j] = tap[j + 1];
}

// dst[i] = src ? src[i] : 0
__global__ __launch_bounds__(WG) void k_conv_fill(float* __restrict__ dst,
                                                  const float* __restrict__ src, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * WG + threadIdx.x;
    if (i < n) dst[i] = src ? src[i] : 0.0f;
}

// ------------------------------------------------------------------ host side
struct ConvPlan {
    int64_t Bt, L, D, K;
    int io;
    int vec;       // channels per lane (4, or 1 when d_inner % 4 != 0)
    int64_t gx, gy;
};

ssm_status check_conv(const ssm_conv_dims* d) {
    if (!d) return SSM_E_NULLPTR;
    if (d->batch <= 0 || d->seqlen < 0 || d->d_inner <= 0 || d->d_conv <= 0) return SSM_E_SHAPE;
    if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_E_DTYPE;
    if (d->d_conv > KMAX || d->batch > 65535 || d->d_inner > INT_MAX / 4 ||
        d->seqlen > (int64_t)65535 * NWAVE * TT)
        return SSM_E_UNSUPPORTED;
    return SSM_OK;
}

ConvPlan conv_plan(const ssm_conv_dims* d) {
    ConvPlan p;
    p.Bt = d->batch;
    p.L = d->seqlen;
    p.D = d->d_inner;
    p.K = d->d_conv;
    p.io = d->io_dtype;
    p.vec = p.D % 4 == 0 ? 4 : 1;
    p.gx = (p.D / p.vec + 63) / 64;
    p.gy = (p.L + NWAVE * TT - 1) / (NWAVE * TT);
    return p;
}

size_t conv_ws_bytes(const ConvPlan& p) {
    return sizeof(float) * (size_t)(p.Bt * p.gy * p.D * (p.K + 1));
}


struct Launcher {
    ssm::Launcher l;
    template <typename Kern, typename... Args>
    ssm_status operator()(int kid, Kern kern, dim3 grid, Args... args) {
        return l(kid, kern, grid, dim3(WG), args...);
    }
};

template <typename T, int K, int VEC>
ssm_status run_fwd(const ConvPlan& p, const void* x, const float* w, const float* bias,
                   const float* ring0, void* y, float* ring_last, Launcher& launch) {
    return launch(SSM_K_CONV_FWD, k_conv_fwd<T, K, VEC>, dim3((unsigned)p.gx, (unsigned)p.gy, (unsigned)p.Bt),
                  (const T*)x, w, bias, ring0, (T*)y, ring_last, (int)p.L, (int)p.D);
}

template <typename T, int K, int VEC>
ssm_status run_bwd(const ConvPlan& p, const void* x, const float* w, const float* bias,
                   const float* ring0, const void* dy, void* dx, float* dw, float* dbias,
                   float* dring0, float* part, Launcher& launch) {
    SSM_TRY(launch(SSM_K_CONV_BWD, k_conv_bwd<T, K, VEC>,
                   dim3((unsigned)p.gx, (unsigned)p.gy, (unsigned)p.Bt), (const T*)x, w, bias, ring0,
                   (const T*)dy, (T*)dx, dring0, part, (int)p.L, (int)p.D));
    const int64_t per = p.D * (p.K + 1);
    return launch(SSM_K_CONV_BWD_REDUCE, k_conv_bwd_reduce, dim3((unsigned)((per + 63) / 64)),
                  (const float*)part, dw, dbias, p.Bt * p.gy, (int)p.D, (int)p.K);
}

// The forward / backward launch for one (io dtype, K, VEC) instantiation.
struct FwdCall {
    const ConvPlan& p; const void* x; const float* w; const float* bias; const float* ring0;
    void* y; float* ring_last; Launcher& launch;
    template <typename T, int K, int VEC> ssm_status run() {
        return run_fwd<T, K, VEC>(p, x, w, bias, ring0, y, ring_last, launch);
    }
};
struct BwdCall {
    const ConvPlan& p; const void* x; const float* w; const float* bias; const float* ring0;
    const void* dy; void* dx; float* dw; float* dbias; float* dring0; float* part; Launcher& launch;
    template <typename T, int K, int VEC> ssm_status run() {
        return run_bwd<T, K, VEC>(p, x, w, bias, ring0, dy, dx, dw, dbias, dring0, part, launch);
    }
};

// Instantiation over (io dtype, K, VEC) for the forward and backward.
template <int K, int VEC, typename F>
ssm_status by_dtype(int io, F&& f) {
    return io == SSM_F32 ? f.template run<float, K, VEC>() : f.template run<bf16_t, K, VEC>();
}

template <typename F>
ssm_status dispatch(const ConvPlan& p, F&& f) {
    const bool v4 = p.vec == 4;
    switch (p.K) {
        case 1: return v4 ? by_dtype<1, 4>(p.io, f) : by_dtype<1, 1>(p.io, f);
        case 2: return v4 ? by_dtype<2, 4>(p.io, f) : by_dtype<2, 1>(p.io, f);
        case 3: return v4 ? by_dtype<3, 4>(p.io, f) : by_dtype<3, 1>(p.io, f);
        default: return v4 ? by_dtype<4, 4>(p.io, f) : by_dtype<4, 1>(p.io, f);
    }
}

}  // namespace

// Scratch of ssm_conv1d_bwd_noalloc: each GPU the library runs on holds one
// copy, at its own device address.  Host code never uses this name as an
// address (on the host it is a stand-in): the per-device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
__device__ __align__(256) unsigned char scratch[SSM_CONV1D_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void* scratch_ptr[MAX_DEVICES];  // device address of `scratch`, per device

ssm_status scratch_on_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return SSM_E_LAUNCH;
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSM_E_LAUNCH;
        scratch_ptr[dev] = p;
    }
    *out = scratch_ptr[dev];
    return SSM_OK;
}
}  // namespace

extern "C" {

size_t ssm_conv1d_bwd_workspace_bytes(const ssm_conv_dims* dims) {
    if (check_conv(dims) != SSM_OK || dims->seqlen == 0) return 0;
    return conv_ws_bytes(conv_plan(dims));
}

ssm_status ssm_conv1d_fwd(const ssm_conv_dims* dims, const void* x, const float* w,
                          const float* bias, const float* ring0, void* y, float* ring_last,
                          hipStream_t stream, ssm_timing* timing) {
    SSM_TRY(check_conv(dims));
    const ConvPlan p = conv_plan(dims);
    if (!w) return SSM_E_NULLPTR;
    if (p.L > 0 && (!x || !y)) return SSM_E_NULLPTR;
    if (p.K == 1) ring0 = ring_last = nullptr;
    if (ring_last && ring_last == ring0) return SSM_E_UNSUPPORTED;
    const void* ptrs[] = {x, w, bias, ring0, y, ring_last};
    for (const void* q : ptrs)
        if (q && misaligned(q)) return SSM_E_ALIGN;
    (void)hipGetLastError();
    Launcher launch{{stream, timing}};
    if (p.L == 0) {
        if (!ring_last) return SSM_OK;
        const int64_t n = p.Bt * p.D * (p.K - 1);
        return launch(SSM_K_CONV_RING, k_conv_fill, dim3((unsigned)((n + WG - 1) / WG)), ring_last, ring0, n);
    }
    FwdCall f{p, x, w, bias, ring0, y, ring_last, launch};
    return dispatch(p, f);
}

ssm_status ssm_conv1d_bwd(const ssm_conv_dims* dims, const void* x, const float* w,
                          const float* bias, const float* ring0, const void* dy, void* dx,
                          float* dw, float* dbias, float* dring0, void* ws, size_t ws_bytes,
                          hipStream_t stream, ssm_timing* timing) {
    SSM_TRY(check_conv(dims));
    const ConvPlan p = conv_plan(dims);
    if (!w || !dw || !dbias) return SSM_E_NULLPTR;
    if (p.L > 0 && (!x || !dy || !dx)) return SSM_E_NULLPTR;
    if (p.K == 1) ring0 = dring0 = nullptr;
    const void* ptrs[] = {x, w, bias, ring0, dy, dx, dw, dbias, dring0, ws};
    for (const void* q : ptrs)
        if (q && misaligned(q)) return SSM_E_ALIGN;
    const size_t need = p.L > 0 ? conv_ws_bytes(p) : 0;
    if (need > 0 && (!ws || ws_bytes < need)) return SSM_E_WORKSPACE;
    (void)hipGetLastError();
    Launcher launch{{stream, timing}};
    if (p.L == 0) {
        const int64_t nw = p.D * p.K;
        SSM_TRY(launch(SSM_K_CONV_RING, k_conv_fill, dim3((unsigned)((nw + WG - 1) / WG)), dw,
                       (const float*)nullptr, nw));
        SSM_TRY(launch(SSM_K_CONV_RING, k_conv_fill, dim3((unsigned)((p.D + WG - 1) / WG)), dbias,
                       (const float*)nullptr, p.D));
        if (dring0) {
            const int64_t n = p.Bt * p.D * (p.K - 1);
            SSM_TRY(launch(SSM_K_CONV_RING, k_conv_fill, dim3((unsigned)((n + WG - 1) / WG)), dring0,
                           (const float*)nullptr, n));
        }
        return SSM_OK;
    }
    float* part = static_cast<float*>(ws);
    BwdCall f{p, x, w, bias, ring0, dy, dx, dw, dbias, dring0, part, launch};
    return dispatch(p, f);
}

ssm_status ssm_conv1d_bwd_noalloc(const ssm_conv_dims* dims, const void* x, const float* w,
                                  const float* bias, const float* ring0, const void* dy, void* dx,
                                  float* dw, float* dbias, float* dring0, hipStream_t stream,
                                  ssm_timing* timing) {
    SSM_TRY(check_conv(dims));
    const size_t need = dims->seqlen > 0 ? conv_ws_bytes(conv_plan(dims)) : 0;
    if (need > SSM_CONV1D_SCRATCH_BYTES) return SSM_E_WORKSPACE;
    void* ws = nullptr;
    if (need > 0) SSM_TRY(scratch_on_current_device(&ws));
    return ssm_conv1d_bwd(dims, x, w, bias, ring0, dy, dx, dw, dbias, dring0, ws, need, stream, timing);
}

ssm_status ssm_conv1d_step(int64_t batch, int64_t d_inner, int64_t d_conv, int32_t io_dtype,
                           float* ring, const void* x, const float* w, const float* bias, void* y,
                           hipStream_t stream, ssm_timing* timing) {
    const ssm_conv_dims dims{batch, 1, d_inner, d_conv, io_dtype};
    SSM_TRY(check_conv(&dims));
    if (!x || !w || !y || (d_conv > 1 && !ring)) return SSM_E_NULLPTR;
    if (d_conv == 1) ring = nullptr;
    const void* ptrs[] = {ring, x, w, bias, y};
    for (const void* q : ptrs)
        if (q && misaligned(q)) return SSM_E_ALIGN;
    (void)hipGetLastError();
    Launcher launch{{stream, timing}};
    const int64_t n = batch * d_inner;
    const dim3 grid((unsigned)((n + WG - 1) / WG));
    const int D = (int)d_inner;
    const bool f32 = io_dtype == SSM_F32;
    switch (d_conv) {
        case 1:
            return f32 ? launch(SSM_K_CONV_STEP, k_conv_step<float, 1>, grid, ring, (const float*)x, w, bias, (float*)y, n, D)
                       : launch(SSM_K_CONV_STEP, k_conv_step<bf16_t, 1>, grid, ring, (const bf16_t*)x, w, bias, (bf16_t*)y, n, D);
        case 2:
            return f32 ? launch(SSM_K_CONV_STEP, k_conv_step<float, 2>, grid, ring, (const float*)x, w, bias, (float*)y, n, D)
                       : launch(SSM_K_CONV_STEP, k_conv_step<bf16_t, 2>, grid, ring, (const bf16_t*)x, w, bias, (bf16_t*)y, n, D);
        case 3:
            return f32 ? launch(SSM_K_CONV_STEP, k_conv_step<float, 3>, grid, ring, (const float*)x, w, bias, (float*)y, n, D)
                       : launch(SSM_K_CONV_STEP, k_conv_step<bf16_t, 3>, grid, ring, (const bf16_t*)x, w, bias, (bf16_t*)y, n, D);
        default:
            return f32 ? launch(SSM_K_CONV_STEP, k_conv_step<float, 4>, grid, ring, (const float*)x, w, bias, (float*)y, n, D)
                       : launch(SSM_K_CONV_STEP, k_conv_step<bf16_t, 4>, grid, ring, (const bf16_t*)x, w, bias, (bf16_t*)y, n, D);
    }
}

}  // extern "C"
