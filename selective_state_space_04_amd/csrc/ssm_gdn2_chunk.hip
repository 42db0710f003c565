// ssm_gdn2_chunk.hip -- Gated DeltaNet-2 forward in chunks of 64 tokens for
// MI355X (gfx950): the chunked WY form of burn-gdn2 0.1.4, page
// "src/forward.rs", with the decays kept per key dimension (the per-token
// recurrence it regroups is in ssm_gdn2.h).
//
// Per (batch*head pair, chunk of CH tokens), with G the inclusive cumulative
// sum of the log-decays g inside the chunk ([CH, K]) and S the [K, V] state
// entering the chunk:
//   A[i][j] = sum_k b_i k_i k_j exp(G_i - G_j)        (j < i)
//   P[i][j] = sum_k q_i k_j exp(G_i - G_j)            (j <= i)
//   M = I + A,  BKe = b * k * exp(G),  Qe = q * exp(G),  Kd = k * exp(G_last - G)
//   vn = M^{-1} (w * v - BKe S)          (the corrected values)
//   o  = scale (P vn + Qe S)
//   S' = diag(exp(G_last)) S + Kd^T vn
// Every exp(G_i - G_j) used has i >= j, so it is <= 1 for log-decays <= 0.  It
// is never split into exp(G_i) and exp(-G_j) (the second overflows for strong
// gates): inside a 16-token diagonal block it is formed per element, and for
// i, j in blocks bi > bj it is split at the end E of block bj as
// exp(G_i - E) * exp(E - G_j), both factors <= 1, so no gate strength can
// overflow it.
//
// Two kernels:
//   k_gdn2_wy     key side, parallel over (pair, chunk): G, A and P (the
//                 off-diagonal 16-token blocks as MFMA products of the split
//                 decays, the diagonal blocks per element), M^{-1} by forward
//                 substitution, BKe, Qe, Kd, exp(G_last); everything written to
//                 the workspace in the operand order of v_mfma_f32_16x16x4f32.
//   k_gdn2_state  one workgroup per (pair, 16 state columns), sequential over
//                 the chunks, one wave per 16-token tile: the five products
//                 above on MFMA, the state in LDS.  The 16 columns of a pair
//                 run on one XCD, so its L2 serves their shared key-side reads.
// MFMA lane layout (v_mfma_f32_16x16x4f32, one wave): A[i][k] comes from lane
// 16k + i, B[k][j] from lane 16k + j, and D[4q + r][j] lands in lane 16q + j,
// register r.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ssm_common.h"
#include "ssm_gdn2.h"

namespace {

constexpr int CH = 64;       // tokens per chunk
constexpr int WGK = 256;     // threads of the key-side kernel
constexpr int XCDS = 8;
constexpr float LOG2E = 1.4426950408889634f;

typedef float f4 __attribute__((ext_vector_type(4)));

// Workspace per (pair, chunk), in floats, for key dimension K.
template <int K>
struct Lay {
    // A operands, four consecutive contraction blocks per lane as one float4:
    // element (tile, block m, lane) at ((tile * nblocks / 4 + m / 4) * 64 + lane) * 4 + m % 4
    static constexpr int nBKe = 0;                 // -BKe:   [4 row tiles][K/4 k-blocks]
    static constexpr int Qe = nBKe + CH * K;       // Qe:     [4][K/4]
    static constexpr int KdT = Qe + CH * K;        // Kd^T:   [K/16 row tiles][16 token blocks]
    static constexpr int P = KdT + CH * K;         // P:      [4][16]
    static constexpr int Mi = P + CH * CH;         // M^{-1}: [4][16]
    static constexpr int eGl = Mi + CH * CH;       // exp(G_last):       [K]
    static constexpr int total = (eGl + K + 63) / 64 * 64;
};

template <typename TT>
__device__ __forceinline__ float ld(const TT* p, int64_t i) { return ssm::to_f(p[i]); }

// Offset of A-operand element (tile, contraction block m, lane) in a region
// whose tiles have nb blocks each.
__host__ __device__ constexpr int aop(int tile, int m, int lane, int nb) {
    return ((tile * (nb / 4) + m / 4) * 64 + lane) * 4 + m % 4;
}

__device__ __forceinline__ f4 mfma(float a, float b, f4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Key side of one chunk.  grid (chunks, pairs), WGK threads.
//
// A and P by 16-token blocks.  For a block pair bi > bj both factors of
//   exp(G_i - G_j) = exp(G_i - E_bj) * exp(E_bj - G_j),
// E_bj = G at block bj's last token, have exponent <= 0 (G falls along the
// chunk), so the block is a product of two decayed operands on MFMA with no
// overflow for any gate strength: the six block pairs give twelve 16 x 16
// products (A and P), three per wave.  The four diagonal blocks keep the
// per-element exponential (136 entries each, j <= i, spread over all threads).
template <typename TT, int K>
__global__ __launch_bounds__(WGK) void k_gdn2_wy(const TT* __restrict__ q, const TT* __restrict__ k,
                                                 const TT* __restrict__ g, const TT* __restrict__ b,
                                                 float* __restrict__ ws, int T, int nch) {
    constexpr int KC = K < 32 ? K : 32;  // key dimensions staged per pass
    constexpr int RP = CH + 4;           // padded staging row: MFMA operand reads hit 64 banks
    constexpr int NDIAG = 4 * 136;       // entries j <= i of the four diagonal 16 x 16 blocks
    constexpr int DPT = (NDIAG + WGK - 1) / WGK;
    using L = Lay<K>;
    // staging for the passes (g, k, b*k, q as [key][token]); after them the same
    // memory holds A, P and M^-1
    __shared__ float lds[3 * CH * CH];
    float(*As)[CH] = reinterpret_cast<float(*)[CH]>(lds);
    float(*Ps)[CH] = reinterpret_cast<float(*)[CH]>(lds + CH * CH);
    float(*Ms)[CH] = reinterpret_cast<float(*)[CH]>(lds + 2 * CH * CH);
    static_assert(4 * KC * RP <= 3 * CH * CH, "staging must fit the A/P/M^-1 region");
    static_assert(CH * KC % WGK == 0, "whole staged elements per thread");
    const int tid = threadIdx.x;
    const int l = tid & 63;
    const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x;
    const int64_t pair = blockIdx.y;
    const int t0 = c * CH;
    const int n = min(CH, T - t0);
    float* out = ws + (pair * nch + c) * (int64_t)L::total;
    const int64_t row0 = pair * T + t0;
    // this wave's three off-diagonal products: chain h = 3 wv + s over the list
    // (bi, bj) = (1,0) (2,0) (3,0) (2,1) (3,1) (3,2), A then P for each pair
    int cbi[3], cbj[3];
    bool cisP[3];
#pragma unroll
    for (int s3 = 0; s3 < 3; ++s3) {
        const int h = 3 * wv + s3, pr = h >> 1;
        cbi[s3] = pr < 3 ? pr + 1 : (pr < 5 ? pr - 1 : 3);
        cbj[s3] = pr < 3 ? 0 : (pr < 5 ? 1 : 2);
        cisP[s3] = h & 1;
    }
    f4 acc[3];
#pragma unroll
    for (int s3 = 0; s3 < 3; ++s3) acc[s3] = f4{0.0f, 0.0f, 0.0f, 0.0f};
    // this thread's diagonal entries (block db, row il, column jl <= il)
    int dI[DPT], dJ[DPT];
    float dA[DPT], dP[DPT];
#pragma unroll
    for (int r = 0; r < DPT; ++r) {
        const int e = tid + r * WGK;
        const int ee = e < NDIAG ? e : 0;
        const int db = ee / 136;
        int il = 0, jl = ee % 136;
        while (jl > il) {
            jl -= il + 1;
            ++il;
        }
        dI[r] = 16 * db + il;
        dJ[r] = e < NDIAG ? 16 * db + jl : -1;  // -1: no entry
        dA[r] = dP[r] = 0.0f;
    }
    const int i16 = l & 15, kq = l >> 4;  // MFMA operand: row/column i16, key kq of each 4-key step
    // each pass's inputs are fetched into registers during the previous pass
    constexpr int EPT = CH * KC / WGK;  // staged elements per thread and pass
    float pk[EPT], pb[EPT], pq[EPT], pg[EPT];
    auto fetch = [&](int kc) {
#pragma unroll
        for (int r = 0; r < EPT; ++r) {
            const int e = tid + r * WGK;
            const int tok = e / KC, kl = e % KC;
            const bool valid = tok < n;
            const int64_t src = (row0 + min(tok, n - 1)) * K + kc * KC + kl;
            pk[r] = valid ? ld(k, src) : 0.0f;
            pb[r] = valid ? ld(b, src) : 0.0f;
            pq[r] = valid ? ld(q, src) : 0.0f;
            pg[r] = valid ? ld(g, src) : 0.0f;  // a padded token is the identity: g = 0
        }
    };
    fetch(0);
#pragma unroll 1
    for (int kc = 0; kc < K / KC; ++kc) {
        // The staging addresses are the same in every pass; hoisted out of the
        // loop they would hold about 110 more registers for its whole length (one
        // wave per SIMD instead of three).  An opaque zero offset keeps them here.
        int zz = 0;
        asm volatile("" : "+v"(zz));
        float(*Gs)[RP] = reinterpret_cast<float(*)[RP]>(lds + zz);
        float(*ks)[RP] = reinterpret_cast<float(*)[RP]>(lds + zz + KC * RP);
        float(*bks)[RP] = reinterpret_cast<float(*)[RP]>(lds + zz + 2 * KC * RP);
        float(*qs)[RP] = reinterpret_cast<float(*)[RP]>(lds + zz + 3 * KC * RP);
#pragma unroll
        for (int r = 0; r < EPT; ++r) {
            const int e = tid + r * WGK;
            const int tok = e / KC, kl = e % KC;
            ks[kl][tok] = pk[r];
            bks[kl][tok] = pb[r] * pk[r];
            qs[kl][tok] = pq[r];
            Gs[kl][tok] = pg[r];
        }
        if (kc + 1 < K / KC) fetch(kc + 1);
        __syncthreads();
        if (tid < KC) {  // inclusive cumulative sum over the chunk's tokens (in registers)
            float gv[CH];
#pragma unroll
            for (int tok = 0; tok < CH; ++tok) gv[tok] = Gs[tid][tok];
#pragma unroll
            for (int tok = 1; tok < CH; ++tok) gv[tok] += gv[tok - 1];
#pragma unroll
            for (int tok = 0; tok < CH; ++tok) Gs[tid][tok] = gv[tok];
        }
        __syncthreads();
        // off-diagonal blocks on MFMA
#pragma unroll
        for (int st = 0; st < KC / 4; ++st) {
            const int kl = 4 * st + kq;
#pragma unroll
            for (int s3 = 0; s3 < 3; ++s3) {
                const int ti = 16 * cbi[s3] + i16, tj = 16 * cbj[s3] + i16;
                const float E = Gs[kl][16 * cbj[s3] + 15];
                const float li = __builtin_amdgcn_exp2f((Gs[kl][ti] - E) * LOG2E);
                const float rj = __builtin_amdgcn_exp2f((E - Gs[kl][tj]) * LOG2E);
                const float av = (cisP[s3] ? qs[kl][ti] : bks[kl][ti]) * li;
                acc[s3] = mfma(av, ks[kl][tj] * rj, acc[s3]);
            }
        }
        // diagonal blocks, per element
#pragma unroll
        for (int r = 0; r < DPT; ++r) {
            if (dJ[r] >= 0) {
                const int i = dI[r], j = dJ[r];
                float a = dA[r], pv = dP[r];
                for (int kl = 0; kl < KC; ++kl) {
                    const float dec = __builtin_amdgcn_exp2f((Gs[kl][i] - Gs[kl][j]) * LOG2E);
                    const float kd = ks[kl][j] * dec;
                    a = __builtin_fmaf(bks[kl][i], kd, a);
                    pv = __builtin_fmaf(qs[kl][i], kd, pv);
                }
                dA[r] = a;
                dP[r] = pv;
            }
        }
        // the chunk's operands for these KC key dimensions
        for (int e = tid; e < CH * KC; e += WGK) {
            const int ti = e / (KC * 16), rem = e % (KC * 16), ml = rem / 64, ln = rem % 64;
            const int tok = 16 * ti + ln % 16, kl = 4 * ml + ln / 16;
            const float eg = __builtin_amdgcn_exp2f(Gs[kl][tok] * LOG2E);
            const int o = aop(ti, kc * (KC / 4) + ml, ln, K / 4);
            out[L::nBKe + o] = -bks[kl][tok] * eg;
            out[L::Qe + o] = qs[kl][tok] * eg;
        }
        for (int e = tid; e < CH * KC; e += WGK) {
            const int tkl = e / (16 * 64), rem = e % (16 * 64), mj = rem / 64, ln = rem % 64;
            const int tok = 4 * mj + ln / 16, kl = 16 * tkl + ln % 16;
            const float dec = __builtin_amdgcn_exp2f((Gs[kl][CH - 1] - Gs[kl][tok]) * LOG2E);
            out[L::KdT + aop(kc * (KC / 16) + tkl, mj, ln, 16)] = ks[kl][tok] * dec;
        }
        if (tid < KC) out[L::eGl + kc * KC + tid] = __builtin_amdgcn_exp2f(Gs[tid][CH - 1] * LOG2E);
        __syncthreads();
    }
    // A (strictly lower) and P (lower with the diagonal) into LDS, zero elsewhere
    for (int e = tid; e < CH * CH; e += WGK) {
        (&As[0][0])[e] = 0.0f;
        (&Ps[0][0])[e] = 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int s3 = 0; s3 < 3; ++s3) {
        float(*dst)[CH] = cisP[s3] ? Ps : As;
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[16 * cbi[s3] + 4 * kq + r][16 * cbj[s3] + i16] = acc[s3][r];
    }
#pragma unroll
    for (int r = 0; r < DPT; ++r) {
        if (dJ[r] >= 0) {
            if (dJ[r] < dI[r]) As[dI[r]][dJ[r]] = dA[r];
            Ps[dI[r]][dJ[r]] = dP[r];
        }
    }
    __syncthreads();
    if (tid < CH) {
        // column tid of M^{-1}, M = I + A unit lower triangular: forward
        // substitution X[i] = [i == tid] - sum_{j<i} A[i][j] X[j]
        // (each row's sum is split over j mod 4 into four chains, added in a
        // fixed order)
        float X[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) {
            float s4[4] = {i == tid ? 1.0f : 0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int j = 0; j < i; ++j) s4[j & 3] = __builtin_fmaf(-As[i][j], X[j], s4[j & 3]);
            const float s = (s4[0] + s4[1]) + (s4[2] + s4[3]);
            X[i] = s;
            Ms[i][tid] = s;
        }
    } else {
        for (int e = tid - CH; e < CH * CH; e += WGK - CH) {
            const int ti = e / 1024, mj = (e / 64) % 16, ln = e % 64;
            out[L::P + aop(ti, mj, ln, 16)] = Ps[16 * ti + ln % 16][4 * mj + ln / 16];
        }
    }
    __syncthreads();
    for (int e = tid; e < CH * CH; e += WGK) {
        const int ti = e / 1024, mj = (e / 64) % 16, ln = e % 64;
        out[L::Mi + aop(ti, mj, ln, 16)] = Ms[16 * ti + ln % 16][4 * mj + ln / 16];
    }
}

// Four consecutive A-operand blocks (4 m4 .. 4 m4 + 3) of a tile for this lane.
__device__ __forceinline__ f4 opnd(const float* region, int tile, int m4, int lane, int nb) {
    return *reinterpret_cast<const f4*>(region + ((tile * (nb / 4) + m4) * 64 + lane) * 4);
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// State pass: one workgroup of 4 waves per (pair, 16 columns of V), the
// [K, 16] state in LDS.  Per chunk:
//   1. wave w contracts tile w (tokens 16w .. 16w + 15) over all keys:
//      X = w * v - BKe S and oq = Qe S, the state's operand blocks read from LDS;
//   2. (barrier) every wave reads the X tiles up to its own and forms vn = M^{-1} X
//      for its tile;
//   3. (barrier) every wave reads all of vn: o = scale (P vn + oq) for its tile,
//      and S' = diag(exp(G_last)) S + Kd^T vn for its quarter of the key rows;
//   4. (barrier) the updated state is complete for the next chunk.
constexpr int RW = 80;  // padded LDS row: 64 lanes + 16 (B-operand reads hit 64 banks)

template <typename TT, int K>
__global__ __launch_bounds__(256) void k_gdn2_state(
    const TT* __restrict__ v, const TT* __restrict__ w, const float* __restrict__ ws,
    const float* __restrict__ S0, float scale, TT* __restrict__ o, float* __restrict__ S_last, int64_t nbh,
    int64_t nbh8, int T, int V, int nch) {
    using L = Lay<K>;
    constexpr int KB = K / 4;                            // k-blocks of the contraction over keys
    constexpr int NTK = K / 16;                          // 16-row tiles of the state
    constexpr int TKW = NTK < 4 ? 1 : NTK / 4;           // state tiles per updating wave
    __shared__ float Sl[K][16];                          // the state
    __shared__ float xs[4][4][RW];                       // X as [tile][r][lane]
    __shared__ float vs[4][4][RW];                       // vn
    const int l = threadIdx.x & 63;
    const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t pair = blockIdx.x % nbh8;
    const int cb = (int)(blockIdx.x / nbh8);
    if (pair >= nbh) return;  // uniform over the workgroup
    const int c16 = l & 15, quad = l >> 4;
    const int col = cb * 16 + c16;
    const bool upd = wv * TKW < NTK;  // this wave updates state tiles wv*TKW ..
    for (int e = threadIdx.x; e < K * 16; e += 256) {
        const int kr = e / 16, cc = e % 16;
        Sl[kr][cc] = S0 ? S0[(pair * K + kr) * V + cb * 16 + cc] : 0.0f;
    }
    // this wave's tile of the key-side operands for the next chunk, fetched a chunk ahead
    f4 pax[KB / 4], paq[KB / 4];
    {
        const float* b0 = ws + (pair * nch) * (int64_t)L::total;
#pragma unroll
        for (int m4 = 0; m4 < KB / 4; ++m4) {
            pax[m4] = opnd(b0 + L::nBKe, wv, m4, l, KB);
            paq[m4] = opnd(b0 + L::Qe, wv, m4, l, KB);
        }
    }
    f4 po = f4{0.0f, 0.0f, 0.0f, 0.0f};
    int pt0 = -1;
    auto store_o = [&]() {
        if (pt0 < 0) return;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = pt0 + 16 * wv + 4 * quad + r;
            if (tok < T) o[(pair * T + tok) * V + col] = ssm::from_f<TT>(scale * po[r]);
        }
    };
    __syncthreads();
    for (int c = 0; c < nch; ++c) {
        const float* base = ws + (pair * nch + c) * (int64_t)L::total;
        const float* nbase = ws + (pair * nch + min(c + 1, nch - 1)) * (int64_t)L::total;
        const int t0 = c * CH;
        // later phases' operands first
        f4 mi[4], pp[4], kd[TKW][4];
        float eg[TKW][4];
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4) {
            if (m4 <= wv) {
                mi[m4] = opnd(base + L::Mi, wv, m4, l, 16);
                pp[m4] = opnd(base + L::P, wv, m4, l, 16);
            } else {
                mi[m4] = pp[m4] = f4{0.0f, 0.0f, 0.0f, 0.0f};
            }
        }
#pragma unroll
        for (int j = 0; j < TKW; ++j) {
            const int tk = upd ? wv * TKW + j : 0;
#pragma unroll
            for (int m4 = 0; m4 < 4; ++m4) kd[j][m4] = opnd(base + L::KdT, tk, m4, l, 16);
#pragma unroll
            for (int r = 0; r < 4; ++r) eg[j][r] = base[L::eGl + 16 * tk + 4 * quad + r];
        }
        f4 X = f4{0.0f, 0.0f, 0.0f, 0.0f}, oq = X;
        float wvv[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int tok = t0 + 16 * wv + 4 * quad + r;
            const int64_t e = (pair * T + min(tok, T - 1)) * V + col;
            wvv[r] = tok < T ? ld(w, e) * ld(v, e) : 0.0f;
        }
        store_o();  // the previous chunk's outputs, after this chunk's first loads
        // 1. tile wv over all keys; the state's operand block m is S[4m + quad][c16]
#pragma unroll
        for (int m4 = 0; m4 < KB / 4; ++m4)
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float sb = Sl[4 * (4 * m4 + u) + quad][c16];
                X = mfma(pax[m4][u], sb, X);
                oq = mfma(paq[m4][u], sb, oq);
            }
#pragma unroll
        for (int m4 = 0; m4 < KB / 4; ++m4) {
            pax[m4] = opnd(nbase + L::nBKe, wv, m4, l, KB);
            paq[m4] = opnd(nbase + L::Qe, wv, m4, l, KB);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) xs[wv][r][l] = X[r] + wvv[r];
        __syncthreads();
        // 2. vn for this tile from the X tiles up to it
        float Xkb[16];
#pragma unroll
        for (int mj = 0; mj < 16; ++mj) Xkb[mj] = mj < 4 * wv + 4 ? xs[mj / 4][quad][16 * (mj % 4) + c16] : 0.0f;
        f4 vn = f4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4)
            if (m4 <= wv) {
#pragma unroll
                for (int u = 0; u < 4; ++u) vn = mfma(mi[m4][u], Xkb[4 * m4 + u], vn);
            }
#pragma unroll
        for (int r = 0; r < 4; ++r) vs[wv][r][l] = vn[r];
        __syncthreads();
        // 3. outputs of this tile and this wave's rows of the new state
        float vkb[16];
#pragma unroll
        for (int mj = 0; mj < 16; ++mj) vkb[mj] = vs[mj / 4][quad][16 * (mj % 4) + c16];
#pragma unroll
        for (int m4 = 0; m4 < 4; ++m4)
            if (m4 <= wv) {
#pragma unroll
                for (int u = 0; u < 4; ++u) oq = mfma(pp[m4][u], vkb[4 * m4 + u], oq);
            }
        po = oq;
        pt0 = t0;
        if (upd) {
#pragma unroll
            for (int j = 0; j < TKW; ++j) {
                const int tk = wv * TKW + j;
                f4 sn;
#pragma unroll
                for (int r = 0; r < 4; ++r) sn[r] = eg[j][r] * Sl[16 * tk + 4 * quad + r][c16];
#pragma unroll
                for (int m4 = 0; m4 < 4; ++m4)
#pragma unroll
                    for (int u = 0; u < 4; ++u) sn = mfma(kd[j][m4][u], vkb[4 * m4 + u], sn);
#pragma unroll
                for (int r = 0; r < 4; ++r) Sl[16 * tk + 4 * quad + r][c16] = sn[r];
            }
        }
        __syncthreads();
    }
    store_o();
    if (S_last) {
        for (int e = threadIdx.x; e < K * 16; e += 256) {
            const int kr = e / 16, cc = e % 16;
            S_last[(pair * K + kr) * V + cb * 16 + cc] = Sl[kr][cc];
        }
    }
}

ssm_status check_dims(const ssm_gdn2_dims* d) {
    if (!d) return SSM_E_NULLPTR;
    if (d->batch < 1 || d->heads < 1 || d->seqlen < 0 || d->k_dim < 1 || d->v_dim < 1) return SSM_E_SHAPE;
    if (d->io_dtype != SSM_F32 && d->io_dtype != SSM_BF16) return SSM_E_DTYPE;
    if (d->k_dim != 16 && d->k_dim != 32 && d->k_dim != 64 && d->k_dim != 128) return SSM_E_UNSUPPORTED;
    if (d->v_dim % 16 != 0) return SSM_E_UNSUPPORTED;
    const int64_t nbh = d->batch * d->heads, nch = (d->seqlen + CH - 1) / CH;
    if (d->batch > 65535 || d->heads > 65535 || d->seqlen > ((int64_t)1 << 30) ||
        d->v_dim > ((int64_t)1 << 24) || nbh > 65535 || nch > 65535 ||
        (nbh + XCDS - 1) / XCDS * XCDS * (d->v_dim / 16) >= ((int64_t)1 << 31))
        return SSM_E_UNSUPPORTED;
    return SSM_OK;
}

int64_t chunk_floats(int64_t kd) {
    switch (kd) {
        case 16: return Lay<16>::total;
        case 32: return Lay<32>::total;
        case 64: return Lay<64>::total;
        default: return Lay<128>::total;
    }
}

size_t ws_bytes_for(const ssm_gdn2_dims* d) {
    const int64_t nch = (d->seqlen + CH - 1) / CH;
    return sizeof(float) * (size_t)(d->batch * d->heads * nch * chunk_floats(d->k_dim));
}

template <typename TT, int K>
ssm_status run(const ssm_gdn2_dims* d, const void* q, const void* k, const void* v, const void* g,
               const void* b, const void* w, const float* S0, float scale, void* o, float* S_last,
               float* ws, ssm::Launcher& launch) {
    const int64_t nbh = d->batch * d->heads;
    const int T = (int)d->seqlen, V = (int)d->v_dim;
    const int nch = (T + CH - 1) / CH;
    SSM_TRY(launch(SSM_K_GDN2_WY, k_gdn2_wy<TT, K>, dim3((unsigned)nch, (unsigned)nbh), dim3(WGK), (const TT*)q,
                   (const TT*)k, (const TT*)g, (const TT*)b, ws, T, nch));
    const int64_t nbh8 = (nbh + XCDS - 1) / XCDS * XCDS;
    return launch(SSM_K_GDN2_STATE, k_gdn2_state<TT, K>, dim3((unsigned)(nbh8 * (V / 16))),
                  dim3(256), (const TT*)v,
                  (const TT*)w, (const float*)ws, S0, scale, (TT*)o, S_last, nbh, nbh8, T, V, nch);
}

template <typename TT>
ssm_status run_k(const ssm_gdn2_dims* d, const void* q, const void* k, const void* v, const void* g,
                 const void* b, const void* w, const float* S0, float scale, void* o, float* S_last,
                 float* ws, ssm::Launcher& launch) {
    switch (d->k_dim) {
        case 16: return run<TT, 16>(d, q, k, v, g, b, w, S0, scale, o, S_last, ws, launch);
        case 32: return run<TT, 32>(d, q, k, v, g, b, w, S0, scale, o, S_last, ws, launch);
        case 64: return run<TT, 64>(d, q, k, v, g, b, w, S0, scale, o, S_last, ws, launch);
        default: return run<TT, 128>(d, q, k, v, g, b, w, S0, scale, o, S_last, ws, launch);
    }
}

}  // namespace

extern "C" {

size_t ssm_gdn2_chunked_workspace_bytes(const ssm_gdn2_dims* dims) {
    if (check_dims(dims) != SSM_OK) return 0;
    return ws_bytes_for(dims);
}

ssm_status ssm_gdn2_fwd_chunked(const ssm_gdn2_dims* dims, const void* q, const void* k, const void* v,
                                const void* g, const void* b, const void* w, const float* S0, float scale,
                                void* o, float* S_last, void* ws, size_t ws_bytes, hipStream_t stream,
                                ssm_timing* timing) {
    SSM_TRY(check_dims(dims));
    if (dims->seqlen == 0)  // nothing to chunk: S_last = S0 (or zeros)
        return ssm_gdn2_fwd(dims, q, k, v, g, b, w, S0, scale, o, S_last, stream, timing);
    if (!q || !k || !v || !g || !b || !w || !o) return SSM_E_NULLPTR;
    if (S_last && S_last == S0) return SSM_E_UNSUPPORTED;
    const void* ptrs[] = {q, k, v, g, b, w, S0, o, S_last, ws};
    for (const void* p : ptrs)
        if (p && ssm::misaligned(p)) return SSM_E_ALIGN;
    if (!ws || ws_bytes < ws_bytes_for(dims)) return SSM_E_WORKSPACE;
    (void)hipGetLastError();
    ssm::Launcher launch{stream, timing};
    float* wsf = static_cast<float*>(ws);
    if (dims->io_dtype == SSM_BF16)
        return run_k<ssm::bf16_t>(dims, q, k, v, g, b, w, S0, scale, o, S_last, wsf, launch);
    return run_k<float>(dims, q, k, v, g, b, w, S0, scale, o, S_last, wsf, launch);
}

}  // extern "C"
