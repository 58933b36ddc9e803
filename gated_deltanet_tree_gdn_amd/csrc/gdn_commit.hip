// gdn_commit.hip -- MFMA delayed state commitment for bf16 k/v on gfx950.
//
// What is computed (Trees from Marginals technical summary, Methodology,
// "3. Rollback-Free Tree Verification for GDN", delayed state commitment):
// for the accepted node a of sequence b, the state the GDN delta rule
// reaches when it runs from S0 along the root-to-a path t_1 .. t_m,
//     S_t = alpha_t S_{t-1} + u_t k_t^T,   u_t = beta_t (v_t - alpha_t S_{t-1} k_t).
// Only rows of S (value index c) interact with themselves, so one workgroup
// owns one (sequence, value head) state and keeps it in registers from load
// to store.
//
// The path is processed in chunks of 16 nodes.  For a chunk entered with
// state S and chunk-relative cumulative log-gates G_t (gamma_t = exp(G_t),
// D_ts = exp(G_t - G_s)), the same closed form the verify uses restricted
// to one path gives
//     (I + X) U = R,  X_ts = beta_t D_ts (k_t . k_s) (s < t),
//     R_t = beta_t (v_t - gamma_t S k_t),
//     S <- gamma_n S + sum_s D_ns u_s k_s^T          (n the chunk's last node),
// with S k_t (P), k_t . k_s (the Gram) and the rank-16 update on
// v_mfma_f32_16x16x32_bf16 (k exact bf16; S and U split into bf16 hi + lo)
// and the 16 x 16 triangular solve by one lane per value column.
//
// Layout: wavefront w owns value rows c in [w d_v/4, (w+1) d_v/4) as
// d_v/64 column tiles; its registers hold S[c][j] for 16 columns c and
// j = 32 jp + 16 hf + 4 (l / 16) + r, which is at once the B operand of
// S k_t (the k-slot order of k matches) and the accumulator layout of the
// update S[c][j] += sum_s U[s][c] k_s[j] (M = j, N = c).  Each load and
// store moves 64 contiguous bytes of 16 state rows.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"
#include "gdn_mfma.h"
#include "gdn_walk.h"

namespace gdn {
namespace {

constexpr int kChunk = 16;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <int DK, int DV>
__global__ __launch_bounds__(256, 4) void commit_mfma_kernel(CommitArgs a) {
    constexpr int CTW = DV / 64;    // column tiles per wavefront
    constexpr int JP = DK / 32;     // 32-wide k steps
    constexpr int CW = DV / 4;      // value rows per wavefront
    constexpr int KROW = DK + 8;    // staged k row (bf16), padded
    constexpr int KTROW = kChunk + 8;
    constexpr int VTROW = kChunk + 4;
    constexpr int XROW = kChunk + 4;
    constexpr int RROW = kChunk + 4;

    __shared__ int par_s[kMaxN];
    __shared__ int path_s[kMaxN];       // accepted .. root
    __shared__ float gl_s[kMaxN];       // chunk-relative cumulative log-gate, root-first index
    __shared__ float bl_s[kMaxN];       // beta, root-first index
    __shared__ int misc_s[2];
    __shared__ __align__(16) uint16_t kc_s[kChunk][KROW];   // k rows of the chunk
    __shared__ __align__(16) uint16_t kt_s[DK][KTROW];      // the same, transposed
    __shared__ __align__(16) uint16_t vt_s[DV][VTROW];      // v of the head, transposed
    __shared__ __align__(16) float x_s[4][kChunk][XROW];    // X, one copy per wavefront
    __shared__ __align__(16) float rt_s[4][CW][RROW];       // R, then D_ns u_s, per value row

    const int N = a.N, Hv = a.H_v, Hk = a.H_k;
    const int h = blockIdx.x % Hv;
    const int b = blockIdx.x / Hv;
    const int kh = h / (Hv / Hk);
    const int tid = threadIdx.x;
    const int w = tid >> 6, l = tid & 63, lc = l & 15, g = l >> 4;
    const uint16_t* __restrict__ kp = static_cast<const uint16_t*>(a.k);
    const uint16_t* __restrict__ vp = static_cast<const uint16_t*>(a.v);

    // S0 rows of this wavefront, in the fragment layout described above.
    f32x4 S[CTW][JP][2];
    {
        const float* s0 = a.S0 + (static_cast<size_t>(b) * Hv + h) * DV * DK;
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const float* row = s0 + static_cast<size_t>(w * CW + 16 * ct + lc) * DK + 4 * g;
#pragma unroll
            for (int jp = 0; jp < JP; ++jp)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) S[ct][jp][hf] = *reinterpret_cast<const f32x4*>(row + 32 * jp + 16 * hf);
        }
    }

    // Parents (an entry outside [-1, i-1] ends the walk there) and the
    // accepted node (out of range: reported, then treated as -1).
    if (tid < N) {
        int p = a.parent[static_cast<size_t>(b) * N + tid];
        if (p < -1 || p >= tid) p = -1;
        par_s[tid] = p;
    }
    if (tid == 0) {
        int acc = a.accepted[b];
        const bool bad = acc < -1 || acc >= N;
        if (bad) acc = -1;
        if (h == 0) a.accept_status[b] = bad ? GDN_ERR_ACCEPT : 0;
        misc_s[0] = acc;
    }
    __syncthreads();
    if (tid == 0) {
        int m = 0;
        for (int s = misc_s[0]; s >= 0; s = par_s[s]) path_s[m++] = s;
        misc_s[1] = m;
    }
    __syncthreads();
    const int m = misc_s[1];

    // Gates along the path, cumulative within each chunk: one load per
    // path node, then an inclusive scan over the chunk's 16 lanes.
    {
        float G = 0.f, bt = 0.f;
        if (tid < m) {
            const size_t nh = (static_cast<size_t>(b) * N + path_s[m - 1 - tid]) * Hv + h;
            G = a.g[nh];
            bt = a.beta[nh];
        }
#pragma unroll
        for (int o = 1; o < kChunk; o <<= 1) {
            const float x = __shfl_up(G, o, kChunk);
            if ((l & (kChunk - 1)) >= o) G += x;
        }
        if (tid < m) {
            gl_s[tid] = G;
            bl_s[tid] = bt;
        }
    }

    auto stage = [&](int c0, int n) {
        for (int e = tid; e < kChunk * (DK / 8); e += 256) {
            const int t = e / (DK / 8), p = e % (DK / 8);
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (t < n) {
                const int node = path_s[m - 1 - (c0 + t)];
                val = *reinterpret_cast<const uint4*>(kp + ((static_cast<size_t>(b) * N + node) * Hk + kh) * DK + 8 * p);
            }
            *reinterpret_cast<uint4*>(&kc_s[t][8 * p]) = val;
            const uint32_t wd[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                kt_s[8 * p + 2 * q][t] = static_cast<uint16_t>(wd[q] & 0xffffu);
                kt_s[8 * p + 2 * q + 1][t] = static_cast<uint16_t>(wd[q] >> 16);
            }
        }
        for (int e = tid; e < kChunk * (DV / 8); e += 256) {
            const int t = e / (DV / 8), p = e % (DV / 8);
            uint4 val = make_uint4(0u, 0u, 0u, 0u);
            if (t < n) {
                const int node = path_s[m - 1 - (c0 + t)];
                val = *reinterpret_cast<const uint4*>(vp + ((static_cast<size_t>(b) * N + node) * Hv + h) * DV + 8 * p);
            }
            const uint32_t wd[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                vt_s[8 * p + 2 * q][t] = static_cast<uint16_t>(wd[q] & 0xffffu);
                vt_s[8 * p + 2 * q + 1][t] = static_cast<uint16_t>(wd[q] >> 16);
            }
        }
    };

    if (m > 0) stage(0, m < kChunk ? m : kChunk);

    float* xw = &x_s[w][0][0];
    float* rw = &rt_s[w][0][0];
    for (int c0 = 0; c0 < m; c0 += kChunk) {
        const int n = m - c0 < kChunk ? m - c0 : kChunk;
        if (c0 > 0) {
            __syncthreads();
            stage(c0, n);
        }
        __syncthreads();
        const float* Gc = gl_s + c0;
        const float* Bc = bl_s + c0;

        bf16x8 ak[JP];
#pragma unroll
        for (int jp = 0; jp < JP; ++jp) ak[jp] = load_frag2(&kc_s[lc][32 * jp + 4 * g], &kc_s[lc][32 * jp + 16 + 4 * g]);

        // X_ts = beta_t D_ts (k_t . k_s) for s < t < n; D layout: t = 4g + r, s = lc.
        {
            f32x4 gr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jp = 0; jp < JP; ++jp) gr = mfma(ak[jp], ak[jp], gr);
            const float Gs = Gc[lc < n ? lc : n - 1];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g + r;
                float x = 0.f;
                if (lc < t && t < n) x = Bc[t] * __expf(Gc[t] - Gs) * gr[r];
                xw[t * XROW + lc] = x;
            }
        }

        // R_t = beta_t (v_t - gamma_t S k_t): P tile has t = 4g + r, c = lc.
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            f32x4 p = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int jp = 0; jp < JP; ++jp) {
                const float x8[8] = {S[ct][jp][0][0], S[ct][jp][0][1], S[ct][jp][0][2], S[ct][jp][0][3],
                                     S[ct][jp][1][0], S[ct][jp][1][1], S[ct][jp][1][2], S[ct][jp][1][3]};
                bf16x8 hi, lo;
                split8(x8, hi, lo);
                p = mfma(ak[jp], hi, p);
                p = mfma(ak[jp], lo, p);
            }
            const int cl = 16 * ct + lc;
            const uint2 vv = *reinterpret_cast<const uint2*>(&vt_s[w * CW + cl][4 * g]);
            const float v4[4] = {bf16_lo(vv.x), bf16_hi(vv.x), bf16_lo(vv.y), bf16_hi(vv.y)};
            f32x4 R;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * g + r;
                const int tc = t < n ? t : n - 1;
                R[r] = t < n ? Bc[tc] * (v4[r] - __expf(Gc[tc]) * p[r]) : 0.f;
            }
            *reinterpret_cast<f32x4*>(rw + cl * RROW + 4 * g) = R;
        }
        WaveSync::sync();

        // (I + X) U = R by forward substitution, one lane per value row;
        // then u_s <- D_ns u_s.
        if (l < CW) {
            float u[kChunk];
#pragma unroll
            for (int q = 0; q < kChunk / 4; ++q) {
                const f32x4 t4 = *reinterpret_cast<const f32x4*>(rw + l * RROW + 4 * q);
                u[4 * q + 0] = t4[0];
                u[4 * q + 1] = t4[1];
                u[4 * q + 2] = t4[2];
                u[4 * q + 3] = t4[3];
            }
#pragma unroll
            for (int t = 1; t < kChunk; ++t) {
                // one row of X at a time keeps register use flat (the
                // opaque offset stops the loads being hoisted)
                int xo = t * XROW;
                asm volatile("" : "+v"(xo));
                float xr[kChunk];
#pragma unroll
                for (int q = 0; q < (t + 3) / 4; ++q) {
                    const f32x4 x4 = *reinterpret_cast<const f32x4*>(xw + xo + 4 * q);
                    xr[4 * q + 0] = x4[0];
                    xr[4 * q + 1] = x4[1];
                    xr[4 * q + 2] = x4[2];
                    xr[4 * q + 3] = x4[3];
                }
                float acc = u[t];
#pragma unroll
                for (int s = 0; s < t; ++s) acc -= xr[s] * u[s];
                asm volatile("" : "+v"(acc));
                u[t] = acc;
            }
            const float Gn = Gc[n - 1];
#pragma unroll
            for (int s = 0; s < kChunk; ++s) u[s] = s < n ? u[s] * __expf(Gn - Gc[s < n ? s : n - 1]) : 0.f;
#pragma unroll
            for (int q = 0; q < kChunk / 4; ++q) {
                const f32x4 t4 = {u[4 * q + 0], u[4 * q + 1], u[4 * q + 2], u[4 * q + 3]};
                *reinterpret_cast<f32x4*>(rw + l * RROW + 4 * q) = t4;
            }
        }
        WaveSync::sync();

        // S <- gamma_n S + sum_s U[s][c] k_s[j]: B lane (c = lc, g) carries
        // s = 8 (g & 1) .. + 7, the hi parts for g < 2 and the lo parts above.
        const float gam = __expf(Gc[n - 1]);
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            const float* ur = rw + (16 * ct + lc) * RROW + 8 * (g & 1);
            const f32x4 u0 = *reinterpret_cast<const f32x4*>(ur);
            const f32x4 u1 = *reinterpret_cast<const f32x4*>(ur + 4);
            const float x8[8] = {u0[0], u0[1], u0[2], u0[3], u1[0], u1[1], u1[2], u1[3]};
            bf16x8 bu;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float hi = static_cast<float>(static_cast<__bf16>(x8[e]));
                bu[e] = static_cast<__bf16>(g < 2 ? x8[e] : x8[e] - hi);
            }
#pragma unroll
            for (int jp = 0; jp < JP; ++jp)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const bf16x8 at = load_frag(&kt_s[32 * jp + 16 * hf + lc][8 * (g & 1)]);
                    S[ct][jp][hf] = mfma(at, bu, S[ct][jp][hf] * gam);
                }
        }
    }

    {
        float* sn = a.S_new + (static_cast<size_t>(b) * Hv + h) * DV * DK;
#pragma unroll
        for (int ct = 0; ct < CTW; ++ct) {
            float* row = sn + static_cast<size_t>(w * CW + 16 * ct + lc) * DK + 4 * g;
#pragma unroll
            for (int jp = 0; jp < JP; ++jp)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) *reinterpret_cast<f32x4*>(row + 32 * jp + 16 * hf) = S[ct][jp][hf];
        }
    }
}

template <int DK, int DV>
hipError_t commit_mfma(const CommitArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B) * a.H_v);
    hipLaunchKernelGGL((commit_mfma_kernel<DK, DV>), grid, dim3(256), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_commit(const CommitArgs& a, hipStream_t stream) {
    if (a.qkv_dtype != GDN_BF16 || a.force_walk) return launch_commit_simple(a, stream);
    if (a.d_k == 64) return a.d_v == 64 ? commit_mfma<64, 64>(a, stream) : commit_mfma<64, 128>(a, stream);
    return a.d_v == 64 ? commit_mfma<128, 64>(a, stream) : commit_mfma<128, 128>(a, stream);
}

}  // namespace gdn
