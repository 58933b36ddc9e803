// gdn_walk.h -- per-node walk of the tree, one wavefront per 64-column slice.
//
// Nodes are visited in topological order; for node i the wave walks the
// parent chain and applies
//
//   u_i = beta_i (v_i - gamma_i S0 k_i - sum_{s in P°(i)} D_is (k_i.k_s) u_s)
//   o_i = gamma_i S0 q_i + sum_{s in P(i)} D_is (q_i.k_s) u_s
//
// (G_i the path-cumulative log-gate, gamma_i = exp(G_i), D_is = exp(G_i - G_s)):
// the per-node form of the masked triangular solve (I + X) U = beta (V -
// gamma K S0^T), O = gamma Q S0^T + Y U of the Trees from Marginals technical
// summary (Methodology, "3. Rollback-Free Tree Verification for GDN").  Only
// ancestor pairs are touched, so masked entries are exact zeros.
//
// Lane c of the wave owns value column c0 + c.  The caller provides the LDS
// buffers and the synchronisation policy (a block barrier when the wave is
// the whole workgroup, a wave-local fence when it is one wave of a larger
// workgroup whose other waves have left).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"

namespace gdn {

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(uint16_t x) { return __uint_as_float(static_cast<uint32_t>(x) << 16); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}

struct BlockSync {
    __device__ static void sync() { __syncthreads(); }
};

struct WaveSync {
    __device__ static void sync() {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront", "local");
    }
};

// One 64-column slice [c0, c0 + 64) of o for sequence b, value head h.
//   par_s : parents of the N nodes (already validated: each in [-1, i-1])
//   u_s   : [N][64] floats,  G_s: [N] floats,  ki_s, qi_s: [DK] floats
template <typename T, int DK, class Sync>
__device__ void walk_verify_slice(const VerifyArgs& a, int b, int h, int c0, const int* par_s, float* u_s,
                                  float* G_s, float* ki_s, float* qi_s) {
    const int N = a.N, Hv = a.H_v, Hk = a.H_k, DV = a.d_v;
    const int kh = h / (Hv / Hk);
    const int lane = threadIdx.x & 63;
    const int c = c0 + lane;
    const T* __restrict__ q = static_cast<const T*>(a.q);
    const T* __restrict__ k = static_cast<const T*>(a.k);
    const T* __restrict__ v = static_cast<const T*>(a.v);

    float srow[DK];
    {
        const float4* src = reinterpret_cast<const float4*>(a.S0 + ((static_cast<size_t>(b) * Hv + h) * DV + c) * DK);
#pragma unroll
        for (int j = 0; j < DK / 4; ++j) {
            const float4 t = src[j];
            srow[4 * j + 0] = t.x;
            srow[4 * j + 1] = t.y;
            srow[4 * j + 2] = t.z;
            srow[4 * j + 3] = t.w;
        }
    }

    for (int i = 0; i < N; ++i) {
        const int p = par_s[i];
        const size_t nh = (static_cast<size_t>(b) * N + i) * Hv + h;
        const float bi = a.beta[nh];
        const float Gi = (p < 0 ? 0.f : G_s[p]) + a.g[nh];
        const size_t krow = ((static_cast<size_t>(b) * N + i) * Hk + kh) * DK;
        for (int j = lane; j < DK; j += 64) {
            ki_s[j] = to_f32(k[krow + j]);
            qi_s[j] = to_f32(q[krow + j]);
        }
        Sync::sync();
        if (lane == 0) G_s[i] = Gi;

        float sk = 0.f, sq = 0.f;
#pragma unroll
        for (int j = 0; j < DK; ++j) {
            sk += srow[j] * ki_s[j];
            sq += srow[j] * qi_s[j];
        }
        float self_qk = 0.f;
        for (int j = lane; j < DK; j += 64) self_qk += qi_s[j] * ki_s[j];
        self_qk = wave_sum(self_qk);

        float acc_u = 0.f, acc_o = 0.f;
        for (int s = p; s >= 0; s = par_s[s]) {
            const size_t srow_k = ((static_cast<size_t>(b) * N + s) * Hk + kh) * DK;
            float pk = 0.f, pq = 0.f;
            for (int j = lane; j < DK; j += 64) {
                const float ks = to_f32(k[srow_k + j]);
                pk += ki_s[j] * ks;
                pq += qi_s[j] * ks;
            }
            pk = wave_sum(pk);
            pq = wave_sum(pq);
            const float D = __expf(Gi - G_s[s]);
            const float us = u_s[s * 64 + lane];
            acc_u += D * pk * us;
            acc_o += D * pq * us;
        }
        const float gam = __expf(Gi);
        const float vi = to_f32(v[nh * DV + c]);
        const float ui = bi * (vi - gam * sk - acc_u);
        u_s[i * 64 + lane] = ui;
        a.o[nh * DV + c] = gam * sq + acc_o + self_qk * ui;
        Sync::sync();
    }
}

// The same walk with the slice's S0 rows staged in LDS (s0_s: [DK][64],
// column-major so lane c reads consecutive words) instead of registers, for
// use inside kernels whose register budget is set by other work; with
// s0_s == nullptr each lane reads its S0 row from global memory instead
// (for kernels whose LDS budget is set by other work).
template <typename T, int DK, class Sync>
__device__ void walk_verify_slice_lds(const VerifyArgs& a, int b, int h, int c0, const int* par_s, float* u_s,
                                      float* G_s, float* ki_s, float* qi_s, float* s0_s) {
    const int N = a.N, Hv = a.H_v, Hk = a.H_k, DV = a.d_v;
    const int kh = h / (Hv / Hk);
    const int lane = threadIdx.x & 63;
    const int c = c0 + lane;
    const T* __restrict__ q = static_cast<const T*>(a.q);
    const T* __restrict__ k = static_cast<const T*>(a.k);
    const T* __restrict__ v = static_cast<const T*>(a.v);

    const float* S0row = a.S0 + ((static_cast<size_t>(b) * Hv + h) * DV + c) * DK;
    if (s0_s) {
        for (int j = 0; j < DK; ++j) s0_s[j * 64 + lane] = S0row[j];
        Sync::sync();
    }

    for (int i = 0; i < N; ++i) {
        const int p = par_s[i];
        const size_t nh = (static_cast<size_t>(b) * N + i) * Hv + h;
        const float bi = a.beta[nh];
        const float Gi = (p < 0 ? 0.f : G_s[p]) + a.g[nh];
        const size_t krow = ((static_cast<size_t>(b) * N + i) * Hk + kh) * DK;
        for (int j = lane; j < DK; j += 64) {
            ki_s[j] = to_f32(k[krow + j]);
            qi_s[j] = to_f32(q[krow + j]);
        }
        Sync::sync();
        if (lane == 0) G_s[i] = Gi;

        // two loops, so that each source keeps its address space (one
        // pointer that may be either would take generic loads)
        float sk = 0.f, sq = 0.f;
        if (s0_s) {
            for (int j = 0; j < DK; ++j) {
                const float sv = s0_s[j * 64 + lane];
                sk += sv * ki_s[j];
                sq += sv * qi_s[j];
            }
        } else {
            for (int j = 0; j < DK; ++j) {
                const float sv = S0row[j];
                sk += sv * ki_s[j];
                sq += sv * qi_s[j];
            }
        }
        float self_qk = 0.f;
        for (int j = lane; j < DK; j += 64) self_qk += qi_s[j] * ki_s[j];
        self_qk = wave_sum(self_qk);

        float acc_u = 0.f, acc_o = 0.f;
        for (int s = p; s >= 0; s = par_s[s]) {
            const size_t srow_k = ((static_cast<size_t>(b) * N + s) * Hk + kh) * DK;
            float pk = 0.f, pq = 0.f;
            for (int j = lane; j < DK; j += 64) {
                const float ks = to_f32(k[srow_k + j]);
                pk += ki_s[j] * ks;
                pq += qi_s[j] * ks;
            }
            pk = wave_sum(pk);
            pq = wave_sum(pq);
            const float D = __expf(Gi - G_s[s]);
            const float us = u_s[s * 64 + lane];
            acc_u += D * pk * us;
            acc_o += D * pq * us;
        }
        const float gam = __expf(Gi);
        const float vi = to_f32(v[nh * DV + c]);
        const float ui = bi * (vi - gam * sk - acc_u);
        u_s[i * 64 + lane] = ui;
        a.o[nh * DV + c] = gam * sq + acc_o + self_qk * ui;
        Sync::sync();
    }
}

}  // namespace gdn
