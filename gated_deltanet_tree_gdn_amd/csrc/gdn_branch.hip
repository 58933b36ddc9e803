// gdn_branch.hip -- per-branch recurrent tree verification: the baseline the
// fused, rollback-free verification is measured against (Trees from
// Marginals technical summary, Experimental Results: the fused kernel is
// 7.1x faster than per-branch recurrent verification at tree size 128;
// wispaper.ai page, "Systems Innovation: Fused GDN Verification").
//
// Every root-to-leaf branch of the tree is verified as its own sequence:
// a fresh copy of S0 is advanced token by token along the branch with the
// Gated DeltaNet update
//     S <- alpha_t S (I - beta_t k_t k_t^T) + beta_t v_t k_t^T = alpha_t S + u_t k_t^T,
//     u_t = beta_t (v_t - alpha_t S k_t),   o_t = S q_t,
// so a node shared by several branches is recomputed once per branch (the
// redundancy, and the rollback of per-branch states, that the fused solve
// avoids).  The result equals the fused verify's.
//
// Work decomposition: one workgroup per (sequence, value head, slice of the
// leaves); each row c of the state is split over two adjacent lanes, d_k / 2
// fp32 registers each (a whole row per lane would take every register and
// leave one wavefront per SIMD), so S k and S q are per-lane dot products
// over half a row plus one exchange with the neighbour lane.  k_t and q_t go
// through LDS once per step and are read as broadcasts.  Each node's output
// is written by exactly one branch: the one ending at the lowest-index leaf
// below it, so the branches never race on o.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"

namespace gdn {
namespace {

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) { return __uint_as_float(static_cast<uint32_t>(*p) << 16); }
template <>
__device__ __forceinline__ float ld<float>(const float* p) { return *p; }

// x plus the value of the neighbour lane (lane ^ 1)
__device__ __forceinline__ float pair_sum(float x) {
    return x + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(2 * DV, 2) void branch_kernel(VerifyArgs a, int splits) {
    constexpr int NT = 2 * DV;   // threads: two per state row
    constexpr int DH = DK / 2;   // state columns per lane
    __shared__ int par[kMaxN], minleaf[kMaxN], leaves[kMaxN], path[kMaxN];
    __shared__ int nleaf_s, plen_s, bad_s;
    __shared__ __align__(16) float kv[DK], qv[DK];
    const int N = a.N, Hv = a.H_v, Hk = a.H_k;
    const int split = blockIdx.x % splits;
    const int unit = blockIdx.x / splits;
    const int b = unit / Hv, h = unit % Hv, kh = h / (Hv / Hk);
    const int tid = threadIdx.x;
    const int c = tid >> 1, hf = tid & 1;   // state row c, columns DH hf ..
    const T* qg = static_cast<const T*>(a.q);
    const T* kg = static_cast<const T*>(a.k);
    const T* vg = static_cast<const T*>(a.v);

    // parents (an entry outside [-1, i-1] is read as -1; the fused verify
    // reports it), leaves, and for every node the lowest-index leaf below it
    if (tid == 0) bad_s = 0;
    __syncthreads();
    for (int i = tid; i < N; i += NT) {
        const int p = a.parent[static_cast<size_t>(b) * N + i];
        const bool bad = p < -1 || p >= i;
        par[i] = bad ? -1 : p;
        minleaf[i] = 0x7fffffff;
        if (bad) bad_s = 1;
    }
    __syncthreads();
    if (h == 0 && split == 0 && tid == 0) a.tree_status[b] = bad_s ? GDN_ERR_TREE : 0;
    if (tid == 0) {
        // children follow their parents, so one backward pass sees every
        // node's subtree complete before the node itself
        for (int i = N - 1; i >= 0; --i) {
            if (minleaf[i] == 0x7fffffff) minleaf[i] = i;   // no child: a leaf
            const int p = par[i];
            if (p >= 0) minleaf[p] = min(minleaf[p], minleaf[i]);
        }
        int n = 0;
        for (int i = 0; i < N; ++i)
            if (minleaf[i] == i) leaves[n++] = i;
        nleaf_s = n;
    }
    __syncthreads();
    const int nleaf = nleaf_s;
    const float* S0 = a.S0 + ((static_cast<size_t>(b) * Hv + h) * DV + c) * DK + DH * hf;

    for (int li = split; li < nleaf; li += splits) {
        const int leaf = leaves[li];
        __syncthreads();   // the previous branch's path is read
        if (tid == 0) {
            int m = 0;
            for (int s = leaf; s >= 0; s = par[s]) path[m++] = s;
            plen_s = m;
        }
        __syncthreads();
        const int m = plen_s;
        float S[DH];
#pragma unroll
        for (int j = 0; j < DH; j += 4) {
            const float4 x = *reinterpret_cast<const float4*>(S0 + j);
            S[j] = x.x;
            S[j + 1] = x.y;
            S[j + 2] = x.z;
            S[j + 3] = x.w;
        }
        // root first: path[m-1] .. path[0]; the next node's inputs are
        // loaded while the current one is applied
        constexpr int KPT = (DK + NT - 1) / NT;   // k / q elements per thread
        float pk[KPT], pq[KPT], pg = 0.f, pb = 0.f, pv = 0.f;
        auto prefetch = [&](int t) {
            const int i = path[t];
            const size_t nk = ((static_cast<size_t>(b) * N + i) * Hk + kh) * DK;
            const size_t nh = (static_cast<size_t>(b) * N + i) * Hv + h;
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const int j = tid + e * NT;
                pk[e] = j < DK ? ld(kg + nk + j) : 0.f;
                pq[e] = j < DK ? ld(qg + nk + j) : 0.f;
            }
            pg = a.g[nh];
            pb = a.beta[nh];
            pv = ld(vg + nh * DV + c);
        };
        if (m > 0) prefetch(m - 1);
        for (int t = m - 1; t >= 0; --t) {
            const int i = path[t];
            const size_t nh = (static_cast<size_t>(b) * N + i) * Hv + h;
            __syncthreads();   // the previous step's k, q are read
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const int j = tid + e * NT;
                if (j < DK) {
                    kv[j] = pk[e];
                    qv[j] = pq[e];
                }
            }
            const float alpha = __expf(pg);
            const float beta = pb;
            const float vc = pv;
            __syncthreads();
            if (t > 0) prefetch(t - 1);
            const float* kh_ = kv + DH * hf;
            const float* qh_ = qv + DH * hf;
            float sk = 0.f;
#pragma unroll
            for (int j = 0; j < DH; ++j) sk += S[j] * kh_[j];
            sk = pair_sum(sk);
            const float u = beta * (vc - alpha * sk);
            float o = 0.f;
#pragma unroll
            for (int j = 0; j < DH; ++j) {
                S[j] = alpha * S[j] + u * kh_[j];
                o += S[j] * qh_[j];
            }
            o = pair_sum(o);
            if (hf == 0 && minleaf[i] == leaf) a.o[nh * DV + c] = o;
        }
    }
}

template <typename T>
hipError_t go(const VerifyArgs& a, hipStream_t stream, int splits) {
    const dim3 grid(static_cast<unsigned>(a.B) * a.H_v * splits);
    if (a.d_k == 64) {
        if (a.d_v == 64) hipLaunchKernelGGL((branch_kernel<T, 64, 64>), grid, dim3(128), 0, stream, a, splits);
        else hipLaunchKernelGGL((branch_kernel<T, 64, 128>), grid, dim3(256), 0, stream, a, splits);
    } else {
        if (a.d_v == 64) hipLaunchKernelGGL((branch_kernel<T, 128, 64>), grid, dim3(128), 0, stream, a, splits);
        else hipLaunchKernelGGL((branch_kernel<T, 128, 128>), grid, dim3(256), 0, stream, a, splits);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_branches(const VerifyArgs& a, hipStream_t stream) {
    // enough workgroups to fill the device several times over
    const int units = a.B * a.H_v;
    int splits = 1;
    while (splits < 16 && units * splits < 8 * device_cus()) splits *= 2;
    return a.qkv_dtype == GDN_BF16 ? go<uint16_t>(a, stream, splits) : go<float>(a, stream, splits);
}

}  // namespace gdn
