// gdn_simple.hip -- straightforward gfx950 kernels for GDN tree verification:
// the general verify path (any dtype, d in {64, 128}, N <= 256), the
// accepted-path commit and the ancestor-set export.
//
// Verify: one 64-lane wavefront per (sequence b, value head h, 64-column
// slice of d_v) running the per-node walk of gdn_walk.h.
// Commit: the same per-node update restricted to the root-to-accepted path,
// then S_new = gamma_a S0 + sum_{s on the path} D_as u_s k_s^T (the delayed
// state commitment of the Trees from Marginals technical summary, Methodology,
// "3. Rollback-Free Tree Verification for GDN").

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"
#include "gdn_walk.h"

namespace gdn {
namespace {

// Loads parent[b][:] into LDS, replacing any entry outside [-1, i-1] by -1
// (so every parent walk terminates in bounds); returns 1 if one was invalid.
__device__ int load_parents(const int32_t* __restrict__ parent, int N, int* par_s, int* bad_s) {
    const int lane = threadIdx.x;
    if (lane == 0) *bad_s = 0;
    __syncthreads();
    for (int i = lane; i < N; i += 64) {
        int p = parent[i];
        if (p < -1 || p >= i) {
            *bad_s = 1;
            p = -1;
        }
        par_s[i] = p;
    }
    __syncthreads();
    return *bad_s;
}

template <typename T, int DK>
__global__ __launch_bounds__(64) void verify_simple_kernel(VerifyArgs a) {
    const int N = a.N, Hv = a.H_v;
    const int nslice = a.d_v / 64;
    int blk = blockIdx.x;
    const int slice = blk % nslice;
    blk /= nslice;
    const int h = blk % Hv;
    const int b = blk / Hv;

    __shared__ float u_s[kMaxN * 64];
    __shared__ float G_s[kMaxN];
    __shared__ int par_s[kMaxN];
    __shared__ float ki_s[DK];
    __shared__ float qi_s[DK];
    __shared__ int bad_s;

    const int bad = load_parents(a.parent + static_cast<size_t>(b) * N, N, par_s, &bad_s);
    if (h == 0 && slice == 0 && threadIdx.x == 0) a.tree_status[b] = bad ? GDN_ERR_TREE : 0;
    walk_verify_slice<T, DK, BlockSync>(a, b, h, slice * 64, par_s, u_s, G_s, ki_s, qi_s);
}

template <typename T, int DK>
__global__ __launch_bounds__(64) void commit_simple_kernel(CommitArgs a) {
    const int N = a.N, Hv = a.H_v, Hk = a.H_k, DV = a.d_v;
    const int nslice = DV / 64;
    int blk = blockIdx.x;
    const int slice = blk % nslice;
    blk /= nslice;
    const int h = blk % Hv;
    const int b = blk / Hv;
    const int kh = h / (Hv / Hk);
    const int lane = threadIdx.x;
    const int c = slice * 64 + lane;

    __shared__ float u_s[kMaxN][64];
    __shared__ float G_s[kMaxN];
    __shared__ int par_s[kMaxN];
    __shared__ int path_s[kMaxN];
    __shared__ float ks_s[DK];
    __shared__ int bad_s;
    __shared__ int len_s;

    load_parents(a.parent + static_cast<size_t>(b) * N, N, par_s, &bad_s);
    int acc = a.accepted[b];
    const bool bad_acc = acc < -1 || acc >= N;
    if (bad_acc) acc = -1;
    if (h == 0 && slice == 0 && lane == 0) a.accept_status[b] = bad_acc ? GDN_ERR_ACCEPT : 0;
    if (lane == 0) {
        int len = 0;
        for (int s = acc; s >= 0; s = par_s[s]) path_s[len++] = s;
        for (int l = 0, r = len - 1; l < r; ++l, --r) {
            const int t = path_s[l];
            path_s[l] = path_s[r];
            path_s[r] = t;
        }
        len_s = len;
    }
    __syncthreads();
    const int L = len_s;

    const T* __restrict__ k = static_cast<const T*>(a.k);
    const T* __restrict__ v = static_cast<const T*>(a.v);

    float srow[DK];
    const size_t row_off = ((static_cast<size_t>(b) * Hv + h) * DV + c) * DK;
    {
        const float4* src = reinterpret_cast<const float4*>(a.S0 + row_off);
#pragma unroll
        for (int j = 0; j < DK / 4; ++j) {
            float4 t = src[j];
            srow[4 * j + 0] = t.x;
            srow[4 * j + 1] = t.y;
            srow[4 * j + 2] = t.z;
            srow[4 * j + 3] = t.w;
        }
    }

    // u along the accepted path (identical to the verify's u for these nodes)
    for (int t = 0; t < L; ++t) {
        const int s = path_s[t];
        const size_t nh = (static_cast<size_t>(b) * N + s) * Hv + h;
        const float Gs = (t == 0 ? 0.f : G_s[t - 1]) + a.g[nh];
        const float bs = a.beta[nh];
        const size_t krow = ((static_cast<size_t>(b) * N + s) * Hk + kh) * DK;
        for (int j = lane; j < DK; j += 64) ks_s[j] = to_f32(k[krow + j]);
        __syncthreads();
        if (lane == 0) G_s[t] = Gs;
        float sk = 0.f;
#pragma unroll
        for (int j = 0; j < DK; ++j) sk += srow[j] * ks_s[j];
        float acc_u = 0.f;
        for (int t2 = 0; t2 < t; ++t2) {
            const int s2 = path_s[t2];
            const size_t krow2 = ((static_cast<size_t>(b) * N + s2) * Hk + kh) * DK;
            float pk = 0.f;
            for (int j = lane; j < DK; j += 64) pk += ks_s[j] * to_f32(k[krow2 + j]);
            pk = wave_sum(pk);
            acc_u += __expf(Gs - G_s[t2]) * pk * u_s[t2][lane];
        }
        const float ui = bs * (to_f32(v[nh * DV + c]) - __expf(Gs) * sk - acc_u);
        u_s[t][lane] = ui;
        __syncthreads();
    }

    // S_new row c = gamma_a S0 row c + sum_t D_a,path[t] u_t[c] k_path[t]
    const float Ga = L ? G_s[L - 1] : 0.f;
    const float gam_a = __expf(Ga);
    if (L) {
#pragma unroll
        for (int j = 0; j < DK; ++j) srow[j] *= gam_a;
    }
    for (int t = 0; t < L; ++t) {
        const int s = path_s[t];
        const size_t krow = ((static_cast<size_t>(b) * N + s) * Hk + kh) * DK;
        for (int j = lane; j < DK; j += 64) ks_s[j] = to_f32(k[krow + j]);
        __syncthreads();
        const float w = __expf(Ga - G_s[t]) * u_s[t][lane];
#pragma unroll
        for (int j = 0; j < DK; ++j) srow[j] += w * ks_s[j];
        __syncthreads();
    }
    float4* dst = reinterpret_cast<float4*>(a.S_new + row_off);
#pragma unroll
    for (int j = 0; j < DK / 4; ++j) dst[j] = make_float4(srow[4 * j], srow[4 * j + 1], srow[4 * j + 2], srow[4 * j + 3]);
}

// One workgroup per sequence, one thread per node: walk the parent chain.
__global__ __launch_bounds__(256) void ancestors_kernel(int N, const int32_t* __restrict__ parent,
                                                        uint32_t* __restrict__ anc, int32_t* __restrict__ depth,
                                                        int32_t* __restrict__ tree_status) {
    const int b = blockIdx.x;
    const int W = (N + 31) / 32;
    __shared__ int par_s[kMaxN];
    __shared__ uint32_t rows[kMaxN][kMaxN / 32];
    __shared__ int bad_s;
    if (threadIdx.x == 0) bad_s = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        int p = parent[static_cast<size_t>(b) * N + i];
        if (p < -1 || p >= i) {
            bad_s = 1;
            p = -1;
        }
        par_s[i] = p;
#pragma unroll
        for (int w = 0; w < kMaxN / 32; ++w) rows[i][w] = 0u;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < N; i += blockDim.x) {
        int d = 0;
        for (int s = i; s >= 0; s = par_s[s]) {
            rows[i][s >> 5] |= 1u << (s & 31);
            ++d;
        }
        depth[static_cast<size_t>(b) * N + i] = d;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < N * W; e += blockDim.x) anc[static_cast<size_t>(b) * N * W + e] = rows[e / W][e % W];
    if (threadIdx.x == 0 && tree_status) tree_status[b] = bad_s ? GDN_ERR_TREE : 0;
}

template <typename T, int DK>
hipError_t verify_simple(const VerifyArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B) * a.H_v * (a.d_v / 64));
    hipLaunchKernelGGL((verify_simple_kernel<T, DK>), grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int DK>
hipError_t commit_simple(const CommitArgs& a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B) * a.H_v * (a.d_v / 64));
    hipLaunchKernelGGL((commit_simple_kernel<T, DK>), grid, dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_simple(const VerifyArgs& a, hipStream_t stream) {
    if (a.qkv_dtype == GDN_BF16)
        return a.d_k == 64 ? verify_simple<uint16_t, 64>(a, stream) : verify_simple<uint16_t, 128>(a, stream);
    return a.d_k == 64 ? verify_simple<float, 64>(a, stream) : verify_simple<float, 128>(a, stream);
}

hipError_t launch_commit_simple(const CommitArgs& a, hipStream_t stream) {
    if (a.qkv_dtype == GDN_BF16)
        return a.d_k == 64 ? commit_simple<uint16_t, 64>(a, stream) : commit_simple<uint16_t, 128>(a, stream);
    return a.d_k == 64 ? commit_simple<float, 64>(a, stream) : commit_simple<float, 128>(a, stream);
}

hipError_t launch_ancestors(int B, int N, const int32_t* parent, uint32_t* anc, int32_t* depth,
                            int32_t* tree_status, hipStream_t stream) {
    hipLaunchKernelGGL(ancestors_kernel, dim3(B), dim3(256), 0, stream, N, parent, anc, depth, tree_status);
    return hipGetLastError();
}


}  // namespace gdn
