// gdn_draft.hip -- the two steps on either side of tree verification, on the
// device, one wavefront per sequence:
//
//  * tree construction upstream of verify: best-first search over candidate
//    continuations that takes the w best candidates of the heap at a time
//    and expands them together (Trees from Marginals technical summary,
//    Methodology, "2. Tree Construction");
//  * selection of the accepted node that the delayed commit needs (same
//    summary, Methodology, "3. Rollback-Free Tree Verification for GDN": the
//    state is committed once the accepted branch is known), by greedy
//    matching of drafted tokens against the verifier's choices from the
//    root down.
//
// Both are short serial walks over at most 257 positions, so a single
// wavefront holds every position in registers (position u = lane + 64 e)
// and each step is a handful of wave-wide ballots or reductions.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kE = kMaxN / 64;          // nodes per lane
constexpr int kU = (kMaxN + 1 + 63) / 64;  // positions per lane, the prefix included

// ---------------------------------------------------------------- acceptance
// From the prefix (node -1), repeatedly move to the lowest-index child whose
// draft token equals the verifier's choice after the current node
// (target[c + 1]; target[0] follows the prefix), until no child matches.
__global__ __launch_bounds__(64) void accept_kernel(int N, const int32_t* __restrict__ parent,
                                                    const int32_t* __restrict__ draft,
                                                    const int32_t* __restrict__ target, int32_t* accepted,
                                                    int32_t* accept_len, int32_t* tree_status) {
    __shared__ int tgt[kMaxN + 1];
    const int b = blockIdx.x, l = threadIdx.x;
    const size_t pb = static_cast<size_t>(b) * N, tb = static_cast<size_t>(b) * (N + 1);
    int par[kE], tok[kE];
    bool bad = false;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
        const int i = l + 64 * e;
        par[e] = -2;   // past N: never anyone's child
        tok[e] = 0;
        if (i < N) {
            const int p = parent[pb + i];
            const bool inval = p < -1 || p >= i;
            bad |= inval;
            par[e] = inval ? -1 : p;   // an invalid parent is flagged and read as the prefix
            tok[e] = draft[pb + i];
        }
    }
    for (int i = l; i <= N; i += 64) tgt[i] = target[tb + i];
    __syncthreads();
    int cur = -1, len = 0;
    // each step moves to a higher node index, so at most N steps
    for (int step = 0; step < N; ++step) {
        const int want = tgt[cur + 1];
        int found = -1;
#pragma unroll
        for (int e = 0; e < kE; ++e) {
            const uint64_t m = __ballot(par[e] == cur && tok[e] == want);
            if (found < 0 && m != 0ull) found = 64 * e + __ffsll(static_cast<unsigned long long>(m)) - 1;
        }
        if (found < 0) break;
        cur = found;
        ++len;
    }
    const bool any_bad = __ballot(bad) != 0ull;
    if (l == 0) {
        accepted[b] = cur;
        if (accept_len) accept_len[b] = len;
        if (tree_status) tree_status[b] = any_bad ? GDN_ERR_TREE : 0;
    }
}

// ------------------------------------------------------ tree construction
// Position u = p + 1 stands for the prefix (u = 0) or node p.  Every placed
// position with depth below the cap owns a list of candidate children, best
// first; its head is the best one not yet taken.  Popping the heap's best
// candidate is an argmax over the heads (ties to the lower position, and
// within a position the list order is the rank order), after which that
// position's head moves on.  A step pops up to w heads; the nodes it places
// get their own heads only when the step ends.
// Wave-wide max / min with DPP row operations (pairs, quads, half rows,
// rows, then the row broadcasts 15 and 31); the result is read from lane 63
// and returned to every lane.
template <typename T, typename Op>
__device__ __forceinline__ T wave_reduce(T v, Op op) {
    int x = static_cast<int>(v);
    x = static_cast<int>(op(static_cast<T>(x), static_cast<T>(__builtin_amdgcn_update_dpp(x, x, 0xB1, 0xF, 0xF, false))));
    x = static_cast<int>(op(static_cast<T>(x), static_cast<T>(__builtin_amdgcn_update_dpp(x, x, 0x4E, 0xF, 0xF, false))));
    x = static_cast<int>(op(static_cast<T>(x), static_cast<T>(__builtin_amdgcn_update_dpp(x, x, 0x141, 0xF, 0xF, false))));
    x = static_cast<int>(op(static_cast<T>(x), static_cast<T>(__builtin_amdgcn_update_dpp(x, x, 0x140, 0xF, 0xF, false))));
    x = static_cast<int>(op(static_cast<T>(x), static_cast<T>(__builtin_amdgcn_update_dpp(x, x, 0x142, 0xA, 0xF, false))));
    x = static_cast<int>(op(static_cast<T>(x), static_cast<T>(__builtin_amdgcn_update_dpp(x, x, 0x143, 0xC, 0xF, false))));
    return static_cast<T>(__builtin_amdgcn_readlane(x, 63));
}

struct MaxU {
    __device__ uint32_t operator()(uint32_t a, uint32_t b) const { return a > b ? a : b; }
};
struct MinI {
    __device__ int operator()(int a, int b) const { return a < b ? a : b; }
};

__device__ __forceinline__ uint32_t orderable(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__global__ __launch_bounds__(64) void build_kernel(int N, int C, int w, int max_depth,
                                                   const float* __restrict__ root_logp,
                                                   const float* __restrict__ node_logp, int32_t* parent,
                                                   int32_t* cand_rank, float* score, int32_t* steps_out,
                                                   int32_t* build_status) {
    __shared__ float lp[(kMaxN + 1) * kMaxCand];   // row u: the candidates of position u
    __shared__ int o_par[kMaxN], o_rank[kMaxN];
    __shared__ float o_score[kMaxN];
    __shared__ int depth_s[kMaxN + 1];   // depth of position u (the prefix: 0)
    const int b = blockIdx.x, l = threadIdx.x;
    const float* rl = root_logp + static_cast<size_t>(b) * C;
    const float* nl = node_logp + static_cast<size_t>(b) * N * C;
    bool unsorted = false;
    for (int e = l; e < (N + 1) * C; e += 64) {
        const int u = e / C, r = e % C;
        const float x = u == 0 ? rl[r] : nl[static_cast<size_t>(u - 1) * C + r];
        lp[u * kMaxCand + r] = x;
        if (r > 0) {
            const float prev = u == 0 ? rl[r - 1] : nl[static_cast<size_t>(u - 1) * C + r - 1];
            unsorted |= x > prev;
        }
    }
    if (l == 0) depth_s[0] = 0;
    __syncthreads();
    const float NEG = -__builtin_inff();
    // head state per position held by this lane (u = l + 64 e)
    float hs[kU], ns[kU];   // head score; the position's own score
    int hr[kU];             // head rank
#pragma unroll
    for (int e = 0; e < kU; ++e) {
        hs[e] = NEG;
        ns[e] = 0.f;
        hr[e] = 0;
    }
    if (l == 0 && max_depth >= 1) hs[0] = lp[0];   // the prefix's best candidate
    int count = 0, steps = 0;
    bool dry = false;
    while (count < N) {
        const int first = count;
        int taken = 0;
        while (taken < w && count < N) {
            // this lane's best head, then the wavefront's
            uint32_t key = 0u;
#pragma unroll
            for (int e = 0; e < kU; ++e) key = max(key, hs[e] == NEG ? 0u : orderable(hs[e]));
            key = wave_reduce<uint32_t>(key, MaxU{});
            if (key == 0u) break;   // every list is spent
            // lowest position among the lanes holding that key (a lane's own
            // best position is its lowest one with that key)
            int cand = 0x7fffffff;
#pragma unroll
            for (int e = 0; e < kU; ++e)
                if (hs[e] != NEG && orderable(hs[e]) == key) cand = min(cand, l + 64 * e);
            cand = wave_reduce<int>(cand, MinI{});
            const int u = cand, owner = u & 63, eo = u >> 6;
            if (l == owner) {
#pragma unroll
                for (int e = 0; e < kU; ++e)
                    if (e == eo) {
                        o_par[count] = u - 1;
                        o_rank[count] = hr[e];
                        o_score[count] = hs[e];
                        const int nr = hr[e] + 1;
                        hr[e] = nr;
                        // the prefix's candidates score their own log-probability
                        const float x = lp[u * kMaxCand + min(nr, C - 1)];
                        hs[e] = nr < C ? (u == 0 ? x : ns[e] + x) : NEG;
                    }
            }
            ++count;
            ++taken;
        }
        if (taken == 0) {
            dry = true;
            break;
        }
        ++steps;
        __syncthreads();   // the step's nodes are in o_par / o_score
        // the step's nodes get their candidate lists (depth = the parent
        // position's depth + 1, exchanged through LDS: the parent's depth
        // belongs to the lane that holds the parent)
#pragma unroll
        for (int e = 0; e < kU; ++e) {
            const int j = l + 64 * e - 1;
            if (j >= first && j < count) {
                const int d = depth_s[o_par[j] + 1] + 1;
                depth_s[j + 1] = d;
                ns[e] = o_score[j];
                hr[e] = 0;
                hs[e] = d < max_depth ? o_score[j] + lp[(j + 1) * kMaxCand] : NEG;
            }
        }
        __syncthreads();
    }
    for (int i = l; i < N; i += 64) {
        const size_t o = static_cast<size_t>(b) * N + i;
        const bool placed = i < count;
        parent[o] = placed ? o_par[i] : -1;
        if (cand_rank) cand_rank[o] = placed ? o_rank[i] : 0;
        if (score) score[o] = placed ? o_score[i] : NEG;
    }
    const bool any_unsorted = __ballot(unsorted) != 0ull;
    if (l == 0) {
        if (steps_out) steps_out[b] = steps;
        if (build_status) build_status[b] = any_unsorted ? GDN_ERR_SHAPE : (dry ? GDN_ERR_TREE : 0);
    }
}

}  // namespace

hipError_t launch_accept(int B, int N, const int32_t* parent, const int32_t* draft, const int32_t* target,
                         int32_t* accepted, int32_t* accept_len, int32_t* tree_status, hipStream_t stream) {
    hipLaunchKernelGGL(accept_kernel, dim3(B), dim3(64), 0, stream, N, parent, draft, target, accepted, accept_len,
                       tree_status);
    return hipGetLastError();
}

hipError_t launch_build(int B, int N, int C, int w, int max_depth, const float* root_logp, const float* node_logp,
                        int32_t* parent, int32_t* cand_rank, float* score, int32_t* steps, int32_t* build_status,
                        hipStream_t stream) {
    hipLaunchKernelGGL(build_kernel, dim3(B), dim3(64), 0, stream, N, C, w, max_depth, root_logp, node_logp, parent,
                       cand_rank, score, steps, build_status);
    return hipGetLastError();
}

}  // namespace gdn
