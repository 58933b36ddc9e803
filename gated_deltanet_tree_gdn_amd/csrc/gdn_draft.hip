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

// The wavefront's largest 32-bit value, in every lane: DPP max stages over
// pairs, quads, half rows, rows, then the row broadcasts 15 and 31, after
// which lane 63 holds the maximum.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t max_stage_u32(uint32_t v) {
    // lanes without a source read 0, the identity of the unsigned max
    const uint32_t o = static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, ROW_MASK, 0xF, false));
    return o > v ? o : v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max_stage_u32<0xB1, 0xF>(v);
    v = max_stage_u32<0x4E, 0xF>(v);
    v = max_stage_u32<0x141, 0xF>(v);
    v = max_stage_u32<0x140, 0xF>(v);
    v = max_stage_u32<0x142, 0xA>(v);
    v = max_stage_u32<0x143, 0xC>(v);
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

// The wavefront's largest 64-bit key as two 32-bit reductions: the largest
// high word, then the largest low word among the lanes that hold it.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v) {
    const uint32_t hi = wave_max_u32(static_cast<uint32_t>(v >> 32));
    const uint32_t lo = wave_max_u32(static_cast<uint32_t>(v >> 32) == hi ? static_cast<uint32_t>(v) : 0u);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// An fp32 value as an unsigned integer of the same order.
__device__ __forceinline__ uint32_t orderable(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// KU positions per lane (the prefix included): (N + 1 + 63) / 64, up to kU
template <int KU>
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
    // the candidate rows into LDS, 32 loads in flight per lane at a time
    // (entry e = u C + r: the prefix's row, then the nodes' rows, contiguous)
    const int n_lp = (N + 1) * C;
    constexpr int LB = 32;
    for (int e0 = 0; e0 < n_lp; e0 += 64 * LB) {
        float x[LB];
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            const int e = min(e0 + l + 64 * q, n_lp - 1);
            x[q] = e < C ? rl[e] : nl[static_cast<size_t>(e - C)];
        }
#pragma unroll
        for (int q = 0; q < LB; ++q) {
            const int e = e0 + l + 64 * q;
            if (e < n_lp) lp[(e / C) * kMaxCand + e % C] = x[q];
        }
    }
    if (l == 0) depth_s[0] = 0;
    __syncthreads();
    // every row must be sorted best first (a lane walks whole rows)
    bool unsorted = false;
    for (int u = l; u <= N; u += 64) {
        const float* row = lp + u * kMaxCand;
        float prev = row[0];
#pragma unroll 8
        for (int r = 1; r < C; ++r) {
            const float x = row[r];
            unsorted |= x > prev;
            prev = x;
        }
    }
    const float NEG = -__builtin_inff();
    // head state per position held by this lane (u = l + 64 e)
    float hs[KU], ns[KU];   // head score; the position's own score
    float nx[KU];           // log-probability of the candidate after the head
    int hr[KU];             // head rank
    // the head as one key: the score's order in the high word, the
    // position's in the low word (ties go to the lower position); 0: none
    uint64_t hk[KU];
    auto key_of = [](float score, int u) -> uint64_t {
        return score == -__builtin_inff() ? 0ull
                                          : (static_cast<uint64_t>(orderable(score)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(u));
    };
#pragma unroll
    for (int e = 0; e < KU; ++e) {
        hs[e] = NEG;
        ns[e] = 0.f;
        nx[e] = NEG;
        hr[e] = 0;
        hk[e] = 0ull;
    }
    if (l == 0 && max_depth >= 1) {
        hs[0] = lp[0];   // the prefix's best candidate
        nx[0] = lp[min(1, C - 1)];
        hk[0] = key_of(hs[0], 0);
    }
    int count = 0, steps = 0;
    bool dry = false;
    while (count < N) {
        const int first = count;
        int taken = 0;
        while (taken < w && count < N) {
            // this lane's best head, then the wavefront's: the best score,
            // the lowest position among equals
            uint64_t key = hk[0];
#pragma unroll
            for (int e = 1; e < KU; ++e) key = hk[e] > key ? hk[e] : key;
            key = wave_max_key(key);
            if (key == 0ull) break;   // every list is spent
            const int u = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
            const int owner = u & 63, eo = u >> 6;
            if (l == owner) {
#pragma unroll
                for (int e = 0; e < KU; ++e)
                    if (e == eo) {
                        o_par[count] = u - 1;
                        o_rank[count] = hr[e];
                        o_score[count] = hs[e];
                        const int nr = hr[e] + 1;
                        hr[e] = nr;
                        // the prefix's candidates score their own
                        // log-probability; the one after the new head is read
                        // now, for this position's next pop
                        const float x = nx[e];
                        hs[e] = nr < C ? (u == 0 ? x : ns[e] + x) : NEG;
                        hk[e] = key_of(hs[e], u);
                        nx[e] = lp[u * kMaxCand + min(nr + 1, C - 1)];
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
        for (int e = 0; e < KU; ++e) {
            const int j = l + 64 * e - 1;
            if (j >= first && j < count) {
                const int d = depth_s[o_par[j] + 1] + 1;
                depth_s[j + 1] = d;
                ns[e] = o_score[j];
                hr[e] = 0;
                hs[e] = d < max_depth ? o_score[j] + lp[(j + 1) * kMaxCand] : NEG;
                hk[e] = key_of(hs[e], j + 1);
                nx[e] = lp[(j + 1) * kMaxCand + min(1, C - 1)];
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
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, dim3(B), dim3(64), 0, stream, N, C, w, max_depth, root_logp, node_logp, parent,
                           cand_rank, score, steps, build_status);
    };
    static_assert(kU == 5, "one instantiation per count of positions per lane");
    switch ((N + 1 + 63) / 64) {
        case 1: go(build_kernel<1>); break;
        case 2: go(build_kernel<2>); break;
        case 3: go(build_kernel<3>); break;
        case 4: go(build_kernel<4>); break;
        default: go(build_kernel<5>); break;
    }
    return hipGetLastError();
}

}  // namespace gdn
