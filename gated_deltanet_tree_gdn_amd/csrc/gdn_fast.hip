// gdn_fast.hip -- single-launch MFMA tree verification for bf16 q/k/v and
// trees of 129 to 256 nodes on gfx950, used where no workspace is at hand
// (the allocation-free entry point; with a context the two-launch verify of
// gdn_split.hip runs instead, and smaller trees go to gdn_verify_ws.hip),
// and the verify dispatch.
//
// What is computed (Trees from Marginals technical summary, Methodology,
// "3. Rollback-Free Tree Verification for GDN"): with the tree sorted
// topologically, the interaction matrices over ancestor pairs
//     X_is = beta_i D_is (k_i . k_s)   for s a strict ancestor of i,
//     Y_is = D_is (q_i . k_s)          for s an ancestor of i or i itself,
// (D_is = exp(G_i - G_s), G the path-cumulative log-gate, gamma = exp(G)),
// the solve (I + X) U = diag(beta) (V - diag(gamma) K S0^T) and the output
// O = diag(gamma) Q S0^T + Y U.  Here the solve is folded into an N x N
// operator that does not depend on d_v:
//     Z~ = Y (I + X)^-1 diag(beta),     O = gamma o (Q S0^T) + Z~ R',
//     R' = V - gamma o (K S0^T).
// Z~ has the ancestor pattern of the tree.  Row i is found by a
// back-substitution along the root-to-i path, z_b = Y_{i,t_b} -
// sum_{a>b} z_a X_{t_a,t_b}, which needs only the pairs (node, ancestor).
//
// Work decomposition: a persistent grid, one workgroup per compute unit,
// each walking a contiguous run of (sequence, value head) items in head
// order.  Consecutive items of one sequence share the tree structure
// (depth, root paths, ancestor bits).  d_v/16 wavefronts; the wavefront w
// owns value columns [16w, 16w + 16) (one MFMA tile) and keeps its slice of
// S0 (as a bf16 hi + lo pair) and R' in registers.  Dense contractions run on
// v_mfma_f32_16x16x32_bf16: q and k are exact bf16; S0, R' and Z~ are split
// into hi + lo bf16 so products stay near fp32 accuracy.
//
// Per item: (1) S0 and V loads for this item are issued first, and the node
// scalars of the next item are prefetched into registers during this one;
// (2) for a new sequence: depth and root paths (pointer jumping, prefix
// sum), ancestor bits; (3) for a new key head, K into LDS; the Gram values
// of the ancestor pairs (MFMA over the lower 16x16 tiles holding pairs, Q
// rows read per row tile); (4) G, gamma, the rows of Z~ (one thread
// per node, in registers for paths of up to 24 nodes); (5) per wavefront:
// K S0^T -> R', then per 16-row tile, with that tile's Q rows and Z~ blocks
// staged in LDS by the workgroup, the transposed tile S0 Q^T + R'^T Z~^T, so
// that each lane stores 16 contiguous bytes of o.
//
// Trees whose pair list exceeds the LDS budget are verified, inside the same
// workgroup, by the per-node walk of gdn_walk.h.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"
#include "gdn_mfma.h"
#include "gdn_walk.h"

// Phase markers: no-ops here; a profiling build defines them to accumulate
// per-phase cycle counts.
#ifndef GDN_PHASE
#define GDN_PHASE_INIT
#define GDN_PHASE(k)
#define GDN_PHASE_END
#endif

namespace gdn {
namespace {

__device__ __forceinline__ uint4 mask4(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }

// LDS layout (bytes) for trees of at most NMAX = 256 nodes: K staged; Q read
// from global memory per row tile (Gram) and staged per output tile; the
// Gram values of the pairs computed per value head (the rows of Z~ replace
// the q_i . k_s values in place, and the Z~ blocks of an output tile reuse
// the k_i . k_s area).
template <int NMAX, int DK>
struct Lds {
    static_assert(NMAX == 256, "trees of 129 to 256 nodes");
    // pair-list capacity: every tree of depth <= 24
    static constexpr int CAP = 6144;
    static constexpr int AW = NMAX / 32;        // ancestor bit-row words
    static constexpr int KROW = DK * 2 + 16;    // staged k / q row, padded against bank conflicts
    static constexpr int KS_OFF = 0;
    // float[CAP + 32]: k_i . k_s per value head; entries KZERO .. KZERO + 31
    // are zero (the row the solve reads for path positions past a node's depth)
    static constexpr int XC = NMAX * KROW;
    static constexpr int KZERO = CAP;
    static constexpr int YC = XC + 4 * (CAP + 32);  // float[CAP]: q_i . k_s, then the rows of Z~
    static constexpr int PATH = YC + 4 * CAP;   // uint8[CAP]: root..i path of every node
    static constexpr int PNODE = PATH + CAP;    // uint8[CAP]: node owning each pair
    static constexpr int NODE = (PNODE + CAP + 15) & ~15;
    static constexpr int PAR = NODE;            // int[NMAX]
    static constexpr int DEP = PAR + 4 * NMAX;
    static constexpr int OFF = DEP + 4 * NMAX;
    static constexpr int NXT = OFF + 4 * NMAX;
    static constexpr int GV = NXT + 4 * NMAX;   // float[NMAX]: g of the item's head
    static constexpr int BET = GV + 4 * NMAX;   // beta
    static constexpr int GG = BET + 4 * NMAX;   // G (path sum of g)
    static constexpr int GAM = GG + 4 * NMAX;   // gamma (0 past N)
    static constexpr int ANC = GAM + 4 * NMAX;  // uint32[NMAX][AW]: ancestor bit rows
    static constexpr int TMASK = ANC + 4 * AW * NMAX;  // uint32[NMAX/16]: tile (I, J) has pairs
    static constexpr int MISC = TMASK + 4 * (NMAX / 16);
    static constexpr int FBKQ = MISC + 64;      // float[2*DK] for the fallback walk
    // the Q rows of one 16-row tile, staged per output tile
    static constexpr int QT = FBKQ + 8 * DK;
    static constexpr int TOTAL = QT + 16 * KROW;
    static_assert(NMAX * 64 * 4 + DK * 64 * 4 <= NODE, "fallback u and S0 buffers must fit below the node arrays");
};

// NW wavefronts; wavefront w owns CT = d_v / (16 NW) MFMA tiles of 16 value
// columns.  With CT = 2 a lane's two columns are adjacent (32 w + 2 lc + st),
// so V is read in 4-byte and o written in 8-byte pieces.
template <int NMAX, int DK, int DV, int NW>
__global__ __launch_bounds__(64 * NW) void verify_fast_kernel(VerifyArgs a, int items_per_wg) {
    using L = Lds<NMAX, DK>;
    constexpr int NTH = 64 * NW;        // threads
    constexpr int CT = DV / (16 * NW);  // 16-column MFMA tiles per wavefront
    static_assert(CT == 1 || CT == 2, "one or two column tiles per wavefront");
    constexpr int KS = DK / 32;         // MFMA k-steps over d_k
    constexpr int NTMAX = NMAX / 16;    // 16-row tiles
    constexpr int NKMAX = NMAX / 32;    // 32-node k-steps over the tree
    constexpr int KCH = NMAX * DK / 8 / NTH;  // 16-byte chunks of K (and Q) per thread
    static_assert(KCH >= 1 && NMAX * DK / 8 % NTH == 0, "K staging split");
    constexpr int IPT = (NMAX + NTH - 1) / NTH;  // nodes per thread in node loops
    constexpr int ZR = NMAX > 128 ? 24 : 16;   // path length kept in registers when solving a row of Z~

    __shared__ __align__(16) unsigned char smem[L::TOTAL];

    const int N0 = a.N, Hk = a.H_k, Hv = a.H_v;
    const int R = Hv / Hk;
    const int n_items = a.B * Hv;
    // Workgroups go to the 8 XCDs in turn; numbering them so that each XCD
    // takes consecutive items keeps the heads of a sequence on one XCD, whose
    // L2 then serves their shared rows of g, beta and the parents once
    const int wg = gridDim.x % 8 == 0 ? (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8 : blockIdx.x;
    const int it_begin = wg * items_per_wg;
    const int it_end = min(it_begin + items_per_wg, n_items);
    if (it_begin >= it_end) return;

    const int tid0 = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);

    const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
    const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
    const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);

    int* par = reinterpret_cast<int*>(smem + L::PAR);
    int* dep = reinterpret_cast<int*>(smem + L::DEP);
    int* off = reinterpret_cast<int*>(smem + L::OFF);
    int* nxt = reinterpret_cast<int*>(smem + L::NXT);
    float* gv = reinterpret_cast<float*>(smem + L::GV);
    float* bet = reinterpret_cast<float*>(smem + L::BET);
    float* Gs = reinterpret_cast<float*>(smem + L::GG);
    float* gam = reinterpret_cast<float*>(smem + L::GAM);
    uint32_t* anc = reinterpret_cast<uint32_t*>(smem + L::ANC);
    uint32_t* tmask = reinterpret_cast<uint32_t*>(smem + L::TMASK);
    int* misc = reinterpret_cast<int*>(smem + L::MISC);
    float* kk = reinterpret_cast<float*>(smem + L::XC);
    float* qk = reinterpret_cast<float*>(smem + L::YC);   // q_i . k_s, then the rows of Z~ in place
    uint8_t* pathc = smem + L::PATH;
    uint8_t* pnode = smem + L::PNODE;
    unsigned char* Ks = smem + L::KS_OFF;

    // Prefetched state of the next item: node scalars, and the K share of a
    // new key head.  Loads are unconditional with indices clamped into range;
    // out-of-range values are replaced after arrival.
    int p_pf[IPT];
    float g_pf[IPT], b_pf[IPT];
    uint4 k_pf[KCH];
    auto prefetch_scalars = [&](int it, int tid, int N) {
        const int bb = it / Hv, hh = it % Hv;
#pragma unroll
        for (int q = 0; q < IPT; ++q) {
            const int i = min(tid + q * NTH, N - 1);
            p_pf[q] = a.parent[static_cast<size_t>(bb) * N + i];
            const size_t nh = (static_cast<size_t>(bb) * N + i) * Hv + hh;
            g_pf[q] = a.g[nh];
            b_pf[q] = a.beta[nh];
        }
    };
    auto prefetch_kq = [&](int it, int tid, int N) {
        const int bb = it / Hv, kh = (it % Hv) / R;
#pragma unroll
        for (int q = 0; q < KCH; ++q) {
            const int e = tid + q * NTH;
            const int row = min(e / (DK / 8), N - 1);
            const size_t gofs = ((static_cast<size_t>(bb) * N + row) * Hk + kh) * DK + (e % (DK / 8)) * 8;
            k_pf[q] = *reinterpret_cast<const uint4*>(kg + gofs);
        }
    };
    GDN_PHASE_INIT;
    prefetch_scalars(it_begin, tid0, N0);
    __builtin_amdgcn_sched_barrier(0);
    prefetch_kq(it_begin, tid0, N0);

    // k_pf holds the K of the first item; a later key head's K is loaded at
    // the start of its first item
    int cur_b = -1, cur_kh = -1, total = 0;
    for (int it = it_begin; it < it_end; ++it) {
        // Opaque copies of the thread index and N: everything derived from
        // them is recomputed per item instead of being hoisted out of the
        // loop and held in registers across it.
        int tid = tid0, N = N0;
        asm volatile("" : "+v"(tid));
        asm volatile("" : "+s"(N));
        const int lane = tid & 63;
        const int lc = lane & 15;
        const int lg = lane >> 4;
        // value column of (lane, tile st)
        auto column = [&](int st) { return CT == 1 ? 16 * wave + lc : 32 * wave + 2 * lc + st; };
        const int b = it / Hv, h = it % Hv, kh = h / R;
        const bool new_b = b != cur_b;
        const bool new_kh = new_b || kh != cur_kh;
        const int nit = it + 1 < it_end ? it + 1 : -1;
        GDN_PHASE(0);

        // ---- (1) this item's S0 rows (lane (lc, lg) of tile st holds d_k
        // columns [8 KS lg, 8 KS (lg + 1)) of row column(st)) and V columns
        // for every node, in flight during the tree work
        float4 s0r[CT][2 * KS];
#pragma unroll
        for (int st = 0; st < CT; ++st) {
            const float4* src =
                reinterpret_cast<const float4*>(a.S0 + ((static_cast<size_t>(b) * Hv + h) * DV + column(st)) * DK + 8 * KS * lg);
#pragma unroll
            for (int q = 0; q < 2 * KS; ++q) s0r[st][q] = src[q];
        }
        const size_t vbase = static_cast<size_t>(b) * N * Hv * DV + static_cast<size_t>(h) * DV + column(0);
        uint32_t vraw[NTMAX][4];  // CT == 2: the lane's two adjacent bf16 columns
#pragma unroll
        for (int S = 0; S < NTMAX; ++S)
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const uint16_t* vp = vg + vbase + static_cast<size_t>(min(16 * S + 4 * lg + rr, N - 1)) * Hv * DV;
                vraw[S][rr] = CT == 1 ? static_cast<uint32_t>(*vp) : *reinterpret_cast<const uint32_t*>(vp);
            }

        // ---- (2) node scalars; for a new sequence the tree structure
        int bad_local = 0;
#pragma unroll
        for (int q = 0; q < IPT; ++q) {
            const int i = tid + q * NTH;
            if (i < NMAX) {
                gv[i] = i < N ? g_pf[q] : 0.f;
                bet[i] = i < N ? b_pf[q] : 0.f;
                if (new_b) {
                    int p = i < N ? p_pf[q] : -1;
                    if (p < -1 || p >= i) {
                        bad_local = 1;
                        p = -1;
                    }
                    par[i] = p;
                    nxt[i] = p;
                    dep[i] = i < N ? 1 : 0;
                }
            }
        }
        if (nit >= 0) prefetch_scalars(nit, tid, N);
        if (new_b) {
            if (tid < NMAX / 16) tmask[tid] = 0u;
            const int bad = __syncthreads_or(bad_local);
            if (h == 0 && tid == 0) a.tree_status[b] = bad ? GDN_ERR_TREE : 0;
            // depth by pointer jumping: dep[i] counts the nodes from i up to nxt[i]
            for (int round = 0; round < 9; ++round) {
                int c2[IPT], n2[IPT];
                int live = 0;
#pragma unroll
                for (int q = 0; q < IPT; ++q) {
                    const int i = tid + q * NTH;
                    c2[q] = 0;
                    n2[q] = -1;
                    if (i < NMAX) {
                        const int nx = nxt[i];
                        c2[q] = dep[i] + (nx >= 0 ? dep[nx] : 0);
                        n2[q] = nx >= 0 ? nxt[nx] : -1;
                        live |= n2[q] >= 0;
                    }
                }
                __syncthreads();
#pragma unroll
                for (int q = 0; q < IPT; ++q) {
                    const int i = tid + q * NTH;
                    if (i < NMAX) {
                        dep[i] = c2[q];
                        nxt[i] = n2[q];
                    }
                }
                if (!__syncthreads_or(live)) break;
            }
            // offsets of each node's path in the pair list (exclusive scan)
            if (wave == 0) {
                constexpr int E = NMAX / 64;
                int vals[E];
                int sum = 0;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    vals[e] = dep[lane * E + e];
                    sum += vals[e];
                }
                int incl = sum;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const int t = __shfl_up(incl, o, 64);
                    if (lane >= o) incl += t;
                }
                int run = incl - sum;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    off[lane * E + e] = run;
                    run += vals[e];
                }
                if (lane == 63) misc[0] = incl;
            }
            __syncthreads();
            total = misc[0];
            if (total <= L::CAP) {
                // root..i path, owner and ancestor offsets of every pair;
                // ancestor bits; tiles holding pairs
                for (int i = tid; i < NMAX; i += NTH) {
                    uint32_t bits[L::AW];
#pragma unroll
                    for (int w = 0; w < L::AW; ++w) bits[w] = 0u;
                    if (i < N) {
                        int pos = off[i] + dep[i] - 1;
                        uint32_t mask = 0u;
                        for (int s = i; s >= 0; s = par[s]) {
                            pathc[pos] = static_cast<uint8_t>(s);
                            pnode[pos] = static_cast<uint8_t>(i);
                            --pos;
                            mask |= 1u << (s >> 4);
#pragma unroll
                            for (int w = 0; w < L::AW; ++w) bits[w] |= (s >> 5) == w ? 1u << (s & 31) : 0u;
                        }
                        atomicOr(&tmask[i >> 4], mask);
                    }
#pragma unroll
                    for (int w = 0; w < L::AW; ++w) anc[i * L::AW + w] = bits[w];
                }
            }
        }
        __syncthreads();
        GDN_PHASE(1);

        if (total > L::CAP) {
            // deep tree: the per-node walk by wavefront 0, one 64-column
            // slice at a time; it overwrites the staged K/Q
            if (wave == 0) {
                float* u_s = reinterpret_cast<float*>(smem);
                float* s0_s = reinterpret_cast<float*>(smem + NMAX * 64 * 4);
                float* ki = reinterpret_cast<float*>(smem + L::FBKQ);
                for (int c0 = 0; c0 < DV; c0 += 64)
                    walk_verify_slice_lds<uint16_t, DK, WaveSync>(a, b, h, c0, par, u_s, Gs, ki, ki + DK, s0_s);
            }
            cur_b = b;
            cur_kh = -1;
            // this path leaves the S0 and V loads above unused: drain them
            // here so the next item's loads into the same registers need no
            // wait
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            continue;
        }

        // ---- (3) new key head: K (and Q) into LDS (unless the previous item
        // already put them there), rows past N zeroed; then the Gram values
        // of the ancestor pairs
        const int NT = (N + 15) >> 4;
        auto q_frag = [&](int row, int ks) -> bf16x8 {
            return load_frag(qg + ((static_cast<size_t>(b) * N + min(row, N - 1)) * Hk + kh) * DK + 8 * KS * lg + 8 * ks);
        };
        auto k_frag = [&](int row, int ks) -> bf16x8 { return load_frag(Ks + row * L::KROW + 2 * (8 * KS * lg + 8 * ks)); };
        auto stage_kq = [&]() {
#pragma unroll
            for (int q = 0; q < KCH; ++q) {
                const int e = tid + q * NTH;
                const int row = e / (DK / 8);
                const int cc = e % (DK / 8);
                const uint32_t keep = row < N ? 0xFFFFFFFFu : 0u;
                *reinterpret_cast<uint4*>(Ks + row * L::KROW + cc * 16) = mask4(k_pf[q], keep);
            }
        };
        if (new_kh) {
            if (it != it_begin) prefetch_kq(it, tid, N);
            stage_kq();
            __syncthreads();
        }
        // Gram tile (I, J) into the pair list: each value lands at its pair
        // (i, s) = path position dep[s] - 1 of node i
        auto gram_tile = [&](int I, int J, const bf16x8 (&qa)[KS]) {
                    f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 kb = k_frag(16 * J + lc, ks);
                        akk = mfma(k_frag(16 * I + lc, ks), kb, akk);
                        aqk = mfma(qa[ks], kb, aqk);
                    }
                    const int s = 16 * J + lc;
                    const int ds = dep[s];
                    uint32_t aw[4];
                    int oi[4];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int i = 16 * I + 4 * lg + rr;
                        aw[rr] = anc[i * L::AW + (s >> 5)];
                        oi[rr] = off[i];
                    }
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int i = 16 * I + 4 * lg + rr;
                        if (i < N && ((aw[rr] >> (s & 31)) & 1u)) {
                            const int p = oi[rr] + ds - 1;
                            qk[p] = aqk[rr];
                            kk[p] = akk[rr];
                        }
                    }
        };
        {
            // Q rows from global memory: each wavefront takes whole row tiles, whose
            // Q rows it loads once, the next row tile's while it works on
            // this one (rows w, 7 - w, 8 + w, 15 - w balance the triangle)
            // (NTMAX / NW row tiles per wavefront, in pairs w, 2 NW - 1 - w)
            constexpr int RU = NTMAX / NW;
            static_assert(RU % 2 == 0 && RU * NW == NTMAX, "row-tile assignment");
            auto row_tile = [&](int u) { return (u & 1) ? 2 * NW * (u >> 1) + 2 * NW - 1 - wave : 2 * NW * (u >> 1) + wave; };
            bf16x8 qa[KS], qn[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) qa[ks] = q_frag(16 * row_tile(0) + lc, ks);
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int I = row_tile(u);
                if (u + 1 < RU) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) qn[ks] = q_frag(16 * row_tile(u + 1) + lc, ks);
                }
                if (I < NT) {
                    const uint32_t tm = tmask[I];
                    for (int J = 0; J <= I; ++J)
                        if ((tm >> J) & 1u) gram_tile(I, J, qa);
                }
                if (u + 1 < RU) {
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) qa[ks] = qn[ks];
                }
            }
        }

        GDN_PHASE(2);
        // ---- (4) G (path sum of g) and gamma per node; per node its row of
        // Z~ by a right-looking sweep along its path (in registers for paths
        // of up to ZR nodes).  Along the root path t_0 .. t_{m-1} = i the row
        // of Y (I + X)^-1 is D_{i,t_b} y_b with
        //     y_b = q_i . k_{t_b} - sum_{a > b} (beta_{t_a} y_a) (k_{t_a} . k_{t_b})
        // (D_{i,t_a} D_{t_a,t_b} = D_{i,t_b}), so the sweep reads the Gram
        // values and beta only; Z~_{i,t_b} = beta_{t_b} D_{i,t_b} y_b.
        for (int i = tid; i < NMAX; i += NTH) {
            float G = 0.f;
            if (i < N) {
                const int o = off[i], m = dep[i];
                if (m <= ZR) {
                    int t[ZR];
#pragma unroll
                    for (int bb = 0; bb < ZR; ++bb) t[bb] = pathc[o + min(bb, m - 1)];
#pragma unroll
                    for (int bb = 0; bb < ZR; ++bb) G += bb < m ? gv[t[bb]] : 0.f;
                } else {
                    for (int bb = 0; bb < m; ++bb) G += gv[pathc[o + bb]];
                }
            }
            Gs[i] = G;
            gam[i] = i < N ? __expf(G) : 0.f;
        }
        // the zero row read for path positions past a node's depth (a walked
        // item may have overwritten it)
        if (tid < 32) kk[L::KZERO + tid] = 0.f;
        __syncthreads();
        for (int i = tid; i < N; i += NTH) {
            const int o = off[i], m = dep[i];
            const float Gi = Gs[i];
            if (m <= ZR) {
                // branch-free: positions past the path read the zero row, so
                // loads can be issued early
                int oa[ZR];
                float y[ZR], bt[ZR];
#pragma unroll
                for (int bb = 0; bb < ZR; ++bb) {
                    const int pp = o + min(bb, m - 1);
                    const int t = pathc[pp];
                    oa[bb] = bb < m ? off[t] : L::KZERO;
                    bt[bb] = bet[t];
                    y[bb] = bb < m ? qk[pp] : 0.f;
                }
                // one row of k.k in flight ahead of the row being applied
                float xr[ZR - 1];
#pragma unroll
                for (int bb = 0; bb < ZR - 1; ++bb) xr[bb] = kk[oa[ZR - 1] + bb];
#pragma unroll
                for (int aa = ZR - 1; aa >= 1; --aa) {
                    float xn[ZR - 1];
#pragma unroll
                    for (int bb = 0; bb + 1 < aa; ++bb) xn[bb] = kk[oa[aa - 1] + bb];
                    const float ya = y[aa] * bt[aa];
#pragma unroll
                    for (int bb = 0; bb < aa; ++bb) y[bb] -= ya * xr[bb];
#pragma unroll
                    for (int bb = 0; bb + 1 < aa; ++bb) xr[bb] = xn[bb];
                    __builtin_amdgcn_sched_barrier(0);
                }
#pragma unroll
                for (int bb = 0; bb < ZR; ++bb)
                    if (bb < m) qk[o + bb] = y[bb] * bt[bb] * __expf(Gi - Gs[pathc[o + bb]]);
                continue;
            }
            for (int aa = m - 1; aa >= 1; --aa) {
                const int ta = pathc[o + aa];
                const float ya = qk[o + aa] * bet[ta];
                const int oa = off[ta];
                for (int bb = 0; bb < aa; ++bb) qk[o + bb] -= ya * kk[oa + bb];
            }
            for (int bb = 0; bb < m; ++bb) {
                const int t = pathc[o + bb];
                qk[o + bb] *= bet[t] * __expf(Gi - Gs[t]);
            }
        }
        __syncthreads();
        GDN_PHASE(3);

        // ---- (5) dense part for this wavefront's columns
        bf16x8 s0h[CT][KS], s0l[CT][KS];
#pragma unroll
        for (int st = 0; st < CT; ++st)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const float4 x0 = s0r[st][2 * ks], x1 = s0r[st][2 * ks + 1];
                const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                split8(x, s0h[st][ks], s0l[st][ks]);
            }
        // K S0^T of tile S for the wavefront's column tiles
        auto ks0 = [&](int S, f32x4 (&out)[CT]) {
            f32x4 ah[CT], al[CT];
#pragma unroll
            for (int st = 0; st < CT; ++st) ah[st] = al[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 ka = k_frag(16 * S + lc, ks);
#pragma unroll
                for (int st = 0; st < CT; ++st) {
                    ah[st] = mfma(ka, s0h[st][ks], ah[st]);
                    al[st] = mfma(ka, s0l[st][ks], al[st]);
                }
            }
#pragma unroll
            for (int st = 0; st < CT; ++st) out[st] = ah[st] + al[st];
        };

        GDN_PHASE(4);
        // (the next key head's K is loaded at the start of its item: held
        // here, those registers would spill R')

        // R' = V - gamma o (K S0^T) as MFMA fragments (k = node) of the Z~ R' product:
        // k-step kap covers nodes [32 kap, 32 kap + 32); lane (lc, lg) holds
        // rows 32 kap + 16 half + 4 lg + rr in slot 4 half + rr.
        bf16x8 rh[CT][NKMAX], rl[CT][NKMAX];
#pragma unroll
        for (int kap = 0; kap < NKMAX; ++kap) {
            float rt[CT][8];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int S = 2 * kap + half;
                f32x4 pks[CT];
                if (S < NT) {
                    ks0(S, pks);
                } else {
#pragma unroll
                    for (int st = 0; st < CT; ++st) pks[st] = f32x4{0.f, 0.f, 0.f, 0.f};
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int srow = 16 * S + 4 * lg + rr;
                    const uint32_t w = srow < N ? vraw[S][rr] : 0u;
                    const float gm = gam[srow];
#pragma unroll
                    for (int st = 0; st < CT; ++st) {
                        const float vv = __uint_as_float(st == 0 ? w << 16 : w & 0xFFFF0000u);
                        rt[st][4 * half + rr] = vv - gm * pks[st][rr];
                    }
                }
            }
#pragma unroll
            for (int st = 0; st < CT; ++st) split8(rt[st], rh[st][kap], rl[st][kap]);
        }

        GDN_PHASE(5);
        // O tiles: gamma o (Q S0^T) + Z~ R'
        {
            // per 16-row tile: its Q rows and its row blocks of Z~ (from the
            // pair list, in the X area, free after the solve) staged in LDS
            // by the whole workgroup, then each wavefront's columns
            unsigned char* Zt = smem + L::XC;
            unsigned char* Qt = smem + L::QT;
            auto q_frag_t = [&](int r, int ks) -> bf16x8 { return load_frag(Qt + r * L::KROW + 2 * (8 * KS * lg + 8 * ks)); };
            // this thread's 16-byte piece of a tile's Q rows, one tile ahead
            static_assert(16 * (DK / 8) <= NTH, "one Q piece per thread");
            const int qr = tid / (DK / 8), qc = tid % (DK / 8);
            auto load_q = [&](int I) {
                const int row = 16 * I + qr;
                uint4 val = make_uint4(0u, 0u, 0u, 0u);
                if (tid < 16 * (DK / 8) && row < N)
                    val = *reinterpret_cast<const uint4*>(qg + ((static_cast<size_t>(b) * N + row) * Hk + kh) * DK + 8 * qc);
                return val;
            };
            uint4 qv = load_q(0);
            for (int I = 0; I < NT; ++I) {
                const int nb = I / 2 + 1;
                for (int e = tid; e < nb * 128; e += NTH) reinterpret_cast<uint4*>(Zt)[e] = make_uint4(0u, 0u, 0u, 0u);
                if (tid < 16 * (DK / 8)) *reinterpret_cast<uint4*>(Qt + qr * L::KROW + 16 * qc) = qv;
                qv = load_q(min(I + 1, NT - 1));
                __syncthreads();
                // the pairs of rows 16 I .. 16 I + 15 are contiguous in the list
                const int p0 = off[16 * I];
                const int p1 = 16 * I + 16 < N ? off[16 * I + 16] : total;
                for (int p = p0 + tid; p < p1; p += NTH) {
                    const int i = pnode[p], tt = pathc[p];
                    const float zz = qk[p];
                    const __bf16 zh = static_cast<__bf16>(zz);
                    const __bf16 zl = static_cast<__bf16>(zz - static_cast<float>(zh));
                    const int e = (((((tt >> 2) & 3) << 4) | (i & 15)) << 3) + (((tt >> 4) & 1) << 2) + (tt & 3);
                    unsigned char* blk = Zt + 2048 * (tt >> 5);
                    reinterpret_cast<__bf16*>(blk)[e] = zh;
                    reinterpret_cast<__bf16*>(blk + 1024)[e] = zl;
                }
                __syncthreads();
                f32x4 acc[CT];
                {
                    f32x4 ah[CT], al[CT];
#pragma unroll
                    for (int st = 0; st < CT; ++st) ah[st] = al[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 qa = q_frag_t(lc, ks);
#pragma unroll
                        for (int st = 0; st < CT; ++st) {
                            ah[st] = mfma(s0h[st][ks], qa, ah[st]);
                            al[st] = mfma(s0l[st][ks], qa, al[st]);
                        }
                    }
                    const float gi = gam[16 * I + lc];
#pragma unroll
                    for (int st = 0; st < CT; ++st) acc[st] = (ah[st] + al[st]) * gi;
                }
                const unsigned char* blk = Zt + 16 * lane;
#pragma unroll
                for (int kap = 0; kap < NKMAX; ++kap) {
                    if (kap >= nb) break;
                    const bf16x8 zh = load_frag(blk + 2048 * kap);
                    const bf16x8 zl = load_frag(blk + 2048 * kap + 1024);
#pragma unroll
                    for (int st = 0; st < CT; ++st) {
                        acc[st] = mfma(rh[st][kap], zh, acc[st]);
                        acc[st] = mfma(rl[st][kap], zh, acc[st]);
                        acc[st] = mfma(rh[st][kap], zl, acc[st]);
                    }
                }
                // transposed tile: lane (lc, lg) holds value columns
                // 16 w + 4 lg .. + 3 of node 16 I + lc, one 16-byte store;
                // o is not read back here
                {
                    static_assert(CT == 1, "one 16-column tile per wavefront");
                    const int i = 16 * I + lc;
                    if (i < N)
                        __builtin_nontemporal_store(
                            acc[0], reinterpret_cast<f32x4*>(a.o + static_cast<size_t>(b) * N * Hv * DV + static_cast<size_t>(h) * DV +
                                                             16 * wave + 4 * lg + static_cast<size_t>(i) * Hv * DV));
                }
                __syncthreads();  // the tile's LDS is rewritten for the next one
            }
        }
        GDN_PHASE(6);
        cur_b = b;
        cur_kh = kh;
        __syncthreads();  // the next item rewrites LDS
        GDN_PHASE(7);
    }
    GDN_PHASE_END;
}


// wavefronts per workgroup: one 16-column tile each (two per SIMD at
// d_v = 128, which hides more latency than four of two tiles)
#ifndef GDN_FAST_WAVES
#define GDN_FAST_WAVES(dk, dv) ((dv) / 16)
#endif
template <int NMAX, int DK, int DV>
hipError_t verify_fast(const VerifyArgs& a, hipStream_t stream) {
    constexpr int NW = GDN_FAST_WAVES(DK, DV);
    const int items = a.B * a.H_v;
    const int wgs = min(items, device_cus());
    const int per = (items + wgs - 1) / wgs;
    const dim3 grid(static_cast<unsigned>((items + per - 1) / per));
    hipLaunchKernelGGL((verify_fast_kernel<NMAX, DK, DV, NW>), grid, dim3(64 * NW), 0, stream, a, per);
    return hipGetLastError();
}


}  // namespace

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (!cached[dev]) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
    if (a.qkv_dtype != GDN_BF16 || a.force_walk) return launch_verify_simple(a, stream);
    // trees of up to 128 nodes: one workgroup per compute unit, tree and
    // dense parts of consecutive items overlapped on separate wavefronts
    if (a.N <= 128) return launch_verify_ws(a, stream);
    // larger trees: the two-launch verify over the context's workspace;
    // without one (the allocation-free entry point) this file's kernel
    if (a.split_ws) return launch_verify_split(a, stream);
    if (a.d_k == 128) return a.d_v == 128 ? verify_fast<256, 128, 128>(a, stream) : verify_fast<256, 128, 64>(a, stream);
    return a.d_v == 128 ? verify_fast<256, 64, 128>(a, stream) : verify_fast<256, 64, 64>(a, stream);
}

}  // namespace gdn
