// gdn_verify_grp.hip -- MFMA tree verification for bf16 q/k/v and trees of at
// most 128 nodes on gfx950: one 8-wavefront workgroup per compute unit.
//
// The arithmetic is that of gdn_fast.hip (Trees from Marginals technical
// summary, Methodology, "3. Rollback-Free Tree Verification for GDN"):
//     X_is = beta_i D_is (k_i . k_s)  (s a strict ancestor of i),
//     Y_is = D_is (q_i . k_s)         (s an ancestor of i, or i),
//     Z~ = Y (I + X)^-1 diag(beta),  R' = V - gamma o (K S0^T),
//     O = gamma o (Q S0^T) + Z~ R',
// with Z~ built one row per node by back-substitution along its root path.
//
// Layout of the work:
//  - items (sequence b, value head h) are dealt to persistent workgroups in
//    contiguous runs; a run is taken in groups of two heads that share a key
//    head (one head when they do not);
//  - per group (the tree part): the tree structure and the list of 16 x 16
//    tiles holding ancestor pairs (once per sequence), K and Q staged in LDS
//    (once per key head), the Gram values k_i . k_s and q_i . k_s of the
//    pairs on MFMA turned into X and Y of both heads, and the rows of Z~
//    with one thread per (node, head);
//  - per head (the dense part): its Z~ scattered into dense MFMA A
//    fragments, then every wavefront takes 16 value columns: S0 slice split
//    into bf16 hi + lo, K S0^T -> R' (hi + lo), per 16-node tile
//    gamma o (Q S0^T) + Z~ R' -> o.
//  - memory stays busy: while a head's dense part runs, the S0 rows and V
//    columns of the next item are already being loaded into registers (the
//    current item's are consumed by then), and the next group's node scalars
//    and K/Q are prefetched the same way.
//
// Trees whose pair list exceeds the LDS budget are verified, inside the same
// workgroup, by the per-node walk of gdn_walk.h.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"
#include "gdn_mfma.h"
#include "gdn_walk.h"

// Phase boundaries: empty in the product build; a profiling build defines
// them to accumulate per-phase cycle counts.
#ifndef GDN_PHASE
#define GDN_PHASE_INIT
#define GDN_PHASE(k)
#define GDN_PHASE_END
#endif

namespace gdn {
namespace {

// 16 x 32 blocks of Z~ for the first I row tiles (row tile I has k-steps
// 0 .. I/2 of 32 nodes each).
__host__ __device__ constexpr int grp_zblocks(int I) {
    return (I & 1) ? ((I + 1) / 2) * ((I + 1) / 2) : (I / 2) * (I / 2 + 1);
}

template <int NMAX, int DK>
struct GrpLds {
    static constexpr int GH = 2;                 // value heads per group
    // pair-list capacity: every tree of N <= 64 fits; for N <= 128 the
    // paths may sum to 1536 nodes (12 per node on average)
    static constexpr int CAP = NMAX <= 64 ? NMAX * (NMAX + 1) / 2 : 1536;
    static constexpr int AW = NMAX / 32;         // ancestor bit-row words
    static constexpr int NTILE = (NMAX / 16) * (NMAX / 16 + 1) / 2;  // lower 16x16 tiles
    static constexpr int KQ_BYTES = NMAX * DK * 2;
    static constexpr int KS_OFF = 0;             // K rows (k-slot order, chunks XOR-swizzled by row)
    static constexpr int QS_OFF = KQ_BYTES;      // Q rows, same
    static constexpr int ZD = 2 * KQ_BYTES;      // Z~ fragments of the current head
    static constexpr int ZD_BYTES = 2048 * grp_zblocks(NMAX / 16);  // hi 1 KiB + lo 1 KiB per block
    static constexpr int XSTR = CAP + 16;        // X row of a head (16 zero pads)
    static constexpr int XC = ZD + ZD_BYTES;     // float[GH][XSTR]
    static constexpr int YC = XC + 4 * GH * XSTR;  // float[GH][CAP]: Y, then the rows of Z~
    static constexpr int OFP = YC + 4 * GH * CAP;  // uint16[CAP]: path offset of the ancestor
    static constexpr int PATH = OFP + 2 * CAP;   // uint8[CAP]: root..i path of every node
    static constexpr int PNODE = PATH + CAP;     // uint8[CAP]: node owning each pair
    static constexpr int TILES = (PNODE + CAP + 3) & ~3;  // uint16[NTILE]: (I << 4 | J) of tiles with pairs
    static constexpr int NODE = (TILES + 2 * NTILE + 15) & ~15;
    static constexpr int PAR = NODE;             // int[NMAX]
    static constexpr int DEP = PAR + 4 * NMAX;
    static constexpr int OFF = DEP + 4 * NMAX;
    static constexpr int NXT = OFF + 4 * NMAX;
    static constexpr int GV = NXT + 4 * NMAX;    // float[GH][NMAX]: g
    static constexpr int BET = GV + 4 * GH * NMAX;
    static constexpr int GG = BET + 4 * GH * NMAX;   // G (path sum of g)
    static constexpr int GAM = GG + 4 * GH * NMAX;   // gamma (0 past N)
    static constexpr int ANC = GAM + 4 * GH * NMAX;  // uint32[NMAX][AW]
    static constexpr int TMASK = ANC + 4 * AW * NMAX;  // uint32[NMAX/16]
    static constexpr int MISC = TMASK + 4 * (NMAX / 16);
    static constexpr int TOTAL = MISC + 64;
    // the fallback walk's buffers (u [NMAX][64], S0 slice [DK][64], k and q
    // rows) overwrite K/Q, the fragments and X/Y
    static constexpr int FB_S0 = NMAX * 64 * 4;
    static constexpr int FB_KQ = FB_S0 + DK * 64 * 4;
    static_assert(FB_KQ + 8 * DK <= OFP, "fallback buffers must fit below the pair structure");
    static_assert(TOTAL <= 160 * 1024, "LDS of one compute unit");
};

template <int NMAX, int DK, int DV>
__global__ __launch_bounds__(512) void verify_grp_kernel(VerifyArgs a, int items_per_wg) {
    using L = GrpLds<NMAX, DK>;
    constexpr int GH = L::GH;
    constexpr int NW = 8;
    constexpr int NTH = 64 * NW;
    constexpr int NDW = DV / 16;         // wavefronts in the dense part, 16 value columns each
    constexpr int KS = DK / 32;          // MFMA k-steps over d_k
    constexpr int CH = DK / 8;           // 16-byte chunks per K/Q row
    constexpr int NTMAX = NMAX / 16;
    constexpr int NKMAX = NMAX / 32;
    constexpr int KCH = (NMAX * CH + NTH - 1) / NTH;  // K (and Q) chunks staged per thread
    constexpr int ZR = 16;               // path length solved in registers
    constexpr int TPW = (L::NTILE + NW - 1) / NW;     // Gram tiles per wavefront
    static_assert(GH * NMAX <= NTH, "one (node, head) per thread");
    static_assert(NDW <= NW, "dense wavefronts");
    static_assert(L::NTILE <= 64, "tile list built by one wavefront");

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
    const bool dense_on = wave < NDW;

    const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
    const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
    const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);

    unsigned char* Ks = smem + L::KS_OFF;
    unsigned char* Qs = smem + L::QS_OFF;
    unsigned char* Zd = smem + L::ZD;
    float* xc = reinterpret_cast<float*>(smem + L::XC);
    float* yc = reinterpret_cast<float*>(smem + L::YC);
    uint16_t* ofp = reinterpret_cast<uint16_t*>(smem + L::OFP);
    uint8_t* pathc = smem + L::PATH;
    uint8_t* pnode = smem + L::PNODE;
    uint16_t* tiles = reinterpret_cast<uint16_t*>(smem + L::TILES);
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

    // a group: two consecutive heads of one sequence that share a key head,
    // else one head
    auto group_size = [&](int it) {
        const int h = it % Hv;
        return (it + 1 < it_end && h + 1 < Hv && (h + 1) / R == h / R) ? 2 : 1;
    };

    // Prefetched state.  Loads are unconditional with indices clamped into
    // range; out-of-range values are replaced after arrival.
    //  - node scalars of the next group, K/Q of the next key head;
    int p_pf;
    float g_pf[GH], b_pf[GH];
    uint4 k_pf[KCH], q_pf[KCH];
    auto prefetch_scalars = [&](int it, int tid, int N) {
        const int bb = it / Hv, hh = it % Hv, nh = group_size(it);
        const int i = min(tid, N - 1);
        p_pf = a.parent[static_cast<size_t>(bb) * N + i];
#pragma unroll
        for (int e = 0; e < GH; ++e) {
            const size_t idx = (static_cast<size_t>(bb) * N + i) * Hv + hh + min(e, nh - 1);
            g_pf[e] = a.g[idx];
            b_pf[e] = a.beta[idx];
        }
    };
    auto prefetch_kq = [&](int it, int tid, int N) {
        const int bb = it / Hv, kh = (it % Hv) / R;
#pragma unroll
        for (int q = 0; q < KCH; ++q) {
            const int e = min(tid + q * NTH, NMAX * CH - 1);
            const int row = min(e / CH, N - 1);
            const size_t gofs = ((static_cast<size_t>(bb) * N + row) * Hk + kh) * DK + (e % CH) * 8;
            k_pf[q] = *reinterpret_cast<const uint4*>(kg + gofs);
            q_pf[q] = *reinterpret_cast<const uint4*>(qg + gofs);
        }
    };
    //  - S0 rows and V of the next item for this wavefront's 16 value
    //    columns: lane (lc, lg) holds, in s0n[2 ks + h], d_k columns
    //    32 ks + 16 h + 4 lg .. + 3 of S0 row 16 w + lc (64 contiguous bytes
    //    per row and instruction), and in vn[S] value columns
    //    16 w + 4 lg .. + 3 of node 16 S + lc (the A operand of a 16x16x16
    //    MFMA against the identity, which turns it into the layout of
    //    K S0^T: column lc, nodes 16 S + 4 lg + r).
    float4 s0n[2 * KS];
    uint2 vn[NTMAX];
    auto prefetch_sv = [&](int it, int tid, int N) {
        const int bb = it / Hv, hh = it % Hv;
        const int lane = tid & 63, lc = lane & 15, lg = lane >> 4;
        const int c0 = 16 * (wave % NDW);
        const float4* src =
            reinterpret_cast<const float4*>(a.S0 + ((static_cast<size_t>(bb) * Hv + hh) * DV + c0 + lc) * DK + 4 * lg);
#pragma unroll
        for (int q = 0; q < 2 * KS; ++q) s0n[q] = src[4 * q];
        const uint16_t* vsrc = vg + static_cast<size_t>(bb) * N * Hv * DV + static_cast<size_t>(hh) * DV + c0 + 4 * lg;
#pragma unroll
        for (int S = 0; S < NTMAX; ++S)
            vn[S] = *reinterpret_cast<const uint2*>(vsrc + static_cast<size_t>(min(16 * S + lc, N - 1)) * Hv * DV);
    };

    // MFMA k-slot order: in k-step ks, lane group g holds d_k indices
    // 32 ks + 16 h + 4 g + r in slot 4 h + r (h < 2, r < 4).  A staged K/Q
    // row keeps each lane group's 8 slots in one 16-byte chunk: element
    // 32 ks + 16 h + 4 g + r sits at position 32 ks + 8 g + 4 h + r, chunk
    // 4 ks + g, stored at chunk position (4 ks + g) ^ (row mod CH).
    auto stage_kq = [&](int tid, int N) {
#pragma unroll
        for (int q = 0; q < KCH; ++q) {
            const int e = tid + q * NTH;
            if (e < NMAX * CH) {
                // global chunk c holds elements 8c .. 8c + 7 of the row: two
                // 4-element halves for lane groups g0 and g0 + 1
                const int row = e / CH, c = e % CH;
                const int ks = c >> 2, m = c & 3, hh = m >> 1, g0 = (m & 1) << 1;
                const int sw = row & (CH - 1);
                const int rbase = row * (DK * 2) + 8 * hh;
                const int pos0 = rbase + (((4 * ks + g0) ^ sw) << 4);
                const int pos1 = rbase + (((4 * ks + g0 + 1) ^ sw) << 4);
                const uint32_t keep = row < N ? 0xFFFFFFFFu : 0u;
                const uint4 kk = k_pf[q], qq = q_pf[q];
                *reinterpret_cast<uint2*>(Ks + pos0) = make_uint2(kk.x & keep, kk.y & keep);
                *reinterpret_cast<uint2*>(Ks + pos1) = make_uint2(kk.z & keep, kk.w & keep);
                *reinterpret_cast<uint2*>(Qs + pos0) = make_uint2(qq.x & keep, qq.y & keep);
                *reinterpret_cast<uint2*>(Qs + pos1) = make_uint2(qq.z & keep, qq.w & keep);
            }
        }
    };
    // MFMA fragment (row, k-step ks) of staged K or Q for lane group lg
    auto frag = [&](const unsigned char* base, int row, int lg, int ks) -> bf16x8 {
        return load_frag(base + row * (DK * 2) + (((4 * ks + lg) ^ (row & (CH - 1))) << 4));
    };

    GDN_PHASE_INIT;
    prefetch_scalars(it_begin, tid0, N0);
    __builtin_amdgcn_sched_barrier(0);
    prefetch_sv(it_begin, tid0, N0);
    __builtin_amdgcn_sched_barrier(0);
    prefetch_kq(it_begin, tid0, N0);

    int cur_b = -1, cur_kh = -1, total = 0;
    bool zd_clean = false;  // the fragments hold only entries at the current tree's pair positions
    for (int it = it_begin; it < it_end;) {
        // Opaque copies of the thread index and N: values derived from them
        // are recomputed per group instead of being hoisted out of the loop
        // and held in registers across it.
        int tid = tid0, N = N0;
        asm volatile("" : "+v"(tid));
        asm volatile("" : "+s"(N));
        const int lane = tid & 63;
        const int lc = lane & 15;
        const int lg = lane >> 4;
        const int b = it / Hv, h0 = it % Hv;
        const int nh = group_size(it);
        const int kh = h0 / R;
        const bool new_b = b != cur_b;
        const bool new_kh = new_b || kh != cur_kh;
        const int nit = it + nh < it_end ? it + nh : -1;
        const bool next_new_kh = nit >= 0 && (nit / Hv != b || (nit % Hv) / R != kh);
        GDN_PHASE(0);

        // ---- node scalars of the group's heads; for a new sequence the
        // tree structure
        int bad_local = 0;
        if (tid < NMAX) {
            const int i = tid;
#pragma unroll
            for (int e = 0; e < GH; ++e) {
                gv[e * NMAX + i] = i < N ? g_pf[e] : 0.f;
                bet[e * NMAX + i] = i < N ? b_pf[e] : 0.f;
            }
            if (new_b) {
                int p = i < N ? p_pf : -1;
                if (p < -1 || p >= i) {
                    bad_local = 1;
                    p = -1;
                }
                par[i] = p;
                nxt[i] = p;
                dep[i] = i < N ? 1 : 0;
            }
        }
        if (nit >= 0) prefetch_scalars(nit, tid, N);
        GDN_PHASE(9);
        if (new_b) {
            if (tid < NMAX / 16) tmask[tid] = 0u;
            const int bad = __syncthreads_or(bad_local);
            if (h0 == 0 && tid == 0) a.tree_status[b] = bad ? GDN_ERR_TREE : 0;
            // depth by pointer jumping: dep[i] counts the nodes from i up to nxt[i]
            for (int round = 0; round < 9; ++round) {
                int c2 = 0, n2 = -1, live = 0;
                if (tid < NMAX) {
                    const int nx = nxt[tid];
                    c2 = dep[tid] + (nx >= 0 ? dep[nx] : 0);
                    n2 = nx >= 0 ? nxt[nx] : -1;
                    live = n2 >= 0;
                }
                __syncthreads();
                if (tid < NMAX) {
                    dep[tid] = c2;
                    nxt[tid] = n2;
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
            if (total <= L::CAP && tid < NMAX) {
                // root..i path, owner and ancestor offsets of every pair;
                // ancestor bits; tiles holding pairs
                const int i = tid;
                uint32_t bits[L::AW];
#pragma unroll
                for (int w = 0; w < L::AW; ++w) bits[w] = 0u;
                if (i < N) {
                    int pos = off[i] + dep[i] - 1;
                    uint32_t mask = 0u;
                    for (int s = i; s >= 0; s = par[s]) {
                        pathc[pos] = static_cast<uint8_t>(s);
                        pnode[pos] = static_cast<uint8_t>(i);
                        ofp[pos] = static_cast<uint16_t>(off[s]);
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
            zd_clean = false;
        }
        GDN_PHASE(10);
        if (total <= L::CAP && !zd_clean) {
            for (int e = tid; e < L::ZD_BYTES / 16; e += NTH)
                reinterpret_cast<uint4*>(Zd)[e] = make_uint4(0u, 0u, 0u, 0u);
            zd_clean = true;
        }
        __syncthreads();
        GDN_PHASE(1);

        if (total > L::CAP) {
            // deep tree: the per-node walk by wavefront 0, one head and one
            // 64-column slice at a time (it overwrites K/Q and the fragments)
            if (wave == 0) {
                float* u_s = reinterpret_cast<float*>(smem);
                float* s0_s = reinterpret_cast<float*>(smem + L::FB_S0);
                float* ki = reinterpret_cast<float*>(smem + L::FB_KQ);
                for (int e = 0; e < nh; ++e)
                    for (int c0 = 0; c0 < DV; c0 += 64)
                        walk_verify_slice_lds<uint16_t, DK, WaveSync>(a, b, h0 + e, c0, par, u_s, Gs, ki, ki + DK,
                                                                      s0_s);
            }
            // the prefetched S0/V of this group's items are unused on this
            // path: drain them, then prefetch for the next group
            __builtin_amdgcn_s_waitcnt(0);
            if (nit >= 0) {
                prefetch_sv(nit, tid, N);
                prefetch_kq(nit, tid, N);
            }
            zd_clean = false;
            cur_b = b;
            cur_kh = -1;   // K/Q are overwritten: restage for the next group
            it += nh;
            __syncthreads();
            continue;
        }

        // this group's K/Q (prefetched during the previous group) into LDS;
        // for a new sequence, the list of tiles holding pairs
        if (new_kh) stage_kq(tid, N);
        if (new_b && wave == NW - 1) {
            const int NT = (N + 15) >> 4;
            int I = 0;
            while ((I + 1) * (I + 2) / 2 <= lane) ++I;
            const int J = lane - I * (I + 1) / 2;
            const bool has = lane < L::NTILE && I < NT && ((tmask[min(I, NTMAX - 1)] >> J) & 1u);
            const uint64_t m = __ballot(has);
            const int idx = __popcll(m & ((1ull << lane) - 1ull));
            if (has) tiles[idx] = static_cast<uint16_t>((I << 4) | J);
            if (lane == 0) misc[1] = __popcll(m);
        }

        // ---- G and gamma per (node, head)
        if (tid < GH * NMAX) {
            const int e = tid / NMAX, i = tid % NMAX;
            float G = 0.f;
            if (i < N && e < nh) {
                const int o = off[i], m = dep[i];
                const float* ge = gv + e * NMAX;
                if (m <= ZR) {
                    int tt[ZR];
#pragma unroll
                    for (int bb = 0; bb < ZR; ++bb) tt[bb] = pathc[o + min(bb, m - 1)];
#pragma unroll
                    for (int bb = 0; bb < ZR; ++bb) G += bb < m ? ge[tt[bb]] : 0.f;
                } else {
                    for (int bb = 0; bb < m; ++bb) G += ge[pathc[o + bb]];
                }
            }
            Gs[tid] = G;
            gam[tid] = (i < N && e < nh) ? __expf(G) : 0.f;
        }
        __syncthreads();
        GDN_PHASE(2);

        // ---- Gram values of the ancestor pairs on MFMA, turned into X and
        // Y of the group's heads; the listed tiles are dealt round-robin to
        // the wavefronts, all of a wavefront's tiles in flight together.  The
        // value of pair (i, s) lands at path position dep[s] - 1 of node i.
        {
            const int ntiles = misc[1];
            f32x4 akk[TPW], aqk[TPW];
            int tcode[TPW];
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                const int t = wave + NW * j;
                tcode[j] = t < ntiles ? tiles[t] : -1;
                akk[j] = aqk[j] = f32x4{0.f, 0.f, 0.f, 0.f};
                __builtin_amdgcn_sched_barrier(0);   // one tile's fragments in registers at a time
                if (tcode[j] >= 0) {
                    const int I = tcode[j] >> 4, J = tcode[j] & 15;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 kb = frag(Ks, 16 * J + lc, lg, ks);
                        akk[j] = mfma(frag(Ks, 16 * I + lc, lg, ks), kb, akk[j]);
                        aqk[j] = mfma(frag(Qs, 16 * I + lc, lg, ks), kb, aqk[j]);
                    }
                }
            }
            // scatter: every LDS read of a tile issued up front, stores
            // predicated on the ancestor bit
#pragma unroll
            for (int j = 0; j < TPW; ++j) {
                __builtin_amdgcn_sched_barrier(0);
                if (tcode[j] < 0) continue;
                const int I = tcode[j] >> 4, J = tcode[j] & 15;
                const int s = 16 * J + lc;
                const int ds = dep[s];
                float gsv[GH], giv[GH][4], biv[GH][4];
                uint32_t aw[4];
                int oi[4];
#pragma unroll
                for (int e = 0; e < GH; ++e) gsv[e] = Gs[e * NMAX + s];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int i = 16 * I + 4 * lg + rr;
                    aw[rr] = anc[i * L::AW + (s >> 5)];
                    oi[rr] = off[i];
#pragma unroll
                    for (int e = 0; e < GH; ++e) {
                        giv[e][rr] = Gs[e * NMAX + i];
                        biv[e][rr] = bet[e * NMAX + i];
                    }
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int i = 16 * I + 4 * lg + rr;
                    if (i < N && ((aw[rr] >> (s & 31)) & 1u)) {
                        const int p = oi[rr] + ds - 1;
#pragma unroll
                        for (int e = 0; e < GH; ++e) {
                            if (e < nh) {
                                const float D = __expf(giv[e][rr] - gsv[e]);
                                xc[e * L::XSTR + p] = biv[e][rr] * D * akk[j][rr];
                                yc[e * L::CAP + p] = D * aqk[j][rr];
                            }
                        }
                    }
                }
            }
        }
        if (tid < 16) {
#pragma unroll
            for (int e = 0; e < GH; ++e) xc[e * L::XSTR + total + tid] = 0.f;  // pads for the solve below
        }
        __syncthreads();
        GDN_PHASE(3);

        // ---- per (node, head) its row of Z~ by a right-looking sweep along
        // its path, written back over Y
        if (tid < GH * NMAX) {
            const int e = tid / NMAX, i = tid % NMAX;
            if (i < N && e < nh) {
                const float* xe = xc + e * L::XSTR;
                float* ye = yc + e * L::CAP;
                const float* be = bet + e * NMAX;
                const int o = off[i], m = dep[i];
                if (m <= ZR) {
                    // branch-free: entries past the path are zero and their X
                    // reads land on finite values (pairs of later nodes or the
                    // zero pads), so loads can be issued early
                    int tt[ZR], oa[ZR];
                    float z[ZR];
#pragma unroll
                    for (int bb = 0; bb < ZR; ++bb) {
                        const int pp = o + min(bb, m - 1);
                        tt[bb] = pathc[pp];
                        oa[bb] = ofp[pp];
                        z[bb] = bb < m ? ye[pp] : 0.f;
                    }
                    float xr[ZR - 1];
#pragma unroll
                    for (int bb = 0; bb < ZR - 1; ++bb) xr[bb] = xe[oa[ZR - 1] + bb];
#pragma unroll
                    for (int aa = ZR - 1; aa >= 1; --aa) {
                        float xn[ZR - 1];
#pragma unroll
                        for (int bb = 0; bb + 1 < aa; ++bb) xn[bb] = xe[oa[aa - 1] + bb];
                        const float za = z[aa];
#pragma unroll
                        for (int bb = 0; bb < aa; ++bb) z[bb] -= za * xr[bb];
#pragma unroll
                        for (int bb = 0; bb + 1 < aa; ++bb) xr[bb] = xn[bb];
                        __builtin_amdgcn_sched_barrier(0);
                    }
#pragma unroll
                    for (int bb = 0; bb < ZR; ++bb)
                        if (bb < m) ye[o + bb] = z[bb] * be[tt[bb]];
                } else {
                    for (int aa = m - 1; aa >= 1; --aa) {
                        const float za = ye[o + aa];
                        const int oa = ofp[o + aa];
                        for (int bb = 0; bb < aa; ++bb) ye[o + bb] -= za * xe[oa + bb];
                    }
                    for (int bb = 0; bb < m; ++bb) ye[o + bb] *= be[pathc[o + bb]];
                }
            }
        }
        GDN_PHASE(4);

        // ---- dense part, one head at a time
        for (int e = 0; e < nh; ++e) {
            // Opaque copies again: addresses below are recomputed per head
            // rather than hoisted out of this loop.
            int tid = tid0, N = N0;
            asm volatile("" : "+v"(tid));
            asm volatile("" : "+s"(N));
            const int lane = tid & 63;
            const int lc = lane & 15;
            const int lg = lane >> 4;
            const int h = h0 + e;
            const int nxt_it = it + e + 1 < it_end ? it + e + 1 : -1;

            // Z~ of this head into MFMA A fragments: block (I, kap) holds rows
            // 16I.., nodes 32kap..; node t sits in lane group ((t >> 2) & 3),
            // slot 4 ((t >> 4) & 1) + (t & 3).  Heads of one sequence write
            // the same positions, so no clearing is needed between them.
            __syncthreads();   // the rows of Z~ are complete, the previous head's fragments read
            {
                const float* ze = yc + e * L::CAP;
                for (int p = tid; p < total; p += NTH) {
                    const int i = pnode[p], t = pathc[p];
                    const float z = ze[p];
                    const __bf16 zh = static_cast<__bf16>(z);
                    const __bf16 zl = static_cast<__bf16>(z - static_cast<float>(zh));
                    const int el = (((((t >> 2) & 3) << 4) | (i & 15)) << 3) + (((t >> 4) & 1) << 2) + (t & 3);
                    unsigned char* blk = Zd + 2048 * (grp_zblocks(i >> 4) + (t >> 5));
                    reinterpret_cast<__bf16*>(blk)[el] = zh;
                    reinterpret_cast<__bf16*>(blk + 1024)[el] = zl;
                }
            }
            __syncthreads();
            GDN_PHASE(5);

            if (dense_on) {
                const float* ge = gam + e * NMAX;
                // this item's S0 and V from the prefetch registers; then the
                // next item's loads go into them
                bf16x8 s0h[KS], s0l[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const float4 x0 = s0n[2 * ks], x1 = s0n[2 * ks + 1];
                    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                    split8(x, s0h[ks], s0l[ks]);
                }
                uint2 vc[NTMAX];
#pragma unroll
                for (int S = 0; S < NTMAX; ++S) vc[S] = vn[S];
                if (nxt_it >= 0) prefetch_sv(nxt_it, tid, N);
                GDN_PHASE(11);

                // P = M S0^T of row tile S for M = K or Q, this wavefront's columns
                auto ms0 = [&](const unsigned char* base, int S, int lcx, int lgx) -> f32x4 {
                    f32x4 ah = {0.f, 0.f, 0.f, 0.f}, al = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 fa = frag(base, 16 * S + lcx, lgx, ks);
                        ah = mfma(fa, s0h[ks], ah);
                        al = mfma(fa, s0l[ks], al);
                    }
                    return ah + al;
                };

                // R' = V - gamma o (K S0^T) as B fragments of the Z~ R'
                // product: k-step kap covers nodes [32 kap, 32 kap + 32); lane
                // (lc, lg) holds rows 32 kap + 16 half + 4 lg + rr in slot
                // 4 half + rr.
                // identity for the V transpose: lane (n, g) holds B[4g + j][n]
                s16x4 eye;
#pragma unroll
                for (int j = 0; j < 4; ++j) eye[j] = 4 * lg + j == lc ? static_cast<short>(0x3F80) : short(0);
                const int NT = (N + 15) >> 4;
                bf16x8 rh[NKMAX], rl[NKMAX];
#pragma unroll
                for (int kap = 0; kap < NKMAX; ++kap) {
                    float rt[8];
#pragma unroll
                    for (int half = 0; half < 2; ++half) {
                        const int S = 2 * kap + half;
                        if (S < NT) {
                            // gamma is 0 past N; V of the clamped rows is
                            // masked by a select (no branch around the LDS read)
                            const f32x4 pk = ms0(Ks, S, lc, lg);
                            const f32x4 vt = mfma16(__builtin_bit_cast(s16x4, vc[S]), eye, f32x4{0.f, 0.f, 0.f, 0.f});
                            const f32x4 gm = *reinterpret_cast<const f32x4*>(ge + 16 * S + 4 * lg);
#pragma unroll
                            for (int rr = 0; rr < 4; ++rr) {
                                const int srow = 16 * S + 4 * lg + rr;
                                const float vv = srow < N ? vt[rr] : 0.f;
                                rt[4 * half + rr] = vv - gm[rr] * pk[rr];
                            }
                        } else {
#pragma unroll
                            for (int rr = 0; rr < 4; ++rr) rt[4 * half + rr] = 0.f;
                        }
                    }
                    split8(rt, rh[kap], rl[kap]);
                }
                GDN_PHASE(6);

                // O tiles, transposed so that a lane holds 4 adjacent value
                // columns of one node: O^T = gamma o (S0 Q^T) + R'^T Z~^T
                // (the same fragments with A and B swapped); lane (lc, lg)
                // gets columns 16 w + 4 lg .. + 3 of node 16 I + lc.
                float* obase = a.o + static_cast<size_t>(b) * N * Hv * DV + static_cast<size_t>(h) * DV + 16 * wave + 4 * lg;
#pragma unroll
                for (int I = 0; I < NTMAX; ++I) {
                    if (I < NT) {
                        f32x4 ah = {0.f, 0.f, 0.f, 0.f}, al = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int ks = 0; ks < KS; ++ks) {
                            const bf16x8 fb = frag(Qs, 16 * I + lc, lg, ks);
                            ah = mfma(s0h[ks], fb, ah);
                            al = mfma(s0l[ks], fb, al);
                        }
                        f32x4 acc = (ah + al) * ge[16 * I + lc];
                        const unsigned char* blk = Zd + 2048 * grp_zblocks(I) + 16 * lane;
#pragma unroll
                        for (int kap = 0; kap <= I / 2; ++kap) {
                            const bf16x8 zh = load_frag(blk + 2048 * kap);
                            const bf16x8 zl = load_frag(blk + 2048 * kap + 1024);
                            acc = mfma(rh[kap], zh, acc);
                            acc = mfma(rl[kap], zh, acc);
                            acc = mfma(rh[kap], zl, acc);
                        }
                        const int i = 16 * I + lc;
                        if (i < N) *reinterpret_cast<f32x4*>(obase + static_cast<size_t>(i) * Hv * DV) = acc;
                    }
                }
                GDN_PHASE(7);
            } else if (nxt_it >= 0) {
                prefetch_sv(nxt_it, tid, N);   // keeps every wavefront's registers in step
            }
        }
        // the next group's K/Q, when it starts a new key head: into
        // registers now, into LDS once that group has built its structure
        if (next_new_kh) prefetch_kq(nit, tid, N);
        cur_b = b;
        cur_kh = kh;
        it += nh;
        __syncthreads();  // the next group rewrites LDS
    }
    GDN_PHASE_END;
}

}  // namespace

hipError_t launch_verify_grp(const VerifyArgs& a, hipStream_t stream) {
    const int items = a.B * a.H_v;
    const int wgs = min(items, device_cus());
    int per = (items + wgs - 1) / wgs;
    per += per & 1;   // whole head pairs per workgroup
    const dim3 grid((items + per - 1) / per);
    auto go = [&](auto kern) {
        hipLaunchKernelGGL(kern, grid, dim3(512), 0, stream, a, per);
        return hipGetLastError();
    };
    if (a.N <= 64) {
        if (a.d_k == 64) return a.d_v == 64 ? go(verify_grp_kernel<64, 64, 64>) : go(verify_grp_kernel<64, 64, 128>);
        return a.d_v == 64 ? go(verify_grp_kernel<64, 128, 64>) : go(verify_grp_kernel<64, 128, 128>);
    }
    if (a.d_k == 64) return a.d_v == 64 ? go(verify_grp_kernel<128, 64, 64>) : go(verify_grp_kernel<128, 64, 128>);
    return a.d_v == 64 ? go(verify_grp_kernel<128, 128, 64>) : go(verify_grp_kernel<128, 128, 128>);
}

}  // namespace gdn
