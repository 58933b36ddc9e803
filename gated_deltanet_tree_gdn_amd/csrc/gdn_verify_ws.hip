// gdn_verify_ws.hip -- MFMA tree verification for bf16 q/k/v and trees of at
// most 128 nodes on gfx950, with the tree part and the dense part of
// consecutive items running at the same time on different wavefronts.
//
// The arithmetic is that of gdn_fast.hip (Trees from Marginals technical
// summary, Methodology, "3. Rollback-Free Tree Verification for GDN"):
//     X_is = beta_i D_is (k_i . k_s)  (s a strict ancestor of i),
//     Y_is = D_is (q_i . k_s)         (s an ancestor of i, or i),
//     Z~ = Y (I + X)^-1 diag(beta),  R' = V - gamma o (K S0^T),
//     O = gamma o (Q S0^T) + Z~ R',
// with Z~ built one row per node by back-substitution along its root path.
//
// One persistent workgroup per compute unit takes a run of (sequence b,
// value head h) items, with d_v / 16 dense wavefronts (8 at d_v = 128, two
// per SIMD) and 4 tree wavefronts.  Two roles:
//  - tree wavefronts (the last four) prepare item j+1: node scalars; for a
//    new sequence the tree structure (depth, root paths, ancestor bits, the
//    16 x 16 tiles holding ancestor pairs); for a new key head the Gram
//    values k_i . k_s and q_i . k_s of the pairs (MFMA; K and Q of the key
//    head sit in these wavefronts' registers, two row tiles each, and four
//    column tiles at a time are broadcast through LDS); the gates G, gamma;
//    the rows of Z~.  Results go to one of two LDS slots.  The same
//    K/Q registers are written to LDS, in the dense side's fragment order,
//    when the dense side moves to the new key head;
//  - dense wavefronts finish item j meanwhile: its Z~ (from the other slot)
//    scattered into dense MFMA fragments, then per wavefront 16 value
//    columns: S0 split into bf16 hi + lo, K S0^T -> R', and per 16-node tile
//    gamma o (S0 Q^T) + R'^T Z~^T (transposed, so a lane stores 16
//    contiguous bytes).  The two 16-column halves of each 128-byte piece of
//    an o row belong to the two dense wavefronts of one SIMD, which store
//    them close together in time, so L2 mostly writes whole lines.
// The roles meet once per item at a workgroup barrier (twice when K/Q
// change); inside a role the wavefronts synchronise through an LDS counter
// (a bounded spin: a fault in the protocol ends the wait instead of hanging
// the device, and is reported in the sequence status).  The dense
// wavefronts load the next item's S0 and V right after their last MFMA of
// the current item, so those loads overlap the barrier and the scatter; the
// tree wavefronts load the next item's scalars, and the next key head's K/Q,
// one item ahead.
//
// Trees whose pair list exceeds the LDS budget are verified by the per-node
// walk of gdn_walk.h on the dense side.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"
#include "gdn_mfma.h"
#include "gdn_walk.h"

#ifndef GDN_PHASE
#define GDN_PHASE_INIT
#define GDN_PHASE(k)
#define GDN_PHASE_SNAP
#define GDN_PHASE_ITER(j)
#define GDN_PHASE_ARRIVE(j)
#define GDN_PHASE_END
#endif

namespace gdn {
namespace {

__host__ __device__ constexpr int ws_zblocks(int I) {
    return (I & 1) ? ((I + 1) / 2) * ((I + 1) / 2) : (I / 2) * (I / 2 + 1);
}
__host__ __device__ constexpr int ws_align(int x, int a) { return (x + a - 1) / a * a; }

template <int NMAX, int DK>
struct WsLds {
    // pair-list capacity: every tree of N <= 64 fits; for N <= 128 the
    // paths may sum to 2048 nodes, which holds every tree of depth <= 16
    static constexpr int CAP = NMAX <= 64 ? NMAX * (NMAX + 1) / 2 : 2048;
    static constexpr int AW = NMAX / 32;
    // dense side
    static constexpr int KQ_BYTES = NMAX * DK * 2;
    static constexpr int KS_OFF = 0;                 // K rows (k-slot order, chunks XOR-swizzled)
    static constexpr int QS_OFF = KQ_BYTES;          // Q rows
    static constexpr int ZD = 2 * KQ_BYTES;          // Z~ fragments of the dense item
    static constexpr int ZD_BYTES = 2048 * ws_zblocks(NMAX / 16);
    // hand-over slots (tree side writes slot (j+1)&1, dense side reads j&1)
    // hand-over slots s = 0, 1, each: float[CAP] Y, then the rows of Z~;
    // float[NMAX] gamma (0 past N).  The pair positions (ancestor and node
    // of each pair) are the tree side's own arrays, which it rewrites for a
    // new sequence only once the dense side has scattered its last item.
    static constexpr int SLOT = ws_align(4 * CAP + 4 * NMAX, 16);
    static constexpr int SLOTS = ZD + ZD_BYTES;
    static constexpr int S_GAM = 4 * CAP;
    static constexpr int SLOTS_END = SLOTS + 2 * SLOT;
    // tree side
    // k_i . k_s (float[CAP + 4 + 16]) and q_i . k_s (float[CAP + 4]) per key
    // head: entry CAP takes the Gram tile entries that are not ancestor
    // pairs; entries CAP + 4 .. CAP + 19 of k_i . k_s stay zero (the row the
    // solve reads for path positions past a node's depth)
    static constexpr int GB0 = ws_align(SLOTS_END, 16);
    static constexpr int KK = GB0 + 32 * DK;
    static constexpr int KZERO = CAP + 4;
    static constexpr int QK = KK + 4 * (CAP + 4 + 16);
    static constexpr int PATH = QK + 4 * (CAP + 4);  // uint8[CAP]: the root..i path of every node i
    static constexpr int PNODE = PATH + CAP;         // uint8[CAP]: node i owning each pair
    static constexpr int NODE = ws_align(PNODE + CAP, 16);
    static constexpr int PAR = NODE;                 // int[NMAX]
    static constexpr int DEP = PAR + 4 * NMAX;
    static constexpr int OFF = DEP + 4 * NMAX;
    static constexpr int BADP = OFF + 4 * NMAX;   // int[NMAX]: 1 where the parent is invalid
    static constexpr int GV = BADP + 4 * NMAX;        // float[NMAX]: g of the tree item
    static constexpr int BET = GV + 4 * NMAX;        // beta
    static constexpr int GG = BET + 4 * NMAX;        // G
    static constexpr int ANC = GG + 4 * NMAX;        // uint32[NMAX][AW]
    static constexpr int TMASK = ANC + 4 * AW * NMAX;
    static constexpr int MISC = TMASK + 4 * (NMAX / 16);  // int[16]
    // Gram broadcast of 16-row tiles of K (KS fragments x 64 lanes x 16
    // bytes each), four at a time: buffers 0 and 1 are their own, 2 and 3
    // overlay the hand-over slot of the item being built (free until its
    // rows of Z~ are written)
    static constexpr int GB_BYTES = 32 * DK;
    static constexpr int GB1 = MISC + 64;
    static_assert(2 * GB_BYTES <= SLOT, "Gram buffers 2 and 3 must fit in a hand-over slot");
    static constexpr int TOTAL = GB1 + GB_BYTES;
    // misc[]: 0 tree total, 2 dense sync counter, 3 tree sync counter,
    // 4 spin time-outs, 5/6 slot pair totals, 7/8 slot fallback flags,
    // 9 invalid-parent flag, 10 items the dense side has scattered
    // the fallback walk (dense side) overwrites K/Q and the fragments:
    // u [NMAX][64], S0 slice [DK][64], k and q rows, G, parents
    static constexpr int FB_S0 = NMAX * 64 * 4;
    static constexpr int FB_KQ = FB_S0 + DK * 64 * 4;
    static constexpr int FB_G = FB_KQ + 8 * DK;
    static constexpr int FB_PAR = FB_G + 4 * NMAX;
    static constexpr bool HAS_FALLBACK = CAP < NMAX * (NMAX + 1) / 2;
    static_assert(!HAS_FALLBACK || FB_PAR + 4 * NMAX <= SLOTS, "fallback buffers must fit in the dense area");
    static_assert(TOTAL <= 160 * 1024, "LDS of one compute unit");
};

// Barrier among the `nwaves` wavefronts of one role: an LDS counter that
// only grows; the caller tracks how many of these it has passed.  The wait
// is bounded: on a time-out it records the fact and returns, and every
// later wait of the workgroup returns at once.
__device__ __forceinline__ void role_sync(int* ctr, int nwaves, int& count, int* timeouts) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    ++count;
    const int target = count * nwaves;
    for (int spins = 0; __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target; ++spins) {
        // after one time-out the counts no longer match: stop waiting
        if (spins > (1 << 22) || __hip_atomic_load(timeouts, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) {
            __hip_atomic_store(timeouts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Wait until the LDS counter `ctr` reaches `target` (bounded like role_sync).
__device__ __forceinline__ void role_wait(int* ctr, int target, int* timeouts) {
    for (int spins = 0; __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target; ++spins) {
        if (spins > (1 << 22) || __hip_atomic_load(timeouts, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) {
            __hip_atomic_store(timeouts, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            break;
        }
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int NMAX, int DK, int DV, int NWD>
__global__ __launch_bounds__(64 * (NWD + 4)) void verify_ws_kernel(VerifyArgs a, int items_per_wg) {
    using L = WsLds<NMAX, DK>;
    // NWD dense wavefronts
    constexpr int NWT = 4;               // tree wavefronts
    constexpr int TTH = 64 * NWT;
    constexpr int CW = DV / NWD;         // value columns per dense wavefront
    constexpr int CT = CW / 16;          // 16-column tiles per dense wavefront
    constexpr int KS = DK / 32;
    constexpr int CH = DK / 8;           // 16-byte chunks per K/Q row
    constexpr int NTMAX = NMAX / 16;
    constexpr int NKMAX = NMAX / 32;
    constexpr int ZR = 16;
    static_assert(NMAX <= TTH, "one node per tree thread");
    static_assert(CT >= 1 && CW * NWD == DV, "whole 16-column tiles per dense wavefront");
    constexpr int RT = NTMAX / NWT;      // K/Q row tiles held per tree wavefront
    static_assert(RT >= 1 && RT <= 2 && NTMAX == RT * NWT, "row tiles per tree wavefront");

    __shared__ __align__(16) unsigned char smem[L::TOTAL];

    const int Hk = a.H_k, Hv = a.H_v;
    const int R = Hv / Hk;
    const int n_items = a.B * Hv;
    // Workgroups go to the 8 XCDs in turn; numbering them so that each XCD
    // takes consecutive items keeps the heads of a sequence on one XCD, whose
    // L2 then serves their shared rows of g, beta and the parents once
    const int wg = gridDim.x % 8 == 0 ? (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8 : blockIdx.x;
    const int it_begin = wg * items_per_wg;
    const int it_end = min(it_begin + items_per_wg, n_items);
    if (it_begin >= it_end) return;
    const int nit = it_end - it_begin;

    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const bool is_tree = wave >= NWD;
    const int twave = wave - NWD;
    // The thread index and N are refreshed through opaque copies once per
    // item: addresses derived from them are then recomputed per item rather
    // than hoisted out of the item loops and held in registers across them.
    int tid, lane, lc, lg, ttid, N;
    auto refresh = [&]() {
        int t = threadIdx.x, n = a.N;
        asm volatile("" : "+v"(t));
        asm volatile("" : "+s"(n));
        tid = t;
        lane = t & 63;
        lc = lane & 15;
        lg = lane >> 4;
        ttid = t - 64 * NWD;   // tree thread index
        N = n;
    };
    refresh();
    GDN_PHASE_INIT;

    const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
    const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
    const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);

    unsigned char* Ks = smem + L::KS_OFF;
    unsigned char* Qs = smem + L::QS_OFF;
    unsigned char* Zd = smem + L::ZD;
    auto slot_base = [&](int sl) { return smem + L::SLOTS + sl * L::SLOT; };
    auto zout_s = [&](int sl) { return reinterpret_cast<float*>(slot_base(sl)); };
    auto gamd_s = [&](int sl) { return reinterpret_cast<float*>(slot_base(sl) + L::S_GAM); };
    float* kk = reinterpret_cast<float*>(smem + L::KK);
    float* qk = reinterpret_cast<float*>(smem + L::QK);
    uint8_t* pathc = smem + L::PATH;
    uint8_t* pnode = smem + L::PNODE;
    int* par = reinterpret_cast<int*>(smem + L::PAR);
    int* dep = reinterpret_cast<int*>(smem + L::DEP);
    int* off = reinterpret_cast<int*>(smem + L::OFF);
    int* badp = reinterpret_cast<int*>(smem + L::BADP);
    float* gv = reinterpret_cast<float*>(smem + L::GV);
    float* bet = reinterpret_cast<float*>(smem + L::BET);
    float* Gs = reinterpret_cast<float*>(smem + L::GG);
    uint32_t* anc = reinterpret_cast<uint32_t*>(smem + L::ANC);
    uint32_t* tmask = reinterpret_cast<uint32_t*>(smem + L::TMASK);
    int* misc = reinterpret_cast<int*>(smem + L::MISC);
    bf16x8* gbuf0 = reinterpret_cast<bf16x8*>(smem + L::GB0);
    bf16x8* gbuf1 = reinterpret_cast<bf16x8*>(smem + L::GB1);

    auto item_b = [&](int j) { return (it_begin + j) / Hv; };
    auto item_h = [&](int j) { return (it_begin + j) % Hv; };
    auto item_kh = [&](int j) { return item_h(j) / R; };

    int dsync = 0, tsync = 0;
    auto dense_sync = [&]() { role_sync(misc + 2, NWD, dsync, misc + 4); };
    auto tree_sync = [&]() { role_sync(misc + 3, NWT, tsync, misc + 4); };
    // the dense side counts the items whose pair positions it has read
    auto dense_scattered = [&]() {
        if (tid == 0) {
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
            __hip_atomic_fetch_add(misc + 10, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
    };
    auto wait_scattered = [&](int n) { role_wait(misc + 10, n, misc + 4); };

    // ---------------------------------------------------------------- tree side
    // K and Q of an item's key head live in the tree wavefronts' registers,
    // loaded once per key head: tree wavefront w holds row tiles I_0 = w and
    // I_1 = NTMAX - 1 - w (balanced triangle), lane (lc, lg) row 16 I + lc,
    // elements 8 KS lg .. + 8 KS - 1 as KS MFMA fragments (natural k order).
    // They feed the Gram values and are then written to LDS for the dense
    // side in its k-slot order: element 32 ks + 16 h + 4 g + r at position
    // 32 ks + 8 g + 4 h + r, chunk 4 ks + g, stored at chunk position
    // (4 ks + g) ^ (row mod CH).
    auto tile_of = [&](int u) { return u == 0 ? twave : NTMAX - 1 - twave; };
    bf16x8 kf[RT][KS], qf[RT][KS];
    auto load_kq = [&](int j) {
        const int bb = item_b(j), kh = item_kh(j);
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            const int row = min(16 * tile_of(u) + lc, N - 1);
            const size_t gofs = ((static_cast<size_t>(bb) * N + row) * Hk + kh) * DK + 8 * KS * lg;
            const bf16x8* kp = reinterpret_cast<const bf16x8*>(kg + gofs);
            const bf16x8* qp = reinterpret_cast<const bf16x8*>(qg + gofs);
#pragma unroll
            for (int t = 0; t < KS; ++t) {
                kf[u][t] = kp[t];
                qf[u][t] = qp[t];
            }
        }
    };
    // natural 16-byte chunk c of K/Q row `row` (elements 8c .. 8c + 7) into
    // LDS: two 4-element halves, for lane groups g0 and g0 + 1; rows past N
    // are zero
    auto put_chunk = [&](int row, int c, uint4 kv, uint4 qv) {
        const uint32_t keep = row < N ? 0xFFFFFFFFu : 0u;
        const int sw = row & (CH - 1);
        const int ks = c >> 2, m = c & 3, hh = m >> 1, g0 = (m & 1) << 1;
        const int rbase = row * (DK * 2) + 8 * hh;
        const int pos0 = rbase + (((4 * ks + g0) ^ sw) << 4);
        const int pos1 = rbase + (((4 * ks + g0 + 1) ^ sw) << 4);
        *reinterpret_cast<uint2*>(Ks + pos0) = make_uint2(kv.x & keep, kv.y & keep);
        *reinterpret_cast<uint2*>(Ks + pos1) = make_uint2(kv.z & keep, kv.w & keep);
        *reinterpret_cast<uint2*>(Qs + pos0) = make_uint2(qv.x & keep, qv.y & keep);
        *reinterpret_cast<uint2*>(Qs + pos1) = make_uint2(qv.z & keep, qv.w & keep);
    };
    // (sequence, key head) whose K/Q the registers hold; loaded on demand
    int kq_b = -1, kq_kh = -1;
    auto hold_kq = [&](int j) {
        if (item_b(j) != kq_b || item_kh(j) != kq_kh) {
            load_kq(j);
            kq_b = item_b(j);
            kq_kh = item_kh(j);
        }
    };
    auto stage_kq = [&]() {
#pragma unroll
        for (int u = 0; u < RT; ++u)
#pragma unroll
            for (int t = 0; t < KS; ++t)
                put_chunk(16 * tile_of(u) + lc, KS * lg + t, __builtin_bit_cast(uint4, kf[u][t]),
                          __builtin_bit_cast(uint4, qf[u][t]));
    };
    // node scalars of the next tree item, loaded ahead
    float g_pf, b_pf;
    int p_pf;
    auto load_scalars = [&](int j) {
        const int bb = item_b(j), hh = item_h(j);
        const int i = min(ttid, N - 1);
        const size_t nh = (static_cast<size_t>(bb) * N + i) * Hv + hh;
        g_pf = a.g[nh];
        b_pf = a.beta[nh];
        p_pf = a.parent[static_cast<size_t>(bb) * N + i];
    };

    // Gram tile (I, J) (lane: rows 16 I + 4 lg + rr, column 16 J + lc) into
    // the pair list: the value of pair (i, s) lands at path position
    // dep[s] - 1 of node i
    auto put_pairs = [&](int I, int J, const f32x4& akk, const f32x4& aqk) {
        const int sn = 16 * J + lc;
        const int ds = dep[sn];
        uint32_t aw[4];
        int oi[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int i = 16 * I + 4 * lg + rr;
            aw[rr] = anc[i * L::AW + (sn >> 5)];
            oi[rr] = off[i];
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int i = 16 * I + 4 * lg + rr;
            if (i < N && ((aw[rr] >> (sn & 31)) & 1u)) {
                const int p = oi[rr] + ds - 1;
                kk[p] = akk[rr];
                qk[p] = aqk[rr];
            }
        }
    };

    // tree part of item j into slot j & 1
    int t_b = -1, t_kh = -1, t_total = 0;
    // node scalars of item j into LDS; for a new sequence its parents (a
    // parent outside [-1, i - 1] is flagged in badp and treated as a root)
    auto tree_scalars = [&](int j) {
        const bool new_b = item_b(j) != t_b;
        if (ttid < NMAX) {
            const int i = ttid;
            gv[i] = i < N ? g_pf : 0.f;
            bet[i] = i < N ? b_pf : 0.f;
            if (new_b) {
                const int p = i < N ? p_pf : -1;
                const bool bad = p < -1 || p >= i;
                par[i] = bad ? -1 : p;
                badp[i] = bad ? 1 : 0;
            }
        }
        if (new_b && ttid < NMAX / 16) tmask[ttid] = 0u;
    };
    // a new sequence: depth, path offsets, paths, ancestor bits, tile mask
    auto tree_struct = [&](int j) {
        const int b = item_b(j), h = item_h(j);
        GDN_PHASE(5);
        {
            tree_sync();
            GDN_PHASE(1);
            // depth: every node walks up to its root (parents precede their
            // children, so each walk ends)
            if (ttid < NMAX) {
                int d = 0;
                if (ttid < N)
                    for (int s = ttid; s >= 0; s = par[s]) ++d;
                dep[ttid] = d;
            }
            tree_sync();
            GDN_PHASE(2);
            // offsets of the paths in the pair list (exclusive scan) and the
            // invalid-parent flag, by the first tree wavefront
            if (twave == 0) {
                constexpr int E = NMAX / 64;
                int vals[E];
                int sum = 0, bad = 0;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    vals[e] = dep[lane * E + e];
                    sum += vals[e];
                    bad |= badp[lane * E + e];
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
                const bool any_bad = __ballot(bad != 0) != 0ull;
                if (lane == 63) misc[0] = incl;
                if (lane == 0) misc[9] = any_bad ? 1 : 0;
            }
            tree_sync();
            GDN_PHASE(3);
            if (h == 0 && ttid == 0) a.tree_status[b] = misc[9] ? GDN_ERR_TREE : 0;
            t_total = misc[0];
            // the dense side reads the previous sequence's pair positions
            // at the start of its item j - 1
            if (j > 0) wait_scattered(j);
            if (t_total <= L::CAP && ttid < NMAX) {
                const int i = ttid;
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
            tree_sync();
            t_b = b;
            t_kh = -1;
        }
    };
    // the item's pair total and walk flag for the dense side; false for an
    // item the dense side walks
    auto tree_check = [&](int j) -> bool {
        const int slot = j & 1;
        const int total = t_total;
        if (ttid == 0) {
            misc[5 + slot] = total;
            misc[7 + slot] = total > L::CAP ? 1 : 0;
        }
        if (total > L::CAP) {
            tree_sync();
            return false;
        }
        return true;
    };
    // G and gamma per node
    auto tree_g = [&](int j) {
        const int slot = j & 1;
        GDN_PHASE(8);
        // g of every node written, the Gram buffers in the slot read
        tree_sync();
        GDN_PHASE(9);
        // G and gamma per node
        if (ttid < NMAX) {
            const int i = ttid;
            float G = 0.f;
            if (i < N) {
                const int o = off[i], m = dep[i];
                if (m <= ZR) {
                    int tt[ZR];
#pragma unroll
                    for (int bb = 0; bb < ZR; ++bb) tt[bb] = pathc[o + min(bb, m - 1)];
#pragma unroll
                    for (int bb = 0; bb < ZR; ++bb) G += bb < m ? gv[tt[bb]] : 0.f;
                } else {
                    for (int bb = 0; bb < m; ++bb) G += gv[pathc[o + bb]];
                }
            }
            Gs[i] = G;
            gamd_s(slot)[i] = i < N ? __expf(G) : 0.f;
        }
        GDN_PHASE(10);
    };
    // Gram values k_i . k_s and q_i . k_s of the ancestor pairs, for a new key
    // head: rounds of four column tiles J, whose K rows their owners
    // broadcast through LDS; each wavefront multiplies them with its own row
    // tiles I >= J that hold pairs
    auto tree_gram = [&](int j) {
        bf16x8* gbuf[4] = {gbuf0, gbuf1, reinterpret_cast<bf16x8*>(slot_base(j & 1)),
                           reinterpret_cast<bf16x8*>(slot_base(j & 1) + L::GB_BYTES)};
        const int NT = (N + 15) >> 4;
        // this wavefront's row tiles: their tile-mask words and the path
        // offsets of their rows
        uint32_t tmr[RT];
        int offr[RT][4];
#pragma unroll
        for (int u = 0; u < RT; ++u) {
            tmr[u] = tmask[tile_of(u)];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) offr[u][rr] = off[16 * tile_of(u) + 4 * lg + rr];
        }
        for (int J0 = 0; J0 < NT; J0 += 4) {
            if (J0 > 0) tree_sync();   // the previous round's tiles are read
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int J = J0 + v;
                const int owner = J < NWT ? J : NTMAX - 1 - J;
                if (J < NT && twave == owner) {
#pragma unroll
                    for (int t = 0; t < KS; ++t) gbuf[v][t * 64 + lane] = (RT > 1 && J >= NWT) ? kf[RT - 1][t] : kf[0][t];
                }
            }
            tree_sync();
            if (J0 == 0) GDN_PHASE(0); else GDN_PHASE(7);
            // the ancestor words of this wavefront's rows for the round's
            // column tiles (node s = 16 J + lc sits in word J / 2)
            uint32_t aw[RT][4][2];
#pragma unroll
            for (int u = 0; u < RT; ++u)
#pragma unroll
                for (int rr = 0; rr < 4; ++rr)
#pragma unroll
                    for (int x = 0; x < 2; ++x)
                        aw[u][rr][x] = anc[(16 * tile_of(u) + 4 * lg + rr) * L::AW + min((J0 >> 1) + x, L::AW - 1)];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int J = J0 + v;
                if (J >= NT) continue;
                bf16x8 kb[KS];
#pragma unroll
                for (int t = 0; t < KS; ++t) kb[t] = gbuf[v][t * 64 + lane];
                const int sn = 16 * J + lc;
                const int ds = dep[sn];
#pragma unroll
                for (int u = 0; u < RT; ++u) {
                    const int I = tile_of(u);
                    if (I >= J && I < NT && ((tmr[u] >> J) & 1u)) {
                        f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int t = 0; t < KS; ++t) {
                            akk = mfma(kf[u][t], kb[t], akk);
                            aqk = mfma(qf[u][t], kb[t], aqk);
                        }
                        // entries that are not ancestor pairs go to the sink
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const int i = 16 * I + 4 * lg + rr;
                            const bool pair = i < N && ((aw[u][rr][v >> 1] >> (sn & 31)) & 1u);
                            const int p = pair ? offr[u][rr] + ds - 1 : L::CAP;
                            kk[p] = akk[rr];
                            qk[p] = aqk[rr];
                        }
                    }
                }
            }
            if (J0 == 0) GDN_PHASE(4);
        }
        t_kh = item_kh(j);
    };
    // The rows of Z~.  With D_is = exp(G_i - G_s), the row w of node i in
    // Y (I + X)^-1 satisfies w_b = Y_{i,t_b} - sum_{a > b} w_a X_{t_a,t_b}
    // along its root path t_0 .. t_{m-1} = i.  Since D_{i,t_a} D_{t_a,t_b} =
    // D_{i,t_b}, w_b = D_{i,t_b} y_b with
    //     y_b = q_i . k_{t_b} - sum_{a > b} (beta_{t_a} y_a) (k_{t_a} . k_{t_b}),
    // so the sweep runs on the Gram values and beta alone (no per-pair gate
    // factors, no quotient of gates), and Z~_{i,t_b} = y_b beta_{t_b} D_{i,t_b}.
    auto tree_tail = [&](int j) {
        const int slot = j & 1;
        tree_sync();
        GDN_PHASE(11);
        float* ye = zout_s(slot);
        GDN_PHASE(12);
        // per node its row of Z~ by a right-looking sweep along its path
        if (ttid < N) {
            const int i = ttid;
            const int o = off[i], m = dep[i];
            const float Gi = Gs[i];
            if (m <= ZR) {
                // path positions past the depth read the zero row of kk
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
                    if (bb < m) ye[o + bb] = y[bb] * bt[bb] * __expf(Gi - Gs[pathc[o + bb]]);
            } else {
                for (int bb = 0; bb < m; ++bb) ye[o + bb] = qk[o + bb];
                for (int aa = m - 1; aa >= 1; --aa) {
                    const int ta = pathc[o + aa];
                    const float ya = ye[o + aa] * bet[ta];
                    const int oa = off[ta];
                    for (int bb = 0; bb < aa; ++bb) ye[o + bb] -= ya * kk[oa + bb];
                }
                for (int bb = 0; bb < m; ++bb) {
                    const int t = pathc[o + bb];
                    ye[o + bb] *= bet[t] * __expf(Gi - Gs[t]);
                }
            }
        }
        tree_sync();
        GDN_PHASE(13);
    };
    auto tree_item = [&](int j) {
        const bool new_b = item_b(j) != t_b;
        const bool new_kh = new_b || item_kh(j) != t_kh;
        if (new_b) tree_struct(j);
        if (!tree_check(j)) return;
        if (new_kh) {
            hold_kq(j);
            tree_gram(j);
        }
        tree_g(j);
        tree_tail(j);
    };

    // --------------------------------------------------------------- dense side
    // S0 rows and V of an item for this wavefront's CW value columns:
    // s0r[st][2 ks + h] holds d_k columns 32 ks + 16 h + 4 lg .. + 3 of row
    // CW w + 16 st + lc; vr[st][S] holds value columns CW w + 16 st + 4 lg ..
    // + 3 of node 16 S + lc (the A operand of a 16x16x16 MFMA against the
    // identity, which turns it into the layout of K S0^T).
    float4 s0r[CT][2 * KS];
    uint2 vr[CT][NTMAX];
    // value columns of this wavefront: the two 16-column halves of each
    // 128-byte row piece of o go to the two dense wavefronts of one SIMD
    const int colbase = (NWD == 8 && CW == 16) ? 32 * (wave & 3) + 16 * (wave >> 2) : CW * wave;
    // real == 0 (after the last item) keeps the loads, which hold the
    // registers to one value per item, but points every lane at one line
    auto load_sv = [&](int j, int real) {
        const int bb = item_b(j), hh = item_h(j);
        const int lcr = lc * real, lgr = lg * real;
#pragma unroll
        for (int st = 0; st < CT; ++st) {
            const int c0 = (colbase + 16 * st) * real;
            const float4* src = reinterpret_cast<const float4*>(
                a.S0 + ((static_cast<size_t>(bb) * Hv + hh) * DV + c0 + lcr) * DK + 4 * lgr);
#pragma unroll
            for (int q = 0; q < 2 * KS; ++q) s0r[st][q] = src[4 * q * real];
            const uint16_t* vsrc = vg + static_cast<size_t>(bb) * N * Hv * DV + static_cast<size_t>(hh) * DV + c0 + 4 * lgr;
#pragma unroll
            for (int S = 0; S < NTMAX; ++S)
                vr[st][S] = *reinterpret_cast<const uint2*>(
                    vsrc + static_cast<size_t>(min(16 * S + lc, N - 1)) * Hv * DV * real);
        }
    };
    auto frag = [&](const unsigned char* base, int row, int ks) -> bf16x8 {
        return load_frag(base + row * (DK * 2) + (((4 * ks + lg) ^ (row & (CH - 1))) << 4));
    };

    int d_zb = -1;   // sequence whose pair positions the fragments hold (-1: dirty)
    auto dense_item = [&](int j) {
        const int b = item_b(j), h = item_h(j);
        const int slot = j & 1;
        const int total = misc[5 + slot];
        const bool more = j + 1 < nit;
        if (L::HAS_FALLBACK && misc[7 + slot]) {
            // deep tree: the per-node walk by dense wavefront 0 (the others
            // go on to the next item's loads and wait at the item barrier)
            dense_scattered();
            __builtin_amdgcn_s_waitcnt(0);   // this item's S0/V loads are unused
            if (wave == 0) {
                int* par_s = reinterpret_cast<int*>(smem + L::FB_PAR);
                float* G_s = reinterpret_cast<float*>(smem + L::FB_G);
                for (int i = lane; i < N; i += 64) {
                    const int p = a.parent[static_cast<size_t>(b) * N + i];
                    par_s[i] = (p < -1 || p >= i) ? -1 : p;
                }
                WaveSync::sync();
                float* u_s = reinterpret_cast<float*>(smem);
                float* s0_s = reinterpret_cast<float*>(smem + L::FB_S0);
                float* ki = reinterpret_cast<float*>(smem + L::FB_KQ);
                for (int c0 = 0; c0 < DV; c0 += 64)
                    walk_verify_slice_lds<uint16_t, DK, WaveSync>(a, b, h, c0, par_s, u_s, G_s, ki, ki + DK, s0_s);
            }
            d_zb = -1;
            load_sv(more ? j + 1 : j, more ? 1 : 0);
            return;
        }
        if (d_zb != b) {
            for (int e = tid; e < L::ZD_BYTES / 16; e += 64 * NWD) reinterpret_cast<uint4*>(Zd)[e] = make_uint4(0u, 0u, 0u, 0u);
            dense_sync();
            d_zb = b;
        }
        GDN_PHASE(0);
        // Z~ into MFMA A fragments: block (I, kap) holds rows 16I.., nodes
        // 32kap..; node t sits in lane group ((t >> 2) & 3), slot
        // 4 ((t >> 4) & 1) + (t & 3).  Items of one sequence write the same
        // positions, so no clearing is needed between them.
        {
            const float* ze = zout_s(slot);
            const uint8_t* sp = pathc;
            const uint8_t* sn = pnode;
            for (int p = tid; p < total; p += 64 * NWD) {
                const int i = sn[p], t = sp[p];
                const float z = ze[p];
                const __bf16 zh = static_cast<__bf16>(z);
                const __bf16 zl = static_cast<__bf16>(z - static_cast<float>(zh));
                const int el = (((((t >> 2) & 3) << 4) | (i & 15)) << 3) + (((t >> 4) & 1) << 2) + (t & 3);
                unsigned char* blk = Zd + 2048 * (ws_zblocks(i >> 4) + (t >> 5));
                reinterpret_cast<__bf16*>(blk)[el] = zh;
                reinterpret_cast<__bf16*>(blk + 1024)[el] = zl;
            }
        }
        dense_sync();
        dense_scattered();

        GDN_PHASE(1);
        const float* ge = gamd_s(slot);
        const int NT = (N + 15) >> 4;
        bf16x8 s0h[CT][KS], s0l[CT][KS];
#pragma unroll
        for (int st = 0; st < CT; ++st)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const float4 x0 = s0r[st][2 * ks], x1 = s0r[st][2 * ks + 1];
                const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
                split8(x, s0h[st][ks], s0l[st][ks]);
            }
        // identity for the V transpose: lane (n, g) holds B[4g + j][n]
        s16x4 eye;
#pragma unroll
        for (int q = 0; q < 4; ++q) eye[q] = 4 * lg + q == lc ? static_cast<short>(0x3F80) : short(0);

        GDN_PHASE(2);
        // R' = V - gamma o (K S0^T) as B fragments of the Z~ R' product
        bf16x8 rh[CT][NKMAX], rl[CT][NKMAX];
#pragma unroll
        for (int kap = 0; kap < NKMAX; ++kap) {
            float rt[CT][8];
#pragma unroll
            for (int half = 0; half < 2; ++half) {
                const int S = 2 * kap + half;
                if (S < NT) {
                    f32x4 ah[CT], al[CT];
#pragma unroll
                    for (int st = 0; st < CT; ++st) ah[st] = al[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        const bf16x8 fa = frag(Ks, 16 * S + lc, ks);
#pragma unroll
                        for (int st = 0; st < CT; ++st) {
                            ah[st] = mfma(fa, s0h[st][ks], ah[st]);
                            al[st] = mfma(fa, s0l[st][ks], al[st]);
                        }
                    }
                    const f32x4 gm = *reinterpret_cast<const f32x4*>(ge + 16 * S + 4 * lg);
#pragma unroll
                    for (int st = 0; st < CT; ++st) {
                        const f32x4 vt = mfma16(__builtin_bit_cast(s16x4, vr[st][S]), eye, f32x4{0.f, 0.f, 0.f, 0.f});
                        const f32x4 pk = ah[st] + al[st];
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) {
                            const float vv = 16 * S + 4 * lg + rr < N ? vt[rr] : 0.f;
                            rt[st][4 * half + rr] = vv - gm[rr] * pk[rr];
                        }
                    }
                } else {
#pragma unroll
                    for (int st = 0; st < CT; ++st)
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) rt[st][4 * half + rr] = 0.f;
                }
            }
#pragma unroll
            for (int st = 0; st < CT; ++st) split8(rt[st], rh[st][kap], rl[st][kap]);
        }

        GDN_PHASE(3);
        // O tiles, transposed: O^T = gamma o (S0 Q^T) + R'^T Z~^T; lane
        // (lc, lg) gets value columns CW w + 16 st + 4 lg .. + 3 of node 16 I + lc
        float* obase = a.o + static_cast<size_t>(b) * N * Hv * DV + static_cast<size_t>(h) * DV + colbase + 4 * lg;
#pragma unroll
        for (int I = 0; I < NTMAX; ++I) {
            if (I < NT) {
                f32x4 ah[CT], al[CT];
#pragma unroll
                for (int st = 0; st < CT; ++st) ah[st] = al[st] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 fb = frag(Qs, 16 * I + lc, ks);
#pragma unroll
                    for (int st = 0; st < CT; ++st) {
                        ah[st] = mfma(s0h[st][ks], fb, ah[st]);
                        al[st] = mfma(s0l[st][ks], fb, al[st]);
                    }
                }
                const float gi = ge[16 * I + lc];
                f32x4 acc[CT];
#pragma unroll
                for (int st = 0; st < CT; ++st) acc[st] = (ah[st] + al[st]) * gi;
                const unsigned char* blk = Zd + 2048 * ws_zblocks(I) + 16 * lane;
#pragma unroll
                for (int kap = 0; kap <= I / 2; ++kap) {
                    const bf16x8 zh = load_frag(blk + 2048 * kap);
                    const bf16x8 zl = load_frag(blk + 2048 * kap + 1024);
#pragma unroll
                    for (int st = 0; st < CT; ++st) {
                        acc[st] = mfma(rh[st][kap], zh, acc[st]);
                        acc[st] = mfma(rl[st][kap], zh, acc[st]);
                        acc[st] = mfma(rh[st][kap], zl, acc[st]);
                    }
                }
                // o is written once and not read back here: streaming stores
                const int i = 16 * I + lc;
                if (i < N) {
#pragma unroll
                    for (int st = 0; st < CT; ++st)
                        __builtin_nontemporal_store(acc[st], reinterpret_cast<f32x4*>(obase + static_cast<size_t>(i) * Hv * DV + 16 * st));
                }
            }
        }
        GDN_PHASE(4);
        // the next item's S0 and V: in flight across the barrier and scatter
        // (unconditional, so that the registers hold one value per item)
        load_sv(more ? j + 1 : j, more ? 1 : 0);
        GDN_PHASE(5);
    };

    // ----------------------------------------------------------------- schedule
    // The two roles run separate loops that pass the same workgroup barriers
    // in the same order: per item one barrier, and a second one when K/Q in
    // LDS change for the next item (its key head or sequence differs, or a
    // walk overwrote them); the tree side writes them from its registers
    // between the two.
    auto restage_after = [&](int j) {
        return j + 1 < nit && (item_b(j + 1) != item_b(j) || item_kh(j + 1) != item_kh(j) ||
                               (L::HAS_FALLBACK && misc[7 + (j & 1)]));
    };
    if (tid < 16) misc[tid] = 0;
    if (tid >= 64 && tid < 64 + 16) kk[L::KZERO + tid - 64] = 0.f;
    __syncthreads();
    // a key head (or sequence) starts at item j: K/Q go into the registers
    auto new_kq_at = [&](int j) {
        return j > 0 && j < nit && (item_b(j) != item_b(j - 1) || item_kh(j) != item_kh(j - 1));
    };
    // Start-up (first item): the tree side loads the scalars and builds the
    // structure; meanwhile the dense side stages the first key head's K/Q
    // straight into LDS and computes every lower Gram tile from LDS, which it
    // scatters into the pair list once the structure is known.  Its S0/V
    // loads go out only while the tree side solves for the first item: the
    // memory queue is then free of the start-up's own loads, which would
    // otherwise hold up the Gram tiles behind them.  Workgroup barriers
    // B1 .. B4 order the two.
    constexpr int NTILE0 = NTMAX * (NTMAX + 1) / 2;
    constexpr int GT0 = (NTILE0 + NWD - 1) / NWD;
    auto tile_ij = [&](int t, int& I, int& J) {
        I = 0;
        while ((I + 1) * (I + 2) / 2 <= t) ++I;
        J = t - I * (I + 1) / 2;
    };
    if (is_tree) {
        load_scalars(0);
        tree_scalars(0);
        __syncthreads();   // B1
        tree_struct(0);
        __syncthreads();   // B2
        const bool ok0 = tree_check(0);
        if (ok0) tree_g(0);
        __syncthreads();   // B3: Gram values of the first key head are in
        if (ok0) {
            t_kh = item_kh(0);
            tree_tail(0);
        }
        load_scalars(min(1, nit - 1));
        __syncthreads();   // B4
        // the next key head's K/Q go into the registers as soon as the
        // current ones have been used (Gram and staging)
        auto next_kq = [&](int j) {
            int q = max(j, 1);
            while (q < nit && !new_kq_at(q)) ++q;
            return q;
        };
        if (next_kq(1) < nit) hold_kq(next_kq(1));
        GDN_PHASE(6);
        GDN_PHASE_SNAP;
        for (int j = 0; j < nit; ++j) {
            refresh();
            const bool restage = restage_after(j);
            if (j + 1 < nit) {
                tree_scalars(j + 1);
                tree_item(j + 1);
            }
            load_scalars(min(j + 2, nit - 1));
            GDN_PHASE_ARRIVE(j);
            if (restage) {
                hold_kq(j + 1);   // held already unless a walk forced this
                __syncthreads();
                stage_kq();
                __syncthreads();
            } else {
                __syncthreads();
            }
            if (next_kq(j + 2) < nit) hold_kq(next_kq(j + 2));
            GDN_PHASE(14);
            GDN_PHASE_ITER(j);
        }
    } else {
        {
            constexpr int NDT = 64 * NWD;
            constexpr int KC0 = (NMAX * CH + NDT - 1) / NDT;
            const int bb = item_b(0), kh = item_kh(0);
            uint4 kv[KC0], qv[KC0];
#pragma unroll
            for (int q = 0; q < KC0; ++q) {
                const int e = min(tid + q * NDT, NMAX * CH - 1);
                const size_t gofs = ((static_cast<size_t>(bb) * N + min(e / CH, N - 1)) * Hk + kh) * DK + (e % CH) * 8;
                kv[q] = *reinterpret_cast<const uint4*>(kg + gofs);
                qv[q] = *reinterpret_cast<const uint4*>(qg + gofs);
            }
#pragma unroll
            for (int q = 0; q < KC0; ++q) {
                const int e = tid + q * NDT;
                if (e < NMAX * CH) put_chunk(e / CH, e % CH, kv[q], qv[q]);
            }
        }
        __syncthreads();   // B1
        f32x4 gk[GT0], gq[GT0];
#pragma unroll
        for (int u = 0; u < GT0; ++u) {
            int I, J;
            tile_ij(min(wave + NWD * u, NTILE0 - 1), I, J);
            gk[u] = gq[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 fb = frag(Ks, 16 * J + lc, ks);
                gk[u] = mfma(frag(Ks, 16 * I + lc, ks), fb, gk[u]);
                gq[u] = mfma(frag(Qs, 16 * I + lc, ks), fb, gq[u]);
            }
        }
        __syncthreads();   // B2: the structure is built
        if (misc[0] <= L::CAP) {
            const int NT = (N + 15) >> 4;
#pragma unroll
            for (int u = 0; u < GT0; ++u) {
                const int t = wave + NWD * u;
                int I, J;
                tile_ij(min(t, NTILE0 - 1), I, J);
                if (t < NTILE0 && I < NT && ((tmask[I] >> J) & 1u)) put_pairs(I, J, gk[u], gq[u]);
            }
        }
        __syncthreads();   // B3
        load_sv(0, 1);
        __syncthreads();   // B4
        GDN_PHASE(7);
        GDN_PHASE_SNAP;
        for (int j = 0; j < nit; ++j) {
            refresh();
            const bool restage = restage_after(j);
            dense_item(j);
            GDN_PHASE_ARRIVE(j);
            __syncthreads();
            if (restage) __syncthreads();
            GDN_PHASE(6);
            GDN_PHASE_ITER(j);
        }
    }
    // a timed-out role barrier means the protocol above is broken: report it
    // on the sequences this workgroup touched
    if (tid == 0 && misc[4]) {
        for (int bb = item_b(0); bb <= item_b(nit - 1); ++bb) atomicMax(a.tree_status + bb, static_cast<int>(GDN_ERR_HIP));
    }
    GDN_PHASE_END;
}

}  // namespace

#ifndef GDN_WS_DENSE_WAVES
#define GDN_WS_DENSE_WAVES(dv) ((dv) / 16)
#endif

hipError_t launch_verify_ws(const VerifyArgs& a, hipStream_t stream) {
    const int items = a.B * a.H_v;
    const int wgs = min(items, device_cus());
    const int per = (items + wgs - 1) / wgs;
    const dim3 grid((items + per - 1) / per);
    auto go = [&](auto kern, int dv) {
        hipLaunchKernelGGL(kern, grid, dim3(64 * (GDN_WS_DENSE_WAVES(dv) + 4)), 0, stream, a, per);
        return hipGetLastError();
    };
    // dense wavefronts: one per 16 value columns
    constexpr int W64 = GDN_WS_DENSE_WAVES(64), W128 = GDN_WS_DENSE_WAVES(128);
    if (a.N <= 64) {
        if (a.d_k == 64)
            return a.d_v == 64 ? go(verify_ws_kernel<64, 64, 64, W64>, 64) : go(verify_ws_kernel<64, 64, 128, W128>, 128);
        return a.d_v == 64 ? go(verify_ws_kernel<64, 128, 64, W64>, 64) : go(verify_ws_kernel<64, 128, 128, W128>, 128);
    }
    if (a.d_k == 64)
        return a.d_v == 64 ? go(verify_ws_kernel<128, 64, 64, W64>, 64) : go(verify_ws_kernel<128, 64, 128, W128>, 128);
    return a.d_v == 64 ? go(verify_ws_kernel<128, 128, 64, W64>, 64) : go(verify_ws_kernel<128, 128, 128, W128>, 128);
}

}  // namespace gdn
