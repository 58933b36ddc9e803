// gdn_split.hip -- tree verification in two launches for bf16 q/k/v and
// trees of 129 to 256 nodes on gfx950: a tree kernel that forms, for every
// (sequence, value head), the tree-shaped operator Z~ and gamma into the
// context's workspace, then a dense kernel that streams S0, V, K and Q of
// each (sequence, value head) through the MFMA contractions and writes o.
//
// What is computed (Trees from Marginals technical summary, Methodology,
// "3. Rollback-Free Tree Verification for GDN"): over the ancestor pairs of
// the topologically sorted tree,
//     X_is = beta_i D_is (k_i . k_s)  (s a strict ancestor of i),
//     Y_is = D_is (q_i . k_s)         (s an ancestor of i, or i),
// (D_is = exp(G_i - G_s), G the path sum of the log-gates, gamma = exp(G)),
// the masked triangular solve (I + X) U = diag(beta) (V - gamma o K S0^T)
// and the output O = gamma o Q S0^T + Y U.  The solve is folded into an
// N x N operator with the ancestor pattern of the tree, which does not
// depend on d_v:
//     Z~ = Y (I + X)^-1 diag(beta),  R' = V - gamma o (K S0^T),
//     O = gamma o (Q S0^T) + Z~ R'.
//
// Why two launches: at this size one item's tree side (structure, Gram of
// the ancestor pairs, the row solve) is a long chain of dependent
// phases, and an item's dense side needs most of a compute unit's LDS and
// registers, so the two cannot share a workgroup without running in turn.
// Here the tree kernel runs the chains of the whole batch side by side: one
// persistent workgroup per compute unit walks a run of (sequence, key head)
// items, builds a sequence's structure once for its run, computes the Gram
// once for the value heads of each key head, solves two value heads at a
// time, and loads the next item's rows while it solves; the dense kernel
// runs one item per workgroup, two workgroups per compute unit.
// Between them go the pair values (4 bytes per ancestor pair and value
// head) and gamma; K and Q are read by both.  (For trees of at most 128
// nodes the persistent single-launch kernel of gdn_verify_ws.hip, which
// overlaps one item's tree side with another's dense side, is faster.)
//
// Workspace (per context, written by the tree kernel, read by the dense
// kernel), with P = 24 N pairs per sequence at most (root paths of up to
// ZR = 24 nodes):
//   z     float [B][H_v][P]  Z~ values in pair order (below), times beta of
//                            the ancestor
//   gam   float [B][H_v][N]  gamma
//   zoff  uint16 [B][P]      where each pair's entry goes in the MFMA blocks
//                            of its output row tile (below)
//   off   int32 [B][N + 1]   first pair of each node; off[N] = pair count
//   deep  int32 [B]          1: a root path longer than ZR nodes (the
//                            dense kernel walks that sequence per node)
// Pair order: node by node; node i's pairs are its root path, root first
// (position d holds the ancestor at depth d + 1, the last one i itself).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"
#include "gdn_mfma.h"
#include "gdn_walk.h"

// Phase markers: no-ops here; a timing build defines them to record when
// each phase of a workgroup starts.
#ifndef GDN_SPLIT_PHASE
#define GDN_SPLIT_PHASE_DECL
#define GDN_SPLIT_PHASE(k)
#define GDN_SPLIT_PHASE_END(kind, id)
#endif

namespace gdn {

namespace {

__host__ __device__ constexpr int sp_align(int x, int a) { return (x + a - 1) / a * a; }
__host__ __device__ constexpr int sp_max(int x, int y) { return x > y ? x : y; }
__host__ __device__ constexpr int sp_zr(int n) { return n > 128 ? 24 : 16; }

// ---------------------------------------------------------------- tree kernel

template <int NMAX, int DK>
struct TreeLds {
    static constexpr int ZR = sp_zr(NMAX);
    static constexpr int CAP = NMAX * ZR;
    static constexpr int KROW = DK * 2 + 16;             // staged k row, padded against bank conflicts
    static constexpr int KS_BYTES = NMAX * KROW;
    static constexpr int KS = 0;                         // K rows
    // float[CAP + 4 + 32]: k_i . k_s; entry CAP takes the Gram tile entries
    // that are not pairs, entries KZERO .. KZERO + 31 stay zero (the row the
    // solve reads for path positions past a node's depth)
    static constexpr int KK = sp_align(KS_BYTES, 16);
    static constexpr int KZERO = CAP + 4;
    static constexpr int QK = KK + 4 * (CAP + 4 + 32);   // float[CAP + 4]: q_i . k_s
    static constexpr int PATH = QK + 4 * (CAP + 4);      // uint8[CAP]: ancestor of each pair
    static constexpr int NODE = sp_align(PATH + CAP, 16);
    static constexpr int PAR = NODE;                     // int[NMAX]
    static constexpr int DEP = PAR + 4 * NMAX;           // int[NMAX]: nodes on the root path
    static constexpr int NXT = DEP + 4 * NMAX;           // int[NMAX]: pointer jumping
    static constexpr int OFF = NXT + 4 * NMAX;           // int[NMAX + 16]
    static constexpr int GV = OFF + 4 * (NMAX + 16);     // float[2][NMAX]: g of two value heads
    static constexpr int BET = GV + 8 * NMAX;            // float[2][NMAX]: beta
    static constexpr int GG = BET + 8 * NMAX;            // float[2][NMAX]: G
    static constexpr int TMASK = GG + 8 * NMAX;          // uint32[NMAX / 16]: tile (I, J) holds pairs
    static constexpr int MISC = TMASK + 4 * (NMAX / 16); // int[16]
    // uint32[NMAX / 32][NMAX]: word w of node i's ancestor set (i itself
    // included), bit b for node 32 w + b; the words of consecutive nodes are
    // consecutive, so four rows of one word are one 16-byte read
    static constexpr int ANC = sp_align(MISC + 64, 16);
    static constexpr int TOTAL = ANC + 4 * NMAX * (NMAX / 32);
};

// A persistent grid: one workgroup per compute unit, 2 NMAX threads, walking
// a run of consecutive (sequence, key head) items.  Per item the Gram of the
// key head once, then the value heads of the key head two at a time, thread t
// taking node t mod NMAX of head slot t / NMAX.  Items of one sequence share
// its structure (depth, pair offsets, root paths, the tiles holding pairs),
// built for the first of them; the next item's parents, gates of its first
// two value heads and Q/K rows are loaded while the current item is solved.
template <int NMAX, int DK>
__global__ __launch_bounds__(2 * NMAX) void tree_kernel(VerifyArgs a, SplitWs w, int items_per_wg) {
    using L = TreeLds<NMAX, DK>;
    constexpr int NTH = 2 * NMAX;
    constexpr int NW = NTH / 64;
    constexpr int KS = DK / 32;
    constexpr int NTMAX = NMAX / 16;
    constexpr int ZR = L::ZR;
    constexpr int KCH = NMAX * DK / 8 / NTH;   // 16-byte pieces of K per thread
    static_assert(KCH * NTH == NMAX * DK / 8, "K staging split");
    constexpr int RU = NTMAX / NW;             // Gram row tiles per wavefront
    static_assert(RU == 2, "row tiles w and 2 NW - 1 - w");

    __shared__ __align__(16) unsigned char smem[L::TOTAL];
    GDN_SPLIT_PHASE_DECL

    const int N = a.N, Hk = a.H_k, Hv = a.H_v;
    const int R = Hv / Hk;
    const int n_items = a.B * Hk;
    // Workgroups go to the 8 XCDs in turn; numbering them so that each XCD
    // takes consecutive items keeps the key heads of a sequence on one XCD,
    // whose L2 then serves their shared rows of g, beta and the parents once
    const int wg = gridDim.x % 8 == 0 ? (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8 : blockIdx.x;
    const int it0 = wg * items_per_wg;
    const int it1 = min(it0 + items_per_wg, n_items);
    if (it0 >= it1) return;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    // The thread index is refreshed through an opaque copy once per item:
    // addresses derived from it are then recomputed per item rather than
    // hoisted out of the item loop and held in registers across it.
    int tid, lane, lc, lg, ni, hr;
    auto refresh = [&]() {
        int t = threadIdx.x;
        asm volatile("" : "+v"(t));
        tid = t;
        lane = t & 63;
        lc = lane & 15;
        lg = lane >> 4;
        ni = t % NMAX;
        hr = t / NMAX;
    };
    refresh();

    const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
    const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);

    unsigned char* Ks = smem + L::KS;
    float* kk = reinterpret_cast<float*>(smem + L::KK);
    float* qk = reinterpret_cast<float*>(smem + L::QK);
    uint8_t* pathc = smem + L::PATH;
    int* par = reinterpret_cast<int*>(smem + L::PAR);
    int* dep = reinterpret_cast<int*>(smem + L::DEP);
    int* nxt = reinterpret_cast<int*>(smem + L::NXT);
    int* off = reinterpret_cast<int*>(smem + L::OFF);
    float* gv = reinterpret_cast<float*>(smem + L::GV);
    float* bet = reinterpret_cast<float*>(smem + L::BET);
    float* Gs = reinterpret_cast<float*>(smem + L::GG);
    uint32_t* tmask = reinterpret_cast<uint32_t*>(smem + L::TMASK);
    int* misc = reinterpret_cast<int*>(smem + L::MISC);
    uint32_t* anc = reinterpret_cast<uint32_t*>(smem + L::ANC);

    // g and beta of value head kh R + r0 + hr at node ni
    auto load_gb = [&](int b, int kh, int r0, float& gi, float& bi) {
        const int r = r0 + hr;
        gi = 0.f;
        bi = 0.f;
        if (r < R && ni < N) {
            const size_t nh = (static_cast<size_t>(b) * N + ni) * Hv + kh * R + r;
            gi = a.g[nh];
            bi = a.beta[nh];
        }
    };
    auto store_gb = [&](float gi, float bi) {
        gv[hr * NMAX + ni] = gi;
        bet[hr * NMAX + ni] = bi;
    };
    auto row_tile = [&](int u) { return u == 0 ? wave : 2 * NW - 1 - wave; };

    // ---- (1) an item's loads, in flight until it starts: the parents and
    // the gates of its first two value heads (which the structure phases wait
    // for, so they are issued first), the Q rows of this wavefront's Gram row
    // tiles, and the K rows (written to LDS once the previous item's Gram is
    // done)
    int p_pf = -1;
    float g_pf = 0.f, b_pf = 0.f;
    bf16x8 qa[RU][KS];
    uint4 kv[KCH];
    auto prefetch = [&](int it) {
        const int b = it / Hk, kh = it % Hk;
        p_pf = tid < NMAX && tid < N ? a.parent[static_cast<size_t>(b) * N + tid] : -1;
        load_gb(b, kh, 0, g_pf, b_pf);
#pragma unroll
        for (int u = 0; u < RU; ++u)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qa[u][ks] = load_frag(qg + ((static_cast<size_t>(b) * N + min(16 * row_tile(u) + lc, N - 1)) * Hk + kh) * DK +
                                      8 * KS * lg + 8 * ks);
#pragma unroll
        for (int q = 0; q < KCH; ++q) {
            const int e = tid + q * NTH;
            const int row = min(e / (DK / 8), N - 1);
            kv[q] = *reinterpret_cast<const uint4*>(kg + ((static_cast<size_t>(b) * N + row) * Hk + kh) * DK + (e % (DK / 8)) * 8);
        }
    };
    prefetch(it0);
    if (tid >= 64 && tid < 64 + 32) kk[L::KZERO + tid - 64] = 0.f;

    int cur_b = -1, bad = 0, deep = 0;
    for (int it = it0; it < it1; ++it) {
        GDN_SPLIT_PHASE(0);
        refresh();
        const int b = it / Hk, kh = it % Hk;
        const bool new_b = b != cur_b;
        cur_b = b;
        store_gb(g_pf, b_pf);
        int bad_local = 0;
        if (new_b) {
            if (tid < NMAX) {
                const int i = tid;
                int p = p_pf;
                if (i < N && (p < -1 || p >= i)) {
                    bad_local = 1;
                    p = -1;
                }
                par[i] = p;
                nxt[i] = p;
                dep[i] = i < N ? 1 : 0;
            }
            if (tid < NTMAX) tmask[tid] = 0u;
        }
        {
            const int any_bad = __syncthreads_or(bad_local);
            if (new_b) bad = any_bad;
        }
        GDN_SPLIT_PHASE(1);

        // ---- (2) for a new sequence, the structure: depth by pointer
        // jumping (dep[i] counts the nodes from i up to nxt[i]), pair
        // offsets, root paths, the tiles holding pairs
        if (new_b) {
            for (int round = 0; round < 9; ++round) {
                int c2 = 0, n2 = -1;
                if (tid < NMAX) {
                    const int nx = nxt[tid];
                    c2 = dep[tid] + (nx >= 0 ? dep[nx] : 0);
                    n2 = nx >= 0 ? nxt[nx] : -1;
                }
                __syncthreads();
                if (tid < NMAX) {
                    dep[tid] = c2;
                    nxt[tid] = n2;
                }
                if (!__syncthreads_or(n2 >= 0)) break;
            }
            deep = __syncthreads_or(tid < N && dep[tid] > ZR);
        }
        GDN_SPLIT_PHASE(2);
        if (kh == 0 && tid == 0) {
            a.tree_status[b] = bad ? GDN_ERR_TREE : 0;
            w.deep[b] = deep ? 1 : 0;
        }
        if (deep) {
            // the dense kernel walks this sequence
            if (it + 1 < it1) prefetch(it + 1);
            continue;
        }
        if (new_b && wave == 0) {
            // exclusive scan of dep into off; off[N] = pair count
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
            if (lane == 63) {
                off[NMAX] = incl;
                misc[0] = incl;
            }
        }
        __syncthreads();
        const int total = misc[0];
#pragma unroll
        for (int q = 0; q < KCH; ++q) {
            const int e = tid + q * NTH;
            const int row = e / (DK / 8), cc = e % (DK / 8);
            const uint4 v = row < N ? kv[q] : make_uint4(0u, 0u, 0u, 0u);
            *reinterpret_cast<uint4*>(Ks + row * L::KROW + cc * 16) = v;
        }
        if (new_b && tid < NMAX) {
            // node i's root path, root first, at its pairs; its ancestor
            // words; the tiles that hold pairs; (key head 0) where each
            // pair's entry goes in the dense kernel's blocks: block s / 32
            // (2 KB: 1 KB hi, then 1 KB lo) of the row tile, lane group
            // (s / 4) mod 4, row i mod 16, slot 4 ((s / 16) mod 2) + s mod 4
            // of that lane's 8 bf16.  Key head 0 is always the first item of
            // its sequence in a run.
            const int i = tid;
            constexpr int AW = NMAX / 32;
            uint32_t am[AW];
#pragma unroll
            for (int q = 0; q < AW; ++q) am[q] = 0u;
            if (i < N) {
                uint16_t* zg = w.zoff + static_cast<size_t>(b) * w.P;
                int pos = off[i] + dep[i] - 1;
                uint32_t mask = 0u;
                for (int s = i; s >= 0; s = par[s]) {
                    pathc[pos] = static_cast<uint8_t>(s);
                    if (kh == 0) {
                        const int el = (((((s >> 2) & 3) << 4) | (i & 15)) << 3) + (((s >> 4) & 1) << 2) + (s & 3);
                        zg[pos] = static_cast<uint16_t>(2048 * (s >> 5) + 2 * el);
                    }
                    --pos;
                    mask |= 1u << (s >> 4);
#pragma unroll
                    for (int q = 0; q < AW; ++q) am[q] |= (s >> 5) == q ? 1u << (s & 31) : 0u;
                }
                atomicOr(&tmask[i >> 4], mask);
            }
#pragma unroll
            for (int q = 0; q < AW; ++q) anc[q * NMAX + i] = am[q];
        }
        __syncthreads();
        GDN_SPLIT_PHASE(3);
        if (kh == 0) {
            // the rest of the sequence's pair structure for the dense kernel
            int32_t* offg = w.off + static_cast<size_t>(b) * (N + 1);
            for (int i = tid; i <= N; i += NTH) offg[i] = i < N ? off[i] : total;
        }

        // ---- (3) Gram values of the ancestor pairs: MFMA over the lower
        // 16x16 tiles that hold pairs; wavefront w takes row tiles w and
        // 2 NW - 1 - w (their Q rows came with the item's loads)
        {
            const int NT = (N + 15) >> 4;
            auto k_frag = [&](int row, int ks) -> bf16x8 {
                return load_frag(Ks + row * L::KROW + 2 * (8 * KS * lg + 8 * ks));
            };
#pragma unroll
            for (int u = 0; u < RU; ++u) {
                const int I = row_tile(u);
                if (I >= NT) continue;
                const uint32_t tm = tmask[I];
                bf16x8 ka[KS];
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) ka[ks] = k_frag(16 * I + lc, ks);
                // this lane's rows i = 16 I + 4 lg + rr: first pair
                int oi[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) oi[rr] = off[16 * I + 4 * lg + rr];
                // tiles J <= I that hold pairs, in order; the K fragments of
                // tile J, the depth of its node s = 16 J + lc and the
                // ancestor words of the lane's four rows that hold s's bit
                // are read one tile ahead (none of these reads waits for
                // another)
                const uint32_t todo = tm & ((2u << I) - 1u);
                struct Ahead {
                    bf16x8 kb[KS];
                    int ds;
                    uint4 am;
                };
                auto read_ahead = [&](int J) __attribute__((always_inline)) {
                    Ahead r;
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) r.kb[ks] = k_frag(16 * J + lc, ks);
                    r.ds = dep[16 * J + lc];
                    r.am = *reinterpret_cast<const uint4*>(anc + (J >> 1) * NMAX + 16 * I + 4 * lg);
                    return r;
                };
                uint32_t left = todo;
                if (!left) continue;
                int J = __builtin_ctz(left);
                left &= left - 1;
                Ahead cur = read_ahead(J);
                for (;;) {
                    f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int ks = 0; ks < KS; ++ks) {
                        akk = mfma(ka[ks], cur.kb[ks], akk);
                        aqk = mfma(qa[u][ks], cur.kb[ks], aqk);
                    }
                    const int Jn = left ? __builtin_ctz(left) : -1;
                    left &= left - 1;
                    Ahead nx;
                    if (Jn >= 0) nx = read_ahead(Jn);
                    // lane: rows i = 16 I + 4 lg + rr, column node s = 16 J +
                    // lc; when s is an ancestor of i (or i), the pair sits at
                    // position dep[s] - 1 of i's root path; every other entry
                    // goes to the spare slot CAP (no branches)
                    const int sb = (16 * J + lc) & 31;
                    const uint32_t amw[4] = {cur.am.x, cur.am.y, cur.am.z, cur.am.w};
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const int pp = (amw[rr] >> sb) & 1u ? oi[rr] + cur.ds - 1 : L::CAP;
                        kk[pp] = akk[rr];
                        qk[pp] = aqk[rr];
                    }
                    if (Jn < 0) break;
                    J = Jn;
                    cur = nx;
                }
            }
        }
        // the next item's loads, in flight through the solve below
        if (it + 1 < it1) prefetch(it + 1);
        __syncthreads();
        GDN_SPLIT_PHASE(4);

        // ---- (4) per pair of value heads: G, gamma; rows of Z~.  Along node
        // i's root path t_0 (root) .. t_{m-1} = i the row w of Y (I + X)^-1
        // solves w_b = Y_{i,t_b} - sum_{a > b} w_a X_{t_a,t_b}.  As
        // D_{i,t_a} D_{t_a,t_b} = D_{i,t_b}, w_b = D_{i,t_b} y_b with
        //     y_b = q_i . k_{t_b} - sum_{a > b} (beta_{t_a} y_a) (k_{t_a} . k_{t_b}),
        // a sweep over the Gram values and beta only; Z~_{i,t_b} = beta_{t_b} w_b.
        for (int r0 = 0; r0 < R; r0 += 2) {
            if (r0 > 0) {
                __syncthreads();   // the previous pair's reads of gv, bet and Gs are done
                float gi, bi;
                load_gb(b, kh, r0, gi, bi);
                store_gb(gi, bi);
                __syncthreads();
            }
            const int r = r0 + hr;
            const bool live = r < R && ni < N;
            const int h = kh * R + r;
            const int o = off[ni], m = live ? dep[ni] : 0;
            const float* gvh = gv + hr * NMAX;
            const float* bh = bet + hr * NMAX;
            float* Gh = Gs + hr * NMAX;
            auto path_at = [&](int d) {
                return min(static_cast<int>(pathc[min(o + min(d, max(m - 1, 0)), L::CAP - 1)]), NMAX - 1);
            };
            float G = 0.f;
#pragma unroll
            for (int d = 0; d < ZR; ++d) G += d < m ? gvh[path_at(d)] : 0.f;
            Gh[ni] = G;
            if (live) w.gam[(static_cast<size_t>(b) * Hv + h) * N + ni] = __expf(G);
            __syncthreads();
            GDN_SPLIT_PHASE(5);
            GDN_SPLIT_PHASE(6);
            if (live) {
                // swept from the node end: once y_a is final, y_b -=
                // beta_{t_a} y_a (k_{t_a} . k_{t_b}) for b < a, the Gram value
                // at position b of t_a's root path; positions past the path
                // read the zero row
                int oa[ZR];
                float y[ZR], bt[ZR];
#pragma unroll
                for (int d = 0; d < ZR; ++d) {
                    const int t = path_at(d);
                    oa[d] = d < m ? off[t] : L::KZERO;
                    bt[d] = bh[t];
                    y[d] = d < m ? qk[o + d] : 0.f;
                }
                float xr[ZR - 1];
#pragma unroll
                for (int e = 0; e < ZR - 1; ++e) xr[e] = kk[oa[ZR - 1] + e];
#pragma unroll
                for (int aa = ZR - 1; aa >= 1; --aa) {
                    float xn[ZR - 1];
#pragma unroll
                    for (int e = 0; e + 1 < aa; ++e) xn[e] = kk[oa[aa - 1] + e];
                    const float ya = y[aa] * bt[aa];
#pragma unroll
                    for (int e = 0; e < aa; ++e) y[e] -= ya * xr[e];
#pragma unroll
                    for (int e = 0; e + 1 < aa; ++e) xr[e] = xn[e];
                    __builtin_amdgcn_sched_barrier(0);
                }
                float* zg = w.z + (static_cast<size_t>(b) * Hv + h) * w.P + o;
#pragma unroll
                for (int d = 0; d < ZR; ++d)
                    if (d < m) zg[d] = y[d] * bt[d] * __expf(G - Gh[path_at(d)]);
            }
        }
        // every read of this item's LDS arrays is done before the next item
        // writes them
        __syncthreads();
        GDN_SPLIT_PHASE(7);
    }
    GDN_SPLIT_PHASE_END(0, blockIdx.x);
}

// --------------------------------------------------------------- dense kernel

template <int NMAX, int DK, int DV>
struct DenseLds {
    static_assert(NMAX == 256, "trees of 129 to 256 nodes");
    static constexpr int NTMAX = NMAX / 16;
    static constexpr int CAP = NMAX * sp_zr(NMAX);
    // K for K S0^T, in the k-slot order with chunks swizzled by row; once R'
    // is formed, the same bytes hold three stages of one output row tile's
    // Z~ blocks (bf16 hi + lo) and Q rows, tile I in stage I mod 3
    static constexpr int KQ = 0;
    static constexpr int ZT_BYTES = 2048 * (NTMAX / 2);          // NTMAX / 2 blocks of 2 KB
    static constexpr int ZT = 0;                                  // [3][ZT_BYTES]
    static constexpr int QT = ZT + 3 * ZT_BYTES;                  // [3] bf16[16][DK]
    static constexpr int KQ_BYTES = sp_max(NMAX * DK * 2, QT + 3 * 32 * DK);
    static constexpr int ZOFF = KQ + KQ_BYTES;                    // uint16[CAP]: each pair's place in its tile's blocks
    static constexpr int GAM = ZOFF + 2 * CAP;                    // float[NMAX]
    static constexpr int OFF = GAM + 4 * NMAX;                    // int[NMAX + 16]: first pair of each node
    static constexpr int MISC = OFF + 4 * (NMAX + 16);
    // the per-node walk of a deep tree (S0 read from global memory): u
    // [NMAX][64], G, k and q rows, parents
    static constexpr int FB_G = NMAX * 64 * 4;
    static constexpr int FB_KQ = FB_G + 4 * NMAX;
    static constexpr int FB_PAR = FB_KQ + 8 * DK;
    static constexpr int FB_END = FB_PAR + 4 * NMAX;
    static constexpr int TOTAL = sp_max(MISC + 64, FB_END);
    static_assert(TOTAL <= 80 * 1024, "two workgroups per compute unit");
};

// One (sequence, value head) item per workgroup; each wavefront owns CT
// tiles of 16 value columns (two at d_v = 128: every Z~ block and Q row read
// from LDS then serves two column tiles, and a wavefront writes whole
// 128-byte pieces of o rows).
template <int NMAX, int DK, int DV, int CT>
__global__ __launch_bounds__(4 * DV / CT, 2) void dense_kernel(VerifyArgs a, SplitWs w) {
    using L = DenseLds<NMAX, DK, DV>;
    constexpr int NW = DV / (16 * CT);
    constexpr int NTH = 64 * NW;
    constexpr int KS = DK / 32;
    constexpr int CH = DK / 8;             // 16-byte chunks per K/Q row
    constexpr int NTMAX = NMAX / 16;
    constexpr int NKMAX = NMAX / 32;
    static_assert(NW * 16 * CT == DV, "whole column tiles per wavefront");

    __shared__ __align__(16) unsigned char smem[L::TOTAL];
    GDN_SPLIT_PHASE_DECL
    GDN_SPLIT_PHASE(0);

    const int N = a.N, Hk = a.H_k, Hv = a.H_v;
    const int R = Hv / Hk;
    const int n_items = a.B * Hv;
    // Workgroups go to the 8 XCDs in turn; numbering the items so that each
    // XCD takes a contiguous run keeps the value heads of one key head (which
    // read the same K and Q) on one L2, dispatched close together
    const int g = gridDim.x;
    const int item = (g % 8 == 0 && g == n_items) ? (blockIdx.x % 8) * (g / 8) + blockIdx.x / 8 : blockIdx.x;
    if (item >= n_items) return;
    const int b = item / Hv, h = item % Hv, kh = h / R;
    const int tid = threadIdx.x;
    const int lane = tid & 63, lc = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

    const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
    const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
    const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);
    unsigned char* KQb = smem + L::KQ;
    float* gam = reinterpret_cast<float*>(smem + L::GAM);
    int* offs = reinterpret_cast<int*>(smem + L::OFF);

    if (w.deep[b]) {
        // a root path longer than the tree kernel solves: the per-node walk,
        // by wavefront 0, one 64-column slice at a time
        if (wave == 0) {
            int* par_s = reinterpret_cast<int*>(smem + L::FB_PAR);
            float* G_s = reinterpret_cast<float*>(smem + L::FB_G);
            for (int i = lane; i < N; i += 64) {
                const int pp = a.parent[static_cast<size_t>(b) * N + i];
                par_s[i] = (pp < -1 || pp >= i) ? -1 : pp;
            }
            WaveSync::sync();
            float* u_s = reinterpret_cast<float*>(smem);
            float* ki = reinterpret_cast<float*>(smem + L::FB_KQ);
            for (int c0 = 0; c0 < DV; c0 += 64)
                walk_verify_slice_lds<uint16_t, DK, WaveSync>(a, b, h, c0, par_s, u_s, G_s, ki, ki + DK, nullptr);
        }
        return;
    }

    // ---- (1) loads: S0 rows and V of this wavefront's value columns, the
    // sequence's pair structure, gamma, K into LDS.  Column tile st of the
    // wavefront covers columns col0 + 16 st ..; s0r[st][2 ks + hh]: d_k
    // columns 32 ks + 16 hh + 4 lg .. + 3 of row col0 + 16 st + lc; vr[st][S]:
    // value columns col0 + 16 st + 4 lg .. + 3 of node 16 S + lc
    const int col0 = 16 * CT * wave;
    float4 s0r[CT][2 * KS];
#pragma unroll
    for (int st = 0; st < CT; ++st) {
        const float4* src =
            reinterpret_cast<const float4*>(a.S0 + ((static_cast<size_t>(b) * Hv + h) * DV + col0 + 16 * st + lc) * DK + 4 * lg);
#pragma unroll
        for (int q = 0; q < 2 * KS; ++q) s0r[st][q] = src[4 * q];
    }
    uint2 vr[CT][NTMAX];
    {
        const uint16_t* vsrc = vg + static_cast<size_t>(b) * N * Hv * DV + static_cast<size_t>(h) * DV + col0 + 4 * lg;
#pragma unroll
        for (int S = 0; S < NTMAX; ++S)
#pragma unroll
            for (int st = 0; st < CT; ++st)
                vr[st][S] = *reinterpret_cast<const uint2*>(vsrc + static_cast<size_t>(min(16 * S + lc, N - 1)) * Hv * DV + 16 * st);
    }
    const int total = w.off[static_cast<size_t>(b) * (N + 1) + N];
    const float* zsrc = w.z + (static_cast<size_t>(b) * Hv + h) * w.P;
    {
        // each pair's place in its tile's blocks, as 4-byte words (the pair
        // capacity is a multiple of 2), and the first pair of every node
        const uint32_t* zs = reinterpret_cast<const uint32_t*>(w.zoff + static_cast<size_t>(b) * w.P);
        const int words = (total + 1) >> 1;
        for (int e = tid; e < words; e += NTH) reinterpret_cast<uint32_t*>(smem + L::ZOFF)[e] = zs[e];
        for (int i = tid; i <= NMAX; i += NTH) offs[i] = w.off[static_cast<size_t>(b) * (N + 1) + min(i, N)];
    }
    for (int i = tid; i < NMAX; i += NTH) gam[i] = i < N ? w.gam[(static_cast<size_t>(b) * Hv + h) * N + i] : 0.f;

    // Natural 16-byte chunk c of K or Q row `row` into a buffer in the
    // k-slot order the fragments read: element 32 ks + 16 hh + 4 g + r at
    // position 32 ks + 8 g + 4 hh + r; chunk 4 ks + g stored at chunk
    // position (4 ks + g) ^ (row mod CH); `keep` zeroes rows past N
    auto put_chunk = [&](unsigned char* base, int row, int c, uint4 v, uint32_t keep) {
        const int sw = row & (CH - 1);
        const int ks = c >> 2, m = c & 3, hh = m >> 1, g0 = (m & 1) << 1;
        const int rbase = row * (DK * 2) + 8 * hh;
        *reinterpret_cast<uint2*>(base + rbase + (((4 * ks + g0) ^ sw) << 4)) = make_uint2(v.x & keep, v.y & keep);
        *reinterpret_cast<uint2*>(base + rbase + (((4 * ks + g0 + 1) ^ sw) << 4)) = make_uint2(v.z & keep, v.w & keep);
    };
    {
        // K in passes of at most 4 chunks per thread, which bounds the
        // registers the staging holds beside the S0 and V loads in flight
        constexpr int KCH = NMAX * CH / NTH;
        static_assert(KCH * NTH == NMAX * CH, "K staging split");
        constexpr int KP = KCH < 4 ? KCH : 4;
        static_assert(KCH % KP == 0, "staging passes");
#pragma unroll
        for (int q0 = 0; q0 < KCH; q0 += KP) {
            uint4 v[KP];
#pragma unroll
            for (int q = 0; q < KP; ++q) {
                const int e = tid + (q0 + q) * NTH;
                v[q] = *reinterpret_cast<const uint4*>(kg + ((static_cast<size_t>(b) * N + min(e / CH, N - 1)) * Hk + kh) * DK + (e % CH) * 8);
            }
#pragma unroll
            for (int q = 0; q < KP; ++q) {
                const int e = tid + (q0 + q) * NTH;
                put_chunk(KQb, e / CH, e % CH, v[q], e / CH < N ? 0xFFFFFFFFu : 0u);
            }
        }
    }

    // ---- (2) R' = V - gamma o (K S0^T) on MFMA, S0 as bf16 hi + lo; R' kept
    // as fragments (k = node) of the Z~ R' product
    const int NT = (N + 15) >> 4;
    s16x4 eye;   // identity for the V transposes: lane (n, g) holds B[4 g + j][n]
#pragma unroll
    for (int q = 0; q < 4; ++q) eye[q] = 4 * lg + q == lc ? static_cast<short>(0x3F80) : short(0);
    bf16x8 s0h[CT][KS], s0l[CT][KS];
#pragma unroll
    for (int st = 0; st < CT; ++st)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const float4 x0 = s0r[st][2 * ks], x1 = s0r[st][2 * ks + 1];
            const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            split8(x, s0h[st][ks], s0l[st][ks]);
        }
    __syncthreads();
    GDN_SPLIT_PHASE(1);
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
                    const int row = 16 * S + lc;
                    const bf16x8 fa = load_frag(KQb + row * (DK * 2) + (((4 * ks + lg) ^ (row & (CH - 1))) << 4));
#pragma unroll
                    for (int st = 0; st < CT; ++st) {
                        ah[st] = mfma(fa, s0h[st][ks], ah[st]);
                        al[st] = mfma(fa, s0l[st][ks], al[st]);
                    }
                }
                const f32x4 gq = *reinterpret_cast<const f32x4*>(gam + 16 * S + 4 * lg);
#pragma unroll
                for (int st = 0; st < CT; ++st) {
                    const f32x4 vt = mfma16(__builtin_bit_cast(s16x4, vr[st][S]), eye, f32x4{0.f, 0.f, 0.f, 0.f});
                    const f32x4 pk = ah[st] + al[st];
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        const float vv = 16 * S + 4 * lg + rr < N ? vt[rr] : 0.f;
                        rt[st][4 * half + rr] = vv - gq[rr] * pk[rr];
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
    GDN_SPLIT_PHASE(2);

    // ---- (3) O tiles, O^T = gamma o (S0 Q^T) + R'^T Z~^T, each with its Q
    // rows and its blocks of Z~ staged in LDS by the workgroup, three stages
    // deep so that one barrier per tile orders everything: in the step of
    // tile I the workgroup fills stage I + 1 (zeroed one step earlier) with
    // that tile's pairs (contiguous in pair order) and Q rows, contracts tile
    // I, and zeroes stage I + 2 (last read by tile I - 1).  The pair values
    // and Q rows come from global memory one step ahead of their stage.
    // Block kap of a stage holds nodes 32 kap..; node t of row i sits in lane
    // group ((t >> 2) & 3), slot 4 ((t >> 4) & 1) + (t & 3).
    auto zt = [&](int I) { return smem + L::ZT + L::ZT_BYTES * (I % 3); };
    auto qt = [&](int I) { return smem + L::QT + 32 * DK * (I % 3); };
    static_assert(16 * CH <= NTH, "one Q piece per thread");
    constexpr int TP = (16 * sp_zr(NMAX) + NTH - 1) / NTH;   // pairs of a tile per thread
    // uniform bases with 32-bit lane offsets: no per-lane 64-bit addresses
    // held across the loop
    const uint16_t* qb = qg + (static_cast<size_t>(b) * N * Hk + kh) * DK;
    float* ob = a.o + (static_cast<size_t>(b) * N * Hv + h) * DV;
    auto load_q = [&](int I, int t) {
        const uint32_t row = min(16 * I + t / CH, N - 1);
        return *reinterpret_cast<const uint4*>(qb + row * static_cast<uint32_t>(Hk * DK) + 8u * (t % CH));
    };
    // the pairs of tile I that thread t scatters, read a tile ahead: each
    // one's place in the tile's blocks (-1: none) and its value.  (The pair
    // range comes from LDS: a global load waited on here would also wait
    // for the o stores in flight.)
    const uint16_t* zoffs = reinterpret_cast<const uint16_t*>(smem + L::ZOFF);
    auto load_z = [&](int I, int t, int (&p)[TP], float (&zz)[TP]) {
        const int p0 = I < NT ? offs[16 * I] : total;
        const int p1 = I < NT ? offs[min(16 * I + 16, N)] : total;
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            const bool has = p0 + t + u * NTH < p1;
            const int e = has ? p0 + t + u * NTH : 0;
            zz[u] = zsrc[static_cast<uint32_t>(e)];
            p[u] = has ? static_cast<int>(zoffs[e]) : -1;
        }
    };
    auto fill = [&](int I, int t, const uint4& qv, const int (&p)[TP], const float (&zz)[TP]) {
        unsigned char* Zt = zt(I);
        if (t < 16 * CH) put_chunk(qt(I), t / CH, t % CH, qv, 16 * I + t / CH < N ? 0xFFFFFFFFu : 0u);
#pragma unroll
        for (int u = 0; u < TP; ++u) {
            if (p[u] >= 0) {
                const __bf16 zh = static_cast<__bf16>(zz[u]);
                const __bf16 zl = static_cast<__bf16>(zz[u] - static_cast<float>(zh));
                *reinterpret_cast<__bf16*>(Zt + p[u]) = zh;
                *reinterpret_cast<__bf16*>(Zt + p[u] + 1024) = zl;
            }
        }
    };
    auto zero = [&](int I) {
        const int nb = I / 2 + 1;
        for (int e = tid; e < nb * 128; e += NTH) reinterpret_cast<uint4*>(zt(I))[e] = make_uint4(0u, 0u, 0u, 0u);
    };
    // o is written once: plain stores (the 64-byte pieces of one 128-byte
    // row piece meet in L2)
    auto store_o = [&](int I, int ln, const f32x4 (&v)[CT]) {
        const int i = 16 * I + (ln & 15);
        if (i < N) {
#pragma unroll
            for (int st = 0; st < CT; ++st)
                *reinterpret_cast<f32x4*>(ob + (static_cast<uint32_t>(i) * static_cast<uint32_t>(Hv * DV) +
                                                static_cast<uint32_t>(col0 + 16 * st + 4 * (ln >> 4)))) = v[st];
        }
    };

    __syncthreads();   // K is no longer read
    int pn[TP];
    float zv[TP];
    uint4 qv = load_q(0, tid);
    load_z(0, tid, pn, zv);
    zero(0);
    if (NT > 1) zero(1);
    __syncthreads();
    fill(0, tid, qv, pn, zv);
    qv = load_q(min(1, NT - 1), tid);
    load_z(1, tid, pn, zv);
    GDN_SPLIT_PHASE(3);
    // The o stores of tile I - 1 are issued in the step of tile I, after its
    // wait for the prefetched rows: loads and stores share one wait counter,
    // so a wait for a load also waits for stores issued before it, and this
    // keeps those stores a whole tile old.
    f32x4 prev[CT];
#pragma unroll
    for (int st = 0; st < CT; ++st) prev[st] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int I = 0; I < NT; ++I) {
        // lane indices through an opaque copy: offsets derived from them are
        // formed per tile instead of held in registers
        int t = tid;
        asm volatile("" : "+v"(t));
        const int ln = t & 63, c16 = ln & 15;
        __syncthreads();
        if (I + 1 < NT) fill(I + 1, t, qv, pn, zv);
        if (I > 0) store_o(I - 1, ln, prev);
        if (I + 1 < NT) {
            qv = load_q(min(I + 2, NT - 1), t);
            load_z(I + 2, t, pn, zv);
        }
        f32x4 acc[CT];
#pragma unroll
        for (int st = 0; st < CT; ++st) acc[st] = f32x4{0.f, 0.f, 0.f, 0.f};
        const unsigned char* Qt = qt(I);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 fb = load_frag(Qt + c16 * (DK * 2) + (((4 * ks + (ln >> 4)) ^ (c16 & (CH - 1))) << 4));
#pragma unroll
            for (int st = 0; st < CT; ++st) {
                acc[st] = mfma(s0h[st][ks], fb, acc[st]);
                acc[st] = mfma(s0l[st][ks], fb, acc[st]);
            }
        }
        const float gi = gam[16 * I + c16];
#pragma unroll
        for (int st = 0; st < CT; ++st) acc[st] *= gi;
        const unsigned char* blk = zt(I) + 16 * ln;
        const int nb = I / 2 + 1;
#pragma unroll
        for (int kap = 0; kap < NKMAX; ++kap) {
            if (kap < nb) {
                const bf16x8 zh = load_frag(blk + 2048 * kap);
                const bf16x8 zl = load_frag(blk + 2048 * kap + 1024);
#pragma unroll
                for (int st = 0; st < CT; ++st) {
                    acc[st] = mfma(rh[st][kap], zh, acc[st]);
                    acc[st] = mfma(rl[st][kap], zh, acc[st]);
                    acc[st] = mfma(rh[st][kap], zl, acc[st]);
                }
            }
        }
#pragma unroll
        for (int st = 0; st < CT; ++st) prev[st] = acc[st];
        if (I + 2 < NT) zero(I + 2);
    }
    store_o(NT - 1, lane, prev);
    GDN_SPLIT_PHASE(4);
    GDN_SPLIT_PHASE_END(1, item);
}

template <int NMAX, int DK, int DV>
hipError_t launch_split_t(const VerifyArgs& a, const SplitWs& w, hipStream_t stream) {
    // one tree workgroup per compute unit, each taking a run of
    // (sequence, key head) items
    const int items = a.B * a.H_k;
    const int wgs = min(items, device_cus());
    const int per = (items + wgs - 1) / wgs;
    hipLaunchKernelGGL((tree_kernel<NMAX, DK>), dim3((items + per - 1) / per), dim3(2 * NMAX), 0, stream, a, w, per);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // two column tiles per wavefront at d_v = 128 (4 wavefronts), one at 64
    constexpr int CT = DV == 128 ? 2 : 1;
    hipLaunchKernelGGL((dense_kernel<NMAX, DK, DV, CT>), dim3(static_cast<unsigned>(a.B) * a.H_v), dim3(4 * DV / CT), 0,
                       stream, a, w);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_verify_split(const VerifyArgs& a, hipStream_t stream) {
    if (!a.split_ws || a.N <= 128 || a.N > 256) return hipErrorInvalidValue;
    const SplitWs w = split_ws_at(a.split_ws, a.B, a.N, a.H_v);
    if (a.d_k == 128)
        return a.d_v == 128 ? launch_split_t<256, 128, 128>(a, w, stream) : launch_split_t<256, 128, 64>(a, w, stream);
    return a.d_v == 128 ? launch_split_t<256, 64, 128>(a, w, stream) : launch_split_t<256, 64, 64>(a, w, stream);
}

}  // namespace gdn
