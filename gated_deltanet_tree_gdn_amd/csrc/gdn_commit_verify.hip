// gdn_commit_verify.hip -- the delayed commit fused into the next tree's
// verification (gdn_commit_verify) for bf16 q/k/v and trees of at most 128
// nodes on gfx950: one (sequence, value head) item per workgroup, two
// workgroups resident per compute unit.
//
// What is computed (Trees from Marginals technical summary, Methodology,
// "3. Rollback-Free Tree Verification for GDN"): over the ancestor pairs of
// the topologically sorted tree,
//     X_is = beta_i D_is (k_i . k_s)  (s a strict ancestor of i),
//     Y_is = D_is (q_i . k_s)         (s an ancestor of i, or i),
// (D_is = exp(G_i - G_s), G the path sum of the log-gates, gamma = exp(G))
// and with the masked triangular solve folded into the tree-shaped operator
//     Z~ = Y (I + X)^-1 diag(beta),  R' = V - gamma o (K S0^T),
//     O = gamma o (Q S0^T) + Z~ R'.
// Row i of Z~ is found by back-substitution along the root-to-i path.
//
// One item per workgroup, two independent workgroups per compute unit, each
// taking one item through its phases in order: the loads of one can overlap
// the MFMA work and stores of the other without any hand-over protocol, and
// the LDS of one workgroup (at most 80 KB) leaves room for the commit's
// chunk, which the persistent verify kernel's does not.  The layout:
//   - one 32 KB buffer holds K (for the Gram and K S0^T), then Q (for
//     Q S0^T), in the MFMA k-slot order with chunks XOR-swizzled by row;
//   - one 40 KB area holds the tree arrays (pair lists of k.k and q.k,
//     root paths, ancestor bits, per-node scalars) while the tree is solved,
//     then the Z~ fragments (bf16 hi + lo, lower 16x32 blocks).
// Rows of Z~ stay in registers between the two uses of the area.
//
// Phases per item: (1) parents, gates, K into LDS; (2) depth, root paths,
// G and gamma, ancestor bits, the mask of 16x16 tiles holding pairs; (3) the
// Gram values of the pairs on MFMA (wavefront w takes row tile w, Q rows from
// global memory in the k-slot order); (4) each node's path into registers;
// (5) the rows of Z~ from the Gram values, beta and the gates; (6) S0 and V
// loads, Z~ into fragments; (7) R' = V - gamma o
// (K S0^T) on MFMA with S0 as bf16 hi + lo; (8) Q into the buffer; (9) per
// 16-node tile, gamma o (S0 Q^T) + R'^T Z~^T, stored as 16-byte pieces of o
// rows (the two 16-column halves of each 128-byte piece belong to the two
// wavefronts of one SIMD).
//
// Trees with a root path longer than 16 nodes, or more ancestor pairs than
// the area holds, are verified by the per-node walk of gdn_walk.h.
//
// The commit: the delayed state commitment of the previous tree
// (same page, section 3: the state is committed once the accepted branch is
// known, at the next decoding step) runs inside the next tree's verify, so
// the committed state is formed in registers, written once, and used by
// the verify without being read back.  Along the previous tree's root path
// to its accepted node, taken in chunks of at most 16 nodes (root first,
// chunk-relative log-gate sums G, gamma = exp(G), D_ts = exp(G_t - G_s)):
//     X_ts = beta_t D_ts (k_t . k_s)  (s < t),
//     T' = diag(D_{n-1, .}) (I + X)^-1 diag(beta)   (n nodes in the chunk),
//     S <- gamma_{n-1} S + K^T T' (V - gamma o (K S^T)),
// which is the GDN delta rule applied node by node along the chunk.  One
// wavefront that holds no tree node walks the accepted path, loads the
// chunk's K rows, g and beta once its Gram tiles are done, and forms X and T'
// (16 lanes, one column each, by forward substitution) in the path phase;
// after the Z~ scatter every wavefront applies the chunk to its own 16 state
// rows on MFMA (K S^T with S as bf16 hi + lo, T' and the
// right-hand side as hi + lo, K^T from K by transposing MFMAs against the
// identity).

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"
#include "gdn_mfma.h"
#include "gdn_walk.h"

// Phase markers: no-ops here; a timing build defines them to record the
// time at which each phase of an item starts.
#ifndef GDN_ITEM_PHASE
#define GDN_ITEM_PHASE_DECL
#define GDN_ITEM_PHASE(k)
#define GDN_ITEM_PHASE_END
#endif

namespace gdn {
namespace {

__host__ __device__ constexpr int vi_zblocks(int I) {
    return (I & 1) ? ((I + 1) / 2) * ((I + 1) / 2) : (I / 2) * (I / 2 + 1);
}
__host__ __device__ constexpr int vi_align(int x, int a) { return (x + a - 1) / a * a; }
__host__ __device__ constexpr int vi_max(int x, int y) { return x > y ? x : y; }

template <int NMAX, int DK, int DV>
struct ItemLds {
    static constexpr int NTMAX = NMAX / 16;
    static constexpr int AW = NMAX / 32;
    static constexpr int ZR = 16;                      // root paths of up to 16 nodes
    // node i's path sits in slots i ZR + d, d its distance from i (d = 0: i)
    static constexpr int CAP = NMAX * ZR;
    static constexpr int KQ = 0;                       // K, then Q
    static constexpr int KQ_BYTES = NMAX * DK * 2;
    static constexpr int AREA = KQ_BYTES;
    static constexpr int ZD_BYTES = 2048 * vi_zblocks(NTMAX);
    // tree phase, inside the area
    static constexpr int KK = AREA;                    // float[CAP + 4]: k_i . k_s (entry CAP: sink)
    static constexpr int QK = KK + 4 * (CAP + 4);      // float[CAP + 4]: q_i . k_s
    static constexpr int PATH = QK + 4 * (CAP + 4);    // uint8[CAP]: the node at distance d from i
    static constexpr int NODE = vi_align(PATH + CAP, 16);
    static constexpr int PAR = NODE;                   // int[NMAX]
    static constexpr int DEP = PAR + 4 * NMAX;
    static constexpr int GV = DEP + 4 * NMAX;          // float[NMAX]: g
    static constexpr int ANC = GV + 4 * NMAX;          // uint32[NMAX][AW]
    static constexpr int TMASK = ANC + 4 * AW * NMAX;  // uint32[NTMAX]
    static constexpr int TREE_END = TMASK + 4 * NTMAX;
    static constexpr int AREA_BYTES = vi_align(vi_max(ZD_BYTES, TREE_END - AREA), 16);
    // the per-node walk for deep trees: u [NMAX][64], S0 slice [DK][64],
    // G, k and q rows, parents, all from offset 0
    static constexpr int FB_S0 = NMAX * 64 * 4;
    static constexpr int FB_G = FB_S0 + DK * 64 * 4;
    static constexpr int FB_KQ = FB_G + 4 * NMAX;
    static constexpr int FB_PAR = FB_KQ + 8 * DK;
    static constexpr int FB_END = FB_PAR + 4 * NMAX;
    static constexpr int GAM = vi_align(vi_max(AREA + AREA_BYTES, FB_END), 16);  // float[NMAX]: gamma
    static constexpr int BET = GAM + 4 * NMAX;         // float[NMAX]: beta (kept past the tree phase)
    static constexpr int GG = BET + 4 * NMAX;          // float[NMAX]: G (kept past the tree phase)
    static constexpr int MISC = GG + 4 * NMAX;         // int[16]
    // fused commit: one chunk of the previous tree's accepted path
    static constexpr int CK = MISC + 64;               // bf16[16][DK]: K rows (k-slot order, swizzled)
    static constexpr int CX = CK + 32 * DK;            // float[16][16]: X
    static constexpr int CT = CX + 1024;               // bf16[16][16] T' hi, then lo
    static constexpr int CG = CT + 1024;               // float[16]: G
    static constexpr int CB = CG + 64;                 // float[16]: beta
    static constexpr int CPAR = CB + 64;               // int8[NMAX]: parents of the previous tree
    static constexpr int CPATH = CPAR + NMAX;          // uint8[NMAX]: accepted .. root
    static constexpr int CMISC = CPATH + NMAX;         // int[4]: 0 path length, 1 accepted node
    static constexpr int TOTAL = CMISC + 16;
    static_assert(TOTAL <= 80 * 1024, "two workgroups per compute unit");
    static_assert(NMAX <= 128, "parents of the previous tree as int8");
    // misc[]: 1 a path longer than ZR (1), 2 an invalid parent (1)
};

template <int NMAX, int DK, int DV>
__global__ __launch_bounds__(4 * DV, 4 * DV / 128) void commit_verify_kernel(VerifyArgs a, CommitPrev c) {
    using L = ItemLds<NMAX, DK, DV>;
    constexpr int NW = DV / 16;          // wavefronts, 16 value columns each
    constexpr int NTH = 64 * NW;
    constexpr int KS = DK / 32;
    constexpr int CH = DK / 8;           // 16-byte chunks per K/Q row
    constexpr int NTMAX = NMAX / 16;
    constexpr int NKMAX = NMAX / 32;
    constexpr int RT = NTMAX > NW ? NTMAX / NW : 1;   // Gram row tiles per wavefront
    constexpr int ZR = L::ZR;            // root paths solved in registers
    static_assert(NMAX <= NTH, "one node per thread");
    static_assert(RT * NW >= NTMAX && RT <= 2, "Gram row tiles");
    // the commit's preparing wavefront: the first one past the node threads
    // (idle in the structure and path phases, a light share of the Gram)
    constexpr int PW = NMAX / 64;
    static_assert(PW < NW && 64 * PW >= NMAX, "the preparing wavefront holds no tree node");

    __shared__ __align__(16) unsigned char smem[L::TOTAL];
    GDN_ITEM_PHASE_DECL

    const int Hk = a.H_k, Hv = a.H_v;
    const int R = Hv / Hk;
    const int n_items = a.B * Hv;
    // Workgroups go to the 8 XCDs in turn; numbering the items so that each
    // XCD takes a contiguous run keeps the value heads of one key head (which
    // read the same K and Q) on one L2, dispatched close together
    const int g = gridDim.x;
    const int item = (g % 8 == 0 && g == n_items) ? (blockIdx.x % 8) * (g / 8) + blockIdx.x / 8 : blockIdx.x;
    if (item >= n_items) return;
    const int b = item / Hv, h = item % Hv, kh = h / R;

    int tid, N;
    {
        int t = threadIdx.x, n = a.N;
        asm volatile("" : "+v"(t));
        asm volatile("" : "+s"(n));
        tid = t;
        N = n;
    }
    int lane = tid & 63, lc = lane & 15, lg = lane >> 4;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // The thread index is passed through an opaque copy before the dense
    // phase, so that addresses derived from it are computed there rather
    // than hoisted above the tree phase and held in registers across it.
    auto refresh = [&]() {
        int t = tid;
        asm volatile("" : "+v"(t));
        tid = t;
        lane = t & 63;
        lc = lane & 15;
        lg = lane >> 4;
    };

    const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
    const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
    const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);

    unsigned char* KQb = smem + L::KQ;
    unsigned char* Zd = smem + L::AREA;
    float* kk = reinterpret_cast<float*>(smem + L::KK);
    float* qk = reinterpret_cast<float*>(smem + L::QK);
    uint8_t* pathc = smem + L::PATH;
    int* par = reinterpret_cast<int*>(smem + L::PAR);
    int* dep = reinterpret_cast<int*>(smem + L::DEP);
    float* gv = reinterpret_cast<float*>(smem + L::GV);
    float* bet = reinterpret_cast<float*>(smem + L::BET);
    float* Gs = reinterpret_cast<float*>(smem + L::GG);
    uint32_t* anc = reinterpret_cast<uint32_t*>(smem + L::ANC);
    uint32_t* tmask = reinterpret_cast<uint32_t*>(smem + L::TMASK);
    float* gam = reinterpret_cast<float*>(smem + L::GAM);
    int* misc = reinterpret_cast<int*>(smem + L::MISC);
    unsigned char* CKb = smem + L::CK;
    float* cx = reinterpret_cast<float*>(smem + L::CX);
    uint16_t* ct = reinterpret_cast<uint16_t*>(smem + L::CT);
    float* cg = reinterpret_cast<float*>(smem + L::CG);
    float* cb = reinterpret_cast<float*>(smem + L::CB);
    int8_t* cpar = reinterpret_cast<int8_t*>(smem + L::CPAR);
    uint8_t* cpath = smem + L::CPATH;
    int* cmisc = reinterpret_cast<int*>(smem + L::CMISC);

    // Natural 16-byte chunk c (elements 8c .. 8c + 7) of row `row` of K or Q
    // into the buffer, in the k-slot order the MFMA fragments read: element
    // 32 ks + 16 h + 4 g + r at position 32 ks + 8 g + 4 h + r, chunk 4 ks + g
    // stored at chunk position (4 ks + g) ^ (row mod CH); rows past N are zero
    auto put_chunk_at = [&](unsigned char* base, int row, int c, uint4 v, uint32_t keep) {
        const int sw = row & (CH - 1);
        const int ks = c >> 2, m = c & 3, hh = m >> 1, g0 = (m & 1) << 1;
        const int rbase = row * (DK * 2) + 8 * hh;
        *reinterpret_cast<uint2*>(base + rbase + (((4 * ks + g0) ^ sw) << 4)) = make_uint2(v.x & keep, v.y & keep);
        *reinterpret_cast<uint2*>(base + rbase + (((4 * ks + g0 + 1) ^ sw) << 4)) = make_uint2(v.z & keep, v.w & keep);
    };
    auto put_chunk = [&](int row, int c, uint4 v) { put_chunk_at(KQb, row, c, v, row < N ? 0xFFFFFFFFu : 0u); };
    constexpr int KCH = NMAX * CH / NTH > 0 ? NMAX * CH / NTH : 1;   // chunks per thread
    static_assert(KCH * NTH >= NMAX * CH, "K/Q staging");
    auto stage = [&](const uint16_t* src) {
        uint4 v[KCH];
#pragma unroll
        for (int q = 0; q < KCH; ++q) {
            const int e = min(tid + q * NTH, NMAX * CH - 1);
            v[q] = *reinterpret_cast<const uint4*>(
                src + ((static_cast<size_t>(b) * N + min(e / CH, N - 1)) * Hk + kh) * DK + (e % CH) * 8);
        }
#pragma unroll
        for (int q = 0; q < KCH; ++q) {
            const int e = tid + q * NTH;
            if (e < NMAX * CH) put_chunk(e / CH, e % CH, v[q]);
        }
    };
    auto frag = [&](int row, int ks) -> bf16x8 {
        return load_frag(KQb + row * (DK * 2) + (((4 * ks + lg) ^ (row & (CH - 1))) << 4));
    };
    auto cfrag = [&](int row, int ks) -> bf16x8 {
        return load_frag(CKb + row * (DK * 2) + (((4 * ks + lg) ^ (row & (CH - 1))) << 4));
    };

    // ------------------------------------------------ fused commit
    // One chunk of the accepted path, from root-first position c0 on, by the
    // calling wavefront: K rows into CK, G and beta, X, then T' (hi, lo).
    // Its global loads (the chunk's K rows, g and beta of its nodes), issued
    // ahead of the rest so that their latency passes in other work.
    constexpr int KL = 16 * CH / 64;   // 16-byte pieces of the chunk's K rows per lane
    static_assert(KL * 64 == 16 * CH, "K pieces per lane");
    struct PrepLoads {
        uint4 k[KL];
        float g, beta;
    };
    auto commit_load = [&](int c0) __attribute__((always_inline)) -> PrepLoads {
        PrepLoads r;
        const int m = cmisc[0];
        const int n = min(m - c0, 16);
        const uint16_t* kp = static_cast<const uint16_t*>(c.k);
#pragma unroll
        for (int q = 0; q < KL; ++q) {
            const int e = lane + 64 * q;
            const int t = e / CH, ch = e % CH;
            const int node = cpath[m - 1 - (c0 + min(t, n - 1))];
            r.k[q] = *reinterpret_cast<const uint4*>(kp + ((static_cast<size_t>(b) * N + node) * Hk + kh) * DK + 8 * ch);
        }
        const size_t nh = (static_cast<size_t>(b) * N + cpath[m - 1 - (c0 + min(lane & 15, n - 1))]) * Hv + h;
        r.g = c.g[nh];
        r.beta = c.beta[nh];
        return r;
    };
    auto commit_prep_rest = [&](int c0, const PrepLoads& r) __attribute__((always_inline)) {
        const int m = cmisc[0];
        const int n = min(m - c0, 16);
#pragma unroll
        for (int q = 0; q < KL; ++q) {
            const int e = lane + 64 * q;
            const int t = e / CH, ch = e % CH;
            put_chunk_at(CKb, t, ch, r.k[q], t < n ? 0xFFFFFFFFu : 0u);
        }
        float G = lane < n ? r.g : 0.f;
        const float bt = lane < n ? r.beta : 0.f;
#pragma unroll
        for (int o = 1; o < 16; o <<= 1) {
            const float x = __shfl_up(G, o, 16);
            if ((lane & 15) >= o) G += x;
        }
        if (lane < 16) {
            cg[lane] = G;
            cb[lane] = bt;
        }
        WaveSync::sync();
        // X_ts = beta_t D_ts (k_t . k_s), s < t < n; lane: t = 4 lg + r, s = lc
        f32x4 gr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 af = cfrag(lc, ks);
            gr = mfma(af, af, gr);
        }
        {
            const float Gs = cg[lc];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = 4 * lg + r;
                cx[16 * t + lc] = lc < t && t < n ? cb[t] * __expf(cg[t] - Gs) * gr[r] : 0.f;
            }
        }
        WaveSync::sync();
        // column j of (I + X)^-1 by forward substitution, then
        // T'_sj = D_{n-1, s} [(I + X)^-1]_sj beta_j
        if (lane < 16) {
            const int j = lane;
            float y[16];
#pragma unroll
            for (int t = 0; t < 16; ++t) {
                // one row of X at a time (the opaque offset keeps the loads
                // from being hoisted, which would hold every row at once)
                int xo = 16 * t;
                asm volatile("" : "+v"(xo));
                float xr[16];
#pragma unroll
                for (int q = 0; q < (t + 3) / 4; ++q) {
                    const f32x4 x4 = *reinterpret_cast<const f32x4*>(cx + xo + 4 * q);
#pragma unroll
                    for (int e = 0; e < 4; ++e) xr[4 * q + e] = x4[e];
                }
                float acc = t == j ? 1.f : 0.f;
#pragma unroll
                for (int s = 0; s < t; ++s) acc -= xr[s] * y[s];
                // orders this row's result before the next row's offset
                asm volatile("" : "+v"(acc));
                y[t] = acc;
            }
            const float Gn = cg[max(n - 1, 0)];
            const float bj = j < n ? cb[j] : 0.f;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                const float tv = s < n ? __expf(Gn - cg[s]) * y[s] * bj : 0.f;
                const __bf16 th = static_cast<__bf16>(tv);
                const __bf16 tl = static_cast<__bf16>(tv - static_cast<float>(th));
                ct[16 * s + j] = __builtin_bit_cast(uint16_t, th);
                ct[256 + 16 * s + j] = __builtin_bit_cast(uint16_t, tl);
            }
        }
    };
    auto commit_prep = [&](int c0) __attribute__((always_inline)) { commit_prep_rest(c0, commit_load(c0)); };
    // The prepared chunk from root-first position c0 applied to this
    // wavefront's 16 state rows s0 (the layout of s0r below); cvr: this
    // lane's piece of the chunk's V row lc (value columns col0 + 4 lg .. + 3)
    auto commit_apply = [&](float4 (&s0)[2 * KS], int c0, uint2 cvr, const s16x4& eye) __attribute__((always_inline)) {
        const int m = cmisc[0];
        const int n = min(m - c0, 16);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        // P_tc = k_t . S_c (lane: t = 4 lg + r, value row c = lc), S as hi + lo
        f32x4 ph = zero, pl = zero;
        bf16x8 af[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            af[ks] = cfrag(lc, ks);
            const float4 x0 = s0[2 * ks], x1 = s0[2 * ks + 1];
            const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
            bf16x8 hi, lo;
            split8(x, hi, lo);
            ph = mfma(af[ks], hi, ph);
            pl = mfma(af[ks], lo, pl);
        }
        // right-hand side V - gamma o P (zero past the chunk), as hi + lo
        const f32x4 vt = mfma16(__builtin_bit_cast(s16x4, cvr), eye, zero);
        s16x4 rh4, rl4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 4 * lg + r;
            const float rv = t < n ? vt[r] - __expf(cg[t]) * (ph[r] + pl[r]) : 0.f;
            const __bf16 hv = static_cast<__bf16>(rv);
            rh4[r] = __builtin_bit_cast(short, hv);
            rl4[r] = __builtin_bit_cast(short, static_cast<__bf16>(rv - static_cast<float>(hv)));
        }
        // W = T' (V - gamma o P): lane s = 4 lg + r, c = lc, the B operand
        // layout of the update
        const s16x4 th4 = *reinterpret_cast<const s16x4*>(ct + 16 * lc + 4 * lg);
        const s16x4 tl4 = *reinterpret_cast<const s16x4*>(ct + 256 + 16 * lc + 4 * lg);
        f32x4 w = mfma16(th4, rh4, zero);
        w = mfma16(tl4, rh4, w);
        w = mfma16(th4, rl4, w);
        s16x4 wh4, wl4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const __bf16 hv = static_cast<__bf16>(w[r]);
            wh4[r] = __builtin_bit_cast(short, hv);
            wl4[r] = __builtin_bit_cast(short, static_cast<__bf16>(w[r] - static_cast<float>(hv)));
        }
        // S <- gamma_{n-1} S + K^T W per 16-column block q of d_k: the A
        // operand k_{4 lg + r}[16 q + lc] is the fragment of K row lc
        // transposed by an MFMA against the identity (exact: bf16 values)
        const float gl = __expf(cg[max(n - 1, 0)]);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const uint4 au = __builtin_bit_cast(uint4, af[ks]);
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                const s16x4 ain = __builtin_bit_cast(s16x4, hf == 0 ? make_uint2(au.x, au.y) : make_uint2(au.z, au.w));
                const f32x4 kt = mfma16(ain, eye, zero);
                s16x4 ka;
#pragma unroll
                for (int r = 0; r < 4; ++r) ka[r] = __builtin_bit_cast(short, static_cast<__bf16>(kt[r]));
                f32x4 acc = __builtin_bit_cast(f32x4, s0[2 * ks + hf]) * gl;
                acc = mfma16(ka, wh4, acc);
                acc = mfma16(ka, wl4, acc);
                s0[2 * ks + hf] = __builtin_bit_cast(float4, acc);
            }
        }
    };
    // V piece of the chunk at c0 for commit_apply (row lc of the chunk)
    auto commit_v = [&](int c0, int col) __attribute__((always_inline)) -> uint2 {
        const int m = cmisc[0];
        const int t = min(c0 + lc, m - 1);
        const size_t nh = (static_cast<size_t>(b) * N + cpath[m - 1 - t]) * Hv + h;
        return *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(c.v) + nh * DV + col + 4 * lg);
    };
    // Every chunk of the path.  `ready0`: chunk 0 is prepared and s0 holds
    // the previous state; otherwise both happen here.  Between chunks the
    // state goes out to S_next and comes back (each lane reads what it
    // wrote), so that no state registers are held across a preparation.
    auto commit_all = [&](float4 (&s0)[2 * KS], int col, bool ready0, uint2 cvr0, const s16x4& eye)
                          __attribute__((always_inline)) {
        const int m = cmisc[0];
        const float* prev = c.S0 + ((static_cast<size_t>(b) * Hv + h) * DV + col + lc) * DK + 4 * lg;
        float* next = c.S_next + ((static_cast<size_t>(b) * Hv + h) * DV + col + lc) * DK + 4 * lg;
        for (int c0 = 0; c0 < m; c0 += 16) {
            // lane indices through an opaque copy: LDS addresses are then
            // formed per chunk instead of held across the loop
            refresh();
            if (c0 > 0 || !ready0) {
                __syncthreads();   // the previous chunk is applied
                if (wave == 0) commit_prep(c0);
                __syncthreads();
                __threadfence();   // this lane's stores of the state are visible to its loads
                const float4* src = reinterpret_cast<const float4*>(c0 == 0 ? prev : next);
#pragma unroll
                for (int q = 0; q < 2 * KS; ++q) s0[q] = src[4 * q];
            }
            commit_apply(s0, c0, (ready0 && c0 == 0) ? cvr0 : commit_v(c0, col), eye);
            if (c0 + 16 < m) {
#pragma unroll
                for (int q = 0; q < 2 * KS; ++q) reinterpret_cast<float4*>(next)[4 * q] = s0[q];
            }
        }
    };
    auto commit_store = [&](const float4 (&s0)[2 * KS], int col) __attribute__((always_inline)) {
        float4* dst = reinterpret_cast<float4*>(c.S_next + ((static_cast<size_t>(b) * Hv + h) * DV + col + lc) * DK + 4 * lg);
#pragma unroll
        for (int q = 0; q < 2 * KS; ++q) dst[4 * q] = s0[q];
    };

    // ------------------------------------------------ (1) scalars, K, Q rows
    GDN_ITEM_PHASE(0);
    if (tid < 3) misc[tid] = 0;
    bool bad = false;
    if (tid < NMAX) {
        // a parent outside [-1, i - 1] is flagged and read as -1
        const int i = tid;
        int p = -1;
        float gi = 0.f, bi = 0.f;
        if (i < N) {
            p = a.parent[static_cast<size_t>(b) * N + i];
            const size_t nh = (static_cast<size_t>(b) * N + i) * Hv + h;
            gi = a.g[nh];
            bi = a.beta[nh];
        }
        bad = i < N && (p < -1 || p >= i);
        par[i] = bad ? -1 : p;
        gv[i] = gi;
        bet[i] = bi;
        if (tid < NTMAX) tmask[tid] = 0u;
        {
            // the previous tree's parents (outside [-1, i - 1]: read as -1)
            int pp = -1;
            if (i < N) {
                pp = c.parent[static_cast<size_t>(b) * N + i];
                if (pp < -1 || pp >= i) pp = -1;
            }
            cpar[i] = static_cast<int8_t>(pp);
        }
    }
    {
        if (tid == NTH - 1) {
            // an accepted node out of range is reported and read as -1
            int acc = c.accepted[b];
            const bool badacc = acc < -1 || acc >= N;
            if (h == 0) c.accept_status[b] = badacc ? GDN_ERR_ACCEPT : 0;
            cmisc[1] = badacc ? -1 : acc;
        }
    }
    // Q rows of this wavefront's Gram row tiles, in the k-slot order of the
    // buffer, loaded now so that they arrive with K
    const int NT = (N + 15) >> 4;
    bf16x8 qf[RT][KS];
#pragma unroll
    for (int u = 0; u < RT; ++u) {
        const int I = u == 0 ? wave : NTMAX - 1 - wave;
        const int row = min(16 * min(I, NTMAX - 1) + lc, N - 1);
        const uint16_t* qr = qg + ((static_cast<size_t>(b) * N + row) * Hk + kh) * DK;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) qf[u][ks] = load_frag2(qr + 32 * ks + 4 * lg, qr + 32 * ks + 16 + 4 * lg);
    }
    stage(kg);
    __syncthreads();

    // ------------------------------------------------ (2) structure
    // One walk per node up to its root: its path (slot d = distance from the
    // node), depth, G (the path sum of g), ancestor bits and the tiles that
    // hold pairs
    GDN_ITEM_PHASE(1);
    if (tid < NMAX) {
        const int i = tid;
        uint32_t bits[L::AW];
#pragma unroll
        for (int w = 0; w < L::AW; ++w) bits[w] = 0u;
        int d = 0;
        float G = 0.f;
        uint32_t mask = 0u;
        if (i < N) {
            for (int s = i; s >= 0; s = par[s]) {
                if (d < ZR) pathc[i * ZR + d] = static_cast<uint8_t>(s);
                G += gv[s];
                mask |= 1u << (s >> 4);
#pragma unroll
                for (int w = 0; w < L::AW; ++w) bits[w] |= (s >> 5) == w ? 1u << (s & 31) : 0u;
                ++d;
            }
            atomicOr(&tmask[i >> 4], mask);
            if (d > ZR) misc[1] = 1;
            if (bad) misc[2] = 1;
        }
        dep[i] = d;
        Gs[i] = G;
        gam[i] = i < N ? __expf(G) : 0.f;
#pragma unroll
        for (int w = 0; w < L::AW; ++w) anc[i * L::AW + w] = bits[w];
    }
    // fused commit: one lane of the preparing wavefront walks the accepted
    // path
    {
        if (wave == PW) {
            if (lane == 0) {
                int mm = 0;
                for (int s = cmisc[1]; s >= 0; s = cpar[s]) cpath[mm++] = static_cast<uint8_t>(s);
                cmisc[0] = mm;
            }
        }
    }
    __syncthreads();
    const bool fast = misc[1] == 0;
    if (h == 0 && tid == 0) a.tree_status[b] = misc[2] ? GDN_ERR_TREE : 0;

    if (!fast) {
        // a path longer than ZR: the per-node walk, one wavefront per
        // 64-column slice in turn (the others have nothing to do for this item)
        {
            // the committed state first: the walk reads it back from a.S0
            refresh();
            const int col = NW == 8 ? 32 * (wave & 3) + 16 * (wave >> 2) : 16 * wave;
            float4 s0c[2 * KS];
            if (cmisc[0] == 0) {
                const float4* src = reinterpret_cast<const float4*>(
                    c.S0 + ((static_cast<size_t>(b) * Hv + h) * DV + col + lc) * DK + 4 * lg);
#pragma unroll
                for (int q = 0; q < 2 * KS; ++q) s0c[q] = src[4 * q];
            }
            s16x4 eye;
#pragma unroll
            for (int q = 0; q < 4; ++q) eye[q] = 4 * lg + q == lc ? static_cast<short>(0x3F80) : short(0);
            commit_all(s0c, col, false, make_uint2(0u, 0u), eye);
            commit_store(s0c, col);
            __threadfence();
        }
        __syncthreads();   // every read of the tree arrays is done
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
        return;
    }

    // ------------------------------------------------ (3) Gram values
    GDN_ITEM_PHASE(2);
#pragma unroll
    for (int u = 0; u < RT; ++u) {
        const int I = u == 0 ? wave : NTMAX - 1 - wave;
        if (I >= NT || I >= NTMAX) continue;
        bf16x8 kf[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kf[ks] = frag(16 * I + lc, ks);
        const uint32_t tm = tmask[I];
        int drow[4];
        uint32_t awr[4][L::AW];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int i = 16 * I + 4 * lg + rr;
            drow[rr] = dep[i];
#pragma unroll
            for (int w = 0; w < L::AW; ++w) awr[rr][w] = anc[i * L::AW + w];
        }
        for (int J = 0; J <= I; ++J) {
            if (!((tm >> J) & 1u)) continue;
            f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 kb = frag(16 * J + lc, ks);
                akk = mfma(kf[ks], kb, akk);
                aqk = mfma(qf[u][ks], kb, aqk);
            }
            // lane: rows 16 I + 4 lg + rr, column node s = 16 J + lc; pair
            // (i, s) lands in slot i ZR + dep[i] - dep[s], other entries in the sink
            const int sn = 16 * J + lc;
            const int ds = dep[sn];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const int i = 16 * I + 4 * lg + rr;
                uint32_t w = 0u;
#pragma unroll
                for (int x = 0; x < L::AW; ++x) w = (sn >> 5) == x ? awr[rr][x] : w;
                const bool pair = i < N && ((w >> (sn & 31)) & 1u);
                const int p = pair ? i * ZR + drow[rr] - ds : L::CAP;
                kk[p] = akk[rr];
                qk[p] = aqk[rr];
            }
        }
    }
    // fused commit: the loads of the path's first chunk, issued once this
    // wavefront's (light) share of the Gram is done, arrive during the
    // barrier and the next phase
    PrepLoads pl{};
    {
        if (wave == PW && cmisc[0] > 0) pl = commit_load(0);
    }
    __syncthreads();

    // ------------------------------------------------ (4) paths
    GDN_ITEM_PHASE(3);
    // fused commit: the first chunk's T' by the preparing wavefront, which
    // holds no node
    {
        if (wave == PW && cmisc[0] > 0) commit_prep_rest(0, pl);
    }
    // the path of this thread's node, four node indices (bytes) per register
    uint32_t ttp[ZR / 4];
    auto tt = [&](int d) -> int { return static_cast<int>((ttp[d >> 2] >> (8 * (d & 3))) & 0xFFu); };
    int m = 0;
    if (tid < NMAX) {
        const int i = tid;
        m = dep[i];
#pragma unroll
        for (int q = 0; q < ZR / 4; ++q) {
            uint32_t w = 0u;
#pragma unroll
            for (int r = 0; r < 4; ++r) w |= static_cast<uint32_t>(pathc[i * ZR + min(4 * q + r, max(m - 1, 0))]) << (8 * r);
            ttp[q] = w;
        }
    } else {
#pragma unroll
        for (int q = 0; q < ZR / 4; ++q) ttp[q] = 0u;
    }

    // ------------------------------------------------ (5) rows of Z~
    // Along the path p_0 = i, p_1, .., p_{m-1} (the root) the row z of
    // Y (I + X)^-1 solves z_e = Y_{i,p_e} - sum_{d < e} z_d X_{p_d,p_e}.  As
    // D_{i,p_d} D_{p_d,p_e} = D_{i,p_e}, z_e = D_{i,p_e} y_e with
    //     y_e = q_i . k_{p_e} - sum_{d < e} (beta_{p_d} y_d) (k_{p_d} . k_{p_e}),
    // where k_{p_d} . k_{p_e} sits at slot e - d of row p_d.  Slots past a
    // row's root hold no pair; what they feed is y_e for e >= m, which is
    // dropped.  The scaling by D_{i,p_d} beta_{p_d} follows in (6).
    GDN_ITEM_PHASE(4);
    float z[ZR];
    if (tid < N) {
        const int i = tid;
#pragma unroll
        for (int d = 0; d < ZR; ++d) z[d] = d < m ? qk[i * ZR + d] : 0.f;
        float xr[ZR - 1];
        float bn = bet[tt(0)];
#pragma unroll
        for (int e = 0; e < ZR - 1; ++e) xr[e] = kk[tt(0) * ZR + 1 + e];
#pragma unroll
        for (int d = 0; d < ZR - 1; ++d) {
            float xn[ZR - 1];
#pragma unroll
            for (int e = 0; e + d + 2 < ZR; ++e) xn[e] = kk[tt(d + 1) * ZR + 1 + e];
            const float yd = z[d] * bn;
            bn = bet[tt(d + 1)];
#pragma unroll
            for (int e = 0; e + d + 1 < ZR; ++e) z[d + 1 + e] -= yd * xr[e];
#pragma unroll
            for (int e = 0; e + d + 2 < ZR; ++e) xr[e] = xn[e];
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // ------------------------------------------------ (6) S0, V; Z~ fragments
    GDN_ITEM_PHASE(5);
    refresh();
    // S0 rows and V of this wavefront's 16 value columns: s0r[2 ks + hh]
    // holds d_k columns 32 ks + 16 hh + 4 lg .. + 3 of row col0 + lc; vr[S]
    // holds columns col0 + 4 lg .. + 3 of node 16 S + lc
    const int col0 = NW == 8 ? 32 * (wave & 3) + 16 * (wave >> 2) : 16 * wave;
    float4 s0r[2 * KS];
    uint2 vr[NTMAX];
    uint2 cvr0 = make_uint2(0u, 0u);
    auto load_v = [&]() __attribute__((always_inline)) {
        const uint16_t* vsrc = vg + static_cast<size_t>(b) * N * Hv * DV + static_cast<size_t>(h) * DV + col0 + 4 * lg;
#pragma unroll
        for (int S = 0; S < NTMAX; ++S)
            vr[S] = *reinterpret_cast<const uint2*>(vsrc + static_cast<size_t>(min(16 * S + lc, N - 1)) * Hv * DV);
    };
    // fused commit: an accepted path of more than one chunk is applied
    // after the Z~ scatter with the V loads held back (its chunk
    // preparations run in between and need the registers)
    const int cm = cmisc[0];
    {
        const float4* src = reinterpret_cast<const float4*>(
            c.S0 + ((static_cast<size_t>(b) * Hv + h) * DV + col0 + lc) * DK + 4 * lg);
#pragma unroll
        for (int q = 0; q < 2 * KS; ++q) s0r[q] = src[4 * q];
        if (cm <= 16) load_v();
        {
            if (cm > 0) cvr0 = commit_v(0, col0);
        }
    }
    __syncthreads();   // every read of the tree arrays is done
    for (int e = tid; e < L::ZD_BYTES / 16; e += NTH) reinterpret_cast<uint4*>(Zd)[e] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();
    if (tid < N) {
        // block (I, kap) holds rows 16 I.., nodes 32 kap..; node t of row i
        // sits in lane group ((t >> 2) & 3), slot 4 ((t >> 4) & 1) + (t & 3)
        const int i = tid;
        const float Gi = Gs[i];
#pragma unroll
        for (int d = 0; d < ZR; ++d) {
            if (d < m) {
                const int t = tt(d);
                const float zb = z[d] * bet[t] * __expf(Gi - Gs[t]);
                const __bf16 zh = static_cast<__bf16>(zb);
                const __bf16 zl = static_cast<__bf16>(zb - static_cast<float>(zh));
                const int el = (((((t >> 2) & 3) << 4) | (i & 15)) << 3) + (((t >> 4) & 1) << 2) + (t & 3);
                unsigned char* blk = Zd + 2048 * (vi_zblocks(i >> 4) + (t >> 5));
                reinterpret_cast<__bf16*>(blk)[el] = zh;
                reinterpret_cast<__bf16*>(blk + 1024)[el] = zl;
            }
        }
    }
    __syncthreads();

    // ------------------------------------------------ (7) R'
    GDN_ITEM_PHASE(6);
    // identity for the transposes: lane (n, g) holds B[4 g + j][n]
    s16x4 eye;
#pragma unroll
    for (int q = 0; q < 4; ++q) eye[q] = 4 * lg + q == lc ? static_cast<short>(0x3F80) : short(0);
    {
        if (cm > 16) {
            commit_all(s0r, col0, true, cvr0, eye);
            load_v();
        } else if (cm > 0) {
            commit_apply(s0r, 0, cvr0, eye);
        }
        commit_store(s0r, col0);
    }
    bf16x8 s0h[KS], s0l[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const float4 x0 = s0r[2 * ks], x1 = s0r[2 * ks + 1];
        const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        split8(x, s0h[ks], s0l[ks]);
    }
    bf16x8 rh[NKMAX], rl[NKMAX];
#pragma unroll
    for (int kap = 0; kap < NKMAX; ++kap) {
        float rt[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int S = 2 * kap + half;
            if (S < NT) {
                f32x4 ah = {0.f, 0.f, 0.f, 0.f}, al = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 fa = frag(16 * S + lc, ks);
                    ah = mfma(fa, s0h[ks], ah);
                    al = mfma(fa, s0l[ks], al);
                }
                const f32x4 gm = *reinterpret_cast<const f32x4*>(gam + 16 * S + 4 * lg);
                const f32x4 vt = mfma16(__builtin_bit_cast(s16x4, vr[S]), eye, f32x4{0.f, 0.f, 0.f, 0.f});
                const f32x4 pk = ah + al;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float vv = 16 * S + 4 * lg + rr < N ? vt[rr] : 0.f;
                    rt[4 * half + rr] = vv - gm[rr] * pk[rr];
                }
            } else {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) rt[4 * half + rr] = 0.f;
            }
        }
        split8(rt, rh[kap], rl[kap]);
    }

    // ------------------------------------------------ (8) Q into the buffer
    GDN_ITEM_PHASE(7);
    __syncthreads();
    stage(qg);
    __syncthreads();

    // ------------------------------------------------ (9) O tiles
    GDN_ITEM_PHASE(8);
    // O^T = gamma o (S0 Q^T) + R'^T Z~^T; lane (lc, lg) gets value columns
    // col0 + 4 lg .. + 3 of node 16 I + lc
    float* obase = a.o + static_cast<size_t>(b) * N * Hv * DV + static_cast<size_t>(h) * DV + col0 + 4 * lg;
#pragma unroll
    for (int I = 0; I < NTMAX; ++I) {
        if (I < NT) {
            f32x4 ah = {0.f, 0.f, 0.f, 0.f}, al = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const bf16x8 fb = frag(16 * I + lc, ks);
                ah = mfma(s0h[ks], fb, ah);
                al = mfma(s0l[ks], fb, al);
            }
            f32x4 acc = (ah + al) * gam[16 * I + lc];
            const unsigned char* blk = Zd + 2048 * vi_zblocks(I) + 16 * lane;
#pragma unroll
            for (int kap = 0; kap <= I / 2; ++kap) {
                const bf16x8 zh = load_frag(blk + 2048 * kap);
                const bf16x8 zl = load_frag(blk + 2048 * kap + 1024);
                acc = mfma(rh[kap], zh, acc);
                acc = mfma(rl[kap], zh, acc);
                acc = mfma(rh[kap], zl, acc);
            }
            // o is written once and not read back here: streaming stores
            const int i = 16 * I + lc;
            if (i < N)
                __builtin_nontemporal_store(acc, reinterpret_cast<f32x4*>(obase + static_cast<size_t>(i) * Hv * DV));
        }
    }
    GDN_ITEM_PHASE(9);
    GDN_ITEM_PHASE_END;
}

hipError_t launch_cv(const VerifyArgs& a, const CommitPrev& c, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(a.B) * a.H_v);
    auto go = [&](auto kern, int dv) {
        hipLaunchKernelGGL(kern, grid, dim3(4 * dv), 0, stream, a, c);
        return hipGetLastError();
    };
    if (a.N <= 64) {
        if (a.d_k == 64)
            return a.d_v == 64 ? go(commit_verify_kernel<64, 64, 64>, 64) : go(commit_verify_kernel<64, 64, 128>, 128);
        return a.d_v == 64 ? go(commit_verify_kernel<64, 128, 64>, 64) : go(commit_verify_kernel<64, 128, 128>, 128);
    }
    if (a.d_k == 64)
        return a.d_v == 64 ? go(commit_verify_kernel<128, 64, 64>, 64) : go(commit_verify_kernel<128, 64, 128>, 128);
    return a.d_v == 64 ? go(commit_verify_kernel<128, 128, 64>, 64) : go(commit_verify_kernel<128, 128, 128>, 128);
}

}  // namespace

hipError_t launch_commit_verify(const VerifyArgs& a, const CommitPrev& c, hipStream_t stream) {
    return launch_cv(a, c, stream);
}

}  // namespace gdn
