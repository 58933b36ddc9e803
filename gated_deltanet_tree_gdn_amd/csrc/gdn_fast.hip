// gdn_fast.hip -- MFMA tree verification for bf16 q/k/v on gfx950.
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
// Work decomposition: one workgroup per (sequence, value head), d_v/32
// wavefronts; wavefront w owns value columns [32w, 32w + 32) as two 16-wide
// MFMA tiles and keeps its slice of S0 (as a bf16 hi + lo pair), and R', in
// registers.  K is staged in LDS (read by every wavefront); Q rows are read
// straight from global memory.  Dense contractions run on
// v_mfma_f32_16x16x32_bf16: q and k are exact bf16, S0, R' and Z~ are split
// into hi + lo bf16 so products stay near fp32 accuracy.
//
// Phases: (1) issue the S0 and K loads; (2) parents, depth by pointer
// jumping, offsets of each node's path in a pair list; (3) pair Gram values
// (MFMA over the lower 16x16 tiles that contain ancestor pairs, scattered
// into the pair list); (4) G, gamma, X, Y and the rows of Z~, one thread per
// node; (5) per wavefront: K S0^T -> R', then per 16-row tile Q S0^T and
// Z~ R' -> o.
//
// Trees whose pair list exceeds the LDS budget fall back, inside the same
// workgroup, to the per-node walk of gdn_walk.h.

#include <hip/hip_runtime.h>

#include <cstdint>

#include "gdn_internal.h"
#include "gdn_walk.h"

namespace gdn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// x ~= hi + lo with hi = bf16(x) (nearest) and lo = bf16(x - hi).
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const __bf16 h = static_cast<__bf16>(x[j]);
        hi[j] = h;
        lo[j] = static_cast<__bf16>(x[j] - static_cast<float>(h));
    }
}

__device__ __forceinline__ bf16x8 zero_frag() {
    bf16x8 z;
#pragma unroll
    for (int j = 0; j < 8; ++j) z[j] = static_cast<__bf16>(0.f);
    return z;
}

__device__ __forceinline__ bf16x8 load_frag(const void* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ uint4 mask4(uint4 v, uint32_t m) { return make_uint4(v.x & m, v.y & m, v.z & m, v.w & m); }

// Number of 16x32 blocks of Z~ for the first I row tiles: row tile I has
// floor(I/2) + 1 blocks (k-steps of 32 nodes up to its diagonal).
__host__ __device__ constexpr int zblocks_before(int I) {
    return (I & 1) ? ((I + 1) / 2) * ((I + 1) / 2) : (I / 2) * (I / 2 + 1);
}

// LDS layout (bytes) for trees of at most NMAX nodes.  For NMAX <= 128
// (DENSE) Q is staged next to K and Z~ is stored as ready-made MFMA A
// fragments; for larger trees Q is read from global memory and the
// fragments are built from the pair list.
template <int NMAX, int DK>
struct Lds {
    static constexpr bool DENSE = NMAX <= 128;
    // pair-list capacity: every tree of N <= 64 fits; N <= 128 covers depth
    // <= 16 everywhere; N <= 256 covers 16 ancestors per node on average
    static constexpr int CAP = NMAX <= 64 ? NMAX * (NMAX + 1) / 2 : (NMAX <= 128 ? 2048 : 4096);
    static constexpr int AW = NMAX / 32;        // ancestor bit-row words
    static constexpr int KROW = DK * 2 + 16;    // staged k / q row, padded against bank conflicts
    static constexpr int KS_OFF = 0;
    static constexpr int QS_OFF = NMAX * KROW;
    static constexpr int ZD = QS_OFF + (DENSE ? NMAX * KROW : 0);      // Z~ fragment blocks (hi 1 KiB + lo 1 KiB)
    static constexpr int ZD_BYTES = DENSE ? 2048 * zblocks_before(NMAX / 16) : 0;
    static constexpr int XC = ZD + ZD_BYTES;    // float[CAP]: k.k, then X
    static constexpr int YC = XC + 4 * CAP;     // float[CAP]: q.k, then Y
    static constexpr int ZC = YC + 4 * CAP;     // float[CAP]: rows of Z~
    static constexpr int OFP = ZC + 4 * CAP;    // uint16[CAP]: path offset of the ancestor
    static constexpr int PATH = OFP + 2 * CAP;  // uint8[CAP]: root..i path of every node
    static constexpr int NODE = (PATH + CAP + 15) & ~15;
    static constexpr int PAR = NODE;            // int[NMAX]
    static constexpr int DEP = PAR + 4 * NMAX;
    static constexpr int OFF = DEP + 4 * NMAX;
    static constexpr int NXT = OFF + 4 * NMAX;
    static constexpr int BET = NXT + 4 * NMAX;  // float[NMAX]: beta
    static constexpr int GG = BET + 4 * NMAX;   // G (path sum of g)
    static constexpr int GAM = GG + 4 * NMAX;   // gamma (0 past N)
    static constexpr int ANC = GAM + 4 * NMAX;  // uint32[NMAX][AW]: ancestor bit rows
    static constexpr int TMASK = ANC + 4 * AW * NMAX;  // uint32[NMAX/16]: tile (I, J) has pairs
    static constexpr int MISC = TMASK + 4 * (NMAX / 16);
    static constexpr int FBKQ = MISC + 64;      // float[2*DK] for the fallback walk
    static constexpr int TOTAL = FBKQ + 8 * DK;
    static_assert(NMAX * 64 * 4 + DK * 64 * 4 <= NODE, "fallback u and S0 buffers must fit below the node arrays");
};

// One wavefront owns 16 value columns (one MFMA tile): column 16 w + lc.
template <int NMAX, int DK, int DV>
__global__ __launch_bounds__(64 * (DV / 16)) void verify_fast_kernel(VerifyArgs a) {
    using L = Lds<NMAX, DK>;
    constexpr bool DENSE = L::DENSE;
    constexpr int NW = DV / 16;         // wavefronts
    constexpr int NTH = 64 * NW;        // threads
    constexpr int KS = DK / 32;         // MFMA k-steps over d_k
    constexpr int NTMAX = NMAX / 16;    // 16-row tiles
    constexpr int NKMAX = NMAX / 32;    // 32-node k-steps over the tree
    constexpr int KCH = NMAX * DK / 8 / NTH;  // 16-byte chunks of K (and Q) per thread
    static_assert(KCH >= 1 && NMAX * DK / 8 % NTH == 0, "K staging split");
    constexpr int IPT = (NMAX + NTH - 1) / NTH;  // nodes per thread in node loops
    constexpr int ZR = 16;              // path length kept in registers when solving a row of Z~

    __shared__ __align__(16) unsigned char smem[L::TOTAL];

    // ---- which (sequence, value head): the value heads sharing a key head
    // sit 8 blocks apart, so they land on the same XCD and share its L2.
    const int R = a.H_v / a.H_k;
    const int Lb = blockIdx.x;
    const int rem = Lb % (8 * R);
    const int grp = (Lb / (8 * R)) * 8 + (rem & 7);
    if (grp >= a.B * a.H_k) return;
    const int r = rem >> 3;
    const int b = grp / a.H_k;
    const int kh = grp % a.H_k;
    const int h = kh * R + r;
    const int N = a.N, Hk = a.H_k, Hv = a.H_v;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lc = lane & 15;
    const int lg = lane >> 4;
    const int col = 16 * wave + lc;  // this lane's value column

    const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(a.q);
    const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(a.k);
    const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(a.v);

    int* par = reinterpret_cast<int*>(smem + L::PAR);
    int* dep = reinterpret_cast<int*>(smem + L::DEP);
    int* off = reinterpret_cast<int*>(smem + L::OFF);
    int* nxt = reinterpret_cast<int*>(smem + L::NXT);
    float* bet = reinterpret_cast<float*>(smem + L::BET);
    float* Gs = reinterpret_cast<float*>(smem + L::GG);
    float* gam = reinterpret_cast<float*>(smem + L::GAM);
    uint32_t* anc = reinterpret_cast<uint32_t*>(smem + L::ANC);
    uint32_t* tmask = reinterpret_cast<uint32_t*>(smem + L::TMASK);
    int* misc = reinterpret_cast<int*>(smem + L::MISC);
    float* xc = reinterpret_cast<float*>(smem + L::XC);
    float* yc = reinterpret_cast<float*>(smem + L::YC);
    float* zc = reinterpret_cast<float*>(smem + L::ZC);
    uint16_t* ofp = reinterpret_cast<uint16_t*>(smem + L::OFP);
    uint8_t* pathc = smem + L::PATH;
    unsigned char* Ks = smem + L::KS_OFF;
    unsigned char* Qs = smem + L::QS_OFF;
    unsigned char* Zd = smem + L::ZD;

    // ---- (1) every global load this workgroup needs, issued up front and
    // unconditionally (indices clamped into range, out-of-range values
    // replaced after the load) so they all fly during the prologue: node
    // scalars, this wavefront's S0 rows (lane (lc, lg) holds d_k columns
    // [8 KS lg, 8 KS (lg + 1)) of row `col`), its V column for every node,
    // and a share of K and Q.
    int p_in[IPT];
    float g_in[IPT], b_in[IPT];
#pragma unroll
    for (int q = 0; q < IPT; ++q) {
        const int i = min(tid + q * NTH, N - 1);
        p_in[q] = a.parent[static_cast<size_t>(b) * N + i];
        const size_t nh = (static_cast<size_t>(b) * N + i) * Hv + h;
        g_in[q] = a.g[nh];
        b_in[q] = a.beta[nh];
    }
    // keep the node scalars ahead of the bulk loads: the prologue waits on
    // them only
    __builtin_amdgcn_sched_barrier(0);
    float4 s0r[2 * KS];
    {
        const float4* src = reinterpret_cast<const float4*>(a.S0 + ((static_cast<size_t>(b) * Hv + h) * DV + col) * DK + 8 * KS * lg);
#pragma unroll
        for (int q = 0; q < 2 * KS; ++q) s0r[q] = src[q];
    }
    uint4 kraw[KCH], qraw[DENSE ? KCH : 1];
#pragma unroll
    for (int q = 0; q < KCH; ++q) {
        const int e = tid + q * NTH;
        const int row = min(e / (DK / 8), N - 1);
        const size_t gofs = ((static_cast<size_t>(b) * N + row) * Hk + kh) * DK + (e % (DK / 8)) * 8;
        kraw[q] = *reinterpret_cast<const uint4*>(kg + gofs);
        if (DENSE) qraw[q] = *reinterpret_cast<const uint4*>(qg + gofs);
    }
    const size_t vbase = static_cast<size_t>(b) * N * Hv * DV + static_cast<size_t>(h) * DV + col;
    uint16_t vraw[NTMAX][4];
#pragma unroll
    for (int S = 0; S < NTMAX; ++S)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) vraw[S][rr] = vg[vbase + static_cast<size_t>(min(16 * S + 4 * lg + rr, N - 1)) * Hv * DV];

    // ---- (2) parents (invalid entries become -1 so every walk ends); depth
    // and the path sum G of g by pointer jumping: dep[i] counts the nodes and
    // Gs[i] sums g from i up to (excluding) nxt[i].
    int bad_local = 0;
#pragma unroll
    for (int q = 0; q < IPT; ++q) {
        const int i = tid + q * NTH;
        if (i < NMAX) {
            int p = i < N ? p_in[q] : -1;
            if (p < -1 || p >= i) {
                bad_local = 1;
                p = -1;
            }
            par[i] = p;
            nxt[i] = p;
            dep[i] = i < N ? 1 : 0;
            Gs[i] = i < N ? g_in[q] : 0.f;
            bet[i] = i < N ? b_in[q] : 0.f;
        }
    }
    if (tid < NMAX / 16) tmask[tid] = 0u;
    if (DENSE)
        for (int e = tid; e < L::ZD_BYTES / 16; e += NTH) reinterpret_cast<uint4*>(Zd)[e] = make_uint4(0u, 0u, 0u, 0u);
    const int bad = __syncthreads_or(bad_local);
    if (kh == 0 && r == 0 && tid == 0) a.tree_status[b] = bad ? GDN_ERR_TREE : 0;

    for (int round = 0; round < 9; ++round) {
        int c2[IPT], n2[IPT];
        float G2[IPT];
        int live = 0;
#pragma unroll
        for (int q = 0; q < IPT; ++q) {
            const int i = tid + q * NTH;
            c2[q] = 0;
            n2[q] = -1;
            G2[q] = 0.f;
            if (i < NMAX) {
                const int nx = nxt[i];
                c2[q] = dep[i] + (nx >= 0 ? dep[nx] : 0);
                G2[q] = Gs[i] + (nx >= 0 ? Gs[nx] : 0.f);
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
                Gs[i] = G2[q];
                nxt[i] = n2[q];
            }
        }
        if (!__syncthreads_or(live)) break;
    }

    // offsets of each node's path in the pair list (exclusive scan of depth);
    // gamma = exp(G)
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
    for (int i = tid; i < NMAX; i += NTH) gam[i] = i < N ? __expf(Gs[i]) : 0.f;
    __syncthreads();
    const int total = misc[0];

    if (total > L::CAP) {
        // deep tree: the per-node walk, one wavefront, one 64-column slice at a time
        if (wave != 0) return;
        float* u_s = reinterpret_cast<float*>(smem);
        float* s0_s = reinterpret_cast<float*>(smem + NMAX * 64 * 4);
        float* ki = reinterpret_cast<float*>(smem + L::FBKQ);
        for (int c0 = 0; c0 < DV; c0 += 64)
            walk_verify_slice_lds<uint16_t, DK, WaveSync>(a, b, h, c0, par, u_s, Gs, ki, ki + DK, s0_s);
        return;
    }

    // ---- K (and Q) into LDS (rows past N zeroed); root..i path, ancestor
    // bits and the tiles holding pairs, per node
#pragma unroll
    for (int q = 0; q < KCH; ++q) {
        const int e = tid + q * NTH;
        const int row = e / (DK / 8);
        const int cc = e % (DK / 8);
        const uint32_t keep = row < N ? 0xFFFFFFFFu : 0u;  // rows past N become zeros
        *reinterpret_cast<uint4*>(Ks + row * L::KROW + cc * 16) = mask4(kraw[q], keep);
        if (DENSE) *reinterpret_cast<uint4*>(Qs + row * L::KROW + cc * 16) = mask4(qraw[q], keep);
    }
    for (int i = tid; i < NMAX; i += NTH) {
        uint32_t bits[L::AW];
#pragma unroll
        for (int w = 0; w < L::AW; ++w) bits[w] = 0u;
        if (i < N) {
            int pos = off[i] + dep[i] - 1;
            uint32_t mask = 0u;
            for (int s = i; s >= 0; s = par[s]) {
                pathc[pos] = static_cast<uint8_t>(s);
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
    __syncthreads();

    auto q_frag = [&](int row, int ks) -> bf16x8 {
        if (DENSE) return load_frag(Qs + row * L::KROW + 2 * (8 * KS * lg + 8 * ks));
        return load_frag(qg + ((static_cast<size_t>(b) * N + min(row, N - 1)) * Hk + kh) * DK + 8 * KS * lg + 8 * ks);
    };
    auto k_frag = [&](int row, int ks) -> bf16x8 { return load_frag(Ks + row * L::KROW + 2 * (8 * KS * lg + 8 * ks)); };

    // ---- (3) Gram values of the ancestor pairs: the lower 16x16 tiles that
    // hold pairs, dealt round-robin to the wavefronts; each value lands at
    // its pair (i, s) = path position dep[s] - 1 of node i.
    const int NT = (N + 15) >> 4;
    {
        int t = 0;
        for (int I = 0; I < NT; ++I) {
            const uint32_t tm = tmask[I];
            for (int J = 0; J <= I; ++J) {
                if (!((tm >> J) & 1u)) continue;
                if (t++ % NW != wave) continue;
                f32x4 akk = {0.f, 0.f, 0.f, 0.f}, aqk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 kb = k_frag(16 * J + lc, ks);
                    akk = mfma(k_frag(16 * I + lc, ks), kb, akk);
                    aqk = mfma(q_frag(16 * I + lc, ks), kb, aqk);
                }
                const int s = 16 * J + lc;
                const int ds = dep[s];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int i = 16 * I + 4 * lg + rr;
                    const bool pair = i < N && ((anc[i * L::AW + (s >> 5)] >> (s & 31)) & 1u);
                    if (pair) {
                        const int p = off[i] + ds - 1;
                        yc[p] = aqk[rr];
                        if (s != i) xc[p] = akk[rr];
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- (4) per node: X and Y on its pairs, then its row of Z~ by a
    // right-looking sweep along its path (in registers for paths of up to
    // ZR nodes), scaled by beta of the column's node
    for (int i = tid; i < N; i += NTH) {
        const int o = off[i], m = dep[i];
        const float Gi = Gs[i], bi = bet[i];
        for (int t = 0; t < m - 1; ++t) {
            const float D = __expf(Gi - Gs[pathc[o + t]]);
            xc[o + t] *= bi * D;
            yc[o + t] *= D;
        }
    }
    __syncthreads();
    for (int i = tid; i < N; i += NTH) {
        const int o = off[i], m = dep[i];
        if (m <= ZR) {
            float z[ZR];
#pragma unroll
            for (int bb = 0; bb < ZR; ++bb) z[bb] = yc[o + min(bb, m - 1)];
#pragma unroll
            for (int aa = ZR - 1; aa >= 1; --aa) {
                if (aa < m) {
                    const float za = z[aa];
                    const int oa = ofp[o + aa];
#pragma unroll
                    for (int bb = 0; bb < aa; ++bb) z[bb] -= za * xc[oa + bb];
                }
            }
#pragma unroll
            for (int bb = 0; bb < ZR; ++bb)
                if (bb < m) zc[o + bb] = z[bb] * bet[pathc[o + bb]];
        } else {
            for (int bb = 0; bb < m; ++bb) zc[o + bb] = yc[o + bb];
            for (int aa = m - 1; aa >= 1; --aa) {
                const float za = zc[o + aa];
                const int oa = ofp[o + aa];
                for (int bb = 0; bb < aa; ++bb) zc[o + bb] -= za * xc[oa + bb];
            }
            for (int bb = 0; bb < m; ++bb) zc[o + bb] *= bet[pathc[o + bb]];
        }
        if (DENSE) {
            // scatter the row into the A-fragment blocks of the Z~ R' product:
            // block (I, kap) = rows 16I.., nodes 32kap..; node t sits in lane
            // group ((t >> 2) & 3), slot 4 ((t >> 4) & 1) + (t & 3)
            const int I = i >> 4;
            unsigned char* rowblk = Zd + 2048 * zblocks_before(I);
            for (int bb = 0; bb < m; ++bb) {
                const int t = pathc[o + bb];
                const float zz = zc[o + bb];
                const __bf16 zh = static_cast<__bf16>(zz);
                const __bf16 zl = static_cast<__bf16>(zz - static_cast<float>(zh));
                const int ln = (((t >> 2) & 3) << 4) | (i & 15);
                const int e = ln * 8 + (((t >> 4) & 1) << 2) + (t & 3);
                unsigned char* blk = rowblk + 2048 * (t >> 5);
                reinterpret_cast<__bf16*>(blk)[e] = zh;
                reinterpret_cast<__bf16*>(blk + 1024)[e] = zl;
            }
        }
    }
    __syncthreads();

    // ---- (5) dense part for this wavefront's 16 value columns
    bf16x8 s0h[KS], s0l[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        const float4 x0 = s0r[2 * ks], x1 = s0r[2 * ks + 1];
        const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        split8(x, s0h[ks], s0l[ks]);
    }

    // R' = V - gamma o (K S0^T) as B fragments of the Z~ R' product: k-step
    // kap covers nodes [32 kap, 32 kap + 32); lane (lc, lg) holds rows
    // 32 kap + 16 half + 4 lg + rr in slot 4 half + rr.
    bf16x8 rh[NKMAX], rl[NKMAX];
#pragma unroll
    for (int kap = 0; kap < NKMAX; ++kap) {
        float rt[8];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            const int S = 2 * kap + half;
            if (S < NT) {
                f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    const bf16x8 ka = k_frag(16 * S + lc, ks);
                    acc = mfma(ka, s0h[ks], acc);
                    acc = mfma(ka, s0l[ks], acc);
                }
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int srow = 16 * S + 4 * lg + rr;
                    const float vv = srow < N ? to_f32(vraw[S][rr]) : 0.f;
                    rt[4 * half + rr] = vv - gam[srow] * acc[rr];
                }
            } else {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) rt[4 * half + rr] = 0.f;
            }
        }
        split8(rt, rh[kap], rl[kap]);
    }

    // O tiles: gamma o (Q S0^T) + Z~ R'
    for (int I = 0; I < NT; ++I) {
        const int irow = 16 * I + lc;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 qa = q_frag(irow, ks);
            acc = mfma(qa, s0h[ks], acc);
            acc = mfma(qa, s0l[ks], acc);
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) acc[rr] *= gam[16 * I + 4 * lg + rr];
        if (DENSE) {
            const unsigned char* rowblk = Zd + 2048 * zblocks_before(I) + 16 * lane;
#pragma unroll
            for (int kap = 0; kap < NKMAX; ++kap) {
                if (2 * kap <= I) {
                    const bf16x8 zh = load_frag(rowblk + 2048 * kap);
                    const bf16x8 zl = load_frag(rowblk + 2048 * kap + 1024);
                    acc = mfma(zh, rh[kap], acc);
                    acc = mfma(zh, rl[kap], acc);
                    acc = mfma(zl, rh[kap], acc);
                }
            }
        } else {
            // this lane's row of Z~, scanned once in node order
            int p = 0, pend = 0;
            if (irow < N) {
                p = off[irow];
                pend = p + dep[irow];
            }
#pragma unroll
            for (int kap = 0; kap < NKMAX; ++kap) {
                if (2 * kap > I) continue;
                float f[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) f[j] = 0.f;
                while (p < pend) {
                    const int t = pathc[p];
                    if (t >= 32 * kap + 32) break;
                    const int dt = t - 32 * kap;
                    if (((dt >> 2) & 3) == lg) {
                        const int slot = ((dt >> 4) << 2) | (dt & 3);
                        const float z = zc[p];
#pragma unroll
                        for (int j = 0; j < 8; ++j) f[j] = slot == j ? z : f[j];
                    }
                    ++p;
                }
                bf16x8 zh, zl;
                split8(f, zh, zl);
                acc = mfma(zh, rh[kap], acc);
                acc = mfma(zh, rl[kap], acc);
                acc = mfma(zl, rh[kap], acc);
            }
        }
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int i = 16 * I + 4 * lg + rr;
            if (i < N) a.o[(static_cast<size_t>(b) * N + i) * Hv * DV + static_cast<size_t>(h) * DV + col] = acc[rr];
        }
    }
}

template <int NMAX, int DK, int DV>
hipError_t verify_fast(const VerifyArgs& a, hipStream_t stream) {
    const int R = a.H_v / a.H_k;
    const int groups = a.B * a.H_k;
    const dim3 grid(static_cast<unsigned>(8 * R) * static_cast<unsigned>((groups + 7) / 8));
    hipLaunchKernelGGL((verify_fast_kernel<NMAX, DK, DV>), grid, dim3(64 * (DV / 16)), 0, stream, a);
    return hipGetLastError();
}

template <int DK, int DV>
hipError_t verify_fast_n(const VerifyArgs& a, hipStream_t stream) {
    if (a.N <= 64) return verify_fast<64, DK, DV>(a, stream);
    if (a.N <= 128) return verify_fast<128, DK, DV>(a, stream);
    return verify_fast<256, DK, DV>(a, stream);
}

}  // namespace

hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream) {
    if (a.qkv_dtype != GDN_BF16 || a.force_walk) return launch_verify_simple(a, stream);
    if (a.d_k == 128) return a.d_v == 128 ? verify_fast_n<128, 128>(a, stream) : verify_fast_n<128, 64>(a, stream);
    return a.d_v == 128 ? verify_fast_n<64, 128>(a, stream) : verify_fast_n<64, 64>(a, stream);
}

}  // namespace gdn
