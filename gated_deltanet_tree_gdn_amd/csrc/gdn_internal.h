// gdn_internal.h -- host-side launch interface shared by the C-ABI layer and
// the kernel translation units of the GDN tree-verification library.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <string>

#include "gdn_tree.h"

namespace gdn {

constexpr int kMaxN = 256;  // largest tree the kernels accept

// Arguments of one tree verification (all device pointers, layouts as in
// gdn_tree.h).
struct VerifyArgs {
    int B, N, H_k, H_v, d_k, d_v;
    int qkv_dtype;
    const void* q;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* parent;
    const float* S0;
    float* o;
    int32_t* tree_status;  // [B]: 0 or GDN_ERR_TREE
    int force_walk;        // 1: per-node walk even for bf16 (GDN_FORCE_SIMPLE=1)
    void* split_ws;        // split_ws_bytes(B, N, H_v) bytes of device workspace for the
                           // two-launch verify of N > 128, or NULL (single-launch kernels)
};

// The two-launch verify's workspace (gdn_split.hip): per (sequence, value
// head) the pair values of Z~ and gamma, per sequence the pair structure.
struct SplitWs {
    float* z;        // [B][H_v][P]
    float* gam;      // [B][H_v][N]
    uint16_t* zoff;  // [B][P]: byte offset of each pair's Z~ entry in its output tile's blocks
    int32_t* off;    // [B][N + 1]: first pair of each node, then the count
    int32_t* deep;   // [B]: 1 for a root path the tree kernel does not solve
    int P;           // pair capacity per sequence
};
// Byte offsets of the arrays in the workspace (each 256-aligned); pairs per
// sequence at most N ZR, ZR the longest root path the tree kernel solves.
struct SplitLayout {
    size_t z, gam, zoff, off, deep, total;
    int P;
};
inline int split_zr(int N) { return N > 128 ? 24 : 16; }
inline SplitLayout split_layout(int B, int N, int Hv) {
    auto r256 = [](size_t x) { return (x + 255) & ~size_t(255); };
    SplitLayout l{};
    l.P = (N > 0 ? N : 1) * split_zr(N);
    const size_t b = B > 0 ? B : 1, n = N > 0 ? N : 1, h = Hv > 0 ? Hv : 1;
    l.z = 0;
    l.gam = l.z + r256(b * h * l.P * sizeof(float));
    l.zoff = l.gam + r256(b * h * n * sizeof(float));
    l.off = l.zoff + r256(b * l.P * sizeof(uint16_t));
    l.deep = l.off + r256(b * (n + 1) * sizeof(int32_t));
    l.total = l.deep + r256(b * sizeof(int32_t));
    return l;
}
// Zero for trees of at most 128 nodes, which the single-launch kernel verifies.
inline size_t split_ws_bytes(int B, int N, int Hv) { return N > 128 ? split_layout(B, N, Hv).total : 0; }
inline SplitWs split_ws_at(void* base, int B, int N, int Hv) {
    const SplitLayout l = split_layout(B, N, Hv);
    unsigned char* p = static_cast<unsigned char*>(base);
    SplitWs w;
    w.z = reinterpret_cast<float*>(p + l.z);
    w.gam = reinterpret_cast<float*>(p + l.gam);
    w.zoff = reinterpret_cast<uint16_t*>(p + l.zoff);
    w.off = reinterpret_cast<int32_t*>(p + l.off);
    w.deep = reinterpret_cast<int32_t*>(p + l.deep);
    w.P = l.P;
    return w;
}

// Arguments of one accepted-path commit.
struct CommitArgs {
    int B, N, H_k, H_v, d_k, d_v;
    int qkv_dtype;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* parent;
    const float* S0;
    const int32_t* accepted;
    float* S_new;
    int32_t* accept_status;  // [B]: 0 or GDN_ERR_ACCEPT
    int force_walk;          // 1: per-node path walk even for bf16 (GDN_FORCE_SIMPLE=1)
};

// The previous tree of a fused commit-then-verify: its inputs (same B, N and
// heads as the tree being verified), the state it started from, the
// accepted node per sequence, and where the committed state goes (the
// verify's S0).
struct CommitPrev {
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* parent;
    const float* S0;
    const int32_t* accepted;
    float* S_next;
    int32_t* accept_status;  // [B]: 0 or GDN_ERR_ACCEPT
};

// Verify dispatch: the MFMA path for bf16 q/k/v, the per-node walk otherwise.
hipError_t launch_verify(const VerifyArgs& a, hipStream_t stream);
// The MFMA verify for bf16 and N <= 128.
hipError_t launch_verify_ws(const VerifyArgs& a, hipStream_t stream);
// The two-launch MFMA verify (tree kernel, then dense kernel) for bf16 and
// 128 < N <= 256 over a.split_ws.
hipError_t launch_verify_split(const VerifyArgs& a, hipStream_t stream);
// The commit of the previous tree's accepted path into c.S_next (== a.S0)
// fused into the verify of the tree in `a` (bf16, N <= 128).
hipError_t launch_commit_verify(const VerifyArgs& a, const CommitPrev& c, hipStream_t stream);
// Per-branch recurrent verification (the comparison baseline).
hipError_t launch_verify_branches(const VerifyArgs& a, hipStream_t stream);
// Sets the calling thread's detail message (gdn_last_error).
void set_last_error(const std::string& msg);
// Compute units of the current device (cached per device).
int device_cus();
// The per-node walk for every batch element (any dtype).
hipError_t launch_verify_simple(const VerifyArgs& a, hipStream_t stream);
// Commit dispatch: the MFMA chunked path for bf16 k/v, the per-node walk otherwise.
hipError_t launch_commit(const CommitArgs& a, hipStream_t stream);
hipError_t launch_commit_simple(const CommitArgs& a, hipStream_t stream);
hipError_t launch_ancestors(int B, int N, const int32_t* parent, uint32_t* anc, int32_t* depth,
                            int32_t* tree_status, hipStream_t stream);
// Greedy accepted-node selection, one wavefront per sequence.
hipError_t launch_accept(int B, int N, const int32_t* parent, const int32_t* draft, const int32_t* target,
                         int32_t* accepted, int32_t* accept_len, int32_t* tree_status, hipStream_t stream);
// Top-w best-first tree construction, one wavefront per sequence (C <= kMaxCand).
constexpr int kMaxCand = 32;
hipError_t launch_build(int B, int N, int C, int w, int max_depth, const float* root_logp, const float* node_logp,
                        int32_t* parent, int32_t* cand_rank, float* score, int32_t* steps, int32_t* build_status,
                        hipStream_t stream);

}  // namespace gdn
