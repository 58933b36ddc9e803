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
};

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
