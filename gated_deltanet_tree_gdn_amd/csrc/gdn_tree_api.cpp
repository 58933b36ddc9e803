// gdn_tree_api.cpp -- the C ABI declared in include/gdn_tree.h.
//
// Host-side only: O(1) argument checks (made before any HIP call, so they
// are testable without a GPU), the context that ties a verify to its delayed
// commit, and dispatch to the kernel launchers.  No allocation and no
// synchronisation happen on the verify/commit path.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "gdn_internal.h"
#include "gdn_tree.h"

struct gdn_ctx {
    gdn_tree_dims dims;
    int32_t* status;  // device: [B] tree verdicts, then [B] accept verdicts
    void* split;      // device: the two-launch verify's workspace (after the verdicts)
    bool validate;    // GDN_VALIDATE=1: synchronous host checks of parent/accepted
    bool force_walk;  // GDN_FORCE_SIMPLE=1: per-node walk kernels only
    bool have_verify;
    bool have_commit;
    const void* k;
    const void* v;
    const float* g;
    const float* beta;
    const int32_t* parent;
    const float* S0;
};

namespace {

thread_local std::string g_last_error;

gdn_status fail(gdn_status s, const std::string& msg) {
    g_last_error = msg;
    return s;
}

gdn_status ok() {
    g_last_error.clear();
    return GDN_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

gdn_status check_dims(const gdn_tree_dims* d) {
    if (!d) return fail(GDN_ERR_NULL, "dims is NULL");
    if (d->qkv_dtype != GDN_BF16 && d->qkv_dtype != GDN_F32)
        return fail(GDN_ERR_DTYPE, "qkv_dtype must be GDN_BF16 or GDN_F32");
    if (d->B < 0) return fail(GDN_ERR_SHAPE, "B must be >= 0");
    if (d->N < 0 || d->N > gdn::kMaxN) return fail(GDN_ERR_SHAPE, "N must be in [0, 256]");
    if (d->H_k < 1 || d->H_v < 1) return fail(GDN_ERR_SHAPE, "H_k and H_v must be >= 1");
    if (d->H_v % d->H_k != 0) return fail(GDN_ERR_SHAPE, "H_v must be a multiple of H_k");
    if ((d->d_k != 64 && d->d_k != 128) || (d->d_v != 64 && d->d_v != 128))
        return fail(GDN_ERR_SHAPE, "d_k and d_v must be 64 or 128");
    return GDN_OK;
}

gdn_status check_ptr(const void* p, const char* name) {
    if (!p) return fail(GDN_ERR_NULL, std::string(name) + " is NULL");
    if (!aligned16(p)) return fail(GDN_ERR_ALIGN, std::string(name) + " is not 16-byte aligned");
    return GDN_OK;
}

#define GDN_TRY(expr)                       \
    do {                                    \
        gdn_status _s = (expr);             \
        if (_s != GDN_OK) return _s;        \
    } while (0)

gdn_status hip_fail(hipError_t e, const char* what) {
    return fail(GDN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

// GDN_VALIDATE=1: copy parent[] back and check it on the host (synchronous).
gdn_status host_check_tree(const gdn_tree_dims& d, const int32_t* parent, hipStream_t stream) {
    std::vector<int32_t> h(static_cast<size_t>(d.B) * d.N);
    hipError_t e = hipMemcpyAsync(h.data(), parent, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "GDN_VALIDATE copy of parent");
    for (int b = 0; b < d.B; ++b)
        for (int i = 0; i < d.N; ++i) {
            int p = h[static_cast<size_t>(b) * d.N + i];
            if (p < -1 || p >= i) {
                char msg[128];
                std::snprintf(msg, sizeof msg, "parent[%d][%d] = %d is outside [-1, %d]", b, i, p, i - 1);
                return fail(GDN_ERR_TREE, msg);
            }
        }
    return GDN_OK;
}

gdn_status host_check_accepted(const gdn_tree_dims& d, const int32_t* accepted, hipStream_t stream) {
    std::vector<int32_t> h(static_cast<size_t>(d.B));
    hipError_t e = hipMemcpyAsync(h.data(), accepted, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "GDN_VALIDATE copy of accepted");
    for (int b = 0; b < d.B; ++b)
        if (h[b] < -1 || h[b] >= d.N) {
            char msg[128];
            std::snprintf(msg, sizeof msg, "accepted[%d] = %d is outside [-1, %d]", b, h[b], d.N - 1);
            return fail(GDN_ERR_ACCEPT, msg);
        }
    return GDN_OK;
}

}  // namespace

namespace gdn {
void set_last_error(const std::string& msg) { g_last_error = msg; }
}  // namespace gdn

extern "C" {

namespace {
size_t status_bytes(const gdn_tree_dims* dims) {
    return round256(2 * static_cast<size_t>(dims->B > 0 ? dims->B : 1) * sizeof(int32_t));
}
}  // namespace

size_t gdn_tree_workspace_bytes(const gdn_tree_dims* dims) {
    if (!dims || dims->B < 0) return 0;
    return status_bytes(dims) + gdn::split_ws_bytes(dims->B, dims->N, dims->H_v);
}

gdn_status gdn_ctx_create(const gdn_tree_dims* dims, void* workspace, size_t workspace_bytes,
                          gdn_ctx** out) {
    if (!out) return fail(GDN_ERR_NULL, "out is NULL");
    *out = nullptr;
    GDN_TRY(check_dims(dims));
    if (!workspace) return fail(GDN_ERR_WORKSPACE, "workspace is NULL");
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(GDN_ERR_ALIGN, "workspace is not 256-byte aligned");
    if (workspace_bytes < gdn_tree_workspace_bytes(dims))
        return fail(GDN_ERR_WORKSPACE, "workspace smaller than gdn_tree_workspace_bytes(dims)");
    gdn_ctx* c = new (std::nothrow) gdn_ctx();
    if (!c) return fail(GDN_ERR_WORKSPACE, "out of host memory");
    c->dims = *dims;
    c->status = static_cast<int32_t*>(workspace);
    c->split = gdn::split_ws_bytes(dims->B, dims->N, dims->H_v) > 0
                   ? static_cast<unsigned char*>(workspace) + status_bytes(dims)
                   : nullptr;
    const char* env = std::getenv("GDN_VALIDATE");
    c->validate = env && std::strcmp(env, "1") == 0;
    const char* fw = std::getenv("GDN_FORCE_SIMPLE");
    c->force_walk = fw && std::strcmp(fw, "1") == 0;
    *out = c;
    return ok();
}

gdn_status gdn_ctx_destroy(gdn_ctx* ctx) {
    delete ctx;
    return ok();
}

namespace {

// Shared by both verify entry points: argument checks, the launch, and the
// record of borrowed inputs for the delayed commit.
gdn_status verify_with(hipError_t (*launch)(const gdn::VerifyArgs&, hipStream_t), const char* what, gdn_ctx* ctx,
                       const void* q, const void* k, const void* v, const float* g, const float* beta,
                       const int32_t* parent, const float* S0, float* o, hipStream_t stream) {
    if (!ctx) return fail(GDN_ERR_NULL, "ctx is NULL");
    const gdn_tree_dims d = ctx->dims;
    ctx->have_verify = false;
    ctx->have_commit = false;
    if (d.B == 0 || d.N == 0) {
        ctx->have_verify = true;
        ctx->k = k; ctx->v = v; ctx->g = g; ctx->beta = beta; ctx->parent = parent; ctx->S0 = S0;
        return ok();
    }
    GDN_TRY(check_ptr(q, "q"));
    GDN_TRY(check_ptr(k, "k"));
    GDN_TRY(check_ptr(v, "v"));
    GDN_TRY(check_ptr(g, "g"));
    GDN_TRY(check_ptr(beta, "beta"));
    GDN_TRY(check_ptr(parent, "parent"));
    GDN_TRY(check_ptr(S0, "S0"));
    GDN_TRY(check_ptr(o, "o"));
    if (ctx->validate) GDN_TRY(host_check_tree(d, parent, stream));
    gdn::VerifyArgs a{d.B, d.N, d.H_k, d.H_v, d.d_k, d.d_v, d.qkv_dtype, q, k, v, g, beta, parent, S0, o,
                      ctx->status, ctx->force_walk ? 1 : 0, ctx->split};
    hipError_t e = launch(a, stream);
    if (e != hipSuccess) return hip_fail(e, what);
    ctx->have_verify = true;
    ctx->k = k; ctx->v = v; ctx->g = g; ctx->beta = beta; ctx->parent = parent; ctx->S0 = S0;
    return ok();
}

}  // namespace

gdn_status gdn_tree_verify(gdn_ctx* ctx, const void* q, const void* k, const void* v, const float* g,
                           const float* beta, const int32_t* parent, const float* S0, float* o,
                           hipStream_t stream) {
    return verify_with(gdn::launch_verify, "verify launch", ctx, q, k, v, g, beta, parent, S0, o, stream);
}

gdn_status gdn_tree_verify_branches(gdn_ctx* ctx, const void* q, const void* k, const void* v, const float* g,
                                    const float* beta, const int32_t* parent, const float* S0, float* o,
                                    hipStream_t stream) {
    return verify_with(gdn::launch_verify_branches, "per-branch verify launch", ctx, q, k, v, g, beta, parent,
                       S0, o, stream);
}

gdn_status gdn_commit_path(gdn_ctx* ctx, const int32_t* accepted, float* S_new, hipStream_t stream) {
    if (!ctx) return fail(GDN_ERR_NULL, "ctx is NULL");
    if (!ctx->have_verify) return fail(GDN_ERR_STATE, "gdn_commit_path without a prior gdn_tree_verify");
    const gdn_tree_dims d = ctx->dims;
    ctx->have_commit = false;
    if (d.B == 0) return ok();
    GDN_TRY(check_ptr(accepted, "accepted"));
    GDN_TRY(check_ptr(S_new, "S_new"));
    if (d.N == 0) {
        // every accepted node must be -1: S_new = S0
        GDN_TRY(check_ptr(ctx->S0, "S0"));
    }
    if (ctx->validate) GDN_TRY(host_check_accepted(d, accepted, stream));
    gdn::CommitArgs a{d.B, d.N, d.H_k, d.H_v, d.d_k, d.d_v, d.qkv_dtype, ctx->k, ctx->v, ctx->g, ctx->beta,
                      ctx->parent, ctx->S0, accepted, S_new, ctx->status + d.B, ctx->force_walk ? 1 : 0};
    hipError_t e = gdn::launch_commit(a, stream);
    if (e != hipSuccess) return hip_fail(e, "commit launch");
    ctx->have_commit = true;
    return ok();
}

gdn_status gdn_commit_verify(gdn_ctx* ctx, const int32_t* accepted, const void* q, const void* k, const void* v,
                             const float* g, const float* beta, const int32_t* parent, float* S_next, float* o,
                             hipStream_t stream) {
    if (!ctx) return fail(GDN_ERR_NULL, "ctx is NULL");
    if (!ctx->have_verify) return fail(GDN_ERR_STATE, "gdn_commit_verify without a prior gdn_tree_verify");
    const gdn_tree_dims d = ctx->dims;
    auto record = [&]() {
        ctx->have_verify = true;
        ctx->have_commit = d.B > 0;
        ctx->k = k; ctx->v = v; ctx->g = g; ctx->beta = beta; ctx->parent = parent; ctx->S0 = S_next;
    };
    if (d.B == 0) {
        record();
        return ok();
    }
    GDN_TRY(check_ptr(accepted, "accepted"));
    GDN_TRY(check_ptr(S_next, "S_next"));
    GDN_TRY(check_ptr(ctx->S0, "S0 of the recorded verify"));
    if (d.N > 0) {
        GDN_TRY(check_ptr(q, "q"));
        GDN_TRY(check_ptr(k, "k"));
        GDN_TRY(check_ptr(v, "v"));
        GDN_TRY(check_ptr(g, "g"));
        GDN_TRY(check_ptr(beta, "beta"));
        GDN_TRY(check_ptr(parent, "parent"));
        GDN_TRY(check_ptr(o, "o"));
    }
    if (ctx->validate) {
        GDN_TRY(host_check_accepted(d, accepted, stream));
        if (d.N > 0) GDN_TRY(host_check_tree(d, parent, stream));
    }
    gdn::CommitArgs ca{d.B, d.N, d.H_k, d.H_v, d.d_k, d.d_v, d.qkv_dtype, ctx->k, ctx->v, ctx->g, ctx->beta,
                       ctx->parent, ctx->S0, accepted, S_next, ctx->status + d.B, ctx->force_walk ? 1 : 0};
    hipError_t e = hipSuccess;
    if (d.N == 0) {
        e = gdn::launch_commit(ca, stream);
    } else {
        gdn::VerifyArgs va{d.B, d.N, d.H_k, d.H_v, d.d_k, d.d_v, d.qkv_dtype, q, k, v, g, beta, parent, S_next, o,
                           ctx->status, ctx->force_walk ? 1 : 0, ctx->split};
        if (d.qkv_dtype == GDN_BF16 && d.N <= 128 && !ctx->force_walk) {
            gdn::CommitPrev cp{ctx->k, ctx->v, ctx->g, ctx->beta, ctx->parent, ctx->S0, accepted, S_next,
                               ctx->status + d.B};
            e = gdn::launch_commit_verify(va, cp, stream);
        } else {
            e = gdn::launch_commit(ca, stream);
            if (e == hipSuccess) e = gdn::launch_verify(va, stream);
        }
    }
    if (e != hipSuccess) {
        ctx->have_verify = false;
        ctx->have_commit = false;
        return hip_fail(e, "commit-verify launch");
    }
    record();
    return ok();
}

gdn_status gdn_tree_ancestors(const gdn_tree_dims* dims, const int32_t* parent, uint32_t* anc,
                              int32_t* depth, int32_t* tree_status, hipStream_t stream) {
    if (!dims) return fail(GDN_ERR_NULL, "dims is NULL");
    if (dims->B < 0) return fail(GDN_ERR_SHAPE, "B must be >= 0");
    if (dims->N < 0 || dims->N > gdn::kMaxN) return fail(GDN_ERR_SHAPE, "N must be in [0, 256]");
    if (dims->B == 0 || dims->N == 0) return ok();
    GDN_TRY(check_ptr(parent, "parent"));
    GDN_TRY(check_ptr(anc, "anc"));
    GDN_TRY(check_ptr(depth, "depth"));
    if (tree_status && !aligned16(tree_status)) return fail(GDN_ERR_ALIGN, "tree_status is not 16-byte aligned");
    hipError_t e = gdn::launch_ancestors(dims->B, dims->N, parent, anc, depth, tree_status, stream);
    if (e != hipSuccess) return hip_fail(e, "ancestors launch");
    return ok();
}

gdn_status gdn_accept_path(const gdn_tree_dims* dims, const int32_t* parent, const int32_t* draft_token,
                           const int32_t* target_token, int32_t* accepted, int32_t* accept_len,
                           int32_t* tree_status, hipStream_t stream) {
    if (!dims) return fail(GDN_ERR_NULL, "dims is NULL");
    if (dims->B < 0) return fail(GDN_ERR_SHAPE, "B must be >= 0");
    if (dims->N < 0 || dims->N > gdn::kMaxN) return fail(GDN_ERR_SHAPE, "N must be in [0, 256]");
    if (dims->B == 0) return ok();
    GDN_TRY(check_ptr(accepted, "accepted"));
    GDN_TRY(check_ptr(target_token, "target_token"));
    if (dims->N > 0) {
        GDN_TRY(check_ptr(parent, "parent"));
        GDN_TRY(check_ptr(draft_token, "draft_token"));
    }
    if (accept_len && !aligned16(accept_len)) return fail(GDN_ERR_ALIGN, "accept_len is not 16-byte aligned");
    if (tree_status && !aligned16(tree_status)) return fail(GDN_ERR_ALIGN, "tree_status is not 16-byte aligned");
    hipError_t e = gdn::launch_accept(dims->B, dims->N, parent, draft_token, target_token, accepted, accept_len,
                                      tree_status, stream);
    if (e != hipSuccess) return hip_fail(e, "accept launch");
    return ok();
}

gdn_status gdn_tree_build(const gdn_tree_dims* dims, int32_t n_cand, int32_t w, int32_t max_depth,
                          const float* root_logp, const float* node_logp, int32_t* parent, int32_t* cand_rank,
                          float* score, int32_t* steps, int32_t* build_status, hipStream_t stream) {
    if (!dims) return fail(GDN_ERR_NULL, "dims is NULL");
    if (dims->B < 0) return fail(GDN_ERR_SHAPE, "B must be >= 0");
    if (dims->N < 0 || dims->N > gdn::kMaxN) return fail(GDN_ERR_SHAPE, "N must be in [0, 256]");
    if (n_cand < 1 || n_cand > gdn::kMaxCand) return fail(GDN_ERR_SHAPE, "n_cand must be in [1, 32]");
    if (w < 1) return fail(GDN_ERR_SHAPE, "w must be >= 1");
    if (max_depth < 1) return fail(GDN_ERR_SHAPE, "max_depth must be >= 1");
    if (dims->B == 0 || dims->N == 0) return ok();
    GDN_TRY(check_ptr(root_logp, "root_logp"));
    GDN_TRY(check_ptr(node_logp, "node_logp"));
    GDN_TRY(check_ptr(parent, "parent"));
    if (cand_rank && !aligned16(cand_rank)) return fail(GDN_ERR_ALIGN, "cand_rank is not 16-byte aligned");
    if (score && !aligned16(score)) return fail(GDN_ERR_ALIGN, "score is not 16-byte aligned");
    if (steps && !aligned16(steps)) return fail(GDN_ERR_ALIGN, "steps is not 16-byte aligned");
    if (build_status && !aligned16(build_status)) return fail(GDN_ERR_ALIGN, "build_status is not 16-byte aligned");
    hipError_t e = gdn::launch_build(dims->B, dims->N, n_cand, w, max_depth, root_logp, node_logp, parent,
                                     cand_rank, score, steps, build_status, stream);
    if (e != hipSuccess) return hip_fail(e, "tree-build launch");
    return ok();
}

gdn_status gdn_ctx_status(gdn_ctx* ctx, hipStream_t stream) {
    if (!ctx) return fail(GDN_ERR_NULL, "ctx is NULL");
    const int B = ctx->dims.B;
    if (B == 0 || ctx->dims.N == 0 || (!ctx->have_verify && !ctx->have_commit)) {
        hipError_t e = hipStreamSynchronize(stream);
        if (e != hipSuccess) return hip_fail(e, "stream synchronise");
        return ok();
    }
    std::vector<int32_t> h(2 * static_cast<size_t>(B));
    hipError_t e = hipMemcpyAsync(h.data(), ctx->status, h.size() * sizeof(int32_t), hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipStreamSynchronize(stream);
    if (e != hipSuccess) return hip_fail(e, "status copy");
    if (ctx->have_verify)
        for (int b = 0; b < B; ++b)
            if (h[b] == GDN_ERR_HIP) {
                char msg[96];
                std::snprintf(msg, sizeof msg, "sequence %d: a wait inside the verify kernel timed out", b);
                return fail(GDN_ERR_HIP, msg);
            }
    if (ctx->have_verify)
        for (int b = 0; b < B; ++b)
            if (h[b] != 0) {
                char msg[96];
                std::snprintf(msg, sizeof msg, "sequence %d: parent array is not a topological tree", b);
                return fail(GDN_ERR_TREE, msg);
            }
    if (ctx->have_commit)
        for (int b = 0; b < B; ++b)
            if (h[B + b] != 0) {
                char msg[96];
                std::snprintf(msg, sizeof msg, "sequence %d: accepted node out of range", b);
                return fail(GDN_ERR_ACCEPT, msg);
            }
    return ok();
}

const char* gdn_status_string(gdn_status s) {
    switch (s) {
        case GDN_OK: return "GDN_OK";
        case GDN_ERR_NULL: return "GDN_ERR_NULL";
        case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE";
        case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE";
        case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN";
        case GDN_ERR_WORKSPACE: return "GDN_ERR_WORKSPACE";
        case GDN_ERR_TREE: return "GDN_ERR_TREE";
        case GDN_ERR_ACCEPT: return "GDN_ERR_ACCEPT";
        case GDN_ERR_STATE: return "GDN_ERR_STATE";
        case GDN_ERR_HIP: return "GDN_ERR_HIP";
    }
    return "GDN_ERR_UNKNOWN";
}

const char* gdn_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
