// abi_driver.cpp -- drives every host-side path of the C ABI (argument
// checks, the context, GDN_VALIDATE host checks, status read-back) against
// the stand-ins of host_stubs.cpp, under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Exit status 0 when every check holds.

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "gdn_tree.h"
#include "host_stubs.h"

static int g_fail = 0;

#define CHECK(cond)                                                                 \
    do {                                                                            \
        if (!(cond)) {                                                              \
            std::fprintf(stderr, "%s:%d: check failed: %s\n", __FILE__, __LINE__, #cond); \
            ++g_fail;                                                               \
        }                                                                           \
    } while (0)

// "device" memory: 256-byte aligned host memory of exactly the asked size
// (rounded up to the alignment), so a read or write past it is caught
static void* dev_alloc(size_t bytes) {
    size_t n = (bytes + 255) / 256 * 256;
    void* p = std::aligned_alloc(256, n ? n : 256);
    std::memset(p, 0, n ? n : 256);
    return p;
}

struct Tensors {
    void *q, *k, *v;
    float *g, *beta, *S0, *o, *S_new;
    int32_t *parent, *accepted;
    explicit Tensors(const gdn_tree_dims& d) {
        const size_t e = d.qkv_dtype == GDN_BF16 ? 2 : 4;
        const size_t B = d.B, N = d.N;
        q = dev_alloc(B * N * d.H_k * d.d_k * e);
        k = dev_alloc(B * N * d.H_k * d.d_k * e);
        v = dev_alloc(B * N * d.H_v * d.d_v * e);
        g = static_cast<float*>(dev_alloc(B * N * d.H_v * 4));
        beta = static_cast<float*>(dev_alloc(B * N * d.H_v * 4));
        S0 = static_cast<float*>(dev_alloc(B * d.H_v * d.d_v * d.d_k * 4));
        o = static_cast<float*>(dev_alloc(B * N * d.H_v * d.d_v * 4));
        S_new = static_cast<float*>(dev_alloc(B * d.H_v * d.d_v * d.d_k * 4));
        parent = static_cast<int32_t*>(dev_alloc(B * N * 4));
        accepted = static_cast<int32_t*>(dev_alloc(B * 4));
        for (size_t b = 0; b < B; ++b)
            for (size_t i = 0; i < N; ++i) parent[b * N + i] = static_cast<int32_t>(i) - 1;  // chains
    }
    ~Tensors() {
        for (void* p : {q, k, v, static_cast<void*>(g), static_cast<void*>(beta), static_cast<void*>(S0),
                        static_cast<void*>(o), static_cast<void*>(S_new), static_cast<void*>(parent),
                        static_cast<void*>(accepted)})
            std::free(p);
    }
};

static gdn_status verify(gdn_ctx* c, const Tensors& t) {
    return gdn_tree_verify(c, t.q, t.k, t.v, t.g, t.beta, t.parent, t.S0, t.o, nullptr);
}

int main() {
    const gdn_tree_dims d{3, 40, 2, 4, 128, 64, GDN_BF16};
    Tensors t(d);

    // workspace sizing
    CHECK(gdn_tree_workspace_bytes(nullptr) == 0);
    const size_t ws = gdn_tree_workspace_bytes(&d);
    CHECK(ws % 256 == 0 && ws >= 2 * sizeof(int32_t) * d.B);
    void* work = dev_alloc(ws);

    // context creation: every argument error
    gdn_ctx* c = nullptr;
    CHECK(gdn_ctx_create(&d, work, ws, nullptr) == GDN_ERR_NULL);
    CHECK(gdn_ctx_create(nullptr, work, ws, &c) == GDN_ERR_NULL && c == nullptr);
    gdn_tree_dims bad = d;
    bad.qkv_dtype = 7;
    CHECK(gdn_ctx_create(&bad, work, ws, &c) == GDN_ERR_DTYPE);
    bad = d; bad.B = -1;
    CHECK(gdn_ctx_create(&bad, work, ws, &c) == GDN_ERR_SHAPE);
    bad = d; bad.N = 257;
    CHECK(gdn_ctx_create(&bad, work, ws, &c) == GDN_ERR_SHAPE);
    bad = d; bad.H_v = 5;
    CHECK(gdn_ctx_create(&bad, work, ws, &c) == GDN_ERR_SHAPE);
    bad = d; bad.d_k = 96;
    CHECK(gdn_ctx_create(&bad, work, ws, &c) == GDN_ERR_SHAPE);
    CHECK(gdn_ctx_create(&d, nullptr, ws, &c) == GDN_ERR_WORKSPACE);
    CHECK(gdn_ctx_create(&d, static_cast<char*>(work) + 16, ws, &c) == GDN_ERR_ALIGN);
    CHECK(gdn_ctx_create(&d, work, ws - 1, &c) == GDN_ERR_WORKSPACE);
    CHECK(std::strlen(gdn_last_error()) > 0);
    CHECK(gdn_ctx_create(&d, work, ws, &c) == GDN_OK && c != nullptr);
    CHECK(std::strlen(gdn_last_error()) == 0);

    // commit before any verify; verify argument errors (no launch happens)
    CHECK(gdn_commit_path(c, t.accepted, t.S_new, nullptr) == GDN_ERR_STATE);
    CHECK(gdn_tree_verify(nullptr, t.q, t.k, t.v, t.g, t.beta, t.parent, t.S0, t.o, nullptr) == GDN_ERR_NULL);
    CHECK(gdn_tree_verify(c, nullptr, t.k, t.v, t.g, t.beta, t.parent, t.S0, t.o, nullptr) == GDN_ERR_NULL);
    CHECK(gdn_tree_verify(c, t.q, static_cast<char*>(t.k) + 2, t.v, t.g, t.beta, t.parent, t.S0, t.o, nullptr) ==
          GDN_ERR_ALIGN);
    CHECK(gdn_tree_verify(c, t.q, t.k, t.v, t.g, t.beta, t.parent, t.S0, nullptr, nullptr) == GDN_ERR_NULL);
    CHECK(g_stub.verifies == 0);
    CHECK(gdn_commit_path(c, t.accepted, t.S_new, nullptr) == GDN_ERR_STATE);  // failed verify records nothing

    // a verify launches with the caller's pointers and records them for the commit
    CHECK(verify(c, t) == GDN_OK && g_stub.verifies == 1);
    CHECK(g_stub.last_verify.q == t.q && g_stub.last_verify.o == t.o && g_stub.last_verify.N == d.N);
    CHECK(gdn_commit_path(c, nullptr, t.S_new, nullptr) == GDN_ERR_NULL);
    CHECK(gdn_commit_path(c, t.accepted, t.S_new, nullptr) == GDN_OK && g_stub.commits == 1);
    CHECK(g_stub.last_commit.S0 == t.S0 && g_stub.last_commit.k == t.k && g_stub.last_commit.S_new == t.S_new);
    CHECK(g_stub.last_commit.accept_status == g_stub.last_verify.tree_status + d.B);

    // device verdicts read back by gdn_ctx_status
    CHECK(gdn_ctx_status(nullptr, nullptr) == GDN_ERR_NULL);
    CHECK(gdn_ctx_status(c, nullptr) == GDN_OK);
    g_stub.verify_verdict = GDN_ERR_TREE;
    CHECK(verify(c, t) == GDN_OK);
    CHECK(gdn_ctx_status(c, nullptr) == GDN_ERR_TREE);
    g_stub.verify_verdict = GDN_ERR_HIP;
    CHECK(verify(c, t) == GDN_OK);
    CHECK(gdn_ctx_status(c, nullptr) == GDN_ERR_HIP);
    g_stub.verify_verdict = 0;
    CHECK(verify(c, t) == GDN_OK);
    g_stub.commit_verdict = GDN_ERR_ACCEPT;
    CHECK(gdn_commit_path(c, t.accepted, t.S_new, nullptr) == GDN_OK);
    CHECK(gdn_ctx_status(c, nullptr) == GDN_ERR_ACCEPT);
    g_stub.commit_verdict = 0;

    // a failing launch is GDN_ERR_HIP
    g_stub.launch_error = hipErrorInvalidValue;
    CHECK(verify(c, t) == GDN_ERR_HIP);
    CHECK(gdn_commit_path(c, t.accepted, t.S_new, nullptr) == GDN_ERR_STATE);
    g_stub.launch_error = hipSuccess;
    CHECK(gdn_ctx_destroy(c) == GDN_OK);
    CHECK(gdn_ctx_destroy(nullptr) == GDN_OK);

    // GDN_VALIDATE=1: parent and accepted checked on the host before launching
    setenv("GDN_VALIDATE", "1", 1);
    CHECK(gdn_ctx_create(&d, work, ws, &c) == GDN_OK);
    unsetenv("GDN_VALIDATE");
    const int before = g_stub.verifies;
    t.parent[1 * d.N + 7] = 9;  // a forward edge in sequence 1
    CHECK(verify(c, t) == GDN_ERR_TREE && g_stub.verifies == before);
    t.parent[1 * d.N + 7] = -2;
    CHECK(verify(c, t) == GDN_ERR_TREE);
    t.parent[1 * d.N + 7] = 6;
    CHECK(verify(c, t) == GDN_OK && g_stub.verifies == before + 1);
    t.accepted[0] = 0; t.accepted[1] = d.N; t.accepted[2] = -1;
    CHECK(gdn_commit_path(c, t.accepted, t.S_new, nullptr) == GDN_ERR_ACCEPT);
    t.accepted[1] = d.N - 1;
    CHECK(gdn_commit_path(c, t.accepted, t.S_new, nullptr) == GDN_OK);
    CHECK(gdn_ctx_destroy(c) == GDN_OK);

    // empty batch or tree: no-ops
    const gdn_tree_dims e{2, 0, 1, 1, 64, 64, GDN_F32};
    CHECK(gdn_ctx_create(&e, work, ws, &c) == GDN_OK);
    const int nv = g_stub.verifies;
    CHECK(gdn_tree_verify(c, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, t.S0, nullptr, nullptr) == GDN_OK);
    CHECK(g_stub.verifies == nv);
    CHECK(gdn_ctx_destroy(c) == GDN_OK);

    // ancestors export: argument errors, then a launch
    CHECK(gdn_tree_ancestors(nullptr, t.parent, nullptr, nullptr, nullptr, nullptr) == GDN_ERR_NULL);
    bad = d; bad.N = 300;
    CHECK(gdn_tree_ancestors(&bad, t.parent, reinterpret_cast<uint32_t*>(t.o), t.accepted, nullptr, nullptr) ==
          GDN_ERR_SHAPE);
    CHECK(gdn_tree_ancestors(&d, t.parent, nullptr, t.accepted, nullptr, nullptr) == GDN_ERR_NULL);
    CHECK(gdn_tree_ancestors(&d, t.parent, reinterpret_cast<uint32_t*>(t.o), t.accepted,
                             reinterpret_cast<int32_t*>(reinterpret_cast<char*>(t.g) + 4), nullptr) == GDN_ERR_ALIGN);
    CHECK(gdn_tree_ancestors(&d, t.parent, reinterpret_cast<uint32_t*>(t.o), t.accepted, nullptr, nullptr) == GDN_OK);
    CHECK(g_stub.ancestors == 1);

    // per-branch verify: same checks, and it arms the commit
    CHECK(gdn_ctx_create(&d, work, ws, &c) == GDN_OK);
    CHECK(gdn_tree_verify_branches(c, t.q, t.k, nullptr, t.g, t.beta, t.parent, t.S0, t.o, nullptr) == GDN_ERR_NULL);
    CHECK(gdn_commit_path(c, t.accepted, t.S_new, nullptr) == GDN_ERR_STATE);
    CHECK(gdn_tree_verify_branches(c, t.q, t.k, t.v, t.g, t.beta, t.parent, t.S0, t.o, nullptr) == GDN_OK);
    CHECK(g_stub.branch_verifies == 1 && g_stub.last_verify.v == t.v);
    CHECK(gdn_commit_path(c, t.accepted, t.S_new, nullptr) == GDN_OK);
    CHECK(gdn_ctx_destroy(c) == GDN_OK);

    // fused commit-then-verify: needs a recorded verify; for bf16 and N <= 128
    // one launch with the recorded tree as the previous one; afterwards the
    // new tree is recorded with S0 = S_next
    {
        CHECK(gdn_ctx_create(&d, work, ws, &c) == GDN_OK);
        auto cv = [&](const int32_t* acc, float* s_next, float* o) {
            return gdn_commit_verify(c, acc, t.q, t.k, t.v, t.g, t.beta, t.parent, s_next, o, nullptr);
        };
        CHECK(gdn_commit_verify(nullptr, t.accepted, t.q, t.k, t.v, t.g, t.beta, t.parent, t.S_new, t.o,
                                nullptr) == GDN_ERR_NULL);
        CHECK(cv(t.accepted, t.S_new, t.o) == GDN_ERR_STATE);
        CHECK(verify(c, t) == GDN_OK);
        const int nv = g_stub.verifies, nc = g_stub.commits;
        CHECK(cv(nullptr, t.S_new, t.o) == GDN_ERR_NULL);
        CHECK(cv(t.accepted, nullptr, t.o) == GDN_ERR_NULL);
        CHECK(cv(t.accepted, t.S_new, nullptr) == GDN_ERR_NULL);
        CHECK(cv(t.accepted, t.S_new + 1, t.o) == GDN_ERR_ALIGN);
        CHECK(g_stub.commit_verifies == 0);
        CHECK(cv(t.accepted, t.S_new, t.o) == GDN_OK && g_stub.commit_verifies == 1);
        CHECK(g_stub.verifies == nv && g_stub.commits == nc);
        CHECK(g_stub.last_prev.S0 == t.S0 && g_stub.last_prev.S_next == t.S_new && g_stub.last_verify.S0 == t.S_new);
        CHECK(g_stub.last_prev.accepted == t.accepted && g_stub.last_prev.k == t.k && g_stub.last_verify.q == t.q);
        CHECK(g_stub.last_prev.accept_status == g_stub.last_verify.tree_status + d.B);
        // the record now holds S_next: the next commit starts from it
        CHECK(gdn_commit_path(c, t.accepted, t.S0, nullptr) == GDN_OK && g_stub.last_commit.S0 == t.S_new);
        g_stub.commit_verdict = GDN_ERR_ACCEPT;
        CHECK(cv(t.accepted, t.S_new, t.o) == GDN_OK);
        CHECK(gdn_ctx_status(c, nullptr) == GDN_ERR_ACCEPT);
        g_stub.commit_verdict = 0;
        g_stub.launch_error = hipErrorInvalidValue;
        CHECK(cv(t.accepted, t.S_new, t.o) == GDN_ERR_HIP);
        CHECK(gdn_commit_path(c, t.accepted, t.S_new, nullptr) == GDN_ERR_STATE);
        g_stub.launch_error = hipSuccess;
        CHECK(gdn_ctx_destroy(c) == GDN_OK);
        // fp32 q/k/v: a commit launch, then a verify launch on S_next
        const gdn_tree_dims f{3, 40, 2, 4, 128, 64, GDN_F32};
        CHECK(gdn_ctx_create(&f, work, ws, &c) == GDN_OK);
        CHECK(verify(c, t) == GDN_OK);
        const int nv2 = g_stub.verifies, nc2 = g_stub.commits, ncv = g_stub.commit_verifies;
        CHECK(cv(t.accepted, t.S_new, t.o) == GDN_OK);
        CHECK(g_stub.verifies == nv2 + 1 && g_stub.commits == nc2 + 1 && g_stub.commit_verifies == ncv);
        CHECK(g_stub.last_commit.S_new == t.S_new && g_stub.last_verify.S0 == t.S_new);
        CHECK(gdn_ctx_destroy(c) == GDN_OK);
    }

    // accepted-node selection and tree construction
    int32_t* target = static_cast<int32_t*>(dev_alloc(static_cast<size_t>(d.B) * (d.N + 1) * 4));
    int32_t* lens = static_cast<int32_t*>(dev_alloc(d.B * 4));
    CHECK(gdn_accept_path(&d, t.parent, t.parent, target, t.accepted, lens, nullptr, nullptr) == GDN_OK);
    CHECK(g_stub.accepts == 1 && t.accepted[0] == -1);
    CHECK(gdn_accept_path(&d, t.parent, nullptr, target, t.accepted, lens, nullptr, nullptr) == GDN_ERR_NULL);
    CHECK(gdn_accept_path(&d, t.parent, t.parent, target, t.accepted, lens + 1, nullptr, nullptr) == GDN_ERR_ALIGN);
    float* root = static_cast<float*>(dev_alloc(static_cast<size_t>(d.B) * 8 * 4));
    float* node = static_cast<float*>(dev_alloc(static_cast<size_t>(d.B) * d.N * 8 * 4));
    CHECK(gdn_tree_build(&d, 8, 4, 16, root, node, t.parent, reinterpret_cast<int32_t*>(t.o) + 1, nullptr, nullptr,
                         nullptr, nullptr) == GDN_ERR_ALIGN);
    CHECK(gdn_tree_build(&d, 0, 4, 16, root, node, t.parent, nullptr, nullptr, nullptr, nullptr, nullptr) ==
          GDN_ERR_SHAPE);
    CHECK(gdn_tree_build(&d, 8, 4, 16, root, node, t.parent, nullptr, nullptr, lens, nullptr, nullptr) == GDN_OK);
    CHECK(g_stub.builds == 1 && lens[0] == 1 && t.parent[0] == -1);
    std::free(target);
    std::free(lens);
    std::free(root);
    std::free(node);

    // status names
    for (int s = 0; s <= GDN_ERR_HIP; ++s) CHECK(std::strncmp(gdn_status_string(static_cast<gdn_status>(s)), "GDN_", 4) == 0);
    CHECK(std::strcmp(gdn_status_string(static_cast<gdn_status>(99)), "GDN_ERR_UNKNOWN") == 0);

    std::free(work);
    std::printf("abi_driver: %d failed checks\n", g_fail);
    return g_fail == 0 ? 0 : 1;
}
