// host_stubs.cpp -- stand-ins for the HIP runtime and the kernel launchers,
// so that the host side of the C ABI (gdn_tree_api.cpp) can be built and
// run under AddressSanitizer / UndefinedBehaviorSanitizer on a machine
// without a GPU.  "Device" pointers are ordinary host memory here: the
// copy stand-in is memcpy, and the launch stand-ins record their arguments
// and write the verdicts a real launch would (all zero unless a test asks
// for a flagged sequence).

#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstring>

#include "gdn_internal.h"
#include "host_stubs.h"

StubLog g_stub;

extern "C" hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind, hipStream_t) {
    ++g_stub.copies;
    std::memcpy(dst, src, bytes);
    return hipSuccess;
}

extern "C" hipError_t hipStreamSynchronize(hipStream_t) {
    ++g_stub.syncs;
    return hipSuccess;
}

extern "C" const char* hipGetErrorString(hipError_t e) { return e == hipSuccess ? "hipSuccess" : "stub error"; }

namespace gdn {

hipError_t launch_verify(const VerifyArgs& a, hipStream_t) {
    ++g_stub.verifies;
    g_stub.last_verify = a;
    for (int b = 0; b < a.B; ++b) a.tree_status[b] = g_stub.verify_verdict;
    return g_stub.launch_error;
}

hipError_t launch_commit(const CommitArgs& a, hipStream_t) {
    ++g_stub.commits;
    g_stub.last_commit = a;
    for (int b = 0; b < a.B; ++b) a.accept_status[b] = g_stub.commit_verdict;
    return g_stub.launch_error;
}

hipError_t launch_commit_verify(const VerifyArgs& a, const CommitPrev& c, hipStream_t) {
    ++g_stub.commit_verifies;
    g_stub.last_verify = a;
    g_stub.last_prev = c;
    for (int b = 0; b < a.B; ++b) {
        a.tree_status[b] = g_stub.verify_verdict;
        c.accept_status[b] = g_stub.commit_verdict;
    }
    return g_stub.launch_error;
}

hipError_t launch_verify_branches(const VerifyArgs& a, hipStream_t) {
    ++g_stub.branch_verifies;
    g_stub.last_verify = a;
    for (int b = 0; b < a.B; ++b) a.tree_status[b] = g_stub.verify_verdict;
    return g_stub.launch_error;
}

hipError_t launch_accept(int B, int, const int32_t*, const int32_t*, const int32_t*, int32_t* accepted,
                         int32_t* accept_len, int32_t* tree_status, hipStream_t) {
    ++g_stub.accepts;
    for (int b = 0; b < B; ++b) {
        accepted[b] = -1;
        if (accept_len) accept_len[b] = 0;
        if (tree_status) tree_status[b] = 0;
    }
    return g_stub.launch_error;
}

hipError_t launch_build(int B, int N, int, int, int, const float*, const float*, int32_t* parent, int32_t* cand_rank,
                        float* score, int32_t* steps, int32_t* build_status, hipStream_t) {
    ++g_stub.builds;
    for (int i = 0; i < B * N; ++i) {
        parent[i] = -1;
        if (cand_rank) cand_rank[i] = 0;
        if (score) score[i] = 0.f;
    }
    for (int b = 0; b < B; ++b) {
        if (steps) steps[b] = 1;
        if (build_status) build_status[b] = 0;
    }
    return g_stub.launch_error;
}

hipError_t launch_ancestors(int B, int N, const int32_t*, uint32_t*, int32_t*, int32_t* tree_status, hipStream_t) {
    ++g_stub.ancestors;
    if (tree_status)
        for (int b = 0; b < B; ++b) tree_status[b] = 0;
    (void)N;
    return g_stub.launch_error;
}

}  // namespace gdn
