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

hipError_t launch_ancestors(int B, int N, const int32_t*, uint32_t*, int32_t*, int32_t* tree_status, hipStream_t) {
    ++g_stub.ancestors;
    if (tree_status)
        for (int b = 0; b < B; ++b) tree_status[b] = 0;
    (void)N;
    return g_stub.launch_error;
}

}  // namespace gdn
