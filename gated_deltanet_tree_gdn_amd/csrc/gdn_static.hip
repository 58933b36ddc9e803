// gdn_static.hip -- gdn_tree_verify_static: tree verification for callers
// that cannot allocate device memory (code under HIP graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The verify kernels write one verdict word per sequence (0, GDN_ERR_TREE,
// or GDN_ERR_HIP after a bounded wait timed out) into scratch memory that
// the context path takes from the caller's workspace.  Here that scratch is
// a file-scope device array, `scratch`, of kStaticMaxB words: each GPU the
// library runs on holds its own copy until the process ends.  Its device
// address is looked up once per device (with that device current) and kept;
// host code never passes the array's name itself to a kernel.
//
// Every call on one GPU shares that GPU's array.  Every verify kernel writes
// the word of each sequence it verifies, so nothing has to start at zero;
// calls that overlap on one GPU (different streams, no ordering) race on the
// words.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "gdn_internal.h"
#include "gdn_tree.h"

namespace gdn {

constexpr int kStaticMaxB = GDN_STATIC_MAX_B;

static __device__ __align__(256) int32_t scratch[kStaticMaxB];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
int32_t* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's copy of `scratch`.
hipError_t scratch_for_current_device(int32_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = static_cast<int32_t*>(p);
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace

}  // namespace gdn

extern "C" gdn_status gdn_tree_verify_static(const gdn_tree_dims* dims, const void* q, const void* k,
                                             const void* v, const float* g, const float* beta,
                                             const int32_t* parent, const float* S0, float* o,
                                             hipStream_t stream) {
    auto fail = [&](gdn_status s, const std::string& m) {
        gdn::set_last_error(m);
        return s;
    };
    if (!dims) return fail(GDN_ERR_NULL, "dims is NULL");
    const gdn_tree_dims d = *dims;
    if (d.qkv_dtype != GDN_BF16 && d.qkv_dtype != GDN_F32)
        return fail(GDN_ERR_DTYPE, "qkv_dtype must be GDN_BF16 or GDN_F32");
    if (d.B < 0) return fail(GDN_ERR_SHAPE, "B must be >= 0");
    if (d.B > gdn::kStaticMaxB)
        return fail(GDN_ERR_SHAPE, "B must be at most " + std::to_string(gdn::kStaticMaxB) +
                                       " for gdn_tree_verify_static (its fixed scratch holds one word per sequence)");
    if (d.N < 0 || d.N > gdn::kMaxN) return fail(GDN_ERR_SHAPE, "N must be in [0, 256]");
    if (d.H_k < 1 || d.H_v < 1) return fail(GDN_ERR_SHAPE, "H_k and H_v must be >= 1");
    if (d.H_v % d.H_k != 0) return fail(GDN_ERR_SHAPE, "H_v must be a multiple of H_k");
    if ((d.d_k != 64 && d.d_k != 128) || (d.d_v != 64 && d.d_v != 128))
        return fail(GDN_ERR_SHAPE, "d_k and d_v must be 64 or 128");
    if (d.B == 0 || d.N == 0) {
        gdn::set_last_error("");
        return GDN_OK;
    }
    const void* ptrs[8] = {q, k, v, g, beta, parent, S0, o};
    const char* names[8] = {"q", "k", "v", "g", "beta", "parent", "S0", "o"};
    for (int i = 0; i < 8; ++i) {
        if (!ptrs[i]) return fail(GDN_ERR_NULL, std::string(names[i]) + " is NULL");
        if (reinterpret_cast<uintptr_t>(ptrs[i]) & 15u)
            return fail(GDN_ERR_ALIGN, std::string(names[i]) + " is not 16-byte aligned");
    }
    int32_t* status = nullptr;
    hipError_t e = gdn::scratch_for_current_device(&status);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, std::string("scratch address: ") + hipGetErrorString(e));
    gdn::VerifyArgs a{d.B, d.N, d.H_k, d.H_v, d.d_k, d.d_v, d.qkv_dtype, q, k, v, g, beta, parent, S0, o,
                      status, 0};
    e = gdn::launch_verify(a, stream);
    if (e != hipSuccess) return fail(GDN_ERR_HIP, std::string("verify launch: ") + hipGetErrorString(e));
    gdn::set_last_error("");
    return GDN_OK;
}
