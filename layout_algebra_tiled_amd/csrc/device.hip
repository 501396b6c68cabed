// Device side of the layout library: the gfx950 capability gate and the
// device layout maps (evaluate / gather through a layout).
//
// The gate follows "CUTLASS and CuTe layouts", "Results" and "Pitfalls": a
// build for one architecture refuses a device of another before anything is
// allocated or launched. The layout maps are that page's device gather: the
// same layout the host evaluates, walked by a kernel.

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
#include <string>

#include "layout_host.hpp"
#include "lt.h"

namespace lt {

namespace {

std::mutex g_arch_mu;
std::string g_arch_override;
bool g_have_override = false;
int g_checked_device = -1;
lt_status g_checked_status = LT_OK;

// Leaves of a layout in the order of colexicographic unravelling; the tree is
// not needed to evaluate at a 1-D index.
struct DevLeaves {
    int n;
    int wide;                 // 1: 64-bit arithmetic needed
    int64_t s[LT_MAX_LEAVES];
    int64_t d[LT_MAX_LEAVES];
};

template <bool WIDE>
__device__ __forceinline__ int64_t eval_at(const DevLeaves& L, int64_t x) {
    if (WIDE) {
        int64_t off = 0;
        for (int i = 0; i < L.n; ++i) {
            off += (x % L.s[i]) * L.d[i];
            x /= L.s[i];
        }
        return off;
    }
    uint32_t y = static_cast<uint32_t>(x), off = 0;
    for (int i = 0; i < L.n; ++i) {
        const uint32_t s = static_cast<uint32_t>(L.s[i]);
        off += (y % s) * static_cast<uint32_t>(L.d[i]);
        y /= s;
    }
    return off;
}

template <bool WIDE>
__global__ __launch_bounds__(256) void layout_eval_kernel(DevLeaves L, int64_t* out, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += stride) out[x] = eval_at<WIDE>(L, x);
}

template <bool WIDE, typename E>
__global__ __launch_bounds__(256) void layout_gather_kernel(DevLeaves L, const E* src, E* dst, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; x < n; x += stride)
        dst[x] = src[eval_at<WIDE>(L, x)];
}

lt_status prepare(const lt_layout* L, int64_t n, DevLeaves* dl, int64_t* cos) {
    Tree t;
    lt_status st = from_pod(L, &t);
    if (st != LT_OK) return st;
    int64_t sz;
    st = tree_size(t, &sz);
    if (st != LT_OK) return st;
    if (n < 0 || n > sz) return LT_ERR_OUT_OF_RANGE;
    st = tree_cosize(t, cos);
    if (st != LT_OK) return st;
    std::memset(dl, 0, sizeof(*dl));
    dl->n = static_cast<int>(t.s.size());
    for (int i = 0; i < dl->n; ++i) {
        dl->s[i] = t.s[i];
        dl->d[i] = t.d[i];
    }
    dl->wide = (sz > (int64_t(1) << 31) || *cos > (int64_t(1) << 31)) ? 1 : 0;
    return LT_OK;
}

dim3 grid_for(int64_t n) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    return dim3(static_cast<unsigned>(blocks));
}

}  // namespace

// Capability gate, shared with the GEMM entry points.
lt_status ensure_device() {
    std::lock_guard<std::mutex> lk(g_arch_mu);
    if (g_have_override) {
        return g_arch_override.rfind("gfx950", 0) == 0 ? LT_OK : LT_ERR_ARCH_MISMATCH;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return LT_ERR_HIP;
    if (dev == g_checked_device) return g_checked_status;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return LT_ERR_HIP;
    g_checked_device = dev;
    g_checked_status = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? LT_OK : LT_ERR_ARCH_MISMATCH;
    return g_checked_status;
}

}  // namespace lt

extern "C" {

lt_status lt_set_arch_override(const char* arch) {
    std::lock_guard<std::mutex> lk(lt::g_arch_mu);
    if (arch) {
        lt::g_arch_override = arch;
        lt::g_have_override = true;
    } else {
        lt::g_arch_override.clear();
        lt::g_have_override = false;
    }
    return LT_OK;
}

lt_status lt_device_check(char* arch_out, size_t cap) {
    std::string name;
    {
        std::lock_guard<std::mutex> lk(lt::g_arch_mu);
        if (lt::g_have_override) name = lt::g_arch_override;
    }
    if (name.empty()) {
        int dev = 0;
        hipDeviceProp_t prop;
        if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess) return LT_ERR_HIP;
        name = prop.gcnArchName;
    }
    if (arch_out && cap > 0) {
        std::strncpy(arch_out, name.c_str(), cap - 1);
        arch_out[cap - 1] = '\0';
    }
    return lt::ensure_device();
}

lt_status lt_layout_eval_device(const lt_layout* L, int64_t* d_out, int64_t n, void* stream) {
    if (!d_out && n > 0) return LT_ERR_INVALID_ARGUMENT;
    lt::DevLeaves dl;
    int64_t cos;
    lt_status st = lt::prepare(L, n, &dl, &cos);
    if (st != LT_OK) return st;
    if (n == 0) return LT_OK;
    st = lt::ensure_device();
    if (st != LT_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (dl.wide)
        hipLaunchKernelGGL(lt::layout_eval_kernel<true>, lt::grid_for(n), dim3(256), 0, s, dl, d_out, n);
    else
        hipLaunchKernelGGL(lt::layout_eval_kernel<false>, lt::grid_for(n), dim3(256), 0, s, dl, d_out, n);
    return hipGetLastError() == hipSuccess ? LT_OK : LT_ERR_HIP;
}

lt_status lt_gather_device(const lt_layout* L, const void* d_src, void* d_dst, int32_t elem_bytes, int64_t n,
                           void* stream) {
    if ((!d_src || !d_dst) && n > 0) return LT_ERR_INVALID_ARGUMENT;
    if (elem_bytes != 1 && elem_bytes != 2 && elem_bytes != 4 && elem_bytes != 8) return LT_ERR_INVALID_ARGUMENT;
    lt::DevLeaves dl;
    int64_t cos;
    lt_status st = lt::prepare(L, n, &dl, &cos);
    if (st != LT_OK) return st;
    if (n == 0) return LT_OK;
    st = lt::ensure_device();
    if (st != LT_OK) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    dim3 g = lt::grid_for(n), b(256);
#define LT_GATHER(E)                                                                                     \
    do {                                                                                                 \
        if (dl.wide)                                                                                     \
            hipLaunchKernelGGL((lt::layout_gather_kernel<true, E>), g, b, 0, s, dl, (const E*)d_src, (E*)d_dst, n); \
        else                                                                                             \
            hipLaunchKernelGGL((lt::layout_gather_kernel<false, E>), g, b, 0, s, dl, (const E*)d_src, (E*)d_dst, n); \
    } while (0)
    switch (elem_bytes) {
        case 1: LT_GATHER(uint8_t); break;
        case 2: LT_GATHER(uint16_t); break;
        case 4: LT_GATHER(uint32_t); break;
        default: LT_GATHER(uint64_t); break;
    }
#undef LT_GATHER
    return hipGetLastError() == hipSuccess ? LT_OK : LT_ERR_HIP;
}

}  // extern "C"
