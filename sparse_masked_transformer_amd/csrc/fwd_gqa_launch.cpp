// Launch of the generated gfx950 assembly kernel swa_fwd_gqa_d128 (grouped-
// query sliding-window forward, bf16, d = 128): see gen_fwd_gqa.py for the
// kernel.  Its code object is embedded in this library (fwd_gqa_blob.cpp, made
// by the build from the generated .s) and loaded once per device.
#include <mutex>

#include "swa_internal.h"

namespace swa {

extern const unsigned char kFwdGqaCodeObject[];
extern const size_t kFwdGqaCodeObjectSize;

namespace {

// Kernel arguments, in the layout the kernel's prologue loads (80 bytes).
struct GqaArgs {
    const void *q, *k, *v;
    void *out;
    float *lse;
    int32_t N, window, G, head_blocks, row_blocks;
    float c;
    int32_t items, stride, Hkv, Hq;
};
static_assert(sizeof(GqaArgs) == 80, "kernel argument block is 80 bytes");

constexpr int kMaxDevices = 64;

// The kernel function on the current device and that device's compute unit
// count.
hipError_t gqa_function(hipFunction_t *fn, int *cus) {
    static std::mutex mu;
    static hipFunction_t fns[kMaxDevices] = {};
    static int cu_count[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (fns[dev] == nullptr) {
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        cu_count[dev] = n;
        hipModule_t mod = nullptr;
        e = hipModuleLoadData(&mod, kFwdGqaCodeObject);
        if (e != hipSuccess)
            return e;
        hipFunction_t f = nullptr;
        e = hipModuleGetFunction(&f, mod, "swa_fwd_gqa_d128");
        if (e != hipSuccess)
            return e;
        fns[dev] = f;
    }
    *fn = fns[dev];
    *cus = cu_count[dev];
    return hipSuccess;
}

}  // namespace

bool fwd_gqa_applies(const FwdArgs &a) {
    return a.nmaps == 1 && a.d == 128 && a.dv == 128 && a.stride == 0 && a.dilation == 1 &&
           a.n_global == 0 && (a.Hq / a.Hkv) % 4 == 0;
}

int64_t fwd_gqa_items(const FwdArgs &a) {
    // one item per (batch, key/value head, block of 4 query heads, block of
    // 64 query rows)
    return static_cast<int64_t>(a.B) * a.Hkv * ((a.Hq / a.Hkv) / 4) * ((a.N + 63) / 64);
}

hipError_t launch_fwd_gqa(const FwdArgs &a, hipStream_t stream) {
    hipFunction_t fn = nullptr;
    int cus = 0;
    hipError_t e = gqa_function(&fn, &cus);
    if (e != hipSuccess)
        return e;
    GqaArgs k{};
    k.q = a.q[0];
    k.k = a.k[0];
    k.v = a.v;
    k.out = a.out;
    k.lse = a.lse;
    k.N = a.N;
    // distances are < N, so a window of N or more is the full causal mask
    k.window = a.window < a.N ? a.window : a.N;
    k.G = a.Hq / a.Hkv;
    k.head_blocks = k.G / 4;
    k.row_blocks = (a.N + 63) / 64;
    k.c = a.scale * 1.4426950408889634f;
    const int64_t items = fwd_gqa_items(a);
    if (items <= 0 || items > INT32_MAX)
        return hipErrorInvalidValue;
    k.items = static_cast<int32_t>(items);
    // Persistent grid: one workgroup per compute unit (the kernel's LDS
    // allows one), each taking items g, g + grid, ...  A grid that is a
    // multiple of 8 keeps every item of a workgroup on its XCD's
    // contiguous run of items.
    const int64_t per_pass = cus >= 8 ? cus - cus % 8 : items;
    k.stride = static_cast<int32_t>(items < per_pass ? items : per_pass);
    k.Hkv = a.Hkv;
    k.Hq = a.Hq;
    size_t size = sizeof(k);
    void *config[] = {HIP_LAUNCH_PARAM_BUFFER_POINTER, &k, HIP_LAUNCH_PARAM_BUFFER_SIZE, &size,
                      HIP_LAUNCH_PARAM_END};
    e = hipModuleLaunchKernel(fn, static_cast<unsigned>(k.stride), 1, 1, 512, 1, 1, 0, stream, nullptr,
                              config);
    if (e != hipSuccess)
        return e;
    return hipGetLastError();
}

}  // namespace swa
