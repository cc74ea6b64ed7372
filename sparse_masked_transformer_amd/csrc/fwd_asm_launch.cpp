// Launch of the generated gfx950 assembly kernels: swa_fwd_gqa_d128
// (grouped-query sliding-window forward, bf16, d = 128; gen_fwd_gqa.py), its
// dilated variant swa_fwd_gqa_d128_dil (each residue class of the rows mod
// the dilation walked as a plain window) and global-token variant
// swa_fwd_gqa_d128_glb (the global columns' tiles walked ahead of the band),
// diff_fwd_d64_dv128
// (differential sliding-window forward, bf16, d = 64, dv = 128;
// gen_fwd_diff.py) and swa_fwd_mha_d64_str (multi-head window with an
// optional power-of-two stride pattern, bf16, d = 64; gen_fwd_str.py).
// Their code objects are embedded in this library
// (fwd_gqa_blob.cpp, fwd_gqa_dil_blob.cpp, fwd_gqa_glb_blob.cpp,
// fwd_diff_blob.cpp, fwd_str_blob.cpp, made by the
// build from the generated .s files) and loaded once per device.  All run a
// persistent grid of one 512-lane workgroup per compute unit.
#include <mutex>

#include "swa_internal.h"

namespace swa {

extern const unsigned char kFwdGqaCodeObject[];
extern const size_t kFwdGqaCodeObjectSize;
extern const unsigned char kFwdGqaDilCodeObject[];
extern const size_t kFwdGqaDilCodeObjectSize;
extern const unsigned char kFwdGqaGlbCodeObject[];
extern const size_t kFwdGqaGlbCodeObjectSize;
extern const unsigned char kFwdDiffCodeObject[];
extern const size_t kFwdDiffCodeObjectSize;
extern const unsigned char kFwdStrCodeObject[];
extern const size_t kFwdStrCodeObjectSize;

namespace {

// Kernel arguments, in the layouts the kernels' prologues load (80 bytes).
struct GqaArgs {
    const void *q, *k, *v;
    void *out;
    float *lse;
    int32_t N, window, G, head_blocks, row_blocks;
    float c;
    int32_t items, stride;
    int32_t aux;        // dilated variant: the dilation r; global-token variant: n_global
    int32_t classes;    // dilated variant: the residue classes min(r, N)
};
static_assert(sizeof(GqaArgs) == 80, "kernel argument block is 80 bytes");

struct DiffArgs {
    const void *q1, *k1, *q2, *k2, *v;
    void *out;
    int32_t N, window, G;
    float c;
    float lambda;
    int32_t items, stride, row_blocks;
};
static_assert(sizeof(DiffArgs) == 80, "kernel argument block is 80 bytes");

struct StrArgs {
    const void *q, *k, *v;
    void *out;
    float *lse;
    int32_t N, window, items, stride, row_blocks;
    float c;
    int32_t key_stride;   // stride pattern s (a power of two), or 0
    int32_t log2_stride;  // log2 s (0 without a stride)
    int32_t pad[2];
};
static_assert(sizeof(StrArgs) == 80, "kernel argument block is 80 bytes");

constexpr int kMaxDevices = 64;

enum AsmKernel { kGqa = 0, kGqaDil = 1, kGqaGlb = 2, kDiff = 3, kStr = 4, kNumAsm = 5 };

// The kernel function `which` on the current device and that device's
// compute unit count.
hipError_t asm_function(AsmKernel which, hipFunction_t *fn, int *cus) {
    static std::mutex mu;
    static hipFunction_t fns[kMaxDevices][kNumAsm] = {};
    static int cu_count[kMaxDevices] = {};
    static const unsigned char *const images[kNumAsm] = {kFwdGqaCodeObject, kFwdGqaDilCodeObject,
                                                         kFwdGqaGlbCodeObject, kFwdDiffCodeObject,
                                                         kFwdStrCodeObject};
    static const char *const names[kNumAsm] = {"swa_fwd_gqa_d128", "swa_fwd_gqa_d128_dil",
                                               "swa_fwd_gqa_d128_glb", "diff_fwd_d64_dv128",
                                               "swa_fwd_mha_d64_str"};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (cu_count[dev] == 0) {
        int n = 0;
        e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        cu_count[dev] = n;
    }
    if (fns[dev][which] == nullptr) {
        hipModule_t mod = nullptr;
        e = hipModuleLoadData(&mod, images[which]);
        if (e != hipSuccess)
            return e;
        hipFunction_t f = nullptr;
        e = hipModuleGetFunction(&f, mod, names[which]);
        if (e != hipSuccess)
            return e;
        fns[dev][which] = f;
    }
    *fn = fns[dev][which];
    *cus = cu_count[dev];
    return hipSuccess;
}

// Persistent grid: one workgroup per compute unit (the kernels' LDS allows
// one), each taking items g, g + grid, ...  A grid that is a multiple of 8
// keeps every item of a workgroup on its XCD's contiguous run of items.
int32_t persistent_grid(int64_t items, int cus) {
    const int64_t per_pass = cus >= 8 ? cus - cus % 8 : items;
    return static_cast<int32_t>(items < per_pass ? items : per_pass);
}

hipError_t launch(hipFunction_t fn, void *args, size_t size, int32_t grid, hipStream_t stream) {
    void *config[] = {HIP_LAUNCH_PARAM_BUFFER_POINTER, args, HIP_LAUNCH_PARAM_BUFFER_SIZE, &size,
                      HIP_LAUNCH_PARAM_END};
    hipError_t e = hipModuleLaunchKernel(fn, static_cast<unsigned>(grid), 1, 1, 512, 1, 1, 0, stream,
                                         nullptr, config);
    if (e != hipSuccess)
        return e;
    return hipGetLastError();
}

}  // namespace

bool fwd_gqa_applies(const FwdArgs &a) {
    // a window, dilated or with global tokens (not both)
    return a.nmaps == 1 && a.d == 128 && a.dv == 128 && a.stride == 0 &&
           (a.dilation == 1 || a.n_global == 0) && (a.Hq / a.Hkv) % 4 == 0;
}

namespace {
// rows of the longest residue class, the number of classes with rows, and
// 64-row blocks per class (dilation 1: one class of N rows)
int64_t class_rows(const FwdArgs &a) { return (static_cast<int64_t>(a.N) + a.dilation - 1) / a.dilation; }
int64_t class_count(const FwdArgs &a) { return a.dilation < a.N ? a.dilation : a.N; }
int64_t class_blocks(const FwdArgs &a) { return (class_rows(a) + 63) / 64; }
}  // namespace

int64_t fwd_gqa_items(const FwdArgs &a) {
    // one item per (batch, key/value head, block of 4 query heads, residue
    // class of the rows mod the dilation, block of 64 rows of the class)
    return static_cast<int64_t>(a.B) * a.Hkv * ((a.Hq / a.Hkv) / 4) * class_count(a) * class_blocks(a);
}

hipError_t launch_fwd_gqa(const FwdArgs &a, hipStream_t stream) {
    hipFunction_t fn = nullptr;
    int cus = 0;
    const AsmKernel which = a.dilation > 1 ? kGqaDil : (a.n_global > 0 ? kGqaGlb : kGqa);
    hipError_t e = asm_function(which, &fn, &cus);
    if (e != hipSuccess)
        return e;
    GqaArgs k{};
    k.q = a.q[0];
    k.k = a.k[0];
    k.v = a.v;
    k.out = a.out;
    k.lse = a.lse;
    k.N = a.N;
    // distances within a class are below its length, so a window of that
    // length or more is the full causal mask of the class
    const int64_t rows = class_rows(a);
    k.window = static_cast<int32_t>(a.window < rows ? a.window : rows);
    k.G = a.Hq / a.Hkv;
    k.head_blocks = k.G / 4;
    k.row_blocks = static_cast<int32_t>(class_blocks(a));
    k.c = a.scale * 1.4426950408889634f;
    const int64_t items = fwd_gqa_items(a);
    if (items <= 0 || items > INT32_MAX)
        return hipErrorInvalidValue;
    k.items = static_cast<int32_t>(items);
    k.stride = persistent_grid(items, cus);
    k.aux = which == kGqaGlb ? (a.n_global < a.N ? a.n_global : a.N) : a.dilation;
    k.classes = static_cast<int32_t>(class_count(a));
    return launch(fn, &k, sizeof(k), k.stride, stream);
}

bool fwd_diff_asm_applies(const FwdArgs &a) {
    return a.nmaps == 2 && a.d == 64 && a.dv == 128 && a.stride == 0 && a.dilation == 1 &&
           a.n_global == 0;
}

int64_t fwd_diff_asm_items(const FwdArgs &a) {
    // one item per (batch, query head, block of 128 query rows)
    return static_cast<int64_t>(a.B) * a.Hq * ((a.N + 127) / 128);
}

hipError_t launch_fwd_diff_asm(const FwdArgs &a, hipStream_t stream) {
    hipFunction_t fn = nullptr;
    int cus = 0;
    hipError_t e = asm_function(kDiff, &fn, &cus);
    if (e != hipSuccess)
        return e;
    DiffArgs k{};
    k.q1 = a.q[0];
    k.k1 = a.k[0];
    k.q2 = a.q[1];
    k.k2 = a.k[1];
    k.v = a.v;
    k.out = a.out;
    k.N = a.N;
    k.window = a.window < a.N ? a.window : a.N;
    k.G = a.Hq / a.Hkv;
    k.c = a.scale * 1.4426950408889634f;
    k.lambda = a.lambda;
    const int64_t items = fwd_diff_asm_items(a);
    if (items <= 0 || items > INT32_MAX)
        return hipErrorInvalidValue;
    k.items = static_cast<int32_t>(items);
    k.stride = persistent_grid(items, cus);
    k.row_blocks = (a.N + 127) / 128;
    return launch(fn, &k, sizeof(k), k.stride, stream);
}

namespace {
// log2 of a stride the multi-head kernel takes (a power of two from 64 to
// 2^18: a 64-key tile then holds at most one stride key, and gathered key
// offsets stay below 2^32 bytes for N up to 2^22), else -1
int str_log2(int stride) {
    for (int k = 6; k <= 18; ++k)
        if (stride == (1 << k))
            return k;
    return -1;
}
}  // namespace

bool fwd_str_applies(const FwdArgs &a) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.Hq;
    return a.nmaps == 1 && a.d == 64 && a.dv == 64 && a.Hq == a.Hkv && heads % 2 == 0 &&
           a.dilation == 1 && a.n_global == 0 && (a.stride == 0 || str_log2(a.stride) > 0);
}

int64_t fwd_str_items(const FwdArgs &a) {
    // one item per (pair of consecutive (batch, head) indices, block of 128
    // query rows)
    return static_cast<int64_t>(a.B) * a.Hq / 2 * ((a.N + 127) / 128);
}

hipError_t launch_fwd_str(const FwdArgs &a, hipStream_t stream) {
    hipFunction_t fn = nullptr;
    int cus = 0;
    hipError_t e = asm_function(kStr, &fn, &cus);
    if (e != hipSuccess)
        return e;
    StrArgs k{};
    k.q = a.q[0];
    k.k = a.k[0];
    k.v = a.v;
    k.out = a.out;
    k.lse = a.lse;
    k.N = a.N;
    k.window = a.window < a.N ? a.window : a.N;
    k.c = a.scale * 1.4426950408889634f;
    const int64_t items = fwd_str_items(a);
    if (items <= 0 || items > INT32_MAX)
        return hipErrorInvalidValue;
    k.items = static_cast<int32_t>(items);
    k.stride = persistent_grid(items, cus);
    k.row_blocks = (a.N + 127) / 128;
    k.key_stride = a.stride;
    k.log2_stride = a.stride > 0 ? str_log2(a.stride) : 0;
    return launch(fn, &k, sizeof(k), k.stride, stream);
}

}  // namespace swa
