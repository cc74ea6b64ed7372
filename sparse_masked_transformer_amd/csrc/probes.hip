// Measurement probes (include/swa_probe.h): a dense bf16 MFMA loop and a
// streaming HBM read, the sustained rates the benchmark reports beside the
// published MI355X peaks.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/swa.h"
#include "../../include/swa_probe.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Four independent accumulators per wave (a new product can start every
// issue slot), 32 products per loop trip; the operand pairs rotate so the
// inputs change from one product to the next, as they do in a real
// contraction.  One workgroup (8 waves, two per SIMD) per CU: the LDS array
// (never read for data) keeps a second workgroup off the CU.
__global__ __launch_bounds__(512) void probe_mfma_kernel(const bf16x8 *__restrict__ ops,
                                                         float *__restrict__ out, int iters) {
    __shared__ float hold[24576];
    const int lane = threadIdx.x & 63;
    const bf16x8 a0 = ops[lane], a1 = ops[64 + lane], a2 = ops[128 + lane], a3 = ops[192 + lane];
    const bf16x8 b0 = ops[256 + lane], b1 = ops[320 + lane], b2 = ops[384 + lane], b3 = ops[448 + lane];
    f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b2, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b3, c3, 0, 0, 0);
            c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b0, c0, 0, 0, 0);
            c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a2, b1, c1, 0, 0, 0);
            c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a3, b2, c2, 0, 0, 0);
            c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b3, c3, 0, 0, 0);
        }
    }
    float s = 0.f;
#pragma unroll
    for (int k = 0; k < 16; ++k)
        s += c0[k] + c1[k] + c2[k] + c3[k];
    hold[threadIdx.x] = s;
    __syncthreads();
    out[blockIdx.x * 512 + threadIdx.x] = hold[511 - threadIdx.x];
}

// Each workgroup reads a contiguous share of the buffer, four 16-byte loads
// per thread in flight per trip.
__global__ __launch_bounds__(256) void probe_stream_kernel(const u32x4 *__restrict__ p, size_t n16,
                                                           uint32_t *__restrict__ out) {
    const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
    const size_t lo = blockIdx.x * per;
    const size_t hi = lo + per < n16 ? lo + per : n16;
    uint32_t acc = 0;
    size_t i = lo + threadIdx.x;
    for (; i + 768 < hi; i += 1024) {
        const u32x4 x0 = __builtin_nontemporal_load(p + i);
        const u32x4 x1 = __builtin_nontemporal_load(p + i + 256);
        const u32x4 x2 = __builtin_nontemporal_load(p + i + 512);
        const u32x4 x3 = __builtin_nontemporal_load(p + i + 768);
        acc ^= x0.x ^ x0.y ^ x0.z ^ x0.w ^ x1.x ^ x1.y ^ x1.z ^ x1.w;
        acc ^= x2.x ^ x2.y ^ x2.z ^ x2.w ^ x3.x ^ x3.y ^ x3.z ^ x3.w;
    }
    for (; i < hi; i += 256) {
        const u32x4 x = p[i];
        acc ^= x.x ^ x.y ^ x.z ^ x.w;
    }
    out[blockIdx.x * 256 + threadIdx.x] = acc;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int launched() { return hipGetLastError() == hipSuccess ? SWA_OK : SWA_ERR_HIP; }

}  // namespace

extern "C" int swa_probe_mfma_bf16(const void *operands, float *out, int workgroups, int iters,
                                   hipStream_t stream) {
    if (!operands || !out || !aligned16(operands) || workgroups < 1 || workgroups > 65535 || iters < 1 ||
        iters > (1 << 24))
        return SWA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(probe_mfma_kernel, dim3(workgroups), dim3(512), 0, stream,
                       static_cast<const bf16x8 *>(operands), out, iters);
    return launched();
}

extern "C" int swa_probe_stream_read(const void *buf, size_t bytes, uint32_t *out, int workgroups,
                                     hipStream_t stream) {
    if (!buf || !out || !aligned16(buf) || bytes == 0 || (bytes & 15) != 0 || workgroups < 1 ||
        workgroups > 65535)
        return SWA_ERR_INVALID_ARG;
    hipLaunchKernelGGL(probe_stream_kernel, dim3(workgroups), dim3(256), 0, stream,
                       static_cast<const u32x4 *>(buf), bytes / 16, out);
    return launched();
}
