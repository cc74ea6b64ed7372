// Internal interface between the C-ABI front end (swa_abi.cpp) and the HIP
// kernels.  Not installed; the public interface is include/swa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/swa.h"

namespace swa {

// Query tile rows and key tile size every attention kernel walks.
constexpr int kBM = 128;
constexpr int kBN = 64;

// Device view of a block mask.
struct MaskView {
    const int32_t *row_ptr;
    const int32_t *kv_tile;
    const uint8_t *kind;
    const int32_t *stride_keys;
    const int32_t *band_begin;
    int32_t num_q_tiles;
};

// One masked-attention forward problem (one or two score maps).
struct FwdArgs {
    const void *q[2];
    const void *k[2];
    const void *v;
    void *out;
    float *lse;
    int B, Hq, Hkv, N, d, dv, window, stride;
    float scale;
    float lambda;   // weight of the second map (two-map problems only)
    int nmaps;      // 1 or 2
    MaskView mask;
};

struct DecodeArgs {
    const void *q;
    const void *k_ring;
    const void *v_ring;
    void *out;
    const int32_t *seq_len;
    void *workspace;
    int B, Hq, Hkv, N, d, window;
    float scale;
};

// Number of key splits the decode kernel uses for a ring of `window` slots.
int decode_splits(int window);

hipError_t launch_block_mask_build(const swa_block_mask_t &m, hipStream_t stream);
hipError_t launch_mask_dense(int N, int window, int stride, uint8_t *out, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeArgs &a, hipStream_t stream);

}  // namespace swa
