// Internal interface between the C-ABI front end (swa_abi.cpp) and the HIP
// kernels.  Not installed; the public interface is include/swa.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/swa.h"

namespace swa {

// Key tile size every attention kernel walks.
constexpr int kBN = 64;
// bf16 kernels: 4 waves per workgroup, each owning this many groups of 32
// query rows (128-row query tiles for one map and for two).
constexpr int kFwdRowGroups = 1;
constexpr int kDiffRowGroups = 1;
// fp32 kernels: 8 lanes per row of a 32-row query tile (256-lane
// workgroups: one wave per SIMD, the full 256-VGPR budget per lane, and
// small problems spread over many compute units).
constexpr int kF32BM = 32;
constexpr int kF32TPR = 8;   // lanes per query row (fp32 forward and decode)
// Lanes per workgroup of the forward kernels: 256, except the bf16
// two-map kernel (its maps run on separate waves).
constexpr int kFwdThreads = 256;
constexpr int kDiffFwdThreads = 512;
static_assert(kF32BM * kF32TPR == kFwdThreads, "fp32 forward tile = one 256-lane workgroup");
// A dispatch holds at most 2^32 - 1 work-items per grid dimension; every
// launch here uses one dimension.
constexpr int64_t kMaxGridItems = 0xffffffffLL;

// Query tile rows of the kernel serving (op, dtype).
inline int tile_rows(int op, int dt) {
    if (dt == SWA_F32)
        return kF32BM;
    return 128 * (op == SWA_OP_DIFF ? kDiffRowGroups : kFwdRowGroups);
}

// Device view of a block mask.
struct MaskView {
    const int32_t *row_ptr;
    const int32_t *kv_tile;
    const uint8_t *kind;
    const int32_t *prefix_keys;
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
    int B, Hq, Hkv, N, d, dv, window, stride, dilation, n_global;
    float scale;
    float lambda;   // weight of the second map (two-map problems only)
    int nmaps;      // 1 or 2
    MaskView mask;
};

// The bf16 single-map forward over a dilated window alone (no stride, no
// global tokens) walks each residue class of the rows mod dilation as a dense
// band: one workgroup per (batch, head, residue class, class-local tile).
// Every other forward has one workgroup per (batch, head, query tile).
inline bool fwd_by_residue_class(const FwdArgs &a, int dt) {
    return dt == SWA_BF16 && a.nmaps == 1 && a.dilation > 1 && a.stride == 0 && a.n_global == 0;
}

// Lanes per workgroup of the forward launch for (a, dt).
inline int fwd_threads(const FwdArgs &a, int dt) {
    return dt == SWA_BF16 && a.nmaps == 2 ? kDiffFwdThreads : kFwdThreads;
}

// Workgroups of the forward launch for (a, dt).
inline int64_t fwd_workgroups(const FwdArgs &a, int dt) {
    const int64_t heads = static_cast<int64_t>(a.B) * a.Hq;
    if (fwd_by_residue_class(a, dt)) {
        const int64_t bm = 128 * kFwdRowGroups;
        const int64_t rows = (static_cast<int64_t>(a.N) + a.dilation - 1) / a.dilation;
        return (rows + bm - 1) / bm * a.dilation * heads;
    }
    return static_cast<int64_t>(a.mask.num_q_tiles) * heads;
}

// k-th prefix key (0 <= k < count) of a query tile whose prefix-only tiles
// hold `count` prefix keys: the global columns 0 .. g'-1 (g' = min(n_global,
// count)), then the multiples of stride from g' on.
__host__ __device__ inline int prefix_key(int k, int count, int stride, int n_global) {
    const int gp = n_global < count ? n_global : count;
    if (k < gp)
        return k;
    const int first = (gp + stride - 1) / stride;   // stride > 0 whenever k >= gp
    return (first + (k - gp)) * stride;
}

// One decode step (one or two score maps, optional sink slots).
struct DecodeArgs {
    const void *q[2];
    const void *k_ring[2];
    const void *v_ring;
    const void *k_sink[2];   // used when n_sink > 0
    const void *v_sink;
    void *out;
    const int32_t *seq_len;
    void *workspace;
    int B, Hq, Hkv, N, d, dv, window, n_sink, nmaps;
    float scale;
    float lambda;   // weight of the second map (two-map problems only)
};

// Decode work split (bf16 kernel): slots are walked in steps of kDecodeStep;
// a workgroup of `waves` waves (at most kDecodeMaxWaves) covers one split of
// one (sequence, key/value head), each wave `steps_per_wave` steps.
constexpr int kDecodeStep = 32;
constexpr int kDecodeMaxWaves = 4;
constexpr int kDecodeMaxSplits = 16;
// Waves resident on the chip at two per SIMD (256 CUs x 4 SIMDs x 2).
constexpr int kDecodeTargetWaves = 2048;

struct DecodePlan {
    int waves, splits, steps_per_wave;
};
// Plan for B*Hkv (sequence, key/value head) pairs and at most `slots` cache
// slots (window + sink slots) per pair.
DecodePlan decode_plan(int B, int Hkv, int slots);
// The bf16 decode kernel takes the query heads of a key/value head 16 at a
// time (the columns of one MFMA tile): blocks per key/value head.
inline int decode_head_blocks(int Hq, int Hkv) { return (Hq / Hkv + 15) / 16; }
// The plan of a decode call: each block of query heads counts as a pair.
inline DecodePlan decode_plan_for(const DecodeArgs &a) {
    return decode_plan(a.B, a.Hkv * decode_head_blocks(a.Hq, a.Hkv), a.window + a.n_sink);
}
// Work-items of the largest dispatch one decode call makes.
int64_t decode_launch_items(const DecodeArgs &a, int dt);
// fp32 count of the (max, sum) section of the decode workspace for `parts`
// partial results, padded so the output section starts 16-byte aligned.
inline int64_t decode_ws_ml_floats(int64_t parts) { return (parts * 2 + 3) / 4 * 4; }

// Address, on the current device, of the decode kernels' static scratch
// array (SWA_DECODE_SCRATCH_BYTES): looked up once per device.
hipError_t decode_static_scratch(void **ptr);

hipError_t launch_block_mask_build(const swa_block_mask_t &m, hipStream_t stream);
hipError_t launch_mask_dense(int N, int window, int stride, int dilation, int n_global, uint8_t *out,
                             hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream);
// The generated assembly kernel for grouped-query sliding windows (bf16,
// d = dv = 128, no stride, dilation or global tokens, a multiple of 4 query
// heads per key/value head): whether it serves `a`, its workgroup count,
// and its launch.
bool fwd_gqa_applies(const FwdArgs &a);
int64_t fwd_gqa_items(const FwdArgs &a);
hipError_t launch_fwd_gqa(const FwdArgs &a, hipStream_t stream);
// The differential kernel for bf16, d = 64, dv = 128, window only.
bool fwd_diff_asm_applies(const FwdArgs &a);
int64_t fwd_diff_asm_items(const FwdArgs &a);
hipError_t launch_fwd_diff_asm(const FwdArgs &a, hipStream_t stream);
// The multi-head kernel for bf16, d = dv = 64, a window with an optional
// power-of-two stride pattern (64 .. 2^18), B * Hq even.
bool fwd_str_applies(const FwdArgs &a);
int64_t fwd_str_items(const FwdArgs &a);
hipError_t launch_fwd_str(const FwdArgs &a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t stream);
hipError_t launch_decode_f32(const DecodeArgs &a, hipStream_t stream);

}  // namespace swa
