// C-ABI front end: host-side argument checks, block-mask sizing and kernel
// dispatch.  Every check runs before the first HIP call, so a rejected call
// touches no device state (and every error path can be exercised without a
// GPU).
#include <cmath>
#include <cstdint>
#include <cstring>

#include "swa_internal.h"

using swa::kBN;

namespace {

bool aligned16(const void *p) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool head_dim_ok(int d) { return d == 32 || d == 64 || d == 128; }

bool tile_ok(int t) { return t == 16 || t == 32 || t == 64 || t == 128 || t == 256; }

// List length of one query tile: the band tiles form one contiguous range
// [t_lo, t_hi] covering keys max(0, r0 - (window-1)*dilation) .. r1 (r0, r1 =
// first and last row of the tile; with dilation <= bn each of them holds an
// attended cell); every prefix key (global column or multiple of stride) left
// of that range is attended by every row of the tile, and the tiles holding
// one are listed first.
void q_tile_counts(int64_t q, int64_t N, int64_t window, int64_t stride, int64_t dilation,
                   int64_t n_global, int64_t bm, int64_t bn, int64_t *n_band,
                   int64_t *n_prefix_only) {
    int64_t r0 = q * bm;
    int64_t r1 = (r0 + bm < N ? r0 + bm : N) - 1;
    int64_t span = (window - 1) * dilation;
    int64_t lo = r0 - span > 0 ? r0 - span : 0;
    int64_t t_lo = lo / bn, t_hi = r1 / bn;
    *n_band = t_hi - t_lo + 1;
    // tiles [0, a) hold a global column; stride tiles are counted from a on
    int64_t a = (n_global + bn - 1) / bn;
    a = a < t_lo ? a : t_lo;
    int64_t ns = 0;
    if (stride > 0 && t_lo > a) {
        if (stride <= bn)
            ns = t_lo - a;  // every tile of bn >= stride keys holds a multiple
        else                // one multiple per tile at most
            ns = (t_lo * bn + stride - 1) / stride - (a * bn + stride - 1) / stride;
    }
    *n_prefix_only = a + ns;
}

int mask_query(int N, int window, int stride, int dilation, int n_global, int bm, int bn,
               int32_t *nq_out, int32_t *nnz_out) {
    if (N < 1 || N > SWA_MAX_N || window < 1 || stride < 0 || !tile_ok(bm) || !tile_ok(bn) ||
        dilation < 1 || dilation > bn || n_global < 0 || n_global > SWA_MAX_N)
        return SWA_ERR_INVALID_ARG;
    int64_t nq = (static_cast<int64_t>(N) + bm - 1) / bm, nnz = 0;
    for (int64_t q = 0; q < nq; ++q) {
        int64_t nb, np;
        q_tile_counts(q, N, window, stride, dilation, n_global, bm, bn, &nb, &np);
        nnz += nb + np;
    }
    if (nnz > INT32_MAX)
        return SWA_ERR_UNSUPPORTED;
    if (nq_out)
        *nq_out = static_cast<int32_t>(nq);
    if (nnz_out)
        *nnz_out = static_cast<int32_t>(nnz);
    return SWA_OK;
}

bool mask_arrays_ok(const swa_block_mask_t *m) {
    return m->row_ptr && m->kv_tile && m->kind && m->cells && m->prefix_keys && m->band_begin;
}

// The mask must describe exactly this problem and the kernel's tiling.
int check_mask(const swa_block_mask_t *m, int N, int window, int stride, int dilation,
               int n_global, int bm) {
    if (m == nullptr)
        return SWA_ERR_INVALID_ARG;
    if (m->N != N || m->window != window || m->stride != stride || m->dilation != dilation ||
        m->n_global != n_global || m->bm != bm || m->bn != kBN)
        return SWA_ERR_INVALID_ARG;
    int32_t nq = 0, nnz = 0;
    int st = mask_query(N, window, stride, dilation, n_global, bm, kBN, &nq, &nnz);
    if (st != SWA_OK)
        return st;
    if (m->num_q_tiles != nq || m->nnz != nnz || !mask_arrays_ok(m))
        return SWA_ERR_INVALID_ARG;
    return SWA_OK;
}

int check_sizes(int B, int Hq, int Hkv, int N, int window, int stride, int dilation,
                int n_global) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || N < 1 || N > SWA_MAX_N || window < 1 ||
        stride < 0 || dilation < 1 || n_global < 0)
        return SWA_ERR_INVALID_ARG;
    // every flat row index (b*Hq + h)*N + i fits in int32
    if (static_cast<int64_t>(B) * Hq * N > INT32_MAX)
        return SWA_ERR_UNSUPPORTED;
    return SWA_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? SWA_OK : SWA_ERR_HIP; }

int fwd_run(const swa::FwdArgs &a, int dt, hipStream_t stream) {
    if (swa::fwd_workgroups(a, dt) * swa::fwd_threads(a, dt) > swa::kMaxGridItems)
        return SWA_ERR_UNSUPPORTED;  // more work-items than one dispatch holds
    return hip_status(dt == SWA_BF16 ? swa::launch_fwd_bf16(a, stream) : swa::launch_fwd_f32(a, stream));
}

swa::MaskView view_of(const swa_block_mask_t *m) {
    return swa::MaskView{m->row_ptr, m->kv_tile, m->kind, m->prefix_keys, m->band_begin,
                         m->num_q_tiles};
}

}  // namespace

namespace swa {
DecodePlan decode_plan(int B, int Hkv, int slots) {
    // At least 8 steps per wave where the cache allows; enough workgroups to
    // fill the chip once; every wave at least one step.
    const int64_t steps = (static_cast<int64_t>(slots > 0 ? slots : 1) + kDecodeStep - 1) / kDecodeStep;
    int64_t waves = (steps + 7) / 8;
    waves = waves < 1 ? 1 : (waves > kDecodeMaxWaves ? kDecodeMaxWaves : waves);
    const int64_t pairs = static_cast<int64_t>(B) * Hkv;
    const int64_t want_wgs = (kDecodeTargetWaves + waves - 1) / waves;
    int64_t splits = (want_wgs + pairs - 1) / pairs;
    int64_t max_splits = (steps + waves - 1) / waves;
    max_splits = max_splits < kDecodeMaxSplits ? max_splits : kDecodeMaxSplits;
    splits = splits < 1 ? 1 : (splits > max_splits ? max_splits : splits);
    const int64_t spw = (steps + splits * waves - 1) / (splits * waves);
    return DecodePlan{static_cast<int>(waves), static_cast<int>(splits), static_cast<int>(spw)};
}

int64_t decode_launch_items(const DecodeArgs &a, int dt) {
    const int64_t rows = static_cast<int64_t>(a.B) * a.Hq;   // (sequence, query head) pairs
    if (dt == SWA_F32) {
        // 64-lane workgroups of 64 / kF32TPR rows
        const int64_t per_wg = 64 / kF32TPR;
        return (rows + per_wg - 1) / per_wg * 64;
    }
    const DecodePlan plan = decode_plan_for(a);
    // grid x: (sequence, key/value head, split); y: blocks of 16 query heads
    const int64_t main_items = static_cast<int64_t>(a.B) * a.Hkv * plan.splits * 64 * plan.waves;
    // the combine kernel: 256-lane workgroups of 4 rows
    const int64_t combine_items = plan.splits > 1 ? (rows + 3) / 4 * 256 : 0;
    return main_items > combine_items ? main_items : combine_items;
}
}  // namespace swa

namespace {

size_t decode_ws_bytes(int nmaps, int B, int Hq, int Hkv, int dv, int window, int n_sink) {
    if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || !head_dim_ok(dv) || window < 1 ||
        window > SWA_MAX_N || n_sink < 0 || n_sink > SWA_MAX_N)
        return 0;
    const swa::DecodePlan plan = swa::decode_plan(B, Hkv * swa::decode_head_blocks(Hq, Hkv), window + n_sink);
    if (plan.splits == 1)
        return 0;  // the workgroups write the output directly
    // per (sequence, query head, split, map): running max and sum (section
    // padded to 16 bytes), then dv partial sums; all fp32
    const int64_t parts = static_cast<int64_t>(B) * Hq * plan.splits * nmaps;
    return static_cast<size_t>(swa::decode_ws_ml_floats(parts) + parts * dv) * sizeof(float);
}

// Checks shared by the decode entry points, all but the workspace's; fills
// nothing on failure.
int decode_arg_checks(const swa::DecodeArgs &a, int dt, int stride) {
    for (int m = 0; m < a.nmaps; ++m) {
        if (!aligned16(a.q[m]) || !aligned16(a.k_ring[m]))
            return SWA_ERR_INVALID_ARG;
        if (a.n_sink > 0 && !aligned16(a.k_sink[m]))
            return SWA_ERR_INVALID_ARG;
    }
    if (!aligned16(a.v_ring) || !aligned16(a.out) || (a.n_sink > 0 && !aligned16(a.v_sink)))
        return SWA_ERR_INVALID_ARG;
    if (a.seq_len != nullptr && (reinterpret_cast<uintptr_t>(a.seq_len) & 3u) != 0)
        return SWA_ERR_INVALID_ARG;
    if (dt != SWA_F32 && dt != SWA_BF16)
        return SWA_ERR_INVALID_ARG;
    if (!std::isfinite(a.scale) || !(a.scale > 0.f) || !std::isfinite(a.lambda))
        return SWA_ERR_INVALID_ARG;
    if (a.B < 1 || a.Hq < 1 || a.Hkv < 1 || a.Hq % a.Hkv != 0 || a.window < 1 ||
        a.window > SWA_MAX_N || a.n_sink < 0 || a.n_sink > SWA_MAX_N || stride < 0 ||
        (a.seq_len == nullptr && a.N < 0))
        return SWA_ERR_INVALID_ARG;
    if (static_cast<int64_t>(a.B) * a.Hkv * (a.window + a.n_sink) > INT32_MAX ||
        static_cast<int64_t>(a.B) * a.Hq > INT32_MAX)
        return SWA_ERR_UNSUPPORTED;
    if (!head_dim_ok(a.d) || !head_dim_ok(a.dv))
        return SWA_ERR_UNSUPPORTED;
    if (stride != 0)
        return SWA_ERR_UNSUPPORTED;  // stride keys older than the window are not in the ring
    if (swa::decode_launch_items(a, dt) > swa::kMaxGridItems)
        return SWA_ERR_UNSUPPORTED;  // more work-items than one dispatch holds
    if (dt == SWA_BF16 && swa::decode_head_blocks(a.Hq, a.Hkv) > 65535)
        return SWA_ERR_UNSUPPORTED;  // blocks of 16 query heads fill the grid's y dimension
    return SWA_OK;
}

int decode_checks(const swa::DecodeArgs &a, int dt, int stride, size_t workspace_bytes) {
    int st = decode_arg_checks(a, dt, stride);
    if (st != SWA_OK)
        return st;
    const size_t need = decode_ws_bytes(a.nmaps, a.B, a.Hq, a.Hkv, a.dv, a.window, a.n_sink);
    if (need > 0 && (a.workspace == nullptr || !aligned16(a.workspace) || workspace_bytes < need))
        return SWA_ERR_WORKSPACE;
    return SWA_OK;
}

int decode_run(const swa::DecodeArgs &a, int dt, int stride, size_t workspace_bytes,
               hipStream_t stream) {
    int st = decode_checks(a, dt, stride, workspace_bytes);
    if (st != SWA_OK)
        return st;
    return hip_status(dt == SWA_BF16 ? swa::launch_decode_bf16(a, stream)
                                     : swa::launch_decode_f32(a, stream));
}

}  // namespace

extern "C" {

int swa_tile_config(int op, int dt, int d, int dv, int32_t *bm, int32_t *bn) {
    if ((op != SWA_OP_ATTN && op != SWA_OP_DIFF) || (dt != SWA_F32 && dt != SWA_BF16) ||
        !head_dim_ok(d) || !head_dim_ok(dv) || !bm || !bn)
        return SWA_ERR_INVALID_ARG;
    *bm = swa::tile_rows(op, dt);
    *bn = kBN;
    return SWA_OK;
}

int swa_block_mask_query(int N, int window, int stride, int dilation, int n_global, int bm, int bn,
                         int32_t *num_q_tiles, int32_t *nnz) {
    if (!num_q_tiles || !nnz)
        return SWA_ERR_INVALID_ARG;
    return mask_query(N, window, stride, dilation, n_global, bm, bn, num_q_tiles, nnz);
}

int swa_block_mask_build(const swa_block_mask_t *mask, hipStream_t stream) {
    if (!mask)
        return SWA_ERR_INVALID_ARG;
    int32_t nq = 0, nnz = 0;
    int st = mask_query(mask->N, mask->window, mask->stride, mask->dilation, mask->n_global,
                        mask->bm, mask->bn, &nq, &nnz);
    if (st != SWA_OK)
        return st;
    if (mask->num_q_tiles != nq || mask->nnz != nnz || !mask_arrays_ok(mask))
        return SWA_ERR_INVALID_ARG;
    return hip_status(swa::launch_block_mask_build(*mask, stream));
}

int swa_mask_dense(int N, int window, int stride, int dilation, int n_global, uint8_t *out,
                   hipStream_t stream) {
    if (N < 1 || N > 16384 || window < 1 || stride < 0 || dilation < 1 || n_global < 0 ||
        out == nullptr)
        return SWA_ERR_INVALID_ARG;
    return hip_status(swa::launch_mask_dense(N, window, stride, dilation, n_global, out, stream));
}

int swa_attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
                 int dt, int B, int Hq, int Hkv, int N, int d, int window, int stride,
                 int dilation, int n_global, float scale, const swa_block_mask_t *mask,
                 hipStream_t stream) {
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
        return SWA_ERR_INVALID_ARG;
    if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
        return SWA_ERR_INVALID_ARG;
    if (dt != SWA_F32 && dt != SWA_BF16)
        return SWA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f))
        return SWA_ERR_INVALID_ARG;
    int st = check_sizes(B, Hq, Hkv, N, window, stride, dilation, n_global);
    if (st != SWA_OK)
        return st;
    if (!head_dim_ok(d))
        return SWA_ERR_UNSUPPORTED;
    st = check_mask(mask, N, window, stride, dilation, n_global, swa::tile_rows(SWA_OP_ATTN, dt));
    if (st != SWA_OK)
        return st;
    swa::FwdArgs a{};
    a.q[0] = q;
    a.k[0] = k;
    a.v = v;
    a.out = out;
    a.lse = lse;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.dv = d;
    a.window = window;
    a.stride = stride;
    a.dilation = dilation;
    a.n_global = n_global;
    a.scale = scale;
    a.lambda = 0.f;
    a.nmaps = 1;
    a.mask = view_of(mask);
    return fwd_run(a, dt, stream);
}

size_t swa_attn_decode_workspace_bytes(int op, int B, int Hq, int Hkv, int dv, int window,
                                       int n_sink) {
    if (op != SWA_OP_ATTN && op != SWA_OP_DIFF)
        return 0;
    return decode_ws_bytes(op == SWA_OP_DIFF ? 2 : 1, B, Hq, Hkv, dv, window, n_sink);
}

int swa_attn_decode(const void *q, const void *k_ring, const void *v_ring, void *out,
                    const int32_t *seq_len, void *workspace, size_t workspace_bytes,
                    int dt, int B, int Hq, int Hkv, int N, int d, int window, int stride,
                    float scale, hipStream_t stream) {
    swa::DecodeArgs a{};
    a.q[0] = q;
    a.k_ring[0] = k_ring;
    a.v_ring = v_ring;
    a.out = out;
    a.seq_len = seq_len;
    a.workspace = workspace;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.dv = d;
    a.window = window;
    a.n_sink = 0;
    a.nmaps = 1;
    a.scale = scale;
    a.lambda = 0.f;
    return decode_run(a, dt, stride, workspace_bytes, stream);
}

int swa_attn_decode_noalloc(const void *q, const void *k_ring, const void *v_ring, void *out,
                            const int32_t *seq_len, int dt, int B, int Hq, int Hkv,
                            int N, int d, int window, int stride, float scale,
                            hipStream_t stream) {
    swa::DecodeArgs a{};
    a.q[0] = q;
    a.k_ring[0] = k_ring;
    a.v_ring = v_ring;
    a.out = out;
    a.seq_len = seq_len;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.dv = d;
    a.window = window;
    a.n_sink = 0;
    a.nmaps = 1;
    a.scale = scale;
    a.lambda = 0.f;
    // every check, the scratch bound included, before the first HIP call
    int st = decode_arg_checks(a, dt, stride);
    if (st != SWA_OK)
        return st;
    const size_t need = decode_ws_bytes(a.nmaps, a.B, a.Hq, a.Hkv, a.dv, a.window, a.n_sink);
    if (need > SWA_DECODE_SCRATCH_BYTES)
        return SWA_ERR_SCRATCH;
    if (need > 0) {
        st = hip_status(swa::decode_static_scratch(&a.workspace));
        if (st != SWA_OK)
            return st;
    }
    return decode_run(a, dt, stride, need > 0 ? SWA_DECODE_SCRATCH_BYTES : 0, stream);
}

int swa_attn_decode_sinks(const void *q, const void *k_sink, const void *v_sink, int n_sink,
                          const void *k_ring, const void *v_ring, void *out,
                          const int32_t *seq_len, void *workspace, size_t workspace_bytes,
                          int dt, int B, int Hq, int Hkv, int N, int d, int window,
                          float scale, hipStream_t stream) {
    swa::DecodeArgs a{};
    a.q[0] = q;
    a.k_ring[0] = k_ring;
    a.v_ring = v_ring;
    a.k_sink[0] = k_sink;
    a.v_sink = v_sink;
    a.out = out;
    a.seq_len = seq_len;
    a.workspace = workspace;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.dv = d;
    a.window = window;
    a.n_sink = n_sink;
    a.nmaps = 1;
    a.scale = scale;
    a.lambda = 0.f;
    return decode_run(a, dt, 0, workspace_bytes, stream);
}

int diff_attn_decode(const void *q1, const void *k1_ring, const void *q2, const void *k2_ring,
                     const void *v_ring, void *out, const int32_t *seq_len, void *workspace,
                     size_t workspace_bytes, int dt, int B, int Hq, int Hkv, int N, int d,
                     int dv, int window, float scale, float lambda, hipStream_t stream) {
    swa::DecodeArgs a{};
    a.q[0] = q1;
    a.q[1] = q2;
    a.k_ring[0] = k1_ring;
    a.k_ring[1] = k2_ring;
    a.v_ring = v_ring;
    a.out = out;
    a.seq_len = seq_len;
    a.workspace = workspace;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.dv = dv;
    a.window = window;
    a.n_sink = 0;
    a.nmaps = 2;
    a.scale = scale;
    a.lambda = lambda;
    return decode_run(a, dt, 0, workspace_bytes, stream);
}

int diff_attn_fwd(const void *q1, const void *k1, const void *q2, const void *k2, const void *v,
                  void *out, int dt, int B, int Hq, int Hkv, int N, int d, int dv,
                  int window, int stride, int dilation, int n_global, float scale, float lambda,
                  const swa_block_mask_t *mask, hipStream_t stream) {
    if (!aligned16(q1) || !aligned16(k1) || !aligned16(q2) || !aligned16(k2) || !aligned16(v) ||
        !aligned16(out))
        return SWA_ERR_INVALID_ARG;
    if (dt != SWA_F32 && dt != SWA_BF16)
        return SWA_ERR_INVALID_ARG;
    if (!std::isfinite(scale) || !(scale > 0.f) || !std::isfinite(lambda))
        return SWA_ERR_INVALID_ARG;
    int st = check_sizes(B, Hq, Hkv, N, window, stride, dilation, n_global);
    if (st != SWA_OK)
        return st;
    if (!head_dim_ok(d) || !head_dim_ok(dv))
        return SWA_ERR_UNSUPPORTED;
    st = check_mask(mask, N, window, stride, dilation, n_global, swa::tile_rows(SWA_OP_DIFF, dt));
    if (st != SWA_OK)
        return st;
    swa::FwdArgs a{};
    a.q[0] = q1;
    a.k[0] = k1;
    a.q[1] = q2;
    a.k[1] = k2;
    a.v = v;
    a.out = out;
    a.lse = nullptr;
    a.B = B;
    a.Hq = Hq;
    a.Hkv = Hkv;
    a.N = N;
    a.d = d;
    a.dv = dv;
    a.window = window;
    a.stride = stride;
    a.dilation = dilation;
    a.n_global = n_global;
    a.scale = scale;
    a.lambda = lambda;
    a.nmaps = 2;
    a.mask = view_of(mask);
    return fwd_run(a, dt, stream);
}

const char *swa_strerror(int status) {
    switch (status) {
    case SWA_OK:
        return "success";
    case SWA_ERR_INVALID_ARG:
        return "invalid argument";
    case SWA_ERR_UNSUPPORTED:
        return "unsupported configuration";
    case SWA_ERR_WORKSPACE:
        return "decode workspace missing or too small";
    case SWA_ERR_HIP:
        return "HIP launch error";
    case SWA_ERR_SCRATCH:
        return "decode needs more scratch than the no-allocation entry point holds "
               "(SWA_DECODE_SCRATCH_BYTES)";
    default:
        return "unknown status";
    }
}

}  // extern "C"
