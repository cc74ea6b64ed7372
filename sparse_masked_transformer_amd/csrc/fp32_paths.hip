// fp32 paths: masked attention forward (one or two maps) and window decode
// with fp32 inputs, fp32 arithmetic and fp32 outputs.  These serve small
// fp32 problems; they are simple rather than fast.
//
// Forward: one thread per query row of a 128-row query tile walks the tiles
// the block mask lists (prefix keys first, then band tiles), staging
// 16 keys at a time in LDS, with a per-key online softmax
// (Attention Variants Compared, "Flash style softmax").
// Decode: one thread per (sequence, query head) over the sink and ring slots.
#include "swa_internal.h"

namespace swa {
namespace {

constexpr int kSub = 16;  // keys staged per LDS step

template <int D, int DV, int NMAPS>
__global__ __launch_bounds__(kF32BM) void fwd_f32_kernel(const float *q0p, const float *k0p,
                                                      const float *q1p, const float *k1p,
                                                      const float *vp, float *out, float *lse,
                                                      MaskView mask, int Hq, int Hkv, int N,
                                                      int window, int stride, int dilation,
                                                      int n_global, float scale, float lambda) {
    __shared__ float ks[NMAPS][kSub][D];
    __shared__ float vs[kSub][DV];
    const float *qp[2] = {q0p, q1p};
    const float *kp[2] = {k0p, k1p};

    const int nq = mask.num_q_tiles;
    const int qt = blockIdx.x % nq;
    const int bh = blockIdx.x / nq;
    const int h = bh % Hq, b = bh / Hq;
    const int g = h / (Hq / Hkv);
    const int i = qt * kF32BM + threadIdx.x;
    const int irow = i < N ? i : N - 1;

    float qr[NMAPS][D], o[NMAPS][DV], m[NMAPS], l[NMAPS];
    for (int mp = 0; mp < NMAPS; ++mp) {
        const float *src = qp[mp] + ((int64_t)bh * N + irow) * D;
        for (int c = 0; c < D; ++c)
            qr[mp][c] = src[c];
        for (int c = 0; c < DV; ++c)
            o[mp][c] = 0.f;
        m[mp] = -__builtin_inff();
        l[mp] = 0.f;
    }

    const int sk = mask.prefix_keys[qt];
    const int n_pre = (sk + kBN - 1) / kBN;
    const int band0 = mask.band_begin[qt];
    const int n_items = n_pre + (mask.row_ptr[qt + 1] - band0);
    const int64_t kvh = (int64_t)(b * Hkv + g) * N;

    for (int it = 0; it < n_items; ++it) {
        const bool pre = it < n_pre;
        const int key0 = pre ? 0 : mask.kv_tile[band0 + it - n_pre] * kBN;
        for (int sub = 0; sub < kBN / kSub; ++sub) {
            // stage kSub keys: key index and whether it exists
            for (int x = threadIdx.x; x < kSub * (NMAPS * D + DV); x += blockDim.x) {
                int r = x % kSub, c = x / kSub;
                int kk = sub * kSub + r;
                int j = pre ? (it * kBN + kk < sk ? prefix_key(it * kBN + kk, sk, stride, n_global) : 0)
                            : (key0 + kk < N ? key0 + kk : N - 1);
                if (c < NMAPS * D)
                    ks[c / D][r][c % D] = kp[c / D][(kvh + j) * D + c % D];
                else
                    vs[r][c - NMAPS * D] = vp[(kvh + j) * DV + (c - NMAPS * D)];
            }
            __syncthreads();
            for (int r = 0; r < kSub; ++r) {
                int kk = sub * kSub + r;
                bool ok;
                if (pre) {
                    ok = it * kBN + kk < sk;
                } else {
                    const int j = key0 + kk, dist = i - j;
                    ok = j < N && j <= i &&
                         ((dist % dilation == 0 && dist / dilation < window) ||
                          (stride > 0 && j % stride == 0) || j < n_global);
                }
                if (!ok)
                    continue;
                for (int mp = 0; mp < NMAPS; ++mp) {
                    float s = 0.f;
                    for (int c = 0; c < D; ++c)
                        s = fmaf(qr[mp][c], ks[mp][r][c], s);
                    s *= scale;
                    float mn = fmaxf(m[mp], s);
                    float alpha = expf(m[mp] - mn);  // m = -inf on the first key -> 0
                    float e = expf(s - mn);
                    l[mp] = l[mp] * alpha + e;
                    for (int c = 0; c < DV; ++c)
                        o[mp][c] = fmaf(o[mp][c], alpha, e * vs[r][c]);
                    m[mp] = mn;
                }
            }
            __syncthreads();
        }
    }
    if (i >= N)
        return;
    float *dst = out + ((int64_t)bh * N + i) * DV;
    for (int c = 0; c < DV; ++c) {
        float x = o[0][c] / l[0];
        if (NMAPS == 2)
            x -= lambda * (o[NMAPS - 1][c] / l[NMAPS - 1]);
        dst[c] = x;
    }
    if (NMAPS == 1 && lse != nullptr)
        lse[(int64_t)bh * N + i] = m[0] + logf(l[0]);
}

// One thread per (sequence, query head): the sink slots the ring no longer
// covers, then the valid ring slots, each with a per-key online softmax per
// map; out = o1 / l1 - lambda * o2 / l2 for two maps.
template <int D, int DV, int NMAPS>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
    const int row = blockIdx.x * blockDim.x + threadIdx.x;  // b * Hq + h
    if (row >= a.B * a.Hq)
        return;
    const int b = row / a.Hq, h = row % a.Hq, g = h / (a.Hq / a.Hkv);
    const int L = a.seq_len ? a.seq_len[b] : a.N;
    const int nvalid = L <= 0 ? 0 : (L < a.window ? L : a.window);
    const int first = L - a.window > 0 ? L - a.window : 0;
    const int s_eff = first < a.n_sink ? first : a.n_sink;
    const int64_t kv = static_cast<int64_t>(b) * a.Hkv + g;
    float o[NMAPS][DV], m[NMAPS], l[NMAPS];
    for (int mp = 0; mp < NMAPS; ++mp) {
        for (int c = 0; c < DV; ++c)
            o[mp][c] = 0.f;
        m[mp] = -__builtin_inff();
        l[mp] = 0.f;
    }
    for (int t = 0; t < s_eff + nvalid; ++t) {
        const bool in_sink = t < s_eff;
        const int64_t r = in_sink ? kv * a.n_sink + t : kv * a.window + (t - s_eff);
        const float *vrow = static_cast<const float *>(in_sink ? a.v_sink : a.v_ring) + r * DV;
        for (int mp = 0; mp < NMAPS; ++mp) {
            const float *qv = static_cast<const float *>(a.q[mp]) + static_cast<int64_t>(row) * D;
            const float *krow = static_cast<const float *>(in_sink ? a.k_sink[mp] : a.k_ring[mp]) + r * D;
            float s = 0.f;
            for (int c = 0; c < D; ++c)
                s = fmaf(qv[c], krow[c], s);
            s *= a.scale;
            const float mn = fmaxf(m[mp], s);
            const float alpha = expf(m[mp] - mn);  // m = -inf on the first key -> 0
            const float e = expf(s - mn);
            l[mp] = l[mp] * alpha + e;
            for (int c = 0; c < DV; ++c)
                o[mp][c] = fmaf(o[mp][c], alpha, e * vrow[c]);
            m[mp] = mn;
        }
    }
    float *dst = static_cast<float *>(a.out) + static_cast<int64_t>(row) * DV;
    for (int c = 0; c < DV; ++c) {
        float x = l[0] > 0.f ? o[0][c] / l[0] : 0.f;
        if (NMAPS == 2)
            x -= a.lambda * (l[NMAPS - 1] > 0.f ? o[NMAPS - 1][c] / l[NMAPS - 1] : 0.f);
        dst[c] = x;
    }
}

template <int D, int DV, int NMAPS>
hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream) {
    unsigned grid = static_cast<unsigned>(a.mask.num_q_tiles) * a.Hq * a.B;
    hipLaunchKernelGGL((fwd_f32_kernel<D, DV, NMAPS>), dim3(grid), dim3(kF32BM), 0, stream,
                       static_cast<const float *>(a.q[0]), static_cast<const float *>(a.k[0]),
                       static_cast<const float *>(a.q[1]), static_cast<const float *>(a.k[1]),
                       static_cast<const float *>(a.v), static_cast<float *>(a.out), a.lse, a.mask,
                       a.Hq, a.Hkv, a.N, a.window, a.stride, a.dilation, a.n_global, a.scale,
                       a.lambda);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs &a, hipStream_t stream) {
#define SWA_F32_CASE(DQ, DVV)                                                   \
    if (a.d == DQ && a.dv == DVV)                                               \
        return a.nmaps == 1 ? launch_fwd<DQ, DVV, 1>(a, stream)                 \
                            : launch_fwd<DQ, DVV, 2>(a, stream);
    SWA_F32_CASE(32, 32)
    SWA_F32_CASE(32, 64)
    SWA_F32_CASE(32, 128)
    SWA_F32_CASE(64, 32)
    SWA_F32_CASE(64, 64)
    SWA_F32_CASE(64, 128)
    SWA_F32_CASE(128, 32)
    SWA_F32_CASE(128, 64)
    SWA_F32_CASE(128, 128)
#undef SWA_F32_CASE
    return hipErrorInvalidValue;
}

hipError_t launch_decode_f32(const DecodeArgs &a, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>((static_cast<int64_t>(a.B) * a.Hq + 63) / 64);
#define SWA_DEC_CASE(DQ, DVV)                                                            \
    if (a.d == DQ && a.dv == DVV) {                                                      \
        if (a.nmaps == 1)                                                                \
            hipLaunchKernelGGL((decode_f32_kernel<DQ, DVV, 1>), dim3(grid), dim3(64), 0, \
                               stream, a);                                               \
        else                                                                             \
            hipLaunchKernelGGL((decode_f32_kernel<DQ, DVV, 2>), dim3(grid), dim3(64), 0, \
                               stream, a);                                               \
        return hipGetLastError();                                                        \
    }
    SWA_DEC_CASE(32, 32)
    SWA_DEC_CASE(32, 64)
    SWA_DEC_CASE(32, 128)
    SWA_DEC_CASE(64, 32)
    SWA_DEC_CASE(64, 64)
    SWA_DEC_CASE(64, 128)
    SWA_DEC_CASE(128, 32)
    SWA_DEC_CASE(128, 64)
    SWA_DEC_CASE(128, 128)
#undef SWA_DEC_CASE
    return hipErrorInvalidValue;
}

}  // namespace swa
