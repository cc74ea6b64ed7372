// fp32 paths: masked attention forward (one or two maps) and window decode
// with fp32 inputs, fp32 arithmetic and fp32 outputs.  These serve small
// fp32 problems; they are simple rather than fast.
//
// Both kernels give each query row kTPR = 8 adjacent lanes.  Lane t of a row
// owns the float4 groups t, t + 8, t + 16, ... of q, k, v and o, so a row
// keeps (NMAPS * d + dv) / 8 floats per lane in registers at every head size,
// and the 8 lanes of a row read 128 contiguous bytes of a staged key.  A score
// is the sum of the 8 lanes' partial dot products (xor shuffles).
//
// Forward: a 32-row query tile (256 lanes) walks the tiles the block mask
// lists (prefix keys first, then band tiles), staging 16 to 64 keys at a time
// in LDS (more for smaller heads) with the next step's loads in flight, and
// updates an online softmax once per block of 16 keys (8 with two maps)
// (Attention Variants Compared, "Flash style softmax").
// Decode: one row per (sequence, query head) over the sink and ring slots.
#include "swa_internal.h"

namespace swa {
namespace {

// Keys staged per LDS step, for kw float4 groups of K and V per key: at most
// 16 KiB per step, so that small heads walk a key tile in few steps (each
// step costs a barrier and a load latency).
constexpr int sub_keys(int kw) { return kw <= 16 ? 64 : (kw <= 32 ? 32 : 16); }
// 16 bytes as a native vector (arrays of HIP's float4 struct are kept in
// scratch memory rather than in registers)
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kTPR = kF32TPR;            // lanes per query row
constexpr int kF32Threads = kFwdThreads;   // lanes per forward workgroup

__device__ inline float dot4(f32x4v a, f32x4v b, float acc) {
    acc = fmaf(a.x, b.x, acc);
    acc = fmaf(a.y, b.y, acc);
    acc = fmaf(a.z, b.z, acc);
    return fmaf(a.w, b.w, acc);
}

template <int CTRL> __device__ inline float dpp(float x) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL,
                                                                 0xF, 0xF, false));
}

// Sum over the kTPR = 8 adjacent lanes of a row, every lane getting the sum:
// lane pairs (quad_perm 1,0,3,2), then quad halves (quad_perm 2,3,0,1), then
// the two quads of the 8-lane half row (row_half_mirror maps lane k to 7 - k,
// which lies in the other quad).
__device__ inline float row_sum(float x) {
    x += dpp<0xB1>(x);
    x += dpp<0x4E>(x);
    x += dpp<0x141>(x);
    return x;
}

__device__ inline void fma4(f32x4v &acc, float e, f32x4v v) {
    acc.x = fmaf(e, v.x, acc.x);
    acc.y = fmaf(e, v.y, acc.y);
    acc.z = fmaf(e, v.z, acc.z);
    acc.w = fmaf(e, v.w, acc.w);
}

// Staging of the forward kernel's K and V rows, one step of kSub keys at a
// time.  A step's kSub * KW float4 groups are spread over the workgroup:
// group c of a key is K of map c / (D/4) below NMAPS * D/4, else V.  Slot u
// of a lane holds group x = lane + u * threads; where a step is not a whole
// number of workgroup rows, the lanes past its end repeat its last group
// (same value, same LDS address).  Plain functions rather than lambdas that
// capture one another: through a chain of captured closures the compiler
// kept the staged registers in scratch memory.
template <int kSub, int KW>
__device__ __forceinline__ int stage_slot(int u) {
    const int x = static_cast<int>(threadIdx.x) + u * kF32Threads;
    return (kSub * KW) % kF32Threads == 0 || x < kSub * KW ? x : kSub * KW - 1;
}

// First key of step s (prefix items count their keys from 0).
template <int kSub>
__device__ __forceinline__ int step_key0(int s, int n_pre, const int32_t *kv_tile, int band0) {
    const int it = s / (kBN / kSub), sub = s % (kBN / kSub);
    return it < n_pre ? it * kBN + sub * kSub : kv_tile[band0 + it - n_pre] * kBN + sub * kSub;
}

// Loads of one step's groups into registers, one load per slot through a
// selected row pointer (no branch on the group's kind).
template <int D, int DV, int NMAPS, int kSub, int KW, int PER>
__device__ __forceinline__ void fetch_step(f32x4v (&stage)[PER], int key0, bool pre, int sk, int stride,
                                           int n_global, int N, int64_t kvh, const float *k0p,
                                           const float *k1p, const float *vp) {
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int x = stage_slot<kSub, KW>(u);
        const int r = x / KW, c = x % KW;
        const int kk = key0 + r;
        const int j = pre ? (kk < sk ? prefix_key(kk, sk, stride, n_global) : 0) : (kk < N ? kk : N - 1);
        const bool is_k = c < NMAPS * D / 4;
        const float *base = is_k ? (c < D / 4 ? k0p : k1p) : vp;
        const int width = is_k ? D : DV;
        const int col = is_k ? c % (D / 4) : c - NMAPS * D / 4;
        stage[u] = reinterpret_cast<const f32x4v *>(base + (kvh + j) * width)[col];
    }
}

template <int D, int DV, int NMAPS>
__global__ __launch_bounds__(kF32Threads) void fwd_f32_kernel(const float *q0p, const float *k0p,
                                                           const float *q1p, const float *k1p,
                                                           const float *vp, float *out, float *lse,
                                                           MaskView mask, int Hq, int Hkv, int N,
                                                           int window, int stride, int dilation,
                                                           int n_global, float scale, float lambda) {
    static_assert(D % (4 * kTPR) == 0 && DV % (4 * kTPR) == 0, "head sizes are multiples of 32");
    constexpr int QG = D / 4 / kTPR, VG = DV / 4 / kTPR;   // float4 groups per lane
    constexpr int KW = NMAPS * D / 4 + DV / 4;             // float4 groups per staged key
    constexpr int kSub = sub_keys(KW);                     // keys per LDS step
    static_assert(kBN % kSub == 0, "steps tile a key tile");
    constexpr int PER = (kSub * KW + kF32Threads - 1) / kF32Threads;
    __shared__ f32x4v ks[NMAPS][kSub][D / 4];
    __shared__ f32x4v vs[kSub][DV / 4];

    const int nq = mask.num_q_tiles;
    const int qt = blockIdx.x % nq;
    const int bh = blockIdx.x / nq;
    const int h = bh % Hq, b = bh / Hq;
    const int g = h / (Hq / Hkv);
    const int t = threadIdx.x % kTPR;
    const int i = qt * kF32BM + static_cast<int>(threadIdx.x) / kTPR;
    const int irow = i < N ? i : N - 1;
    // earliest key of the dilated window (clamped: keys are >= 0)
    const int64_t lo64 = static_cast<int64_t>(i) - static_cast<int64_t>(window - 1) * dilation;
    const int lo = lo64 > -1 ? static_cast<int>(lo64) : -1;

    f32x4v qr[NMAPS][QG], o[NMAPS][VG];
    float m[NMAPS], l[NMAPS];
#pragma unroll
    for (int mp = 0; mp < NMAPS; ++mp) {
        const f32x4v *src = reinterpret_cast<const f32x4v *>((mp == 0 ? q0p : q1p) + ((int64_t)bh * N + irow) * D);
#pragma unroll
        for (int k = 0; k < QG; ++k)
            qr[mp][k] = src[t + kTPR * k];
#pragma unroll
        for (int k = 0; k < VG; ++k)
            o[mp][k] = f32x4v{0.f, 0.f, 0.f, 0.f};
        m[mp] = -__builtin_inff();
        l[mp] = 0.f;
    }

    const int sk = mask.prefix_keys[qt];
    const int n_pre = (sk + kBN - 1) / kBN;
    const int band0 = mask.band_begin[qt];
    const int n_items = n_pre + (mask.row_ptr[qt + 1] - band0);
    const int n_steps = n_items * (kBN / kSub);
    const int64_t kvh = (int64_t)(b * Hkv + g) * N;

    f32x4v stage[PER];
    auto fetch = [&](int s) {   // loads of step s, in flight until the next store
        fetch_step<D, DV, NMAPS, kSub, KW, PER>(stage, step_key0<kSub>(s, n_pre, mask.kv_tile, band0),
                                                 s / (kBN / kSub) < n_pre, sk, stride, n_global, N,
                                                 kvh, k0p, k1p, vp);
    };
    if (n_steps > 0)
        fetch(0);
    for (int s = 0; s < n_steps; ++s) {
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int x = stage_slot<kSub, KW>(u);
            const int r = x / KW, c = x % KW;
            const bool is_k = c < NMAPS * D / 4;
            const int ck = is_k ? c : 0, cv = is_k ? 0 : c - NMAPS * D / 4;
            f32x4v *dst = is_k ? &ks[ck / (D / 4)][r][ck % (D / 4)] : &vs[r][cv];
            *dst = stage[u];
        }
        __syncthreads();
        const bool pre = s / (kBN / kSub) < n_pre;
        const int key0 = step_key0<kSub>(s, n_pre, mask.kv_tile, band0);
        if (s + 1 < n_steps)
            fetch(s + 1);   // in flight while this block is processed

        // softmax blocks of KB keys (8 with two maps, to bound live registers)
        constexpr int KB = NMAPS == 2 ? 8 : 16;
#pragma unroll 1
        for (int hb = 0; hb < kSub; hb += KB) {
            // the mask of the KB keys.  Band keys: j <= i, and j in the dilated
            // window (i - j a multiple of dilation and j >= lo), a multiple of
            // stride, or global.  The remainders of i - j by dilation and of j
            // by stride are stepped per key from one division per block; with
            // no stride the stride remainder starts at 1 and never returns to 0.
            bool ok[KB];
            const int jb = key0 + hb;
            if (pre) {
#pragma unroll
                for (int r = 0; r < KB; ++r)
                    ok[r] = jb + r < sk;
            } else {
                const int db = i - jb;
                int dr = db >= 0 ? db % dilation : 0;
                int sr = stride > 0 ? jb % stride : 1;
#pragma unroll
                for (int r = 0; r < KB; ++r) {
                    const int j = jb + r;
                    ok[r] = (j <= i) & (((dr == 0) & (j >= lo)) | (sr == 0) | (j < n_global));
                    dr = dr == 0 ? dilation - 1 : dr - 1;   // remainder of i - (j + 1)
                    sr = sr + 1 == stride ? 0 : sr + 1;       // remainder of j + 1
                }
            }
#pragma unroll
            for (int mp = 0; mp < NMAPS; ++mp) {
                float sc[KB];
                float bmax = -__builtin_inff();
#pragma unroll
                for (int r = 0; r < KB; ++r) {
                    float a = 0.f;
#pragma unroll
                    for (int k = 0; k < QG; ++k)
                        a = dot4(qr[mp][k], ks[mp][hb + r][t + kTPR * k], a);
                    a = row_sum(a);
                    sc[r] = ok[r] ? a * scale : -__builtin_inff();
                    bmax = fmaxf(bmax, sc[r]);
                }
                // no branch on an empty block: with no attended key so far the
                // base is 0, so alpha and every e are exp(-inf) = 0 and o, l stay 0
                const float mn = fmaxf(m[mp], bmax);
                const float base = mn == -__builtin_inff() ? 0.f : mn;
                const float alpha = expf(m[mp] - base);  // m = -inf before the first key -> 0
                l[mp] *= alpha;
#pragma unroll
                for (int k = 0; k < VG; ++k) {
                    o[mp][k].x *= alpha;
                    o[mp][k].y *= alpha;
                    o[mp][k].z *= alpha;
                    o[mp][k].w *= alpha;
                }
#pragma unroll
                for (int r = 0; r < KB; ++r) {
                    const float e = expf(sc[r] - base);   // masked keys: exp(-inf) = 0
                    l[mp] += e;
#pragma unroll
                    for (int k = 0; k < VG; ++k)
                        fma4(o[mp][k], e, vs[hb + r][t + kTPR * k]);
                }
                m[mp] = mn;
            }
        }
        __syncthreads();
    }
    if (i >= N)
        return;
    f32x4v *dst = reinterpret_cast<f32x4v *>(out + ((int64_t)bh * N + i) * DV);
#pragma unroll
    for (int k = 0; k < VG; ++k) {
        const float r0 = 1.f / l[0];
        f32x4v x = f32x4v{o[0][k].x * r0, o[0][k].y * r0, o[0][k].z * r0, o[0][k].w * r0};
        if (NMAPS == 2) {
            const float r1 = lambda / l[NMAPS - 1];
            x.x -= o[NMAPS - 1][k].x * r1;
            x.y -= o[NMAPS - 1][k].y * r1;
            x.z -= o[NMAPS - 1][k].z * r1;
            x.w -= o[NMAPS - 1][k].w * r1;
        }
        dst[t + kTPR * k] = x;
    }
    if (NMAPS == 1 && lse != nullptr && t == 0)
        lse[(int64_t)bh * N + i] = m[0] + logf(l[0]);
}

// One row (8 lanes) per (sequence, query head): the sink slots the ring no
// longer covers, then the valid ring slots, each with a per-key online softmax
// per map; out = o1 / l1 - lambda * o2 / l2 for two maps.
template <int D, int DV, int NMAPS>
__global__ __launch_bounds__(64) void decode_f32_kernel(DecodeArgs a) {
    constexpr int QG = D / 4 / kTPR, VG = DV / 4 / kTPR;
    const int t = threadIdx.x % kTPR;
    const int row0 = blockIdx.x * (64 / kTPR) + static_cast<int>(threadIdx.x) / kTPR;  // b * Hq + h
    const bool live = row0 < a.B * a.Hq;
    const int row = live ? row0 : a.B * a.Hq - 1;   // dead rows mirror the last row, store nothing
    const int b = row / a.Hq, h = row % a.Hq, g = h / (a.Hq / a.Hkv);
    const int L = a.seq_len ? a.seq_len[b] : a.N;
    const int nvalid = L <= 0 ? 0 : (L < a.window ? L : a.window);
    const int first = L - a.window > 0 ? L - a.window : 0;
    const int s_eff = first < a.n_sink ? first : a.n_sink;
    const int64_t kv = static_cast<int64_t>(b) * a.Hkv + g;
    f32x4v qr[NMAPS][QG], o[NMAPS][VG];
    float m[NMAPS], l[NMAPS];
    for (int mp = 0; mp < NMAPS; ++mp) {
        const f32x4v *qv = static_cast<const f32x4v *>(a.q[mp]) + static_cast<int64_t>(row) * (D / 4);
#pragma unroll
        for (int k = 0; k < QG; ++k)
            qr[mp][k] = qv[t + kTPR * k];
#pragma unroll
        for (int k = 0; k < VG; ++k)
            o[mp][k] = f32x4v{0.f, 0.f, 0.f, 0.f};
        m[mp] = -__builtin_inff();
        l[mp] = 0.f;
    }
    for (int s = 0; s < s_eff + nvalid; ++s) {
        const bool in_sink = s < s_eff;
        const int64_t r = in_sink ? kv * a.n_sink + s : kv * a.window + (s - s_eff);
        const f32x4v *vrow = static_cast<const f32x4v *>(in_sink ? a.v_sink : a.v_ring) + r * (DV / 4);
        for (int mp = 0; mp < NMAPS; ++mp) {
            const f32x4v *krow =
                static_cast<const f32x4v *>(in_sink ? a.k_sink[mp] : a.k_ring[mp]) + r * (D / 4);
            float x = 0.f;
#pragma unroll
            for (int k = 0; k < QG; ++k)
                x = dot4(qr[mp][k], krow[t + kTPR * k], x);
            x = row_sum(x) * a.scale;
            const float mn = fmaxf(m[mp], x);
            const float alpha = expf(m[mp] - mn);  // m = -inf on the first key -> 0
            const float e = expf(x - mn);
            l[mp] = l[mp] * alpha + e;
#pragma unroll
            for (int k = 0; k < VG; ++k) {
                const f32x4v v = vrow[t + kTPR * k];
                o[mp][k].x = fmaf(o[mp][k].x, alpha, e * v.x);
                o[mp][k].y = fmaf(o[mp][k].y, alpha, e * v.y);
                o[mp][k].z = fmaf(o[mp][k].z, alpha, e * v.z);
                o[mp][k].w = fmaf(o[mp][k].w, alpha, e * v.w);
            }
            m[mp] = mn;
        }
    }
    if (!live)
        return;
    f32x4v *dst = static_cast<f32x4v *>(a.out) + static_cast<int64_t>(row) * (DV / 4);
#pragma unroll
    for (int k = 0; k < VG; ++k) {
        const float r0 = l[0] > 0.f ? 1.f / l[0] : 0.f;
        f32x4v x = f32x4v{o[0][k].x * r0, o[0][k].y * r0, o[0][k].z * r0, o[0][k].w * r0};
        if (NMAPS == 2) {
            const float r1 = l[NMAPS - 1] > 0.f ? a.lambda / l[NMAPS - 1] : 0.f;
            x.x -= o[NMAPS - 1][k].x * r1;
            x.y -= o[NMAPS - 1][k].y * r1;
            x.z -= o[NMAPS - 1][k].z * r1;
            x.w -= o[NMAPS - 1][k].w * r1;
        }
        dst[t + kTPR * k] = x;
    }
}

template <int D, int DV, int NMAPS>
hipError_t launch_fwd(const FwdArgs &a, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>(fwd_workgroups(a, SWA_F32));
    hipLaunchKernelGGL((fwd_f32_kernel<D, DV, NMAPS>), dim3(grid), dim3(kF32Threads), 0, stream,
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
    constexpr int rows = 64 / kTPR;   // (sequence, head) rows per workgroup
    const unsigned grid = static_cast<unsigned>((static_cast<int64_t>(a.B) * a.Hq + rows - 1) / rows);
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
