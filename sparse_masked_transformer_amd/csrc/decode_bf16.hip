// One decode step over a rolling KV window, bf16 on gfx950.
//
// Learn: Sparse & Sliding-Window Attention, §4 and §6: decoding keeps only
// the last `window` tokens' keys and values in a fixed-size rolling buffer
// (position p in slot p mod window), so the step reads the whole window once
// and is bound by HBM bandwidth; each K and V byte is read exactly once.
//
// Split kernel: one wave per (sequence, key/value head, split of the ring).
//   * The wave streams its slots 32 at a time: coalesced 16-byte loads into
//     registers two steps ahead (two register stages), then into LDS.  LDS
//     rows are padded (K +16 bytes, V +64 bytes) so the 16-byte and the
//     transposed reads are free of bank conflicts.
//   * The G query heads sharing the key/value head form the 16 columns of a
//     v_mfma_f32_16x16x32_bf16 (unused columns are zero): S^T = K Q^T with K
//     from LDS as the A operand; lane l holds head l%16 and keys 4(l/16)+i.
//   * fp32 online softmax in registers (exp2, log2(e) folded into the scale);
//     O^T += V^T P^T with V^T fragments from ds_read_b64_tr_b16.
//   * The split's (max, sum, unnormalised output) go to the workspace.
// Combine kernel: one wave per (sequence, query head) merges the splits:
//   m* = max m_s, l* = sum l_s 2^(m_s - m*), out = sum o_s 2^(m_s - m*) / l*.
#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1e30f;
constexpr int kStepKeys = 32;
constexpr int kMaxSplits = 16;

template <int D>
struct Lay {
    static constexpr int kRow = 2 * D + 16;   // K row stride in LDS, bytes
    static constexpr int vRow = 2 * D + 64;   // V row stride in LDS, bytes
    static constexpr int kTile = kStepKeys * kRow;
    static constexpr int vTile = kStepKeys * vRow;
    static constexpr int chunks = kStepKeys * D / 8 / 64;  // 16-byte chunks per lane per tensor
};

struct SplitParams {
    const __bf16 *q;
    const __bf16 *k;
    const __bf16 *v;
    const int32_t *seq_len;
    float *ws_ml;   // [B*Hq*S][2]  (max in log2 units, sum)
    float *ws_o;    // [B*Hq*S][D]
    int B, Hq, Hkv, N, window, splits, split_len;
    float c;        // scale * log2(e)
};

template <int D>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2, 2)))
void decode_split_kernel(SplitParams p) {
    using Y = Lay<D>;
    __shared__ __attribute__((aligned(16))) char smem[Y::kTile + Y::vTile];

    const int lane = threadIdx.x;
    const int split = blockIdx.x % p.splits;
    const int bg = blockIdx.x / p.splits;
    const int g = bg % p.Hkv, b = bg / p.Hkv;
    const int G = p.Hq / p.Hkv;

    const int L = p.seq_len ? p.seq_len[b] : p.N;
    const int nvalid = L <= 0 ? 0 : (L < p.window ? L : p.window);
    const int s0 = split * p.split_len;
    int s1 = s0 + p.split_len;
    s1 = s1 < nvalid ? s1 : nvalid;
    const int nsteps = s1 > s0 ? (s1 - s0 + kStepKeys - 1) / kStepKeys : 0;

    const int64_t ring = (int64_t)(b * p.Hkv + g) * p.window;
    const __bf16 *kbase = p.k + ring * D;
    const __bf16 *vbase = p.v + ring * D;

    // ---- Q^T fragments: column = query head within the group ----------------
    const int colq = lane & 15, grp = lane >> 4, sl = lane & 15;
    bf16x8 qf[D / 32];
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        if (colq < G)
            qf[ks] = *reinterpret_cast<const bf16x8 *>(
                p.q + ((int64_t)b * p.Hq + g * G + colq) * D + ks * 32 + grp * 8);
        else
            qf[ks] = bf16x8{};
    }

    // A step's K and V rows, 16 bytes per lane per load, consecutive lanes
    // reading consecutive chunks of a row (coalesced); slots past the ring
    // end are clamped (and masked out below).
    u32x4 kst[2][Y::chunks], vst[2][Y::chunks];
    auto load = [&](int st, int reg) {
#pragma unroll
        for (int u = 0; u < Y::chunks; ++u) {
            const int x = lane + 64 * u;
            const int r = x / (D / 8), c = x % (D / 8);
            int slot = s0 + st * kStepKeys + r;
            slot = slot < p.window ? slot : p.window - 1;
            kst[reg][u] = *reinterpret_cast<const u32x4 *>(kbase + (int64_t)slot * D + c * 8);
            vst[reg][u] = *reinterpret_cast<const u32x4 *>(vbase + (int64_t)slot * D + c * 8);
        }
    };
    // one wave: its LDS writes land after its reads of the previous step
    auto store = [&](int reg) {
#pragma unroll
        for (int u = 0; u < Y::chunks; ++u) {
            const int x = lane + 64 * u;
            const int r = x / (D / 8), c = x % (D / 8);
            *reinterpret_cast<u32x4 *>(smem + r * Y::kRow + c * 16) = kst[reg][u];
            *reinterpret_cast<u32x4 *>(smem + Y::kTile + r * Y::vRow + c * 16) = vst[reg][u];
        }
    };

    f32x4 o[D / 16];
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
        o[db] = f32x4{};
    float m_run = kNegBig, l_run = 0.f;

    // per-lane LDS read bases (the rest are compile-time offsets)
    const char *kb = smem + colq * Y::kRow + grp * 16;
    const char *vb = smem + Y::kTile + (4 * grp + (sl >> 2)) * Y::vRow + 4 * (sl & 3) * 2;

    auto compute = [&](int st) {
        // ---- S^T = K Q^T for two 16-key blocks -----------------------------
        f32x4 s[2];
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk) {
            f32x4 acc = f32x4{};
#pragma unroll
            for (int ks = 0; ks < D / 32; ++ks) {
                const bf16x8 a = *reinterpret_cast<const bf16x8 *>(kb + kbk * 16 * Y::kRow + ks * 64);
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], acc, 0, 0, 0);
            }
            s[kbk] = acc;
        }
        // ---- mask slots past the valid range -------------------------------
        const int base_slot = s0 + st * kStepKeys;
        if (base_slot + kStepKeys > s1) {
#pragma unroll
            for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    s[kbk][i] = base_slot + kbk * 16 + grp * 4 + i < s1 ? s[kbk][i] : -__builtin_inff();
        }
        // ---- online softmax (row = query head column) ------------------------
        float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mxs = mx * p.c;
        if (mxs > m_run) {
            const float alpha = __builtin_amdgcn_exp2f(m_run - mxs);
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < D / 16; ++db)
                o[db] *= alpha;
            m_run = mxs;
        }
        bf16x8 pf;
#pragma unroll
        for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = __builtin_amdgcn_exp2f(fmaf(s[kbk][i], p.c, -m_run));
                l_run += pv;
                pf[kbk * 4 + i] = (__bf16)pv;
            }
        // ---- O^T += V^T P^T -------------------------------------------------
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
            const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vb + db * 32));
            const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vb + 16 * Y::vRow + db * 32));
            const bf16x4 a0 = __builtin_bit_cast(bf16x4, t0);
            const bf16x4 a1 = __builtin_bit_cast(bf16x4, t1);
            const bf16x8 va = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            o[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, o[db], 0, 0, 0);
        }
    };

    // two register stages: steps st (even) and st+1 (odd) alternate
    if (nsteps > 0)
        load(0, 0);
    if (nsteps > 1)
        load(1, 1);
    for (int st = 0; st < nsteps; st += 2) {
        store(0);
        if (st + 2 < nsteps)
            load(st + 2, 0);
        compute(st);
        if (st + 1 < nsteps) {
            store(1);
            if (st + 3 < nsteps)
                load(st + 3, 1);
            compute(st + 1);
        }
    }

    // ---- partial results of this split ---------------------------------------
    float lt = l_run + __shfl_xor(l_run, 16);
    lt += __shfl_xor(lt, 32);
    if (colq < G) {
        const int64_t row = ((int64_t)b * p.Hq + g * G + colq) * p.splits + split;
        if (grp == 0) {
            p.ws_ml[row * 2] = m_run;
            p.ws_ml[row * 2 + 1] = lt;
        }
#pragma unroll
        for (int db = 0; db < D / 16; ++db)
            *reinterpret_cast<f32x4 *>(p.ws_o + row * D + db * 16 + grp * 4) = o[db];
    }
}

// One wave per (sequence, query head).  All split partials are loaded up
// front (the split count is at most kMaxSplits), so the loads overlap.
template <int D>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float *ws_ml, const float *ws_o,
                                                             __bf16 *out, int rows, int splits) {
    constexpr int kPerLane = (D + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // (b, query head)
    if (row >= rows)
        return;
    float ms[kMaxSplits], ls[kMaxSplits], os[kMaxSplits][kPerLane];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        const int64_t r = (int64_t)row * splits + (s < splits ? s : 0);
        ms[s] = s < splits ? ws_ml[r * 2] : kNegBig;
        ls[s] = s < splits ? ws_ml[r * 2 + 1] : 0.f;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            os[s][i] = (s < splits && lane + 64 * i < D) ? ws_o[r * D + lane + 64 * i] : 0.f;
    }
    float mstar = kNegBig;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s)
        mstar = fmaxf(mstar, ms[s]);
    float lsum = 0.f, acc[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
        acc[i] = 0.f;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        const float wgt = __builtin_amdgcn_exp2f(ms[s] - mstar);
        lsum += wgt * ls[s];
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            acc[i] += wgt * os[s][i];
    }
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
        if (lane + 64 * i < D)
            out[(int64_t)row * D + lane + 64 * i] = (__bf16)(acc[i] * inv);
}

template <int D>
hipError_t launch(const DecodeArgs &a, hipStream_t stream) {
    SplitParams p;
    p.q = static_cast<const __bf16 *>(a.q);
    p.k = static_cast<const __bf16 *>(a.k_ring);
    p.v = static_cast<const __bf16 *>(a.v_ring);
    p.seq_len = a.seq_len;
    p.splits = decode_splits(a.window);
    p.split_len = ((a.window + p.splits - 1) / p.splits + kStepKeys - 1) / kStepKeys * kStepKeys;
    const int64_t rows = (int64_t)a.B * a.Hq;
    p.ws_ml = static_cast<float *>(a.workspace);
    p.ws_o = p.ws_ml + (rows * p.splits * 2 + 3) / 4 * 4;  // 16-byte aligned section
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.N = a.N;
    p.window = a.window;
    p.c = a.scale * kLog2e;
    unsigned grid = static_cast<unsigned>((int64_t)a.B * a.Hkv * p.splits);
    hipLaunchKernelGGL(decode_split_kernel<D>, dim3(grid), dim3(64), 0, stream, p);
    hipLaunchKernelGGL(decode_combine_kernel<D>, dim3(static_cast<unsigned>((rows + 3) / 4)),
                       dim3(256), 0, stream, p.ws_ml, p.ws_o, static_cast<__bf16 *>(a.out),
                       static_cast<int>(rows), p.splits);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t stream) {
    static_assert(kMaxSplits >= 16, "decode_splits() returns at most 16");
    switch (a.d) {
    case 32: return launch<32>(a, stream);
    case 64: return launch<64>(a, stream);
    case 128: return launch<128>(a, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace swa
