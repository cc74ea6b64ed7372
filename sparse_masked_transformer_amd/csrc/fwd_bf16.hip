// Masked causal attention forward on gfx950 matrix cores (bf16 in, fp32
// accumulate), for one score map (sliding window / local+strided prefill) or
// two maps (differential attention).
//
// The operation is A = softmax(Q K^T * scale + log M) V (Learn: Sparse &
// Sliding-Window Attention, §3), computed with the tiled online softmax of
// "Attention Variants Compared" ("Flash style softmax"): the score matrix is
// never written out; each workgroup keeps a running maximum, running sum and
// running weighted sum for its 128 query rows while it walks the key tiles
// the block mask lists.
//
// Workgroup: 256 threads = 4 waves; wave w owns query rows q0 .. q0+31 of the
// 128-row query tile.  Per 64-key tile:
//   * K (and V) tiles are staged HBM -> VGPR -> LDS, double-buffered, with a
//     16-byte-chunk XOR swizzle on every row.
//   * S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (K from LDS as the A operand,
//     Q^T held in registers as the B operand).  In the 32x32 accumulator
//     layout lane l holds query column l%32 and keys (r%4) + 8(r/4) + 4(l/32)
//     of register r, so each lane owns one query row's scores.
//   * The online softmax runs in registers; a row's maximum needs a single
//     exchange with lane l^32.  exp2 with log2(e) folded into the scale; the
//     running maximum is only raised when a tile's maximum exceeds it by more
//     than 8 (log2 units), which keeps every p <= 256 and leaves the result
//     unchanged (softmax is invariant to the reference value).
//   * The probabilities, rounded to bf16, are already in the B-operand layout
//     of O^T += V^T P^T, so they never leave registers.  V stays row-major in
//     LDS and its transposed A-operand fragments come from ds_read_b64_tr_b16.
//   * Tiles a wave's rows cannot see are skipped by that wave; tiles entirely
//     inside every row's window skip the per-cell mask.
// Local+strided problems first visit a dense prefix of stride keys
// (0, s, 2s, ... below the query tile's first window tile), which every row
// of the tile attends, gathered 64 at a time, then the window tiles.
#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;       // log2 units the running maximum may lag
constexpr float kNegBig = -1e30f;    // running maximum before any key
constexpr int kThreads = 256;

__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }

// Byte offset of 16-byte chunk c of row r in a tile of rows with `cols`
// bf16 elements.
template <int COLS>
__device__ __forceinline__ int chunk_off(int r, int c) {
    constexpr int cpr = COLS / 8;
    constexpr int cmask = (cpr < 8 ? cpr : 8) - 1;
    return r * (COLS * 2) + ((c ^ (swz(r) & cmask)) << 4);
}

template <int D, int DV, int NMAPS>
struct Cfg {
    static constexpr int kTile = 64 * D * 2;                  // one K tile, bytes
    static constexpr int vTile = 64 * DV * 2;                 // one V tile, bytes
    static constexpr int buf = NMAPS * kTile + vTile;         // one stage
    static constexpr int chunks = buf / 16;                   // 16-byte chunks per stage
    static constexpr int per_thread = chunks / kThreads;
    static_assert(chunks % kThreads == 0, "stage must split evenly over the workgroup");
};

struct Params {
    const __bf16 *q[2];
    const __bf16 *k[2];
    const __bf16 *v;
    __bf16 *out;
    float *lse;
    MaskView mask;
    int B, Hq, Hkv, N, window, stride;
    float c;        // scale * log2(e)
    float lambda;
};

// Key index of row r of item `it` of a query tile's walk: items below
// n_pre are stride-prefix chunks, the rest window tiles.
struct Walk {
    int n_pre;     // number of 64-key stride-prefix chunks
    int sk;        // stride keys in the prefix
    int band0;     // list index of the first window tile
};

template <int D, int DV, int NMAPS>
__global__ __launch_bounds__(kThreads) void fwd_bf16_kernel(Params p) {
    using C = Cfg<D, DV, NMAPS>;
    __shared__ __attribute__((aligned(16))) char smem[2 * C::buf];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hl = lane >> 5;          // which half of the wave
    const int col = lane & 31;         // query column within the wave
    const int G = p.Hq / p.Hkv;
    const int nq = p.mask.num_q_tiles;

    // ---- workgroup -> (b, kv head, query tile, head in group) -------------
    // Consecutive workgroup ids go to the 8 XCDs in turn; remap so each XCD
    // receives a contiguous run of logical ids (the same key/value head, so
    // its L2 serves the 4 query heads and neighbouring query tiles).
    int total = gridDim.x, pid = blockIdx.x, lid = pid;
    if ((total & 7) == 0)
        lid = (pid & 7) * (total >> 3) + (pid >> 3);
    const int hg = lid % G;
    int rest = lid / G;
    const int qt = nq - 1 - (rest % nq);  // long (late) query tiles first
    rest /= nq;
    const int g = rest % p.Hkv;
    const int b = rest / p.Hkv;
    const int h = g * G + hg;

    const int q0 = qt * kBM + wave * 32;  // first row of this wave
    const int my_row = q0 + col;
    const int64_t q_off = ((int64_t)(b * p.Hq + h) * p.N + (my_row < p.N ? my_row : p.N - 1)) * D;

    // ---- Q^T fragments (B operand), one per 16-channel step ----------------
    bf16x8 qf[NMAPS][D / 16];
#pragma unroll
    for (int m = 0; m < NMAPS; ++m)
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qf[m][ks] = *reinterpret_cast<const bf16x8 *>(p.q[m] + q_off + ks * 16 + hl * 8);

    // ---- the walk -----------------------------------------------------------
    Walk w;
    w.sk = p.mask.stride_keys[qt];
    w.n_pre = (w.sk + 63) >> 6;
    w.band0 = p.mask.band_begin[qt];
    const int n_items = w.n_pre + (p.mask.row_ptr[qt + 1] - w.band0);

    const int64_t kv_head = (int64_t)(b * p.Hkv + g) * p.N;
    auto item_key0 = [&](int it) -> int {  // first key of a window tile
        return p.mask.kv_tile[w.band0 + (it - w.n_pre)] * 64;
    };
    // key index (global row) of tile row r of item it, clamped into [0, N)
    auto key_of = [&](int it, int key0, int r) -> int {
        if (it < w.n_pre) {
            int kn = it * 64 + r;
            return kn < w.sk ? kn * p.stride : 0;
        }
        int j = key0 + r;
        return j < p.N ? j : p.N - 1;
    };

    u32x4 stage[C::per_thread];
    auto load_stage = [&](int it) {
        int key0 = it >= w.n_pre ? item_key0(it) : 0;
#pragma unroll
        for (int u = 0; u < C::per_thread; ++u) {
            int x = tid + u * kThreads;
            const __bf16 *src;
            int r, c;
            if (x < NMAPS * (C::kTile / 16)) {
                int m = x / (C::kTile / 16);
                int y = x - m * (C::kTile / 16);
                r = y / (D / 8);
                c = y % (D / 8);
                src = p.k[m] + (kv_head + key_of(it, key0, r)) * D + c * 8;
            } else {
                int y = x - NMAPS * (C::kTile / 16);
                r = y / (DV / 8);
                c = y % (DV / 8);
                src = p.v + (kv_head + key_of(it, key0, r)) * DV + c * 8;
            }
            stage[u] = *reinterpret_cast<const u32x4 *>(src);
        }
    };
    auto store_stage = [&](int buf) {
        char *base = smem + buf * C::buf;
#pragma unroll
        for (int u = 0; u < C::per_thread; ++u) {
            int x = tid + u * kThreads;
            int off;
            if (x < NMAPS * (C::kTile / 16)) {
                int m = x / (C::kTile / 16);
                int y = x - m * (C::kTile / 16);
                off = m * C::kTile + chunk_off<D>(y / (D / 8), y % (D / 8));
            } else {
                int y = x - NMAPS * (C::kTile / 16);
                off = NMAPS * C::kTile + chunk_off<DV>(y / (DV / 8), y % (DV / 8));
            }
            *reinterpret_cast<u32x4 *>(base + off) = stage[u];
        }
    };

    // ---- running state ------------------------------------------------------
    f32x16 o[NMAPS][DV / 32];
    float m_run[NMAPS], l_run[NMAPS];
#pragma unroll
    for (int m = 0; m < NMAPS; ++m) {
        m_run[m] = kNegBig;
        l_run[m] = 0.f;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db)
            o[m][db] = f32x16{};
    }

    if (n_items > 0) {
        load_stage(0);
        store_stage(0);
    }
    __syncthreads();

    const int last_row = q0 + 31;
    for (int it = 0; it < n_items; ++it) {
        const int buf = it & 1;
        if (it + 1 < n_items)
            load_stage(it + 1);

        // ---- classify this tile for this wave's rows -----------------------
        const bool pre = it < w.n_pre;
        const int key0 = pre ? 0 : item_key0(it);
        bool empty = false, full;
        uint64_t smask = 0;  // stride keys of a window tile, bit per tile row
        if (pre) {
            full = (it + 1) * 64 <= w.sk;
        } else {
            if (p.stride > 0) {
                int f = ((key0 + p.stride - 1) / p.stride) * p.stride;
                for (int j = f; j < key0 + 64; j += p.stride)
                    smask |= 1ull << (j - key0);
            }
            empty = key0 > last_row || (key0 + 63 < q0 - p.window + 1 && smask == 0);
            full = key0 + 63 <= q0 && key0 >= last_row - p.window + 1 && key0 + 64 <= p.N;
        }

        if (!empty) {
            const char *kb_base = smem + buf * C::buf;
            const char *vb_base = kb_base + NMAPS * C::kTile;

            // ---- S^T = K Q^T -------------------------------------------------
            f32x16 s[NMAPS][2];
#pragma unroll
            for (int m = 0; m < NMAPS; ++m)
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    f32x16 acc = f32x16{};
                    const char *kt = kb_base + m * C::kTile;
#pragma unroll
                    for (int ks = 0; ks < D / 16; ++ks) {
                        bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                            kt + chunk_off<D>(kb * 32 + col, ks * 2 + hl));
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[m][ks], acc, 0, 0, 0);
                    }
                    s[m][kb] = acc;
                }

            // ---- per-cell mask on partial tiles -------------------------------
            if (!full) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        int kk = kb * 32 + (r & 3) + 8 * (r >> 2) + 4 * hl;
                        bool ok;
                        if (pre) {
                            ok = it * 64 + kk < w.sk;
                        } else {
                            int j = key0 + kk;
                            int dist = my_row - j;
                            ok = j < p.N && dist >= 0 &&
                                 (dist < p.window || ((smask >> kk) & 1ull));
                        }
                        if (!ok) {
#pragma unroll
                            for (int m = 0; m < NMAPS; ++m)
                                s[m][kb][r] = -__builtin_inff();
                        }
                    }
            }

            // ---- online softmax ------------------------------------------------
            bf16x8 pf[NMAPS][4];
#pragma unroll
            for (int m = 0; m < NMAPS; ++m) {
                float mx = s[m][0][0];
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        mx = fmaxf(mx, s[m][kb][r]);
                mx = fmaxf(mx, __shfl_xor(mx, 32));
                float mxs = mx * p.c;
                if (__builtin_amdgcn_ballot_w64(mxs > m_run[m] + kSlack) != 0) {
                    float m_new = fmaxf(m_run[m], mxs);
                    float alpha = __builtin_amdgcn_exp2f(m_run[m] - m_new);
                    l_run[m] *= alpha;
#pragma unroll
                    for (int db = 0; db < DV / 32; ++db)
                        o[m][db] *= alpha;
                    m_run[m] = m_new;
                }
                const float nm = -m_run[m];
                float lsum = 0.f;
#pragma unroll
                for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        bf16x8 v8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            float pv = __builtin_amdgcn_exp2f(fmaf(s[m][kb][hf * 8 + e], p.c, nm));
                            lsum += pv;
                            v8[e] = (__bf16)pv;
                        }
                        pf[m][kb * 2 + hf] = v8;
                    }
                l_run[m] += lsum;
            }

            // ---- O^T += V^T P^T --------------------------------------------
            const int grp = lane >> 4, sl = lane & 15;
#pragma unroll
            for (int kb = 0; kb < 2; ++kb)
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int kbase = kb * 32 + hf * 16;
#pragma unroll
                    for (int db = 0; db < DV / 32; ++db) {
                        const int d0 = db * 32 + 16 * (grp & 1) + 4 * (sl & 3);
                        const int r0 = kbase + 4 * (grp >> 1) + (sl >> 2);
                        const int r1 = r0 + 8;
                        typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
                        i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_i16x4 *)(vb_base + chunk_off<DV>(r0, d0 >> 3) + (d0 & 7) * 2));
                        i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                            (lds_i16x4 *)(vb_base + chunk_off<DV>(r1, d0 >> 3) + (d0 & 7) * 2));
                        bf16x4 a0 = __builtin_bit_cast(bf16x4, t0);
                        bf16x4 a1 = __builtin_bit_cast(bf16x4, t1);
                        bf16x8 va = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
                        for (int m = 0; m < NMAPS; ++m)
                            o[m][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                                va, pf[m][kb * 2 + hf], o[m][db], 0, 0, 0);
                    }
                }
        }

        if (it + 1 < n_items)
            store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O / l -> bf16 ------------------------------------------
    float inv[NMAPS];
#pragma unroll
    for (int m = 0; m < NMAPS; ++m) {
        float lt = l_run[m] + __shfl_xor(l_run[m], 32);
        inv[m] = lt > 0.f ? 1.f / lt : 0.f;
        if (NMAPS == 1 && p.lse != nullptr && hl == 0 && my_row < p.N)
            p.lse[(int64_t)(b * p.Hq + h) * p.N + my_row] =
                lt > 0.f ? (m_run[m] + __builtin_log2f(lt)) * kLn2 : -__builtin_inff();
        l_run[m] = lt;
    }
    if (my_row < p.N) {
        __bf16 *dst = p.out + ((int64_t)(b * p.Hq + h) * p.N + my_row) * DV;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db)
#pragma unroll
            for (int r4 = 0; r4 < 4; ++r4) {
                bf16x4 v4;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float x = o[0][db][r4 * 4 + i] * inv[0];
                    if (NMAPS == 2)
                        x -= p.lambda * (o[NMAPS - 1][db][r4 * 4 + i] * inv[NMAPS - 1]);
                    v4[i] = (__bf16)x;
                }
                *reinterpret_cast<bf16x4 *>(dst + db * 32 + 8 * r4 + 4 * hl) = v4;
            }
    }
}

template <int D, int DV, int NMAPS>
hipError_t launch(const FwdArgs &a, hipStream_t stream) {
    Params p;
    for (int m = 0; m < 2; ++m) {
        p.q[m] = static_cast<const __bf16 *>(a.q[m]);
        p.k[m] = static_cast<const __bf16 *>(a.k[m]);
    }
    p.v = static_cast<const __bf16 *>(a.v);
    p.out = static_cast<__bf16 *>(a.out);
    p.lse = a.lse;
    p.mask = a.mask;
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.N = a.N;
    p.window = a.window;
    p.stride = a.stride;
    p.c = a.scale * kLog2e;
    p.lambda = a.lambda;
    unsigned grid = static_cast<unsigned>(a.mask.num_q_tiles) * a.Hq * a.B;
    hipLaunchKernelGGL((fwd_bf16_kernel<D, DV, NMAPS>), dim3(grid), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream) {
    if (a.nmaps == 1) {
        switch (a.d) {
        case 32: return launch<32, 32, 1>(a, stream);
        case 64: return launch<64, 64, 1>(a, stream);
        case 128: return launch<128, 128, 1>(a, stream);
        }
    } else {
#define SWA_DIFF_CASE(DQ, DVV) \
    if (a.d == DQ && a.dv == DVV) return launch<DQ, DVV, 2>(a, stream);
        SWA_DIFF_CASE(32, 32)
        SWA_DIFF_CASE(32, 64)
        SWA_DIFF_CASE(32, 128)
        SWA_DIFF_CASE(64, 32)
        SWA_DIFF_CASE(64, 64)
        SWA_DIFF_CASE(64, 128)
#undef SWA_DIFF_CASE
    }
    return hipErrorInvalidValue;
}

}  // namespace swa
