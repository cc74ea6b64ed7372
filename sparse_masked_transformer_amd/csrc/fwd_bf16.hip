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
//   * K (and V) tiles are staged HBM -> VGPR -> LDS, double-buffered; the
//     next tile's loads are in flight while the current tile is computed.
//     LDS rows are padded by 32 bytes (bank spread).
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
#include <type_traits>

#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kSlack = 8.0f;       // log2 units the running maximum may lag
constexpr float kNegBig = -1e30f;    // running maximum before any key
constexpr int kThreads = 256;
// dword 3 of a raw (untyped) buffer descriptor on gfx950
constexpr int kBufferDword3 = 0x00020000;

template <int D, int DV, int NMAPS>
struct Cfg {
    // Row padding (bank spread, with every LDS address a per-lane base plus
    // a compile-time offset):
    //   K rows +16 bytes: consecutive rows start 4 banks apart, so the
    //     16-byte reads of 16 rows at one column cover all 64 banks once;
    //   V rows +64 bytes: consecutive rows start 16 banks apart, so the
    //     transposed 8-byte reads of 4 rows x 64 bytes do not overlap.
    static constexpr int kRow = 2 * D + 16;                   // K row stride, bytes
    static constexpr int vRow = 2 * DV + 64;                  // V row stride, bytes
    static constexpr int kTile = 64 * kRow;                   // one K tile
    static constexpr int vTile = 64 * vRow;                   // one V tile
    static constexpr int stage = NMAPS * kTile + vTile;       // one buffer
    static constexpr int kPer = D / 32;                       // K chunks per thread
    static constexpr int vPer = DV / 32;                      // V chunks per thread
    static constexpr int kRowStep = kThreads / (D / 8);       // rows between a thread's chunks
    static constexpr int vRowStep = kThreads / (DV / 8);
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

template <int D, int DV, int NMAPS>
__device__ __forceinline__ void fwd_bf16_body(const Params &p) {
    using C = Cfg<D, DV, NMAPS>;
    __shared__ __attribute__((aligned(16))) char smem[2 * C::stage];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int hl = lane >> 5;          // which half of the wave
    const int col = lane & 31;         // query column within the wave
    const int G = p.Hq / p.Hkv;
    const int nq = p.mask.num_q_tiles;

    // ---- workgroup -> (b, kv head, query tile, head in group) -------------
    // Consecutive workgroup ids go to the 8 XCDs in turn; remap so each XCD
    // receives a contiguous run of logical ids (the same key/value head, so
    // its L2 serves the query heads of the group and neighbouring tiles).
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

    // ---- the walk: stride-prefix chunks, then window tiles ----------------
    const int sk = p.mask.stride_keys[qt];
    const int n_pre = (sk + 63) >> 6;
    const int band0 = p.mask.band_begin[qt];
    const int n_items = n_pre + (p.mask.row_ptr[qt + 1] - band0);
    const int64_t kv_head = (int64_t)(b * p.Hkv + g) * p.N;

    // first key of item it (window tiles only)
    auto item_key0 = [&](int it) -> int {
        return it >= n_pre ? p.mask.kv_tile[band0 + (it - n_pre)] * 64 : 0;
    };

    // per-thread staging: thread t owns chunk column t % (D/8) of rows
    // t / (D/8) + u * kRowStep (same for V with DV)
    const int kc = tid % (D / 8), kr0 = tid / (D / 8);
    const int vc = tid % (DV / 8), vr0 = tid / (DV / 8);
    u32x4 kst[NMAPS][C::kPer], vst[C::vPer];
    // Buffer descriptors over this (b, kv head)'s K and V rows: N rows of D
    // (DV) bf16.  Reads at or past row N return zeros (no clamping needed);
    // the per-tile offset lives in a scalar register.
    __amdgpu_buffer_rsrc_t krs[NMAPS];
#pragma unroll
    for (int m = 0; m < NMAPS; ++m)
        krs[m] = __builtin_amdgcn_make_buffer_rsrc((void *)(p.k[m] + kv_head * D), 0,
                                                   p.N * D * 2, kBufferDword3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(p.v + kv_head * DV), 0, p.N * DV * 2, kBufferDword3);
    const int k_goff = (kr0 * D + kc * 8) * 2;
    const int v_goff = (vr0 * DV + vc * 8) * 2;
    auto load_stage = [&](int it) {
        if (it >= n_pre) {
            // window tile: rows key0 .. key0+63
            const int key0 = item_key0(it);
#pragma unroll
            for (int m = 0; m < NMAPS; ++m)
#pragma unroll
                for (int u = 0; u < C::kPer; ++u)
                    kst[m][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        krs[m], k_goff, (key0 + u * C::kRowStep) * D * 2, 0));
#pragma unroll
            for (int u = 0; u < C::vPer; ++u)
                vst[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    vrs, v_goff, (key0 + u * C::vRowStep) * DV * 2, 0));
        } else {
            // stride-prefix chunk: rows kn * stride for kn < sk (others read
            // past the end, i.e. zeros)
#pragma unroll
            for (int u = 0; u < C::kPer; ++u) {
                const int kn = it * 64 + kr0 + u * C::kRowStep;
                const int row = kn < sk ? kn * p.stride : p.N;
#pragma unroll
                for (int m = 0; m < NMAPS; ++m)
                    kst[m][u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                        krs[m], (row * D + kc * 8) * 2, 0, 0));
            }
#pragma unroll
            for (int u = 0; u < C::vPer; ++u) {
                const int kn = it * 64 + vr0 + u * C::vRowStep;
                const int row = kn < sk ? kn * p.stride : p.N;
                vst[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                    vrs, (row * DV + vc * 8) * 2, 0, 0));
            }
        }
    };
    auto store_stage = [&](int buf) {
        char *kbase = smem + buf * C::stage + kr0 * C::kRow + kc * 16;
        char *vbase = smem + buf * C::stage + NMAPS * C::kTile + vr0 * C::vRow + vc * 16;
#pragma unroll
        for (int u = 0; u < C::kPer; ++u)
#pragma unroll
            for (int m = 0; m < NMAPS; ++m)
                *reinterpret_cast<u32x4 *>(kbase + m * C::kTile + u * C::kRowStep * C::kRow) = kst[m][u];
#pragma unroll
        for (int u = 0; u < C::vPer; ++u)
            *reinterpret_cast<u32x4 *>(vbase + u * C::vRowStep * C::vRow) = vst[u];
    };

    // per-lane LDS read bases (everything else is a compile-time offset)
    const int grp = lane >> 4, sl = lane & 15;
    const int k_lane = col * C::kRow + hl * 16;
    const int v_lane = (4 * (grp >> 1) + (sl >> 2)) * C::vRow + (16 * (grp & 1) + 4 * (sl & 3)) * 2;

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
        // prefetch the next item (the last item re-reads itself; harmless)
        load_stage(it + 1 < n_items ? it + 1 : it);

        // ---- classify this tile for this wave's rows -----------------------
        const bool pre = it < n_pre;
        const int key0 = item_key0(it);
        bool empty = false, full;
        uint64_t smask = 0;  // stride keys of a window tile, bit per tile row
        if (pre) {
            full = (it + 1) * 64 <= sk;
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
            const char *kb_base = smem + buf * C::stage + k_lane;
            const char *vb_base = smem + buf * C::stage + NMAPS * C::kTile + v_lane;

            // Two 32-key halves, software-pipelined so MFMA and VALU work of
            // one wave overlap: QK^T(half 1) is in flight during the softmax
            // of half 0, and PV(half 0) during the softmax of half 1.
            f32x16 sh[2][NMAPS];
            auto qk_half = [&](int kb) {
#pragma unroll
                for (int m = 0; m < NMAPS; ++m) {
                    bf16x8 ka[D / 16];
#pragma unroll
                    for (int ks = 0; ks < D / 16; ++ks)
                        ka[ks] = *reinterpret_cast<const bf16x8 *>(
                            kb_base + m * C::kTile + kb * 32 * C::kRow + ks * 32);
                    f32x16 acc = f32x16{};
#pragma unroll
                    for (int ks = 0; ks < D / 16; ++ks)
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[m][ks], acc, 0, 0, 0);
                    sh[kb][m] = acc;
                }
            };
            // per-cell mask of half kb on partial tiles (branch-free selects);
            // lane key kk = kb*32 + kc + 4*hl with kc a compile-time constant
            auto mask_half = [&](int kb) {
                const float ninf = -__builtin_inff();
                if (pre) {
                    const int lim = sk - it * 64 - kb * 32 - 4 * hl;  // attended iff kc < lim
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kcst = (r & 3) + 8 * (r >> 2);
#pragma unroll
                        for (int m = 0; m < NMAPS; ++m)
                            sh[kb][m][r] = kcst < lim ? sh[kb][m][r] : ninf;
                    }
                } else {
                    // dist = i - j = base - kc; window part iff 0 <= dist < W
                    const int base = my_row - key0 - kb * 32 - 4 * hl;
                    const unsigned W = (unsigned)p.window;
                    if (smask == 0) {
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int kcst = (r & 3) + 8 * (r >> 2);
                            const bool ok = (unsigned)(base - kcst) < W;
#pragma unroll
                            for (int m = 0; m < NMAPS; ++m)
                                sh[kb][m][r] = ok ? sh[kb][m][r] : ninf;
                        }
                    } else {
                        const uint32_t lm = (uint32_t)(smask >> (kb * 32 + 4 * hl));
#pragma unroll
                        for (int r = 0; r < 16; ++r) {
                            const int kcst = (r & 3) + 8 * (r >> 2);
                            const int dist = base - kcst;
                            // bitwise, not short-circuit: no per-cell branch
                            const bool ok = ((unsigned)dist < W) |
                                            ((dist >= 0) & (((lm >> kcst) & 1u) != 0));
#pragma unroll
                            for (int m = 0; m < NMAPS; ++m)
                                sh[kb][m][r] = ok ? sh[kb][m][r] : ninf;
                        }
                    }
                }
            };
            // online softmax of half kb, split in two phases: the row maximum
            // and rescale (with a wave-uniform branch), then the exponentials
            // (branch-free, so the scheduler can interleave them with MFMAs)
            bf16x8 pf[NMAPS][2];
            // Returns whether the running maximum moved; l is rescaled here,
            // O by the caller (alpha[m]) once every PV product that used the
            // old maximum has been accumulated.
            float alpha[NMAPS];
            auto softmax_max = [&](int kb) -> bool {
                bool moved = false;
#pragma unroll
                for (int m = 0; m < NMAPS; ++m) {
                    const f32x16 &sv = sh[kb][m];
                    float mx = fmaxf(fmaxf(fmaxf(sv[0], sv[1]), fmaxf(sv[2], sv[3])),
                                     fmaxf(fmaxf(sv[4], sv[5]), fmaxf(sv[6], sv[7])));
                    mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(sv[8], sv[9]), fmaxf(sv[10], sv[11])),
                                         fmaxf(fmaxf(sv[12], sv[13]), fmaxf(sv[14], sv[15]))));
                    // row maximum across the two lane halves holding the row
                    const auto sw = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, mx),
                                                                     __builtin_bit_cast(unsigned, mx),
                                                                     false, false);
                    mx = fmaxf(__builtin_bit_cast(float, (unsigned)sw[0]),
                               __builtin_bit_cast(float, (unsigned)sw[1]));
                    const float mxs = mx * p.c;
                    alpha[m] = 1.f;
                    if (__builtin_amdgcn_ballot_w64(mxs > m_run[m] + kSlack) != 0) {
                        const float m_new = fmaxf(m_run[m], mxs);
                        alpha[m] = __builtin_amdgcn_exp2f(m_run[m] - m_new);
                        l_run[m] *= alpha[m];
                        m_run[m] = m_new;
                        moved = true;
                    }
                }
                return moved;
            };
            auto rescale_o = [&]() {
#pragma unroll
                for (int m = 0; m < NMAPS; ++m)
#pragma unroll
                    for (int db = 0; db < DV / 32; ++db)
                        o[m][db] *= alpha[m];
            };
            auto softmax_exp = [&](int kb) {
#pragma unroll
                for (int m = 0; m < NMAPS; ++m) {
                    const f32x16 &sv = sh[kb][m];
                    const float nm = -m_run[m];
                    float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // independent partial sums
#pragma unroll
                    for (int hf = 0; hf < 2; ++hf) {
                        bf16x8 v8;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float pv = __builtin_amdgcn_exp2f(fmaf(sv[hf * 8 + e], p.c, nm));
                            lsum[e & 3] += pv;
                            v8[e] = (__bf16)pv;
                        }
                        pf[m][hf] = v8;
                    }
                    l_run[m] += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
                }
            };
            // O^T += V^T P^T over the 32 keys of half kb
            auto pv_half = [&](int kb) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    const int kbase = kb * 32 + hf * 16;
#pragma unroll
                    for (int db = 0; db < DV / 32; ++db) {
                        const char *a = vb_base + kbase * C::vRow + db * 64;
                        const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)a);
                        const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a + 8 * C::vRow));
                        const bf16x4 a0 = __builtin_bit_cast(bf16x4, t0);
                        const bf16x4 a1 = __builtin_bit_cast(bf16x4, t1);
                        const bf16x8 va = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
                        for (int m = 0; m < NMAPS; ++m)
                            o[m][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[m][hf], o[m][db], 0, 0, 0);
                    }
                }
            };
            // scheduling hint for one branch-free block: after its n_ds LDS
            // reads, alternate one MFMA with a few VALU instructions
            auto interleave = [&](auto n_ds, auto n_mfma, auto n_valu) {
                __builtin_amdgcn_sched_group_barrier(0x100, decltype(n_ds)::value, 0);
#pragma unroll
                for (int i = 0; i < decltype(n_mfma)::value; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, decltype(n_valu)::value, 0);
                }
            };
            using QkDs = std::integral_constant<int, NMAPS * D / 16>;
            using QkMfma = std::integral_constant<int, NMAPS * D / 16>;
            using PvDs = std::integral_constant<int, 4 * (DV / 32)>;
            using PvMfma = std::integral_constant<int, NMAPS * 2 * (DV / 32)>;
            using Valu = std::integral_constant<int, 6>;

            qk_half(0);
            if (!full)
                mask_half(0);
            if (softmax_max(0))
                rescale_o();
            qk_half(1);       // matrix work ...
            softmax_exp(0);   // ... overlapped with the exponentials of half 0
            interleave(QkDs{}, QkMfma{}, Valu{});
            // keep the half-0 exponentials in this block (otherwise they are
            // sunk past the next branch, next to their use)
#pragma unroll
            for (int m = 0; m < NMAPS; ++m)
                asm volatile("" ::"v"(pf[m][0]), "v"(pf[m][1]), "v"(l_run[m]));
            if (!full)
                mask_half(1);
            const bool moved1 = softmax_max(1);
            pv_half(0);       // matrix work (probabilities of the old maximum) ...
            softmax_exp(1);   // ... overlapped with the exponentials of half 1
            interleave(PvDs{}, PvMfma{}, Valu{});
            if (moved1)
                rescale_o();
            pv_half(1);
        }

        store_stage(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O / l -> bf16 ------------------------------------------
    float inv[NMAPS];
#pragma unroll
    for (int m = 0; m < NMAPS; ++m) {
        const float lt = l_run[m] + __shfl_xor(l_run[m], 32);
        inv[m] = lt > 0.f ? 1.f / lt : 0.f;
        if (NMAPS == 1 && p.lse != nullptr && hl == 0 && my_row < p.N)
            p.lse[(int64_t)(b * p.Hq + h) * p.N + my_row] =
                lt > 0.f ? (m_run[m] + __builtin_log2f(lt)) * kLn2 : -__builtin_inff();
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

// Single-map kernels fit in 256 registers per lane, which lets two waves
// share each SIMD (one wave's softmax overlaps the other's matrix work);
// two-map kernels need more state and run one wave per SIMD.
template <int D, int DV>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(Params p) {
    fwd_bf16_body<D, DV, 1>(p);
}

template <int D, int DV>
__global__ __launch_bounds__(kThreads) void diff_bf16_kernel(Params p) {
    fwd_bf16_body<D, DV, 2>(p);
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
    if constexpr (NMAPS == 1)
        hipLaunchKernelGGL((fwd_bf16_kernel<D, DV>), dim3(grid), dim3(kThreads), 0, stream, p);
    else
        hipLaunchKernelGGL((diff_bf16_kernel<D, DV>), dim3(grid), dim3(kThreads), 0, stream, p);
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
