// One decode step over a rolling KV window, bf16 on gfx950, with optional
// sink slots and one or two score maps.
//
// Learn: Sparse & Sliding-Window Attention, §4 and §6: decoding keeps only
// the last `window` tokens' keys and values in a fixed-size rolling buffer
// (position p in slot p mod window), so the step reads the whole window once
// and is bound by HBM bandwidth; StreamingLLM (same page, §4) also keeps the
// first few tokens in sink slots.  Attention Variants — Sliding Window,
// Sparse, Differential, "Differential attention": two maps share one value
// cache; the symptom/cause/fix table of "Attention Variants Compared" lists
// a differential decode that loads the value cache twice as slower than the
// baseline (each K and V byte is read once here).
//
// A sequence's cache is walked as one list of "virtual slots": first the
// sink slots that the ring no longer covers, then the valid ring slots
// (attention does not depend on key order).
//
// Workgroup: `waves` waves for one (sequence, key/value head, split of the
// virtual slots) and one block of up to 16 of the head's query heads (grid
// dimension y); each wave takes a contiguous run of whole 32-slot steps.
// (With more than 16 query heads per key/value head, each block of 16 reads
// the head's keys and values again; the blocks run side by side, so the
// repeats mostly hit L2.  With a single block the loads carry the
// nontemporal hint instead.)
//   * A wave streams its slots 32 at a time: coalesced 16-byte loads into
//     registers two steps ahead (two register stages; one for two maps with
//     2 d + dv > 256), then into its own LDS area, rows padded by 32 bytes
//     against bank conflicts.
//   * The G query heads sharing the key/value head form the 16 columns of a
//     v_mfma_f32_16x16x32_bf16 (unused columns are zero): S^T = K Q^T with K
//     from LDS as the A operand; lane l holds head l%16 and keys 4(l/16)+i.
//   * fp32 online softmax per map (exp2, log2(e) folded into the scale);
//     O^T += V^T P^T with V^T fragments from ds_read_b64_tr_b16, one V
//     fragment feeding both maps.
//   * The waves' (max, sum, output) are merged through LDS in a fixed order.
//     With one split the workgroup writes the output; otherwise it writes a
//     partial to the workspace and a combine kernel merges the splits:
//     m* = max m_s, l* = sum l_s 2^(m_s - m*), o = sum o_s 2^(m_s - m*) / l*.
#include <mutex>

#include "swa_internal.h"

namespace swa {

// Scratch of swa_attn_decode_noalloc: the split partials (max, sum, output)
// that the combine kernel merges, in a file-scope array instead of a
// caller's workspace.  Each GPU holds its own copy.  In host code the name
// `scratch` is only a stand-in for the symbol; the device address comes from
// decode_static_scratch.
static __device__ __align__(256) char scratch[SWA_DECODE_SCRATCH_BYTES];

hipError_t decode_static_scratch(void **ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        // once per device, with that device current (the caller's current
        // device is the one its stream belongs to)
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        if (p == nullptr)
            return hipErrorInvalidSymbol;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef const __attribute__((address_space(1))) u32x4 global_u32x4;

// 16-byte load from a global byte address (a global load; a generic pointer
// rebuilt from an integer would become a flat load).  NT adds the
// nontemporal hint (`nt`), for rings that one workgroup reads once: the
// window decode workload then reads KV at 6.6 TB/s against 5.8 TB/s without.
// Where several blocks of query heads read the same ring the hint costs the
// L2 hits of the later blocks (64 query heads on one KV head: 66 against
// 50 us), so those launches load without it.
template <bool NT>
__device__ inline u32x4 load16(uintptr_t addr) {
    if constexpr (NT)
        return __builtin_nontemporal_load(reinterpret_cast<global_u32x4 *>(addr));
    else
        return *reinterpret_cast<global_u32x4 *>(addr);
}

// dword 3 of a raw (untyped) buffer descriptor on gfx950
constexpr int kBufferDword3 = 0x00020000;

// The same load through a buffer descriptor held in scalar registers: a
// 32-bit lane offset instead of a 64-bit lane address (fewer VALU
// instructions per load; window decode 161 -> 158 us).  Bit 1 of the cache
// policy operand is the nontemporal hint.
template <bool NT>
__device__ inline u32x4 load16(__amdgpu_buffer_rsrc_t rsrc, int off) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, off, 0, NT ? 2 : 0));
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegBig = -1e30f;

template <int D, int DV, int NMAPS>
struct Lay {
    // Row strides in LDS, bytes.  Both pad by 32 bytes: measured with the
    // LDS bank-conflict counter, the 16-byte K reads and the transposed
    // 8-byte V reads are then conflict-free (K +16 and V +64, the earlier
    // paddings, left conflicts on 15% and 25% of the LDS cycles).
    static constexpr int kRow = 2 * D + 32;
    static constexpr int vRow = 2 * DV + 32;
    static constexpr int kTile = kDecodeStep * kRow;
    static constexpr int vTile = kDecodeStep * vRow;
    static constexpr int wave_bytes = NMAPS * kTile + vTile;
    static constexpr int kChunks = kDecodeStep * D / 8 / 64;   // 16-byte chunks per lane
    static constexpr int vChunks = kDecodeStep * DV / 8 / 64;
};

// Register stages of a wave's step loads: two (the next two steps in flight),
// or one where two stages would not fit the register file -- two maps whose
// K rows and V row span more than 256 channels (2 d + dv > 256).
template <int D, int DV, int NMAPS>
constexpr int reg_stages() { return NMAPS * D + DV > 256 ? 1 : 2; }

// Waves per SIMD, at least: two, unless two register stages of two K rows
// and a V row (2 d + dv > 192), or two maps' 128-wide outputs, no longer fit
// half the register file.  (A minimum only: a maximum makes the compiler
// declare extra registers to enforce it, which would keep small head sizes
// from running more waves.)
template <int D, int DV, int NMAPS>
constexpr int occupancy() { return NMAPS == 2 && (2 * D + DV > 192 || DV == 128) ? 1 : 2; }

// Row stride (floats) of the waves' outputs in the merge area: 16 floats of
// padding put the rows of four query heads, which one 16-byte store per
// lane writes, on different banks.
template <int DV>
constexpr int kMergeRow = DV + 16;

// LDS bytes of a workgroup: the waves' tiles, or the merge area if larger.
template <int D, int DV, int NMAPS>
size_t lds_bytes(int waves, int G) {
    size_t tiles = static_cast<size_t>(waves) * Lay<D, DV, NMAPS>::wave_bytes;
    size_t merge = static_cast<size_t>(waves) * NMAPS * (2 * 16 + G * kMergeRow<DV>) * sizeof(float);
    return tiles > merge ? tiles : merge;
}

struct Params {
    const __bf16 *q[2];   // [B, Hq, D]
    const __bf16 *k[2];   // rings [B, Hkv, window, D]
    const __bf16 *v;      // ring  [B, Hkv, window, DV]
    const __bf16 *ks[2];  // sink slots [B, Hkv, n_sink, D] (n_sink == 0: unused)
    const __bf16 *vs;     // sink slots [B, Hkv, n_sink, DV]
    const int32_t *seq_len;
    __bf16 *out;          // [B, Hq, DV]
    float *ws_ml;         // [B*Hq*splits*NMAPS][2]  (max in log2 units, sum)
    float *ws_o;          // [B*Hq*splits*NMAPS][DV]
    int B, Hq, Hkv, N, window, n_sink, splits, steps_per_wave;
    float c;              // scale * log2(e)
    float lambda;
};

template <int D, int DV, int NMAPS, bool NT, bool SINK>
__global__ __launch_bounds__(64 * kDecodeMaxWaves)
__attribute__((amdgpu_waves_per_eu(occupancy<D, DV, NMAPS>())))
void decode_kernel(Params p) {
    using Y = Lay<D, DV, NMAPS>;
    extern __shared__ __attribute__((aligned(16))) char dsm[];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int waves = blockDim.x >> 6;
    const int split = blockIdx.x % p.splits;
    const int bg = blockIdx.x / p.splits;
    const int g = bg % p.Hkv, b = bg / p.Hkv;
    const int G = p.Hq / p.Hkv;                   // query heads per key/value head
    const int h0 = 16 * blockIdx.y;               // this block of up to 16 of them
    const int Gb = G - h0 < 16 ? G - h0 : 16;

    // ---- this wave's virtual slots -------------------------------------------
    // wave-uniform (one sequence per workgroup); made explicit so the step
    // loop below compiles as a uniform loop, not an exec-masked one whose
    // load waits fall back to waiting for every outstanding load
    const int L = __builtin_amdgcn_readfirstlane(p.seq_len ? p.seq_len[b] : p.N);
    const int nvalid = L <= 0 ? 0 : (L < p.window ? L : p.window);
    const int first = L - p.window > 0 ? L - p.window : 0;   // oldest position in the ring
    const int s_eff = SINK ? (first < p.n_sink ? first : p.n_sink) : 0;   // sink slots not in the ring
    const int T = s_eff + nvalid;
    const int v0 = (split * waves + wave) * p.steps_per_wave * kDecodeStep;
    int v1 = v0 + p.steps_per_wave * kDecodeStep;
    v1 = v1 < T ? v1 : T;
    const int nsteps = v1 > v0 ? (v1 - v0 + kDecodeStep - 1) / kDecodeStep : 0;

    const int64_t kv = static_cast<int64_t>(b) * p.Hkv + g;
    const int64_t ring = kv * p.window, sink = kv * p.n_sink;

    // Each wave walks its run from a step of its own, wrapping around (the
    // online softmax does not depend on the order).  The runs start a whole
    // number of runs apart in memory; walked in lock step from their starts,
    // every wave would read the same offset within its run at the same time
    // and the reads would crowd onto few HBM channels (window decode: 190 us
    // in order, 182 us rotated).
    const int rot = nsteps > 0 ? ((static_cast<int>(blockIdx.x) * waves + wave) * 7) % nsteps : 0;
    auto run_step = [&](int st) {   // step st of the walk -> step of the run
        const int r = st + rot >= nsteps ? st + rot - nsteps : st + rot;
        return st < nsteps ? r : st;   // steps past the run stay past it (fully masked)
    };

    // ---- Q^T fragments: column = query head within the group ----------------
    const int colq = lane & 15, grp = lane >> 4, sl = lane & 15;
    bf16x8 qf[NMAPS][D / 32];
#pragma unroll
    for (int m = 0; m < NMAPS; ++m)
#pragma unroll
        for (int ks = 0; ks < D / 32; ++ks) {
            if (colq < Gb)
                qf[m][ks] = *reinterpret_cast<const bf16x8 *>(
                    p.q[m] + (kv * G + h0 + colq) * D + ks * 32 + grp * 8);
            else
                qf[m][ks] = bf16x8{};
        }

    // A step's K and V rows, 16 bytes per lane per load, consecutive lanes
    // reading consecutive chunks of a row (coalesced); virtual slots past the
    // wave's run are clamped to its last one (and masked out below).  Addresses are
    // built from wave-uniform byte bases: selecting between two pointers held
    // in the argument block would turn into a per-lane load of the pointer.
    uintptr_t kring_b[NMAPS], ksink_b[NMAPS];
#pragma unroll
    for (int m = 0; m < NMAPS; ++m) {
        kring_b[m] = reinterpret_cast<uintptr_t>(p.k[m]) + static_cast<uintptr_t>(ring) * (2 * D);
        ksink_b[m] = reinterpret_cast<uintptr_t>(p.ks[m]) + static_cast<uintptr_t>(sink) * (2 * D);
    }
    const uintptr_t vring_b = reinterpret_cast<uintptr_t>(p.v) + static_cast<uintptr_t>(ring) * (2 * DV);
    const uintptr_t vsink_b = reinterpret_cast<uintptr_t>(p.vs) + static_cast<uintptr_t>(sink) * (2 * DV);
    // Without sink slots every slot is a ring slot and the loads go through
    // ring descriptors: one (sequence, head) ring is at most SWA_MAX_N slots
    // of at most 256 bytes (1 GiB), so every offset in it fits an int.  (A
    // per-step choice between the two forms in one kernel spills registers.)
    __amdgpu_buffer_rsrc_t krs[NMAPS];
#pragma unroll
    for (int m = 0; m < NMAPS; ++m)
        krs[m] = __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(kring_b[m]), 0,
                                                   p.window * (2 * D), kBufferDword3);
    const __amdgpu_buffer_rsrc_t vrs =
        __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(vring_b), 0, p.window * (2 * DV),
                                          kBufferDword3);
    constexpr int S = reg_stages<D, DV, NMAPS>();
    u32x4 kst[S][NMAPS][Y::kChunks], vst[S][Y::vChunks];
    auto load = [&](int st, int reg) {
        const int base = v0 + run_step(st) * kDecodeStep;
        if constexpr (!SINK) {   // s_eff = 0: virtual slot = ring slot
#pragma unroll
            for (int u = 0; u < Y::kChunks; ++u) {
                const int x = lane + 64 * u;
                const int r = x / (D / 8), c = x % (D / 8);
                const int vs = base + r < v1 ? base + r : v1 - 1;
                const int off = vs * (2 * D) + c * 16;
#pragma unroll
                for (int m = 0; m < NMAPS; ++m)
                    kst[reg][m][u] = load16<NT>(krs[m], off);
            }
#pragma unroll
            for (int u = 0; u < Y::vChunks; ++u) {
                const int x = lane + 64 * u;
                const int r = x / (DV / 8), c = x % (DV / 8);
                const int vs = base + r < v1 ? base + r : v1 - 1;
                vst[reg][u] = load16<NT>(vrs, vs * (2 * DV) + c * 16);
            }
            return;
        }
#pragma unroll
        for (int u = 0; u < Y::kChunks; ++u) {
            const int x = lane + 64 * u;
            const int r = x / (D / 8), c = x % (D / 8);
            const int vs = base + r < v1 ? base + r : v1 - 1;
            const bool in_sink = vs < s_eff;
            const uintptr_t off = static_cast<uintptr_t>(in_sink ? vs : vs - s_eff) * (2 * D) + c * 16;
#pragma unroll
            for (int m = 0; m < NMAPS; ++m)
                kst[reg][m][u] = load16<NT>((in_sink ? ksink_b[m] : kring_b[m]) + off);
        }
#pragma unroll
        for (int u = 0; u < Y::vChunks; ++u) {
            const int x = lane + 64 * u;
            const int r = x / (DV / 8), c = x % (DV / 8);
            const int vs = base + r < v1 ? base + r : v1 - 1;
            const bool in_sink = vs < s_eff;
            const uintptr_t off = static_cast<uintptr_t>(in_sink ? vs : vs - s_eff) * (2 * DV) + c * 16;
            vst[reg][u] = load16<NT>((in_sink ? vsink_b : vring_b) + off);
        }
    };
    char *smem = dsm + wave * Y::wave_bytes;
    // one wave per LDS area: its writes land after its reads of the previous step
    auto store = [&](int reg) {
#pragma unroll
        for (int u = 0; u < Y::kChunks; ++u) {
            const int x = lane + 64 * u;
            const int r = x / (D / 8), c = x % (D / 8);
#pragma unroll
            for (int m = 0; m < NMAPS; ++m)
                *reinterpret_cast<u32x4 *>(smem + m * Y::kTile + r * Y::kRow + c * 16) = kst[reg][m][u];
        }
#pragma unroll
        for (int u = 0; u < Y::vChunks; ++u) {
            const int x = lane + 64 * u;
            const int r = x / (DV / 8), c = x % (DV / 8);
            *reinterpret_cast<u32x4 *>(smem + NMAPS * Y::kTile + r * Y::vRow + c * 16) = vst[reg][u];
        }
    };

    f32x4 o[NMAPS][DV / 16];
    float m_run[NMAPS], l_run[NMAPS];
#pragma unroll
    for (int m = 0; m < NMAPS; ++m) {
#pragma unroll
        for (int db = 0; db < DV / 16; ++db)
            o[m][db] = f32x4{};
        m_run[m] = kNegBig;
        l_run[m] = 0.f;
    }

    // per-lane LDS read bases (the rest are compile-time offsets)
    const char *kb = smem + colq * Y::kRow + grp * 16;
    const char *vb = smem + NMAPS * Y::kTile + (4 * grp + (sl >> 2)) * Y::vRow + 4 * (sl & 3) * 2;

    auto compute = [&](int st) {
        const int base = v0 + run_step(st) * kDecodeStep;
        bf16x8 pf[NMAPS];
#pragma unroll
        for (int m = 0; m < NMAPS; ++m) {
            // ---- S^T = K Q^T for two 16-key blocks ---------------------------
            f32x4 s[2];
#pragma unroll
            for (int kbk = 0; kbk < 2; ++kbk) {
                f32x4 acc = f32x4{};
#pragma unroll
                for (int ks = 0; ks < D / 32; ++ks) {
                    const bf16x8 a = *reinterpret_cast<const bf16x8 *>(
                        kb + m * Y::kTile + kbk * 16 * Y::kRow + ks * 64);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[m][ks], acc, 0, 0, 0);
                }
                s[kbk] = acc;
            }
            // ---- mask virtual slots past this wave's run -----------------------
            if (base + kDecodeStep > v1) {
#pragma unroll
                for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        s[kbk][i] = base + kbk * 16 + grp * 4 + i < v1 ? s[kbk][i] : -__builtin_inff();
            }
            // ---- online softmax (row = query head column) ----------------------
            float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                             fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const float mxs = mx * p.c;
            if (mxs > m_run[m]) {
                const float alpha = __builtin_amdgcn_exp2f(m_run[m] - mxs);
                l_run[m] *= alpha;
#pragma unroll
                for (int db = 0; db < DV / 16; ++db)
                    o[m][db] *= alpha;
                m_run[m] = mxs;
            }
#pragma unroll
            for (int kbk = 0; kbk < 2; ++kbk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = __builtin_amdgcn_exp2f(fmaf(s[kbk][i], p.c, -m_run[m]));
                    l_run[m] += pv;
                    pf[m][kbk * 4 + i] = (__bf16)pv;
                }
        }
        // ---- O^T += V^T P^T, one V fragment for every map ---------------------
#pragma unroll
        for (int db = 0; db < DV / 16; ++db) {
            const i16x4 t0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vb + db * 32));
            const i16x4 t1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vb + 16 * Y::vRow + db * 32));
            const bf16x4 a0 = __builtin_bit_cast(bf16x4, t0);
            const bf16x4 a1 = __builtin_bit_cast(bf16x4, t1);
            const bf16x8 va = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
            for (int m = 0; m < NMAPS; ++m)
                o[m][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[m], o[m][db], 0, 0, 0);
        }
    };

    // Two register stages: steps st (even) and st+1 (odd) alternate.  Every
    // load is issued unconditionally (a step past the wave's run re-reads its
    // last slot and is fully masked, so it adds nothing): conditional loads
    // would make the compiler's load-counter waits assume the fewest loads in
    // flight and wait for the other stage too.  With one stage the next
    // step's loads are in flight while the current step, already in LDS, is
    // computed.
    if (nsteps > 0) {
        if constexpr (S == 2) {
            load(0, 0);
            load(1, 1);
            for (int st = 0; st < nsteps; st += 2) {
                store(0);
                load(st + 2, 0);
                compute(st);
                store(1);
                load(st + 3, 1);
                compute(st + 1);
            }
        } else {
            load(0, 0);
            for (int st = 0; st < nsteps; ++st) {
                store(0);
                load(st + 1, 0);
                compute(st);
            }
        }
    }

    // ---- merge the waves through LDS ------------------------------------------
    float lt[NMAPS];
#pragma unroll
    for (int m = 0; m < NMAPS; ++m) {
        lt[m] = l_run[m] + __shfl_xor(l_run[m], 16);
        lt[m] += __shfl_xor(lt[m], 32);
    }
    __syncthreads();  // every wave is done with its tiles
    float *mw = reinterpret_cast<float *>(dsm);   // [waves][NMAPS][16]
    float *lw = mw + waves * NMAPS * 16;          // [waves][NMAPS][16]
    float *ow = lw + waves * NMAPS * 16;          // [waves][NMAPS][Gb][kMergeRow]
    if (grp == 0) {
#pragma unroll
        for (int m = 0; m < NMAPS; ++m) {
            mw[(wave * NMAPS + m) * 16 + colq] = m_run[m];
            lw[(wave * NMAPS + m) * 16 + colq] = lt[m];
        }
    }
    if (colq < Gb) {
#pragma unroll
        for (int m = 0; m < NMAPS; ++m)
#pragma unroll
            for (int db = 0; db < DV / 16; ++db)
                *reinterpret_cast<f32x4 *>(ow + ((wave * NMAPS + m) * Gb + colq) * kMergeRow<DV> + db * 16 +
                                           grp * 4) =
                    o[m][db];
    }
    __syncthreads();
    for (int e = threadIdx.x; e < Gb * DV; e += blockDim.x) {
        const int col = e / DV, dd = e % DV;
        const int64_t head = kv * G + h0 + col;   // b * Hq + query head
        float res = 0.f;
#pragma unroll
        for (int m = 0; m < NMAPS; ++m) {
            float mstar = kNegBig;
            for (int w = 0; w < waves; ++w)
                mstar = fmaxf(mstar, mw[(w * NMAPS + m) * 16 + col]);
            float l = 0.f, acc = 0.f;
            for (int w = 0; w < waves; ++w) {
                const float wgt = __builtin_amdgcn_exp2f(mw[(w * NMAPS + m) * 16 + col] - mstar);
                l += wgt * lw[(w * NMAPS + m) * 16 + col];
                acc += wgt * ow[((w * NMAPS + m) * Gb + col) * kMergeRow<DV> + dd];
            }
            if (p.splits == 1) {
                const float r = l > 0.f ? acc / l : 0.f;
                res += m == 0 ? r : -p.lambda * r;
            } else {
                const int64_t part = (head * p.splits + split) * NMAPS + m;
                p.ws_o[part * DV + dd] = acc;
                if (dd == 0) {
                    p.ws_ml[part * 2] = mstar;
                    p.ws_ml[part * 2 + 1] = l;
                }
            }
        }
        if (p.splits == 1)
            p.out[head * DV + dd] = (__bf16)res;
    }
}

// One wave per (sequence, query head) merges the splits of every map.  All
// partials are loaded up front (at most kDecodeMaxSplits), so the loads overlap.
template <int DV, int NMAPS>
__global__ __launch_bounds__(256) void decode_combine_kernel(const float *ws_ml, const float *ws_o,
                                                             __bf16 *out, int rows, int splits,
                                                             float lambda) {
    constexpr int kPerLane = (DV + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int row = blockIdx.x * 4 + (threadIdx.x >> 6);  // b * Hq + query head
    if (row >= rows)
        return;
    float res[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
        res[i] = 0.f;
#pragma unroll
    for (int m = 0; m < NMAPS; ++m) {
        float ms[kDecodeMaxSplits], ls[kDecodeMaxSplits], os[kDecodeMaxSplits][kPerLane];
#pragma unroll
        for (int s = 0; s < kDecodeMaxSplits; ++s) {
            const int64_t part = (static_cast<int64_t>(row) * splits + (s < splits ? s : 0)) * NMAPS + m;
            ms[s] = s < splits ? ws_ml[part * 2] : kNegBig;
            ls[s] = s < splits ? ws_ml[part * 2 + 1] : 0.f;
#pragma unroll
            for (int i = 0; i < kPerLane; ++i)
                os[s][i] = (s < splits && lane + 64 * i < DV) ? ws_o[part * DV + lane + 64 * i] : 0.f;
        }
        float mstar = kNegBig;
#pragma unroll
        for (int s = 0; s < kDecodeMaxSplits; ++s)
            mstar = fmaxf(mstar, ms[s]);
        float lsum = 0.f, acc[kPerLane];
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            acc[i] = 0.f;
#pragma unroll
        for (int s = 0; s < kDecodeMaxSplits; ++s) {
            const float wgt = __builtin_amdgcn_exp2f(ms[s] - mstar);
            lsum += wgt * ls[s];
#pragma unroll
            for (int i = 0; i < kPerLane; ++i)
                acc[i] += wgt * os[s][i];
        }
        const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            res[i] += (m == 0 ? 1.f : -lambda) * (acc[i] * inv);
    }
#pragma unroll
    for (int i = 0; i < kPerLane; ++i)
        if (lane + 64 * i < DV)
            out[static_cast<int64_t>(row) * DV + lane + 64 * i] = (__bf16)res[i];
}

template <int D, int DV, int NMAPS>
hipError_t launch(const DecodeArgs &a, hipStream_t stream) {
    const DecodePlan plan = decode_plan_for(a);
    Params p;
    for (int m = 0; m < 2; ++m) {
        p.q[m] = static_cast<const __bf16 *>(a.q[m]);
        p.k[m] = static_cast<const __bf16 *>(a.k_ring[m]);
        p.ks[m] = static_cast<const __bf16 *>(a.k_sink[m]);
    }
    p.v = static_cast<const __bf16 *>(a.v_ring);
    p.vs = static_cast<const __bf16 *>(a.v_sink);
    p.seq_len = a.seq_len;
    p.out = static_cast<__bf16 *>(a.out);
    const int64_t rows = static_cast<int64_t>(a.B) * a.Hq;
    p.ws_ml = static_cast<float *>(a.workspace);
    p.ws_o = p.ws_ml + decode_ws_ml_floats(rows * plan.splits * NMAPS);
    p.B = a.B;
    p.Hq = a.Hq;
    p.Hkv = a.Hkv;
    p.N = a.N;
    p.window = a.window;
    p.n_sink = a.n_sink;
    p.splits = plan.splits;
    p.steps_per_wave = plan.steps_per_wave;
    p.c = a.scale * kLog2e;
    p.lambda = a.lambda;

    const int group = a.Hq / a.Hkv;
    const size_t lds = lds_bytes<D, DV, NMAPS>(plan.waves, group < 16 ? group : 16);
    const unsigned grid = static_cast<unsigned>(static_cast<int64_t>(a.B) * a.Hkv * plan.splits);
    const unsigned blocks = static_cast<unsigned>(decode_head_blocks(a.Hq, a.Hkv));
    // one block of query heads reads each ring once: nontemporal loads;
    // without sink slots, loads through ring descriptors
    void (*kernel)(Params) =
        a.n_sink > 0 ? (blocks == 1 ? decode_kernel<D, DV, NMAPS, true, true>
                                    : decode_kernel<D, DV, NMAPS, false, true>)
                     : (blocks == 1 ? decode_kernel<D, DV, NMAPS, true, false>
                                    : decode_kernel<D, DV, NMAPS, false, false>);
    if (lds > 65536) {
        hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           static_cast<int>(lds));
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(kernel, dim3(grid, blocks), dim3(64 * plan.waves),
                       static_cast<unsigned>(lds), stream, p);
    if (plan.splits > 1)
        hipLaunchKernelGGL((decode_combine_kernel<DV, NMAPS>), dim3(static_cast<unsigned>((rows + 3) / 4)),
                           dim3(256), 0, stream, p.ws_ml, p.ws_o, p.out, static_cast<int>(rows),
                           plan.splits, p.lambda);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs &a, hipStream_t stream) {
    static_assert(kDecodeMaxWaves <= 4, "two waves per SIMD: at most 4 waves fit 2 per CU");
    if (a.nmaps == 1) {
        if (a.d != a.dv)
            return hipErrorInvalidValue;
        if (a.d == 32)
            return launch<32, 32, 1>(a, stream);
        if (a.d == 64)
            return launch<64, 64, 1>(a, stream);
        if (a.d == 128)
            return launch<128, 128, 1>(a, stream);
        return hipErrorInvalidValue;
    }
    // two maps: every (d, dv); wide pairs take one register stage
    if (a.d == 32 && a.dv == 32)
        return launch<32, 32, 2>(a, stream);
    if (a.d == 32 && a.dv == 64)
        return launch<32, 64, 2>(a, stream);
    if (a.d == 32 && a.dv == 128)
        return launch<32, 128, 2>(a, stream);
    if (a.d == 64 && a.dv == 32)
        return launch<64, 32, 2>(a, stream);
    if (a.d == 64 && a.dv == 64)
        return launch<64, 64, 2>(a, stream);
    if (a.d == 64 && a.dv == 128)
        return launch<64, 128, 2>(a, stream);
    if (a.d == 128 && a.dv == 32)
        return launch<128, 32, 2>(a, stream);
    if (a.d == 128 && a.dv == 64)
        return launch<128, 64, 2>(a, stream);
    if (a.d == 128 && a.dv == 128)
        return launch<128, 128, 2>(a, stream);
    return hipErrorInvalidValue;
}

}  // namespace swa
