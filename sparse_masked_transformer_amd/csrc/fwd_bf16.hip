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
// Workgroup: 4 waves per score map; wave w of a map owns query rows
// q0 + 32 w .. q0 + 32 w + 31 of the 128-row query tile.  With two maps
// (differential attention) waves 0-3 compute the first map and waves 4-7 the
// second, on the same rows and the same staged K and V tiles; at the end the
// second map's waves hand lambda * O2 / l2 to the first's through LDS.  Per
// 64-key tile:
//   * K (and V) tiles go HBM -> LDS by LDS-DMA (buffer_load ... lds, no
//     registers), double-buffered; the next tile's loads are in flight while
//     the current tile is computed.  LDS rows are padded (bank spread).
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
//     inside every row's window (or made of global columns only) skip the
//     per-cell mask.
// Problems with a stride or global tokens first visit a dense prefix of the
// keys left of the query tile's band that every row of the tile attends (the
// global columns 0 .. g-1, then the stride keys s, 2s, ...), gathered 64 at a
// time, then the band tiles.  In a band tile a cell attends if it lies on the
// (dilated) window -- distance i - j a multiple of the dilation, at most
// (window-1)*dilation -- or its key is a stride key or a global column
// (Learn: Sparse & Sliding-Window Attention, §3b, for dilation and global
// tokens).
#include <type_traits>

#include "swa_internal.h"

namespace swa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// log2 units the running maximum may lag: p = exp2(s c - m) stays below
// 2^kSlack, so bf16 P keeps its relative precision, the fp32 sums of p and
// p v stay finite for |v| up to 2^(128 - kSlack - 10) over 2^10 keys, and
// sharply peaked rows seldom move the maximum (and rescale O)
constexpr float kSlack = 32.0f;
constexpr float kNegBig = -1e30f;    // running maximum before any key
constexpr int kThreads = kFwdThreads;
constexpr int kDiffThreads = kDiffFwdThreads;
// dword 3 of a raw (untyped) buffer descriptor on gfx950
constexpr int kBufferDword3 = 0x00020000;
// cache-policy bits of the band-tile loads: sc0 (with LDS-DMA staging equal
// to the default and to sc1 on the window prefill; nt, alone or with sc0, is
// ~8% slower)
constexpr int kTileLoadPolicy = 1;

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
    static_assert(kTile % 1024 == 0 && vTile % 1024 == 0, "tiles are whole 1 KiB DMA chunks");
};

struct Params {
    const __bf16 *q[2];
    const __bf16 *k[2];
    const __bf16 *v;
    __bf16 *out;
    float *lse;
    MaskView mask;
    int B, Hq, Hkv, N, window, stride, dilation, n_global;
    float c;        // scale * log2(e)
    float lambda;
};

// MODE 0: the window (and stride) pattern.  MODE 1: the pattern may also
// have a dilated window or global tokens (tested per cell).  MODE 2: a
// dilated window alone, computed as a plain window of `window` keys on each
// residue class r, r + dil, r + 2 dil, ... of the sequence (Learn: Sparse &
// Sliding-Window Attention, §3b: row i attends keys i - m dil; rows and keys
// of one class form an ordinary sliding-window problem of length
// ceil((N - r) / dil)), so no cell off the lattice is computed.  In MODE 2
// the workgroup's class is part of its tile index, row and key indices are
// class-local, and position = r + dil * index.
// Bits lo..hi (inclusive) of a 32-bit word, the range clipped to 0..31;
// zero when it is empty.
__device__ __forceinline__ uint32_t bit_range(int lo, int hi) {
    lo = lo < 0 ? 0 : lo;
    hi = hi > 31 ? 31 : hi;
    if (hi < lo)
        return 0u;
    return ((2u << hi) - 1u) & (~0u << lo);   // 2u << 31 wraps to 0: all bits
}

constexpr int kNegInfBits = static_cast<int>(0xff800000u);   // -inf as fp32 bits

template <int D, int DV, int NMAPS, int RG, int MODE>
__device__ __forceinline__ void fwd_bf16_body(const Params &p) {
    constexpr int WAVES = 4 * NMAPS;   // waves per workgroup: 4 per score map
    constexpr bool EXT = MODE == 1;
    const int dil = EXT ? p.dilation : 1;
    const int n_glob = EXT ? p.n_global : 0;
    const int rdil = MODE == 2 ? p.dilation : 1;   // position stride of the rows
    using C = Cfg<D, DV, NMAPS>;
    constexpr int BM = 128 * RG;       // query rows per workgroup
    constexpr int ROWS = 32 * RG;      // query rows per wave (RG groups of 32)
    // two K/V stages; with two maps also the second map's output at the end
    constexpr int kXo = NMAPS == 2 ? 4 * RG * (DV / 32) * 16 * 64 * 4 : 0;
    __shared__ __attribute__((aligned(16))) char smem[2 * C::stage > kXo ? 2 * C::stage : kXo];

    const int tid = threadIdx.x, lane = tid & 63, wave_id = tid >> 6;
    const int wmap = wave_id >> 2;     // score map of this wave
    const int wave = wave_id & 3;      // its rows within the query tile
    const int hl = lane >> 5;          // which half of the wave
    const int col = lane & 31;         // query column within a row group
    const int G = p.Hq / p.Hkv;
    // query tiles per (batch, head): MODE 2 has rdil classes of up to
    // ceil(N / rdil) rows each
    const int nq_cls = ((p.N + rdil - 1) / rdil + BM - 1) / BM;
    const int nq = MODE == 2 ? nq_cls * rdil : p.mask.num_q_tiles;

    // ---- workgroup -> (b, kv head, query tile, head in group) -------------
    // Consecutive workgroup ids go to the 8 XCDs in turn; remap so each XCD
    // receives a contiguous run of logical ids (the same key/value head, so
    // its L2 serves the query heads of the group and neighbouring tiles).
    int total = gridDim.x, pid = blockIdx.x, lid = pid;
    if ((total & 7) == 0)
        lid = (pid & 7) * (total >> 3) + (pid >> 3);
    const int hg = lid % G;
    int rest = lid / G;
    const int qt_lin = nq - 1 - (rest % nq);  // long (late) query tiles first
    rest /= nq;
    const int qt = MODE == 2 ? qt_lin / rdil : qt_lin;   // tile within the class
    const int res = MODE == 2 ? qt_lin % rdil : 0;       // residue class
    const int Nr = MODE == 2 ? (p.N - res + rdil - 1) / rdil : p.N;  // rows of the class
    // MODE 2: classes differ in length by one row; a class may have no rows
    // (N < dil) or none in its last tile -- nothing to do (uniform exit)
    if (MODE == 2 && qt * BM >= Nr)
        return;
    const int g = rest % p.Hkv;
    const int b = rest / p.Hkv;
    const int h = g * G + hg;

    const int q0 = qt * BM + wave * ROWS;  // first row of this wave
    int my_row[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
        my_row[rg] = q0 + 32 * rg + col;

    // ---- Q^T fragments (B operand), one per 16-channel step ----------------
    bf16x8 qf[RG][D / 16];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const int row = my_row[rg] < Nr ? my_row[rg] : Nr - 1;
        const int64_t q_off = ((int64_t)(b * p.Hq + h) * p.N + res + rdil * row) * D;
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            qf[rg][ks] = *reinterpret_cast<const bf16x8 *>(p.q[wmap] + q_off + ks * 16 + hl * 8);
    }

    // ---- the walk: prefix chunks, then band tiles --------------------------
    // (MODE 2: the band of the class-local rows in closed form, no prefix)
    const int cls_r0 = qt * BM, cls_r1 = (cls_r0 + BM < Nr ? cls_r0 + BM : Nr) - 1;
    const int cls_lo = cls_r0 - p.window + 1 > 0 ? cls_r0 - p.window + 1 : 0;
    const int sk = MODE == 2 ? 0 : p.mask.prefix_keys[qt];
    // prefix key kn: kn itself below gp (global columns), then stride multiples
    const int gp = n_glob < sk ? n_glob : sk;
    const int s_first = p.stride > 0 ? (gp + p.stride - 1) / p.stride - gp : 0;
    const int n_pre = (sk + 63) >> 6;
    const int band0 = MODE == 2 ? 0 : p.mask.band_begin[qt];
    const int n_items = MODE == 2 ? cls_r1 / 64 - cls_lo / 64 + 1
                                  : n_pre + (p.mask.row_ptr[qt + 1] - band0);
    // The band tiles of a query tile are one ascending run of consecutive key
    // tiles, so only the first is read (once, here).  A per-tile read of the
    // list inside the loop is a vector load whose wait also waits for the
    // next tile's prefetch, which would serialise every tile behind it.
    const int band_t0 = MODE == 2 ? cls_lo / 64 : p.mask.kv_tile[band0];
    const int64_t kv_head = (int64_t)(b * p.Hkv + g) * p.N;

    // window span in keys, and the dilation lattice: bit m set iff m is a
    // multiple of the dilation (m < 64)
    const int64_t span64 = static_cast<int64_t>(p.window - 1) * dil;
    const int span = span64 < p.N ? static_cast<int>(span64) : p.N;  // distances are < N
    uint64_t lattice = 0;
    for (int m = 0; m < 64; m += dil)
        lattice |= 1ull << m;

    // first key of item it (band tiles only)
    auto item_key0 = [&](int it) -> int {
        return it >= n_pre ? (band_t0 + (it - n_pre)) * 64 : 0;
    };

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
    // LDS-DMA staging: buffer_load ... lds writes 16 bytes per lane straight
    // into LDS, lane l at bytes 16 l .. 16 l + 15 of a wave-uniform 1 KiB
    // chunk.  A tile of 64 padded rows is a whole number of chunks; wave w
    // writes chunks w, w + WAVES, ...  Lane l of chunk ch covers tile byte
    // 1024 ch + 16 l, i.e. a row and a column of the padded layout; lanes on
    // padding fetch their row's first 16 bytes (padding is never read).
    constexpr int kCh = C::kTile / 1024, vCh = C::vTile / 1024;
    constexpr int kChW = (kCh + WAVES - 1) / WAVES, vChW = (vCh + WAVES - 1) / WAVES;   // chunks per wave, at most
    const int wv = __builtin_amdgcn_readfirstlane(wave_id);
    int dk_row[kChW], dk_col[kChW], dv_row[vChW], dv_col[vChW];
#pragma unroll
    for (int j = 0; j < kChW; ++j) {
        const int pos = (wv + WAVES * j) * 1024 + 16 * lane;
        const int cb = pos % C::kRow;
        dk_row[j] = pos / C::kRow;
        dk_col[j] = cb < 2 * D ? cb : 0;
    }
#pragma unroll
    for (int j = 0; j < vChW; ++j) {
        const int pos = (wv + WAVES * j) * 1024 + 16 * lane;
        const int cb = pos % C::vRow;
        dv_row[j] = pos / C::vRow;
        dv_col[j] = cb < 2 * DV ? cb : 0;
    }
    typedef __attribute__((address_space(3))) void lds_void;
    auto dma_stage = [&](int it, int buf) {
        char *sb = smem + buf * C::stage;
        if (it >= n_pre) {
            // window tile: rows key0 .. key0+63 (the tile offset is scalar)
            const int key0 = item_key0(it);
            const int kso = (res + rdil * key0) * D * 2, vso = (res + rdil * key0) * DV * 2;
#pragma unroll
            for (int j = 0; j < kChW; ++j)
                if (wv + WAVES * j < kCh)
#pragma unroll
                    for (int m = 0; m < NMAPS; ++m)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            krs[m], (lds_void *)(sb + m * C::kTile + (wv + WAVES * j) * 1024), 16,
                            rdil * dk_row[j] * D * 2 + dk_col[j], kso, 0, kTileLoadPolicy);
#pragma unroll
            for (int j = 0; j < vChW; ++j)
                if (wv + WAVES * j < vCh)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        vrs, (lds_void *)(sb + NMAPS * C::kTile + (wv + WAVES * j) * 1024), 16,
                        rdil * dv_row[j] * DV * 2 + dv_col[j], vso, 0, kTileLoadPolicy);
        } else {
            // prefix chunk: key rows of prefix keys kn < sk (others read past
            // the end, i.e. zeros)
#pragma unroll
            for (int j = 0; j < kChW; ++j)
                if (wv + WAVES * j < kCh) {
                    const int kn = it * 64 + dk_row[j];
                    const int row = kn < gp ? kn : (kn < sk ? (s_first + kn) * p.stride : p.N);
#pragma unroll
                    for (int m = 0; m < NMAPS; ++m)
                        __builtin_amdgcn_raw_ptr_buffer_load_lds(
                            krs[m], (lds_void *)(sb + m * C::kTile + (wv + WAVES * j) * 1024), 16,
                            row * D * 2 + dk_col[j], 0, 0, 0);
                }
#pragma unroll
            for (int j = 0; j < vChW; ++j)
                if (wv + WAVES * j < vCh) {
                    const int kn = it * 64 + dv_row[j];
                    const int row = kn < gp ? kn : (kn < sk ? (s_first + kn) * p.stride : p.N);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        vrs, (lds_void *)(sb + NMAPS * C::kTile + (wv + WAVES * j) * 1024), 16,
                        row * DV * 2 + dv_col[j], 0, 0, 0);
                }
        }
    };

    // per-lane LDS read bases (everything else is a compile-time offset)
    const int grp = lane >> 4, sl = lane & 15;
    const int k_lane = col * C::kRow + hl * 16;
    const int v_lane = (4 * (grp >> 1) + (sl >> 2)) * C::vRow + (16 * (grp & 1) + 4 * (sl & 3)) * 2;

    // ---- running state of this wave's map, per row group ---------------------
    f32x16 o[RG][DV / 32];
    float m_run[RG], l_run[RG];
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        m_run[rg] = kNegBig;
        l_run[rg] = 0.f;
#pragma unroll
        for (int db = 0; db < DV / 32; ++db)
            o[rg][db] = f32x16{};
    }

    if (n_items > 0)
        dma_stage(0, 0);
    __syncthreads();
    // Wait for Q here, after the first tile's staging, so that its loads
    // overlap the block-mask reads and the first tile's loads.  Left pending
    // into the loop, its first use there gets a count-based wait on every
    // iteration, and as the load counter runs in issue order that wait would
    // also wait for the next tile's prefetch.
#pragma unroll
    for (int rg = 0; rg < RG; ++rg)
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
            asm volatile("" ::"v"(qf[rg][ks]));

    for (int it = 0; it < n_items; ++it) {
        const int buf = it & 1;
        // prefetch the next item straight into the other buffer, whose last
        // reads ended at the previous barrier
        if (it + 1 < n_items)
            dma_stage(it + 1, buf ^ 1);

        // ---- classify this tile for each row group of this wave -------------
        const bool pre = it < n_pre;
        const int key0 = item_key0(it);
        // column keys of a band tile (stride keys, global columns), one bit per
        // key of the tile; every row at or after such a key attends it
        uint64_t smask = 0;
        if (!pre && p.stride > 0) {
            const int f = ((key0 + p.stride - 1) / p.stride) * p.stride;
            for (int j = f; j < key0 + 64; j += p.stride)
                smask |= 1ull << (j - key0);
        }
        if (!pre && key0 < n_glob)
            smask |= n_glob - key0 >= 64 ? ~0ull : (1ull << (n_glob - key0)) - 1;
        bool full[RG], any = false;
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
            const int r0 = q0 + 32 * rg, r1 = r0 + 31;
            bool empty;
            if (pre) {
                empty = false;
                full[rg] = (it + 1) * 64 <= sk;
            } else {
                empty = key0 > r1 || (key0 + 63 < r0 - span && smask == 0);
                full[rg] = !empty && key0 + 63 <= r0 && key0 + 64 <= Nr &&
                           ((dil == 1 && key0 >= r1 - p.window + 1) || key0 + 64 <= n_glob);
            }
            any = any || !empty;
        }

        if (any) {
            const char *kb_base = smem + buf * C::stage + k_lane;
            const char *vb_base = smem + buf * C::stage + NMAPS * C::kTile + v_lane;

            // Scores of row group rg, key half kb (32 keys): S^T = K Q^T.
            f32x16 sh[RG][2];
            bf16x8 ka[D / 16];
            auto read_k = [&](int kb) {
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks)
                    ka[ks] = *reinterpret_cast<const bf16x8 *>(
                        kb_base + wmap * C::kTile + kb * 32 * C::kRow + ks * 32);
            };
            auto qk = [&](int rg, int kb) {
                f32x16 acc = f32x16{};
#pragma unroll
                for (int ks = 0; ks < D / 16; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[ks], qf[rg][ks], acc, 0, 0, 0);
                sh[rg][kb] = acc;
            };
            // per-cell mask (branch-free selects); lane key kk = kb*32 + kc +
            // 4*hl with kc a compile-time constant
            auto mask = [&](int rg, int kb) {
                const float ninf = -__builtin_inff();
                if (pre) {
                    const int lim = sk - it * 64 - kb * 32 - 4 * hl;  // attended iff kc < lim
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kcst = (r & 3) + 8 * (r >> 2);
                        sh[rg][kb][r] = kcst < lim ? sh[rg][kb][r] : ninf;
                    }
                } else {
                    // One bit word per lane for its 16 cells (bit kc: key
                    // kb*32 + kc + 4*hl), then one bit-field select per cell.
                    // dist = i - j = base - kc; the window part is 0 <= dist < W
                    // (dilation 1), else dist <= span on the dilation lattice;
                    // column keys (smask) count wherever dist >= 0.
                    const int base = my_row[rg] - key0 - kb * 32 - 4 * hl;
                    uint32_t bits;
                    if (dil == 1) {
                        const int64_t lo = static_cast<int64_t>(base) - p.window + 1;
                        bits = bit_range(lo > 0 ? static_cast<int>(lo) : 0, base);
                    } else {
                        // lattice bit kc set iff base - kc is a multiple of the dilation
                        int res = base % dil;
                        res += res < 0 ? dil : 0;
                        bits = bit_range(base - span, base) & static_cast<uint32_t>(lattice << res);
                    }
                    if (smask != 0)
                        bits |= static_cast<uint32_t>(smask >> (kb * 32 + 4 * hl)) & bit_range(0, base);
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int kcst = (r & 3) + 8 * (r >> 2);
                        // all ones iff bit kcst is set (sign-extended bit field)
                        const int keep = static_cast<int>(bits << (31 - kcst)) >> 31;
                        // through a scalar: a bit_cast of the vector element itself
                        // reads element 0 (hipcc of ROCm 7.2)
                        const float sc = sh[rg][kb][r];
                        const int sv = __builtin_bit_cast(int, sc);
                        sh[rg][kb][r] = __builtin_bit_cast(float, (sv & keep) | (kNegInfBits & ~keep));
                    }
                }
            };
            // Online softmax, split in two phases: the row maximum and the
            // rescale decision (wave-uniform branch), then the exponentials
            // (branch-free, so the scheduler can interleave them with MFMAs).
            // l is rescaled here, O by rescale_o once every PV product that
            // used the old maximum has been accumulated.
            float alpha[RG];
            auto softmax_max = [&](int rg, int kb) -> bool {
                bool moved = false;
                const f32x16 &sv = sh[rg][kb];
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
                alpha[rg] = 1.f;
                if (__builtin_amdgcn_ballot_w64(mxs > m_run[rg] + kSlack) != 0) {
                    const float m_new = fmaxf(m_run[rg], mxs);
                    alpha[rg] = __builtin_amdgcn_exp2f(m_run[rg] - m_new);
                    l_run[rg] *= alpha[rg];
                    m_run[rg] = m_new;
                    moved = true;
                }
                return moved;
            };
            auto rescale_o = [&](int rg) {
#pragma unroll
                for (int db = 0; db < DV / 32; ++db)
                    o[rg][db] *= alpha[rg];
            };
            bf16x8 pf[RG][2][2];
            // Row sums over the bf16-rounded p, the values the P V product
            // accumulates (v_dot2 of a packed pair with ones): the weights of
            // a row then sum to one exactly after the division, whatever the
            // running maximum's lag.
            auto softmax_exp = [&](int rg, int kb) {
                const f32x16 &sv = sh[rg][kb];
                const float nm = -m_run[rg];
                const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
                float lsum[4] = {0.f, 0.f, 0.f, 0.f};  // independent partial sums
#pragma unroll
                for (int hf = 0; hf < 2; ++hf) {
                    bf16x8 v8;
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        v8[e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sv[hf * 8 + e], p.c, nm));
                    pf[rg][kb][hf] = v8;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        lsum[e] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{v8[2 * e], v8[2 * e + 1]}, ones, lsum[e],
                                                                  false);
                }
                l_run[rg] += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
            };
            // keep a block's exponentials in that block (otherwise they are
            // sunk past the next branch, next to their use)
            auto pin = [&](int rg, int kb) {
                asm volatile("" ::"v"(pf[rg][kb][0]), "v"(pf[rg][kb][1]), "v"(l_run[rg]));
            };
            // V^T fragments of key half kb, shared by every row group
            bf16x8 va[2][DV / 32];
            auto join = [](i16x4 t0, i16x4 t1) {
                const bf16x4 a0 = __builtin_bit_cast(bf16x4, t0);
                const bf16x4 a1 = __builtin_bit_cast(bf16x4, t1);
                return bf16x8{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            };
            // (the compiler waits for the outstanding LDS-DMA loads before
            // these reads, as it cannot tell their buffers apart; the next
            // tile's loads, issued at the top of the tile, have landed by then)
            auto read_v = [&](int kb) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int db = 0; db < DV / 32; ++db) {
                        const char *a = vb_base + (kb * 32 + hf * 16) * C::vRow + db * 64;
                        va[hf][db] = join(__builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)a),
                                          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a + 8 * C::vRow)));
                    }
            };
            // O^T += V^T P^T over the 32 keys of half kb
            auto pv = [&](int rg, int kb) {
#pragma unroll
                for (int hf = 0; hf < 2; ++hf)
#pragma unroll
                    for (int db = 0; db < DV / 32; ++db)
                        o[rg][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            va[hf][db], pf[rg][kb][hf], o[rg][db], 0, 0, 0);
            };
            // scheduling hint for one branch-free block: alternate one MFMA
            // with a few VALU instructions
            auto interleave = [&](auto n_mfma) {
#pragma unroll
                for (int i = 0; i < decltype(n_mfma)::value; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
                }
            };
            using QkMfma = std::integral_constant<int, D / 16>;
            using PvMfma = std::integral_constant<int, 2 * (DV / 32)>;

            // ---- the tile, software-pipelined over (row group, key half) ----
            read_k(0);
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
                qk(rg, 0);
            read_k(1);                     // in flight during the maxima below
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                if (!full[rg])
                    mask(rg, 0);
                if (softmax_max(rg, 0))
                    rescale_o(rg);
            }
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                qk(rg, 1);                 // matrix work ...
                softmax_exp(rg, 0);        // ... overlapped with exponentials
                interleave(QkMfma{});
                pin(rg, 0);
            }
            read_v(0);                     // in flight during the maxima below
            bool moved[RG];
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                if (!full[rg])
                    mask(rg, 1);
                moved[rg] = softmax_max(rg, 1);
            }
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                pv(rg, 0);                 // probabilities of the old maximum ...
                softmax_exp(rg, 1);        // ... overlapped with exponentials
                interleave(PvMfma{});
                pin(rg, 1);
                if (moved[rg])
                    rescale_o(rg);
            }
            read_v(1);
#pragma unroll
            for (int rg = 0; rg < RG; ++rg)
                pv(rg, 1);
        }

        __syncthreads();   // preceded by a wait for this wave's DMA loads
    }

    // ---- epilogue: O / l -> bf16 ------------------------------------------
    // Two maps: the second map's waves hand lambda * O2 / l2 to the first
    // map's waves through LDS (the stages are free after the last barrier),
    // in register order, lane-major; those store O1 / l1 minus it.
    static_assert(kXo <= sizeof(smem), "the second map's output fits the LDS array");
    float *xo = reinterpret_cast<float *>(smem);
    auto xo_at = [&](int rg, int db, int r) -> float & {
        return xo[(((wave * RG + rg) * (DV / 32) + db) * 16 + r) * 64 + lane];
    };
    if constexpr (NMAPS == 2) {
        if (wmap == 1) {
#pragma unroll
            for (int rg = 0; rg < RG; ++rg) {
                const float lt = l_run[rg] + __shfl_xor(l_run[rg], 32);
                const float sc = lt > 0.f ? p.lambda / lt : 0.f;
#pragma unroll
                for (int db = 0; db < DV / 32; ++db)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        xo_at(rg, db, r) = o[rg][db][r] * sc;
            }
        }
        __syncthreads();
        if (wmap == 1)
            return;
    }
#pragma unroll
    for (int rg = 0; rg < RG; ++rg) {
        const float lt = l_run[rg] + __shfl_xor(l_run[rg], 32);
        const float inv = lt > 0.f ? 1.f / lt : 0.f;
        if (NMAPS == 1 && p.lse != nullptr && hl == 0 && my_row[rg] < Nr)
            p.lse[(int64_t)(b * p.Hq + h) * p.N + res + rdil * my_row[rg]] =
                lt > 0.f ? (m_run[rg] + __builtin_log2f(lt)) * kLn2 : -__builtin_inff();
        if (my_row[rg] < Nr) {
            __bf16 *dst = p.out + ((int64_t)(b * p.Hq + h) * p.N + res + rdil * my_row[rg]) * DV;
#pragma unroll
            for (int db = 0; db < DV / 32; ++db)
#pragma unroll
                for (int r4 = 0; r4 < 4; ++r4) {
                    bf16x4 v4;
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        float x = o[rg][db][r4 * 4 + i] * inv;
                        if (NMAPS == 2)
                            x -= xo_at(rg, db, r4 * 4 + i);
                        v4[i] = (__bf16)x;
                    }
                    *reinterpret_cast<bf16x4 *>(dst + db * 32 + 8 * r4 + 4 * hl) = v4;
                }
        }
    }
}

// Single-map kernels with one row group (32 rows per wave) fit in 256
// registers per lane, so at least two waves share each SIMD (one wave's
// softmax overlaps another's matrix work).  Only the minimum is given: a
// maximum of two makes the compiler declare extra registers to enforce it,
// and at d=64 (143 registers, 42 KiB LDS) a third workgroup per CU runs the
// local+strided workload 17% faster.
template <int D, int DV, int MODE>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kFwdRowGroups == 1 ? 2 : 1)))
void fwd_bf16_kernel(Params p) {
    fwd_bf16_body<D, DV, 1, kFwdRowGroups, MODE>(p);
}

// Two maps on separate waves (8 per workgroup, two per SIMD): a wave holds one
// map's state (191 registers at d=64, dv=128).  Both maps in every wave need
// ~316 registers, one wave per SIMD, and run the differential workload 13%
// slower.
template <int D, int DV, int MODE>
__global__ __launch_bounds__(kDiffThreads) __attribute__((amdgpu_waves_per_eu(2)))
void diff_bf16_kernel(Params p) {
    fwd_bf16_body<D, DV, 2, kDiffRowGroups, MODE>(p);
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
    p.dilation = a.dilation;
    p.n_global = a.n_global;
    p.c = a.scale * kLog2e;
    p.lambda = a.lambda;
    const bool ext = a.dilation != 1 || a.n_global != 0;
    const unsigned grid = static_cast<unsigned>(fwd_workgroups(a, SWA_BF16));
    if constexpr (NMAPS == 1) {
        if (fwd_by_residue_class(a, SWA_BF16)) {
            hipLaunchKernelGGL((fwd_bf16_kernel<D, DV, 2>), dim3(grid), dim3(kThreads), 0, stream, p);
            return hipGetLastError();
        }
    }
    if constexpr (NMAPS == 1) {
        if (ext)
            hipLaunchKernelGGL((fwd_bf16_kernel<D, DV, 1>), dim3(grid), dim3(kThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((fwd_bf16_kernel<D, DV, 0>), dim3(grid), dim3(kThreads), 0, stream, p);
    } else {
        if (ext)
            hipLaunchKernelGGL((diff_bf16_kernel<D, DV, 1>), dim3(grid), dim3(kDiffThreads), 0, stream, p);
        else
            hipLaunchKernelGGL((diff_bf16_kernel<D, DV, 0>), dim3(grid), dim3(kDiffThreads), 0, stream, p);
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs &a, hipStream_t stream) {
    if (fwd_gqa_applies(a))
        return launch_fwd_gqa(a, stream);
    if (fwd_diff_asm_applies(a))
        return launch_fwd_diff_asm(a, stream);
    if (fwd_str_applies(a))
        return launch_fwd_str(a, stream);
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
        SWA_DIFF_CASE(128, 32)
        SWA_DIFF_CASE(128, 64)
        SWA_DIFF_CASE(128, 128)
#undef SWA_DIFF_CASE
    }
    return hipErrorInvalidValue;
}

}  // namespace swa
