// Block-mask builder ("Attention Variants Compared": create_block_mask turns
// the mask pattern into a per-block keep/skip map once per shape; blocks
// with no attended cell are skipped by the attention kernel).
//
// Three small integer kernels on the caller's stream:
//   1. per query tile, the length of its list            (one thread / tile)
//   2. exclusive scan of the lengths into row_ptr          (one workgroup)
//   3. per list entry, its key tile, kind and cell count   (one workgroup of
//      four waves per query tile)
// Cell counts of band tiles: for the plain window (+ stride) pattern a per-row
// closed form (row i attends the keys max(0, i-window+1) .. i plus the
// multiples of stride in 0 .. i-window, an interval and a progression clipped
// to the key tile); with a dilated window or global tokens every cell of the
// tile is tested, the wave's lanes splitting its rows.  Prefix-only tiles: every row attends every prefix key of
// the tile, so their count is rows x prefix keys.
#include "swa_internal.h"

namespace swa {
namespace {

struct Pattern {
    int64_t N, window, stride, dilation, n_global, bm, bn;
};

// The mask predicate (same definition as the public header).
__device__ bool allowed(const Pattern &p, int64_t i, int64_t j) {
    if (j > i || j < 0 || i >= p.N)
        return false;
    const int64_t dist = i - j;
    return (dist % p.dilation == 0 && dist / p.dilation < p.window) ||
           (p.stride > 0 && j % p.stride == 0) || j < p.n_global || i < p.n_global;
}

// The same predicate in 32-bit arithmetic for indices 0 <= i, j < N (N is at
// most 2^22), the window span clamped to N: the per-cell counting loop.
__device__ bool allowed32(int i, int j, int N, int span, int dil, int stride, int n_global) {
    if (j > i || i >= N)
        return false;
    const int dist = i - j;
    return (dist <= span && dist % dil == 0) || (stride > 0 && j % stride == 0) || j < n_global ||
           i < n_global;
}

struct TileGeom {
    int64_t t_lo;        // first band tile of the query tile
    int64_t n_band;      // number of band tiles
    int64_t a;           // prefix-only tiles [0, a) hold a global column
    int64_t n_prefix;    // number of prefix-only tiles (all left of t_lo)
    int64_t prefix_keys; // prefix keys left of the band
};

// multiples of s (s > 0) in [a, b), a >= 0
__device__ int64_t multiples_in(int64_t a, int64_t b, int64_t s) {
    if (b <= a)
        return 0;
    return (b + s - 1) / s - (a + s - 1) / s;
}

__device__ TileGeom tile_geom(int64_t q, const Pattern &p) {
    TileGeom g;
    const int64_t r0 = q * p.bm;
    const int64_t r1 = (r0 + p.bm < p.N ? r0 + p.bm : p.N) - 1;
    const int64_t span = (p.window - 1) * p.dilation;
    const int64_t lo = r0 - span > 0 ? r0 - span : 0;
    g.t_lo = lo / p.bn;
    g.n_band = r1 / p.bn - g.t_lo + 1;
    g.a = (p.n_global + p.bn - 1) / p.bn;
    g.a = g.a < g.t_lo ? g.a : g.t_lo;
    int64_t ns = 0;
    if (p.stride > 0 && g.t_lo > g.a)
        ns = p.stride <= p.bn ? g.t_lo - g.a : multiples_in(g.a * p.bn, g.t_lo * p.bn, p.stride);
    g.n_prefix = g.a + ns;
    const int64_t P = g.t_lo * p.bn;
    const int64_t gp = p.n_global < P ? p.n_global : P;
    g.prefix_keys = gp + (p.stride > 0 ? multiples_in(gp, P, p.stride) : 0);
    return g;
}

__global__ void mask_count_kernel(int32_t *row_ptr, int nq, Pattern p) {
    int q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q == 0)
        row_ptr[0] = 0;
    if (q >= nq)
        return;
    TileGeom g = tile_geom(q, p);
    row_ptr[q + 1] = static_cast<int32_t>(g.n_band + g.n_prefix);
}

// In-place inclusive scan of row_ptr[1..nq] by one workgroup of 1024 threads:
// each thread owns a contiguous chunk, chunk totals are scanned in LDS.
__global__ __launch_bounds__(1024) void mask_scan_kernel(int32_t *row_ptr, int nq) {
    __shared__ int64_t part[1024];
    int t = threadIdx.x;
    int per = (nq + 1023) / 1024;
    int a = t * per, b = a + per < nq ? a + per : nq;
    int64_t s = 0;
    for (int i = a; i < b; ++i)
        s += row_ptr[i + 1];
    part[t] = s;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
        int64_t add = t >= off ? part[t - off] : 0;
        __syncthreads();
        part[t] += add;
        __syncthreads();
    }
    int64_t run = t > 0 ? part[t - 1] : 0;
    for (int i = a; i < b; ++i) {
        run += row_ptr[i + 1];
        row_ptr[i + 1] = static_cast<int32_t>(run);
    }
}

__global__ __launch_bounds__(256) void mask_fill_kernel(const int32_t *row_ptr, int32_t *kv_tile,
                                                       uint8_t *kind, int32_t *cells,
                                                       int32_t *prefix_keys, int32_t *band_begin,
                                                       Pattern p) {
    const int64_t q = blockIdx.x;
    const TileGeom g = tile_geom(q, p);
    const int64_t base = row_ptr[q];
    if (threadIdx.x == 0) {
        prefix_keys[q] = static_cast<int32_t>(g.prefix_keys);
        band_begin[q] = static_cast<int32_t>(base + g.n_prefix);
    }
    const bool plain = p.dilation == 1 && p.n_global == 0;
    const int64_t i0 = q * p.bm, i1 = i0 + p.bm < p.N ? i0 + p.bm : p.N;
    const int64_t count = g.n_band + g.n_prefix;
    if (!plain) {
        // dilated window or global tokens: each wave takes every fourth band
        // tile, its lanes splitting the tile's rows (each lane tests its rows'
        // cells), then a wave sum of the counts.  dist <= span with dist a
        // multiple of the dilation is the window term of the predicate.
        const int span = static_cast<int>((p.window - 1) * p.dilation < p.N ? (p.window - 1) * p.dilation : p.N);
        const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
        for (int64_t e = g.n_prefix + wave; e < count; e += blockDim.x >> 6) {
            const int64_t t = g.t_lo + (e - g.n_prefix);
            const int j0 = static_cast<int>(t * p.bn), j1 = static_cast<int>(j0 + p.bn < p.N ? j0 + p.bn : p.N);
            int c = 0;
            for (int i = static_cast<int>(i0) + lane; i < i1; i += 64)
                for (int j = j0; j < j1; ++j)
                    c += allowed32(i, j, static_cast<int>(p.N), span, static_cast<int>(p.dilation),
                                   static_cast<int>(p.stride), static_cast<int>(p.n_global));
            for (int off = 32; off > 0; off >>= 1)
                c += __shfl_xor(c, off);
            if (lane == 0) {
                kv_tile[base + e] = static_cast<int32_t>(t);
                kind[base + e] = c == (i1 - i0) * (j1 - j0) ? 0 : 1;
                cells[base + e] = static_cast<int32_t>(c);
            }
        }
    }
    // prefix-only tiles (closed form), and every tile of the plain pattern
    const int64_t n_lane = plain ? count : g.n_prefix;
    for (int64_t e = threadIdx.x; e < n_lane; e += blockDim.x) {
        int64_t t;
        if (e < g.a)
            t = e;  // holds a global column
        else if (e < g.n_prefix)
            t = p.stride <= p.bn ? e  // every tile holds a multiple of stride
                                 : ((g.a * p.bn + p.stride - 1) / p.stride + (e - g.a)) * p.stride / p.bn;
        else
            t = g.t_lo + (e - g.n_prefix);
        const int64_t j0 = t * p.bn, j1 = j0 + p.bn < p.N ? j0 + p.bn : p.N;
        int64_t c = 0;
        uint8_t k;
        if (e < g.n_prefix) {
            // every row attends the tile's global columns and stride multiples
            const int64_t ge = j1 < p.n_global ? j1 : p.n_global;
            const int64_t ng = ge > j0 ? ge - j0 : 0;
            const int64_t from = j0 > p.n_global ? j0 : p.n_global;
            const int64_t nsk = p.stride > 0 ? multiples_in(from, j1, p.stride) : 0;
            c = (i1 - i0) * (ng + nsk);
            k = 2;
        } else {
            for (int64_t i = i0; i < i1; ++i) {
                const int64_t lo = i - p.window + 1 > 0 ? i - p.window + 1 : 0;
                const int64_t a = lo > j0 ? lo : j0;
                const int64_t b = i < j1 - 1 ? i : j1 - 1;
                if (b >= a)
                    c += b - a + 1;
                if (p.stride > 0) {
                    const int64_t sb = j1 < lo ? j1 : lo;
                    c += multiples_in(j0, sb, p.stride);
                }
            }
            k = c == (i1 - i0) * (j1 - j0) ? 0 : 1;
        }
        kv_tile[base + e] = static_cast<int32_t>(t);
        kind[base + e] = k;
        cells[base + e] = static_cast<int32_t>(c);
    }
}

__global__ void mask_dense_kernel(uint8_t *out, Pattern p) {
    const int64_t total = p.N * p.N;
    for (int64_t x = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; x < total;
         x += static_cast<int64_t>(gridDim.x) * blockDim.x)
        out[x] = allowed(p, x / p.N, x % p.N) ? 1 : 0;
}

}  // namespace

hipError_t launch_block_mask_build(const swa_block_mask_t &m, hipStream_t stream) {
    const int nq = m.num_q_tiles;
    const Pattern p{m.N, m.window, m.stride, m.dilation, m.n_global, m.bm, m.bn};
    hipLaunchKernelGGL(mask_count_kernel, dim3((nq + 255) / 256), dim3(256), 0, stream, m.row_ptr,
                       nq, p);
    hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(1024), 0, stream, m.row_ptr, nq);
    hipLaunchKernelGGL(mask_fill_kernel, dim3(nq), dim3(256), 0, stream, m.row_ptr, m.kv_tile,
                       m.kind, m.cells, m.prefix_keys, m.band_begin, p);
    return hipGetLastError();
}

hipError_t launch_mask_dense(int N, int window, int stride, int dilation, int n_global, uint8_t *out,
                             hipStream_t stream) {
    const Pattern p{N, window, stride, dilation, n_global, 1, 1};
    int64_t blocks = (p.N * p.N + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(mask_dense_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       out, p);
    return hipGetLastError();
}

}  // namespace swa
