// Block-mask builder ("Attention Variants Compared": create_block_mask turns
// the window/stride pattern into a per-block keep/skip map once per shape;
// blocks with no attended cell are skipped by the attention kernel).
//
// Three small integer kernels on the caller's stream:
//   1. per query tile, the length of its list            (one thread / tile)
//   2. exclusive scan of the lengths into row_ptr          (one workgroup)
//   3. per list entry, its key tile, kind and cell count   (one wave / tile)
// Cell counts use a per-row closed form: row i attends the keys
// max(0, i-window+1) .. i of the window plus the multiples of stride in
// 0 .. i-window; both sets are intervals (or an arithmetic progression)
// clipped to the key tile.
#include "swa_internal.h"

namespace swa {
namespace {

struct TileGeom {
    int64_t t_lo;       // first window tile of the query tile
    int64_t n_band;     // number of window tiles
    int64_t n_stride;   // number of stride-only tiles (all left of t_lo)
};

__device__ TileGeom tile_geom(int64_t q, int64_t N, int64_t window, int64_t stride, int64_t bm,
                              int64_t bn) {
    TileGeom g;
    int64_t r0 = q * bm;
    int64_t r1 = (r0 + bm < N ? r0 + bm : N) - 1;
    int64_t lo = r0 - window + 1 > 0 ? r0 - window + 1 : 0;
    g.t_lo = lo / bn;
    g.n_band = r1 / bn - g.t_lo + 1;
    if (stride <= 0 || g.t_lo == 0)
        g.n_stride = 0;
    else if (stride <= bn)
        g.n_stride = g.t_lo;
    else
        g.n_stride = (g.t_lo * bn + stride - 1) / stride;
    return g;
}

// multiples of s (s > 0) in [a, b], a >= 0
__device__ int64_t multiples_in(int64_t a, int64_t b, int64_t s) {
    if (b < a)
        return 0;
    return b / s - (a + s - 1) / s + 1;
}

__global__ void mask_count_kernel(int32_t *row_ptr, int nq, int N, int window, int stride, int bm,
                                  int bn) {
    int q = blockIdx.x * blockDim.x + threadIdx.x;
    if (q == 0)
        row_ptr[0] = 0;
    if (q >= nq)
        return;
    TileGeom g = tile_geom(q, N, window, stride, bm, bn);
    row_ptr[q + 1] = static_cast<int32_t>(g.n_band + g.n_stride);
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

__global__ __launch_bounds__(64) void mask_fill_kernel(const int32_t *row_ptr, int32_t *kv_tile,
                                                       uint8_t *kind, int32_t *cells,
                                                       int32_t *stride_keys, int32_t *band_begin,
                                                       int N, int window, int stride, int bm,
                                                       int bn) {
    int64_t q = blockIdx.x;
    TileGeom g = tile_geom(q, N, window, stride, bm, bn);
    int64_t base = row_ptr[q];
    if (threadIdx.x == 0) {
        stride_keys[q] = stride > 0 ? static_cast<int32_t>((g.t_lo * bn + stride - 1) / stride) : 0;
        band_begin[q] = static_cast<int32_t>(base + g.n_stride);
    }
    int64_t i0 = q * bm, i1 = i0 + bm < N ? i0 + bm : N;
    int64_t count = g.n_band + g.n_stride;
    for (int64_t e = threadIdx.x; e < count; e += blockDim.x) {
        int64_t t;
        if (e < g.n_stride)
            t = stride <= bn ? e : (e * stride) / bn;
        else
            t = g.t_lo + (e - g.n_stride);
        int64_t j0 = t * bn, j1 = j0 + bn < N ? j0 + bn : N;
        int64_t c = 0;
        bool any_band = false;
        for (int64_t i = i0; i < i1; ++i) {
            int64_t lo = i - window + 1 > 0 ? i - window + 1 : 0;
            int64_t a = lo > j0 ? lo : j0;
            int64_t b = i < j1 - 1 ? i : j1 - 1;
            if (b >= a) {
                c += b - a + 1;
                any_band = true;
            }
            if (stride > 0) {
                int64_t sb = j1 - 1 < lo - 1 ? j1 - 1 : lo - 1;
                c += multiples_in(j0, sb, stride);
            }
        }
        uint8_t k = !any_band ? 2 : (c == (i1 - i0) * (j1 - j0) ? 0 : 1);
        kv_tile[base + e] = static_cast<int32_t>(t);
        kind[base + e] = k;
        cells[base + e] = static_cast<int32_t>(c);
    }
}

__global__ void mask_dense_kernel(uint8_t *out, int N, int window, int stride) {
    int64_t total = static_cast<int64_t>(N) * N;
    for (int64_t x = blockIdx.x * static_cast<int64_t>(blockDim.x) + threadIdx.x; x < total;
         x += static_cast<int64_t>(gridDim.x) * blockDim.x) {
        int64_t i = x / N, j = x % N;
        bool in_window = j <= i && i - j < window;
        bool on_stride = stride > 0 && j <= i && j % stride == 0;
        out[x] = (in_window || on_stride) ? 1 : 0;
    }
}

}  // namespace

hipError_t launch_block_mask_build(const swa_block_mask_t &m, hipStream_t stream) {
    int nq = m.num_q_tiles;
    hipLaunchKernelGGL(mask_count_kernel, dim3((nq + 255) / 256), dim3(256), 0, stream, m.row_ptr,
                       nq, m.N, m.window, m.stride, m.bm, m.bn);
    hipLaunchKernelGGL(mask_scan_kernel, dim3(1), dim3(1024), 0, stream, m.row_ptr, nq);
    hipLaunchKernelGGL(mask_fill_kernel, dim3(nq), dim3(64), 0, stream, m.row_ptr, m.kv_tile,
                       m.kind, m.cells, m.stride_keys, m.band_begin, m.N, m.window, m.stride, m.bm,
                       m.bn);
    return hipGetLastError();
}

hipError_t launch_mask_dense(int N, int window, int stride, uint8_t *out, hipStream_t stream) {
    int64_t total = static_cast<int64_t>(N) * N;
    int64_t blocks = (total + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(mask_dense_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                       out, N, window, stride);
    return hipGetLastError();
}

}  // namespace swa
