/*
 * swa.h -- C ABI of the MI355X (gfx950) masked causal attention library.
 *
 * The operation (Learn: Sparse & Sliding-Window Attention, §3 equation):
 *
 *     A = softmax(Q K^T * scale + log M) V,   log M_ij in {0, -inf}
 *
 * with the mask M_ij = 1 iff  0 <= j <= i < N  and at least one of
 *   (window)  (i - j) mod dilation == 0 and (i - j) / dilation < window:
 *             the `window` keys i, i - dilation, ..., i - (window-1)*dilation.
 *             dilation = 1 is swa_mask(n, window) of "Attention Variants
 *             Compared" (exactly `window` keys per row once i >= window-1;
 *             window >= N gives full causal); dilation > 1 is Longformer's
 *             dilated window (Learn: Sparse & Sliding-Window Attention, §3b).
 *   (stride)  stride > 0 and j mod stride == 0 -- strided_mask(n, window,
 *             stride) of "Attention Variants Compared", anchored at key 0.
 *   (global)  j < n_global or i < n_global -- Longformer's global tokens
 *             (same page, §3b), here the first n_global positions, kept
 *             causal.  Since j <= i, a global row's keys are all global
 *             columns: the global tokens act as key columns every later row
 *             attends.
 *
 * Conventions shared by every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller, 16-byte
 *     aligned, row-major and contiguous:
 *        Q, O        [B, Hq,  N, d]     (O: [B, Hq, N, dv] for diff_attn_fwd)
 *        K           [B, Hkv, N, d]
 *        V           [B, Hkv, N, dv]    (dv = d except in diff_attn_fwd)
 *     Query head h reads key/value head h / (Hq / Hkv) (grouped-query
 *     attention in contiguous groups).
 *   - The library never allocates, frees or synchronizes.  Every call that
 *     launches work is asynchronous on `stream` (0 = the null stream).
 *   - Every argument is checked on the host BEFORE any HIP call; a rejected
 *     call launches nothing and returns a negative swa_status_t.  Launch
 *     failures return SWA_ERR_HIP.
 *   - Each call launches its kernels as one-dimensional grids, and a dispatch
 *     holds at most 2^32 - 1 work-items: a call that would need more returns
 *     SWA_ERR_UNSUPPORTED.  Forward calls have one workgroup per (batch,
 *     query head, query tile) of 256 lanes (512 for diff_attn_fwd in bf16),
 *     except three bf16 shapes that run a persistent grid of at most one
 *     512-lane workgroup per compute unit: swa_attn_fwd with d = dv = 128,
 *     no stride, a window that may be dilated or have global tokens (not
 *     both) and a multiple of 4 query heads per key/value head;
 *     swa_attn_fwd with d = dv = 64, one query head per key/value head,
 *     B * Hq even, no dilation or global tokens and a stride of 0 or a
 *     power of two from 64 to 2^18; and diff_attn_fwd with d = 64,
 *     dv = 128 and a window only.  The decode calls' launches are sized by
 *     their own work split.
 *   - Results are deterministic: the same inputs give bit-identical outputs.
 *   - No global mutable state, except the static scratch array of
 *     swa_attn_decode_noalloc: calls on different streams may overlap as
 *     long as their output buffers do not (and, for swa_attn_decode_noalloc,
 *     as long as they run on different GPUs).
 */
#ifndef SWA_H
#define SWA_H

#include <stddef.h>
#include <stdint.h>

#if !defined(HIP_INCLUDE_HIP_HIP_RUNTIME_API_H)
typedef struct ihipStream_t *hipStream_t;
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SWA_OK = 0,
    SWA_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size, inconsistent mask */
    SWA_ERR_UNSUPPORTED = -2, /* valid request this library does not implement      */
    SWA_ERR_WORKSPACE = -3,   /* decode workspace missing or too small               */
    SWA_ERR_HIP = -4,         /* a HIP launch reported an error                       */
    SWA_ERR_SCRATCH = -5      /* swa_attn_decode_noalloc: the call needs more than    */
                              /* SWA_DECODE_SCRATCH_BYTES of scratch                  */
} swa_status_t;

/* Element type of Q, K, V and the output.  Entry points take it as an int
 * `dt` holding one of these values; any other value is SWA_ERR_INVALID_ARG
 * (an int, not the enum type, so that an out-of-range value is a defined
 * input the library rejects). */
typedef enum { SWA_F32 = 0, SWA_BF16 = 1 } swa_dtype_t;

/* The attention call a block mask is built for (their tile shapes differ);
 * taken as an int `op` holding one of these values, like `dt`. */
typedef enum { SWA_OP_ATTN = 0, SWA_OP_DIFF = 1 } swa_op_t;

/* Largest sequence length any entry point accepts (keeps every index and
 * cell count of one (batch, head) inside int32). */
#define SWA_MAX_N (1 << 22)

/*
 * Block mask: for each query tile of `bm` rows, the key tiles of `bn` keys
 * that hold at least one attended cell ("Attention Variants Compared":
 * create_block_mask builds the per-block keep/skip map once, blocks with no
 * attended cell are skipped; it is then handed to the attention call).
 * Stored as a CSR over query tiles; within a query tile the key tiles are
 * ascending.  The mask depends only on (N, window, stride, dilation,
 * n_global, bm, bn) and is shared by every batch and head.
 *
 * The "band" of query tile q is the key range max(0, r0 - (window-1) *
 * dilation) .. r1 (r0, r1 its first and last row); every key left of the
 * band that is a multiple of stride or a global column (a "prefix key") is
 * attended by every row of the tile.
 *
 *   row_ptr[num_q_tiles + 1]   list of query tile q is [row_ptr[q], row_ptr[q+1])
 *   kv_tile[nnz]               key tile index
 *   kind[nnz]                  0 FULL: every in-range cell attends
 *                              1 PARTIAL: some cells attend (mask applied per cell)
 *                              2 PREFIX_ONLY: the tile lies left of the band;
 *                                only its prefix keys attend, from every row
 *   cells[nnz]                 attended cells of the tile (rows, keys < N)
 *   prefix_keys[num_q_tiles]   prefix keys inside the PREFIX_ONLY tiles of q;
 *                              in order they are 0 .. g'-1 (g' = min(n_global,
 *                              prefix_keys[q])), then the multiples of stride
 *                              from g' on
 *   band_begin[num_q_tiles]    index of the first non-PREFIX_ONLY entry of q
 *                              (PREFIX_ONLY entries come first)
 *
 * The caller allocates the five device arrays with the sizes that
 * swa_block_mask_query returns and fills the scalar fields.
 */
typedef struct {
    int32_t N, window, stride, dilation, n_global, bm, bn;
    int32_t num_q_tiles, nnz;
    int32_t *row_ptr;
    int32_t *kv_tile;
    uint8_t *kind;
    int32_t *cells;
    int32_t *prefix_keys;
    int32_t *band_begin;
} swa_block_mask_t;

/* Tile shape (query rows bm, keys bn) the kernel of `op` walks for this
 * dtype and head sizes (swa_attn_fwd: SWA_OP_ATTN, diff_attn_fwd:
 * SWA_OP_DIFF); a block mask built with other sizes is rejected by that
 * call.  Host only, no HIP call.  d, dv in {32, 64, 128}. */
int swa_tile_config(int op, int dt, int d, int dv, int32_t *bm, int32_t *bn);

/* Number of query tiles and list entries of the block mask of
 * (N, window, stride, dilation, n_global, bm, bn): the sizes of the arrays
 * swa_block_mask_build fills (the per-query-tile key-tile lists of the
 * band, stride, dilation and global-token patterns; sparsity as which
 * (query, key) pairs are scored, Learn: Sparse & Sliding-Window Attention,
 * §3, tiled as in the "Flash style softmax" task of "Attention Variants
 * Compared").  Host only, no HIP call.
 * N in [1, SWA_MAX_N], window >= 1, stride >= 0 (0 = no stride pattern),
 * dilation in [1, bn] (so every tile of a band holds an attended cell),
 * n_global in [0, SWA_MAX_N], bm, bn in {16, 32, 64, 128, 256}. */
int swa_block_mask_query(int N, int window, int stride, int dilation, int n_global, int bm, int bn,
                         int32_t *num_q_tiles, int32_t *nnz);

/* Fill the device arrays of *mask on `stream` from its scalar fields, which
 * must equal what swa_block_mask_query reports.  Integer work only; the
 * result is bit-exact. */
int swa_block_mask_build(const swa_block_mask_t *mask, hipStream_t stream);

/* Debug export of the dense mask M of Learn: Sparse & Sliding-Window
 * Attention, §3 (the swa_mask / strided_mask matrices of "Attention Variants
 * Compared", OR'd with the dilation and global-token patterns):
 * out[i*N + j] = 1 if query i attends key j, else 0, for N <= 16384 (device
 * array of N*N bytes).  Not on the hot path; the tests compare it with the
 * oracle bit for bit. */
int swa_mask_dense(int N, int window, int stride, int dilation, int n_global, uint8_t *out,
                   hipStream_t stream);

/*
 * Masked attention forward (prefill) -- the §3 equation above over the block
 * mask, with an fp32 online softmax ("Attention Variants Compared": the
 * Flash-style tiled softmax) so the N x N score matrix never exists.
 *   q, k, v, out   layouts above, dtype dt, dv = d
 *   lse            nullable; fp32 [B, Hq, N] natural-log sum of
 *                  exp(score * scale) over the attended keys
 *   d in {32, 64, 128} for SWA_BF16 and SWA_F32
 *   mask           built for (N, window, stride, dilation, n_global) and the
 *                  tiles of swa_tile_config(SWA_OP_ATTN, dt, d, d)
 * Arithmetic: bf16 inputs, fp32 accumulation, output rounded to bf16
 * (SWA_BF16) or kept fp32 (SWA_F32).
 */
int swa_attn_fwd(const void *q, const void *k, const void *v, void *out, float *lse,
                 int dt, int B, int Hq, int Hkv, int N, int d, int window, int stride,
                 int dilation, int n_global, float scale, const swa_block_mask_t *mask,
                 hipStream_t stream);

/* Bytes of device workspace a decode call needs: op SWA_OP_ATTN for
 * swa_attn_decode and swa_attn_decode_sinks (dv = d), SWA_OP_DIFF for
 * diff_attn_decode; n_sink = 0 except for swa_attn_decode_sinks.  0 means
 * the call needs none (workspace may then be NULL); also 0 for invalid
 * sizes, which the call itself rejects. */
size_t swa_attn_decode_workspace_bytes(int op, int B, int Hq, int Hkv, int dv, int window,
                                       int n_sink);

/*
 * One decode step over a rolling KV window (Learn: Sparse & Sliding-Window
 * Attention, §4 and §6: keep only the last `window` tokens' keys and values
 * in a fixed-size rolling buffer).
 *   q          [B, Hq, d]            the current token's queries
 *   k_ring     [B, Hkv, window, d]   position p of a sequence lives in slot
 *   v_ring     [B, Hkv, window, d]   p mod window; the caller has already
 *                                    written the current token
 *   out        [B, Hq, d]
 *   seq_len    device int32 [B]: tokens so far, the current one included
 *              (the attended positions are max(0, L-window) .. L-1), or NULL
 *              for every sequence at length N.  A sequence with L <= 0
 *              attends nothing and gets zeros.
 *   workspace  device scratch of swa_attn_decode_workspace_bytes(SWA_OP_ATTN,
 *              B, Hq, Hkv, d, window, 0) bytes, owned by the caller; contents
 *              on entry do not matter.
 *   stride     must be 0: stride keys older than the window are not in the
 *              ring (SWA_ERR_UNSUPPORTED otherwise).
 * B * Hq and B * Hkv * window must fit int32 (SWA_ERR_UNSUPPORTED
 * otherwise).
 */
int swa_attn_decode(const void *q, const void *k_ring, const void *v_ring, void *out,
                    const int32_t *seq_len, void *workspace, size_t workspace_bytes,
                    int dt, int B, int Hq, int Hkv, int N, int d, int window, int stride,
                    float scale, hipStream_t stream);

/*
 * Decode step with attention sinks (Learn: Sparse & Sliding-Window Attention,
 * §4, StreamingLLM: the first few tokens stay in the cache next to the
 * rolling window).  As swa_attn_decode, plus
 *   k_sink, v_sink  [B, Hkv, n_sink, d]: positions 0 .. n_sink-1 in sink
 *                   slots (nullable when n_sink == 0)
 * The attended positions are {p < n_sink} united with the window
 * max(0, L-window) .. L-1; a position in both is attended once (from the
 * ring), and only positions < L are attended.  n_sink = 0 is swa_attn_decode.
 * workspace: swa_attn_decode_workspace_bytes(SWA_OP_ATTN, B, Hq, Hkv, d,
 * window, n_sink) bytes.
 */
int swa_attn_decode_sinks(const void *q, const void *k_sink, const void *v_sink, int n_sink,
                          const void *k_ring, const void *v_ring, void *out,
                          const int32_t *seq_len, void *workspace, size_t workspace_bytes,
                          int dt, int B, int Hq, int Hkv, int N, int d, int window,
                          float scale, hipStream_t stream);

/*
 * Differential-attention decode step over a rolling window ("Attention
 * Variants — Sliding Window, Sparse, Differential": two maps from separate
 * query/key projections, the second subtracted with weight lambda).  The
 * symptom/cause/fix table of "Attention Variants Compared" lists a
 * differential decode that loads the value cache twice as slower than the
 * baseline, so V is read once for both maps:
 *
 *   out = softmax(q1 K1^T * scale) V - lambda * softmax(q2 K2^T * scale) V
 *
 * over the window positions of swa_attn_decode.
 *   q1, q2          [B, Hq, d]            k1_ring, k2_ring  [B, Hkv, window, d]
 *   v_ring          [B, Hkv, window, dv]  out               [B, Hq, dv]
 * d, dv in {32, 64, 128}.
 * workspace: swa_attn_decode_workspace_bytes(SWA_OP_DIFF, B, Hq, Hkv, dv,
 * window, 0) bytes.
 */
int diff_attn_decode(const void *q1, const void *k1_ring, const void *q2, const void *k2_ring,
                     const void *v_ring, void *out, const int32_t *seq_len, void *workspace,
                     size_t workspace_bytes, int dt, int B, int Hq, int Hkv, int N, int d,
                     int dv, int window, float scale, float lambda, hipStream_t stream);

/*
 * Differential attention ("Attention Variants — Sliding Window, Sparse,
 * Differential": two attention maps from separate query/key projections,
 * one subtracted from the other; "Attention Variants Compared": the two maps
 * read the same value cache):
 *
 *   out = (softmax(Q1 K1^T * scale + log M) - lambda * softmax(Q2 K2^T * scale + log M)) V
 *
 *   q1, q2     [B, Hq, N, d]      k1, k2  [B, Hkv, N, d]
 *   v          [B, Hkv, N, dv]    out     [B, Hq, N, dv]
 *   d in {32, 64, 128}, dv in {32, 64, 128}; no normalisation follows the
 *   subtraction.  mask: built for (N, window, stride, dilation, n_global)
 *   and the tiles of swa_tile_config(SWA_OP_DIFF, dt, d, dv).
 */
int diff_attn_fwd(const void *q1, const void *k1, const void *q2, const void *k2,
                  const void *v, void *out, int dt, int B, int Hq, int Hkv, int N,
                  int d, int dv, int window, int stride, int dilation, int n_global, float scale,
                  float lambda, const swa_block_mask_t *mask, hipStream_t stream);

/*
 * swa_attn_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  It runs the kernels of swa_attn_decode
 * and gives them a file-scope device array of SWA_DECODE_SCRATCH_BYTES in
 * place of the caller's workspace; the library calls no allocating routine.
 *   Arguments: as swa_attn_decode minus workspace and workspace_bytes.
 *   A call whose swa_attn_decode_workspace_bytes(SWA_OP_ATTN, B, Hq, Hkv, d,
 *   window, 0) exceeds SWA_DECODE_SCRATCH_BYTES returns SWA_ERR_SCRATCH
 *   (checked on the host before any HIP call); other checks and errors as
 *   swa_attn_decode.
 *   Each GPU holds its own copy of the array from the first call on that GPU
 *   (its address is looked up once per device, with that device current)
 *   until the process ends.  Every call on one GPU uses that GPU's array:
 *   calls that overlap in time on one GPU (other streams, other host threads)
 *   race on it and must be serialized by the caller, e.g. on one stream.  The
 *   kernels write every partial result before reading it, so what an earlier
 *   call left in the array does not matter.
 */
#define SWA_DECODE_SCRATCH_BYTES ((size_t)4 << 20)
int swa_attn_decode_noalloc(const void *q, const void *k_ring, const void *v_ring, void *out,
                            const int32_t *seq_len, int dt, int B, int Hq, int Hkv,
                            int N, int d, int window, int stride, float scale,
                            hipStream_t stream);

/* Static description of a status code. */
const char *swa_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* SWA_H */
