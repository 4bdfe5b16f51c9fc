// Internal declarations shared by the host API (lce_api.cpp) and the device
// kernels (lce_kernels.hip). Not part of the public C ABI.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "lce.h"

namespace lce {

// lce_forward_traced with the (max, sum-exp) partials held for `group` rows
// at a time (a multiple of 256; 0 = all rows at once), and the workspace it
// needs (0 when *p is invalid).
size_t forward_workspace_bytes(const lce_problem* p, int64_t group);
int forward_grouped(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                    const int64_t* labels, float* loss, float* lse, float* chunk_loss, int64_t* n_valid,
                    int32_t* status, void* workspace, size_t workspace_bytes, int64_t group, hipStream_t stream,
                    lce_trace* trace);

struct Shapes {
  int64_t N, Np;     // rows, rows rounded up to a multiple of 256
  int64_t H;         // hidden
  int64_t V, Vp;     // vocabulary, rounded up to a multiple of 256
  int64_t ldh, ldw;  // row strides (elements)
  int64_t chunk_rows;
};

hipError_t launch_zero(void* p, int64_t bytes, hipStream_t st);
// block_cnt (nullable): valid rows of each 256-row block (for the partition).
hipError_t launch_prepare_labels(const int64_t* labels, int64_t N, int64_t Np, int64_t V, int64_t ignore,
                                 int32_t* label32, unsigned long long* n_valid, int32_t* status,
                                 int32_t* block_cnt, hipStream_t st);
// Valid rows first: perm[slot] = original row, labp[slot] = its label, valid
// rows (label32 >= 0) in order in slots [0, n_valid), the others after them
// in order (rows N..Np-1 last). block_off: Np/256 ints of scratch.
hipError_t launch_partition_rows(const int32_t* label32, const int32_t* block_cnt, int32_t* block_off,
                                 const unsigned long long* n_valid, int64_t Np, int32_t* perm, int32_t* labp,
                                 hipStream_t st);
// out [N][H] (row stride H) = in[perm[slot]] (row stride ld_in), H % 8 == 0.
hipError_t launch_gather_rows(const void* in, int64_t ld_in, const int32_t* perm, int64_t N, int64_t H, void* out,
                              hipStream_t st);
// Forward tiles for rows [g0, g0 + rows) (rows a multiple of 256): quarter-tile
// (max, sumexp) partials into part_m/part_s [4 * Vp/256][rows] and, when
// p_out is non-null, bf16 softmax numerators into p_out, stored as K-slabs
// [Vp/64][rows][64] (element (i, j) at ((j/64) * rows + i) * 64 + j % 64).
// tile_ctr: 8 ints of scratch (the per-XCD tile counters, zeroed here).
// With p_out and rref non-null the stored values are exp(z - rref[i]) for
// rows with a finite rref (capped at e^60; a larger gap sets *ovf = 1) and
// exp(z - max_quarter) for NaN entries. only_if (nullable): run only if
// *only_if != 0. Partials are base 2: (max t, sum 2^(t - max t)), t =
// z log2(e). label32 [Np] (-1: no label): for each row with a label the
// tile holding that column writes its t to zy2[row] (zy2 [Np], global rows).
// row_limit (nullable): only rows below *row_limit (global index) get tiles.
hipError_t launch_fwd_tiles(const Shapes& s, const void* hidden, const void* weight, const void* bias, int64_t g0,
                            int64_t rows, float* part_m, float* part_s, void* p_out, int* tile_ctr,
                            const float* rref, int* ovf, const int* only_if, const int32_t* label32, float* zy2,
                            const unsigned long long* row_limit, hipStream_t st);
// zlab[i] = h_i . W_{y_i} + b_{y_i} for valid rows (FP32 dot product: the
// backward's per-row references, needed before the row's tiles run).
hipError_t launch_label_logit(const Shapes& s, const void* hidden, const void* weight, const void* bias,
                              const int32_t* label32, float* zlab, hipStream_t st);
// lse and l_i of rows [g0, g0 + rows) from the base-2 partials and the label
// values zy2 written by the forward tiles; rows at or past *row_limit
// (nullable) are skipped. perm (nullable): row i is the caller's row
// perm[i] for lse_out, rowloss_out and its chunk.
hipError_t launch_finalize_rows(const Shapes& s, const float* part_m, const float* part_s, int64_t g0,
                                int64_t rows, const float* zy2, const int32_t* label32, const int32_t* status,
                                int reduction, float* lse_ws, float* lse_out, float* rowloss_out,
                                double* chunk_acc, const unsigned long long* row_limit, const int32_t* perm,
                                hipStream_t st);
hipError_t launch_finalize_loss(const double* chunk_acc, int64_t T, const unsigned long long* n_valid,
                                const int32_t* status, int reduction, float* loss, float* chunk_out,
                                hipStream_t st);
// out = rows [r0, r0 + R_valid) of in [.][ld_in] (first C columns), transposed
// and stored as K-slabs [R_pad/64][C][64]: element (c, r) at
// ((r/64) * C + c) * 64 + r % 64; rows R_valid..R_pad-1 are zero. With rowc
// non-null, row r is scaled by rowc[r] (rounded to bf16).
hipError_t launch_transpose(const void* in, int64_t ld_in, int64_t r0, int64_t R_valid, int64_t C, void* out,
                            int64_t R_pad, const float* rowc, hipStream_t st);
// Row references of one group for the stored softmax numerators: rref[i] =
// src[g0 + i] for valid rows, NaN otherwise; only_if as above.
hipError_t launch_prep_ref(const int32_t* label32, const float* src, int64_t g0, int64_t G, float* rref,
                           const int* only_if, hipStream_t st);
// Row scales rowc[i] = s row_scale_i valid_i exp(rref_i - lse_i) and the label
// entry of each valid row of dlog (K-slabs [Vp/64][G][64]) set to
// exp(z_y - rref_i) - exp(lse_i - rref_i), z_y = zy2 ln 2. Runs when
// (*ovf != 0) == retry. gb_f32 (nullable) receives rowc[i] times the bf16
// rounding of that entry.
// perm (nullable): row_scale is indexed by the caller's row perm[row].
hipError_t launch_rowscale(const int32_t* label32, const float* zy2, const float* lse_ws, const float* rref,
                           const float* row_scale, const unsigned long long* n_valid, float grad_scale, int is_mean,
                           int64_t g0, int64_t G, void* dlog, float* rowc, const int* ovf, int retry,
                           float* gb_f32, const int32_t* perm, hipStream_t st);
// gb_f32[v] += sum_i rowc[i] dlog[i][v] over the group's G rows (used when
// grad_weight is not computed or cannot add these sums itself).
hipError_t launch_bias_sums(const Shapes& s, const void* dlog, const float* rowc, int64_t G, float* gb_f32,
                            hipStream_t st);
// data[k] *= *scale (bf16 or f32 elements).
hipError_t launch_scale(void* data, bool f32, int64_t n, const float* scale, hipStream_t st);
// grad_hidden rows [g0, g0 + G): row i = rowc[i] (dlog wT^T)_i over K = Vp
// (dlog: K-slabs [Vp/64][G][64], wT: [Vp/64][H][64]).
// Row tiles at or past *row_limit (nullable) only write zero rows. perm
// (nullable): row i goes to the caller's row perm[i].
// part: part_items * 256 * 256 floats of scratch; when the group's real tiles
// do not fill whole rounds of the GPU, the tiles left over are split along K
// into pieces written there and summed by a second kernel (k_gh_reduce).
hipError_t launch_grad_hidden(const Shapes& s, const void* dlog, const void* wT, int64_t g0, int64_t G,
                              const float* rowc, void* grad_hidden, const unsigned long long* row_limit,
                              const int32_t* perm, float* part, int64_t part_items, hipStream_t st);
// gw (+)= sum over the group's rows i < rows_valid of G[i][v] h[g0 + i][:]
// (dlog: K-slabs [Vp/64][G][64] holding G; hT: the group's rows of h as
// K-slabs [G/64][H][64], zero past N). part: part_items * 256 * 256 floats
// of scratch for split tiles (no more pieces are made). first: store instead
// of add. gw_bf16 (nullable): also write each final sum rounded to bf16 (the
// last row group); keep32 = 0: do not write the FP32 sums back. gb_f32
// (nullable): also add the group's grad_bias column sums, sum_i rowc[i]
// dlog[i][v] (FP32 atomics; rowc [G], the group's row scales).
// row_limit (nullable): K stays below row *row_limit - g0 of the group.
hipError_t launch_grad_weight(const Shapes& s, const void* dlog, int64_t G, const void* hT, int64_t rows_valid,
                              float* part, int64_t part_items, int first, float* gw_f32, void* gw_bf16, int keep32,
                              const float* rowc, float* gb_f32, const unsigned long long* row_limit, int64_t g0,
                              hipStream_t st);
// grad_weight's tiles: the first n_full run whole (a multiple of the CU
// count), the rest are split `split` ways along K (split = 1: none) so that
// they fill one round; at most min(max_items, kMaxGwItems) split pieces.
constexpr int kMaxGwSplit = 8;
constexpr int kMaxGwItems = 256;
void grad_weight_split(int n_tiles, int nk, int cus, int max_items, int* n_full, int* split);
// Rows of each 64-row stage that one wave of a grad_weight tile adds to the
// grad_bias sums for hidden size H: the least power of two r with
// r ceil(H / 256) >= 16 (four waves per column half, every tile of the row).
int grad_weight_bias_rows(int64_t H);
int device_cus();
hipError_t launch_cast(const float* in, void* out, int64_t n, hipStream_t st);

}  // namespace lce
