// Host side of the C ABI declared in include/lce.h: argument validation,
// workspace carve-up and the launch sequence on the caller's stream. The
// library allocates nothing and keeps no state.
#include "lce.h"

#include <hip/hip_runtime_api.h>
#include <stdint.h>
#include <string.h>

#include "lce_internal.h"

namespace {

using lce::Shapes;

constexpr int64_t kTile = 256;
constexpr int64_t kDefaultRowsInFlight = 16384;
constexpr int64_t kMaxRowsInFlight = int64_t(1) << 20;
constexpr int64_t kMaxStride = int64_t(1) << 22;
int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  // forward
  size_t label32 = 0, n_valid = 0, status = 0, zy2 = 0, lse = 0, part_m = 0, part_s = 0, chunk_acc = 0,
         tile_ctr = 0;
  // backward
  size_t zlab = 0, wT = 0, hT = 0, gw_part = 0, dlog = 0, gw_f32 = 0, gb_f32 = 0, rref = 0, rowc = 0, ovf = 0;
  size_t block_cnt = 0, block_off = 0, perm = 0, labp = 0, hperm = 0;   // valid rows first
  size_t total = 0;
};

int validate_problem(const lce_problem* p) {
  if (p == nullptr) return LCE_ERR_INVALID_ARG;
  if (p->n_rows < 0 || p->hidden <= 0 || p->vocab <= 0) return LCE_ERR_INVALID_ARG;
  if (p->ld_hidden < p->hidden || p->ld_weight < p->hidden) return LCE_ERR_INVALID_ARG;
  if (p->chunk_rows <= 0) return LCE_ERR_INVALID_ARG;
  if (p->rows_in_flight < 0) return LCE_ERR_INVALID_ARG;
  if (p->reduction < LCE_REDUCTION_NONE || p->reduction > LCE_REDUCTION_MEAN) return LCE_ERR_INVALID_ARG;
  if (p->dtype != LCE_DTYPE_BF16) return LCE_ERR_UNSUPPORTED;
  if (p->hidden % 64 != 0) return LCE_ERR_UNSUPPORTED;
  if (p->ld_hidden % 8 != 0 || p->ld_weight % 8 != 0) return LCE_ERR_UNSUPPORTED;
  // 256 rows of any operand must span < 4 GiB (32-bit load offsets)
  if (p->ld_hidden > kMaxStride || p->ld_weight > kMaxStride || p->vocab > kMaxStride) return LCE_ERR_UNSUPPORTED;
  // labels and tile indices are 32-bit on the device
  if (p->vocab > (int64_t)INT32_MAX - 1024 || p->n_rows > (int64_t)INT32_MAX - 1024) return LCE_ERR_UNSUPPORTED;
  const int64_t tiles = round_up(p->n_rows, kTile) / kTile * (round_up(p->vocab, kTile) / kTile);
  if (tiles > (int64_t)INT32_MAX) return LCE_ERR_UNSUPPORTED;
  return LCE_OK;
}

Shapes shapes_of(const lce_problem* p) {
  Shapes s;
  s.N = p->n_rows;
  s.Np = round_up(p->n_rows, kTile);
  s.H = p->hidden;
  s.V = p->vocab;
  s.Vp = round_up(p->vocab, kTile);
  s.ldh = p->ld_hidden;
  s.ldw = p->ld_weight;
  s.chunk_rows = p->chunk_rows;
  return s;
}

// Rows of one backward row group. A caller's rows_in_flight is taken as
// given (clamped, rounded up to whole tiles). The default is 16384 rows but
// at most a quarter of the rows (whole tiles, at least one): the group's bf16
// softmax numerators then take at most half the bytes of bf16 [N, V] logits,
// at any N (one tile of 256 rows when N <= 256, the size of one of the pages'
// 256-row chunks).
int64_t group_rows(const lce_problem* p, const Shapes& s) {
  int64_t g;
  if (p->rows_in_flight > 0) {
    g = round_up(p->rows_in_flight < kMaxRowsInFlight ? p->rows_in_flight : kMaxRowsInFlight, kTile);
  } else {
    const int64_t quarter = s.Np / 4 / kTile * kTile;
    g = quarter < kTile ? kTile : quarter;
    if (g > kDefaultRowsInFlight) g = kDefaultRowsInFlight;
  }
  return g < s.Np ? g : s.Np;
}

// FP32 partial tiles for grad_weight's split last round: each split item is
// one 256 x 256 tile; a tile is split at most min(kMaxGwSplit, G / 256) ways
// (at least 4 K stages of 64 rows per piece), so nothing is reserved when no
// split can happen.
int64_t gw_part_items(const Shapes& s, int64_t G) {
  int64_t split_max = G / kTile;
  if (split_max > lce::kMaxGwSplit) split_max = lce::kMaxGwSplit;
  if (split_max < 2) return 0;
  const int64_t n_tiles = (s.Vp / kTile) * ((s.H + kTile - 1) / kTile);
  const int64_t items = n_tiles * split_max;
  return items < lce::kMaxGwItems ? items : lce::kMaxGwItems;
}

int64_t n_chunks(const lce_problem* p) { return (p->n_rows + p->chunk_rows - 1) / p->chunk_rows; }

// fwd_group (forward only): rows whose (max, sum-exp) partials are held at
// once; 0 = all rows (one pass over every row).
Layout make_layout(const lce_problem* p, int kind, int64_t fwd_group = 0) {
  const Shapes s = shapes_of(p);
  Layout L;
  size_t off = 0;
  // Regions of 1 MiB or more start on 2 MiB boundaries (relative to the
  // workspace start): the operand streams of the product kernels then keep
  // the same placement across DRAM pages whatever precedes them.
  auto take = [&](size_t bytes) {
    if (bytes >= (size_t(1) << 20)) off = (off + (size_t(2) << 20) - 1) & ~((size_t(2) << 20) - 1);
    const size_t at = off;
    off = align256(off + bytes);
    return at;
  };
  const int64_t n_vt = s.Vp / kTile;
  L.label32 = take((size_t)s.Np * 4);
  L.n_valid = take(8);
  L.status = take(4);
  L.zy2 = take((size_t)s.Np * 4);    // label logits from the forward tiles (base 2)
  L.lse = take((size_t)s.Np * 4);
  // (max, sumexp) partials per 64-column quarter tile: for every row in the
  // forward, for one row group at a time in the backward.
  const bool bwd = kind == LCE_WS_BACKWARD || kind == LCE_WS_BACKWARD_EXTERNAL_F32;
  const int64_t part_rows = bwd ? group_rows(p, s) : (fwd_group > 0 && fwd_group < s.Np ? fwd_group : s.Np);
  L.part_m = take((size_t)4 * n_vt * part_rows * 4);
  L.part_s = take((size_t)4 * n_vt * part_rows * 4);
  L.chunk_acc = take((size_t)n_chunks(p) * 8);
  L.tile_ctr = take(8 * sizeof(int));   // per-XCD tile counters of the forward tiles
  if (bwd) {
    const int64_t G = group_rows(p, s);
    L.zlab = take((size_t)s.Np * 4);   // label logits by a gather: the row references
    // rows in the valid-first order: per-block counts and offsets, the
    // permutation, its labels and the hidden rows gathered in that order
    L.block_cnt = take((size_t)(s.Np / kTile) * 4);
    L.block_off = take((size_t)(s.Np / kTile) * 4);
    L.perm = take((size_t)s.Np * 4);
    L.labp = take((size_t)s.Np * 4);
    L.hperm = take((size_t)s.Np * s.H * 2);
    // W^T, the group's h^T and its p~ / G, all stored as K-slabs
    // [K/64][rows][64]
    L.wT = take((size_t)s.H * s.Vp * 2);
    L.hT = take((size_t)s.H * G * 2);
    L.gw_part = take((size_t)gw_part_items(s, G) * 256 * 256 * 4);   // split grad_weight tiles
    L.dlog = take((size_t)G * s.Vp * 2);
    L.gb_f32 = take((size_t)s.Vp * 4);
    L.rref = take((size_t)G * 4);   // the group's row references of the stored softmax numerators
    L.rowc = take((size_t)G * 4);   // the group's dlogits row scales
    L.ovf = take(4);                // set by the forward tiles when a row needs the retry
    if (kind == LCE_WS_BACKWARD) L.gw_f32 = take((size_t)s.V * s.H * 4);
  }
  L.total = off;
  return L;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

#define LCE_TRY(expr)                       \
  do {                                      \
    if ((expr) != hipSuccess) return LCE_ERR_HIP; \
  } while (0)

// Optional per-launch event recording (lce_trace in include/lce.h).
struct Tracer {
  lce_trace* t = nullptr;
  hipStream_t st = nullptr;
  bool pending = false;
  void before(int kind, int64_t m, int64_t n, int64_t k) {
    if (t == nullptr || t->count >= t->capacity) return;
    if (hipEventRecord(t->events[2 * t->count], st) != hipSuccess) return;
    t->kinds[t->count] = kind;
    if (t->dims) {
      t->dims[3 * t->count] = m;
      t->dims[3 * t->count + 1] = n;
      t->dims[3 * t->count + 2] = k;
    }
    pending = true;
  }
  void after() {
    if (!pending) return;
    pending = false;
    if (hipEventRecord(t->events[2 * t->count + 1], st) == hipSuccess) t->count++;
  }
};

#define LCE_LAUNCH(tr, kind, m, n, k, call) \
  do {                                      \
    (tr).before((kind), (m), (n), (k));     \
    const hipError_t e_ = (call);           \
    (tr).after();                           \
    if (e_ != hipSuccess) return LCE_ERR_HIP; \
  } while (0)

struct Common {
  const lce_problem* p;
  Shapes s;
  Layout L;
  char* ws;
  int32_t* label32;
  unsigned long long* n_valid;
  int32_t* status;
  float* lse_ws;
  float* part_m;
  float* part_s;
  float* zlab;
  float* zy2;
  double* chunk_acc;
  int* tile_ctr;
  // valid-first row order (backward calls): row i of the work is the
  // caller's row perm[i]; the forward covers rows below *fwd_limit and the
  // backward rows below *bwd_limit (null: every row)
  const int32_t* perm = nullptr;
  const unsigned long long* fwd_limit = nullptr;
  const unsigned long long* bwd_limit = nullptr;

  int64_t T;
};

int check_common(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                 const int64_t* labels, const float* loss, void* workspace, size_t workspace_bytes, int kind,
                 Common& c, int64_t fwd_group = 0) {
  int st = validate_problem(p);
  if (st != LCE_OK) return st;
  if (loss == nullptr) return LCE_ERR_INVALID_ARG;
  if (p->n_rows > 0 && (hidden == nullptr || labels == nullptr)) return LCE_ERR_INVALID_ARG;
  if (weight == nullptr) return LCE_ERR_INVALID_ARG;
  if (!aligned(hidden, 16) || !aligned(weight, 16) || !aligned(bias, 2) || !aligned(labels, 8))
    return LCE_ERR_UNSUPPORTED;
  c.p = p;
  c.s = shapes_of(p);
  c.L = make_layout(p, kind, fwd_group);
  if (c.L.total > 0 && (workspace == nullptr || workspace_bytes < c.L.total)) return LCE_ERR_WORKSPACE;
  if (!aligned(workspace, 16)) return LCE_ERR_WORKSPACE;
  c.ws = (char*)workspace;
  c.T = n_chunks(p);
  return LCE_OK;
}

// Zeroes the counters and validates the labels (label32, n_valid, status):
// every later step, including the MEAN scale of the first row group's
// gradients, sees the final n_valid.
int run_prepare(Common& c, const int64_t* labels, int64_t* n_valid_out, int32_t* status_out, hipStream_t st,
                Tracer& tr, bool block_counts = false) {
  const Shapes& s = c.s;
  char* ws = c.ws;
  c.label32 = (int32_t*)(ws + c.L.label32);
  c.n_valid = n_valid_out ? (unsigned long long*)n_valid_out : (unsigned long long*)(ws + c.L.n_valid);
  c.status = status_out ? status_out : (int32_t*)(ws + c.L.status);
  c.lse_ws = (float*)(ws + c.L.lse);
  c.chunk_acc = (double*)(ws + c.L.chunk_acc);
  c.tile_ctr = (int*)(ws + c.L.tile_ctr);
  c.part_m = (float*)(ws + c.L.part_m);
  c.part_s = (float*)(ws + c.L.part_s);
  c.zlab = (float*)(ws + c.L.zlab);
  c.zy2 = (float*)(ws + c.L.zy2);
  LCE_LAUNCH(tr, LCE_K_ZERO, 0, 0, 0, lce::launch_zero(c.n_valid, 8, st));
  LCE_LAUNCH(tr, LCE_K_ZERO, 0, 0, 0, lce::launch_zero(c.status, 4, st));
  LCE_LAUNCH(tr, LCE_K_ZERO, 0, 0, 0, lce::launch_zero(c.chunk_acc, c.T * 8, st));
  if (s.N == 0) return LCE_OK;
  LCE_LAUNCH(tr, LCE_K_PREPARE_LABELS, 0, 0, 0,
             lce::launch_prepare_labels(labels, s.N, s.Np, s.V, c.p->ignore_index, c.label32, c.n_valid,
                                        c.status, block_counts ? (int32_t*)(ws + c.L.block_cnt) : nullptr, st));
  return LCE_OK;
}

// Puts the rows in the valid-first order (labels and gathered hidden rows)
// and makes every later step work on it: returns the gathered hidden rows.
int run_valid_first(Common& c, const void* hidden, bool lse_for_all_rows, hipStream_t st, Tracer& tr,
                    const void** hidden_out) {
  char* ws = c.ws;
  int32_t* perm = (int32_t*)(ws + c.L.perm);
  int32_t* labp = (int32_t*)(ws + c.L.labp);
  void* hperm = ws + c.L.hperm;
  LCE_LAUNCH(tr, LCE_K_PARTITION, 0, 0, 0,
             lce::launch_partition_rows(c.label32, (const int32_t*)(ws + c.L.block_cnt), (int32_t*)(ws + c.L.block_off),
                                        c.n_valid, c.s.Np, perm, labp, st));
  LCE_LAUNCH(tr, LCE_K_GATHER_ROWS, c.s.N, c.s.H, 0,
             lce::launch_gather_rows(hidden, c.s.ldh, perm, c.s.N, c.s.H, hperm, st));
  c.label32 = labp;
  c.perm = perm;
  c.s.ldh = c.s.H;
  c.bwd_limit = c.n_valid;
  c.fwd_limit = lse_for_all_rows ? nullptr : c.n_valid;
  *hidden_out = hperm;
  return LCE_OK;
}

// Label logits of every valid row by a gather: the backward's per-row
// references (the loss takes its label logits from the forward tiles).
int run_label_logits(Common& c, const void* hidden, const void* weight, const void* bias, hipStream_t st,
                     Tracer& tr) {
  LCE_LAUNCH(tr, LCE_K_LABEL_LOGIT, 0, 0, 0,
             lce::launch_label_logit(c.s, hidden, weight, bias, c.label32, c.zlab, st));
  return LCE_OK;
}

// Logits tiles with the online log-sum-exp epilogue for rows [g0, g0+rows),
// then per-row lse / NLL / chunk sums. With p_out the tiles also leave the
// softmax numerators exp(z - rref_i) behind for the gradient of the same rows.
int run_rows(Common& c, const void* hidden, const void* weight, const void* bias, int64_t g0, int64_t rows,
             void* p_out, float* loss, float* lse_out, hipStream_t st, Tracer& tr, const float* rref = nullptr,
             int* ovf = nullptr) {
  const Shapes& s = c.s;
  const int64_t rows_valid = (s.N - g0) < rows ? (s.N - g0) : rows;
  LCE_LAUNCH(tr, LCE_K_FWD_LSE, rows_valid, s.V, s.H,
             lce::launch_fwd_tiles(s, hidden, weight, bias, g0, rows, c.part_m, c.part_s, p_out, c.tile_ctr, rref,
                                   ovf, nullptr, c.label32, c.zy2, c.fwd_limit, st));
  LCE_LAUNCH(tr, LCE_K_FINALIZE_ROWS, 0, 0, 0,
             lce::launch_finalize_rows(s, c.part_m, c.part_s, g0, rows, c.zy2, c.label32, c.status,
                                       c.p->reduction, c.lse_ws, lse_out,
                                       c.p->reduction == LCE_REDUCTION_NONE ? loss : nullptr, c.chunk_acc,
                                       c.fwd_limit, c.perm, st));
  return LCE_OK;
}

}  // namespace

extern "C" {

int lce_abi_version(void) { return 105; }

const char* lce_status_string(int status) {
  switch (status) {
    case LCE_OK: return "ok";
    case LCE_ERR_INVALID_ARG: return "invalid argument";
    case LCE_ERR_UNSUPPORTED: return "unsupported configuration";
    case LCE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case LCE_ERR_HIP: return "HIP launch failed";
    case LCE_ERR_LABEL_RANGE: return "label outside [0, vocab) that is not ignore_index";
    case LCE_ERR_TOO_LARGE: return "problem needs more than the allocation-free entry point's scratch";
    default: return "unknown status";
  }
}

size_t lce_workspace_bytes(const lce_problem* p, int kind) {
  if (validate_problem(p) != LCE_OK) return 0;
  if (kind < LCE_WS_FORWARD || kind > LCE_WS_BACKWARD_EXTERNAL_F32) return 0;
  return make_layout(p, kind).total;
}

int lce_forward_traced(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                       const int64_t* labels, float* loss, float* lse, float* chunk_loss, int64_t* n_valid,
                       int32_t* status, void* workspace, size_t workspace_bytes, hipStream_t stream,
                       lce_trace* trace) {
  return lce::forward_grouped(p, hidden, weight, bias, labels, loss, lse, chunk_loss, n_valid, status, workspace,
                              workspace_bytes, 0, stream, trace);
}

}  // extern "C"

namespace lce {

size_t forward_workspace_bytes(const lce_problem* p, int64_t group) {
  if (validate_problem(p) != LCE_OK) return 0;
  return make_layout(p, LCE_WS_FORWARD, group).total;
}

int forward_grouped(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                    const int64_t* labels, float* loss, float* lse, float* chunk_loss, int64_t* n_valid,
                    int32_t* status, void* workspace, size_t workspace_bytes, int64_t group, hipStream_t stream,
                    lce_trace* trace) {
  Common c;
  int st = check_common(p, hidden, weight, bias, labels, loss, workspace, workspace_bytes, LCE_WS_FORWARD, c,
                        group);
  if (st != LCE_OK) return st;
  Tracer tr;
  tr.t = trace;
  tr.st = stream;
  if (trace) trace->count = 0;
  st = run_prepare(c, labels, n_valid, status, stream, tr);
  if (st != LCE_OK) return st;
  const int64_t step = group > 0 && group < c.s.Np ? group : c.s.Np;
  for (int64_t g0 = 0; g0 < c.s.N; g0 += step) {
    st = run_rows(c, hidden, weight, bias, g0, (c.s.Np - g0) < step ? (c.s.Np - g0) : step, nullptr, loss, lse,
                  stream, tr);
    if (st != LCE_OK) return st;
  }
  LCE_LAUNCH(tr, LCE_K_FINALIZE_LOSS, 0, 0, 0,
             lce::launch_finalize_loss(c.chunk_acc, c.T, c.n_valid, c.status, p->reduction, loss, chunk_loss,
                                       stream));
  return LCE_OK;
}

}  // namespace lce

extern "C" {

int lce_forward(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                const int64_t* labels, float* loss, float* lse, float* chunk_loss, int64_t* n_valid,
                int32_t* status, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return lce_forward_traced(p, hidden, weight, bias, labels, loss, lse, chunk_loss, n_valid, status, workspace,
                            workspace_bytes, stream, nullptr);
}

int lce_forward_backward_ex(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                            const int64_t* labels, float grad_scale, float* loss, float* lse, float* chunk_loss,
                            int64_t* n_valid, void* grad_hidden, void* grad_weight, void* grad_bias,
                            float* grad_weight_f32, float* grad_bias_f32, int32_t* status, void* workspace,
                            size_t workspace_bytes, hipStream_t stream, const lce_backward_options* options,
                            lce_trace* trace) {
  int st = validate_problem(p);
  if (st != LCE_OK) return st;
  const float* row_scale = options ? options->row_scale : nullptr;
  const bool accumulate = options && options->accumulate != 0;
  if (options && options->reserved != 0) return LCE_ERR_INVALID_ARG;
  if (p->reduction == LCE_REDUCTION_NONE && row_scale == nullptr) return LCE_ERR_UNSUPPORTED;
  if (row_scale != nullptr && !aligned(row_scale, 4)) return LCE_ERR_UNSUPPORTED;
  if ((grad_bias != nullptr || grad_bias_f32 != nullptr) && bias == nullptr) return LCE_ERR_INVALID_ARG;
  if (!aligned(grad_hidden, 2) || !aligned(grad_weight, 2) || !aligned(grad_bias, 2) ||
      !aligned(grad_weight_f32, 4) || !aligned(grad_bias_f32, 4))
    return LCE_ERR_UNSUPPORTED;
  const bool need_gh = grad_hidden != nullptr && p->n_rows > 0;
  const bool need_gw = grad_weight != nullptr || grad_weight_f32 != nullptr;
  const bool need_gb = grad_bias != nullptr || grad_bias_f32 != nullptr;
  // accumulating needs the caller's FP32 totals for every requested weight / bias gradient
  if (accumulate && ((need_gw && grad_weight_f32 == nullptr) || (need_gb && grad_bias_f32 == nullptr)))
    return LCE_ERR_INVALID_ARG;
  const int kind = (need_gw && grad_weight_f32 == nullptr) ? LCE_WS_BACKWARD : LCE_WS_BACKWARD_EXTERNAL_F32;
  Common c;
  st = check_common(p, hidden, weight, bias, labels, loss, workspace, workspace_bytes, kind, c);
  if (st != LCE_OK) return st;
  Tracer tr;
  tr.t = trace;
  tr.st = stream;
  if (trace) trace->count = 0;
  const bool any_grad = need_gh || need_gw || need_gb;
  const bool gb_in_gw = need_gb && need_gw;   // grad_weight adds the grad_bias sums when it runs
  st = run_prepare(c, labels, n_valid, status, stream, tr, any_grad);
  if (st != LCE_OK) return st;
  // the gradients only need the rows with a label: valid rows first, and
  // the backward stops at the device-side valid count (the forward too,
  // unless every row's lse or loss is an output)
  const void* hid = hidden;
  if (any_grad && c.s.N > 0) {
    st = run_valid_first(c, hidden, lse != nullptr || p->reduction == LCE_REDUCTION_NONE, stream, tr, &hid);
    if (st != LCE_OK) return st;
  }

  const Shapes& s = c.s;
  char* ws = c.ws;
  float* gw = grad_weight_f32 ? grad_weight_f32 : (float*)(ws + c.L.gw_f32);
  float* gb = grad_bias_f32 ? grad_bias_f32 : (float*)(ws + c.L.gb_f32);
  if (need_gb && !accumulate) LCE_LAUNCH(tr, LCE_K_ZERO, 0, 0, 0, lce::launch_zero(gb, s.V * 4, stream));
  // the last row group's grad_weight writes the bf16 result itself
  bool gw_cast_done = false;
  if (s.N == 0) {
    if (need_gw && !accumulate) LCE_LAUNCH(tr, LCE_K_ZERO, 0, 0, 0, lce::launch_zero(gw, s.V * s.H * 4, stream));
  } else {
    // Row groups: the logits of a group are computed once. The tiles leave
    // exp(z - r_i) in dlog, r_i the row's label logit; once the group's lse
    // is known, k_rowscale patches the label entries and forms the row
    // scales c_i with G = diag(c) p~'. If a row's maximum is too far above
    // its label logit (overflow flag), the flag-gated retry launches
    // recompute the group's p~ against r_i = lse_i; they do nothing
    // otherwise.
    const int64_t G = group_rows(p, s);
    void* wT = ws + c.L.wT;
    void* hT = ws + c.L.hT;
    float* gw_part = (float*)(ws + c.L.gw_part);
    void* dlog = ws + c.L.dlog;
    float* rref = (float*)(ws + c.L.rref);
    float* rowc = (float*)(ws + c.L.rowc);
    int* ovf = (int*)(ws + c.L.ovf);
    const int is_mean = p->reduction == LCE_REDUCTION_MEAN;
    if (any_grad) {
      st = run_label_logits(c, hid, weight, bias, stream, tr);
      if (st != LCE_OK) return st;
    }
    if (need_gh)
      LCE_LAUNCH(tr, LCE_K_TRANSPOSE, 0, 0, 0,
                 lce::launch_transpose(weight, s.ldw, 0, s.V, s.H, wT, s.Vp, nullptr, stream));
    for (int64_t g0 = 0; g0 < s.Np; g0 += G) {
      const bool last = g0 + G >= s.Np;
      const int64_t Gc = (s.Np - g0) < G ? (s.Np - g0) : G;
      const int64_t rows_valid = (s.N - g0) < Gc ? (s.N - g0) : Gc;
      if (!any_grad) {
        st = run_rows(c, hid, weight, bias, g0, Gc, nullptr, loss, lse, stream, tr);
        if (st != LCE_OK) return st;
        continue;
      }
      LCE_LAUNCH(tr, LCE_K_ROW_REF, 0, 0, 0,
                 lce::launch_prep_ref(c.label32, c.zlab, g0, Gc, rref, nullptr, stream));
      LCE_LAUNCH(tr, LCE_K_ZERO, 0, 0, 0, lce::launch_zero(ovf, 4, stream));
      st = run_rows(c, hid, weight, bias, g0, Gc, dlog, loss, lse, stream, tr, rref, ovf);
      if (st != LCE_OK) return st;
      LCE_LAUNCH(tr, LCE_K_BWD_DLOGITS, rows_valid, s.V, 0,
                 lce::launch_rowscale(c.label32, c.zy2, c.lse_ws, rref, row_scale, c.n_valid, grad_scale, is_mean,
                                      g0, Gc, dlog, rowc, ovf, 0, need_gb ? gb : nullptr, c.perm, stream));
      // retry, only when the overflow flag is set
      LCE_LAUNCH(tr, LCE_K_ROW_REF, 0, 0, 0,
                 lce::launch_prep_ref(c.label32, c.lse_ws, g0, Gc, rref, ovf, stream));
      LCE_LAUNCH(tr, LCE_K_FWD_RETRY, 0, 0, 0,
                 lce::launch_fwd_tiles(s, hid, weight, bias, g0, Gc, c.part_m, c.part_s, dlog, c.tile_ctr, rref,
                                       nullptr, ovf, c.label32, c.zy2, c.fwd_limit, stream));
      LCE_LAUNCH(tr, LCE_K_BWD_DLOGITS, rows_valid, s.V, 0,
                 lce::launch_rowscale(c.label32, c.zy2, c.lse_ws, rref, row_scale, c.n_valid, grad_scale, is_mean,
                                      g0, Gc, dlog, rowc, ovf, 1, need_gb ? gb : nullptr, c.perm, stream));
      // grad_bias column sums: inside grad_weight's K loop when it runs
      if (need_gb && !gb_in_gw)
        LCE_LAUNCH(tr, LCE_K_BIAS_SUMS, rows_valid, s.V, 0, lce::launch_bias_sums(s, dlog, rowc, Gc, gb, stream));
      if (need_gh)
        LCE_LAUNCH(tr, LCE_K_GRAD_HIDDEN, rows_valid, s.H, s.V,
                   lce::launch_grad_hidden(s, dlog, wT, g0, Gc, rowc, grad_hidden, c.bwd_limit, c.perm, gw_part,
                                           gw_part_items(s, G), stream));
      if (need_gw) {
        LCE_LAUNCH(tr, LCE_K_TRANSPOSE, 0, 0, 0,
                   lce::launch_transpose(hid, s.ldh, g0, rows_valid, s.H, hT, Gc, rowc, stream));
        LCE_LAUNCH(tr, LCE_K_GRAD_WEIGHT, s.V, s.H, rows_valid,
                   lce::launch_grad_weight(s, dlog, Gc, hT, rows_valid, gw_part, gw_part_items(s, G),
                                           (g0 == 0 && !accumulate) ? 1 : 0,
                                           gw, last ? grad_weight : nullptr,
                                           (!last || grad_weight == nullptr || grad_weight_f32 != nullptr) ? 1 : 0,
                                           rowc, gb_in_gw ? gb : nullptr, c.bwd_limit, g0, stream));
        if (last) gw_cast_done = true;
      }
    }
  }
  if (need_gw && grad_weight && !gw_cast_done)
    LCE_LAUNCH(tr, LCE_K_CAST, 0, 0, 0, lce::launch_cast(gw, grad_weight, s.V * s.H, stream));
  if (need_gb && grad_bias) LCE_LAUNCH(tr, LCE_K_CAST, 0, 0, 0, lce::launch_cast(gb, grad_bias, s.V, stream));
  LCE_LAUNCH(tr, LCE_K_FINALIZE_LOSS, 0, 0, 0,
             lce::launch_finalize_loss(c.chunk_acc, c.T, c.n_valid, c.status, p->reduction, loss, chunk_loss,
                                       stream));
  return LCE_OK;
}

int lce_forward_backward_traced(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                                const int64_t* labels, float grad_scale, float* loss, float* lse,
                                float* chunk_loss, int64_t* n_valid, void* grad_hidden, void* grad_weight,
                                void* grad_bias, float* grad_weight_f32, float* grad_bias_f32, int32_t* status,
                                void* workspace, size_t workspace_bytes, hipStream_t stream, lce_trace* trace) {
  return lce_forward_backward_ex(p, hidden, weight, bias, labels, grad_scale, loss, lse, chunk_loss, n_valid,
                                 grad_hidden, grad_weight, grad_bias, grad_weight_f32, grad_bias_f32, status,
                                 workspace, workspace_bytes, stream, nullptr, trace);
}

int lce_scale(void* data, int32_t dtype, int64_t n, const float* scale, hipStream_t stream) {
  if (n < 0) return LCE_ERR_INVALID_ARG;
  if (n == 0) return LCE_OK;
  if (data == nullptr || scale == nullptr) return LCE_ERR_INVALID_ARG;
  if (dtype != LCE_DTYPE_BF16 && dtype != LCE_DTYPE_F32) return LCE_ERR_INVALID_ARG;
  return lce::launch_scale(data, dtype == LCE_DTYPE_F32, n, scale, stream) == hipSuccess ? LCE_OK : LCE_ERR_HIP;
}

int lce_forward_backward(const lce_problem* p, const void* hidden, const void* weight, const void* bias,
                         const int64_t* labels, float grad_scale, float* loss, float* lse, float* chunk_loss,
                         int64_t* n_valid, void* grad_hidden, void* grad_weight, void* grad_bias,
                         float* grad_weight_f32, float* grad_bias_f32, int32_t* status, void* workspace,
                         size_t workspace_bytes, hipStream_t stream) {
  return lce_forward_backward_traced(p, hidden, weight, bias, labels, grad_scale, loss, lse, chunk_loss, n_valid,
                                     grad_hidden, grad_weight, grad_bias, grad_weight_f32, grad_bias_f32, status,
                                     workspace, workspace_bytes, stream, nullptr);
}

}  // extern "C"
