// Device kernels of the chunked linear-cross-entropy library, written for
// gfx950 (CDNA4, MI355X): 64-lane wavefronts, v_mfma_f32_16x16x32_bf16,
// 160 KB of LDS per workgroup, direct global->LDS loads.
//
// What is computed (LlamaFactory PR #10762 analysis, section 4; TRL
// "training on 1M+ tokens", section "chunking"):
//   z = h W^T + b, lse_i = log sum_j exp z_ij, l_i = valid_i (lse_i - z_{i,y_i}),
//   G = s valid (softmax - onehot), grad_hidden = G W, grad_weight = G^T h,
//   grad_bias = sum_i G_i  (FP32 accumulation, one cast at the end).
//
// Every contraction runs through one bf16 MFMA tile routine that computes
//   C[m][n] = sum_k X[m][k] * Y[n][k]
// for a 256 x 256 output tile, so the kernels differ only in their operands
// and epilogues:
//   z tile       X = hidden rows,  Y = weight rows,  K = H
//                (per backward row group the epilogue also keeps bf16
//                p~ = exp(z - r_i), r_i the row's label logit; with one
//                patched entry per row and a row scale c, G = diag(c) p~')
//   grad_hidden  X = p~',          Y = W^T,          K = Vp   (rows scaled by c)
//   grad_weight  X = p~'^T,        Y = (c h)^T,      K = the group's rows
// Operands are K-contiguous in memory except p~' in grad_weight, which is read
// K-major and transposed by the LDS reads (FragAT). The backward operands
// are written by this library's own passes, so they are stored as K-slabs:
// [K/64][rows][64], each 64-deep stage of a 256-row tile one contiguous
// 32 KB block (row-major operands with row strides of 30-300 KB touch
// hundreds of DRAM pages per stage; measured 1-6% slower).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "lce_internal.h"

#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))

namespace lce {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int TILE = 256;                 // output tile edge (rows and columns)
constexpr int BK = 64;                    // K depth of one LDS stage (two MFMA steps)
constexpr int NTHREADS = 512;             // 8 waves (two per SIMD), 2 x 4, each owns 128 x 64
constexpr int NB = 8;                     // 16 x 16 MFMA row blocks per wave (128 / 16)
constexpr int NBJ = 4;                    // 16 x 16 MFMA column blocks per wave (64 / 16)
constexpr int NQ = TILE / 64;             // column quarters of a tile (one per wave column)
constexpr int OPERAND_STAGE = TILE * BK * 2;       // 32 KB: one operand, one stage
constexpr int STAGE = 2 * OPERAND_STAGE;           // 64 KB: both operands
constexpr int MAINLOOP_LDS = 2 * STAGE;            // 128 KB: double buffered
constexpr float LOG2E = 1.4426950408889634f;       // log2(e): exp(x) = 2^(x log2 e)
constexpr float LN2 = 0.6931471805599453f;         // ln(2) = 1 / log2(e)
constexpr float REF_CAP2 = 60.f * LOG2E;           // largest exponent (base 2) of a stored p~: e^60
constexpr float REF_SUM_CAP = 1.1420074e26f;       // e^60: largest partial sum against a reference
// s_waitcnt immediates (gfx9 encoding: vmcnt [3:0]+[15:14], expcnt [6:4],
// lgkmcnt [11:8]); the other counters are left at their maximum (no wait).
constexpr int WAIT_LGKM0 = 0xC07F;   // lgkmcnt(0)
constexpr int WAIT_VM0 = 0x0F70;     // vmcnt(0)
#define WAIT_VM(n) (((n) & 15) | (((n) >> 4) << 14) | 0x0F70)   // vmcnt(n), n <= 63

__device__ __forceinline__ float bf2f(u16 u) { return __builtin_bit_cast(float, (uint32_t)u << 16); }
__device__ __forceinline__ u16 f2bf(float x) {
  __bf16 b = (__bf16)x;                    // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(u16, b);
}

// Reductions across the 16 lanes that hold one accumulator row, with DPP
// lane permutations (plain VALU operations, no LDS round trip): swap lanes
// within pairs, then within quads, then mirror each 8-lane half, then mirror
// the 16-lane row; each step combines two disjoint groups, so after four
// steps every lane holds the result over its 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_XOR1 = 0xB1;          // quad_perm [1,0,3,2]
constexpr int DPP_XOR2 = 0x4E;          // quad_perm [2,3,0,1]
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <- 7 - i within each 8 lanes
constexpr int DPP_MIRROR = 0x140;       // lane i <- 15 - i within each 16 lanes
__device__ __forceinline__ float sum16(float v) {
  v += dpp<DPP_XOR1>(v);
  v += dpp<DPP_XOR2>(v);
  v += dpp<DPP_HALF_MIRROR>(v);
  return v + dpp<DPP_MIRROR>(v);
}

// Max / sum over the 16 lanes of each row group for four rows at once, by
// the same butterfly (xor 1, xor 2, half mirror, mirror): every lane ends
// with its row's result. One block of fused DPP instructions: the compiler
// lowers fmaxf over a DPP move to a zeroing move, the move, a canonicalising
// max and the max. The leading s_nop 4 covers the DPP hazards (a VALU write
// of the source needs 2 wait states before a DPP read of it, an EXEC write
// 5); inside the block each source was written four instructions earlier.
#define LCE_DPP_STEP4(OP, CTRL)                                      \
  OP " %0, %0, %0 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
  OP " %1, %1, %1 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
  OP " %2, %2, %2 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
  OP " %3, %3, %3 " CTRL " row_mask:0xf bank_mask:0xf\n\t"
#define LCE_DPP_BUTTERFLY4(OP)                                       \
  "s_nop 4\n\t"                                                     \
  LCE_DPP_STEP4(OP, "quad_perm:[1,0,3,2]")                           \
  LCE_DPP_STEP4(OP, "quad_perm:[2,3,0,1]")                           \
  LCE_DPP_STEP4(OP, "row_half_mirror")                               \
  LCE_DPP_STEP4(OP, "row_mirror")
__device__ __forceinline__ void max16x4(float (&v)[4]) {
  asm volatile(LCE_DPP_BUTTERFLY4("v_max_f32_dpp") : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}
__device__ __forceinline__ void sum16x4(float (&v)[4]) {
  asm volatile(LCE_DPP_BUTTERFLY4("v_add_f32_dpp") : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]));
}
// Two floats to bf16 (round to nearest even) in one v_cvt_pk_bf16_f32: a in
// the low half, b in the high half.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f2bf2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// ---------------------------------------------------------------------------
// Tile order. Workgroups are dispatched round-robin over the 8 XCDs, so
// dispatch id b runs on XCD b % 8. Remap so each XCD walks a contiguous range
// of logical tiles, and walk them GROUP_M row-tiles at a time across all
// column tiles, so concurrently running tiles on one XCD share operand panels
// in that XCD's L2.
// ---------------------------------------------------------------------------
template <int GROUP_M = 4>
__device__ __forceinline__ void tile_from_index(int t, int n_m, int n_n, int& tm, int& tn) {
  const int per_group = GROUP_M * n_n;
  const int g = t / per_group;
  const int first_m = g * GROUP_M;
  const int gm = min(n_m - first_m, GROUP_M);
  const int in_g = t - g * per_group;
  tm = first_m + in_g % gm;
  tn = in_g / gm;
}
// One workgroup per tile (grid = n_m * n_n).
__device__ __forceinline__ void tile_coords(int n_m, int n_n, int& tm, int& tn) {
  const int nb = gridDim.x;
  int t = blockIdx.x;
  if ((nb & 7) == 0) t = (t & 7) * (nb >> 3) + (t >> 3);
  tile_from_index(t, n_m, n_n, tm, tn);
}
// Persistent kernels (grid a multiple of 8, at most one workgroup per CU):
// tile k of this workgroup's XCD (x = blockIdx % 8), taken in order by the
// XCD's workgroups; false past the XCD's last tile. The 8 XCDs should walk
// the column (weight) tiles in step, so that each weight panel comes from
// HBM once and the other XCDs find it in the MALL. The row tiles go in
// blocks of 64 and a remainder of r = n_m % 64:
// * in each block of 64, XCD x owns the 8-row group 8x .. 8x+7 across all
//   column tiles (tile_from_index<8>: windows of 8 x 4 tiles, measured ~1%
//   faster than 4 x 8), so the XCDs stay in step on equal work;
// * a remainder r >= 32: the r x C tiles of each group of C column tiles
//   (C = 4, or 8 for odd r) are dealt out in row-major order, q = r C / 8 to
//   each XCD, so every XCD takes the same number of tiles per column group
//   (a block of r / 8 rows x C columns: at least 4 x 4);
// * a remainder r < 32: XCD x takes the slice [x, x + 1) / 8 of the
//   remainder's tiles in row-group order, about n_n / 8 adjacent columns of
//   all its rows (dealt blocks would be thin slivers with little L2 reuse).
// Slices of the row-group order over all n_m row tiles put the XCDs on up to
// 8 unrelated column phases when n_m is not a multiple of 64: the forward
// tiles ran 3-7% slower per tile there (40-96 row tiles) than at 64; dealt,
// 40-60 row tiles gained 2-4% per tile.
__device__ __forceinline__ bool xcd_tile(int n_m, int n_n, int k, int& tm, int& tn) {
  const int x = (int)(blockIdx.x & 7);
  const int full = n_m & ~63, r = n_m - full;
  const int per_block = 8 * n_n;                  // this XCD's tiles in each block of 64 row tiles
  const int in_blocks = (full >> 6) * per_block;
  if (k < in_blocks) {
    const int blk = k / per_block;
    tile_from_index<8>(k - blk * per_block, 8, n_n, tm, tn);
    tm += 64 * blk + 8 * x;
    return true;
  }
  k -= in_blocks;
  if (r >= 32) {
    const int C = (r & 1) ? 8 : 4, q = r * C / 8;
    const int cg = k / q;
    const int cw = min(C, n_n - cg * C);   // columns in this group (the last may be narrower)
    const int j = x * q + (k - cg * q);    // row-major index in the group
    if (cw <= 0 || j >= r * cw) return false;
    const int row = j / cw;
    tm = full + row;
    tn = cg * C + (j - row * cw);
    return true;
  }
  const int ntiles = r * n_n;
  const int per_xcd = (ntiles + 7) >> 3;
  const int t = x * per_xcd + k;
  if (k >= per_xcd || t >= ntiles) return false;
  tile_from_index<8>(t, r, n_n, tm, tn);
  tm += full;
  return true;
}

// ---------------------------------------------------------------------------
// LDS stage layout: operand tile [256 rows][64 k] bf16, 128 B per row (one
// 128-byte line of the operand, so every line the loads touch is used
// whole), the eight 16-byte k-chunks of row r stored at chunk slot
// (c ^ swz(r)). A fragment read (ds_read_b128) takes chunk c of 16 rows; the
// LDS serves 16 lanes x 16 B per clock across 64 banks and rows r and r+2
// share banks: swz(r) = (r >> 1) & 7 gives the 16 lanes 16 distinct 16-byte
// bank groups, so the reads are conflict-free.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int lds_off(int r, int c) { return r * 128 + ((c ^ swz(r)) << 4); }

// Direct global->LDS fills. One global_load_lds_dwordx4 writes 64 x 16 B
// contiguously (lane i at +16 i), i.e. 8 tile rows of 128 B; lane i fetches
// the logical chunk stored at slot (i & 7) of row (i >> 3) of its 8-row
// block: c = (i & 7) ^ swz(row). Each of the 8 waves fills 32 rows of each
// operand per stage (4 loads per operand). Rows past the operand's end are
// clamped to its last row (finite values the epilogues discard).
//
// The per-lane byte offsets inside the tile are fixed for the whole K loop
// (StageOffsets, computed once); the tile base is wave-uniform (scalar
// registers) and each stage only adds 128 bytes to the 32-bit offsets.
constexpr int FILLS = 4;                   // loads per wave per operand per stage
struct StageOffsets {
  uint32_t off[FILLS];
};
__device__ __forceinline__ StageOffsets stage_offsets(int64_t ld, int64_t row0, int64_t nrows, int wave,
                                                      int lane) {
  StageOffsets o;
#pragma unroll
  for (int b = 0; b < FILLS; ++b) {
    const int r = wave * 32 + b * 8 + (lane >> 3);
    const int c = (lane & 7) ^ swz(r);
    int64_t lr = r;
    if (row0 + lr > nrows - 1) lr = nrows - 1 - row0;
    o.off[b] = (uint32_t)((lr * ld + c * 8) * 2);
  }
  return o;
}
// One 16-byte-per-lane global->LDS load: lane i's 16 bytes from gbase + voff
// land at LDS address lds_addr + 16 i (lds_addr in M0). Written as inline
// assembly so the compiler does not treat the in-flight LDS writes as
// possibly aliasing every later LDS read (it would wait for the loads to
// complete before each read); the main loop orders them explicitly with
// s_waitcnt vmcnt and a barrier before any read of a refilled buffer.
// M0 is used for nothing else in these kernels.
__device__ __forceinline__ void lds_dma16(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory", "m0");
}

__device__ __forceinline__ bf16x8 frag(const LDS_AS char* stage, int r, int c) {
  return *(const LDS_AS bf16x8*)(stage + lds_off(r, c));
}

struct Acc {
  f32x4 v[NB][NBJ];   // [row block i][col block j], 16 x 16 each
};

// Accumulator layout (v_mfma_f32_16x16x32_bf16): lane l, register r (0..3) of
// block (i, j) of wave (wm, wn) holds C[row][col] with
//   row = wm*128 + i*16 + 4*(l/16) + r,   col = wn*64 + j*16 + (l%16).
// Operand fragments: lane l supplies row (l%16) of its 16-row block and the
// 8 consecutive k at 8*(l/16) of the 32-deep step, for A and for B alike.
__device__ __forceinline__ int acc_row(int wm, int i, int r, int lane) {
  return wm * 128 + i * 16 + 4 * (lane >> 4) + r;
}
__device__ __forceinline__ int acc_col(int wn, int j, int lane) { return wn * 64 + j * 16 + (lane & 15); }

// Operand tiles of one GEMM tile and where their stages go. Stage s of an
// operand starts at base + s * kstride bytes: 128 for a row-major operand
// (the next 64 k of the same rows), rows * 128 for one stored as K-slabs
// [K/64][rows][64] (the next slab).
struct TileLoads {
  const void* xbase;
  const void* ybase;
  int64_t kx, ky;
  StageOffsets ox, oy;
  uint32_t lds_wave;     // LDS byte address of this wave's 32 rows in stage buffer 0
};

__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t b64 = (uint64_t)(uintptr_t)p;
  const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  return (const void*)(uintptr_t)((hi << 32) | lo);
}

// 16 x the lane index, computed where it is used: kept live across the K
// loop it would be spilled, and its reload waits for every store in flight.
__device__ __forceinline__ uint32_t lane_x16() {
  uint32_t v;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0\n\tv_lshlrev_b32 %0, 4, %0"
               : "=v"(v));
  return v;
}

// Issues load f (0..7) of stage s: f < 4 fill X rows, f >= 4 fill Y rows.
__device__ __forceinline__ void stage_load(const TileLoads& t, int s, int f) {
  const uint32_t buf = t.lds_wave + (uint32_t)((s & 1) * STAGE);
  if (f < FILLS)
    lds_dma16((const char*)t.xbase + s * t.kx, t.ox.off[f], buf + f * 1024);
  else
    lds_dma16((const char*)t.ybase + s * t.ky, t.oy.off[f - FILLS], buf + OPERAND_STAGE + (f - FILLS) * 1024);
}

#define FENCE() __builtin_amdgcn_sched_barrier(0)

// Workgroup barrier without the memory fence __syncthreads() adds (the fence
// would drain every outstanding LDS read); the main loop orders its LDS
// traffic itself with explicit s_waitcnt. The memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void bare_barrier() { asm volatile("s_barrier" ::: "memory"); }

// Fragments of one 32-deep sub-step: A row blocks 0..7, B column blocks 0..3.
struct Frags {
  bf16x8 a[NB], b[NBJ];
};
// Fragment read n (0..11) of sub-step `sub` (0, 1) of the stage in `buf`: B
// blocks first (every MFMA of the first row block needs all of them), then A.
// FragK: both operands K-contiguous in LDS (the layout above).
struct FragK {
  static constexpr int kBar = 9;
  static constexpr bool kPrio = true;        // raise the wave's priority around its MFMAs
  static constexpr bool kPrioLoads = true;   // ... and while it issues its direct loads (see mainloop_stage)
  int rA, rB, q;
  __device__ __forceinline__ FragK(int wave, int lane)
      : rA((wave >> 2) * 128 + (lane & 15)), rB((wave & 3) * 64 + (lane & 15)), q(lane >> 4) {}
  __device__ __forceinline__ void read(Frags& f, const LDS_AS char* buf, int sub, int n) const {
    if (n < NBJ) f.b[n] = frag(buf + OPERAND_STAGE, rB + n * 16, sub * 4 + q);
    else f.a[n - NBJ] = frag(buf, rA + (n - NBJ) * 16, sub * 4 + q);
  }
  // work beside the fragment reads and the loads of each slot (none here;
  // see FragATBias)
  __device__ __forceinline__ void side(int, int, const LDS_AS char*) {}
  __device__ __forceinline__ void side_load(int, int, int) const {}
};

// K-major stage layout, for operands whose rows run along K in memory: tile
// [64 k][256 m] bf16, 512 B per k row, the 16-byte m-chunk c of row k at
// chunk slot c ^ (2 tr_swz(k)). Fragments come from ds_read_b64_tr_b16, which
// within each 16-lane group hands lane i element i % 4 of the 8-byte reads of
// lanes i/4, i/4 + 4, i/4 + 8 and i/4 + 12. So lane j of group q points at
// row k0 + j/4, m = m0 + 4 (j % 4): lane i then holds m0 + i for k0 .. k0+3,
// half of its MFMA operand (k0 = 8q, then 8q + 4). One read of half a wave
// (two groups) touches rows k0 + 0..3 and k0 + 8..11; tr_swz gives those
// eight rows eight different 32-byte bank groups.
constexpr int TR_ROW = 512;
__device__ __forceinline__ int tr_swz(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 frag_tr(const LDS_AS char* p) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)p);
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS s16x4*)(p + 4 * TR_ROW));
  return __builtin_bit_cast(bf16x8, (s16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// FragAT: A K-major (transposing reads; per-lane byte offsets of its 8
// fragments in a stage, sub-step 0, first half, fixed for the whole K loop),
// B K-contiguous (as FragK). (Raising the wave priority as FragK does
// measured no faster here.)
struct FragAT {
  static constexpr int kBar = 10;
  static constexpr bool kPrio = false;
  static constexpr bool kPrioLoads = false;
  uint32_t a[NB];
  int rB, q;
  __device__ __forceinline__ FragAT(int wave, int lane) : rB((wave & 3) * 64 + (lane & 15)), q(lane >> 4) {
    const int j = lane & 15, t = tr_swz(8 * q + (j >> 2));
    const uint32_t row = (uint32_t)(8 * q + (j >> 2)) * TR_ROW + 8 * (j & 3);
#pragma unroll
    for (int i = 0; i < NB; ++i) a[i] = row + 32 * (((wave >> 2) * NB + i) ^ t);
  }
  __device__ __forceinline__ void read(Frags& f, const LDS_AS char* buf, int sub, int n) const {
    if (n < NBJ) f.b[n] = frag(buf + OPERAND_STAGE, rB + n * 16, sub * 4 + q);
    else f.a[n - NBJ] = frag_tr(buf + a[n - NBJ] + sub * 32 * TR_ROW);
  }
  __device__ __forceinline__ void side(int, int, const LDS_AS char*) {}
  __device__ __forceinline__ void side_load(int, int, int) const {}
};

// FragAT for grad_weight with grad_bias folded in: grad_bias[v] = sum_k
// c_k G'[k][v] over the group's rows k is a column sum of the A operand
// already in LDS. All n_nt tiles of vocabulary tile tm see every stage of
// G'; the one with hidden-tile index tn sums rows r = tn + j n_nt of each
// stage for j < 4 R, which covers the 64 rows once over the n_nt tiles
// when R n_nt >= 16 (R from grad_weight_bias_rows). Wave w takes columns
// 128 (w%2) .. +127 of rows j = w/2 + 4 m (m < R): L = 2, 4 or 8 adjacent
// columns per lane (R = 1, 2, >= 4), so one read of 4, 8 or 16 bytes per
// lane covers 1, 2 or 4 rows (lane groups of 64 / (L/2) lanes), and R / (L/2)
// such reads (1, 2 or 4) cover the wave's rows. Read i and the row scales
// of its rows go out in slot 6 + i, their FMAs follow in slot 8 (one read)
// or in the next slot (slots 6..9 have no fragment reads, and the stage's
// buffer is read-only until the barrier of slot 10, FragAT's kBar). A lane
// whose row would be past 63 reads row 0 with a row scale of zero (R = 1:
// the whole wave, whose sums are dropped at the end instead). Each wave
// brings the 64 row scales of every stage into two LDS slots of its own (one
// 256-byte direct load issued with the stage's operand loads and covered by
// the same wait), so every wait stays in LDS order and the K loop takes no
// extra branch. (Summing whole stages in one tile out of n_nt instead,
// behind per-slot tests of the stage index, measured 2-3% slower for
// grad_weight even with the sums removed.)
__device__ __forceinline__ void lds_dma4(const void* gbase, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :: "s"(lds_addr), "v"(voff), "s"(gbase) : "memory", "m0");
}
template <int W> struct LdsWord;   // one lane's read of W 32-bit words
template <> struct LdsWord<1> { typedef uint32_t T; };
template <> struct LdsWord<2> { typedef u32x2 T; };
template <> struct LdsWord<4> { typedef u32x4 T; };
__device__ __forceinline__ uint32_t word_at(uint32_t w, int) { return w; }
__device__ __forceinline__ uint32_t word_at(u32x2 w, int e) { return w[e]; }
__device__ __forceinline__ uint32_t word_at(u32x4 w, int e) { return w[e]; }
template <int R>
struct FragATBias : FragAT {
  static_assert(R == 1 || R == 2 || R == 4 || R == 8 || R == 16, "rows per wave and stage");
  static constexpr int L = R == 1 ? 2 : R == 2 ? 4 : 8;   // adjacent columns per lane
  static constexpr int RPR = L / 2;                        // rows per read
  static constexpr int NRD = R / RPR;                      // reads per stage
  static constexpr int D = NRD == 1 ? 2 : 1;               // slots from a read to its FMAs
  static_assert(6 + NRD - 1 < kBar, "the reads of a stage precede its barrier");
  typedef typename LdsWord<L / 2>::T Word;
  float gb[L];
  const float* rowc;     // row scales of the tile's first K row (uniform)
  uint32_t c_lds;        // LDS byte address of this wave's two slots of 64 row scales
  uint32_t x_off0;       // byte offset of this lane's read 0 in a stage: row * TR_ROW + (< TR_ROW)
  uint32_t c_off0;       // byte offset of read 0's row scale in a slot
  int step;              // rows from one read to the next (several reads)
  bool ok[NRD];          // read i's row is below 64
  Word x[NRD];           // read i's G' values ...
  float c[NRD];          // ... and row scale
  __device__ __forceinline__ FragATBias(int wave, int lane, const float* rowc_, uint32_t c_lds_, int tn, int n_nt)
      : FragAT(wave, lane), rowc(rowc_), c_lds(c_lds_) {
    const int lpr = 64 / RPR, g = lane / lpr, cl = lane % lpr;
    const uint32_t byte = (uint32_t)((wave & 1) * 256 + cl * 2 * L);   // in the row, before the swizzle
    // read i covers m = i RPR + g, row r0 + 16 i n_nt (several reads: RPR = 4)
    const int r0 = tn + ((wave >> 1) + 4 * g) * n_nt;
    step = 16 * (R == 16 ? 1 : n_nt);   // R = 16 only for n_nt = 1, where every row is below 64
#pragma unroll
    for (int i = 0; i < NRD; ++i) ok[i] = R == 16 || r0 + i * step < 64;
    // one read: a row past 63 reads row 0. Several (R >= 8, n_nt <= 3): r0 <= 47
    // and every row is below 128, so each read stays inside the stage buffers.
    const int rr = NRD == 1 && !ok[0] ? 0 : r0;
    // the 16-byte chunk byte/16 of row rr sits at slot chunk ^ 2 tr_swz(rr),
    // and rows 16 apart share the swizzle
    x_off0 = (uint32_t)rr * TR_ROW + ((((byte >> 4) ^ (uint32_t)(2 * tr_swz(rr)))) << 4) + (byte & 15);
    c_off0 = (uint32_t)rr * 4;
#pragma unroll
    for (int e = 0; e < L; ++e) gb[e] = 0.f;
  }
  __device__ __forceinline__ uint32_t x_off(int i) const { return x_off0 + (uint32_t)(i * step * TR_ROW); }
  __device__ __forceinline__ uint32_t c_off(int i) const {
    return NRD == 1 || ok[i] ? c_off0 + (uint32_t)(i * step * 4) : 0u;
  }
  // the 64 row scales of stage s into this wave's slot s & 1
  __device__ __forceinline__ void load_c(int s) const {
    lds_dma4(uniform_ptr(rowc + (int64_t)s * 64), lane_x16() >> 2, c_lds + (uint32_t)((s & 1) * 256));
  }
  __device__ __forceinline__ void side(int slot, int s, const LDS_AS char* cur) {
#pragma unroll
    for (int i = 0; i < NRD; ++i)
      if (slot == 6 + i + D) {
#pragma unroll
        for (int e = 0; e < L / 2; ++e) {
          const uint32_t w = word_at(x[i], e);
          gb[2 * e] = fmaf(c[i], __builtin_bit_cast(float, w << 16), gb[2 * e]);
          gb[2 * e + 1] = fmaf(c[i], __builtin_bit_cast(float, w & 0xFFFF0000u), gb[2 * e + 1]);
        }
      }
#pragma unroll
    for (int i = 0; i < NRD; ++i)
      if (slot == 6 + i) {
        x[i] = *(const LDS_AS Word*)(cur + x_off(i));
        const float cv = *(const LDS_AS float*)((const LDS_AS char*)0 + c_lds + (uint32_t)((s & 1) * 256) + c_off(i));
        c[i] = R == 1 || ok[i] ? cv : 0.f;   // R = 1: the row is the wave's, dropped at the end instead
      }
  }
  // row scales of stage s + 2, issued with its operand loads (stages 0 and
  // 1: before the K loop)
  __device__ __forceinline__ void side_load(int slot, int s, int nk) const {
    if (slot == kBar && s + 2 < nk) load_c(s + 2);
  }
};

// Schedule of one 64-deep stage s, in 16 slots of 4 MFMAs (slots 0..7:
// sub-step 0 from fragment set f0, slots 8..15: sub-step 1 from f1), two
// waves per SIMD, with the barrier in slot B = FS::kBar (9 for FragK, 10
// for FragAT):
//   slots 0..5    read f1 (stage s, sub-step 1), two fragments per slot
//   slot B        wait for this wave's loads of stage s+1 and its LDS reads,
//                 barrier: stage s+1 is visible from every wave, and buffer
//                 s&1 is no longer read (f0 and f1 of stage s are in registers)
//   slots B..15   read f0 of stage s+1 (12 fragments spread over 16 - B slots)
//   slots B..15, and 0..B-9 of stage s+1: the 8 global->LDS loads of stage
//                 s+2 into buffer s&1, one per slot (after the second MFMA)
// so every load has at least eight slots to land before the barrier that
// publishes it. (Measured: two waves per SIMD with this schedule beat one
// wave per SIMD with 128 x 128 per wave by 1.5-5%; issuing the loads two per
// slot was slower here. The barrier in slot 9 instead of 10 made the
// forward tiles 1% faster and grad_hidden no slower, slot 11 or 8 slower;
// grad_weight is best with 10.) With FragK the wave raises its priority for
// its MFMA pairs and while it issues its direct loads, so that when both
// waves of a SIMD are ready those go before fragment reads: measured
// 1.3-1.6% faster for the MFMA pairs alone, then another 0.5% (grad_hidden)
// to 3.8% (the forward tiles) with the loads.
// At entry: f0 holds stage s sub-step 0; loads 0..15-B of stage s+1 went out
// in the previous stage (slots B..15), the rest go out in slots 0..B-9.
template <class FS>
__device__ __forceinline__ void mainloop_stage(Acc& acc, Frags& f0, Frags& f1, int s, int nk, LDS_AS char* smem,
                                               const TileLoads& t, FS& fs) {
  // f1's reads (slots 0..5) and FragATBias's (slot 6) precede the barrier;
  // the loads of stage s+1 left for this stage fit in slots 0..kBar-9
  static_assert(FS::kBar >= 8 && FS::kBar <= 15, "barrier slot out of range");
  LDS_AS char* cur = smem + (s & 1) * STAGE;
  LDS_AS char* nxt = smem + ((s + 1) & 1) * STAGE;
#pragma unroll
  for (int slot = 0; slot < 16; ++slot) {
    const int i = slot & 7;
    Frags& f = slot < 8 ? f0 : f1;
    if (slot == FS::kBar) {
      if (s + 1 < nk) __builtin_amdgcn_s_waitcnt(WAIT_VM0);
      __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
      bare_barrier();
    }
    FENCE();
    if (FS::kPrio) __builtin_amdgcn_s_setprio(1);
    acc.v[i][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[0], acc.v[i][0], 0, 0, 0);
    acc.v[i][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[1], acc.v[i][1], 0, 0, 0);
    if (FS::kPrio) __builtin_amdgcn_s_setprio(0);
    FENCE();
    if (FS::kPrioLoads) __builtin_amdgcn_s_setprio(1);
    if (slot < FS::kBar - 8) {
      if (s + 1 < nk) stage_load(t, s + 1, (16 - FS::kBar) + slot);
    } else if (slot >= FS::kBar) {
      if (s + 2 < nk) stage_load(t, s + 2, slot - FS::kBar);
    }
    fs.side_load(slot, s, nk);
    if (FS::kPrioLoads) __builtin_amdgcn_s_setprio(0);
    // fragment reads: f1 of this stage in slots 0..5, f0 of the next in 10..15
    constexpr int NS = 16 - FS::kBar;   // slots for the 12 reads of the next f0
    const int rlo = slot >= FS::kBar ? (slot - FS::kBar) * 12 / NS : 0;
    const int rhi = slot >= FS::kBar ? (slot - FS::kBar + 1) * 12 / NS : 0;
    const int rmid = rlo + (rhi - rlo + 1) / 2;
    if (slot < 6) fs.read(f1, cur, 1, 2 * slot);
    else if (slot >= FS::kBar)
      for (int n = rlo; n < rmid; ++n) fs.read(f0, nxt, 0, n);
    fs.side(slot, s, cur);
    FENCE();
    if (FS::kPrio) __builtin_amdgcn_s_setprio(1);
    acc.v[i][2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[2], acc.v[i][2], 0, 0, 0);
    acc.v[i][3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.a[i], f.b[3], acc.v[i][3], 0, 0, 0);
    if (FS::kPrio) __builtin_amdgcn_s_setprio(0);
    FENCE();
    if (slot < 6) fs.read(f1, cur, 1, 2 * slot + 1);
    else if (slot >= FS::kBar)
      for (int n = rmid; n < rhi; ++n) fs.read(f0, nxt, 0, n);
  }
  FENCE();
}

// C tile (256 x 256, fp32 in registers) = X[x_row0 : +256][0:K] * Y[y_row0 : +256][0:K]^T.
// K % 64 == 0; ldx / ldy are the row strides in elements (64 for K-slab
// operands) and kx / ky the bytes from one 64-deep stage to the next (see
// TileLoads); 256 rows of either operand span < 4 GiB (row strides below
// 2^22 elements). smem must hold MAINLOOP_LDS bytes. Every LDS access of the
// stages (loads and reads) completes before the routine returns, but without
// a final barrier: a caller that reuses smem must synchronise first.
//
// In three steps, so that a persistent kernel can issue the next tile's first
// loads before it runs the current tile's epilogue: tile_setup (addresses
// only), tile_prologue (stage 0 and the first 16 - kBar loads of stage 1;
// the rest go out in the first slots of stage 0) and tile_run (the K loop),
// both for the fragment set FS the K loop uses. Between
// tile_prologue and tile_run the caller may issue any other memory accesses
// except to the stage buffers: tile_run's first wait (vmcnt <= 16 - kBar) is then
// only stricter, since direct loads complete in issue order.
__device__ __forceinline__ TileLoads tile_setup(const u16* __restrict__ X, int64_t ldx, int64_t kx, int64_t x_row0,
                                                int64_t x_rows, const u16* __restrict__ Y, int64_t ldy, int64_t ky,
                                                int64_t y_row0, int64_t y_rows, LDS_AS char* smem) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  TileLoads t;
  t.ox = stage_offsets(ldx, x_row0, x_rows, wave, lane);
  t.oy = stage_offsets(ldy, y_row0, y_rows, wave, lane);
  t.xbase = uniform_ptr(X + x_row0 * ldx);
  t.ybase = uniform_ptr(Y + y_row0 * ldy);
  t.kx = kx;
  t.ky = ky;
  t.lds_wave = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem + (uint32_t)wave * 32 * 128);
  return t;
}
template <class FS>
__device__ __forceinline__ void tile_prologue(const TileLoads& t, int nk) {
#pragma unroll
  for (int f = 0; f < 2 * FILLS; ++f) stage_load(t, 0, f);
  if (nk > 1)
#pragma unroll
    for (int f = 0; f < 16 - FS::kBar; ++f) stage_load(t, 1, f);
}
template <class FS>
__device__ __forceinline__ void tile_run(Acc& acc, const TileLoads& t, int nk, LDS_AS char* smem, FS& fs) {
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NBJ; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc.v[i][j][r] = 0.f;
  if (nk > 1) __builtin_amdgcn_s_waitcnt(WAIT_VM(16 - FS::kBar));
  else __builtin_amdgcn_s_waitcnt(WAIT_VM0);
  __syncthreads();
  Frags f0, f1;
#pragma unroll
  for (int n = 0; n < NB + NBJ; ++n) fs.read(f0, smem, 0, n);
  for (int s = 0; s < nk; ++s) mainloop_stage(acc, f0, f1, s, nk, smem, t, fs);
  __builtin_amdgcn_s_waitcnt(WAIT_LGKM0);
}
__device__ __forceinline__ void tile_run(Acc& acc, const TileLoads& t, int nk, LDS_AS char* smem) {
  const int tid = threadIdx.x;
  FragK fs(__builtin_amdgcn_readfirstlane(tid >> 6), tid & 63);
  tile_run(acc, t, nk, smem, fs);
}
__device__ __forceinline__ void gemm_tile(Acc& acc, const u16* __restrict__ X, int64_t ldx, int64_t kx,
                                          int64_t x_row0, int64_t x_rows, const u16* __restrict__ Y, int64_t ldy,
                                          int64_t ky, int64_t y_row0, int64_t y_rows, int64_t K,
                                          LDS_AS char* smem) {
  const int nk = (int)(K / BK);
  const TileLoads t = tile_setup(X, ldx, kx, x_row0, x_rows, Y, ldy, ky, y_row0, y_rows, smem);
  tile_prologue<FragK>(t, nk);
  tile_run(acc, t, nk, smem);
}

// ---------------------------------------------------------------------------
// Small kernels
// ---------------------------------------------------------------------------
__global__ void k_zero(uint32_t* __restrict__ p, int64_t n_words) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t s = (int64_t)gridDim.x * blockDim.x;
  for (; i < n_words; i += s) p[i] = 0u;
}

// label32[i] = y_i if valid and in range, else -1 (rows N..Np-1 too).
// n_valid += #valid rows; *status = LCE_ERR_LABEL_RANGE if any label is out of range.
// block_cnt (nullable): valid rows of each 256-row block.
__global__ void __launch_bounds__(256) k_prepare_labels(const int64_t* __restrict__ labels, int64_t N,
                                                        int64_t V, int64_t ignore_index,
                                                        int32_t* __restrict__ label32,
                                                        unsigned long long* __restrict__ n_valid,
                                                        int32_t* __restrict__ status, int32_t* __restrict__ block_cnt) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int lab = -1, bad = 0;
  if (i < N) {
    const int64_t y = labels[i];
    if (y != ignore_index) {
      if (y >= 0 && y < V) lab = (int)y;
      else bad = 1;
    }
  }
  label32[i] = lab;
  const int cnt = __syncthreads_count(lab >= 0);
  const int anybad = __syncthreads_or(bad);
  if (threadIdx.x == 0) {
    if (cnt) atomicAdd(n_valid, (unsigned long long)cnt);
    if (anybad) *status = 5;  // LCE_ERR_LABEL_RANGE
    if (block_cnt) block_cnt[blockIdx.x] = cnt;
  }
}

// ---------------------------------------------------------------------------
// Valid rows first. The backward only needs the rows with a label, so the
// rows are put in a stable order with every valid row before every ignored
// one (perm[slot] = original row; rows past N, which count as ignored, stay
// last) and the hidden rows are gathered in that order. Every backward
// kernel then stops at the device-side valid count: the host, which does not
// know that count, launches for all rows, and the launches past it return
// at once (grad_hidden writes the zero rows of ignored rows there).
// ---------------------------------------------------------------------------
// block_off[b] = sum of block_cnt[0 .. b-1]; one workgroup of 1024 threads.
__global__ void __launch_bounds__(1024) k_scan_blocks(const int32_t* __restrict__ block_cnt, int64_t nb,
                                                      int32_t* __restrict__ block_off) {
  __shared__ int32_t s_w[16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int32_t carry = 0;
  for (int64_t base = 0; base < nb; base += 1024) {
    const int64_t i = base + tid;
    const int32_t v = i < nb ? block_cnt[i] : 0;
    int32_t x = v;   // inclusive scan within the wave
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int32_t y = __shfl_up(x, d, 64);
      if (lane >= d) x += y;
    }
    if (lane == 63) s_w[wave] = x;
    __syncthreads();
    int32_t before = 0;
    for (int w = 0; w < wave; ++w) before += s_w[w];
    int32_t total = 0;
    for (int w = 0; w < 16; ++w) total += s_w[w];
    if (i < nb) block_off[i] = carry + before + x - v;
    carry += total;
    __syncthreads();
  }
}

// Slot of each row in the valid-first order; perm[slot] = row, labp[slot] =
// its label (-1 ignored). 256 rows per workgroup, ranks by wave ballots.
__global__ void __launch_bounds__(256) k_partition_rows(const int32_t* __restrict__ label32,
                                                        const int32_t* __restrict__ block_off,
                                                        const unsigned long long* __restrict__ n_valid, int64_t Np,
                                                        int32_t* __restrict__ perm, int32_t* __restrict__ labp) {
  __shared__ int32_t s_w[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b = blockIdx.x, row = b * 256 + tid;
  const int32_t lab = label32[row];
  const uint64_t m = __ballot(lab >= 0);
  if (lane == 0) s_w[wave] = (int32_t)__popcll(m);
  __syncthreads();
  int32_t rank = (int32_t)__popcll(m & ((1ull << lane) - 1ull));   // valid rows before this one in the wave
  for (int w = 0; w < wave; ++w) rank += s_w[w];
  const int64_t off = block_off[b];
  const int64_t slot = lab >= 0 ? off + rank
                                : (int64_t)*n_valid + (b * 256 - off) + (tid - rank);   // ignored rows in order
  if (slot >= 0 && slot < Np) {   // always (the counts add up to Np); a guard against a stale count
    perm[slot] = (int32_t)row;
    labp[slot] = lab;
  }
}

// out[slot][:] = in[perm[slot]][:] for slot < N (H columns, 16-byte copies).
__global__ void __launch_bounds__(256) k_gather_rows(const u16* __restrict__ in, int64_t ld_in,
                                                     const int32_t* __restrict__ perm, int64_t N, int64_t H,
                                                     u16* __restrict__ out) {
  const int64_t chunks = H / 8;
  const int64_t total = N * chunks;
  for (int64_t k = (int64_t)blockIdx.x * 256 + threadIdx.x; k < total; k += (int64_t)gridDim.x * 256) {
    const int64_t slot = k / chunks, c = k - slot * chunks;
    const u32x4 v = *(const u32x4*)(in + (int64_t)perm[slot] * ld_in + c * 8);
    *(u32x4*)(out + slot * H + c * 8) = v;
  }
}

// Staging tile for bf16 outputs that leave through LDS: 256 rows x 256
// columns, rows padded to 528 B (16-B aligned) so that the epilogue's 2-byte
// writes of lanes 0..31 and 32..63 (rows r and r+4) use different banks.
// Per-wave staging of one 16-row block of p~ (16 x 64 bf16, rows padded to
// 144 B: the 16-bit writes of the four 4-row groups of a wave land 16 banks
// apart), outside the stage buffers so that the next tile's loads can fill
// those while this tile's epilogue runs.
constexpr int PST_LD = 72;                     // u16 per staged row
constexpr int PST_WAVE = 16 * PST_LD;          // u16 per wave


// Forward tiles: z = h W^T + b for 256 rows x 256 vocabulary ids, reduced in
// the epilogue to each row's (max, sum exp(z - max)) over each wave's
// 64-column quarter of the tile (part index NQ*tile + quarter), in base-2
// units: t = z log2(e), partials (max t, sum 2^(t - max t)). The tile that
// holds a row's label column also stores that t (zy2, rows of label32 >= 0),
// so the loss l = ln2 ((M - t_y) + log2 S) comes from the same accumulators
// as the lse and is never negative (M >= t_y, S >= 1). z never leaves
// registers. With STORE_P (backward row groups) the tile also writes
// the bf16 unnormalised softmax exp(z - r_i) into p (K-slabs
// [Vp/64][ld_part][64]), r_i the row's reference from rref (its label logit,
// or its lse in the retry; see k_rowscale), or the quarter maximum where
// rref is NaN (ignored rows, rows past N); the logits are computed only once
// per call. Columns past V count as z = -inf (p = 0); a quarter with no
// column below V stores max = -inf and sum = 0.
//
// Persistent: one workgroup per CU takes tiles of its XCD's range
// (xcd_tile) and issues the next tile's first loads before this tile's
// epilogue, so their latency is covered by the epilogue's arithmetic and
// stores. The epilogue keeps out of the stage buffers: partials go straight
// from registers to global memory, p~ through a per-wave staging block, and
// the bias is read into registers at the start of the tile.
//
// Tiles are handed out in order by a per-XCD counter (tile_ctr[8], zero at
// launch): a workgroup that runs ahead takes the next unclaimed tile, so the
// tiles running at once on an XCD stay neighbours and share operand panels
// in its L2 (a fixed stride per workgroup let them drift apart: 38% more
// fabric reads). Lane 0 claims the tile after next during each epilogue and
// passes it through LDS.
template <bool STORE_P>
__global__ void __launch_bounds__(NTHREADS, 1)
k_fwd_tile(const u16* __restrict__ hidden, int64_t ldh, const u16* __restrict__ weight, int64_t ldw,
           const u16* __restrict__ bias, int64_t N, int64_t V, int64_t H, int64_t g0, int64_t ld_part, int n_mt,
           int n_vt, float* __restrict__ part_m, float* __restrict__ part_s, u16* __restrict__ p_out,
           int* __restrict__ tile_ctr, const float* __restrict__ rref, int* __restrict__ ovf,
           const int* __restrict__ only_if, const int32_t* __restrict__ label32, float* __restrict__ zy2,
           const unsigned long long* __restrict__ row_limit) {
  __shared__ __attribute__((aligned(16))) char smem_raw[MAINLOOP_LDS];
  __shared__ __attribute__((aligned(16))) u16 s_pst[STORE_P ? 8 * PST_WAVE : 8];
  __shared__ __attribute__((aligned(16))) float s_ref[STORE_P ? 2 * TILE : 4];   // per-row references, two tiles
  __shared__ __attribute__((aligned(16))) int s_lab[2 * TILE];                    // per-row labels, two tiles
  __shared__ int s_next;
  if (only_if != nullptr && *only_if == 0) return;   // a retry launch with nothing to retry
  if (row_limit != nullptr) {   // only the row tiles below the device-side limit (global row index)
    const int64_t lim = (int64_t)*row_limit - g0;
    const int64_t mt = lim <= 0 ? 0 : (lim + TILE - 1) / TILE;
    if (mt < n_mt) n_mt = (int)mt;
  }
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  LDS_AS u16* pst = (LDS_AS u16*)s_pst + (STORE_P ? wave * PST_WAVE : 0);
  const int nk = (int)(H / BK);
  const int xcd = (int)(blockIdx.x & 7), per_step = (int)(gridDim.x >> 3);
  int tm, tn;
  if (!xcd_tile(n_mt, n_vt, (int)(blockIdx.x >> 3), tm, tn)) return;
  if (tid == 0) s_next = per_step + atomicAdd(tile_ctr + xcd, 1);
  // The tile's 256 row references go to LDS ahead of its stage loads (one
  // direct load by wave 0; the K loop's first wait and barrier cover it).
  const bool use_ref = STORE_P && rref != nullptr;
  int par = 0;
  const uint32_t ref_lds = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS char*)s_ref);
  const uint32_t lab_lds = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS char*)s_lab);
  if (use_ref && wave == 0) lds_dma16(uniform_ptr(rref + (int64_t)tm * TILE), lane_x16(), ref_lds);
  if (wave == 1) lds_dma16(uniform_ptr(label32 + g0 + (int64_t)tm * TILE), lane_x16(), lab_lds);
  TileLoads t = tile_setup(hidden, ldh, BK * 2, g0 + (int64_t)tm * TILE, N, weight, ldw, BK * 2,
                           (int64_t)tn * TILE, V, smem);
  tile_prologue<FragK>(t, nk);
  for (;;) {
    const int64_t lrow0 = (int64_t)tm * TILE;       // row inside the group (or global row)
    const int64_t col0 = (int64_t)tn * TILE;
    const int ptn = tn;
    // Bias of this lane's four columns, loaded unconditionally (clamped
    // address, any valid pointer when there is no bias) and first used after
    // the K loop: a conditional load would make the compiler wait for it on
    // the spot, and with it for every direct load in flight.
    // (32-bit column offsets from a scalar base: V < 2^22.)
    const GLOBAL_AS u16* bsrc = (const GLOBAL_AS u16*)uniform_ptr(bias != nullptr ? bias : hidden);
    const int vmax = (int)V - 1;
    u16 braw[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int col = (int)col0 + acc_col(wn, j, lane);
      braw[j] = bsrc[bias != nullptr ? (col < vmax ? col : vmax) : 0];
    }
    Acc acc;
    tile_run(acc, t, nk, smem);
    // Bias pre-scaled by log2(e), -inf past V: exp(z - m) = exp2(acc*L + b*L
    // - m*L) is one FMA and one exp2 per element.
    float cbl[NBJ];
#pragma unroll
    for (int j = 0; j < NBJ; ++j) {
      const int col = (int)col0 + acc_col(wn, j, lane);
      cbl[j] = col <= vmax ? (bias != nullptr ? bf2f(braw[j]) * LOG2E : 0.f) : -INFINITY;
      // pinned here: computed later, the wait for braw would also wait for
      // the next tile's loads
      asm volatile("" ::"v"(cbl[j]));
    }
    const int k_next = s_next;   // claimed before this tile's K loop (whose barriers publish it)
    const bool more = xcd_tile(n_mt, n_vt, k_next, tm, tn);
    bare_barrier();   // every wave is past its last read of the stage buffers (and of s_next)
    if (more) {
      if (use_ref && wave == 0)
        lds_dma16(uniform_ptr(rref + (int64_t)tm * TILE), lane_x16(), ref_lds + (uint32_t)((par ^ 1) * TILE * 4));
      if (wave == 1)
        lds_dma16(uniform_ptr(label32 + g0 + (int64_t)tm * TILE), lane_x16(), lab_lds + (uint32_t)((par ^ 1) * TILE * 4));
      t = tile_setup(hidden, ldh, BK * 2, g0 + (int64_t)tm * TILE, N, weight, ldw, BK * 2, (int64_t)tn * TILE, V,
                     smem);
      tile_prologue<FragK>(t, nk);
    }
    // claim the tile after next now; the result is needed only after the
    // next K loop, and waiting for it at the end of the epilogue costs
    // nothing (the next tile's first loads, issued earlier, have landed)
    int claimed = 0;
    if (more && tid == 0) claimed = atomicAdd(tile_ctr + xcd, 1);
    float* pm = part_m + (int64_t)(NQ * ptn + wn) * ld_part + lrow0 + wm * 128 + 4 * (lane >> 4);
    float* ps = part_s + (int64_t)(NQ * ptn + wn) * ld_part + lrow0 + wm * 128 + 4 * (lane >> 4);
    u16* pq = STORE_P ? p_out + ((col0 >> 6) + wn) * ld_part * 64 + (lrow0 + wm * 128) * 64 : nullptr;
    // Label logits from these accumulators: a row's label column falls in
    // this wave's 64 columns for a few of its 128 rows at most, found with
    // two ballots (bit k: row wm*128 + k, then + 64); only a 16-row block
    // with such a row reads its labels and stores t_y = z_{i,y_i} log2(e),
    // the same value that enters the row's maximum and sum below.
    const LDS_AS int* labs = (const LDS_AS int*)s_lab + par * TILE + wm * 128;
    const int cw = (int)col0 + wn * 64;
    bool overflow = false;   // some row of this lane needs the retry
    uint64_t hit_lo, hit_hi;
    {
      const LDS_AS int* lp = (const LDS_AS int*)((const LDS_AS char*)labs + (lane_x16() >> 2));
      hit_lo = __ballot((unsigned)(lp[0] - cw) < 64u);
      hit_hi = __ballot((unsigned)(lp[64] - cw) < 64u);
    }
    // Whether every one of this wave's 128 rows has a reference (NaN: none),
    // a wave-uniform choice of the partial sums' shift below.
    bool all_ref = false;
    if (use_ref) {
      const LDS_AS float* wr = (const LDS_AS float*)s_ref + par * TILE + wm * 128;
      all_ref = __ballot(__builtin_isnan(wr[lane]) || __builtin_isnan(wr[lane + 64])) == 0;
    }
    // The four rows r of a row block are reduced together so their DPP
    // steps interleave instead of waiting on each other.
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      // t = z log2(e) in place, formed once: the label capture, the maximum
      // and the sum all use these values, so the maximum's own term below is
      // 2^0 = 1 exactly.
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < NBJ; ++j) acc.v[i][j][r] = fmaf(acc.v[i][j][r], LOG2E, cbl[j]);
      if (((i < 4 ? hit_lo : hit_hi) >> ((i & 3) * 16)) & 0xFFFFull) {   // rare, wave-uniform
        const uint32_t l16 = lane_x16();
        // rows wm*128 + i*16 + 4*(lane/16) + r of this tile, r = 0..3
        const uint32_t rb = (uint32_t)(i * 16) + ((l16 >> 8) << 2);
        GLOBAL_AS float* zrow = (GLOBAL_AS float*)uniform_ptr(zy2 + g0 + lrow0 + wm * 128);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int d = labs[rb + r] - cw;
          if ((unsigned)d < 64u && (uint32_t)(d & 15) == ((l16 >> 4) & 15)) {
            const int jj = d >> 4;
            zrow[rb + r] = jj == 0 ? acc.v[i][0][r] : jj == 1 ? acc.v[i][1][r] : jj == 2 ? acc.v[i][2][r] : acc.v[i][3][r];
          }
        }
      }
      // Stored p~ = exp(z - ref), ref the row's reference (its label logit)
      // when it has one, else the quarter maximum. When all of the wave's
      // 128 rows have a reference (all_ref), the partial sums are taken
      // against it too, (ref, sum 2^(t - ref)): no row maximum, no second
      // scale, and the stored values are the summed ones. If a sum exceeds
      // e^60 (some value may, or is infinite), or without all_ref, the
      // block takes (max, sum 2^(t - max)) and scales each stored value by
      // fr = exp(max - ref), capped at e^60; a valid row whose maximum lies
      // more than 60 above its reference raises the overflow flag (the group
      // is redone against r = lse).
      const LDS_AS float* refs = (const LDS_AS float*)s_ref + par * TILE + wm * 128 + i * 16 + 4 * (lane >> 4);   // this lane's 4 rows
      float mo[4], sm[4];                       // the partial: its shift and its sum, base 2
#pragma unroll
      for (int r = 0; r < 4; ++r) sm[r] = 0.f;
      bool ref_sums = all_ref;
      if (ref_sums) {
        float rf[4];                            // reference * log2(e)
#pragma unroll
        for (int r = 0; r < 4; ++r) rf[r] = refs[r] * LOG2E;
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
          float e[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            e[r] = __builtin_amdgcn_exp2f(acc.v[i][j][r] - rf[r]);
            sm[r] += e[r];
          }
          if (STORE_P)
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const uint32_t pk = f2bf2(e[r], e[r + 1]);
              pst[(4 * (lane >> 4) + r) * PST_LD + j * 16 + (lane & 15)] = (u16)pk;
              pst[(4 * (lane >> 4) + r + 1) * PST_LD + j * 16 + (lane & 15)] = (u16)(pk >> 16);
            }
        }
        sum16x4(sm);
        bool big = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mo[r] = rf[r];
          big |= !(sm[r] <= REF_SUM_CAP);
        }
        if (__ballot(big) != 0) {   // rare: the block's sums against its maxima instead (which raise the flag)
          ref_sums = false;
#pragma unroll
          for (int r = 0; r < 4; ++r) sm[r] = 0.f;
        }
      }
      if (!ref_sums) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          mo[r] = -INFINITY;
#pragma unroll
          for (int j = 0; j < NBJ; ++j) mo[r] = fmaxf(mo[r], acc.v[i][j][r]);
        }
        max16x4(mo);
        float ms[4], fr[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ms[r] = mo[r] == -INFINITY ? 0.f : mo[r];   // all columns past V: every e = 0
          fr[r] = 1.f;
        }
        if (use_ref) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float rr = refs[r];
            const float d = ms[r] - rr * LOG2E;        // NaN when the row has no reference
            overflow |= mo[r] != -INFINITY && d > REF_CAP2;
            fr[r] = __builtin_isnan(rr) ? 1.f : __builtin_amdgcn_exp2f(fminf(d, REF_CAP2));
          }
        }
#pragma unroll
        for (int j = 0; j < NBJ; ++j) {
          float e[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            e[r] = __builtin_amdgcn_exp2f(acc.v[i][j][r] - ms[r]);
            sm[r] += e[r];
          }
          if (STORE_P)
#pragma unroll
            for (int r = 0; r < 4; r += 2) {
              const uint32_t pk = f2bf2(e[r] * fr[r], e[r + 1] * fr[r + 1]);
              pst[(4 * (lane >> 4) + r) * PST_LD + j * 16 + (lane & 15)] = (u16)pk;
              pst[(4 * (lane >> 4) + r + 1) * PST_LD + j * 16 + (lane & 15)] = (u16)(pk >> 16);
            }
        }
        sum16x4(sm);
      }
      if ((lane & 15) == 0) {   // rows 4*(lane/16) .. +3 of the block, in base-2 units
        *(f32x4*)(pm + i * 16) = (f32x4){mo[0], mo[1], mo[2], mo[3]};
        *(f32x4*)(ps + i * 16) = (f32x4){sm[0], sm[1], sm[2], sm[3]};
      }
      if (STORE_P) {
        // The wave reads back its own staged block (LDS serves a wave's
        // accesses in order); 16 rows x 128 B, 8 lanes per row, streamed out.
        asm volatile("" ::: "memory");
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int id = k * 64 + lane, rr = id >> 3, ch = id & 7;
          const u32x4 val = *(const LDS_AS u32x4*)(pst + rr * PST_LD + ch * 8);
          __builtin_nontemporal_store(val, (u32x4*)(pq + (i * 16 + rr) * 64 + ch * 8));
        }
        asm volatile("" ::: "memory");
      }
    }
    if (overflow && ovf != nullptr) *ovf = 1;   // rare: the group is redone
    // First use of `claimed`, so the compiler's wait for the atomic lands
    // here. (The library is built with the atomic optimizer off: its
    // wave-wide rewrite of a uniform-address atomic reads the result at once.)
    asm volatile("" ::: "memory");
    if (more && tid == 0) s_next = per_step + claimed;
    par ^= 1;
    if (!more) break;
  }
}

// Label logit z_{i,y_i} = h_i . W_{y_i} + b_{y_i} (FP32 accumulation of the
// bf16 products) for every valid row; one wave per row, 16-byte loads.
__global__ void __launch_bounds__(256) k_label_logit(const u16* __restrict__ hidden, int64_t ldh,
                                                     const u16* __restrict__ weight, int64_t ldw,
                                                     const u16* __restrict__ bias, const int32_t* __restrict__ label32,
                                                     int64_t N, int64_t H, float* __restrict__ zlab) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= N) return;
  const int lab = label32[row];
  if (lab < 0) return;                     // wave-uniform
  const u16* hr = hidden + row * ldh;
  const u16* wr = weight + (int64_t)lab * ldw;
  float acc = 0.f;
  for (int64_t c = lane; c < H / 8; c += 64) {
    const u32x4 hv = *(const u32x4*)(hr + c * 8);
    const u32x4 wv = *(const u32x4*)(wr + c * 8);
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      acc += bf2f((u16)(hv[w] & 0xFFFF)) * bf2f((u16)(wv[w] & 0xFFFF));
      acc += bf2f((u16)(hv[w] >> 16)) * bf2f((u16)(wv[w] >> 16));
    }
  }
  acc = sum16(acc);
  acc += __shfl_xor(acc, 16, 64);
  acc += __shfl_xor(acc, 32, 64);
  if (lane == 0) zlab[row] = acc + (bias != nullptr ? bf2f(bias[lab]) : 0.f);
}

// Per row i in [row_begin, row_end): merge the quarter-tile base-2 (max,
// sumexp) partials into lse, form l_i from the row's label t_y (zy2), write
// lse (and l_i for reduction NONE), and add l_i into its chunk's float64 sum. Partials of row i sit at
// part[k * ld_part + (i - part_row0)], k < n_part. Rows in [N, row_end) only
// get lse_ws = 0. A block takes 64 rows; its 16 waves each merge every 16th
// partial of those rows (256-byte coalesced reads), then combine in LDS.
constexpr int FIN_ROWS = 64;
constexpr int FIN_WAVES = 16;

// (M, S) <- the merge of two base-2 partials (max t, sum 2^(t - max t)).
__device__ __forceinline__ void merge_ms(float& M, float& S, float mk, float sk) {
  if (mk == -INFINITY) return;
  const float mn = fmaxf(M, mk);
  S = S * __builtin_amdgcn_exp2f(M - mn) + sk * __builtin_amdgcn_exp2f(mk - mn);
  M = mn;
}

__global__ void __launch_bounds__(64 * FIN_WAVES) k_finalize_rows(
    const float* __restrict__ part_m, const float* __restrict__ part_s, int64_t ld_part, int64_t part_row0,
    int n_part, const float* __restrict__ zy2, const int32_t* __restrict__ label32, int64_t N,
    int64_t row_begin, int64_t row_end, int64_t chunk_rows, const int32_t* __restrict__ status, int reduction,
    float* __restrict__ lse_ws, float* __restrict__ lse_out, float* __restrict__ rowloss_out,
    double* __restrict__ chunk_acc, const unsigned long long* __restrict__ row_limit,
    const int32_t* __restrict__ perm) {
  __shared__ float s_m[FIN_WAVES][FIN_ROWS], s_s[FIN_WAVES][FIN_ROWS];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t i = row_begin + (int64_t)blockIdx.x * FIN_ROWS + lane;
  // rows at or past the device-side limit had no tiles (their partials are stale)
  const int64_t lim = row_limit != nullptr ? (int64_t)*row_limit : N;
  if (row_begin + (int64_t)blockIdx.x * FIN_ROWS >= lim) return;   // uniform: the whole block
  const bool live = i < row_end && i < N && i < lim;
  float M = -INFINITY, S = 0.f;
  if (live) {
    // four independent running (max, sum) pairs, so that four loads and four
    // merges are in flight per lane instead of one dependent chain
    const int64_t pi = i - part_row0;
    float Mc[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY}, Sc[4] = {0.f, 0.f, 0.f, 0.f};
    int k = wave;
#pragma unroll 2
    for (; k + 3 * FIN_WAVES < n_part; k += 4 * FIN_WAVES) {
      float mk[4], sk[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        mk[u] = part_m[(int64_t)(k + u * FIN_WAVES) * ld_part + pi];
        sk[u] = part_s[(int64_t)(k + u * FIN_WAVES) * ld_part + pi];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) merge_ms(Mc[u], Sc[u], mk[u], sk[u]);
    }
    for (; k < n_part; k += FIN_WAVES)
      merge_ms(Mc[0], Sc[0], part_m[(int64_t)k * ld_part + pi], part_s[(int64_t)k * ld_part + pi]);
#pragma unroll
    for (int u = 0; u < 4; ++u) merge_ms(M, S, Mc[u], Sc[u]);
  }
  s_m[wave][lane] = M;
  s_s[wave][lane] = S;
  __syncthreads();
  if (wave != 0 || i >= row_end) return;
  if (i >= N || i >= lim) {
    lse_ws[i] = 0.f;
    return;
  }
  for (int w = 1; w < FIN_WAVES; ++w) merge_ms(M, S, s_m[w][lane], s_s[w][lane]);
  // Against a row maximum M, S >= 1 (the maximum's own term is 2^0 = 1);
  // against a row reference M = r (its label logit from a separate dot
  // product), S holds the label's term 2^(t_y - r), ~1. Mathematically
  // l = lse - z_y >= 0; the clamp only takes off the rounding of r - t_y.
  const float L = __log2f(S);
  const float lse = LN2 * (M + L);
  const int lab = label32[i];
  const float l = lab >= 0 ? fmaxf(LN2 * ((M - zy2[i]) + L), 0.f) : 0.f;
  lse_ws[i] = lse;
  const int64_t oi = perm != nullptr ? (int64_t)perm[i] : i;   // the caller's row
  if (lse_out) lse_out[oi] = lse;
  if (reduction == 0 && rowloss_out) rowloss_out[oi] = (*status != 0) ? NAN : l;
  atomicAdd(&chunk_acc[oi / chunk_rows], (double)l);
}

// One block: total loss from the chunk sums (float64), MEAN scaling, NaN on a
// device-side label error; optional per-chunk output.
__global__ void __launch_bounds__(256) k_finalize_loss(const double* __restrict__ chunk_acc, int64_t T,
                                                       const unsigned long long* __restrict__ n_valid,
                                                       const int32_t* __restrict__ status, int reduction,
                                                       float* __restrict__ loss, float* __restrict__ chunk_out) {
  __shared__ double s_part[256];
  double acc = 0.0;
  for (int64_t k = threadIdx.x; k < T; k += 256) {
    const double c = chunk_acc[k];
    acc += c;
    if (chunk_out) chunk_out[k] = (float)c;
  }
  s_part[threadIdx.x] = acc;
  __syncthreads();
  for (int o = 128; o >= 1; o >>= 1) {
    if ((int)threadIdx.x < o) s_part[threadIdx.x] += s_part[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0 && reduction != 0) {
    double total = s_part[0];
    if (reduction == 2) {
      const unsigned long long nv = *n_valid;
      total /= (double)(nv > 0 ? nv : 1ull);
    }
    loss[0] = (*status != 0) ? NAN : (float)total;
  }
}

// out[c][r_out] = in[r0 + r_out][c] for r_out < R_valid (else 0), c < C,
// r_out < R_pad (C % 8 == 0, R_pad % 128 == 0, 16-byte aligned rows). One
// block moves a 128 x 128 tile: each thread loads 8 rows of one 16-byte
// column chunk (a quarter-wave reads 256 contiguous bytes of a row),
// transposes the 8 x 8 block in registers, and stages it through LDS as
// [column][row chunk] with the chunk slot XOR-swizzled by the column chunk
// (16 writing lanes, 16 distinct slots), so the
// output rows leave as 256-byte coalesced 16-byte stores.
constexpr int TT = 128;
__global__ void __launch_bounds__(256) k_transpose(const u16* __restrict__ in, int64_t ld_in, int64_t r0,
                                                   int64_t R_valid, int64_t C, u16* __restrict__ out,
                                                   int64_t R_pad, const float* __restrict__ rowc) {
  __shared__ __attribute__((aligned(16))) u16 t[TT * TT];
  const int64_t cb = (int64_t)blockIdx.x * TT, rb = (int64_t)blockIdx.y * TT;
  const int tid = threadIdx.x;
  const int cc = tid & 15, rk = tid >> 4;   // column chunk (8 columns), row block (8 rows)
  const int64_t c0 = cb + cc * 8;
  u32x4 v[8];
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int64_t row = rb + rk * 8 + r;
    v[r] = (row < R_valid && c0 < C) ? *(const u32x4*)(in + (r0 + row) * ld_in + c0) : (u32x4){0, 0, 0, 0};
  }
  if (rowc != nullptr) {     // out rows scaled by rowc[row] (bf16, round to nearest even)
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int64_t row = rb + rk * 8 + r;
      const float c = row < R_valid ? rowc[row] : 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = v[r][w];
        v[r][w] = (uint32_t)f2bf(c * bf2f((u16)(x & 0xFFFF))) | ((uint32_t)f2bf(c * bf2f((u16)(x >> 16))) << 16);
      }
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int col = cc * 8 + e;
    u32x4 o;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t lo = (v[2 * w][e >> 1] >> ((e & 1) * 16)) & 0xFFFF;
      const uint32_t hi = (v[2 * w + 1][e >> 1] >> ((e & 1) * 16)) & 0xFFFF;
      o[w] = lo | (hi << 16);
    }
    *(LDS_AS u32x4*)((LDS_AS u16*)t + col * TT + ((rk ^ ((col >> 3) & 15)) << 3)) = o;
  }
  __syncthreads();
  // 128 output rows (columns of `in`) x 16 sixteen-byte chunks; 16 lanes per
  // row, 8 per K-slab (out is [R_pad/64][C][64]).
#pragma unroll
  for (int it = 0; it < TT * TT / 8 / 256; ++it) {
    const int id = it * 256 + tid;
    const int col = id >> 4, ch = id & 15;
    const int64_t c = cb + col, r = rb + ch * 8;
    if (c < C && r < R_pad) {
      const u32x4 val = *(const LDS_AS u32x4*)((LDS_AS u16*)t + col * TT + ((ch ^ ((col >> 3) & 15)) << 3));
      *(u32x4*)(out + ((r >> 6) * C + c) * 64 + (r & 63)) = val;
    }
  }
}

// ---------------------------------------------------------------------------
// dlogits of a row group without a pass over it. The forward tiles store
// p~_ij = exp(z_ij - r_i) against one reference per row, r_i = z_{i,y_i} (the
// label logit), so that
//   G_ij = s valid_i (exp(z_ij - lse_i) - 1[j = y_i]) = c_i p~'_ij,
//   c_i = s valid_i exp(r_i - lse_i),   p~'_ij = p~_ij - 1[j = y_i] exp(lse_i - r_i).
// Only the label entry of each row changes (k_rowscale patches it, from the
// FP32 label logit and lse: exp(z_y - r) - exp(lse - r), no cancellation
// through bf16); c_i becomes a row scale of grad_hidden's output and of h^T
// in grad_weight, and grad_bias is a c-weighted column sum of p~'
// (inside grad_weight, or k_bias_sums when grad_weight is not computed). A valid row whose maximum lies more than 60 above its label
// logit would leave the range of the stored values: the forward tiles then
// set the overflow flag, and the group's p~ is recomputed against r_i =
// lse_i (k_prep_ref, k_fwd_tile and k_rowscale in their retry mode: every
// stored value is then at most 1).
// ---------------------------------------------------------------------------
// rref[i] = src[g0 + i] for valid rows (the label logit, or lse in the retry),
// NaN for ignored rows and rows past N (their tiles keep the quarter maximum).
// With only_if non-null the kernel does nothing unless *only_if != 0.
__global__ void __launch_bounds__(256) k_prep_ref(const int32_t* __restrict__ label32, const float* __restrict__ src,
                                                  int64_t g0, int64_t G, float* __restrict__ rref,
                                                  const int* __restrict__ only_if) {
  if (only_if != nullptr && *only_if == 0) return;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= G) return;
  rref[i] = label32[g0 + i] >= 0 ? src[g0 + i] : NAN;
}

// Row scales c_i of one group and the label entries of p~' (see above).
// retry = 0 runs unless the overflow flag is set, retry = 1 only if it is.
__global__ void __launch_bounds__(256) k_rowscale(const int32_t* __restrict__ label32, const float* __restrict__ zy2,
                                                  const float* __restrict__ lse_ws, const float* __restrict__ rref,
                                                  const float* __restrict__ row_scale,
                                                  const unsigned long long* __restrict__ n_valid, float grad_scale,
                                                  int is_mean, int64_t g0, int64_t G, u16* __restrict__ dlog,
                                                  float* __restrict__ rowc, const int* __restrict__ ovf, int retry,
                                                  float* __restrict__ gb_f32, const int32_t* __restrict__ perm) {
  if ((*ovf != 0) != (retry != 0)) return;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= G) return;
  const int64_t row = g0 + i;
  const int lab = label32[row];
  if (lab < 0) {                       // ignored rows and rows past N
    rowc[i] = 0.f;
    return;
  }
  float scale = grad_scale;
  if (is_mean) {
    const unsigned long long nv = *n_valid;
    scale = grad_scale / (float)(nv > 0 ? nv : 1ull);
  }
  const float r = rref[i], lse = lse_ws[row];
  const float c = scale * (row_scale != nullptr ? row_scale[perm != nullptr ? perm[row] : row] : 1.f) * expf(r - lse);
  const float pl = expf(zy2[row] * LN2 - r) - expf(lse - r);
  const u16 pb = f2bf(pl);
  rowc[i] = c;
  dlog[((int64_t)(lab >> 6) * G + i) * 64 + (lab & 63)] = pb;
  // grad_bias sums the stored (bf16) entries; the label entry's rounding is
  // added back here, so that its term is exact to FP32
  if (gb_f32 != nullptr) atomicAdd(gb_f32 + lab, c * (pl - bf2f(pb)));
}

// grad_bias += sum_i c_i p~'[i][v] over one group, for calls without
// grad_weight (which otherwise adds these sums): one workgroup per 64-id
// K-slab and 1024 rows (a contiguous 128 KB block of the slab), 8 ids x 32
// rows per thread, then 32 partial sums per id added through LDS.
constexpr int BS_ROWS = 1024;
__global__ void __launch_bounds__(256) k_bias_sums(const u16* __restrict__ dlog, const float* __restrict__ rowc,
                                                   int64_t G, int64_t V, float* __restrict__ gb_f32) {
  __shared__ float s_c[BS_ROWS];
  __shared__ float s_sum[32][64];
  const int tid = threadIdx.x;
  const int64_t slab = blockIdx.x, r0 = (int64_t)blockIdx.y * BS_ROWS;
  for (int k = tid; k < BS_ROWS; k += 256) s_c[k] = r0 + k < G ? rowc[r0 + k] : 0.f;
  __syncthreads();
  const int ch = tid & 7, rg = tid >> 3;       // 8 ids, one of 32 row lanes
  const u16* base = dlog + (slab * G + r0) * 64 + ch * 8;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
#pragma unroll 1
  for (int k = 0; k < BS_ROWS / 32; k += 8) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int64_t row = rg + 32 * (k + u);
      v[u] = r0 + row < G ? __builtin_nontemporal_load((const u32x4*)(base + row * 64)) : (u32x4){0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float c = s_c[rg + 32 * (k + u)];
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] = fmaf(c, bf2f((u16)((e & 1) ? (v[u][e >> 1] >> 16) : (v[u][e >> 1] & 0xFFFF))), acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) s_sum[rg][ch * 8 + e] = acc[e];
  __syncthreads();
  if (tid < 64) {
    float sum = 0.f;
#pragma unroll 8
    for (int k = 0; k < 32; ++k) sum += s_sum[k][tid];
    const int64_t col = slab * 64 + tid;
    if (col < V) atomicAdd(gb_f32 + col, sum);
  }
}

// How grad_hidden's tiles of one group are shared out, the same in every
// workgroup and in k_gh_reduce: the row tiles below the device-side row limit
// are real. When the real tiles do not fill whole rounds of the GPU, the
// rem tiles left over are each split along K into sp <= 32 pieces that
// together fill the last round (FP32 partial tiles, summed by k_gh_reduce); the row
// tiles past the limit only write zero rows.
// grad_hidden's K is the whole vocabulary (thousands of stages), so a
// small group's few tiles can be cut finer than grad_weight's.
constexpr int kMaxGhSplit = 32;
struct GhPlan {
  int nr;       // real row tiles
  int n_full;   // tiles computed whole
  int rem;      // tiles split along K (0: none)
  int sp;       // pieces per split tile
};
__device__ __forceinline__ GhPlan gh_plan(const unsigned long long* row_limit, int64_t g0, int n_mt, int n_nt,
                                          int nk, int cus, int max_items) {
  GhPlan p;
  int64_t lim = row_limit != nullptr ? (int64_t)*row_limit - g0 : (int64_t)n_mt * TILE;
  if (lim < 0) lim = 0;
  const int64_t nr = (lim + TILE - 1) / TILE;
  p.nr = nr < n_mt ? (int)nr : n_mt;
  const int real = p.nr * n_nt;
  p.rem = real % cus;
  p.sp = 1;
  if (p.rem != 0) {
    int sp = cus / p.rem;
    if (sp > kMaxGhSplit) sp = kMaxGhSplit;
    if (sp > nk / 4) sp = nk / 4;   // at least four 64-deep stages per piece
    if (sp * p.rem > max_items) sp = max_items / p.rem;
    if (sp >= 2) p.sp = sp;
  }
  if (p.sp == 1) p.rem = 0;
  p.n_full = real - p.rem;
  return p;
}

// grad_hidden rows of one group: row i = c_i (p~' W)_i over K = Vp, cast to
// bf16; p~' is stored as K-slabs [Vp/64][G][64], W^T as [Vp/64][H][64].
// Workgroup b (see GhPlan): b < n_full a whole tile, then the K pieces of the
// split tiles (partial tiles to part[item], [256][256] FP32), then the zero
// rows of the row tiles past the limit; the rest return at once.
__global__ void __launch_bounds__(NTHREADS, 1)
k_gemm_grad_hidden(const u16* __restrict__ dlog, const u16* __restrict__ wT, int64_t Vp, int64_t H,
                   int64_t N, int64_t g0, int64_t G, int n_mt, int n_nt, const float* __restrict__ rowc,
                   u16* __restrict__ grad_hidden, const unsigned long long* __restrict__ row_limit,
                   const int32_t* __restrict__ perm, float* __restrict__ part, int cus, int max_items) {
  __shared__ __attribute__((aligned(16))) char smem_raw[MAINLOOP_LDS];
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  const int nk = (int)(Vp / BK);
  const GhPlan pl = gh_plan(row_limit, g0, n_mt, n_nt, nk, cus, max_items);
  const int b = (int)blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 2, wn = wave & 3;
  int t, s0 = 0, s1 = nk, item = -1;
  if (b < pl.n_full) {
    t = b;
    if ((pl.n_full & 7) == 0) t = (b & 7) * (pl.n_full >> 3) + (b >> 3);
  } else if (b < pl.n_full + pl.rem * pl.sp) {
    item = b - pl.n_full;
    t = pl.n_full + item / pl.sp;
    const int piece = item % pl.sp;
    s0 = (int)((int64_t)nk * piece / pl.sp);
    s1 = (int)((int64_t)nk * (piece + 1) / pl.sp);
  } else {
    // rows without a label (whole row tiles past the limit): zero grad_hidden
    const int z = b - pl.n_full - pl.rem * pl.sp;
    if (z >= (n_mt - pl.nr) * n_nt) return;
    const int64_t lrow0 = (int64_t)(pl.nr + z / n_nt) * TILE, col0 = (int64_t)(z % n_nt) * TILE;
    const int64_t c0 = col0 + tid % 32 * 8;
    if (c0 < H)
      for (int r = tid / 32; r < TILE; r += NTHREADS / 32) {
        const int64_t row = g0 + lrow0 + r;
        if (row >= N) break;
        *(u32x4*)(grad_hidden + (int64_t)(perm != nullptr ? perm[row] : row) * H + c0) = (u32x4){0, 0, 0, 0};
      }
    return;
  }
  int tm, tn;
  tile_from_index(t, pl.nr, n_nt, tm, tn);
  const int64_t lrow0 = (int64_t)tm * TILE, col0 = (int64_t)tn * TILE;
  Acc acc;
  gemm_tile(acc, dlog + (int64_t)s0 * G * BK, BK, G * BK * 2, lrow0, G, wT + (int64_t)s0 * H * BK, BK, H * BK * 2,
            col0, H, (int64_t)(s1 - s0) * BK, smem);
  if (item >= 0) {   // a K piece: plain FP32 stores, summed and scaled by k_gh_reduce
    float* dst = part + (int64_t)item * TILE * TILE + wn * 64 + (lane & 15);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < NBJ; ++j) dst[acc_row(wm, i, r, lane) * TILE + j * 16] = acc.v[i][j][r];
    return;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t row = g0 + lrow0 + acc_row(wm, i, r, lane);
      if (row >= N) continue;
      const float c = rowc[lrow0 + acc_row(wm, i, r, lane)];
      const int64_t orow = perm != nullptr ? (int64_t)perm[row] : row;   // the caller's row
#pragma unroll
      for (int j = 0; j < NBJ; ++j) {
        const int64_t col = col0 + acc_col(wn, j, lane);
        if (col < H) grad_hidden[orow * H + col] = f2bf(c * acc.v[i][j][r]);
      }
    }
}

// grad_hidden rows of the split tiles: the sum of their K pieces in piece
// order, times the row scale, cast to bf16. One workgroup per row of one
// split tile (64 threads, four columns each); blockIdx.y past the plan's
// split tiles returns at once.
__global__ void __launch_bounds__(64) k_gh_reduce(const float* __restrict__ part, const float* __restrict__ rowc,
                                                  u16* __restrict__ grad_hidden, const int32_t* __restrict__ perm,
                                                  int64_t Vp, int64_t H, int64_t N, int64_t g0, int n_mt, int n_nt,
                                                  const unsigned long long* __restrict__ row_limit, int cus,
                                                  int max_items) {
  const GhPlan pl = gh_plan(row_limit, g0, n_mt, n_nt, (int)(Vp / BK), cus, max_items);
  const int lt = (int)blockIdx.y;
  if (lt >= pl.rem) return;
  int tm, tn;
  tile_from_index(pl.n_full + lt, pl.nr, n_nt, tm, tn);
  const int r = (int)blockIdx.x, c = (int)threadIdx.x * 4;
  const int64_t lrow = (int64_t)tm * TILE + r, row = g0 + lrow, col = (int64_t)tn * TILE + c;
  if (row >= N || col >= H) return;   // H % 64 == 0: all four columns in or out
  f32x4 sum = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < pl.sp; ++p) sum += *(const f32x4*)(part + ((int64_t)(lt * pl.sp + p) * TILE + r) * TILE + c);
  const float cs = rowc[lrow];
  *(u32x2*)(grad_hidden + (int64_t)(perm != nullptr ? perm[row] : row) * H + col) =
      (u32x2){f2bf2(cs * sum[0], cs * sum[1]), f2bf2(cs * sum[2], cs * sum[3])};
}

// gw rows of one tile (+)= the accumulators: base points at column
// (col0 + wn*64 + lane%16) of row 0; rows past V are skipped when CHECK. The
// read-modify-write goes two 16-row blocks at a time with all their reads
// issued before the adds and stores, so 32 reads per lane are in flight.
// For the last row group, base16 (the same column of the bf16 output, or
// null) also receives each final sum rounded to bf16, and keep32 = 0 skips
// writing the FP32 sum back (the accumulator is then only workspace).
template <bool CHECK>
__device__ __forceinline__ void gw_update(const Acc& acc, float* __restrict__ base, u16* __restrict__ base16,
                                          int keep32, int64_t row0, int64_t H, int64_t V, int wm, int lane,
                                          int first) {
  auto put = [&](int64_t v, int j, float x) {
    if (keep32) base[v * H + j * 16] = x;
    if (base16) base16[v * H + j * 16] = f2bf(x);
  };
  if (first) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t v = row0 + acc_row(wm, i, r, lane);
        if (CHECK && v >= V) continue;
#pragma unroll
        for (int j = 0; j < NBJ; ++j) put(v, j, acc.v[i][j][r]);
      }
    return;
  }
#pragma unroll
  for (int i0 = 0; i0 < NB; i0 += 2) {
    float old[2][4][NBJ];
#pragma unroll
    for (int di = 0; di < 2; ++di)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t v = row0 + acc_row(wm, i0 + di, r, lane);
        const float* src = base + (CHECK && v >= V ? 0 : v) * H;
#pragma unroll
        for (int j = 0; j < NBJ; ++j) old[di][r][j] = src[j * 16];
      }
#pragma unroll
    for (int di = 0; di < 2; ++di)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t v = row0 + acc_row(wm, i0 + di, r, lane);
        if (CHECK && v >= V) continue;
#pragma unroll
        for (int j = 0; j < NBJ; ++j) put(v, j, old[di][r][j] + acc.v[i0 + di][j][r]);
      }
  }
}

// grad_weight walks 2 vocabulary tiles across all hidden tiles at a time
// (a 2 x 16 window per XCD at H = 4096): measured 1% faster than 4 x 8 with
// its K-major operands (8 x 4: 3% slower, 16 x 2: 12% slower).
constexpr int GW_GROUP_M = 2;

// DMA offsets of the K-major layout: fill b of a wave covers rows
// k = 8 wave + 2b + lane/32, lane % 32 the 16-byte slot p, which holds m-chunk
// c = p ^ (2 tr_swz(k)).
__device__ __forceinline__ void tr_slot(int wave, int lane, int b, int& k, int& c) {
  k = wave * 8 + 2 * b + (lane >> 5);
  c = (lane & 31) ^ (2 * tr_swz(k));
}

// grad_weight FP32 accumulation for one group: gw[v][:] (+)= sum_i G[i][v] h[i][:]
// over the group's rows. G is read as it is stored, K-major for this
// product (K-slabs [Vp/64][slab_rows][64], transposing LDS reads); h comes as
// hT, the group's rows transposed into K-slabs [slab_rows/64][H][64] (zero
// past N), read like the other kernels' operands. (Reading h K-major too
// saved that transpose but made the loop 1.8% slower: two 8-byte reads per
// fragment instead of one 16-byte read.)
//
// The first n_full tiles (whole rounds of the GPU) are one workgroup each.
// The n_tiles - n_full left over would run as one thin last round, so each
// is split over `split` workgroups by K; those write FP32 partial tiles to
// part ([item][256][256]) and k_gw_reduce adds them in a fixed order.
template <int R>   // R > 0: also the grad_bias sums, R rows per wave and stage (FragATBias)
__global__ void __launch_bounds__(NTHREADS, 1)
k_gemm_grad_weight(const u16* __restrict__ G, int64_t slab_rows, const u16* __restrict__ hT, int nk, int64_t H,
                   int64_t V, int n_mt, int n_nt, int n_full, int split, int first, float* __restrict__ gw_f32,
                   float* __restrict__ part, u16* __restrict__ gw_bf16, int keep32, const float* __restrict__ rowc,
                   float* __restrict__ gb_f32, const unsigned long long* __restrict__ row_limit, int64_t g0) {
  __shared__ __attribute__((aligned(16))) char smem_raw[MAINLOOP_LDS];
  __shared__ __attribute__((aligned(16))) float s_c[R ? NTHREADS / 64 * 2 * 64 : 4];   // per wave, two stages
  LDS_AS char* smem = (LDS_AS char*)smem_raw;
  int tm, tn, s0 = 0, s1 = nk, item = -1;
  if ((int)blockIdx.x < n_full) {
    int t = blockIdx.x;
    if ((n_full & 7) == 0) t = (t & 7) * (n_full >> 3) + (t >> 3);
    tile_from_index<GW_GROUP_M>(t, n_mt, n_nt, tm, tn);
  } else {
    item = (int)blockIdx.x - n_full;
    const int sp = item % split;
    tile_from_index<GW_GROUP_M>(n_full + item / split, n_mt, n_nt, tm, tn);
    s0 = (int)((int64_t)nk * sp / split);
    s1 = (int)((int64_t)nk * (sp + 1) / split);
  }
  if (row_limit != nullptr) {   // K stages past the device-side row limit hold only rows without a label
    const int64_t lim = (int64_t)*row_limit - g0;
    const int nk_lim = lim <= 0 ? 0 : (int)((lim + 63) / 64);
    if (s1 > nk_lim) s1 = nk_lim;
    if (s0 > s1) s0 = s1;
  }
  const int64_t row0 = (int64_t)tm * TILE, col0 = (int64_t)tn * TILE;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  TileLoads t;
#pragma unroll
  for (int b = 0; b < FILLS; ++b) {
    int k, c;
    tr_slot(wave, lane, b, k, c);
    t.ox.off[b] = (uint32_t)((((int64_t)(c >> 3) * slab_rows + k) * 64 + (c & 7) * 8) * 2);
  }
  t.oy = stage_offsets(BK, col0, H, wave, lane);
  // stages s0 .. s1-1 of the K loop (all of them for a whole tile)
  t.xbase = uniform_ptr(G + (row0 >> 6) * slab_rows * 64 + (int64_t)s0 * 64 * 64);
  t.ybase = uniform_ptr(hT + ((int64_t)s0 * H + col0) * 64);
  t.kx = 64 * 64 * 2;
  t.ky = H * BK * 2;
  t.lds_wave = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem + (uint32_t)wave * 32 * 128);
  Acc acc;
  if (s1 == s0) {   // nothing below the row limit: the tile adds zero
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NBJ; ++j) acc.v[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  } else if constexpr (R > 0) {
    FragATBias<R> fs(wave, lane, rowc + (int64_t)s0 * 64,
                     (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS char*)s_c) +
                         (uint32_t)wave * 2 * 256,
                     tn, n_nt);
    // the row scales of stages 0 and 1 go out before the operand loads, so
    // tile_run's first wait covers them
    for (int sb = 0; sb < 2 && sb < s1 - s0; ++sb) fs.load_c(sb);
    tile_prologue<FragATBias<R>>(t, s1 - s0);
    tile_run(acc, t, s1 - s0, smem, fs);
    if (tn < 64) {      // some wave summed a row: add the tile's 256 column sums
      constexpr int L = FragATBias<R>::L, RPR = FragATBias<R>::RPR;
      __syncthreads();  // every wave is past its last read of the stage buffers
      // wave w, lane = g 128 / L + cl: columns 128 (w%2) + cl L + e of its rows of group g
      LDS_AS float* red = (LDS_AS float*)smem;
#pragma unroll
      for (int e = 0; e < L; ++e) red[wave * 128 * RPR + lane * L + e] = R > 1 || fs.ok[0] ? fs.gb[e] : 0.f;
      __syncthreads();
      if (tid < TILE) {   // column tid: waves 2 j + tid / 128 (j = 0..3), their groups g
        float sum = 0.f;
#pragma unroll
        for (int j = 0; j < NTHREADS / 128; ++j)
#pragma unroll
          for (int g = 0; g < RPR; ++g) sum += red[(2 * j + (tid >> 7)) * 128 * RPR + g * 128 + (tid & 127)];
        if (row0 + tid < V) atomicAdd(gb_f32 + row0 + tid, sum);
      }
    }
  } else {
    FragAT fs(wave, lane);
    tile_prologue<FragAT>(t, s1 - s0);
    tile_run(acc, t, s1 - s0, smem, fs);
  }
  if (item >= 0) {   // partial tile of a split item: plain stores, summed by k_gw_reduce
    float* dst = part + (int64_t)item * TILE * TILE + wn * 64 + (lane & 15);
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int j = 0; j < NBJ; ++j) dst[acc_row(wm, i, r, lane) * TILE + j * 16] = acc.v[i][j][r];
    return;
  }
  // H % 64 == 0: a wave's 64 columns are all below H or all past it; only
  // the last vocabulary tile has rows past V.
  if (col0 + wn * 64 < H) {
    float* base = gw_f32 + col0 + wn * 64 + (lane & 15);
    u16* base16 = gw_bf16 ? gw_bf16 + col0 + wn * 64 + (lane & 15) : nullptr;
    if (row0 + TILE <= V) gw_update<false>(acc, base, base16, keep32, row0, H, V, wm, lane, first);
    else gw_update<true>(acc, base, base16, keep32, row0, H, V, wm, lane, first);
  }
}

// gw (+)= the sum, in split order, of the partial tiles of the split items:
// item e = tile n_full + e / split, part index e % split. One workgroup per
// 256 x 4 strip of one tile (64 threads, one float4 each).
__global__ void __launch_bounds__(64) k_gw_reduce(const float* __restrict__ part, int n_full, int split, int n_mt,
                                                  int n_nt, int64_t H, int64_t V, int first,
                                                  float* __restrict__ gw_f32, u16* __restrict__ gw_bf16,
                                                  int keep32) {
  const int tile = blockIdx.y;
  int tm, tn;
  tile_from_index<GW_GROUP_M>(n_full + tile, n_mt, n_nt, tm, tn);
  const int r = blockIdx.x;                       // row of the tile
  const int c = threadIdx.x * 4;                  // first of four columns
  const int64_t v = (int64_t)tm * TILE + r, col = (int64_t)tn * TILE + c;
  if (v >= V || col >= H) return;                 // H % 64 == 0: all four in or out
  f32x4 sum = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int sp = 0; sp < split; ++sp)
    sum += *(const f32x4*)(part + ((int64_t)tile * split + sp) * TILE * TILE + r * TILE + c);
  f32x4* dst = (f32x4*)(gw_f32 + v * H + col);
  const f32x4 out = first ? sum : *dst + sum;
  if (keep32) *dst = out;
  if (gw_bf16) {
    u16* d16 = gw_bf16 + v * H + col;
#pragma unroll
    for (int e = 0; e < 4; ++e) d16[e] = f2bf(out[e]);
  }
}

// data[k] *= *scale (the scale read from device memory).
__global__ void k_scale_bf16(u16* __restrict__ data, int64_t n, const float* __restrict__ scale) {
  const float sc = *scale;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t st = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += st) data[i] = f2bf(bf2f(data[i]) * sc);
}
__global__ void k_scale_f32(float* __restrict__ data, int64_t n, const float* __restrict__ scale) {
  const float sc = *scale;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t st = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += st) data[i] *= sc;
}

__global__ void k_cast_bf16(const float* __restrict__ in, u16* __restrict__ out, int64_t n) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t s = (int64_t)gridDim.x * blockDim.x;
  for (; i < n; i += s) out[i] = f2bf(in[i]);
}

// ---------------------------------------------------------------------------
// Launchers (host side). Each returns the launch's hipError_t.
// ---------------------------------------------------------------------------
static int grid_1d(int64_t n, int per_block = 256, int cap = 65536) {
  int64_t b = (n + per_block - 1) / per_block;
  if (b < 1) b = 1;
  return (int)(b < cap ? b : cap);
}

hipError_t launch_zero(void* p, int64_t bytes, hipStream_t st) {
  if (bytes <= 0) return hipSuccess;
  const int64_t words = (bytes + 3) / 4;
  hipLaunchKernelGGL(k_zero, dim3(grid_1d(words, 256, 4096)), dim3(256), 0, st, (uint32_t*)p, words);
  return hipGetLastError();
}

hipError_t launch_prepare_labels(const int64_t* labels, int64_t N, int64_t Np, int64_t V, int64_t ignore,
                                 int32_t* label32, unsigned long long* n_valid, int32_t* status,
                                 int32_t* block_cnt, hipStream_t st) {
  hipLaunchKernelGGL(k_prepare_labels, dim3((unsigned)(Np / 256)), dim3(256), 0, st, labels, N, V, ignore,
                     label32, n_valid, status, block_cnt);
  return hipGetLastError();
}

hipError_t launch_partition_rows(const int32_t* label32, const int32_t* block_cnt, int32_t* block_off,
                                 const unsigned long long* n_valid, int64_t Np, int32_t* perm, int32_t* labp,
                                 hipStream_t st) {
  const int64_t nb = Np / 256;
  hipLaunchKernelGGL(k_scan_blocks, dim3(1), dim3(1024), 0, st, block_cnt, nb, block_off);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_partition_rows, dim3((unsigned)nb), dim3(256), 0, st, label32, block_off, n_valid, Np, perm,
                     labp);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void* in, int64_t ld_in, const int32_t* perm, int64_t N, int64_t H, void* out,
                              hipStream_t st) {
  if (N <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_gather_rows, dim3(grid_1d(N * (H / 8), 256, 16384)), dim3(256), 0, st, (const u16*)in, ld_in,
                     perm, N, H, (u16*)out);
  return hipGetLastError();
}

// Compute units of the current device (cached per device).
int device_cus() {
  static int cu_count[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (cu_count[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 8) n = 8;
    cu_count[dev] = n;
  }
  return cu_count[dev];
}

// Grid of a persistent tile kernel: one workgroup per CU (the kernels' LDS
// admits no second one), a multiple of 8 so that blockIdx % 8 names the XCD,
// and no more than the tiles need.
static int persistent_grid(int64_t ntiles) {
  const int cus = device_cus();
  const int64_t per_xcd = (ntiles + 7) / 8;
  const int64_t nx = cus / 8 < per_xcd ? cus / 8 : per_xcd;
  return (int)(8 * nx);
}

hipError_t launch_fwd_tiles(const Shapes& s, const void* hidden, const void* weight, const void* bias, int64_t g0,
                            int64_t rows, float* part_m, float* part_s, void* p_out, int* tile_ctr,
                            const float* rref, int* ovf, const int* only_if, const int32_t* label32, float* zy2,
                            const unsigned long long* row_limit, hipStream_t st) {
  const int n_mt = (int)(rows / TILE), n_vt = (int)(s.Vp / TILE);
  const int nb = persistent_grid((int64_t)n_mt * n_vt);
  if (nb == 0) return hipSuccess;
  hipError_t e = launch_zero(tile_ctr, 8 * sizeof(int), st);
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)nb), block(NTHREADS);
  if (p_out)
    hipLaunchKernelGGL(k_fwd_tile<true>, grid, block, 0, st, (const u16*)hidden, s.ldh, (const u16*)weight, s.ldw,
                       (const u16*)bias, s.N, s.V, s.H, g0, rows, n_mt, n_vt, part_m, part_s, (u16*)p_out, tile_ctr,
                       rref, ovf, only_if, label32, zy2, row_limit);
  else
    hipLaunchKernelGGL(k_fwd_tile<false>, grid, block, 0, st, (const u16*)hidden, s.ldh, (const u16*)weight,
                       s.ldw, (const u16*)bias, s.N, s.V, s.H, g0, rows, n_mt, n_vt, part_m, part_s, (u16*)nullptr,
                       tile_ctr, (const float*)nullptr, (int*)nullptr, only_if, label32, zy2, row_limit);
  return hipGetLastError();
}

hipError_t launch_label_logit(const Shapes& s, const void* hidden, const void* weight, const void* bias,
                              const int32_t* label32, float* zlab, hipStream_t st) {
  if (s.N <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_label_logit, dim3((unsigned)((s.N + 3) / 4)), dim3(256), 0, st, (const u16*)hidden, s.ldh,
                     (const u16*)weight, s.ldw, (const u16*)bias, label32, s.N, s.H, zlab);
  return hipGetLastError();
}

hipError_t launch_finalize_rows(const Shapes& s, const float* part_m, const float* part_s, int64_t g0,
                                int64_t rows, const float* zy2, const int32_t* label32, const int32_t* status,
                                int reduction, float* lse_ws, float* lse_out, float* rowloss_out,
                                double* chunk_acc, const unsigned long long* row_limit, const int32_t* perm,
                                hipStream_t st) {
  hipLaunchKernelGGL(k_finalize_rows, dim3((unsigned)(rows / FIN_ROWS)), dim3(64 * FIN_WAVES), 0, st, part_m, part_s, rows, g0,
                     (int)(NQ * (s.Vp / TILE)), zy2, label32, s.N, g0, g0 + rows, s.chunk_rows, status, reduction,
                     lse_ws, lse_out, rowloss_out, chunk_acc, row_limit, perm);
  return hipGetLastError();
}

hipError_t launch_finalize_loss(const double* chunk_acc, int64_t T, const unsigned long long* n_valid,
                                const int32_t* status, int reduction, float* loss, float* chunk_out,
                                hipStream_t st) {
  hipLaunchKernelGGL(k_finalize_loss, dim3(1), dim3(256), 0, st, chunk_acc, T, n_valid, status, reduction,
                     loss, chunk_out);
  return hipGetLastError();
}

hipError_t launch_transpose(const void* in, int64_t ld_in, int64_t r0, int64_t R_valid, int64_t C, void* out,
                            int64_t R_pad, const float* rowc, hipStream_t st) {
  dim3 grid((unsigned)((C + TT - 1) / TT), (unsigned)((R_pad + TT - 1) / TT));
  hipLaunchKernelGGL(k_transpose, grid, dim3(256), 0, st, (const u16*)in, ld_in, r0, R_valid, C, (u16*)out,
                     R_pad, rowc);
  return hipGetLastError();
}

hipError_t launch_prep_ref(const int32_t* label32, const float* src, int64_t g0, int64_t G, float* rref,
                           const int* only_if, hipStream_t st) {
  hipLaunchKernelGGL(k_prep_ref, dim3((unsigned)((G + 255) / 256)), dim3(256), 0, st, label32, src, g0, G, rref,
                     only_if);
  return hipGetLastError();
}

hipError_t launch_rowscale(const int32_t* label32, const float* zy2, const float* lse_ws, const float* rref,
                           const float* row_scale, const unsigned long long* n_valid, float grad_scale, int is_mean,
                           int64_t g0, int64_t G, void* dlog, float* rowc, const int* ovf, int retry,
                           float* gb_f32, const int32_t* perm, hipStream_t st) {
  hipLaunchKernelGGL(k_rowscale, dim3((unsigned)((G + 255) / 256)), dim3(256), 0, st, label32, zy2, lse_ws, rref,
                     row_scale, n_valid, grad_scale, is_mean, g0, G, (u16*)dlog, rowc, ovf, retry, gb_f32, perm);
  return hipGetLastError();
}

hipError_t launch_bias_sums(const Shapes& s, const void* dlog, const float* rowc, int64_t G, float* gb_f32,
                            hipStream_t st) {
  const dim3 grid((unsigned)(s.Vp / 64), (unsigned)((G + BS_ROWS - 1) / BS_ROWS));
  hipLaunchKernelGGL(k_bias_sums, grid, dim3(256), 0, st, (const u16*)dlog, rowc, G, s.V, gb_f32);
  return hipGetLastError();
}

hipError_t launch_grad_hidden(const Shapes& s, const void* dlog, const void* wT, int64_t g0, int64_t G,
                              const float* rowc, void* grad_hidden, const unsigned long long* row_limit,
                              const int32_t* perm, float* part, int64_t part_items, hipStream_t st) {
  const int n_mt = (int)(G / TILE), n_nt = (int)((s.H + TILE - 1) / TILE);
  const int cus = device_cus();
  const int max_items = (int)(part_items < kMaxGwItems ? part_items : kMaxGwItems);
  // whole tiles, K pieces and zero-row tiles need at most rem * (sp - 1) < min(cus, max_items)
  // workgroups beyond one per tile
  const int extra = max_items >= 2 ? (cus < max_items ? cus : max_items) : 0;
  hipLaunchKernelGGL(k_gemm_grad_hidden, dim3((unsigned)(n_mt * n_nt + extra)), dim3(NTHREADS), 0, st,
                     (const u16*)dlog, (const u16*)wT, s.Vp, s.H, s.N, g0, G, n_mt, n_nt, rowc, (u16*)grad_hidden,
                     row_limit, perm, part, cus, max_items);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || max_items < 2) return e;
  // at most max_items / 2 split tiles (sp >= 2), and never more than there are tiles
  int max_rem = max_items / 2;
  if (max_rem > n_mt * n_nt) max_rem = n_mt * n_nt;
  hipLaunchKernelGGL(k_gh_reduce, dim3(TILE, (unsigned)max_rem), dim3(64), 0, st, part, rowc, (u16*)grad_hidden,
                     perm, s.Vp, s.H, s.N, g0, n_mt, n_nt, row_limit, cus, max_items);
  return hipGetLastError();
}

hipError_t launch_grad_weight(const Shapes& s, const void* dlog, int64_t G, const void* hT, int64_t rows_valid,
                              float* part, int64_t part_items, int first, float* gw_f32, void* gw_bf16, int keep32,
                              const float* rowc, float* gb_f32, const unsigned long long* row_limit, int64_t g0,
                              hipStream_t st) {
  const int n_mt = (int)(s.Vp / TILE), n_nt = (int)((s.H + TILE - 1) / TILE);
  const int nk = (int)((rows_valid + 63) / 64);
  const int n_tiles = n_mt * n_nt;
  int n_full = n_tiles, split = 1;
  grad_weight_split(n_tiles, nk, device_cus(), (int)part_items, &n_full, &split);
  const dim3 grid((unsigned)(n_full + (n_tiles - n_full) * split)), block(NTHREADS);
#define LCE_GW_LAUNCH(R_, RC, GB)                                                                              \
  hipLaunchKernelGGL(k_gemm_grad_weight<R_>, grid, block, 0, st, (const u16*)dlog, G, (const u16*)hT, nk, s.H, s.V, \
                     n_mt, n_nt, n_full, split, first, gw_f32, part, (u16*)gw_bf16, keep32, RC, GB, row_limit, g0)
  switch (gb_f32 == nullptr ? 0 : grad_weight_bias_rows(s.H)) {
    case 0: LCE_GW_LAUNCH(0, (const float*)nullptr, (float*)nullptr); break;
    case 1: LCE_GW_LAUNCH(1, rowc, gb_f32); break;
    case 2: LCE_GW_LAUNCH(2, rowc, gb_f32); break;
    case 4: LCE_GW_LAUNCH(4, rowc, gb_f32); break;
    case 8: LCE_GW_LAUNCH(8, rowc, gb_f32); break;
    default: LCE_GW_LAUNCH(16, rowc, gb_f32); break;
  }
#undef LCE_GW_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_full == n_tiles) return e;
  hipLaunchKernelGGL(k_gw_reduce, dim3(TILE, (unsigned)(n_tiles - n_full)), dim3(64), 0, st, part, n_full, split,
                     n_mt, n_nt, s.H, s.V, first, gw_f32, (u16*)gw_bf16, keep32);
  return hipGetLastError();
}

int grad_weight_bias_rows(int64_t H) {
  const int64_t n_nt = (H + TILE - 1) / TILE;
  int r = 1;
  while (r * n_nt < 16) r *= 2;   // 4 waves x r rows x n_nt tiles cover the 64 rows of a stage
  return r;
}

void grad_weight_split(int n_tiles, int nk, int cus, int max_items, int* n_full, int* split) {
  const int rem = n_tiles % cus;
  *n_full = n_tiles;
  *split = 1;
  if (rem == 0) return;
  int sp = cus / rem;
  if (sp > kMaxGwSplit) sp = kMaxGwSplit;
  if (sp > nk / 4) sp = nk / 4;
  if (max_items > kMaxGwItems) max_items = kMaxGwItems;
  if (sp * rem > max_items) sp = max_items / rem;
  if (sp < 2) return;
  *n_full = n_tiles - rem;
  *split = sp;
}

hipError_t launch_scale(void* data, bool f32, int64_t n, const float* scale, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (f32)
    hipLaunchKernelGGL(k_scale_f32, dim3(grid_1d(n, 256, 16384)), dim3(256), 0, st, (float*)data, n, scale);
  else
    hipLaunchKernelGGL(k_scale_bf16, dim3(grid_1d(n, 256, 16384)), dim3(256), 0, st, (u16*)data, n, scale);
  return hipGetLastError();
}

hipError_t launch_cast(const float* in, void* out, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_cast_bf16, dim3(grid_1d(n, 256, 16384)), dim3(256), 0, st, in, (u16*)out, n);
  return hipGetLastError();
}

}  // namespace lce
