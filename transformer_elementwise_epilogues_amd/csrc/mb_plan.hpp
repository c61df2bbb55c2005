// mb_plan.hpp -- launch planning: the launch shape of every kernel family,
// as plain host arithmetic (no HIP call), shared by the C ABI (mb_abi.cpp),
// the kernels (compile-time shapes) and a CPU test of the plans.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mb {

// Block counts below are tuned on a whole MI355X (256 compute units); a plan
// scales them by the compute units of the device it runs on (a partitioned
// device has fewer), so that the persistent grids keep the same number of
// resident blocks per CU instead of running in several rounds.
constexpr int kTunedCUs = 256;

// Row tiling of a [T, nvec] array of 16-byte column vectors: grid.x covers
// column strips of 64 vectors (one wave each), grid.y = G row groups; wave w
// of row group y walks rows y*4 + w, y*4 + w + 4G, ...
struct Tiling {
  int64_t T = 0;     // rows
  int nvec = 0;      // 16-byte vectors per (output) row
  int strips = 0;    // ceil(nvec / 64)
  int G = 0;         // row groups
};

// Launch shape per kernel family: blocks of 256 threads to aim for (row groups
// are rounded down so the grid never exceeds it by a partial wave of blocks)
// and rows in flight per wave, measured on MI355X (bench-order sweeps). The
// forward kernels without reductions stream best as many short-lived blocks
// (one to four rows per wave). Of the backward kernels that keep bias-gradient
// sums per lane, the GeLU pair also runs many blocks (8 rows per wave, 4 in
// flight): the dispatcher's balancing beat a persistent grid of one block per
// CU by 3-4 % and removed its slow calls, although the partial rows grow to
// 1/16 of dgrad's bytes. The others do best with few resident blocks.
#ifndef MB_GELU_FWD_BLOCKS
#define MB_GELU_FWD_BLOCKS 65536
#endif
#ifndef MB_GELU_FWD_UNROLL
#define MB_GELU_FWD_UNROLL 1
#endif
#ifndef MB_GELU_BWD_BLOCKS
#define MB_GELU_BWD_BLOCKS 32768
#endif
#ifndef MB_GELU_BWD_UNROLL
#define MB_GELU_BWD_UNROLL 4
#endif
// rows every wave of the GeLU backward walks at least: its partial rows (one
// per row group) then stay a small fraction of the bytes at any row count.
// With one row per wave, [4096, 8192] bf16 wrote 1024 partial rows (a sixth of
// its bytes) and ran at 2.75 TB/s; 4 rows per wave took it to 4.4 TB/s and
// [8192, 8192], [32768, 4096], [2048, 14336], [1024, 32768] from 2.7-3.8 to
// 4.2-5.3 TB/s, with [16384, 32768] unchanged (8 rows per wave already; MI355X,
// same process).
#ifndef MB_GELU_BWD_MIN_ROWS
#define MB_GELU_BWD_MIN_ROWS 4
#endif
#ifndef MB_GELU_ERF_BWD_MIN_ROWS
#define MB_GELU_ERF_BWD_MIN_ROWS 4
#endif
#ifndef MB_GELU_ERF_BWD_BLOCKS
#define MB_GELU_ERF_BWD_BLOCKS 32768
#endif
#ifndef MB_GELU_ERF_BWD_UNROLL
#define MB_GELU_ERF_BWD_UNROLL 4
#endif
#ifndef MB_BDA_BLOCKS
#define MB_BDA_BLOCKS 65536
#endif
#ifndef MB_BDA_UNROLL
#define MB_BDA_UNROLL 1
#endif
#ifndef MB_BDA_MIXED_BLOCKS
#define MB_BDA_MIXED_BLOCKS 512
#endif
#ifndef MB_BDA_MIXED_UNROLL
#define MB_BDA_MIXED_UNROLL 2
#endif
// its training pass (with the mask) streams best as many blocks (+4 % over
// 512 with buffer nt sc1 stores); the in-place inference pass does not
#ifndef MB_BDA_MIXED_TRAIN_BLOCKS
#define MB_BDA_MIXED_TRAIN_BLOCKS 16384
#endif
#ifndef MB_BDA_MIXED_TRAIN_UNROLL
#define MB_BDA_MIXED_TRAIN_UNROLL 1
#endif
#ifndef MB_BDA_BWD_BLOCKS
#define MB_BDA_BWD_BLOCKS 768
#endif
#ifndef MB_BDA_BWD_UNROLL
#define MB_BDA_BWD_UNROLL 2
#endif
// fp32 residual gradient beside bf16/fp16: the grid that splits the rows
// evenly over the waves (64 rows each at [8192, 4096]) beat 768 blocks by 5 %
#ifndef MB_BDA_BWD_MIXED_BLOCKS
#define MB_BDA_BWD_MIXED_BLOCKS 512
#endif
#ifndef MB_BDA_BWD_MIXED_UNROLL
#define MB_BDA_BWD_MIXED_UNROLL 2
#endif
// Without the bias gradient nothing is summed over rows, so the backward
// streams as many short-lived blocks, either residual dtype: 32768 blocks of
// one row per wave took [16384, 8192] from 93.2 to 86.8 us and the
// fp32-residual [8192, 4096] from 51.3 to 48.4 us against the persistent
// grid (MI355X, same process; 16384 or 65536 blocks, or 4096 of two rows,
// were up to 10 % slower on one of the two)
#ifndef MB_BDA_BWD_NODBIAS_BLOCKS
#define MB_BDA_BWD_NODBIAS_BLOCKS 32768
#endif
#ifndef MB_BDA_BWD_NODBIAS_UNROLL
#define MB_BDA_BWD_NODBIAS_UNROLL 1
#endif
#ifndef MB_GLU_FWD_BLOCKS
#define MB_GLU_FWD_BLOCKS 65536
#endif
#ifndef MB_GLU_FWD_UNROLL
#define MB_GLU_FWD_UNROLL 1
#endif
#ifndef MB_GLU_BWD_BLOCKS
#define MB_GLU_BWD_BLOCKS 512
#endif
#ifndef MB_GLU_BWD_UNROLL
#define MB_GLU_BWD_UNROLL 1
#endif
// Without the bias gradient (bias-free layers) the gated backward streams as
// many short-lived blocks, like the forward: 65536 blocks took the SwiGLU,
// weighted SwiGLU (with dweights) and GEGLU backward at [8192, 14336] from
// 185.0 / 201.7 / 185.1 to 174.3 / 182.0 / 176.6 us and at [16384, 8192] from
// 203.0 / 223.9 / 201.9 to 200.0 / 201.3 / 197.1 us against 512 blocks
// (MI355X, same process; 4096 or 16384 blocks were slower than both)
#ifndef MB_GLU_BWD_NODBIAS_BLOCKS
#define MB_GLU_BWD_NODBIAS_BLOCKS 65536
#endif

#ifndef MB_SRELU_FWD_BLOCKS
#define MB_SRELU_FWD_BLOCKS 65536
#endif
#ifndef MB_SRELU_FWD_UNROLL
#define MB_SRELU_FWD_UNROLL 1
#endif
#ifndef MB_SRELU_BWD_BLOCKS
#define MB_SRELU_BWD_BLOCKS 16384
#endif
#ifndef MB_SRELU_BWD_UNROLL
#define MB_SRELU_BWD_UNROLL 1
#endif
#ifndef MB_LN_FWD_BLOCKS
#define MB_LN_FWD_BLOCKS 2048
#endif
// backward blocks = partial rows of dgamma / dbeta: fewer for wide rows
// (1024 or more vectors), where each partial row is large
#ifndef MB_LN_BWD_BLOCKS
#define MB_LN_BWD_BLOCKS 512
#endif
#ifndef MB_LN_BWD_BLOCKS_WIDE
#define MB_LN_BWD_BLOCKS_WIDE 256
#endif
// preferred vectors per thread (the row is split over more threads below it)
#ifndef MB_LN_FWD_NV
#define MB_LN_FWD_NV 4
#endif
// forward rows of 4096 vectors: 512 threads of 8 (two blocks per CU) instead
// of 1024 threads of 4 (one)
#ifndef MB_LN_FWD_WIDE_HALF
#define MB_LN_FWD_WIDE_HALF 1
#endif
#ifndef MB_LN_BWD_NV
#define MB_LN_BWD_NV 2
#endif


// Blocks to aim for on a device of `cus` compute units (at least 1).
int scaled_blocks(int target_blocks, int cus);

// The tiling of one call (it also sizes the workspaces): target_blocks as
// tuned for kTunedCUs, scaled to `cus`; G rounded down so that the grid never
// exceeds the scaled target, at most ceil(T / 4) (every row group owns a row),
// at most ceil(T / (4 min_rows)) so that every wave walks at least min_rows
// rows (fewer partial rows for the reductions), and at most 65535.
Tiling plan_tiling(int64_t T, int nvec, int target_blocks, int cus, int min_rows = 1);

// Floats of chunk sums launch_colsum_tall needs for R partial rows of C
// columns (none up to 32 rows).
int64_t colsum_tall_tmp_floats(int R, int64_t C);

// Elements a dropout-add lane handles: 8 bf16/fp16 values, or 4 when the
// residual (and so its gradient) is fp32 beside them, or 4 fp32 values. The
// tiling's vectors per row are hidden / this. (dt: 0 fp32, 1 fp16, 2 bf16)
int bda_elems_per_lane(int dt, int res_dt);

// ---- residual add + LayerNorm row kernels
// Row-group shapes: (threads per row, vectors per thread, rows per block).
// Groups of 64 threads run 4 rows per block (no barrier); wider groups are the
// whole block.
struct LnShape {
  int tpr, nv, rpb;
};
constexpr LnShape kLnShapes[] = {{64, 1, 4},  {64, 2, 4},  {64, 4, 4},  {256, 1, 1},  {256, 2, 1},
                                 {256, 4, 1}, {512, 1, 1}, {512, 2, 1}, {512, 4, 1},  {1024, 1, 1},
                                 {1024, 2, 1}, {1024, 4, 1}, {1024, 8, 1}, {512, 8, 1}, {512, 16, 1}};
constexpr int kLnNumShapes = sizeof(kLnShapes) / sizeof(kLnShapes[0]);
struct LnPlan {
  int nvec = 0;           // vectors of ln_elems_per_vector elements per row
  int shape = -1;         // row-group shape; -1: the row is too wide
  int grid = 0;           // blocks of the row kernels
  int partial_rows = 0;   // partial rows the backward writes (one per block)
  int cus = 0;            // compute units of the device planned for
};
int ln_elems_per_vector(int dt, int rdt);
LnPlan plan_ln(int64_t T, int64_t H, int dt, int rdt, int target_blocks, int nv_pref, int cus);

// ---- backward of wide LayerNorm rows (more than MB_LN2_ROW_VEC vectors,
// too wide to keep the parameter-gradient sums beside a register-resident
// row): a row-sum kernel (one block per row), then a column-strip kernel for
// dx and the parameter-gradient partial rows
#ifndef MB_LN2_ROW_VEC
#define MB_LN2_ROW_VEC 1024
#endif
#ifndef MB_LN2_B_BLOCKS
#define MB_LN2_B_BLOCKS 512
#endif
struct Ln2Plan {
  int nvec = 0;       // vectors of ln_elems_per_vector elements per row
  int rows_grid = 0;  // blocks of the row-sum kernel (one row each, grid-stride)
  int strips = 0;     // column strips of 64 vectors
  int G = 0;          // row groups of the column-strip kernel: dgamma / dbeta partial rows
};
// rows of H elements are too wide for the block backward (H a whole number of
// vectors): they take the team backward where it applies and no output
// overwrites an input, else the wide-row kernels
bool ln2_applies(int64_t H, int dt, int rdt);

// ---- backward of rows of more than MB_LN2_ROW_VEC and at most
// MB_LN_BLOCK_MAX_VEC vectors: a resident block of 512 threads (4 vectors
// each) per CU walks a range of rows with the row and its thread's parameter
// sums in registers; the blocks' partial rows are summed after (0: off, such
// rows then take the wide-row kernels)
#ifndef MB_LN_BLOCK_MAX_VEC
#define MB_LN_BLOCK_MAX_VEC 2048
#endif
struct LnBlockPlan {
  int nvec = 0;
  int64_t rows_per_block = 0;
  int grid = 0;  // blocks, and partial rows of dgamma / dbeta
};
bool ln_block_applies(int64_t H, int dt, int rdt);
LnBlockPlan plan_ln_block(int64_t T, int64_t H, int dt, int rdt, int cus);

// ---- backward of rows of more than MB_LN_BLOCK_MAX_VEC and at most
// kLnTeamMaxMembers * kLnTeamVec vectors: a row is split over a team of
// blocks (up to kLnTeamVec vectors each) that exchange their two partial row
// sums through the workspace; a team walks a contiguous range of rows (0:
// off, such rows then take the wide-row kernels, as they do when an output
// overwrites an input)
#ifndef MB_LN_TEAM
#define MB_LN_TEAM 1
#endif
constexpr int kLnTeamVec = 1024;       // vectors per member: 256 threads of 4
constexpr int kLnTeamMaxMembers = 8;   // 8192 vectors, the widest row
constexpr int kLnTeamMaxBlocksPerCu = 2;
// polls of a partner's slot before a block computes the partner's row-sum
// terms itself (a pair normally arrives within a few polls)
#ifndef MB_LN_TEAM_SPIN_LIMIT
#define MB_LN_TEAM_SPIN_LIMIT 4096
#endif
struct LnTeamPlan {
  int nvec = 0;
  int members = 0;             // blocks per row
  int slice = 0;               // vectors per member (the last one may hold fewer)
  int teams = 0;               // and partial rows of dgamma / dbeta
  int64_t rows_per_team = 0;
  int grid = 0;                // teams * members
};
bool ln_team_applies(int64_t H, int dt, int rdt);
// blocks_per_cu: how many of the kernel's blocks a compute unit holds at once
// (at most kLnTeamMaxBlocksPerCu): every block of the grid is resident
LnTeamPlan plan_ln_team(int64_t T, int64_t H, int dt, int rdt, int cus, int blocks_per_cu);
Ln2Plan plan_ln2(int64_t T, int64_t H, int dt, int rdt, int cus);
// the plan's row group is `tpr` threads of `nv` vectors
bool ln_plan_is(const LnPlan& p, int tpr, int nv);

}  // namespace mb
