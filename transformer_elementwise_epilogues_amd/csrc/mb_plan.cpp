// mb_plan.cpp -- launch planning (see mb_plan.hpp): host arithmetic only.
#include "mb_plan.hpp"

#include <algorithm>

namespace mb {

namespace {
constexpr int kWavesPerBlock = 4;  // every tiled kernel: blocks of 4 waves
constexpr int kStripVectors = 64;  // a wave covers 64 16-byte column vectors
}  // namespace

int scaled_blocks(int target_blocks, int cus) {
  if (cus <= 0) cus = kTunedCUs;
  const int64_t b = static_cast<int64_t>(target_blocks) * cus / kTunedCUs;
  return static_cast<int>(std::max<int64_t>(1, b));
}

Tiling plan_tiling(int64_t T, int nvec, int target_blocks, int cus, int min_rows) {
  Tiling t;
  t.T = T;
  t.nvec = nvec;
  t.strips = std::max(1, (nvec + kStripVectors - 1) / kStripVectors);  // at least one strip, even for nvec 0
  // Round down: a grid slightly larger than the resident capacity would leave a
  // few straggler blocks running alone after the rest finish.
  const int64_t want = std::max<int64_t>(1, scaled_blocks(target_blocks, cus) / t.strips);
  const int64_t rows_per_group = static_cast<int64_t>(kWavesPerBlock) * std::max(1, min_rows);
  const int64_t most = std::max<int64_t>(1, (T + rows_per_group - 1) / rows_per_group);
  t.G = static_cast<int>(std::min<int64_t>(std::min(want, most), 65535));
  return t;
}

int64_t colsum_tall_tmp_floats(int R, int64_t C) { return R <= 32 ? 0 : static_cast<int64_t>((R + 31) / 32) * C; }

int bda_elems_per_lane(int dt, int res_dt) {
  if (dt == 0) return 4;
  return res_dt == 0 ? 4 : 8;
}

int ln_elems_per_vector(int dt, int rdt) {
  if (rdt == 0 && dt != 0) return 4;
  return dt == 0 ? 4 : 8;
}

// Threads per row: the smallest of 64, 256, 512, 1024 that holds the row in
// at most `nv_pref` vectors per thread (1024 takes up to 8).
LnPlan plan_ln(int64_t T, int64_t H, int dt, int rdt, int target_blocks, int nv_pref, int cus) {
  LnPlan p;
  const int E = ln_elems_per_vector(dt, rdt);
  p.nvec = static_cast<int>(H / E);
  p.shape = -1;
  int tpr = 64;
  while (tpr < 1024 && static_cast<int64_t>(tpr) * nv_pref < p.nvec) tpr = tpr == 64 ? 256 : tpr * 2;
  int nv = 1;
  while (nv < 16 && static_cast<int64_t>(tpr) * nv < p.nvec) nv *= 2;
  if (static_cast<int64_t>(tpr) * nv < p.nvec) return p;  // wider than 8192 vectors
  for (int i = 0; i < kLnNumShapes; ++i)
    if (kLnShapes[i].tpr == tpr && kLnShapes[i].nv == nv) p.shape = i;
  if (p.shape < 0) return p;
  const LnShape sh = kLnShapes[p.shape];
  const int64_t groups = (T + sh.rpb - 1) / sh.rpb;
  p.grid = static_cast<int>(std::min<int64_t>(std::max<int64_t>(groups, 1), scaled_blocks(target_blocks, cus)));
  p.partial_rows = p.grid;
  p.cus = cus > 0 ? cus : kTunedCUs;
  return p;
}

bool ln_block_applies(int64_t H, int dt, int rdt) {
  const int64_t nvec = H / ln_elems_per_vector(dt, rdt);
  return nvec > MB_LN2_ROW_VEC && nvec <= MB_LN_BLOCK_MAX_VEC;
}

bool ln_team_applies(int64_t H, int dt, int rdt) {
  const int64_t nvec = H / ln_elems_per_vector(dt, rdt);
  return MB_LN_TEAM && nvec > std::max<int64_t>(MB_LN2_ROW_VEC, MB_LN_BLOCK_MAX_VEC) &&
         nvec <= static_cast<int64_t>(kLnTeamMaxMembers) * kLnTeamVec;
}

bool ln2_applies(int64_t H, int dt, int rdt) {
  return H / ln_elems_per_vector(dt, rdt) > std::max<int64_t>(MB_LN2_ROW_VEC, MB_LN_BLOCK_MAX_VEC);
}

LnTeamPlan plan_ln_team(int64_t T, int64_t H, int dt, int rdt, int cus, int blocks_per_cu) {
  LnTeamPlan p;
  p.nvec = static_cast<int>(H / ln_elems_per_vector(dt, rdt));
  p.members = std::max(1, (p.nvec + kLnTeamVec - 1) / kLnTeamVec);
  p.slice = (p.nvec + p.members - 1) / p.members;  // balanced: the slices differ by at most members - 1
  const int64_t resident = static_cast<int64_t>(cus > 0 ? cus : kTunedCUs) *
                           std::max(1, std::min(blocks_per_cu, kLnTeamMaxBlocksPerCu));
  const int64_t teams = std::max<int64_t>(1, std::min<int64_t>(T, resident / p.members));
  p.rows_per_team = std::max<int64_t>(1, (T + teams - 1) / teams);
  p.teams = static_cast<int>(std::max<int64_t>(1, (T + p.rows_per_team - 1) / p.rows_per_team));
  p.grid = p.teams * p.members;
  return p;
}

LnBlockPlan plan_ln_block(int64_t T, int64_t H, int dt, int rdt, int cus) {
  LnBlockPlan p;
  p.nvec = static_cast<int>(H / ln_elems_per_vector(dt, rdt));
  const int64_t resident = std::max<int64_t>(1, cus > 0 ? cus : kTunedCUs);
  const int64_t blocks = std::max<int64_t>(1, std::min<int64_t>(T, resident));
  p.rows_per_block = std::max<int64_t>(1, (T + blocks - 1) / blocks);
  p.grid = static_cast<int>(std::max<int64_t>(1, (T + p.rows_per_block - 1) / p.rows_per_block));
  return p;
}

Ln2Plan plan_ln2(int64_t T, int64_t H, int dt, int rdt, int cus) {
  Ln2Plan p;
  p.nvec = static_cast<int>(H / ln_elems_per_vector(dt, rdt));
  p.rows_grid = static_cast<int>(std::min<int64_t>(std::max<int64_t>(T, 1), 1 << 20));
  const Tiling t = plan_tiling(T, p.nvec, MB_LN2_B_BLOCKS, cus);
  p.strips = t.strips;
  p.G = t.G;
  return p;
}

bool ln_plan_is(const LnPlan& p, int tpr, int nv) {
  return p.shape >= 0 && kLnShapes[p.shape].tpr == tpr && kLnShapes[p.shape].nv == nv;
}

}  // namespace mb
