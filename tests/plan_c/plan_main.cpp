// Prints launch plans (mb_plan.cpp, host arithmetic only) for queries read
// from stdin, one per line:
//   tiling T nvec target_blocks cus min_rows   -> "tiling strips G"
//   ln T H dt rdt target_blocks nv_pref cus     -> "ln nvec shape tpr nv grid partial_rows"
//   ln2 T H dt rdt cus                          -> "ln2 applies nvec rows_grid strips G"
//   lnb T H dt rdt cus                          -> "lnb applies nvec rows_per_block grid"
//   lnt T H dt rdt cus blocks_per_cu            -> "lnt applies nvec members slice teams rows_per_team grid"
#include <cstdio>
#include <cstring>

#include "mb_plan.hpp"

int main() {
  char kind[16];
  while (std::scanf("%15s", kind) == 1) {
    if (std::strcmp(kind, "tiling") == 0) {
      long long T;
      int nvec, target, cus, min_rows;
      if (std::scanf("%lld %d %d %d %d", &T, &nvec, &target, &cus, &min_rows) != 5) return 2;
      const mb::Tiling t = mb::plan_tiling(T, nvec, target, cus, min_rows);
      std::printf("tiling %d %d\n", t.strips, t.G);
    } else if (std::strcmp(kind, "ln") == 0) {
      long long T, H;
      int dt, rdt, target, nv_pref, cus;
      if (std::scanf("%lld %lld %d %d %d %d %d", &T, &H, &dt, &rdt, &target, &nv_pref, &cus) != 7) return 2;
      const mb::LnPlan p = mb::plan_ln(T, H, dt, rdt, target, nv_pref, cus);
      const int tpr = p.shape >= 0 ? mb::kLnShapes[p.shape].tpr : 0, nv = p.shape >= 0 ? mb::kLnShapes[p.shape].nv : 0;
      std::printf("ln %d %d %d %d %d %d\n", p.nvec, p.shape, tpr, nv, p.grid, p.partial_rows);
    } else if (std::strcmp(kind, "ln2") == 0) {
      long long T, H;
      int dt, rdt, cus;
      if (std::scanf("%lld %lld %d %d %d", &T, &H, &dt, &rdt, &cus) != 5) return 2;
      const mb::Ln2Plan p = mb::plan_ln2(T, H, dt, rdt, cus);
      std::printf("ln2 %d %d %d %d %d\n", mb::ln2_applies(H, dt, rdt) ? 1 : 0, p.nvec, p.rows_grid, p.strips, p.G);
    } else if (std::strcmp(kind, "lnb") == 0) {
      long long T, H;
      int dt, rdt, cus;
      if (std::scanf("%lld %lld %d %d %d", &T, &H, &dt, &rdt, &cus) != 5) return 2;
      const mb::LnBlockPlan p = mb::plan_ln_block(T, H, dt, rdt, cus);
      std::printf("lnb %d %d %lld %d\n", mb::ln_block_applies(H, dt, rdt) ? 1 : 0, p.nvec,
                  static_cast<long long>(p.rows_per_block), p.grid);
    } else if (std::strcmp(kind, "lnt") == 0) {
      long long T, H;
      int dt, rdt, cus, bpc;
      if (std::scanf("%lld %lld %d %d %d %d", &T, &H, &dt, &rdt, &cus, &bpc) != 6) return 2;
      const mb::LnTeamPlan p = mb::plan_ln_team(T, H, dt, rdt, cus, bpc);
      std::printf("lnt %d %d %d %d %d %lld %d\n", mb::ln_team_applies(H, dt, rdt) ? 1 : 0, p.nvec, p.members,
                  p.slice, p.teams, static_cast<long long>(p.rows_per_team), p.grid);
    } else {
      return 3;
    }
  }
  return 0;
}
