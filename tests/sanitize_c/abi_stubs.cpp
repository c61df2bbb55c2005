// Stand-ins for the kernel launches, so that the C ABI's host code
// (validation, workspace sizing, launch planning) links and runs without a
// GPU under the address and undefined-behaviour sanitizers. Each launch
// only counts the call.
#include "mb_launch.hpp"

namespace mb {

int stub_launches = 0;

static hipError_t launched() {
  ++stub_launches;
  return hipSuccess;
}

hipError_t noalloc_scratch(hipStream_t, void** ptr) {
  static char fake[256];
  *ptr = fake;
  return launched();
}
hipError_t launch_fill_zero(float*, int64_t, hipStream_t) { return launched(); }
hipError_t launch_colsum2(const ColSum&, const ColSum&, hipStream_t) { return launched(); }
hipError_t launch_colsum_tall(const float*, int, int64_t, float*, float*, hipStream_t) { return launched(); }
hipError_t launch_colsum_tall2(const float*, const float*, int, int64_t, float*, float*, float*, float*, hipStream_t) {
  return launched();
}
hipError_t launch_colsum(const float*, int, int64_t, float*, hipStream_t) { return launched(); }
hipError_t launch_gelu_fwd(int, bool, const void*, const void*, void*, const Tiling&, hipStream_t) {
  return launched();
}
hipError_t launch_gelu_bwd(int, bool, const void*, const void*, const void*, void*, float*, const Tiling&,
                           hipStream_t) {
  return launched();
}
hipError_t launch_bda(int, int, bool, const void*, const void*, const void*, void*, int64_t, const Tiling&,
                      const DropoutArgs&, hipStream_t) {
  return launched();
}
hipError_t launch_dropout_mask(uint8_t*, int64_t, const DropoutArgs&, hipStream_t) { return launched(); }
hipError_t launch_bda_bwd(int, int, const void*, void*, void*, float*, int64_t, const Tiling&, const DropoutArgs&,
                          hipStream_t) {
  return launched();
}
hipError_t launch_glu_fwd(int, int, const void*, const void*, const void*, int, void*, int64_t, const Tiling&,
                          hipStream_t) {
  return launched();
}
hipError_t launch_glu_bwd(int, int, const void*, const void*, const void*, const void*, int, void*, float*, float*,
                          int64_t, const Tiling&, hipStream_t) {
  return launched();
}
hipError_t launch_srelu_fwd(int, int, const void*, const void*, void*, const Tiling&, hipStream_t) {
  return launched();
}
hipError_t launch_srelu_bwd(int, int, const void*, const void*, const void*, void*, float*, const Tiling&,
                            hipStream_t) {
  return launched();
}
hipError_t launch_ln_fwd(const LnArgs&, const LnPlan&, hipStream_t) { return launched(); }
hipError_t launch_ln_bwd(const LnArgs&, const LnPlan&, hipStream_t) { return launched(); }
hipError_t launch_ln2_bwd(const LnArgs&, const Ln2Plan&, hipStream_t) { return launched(); }
hipError_t launch_ln_block_bwd(const LnArgs&, const LnBlockPlan&, hipStream_t) { return launched(); }
hipError_t launch_ln_team_bwd(const LnArgs&, const LnTeamPlan&, hipStream_t) { return launched(); }
int ln_team_blocks_per_cu(int, int) { return 2; }
void set_ln_team_spin_limit(int) {}

}  // namespace mb
