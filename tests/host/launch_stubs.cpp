// Stand-ins for the kernel launchers of the HIP library, for a host-only
// build of the C-ABI layer (api.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every one refuses with hipErrorNotSupported:
// the CPU tests that use this build only exercise validation, planning and
// workspace sizing, which return before any launch.
#include "internal.h"

namespace tsel {

hipError_t launch_lse(const AttnPlan &, const AttnArgs &, const JobPerm *, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_colscore(const AttnPlan &, const AttnArgs &, const JobPerm *, float *, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_fwd(const AttnPlan &, const FwdArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_topk(const DevLayout &, const float *, const TopkChunk &, int, uint8_t *, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_topk_large(const DevLayout &, const float *, const TopkLarge &, const TopkLargeWs &, uint8_t *,
                             hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_mass_budget(const DevLayout &, const float *, const MassChunk &, int, int *, uint8_t *,
                              hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_compact(const CompactArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_gather(const void *, long long, long long, void *, long long, const int *, const int *, int,
                         hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_mrope(const DevLayout &, int *, const int *, const int *, int, int *, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t static_scratch(void **out) {
  *out = nullptr;
  return hipErrorNotSupported;
}

}  // namespace tsel
