// Host-only stand-ins for libkvattn's kernel launchers, so that the C ABI's
// argument checks, split planning and workspace layout (api.cpp) can be
// built and run on a machine without a GPU, under the address and
// undefined-behaviour sanitizers.  Each stand-in records the arguments it was
// given and launches nothing.
#include "stub_launch.h"

namespace stub {
Record last;
}

namespace kvattn {

static hipError_t record(const char* kernel, const DecodeArgs& a) {
  stub::last.kernel = kernel;
  stub::last.args = a;
  ++stub::last.launches;
  return hipSuccess;
}

hipError_t launch_gqa_f32(const DecodeArgs& a, hipStream_t, const LaunchEvents&) { return record("gqa_f32", a); }
hipError_t launch_gqa_bf16(const DecodeArgs& a, hipStream_t, const LaunchEvents&) { return record("gqa_bf16", a); }
hipError_t launch_gqa_fp8(const DecodeArgs& a, hipStream_t, const LaunchEvents&) { return record("gqa_fp8", a); }
hipError_t launch_mla_bf16(const DecodeArgs& a, hipStream_t, const LaunchEvents&) { return record("mla_bf16", a); }
hipError_t launch_mla_plan(const MlaPlanArgs& p, hipStream_t) {
  stub::last.plan = p;
  ++stub::last.launches;
  return hipSuccess;
}
hipError_t launch_gqa_plan(const GqaPlanArgs& p, hipStream_t) {
  stub::last.gqa_plan = p;
  ++stub::last.gqa_plans;
  ++stub::last.launches;
  return hipSuccess;
}
hipError_t launch_mla_merge_pieces(const DecodeArgs&, hipStream_t) {
  ++stub::last.launches;
  return hipSuccess;
}
hipError_t launch_hbm_read_probe(const void*, int64_t, uint32_t*, int, hipStream_t) { return hipSuccess; }
hipError_t launch_latent_project(const ProjectArgs& p, hipStream_t) {
  stub::last.projects[stub::last.n_projects % 2] = p;
  ++stub::last.n_projects;
  ++stub::last.launches;
  return hipSuccess;
}
hipError_t launch_latent_rebuild(const ProjectArgs& p, hipStream_t s) { return launch_latent_project(p, s); }
hipError_t launch_mla_explicit_attend(const DecodeArgs& a, hipStream_t, const LaunchEvents&) {
  return record("mla_explicit_attend", a);
}
hipError_t launch_transpose_heads(const void* src, void* dst, int heads, int rows, int cols, hipStream_t) {
  stub::last.transposes[stub::last.n_transposes % 2] = {src, dst, heads, rows, cols};
  ++stub::last.n_transposes;
  ++stub::last.launches;
  return hipSuccess;
}
hipError_t launch_merge(const DecodeArgs&, bool, hipStream_t) {
  ++stub::last.launches;
  ++stub::last.merges;
  return hipSuccess;
}

}  // namespace kvattn
