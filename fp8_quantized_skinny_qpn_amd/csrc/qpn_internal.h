// qpn_internal.h -- launchers shared between the C-ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qpn {

struct GemmArgs {
  const void* packed;
  const uint16_t* x;
  uint16_t* y;
  int m;
  int64_t n;
  int64_t k;
  uint64_t* keys;  // lm_head only: [m, panels] argmax keys
  void* stream;
};

// One compiled GEMM configuration: W compute wavefronts per 16-row panel,
// G panels per workgroup (plus one loader wavefront), D k-step windows of
// weight loads in flight per wavefront, NB activation windows in the LDS ring.
struct GemmPlan {
  int waves_per_panel;
  int panels_per_workgroup;
  int depth;
  int lds_slots;
};

// The plan used when none is forced: a pure function of the call's shape,
// so launch geometry never depends on anything else.
int gemm_auto_plan(uint32_t fmt, int m, int64_t n, int64_t k);

// Activation rows staged per LDS window for m rows (1, 2, 4 or 8).
int gemm_activation_rows(int m);

// Activation ring slots a plan with `slots` gets for m rows (fewer when its
// windows are wide).
int gemm_ring_slots(uint32_t fmt, int waves_per_panel, int m, int slots);

// Plan `id` (1-based) of the compiled table; false if there is none.
bool gemm_plan_info(int id, GemmPlan* out);

// Launch the GEMM (and, with `argmax`, the per-panel argmax keys) with plan
// `plan`, or the automatic plan when `plan` is 0.
hipError_t launch_gemm(uint32_t fmt, bool argmax, const GemmArgs& a, int plan);
hipError_t launch_argmax_finalize(const uint64_t* keys, int64_t panels, int m, int32_t* argmax,
                                  void* stream);

hipError_t launch_pack_nvfp4(const float* w, int64_t n, int64_t k, void* packed, void* stream);
hipError_t launch_pack_fp8(const float* w, int64_t n, int64_t k, void* packed, void* stream);

hipError_t launch_unpack_nvfp4(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                               uint8_t* scales, float* g, void* stream);
hipError_t launch_unpack_fp8(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                             float* row_scale, void* stream);
hipError_t launch_decode_nvfp4(const uint8_t* codes16, const uint8_t* scales2, int64_t count,
                               uint16_t* out, void* stream);
hipError_t launch_decode_fp8(const uint8_t* codes16, int64_t count, uint16_t* out, void* stream);
hipError_t launch_read_ceiling(const void* buf, int64_t count16, uint32_t* sink, void* stream);

}  // namespace qpn
