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

// Wavefronts per 16-row panel chosen for an (n, k) call; a pure function of
// the shape, so launch geometry never depends on anything else.
int gemm_waves_per_panel(uint32_t fmt, int64_t n, int64_t k);

// k-steps each wavefront keeps in flight (a compile-time constant per format).
int gemm_prefetch_depth(uint32_t fmt);

hipError_t launch_gemm(uint32_t fmt, bool argmax, const GemmArgs& a, int waves);
hipError_t launch_stream(uint32_t fmt, bool argmax, const GemmArgs& a, int plan);
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
