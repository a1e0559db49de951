// qpn_gemm.hip -- the QPN skinny GEMM and lm_head kernels for gfx950.
//
// Y[m, n] = FP16( scale * sum_k X[m, k] * Wq[n, k] ) for m < M <= 8, with the
// weights read once, compressed, straight from HBM and expanded in registers
// (taozi.news page, section "自研 QPN 内核"; aiwitness.kr page, section
// "내가 실제로 만든 것").  The pages map the 8 verify rows onto Volta's
// 8-row FP16 tensor-core tile; on CDNA4 the matrix unit's narrowest f16 tile
// is 16 wide, so the M <= 8 activation rows fill half of the B operand of a
// 16x16x32 MFMA and the other half is zero.  At these arithmetic intensities
// (2M flops per weight) the MFMA runs at a few percent of its peak; the
// kernel is bound by HBM, and the MFMA is used because it performs the
// K-reduction across lanes for free and keeps VALU time for decoding.
//
// Work split: one workgroup per 16-row panel; its W wavefronts split the
// panel's k-steps into W contiguous ranges and reduce their partial tiles
// through LDS in a fixed order (deterministic, and independent of where a
// row sits in the matrix).  Each wavefront keeps D k-steps of weights and
// the matching activations in flight: the activation loads of a k-step are
// issued together with its weight loads, because vector loads complete in
// order and a later activation load would otherwise make the wave wait for
// the whole prefetch.
#include "qpn_common.h"
#include "qpn_internal.h"

namespace qpn {

namespace {

template <uint32_t FMT>
struct Fmt;

template <>
struct Fmt<kFmtNvfp4> {
  static constexpr int kKStep = kNvKStep;
  static constexpr int kChunk = kNvChunkBytes;
  static constexpr int kGroups = 4;  // MFMAs (8 codes each per lane) per k-step
};

template <>
struct Fmt<kFmtFp8> {
  static constexpr int kKStep = kF8KStep;
  static constexpr int kChunk = kF8ChunkBytes;
  static constexpr int kGroups = 2;
};

// Activation operand of one k-step: B[k][col] for col = lane & 15 (the
// activation row), 8 consecutive K values per MFMA group.  Lanes whose
// column is >= m, and K past k, read zeros.
template <int G>
struct XStep {
  half8 b[G];
};

// Weight bytes of one k-step for this lane.
struct WStep {
  u32x4 codes;
  uint32_t scales;  // two UE4M3 bytes (NVFP4 only)
};

__device__ __forceinline__ uint64_t argmax_key(uint16_t h, uint32_t col) {
  // order-preserving map of FP16 bit patterns; -0 counts as +0
  if (h == 0x8000u) h = 0;
  uint32_t ord = (h & 0x8000u) ? (~(uint32_t)h & 0xFFFFu) : ((uint32_t)h | 0x8000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - col);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, mask, 64);
  hi = __shfl_xor(hi, mask, 64);
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace

template <uint32_t FMT, int W, int D, bool ARGMAX>
__global__ __launch_bounds__(kLanes * W) void skinny_gemm_kernel(
    const uint8_t* __restrict__ blob, const uint16_t* __restrict__ x,
    uint16_t* __restrict__ y, int m, int64_t n, int64_t k,
    uint64_t* __restrict__ keys) {
  using F = Fmt<FMT>;
  constexpr int G = F::kGroups;
  constexpr int R = D + 1;  // ring slots: one being consumed, D in flight
  const int lane = threadIdx.x & (kLanes - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int64_t p = blockIdx.x;
  const int J = (int)((k + F::kKStep - 1) / F::kKStep);  // k-steps, last may be partial
  const int Jfull = (int)(k / F::kKStep);                // full k-steps
  const int row = lane & 15;  // weight row in the panel / activation row (B column)
  const int kg = lane >> 4;   // K group of this lane inside a k-step

  const BlobHeader* hdr = reinterpret_cast<const BlobHeader*>(blob);
  const bool valid = hdr->magic == kMagic && hdr->format == FMT &&
                     hdr->layout_version == kLayoutVersion && hdr->n == n && hdr->k == k;

  const uint8_t* pbase = blob + (FMT == kFmtNvfp4 ? (uint64_t)kHeaderBytes : f8_codes_offset(n)) +
                         (uint64_t)p * (uint64_t)J * F::kChunk;

  // Activations through a raw buffer resource covering exactly x[m, k]:
  // lanes whose row is >= m fall outside it and read zeros, so every load is
  // unconditional (no lane branches, static wait counts).  The lane part of
  // the offset is fixed; the k-step part is a scalar offset.
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)x, (short)0, (int)((int64_t)m * k * 2), 0x00020000);
  const int xlane_off = (int)(((int64_t)row * k + kg * (F::kKStep / 4)) * 2);

  float4v acc = {0.f, 0.f, 0.f, 0.f};

  auto issue = [&](int j, WStep& w, XStep<G>& xs) {
    const uint8_t* ch = pbase + (uint32_t)(j * F::kChunk);
    w.codes = load_nt_16(ch + 16 * lane);
    if constexpr (FMT == kFmtNvfp4)
      w.scales = *reinterpret_cast<const uint16_t*>(ch + kNvCodeBytes + 2 * lane);
    const int soff = j * F::kKStep * 2;
#pragma unroll
    for (int t = 0; t < G; ++t)
      xs.b[t] = __builtin_bit_cast(
          half8, __builtin_amdgcn_raw_buffer_load_b128(xres, xlane_off + 16 * t, soff, 0));
  };

  auto compute = [&](const WStep& w, const XStep<G>& xs) {
    half8 a[G];
    if constexpr (FMT == kFmtNvfp4)
      decode_nvfp4_fragment(w.codes, w.scales, a);
    else
      decode_fp8_fragment(w.codes, a);
#pragma unroll
    for (int t = 0; t < G; ++t)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], xs.b[t], acc, 0, 0, 0);
  };

  if (valid) {
    // This wavefront's full k-steps [j0, j1).
    const int j0 = (int)((int64_t)Jfull * wave / W);
    const int j1 = (int)((int64_t)Jfull * (wave + 1) / W);
    const int nsteps = j1 - j0;
    WStep ws[R];
    XStep<G> xs[R];
    if (nsteps >= D + R) {
      // Prologue, steady state and drain.  The steady loop issues k-step
      // j+i+D into the slot freed by k-step j+i-1 and then consumes k-step
      // j+i; every load in it is unconditional.
#pragma unroll
      for (int i = 0; i < D; ++i) issue(j0 + i, ws[i], xs[i]);
      int j = j0;
      for (; j + D + R <= j1; j += R) {
#pragma unroll
        for (int i = 0; i < R; ++i) {
          // scheduling fences keep the issue-ahead order: the scheduler would
          // otherwise hoist later slots' decode and shorten the prefetch
          issue(j + i + D, ws[(i + D) % R], xs[(i + D) % R]);
          __builtin_amdgcn_sched_barrier(0);
          compute(ws[i], xs[i]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
#pragma unroll
      for (int i = 0; i < D + R - 1; ++i) {
        if (j + i + D < j1) issue(j + i + D, ws[(i + D) % R], xs[(i + D) % R]);
        if (j + i < j1) compute(ws[i % R], xs[i % R]);
      }
    } else {
      // Short range: batches of R k-steps, issued together then consumed.
      for (int j = j0; j < j1; j += R) {
#pragma unroll
        for (int i = 0; i < R; ++i)
          if (j + i < j1) issue(j + i, ws[i], xs[i]);
#pragma unroll
        for (int i = 0; i < R; ++i)
          if (j + i < j1) compute(ws[i], xs[i]);
      }
    }
    // A partial last k-step (k not a multiple of the k-step) goes to the last
    // wavefront; its K positions past k read zero activations.
    if (J > Jfull && wave == W - 1) {
      const uint8_t* ch = pbase + (uint32_t)(Jfull * F::kChunk);
      WStep w;
      XStep<G> xt;
      w.codes = load_nt_16(ch + 16 * lane);
      if constexpr (FMT == kFmtNvfp4)
        w.scales = *reinterpret_cast<const uint16_t*>(ch + kNvCodeBytes + 2 * lane);
#pragma unroll
      for (int t = 0; t < G; ++t) {
        const int64_t kk = (int64_t)Jfull * F::kKStep + kg * (F::kKStep / 4) + 8 * t;
        const int off = kk < k ? (int)(((int64_t)row * k + kk) * 2) : 0x7FFFFFF0;
        xt.b[t] = __builtin_bit_cast(half8, __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0));
      }
      compute(w, xt);
    }
  }

  // Cross-wave reduction in a fixed order: wave 0 + wave 1 + ... + wave W-1.
  if constexpr (W > 1) {
    __shared__ float4v red[W][kLanes];
    red[wave][lane] = acc;
    __syncthreads();
    if (wave != 0) return;
    acc = red[0][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) acc += red[w][lane];
  }

  // Epilogue.  Lane holds D[i][j] for j = lane & 15 (activation row) and
  // i = 4 (lane >> 4) + v (panel row).
  const int mcol = lane & 15;
  const int64_t n0 = p * kPanelRows + 4 * (lane >> 4);
  uint16_t h[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t nn = n0 + v;
    float s = 0.f;  // the blob is only read past its header when the header matched
    if (valid) {
      if constexpr (FMT == kFmtNvfp4)
        s = hdr->tensor_scale;
      else
        s = nn < n ? reinterpret_cast<const float*>(blob + kHeaderBytes)[nn] : 0.f;
    }
    _Float16 o = valid ? (_Float16)(s * acc[v]) : (_Float16)__builtin_nanf("");
    h[v] = __builtin_bit_cast(uint16_t, o);
    if (mcol < m && nn < n) y[(int64_t)mcol * n + nn] = h[v];
  }

  if constexpr (ARGMAX) {
    // best (value, lowest index) over this lane's 4 rows, then over the 4
    // lanes that share the activation row
    uint64_t best = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t nn = n0 + v;
      if (nn < n) {
        uint64_t key = argmax_key(h[v], (uint32_t)nn);
        best = key > best ? key : best;
      }
    }
    uint64_t o16 = shfl_xor_u64(best, 16);
    best = o16 > best ? o16 : best;
    uint64_t o32 = shfl_xor_u64(best, 32);
    best = o32 > best ? o32 : best;
    if (lane < 16 && mcol < m) keys[(int64_t)mcol * gridDim.x + p] = best;
  }
}

// Final argmax: one block per activation row reduces that row's panel keys.
__global__ __launch_bounds__(256) void argmax_finalize_kernel(const uint64_t* __restrict__ keys,
                                                              int64_t panels,
                                                              int32_t* __restrict__ argmax) {
  __shared__ uint64_t part[256];
  const int mi = blockIdx.x;
  uint64_t best = 0;
  for (int64_t i = threadIdx.x; i < panels; i += 256) {
    uint64_t kv = keys[(int64_t)mi * panels + i];
    best = kv > best ? kv : best;
  }
  part[threadIdx.x] = best;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) {
      uint64_t o = part[threadIdx.x + s];
      if (o > part[threadIdx.x]) part[threadIdx.x] = o;
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) argmax[mi] = (int32_t)(0xFFFFFFFFu - (uint32_t)(part[0] & 0xFFFFFFFFu));
}

// ---------------------------------------------------------------------------
// Launch plumbing.
// ---------------------------------------------------------------------------
namespace {

template <uint32_t FMT>
constexpr int kDepth = (FMT == kFmtNvfp4) ? 3 : 4;

template <uint32_t FMT, bool ARGMAX, int W>
hipError_t launch_w(const GemmArgs& a) {
  constexpr int D = kDepth<FMT>;
  hipLaunchKernelGGL((skinny_gemm_kernel<FMT, W, D, ARGMAX>), dim3((unsigned)panels_of(a.n)),
                     dim3(kLanes * W), 0, (hipStream_t)a.stream, (const uint8_t*)a.packed,
                     a.x, a.y, a.m, a.n, a.k, a.keys);
  return hipGetLastError();
}

template <uint32_t FMT, bool ARGMAX>
hipError_t launch_fmt(const GemmArgs& a, int waves) {
  switch (waves) {
    case 1: return launch_w<FMT, ARGMAX, 1>(a);
    case 2: return launch_w<FMT, ARGMAX, 2>(a);
    case 4: return launch_w<FMT, ARGMAX, 4>(a);
    case 8: return launch_w<FMT, ARGMAX, 8>(a);
    case 16: return launch_w<FMT, ARGMAX, 16>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gemm_prefetch_depth(uint32_t fmt) { return fmt == kFmtNvfp4 ? kDepth<kFmtNvfp4> : kDepth<kFmtFp8>; }

int gemm_waves_per_panel(uint32_t fmt, int64_t n, int64_t k) {
  const int64_t P = panels_of(n);
  const int64_t J = fmt == kFmtNvfp4 ? nv_ksteps_of(k) : f8_ksteps_of(k);
  int w = 1;
  // Aim for >= 2560 wavefronts in flight (10 per CU) while every wavefront
  // still owns at least 4 k-steps.
  while (w < 16 && P * w < 2560 && J / (2 * w) >= 4) w *= 2;
  return w;
}

hipError_t launch_gemm(uint32_t fmt, bool argmax, const GemmArgs& a, int waves) {
  if (fmt == kFmtNvfp4)
    return argmax ? launch_fmt<kFmtNvfp4, true>(a, waves) : launch_fmt<kFmtNvfp4, false>(a, waves);
  if (argmax) return hipErrorInvalidValue;
  return launch_fmt<kFmtFp8, false>(a, waves);
}

hipError_t launch_argmax_finalize(const uint64_t* keys, int64_t panels, int m, int32_t* argmax,
                                  void* stream) {
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(m), dim3(256), 0, (hipStream_t)stream, keys,
                     panels, argmax);
  return hipGetLastError();
}

}  // namespace qpn
