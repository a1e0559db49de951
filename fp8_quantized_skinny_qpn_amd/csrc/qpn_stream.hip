// qpn_stream.hip -- the streaming QPN skinny GEMM: activations through an LDS
// ring fed by a dedicated loader wavefront, weights streamed by the compute
// wavefronts with a deep register prefetch.
//
// Why this shape (CDNA4 specifics; the pages' own kernel was built around
// Volta's 8-row tensor-core tile, taozi.news page, section "自研 QPN 内核"):
//   * Vector memory loads of one wavefront complete in order.  If a compute
//     wavefront also loaded activations, every wait for activation data would
//     also wait for all weight loads issued before it and the weight prefetch
//     would collapse.  So the compute wavefronts issue weight loads only; the
//     activations are staged into LDS by one extra wavefront per workgroup and
//     read back with ds_read (a separate counter).
//   * Every activation row is needed by every 16-row panel.  Staging it once
//     per workgroup into LDS replaces per-panel, per-lane activation loads
//     (which cost more L2->CU bytes than the weights themselves at M = 8).
//
// Schedule.  A workgroup owns G consecutive 16-row panels.  Each panel is
// worked on by W compute wavefronts that interleave its k-steps: "window" c is
// k-steps [cW, cW + W), and wavefront w of the panel consumes k-step cW + w.
// The loader wavefront writes window c's activations into LDS ring slot
// c % NB, NB - 1 windows ahead, with direct-to-LDS buffer loads whose
// out-of-range lanes (rows >= m, K >= k) deliver zeros.  One s_barrier per
// window hands a filled slot to the compute wavefronts and a drained one back
// to the loader.  The compute wavefronts keep D windows of weight loads in
// flight (5 VGPRs per k-step); near the end they keep issuing loads aimed at
// one shared chunk instead of branching, so every wait count is static.  Partial tiles
// of a panel's W wavefronts are summed through LDS in a fixed order.
#include "qpn_common.h"
#include "qpn_internal.h"

namespace qpn {

namespace {

template <uint32_t FMT>
struct SFmt;
template <>
struct SFmt<kFmtNvfp4> {
  static constexpr int kKStep = kNvKStep;
  static constexpr int kChunk = kNvChunkBytes;
  static constexpr int kGroups = 4;
};
template <>
struct SFmt<kFmtFp8> {
  static constexpr int kKStep = kF8KStep;
  static constexpr int kChunk = kF8ChunkBytes;
  static constexpr int kGroups = 2;
};

// Weight bytes of one k-step for one lane.  The scale pair stays 16-bit in
// the ring (widened only where it is used), so no instruction touches a
// register whose load may still be in flight.
struct WFrag {
  u32x4 codes;
  uint16_t scales;
};

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt 6:4, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));
}

// Workgroup barrier without any memory fence: LDS hand-offs are ordered by
// the explicit waits around it; weight loads stay in flight across it.
__device__ __forceinline__ void bare_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ uint64_t s_argmax_key(uint16_t h, uint32_t col) {
  if (h == 0x8000u) h = 0;  // -0 counts as +0
  uint32_t ord = (h & 0x8000u) ? (~(uint32_t)h & 0xFFFFu) : ((uint32_t)h | 0x8000u);
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - col);
}

__device__ __forceinline__ uint64_t s_shfl_xor_u64(uint64_t v, int mask) {
  uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  lo = __shfl_xor(lo, mask, 64);
  hi = __shfl_xor(hi, mask, 64);
  return ((uint64_t)hi << 32) | lo;
}

}  // namespace

// Bytes of one LDS activation window (padded to whole 1 KiB loader loads).
template <uint32_t FMT, int W, int MB>
constexpr int window_bytes() {
  return ((W * (SFmt<FMT>::kKStep / 8) * MB + 63) / 64) * 1024;
}

template <uint32_t FMT, int W, int G, int D, int NB, int MB, bool ARGMAX>
__global__ __launch_bounds__(kLanes * (G * W + 1)) void stream_gemm_kernel(
    const uint8_t* __restrict__ blob, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    int m, int64_t n, int64_t k, uint64_t* __restrict__ keys) {
  using F = SFmt<FMT>;
  constexpr int KS = F::kKStep;
  constexpr int GR = F::kGroups;
  constexpr int NCW = G * W;                      // compute wavefronts
  constexpr int UNITS = W * (KS / 8) * MB;        // 16-byte activation units per window
  constexpr int LPW = (UNITS + 63) / 64;          // loader loads per window
  constexpr int WINB = LPW * 1024;
  constexpr int R = D + 1;                        // weight ring slots
  static_assert(NB >= 2, "ring needs two slots");
  static_assert(NCW + 1 <= 16, "at most 16 wavefronts");
  static_assert((NB - 2) * LPW < 64, "loader wait count");

  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int lane = threadIdx.x & (kLanes - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int64_t P = panels_of(n);
  const int J = (int)((k + KS - 1) / KS);

  const BlobHeader* hdr = reinterpret_cast<const BlobHeader*>(blob);
  const bool valid = hdr->magic == kMagic && hdr->format == FMT &&
                     hdr->layout_version == kLayoutVersion && hdr->n == n && hdr->k == k;
  // Windows of real work, padded to whole weight-ring cycles so the compute
  // loop body is straight-line with static ring slots (and so exact wait
  // counts).  Padded windows cost a barrier and an L2-resident spare load;
  // the loader does nothing in them.  Every wavefront of the workgroup runs
  // the same number of windows, hence of barriers.
  const int nwin = valid ? (J + W - 1) / W : 0;
  const int nwin_pad = ((nwin + R - 1) / R) * R;

  if (wv == NCW) {
    // ---------------- loader wavefront ----------------
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x, (short)0, (int)((int64_t)m * k * 2), 0x00020000);
    // Load q, lane l fills 16-byte unit u = 64 q + l of a window:
    // u = ((jw * GR + t) * 4 + kg) * MB + mm  (step-in-window jw, MFMA group t,
    // K group kg, activation row mm), at K = window start + koff.
    // K positions stay below 2^21 and byte offsets below 2^25: 32-bit math.
    const int kk = (int)k;
    int rowoff[LPW], koff[LPW];
#pragma unroll
    for (int q = 0; q < LPW; ++q) {
      const int u = q * 64 + lane;
      const int mm = u % MB;
      const int rest = u / MB;
      koff[q] = (rest / (4 * GR)) * KS + (rest % 4) * (KS / 4) + 8 * ((rest / 4) % GR);
      // rows >= m and padding units never address the buffer: push their K
      // position out of range instead
      rowoff[q] = mm * kk * 2;
      if (!(u < UNITS && mm < m)) koff[q] = 1 << 24;
    }
    auto issue_window = [&](int c) {
      uint8_t* slot = smem + (c % NB) * WINB;
      const int kbase = c * W * KS;  // first K of the window
#pragma unroll
      for (int q = 0; q < LPW; ++q) {
        // K past k (ragged tail, padded windows) reads zeros: out of range
        const int kpos = kbase + koff[q];
        const int off = kpos < kk ? rowoff[q] + 2 * kpos : 0x7FFFFFF0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xres, (__attribute__((address_space(3))) void*)(slot + q * 1024), 16, off, 0, 0, 0);
      }
    };
#pragma unroll
    for (int c = 0; c < NB - 1; ++c) issue_window(c);
    wait_vmcnt<(NB - 2) * LPW>();
    bare_barrier();  // window 0 is in LDS
    for (int c = 0; c < nwin; ++c) {
      issue_window(c + NB - 1);  // into the slot drained in window c - 1
      wait_vmcnt<(NB - 2) * LPW>();
      bare_barrier();  // window c + 1 is in LDS; window c is consumed
    }
    for (int c = nwin; c < nwin_pad; ++c) bare_barrier();
    wait_vmcnt<0>();
    bare_barrier();  // no LDS writes in flight any more
    bare_barrier();  // partial tiles written
    return;
  }

  // ---------------- compute wavefronts ----------------
  const int gi = wv / W;  // panel of this wavefront inside the workgroup
  const int w = wv % W;   // its position inside each window
  const int64_t p = (int64_t)blockIdx.x * G + gi;
  const bool active = p < P;
  const int row = lane & 15, kg = lane >> 4;
  const uint8_t* pbase = blob + (FMT == kFmtNvfp4 ? (uint64_t)kHeaderBytes : f8_codes_offset(n)) +
                         (uint64_t)(active ? p : 0) * (uint64_t)J * F::kChunk;
  // this wavefront's k-steps are w, w + W, ...; its last valid one:
  const int slast = (J > w) ? w + ((J - 1 - w) / W) * W : 0;
  const bool any_step = active && J > w;

  // Past the end of its k-steps a wavefront keeps issuing loads (so wait
  // counts stay static) but aims them at chunk 0 of panel 0: every
  // workgroup's surplus loads hit the same 1 KiB, which stays in L2.
  const uint8_t* spare = blob + (FMT == kFmtNvfp4 ? (uint64_t)kHeaderBytes : f8_codes_offset(n));
  auto issue = [&](int c, WFrag& f) {
    const int s = c * W + w;
    const uint8_t* ch = s <= slast ? pbase + (uint32_t)(s * F::kChunk) : spare;
    f.codes = load_nt_16(ch + 16 * lane);
    if constexpr (FMT == kFmtNvfp4)
      f.scales = *reinterpret_cast<const uint16_t*>(ch + kNvCodeBytes + 2 * lane);
  };

  float4v acc = {0.f, 0.f, 0.f, 0.f};
  // activation operand for this lane: row min(row, MB-1) (columns >= m are
  // discarded by the epilogue), K group kg, own step jw = w of the window
  const int xrow = row < MB ? row : MB - 1;
  const int xoff0 = (((w * GR) * 4 + kg) * MB + xrow) * 16;

  auto compute = [&](int c, const WFrag& f) {
    half8 a[GR];
    if constexpr (FMT == kFmtNvfp4)
      decode_nvfp4_fragment(f.codes, (uint32_t)f.scales, a);
    else
      decode_fp8_fragment(f.codes, a);
    const uint8_t* xs = smem + (c % NB) * WINB + xoff0;
#pragma unroll
    for (int t = 0; t < GR; ++t) {
      const half8 b = *reinterpret_cast<const half8*>(xs + t * 4 * MB * 16);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], b, acc, 0, 0, 0);
    }
  };

  WFrag ring[R];
  if (any_step) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      issue(i, ring[i]);
      __builtin_amdgcn_sched_barrier(0);  // keep codes and scales of a k-step adjacent
    }
    bare_barrier();  // window 0 ready
    for (int c0 = 0; c0 < nwin_pad; c0 += R) {
#pragma unroll
      for (int i = 0; i < R; ++i) {
        const int c = c0 + i;
        issue(c + D, ring[(i + D) % R]);
        __builtin_amdgcn_sched_barrier(0);
        if (c * W + w < J) compute(c, ring[i]);  // no loads inside: waits unaffected
        __builtin_amdgcn_sched_barrier(0);
        bare_barrier();
      }
    }
  } else {
    bare_barrier();
    for (int c = 0; c < nwin_pad; ++c) bare_barrier();
  }
  bare_barrier();  // loader drained: LDS is free for the reduction

  // Fixed-order sum of the W partial tiles of each panel.
  float4v* red = reinterpret_cast<float4v*>(smem);
  if constexpr (W > 1) red[wv * kLanes + lane] = acc;
  wait_lgkmcnt0();  // this wavefront's partial tile has reached LDS
  bare_barrier();
  if (w != 0 || !active) return;
  if constexpr (W > 1) {
    acc = red[(gi * W) * kLanes + lane];
#pragma unroll
    for (int i = 1; i < W; ++i) acc += red[(gi * W + i) * kLanes + lane];
  }

  const int mcol = lane & 15;
  const int64_t n0 = p * kPanelRows + 4 * (lane >> 4);
  uint16_t h[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t nn = n0 + v;
    float s = 0.f;
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
    uint64_t best = 0;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int64_t nn = n0 + v;
      if (nn < n) {
        const uint64_t key = s_argmax_key(h[v], (uint32_t)nn);
        best = key > best ? key : best;
      }
    }
    uint64_t o16 = s_shfl_xor_u64(best, 16);
    best = o16 > best ? o16 : best;
    uint64_t o32 = s_shfl_xor_u64(best, 32);
    best = o32 > best ? o32 : best;
    if (lane < 16 && mcol < m) keys[(int64_t)mcol * P + p] = best;
  }
}

// ---------------------------------------------------------------------------
// Launch plumbing and plan table.
// ---------------------------------------------------------------------------
namespace {

template <uint32_t FMT, int W, int G, int D, int NB, int MB, bool ARGMAX>
hipError_t launch_stream_t(const GemmArgs& a) {
  constexpr int WINB = window_bytes<FMT, W, MB>();
  size_t lds = (size_t)NB * WINB;
  const size_t red = (size_t)G * W * kLanes * 16;
  if (lds < red) lds = red;
  const int64_t wgs = (panels_of(a.n) + G - 1) / G;
  hipLaunchKernelGGL((stream_gemm_kernel<FMT, W, G, D, NB, MB, ARGMAX>), dim3((unsigned)wgs),
                     dim3(kLanes * (G * W + 1)), lds, (hipStream_t)a.stream,
                     (const uint8_t*)a.packed, a.x, a.y, a.m, a.n, a.k, a.keys);
  return hipGetLastError();
}

template <uint32_t FMT, int W, int G, int D, int NB, bool ARGMAX>
hipError_t launch_stream_mb(const GemmArgs& a) {
  if (a.m <= 2) return launch_stream_t<FMT, W, G, D, NB, 2, ARGMAX>(a);
  if (a.m <= 4) return launch_stream_t<FMT, W, G, D, NB, 4, ARGMAX>(a);
  return launch_stream_t<FMT, W, G, D, NB, 8, ARGMAX>(a);
}

}  // namespace

// Variants selectable by plan id (all with NB = 4 activation slots).
hipError_t launch_stream(uint32_t fmt, bool argmax, const GemmArgs& a, int plan) {
  if (fmt == kFmtNvfp4) {
    if (argmax) {
      switch (plan) {
        case 1: return launch_stream_mb<kFmtNvfp4, 4, 1, 4, 4, true>(a);
        case 2: return launch_stream_mb<kFmtNvfp4, 4, 2, 4, 4, true>(a);
        case 3: return launch_stream_mb<kFmtNvfp4, 8, 1, 4, 4, true>(a);
        case 4: return launch_stream_mb<kFmtNvfp4, 2, 4, 4, 4, true>(a);
        default: return hipErrorInvalidValue;
      }
    }
    switch (plan) {
      case 1: return launch_stream_mb<kFmtNvfp4, 4, 1, 4, 4, false>(a);
      case 2: return launch_stream_mb<kFmtNvfp4, 4, 2, 4, 4, false>(a);
      case 3: return launch_stream_mb<kFmtNvfp4, 8, 1, 4, 4, false>(a);
      case 4: return launch_stream_mb<kFmtNvfp4, 2, 4, 4, 4, false>(a);
      case 5: return launch_stream_mb<kFmtNvfp4, 4, 1, 8, 4, false>(a);
      case 6: return launch_stream_mb<kFmtNvfp4, 8, 1, 6, 4, false>(a);
      case 7: return launch_stream_mb<kFmtNvfp4, 4, 2, 6, 4, false>(a);
      case 8: return launch_stream_mb<kFmtNvfp4, 4, 3, 4, 4, false>(a);
      case 9: return launch_stream_mb<kFmtNvfp4, 2, 2, 8, 4, false>(a);
      case 10: return launch_stream_mb<kFmtNvfp4, 2, 1, 8, 4, false>(a);
      case 11: return launch_stream_mb<kFmtNvfp4, 1, 4, 8, 4, false>(a);
      case 12: return launch_stream_mb<kFmtNvfp4, 4, 1, 6, 3, false>(a);
      default: return hipErrorInvalidValue;
    }
  }
  if (argmax) return hipErrorInvalidValue;
  switch (plan) {
    case 1: return launch_stream_mb<kFmtFp8, 4, 1, 4, 4, false>(a);
    case 2: return launch_stream_mb<kFmtFp8, 4, 2, 4, 4, false>(a);
    case 3: return launch_stream_mb<kFmtFp8, 8, 1, 4, 4, false>(a);
    case 4: return launch_stream_mb<kFmtFp8, 2, 4, 4, 4, false>(a);
    case 5: return launch_stream_mb<kFmtFp8, 4, 1, 8, 4, false>(a);
    case 6: return launch_stream_mb<kFmtFp8, 8, 1, 6, 4, false>(a);
    case 7: return launch_stream_mb<kFmtFp8, 4, 2, 6, 4, false>(a);
    case 8: return launch_stream_mb<kFmtFp8, 4, 3, 4, 4, false>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace qpn
