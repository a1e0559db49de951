// qpn_gemm.hip -- the QPN skinny GEMM and lm_head kernel for gfx950.
//
// Y[m, n] = FP16( scale * sum_k X[m, k] * Wq[n, k] ) for m < M <= 8, with the
// weights read once, compressed, straight from HBM and expanded in registers
// (taozi.news page, section "自研 QPN 内核"; aiwitness.kr page, section
// "내가 실제로 만든 것").  The pages map the 8 verify rows onto Volta's
// 8-row FP16 tensor-core tile; on CDNA4 the matrix unit's narrowest f16 tile
// is 16 wide, so the M <= 8 activation rows fill part of the B operand of a
// 16x16x32 MFMA (the other columns are discarded).  At 2M flops per weight
// the MFMA runs at a few percent of its peak: the kernel is bound by HBM, and
// the MFMA is used because it does the K-reduction across lanes for free and
// leaves the VALU to the decode.
//
// Why this shape (CDNA4 specifics):
//   * Vector memory loads of one wavefront complete in order.  If a compute
//     wavefront also loaded activations, every wait for activation data would
//     also wait for all weight loads issued before it and the weight prefetch
//     would collapse.  So the compute wavefronts issue weight loads only; the
//     activations are staged into LDS by one extra wavefront per workgroup and
//     read back with ds_read (a separate counter).
//   * Every activation row is needed by every 16-row panel.  Staging it once
//     per workgroup into LDS replaces per-panel, per-lane activation loads
//     (which cost more L2->CU bytes than the weights themselves at M = 8).
//   * Weight loads go through buffer descriptors: 32-bit offsets, and, being
//     memory intrinsics, they keep program order in the load queue, so every
//     wait count the compiler derives is exact.
//
// Schedule.  A workgroup owns G consecutive 16-row panels.  Each panel is
// worked on by W compute wavefronts that interleave its k-steps: "window" c is
// k-steps [cW, cW + W), and wavefront w of the panel consumes k-step cW + w.
// The loader wavefront writes window c's activations into LDS ring slot
// c % NB, NB - 1 windows ahead, with direct-to-LDS buffer loads whose
// out-of-range lanes (rows >= m, K >= k) deliver zeros.  One s_barrier per
// window hands a filled slot to the compute wavefronts and a drained one back
// to the loader.  The compute wavefronts keep D windows of weight loads in
// flight (5 VGPRs per k-step); past their last k-step they keep issuing
// loads through a descriptor of size zero (no memory access, zeros back)
// instead of branching, so every wait count is static.  Partial tiles of a
// panel's W wavefronts are summed through LDS in a fixed order, so results
// are deterministic and independent of where a row sits in the matrix.
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
  static constexpr int kGroups = 4;  // MFMAs (8 K values per lane each) per k-step
};
template <>
struct Fmt<kFmtFp8> {
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

// Buffer descriptor word 3 for raw (unswizzled, unformatted) dword access.
constexpr int kRsrcFlags = 0x00020000;

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

// Order-preserving map of an FP16 logit to an unsigned key, lowest column
// winning ties; -0 counts as +0.
__device__ __forceinline__ uint64_t argmax_key(uint16_t h, uint32_t col) {
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

// Bytes of one LDS activation window (padded to whole 1 KiB loader loads).
template <uint32_t FMT, int W, int MB>
constexpr int window_bytes() {
  return ((W * (Fmt<FMT>::kKStep / 8) * MB + 63) / 64) * 1024;
}

template <uint32_t FMT, int W, int G, int D, int NB, int MB, bool ARGMAX>
__global__ __launch_bounds__(kLanes * (G * W + 1)) void skinny_gemm_kernel(
    const uint8_t* __restrict__ blob, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    int m, int64_t n, int64_t k, uint64_t* __restrict__ keys) {
  using F = Fmt<FMT>;
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
  // counts).  Padded windows cost a barrier and an out-of-range load; the
  // loader does nothing in them.  Every wavefront of the workgroup runs the
  // same number of windows, hence of barriers.
  const int nwin = valid ? (J + W - 1) / W : 0;
  const int nwin_pad = ((nwin + R - 1) / R) * R;

  if (wv == NCW) {
    // ---------------- loader wavefront ----------------
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x, (short)0, (int)((int64_t)m * k * 2), kRsrcFlags);
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
  // chunk (p, s) = codes + (s * P + p) * chunk bytes (step-major layout)
  const uint8_t* cbase = blob + (FMT == kFmtNvfp4 ? (uint64_t)kHeaderBytes : f8_codes_offset(n)) +
                         (uint64_t)(active ? p : 0) * F::kChunk;
  const uint64_t sstride = (uint64_t)P * F::kChunk;
  // this wavefront's k-steps are w, w + W, ...; its last valid one:
  const int slast = (J > w) ? w + ((J - 1 - w) / W) * W : 0;
  const bool any_step = active && J > w;

  // One descriptor per load, covering exactly its chunk; past the end of the
  // wavefront's k-steps the descriptor has size zero (no memory access).
  auto issue = [&](int c, WFrag& f) {
    const int s = c * W + w;
    const bool ok = s <= slast;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(cbase + (uint64_t)s * sstride), (short)0, ok ? F::kChunk : 0, kRsrcFlags);
    // aux 2: nontemporal (streamed once)
    f.codes = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * lane, 0, 2));
    if constexpr (FMT == kFmtNvfp4)
      f.scales = __builtin_amdgcn_raw_buffer_load_b16(r, kNvCodeBytes + 2 * lane, 0, 0);
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
      __builtin_amdgcn_sched_barrier(0);
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
        const uint64_t key = argmax_key(h[v], (uint32_t)nn);
        best = key > best ? key : best;
      }
    }
    uint64_t o16 = shfl_xor_u64(best, 16);
    best = o16 > best ? o16 : best;
    uint64_t o32 = shfl_xor_u64(best, 32);
    best = o32 > best ? o32 : best;
    if (lane < 16 && mcol < m) keys[(int64_t)mcol * P + p] = best;
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
// Launch plumbing and the plan table.
// ---------------------------------------------------------------------------
namespace {

// Ring slots actually used: the loader's wait count (vmcnt) is 6 bits wide,
// so wide windows (many loads each) get fewer slots.
constexpr int ring_slots_of(int kstep, int W, int MB, int NB) {
  const int lpw = (W * (kstep / 8) * MB + 63) / 64;
  return (NB - 2) * lpw < 64 ? NB : 2 + 63 / lpw;
}

template <uint32_t FMT, int W, int G, int D, int NB0, int MB, bool ARGMAX>
hipError_t launch_t(const GemmArgs& a) {
  constexpr int NB = ring_slots_of(Fmt<FMT>::kKStep, W, MB, NB0);
  constexpr int WINB = window_bytes<FMT, W, MB>();
  size_t lds = (size_t)NB * WINB;
  const size_t red = (size_t)G * W * kLanes * 16;
  if (lds < red) lds = red;
  const int64_t wgs = (panels_of(a.n) + G - 1) / G;
  hipLaunchKernelGGL((skinny_gemm_kernel<FMT, W, G, D, NB, MB, ARGMAX>), dim3((unsigned)wgs),
                     dim3(kLanes * (G * W + 1)), lds, (hipStream_t)a.stream,
                     (const uint8_t*)a.packed, a.x, a.y, a.m, a.n, a.k, a.keys);
  return hipGetLastError();
}

template <uint32_t FMT, int W, int G, int D, int NB, bool ARGMAX>
hipError_t launch_mb(const GemmArgs& a) {
  switch (gemm_activation_rows(a.m)) {
    case 1: return launch_t<FMT, W, G, D, NB, 1, ARGMAX>(a);
    case 2: return launch_t<FMT, W, G, D, NB, 2, ARGMAX>(a);
    case 4: return launch_t<FMT, W, G, D, NB, 4, ARGMAX>(a);
    default: return launch_t<FMT, W, G, D, NB, 8, ARGMAX>(a);
  }
}

// The compiled plans: (W, G, D, NB).
constexpr GemmPlan kPlans[] = {
    {0, 0, 0, 0},  // 0: automatic
    {4, 1, 4, 8},  // 1
    {4, 2, 4, 4},  // 2
    {4, 3, 4, 8},  // 3
    {4, 2, 4, 6},  // 4
    {8, 1, 4, 8},  // 5
    {2, 4, 4, 8},  // 6
    {4, 2, 6, 4},  // 7
    {4, 1, 6, 8},  // 8
};
constexpr int kNumPlans = sizeof(kPlans) / sizeof(kPlans[0]);

template <uint32_t FMT, bool ARGMAX>
hipError_t launch_plan(const GemmArgs& a, int id) {
  switch (id) {
    case 1: return launch_mb<FMT, 4, 1, 4, 8, ARGMAX>(a);
    case 2: return launch_mb<FMT, 4, 2, 4, 4, ARGMAX>(a);
    case 3: return launch_mb<FMT, 4, 3, 4, 8, ARGMAX>(a);
    case 4: return launch_mb<FMT, 4, 2, 4, 6, ARGMAX>(a);
    case 5: return launch_mb<FMT, 8, 1, 4, 8, ARGMAX>(a);
    case 6: return launch_mb<FMT, 2, 4, 4, 8, ARGMAX>(a);
    case 7: return launch_mb<FMT, 4, 2, 6, 4, ARGMAX>(a);
    case 8: return launch_mb<FMT, 4, 1, 6, 8, ARGMAX>(a);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int gemm_activation_rows(int m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : 8; }

// Automatic plan: a pure function of (format, m, n, k).  Measured on
// MI355X (kernel durations, 17408x5120 and 5120x17408 NVFP4):
//   m <= 2: one panel per workgroup and an 8-window activation ring (the
//     loader's activation loads queue behind the weight misses of its CU,
//     so the ring must be about as deep as the weight prefetch);
//   m <= 4: two panels per workgroup share each staged activation window;
//   m >  4: staging the activations is the bottleneck (every workgroup reads
//     all of X), so panels per workgroup go up as far as the panel count
//     still gives about one workgroup per CU or more.
int gemm_auto_plan(uint32_t fmt, int m, int64_t n, int64_t k) {
  (void)fmt;
  (void)k;
  if (m <= 2) return 1;
  if (m <= 4) return 4;
  return panels_of(n) >= 768 ? 3 : 2;
}

int gemm_ring_slots(uint32_t fmt, int waves_per_panel, int m, int slots) {
  const int ks = fmt == kFmtNvfp4 ? kNvKStep : kF8KStep;
  return ring_slots_of(ks, waves_per_panel, gemm_activation_rows(m), slots);
}

bool gemm_plan_info(int id, GemmPlan* out) {
  if (id < 1 || id >= kNumPlans) return false;
  *out = kPlans[id];
  return true;
}

hipError_t launch_gemm(uint32_t fmt, bool argmax, const GemmArgs& a, int plan) {
  const int id = plan > 0 ? plan : gemm_auto_plan(fmt, a.m, a.n, a.k);
  if (fmt == kFmtNvfp4)
    return argmax ? launch_plan<kFmtNvfp4, true>(a, id) : launch_plan<kFmtNvfp4, false>(a, id);
  if (argmax) return hipErrorInvalidValue;
  return launch_plan<kFmtFp8, false>(a, id);
}

hipError_t launch_argmax_finalize(const uint64_t* keys, int64_t panels, int m, int32_t* argmax,
                                  void* stream) {
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(m), dim3(256), 0, (hipStream_t)stream, keys,
                     panels, argmax);
  return hipGetLastError();
}

}  // namespace qpn
