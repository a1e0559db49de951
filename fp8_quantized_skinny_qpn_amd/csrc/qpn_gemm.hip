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
// leaves the VALU to the decode.  (A VALU dot-product contraction of the same
// launch shapes, kept as diagnostic plans, measures 2x slower at M = 8 and
// about 15% slower at M = 1 on MI355X.)
//
// Work split.  A workgroup owns G consecutive 16-row panels and one of S
// contiguous K ranges ("splits") of them.  Each panel is worked on by W
// wavefronts that interleave the split's k-steps (wavefront w takes local
// k-steps w, w + W, ...).
//
// Why this shape (CDNA4 specifics):
//   * Every activation row is needed by every panel.  The workgroup stages
//     its split's activation slice X[:, K range] into LDS once, with
//     direct-to-LDS buffer loads spread over all its wavefronts, and all G
//     panels read it from there (ds_read, a separate counter from the weight
//     loads).  Activation traffic from L2 is (panels / G) * M * K * 2 bytes,
//     so at M = 8 G is raised to keep it well below the weight bytes.
//   * Vector memory loads of one wavefront complete in order.  Each
//     wavefront sends its first weight k-step to memory, then its share of
//     the activation loads, then the rest of its weight prefetch; waiting for
//     the activations therefore waits for one weight k-step only (its HBM
//     latency overlaps the L2-served activation reads).  After one barrier
//     the main loop has no barriers and no activation loads at all.
//   * Weight loads go through one buffer descriptor per chunk: 32-bit
//     offsets, and, being memory intrinsics, they keep program order in the
//     load queue, so every wait count the compiler derives is exact.  Past
//     its last k-step a wavefront keeps issuing loads through a descriptor
//     of size zero (no memory access, zeros back) instead of branching, so
//     the ring of D loads in flight has static slots and static waits.
//   * When S > 1, the S partial tiles of a panel meet pairwise up a fixed
//     binary tree over the split index, each pair of accumulators inside one
//     64-bit atomic exchange (step 5): one device-scope round trip per tree
//     level, no arrival counter, barrier or cache maintenance.
//
// The partial tiles of a panel's W wavefronts are summed through LDS in a
// fixed order and splits by a fixed tree of commutative additions, so
// results are deterministic and independent of where a row sits in the
// matrix.
#include <algorithm>

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

// Split-K arguments of one launch (all unused when splits == 1).
struct SplitArgs {
  int splits;            // S: K ranges per panel group
  int split_steps;       // k-steps per K range (the last may be shorter)
  uint64_t* slots;       // [tree nodes][groups][G][64 lanes][2] exchange slots; zero between calls
  int split_wgs;         // workgroups [0, split_wgs) work on K ranges of panels [full_panels, P)
  int full_panels;       // workgroups from split_wgs on take panels [0, full_panels) whole
};

// VDOT selects the contraction: false = the 16x16x32 MFMA; true = VALU dot
// products (v_dot2_f32_f16 per activation row on the decoded weight pairs),
// compiled only as a diagnostic plan to compare the two on identical work.
template <uint32_t FMT, int W, int G, int D, int MB, bool ARGMAX, bool VDOT>
__global__ __launch_bounds__(kLanes * G * W) void skinny_gemm_kernel(
    const uint8_t* __restrict__ blob, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    int m, int64_t n, int64_t k, SplitArgs sp, uint64_t* __restrict__ keys) {
  using F = Fmt<FMT>;
  constexpr int KS = F::kKStep;
  constexpr int GR = F::kGroups;
  constexpr int NW = G * W;                          // wavefronts
  constexpr int LPS = FMT == kFmtNvfp4 ? 2 : 1;      // weight loads per k-step
  constexpr int R = D + 1;                           // weight ring slots
  constexpr int XSTEP = (KS / 8) * MB;               // 16-byte activation units per k-step
  static_assert(NW <= 16, "at most 16 wavefronts");
  static_assert(D * LPS < 64, "wait count");
  // Order of a k-step's activation units in LDS.  Unit xunit(t, kg, mm)
  // feeds MFMA t of lane (mm, kg), i.e. X[mm][kg * KS / 4 + 8 t, + 8).  The
  // plain order (t, kg, mm) makes one 64-lane staging load cover whole
  // 128-byte lines of every row up to 4 rows.  For NVFP4 at 8 rows it would
  // take half of 16 lines (each line then read by two loads); there the
  // order (kg / 2, t, kg % 2, mm) gives each load the first or second 64 K
  // of the k-step, one whole line per row.  At 16 rows the order
  // (kg, t, mm) gives each load 64 contiguous bytes of every row.
  constexpr int XORD = FMT == kFmtNvfp4 && MB == 8 ? 1 : MB == 16 ? 2 : 0;
  constexpr bool XLINE = XORD != 0;
  constexpr int XT = XORD == 1 ? 2 * MB : XORD == 2 ? MB : 4 * MB;  // units between MFMA t and t + 1
  auto xunit = [](int t, int kg, int mm) {
    return XORD == 1   ? (((kg >> 1) * GR + t) * 2 + (kg & 1)) * MB + mm
           : XORD == 2 ? (kg * GR + t) * MB + mm
                       : (t * 4 + kg) * MB + mm;
  };

  extern __shared__ __attribute__((aligned(1024))) uint8_t smem[];
  const int lane = threadIdx.x & (kLanes - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int64_t P = panels_of(n);
  const int J = (int)((k + KS - 1) / KS);
  // Two segments of workgroups.  The first sp.split_wgs split the panels
  // [full_panels, P) into S K ranges each (these are dispatched first and
  // carry the split-K fix-up); the rest take whole panels of [0, full_panels).
  const bool in_split = (int)blockIdx.x < sp.split_wgs;
  const int S = in_split ? sp.splits : 1;
  const int bi = in_split ? (int)blockIdx.x : (int)blockIdx.x - sp.split_wgs;
  const int grp = bi / S;
  const int split = bi % S;
  const int steps = in_split ? sp.split_steps : J;
  const int j0 = split * steps;                          // first k-step of the range
  const int nj = max(0, min(J - j0, steps));             // k-steps in the range

  const int gi = wv / W;  // panel of this wavefront inside the workgroup
  const int w = wv % W;   // its interleave position
  // panel group grp of a segment owns panels [grp * len / groups, (grp + 1) *
  // len / groups) of it: G or fewer, spread evenly so that every workgroup
  // has about the same work
  const int64_t groups = in_split ? sp.split_wgs / S : (int64_t)gridDim.x - sp.split_wgs;
  const int64_t seg0 = in_split ? sp.full_panels : 0;
  const int64_t seglen = in_split ? P - sp.full_panels : sp.full_panels;
  const int64_t pbeg = seg0 + (int64_t)grp * seglen / groups;
  const int64_t pend = seg0 + (int64_t)(grp + 1) * seglen / groups;
  const int64_t p = pbeg + gi;
  const bool active = p < pend;
  const int row = lane & 15, kg = lane >> 4;

  // ---- 0. header and FP8 row scales: loaded now, used in the epilogue, so
  // their latency overlaps the stream instead of adding to the tail ----
  // (vector loads: they join the in-order load queue ahead of the activation
  // loads and are covered by the same wait; scalar loads would be waited for
  // together with the kernel arguments, before anything else is issued)
  const __amdgpu_buffer_rsrc_t hres =
      __builtin_amdgcn_make_buffer_rsrc((void*)blob, (short)0, kHeaderBytes, kRsrcFlags);
  const u32x4 hd0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hres, 0, 0, 0));
  const u32x4 hd1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hres, 16, 0, 0));
  const uint32_t hd2 = __builtin_amdgcn_raw_buffer_load_b32(hres, 48, 0, 0);
  float4v row_scale = {0.f, 0.f, 0.f, 0.f};
  if constexpr (FMT == kFmtFp8) {
    // rows 16 p + 4 (lane >> 4) + v; the padded scale area holds 16 P floats
    const __amdgpu_buffer_rsrc_t rres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(blob + kHeaderBytes), (short)0, (int)(P * kPanelRows * 4), kRsrcFlags);
    const int64_t r0 = (active ? p : 0) * kPanelRows + 4 * (lane >> 4);
    row_scale = __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(
                                                rres, (int)(r0 * 4), 0, 0));
  }
  asm volatile("" ::: "memory");

  // ---- 2. weight prefetch ----
  // chunk (p, j) = codes + (j * P + p) * chunk bytes (step-major layout)
  const uint8_t* cbase = blob + (FMT == kFmtNvfp4 ? (uint64_t)kHeaderBytes : f8_codes_offset(n)) +
                         (uint64_t)(active ? p : 0) * F::kChunk;
  const uint64_t sstride = (uint64_t)P * F::kChunk;
  // this wavefront's local k-steps: w + c W for c < nc
  const int nc = (active && nj > w) ? (nj - w + W - 1) / W : 0;
  const int nc_pad = ((nc + R - 1) / R) * R;

  // One descriptor per load, covering exactly its chunk; past the end of the
  // wavefront's k-steps the descriptor has size zero (no memory access).
  auto issue = [&](int c, WFrag& f) {
    const bool ok = c < nc;
    const int jg = j0 + c * W + w;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(cbase + (uint64_t)(ok ? jg : 0) * sstride), (short)0, ok ? F::kChunk : 0,
        kRsrcFlags);
    // aux 2: nontemporal (streamed once).  The scales too: 5120x4352 went
    // from 5.83 / 7.90 to 5.65 / 7.73 us at M = 1 / 8, the decoder calls
    // within noise (the tiled prefill kernel, 3-4% slower at 128 rows with
    // it, keeps them cached)
    f.codes = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * lane, 0, 2));
    if constexpr (FMT == kFmtNvfp4)
      f.scales = __builtin_amdgcn_raw_buffer_load_b16(r, kNvCodeBytes + 2 * lane, 0, 2);
  };

  WFrag ring[R];
  // the first k-step goes out before the activation loads, the rest after
  issue(0, ring[0]);
  __builtin_amdgcn_sched_barrier(0);

  // ---- 1. activation slice -> LDS (after the first weight k-step) ----
  // Unit jl * XSTEP + xunit(t, kg, mm) (16 bytes) holds X[mm][K .. K + 8),
  // K = (j0 + jl) * KS + kg * KS / 4 + 8 t: what lane (mm, kg) feeds MFMA t
  // of local k-step jl.  Load q of the slice fills units [64 q, 64 q + 64).
  // Rows >= m and K outside the range read zeros (out-of-range buffer
  // offsets).  Offsets stay below 2^25.
  {
    const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)x, (short)0, (int)((int64_t)m * k * 2), kRsrcFlags);
    const int units = nj * XSTEP;
    const int nq = (units + 63) / 64;
    for (int q = wv; q < nq; q += NW) {
      const int u = q * 64 + lane;
      const int mm = u % MB;
      const int rest = u / MB;
      int kpos;
      if constexpr (XORD == 1) {
        const int jl = u / XSTEP;
        const int r = rest % (XSTEP / MB);
        kpos = (j0 + jl) * KS + (2 * (r / (2 * GR)) + (r & 1)) * (KS / 4) + 8 * ((r / 2) % GR);
      } else if constexpr (XORD == 2) {
        const int jl = u / XSTEP;
        const int r = rest % (XSTEP / MB);
        kpos = (j0 + jl) * KS + (r / GR) * (KS / 4) + 8 * (r % GR);
      } else {
        const int jl = rest / (4 * GR);
        kpos = (j0 + jl) * KS + (rest % 4) * (KS / 4) + 8 * ((rest / 4) % GR);
      }
      const bool ok = u < units && mm < m && kpos < k;
      const int off = ok ? (int)(((int64_t)mm * k + kpos) * 2) : 0x7FFFFFF0;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          xres, (__attribute__((address_space(3))) void*)(smem + q * 1024), 16, off, 0, 0, 0);
    }
  }
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);

#pragma unroll
  for (int i = 1; i < D; ++i) {
    issue(i, ring[i]);
    __builtin_amdgcn_sched_barrier(0);
  }
  // this wavefront's first k-step and activation loads are in (older than
  // the other D - 1 weight steps); after the barrier everyone's are
  wait_vmcnt<(D - 1) * LPS>();
  bare_barrier();
  // the header loads were older than the activation loads: they are in
  // (BlobHeader: magic, format, layout_version, reserved, n, k, ..., tensor_scale at 48)
  const uint32_t h_magic = __builtin_amdgcn_readfirstlane(hd0[0]);
  const uint32_t h_format = __builtin_amdgcn_readfirstlane(hd0[1]);
  const uint32_t h_version = __builtin_amdgcn_readfirstlane(hd0[2]);
  const int64_t h_n = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane(hd1[1]) << 32) |
                                __builtin_amdgcn_readfirstlane(hd1[0]));
  const int64_t h_k = (int64_t)(((uint64_t)__builtin_amdgcn_readfirstlane(hd1[3]) << 32) |
                                __builtin_amdgcn_readfirstlane(hd1[2]));
  const float h_scale = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(hd2));
  const bool valid = h_magic == kMagic && h_format == FMT && h_version == kLayoutVersion &&
                     h_n == n && h_k == k;

  // ---- 3. stream ----
  float4v acc = {0.f, 0.f, 0.f, 0.f};
  // activation operand for this lane: row min(row, MB-1) (columns >= m are
  // discarded by the epilogue), K group kg, local step w + c W
  const int xrow = row < MB ? row : MB - 1;
  const uint8_t* xlane =
      XLINE ? smem + (w * XSTEP + xunit(0, kg, xrow)) * 16 : smem + ((w * GR * 4 + kg) * MB + xrow) * 16;
  constexpr int XC = W * XSTEP * 16;  // LDS bytes per interleave round

  // VALU-dot contraction: lane (row, kg) keeps one FP32 sum per activation
  // row over its own K positions, reading all MB rows' units of its K group
  float vacc[MB];
#pragma unroll
  for (int mm = 0; mm < MB; ++mm) vacc[mm] = 0.f;
  const uint8_t* xkg = smem + (w * XSTEP + xunit(0, kg, 0)) * 16;

  auto compute = [&](int c, const WFrag& f) {
    half8 a[GR];
    if constexpr (FMT == kFmtNvfp4)
      decode_nvfp4_fragment(f.codes, (uint32_t)f.scales, a);
    else
      decode_fp8_fragment(f.codes, a);
    if constexpr (VDOT) {
      const uint8_t* xs = xkg + c * XC;
#pragma unroll
      for (int t = 0; t < GR; ++t) {
#pragma unroll
        for (int mm = 0; mm < MB; ++mm) {
          const half8 b = *reinterpret_cast<const half8*>(xs + (t * XT + mm) * 16);
          float sacc = vacc[mm];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sacc = __builtin_amdgcn_fdot2(half2v{a[t][2 * e], a[t][2 * e + 1]},
                                          half2v{b[2 * e], b[2 * e + 1]}, sacc, false);
          vacc[mm] = sacc;
        }
      }
    } else {
      const uint8_t* xs = xlane + c * XC;
#pragma unroll
      for (int t = 0; t < GR; ++t) {
        const half8 b = *reinterpret_cast<const half8*>(xs + t * XT * 16);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], b, acc, 0, 0, 0);
      }
    }
  };

  // At least one ring cycle runs even when this wavefront has no k-steps, so
  // the prologue loads are used on every path and stay ahead of the barrier.
  int c0 = 0;
  do {
#pragma unroll
    for (int i = 0; i < R; ++i) {
      const int c = c0 + i;
      issue(c + D, ring[(i + D) % R]);
      __builtin_amdgcn_sched_barrier(0);
      if (c < nc) compute(c, ring[i]);  // no loads inside: waits unaffected
      __builtin_amdgcn_sched_barrier(0);
    }
    c0 += R;
  } while (c0 < nc_pad);

  if constexpr (VDOT) {
    // sum the four K groups of each row (fixed order), then move the sums
    // into the MFMA tile layout: lane L holds rows 4 (L >> 4) + v of
    // activation row L & 15
#pragma unroll
    for (int mm = 0; mm < MB; ++mm) {
      vacc[mm] += __shfl_xor(vacc[mm], 16, 64);
      vacc[mm] += __shfl_xor(vacc[mm], 32, 64);
    }
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int src = 4 * (lane >> 4) + v;
#pragma unroll
      for (int mm = 0; mm < MB; ++mm) {
        const float t = __shfl(vacc[mm], src, 64);
        if ((lane & 15) == mm) acc[v] = t;
      }
    }
  }

  // ---- 4. fixed-order sum of the W partial tiles of each panel ----
  wait_vmcnt<0>();  // surplus (size-zero) loads retired before the wavefront ends
  bare_barrier();   // every wavefront is done reading activations
  float4v* red = reinterpret_cast<float4v*>(smem);
  if constexpr (W > 1) red[wv * kLanes + lane] = acc;
  wait_lgkmcnt0();
  bare_barrier();
  const bool lead = w == 0;  // this wavefront holds its panel's tile below
  if constexpr (W > 1) {
    if (lead) {
      acc = red[(gi * W) * kLanes + lane];
#pragma unroll
      for (int i = 1; i < W; ++i) acc += red[(gi * W + i) * kLanes + lane];
    }
  }

  if (!lead || !active) return;
  const int mcol = lane & 15;
  const int64_t n0 = p * kPanelRows + 4 * (lane >> 4);

  // ---- 5. split-K: pairwise exchange up a fixed binary tree ----
  // The S partial tiles of a panel are summed by a binary tree over the
  // split index (node (l, i) adds children 2i and 2i + 1 of level l - 1; an
  // odd last child moves up unchanged).  Each node is one 64-bit slot per
  // lane and pair of accumulators.  The two children meet with an atomic
  // exchange of their bit-inverted values: the first to arrive finds the
  // slot at zero and leaves its value there (it is done with that pair);
  // the second gets it back, adds it to its own and climbs on.  FP32
  // addition is commutative, so every node's value, and the result, has the
  // same bits whatever the arrival order.  The data travels inside the
  // atomic itself (agent scope), so no store acknowledgement, arrival
  // counter, barrier or cache maintenance is needed, and every slot is
  // reset to zero by the partner that read it.  An inverted partial is
  // never zero: that would need two FP32 values with all bits set, a NaN
  // pattern no arithmetic produces.
  if (S > 1) {
    const int64_t node_stride = groups * G * kLanes * 2;  // slots per tree node
    uint64_t* const mine = sp.slots + ((int64_t)grp * G + gi) * kLanes * 2 + lane * 2;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      float v0 = acc[2 * q], v1 = acc[2 * q + 1];
      int idx = split, first = 0, width = S;
      bool last = true;
      while (width > 1) {
        const int parents = (width + 1) >> 1;
        if ((idx ^ 1) < width) {
          uint64_t* slot = mine + (int64_t)(first + (idx >> 1)) * node_stride + q;
          const uint64_t val =
              ~(((uint64_t)__builtin_bit_cast(uint32_t, v1) << 32) | __builtin_bit_cast(uint32_t, v0));
          const uint64_t old =
              __hip_atomic_exchange(slot, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (old == 0) {
            last = false;
            break;
          }
          const uint64_t o = ~old;
          v0 = __builtin_bit_cast(float, (uint32_t)o) + v0;
          v1 = __builtin_bit_cast(float, (uint32_t)(o >> 32)) + v1;
          __hip_atomic_store(slot, (uint64_t)0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        idx >>= 1;
        first += parents;
        width = parents;
      }
      if (!last) continue;
      // this lane holds the sums of panel rows 4 (lane >> 4) + 2 q + e
      uint16_t hq[2];
      uint64_t best = 0;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int v = 2 * q + e;
        const int64_t nn = n0 + v;
        const float sc = FMT == kFmtNvfp4 ? h_scale : row_scale[v];
        const _Float16 o = valid ? (_Float16)(sc * (e ? v1 : v0)) : (_Float16)__builtin_nanf("");
        hq[e] = __builtin_bit_cast(uint16_t, o);
        if (mcol < m && nn < n) y[(int64_t)mcol * n + nn] = hq[e];
        if (ARGMAX && nn < n) {
          const uint64_t key = argmax_key(hq[e], (uint32_t)nn);
          best = key > best ? key : best;
        }
      }
      if constexpr (ARGMAX) {
        if (mcol < m && best != 0)
          __hip_atomic_fetch_max(keys + (int64_t)mcol * kArgmaxSlots + (int)(p % kArgmaxSlots), best,
                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    return;
  }

  // ---- 6. epilogue.  Lane holds D[i][j] for j = lane & 15 (activation
  // row) and i = 4 (lane >> 4) + v (panel row). ----
  uint16_t h[4];
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int64_t nn = n0 + v;
    const float sc = FMT == kFmtNvfp4 ? h_scale : row_scale[v];
    _Float16 o = valid ? (_Float16)(sc * acc[v]) : (_Float16)__builtin_nanf("");
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
    if (lane < 16 && mcol < m)
      __hip_atomic_fetch_max(keys + (int64_t)mcol * kArgmaxSlots + (int)(p % kArgmaxSlots), best,
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Final argmax: one workgroup, wavefront r reduces activation row r's key
// slots (and zeroes them).  With drafts, one thread then checks the round:
// row i's argmax is the target's token for position i + 1 and draft[i] the
// drafter's, so the drafts are accepted up to the first mismatch and the
// next token is the target's at that position (result = {accepted, next}).
__global__ __launch_bounds__(kLanes * kMaxM) void argmax_finalize_kernel(
    uint64_t* __restrict__ keys, int m, int32_t* __restrict__ argmax,
    const int32_t* __restrict__ draft, int32_t* __restrict__ result) {
  static_assert(kArgmaxSlots % kLanes == 0, "whole slots per lane");
  __shared__ int32_t best_index[kMaxM];
  const int r = threadIdx.x / kLanes;
  const int lane = threadIdx.x % kLanes;
  if (r < m) {
    uint64_t* row = keys + (int64_t)r * kArgmaxSlots;
    uint64_t best = 0;
#pragma unroll
    for (int i = lane; i < kArgmaxSlots; i += kLanes) {
      const uint64_t v = row[i];
      best = v > best ? v : best;
      row[i] = 0;  // leave the workspace all zeros
    }
#pragma unroll
    for (int off = kLanes / 2; off > 0; off >>= 1) {
      const uint64_t o = shfl_xor_u64(best, off);
      best = o > best ? o : best;
    }
    if (lane == 0) {
      const int32_t idx = (int32_t)(0xFFFFFFFFu - (uint32_t)(best & 0xFFFFFFFFu));
      argmax[r] = idx;
      best_index[r] = idx;
    }
  }
  if (result == nullptr) return;  // uniform over the workgroup
  __syncthreads();
  if (threadIdx.x == 0) {
    int accepted = 0;
    while (accepted < m - 1 && draft[accepted] == best_index[accepted]) ++accepted;
    result[0] = accepted;
    result[1] = best_index[accepted];
  }
}

// ---------------------------------------------------------------------------
// Launch plumbing and the plan table.
// ---------------------------------------------------------------------------
namespace {

// Activation bytes one k-step of a slice occupies in LDS.
int x_step_bytes(uint32_t fmt, int m) {
  return (fmt == kFmtNvfp4 ? kNvKStep : kF8KStep) * gemm_activation_rows(m) * 2;
}

// LDS activation budget per workgroup: two workgroups fit in the 160 KiB of a CU.
constexpr int kSliceBudget = 80 * 1024;

template <uint32_t FMT, int W, int G, int D, int MB, bool ARGMAX, bool VDOT>
hipError_t launch_t(const GemmArgs& a, const GemmLaunch& l) {
  const int xbytes = ((l.slice_steps * (Fmt<FMT>::kKStep / 8) * MB + 63) / 64) * 1024;
  const int red = G * W * kLanes * 16;
  const size_t lds = (size_t)(xbytes > red ? xbytes : red);
  SplitArgs sp{l.splits, l.split_steps, nullptr, (int)l.split_wgs, (int)l.full_panels};
  if (l.splits > 1) sp.slots = reinterpret_cast<uint64_t*>((uint8_t*)a.ws + l.ws_slots_offset);
  hipLaunchKernelGGL((skinny_gemm_kernel<FMT, W, G, D, MB, ARGMAX, VDOT>),
                     dim3((unsigned)l.workgroups), dim3(kLanes * G * W), lds,
                     (hipStream_t)a.stream, (const uint8_t*)a.packed, a.x, a.y, a.m, a.n, a.k, sp,
                     a.keys);
  return hipGetLastError();
}

template <uint32_t FMT, int W, int G, int D, bool ARGMAX, bool VDOT = false>
hipError_t launch_mb(const GemmArgs& a, const GemmLaunch& l) {
  switch (gemm_activation_rows(a.m)) {
    case 1: return launch_t<FMT, W, G, D, 1, ARGMAX, VDOT>(a, l);
    case 2: return launch_t<FMT, W, G, D, 2, ARGMAX, VDOT>(a, l);
    case 4: return launch_t<FMT, W, G, D, 4, ARGMAX, VDOT>(a, l);
    case 8: return launch_t<FMT, W, G, D, 8, ARGMAX, VDOT>(a, l);
    default:  // 16 rows: prefill-sized calls of 9..16 rows, never the lm_head
      if constexpr (ARGMAX) return hipErrorInvalidValue;
      else return launch_t<FMT, W, G, D, 16, false, VDOT>(a, l);
  }
}

// The compiled plans: (W, G, D, placement, workgroups wanted, contraction).
// Plans 11 and 12 repeat plans 2 and 1 with the VALU-dot contraction; the
// automatic choice never uses them.
constexpr GemmPlan kPlans[] = {
    {0, 0, 0, 0, 0},          // 0: automatic
    {4, 1, 4, 0, 128},        // 1
    {3, 5, 3, 0, 192},        // 2
    {4, 2, 6, 0, 192},        // 3
    {8, 1, 3, 2, 256},        // 4
    {4, 1, 4, 2, 256},        // 5
    {4, 1, 10, 0, 256},       // 6
    {8, 1, 5, 0, 256},        // 7
    {3, 5, 14, 0, 256},       // 8
    {4, 4, 10, 0, 256},       // 9
    {3, 4, 4, 2, 256},        // 10
    {3, 5, 3, 0, 192, 1},     // 11: plan 2, VALU dot
    {4, 1, 4, 0, 128, 1},     // 12: plan 1, VALU dot
    {2, 8, 4, 0, 256},        // 13
    {1, 16, 4, 0, 256},       // 14
};
constexpr int kNumPlans = sizeof(kPlans) / sizeof(kPlans[0]);

template <uint32_t FMT, bool ARGMAX>
hipError_t launch_plan(const GemmArgs& a, const GemmLaunch& l) {
  switch (l.plan) {
    case 1: return launch_mb<FMT, 4, 1, 4, ARGMAX>(a, l);
    case 2: return launch_mb<FMT, 3, 5, 3, ARGMAX>(a, l);
    case 3: return launch_mb<FMT, 4, 2, 6, ARGMAX>(a, l);
    case 4: return launch_mb<FMT, 8, 1, 3, ARGMAX>(a, l);
    case 5: return launch_mb<FMT, 4, 1, 4, ARGMAX>(a, l);
    case 6: return launch_mb<FMT, 4, 1, 10, ARGMAX>(a, l);
    case 7: return launch_mb<FMT, 8, 1, 5, ARGMAX>(a, l);
    case 8: return launch_mb<FMT, 3, 5, 14, ARGMAX>(a, l);
    case 9: return launch_mb<FMT, 4, 4, 10, ARGMAX>(a, l);
    case 10: return launch_mb<FMT, 3, 4, 4, ARGMAX>(a, l);
    case 11: return launch_mb<FMT, 3, 5, 3, ARGMAX, true>(a, l);
    case 12: return launch_mb<FMT, 4, 1, 4, ARGMAX, true>(a, l);
    case 13: return launch_mb<FMT, 2, 8, 4, ARGMAX>(a, l);
    case 14: return launch_mb<FMT, 1, 16, 4, ARGMAX>(a, l);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int split_tree_nodes(int s) {
  int nodes = 0;
  for (int width = s; width > 1; width = (width + 1) / 2) nodes += (width + 1) / 2;
  return nodes;
}

int gemm_activation_rows(int m) { return m <= 1 ? 1 : m <= 2 ? 2 : m <= 4 ? 4 : m <= 8 ? 8 : 16; }

// Automatic plan: a pure function of (format, m, n, k).  From kernel-duration
// sweeps on MI355X (NVFP4 17408x5120 and 5120x17408, FP8 6144x5120, warm
// clocks):
//   m <= 2 (FP8: m <= 4): one panel per workgroup, its k-steps interleaved
//     over the wavefronts; activations are a few KiB and cost little.  K is
//     split only until there are 128 workgroups: a split-K fix-up costs
//     more than the CUs it would add (2048x2048 M=1: 128 workgroups 3.75 us
//     against 256 with two splits 5.71 us; FP8 3072x5120 M=1: 5.9 against
//     7.45 us).  When
//     there are 1-3 panels per CU with a remainder (e.g. 320 panels), whole
//     panels alone would leave some CUs with twice the bytes of others, so
//     placement 2 splits only the remainder panels in K (8 wavefronts per
//     panel for NVFP4): 5120x17408 M=1 went from 13.0 to 11.7 us.
//   m > 2: every workgroup reads all of its activation slice from L2, and
//     all workgroups read the same lines, so the slice traffic must be cut:
//     one workgroup per CU, each owning up to five panels (three wavefronts
//     per panel, three k-steps in flight each: 0.2-0.4 us faster than four
//     on every 5-panel headline call) that share one staged slice.  FP8 at m > 4 does best with
//     two panels per workgroup and a six k-step prefetch (0.35-0.4 us
//     faster than ten at 5120-7168x5120 M=8).  Both aim
//     at 192 workgroups rather than one per CU: spreading panels thinner
//     to occupy all 256 CUs costs more slice staging than the extra CUs
//     bring (17408x5120 M=8: 218 workgroups of 5 panels 13.9 us against 256
//     of ~4.25 panels 14.8 us; FP8 1792x5120 M=8: 224 workgroups, 2 splits,
//     8.4 us against 336 workgroups, 3 splits, 10.7 us).
//   NVFP4 m >= 2 with many panels (lm_head-sized N): eight panels per
//     workgroup with two wavefronts each stage the slice once for 8 panels
//     instead of 5 (a third less slice traffic).  It is used when the
//     workgroups it gives fill whole rounds of 256 about as well as the
//     five-panel plan's (0.927 against 0.928 at 151936x5120): 151936x5120
//     M=8 went from 88.6 to 75.8 us, M=4 from 78.4 to 69.0 us, 65536x5120
//     M=8 from 42.3 to 34.3 us, and at M=2 151936x5120 from 72.0 to 67.1 us;
//     with 297 workgroups (37984x5120) it lost, and at M=1 it ties plan 1.
//   NVFP4 m >= 2 with 8-16 panels per CU where neither the eight- nor the
//     five-panel workgroups fill their rounds of 256 CUs to 82%: one
//     workgroup per CU holding all of its panels, one wavefront each, so
//     each CU stages the slice once.  49152x5120 (3072 panels; 615
//     five-panel workgroups fill 80%) at M = 2 / 4 / 8 went from 25.4 / 27.5
//     / 30.6 to 24.3 / 24.8 / 26.1 us.  At 34816x5120 (2176 panels, 85%) it
//     won at M = 8 on one box (23.7 -> 22.0 us) and lost at M = 2 and 4 on
//     another (19.0 -> 20.1, 19.9 -> 21.4), so it is not used there.  Where a
//     plan fills its rounds (2048, 2560, 3968 panels) it lost by 2-7%, and
//     with 4.25 panels per CU (17408x5120 M=8) by 13%: a workgroup of four
//     or five wavefronts hides less latency than fifteen.
namespace {
double round_fill(int64_t workgroups) {  // average / largest workgroups per CU
  const int64_t rounds = (workgroups + 255) / 256;
  return rounds > 0 ? (double)workgroups / (256.0 * (double)rounds) : 1.0;
}
}  // namespace

int gemm_auto_plan(uint32_t fmt, int m, int64_t n, int64_t k) {
  const int64_t P = panels_of(n);
  // The remainder split pays off over a long K (at least 64 k-steps): at 136
  // k-steps (NVFP4 5120x17408 M=1) it saves 1.3 us.  Over a short K it pays
  // off only with two or more panels per CU, where the remainder is a small
  // share, and then with four wavefronts per panel (NVFP4 10240x5120 M=1:
  // 7.9 against 8.4-8.5 us); with ~1.25 panels per CU its fix-up cost more
  // than the balance gained (FP8 5120x1280 M=4: 6.05 against 4.80 us with
  // whole panels; NVFP4 5120x5120 M=1: 7.1 against 6.2).
  const int64_t J = fmt == kFmtNvfp4 ? nv_ksteps_of(k) : f8_ksteps_of(k);
  const bool remainder = P >= 256 && P < 3 * 256 && P % 256 >= 16;
  const bool uneven = remainder && J >= 64;
  // (and a remainder of a quarter round or more: 8704x5120 M=1, 544 panels,
  // ran 8.2 us whole against 8.7-10.0 split; 9216x5120, 576 panels, 8.15
  // split against 8.3 whole)
  const bool uneven_short = remainder && J < 64 && P >= 2 * 256 && P % 256 >= 64;
  // fewer panels than CUs: one panel per workgroup at any m (the slice of a
  // few panels is cheap to stage, and sharing it costs parallelism):
  // 2048x2048 M=8 4.8 us against 7.7 us with five-panel workgroups,
  // NVFP4 1792x5120 M=4 6.6 against 8.2 us, FP8 1792x5120 M=8 7.4 against 8.4
  if (P < 256) return 1;
  if (fmt == kFmtNvfp4) {
    if (m >= 2 && P >= 8 * 256 && P <= 16 * 256 &&
        std::max(round_fill((P + 7) / 8), round_fill((P + 4) / 5)) < 0.82)
      return 14;
    if (m >= 2 && P >= 8 * 256 && round_fill((P + 7) / 8) >= round_fill((P + 4) / 5) - 0.02)
      return 13;
    if (m <= 2) return uneven ? 4 : uneven_short ? 5 : 1;
    // Up to 8 rows over 1-2 panels per CU whose whole activation slice fits
    // the LDS budget: two panels per workgroup, four wavefronts each, six
    // k-steps in flight
    // (more workgroups and deeper prefetch than five-panel workgroups spread
    // this thin): M=8 5120x4352 / 5120x5120 / 6144x5120 / 7168x5120 went from
    // 8.41 / 9.13 / 9.16 / 10.18 to 8.08 / 8.45 / 8.51 / 8.55 us, M=4
    // 6144x5120 from 8.22 to 7.60.  A slice that must be split (4352x8192
    // M=8) took 13.2 against 10.2 us.
    if (m <= 8 && P < 2 * 256 && J * x_step_bytes(fmt, m) <= kSliceBudget) return 3;
    return 2;
  }
  // FP8 above 2 rows: two panels per workgroup over 1-2 panels per CU when
  // the whole slice fits the LDS budget (6144 / 5120 / 7168 x 5120 M=4:
  // 9.05 / 8.72 / 9.66 us with one panel per workgroup -> 8.77 / 8.51 /
  // 9.22); otherwise the five-panel plan, or all of a CU's panels in one
  // workgroup where those fill their rounds poorly, as for NVFP4.  Against
  // one or two panels per workgroup at M = 4 / 8: 8704x5120 13.4 / 15.4 ->
  // 11.2 / 12.3 us, 17408x5120 19.3 / 23.1 -> 17.6 / 18.6, 5120x17408 23.3 /
  // 25.5 -> 20.2 / 20.9, 37984x5120 38.1 / 40.6 -> 32.4 / 34.0, 49152x5120
  // 43.3 / 47.5 -> 39.9 / 41.1 (sixteen panels).
  // At 9-16 rows (prefill-sized calls with a 16-row tile) two panels per
  // workgroup stay best below 512 panels, whether or not the slice fits; from
  // 512 the five- or sixteen-panel plans (M = 9 / 16: 17408x5120 29.2 / 33.3
  // -> 23.0 / 24.9 us, 34816x5120 52.2 / 58.9 -> 42.1 / 45.7, 10240x17408
  // 58.5 / 64.2 -> 46.0 / 49.1).
  if (m <= 2) return uneven || uneven_short ? 5 : 1;
  if (m <= 8 && P < 2 * 256 && J * x_step_bytes(fmt, m) <= kSliceBudget) return 3;
  if (m > 8 && P < 2 * 256) return 3;
  if (P >= 8 * 256 && P <= 16 * 256 &&
      std::max(round_fill((P + 7) / 8), round_fill((P + 4) / 5)) < 0.82)
    return 14;
  return 2;
}

bool gemm_plan_info(int id, GemmPlan* out) {
  if (id < 1 || id >= kNumPlans) return false;
  *out = kPlans[id];
  return true;
}

// Splits for a plan: the fewest K ranges whose activation slice fits the LDS
// budget, then more (while each wavefront keeps >= 2 k-steps per range) until
// there are at least the plan's wanted number of workgroups.  Splits > 1 need workspace;
// with less of it the launch uses fewer splits, down to the fewest that fit
// LDS (kGemmNoWorkspace when even those do not fit the workspace).
int gemm_launch_for(uint32_t fmt, int m, int64_t n, int64_t k, int plan, size_t ws_bytes,
                    size_t ws_offset, GemmLaunch* out) {
  GemmPlan pl;
  const int id = plan > 0 ? plan : gemm_auto_plan(fmt, m, n, k);
  if (!gemm_plan_info(id, &pl)) return kGemmBadPlan;
  const int64_t P = panels_of(n);
  const int64_t J = fmt == kFmtNvfp4 ? nv_ksteps_of(k) : f8_ksteps_of(k);
  // Panel groups per K range: enough to give every CU a workgroup when the
  // panel count allows it, with at most G panels each (spread evenly).
  int64_t groups = (P + pl.panels_per_workgroup - 1) / pl.panels_per_workgroup;
  const int64_t xs = x_step_bytes(fmt, m);
  const int64_t want = pl.min_workgroups;
  auto steps_of = [&](int64_t s) { return J > 0 ? (J + s - 1) / s : 1; };
  // fewest splits whose slice fits the budget
  int64_t smin = J > 0 ? (J * xs + kSliceBudget - 1) / kSliceBudget : 1;
  if (smin < 1) smin = 1;
  if (smin > J && J > 0) smin = J;
  int64_t S = smin;
  // exchange slots: one 1 KiB tile (64 lanes x two 64-bit slots) per panel
  // per node of the split tree
  auto need_for = [&](int64_t s, int64_t g) -> size_t {
    if (s <= 1) return 0;
    return (size_t)split_tree_nodes((int)s) * g * pl.panels_per_workgroup * kLanes * 16;
  };
  // the kernel addresses the workspace with 32-bit offsets: a split launch
  // must fit below 2^31 bytes (and the given workspace)
  auto fits = [&](int64_t s, int64_t g) {
    const size_t need = ws_offset + need_for(s, g);
    return s <= 1 || (need <= ws_bytes && need < ((size_t)1 << 31));
  };
  // Placement 2: every wanted workgroup slot (one per CU) gets the same
  // number of whole panels, and the remainder panels are split in K into
  // about one more workgroup per slot, so that every CU streams the same
  // bytes.  The split workgroups come first in dispatch order.
  if (pl.placement == 2 && smin == 1 && J > 0) {
    const int64_t G = pl.panels_per_workgroup;
    const int64_t q = P / (want * G);
    const int64_t full = q * want * G;
    const int64_t rem = P - full;
    if (q >= 1 && rem > 0) {
      const int64_t gs = rem;  // one remainder panel per split group
      int64_t s0 = std::max<int64_t>(1, (want + gs / 2) / gs);
      s0 = std::min<int64_t>(s0, std::max<int64_t>(1, J / (2 * pl.waves_per_panel)));
      const int64_t st0 = steps_of(s0);
      s0 = (J + st0 - 1) / st0;
      if (fits(s0, gs)) {
        out->plan = id;
        out->waves_per_panel = pl.waves_per_panel;
        out->panels_per_workgroup = pl.panels_per_workgroup;
        out->depth = pl.depth;
        out->valu_dot = pl.valu_dot;
        out->groups = gs;
        out->splits = (int)s0;
        out->split_steps = (int)st0;
        out->split_wgs = gs * s0;
        out->full_panels = full;
        out->workgroups = gs * s0 + full / G;
        out->slice_steps = (int)J;
        out->ws_slots_offset = ws_offset;
        out->ws_needed = ws_offset + need_for(s0, gs);
        return kGemmLaunchOk;
      }
    }
  }
  // placement 0 spreads the panels thinner (down to one per workgroup)
  // before splitting K further; placement 1 keeps every workgroup's G panel
  // slots filled and splits K instead.
  // Shared-slice plans whose K the LDS budget already splits: when twice
  // the splits of G-panel groups still fit in one workgroup per CU (256),
  // take them instead of spreading panels thinner.  Each workgroup then
  // stages half the activation slice for the same weight bytes, and the
  // per-CU fetch is what sets the pace: 5120x17408 at M = 4 (S = 2 -> 4, 192
  // -> 256 workgroups of five panels) went from 14.95 to 13.77 us on one box
  // and measured the same either way (14.7-15.1 us) on another.
  if (pl.placement == 0 && pl.panels_per_workgroup > 2 && S > 1 && groups * S < want &&
      groups * 2 * S <= 256 && (J + 2 * S - 1) / (2 * S) >= 2 * pl.waves_per_panel)
    S *= 2;
  else if (pl.placement == 0 && groups * S < want)
    groups = std::min<int64_t>(P, (want + S - 1) / S);
  if (groups < 1) groups = 1;
  while (groups * S < want && (J + S) / (S + 1) >= 2 * pl.waves_per_panel) ++S;
  auto need = [&](int64_t s) -> size_t { return need_for(s, groups); };
  while (S > smin && !fits(S, groups)) --S;
  if (!fits(S, groups)) return kGemmNoWorkspace;
  const int64_t steps = steps_of(S);
  S = J > 0 ? (J + steps - 1) / steps : 1;  // drop empty trailing ranges
  out->plan = id;
  out->waves_per_panel = pl.waves_per_panel;
  out->panels_per_workgroup = pl.panels_per_workgroup;
  out->depth = pl.depth;
  out->valu_dot = pl.valu_dot;
  out->groups = groups;
  out->splits = (int)S;
  out->split_steps = (int)steps;
  out->split_wgs = groups * S;
  out->full_panels = 0;
  out->workgroups = groups * S;
  out->slice_steps = (int)steps;
  out->ws_slots_offset = ws_offset;
  out->ws_needed = ws_offset + need(S);
  return kGemmLaunchOk;
}

hipError_t launch_gemm(uint32_t fmt, bool argmax, const GemmArgs& a, const GemmLaunch& l) {
  if (fmt == kFmtNvfp4)
    return argmax ? launch_plan<kFmtNvfp4, true>(a, l) : launch_plan<kFmtNvfp4, false>(a, l);
  if (argmax) return hipErrorInvalidValue;
  return launch_plan<kFmtFp8, false>(a, l);
}

namespace {
__global__ __launch_bounds__(256) void zero_fill_kernel(u32x4* __restrict__ p, int64_t count16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count16; i += stride)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}
}  // namespace

hipError_t launch_zero_fill(void* p, size_t bytes, void* stream) {
  const int64_t count16 = (int64_t)(bytes / 16);
  const int64_t blocks = std::min<int64_t>(1024, (count16 + 255) / 256);
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                     (u32x4*)p, count16);
  return hipGetLastError();
}

hipError_t launch_argmax_finalize(uint64_t* keys, int m, int32_t* argmax, const int32_t* draft,
                                  int32_t* result, void* stream) {
  hipLaunchKernelGGL(argmax_finalize_kernel, dim3(1), dim3(kLanes * m), 0, (hipStream_t)stream,
                     keys, m, argmax, draft, result);
  return hipGetLastError();
}

}  // namespace qpn
