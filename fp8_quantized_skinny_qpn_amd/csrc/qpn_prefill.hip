// qpn_prefill.hip -- the same compressed weights against prefill-sized
// activation blocks (M = 9 .. 256 rows) on gfx950.
//
// Y[m, n] = FP16( scale * sum_k X[m, k] * Wq[n, k] ), FP32 accumulation, the
// weights read from the packed blob and decoded in registers exactly as in
// the skinny kernel.  The pages run prefill on FP16 tensor-core tiles and
// name it as the phase where the old card falls furthest behind (lcz.me
// page, "strata" section; aiwitness.kr page, questions section); here it
// is the f16 MFMA with the activation block filling whole 16-column tiles.
// At 2M flops per weight the work turns from HBM-bound (M below ~90 on
// MI355X) to matrix-unit-bound.
//
// Tiles.  A workgroup of eight wavefronts owns one tile: 8 consecutive
// 16-row panels (128 output channels, "narrow") or 16 panels (256 channels,
// "wide"), by a block of 32, 64 or 128 activation rows.  In the narrow tile
// the wavefronts are 4 across the panels by 2 across the rows (each decodes
// 2 panels against half the rows); in the wide tile they stand side by side
// (each decodes 2 panels against all the rows), so a k-step's activation
// slice serves twice the channels.  Each decoded weight fragment feeds one
// MFMA per 16-row activation tile, each activation fragment read from LDS
// feeds 2.  A CU pulls only ~25-30 GB/s from L2 and beyond on MI355X, so the
// bytes a workgroup fetches per k-step set the pace, and the wide tile
// fetches half the activation bytes per channel: it runs above 128 rows
// (two row blocks from 129 rows), at 65-128 rows on large calls and, for
// NVFP4, up to 64 rows when it still gives half the CUs a workgroup (launch
// choice below).  The
// activation slice of a k-step reaches LDS through loads of whole 128-byte
// lines, swizzled so that the MFMA operand reads are free of bank conflicts
// (see issue_x).
//
// Pipeline per k-step c (static wait counts; loads of a wavefront complete
// in order): wait until this wavefront's loads for step c are in; barrier
// (everyone's slice for c is in LDS, and everyone is done reading the stage
// the next slice goes to); send the slice of step c + NS - 1 to its LDS
// stage (direct-to-LDS loads) and the weights of step c + D to the register
// ring; decode step c's weights, MFMAs against the slice in LDS.  The NS
// stages are separate LDS objects and the loop is unrolled by the ring
// length, so the compiler sees that the reads of one stage never alias the
// direct-to-LDS writes of another and keeps the waits exact.
//
// Work split (stream-K).  The (tile, k-step) pairs are cut into contiguous
// ranges, one per workgroup (up to 256, one per CU, when the tiles are
// fewer, and 256 when whole tiles would leave their last round of 256 part
// empty), so every CU streams about the same bytes in a single wave.  A
// workgroup runs its range as pieces, one per tile it touches; where the
// ranges can be whole pieces of one tile each, they are.  The partial
// tiles of a tile cut between workgroups are summed deterministically, up
// a fixed pairwise tree or in shares (see the kernel).
#include <algorithm>

#include "qpn_common.h"
#include "qpn_internal.h"

namespace qpn {

namespace {

template <uint32_t FMT>
struct PFmt;
template <>
struct PFmt<kFmtNvfp4> {
  static constexpr int kKStep = kNvKStep;
  static constexpr int kChunk = kNvChunkBytes;
  static constexpr int kGroups = 4;
};
template <>
struct PFmt<kFmtFp8> {
  static constexpr int kKStep = kF8KStep;
  static constexpr int kChunk = kF8ChunkBytes;
  static constexpr int kGroups = 2;
};

constexpr int kRsrc = 0x00020000;  // raw dword access
constexpr int kTreePieces = 3;     // cut tiles of up to this many pieces use the pairwise tree
constexpr int kPanelsPerBlock = 8;       // narrow tile: 128 output channels per workgroup
constexpr int kWidePanelsPerBlock = 16;  // wide tile: 256 output channels per workgroup
constexpr int kWaves = 4;
// Wavefronts per workgroup.  With four, the accumulators of a 128- or
// 256-row tile fill a SIMD's registers, one wavefront per SIMD, and a wait
// for a load left the SIMD idle: in a per-k-step ablation the MFMA time
// (0.85 us of ~2.5 us per step at 256 rows) added to everything else.  Eight
// wavefronts, each decoding half as many panels, put two on every SIMD:
// 17408x5120 at 256 rows went from 75.4 to 67.3 us, at 128 rows from 52.6
// to 47.4, at 64 rows from 36 to 33.8, at 32 rows from 27.6 to 25.8;
// 5120x17408 at 128 rows from 57.3 to 52.5, FP8 6144x5120 at 256 rows from
// 56.5 to 47.6 us.
constexpr int kWideWaves = 8;  // wavefronts of a 256-channel workgroup (two panels each)
// wavefronts of a 128-channel workgroup of 32 mt rows (8 needs a whole slice
// load per wavefront: 2 mt 16-row tiles x the k-step's 128-byte line pairs)
constexpr int narrow_waves(uint32_t fmt, int mt) { return mt * (fmt == kFmtNvfp4 ? 2 : 1) >= 2 ? 8 : 4; }

template <int N>
__device__ __forceinline__ void pf_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void pf_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

struct PFrag {
  u32x4 codes;
  uint16_t scales;
};

// Slice buffer `I` of a kernel instantiation: one LDS object per stage, so
// the compiler can tell the reads of one stage from the direct-to-LDS
// writes of another and keeps its waits exact.
template <int I, int BYTES>
__device__ __forceinline__ uint8_t* slice_stage() {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[BYTES];
  return buf;
}

}  // namespace

struct PrefillWork {
  int64_t tiles;       // output tiles: channel blocks x row blocks
  int row_blocks;      // blocks of activation rows (WIDE only; 1 otherwise)
  int64_t wgs;         // workgroups; the tiles x k-steps units are cut into wgs equal ranges
  int state_words;     // per cut tile: arrivals, departures, one claim per contributor
  int spin_limit;      // polls of the arrival count before a contributor stops waiting
  float* partial;      // [2 wgs][4 MT fragments][256 threads] float4 partial tiles
  uint32_t* counters;  // [tiles][state_words]; zero between calls
};

// D: k-steps of weights in flight (ring R = D + 1); NS: activation slice
// stages in LDS (2, or R when they fit), the slice being sent NS - 1 steps
// ahead; WIDE: 16 panels x 16 MT rows per workgroup instead of 8 x 32 MT.
// SHARES: cut tiles are summed in shares (else up the pairwise tree).  WV:
// wavefronts per workgroup, 4 or 8 (with 8, each decodes half as many
// panels, so that two wavefronts fit a SIMD).
template <uint32_t FMT, int MT, int D, int NS, bool WIDE, bool SHARES, int WV>
__global__ __launch_bounds__(kLanes * WV) void prefill_gemm_kernel(
    const uint8_t* __restrict__ blob, const uint16_t* __restrict__ x, uint16_t* __restrict__ y,
    int m, int64_t n, int64_t k, PrefillWork pw) {
  using F = PFmt<FMT>;
  constexpr int KS = F::kKStep;
  constexpr int GR = F::kGroups;
  constexpr int WNN = WIDE ? WV : WV / 2;            // wavefronts across panels
  constexpr int PPB = WIDE ? kWidePanelsPerBlock : kPanelsPerBlock;  // panels per workgroup
  constexpr int PW = PPB / WNN;                      // panels per wavefront
  constexpr int MTW = (WV / WNN) * MT;               // 16-row activation tiles per workgroup
  static_assert(PW * WNN == PPB && (WV == 4 || WV == 8), "tile shape");
  constexpr int STAGE = GR * MTW * 1024;             // LDS bytes of one step's slice
  constexpr int XQ = GR * MTW / WV;                  // slice loads per wavefront per step
  constexpr int LPS = FMT == kFmtNvfp4 ? 2 : 1;      // weight loads per chunk
  constexpr int WL = PW * LPS;                       // weight loads per wavefront per step
  constexpr int R = D + 1;
  constexpr int AX = NS - 1;  // slice distance
  // Step c needs slice c and weights c.  Both went out in step c - AX when
  // AX == D (weights second), else the weights went earlier; younger loads
  // are then the AX - 1 whole steps after that (plus, when AX < D, the
  // weights sent together with slice c).
  constexpr int WAITN = (AX < D ? WL : 0) + (AX - 1) * (XQ + WL);
  static_assert(AX >= 1 && AX <= D, "weights go at least as far ahead as slices");
  static_assert(R % NS == 0, "stages repeat within one ring cycle");
  static_assert(WAITN < 64, "vmcnt range");
  static_assert(XQ * WV == GR * MTW, "slice loads split evenly");
  auto stage = [](int c) -> uint8_t* {
    switch (c % NS) {
      case 0: return slice_stage<0, STAGE>();
      case 1: return slice_stage<1, STAGE>();
      case 2: if constexpr (NS > 2) return slice_stage<2, STAGE>(); else return nullptr;
      case 3: if constexpr (NS > 3) return slice_stage<3, STAGE>(); else return nullptr;
      case 4: if constexpr (NS > 4) return slice_stage<4, STAGE>(); else return nullptr;
      default: if constexpr (NS > 5) return slice_stage<5, STAGE>(); else return nullptr;
    }
  };
  static_assert(NS <= 6, "stage objects");

  const int lane = threadIdx.x & (kLanes - 1);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x / kLanes);
  const int wn = wv % WNN, wm = wv / WNN;
  const int64_t P = panels_of(n);
  const int J = (int)((k + KS - 1) / KS);
  // Work units: (tile, k-step) pairs, tile-major; a tile with no k-step
  // (k = 0) still counts one unit, so that its output gets written.
  // Workgroup w owns units [w U / G, (w + 1) U / G); the owner of unit u is
  // ceil((u + 1) G / U) - 1.  A tile whose units fall to several workgroups
  // is summed by the last of them to finish (below).
  const int64_t Jt = J > 0 ? J : 1;
  const int64_t U = pw.tiles * Jt;
  const int64_t G = pw.wgs;
  auto first_unit = [&](int64_t w) -> int64_t { return w * U / G; };
  auto owner = [&](int64_t u) -> int64_t { return ((u + 1) * G + U - 1) / U - 1; };
  // Workgroups go to the 8 XCDs round robin by launch index, and each XCD has
  // its own L2.  Workgroup w (the order of the units above) is launch index
  // p with w = x q + min(x, r) + p / 8, where x = p mod 8, q = G / 8, r = G
  // mod 8 (a bijection): XCD x runs one contiguous block of w.  The pieces of
  // a tile are neighbours in w, so they mostly share an XCD, and the partial
  // tiles one leaves for another pass through that XCD's L2 (7-13% faster on
  // 16 of 23 measured calls at 32-256 rows, none slower).
  const int64_t wg = [&] {
    const int64_t p = blockIdx.x, q8 = G / 8, r8 = G % 8, x = p % 8;
    return x * q8 + (x < r8 ? x : r8) + p / 8;
  }();
  const int64_t u_end = first_unit(wg + 1);

  // ---- header: checked in the epilogue ----
  const __amdgpu_buffer_rsrc_t hres =
      __builtin_amdgcn_make_buffer_rsrc((void*)blob, (short)0, kHeaderBytes, kRsrc);
  const u32x4 hd0 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hres, 0, 0, 0));
  const u32x4 hd1 = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(hres, 16, 0, 0));
  const uint32_t hd2 = __builtin_amdgcn_raw_buffer_load_b32(hres, 48, 0, 0);

  const uint8_t* codes = blob + (FMT == kFmtNvfp4 ? (uint64_t)kHeaderBytes : f8_codes_offset(n));
  const uint64_t sstride = (uint64_t)P * F::kChunk;
  const __amdgpu_buffer_rsrc_t xres =
      __builtin_amdgcn_make_buffer_rsrc((void*)x, (short)0, (int)((int64_t)m * k * 2), kRsrc);
  const int col = lane & 15, kg = lane >> 4;
  const int lq = lane >> 4, lslot = lane & 15;
  constexpr int H = KS / 64;  // 128-byte parts of a row's k-step
  static_assert(XQ * WV == 2 * MTW * H, "one load per 8 rows and 128 bytes");
  // This lane's B operand of MFMA group t in the wave's first activation
  // tile: row 16 (MT wm) + col, piece kg KS / 32 + t of the k-step; the
  // next tile is 2 H loads further (two more row groups, same parity).
  int xoff[GR];
#pragma unroll
  for (int t = 0; t < GR; ++t) {
    const int eg = kg * (KS / 32) + t;
    const int h = eg >> 3, e = eg & 7;
    const int g = 2 * (wm * MT) + (col >> 3);
    const int slot = (2 * (col & 7) + (g & 1) + e) & 15;
    xoff[t] = (g * H + h) * 1024 + (16 * (e >> 1) + slot) * 16;
  }

  for (int64_t u = first_unit(wg); u < u_end;) {
    // ---- this piece: k-steps j0 .. j0 + nj - 1 of one tile ----
    const int64_t tile = u / Jt;
    const int64_t piece_end = min((tile + 1) * Jt, u_end);
    const int j0 = (int)(u - tile * Jt);
    const int nj = J > 0 ? (int)(piece_end - u) : 0;
    const bool later_piece = u != first_unit(wg);
    const bool final_piece = piece_end == u_end;
    u = piece_end;
    const int64_t cblk = tile / pw.row_blocks;
    const int row0 = (int)(tile % pw.row_blocks) * 16 * MTW;
    const int64_t pbase = cblk * PPB + PW * wn;  // first of this wavefront's PW panels
    if (later_piece) {
      // the previous piece's stores are done and every wavefront has
      // finished reading its LDS stages
      pf_wait_vmcnt<0>();
      pf_barrier();
    }

    float4v row_scale[PW] = {};
    if constexpr (FMT == kFmtFp8) {
      // the padded scale area holds 16 P floats; panels past P read zeros
      const __amdgpu_buffer_rsrc_t rres = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(blob + kHeaderBytes), (short)0, (int)(P * kPanelRows * 4), kRsrc);
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        const int64_t r0 = (pbase + i) * kPanelRows + 4 * (lane >> 4);
        const int off = pbase + i < P ? (int)(r0 * 4) : 0x7FFFFFF0;
        row_scale[i] = __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(rres, off, 0, 0));
      }
    }
    asm volatile("" ::: "memory");

    // ---- weights: chunk (p, j) at codes + (j P + p) * chunk bytes ----
    auto issue_w = [&](int c, PFrag (&f)[PW]) {
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        // the address is formed unconditionally (no access happens through a
        // descriptor of size zero), so the load itself never sits behind a branch
        const bool ok = c < nj && pbase + i < P;
        const uint8_t* ch = codes + (uint64_t)(j0 + c) * sstride + (uint64_t)(pbase + i) * F::kChunk;
        const __amdgpu_buffer_rsrc_t r =
            __builtin_amdgcn_make_buffer_rsrc((void*)ch, (short)0, ok ? F::kChunk : 0, kRsrc);
        f[i].codes = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, 16 * lane, 0, 2));
        if constexpr (FMT == kFmtNvfp4)
          f[i].scales = __builtin_amdgcn_raw_buffer_load_b16(r, kNvCodeBytes + 2 * lane, 0, 0);
      }
    };

    // ---- activation slice of step c -> LDS.  Each direct-to-LDS load reads
    // eight whole 128-byte lines: 8 rows x 128 bytes of the step's K.  Load q
    // (1 KiB of LDS) covers rows 8 g .. 8 g + 7 and the h-th 128-byte part of
    // their k-step (g = q / H, h = q % H).  A lane lands at 16 lane bytes of its
    // load; lane 16 qq + slot holds piece e = 2 qq + ((slot - g) & 1) (16 bytes
    // of K) of row 8 g + r, where slot = (2 r + (g & 1) + e) mod 16.  The MFMA
    // operand of lane (col, kg) then sits at a slot that differs for the 16
    // lanes of every read group, so the fragment reads are free of bank
    // conflicts, and each load touches 8 lines instead of 32 (an MFMA fragment
    // itself spans 16 rows and four 16-byte pieces 64 bytes apart).  Rows >= m
    // and K >= k read zeros. ----
    auto issue_x = [&](int c, uint8_t* buf) {
#pragma unroll
      for (int i = 0; i < XQ; ++i) {
        const int q = wv + WV * i;
        const int g = q / H, h = q % H;
        const int e = 2 * lq + ((lslot - g) & 1);
        const int row = row0 + 8 * g + (((lslot - (g & 1) - e) & 15) >> 1);
        const int64_t kpos = (int64_t)(j0 + c) * KS + (h * 8 + e) * 8;
        const bool ok = c < nj && row < m && kpos < k;
        const int off = ok ? (int)(((int64_t)row * k + kpos) * 2) : 0x7FFFFFF0;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            xres, (__attribute__((address_space(3))) void*)(buf + q * 1024), 16, off, 0, 0, 0);
      }
    };

    float4v acc[PW][MT];
#pragma unroll
    for (int i = 0; i < PW; ++i)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[i][t] = float4v{0.f, 0.f, 0.f, 0.f};

    PFrag ring[R][PW];
    // prologue: what steps -D .. -1 would have sent (slice s + AX when it is
    // >= 0, weights s + D), in the same order, so that the wait count at the
    // top of every step is the same.  The scheduler may not move loads across
    // these points.
#pragma unroll
    for (int sidx = -D; sidx < 0; ++sidx) {
      if (sidx + AX >= 0) issue_x(sidx + AX, stage(sidx + AX));
      __builtin_amdgcn_sched_barrier(0);
      issue_w(sidx + D, ring[sidx + D]);
      __builtin_amdgcn_sched_barrier(0);
    }

    auto step = [&](int c, const uint8_t* xread, uint8_t* xnext, PFrag (&cur)[PW], PFrag (&ahead)[PW]) {
      // everything up to this step's slice is in, then everyone's slice is
      // (and everyone is done reading the stage the next slice goes to)
      pf_wait_vmcnt<WAITN>();
      pf_barrier();
      __builtin_amdgcn_sched_barrier(0);
      issue_x(c + AX, xnext);
      __builtin_amdgcn_sched_barrier(0);  // all of the slice before any of the weights
      issue_w(c + D, ahead);
      __builtin_amdgcn_sched_barrier(0);
      if (c >= nj) return;  // padding step: loads only (no memory access)
      half8 a[PW][GR];
#pragma unroll
      for (int i = 0; i < PW; ++i) {
        if constexpr (FMT == kFmtNvfp4)
          decode_nvfp4_fragment(cur[i].codes, (uint32_t)cur[i].scales, a[i]);
        else
          decode_fp8_fragment(cur[i].codes, a[i]);
      }
      // the activation fragments of group t + 1 are read while group t's
      // MFMAs run
      half8 b[2][MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        b[0][mt] = *reinterpret_cast<const half8*>(xread + xoff[0] + mt * 2048 * H);
#pragma unroll
      for (int t = 0; t < GR; ++t) {
        if (t + 1 < GR) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            b[(t + 1) & 1][mt] = *reinterpret_cast<const half8*>(xread + xoff[t + 1] + mt * 2048 * H);
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < PW; ++i)
            acc[i][mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[i][t], b[t & 1][mt], acc[i][mt], 0, 0, 0);
      }
    };

    // unrolled by the ring length (a multiple of the stage count, so stages
    // and ring slots are static) over a whole number of ring cycles; steps
    // past nj only issue size-zero loads, so every wait count is static
    const int nj_pad = ((nj + R - 1) / R) * R;
    for (int c0 = 0; c0 < nj_pad; c0 += R) {
#pragma unroll
      for (int i = 0; i < R; ++i)
        step(c0 + i, stage(i), stage(i + AX), ring[i], ring[(i + D) % R]);
    }
    pf_wait_vmcnt<0>();  // size-zero surplus loads retired

    // ---- output of fragment (i, t): this lane holds output channels 16 p +
    // 4 (lane >> 4) + v (v < 4) of activation row row0 + 16 (MT wm + t) +
    // (lane & 15).  A blob whose header does not match gives NaN. ----
    auto emit = [&](int i, int t, float4v sum) {
      const int64_t n0 = (pbase + i) * kPanelRows + 4 * (lane >> 4);
      const int row = row0 + (wm * MT + t) * 16 + col;
      if (n0 >= n || row >= m) return;
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
      float4v rs = {h_scale, h_scale, h_scale, h_scale};
      if constexpr (FMT == kFmtFp8) {
        rs = row_scale[0];
#pragma unroll
        for (int q = 1; q < PW; ++q)
          if (i == q) rs = row_scale[q];
      }
      uint16_t h[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const _Float16 o = valid ? (_Float16)(rs[v] * sum[v]) : (_Float16)__builtin_nanf("");
        h[v] = __builtin_bit_cast(uint16_t, o);
      }
      uint16_t* dst = y + (int64_t)row * n + n0;
      if ((n & 3) == 0 && (((uintptr_t)y) & 7) == 0 && n0 + 3 < n) {
        *reinterpret_cast<uint2*>(dst) = uint2{(uint32_t)h[0] | ((uint32_t)h[1] << 16),
                                               (uint32_t)h[2] | ((uint32_t)h[3] << 16)};
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v)
          if (n0 + v < n) dst[v] = h[v];
      }
    };

    const int64_t w_first = owner(tile * Jt), w_last = owner(tile * Jt + Jt - 1);
    if (w_first != w_last) {
    // ---- a tile cut between P workgroups (contributors c = w - w_first).
    // Their FP32 partial tiles live in per-workgroup slots: a workgroup's
    // piece of its first tile in slot 2 w, of its last (another tile) in
    // slot 2 w + 1; only a workgroup's first and last piece can be cut.
    // Up to kTreePieces contributors meet pairwise up a fixed binary tree
    // (at each level subtree pos pairs with pos ^ 1, an odd one out passes
    // up): the first to arrive at a node leaves its partial tile in its slot
    // and names the slot in the node's state word; the second adds it (FP32
    // addition is commutative, so the sum does not depend on who came first)
    // and climbs, and the one that leaves the root writes the output.  The
    // contributors of such tiles mostly finish at different times, so a
    // partner is usually there already.  With more contributors, which
    // mostly finish together, each sums a share of the fragments instead (see
    // below).  Readers clear what they read, so the workspace ends all
    // zeros. ----
    constexpr int kDevScope = 16;  // sc1: write-through stores, coherent loads
    constexpr int kTile = kLanes * WV * 16;      // bytes of one fragment of the workgroup
    constexpr int kSlot = PW * MT * kTile;       // bytes of one partial tile
    constexpr int NF = PW * MT;                  // fragments
    const __amdgpu_buffer_rsrc_t pres = __builtin_amdgcn_make_buffer_rsrc(
        (void*)pw.partial, (short)0, (int)(2 * G * kSlot), kRsrc);
    const int mine = (int)threadIdx.x * 16;
    const int P = (int)(w_last - w_first + 1), c = (int)(wg - w_first);
    // a wavefront's own LDS region for staging partial tiles: a stage, or
    // half of one when two wavefronts share it
    constexpr int WPS = (WV + NS - 1) / NS;
    constexpr int WSTAGE = STAGE / WPS;
    static_assert(NS * WPS >= WV, "an LDS region per wavefront");
    if constexpr (!SHARES) {
        const int my_slot = (int)(2 * wg + (first_unit(wg) / Jt == tile ? 0 : 1));
        uint32_t* state = pw.counters + tile * pw.state_words;
        __shared__ int partner_slot;  // -1: this workgroup leaves the tree
        int width = (int)(w_last - w_first + 1), pos = (int)(wg - w_first), node_base = 0;
        bool leave = false;
        while (width > 1) {
          if ((pos ^ 1) < width) {
            uint32_t* node = state + node_base + (pos >> 1);
            pf_barrier();  // every wavefront has read the last partner_slot
            if (threadIdx.x == 0) {
              const uint32_t seen = __hip_atomic_load(node, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              partner_slot = (int)seen - 1;
            }
            __syncthreads();
            int ps = partner_slot;
            bool wrote = false;
            if (ps < 0) {
              // first here as far as this workgroup saw: leave the partial
              // tile, then name it (a partner that got in meanwhile is found
              // by the failed exchange)
#pragma unroll
              for (int i = 0; i < PW; ++i)
#pragma unroll
                for (int t = 0; t < MT; ++t)
                  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][t]), pres,
                                                         my_slot * kSlot + mine + (i * MT + t) * kTile, 0,
                                                         kDevScope);
              pf_wait_vmcnt<0>();
              pf_barrier();
              if (threadIdx.x == 0) {
                uint32_t expected = 0u;
                const bool named = __hip_atomic_compare_exchange_strong(
                    node, &expected, (uint32_t)my_slot + 1u, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                    __HIP_MEMORY_SCOPE_AGENT);
                partner_slot = named ? -1 : (int)expected - 1;
              }
              __syncthreads();
              ps = partner_slot;
              if (ps < 0) {
                leave = true;
                break;
              }
              wrote = true;
            }
            // second: add the partner's partial tile, clear what was written
            float4v v[PW][MT];
#pragma unroll
            for (int i = 0; i < PW; ++i)
#pragma unroll
              for (int t = 0; t < MT; ++t)
                v[i][t] = __builtin_bit_cast(float4v, __builtin_amdgcn_raw_buffer_load_b128(
                                                          pres, ps * kSlot + mine + (i * MT + t) * kTile, 0,
                                                          kDevScope));
            pf_wait_vmcnt<0>();  // read before the slot is cleared
#pragma unroll
            for (int i = 0; i < PW; ++i)
#pragma unroll
              for (int t = 0; t < MT; ++t) acc[i][t] = acc[i][t] + v[i][t];
#pragma unroll
            for (int i = 0; i < PW * MT; ++i)
              __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, pres, ps * kSlot + mine + i * kTile,
                                                     0, 0);
            if (wrote) {
#pragma unroll
              for (int i = 0; i < PW * MT; ++i)
                __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, pres,
                                                       my_slot * kSlot + mine + i * kTile, 0, 0);
            }
            if (threadIdx.x == 0) __hip_atomic_store(node, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          node_base += width >> 1;
          width = (width + 1) >> 1;
          pos >>= 1;
        }
        if (leave) continue;  // uniform over the workgroup
    } else {

    // ---- shares (the other kind of launch): every contributor leaves its partial tile in its slot
    // and counts itself in; then each sums its share of the tile's fragments
    // (f = c, c + P, c + 2 P, ...) over all P partial tiles, in contributor
    // order (deterministic whoever sums it), writes those outputs and clears
    // them in every slot.  Only a contributor on its last piece waits for the
    // others, and only for a bounded time: one that does not wait (or stops
    // waiting) leaves its share unclaimed, and the last one to arrive, which
    // never waits, takes every share still unclaimed.  The last contributor
    // to leave resets the tile's counters. ----
    {
      const int b_first = first_unit(w_first) < tile * Jt ? 1 : 0;  // w_first's side
      auto slot_of = [&](int64_t w) -> int { return (int)(2 * w + (w == w_first ? b_first : 0)) * kSlot; };
      uint32_t* const st = pw.counters + tile * pw.state_words;  // arrivals, departures, claims[P]
      __shared__ uint32_t sh_arrival, sh_claim;

#pragma unroll
      for (int i = 0; i < PW; ++i)
#pragma unroll
        for (int t = 0; t < MT; ++t)
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][t]), pres,
                                                 slot_of(wg) + mine + (i * MT + t) * kTile, 0, kDevScope);
      pf_wait_vmcnt<0>();
      pf_barrier();  // (also: every wavefront is done reading the LDS stages)
      if (threadIdx.x == 0)
        sh_arrival = __hip_atomic_fetch_add(st, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __syncthreads();
      const bool last = sh_arrival == (uint32_t)(P - 1);
      if (threadIdx.x == 0) {
        // only a workgroup's final piece waits: an earlier one has more work
        // to do, and the others of its tile may be waiting for that work
        bool ready = last;
        for (int s = 0; final_piece && !ready && s < pw.spin_limit; ++s) {
          __builtin_amdgcn_s_sleep(2);
          ready = __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) >= (uint32_t)P;
        }
        uint32_t expected = 0u;
        sh_claim = ready && __hip_atomic_compare_exchange_strong(st + 2 + c, &expected, 1u, __ATOMIC_RELAXED,
                                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      __syncthreads();

      // The share of contributor cc, through this wavefront's LDS stage: per
      // round up to `cf` fragments of all P partial tiles, one 1 KiB load per
      // fragment, wavefront and partial tile (each lane reads back only its
      // own 16 bytes).
      uint8_t* const lds = stage(wv / WPS) + (wv % WPS) * WSTAGE;
      auto sum_share = [&](int cc) {
        const int nfs = cc < NF ? (NF - 1 - cc) / P + 1 : 0;
        const int cf = WSTAGE / (P * 1024);  // >= 1: the launch keeps P within the stage
        for (int f0 = 0; f0 < nfs; f0 += cf > 0 ? cf : nfs) {
          const int nj = min(cf, nfs - f0);
          __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): earlier reads of the stage are done
          for (int wi = 0; wi < P; ++wi) {
            const int so = slot_of(w_first + wi) + mine;
            for (int j = 0; j < nj; ++j)
              __builtin_amdgcn_raw_ptr_buffer_load_lds(
                  pres, (__attribute__((address_space(3))) void*)(lds + (wi * cf + j) * 1024), 16,
                  so + (cc + (f0 + j) * P) * kTile, 0, 0, kDevScope);
          }
          pf_wait_vmcnt<0>();
          for (int j = 0; j < nj; ++j) {
            const int f = cc + (f0 + j) * P;
            float4v sum = *reinterpret_cast<const float4v*>(lds + j * 1024 + lane * 16);
            for (int wi = 1; wi < P; ++wi)
              sum += *reinterpret_cast<const float4v*>(lds + (wi * cf + j) * 1024 + lane * 16);
            emit(f / MT, f % MT, sum);
            for (int wi = 0; wi < P; ++wi)
              __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, pres,
                                                     slot_of(w_first + wi) + mine + f * kTile, 0, 0);
          }
        }
      };
      if (sh_claim) sum_share(c);
      if (last) {
        for (int cc = 0; cc < P; ++cc) {
          if (cc == c) continue;
          __syncthreads();  // sh_claim of the previous share has been read
          if (threadIdx.x == 0) {
            uint32_t expected = 0u;
            sh_claim = __hip_atomic_compare_exchange_strong(st + 2 + cc, &expected, 1u, __ATOMIC_RELAXED,
                                                            __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          __syncthreads();
          if (sh_claim) sum_share(cc);
        }
      }
      pf_wait_vmcnt<0>();  // this workgroup's outputs and clears are done
      pf_barrier();
      if (threadIdx.x == 0 &&
          __hip_atomic_fetch_add(st + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(P - 1)) {
        for (int q = 0; q < 2 + P; ++q) __hip_atomic_store(st + q, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    continue;
    }
    }

    // ---- a whole tile, or the root of a tree: the outputs ----
#pragma unroll
    for (int i = 0; i < PW; ++i)
#pragma unroll
      for (int t = 0; t < MT; ++t) emit(i, t, acc[i][t]);
  }
}

// ---------------------------------------------------------------------------
// Launch plumbing
// ---------------------------------------------------------------------------

int prefill_tiles(int m) { return m <= 32 ? 1 : m <= 64 ? 2 : m <= 128 ? 4 : 8; }

// Work split (stream-K).  The tiles x k-steps units are cut into equal
// contiguous ranges, one per workgroup, so that every CU streams the same
// bytes in one wave.  A tile cut between workgroups costs FP32 partial tiles
// written and read back (16 KiB per 32 activation rows and 128 channels).
// Each range is at least kPrefillMinK of K long, and with kPrefillWorkgroups
// or more tiles every workgroup takes whole tiles (no partials; the hardware
// balances the waves).  Measured on MI355X against the earlier equal K
// splits (at most 200 workgroups up to 64 rows, a last arriver reading every
// partial tile): 17408x5120 m = 256 85 -> 74 us, m = 128 59 -> 52 us.  512
// workgroups (two per CU) lost at 32 and 64 rows (28 -> 34 us).
//
// Whole pieces.  A range that straddles two tiles leaves its workgroup two
// partial tiles to write and two shares to sum, and restarts its pipeline.
// So the workgroup count is a multiple c of the tiles wherever that keeps
// the pieces between kPrefillPieceK and kPrefillMaxPieceK of K, and every
// workgroup runs exactly one piece of one tile; c is as large as 256
// workgroups and the shares' LDS staging allow.  The pieces of a tile then
// finish together, so they are summed in shares (above kTreePieces).
// Same-box A/B against equal ranges over 256 workgroups: 5120x17408 at 128
// / 256 rows 52.4 -> 45.4 / 72.1 -> 65.7 us; FP8 6144x5120 at 64 / 128 /
// 256 rows 26.3 -> 21.5 / 36.1 -> 30.0 / 47.4 -> 39.8; FP8 5120x5120 at 32 /
// 64 / 128 / 256 rows 19.7 -> 18.6 / 27.7 -> 20.6 / 35.6 -> 28.3 / 46.1 ->
// 36.9; NVFP4 5120x4096 at 32 / 64 / 128 / 256 rows 18.9 -> 15.6 / 26.1 ->
// 18.5 / 33.4 -> 25.4 / 42.9 -> 37.3; FP8 7168x5120 at 32 / 64 / 256 rows
// 20.8 -> 19.7 / 27.1 -> 22.2 / 51.0 -> 44.5.  With pieces of 512 K (more of
// them) the FP8 5120x5120 and NVFP4 5120x4096 calls were 4-12% slower
// again.  5120x17408 at 32 rows would get four pieces of 4352 K (its 32-row
// shares stage holds four): 160 workgroups, 27.7 -> 29.3 us, hence the
// longest piece.  With 136 or more tiles (17408x5120) only c = 1 fits,
// whole tiles on 136 CUs, which lost to 256 equal ranges (45.4 against 50.9
// us at 128 rows).
//
// The wide tile at up to 64 NVFP4 rows (from 9 rows where the call runs the
// tiled kernel).  Fewer, larger tiles: taken when that launch still has at
// least 128 workgroups.  A/B: 17408x5120 at 32 / 64 rows
// 25.9 -> 22.2 / 34.8 -> 32.4 us; 5120x17408 at 64 rows 37.4 -> 37.0.  At
// 5120x17408 and 32 rows it would have 60 workgroups (three pieces of each
// of 20 tiles, the most its 32-row shares stage holds) and took 37 against
// 28 us; at 128 rows it lost on every shape tried (5120x17408: 45.7 against
// 43.5 us with whole pieces both).
//
// Summing a cut tile: up the pairwise tree, or in shares where the partial
// tiles are 64 KiB or more and a tile is cut more than kTreePieces ways
// (5120x17408 at 128 and 256 rows, FP8 6144x5120 at 256 rows).  There all
// but one contributor finish together, and the tree's levels, each a store,
// a compare-exchange and a load of 64-128 KiB in series, made up a third of
// the time: in shares 5120x17408 m = 128 went from 63 to 57.6 us, m = 256
// from 90 to 80 us, and FP8 6144x5120 m = 256 from 71 to 55.5 us.  With
// small partial tiles, or two or three contributors that finish at
// different times, the tree measured as fast or faster.  Per-lane atomic
// exchanges of the partial tiles (as the skinny kernel's split-K does) were
// 1.3-1.5x slower on every shape: the atomics' throughput, not latency,
// bounds tiles this large.
namespace {

// One tile shape's launch: the workgroup count and the most pieces a tile
// is cut into.
struct PfShape {
  bool wide, shares;
  int mt;
  int64_t rb, tiles, J, G, pieces;
  size_t states, need;
};

PfShape prefill_shape(uint32_t fmt, int m, int64_t n, int64_t k, size_t ws_bytes, bool wide) {
  PfShape sh{};
  sh.wide = wide;
  const int mt = wide ? (m <= 32 ? 2 : m <= 64 ? 4 : 8) : prefill_tiles(m);
  sh.mt = mt;
  sh.rb = (m + 16 * (wide ? mt : 2 * mt) - 1) / (16 * (wide ? mt : 2 * mt));
  const int64_t P = panels_of(n);
  const int64_t ppb = wide ? kWidePanelsPerBlock : kPanelsPerBlock;
  const int64_t tiles = (P + ppb - 1) / ppb * sh.rb;
  sh.tiles = tiles;
  const int64_t ks = fmt == kFmtNvfp4 ? kNvKStep : kF8KStep;
  const int64_t J = fmt == kFmtNvfp4 ? nv_ksteps_of(k) : f8_ksteps_of(k);
  sh.J = J;
  const int64_t Jt = std::max<int64_t>(J, 1);
  const int64_t U = tiles * Jt;
  // one partial tile: 128 or 256 channels x the tile's rows, FP32
  const size_t slot = (size_t)ppb * kPanelRows * 16 * (wide ? mt : 2 * mt) * 4;
  // the most workgroups one tile is cut between, for g workgroups
  auto max_pieces = [&](int64_t g) -> int64_t {
    if (g == tiles) return 1;
    auto owner = [&](int64_t u) { return ((u + 1) * g + U - 1) / U - 1; };
    int64_t p = 1;
    for (int64_t t = 0; t < tiles; ++t) p = std::max<int64_t>(p, owner(t * Jt + Jt - 1) - owner(t * Jt) + 1);
    return p;
  };
  // per cut tile: arrival and departure counts and one claim per
  // contributor; then two partial tiles per workgroup
  auto states = [&](int64_t g) -> size_t { return ((size_t)tiles * (2 + max_pieces(g)) * 4 + 255) / 256 * 256; };
  auto need = [&](int64_t g) -> size_t { return g == tiles ? 0 : states(g) + 2 * (size_t)g * slot; };
  int64_t G = tiles;
  bool whole = false;
  const int64_t target = kPrefillWorkgroups;
  if (J > 0 && tiles < target) {
    const int64_t min_units = std::max<int64_t>(1, kPrefillMinK / ks);
    G = std::max<int64_t>(tiles, std::min<int64_t>(target, U / min_units));
    // A contributor sums its share of a cut tile through its wavefronts' 1
    // KiB-per-partial LDS stages, so at most (stage bytes / 1 KiB)
    // contributors where tiles are summed in shares.
    const int64_t stage_kib = (fmt == kFmtNvfp4 ? 4 : 2) * (wide ? mt : 2 * mt) /
                              (((wide ? kWideWaves : narrow_waves(fmt, mt)) + 3) / 4);
    // Whole pieces: every workgroup takes one piece of one tile (G a
    // multiple of the tiles), as many pieces per tile as 256 workgroups and
    // the staging allow, each at least kPrefillPieceK of K; a range that
    // straddles two tiles leaves two partial tiles to write and sum and
    // restarts the pipeline.  Unless that leaves pieces longer than
    // kPrefillMaxPieceK of K: then equal ranges over all the CUs.
    // 32-row tiles of 128 channels take at most three pieces, summed up the
    // pairwise tree (their small partial tiles make the fix-up latency-bound,
    // and fewer pieces mean fewer round trips): FP8 7168x5120 at 20 / 32 rows
    // 19.3 / 19.8 -> 17.8 / 18.1 us, 6144x5120 18.2 / 18.9 -> 17.0 / 18.1,
    // 5120x4096 at 32 rows 17.1 -> 15.8; NVFP4 5120x4096 and 6144x5120 at 32
    // rows 15.0 / 17.0 -> 13.6 / 15.8.  Two pieces lost (FP8 6144x5120 at 32
    // rows 20.4 us), and at 33-64 rows the cap made no difference or lost.
    const int64_t cmax = !wide && mt == 1 ? std::min<int64_t>(stage_kib, 3) : stage_kib;
    const int64_t c = std::min<int64_t>(std::min<int64_t>(target / tiles, cmax),
                                        std::max<int64_t>(1, J * ks / kPrefillPieceK));
    if (c >= 2 && J * ks <= c * kPrefillMaxPieceK) {
      G = tiles * c;
      whole = true;
    } else if ((wide || mt >= 4) && max_pieces(G) > stage_kib) {
      G = std::max<int64_t>(tiles, tiles * (stage_kib - 1));
    }
  } else if (J > 0 && tiles % target != 0 && U / target >= std::max<int64_t>(1, kPrefillMinK / ks)) {
    // More tiles than CUs: whole tiles leave their last round part empty.
    // Where the rounds are less than 85% full, equal ranges over one round
    // of 256 workgroups (each tile cut between at most two): 34816x5120 at
    // 80 / 128 / 256 rows (272 tiles) went from 99 / 105 / 151 to 75 / 80 /
    // 114 us, 37984x5120 (297) at 128 / 256 rows from 107 / 151 to 90 / 127,
    // FP8 34816x5120 from 101 / 146 to 81 / 117, 49152x5120 (384) from 111 /
    // 165 to 98 / 153, 102400x5120 at 128 rows (800) from 212 to 192; with
    // 1187 tiles (93% full) 2% faster at 128 rows and 6% slower at 256.
    const int64_t rounds = (tiles + target - 1) / target;
    if ((double)tiles < 0.85 * (double)(rounds * target)) G = target;
  }
  if (need(G) > ws_bytes) {
    G = tiles;
    whole = false;
  }
  sh.G = G;
  sh.pieces = max_pieces(G);
  // Summing in shares pays where the contributors mostly finish together:
  // whole pieces, or large partial tiles (128 rows, 256 channels) cut more
  // than kTreePieces ways; otherwise the pairwise tree is cheaper.
  sh.shares = sh.pieces > kTreePieces && (whole || wide || mt >= 4);
  sh.states = states(G);
  sh.need = need(G);
  return sh;
}

}  // namespace

// 9-16 rows: the skinny kernel stages a 16-row slice per workgroup and must
// split K to fit it in LDS; the tiled kernel streams the slice through
// stages and splits K only to fill the CUs.  The tiled kernel (a 32-row tile,
// half of it zeros) measured faster on large calls, the skinny kernel on the
// rest (M = 9 / 16, us, skinny -> tiled): NVFP4 25600x5120 24.9 / 28.3 ->
// 22.3 / 22.9, 65536x5120 46.0 / 51.1 -> 41.2 / 37.4, 20480x17408 63.7 / 66.9
// -> 52.8 / 51.3; FP8 5120x17408 33.0 / 36.1 -> 28.9 / 29.2, 10240x17408 46.0
// / 49.1 -> 43.1 / 43.1, 65536x5120 74.1 / 79.5 -> 68.5 / 66.7; but NVFP4
// 17408x5120 16.7 / 19.2 against 19.3 / 19.1, 5120x17408 19.0 / 21.3 against
// 25.3 / 25.0, FP8 34816x5120 42.1 / 45.7 against 56.3 / 58.0.
bool prefill_on_skinny(uint32_t fmt, int m, int64_t n, int64_t k) {
  if (m > kPrefillSkinnyRows) return false;
  if (m <= kMaxM) return true;
  const int64_t P = panels_of(n);
  if (fmt == kFmtNvfp4) {
    const int64_t J = nv_ksteps_of(k);
    return !(P >= 1536 || (P >= 1024 && J >= 64));
  }
  const int64_t J = f8_ksteps_of(k);
  return !(J >= 128 || P >= 3072);
}

int prefill_launch_for(uint32_t fmt, int m, int64_t n, int64_t k, size_t ws_bytes,
                       PrefillLaunch* out) {
  PfShape sh = prefill_shape(fmt, m, n, k, ws_bytes, m > 128);
  // NVFP4 blocks of up to 64 rows: the 256-channel tile when it still fills
  // half the CUs or more.  65-128 rows: the 256-channel tile when there are
  // more than 128 tiles of 128 channels and it still gives three quarters of
  // the CUs a workgroup (half the activation fetches per channel):
  // 37984x5120 at 128 rows 86 -> 78 us, 49152x5120 99 -> 87, 65536x5120 125
  // -> 106, 151936x5120 279 -> 231, 20480x17408 134 -> 125, FP8 34816x5120
  // at 80 / 128 rows 74 / 72 -> 70 / 68; with fewer tiles it lost
  // (5120x17408 45.7 against 43.5 us), and at 136 tiles (17408x5120) it ties.
  if (fmt == kFmtNvfp4 && m <= 64) {
    const PfShape w = prefill_shape(fmt, m, n, k, ws_bytes, true);
    if (w.G >= kPrefillWorkgroups / 2) sh = w;
  } else if (m > 64 && m <= 128 && sh.tiles > kPrefillWorkgroups / 2) {
    const PfShape w = prefill_shape(fmt, m, n, k, ws_bytes, true);
    if (w.G >= 3 * kPrefillWorkgroups / 4) sh = w;
  }
  // the partial area is addressed with 32-bit offsets
  if (sh.need >= ((size_t)1 << 31)) return kGemmNoWorkspace;
  const int64_t G = sh.G, tiles = sh.tiles, J = sh.J;
  const int mt = sh.mt;
  const bool wide = sh.wide;
  const int64_t rb = sh.rb;
  const int64_t pieces = sh.pieces;
  out->mt = mt;
  out->wide = wide;
  out->row_blocks = (int)rb;
  out->depth = 3;  // as compiled below
  out->tiles = tiles;
  out->ksteps = J;
  out->workgroups = G;
  out->max_pieces = (int)pieces;
  out->state_words = (int)(2 + pieces);
  out->shares = sh.shares;
  out->spin_limit = kPrefillSpinLimit;
  out->ws_counters_offset = 0;
  out->ws_partial_offset = sh.states;
  out->ws_needed = sh.need;
  return kGemmLaunchOk;
}

namespace {

template <uint32_t FMT, int MT, int D, int NS, bool WIDE, bool SHARES, int WV = kWaves>
hipError_t launch_pf(const GemmArgs& a, const PrefillLaunch& l) {
  PrefillWork pw{l.tiles, l.row_blocks, l.workgroups, l.state_words, l.spin_limit, nullptr, nullptr};
  if (l.ws_needed > 0) {
    pw.counters = reinterpret_cast<uint32_t*>((uint8_t*)a.ws + l.ws_counters_offset);
    pw.partial = reinterpret_cast<float*>((uint8_t*)a.ws + l.ws_partial_offset);
  }
  hipLaunchKernelGGL((prefill_gemm_kernel<FMT, MT, D, NS, WIDE, SHARES, WV>), dim3((unsigned)l.workgroups),
                     dim3(kLanes * WV), 0, (hipStream_t)a.stream, (const uint8_t*)a.packed,
                     a.x, a.y, a.m, a.n, a.k, pw);
  return hipGetLastError();
}

template <uint32_t FMT>
hipError_t launch_pf_fmt(const GemmArgs& a, const PrefillLaunch& l) {
  // 3 k-steps of weights ahead; up to 64 rows 4 slice stages measured 3-6%
  // faster than 5 ahead in 6 stages.  The wide tile's 32 KiB slices also fit
  // 4 stages.
  if (l.wide) {
    if constexpr (FMT == kFmtNvfp4) {
      if (l.mt == 2)
        return l.shares ? launch_pf<FMT, 2, 3, 4, true, true, kWideWaves>(a, l)
                        : launch_pf<FMT, 2, 3, 4, true, false, kWideWaves>(a, l);
      if (l.mt == 4)
        return l.shares ? launch_pf<FMT, 4, 3, 4, true, true, kWideWaves>(a, l)
                        : launch_pf<FMT, 4, 3, 4, true, false, kWideWaves>(a, l);
    }
    return l.shares ? launch_pf<FMT, 8, 3, 4, true, true, kWideWaves>(a, l)
                    : launch_pf<FMT, 8, 3, 4, true, false, kWideWaves>(a, l);
  }
  switch (l.mt) {
    case 1:
      return l.shares ? launch_pf<FMT, 1, 3, 4, false, true, narrow_waves(FMT, 1)>(a, l)
                      : launch_pf<FMT, 1, 3, 4, false, false, narrow_waves(FMT, 1)>(a, l);
    case 2:
      return l.shares ? launch_pf<FMT, 2, 3, 4, false, true, narrow_waves(FMT, 2)>(a, l)
                      : launch_pf<FMT, 2, 3, 4, false, false, narrow_waves(FMT, 2)>(a, l);
    default:
      return l.shares ? launch_pf<FMT, 4, 3, 4, false, true, narrow_waves(FMT, 4)>(a, l)
                      : launch_pf<FMT, 4, 3, 4, false, false, narrow_waves(FMT, 4)>(a, l);
  }
}

}  // namespace

hipError_t launch_prefill(uint32_t fmt, const GemmArgs& a, const PrefillLaunch& l) {
  return fmt == kFmtNvfp4 ? launch_pf_fmt<kFmtNvfp4>(a, l) : launch_pf_fmt<kFmtFp8>(a, l);
}

}  // namespace qpn
