// qpn_common.h -- packed-blob layout and device helpers shared by the QPN
// kernels (pack, GEMM, lm_head, debug exports).
//
// Packed layout v2 (designed for CDNA4; the pages fix no layout: the taozi.news
// page, section "自研 QPN 内核", only asks that weights stay compressed in HBM
// and are expanded in registers in small pieces).
//
//   Every blob starts with a 256-byte BlobHeader.  Output rows are grouped in
//   panels of 16 rows (the M/N extent of the 16x16x32 f16 MFMA); a panel's K
//   extent is cut into k-steps.  One k-step of one panel is one "chunk": the
//   bytes one wavefront fetches with a single 16-byte-per-lane load, so each
//   load instruction reads 1 KiB of contiguous codes.
//
//   Chunks are stored step-major: chunk (p, j) is number j * P + p, so the
//   chunks of one k-step of all panels are adjacent.  Workgroups that work
//   on neighbouring panels at the same pace then read neighbouring bytes;
//   a panel-major order (each panel's K run contiguous) measured up to 30%
//   slower on gfx950 for the same bytes.
//
//   Lane l of a wavefront owns row (l & 15) of the panel and K group (l >> 4).
//
//   NVFP4, k-step = 128 K elements, chunk = 1152 bytes:
//     bytes [16 l, 16 l + 16): the 32 E2M1 codes of row 16p + (l & 15) at
//         K = 128 j + 32 (l >> 4) + e, e = 0..31, code e in byte e/2, low
//         nibble first;
//     bytes [1024 + 2 l, 1024 + 2 l + 2): the two UE4M3 scales of those 32
//         codes (first for e < 16).
//     Chunk (p, j) starts at 256 + (j * P + p) * 1152, J = ceil(k / 128).
//   FP8, k-step = 64 K elements, chunk = 1024 bytes:
//     bytes [16 l, 16 l + 16): the 16 E4M3 codes of row 16p + (l & 15) at
//         K = 64 j + 16 (l >> 4) + e, code e in byte e;
//     row scales: float[16 P] at byte 256; chunk (p, j) starts at
//     codes_offset + (j * P + p) * 1024.
//   Rows past n and K past k are padding: zero codes and zero scales.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace qpn {

constexpr uint32_t kMagic = 0x314E5051u;  // "QPN1" little-endian
constexpr uint32_t kLayoutVersion = 2;
constexpr uint32_t kFmtNvfp4 = 1;
constexpr uint32_t kFmtFp8 = 2;

constexpr int kHeaderBytes = 256;
constexpr int kPanelRows = 16;
constexpr int kLanes = 64;

constexpr int kNvKStep = 128;
constexpr int kNvCodeBytes = 1024;
constexpr int kNvChunkBytes = 1152;

constexpr int kF8KStep = 64;
constexpr int kF8ChunkBytes = 1024;

constexpr int64_t kMaxN = int64_t(1) << 24;
constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int kMaxM = 8;

struct BlobHeader {
  uint32_t magic;
  uint32_t format;
  uint32_t layout_version;
  uint32_t reserved0;
  int64_t n;
  int64_t k;
  int64_t panels;
  int64_t ksteps;
  float tensor_scale;   // NVFP4 g (written by the pack kernel)
  uint32_t amax_bits;   // NVFP4: max |w| as FP32 bits (pack scratch)
  uint64_t row_scale_offset;
  uint64_t codes_offset;
  uint64_t total_bytes;
  uint8_t pad[256 - 80];
};
static_assert(sizeof(BlobHeader) == kHeaderBytes, "header is 256 bytes");

__host__ __device__ inline int64_t panels_of(int64_t n) { return (n + kPanelRows - 1) / kPanelRows; }
__host__ __device__ inline int64_t nv_ksteps_of(int64_t k) { return (k + kNvKStep - 1) / kNvKStep; }
__host__ __device__ inline int64_t f8_ksteps_of(int64_t k) { return (k + kF8KStep - 1) / kF8KStep; }

// Index of chunk (panel p, k-step j) among the P * J chunks (step-major).
__host__ __device__ inline uint64_t chunk_index(int64_t p, int64_t j, int64_t P) {
  return (uint64_t)j * (uint64_t)P + (uint64_t)p;
}

__host__ __device__ inline uint64_t nv_blob_bytes(int64_t n, int64_t k) {
  return (uint64_t)kHeaderBytes + (uint64_t)panels_of(n) * nv_ksteps_of(k) * kNvChunkBytes;
}
__host__ __device__ inline uint64_t f8_codes_offset(int64_t n) {
  uint64_t rs = (uint64_t)panels_of(n) * kPanelRows * 4;
  return kHeaderBytes + ((rs + 255) / 256) * 256;
}
__host__ __device__ inline uint64_t f8_blob_bytes(int64_t n, int64_t k) {
  return f8_codes_offset(n) + (uint64_t)panels_of(n) * f8_ksteps_of(k) * kF8ChunkBytes;
}

// ---------------------------------------------------------------------------
// Vector types and register decode.
// ---------------------------------------------------------------------------
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Two UE4M3 block scales (low byte first) -> two exact FP16 values.  The
// gfx950 FP8 conversion reads OCP E4M3 (bias 7, max 448); a conversion scale
// of 1.0 leaves the value unscaled, and every E4M3 value is an FP16 normal.
__device__ __forceinline__ half2v ue4m3_pair_to_f16(uint32_t two_bytes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two_bytes, 1.0f, false);
}

// Eight E2M1 codes (one dword, code 0 in the low nibble) times one block
// scale S -> the eight FP16 MFMA operands.  The conversion with scale 1.0
// yields the exact E2M1 values; E2M1 * UE4M3 has at most 6 significant bits
// and lies in [2^-10, 2688], so the FP16 product is exact.
__device__ __forceinline__ half8 decode_e2m1x8(uint32_t c, half2v s) {
  half2v h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0) * s;
  half2v h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1) * s;
  half2v h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2) * s;
  half2v h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3) * s;
  half8 r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

// Eight E4M3 codes (two dwords, byte 0 first) -> eight exact FP16 operands.
__device__ __forceinline__ half8 decode_e4m3x8(uint32_t lo, uint32_t hi) {
  half2v h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  half2v h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  half2v h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  half2v h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  half8 r;
  r[0] = h0[0]; r[1] = h0[1]; r[2] = h1[0]; r[3] = h1[1];
  r[4] = h2[0]; r[5] = h2[1]; r[6] = h3[0]; r[7] = h3[1];
  return r;
}

// One NVFP4 fragment (16 code bytes + 2 scale bytes) -> four 8-operand
// groups, group t holding codes 8t..8t+7.
__device__ __forceinline__ void decode_nvfp4_fragment(u32x4 c, uint32_t sc2, half8 out[4]) {
  half2v s = ue4m3_pair_to_f16(sc2);
  half2v s_lo = {s[0], s[0]};
  half2v s_hi = {s[1], s[1]};
  out[0] = decode_e2m1x8(c[0], s_lo);
  out[1] = decode_e2m1x8(c[1], s_lo);
  out[2] = decode_e2m1x8(c[2], s_hi);
  out[3] = decode_e2m1x8(c[3], s_hi);
}

// One FP8 fragment (16 code bytes) -> two 8-operand groups.
__device__ __forceinline__ void decode_fp8_fragment(u32x4 c, half8 out[2]) {
  out[0] = decode_e4m3x8(c[0], c[1]);
  out[1] = decode_e4m3x8(c[2], c[3]);
}

__device__ __forceinline__ u32x4 load_nt_16(const uint8_t* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

}  // namespace qpn
