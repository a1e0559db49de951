// qpn_pack.hip -- NVFP4 and FP8 pack kernels (FP32 -> codes + scales in the
// packed layout of qpn_common.h), the FP8 -> NVFP4 conversion of a packed
// weight, and the canonical-export / decode kernels used by the parity tests.
//
// Quantisation is "pure round" (lcz.me page, quantisation option table,
// NVFP4-NVIDIA row): round to nearest, ties to the even code, saturating at
// the largest finite value.  Element formats per the lcz.me NVFP4 support
// table (E2M1 codes, UE4M3 scales); FP8 regions stay FP8 (taozi.news page,
// section "v1.1 的关键改进").  Every FP32 step is one IEEE operation in the
// order documented in include/qpn.h; the library is built with contraction
// off and correctly rounded division.
#include <algorithm>

#include "qpn_common.h"
#include "qpn_internal.h"

namespace qpn {

namespace {

// FP32 -> E4M3 code, nearest-even on the FP32 bit pattern, saturating at 448.
__device__ __forceinline__ uint32_t quant_e4m3(float t) {
  const uint32_t u = __float_as_uint(t);
  const uint32_t sign = (u >> 24) & 0x80u;
  const float a = fabsf(t);
  if (!(a == a)) return 0;  // NaN (only 0/0 in degenerate blocks)
  uint32_t code;
  if (a >= 448.0f) {
    code = 0x7E;
  } else if (a < 0.015625f) {
    // below 2^-6 the codes are evenly spaced by 2^-9 (subnormals, then the
    // first normal 0x08); a * 512 is exact and rintf rounds half to even
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // keep 3 mantissa bits: add half an ulp (minus one) plus the kept LSB,
    // then rebias the exponent from 127 to 7
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);
    code = (b >> 20) - (120u << 3);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}

// FP32 -> E2M1 code: count the decision thresholds passed (midpoints between
// neighbours; '>' where the tie goes down to the even code, '>=' where it
// goes up), saturating at 6.
__device__ __forceinline__ uint32_t quant_e2m1(float t) {
  if (!(t == t)) return 0;
  const float a = fabsf(t);
  uint32_t c = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  return c | ((__float_as_uint(t) >> 28) & 8u);
}

// E4M3 code (0x00..0x7E) -> exact FP32 value.
__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, mnt = c & 7u;
  if (e == 0) return (float)mnt * 0.001953125f;  // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (mnt << 20));
}

// With `source` (an FP8 blob being converted) the new header is marked
// invalid (magic 0) unless the source's header describes an FP8 [n, k]
// weight of this layout version; GEMMs then write NaN for the blob.
__global__ void header_kernel(uint8_t* blob, uint32_t fmt, int64_t n, int64_t k,
                              const uint8_t* source) {
  // 64 threads zero the 256-byte header, then thread 0 fills the fields
  reinterpret_cast<uint32_t*>(blob)[threadIdx.x] = 0;
  __syncthreads();
  if (threadIdx.x != 0) return;
  BlobHeader* h = reinterpret_cast<BlobHeader*>(blob);
  bool ok = true;
  if (source != nullptr) {
    const BlobHeader* sh = reinterpret_cast<const BlobHeader*>(source);
    ok = sh->magic == kMagic && sh->format == kFmtFp8 && sh->layout_version == kLayoutVersion &&
         sh->n == n && sh->k == k;
  }
  h->magic = ok ? kMagic : 0u;
  h->format = fmt;
  h->layout_version = kLayoutVersion;
  h->n = n;
  h->k = k;
  h->panels = panels_of(n);
  if (fmt == kFmtNvfp4) {
    h->ksteps = nv_ksteps_of(k);
    h->row_scale_offset = 0;
    h->codes_offset = kHeaderBytes;
    h->total_bytes = nv_blob_bytes(n, k);
  } else {
    h->ksteps = f8_ksteps_of(k);
    h->row_scale_offset = kHeaderBytes;
    h->codes_offset = f8_codes_offset(n);
    h->total_bytes = f8_blob_bytes(n, k);
  }
  h->tensor_scale = 0.0f;
  h->amax_bits = 0;
}

// max |w| over count floats (count % 4 == 0), merged with an unsigned max
// on the FP32 bit pattern, which orders non-negative finite floats.
__global__ __launch_bounds__(256) void amax_kernel(const float* __restrict__ w, int64_t count,
                                                   uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t part[256];
  uint32_t best = 0;
  const int64_t n4 = count / 4;
  const float4* w4 = reinterpret_cast<const float4*>(w);
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 v = w4[i];
    uint32_t a = __float_as_uint(v.x) & 0x7FFFFFFFu;
    uint32_t b = __float_as_uint(v.y) & 0x7FFFFFFFu;
    uint32_t c = __float_as_uint(v.z) & 0x7FFFFFFFu;
    uint32_t d = __float_as_uint(v.w) & 0x7FFFFFFFu;
    a = a > b ? a : b;
    c = c > d ? c : d;
    a = a > c ? a : c;
    best = best > a ? best : a;
  }
  part[threadIdx.x] = best;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s && part[threadIdx.x + s] > part[threadIdx.x])
      part[threadIdx.x] = part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(amax_bits, part[0]);
}

// Where the NVFP4 pack reads its weights: 16 consecutive K elements of one
// row (k0 % 16 == 0, k0 < k) as FP32 values.
struct F32Weights {
  const float* __restrict__ w;
  int64_t k;
  __device__ __forceinline__ void load16(int64_t r, int64_t k0, float v[16]) const {
    const float4* src = reinterpret_cast<const float4*>(w + r * k + k0);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 t = src[q];
      v[4 * q + 0] = t.x;
      v[4 * q + 1] = t.y;
      v[4 * q + 2] = t.z;
      v[4 * q + 3] = t.w;
    }
  }
};

// An FP8 blob as the source of an FP8 -> NVFP4 conversion: the 16 codes are
// one 16-byte lane slot of a chunk, each decoded as E4M3(code) * s_r (one
// FP32 multiply, the exact product rounded once).  NaN codes never occur in
// blobs written by the FP8 pack.
struct Fp8BlobWeights {
  const uint8_t* __restrict__ blob;
  int64_t n;
  __device__ __forceinline__ void load16(int64_t r, int64_t k0, float v[16]) const {
    const float s = reinterpret_cast<const float*>(blob + kHeaderBytes)[r];
    const int64_t f = k0 / 16;
    const int lane = (int)(r % kPanelRows) + 16 * (int)(f % 4);
    const uint8_t* ch = blob + f8_codes_offset(n) +
                        chunk_index(r / kPanelRows, f / 4, panels_of(n)) * kF8ChunkBytes;
    const u32x4 c = *reinterpret_cast<const u32x4*>(ch + 16 * lane);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t code = (c[i / 4] >> (8 * (i % 4))) & 0xFFu;
      const float mag = e4m3_to_f32(code & 0x7Fu);
      v[i] = ((code & 0x80u) ? -mag : mag) * s;
    }
  }
};

// max |w| over the n x k weights of a source, one 16-element block per
// thread-iteration; merged as in amax_kernel.
template <class Src>
__global__ __launch_bounds__(256) void amax_blocks_kernel(Src src, int64_t n, int64_t k,
                                                          uint32_t* __restrict__ amax_bits) {
  __shared__ uint32_t part[256];
  uint32_t best = 0;
  const int64_t per_row = k / 16;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n * per_row;
       i += (int64_t)gridDim.x * 256) {
    float v[16];
    src.load16(i / per_row, 16 * (i % per_row), v);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t a = __float_as_uint(v[e]) & 0x7FFFFFFFu;
      best = best > a ? best : a;
    }
  }
  part[threadIdx.x] = best;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s && part[threadIdx.x + s] > part[threadIdx.x])
      part[threadIdx.x] = part[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x == 0) atomicMax(amax_bits, part[0]);
}

// One thread per 32-code fragment (row r, fragment f of 32 K elements).
template <class Src>
__global__ __launch_bounds__(256) void pack_nvfp4_kernel(Src src, int64_t n, int64_t k,
                                                         uint8_t* __restrict__ blob) {
  BlobHeader* hdr = reinterpret_cast<BlobHeader*>(blob);
  const int64_t P = panels_of(n);
  const int64_t J = nv_ksteps_of(k);
  const int64_t frags_per_row = 4 * J;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= P * kPanelRows * frags_per_row) return;
  const int64_t r = idx / frags_per_row;
  const int64_t f = idx % frags_per_row;

  const float amax = __uint_as_float(hdr->amax_bits);
  const float g = amax / 2688.0f;
  if (idx == 0) hdr->tensor_scale = g;

  uint32_t words[4] = {0, 0, 0, 0};
  uint32_t sc2 = 0;
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t k0 = 32 * f + 16 * b;
    if (r >= n || k0 >= k) continue;  // padding block: zero scale, zero codes
    float v[16];
    src.load16(r, k0, v);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) a = fabsf(v[i]) > a ? fabsf(v[i]) : a;
    uint32_t sc = 0;
    if (g != 0.0f) {
      float ratio = a / 6.0f;
      ratio = ratio / g;
      sc = quant_e4m3(ratio);
    }
    sc2 |= sc << (8 * b);
    const float S = e4m3_to_f32(sc);
    if (S != 0.0f) {
      const float d = S * g;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t q = quant_e2m1(v[i] / d);
        words[2 * b + i / 8] |= q << (4 * (i % 8));
      }
    }
  }
  // chunk (panel, k-step), lane (row in panel, K group)
  const int64_t p = r / kPanelRows;
  const int64_t j = f / 4;
  const int lane = (int)(r % kPanelRows) + 16 * (int)(f % 4);
  uint8_t* ch = blob + kHeaderBytes + chunk_index(p, j, P) * kNvChunkBytes;
  *reinterpret_cast<u32x4*>(ch + 16 * lane) = u32x4{words[0], words[1], words[2], words[3]};
  *reinterpret_cast<uint16_t*>(ch + kNvCodeBytes + 2 * lane) = (uint16_t)sc2;
}

// One block per (padded) row: row amax, row scale, then 16-code fragments.
__global__ __launch_bounds__(256) void pack_fp8_kernel(const float* __restrict__ w, int64_t n,
                                                       int64_t k, uint8_t* __restrict__ blob) {
  __shared__ float part[256];
  const int64_t J = f8_ksteps_of(k);
  const int64_t rows = panels_of(n) * kPanelRows;
  uint8_t* chunks = blob + f8_codes_offset(n);
  // one block per row, striding over the rows (the grid is capped so that
  // the launch stays within the work-item limit at n = 2^24)
  for (int64_t r = blockIdx.x; r < rows; r += gridDim.x) {
    const bool real = r < n;
    float a = 0.0f;
    if (real)
      for (int64_t i = threadIdx.x; i < k; i += 256) a = fmaxf(a, fabsf(w[r * k + i]));
    part[threadIdx.x] = a;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
      if ((int)threadIdx.x < s) part[threadIdx.x] = fmaxf(part[threadIdx.x], part[threadIdx.x + s]);
      __syncthreads();
    }
    const float s = part[0] / 448.0f;
    __syncthreads();  // everyone has read part[0] before the next row reuses it
    if (threadIdx.x == 0) reinterpret_cast<float*>(blob + kHeaderBytes)[r] = s;
    const int64_t p = r / kPanelRows;
    for (int64_t f = threadIdx.x; f < 4 * J; f += 256) {
      uint32_t words[4] = {0, 0, 0, 0};
      if (real && s != 0.0f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t kk = 16 * f + i;
          if (kk < k) words[i / 4] |= quant_e4m3(w[r * k + kk] / s) << (8 * (i % 4));
        }
      }
      const int64_t j = f / 4;
      const int lane = (int)(r % kPanelRows) + 16 * (int)(f % 4);
      uint8_t* ch = chunks + chunk_index(p, j, panels_of(n)) * kF8ChunkBytes;
      *reinterpret_cast<u32x4*>(ch + 16 * lane) = u32x4{words[0], words[1], words[2], words[3]};
    }
  }
}

// ---- canonical export (reads the blob with the GEMM's layout map) --------

__global__ __launch_bounds__(256) void unpack_nvfp4_kernel(const uint8_t* __restrict__ blob,
                                                           int64_t n, int64_t k,
                                                           uint8_t* __restrict__ codes,
                                                           uint8_t* __restrict__ scales,
                                                           float* __restrict__ g) {
  const int64_t J = nv_ksteps_of(k);
  const int64_t fr = (k + 31) / 32;  // fragments per row holding real codes
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx == 0) *g = reinterpret_cast<const BlobHeader*>(blob)->tensor_scale;
  if (idx >= n * fr) return;
  const int64_t r = idx / fr, f = idx % fr;
  const int64_t p = r / kPanelRows, j = f / 4;
  const int lane = (int)(r % kPanelRows) + 16 * (int)(f % 4);
  const uint8_t* ch = blob + kHeaderBytes + chunk_index(p, j, panels_of(n)) * kNvChunkBytes;
  for (int b = 0; b < 16; ++b) {
    const int64_t cb = 16 * f + b;  // canonical byte (2 codes) index in the row
    if (2 * cb < k) codes[r * (k / 2) + cb] = ch[16 * lane + b];
  }
  for (int b = 0; b < 2; ++b) {
    const int64_t blk = 2 * f + b;
    if (16 * blk < k) scales[r * (k / 16) + blk] = ch[kNvCodeBytes + 2 * lane + b];
  }
}

__global__ __launch_bounds__(256) void unpack_fp8_kernel(const uint8_t* __restrict__ blob,
                                                         int64_t n, int64_t k,
                                                         uint8_t* __restrict__ codes,
                                                         float* __restrict__ row_scale) {
  const int64_t J = f8_ksteps_of(k);
  const int64_t fr = (k + 15) / 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx < n) row_scale[idx] = reinterpret_cast<const float*>(blob + kHeaderBytes)[idx];
  if (idx >= n * fr) return;
  const int64_t r = idx / fr, f = idx % fr;
  const int64_t p = r / kPanelRows, j = f / 4;
  const int lane = (int)(r % kPanelRows) + 16 * (int)(f % 4);
  const uint8_t* ch = blob + f8_codes_offset(n) + chunk_index(p, j, panels_of(n)) * kF8ChunkBytes;
  for (int b = 0; b < 16; ++b) {
    const int64_t kk = 16 * f + b;
    if (kk < k) codes[r * k + kk] = ch[16 * lane + b];
  }
}

// ---- the GEMM's own register decode, exported for exhaustive checks -------

__global__ __launch_bounds__(256) void decode_nvfp4_kernel(const uint8_t* __restrict__ codes16,
                                                           const uint8_t* __restrict__ scales2,
                                                           int64_t count,
                                                           uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  u32x4 c;
  for (int q = 0; q < 4; ++q) {
    const uint8_t* s = codes16 + 16 * i + 4 * q;
    c[q] = (uint32_t)s[0] | ((uint32_t)s[1] << 8) | ((uint32_t)s[2] << 16) | ((uint32_t)s[3] << 24);
  }
  const uint32_t sc2 = (uint32_t)scales2[2 * i] | ((uint32_t)scales2[2 * i + 1] << 8);
  half8 a[4];
  decode_nvfp4_fragment(c, sc2, a);
  u32x4* dst = reinterpret_cast<u32x4*>(out + 32 * i);
  for (int t = 0; t < 4; ++t) dst[t] = __builtin_bit_cast(u32x4, a[t]);
}

__global__ __launch_bounds__(256) void decode_fp8_kernel(const uint8_t* __restrict__ codes16,
                                                         int64_t count,
                                                         uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  u32x4 c;
  for (int q = 0; q < 4; ++q) {
    const uint8_t* s = codes16 + 16 * i + 4 * q;
    c[q] = (uint32_t)s[0] | ((uint32_t)s[1] << 8) | ((uint32_t)s[2] << 16) | ((uint32_t)s[3] << 24);
  }
  half8 a[2];
  decode_fp8_fragment(c, a);
  u32x4* dst = reinterpret_cast<u32x4*>(out + 16 * i);
  for (int t = 0; t < 2; ++t) dst[t] = __builtin_bit_cast(u32x4, a[t]);
}

// Streaming-read ceiling: block b reads 2048 consecutive 16-byte units with
// nontemporal loads (eight per thread, all in flight together).
// Streaming read of count16 16-byte units.  A grid-stride loop in which every
// pass of the grid covers one contiguous window (all workgroups read
// neighbouring lines at the same time) with four loads in flight per thread.
// Of the shapes measured on MI355X (one-shot blocks, per-workgroup slabs,
// grid-stride windows; 256 to 2048 workgroups of 256 to 1024 threads), 1024
// workgroups of 512 threads striding over the buffer read a 50 MB buffer
// fastest; on multi-GiB buffers a single pass (one workgroup per window) read
// about 4% faster than the capped grid, so the grid is capped only up to
// kCeilCappedUnits.
constexpr int kCeilThreads = 512;
constexpr int kCeilUnroll = 4;
constexpr int64_t kCeilMaxBlocks = 1024;
constexpr int64_t kCeilCappedUnits = (int64_t)1 << 24;  // 256 MiB

__global__ __launch_bounds__(kCeilThreads) void read_ceiling_kernel(const u32x4* __restrict__ buf,
                                                                    int64_t count16,
                                                                    uint32_t* __restrict__ sink) {
  u32x4 acc = {0, 0, 0, 0};
  const int64_t window = (int64_t)gridDim.x * kCeilThreads * kCeilUnroll;
  for (int64_t b = (int64_t)blockIdx.x * kCeilThreads * kCeilUnroll + threadIdx.x; b < count16;
       b += window) {
    u32x4 v[kCeilUnroll];
#pragma unroll
    for (int u = 0; u < kCeilUnroll; ++u) {
      const int64_t i = b + (int64_t)u * kCeilThreads;
      v[u] = i < count16 ? __builtin_nontemporal_load(buf + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < kCeilUnroll; ++u) acc ^= v[u];
  }
  // The fold is stored only when it equals a fixed value, which keeps the
  // loads alive without tens of thousands of atomics on one word.
  const uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (r == 0x9E3779B9u) *sink = r;
}

inline unsigned blocks_for(int64_t threads) { return (unsigned)((threads + 255) / 256); }

// Grid cap for the row-per-block FP8 pack (it strides over the rows).
constexpr int64_t kMaxPackBlocks = 1 << 16;

}  // namespace

hipError_t launch_pack_nvfp4(const float* w, int64_t n, int64_t k, void* packed, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  uint8_t* blob = (uint8_t*)packed;
  hipLaunchKernelGGL(header_kernel, dim3(1), dim3(64), 0, s, blob, kFmtNvfp4, n, k, nullptr);
  const int64_t count = n * k;
  if (count > 0) {
    int64_t blocks = (count / 4 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)blocks), dim3(256), 0, s, w, count,
                       &reinterpret_cast<BlobHeader*>(blob)->amax_bits);
  }
  const int64_t frags = panels_of(n) * kPanelRows * 4 * nv_ksteps_of(k);
  if (frags > 0)
    hipLaunchKernelGGL(pack_nvfp4_kernel<F32Weights>, dim3(blocks_for(frags)), dim3(256), 0, s,
                       F32Weights{w, k}, n, k, blob);
  return hipGetLastError();
}

hipError_t launch_requant_fp8_to_nvfp4(const void* fp8, int64_t n, int64_t k, void* packed,
                                       void* stream) {
  hipStream_t s = (hipStream_t)stream;
  uint8_t* blob = (uint8_t*)packed;
  const uint8_t* src = (const uint8_t*)fp8;
  hipLaunchKernelGGL(header_kernel, dim3(1), dim3(64), 0, s, blob, kFmtNvfp4, n, k, src);
  const Fp8BlobWeights w{src, n};
  const int64_t units = n * (k / 16);
  if (units > 0) {
    int64_t blocks = (units + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(amax_blocks_kernel<Fp8BlobWeights>, dim3((unsigned)blocks), dim3(256), 0, s,
                       w, n, k, &reinterpret_cast<BlobHeader*>(blob)->amax_bits);
  }
  const int64_t frags = panels_of(n) * kPanelRows * 4 * nv_ksteps_of(k);
  if (frags > 0)
    hipLaunchKernelGGL(pack_nvfp4_kernel<Fp8BlobWeights>, dim3(blocks_for(frags)), dim3(256), 0, s,
                       w, n, k, blob);
  return hipGetLastError();
}

hipError_t launch_pack_fp8(const float* w, int64_t n, int64_t k, void* packed, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  uint8_t* blob = (uint8_t*)packed;
  hipLaunchKernelGGL(header_kernel, dim3(1), dim3(64), 0, s, blob, kFmtFp8, n, k, nullptr);
  const int64_t rows = panels_of(n) * kPanelRows;
  if (rows > 0)
    hipLaunchKernelGGL(pack_fp8_kernel, dim3((unsigned)(rows < kMaxPackBlocks ? rows : kMaxPackBlocks)),
                       dim3(256), 0, s, w, n, k, blob);
  return hipGetLastError();
}

hipError_t launch_unpack_nvfp4(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                               uint8_t* scales, float* g, void* stream) {
  const int64_t t = n * ((k + 31) / 32);
  hipLaunchKernelGGL(unpack_nvfp4_kernel, dim3(blocks_for(t > 0 ? t : 1)), dim3(256), 0,
                     (hipStream_t)stream, (const uint8_t*)packed, n, k, codes, scales, g);
  return hipGetLastError();
}

hipError_t launch_unpack_fp8(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                             float* row_scale, void* stream) {
  int64_t t = n * ((k + 15) / 16);
  if (t < n) t = n;
  hipLaunchKernelGGL(unpack_fp8_kernel, dim3(blocks_for(t > 0 ? t : 1)), dim3(256), 0,
                     (hipStream_t)stream, (const uint8_t*)packed, n, k, codes, row_scale);
  return hipGetLastError();
}

hipError_t launch_decode_nvfp4(const uint8_t* codes16, const uint8_t* scales2, int64_t count,
                               uint16_t* out, void* stream) {
  hipLaunchKernelGGL(decode_nvfp4_kernel, dim3(blocks_for(count)), dim3(256), 0,
                     (hipStream_t)stream, codes16, scales2, count, out);
  return hipGetLastError();
}

hipError_t launch_read_ceiling(const void* buf, int64_t count16, uint32_t* sink, void* stream) {
  const int64_t per_block = (int64_t)kCeilThreads * kCeilUnroll;
  const int64_t needed = (count16 + per_block - 1) / per_block;
  const int64_t blocks = count16 > kCeilCappedUnits ? needed : std::min<int64_t>(kCeilMaxBlocks, needed);
  hipLaunchKernelGGL(read_ceiling_kernel, dim3((unsigned)blocks), dim3(kCeilThreads), 0,
                     (hipStream_t)stream,
                     (const u32x4*)buf, count16, sink);
  return hipGetLastError();
}

hipError_t launch_decode_fp8(const uint8_t* codes16, int64_t count, uint16_t* out, void* stream) {
  hipLaunchKernelGGL(decode_fp8_kernel, dim3(blocks_for(count)), dim3(256), 0,
                     (hipStream_t)stream, codes16, count, out);
  return hipGetLastError();
}

}  // namespace qpn
