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
  uint64_t* keys;  // lm_head only: [m, kArgmaxSlots] argmax keys (atomic max)
  void* ws;        // caller workspace (split-K partials and counters), may be NULL
  void* stream;
};

// One compiled GEMM configuration: W wavefronts per 16-row panel, G panels
// per workgroup, D k-steps of weight loads in flight per wavefront.
// Placement 0 spreads panels thinner (fewer per workgroup) before splitting
// K to reach the wanted workgroup count; placement 1 keeps G panels per
// workgroup and splits K; placement 2 gives every wanted workgroup slot the
// same whole panels and splits only the remainder.
struct GemmPlan {
  int waves_per_panel;
  int panels_per_workgroup;
  int depth;
  int placement;
  int min_workgroups;  // workgroups wanted per launch
  int valu_dot;        // 1: VALU dot products instead of MFMA (diagnostic plans)
};

// Everything one launch needs: the plan plus its K split and workspace use.
struct GemmLaunch {
  int plan;
  int waves_per_panel;
  int panels_per_workgroup;
  int depth;
  int valu_dot;
  int64_t groups;       // panel groups of the split segment
  int splits;           // K ranges per split-segment group
  int split_steps;      // k-steps per K range
  int64_t split_wgs;    // workgroups of the split segment (groups * splits), dispatched first
  int64_t full_panels;  // panels [0, full_panels) taken whole by the other workgroups
  int64_t workgroups;   // grid size
  int slice_steps;      // k-steps of the largest activation slice a workgroup stages
  size_t ws_slots_offset;  // split-K exchange slots (zero between calls)
  size_t ws_needed;     // bytes of workspace this launch uses (from offset 0)
};

// Nodes of the binary tree that sums s split partials pairwise (an odd last
// child moves up a level unchanged): sum over levels of ceil(width / 2).
int split_tree_nodes(int s);

// Activation rows staged per LDS slice for m rows (1, 2, 4 or 8).
int gemm_activation_rows(int m);

// The plan used when none is forced: a pure function of the call's shape.
int gemm_auto_plan(uint32_t fmt, int m, int64_t n, int64_t k);

// Plan `id` (1-based) of the compiled table; false if there is none.
bool gemm_plan_info(int id, GemmPlan* out);

// The launch for plan `plan` (0 = automatic) given `ws_bytes` of workspace
// whose first `ws_offset` bytes are taken; a pure function of its arguments.
constexpr int kGemmLaunchOk = 0;
constexpr int kGemmBadPlan = 1;       // unknown plan id
constexpr int kGemmNoWorkspace = 2;   // K must be split and the workspace is too small
int gemm_launch_for(uint32_t fmt, int m, int64_t n, int64_t k, int plan, size_t ws_bytes,
                    size_t ws_offset, GemmLaunch* out);

// Argmax key slots per activation row: panel p folds its key into slot
// p % kArgmaxSlots with a 64-bit atomic max, so the final pass reads a few
// keys per row instead of one per panel.  The 151936-row lm_head folds
// ~37 panels into each of 256 slots; with 64 slots (~148 per slot) the
// atomics on one address queued behind each other and the M=8 lm_head took
// 3.2 us longer, and with 1024 slots the final pass's reads cost as much.
constexpr int kArgmaxSlots = 256;

// Zero `bytes` (a multiple of 16) of device memory at p (16-byte aligned)
// with a kernel on `stream`: a plain kernel node when captured into a graph.
hipError_t launch_zero_fill(void* p, size_t bytes, void* stream);

// Launch the GEMM (and, with `argmax`, the per-panel argmax keys).
hipError_t launch_gemm(uint32_t fmt, bool argmax, const GemmArgs& a, const GemmLaunch& l);

// Final argmax of the lm_head; with drafts (m - 1 of them) and result (2
// ints) also the greedy verification of the round.  draft and result may
// be NULL together.
hipError_t launch_argmax_finalize(uint64_t* keys, int m, int32_t* argmax, const int32_t* draft,
                                  int32_t* result, void* stream);

// Prefill-sized activation blocks (9 <= m <= 256): one launch of the tiled
// MFMA kernel, 128 output channels by 32 mt activation rows per workgroup up
// to 128 rows, 256 channels by 128-row blocks above (and by 32 or 64 rows
// for NVFP4 blocks of up to 64 rows when that fills half the CUs, and by
// 128 rows at 65-128 rows of large calls).
// Calls of up to kPrefillSkinnyRows rows run the skinny kernel instead, with
// a 16-row activation tile that fills the MFMA's B operand exactly (the
// weights stream once, as at m <= 8), where prefill_on_skinny says so and
// the workspace given holds the K splits its LDS budget needs.
constexpr int kMaxPrefillM = 256;
constexpr int kPrefillSkinnyRows = 16;
constexpr int64_t kPrefillWorkgroups = 256;  // one per CU of an MI355X
constexpr int64_t kPrefillMinK = 512;        // shortest K range of a workgroup
constexpr int64_t kPrefillPieceK = 1024;     // shortest piece of a tile cut into whole pieces
constexpr int64_t kPrefillMaxPieceK = 4096;  // longest such piece (else equal ranges)
constexpr int kPrefillSpinLimit = 1 << 16;   // polls (~1 us each) a contributor waits for a cut tile's others
struct PrefillLaunch {
  int mt;               // 16-row activation tiles per wavefront (workgroup rows: narrow 32 mt, wide 16 mt)
  bool wide;            // 256 channels per workgroup (else 128)
  int row_blocks;       // blocks of 16 mt rows (wide), else 1
  int depth;            // k-steps of weight loads in flight per wavefront
  int64_t tiles;        // output tiles: channel blocks x row blocks
  int64_t ksteps;       // k-steps per tile
  int64_t workgroups;   // equal ranges of the tiles x k-steps units (tiles: whole tiles)
  int max_pieces;       // the most workgroups one tile is cut between
  int state_words;      // per cut tile: arrivals, departures, a claim per contributor
  int spin_limit;       // polls of the arrival count before a contributor stops waiting
  bool shares;          // cut tiles summed in shares (else up the pairwise tree)
  size_t ws_counters_offset;
  size_t ws_partial_offset;
  size_t ws_needed;
};
int prefill_tiles(int m);
// Whether a prefill-sized call of m <= kPrefillSkinnyRows rows runs the
// skinny kernel (else the tiled one).  A pure function of its arguments.
bool prefill_on_skinny(uint32_t fmt, int m, int64_t n, int64_t k);
// A pure function of its arguments; fewer K splits when ws_bytes is short.
int prefill_launch_for(uint32_t fmt, int m, int64_t n, int64_t k, size_t ws_bytes,
                       PrefillLaunch* out);
hipError_t launch_prefill(uint32_t fmt, const GemmArgs& a, const PrefillLaunch& l);

hipError_t launch_pack_nvfp4(const float* w, int64_t n, int64_t k, void* packed, void* stream);
hipError_t launch_pack_fp8(const float* w, int64_t n, int64_t k, void* packed, void* stream);
hipError_t launch_requant_fp8_to_nvfp4(const void* fp8, int64_t n, int64_t k, void* packed,
                                       void* stream);

hipError_t launch_unpack_nvfp4(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                               uint8_t* scales, float* g, void* stream);
hipError_t launch_unpack_fp8(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                             float* row_scale, void* stream);
hipError_t launch_decode_nvfp4(const uint8_t* codes16, const uint8_t* scales2, int64_t count,
                               uint16_t* out, void* stream);
hipError_t launch_decode_fp8(const uint8_t* codes16, int64_t count, uint16_t* out, void* stream);
hipError_t launch_read_ceiling(const void* buf, int64_t count16, uint32_t* sink, void* stream);

}  // namespace qpn
