// qpn_api.cpp -- the C ABI declared in include/qpn.h: host-side argument
// checks, plan selection and launches.  Every check runs before anything is
// enqueued; nothing here allocates, copies, synchronises or prints.
#include "qpn.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "qpn_common.h"
#include "qpn_internal.h"

namespace {

using namespace qpn;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

bool nv_shape_ok(int64_t n, int64_t k) {
  return n >= 0 && k >= 0 && n <= kMaxN && k <= kMaxK && k % 16 == 0;
}
bool f8_shape_ok(int64_t n, int64_t k) {
  return n >= 0 && k >= 0 && n <= kMaxN && k <= kMaxK && k % 8 == 0;
}

// The library's own scratch for callers that cannot allocate
// (qpn_gemm_nvfp4_noalloc): split-K partials and counters in a file-scope
// device array.  Each GPU the library runs on holds its own copy, at its
// own address, until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: only the address that
// hipGetSymbolAddress returns for each device (g_scratch) is passed to
// kernels.  It starts zero-filled (static storage) and every call leaves it
// zero-filled, as any workspace.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device check and set-up, once per device id with that device current:
// the device must be gfx950, and the device address of `scratch` is
// looked up.  Every entry point runs it before anything is enqueued.
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
int g_ok[kMaxDevices];
void* g_scratch[kMaxDevices];  // device address of `scratch` on each device (NULL if unknown)
std::once_flag g_scratch_cleared[kMaxDevices];

int device_check() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return QPN_ERR_DEVICE;
  std::call_once(g_once[dev], [dev]() {
    hipDeviceProp_t prop;
    g_ok[dev] = 0;
    if (hipGetDeviceProperties(&prop, dev) == hipSuccess &&
        std::strncmp(prop.gcnArchName, "gfx950", 6) == 0)
      g_ok[dev] = 1;
    void* p = nullptr;
    if (g_ok[dev] && hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess &&
        p != nullptr && ((uintptr_t)p % 256) == 0)
      g_scratch[dev] = p;
    else
      (void)hipGetLastError();  // no scratch: only the no-allocation entry point reports it
  });
  return g_ok[dev] ? QPN_OK : QPN_ERR_DEVICE;
}

int launch_status(hipError_t e) { return e == hipSuccess ? QPN_OK : QPN_ERR_LAUNCH; }

// Bytes of lm_head argmax keys at the start of its workspace, and where the
// split-K area starts after them.
size_t lmhead_keys_bytes(int m, int64_t n) {
  (void)n;
  return (size_t)8 * (size_t)m * (size_t)kArgmaxSlots;
}
size_t lmhead_split_offset(int m, int64_t n) { return (lmhead_keys_bytes(m, n) + 255) / 256 * 256; }

int gemm_common_checks(uint32_t fmt, const void* packed, const uint16_t* x, const void* y,
                       int m, int64_t n, int64_t k) {
  if (m < 0 || m > kMaxM) return QPN_ERR_SHAPE;
  if (!(fmt == kFmtNvfp4 ? nv_shape_ok(n, k) : f8_shape_ok(n, k))) return QPN_ERR_SHAPE;
  if (m == 0 || n == 0) return QPN_OK;  // empty call: nothing is read or written
  if (!packed || (!x && k > 0) || !y) return QPN_ERR_NULL;
  if (!aligned(packed, 256) || !aligned(x, 16) || !aligned(y, 2)) return QPN_ERR_ALIGN;
  return QPN_OK;
}

// plan: 0 = the automatic choice; otherwise a compiled plan id (diagnostics).
int gemm_entry(uint32_t fmt, int plan, const void* packed, const uint16_t* x, uint16_t* y, int m,
               int64_t n, int64_t k, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = gemm_common_checks(fmt, packed, x, y, m, n, k);
  if (rc != QPN_OK) return rc;
  if (m == 0 || n == 0) return QPN_OK;
  if (workspace && !aligned(workspace, 8)) return QPN_ERR_ALIGN;
  rc = device_check();
  if (rc != QPN_OK) return rc;
  GemmLaunch l;
  const int lr = gemm_launch_for(fmt, m, n, k, plan, workspace ? workspace_bytes : 0, 0, &l);
  if (lr != kGemmLaunchOk) return lr == kGemmNoWorkspace ? QPN_ERR_BUFFER : QPN_ERR_SHAPE;
  GemmArgs a{packed, x, y, m, n, k, nullptr, workspace, stream};
  return launch_status(launch_gemm(fmt, false, a, l));
}

}  // namespace

extern "C" {

const char* qpn_status_string(int status) {
  switch (status) {
    case QPN_OK: return "QPN_OK";
    case QPN_ERR_NULL: return "QPN_ERR_NULL: a required pointer is NULL";
    case QPN_ERR_SHAPE: return "QPN_ERR_SHAPE: m, n or k outside the supported range";
    case QPN_ERR_ALIGN: return "QPN_ERR_ALIGN: a pointer is not aligned as required";
    case QPN_ERR_BUFFER: return "QPN_ERR_BUFFER: buffer smaller than required";
    case QPN_ERR_DEVICE: return "QPN_ERR_DEVICE: current device is not a usable gfx950";
    case QPN_ERR_LAUNCH: return "QPN_ERR_LAUNCH: kernel launch failed";
    case QPN_ERR_SCRATCH:
      return "QPN_ERR_SCRATCH: the call needs more than the library's static scratch";
    default: return "QPN: unknown status";
  }
}

int qpn_layout_version(void) { return (int)kLayoutVersion; }

size_t qpn_nvfp4_packed_bytes(int64_t n, int64_t k) {
  if (!nv_shape_ok(n, k)) return 0;
  return (size_t)nv_blob_bytes(n, k);
}

size_t qpn_fp8_packed_bytes(int64_t n, int64_t k) {
  if (!f8_shape_ok(n, k)) return 0;
  return (size_t)f8_blob_bytes(n, k);
}

}  // extern "C"

namespace {

// Launch plan and workspace of one call, as the plan queries report them.
struct PlanInfo {
  int64_t workgroups;
  int waves_per_panel;
  int panels_per_workgroup;
  int depth;
  int splits;
  int activation_rows;
  int64_t split_wgs;
  int valu_dot;
  size_t ws_bytes;  // workspace the call uses for this plan (0 = none needed)
};

void fill_skinny(const GemmLaunch& g, int m, PlanInfo* o) {
  o->workgroups = g.workgroups;
  o->waves_per_panel = g.waves_per_panel;
  o->panels_per_workgroup = g.panels_per_workgroup;
  o->depth = g.depth;
  o->splits = g.splits;
  o->activation_rows = gemm_activation_rows(m > 0 ? m : 1);
  o->split_wgs = g.split_wgs;
  o->valu_dot = g.valu_dot;
}

// The plan a call of kind `op` uses for (m, n, k) given all the workspace it
// asks for; `plan` 0 is the automatic choice, 1.. a compiled plan (skinny
// ops only).  A pure function of its arguments.  QPN_OK or QPN_ERR_SHAPE.
int plan_query(int op, int plan, int m, int64_t n, int64_t k, PlanInfo* o) {
  GemmPlan pl;
  if (plan != 0 && !gemm_plan_info(plan, &pl)) return QPN_ERR_SHAPE;
  if (op == QPN_OP_PREFILL_NVFP4 || op == QPN_OP_PREFILL_FP8) {
    const uint32_t fmt = op == QPN_OP_PREFILL_NVFP4 ? kFmtNvfp4 : kFmtFp8;
    if (plan != 0) return QPN_ERR_SHAPE;
    if (m < 0 || m > kMaxPrefillM) return QPN_ERR_SHAPE;
    if (!(fmt == kFmtNvfp4 ? nv_shape_ok(n, k) : f8_shape_ok(n, k))) return QPN_ERR_SHAPE;
    if (prefill_on_skinny(fmt, m, n, k)) {  // the skinny kernel (a 16-row tile above 8 rows)
      GemmLaunch g;
      if (gemm_launch_for(fmt, m > 0 ? m : 1, n, k, 0, (size_t)-1, 0, &g) != kGemmLaunchOk)
        return QPN_ERR_SHAPE;
      fill_skinny(g, m, o);
      o->ws_bytes = (m == 0 || n == 0 || g.splits <= 1) ? 0 : g.ws_needed;
      return QPN_OK;
    }
    PrefillLaunch l;
    if (prefill_launch_for(fmt, m, n, k, (size_t)-1, &l) != kGemmLaunchOk) return QPN_ERR_SHAPE;
    o->workgroups = l.workgroups;
    // narrow: two wavefronts per panel (one per half of the rows); wide: one
    o->waves_per_panel = l.wide ? 1 : 2;
    o->panels_per_workgroup = l.wide ? 16 : 8;
    o->depth = l.depth;
    o->splits = l.max_pieces;  // the most workgroups one output tile is cut between
    o->activation_rows = (l.wide ? 16 : 32) * l.mt;  // rows per workgroup
    o->split_wgs = l.workgroups;
    o->valu_dot = 0;
    o->ws_bytes = n == 0 ? 0 : l.ws_needed;
    return QPN_OK;
  }
  if (m < 0 || m > kMaxM) return QPN_ERR_SHAPE;
  uint32_t fmt;
  switch (op) {
    case QPN_OP_GEMM_NVFP4:
    case QPN_OP_LMHEAD_NVFP4:
      if (!nv_shape_ok(n, k)) return QPN_ERR_SHAPE;
      fmt = kFmtNvfp4;
      break;
    case QPN_OP_GEMM_FP8:
      if (!f8_shape_ok(n, k)) return QPN_ERR_SHAPE;
      fmt = kFmtFp8;
      break;
    default: return QPN_ERR_SHAPE;
  }
  const bool lm = op == QPN_OP_LMHEAD_NVFP4;
  GemmLaunch l;
  if (gemm_launch_for(fmt, m > 0 ? m : 1, n, k, plan, (size_t)-1,
                      lm ? lmhead_split_offset(m, n) : 0, &l) != kGemmLaunchOk)
    return QPN_ERR_SHAPE;
  fill_skinny(l, m, o);
  if (m == 0 || n == 0) o->ws_bytes = 0;
  else if (l.splits <= 1) o->ws_bytes = lm ? lmhead_keys_bytes(m, n) : 0;
  else o->ws_bytes = l.ws_needed;
  return QPN_OK;
}

template <class T>
void put(T* dst, T v) {
  if (dst) *dst = v;
}

}  // namespace

extern "C" {

size_t qpn_workspace_bytes(int op, int m, int64_t n, int64_t k) {
  PlanInfo o;
  return plan_query(op, 0, m, n, k, &o) == QPN_OK ? o.ws_bytes : (size_t)-1;
}

int qpn_gemm_plan(int op, int m, int64_t n, int64_t k, int64_t* workgroups, int* waves_per_panel,
                  int* panels_per_workgroup, int* prefetch_depth, int* splits,
                  int* activation_rows, int64_t* split_workgroups) {
  PlanInfo o;
  const int rc = plan_query(op, 0, m, n, k, &o);
  if (rc != QPN_OK) return rc;
  put(workgroups, o.workgroups);
  put(waves_per_panel, o.waves_per_panel);
  put(panels_per_workgroup, o.panels_per_workgroup);
  put(prefetch_depth, o.depth);
  put(splits, o.splits);
  put(activation_rows, o.activation_rows);
  put(split_workgroups, o.split_wgs);
  return QPN_OK;
}

int qpn_pack_nvfp4(const float* w, int64_t n, int64_t k, void* packed, size_t packed_bytes,
                   void* stream) {
  if (!nv_shape_ok(n, k)) return QPN_ERR_SHAPE;
  if (!packed || (!w && n * k > 0)) return QPN_ERR_NULL;
  if (!aligned(packed, 256) || !aligned(w, 16)) return QPN_ERR_ALIGN;
  if (packed_bytes < nv_blob_bytes(n, k)) return QPN_ERR_BUFFER;
  int rc = device_check();
  if (rc != QPN_OK) return rc;
  return launch_status(launch_pack_nvfp4(w, n, k, packed, stream));
}

int qpn_pack_fp8(const float* w, int64_t n, int64_t k, void* packed, size_t packed_bytes,
                 void* stream) {
  if (!f8_shape_ok(n, k)) return QPN_ERR_SHAPE;
  if (!packed || (!w && n * k > 0)) return QPN_ERR_NULL;
  if (!aligned(packed, 256) || !aligned(w, 16)) return QPN_ERR_ALIGN;
  if (packed_bytes < f8_blob_bytes(n, k)) return QPN_ERR_BUFFER;
  int rc = device_check();
  if (rc != QPN_OK) return rc;
  return launch_status(launch_pack_fp8(w, n, k, packed, stream));
}

int qpn_requant_fp8_to_nvfp4(const void* fp8_packed, size_t fp8_bytes, int64_t n, int64_t k,
                             void* nvfp4_packed, size_t nvfp4_bytes, void* stream) {
  if (!nv_shape_ok(n, k) || !f8_shape_ok(n, k)) return QPN_ERR_SHAPE;
  if (!fp8_packed || !nvfp4_packed) return QPN_ERR_NULL;
  if (!aligned(fp8_packed, 256) || !aligned(nvfp4_packed, 256)) return QPN_ERR_ALIGN;
  if (fp8_bytes < f8_blob_bytes(n, k) || nvfp4_bytes < nv_blob_bytes(n, k)) return QPN_ERR_BUFFER;
  const uintptr_t a = (uintptr_t)fp8_packed, b = (uintptr_t)nvfp4_packed;
  if (a < b + nv_blob_bytes(n, k) && b < a + f8_blob_bytes(n, k)) return QPN_ERR_BUFFER;  // overlap
  int rc = device_check();
  if (rc != QPN_OK) return rc;
  return launch_status(launch_requant_fp8_to_nvfp4(fp8_packed, n, k, nvfp4_packed, stream));
}

int qpn_gemm_nvfp4(const void* packed, const uint16_t* x, uint16_t* y, int m, int64_t n,
                   int64_t k, void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_entry(kFmtNvfp4, 0, packed, x, y, m, n, k, workspace, workspace_bytes, stream);
}

int qpn_gemm_fp8(const void* packed, const uint16_t* x, uint16_t* y, int m, int64_t n, int64_t k,
                 void* workspace, size_t workspace_bytes, void* stream) {
  return gemm_entry(kFmtFp8, 0, packed, x, y, m, n, k, workspace, workspace_bytes, stream);
}

int qpn_gemm_nvfp4_noalloc(const void* packed, const uint16_t* x, uint16_t* y, int m, int64_t n,
                           int64_t k, void* stream) {
  int rc = gemm_common_checks(kFmtNvfp4, packed, x, y, m, n, k);
  if (rc != QPN_OK) return rc;
  if (m == 0 || n == 0) return QPN_OK;
  rc = device_check();
  if (rc != QPN_OK) return rc;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices || !g_scratch[dev])
    return QPN_ERR_DEVICE;
  void* ws = g_scratch[dev];
  // the plan qpn_gemm_nvfp4 uses with a workspace of kScratchBytes: the same
  // kernels, with fewer K splits only where more would not fit
  GemmLaunch l;
  const int lr = gemm_launch_for(kFmtNvfp4, m, n, k, 0, kScratchBytes, 0, &l);
  if (lr != kGemmLaunchOk) return lr == kGemmNoWorkspace ? QPN_ERR_SCRATCH : QPN_ERR_SHAPE;
  // belt and braces: clear the scratch in stream order before its first use
  // on this device (it is zero-filled from the start and every call leaves it so)
  hipError_t fe = hipSuccess;
  std::call_once(g_scratch_cleared[dev], [&]() { fe = launch_zero_fill(ws, kScratchBytes, stream); });
  if (fe != hipSuccess) return QPN_ERR_LAUNCH;
  GemmArgs a{packed, x, y, m, n, k, nullptr, ws, stream};
  return launch_status(launch_gemm(kFmtNvfp4, false, a, l));
}

namespace {

int prefill_entry(uint32_t fmt, const void* packed, const uint16_t* x, uint16_t* y, int m,
                  int64_t n, int64_t k, void* workspace, size_t workspace_bytes, void* stream,
                  int spin_limit = kPrefillSpinLimit) {
  if (m < 0 || m > kMaxPrefillM) return QPN_ERR_SHAPE;
  if (!(fmt == kFmtNvfp4 ? nv_shape_ok(n, k) : f8_shape_ok(n, k))) return QPN_ERR_SHAPE;
  if (m == 0 || n == 0) return QPN_OK;
  if (!packed || (!x && k > 0) || !y) return QPN_ERR_NULL;
  if (!aligned(packed, 256) || !aligned(x, 16) || !aligned(y, 2)) return QPN_ERR_ALIGN;
  if (workspace && !aligned(workspace, 16)) return QPN_ERR_ALIGN;
  int rc = device_check();
  if (rc != QPN_OK) return rc;
  GemmArgs a{packed, x, y, m, n, k, nullptr, workspace, stream};
  if (prefill_on_skinny(fmt, m, n, k)) {
    // the skinny kernel with a 16-row tile, when the workspace holds the K
    // splits it needs; otherwise the tiled kernel below (which runs with any)
    GemmLaunch g;
    if (gemm_launch_for(fmt, m, n, k, 0, workspace ? workspace_bytes : 0, 0, &g) == kGemmLaunchOk)
      return launch_status(launch_gemm(fmt, false, a, g));
  }
  PrefillLaunch l;
  if (prefill_launch_for(fmt, m, n, k, workspace ? workspace_bytes : 0, &l) != kGemmLaunchOk)
    return QPN_ERR_BUFFER;
  l.spin_limit = spin_limit;
  return launch_status(launch_prefill(fmt, a, l));
}

int lmhead_common(int plan, const void* packed, const uint16_t* x, uint16_t* logits,
                  int32_t* argmax, const int32_t* draft, int32_t* result, int m, int64_t n,
                  int64_t k, void* workspace, size_t workspace_bytes, void* stream) {
  if (n < 1) return QPN_ERR_SHAPE;
  int rc = gemm_common_checks(kFmtNvfp4, packed, x, logits, m, n, k);
  if (rc != QPN_OK) return rc;
  if (m == 0) return QPN_OK;
  if (!argmax) return QPN_ERR_NULL;
  if (!aligned(argmax, 4)) return QPN_ERR_ALIGN;
  if (!workspace) return QPN_ERR_NULL;
  if (!aligned(workspace, 8)) return QPN_ERR_ALIGN;
  if (workspace_bytes < lmhead_keys_bytes(m, n)) return QPN_ERR_BUFFER;
  rc = device_check();
  if (rc != QPN_OK) return rc;
  GemmLaunch l;
  const int lr = gemm_launch_for(kFmtNvfp4, m, n, k, plan, workspace_bytes,
                                 lmhead_split_offset(m, n), &l);
  if (lr != kGemmLaunchOk) return lr == kGemmNoWorkspace ? QPN_ERR_BUFFER : QPN_ERR_SHAPE;
  GemmArgs a{packed, x, logits, m, n, k, (uint64_t*)workspace, workspace, stream};
  hipError_t e = launch_gemm(kFmtNvfp4, true, a, l);
  if (e != hipSuccess) return QPN_ERR_LAUNCH;
  return launch_status(launch_argmax_finalize((uint64_t*)workspace, m, argmax, draft, result, stream));
}

}  // namespace

int qpn_gemm_prefill_nvfp4(const void* packed, const uint16_t* x, uint16_t* y, int m, int64_t n,
                           int64_t k, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_entry(kFmtNvfp4, packed, x, y, m, n, k, workspace, workspace_bytes, stream);
}

int qpn_gemm_prefill_fp8(const void* packed, const uint16_t* x, uint16_t* y, int m, int64_t n,
                         int64_t k, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_entry(kFmtFp8, packed, x, y, m, n, k, workspace, workspace_bytes, stream);
}

int qpn_lmhead_nvfp4(const void* packed, const uint16_t* x, uint16_t* logits, int32_t* argmax,
                     int m, int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                     void* stream) {
  return lmhead_common(0, packed, x, logits, argmax, nullptr, nullptr, m, n, k, workspace,
                       workspace_bytes, stream);
}

int qpn_lmhead_verify_nvfp4(const void* packed, const uint16_t* x, uint16_t* logits,
                            int32_t* argmax, const int32_t* draft, int32_t* result, int m,
                            int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (m > 0) {
    if (!result || (m > 1 && !draft)) return QPN_ERR_NULL;
    if (!aligned(result, 4) || (draft && !aligned(draft, 4))) return QPN_ERR_ALIGN;
  }
  return lmhead_common(0, packed, x, logits, argmax, m > 1 ? draft : nullptr, result, m, n, k,
                       workspace, workspace_bytes, stream);
}

int qpn_debug_unpack_nvfp4(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                           uint8_t* scales, float* g, void* stream) {
  if (!nv_shape_ok(n, k)) return QPN_ERR_SHAPE;
  if (!packed || !g || ((!codes || !scales) && n * k > 0)) return QPN_ERR_NULL;
  if (!aligned(packed, 256) || !aligned(g, 4)) return QPN_ERR_ALIGN;
  int rc = device_check();
  if (rc != QPN_OK) return rc;
  return launch_status(launch_unpack_nvfp4(packed, n, k, codes, scales, g, stream));
}

int qpn_debug_unpack_fp8(const void* packed, int64_t n, int64_t k, uint8_t* codes,
                         float* row_scale, void* stream) {
  if (!f8_shape_ok(n, k)) return QPN_ERR_SHAPE;
  if (!packed || (!codes && n * k > 0) || (!row_scale && n > 0)) return QPN_ERR_NULL;
  if (!aligned(packed, 256) || !aligned(row_scale, 4)) return QPN_ERR_ALIGN;
  if (n == 0) return QPN_OK;
  int rc = device_check();
  if (rc != QPN_OK) return rc;
  return launch_status(launch_unpack_fp8(packed, n, k, codes, row_scale, stream));
}

int qpn_debug_decode_nvfp4(const uint8_t* codes16, const uint8_t* scales2, int64_t count,
                           uint16_t* out, void* stream) {
  if (count < 0 || count > (int64_t(1) << 24)) return QPN_ERR_SHAPE;
  if (count == 0) return QPN_OK;
  if (!codes16 || !scales2 || !out) return QPN_ERR_NULL;
  if (!aligned(out, 16)) return QPN_ERR_ALIGN;
  int rc = device_check();
  if (rc != QPN_OK) return rc;
  return launch_status(launch_decode_nvfp4(codes16, scales2, count, out, stream));
}

int qpn_debug_decode_fp8(const uint8_t* codes16, int64_t count, uint16_t* out, void* stream) {
  if (count < 0 || count > (int64_t(1) << 24)) return QPN_ERR_SHAPE;
  if (count == 0) return QPN_OK;
  if (!codes16 || !out) return QPN_ERR_NULL;
  if (!aligned(out, 16)) return QPN_ERR_ALIGN;
  int rc = device_check();
  if (rc != QPN_OK) return rc;
  return launch_status(launch_decode_fp8(codes16, count, out, stream));
}

int qpn_debug_plan(int op, int plan, int m, int64_t n, int64_t k, int64_t* workgroups,
                   int* waves_per_panel, int* panels_per_workgroup, int* prefetch_depth,
                   int* splits, int* activation_rows, int64_t* split_workgroups, int* valu_dot,
                   size_t* workspace_bytes) {
  if (op != QPN_OP_GEMM_NVFP4 && op != QPN_OP_GEMM_FP8 && op != QPN_OP_LMHEAD_NVFP4)
    return QPN_ERR_SHAPE;
  PlanInfo o;
  const int rc = plan_query(op, plan, m, n, k, &o);
  if (rc != QPN_OK) return rc;
  put(workgroups, o.workgroups);
  put(waves_per_panel, o.waves_per_panel);
  put(panels_per_workgroup, o.panels_per_workgroup);
  put(prefetch_depth, o.depth);
  put(splits, o.splits);
  put(activation_rows, o.activation_rows);
  put(split_workgroups, o.split_wgs);
  put(valu_dot, o.valu_dot);
  put(workspace_bytes, o.ws_bytes);
  return QPN_OK;
}

int qpn_debug_run_plan(int op, int plan, const void* packed, const uint16_t* x, uint16_t* y,
                       int32_t* argmax, int m, int64_t n, int64_t k, void* workspace,
                       size_t workspace_bytes, void* stream) {
  GemmPlan pl;
  if (plan != 0 && !gemm_plan_info(plan, &pl)) return QPN_ERR_SHAPE;
  switch (op) {
    case QPN_OP_GEMM_NVFP4:
      return gemm_entry(kFmtNvfp4, plan, packed, x, y, m, n, k, workspace, workspace_bytes, stream);
    case QPN_OP_GEMM_FP8:
      return gemm_entry(kFmtFp8, plan, packed, x, y, m, n, k, workspace, workspace_bytes, stream);
    case QPN_OP_LMHEAD_NVFP4:
      return lmhead_common(plan, packed, x, y, argmax, nullptr, nullptr, m, n, k, workspace,
                           workspace_bytes, stream);
    default: return QPN_ERR_SHAPE;
  }
}

int qpn_debug_prefill_no_wait(int op, const void* packed, const uint16_t* x, uint16_t* y, int m,
                              int64_t n, int64_t k, void* workspace, size_t workspace_bytes,
                              void* stream) {
  if (op != QPN_OP_PREFILL_NVFP4 && op != QPN_OP_PREFILL_FP8) return QPN_ERR_SHAPE;
  return prefill_entry(op == QPN_OP_PREFILL_NVFP4 ? kFmtNvfp4 : kFmtFp8, packed, x, y, m, n, k,
                       workspace, workspace_bytes, stream, 0);
}

int qpn_debug_read_ceiling(const void* buf, size_t bytes, uint32_t* sink, void* stream) {
  if (!buf || !sink) return QPN_ERR_NULL;
  if (bytes == 0 || bytes % 16 != 0 || bytes > ((size_t)1 << 40)) return QPN_ERR_SHAPE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return QPN_ERR_ALIGN;
  int rc = device_check();
  if (rc != QPN_OK) return rc;
  return launch_status(launch_read_ceiling(buf, (int64_t)(bytes / 16), sink, stream));
}

}  // extern "C"
