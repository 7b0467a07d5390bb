// attn_abi.hip - the C ABI declared in include/attn.h: argument validation, path planning,
// workspace sizing, device check and kernel launches. No allocation, no global mutable
// state beyond a once-per-device architecture check.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>

#include "attn.h"
#include "attn_internal.h"

namespace {

using attn::FwdArgs;

struct Plan {
  int path;        // ATTN_PATH_PREFILL or ATTN_PATH_SPLITK
  int nsb;         // split-K: key-range blocks per (sequence, K/V head)
  int chunk;       // split-K: keys per block (multiple of the stage size)
  size_t workspace;
};

int validate_common(int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_q,
                    int32_t max_k, int32_t hq, int32_t hkv, int32_t d, int32_t dtype,
                    int32_t mode, int32_t window) {
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0)
    return ATTN_ERR_BAD_SHAPE;
  if (d != 64 && d != 128) return ATTN_ERR_BAD_SHAPE;
  if (max_q > total_q || max_k > total_k) return ATTN_ERR_BAD_SHAPE;
  if (hq < 1 || hkv < 1 || hq % hkv != 0) return ATTN_ERR_BAD_HEADS;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_BAD_DTYPE;
  if (mode != ATTN_MASK_NONE && mode != ATTN_MASK_CAUSAL_TOP_LEFT &&
      mode != ATTN_MASK_CAUSAL_BOTTOM_RIGHT)
    return ATTN_ERR_BAD_MASK;
  if (window > 0 && mode == ATTN_MASK_NONE) return ATTN_ERR_BAD_MASK;
  // Element offsets must fit the kernels' 32-bit token indices.
  if ((long long)total_q * hq * d >= (1LL << 40) || (long long)total_k * hkv * d >= (1LL << 40))
    return ATTN_ERR_BAD_SHAPE;
  return ATTN_OK;
}

std::atomic<int> g_device_ok[64];  // 0 unknown, 1 gfx950, 2 other
std::atomic<int> g_device_cu[64];  // compute units per device (0 unknown)

// Checks that the current device is gfx950 (once per device) and reports its CU count.
int check_device(int* num_cu = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_ERR_UNSUPPORTED_DEVICE;
  if (dev < 0 || dev >= 64) return ATTN_ERR_UNSUPPORTED_DEVICE;
  int state = g_device_ok[dev].load(std::memory_order_relaxed);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ATTN_ERR_UNSUPPORTED_DEVICE;
    state = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_cu[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_device_ok[dev].store(state, std::memory_order_relaxed);
  }
  if (num_cu) *num_cu = g_device_cu[dev].load(std::memory_order_relaxed);
  return state == 1 ? ATTN_OK : ATTN_ERR_UNSUPPORTED_DEVICE;
}

// CU count used for planning: the current device's when it is a gfx950 (so the sizes a
// caller queries match the launch on that device), else MI355X's 256.
int planning_cu_count() {
  int n = 0;
  if (check_device(&n) != ATTN_OK || n <= 0) n = 256;
  return n;
}

// Path choice. Split-K when the query rows of one K/V head fit one wave's two 32-row
// blocks and the key range is long enough to be worth splitting; prefill otherwise.
// num_cu sizes the split-K grid: the path is bound by HBM reads, and one CU keeps only so
// many bytes in flight, so every CU must stream (one workgroup per CU fits in LDS).
int make_plan(int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_q,
              int32_t max_k, int32_t hq, int32_t hkv, int32_t d, int32_t dtype, int32_t path,
              int32_t num_splits, int num_cu, Plan* plan) {
  const int group = hq / hkv;
  const long rows = (long)group * max_q;
  // Two 128-key fp32 stages of head_dim 128 exceed the 160 KiB of LDS.
  const bool splitk_ok = rows <= attn::SPLITK_MAX_ROWS && !(dtype == ATTN_F32 && d == 128);
  if (path == ATTN_PATH_AUTO) path = (splitk_ok && max_k >= 1024) ? ATTN_PATH_SPLITK : ATTN_PATH_PREFILL;
  if (path != ATTN_PATH_PREFILL && path != ATTN_PATH_SPLITK) return ATTN_ERR_BAD_PLAN;
  if (num_splits < 0) return ATTN_ERR_BAD_PLAN;
  plan->path = path;
  plan->nsb = 0;
  plan->chunk = 0;
  plan->workspace = 0;
  if (path == ATTN_PATH_PREFILL) {
    // Batches of unequal lengths sort their tiles by cost (one int32 per tile slot).
    attn::FwdArgs a{};
    a.num_seqs = num_seqs;
    a.total_q = total_q;
    a.total_k = total_k;
    a.max_q = max_q;
    a.max_k = max_k;
    plan->workspace = attn::fwd_prefill_workspace_bytes(a);
    return ATTN_OK;
  }
  if (!splitk_ok) return ATTN_ERR_BAD_PLAN;
  const int stage = attn::SPLITK_STAGE;
  const long max_blocks = std::max<long>(1, (max_k + stage - 1) / stage);
  long nsb = num_splits;
  if (nsb == 0) {
    // Fill every CU with as little imbalance as possible: among 1..4 times the smallest
    // count that covers all CUs, the split count whose last round of workgroups is the
    // fullest (ties: fewer splits, i.e. fewer partials to combine). At least 4 stages each.
    const long units = std::max<long>(1, (long)num_seqs * hkv);
    const long cus = std::max(1, num_cu);
    const long base = std::max<long>(1, (cus + units - 1) / units);
    double best = -1.0;
    for (long c = base; c <= 4 * base; ++c) {
      const long wgs = units * c, rounds = (wgs + cus - 1) / cus;
      const double eff = (double)wgs / (double)(rounds * cus);
      if (eff > best + 1e-9) {
        best = eff;
        nsb = c;
      }
    }
    nsb = std::min<long>(nsb, std::max<long>(1, (max_k + 4 * stage - 1) / (4 * stage)));
  }
  nsb = std::max<long>(1, std::min<long>(nsb, max_blocks));
  long chunk = (max_k + nsb - 1) / nsb;
  chunk = ((chunk + stage - 1) / stage) * stage;
  if (chunk == 0) chunk = stage;
  nsb = std::max<long>(1, (max_k + chunk - 1) / chunk);
  plan->nsb = (int)nsb;
  plan->chunk = (int)chunk;
  plan->workspace = attn::splitk_workspace_bytes(
      (int)nsb * attn::splitk_partials_per_chunk((int)rows), total_q, hq, d);
  return ATTN_OK;
}

FwdArgs make_args(const void* q, const void* k, const void* v, const int32_t* cu_q,
                  const int32_t* cu_k, int32_t num_seqs, int32_t total_q, int32_t total_k,
                  int32_t max_q, int32_t max_k, int32_t hq, int32_t hkv, int32_t d,
                  int32_t dtype, float scale, int32_t mode, int32_t window, void* out,
                  float* lse) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.num_seqs = num_seqs;
  a.total_q = total_q;
  a.total_k = total_k;
  a.max_q = max_q;
  a.max_k = max_k;
  a.hq = hq;
  a.hkv = hkv;
  a.d = d;
  a.dtype = dtype;
  a.scale = scale;
  a.mode = mode;
  a.window = window > 0 ? window : 0;
  a.out = out;
  a.lse = lse;
  return a;
}

// Byte threshold t8 = round(256 p) and the keep scale 1 / (1 - t8 / 256) of a dropout
// probability; false unless 0 <= p and t8 <= 255.
bool dropout_threshold(float p, uint32_t* thr, float* scale) {
  if (!(p >= 0.0f) || !std::isfinite(p)) return false;
  const double t = std::floor((double)p * 256.0 + 0.5);
  if (t > 255.0) return false;
  *thr = (uint32_t)t;
  *scale = (float)(256.0 / (256.0 - t));
  return true;
}

// Fixed device scratch of attn_fwd_no_workspace, for callers that cannot allocate (code
// under graph capture, serving loops). Every GPU the library runs on holds its own copy
// of this array until the process ends. In host code `scratch` names a host-side stand-in,
// not device memory: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is ever handed to kernels.
static __device__ __align__(256) char scratch[ATTN_SCRATCH_BYTES];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64];  // device address of `scratch` per device (null until looked up)

// Device address of `scratch` on the current device.
int scratch_address(void** ptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ATTN_ERR_UNSUPPORTED_DEVICE;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return ATTN_ERR_LAUNCH_FAILED;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_version(void) { return ATTN_VERSION; }

const char* attn_status_string(int status) {
  switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULL_PTR: return "a required pointer is NULL";
    case ATTN_ERR_BAD_SHAPE: return "bad shape (negative size, max_seqlen above total, or head_dim not 64/128)";
    case ATTN_ERR_BAD_HEADS: return "bad head counts (need Hq >= 1, Hkv >= 1, Hq % Hkv == 0)";
    case ATTN_ERR_BAD_DTYPE: return "unsupported dtype (ATTN_BF16 or ATTN_F32)";
    case ATTN_ERR_BAD_MASK: return "bad mask (unknown mode, or window without a causal alignment)";
    case ATTN_ERR_WORKSPACE_TOO_SMALL: return "workspace smaller than the size query's answer";
    case ATTN_ERR_UNSUPPORTED_DEVICE: return "current device is not a gfx950 GPU";
    case ATTN_ERR_LAUNCH_FAILED: return "kernel launch failed";
    case ATTN_ERR_BAD_SCALE: return "scale is not finite";
    case ATTN_ERR_BAD_PLAN: return "forced path or split count not usable for this shape";
    case ATTN_ERR_BAD_RANGE: return "probe window outside the token ranges";
    case ATTN_ERR_BAD_DROPOUT: return "dropout probability not in [0, 255.5/256)";
    case ATTN_ERR_SCRATCH_TOO_SMALL:
      return "the call needs more scratch than the library's fixed 16 MiB (use attn_fwd)";
    default: return "unknown status";
  }
}

size_t attn_fwd_ex_workspace_size(int32_t num_seqs, int32_t total_q, int32_t total_k,
                                  int32_t max_q, int32_t max_k, int32_t hq, int32_t hkv,
                                  int32_t d, int32_t dtype, int32_t mode, int32_t window,
                                  int32_t path, int32_t num_splits) {
  if (validate_common(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, mode,
                      window) != ATTN_OK)
    return 0;
  Plan plan;
  if (make_plan(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, path, num_splits,
                planning_cu_count(), &plan) != ATTN_OK)
    return 0;
  return plan.workspace;
}

size_t attn_fwd_workspace_size(int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_q,
                               int32_t max_k, int32_t hq, int32_t hkv, int32_t d, int32_t dtype,
                               int32_t mode, int32_t window) {
  return attn_fwd_ex_workspace_size(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype,
                                    mode, window, ATTN_PATH_AUTO, 0);
}

int attn_fwd_ex(const void* q, const void* k, const void* v, const int32_t* cu_q,
                const int32_t* cu_k, int32_t num_seqs, int32_t total_q, int32_t total_k,
                int32_t max_q, int32_t max_k, int32_t hq, int32_t hkv, int32_t d, int32_t dtype,
                float scale, int32_t mode, int32_t window, int32_t path, int32_t num_splits,
                void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_common(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, mode,
                           window);
  if (rc != ATTN_OK) return rc;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  Plan plan;
  rc = make_plan(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, path, num_splits,
                 planning_cu_count(), &plan);
  if (rc != ATTN_OK) return rc;
  if (num_seqs == 0 || total_q == 0) return ATTN_OK;
  if (!cu_q || !cu_k || !out || !lse || !q) return ATTN_ERR_NULL_PTR;
  if (total_k > 0 && (!k || !v)) return ATTN_ERR_NULL_PTR;
  if (plan.workspace > 0 && (!workspace)) return ATTN_ERR_NULL_PTR;
  if (workspace_bytes < plan.workspace) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  rc = check_device();
  if (rc != ATTN_OK) return rc;
  const FwdArgs a = make_args(q, k, v, cu_q, cu_k, num_seqs, total_q, total_k, max_q, max_k, hq,
                              hkv, d, dtype, scale, mode, window, out, lse);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = plan.path == ATTN_PATH_PREFILL
                     ? attn::launch_fwd_prefill(a, workspace, st)
                     : attn::launch_fwd_splitk(a, plan.nsb, plan.chunk, workspace, st);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH_FAILED;
}

int attn_fwd(const void* q, const void* k, const void* v, const int32_t* cu_q, const int32_t* cu_k,
             int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_q, int32_t max_k,
             int32_t hq, int32_t hkv, int32_t d, int32_t dtype, float scale, int32_t mode,
             int32_t window, void* out, float* lse, void* workspace, size_t workspace_bytes,
             void* stream) {
  return attn_fwd_ex(q, k, v, cu_q, cu_k, num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d,
                     dtype, scale, mode, window, ATTN_PATH_AUTO, 0, out, lse, workspace,
                     workspace_bytes, stream);
}

int attn_fwd_no_workspace(const void* q, const void* k, const void* v, const int32_t* cu_q,
                          const int32_t* cu_k, int32_t num_seqs, int32_t total_q,
                          int32_t total_k, int32_t max_q, int32_t max_k, int32_t hq,
                          int32_t hkv, int32_t d, int32_t dtype, float scale, int32_t mode,
                          int32_t window, void* out, float* lse, void* stream) {
  // The same validation and plan as attn_fwd, in the same order, so errors match it.
  int rc = validate_common(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, mode,
                           window);
  if (rc != ATTN_OK) return rc;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  Plan plan;
  rc = make_plan(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, ATTN_PATH_AUTO, 0,
                 planning_cu_count(), &plan);
  if (rc != ATTN_OK) return rc;
  if (plan.workspace > (size_t)ATTN_SCRATCH_BYTES) return ATTN_ERR_SCRATCH_TOO_SMALL;
  if (num_seqs == 0 || total_q == 0) return ATTN_OK;
  rc = check_device();
  if (rc != ATTN_OK) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc != ATTN_OK) return rc;
  return attn_fwd_ex(q, k, v, cu_q, cu_k, num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d,
                     dtype, scale, mode, window, ATTN_PATH_AUTO, 0, out, lse, ws,
                     (size_t)ATTN_SCRATCH_BYTES, stream);
}

size_t attn_bwd_workspace_size(int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_q,
                               int32_t max_k, int32_t hq, int32_t hkv, int32_t d, int32_t dtype,
                               int32_t mode, int32_t window) {
  if (validate_common(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, mode,
                      window) != ATTN_OK)
    return 0;
  return attn::bwd_workspace_bytes(total_q, hq, d);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
             const void* dout, const int32_t* cu_q, const int32_t* cu_k, int32_t num_seqs,
             int32_t total_q, int32_t total_k, int32_t max_q, int32_t max_k, int32_t hq,
             int32_t hkv, int32_t d, int32_t dtype, float scale, int32_t mode, int32_t window,
             void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_common(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, mode,
                           window);
  if (rc != ATTN_OK) return rc;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  const size_t need = attn::bwd_workspace_bytes(total_q, hq, d);
  if (num_seqs == 0 || (total_q == 0 && total_k == 0)) return ATTN_OK;
  if (!cu_q || !cu_k) return ATTN_ERR_NULL_PTR;
  if (total_q > 0 && (!q || !out || !lse || !dout || !dq)) return ATTN_ERR_NULL_PTR;
  if (total_k > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL_PTR;
  if (need > 0 && !workspace) return ATTN_ERR_NULL_PTR;
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  rc = check_device();
  if (rc != ATTN_OK) return rc;
  attn::BwdArgs a;
  a.f = make_args(q, k, v, cu_q, cu_k, num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d,
                  dtype, scale, mode, window, nullptr, nullptr);
  a.out = out;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  hipError_t e = attn::launch_bwd(a, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH_FAILED;
}

int attn_mask_probe_ex(const int32_t* cu_q, const int32_t* cu_k, int32_t num_seqs,
                       int32_t total_q, int32_t total_k, int32_t max_q, int32_t max_k,
                       int32_t hq, int32_t hkv, int32_t mode, int32_t window, int32_t unit,
                       int32_t head, int32_t num_splits, int32_t q0, int32_t nq, int32_t k0,
                       int32_t nk, uint8_t* bits, void* stream) {
  if (num_seqs < 0 || total_q < 0 || total_k < 0) return ATTN_ERR_BAD_SHAPE;
  if (mode != ATTN_MASK_NONE && mode != ATTN_MASK_CAUSAL_TOP_LEFT &&
      mode != ATTN_MASK_CAUSAL_BOTTOM_RIGHT)
    return ATTN_ERR_BAD_MASK;
  if (window > 0 && mode == ATTN_MASK_NONE) return ATTN_ERR_BAD_MASK;
  if (unit < ATTN_PROBE_PREFILL || unit > ATTN_PROBE_BWD_Q_F32) return ATTN_ERR_BAD_PLAN;
  if (q0 < 0 || nq < 0 || k0 < 0 || nk < 0 || (long)q0 + nq > total_q || (long)k0 + nk > total_k)
    return ATTN_ERR_BAD_RANGE;
  attn::ProbeArgs a{};
  a.cu_q = cu_q;
  a.cu_k = cu_k;
  a.num_seqs = num_seqs;
  a.mode = mode;
  a.window = window > 0 ? window : 0;
  a.unit = unit;
  a.q0 = q0;
  a.nq = nq;
  a.k0 = k0;
  a.nk = nk;
  if (unit == ATTN_PROBE_SPLITK) {
    // The split-K plan attn_fwd_ex would run for these shapes (bf16, head_dim 128).
    int rc = validate_common(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, 128, ATTN_BF16,
                             mode, window);
    if (rc != ATTN_OK) return rc;
    if (head < 0 || head >= hq) return ATTN_ERR_BAD_RANGE;
    Plan plan;
    rc = make_plan(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, 128, ATTN_BF16,
                   ATTN_PATH_SPLITK, num_splits, planning_cu_count(), &plan);
    if (rc != ATTN_OK) return rc;
    a.group = hq / hkv;
    a.head = head;
    a.nsb = plan.nsb;
    a.chunk = plan.chunk;
    a.nrb = (long)a.group * max_q <= 32 ? 1 : 2;
  }
  if (nq == 0 || nk == 0 || num_seqs == 0) return ATTN_OK;
  if (!cu_q || !cu_k || !bits) return ATTN_ERR_NULL_PTR;
  int rc = check_device();
  if (rc != ATTN_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = unit <= ATTN_PROBE_SPLITK ? attn::launch_mask_probe_fwd(a, bits, st)
                                           : attn::launch_mask_probe_bwd(a, bits, st);
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH_FAILED;
}

int attn_mask_probe(const int32_t* cu_q, const int32_t* cu_k, int32_t num_seqs, int32_t total_q,
                    int32_t total_k, int32_t mode, int32_t window, int32_t q0, int32_t nq,
                    int32_t k0, int32_t nk, uint8_t* bits, void* stream) {
  return attn_mask_probe_ex(cu_q, cu_k, num_seqs, total_q, total_k, 0, 0, 1, 1, mode, window,
                            ATTN_PROBE_PREFILL, 0, 0, q0, nq, k0, nk, bits, stream);
}

size_t attn_fwd_dropout_workspace_size(int32_t num_seqs, int32_t total_q, int32_t total_k,
                                       int32_t max_q, int32_t max_k, int32_t hq, int32_t hkv,
                                       int32_t d, int32_t dtype, int32_t mode, int32_t window) {
  return attn_fwd_ex_workspace_size(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype,
                                    mode, window, ATTN_PATH_PREFILL, 0);
}

int attn_fwd_dropout(const void* q, const void* k, const void* v, const int32_t* cu_q,
                     const int32_t* cu_k, int32_t num_seqs, int32_t total_q, int32_t total_k,
                     int32_t max_q, int32_t max_k, int32_t hq, int32_t hkv, int32_t d,
                     int32_t dtype, float scale, int32_t mode, int32_t window, float dropout_p,
                     uint64_t seed, void* out, float* lse, void* out_residual,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int rc = validate_common(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, mode,
                           window);
  if (rc != ATTN_OK) return rc;
  if (out_residual != nullptr && dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  uint32_t thr = 0;
  float dscale = 1.0f;
  if (!dropout_threshold(dropout_p, &thr, &dscale)) return ATTN_ERR_BAD_DROPOUT;
  Plan plan;
  rc = make_plan(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, ATTN_PATH_PREFILL,
                 0, planning_cu_count(), &plan);
  if (rc != ATTN_OK) return rc;
  if (num_seqs == 0 || total_q == 0) return ATTN_OK;
  if (!cu_q || !cu_k || !out || !lse || !q) return ATTN_ERR_NULL_PTR;
  if (total_k > 0 && (!k || !v)) return ATTN_ERR_NULL_PTR;
  if (plan.workspace > 0 && (!workspace)) return ATTN_ERR_NULL_PTR;
  if (workspace_bytes < plan.workspace) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  rc = check_device();
  if (rc != ATTN_OK) return rc;
  FwdArgs a = make_args(q, k, v, cu_q, cu_k, num_seqs, total_q, total_k, max_q, max_k, hq, hkv,
                        d, dtype, scale, mode, window, out, lse);
  a.drop_thr = thr;
  a.drop_scale = dscale;
  a.seed = seed;
  a.out_res = out_residual;
  hipError_t e = attn::launch_fwd_prefill(a, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH_FAILED;
}

int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const void* out_residual, const void* dout,
                     const int32_t* cu_q, const int32_t* cu_k,
                     int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_q,
                     int32_t max_k, int32_t hq, int32_t hkv, int32_t d, int32_t dtype,
                     float scale, int32_t mode, int32_t window, float dropout_p, uint64_t seed,
                     void* dq, void* dk, void* dv, void* workspace, size_t workspace_bytes,
                     void* stream) {
  int rc = validate_common(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, mode,
                           window);
  if (rc != ATTN_OK) return rc;
  if (out_residual != nullptr && dtype != ATTN_BF16) return ATTN_ERR_BAD_DTYPE;
  if (!std::isfinite(scale)) return ATTN_ERR_BAD_SCALE;
  uint32_t thr = 0;
  float dscale = 1.0f;
  if (!dropout_threshold(dropout_p, &thr, &dscale)) return ATTN_ERR_BAD_DROPOUT;
  const size_t need = attn::bwd_workspace_bytes(total_q, hq, d);
  if (num_seqs == 0 || (total_q == 0 && total_k == 0)) return ATTN_OK;
  if (!cu_q || !cu_k) return ATTN_ERR_NULL_PTR;
  if (total_q > 0 && (!q || !out || !lse || !dout || !dq)) return ATTN_ERR_NULL_PTR;
  if (total_k > 0 && (!k || !v || !dk || !dv)) return ATTN_ERR_NULL_PTR;
  if (need > 0 && !workspace) return ATTN_ERR_NULL_PTR;
  if (workspace_bytes < need) return ATTN_ERR_WORKSPACE_TOO_SMALL;
  rc = check_device();
  if (rc != ATTN_OK) return rc;
  attn::BwdArgs a;
  a.f = make_args(q, k, v, cu_q, cu_k, num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d,
                  dtype, scale, mode, window, nullptr, nullptr);
  a.f.drop_thr = thr;
  a.f.drop_scale = dscale;
  a.f.seed = seed;
  a.out = out;
  a.out_res = out_residual;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  hipError_t e = attn::launch_bwd(a, workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH_FAILED;
}

int attn_dropout_probe(int32_t seq, int32_t head, int32_t q0, int32_t nq, int32_t k0,
                       int32_t nk, float dropout_p, uint64_t seed, uint8_t* keep,
                       void* stream) {
  if (seq < 0 || head < 0 || q0 < 0 || nq < 0 || k0 < 0 || nk < 0) return ATTN_ERR_BAD_RANGE;
  if ((int64_t)q0 + nq > INT32_MAX - 64 || (int64_t)k0 + nk > INT32_MAX - 64)
    return ATTN_ERR_BAD_RANGE;
  if (((q0 + nq + 31) >> 5) - (q0 >> 5) > 65535) return ATTN_ERR_BAD_RANGE;  // grid rows
  uint32_t thr = 0;
  float dscale = 1.0f;
  if (!dropout_threshold(dropout_p, &thr, &dscale)) return ATTN_ERR_BAD_DROPOUT;
  if (nq == 0 || nk == 0) return ATTN_OK;
  if (!keep) return ATTN_ERR_NULL_PTR;
  int rc = check_device();
  if (rc != ATTN_OK) return rc;
  hipError_t e = attn::launch_dropout_probe(seed, thr, seq, head, q0, nq, k0, nk, keep,
                                            static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH_FAILED;
}

int attn_check_seqlens(const int32_t* cu_q, const int32_t* cu_k, int32_t num_seqs,
                       int32_t total_q, int32_t total_k, int32_t max_q, int32_t max_k,
                       int32_t* word, void* stream) {
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_q < 0 || max_k < 0)
    return ATTN_ERR_BAD_SHAPE;
  if (!cu_q || !cu_k || !word) return ATTN_ERR_NULL_PTR;
  int rc = check_device();
  if (rc != ATTN_OK) return rc;
  hipError_t e = attn::launch_check_seqlens(cu_q, cu_k, num_seqs, total_q, total_k, max_q, max_k,
                                            word, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? ATTN_OK : ATTN_ERR_LAUNCH_FAILED;
}

#ifdef ATTN_DEBUG_POISON_LDS
static const char BUILD_TAG[] = " lds=poisoned";   // race-exposure build
#else
static const char BUILD_TAG[] = "";
#endif

int attn_describe_plan(int32_t num_seqs, int32_t total_q, int32_t total_k, int32_t max_q,
                       int32_t max_k, int32_t hq, int32_t hkv, int32_t d, int32_t dtype,
                       int32_t mode, int32_t window, int32_t path, int32_t num_splits, char* buf,
                       size_t len) {
  int rc = validate_common(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, mode,
                           window);
  if (rc != ATTN_OK) return rc;
  Plan plan;
  rc = make_plan(num_seqs, total_q, total_k, max_q, max_k, hq, hkv, d, dtype, path, num_splits,
                 planning_cu_count(), &plan);
  if (rc != ATTN_OK) return rc;
  if (!buf || len == 0) return ATTN_ERR_NULL_PTR;
  const char* dt = dtype == ATTN_BF16 ? "bf16" : "f32";
  if (plan.path == ATTN_PATH_PREFILL) {
    FwdArgs a = make_args(nullptr, nullptr, nullptr, nullptr, nullptr, num_seqs, total_q, total_k,
                          max_q, max_k, hq, hkv, d, dtype, 1.0f, mode, window, nullptr, nullptr);
    std::snprintf(buf, len,
                  "path=prefill dtype=%s d=%d tile=%dx%d waves=4 order=%s grid=%d workspace=%zu "
                  "version=%d%s",
                  dt, d, attn::FWD_BM, attn::FWD_BN,
                  attn::equal_lengths(a) ? "largest_first" : "cost_sorted",
                  attn::fwd_prefill_grid(a), plan.workspace, ATTN_VERSION, BUILD_TAG);
  } else {
    std::snprintf(buf, len,
                  "path=splitk dtype=%s d=%d stage=%d rows_per_kvhead<=%d blocks_per_kvhead=%d "
                  "chunk=%d partials=%d grid=%ld workspace=%zu version=%d%s",
                  dt, d, attn::SPLITK_STAGE, (hq / hkv) * max_q, plan.nsb, plan.chunk,
                  plan.nsb * attn::splitk_partials_per_chunk((hq / hkv) * max_q),
                  (long)num_seqs * hkv * plan.nsb, plan.workspace, ATTN_VERSION, BUILD_TAG);
  }
  return ATTN_OK;
}

}  // extern "C"
