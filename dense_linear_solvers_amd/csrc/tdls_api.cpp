// Host side of the C interface: argument validation, the launch planner and
// the dispatch to the kernel instantiations.  No allocation, no
// synchronization, no state beyond a per-device architecture check.
//
// Validation before any launch, no launch for an empty batch and exactly one
// otherwise, and an error (never a silent fallback) for what is not
// supported follow the ruSOLVER small-matrix page ("ruSOLVER：小矩阵 kernel
// 优化（实验性）", sections on the unchanged numerical and failure contract
// and on support and trade-offs).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "../../include/tdls.h"
#include "tdls_internal.h"

namespace tdls {
namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_state[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

struct ShapeEntry {
  int dtype, N, NRHS;
  GesvLauncher launch;
};

#define TDLS_SHAPE_ENTRY(sfx, Real, N, NRHS) \
  {sizeof(Real) == 8 ? 1 : 0, N, NRHS, &launch_gesv_##sfx##_n##N##_r##NRHS},
const ShapeEntry kShapes[] = {TDLS_FOR_EACH_SHAPE(TDLS_SHAPE_ENTRY)};
#undef TDLS_SHAPE_ENTRY

GesvLauncher find_launcher(int dtype, int N, int NRHS) {
  for (const ShapeEntry& e : kShapes)
    if (e.dtype == dtype && e.N == N && e.NRHS == NRHS) return e.launch;
  return nullptr;
}

int check_scalars(int dtype, int layout, int n, int nrhs, int64_t batch) {
  if (dtype != TDLS_F32 && dtype != TDLS_F64) return -1;
  if (layout != TDLS_ROW_MAJOR && layout != TDLS_COL_MAJOR) return -2;
  if (n < 1 || n > 64) return -3;
  if (nrhs < 1 || nrhs > 8) return -4;
  if (batch < 0) return -5;
  return 0;
}

// Group-size override for tests: TDLS_GROUP_SIZE=<T>.
int group_size_override() {
  const char* s = getenv("TDLS_GROUP_SIZE");
  if (s == nullptr || *s == '\0') return 0;
  return atoi(s);
}

int make_plan(int dtype, int layout, int n, int nrhs, int64_t batch, LaunchPlan* p) {
  int rc = check_scalars(dtype, layout, n, nrhs, batch);
  if (rc != 0) return rc;
  const bool is64 = dtype == TDLS_F64;
  int N = 0, NRHS = 0;
  for (int v : kNValues)
    if (v >= n) { N = v; break; }
  for (int v : kNrhsValues)
    if (v >= nrhs) { NRHS = v; break; }
  const int T0 = pick_group_size(N, NRHS, is64);
  const int T1 = alt_group_size(N, NRHS, is64);
  int T = T0;
  const int forced = group_size_override();
  if (forced != 0) {
    if (forced != T0 && (T1 == 0 || forced != T1)) return TDLS_ERR_NO_KERNEL;
    T = forced;
  }
  p->dtype = dtype;
  p->layout = layout;
  p->n = n;
  p->nrhs = nrhs;
  p->N = N;
  p->NRHS = NRHS;
  p->T = T;
  p->R = (N + T - 1) / T;
  p->G = kWaveSize / T;
  p->batch = batch;
  p->threads_per_block = kWaveSize * kWavesPerBlock;
  p->systems_per_block = (int64_t)kWavesPerBlock * p->G;
  p->grid = (batch + p->systems_per_block - 1) / p->systems_per_block;
  if (p->grid > 0x7fffffffLL) return -5;
  p->lds_bytes = gesv_lds_bytes(N, NRHS, T, is64);
  return 0;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na != 0 && nb != 0 && x < y + nb && y < x + na;
}

bool misaligned(const void* ptr, size_t align) { return ((uintptr_t)ptr % align) != 0; }

int check_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return TDLS_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return TDLS_ERR_DEVICE;
  int st = g_arch_state[dev].load(std::memory_order_relaxed);
  if (st == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return TDLS_ERR_HIP;
    st = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_arch_state[dev].store(st, std::memory_order_relaxed);
  }
  return st == 1 ? 0 : TDLS_ERR_DEVICE;
}

}  // namespace
}  // namespace tdls

extern "C" {

int tdls_plan_gesv(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                   tdls_plan* out) {
  tdls::LaunchPlan p;
  int rc = tdls::make_plan((int)dtype, (int)layout, n, nrhs, batch, &p);
  if (rc != 0) return rc;
  if (out == nullptr) return -6;
  out->n = p.n;
  out->nrhs = p.nrhs;
  out->n_kernel = p.N;
  out->nrhs_kernel = p.NRHS;
  out->group_size = p.T;
  out->rows_per_lane = p.R;
  out->systems_per_wave = p.G;
  out->threads_per_block = p.threads_per_block;
  out->systems_per_block = p.systems_per_block;
  out->grid = p.grid;
  out->lds_bytes = p.lds_bytes;
  return 0;
}

int tdls_gesv_batched(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                      const void* A, const void* B, void* X, int32_t* piv, int32_t* info,
                      hipStream_t stream) {
  tdls::LaunchPlan p;
  int rc = tdls::make_plan((int)dtype, (int)layout, n, nrhs, batch, &p);
  if (rc != 0) return rc;
  if (batch == 0) return TDLS_SUCCESS;  // nothing to read or write, nothing launched

  const size_t es = dtype == TDLS_F64 ? 8 : 4;
  const size_t bytesA = (size_t)batch * n * n * es;
  const size_t bytesB = (size_t)batch * n * nrhs * es;
  const size_t bytesP = (size_t)batch * n * 4;
  const size_t bytesI = (size_t)batch * 4;
  if (A == nullptr || tdls::misaligned(A, es)) return -6;
  if (B == nullptr || tdls::misaligned(B, es)) return -7;
  if (X == nullptr || tdls::misaligned(X, es) || tdls::overlaps(X, bytesB, A, bytesA) ||
      tdls::overlaps(X, bytesB, B, bytesB))
    return -8;
  if (piv == nullptr || tdls::misaligned(piv, 4) || tdls::overlaps(piv, bytesP, A, bytesA) ||
      tdls::overlaps(piv, bytesP, B, bytesB) || tdls::overlaps(piv, bytesP, X, bytesB))
    return -9;
  if (info == nullptr || tdls::misaligned(info, 4) || tdls::overlaps(info, bytesI, A, bytesA) ||
      tdls::overlaps(info, bytesI, B, bytesB) || tdls::overlaps(info, bytesI, X, bytesB) ||
      tdls::overlaps(info, bytesI, piv, bytesP))
    return -10;

  rc = tdls::check_device();
  if (rc != 0) return rc;
  tdls::GesvLauncher launch = tdls::find_launcher(p.dtype, p.N, p.NRHS);
  if (launch == nullptr) return TDLS_ERR_NO_KERNEL;
  const int err = launch(p, A, B, X, piv, info, stream);
  if (err == (int)hipErrorInvalidConfiguration) return TDLS_ERR_NO_KERNEL;
  return err == 0 ? TDLS_SUCCESS : TDLS_ERR_LAUNCH;
}

const char* tdls_strerror(int code) {
  switch (code) {
    case TDLS_SUCCESS: return "success";
    case -1: return "argument 1 (dtype) is invalid";
    case -2: return "argument 2 (layout) is invalid";
    case -3: return "argument 3 (n) is outside 1..64";
    case -4: return "argument 4 (nrhs) is outside 1..8";
    case -5: return "argument 5 (batch) is negative or too large";
    case -6: return "argument 6 (A) is null or misaligned";
    case -7: return "argument 7 (B) is null or misaligned";
    case -8: return "argument 8 (X) is null, misaligned or overlaps an input";
    case -9: return "argument 9 (piv) is null, misaligned or overlaps another buffer";
    case -10: return "argument 10 (info) is null, misaligned or overlaps another buffer";
    case TDLS_ERR_LAUNCH: return "the kernel launch failed";
    case TDLS_ERR_DEVICE: return "the current device is not an MI355X (gfx950)";
    case TDLS_ERR_HIP: return "a HIP runtime query failed";
    case TDLS_ERR_NO_KERNEL: return "no kernel is built for this shape and group size";
    default: return "unknown tdls return code";
  }
}

const char* tdls_version(void) { return "tdls-mi355x 0.1.0 gfx950"; }

}  // extern "C"
