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
#include <cmath>

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

int check_device();

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

// Scalar checks and launch plan of one operation.  The factorization runs
// with one (unused) right-hand side, so `nrhs` is 1 for it.
int make_plan(int op, int dtype, int layout, int n, int nrhs, int64_t batch, LaunchPlan* p) {
  int rc = check_scalars(dtype, layout, n, nrhs, batch);
  if (rc != 0) return rc;
  const bool is64 = dtype == TDLS_F64;
  int N = 0, NRHS = 0;
  for (int v : kNValues)
    if (v >= n) { N = v; break; }
  for (int v : kNrhsValues)
    if (v >= nrhs) { NRHS = v; break; }
  p->op = op;
  const int T0 = pick_group_size(N, NRHS, is64);
  const int T1 = alt_group_size(N, NRHS, is64);
  int T = T0;
  const int64_t waves0 = (batch + kWaveSize / T0 - 1) / (kWaveSize / T0);
  if (T1 > T0 && waves0 * (T1 / T0) <= kSimds) T = T1;   // small batch: more, shorter waves
  if (lu_prefers_wider(op, N, is64, T0, T1)) T = T1;
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
  p->shift = 0.0;
  p->flags = 0;
  p->interleave = 1;
  p->lds_bytes = op == kOpGetrs                    ? getrs_lds_bytes(N, NRHS, T, is64)
                 : (op == kOpPotrf || op == kOpPosv || op == kOpPotrs)
                     ? chol_lds_bytes(N, NRHS, T, is64)
                                                     : gesv_lds_bytes(N, NRHS, T, is64);
  return 0;
}

int fill_plan(const LaunchPlan& p, tdls_plan* out) {
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

int launch(const LaunchPlan& p, const void* in0, const void* in1, void* out, int32_t* piv,
           int32_t* info, hipStream_t stream) {
  int rc = check_device();
  if (rc != 0) return rc;
  GesvLauncher l = find_launcher(p.dtype, p.N, p.NRHS);
  if (l == nullptr) return TDLS_ERR_NO_KERNEL;
  const int err = l(p, in0, in1, out, piv, info, stream);
  if (err == (int)hipErrorInvalidConfiguration) return TDLS_ERR_NO_KERNEL;
  return err == 0 ? TDLS_SUCCESS : TDLS_ERR_LAUNCH;
}

// Options of the *_ex calls: flags allowed for the operation, reserved
// field zero, an interleave of 0 or 1 (systems one after another) or of 2 ..
// batch systems.
bool bad_options(const tdls_options* opt, uint32_t allowed_flags, int64_t batch) {
  if (opt == nullptr) return false;
  if ((opt->flags & ~allowed_flags) != 0 || opt->reserved != 0) return true;
  return opt->interleave < 0 || (opt->interleave > 1 && batch > 0 && opt->interleave > batch);
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
  int rc = tdls::make_plan(tdls::kOpGesv, (int)dtype, (int)layout, n, nrhs, batch, &p);
  if (rc != 0) return rc;
  return tdls::fill_plan(p, out);
}

int tdls_plan_op(tdls_op op, tdls_dtype dtype, tdls_layout layout, int n, int nrhs,
                 int64_t batch, tdls_plan* out) {
  if (op != TDLS_OP_GESV && op != TDLS_OP_GETRF && op != TDLS_OP_GETRS && op != TDLS_OP_POTRF &&
      op != TDLS_OP_POSV && op != TDLS_OP_POTRS)
    return -1;
  tdls::LaunchPlan p;
  const bool factor = op == TDLS_OP_GETRF || op == TDLS_OP_POTRF;
  int rc = tdls::make_plan((int)op, (int)dtype, (int)layout, n, factor ? 1 : nrhs, batch, &p);
  if (rc != 0) return rc < 0 ? rc - 1 : rc;   // argument numbers shift by one
  rc = tdls::fill_plan(p, out);
  return rc == -6 ? -7 : rc;
}

}  // extern "C"

namespace tdls {
namespace {

// What the *_ex calls add: option flags, the batch interleave W (element e
// of system s at (s / W) W E + (s % W) + e W for systems of E elements), and
// `po`, the shift of the pointer arguments' numbers (1 after an options
// argument).
struct Extra {
  uint32_t flags = 0;
  int64_t ilv = 1;
  int po = 0;
};

Extra extra_of(const tdls_options* opt) {
  Extra x;
  x.po = 1;
  if (opt != nullptr) {
    x.flags = opt->flags;
    x.ilv = opt->interleave <= 1 ? 1 : opt->interleave;
  }
  return x;
}

// Bytes spanned by a buffer of `batch` systems of E elements under
// interleave W: whole blocks of W systems.
size_t span(int64_t batch, int64_t W, int64_t E, size_t es) {
  const int64_t blocks = (batch + W - 1) / W;
  return (size_t)blocks * (size_t)W * (size_t)E * es;
}

int gesv_call(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
              const Extra& x, const void* A, const void* B, void* X, int32_t* piv,
              int32_t* info, hipStream_t stream) {
  tdls::LaunchPlan p;
  int rc = tdls::make_plan(tdls::kOpGesv, (int)dtype, (int)layout, n, nrhs, batch, &p);
  if (rc != 0) return rc;
  if (batch == 0) return TDLS_SUCCESS;  // nothing to read or write, nothing launched
  p.flags = x.flags;
  p.interleave = x.ilv;
  const int po = x.po;

  const size_t es = dtype == TDLS_F64 ? 8 : 4;
  const size_t bytesA = span(batch, x.ilv, (int64_t)n * n, es);
  const size_t bytesB = span(batch, x.ilv, (int64_t)n * nrhs, es);
  const size_t bytesP = span(batch, x.ilv, n, 4);
  const size_t bytesI = (size_t)batch * 4;
  if (A == nullptr || tdls::misaligned(A, es)) return -6 - po;
  if (B == nullptr || tdls::misaligned(B, es)) return -7 - po;
  if (X == nullptr || tdls::misaligned(X, es) || tdls::overlaps(X, bytesB, A, bytesA) ||
      tdls::overlaps(X, bytesB, B, bytesB))
    return -8 - po;
  if (piv == nullptr || tdls::misaligned(piv, 4) || tdls::overlaps(piv, bytesP, A, bytesA) ||
      tdls::overlaps(piv, bytesP, B, bytesB) || tdls::overlaps(piv, bytesP, X, bytesB))
    return -9 - po;
  if (info == nullptr || tdls::misaligned(info, 4) || tdls::overlaps(info, bytesI, A, bytesA) ||
      tdls::overlaps(info, bytesI, B, bytesB) || tdls::overlaps(info, bytesI, X, bytesB) ||
      tdls::overlaps(info, bytesI, piv, bytesP))
    return -10 - po;
  return tdls::launch(p, A, B, X, piv, info, stream);
}

int getrf_call(tdls_dtype dtype, tdls_layout layout, int n, int64_t batch, const Extra& x,
               const void* A, void* LU, int32_t* piv, int32_t* info, hipStream_t stream) {
  tdls::LaunchPlan p;
  int rc = tdls::make_plan(tdls::kOpGetrf, (int)dtype, (int)layout, n, 1, batch, &p);
  if (rc == -5) return -4;   // batch is argument 4 here
  if (rc != 0) return rc;
  if (batch == 0) return TDLS_SUCCESS;
  p.flags = x.flags;
  p.interleave = x.ilv;
  const int po = x.po;

  const size_t es = dtype == TDLS_F64 ? 8 : 4;
  const size_t bytesA = span(batch, x.ilv, (int64_t)n * n, es);
  const size_t bytesP = span(batch, x.ilv, n, 4);
  const size_t bytesI = (size_t)batch * 4;
  if (A == nullptr || tdls::misaligned(A, es)) return -5 - po;
  if (LU == nullptr || tdls::misaligned(LU, es) || tdls::overlaps(LU, bytesA, A, bytesA))
    return -6 - po;
  if (piv == nullptr || tdls::misaligned(piv, 4) || tdls::overlaps(piv, bytesP, A, bytesA) ||
      tdls::overlaps(piv, bytesP, LU, bytesA))
    return -7 - po;
  if (info == nullptr || tdls::misaligned(info, 4) || tdls::overlaps(info, bytesI, A, bytesA) ||
      tdls::overlaps(info, bytesI, LU, bytesA) || tdls::overlaps(info, bytesI, piv, bytesP))
    return -8 - po;
  return tdls::launch(p, A, nullptr, LU, piv, info, stream);
}

int getrs_call(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
               const Extra& x, const void* LU, const int32_t* piv, const void* B, void* X,
               hipStream_t stream) {
  tdls::LaunchPlan p;
  int rc = tdls::make_plan(tdls::kOpGetrs, (int)dtype, (int)layout, n, nrhs, batch, &p);
  if (rc != 0) return rc;
  if (batch == 0) return TDLS_SUCCESS;
  p.interleave = x.ilv;
  const int po = x.po;

  const size_t es = dtype == TDLS_F64 ? 8 : 4;
  const size_t bytesLU = span(batch, x.ilv, (int64_t)n * n, es);
  const size_t bytesP = span(batch, x.ilv, n, 4);
  const size_t bytesB = span(batch, x.ilv, (int64_t)n * nrhs, es);
  if (LU == nullptr || tdls::misaligned(LU, es)) return -6 - po;
  if (piv == nullptr || tdls::misaligned(piv, 4)) return -7 - po;
  if (B == nullptr || tdls::misaligned(B, es)) return -8 - po;
  if (X == nullptr || tdls::misaligned(X, es) || tdls::overlaps(X, bytesB, LU, bytesLU) ||
      tdls::overlaps(X, bytesB, piv, bytesP) || tdls::overlaps(X, bytesB, B, bytesB))
    return -9 - po;
  return tdls::launch(p, LU, B, X, const_cast<int32_t*>(piv), nullptr, stream);
}

int potrf_call(tdls_dtype dtype, tdls_layout layout, int n, int64_t batch, double shift,
               const Extra& x, const void* A, void* L, int32_t* info, hipStream_t stream) {
  tdls::LaunchPlan p;
  int rc = tdls::make_plan(tdls::kOpPotrf, (int)dtype, (int)layout, n, 1, batch, &p);
  if (rc == -5) return -4;   // batch is argument 4 here
  if (rc != 0) return rc;
  if (!std::isfinite(shift)) return -5;
  if (batch == 0) return TDLS_SUCCESS;
  p.shift = shift;
  p.interleave = x.ilv;
  const int po = x.po;

  const size_t es = dtype == TDLS_F64 ? 8 : 4;
  const size_t bytesA = span(batch, x.ilv, (int64_t)n * n, es);
  const size_t bytesI = (size_t)batch * 4;
  if (A == nullptr || tdls::misaligned(A, es)) return -6 - po;
  if (L == nullptr || tdls::misaligned(L, es) || tdls::overlaps(L, bytesA, A, bytesA))
    return -7 - po;
  if (info == nullptr || tdls::misaligned(info, 4) || tdls::overlaps(info, bytesI, A, bytesA) ||
      tdls::overlaps(info, bytesI, L, bytesA))
    return -8 - po;
  return tdls::launch(p, A, nullptr, L, nullptr, info, stream);
}

int potrs_call(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
               const Extra& x, const void* L, const void* B, void* X, hipStream_t stream) {
  tdls::LaunchPlan p;
  int rc = tdls::make_plan(tdls::kOpPotrs, (int)dtype, (int)layout, n, nrhs, batch, &p);
  if (rc != 0) return rc;
  if (batch == 0) return TDLS_SUCCESS;
  p.interleave = x.ilv;
  const int po = x.po;

  const size_t es = dtype == TDLS_F64 ? 8 : 4;
  const size_t bytesL = span(batch, x.ilv, (int64_t)n * n, es);
  const size_t bytesB = span(batch, x.ilv, (int64_t)n * nrhs, es);
  if (L == nullptr || tdls::misaligned(L, es)) return -6 - po;
  if (B == nullptr || tdls::misaligned(B, es)) return -7 - po;
  if (X == nullptr || tdls::misaligned(X, es) || tdls::overlaps(X, bytesB, L, bytesL) ||
      tdls::overlaps(X, bytesB, B, bytesB))
    return -8 - po;
  return tdls::launch(p, L, B, X, nullptr, nullptr, stream);
}

int posv_call(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
              double shift, const Extra& x, const void* A, const void* B, void* X,
              int32_t* info, hipStream_t stream) {
  tdls::LaunchPlan p;
  int rc = tdls::make_plan(tdls::kOpPosv, (int)dtype, (int)layout, n, nrhs, batch, &p);
  if (rc != 0) return rc;
  if (!std::isfinite(shift)) return -6;
  if (batch == 0) return TDLS_SUCCESS;
  p.shift = shift;
  p.interleave = x.ilv;
  const int po = x.po;

  const size_t es = dtype == TDLS_F64 ? 8 : 4;
  const size_t bytesA = span(batch, x.ilv, (int64_t)n * n, es);
  const size_t bytesB = span(batch, x.ilv, (int64_t)n * nrhs, es);
  const size_t bytesI = (size_t)batch * 4;
  if (A == nullptr || tdls::misaligned(A, es)) return -7 - po;
  if (B == nullptr || tdls::misaligned(B, es)) return -8 - po;
  if (X == nullptr || tdls::misaligned(X, es) || tdls::overlaps(X, bytesB, A, bytesA) ||
      tdls::overlaps(X, bytesB, B, bytesB))
    return -9 - po;
  if (info == nullptr || tdls::misaligned(info, 4) || tdls::overlaps(info, bytesI, A, bytesA) ||
      tdls::overlaps(info, bytesI, B, bytesB) || tdls::overlaps(info, bytesI, X, bytesB))
    return -10 - po;
  return tdls::launch(p, A, B, X, nullptr, info, stream);
}

}  // namespace
}  // namespace tdls

extern "C" {

int tdls_gesv_batched(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                      const void* A, const void* B, void* X, int32_t* piv, int32_t* info,
                      hipStream_t stream) {
  return tdls::gesv_call(dtype, layout, n, nrhs, batch, tdls::Extra(), A, B, X, piv, info,
                         stream);
}

int tdls_gesv_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                         const tdls_options* opt, const void* A, const void* B, void* X,
                         int32_t* piv, int32_t* info, hipStream_t stream) {
  const int rc = tdls::check_scalars((int)dtype, (int)layout, n, nrhs, batch);
  if (rc != 0) return rc;
  if (tdls::bad_options(opt, TDLS_SCALE_MAXABS, batch)) return -6;
  return tdls::gesv_call(dtype, layout, n, nrhs, batch, tdls::extra_of(opt), A, B, X, piv,
                         info, stream);
}

int tdls_getrf_batched(tdls_dtype dtype, tdls_layout layout, int n, int64_t batch,
                       const void* A, void* LU, int32_t* piv, int32_t* info,
                       hipStream_t stream) {
  return tdls::getrf_call(dtype, layout, n, batch, tdls::Extra(), A, LU, piv, info, stream);
}

int tdls_getrf_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int64_t batch,
                          const tdls_options* opt, const void* A, void* LU, int32_t* piv,
                          int32_t* info, hipStream_t stream) {
  const int rc = tdls::check_scalars((int)dtype, (int)layout, n, 1, batch);
  if (rc != 0) return rc == -5 ? -4 : rc;
  if (tdls::bad_options(opt, TDLS_SCALE_MAXABS, batch)) return -5;
  return tdls::getrf_call(dtype, layout, n, batch, tdls::extra_of(opt), A, LU, piv, info,
                          stream);
}

int tdls_getrs_batched(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                       const void* LU, const int32_t* piv, const void* B, void* X,
                       hipStream_t stream) {
  return tdls::getrs_call(dtype, layout, n, nrhs, batch, tdls::Extra(), LU, piv, B, X, stream);
}

int tdls_getrs_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                          const tdls_options* opt, const void* LU, const int32_t* piv,
                          const void* B, void* X, hipStream_t stream) {
  const int rc = tdls::check_scalars((int)dtype, (int)layout, n, nrhs, batch);
  if (rc != 0) return rc;
  if (tdls::bad_options(opt, 0u, batch)) return -6;
  return tdls::getrs_call(dtype, layout, n, nrhs, batch, tdls::extra_of(opt), LU, piv, B, X,
                          stream);
}

int tdls_potrf_batched(tdls_dtype dtype, tdls_layout layout, int n, int64_t batch, double shift,
                       const void* A, void* L, int32_t* info, hipStream_t stream) {
  return tdls::potrf_call(dtype, layout, n, batch, shift, tdls::Extra(), A, L, info, stream);
}

int tdls_potrf_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int64_t batch,
                          double shift, const tdls_options* opt, const void* A, void* L,
                          int32_t* info, hipStream_t stream) {
  const int rc = tdls::check_scalars((int)dtype, (int)layout, n, 1, batch);
  if (rc != 0) return rc == -5 ? -4 : rc;
  if (!std::isfinite(shift)) return -5;
  if (tdls::bad_options(opt, 0u, batch)) return -6;
  return tdls::potrf_call(dtype, layout, n, batch, shift, tdls::extra_of(opt), A, L, info,
                          stream);
}

int tdls_potrs_batched(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                       const void* L, const void* B, void* X, hipStream_t stream) {
  return tdls::potrs_call(dtype, layout, n, nrhs, batch, tdls::Extra(), L, B, X, stream);
}

int tdls_potrs_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                          const tdls_options* opt, const void* L, const void* B, void* X,
                          hipStream_t stream) {
  const int rc = tdls::check_scalars((int)dtype, (int)layout, n, nrhs, batch);
  if (rc != 0) return rc;
  if (tdls::bad_options(opt, 0u, batch)) return -6;
  return tdls::potrs_call(dtype, layout, n, nrhs, batch, tdls::extra_of(opt), L, B, X, stream);
}

int tdls_posv_batched(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                      double shift, const void* A, const void* B, void* X, int32_t* info,
                      hipStream_t stream) {
  return tdls::posv_call(dtype, layout, n, nrhs, batch, shift, tdls::Extra(), A, B, X, info,
                         stream);
}

int tdls_posv_batched_ex(tdls_dtype dtype, tdls_layout layout, int n, int nrhs, int64_t batch,
                         double shift, const tdls_options* opt, const void* A, const void* B,
                         void* X, int32_t* info, hipStream_t stream) {
  const int rc = tdls::check_scalars((int)dtype, (int)layout, n, nrhs, batch);
  if (rc != 0) return rc;
  if (!std::isfinite(shift)) return -6;
  if (tdls::bad_options(opt, 0u, batch)) return -7;
  return tdls::posv_call(dtype, layout, n, nrhs, batch, shift, tdls::extra_of(opt), A, B, X,
                         info, stream);
}

const char* tdls_strerror(int code) {
  switch (code) {
    case TDLS_SUCCESS: return "success";
    case -1: return "argument 1 is invalid (dtype, or op for tdls_plan_op)";
    case -2: return "argument 2 is invalid (layout, or dtype for tdls_plan_op)";
    case -3: return "argument 3 is invalid (n outside 1..64, or layout for tdls_plan_op)";
    case -4: return "argument 4 is invalid (nrhs outside 1..8; batch for getrf; n for plan_op)";
    case -5: return "argument 5 is invalid (batch; A for getrf; shift for potrf; nrhs for plan_op; options for getrf_ex)";
    case -6: return "argument 6 is invalid (null, misaligned or overlapping buffer; shift for posv; batch for plan_op; options for gesv_ex, getrs_ex, potrf_ex)";
    case -7: return "argument 7 is invalid (null, misaligned or overlapping buffer; options for posv_ex)";
    case -8: return "argument 8 is invalid (null, misaligned or overlapping buffer)";
    case -9: return "argument 9 is invalid (null, misaligned or overlapping buffer)";
    case -10: return "argument 10 is invalid (null, misaligned or overlapping buffer)";
    case -11: return "argument 11 is invalid (null, misaligned or overlapping buffer)";
    case TDLS_ERR_LAUNCH: return "the kernel launch failed";
    case TDLS_ERR_DEVICE: return "the current device is not an MI355X (gfx950)";
    case TDLS_ERR_HIP: return "a HIP runtime query failed";
    case TDLS_ERR_NO_KERNEL: return "no kernel is built for this shape and group size";
    default: return "unknown tdls return code";
  }
}

const char* tdls_version(void) { return "tdls-mi355x 0.1.0 gfx950"; }

}  // extern "C"
