// One shape's launcher: compiled once per entry of TDLS_FOR_EACH_SHAPE with
// -DTDLS_INST_SFX=<f32|f64> -DTDLS_INST_REAL=<float|double>
// -DTDLS_INST_N=<N> -DTDLS_INST_NRHS=<NRHS>, so that the kernels build in
// parallel.
#include "gesv_panel.hpp"
#include "getrs_kernel.hpp"
#include "chol_kernel.hpp"

#include <tuple>

#if !defined(TDLS_INST_SFX) || !defined(TDLS_INST_REAL) || !defined(TDLS_INST_N) || \
    !defined(TDLS_INST_NRHS)
#error "gesv_inst.hip is compiled once per shape with the TDLS_INST_* macros defined"
#endif

#define TDLS_LAUNCHER_NAME_(sfx, N, NRHS) launch_gesv_##sfx##_n##N##_r##NRHS
#define TDLS_LAUNCHER_NAME(sfx, N, NRHS) TDLS_LAUNCHER_NAME_(sfx, N, NRHS)

namespace tdls {

// Enqueue `kernel` and return the status of this launch alone.  The
// arguments are converted to the kernel's parameter types and passed by
// address (hipLaunchKernel), so the per-thread "last error" of the HIP
// runtime is neither read nor cleared here: an earlier error of the caller
// is left for the caller, and a failure of this launch is reported as this
// launch's.
template <typename... P, typename... Arg>
static int launch_kernel(void (*kernel)(P...), unsigned grid, unsigned threads, int lds,
                         hipStream_t stream, Arg... arg) {
  static_assert(sizeof...(P) == sizeof...(Arg), "argument count of the kernel");
  std::tuple<P...> vals(static_cast<P>(arg)...);
  void* ptrs[sizeof...(P)];
  std::apply([&](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return (int)hipLaunchKernel(reinterpret_cast<const void*>(kernel), dim3(grid), dim3(threads),
                              ptrs, (size_t)lds, stream);
}

template <typename Real, int N, int NRHS, int T, bool FACT>
static int launch_panel(const LaunchPlan& p, const void* A, const void* B, void* X,
                        int32_t* piv, int32_t* info, hipStream_t stream) {
  constexpr int PB = panel_width(N, NRHS, sizeof(Real) == 8, T, FACT);
  using S = PanelShape<Real, N, NRHS, T, PB>;
  static_assert(S::BLOCK_BYTES == gesv_lds_bytes(N, NRHS, T, sizeof(Real) == 8),
                "host and device LDS sizes disagree");
  if (p.lds_bytes != S::BLOCK_BYTES) return (int)hipErrorInvalidConfiguration;
  if constexpr (S::BLOCK_BYTES > 65536) {
    // Dynamic LDS above 64 KiB has to be allowed per kernel; done once (the
    // static is initialised thread-safely) and the outcome kept.
    static const hipError_t allowed = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&gesv_panel_kernel<Real, N, NRHS, T, PB, FACT>),
        hipFuncAttributeMaxDynamicSharedMemorySize, S::BLOCK_BYTES);
    if (allowed != hipSuccess) return (int)allowed;
  }
  return launch_kernel(&gesv_panel_kernel<Real, N, NRHS, T, PB, FACT>, (unsigned)p.grid,
                       (unsigned)p.threads_per_block, S::BLOCK_BYTES, stream, p.layout, p.n,
                       p.nrhs, p.batch, static_cast<const Real*>(A), static_cast<const Real*>(B),
                       static_cast<Real*>(X), piv, info, p.flags, p.interleave);
}

template <typename Real, int N, int NRHS, int T>
static int launch_getrs(const LaunchPlan& p, const void* LU, const void* B, void* X,
                        const int32_t* piv, hipStream_t stream) {
  using S = GetrsShape<Real, N, NRHS, T>;
  static_assert(S::BLOCK_BYTES == getrs_lds_bytes(N, NRHS, T, sizeof(Real) == 8),
                "host and device LDS sizes disagree");
  if (p.lds_bytes != S::BLOCK_BYTES) return (int)hipErrorInvalidConfiguration;
  return launch_kernel(&getrs_kernel<Real, N, NRHS, T>, (unsigned)p.grid,
                       (unsigned)p.threads_per_block, S::BLOCK_BYTES, stream, p.layout, p.n,
                       p.nrhs, p.batch, static_cast<const Real*>(LU), piv,
                       static_cast<const Real*>(B), static_cast<Real*>(X), p.interleave);
}

template <typename Real, int N, int NRHS, int T, bool FACT, bool SOLVE = false>
static int launch_chol(const LaunchPlan& p, const void* A, const void* B, void* X,
                       int32_t* info, hipStream_t stream) {
  if constexpr (T == 32) {
    return (int)hipErrorInvalidConfiguration;   // no Cholesky kernel for 32-lane groups
  } else {
    using S = CholShape<Real, N, NRHS, T>;
    static_assert(S::BLOCK_BYTES == chol_lds_bytes(N, NRHS, T, sizeof(Real) == 8),
                  "host and device LDS sizes disagree");
    static_assert(S::BLOCK_BYTES <= 65536, "Cholesky LDS stays within the default limit");
    if (p.lds_bytes != S::BLOCK_BYTES) return (int)hipErrorInvalidConfiguration;
    return launch_kernel(&chol_kernel<Real, N, NRHS, T, FACT, SOLVE>, (unsigned)p.grid,
                         (unsigned)p.threads_per_block, S::BLOCK_BYTES, stream, p.layout, p.n,
                         p.nrhs, p.batch, (Real)p.shift, static_cast<const Real*>(A),
                         static_cast<const Real*>(B), static_cast<Real*>(X), info, p.interleave);
  }
}

template <typename Real, int N, int NRHS, int T>
static int launch_op(const LaunchPlan& p, const void* in0, const void* in1, void* out,
                     int32_t* piv, int32_t* info, hipStream_t stream) {
  switch (p.op) {
    case kOpGesv:
      return launch_panel<Real, N, NRHS, T, false>(p, in0, in1, out, piv, info, stream);
    case kOpGetrf:
      if constexpr (NRHS == 1)
        return launch_panel<Real, N, NRHS, T, true>(p, in0, nullptr, out, piv, info, stream);
      else
        return (int)hipErrorInvalidConfiguration;
    case kOpGetrs:
      return launch_getrs<Real, N, NRHS, T>(p, in0, in1, out, piv, stream);
    case kOpPotrf:
      if constexpr (NRHS == 1)
        return launch_chol<Real, N, NRHS, T, true>(p, in0, nullptr, out, info, stream);
      else
        return (int)hipErrorInvalidConfiguration;
    case kOpPosv:
      return launch_chol<Real, N, NRHS, T, false>(p, in0, in1, out, info, stream);
    case kOpPotrs:
      return launch_chol<Real, N, NRHS, T, false, true>(p, in0, in1, out, nullptr, stream);
    default:
      return (int)hipErrorInvalidConfiguration;
  }
}

int TDLS_LAUNCHER_NAME(TDLS_INST_SFX, TDLS_INST_N, TDLS_INST_NRHS)(
    const LaunchPlan& p, const void* in0, const void* in1, void* out, int32_t* piv,
    int32_t* info, hipStream_t stream) {
  using Real = TDLS_INST_REAL;
  constexpr int N = TDLS_INST_N;
  constexpr int NRHS = TDLS_INST_NRHS;
  constexpr bool is64 = sizeof(Real) == 8;
  constexpr int T0 = pick_group_size(N, NRHS, is64);
  constexpr int T1 = alt_group_size(N, NRHS, is64);
  if (p.N != N || p.NRHS != NRHS) return (int)hipErrorInvalidConfiguration;
  if (p.T == T0) return launch_op<Real, N, NRHS, T0>(p, in0, in1, out, piv, info, stream);
  if constexpr (T1 != 0) {
    if (p.T == T1) return launch_op<Real, N, NRHS, T1>(p, in0, in1, out, piv, info, stream);
  }
  return (int)hipErrorInvalidConfiguration;
}

}  // namespace tdls
