// Internal declarations shared by the host-side entry points and the kernel
// translation units.  Not part of the public interface (include/tdls.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tdls {

// Compile-time shapes the kernels are built for, as X(sfx, Real, N, NRHS).
// A call with n <= N and nrhs <= NRHS runs the smallest such (N, NRHS)
// kernel with the matrix padded by an identity block and the right-hand
// sides by zero columns (see the loader).  The build script reads this list.
#define TDLS_FOR_EACH_SHAPE(X)                                                              \
  X(f32, float, 8, 1) X(f32, float, 8, 2) X(f32, float, 8, 4) X(f32, float, 8, 8)            \
  X(f32, float, 16, 1) X(f32, float, 16, 2) X(f32, float, 16, 4) X(f32, float, 16, 8)        \
  X(f32, float, 24, 1) X(f32, float, 24, 2) X(f32, float, 24, 4) X(f32, float, 24, 8)        \
  X(f32, float, 32, 1) X(f32, float, 32, 2) X(f32, float, 32, 4) X(f32, float, 32, 8)        \
  X(f32, float, 48, 1) X(f32, float, 48, 2) X(f32, float, 48, 4) X(f32, float, 48, 8)        \
  X(f32, float, 64, 1) X(f32, float, 64, 2) X(f32, float, 64, 4) X(f32, float, 64, 8)        \
  X(f64, double, 8, 1) X(f64, double, 8, 2) X(f64, double, 8, 4) X(f64, double, 8, 8)        \
  X(f64, double, 16, 1) X(f64, double, 16, 2) X(f64, double, 16, 4) X(f64, double, 16, 8)    \
  X(f64, double, 24, 1) X(f64, double, 24, 2) X(f64, double, 24, 4) X(f64, double, 24, 8)    \
  X(f64, double, 32, 1) X(f64, double, 32, 2) X(f64, double, 32, 4) X(f64, double, 32, 8)    \
  X(f64, double, 48, 1) X(f64, double, 48, 2) X(f64, double, 48, 4) X(f64, double, 48, 8)    \
  X(f64, double, 64, 1) X(f64, double, 64, 2) X(f64, double, 64, 4) X(f64, double, 64, 8)

constexpr int kNumN = 6;
constexpr int kNValues[kNumN] = {8, 16, 24, 32, 48, 64};
constexpr int kNumNrhs = 4;
constexpr int kNrhsValues[kNumNrhs] = {1, 2, 4, 8};

constexpr int kWaveSize = 64;
// One wave per block: waves share nothing, and the LDS a block holds is then
// one wave's records and triangular store, so as many waves fit on a CU as
// its 160 KiB of LDS and the register file allow (a 4-wave block of n = 64
// float64 systems would need 81 KiB and leave one wave per SIMD).
constexpr int kWavesPerBlock = 1;

// Options of a call (tdls_options.flags): whole-matrix max-abs scaling of
// the LU (gesv, getrf).
constexpr uint32_t kFlagScaleMaxAbs = 1u;

// Operations the library launches.
enum OpKind : int {
  kOpGesv = 0,
  kOpGetrf = 1,
  kOpGetrs = 2,
  kOpPotrf = 3,
  kOpPosv = 4,
  kOpPotrs = 5
};

// Everything a launch needs, decided on the host before any launch.
struct LaunchPlan {
  int op;             // OpKind
  int dtype;          // 0 f32, 1 f64
  int layout;         // 0 row-major, 1 column-major
  int n, nrhs;        // problem
  int N, NRHS;        // kernel instantiation (N >= n, NRHS >= nrhs)
  int T;              // lanes per system (group size), power of two
  int R;              // rows per lane, ceil(N / T)
  int G;              // systems per wave, 64 / T
  int64_t batch;
  double shift;       // Cholesky: explicit diagonal shift (0 otherwise)
  uint32_t flags;     // kFlag* options of the call
  int64_t interleave; // systems interleaved element by element (1: one after another)
  int64_t systems_per_block;
  int64_t grid;
  int threads_per_block;
  int lds_bytes;
};

// Group size chosen at compile time for each instantiation: the smallest of
// 4, 16, 64 lanes whose rows fit a register budget (4 lanes up to N = 24).
// Registers per lane for the data rows are R * (N + NRHS) * (element size /
// 4) with R = ceil(N / T); fewer lanes per system means more systems share
// each wave's pivot search, divisions and exchanges, and fewer phantom rows
// (N = 24 in 16-lane groups pads its second slot with 8 of them).  4 and 16
// lanes are DPP broadcast domains (quad, row); 64 lanes is the whole wave.
// Measured at N = 24 float32 on 1,000,000 row-major systems, 16 -> 4 lanes:
// gesv 1.18 -> 0.85 ms (one right-hand side) and 1.24 -> 0.95 ms (two),
// getrf 1.23 -> 1.07, potrf 1.31 -> 1.00, posv 1.02 -> 0.57, potrs 0.62 ->
// 0.51 ms, at two waves per SIMD against five.
constexpr int kRegBudget = 160;
constexpr int rows_per_lane(int N, int T) { return (N + T - 1) / T; }
constexpr int row_regs(int N, int NRHS, int T, bool is64) {
  return rows_per_lane(N, T) * (N + NRHS) * (is64 ? 2 : 1);
}
constexpr int pick_group_size(int N, int NRHS, bool is64) {
  if (N <= 24 && row_regs(N, NRHS, 4, is64) <= kRegBudget) return 4;
  if (row_regs(N, NRHS, 16, is64) <= kRegBudget) return 16;
  return 64;
}

// A second group size built for the smaller shapes (the next larger of 4,
// 16, 64), so that the tests can check that results do not depend on it
// (the arithmetic and its order are the same).  0 when none is built.
// SIMDs of an MI355X (256 CUs x 4).  A batch small enough that even the
// wider alternative group gives at most one wave per SIMD runs at that
// wider group: more waves, each with a shorter chain.  Measured: n = 16
// float32 with 4 right-hand sides, 4096 systems, 16.1 -> 9.0 us; n = 32
// float64, 512 systems, 19.6 -> 16.0 us, while at 2048 systems the
// narrower group stays ahead (21.6 vs 23.2 us).
constexpr int64_t kSimds = 1024;

constexpr int alt_group_size(int N, int NRHS, bool is64) {
  const int t0 = pick_group_size(N, NRHS, is64);
  return (N <= 32 && t0 < 64) ? (t0 == 4 ? 16 : 64) : 0;
}

// The LU operations in float64 at N = 16 run the 16-lane group (one row per
// lane) rather than the quad (four rows per lane, twice the registers of a
// float32 row): measured on 65,536 and 1,048,576 systems, gesv 0.102 ->
// 0.059 ms and 1.29 -> 0.95 ms (nrhs = 4), getrs 0.81 -> 0.62 ms, getrf
// even.  The Cholesky kernels keep the quad (potrf 0.94 against 1.14 ms,
// posv 0.68 against 1.07 ms at the larger batch); at N = 8 and in float32
// the quad is ahead for every operation but getrs at N = 24 (six rows per
// lane), which keeps the 16-lane group: 0.48 against 0.49 ms with one
// right-hand side, 0.53 against 0.58 ms with two (1,000,000 systems).
constexpr bool lu_prefers_wider(int op, int N, bool is64, int T0, int T1) {
  if (T0 != 4 || T1 != 16) return false;
  if (is64 && N == 16) return op == kOpGesv || op == kOpGetrf || op == kOpGetrs;
  return !is64 && N == 24 && op == kOpGetrs;
}

// LU solves (gesv) whose registers, with panels of two columns instead of
// four, fit one more wave per SIMD, and that wave count, which the kernel
// declares as its minimum occupancy (0: panels of four, no declaration).
// Two columns halve the pivot-row entries and multipliers a step holds in
// registers; the records are exchanged twice as often, which costs more
// than it gives at the same occupancy (n = 32 float64: 0.887 -> 0.923 ms).
// Measured against panels of four (HIP events, 262,144 row-major systems
// unless stated; VGPRs before -> after):
//   float64 n = 32, 1 rhs, 16 lanes: 203 -> 168 (4 spilled), 2 -> 3 waves,
//     0.780 -> 0.753 ms (column-major headline shape);
//   float64 n = 24, 16 lanes: 1 rhs 171 -> 143, 0.587 -> 0.559 ms; 2 rhs
//     177 -> 149, 0.655 -> 0.622 ms; 4 rhs 187 -> 157, 0.702 -> 0.664 ms;
//   float64 n = 48, 64 lanes (131,072 systems): 4 rhs 169 -> 145, 1.690 ->
//     1.608 ms; 8 rhs 181 -> 153, 1.845 -> 1.788 ms;
//   float32 n = 32, 8 rhs, 16 lanes: 129 -> 113, 3 -> 4 waves, 0.675 ->
//     0.662 ms.
// Not taken: getrf (n = 32 float64 spills 14 at three waves, 0.895 -> 0.927
// ms; n = 24 even), float32 n = 16 quads with 2 or 4 rhs (even or slower),
// float64 n = 8 quads with 8 rhs (a fourth wave spills 35 registers: 0.432
// -> 0.549 ms).
constexpr int lu_min_waves(int N, int NRHS, bool is64, int T, bool fact) {
  if (fact) return 0;
  if (is64 && N == 32 && NRHS == 1 && T == 16) return 3;
  if (is64 && N == 24 && NRHS <= 4 && T == 16) return 3;
  if (is64 && N == 48 && NRHS >= 4 && T == 64) return 3;
  if (!is64 && N == 32 && NRHS == 8 && T == 16) return 4;
  return 0;
}

// Panel width of the factorization (columns whose pivot rows are exchanged
// together through LDS): kPanelMax, or 2 where that gives another wave per
// SIMD (lu_min_waves).
constexpr int kPanelMax = 4;
constexpr int panel_width(int N, int NRHS, bool is64, int T, bool fact) {
  if (N < kPanelMax) return N;
  return lu_min_waves(N, NRHS, is64, T, fact) > 0 ? 2 : kPanelMax;
}

// The LU solve keeps U in registers for the back substitution when one
// right-hand side is broadcast inside a DPP domain (quads, 16-lane rows):
// after a last compaction every slot holds its positions in order, so x_k
// reaches the rows above from a fixed lane.  Otherwise U goes to a packed
// triangle in LDS (several right-hand sides split over column classes;
// whole-wave groups).
constexpr bool lu_solve_in_registers(int NRHS, int T) { return NRHS == 1 && (T == 4 || T == 16); }

// LDS a wave of the LU kernels may take so that twelve waves (three per
// SIMD) fit the 160 KiB of a CU.
constexpr int kLuLdsPerWave = 13312;

// LDS elements of one group of the LU kernels: the B pivot-row records of
// N + NRHS entries (rounded up to 16 bytes) and, where U stays in
// registers, a staging area for putting rows back in position order (the
// whole tile when it fits kLuLdsPerWave, else chunks of it); otherwise the
// N x NRHS right-hand sides by position and the packed upper triangle of U
// of the back substitution (the last two occupy the same area one after the
// other).
constexpr int lu_group_elems(int N, int NRHS, int T, bool is64) {
  const int es = is64 ? 8 : 4;
  const int vec = 16 / es;
  const int stride = (N + NRHS + vec - 1) / vec * vec;
  const int B = N < kPanelMax ? N : kPanelMax;   // records of the widest panel
  const int rec = B * stride;
  if (lu_solve_in_registers(NRHS, T)) {
    const int budget = kLuLdsPerWave / (kWaveSize / T) / es / vec * vec;
    const int tile = (N * (N + NRHS) + vec - 1) / vec * vec;
    const int stage = tile < budget ? tile : budget;
    return rec > stage ? rec : stage;
  }
  const int utri = (N * (N + 1) / 2 + vec - 1) / vec * vec;
  const int big1 = rec > utri ? rec : utri;
  return big1 > N * NRHS ? big1 : N * NRHS;
}

// LDS bytes of one block (one wave) of the LU kernels (gesv, getrf).
constexpr int gesv_lds_bytes(int N, int NRHS, int T, bool is64) {
  return kWavesPerBlock * (kWaveSize / T) * lu_group_elems(N, NRHS, T, is64) * (is64 ? 8 : 4);
}

// LDS bytes of one block (one wave) of the getrs kernel: per group, the
// swap sequence (N int32, rounded up to 16 bytes) and, with four or more
// right-hand sides, the larger of the right-hand sides by position and a
// packed triangle (L for the forward, then U for the back substitution).
constexpr int getrs_lds_bytes(int N, int NRHS, int T, bool is64) {
  const int es = is64 ? 8 : 4;
  const int vec = 16 / es;
  const int piv = (N * 4 + 15) / 16 * 16;
  const int utri = (N * (N + 1) / 2 + vec - 1) / vec * vec;
  const int tri = utri > N * NRHS ? utri : N * NRHS;
  const int elems = NRHS >= 4 ? (tri + vec - 1) / vec * vec : 0;
  // 16- and 64-lane groups put B in pivoted order through LDS: the class
  // area when there is one, else a staging area of N x NRHS
  const int stage = (T >= 16 && NRHS < 4) ? (N * NRHS * es + 15) / 16 * 16 : 0;
  return kWavesPerBlock * (kWaveSize / T) * (piv + elems * es + stage);
}

// LDS bytes of one block (one wave) of the Cholesky kernel: per group, the
// largest of a symmetry-check chunk (min(T, 16) rows of stride N + 1), the
// right-hand sides by position and the packed triangle of the back
// substitution, rounded up to 16 bytes.
constexpr int chol_lds_bytes(int N, int NRHS, int T, bool is64) {
  const int es = is64 ? 8 : 4;
  const int vec = 16 / es;
  const int ch = T < 16 ? T : 16;
  const int utri = (N * (N + 1) / 2 + vec - 1) / vec * vec;
  const int big1 = ch * (N + 1) > utri ? ch * (N + 1) : utri;
  const int big2 = big1 > N * NRHS ? big1 : N * NRHS;
  return kWavesPerBlock * (kWaveSize / T) * ((big2 + vec - 1) / vec * vec) * es;
}

// Launchers, one per shape of TDLS_FOR_EACH_SHAPE, defined in the
// instantiation translation units.  They enqueue the kernel of p.op and p.T
// and return a hipError_t value cast to int.  Operands by op:
//   gesv:  in0 = A, in1 = B, out = X, piv and info written;
//   getrf: in0 = A, out = LU, piv and info written (NRHS = 1 shapes only);
//   getrs: in0 = LU, in1 = B, out = X, piv read, info unused;
//   potrf: in0 = A, out = L, info written (NRHS = 1 shapes only);
//   posv:  in0 = A, in1 = B, out = X, info written.
using GesvLauncher = int (*)(const LaunchPlan& p, const void* in0, const void* in1, void* out,
                             int32_t* piv, int32_t* info, hipStream_t stream);
#define TDLS_DECLARE_LAUNCHER(sfx, Real, N, NRHS)                                              \
  int launch_gesv_##sfx##_n##N##_r##NRHS(const LaunchPlan& p, const void* in0,                \
                                         const void* in1, void* out, int32_t* piv,            \
                                         int32_t* info, hipStream_t stream);
TDLS_FOR_EACH_SHAPE(TDLS_DECLARE_LAUNCHER)
#undef TDLS_DECLARE_LAUNCHER

}  // namespace tdls
