// Batched gesv, panel kernel: LU with partial row pivoting plus forward and
// back substitution, one n x n system per group of T lanes of a wave64
// (T = 4, 16 or 64 as the planner picks; the templates also take T = 32,
// which was measured slower and is not planned), rows held in VGPRs.
//
// What is computed (cited by page title and section):
//  * "solver_static.hpp File Reference" (TDLS CooperativeLUpp), Detailed
//    Description: right-looking LU with partial pivoting of rows held by a
//    group of lanes, lane tx holding rows tx, tx+T, ...; the forward
//    substitution L y = P b carried by every elimination step, then U x = y.
//    Its logical row interchanges (rows never move, each row tracks its
//    position in the pivoted order) are the scheme used here.  "Departures
//    from the MAGMA kernel": several systems per wave, phantom rows skipped,
//    each solution entry kept by the lane owning its row, a zero pivot
//    replaced by a divisor of 1.  "Fixed barrier sequence": the sequence of
//    exchanges never depends on the data.
//  * "ruSOLVER：小矩阵 kernel 优化（实验性）", section on the unchanged
//    numerical and failure contract: partial row pivoting, ties to the
//    lowest row number, exact quotients, status 0 / first failed pivot,
//    failed systems zeroed with pivots -1, read-only inputs.
//
// Arithmetic: every element receives exactly the fused multiply-adds of the
// unblocked right-looking algorithm, in the same order (step by step), so
// results do not depend on the blocking below.
//
// gfx950 design.  Moving a row out of one lane costs one LDS write
// instruction per 16 bytes whatever the number of active lanes, while a DPP
// broadcast from a fixed lane of a 16-lane row rides for free on the fused
// multiply-add (v_fmac_*_dpp row_newbcast / quad_perm).  The factorization
// therefore goes by panels of B columns:
//   * inside a panel, step k searches column k: the largest flagged high word
//     of |a| (flag = row still at a position >= k) by a DPP max over the
//     group, a ballot of the slots that hold it, and, when every group of the
//     wave has exactly one such slot (decided uniformly), that slot wins;
//     otherwise the low word and then the lowest position decide exactly.
//     The winning lane hands its key, value and panel entries right of k to
//     the group in one batch of lane fetches; the rows relabel, form their
//     multipliers by IEEE division, and the rest of the panel takes the
//     update at once, so column k+1 is complete when its search starts;
//   * at the end of the panel, each of its B pivot rows is written once to an
//     LDS record (trailing columns and right-hand sides); every lane reads
//     back the entries it serves as DPP source (trailing column t from lane
//     t mod 16), and every row of the group takes the panel's B rank-1
//     updates on its trailing columns in step order, the pivot-row entry
//     broadcast by DPP inside the FMA.
// Back substitution (upper_solve_store, shared with the Cholesky kernel):
// the rows go by position to a packed triangular LDS store, then x_k is
// formed by the owner of position k and removed from the rows above.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tdls_internal.h"

namespace tdls {

// Fused multiply-add and magnitude in the working precision.  The plain
// __builtin_fma / __builtin_fabs take and return double: on float operands
// they would compute in double and round back, and a double fma rounded to
// float is not always the float fma (the exact sum can round twice to the
// other side of a float midpoint).  Every kernel uses these instead.
__device__ __forceinline__ float fma_r(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_r(double a, double b, double c) { return __builtin_fma(a, b, c); }
__device__ __forceinline__ float fabs_r(float v) { return __builtin_fabsf(v); }
__device__ __forceinline__ double fabs_r(double v) { return __builtin_fabs(v); }

// float64 division with the divisor's reciprocal formed ahead of time.
// The IEEE quotient n / d is what the compiler's division sequence computes:
// scale d and n (v_div_scale), a reciprocal of the scaled d refined by two
// Newton-Raphson steps, q = n r, the residual e = fma(-d, q, n), q' =
// fma(e, r, q) (v_div_fmas), then the special cases (v_div_fixup).  When
// neither operand is scaled (the scale steps return them unchanged, no
// scaling flag) and the fix-up leaves q' unchanged, the quotient is q'
// computed from the same reciprocal: recip_div64 forms that reciprocal from
// d alone, quot_div64 the quotient in three dependent operations, and
// quot_div64_exact tells afterwards whether the shortcut was the sequence's
// own result (else the caller divides).
__device__ __forceinline__ double recip_div64(double d) {
  double r = __builtin_amdgcn_rcp(d);
  double e = __builtin_fma(-d, r, 1.0);
  r = __builtin_fma(r, e, r);
  e = __builtin_fma(-d, r, 1.0);
  return __builtin_fma(r, e, r);
}
__device__ __forceinline__ double quot_div64(double n, double d, double r) {
  const double q = n * r;
  return __builtin_fma(__builtin_fma(-d, q, n), r, q);
}
__device__ __forceinline__ bool quot_div64_exact(double n, double d, double x) {
  bool fd, fn;
  const double ds = __builtin_amdgcn_div_scale(n, d, false, &fd);
  const double ns = __builtin_amdgcn_div_scale(n, d, true, &fn);
  const double fx = __builtin_amdgcn_div_fixup(x, d, n);
  return (__builtin_bit_cast(uint64_t, ds) == __builtin_bit_cast(uint64_t, d)) &
         (__builtin_bit_cast(uint64_t, ns) == __builtin_bit_cast(uint64_t, n)) & !fn &
         (__builtin_bit_cast(uint64_t, fx) == __builtin_bit_cast(uint64_t, x));
}

template <int B, int E, typename F>
__device__ __forceinline__ void sfor(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    sfor<B + 1, E>(f);
  }
}

template <typename Real>
struct RealTraits;
template <>
struct RealTraits<float> {
  typedef float vec16 __attribute__((ext_vector_type(4)));
  static constexpr int VEC = 4;
};
template <>
struct RealTraits<double> {
  typedef double vec16 __attribute__((ext_vector_type(2)));
  static constexpr int VEC = 2;
};

template <typename Real, int N, int NRHS, int T, int B>
struct PanelShape {
  static_assert(T == 4 || T == 16 || T == 32 || T == 64, "group size must be 4, 16, 32 or 64");
  static constexpr int R = (N + T - 1) / T;        // rows (slots) per lane
  static constexpr int G = kWaveSize / T;          // systems per wave
  static constexpr int SL = T < 16 ? T : 16;       // lanes per DPP broadcast domain
  static constexpr int VEC = RealTraits<Real>::VEC;
  static constexpr int REC = N + NRHS;             // largest record: panel 0
  static constexpr int REC_STRIDE = (REC + VEC - 1) / VEC * VEC;
  // U stays in registers for the back substitution (else: the right-hand
  // sides by position, then over them the packed upper triangle of U, row q
  // holding columns q..N-1); the group's LDS area, lu_group_elems
  static constexpr bool REG_SOLVE = lu_solve_in_registers(NRHS, T);
  static_assert(B <= kPanelMax && B <= N, "records sized for the widest panel");
  static constexpr int GROUP_ELEMS = lu_group_elems(N, NRHS, T, sizeof(Real) == 8);
  static constexpr int WAVE_BYTES = G * GROUP_ELEMS * (int)sizeof(Real);
  static constexpr int BLOCK_BYTES = kWavesPerBlock * WAVE_BYTES;
};

// Row stride (elements) of rows staged through LDS, at most `cap`, a
// multiple of the 16-byte vector: where possible one whose dword count is
// 4 mod 8, so that eight lanes writing or reading 16 bytes each at the same
// offset of eight consecutive rows start on eight different 4-bank groups
// (no bank conflict); else the largest multiple of the vector that fits.
constexpr int stage_stride(int cap, int es) {
  const int vec = 16 / es;
  for (int r = cap / vec * vec; r >= vec; r -= vec)
    if ((r * es / 4) % 8 == 4) return r;
  return cap / vec * vec;
}

// ---------------------------------------------------------------- lanes

// Reduction over the T lanes of a group (groups are aligned, T | 64).
template <int T, bool MAX>
__device__ __forceinline__ uint32_t group_reduce(uint32_t v) {
  auto op = [](uint32_t a, uint32_t b) { return MAX ? (a > b ? a : b) : (a < b ? a : b); };
  {
    if constexpr (T == 4) {
      v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, true));  // xor 1
      v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, true));  // xor 2
    } else {
      v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, true));  // ror 8
      v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, true));  // ror 4
      v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, true));  // ror 2
      v = op(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, true));  // ror 1
      if constexpr (T == 32) {
        // combine the two 16-lane rows of each group: after the swap the
        // first value holds row 2i in both rows of the pair, the second row 2i+1
        const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = op((uint32_t)sw[0], (uint32_t)sw[1]);
      }
      if constexpr (T == 64) {
        // every 16-lane row holds its own result: combine the four rows
        uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
        uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
        uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
        uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
        v = op(op(r0, r1), op(r2, r3));
      }
    }
  }
  return v;
}

// Bitwise OR over the T lanes of a group (T < 64: DPP only, nothing goes
// through the LDS crossbar).  With exactly one lane of each group holding a
// non-zero value this hands that value to the whole group.
template <int T>
__device__ __forceinline__ uint32_t group_or(uint32_t v) {
  static_assert(T < 64, "whole-wave groups use readlane");
  if constexpr (T == 4) {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xf, 0xf, true);  // xor 1
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xf, 0xf, true);  // xor 2
  } else {
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xf, 0xf, true);  // ror 8
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x124, 0xf, 0xf, true);  // ror 4
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x122, 0xf, 0xf, true);  // ror 2
    v |= (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x121, 0xf, 0xf, true);  // ror 1
    if constexpr (T == 32) {
      const auto sw = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      v = (uint32_t)sw[0] | (uint32_t)sw[1];
    }
  }
  return v;
}

// Value of `x` held by lane `src` (absolute lane index, may differ per lane).
__device__ __forceinline__ double lane_fetch_any(double x, int src) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ float lane_fetch_any(float x, int src) {
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
}

// 32-bit value of `x` held by lane KP of this lane's class, a class being
// CL consecutive lanes (CL = 2, 4, 8 or 16, aligned to CL): a quad permute
// for classes inside a quad, a broadcast from a fixed lane of each 16-lane
// row otherwise (half rows take two, one per pair of 4-lane banks).  The
// source may have been written by the instruction just before (two wait
// states before the DPP read).
template <int CL, int KP>
__device__ __forceinline__ uint32_t class_bcast_u32(uint32_t x) {
  static_assert(CL == 2 || CL == 4 || CL == 8 || CL == 16, "class of 2, 4, 8 or 16 lanes");
  static_assert(KP >= 0 && KP < CL, "source lane inside the class");
  uint32_t out;
  if constexpr (CL <= 4) {
    constexpr int q0 = KP, q1 = CL == 4 ? KP : 2 + KP;
    constexpr int qp = q0 | (q0 << 2) | (q1 << 4) | (q1 << 6);
    out = (uint32_t)__builtin_amdgcn_mov_dpp((int)x, qp, 0xf, 0xf, false);
  } else if constexpr (CL == 8) {
    asm volatile(
        "s_nop 1\n\tv_mov_b32_dpp %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0x3\n\t"
        "v_mov_b32_dpp %0, %1 row_newbcast:%3 row_mask:0xf bank_mask:0xc"
        : "=&v"(out)
        : "v"(x), "i"(KP), "i"(8 + KP));
  } else {
    asm volatile("s_nop 1\n\tv_mov_b32_dpp %0, %1 row_newbcast:%2 row_mask:0xf bank_mask:0xf"
                 : "=v"(out)
                 : "v"(x), "i"(KP));
  }
  return out;
}
template <int CL, int KP>
__device__ __forceinline__ double class_bcast(double x) {
  const uint64_t b = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = class_bcast_u32<CL, KP>((uint32_t)b);
  const uint32_t hi = class_bcast_u32<CL, KP>((uint32_t)(b >> 32));
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <int CL, int KP>
__device__ __forceinline__ float class_bcast(float x) {
  return __builtin_bit_cast(float, class_bcast_u32<CL, KP>(__builtin_bit_cast(uint32_t, x)));
}

// 32-bit value of `x` held by lane `src` (absolute lane index) of this wave;
// `src` is wave-uniform when T = 64.
template <int T>
__device__ __forceinline__ uint32_t lane_fetch_u32(uint32_t x, int src) {
  if constexpr (T == 64)
    return (uint32_t)__builtin_amdgcn_readlane((int)x, __builtin_amdgcn_readfirstlane(src));
  else
    return (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)x);
}

// Value of `x` held by lane `src` (absolute lane index) of this wave.
template <int T>
__device__ __forceinline__ double lane_fetch(double x, int src) {
  if constexpr (T == 64) {
    const int s = __builtin_amdgcn_readfirstlane(src);
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, s);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), s);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
  } else {
    const uint64_t b = __builtin_bit_cast(uint64_t, x);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)b);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_ds_bpermute(src << 2, (int)(uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
  }
}
template <int T>
__device__ __forceinline__ float lane_fetch(float x, int src) {
  if constexpr (T == 64) {
    const int s = __builtin_amdgcn_readfirstlane(src);
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), s));
  } else {
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_ds_bpermute(src << 2, __builtin_bit_cast(int, x)));
  }
}

// acc -= (u taken from lane L of its DPP domain) * m, one fused multiply-add
// (the DPP source carries the negation: -u * m + acc rounds as fma(-m, u, acc)).
// A DPP source written by a VALU instruction needs two wait states before
// the DPP read; NOP adds them, and the caller sets it on the first read of
// each source register after it was computed (the asm statements are volatile,
// so they stay in program order).
template <int T, int L, bool NOP>
__device__ __forceinline__ void fnmac_bcast(double& acc, double u, double m) {
  if constexpr (T >= 16) {
    if constexpr (NOP)
      asm volatile("s_nop 1\n\tv_fmac_f64_dpp %0, -%1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                   : "+v"(acc)
                   : "v"(u), "v"(m), "i"(L));
    else
      asm volatile("v_fmac_f64_dpp %0, -%1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                   : "+v"(acc)
                   : "v"(u), "v"(m), "i"(L));
  } else {
    // 64-bit DPP allows only row_newbcast: move the two halves across the quad
    const uint64_t b = __builtin_bit_cast(uint64_t, u);
    constexpr int qp = L | (L << 2) | (L << 4) | (L << 6);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, qp, 0xf, 0xf, true);
    const uint32_t hi =
        (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), qp, 0xf, 0xf, true);
    acc = fma_r(-m, __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo), acc);
  }
}
template <int T, int L, bool NOP>
__device__ __forceinline__ void fnmac_bcast(float& acc, float u, float m) {
  if constexpr (T >= 16) {
    if constexpr (NOP)
      asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, -%1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                   : "+v"(acc)
                   : "v"(u), "v"(m), "i"(L));
    else
      asm volatile("v_fmac_f32_dpp %0, -%1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
                   : "+v"(acc)
                   : "v"(u), "v"(m), "i"(L));
  } else {
    if constexpr (NOP)
      asm volatile("s_nop 1\n\tv_fmac_f32_dpp %0, -%1, %2 quad_perm:[%3,%3,%3,%3] row_mask:0xf "
                   "bank_mask:0xf"
                   : "+v"(acc)
                   : "v"(u), "v"(m), "i"(L));
    else
      asm volatile("v_fmac_f32_dpp %0, -%1, %2 quad_perm:[%3,%3,%3,%3] row_mask:0xf bank_mask:0xf"
                   : "+v"(acc)
                   : "v"(u), "v"(m), "i"(L));
  }
}

__device__ __forceinline__ void wave_sync_lds() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

// True on every lane of the group (T lanes from gbase; the whole wave when
// T = 64) when `v` holds on any of them.  Called by the whole wave.
template <int T>
__device__ __forceinline__ bool group_any(bool v, int gbase) {
  const uint64_t b = __builtin_amdgcn_ballot_w64(v);
  if constexpr (T == 64) {
    return b != 0;
  } else {
    constexpr uint64_t GM = T == 32 ? 0xffffffffull : ((1ull << T) - 1ull);
    return ((b >> gbase) & GM) != 0;
  }
}

// NaN or an infinity (the status codes -1 and -3 of the ruSOLVER contract)
__device__ __forceinline__ bool not_finite(double v) { return !__builtin_isfinite(v); }
__device__ __forceinline__ bool not_finite(float v) { return !__builtin_isfinite(v); }

// Block of systems a workgroup takes.  Workgroups go to the 8 XCDs of the
// chip in turn (workgroup b on XCD b mod 8), each XCD with its own L2.  One
// after another (interleave 1) a block's systems fill whole cache lines by
// themselves, and blocks follow the workgroup order.  Interleaved, a cache
// line holds the same element of neighbouring blocks, so the blocks are
// renumbered to give each XCD a contiguous range: its L2 then serves the
// neighbours from one fetch instead of each XCD fetching the line.
__device__ __forceinline__ int64_t block_of(int64_t ilv) {
  const int64_t b = blockIdx.x;
  if (ilv == 1) return b;
  constexpr int64_t kXcds = 8;
  const int64_t nb = gridDim.x;
  const int64_t q = nb / kXcds, r = nb % kXcds;
  const int64_t x = b % kXcds, i = b / kXcds;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + i;
}

// Start of system s in a batch of systems of E elements each, stored with W
// systems interleaved element by element (the single strided form of the
// TDLS page, section Residency: W = 1 one system after another, W = batch
// a structure of arrays, other W blocks of W systems): element e of system
// s lives at sys_start(s) + e * W.
__device__ __forceinline__ int64_t sys_start(int64_t s, int64_t W, int64_t E) {
  return W == 1 ? s * E : (s / W) * W * E + s % W;
}

__device__ __forceinline__ uint32_t hi_word(double v) {
  return (uint32_t)(__builtin_bit_cast(uint64_t, v) >> 32);
}
__device__ __forceinline__ uint32_t lo_word(double v) {
  return (uint32_t)__builtin_bit_cast(uint64_t, v);
}

// ------------------------------------------------------------- kernel

// ---- back substitution shared by the LU and Cholesky kernels
//
// Row q of the packed upper-triangular store (columns q..N-1) starts at
// utri_row(q).
template <int N>
__device__ __forceinline__ int utri_row(int q) { return q * N - q * (q - 1) / 2; }

// U x = y for the group's system, then X stored (all +0.0 when `failed` or,
// with ZERO_NONFINITE, when an entry of x is not finite).  Returns true on
// the group's lanes when an entry of x (positions below n) is not finite.
// `ut` is the group's LDS area (at least max(N * NRHS, N (N + 1) / 2)
// entries).  write_rhs(ut) must store the right-hand sides by position
// (entry (q, j) at ut[q * NRHS + j]); write_u(ut) must then store row q of U
// at ut + utri_row(q) - q + c for columns c >= q, over them.
//
// x_k = y_k / U(k,k) by IEEE division for k = n-1 .. 0, each x_k removed from
// the rows above by fused multiply-adds (the order of the TDLS page's
// Detailed Description, the solution entry kept by its owner).  One
// right-hand side: lane tx holds the positions tx + K*T, x_k is formed on
// lane k % T and reaches the rows above by DPP inside the FMA (a lane fetch
// for groups wider than a 16-lane row).  Several: the group's lanes split
// into NJ column classes and P row phases; lane j0 * P + ph holds the columns
// j = j0 + NJ*jj of the positions ph + P*m, so x_k costs one division per
// column class on the lanes of phase k % P, handed to the lanes of the same
// class by DPP (classes are P consecutive lanes); U(q, k) is read from the
// store.
template <typename Real, int N, int NRHS, int T, bool ZERO_NONFINITE = true, typename WR,
          typename WU>
__device__ __forceinline__ bool upper_solve_store(Real* ut, int tx, int gbase, bool live,
                                                  bool failed, int64_t sys, int n, int nrhs,
                                                  int col, int64_t ilv, Real* X, WR&& write_rhs,
                                                  WU&& write_u) {
  constexpr int R = (N + T - 1) / T;
  bool xbad = false;
  write_rhs(ut);
  wave_sync_lds();
  Real* Xs = X + sys_start(sys, ilv, (int64_t)n * nrhs);
  // layout of the solve (see below): one right-hand side by slots; several
  // by column classes and row phases
  constexpr int NJ = NRHS < T ? NRHS : T;
  constexpr int P = NRHS == 1 ? T : T / NJ;
  constexpr int JR = NRHS / NJ;
  constexpr int QR = (N + P - 1) / P;
  const int j0 = NRHS == 1 ? 0 : tx / P;   // column class: P consecutive lanes
  const int ph = NRHS == 1 ? tx : tx % P;
  Real yv[QR][JR];
  sfor<0, QR>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    const int q = ph + P * m;
    const int qq = q < N ? q : N - 1;
    sfor<0, JR>([&](auto jc) {
      constexpr int jj = decltype(jc)::value;
      yv[m][jj] = ut[qq * NRHS + j0 + NJ * jj];
    });
  });
  wave_sync_lds();  // read before U overwrites them
  write_u(ut);
  wave_sync_lds();
  const Real* rw[QR];
  sfor<0, QR>([&](auto mc) {
    constexpr int m = decltype(mc)::value;
    const int q = ph + P * m;
    const int qq = q < N ? q : N - 1;
    rw[m] = ut + utri_row<N>(qq) - qq;   // entry of column c at rw[m][c]
  });

  if constexpr (NRHS == 1) {
    // One right-hand side: lane tx holds the positions tx + K*T; x_k is
    // formed by lane k % T (slot k / T) and reaches the rows above by DPP
    // inside the FMA (a lane fetch for groups wider than a 16-lane row).
    // x of the positions tx + K*T, kept by this lane until the final store
    // (every entry is assigned at its own step)
    Real xr[R];
    sfor<0, R>([&](auto Kc) { xr[decltype(Kc)::value] = Real(0); });
    // u(q, k) of this lane's rows, read one step ahead (two buffers) so that
    // a step's LDS reads overlap the step before; each step's instructions
    // stay together (hoisting every read ahead of the loop costs registers)
    Real ub[2][R];
    auto read_u = [&](auto icc) {
      constexpr int k2 = N - 1 - decltype(icc)::value;
      sfor<0, k2 / T + 1>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        ub[decltype(icc)::value % 2][K] = rw[K][k2];
      });
    };
    read_u(std::integral_constant<int, 0>{});
    sfor<0, N>([&](auto ic) {
      constexpr int k = N - 1 - decltype(ic)::value;
      constexpr int kl = k % T;
      constexpr int ks = k / T;
      constexpr int SLK = kl % (T < 16 ? T : 16);   // lane of k inside its DPP domain
      constexpr int cur = decltype(ic)::value % 2;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(ic)::value + 1 < N)
        read_u(std::integral_constant<int, decltype(ic)::value + 1>{});
      Real(&uk)[R] = ub[cur];
      const Real x = yv[ks][0] / uk[ks];   // meaningful on lane kl
      xr[ks] = tx == kl ? x : xr[ks];
      asm volatile("" : "+v"(xr[ks]));   // select now, not at the store
      // rows above k take x_k (rows at k and below are done: their updates
      // are never read)
      if constexpr (T <= 16) {
        sfor<0, ks + 1>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          fnmac_bcast<T, SLK, K == 0>(yv[K][0], x, uk[K]);
        });
      } else {
        const Real xk = lane_fetch<T>(x, gbase + kl);
        sfor<0, ks + 1>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          yv[K][0] = fma_r(-uk[K], xk, yv[K][0]);
        });
      }
    });
    bool bad = false;
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      bad |= (tx + K * T < n) & not_finite(xr[K]);
    });
    xbad = group_any<T>(bad, gbase);
    if (live) {
      const bool zero = failed || (ZERO_NONFINITE && xbad);
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        if (q < n) Xs[q * ilv] = zero ? Real(0) : xr[K];   // one column: same address in both layouts
      });
    }
  } else {
    // Several right-hand sides: the group's lanes split into NJ column
    // classes of P consecutive lanes (lane j0 * P + ph is phase ph of class
    // j0).  It holds the right-hand-side columns j = j0 + NJ*jj of the
    // positions q = ph + P*m, so each x_k is one division per column on the
    // NJ lanes of phase k % P, handed to the other lanes of its class by a
    // DPP broadcast (a lane fetch for classes wider than a 16-lane row);
    // every lane then folds it into its rows, reading u(q, k) from the
    // triangular store.
    Real xr[QR][JR];
    sfor<0, QR>([&](auto mc) {
      sfor<0, JR>([&](auto jc) { xr[decltype(mc)::value][decltype(jc)::value] = Real(0); });
    });
    // u(q, k) of this lane's rows, read one step ahead as above
    Real ub[2][QR];
    auto read_u = [&](auto icc) {
      constexpr int k2 = N - 1 - decltype(icc)::value;
      sfor<0, k2 / P + 1>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        ub[decltype(icc)::value % 2][m] = rw[m][k2];   // u(q, k2), q = ph + P*m
      });
    };
    read_u(std::integral_constant<int, 0>{});
    sfor<0, N>([&](auto ic) {
      constexpr int k = N - 1 - decltype(ic)::value;
      constexpr int kp = k % P;
      constexpr int km = k / P;
      constexpr int cur = decltype(ic)::value % 2;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (decltype(ic)::value + 1 < N)
        read_u(std::integral_constant<int, decltype(ic)::value + 1>{});
      Real(&uk)[QR] = ub[cur];   // meaningful for q <= k
      sfor<0, JR>([&](auto jc) {
        constexpr int jj = decltype(jc)::value;
        const Real x = yv[km][jj] / uk[km];   // meaningful on the lanes of phase kp
        xr[km][jj] = ph == kp ? x : xr[km][jj];
        asm volatile("" : "+v"(xr[km][jj]));
        Real xk;
        if constexpr (P == 1)
          xk = x;   // every lane is the owner of its own column class
        else if constexpr (P <= 16)
          xk = class_bcast<P, kp>(x);   // lane kp of the class, by DPP
        else
          xk = lane_fetch_any(x, gbase + j0 * P + kp);
        sfor<0, km + 1>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          yv[m][jj] = fma_r(-uk[m], xk, yv[m][jj]);
        });
      });
    });
    bool bad = false;
    sfor<0, QR>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      sfor<0, JR>([&](auto jc) {
        constexpr int jj = decltype(jc)::value;
        bad |= (ph + P * m < n) & (j0 + NJ * jj < nrhs) & not_finite(xr[m][jj]);
      });
    });
    xbad = group_any<T>(bad, gbase);
    if (live) {
      const bool zero = failed || (ZERO_NONFINITE && xbad);
      sfor<0, QR>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        const int q = ph + P * m;
        sfor<0, JR>([&](auto jc) {
          constexpr int jj = decltype(jc)::value;
          const int j = j0 + NJ * jj;
          if (q < n && j < nrhs) {
            const Real v = zero ? Real(0) : xr[m][jj];
            if (col)
              Xs[((int64_t)j * n + q) * ilv] = v;
            else
              Xs[((int64_t)q * nrhs + j) * ilv] = v;
          }
        });
      });
    }
  }
  return xbad;
}

// FACT = false: gesv, X receives the solutions.  FACT = true: getrf (NRHS
// must be 1 and Bm is not read), X receives the factors in the layout of A:
// LAPACK's row order, unit-lower L below the diagonal and U on and above it.
template <typename Real, int N, int NRHS, int T, int B, bool FACT = false>
__global__ void __launch_bounds__(kWaveSize* kWavesPerBlock,
                                  lu_min_waves(N, NRHS, sizeof(Real) == 8, T, FACT) > 0
                                      ? lu_min_waves(N, NRHS, sizeof(Real) == 8, T, FACT)
                                      : 1)
    gesv_panel_kernel(int col, int n, int nrhs, int64_t batch, const Real* __restrict__ A,
                      const Real* __restrict__ Bm, Real* __restrict__ X, int32_t* __restrict__ piv,
                      int32_t* __restrict__ info, uint32_t flags, int64_t ilv) {
  static_assert(B == panel_width(N, NRHS, sizeof(Real) == 8, T, FACT), "panel width");
  static_assert(!FACT || NRHS == 1, "the factorization runs with one (unused) right-hand side");
  static_assert(N > B, "the first panel has trailing columns (input check)");
  using S = PanelShape<Real, N, NRHS, T, B>;
  constexpr int R = S::R;
  constexpr int G = S::G;
  constexpr int SL = S::SL;
  constexpr int VEC = S::VEC;
  constexpr bool is64 = sizeof(Real) == 8;
  extern __shared__ __align__(16) unsigned char lds_raw[];

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = threadIdx.x / kWaveSize;
  const int g = lane / T;
  const int tx = lane & (T - 1);
  const int gbase = g * T;  // first lane of the group
  const int64_t wave_first = (block_of(ilv) * kWavesPerBlock + wave) * G;
  if (wave_first >= batch) return;  // the whole wave is past the batch
  const int64_t sys = wave_first + g;
  const bool live = sys < batch;

  unsigned char* wave_lds = lds_raw + wave * S::WAVE_BYTES;
  Real* rec = reinterpret_cast<Real*>(wave_lds) + g * S::GROUP_ELEMS;

  Real a[R][N];
  Real y[R][NRHS];
  int lab[R];   // current position of the row in slot K (LAPACK order), -1 for phantom
  int pv[R];    // pivot output for the fixed position tx + K*T

  // ---- load: slot K of lane tx holds original row q = tx + K*T.  Rows and
  // columns n..N-1 form an identity block, right-hand sides nrhs..NRHS-1 are
  // zero.  Phantom rows (q >= N) and the groups past the batch load row 0 of
  // a valid system: they never take part (never a candidate, never a pivot,
  // never stored), so their contents do not matter.  When the problem has the
  // kernel's shape every address is a per-slot base plus a compile-time
  // offset and every load lands directly in its row register.
  {
    const Real* As = A + sys_start(live ? sys : 0, ilv, (int64_t)n * n);
    const Real* Bs = Bm + sys_start(live ? sys : 0, ilv, (int64_t)n * nrhs);
    if (n == N && nrhs == NRHS && ilv == 1) {
      // Loads are issued column by column over the slots, so the first
      // pivot search waits only for the first column to arrive while the
      // rest of the tile streams in behind it.
      auto load_exact = [&](auto colc) {
        constexpr bool COL = decltype(colc)::value;
        const Real* ar[R];
        const Real* br[R];
        sfor<0, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          const int q = tx + K * T;
          const int qq = q < N ? q : 0;
          ar[K] = As + (COL ? qq : qq * N);
          br[K] = Bs + (COL ? qq : qq * NRHS);
        });
        sfor<0, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          sfor<0, R>([&](auto Kc) {
            constexpr int K = decltype(Kc)::value;
            a[K][c] = ar[K][COL ? c * N : c];
          });
        });
        sfor<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          sfor<0, R>([&](auto Kc) {
            constexpr int K = decltype(Kc)::value;
            if constexpr (FACT)
              y[K][j] = Real(0);
            else
              y[K][j] = br[K][COL ? j * N : j];
          });
        });
      };
      if (col)
        load_exact(std::true_type{});
      else
        load_exact(std::false_type{});
    } else {
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        const bool qrow = live && q < n;
        const int qq = qrow ? q : 0;
        const int64_t cs = (col ? n : 1) * ilv;  // element stride between columns
        const Real* ar = As + (col ? qq : (int64_t)qq * n) * ilv;
        const int64_t js = (col ? n : 1) * ilv;
        const Real* br = Bs + (col ? qq : (int64_t)qq * nrhs) * ilv;
        // identity block, then the stored entries; the scheduling barriers
        // keep few loads (and their 64-bit addresses) in flight at a time
        sfor<0, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          a[K][c] = (q == c) ? Real(1) : Real(0);
        });
        sfor<0, NRHS>([&](auto jc) { y[K][decltype(jc)::value] = Real(0); });
        sfor<0, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if (qrow && c < n) a[K][c] = ar[c * cs];
          if constexpr (c % 8 == 7) __builtin_amdgcn_sched_barrier(0);
        });
        sfor<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          if constexpr (!FACT)
            if (qrow && j < nrhs) y[K][j] = br[j * js];
        });
        __builtin_amdgcn_sched_barrier(0);
      });
    }
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      lab[K] = q < N ? q : -1;
      pv[K] = q;
    });
  }

  // ---- whole-matrix max-abs scaling (an option; ruSOLVER page, section on
  // the unchanged numerical and failure contract): the system is divided by
  // the largest magnitude sc of its matrix, entry by entry (IEEE division),
  // which leaves the solution unchanged; the factorization multiplies U back
  // by sc at the end.  A zero (or non-finite) maximum leaves it as it is.
  Real sc = Real(1);
  if (flags & kFlagScaleMaxAbs) {
    uint32_t mh = 0, ml = 0;   // lane maximum of |a|, as the bits of a non-negative value
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      sfor<0, N>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        const Real v = (q < n && c < n) ? fabs_r(a[K][c]) : Real(0);
        if constexpr (is64) {
          const uint32_t h = hi_word(v), l = lo_word(v);
          const bool gt = h > mh || (h == mh && l > ml);
          mh = gt ? h : mh;
          ml = gt ? l : ml;
        } else {
          const uint32_t h = __builtin_bit_cast(uint32_t, v);
          mh = h > mh ? h : mh;
        }
      });
    });
    const uint32_t gh = group_reduce<T, true>(mh);
    Real s;
    if constexpr (is64) {
      const uint32_t gl = group_reduce<T, true>(mh == gh ? ml : 0u);
      s = __builtin_bit_cast(double, ((uint64_t)gh << 32) | gl);
    } else {
      s = __builtin_bit_cast(float, gh);
    }
    sc = (s > Real(0) && !not_finite(s)) ? s : Real(1);
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      sfor<0, N>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        a[K][c] = (q < n && c < n) ? a[K][c] / sc : a[K][c];
      });
      sfor<0, NRHS>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        y[K][j] = (q < n && j < nrhs) ? y[K][j] / sc : y[K][j];
      });
    });
  }

  // Status, in the ruSOLVER contract's order of precedence: -1 for a
  // non-finite input entry (checked column by column as the first panel
  // reaches them), the first exactly zero pivot (k + 1), then -3 when a
  // computed value is not finite: a pivot (nf), an entry of x, or an entry
  // of the factors.  A non-finite value never turns finite again in the
  // updates that follow, so a non-finite multiplier or U entry shows in x.
  int status = 0;
  int inbad = 0;   // a lane flag, settled where it is formed (asm barrier
                   // below): left to its use it keeps values alive
  // Non-finite pivots: every pivot enters pz as a fused multiply-add by
  // zero, which leaves pz +0.0 unless a pivot is an infinity or a NaN (then
  // pz is NaN for good); one instruction a step instead of a compare and a
  // flag update.
  Real pz = Real(0);
  // Key of slot K for the exact pivot comparison: position << 13 | lane << 5
  // | slot << 1.  Positions are unique, so comparing keys compares
  // positions; keys are formed only when a group has a tie on the high word.
  auto key = [&](auto Kc) -> uint32_t {
    constexpr int K = decltype(Kc)::value;
    return ((uint32_t)(lab[K] < 0 ? 0 : lab[K]) << 13) | ((uint32_t)lane << 5) | (K << 1);
  };

  // ---- factorization, panel by panel
  //
  // Slot compaction.  Rows never move during the steps, so a lane's slots
  // hold rows of any position and every slot takes part in every step.  At
  // each slot boundary k0 = m*T (m >= 1, a panel boundary when B divides T)
  // the rows of slots m-1 .. R-1 go through LDS and come back in position
  // order: slot K then holds the positions K*T .. K*T+T-1, so slots below m
  // hold only finished rows (positions < k0) and the steps and trailing
  // updates from k0 on skip them at compile time.  Arithmetic is unchanged:
  // a finished row takes only zero multipliers.
  constexpr bool COMPACT = R > 1 && T % B == 0;
  constexpr int NP = (N + B - 1) / B;
  sfor<0, NP>([&](auto pc) {
    constexpr int k0 = decltype(pc)::value * B;
    constexpr int bw = (N - k0) < B ? (N - k0) : B;   // panel width
    constexpr int NT = N - k0 - bw;                    // trailing matrix columns
    constexpr int W = NT + NRHS;                       // trailing entries per row
    constexpr int K0 = COMPACT ? k0 / T : 0;           // slots of finished rows only
    Real lm[B][R];                                     // multiplier, 0 unless below
    if constexpr (COMPACT && k0 > 0 && k0 % T == 0) {
      constexpr int KP = K0 - 1;                 // slots already in position order
      constexpr int NS = N - KP * T;             // rows staged (positions KP*T .. N-1)
      constexpr int E = N + (FACT ? 0 : NRHS);   // entries per row: columns, right-hand sides
      // entries below EB are needed by no staged row: the solve keeps only U
      // (columns from the row's position on), the factorization all of L\U
      constexpr int EB = FACT ? 0 : KP * T;
      // row stride in LDS: a multiple of the vector width, not of 32 banks
      constexpr int RS = stage_stride(S::GROUP_ELEMS / NS, (int)sizeof(Real));
      static_assert(RS >= VEC && NS * RS <= S::GROUP_ELEMS, "staging fits the group area");
      constexpr int NCH = (E - EB + RS - 1) / RS;
      auto ent = [&](auto Kc, auto ec) -> Real& {
        constexpr int K = decltype(Kc)::value;
        constexpr int e = decltype(ec)::value;
        if constexpr (e < N) return a[K][e];
        else return y[K][e - N];
      };
      sfor<0, NCH>([&](auto hc) {
        constexpr int e0 = EB + decltype(hc)::value * RS;
        constexpr int e1 = (e0 + RS) < E ? (e0 + RS) : E;
        sfor<KP, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          const int p = lab[K];
          if (p >= 0) {
            Real* dst = rec + (p - KP * T) * RS - e0;   // entry e at dst[e]
            sfor<e0, e1>([&](auto ec) { dst[decltype(ec)::value] = ent(Kc, ec); });
          }
        });
        wave_sync_lds();
        sfor<KP, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          // first entry slot K needs: a finished slot its U part, an active
          // one its trailing columns (the factorization: the whole row)
          constexpr int es = FACT ? 0 : (K < K0 ? K * T : k0);
          constexpr int b0 = e0 > es ? e0 : es;
          if (K * T + T <= N || tx + K * T < N) {
            const Real* src = rec + (tx + K * T - KP * T) * RS - e0;
            sfor<b0, e1>([&](auto ec) { ent(Kc, ec) = src[decltype(ec)::value]; });
          }
        });
        wave_sync_lds();
      });
      sfor<KP, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        lab[K] = q < N ? q : -1;
      });
    }
    if constexpr (k0 == 0) {
      // input check of the panel's own columns (the others below)
      sfor<0, R>([&](auto Kc) {
        sfor<0, bw>([&](auto cc) { inbad |= not_finite(a[decltype(Kc)::value][decltype(cc)::value]); });
      });
      asm volatile("" : "+v"(inbad));
    }

    sfor<0, bw>([&](auto ic) {
      constexpr int i = decltype(ic)::value;
      constexpr int k = k0 + i;
      constexpr int kl = k % T;
      constexpr int ks = k / T;
      constexpr int PC = bw - 1 - i;   // panel columns right of k

      // (b) pivot search on column k over the rows at positions >= k.
      // Candidates compare as integers: the high word of |a| with bit 31 set
      // for a row at a position >= k (0 for the others), then the low word
      // (float64), then the position.  The group maximum of the flagged
      // high words comes from a DPP max over each lane's largest slot; the
      // slots that hold it are balloted.  When every group has exactly one
      // (the common case, decided uniformly) that slot wins and its lane is
      // the group's set ballot bit.  Otherwise each lane picks its best slot
      // exactly and the low word, then the lowest position, decide among
      // the lanes that hold the maximum.
      uint32_t hw[R], lw[R], hf[R];
      sfor<K0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        if constexpr (is64) {
          hw[K] = hi_word(a[K][k]);
          lw[K] = lo_word(a[K][k]);
        } else {
          hw[K] = __builtin_bit_cast(uint32_t, a[K][k]);
          lw[K] = 0u;
        }
        hf[K] = lab[K] >= k ? (hw[K] | 0x80000000u) : 0u;
      });
      uint32_t lmax = hf[K0];
      sfor<K0 + 1, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        lmax = lmax > hf[K] ? lmax : hf[K];
      });
      // every group has a candidate, so mh has bit 31 set and only flagged
      // slots can equal it
      const uint32_t mh = group_reduce<T, true>(lmax);
      bool tp[R];
      uint64_t tmask = 0;
      int ntop = 0;
      sfor<K0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        tp[K] = hf[K] == mh;
        const uint64_t b = __builtin_amdgcn_ballot_w64(tp[K]);
        tmask |= b;
        ntop += __builtin_popcountll(b);
      });
      // The lane's chosen slot (its top slot, or its best one when the
      // exact comparison runs): its position, value and entries right of k
      // in the panel are what the winning lane hands to its group.
      uint32_t ch = hw[K0], cl = lw[K0];
      int cp = lab[K0];
      Real cpan[PC > 0 ? PC : 1];
      sfor<0, PC>([&](auto cc) { cpan[decltype(cc)::value] = a[K0][k + 1 + decltype(cc)::value]; });
      auto choose = [&](auto Kc, bool take) {
        constexpr int K = decltype(Kc)::value;
        ch = take ? hw[K] : ch;
        cl = take ? lw[K] : cl;
        cp = take ? lab[K] : cp;
        sfor<0, PC>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          cpan[c] = take ? a[K][k + 1 + c] : cpan[c];
        });
      };
      int wl;       // winning lane
      bool iswin;   // this lane holds its group's pivot row
      if (__builtin_expect(ntop == G, 1)) {
        sfor<K0 + 1, R>([&](auto Kc) { choose(Kc, tp[decltype(Kc)::value]); });
        iswin = false;
        sfor<K0, R>([&](auto Kc) { iswin |= tp[decltype(Kc)::value]; });
        if constexpr (T == 64) {
          wl = __builtin_ctzll(tmask);
        } else {
          constexpr uint32_t GM = T == 32 ? 0xffffffffu : ((1u << T) - 1u);
          wl = gbase + __builtin_ctz((uint32_t)(tmask >> gbase) & GM);
        }
      } else {
        uint32_t bh = hf[K0], bl = lw[K0];
        uint32_t ck = key(std::integral_constant<int, K0>{});
        sfor<K0 + 1, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          const uint32_t kk = key(Kc);
          bool take;
          if constexpr (is64) {
            const uint64_t c = ((uint64_t)hf[K] << 32) | lw[K];
            const uint64_t bb = ((uint64_t)bh << 32) | bl;
            take = (c > bb) | ((c == bb) & (kk < ck));
          } else {
            take = (hf[K] > bh) | ((hf[K] == bh) & (kk < ck));
          }
          bh = take ? hf[K] : bh;
          bl = take ? lw[K] : bl;
          ck = take ? kk : ck;
          choose(Kc, take);
        });
        bool top = bh == mh;
        if constexpr (is64) {
          const uint32_t ml = group_reduce<T, true>(top ? bl : 0u);
          top = top & (bl == ml);
        }
        const uint32_t kmin = group_reduce<T, false>(top ? ck : 0xffffffffu);
        wl = (int)((kmin >> 5) & 63u);
        iswin = lane == wl;
      }
      // The winner's position and pivot value reach its group.  The group
      // maximum mh already holds the pivot's magnitude bits (of the high
      // word in float64); the winner adds its sign and position, and in
      // float64 its low word, by a DPP OR over the group of values only it
      // holds (nothing through the LDS crossbar); whole-wave groups read
      // them from the winning lane.
      int p;          // winner's position
      Real dpiv;      // the pivot
      if constexpr (T == 64) {
        p = (int)lane_fetch_u32<T>((uint32_t)cp, wl);
        if constexpr (is64)
          dpiv = __builtin_bit_cast(double, ((uint64_t)lane_fetch_u32<T>(ch, wl) << 32) |
                                                lane_fetch_u32<T>(cl, wl));
        else
          dpiv = __builtin_bit_cast(float, lane_fetch_u32<T>(ch, wl));
      } else {
        const uint32_t sp = group_or<T>(iswin ? ((ch & 0x80000000u) | (uint32_t)cp) : 0u);
        p = (int)(sp & 0x7fffffffu);
        const uint32_t dh = (mh & 0x7fffffffu) | (sp & 0x80000000u);
        if constexpr (is64)
          dpiv = __builtin_bit_cast(double, ((uint64_t)dh << 32) | group_or<T>(iswin ? cl : 0u));
        else
          dpiv = __builtin_bit_cast(float, dh);
      }
      // the winner's entries right of k inside the panel, the same way (the
      // LDS crossbar is the busier resource: measured, DPP ORs beat lane
      // fetches here even in 16-lane groups)
      Real upan[PC > 0 ? PC : 1];                          // pivot row, right of k
      sfor<0, PC>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        if constexpr (T == 64) {
          upan[c] = lane_fetch<T>(cpan[c], wl);
        } else if constexpr (is64) {
          const uint64_t b = __builtin_bit_cast(uint64_t, cpan[c]);
          const uint32_t h = group_or<T>(iswin ? (uint32_t)(b >> 32) : 0u);
          const uint32_t l = group_or<T>(iswin ? (uint32_t)b : 0u);
          upan[c] = __builtin_bit_cast(double, ((uint64_t)h << 32) | l);
        } else {
          upan[c] = __builtin_bit_cast(
              float, group_or<T>(iswin ? __builtin_bit_cast(uint32_t, cpan[c]) : 0u));
        }
      });
      const bool zero_pivot = dpiv == Real(0);
      pz = fma_r(dpiv, Real(0), pz);
      asm volatile("" : "+v"(pz));   // in place, not sunk to the end
      if (zero_pivot && status == 0) status = k + 1;
      // settle the status here: left to the end, the per-step zero flags of
      // every step stay live in scalar registers
      asm volatile("" : "+v"(status));
      const Real d = zero_pivot ? Real(1) : dpiv;

      // (c) logical interchange of positions k and p
      sfor<K0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int old = lab[K];
        const int nl = old == k ? p : (old == p ? k : old);
        lab[K] = nl;
      });
      if (tx == kl) pv[ks] = p;
      asm volatile("" : "+v"(pv[ks]));   // likewise for the pivot record

      // (d) multipliers of the rows now below position k (IEEE division);
      // column k itself keeps its values (the U entries of the rows above)
      sfor<K0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const Real l = a[K][k] / d;
        lm[i][K] = lab[K] > k ? l : Real(0);
        if constexpr (FACT) {
          a[K][k] = lab[K] > k ? l : a[K][k];   // L below the diagonal
          asm volatile("" : "+v"(a[K][k]));       // settled now, not at the store
        }
      });
      // (e) the rest of the panel takes this pivot's update now, so the next
      // column is complete when its search starts
      sfor<0, PC>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        sfor<K0, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          a[K][k + 1 + c] = fma_r(-lm[i][K], upan[c], a[K][k + 1 + c]);
        });
      });
    });

    // ---- end of panel: pivot rows to LDS records, read back as DPP sources
    if constexpr (W > 0) {
      if constexpr (k0 == 0) {
        // input check of the trailing columns and right-hand sides, not
        // touched before this first trailing update; -1 outranks a zero
        // pivot of the first panel
        sfor<0, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          sfor<bw, N>([&](auto cc) { inbad |= not_finite(a[K][decltype(cc)::value]); });
          sfor<0, NRHS>([&](auto jc) { inbad |= not_finite(y[K][decltype(jc)::value]); });
        });
        status = group_any<T>(inbad != 0, gbase) ? -1 : status;
      }
      constexpr int RECN = W + bw;                           // trailing entries + multipliers
      constexpr int NU = (W + SL - 1) / SL;                  // DPP source registers per pivot
      auto entry = [&](auto Kc, auto ec) -> Real {
        constexpr int K = decltype(Kc)::value;
        constexpr int e = decltype(ec)::value;
        if constexpr (e < NT) return a[K][k0 + bw + e];
        else if constexpr (e < W) return y[K][e - NT];
        else return lm[e - W][K];
      };
      // The owner of each pivot row writes its record (exec-masked: an LDS
      // write costs the same whatever the number of active lanes), one
      // register (pair) per entry at a compile-time offset.
      sfor<K0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int j = lab[K] - k0;
        if (j >= 0 && j < bw) {
          Real* dst = rec + j * S::REC_STRIDE;
          sfor<0, RECN>([&](auto ec) {
            constexpr int e = decltype(ec)::value;
            dst[e] = entry(Kc, ec);
          });
        }
      });
      wave_sync_lds();

      Real u[B][NU];
      const int st = tx % SL;
      sfor<0, bw>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        sfor<0, NU>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          u[m][r] = rec[m * S::REC_STRIDE + r * SL + st];   // entries past W are unused
        });
      });
      // the panel's own updates of its pivot rows (entries in step order)
      sfor<1, bw>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        sfor<0, j>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          const Real lmj = rec[j * S::REC_STRIDE + W + m];
          sfor<0, NU>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            u[j][r] = fma_r(-lmj, u[m][r], u[j][r]);
          });
        });
      });
      // trailing update: every row takes the panel's rank-1 updates in order.
      // Whole-wave groups go pivot by pivot (each accumulator is read again
      // only a full row later, so consecutive fused multiply-adds are
      // independent: about 5% faster at n = 64); the others entry by entry
      // (no gain from the reordering there).  Either way every element
      // takes the updates in step order.
      auto update = [&](auto ec, auto mc) {
        constexpr int e = decltype(ec)::value;
        constexpr int m = decltype(mc)::value;
        constexpr int L = e % SL;
        constexpr int r = e / SL;
        sfor<K0, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          constexpr bool first = (L == 0) && (K == K0);
          if constexpr (e < NT)
            fnmac_bcast<T, L, first>(a[K][k0 + bw + e], u[m][r], lm[m][K]);
          else
            fnmac_bcast<T, L, first>(y[K][e - NT], u[m][r], lm[m][K]);
        });
      };
      if constexpr (T == 64) {
        sfor<0, bw>([&](auto mc) { sfor<0, W>([&](auto ec) { update(ec, mc); }); });
      } else {
        sfor<0, W>([&](auto ec) { sfor<0, bw>([&](auto mc) { update(ec, mc); }); });
      }
      wave_sync_lds();  // records are rewritten by the next panel
    }
  });

  const bool nf = pz != pz;   // a pivot was an infinity or a NaN
  // The system index and group base again, from the wave's first system
  // and a lane index read anew: kept from the load, they held registers
  // through the whole factorization (spilled at three waves per SIMD).
  int lane_e = (int)threadIdx.x & (kWaveSize - 1);
  asm("" : "+v"(lane_e));
  const int64_t sys_e = wave_first + lane_e / T;
  const bool live_e = sys_e < batch;
  const int gbase_e = lane_e / T * T;   // the group's first lane, likewise

  if constexpr (FACT) {
    // ---- factors: every row, whatever lane holds it, is row lab of L\U
    // (multipliers before its position, U from it on); a failed system gets
    // +0.0 everywhere and pivots -1.  Under scaling, U takes its scale back.
    if (flags & kFlagScaleMaxAbs) {
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = lab[K];
        sfor<0, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          a[K][c] = (c >= q && c < n) ? a[K][c] * sc : a[K][c];
        });
      });
    }
    {
      bool bad = nf;
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = lab[K];
        const bool real = q >= 0 && q < n;
        sfor<0, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          bad |= real & (c < n) & not_finite(a[K][c]);
        });
      });
      if (group_any<T>(bad, gbase_e) && status == 0) status = -3;
    }
    const bool failed = status != 0;
    if (live_e) {
      Real* LUs = X + sys_start(sys_e, ilv, (int64_t)n * n);
      int32_t* Ps = piv + sys_start(sys_e, ilv, n);
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = lab[K];
        if (q >= 0 && q < n) {
          // row q: one base address and column offsets, compile-time ones
          // for the kernel's own size (a row-major row is then one run of
          // vector stores); a few stores at a time so that addresses are
          // not all formed ahead of them
          auto store_row = [&](auto colc, auto exactc) {
            constexpr bool COL = decltype(colc)::value;
            constexpr bool EXACT = decltype(exactc)::value;
            const int64_t ld = EXACT ? N : n;
            const int64_t es = EXACT ? 1 : ilv;  // element stride
            Real* rowp = LUs + (COL ? (int64_t)q : (int64_t)q * ld) * es;
            sfor<0, N>([&](auto cc) {
              constexpr int c = decltype(cc)::value;
              if (EXACT || c < n) rowp[(COL ? c * ld : c) * es] = failed ? Real(0) : a[K][c];
              if constexpr (c % 8 == 7) __builtin_amdgcn_sched_barrier(0);
            });
          };
          if (n == N && ilv == 1) {
            if (col)
              store_row(std::true_type{}, std::true_type{});
            else
              store_row(std::false_type{}, std::true_type{});
          } else {
            if (col)
              store_row(std::true_type{}, std::false_type{});
            else
              store_row(std::false_type{}, std::false_type{});
          }
        }
        const int qf = tx + K * T;
        if (qf < n) Ps[qf * ilv] = failed ? -1 : pv[K];
      });
      if (tx == 0) info[sys_e] = status;
    }
  } else {
    // ---- back substitution (see upper_solve_store): every row, whatever lane
    // holds it, stores its right-hand sides and then its U entries (columns
    // from its position on) by position
    int32_t* Ps = piv + sys_start(live_e ? sys_e : 0, ilv, n);
    wave_sync_lds();  // the last records have been read
    bool xbad;
    if constexpr (S::REG_SOLVE) {
      // ---- back substitution from registers (one right-hand side, the
      // group a DPP domain).  Every slot but the last already holds its
      // positions in order (slot K, lane tx: position K*T + tx) since the
      // last slot boundary; the rows of the last slot, permuted among
      // themselves by the steps since, go through LDS and come back in
      // position order (their U part, columns from the slot's first
      // position on, and their right-hand side).
      static_assert(R == 1 || COMPACT, "slots below the last are in position order");
      constexpr int KL = R - 1;
      constexpr int Q0 = KL * T;                 // first position of the last slot
      constexpr int NS2 = N - Q0;                // its rows
      constexpr int E2 = N - Q0 + NRHS;          // entries moved per row
      constexpr int RS2 = stage_stride(S::GROUP_ELEMS / NS2, (int)sizeof(Real));
      static_assert(RS2 >= VEC && NS2 * RS2 <= S::GROUP_ELEMS, "staging fits the group area");
      constexpr int NCH2 = (E2 + RS2 - 1) / RS2;
      auto ent2 = [&](auto ec) -> Real& {
        constexpr int e = decltype(ec)::value;
        if constexpr (e < N - Q0) return a[KL][Q0 + e];
        else return y[KL][e - (N - Q0)];
      };
      sfor<0, NCH2>([&](auto hc) {
        constexpr int e0 = decltype(hc)::value * RS2;
        constexpr int e1 = (e0 + RS2) < E2 ? (e0 + RS2) : E2;
        const int p = lab[KL];
        if (p >= Q0) {
          Real* dst = rec + (p - Q0) * RS2 - e0;   // entry e at dst[e]
          sfor<e0, e1>([&](auto ec) { dst[decltype(ec)::value] = ent2(ec); });
        }
        wave_sync_lds();
        if (Q0 + tx < N) {
          const Real* src = rec + tx * RS2 - e0;
          sfor<e0, e1>([&](auto ec) { ent2(ec) = src[decltype(ec)::value]; });
        }
        wave_sync_lds();
      });
      // U x = y: x_k = y_k / U(k,k) by IEEE division on lane k % T (slot
      // k / T) for k = n-1 .. 0, removed from the rows above by DPP inside
      // the fused multiply-add (the order of the TDLS page's Detailed
      // Description, the solution entry kept by its owner)
      Real xr[R];
      sfor<0, R>([&](auto Kc) { xr[decltype(Kc)::value] = Real(0); });
      auto solve_divide = [&]() __attribute__((always_inline)) {
        sfor<0, N>([&](auto ic) {
          constexpr int k = N - 1 - decltype(ic)::value;
          constexpr int kl = k % T;
          constexpr int ks = k / T;
          constexpr int SLK = kl % SL;
          const Real x = y[ks][0] / a[ks][k];   // meaningful on lane kl
          xr[ks] = tx == kl ? x : xr[ks];
          asm volatile("" : "+v"(xr[ks]));   // select now, not at the store
          sfor<0, ks + 1>([&](auto Kc) {
            constexpr int K = decltype(Kc)::value;
            fnmac_bcast<T, SLK, K == 0>(y[K][0], x, a[K][k]);
          });
        });
      };
      if constexpr (is64) {
        // float64: every lane forms the reciprocal of its own rows' diagonal
        // (slot K holds position K*T + tx) before the chain starts, so each
        // step costs three dependent operations instead of the division
        // sequence; afterwards each lane checks the steps it owned
        // (quot_div64_exact) and a wave with any miss solves again by
        // division from the saved right-hand sides (the same bits either way)
        double dg[R], rinv[R];
        sfor<0, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          constexpr int c0 = K * T < N ? K * T : N - 1;
          constexpr int c1 = (K + 1) * T < N ? (K + 1) * T : N;
          double d = a[K][c0];
          sfor<c0 + 1, c1>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            d = tx == c - K * T ? a[K][c] : d;
            asm volatile("" : "+v"(d));   // a chain of selects, not an indexed load
          });
          dg[K] = d;
          rinv[K] = recip_div64(d);
        });
        Real ysave[R], ny[R];
        sfor<0, R>([&](auto Kc) {
          ysave[decltype(Kc)::value] = y[decltype(Kc)::value][0];
          ny[decltype(Kc)::value] = Real(0);
        });
        sfor<0, N>([&](auto ic) {
          constexpr int k = N - 1 - decltype(ic)::value;
          constexpr int kl = k % T;
          constexpr int ks = k / T;
          constexpr int SLK = kl % SL;
          const double x = quot_div64(y[ks][0], a[ks][k], rinv[ks]);   // meaningful on lane kl
          xr[ks] = tx == kl ? x : xr[ks];
          ny[ks] = tx == kl ? y[ks][0] : ny[ks];
          asm volatile("" : "+v"(xr[ks]), "+v"(ny[ks]));   // select now, not at the store
          sfor<0, ks + 1>([&](auto Kc) {
            constexpr int K = decltype(Kc)::value;
            fnmac_bcast<T, SLK, K == 0>(y[K][0], x, a[K][k]);
          });
        });
        bool miss = false;
        sfor<0, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          miss |= (tx + K * T < N) & !quot_div64_exact(ny[K], dg[K], xr[K]);
        });
        if (__builtin_amdgcn_ballot_w64(miss) != 0) {
          sfor<0, R>([&](auto Kc) { y[decltype(Kc)::value][0] = ysave[decltype(Kc)::value]; });
          solve_divide();
        }
      } else {
        solve_divide();
      }
      bool bad = false;
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        bad |= (tx + K * T < n) & not_finite(xr[K]);
      });
      xbad = group_any<T>(bad, gbase_e);
      if (live_e) {
        const bool zero = status != 0 || nf || xbad;
        Real* Xs = X + sys_start(sys_e, ilv, (int64_t)n * nrhs);
        sfor<0, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          const int q = tx + K * T;
          if (q < n) Xs[q * ilv] = zero ? Real(0) : xr[K];   // one column: same address in both layouts
        });
      }
    } else
    xbad = upper_solve_store<Real, N, NRHS, T>(
        rec, tx, gbase_e, live_e, status != 0 || nf, live_e ? sys_e : 0, n, nrhs, col, ilv, X,
        [&](Real* yt) {
          sfor<0, R>([&](auto Kc) {
            constexpr int K = decltype(Kc)::value;
            const int q = lab[K];
            if (q >= 0) {
              sfor<0, NRHS>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                yt[q * NRHS + j] = y[K][j];
              });
            }
          });
        },
        [&](Real* ut) {
          sfor<0, R>([&](auto Kc) {
            constexpr int K = decltype(Kc)::value;
            const int q = lab[K];
            if (q >= 0) {
              Real* row = ut + utri_row<N>(q) - q;   // entry of column c at row[c]
              sfor<0, N>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                if (c >= q) row[c] = a[K][c];
              });
            }
          });
        });

    if (status == 0 && (nf || xbad)) status = -3;
    const bool failed = status != 0;

    // ---- piv (all -1 for a failed system) and info
    if (live_e) {
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        if (q < n) Ps[q * ilv] = failed ? -1 : pv[K];
      });
      if (tx == 0) info[sys_e] = status;
    }
  }
}

}  // namespace tdls
