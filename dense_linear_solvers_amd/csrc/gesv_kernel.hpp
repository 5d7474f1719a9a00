// Batched gesv kernel: LU with partial row pivoting plus forward and back
// substitution, one n x n system per group of T lanes of a wave64, rows held
// in VGPRs.
//
// Method (cited by page title and section):
//  * "solver_static.hpp File Reference" (TDLS CooperativeLUpp), Detailed
//    Description: right-looking LU with partial pivoting of the rows held by
//    a group of lanes; lane tx holds rows tx, tx+T, tx+2T, ... ; the forward
//    substitution L y = P b is carried along with every rank-1 step, then
//    U x = y; with physical row interchanges position k always lives in slot
//    k / T of lane k % T.  "Departures from the MAGMA kernel": several
//    systems per wave, phantom rows skipped, x_i kept in a register of the
//    lane owning row i during the back substitution, a zero pivot replaced
//    by a divisor of 1 so that the factorization stays finite.
//    "Fixed barrier sequence": the sequence of exchanges never depends on
//    the data; a singular verdict is returned at the end.  "Workspace":
//    two exchange records per step (the row entering position k and the row
//    leaving it).
//  * "ruSOLVER：小矩阵 kernel 优化（实验性）", section on the unchanged
//    numerical and failure contract: partial row pivoting, ties to the lowest
//    row number, exact quotients (no reciprocal approximation), status 0 or
//    first failed pivot, failed system zeroed with all pivots -1, input
//    read-only and separate outputs.
//
// gfx950 design: a group never spans two waves (T <= 64), so the lanes of a
// group run in lockstep and the exchanges need only ordering inside the
// wave (an LDS fence), never a workgroup barrier.  Each step k of the
// unrolled factorization:
//   1. pivot search: first maximum of |a(q,k)| over the lane's slots in
//      increasing position (strict >), then a butterfly over the T lanes on
//      the key (magnitude descending, position ascending): the lowest current
//      position wins a tie.
//   2. status: the first exactly zero pivot sets info = k + 1.
//   3. exchange: the owner of the pivot position p writes that row to record
//      P, the owner of position k writes its row to record K (LDS,
//      double-buffered over k so one fence per step suffices); every lane
//      reads the pivot row from P, the owner of p takes the old row k from K,
//      the owner of k keeps the pivot row as row k of U.
//   4. elimination: l = a(q,k) / u_kk by IEEE division for every position
//      q > k, then a(q,c) = fma(-l, u_kc, a(q,c)) for c > k and the same for
//      the right-hand sides.
// Back substitution, k = n-1 .. 0: the owner of position k divides, the
// quotient is broadcast to the group and every lane folds it into the rows
// above k that it owns.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "tdls_internal.h"

namespace tdls {

template <typename Real, int N, int NRHS, int T>
struct GesvShape {
  static_assert((T & (T - 1)) == 0 && T >= 1 && T <= kWaveSize, "T must be a power of two <= 64");
  static constexpr int R = (N + T - 1) / T;           // slots (rows) per lane
  static constexpr int G = kWaveSize / T;             // systems per wave
  static constexpr int REC = N + NRHS;                // entries of one exchange record
  static constexpr int REC_STRIDE = REC + 1;          // odd pitch in elements
  static constexpr int GROUP_ELEMS = gesv_group_elems(N, NRHS);  // 2 buffers x 2 records
  static_assert(GROUP_ELEMS == 4 * REC_STRIDE, "record layout");
  static constexpr int BLOCK_ELEMS = kWavesPerBlock * G * GROUP_ELEMS;
  static constexpr int LDS_BYTES = BLOCK_ELEMS * (int)sizeof(Real);
};

__device__ __forceinline__ float abs_val(float x) { return __builtin_fabsf(x); }
__device__ __forceinline__ double abs_val(double x) { return __builtin_fabs(x); }
__device__ __forceinline__ float fma_op(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_op(double a, double b, double c) { return __builtin_fma(a, b, c); }

// Orders the LDS writes of the lanes of this wave before the reads that
// follow.  Lanes of a wave issue in lockstep and the LDS serves one wave's
// requests in order; the fences keep the compiler from moving LDS accesses
// across this point and wait for the outstanding ones.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int T>
__device__ __forceinline__ int lane_xor_i(int v, int mask) {
  return __shfl_xor(v, mask, T);
}
template <int T, typename Real>
__device__ __forceinline__ Real lane_xor_r(Real v, int mask) {
  return __shfl_xor(v, mask, T);
}
template <int T, typename Real>
__device__ __forceinline__ Real lane_bcast_r(Real v, int src) {
  return __shfl(v, src, T);
}

// Compile-time loop: calls f(std::integral_constant<int, I>) for I = B..E-1
// in increasing order, so that every register-array index below is a
// constant whatever the unroller decides (no dynamic VGPR indexing, no
// scratch).
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <typename Real, int N, int NRHS, int T>
__global__ void __launch_bounds__(kWaveSize* kWavesPerBlock)
    gesv_kernel(int col, int n, int nrhs, int64_t batch, const Real* __restrict__ A,
                const Real* __restrict__ B, Real* __restrict__ X, int32_t* __restrict__ piv,
                int32_t* __restrict__ info) {
  using S = GesvShape<Real, N, NRHS, T>;
  constexpr int R = S::R;
  constexpr int G = S::G;
  __shared__ Real lds[S::BLOCK_ELEMS];

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = threadIdx.x / kWaveSize;
  const int g = lane / T;
  const int tx = lane & (T - 1);
  const int64_t wave_first = ((int64_t)blockIdx.x * kWavesPerBlock + wave) * G;
  if (wave_first >= batch) return;  // the whole wave is past the batch
  const int64_t sys = wave_first + g;
  const bool live = sys < batch;
  Real* rec = lds + (wave * G + g) * S::GROUP_ELEMS;

  Real a[R][N];
  Real y[R][NRHS];
  int pv[R];

  // ---- load: lane tx takes positions q = tx + K*T.  Positions n..N-1 are
  // an identity block and right-hand-side columns nrhs..NRHS-1 are zero, so
  // a padded system has the pivots, status and solution of the original.
  {
    const int64_t nn = (int64_t)n * n;
    const int64_t nb = (int64_t)n * nrhs;
    const Real* As = A + (live ? sys : 0) * nn;
    const Real* Bs = B + (live ? sys : 0) * nb;
    static_for<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      const bool qrow = live && q < n;
      static_for<0, N>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        Real v = (q == c) ? Real(1) : Real(0);
        if (qrow && c < n) v = col ? As[(int64_t)c * n + q] : As[(int64_t)q * n + c];
        a[K][c] = v;
      });
      static_for<0, NRHS>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        Real v = Real(0);
        if (qrow && j < nrhs) v = col ? Bs[(int64_t)j * n + q] : Bs[(int64_t)q * nrhs + j];
        y[K][j] = v;
      });
      pv[K] = q;
    });
  }

  int status = 0;

  // ---- factorization with the forward substitution folded in
  static_for<0, N>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int kl = k % T;  // lane owning position k
    constexpr int ks = k / T;  // its slot

    // 1. pivot search: first maximum over this lane's slots, then the group
    Real best = Real(-1);
    int bpos = 0x7fffffff;
    Real bval = Real(0);
    static_for<ks, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      const bool act = (K > ks || tx >= kl) && (K * T + T <= N || q < N);
      const Real v = abs_val(a[K][k]);
      if (act && v > best) {
        best = v;
        bpos = q;
        bval = a[K][k];
      }
    });
    static_for<0, 6>([&](auto mc) {
      constexpr int m = 1 << decltype(mc)::value;
      if constexpr (m < T) {
        const Real ob = lane_xor_r<T>(best, m);
        const int op = lane_xor_i<T>(bpos, m);
        const Real ov = lane_xor_r<T>(bval, m);
        const bool take = (ob > best) || (ob == best && op < bpos);
        best = take ? ob : best;
        bpos = take ? op : bpos;
        bval = take ? ov : bval;
      }
    });
    // 2. status.  No candidate compared (every magnitude NaN) counts as zero.
    const int p = bpos == 0x7fffffff ? k : bpos;
    const bool zero_pivot = !(best > Real(0));
    if (zero_pivot && status == 0) status = k + 1;
    const Real d = zero_pivot ? Real(1) : bval;

    // 3. exchange through the double-buffered records
    Real* recP = rec + (k & 1) * 2 * S::REC_STRIDE;
    Real* recK = recP + S::REC_STRIDE;
    static_for<ks, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      if (tx + K * T == p) {
        static_for<k, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          recP[c] = a[K][c];
        });
        static_for<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          recP[N + j] = y[K][j];
        });
      }
    });
    if (tx == kl) {
      static_for<k, N>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        recK[c] = a[ks][c];
      });
      static_for<0, NRHS>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        recK[N + j] = y[ks][j];
      });
    }
    wave_lds_sync();

    // the owner of p takes the row that leaves position k
    static_for<ks, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      if (tx + K * T == p) {
        static_for<k, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          a[K][c] = recK[c];
        });
        static_for<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          y[K][j] = recK[N + j];
        });
      }
    });

    // 4. multipliers of the positions below k (IEEE division), then the
    // rank-1 update with the pivot row read once per column
    Real l[R];
    static_for<ks, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      l[K] = (q > k && q < N) ? a[K][k] / d : Real(0);
    });
    static_for<k + 1, N>([&](auto cc) {
      constexpr int c = decltype(cc)::value;
      const Real uc = recP[c];
      static_for<ks, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        if (q > k && q < N) a[K][c] = fma_op(-l[K], uc, a[K][c]);
      });
    });
    static_for<0, NRHS>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const Real uj = recP[N + j];
      static_for<ks, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        if (q > k && q < N) y[K][j] = fma_op(-l[K], uj, y[K][j]);
      });
    });
    // the owner of k keeps the pivot row as row k of U
    if (tx == kl) {
      static_for<k, N>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        a[ks][c] = recP[c];
      });
      static_for<0, NRHS>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        y[ks][j] = recP[N + j];
      });
      pv[ks] = p;
    }
  });

  // ---- back substitution: x_k = y_k / u_kk on the owner of k, broadcast,
  // then folded into the rows above k.  x_k stays in its owner's register.
  static_for<0, N>([&](auto ic) {
    constexpr int k = N - 1 - decltype(ic)::value;
    constexpr int kl = k % T;
    constexpr int ks = k / T;
    Real xk[NRHS];
    static_for<0, NRHS>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const Real xo = y[ks][j] / a[ks][k];
      if constexpr (T > 1)
        xk[j] = lane_bcast_r<T>(xo, kl);
      else
        xk[j] = xo;
    });
    if (tx == kl) {
      static_for<0, NRHS>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        y[ks][j] = xk[j];
      });
    }
    static_for<0, ks + 1>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      if (q < k) {
        static_for<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          y[K][j] = fma_op(-a[K][k], xk[j], y[K][j]);
        });
      }
    });
  });

  // ---- store: X in B's layout, piv, info.  A failed system gets +0.0 and -1.
  if (live) {
    const int64_t nb = (int64_t)n * nrhs;
    Real* Xs = X + sys * nb;
    int32_t* Ps = piv + sys * (int64_t)n;
    const bool failed = status != 0;
    static_for<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      if (q < n) {
        static_for<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          if (j < nrhs) {
            const Real v = failed ? Real(0) : y[K][j];
            if (col)
              Xs[(int64_t)j * n + q] = v;
            else
              Xs[(int64_t)q * nrhs + j] = v;
          }
        });
        Ps[q] = failed ? -1 : pv[K];
      }
    });
    if (tx == 0) info[sys] = status;
  }
}

}  // namespace tdls
