// Batched getrs: X = A^-1 B from the factors that the factorization kernel
// writes (P A = L U in LAPACK's row order, unit-lower L below the diagonal,
// U on and above it, the 0-based swap sequence), one system per group of T
// lanes of a wave64, lane tx holding the fixed positions tx, tx+T, ...
//
// What is computed (cited by page title and section):
//  * "solver_static.hpp File Reference" (TDLS CooperativeLUpp), section
//    Factored format: under physical interchanges the rows end in the
//    pivoted order as in LAPACK, L's multipliers before the diagonal, U from
//    it on, the pivots themselves on the diagonal, and the factorization is
//    consumed by the substitution routines of the same solver; Detailed
//    Description: the forward substitution L y = P b, then U x = y, the
//    solution entry kept by the lane that owns its row.
//  * "ruSOLVER：小矩阵 kernel 优化（实验性）", section on the unchanged
//    numerical and failure contract: a failed factorization (every pivot
//    -1) yields no usable solution, so its X is +0.0 everywhere; inputs are
//    read only and results go to a separate buffer.
//
// Arithmetic order: the right-hand sides are gathered in the pivoted order
// (the swaps applied in sequence), then y_r -= L(r,k) y_k for k = 0, 1, ...
// and x_k = y_k / U(k,k), y_r -= U(r,k) x_k for k = n-1, ..., 0, each a
// fused multiply-add; every element sees the operations of the elimination
// that produced the factors in the same order, so factor-then-solve gives
// the same bits as the one-call solve.
//
// Layouts: up to two right-hand sides go by fixed positions, the
// broadcasts by DPP inside the fused multiply-adds; four or more go by
// column classes (each lane holds a few positions of one class of columns,
// so a step's divisions are spread over the lanes), with the factors staged
// through LDS.
#pragma once

#include "gesv_panel.hpp"

namespace tdls {

template <typename Real, int N, int NRHS, int T>
struct GetrsShape {
  static_assert(T == 4 || T == 16 || T == 32 || T == 64, "group size must be 4, 16, 32 or 64");
  static constexpr int R = (N + T - 1) / T;   // positions per lane
  static constexpr int G = kWaveSize / T;     // systems per wave
  static constexpr int SL = T < 16 ? T : 16;  // lanes per DPP broadcast domain
  static constexpr int VEC = RealTraits<Real>::VEC;
  static constexpr int PIV_BYTES = (N * 4 + 15) / 16 * 16;
  static constexpr int UTRI_PAD = (N * (N + 1) / 2 + VEC - 1) / VEC * VEC;
  static constexpr int TRI = UTRI_PAD > N * NRHS ? UTRI_PAD : N * NRHS;
  // column classes from 4 right-hand sides on (measured: 2.2x faster at
  // n = 64 with 8, 1.8x at n = 16 with 4, 13% slower at n = 24 with 2)
  static constexpr bool CLASSES = NRHS >= 4;
  static constexpr int ELEMS = CLASSES ? (TRI + VEC - 1) / VEC * VEC : 0;
  // 16- and 64-lane groups load B unpermuted with L\U and permute it
  // through LDS (the class area when there is one, else a staging area)
  static constexpr bool EARLY = T >= 16;
  static constexpr int STAGE =
      (EARLY && !CLASSES) ? (N * NRHS * (int)sizeof(Real) + 15) / 16 * 16 : 0;
  static constexpr int GROUP_BYTES = PIV_BYTES + ELEMS * (int)sizeof(Real) + STAGE;
  static constexpr int BLOCK_BYTES = kWavesPerBlock * G * GROUP_BYTES;
};

template <typename Real, int N, int NRHS, int T>
__global__ void __launch_bounds__(kWaveSize* kWavesPerBlock)
    getrs_kernel(int col, int n, int nrhs, int64_t batch, const Real* __restrict__ LU,
                 const int32_t* __restrict__ piv, const Real* __restrict__ Bm,
                 Real* __restrict__ X, int64_t ilv) {
  using S = GetrsShape<Real, N, NRHS, T>;
  constexpr int R = S::R;
  constexpr int G = S::G;
  constexpr int SL = S::SL;
  extern __shared__ __align__(16) unsigned char lds_raw[];

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = threadIdx.x / kWaveSize;
  const int g = lane / T;
  const int tx = lane & (T - 1);
  const int gbase = g * T;
  const int64_t wave_first = (block_of(ilv) * kWavesPerBlock + wave) * G;
  if (wave_first >= batch) return;  // the whole wave is past the batch
  const int64_t sys = wave_first + g;
  const bool live = sys < batch;
  unsigned char* glds = lds_raw + (wave * G + g) * S::GROUP_BYTES;
  int32_t* pl = reinterpret_cast<int32_t*>(glds);

  // ---- load: row q of L\U for each position q of the lane (past n the
  // identity), and row src(q) of B (past n zero), src(q) being the row the
  // pivot walk below brings to position q.  Source rows are clamped into
  // the matrix, so a malformed pivot cannot address outside it.  With 16-
  // and 64-lane groups both are loaded before the walk, which they do not
  // depend on, so their latency overlaps it: B by original row, put in
  // pivoted order through LDS afterwards (n = 32 float64: 0.444 -> 0.415 ms
  // for the early L\U alone).  With quads (four rows per lane) the rows
  // would stay live through the walk and cost occupancy (n = 16 float32:
  // 0.0265 -> 0.031 ms), so there both follow it and B is read in pivoted
  // order directly.
  constexpr bool EARLY_LU = S::EARLY;
  Real a[R][N];
  Real y[R][NRHS];
  const bool exact = n == N && nrhs == NRHS && ilv == 1;
  const Real* Bs = Bm + sys_start(live ? sys : 0, ilv, (int64_t)n * nrhs);
  auto load_lu = [&]() {
    const Real* Ls = LU + sys_start(live ? sys : 0, ilv, (int64_t)n * n);
    if (exact) {
      // the kernel's own size: compile-time offsets from one base per row
      // (a row-major row is one run of vector loads)
      auto load_exact = [&](auto colc) {
        constexpr bool COL = decltype(colc)::value;
        sfor<0, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          const int q = tx + K * T;
          const int qq = live && q < n ? q : 0;
          const Real* lr = Ls + (COL ? qq : qq * N);
          sfor<0, N>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            a[K][c] = lr[COL ? c * N : c];
          });
          if constexpr (EARLY_LU) {   // row q of B, put in pivoted order later
            const Real* br = Bs + (COL ? qq : qq * NRHS);
            sfor<0, NRHS>([&](auto jc) {
              constexpr int j = decltype(jc)::value;
              y[K][j] = br[COL ? j * N : j];
            });
          }
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
        sfor<0, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          a[K][c] = (q == c) ? Real(1) : Real(0);
          if (qrow && c < n) a[K][c] = Ls[(col ? (int64_t)c * n + qq : (int64_t)qq * n + c) * ilv];
        });
        if constexpr (EARLY_LU) {   // row q of B, put in pivoted order later
          sfor<0, NRHS>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            y[K][j] = Real(0);
            if (qrow && j < nrhs)
              y[K][j] = Bs[(col ? (int64_t)j * n + qq : (int64_t)qq * nrhs + j) * ilv];
          });
        }
      });
    }
  };
  if constexpr (EARLY_LU) load_lu();

  // ---- the swap sequence to LDS (the identity past n and for groups past
  // the batch), then the source row of each position: walking the swaps
  // from the last to the first maps a position to the row it receives.
  const int32_t* Ps = piv + sys_start(live ? sys : 0, ilv, n);
  sfor<0, R>([&](auto Kc) {
    constexpr int K = decltype(Kc)::value;
    const int q = tx + K * T;
    if (q < N) pl[q] = (live && q < n) ? Ps[q * ilv] : q;
  });
  wave_sync_lds();
  const bool failed = pl[0] < 0;   // a failed factorization: every pivot -1
  int src[R];
  sfor<0, R>([&](auto Kc) { src[decltype(Kc)::value] = tx + decltype(Kc)::value * T; });
  sfor<0, N>([&](auto ic) {
    constexpr int k = N - 1 - decltype(ic)::value;
    const int pk = failed ? k : pl[k];
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      src[K] = src[K] == k ? pk : (src[K] == pk ? k : src[K]);
    });
  });
  if constexpr (!EARLY_LU) load_lu();

  auto src_row = [&](int K) { return src[K] < 0 ? 0 : (src[K] >= n ? n - 1 : src[K]); };
  if constexpr (EARLY_LU) {
    // B by original row to LDS (after the swap sequence, which it follows
    // in memory), then each position reads its source row
    Real* stg = reinterpret_cast<Real*>(glds + S::PIV_BYTES);
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      if (q < n) {
        sfor<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          stg[q * NRHS + j] = y[K][j];
        });
      }
    });
    wave_sync_lds();
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      const Real* sr = stg + src_row(K) * NRHS;
      sfor<0, NRHS>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        y[K][j] = (q < n) ? sr[j] : Real(0);
      });
    });
    wave_sync_lds();   // read before the staging area is reused
  } else {
    if (exact) {
      auto load_b = [&](auto colc) {
        constexpr bool COL = decltype(colc)::value;
        sfor<0, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          const int q = tx + K * T;
          const int sr = src_row(K);
          const Real* br = Bs + (COL ? sr : sr * NRHS);
          sfor<0, NRHS>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            y[K][j] = q < N ? br[COL ? j * N : j] : Real(0);
          });
        });
      };
      if (col)
        load_b(std::true_type{});
      else
        load_b(std::false_type{});
    } else {
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        const bool qrow = live && q < n;
        const int sr = src_row(K);
        sfor<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          y[K][j] = Real(0);
          if (qrow && j < nrhs)
            y[K][j] = Bs[(col ? (int64_t)j * n + sr : (int64_t)sr * nrhs + j) * ilv];
        });
      });
    }
  }

  if constexpr (S::CLASSES) {
    // ---- several right-hand sides: both substitutions in the column-class
    // / row-phase layout of the back substitution of the LU kernel (lane
    // j0 * P + ph holds the right-hand-side columns j0 + NJ*jj of the
    // positions ph + P*m; a class is P consecutive lanes, so y_k reaches its
    // class by DPP), so a step costs one division per column class rather
    // than NRHS divisions on one lane.  The forward substitution reads L from a
    // row-packed lower triangle in LDS (row i at i (i + 1) / 2, unit
    // diagonal implied); the back substitution is the LU kernel's.
    Real* ws = reinterpret_cast<Real*>(glds + S::PIV_BYTES);
    constexpr int NJ = NRHS < T ? NRHS : T;
    constexpr int P = T / NJ;
    constexpr int JR = NRHS / NJ;
    constexpr int QR = (N + P - 1) / P;
    const int j0 = tx / P;   // column class: P consecutive lanes
    const int ph = tx % P;
    auto ltri = [](int i) { return i * (i + 1) / 2; };
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      if (q < N) {
        sfor<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          ws[q * NRHS + j] = y[K][j];
        });
      }
    });
    wave_sync_lds();
    Real yv[QR][JR];
    const Real* lrow[QR];
    sfor<0, QR>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      const int q = ph + P * m;
      const int qq = q < N ? q : N - 1;
      sfor<0, JR>([&](auto jc) {
        constexpr int jj = decltype(jc)::value;
        yv[m][jj] = ws[qq * NRHS + j0 + NJ * jj];
      });
      lrow[m] = ws + ltri(qq);   // L(q, c) at lrow[m][c], c < q
    });
    wave_sync_lds();   // read before L overwrites them
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      if (q < N) {
        Real* rowp = ws + ltri(q);
        sfor<0, (K + 1) * T < N ? (K + 1) * T : N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if (c < q) rowp[c] = a[K][c];
        });
      }
    });
    wave_sync_lds();
    // L y = P b: y_k (final on the lanes of phase k % P) leaves the rows
    // below it
    // L(i, k) of this lane's rows read one step ahead (two register
    // buffers), so a step's LDS reads overlap the step before
    Real lb[2][QR];
    auto read_l = [&](auto kcc) {
      constexpr int k2 = decltype(kcc)::value;
      sfor<k2 / P, QR>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        lb[k2 % 2][m] = lrow[m][k2];   // L(i, k2), i = ph + P*m (meaningful for i > k2)
      });
    };
    read_l(std::integral_constant<int, 0>{});
    sfor<0, N - 1>([&](auto kc) {
      constexpr int k = decltype(kc)::value;
      constexpr int kp = k % P;
      constexpr int km = k / P;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (k + 1 < N - 1) read_l(std::integral_constant<int, k + 1>{});
      Real lik[QR];
      sfor<km, QR>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        const Real v = lb[k % 2][m];
        if constexpr (m == km)
          lik[m] = ph > kp ? v : Real(0);
        else
          lik[m] = v;
      });
      sfor<0, JR>([&](auto jc) {
        constexpr int jj = decltype(jc)::value;
        Real yb;
        if constexpr (P == 1)
          yb = yv[km][jj];
        else if constexpr (P <= 16)
          yb = class_bcast<P, kp>(yv[km][jj]);   // lane kp of the class, by DPP
        else
          yb = lane_fetch_any(yv[km][jj], gbase + j0 * P + kp);
        sfor<km, QR>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          yv[m][jj] = fma_r(-lik[m], yb, yv[m][jj]);
        });
      });
    });
    wave_sync_lds();   // L read before the back substitution rewrites the area
    upper_solve_store<Real, N, NRHS, T, false>(
        ws, tx, gbase, live, failed, live ? sys : 0, n, nrhs, col, ilv, X,
        [&](Real* yt) {
          sfor<0, QR>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            const int q = ph + P * m;
            if (q < N) {
              sfor<0, JR>([&](auto jc) {
                constexpr int jj = decltype(jc)::value;
                yt[q * NRHS + j0 + NJ * jj] = yv[m][jj];
              });
            }
          });
        },
        [&](Real* ut) {
          sfor<0, R>([&](auto Kc) {
            constexpr int K = decltype(Kc)::value;
            const int q = tx + K * T;
            if (q < N) {
              Real* row = ut + utri_row<N>(q) - q;   // entry of column c at row[c]
              sfor<0, N>([&](auto cc) {
                constexpr int c = decltype(cc)::value;
                if (c >= q) row[c] = a[K][c];
              });
            }
          });
        });
    return;
  }

  // ---- L y = P b: y_k (lane k % T, slot k / T) leaves the rows below it.
  // The slot of k itself goes last, so the broadcast source is not rewritten
  // before the other slots have read it.
  sfor<0, N - 1>([&](auto kc) {
    constexpr int k = decltype(kc)::value;
    constexpr int kl = k % T;
    constexpr int ks = k / T;
    constexpr int SLK = kl % SL;
    const Real mk = tx > kl ? a[ks][k] : Real(0);   // rows of slot ks below k
    sfor<0, NRHS>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      if constexpr (T <= 16) {
        sfor<ks + 1, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          fnmac_bcast<T, SLK, K == ks + 1>(y[K][j], y[ks][j], a[K][k]);
        });
        fnmac_bcast<T, SLK, ks + 1 == R>(y[ks][j], y[ks][j], mk);
      } else {
        const Real yk = lane_fetch<T>(y[ks][j], gbase + kl);
        sfor<ks + 1, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          y[K][j] = fma_r(-a[K][k], yk, y[K][j]);
        });
        y[ks][j] = fma_r(-mk, yk, y[ks][j]);
      }
    });
  });

  // ---- U x = y: x_k = y_k / U(k,k) on lane k % T, kept there, and removed
  // from the rows above.
  Real xr[R][NRHS];
  sfor<0, R>([&](auto Kc) {
    sfor<0, NRHS>([&](auto jc) { xr[decltype(Kc)::value][decltype(jc)::value] = Real(0); });
  });
  sfor<0, N>([&](auto ic) {
    constexpr int k = N - 1 - decltype(ic)::value;
    constexpr int kl = k % T;
    constexpr int ks = k / T;
    constexpr int SLK = kl % SL;
    const Real mk = tx < kl ? a[ks][k] : Real(0);   // rows of slot ks above k
    sfor<0, NRHS>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      const Real x = y[ks][j] / a[ks][k];   // meaningful on lane kl
      xr[ks][j] = tx == kl ? x : xr[ks][j];
      asm volatile("" : "+v"(xr[ks][j]));   // select now, not at the store
      if constexpr (T <= 16) {
        sfor<0, ks>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          fnmac_bcast<T, SLK, K == 0>(y[K][j], x, a[K][k]);
        });
        fnmac_bcast<T, SLK, ks == 0>(y[ks][j], x, mk);
      } else {
        const Real xk = lane_fetch<T>(x, gbase + kl);
        sfor<0, ks>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          y[K][j] = fma_r(-a[K][k], xk, y[K][j]);
        });
        y[ks][j] = fma_r(-mk, xk, y[ks][j]);
      }
    });
  });

  // ---- store X (all +0.0 when the factorization failed)
  if (live) {
    Real* Xs = X + sys_start(sys, ilv, (int64_t)n * nrhs);
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      if (q < n) {
        sfor<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          if (j < nrhs) {
            const Real v = failed ? Real(0) : xr[K][j];
            if (col)
              Xs[((int64_t)j * n + q) * ilv] = v;
            else
              Xs[((int64_t)q * nrhs + j) * ilv] = v;
          }
        });
      }
    });
  }
}

}  // namespace tdls
