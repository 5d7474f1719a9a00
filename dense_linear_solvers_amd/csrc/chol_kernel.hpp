// Batched Cholesky: (A + shift I) = L L^T, then (posv) L y = b and L^T x = y,
// one n x n symmetric system per group of T lanes (T = 4, 16 or 64) of a
// wave64, lane tx holding the fixed rows tx, tx+T, ... in VGPRs.
//
// What is computed (cited by page title and section):
//  * "ruSOLVER：小矩阵 kernel 优化（实验性）", section on the unchanged
//    numerical and failure contract: the Cholesky inner products accumulate
//    in increasing k and only independent rows run in parallel; the diagonal
//    shift is explicit and nothing else is added; status 0, the first failed
//    pivot (positive), -2 for a matrix that is not symmetric; a failed
//    system's factors and solutions are all zero; inputs read only.
//  * "cuSolverDx potrf" function page: the status of a failed factorization
//    is the smallest leading minor that is not positive definite (1-based);
//    L is lower triangular.
//
// Order of the arithmetic, element by element: a(i,j) gets fma(-L(i,k),
// L(j,k), .) for k = 0, 1, ..., j-1 in that order (here applied right-looking,
// one k per step, which is the same sequence of fused multiply-adds as the
// left-looking inner product), the diagonal starts from A(j,j) + shift
// rounded once, L(j,j) = sqrt of it, L(i,j) = a(i,j) / L(j,j) by IEEE
// division.  The forward substitution is folded into the steps (y_j / L(j,j),
// then y_j leaves the rows below); the back substitution takes x_j =
// y_j / L(j,j) for j = n-1 .. 0 and removes it from the rows above.
//
// gfx950 design.  There is no pivot search: row r stays in lane r % T, slot
// r / T.  The column of multipliers just formed is itself the broadcast
// source of the rank-1 update: L(c,j) sits in lane c % T, slot c / T, which
// is the lane a DPP row_newbcast (T = 16) or quad_perm (T = 4) reads, with
// no exchange through LDS.  A whole-wave group (T = 64) spans four DPP rows,
// so its column goes through LDS once per step and each row reads back the
// entries it broadcasts.  Only slots that hold rows at or below column c
// take the update of column c.  The symmetry check and
// the back substitution read a row-major copy of the matrix (then of L) in
// LDS with an odd row stride.
#pragma once

#include "gesv_panel.hpp"

namespace tdls {

template <typename Real, int N, int NRHS, int T>
struct CholShape {
  static_assert(T == 4 || T == 16 || T == 64, "Cholesky groups are 4, 16 or 64 lanes");
  static constexpr int R = (N + T - 1) / T;
  static constexpr int G = kWaveSize / T;
  static constexpr int SL = T < 16 ? T : 16;
  static constexpr int S = N + 1;   // LDS row stride of the symmetry chunks (odd)
  static constexpr int CH = T < 16 ? T : 16;   // rows per symmetry chunk (within one slot)
  static constexpr int VEC = RealTraits<Real>::VEC;
  static constexpr int UTRI_PAD = (N * (N + 1) / 2 + VEC - 1) / VEC * VEC;
  static constexpr int BIG1 = CH * S > UTRI_PAD ? CH * S : UTRI_PAD;
  static constexpr int BIG2 = BIG1 > N * NRHS ? BIG1 : N * NRHS;
  static constexpr int GROUP_ELEMS = (BIG2 + VEC - 1) / VEC * VEC;
  static constexpr int WAVE_BYTES = G * GROUP_ELEMS * (int)sizeof(Real);
  static constexpr int BLOCK_BYTES = kWavesPerBlock * WAVE_BYTES;
};

// Value of `v` on lane L of the caller's group (T = 4, 16) or of the wave
// (T = 64).
template <int T, int L>
__device__ __forceinline__ double group_bcast(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  uint32_t lo, hi;
  if constexpr (T == 64) {
    lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, L);
    hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), L);
  } else if constexpr (T == 16) {
    lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, 0x150 + L, 0xf, 0xf, true);
    hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), 0x150 + L, 0xf, 0xf, true);
  } else {
    constexpr int qp = L | (L << 2) | (L << 4) | (L << 6);
    lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)b, qp, 0xf, 0xf, true);
    hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(b >> 32), qp, 0xf, 0xf, true);
  }
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}
template <int T, int L>
__device__ __forceinline__ float group_bcast(float v) {
  const int b = __builtin_bit_cast(int, v);
  if constexpr (T == 64)
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, L));
  else if constexpr (T == 16)
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(b, 0x150 + L, 0xf, 0xf, true));
  else
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(b, L | (L << 2) | (L << 4) | (L << 6), 0xf, 0xf, true));
}

__device__ __forceinline__ double sqrt_ieee(double v) { return __builtin_sqrt(v); }
__device__ __forceinline__ float sqrt_ieee(float v) { return __builtin_sqrtf(v); }

// FACT = false: posv, X receives the solutions.  FACT = true: potrf (NRHS
// must be 1, Bm is not read), X receives L in the layout of A, zero above
// the diagonal.  SOLVE = true: potrs, A holds L as potrf writes it, X
// receives the solutions, info is not written.
template <typename Real, int N, int NRHS, int T, bool FACT, bool SOLVE = false>
__global__ void __launch_bounds__(kWaveSize* kWavesPerBlock)
    chol_kernel(int col, int n, int nrhs, int64_t batch, Real shift, const Real* __restrict__ A,
                const Real* __restrict__ Bm, Real* __restrict__ X, int32_t* __restrict__ info,
                int64_t ilv) {
  static_assert(!FACT || NRHS == 1, "the factorization runs with one (unused) right-hand side");
  static_assert(!(FACT && SOLVE), "potrs solves from given factors");
  using S = CholShape<Real, N, NRHS, T>;
  constexpr int R = S::R;
  constexpr int G = S::G;
  constexpr int SL = S::SL;
  constexpr int ST = S::S;
  extern __shared__ __align__(16) unsigned char lds_raw[];

  const int lane = threadIdx.x & (kWaveSize - 1);
  const int wave = threadIdx.x / kWaveSize;
  const int g = lane / T;
  const int tx = lane & (T - 1);
  const int64_t wave_first = (block_of(ilv) * kWavesPerBlock + wave) * G;
  if (wave_first >= batch) return;  // the whole wave is past the batch
  const int64_t sys = wave_first + g;
  const bool live = sys < batch;
  Real* sq = reinterpret_cast<Real*>(lds_raw + wave * S::WAVE_BYTES) + g * S::GROUP_ELEMS;

  // ---- load: row q = tx + K*T of A and of B; past n the identity and zero.
  // With several right-hand sides and whole-wave groups B is loaded after
  // the factorization (it plays no part in it), which keeps its registers
  // free meanwhile (n = 64 with 8: 171 -> 161 VGPRs, a third wave per SIMD);
  // smaller groups keep their occupancy either way and load it up front.
  constexpr bool LATE_B = !FACT && !SOLVE && NRHS > 1 && T == 64;
  Real a[R][N];
  Real y[R][NRHS];
  {
    const Real* As = A + sys_start(live ? sys : 0, ilv, (int64_t)n * n);
    const Real* Bs = Bm + sys_start(live ? sys : 0, ilv, (int64_t)n * nrhs);
    if (n == N && nrhs == NRHS && ilv == 1) {
      // the kernel's own size: compile-time offsets from one base per row
      auto load_exact = [&](auto colc) {
        constexpr bool COL = decltype(colc)::value;
        sfor<0, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          const int q = tx + K * T;
          const int qq = live && q < n ? q : 0;
          const Real* ar = As + (COL ? qq : qq * N);
          const Real* br = Bs + (COL ? qq : qq * NRHS);
          sfor<0, N>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            if constexpr (!SOLVE)
              a[K][c] = ar[COL ? c * N : c];
            else if constexpr (c >= (K + 1) * T)   // above the diagonal on every lane
              a[K][c] = Real(0);
            else if (c <= q)                       // potrs reads L's lower triangle only
              a[K][c] = ar[COL ? c * N : c];
            else
              a[K][c] = Real(0);
          });
          sfor<0, NRHS>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            if constexpr (FACT || LATE_B)
              y[K][j] = Real(0);
            else
              y[K][j] = br[COL ? j * N : j];
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
        sfor<0, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          a[K][c] = (q == c) ? Real(1) : Real(0);
          if (qrow && c < n && (!SOLVE || c <= q))
            a[K][c] = As[(col ? (int64_t)c * n + qq : (int64_t)qq * n + c) * ilv];
        });
        sfor<0, NRHS>([&](auto jc) {
          constexpr int j = decltype(jc)::value;
          y[K][j] = Real(0);
          if constexpr (!FACT && !LATE_B)
            if (qrow && j < nrhs)
              y[K][j] = Bs[(col ? (int64_t)j * n + qq : (int64_t)qq * nrhs + j) * ilv];
        });
      });
    }
  }

  int status = 0;
  int nf = 0;                  // a lane flag, settled at each step (asm barrier below)
  bool given_failed = false;   // potrs: the factor of a failed factorization
  if constexpr (SOLVE) {
    // ---- potrs: the rows hold L as potrf writes it (the entries above the
    // diagonal are never read).  A failed factorization leaves L all +0.0,
    // so L(0,0) == 0 marks it.  With one right-hand side L y = b runs here,
    // step by step exactly as the factorization's folded forward
    // substitution; with several, in the column-class solve below.
    given_failed = group_bcast<T, 0>(a[0][0]) == Real(0);
    if constexpr (NRHS == 1) {
      sfor<0, N>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        constexpr int js = j / T;
        constexpr int jl = j % T;
        constexpr int BL = T == 64 ? jl : jl % SL;
        const Real d = group_bcast<T, BL>(a[js][j]);
        const Real yj = y[js][0] / d;
        y[js][0] = tx == jl ? yj : y[js][0];
        const Real yb = group_bcast<T, BL>(y[js][0]);
        sfor<js, R>([&](auto Kc) {
          constexpr int K = decltype(Kc)::value;
          const Real l = K > js ? a[K][j] : (tx > jl ? a[K][j] : Real(0));
          y[K][0] = fma_r(-l, yb, y[K][0]);
        });
      });
    }
  } else {
    // ---- exact symmetry: CH rows at a time (lanes of one slot) go to LDS,
    // and every lane compares its row q with column q of the chunk
    int asym = 0;   // a lane value, settled per chunk (see below)
    sfor<0, (N + S::CH - 1) / S::CH>([&](auto cic) {
      constexpr int r0 = decltype(cic)::value * S::CH;
      constexpr int KC = r0 / T;                  // the slot holding rows r0 .. r0+CH-1
      constexpr int t0 = r0 - KC * T;             // and the first lane
      if (tx >= t0 && tx < t0 + S::CH && tx + KC * T < N) {
        sfor<0, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          sq[(tx - t0) * ST + c] = a[KC][c];
        });
      }
      wave_sync_lds();
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        const int qq = q < N ? q : N - 1;
        sfor<0, S::CH>([&](auto rc) {
          constexpr int r = r0 + decltype(rc)::value;
          if constexpr (r < N)
            asym |= (int)((q < N) & !(sq[(r - r0) * ST + qq] == a[K][r]));   // phantom rows excluded
        });
      });
      // settled now: left to the end, every comparison's lane mask stays live
      // in scalar registers
      asm volatile("" : "+v"(asym));
      wave_sync_lds();   // the chunk is rewritten next
    });
    // Status, in the ruSOLVER contract's order of precedence: -1 for a
    // non-finite input entry, -2 for a matrix that is not symmetric, the
    // first step whose pivot is not > 0 (j + 1), then -3 when a computed value
    // is not finite: a diagonal entry of L (nf), an entry of x, or an entry of
    // L.  A non-finite value never turns finite again in the updates that
    // follow, so a non-finite entry of L shows in x.
    {
      bool inbad = false;
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        sfor<0, N>([&](auto cc) { inbad |= not_finite(a[K][decltype(cc)::value]); });
        sfor<0, NRHS>([&](auto jc) { inbad |= not_finite(y[K][decltype(jc)::value]); });
      });
      // one status per group: any lane of the group that saw a non-finite
      // entry, else a mismatch
      status = group_any<T>(inbad, g * T) ? -1 : (group_any<T>(asym != 0, g * T) ? -2 : 0);
    }

    // ---- the explicit diagonal shift, added once to A(q,q)
    if (shift != Real(0)) {
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        sfor<0, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          if constexpr (c >= K * T && c < (K + 1) * T)
            a[K][c] = (q == c && q < n) ? a[K][c] + shift : a[K][c];
        });
      });
    }

    // ---- factorization with the forward substitution folded in
    sfor<0, N>([&](auto jc) {
      constexpr int j = decltype(jc)::value;
      constexpr int js = j / T;
      constexpr int jl = j % T;
      constexpr int BL = T == 64 ? jl : jl % SL;   // lane of row j in the broadcast domain
      const Real s = group_bcast<T, BL>(a[js][j]);
      const bool bad = !(s > Real(0));
      if (bad && status == 0) status = j + 1;
      asm volatile("" : "+v"(status));   // settled now, not at the store
      const Real d = bad ? Real(1) : sqrt_ieee(s);
      nf |= not_finite(d);
      asm volatile("" : "+v"(nf));
      // multipliers of the rows below j; row j itself takes d
      Real lm[R];
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        if constexpr (K < js) {
          lm[K] = Real(0);
        } else {
          const Real l = a[K][j] / d;
          if constexpr (K > js) {
            lm[K] = l;
            a[K][j] = l;
          } else {
            lm[K] = tx > jl ? l : Real(0);
            a[K][j] = tx > jl ? l : (tx == jl ? d : a[K][j]);
          }
          asm volatile("" : "+v"(a[K][j]));
        }
      });
      // forward substitution (one right-hand side: folded into the steps):
      // y_j / d on its lane, then y_j leaves the rows below
      sfor<0, NRHS>([&](auto rc) {
        constexpr int r = decltype(rc)::value;
        if constexpr (!FACT && NRHS == 1) {
          const Real yj = y[js][r] / d;
          y[js][r] = tx == jl ? yj : y[js][r];
          const Real yb = group_bcast<T, BL>(y[js][r]);
          sfor<js, R>([&](auto Kc) {
            constexpr int K = decltype(Kc)::value;
            y[K][r] = fma_r(-lm[K], yb, y[K][r]);
          });
        }
      });
      // rank-1 update of the columns right of j, on the slots holding rows at
      // or below each column; L(c, j) comes from lane c % T, slot c / T.  A
      // whole-wave group stages the column through LDS so that every 16-lane
      // row holds the entries it serves, then broadcasts by DPP inside the
      // fused multiply-add (instead of two readlanes per entry).
      if constexpr (T == 64) {
        static_assert(R == 1, "one row per lane in whole-wave groups");
        if (tx > j && tx < N) sq[tx] = a[0][j];
        wave_sync_lds();
        constexpr int NU = (N + 15) / 16;
        constexpr int U0 = (j + 1) / 16;
        // one 16-entry block at a time keeps one source register live
        sfor<U0, NU>([&](auto rc) {
          constexpr int r = decltype(rc)::value;
          const Real uc = sq[r * 16 + (tx & 15)];
          constexpr int c0 = r * 16 > j + 1 ? r * 16 : j + 1;
          constexpr int c1 = (r + 1) * 16 < N ? (r + 1) * 16 : N;
          sfor<c0, c1>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            fnmac_bcast<T, c % 16, c == c0>(a[0][c], uc, lm[0]);
          });
        });
        wave_sync_lds();   // read before the next column is written
      }
      if constexpr (T != 64) sfor<j + 1, N>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        constexpr int cs = c / T;
        constexpr int cl = c % T;
        if constexpr (T <= 16) {
          sfor<cs, R>([&](auto Kc) {
            constexpr int K = decltype(Kc)::value;
            // the first read of each source register after its write above
            // needs the DPP wait states
            if constexpr (K >= js)
              fnmac_bcast<T, cl % SL, K == cs && (c == j + 1 || cl == 0)>(a[K][c], a[cs][j],
                                                                          lm[K]);
          });
        }
      });
    });
  }

  if constexpr (LATE_B) {
    // the right-hand sides, and their part of the input check (-1 outranks
    // every other status)
    const Real* Bs = Bm + sys_start(live ? sys : 0, ilv, (int64_t)n * nrhs);
    bool bbad = false;
    sfor<0, R>([&](auto Kc) {
      constexpr int K = decltype(Kc)::value;
      const int q = tx + K * T;
      const bool qrow = live && q < n;
      const int qq = qrow ? q : 0;
      sfor<0, NRHS>([&](auto jc) {
        constexpr int j = decltype(jc)::value;
        y[K][j] = Real(0);
        if (qrow && j < nrhs)
          y[K][j] = Bs[(col ? (int64_t)j * n + qq : (int64_t)qq * nrhs + j) * ilv];
        bbad |= not_finite(y[K][j]);
      });
    });
    status = group_any<T>(bbad, g * T) ? -1 : status;
  }

  if constexpr (FACT) {
    // ---- L in the layout of A, zero above the diagonal; zero when failed
    {
      bool bad = nf != 0;
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        sfor<0, N>([&](auto cc) {
          constexpr int c = decltype(cc)::value;
          bad |= (q < n) & (c <= q) & not_finite(a[K][c]);
        });
      });
      if (group_any<T>(bad, g * T) && status == 0) status = -3;
    }
    const bool failed = status != 0;
    if (live) {
      Real* Ls = X + sys_start(sys, ilv, (int64_t)n * n);
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        if (q < n) {
          auto store_row = [&](auto colc, auto exactc) {
            constexpr bool COL = decltype(colc)::value;
            constexpr bool EXACT = decltype(exactc)::value;
            const int64_t ld = EXACT ? N : n;
            const int64_t es = EXACT ? 1 : ilv;  // element stride
            Real* rowp = Ls + (COL ? (int64_t)q : (int64_t)q * ld) * es;
            sfor<0, N>([&](auto cc) {
              constexpr int c = decltype(cc)::value;
              const Real v = (failed || c > q) ? Real(0) : a[K][c];
              if (EXACT || c < n) rowp[(COL ? c * ld : c) * es] = v;
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
      });
      if (tx == 0) info[sys] = status;
    }
  } else {
    const bool failed = SOLVE ? given_failed : (status != 0 || nf != 0);
    bool xbad = false;
    if constexpr (NRHS == 1) {
      // ---- L^T x = y with the solver of the LU path: U = L^T, so lane c
      // writes L(c, q) into row q of the triangular store for every q <= c
      // (potrs has no status: non-finite entries of x are kept)
      xbad = upper_solve_store<Real, N, NRHS, T, !SOLVE>(
          sq, tx, (int)(g * T), live, failed, live ? sys : 0, n, nrhs, col, ilv, X,
          [&](Real* yt) {
            sfor<0, R>([&](auto Kc) {
              constexpr int K = decltype(Kc)::value;
              const int q = tx + K * T;
              if (q < N) yt[q] = y[K][0];
            });
          },
          [&](Real* ut) {
            sfor<0, R>([&](auto Kc) {
              constexpr int K = decltype(Kc)::value;
              const int c = tx + K * T;
              if (c < N) {
                Real* colp = ut + c;
                sfor<0, (K + 1) * T < N ? (K + 1) * T : N>([&](auto qc) {
                  constexpr int q = decltype(qc)::value;
                  if (q <= c) colp[utri_row<N>(q) - q] = a[K][q];
                });
              }
            });
          });
    } else {
      // ---- several right-hand sides: both triangular solves run after the
      // factorization in the column-class / row-phase layout of the LU
      // path (a class is P consecutive lanes, lane j0 * P + ph; y_k and x_k
      // reach their class by DPP), one division per column class per step,
      // L read from a row-packed lower triangle in LDS (row i at
      // i (i + 1) / 2).
      constexpr int NJ = NRHS < T ? NRHS : T;
      constexpr int P = T / NJ;
      constexpr int JR = NRHS / NJ;
      constexpr int QR = (N + P - 1) / P;
      const int j0 = tx / P;   // column class: P consecutive lanes
      const int ph = tx % P;
      const int gb = g * T;
      auto ltri = [](int i) { return i * (i + 1) / 2; };
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        if (q < N) {
          sfor<0, NRHS>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            sq[q * NRHS + r] = y[K][r];
          });
        }
      });
      wave_sync_lds();
      Real yv[QR][JR], xr[QR][JR];
      const Real* lrow[QR];
      sfor<0, QR>([&](auto mc) {
        constexpr int m = decltype(mc)::value;
        const int q = ph + P * m;
        const int qq = q < N ? q : N - 1;
        sfor<0, JR>([&](auto jc) {
          constexpr int jj = decltype(jc)::value;
          yv[m][jj] = sq[qq * NRHS + j0 + NJ * jj];
          xr[m][jj] = Real(0);
        });
        lrow[m] = sq + ltri(qq);   // L(q, c) at lrow[m][c], c <= q
      });
      wave_sync_lds();   // right-hand sides read before L overwrites them
      sfor<0, R>([&](auto Kc) {
        constexpr int K = decltype(Kc)::value;
        const int q = tx + K * T;
        if (q < N) {
          Real* rowp = sq + ltri(q);
          sfor<0, (K + 1) * T < N ? (K + 1) * T : N>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            if (c <= q) rowp[c] = a[K][c];
          });
        }
      });
      wave_sync_lds();
      // L y = b: y_k / L(k,k) on the lanes of phase k % P, then y_k leaves
      // the rows below it (rows at or above k are final and keep their value)
      // L(i, k) of this lane's rows (L(k,k) on the lanes of phase k % P)
      // read one step ahead, two register buffers, so that a step's LDS
      // reads overlap the step before; likewise L(k, q) below
      Real lb[2][QR];
      auto read_l = [&](auto kcc) {
        constexpr int k2 = decltype(kcc)::value;
        sfor<k2 / P, QR>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          lb[k2 % 2][m] = lrow[m][k2];   // L(i, k2), i = ph + P*m (meaningful for i >= k2)
        });
      };
      read_l(std::integral_constant<int, 0>{});
      sfor<0, N>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        constexpr int kp = k % P;
        constexpr int km = k / P;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (k + 1 < N) read_l(std::integral_constant<int, k + 1>{});
        const Real lkk = lb[k % 2][km];   // L(k,k) on the lanes of phase kp
        Real lik[QR];
        sfor<km, QR>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          const Real v = lb[k % 2][m];    // L(i,k), i = ph + P*m (meaningful for i > k)
          if constexpr (m == km)
            lik[m] = ph > kp ? v : Real(0);
          else
            lik[m] = v;
        });
        sfor<0, JR>([&](auto jc) {
          constexpr int jj = decltype(jc)::value;
          const Real yk = yv[km][jj] / lkk;
          yv[km][jj] = ph == kp ? yk : yv[km][jj];
          Real yb;
          if constexpr (P == 1)
            yb = yk;
          else if constexpr (P <= 16)
            yb = class_bcast<P, kp>(yk);   // lane kp of the class, by DPP
          else
            yb = lane_fetch_any(yk, gb + j0 * P + kp);
          sfor<km, QR>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            yv[m][jj] = fma_r(-lik[m], yb, yv[m][jj]);
          });
        });
      });
      // L^T x = y: x_k = y_k / L(k,k) on the lanes of phase k % P, removed
      // from the rows above with L(k, q) (rows at or below k are done)
      Real qb[2][QR + 1];   // [QR]: L(k,k)
      auto read_q = [&](auto icc) {
        constexpr int k2 = N - 1 - decltype(icc)::value;
        qb[decltype(icc)::value % 2][QR] = lrow[k2 / P][k2];
        sfor<0, k2 / P + 1>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          qb[decltype(icc)::value % 2][m] =
              sq[ltri(k2) + (ph + P * m < N ? ph + P * m : N - 1)];   // L(k2, q)
        });
      };
      read_q(std::integral_constant<int, 0>{});
      sfor<0, N>([&](auto ic) {
        constexpr int k = N - 1 - decltype(ic)::value;
        constexpr int kp = k % P;
        constexpr int km = k / P;
        constexpr int cur = decltype(ic)::value % 2;
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(ic)::value + 1 < N)
          read_q(std::integral_constant<int, decltype(ic)::value + 1>{});
        const Real lkk = qb[cur][QR];
        Real(&lkq)[QR + 1] = qb[cur];
        sfor<0, JR>([&](auto jc) {
          constexpr int jj = decltype(jc)::value;
          const Real x = yv[km][jj] / lkk;   // meaningful on the lanes of phase kp
          xr[km][jj] = ph == kp ? x : xr[km][jj];
          asm volatile("" : "+v"(xr[km][jj]));
          Real xb;
          if constexpr (P == 1)
            xb = x;
          else if constexpr (P <= 16)
            xb = class_bcast<P, kp>(x);   // lane kp of the class, by DPP
          else
            xb = lane_fetch_any(x, gb + j0 * P + kp);
          sfor<0, km + 1>([&](auto mc) {
            constexpr int m = decltype(mc)::value;
            yv[m][jj] = fma_r(-lkq[m], xb, yv[m][jj]);
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
      xbad = group_any<T>(bad, gb);
      if (live) {
        Real* Xs = X + sys_start(sys, ilv, (int64_t)n * nrhs);
        const bool zero = failed || (!SOLVE && xbad);
        sfor<0, QR>([&](auto mc) {
          constexpr int m = decltype(mc)::value;
          const int q = ph + P * m;
          sfor<0, JR>([&](auto jc) {
            constexpr int jj = decltype(jc)::value;
            const int r = j0 + NJ * jj;
            if (q < n && r < nrhs) {
              const Real v = zero ? Real(0) : xr[m][jj];
              if (col)
                Xs[((int64_t)r * n + q) * ilv] = v;
              else
                Xs[((int64_t)q * nrhs + r) * ilv] = v;
            }
          });
        });
      }
    }
    if (status == 0 && (nf != 0 || xbad)) status = -3;
    if constexpr (!SOLVE) {
      if (live && tx == 0) info[sys] = status;
    }
  }
}

}  // namespace tdls
