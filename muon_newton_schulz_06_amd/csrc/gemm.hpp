// MFMA products for the Gram Newton–Schulz step on gfx950 (CDNA4).
//
// One kernel template serves every dense contraction of the step
// (DMuon technical summary, gist.science Korean, §2.2):
//   * the SYRK G = X₀·X₀ᵀ,
//   * the symmetric Gram-space products A², B·Q, B·A, B·(P·A),
//   * the final product Q·X₀ (or X₀ᵀ·Q for tall matrices) with the weight
//     update fused into its epilogue.
// Every product has the form C[i][j] = Σ_k A[i][k]·B[j][k]: the Gram-space
// operands are symmetric (polynomials in G), so a row of one is also its
// column.
//
// Symmetric outputs (every Gram-space product is a product of commuting
// polynomials in G, hence symmetric) are computed on upper-triangle tiles
// only.  Diagonal tiles store the element of the upper half into both (i, j)
// and (j, i), so every stored iterate is exactly symmetric.
//
// Three kernels share the tile mapping and the epilogues:
//  * gemm256_kernel: 256×256 fp16 tiles, 8 waves, direct global→LDS loads
//    into a 4-slot ring.  Gram-space iterates are stored block-upper (only
//    the 256×256 blocks on or above the diagonal, except the last Q, which
//    the final product reads whole); a product reads an operand's k-tiles
//    left of its diagonal block from the transposed position, and the final
//    product reads X₀ᵀ as transposed panels of X₀ (X₀ is kept in one layout);
//  * gemm_kernel: 128×128 (fp32: also 64×64) tiles, 4 waves, register-staged
//    double buffering (fp32 groups with m > 256 and groups carrying fp32
//    state); full, mirrored operands and both layouts of X₀;
//  * gemm32_kernel: fp32 groups with m ≤ 256, 32×32 tiles whose contraction
//    is split over four waves, with gemm_kernel's operands and epilogues.
// All keep k-rows in LDS with a 16-byte-chunk XOR swizzle chosen for the
// 64-bank LDS (conflict-free ds_read_b128 fragment reads).
//
// This header holds the kernel templates; each gemm_*.hip translation unit
// instantiates the launches of one epilogue family (so they compile in
// parallel), and gemm_final.hip also holds the dispatcher launch_gemm.
#pragma once

#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace muon {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
// Native 16-byte vector (scalarisable, unlike HIP's uint4 class type).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

// Compile-time loop: f(std::integral_constant<int, P>) for P in [B, E).  The
// index reaches the body as a constant, so register arrays indexed by it are
// scalarised no matter how the optimiser orders unrolling.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

template <typename T> struct OpInfo;
template <> struct OpInfo<_Float16> { static constexpr int BK = 64; };
template <> struct OpInfo<float> { static constexpr int BK = 32; };

// Workgroups are dispatched round-robin over the 8 XCDs, each with its own
// L2.  Logical tiles are handed out in windows of 8 × C: inside a window
// XCD x runs a contiguous run of C logical tiles (which share operand row
// panels in its L2), and all XCDs work inside the same window (which keeps
// the working set of the shared last-level cache small).  The tail of the
// grid that does not fill a window keeps the identity mapping.  C = 2^cShift
// (32 unless the launch's tuning entry says otherwise).
__device__ __forceinline__ int xcd_window_remap(int b, int G, int cShift) {
  constexpr int X = 8;
  const int C = 1 << cShift, W = X * C;
  const int full = G / W;
  if (b >= full * W) return b;
  const int x = b % X, i = b / X;
  return (i >> cShift) * W + x * C + (i & (C - 1));
}

// Tile order inside one matrix: bands of `band` tile rows (4 unless the
// launch's tuning entry says otherwise), column by column inside a band, so
// consecutive tiles reuse the band's row panels of A and a short run of B
// panels.  sym: upper triangle only (ti ≤ tj).
constexpr int kBand = 4;
constexpr int kXcdShift = 5;

__device__ __forceinline__ void decode_tile(int t, int tilesM, int tilesN, bool sym, int band,
                                            int& ti, int& tj) {
  int r0 = 0;
  for (;;) {
    const int h = min(band, tilesM - r0);
    const int cnt = sym ? h * (h + 1) / 2 + h * (tilesN - r0 - h) : h * tilesN;
    if (t < cnt || r0 + h >= tilesM) break;
    t -= cnt;
    r0 += h;
  }
  const int h = min(band, tilesM - r0);
  if (sym) {
    int col = r0;
    for (;;) {
      const int cnt = min(col - r0 + 1, h);
      if (t < cnt) break;
      t -= cnt;
      ++col;
    }
    ti = r0 + t;
    tj = col;
  } else {
    tj = t / h;
    ti = r0 + (t - tj * h);
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

template <typename T> __device__ __forceinline__ T to_op(float v);
template <> __device__ __forceinline__ _Float16 to_op<_Float16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ float to_op<float>(float v) { return v; }

template <typename T>
__device__ __forceinline__ void store_mirror(T* base, int ldc, int i, int j, T v) {
  base[(int64_t)i * ldc + j] = v;
  if (i != j) base[(int64_t)j * ldc + i] = v;
}

// Everything the epilogue needs, resolved for this workgroup's matrix and
// copied out of the kernel arguments into locals (so the kernel-argument
// struct is only ever read, never addressed, and no private copy is made).
template <typename T>
struct EpiArgs {
  const T* inh;
  const float* in32;
  float* out32;
  T* outh;
  T* outhb;
  void* user;
  int64_t userLd;
  int ldc, mReal, nReal, writeIdentity, userDtype;
  float u, sOut, sOutB, sIn, p0, p1, p2, lrsc, decay;
};

// Epilogue for one accumulator element (i, j) of a dense result (register-
// staged kernel; symmetric results go through sym_value / mirror_rows).  EPI
// is a compile-time constant so each instantiation carries only its own code.
template <typename T, int EPI>
__device__ __forceinline__ void epilogue(const EpiArgs<T>& E, int i, int j, float acc) {
  static_assert(EPI == EPI_UPDATE || EPI == EPI_OUT, "dense epilogues only");
  if constexpr (EPI == EPI_UPDATE) {
    if (i >= E.mReal || j >= E.nReal) return;
    const int64_t e = (int64_t)i * E.userLd + j;
    const float o = E.u * acc;
    if (E.userDtype == 1) {
      uint16_t* w = (uint16_t*)E.user;
      w[e] = f32_to_bf16_rne(fmaf(-E.lrsc, o, bf16_to_f32(w[e]) * E.decay));
    } else {
      float* w = (float*)E.user;
      w[e] = fmaf(-E.lrsc, o, w[e] * E.decay);
    }
  } else if constexpr (EPI == EPI_OUT) {
    if (i >= E.mReal || j >= E.nReal) return;
    const int64_t e = (int64_t)i * E.userLd + j;
    const float v = E.u * acc;
    if (E.userDtype == 1) ((uint16_t*)E.user)[e] = f32_to_bf16_rne(v);
    else ((float*)E.user)[e] = v;
  }
}

// Symmetric results of the register-staged kernel: the element (i, j), i ≤ j,
// is stored at (i, j) only (and its fp32 copy, and the second copy's value at
// (i, j)); the returned stored value is staged so that the transposed
// position is written afterwards from LDS with coalesced rows (mirror_rows).
// The previous iterate's (i, j) element that the A² and a·Y + B·Y epilogues
// combine with the product (A for A², Y for a·Y + B·Y).
template <typename T>
__device__ __forceinline__ float sym_prev(const EpiArgs<T>& E, int i, int j) {
  const int64_t e = (int64_t)i * E.ldc + j;
  return E.in32 ? E.in32[e] : E.sIn * (float)E.inh[e];
}

template <typename T, int EPI>
__device__ __forceinline__ T sym_value_with(const EpiArgs<T>& E, int i, int j, float acc, float prev) {
  const int ldc = E.ldc;
  const int64_t e = (int64_t)i * ldc + j;
  if constexpr (EPI == EPI_SYRK) {
    (void)prev;
    const float g = E.u * acc;
    if (E.out32) E.out32[e] = g;
    const T v = to_op<T>(E.sOut * g);
    E.outh[e] = v;
    if (E.writeIdentity) E.outhb[e] = to_op<T>((i == j && i < E.mReal) ? E.sOutB : 0.f);
    return v;
  } else if constexpr (EPI == EPI_SQ) {
    const float a = prev;
    const float bb = E.p1 * a + E.p2 * (E.u * acc);
    const T bh = to_op<T>(E.sOut * bb);
    E.outh[e] = bh;
    if (E.outhb) {  // Q₁ = a·I + B₀ from the stored B₀ (as the 256-tile kernel does)
      const float q = (E.sOutB / E.sOut) * (float)bh + ((i == j && i < E.mReal) ? E.sOutB * E.p0 : 0.f);
      E.outhb[e] = to_op<T>(q);
    }
    return bh;
  } else {
    static_assert(EPI == EPI_AXPY, "symmetric epilogues only");
    const float y = E.p0 * prev + E.u * acc;
    if (E.out32) E.out32[e] = y;
    const T v = to_op<T>(E.sOut * y);
    E.outh[e] = v;
    return v;
  }
}

template <typename T, int EPI>
__device__ __forceinline__ T sym_value(const EpiArgs<T>& E, int i, int j, float acc) {
  return sym_value_with<T, EPI>(E, i, j, acc, EPI == EPI_SYRK ? 0.f : sym_prev(E, i, j));
}

// Staged symmetric tile: element (il, jl) at il·BN + (jl ^ (il/4)): the
// column reads of mirror_rows (32 or 16 lanes at rows il = 4a + e, one
// column) then fall in distinct banks, as do the staging writes (one row, 32
// consecutive columns), and the tile needs no padding.
template <int BN>
__device__ __forceinline__ int sym_stage_idx(int il, int jl) {
  return il * BN + (jl ^ ((il >> 2) & (BN - 1)));
}

// The transposed copy of a staged symmetric tile (ti, tj): block (tj, ti) of
// the result, row by row (each thread writes 4 consecutive elements of a
// row; the staged tile is read down its columns).  On a
// diagonal tile only the strictly lower elements are written, from the
// upper ones.  The second copy (first-step Q₁, or the zero-step identity)
// has no identity term off the diagonal, so its transposed values follow
// from the staged ones as at (i, j).
template <typename T, int EPI, int BM, int BN, int NT>
__device__ __forceinline__ void mirror_rows(const EpiArgs<T>& E, const T* st, int ti, int tj, int tid) {
  static_assert(BM == BN, "square tiles");
  constexpr int TPR = BM / 4;        // threads per row of the transposed block
  constexpr int RPP = NT / TPR;      // rows per pass
  const bool diag = ti == tj;
  const int il0 = (tid % TPR) * 4;
  const float qs = EPI == EPI_SQ ? E.sOutB / E.sOut : 0.f;
#pragma unroll 1
  for (int jl = tid / TPR; jl < BN; jl += RPP) {
    const int64_t row = (int64_t)(tj * BN + jl) * E.ldc + ti * BM + il0;
    T v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = st[sym_stage_idx<BN>(il0 + e, jl)];
    if (!diag || il0 + 3 < jl) {
      if constexpr (sizeof(T) == 4) {
        *(float4*)(E.outh + row) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        typedef T t4 __attribute__((ext_vector_type(4)));
        t4 h = {v[0], v[1], v[2], v[3]};
        *(t4*)(E.outh + row) = h;
      }
      if (EPI == EPI_SQ && E.outhb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) E.outhb[row + e] = to_op<T>(qs * (float)v[e] + 0.f);
      } else if (EPI == EPI_SYRK && E.writeIdentity) {
#pragma unroll
        for (int e = 0; e < 4; ++e) E.outhb[row + e] = to_op<T>(0.f);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (il0 + e >= jl) continue;
        E.outh[row + e] = v[e];
        if (EPI == EPI_SQ && E.outhb) E.outhb[row + e] = to_op<T>(qs * (float)v[e] + 0.f);
        else if (EPI == EPI_SYRK && E.writeIdentity) E.outhb[row + e] = to_op<T>(0.f);
      }
    }
  }
}

// Applies the epilogue to every accumulator element.  Template recursion
// makes (fi, fj, r) compile-time constants, so acc stays in registers.
template <typename T, int EPI, int FM, int FN, int IDX = 0>
__device__ __forceinline__ void epilogue_all(const EpiArgs<T>& E, int gi0, int gj0, int lh, int lr,
                                             const floatx16 (&acc)[FM][FN]) {
  if constexpr (IDX < FM * FN * 16) {
    constexpr int fi = IDX / (FN * 16), fj = (IDX / 16) % FN, r = IDX % 16;
    const int i = gi0 + fi * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
    const int j = gj0 + fj * 32 + lr;
    epilogue<T, EPI>(E, i, j, acc[fi][fj][r]);
    epilogue_all<T, EPI, FM, FN, IDX + 1>(E, gi0, gj0, lh, lr, acc);
  }
}

// Locates this workgroup's segment, matrix and tile.
struct TilePos {
  int seg, mat, ti, tj;
};

__device__ __forceinline__ TilePos locate(const GemmLaunch& L) {
  const int lid = xcd_window_remap(blockIdx.x, gridDim.x, L.xcdShift > 0 ? L.xcdShift : kXcdShift);
  TilePos p;
  p.seg = 0;
  while (p.seg + 1 < L.nseg && lid >= L.segStart[p.seg + 1]) ++p.seg;
  const GemmSeg& S = L.seg[p.seg];
  int t = lid - L.segStart[p.seg];
  p.mat = t / S.tilesPerMat;
  t -= p.mat * S.tilesPerMat;
  decode_tile(t, S.tilesM, S.tilesN, S.sym != 0, L.band > 0 ? L.band : kBand, p.ti, p.tj);
  return p;
}

template <typename T, int EPI>
__device__ __forceinline__ EpiArgs<T> make_epi(const GemmLaunch& L, const GemmSeg& S, int mat) {
  EpiArgs<T> E;
  E.ldc = S.ldc;
  E.mReal = S.mReal;
  E.nReal = S.nReal;
  E.writeIdentity = S.writeIdentity;
  E.u = S.u;
  E.sOut = S.sOut;
  E.sOutB = S.sOutB;
  E.sIn = S.sIn;
  E.p0 = S.p0;
  E.p1 = S.p1;
  E.p2 = S.p2;
  E.inh = S.inh ? (const T*)S.inh + mat * S.strideInh : nullptr;
  E.in32 = S.in32 ? S.in32 + mat * S.strideIn32 : nullptr;
  E.out32 = S.out32 ? S.out32 + mat * S.strideOut32 : nullptr;
  E.outh = S.outh ? (T*)S.outh + mat * S.strideOuth : nullptr;
  E.outhb = S.outhb ? (T*)S.outhb + mat * S.strideOuth : nullptr;
  E.user = nullptr;
  E.userLd = 0;
  E.lrsc = 0.f;
  E.decay = L.decay;
  E.userDtype = L.userDtype;
  if constexpr (EPI == EPI_UPDATE || EPI == EPI_OUT) {
    const int k = S.userBase + mat;
    E.user = L.user[k];
    E.userLd = L.userLd[k];
    E.lrsc = L.lrsc[k];
    if (S.rho) E.lrsc *= S.rho[mat];  // O = Q·X₀ = ρ·Q·(stored operand)
  }
  if constexpr (EPI == EPI_SYRK) {
    if (S.rho) E.u *= S.rho[mat] * S.rho[mat];  // G = ρ²·(stored operand)(stored operand)ᵀ
  }
  return E;
}

// ---------------------------------------------------------------------------
// Register-staged kernel: 128×128 tiles (fp16 and fp32 operands).

// Chunk swizzle for 128-byte rows (8 chunks): 16 consecutive rows read by 16
// lanes must cover the 64 banks once, so the swizzle is constant on row
// pairs (which already differ in bank half) and distinct across 8 pairs.
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }
template <typename T, int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__(64 * WM * WN) void gemm_kernel(const GemmLaunch L) {
  constexpr int NT = 64 * WM * WN;
  constexpr int BK = OpInfo<T>::BK;
  constexpr int CH = 8;                    // 16-byte chunks per 128-byte k-row
  constexpr int EPC = 16 / (int)sizeof(T); // elements per chunk
  constexpr int WTM = BM / WM, WTN = BN / WN;
  constexpr int FM = WTM / 32, FN = WTN / 32;
  constexpr int RPP = NT / CH;             // tile rows loaded per pass
  constexpr int LA = BM / RPP, LB = BN / RPP;
  static_assert(BK * sizeof(T) == 128, "k-row must be 128 bytes");
  static_assert(BM % RPP == 0 && BN % RPP == 0, "load passes");

  __shared__ u32x4 smem[2][(BM + BN) * CH];

  const TilePos tp = locate(L);
  const GemmSeg& S = L.seg[tp.seg];
  const int mat = tp.mat, ti = tp.ti, tj = tp.tj;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave - wm * WN;
  const int lr = lane & 31, lh = lane >> 5;

  const T* Ag = (const T*)S.A + mat * S.strideA + (int64_t)ti * BM * S.lda;
  const T* Bg = (const T*)S.B + mat * S.strideB + (int64_t)tj * BN * S.ldb;
  const int c = tid % CH, r0 = tid / CH;

  // Register staging of the next k-tile.  The lambdas capture locals only
  // (never the kernel-argument struct, whose address must not escape), and
  // the compile-time loop index keeps ra/rb in registers.
  u32x4 ra[LA], rb[LB];
  const int lda = S.lda, ldb = S.ldb;
  auto gload = [&ra, &rb, Ag, Bg, lda, ldb, c, r0](int kt) {
    const int k0 = kt * BK + c * EPC;
    static_for<0, LA>([&](auto p) {
      ra[p] = *(const u32x4*)(Ag + (int64_t)(r0 + p * RPP) * lda + k0);
    });
    static_for<0, LB>([&](auto p) {
      rb[p] = *(const u32x4*)(Bg + (int64_t)(r0 + p * RPP) * ldb + k0);
    });
  };
  auto lstore = [&ra, &rb, c, r0](u32x4* sm) {
    static_for<0, LA>([&](auto p) {
      const int r = r0 + p * RPP;
      sm[r * CH + (c ^ swz8(r))] = ra[p];
    });
    static_for<0, LB>([&](auto p) {
      const int r = r0 + p * RPP;
      sm[(BM + r) * CH + (c ^ swz8(r))] = rb[p];
    });
  };

  floatx16 acc[FM][FN];
#pragma unroll
  for (int fi = 0; fi < FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < FN; ++fj)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[fi][fj][e] = 0.f;

  const int KT = S.K / BK;
  gload(0);
  lstore(smem[0]);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const u32x4* sa = smem[buf];
    const u32x4* sb = smem[buf] + BM * CH;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int cc = 2 * kk + lh;
        half8 af[FM], bf[FN];
#pragma unroll
        for (int fi = 0; fi < FM; ++fi) {
          const int row = wm * WTM + fi * 32 + lr;
          u32x4 v = sa[row * CH + (cc ^ swz8(row))];
          af[fi] = __builtin_bit_cast(half8, v);
        }
#pragma unroll
        for (int fj = 0; fj < FN; ++fj) {
          const int row = wn * WTN + fj * 32 + lr;
          u32x4 v = sb[row * CH + (cc ^ swz8(row))];
          bf[fj] = __builtin_bit_cast(half8, v);
        }
#pragma unroll
        for (int fi = 0; fi < FM; ++fi)
#pragma unroll
          for (int fj = 0; fj < FN; ++fj)
            acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[fi], bf[fj], acc[fi][fj], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int c0 = 4 * kk + 2 * lh;
        float av[FM][8], bv[FN][8];
#pragma unroll
        for (int fi = 0; fi < FM; ++fi) {
          const int row = wm * WTM + fi * 32 + lr;
          u32x4 v0 = sa[row * CH + (c0 ^ swz8(row))];
          u32x4 v1 = sa[row * CH + ((c0 + 1) ^ swz8(row))];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            av[fi][e] = __uint_as_float(v0[e]);
            av[fi][4 + e] = __uint_as_float(v1[e]);
          }
        }
#pragma unroll
        for (int fj = 0; fj < FN; ++fj) {
          const int row = wn * WTN + fj * 32 + lr;
          u32x4 v0 = sb[row * CH + (c0 ^ swz8(row))];
          u32x4 v1 = sb[row * CH + ((c0 + 1) ^ swz8(row))];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bv[fj][e] = __uint_as_float(v0[e]);
            bv[fj][4 + e] = __uint_as_float(v1[e]);
          }
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
#pragma unroll
          for (int fi = 0; fi < FM; ++fi)
#pragma unroll
            for (int fj = 0; fj < FN; ++fj)
              acc[fi][fj] = __builtin_amdgcn_mfma_f32_32x32x2f32(av[fi][e], bv[fj][e], acc[fi][fj], 0, 0, 0);
      }
    }
    if (kt + 1 < KT) lstore(smem[buf ^ 1]);
    __syncthreads();
  }

  // 32×32 accumulator layout: lane l, register r holds
  // row 8·(r/4) + 4·(l/32) + r%4, column l%32 of the block.
  const EpiArgs<T> E = make_epi<T, EPI>(L, S, mat);
  const int gi0 = ti * BM + wm * WTM, gj0 = tj * BN + wn * WTN;
  if constexpr (EPI == EPI_SYRK || EPI == EPI_SQ || EPI == EPI_AXPY) {
    // Symmetric results: the tile's elements i ≤ j are stored directly and
    // staged in LDS (the ring is free: the loop ended with a barrier); the
    // transposed block is then written row by row from the staged tile, so
    // that copy is exactly the transpose of what was stored.
    static_assert(BM * BN * sizeof(T) <= sizeof(smem), "staged tile must fit");
    T* st = (T*)smem;
    static_for<0, FM * FN * 16>([&](auto ic) {
      constexpr int idx = decltype(ic)::value;
      constexpr int fi = idx / (FN * 16), fj = (idx / 16) % FN, r = idx % 16;
      const int il = wm * WTM + fi * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
      const int jl = wn * WTN + fj * 32 + lr;
      if (ti < tj || il <= jl)
        st[sym_stage_idx<BN>(il, jl)] = sym_value<T, EPI>(E, ti * BM + il, tj * BN + jl, acc[fi][fj][r]);
    });
    __syncthreads();
    mirror_rows<T, EPI, BM, BN, NT>(E, st, ti, tj, tid);
  } else {
    epilogue_all<T, EPI, FM, FN>(E, gi0, gj0, lh, lr, acc);
  }
}

// fp32 products of small matrices (m ≤ 256): 32×32 tiles with each k-tile's
// 32-wide contraction split over the workgroup's four waves, so a wave runs a
// quarter of the MFMAs of a 32×32 block (the register-staged kernel's wave
// runs all of them) and a single matrix's launch spreads over four times the
// compute units of a 64-tile launch.  Wave w takes the 16-byte k-chunk
// 4·(w/2) + 2·(lane/32) + w%2 of every 128-byte k-row: four 32×32×2 MFMAs
// per k-tile, lanes 0-31 and 32-63 supplying the two k of each, so the four
// waves cover k = 16·(w/2) + 8·(lane/32) + 4·(w%2) + 0..3 once.  The partial
// sums are added in wave order (0, 1, 2, 3), so a result does not depend on
// timing: wave w adds them for accumulator registers 4w .. 4w + 3 (rows
// 8w + 4·(lane/32) + 0..3 of the block, 32×32 accumulator layout as in the
// register-staged kernel) and applies that kernel's epilogue to those rows.
// The epilogue inputs of the Gram products (A or Y at the block's upper
// elements) are read before the main loop, hiding their latency; all
// threads write the mirrored rows.
template <int EPI>
__global__ __launch_bounds__(256) void gemm32_kernel(const GemmLaunch L) {
  using T = float;
  constexpr int BM = 32, BN = 32, BK = 32, CH = 8, NT = 256;
  constexpr bool kSym = EPI == EPI_SYRK || EPI == EPI_SQ || EPI == EPI_AXPY;
  constexpr bool kPrev = EPI == EPI_SQ || EPI == EPI_AXPY;
  __shared__ u32x4 smem[2][(BM + BN) * CH];  // double-buffered k-tile, 16 KiB
  __shared__ floatx16 part[4][64];           // partial sums of the four waves

  const TilePos tp = locate(L);
  const GemmSeg& S = L.seg[tp.seg];
  const int mat = tp.mat, ti = tp.ti, tj = tp.tj;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lr = lane & 31, lh = lane >> 5;

  // Thread t stages 16-byte chunk t % 8 of row t / 8 of the A and B tiles.
  const T* Ag = (const T*)S.A + mat * S.strideA + (int64_t)ti * BM * S.lda;
  const T* Bg = (const T*)S.B + mat * S.strideB + (int64_t)tj * BN * S.ldb;
  const int c = tid % CH, r = tid / CH;
  const T* ap = Ag + (int64_t)r * S.lda + c * 4;
  const T* bp = Bg + (int64_t)r * S.ldb + c * 4;
  const int so = r * CH + (c ^ swz8(r));

  const EpiArgs<T> E = make_epi<T, EPI>(L, S, mat);
  // this wave's output rows: il0 + q, q = 0..3 (registers 4w + q)
  const int il0 = 8 * wave + 4 * lh;
  float prev[4];
  if constexpr (kPrev) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      prev[q] = (ti < tj || il0 + q <= lr) ? sym_prev(E, ti * BM + il0 + q, tj * BN + lr) : 0.f;
  }

  floatx16 acc[1][1];
#pragma unroll
  for (int e = 0; e < 16; ++e) acc[0][0][e] = 0.f;

  const int KT = S.K / BK;
  u32x4 ra = *(const u32x4*)ap, rb = *(const u32x4*)bp;
  smem[0][so] = ra;
  smem[0][BM * CH + so] = rb;
  __syncthreads();
  const int ch = 4 * (wave >> 1) + 2 * lh + (wave & 1);
  const int ro = lr * CH + (ch ^ swz8(lr));
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) {
      ra = *(const u32x4*)(ap + (kt + 1) * BK);
      rb = *(const u32x4*)(bp + (kt + 1) * BK);
    }
    const u32x4 va = smem[buf][ro];
    const u32x4 vb = smem[buf][BM * CH + ro];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc[0][0] = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(va[e]), __uint_as_float(vb[e]),
                                                        acc[0][0], 0, 0, 0);
    if (kt + 1 < KT) {
      smem[buf ^ 1][so] = ra;
      smem[buf ^ 1][BM * CH + so] = rb;
    }
    __syncthreads();
  }
  part[wave][lane] = acc[0][0];
  __syncthreads();
  // 32×32 accumulator layout: lane l, register r holds
  // row 8·(r/4) + 4·(l/32) + r%4, column l%32 of the block.
  float v[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float* pp = (const float*)&part[0][lane] + 4 * wave + q;
    float x = pp[0];
#pragma unroll
    for (int w = 1; w < 4; ++w) x += pp[w * 64 * 16];
    v[q] = x;
  }

  if constexpr (kSym) {
    // The ring is free (the loop ended with a barrier): the block is staged
    // there for the mirrored rows, as in the register-staged kernel.
    T* st = (T*)smem;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int il = il0 + q;
      if (ti < tj || il <= lr)
        st[sym_stage_idx<BN>(il, lr)] =
            sym_value_with<T, EPI>(E, ti * BM + il, tj * BN + lr, v[q], kPrev ? prev[q] : 0.f);
    }
    __syncthreads();
    mirror_rows<T, EPI, BM, BN, NT>(E, st, ti, tj, tid);
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) epilogue<T, EPI>(E, ti * BM + il0 + q, tj * BN + lr, v[q]);
  }
}

// ---------------------------------------------------------------------------
// 256×256 fp16 kernel with direct global→LDS loads.
//
// 8 waves (2 × 4, each a 128×64 block of 16×16×32 MFMAs), k-tile 32, and a
// 4-stage LDS ring (4 × 32 KiB): a slot is refilled as soon as every wave
// has read it, so the loads of k-tiles kt+1 .. kt+3 are in flight while
// k-tile kt is multiplied, without registers for staging.  Each 16-byte load lands straight
// in LDS (global_load_lds_dwordx4: a wave writes 1 KiB contiguously); the
// bank swizzle is applied on the global side by choosing which chunk each
// lane fetches.  One barrier per k-tile.  Each ring slot is its own LDS
// object so that waits on outstanding loads into one slot do not serialise
// reads of another.
constexpr int kRowB = 64;                 // bytes per 32-element fp16 k-row
constexpr int kStageA = 256 * kRowB;      // 16 KiB
constexpr int kStage = 2 * kStageA;       // A + B tiles, 32 KiB

// Chunk swizzle for 64-byte rows: the physical 16-byte chunk of logical
// chunk c of row r is c ^ swz4(r).  A fragment read (lane l: row r0 + l%16,
// chunk l/16) takes 4 LDS cycles per ds_read_b128 without bank conflicts only
// for some swizzles, which were found by measurement on gfx950 (hardware
// counters SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE over all 256 swizzles
// that XOR two parities of the row's low four bits into the chunk index):
// 96 of them are conflict-free, 144 take 8 cycles (among them (r ^ r>>2) & 3,
// which separates any 16 consecutive rows across the 64 banks and would be
// conflict-free if the LDS served 16 consecutive lanes per cycle), 16 take
// 16.  The chosen one flips chunk bit 1 on rows with bit 2 set.
__device__ __forceinline__ int swz4(int r) { return (r >> 1) & 2; }

typedef __attribute__((address_space(3))) char* lds_ptr_t;

// One 16-byte global→LDS load per lane: lane l writes lds_base + 16·l.
// Issued through inline asm so that the compiler, which cannot tell the ring
// slots apart, does not add a wait for all outstanding loads before every
// LDS read; the kernel counts these loads itself (s_waitcnt vmcnt).
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds_base)
               : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(lds_ptr_t)p;
}

// acc += a·bᵀ with a 16×16×32 fp16 MFMA whose result register is its
// accumulator input.  Written as inline asm with a tied operand: the
// built-in lets the register allocator give each result a fresh register
// (a rotating accumulator), which at 128 accumulator registers per lane
// leaves too few for the operand pipeline.  The asm is opaque to the
// compiler's hazard tracking, so the kernel keeps the rules itself: the
// accumulators are written only by these MFMAs between the wait after
// their initialisation and the wait before the epilogue reads them
// (s_nop, below), and operand registers are only overwritten by LDS reads,
// which read-after-MFMA ordering does not constrain.
__device__ __forceinline__ void mfma16_acc(floatx4& acc, const half8& a, const half8& b) {
  asm volatile("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}

// ----- transposed operand panels ---------------------------------------------
// A block-upper symmetric operand (only blocks bi ≤ bj stored) supplies the
// k-tiles left of its diagonal block from the transposed position: rows k of
// the stored matrix, 256 values each.  Such a panel sits in the same 16 KiB
// of the ring slot as 32 k-rows of 512 bytes; 16-byte chunk c of row k is
// stored at c ^ tswz(k).  A transposed fragment read touches k-rows
// 8·g + 0..3 (or + 4..7) for the four 16-lane groups g, so the swizzle must
// separate both the rows inside a group (k bits 0, 1) and the groups (k bits
// 3, 4).  Measured on gfx950 (shader-clock timing of the kernel's transposed
// reads for all 65536 XOR maps from k bits 0, 1, 3, 4 to the chunk's low
// four bits): 4·(k & 3) alone runs 1.41× the fastest, this one 1.08×.
__device__ __forceinline__ int tswz(int k) {
  return (4 * (k & 3)) ^ (2 * ((k >> 3) & 1)) ^ ((k >> 4) & 1);
}

typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t* lds_s4_t;

__device__ __forceinline__ int tpan_off(int k, int i) {
  return k * 512 + (((i >> 3) ^ tswz(k)) << 4) + (i & 7) * 2;
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j supplies the
// address of 4 consecutive 16-bit values; lane i of the group receives
// value i % 4 of the chunks of lanes i/4, 4 + i/4, 8 + i/4, 12 + i/4.  With
// lane j pointing at (k0 + j/4, c0 + 4·(j%4)) of a k-major panel, lane i
// receives column c0 + i at rows k0 .. k0+3: four consecutive k of one row
// of the operand, which is the MFMA operand layout.
__device__ __forceinline__ half4 tr_read4(const char* pan, int k0, int c0, int j) {
  const short4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s4_t)(pan + tpan_off(k0 + (j >> 2), c0 + 4 * (j & 3))));
  return __builtin_bit_cast(half4, v);
}

// ----- staged epilogues of the 256-tile kernel ------------------------------

// Symmetric results: every value is written through LDS twice, once as the
// tile itself (rows of C) and once transposed (the mirrored tile), each time
// with 16-byte global stores covering 512 contiguous bytes per half-wave.
// LDS holds one 256×256 fp16 tile (128 KiB): row r = 512 bytes, 16-byte chunk
// c at c ^ (r & 31).
__device__ __forceinline__ int stage_off(int row, int col) {
  return row * 512 + ((((col >> 3) ^ (row & 31))) << 4) + (col & 7) * 2;
}

// Gram-space products fetch the previous iterate's block into this staged
// format during their last k-tiles (see issue_y): rows 0..191 into ring
// slots 0..2 as those are released, rows 192..255 one slot beyond the ring
// (fetched while slot 3 still holds the last k-tile).  kY selects that
// placement for every staged access of the tile.
template <bool kY>
__device__ __forceinline__ int soff(int row, int col) {
  return stage_off(row, col) + ((kY && row >= 192) ? kStage : 0);
}

// Accumulators of the 256-tile kernel: 16×16×32 MFMAs, block (fi, fj) of a
// wave's 128×64 region (lc = l%16, lg = l/16 below), operand roles swapped
// (B fragments as the MFMA's first operand): lane l, register r holds row
// 16·fi + lc, column 16·fj + 4·lg + r — four consecutive columns of one row,
// so every epilogue reads and writes a 16-bit tile with one 8-byte access
// per block.

// Symmetric layout: acc → LDS as rows of C (one 8-byte write per block).
template <bool kY, int FM, int FN>
__device__ __forceinline__ void stage_rows(char* lds, int wm, int wn, int lc, int lg,
                                           const floatx4 (&acc)[FM][FN]) {
  static_for<0, FM>([&](auto fi) {
    static_for<0, FN>([&](auto fj) {
      const int il = wm * 128 + fi * 16 + lc;
      const int jl = wn * 64 + fj * 16 + 4 * lg;
      half4 v;
      v[0] = (_Float16)acc[fi][fj][0];
      v[1] = (_Float16)acc[fi][fj][1];
      v[2] = (_Float16)acc[fi][fj][2];
      v[3] = (_Float16)acc[fi][fj][3];
      *(half4*)(lds + soff<kY>(il, jl)) = v;
    });
  });
}

// Second copy written from the same staged values (EPI_SQ, first step):
// dst2 = rs·v + dv on the diagonal of the matrix (global index < mReal).
struct SecondCopy {
  _Float16* dst2;
  float rs, dv;
  int mReal;
};

__device__ __forceinline__ u32x4 second_value(u32x4 v, const SecondCopy& sc, int grow, int gcol0) {
  half8 h = __builtin_bit_cast(half8, v);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float f = sc.rs * (float)h[e];
    if (gcol0 + e == grow && grow < sc.mReal) f += sc.dv;
    h[e] = (_Float16)f;
  }
  return __builtin_bit_cast(u32x4, h);
}

// Staged tile → global tile (tr, tc) of dst (and of sc.dst2 when kTwo):
// half-wave h of an instruction writes one 512-byte row.
template <bool kTwo, bool kY>
__device__ __forceinline__ void store_staged(_Float16* dst, int ldc, const char* lds, int tr,
                                             int tc, int tid, const SecondCopy& sc) {
#pragma unroll
  for (int it = 0; it < 16; ++it) {
    const int idx = it * 512 + tid;
    const int rl = idx >> 5, c = idx & 31;
    const u32x4 v = *(const u32x4*)(lds + soff<kY>(rl, c * 8));
    const int64_t off = ((int64_t)tr * 256 + rl) * ldc + (int64_t)tc * 256 + c * 8;
    *(u32x4*)(dst + off) = v;
    if constexpr (kTwo) *(u32x4*)(sc.dst2 + off) = second_value(v, sc, tr * 256 + rl, tc * 256 + c * 8);
  }
}

// Transposed LDS reads (ds_read_b64_tr_b16) of the staged tile, 16 output
// rows at a time: 16-lane group g of wave w handles the 16-byte column chunk
// q = 4w + g (c0 = 8q), lane i row r0 + i.  Two reads give a lane its
// chunk's 8 values from staged rows c0 .. c0 + 7 at column r0 + i (lane j of
// the group points at staged row c0 + j/4, then c0 + 4 + j/4, columns
// r0 + 4·(j%4) .. +3).
template <bool kY>
__device__ __forceinline__ half8 tr_chunk(const char* lds, int r0, int c0, int j) {
  const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s4_t)(lds + soff<kY>(c0 + (j >> 2), r0 + 4 * (j & 3))));
  const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s4_t)(lds + soff<kY>(c0 + 4 + (j >> 2), r0 + 4 * (j & 3))));
  return __builtin_bit_cast(half8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Diagonal tile: only its upper elements (c ≥ r) were computed.  Each lower
// element (r, c) of the staged tile is replaced by the staged (c, r), in
// place, which makes the tile exactly symmetric.  The reads touch upper
// positions only (a chunk's lower lanes discard what they read elsewhere),
// and a chunk that straddles the diagonal is written back with its upper
// values unchanged, so no read sees a value other than the one it needs.
// Which reads a wave needs depends on it and w only (uniform branches).
template <bool kY>
__device__ __forceinline__ void diag_fill(char* lds, int tid) {
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, c0 = 8 * (4 * w + (lane >> 4));
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
    const int r0 = 16 * it, r = r0 + i;
    // the wave's columns 32w .. 32w + 31 against rows r0 .. r0 + 15
    if (32 * w >= r0 + 15) continue;  // no lower element
    half8 t = tr_chunk<kY>(lds, r0, c0, i);
    if (32 * w + 31 >= r0) {  // some upper element: merge
      const half8 d = *(const half8*)(lds + soff<kY>(r, c0));
#pragma unroll
      for (int e = 0; e < 8; ++e) t[e] = c0 + e >= r ? d[e] : t[e];
    }
    if (c0 < r) *(half8*)(lds + soff<kY>(r, c0)) = t;
  }
}

// Staged tile → global tile (tr, tc), transposed: output element (r, c) is
// staged element (c, r) (the mirrored tile of an off-diagonal result).
template <bool kTwo, bool kY>
__device__ __forceinline__ void store_transposed(_Float16* dst, int ldc, const char* lds, int tr,
                                                 int tc, int tid, const SecondCopy& sc) {
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int i = lane & 15, c0 = 8 * (4 * w + (lane >> 4));
#pragma unroll 4
  for (int it = 0; it < 16; ++it) {
    const int r = 16 * it + i;
    const u32x4 v = __builtin_bit_cast(u32x4, tr_chunk<kY>(lds, 16 * it, c0, i));
    const int64_t off = ((int64_t)tr * 256 + r) * ldc + (int64_t)tc * 256 + c0;
    *(u32x4*)(dst + off) = v;
    if constexpr (kTwo) *(u32x4*)(sc.dst2 + off) = second_value(v, sc, tr * 256 + r, tc * 256 + c0);
  }
}

// Writes the symmetric result held in acc (already scaled for storage) to
// dst: the tile (ti, tj) from its rows, the tile (tj, ti) from its columns.
// kY (Gram-space products): the rows are already in LDS, in the Y placement
// (written there while the previous iterate was added).
template <int FM, int FN, bool kTwo, bool kY>
__device__ __forceinline__ void write_symmetric(_Float16* dst, int ldc, char* lds, int ti, int tj,
                                                int wm, int wn, int lc, int lg, int tid,
                                                const floatx4 (&acc)[FM][FN],
                                                const SecondCopy& sc, bool mirror) {
  if constexpr (!kY) stage_rows<kY, FM, FN>(lds, wm, wn, lc, lg, acc);
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  // A diagonal tile is completed in LDS from its upper elements and written
  // whole; block-upper output stores an off-diagonal tile alone, mirrored
  // output its transpose as well (the kernel ends after the stores).
  if (ti == tj) {
    diag_fill<kY>(lds, tid);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    store_staged<kTwo, kY>(dst, ldc, lds, ti, tj, tid, sc);
    return;
  }
  store_staged<kTwo, kY>(dst, ldc, lds, ti, tj, tid, sc);
  if (mirror) store_transposed<kTwo, kY>(dst, ldc, lds, tj, ti, tid, sc);
}

// Caller-facing outputs (weight update or plain output).  The accumulators
// have the same layout as the symmetric products' (lane: one row, four
// consecutive columns per 16×16 block).  A bf16 tile wholly inside the matrix
// with 16-byte aligned rows (dense_fast_ok) is staged in LDS and written with
// the symmetric results' 16-byte row stores; for the weight update the
// tile's current weights are fetched into that staging during the last
// k-tiles (as the Gram products fetch Y) and updated in place.  Any other
// tile (fp32 caller tensors, edge tiles, unaligned rows) is written from the
// registers, element by element where needed.
__device__ __forceinline__ bool dense_fast_ok(const EpiArgs<_Float16>& E, int ti, int tj) {
  return E.userDtype == 1 && (E.userLd % 8 == 0) && (((uintptr_t)E.user & 15) == 0) &&
         (int64_t)ti * 256 + 256 <= E.mReal && (int64_t)tj * 256 + 256 <= E.nReal;
}

// Staged fast path: row il, columns jl .. jl + 3 of the tile, in the staged
// layout soff<kPre> (kPre: the weights were fetched there).
template <int EPI, bool kPre, int FM, int FN>
__device__ __forceinline__ void dense_stage(const EpiArgs<_Float16>& E, char* lds, int wm, int wn,
                                            int lc, int lg, const floatx4 (&acc)[FM][FN]) {
  static_for<0, FM>([&](auto fi) {
    static_for<0, FN>([&](auto fj) {
      char* p = lds + soff<kPre>(wm * 128 + fi * 16 + lc, wn * 64 + fj * 16 + 4 * lg);
      uint32_t o[2];
      if constexpr (EPI == EPI_UPDATE) {
        const uint2 wv = *(const uint2*)p;
        const uint32_t in[2] = {wv.x, wv.y};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float a0 = fmaf(-E.lrsc, E.u * acc[fi][fj][2 * h], bf16_to_f32((uint16_t)(in[h] & 0xffffu)) * E.decay);
          const float a1 = fmaf(-E.lrsc, E.u * acc[fi][fj][2 * h + 1], bf16_to_f32((uint16_t)(in[h] >> 16)) * E.decay);
          o[h] = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
        }
      } else {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          o[h] = (uint32_t)f32_to_bf16_rne(E.u * acc[fi][fj][2 * h]) |
                 ((uint32_t)f32_to_bf16_rne(E.u * acc[fi][fj][2 * h + 1]) << 16);
      }
      *(uint2*)p = make_uint2(o[0], o[1]);
    });
  });
}

// Register path: each lane writes its four consecutive columns of a row per
// block, as one 8- or 16-byte access where the row allows, else by element.
template <int EPI, int FM, int FN>
__device__ __forceinline__ void dense_direct(const EpiArgs<_Float16>& E, int ti, int tj, int wm,
                                             int wn, int lc, int lg, const floatx4 (&acc)[FM][FN]) {
  const bool vec = (E.userLd % 4 == 0) && (((uintptr_t)E.user & 15) == 0);
  static_for<0, FM>([&](auto fi) {
    const int64_t i = (int64_t)ti * 256 + wm * 128 + fi * 16 + lc;
    static_for<0, FN>([&](auto fj) {
      const int64_t j = (int64_t)tj * 256 + wn * 64 + fj * 16 + 4 * lg;
      if (i >= E.mReal || j >= E.nReal) return;
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = E.u * acc[fi][fj][e];
      const int64_t base = i * E.userLd + j;
      const bool full = vec && (j + 3 < E.nReal);
      if constexpr (EPI == EPI_UPDATE) {
        if (E.userDtype == 1) {
          uint16_t* w = (uint16_t*)E.user + base;
          if (full) {
            const uint2 wv = *(const uint2*)w;
            const uint32_t in[2] = {wv.x, wv.y};
            uint32_t o[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float a0 = fmaf(-E.lrsc, v[2 * h], bf16_to_f32((uint16_t)(in[h] & 0xffffu)) * E.decay);
              const float a1 = fmaf(-E.lrsc, v[2 * h + 1], bf16_to_f32((uint16_t)(in[h] >> 16)) * E.decay);
              o[h] = (uint32_t)f32_to_bf16_rne(a0) | ((uint32_t)f32_to_bf16_rne(a1) << 16);
            }
            *(uint2*)w = make_uint2(o[0], o[1]);
          } else {
            for (int e = 0; e < 4 && j + e < E.nReal; ++e)
              w[e] = f32_to_bf16_rne(fmaf(-E.lrsc, v[e], bf16_to_f32(w[e]) * E.decay));
          }
        } else {
          float* w = (float*)E.user + base;
          if (full) {
            float4 wv = *(const float4*)w;
            wv.x = fmaf(-E.lrsc, v[0], wv.x * E.decay);
            wv.y = fmaf(-E.lrsc, v[1], wv.y * E.decay);
            wv.z = fmaf(-E.lrsc, v[2], wv.z * E.decay);
            wv.w = fmaf(-E.lrsc, v[3], wv.w * E.decay);
            *(float4*)w = wv;
          } else {
            for (int e = 0; e < 4 && j + e < E.nReal; ++e) w[e] = fmaf(-E.lrsc, v[e], w[e] * E.decay);
          }
        }
      } else {  // EPI_OUT
        if (E.userDtype == 1) {
          uint16_t* o = (uint16_t*)E.user + base;
          if (full) {
            const uint32_t p0 = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
            const uint32_t p1 = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
            *(uint2*)o = make_uint2(p0, p1);
          } else {
            for (int e = 0; e < 4 && j + e < E.nReal; ++e) o[e] = f32_to_bf16_rne(v[e]);
          }
        } else {
          float* o = (float*)E.user + base;
          if (full) *(float4*)o = make_float4(v[0], v[1], v[2], v[3]);
          else
            for (int e = 0; e < 4 && j + e < E.nReal; ++e) o[e] = v[e];
        }
      }
    });
  });
}

// TR (dense products only): 0 both operands direct, 1 A read transposed,
// 2 B read transposed, for every k-tile.
template <int EPI, int TR = 0>
__global__ __launch_bounds__(512) void gemm256_kernel(const GemmLaunch L) {
  using T = _Float16;
  constexpr int BM = 256, BN = 256, BK = 32, WN = 4;
  constexpr int WTM = 128, WTN = 64, FM = 8, FN = 4;  // 16×16 blocks per wave
  constexpr bool kSym = EPI == EPI_SYRK || EPI == EPI_SQ || EPI == EPI_AXPY;
  // Gram-space products: block-upper operands, and the previous iterate Y
  // (their B operand) added in the epilogue.
  constexpr bool kGram = EPI == EPI_SQ || EPI == EPI_AXPY;
  // 4-slot ring for the main loop, plus one slot for the last quarter of
  // the Y block (Gram products) or of the weights (update); reused by the
  // staged epilogues (one 256×256 16-bit tile).
  constexpr int kLds = (kGram || EPI == EPI_UPDATE) ? 5 * kStage : 4 * kStage;
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  static_assert(4 * kStage >= 256 * 512, "a staged symmetric tile must fit");
  char* const st0 = lds;
  char* const st1 = lds + kStage;
  char* const st2 = lds + 2 * kStage;
  char* const st3 = lds + 3 * kStage;

  const TilePos tp = locate(L);
  const GemmSeg& S = L.seg[tp.seg];
  const int mat = tp.mat, ti = tp.ti, tj = tp.tj;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // A diagonal tile of a Gram-space product needs only its 16×16 blocks on or
  // above the diagonal: the epilogue writes the upper elements and takes the
  // lower ones from the transposed upper half.  Each wave skips the MFMAs of
  // the quarters of its 128×64 region (two block rows) that lie wholly below
  // the diagonal: wave (wm, wn) runs 2, 4, 4, 4 quarters in row half 0
  // (wn = 0..3) and 0, 0, 2, 4 in row half 1.  The waves of a workgroup are
  // dealt to the CU's four SIMDs in turn (waves w and w + 4 share one), so on
  // diagonal tiles row half 0 takes the column strips in reverse order: each
  // SIMD then has 4 or 6 of its 8 quarters to run, not up to 8.  (The SYRK,
  // whose contraction is up to 5× longer, ran 3% slower with the per-quarter
  // branches than the diagonal tiles saved, so it computes its tiles in full.)
  const bool diagT = kGram && ti == tj;
  const int wm = wave / WN;
  const int wn = (diagT && wm == 0) ? WN - 1 - wave : wave - wm * WN;
  int runMask = 0xf;  // bit q: quarter q (block rows 2q, 2q + 1) has work
  if (diagT)
    for (int q = 0; q < 4; ++q)
      if (wm * 8 + 2 * q > wn * 4 + 3) runMask &= ~(1 << q);
  runMask = __builtin_amdgcn_readfirstlane(runMask);
  const int lc = lane & 15, lg = lane >> 4;

  const T* Ag = (const T*)S.A + mat * S.strideA + (int64_t)ti * BM * S.lda;
  const T* Bg = (const T*)S.B + mat * S.strideB + (int64_t)tj * BN * S.ldb;

  // wave w fills rows [32w, 32w + 32) of the A and of the B tile, 16 rows
  // (1 KiB) per instruction; lane l writes row 16p + l/4, physical chunk l%4
  // and therefore fetches logical chunk (l%4) ^ swz4(row).
  const int lrow = lane >> 2, lpc = lane & 3;
  const T* gA[2];
  const T* gB[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = wave * 32 + p * 16 + lrow;
    const int lc = lpc ^ swz4(r);
    gA[p] = Ag + (int64_t)r * S.lda + lc * 8;
    gB[p] = Bg + (int64_t)r * S.ldb + lc * 8;
  }
  const int dstA = wave * 32 * kRowB;
  // Block-upper operands: k-tiles kt < dA (dB) of A (B) come from the
  // transposed position, k-rows kt·32 .. kt·32+31 of the stored matrix at
  // columns ti·256 (tj·256) onwards.  Wave w fills k-rows 4w .. 4w+3, two
  // rows (1 KiB) per instruction, so the instruction count per k-tile (and
  // hence every vmcnt below) is the same in both layouts.
  // The final product reads X₀ transposed for every k-tile instead (transA
  // or transB).  A lane's offset inside a 32-row transposed panel,
  // r·ld + column, fits 32 bits for every supported shape (ld < 2^25).
  const int KT = S.K / BK;
  const int dA = kGram ? (S.upperA ? ti * (BM / BK) : 0) : (TR == 1 ? KT : 0);
  const int dB = kGram ? (S.upperB ? tj * (BN / BK) : 0) : (TR == 2 ? KT : 0);
  const T* const baseAT = (const T*)S.A + mat * S.strideA + ti * BM;
  const T* const baseBT = (const T*)S.B + mat * S.strideB + tj * BN;
  // Only one leading dimension is ever read transposed in a launch (Gram
  // products have lda = ldb; the final product transposes one operand), so
  // a lane's two offsets are computed once.
  const int ldTA = S.lda, ldTB = kGram ? S.lda : S.ldb;
  const int ldT = TR == 2 ? ldTB : ldTA;  // the one transposed operand's (Gram: lda = ldb)
  int offT[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int r = wave * 4 + 2 * p + (lane >> 5);
    offT[p] = r * ldT + (((lane & 31) ^ tswz(r)) << 3);
  }
  auto tr_off = [offT](int p, int ld) __attribute__((always_inline)) {
    (void)ld;
    return offT[p];
  };
  const int dstT = wave * 4 * 512;
  auto issue = [&gA, &gB, tr_off, baseAT, baseBT, ldTA, ldTB, dstA, dstT, dA, dB](char* st, int kt) __attribute__((always_inline)) {
    const int k0 = kt * BK;
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(st));
    if (kt < dA) {
      const T* b = baseAT + (int64_t)k0 * ldTA;
#pragma unroll
      for (int p = 0; p < 2; ++p)
        dma16(b + tr_off(p, ldTA), __builtin_amdgcn_readfirstlane(sbase + dstT + p * 1024));
    } else {
#pragma unroll
      for (int p = 0; p < 2; ++p) dma16(gA[p] + k0, __builtin_amdgcn_readfirstlane(sbase + dstA + p * 16 * kRowB));
    }
    if (kt < dB) {
      const T* b = baseBT + (int64_t)k0 * ldTB;
#pragma unroll
      for (int p = 0; p < 2; ++p)
        dma16(b + tr_off(p, ldTB), __builtin_amdgcn_readfirstlane(sbase + kStageA + dstT + p * 1024));
    } else {
#pragma unroll
      for (int p = 0; p < 2; ++p) dma16(gB[p] + k0, __builtin_amdgcn_readfirstlane(sbase + kStageA + dstA + p * 16 * kRowB));
    }
  };

  // Load j (0, 1: the A tile, 2, 3: the B tile) of issue(st, kt), the
  // layout chosen by a select on the uniform ta / tb (kt < dA, kt < dB), the
  // address formed where the load is issued.
  auto refill_one = [&gA, &gB, offT, baseAT, baseBT, ldTA, ldTB, dstA, dstT](uint32_t sbase, int k0, bool ta, bool tb, auto jc) __attribute__((always_inline)) {
    constexpr int j = decltype(jc)::value;
    constexpr int p = j & 1;
    if constexpr (j < 2) {
      const T* g = ta ? baseAT + (int64_t)k0 * ldTA + offT[p] : gA[p] + k0;
      dma16(g, __builtin_amdgcn_readfirstlane(sbase + (ta ? dstT + p * 1024 : dstA + p * 16 * kRowB)));
    } else {
      const T* g = tb ? baseBT + (int64_t)k0 * ldTB + offT[p] : gB[p] + k0;
      dma16(g, __builtin_amdgcn_readfirstlane(sbase + kStageA + (tb ? dstT + p * 1024 : dstA + p * 16 * kRowB)));
    }
  };

  floatx4 acc[FM][FN];
#pragma unroll
  for (int fi = 0; fi < FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < FN; ++fj)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[fi][fj][e] = 0.f;
  // The zeros are written (in order) before the wait that precedes the
  // first MFMA reading them.
#pragma unroll
  for (int fi = 0; fi < FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < FN; ++fj) asm volatile("" : "+v"(acc[fi][fj]));
  asm volatile("s_nop 7");

  // The Gram products' epilogue adds the previous iterate Y (the B operand,
  // block-upper) at the output positions: block (ti, tj) of Y, stored since
  // ti ≤ tj.  It is fetched into LDS during the last four k-tiles, in the
  // staged format of the output tile (row r at r·512, 16-byte chunk c at
  // c ^ (r & 31); see soff), a quarter of 64 rows (32 KiB, four loads per
  // wave, like a k-tile) at a time: rows 0..63 and 192..255 (the latter
  // beyond the ring) once k-tile KT − 4 has released slot 0, then rows
  // 64..127 and 128..191 into slots 1 and 2 as k-tiles KT − 3 and KT − 2
  // release them.  Wave w fetches
  // rows 8w .. 8w + 7 of a quarter, two 512-byte rows per instruction; a
  // lane fetches the logical chunk that lands at its physical position.
  [[maybe_unused]] int offY[4];
  [[maybe_unused]] const T* ybase = nullptr;
  if constexpr (kGram) {
    ybase = (const T*)S.inh + mat * S.strideInh + (int64_t)ti * BM * S.ldc + (int64_t)tj * BN;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = wave * 8 + 2 * p + (lane >> 5);
      offY[p] = r * S.ldc + (((lane & 31) ^ (r & 31)) << 3);
    }
  }
  auto issue_y = [&](int q) __attribute__((always_inline)) {
    char* dst = q == 3 ? lds + 4 * kStage : lds + q * kStage;
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(dst));
    const T* b = ybase + (int64_t)(64 * q) * S.ldc;
#pragma unroll
    for (int p = 0; p < 4; ++p)
      dma16(b + offY[p], __builtin_amdgcn_readfirstlane(sbase + (wave * 8 + 2 * p) * 512));
  };

  // Operand fragments of a 16×16×32 MFMA: lane l holds row row0 + l%16 at
  // k = 8·(l/16) .. +7 of the k-tile, i.e. 16-byte chunk l/16 of the row
  // (row0 is a multiple of 16, so the swizzle depends on l%16 only).  A
  // transposed panel gives the same fragment from two transposed reads.
  const int sw = swz4(lc);
  auto frag_n = [lc, lg, sw](const char* pan, int row0) __attribute__((always_inline)) {
    return *(const half8*)(pan + (row0 + lc) * kRowB + ((lg ^ sw) << 4));
  };
  auto frag_t = [lc, lg](const char* pan, int row0) __attribute__((always_inline)) {
    const half4 lo = tr_read4(pan, 8 * lg, row0, lc);
    const half4 hi = tr_read4(pan, 8 * lg + 4, row0, lc);
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };

  // A k-tile is one 32-wide k-step: 8 × 4 MFMAs per wave, in four
  // quarters by rows (A blocks 2q, 2q+1).  Registers: the B fragments of the
  // current and of the next k-tile (alternating by k-tile parity) and two
  // sets of A-quarter fragments; the fragments of the next quarter are read
  // from LDS while the MFMAs of the current one run, across k-tile
  // boundaries too.  The layout (direct or transposed panel) of each
  // operand is a template argument wherever it is known at compile time.
  half8 fb0[FN], fb1[FN], fax[2], fay[2];
  auto bset = [&](auto pc) -> half8 (&)[FN] {
    if constexpr (decltype(pc)::value) return fb1;
    else return fb0;
  };
  auto load_a = [&](half8 (&fa)[2], const char* st, int q, auto tac) __attribute__((always_inline)) {
#pragma unroll
    for (int f = 0; f < 2; ++f) {
      const int row0 = wm * WTM + (2 * q + f) * 16;
      fa[f] = decltype(tac)::value ? frag_t(st, row0) : frag_n(st, row0);
    }
  };
  auto load_b = [&](half8 (&fb)[FN], const char* st, auto tbc) __attribute__((always_inline)) {
#pragma unroll
    for (int fj = 0; fj < FN; ++fj) {
      const int row0 = wn * WTN + fj * 16;
      fb[fj] = decltype(tbc)::value ? frag_t(st + kStageA, row0) : frag_n(st + kStageA, row0);
    }
  };
  // The operand roles are swapped (B fragments first), which transposes the
  // accumulator layout: a lane holds four consecutive columns of one row.
  auto mma = [&acc, runMask](const half8 (&fa)[2], const half8 (&fb)[FN], auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    if constexpr (kGram) {
      if (!(runMask & (1 << q))) return;
    }
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int fj = 0; fj < FN; ++fj) {
        mfma16_acc(acc[2 * q + f][fj], fb[fj], fa[f]);
      }
  };
  // Quarter q's MFMAs with the refill of slot st (k-tile kt) spread over
  // them: one load after each of the first FN MFMAs, so the matrix pipe
  // keeps issuing while the loads go out (both are asm volatile, so their
  // order is the source order).  A skipped quarter issues the loads alone.
  static_assert(FN == 4, "four refill loads per k-tile and wave");
  auto mma_refill = [&](const half8 (&fa)[2], const half8 (&fb)[FN], auto qc, char* st, int kt) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(st));
    const int k0 = kt * BK;
    const bool ta = kt < dA, tb = kt < dB;
    if constexpr (kGram) {
      if (!(runMask & (1 << q))) {
        issue(st, kt);
        return;
      }
    }
    static_for<0, 2>([&](auto fc) {
      constexpr int f = decltype(fc)::value;
      static_for<0, FN>([&](auto jc) {
        constexpr int fj = decltype(jc)::value;
        mfma16_acc(acc[2 * q + f][fj], fb[fj], fa[f]);
        if constexpr (f == 0) refill_one(sbase, k0, ta, tb, std::integral_constant<int, fj>{});
      });
    });
  };
  constexpr auto kQ0 = std::integral_constant<int, 0>{};
  constexpr auto kQ1 = std::integral_constant<int, 1>{};
  constexpr auto kQ2 = std::integral_constant<int, 2>{};
  constexpr auto kQ3 = std::integral_constant<int, 3>{};

  // Weight update on the staged path: the tile's bf16 weights are fetched
  // into the epilogue's staging during the last four k-tiles, a quarter of
  // 64 rows at a time into the slots the Gram products' Y block uses (same
  // placement, same wave/lane assignment, so the same vmcnt counts hold).
  [[maybe_unused]] const uint16_t* wbase = nullptr;
  [[maybe_unused]] int64_t wld = 0;
  bool pref = false;
  if constexpr (EPI == EPI_UPDATE) {
    const EpiArgs<T> Ew = make_epi<T, EPI>(L, S, mat);
    pref = dense_fast_ok(Ew, ti, tj);
    wbase = (const uint16_t*)Ew.user + (int64_t)ti * BM * Ew.userLd + (int64_t)tj * BN;
    wld = Ew.userLd;
  }
  auto issue_w = [&](int q) __attribute__((always_inline)) {
    char* dst = q == 3 ? lds + 4 * kStage : lds + q * kStage;
    const uint32_t sbase = __builtin_amdgcn_readfirstlane(lds_addr(dst));
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int r = wave * 8 + 2 * p + (lane >> 5);
      const uint16_t* g = wbase + (int64_t)(64 * q + r) * wld + (((lane & 31) ^ (r & 31)) << 3);
      dma16(g, __builtin_amdgcn_readfirstlane(sbase + (wave * 8 + 2 * p) * 512));
    }
  };

  // One k-tile k (ring slot cur = k mod 4; nxt holds k + 1; pc its parity,
  // selecting the B registers):
  //   quarters 0-2: read the next A quarter of k while the MFMAs of the
  //   current one run — the last reads of slot cur;
  //   wait until k-tile k + 1 has landed for every wave (each k-tile is four
  //   loads per wave; k + 2 and k + 3 stay in flight) and until the wave's
  //   own LDS reads have completed — after the barrier no wave reads slot
  //   cur again, so it is refilled at once with k + 4 (or the tail loads):
  //   three k-tiles are in flight while one is multiplied;
  //   quarter 3: read B and A quarter 0 of k + 1 (same phase) while its
  //   MFMAs run.
  // The barrier is a bare s_barrier: a __syncthreads() would also wait for
  // every outstanding load.  The "memory" clobber keeps the compiler from
  // moving LDS accesses across it; sched_barrier keeps the MFMAs in place.
  auto first_half = [&](const char* cur, auto pc, auto tac) __attribute__((always_inline)) {
    half8 (&fb)[FN] = bset(pc);
    load_a(fay, cur, 1, tac);
    __builtin_amdgcn_sched_barrier(0);
    mma(fax, fb, kQ0);
    __builtin_amdgcn_sched_barrier(0);
    load_a(fax, cur, 2, tac);
    __builtin_amdgcn_sched_barrier(0);
    mma(fay, fb, kQ1);
    __builtin_amdgcn_sched_barrier(0);
    load_a(fay, cur, 3, tac);
    __builtin_amdgcn_sched_barrier(0);
    mma(fax, fb, kQ2);
    __builtin_amdgcn_sched_barrier(0);
  };
  auto head = [&](const char* st, auto pc, auto tac, auto tbc) __attribute__((always_inline)) {
    load_b(bset(pc), st, tbc);
    load_a(fax, st, 0, tac);
  };
  auto second_half = [&](const char* nxt, auto pc, auto tac, auto tbc) __attribute__((always_inline)) {
    head(nxt, std::bool_constant<!decltype(pc)::value>{}, tac, tbc);
    __builtin_amdgcn_sched_barrier(0);
    mma(fay, bset(pc), kQ3);
  };
  // Steps with k + 1 in the same phase and at least four k-tiles after k.
  auto plain = [&](char* cur, const char* nxt, int k, auto pc, auto tac, auto tbc) __attribute__((always_inline)) {
    first_half(cur, pc, tac);
    asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (kGram) {
      issue(cur, k + 4);
      second_half(nxt, pc, tac, tbc);
    } else {
      head(nxt, std::bool_constant<!decltype(pc)::value>{}, tac, tbc);
      __builtin_amdgcn_sched_barrier(0);
      mma_refill(fay, bset(pc), kQ3, cur, k + 4);
    }
  };
  // Any step: phase ends and the last k-tiles (tail loads, shorter waits).
  // Loads younger than k-tile k + 1 when step k waits for it: k + 2 and
  // k + 3 while they exist; for the Gram products the Y quarters 0 and 3
  // (issued in step KT − 4) and 1 (step KT − 3); the weight update's
  // quarters likewise.
  auto step = [&](char* cur, const char* nxt, int k, int k1, auto pc, auto tac,
                  auto tbc) __attribute__((always_inline)) {
    first_half(cur, pc, tac);
    const int r = KT - 1 - k;  // k-tiles after this one
    if (r >= 3) {
      asm volatile("s_waitcnt vmcnt(8) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else if (kGram && r >= 1) {
      asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else if (pref && r >= 1) {
      asm volatile("s_waitcnt vmcnt(12) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    } else if (r == 2) {
      asm volatile("s_waitcnt vmcnt(4)\n\ts_barrier" ::: "memory");
    } else if (r == 1) {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (r >= 4) issue(cur, k + 4);
    if constexpr (kGram) {
      // k-tiles KT − 4 .. KT − 2 sit in slots 0..2 (KT is a multiple of 8)
      if (r == 3) {
        issue_y(0);
        issue_y(3);
      } else if (r == 2 || r == 1) {
        issue_y(3 - r);
      }
    }
    if constexpr (EPI == EPI_UPDATE) {
      if (pref) {
        if (r == 3) {
          issue_w(0);
          issue_w(3);
        } else if (r == 2 || r == 1) {
          issue_w(3 - r);
        }
      }
    }
    if (k + 1 < k1) head(nxt, std::bool_constant<!decltype(pc)::value>{}, tac, tbc);
    __builtin_amdgcn_sched_barrier(0);
    mma(fay, bset(pc), kQ3);
  };
  constexpr auto kEven = std::false_type{};
  constexpr auto kOdd = std::true_type{};
  // k-tiles in three phases of fixed operand layouts: [0, dA) both
  // transposed, [dA, dB) B transposed, [dB, KT) both direct (dA ≤ dB since
  // ti ≤ tj).  Phase lengths are multiples of 8 (KT, dA, dB are), so every
  // phase starts on ring slot 0 with an even k-tile and runs in whole groups
  // of four k-tiles.  The first fragments of a phase are read at its start
  // (the step before it does not know the layout).
  auto phase = [&](int k0, int k1, auto tac, auto tbc) __attribute__((always_inline)) {
    if (k0 < k1) head(st0, kEven, tac, tbc);
    int kt = k0;
    for (; kt + 4 < k1 && kt + 8 <= KT; kt += 4) {
      plain(st0, st1, kt, kEven, tac, tbc);
      plain(st1, st2, kt + 1, kOdd, tac, tbc);
      plain(st2, st3, kt + 2, kEven, tac, tbc);
      plain(st3, st0, kt + 3, kOdd, tac, tbc);
    }
    for (; kt < k1; kt += 4) {
      step(st0, st1, kt, k1, kEven, tac, tbc);
      step(st1, st2, kt + 1, k1, kOdd, tac, tbc);
      step(st2, st3, kt + 2, k1, kEven, tac, tbc);
      step(st3, st0, kt + 3, k1, kOdd, tac, tbc);
    }
  };

  if constexpr (kGram) {
    // KT is a multiple of 8 (K = m padded to the tile), or 0 for the A²
    // launch with c = 0 (B = b·A: no product, Y is fetched below)
    if (KT > 0) {
      issue(st0, 0);
      issue(st1, 1);
      issue(st2, 2);
      issue(st3, 3);
      asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
      phase(0, dA, std::true_type{}, std::true_type{});
      phase(dA, dB, std::false_type{}, std::true_type{});
      phase(dB, KT, std::false_type{}, std::false_type{});
    } else {
      issue_y(0);
      issue_y(1);
      issue_y(2);
      issue_y(3);
    }
  } else {
    // One layout for every k-tile: KT ≥ 8 (a multiple of 8), so the loop of
    // whole groups runs at least once (written so, which keeps the
    // accumulators in place).
    issue(st0, 0);
    issue(st1, 1);
    issue(st2, 2);
    issue(st3, 3);
    asm volatile("s_waitcnt vmcnt(12)\n\ts_barrier" ::: "memory");
    constexpr auto ta = std::bool_constant<TR == 1>{};
    constexpr auto tb = std::bool_constant<TR == 2>{};
    head(st0, kEven, ta, tb);
    int kt = 0;
    do {
      plain(st0, st1, kt, kEven, ta, tb);
      plain(st1, st2, kt + 1, kOdd, ta, tb);
      plain(st2, st3, kt + 2, kEven, ta, tb);
      plain(st3, st0, kt + 3, kOdd, ta, tb);
      kt += 4;
    } while (kt + 4 < KT);
    step(st0, st1, kt, KT, kEven, ta, tb);
    step(st1, st2, kt + 1, KT, kOdd, ta, tb);
    step(st2, st3, kt + 2, KT, kEven, ta, tb);
    step(st3, st0, kt + 3, KT, kOdd, ta, tb);
  }

  // Wait states between the last MFMA writing an accumulator and the first
  // other instruction reading it (more than the deepest MFMA needs); the
  // empty statements order every later use of acc after them.
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");
#pragma unroll
  for (int fi = 0; fi < FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < FN; ++fj) asm volatile("" : "+v"(acc[fi][fj]));

  const EpiArgs<T> E = make_epi<T, EPI>(L, S, mat);
  if constexpr (kSym) {
    // Every wave is done with the ring, and every load (the Y block of the
    // Gram products included) has landed, before LDS is read or reused.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if constexpr (kGram) {
      // y = λ·acc + μ·Y (a·Y + u·B·Y, or b·A + c·u·A²), stored as sOut·y.
      // A lane reads Y at its four consecutive columns of a row and writes
      // the result back to the same LDS address: no other lane touches it,
      // so the rows of the output tile are staged with no barrier between.
      const float lam = E.sOut * S.ylam, mu = E.sOut * S.ymu;
      static_for<0, FM>([&](auto fi) {
        static_for<0, FN>([&](auto fj) {
          char* p = lds + soff<true>(wm * WTM + fi * 16 + lc, wn * WTN + fj * 16 + 4 * lg);
          const half4 y = *(const half4*)p;
          half4 h;
          static_for<0, 4>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            acc[fi][fj][r] = lam * acc[fi][fj][r] + mu * (float)y[r];
            h[r] = (_Float16)acc[fi][fj][r];
          });
          *(half4*)p = h;
        });
      });
    } else {
      // acc ← storage value of the result, sOut·u·acc
      const float scale = E.sOut * E.u;
      static_for<0, FM>([&](auto fi) {
        static_for<0, FN>([&](auto fj) {
          static_for<0, 4>([&](auto rc) {
            constexpr int r = decltype(rc)::value;
            acc[fi][fj][r] *= scale;
          });
        });
      });
    }
    SecondCopy sc{E.outhb, E.sOutB / E.sOut, E.sOutB * E.p0, E.mReal};
    if (EPI == EPI_SQ && E.outhb) {
      // first step: Q₁ = a·I + B₀ written from the same staged B₀ values
      write_symmetric<FM, FN, true, kGram>(E.outh, E.ldc, lds, ti, tj, wm, wn, lc, lg, tid, acc, sc,
                                           S.mirrorOut != 0);
    } else {
      write_symmetric<FM, FN, false, kGram>(E.outh, E.ldc, lds, ti, tj, wm, wn, lc, lg, tid, acc, sc,
                                            S.mirrorOut != 0);
    }
    if constexpr (EPI == EPI_SYRK) {
      if (E.writeIdentity) {  // zero steps: Q₀ = I (rare; element by element)
        const int gi0 = ti * BM + wm * WTM, gj0 = tj * BN + wn * WTN;
        static_for<0, FM>([&](auto fi) {
          static_for<0, FN>([&](auto fj) {
            static_for<0, 4>([&](auto rc) {
              constexpr int r = decltype(rc)::value;
              const int i = gi0 + fi * 16 + lc;
              const int j = gj0 + fj * 16 + 4 * lg + r;
              if (i <= j)
                store_mirror<T>(E.outhb, E.ldc, i, j, (T)((i == j && i < E.mReal) ? E.sOutB : 0.f));
            });
          });
        });
      }
    }
  } else if (EPI == EPI_UPDATE ? pref : dense_fast_ok(E, ti, tj)) {
    // Every wave is done with the ring, and the weights have landed, before
    // the staging is written; the rows are stored once all of it is.
    constexpr bool kPre = EPI == EPI_UPDATE;
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    dense_stage<EPI, kPre, FM, FN>(E, lds, wm, wn, lc, lg, acc);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const SecondCopy none{nullptr, 0.f, 0.f, 0};
    store_staged<false, kPre>((_Float16*)E.user, (int)E.userLd, lds, ti, tj, tid, none);
  } else {
    dense_direct<EPI, FM, FN>(E, ti, tj, wm, wn, lc, lg, acc);
  }
}

template <int EPI>
hipError_t launch_epi(int op, int tile, const GemmLaunch& L, int blocks, hipStream_t st) {
  if (op == OP_F16 && tile == 256) {
    // the main loop runs whole groups of four k-tiles, phases of eight
    // (K = 0 only for the A² launch: with c = 0, B = b·A needs no product)
    for (int k = 0; k < L.nseg; ++k)
      if (L.seg[k].K < (EPI == EPI_SQ ? 0 : 1) || L.seg[k].K % 256 != 0) return hipErrorInvalidValue;
    if constexpr (EPI == EPI_UPDATE || EPI == EPI_OUT) {
      // one bucket per launch, so every segment shares the operand layout
      if (L.seg[0].transA)
        hipLaunchKernelGGL((gemm256_kernel<EPI, 1>), dim3(blocks), dim3(512), 0, st, L);
      else if (L.seg[0].transB)
        hipLaunchKernelGGL((gemm256_kernel<EPI, 2>), dim3(blocks), dim3(512), 0, st, L);
      else
        hipLaunchKernelGGL((gemm256_kernel<EPI, 0>), dim3(blocks), dim3(512), 0, st, L);
    } else {
      hipLaunchKernelGGL((gemm256_kernel<EPI>), dim3(blocks), dim3(512), 0, st, L);
    }
  } else if (op == OP_F16 && tile == 128) {
    hipLaunchKernelGGL((gemm_kernel<_Float16, 128, 128, 2, 2, EPI>), dim3(blocks), dim3(256), 0, st, L);
  } else if (op == OP_F32 && tile == 128) {
    hipLaunchKernelGGL((gemm_kernel<float, 128, 128, 2, 2, EPI>), dim3(blocks), dim3(256), 0, st, L);
  } else if (op == OP_F32 && tile == 64) {
    hipLaunchKernelGGL((gemm_kernel<float, 64, 64, 2, 2, EPI>), dim3(blocks), dim3(256), 0, st, L);
  } else if (op == OP_F32 && tile == 32) {
    hipLaunchKernelGGL((gemm32_kernel<EPI>), dim3(blocks), dim3(256), 0, st, L);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

extern template hipError_t launch_epi<EPI_SYRK>(int, int, const GemmLaunch&, int, hipStream_t);
extern template hipError_t launch_epi<EPI_SQ>(int, int, const GemmLaunch&, int, hipStream_t);
extern template hipError_t launch_epi<EPI_AXPY>(int, int, const GemmLaunch&, int, hipStream_t);
extern template hipError_t launch_epi<EPI_UPDATE>(int, int, const GemmLaunch&, int, hipStream_t);
extern template hipError_t launch_epi<EPI_OUT>(int, int, const GemmLaunch&, int, hipStream_t);

}  // namespace muon
