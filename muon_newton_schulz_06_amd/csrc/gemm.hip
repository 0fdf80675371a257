// MFMA products for the Gram Newton–Schulz step on gfx950 (CDNA4).
//
// One kernel template serves every dense contraction of the step
// (DMuon technical summary, gist.science Korean, §2.2):
//   * the SYRK G = X₀·X₀ᵀ,
//   * the symmetric Gram-space products A², B·Q, B·A, B·(P·A),
//   * the final product Q·X₀ (or X₀ᵀ·Q for tall matrices) with the weight
//     update fused into its epilogue.
// Every product has the form C[i][j] = Σ_k A[i][k]·B[j][k] with both operands
// stored row-major with k contiguous: for the Gram-space products this holds
// because every operand is symmetric (a polynomial in G), for the SYRK and
// the final product because X₀ is kept in both layouts.
//
// Symmetric outputs (every Gram-space product is a product of commuting
// polynomials in G, hence symmetric) are computed on upper-triangle tiles
// only; the fp16 operand copy is written mirrored so the next product can
// read whole rows, and the fp32 state is kept on the upper triangle.
// Diagonal tiles store the element of the upper half into both (i, j) and
// (j, i), so every stored iterate is exactly symmetric.
//
// Tiling: BM×BN workgroup tile, WM×WN waves, 32×32 MFMA blocks per wave,
// 128-byte k-rows in LDS (64 halves or 32 floats) with a 16-byte-chunk XOR
// swizzle (conflict-free ds_read_b128), double-buffered through registers.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "common.hpp"
#include "launch.hpp"

namespace muon {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
// Native 16-byte vector (scalarisable, unlike HIP's uint4 class type).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

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

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own
// L2).  Give every XCD a contiguous range of logical tiles, so that tiles
// sharing operand row panels run under the same L2.
__device__ __forceinline__ int xcd_remap(int b, int G) {
  constexpr int X = 8;
  const int x = b % X, i = b / X;
  const int q = G / X, r = G % X;
  const int base = x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q;
  return base + i;
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
  float* out32;
  const float* in32;
  T* outh;
  float* out32b;
  T* outhb;
  void* user;
  int64_t userLd;
  int ldc, mReal, nReal, writeIdentity, userDtype;
  float u, sOut, sOutB, p0, p1, p2, lrsc;
};

// Epilogue for one accumulator element (i, j).  EPI is a compile-time
// constant so each instantiation carries only its own code.
template <typename T, int EPI>
__device__ __forceinline__ void epilogue(const EpiArgs<T>& E, int i, int j, float acc) {
  const int ldc = E.ldc;
  if constexpr (EPI == EPI_SYRK) {
    if (i > j) return;
    const float g = E.u * acc;
    E.out32[(int64_t)i * ldc + j] = g;
    store_mirror<T>(E.outh, ldc, i, j, to_op<T>(E.sOut * g));
    if (E.writeIdentity) {
      const float q = (i == j && i < E.mReal) ? E.sOutB : 0.f;
      store_mirror<T>(E.outhb, ldc, i, j, to_op<T>(q));
    }
  } else if constexpr (EPI == EPI_SQ) {
    if (i > j) return;
    const int64_t e = (int64_t)i * ldc + j;
    const float bb = E.p1 * E.in32[e] + E.p2 * (E.u * acc);
    store_mirror<T>(E.outh, ldc, i, j, to_op<T>(E.sOut * bb));
    if (E.out32b) {
      const float q = bb + ((i == j && i < E.mReal) ? E.p0 : 0.f);
      E.out32b[e] = q;
      store_mirror<T>(E.outhb, ldc, i, j, to_op<T>(E.sOutB * q));
    }
  } else if constexpr (EPI == EPI_AXPY) {
    if (i > j) return;
    const int64_t e = (int64_t)i * ldc + j;
    const float y = E.p0 * E.in32[e] + E.u * acc;
    E.out32[e] = y;
    store_mirror<T>(E.outh, ldc, i, j, to_op<T>(E.sOut * y));
  } else if constexpr (EPI == EPI_UPDATE) {
    if (i >= E.mReal || j >= E.nReal) return;
    const int64_t e = (int64_t)i * E.userLd + j;
    const float d = E.lrsc * (E.u * acc);
    if (E.userDtype == 1) {
      uint16_t* w = (uint16_t*)E.user;
      w[e] = f32_to_bf16_rne(bf16_to_f32(w[e]) - d);
    } else {
      float* w = (float*)E.user;
      w[e] = w[e] - d;
    }
  } else if constexpr (EPI == EPI_OUT) {
    if (i >= E.mReal || j >= E.nReal) return;
    const int64_t e = (int64_t)i * E.userLd + j;
    const float v = E.u * acc;
    if (E.userDtype == 1) ((uint16_t*)E.user)[e] = f32_to_bf16_rne(v);
    else ((float*)E.user)[e] = v;
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

  const int lid = xcd_remap(blockIdx.x, gridDim.x);
  int s = 0;
  while (s + 1 < L.nseg && lid >= L.segStart[s + 1]) ++s;
  const GemmSeg& S = L.seg[s];
  int t = lid - L.segStart[s];
  const int mat = t / S.tilesPerMat;
  t -= mat * S.tilesPerMat;
  int ti, tj;
  if (S.sym) {
    int rowlen = S.tilesM;
    ti = 0;
    while (t >= rowlen) {
      t -= rowlen;
      ++ti;
      --rowlen;
    }
    tj = ti + t;
  } else {
    ti = t / S.tilesN;
    tj = t - ti * S.tilesN;
  }

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
      sm[r * CH + (c ^ (r & 7))] = ra[p];
    });
    static_for<0, LB>([&](auto p) {
      const int r = r0 + p * RPP;
      sm[(BM + r) * CH + (c ^ (r & 7))] = rb[p];
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
          u32x4 v = sa[row * CH + (cc ^ (row & 7))];
          af[fi] = __builtin_bit_cast(half8, v);
        }
#pragma unroll
        for (int fj = 0; fj < FN; ++fj) {
          const int row = wn * WTN + fj * 32 + lr;
          u32x4 v = sb[row * CH + (cc ^ (row & 7))];
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
          u32x4 v0 = sa[row * CH + (c0 ^ (row & 7))];
          u32x4 v1 = sa[row * CH + ((c0 + 1) ^ (row & 7))];
          av[fi][0] = __uint_as_float(v0[0]); av[fi][1] = __uint_as_float(v0[1]);
          av[fi][2] = __uint_as_float(v0[2]); av[fi][3] = __uint_as_float(v0[3]);
          av[fi][4] = __uint_as_float(v1[0]); av[fi][5] = __uint_as_float(v1[1]);
          av[fi][6] = __uint_as_float(v1[2]); av[fi][7] = __uint_as_float(v1[3]);
        }
#pragma unroll
        for (int fj = 0; fj < FN; ++fj) {
          const int row = wn * WTN + fj * 32 + lr;
          u32x4 v0 = sb[row * CH + (c0 ^ (row & 7))];
          u32x4 v1 = sb[row * CH + ((c0 + 1) ^ (row & 7))];
          bv[fj][0] = __uint_as_float(v0[0]); bv[fj][1] = __uint_as_float(v0[1]);
          bv[fj][2] = __uint_as_float(v0[2]); bv[fj][3] = __uint_as_float(v0[3]);
          bv[fj][4] = __uint_as_float(v1[0]); bv[fj][5] = __uint_as_float(v1[1]);
          bv[fj][6] = __uint_as_float(v1[2]); bv[fj][7] = __uint_as_float(v1[3]);
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
  EpiArgs<T> E;
  E.ldc = S.ldc;
  E.mReal = S.mReal;
  E.nReal = S.nReal;
  E.writeIdentity = S.writeIdentity;
  E.u = S.u;
  E.sOut = S.sOut;
  E.sOutB = S.sOutB;
  E.p0 = S.p0;
  E.p1 = S.p1;
  E.p2 = S.p2;
  E.out32 = S.out32 ? S.out32 + mat * S.strideOut32 : nullptr;
  E.in32 = S.in32 ? S.in32 + mat * S.strideIn32 : nullptr;
  E.outh = S.outh ? (T*)S.outh + mat * S.strideOuth : nullptr;
  E.out32b = S.out32b ? S.out32b + mat * S.strideOut32 : nullptr;
  E.outhb = S.outhb ? (T*)S.outhb + mat * S.strideOuth : nullptr;
  E.user = nullptr;
  E.userLd = 0;
  E.lrsc = 0.f;
  E.userDtype = L.userDtype;
  if constexpr (EPI == EPI_UPDATE || EPI == EPI_OUT) {
    const int k = S.userBase + mat;
    E.user = L.user[k];
    E.userLd = L.userLd[k];
    E.lrsc = L.lrsc[k];
  }
  const int gi0 = ti * BM + wm * WTM, gj0 = tj * BN + wn * WTN;
  epilogue_all<T, EPI, FM, FN>(E, gi0, gj0, lh, lr, acc);
}

template <int EPI>
hipError_t launch_epi(int op, int tile, const GemmLaunch& L, int blocks, hipStream_t st) {
  if (op == OP_F16 && tile == 256) {
    hipLaunchKernelGGL((gemm_kernel<_Float16, 256, 256, 2, 4, EPI>), dim3(blocks), dim3(512), 0, st, L);
  } else if (op == OP_F16 && tile == 128) {
    hipLaunchKernelGGL((gemm_kernel<_Float16, 128, 128, 2, 2, EPI>), dim3(blocks), dim3(256), 0, st, L);
  } else if (op == OP_F32 && tile == 128) {
    hipLaunchKernelGGL((gemm_kernel<float, 128, 128, 2, 2, EPI>), dim3(blocks), dim3(256), 0, st, L);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(int op, int tile, const GemmLaunch& L, int blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  const int epi = L.seg[0].epi;
  for (int k = 1; k < L.nseg; ++k)
    if (L.seg[k].epi != epi) return hipErrorInvalidValue;  // one epilogue per launch
  switch (epi) {
    case EPI_SYRK: return launch_epi<EPI_SYRK>(op, tile, L, blocks, st);
    case EPI_SQ: return launch_epi<EPI_SQ>(op, tile, L, blocks, st);
    case EPI_AXPY: return launch_epi<EPI_AXPY>(op, tile, L, blocks, st);
    case EPI_UPDATE: return launch_epi<EPI_UPDATE>(op, tile, L, blocks, st);
    case EPI_OUT: return launch_epi<EPI_OUT>(op, tile, L, blocks, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace muon
