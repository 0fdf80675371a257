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

#include "common.hpp"
#include "launch.hpp"

namespace muon {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

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

// Epilogue for one accumulator element (i, j) of matrix `mat` of segment S.
template <typename T>
__device__ __forceinline__ void epilogue(const GemmLaunch& L, const GemmSeg& S, int mat, int i,
                                         int j, float acc) {
  const int ldc = S.ldc;
  switch (S.epi) {
    case EPI_SYRK: {
      if (i > j) return;
      const float g = S.u * acc;
      S.out32[mat * S.strideOut32 + (int64_t)i * ldc + j] = g;
      store_mirror<T>((T*)S.outh + mat * S.strideOuth, ldc, i, j, to_op<T>(S.sOut * g));
      if (S.writeIdentity) {
        const float q = (i == j && i < S.mReal) ? S.sOutB : 0.f;
        store_mirror<T>((T*)S.outhb + mat * S.strideOuth, ldc, i, j, to_op<T>(q));
      }
      return;
    }
    case EPI_SQ: {
      if (i > j) return;
      const int64_t e = (int64_t)i * ldc + j;
      const float a2 = S.u * acc;
      const float bb = S.p1 * S.in32[mat * S.strideIn32 + e] + S.p2 * a2;
      store_mirror<T>((T*)S.outh + mat * S.strideOuth, ldc, i, j, to_op<T>(S.sOut * bb));
      if (S.out32b) {
        const float q = bb + ((i == j && i < S.mReal) ? S.p0 : 0.f);
        S.out32b[mat * S.strideOut32 + e] = q;
        store_mirror<T>((T*)S.outhb + mat * S.strideOuth, ldc, i, j, to_op<T>(S.sOutB * q));
      }
      return;
    }
    case EPI_AXPY: {
      if (i > j) return;
      const int64_t e = (int64_t)i * ldc + j;
      const float y = S.p0 * S.in32[mat * S.strideIn32 + e] + S.u * acc;
      S.out32[mat * S.strideOut32 + e] = y;
      store_mirror<T>((T*)S.outh + mat * S.strideOuth, ldc, i, j, to_op<T>(S.sOut * y));
      return;
    }
    case EPI_UPDATE: {
      if (i >= S.mReal || j >= S.nReal) return;
      const int k = S.userBase + mat;
      const int64_t e = (int64_t)i * L.userLd[k] + j;
      const float d = L.lrsc[k] * (S.u * acc);
      if (L.userDtype == 1) {
        uint16_t* w = (uint16_t*)L.user[k];
        w[e] = f32_to_bf16_rne(bf16_to_f32(w[e]) - d);
      } else {
        float* w = (float*)L.user[k];
        w[e] = w[e] - d;
      }
      return;
    }
    case EPI_OUT: {
      if (i >= S.mReal || j >= S.nReal) return;
      const int k = S.userBase + mat;
      const int64_t e = (int64_t)i * L.userLd[k] + j;
      const float v = S.u * acc;
      if (L.userDtype == 1) ((uint16_t*)L.user[k])[e] = f32_to_bf16_rne(v);
      else ((float*)L.user[k])[e] = v;
      return;
    }
    default:
      return;
  }
}

template <typename T, int BM, int BN, int WM, int WN>
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

  __shared__ uint4 smem[2][(BM + BN) * CH];

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

  uint4 ra[LA], rb[LB];
  auto gload = [&](int kt) {
    const int k0 = kt * BK + c * EPC;
#pragma unroll
    for (int p = 0; p < LA; ++p)
      ra[p] = *(const uint4*)(Ag + (int64_t)(r0 + p * RPP) * S.lda + k0);
#pragma unroll
    for (int p = 0; p < LB; ++p)
      rb[p] = *(const uint4*)(Bg + (int64_t)(r0 + p * RPP) * S.ldb + k0);
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int p = 0; p < LA; ++p) {
      const int r = r0 + p * RPP;
      smem[buf][r * CH + (c ^ (r & 7))] = ra[p];
    }
#pragma unroll
    for (int p = 0; p < LB; ++p) {
      const int r = r0 + p * RPP;
      smem[buf][(BM + r) * CH + (c ^ (r & 7))] = rb[p];
    }
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
  lstore(0);
  __syncthreads();

  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    const uint4* sa = smem[buf];
    const uint4* sb = smem[buf] + BM * CH;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int kk = 0; kk < BK / 16; ++kk) {
        const int cc = 2 * kk + lh;
        half8 af[FM], bf[FN];
#pragma unroll
        for (int fi = 0; fi < FM; ++fi) {
          const int row = wm * WTM + fi * 32 + lr;
          uint4 v = sa[row * CH + (cc ^ (row & 7))];
          af[fi] = __builtin_bit_cast(half8, v);
        }
#pragma unroll
        for (int fj = 0; fj < FN; ++fj) {
          const int row = wn * WTN + fj * 32 + lr;
          uint4 v = sb[row * CH + (cc ^ (row & 7))];
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
          uint4 v0 = sa[row * CH + (c0 ^ (row & 7))];
          uint4 v1 = sa[row * CH + ((c0 + 1) ^ (row & 7))];
          av[fi][0] = __uint_as_float(v0.x); av[fi][1] = __uint_as_float(v0.y);
          av[fi][2] = __uint_as_float(v0.z); av[fi][3] = __uint_as_float(v0.w);
          av[fi][4] = __uint_as_float(v1.x); av[fi][5] = __uint_as_float(v1.y);
          av[fi][6] = __uint_as_float(v1.z); av[fi][7] = __uint_as_float(v1.w);
        }
#pragma unroll
        for (int fj = 0; fj < FN; ++fj) {
          const int row = wn * WTN + fj * 32 + lr;
          uint4 v0 = sb[row * CH + (c0 ^ (row & 7))];
          uint4 v1 = sb[row * CH + ((c0 + 1) ^ (row & 7))];
          bv[fj][0] = __uint_as_float(v0.x); bv[fj][1] = __uint_as_float(v0.y);
          bv[fj][2] = __uint_as_float(v0.z); bv[fj][3] = __uint_as_float(v0.w);
          bv[fj][4] = __uint_as_float(v1.x); bv[fj][5] = __uint_as_float(v1.y);
          bv[fj][6] = __uint_as_float(v1.z); bv[fj][7] = __uint_as_float(v1.w);
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
    if (kt + 1 < KT) lstore(buf ^ 1);
    __syncthreads();
  }

  // 32×32 accumulator layout: lane l, register r holds
  // row 8·(r/4) + 4·(l/32) + r%4, column l%32 of the block.
  const int gi0 = ti * BM + wm * WTM, gj0 = tj * BN + wn * WTN;
#pragma unroll
  for (int fi = 0; fi < FM; ++fi)
#pragma unroll
    for (int fj = 0; fj < FN; ++fj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int i = gi0 + fi * 32 + 8 * (r >> 2) + 4 * lh + (r & 3);
        const int j = gj0 + fj * 32 + lr;
        epilogue<T>(L, S, mat, i, j, acc[fi][fj][r]);
      }
}

hipError_t launch_gemm(int op, int tile, const GemmLaunch& L, int blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  if (op == OP_F16 && tile == 256) {
    hipLaunchKernelGGL((gemm_kernel<_Float16, 256, 256, 2, 4>), dim3(blocks), dim3(512), 0, st, L);
  } else if (op == OP_F16 && tile == 128) {
    hipLaunchKernelGGL((gemm_kernel<_Float16, 128, 128, 2, 2>), dim3(blocks), dim3(256), 0, st, L);
  } else if (op == OP_F32 && tile == 128) {
    hipLaunchKernelGGL((gemm_kernel<float, 128, 128, 2, 2>), dim3(blocks), dim3(256), 0, st, L);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace muon
