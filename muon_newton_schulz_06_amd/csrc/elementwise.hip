// HBM-bound stages of the Muon step on gfx950.
//
//  * momentum + sum of squares: M ← β·M + g (one fused multiply-add) and the
//    per-workgroup partial Σ M², in one pass over g and M (DeMuon technical
//    summary, gist.science Korean, Method §1: the momentum is a moving
//    average of the gradients; DMuon technical summary §1: NS runs on the
//    momentum-accumulated gradient).  With the Nesterov option the value
//    orthogonalised is u = g + β·M (after the update), and Σ u² is summed;
//    gradients may be fp32 or bf16;
//  * norm finish: α = 1/(√ΣM² + eps) per matrix, summing the partials in a
//    fixed order (deterministic, no float atomics);
//  * scaled cast: X₀ = α·sX·M rounded to the MFMA operand type, written in
//    both the stored and the transposed layout (with zero padding to the
//    tile), so every later product reads k-contiguous rows;
//  * momentum fused with the cast, for callers that carry a power-of-two
//    operand exponent e per matrix from the previous step: the momentum pass
//    writes the fp16 operand as u·2^e directly (no second pass over the
//    fp32 momentum), the norm finish checks that ‖u‖·2^e keeps it in range
//    and hands the products the exact factor ρ = α·sX·2^(−e) (X₀ = ρ·u·2^e),
//    and the cast runs only for matrices that fail the check.
// Reductions use 64-lane wavefront shuffles, then one LDS slot per wave.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"

namespace muon {

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float load_as_f32(const void* p, int64_t e, int dtype) {
  if (dtype == 1) return __uint_as_float((uint32_t)((const uint16_t*)p)[e] << 16);
  return ((const float*)p)[e];
}

// Four consecutive values at element e (e % 4 == 0, 8-byte aligned for
// bf16, 16-byte aligned for fp32), widened to fp32.
template <int GD>
__device__ __forceinline__ f32x4 load4(const void* p, int64_t e) {
  f32x4 r;
  if constexpr (GD == 1) {
    const uint2 u = *(const uint2*)((const uint16_t*)p + e);
    r[0] = __uint_as_float(u.x << 16);
    r[1] = __uint_as_float(u.x & 0xffff0000u);
    r[2] = __uint_as_float(u.y << 16);
    r[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    r = __builtin_nontemporal_load((const f32x4*)((const float*)p + e));
  }
  return r;
}

// Momentum of one block of kEwElems elements wholly inside the matrix: every
// load is issued before the first store (the compiler cannot prove that g
// and M do not overlap, so interleaved load/store pairs would serialise on
// memory latency).  Returns this thread's part of Σ u².
template <int GD, bool NEST>
__device__ __forceinline__ float momentum_block(const void* g, float* m, int64_t e0, float beta,
                                                int tid) {
  constexpr int Q = kEwElems / (4 * kEwThreads);
  f32x4 gv[Q], mv[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int64_t e = e0 + (int64_t)(q * kEwThreads + tid) * 4;
    gv[q] = load4<GD>(g, e);
    mv[q] = *(const f32x4*)(m + e);
  }
  float ss = 0.f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int64_t e = e0 + (int64_t)(q * kEwThreads + tid) * 4;
    f32x4 v;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      v[c] = fmaf(beta, mv[q][c], gv[q][c]);
      const float u = NEST ? fmaf(beta, v[c], gv[q][c]) : v[c];
      ss += u * u;
    }
    *(f32x4*)(m + e) = v;
  }
  return ss;
}

__global__ __launch_bounds__(kEwThreads) void ew_kernel(const EwLaunch L) {
  const int64_t b = blockIdx.x;
  int mi = 0;
  while (mi + 1 < L.n && b >= L.mat[mi + 1].blockStart) ++mi;
  const EwMat& M = L.mat[mi];
  const int64_t blk = b - M.blockStart;
  const int64_t e0 = blk * kEwElems;
  const int tid = threadIdx.x;
  float ss = 0.f;
  if (L.mode == 0) {
    const void* g = M.x;
    float* m = M.mom;
    if (L.vec && e0 + kEwElems <= M.numel) {
      if (L.xDtype == 1) ss = L.nesterov ? momentum_block<1, true>(g, m, e0, L.beta, tid)
                                         : momentum_block<1, false>(g, m, e0, L.beta, tid);
      else ss = L.nesterov ? momentum_block<0, true>(g, m, e0, L.beta, tid)
                           : momentum_block<0, false>(g, m, e0, L.beta, tid);
    } else {
      for (int q = 0; q < kEwElems / kEwThreads; ++q) {
        const int64_t e = e0 + q * kEwThreads + tid;
        if (e < M.numel) {
          const float gv = load_as_f32(g, e, L.xDtype);
          const float v = fmaf(L.beta, m[e], gv);
          m[e] = v;
          const float u = L.nesterov ? fmaf(L.beta, v, gv) : v;
          ss += u * u;
        }
      }
    }
  } else if (L.vec && e0 + kEwElems <= M.numel) {
    // contiguous input (ld == cols): 16-byte loads of the flat block, every
    // load of the block issued before the first product
    constexpr int Q = kEwElems / (4 * kEwThreads);
    if (L.xDtype == 1) {
      u32x4 u[Q / 2];
#pragma unroll
      for (int q = 0; q < Q / 2; ++q)
        u[q] = __builtin_nontemporal_load((const u32x4*)((const uint16_t*)M.x + e0 + (int64_t)(q * kEwThreads + tid) * 8));
#pragma unroll
      for (int q = 0; q < Q / 2; ++q) {
        const uint32_t w[4] = {u[q][0], u[q][1], u[q][2], u[q][3]};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float a = __uint_as_float(w[h] << 16), b = __uint_as_float(w[h] & 0xffff0000u);
          ss += a * a;
          ss += b * b;
        }
      }
    } else {
      f32x4 x[Q];
#pragma unroll
      for (int q = 0; q < Q; ++q)
        x[q] = __builtin_nontemporal_load((const f32x4*)((const float*)M.x + e0 + (int64_t)(q * kEwThreads + tid) * 4));
#pragma unroll
      for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) ss += x[q][c] * x[q][c];
    }
  } else {
    for (int q = 0; q < kEwElems / kEwThreads; ++q) {
      const int64_t e = e0 + q * kEwThreads + tid;
      if (e < M.numel) {
        const int64_t r = e / M.cols;
        const int64_t cc = e - r * M.cols;
        const float v = load_as_f32(M.x, r * M.ld + cc, L.xDtype);
        ss += v * v;
      }
    }
  }
  __shared__ float part[kEwThreads / 64];
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < kEwThreads / 64; ++w) t += part[w];
    L.partials[M.partialOff + blk] = t;
  }
}

__device__ __forceinline__ bool exp_known(int e) { return e >= -kFuseExpMax && e <= kFuseExpMax; }

__global__ __launch_bounds__(256) void norm_kernel(const NormLaunch L) {
  const int i = blockIdx.x;
  const int tid = threadIdx.x;
  const float* p = L.partials + L.off[i];
  double s = 0.0;
  for (int64_t k = tid; k < L.cnt[i]; k += 256) s += (double)p[k];
  __shared__ double part[4];
  s = wave_sum_d(s);
  if ((tid & 63) == 0) part[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) {
    const double t = part[0] + part[1] + part[2] + part[3];
    const double nrm = sqrt(t);
    const float alpha = (float)(1.0 / (nrm + (double)L.eps));
    L.alpha[L.alphaIdx[i]] = alpha;
    int32_t* h = L.hint[i];
    if (h) {
      // The fused operand u·2^e stands when ‖u‖·2^e ∈ [2^kFuseLo, 2^kFuseHi]:
      // every entry is then below 2^15 (|u_ij| ≤ ‖u‖) and the bulk of them far
      // above fp16's subnormal range.  (A NaN norm fails the comparison.)
      const int e = *h;
      const bool known = exp_known(e);
      const double x = known ? ldexp(nrm, e) : 0.0;
      const bool ok = known && x >= ldexp(1.0, kFuseLo) && x <= ldexp(1.0, kFuseHi);
      L.ok[L.alphaIdx[i]] = ok ? 1 : 0;
      L.rho[L.rhoIdx[i]] = ok ? (alpha * L.sX) * ldexpf(1.f, -e) : 1.f;
      // next step's exponent: ‖u‖ = f·2^q (f ∈ [0.5, 1)) → e' = kFuseTarget − q
      int en = INT32_MIN;
      if (nrm > 0.0 && nrm < 1e300) {
        int q;
        (void)frexp(nrm, &q);
        if (exp_known(kFuseTarget - q)) en = kFuseTarget - q;
      }
      *h = en;
    }
  }
}

template <typename T> __device__ __forceinline__ T cvt(float v);
template <> __device__ __forceinline__ _Float16 cvt<_Float16>(float v) { return (_Float16)v; }
template <> __device__ __forceinline__ float cvt<float>(float v) { return v; }

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));

// One 64×64 tile: 16 threads per 64-element row (16-byte fp32 loads when the
// source allows), the stored-layout copy written straight from registers
// (8 bytes per thread for fp16), the transposed copy through an fp32 LDS
// tile (pitch 65: conflict-free column reads) with 16-byte stores of 8
// consecutive elements.  Out-of-range elements (padding) are written as 0.
template <typename T>
__device__ void cast_tile(const CastLaunch& L, const CastMat& C, int64_t t) {
  __shared__ float tile[kCastTile][kCastTile + 1];
  const int tr = (int)(t / C.tilesC), tc = (int)(t - (int64_t)tr * C.tilesC);
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const float scale = L.alpha[C.alphaIdx] * L.sX;
  const bool nest = L.nesterov != 0;
  T* S = (T*)C.S;
  T* Tt = (T*)C.T;
  const int64_t r0 = (int64_t)tr * kCastTile, c0 = (int64_t)tc * kCastTile;
  const bool full = (r0 + kCastTile <= C.rows) && (c0 + kCastTile <= C.cols);
  const bool vec = full && L.srcDtype == 0 && (C.ld % 4 == 0) && (((uintptr_t)C.src & 15) == 0) &&
                   (!L.nesterov || (((uintptr_t)C.grad & (L.gradDtype == 1 ? 7 : 15)) == 0));
  // All four source rows are loaded before anything is stored (the
  // compiler cannot prove that the source and the copies do not overlap).
  // bf16 input (the batched orthogonalisation of bf16 matrices): 8-byte loads
  const bool vecb = full && !nest && L.srcDtype == 1 && (C.ld % 4 == 0) &&
                    (((uintptr_t)C.src & 7) == 0);
  const int cl = 4 * tx;
  float v[4][4];
  if (vecb) {
    uint2 x[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      x[q] = *(const uint2*)((const uint16_t*)C.src + (r0 + ty + 16 * q) * C.ld + c0 + cl);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q][0] = __uint_as_float(x[q].x << 16) * scale;
      v[q][1] = __uint_as_float(x[q].x & 0xffff0000u) * scale;
      v[q][2] = __uint_as_float(x[q].y << 16) * scale;
      v[q][3] = __uint_as_float(x[q].y & 0xffff0000u) * scale;
    }
  } else if (vec && !nest) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 x = *(const f32x4*)((const float*)C.src + (r0 + ty + 16 * q) * C.ld + c0 + cl);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[q][e] = x[e] * scale;
    }
  } else if (vec) {  // Nesterov: u = g + β·M', M' fp32, g fp32 or bf16 (contiguous)
    f32x4 x[4], gq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t e = (r0 + ty + 16 * q) * C.ld + c0 + cl;
      x[q] = *(const f32x4*)((const float*)C.src + e);
      gq[q] = L.gradDtype == 1 ? load4<1>(C.grad, e) : load4<0>(C.grad, e);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) v[q][e] = fmaf(L.beta, x[q][e], gq[q][e]) * scale;
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t r = r0 + ty + 16 * q;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t cc = c0 + cl + e;
        float x = 0.f;
        if (r < C.rows && cc < C.cols) {
          x = load_as_f32(C.src, r * C.ld + cc, L.srcDtype);
          if (nest) x = fmaf(L.beta, x, load_as_f32(C.grad, r * C.ld + cc, L.gradDtype));
        }
        v[q][e] = x * scale;
      }
    }
  }
  // Either copy may be absent (a null pointer): the operand layouts a
  // bucket keeps depend on the kernel that reads them.
  if (Tt) {
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) tile[ty + 16 * q][cl + e] = v[q][e];
  }
  if (S) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t r = r0 + ty + 16 * q;
      T* dst = S + r * C.cp + c0 + cl;
      if constexpr (sizeof(T) == 2) {
        half4_t h;
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = (_Float16)v[q][e];
        *(half4_t*)dst = h;
      } else {
        *(float4*)dst = make_float4(v[q][0], v[q][1], v[q][2], v[q][3]);
      }
    }
  }
  if (!Tt) return;
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int id = p * 256 + tid;
    const int cl = id >> 3, rl0 = (id & 7) * 8;
    T* dst = Tt + (c0 + cl) * C.rp + r0 + rl0;
    if constexpr (sizeof(T) == 2) {
      half8_t h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = (_Float16)tile[rl0 + e][cl];
      *(half8_t*)dst = h;
    } else {
      *(float4*)dst = make_float4(tile[rl0][cl], tile[rl0 + 1][cl], tile[rl0 + 2][cl], tile[rl0 + 3][cl]);
      *(float4*)(dst + 4) = make_float4(tile[rl0 + 4][cl], tile[rl0 + 5][cl], tile[rl0 + 6][cl], tile[rl0 + 7][cl]);
    }
  }
}

__global__ __launch_bounds__(256) void cast_kernel(const CastLaunch L) {
  if (L.strided) {
    // fallback for fused operands: almost always every matrix is skipped
    for (int mi = 0; mi < L.n; ++mi) {
      const CastMat& C = L.mat[mi];
      if (L.ok[C.okIdx]) continue;
      const int64_t tiles = (int64_t)(C.rp / kCastTile) * C.tilesC;
      for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        if (L.outOp == OP_F16) cast_tile<_Float16>(L, C, t);
        else cast_tile<float>(L, C, t);
        __syncthreads();  // the next tile reuses the LDS tile
      }
    }
    return;
  }
  const int64_t b = blockIdx.x;
  int mi = 0;
  while (mi + 1 < L.n && b >= L.mat[mi + 1].blockStart) ++mi;
  const CastMat& C = L.mat[mi];
  if (C.okIdx >= 0 && L.ok[C.okIdx]) return;  // the momentum pass wrote the operand
  const int64_t t = b - C.blockStart;
  if (L.outOp == OP_F16) cast_tile<_Float16>(L, C, t);
  else cast_tile<float>(L, C, t);
}

// Momentum fused with the cast: one TR×TC tile of the stored matrix per
// workgroup (TC/4 threads per row, each 4 consecutive columns of rows ty,
// ty + RPI, …).  Elements outside rows × cols are not touched in M, add
// nothing to Σu² and are written as 0 in the operand (so the padding needs
// no other pass).  The operand is written only when the carried exponent is
// known; otherwise the cast writes it after the norm finish.  TALL: the
// operand is the transpose, staged through an fp32 LDS tile (pitch TC + 1)
// and written as 16-byte runs of 8 consecutive stored rows.
template <int TR, int TC, bool TALL, int GD, bool NEST>
__device__ void momcast_tile(const MomCastLaunch& L, const MomCastMat& C, int64_t t) {
  constexpr int TPR = TC / 4, RPI = 256 / TPR, Q = TR / RPI;
  __shared__ float tile[TALL ? TR : 1][TALL ? TC + 1 : 1];
  __shared__ float part[4];
  const int tr = (int)(t / C.tilesC), tc = (int)(t - (int64_t)tr * C.tilesC);
  const int tid = threadIdx.x;
  const int tx = tid % TPR, ty = tid / TPR;
  const int cl = 4 * tx;
  const int64_t r0 = (int64_t)tr * TR, c0 = (int64_t)tc * TC;
  const int e = *C.hint;
  const bool wr = exp_known(e);
  const float s2 = wr ? ldexpf(1.f, e) : 0.f;
  const bool full = (r0 + TR <= C.rows) && (c0 + TC <= C.cols);
  const bool vec = full && (C.cols % 4 == 0) && (((uintptr_t)C.mom & 15) == 0) &&
                   (((uintptr_t)C.grad & (GD == 1 ? 7 : 15)) == 0);
  float v[Q][4];
  float ss = 0.f;
  if (vec) {
    // every load of the tile is issued before the first store (g and M may
    // not be proven disjoint by the compiler)
    f32x4 mq[Q], gq[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int64_t ix = (r0 + ty + RPI * q) * C.cols + c0 + cl;
      gq[q] = load4<GD>(C.grad, ix);
      mq[q] = *(const f32x4*)(C.mom + ix);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const float mv = fmaf(L.beta, mq[q][c], gq[q][c]);
        mq[q][c] = mv;
        const float u = NEST ? fmaf(L.beta, mv, gq[q][c]) : mv;
        v[q][c] = u;
        ss += u * u;
      }
      *(f32x4*)(C.mom + (r0 + ty + RPI * q) * C.cols + c0 + cl) = mq[q];
    }
  } else {
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int64_t r = r0 + ty + RPI * q;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const int64_t cc = c0 + cl + c;
        float u = 0.f;
        if (r < C.rows && cc < C.cols) {
          const int64_t ix = r * C.cols + cc;
          const float gv = load_as_f32(C.grad, ix, GD);
          const float mv = fmaf(L.beta, C.mom[ix], gv);
          C.mom[ix] = mv;
          u = NEST ? fmaf(L.beta, mv, gv) : mv;
          ss += u * u;
        }
        v[q][c] = u;
      }
    }
  }
  ss = wave_sum(ss);
  if ((tid & 63) == 0) part[tid >> 6] = ss;
  if (wr) {
    if constexpr (TALL) {
#pragma unroll
      for (int q = 0; q < Q; ++q)
#pragma unroll
        for (int c = 0; c < 4; ++c) tile[ty + RPI * q][cl + c] = v[q][c] * s2;
    } else {
      _Float16* S = (_Float16*)C.xh;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        half4_t h;
#pragma unroll
        for (int c = 0; c < 4; ++c) h[c] = (_Float16)(v[q][c] * s2);
        *(half4_t*)(S + (r0 + ty + RPI * q) * C.cp + c0 + cl) = h;
      }
    }
  }
  __syncthreads();
  if (tid == 0) L.partials[C.partialOff + t] = part[0] + part[1] + part[2] + part[3];
  if constexpr (TALL) {
    if (!wr) return;
    // TC output rows of TR values: TR/8 runs of 8 per row
    constexpr int RUNS = TR / 8;
    _Float16* Tt = (_Float16*)C.xh;
#pragma unroll
    for (int p = 0; p < TC * RUNS / 256; ++p) {
      const int id = p * 256 + tid;
      const int cl2 = id / RUNS, rl0 = (id % RUNS) * 8;
      half8_t h;
#pragma unroll
      for (int k = 0; k < 8; ++k) h[k] = (_Float16)tile[rl0 + k][cl2];
      *(half8_t*)(Tt + (c0 + cl2) * C.rp + r0 + rl0) = h;
    }
  }
}

template <int GD, bool NEST>
__device__ __forceinline__ void momcast_any(const MomCastLaunch& L, const MomCastMat& C, int64_t t) {
  if (C.tall) momcast_tile<kFuseTallR, kFuseTallC, true, GD, NEST>(L, C, t);
  else momcast_tile<kFuseWideR, kFuseWideC, false, GD, NEST>(L, C, t);
}

__global__ __launch_bounds__(256) void momcast_kernel(const MomCastLaunch L) {
  const int64_t b = blockIdx.x;
  int mi = 0;
  while (mi + 1 < L.n && b >= L.mat[mi + 1].blockStart) ++mi;
  const MomCastMat& C = L.mat[mi];
  const int64_t t = b - C.blockStart;
  if (L.gradDtype == 1) {
    if (L.nesterov) momcast_any<1, true>(L, C, t);
    else momcast_any<1, false>(L, C, t);
  } else {
    if (L.nesterov) momcast_any<0, true>(L, C, t);
    else momcast_any<0, false>(L, C, t);
  }
}

hipError_t launch_momcast(const MomCastLaunch& L, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(momcast_kernel, dim3((unsigned)blocks), dim3(256), 0, st, L);
  return hipGetLastError();
}

hipError_t launch_ew(const EwLaunch& L, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(ew_kernel, dim3((unsigned)blocks), dim3(kEwThreads), 0, st, L);
  return hipGetLastError();
}

hipError_t launch_norm(const NormLaunch& L, hipStream_t st) {
  if (L.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(norm_kernel, dim3(L.n), dim3(256), 0, st, L);
  return hipGetLastError();
}

hipError_t launch_cast(const CastLaunch& L, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(cast_kernel, dim3((unsigned)blocks), dim3(256), 0, st, L);
  return hipGetLastError();
}

}  // namespace muon
