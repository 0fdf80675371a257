// Row/column-selected Muon step with error feedback on gfx950.
//
// Dion3 review (blog.secrett2633.cloud), §3 "Method & Key Results": the update
// rule uses only part of the rows / columns of the momentum matrix, which
// shrinks the orthogonalisation; §1 "Key Terms & Definitions", Error
// Feedback: what a reduced-size update leaves out is carried into later
// steps.  Per matrix, with m = min(rows, cols) and the oriented m×n view
// (stored rows of a wide or square matrix, stored columns of a tall one):
//
//   B = M + g                       (one pass, with the squared ℓ2 norm of
//                                     every oriented row as its score)
//   S = the k = ⌈ρ·m⌉ highest scores, equal scores to the lower index
//   X_S = B restricted to S          (gathered into a dense fp32 block)
//   O_S = NS(X_S / (‖X_S‖_F + eps))  (the batched Gram pipeline, in place;
//                                     ‖X_S‖²_F is the sum of the selected
//                                     scores, so it needs no pass of its own)
//   W_S ← round(W_S − lr·√max(1, rows/cols)·O_S),  M_S ← β·B_S,
//   M elsewhere keeps B (the error that later steps pick up).
//
// The passes here are HBM-bound; the top-k is one workgroup per matrix and
// works on at most 32768 scores: an MSB-first 8-bit radix select over the
// fp32 bit patterns (non-negative floats order like their bits) finds the
// k-th largest score exactly, then two block-wide scans write the selected
// indices in ascending order.  Integer counts only, so the selection is
// deterministic.
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "launch.hpp"

namespace muon {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sel_wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ uint16_t to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ int find_mat(const SelLaunch& L, int64_t b) {
  int mi = 0;
  while (mi + 1 < L.n && b >= L.mat[mi + 1].blockStart) ++mi;
  return mi;
}

// ---------------------------------------------------------------------------
// B = M + g and the row scores.
//  * wide / square (rows ≤ cols): one wave per stored row, 16-byte accesses
//    when allowed, lane sums then a wavefront butterfly → score[row];
//  * tall: a workgroup covers 256 stored columns (4 per lane; 64 without
//    16-byte alignment) of a chunk of kSelChunk rows, each wave a quarter of
//    the rows, so a wave reads 1 KiB contiguous per row → score[chunk·m +
//    col]; the top-k kernel adds the chunks in order.
__global__ __launch_bounds__(kSelThreads) void sel_accum_kernel(const SelLaunch L) {
  const int64_t b = blockIdx.x;
  const SelMat& S = L.mat[find_mat(L, b)];
  const int64_t blk = b - S.blockStart;
  const int tid = threadIdx.x, lane = tid & 63;
  if (!S.tall) {
    const int64_t r = blk * (kSelThreads / 64) + (tid >> 6);
    if (r >= S.rows) return;  // whole wave: no cross-lane work follows
    const float* g = S.g + r * S.cols;
    float* mo = S.mom + r * S.cols;
    float ss = 0.f;
    if (L.vec) {
      for (int64_t c0 = (int64_t)lane * 4; c0 < S.cols; c0 += 4 * 256) {
        f32x4 gv[4], mv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = c0 + q * 256;
          if (c < S.cols) {
            gv[q] = __builtin_nontemporal_load((const f32x4*)(g + c));
            mv[q] = *(const f32x4*)(mo + c);
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = c0 + q * 256;
          if (c < S.cols) {
            const f32x4 v = mv[q] + gv[q];
            *(f32x4*)(mo + c) = v;
            ss += v[0] * v[0];
            ss += v[1] * v[1];
            ss += v[2] * v[2];
            ss += v[3] * v[3];
          }
        }
      }
    } else {
      for (int64_t c = lane; c < S.cols; c += 64) {
        const float v = mo[c] + g[c];
        mo[c] = v;
        ss += v * v;
      }
    }
    ss = sel_wave_sum(ss);
    if (lane == 0) S.score[r] = ss;
  } else {
    // V consecutive columns per lane (16-byte accesses when allowed); the
    // four waves take rows r0 + w, r0 + w + 4, … of the chunk and their sums
    // are added in wave order through LDS.
    const int V = L.vec ? 4 : 1;
    const int64_t span = 64 * V;
    const int64_t colBlocks = (S.cols + span - 1) / span;
    const int64_t chunk = blk / colBlocks;
    const int64_t c = (blk - chunk * colBlocks) * span + (int64_t)lane * V;
    const int w = tid >> 6;
    const int64_t r0 = chunk * kSelChunk;
    const int64_t r1 = r0 + kSelChunk < S.rows ? r0 + kSelChunk : S.rows;
    __shared__ f32x4 part[kSelThreads / 64][64];
    f32x4 ss = {0.f, 0.f, 0.f, 0.f};
    if (c < S.cols) {
      if (V == 4) {
        for (int64_t rb = r0 + w; rb < r1; rb += 16) {
          f32x4 gv[4], mv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (rb + 4 * q < r1) {
              gv[q] = __builtin_nontemporal_load((const f32x4*)(S.g + (rb + 4 * q) * S.cols + c));
              mv[q] = *(const f32x4*)(S.mom + (rb + 4 * q) * S.cols + c);
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (rb + 4 * q < r1) {
              const f32x4 v = mv[q] + gv[q];
              *(f32x4*)(S.mom + (rb + 4 * q) * S.cols + c) = v;
              ss[0] += v[0] * v[0];
              ss[1] += v[1] * v[1];
              ss[2] += v[2] * v[2];
              ss[3] += v[3] * v[3];
            }
          }
        }
      } else {
        for (int64_t rb = r0 + w; rb < r1; rb += 16) {
          float gv[4], mv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (rb + 4 * q < r1) {
              gv[q] = __builtin_nontemporal_load(S.g + (rb + 4 * q) * S.cols + c);
              mv[q] = S.mom[(rb + 4 * q) * S.cols + c];
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (rb + 4 * q < r1) {
              const float v = mv[q] + gv[q];
              S.mom[(rb + 4 * q) * S.cols + c] = v;
              ss[0] += v * v;
            }
          }
        }
      }
    }
    part[w][lane] = ss;
    __syncthreads();
    if (w == 0 && c < S.cols) {
      const f32x4 t = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
      float* dst = S.score + chunk * S.m + c;
      if (V == 4) *(f32x4*)dst = t;
      else dst[0] = t[0];
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k: one workgroup of 1024 threads per matrix; thread t owns the
// contiguous scores [t·per, t·per + per), per = ⌈m / 1024⌉ ≤ 32.

// Exclusive prefix sum of one int per thread over the workgroup, in thread
// order.  `sh` holds one slot per wave.
__device__ __forceinline__ int block_exclusive_scan(int v, int* sh) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) sh[w] = x;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < w; ++i) base += sh[i];
  __syncthreads();  // sh is reused by the next scan
  return base + x - v;
}

__global__ __launch_bounds__(kSelTopThreads) void sel_topk_kernel(const SelLaunch L) {
  const SelMat& S = L.mat[blockIdx.x];
  const int tid = threadIdx.x;
  const int m = S.m;
  const int per = (m + kSelTopThreads - 1) / kSelTopThreads;
  const int j0 = tid * per;
  const int cnt = m - j0 < 0 ? 0 : (m - j0 < per ? m - j0 : per);

  // A key is the sum of its chunk partials (one chunk for a wide matrix), in
  // eight interleaved running sums added in a fixed tree at the end, so
  // eight loads are in flight per thread.
  uint32_t key[kSelMaxPer];
#pragma unroll
  for (int q = 0; q < kSelMaxPer; ++q) {
    float s = 0.f;
    if (q < cnt) {
      const float* sp = S.score + j0 + q;
      float a[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      int c = 0;
      for (; c + 8 <= S.nChunks; c += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) a[u] += sp[(int64_t)(c + u) * m];
      }
      for (; c < S.nChunks; ++c) a[0] += sp[(int64_t)c * m];
      s = ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
    }
    key[q] = __float_as_uint(s);
  }

  __shared__ uint32_t hist[256];
  __shared__ uint32_t shPrefix, shKrem;
  __shared__ int shScan[kSelTopThreads / 64];
  __shared__ uint32_t shOr[kSelTopThreads / 64], shAnd[kSelTopThreads / 64];
  // Scores of one matrix usually share their top byte (sign and high
  // exponent bits), which would send every key of the first pass to one
  // histogram bin; a byte common to all keys is taken without a pass (it
  // changes neither the prefix's rank nor krem).
  uint32_t kor = 0u, kand = 0xffffffffu;
#pragma unroll
  for (int q = 0; q < kSelMaxPer; ++q)
    if (q < cnt) {
      kor |= key[q];
      kand &= key[q];
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    kor |= (uint32_t)__shfl_xor((int)kor, o, 64);
    kand &= (uint32_t)__shfl_xor((int)kand, o, 64);
  }
  if ((tid & 63) == 0) {
    shOr[tid >> 6] = kor;
    shAnd[tid >> 6] = kand;
  }
  __syncthreads();
  kor = 0u;
  kand = 0xffffffffu;
  for (int w = 0; w < kSelTopThreads / 64; ++w) {
    kor |= shOr[w];
    kand &= shAnd[w];
  }
  uint32_t prefix = 0, mask = 0, krem = (uint32_t)S.k;
  int pass0 = 0;
  if (((kor ^ kand) >> 24) == 0u) {
    prefix = kand & 0xff000000u;
    mask = 0xff000000u;
    pass0 = 1;
  }
  for (int pass = pass0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kSelMaxPer; ++q)
      if (q < cnt && (key[q] & mask) == prefix) atomicAdd(&hist[(key[q] >> shift) & 255u], 1u);
    __syncthreads();
    if (tid == 0) {
      // Largest digit d with (keys of digit > d) < krem ≤ (keys of digit ≥ d);
      // the keys matching the prefix number at least krem, so d exists.
      uint32_t above = 0;
      int d = 255;
      for (; d > 0; --d) {
        if (above + hist[d] >= krem) break;
        above += hist[d];
      }
      shPrefix = prefix | ((uint32_t)d << shift);
      shKrem = krem - above;
    }
    __syncthreads();
    prefix = shPrefix;
    krem = shKrem;
    mask |= 255u << shift;
  }
  // prefix is the k-th largest key T; krem of the keys equal to T are taken,
  // lowest indices first, together with every key above T.
  const uint32_t T = prefix;
  int eqc = 0;
#pragma unroll
  for (int q = 0; q < kSelMaxPer; ++q)
    if (q < cnt && key[q] == T) ++eqc;
  int eqSeen = block_exclusive_scan(eqc, shScan);
  uint32_t take = 0;
  int selc = 0;
#pragma unroll
  for (int q = 0; q < kSelMaxPer; ++q) {
    if (q < cnt) {
      bool t = key[q] > T;
      if (key[q] == T) {
        t = eqSeen < (int)krem;
        ++eqSeen;
      }
      if (t) {
        take |= 1u << q;
        ++selc;
      }
    }
  }
  int pos = block_exclusive_scan(selc, shScan);
  float tsum = 0.f;
#pragma unroll
  for (int q = 0; q < kSelMaxPer; ++q) {
    if (q < cnt) {
      const bool t = ((take >> q) & 1u) && pos < S.k;
      S.pos[j0 + q] = t ? pos : -1;
      if (t) {
        S.idx[pos++] = j0 + q;
        tsum += __uint_as_float(key[q]);
      }
    }
  }
  // ‖B_S‖²_F for the normalisation of the block: thread sums in index
  // order, then a fixed butterfly per wave and the waves in order.
  tsum = sel_wave_sum(tsum);
  __shared__ float shSum[kSelTopThreads / 64];
  if ((tid & 63) == 0) shSum[tid >> 6] = tsum;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int w = 0; w < kSelTopThreads / 64; ++w) t += shSum[w];
    *S.nsSum = t;
  }
}

// ---------------------------------------------------------------------------
// Gather, with the buffer's decay on the selection: one wave per row of the
// block; X_S takes B_S and the buffer keeps β·B_S there (the rows are read
// here anyway, so the decay costs only the write).
//  * wide: block row i = B row idx[i] (contiguous);
//  * tall: block row r = B row r at the columns idx[0..k) (ascending).
__global__ __launch_bounds__(kSelThreads) void sel_gather_kernel(const SelLaunch L) {
  const int64_t b = blockIdx.x;
  const SelMat& S = L.mat[find_mat(L, b)];
  const int64_t row = (b - S.blockStart) * (kSelThreads / 64) + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (!S.tall) {
    if (row >= S.k) return;
    float* src = S.mom + (int64_t)S.idx[row] * S.cols;
    float* dst = S.xs + row * S.cols;
    if (L.vec) {
      for (int64_t c0 = (int64_t)lane * 4; c0 < S.cols; c0 += 4 * 256) {
        f32x4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (c0 + q * 256 < S.cols) v[q] = *(const f32x4*)(src + c0 + q * 256);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = c0 + q * 256;
          if (c < S.cols) {
            *(f32x4*)(dst + c) = v[q];
            *(f32x4*)(src + c) = L.beta * v[q];
          }
        }
      }
    } else {
      for (int64_t c = lane; c < S.cols; c += 64) {
        const float v = src[c];
        dst[c] = v;
        src[c] = L.beta * v;
      }
    }
  } else {
    if (row >= S.rows) return;
    float* src = S.mom + row * S.cols;
    float* dst = S.xs + row * S.k;
    for (int i = lane; i < S.k; i += 64) {
      const int c = S.idx[i];
      const float v = src[c];
      dst[i] = v;
      src[c] = L.beta * v;
    }
  }
}

// ---------------------------------------------------------------------------
// Gather fused with the operand cast (blocks on the fp16 256-tile path).  The
// operand values are those the cast would write from the fp32 block: the
// same fp32 product v·(α·sX), rounded to fp16.
//  * wide: a wave per operand row i: row idx[i] of B for i < k (the buffer
//    decayed as it is read), zeros for the padding rows and columns;
//  * tall: the operand is the block's transpose; a 64×64 tile of (stored
//    rows, selections) is gathered — a wave reads 64 selected columns of one
//    row — staged in LDS (pitch 65) and written as 16-byte runs of 8
//    operand columns.
typedef _Float16 half4s __attribute__((ext_vector_type(4)));
typedef _Float16 half8s __attribute__((ext_vector_type(8)));

__global__ __launch_bounds__(kSelThreads) void sel_gather_cast_kernel(const SelCastLaunch L) {
  const int64_t b = blockIdx.x;
  int mi = 0;
  while (mi + 1 < L.n && b >= L.mat[mi + 1].blockStart) ++mi;
  const SelCastMat& S = L.mat[mi];
  const int64_t t = b - S.blockStart;
  const float scale = L.alpha[S.alphaIdx] * L.sX;
  const int tid = threadIdx.x, lane = tid & 63;
  if (!S.tall) {
    const int64_t i = t * (kSelThreads / 64) + (tid >> 6);
    if (i >= S.Mp) return;
    _Float16* dst = S.x0 + i * S.Np;
    if (i >= S.k) {
      for (int64_t c = (int64_t)lane * 8; c < S.Np; c += 512) *(half8s*)(dst + c) = half8s{};
      return;
    }
    float* src = S.mom + (int64_t)S.idx[i] * S.cols;
    if (L.vec) {
      for (int64_t c0 = (int64_t)lane * 4; c0 < S.Np; c0 += 4 * 256) {
        f32x4 v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = c0 + q * 256;
          v[q] = c < S.cols ? *(const f32x4*)(src + c) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = c0 + q * 256;
          if (c >= S.Np) continue;
          half4s h;
#pragma unroll
          for (int e = 0; e < 4; ++e) h[e] = (_Float16)(v[q][e] * scale);
          *(half4s*)(dst + c) = h;
          if (c < S.cols) *(f32x4*)(src + c) = L.beta * v[q];
        }
      }
    } else {
      for (int64_t c = lane; c < S.Np; c += 64) {
        const float v = c < S.cols ? src[c] : 0.f;
        dst[c] = (_Float16)(v * scale);
        if (c < S.cols) src[c] = L.beta * v;
      }
    }
    return;
  }
  __shared__ float tile[64][65];  // [selection][stored row]
  const int tilesN = S.Np / 64;
  const int64_t s0 = (t / tilesN) * 64, r0 = (t % tilesN) * 64;
  const int w = tid >> 6;
  const int64_t s = s0 + lane;
  const bool sel = s < S.k;
  const int64_t col = sel ? S.idx[s] : 0;
#pragma unroll 4
  for (int q = 0; q < 16; ++q) {
    const int64_t r = r0 + w + 4 * q;
    float v = 0.f;
    if (sel && r < S.rows) {
      float* p = S.mom + r * S.cols + col;
      v = *p;
      *p = L.beta * v;
    }
    tile[lane][w + 4 * q] = v * scale;
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int id = p * 256 + tid;
    const int sl = id >> 3, rl0 = (id & 7) * 8;
    half8s h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (_Float16)tile[sl][rl0 + e];
    *(half8s*)(S.x0 + (s0 + sl) * S.Np + r0 + rl0) = h;
  }
}

// ---------------------------------------------------------------------------
// Scatter: W_S ← round(W_S − lrsc·O_S), one wave per row of the block.
//  * wide: block row i → stored row idx[i], a contiguous row update;
//  * tall: block row r → stored row r at the selected columns.  The row is
//    walked densely through the inverse map (selected columns are spread
//    over every 64-byte segment, so a dense walk moves no more data than a
//    gather would, with full-width accesses); groups of 4 columns with no
//    selected column are skipped.
template <int PD>
__device__ __forceinline__ float w_load(const void* w, int64_t e) {
  if constexpr (PD == 1) return __uint_as_float((uint32_t)((const uint16_t*)w)[e] << 16);
  else return ((const float*)w)[e];
}
template <int PD>
__device__ __forceinline__ void w_store(void* w, int64_t e, float v) {
  if constexpr (PD == 1) ((uint16_t*)w)[e] = to_bf16_rne(v);
  else ((float*)w)[e] = v;
}

// Four consecutive weights at e (e % 4 == 0, aligned), widened to fp32.
template <int PD>
__device__ __forceinline__ f32x4 w_load4(const void* w, int64_t e) {
  f32x4 r;
  if constexpr (PD == 1) {
    const uint2 u = *(const uint2*)((const uint16_t*)w + e);
    r[0] = __uint_as_float(u.x << 16);
    r[1] = __uint_as_float(u.x & 0xffff0000u);
    r[2] = __uint_as_float(u.y << 16);
    r[3] = __uint_as_float(u.y & 0xffff0000u);
  } else {
    r = *(const f32x4*)((const float*)w + e);
  }
  return r;
}
template <int PD>
__device__ __forceinline__ void w_store4(void* w, int64_t e, f32x4 v) {
  if constexpr (PD == 1) {
    const uint32_t p0 = (uint32_t)to_bf16_rne(v[0]) | ((uint32_t)to_bf16_rne(v[1]) << 16);
    const uint32_t p1 = (uint32_t)to_bf16_rne(v[2]) | ((uint32_t)to_bf16_rne(v[3]) << 16);
    *(uint2*)((uint16_t*)w + e) = make_uint2(p0, p1);
  } else {
    *(f32x4*)((float*)w + e) = v;
  }
}

template <int PD>
__device__ __forceinline__ void scatter_row(const SelLaunch& L, const SelMat& S, int64_t row, int lane) {
  if (!S.tall) {
    const int64_t r = S.idx[row];
    const float* o = S.xs + row * S.cols;
    const int64_t wb = r * S.cols;
    if (L.vec) {
      // four 4-column groups per lane per iteration, every load first
      for (int64_t c0 = (int64_t)lane * 4; c0 < S.cols; c0 += 4 * 256) {
        f32x4 ov[4], wv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = c0 + q * 256;
          if (c < S.cols) {
            ov[q] = *(const f32x4*)(o + c);
            wv[q] = w_load4<PD>(S.w, wb + c);
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = c0 + q * 256;
          if (c < S.cols) {
#pragma unroll
            for (int e = 0; e < 4; ++e) wv[q][e] = fmaf(-S.lrsc, ov[q][e], wv[q][e]);
            w_store4<PD>(S.w, wb + c, wv[q]);
          }
        }
      }
    } else {
      for (int64_t c = lane; c < S.cols; c += 64)
        w_store<PD>(S.w, wb + c, fmaf(-S.lrsc, o[c], w_load<PD>(S.w, wb + c)));
    }
  } else {
    const float* o = S.xs + row * S.k;
    const int64_t wb = row * S.cols;
    if (L.vec) {
      for (int64_t c0 = (int64_t)lane * 4; c0 < S.cols; c0 += 4 * 256) {
        int4 p[4];
        f32x4 wv[4];
        bool any[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int64_t c = c0 + q * 256;
          any[q] = false;
          if (c < S.cols) {
            p[q] = *(const int4*)(S.pos + c);
            any[q] = (p[q].x & p[q].y & p[q].z & p[q].w) >= 0;  // some entry is not −1
          }
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (any[q]) wv[q] = w_load4<PD>(S.w, wb + c0 + q * 256);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (any[q]) {
            const int pp[4] = {p[q].x, p[q].y, p[q].z, p[q].w};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (pp[e] >= 0) wv[q][e] = fmaf(-S.lrsc, o[pp[e]], wv[q][e]);
            w_store4<PD>(S.w, wb + c0 + q * 256, wv[q]);
          }
        }
      }
    } else {
      for (int i = lane; i < S.k; i += 64) {
        const int64_t c = S.idx[i];
        w_store<PD>(S.w, wb + c, fmaf(-S.lrsc, o[i], w_load<PD>(S.w, wb + c)));
      }
    }
  }
}

__global__ __launch_bounds__(kSelThreads) void sel_scatter_kernel(const SelLaunch L) {
  const int64_t b = blockIdx.x;
  const SelMat& S = L.mat[find_mat(L, b)];
  const int64_t row = (b - S.blockStart) * (kSelThreads / 64) + (threadIdx.x >> 6);
  if (row >= (S.tall ? S.rows : (int64_t)S.k)) return;
  if (L.paramDtype == 1) scatter_row<1>(L, S, row, threadIdx.x & 63);
  else scatter_row<0>(L, S, row, threadIdx.x & 63);
}

}  // namespace

hipError_t launch_sel_accum(const SelLaunch& L, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(sel_accum_kernel, dim3((unsigned)blocks), dim3(kSelThreads), 0, st, L);
  return hipGetLastError();
}

hipError_t launch_sel_topk(const SelLaunch& L, hipStream_t st) {
  if (L.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(sel_topk_kernel, dim3((unsigned)L.n), dim3(kSelTopThreads), 0, st, L);
  return hipGetLastError();
}

hipError_t launch_sel_gather(const SelLaunch& L, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(sel_gather_kernel, dim3((unsigned)blocks), dim3(kSelThreads), 0, st, L);
  return hipGetLastError();
}

hipError_t launch_sel_gather_cast(const SelCastLaunch& L, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(sel_gather_cast_kernel, dim3((unsigned)blocks), dim3(kSelThreads), 0, st, L);
  return hipGetLastError();
}

hipError_t launch_sel_scatter(const SelLaunch& L, int64_t blocks, hipStream_t st) {
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(sel_scatter_kernel, dim3((unsigned)blocks), dim3(kSelThreads), 0, st, L);
  return hipGetLastError();
}

}  // namespace muon
