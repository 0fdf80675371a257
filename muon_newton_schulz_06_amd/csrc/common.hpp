// Launch descriptors shared by the host sequencer and the gfx950 kernels.
//
// Every launch takes one of these structs by value (kernel arguments), so no
// descriptor table ever has to be copied to the device: matrices of a group
// sit at base + index * stride inside the workspace, and the few pointers the
// caller owns (gradients, momentum, weights, inputs, outputs) travel in
// fixed-size tables of at most kMaxUser entries per launch.
#pragma once

#include <stdint.h>

namespace muon {

constexpr int kMaxSegs = 4;   // problem groups served by one GEMM launch
constexpr int kMaxUser = 32;  // caller matrices per launch (kernel-arg tables)

enum OpType : int32_t { OP_F16 = 0, OP_F32 = 1 };

// Epilogues of the Gram-space products.  acc is the raw fp32 MFMA sum and u
// its unscale factor (operands are stored multiplied by powers of two).  An
// epilogue that needs the previous iterate Y reads it as in32[i][j] when the
// group keeps fp32 state for the A-chain (A and P·A), else as sIn·inh[i][j]
// from the scaled operand copy (on the 256-tile kernel: see ylam, ymu).
enum Epi : int32_t {
  // G = u·acc → outh = sOut·G (mirrored).
  // writeIdentity: also outhb = sOutB·I (zero steps: Q₀ = I).
  EPI_SYRK = 0,
  // A² = u·acc; B = p1·A + p2·A² (A from inh) → outh = sOut·B (mirrored).
  // If outhb: Q₁ = p0·I + B → outhb = sOutB·Q₁ (mirrored).
  EPI_SQ = 1,
  // Y' = p0·Y + u·acc (Y from inh) → outh = sOut·Y' (mirrored).
  EPI_AXPY = 2,
  // caller weights W ← round(decay·W − lrsc·u·acc), full tiles, real extent
  // only (decay = 1 − lr·weight_decay, exactly 1 without weight decay).
  EPI_UPDATE = 3,
  // caller output out = round(u·acc), full tiles, real extent only.
  EPI_OUT = 4,
};

struct GemmSeg {
  const void* A;       // operand rows of C: A[row * lda + k]
  const void* B;       // operand cols of C: B[col * ldb + k]
  int64_t strideA;     // elements between consecutive matrices
  int64_t strideB;
  int32_t lda, ldb;
  int32_t K;           // contraction length, a multiple of the k-tile
  int32_t tilesM;      // C tile rows per matrix
  int32_t tilesN;      // C tile cols per matrix
  int32_t tilesPerMat; // sym ? tilesM(tilesM+1)/2 : tilesM·tilesN
  int32_t count;       // matrices in this segment
  int32_t sym;         // 1: upper-triangle tiles only (C symmetric)
  int32_t epi;
  int32_t mReal;       // real C rows  (identity term, caller writes)
  int32_t nReal;       // real C cols
  int32_t ldc;         // row stride of the workspace C matrices
  int32_t writeIdentity;
  int32_t inIsB;       // inh is the B operand of this product (same matrix)
  float u, sOut, sOutB, sIn;
  float p0, p1, p2;
  const void* inh;     // previous iterate (operand copy), read at (i, j)
  int64_t strideInh;
  const float* in32;   // previous iterate in fp32 (upper triangle) or null
  int64_t strideIn32;
  float* out32;        // result in fp32 (upper triangle) or null
  int64_t strideOut32;
  void* outh;          // result copy, written mirrored
  int64_t strideOuth;
  void* outhb;         // second result copy (EPI_SQ first step, EPI_SYRK zero steps)
  int32_t userBase;    // first caller-table entry of this segment
  // 256-tile kernel only.  A symmetric matrix may be stored "block-upper":
  // only its 256×256 blocks (bi, bj) with bi ≤ bj are valid (diagonal blocks
  // in full).  An operand stored that way reads the k-tiles left of its
  // diagonal block transposed (rows k of the stored matrix).
  int32_t upperA, upperB;
  // symmetric outputs: 1 writes the tile and its mirror (full matrix),
  // 0 writes the tile only (block-upper, diagonal tiles in full)
  int32_t mirrorOut;
  // dense products: 1 reads every k-tile of A (B) transposed, i.e. A[i][k]
  // from row k of the stored matrix (X₀ for the final product)
  int32_t transA, transB;
  // 256-tile Gram-space products: the result is ylam·acc + ymu·Y (Y = inh
  // at the output position, as stored):
  //   EPI_AXPY: ylam = u,    ymu = p0·sIn
  //   EPI_SQ:   ylam = p2·u, ymu = p1·sIn (with p2 = 0 the launch has K = 0)
  float ylam, ymu;
  int32_t pad_;
  // Fused operands (muon_step with carried exponents): per matrix of the
  // segment, X₀ = rho[mat]·(the stored operand); the SYRK scales by rho²,
  // the final product by rho.  Null: 1.
  const float* rho;
};

struct GemmLaunch {
  int32_t nseg;
  int32_t userDtype;          // muon_dtype_t of the caller matrices
  float decay;                // EPI_UPDATE: factor applied to W before the update
  int32_t xcdShift;           // log2 of the logical tiles per XCD run (0: the default, 5)
  int32_t band;               // tile rows per band of the tile order (0: the default, 4)
  int32_t segStart[kMaxSegs + 1];  // prefix of workgroups per segment
  GemmSeg seg[kMaxSegs];
  void* user[kMaxUser];        // caller weights (EPI_UPDATE) or outputs (EPI_OUT)
  int64_t userLd[kMaxUser];
  float lrsc[kMaxUser];        // lr · √max(1, rows/cols) for EPI_UPDATE
};

// Momentum + sum of squares, or sum of squares alone.
constexpr int kEwThreads = 256;
constexpr int kEwElems = 4096;  // elements per workgroup (16 per thread)

struct EwMat {
  const void* x;       // gradient (momentum mode) or input (norm mode)
  float* mom;          // momentum, read + written (momentum mode)
  int64_t rows, cols, ld;
  int64_t numel;
  int64_t blockStart;  // first workgroup of this matrix in the launch
  int64_t partialOff;  // first partial sum of this matrix
};

struct EwLaunch {
  int32_t n;
  int32_t mode;        // 0: momentum, 1: sum of squares of x
  int32_t xDtype;      // muon_dtype_t of x (the gradient in momentum mode)
  int32_t vec;         // 1: every matrix contiguous (ld == cols) and 16-B aligned (momentum
                       //    mode: also numel % 4 == 0); partial blocks take the scalar path
  float beta;
  int32_t nesterov;    // momentum mode: Σ of (g + β·M')² instead of Σ M'²
  float* partials;
  EwMat mat[kMaxUser];
};

// Carried operand exponents (muon_step with scale_exp): a matrix whose
// momentum pass wrote its fp16 operand as u·2^e keeps that operand when
// ‖u‖·2^e lies in [2^kFuseLo, 2^kFuseHi]; the exponent written back for the
// next step puts ‖u‖·2^e in [2^12, 2^13).  Entries outside
// [-kFuseExpMax, kFuseExpMax] mean "unknown".
constexpr int kFuseLo = 9, kFuseHi = 14, kFuseTarget = 13, kFuseExpMax = 100;

struct NormLaunch {
  int32_t n;
  float eps;
  const float* partials;
  float* alpha;
  int64_t off[kMaxUser];
  int64_t cnt[kMaxUser];
  int32_t alphaIdx[kMaxUser];
  // fused operands (null hint: the matrix was not fused)
  float sX;                   // operand scale of the exact cast
  int32_t pad_;
  float* rho;                 // per matrix (rhoIdx): factor from the fused operand to X₀
  int32_t* ok;                // per matrix (alphaIdx): 1 when the fused operand stands
  int32_t* hint[kMaxUser];    // carried exponent, read and rewritten
  int32_t rhoIdx[kMaxUser];
};

// Cast (scaled) + transpose into the two operand layouts.
constexpr int kCastTile = 64;

struct CastMat {
  const void* src;     // stored rows × cols, row stride ld
  const void* grad;    // Nesterov input: gradient, same layout as src (else unused)
  void* S;             // same orientation, padded rp × cp (null: not written)
  void* T;             // transposed, padded cp × rp (null: not written)
  int64_t rows, cols, ld;
  int32_t rp, cp;      // padded extents (multiples of kCastTile)
  int32_t alphaIdx;
  int32_t tilesC;      // cp / kCastTile
  int64_t blockStart;
  int32_t okIdx;       // ≥ 0: skip the matrix when ok[okIdx] (its fused operand stands)
  int32_t pad_;
};

struct CastLaunch {
  int32_t n;
  int32_t srcDtype;    // muon_dtype_t
  int32_t outOp;       // OpType of S and T
  float sX;            // operand scale
  int32_t nesterov;    // 1: the value cast is g + β·src (src = M', g = grad)
  int32_t gradDtype;   // muon_dtype_t of grad
  float beta;
  int32_t pad_;
  const float* alpha;  // per-matrix 1 / (‖x‖_F + eps)
  const int32_t* ok;   // per-matrix flags written by the norm finish (fused operands)
  // 1: a small grid walks the tiles of every matrix whose fused operand
  // failed its check (okIdx ≥ 0 and !ok), skipping the others whole; the
  // matrices' blockStart is then the running sum of their tile counts
  int32_t strided;
  int32_t pad2_;
  CastMat mat[kMaxUser];
};

// Momentum fused with the operand cast: one tile of the stored matrix per
// workgroup, M ← β·M + g, the tile's Σu², and, when the matrix's carried
// exponent e is known, the fp16 operand u·2^e with its zero padding (stored
// layout for wide matrices, transposed for tall ones).  Wide matrices take
// 16×256 tiles (a wave reads 1 KiB of a row), tall ones 64×64 (the cast's
// tile: 128-byte rows of the transposed operand; 64×128 tiles, with twice
// the LDS per workgroup, measured 10% slower on the Qwen-shaped set).
constexpr int kFuseWideR = 16, kFuseWideC = 256, kFuseTallR = 64, kFuseTallC = 64;

struct MomCastMat {
  const void* grad;     // stored rows × cols, contiguous
  float* mom;           // momentum, read + written
  void* xh;             // fp16 operand X₀: rp × cp (wide) or cp × rp (tall), padded
  const int32_t* hint;  // carried exponent
  int64_t rows, cols;
  int32_t rp, cp;       // padded stored extents (multiples of 256)
  int32_t tilesC;       // cp / tile width
  int32_t tall;         // 1: X₀ is the transpose of the stored matrix
  int64_t blockStart;
  int64_t partialOff;   // one partial per tile
};

struct MomCastLaunch {
  int32_t n;
  int32_t gradDtype;    // muon_dtype_t
  int32_t nesterov;     // 1: u = g + β·M' (else u = M')
  float beta;
  float* partials;
  MomCastMat mat[kMaxUser];
};


// Row/column-selected step with error feedback: only the k = ⌈ρ·m⌉ highest-
// scoring rows of the oriented m×n buffer (stored rows of a wide matrix,
// stored columns of a tall one) are orthogonalised and applied.
constexpr int kSelThreads = 256;      // accumulate / gather / scatter: 4 waves
constexpr int kSelChunk = 256;        // stored rows per workgroup, column pass of a tall matrix
constexpr int kSelTopThreads = 1024;  // top-k: one workgroup per matrix
constexpr int kSelMaxPer = 32;        // scores per top-k thread (m ≤ 32768)

struct SelMat {
  const float* g;      // gradient, rows × cols
  float* mom;          // buffer, rows × cols; holds B = M + g after the first pass
  void* w;             // weights, rows × cols, param dtype
  float* xs;           // selected block, fp32: k × cols (wide) or rows × k (tall)
  float* score;        // partial scores, nChunks × m (nChunks = 1 for a wide matrix)
  int32_t* idx;        // the k selected indices along the short side, ascending
  int32_t* pos;        // inverse map, m entries: position in idx, or −1
  float* nsSum;        // Σ of the selected scores = ‖B_S‖²_F (the block's norm partial)
  int64_t rows, cols;
  int32_t m, k, tall, nChunks;
  int64_t blockStart;  // first workgroup of this matrix in the launch
  float lrsc;          // lr · √max(1, rows/cols)
  int32_t pad_;
};

struct SelLaunch {
  int32_t n;
  int32_t paramDtype;  // muon_dtype_t of the weights
  float beta;
  int32_t vec;         // 1: every matrix has cols % 4 == 0 and 4-element aligned rows
  SelMat mat[kMaxUser];
};

// Gather of the selected block fused with its operand cast (blocks whose
// Gram group runs fp16 on the 256-tile path): the operand X₀ = α·sX·B_S (the
// k selected rows of the oriented view) is written directly, padded to
// Mp × Np with zeros, and the buffer keeps β·B_S on S.  No fp32 copy of the
// block is made (the block's fp32 buffer then only receives the product).
struct SelCastMat {
  float* mom;           // B = M + g (rows × cols), decayed on S
  const int32_t* idx;   // the k selected indices along the short side, ascending
  _Float16* x0;         // operand: Mp × Np, row stride Np
  int64_t rows, cols;
  int32_t k, tall;
  int32_t Mp, Np;       // padded operand extents (multiples of 256)
  int32_t alphaIdx;     // α of the block (norm finish)
  int32_t pad_;
  int64_t blockStart;   // wide: Mp / 4 workgroups (a wave per operand row); tall: (Mp/64)·(Np/64) tiles
};
struct SelCastLaunch {
  int32_t n;
  float beta;
  float sX;
  int32_t vec;          // 1: cols % 4 == 0 and 16-byte aligned rows (wide blocks)
  const float* alpha;
  SelCastMat mat[kMaxUser];
};

}  // namespace muon
