// Host-side planning: grouping of matrices, tile choice, padded sizes,
// workspace layout and the static power-of-two operand scales.  Pure C++,
// no HIP calls, so every part of it runs (and is tested) without a GPU.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <string>
#include <vector>

namespace muon {

struct MatPlan {
  int64_t rows = 0, cols = 0;  // stored shape
  int64_t m = 0, n = 0;        // Gram-space m ≤ n
  bool tall = false;           // rows > cols: processed as the transpose
  bool empty = false;
  int bucket = -1;             // index into Plan::buckets
  int posBucket = -1;
  int group = -1;              // index into Plan::groups
  int posGroup = -1;
  int64_t numel = 0;
  // partial sums of squares: partialCnt for the flat momentum / norm pass,
  // tileCnt (64×64 tiles of the padded stored matrix) for the fused
  // momentum + cast pass (fusable buckets only); max of both reserved
  int64_t partialOff = 0, partialCnt = 0, tileCnt = 0;
  int rhoPos = -1;             // position in bucket order (operand factor ρ)
};

// Matrices of one stored shape: they share the SYRK, cast and final launches.
struct BucketPlan {
  int64_t rows = 0, cols = 0, m = 0, n = 0;
  bool tall = false;
  int op = 0;               // OpType of this bucket's operand copies
  int group = -1;
  int64_t Mp = 0, Np = 0;   // padded m, n
  std::vector<int> mats;    // matrix indices in call order
  int gramStart = 0;        // position of mats[0] inside its group
  size_t offXh = 0;         // X₀  (Mp × Np), operand type
  size_t offXTh = 0;        // X₀ᵀ (Np × Mp), operand type; only when xT
  size_t strideX = 0;       // bytes per matrix of either buffer
  // The 128-tile kernel reads X₀ᵀ for the final product; the 256-tile kernel
  // reads X₀ through transposed panels, so its buckets keep X₀ alone.
  bool xT = true;
  // Step plans: fp16 operand on the 256-tile path (X₀ alone), so the
  // momentum pass can write the operand itself (carried exponents).
  bool fusable = false;
  int rhoStart = 0;         // bucket-order position of mats[0]
};

// Matrices of one Gram size m: they share every Gram-space launch.
struct GroupPlan {
  int64_t m = 0, Mp = 0;
  int64_t nMax = 0;         // largest n among the group's matrices (tuning key)
  int op = 0;               // OpType of the group's MFMA operands
  int tile = 128;
  int xcdShift = 0;         // launch tile order: log2 tiles per XCD run (0: default)
  int band = 0;             // launch tile order: tile rows per band (0: default)
  int count = 0;
  std::vector<int> buckets;
  // Gram-space iterates, operand type, scaled, full (mirrored) matrices.
  size_t offAh = 0, offBh = 0, offPAh = 0, offQh[2] = {0, 0};
  size_t strideh = 0;  // bytes per matrix
  // fp32 copies of A and P·A (upper triangle used) when state32.
  bool state32 = false;
  size_t offA32 = 0, offPA32 = 0;
  size_t stride32 = 0;
};

// Static operand scales (powers of two) for the half-precision path, derived
// from bounds on the spectra of the Gram-space iterates.
struct ScalePlan {
  float sX = 1.f;                  // X₀ (entries ≤ 1 after normalisation)
  std::vector<float> sA, sB, sPA;  // per step k: A_k, B_k, P_k·A_k
  std::vector<float> sQ;           // per step k: Q_k (k = 0..steps)
};

struct Plan {
  int op = 0;              // requested OpType (groups may use fp32, see below)
  int steps = 0;
  bool forStep = false;
  float a = 0, b = 0, c = 0;
  std::vector<MatPlan> mats;
  std::vector<BucketPlan> buckets;
  std::vector<GroupPlan> groups;
  size_t offPartials = 0;
  size_t offAlpha = 0;
  size_t offRho = 0;       // float per matrix, bucket order (fused operand factor ρ)
  size_t offOk = 0;        // int32 per matrix, call order (fused operand stands)
  int64_t totalPartials = 0;
  size_t totalBytes = 0;
  ScalePlan scales;
  std::string json() const;
};

// Environment override of the tile (MUON_TILE=128|256), 0 when unset.
int tile_override();

// Tuning table installed through the C ABI: (m, n, op, count class) →
// (tile, XCD run length, band).  n = 0 in a key matches any n; an entry for
// the group's own n (its largest matrix's) takes precedence.
struct TileKey {
  int64_t m, n;
  int op, countClass;
  bool operator<(const TileKey& o) const {
    if (m != o.m) return m < o.m;
    if (n != o.n) return n < o.n;
    return op != o.op ? op < o.op : countClass < o.countClass;
  }
};
struct TileConf {
  int tile = 0;      // 0: the built-in choice
  int xcdShift = 0;  // 0: the built-in 5 (32 tiles per XCD run)
  int band = 0;      // 0: the built-in 4
};
void set_tile_table(const std::vector<std::pair<TileKey, TileConf>>& entries);
TileConf conf_from_table(int64_t m, int64_t n, int op, int count);  // zeros when absent
int count_class(int count);

// Largest Gram size m that keeps fp32 state for the A-chain on the
// half-precision path, for groups holding nearly square matrices (n ≤ 2m).
constexpr int64_t kState32MaxM = 2048;

// Small, nearly square matrices run in fp32 MFMA even on the half-precision
// path: their smallest singular values sit near zero, where 5 quintic steps
// amplify input perturbations ≈ a⁵ ≈ 490×, and fp16 operands then miss the
// bf16 tolerance (measured 1–3% for 32–128 squares).  The fp32 products cost
// little at these sizes.
constexpr int64_t kF32NearSquareMaxM = 1024;
inline bool needs_f32(int64_t m, int64_t n) { return m <= kF32NearSquareMaxM && n <= 2 * m; }

// Build the plan.  `op` selects operand type (OP_F16 / OP_F32); with OP_F16
// the groups that needs_f32 selects use OP_F32.  Returns an empty string on
// success, else a message.
std::string build_plan(const int64_t* rows, const int64_t* cols, int count, int op, int steps,
                       float a, float b, float c, bool forStep, Plan* plan);

ScalePlan make_scales(int op, int steps, double a, double b, double c);

inline int64_t round_up(int64_t x, int64_t q) { return (x + q - 1) / q * q; }

}  // namespace muon
