// Host planning for the batched Gram Newton–Schulz step (no HIP calls).
//
// Grouping follows DMuon's technical summary (gist.science, Korean), §2.2:
// matrices of similar shape are batched so that one dispatch serves all of
// them.  Here the Gram-space state is grouped by m alone (the m×m recursion
// does not depend on n), while the products that touch the m×n operand
// (SYRK, final product) are grouped by stored shape.
#include "plan.hpp"

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <map>
#include <mutex>
#include <sstream>

#include "common.hpp"

namespace muon {

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Largest power of two s with s·bound ≤ 2^13, so that every stored operand
// stays 8× below the fp16 maximum (65504) even with rounding.
float pow2_scale(double bound) {
  if (!(bound > 0.0) || !std::isfinite(bound)) return 1.f;
  int e = (int)std::floor(std::log2(8192.0 / bound));
  e = std::max(-60, std::min(60, e));
  return std::ldexp(1.0f, e);
}

std::mutex g_table_mu;
std::map<TileKey, TileConf> g_table;

int choose_tile(int op, int64_t m, int count) {
  if (op == OP_F32) {
    // Small matrices: 32-tiles with the contraction split over four waves
    // (a quarter of a 64-tile wave's MFMAs per wave, four times the
    // workgroups).  Decided by m alone: the split changes the order of the
    // fp32 sums, and a chunked call must pick the tiles one plan would.
    if (m <= 256) return 32;
    // fp32 products are latency-bound for small groups: 64-tiles give four
    // times the workgroups when 128-tiles would not fill the 256 CUs twice
    // (both kernels add each element's products in the same order).
    const int64_t t = (m + 127) / 128;
    return double(count) * double(t * (t + 1) / 2) < 512.0 ? 64 : 128;
  }
  // The 256-tile kernel (direct-to-LDS ring, staged epilogues) is several
  // times faster per tile than the register-staged 128-tile kernel, which
  // outweighs the padding of m up to a multiple of 256 and a partly filled
  // last wave, down to the smallest Gram sizes (measured: 32 × 1024×4096 in
  // 2.6 ms vs 3.6 ms, the 176-matrix small mix — m = 64 … 512 — in 1.34 ms
  // vs 1.73 ms).
  (void)m;
  return 256;
}

}  // namespace

int count_class(int count) {
  int c = 0;
  while (count > 1) {
    count >>= 1;
    ++c;
  }
  return c;
}

void set_tile_table(const std::vector<std::pair<TileKey, TileConf>>& entries) {
  std::lock_guard<std::mutex> lk(g_table_mu);
  g_table.clear();
  for (const auto& e : entries) g_table[e.first] = e.second;
}

TileConf conf_from_table(int64_t m, int64_t n, int op, int count) {
  std::lock_guard<std::mutex> lk(g_table_mu);
  auto it = g_table.find(TileKey{m, n, op, count_class(count)});
  if (it == g_table.end()) it = g_table.find(TileKey{m, 0, op, count_class(count)});
  return it == g_table.end() ? TileConf{} : it->second;
}

int tile_override() {
  const char* s = std::getenv("MUON_TILE");
  if (!s) return 0;
  int v = std::atoi(s);
  return (v == 128 || v == 256) ? v : 0;
}

ScalePlan make_scales(int op, int steps, double a, double b, double c) {
  ScalePlan sp;
  sp.sA.assign(std::max(steps, 1), 1.f);
  sp.sB.assign(std::max(steps, 1), 1.f);
  sp.sPA.assign(std::max(steps, 1), 1.f);
  sp.sQ.assign(steps + 1, 1.f);
  if (op == OP_F32) return sp;
  // X₀ = M/(‖M‖_F + eps): every entry and every singular value is ≤ 1, so the
  // eigenvalues of A₀ = X₀X₀ᵀ lie in [0, 1].  Each iterate is a polynomial in
  // A₀, so its eigenvalues follow from the scalar maps below; for a symmetric
  // matrix |entry| ≤ spectral norm, which bounds what the fp16 copy stores.
  const double safety = 1.25;
  const int N = 4096;
  double L = 1.0;   // bound on eigenvalues of A_k
  double Q = 1.0;   // bound on eigenvalues of Q_k
  sp.sX = pow2_scale(1.0 * safety);
  sp.sQ[0] = pow2_scale(Q * safety);
  for (int k = 0; k < steps; ++k) {
    double bmax = 0, pmax = 0, pamax = 0, lnext = 0;
    for (int i = 0; i <= N; ++i) {
      const double lam = L * i / N;
      const double beta = b * lam + c * lam * lam;
      const double p = a + beta;
      bmax = std::max(bmax, std::fabs(beta));
      pmax = std::max(pmax, std::fabs(p));
      pamax = std::max(pamax, std::fabs(lam * p));
      lnext = std::max(lnext, lam * p * p);
    }
    sp.sA[k] = pow2_scale(L * safety);
    sp.sB[k] = pow2_scale(bmax * safety);
    sp.sPA[k] = pow2_scale(pamax * safety);
    Q *= pmax;
    sp.sQ[k + 1] = pow2_scale(Q * safety);
    L = lnext;
  }
  return sp;
}

std::string build_plan(const int64_t* rows, const int64_t* cols, int count, int op, int steps,
                       float a, float b, float c, bool forStep, Plan* plan) {
  Plan& P = *plan;
  P = Plan();
  P.op = op;
  P.steps = steps;
  P.forStep = forStep;
  P.a = a;
  P.b = b;
  P.c = c;
  P.mats.resize(count);
  auto esz_of = [](int o) -> size_t { return o == OP_F32 ? 4 : 2; };

  // buckets keyed by stored shape, groups keyed by m; both in order of first
  // appearance so the plan is a pure function of the shape list.
  std::map<std::pair<int64_t, int64_t>, int> bucketOf;
  std::map<std::pair<int64_t, int>, int> groupOf;  // (m, op)
  for (int i = 0; i < count; ++i) {
    MatPlan& mp = P.mats[i];
    mp.rows = rows[i];
    mp.cols = cols[i];
    mp.numel = mp.rows * mp.cols;
    mp.empty = (mp.rows == 0 || mp.cols == 0);
    if (mp.empty) continue;
    mp.tall = mp.rows > mp.cols;
    mp.m = std::min(mp.rows, mp.cols);
    mp.n = std::max(mp.rows, mp.cols);
    auto key = std::make_pair(mp.rows, mp.cols);
    auto it = bucketOf.find(key);
    if (it == bucketOf.end()) {
      BucketPlan bp;
      bp.rows = mp.rows;
      bp.cols = mp.cols;
      bp.m = mp.m;
      bp.n = mp.n;
      bp.tall = mp.tall;
      bp.op = (op == OP_F32 || needs_f32(bp.m, bp.n)) ? OP_F32 : OP_F16;
      it = bucketOf.emplace(key, (int)P.buckets.size()).first;
      P.buckets.push_back(bp);
    }
    mp.bucket = it->second;
    mp.posBucket = (int)P.buckets[mp.bucket].mats.size();
    P.buckets[mp.bucket].mats.push_back(i);
  }
  for (int bi = 0; bi < (int)P.buckets.size(); ++bi) {
    BucketPlan& bp = P.buckets[bi];
    const auto gkey = std::make_pair(bp.m, bp.op);
    auto it = groupOf.find(gkey);
    if (it == groupOf.end()) {
      GroupPlan gp;
      gp.m = bp.m;
      gp.op = bp.op;
      it = groupOf.emplace(gkey, (int)P.groups.size()).first;
      P.groups.push_back(gp);
    }
    GroupPlan& gp = P.groups[it->second];
    bp.group = it->second;
    bp.gramStart = gp.count;
    gp.count += (int)bp.mats.size();
    gp.buckets.push_back(bi);
  }
  for (GroupPlan& gp : P.groups) {
    // For nearly square matrices (smallest singular values near zero) fp16
    // operands lose the relative accuracy of the small eigenvalues of A
    // unless the a·A terms of the A-chain are carried in fp32; only the
    // 128-tile kernel carries that state.  Wide matrices (n > 2m) are well
    // conditioned and run state-free.
    bool nearSquare = false;
    for (int bi : gp.buckets) {
      nearSquare |= P.buckets[bi].n <= 2 * P.buckets[bi].m;
      gp.nMax = std::max(gp.nMax, P.buckets[bi].n);
    }
    gp.state32 = (gp.op == OP_F16) && gp.m <= kState32MaxM && nearSquare;
    const TileConf tc = conf_from_table(gp.m, gp.nMax, gp.op, gp.count);
    const int ov = gp.op == OP_F16 ? tile_override() : 0;
    gp.tile = gp.state32 ? 128 : tc.tile ? tc.tile : ov ? ov : choose_tile(gp.op, gp.m, gp.count);
    gp.xcdShift = tc.xcdShift;
    gp.band = tc.band;
    gp.Mp = round_up(gp.m, std::max(gp.tile, kCastTile));  // the cast pads in 64×64 tiles
  }
  for (BucketPlan& bp : P.buckets) {
    const GroupPlan& gp = P.groups[bp.group];
    bp.Mp = gp.Mp;
    bp.Np = round_up(bp.n, std::max(gp.tile, kCastTile));
    for (int k = 0; k < (int)bp.mats.size(); ++k) {
      MatPlan& mp = P.mats[bp.mats[k]];
      mp.group = bp.group;
      mp.posGroup = bp.gramStart + k;
    }
  }

  int rpos = 0;
  for (BucketPlan& bp : P.buckets) {
    bp.fusable = forStep && bp.op == OP_F16 && P.groups[bp.group].tile == 256;
    bp.rhoStart = rpos;
    for (int k = 0; k < (int)bp.mats.size(); ++k) P.mats[bp.mats[k]].rhoPos = rpos + k;
    rpos += (int)bp.mats.size();
  }

  // partial sums of squares: one per elementwise workgroup (flat pass) or
  // per 64×64 tile (fused pass)
  int64_t np = 0;
  for (MatPlan& mp : P.mats) {
    if (mp.empty) continue;
    mp.partialOff = np;
    mp.partialCnt = (mp.numel + kEwElems - 1) / kEwElems;
    const BucketPlan& bp = P.buckets[mp.bucket];
    if (bp.fusable)
      mp.tileCnt = mp.tall ? (bp.Np / kFuseTallR) * (bp.Mp / kFuseTallC)
                           : (bp.Mp / kFuseWideR) * (bp.Np / kFuseWideC);
    np += std::max(mp.partialCnt, mp.tileCnt);
  }
  P.totalPartials = np;

  size_t off = 0;
  P.offPartials = off;
  off = align_up(off + size_t(np) * 4);
  P.offAlpha = off;
  off = align_up(off + size_t(count) * 4);
  P.offRho = off;
  off = align_up(off + size_t(count) * 4);
  P.offOk = off;
  off = align_up(off + size_t(count) * 4);
  for (GroupPlan& gp : P.groups) {
    gp.strideh = size_t(gp.Mp) * size_t(gp.Mp) * esz_of(gp.op);
    const size_t nh = gp.strideh * gp.count;
    gp.offAh = off;   off = align_up(off + nh);
    gp.offBh = off;   off = align_up(off + nh);
    gp.offPAh = off;  off = align_up(off + nh);
    gp.offQh[0] = off; off = align_up(off + nh);
    gp.offQh[1] = off; off = align_up(off + nh);
    if (gp.state32) {
      gp.stride32 = size_t(gp.Mp) * size_t(gp.Mp) * 4;
      gp.offA32 = off;  off = align_up(off + gp.stride32 * gp.count);
      gp.offPA32 = off; off = align_up(off + gp.stride32 * gp.count);
    }
  }
  for (BucketPlan& bp : P.buckets) {
    bp.strideX = size_t(bp.Mp) * size_t(bp.Np) * esz_of(bp.op);
    bp.xT = P.groups[bp.group].tile != 256;
    bp.offXh = off;  off = align_up(off + bp.strideX * bp.mats.size());
    if (bp.xT) {
      bp.offXTh = off; off = align_up(off + bp.strideX * bp.mats.size());
    }
  }
  P.totalBytes = off;
  // Power-of-two scales are exact in fp32 too, so fp32 groups of a
  // half-precision plan share its scales.
  P.scales = make_scales(op, steps, a, b, c);
  return std::string();
}

std::string Plan::json() const {
  std::ostringstream o;
  o.precision(9);
  o << "{\"op\":\"" << (op == OP_F32 ? "f32" : "f16") << "\",\"steps\":" << steps
    << ",\"for_step\":" << (forStep ? 1 : 0) << ",\"workspace_bytes\":" << totalBytes
    << ",\"partials\":" << totalPartials << ",\"sX\":" << scales.sX << ",\"groups\":[";
  for (size_t g = 0; g < groups.size(); ++g) {
    const GroupPlan& gp = groups[g];
    o << (g ? "," : "") << "{\"m\":" << gp.m << ",\"n_max\":" << gp.nMax << ",\"Mp\":" << gp.Mp
      << ",\"tile\":" << gp.tile << ",\"xcd_window\":" << (1 << (gp.xcdShift ? gp.xcdShift : 5))
      << ",\"band\":" << (gp.band ? gp.band : 4)
      << ",\"op\":\"" << (gp.op == OP_F32 ? "f32" : "f16") << "\""
      << ",\"state32\":" << (gp.state32 ? "true" : "false")
      << ",\"count\":" << gp.count << ",\"buckets\":[";
    for (size_t k = 0; k < gp.buckets.size(); ++k) o << (k ? "," : "") << gp.buckets[k];
    o << "],\"offAh\":" << gp.offAh << ",\"offBh\":" << gp.offBh << ",\"offPAh\":" << gp.offPAh
      << ",\"offQh\":[" << gp.offQh[0] << "," << gp.offQh[1] << "],\"strideh\":" << gp.strideh
      << "}";
  }
  o << "],\"buckets\":[";
  for (size_t bi = 0; bi < buckets.size(); ++bi) {
    const BucketPlan& bp = buckets[bi];
    o << (bi ? "," : "") << "{\"rows\":" << bp.rows << ",\"cols\":" << bp.cols << ",\"m\":" << bp.m
      << ",\"n\":" << bp.n << ",\"tall\":" << (bp.tall ? "true" : "false") << ",\"op\":\""
      << (bp.op == OP_F32 ? "f32" : "f16") << "\",\"x_transposed_copy\":" << (bp.xT ? "true" : "false")
      << ",\"group\":"
      << bp.group << ",\"Mp\":" << bp.Mp << ",\"Np\":" << bp.Np << ",\"gram_start\":"
      << bp.gramStart << ",\"fusable\":" << (bp.fusable ? "true" : "false")
      << ",\"rho_start\":" << bp.rhoStart << ",\"mats\":[";
    for (size_t k = 0; k < bp.mats.size(); ++k) o << (k ? "," : "") << bp.mats[k];
    o << "]}";
  }
  o << "],\"mats\":[";
  for (size_t i = 0; i < mats.size(); ++i) {
    const MatPlan& mp = mats[i];
    o << (i ? "," : "") << "{\"empty\":" << (mp.empty ? "true" : "false") << ",\"bucket\":" << mp.bucket
      << ",\"partial_off\":" << mp.partialOff << ",\"partial_cnt\":" << mp.partialCnt
      << ",\"tile_cnt\":" << mp.tileCnt << ",\"rho_pos\":" << mp.rhoPos << "}";
  }
  o << "],\"scales\":{\"sA\":[";
  for (size_t k = 0; k < scales.sA.size(); ++k) o << (k ? "," : "") << scales.sA[k];
  o << "],\"sB\":[";
  for (size_t k = 0; k < scales.sB.size(); ++k) o << (k ? "," : "") << scales.sB[k];
  o << "],\"sPA\":[";
  for (size_t k = 0; k < scales.sPA.size(); ++k) o << (k ? "," : "") << scales.sPA[k];
  o << "],\"sQ\":[";
  for (size_t k = 0; k < scales.sQ.size(); ++k) o << (k ? "," : "") << scales.sQ[k];
  o << "]}}";
  return o.str();
}

}  // namespace muon
