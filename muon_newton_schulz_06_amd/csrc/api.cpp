// C ABI of the Muon / Gram Newton–Schulz library: argument checks, planning
// and the launch sequence on the caller's stream.
//
// Sequence for one call (all asynchronous on one stream):
//   1. momentum + partial Σx²   (muon_step)  |  partial Σx²  (muon_ns_batched)
//   2. α = 1/(‖·‖_F + eps) per matrix
//   3. X₀ = α·sX·x cast to the MFMA operand type, in both layouts
//   4. SYRK  G = X₀·X₀ᵀ, upper tiles, per stored shape
//   5. Gram recursion (DMuon technical summary, gist.science Korean, §2.2),
//      per step k with P_k = a·I + B_k, B_k = b·A_k + c·A_k²:
//        A_k² (epilogue forms B_k; at k = 0 also Q₁ = P₀)
//        Q_{k+1} = a·Q_k + B_k·Q_k  and  P_k·A_k = a·A_k + B_k·A_k  (one launch)
//        A_{k+1} = a·(P_k·A_k) + B_k·(P_k·A_k)
//      one launch per product serving every matrix of every Gram group.
//   6. O = Q_s·X₀ (X₀ᵀ·Q_s for tall matrices) with the output / weight
//      update fused in the epilogue.
//
// muon_step_selected (Dion3 review, §3 and §1 "Error Feedback") runs, per
// chunk of matrices: B = M + g with row scores, top-k (which also writes the
// block's Σx²), gather of the selected block with the buffer's β decay; then
// steps 2–6 above on the fp32 blocks (step 1 skipped), writing O_S in place;
// then the scatter of the weight update.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/muon_ns.h"
#include "common.hpp"
#include "launch.hpp"
#include "plan.hpp"

namespace muon {
namespace {

thread_local std::string g_err;
// Set by entry points that must not create HIP objects: no event pairs are
// recorded for their launches even while profiling is enabled.
thread_local bool g_no_events = false;

muon_status_t fail(muon_status_t st, const std::string& msg) {
  g_err = msg;
  return st;
}

// ----------------------------------------------------------------------------
// instrumentation: HIP event pairs around launches
struct ProfRec {
  int kind;
  hipEvent_t e0, e1;
  double work;
};
// Shared by every thread that calls the library: guarded by g_prof_mu.
std::atomic<bool> g_prof_on{false};
std::mutex g_prof_mu;
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t take_event() {  // g_prof_mu held
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// Debugging aid: with MUON_DEBUG_SYNC=1 in the environment every launch is
// followed by a synchronisation of its stream and an error check, so a
// failing kernel is named by muon_last_error().  Skipped while the stream is
// being captured into a graph (a synchronisation is not allowed there).
bool debug_sync() {
  const char* e = std::getenv("MUON_DEBUG_SYNC");
  return e && e[0] == '1';
}

// A launch recorded for later submission (see enqueue_lanes).
using Thunk = std::function<muon_status_t()>;

struct Launcher {
  hipStream_t st;
  // When set, launches are recorded here (with their stream) instead of
  // being made; the launch functors hold copies of their arguments.
  std::vector<Thunk>* defer = nullptr;
  template <typename F>
  muon_status_t run(int kind, double work, const char* what, F&& f) {
    if (defer) {
      const hipStream_t s0 = st;
      defer->push_back([s0, kind, work, what, f]() { return Launcher{s0}.run(kind, work, what, f); });
      return MUON_OK;
    }
    muon_status_t s = run_(kind, work, what, f);
    if (s != MUON_OK || !debug_sync()) return s;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return s;
    hipError_t e = hipStreamSynchronize(st);
    if (e == hipSuccess) e = hipGetLastError();
    if (e != hipSuccess)
      return fail(MUON_ERR_HIP, std::string(what) + " (debug synchronisation): " + hipGetErrorString(e));
    return s;
  }
  template <typename F>
  muon_status_t run_(int kind, double work, const char* what, F&& f) {
    hipEvent_t e0 = nullptr, e1 = nullptr;
    const bool prof = g_prof_on.load() && !g_no_events;
    if (prof) {
      std::lock_guard<std::mutex> lk(g_prof_mu);
      e0 = take_event();
      e1 = take_event();
    }
    if (e0) hipEventRecord(e0, st);
    hipError_t err = f();
    if (prof && e0 && e1) {
      hipEventRecord(e1, st);
      std::lock_guard<std::mutex> lk(g_prof_mu);
      g_prof.push_back({kind, e0, e1, work});
    } else if (prof) {
      std::lock_guard<std::mutex> lk(g_prof_mu);
      if (e0) g_event_pool.push_back(e0);
      if (e1) g_event_pool.push_back(e1);
    }
    if (err != hipSuccess)
      return fail(MUON_ERR_HIP, std::string(what) + ": " + hipGetErrorString(err));
    return MUON_OK;
  }
};

// ----------------------------------------------------------------------------
// argument checks (host only, before any HIP call)
struct Range {
  uintptr_t lo, hi;
  int owner;
};

bool overlaps(std::vector<Range> v, int* a, int* b) {
  std::sort(v.begin(), v.end(), [](const Range& x, const Range& y) { return x.lo < y.lo; });
  for (size_t i = 1; i < v.size(); ++i) {
    if (v[i].lo < v[i - 1].hi) {
      *a = v[i - 1].owner;
      *b = v[i].owner;
      return true;
    }
  }
  return false;
}

// The workspace must not overlap any caller tensor (it is scratch the
// kernels overwrite while the tensors are read).
bool workspace_overlaps(const std::vector<Range>& v, uintptr_t lo, uintptr_t hi, int* who) {
  for (const Range& r : v)
    if (r.lo < hi && lo < r.hi) {
      *who = r.owner;
      return true;
    }
  return false;
}

bool finite3(const float* c) {
  return c && std::isfinite(c[0]) && std::isfinite(c[1]) && std::isfinite(c[2]);
}

constexpr int64_t kMaxDim = int64_t(1) << 24;   // rows / cols
constexpr int64_t kMaxGramM = 32768;           // five m×m operand copies per matrix ≤ 10 GiB
constexpr int kMaxSteps = 64;

muon_status_t check_shape(int i, int64_t r, int64_t c) {
  if (r < 0 || c < 0)
    return fail(MUON_ERR_INVALID_ARG, "matrix " + std::to_string(i) + ": negative rows/cols");
  if (r > kMaxDim || c > kMaxDim)
    return fail(MUON_ERR_UNSUPPORTED, "matrix " + std::to_string(i) + ": rows/cols above 2^24");
  if (std::min(r, c) > kMaxGramM)
    return fail(MUON_ERR_UNSUPPORTED,
                "matrix " + std::to_string(i) + ": min(rows, cols) above 32768");
  return MUON_OK;
}

muon_status_t check_device() {
  int n = 0;
  if (hipGetDeviceCount(&n) != hipSuccess || n <= 0)
    return fail(MUON_ERR_NO_DEVICE, "no HIP device visible");
  return MUON_OK;
}

// ----------------------------------------------------------------------------
// launch sequence shared by both entry points

struct CallerMat {
  const void* src;   // momentum (step) or x (ns)
  int64_t ldSrc;
  void* dst;         // weights (step) or out (ns)
  int64_t ldDst;
  const void* grad;  // step only
  float lrsc;
  int32_t* hint = nullptr;  // step only: carried operand exponent (null: none)
};

// A bucket whose momentum pass writes the fp16 operand itself: fusable and
// every matrix of the call carries an exponent (a call passes all or none).
bool fused_bucket(const Plan& P, const BucketPlan& bp, const std::vector<CallerMat>& cm) {
  return P.forStep && bp.fusable && !bp.mats.empty() && cm[bp.mats[0]].hint != nullptr;
}

// Step options resolved on the host (defaults: the plain step).
struct StepVariant {
  int gradDtype = MUON_DTYPE_F32;
  int nesterov = 0;
  float decay = 1.f;  // 1 − lr·weight_decay
  // 1: each matrix's Σx² is already in its first partial (the selected
  // step's top-k writes it), so the sum-of-squares pass is skipped
  int presummed = 0;
  // passes enqueue_passes runs: bit 0 momentum / sum of squares, bit 1 norm
  // finish, bit 2 cast
  int stages = 7;
};

template <typename T>
T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

// Workgroups of the fallback cast of fused operands (it walks the tiles of
// the matrices that failed their check with a grid stride).
constexpr int64_t kCastFallbackBlocks = 1024;

// Steps 1–3 (HBM-bound passes): momentum / sum of squares, α, cast.
// The HBM-bound passes (momentum / sum of squares, norm finish, cast) over
// every matrix of the plan, or over the matrices `only` lists.
muon_status_t enqueue_passes(const Plan& P, const std::vector<CallerMat>& cm, int srcDtype,
                             float beta, float eps, const StepVariant& V, void* ws, hipStream_t st,
                             const std::vector<int>* only = nullptr,
                             std::vector<Thunk>* defer = nullptr) {
  Launcher Lr{st, defer};
  const int count = (int)P.mats.size();
  std::vector<int> live;
  if (only) {
    for (int i : *only)
      if (!P.mats[i].empty) live.push_back(i);
  } else {
    for (int i = 0; i < count; ++i)
      if (!P.mats[i].empty) live.push_back(i);
  }
  if (live.empty()) return MUON_OK;
  float* partials = at<float>(ws, P.offPartials);
  float* alpha = at<float>(ws, P.offAlpha);
  float* rho = at<float>(ws, P.offRho);
  int32_t* okf = at<int32_t>(ws, P.offOk);
  const ScalePlan& sc = P.scales;
  // matrices whose momentum pass also writes the operand (carried exponents)
  std::vector<char> fused(count, 0);
  std::vector<int> flat, fz;
  for (int i : live) {
    fused[i] = !V.presummed && fused_bucket(P, P.buckets[P.mats[i].bucket], cm);
    (fused[i] ? fz : flat).push_back(i);
  }

  // 1a. momentum fused with the cast (tiles of the padded stored matrix)
  for (size_t c0 = 0; c0 < ((V.stages & 1) ? fz.size() : 0); c0 += kMaxUser) {
    MomCastLaunch L;
    std::memset(&L, 0, sizeof(L));
    L.gradDtype = V.gradDtype;
    L.nesterov = V.nesterov;
    L.beta = beta;
    L.partials = partials;
    int64_t blocks = 0;
    double bytes = 0;
    const size_t cn = std::min(fz.size() - c0, (size_t)kMaxUser);
    for (size_t k = 0; k < cn; ++k) {
      const int i = fz[c0 + k];
      const MatPlan& mp = P.mats[i];
      const BucketPlan& bp = P.buckets[mp.bucket];
      MomCastMat& C = L.mat[k];
      C.grad = cm[i].grad;
      C.mom = (float*)cm[i].src;
      C.xh = at<char>(ws, bp.offXh + bp.strideX * mp.posBucket);
      C.hint = cm[i].hint;
      C.rows = mp.rows;
      C.cols = mp.cols;
      C.tall = mp.tall ? 1 : 0;
      C.rp = (int32_t)(mp.tall ? bp.Np : bp.Mp);
      C.cp = (int32_t)(mp.tall ? bp.Mp : bp.Np);
      C.tilesC = C.cp / (mp.tall ? kFuseTallC : kFuseWideC);
      C.blockStart = blocks;
      C.partialOff = mp.partialOff;
      blocks += mp.tileCnt;
      bytes += (V.gradDtype == MUON_DTYPE_BF16 ? 10.0 : 12.0) * mp.numel + 2.0 * (double)bp.Mp * (double)bp.Np;
    }
    L.n = (int)cn;
    muon_status_t s = Lr.run(0, bytes, "momentum + cast kernel", [=] { return launch_momcast(L, blocks, st); });
    if (s != MUON_OK) return s;
  }

  // 1b. momentum / sum of squares
  for (size_t c0 = 0; c0 < ((V.presummed || !(V.stages & 1)) ? 0 : flat.size()); c0 += kMaxUser) {
    EwLaunch L;
    std::memset(&L, 0, sizeof(L));
    L.mode = P.forStep ? 0 : 1;
    L.xDtype = P.forStep ? V.gradDtype : srcDtype;
    L.nesterov = P.forStep ? V.nesterov : 0;
    L.beta = beta;
    L.partials = partials;
    L.vec = 1;
    int64_t blocks = 0;
    double bytes = 0;
    const size_t cn = std::min(flat.size() - c0, (size_t)kMaxUser);
    for (size_t k = 0; k < cn; ++k) {
      const int i = flat[c0 + k];
      const MatPlan& mp = P.mats[i];
      EwMat& e = L.mat[k];
      e.rows = mp.rows;
      e.cols = mp.cols;
      e.numel = mp.numel;
      e.blockStart = blocks;
      e.partialOff = mp.partialOff;
      if (P.forStep) {
        e.x = cm[i].grad;
        e.mom = (float*)cm[i].src;
        e.ld = mp.cols;
        const uintptr_t galign = V.gradDtype == MUON_DTYPE_BF16 ? 7 : 15;
        if ((mp.numel & 3) || ((uintptr_t)e.x & galign) || ((uintptr_t)e.mom & 15)) L.vec = 0;
        bytes += (V.gradDtype == MUON_DTYPE_BF16 ? 10.0 : 12.0) * mp.numel;
      } else {
        e.x = cm[i].src;
        e.ld = cm[i].ldSrc;
        if (e.ld != mp.cols || ((uintptr_t)e.x & 15)) L.vec = 0;
        bytes += (srcDtype == MUON_DTYPE_BF16 ? 2.0 : 4.0) * mp.numel;
      }
      blocks += mp.partialCnt;
    }
    L.n = (int)cn;
    muon_status_t s = Lr.run(0, bytes, "momentum/norm kernel", [=] { return launch_ew(L, blocks, st); });
    if (s != MUON_OK) return s;
  }
  // 2. alpha
  for (size_t c0 = 0; c0 < ((V.stages & 2) ? live.size() : 0); c0 += kMaxUser) {
    NormLaunch L;
    std::memset(&L, 0, sizeof(L));
    L.eps = eps;
    L.partials = partials;
    L.alpha = alpha;
    L.sX = sc.sX;
    L.rho = rho;
    L.ok = okf;
    const size_t cn = std::min(live.size() - c0, (size_t)kMaxUser);
    double bytes = 0;
    for (size_t k = 0; k < cn; ++k) {
      const int i = live[c0 + k];
      const int64_t cnt = V.presummed ? 1 : fused[i] ? P.mats[i].tileCnt : P.mats[i].partialCnt;
      L.off[k] = P.mats[i].partialOff;
      L.cnt[k] = cnt;
      L.alphaIdx[k] = i;
      L.hint[k] = fused[i] ? cm[i].hint : nullptr;
      L.rhoIdx[k] = P.mats[i].rhoPos;
      bytes += 4.0 * cnt;
    }
    L.n = (int)cn;
    muon_status_t s = Lr.run(1, bytes, "norm finish kernel", [=] { return launch_norm(L, st); });
    if (s != MUON_OK) return s;
  }
  // 3. cast into both operand layouts (one launch sequence per operand type)
  // Fused matrices go through the strided fallback launch (a small grid that
  // casts only the matrices whose fused operand failed its check).
  for (int strided = 0; strided < ((V.stages & 4) ? 2 : 0); ++strided)
  for (int op : {(int)OP_F16, (int)OP_F32}) {
  std::vector<int> castMats;
  for (int i : (strided ? fz : flat))
    if (P.buckets[P.mats[i].bucket].op == op) castMats.push_back(i);
  const size_t esz = op == OP_F32 ? 4 : 2;
  for (size_t c0 = 0; c0 < castMats.size(); c0 += kMaxUser) {
    CastLaunch L;
    std::memset(&L, 0, sizeof(L));
    L.strided = strided;
    L.ok = okf;
    L.srcDtype = P.forStep ? MUON_DTYPE_F32 : srcDtype;
    L.outOp = op;
    L.sX = sc.sX;
    L.alpha = alpha;
    L.nesterov = P.forStep ? V.nesterov : 0;
    L.gradDtype = V.gradDtype;
    L.beta = beta;
    const size_t cn = std::min(castMats.size() - c0, (size_t)kMaxUser);
    int64_t blocks = 0;
    double bytes = 0;
    for (size_t k = 0; k < cn; ++k) {
      const int i = castMats[c0 + k];
      const MatPlan& mp = P.mats[i];
      const BucketPlan& bp = P.buckets[mp.bucket];
      CastMat& C = L.mat[k];
      C.src = cm[i].src;
      C.grad = cm[i].grad;
      C.rows = mp.rows;
      C.cols = mp.cols;
      C.ld = P.forStep ? mp.cols : cm[i].ldSrc;
      void* xh = at<char>(ws, bp.offXh + bp.strideX * mp.posBucket);
      void* xth = bp.xT ? at<char>(ws, bp.offXTh + bp.strideX * mp.posBucket) : nullptr;
      if (!mp.tall) {  // stored = X₀ (m × n)
        C.S = xh;
        C.T = xth;
        C.rp = (int32_t)bp.Mp;
        C.cp = (int32_t)bp.Np;
      } else {         // stored = X₀ᵀ (n × m)
        C.S = xth;
        C.T = xh;
        C.rp = (int32_t)bp.Np;
        C.cp = (int32_t)bp.Mp;
      }
      C.alphaIdx = i;
      C.okIdx = strided ? i : -1;
      C.tilesC = C.cp / kCastTile;
      C.blockStart = blocks;
      blocks += (int64_t)(C.rp / kCastTile) * C.tilesC;
      // the fallback moves nothing unless a check fails
      if (!strided) {
        bytes += (P.forStep ? 4.0 : (srcDtype == MUON_DTYPE_BF16 ? 2.0 : 4.0)) * mp.numel +
                 (bp.xT ? 2.0 : 1.0) * esz * (double)bp.Mp * (double)bp.Np;
        if (L.nesterov) bytes += (V.gradDtype == MUON_DTYPE_BF16 ? 2.0 : 4.0) * mp.numel;
      }
    }
    L.n = (int)cn;
    if (strided) blocks = std::min<int64_t>(blocks, kCastFallbackBlocks);
    muon_status_t s = Lr.run(2, bytes, "cast kernel", [=] { return launch_cast(L, blocks, st); });
    if (s != MUON_OK) return s;
  }
  }
  return MUON_OK;
}

// Steps 4–6 (MFMA products): SYRK, Gram recursion, final product + update.
// Relative cost of one matrix's step (SYRK, final product and the Gram
// products of five steps, in units of m²n and m³ multiply-adds).
double mat_work(int64_t r, int64_t c) {
  const double m = (double)std::min(r, c), n = (double)std::max(r, c);
  return 3.0 * m * m * n + 17.0 * m * m * m;
}

// The matrices one stream processes: pieces [b0, b1) of the plan's buckets
// (bucket-local positions).  A lane runs the whole product chain of its
// matrices; lanes share nothing but the plan's scales.
struct Piece {
  int bucket, b0, b1;
};
using Lane = std::vector<Piece>;

muon_status_t enqueue_lane(const Plan& P, const Lane& lane, const std::vector<CallerMat>& cm,
                           int dstDtype, const StepVariant& V, void* ws, hipStream_t st,
                           std::vector<Thunk>* defer = nullptr) {
  Launcher Lr{st, defer};
  const ScalePlan& sc = P.scales;
  // the lane's matrices of each group, as merged ranges of group positions
  std::vector<std::vector<std::pair<int, int>>> granges(P.groups.size());
  for (const Piece& pc : lane) {
    const BucketPlan& bp = P.buckets[pc.bucket];
    if (pc.b1 > pc.b0) granges[bp.group].push_back({bp.gramStart + pc.b0, bp.gramStart + pc.b1});
  }
  for (auto& r : granges) {
    std::sort(r.begin(), r.end());
    std::vector<std::pair<int, int>> merged;
    for (const auto& x : r) {
      if (!merged.empty() && merged.back().second == x.first) merged.back().second = x.second;
      else merged.push_back(x);
    }
    r.swap(merged);
  }
  // A Gram-space segment built at the group's base, emitted once per range
  // of the lane (every operand and result of these products is a group array).
  auto emit = [&](size_t gi, const GemmSeg& S0, std::vector<GemmSeg>& segs, std::vector<double>& works) {
    const GroupPlan& g = P.groups[gi];
    for (const auto& r : granges[gi]) {
      GemmSeg S = S0;
      const size_t oh = g.strideh * (size_t)r.first, o32 = g.stride32 * (size_t)r.first;
      S.A = static_cast<const char*>(S.A) + oh;
      S.B = static_cast<const char*>(S.B) + oh;
      if (S.inh) S.inh = static_cast<const char*>(S.inh) + oh;
      S.outh = static_cast<char*>(S.outh) + oh;
      if (S.outhb) S.outhb = static_cast<char*>(S.outhb) + oh;
      if (S.in32) S.in32 += o32 / sizeof(float);
      if (S.out32) S.out32 += o32 / sizeof(float);
      S.count = r.second - r.first;
      segs.push_back(S);
      works.push_back((double)S.count * g.m * g.m * (double)(g.m + 1));
    }
  };

  // Kernel configurations (tile, operand type, tile order) present, each
  // launched separately.
  struct Cfg {
    int tile, op, xcdShift, band;
    bool operator==(const Cfg& o) const {
      return tile == o.tile && op == o.op && xcdShift == o.xcdShift && band == o.band;
    }
    bool has(const GroupPlan& g) const { return *this == Cfg{g.tile, g.op, g.xcdShift, g.band}; }
  };
  std::vector<Cfg> cfgs;
  for (size_t gi = 0; gi < P.groups.size(); ++gi) {
    const GroupPlan& g = P.groups[gi];
    if (granges[gi].empty()) continue;
    const Cfg cf{g.tile, g.op, g.xcdShift, g.band};
    if (std::find(cfgs.begin(), cfgs.end(), cf) == cfgs.end()) cfgs.push_back(cf);
  }

  // Helper: launch a list of segments (≤ kMaxSegs per launch).
  auto launch_segs = [&](const Cfg& cf, std::vector<GemmSeg>& segs, std::vector<double>& works,
                         int kind, const char* what) -> muon_status_t {
    const int tile = cf.tile, op = cf.op;
    for (const GemmSeg& S : segs)
      if (tile == 256 && (S.in32 || S.out32))
        return fail(MUON_ERR_UNSUPPORTED, "internal: fp32 state on a 256-tile launch");
    for (size_t s0 = 0; s0 < segs.size(); s0 += kMaxSegs) {
      GemmLaunch L;
      std::memset(&L, 0, sizeof(L));
      L.decay = 1.f;
      const size_t ns = std::min(segs.size() - s0, (size_t)kMaxSegs);
      int blocks = 0;
      double work = 0;
      for (size_t k = 0; k < ns; ++k) {
        L.seg[k] = segs[s0 + k];
        L.segStart[k] = blocks;
        blocks += L.seg[k].tilesPerMat * L.seg[k].count;
        work += works[s0 + k];
      }
      L.segStart[ns] = blocks;
      L.nseg = (int)ns;
      L.xcdShift = cf.xcdShift;
      L.band = cf.band;
      int k = kind;
      if (kind == 4 && tile == 256) k = (L.seg[0].epi == EPI_AXPY) ? 6 : 7;
      muon_status_t s = Lr.run(k, work, what, [=] { return launch_gemm(op, tile, L, blocks, st); });
      if (s != MUON_OK) return s;
    }
    return MUON_OK;
  };

  auto sym_seg = [&](const GroupPlan& g, int tile) {
    GemmSeg S;
    std::memset(&S, 0, sizeof(S));
    const int t = (int)(g.Mp / tile);
    S.tilesM = S.tilesN = t;
    S.tilesPerMat = t * (t + 1) / 2;
    S.sym = 1;
    S.count = g.count;
    S.lda = S.ldb = S.ldc = (int32_t)g.Mp;
    S.K = (int32_t)g.Mp;
    S.strideA = S.strideB = g.Mp * g.Mp;
    S.strideInh = S.strideOuth = g.Mp * g.Mp;
    S.strideIn32 = S.strideOut32 = g.Mp * g.Mp;
    S.mReal = S.nReal = (int32_t)g.m;
    S.mirrorOut = 1;
    return S;
  };
  // On the 256-tile kernel every Gram-space iterate is stored block-upper
  // (tile only, no mirror) and read back through transposed panels; only
  // the last Q, which the final product reads as a dense operand, is
  // written in full.  The 128-tile kernel always works on full matrices.
  auto upper = [](GemmSeg& S, int tile, bool lastQ) {
    if (tile != 256) return;
    S.mirrorOut = lastQ ? 1 : 0;
  };
  auto upper_in = [](GemmSeg& S, int tile) {
    if (tile != 256) return;
    S.upperA = S.upperB = 1;
  };
  auto f32 = [&](const GroupPlan& g, size_t off) -> float* {
    return g.state32 ? at<float>(ws, off) : nullptr;
  };

  // 4. SYRK per stored shape
  for (const Cfg& cf : cfgs) {
    const int tile = cf.tile;
    std::vector<GemmSeg> segs;
    std::vector<double> works;
    for (const Piece& pc : lane) {
      const BucketPlan& bp = P.buckets[pc.bucket];
      const GroupPlan& g = P.groups[bp.group];
      if (!cf.has(g) || pc.b1 <= pc.b0) continue;
      const int pos = bp.gramStart + pc.b0;  // group position of the piece's first matrix
      {
        GemmSeg S = sym_seg(g, tile);
        S.count = pc.b1 - pc.b0;
        S.A = S.B = at<char>(ws, bp.offXh + bp.strideX * pc.b0);
        S.strideA = S.strideB = bp.Mp * bp.Np;
        S.lda = S.ldb = (int32_t)bp.Np;
        S.K = (int32_t)bp.Np;
        S.epi = EPI_SYRK;
        upper(S, tile, false);
        S.u = 1.0f / (sc.sX * sc.sX);
        if (fused_bucket(P, bp, cm)) S.rho = at<float>(ws, P.offRho) + bp.rhoStart + pc.b0;
        S.sOut = sc.sA[0];
        S.outh = at<char>(ws, g.offAh + g.strideh * pos);
        if (g.state32) S.out32 = at<float>(ws, g.offA32 + g.stride32 * pos);
        if (P.steps == 0) {
          S.writeIdentity = 1;
          S.outhb = at<char>(ws, g.offQh[0] + g.strideh * pos);
          S.sOutB = sc.sQ[0];
        }
        segs.push_back(S);
        works.push_back((double)S.count * bp.m * (double)(bp.m + 1) * bp.n);
      }
    }
    muon_status_t s = launch_segs(cf, segs, works, 3, "SYRK kernel");
    if (s != MUON_OK) return s;
  }

  // 5. Gram-space recursion.  Every product's previous iterate (the a·Y and
  // b·A terms) is its B operand, read back from the operand copy.
  const float a = P.a, b = P.b, c = P.c;
  int qcur = 0;  // Qh buffer holding the current Q
  for (int k = 0; k < P.steps; ++k) {
    const bool hasQ = k >= 1, hasA = k <= P.steps - 2;
    for (const Cfg& cf : cfgs) {
    const int tile = cf.tile;
      // (i) A² → B (and Q₁ at k = 0)
      std::vector<GemmSeg> segs;
      std::vector<double> works;
      for (size_t gi = 0; gi < P.groups.size(); ++gi) {
        const GroupPlan& g = P.groups[gi];
        if (!cf.has(g) || granges[gi].empty()) continue;
        GemmSeg S = sym_seg(g, tile);
        S.A = S.B = S.inh = at<char>(ws, g.offAh);
        S.in32 = f32(g, g.offA32);
        S.inIsB = 1;
        S.sIn = 1.0f / sc.sA[k];
        S.epi = EPI_SQ;
        upper_in(S, tile);
        upper(S, tile, k == 0 && P.steps == 1);  // Q₁ is written here and is last when s = 1
        S.u = 1.0f / (sc.sA[k] * sc.sA[k]);
        S.p0 = a;
        S.p1 = b;
        S.p2 = c;
        S.ylam = c * S.u;
        S.ymu = b * S.sIn;
        if (c == 0.f && tile == 256) S.K = 0;  // B = b·A: no product, a scaled copy
        S.outh = at<char>(ws, g.offBh);
        S.sOut = sc.sB[k];
        if (k == 0) {
          S.outhb = at<char>(ws, g.offQh[0]);
          S.sOutB = sc.sQ[1];
        }
        emit(gi, S, segs, works);
      }
      muon_status_t s = launch_segs(cf, segs, works, 4, "Gram A^2 kernel");
      if (s != MUON_OK) return s;
      // (ii) Q ← a·Q + B·Q and P·A = a·A + B·A
      segs.clear();
      works.clear();
      for (size_t gi = 0; gi < P.groups.size(); ++gi) {
        const GroupPlan& g = P.groups[gi];
        if (!cf.has(g) || granges[gi].empty()) continue;
        if (hasQ) {
          GemmSeg S = sym_seg(g, tile);
          S.A = at<char>(ws, g.offBh);
          S.B = S.inh = at<char>(ws, g.offQh[qcur]);
          S.inIsB = 1;
          S.sIn = 1.0f / sc.sQ[k];
          S.epi = EPI_AXPY;
          upper_in(S, tile);
          upper(S, tile, k + 1 == P.steps);
          S.u = 1.0f / (sc.sB[k] * sc.sQ[k]);
          S.p0 = a;
          S.ylam = S.u;
          S.ymu = a * S.sIn;
          S.outh = at<char>(ws, g.offQh[qcur ^ 1]);
          S.sOut = sc.sQ[k + 1];
          emit(gi, S, segs, works);
        }
        if (hasA) {
          GemmSeg S = sym_seg(g, tile);
          S.A = at<char>(ws, g.offBh);
          S.B = S.inh = at<char>(ws, g.offAh);
          S.in32 = f32(g, g.offA32);
          S.out32 = f32(g, g.offPA32);
          S.inIsB = 1;
          S.sIn = 1.0f / sc.sA[k];
          S.epi = EPI_AXPY;
          upper_in(S, tile);
          upper(S, tile, false);
          S.u = 1.0f / (sc.sB[k] * sc.sA[k]);
          S.p0 = a;
          S.ylam = S.u;
          S.ymu = a * S.sIn;
          S.outh = at<char>(ws, g.offPAh);
          S.sOut = sc.sPA[k];
          emit(gi, S, segs, works);
        }
      }
      s = launch_segs(cf, segs, works, 4, "Gram Q/PA kernel");
      if (s != MUON_OK) return s;
      // (iii) A ← a·PA + B·PA
      if (hasA) {
        segs.clear();
        works.clear();
        for (size_t gi = 0; gi < P.groups.size(); ++gi) {
          const GroupPlan& g = P.groups[gi];
          if (!cf.has(g) || granges[gi].empty()) continue;
          GemmSeg S = sym_seg(g, tile);
          S.A = at<char>(ws, g.offBh);
          S.B = S.inh = at<char>(ws, g.offPAh);
          S.in32 = f32(g, g.offPA32);
          S.out32 = f32(g, g.offA32);
          S.inIsB = 1;
          S.sIn = 1.0f / sc.sPA[k];
          S.epi = EPI_AXPY;
          upper_in(S, tile);
          upper(S, tile, false);
          S.u = 1.0f / (sc.sB[k] * sc.sPA[k]);
          S.p0 = a;
          S.ylam = S.u;
          S.ymu = a * S.sIn;
          S.outh = at<char>(ws, g.offAh);
          S.sOut = sc.sA[k + 1];
          emit(gi, S, segs, works);
        }
        s = launch_segs(cf, segs, works, 4, "Gram A-update kernel");
        if (s != MUON_OK) return s;
      }
    }
    if (hasQ) qcur ^= 1;
  }

  // 6. final product with the fused output / update
  for (const Piece& pc : lane) {
    const BucketPlan& bp = P.buckets[pc.bucket];
    const GroupPlan& g = P.groups[bp.group];
    const int tile = g.tile;
    for (size_t c0 = (size_t)pc.b0; c0 < (size_t)pc.b1; c0 += kMaxUser) {
      const size_t cn = std::min((size_t)pc.b1 - c0, (size_t)kMaxUser);
      GemmLaunch L;
      std::memset(&L, 0, sizeof(L));
      L.userDtype = dstDtype;
      L.decay = P.forStep ? V.decay : 1.f;
      L.xcdShift = g.xcdShift;
      L.band = g.band;
      GemmSeg& S = L.seg[0];
      const char* qh = at<char>(ws, g.offQh[qcur] + g.strideh * (bp.gramStart + c0));
      // X₀ᵀ as rows (128-tile kernel), or X₀ read through transposed panels
      // (256-tile kernel; its rows are k, so the row stride is Np).
      const char* xop = bp.xT ? at<char>(ws, bp.offXTh + bp.strideX * c0)
                              : at<char>(ws, bp.offXh + bp.strideX * c0);
      const int32_t ldx = (int32_t)(bp.xT ? bp.Mp : bp.Np);
      if (!bp.tall) {  // O = Q·X₀ : rows of Q, rows of X₀ᵀ
        S.A = qh;
        S.strideA = bp.Mp * bp.Mp;
        S.B = xop;
        S.strideB = bp.Np * bp.Mp;
        S.lda = (int32_t)bp.Mp;
        S.ldb = ldx;
        S.transB = bp.xT ? 0 : 1;
        S.tilesM = (int32_t)(bp.Mp / tile);
        S.tilesN = (int32_t)(bp.Np / tile);
        S.mReal = (int32_t)bp.m;
        S.nReal = (int32_t)bp.n;
      } else {         // Oᵀ = X₀ᵀ·Q : rows of X₀ᵀ, rows of Q
        S.A = xop;
        S.strideA = bp.Np * bp.Mp;
        S.B = qh;
        S.strideB = bp.Mp * bp.Mp;
        S.lda = ldx;
        S.ldb = (int32_t)bp.Mp;
        S.transA = bp.xT ? 0 : 1;
        S.tilesM = (int32_t)(bp.Np / tile);
        S.tilesN = (int32_t)(bp.Mp / tile);
        S.mReal = (int32_t)bp.n;
        S.nReal = (int32_t)bp.m;
      }
      S.K = (int32_t)bp.Mp;
      S.tilesPerMat = S.tilesM * S.tilesN;
      S.count = (int)cn;
      S.sym = 0;
      S.epi = P.forStep ? EPI_UPDATE : EPI_OUT;
      S.u = 1.0f / (sc.sQ[P.steps] * sc.sX);
      if (fused_bucket(P, bp, cm)) S.rho = at<float>(ws, P.offRho) + bp.rhoStart + c0;
      S.userBase = 0;
      for (size_t k = 0; k < cn; ++k) {
        const int i = bp.mats[c0 + k];
        L.user[k] = cm[i].dst;
        L.userLd[k] = cm[i].ldDst;
        L.lrsc[k] = cm[i].lrsc;
      }
      L.nseg = 1;
      L.segStart[0] = 0;
      const int blocks = S.tilesPerMat * S.count;
      L.segStart[1] = blocks;
      const double work = 2.0 * (double)cn * bp.m * (double)bp.m * bp.n;
      const int op = g.op;
      muon_status_t s = Lr.run(5, work, "final product kernel",
                               [=] { return launch_gemm(op, tile, L, blocks, st); });
      if (s != MUON_OK) return s;
    }
  }
  return MUON_OK;
}


// ----------------------------------------------------------------------------
// Concurrent lanes.  A launch whose tiles do not fill the GPU a whole number
// of times leaves compute units idle in its last round, and a chain of
// dependent launches that fill less than one round idles between products.
// Splitting the plan's matrices over several streams ("lanes"), each running
// the whole product chain of its matrices, lets one lane's tiles fill the
// gaps another leaves.  A matrix's arithmetic does not depend on its lane, so
// the results are the same bit for bit.

constexpr int kMaxLanes = 4;
constexpr int kMaxLaneDevices = 64;
// Gram-space tiles per product (all groups of the call) below which the
// products run in two lanes, and below which three (when the call has at
// least three groups).  Measured on MI355X (whole calls, one lane against
// several): two lanes are faster up to 4.2 rounds of the 256 compute units
// (1062 tiles: two Qwen2.5-7B-shaped layers, 3%; one layer 10%, 32 and 64 ×
// 1024×4096 13% and 6%) and slower from 8.3 rounds on (2124 tiles: four
// layers, 2%; the 28-layer set 6%); three lanes are best for the small mix
// (240 tiles in four groups: 16% against 7% with two) and no better than two
// for one group.
constexpr double kLaneTwoBelow = 1536;
constexpr double kLaneThreeBelow = 256;

int lane_count(const Plan& P) {
  if (const char* e = std::getenv("MUON_LANES")) {
    const int v = std::atoi(e);
    if (v >= 1 && v <= kMaxLanes) return v;
  }
  double tiles = 0;
  int mats = 0, groups = 0;
  for (const GroupPlan& g : P.groups) {
    if (g.count == 0) continue;
    const double t = (double)(g.Mp / g.tile);
    tiles += g.count * t * (t + 1) / 2;
    mats += g.count;
    ++groups;
  }
  if (mats < 2 || tiles >= kLaneTwoBelow) return 1;
  return (tiles < kLaneThreeBelow && groups >= 3) ? 3 : 2;
}

Lane whole_lane(const Plan& P) {
  Lane l;
  for (size_t b = 0; b < P.buckets.size(); ++b)
    l.push_back(Piece{(int)b, 0, (int)P.buckets[b].mats.size()});
  return l;
}

// Lanes of about equal work: a group whose work exceeds a lane's share is cut
// into ranges of consecutive group positions of about equal work; groups and
// ranges then go to the least loaded lane, largest first.
std::vector<Lane> plan_lanes(const Plan& P, int L) {
  if (L <= 1) return {whole_lane(P)};
  struct Item {
    int group, s, e;
    double work;
  };
  // work of every group position (positions follow the buckets' gramStart)
  std::vector<std::vector<double>> pw(P.groups.size());
  double total = 0;
  for (size_t gi = 0; gi < P.groups.size(); ++gi) pw[gi].assign(P.groups[gi].count, 0.0);
  for (const BucketPlan& bp : P.buckets)
    for (size_t k = 0; k < bp.mats.size(); ++k) {
      const double w = mat_work(bp.m, bp.n);
      pw[bp.group][bp.gramStart + k] = w;
      total += w;
    }
  if (total <= 0) return {whole_lane(P)};
  const double share = total / L;
  std::vector<Item> items;
  for (size_t gi = 0; gi < P.groups.size(); ++gi) {
    const std::vector<double>& w = pw[gi];
    double gw = 0;
    for (double x : w) gw += x;
    if (w.empty() || gw <= 0) continue;
    const int pieces = std::max(1, std::min((int)w.size(), (int)std::ceil(gw / share - 1e-9)));
    double acc = 0;
    int s = 0, cut = 1;
    for (int k = 0; k < (int)w.size(); ++k) {
      acc += w[k];
      const bool last = k + 1 == (int)w.size();
      if (last || (cut < pieces && acc >= gw * cut / pieces)) {
        double iw = 0;
        for (int j = s; j <= k; ++j) iw += w[j];
        items.push_back(Item{(int)gi, s, k + 1, iw});
        s = k + 1;
        ++cut;
      }
    }
  }
  std::stable_sort(items.begin(), items.end(), [](const Item& a, const Item& b) { return a.work > b.work; });
  std::vector<double> load(L, 0.0);
  std::vector<std::vector<Item>> assigned(L);
  for (const Item& it : items) {
    const int l = (int)(std::min_element(load.begin(), load.end()) - load.begin());
    load[l] += it.work;
    assigned[l].push_back(it);
  }
  std::vector<Lane> lanes;
  for (int l = 0; l < L; ++l) {
    Lane lane;
    for (const Item& it : assigned[l]) {
      for (int bi : P.groups[it.group].buckets) {
        const BucketPlan& bp = P.buckets[bi];
        const int lo = std::max(it.s, bp.gramStart);
        const int hi = std::min(it.e, bp.gramStart + (int)bp.mats.size());
        if (hi > lo) lane.push_back(Piece{bi, lo - bp.gramStart, hi - bp.gramStart});
      }
    }
    if (!lane.empty()) lanes.push_back(std::move(lane));
  }
  if (lanes.empty()) lanes.push_back(whole_lane(P));
  return lanes;
}

// Streams and events of the lanes, one set per device, created on the first
// call that needs them (never while the caller's stream is being captured);
// the mutex also keeps each call's event records and waits together.
struct LaneRes {
  hipStream_t side[kMaxLanes - 1] = {};
  hipEvent_t ev[kMaxLanes] = {};
  bool ready = false;
};
std::mutex g_lane_mu;
LaneRes g_lane[kMaxLaneDevices];

bool lane_resources(hipStream_t st, LaneRes** out) {  // g_lane_mu held
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxLaneDevices) return false;
  LaneRes& R = g_lane[dev];
  if (!R.ready) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
    bool ok = true;
    for (hipStream_t& s : R.side)
      if (ok && hipStreamCreateWithFlags(&s, hipStreamNonBlocking) != hipSuccess) s = nullptr, ok = false;
    for (hipEvent_t& e : R.ev)
      if (ok && hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) e = nullptr, ok = false;
    if (!ok) {
      for (hipStream_t& s : R.side)
        if (s) hipStreamDestroy(s), s = nullptr;
      for (hipEvent_t& e : R.ev)
        if (e) hipEventDestroy(e), e = nullptr;
      return false;
    }
    R.ready = true;
  }
  *out = &R;
  return true;
}

// The products (and, with passes, the HBM-bound passes before them) of a
// plan.  With several lanes every lane's launches are recorded first and
// then submitted round-robin, one launch per lane at a time, so that every
// lane has work on the GPU from the start (submitting one lane's whole chain
// before the next would start the later lanes only after the host has made
// the earlier lanes' launches); each lane runs its own passes, so its
// products wait for its matrices only.
muon_status_t enqueue_lanes(const Plan& P, const std::vector<CallerMat>& cm, int srcDtype,
                            int dstDtype, float beta, float eps, const StepVariant& V, void* ws,
                            hipStream_t st, bool passes) {
  bool any = false;
  for (const MatPlan& m : P.mats) any |= !m.empty;
  if (!any) return MUON_OK;
  // callers that must not make the library create streams or events (the
  // entry point that allocates nothing) run on their stream alone
  const std::vector<Lane> lanes = plan_lanes(P, g_no_events ? 1 : lane_count(P));
  if (lanes.size() > 1) {
    std::lock_guard<std::mutex> lk(g_lane_mu);
    LaneRes* R = nullptr;
    if (lane_resources(st, &R)) {
      auto hip = [](hipError_t e, const char* what) {
        return e == hipSuccess ? MUON_OK : fail(MUON_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
      };
      // record every lane's launches (nothing is enqueued yet)
      std::vector<std::vector<Thunk>> q(lanes.size());
      muon_status_t s = MUON_OK;
      for (size_t i = 0; s == MUON_OK && i < lanes.size(); ++i) {
        const hipStream_t ls = i ? R->side[i - 1] : st;
        if (passes) {
          std::vector<int> mats;
          for (const Piece& pc : lanes[i])
            for (int k = pc.b0; k < pc.b1; ++k) mats.push_back(P.buckets[pc.bucket].mats[k]);
          s = enqueue_passes(P, cm, srcDtype, beta, eps, V, ws, ls, &mats, &q[i]);
        }
        if (s == MUON_OK) s = enqueue_lane(P, lanes[i], cm, dstDtype, V, ws, ls, &q[i]);
      }
      if (s != MUON_OK) return s;
      s = hip(hipEventRecord(R->ev[0], st), "hipEventRecord");
      for (size_t i = 1; s == MUON_OK && i < lanes.size(); ++i)
        s = hip(hipStreamWaitEvent(R->side[i - 1], R->ev[0], 0), "hipStreamWaitEvent");
      if (s != MUON_OK) return s;
      size_t most = 0;
      for (const auto& v : q) most = std::max(most, v.size());
      for (size_t k = 0; s == MUON_OK && k < most; ++k)
        for (size_t i = 0; s == MUON_OK && i < lanes.size(); ++i)
          if (k < q[i].size()) s = q[i][k]();
      // every lane is joined back, after a failure too, so that later work
      // on the caller's stream stays ordered after what was enqueued
      for (size_t i = 1; i < lanes.size(); ++i) {
        muon_status_t j = hip(hipEventRecord(R->ev[i], R->side[i - 1]), "hipEventRecord");
        if (j == MUON_OK) j = hip(hipStreamWaitEvent(st, R->ev[i], 0), "hipStreamWaitEvent");
        if (s == MUON_OK) s = j;
      }
      return s;
    }
  }
  if (passes) {
    muon_status_t s = enqueue_passes(P, cm, srcDtype, beta, eps, V, ws, st);
    if (s != MUON_OK) return s;
  }
  return enqueue_lane(P, whole_lane(P), cm, dstDtype, V, ws, st);
}

muon_status_t enqueue_products(const Plan& P, const std::vector<CallerMat>& cm, int dstDtype,
                               const StepVariant& V, void* ws, hipStream_t st) {
  return enqueue_lanes(P, cm, MUON_DTYPE_F32, dstDtype, 0.f, 0.f, V, ws, st, false);
}

muon_status_t enqueue(const Plan& P, const std::vector<CallerMat>& cm, int srcDtype, int dstDtype,
                      float beta, float eps, const StepVariant& V, void* ws, hipStream_t st) {
  return enqueue_lanes(P, cm, srcDtype, dstDtype, beta, eps, V, ws, st, true);
}

// ----------------------------------------------------------------------------
// Chunked steps.
//
// A step may run as consecutive chunks of the call's matrix list (in call
// order), each with a plan of its own:
//  * overlapped (on request, for calls of at least kOverlapMinElems
//    elements): every chunk has its own workspace region; the chunks'
//    HBM-bound passes run back to back on a side stream, and each chunk's
//    products wait for its passes on the caller's stream, so the passes of
//    the later chunk run while the products of the earlier one do (measured
//    on the 196-matrix Qwen2.5-7B-shaped step: at most 0.4% faster than one
//    stream — the products slow down by nearly as much as the passes they
//    hide, the card being at its power limit — so it is not the default);
//  * under a workspace budget: the chunks share one region and run one
//    after another on the caller's stream.
// A matrix's arithmetic depends only on the configuration of its Gram group
// (tile, operand type, fp32 state), so chunking leaves each result bit for
// bit unchanged whenever those configurations do not change with the split
// (they can when a group mixes nearly square and wide matrices of one m, or
// under a tile table keyed by batch size).

constexpr int kMaxChunks = 2;
constexpr int64_t kOverlapMinElems = int64_t(1) << 30;
// Share of the algorithmic work in each overlapped chunk: the first chunk's
// passes cannot be hidden, so it is the small one (2 chunks of 1/4 and 3/4
// measured best among 2, 3 and 4 chunks).
constexpr double kChunkShare[kMaxChunks] = {0.25, 0.75};

struct ChunkPlan {
  std::vector<int> idx;  // matrices of the call in this chunk
  Plan plan;
  size_t off = 0;        // offset of this chunk's workspace region
};

struct StepLayout {
  std::vector<ChunkPlan> chunks;
  size_t totalBytes = 0;
  bool overlap = false;
};

std::string plan_chunk(const int64_t* rows, const int64_t* cols, const std::vector<int>& idx, int steps,
                       const float* coeffs, Plan* P) {
  std::vector<int64_t> r, c;
  for (int i : idx) {
    r.push_back(rows[i]);
    c.push_back(cols[i]);
  }
  return build_plan(r.data(), c.data(), (int)idx.size(), OP_F16, steps, coeffs[0], coeffs[1],
                    coeffs[2], true, P);
}

// overlap: overlapped chunks when the call is large enough; otherwise one
// plan (or the budget's chunks).  budget = 0: no workspace budget.
std::string step_layout(const int64_t* rows, const int64_t* cols, int count, int steps,
                        const float* coeffs, bool overlap, uint64_t budget, StepLayout* out) {
  StepLayout& Lo = *out;
  Lo = StepLayout();
  int64_t elems = 0;
  double work = 0;
  for (int i = 0; i < count; ++i) {
    elems += rows[i] * cols[i];
    work += mat_work(rows[i], cols[i]);
  }
  std::vector<std::vector<int>> parts;
  if (budget > 0) {
    std::vector<int> cur;
    for (int i = 0; i < count; ++i) {
      std::vector<int> trial = cur;
      trial.push_back(i);
      Plan P;
      std::string e = plan_chunk(rows, cols, trial, steps, coeffs, &P);
      if (!e.empty()) return e;
      if (P.totalBytes <= budget) {
        cur.swap(trial);
        continue;
      }
      if (cur.empty())
        return "matrix " + std::to_string(i) + " alone needs " + std::to_string(P.totalBytes) +
               " bytes of workspace, above the budget of " + std::to_string(budget);
      parts.push_back(cur);
      cur.assign(1, i);
      std::string e2 = plan_chunk(rows, cols, cur, steps, coeffs, &P);
      if (!e2.empty()) return e2;
      if (P.totalBytes > budget)
        return "matrix " + std::to_string(i) + " alone needs " + std::to_string(P.totalBytes) +
               " bytes of workspace, above the budget of " + std::to_string(budget);
    }
    if (!cur.empty()) parts.push_back(cur);
  } else if (overlap && elems >= kOverlapMinElems && count >= kMaxChunks && work > 0) {
    double acc = 0, edge = 0;
    int k = 0;
    parts.assign(1, {});
    for (int i = 0; i < count; ++i) {
      if (k + 1 < kMaxChunks && acc >= (edge + kChunkShare[k]) * work && !parts[k].empty()) {
        edge += kChunkShare[k];
        ++k;
        parts.push_back({});
      }
      parts[k].push_back(i);
      acc += mat_work(rows[i], cols[i]);
    }
    Lo.overlap = parts.size() > 1;
  } else {
    parts.assign(1, {});
    for (int i = 0; i < count; ++i) parts[0].push_back(i);
  }
  size_t off = 0, most = 0;
  for (auto& idx : parts) {
    ChunkPlan C;
    C.idx = idx;
    std::string e = plan_chunk(rows, cols, idx, steps, coeffs, &C.plan);
    if (!e.empty()) return e;
    if (budget > 0) {
      C.off = 0;  // chunks share one region, one after another
      most = std::max(most, C.plan.totalBytes);
    } else {
      C.off = off;
      off += (C.plan.totalBytes + 255) / 256 * 256;
    }
    Lo.chunks.push_back(std::move(C));
  }
  Lo.totalBytes = budget > 0 ? most : off;
  return "";
}

// Side stream and events of the overlapped step, one set per device; the
// mutex also keeps each call's event records and waits together.
struct SideRes {
  hipStream_t side = nullptr;
  hipEvent_t ev[kMaxChunks + 1] = {};
  bool ready = false;
};
constexpr int kMaxSideDevices = 64;
std::mutex g_side_mu;
SideRes g_side[kMaxSideDevices];

// g_side_mu held.  False: no side stream (the call then runs on its stream alone).
bool side_resources(hipStream_t st, SideRes** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxSideDevices) return false;
  SideRes& R = g_side[dev];
  if (!R.ready) {
    // never create the stream while the caller's stream is being captured
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return false;
    if (hipStreamCreateWithFlags(&R.side, hipStreamNonBlocking) != hipSuccess) {
      R.side = nullptr;
      return false;
    }
    for (hipEvent_t& e : R.ev) {
      if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
        for (hipEvent_t& f : R.ev)
          if (f) hipEventDestroy(f), f = nullptr;
        hipStreamDestroy(R.side);
        R.side = nullptr;
        return false;
      }
    }
    R.ready = true;
  }
  *out = &R;
  return true;
}

std::vector<CallerMat> subset(const std::vector<CallerMat>& cm, const std::vector<int>& idx) {
  std::vector<CallerMat> v;
  for (int i : idx) v.push_back(cm[i]);
  return v;
}

muon_status_t enqueue_step(const StepLayout& Lo, const std::vector<CallerMat>& cm, int dstDtype,
                           float beta, float eps, const StepVariant& V, void* ws, hipStream_t st) {
  if (Lo.overlap) {
    std::lock_guard<std::mutex> lk(g_side_mu);
    SideRes* R = nullptr;
    if (side_resources(st, &R)) {
      auto hip = [](hipError_t e, const char* what) {
        return e == hipSuccess ? MUON_OK : fail(MUON_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
      };
      muon_status_t s = hip(hipEventRecord(R->ev[0], st), "hipEventRecord");
      if (s == MUON_OK) s = hip(hipStreamWaitEvent(R->side, R->ev[0], 0), "hipStreamWaitEvent");
      for (size_t c = 0; s == MUON_OK && c < Lo.chunks.size(); ++c) {
        const ChunkPlan& C = Lo.chunks[c];
        s = enqueue_passes(C.plan, subset(cm, C.idx), MUON_DTYPE_F32, beta, eps, V,
                           static_cast<char*>(ws) + C.off, R->side);
        if (s == MUON_OK) s = hip(hipEventRecord(R->ev[c + 1], R->side), "hipEventRecord");
      }
      for (size_t c = 0; s == MUON_OK && c < Lo.chunks.size(); ++c) {
        const ChunkPlan& C = Lo.chunks[c];
        s = hip(hipStreamWaitEvent(st, R->ev[c + 1], 0), "hipStreamWaitEvent");
        if (s == MUON_OK)
          s = enqueue_products(C.plan, subset(cm, C.idx), dstDtype, V, static_cast<char*>(ws) + C.off, st);
      }
      return s;
    }
  }
  for (const ChunkPlan& C : Lo.chunks) {
    muon_status_t s = enqueue(C.plan, subset(cm, C.idx), MUON_DTYPE_F32, dstDtype, beta, eps, V,
                              static_cast<char*>(ws) + C.off, st);
    if (s != MUON_OK) return s;
  }
  return MUON_OK;
}

// ----------------------------------------------------------------------------
// Row/column-selected step (Dion3 review, §3 "Method & Key Results" and §1
// "Key Terms & Definitions", Error Feedback): per matrix the k = ⌈ρ·m⌉
// highest-scoring rows of the oriented buffer are gathered into a dense fp32
// block, orthogonalised by the batched pipeline above (in place) and
// scattered back into the weights.

struct SelMatLayout {
  int64_t m = 0, k = 0, gr = 0, gc = 0;  // short side, kept rows, block shape
  int tall = 0, nChunks = 0;
  size_t offXs = 0, offScore = 0, offIdx = 0, offPos = 0;
};

struct SelLayout {
  Plan ns;                     // plan of the batched NS over the blocks
  std::vector<SelMatLayout> mats;
  size_t totalBytes = 0;
};

size_t sel_align(size_t x) { return (x + 255) / 256 * 256; }

int64_t sel_count(int64_t m, double fraction) {
  if (m == 0) return 0;
  const int64_t k = (int64_t)std::ceil(fraction * (double)m);
  return std::max<int64_t>(1, std::min<int64_t>(m, k));
}

std::string sel_layout(const int64_t* rows, const int64_t* cols, int count, double fraction,
                       int steps, const float* coeffs, SelLayout* out) {
  SelLayout& Lo = *out;
  Lo.mats.assign(count, SelMatLayout{});
  std::vector<int64_t> gr(count), gc(count);
  for (int i = 0; i < count; ++i) {
    SelMatLayout& s = Lo.mats[i];
    const int64_t r = rows[i], c = cols[i];
    s.tall = r > c ? 1 : 0;
    s.m = std::min(r, c);
    s.k = (r == 0 || c == 0) ? 0 : sel_count(s.m, fraction);
    s.gr = s.tall ? r : s.k;
    s.gc = s.tall ? s.k : c;
    s.nChunks = s.tall ? (int)((r + kSelChunk - 1) / kSelChunk) : 1;
    gr[i] = s.k ? s.gr : 0;
    gc[i] = s.k ? s.gc : 0;
  }
  std::string e = build_plan(gr.data(), gc.data(), count, OP_F16, steps, coeffs[0], coeffs[1],
                             coeffs[2], false, &Lo.ns);
  if (!e.empty()) return e;
  size_t off = sel_align(Lo.ns.totalBytes);
  for (SelMatLayout& s : Lo.mats) {
    if (!s.k) continue;
    s.offXs = off;    off = sel_align(off + 4 * (size_t)s.gr * (size_t)s.gc);
    s.offScore = off; off = sel_align(off + 4 * (size_t)s.nChunks * (size_t)s.m);
    s.offIdx = off;   off = sel_align(off + 4 * (size_t)s.k);
    s.offPos = off;   off = sel_align(off + 4 * (size_t)s.m);
  }
  Lo.totalBytes = off;
  return "";
}

muon_status_t enqueue_selected(const SelLayout& Lo, void* const* params, const float* const* grads,
                               float* const* momentum, const int64_t* rows, const int64_t* cols,
                               int count, int paramDtype, float beta, float lr, float eps,
                               void* ws, hipStream_t st) {
  Launcher Lr{st};
  std::vector<int> live;
  for (int i = 0; i < count; ++i)
    if (Lo.mats[i].k) live.push_back(i);
  if (live.empty()) return MUON_OK;
  const size_t psz = paramDtype == MUON_DTYPE_F32 ? 4 : 2;
  int vec = 1;
  for (int i : live)
    if ((cols[i] & 3) || ((uintptr_t)grads[i] & 15) || ((uintptr_t)momentum[i] & 15) ||
        ((uintptr_t)params[i] & (4 * psz - 1)))
      vec = 0;

  auto fill_from = [&](SelLaunch& L, const std::vector<int>& lst, size_t c0, size_t cn) {
    std::memset(&L, 0, sizeof(L));
    L.n = (int)cn;
    L.paramDtype = paramDtype;
    L.beta = beta;
    L.vec = vec;
    for (size_t q = 0; q < cn; ++q) {
      const int i = lst[c0 + q];
      const SelMatLayout& s = Lo.mats[i];
      SelMat& M = L.mat[q];
      M.g = grads[i];
      M.mom = momentum[i];
      M.w = params[i];
      M.xs = at<float>(ws, s.offXs);
      M.score = at<float>(ws, s.offScore);
      M.idx = at<int32_t>(ws, s.offIdx);
      M.pos = at<int32_t>(ws, s.offPos);
      M.nsSum = at<float>(ws, Lo.ns.offPartials) + Lo.ns.mats[i].partialOff;
      M.rows = rows[i];
      M.cols = cols[i];
      M.m = (int32_t)s.m;
      M.k = (int32_t)s.k;
      M.tall = s.tall;
      M.nChunks = s.nChunks;
      M.lrsc = (float)(lr * std::sqrt(std::max(1.0, (double)rows[i] / (double)cols[i])));
    }
  };
  auto fill = [&](SelLaunch& L, size_t c0, size_t cn) { fill_from(L, live, c0, cn); };
  // 1. B = M + g and the row scores
  for (size_t c0 = 0; c0 < live.size(); c0 += kMaxUser) {
    SelLaunch L;
    const size_t cn = std::min(live.size() - c0, (size_t)kMaxUser);
    fill(L, c0, cn);
    int64_t blocks = 0;
    double bytes = 0;
    for (size_t q = 0; q < cn; ++q) {
      SelMat& M = L.mat[q];
      M.blockStart = blocks;
      const int64_t span = 64 * (vec ? 4 : 1);  // columns per workgroup (tall)
      blocks += M.tall ? (int64_t)M.nChunks * ((M.cols + span - 1) / span) : (M.rows + 3) / 4;
      bytes += 12.0 * (double)M.rows * (double)M.cols + 4.0 * M.nChunks * (double)M.m;
    }
    muon_status_t s = Lr.run(8, bytes, "selected accumulate kernel",
                             [&] { return launch_sel_accum(L, blocks, st); });
    if (s != MUON_OK) return s;
  }
  // 2. top-k per matrix
  for (size_t c0 = 0; c0 < live.size(); c0 += kMaxUser) {
    SelLaunch L;
    const size_t cn = std::min(live.size() - c0, (size_t)kMaxUser);
    fill(L, c0, cn);
    double bytes = 0;
    for (size_t q = 0; q < cn; ++q)
      bytes += 4.0 * L.mat[q].nChunks * (double)L.mat[q].m + 4.0 * L.mat[q].k + 4.0 * L.mat[q].m;
    muon_status_t s = Lr.run(9, bytes, "selected top-k kernel", [&] { return launch_sel_topk(L, st); });
    if (s != MUON_OK) return s;
  }
  // 3. the blocks' norms (the top-k wrote ‖B_S‖²_F), then the gather: blocks
  // on the fp16 256-tile path have the gather write their operand directly
  // (no fp32 copy, no cast pass); the others are copied and cast.
  std::vector<CallerMat> cm(count);
  for (int i = 0; i < count; ++i) {
    const SelMatLayout& s = Lo.mats[i];
    cm[i].src = s.k ? at<float>(ws, s.offXs) : nullptr;
    cm[i].ldSrc = std::max<int64_t>(s.gc, 1);
    cm[i].dst = s.k ? at<float>(ws, s.offXs) : nullptr;
    cm[i].ldDst = std::max<int64_t>(s.gc, 1);
    cm[i].grad = nullptr;
    cm[i].lrsc = 0.f;
  }
  StepVariant V;
  V.presummed = 1;  // ‖B_S‖²_F = Σ of the selected scores, written by the top-k
  V.stages = 2;     // norm finish only
  muon_status_t s = enqueue_passes(Lo.ns, cm, MUON_DTYPE_F32, 0.f, eps, V, ws, st);
  if (s != MUON_OK) return s;
  std::vector<int> direct, copied;
  for (int i : live) {
    const BucketPlan& bp = Lo.ns.buckets[Lo.ns.mats[i].bucket];
    (bp.op == OP_F16 && !bp.xT ? direct : copied).push_back(i);
  }
  for (size_t c0 = 0; c0 < copied.size(); c0 += kMaxUser) {
    SelLaunch L;
    const size_t cn = std::min(copied.size() - c0, (size_t)kMaxUser);
    fill_from(L, copied, c0, cn);
    int64_t blocks = 0;
    double bytes = 0;
    for (size_t q = 0; q < cn; ++q) {
      SelMat& M = L.mat[q];
      M.blockStart = blocks;
      blocks += ((M.tall ? M.rows : (int64_t)M.k) + 3) / 4;
      bytes += 12.0 * (double)(M.tall ? M.rows : M.k) * (double)(M.tall ? M.k : M.cols);
    }
    s = Lr.run(10, bytes, "selected gather kernel", [&] { return launch_sel_gather(L, blocks, st); });
    if (s != MUON_OK) return s;
  }
  int gvec = 1;
  for (int i : direct)
    if ((cols[i] & 3) || ((uintptr_t)momentum[i] & 15)) gvec = 0;
  for (size_t c0 = 0; c0 < direct.size(); c0 += kMaxUser) {
    SelCastLaunch L;
    std::memset(&L, 0, sizeof(L));
    const size_t cn = std::min(direct.size() - c0, (size_t)kMaxUser);
    L.n = (int)cn;
    L.beta = beta;
    L.sX = Lo.ns.scales.sX;
    L.vec = gvec;
    L.alpha = at<float>(ws, Lo.ns.offAlpha);
    int64_t blocks = 0;
    double bytes = 0;
    for (size_t q = 0; q < cn; ++q) {
      const int i = direct[c0 + q];
      const SelMatLayout& sl = Lo.mats[i];
      const MatPlan& mp = Lo.ns.mats[i];
      const BucketPlan& bp = Lo.ns.buckets[mp.bucket];
      SelCastMat& M = L.mat[q];
      M.mom = momentum[i];
      M.idx = at<int32_t>(ws, sl.offIdx);
      M.x0 = at<_Float16>(ws, bp.offXh + bp.strideX * mp.posBucket);
      M.rows = rows[i];
      M.cols = cols[i];
      M.k = (int32_t)sl.k;
      M.tall = sl.tall;
      M.Mp = (int32_t)bp.Mp;
      M.Np = (int32_t)bp.Np;
      M.alphaIdx = i;
      M.blockStart = blocks;
      blocks += sl.tall ? (int64_t)(bp.Mp / 64) * (bp.Np / 64) : (int64_t)(bp.Mp + 3) / 4;
      bytes += 12.0 * (double)sl.k * (double)(sl.tall ? rows[i] : cols[i]) + 2.0 * (double)bp.Mp * (double)bp.Np;
    }
    s = Lr.run(10, bytes, "selected gather + cast kernel",
               [&] { return launch_sel_gather_cast(L, blocks, st); });
    if (s != MUON_OK) return s;
  }
  // 4. cast the copied blocks, orthogonalise every block in place
  V.stages = 4;
  s = enqueue_passes(Lo.ns, cm, MUON_DTYPE_F32, 0.f, eps, V, ws, st, &copied);
  if (s != MUON_OK) return s;
  s = enqueue_products(Lo.ns, cm, MUON_DTYPE_F32, V, ws, st);
  if (s != MUON_OK) return s;
  // 5. scatter the update (the gather has already decayed the buffer on S)
  for (size_t c0 = 0; c0 < live.size(); c0 += kMaxUser) {
    SelLaunch L;
    const size_t cn = std::min(live.size() - c0, (size_t)kMaxUser);
    fill(L, c0, cn);
    int64_t blocks = 0;
    double bytes = 0;
    for (size_t q = 0; q < cn; ++q) {
      SelMat& M = L.mat[q];
      M.blockStart = blocks;
      blocks += ((M.tall ? M.rows : (int64_t)M.k) + 3) / 4;
      bytes += (4.0 + 2.0 * psz) * (double)(M.tall ? M.rows : M.k) * (double)(M.tall ? M.k : M.cols);
    }
    s = Lr.run(11, bytes, "selected scatter kernel", [&] { return launch_sel_scatter(L, blocks, st); });
    if (s != MUON_OK) return s;
  }
  return MUON_OK;
}

}  // namespace

void set_last_error(const std::string& msg) { g_err = msg; }
void set_no_events(bool on) { g_no_events = on; }

}  // namespace muon

using namespace muon;

extern "C" {

int32_t muon_abi_version(void) { return MUON_NS_ABI_VERSION; }

const char* muon_last_error(void) { return g_err.c_str(); }

muon_status_t muon_ns_workspace_size(const muon_ns_desc_t* desc, int32_t count, muon_dtype_t dtype,
                                     size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
  if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
  if (count > 0 && !desc) return fail(MUON_ERR_INVALID_ARG, "desc is NULL");
  if (dtype != MUON_DTYPE_F32 && dtype != MUON_DTYPE_BF16)
    return fail(MUON_ERR_INVALID_ARG, "unknown dtype");
  std::vector<int64_t> r(count), c(count);
  for (int i = 0; i < count; ++i) {
    muon_status_t s = check_shape(i, desc[i].rows, desc[i].cols);
    if (s != MUON_OK) return s;
    r[i] = desc[i].rows;
    c[i] = desc[i].cols;
  }
  Plan P;
  std::string e = build_plan(r.data(), c.data(), count, dtype == MUON_DTYPE_F32 ? OP_F32 : OP_F16,
                             5, 1.f, 0.f, 0.f, false, &P);
  if (!e.empty()) return fail(MUON_ERR_INVALID_ARG, e);
  *bytes = P.totalBytes;
  return MUON_OK;
}

muon_status_t muon_step_workspace_size(const int64_t* rows, const int64_t* cols, int32_t count,
                                       size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
  if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
  if (count > 0 && (!rows || !cols)) return fail(MUON_ERR_INVALID_ARG, "rows/cols is NULL");
  for (int i = 0; i < count; ++i) {
    muon_status_t s = check_shape(i, rows[i], cols[i]);
    if (s != MUON_OK) return s;
  }
  // enough for the default (one plan) and for opts->overlap (a region per chunk)
  const float unit[3] = {1.f, 0.f, 0.f};
  StepLayout Ld, Ls;
  std::string e = step_layout(rows, cols, count, 5, unit, false, 0, &Ld);
  if (e.empty()) e = step_layout(rows, cols, count, 5, unit, true, 0, &Ls);
  if (!e.empty()) return fail(MUON_ERR_INVALID_ARG, e);
  *bytes = std::max(Ld.totalBytes, Ls.totalBytes);
  return MUON_OK;
}

muon_status_t muon_describe_plan(const int64_t* rows, const int64_t* cols, int32_t count,
                                 int32_t for_step, muon_dtype_t dtype, int32_t steps,
                                 const float coeffs[3], char* buf, size_t buf_len) {
  g_err.clear();
  if (!buf || buf_len == 0) return fail(MUON_ERR_INVALID_ARG, "buf is NULL or empty");
  if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
  if (count > 0 && (!rows || !cols)) return fail(MUON_ERR_INVALID_ARG, "rows/cols is NULL");
  if (steps < 0 || steps > kMaxSteps) return fail(MUON_ERR_INVALID_ARG, "steps out of range");
  if (!finite3(coeffs)) return fail(MUON_ERR_INVALID_ARG, "coeffs NULL or not finite");
  if (dtype != MUON_DTYPE_F32 && dtype != MUON_DTYPE_BF16)
    return fail(MUON_ERR_INVALID_ARG, "unknown dtype");
  for (int i = 0; i < count; ++i) {
    muon_status_t s = check_shape(i, rows[i], cols[i]);
    if (s != MUON_OK) return s;
  }
  const int op = (!for_step && dtype == MUON_DTYPE_F32) ? OP_F32 : OP_F16;
  Plan P;
  std::string e = build_plan(rows, cols, count, op, steps, coeffs[0], coeffs[1], coeffs[2],
                             for_step != 0, &P);
  if (!e.empty()) return fail(MUON_ERR_INVALID_ARG, e);
  std::string j = P.json();
  // the concurrent lanes the products would run in: [bucket, b0, b1] pieces
  {
    std::string l = ",\"lanes\":[";
    const std::vector<Lane> lanes = plan_lanes(P, lane_count(P));
    for (size_t i = 0; i < lanes.size(); ++i) {
      l += i ? ",[" : "[";
      for (size_t k = 0; k < lanes[i].size(); ++k) {
        const Piece& pc = lanes[i][k];
        l += (k ? ",[" : "[") + std::to_string(pc.bucket) + "," + std::to_string(pc.b0) + "," +
             std::to_string(pc.b1) + "]";
      }
      l += "]";
    }
    l += "]";
    if (!j.empty() && j.back() == '}') j.insert(j.size() - 1, l);
  }
  const size_t n = std::min(j.size(), buf_len - 1);
  std::memcpy(buf, j.data(), n);
  buf[n] = '\0';
  return MUON_OK;
}

muon_status_t muon_ns_batched(const muon_ns_desc_t* desc, int32_t count, int32_t steps,
                              const float coeffs[3], muon_dtype_t dtype, float eps, void* workspace,
                              size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
  if (count == 0) return MUON_OK;
  if (!desc) return fail(MUON_ERR_INVALID_ARG, "desc is NULL");
  if (steps < 0 || steps > kMaxSteps) return fail(MUON_ERR_INVALID_ARG, "steps out of range [0, 64]");
  if (!finite3(coeffs)) return fail(MUON_ERR_INVALID_ARG, "coeffs NULL or not finite");
  if (dtype != MUON_DTYPE_F32 && dtype != MUON_DTYPE_BF16)
    return fail(MUON_ERR_INVALID_ARG, "unknown dtype");
  if (!std::isfinite(eps) || eps < 0) return fail(MUON_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const size_t esz = dtype == MUON_DTYPE_F32 ? 4 : 2;
  std::vector<int64_t> r(count), c(count);
  std::vector<Range> outs, ins;
  for (int i = 0; i < count; ++i) {
    const muon_ns_desc_t& d = desc[i];
    muon_status_t s = check_shape(i, d.rows, d.cols);
    if (s != MUON_OK) return s;
    r[i] = d.rows;
    c[i] = d.cols;
    if (d.rows == 0 || d.cols == 0) continue;
    if (!d.x || !d.out) return fail(MUON_ERR_INVALID_ARG, "matrix " + std::to_string(i) + ": NULL x/out");
    if (d.ld_x < d.cols || d.ld_out < d.cols)
      return fail(MUON_ERR_INVALID_ARG, "matrix " + std::to_string(i) + ": ld < cols");
    const uintptr_t lo = (uintptr_t)d.out;
    outs.push_back({lo, lo + (uintptr_t)(((d.rows - 1) * d.ld_out + d.cols) * esz), i});
    const uintptr_t xl = (uintptr_t)d.x;
    ins.push_back({xl, xl + (uintptr_t)(((d.rows - 1) * d.ld_x + d.cols) * esz), i});
  }
  int oa = 0, ob = 0;
  if (overlaps(outs, &oa, &ob))
    return fail(MUON_ERR_ALIAS, "outputs of matrices " + std::to_string(oa) + " and " +
                                    std::to_string(ob) + " overlap");
  Plan P;
  const int op = dtype == MUON_DTYPE_F32 ? OP_F32 : OP_F16;
  std::string e = build_plan(r.data(), c.data(), count, op, steps, coeffs[0], coeffs[1], coeffs[2],
                             false, &P);
  if (!e.empty()) return fail(MUON_ERR_INVALID_ARG, e);
  if (P.totalBytes > 0) {
    if (!workspace) return fail(MUON_ERR_WORKSPACE, "workspace is NULL");
    if ((uintptr_t)workspace & 255) return fail(MUON_ERR_WORKSPACE, "workspace not 256-byte aligned");
    if (workspace_bytes < P.totalBytes)
      return fail(MUON_ERR_WORKSPACE, "workspace too small: need " + std::to_string(P.totalBytes) +
                                          " bytes, got " + std::to_string(workspace_bytes));
    const uintptr_t wl = (uintptr_t)workspace, wh = wl + P.totalBytes;
    int who = 0;
    if (workspace_overlaps(outs, wl, wh, &who) || workspace_overlaps(ins, wl, wh, &who))
      return fail(MUON_ERR_ALIAS, "workspace overlaps matrix " + std::to_string(who));
  }
  std::vector<CallerMat> cm(count);
  for (int i = 0; i < count; ++i) {
    cm[i].src = desc[i].x;
    cm[i].ldSrc = desc[i].ld_x;
    cm[i].dst = desc[i].out;
    cm[i].ldDst = desc[i].ld_out;
    cm[i].grad = nullptr;
    cm[i].lrsc = 0.f;
  }
  muon_status_t s = check_device();
  if (s != MUON_OK) return s;
  return enqueue(P, cm, dtype, dtype, 0.f, eps, StepVariant{}, workspace, (hipStream_t)stream);
}

muon_status_t muon_step_ex(void* const* params, const void* const* grads, float* const* momentum,
                           const int64_t* rows, const int64_t* cols, int32_t count,
                           muon_dtype_t param_dtype, float beta, float lr, int32_t steps,
                           const float coeffs[3], float eps, const muon_step_opts_t* opts,
                           void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
  StepVariant V;
  float wd = 0.f;
  bool overlap = false;
  uint64_t budget = 0;
  int32_t* scaleExp = nullptr;
  if (opts) {
    if (opts->nesterov != 0 && opts->nesterov != 1)
      return fail(MUON_ERR_INVALID_ARG, "opts->nesterov must be 0 or 1");
    if (!std::isfinite(opts->weight_decay) || opts->weight_decay < 0)
      return fail(MUON_ERR_INVALID_ARG, "opts->weight_decay must be finite and >= 0");
    if (opts->grad_dtype != MUON_DTYPE_F32 && opts->grad_dtype != MUON_DTYPE_BF16)
      return fail(MUON_ERR_INVALID_ARG, "unknown opts->grad_dtype");
    if (opts->overlap != 0 && opts->overlap != 1)
      return fail(MUON_ERR_INVALID_ARG, "opts->overlap must be 0 or 1");
    V.nesterov = opts->nesterov;
    V.gradDtype = opts->grad_dtype;
    wd = opts->weight_decay;
    overlap = opts->overlap != 0;
    budget = opts->max_workspace_bytes;
    scaleExp = opts->scale_exp;
  }
  if (count == 0) return MUON_OK;
  if (!params || !grads || !momentum || !rows || !cols)
    return fail(MUON_ERR_INVALID_ARG, "NULL pointer array");
  if (param_dtype != MUON_DTYPE_F32 && param_dtype != MUON_DTYPE_BF16)
    return fail(MUON_ERR_INVALID_ARG, "unknown param dtype");
  if (steps < 0 || steps > kMaxSteps) return fail(MUON_ERR_INVALID_ARG, "steps out of range [0, 64]");
  if (!finite3(coeffs)) return fail(MUON_ERR_INVALID_ARG, "coeffs NULL or not finite");
  if (!std::isfinite(beta) || !std::isfinite(lr))
    return fail(MUON_ERR_INVALID_ARG, "beta and lr must be finite");
  if (!std::isfinite(eps) || eps < 0) return fail(MUON_ERR_INVALID_ARG, "eps must be finite and >= 0");
  V.decay = (float)(1.0 - (double)lr * (double)wd);
  if (!std::isfinite(V.decay)) return fail(MUON_ERR_INVALID_ARG, "1 - lr*weight_decay is not finite");
  const size_t psz = param_dtype == MUON_DTYPE_F32 ? 4 : 2;
  const size_t gsz = V.gradDtype == MUON_DTYPE_F32 ? 4 : 2;
  std::vector<Range> ranges;
  for (int i = 0; i < count; ++i) {
    muon_status_t s = check_shape(i, rows[i], cols[i]);
    if (s != MUON_OK) return s;
    if (rows[i] == 0 || cols[i] == 0) continue;
    if (!params[i] || !grads[i] || !momentum[i])
      return fail(MUON_ERR_INVALID_ARG, "matrix " + std::to_string(i) + ": NULL tensor");
    const uintptr_t n = (uintptr_t)(rows[i] * cols[i]);
    ranges.push_back({(uintptr_t)params[i], (uintptr_t)params[i] + n * psz, i});
    ranges.push_back({(uintptr_t)grads[i], (uintptr_t)grads[i] + n * gsz, i});
    ranges.push_back({(uintptr_t)momentum[i], (uintptr_t)momentum[i] + n * 4, i});
  }
  int oa = 0, ob = 0;
  if (overlaps(ranges, &oa, &ob))
    return fail(MUON_ERR_ALIAS, "tensors of matrices " + std::to_string(oa) + " and " +
                                    std::to_string(ob) + " overlap");
  if (scaleExp) {
    if ((uintptr_t)scaleExp & 3) return fail(MUON_ERR_INVALID_ARG, "opts->scale_exp not 4-byte aligned");
    const uintptr_t lo = (uintptr_t)scaleExp, hi = lo + (uintptr_t)count * 4;
    int who = 0;
    if (workspace_overlaps(ranges, lo, hi, &who))
      return fail(MUON_ERR_ALIAS, "opts->scale_exp overlaps a tensor of matrix " + std::to_string(who));
  }
  StepLayout Lo;
  std::string e = step_layout(rows, cols, count, steps, coeffs, overlap, budget, &Lo);
  if (!e.empty()) return fail(budget > 0 ? MUON_ERR_WORKSPACE : MUON_ERR_INVALID_ARG, e);
  if (!workspace) return fail(MUON_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)workspace & 255) return fail(MUON_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (workspace_bytes < Lo.totalBytes)
    return fail(MUON_ERR_WORKSPACE, "workspace too small: need " + std::to_string(Lo.totalBytes) +
                                        " bytes, got " + std::to_string(workspace_bytes));
  {
    int who = 0;
    if (workspace_overlaps(ranges, (uintptr_t)workspace, (uintptr_t)workspace + Lo.totalBytes, &who))
      return fail(MUON_ERR_ALIAS, "workspace overlaps a tensor of matrix " + std::to_string(who));
    const uintptr_t lo = (uintptr_t)scaleExp, hi = lo + (uintptr_t)count * 4;
    if (scaleExp && lo < (uintptr_t)workspace + Lo.totalBytes && (uintptr_t)workspace < hi)
      return fail(MUON_ERR_ALIAS, "opts->scale_exp overlaps the workspace");
  }
  std::vector<CallerMat> cm(count);
  for (int i = 0; i < count; ++i) {
    cm[i].hint = scaleExp ? scaleExp + i : nullptr;
    cm[i].src = momentum[i];
    cm[i].ldSrc = cols[i];
    cm[i].dst = params[i];
    cm[i].ldDst = cols[i];
    cm[i].grad = grads[i];
    cm[i].lrsc = (float)(lr * std::sqrt(std::max(1.0, (double)rows[i] / (double)std::max<int64_t>(cols[i], 1))));
  }
  muon_status_t s = check_device();
  if (s != MUON_OK) return s;
  return enqueue_step(Lo, cm, param_dtype, beta, eps, V, workspace, (hipStream_t)stream);
}

muon_status_t muon_step(void* const* params, const float* const* grads, float* const* momentum,
                        const int64_t* rows, const int64_t* cols, int32_t count,
                        muon_dtype_t param_dtype, float beta, float lr, int32_t steps,
                        const float coeffs[3], float eps, void* workspace, size_t workspace_bytes,
                        void* stream) {
  return muon_step_ex(params, (const void* const*)grads, momentum, rows, cols, count, param_dtype,
                      beta, lr, steps, coeffs, eps, nullptr, workspace, workspace_bytes, stream);
}

muon_status_t muon_step_selected_workspace_size(const int64_t* rows, const int64_t* cols,
                                                int32_t count, double fraction, size_t* bytes) {
  g_err.clear();
  if (!bytes) return fail(MUON_ERR_INVALID_ARG, "bytes is NULL");
  if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
  if (count > 0 && (!rows || !cols)) return fail(MUON_ERR_INVALID_ARG, "rows/cols is NULL");
  if (!std::isfinite(fraction) || !(fraction > 0.0) || fraction > 1.0)
    return fail(MUON_ERR_INVALID_ARG, "fraction must lie in (0, 1]");
  for (int i = 0; i < count; ++i) {
    muon_status_t s = check_shape(i, rows[i], cols[i]);
    if (s != MUON_OK) return s;
  }
  const float unit[3] = {1.f, 0.f, 0.f};
  SelLayout Lo;
  std::string e = sel_layout(rows, cols, count, fraction, 5, unit, &Lo);
  if (!e.empty()) return fail(MUON_ERR_INVALID_ARG, e);
  *bytes = Lo.totalBytes;
  return MUON_OK;
}

muon_status_t muon_step_selected(void* const* params, const float* const* grads,
                                 float* const* momentum, const int64_t* rows, const int64_t* cols,
                                 int32_t count, muon_dtype_t param_dtype, float beta, float lr,
                                 int32_t steps, const float coeffs[3], float eps, double fraction,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  if (count < 0) return fail(MUON_ERR_INVALID_ARG, "count < 0");
  if (!std::isfinite(fraction) || !(fraction > 0.0) || fraction > 1.0)
    return fail(MUON_ERR_INVALID_ARG, "fraction must lie in (0, 1]");
  if (count == 0) return MUON_OK;
  if (!params || !grads || !momentum || !rows || !cols)
    return fail(MUON_ERR_INVALID_ARG, "NULL pointer array");
  if (param_dtype != MUON_DTYPE_F32 && param_dtype != MUON_DTYPE_BF16)
    return fail(MUON_ERR_INVALID_ARG, "unknown param dtype");
  if (steps < 0 || steps > kMaxSteps) return fail(MUON_ERR_INVALID_ARG, "steps out of range [0, 64]");
  if (!finite3(coeffs)) return fail(MUON_ERR_INVALID_ARG, "coeffs NULL or not finite");
  if (!std::isfinite(beta) || !std::isfinite(lr))
    return fail(MUON_ERR_INVALID_ARG, "beta and lr must be finite");
  if (!std::isfinite(eps) || eps < 0) return fail(MUON_ERR_INVALID_ARG, "eps must be finite and >= 0");
  const size_t psz = param_dtype == MUON_DTYPE_F32 ? 4 : 2;
  std::vector<Range> ranges;
  for (int i = 0; i < count; ++i) {
    muon_status_t s = check_shape(i, rows[i], cols[i]);
    if (s != MUON_OK) return s;
    if (rows[i] == 0 || cols[i] == 0) continue;
    if (!params[i] || !grads[i] || !momentum[i])
      return fail(MUON_ERR_INVALID_ARG, "matrix " + std::to_string(i) + ": NULL tensor");
    const uintptr_t n = (uintptr_t)(rows[i] * cols[i]);
    ranges.push_back({(uintptr_t)params[i], (uintptr_t)params[i] + n * psz, i});
    ranges.push_back({(uintptr_t)grads[i], (uintptr_t)grads[i] + n * 4, i});
    ranges.push_back({(uintptr_t)momentum[i], (uintptr_t)momentum[i] + n * 4, i});
  }
  int oa = 0, ob = 0;
  if (overlaps(ranges, &oa, &ob))
    return fail(MUON_ERR_ALIAS, "tensors of matrices " + std::to_string(oa) + " and " +
                                    std::to_string(ob) + " overlap");
  SelLayout Lo;
  std::string e = sel_layout(rows, cols, count, fraction, steps, coeffs, &Lo);
  if (!e.empty()) return fail(MUON_ERR_INVALID_ARG, e);
  if (!workspace) return fail(MUON_ERR_WORKSPACE, "workspace is NULL");
  if ((uintptr_t)workspace & 255) return fail(MUON_ERR_WORKSPACE, "workspace not 256-byte aligned");
  if (workspace_bytes < Lo.totalBytes)
    return fail(MUON_ERR_WORKSPACE, "workspace too small: need " + std::to_string(Lo.totalBytes) +
                                        " bytes, got " + std::to_string(workspace_bytes));
  {
    int who = 0;
    if (workspace_overlaps(ranges, (uintptr_t)workspace, (uintptr_t)workspace + Lo.totalBytes, &who))
      return fail(MUON_ERR_ALIAS, "workspace overlaps a tensor of matrix " + std::to_string(who));
  }
  muon_status_t s = check_device();
  if (s != MUON_OK) return s;
  return enqueue_selected(Lo, params, grads, momentum, rows, cols, count, param_dtype, beta, lr, eps,
                          workspace, (hipStream_t)stream);
}

muon_status_t muon_set_tile_table(const muon_tile_entry_t* entries, int32_t n) {
  g_err.clear();
  if (n < 0 || n > 4096) return fail(MUON_ERR_INVALID_ARG, "n outside [0, 4096]");
  if (n > 0 && !entries) return fail(MUON_ERR_INVALID_ARG, "entries is NULL");
  std::vector<std::pair<TileKey, TileConf>> v;
  for (int i = 0; i < n; ++i) {
    const muon_tile_entry_t& e = entries[i];
    const bool okTile = e.op == OP_F16 ? (e.tile == 0 || e.tile == 128 || e.tile == 256)
                                       : (e.op == OP_F32 && (e.tile == 0 || e.tile == 32 || e.tile == 64 || e.tile == 128));
    int xs = 0;
    if (e.xcd_window != 0) {
      for (int k = 3; k <= 6; ++k)
        if (e.xcd_window == (1 << k)) xs = k;
    }
    const bool okWin = e.xcd_window == 0 || xs != 0;
    const bool okBand = e.band == 0 || e.band == 1 || e.band == 2 || e.band == 4 || e.band == 8;
    if (e.m < 1 || e.n < 0 || e.count_class < 0 || e.count_class > 31 || !okTile || !okWin || !okBand ||
        e.reserved != 0)
      return fail(MUON_ERR_INVALID_ARG, "tile entry " + std::to_string(i) + " is invalid");
    v.push_back({TileKey{e.m, e.n, e.op, e.count_class}, TileConf{e.tile, xs, e.band}});
  }
  set_tile_table(v);
  return MUON_OK;
}

muon_status_t muon_profile_enable(int32_t on) {
  g_err.clear();
  g_prof_on.store(on != 0);
  return MUON_OK;
}

muon_status_t muon_profile_read(int32_t kind, double* total_ms, int64_t* launches, double* work) {
  g_err.clear();
  if (!total_ms || !launches || !work) return fail(MUON_ERR_INVALID_ARG, "NULL output");
  double ms = 0, w = 0;
  int64_t n = 0;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  std::vector<ProfRec> keep;
  const char* err = nullptr;
  for (ProfRec& r : g_prof) {
    if (r.kind != kind || err) {  // other kinds, and everything after a failure, stay recorded
      keep.push_back(r);
      continue;
    }
    float t = 0;
    if (hipEventSynchronize(r.e1) != hipSuccess) err = "hipEventSynchronize failed";
    else if (hipEventElapsedTime(&t, r.e0, r.e1) != hipSuccess) err = "hipEventElapsedTime failed";
    if (err) {
      keep.push_back(r);
      continue;
    }
    ms += t;
    w += r.work;
    ++n;
    g_event_pool.push_back(r.e0);
    g_event_pool.push_back(r.e1);
  }
  g_prof.swap(keep);
  if (err) return fail(MUON_ERR_HIP, err);
  *total_ms = ms;
  *launches = n;
  *work = w;
  return MUON_OK;
}

}  // extern "C"
