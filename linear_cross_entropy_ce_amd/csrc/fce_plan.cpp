// Planner for fused linear cross-entropy.
//
// Backward block shape.  The pages chunk over tokens only: each chunk of C
// tokens produces a C x V logit slice, then dX_c = dZ_c W and dW += dZ_c^T X_c
// ("Chunked and Fused Cross-Entropy", llms.blog, "Mathematical Mechanics",
// steps 1 and 4; lesson 27, "Trick 2").  Every token chunk after the first
// re-reads and re-writes the whole fp32 dW (8 V H bytes), which on MI355X
// makes the dW product bandwidth-bound for C <= 1024.  The planner keeps the
// pages' logit-space budget of chunk x V elements but lets the block be
// C_N tokens x C_V vocabulary columns: vocabulary blocks re-read dX (N x H)
// instead of dW (V x H), which is an order of magnitude smaller at the
// large-vocabulary shapes.  The shape is picked by a simple time model
// (MFMA work with wave quantisation over 256 CUs plus fp32 RMW bytes).
#include "fce_plan.h"

#include <algorithm>
#include <cmath>
#include <limits>
#include <map>
#include <mutex>
#include <tuple>

#include "fce_tiles.h"

namespace fce {
namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return cdiv(a, b) * b; }

// Makespan of n1 equal jobs of length l1 followed by n2 of length l2, each
// started in order on the first of P workers to come free: how the hardware
// fills the CUs with the workgroups of one grid.  The first run takes
// floor(n1 / P) full rounds plus a partial one; the second run's jobs are
// identical, so it ends at the first time M by which the workers, from the
// times they come free, can have finished n2 of them.
double two_run_makespan(int64_t n1, double l1, int64_t n2, double l2, int64_t P) {
  const int64_t r1 = n1 / P, rem1 = n1 % P;
  const double ta = static_cast<double>(r1) * l1;                     // P - rem1 workers free
  const double tb = static_cast<double>(r1 + (rem1 > 0 ? 1 : 0)) * l1;  // rem1 workers free
  const double end1 = tb;
  if (n2 <= 0) return end1;
  const int64_t na = P - rem1, nb = rem1;
  auto done_by = [&](double M) {
    const double fa = std::floor((M - ta) / l2 + 1e-9), fb = std::floor((M - tb) / l2 + 1e-9);
    return static_cast<double>(na) * std::max(0.0, fa) + static_cast<double>(nb) * std::max(0.0, fb);
  };
  // the answer is ta + k l2 or tb + k l2 for some k; walk k upward
  double best = std::numeric_limits<double>::infinity();
  for (int64_t k = 1; k <= n2 / std::max<int64_t>(na, 1) + 2; ++k) {
    const double m1 = ta + static_cast<double>(k) * l2;
    if (done_by(m1) >= static_cast<double>(n2)) best = std::min(best, m1);
    const double m2 = tb + static_cast<double>(k) * l2;
    if (nb > 0 && done_by(m2) >= static_cast<double>(n2)) best = std::min(best, m2);
    if (best < m1) break;
  }
  return std::max(end1, best);
}

constexpr double kLaunchSeconds = 6e-6;  // per kernel launch
constexpr double kRmwBandwidth = 5.0e12;  // fp32 read-modify-write, bytes per second

// Time of one bf16 or fp32 output tile of the engine with contraction K.
double tile_seconds(Dtype dtype, double tile, double K) {
  const double peak = (dtype == Dtype::BF16) ? 2.5e15 : 1.5e14;
  return 2.0 * tile * tile * K / (peak / kNumCUs);
}

}  // namespace

// The dW and dX grids of a logit block of tok_tiles x voc_tiles tiles share
// one launch.  dX may be split s ways over the vocabulary (fp32 partials
// [s][block tokens][H], then a fixed-order reduce): s is the count with the
// shortest modelled time, the longer of the two tile kinds going first in the
// grid (longest first), and the partials no larger than the dZ block.
GradSchedule grad_schedule(Dtype dtype, int64_t H, int64_t tile, int64_t tok_tiles,
                           int64_t voc_tiles) {
  const int64_t h_tiles = cdiv(H, tile);
  const double t = static_cast<double>(tile);
  const double l_dw = tile_seconds(dtype, t, static_cast<double>(tok_tiles * tile));
  const int64_t elem = (dtype == Dtype::BF16) ? 2 : 4;
  const int64_t smax = std::max<int64_t>(1, std::min<int64_t>(voc_tiles / 4, 16));
  GradSchedule best{1, false, std::numeric_limits<double>::infinity()};
  for (int64_t s = 1; s <= smax; ++s) {
    if (s > 1 && s * 4 * H > voc_tiles * tile * elem) break;  // partials <= the dZ block
    const int64_t ksplit = cdiv(cdiv(voc_tiles, s), 1) * tile;  // whole tiles per split
    const int64_t splits = cdiv(voc_tiles * tile, ksplit);
    if (splits != s) continue;
    const double l_dx = tile_seconds(dtype, t, static_cast<double>(ksplit));
    const int64_t n_dw = voc_tiles * h_tiles, n_dx = tok_tiles * h_tiles * s;
    const bool dx_first = l_dx > l_dw;
    double time = dx_first ? two_run_makespan(n_dx, l_dx, n_dw, l_dw, kNumCUs)
                           : two_run_makespan(n_dw, l_dw, n_dx, l_dx, kNumCUs);
    if (s > 1)
      time += kLaunchSeconds + 4.0 * static_cast<double>(tok_tiles * tile * H) *
                                   static_cast<double>(s + 2) / kRmwBandwidth;
    if (time < best.seconds * (1.0 - 1e-9)) best = GradSchedule{s, dx_first, time};
  }
  return best;
}

namespace {

// Modelled time of one backward schedule, in seconds, per logit block:
//  - the dZ stream: `splits` workgroups per token tile, each over up to
//    ceil(tv / splits) vocabulary tiles of contraction H;
//  - dW and dX in one grid (contractions: the block's tokens, and its
//    vocabulary columns split as grad_schedule says), the longer tiles
//    first, placed as the hardware places workgroups, plus the split dX
//    partials' reduce;
//  - a fixed cost per launch;
// plus the fp32 read-modify-write bytes of dW and dX across blocks.  Only the
// ranking of candidates matters.  Blocks are full except the last in each
// dimension, so four block shapes cover the whole schedule.
double model_time(const Plan& p, int64_t CN, int64_t CV, int64_t a, int64_t b) {
  const double bw = kRmwBandwidth;
  const double t = static_cast<double>(p.tile);
  auto block = [&](int64_t cn, int64_t cv) {
    const int64_t tn = cdiv(cn, p.tile), tv = cdiv(cv, p.tile);
    const int64_t splits = std::max<int64_t>(1, std::min<int64_t>(tv, kNumCUs / tn));
    const double t_dz = two_run_makespan(
        tn * splits,
        static_cast<double>(cdiv(tv, splits)) * tile_seconds(p.dtype, t, static_cast<double>(p.H)),
        0, 0.0, kNumCUs);
    const GradSchedule g = grad_schedule(p.dtype, p.H, p.tile, tn, tv);
    return t_dz + g.seconds + 2.0 * kLaunchSeconds;
  };
  const int64_t cn_last = p.N - (a - 1) * CN, cv_last = p.V - (b - 1) * CV;
  const double time = static_cast<double>((a - 1) * (b - 1)) * block(CN, CV) +
                      static_cast<double>(a - 1) * block(CN, cv_last) +
                      static_cast<double>(b - 1) * block(cn_last, CV) + block(cn_last, cv_last);
  const double rmw = 4.0 * static_cast<double>(p.V * p.H) * static_cast<double>(2 * a - 1) +
                     4.0 * static_cast<double>(p.N * p.H) * static_cast<double>(2 * b - 1);
  return time + rmw / bw;
}

}  // namespace

namespace {

bool build_plan(int64_t N, int64_t H, int64_t V, Dtype dtype, int64_t chunk, Schedule sched,
                Plan* out, Variant variant) {
  if (!out || N < 0 || H < 1 || V < 1 || chunk < 1) return false;
  if (variant != Variant::Recompute && variant != Variant::StoreLogits &&
      variant != Variant::Filtered)
    return false;
  // the filtered products walk kept blocks of one bf16 tile
  if (variant == Variant::Filtered && dtype != Dtype::BF16) return false;
  if (sched != Schedule::Auto && sched != Schedule::Token && sched != Schedule::Vocab) return false;
  // Index arithmetic inside the kernels uses 64-bit row offsets, but tile
  // coordinates are 32-bit: keep every extent comfortably inside int32.
  const int64_t lim = static_cast<int64_t>(1) << 30;
  if (N >= lim || H >= lim || V >= lim) return false;
  // The GEMM engine addresses a 256-row operand tile with 32-bit byte
  // offsets: rows of H elements (X, W) and of the padded vocabulary width
  // (the logit block) must keep 256 rows under 2 GiB.
  const int64_t row_cap = (static_cast<int64_t>(1) << 31) / (256 * ((dtype == Dtype::BF16) ? 2 : 4));
  if (H >= row_cap || V + 512 >= row_cap) return false;
  Plan p;
  p.N = N;
  p.H = H;
  p.V = V;
  p.dtype = dtype;
  p.variant = variant;
  p.elem_bytes = (dtype == Dtype::BF16) ? 2 : 4;
  const int64_t BM = (dtype == Dtype::BF16) ? ShapeBf16::BM : ShapeF32::BM;
  const int64_t BN = (dtype == Dtype::BF16) ? ShapeBf16::BN : ShapeF32::BN;
  p.tile = std::max(BM, BN);
  const bool store = variant == Variant::StoreLogits;
  // StoreLogits: token blocks of `chunk` tokens (a whole number of loss
  // blocks, so each block's loss sums land in their own slots) by all of V;
  // the forward runs once per block.
  const int64_t store_cn =
      round_up(std::max<int64_t>(std::min(chunk, std::max<int64_t>(N, 1)), 1),
               std::max<int64_t>(p.tile, kLossBlock));
  const int64_t Nf = store ? std::min(N, store_cn) : N;

  // ---- forward grid: minimise ceil(tiles/CUs) * vocab tiles per split
  p.fwd_tok_tiles = cdiv(Nf, BN);
  p.fwd_voc_tiles = cdiv(V, BM);
  p.n_pad = std::max<int64_t>(p.fwd_tok_tiles, 1) * BN;
  if (N > 0) {
    int64_t best = 1;
    double best_cost = std::numeric_limits<double>::infinity();
    const int64_t smax = std::min<int64_t>(p.fwd_voc_tiles, 4 * kNumCUs);
    for (int64_t s = 1; s <= smax; ++s) {
      const double cost = static_cast<double>(cdiv(p.fwd_tok_tiles * s, kNumCUs)) *
                          static_cast<double>(cdiv(p.fwd_voc_tiles, s));
      if (cost < best_cost - 1e-9) {
        best_cost = cost;
        best = s;
      }
    }
    p.fwd_splits = best;
  } else {
    p.fwd_splits = 1;
  }

  // ---- backward block
  const int64_t G = p.tile;
  const double budget = static_cast<double>(chunk) * static_cast<double>(V);
  const int64_t Vp = round_up(V, G);
  if (store) {
    p.CN = store_cn;
    p.CV = Vp;
    p.a = cdiv(N, p.CN);
    p.b = 1;
  } else if (N == 0) {
    p.CN = G;
    p.CV = Vp;
    p.a = 0;
    p.b = 1;
  } else if (chunk >= N) {
    p.CN = round_up(N, G);
    p.CV = Vp;
    p.a = 1;
    p.b = 1;
  } else {
    auto vocab_split = [&](int64_t CN, int64_t* CV, int64_t* b) {
      int64_t cv_max = static_cast<int64_t>(std::floor(budget / static_cast<double>(CN) / G)) * G;
      cv_max = std::max(cv_max, G);  // never below one tile
      *b = cdiv(V, cv_max);
      *CV = round_up(cdiv(V, *b), G);
    };
    if (sched == Schedule::Token) {
      p.CN = round_up(chunk, G);
      p.a = cdiv(N, p.CN);
      p.CV = Vp;
      p.b = 1;
    } else if (sched == Schedule::Vocab) {
      p.CN = round_up(N, G);
      p.a = 1;
      vocab_split(p.CN, &p.CV, &p.b);
    } else if (sched == Schedule::Auto) {
      // Candidates: every block height, and for each the balanced widths of
      // the fewest vocabulary blocks the budget allows plus a few more, and
      // every tile multiple from half the widest width up to it (a width
      // whose grids are whole waves over the 256 CUs may leave a small last
      // block and still win).
      double best = std::numeric_limits<double>::infinity();
      auto consider = [&](int64_t CN, int64_t CV) {
        const int64_t aa = cdiv(N, CN), bb = cdiv(V, CV);
        const double t = model_time(p, CN, CV, aa, bb);
        if (t < best * (1.0 - 1e-9)) {
          best = t;
          p.CN = CN;
          p.CV = CV;
          p.a = aa;
          p.b = bb;
        }
      };
      const int64_t amax = cdiv(N, G);
      for (int64_t a = 1; a <= amax; ++a) {
        const int64_t CN = round_up(cdiv(N, a), G);
        if (cdiv(N, CN) != a) continue;  // same block height as a smaller a
        int64_t CV0, b0;
        vocab_split(CN, &CV0, &b0);
        for (int64_t b = b0; b <= b0 + 8; ++b) {
          const int64_t CV = round_up(cdiv(V, b), G);
          if (CV > CV0 && b != b0) continue;
          if (cdiv(V, CV) != b) continue;  // same block width as a smaller b
          consider(CN, CV);
        }
        for (int64_t k = std::max<int64_t>(1, CV0 / G / 2); k * G <= CV0; ++k)
          consider(CN, k * G);
      }
    } else {
      return false;
    }
  }
  p.scratch_rows = p.CN;
  // Row pitch of the dZ block: a pitch that is a multiple of 1 KiB puts the
  // same column of every row on the same memory channel, so pad such pitches
  // by one 128-byte line.
  p.ldz = p.CV;
  if ((p.ldz * p.elem_bytes) % 1024 == 0) p.ldz += 128 / p.elem_bytes;
  // ---- dX split over the vocabulary for the block's shared dW / dX grid
  if (N > 0 && variant != Variant::Filtered)
    p.dx_splits = grad_schedule(dtype, H, p.tile, cdiv(std::min(p.CN, N), BN),
                                cdiv(std::min(p.CV, V), BM))
                      .splits;
  p.grad_rmw_bytes = (N == 0) ? 4 * V * H
                              : 4 * V * H * (2 * p.a - 1) + 4 * N * H * (2 * p.b - 1);
  if (store && N > 0) p.grad_rmw_bytes = 4 * V * H * (2 * p.a - 1) + 4 * N * H;

  // ---- workspace layout
  size_t off = 0;
  p.off_ctrl = off;
  off = align_up(off + sizeof(Ctrl));
  p.off_flags = off;
  off = align_up(off + sizeof(int32_t) * static_cast<size_t>(std::max<int64_t>(p.a, 1)));
  p.off_part = off;
  p.partial_bytes = static_cast<size_t>(p.fwd_splits) * static_cast<size_t>(p.n_pad) * 16u;
  off = align_up(off + p.partial_bytes);
  p.n_loss_blocks = cdiv(std::max<int64_t>(N, 1), kLossBlock);
  p.off_blockloss = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(p.n_loss_blocks));
  p.off_lse = off;
  off = align_up(off + sizeof(float) * static_cast<size_t>(std::max<int64_t>(N, 1)));
  if (dtype == Dtype::F32) {
    p.off_stat = off;
    p.stat_bytes = 8u * static_cast<size_t>(std::max<int64_t>(N, 1));
    off = align_up(off + p.stat_bytes);
  }
  p.off_scratch = off;
  p.scratch_bytes = (N == 0) ? 0
                             : static_cast<size_t>(p.scratch_rows) * static_cast<size_t>(p.ldz) *
                                   static_cast<size_t>(p.elem_bytes);
  off = align_up(off + p.scratch_bytes);
  p.off_dxpart = off;
  p.dxpart_bytes = (p.dx_splits > 1) ? static_cast<size_t>(p.dx_splits) *
                                           static_cast<size_t>(std::min(p.CN, N)) *
                                           static_cast<size_t>(H) * sizeof(float)
                                     : 0;
  off = align_up(off + p.dxpart_bytes);
  // X^T for the dW products of the bf16 paths, taken as (dW)^T = X^T dZ when
  // token blocks hold at least 8192 tokens (the product's K): with one block
  // of 8192 to 32768 tokens it ran faster than dZ^T X, with two accumulating
  // blocks of 4096 or eight of 1024 slower.  The filtered path takes it for
  // the dW tiles that keep every token block.
  // Rows of the token extent are
  // rounded up to a tile, so that the product's K loop runs whole tiles over
  // zeros past N; 256 rows of it stay under 2 GiB (32-bit tile offsets), else
  // dW keeps the untransposed product
  if (dtype == Dtype::BF16 && N > 0 && p.CN >= 8192) {
    const int64_t ldxt = round_up(N, G);
    if (ldxt < row_cap) {
      p.ldxt = ldxt;
      p.off_xt = off;
      p.xt_bytes = static_cast<size_t>(H) * static_cast<size_t>(ldxt) * 2u;
      off = align_up(off + p.xt_bytes);
    }
  }
  if (variant == Variant::Filtered) {
    p.filt_tt = cdiv(std::min(p.CN, std::max<int64_t>(N, 1)), BN);
    p.filt_vt = cdiv(std::min(p.CV, V), BM);
    const size_t tiles = static_cast<size_t>(p.filt_tt * p.filt_vt);
    // kept flags: a region per logit block, all zeroed once per call
    p.off_keep = off;
    p.keep_bytes = tiles * static_cast<size_t>(std::max<int64_t>(p.a, 1) * std::max<int64_t>(p.b, 1));
    off = align_up(off + p.keep_bytes);
    p.off_rowlist = off;
    off = align_up(off + 4 * tiles);
    p.off_collist = off;
    off = align_up(off + 4 * tiles);
    p.off_rowcnt = off;
    off = align_up(off + 4 * static_cast<size_t>(p.filt_tt));
    p.off_colcnt = off;
    off = align_up(off + 4 * static_cast<size_t>(p.filt_vt));
    p.off_roworder = off;
    off = align_up(off + 4 * static_cast<size_t>(p.filt_tt));
    p.off_colorder = off;
    off = align_up(off + 4 * static_cast<size_t>(p.filt_vt));
  }
  p.total = off;
  *out = p;
  return true;
}

// Plans by their arguments: the block-shape search costs milliseconds (tens
// at the largest shapes), and a call that waits for it leaves the GPU idle
// when nothing of the caller's is queued ahead of it.  A plan is a pure
// function of the key, so the cache changes no result.  Guarded by a mutex;
// emptied when full.
struct PlanKey {
  int64_t N, H, V, chunk;
  int dtype, sched, variant;
  bool operator<(const PlanKey& o) const {
    return std::tie(N, H, V, chunk, dtype, sched, variant) <
           std::tie(o.N, o.H, o.V, o.chunk, o.dtype, o.sched, o.variant);
  }
};
constexpr size_t kPlanCacheSize = 256;
std::mutex g_plan_mu;
std::map<PlanKey, Plan> g_plans;

}  // namespace

bool make_plan(int64_t N, int64_t H, int64_t V, Dtype dtype, int64_t chunk, Schedule sched,
               Plan* out, Variant variant) {
  if (!out) return false;
  const PlanKey key{N, H, V, chunk, static_cast<int>(dtype), static_cast<int>(sched),
                    static_cast<int>(variant)};
  {
    std::lock_guard<std::mutex> lock(g_plan_mu);
    const auto it = g_plans.find(key);
    if (it != g_plans.end()) {
      *out = it->second;
      return true;
    }
  }
  Plan p;
  if (!build_plan(N, H, V, dtype, chunk, sched, &p, variant)) return false;
  {
    std::lock_guard<std::mutex> lock(g_plan_mu);
    if (g_plans.size() >= kPlanCacheSize) g_plans.clear();
    g_plans.emplace(key, p);
  }
  *out = p;
  return true;
}

}  // namespace fce
