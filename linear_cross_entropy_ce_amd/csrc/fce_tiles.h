// Tile shapes shared by the host planner and the gfx950 kernels.
//
// Every GEMM-shaped kernel computes a BM x BN output tile per workgroup of
// WAVES_M x WAVES_N wave64s, marching over K in steps of BK staged through
// LDS.  MFMA "A" rows run along M, "B" rows along N.
#pragma once

namespace fce {

template <int BM_, int BN_, int BK_, int WAVES_M_, int WAVES_N_>
struct TileShape {
  static constexpr int BM = BM_;
  static constexpr int BN = BN_;
  static constexpr int BK = BK_;
  static constexpr int WAVES_M = WAVES_M_;
  static constexpr int WAVES_N = WAVES_N_;
  static constexpr int NT = 64 * WAVES_M_ * WAVES_N_;
};

// bf16: 256 x 256 output tiles, 8 waves (two per SIMD) of 128 x 64 (32 MFMA 16x16 blocks each).
using ShapeBf16 = TileShape<256, 256, 64, 2, 4>;
// fp32: 128 x 128 output tiles, 4 waves of 64 x 64.
using ShapeF32 = TileShape<128, 128, 32, 2, 2>;

// Number of compute units the grid heuristics assume (MI355X: 256 CUs in 8 XCDs).
constexpr int kNumCUs = 256;
constexpr int kNumXCDs = 8;

}  // namespace fce
