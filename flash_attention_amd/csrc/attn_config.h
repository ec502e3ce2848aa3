// attn_config.h -- tile shapes shared by the planner (host) and the kernels (device).
//
// One workgroup = kWaves wavefronts of 64 lanes, one wavefront per SIMD.  Each wavefront
// owns 32*QB whole query rows for the workgroup's whole key range, so the online softmax
// never needs a cross-wave reduction.  Keys stream through LDS in tiles of BN rows,
// STAGES tiles in flight.
#pragma once

namespace attn_cfg {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

template <int D>
struct Tile;

template <>
struct Tile<128> {
  static constexpr int QB = 2;      // 32-row query blocks per wavefront
  static constexpr int BN = 32;     // keys per LDS tile
  static constexpr int STAGES = 4;  // K/V tiles resident in LDS at once
};

template <>
struct Tile<256> {
  static constexpr int QB = 2;
  static constexpr int BN = 32;
  static constexpr int STAGES = 4;
};

constexpr int block_m(int qb) { return kWaves * 32 * qb; }

// STAGES x (K tile + V tile), each [BN][D] 16-bit elements, plus the restart flag (16
// bytes reserved).
constexpr int lds_bytes(int d, int bn, int stages) { return stages * 2 * bn * d * 2 + 16; }

}  // namespace attn_cfg
