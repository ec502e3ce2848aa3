// attn_config.h -- tile shapes shared by the planner (host) and the kernels (device).
//
// One workgroup = kWaves wavefronts of 64 lanes.  Each wavefront owns 32*QB query rows of
// one query head for the whole key sequence, so the online softmax never needs a
// cross-wave reduction.  Keys stream through LDS in tiles of BN rows.
#pragma once

namespace attn_cfg {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;

// Padding (in 16-bit elements) appended to every LDS row so that the 16-byte fragment
// reads of 8 consecutive lanes, which hit 8 consecutive rows, fall in distinct banks.
constexpr int kPad = 8;

template <int D>
struct Tile;

template <>
struct Tile<128> {
  static constexpr int QB = 1;   // 32-row query blocks per wavefront
  static constexpr int BN = 64;  // keys per LDS tile
};

template <>
struct Tile<256> {
  static constexpr int QB = 1;
  static constexpr int BN = 64;
};

constexpr int block_m(int qb) { return kWaves * 32 * qb; }

// K tile [BN][D+pad] plus transposed V tile [D][BN+pad], 16-bit elements.
constexpr int lds_bytes(int d, int bn) { return bn * (d + kPad) * 2 + d * (bn + kPad) * 2; }

}  // namespace attn_cfg
