// attn_config.h -- tile shapes shared by the planner (host) and the kernels (device).
//
// One workgroup = WAVES wavefronts of 64 lanes.  Each wavefront owns 32*QB whole query
// rows for the workgroup's whole key range, so the online softmax never needs a cross-wave
// reduction.  Keys stream through LDS in tiles of BN rows, STAGES tiles in flight.
#pragma once

namespace attn_cfg {

template <int D>
struct Tile;

// HD=128: eight wavefronts of one 32-row query block each, two per SIMD.  At this head
// dimension a wavefront's softmax VALU work is as large as at HD=256 but its MFMA work half
// as large; with two wavefronts per SIMD the hardware issues one's exponentials while the
// other's MFMAs run.  One query block keeps a wavefront within half the register file
// (64 accumulator + ~150 other registers).
template <>
struct Tile<128> {
  static constexpr int WAVES = 8;   // wavefronts per workgroup
  static constexpr int QB = 1;      // 32-row query blocks per wavefront
  static constexpr int BN = 32;     // keys per LDS tile
  static constexpr int STAGES = 4;  // K/V tiles resident in LDS at once
};

// HD=256: four wavefronts (one per SIMD) of two 32-row query blocks each, so that every K
// and V fragment read from LDS feeds two MFMAs; a wavefront needs the whole register file
// (256 accumulator registers).
template <>
struct Tile<256> {
  static constexpr int WAVES = 4;
  static constexpr int QB = 2;
  static constexpr int BN = 32;
  static constexpr int STAGES = 4;
};

template <int D>
constexpr int threads() { return Tile<D>::WAVES * 64; }

template <int D>
constexpr int block_m() { return Tile<D>::WAVES * 32 * Tile<D>::QB; }

// STAGES x (K tile + V tile), each [BN][D] 16-bit elements, plus the restart flag (16
// bytes reserved).
constexpr int lds_bytes(int d, int bn, int stages) { return stages * 2 * bn * d * 2 + 16; }

}  // namespace attn_cfg
