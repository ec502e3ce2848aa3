// attn_config.h -- tile shapes shared by the planner (host) and the kernels (device).
//
// One workgroup = WAVES wavefronts of 64 lanes.  Each wavefront owns 32*QB whole query
// rows for the workgroup's whole key range, so the online softmax never needs a cross-wave
// reduction.  Keys stream through LDS in tiles of BN rows, STAGES tiles in flight.
//
// Two shapes per head dimension: the wide one (V = 0, 256 query rows per workgroup) for
// query blocks that fill it, and a narrow one (V = 1, 128 rows: four wavefronts of one
// 32-row block) for key/value groups with at most 128 query rows (decode-sized queries),
// which would leave most of a wide tile's matrix work on rows that do not exist.
#pragma once

namespace attn_cfg {

template <int D, int V>
struct Tile;

// HD=128: eight wavefronts of one 32-row query block each, two per SIMD.  At this head
// dimension a wavefront's softmax VALU work is as large as at HD=256 but its MFMA work half
// as large; with two wavefronts per SIMD the hardware issues one's exponentials while the
// other's MFMAs run.  One query block keeps a wavefront within half the register file
// (64 accumulator + ~150 other registers).
// Six K/V stages (96 KiB): copies two tiles ahead and one workgroup barrier per two tiles.
template <>
struct Tile<128, 0> {
  static constexpr int WAVES = 8;   // wavefronts per workgroup
  static constexpr int QB = 1;      // 32-row query blocks per wavefront
  static constexpr int BN = 32;     // keys per LDS tile
  static constexpr int STAGES = 6;  // K/V tiles resident in LDS at once
  static constexpr int PREFETCH = 2;  // key tiles between a tile's copies and its use
  static constexpr int WG_PER_CU = 1;  // workgroups per compute unit (registers, LDS)
};

// HD=256: four wavefronts (one per SIMD) of two 32-row query blocks each, so that every K
// and V fragment read from LDS feeds two MFMAs; a wavefront needs the whole register file
// (256 accumulator registers).
template <>
struct Tile<256, 0> {
  static constexpr int WAVES = 4;
  static constexpr int QB = 2;
  static constexpr int BN = 32;
  static constexpr int STAGES = 4;
  static constexpr int PREFETCH = 2;
  static constexpr int WG_PER_CU = 1;
};

// Narrow HD=128: four wavefronts of one 32-row block; 64 KiB of LDS and half the register
// file each, so two workgroups share a compute unit (two wavefronts per SIMD, as in the
// wide shape).
template <>
struct Tile<128, 1> {
  static constexpr int WAVES = 4;
  static constexpr int QB = 1;
  static constexpr int BN = 32;
  static constexpr int STAGES = 4;
  static constexpr int PREFETCH = 1;  // (two: 2.4 % slower with two workgroups per CU)
  static constexpr int WG_PER_CU = 2;
};

// Narrow HD=256: four wavefronts of one 32-row block (128 accumulator registers); the
// 128 KiB of LDS keep it at one workgroup per compute unit.
template <>
struct Tile<256, 1> {
  static constexpr int WAVES = 4;
  static constexpr int QB = 1;
  static constexpr int BN = 32;
  static constexpr int STAGES = 4;
  static constexpr int PREFETCH = 2;
  static constexpr int WG_PER_CU = 1;
};

template <int D, int V>
constexpr int threads() { return Tile<D, V>::WAVES * 64; }

template <int D, int V>
constexpr int block_m() { return Tile<D, V>::WAVES * 32 * Tile<D, V>::QB; }

// Wavefronts that share one SIMD (four SIMDs per compute unit).
template <int D, int V>
constexpr int waves_per_simd() { return Tile<D, V>::WAVES * Tile<D, V>::WG_PER_CU / 4; }

// Query rows per key/value group up to which the narrow shape is used.
constexpr int kNarrowRows = 128;

// STAGES x (K tile + V tile), each [BN][D] 16-bit elements.
constexpr int lds_bytes(int d, int bn, int stages) { return stages * 2 * bn * d * 2; }

}  // namespace attn_cfg
