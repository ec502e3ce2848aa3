// attn_fwd.hip -- fused attention forward for gfx950 (MI355X, CDNA4) and the launching half
// of the C ABI.
//
// Method: the flash-attention forward of the "Xe2 (Lunar Lake/LNL, Battlemage/BMG) ESIMD
// Flash Attention -- HD=256" page (GQA, online softmax over key tiles, one reciprocal of
// the row sum at the end: sections "Key Optimization Insights / What Worked") with the
// fp32-softmax data flow of "Xe2 Sdp Bf16" (section "Kernel Architecture: bf16io",
// data-flow diagram).  The Xe2 register and SLM choreography is not reused; the layout
// below is built around CDNA4's 32x32x16 MFMA.
//
// Work decomposition.  The G = Hq/Hkv query heads that read one key/value head are
// adjacent in Q, O and LSE, so the host hands them over as one block of G*Lq query rows
// (the grouped-query head map h -> h / G becomes row block -> key/value head).  A workgroup
// owns BLOCK_M rows of such a block and one range of keys (the whole sequence, or one split
// of it); each wavefront owns 32*QB whole rows, so a row's max and sum never cross
// wavefronts.  BLOCK_M is 256 (the wide shape), or 128 (the narrow shape: four wavefronts
// of one 32-row block) when a key/value group has no more rows than that, as with
// decode-sized queries, so that the matrix work is not spent on rows that do not exist.
// Under the causal mask a row's position in its own head is its index modulo Lq.
//
// Transposed scores.  Each wavefront computes S^T = K * Q^T with K as the MFMA A operand
// (32 keys x 16 dims) and Q^T as the B operand (16 dims x 32 queries, register resident
// for the whole key loop).  The 32x32 fp32 result then holds one query per lane column:
// lane l owns query l%32 and 16 of the 32 keys, the other 16 sitting in lane l^32.  Row
// max = an in-lane max plus one cross-half exchange (needed for the first tile, whose
// maximum is the row's softmax reference, and for the rare tile whose scores outgrow it);
// the row sum stays per-lane until the end.
// Those same registers, rounded to 16 bits, are directly the B operand of
// O^T += V^T * P^T (k index = key): no trip through LDS for P.  The key order inside the
// B operand is fixed by the accumulator layout, so V^T must be read in that same
// key order, which the transposing LDS reads of V provide.  O^T lives in 32x32 accumulators
// with one query per lane column as well.
//
// Pipeline.  K and V tiles of 32 keys are copied straight from HBM into LDS (no register
// staging) into rings of four stages.  Iteration t of the key loop reads K of tile t (S^T)
// and V of tile t-1 (the P.V product of the previous tile).  Under the S^T MFMAs run the
// copies of tile t+1 (one per few MFMA windows, no branch around any) and the rounding and
// row sums of tile t-1's weights; under the P.V MFMAs, the exponentials of tile t.  The one
// workgroup barrier of the iteration, at its end, makes tile t+1 visible to every wave.  At HD=256 each wavefront owns 64 query rows (two 32-row MFMA blocks), so every
// K and V fragment read from LDS feeds two MFMAs (in the wide shape); at HD=128 two
// wavefronts of 32 rows share each SIMD, the one in its S^T phase at the higher issue
// priority.  Q stays in registers and the output accumulator in pinned AGPRs for the whole
// key loop.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>
#include <type_traits>

#include "../../include/attn.h"
#include "attn_agpr.h"
#include "attn_config.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

struct Params {
  const uint16_t* __restrict__ q;
  const uint16_t* __restrict__ k;
  const uint16_t* __restrict__ v;
  uint16_t* __restrict__ o;  // final output (o_part == nullptr)
  float* __restrict__ lse;
  // Partial results over key splits (nullptr: one split, final output in o): split s of
  // row r at o_part[(s * part_rows + r) * D], its LSE at lse_part[s * part_rows + r].
  float* __restrict__ o_part;
  float* __restrict__ lse_part;
  int64_t part_rows;  // B * Hq * Lq
  int Hq, Hkv, G, Lq, Lk;
  int n_qtiles;
  int n_work;     // workgroups with work: n_qtiles * (row blocks) * nsplit
  int nsplit;     // key splits (workgroups per query tile)
  int split_len;  // keys per split, a multiple of the key tile (split s: [s*len, (s+1)*len))
  int diag;       // row i sees key j only if j <= i + diag (Lk - Lq if causal, else Lk)
  int causal;     // heaviest query tiles first (their key range is the longest)
  // Causal dispatch order when each head's rows fill whole query tiles (tiles_per_head
  // tiles per head): the tiles of qperm_heads consecutive heads are dealt position-major,
  // the last position of each of those heads first, then the one before it, and so on, so
  // that the workgroups running at once on an XCD see nearly the same key range (and
  // stream it through that XCD's L2 together).  qperm_heads <= 1: plain descending order.
  int qperm_heads;
  int tiles_per_head;
  // Query position of row r: r % lq_head.  The host passes the G query heads that share a
  // key/value head as one block of G*Lq rows (Hq = Hkv, G = 1 here), so a row's position
  // in its own head is its index modulo the per-head length; floor(r / lq_head) =
  // (r * lq_magic) >> lq_shift exactly for 0 <= r < 2^31.
  int lq_head;
  uint32_t lq_magic;
  int lq_shift;
  float c;        // scale * log2(e): scores are kept in base-2 units
};

// 32x32x16 MFMA issued through inline asm.  The score accumulator is pinned to VGPRs ("v":
// the softmax reads it with VALU instructions); the output accumulator lives in fixed AGPRs
// (attn_agpr.h), written only by MFMAs inside the key loop.  The compiler does not look for
// hazards inside inline asm.  The MFMA sources here are LDS/global loads or VALU results
// written far earlier, so no wait states precede the MFMAs (each s_nop in front of one
// costs about a tenth of the matrix-core rate); tests/test_kernel_asm.py checks on the
// emitted code that no VALU write lands within 2 wait states of an MFMA reading it.  Every
// VALU reader of an MFMA result is ordered behind a fence of 12 wait states (what the
// compiler's own hazard recognizer puts between this 8-pass MFMA and a VALU read on gfx950),
// also checked there.
#define ATTN_MFMA_F16 "v_mfma_f32_32x32x16_f16"
#define ATTN_MFMA_BF16 "v_mfma_f32_32x32x16_bf16"
#define ATTN_MFMA_STMTS(OPC)                                                              \
  static __device__ __forceinline__ void mfma_v0(u32x4 a, u32x4 b, f32x16& c) {           \
    asm volatile(OPC " %0, %1, %2, 0" : "=&v"(c) : "v"(a), "v"(b));                        \
  }                                                                                       \
  static __device__ __forceinline__ void mfma_v(u32x4 a, u32x4 b, f32x16& c) {            \
    asm volatile(OPC " %0, %1, %2, %0" : "+v"(c) : "v"(a), "v"(b));                        \
  }                                                                                       \
  /* the same with the B operand held in AGPRs */                                         \
  static __device__ __forceinline__ void mfma_va0(u32x4 a, u32x4 b, f32x16& c) {          \
    asm volatile(OPC " %0, %1, %2, 0" : "=&v"(c) : "v"(a), "a"(b));                        \
  }                                                                                       \
  static __device__ __forceinline__ void mfma_va(u32x4 a, u32x4 b, f32x16& c) {           \
    asm volatile(OPC " %0, %1, %2, %0" : "+v"(c) : "v"(a), "a"(b));                        \
  }

template <typename T>
struct Elt;

template <>
struct Elt<_Float16> {
  ATTN_MFMA_STMTS(ATTN_MFMA_F16)
  // output accumulator block n += a * b (block n: AGPRs 16n..16n+15)
  static __device__ __forceinline__ void acc_mfma(int n, u32x4 a, u32x4 b) {
    attn_agpr::mfma_f16(n, a, b);
  }
  // two fp32 -> two fp16, round to nearest even
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f16x2 r = __builtin_convertvector((f32x2){x, y}, f16x2);
    return __builtin_bit_cast(uint32_t, r);
  }
  // Row-sum update by a pair of weights x, y: their fp32 values (a v_dot2 of the packed
  // 16-bit values would be one instruction instead of two, but on gfx950 each dot
  // instruction placed between MFMAs holds the matrix pipe for ~20 cycles).
  static __device__ __forceinline__ float sum2(uint32_t, float x, float y, float acc) {
    return acc + (x + y);
  }
};

template <>
struct Elt<__bf16> {
  ATTN_MFMA_STMTS(ATTN_MFMA_BF16)
  static __device__ __forceinline__ void acc_mfma(int n, u32x4 a, u32x4 b) {
    attn_agpr::mfma_bf16(n, a, b);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    bf16x2 r = __builtin_convertvector((f32x2){x, y}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
  }
  // The fp32 values (bf16 rounding, 2^-8, would move the log-sum-exp by up to ~4e-3).
  static __device__ __forceinline__ float sum2(uint32_t, float x, float y, float acc) {
    return acc + (x + y);
  }
};

// Wait states between the last MFMA writing the score accumulators and any other use of
// them (see above).
template <int N>
__device__ __forceinline__ void mfma_fence_v(f32x16 (&x)[N]) {
  if constexpr (N == 1) asm volatile("s_nop 11" : "+v"(x[0]));
  else asm volatile("s_nop 11" : "+v"(x[0]), "+v"(x[1]));
}

// Materialise x here: the compiler may not sink its computation past this point (the
// softmax slices have to stay between the MFMAs they are meant to run under).
template <typename X>
__device__ __forceinline__ void pin(X& x) {
  asm volatile("" : "+v"(x));
}

// ---------------------------------------------------------------------------------------
// LDS layouts.  K and V tiles are stored row-major [key][d] exactly as in HBM, except that
// the 16-byte chunks of each row are XOR-permuted so the fragment reads are bank-conflict
// free; the permutation is applied on the global side of the direct global->LDS copy
// (lane i of a wave always lands at LDS base + 16*i, so each lane fetches the chunk that
// belongs at its slot).
//   K: chunk c of row r sits at slot c ^ (r & 15).  The S^T A-operand read (ds_read_b128)
//      serves 16 lanes per LDS cycle, here rows 0..15 (or 16..31) at one chunk: sixteen
//      distinct 16-byte slots, all 64 banks.
//   V: chunk c of row r sits at slot c ^ 4*(r & 3).  A transposing read (ds_read_b64_tr_b16)
//      serves 32 lanes per cycle: 4 consecutive rows x 64 bytes, which the XOR moves to 4
//      distinct 64-byte bank groups.
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 2; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima).
#define WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 15) | (((n) >> 4) << 14) | 0x0F70)

// Direct global->LDS copy of 16 bytes per lane (buffer_load_dwordx4 ... lds): lane i's
// bytes land at LDS address dst + 16*i (dst wave-uniform, passed in M0).  The source is a
// buffer resource (base, size in bytes) plus a per-lane byte offset: offsets at or past the
// size read as zero, which is how rows past the end of K and V are filled.  Written as
// inline asm so that the compiler does not add its own conservative vmcnt waits before every
// LDS read in the loop; completion is tracked by hand with WAIT_VMCNT + a workgroup
// barrier.  M0 is used by nothing else in these kernels.
typedef int i32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uintptr_t>(base);
  // dword3: 32-bit data format, no swizzle, raw (stride 0) addressing.  The descriptor must
  // sit in SGPRs: every field is wave-uniform, readfirstlane says so to the compiler.
  return (i32x4){__builtin_amdgcn_readfirstlane(static_cast<int>(a & 0xffffffffu)),
                 __builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)),
                 __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), 0x00020000};
}

__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t voffset, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds_dst), "v"(voffset), "s"(rsrc)
               : "memory");
}

// The key loop's copy: M0 <- wlds + dc (this wavefront's LDS slot plus a constant), the byte
// offset <- soff + voff, then the copy; the vector add between the M0 write and the copy is
// the wait state the copy needs after M0 is written.  Three instructions.
__device__ __forceinline__ void lds_dma16_loop(i32x4 rsrc, uint32_t soff, uint32_t voff,
                                               uint32_t wlds, uint32_t dc) {
  uint32_t tmp;
  asm volatile(
      "s_add_u32 m0, %1, %2\n\tv_add_u32 %0, %3, %4\n\tbuffer_load_dwordx4 %0, %5, 0 offen lds"
      : "=&v"(tmp)
      : "s"(wlds), "i"(dc), "s"(soff), "v"(voff), "s"(rsrc)
      : "memory", "scc");
}

// f(std::integral_constant<int, I>{}, t + I - I0) for I = I0 .. N-1 in order while
// t + I - I0 < n; the first t not done.
template <int I, int N, typename F>
__device__ __forceinline__ int unroll_steps(int t, int n, F&& f) {
  if constexpr (I < N) {
    if (t >= n) return t;
    f(std::integral_constant<int, I>{}, t);
    return unroll_steps<I + 1, N>(t + 1, n, static_cast<F&&>(f));
  } else {
    return t;
  }
}

// Growth threshold of the lazy rescale.  The exponentials use a per-row reference m: the
// first key tile's maximum, raised only when a later tile outgrows it by this factor.  All
// weights are non-negative, so a lane whose partial sum over a tile stays at or below the
// threshold has no weight above it.  fp16 weights must stay below 65504: the fp16 kernel
// rescales past 2^15.  bf16 weights have fp32's range, and the bf16 kernel waits until 2^24
// (row sums and the fp32 accumulator stay far from overflow).  Exact in real arithmetic for
// any m: numerator and denominator share it.
template <typename T>
constexpr float kGrowth = std::is_same<T, _Float16>::value ? 32768.0f : 16777216.0f;

// V selects the tile shape (attn_config.h): 0 wide, 1 narrow.  The second launch bound is
// the number of wavefronts that share a SIMD, which caps the registers of one wavefront.
template <int D, int V, typename T, bool NEG>
__global__ __launch_bounds__((attn_cfg::threads<D, V>()), (attn_cfg::waves_per_simd<D, V>()))
void attn_fwd_kernel(Params p) {
  constexpr int QB = attn_cfg::Tile<D, V>::QB;
  constexpr int BN = attn_cfg::Tile<D, V>::BN;
  constexpr int NSTAGE = attn_cfg::Tile<D, V>::STAGES;
  static_assert(BN == 32 && (QB == 1 || QB == 2), "one or two 32-row query blocks per wave, "
                "one 32-key block per tile");
  constexpr int THREADS = attn_cfg::threads<D, V>();
  constexpr int WAVES = attn_cfg::Tile<D, V>::WAVES;
  // Four stages, every iteration ending at a workgroup barrier: tiles t-1 (V, and K for a
  // rescale) and t are read, the copies of tile t+PF are issued in iteration t.  With PF = 1
  // the fourth stage keeps the unrolled loop's stage offsets static; with PF = 2 it holds
  // tile t+2 in flight while the barrier waits only for tile t+1, so a copy has one and a
  // half iterations to land instead of a half.  Six stages (HD=128 wide shape): copies two
  // tiles ahead, and only odd iterations end at a barrier, which then covers the two tiles
  // landed for the next two iterations (the barrier is a measured 4 % of that kernel's
  // time).
  constexpr int PF = attn_cfg::Tile<D, V>::PREFETCH;  // tiles between a tile's copies and use
  static_assert((NSTAGE == 4 && (PF == 1 || PF == 2)) || (NSTAGE == 6 && PF == 2),
                "four stages with copies one or two tiles ahead, or six with two");
  constexpr int KS = D / 16;    // contraction steps of S^T
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int TILE = BN * D;  // elements of one K (or V) tile
  constexpr int LOADS = BN * CPR / THREADS;     // 16-byte copies per thread per tile
  constexpr int ROWS_PER_LOAD = THREADS / CPR;  // tile rows one copy round covers
  static_assert(LOADS >= 1 && BN * CPR % THREADS == 0, "whole copy rounds per tile");
  constexpr int BM = attn_cfg::block_m<D, V>();
  constexpr int NSTEP = 2 * DB;  // P.V steps per tile, QB MFMAs (one per query block) each
  constexpr int NELEM = 16 * QB;  // scores per lane per tile
  constexpr int VPRE = 2;        // S^T steps before the end at which the first V reads issue
  // NEG: scale < 0, so the largest scaled score comes from the smallest raw score.
  constexpr float kWorst = NEG ? __builtin_inff() : -__builtin_inff();

  extern __shared__ u32x4 smem_raw[];
  uint16_t* const smem = reinterpret_cast<uint16_t*>(smem_raw);
  // LDS byte address of the stages, for the copy destinations (M0).
  const uint32_t lds_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_void*)smem));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, hi = lane >> 5;

  // Workgroups are dealt round-robin to the 8 XCDs; renumber so each XCD runs a contiguous
  // range of (batch, head, query tile, key split) and its concurrent workgroups share
  // key/value heads in that XCD's L2.
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
  // (integer division is expanded into VALU code; readfirstlane keeps the results in SGPRs)
  // (a grid larger than the work, which the host never launches, would find nothing here
  // rather than rows outside the tensors)
  if (logical >= p.n_work) return;
  const int split = __builtin_amdgcn_readfirstlane(logical % p.nsplit);
  const int tile_id = __builtin_amdgcn_readfirstlane(logical / p.nsplit);
  int qtile = __builtin_amdgcn_readfirstlane(tile_id % p.n_qtiles);
  // causal: the last query tiles see the most keys; dispatching them first keeps the
  // light tiles for the end of the grid
  if (p.causal) {
    if (p.qperm_heads > 1) {
      // chunk c of H heads (fewer in a last partial chunk): position rank r of head h at
      // index r*hc + h, positions from the last one down
      const int tph = p.tiles_per_head, H = p.qperm_heads;
      const int c = __builtin_amdgcn_readfirstlane(qtile / (H * tph));
      const int j = qtile - c * (H * tph);
      const int hc = min(H, p.n_qtiles / tph - c * H);
      const int r = __builtin_amdgcn_readfirstlane(j / hc);
      qtile = (c * H + (j - r * hc)) * tph + (tph - 1 - r);
    } else {
      qtile = p.n_qtiles - 1 - qtile;
    }
  }
  // (row blocks as the host passes them: with each key/value group as one block, p.Hq =
  // Hkv and p.G = 1)
  const int bh = __builtin_amdgcn_readfirstlane(tile_id / p.n_qtiles);  // b*p.Hq + hq
  const int hq = __builtin_amdgcn_readfirstlane(bh % p.Hq);
  const int b = __builtin_amdgcn_readfirstlane(bh / p.Hq);
  const int hkv = __builtin_amdgcn_readfirstlane(hq / p.G);

  // Position of row r in its head's query sequence (rows of several heads may share a
  // workgroup or a wavefront).
  auto pos_of = [&](int r) {
    const int hd = static_cast<int>((static_cast<uint64_t>(static_cast<uint32_t>(r)) *
                                     p.lq_magic) >> p.lq_shift);
    return r - hd * p.lq_head;
  };
  // Largest position among rows first..last: the last row's, unless they cross into the
  // next head (then some row is its head's last).
  auto max_pos = [&](int first, int last) {
    return pos_of(first) + (last - first) >= p.lq_head ? p.lq_head - 1 : pos_of(last);
  };
  // Smallest position among rows first..last.
  auto min_pos = [&](int first, int last) {
    return pos_of(first) + (last - first) >= p.lq_head ? 0 : pos_of(first);
  };

  // Keys of this workgroup: its split [kbeg, kbeg + split_len), cut at Lk and, under the
  // causal mask, after the last key its rows see.  Tile t holds keys
  // kbeg + 32t .. kbeg + 32t + 31.
  const int Lk = p.Lk;
  const int kbeg = min(split * p.split_len, Lk);
  const int qlast = min(qtile * BM + BM - 1, p.Lq - 1);
  const int imax = __builtin_amdgcn_readfirstlane(max_pos(qtile * BM, qlast));
  const int kend = min(min(Lk, kbeg + p.split_len), imax + p.diag + 1);
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const uint16_t* qh = p.q + (size_t)bh * p.Lq * D;
  const uint16_t* kh = p.k + (((size_t)b * p.Hkv + hkv) * p.Lk + kbeg) * D;
  const uint16_t* vh = p.v + (((size_t)b * p.Hkv + hkv) * p.Lk + kbeg) * D;
  const int qrow0 = qtile * BM + wave * 32 * QB;
  // Key limits relative to kbeg: keys past key_lim do not exist, and row r sees keys up
  // to r + row_off.  Every row of this wave sees keys 0..wave_lim; tiles past that need
  // masks.
  const int key_lim = Lk - 1 - kbeg;
  const int row_off = p.diag - kbeg;
  const int wave_lim =
      min(key_lim, __builtin_amdgcn_readfirstlane(min_pos(qrow0, qrow0 + 32 * QB - 1)) + row_off);

  // ---- direct HBM->LDS copies of K and V tiles ----
  // Copy round i of this thread moves tile row r = i*ROWS_PER_LOAD + r0, 16-byte chunk c0
  // (r0, c0 fixed per lane), into LDS slot i*THREADS + tid.  The buffer starts at the tile and
  // holds the bytes left in K (V), so rows past Lk read as zeros (their scores are masked,
  // their weights zero).  The K swizzle depends on i only through its parity (when a round
  // covers 8 rows), the V swizzle not at all.
  uint32_t vk[2], vv;
  {
    const int pos0 = wave * 64 + lane;
    const int r0 = pos0 / CPR, c0 = pos0 % CPR;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      vk[par] = static_cast<uint32_t>(r0 * D * 2 + (c0 ^ swz_k(par * ROWS_PER_LOAD + r0)) * 16);
    vv = static_cast<uint32_t>(r0 * D * 2 + (c0 ^ swz_v(r0)) * 16);
  }
  // Bytes of K (V) this workgroup may copy: its tiles, cut at the end of K (V).  One buffer
  // descriptor per tensor covers them for the whole sweep (base: this workgroup's first
  // key); a copy's byte offset at or past the size reads zeros, which fills the rows past Lk
  // of a partial last tile, and the copies of tiles past the last one (the key loop issues
  // the copies of tile t+PF without checking it against ntiles, which would cost a branch
  // per copy) read zeros or, where their 32-bit offset wraps, bytes inside the buffer; the
  // stages they fill are never read.  The offsets of the tiles that are read stay below
  // 2^32: the validation keeps Lk*D below 2^31, and D (128 or 256) divides 2^31 by a
  // multiple of 32 keys, so ntiles*TILE*2 <= 2^32.
  // (64-bit: ntiles*TILE*2 reaches 2^32 at the longest key sequences; the K bytes stay
  // below it)
  const uint32_t kv_lim = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(
      min(static_cast<uint64_t>(Lk - kbeg) * D * 2, static_cast<uint64_t>(ntiles) * TILE * 2)));
  const i32x4 krs = make_rsrc(kh, kv_lim), vrs = make_rsrc(vh, kv_lim);
  // Copy j (0 <= j < 2*LOADS) of this thread's share of tile t, into stage st: K copy
  // round j/2 for even j, V round j/2 for odd j.  Per copy: the LDS destination into M0,
  // one vector add for the byte offset, the copy.
  const uint32_t wlds = __builtin_amdgcn_readfirstlane(lds_base + wave * 64 * 16);
  auto issue_copy = [&](int t, int st, int j) {
    const bool isv = j & 1;
    const int i = j >> 1;
    const uint32_t dc = (st + (isv ? NSTAGE : 0)) * 2 * TILE + i * THREADS * 16;
    const uint32_t off = static_cast<uint32_t>(t) * (TILE * 2) + i * ROWS_PER_LOAD * D * 2;
    lds_dma16_loop(isv ? vrs : krs, off, isv ? vv : vk[i & 1], wlds, dc);
  };
  // Six stages (the HD=128 wide shape, two wavefronts per SIMD): inside the key loop only
  // the first half of the wavefronts copies (waves w and w + WAVES/2 share a SIMD), so that
  // the second half can meet the barrier at another point of its iteration than the first
  // (see the sync point below); elsewhere every thread copies, as in the prologue.
  constexpr bool PP = NSTAGE == 6;
  constexpr int CT = PP ? THREADS / 2 : THREADS;  // threads that copy inside the key loop
  constexpr int LOADS_L = BN * CPR / CT;           // their copies per tile, K (or V)
  constexpr int ROWS_L = CT / CPR;
  static_assert(LOADS_L >= 1 && BN * CPR % CT == 0, "whole copy rounds per tile");
  uint32_t vkL[2], vvL;
  {
    const int pos0 = (wave * 64 + lane) % CT;
    const int r0 = pos0 / CPR, c0 = pos0 % CPR;
#pragma unroll
    for (int par = 0; par < 2; ++par)
      vkL[par] = static_cast<uint32_t>(r0 * D * 2 + (c0 ^ swz_k(par * ROWS_L + r0)) * 16);
    vvL = static_cast<uint32_t>(r0 * D * 2 + (c0 ^ swz_v(r0)) * 16);
  }
  // Copy j (0 <= j < 2*LOADS_L) of a copying thread's share of tile t, as issue_copy with
  // CT threads.
  auto issue_copy_loop = [&](int t, int st, int j) {
    const bool isv = j & 1;
    const int i = j >> 1;
    const uint32_t dc = (st + (isv ? NSTAGE : 0)) * 2 * TILE + i * CT * 16;
    const uint32_t off = static_cast<uint32_t>(t) * (TILE * 2) + i * ROWS_L * D * 2;
    lds_dma16_loop(isv ? vrs : krs, off, isv ? vvL : vkL[i & 1], wlds, dc);
  };
  auto issue_tile = [&](int t, int st) {
#pragma unroll
    for (int j = 0; j < 2 * LOADS; ++j) issue_copy(t, st, j);
  };

  // With two wavefronts per SIMD (HD=128) a wavefront has 256 registers, which the compiler
  // splits evenly between VGPRs and AGPRs once AGPRs are in use; the Q^T fragments, read
  // only by the S^T MFMAs, then live in AGPRs next to the output accumulator.
  constexpr bool Q_AGPR = attn_cfg::waves_per_simd<D, V>() > 1;
  // Q^T operand fragments, register resident for the whole key loop: lane l holds query
  // row l%32 of block qb, dims 16*kk + 8*(l/32) .. +7.  Q is staged once in LDS: direct
  // copies of 1 KiB of contiguous bytes each (loaded straight into this layout, every
  // instruction would touch 32 rows), then one 16-byte LDS read per fragment.  A 32-row
  // query block is as large as a K tile, so block b of the workgroup takes one stage slot,
  // slot s at byte s*TILE*2 (the K stages 0-3, then the V stages 0-3).  The narrow shape's
  // four blocks avoid the slots of tile 0 (K and V of stage 0), whose copies run beside
  // Q's; the wide shape's eight fill the LDS, and tile 0 is copied once they are read.
  // Within a slot, chunk c of row r sits at position c ^ (r % CPR): the 32 rows of one
  // fragment read spread over distinct banks.  Rows past Lq re-read row Lq-1 (never
  // stored).
  constexpr int NQB = BM / 32;                           // query blocks per workgroup
  constexpr bool Q_FILLS_LDS = NQB > 2 * (NSTAGE - PF);  // the first tiles wait for Q
  constexpr int QCOPY_PER_BLOCK = TILE * 2 / 1024;       // 1 KiB copies per block
  constexpr int QCOPIES = NQB * QCOPY_PER_BLOCK / WAVES;  // per wave
  static_assert(NQB <= 2 * NSTAGE && QCOPIES * WAVES == NQB * QCOPY_PER_BLOCK,
                "Q fits the stage slots, in whole copies per wave");
  // (the slots of tiles 0 .. PF-1 are K stages 0 .. PF-1 and V stages 0 .. PF-1)
  auto qslot = [](int b) { return Q_FILLS_LDS ? b : b < NSTAGE - PF ? b + PF : b + 2 * PF; };
  {
    const i32x4 qrsrc = make_rsrc(qh, static_cast<uint32_t>(p.Lq) * D * 2);
    if (!Q_FILLS_LDS && ntiles > 0) {
#pragma unroll
      for (int t0 = 0; t0 < PF; ++t0) issue_tile(t0, t0);
    }
#pragma unroll
    for (int j = 0; j < QCOPIES; ++j) {
      const int n = wave + WAVES * j;
      const int b = n / QCOPY_PER_BLOCK, i = n % QCOPY_PER_BLOCK;
      const int pos = i * 1024 + 16 * lane;  // byte of the slot this lane fills
      const int r = pos / (2 * D);
      const int c = ((pos % (2 * D)) / 16) ^ (r % CPR);
      const int row = min(qtile * BM + 32 * b + r, p.Lq - 1);
      lds_dma16(qrsrc, static_cast<uint32_t>(row * D * 2 + 16 * c),
                lds_base + static_cast<uint32_t>(qslot(b) * TILE * 2 + i * 1024));
    }
    WAIT_VMCNT(0);
    __syncthreads();
  }
  u32x4 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const char* qs = reinterpret_cast<const char*>(smem) + qslot(wave * QB + qb) * TILE * 2 +
                     l32 * D * 2;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk)
      qf[qb][kk] = *reinterpret_cast<const u32x4*>(qs + 16 * ((2 * kk + hi) ^ (l32 % CPR)));
  }
  if constexpr (Q_FILLS_LDS) {
    __syncthreads();  // every wave has its Q: the slots take the first tiles
    if (ntiles > 0) {
#pragma unroll
      for (int t0 = 0; t0 < PF; ++t0) issue_tile(t0, t0);
    }
  }

  // ---- per-lane LDS byte offsets of the fragment reads (stage base added later) ----
  // K (A operand of S^T): row l%32, chunk 2kk+hi at slot (2kk+hi) ^ sw, sw = swz_k(l%32);
  // in bytes that is (32kk) ^ k0 with k0 below 256, added to the row start.
  const int sw = swz_k(l32);
  const uint32_t krow = static_cast<uint32_t>(l32 * D * 2);
  const uint32_t k0 = static_cast<uint32_t>(16 * (hi ^ (sw & 1)) + 32 * (sw >> 1));
  // V^T (A operand of O^T) through ds_read_b64_tr_b16: in each 16-lane block, source lane
  // 4e+c supplies row (key) e, 4 dims at 4c of the block's 16 dims; lane i then receives
  // dim i of those 4 rows.  Lane block b16 = lane/16: half h = b16/2 selects keys 4h..4h+3
  // (of each group of 8), b16%2 selects dims 16..31 of the 32-dim block db.  The chunk of
  // those dims sits at slot (4db + 2*(b16%2) + c/2) ^ 4e: in bytes (64db) ^ v0, v0 < 256.
  // With the row start (a multiple of 256) and the 8-byte half (bit 3) that is
  // vbase ^ (64*(db%4)) + 256*(db/4): the XOR touches bits 6-7 only.
  uint32_t vbase;
  {
    const int b16 = lane >> 4, e = (lane >> 2) & 3, c = lane & 3;
    const int h = b16 >> 1, dh = b16 & 1;
    const uint32_t v0 = static_cast<uint32_t>(16 * (2 * dh + (c >> 1)) + 64 * e);
    vbase = static_cast<uint32_t>((4 * h + e) * D * 2 + (c & 1) * 8) + v0;
  }
  const char* const smem_b = reinterpret_cast<const char*>(smem);

  // Output accumulator O^T, block (qb, db) = AGPR block qb*DB + db (pinned, attn_agpr.h).
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -__builtin_inff();
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) attn_agpr::zero(qb * DB + db);
  }
  const float c = p.c;

  // ---- building blocks of one key-loop iteration ----
  // LDS: the K tiles of the four stages, then their V tiles.  Each ring spans at most
  // 64 KiB, so with the stage known at compile time the stage offset is the immediate
  // offset of the LDS reads (no address arithmetic in the loop).
  auto kstage = [&](int st) { return smem_b + st * 2 * TILE; };
  // K fragment kk of a tile: the A operand of S^T step kk.
  auto kfrag = [&](const char* ks, int kk) {
    return *reinterpret_cast<const u32x4*>(ks + krow + ((32u * kk) ^ k0));
  };
  // S^T(t) = K(t) Q^T, fp32 accumulation, the QB query blocks sharing each K fragment.  The
  // first two fragments arrive prefetched in kf[0..1]; the rest are fetched two steps ahead,
  // and the scheduling barriers keep the compiler from hoisting all of them (64 registers).
  // Where two wavefronts share a SIMD (HD=128), the one in this MFMA-only phase gets the
  // higher issue priority, so that its MFMAs go out while the other wavefront's softmax
  // VALU work fills the gaps (measured: +1.6 % at 8K x 8K, +3.7 % of the cycles with the
  // clock unconstrained; the level does not matter).
  constexpr bool kShareSimd = attn_cfg::waves_per_simd<D, V>() > 1;
  // window(w) places VALU work after MFMA w (w = kk*QB + qb) of the phase, to run under it.
  auto qk = [&](const char* ks, f32x16 (&sacc)[QB], u32x4 (&kf)[3], auto&& tail_loads,
                auto&& window) {
    if constexpr (kShareSimd) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      if (kk + 2 < KS) kf[(kk + 2) % 3] = kfrag(ks, kk + 2);
      if (kk == KS - VPRE) tail_loads();  // first V fragments of the P.V steps
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (Q_AGPR) {
          if (kk == 0) Elt<T>::mfma_va0(kf[kk % 3], qf[qb][kk], sacc[qb]);
          else Elt<T>::mfma_va(kf[kk % 3], qf[qb][kk], sacc[qb]);
        } else {
          if (kk == 0) Elt<T>::mfma_v0(kf[kk % 3], qf[qb][kk], sacc[qb]);
          else Elt<T>::mfma_v(kf[kk % 3], qf[qb][kk], sacc[qb]);
        }
        __builtin_amdgcn_sched_barrier(0);
        window(kk * QB + qb);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if constexpr (kShareSimd) __builtin_amdgcn_s_setprio(0);
  };
  auto no_window = [](int) {};
  // One P.V step s of a tile: V^T fragment (32 dims x 16 keys) for MFMA step s, times both
  // P^T blocks.  MFMA step ks covers keys 16ks..16ks+15; its P^T operand is accumulator
  // registers 8ks..8ks+7, whose keys for lane half h are 16ks + {4h..4h+3, 8+4h..8+4h+3}:
  // the two transposing reads (rows +0 and +8) fetch exactly those rows of V.
  // Per-lane LDS byte addresses of V fragment group j = db % 4 in stage 0 of the V ring
  // (laundered, so that the stage and the remaining offsets stay immediate offsets of the
  // reads instead of being folded into per-stage address registers).
  uint32_t vlane[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vlane[j] = lds_base + NSTAGE * 2 * TILE + (vbase ^ (64u * j));
    asm volatile("" : "+v"(vlane[j]));
  }
  auto vfrag_load = [&](int st, int s) -> u32x4 {
    const int db = s >> 1, ks16 = s & 1;
    const uint32_t base = vlane[db & 3] + st * 2 * TILE + 256 * (db >> 2) + 16 * ks16 * D * 2;
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(base));
    const s16x4 up =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(uintptr_t)(base + 8 * D * 2));
    const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), up2 = __builtin_bit_cast(u32x2, up);
    return (u32x4){lo2[0], lo2[1], up2[0], up2[1]};
  };

  // Online softmax of tile t, fp32 in base 2, in slices that run underneath the P.V MFMAs
  // of tile t-1.  Max slices (first tile only): its row maximum per query block, which sets
  // the reference.  Exp slices: P = exp2(c*s - m) element by element, rounding to 16 bits,
  // partial row sums.
  float mt[QB];
  auto mask_keys = [&](f32x16 (&sacc)[QB], int t) {
    // Keys past Lk, and under the causal mask keys past a row's diagonal: the score becomes
    // the worst value, so the key drops out of the maximum and its weight
    // exp2(c*score - m) is exactly 0.  Accumulator register r of this lane holds key
    // kbeg + t*BN + 8*(r/4) + 4*hi + r%4 of query row qrow0 + 32*qb + l%32.  Only tiles
    // past the wave's common limit get here (the last tile, the diagonal band).
    if (__builtin_expect(t * BN + BN - 1 > wave_lim, 0)) {
      // (t laundered: the per-register compares must not be hoisted out of the loop as
      // 16 loop-invariant lane masks held in scalar registers; the lane index recomputed
      // here rather than kept live across the loop)
      int tt = t;
      asm volatile("" : "+s"(tt));
      const int ln = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = qrow0 + qb * 32 + (ln & 31);
        const int lim = min(key_lim, pos_of(row) + row_off) - tt * BN - 4 * (ln >> 5);
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + (r & 3) > lim) sacc[qb][r] = kWorst;
      }
    }
  };
  // Largest scaled score: max (min for a negative scale) as a tree of depth 3 over the 16
  // registers, so that no long chain of dependent instructions holds up the MFMA issue.
  auto ext3 = [](float a, float b, float d) {
    float r;
    if constexpr (NEG) asm("v_min3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(d));
    else asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(d));
    return r;
  };
  auto ext2 = [](float a, float b) {
    float r;
    if constexpr (NEG) asm("v_min_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    else asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
  };
  auto row_max = [&](f32x16 (&sacc)[QB], int qb) {
    const f32x16& a = sacc[qb];
    const float m0 = ext3(a[0], a[1], a[2]), m1 = ext3(a[3], a[4], a[5]);
    const float m2 = ext3(a[6], a[7], a[8]), m3 = ext3(a[9], a[10], a[11]);
    const float m4 = ext3(a[12], a[13], a[14]);
    float x = ext2(ext3(m0, m1, m2), ext3(m3, m4, a[15]));
    // the other 16 keys of this row sit in lane l^32
    const auto sw2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                      false, false);
    x = ext2(__uint_as_float(sw2[0]), __uint_as_float(sw2[1]));
    mt[qb] = x * c;  // this tile's maximum of scale*log2(e)*score for the row
    pin(mt[qb]);
  };
  // The first tile fixes the reference: m = its row maximum.
  auto set_reference = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m[qb] = fmaxf(m[qb], mt[qb]);
  };
  // A row that sees no key of this split (causal mask) has m = -inf; any finite reference
  // then gives it weights exp2(-inf) = 0, an empty sum and LSE -inf.  (A row that sees any
  // key of the split sees its first key, so its first tile has a finite maximum.)
  auto finite_reference = [&]() {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) m[qb] = m[qb] == -__builtin_inff() ? 0.f : m[qb];
  };
  // Weights of a tile in two halves.  Under the P.V MFMAs of iteration t: the exponentials
  // of tile t, ew = exp2(c*s - m), kept in fp32 (element e: register e%16 of query block
  // e/16).  Under the S^T MFMAs of iteration t+1, whose windows have no other VALU work:
  // ew rounded to 16 bits in the register layout of the P^T operand (pw), the partial row
  // sums lt, and the growth check, just before the P.V MFMAs of iteration t+1 read pw.
  float ew[QB][16], lt[QB];
  u32x4 pw[QB][2];
  auto exp_slice = [&](f32x16 (&sacc)[QB], int e0, int e1) {
#pragma unroll
    for (int e = e0; e < e1; ++e) {
      const int qb = e >> 4, r = e & 15;
      ew[qb][r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][r], c, -m[qb]));
      pin(ew[qb][r]);
    }
  };
  // pairs p0..p1-1 of ew (pair p: elements 2p, 2p+1) into pw, with their partial row sums
  auto pack_slice = [&](int p0, int p1) {
#pragma unroll
    for (int p = p0; p < p1; ++p) {
      const int qb = (2 * p) >> 4, r = (2 * p) & 15;
      uint32_t w = Elt<T>::pack2(ew[qb][r], ew[qb][r + 1]);
      pin(w);
      // this tile's part of the row sum (lane-local 16 keys)
      lt[qb] = Elt<T>::sum2(w, ew[qb][r], ew[qb][r + 1], r == 0 ? 0.f : lt[qb]);
      pw[qb][r >> 3][(r & 7) >> 1] = w;
    }
  };
  // Lazy rescale of tile tp, after its weights are packed (the deferred compensation of the
  // online softmax, "Key Optimization Insights / What Worked" of the HD=256 page, done only
  // where a tile's scores outgrow the reference).  A lane whose partial sum of the tile's
  // weights exceeds kGrowth holds a weight above it (weights are non-negative).  For each
  // query block where any lane does, the wave raises each row's reference to the tile's
  // maximum where that is larger, m' = max(m, mt), multiplies the row's output accumulator
  // and sum by exp2(m - m') <= 1, and recomputes the tile's weights against m' (now at most
  // 1).  The accumulator then holds tiles 0..tp-1 against m', as the P.V product of tile tp
  // expects.  The scores of tile tp are computed again from K(tp), still in its LDS stage
  // (until tile tp+4 is copied), into sacc; sacc held the scores of tile tp+1, which are
  // then computed once more from K(tp+1) (ksr; nullptr: nothing to restore).  Each wave
  // decides for its own rows; no other wave waits beyond the next barrier.
  auto rescale_if_grown = [&](int tp, const char* ksp, const char* ksr, f32x16 (&sacc)[QB]) {
    bool grown[QB], any = false;  // per query block, wave-uniform
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      grown[qb] = __builtin_amdgcn_ballot_w64(lt[qb] > kGrowth<T>) != 0;
      any |= grown[qb];
    }
    if (__builtin_expect(!any, 1)) return;
    u32x4 kf2[3];
    kf2[0] = kfrag(ksp, 0);
    kf2[1] = kfrag(ksp, 1);
    qk(ksp, sacc, kf2, [] {}, no_window);
    mfma_fence_v(sacc);
    mask_keys(sacc, tp);
    attn_agpr::fence();  // the last P.V MFMA's results have landed
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (!grown[qb]) continue;  // that block's rows keep their reference
      row_max(sacc, qb);
      const float mn = fmaxf(m[qb], mt[qb]);
      const float delta = __builtin_amdgcn_exp2f(m[qb] - mn);
      m[qb] = mn;
      l[qb] *= delta;
      // this block's weights against m', a pair at a time (the scheduling barriers keep the
      // compiler from computing all of them before packing any)
#pragma unroll
      for (int e = 16 * qb; e < 16 * qb + 16; e += 2) {
        exp_slice(sacc, e, e + 2);
        pack_slice(e / 2, e / 2 + 1);
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) attn_agpr::scale(qb * DB + db, delta);
    }
    attn_agpr::fence_write();
    if (ksr != nullptr) {
      kf2[0] = kfrag(ksr, 0);
      kf2[1] = kfrag(ksr, 1);
      qk(ksr, sacc, kf2, [] {}, no_window);
    }
  };

  constexpr int NCOPY = 2 * LOADS;      // copies per thread and tile (prologue)
  constexpr int NCOPY_L = 2 * LOADS_L;  // the same inside the key loop, per copying thread

  // Synchronisation point at the end of iteration t.  Four stages (every iteration): tile
  // t+1 has landed everywhere (copied in iteration t, or t-1 with PF = 2, whose copies of
  // tile t+2 may still be in flight: a wave waits until at most its own NCOPY newest copies
  // are), and every wave is done with tile t-1, so the next iteration may read tile t+1 and
  // copy tile t+1+PF into the stage of tile t+1+PF-4.  Six stages (odd t only; only the
  // first half of the wavefronts copies, and the second half meets this barrier in the
  // middle of its S^T phase of iteration t, about three quarters of an iteration behind, so
  // that the two wavefronts of a SIMD do not fall into the same phase): the copying
  // wavefronts have waited for their copies of tiles t+1 and t+2 (issued in iterations t-1
  // and t), so those tiles have landed everywhere; every wave has finished iteration t-1.
  // Until the next barrier the first half runs iterations t+1, t+2 and copies tiles t+3 and
  // t+4 into the stages of tiles t-3 and t-2, which no wave reads any more; the second half
  // reads tiles t-1 .. t+2 only (the rest of iteration t, iteration t+1 and half of the
  // S^T phase of iteration t+2), all landed.
  auto sync_point = [&]() {
    if constexpr (NSTAGE == 4 && PF == 2) {
      WAIT_VMCNT(NCOPY_L);  // this thread's copies of tile t+1 (those of t+2 may fly)
    } else {
      WAIT_VMCNT(0);  // this thread's copies of the tiles to come (after the last tile:
                      // those of the tiles past it)
    }
    // A bare s_barrier: every LDS read of this iteration has been waited for by the MFMA
    // that consumed it.
    __builtin_amdgcn_s_barrier();
  };

  // One key-loop iteration for tile t: S^T(t) = K(t) Q^T, then the P.V MFMAs of tile t-1
  // (PV) with the softmax of tile t in slices underneath.
  u32x4 kf[3];
  constexpr int NPAIR = NELEM / 2;  // packed weight pairs per lane and tile
  // ST = t % NSTAGE, a compile-time constant: the key loop is unrolled by NSTAGE.
  auto iteration = [&](auto pv_tag, auto st_tag, auto gb_tag, int t, f32x16 (&sacc)[QB]) {
    constexpr bool PV = decltype(pv_tag)::value;
    constexpr int ST = decltype(st_tag)::value;
    constexpr bool GB = decltype(gb_tag)::value;  // the second half of the wavefronts (PP)
    constexpr int VST = (ST + NSTAGE - 1) % NSTAGE;  // stage of tile t-1
    u32x4 vf[3];
    // S^T(t); under its MFMAs the weights of tile t-1 are packed, and the copies of tile
    // t+PF issued into the stage of tile t+PF-NSTAGE (t-3, or t-4 with six stages: free,
    // every wave is past the iteration that last read it), copy j after MFMA j*W/NCOPY
    constexpr int W = QB * KS;  // S^T windows
    static_assert(W % NCOPY_L == 0, "whole S^T windows per copy");
    qk(kstage(ST), sacc, kf,
       [&]() {
         if constexpr (PV) {
           vf[0] = vfrag_load(VST, 0);
           vf[1] = vfrag_load(VST, 1);
         }
       },
       [&](int w) {
         // the second half of the wavefronts meets the barrier of odd iterations here, in
         // the middle of its S^T phase (it has no copies of its own in flight)
         if constexpr (GB && ST % 2 == 1) {
           if (w == W / 2) __builtin_amdgcn_s_barrier();
         }
         if constexpr (PV) pack_slice(NPAIR * w / W, NPAIR * (w + 1) / W);
         if constexpr (!GB) {
           if (w % (W / NCOPY_L) == 0)
             issue_copy_loop(t + PF, (ST + PF) % NSTAGE, w / (W / NCOPY_L));
         }
       });
    if constexpr (PV) {
      rescale_if_grown(t - 1, kstage(VST), kstage(ST), sacc);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) l[qb] += lt[qb];
    }
    // Each P.V step is QB sub-steps: one MFMA (query block qb), then a slice of VALU or
    // copy work that issues while that MFMA runs.  A wave issues in order, so work placed
    // after an MFMA overlaps it only until the next MFMA: one sub-step per MFMA gives
    // every MFMA its own window.  Exponentials are spread about one per window over all
    // sub-steps after the first (tile 0: after its row maxima).
    constexpr int H = QB * NSTEP;          // sub-steps
    constexpr int EXP0 = PV ? 1 : QB + 1;  // first sub-step with exponentials
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      if constexpr (PV) {
        if (s + 2 < NSTEP) vf[(s + 2) % 3] = vfrag_load(VST, s + 2);
      }
#pragma unroll
      for (int hb = 0; hb < QB; ++hb) {
        const int h = QB * s + hb;
        if constexpr (PV) Elt<T>::acc_mfma(hb * DB + (s >> 1), vf[s % 3], pw[hb][s & 1]);
        __builtin_amdgcn_sched_barrier(0);
        if (h == 0) {
          mfma_fence_v(sacc);
          mask_keys(sacc, t);
        }
        // tile 0 only: its row maxima fix the reference
        if (!PV && h < QB) row_max(sacc, h);
        if (!PV && h == QB) {
          set_reference();
          finite_reference();
        }
        if (h >= EXP0)
          exp_slice(sacc, NELEM * (h - EXP0) / (H - EXP0), NELEM * (h - EXP0 + 1) / (H - EXP0));
        // (six stages: odd iterations only; the stage parity is the iteration's parity)
        if (h == H - 1 && (NSTAGE == 4 || (ST % 2 == 1 && !GB))) sync_point();
        if (h == H - 1) {
          // first two K fragments of tile t+1 (landed at the sync point; after the last
          // tile an unused stage: reading it is harmless, a branch around it is not)
          kf[0] = kfrag(kstage((ST + 1) % NSTAGE), 0);
          kf[1] = kfrag(kstage((ST + 1) % NSTAGE), 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  // The last tile: its weights packed (with the growth check), then its P.V product.
  auto drain = [&](int t, f32x16 (&sacc)[QB]) {
    const int st = t % NSTAGE;
    pack_slice(0, NPAIR);
    rescale_if_grown(t, kstage(st), nullptr, sacc);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) l[qb] += lt[qb];
    u32x4 vf[3];
    vf[0] = vfrag_load(st, 0);
    vf[1] = vfrag_load(st, 1);
#pragma unroll
    for (int s = 0; s < NSTEP; ++s) {
      if (s + 2 < NSTEP) vf[(s + 2) % 3] = vfrag_load(st, s + 2);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        Elt<T>::acc_mfma(qb * DB + (s >> 1), vf[s % 3], pw[qb][s & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // ---- the key loop ----
  // The weights use a per-row reference m set by the first key tile instead of a maximum
  // kept up to date at every tile, so the output accumulator is rescaled only in the rare
  // tile whose scores outgrow m by more than a factor kGrowth (rescale_if_grown).  The loop
  // is unrolled by NSTAGE: the stage of each iteration is a compile-time constant.
  f32x16 sacc[QB];  // scores of the current tile
  // (a workgroup with no key to look at, under the causal mask or past the last split,
  // skips the loop: its rows are empty)
  if (ntiles > 0) {
    WAIT_VMCNT(0);  // the first tiles landed
    __syncthreads();
    kf[0] = kfrag(kstage(0), 0);
    kf[1] = kfrag(kstage(0), 1);
    // unrolled by NSTAGE: iteration t runs with stage t % NSTAGE as a compile-time constant;
    // one copy of the loop per half of the wavefronts where they differ (PP)
#define ATTN_ITER(J, GBT)                                                                 \
  iteration(std::true_type{}, std::integral_constant<int, (1 + (J)) % NSTAGE>{}, GBT{}, t, \
            sacc);                                                                        \
  if (++t >= ntiles) break;
#define ATTN_KEY_LOOP(GBT)                                                                \
  {                                                                                       \
    iteration(std::false_type{}, std::integral_constant<int, 0>{}, GBT{}, 0, sacc);      \
    int t = 1;                                                                            \
    while (t < ntiles) {                                                                  \
      ATTN_ITER(0, GBT)                                                                   \
      ATTN_ITER(1, GBT)                                                                   \
      ATTN_ITER(2, GBT)                                                                   \
      ATTN_ITER(3, GBT)                                                                   \
      if constexpr (NSTAGE == 6) {                                                        \
        ATTN_ITER(4, GBT)                                                                 \
        ATTN_ITER(5, GBT)                                                                 \
      }                                                                                   \
    }                                                                                     \
  }
    // (written out twice rather than as a lambda: the backend mishandles the key loop inside
    // a lambda)
    if (PP && wave >= WAVES / 2) ATTN_KEY_LOOP(std::true_type)
    else ATTN_KEY_LOOP(std::false_type)
#undef ATTN_KEY_LOOP
#undef ATTN_ITER
    drain(ntiles - 1, sacc);
    // the last iteration copied (zeros) for a tile past the end: let it land before the
    // workgroup's LDS is released
    WAIT_VMCNT(0);
  }

  // Epilogue: O = O^T / l (one reciprocal per row), LSE = ln2 * (m + log2 l).  An empty
  // row (l = 0) gets O = 0 and LSE = -inf.  Partial results (key splits) are stored in
  // fp32 for the merge.
  attn_agpr::fence();
  // (lane index recomputed here rather than kept live across the key loop)
  const int lane_e = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const bool partial = p.o_part != nullptr;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    const float inv = lt > 0.f ? 1.0f / lt : 0.f;
    const int row = qrow0 + qb * 32 + (lane_e & 31);
    const size_t orow = (size_t)bh * p.Lq + min(row, p.Lq - 1);
    const size_t prow = (size_t)split * p.part_rows + orow;
    uint16_t* dst16 = p.o + orow * D + 8 * (lane_e >> 5);  // 16-byte stores (see below)
    float* pdst = p.o_part + prow * D + 4 * (lane_e >> 5);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      float x[16];
      attn_agpr::read4<0>(qb * DB + db, x[0], x[1], x[2], x[3]);
      attn_agpr::read4<1>(qb * DB + db, x[4], x[5], x[6], x[7]);
      attn_agpr::read4<2>(qb * DB + db, x[8], x[9], x[10], x[11]);
      attn_agpr::read4<3>(qb * DB + db, x[12], x[13], x[14], x[15]);
      if (row < p.Lq) {
        if (partial) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(pdst + db * 32 + 8 * g) =
                make_float4(x[4 * g] * inv, x[4 * g + 1] * inv, x[4 * g + 2] * inv,
                            x[4 * g + 3] * inv);
        } else {
          // Chunk g of this lane holds dims 8g + 4hi .. +3 of the 32-dim block; the lane
          // l^32 holds the other four dims of each group of eight.  Exchanging one chunk of
          // two per pair lets each lane store 16 contiguous bytes: lane hi = 0 dims 0-7 and
          // 16-23, lane hi = 1 dims 8-15 and 24-31.
          u32x2 w[4];
#pragma unroll
          for (int g = 0; g < 4; ++g)
            w[g] = (u32x2){Elt<T>::pack2(x[4 * g] * inv, x[4 * g + 1] * inv),
                           Elt<T>::pack2(x[4 * g + 2] * inv, x[4 * g + 3] * inv)};
          const int h = lane_e >> 5;
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const u32x2 send = h ? w[2 * j] : w[2 * j + 1];
            const u32x2 recv = {static_cast<uint32_t>(__shfl_xor(static_cast<int>(send[0]), 32)),
                                static_cast<uint32_t>(__shfl_xor(static_cast<int>(send[1]), 32))};
            const u32x2 lo = h ? recv : w[2 * j];
            const u32x2 up = h ? w[2 * j + 1] : recv;
            *reinterpret_cast<u32x4*>(dst16 + db * 32 + 16 * j) = (u32x4){lo[0], lo[1], up[0], up[1]};
          }
        }
      }
    }
    const float lse_row = (m[qb] + __builtin_log2f(lt)) * 0.69314718055994531f;
    if (lane_e < 32 && row < p.Lq) {
      if (partial) p.lse_part[prow] = lse_row;
      else if (p.lse) p.lse[orow] = lse_row;
    }
  }
}

template <int D, int V, typename T>
int launch(const Params& prm, int64_t grid, hipStream_t stream) {
  constexpr int lds =
      attn_cfg::lds_bytes(D, attn_cfg::Tile<D, V>::BN, attn_cfg::Tile<D, V>::STAGES);
  static_assert(lds * attn_cfg::Tile<D, V>::WG_PER_CU <= 160 * 1024,
                "LDS budget of one CU exceeded");
  const void* fn = prm.c < 0.f ? reinterpret_cast<const void*>(&attn_fwd_kernel<D, V, T, true>)
                               : reinterpret_cast<const void*>(&attn_fwd_kernel<D, V, T, false>);
  // The LDS size above the default limit is a per-device attribute of the kernel: set it
  // the first time a device launches this instantiation (one bit per device; a device past
  // the 64th sets it on every launch).
  static std::atomic<uint64_t> lds_ready{0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return ATTN_E_LAUNCH;
  const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
  if (bit == 0 || (lds_ready.load(std::memory_order_acquire) & bit) == 0) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<D, V, T, false>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess ||
        hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_kernel<D, V, T, true>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess)
      return ATTN_E_LAUNCH;
    lds_ready.fetch_or(bit, std::memory_order_release);
  }
  Params local = prm;
  void* args[] = {&local};
  const hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)),
                                       dim3(attn_cfg::threads<D, V>()), args, lds, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

// Fill the kernel parameters shared by every entry point; the arguments are validated.
Params make_params(const void* q, const void* k, const void* v, void* o, float* lse,
                   float* o_part, float* lse_part, int64_t B, int64_t Hq, int64_t Hkv,
                   int64_t Lq, int64_t Lk, int64_t D, float scale, uint32_t flags,
                   int64_t nsplit, int block_m) {
  Params prm;
  prm.q = static_cast<const uint16_t*>(q);
  prm.k = static_cast<const uint16_t*>(k);
  prm.v = static_cast<const uint16_t*>(v);
  prm.o = static_cast<uint16_t*>(o);
  prm.lse = lse;
  prm.o_part = o_part;
  prm.lse_part = lse_part;
  prm.part_rows = B * Hq * Lq;
  // The G query heads of each key/value head are adjacent in Q, O and LSE, so they are
  // handed to the kernel as one head of G*Lq rows: short query sequences still fill the
  // workgroups' rows.  Addresses are unchanged; only the causal mask needs a row's own
  // position (row % Lq).
  const int64_t G = Hq / Hkv;
  prm.Hq = static_cast<int>(Hkv);
  prm.Hkv = static_cast<int>(Hkv);
  prm.G = 1;
  prm.Lq = static_cast<int>(G * Lq);
  prm.Lk = static_cast<int>(Lk);
  prm.n_qtiles = static_cast<int>((G * Lq + block_m - 1) / block_m);
  prm.n_work = static_cast<int>(prm.n_qtiles * B * Hkv * nsplit);  // < 2^31 (validated)
  prm.lq_head = static_cast<int>(Lq);
  {
    int l = 0;
    while ((int64_t(1) << l) < Lq) ++l;
    const uint64_t two = uint64_t(1) << (31 + l);
    prm.lq_magic = static_cast<uint32_t>((two + static_cast<uint64_t>(Lq) - 1) / Lq);
    prm.lq_shift = 31 + l;
  }
  prm.nsplit = static_cast<int>(nsplit);
  int64_t b0 = 0, e0 = Lk;
  attn_split_range(Lk, nsplit, 0, &b0, &e0);
  prm.split_len = static_cast<int>(e0 - b0);
  const bool causal = (flags & ATTN_CAUSAL) != 0;
  prm.diag = static_cast<int>(causal ? Lk - Lq : Lk);
  prm.causal = causal ? 1 : 0;
  // Causal dispatch order: heads whose query rows fill whole tiles are dealt position-major
  // in chunks of as many heads as one XCD's share of the grid holds (workgroups go to the
  // 8 XCDs in contiguous ranges).
  prm.qperm_heads = 1;
  prm.tiles_per_head = 1;
  if (causal && Lq > 0 && Lq % block_m == 0) {
    const int64_t T = Lq / block_m;
    const int64_t per_xcd = (static_cast<int64_t>(prm.n_work) + 7) / 8 / nsplit;
    prm.qperm_heads = static_cast<int>(std::max<int64_t>(1, std::min<int64_t>(G, per_xcd / T)));
    prm.tiles_per_head = static_cast<int>(T);
  }
  prm.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  // scale == 0: every weight is 1.  A positive c this small gives c*score below 2^-60 for
  // any finite fp16/bf16 dot product, so exp2 rounds to exactly 1 and the LSE term c*m
  // vanishes against ln(Lk) -- the same fp32 results, while masked keys (score -inf) still
  // get weight exp2(-inf) = 0 instead of exp2(0 * -inf) = NaN.
  if (prm.c == 0.f) prm.c = 1e-30f;
  return prm;
}

// The planner's tile shape, told apart by its rows per workgroup (attn_plan_t.block_m).
static_assert(attn_cfg::block_m<128, 1>() == attn_cfg::block_m<256, 1>() &&
                  attn_cfg::block_m<128, 0>() == attn_cfg::block_m<256, 0>() &&
                  attn_cfg::block_m<128, 1>() < attn_cfg::block_m<128, 0>(),
              "one row count per tile shape");

template <int V>
int launch_v(const Params& prm, int64_t D, int in_dtype, int64_t grid, hipStream_t s) {
  if (D == 128)
    return in_dtype == ATTN_F16 ? launch<128, V, _Float16>(prm, grid, s)
                                : launch<128, V, __bf16>(prm, grid, s);
  return in_dtype == ATTN_F16 ? launch<256, V, _Float16>(prm, grid, s)
                              : launch<256, V, __bf16>(prm, grid, s);
}

int launch_attn(const Params& prm, int64_t D, int in_dtype, int block_m, int64_t grid,
                hipStream_t s) {
  return block_m == attn_cfg::block_m<128, 1>() ? launch_v<1>(prm, D, in_dtype, grid, s)
                                                : launch_v<0>(prm, D, in_dtype, grid, s);
}

}  // namespace

// The library's own workspace for attn_fwd_ex_noalloc, the entry point for callers that
// cannot allocate: one copy of this array on every GPU the library runs on, held until the
// process ends.  In host code `scratch` is a host-side stand-in, not a device address; the
// device address of each GPU's copy comes from hipGetSymbolAddress, is kept in
// scratch_addr below, and is the only form in which the array reaches a kernel.
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_WORKSPACE_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<uintptr_t> scratch_addr[kMaxDevices];

// Device address of `scratch` on the current device, looked up on the first call made with
// that device current; nullptr if the HIP runtime cannot say (no device, or past the 64th).
void* scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  uintptr_t a = scratch_addr[dev].load(std::memory_order_acquire);
  if (a == 0) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr)
      return nullptr;
    a = reinterpret_cast<uintptr_t>(ptr);
    scratch_addr[dev].store(a, std::memory_order_release);  // (a racing caller stores the same)
  }
  return reinterpret_cast<void*>(a);
}

}  // namespace

extern "C" {

int attn_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                    float scale, int in_dtype, void* stream) {
  const int rc = attn_validate(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype);
  if (rc != ATTN_OK) return rc;
  if (B * Hq * Lq == 0) return ATTN_OK;  // no query row: nothing to launch
  attn_plan_t plan;
  attn_plan(B, Hq, Hkv, Lq, Lk, D, in_dtype, &plan);
  const Params prm = make_params(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, Lq, Lk, D,
                                 scale, 0, 1, plan.block_m);
  return launch_attn(prm, D, in_dtype, plan.block_m, plan.grid,
                     static_cast<hipStream_t>(stream));
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
             int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, float scale,
             int in_dtype) {
  return attn_fwd_stream(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, nullptr);
}

int attn_fwd_partial(const void* q, const void* k, const void* v, float* o_part,
                     float* lse_part, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                     int64_t Lk, int64_t D, float scale, int in_dtype, uint32_t flags,
                     int64_t nsplit, void* stream) {
  const int rc = attn_validate_partial(q, k, v, o_part, lse_part, B, Hq, Hkv, Lq, Lk, D, scale,
                                       in_dtype, flags, nsplit);
  if (rc != ATTN_OK) return rc;
  if (B * Hq * Lq == 0) return ATTN_OK;
  attn_plan_t plan;
  attn_plan(B, Hq, Hkv, Lq, Lk, D, in_dtype, &plan);
  const Params prm = make_params(q, k, v, nullptr, nullptr, o_part, lse_part, B, Hq, Hkv, Lq,
                                 Lk, D, scale, flags, nsplit, plan.block_m);
  return launch_attn(prm, D, in_dtype, plan.block_m, plan.grid * nsplit,
                     static_cast<hipStream_t>(stream));
}

int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, float scale,
                int in_dtype, uint32_t flags, int64_t nsplit, void* workspace,
                int64_t workspace_bytes, void* stream) {
  int rc = attn_validate_ex(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, flags,
                            nsplit);
  if (rc != ATTN_OK) return rc;
  if (B * Hq * Lq == 0) return ATTN_OK;  // (no workspace needed either)
  // plan.grid: the workgroups of the attention launch, every split included (attn_plan_ex
  // counts its splits already; attn_plan plans one pass)
  attn_plan_t plan;
  if (nsplit == 0) {
    attn_plan_ex(B, Hq, Hkv, Lq, Lk, D, in_dtype, flags, &plan);
    nsplit = plan.nsplit;
  } else {
    attn_plan(B, Hq, Hkv, Lq, Lk, D, in_dtype, &plan);
    plan.grid *= nsplit;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (nsplit == 1) {
    const Params prm = make_params(q, k, v, o, lse, nullptr, nullptr, B, Hq, Hkv, Lq, Lk, D,
                                   scale, flags, 1, plan.block_m);
    return launch_attn(prm, D, in_dtype, plan.block_m, plan.grid, s);
  }
  // Split keys: partial results into the workspace, then the merge.
  const int64_t need = attn_workspace_bytes(B, Hq, Lq, D, nsplit);
  const uintptr_t ws = reinterpret_cast<uintptr_t>(workspace);
  if (!workspace || workspace_bytes < need || (ws & 255u) != 0) return ATTN_E_WORKSPACE;
  const int64_t rows = B * Hq * Lq;
  const uint64_t wsz = static_cast<uint64_t>(need);
  auto hits = [&](const void* p, uint64_t n) {
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    return p && a < ws + wsz && ws < a + n;
  };
  if (hits(q, uint64_t(rows) * D * 2) || hits(k, uint64_t(B) * Hkv * Lk * D * 2) ||
      hits(v, uint64_t(B) * Hkv * Lk * D * 2) || hits(o, uint64_t(rows) * D * 2) ||
      hits(lse, uint64_t(rows) * 4))
    return ATTN_E_WORKSPACE;
  float* o_part = static_cast<float*>(workspace);
  const int64_t obytes = (nsplit * rows * D * 4 + 255) / 256 * 256;
  float* lse_part = reinterpret_cast<float*>(static_cast<char*>(workspace) + obytes);
  const Params prm = make_params(q, k, v, nullptr, nullptr, o_part, lse_part, B, Hq, Hkv, Lq,
                                 Lk, D, scale, flags, nsplit, plan.block_m);
  rc = launch_attn(prm, D, in_dtype, plan.block_m, plan.grid, s);
  if (rc != ATTN_OK) return rc;
  return attn_merge(o_part, lse_part, nsplit, rows, D, o, lse, in_dtype, stream);
}

int attn_fwd_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                        float scale, int in_dtype, uint32_t flags, int64_t nsplit,
                        void* stream) {
  const int rc = attn_validate_ex(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype,
                                  flags, nsplit);
  if (rc != ATTN_OK) return rc;
  if (B * Hq * Lq == 0) return ATTN_OK;
  const int64_t cap = ATTN_NOALLOC_WORKSPACE_BYTES;
  if (nsplit == 0) {
    // the planner's launch if its partials fit; otherwise the most splits that fit (default
    // tile shape), down to one pass, which needs no workspace
    attn_plan_t plan;
    const int prc = attn_plan_ex(B, Hq, Hkv, Lq, Lk, D, in_dtype, flags, &plan);
    if (prc != ATTN_OK) return prc;
    if (plan.workspace_bytes > cap) {
      int64_t ns = plan.nsplit;
      while (ns > 1 && attn_workspace_bytes(B, Hq, Lq, D, ns) > cap) --ns;
      nsplit = ns;
    }
  } else if (attn_workspace_bytes(B, Hq, Lq, D, nsplit) > cap) {
    return ATTN_E_WORKSPACE;
  }
  void* ws = scratch_on_current_device();
  if (ws == nullptr) return ATTN_E_LAUNCH;
  return attn_fwd_ex(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, flags, nsplit,
                     ws, cap, stream);
}

}  // extern "C"
