// attn_merge.hip -- merge of partial attention results over disjoint key ranges, for gfx950.
//
// Each query row has P partial results (O_s, LSE_s), one per key range: O_s is the row's
// attention output over range s alone, LSE_s the natural log of that range's sum of
// exp(scores) (-inf for a range the row does not see).  The full result is
//
//     LSE = ln sum_s exp(LSE_s),     O = sum_s exp(LSE_s - LSE) * O_s,
//
// the merge of online-softmax state that the SyclKittens summary describes for
// context-parallel ring attention (section I: partial attention per key shard, then a merge
// of the softmax state).  A row with every LSE_s = -inf is empty: O = 0, LSE = -inf.
//
// Memory-bound: every partial element is read once and every output element written once.
// One thread owns 4 consecutive elements of one row (one 16-byte load per part, one 8- or
// 16-byte store), so a wavefront reads 1 KiB of contiguous bytes per part, with the loads
// of four parts (and their LSE values) issued together, in one pass: the running sums are
// rescaled to a new largest LSE when a batch brings one (a separate pass for the maximum
// first would cost another round trip to memory).  When there are few rows (decode-sized
// queries split over many key ranges) one wavefront per 64 output chunks would walk all
// parts one batch after another on a handful of compute units; then the parts are dealt to
// the PG wavefronts of a workgroup (part s to wavefront s % PG).  Each wavefront weighs its
// parts against the largest LSE among them; the PG partial sums meet in LDS, rescaled to
// the common maximum and added in a fixed order, so the result does not depend on timing.
// The row's LSE values are read by all of its threads (the same cache lines).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/attn.h"

namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kVec = 4;     // output elements per thread
constexpr int kBatch = 4;   // parts whose loads are issued together
constexpr int kMaxPG = 16;  // wavefronts sharing the parts of 64 chunks

struct MergeParams {
  const float* __restrict__ o_part;   // [P][rows][D]
  const float* __restrict__ lse_part;  // [P][rows]
  void* __restrict__ o;                // [rows][D], element type out_dtype
  float* __restrict__ lse;             // [rows] or nullptr
  int64_t rows;
  int64_t chunks;  // rows * D / kVec
  int D, nparts;
};

template <int OUT, int PG>  // OUT: ATTN_F16, ATTN_BF16 or ATTN_F32; PG: wavefronts per chunk
__global__ __launch_bounds__(64 * PG) void attn_merge_kernel(MergeParams p) {
  __shared__ f32x4 red_acc[PG > 1 ? PG - 1 : 1][64];
  __shared__ float red_sum[PG > 1 ? PG - 1 : 1][64];
  __shared__ float red_top[PG > 1 ? PG - 1 : 1][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;  // this wavefront takes parts wave, wave + PG, ...
  const int64_t chunk = static_cast<int64_t>(blockIdx.x) * 64 + lane;
  const bool live = chunk < p.chunks;
  const int cpr = p.D / kVec;
  const int64_t row = live ? chunk / cpr : 0;
  const int col = static_cast<int>(chunk - row * cpr) * kVec;
  const float* lse_row = p.lse_part + row;  // part s at lse_row[s * rows]

  // One pass over this wavefront's parts, kBatch at a time with all their loads issued
  // together; the running sums are rescaled when a batch raises the largest LSE.
  constexpr float kLog2e = 1.4426950408889634f;
  float top = -__builtin_inff();
  f32x4 acc = {0, 0, 0, 0};
  float sum = 0.f;
  if (live) {
    const float* src = p.o_part + row * p.D + col;
    const int64_t step = p.rows * p.D;  // one part
    for (int s0 = wave; s0 < p.nparts; s0 += kBatch * PG) {
      f32x4 x[kBatch];
      float lv[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const int s = s0 + j * PG;
        const bool have = s < p.nparts;
        const int sc = have ? s : s0;  // (a part that exists; its weight is zeroed)
        x[j] = *reinterpret_cast<const f32x4*>(src + sc * step);
        const float l = lse_row[sc * p.rows];
        lv[j] = have ? l : -__builtin_inff();
      }
      float bt = top;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) bt = fmaxf(bt, lv[j]);
      if (bt == -__builtin_inff()) continue;
      const float f = __builtin_amdgcn_exp2f((top - bt) * kLog2e);
      acc *= f;
      sum *= f;
      top = bt;
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        const float w = __builtin_amdgcn_exp2f((lv[j] - top) * kLog2e);
        if (w != 0.f) acc += w * x[j];
        sum += w;
      }
    }
  }
  if constexpr (PG > 1) {
    if (wave > 0) {
      red_acc[wave - 1][lane] = acc;
      red_sum[wave - 1][lane] = sum;
      red_top[wave - 1][lane] = top;
    }
    __syncthreads();
    if (wave > 0) return;
    float all = top;
#pragma unroll
    for (int w = 0; w < PG - 1; ++w) all = fmaxf(all, red_top[w][lane]);
    if (all != -__builtin_inff()) {
      // sums relative to top -> relative to all: factor exp(top - all) <= 1 (0 for a
      // wavefront whose parts are all empty, whose sums are 0 anyway)
      const float f0 = top == -__builtin_inff() ? 0.f
                                                : __builtin_amdgcn_exp2f((top - all) * kLog2e);
      acc *= f0;
      sum *= f0;
#pragma unroll
      for (int w = 0; w < PG - 1; ++w) {
        const float tw = red_top[w][lane];
        const float f = tw == -__builtin_inff() ? 0.f : __builtin_amdgcn_exp2f((tw - all) * kLog2e);
        acc += f * red_acc[w][lane];
        sum += f * red_sum[w][lane];
      }
    }
    top = all;
  }
  if (!live) return;
  float lse = -__builtin_inff();
  if (top != -__builtin_inff()) {
    acc *= 1.0f / sum;
    lse = top + __builtin_logf(sum);
  }
  const int64_t off = row * p.D + col;
  if constexpr (OUT == ATTN_F32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(p.o) + off) = acc;
  } else if constexpr (OUT == ATTN_F16) {
    *reinterpret_cast<f16x4*>(static_cast<_Float16*>(p.o) + off) =
        __builtin_convertvector(acc, f16x4);
  } else {
    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.o) + off) =
        __builtin_convertvector(acc, bf16x4);
  }
  if (p.lse && col == 0) p.lse[row] = lse;
}

template <int OUT>
const void* merge_fn(int pg) {
  switch (pg) {
    case 16: return reinterpret_cast<const void*>(&attn_merge_kernel<OUT, 16>);
    case 8: return reinterpret_cast<const void*>(&attn_merge_kernel<OUT, 8>);
    case 4: return reinterpret_cast<const void*>(&attn_merge_kernel<OUT, 4>);
    case 2: return reinterpret_cast<const void*>(&attn_merge_kernel<OUT, 2>);
    default: return reinterpret_cast<const void*>(&attn_merge_kernel<OUT, 1>);
  }
}

// Wavefronts per 64 output chunks: doubled while the whole launch has fewer than 4096
// wavefronts (four per SIMD) and every wavefront still gets a full batch of parts.
int part_groups(int64_t chunks, int64_t nparts) {
  const int64_t waves = (chunks + 63) / 64;
  int pg = 1;
  while (pg < kMaxPG && waves * pg < 4096 && nparts >= 2 * pg * kBatch) pg *= 2;
  return pg;
}

}  // namespace

extern "C" int attn_merge(const float* o_part, const float* lse_part, int64_t nsplit,
                          int64_t rows, int64_t D, void* o, float* lse, int out_dtype,
                          void* stream) {
  const int rc = attn_validate_merge(o_part, lse_part, nsplit, rows, D, o, lse, out_dtype);
  if (rc != ATTN_OK) return rc;
  if (rows == 0) return ATTN_OK;
  MergeParams p;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.o = o;
  p.lse = lse;
  p.rows = rows;
  p.chunks = rows * (D / kVec);
  p.D = static_cast<int>(D);
  p.nparts = static_cast<int>(nsplit);
  const int pg = part_groups(p.chunks, p.nparts);
  const dim3 grid(static_cast<unsigned>((p.chunks + 63) / 64));
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* args[] = {&p};
  const void* fn = out_dtype == ATTN_F16    ? merge_fn<ATTN_F16>(pg)
                   : out_dtype == ATTN_BF16 ? merge_fn<ATTN_BF16>(pg)
                                            : merge_fn<ATTN_F32>(pg);
  const hipError_t e = hipLaunchKernel(fn, grid, dim3(64 * pg), args, 0, s);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}
