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
// 16-byte store), so a wavefront reads 1 KiB of contiguous bytes per part; the loads of
// four parts are issued together, so that a thread has several in flight.  The row's LSE
// values are read by all of its threads (the same cache lines).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/attn.h"

namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeThreads = 256;
constexpr int kVec = 4;    // output elements per thread
constexpr int kBatch = 4;  // parts whose loads are issued together

struct MergeParams {
  const float* __restrict__ o_part;   // [P][rows][D]
  const float* __restrict__ lse_part;  // [P][rows]
  void* __restrict__ o;                // [rows][D], element type out_dtype
  float* __restrict__ lse;             // [rows] or nullptr
  int64_t rows;
  int64_t chunks;  // rows * D / kVec
  int D, nparts;
};

template <int OUT>  // ATTN_F16, ATTN_BF16 or ATTN_F32
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(MergeParams p) {
  const int64_t chunk = static_cast<int64_t>(blockIdx.x) * kMergeThreads + threadIdx.x;
  if (chunk >= p.chunks) return;
  const int cpr = p.D / kVec;
  const int64_t row = chunk / cpr;
  const int col = static_cast<int>(chunk - row * cpr) * kVec;
  const float* lse_row = p.lse_part + row;  // part s at lse_row[s * rows]

  float top = -__builtin_inff();
  for (int s = 0; s < p.nparts; ++s) top = fmaxf(top, lse_row[s * p.rows]);

  f32x4 acc = {0, 0, 0, 0};
  float lse = -__builtin_inff();
  if (top != -__builtin_inff()) {
    // weights relative to the largest part: exp(LSE_s - top) <= 1 (0 for an empty part),
    // their sum >= 1; the partial outputs are summed unnormalised and scaled once
    constexpr float kLog2e = 1.4426950408889634f;
    float sum = 0.f;
    const float* src = p.o_part + row * p.D + col;
    const int64_t step = p.rows * p.D;  // one part
    int s = 0;
    for (; s + kBatch <= p.nparts; s += kBatch) {
      f32x4 x[kBatch];
      float w[kBatch];
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        x[j] = *reinterpret_cast<const f32x4*>(src + (s + j) * step);
        w[j] = __builtin_amdgcn_exp2f((lse_row[(s + j) * p.rows] - top) * kLog2e);
      }
#pragma unroll
      for (int j = 0; j < kBatch; ++j) {
        // an empty part (weight 0) must not bring in its output (not required finite)
        if (w[j] != 0.f) acc += w[j] * x[j];
        sum += w[j];
      }
    }
    for (; s < p.nparts; ++s) {
      const float w = __builtin_amdgcn_exp2f((lse_row[s * p.rows] - top) * kLog2e);
      if (w != 0.f) acc += w * *reinterpret_cast<const f32x4*>(src + s * step);
      sum += w;
    }
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
  const dim3 grid(static_cast<unsigned>((p.chunks + kMergeThreads - 1) / kMergeThreads));
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* args[] = {&p};
  const void* fn = out_dtype == ATTN_F16    ? reinterpret_cast<const void*>(&attn_merge_kernel<ATTN_F16>)
                   : out_dtype == ATTN_BF16 ? reinterpret_cast<const void*>(&attn_merge_kernel<ATTN_BF16>)
                                            : reinterpret_cast<const void*>(&attn_merge_kernel<ATTN_F32>);
  const hipError_t e = hipLaunchKernel(fn, grid, dim3(kMergeThreads), args, 0, s);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}
