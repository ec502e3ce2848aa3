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
// One thread owns 8 consecutive elements of one row (two 16-byte loads per part, one 16- or
// 32-byte store), so a wavefront reads 64 x 32 contiguous bytes per part; the row's P LSE
// values are read by all of its threads (the same cache lines).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/attn.h"

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x8 __attribute__((ext_vector_type(8)));

constexpr int kMergeThreads = 256;

struct MergeParams {
  const float* __restrict__ o_part;   // [P][rows][D]
  const float* __restrict__ lse_part;  // [P][rows]
  void* __restrict__ o;                // [rows][D], element type out_dtype
  float* __restrict__ lse;             // [rows] or nullptr
  int64_t rows;
  int64_t chunks;  // rows * D / 8
  int D, nparts;
};

template <int OUT>  // ATTN_F16, ATTN_BF16 or ATTN_F32
__global__ __launch_bounds__(kMergeThreads) void attn_merge_kernel(MergeParams p) {
  const int64_t chunk = static_cast<int64_t>(blockIdx.x) * kMergeThreads + threadIdx.x;
  if (chunk >= p.chunks) return;
  const int cpr = p.D >> 3;
  const int64_t row = chunk / cpr;
  const int col = static_cast<int>(chunk - row * cpr) * 8;

  float top = -__builtin_inff();
  for (int s = 0; s < p.nparts; ++s) top = fmaxf(top, p.lse_part[s * p.rows + row]);

  f32x8 acc = {0, 0, 0, 0, 0, 0, 0, 0};
  float lse = -__builtin_inff();
  if (top != -__builtin_inff()) {
    // weights relative to the largest part: exp(LSE_s - top) <= 1, their sum >= 1
    constexpr float kLog2e = 1.4426950408889634f;
    float sum = 0.f;
    for (int s = 0; s < p.nparts; ++s)
      sum += __builtin_amdgcn_exp2f((p.lse_part[s * p.rows + row] - top) * kLog2e);
    const float inv = 1.0f / sum;
    for (int s = 0; s < p.nparts; ++s) {
      const float ls = p.lse_part[s * p.rows + row];
      if (ls == -__builtin_inff()) continue;  // an empty part: weight 0, O_s not read
      const float w = __builtin_amdgcn_exp2f((ls - top) * kLog2e) * inv;
      // two 16-byte loads (the partials are only required to be 16-byte aligned)
      const float4* src = reinterpret_cast<const float4*>(p.o_part + (s * p.rows + row) * p.D + col);
      const float4 x0 = src[0], x1 = src[1];
      acc += w * (f32x8){x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    }
    lse = top + __builtin_logf(sum);
  }
  const int64_t off = row * p.D + col;
  if constexpr (OUT == ATTN_F32) {
    float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.o) + off);
    dst[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    dst[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
  } else if constexpr (OUT == ATTN_F16) {
    *reinterpret_cast<f16x8*>(static_cast<_Float16*>(p.o) + off) =
        __builtin_convertvector(acc, f16x8);
  } else {
    *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(p.o) + off) =
        __builtin_convertvector(acc, bf16x8);
  }
  if (p.lse && col == 0) p.lse[row] = lse;
}

}  // namespace

extern "C" int attn_merge(const float* o_part, const float* lse_part, int64_t nsplit,
                          int64_t rows, int64_t D, void* o, float* lse, int out_dtype,
                          void* stream) {
  const int rc = attn_validate_merge(o_part, lse_part, nsplit, rows, D, o, lse, out_dtype);
  if (rc != ATTN_OK) return rc;
  MergeParams p;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.o = o;
  p.lse = lse;
  p.rows = rows;
  p.chunks = rows * (D / 8);
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
