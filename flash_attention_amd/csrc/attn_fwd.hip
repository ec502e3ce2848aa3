// attn_fwd.hip -- fused attention forward for gfx950 (MI355X, CDNA4) and the launching half
// of the C ABI.
//
// Method: the flash-attention forward of the "Xe2 (Lunar Lake/LNL, Battlemage/BMG) ESIMD
// Flash Attention -- HD=256" page (GQA, online softmax over key tiles, deferred rescale of
// the output accumulator, one reciprocal of the row sum at the end: sections "Key
// Optimization Insights / What Worked") with the fp32-softmax data flow of "Xe2 Sdp Bf16"
// (section "Kernel Architecture: bf16io", data-flow diagram).  The Xe2 register and SLM
// choreography is not reused; the layout below is built around CDNA4's 32x32x16 MFMA.
//
// Work decomposition.  A workgroup is 4 wavefronts and owns BLOCK_M = 128*QB query rows of
// one query head; each wavefront owns 32*QB whole rows, so a row's max and sum never cross
// wavefronts.  The grouped-query head map (query head h reads key/value head h / (Hq/Hkv))
// is resolved from the block index.
//
// Transposed scores.  Each wavefront computes S^T = K * Q^T with K as the MFMA A operand
// (32 keys x 16 dims) and Q^T as the B operand (16 dims x 32 queries, register resident
// for the whole key loop).  The 32x32 fp32 result then holds one query per lane column:
// lane l owns query l%32 and 16 of the 32 keys, the other 16 sitting in lane l^32.  Row
// max = an in-lane max plus one cross-half exchange; the row sum stays per-lane until the
// end.  Those same registers, rounded to 16 bits, are directly the B operand of
// O^T += V^T * P^T (k index = key): no trip through LDS for P.  The key order inside the
// B operand is fixed by the accumulator layout, so V^T is stored in LDS in that same
// permuted key order (see vt_pos_group).  O^T lives in 32x32 accumulators with one query
// per lane column as well, so the per-row rescale by alpha is a per-lane scalar multiply.
//
// This is the first, correctness-first version: K and V tiles are staged through registers
// into a single LDS buffer, two barriers per tile.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "../../include/attn.h"
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
  uint16_t* __restrict__ o;
  float* __restrict__ lse;
  int Hq, Hkv, G, Lq, Lk;
  int n_qtiles;
  float c;  // scale * log2(e): scores are kept in base-2 units
};

template <typename T>
struct Elt;

template <>
struct Elt<_Float16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  // two fp32 -> two fp16, round to nearest even
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    f16x2 r = __builtin_convertvector((f32x2){x, y}, f16x2);
    return __builtin_bit_cast(uint32_t, r);
  }
};

template <>
struct Elt<__bf16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float x, float y) {
    bf16x2 r = __builtin_convertvector((f32x2){x, y}, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
  }
};

// The S^T accumulator register r of a lane in half h (= lane/32) holds key
// 8*(r/4) + 4*h + r%4 of its 32-key block.  The P^T operand of MFMA step ks (16 keys) takes
// registers 8*(ks%2) .. +7, i.e. key groups (of 4) 4ks+h and 4ks+2+h for lane half h.  V^T
// is therefore stored with key group kg at position group vt_pos_group(kg): the two middle
// groups of every 4 swap places, so lane half h reads its 8 keys as one 16-byte run.
__device__ __forceinline__ int vt_pos_group(int kg) {
  return (kg & ~3) | ((kg & 1) << 1) | ((kg >> 1) & 1);
}

template <int D, typename T>
__global__ __launch_bounds__(attn_cfg::kThreads, 1) void attn_fwd_kernel(Params p) {
  constexpr int QB = attn_cfg::Tile<D>::QB;
  constexpr int BN = attn_cfg::Tile<D>::BN;
  constexpr int NB = BN / 32;   // 32-key blocks per tile
  constexpr int KS = D / 16;    // contraction steps of S^T
  constexpr int DB = D / 32;    // 32-row blocks of O^T
  constexpr int KROW = D + attn_cfg::kPad;
  constexpr int VROW = BN + attn_cfg::kPad;
  constexpr int BM = attn_cfg::block_m(QB);
  constexpr int NT = attn_cfg::kThreads;

  extern __shared__ u32x4 smem_raw[];
  uint16_t* ks = reinterpret_cast<uint16_t*>(smem_raw);
  uint16_t* vt = ks + BN * KROW;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hi = lane >> 5;

  // Workgroups are dealt round-robin to the 8 XCDs; renumber so each XCD runs a contiguous
  // range of (batch, head, query tile) and its concurrent workgroups share key/value heads
  // in that XCD's L2.
  const int nblk = gridDim.x, bid = blockIdx.x;
  const int xcd = bid & 7, local = bid >> 3;
  const int per = nblk >> 3, rem = nblk & 7;
  const int logical = xcd * per + (xcd < rem ? xcd : rem) + local;
  const int qtile = logical % p.n_qtiles;
  const int bh = logical / p.n_qtiles;  // b*Hq + hq
  const int hq = bh % p.Hq, b = bh / p.Hq;
  const int hkv = hq / p.G;

  const uint16_t* qh = p.q + (size_t)bh * p.Lq * D;
  const uint16_t* kh = p.k + ((size_t)b * p.Hkv + hkv) * p.Lk * D;
  const uint16_t* vh = p.v + ((size_t)b * p.Hkv + hkv) * p.Lk * D;
  const int qrow0 = qtile * BM + wave * 32 * QB;
  const int Lk = p.Lk;

  // Q^T operand fragments, resident for the whole key loop: lane l holds query row l%32,
  // dims 16*kk + 8*(l/32) .. +7.
  u32x4 qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = qrow0 + qb * 32 + l32;
    const u32x4* src = reinterpret_cast<const u32x4*>(qh + (size_t)row * D + 8 * hi);
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) qf[qb][kk] = row < p.Lq ? src[2 * kk] : (u32x4){0, 0, 0, 0};
  }

  f32x16 acc[QB][DB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -__builtin_inff();
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) acc[qb][db] = (f32x16){};
  }

  const int ntiles = (Lk + BN - 1) / BN;
  for (int t = 0; t < ntiles; ++t) {
    const int j0 = t * BN;
    __syncthreads();  // every wave is done reading the previous tile
    // K tile, row-major [key][d], coalesced 16-byte loads.
#pragma unroll
    for (int it = 0; it < BN * D / 8 / NT; ++it) {
      const int id = tid + it * NT;
      const int key = id / (D / 8), c = id % (D / 8);
      u32x4 val = {0, 0, 0, 0};
      if (j0 + key < Lk) val = *reinterpret_cast<const u32x4*>(kh + (size_t)(j0 + key) * D + c * 8);
      *reinterpret_cast<u32x4*>(ks + key * KROW + c * 8) = val;
    }
    // V tile, transposed to [d][key position]: each thread takes 4 keys x 8 dims.
#pragma unroll
    for (int it = 0; it < (BN / 4) * (D / 8) / NT; ++it) {
      const int id = tid + it * NT;
      const int kg = id / (D / 8), c = id % (D / 8);
      u32x4 r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = j0 + kg * 4 + e;
        r[e] = key < Lk ? *reinterpret_cast<const u32x4*>(vh + (size_t)key * D + c * 8)
                        : (u32x4){0, 0, 0, 0};
      }
      const int pg = vt_pos_group(kg);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int sh = 16 * (i & 1);
        const uint32_t e0 = (r[0][i >> 1] >> sh) & 0xffffu, e1 = (r[1][i >> 1] >> sh) & 0xffffu;
        const uint32_t e2 = (r[2][i >> 1] >> sh) & 0xffffu, e3 = (r[3][i >> 1] >> sh) & 0xffffu;
        *reinterpret_cast<u32x2*>(vt + (c * 8 + i) * VROW + pg * 4) =
            (u32x2){e0 | (e1 << 16), e2 | (e3 << 16)};
      }
    }
    __syncthreads();

    // S^T = K * Q^T, fp32 accumulation.
    f32x16 s[NB][QB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[nb][qb] = (f32x16){};
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const u32x4 a =
            *reinterpret_cast<const u32x4*>(ks + (nb * 32 + l32) * KROW + kk * 16 + 8 * hi);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[nb][qb] = Elt<T>::mfma(a, qf[qb][kk], s[nb][qb]);
      }
    }

    // Online softmax in base 2 (fp32).  Keys past Lk get -inf.
    const bool tail = j0 + BN > Lk;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -__builtin_inff();
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float x = s[nb][qb][r] * p.c;
          if (tail) {
            const int key = j0 + nb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key >= Lk) x = -__builtin_inff();
          }
          s[nb][qb][r] = x;
          mx = fmaxf(mx, x);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(m[qb], mx);
      const float alpha = __builtin_amdgcn_exp2f(m[qb] - mnew);
      float sum = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = __builtin_amdgcn_exp2f(s[nb][qb][r] - mnew);
          s[nb][qb][r] = e;
          sum += e;
        }
      }
      l[qb] = l[qb] * alpha + sum;
      m[qb] = mnew;
#pragma unroll
      for (int db = 0; db < DB; ++db) acc[qb][db] *= alpha;
    }

    // O^T += V^T * P^T, P rounded to the input type in registers.
#pragma unroll
    for (int ks16 = 0; ks16 < BN / 16; ++ks16) {
      const int nb = ks16 >> 1, half = ks16 & 1;
      u32x4 pb[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const f32x16& sv = s[nb][qb];
        pb[qb] = (u32x4){Elt<T>::pack2(sv[8 * half + 0], sv[8 * half + 1]),
                         Elt<T>::pack2(sv[8 * half + 2], sv[8 * half + 3]),
                         Elt<T>::pack2(sv[8 * half + 4], sv[8 * half + 5]),
                         Elt<T>::pack2(sv[8 * half + 6], sv[8 * half + 7])};
      }
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const u32x4 a =
            *reinterpret_cast<const u32x4*>(vt + (db * 32 + l32) * VROW + ks16 * 16 + 8 * hi);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) acc[qb][db] = Elt<T>::mfma(a, pb[qb], acc[qb][db]);
      }
    }
  }

  // Epilogue: O = O^T / l (one reciprocal per row), LSE = ln2 * (m + log2 l).
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = l[qb] + __shfl_xor(l[qb], 32);
    const float inv = 1.0f / lt;
    const int row = qrow0 + qb * 32 + l32;
    if (row < p.Lq) {
      uint16_t* dst = p.o + ((size_t)bh * p.Lq + row) * D + 4 * hi;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x16& a = acc[qb][db];
          const u32x2 w = {Elt<T>::pack2(a[4 * g] * inv, a[4 * g + 1] * inv),
                           Elt<T>::pack2(a[4 * g + 2] * inv, a[4 * g + 3] * inv)};
          *reinterpret_cast<u32x2*>(dst + db * 32 + 8 * g) = w;
        }
      }
      if (p.lse && hi == 0)
        p.lse[(size_t)bh * p.Lq + row] = (m[qb] + __builtin_log2f(lt)) * 0.69314718055994531f;
    }
  }
}

template <int D, typename T>
int launch(const Params& prm, int64_t grid, hipStream_t stream) {
  constexpr int lds = attn_cfg::lds_bytes(D, attn_cfg::Tile<D>::BN);
  static_assert(lds <= 160 * 1024, "LDS budget of one CU exceeded");
  const void* fn = reinterpret_cast<const void*>(&attn_fwd_kernel<D, T>);
  static const hipError_t attr =
      hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  (void)attr;
  Params local = prm;
  void* args[] = {&local};
  const hipError_t e = hipLaunchKernel(fn, dim3(static_cast<unsigned>(grid)),
                                       dim3(attn_cfg::kThreads), args, lds, stream);
  return e == hipSuccess ? ATTN_OK : ATTN_E_LAUNCH;
}

}  // namespace

extern "C" {

int attn_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                    float scale, int in_dtype, void* stream) {
  const int rc = attn_validate(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype);
  if (rc != ATTN_OK) return rc;
  attn_plan_t plan;
  attn_plan(B, Hq, Hkv, Lq, Lk, D, in_dtype, &plan);
  Params prm;
  prm.q = static_cast<const uint16_t*>(q);
  prm.k = static_cast<const uint16_t*>(k);
  prm.v = static_cast<const uint16_t*>(v);
  prm.o = static_cast<uint16_t*>(o);
  prm.lse = lse;
  prm.Hq = static_cast<int>(Hq);
  prm.Hkv = static_cast<int>(Hkv);
  prm.G = static_cast<int>(Hq / Hkv);
  prm.Lq = static_cast<int>(Lq);
  prm.Lk = static_cast<int>(Lk);
  prm.n_qtiles = static_cast<int>((Lq + plan.block_m - 1) / plan.block_m);
  prm.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634074);
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (D == 128)
    return in_dtype == ATTN_F16 ? launch<128, _Float16>(prm, plan.grid, s)
                                : launch<128, __bf16>(prm, plan.grid, s);
  return in_dtype == ATTN_F16 ? launch<256, _Float16>(prm, plan.grid, s)
                              : launch<256, __bf16>(prm, plan.grid, s);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
             int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, float scale,
             int in_dtype) {
  return attn_fwd_stream(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype, nullptr);
}

}  // extern "C"
