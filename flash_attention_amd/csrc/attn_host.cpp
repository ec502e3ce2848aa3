// attn_host.cpp -- host-only half of the C ABI: argument validation, the tiling planner,
// error strings and the version.  No HIP call is made here, so everything in this file
// works on a machine without a GPU.
//
// Validation rejects rather than mis-computes: an unsupported head dimension is an error,
// the way the generalised ESIMD GEMM of the GEMM guide "XPU 算子开发最佳实践：GEMM 高性能优化指南"
// (section 四, ESIMD) checks its shape on the host before dispatching to a compiled template.
#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/attn.h"
#include "attn_config.h"

namespace {

bool overlaps(const void* a, uint64_t abytes, const void* b, uint64_t bbytes) {
  const uint64_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bbytes && y < x + abytes;
}

struct PlanInternal {
  int qb, bn, stages, block_m, lds;
};

bool plan_for_d(int64_t D, PlanInternal* p) {
  using namespace attn_cfg;
  if (D == 128) {
    p->qb = Tile<128>::QB;
    p->bn = Tile<128>::BN;
    p->stages = Tile<128>::STAGES;
  } else if (D == 256) {
    p->qb = Tile<256>::QB;
    p->bn = Tile<256>::BN;
    p->stages = Tile<256>::STAGES;
  } else {
    return false;
  }
  p->block_m = block_m(p->qb);
  p->lds = lds_bytes(static_cast<int>(D), p->bn, p->stages);
  return true;
}

int check_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                int in_dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Lq <= 0 || Lk <= 0 || D <= 0) return ATTN_E_SHAPE;
  if (D != 128 && D != 256) return ATTN_E_HEADDIM;
  if (Hq % Hkv != 0) return ATTN_E_GQA;
  if (in_dtype != ATTN_F16 && in_dtype != ATTN_BF16) return ATTN_E_DTYPE;
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (Lq > lim / D || Lk > lim / D) return ATTN_E_SHAPE;  // per-head offsets fit in int32
  if (B > lim || Hq > lim) return ATTN_E_SHAPE;
  PlanInternal p;
  plan_for_d(D, &p);
  const int64_t qtiles = (Lq + p.block_m - 1) / p.block_m;
  if (qtiles > lim / Hq || qtiles * Hq > lim / B) return ATTN_E_SHAPE;  // grid < 2^31
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                  float scale, int in_dtype) {
  if (!q || !k || !v || !o) return ATTN_E_NULLPTR;
  int rc = check_shape(B, Hq, Hkv, Lq, Lk, D, in_dtype);
  if (rc != ATTN_OK) return rc;
  if (!std::isfinite(scale)) return ATTN_E_SCALE;
  auto mis16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (mis16(q) || mis16(k) || mis16(v) || mis16(o)) return ATTN_E_ALIGN;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_E_ALIGN;
  const uint64_t qbytes = uint64_t(B) * Hq * Lq * D * 2;
  const uint64_t kvbytes = uint64_t(B) * Hkv * Lk * D * 2;
  const uint64_t lbytes = uint64_t(B) * Hq * Lq * 4;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kvbytes) ||
      overlaps(o, qbytes, v, kvbytes))
    return ATTN_E_ALIAS;
  if (lse && (overlaps(lse, lbytes, o, qbytes) || overlaps(lse, lbytes, q, qbytes) ||
              overlaps(lse, lbytes, k, kvbytes) || overlaps(lse, lbytes, v, kvbytes)))
    return ATTN_E_ALIAS;
  return ATTN_OK;
}

int attn_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
              int in_dtype, attn_plan_t* plan) {
  if (!plan) return ATTN_E_NULLPTR;
  int rc = check_shape(B, Hq, Hkv, Lq, Lk, D, in_dtype);
  if (rc != ATTN_OK) return rc;
  PlanInternal p;
  plan_for_d(D, &p);
  plan->block_m = p.block_m;
  plan->block_n = p.bn;
  plan->waves = attn_cfg::kWaves;
  plan->lds_bytes = p.lds;
  plan->grid = ((Lq + p.block_m - 1) / p.block_m) * Hq * B;
  std::memset(plan->kernel, 0, sizeof plan->kernel);
  const char* name = D == 128 ? (in_dtype == ATTN_F16 ? "attn_fwd_d128_f16" : "attn_fwd_d128_bf16")
                              : (in_dtype == ATTN_F16 ? "attn_fwd_d256_f16" : "attn_fwd_d256_bf16");
  std::strncpy(plan->kernel, name, sizeof plan->kernel - 1);
  return ATTN_OK;
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULLPTR: return "q, k, v or o is a null pointer";
    case ATTN_E_SHAPE: return "a size is non-positive or past the supported range";
    case ATTN_E_HEADDIM: return "head dimension must be 128 or 256";
    case ATTN_E_GQA: return "Hq must be a multiple of Hkv";
    case ATTN_E_DTYPE: return "in_dtype must be ATTN_F16 or ATTN_BF16";
    case ATTN_E_SCALE: return "scale must be finite";
    case ATTN_E_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_E_ALIAS: return "an output overlaps an input or the other output";
    case ATTN_E_LAUNCH: return "the HIP runtime refused the kernel launch";
    default: return "unknown error code";
  }
}

const char* attn_version(void) { return "0.1.0"; }

}  // extern "C"
