// attn_host.cpp -- host-only half of the C ABI: argument validation, the tiling planner,
// error strings and the version.  No HIP call is made here, so everything in this file
// works on a machine without a GPU.
//
// Validation rejects rather than mis-computes: an unsupported head dimension is an error,
// the way the generalised ESIMD GEMM of the GEMM guide "XPU 算子开发最佳实践：GEMM 高性能优化指南"
// (section 四, ESIMD) checks its shape on the host before dispatching to a compiled template.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/attn.h"
#include "attn_config.h"

namespace {

bool overlaps(const void* a, uint64_t abytes, const void* b, uint64_t bbytes) {
  const uint64_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + bbytes && y < x + abytes;
}

struct PlanInternal {
  int waves, qb, bn, stages, block_m, lds, wg_per_cu, variant;
  double tile_cost;  // time of one key tile of one workgroup, in wide-shape tiles
};

// Tile shape for a key/value group of G*Lq query rows: the narrow shape (128 rows per
// workgroup) when the whole group fits in it, the wide one (256 rows) otherwise.
int variant_for(int64_t Hq, int64_t Hkv, int64_t Lq) {
  return Hq / Hkv * Lq <= attn_cfg::kNarrowRows ? 1 : 0;
}

template <int D, int V>
void fill_internal(PlanInternal* p) {
  using T = attn_cfg::Tile<D, V>;
  p->waves = T::WAVES;
  p->qb = T::QB;
  p->bn = T::BN;
  p->stages = T::STAGES;
  p->block_m = attn_cfg::block_m<D, V>();
  p->wg_per_cu = T::WG_PER_CU;
  p->variant = V;
  p->lds = attn_cfg::lds_bytes(D, T::BN, T::STAGES);
  // A narrow HD=256 workgroup does half the rows' matrix work per tile on a compute unit of
  // its own: about 0.6 of a wide tile's time (measured).  A narrow HD=128 workgroup shares
  // its compute unit with a second one and takes a wide tile's time.
  p->tile_cost = (V == 1 && D == 256) ? 0.6 : 1.0;
}

bool plan_for(int64_t D, int v, PlanInternal* p) {
  if (D == 128) {
    if (v) fill_internal<128, 1>(p);
    else fill_internal<128, 0>(p);
  } else if (D == 256) {
    if (v) fill_internal<256, 1>(p);
    else fill_internal<256, 0>(p);
  } else {
    return false;
  }
  return true;
}

// Workgroups per batch entry and key split: the G = Hq/Hkv query heads of a key/value head
// are one block of G*Lq query rows (adjacent in memory), cut into tiles of block_m rows of
// tile shape v (-1: the default shape for the problem).
int64_t query_tiles(int64_t Hq, int64_t Hkv, int64_t Lq, int64_t D, int v = -1) {
  PlanInternal p;
  plan_for(D, v < 0 ? variant_for(Hq, Hkv, Lq) : v, &p);
  return (Hq / Hkv * Lq + p.block_m - 1) / p.block_m * Hkv;
}

// Sizes may be zero: B, Hq or Lq = 0 leaves no query row (nothing to do), Lk = 0 leaves
// every row without keys (O = 0, LSE = -inf).  Hkv must be positive.
int check_shape(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                int in_dtype, int64_t nsplit = 1, int variant = -1) {
  if (B < 0 || Hq < 0 || Hkv <= 0 || Lq < 0 || Lk < 0 || D <= 0) return ATTN_E_SHAPE;
  if (D != 128 && D != 256) return ATTN_E_HEADDIM;
  if (Hq % Hkv != 0) return ATTN_E_GQA;
  if (in_dtype != ATTN_F16 && in_dtype != ATTN_BF16) return ATTN_E_DTYPE;
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (Lq > lim / D || Lk > lim / D) return ATTN_E_SHAPE;  // per-head offsets fit in int32
  if (B > lim || Hq > lim || Hkv > lim) return ATTN_E_SHAPE;
  if (B * Hkv > lim) return ATTN_E_SHAPE;  // (implied by the grid limit when Hq*Lq > 0)
  // the query heads of one key/value head run as one block of G*Lq rows: its row offsets
  // fit in int32 too
  if (Lq > 0 && Hq / Hkv > lim / D / Lq) return ATTN_E_SHAPE;
  const int64_t groups = query_tiles(Hq, Hkv, Lq, D, variant);  // workgroups per (b, split)
  if (B > 0 && (groups > lim / B || groups * B > lim / nsplit)) return ATTN_E_SHAPE;  // < 2^31
  return ATTN_OK;
}

constexpr int64_t kSplitAlign = 64;  // keys per split: a multiple of two key tiles

int64_t split_len_of(int64_t Lk, int64_t nsplit) {
  const int64_t per = (Lk + nsplit - 1) / nsplit;
  return (per + kSplitAlign - 1) / kSplitAlign * kSplitAlign;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

// Cost model of the planner, in units of one key tile (32 keys) of one workgroup.  The GPU
// runs wg_per_cu workgroups on each of its 256 compute units; a workgroup costs its key
// tiles plus a fixed overhead for pipeline fill, drain and epilogue; splitting adds the
// partial results' round trip through HBM and a second launch.
double split_cost(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                  int64_t ns, const PlanInternal& p) {
  constexpr double kCUs = 256, kOverheadTiles = 4, kLaunchTiles = 3;
  const double slots = kCUs * p.wg_per_cu;
  const int64_t len = split_len_of(Lk, ns);
  const int64_t used = (Lk + len - 1) / len;  // splits with keys
  const int64_t wg = (Hq / Hkv * Lq + p.block_m - 1) / p.block_m * Hkv * B * used;
  const double rounds = std::ceil(static_cast<double>(wg) / slots);
  double cost = rounds * (static_cast<double>(len) / 32.0 * p.tile_cost + kOverheadTiles);
  if (ns > 1) {
    // The unit, one key tile of one wide workgroup: 256 x 32 x D x 4 flop at ~1/256 of
    // ~1.2 PFLOP/s; the partials are written and read in fp32 and the output written once,
    // at ~4 TB/s.
    const double tile_s = 256.0 * 32.0 * D * 4.0 / (1.2e15 / kCUs);
    const double bytes = static_cast<double>(B * Hq * Lq) * D * (8.0 * used + 2.0);
    cost += bytes / 4e12 / tile_s + kLaunchTiles;
  }
  return cost;
}

int64_t choose_nsplit(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                      const PlanInternal& p) {
  int64_t best = 1;
  if (B * Hq * Lq == 0 || Lk == 0) return best;  // no rows or no keys: nothing to spread
  double best_cost = split_cost(B, Hq, Hkv, Lq, Lk, D, 1, p);
  for (int64_t ns = 2; ns <= 128; ++ns) {
    if (split_len_of(Lk, ns) < 256) break;  // splits shorter than 8 tiles do not pay
    const double c = split_cost(B, Hq, Hkv, Lq, Lk, D, ns, p);
    if (c < 0.95 * best_cost) {  // a split must win clearly
      best = ns;
      best_cost = c;
    }
  }
  return best;
}

// The planner's launch: tile shape and key splits.  A key/value group of more than 128 rows
// that needs key splits anyway may do better in the narrow shape: with half the rows per
// workgroup, fewer splits fill the GPU, fewer fp32 partials travel, and a ragged last tile
// wastes fewer rows.  (Measured over ten decode- and split-sized shapes: with this rule the
// planner's plan was within 0.7 % of the fastest measured plan in every one; weighing the
// narrow shape only for groups of up to 256 rows left a 512-row case 20 % behind.)
struct Choice {
  int variant;
  int64_t nsplit;
};

Choice choose_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D) {
  PlanInternal p;
  plan_for(D, variant_for(Hq, Hkv, Lq), &p);
  Choice c{p.variant, choose_nsplit(B, Hq, Hkv, Lq, Lk, D, p)};
  if (c.variant == 0 && c.nsplit > 1) {
    PlanInternal n;
    plan_for(D, 1, &n);
    const int64_t ns = choose_nsplit(B, Hq, Hkv, Lq, Lk, D, n);
    if (split_cost(B, Hq, Hkv, Lq, Lk, D, ns, n) <
        0.95 * split_cost(B, Hq, Hkv, Lq, Lk, D, c.nsplit, p))
      c = Choice{1, ns};
  }
  return c;
}

// attn_fwd_d<D>_<dtype>[_causal][_m128] (_m128: the narrow 128-row shape)
void kernel_name(int64_t D, int in_dtype, uint32_t flags, int variant, char* out, size_t n) {
  std::snprintf(out, n, "attn_fwd_d%d_%s%s%s", static_cast<int>(D),
                in_dtype == ATTN_F16 ? "f16" : "bf16", (flags & ATTN_CAUSAL) ? "_causal" : "",
                variant ? "_m128" : "");
}

int fill_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
              int in_dtype, uint32_t flags, int64_t nsplit, int variant, attn_plan_t* plan) {
  PlanInternal p;
  plan_for(D, variant, &p);
  plan->block_m = p.block_m;
  plan->block_n = p.bn;
  plan->waves = p.waves;
  plan->lds_bytes = p.lds;
  plan->grid = query_tiles(Hq, Hkv, Lq, D, variant) * B * nsplit;
  std::memset(plan->kernel, 0, sizeof plan->kernel);
  kernel_name(D, in_dtype, flags, p.variant, plan->kernel, sizeof plan->kernel);
  plan->nsplit = static_cast<int32_t>(nsplit);
  plan->split_len = static_cast<int32_t>(nsplit == 1 ? Lk : split_len_of(Lk, nsplit));
  plan->workspace_bytes = attn_workspace_bytes(B, Hq, Lq, D, nsplit);
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                  float scale, int in_dtype) {
  int rc = check_shape(B, Hq, Hkv, Lq, Lk, D, in_dtype);
  if (rc != ATTN_OK) return rc;
  const uint64_t qbytes = uint64_t(B) * Hq * Lq * D * 2;
  const uint64_t kvbytes = uint64_t(B) * Hkv * Lk * D * 2;
  const uint64_t lbytes = uint64_t(B) * Hq * Lq * 4;
  // (a tensor of no elements may be NULL: it is never read or written)
  if ((!q && qbytes) || (!k && kvbytes) || (!v && kvbytes) || (!o && qbytes))
    return ATTN_E_NULLPTR;
  if (!std::isfinite(scale)) return ATTN_E_SCALE;
  auto mis16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (mis16(q) || mis16(k) || mis16(v) || mis16(o)) return ATTN_E_ALIGN;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_E_ALIGN;
  if (overlaps(o, qbytes, q, qbytes) || overlaps(o, qbytes, k, kvbytes) ||
      overlaps(o, qbytes, v, kvbytes))
    return ATTN_E_ALIAS;
  if (lse && (overlaps(lse, lbytes, o, qbytes) || overlaps(lse, lbytes, q, qbytes) ||
              overlaps(lse, lbytes, k, kvbytes) || overlaps(lse, lbytes, v, kvbytes)))
    return ATTN_E_ALIAS;
  return ATTN_OK;
}

int attn_validate_ex(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                     int64_t D, float scale, int in_dtype, uint32_t flags, int64_t nsplit) {
  if (flags & ~ATTN_CAUSAL) return ATTN_E_FLAGS;
  if (nsplit < 0 || nsplit > ATTN_MAX_SPLITS) return ATTN_E_SPLIT;
  const int rc = attn_validate(q, k, v, o, lse, B, Hq, Hkv, Lq, Lk, D, scale, in_dtype);
  if (rc != ATTN_OK) return rc;
  // (nsplit = 0: the planner lowers its choice until the grid fits)
  return check_shape(B, Hq, Hkv, Lq, Lk, D, in_dtype, nsplit > 0 ? nsplit : 1);
}

int attn_validate_partial(const void* q, const void* k, const void* v, const float* o_part,
                          const float* lse_part, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                          int64_t Lk, int64_t D, float scale, int in_dtype, uint32_t flags,
                          int64_t nsplit) {
  if (flags & ~ATTN_CAUSAL) return ATTN_E_FLAGS;
  if (nsplit < 1 || nsplit > ATTN_MAX_SPLITS) return ATTN_E_SPLIT;
  int rc = check_shape(B, Hq, Hkv, Lq, Lk, D, in_dtype, nsplit);
  if (rc != ATTN_OK) return rc;
  const uint64_t qbytes = uint64_t(B) * Hq * Lq * D * 2;
  const uint64_t kvbytes = uint64_t(B) * Hkv * Lk * D * 2;
  const uint64_t pbytes = uint64_t(nsplit) * B * Hq * Lq * D * 4;
  const uint64_t lbytes = uint64_t(nsplit) * B * Hq * Lq * 4;
  if ((!q && qbytes) || (!k && kvbytes) || (!v && kvbytes) || (!o_part && pbytes) ||
      (!lse_part && lbytes))
    return ATTN_E_NULLPTR;
  if (!std::isfinite(scale)) return ATTN_E_SCALE;
  auto mis16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (mis16(q) || mis16(k) || mis16(v) || mis16(o_part)) return ATTN_E_ALIGN;
  if ((reinterpret_cast<uintptr_t>(lse_part) & 3u) != 0) return ATTN_E_ALIGN;
  const void* outs[2] = {o_part, lse_part};
  const uint64_t osz[2] = {pbytes, lbytes};
  for (int i = 0; i < 2; ++i)
    if (overlaps(outs[i], osz[i], q, qbytes) || overlaps(outs[i], osz[i], k, kvbytes) ||
        overlaps(outs[i], osz[i], v, kvbytes))
      return ATTN_E_ALIAS;
  if (overlaps(o_part, pbytes, lse_part, lbytes)) return ATTN_E_ALIAS;
  return ATTN_OK;
}

int attn_validate_merge(const float* o_part, const float* lse_part, int64_t nsplit,
                        int64_t rows, int64_t D, const void* o, const float* lse,
                        int out_dtype) {
  if (nsplit < 1 || nsplit > ATTN_MAX_SPLITS) return ATTN_E_SPLIT;
  if (rows < 0 || D <= 0) return ATTN_E_SHAPE;  // (rows = 0: nothing to merge)
  if (rows > 0 && (!o_part || !lse_part || !o)) return ATTN_E_NULLPTR;
  if (D % 8 != 0 || D > 4096) return ATTN_E_HEADDIM;
  if (out_dtype != ATTN_F16 && out_dtype != ATTN_BF16 && out_dtype != ATTN_F32)
    return ATTN_E_DTYPE;
  const int64_t lim = (int64_t(1) << 31) - 1;
  // part offsets (s * rows + row) * D stay below 2^62; workgroups (64 chunks of 4
  // elements each) below 2^31
  if (rows > (int64_t(1) << 40) / D / nsplit) return ATTN_E_SHAPE;
  if ((rows * (D / 4) + 63) / 64 > lim) return ATTN_E_SHAPE;
  auto mis16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; };
  if (mis16(o_part) || mis16(o)) return ATTN_E_ALIGN;
  if ((reinterpret_cast<uintptr_t>(lse_part) & 3u) != 0) return ATTN_E_ALIGN;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return ATTN_E_ALIGN;
  const uint64_t esz = out_dtype == ATTN_F32 ? 4 : 2;
  const uint64_t pbytes = uint64_t(nsplit) * rows * D * 4, lpbytes = uint64_t(nsplit) * rows * 4;
  const uint64_t obytes = uint64_t(rows) * D * esz, lbytes = uint64_t(rows) * 4;
  if (overlaps(o, obytes, o_part, pbytes) || overlaps(o, obytes, lse_part, lpbytes))
    return ATTN_E_ALIAS;
  if (lse && (overlaps(lse, lbytes, o_part, pbytes) || overlaps(lse, lbytes, lse_part, lpbytes) ||
              overlaps(lse, lbytes, o, obytes)))
    return ATTN_E_ALIAS;
  return ATTN_OK;
}

int attn_split_range(int64_t Lk, int64_t nsplit, int64_t s, int64_t* begin, int64_t* end) {
  if (!begin || !end) return ATTN_E_NULLPTR;
  if (Lk < 0) return ATTN_E_SHAPE;
  if (nsplit < 1 || nsplit > ATTN_MAX_SPLITS || s < 0 || s >= nsplit) return ATTN_E_SPLIT;
  if (nsplit == 1) {
    *begin = 0;
    *end = Lk;
    return ATTN_OK;
  }
  const int64_t len = split_len_of(Lk, nsplit);
  *begin = std::min(s * len, Lk);
  *end = std::min(*begin + len, Lk);
  return ATTN_OK;
}

int64_t attn_workspace_bytes(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int64_t nsplit) {
  const int64_t lim = (int64_t(1) << 31) - 1;
  if (B < 0 || Hq < 0 || Lq < 0 || D <= 0 || B > lim || Hq > lim || Lq > lim)
    return ATTN_E_SHAPE;
  if (nsplit < 1 || nsplit > ATTN_MAX_SPLITS) return ATTN_E_SPLIT;
  if (nsplit == 1) return 0;
  if (B * Hq > (int64_t(1) << 40) || (Lq > 0 && B * Hq > (int64_t(1) << 40) / Lq))
    return ATTN_E_SHAPE;
  const int64_t rows = B * Hq * Lq;
  if (rows > (int64_t(1) << 40) / D / nsplit) return ATTN_E_SHAPE;
  return align256(nsplit * rows * D * 4) + align256(nsplit * rows * 4);
}

int attn_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
              int in_dtype, attn_plan_t* plan) {
  if (!plan) return ATTN_E_NULLPTR;
  int rc = check_shape(B, Hq, Hkv, Lq, Lk, D, in_dtype);
  if (rc != ATTN_OK) return rc;
  return fill_plan(B, Hq, Hkv, Lq, Lk, D, in_dtype, 0, 1, variant_for(Hq, Hkv, Lq), plan);
}

int attn_plan_ex(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                 int in_dtype, uint32_t flags, attn_plan_t* plan) {
  if (!plan) return ATTN_E_NULLPTR;
  if (flags & ~ATTN_CAUSAL) return ATTN_E_FLAGS;
  int rc = check_shape(B, Hq, Hkv, Lq, Lk, D, in_dtype);
  if (rc != ATTN_OK) return rc;
  Choice c = choose_plan(B, Hq, Hkv, Lq, Lk, D);
  int64_t ns = c.nsplit;
  while (ns > 1 && check_shape(B, Hq, Hkv, Lq, Lk, D, in_dtype, ns, c.variant) != ATTN_OK) --ns;
  if (check_shape(B, Hq, Hkv, Lq, Lk, D, in_dtype, ns, c.variant) != ATTN_OK) {
    c.variant = variant_for(Hq, Hkv, Lq);  // (the default shape's single pass fits: checked)
    ns = 1;
  }
  return fill_plan(B, Hq, Hkv, Lq, Lk, D, in_dtype, flags, ns, c.variant, plan);
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "ok";
    case ATTN_E_NULLPTR: return "a tensor with elements is passed as a null pointer";
    case ATTN_E_SHAPE: return "a size is negative, Hkv is not positive, or a size is past the supported range";
    case ATTN_E_HEADDIM: return "head dimension must be 128 or 256";
    case ATTN_E_GQA: return "Hq must be a multiple of Hkv";
    case ATTN_E_DTYPE: return "in_dtype must be ATTN_F16 or ATTN_BF16";
    case ATTN_E_SCALE: return "scale must be finite";
    case ATTN_E_ALIGN: return "q, k, v, o must be 16-byte aligned and lse 4-byte aligned";
    case ATTN_E_ALIAS: return "an output overlaps an input or the other output";
    case ATTN_E_LAUNCH: return "the HIP runtime refused the kernel launch";
    case ATTN_E_FLAGS: return "unknown flag bits (only ATTN_CAUSAL is defined)";
    case ATTN_E_SPLIT: return "number of key splits or split index out of range";
    case ATTN_E_WORKSPACE:
      return "workspace missing, too small, not 256-byte aligned or overlapping an argument";
    default: return "unknown error code";
  }
}

const char* attn_version(void) { return "0.3.0"; }

}  // extern "C"
