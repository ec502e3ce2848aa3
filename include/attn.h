/*
 * attn.h -- C ABI of the MI355X (gfx950) attention forward library, libattn.so.
 *
 * Operation.  For every batch b, query head h and query row i,
 *
 *     O[b,h,i,:]  = sum_j softmax_j( scale * Q[b,h,i,:] . K[b,g,j,:] ) * V[b,g,j,:]
 *     LSE[b,h,i]  = ln sum_j exp( scale * Q[b,h,i,:] . K[b,g,j,:] )
 *
 * with the key/value head g = h / (Hq / Hkv): grouped-query attention, in
 * which each key/value head serves Hq/Hkv consecutive query heads.  This is
 * the fused scaled-dot-product attention forward of the "Xe2 (Lunar
 * Lake/LNL, Battlemage/BMG) ESIMD Flash Attention -- HD=256" page (header:
 * GQA with 32 query heads over 2 KV heads, head dimension 256; section
 * "Kernel Constants" for its tiling) and of "Xe2 Sdp Bf16" (head dimension
 * 128, bf16 inputs; section "Kernel Architecture: bf16io" for its data flow:
 * 16-bit Q, K in, fp32 scores and softmax, weighted sum of V, normalisation
 * by 1/sum, 16-bit output).  The log-sum-exp output is not on the pages; it
 * is the natural-log value above (scale included), the quantity needed to
 * merge partial results computed over disjoint key ranges.
 *
 * Numerics.  Q, K, V are fp16 or bf16; both matrix products accumulate in
 * fp32, the softmax runs in fp32 (online/streaming over key tiles), and the
 * probabilities are rounded to the input type before the second product.
 * O is written in the input type (round to nearest even); LSE in fp32.
 *
 * Layouts.  All tensors are contiguous and row-major with the head dimension
 * fastest:  Q, O: [B, Hq, Lq, D];  K, V: [B, Hkv, Lk, D];  LSE: [B, Hq, Lq].
 * Lq and Lk need not be multiples of any tile size.
 *
 * Ownership.  Every pointer is device memory owned by the caller (for
 * example torch tensors).  The library never allocates, frees, retains or
 * synchronises; it keeps no mutable global state and is reentrant.
 *
 * Errors.  Arguments are validated on the host before anything is
 * launched; a negative return means nothing was enqueued and nothing
 * written.  0 means the kernel was enqueued; faults inside the kernel
 * surface at the caller's next synchronisation.  attn_strerror() names
 * every code.
 */
#ifndef ATTN_H
#define ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Input/output element type. */
typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1 } attn_dtype_t;

/* Return codes. */
enum {
  ATTN_OK = 0,
  ATTN_E_NULLPTR = -1, /* q, k, v or o is NULL (lse may be NULL: LSE is then not written) */
  ATTN_E_SHAPE = -2,   /* B, Hq, Hkv, Lq or Lk <= 0, or a size past the supported range:
                          Lq*D and Lk*D must stay below 2^31, the grid below 2^31 blocks */
  ATTN_E_HEADDIM = -3, /* D is not 128 or 256 */
  ATTN_E_GQA = -4,     /* Hq is not a multiple of Hkv */
  ATTN_E_DTYPE = -5,   /* in_dtype is neither ATTN_F16 nor ATTN_BF16 */
  ATTN_E_SCALE = -6,   /* scale is NaN or infinite */
  ATTN_E_ALIGN = -7,   /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
  ATTN_E_ALIAS = -8,   /* o or lse overlaps an input, or lse overlaps o */
  ATTN_E_LAUNCH = -9   /* the HIP runtime refused the launch (stream in an error state,
                          invalid stream, no device) */
};

/*
 * attn_fwd -- enqueue the attention forward pass on the null stream.
 *   q        [B,Hq,Lq,D] input, element type in_dtype
 *   k, v     [B,Hkv,Lk,D] inputs, element type in_dtype
 *   o        [B,Hq,Lq,D] output, element type in_dtype (must not overlap q, k, v)
 *   lse      [B,Hq,Lq] fp32 output, natural log; NULL to skip it
 *   scale    multiplies every q.k product (1/sqrt(D) in the usual setting); any finite value
 * Returns ATTN_OK or a negative code (see above).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
             int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, float scale,
             int in_dtype);

/* attn_fwd on an explicit stream: `stream` is a hipStream_t passed as void* (NULL = null
 * stream), e.g. torch.cuda.current_stream().cuda_stream. */
int attn_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                    float scale, int in_dtype, void* stream);

/* The host-side argument check attn_fwd runs before any launch.  Pure CPU, no HIP call:
 * usable without a GPU.  Returns ATTN_OK or the code attn_fwd would return. */
int attn_validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                  float scale, int in_dtype);

/* Static text for a return code (never NULL). */
const char* attn_strerror(int code);

/* The launch the planner picks for a problem: tile sizes, waves per workgroup, LDS bytes
 * per workgroup and grid size.  kernel receives a NUL-terminated name (at most 63 chars). */
typedef struct {
  int32_t block_m;    /* query rows per workgroup */
  int32_t block_n;    /* keys per K/V tile */
  int32_t waves;      /* 64-lane wavefronts per workgroup */
  int32_t lds_bytes;  /* LDS per workgroup */
  int64_t grid;       /* workgroups launched */
  char kernel[64];
} attn_plan_t;

/* Fill *plan for the given problem without launching anything (pure CPU).  Returns ATTN_OK
 * or the validation code for the shape/dtype arguments. */
int attn_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
              int in_dtype, attn_plan_t* plan);

/* Library version, "major.minor.patch". */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
