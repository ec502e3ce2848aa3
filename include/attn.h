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
 * O is written in the input type (round to nearest even); LSE in fp32.  The scores
 * scale * q.k are formed in fp32 and must be finite there: with fp16 inputs that holds for
 * any |scale| below about 1e26 / D; with bf16 inputs (whose range is fp32's) it is the
 * caller's data that must keep q.k within fp32.  The output accumulates unnormalised
 * weights in fp32, each 32-key tile's weights of a row summing to at most 2^16 (fp16
 * inputs) or 2^25 (bf16 inputs) against the row's softmax reference: with bf16 inputs the
 * values of V must stay below 2^103 / ceil(Lk / 32) in magnitude (about 1e28 at 16K keys,
 * 4e25 at the longest accepted key sequence); fp16 values never reach that bound.
 *
 * Causal masking (attn_fwd_ex, flag ATTN_CAUSAL).  Query row i sees key j
 * only if j <= i + (Lk - Lq): the diagonal is aligned to the end of both
 * sequences, so the queries are the last Lq positions of the key sequence
 * (with Lq = Lk the usual lower triangle).  The SyclKittens summary names
 * partial-tile causal masking (section B.1.2) and causal runs with as few as
 * 8 query rows against long key sequences (sections E.4, E.6), which only
 * this alignment gives meaning.  A row that sees no key (Lq > Lk) has O = 0
 * and LSE = -inf.
 *
 * Key splits (attn_fwd_ex with nsplit > 1, attn_fwd_partial, attn_merge).  The
 * keys are cut into ranges; each range gives a partial result per row (its
 * attention over that range alone and that range's LSE), and the partials
 * merge exactly into the full result:
 *     LSE = ln sum_s exp(LSE_s),   O = sum_s exp(LSE_s - LSE) * O_s,
 * the merge of online-softmax state of the SyclKittens summary, section I
 * (context-parallel ring attention).  Splitting the keys gives short query
 * sequences enough workgroups to fill the GPU (split-K of section E.2).
 *
 * Empty sizes.  B, Hq, Lq and Lk may be 0 (Hkv must be positive).  With no query row
 * (B*Hq*Lq = 0) a call is valid, launches nothing and writes nothing.  With no key (Lk = 0)
 * every row's softmax is over an empty set: its weighted sum is empty, O = 0, and its
 * exponential sum is 0, LSE = ln 0 = -inf -- the values of a causal row that sees no key.
 * A pointer to a tensor of no elements may be NULL.
 *
 * Layouts.  All tensors are contiguous and row-major with the head dimension
 * fastest:  Q, O: [B, Hq, Lq, D];  K, V: [B, Hkv, Lk, D];  LSE: [B, Hq, Lq].
 * Partial results: O_part [nsplit, B, Hq, Lq, D] fp32, LSE_part
 * [nsplit, B, Hq, Lq] fp32.  Lq and Lk need not be multiples of any tile size.
 *
 * Ownership.  Every pointer is device memory owned by the caller (for
 * example torch tensors).  The library never allocates, frees, retains or
 * synchronises, and is reentrant: its only mutable global state is one bit
 * per device and kernel recording that the kernel's LDS limit was raised
 * (hipFuncSetAttribute, set once on first use, updated atomically).
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

/* Input/output element type (ATTN_F32 only as the output type of attn_merge). */
typedef enum { ATTN_F16 = 0, ATTN_BF16 = 1, ATTN_F32 = 2 } attn_dtype_t;

/* Flags of attn_fwd_ex / attn_fwd_partial / attn_plan_ex. */
#define ATTN_CAUSAL 1u

/* Largest number of key splits. */
#define ATTN_MAX_SPLITS 256

/* Return codes. */
enum {
  ATTN_OK = 0,
  ATTN_E_NULLPTR = -1, /* q, k, v or o is NULL while that tensor has elements (lse may
                          be NULL: LSE is then not written) */
  ATTN_E_SHAPE = -2,   /* B, Hq, Lq or Lk < 0, Hkv <= 0, or a size past the supported
                          range: Lq*D, (Hq/Hkv)*Lq*D and Lk*D must stay below 2^31,
                          B*Hkv and the grid below 2^31 */
  ATTN_E_HEADDIM = -3, /* D is not 128 or 256 */
  ATTN_E_GQA = -4,     /* Hq is not a multiple of Hkv */
  ATTN_E_DTYPE = -5,   /* in_dtype is neither ATTN_F16 nor ATTN_BF16 */
  ATTN_E_SCALE = -6,   /* scale is NaN or infinite */
  ATTN_E_ALIGN = -7,   /* q, k, v or o not 16-byte aligned, or lse not 4-byte aligned */
  ATTN_E_LAUNCH = -8,  /* the HIP runtime refused the launch (stream in an error state,
                          invalid stream, no device) */
  /* codes past the first eight: checks of the options and of the extra entry points */
  ATTN_E_ALIAS = -9,   /* o or lse overlaps an input, or lse overlaps o */
  ATTN_E_FLAGS = -10,  /* a flag bit other than ATTN_CAUSAL is set */
  ATTN_E_SPLIT = -11,  /* nsplit outside 0..ATTN_MAX_SPLITS (1..ATTN_MAX_SPLITS where a
                          count is required), or a split index out of range */
  ATTN_E_WORKSPACE = -12 /* workspace NULL, smaller than attn_workspace_bytes(), not
                            256-byte aligned, or overlapping another argument */
};

/*
 * attn_fwd -- enqueue the attention forward pass on the null stream.
 * Defines: the operation at the top of this file, as the "Xe2 ... ESIMD Flash Attention --
 * HD=256" page states it (header: GQA, 32 query over 2 KV heads, HD=256) with the data flow
 * of "Xe2 Sdp Bf16", section "Kernel Architecture: bf16io" (scores, fp32 softmax, weighted
 * V, one reciprocal of the row sum, 16-bit output).
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
 * stream), e.g. torch.cuda.current_stream().cuda_stream.  Same operation and passages as
 * attn_fwd; arguments, ownership and errors as there. */
int attn_fwd_stream(const void* q, const void* k, const void* v, void* o, float* lse,
                    int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                    float scale, int in_dtype, void* stream);

/* The host-side argument check attn_fwd runs before any launch.  Pure CPU, no HIP call:
 * usable without a GPU.  Returns ATTN_OK or the code attn_fwd would return.  Unsupported
 * shapes are refused on the host before any dispatch, the way the generic ESIMD GEMM of
 * "XPU 算子开发最佳实践：GEMM 高性能优化指南" (section 四) checks its shape before choosing a
 * compiled template. */
int attn_validate(const void* q, const void* k, const void* v, const void* o, const float* lse,
                  int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                  float scale, int in_dtype);

/* Static text for a return code (never NULL); the codes are those of the host-side checks
 * above (same GEMM-guide passage, section 四). */
const char* attn_strerror(int code);

/* The launch the planner picks for a problem: tile sizes, waves per workgroup, LDS bytes
 * per workgroup and grid size.  kernel receives a NUL-terminated name (at most 63 chars). */
typedef struct {
  int32_t block_m;    /* query rows per workgroup */
  int32_t block_n;    /* keys per K/V tile */
  int32_t waves;      /* 64-lane wavefronts per workgroup */
  int32_t lds_bytes;  /* LDS per workgroup */
  int64_t grid;       /* workgroups of the attention launch */
  char kernel[64];    /* attn_fwd_d<D>_<f16|bf16>[_causal][_m128]; _m128: the narrow shape of
                         128 rows per workgroup, used when (Hq/Hkv)*Lq <= 128 */
  int32_t nsplit;     /* key splits (1: no merge launch) */
  int32_t split_len;  /* keys per split (the last one may be shorter) */
  int64_t workspace_bytes; /* attn_workspace_bytes for nsplit */
} attn_plan_t;

/* Fill *plan for the given problem without launching anything (pure CPU): the launch of
 * attn_fwd (never split).  Returns ATTN_OK or the validation code for the shape/dtype
 * arguments.  A tiling chosen per head dimension, as the "Xe2 ... ESIMD Flash Attention --
 * HD=256" page fixes its own per head dimension (sections "Kernel Constants" and "HD=256
 * Architecture Differences (vs HD=128)"). */
int attn_plan(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
              int in_dtype, attn_plan_t* plan);

/* The launch attn_fwd_ex makes with nsplit = 0 and these flags: the planner picks the number
 * of key splits from a cost model of the GPU's 256 compute units (one or two workgroups each,
 * by tile shape), the key range per workgroup and the merge traffic.  Shape- and
 * batch-dependent dispatch of the attention launch: SyclKittens summary, section E.5;
 * split-K: section E.2.  Pure CPU; returns ATTN_OK or a validation code. */
int attn_plan_ex(int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                 int in_dtype, uint32_t flags, attn_plan_t* plan);

/*
 * attn_fwd_ex -- attn_fwd with options, on an explicit stream.
 * Defines: attn_fwd's operation, optionally under the causal mask (SyclKittens summary,
 * sections B.1.2, E.4, E.6; diagonal as stated at the top of this file) and computed over
 * key splits whose partial results are merged (split-K: section E.2; merge of online-
 * softmax state: section I.2).
 *   flags      0 or ATTN_CAUSAL
 *   nsplit     1: one pass, as attn_fwd (workspace unused, may be NULL);
 *              2..ATTN_MAX_SPLITS: the keys are cut into nsplit ranges (attn_split_range),
 *              partial results go to the workspace and attn_merge combines them into o and
 *              lse (two launches on `stream`);
 *              0: the planner's choice (attn_plan_ex: more splits when the query tiles
 *              alone would leave compute units idle; for key/value groups of 129-256 query
 *              rows that need splits it may also pick the narrow 128-row tile shape, which
 *              an explicit nsplit never does).
 *   workspace  device memory owned by the caller, 256-byte aligned, at least
 *              attn_workspace_bytes(B, Hq, Lq, D, nsplit) bytes for the nsplit actually
 *              used (query it with attn_plan_ex when passing 0); not retained after the
 *              call's kernels finish.
 * The result is the same as attn_fwd's up to rounding (the merge is exact in real
 * arithmetic).  Returns ATTN_OK or a negative code; nothing is enqueued on error.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int64_t B,
                int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D, float scale,
                int in_dtype, uint32_t flags, int64_t nsplit, void* workspace,
                int64_t workspace_bytes, void* stream);

/* attn_validate for attn_fwd_ex's arguments other than the workspace (pure CPU); host-side
 * refusal before dispatch as for attn_validate (GEMM guide, section 四).  Returns ATTN_OK or
 * the code attn_fwd_ex would return for these arguments. */
int attn_validate_ex(const void* q, const void* k, const void* v, const void* o,
                     const float* lse, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk,
                     int64_t D, float scale, int in_dtype, uint32_t flags, int64_t nsplit);

/*
 * attn_fwd_partial -- partial results over key ranges, one launch.
 * Defines: the per-range online-softmax state (normalised output and log-sum-exp of each
 * row over one key range) that the SyclKittens summary, section I.2, merges across key
 * shards, and that its split-K (section E.2) computes per workgroup.
 *   o_part    [nsplit, B, Hq, Lq, D] fp32 output: split s holds each row's attention over
 *             the keys of attn_split_range(Lk, nsplit, s) alone (0 for a row that sees none)
 *   lse_part  [nsplit, B, Hq, Lq] fp32 output: that range's natural-log sum of
 *             exp(scale * q.k) (-inf for a row that sees no key of the range); required
 *   nsplit    1..ATTN_MAX_SPLITS
 * Other arguments as attn_fwd_ex.  o_part and lse_part must not overlap each other or the
 * inputs; o_part 16-byte, lse_part 4-byte aligned.
 */
int attn_fwd_partial(const void* q, const void* k, const void* v, float* o_part,
                     float* lse_part, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                     int64_t Lk, int64_t D, float scale, int in_dtype, uint32_t flags,
                     int64_t nsplit, void* stream);

/* attn_fwd_partial's argument check (pure CPU; GEMM guide, section 四, as attn_validate).
 * Returns ATTN_OK or the code attn_fwd_partial would return. */
int attn_validate_partial(const void* q, const void* k, const void* v, const float* o_part,
                          const float* lse_part, int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq,
                          int64_t Lk, int64_t D, float scale, int in_dtype, uint32_t flags,
                          int64_t nsplit);

/*
 * attn_merge -- combine nsplit partial results per row into the full result.
 * Defines: the merge of online-softmax state of the SyclKittens summary, section I.2
 * (LSE = ln sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s, as at the top of this file).
 *   o_part    [nsplit, rows, D] fp32;  lse_part [nsplit, rows] fp32 (natural log, -inf for
 *             an empty part)
 *   o         [rows, D] output of element type out_dtype (ATTN_F16, ATTN_BF16, ATTN_F32),
 *             rounded to nearest even
 *   lse       [rows] fp32 output, or NULL
 *   rows      0 or more (0: nothing to do, the pointers may be NULL)
 *   D         a positive multiple of 8, at most 4096
 * The inputs may come from attn_fwd_partial (rows = B*Hq*Lq) or from any source of
 * partial attention results with this layout, e.g. key shards held elsewhere.  o_part and
 * o 16-byte aligned, lse_part and lse 4-byte aligned; the outputs must not overlap the
 * inputs or each other.  Returns ATTN_OK or a negative code.
 */
int attn_merge(const float* o_part, const float* lse_part, int64_t nsplit, int64_t rows,
               int64_t D, void* o, float* lse, int out_dtype, void* stream);

/* attn_merge's argument check (pure CPU; GEMM guide, section 四, as attn_validate).
 * Returns ATTN_OK or the code attn_merge would return. */
int attn_validate_merge(const float* o_part, const float* lse_part, int64_t nsplit,
                        int64_t rows, int64_t D, const void* o, const float* lse,
                        int out_dtype);

/* Key range [*begin, *end) of split s (0 <= s < nsplit) of Lk >= 0 keys: ranges of
 * ceil(ceil(Lk / nsplit) / 64) * 64 keys from key 0, the last ones cut at Lk or empty
 * (begin = end = Lk).  Pure CPU.  Returns ATTN_OK, ATTN_E_NULLPTR, ATTN_E_SHAPE or
 * ATTN_E_SPLIT.  The key ranges of split-K (SyclKittens summary, section E.2). */
int attn_split_range(int64_t Lk, int64_t nsplit, int64_t s, int64_t* begin, int64_t* end);

/* Workspace bytes attn_fwd_ex needs for nsplit splits (0 for nsplit = 1 or no query row),
 * or a negative code for bad sizes.  Layout: O_part at offset 0, LSE_part at the next
 * 256-byte boundary: the per-split state of split-K (SyclKittens summary, section E.2). */
int64_t attn_workspace_bytes(int64_t B, int64_t Hq, int64_t Lq, int64_t D, int64_t nsplit);

/*
 * attn_fwd_ex_noalloc -- attn_fwd_ex without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The partial results of a split launch go to a fixed array of
 * ATTN_NOALLOC_WORKSPACE_BYTES owned by the library: one per GPU, created when the library
 * is loaded and held until the process ends.  No call allocates or frees anything.
 *   nsplit  as attn_fwd_ex; an explicit count whose partials need more than
 *           ATTN_NOALLOC_WORKSPACE_BYTES (attn_workspace_bytes) is refused with
 *           ATTN_E_WORKSPACE; with 0 the planner's count is used when its partials fit,
 *           otherwise the largest count that fits (1, a single pass, always does).
 * Every call on one GPU shares that GPU's array: calls that overlap in time on one GPU
 * (other streams, other host threads) race and must be ordered by the caller.  Nothing in
 * the array needs to start at zero (each split launch writes every partial it merges).
 * Other arguments, results and codes as attn_fwd_ex; ATTN_E_LAUNCH also when the HIP
 * runtime cannot give the array's address on the current device.
 */
#define ATTN_NOALLOC_WORKSPACE_BYTES (64ll << 20)
int attn_fwd_ex_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                        int64_t B, int64_t Hq, int64_t Hkv, int64_t Lq, int64_t Lk, int64_t D,
                        float scale, int in_dtype, uint32_t flags, int64_t nsplit,
                        void* stream);

/* Dense fp16/bf16 MFMA peak of the current HIP device: compute units x peak shader clock x
 * 4096 flop per clock per compute unit (the gfx950 rate of v_mfma_f32_32x32x16_{f16,bf16}).
 * Any pointer may be NULL.  Returns ATTN_OK, or ATTN_E_LAUNCH if the HIP runtime reports no
 * device.  The denominator of "% of peak", as the "Xe2 ... ESIMD Flash Attention -- HD=256"
 * page reports its result (header: TFLOPS and percent of the device's peak). */
int attn_device_peak(double* tflops, int32_t* compute_units, int32_t* clock_khz);

/* Library version, "major.minor.patch" (static string; not a computation of the pages). */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_H */
