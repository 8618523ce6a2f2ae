/*
 * attn.h - C ABI of the exact attention forward (and its backward) for AMD
 * MI355X (gfx950).
 *
 * The library computes O = softmax(scale * Q K^T) V for every (batch, head)
 * in one pass over key/value tiles, keeping a running row maximum, a running
 * denominator and a rescaled output accumulator on chip, and never writing
 * the L x L weights to device memory.  The recurrence is the one the
 * quidproquo.cc guide "NTU Hung-yi Lee ML 2026 Guide: Faster Generation,
 * Part 1: Flash Attention" derives in "Mechanism: run with the wrong answer,
 * then correct it" (its two "Expand" boxes: the running maximum d_k, the
 * running denominator s_k, and the output correction by
 * (s_{k-1}/s_k) exp(d_{k-1} - d_k)); the tiled, fused form is the one the
 * comfyai.app chapter "6.3 FlashAttention" (section 6.3.3) describes.  The
 * result equals standard attention up to floating-point rounding.
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers to contiguous row-major
 *     tensors: q and o are [B, H, Lq, D], k and v are [B, H, Lk, D], lse is
 *     [B, H, Lq] float32.  q, k, v and o share `dtype`.  There are no
 *     strides.  Every tensor pointer must be 16-byte aligned.
 *   - scores are a_ij = scale * (q_i . k_j); any finite scale is accepted.
 *   - causal != 0 applies a bottom-right aligned mask: query i may attend to
 *     key j iff j <= i + (Lk - Lq).  Causal requires Lq <= Lk.
 *   - lse[i] = m_i + ln(sum_j exp(a_ij - m_i)) with m_i the row maximum, in
 *     natural-log units of the scaled scores.
 *   - o is written in `dtype` (round to nearest even from float32); lse in
 *     float32.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call is
 *     asynchronous: it validates, enqueues kernels on `stream` and returns.
 *     Inputs must stay valid and unmodified until the stream reaches the
 *     work; o and lse are complete when the stream has passed it.
 *   - Ownership: the caller owns every buffer; the library frees nothing it
 *     did not allocate.  o and lse must not overlap q, k, v or each other.
 *     The library keeps no state between calls and may be called from
 *     several host threads.
 *   - Errors: a negative attn_status_t.  All argument checks run before any
 *     HIP call, so a rejected call has no effect.  ATTN_ERR_HIP reports a
 *     failed launch or allocation; faults inside a kernel surface later, at
 *     the caller's stream synchronisation.  NaN or Inf in the inputs is not
 *     checked and propagates.
 */
#ifndef IO_AWARE_SOFTMAX_ATTN_H
#define IO_AWARE_SOFTMAX_ATTN_H

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_F32 = 0,  /* IEEE binary32 */
  ATTN_F16 = 1,  /* IEEE binary16 */
  ATTN_BF16 = 2  /* bfloat16 */
} attn_dtype_t;

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,           /* a required pointer is NULL */
  ATTN_ERR_DIM = -2,            /* a dimension <= 0, or a size that overflows the index types */
  ATTN_ERR_UNSUPPORTED_D = -3,  /* head dim D is not 64 or 128 */
  ATTN_ERR_DTYPE = -4,          /* unknown attn_dtype_t, or one the entry point does not take */
  ATTN_ERR_SCALE = -5,          /* scale is NaN or infinite */
  ATTN_ERR_CAUSAL_SHAPE = -6,   /* causal with Lq > Lk */
  ATTN_ERR_SPLITS = -7,         /* num_splits outside [0, ATTN_MAX_SPLITS] */
  ATTN_ERR_ALIAS = -8,          /* o or lse overlaps an input or each other */
  ATTN_ERR_ALIGN = -9,          /* a tensor pointer is not 16-byte aligned */
  ATTN_ERR_HIP = -10,           /* a HIP launch or allocation failed */
  ATTN_ERR_MASK = -11,          /* bad mask_kind, or mask_b / mask_h not 1 or B / H */
  ATTN_ERR_DROPOUT = -12,       /* dropout_p outside [0, 1) */
  ATTN_ERR_WORKSPACE = -13      /* attn_decode_fwd_noalloc: partials exceed ATTN_NOALLOC_SCRATCH_BYTES */
} attn_status_t;

/* Kinds of the general mask of attn_fwd_ex / attn_bwd_ex. */
typedef enum {
  ATTN_MASK_NONE = 0,  /* no mask argument (causal still applies) */
  ATTN_MASK_BOOL = 1,  /* uint8: nonzero = the query attends to the key */
  ATTN_MASK_ADD = 2    /* float32 added to the scaled score; -inf excludes the key */
} attn_mask_kind_t;

/* Largest split count accepted by attn_decode_fwd and attn_decode_varlen_fwd. */
#define ATTN_MAX_SPLITS 256

/* Bytes of the fixed device scratch of attn_decode_fwd_noalloc (16 MiB). */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * attn_fwd - attention forward for any supported shape.
 *
 * q [B,H,Lq,D], k [B,H,Lk,D], v [B,H,Lk,D], o [B,H,Lq,D] (all `dtype`),
 * lse [B,H,Lq] float32.  D must be 64 or 128.
 *
 * Lq == 1 runs the split-KV decode path with the split count chosen by the
 * library (causal is then the same as non-causal); any other Lq runs the
 * tiled prefill kernel (MFMA for every dtype).  The decode path allocates a
 * stream-ordered workspace of (D + 2) * 4 * B * H * splits bytes with
 * hipMallocAsync on `stream` and releases it on the same stream.
 *
 * A 16-bit prefill at D = 128 with at most half as many 256-row query
 * tiles as the device has compute units (one head, a short chunk against a
 * long cache) cuts each query tile's keys into ranges of about equal size
 * (up to 32 per tile; attn_prefill_split_plan reports them), computed in
 * parallel and merged with the guide's output correction, each range taken
 * as one chunk (as attn_decode_fwd below does for one query).  It allocates
 * (D + 1) * 4 * B * H * Lq * R bytes the same stream-ordered way, R the
 * largest range count of a tile.  The environment variable
 * ATTN_PREFILL_SPLITS=n forces n ranges per tile (capped at 16 and so that
 * no range is empty; 1 never splits).  ATTN_PREFILL_KERNEL=single runs every
 * 16-bit prefill on the single-group kernel, =two runs D = 64 on the
 * two-group kernel too (by default D = 64 takes the single-group one).
 * Both variables are read on every call.
 *
 * Returns ATTN_OK or a negative attn_status_t.
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
             int B, int H, int Lq, int Lk, int D, int causal, float scale,
             void* stream, int dtype);

/*
 * attn_decode_fwd - single-query (Lq = 1) attention by split-KV.
 *
 * q and o are [B,H,1,D]; k and v are [B,H,Lk,D]; lse is [B,H,1].  The Lk
 * keys of each (b, h) are cut into `num_splits` contiguous ranges of
 * ceil(Lk / num_splits) keys (the last ones may be short or empty).  One
 * kernel computes, per range p, the partial statistics d_p (maximum),
 * s_p (denominator) and the normalised partial output O_p; a second kernel
 * merges them with the guide's output correction, treating each range as
 * one chunk: d = max_p d_p, s = sum_p s_p exp(d_p - d),
 * O = sum_p O_p (s_p / s) exp(d_p - d).  Empty ranges are skipped.
 *
 * num_splits == 0 lets the library choose.  Workspace as for attn_fwd.
 */
int attn_decode_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                    int B, int H, int Lk, int D, float scale, int num_splits,
                    void* stream, int dtype);

/*
 * attn_decode_fwd_noalloc - attn_decode_fwd for callers that cannot
 * allocate device memory (code under HIP graph capture, serving loops that
 * forbid allocation).
 *
 * Arguments, results and kernels are those of attn_decode_fwd (the same
 * num_splits gives bit-identical o and lse), but the split partials,
 * (D + 2) * 4 * B * H * splits bytes, live in a fixed device array of
 * ATTN_NOALLOC_SCRATCH_BYTES that the library holds on every device it
 * runs on until the process ends; the call makes no allocation of any
 * kind.  Its device address is looked up on the first call per device.
 * Returns ATTN_ERR_WORKSPACE (before any HIP call) when the partials
 * would exceed ATTN_NOALLOC_SCRATCH_BYTES (B * H * splits <= 32263 at
 * D = 128, <= 63550 at D = 64).  All calls on one device share that array:
 * calls that overlap on one device (different streams, or host threads
 * without ordering between them) race and give undefined results; calls
 * ordered on one stream are safe.  Nothing in the array needs clearing:
 * every call writes all partials it reads.
 */
int attn_decode_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                            int B, int H, int Lk, int D, float scale, int num_splits,
                            void* stream, int dtype);

/*
 * attn_decode_varlen_fwd - single-query attention over a KV cache whose
 * sequences have different lengths (the decode step of generation, which
 * the quidproquo.cc guide, slide 5, separates from the prefill).
 *
 * q and o are [B,H,1,D]; k and v are [B,H,Lk_max,D] caches; lse is
 * [B,H,1].  seqlens is a DEVICE pointer to B int32 lengths (4-byte
 * aligned, read when the stream reaches the call): (b, h) attends to its
 * first seqlens[b] keys only, and rows past that length are never read
 * (they may hold anything).  A length is clamped to [0, Lk_max]; a length of
 * 0 gives o = 0 and lse = -inf.  The keys of each (b, h) are cut into
 * num_splits ranges of ceil(len / num_splits) keys and merged as in
 * attn_decode_fwd; num_splits == 0 lets the library choose from Lk_max.
 * Workspace as for attn_fwd.  seqlens must not overlap o or lse.
 */
int attn_decode_varlen_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                           const int* seqlens, int B, int H, int Lk_max, int D, float scale,
                           int num_splits, void* stream, int dtype);

/*
 * attn_bwd - gradients of attn_fwd's O with respect to q, k and v.
 *
 * The comfyai.app chapter "6.3 FlashAttention" notes (after "A simple
 * implementation w/ C++" and in "Computation and GPU Memory") that for
 * training the method stores no score or weight matrix and recomputes what
 * the backward pass needs.  Given the upstream gradient dout = dL/dO, this
 * call recomputes the weights tile by tile as P_ij = exp(a_ij - lse_i) from
 * the forward's lse and returns the chain rule of O = softmax(a) V with
 * a = scale * q k^T (and the same mask):
 *   dv = P^T dout,  ds = P o (dout v^T - rowsum(dout o o)),
 *   dq = scale * ds k,  dk = scale * ds^T q.
 * Nothing of size Lq x Lk is written to device memory.  No gradient flows
 * into lse.
 *
 * q, o, dout, dq are [B,H,Lq,D]; k, v, dk, dv are [B,H,Lk,D] (all `dtype`);
 * lse is [B,H,Lq] float32.  o and lse must be attn_fwd's outputs for the
 * same q, k, v, causal and scale (they are trusted, not checked).  dtype is
 * ATTN_F16 or ATTN_BF16 (ATTN_F32 returns ATTN_ERR_DTYPE); D is 64 or 128.
 * Products run on MFMA with 16-bit operands (P and ds are rounded to
 * `dtype`) and fp32 accumulation; the outputs are rounded once to `dtype`.
 * Every output element has a single writer (no atomics): results are
 * deterministic.
 *
 * The forward's checks apply to q, k, v, o, lse and the sizes; in addition
 * dout, dq, dk, dv must be non-NULL and 16-byte aligned, and dq, dk, dv must
 * overlap neither an input nor each other (ATTN_ERR_ALIAS).  Allocates a
 * stream-ordered workspace of 512 * B * H * ceil(Lq / 64) bytes with
 * hipMallocAsync on `stream` and releases it on the same stream.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk, int D,
             int causal, float scale, void* stream, int dtype);

/*
 * attn_fwd_ex - attention forward with a general mask and dropout fused into
 * the tile.
 *
 * The comfyai.app chapter "6.3 FlashAttention" (section 6.3.3, "Kernel
 * Fusion") runs scores, scale, mask, softmax, dropout and the value product
 * of a tile in one kernel; this entry point does the same with:
 *   - mask: [mask_b, mask_h, Lq, Lk] contiguous (mask_b in {1, B}, mask_h in
 *     {1, H}; a size-1 axis is broadcast), a DEVICE pointer, 16-byte
 *     aligned, of kind ATTN_MASK_BOOL (uint8) or ATTN_MASK_ADD (float32
 *     added to scale * q.k); ignored (may be NULL) for ATTN_MASK_NONE.  It
 *     combines with causal: a key is excluded if either excludes it.
 *   - dropout_p in [0, 1): each weight P_ij is kept iff the 16-bit half
 *     (j mod 2; 0 = low half) of word ((j mod 8) / 2) of Philox4x32-10
 *     (Salmon et al., SC 2011) with counter (j / 8, i, b * H + h, offset)
 *     and key (seed low 32 bits, seed high 32 bits) is >=
 *     floor(dropout_p * 2^16); kept weights are scaled by
 *     1 / (1 - dropout_p).  lse is computed from the weights before dropout.
 *     The same (seed, offset) gives the same pattern in attn_bwd_ex.
 * A row with no key left gets o = 0 and lse = -inf.  Shapes, lse and the
 * other conventions as for attn_fwd; dtype ATTN_F16 or ATTN_BF16.  With
 * ATTN_MASK_NONE and dropout_p == 0 this is attn_fwd.  o and lse must not
 * overlap the mask.  Allocates nothing.
 */
int attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse,
                int B, int H, int Lq, int Lk, int D, int causal, float scale,
                const void* mask, int mask_kind, int mask_b, int mask_h,
                float dropout_p, unsigned long long seed, unsigned int offset,
                void* stream, int dtype);

/*
 * attn_bwd_ex - gradients of attn_fwd_ex's o with respect to q, k, v.
 *
 * Arguments as attn_bwd plus the mask and dropout arguments of the forward
 * call (the same values: the keep pattern is regenerated from seed and
 * offset).  With dropout the chain rule runs through the kept, rescaled
 * weights: dv = (P o Z / (1 - p))^T dout and ds = P o ((Z / (1 - p)) o
 * (dout v^T) - rowsum(dout o o)).  No gradient is returned for the mask.
 * dq, dk, dv must not overlap the mask.  Workspace as for attn_bwd.
 */
int attn_bwd_ex(const void* q, const void* k, const void* v, const void* o, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int B, int H, int Lq, int Lk,
                int D, int causal, float scale, const void* mask, int mask_kind, int mask_b,
                int mask_h, float dropout_p, unsigned long long seed, unsigned int offset,
                void* stream, int dtype);

/*
 * attn_decode_auto_splits - the split count attn_fwd and attn_decode_fwd
 * (with num_splits == 0) use for this shape.  Pure host arithmetic; returns
 * a value in [1, ATTN_MAX_SPLITS], or a negative attn_status_t for invalid
 * dimensions.
 */
int attn_decode_auto_splits(int B, int H, int Lk, int D);

/*
 * attn_prefill_split_plan - how attn_fwd cuts the keys of a prefill that
 * runs on the two-group kernel (fp16 / bf16, D = 128, scale != 0) on a
 * device with num_cus compute units.  Pure host arithmetic, launches
 * nothing.  ranges[ceil(Lq / 256)] (caller-owned) receives the number of key
 * ranges of each 256-row query tile, all 1 when the shape is not split;
 * *items receives the work items per (batch, head), the sum of ranges.
 * forced: as the ATTN_PREFILL_SPLITS environment variable (0 = automatic).
 * Returns ATTN_OK, ATTN_ERR_DIM for a non-positive size, num_cus or a
 * negative forced, ATTN_ERR_NULL for a null pointer.
 */
int attn_prefill_split_plan(int B, int H, int Lq, int Lk, int causal, int num_cus, int forced,
                            int* ranges, int* items);

/*
 * attn_strerror - static description of a status code.  For ATTN_ERR_HIP
 * the text of the last HIP error seen by the calling host thread is
 * appended; the returned pointer stays valid until that thread's next
 * library call.
 */
const char* attn_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* IO_AWARE_SOFTMAX_ATTN_H */
