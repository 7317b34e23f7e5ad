/*
 * Exact attention (FlashAttention) for AMD Instinct MI355X (gfx950): the
 * forward pass (prefill and split-KV decode) and its backward pass.
 *
 * C ABI: plain pointers and sizes, no C++ types, no exceptions across the
 * boundary.  Every pointer argument except `stream` points to device memory
 * (HBM) unless stated otherwise.
 *
 * What is computed (per batch b, query head h, query row i):
 *   S_ij = scale * q_i . k_j over the visible keys j,
 *   P_ij = exp(S_ij - m_i) / l_i   (safe softmax, m_i = max_j S_ij),
 *   O_i  = sum_j P_ij v_j,  LSE_i = m_i + ln l_i.
 * The definition is section 1.1 of the TileLang tutorial chapter 15
 * ("15-operators-attention"); the forward pass streams K/V tiles and keeps the
 * running max and denominator (its section 2.3 recurrence), so the score
 * matrix never reaches HBM.
 *
 * Layout (BHSD, contiguous, row-major; BHSD is the tutorial's section 1.1
 * convention):
 *   q, o : [B, H,   Sq,  d]        k, v : [B, Hkv, Skv, d]
 *   lse  : [B, H,   Sq] fp32       (may be NULL: not written)
 * q, k, v, o must be 16-byte aligned, lse 4-byte aligned; k and v may be NULL
 * when Skv == 0 (they are not read).
 *
 * Grouped-query attention: H % Hkv == 0 and query head h reads KV head
 * h / (H / Hkv) (tutorial section 4.8 (1)).  Hkv == 1 is multi-query.
 *
 * Causal masking is aligned to the bottom right: key j is visible to query i
 * iff j <= i + (Skv - Sq) (tutorial section 3.4 (2) and 5.2).  A row that
 * sees no key gets O = 0 and LSE = -inf (tutorial section 5.1 (2); the LSE
 * value is this library's reading, the page leaves it open).
 *
 * Variable length (cu_seqlens != NULL; tutorial section 5.3): B is the number
 * of sequences and the batch dimension is 1: q, o [1, H, T, d], k, v
 * [1, Hkv, T, d], lse [1, H, T], with Sq == Skv == T.  cu_seqlens is a device
 * array of B+1 int32 prefix sums (cu_seqlens[0] == 0, non-decreasing,
 * cu_seqlens[B] == T).  Each sequence attends to itself only (Sq_b == Skv_b,
 * so the causal offset is 0).  Values outside [0, T] are clamped by the
 * kernels, so a malformed array gives wrong numbers, never an out-of-bounds
 * access.
 *
 * Decode: a dense call with Sq == 1 takes the split-KV path (tutorial section
 * 4.8 (3) and 5.4): the keys are cut into num_splits contiguous chunks of
 * ceil(Skv / num_splits) keys (the last ones may be short or empty; the split
 * count is clamped to Skv), each chunk produces a
 * normalised partial output and a base-2 log-sum-exp, and a second kernel on
 * the same stream combines them with weights l_s / sum l in a fixed split
 * order (bitwise reproducible, no atomics).
 *
 * Precision: attn_fwd takes bf16 q/k/v/o; both products run on bf16 MFMA with
 * fp32 accumulation, the probabilities are rounded to bf16 (round to nearest
 * even) before the second product, the denominator is summed in fp32 before
 * that rounding.  attn_fwd_f32 takes fp32 q/k/v/o and computes in fp32
 * throughout (no low-precision step).
 *
 * Errors: arguments are validated on the host before any HIP call; on
 * failure nothing is launched and no output is touched.  Sizes: H * d must be
 * below 2^23 (a K/V row of a BSHD tensor times the rows of one tile must fit
 * the 32-bit byte range of a buffer descriptor), and every tensor below
 * 9e18 elements.  HIP failures give
 * ATTN_EHIP.  attn_last_error() returns a per-thread message about the last
 * failure.  Execution is asynchronous on `stream`: ATTN_OK means enqueued.
 *
 * Ownership: the caller owns every buffer and the stream; the library keeps
 * no pointer after the call returns.  The only memory the library allocates
 * is a workspace the caller did not pass: the split-KV partials of the decode
 * path, and the per-row Delta and LSE of the backward, taken and released
 * stream-ordered (hipMallocAsync / hipFreeAsync) on `stream`; besides, its
 * code object holds the static scratch array of attn_fwd_noalloc
 * (ATTN_NOALLOC_SCRATCH_BYTES per GPU).
 *
 * `stream` is a hipStream_t; NULL means the default stream.
 */
#ifndef EXACT_ATTENTION_09_ATTN_H
#define EXACT_ATTENTION_09_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_EINVAL = 1,       /* invalid argument (null pointer, bad size, bad scale, ...) */
  ATTN_EUNSUPPORTED = 2, /* valid but not built: d other than 64 or 128 */
  ATTN_ENOMEM = 3,       /* the workspace could not be allocated */
  ATTN_EHIP = 4          /* a HIP runtime call or a kernel launch failed */
} attn_status;

typedef enum { ATTN_BF16 = 0, ATTN_F32 = 1 } attn_dtype;

/* Tensor layouts (TileLang tutorial section 4.6: the two differ only in the
 * index order; BSHD is how KV caches are usually stored).
 *   ATTN_BHSD: q, o [B, H, Sq, d], k, v [B, Hkv, Skv, d]; varlen [1, H, T, d].
 *   ATTN_BSHD: q, o [B, Sq, H, d], k, v [B, Skv, Hkv, d]; varlen (packed
 *              tokens, "THD") [T, H, d] and [T, Hkv, d].
 * lse is [B, H, Sq] (varlen [H, T]) in both. */
typedef enum { ATTN_BHSD = 0, ATTN_BSHD = 1 } attn_layout;

/* Largest split count the decode path accepts. */
#define ATTN_MAX_SPLITS 256

/* Kernel selection flags for attn_opts.flags (bf16 prefill only; every
 * choice computes the same function, these exist to compare kernels and to
 * test one path against another):
 *   ATTN_FLAG_BASIC_PREFILL: run the basic tiled kernel (one wave group,
 *     BHSD, no window or sink; ignored when a window, sinks or BSHD are
 *     requested) instead of the two-group ping-pong kernel.
 *   ATTN_FLAG_NO_PERSIST: one workgroup per query tile instead of the
 *     persistent grid of one workgroup per CU (the result is bitwise the
 *     same). */
#define ATTN_FLAG_BASIC_PREFILL 1u
#define ATTN_FLAG_NO_PERSIST 2u

typedef struct {
  /* Decode path only: 0 = library heuristic (attn_decode_num_splits), else
   * 1 .. ATTN_MAX_SPLITS. */
  int num_splits;
  /* Decode path only: caller-provided device workspace of at least
   * attn_workspace_bytes(...) bytes, 256-byte aligned; NULL lets the library
   * allocate it stream-ordered.  The workspace must not be used by other work
   * until this call's kernels on `stream` have finished. */
  void* workspace;
  size_t workspace_bytes;
  /* ATTN_FLAG_* bits; 0 for the default kernels.  Unknown bits are
   * ATTN_EINVAL. */
  unsigned flags;
} attn_opts;

/* bf16 q, k, v, o; fp32 lse.  The path named by the pages: tiled forward for
 * Sq > 1 (or varlen), split-KV decode for dense Sq == 1. */
attn_status attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                     const int32_t* cu_seqlens, void* stream);

/* Same arguments with fp32 q, k, v, o. */
attn_status attn_fwd_f32(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int H, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                         const int32_t* cu_seqlens, void* stream);

/* Same arguments plus the element type and options (opts may be NULL). */
attn_status attn_fwd_ex(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                        int H, int Hkv, int Sq, int Skv, int d, float scale, int causal,
                        const int32_t* cu_seqlens, void* stream, attn_dtype dtype,
                        const attn_opts* opts);

/* Bytes of scratch memory attn_fwd_noalloc holds per GPU (16 MiB: the split
 * partials of decode with B * H * splits * (d + 1) * 4 bytes up to that, e.g.
 * B = 32, H = 32, d = 128, 16 splits takes 8.5 MB). */
#define ATTN_NOALLOC_SCRATCH_BYTES (16u << 20)

/* attn_fwd_ex without any device allocation, for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments and results as attn_fwd_ex (bf16 or
 * fp32, dense or varlen, prefill or split-KV decode); opts (may be NULL)
 * gives num_splits and flags, and its workspace must be NULL (ATTN_EINVAL
 * otherwise).  The decode path (dense Sq == 1) keeps its split partials in a
 * library-owned static device array of ATTN_NOALLOC_SCRATCH_BYTES on each
 * GPU, held until the process ends, instead of a workspace; a call whose
 * partials need more (attn_workspace_bytes(B, H, d, splits) bytes) is
 * rejected with ATTN_EINVAL before anything is launched.  The prefill path
 * uses no scratch memory.  Every call on a GPU shares that GPU's array: two
 * calls that may run at the same time on one GPU (streams not ordered by the
 * caller) race on it, so order them on one stream or with events.  The split
 * kernel writes every partial the combine reads, so nothing carries over
 * from an earlier call.  The array's device address is looked up once per
 * device, at the first decode call made with that device current.  No
 * hipMalloc, hipFree or allocating library routine is called. */
attn_status attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                             int Hkv, int Sq, int Skv, int d, float scale, int causal, const int32_t* cu_seqlens,
                             void* stream, attn_dtype dtype, const attn_opts* opts);

/* Causal attention with a sliding window and/or attention sinks, bf16.
 * Same arguments and layouts as attn_fwd (dense or varlen), always causal
 * (bottom-right aligned), plus:
 *   window : 0 for none, else W > 0 keeps key j for query i iff
 *            i + (Skv - Sq) - W < j <= i + (Skv - Sq) (the tutorial's
 *            section 5.2 band; the CUDA course chapter 12, section 12.9.5).
 *            The kernels load and compute only the key tiles inside the band.
 *   sinks  : NULL, or [H] fp32 device array, one logit per query head in the
 *            units of the scaled scores.  A sink joins each row's softmax
 *            denominator and contributes no value (tutorial sections 4.6 and
 *            4.7): O_i = sum_j e^(S_ij - m) v_j / (sum_j e^(S_ij - m) +
 *            e^(sink - m)), m = max(max_j S_ij, sink), and LSE includes the
 *            sink.  A row that sees no key gets O = 0 and LSE = sink (-inf
 *            without sinks).
 * Sq == 1 (dense) takes the split-KV decode path: the splits cut the window
 * and the combine adds the sink.  Errors as for attn_fwd_ex; window < 0 is
 * ATTN_EINVAL. */
attn_status attn_fwd_window_sink(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                                 int Hkv, int Sq, int Skv, int d, float scale, const int32_t* cu_seqlens,
                                 int window, const float* sinks, void* stream, const attn_opts* opts);

/* The general bf16 entry point: attn_fwd's arguments plus the tensor
 * layout, a sliding window and sinks (as for attn_fwd_window_sink; window > 0
 * or sinks != NULL need causal != 0, else ATTN_EINVAL).  attn_fwd,
 * attn_fwd_ex (bf16) and attn_fwd_window_sink are this call with
 * layout = ATTN_BHSD.  Errors as for attn_fwd_ex; an unknown layout is
 * ATTN_EINVAL. */
attn_status attn_fwd_layout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int Hkv,
                            int Sq, int Skv, int d, float scale, int causal, const int32_t* cu_seqlens,
                            attn_layout layout, int window, const float* sinks, void* stream,
                            const attn_opts* opts);

/* Split-KV decode over a paged KV cache: one query row per head (Sq == 1),
 * bf16.  A paged cache changes where the key and value bytes live, not what
 * is computed (tutorial section 4.8 (2)): the cache is cut into pages of
 * page_size tokens and block_table maps logical block j of sequence b to a
 * physical page, key t living in page block_table[b * max_pages +
 * t / page_size] at offset t % page_size (the CUDA course chapter 12,
 * section 12.9.4).
 *
 *   q, o        : [B, H, 1, d] bf16          lse: [B, H] fp32 (may be NULL)
 *   k_cache,
 *   v_cache     : [num_pages, Hkv, page_size, d] bf16 (head-major pages)
 *   block_table : [B, max_pages] int32, entries in [0, num_pages)
 *   seqlens_k   : [B] int32, keys of sequence b, in [0, max_pages*page_size]
 *
 * page_size must be a power of two from 16 to 65536 (the CUDA course asks
 * for multiples of 16; powers of two keep the page arithmetic to shifts),
 * else ATTN_EUNSUPPORTED.  Device-side entries are clamped into range, so a
 * malformed table or length gives wrong numbers, never an out-of-bounds
 * access.  A sequence with no key gets O = 0 and LSE = -inf.  Splits: each
 * sequence's keys are cut into num_splits chunks of
 * ceil(seqlens_k[b] / num_splits) keys and combined as in attn_fwd's decode
 * path; opts (may be NULL) gives the split count and the workspace
 * (attn_workspace_bytes(B, H, d, num_splits) bytes), with the same rules.
 * Validation, errors, ownership and ordering on `stream` are as for
 * attn_fwd_ex. */
attn_status attn_fwd_paged(const void* q, const void* k_cache, const void* v_cache, void* o, float* lse,
                           const int32_t* block_table, const int32_t* seqlens_k, int B, int H, int Hkv,
                           int d, int page_size, int max_pages, int num_pages, float scale, void* stream,
                           const attn_opts* opts);

/* Backward pass: gradients of attn_fwd's output with respect to q, k, v
 * (bf16, BHSD, causal or not, dense or packed variable-length sequences;
 * attn_bwd_layout below takes the BSHD layouts as well).
 * The pages name the backward only as the tutorial's section 5.4 Ascend
 * example (dQ partial tiles added with bf16 atomics, with the resulting
 * error); this library computes the derivative of the forward's definition
 * without atomics, bitwise reproducibly:
 *   Delta_i = rowsum(dout_i * o_i),  P = exp(scale q k^T - LSE)
 *   dv = P^T dout,  dS = P * (dout v^T - Delta),  dq = scale dS k,
 *   dk = scale dS^T q
 * with the grouped-query sums over each KV head's query heads.
 *   q, o, dout, dq : [B, H, Sq, d] bf16       lse : [B, H, Sq] fp32 (attn_fwd's)
 *   k, v, dk, dv   : [B, Hkv, Skv, d] bf16
 * cu_seqlens != NULL selects varlen exactly as in attn_fwd_ex: B sequences
 * packed into [1, H, T, d] (q, o, dout, dq), [1, Hkv, T, d] (k, v, dk, dv)
 * and [1, H, T] (lse), Sq == Skv == T == cu_seqlens[B], each sequence
 * attending to itself (causal offset 0).
 * o and lse must be the forward outputs for the same q, k, v, scale,
 * causal flag and cu_seqlens.  P and dS are rounded to bf16 (nearest even)
 * for the products that use them; all sums are fp32.  The workspace (opts,
 * may be NULL) holds Delta and the LSE in log2 units, one fp32 per query row
 * each: attn_bwd_workspace_bytes(B, H, Sq) bytes (varlen: (1, H, T)),
 * 256-byte aligned, else it is allocated stream-ordered.  Validation, errors
 * and ordering on `stream` as for attn_fwd_ex; opts->num_splits and opts->flags
 * are ignored. */
attn_status attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                     void* dq, void* dk, void* dv, int B, int H, int Hkv, int Sq, int Skv, int d, float scale,
                     int causal, const int32_t* cu_seqlens, void* stream, const attn_opts* opts);

/* Backward pass of attn_fwd_window_sink: causal attention with a sliding
 * window (window > 0; 0 = none) and/or per-head attention sinks (sinks: fp32
 * [H] logits, may be NULL), dense or varlen, as attn_bwd otherwise.  The
 * tutorial's sections 5.2 (the window band) and 4.6-4.7 (the sink: a logit in
 * each row's softmax without a value) define the forward; its derivative
 * changes only the mask for the window, while each sink is one more softmax
 * column whose gradient is
 *   dsinks[h] = - sum over the rows i of head h of exp(sink_h - LSE_i) Delta_i
 * (o and lse must be attn_fwd_window_sink's for the same window and sinks; a
 * row that saw no key has LSE = sink and contributes 0).  dsinks: fp32 [H]
 * output, required when sinks != NULL, summed in a fixed order (bitwise
 * reproducible).  Workspace, validation, errors and ordering as for
 * attn_bwd. */
attn_status attn_bwd_window_sink(const void* q, const void* k, const void* v, const void* o, const void* dout,
                                 const float* lse, void* dq, void* dk, void* dv, float* dsinks, int B, int H, int Hkv,
                                 int Sq, int Skv, int d, float scale, const int32_t* cu_seqlens, int window,
                                 const float* sinks, void* stream, const attn_opts* opts);

/* The general backward entry point: attn_bwd's arguments plus the tensor
 * layout, a sliding window and sinks (as for attn_bwd_window_sink; window > 0
 * or sinks != NULL need causal != 0, else ATTN_EINVAL).  attn_bwd and
 * attn_bwd_window_sink are this call with layout = ATTN_BHSD.  Under
 * ATTN_BSHD the bf16 tensors are those of attn_fwd_layout:
 *   q, o, dout, dq : [B, Sq, H, d]      k, v, dk, dv : [B, Skv, Hkv, d]
 *   varlen (cu_seqlens != NULL, packed tokens): [T, H, d] and [T, Hkv, d]
 * while lse stays [B, H, Sq] ([H, T] varlen), as attn_fwd_layout writes it.
 * The gradients are the same numbers in either layout (the same arithmetic
 * in the same order), and the Delta/LSE workspace is the same size.
 * H * d must be below 2^23 (ATTN_EINVAL otherwise), as for the forward.
 * dsinks: fp32 [H], required when sinks != NULL.  Validation, errors,
 * workspace and ordering on `stream` as for attn_bwd; an unknown layout is
 * ATTN_EINVAL. */
attn_status attn_bwd_layout(const void* q, const void* k, const void* v, const void* o, const void* dout,
                            const float* lse, void* dq, void* dk, void* dv, float* dsinks, int B, int H, int Hkv,
                            int Sq, int Skv, int d, float scale, int causal, const int32_t* cu_seqlens,
                            attn_layout layout, int window, const float* sinks, void* stream,
                            const attn_opts* opts);

/* Bytes of workspace attn_bwd needs (0 for invalid sizes). */
size_t attn_bwd_workspace_bytes(int B, int H, int Sq);

/* Bytes of workspace the decode path needs for B, H, d and num_splits
 * (fp32 partial outputs [B,H,splits,d] and base-2 LSEs [B,H,splits]).
 * Returns 0 for invalid sizes. */
size_t attn_workspace_bytes(int B, int H, int d, int num_splits);

/* The split count the decode path uses for these sizes when the caller
 * passes none: enough splits of at least 256 keys for about 1024
 * workgroups. */
int attn_decode_num_splits(int B, int Hkv, int Skv);

/* Static text for a status code. */
const char* attn_status_string(attn_status s);

/* Detail about the last failure on the calling thread ("" if none). */
const char* attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_09_ATTN_H */
