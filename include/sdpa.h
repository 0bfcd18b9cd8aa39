/*
 * sdpa.h -- C ABI of the MI355X (gfx950) fused scaled-dot-product attention: the forward
 * (sdpa_fwd) and its gradients (sdpa_bwd).
 *
 * The operation ("Profiling in PyTorch (part 3): attention", naive causal attention
 * section, five steps; SDPA section, the one-call form that takes a mask or a causal
 * flag; math-backend section, the safe softmax):
 *
 *   out[b,h,i,:] = sum_j P[i,j] v[b,h,j,:],   P[i,:] = softmax over the visible keys j of
 *                                                      scale * q[b,h,i,:].k[b,h,j,:]
 *   lse[b,h,i]   = log sum_{visible j} exp(scale * q[b,h,i,:].k[b,h,j,:])   (natural log)
 *
 *   key j is visible to query i iff causal(i, j) && (mask == NULL || mask[b,h,i,j] != 0),
 *   causal(i, j) = true (SDPA_CAUSAL_NONE), j <= i (SDPA_CAUSAL_TOP_LEFT) or
 *                  j <= i + Lk - Lq (SDPA_CAUSAL_BOTTOM_RIGHT)
 *
 * A query row with no visible key returns an all-zero output row and lse = -inf (the safe
 * softmax of the math-backend section; no NaN is ever produced for finite inputs).  The
 * pages draw the causal triangle only for Lq == Lk, where both alignments agree; top-left
 * is the default reading, and bottom-right (the last query sees every key) serves queries
 * that continue a longer key sequence, such as decoding.
 *
 * Rank-3 and rank-4 inputs take the same fused kernel (the PyTorch 2.14 note on rank-3
 * SDPA inputs): a rank-3 [N,L,D] input is computed exactly as the rank-4 input
 * [1,N,L,D], bit for bit.
 *
 * The library launches exactly one kernel per sdpa_fwd call on the caller's stream,
 * allocates nothing, frees nothing, never synchronises, and keeps no per-call state (its
 * globals are a per-device cache of the architecture check and the static split-key
 * workspace of sdpa_fwd_splitkv_noalloc).  Calls are thread-safe, except that calls of
 * sdpa_fwd_splitkv_noalloc that overlap in time on one device share that workspace.
 */
#ifndef SDPA_MI355X_H_
#define SDPA_MI355X_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types of q, k, v and out (all four share one). */
enum sdpa_dtype {
  SDPA_F32 = 0,  /* IEEE binary32; products and sums in fp32 (matrix cores, fp32 MFMA)   */
  SDPA_BF16 = 1, /* bfloat16; bf16 products on matrix cores with fp32 accumulation, the
                    softmax in fp32, probabilities rounded to bf16 (nearest-even) before
                    the product with V                                                    */
  SDPA_F16 = 2   /* IEEE binary16; as SDPA_BF16 with fp16 products and probabilities
                    rounded to fp16 (nearest-even); outputs are finite when |v| is, since
                    every output is a convex combination of value rows                   */
};

/* Status codes.  On any nonzero status nothing was launched and nothing was written. */
enum sdpa_status {
  SDPA_OK = 0,
  SDPA_ERR_NULL = 1,     /* a required pointer is NULL (strides, or q/k/v/out when read) */
  SDPA_ERR_RANK = 2,     /* rank not 3 or 4, or rank 3 with B != 1                       */
  SDPA_ERR_SHAPE = 3,    /* negative size, or a size/extent beyond the supported maximum */
  SDPA_ERR_HEAD_DIM = 4, /* D not a supported head dim (32, 64, 96, 128, 256)            */
  SDPA_ERR_DTYPE = 5,    /* dtype not an sdpa_dtype                                      */
  SDPA_ERR_STRIDE = 6,   /* innermost stride != 1, or a negative stride                  */
  SDPA_ERR_ALIGN = 7,    /* q/k/v/out base or row stride not 16-byte aligned, lse not 4  */
  SDPA_ERR_SCALE = 8,    /* scale is NaN or infinite                                     */
  SDPA_ERR_DEVICE = 9,   /* the stream's device is not gfx950, or the launch failed      */
  SDPA_ERR_CAUSAL = 10,  /* causal mode not an sdpa_causal value                         */
  SDPA_ERR_WORKSPACE = 11, /* workspace smaller than sdpa_fwd_splitkv_workspace() bytes  */
  SDPA_ERR_STATIC_WORKSPACE = 12 /* sdpa_fwd_splitkv_noalloc: the problem needs more than
                                    SDPA_STATIC_WORKSPACE_BYTES of split-key workspace    */
};

/* Causal modes (the is_causal / causal arguments). */
enum sdpa_causal {
  SDPA_CAUSAL_NONE = 0,
  SDPA_CAUSAL_TOP_LEFT = 1,     /* key j visible to query i iff j <= i                   */
  SDPA_CAUSAL_BOTTOM_RIGHT = 2  /* iff j <= i + Lk - Lq: the last query sees every key  */
};

/*
 * sdpa_fwd -- fused SDPA forward with per-row LSE, one kernel on `stream`.
 *
 *   q, k, v, out  device pointers to elements of `dtype`.  q and out are [B,H,Lq,D]
 *                 (rank 4) or [N,Lq,D] (rank 3); k and v are [B,H,Lk,D] / [N,Lk,D].
 *                 Any layout whose innermost (D) stride is 1 is accepted, e.g. a
 *                 [B,L,H,D] buffer viewed as [B,H,L,D]: there is no transpose or copy.
 *                 Base pointers and every non-innermost stride (in bytes) must be
 *                 multiples of 16.  out must not overlap q, k or v, nor itself.
 *                 k and v may be NULL when Lk == 0; q and out may be NULL when
 *                 B*H*Lq == 0.
 *   lse           NULL, or a device pointer to B*H*Lq contiguous floats ([B,H,Lq] /
 *                 [N,Lq]), 4-byte aligned, receiving the natural-log LSE (-inf for
 *                 rows with no visible key).
 *   rank          3 or 4.  Rank 3 requires B == 1 and H == N.
 *   B,H,Lq,Lk,D   sizes; D in {32, 64, 96, 128, 256} (the head dims an SDPA dispatcher
 *                 routes by, "profiling attention in pytorch" (news.bpdata), section
 *                 Scaled Dot Product Attention (SDPA) es backendes valasztas; every dtype,
 *                 mask kind and causal mode takes every one of them); Lq, Lk and B*H
 *                 below 2^31; (Lk + 64) times the row stride of k (and of v) must stay
 *                 below 2 GiB (one head's rows are addressed with 32-bit offsets).  B*H*Lq == 0 is a no-op returning
 *                 SDPA_OK; Lk == 0 makes every row empty.
 *   strides       5*rank element strides, tensor-major: q, k, v, out, mask, each in its
 *                 own axis order ([N,L,D] / [B,H,L,D]; the mask is [N,Lq,Lk] /
 *                 [B,H,Lq,Lk]).  The mask's entries are ignored when mask == NULL.
 *                 Mask strides may be 0 (broadcast, e.g. one mask for all heads); the
 *                 mask's innermost (key) stride must be 1.
 *   scale         finite multiplier of q.k applied after the dot product (the usual
 *                 choice is 1/sqrt(D); any finite value, including 0 or negative, is
 *                 accepted).
 *   is_causal     an sdpa_causal mode (0 none, 1 top-left, 2 bottom-right); combines
 *                 with a mask by intersection.  Other values: SDPA_ERR_CAUSAL.
 *   mask          NULL, or a device pointer to bytes, nonzero = visible, 0 = hidden.
 *   dtype         an sdpa_dtype.
 *   stream        a hipStream_t (NULL = the null stream of the current device).
 *
 * Ownership: every pointer is owned by the caller and must stay valid until the work on
 * `stream` has completed.  Errors: validation runs on the host before any launch; a
 * failed launch returns SDPA_ERR_DEVICE; faults during execution surface at the
 * caller's next synchronisation.
 */
int sdpa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int rank,
             int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D, const int64_t* strides,
             float scale, int is_causal, const uint8_t* mask, int dtype, void* stream);

/*
 * sdpa_check -- the host-side validation of sdpa_fwd alone (same arguments, no stream).
 * Makes no HIP call and reads no device memory (pointers are only tested for NULL and
 * alignment), so it runs on a machine without a GPU.  Returns the status sdpa_fwd would
 * return before launching.
 */
int sdpa_check(const void* q, const void* k, const void* v, const void* out, const float* lse,
               int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
               const int64_t* strides, float scale, int is_causal, const uint8_t* mask,
               int dtype);

/* sdpa_strerror -- a static, human-readable message for a status code. */
const char* sdpa_strerror(int status);

/*
 * sdpa_fwd_bias -- sdpa_fwd with an additive float mask instead of the boolean one: the
 * scores become scale * q_i.k_j + bias[b,h,i,j] before the softmax (a -inf entry hides the
 * key; a row whose keys are all hidden returns zeros and lse = -inf, as in sdpa_fwd).  The
 * naive module's masked_fill to -inf is this with entries 0 and -inf; the SDPA call the
 * pages profile takes a mask and picks its kernel by dtype, head dim, mask and hardware
 * (the Hungarian edition of "Profiling in PyTorch" part 3, section Scaled Dot Product
 * Attention (SDPA) és backendes választás).
 *
 *   bias          NULL (then this is sdpa_fwd without a mask), or a device pointer to fp32
 *                 values addressed through the fifth group of strides exactly as sdpa_fwd
 *                 addresses its mask: innermost (key) stride 1, strides may be 0 to
 *                 broadcast, 4-byte aligned (16-byte aligned base and row strides let rows
 *                 be read 16 bytes at a time).  Entries must not be +inf or NaN.
 *   everything else
 *                 as in sdpa_fwd (is_causal combines with the bias).
 */
int sdpa_fwd_bias(const void* q, const void* k, const void* v, void* out, float* lse, int rank,
                  int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                  const int64_t* strides, float scale, int is_causal, const float* bias,
                  int dtype, void* stream);

/* sdpa_fwd_bias_check -- the host-side validation of sdpa_fwd_bias alone. */
int sdpa_fwd_bias_check(const void* q, const void* k, const void* v, const void* out,
                        const float* lse, int rank, int64_t B, int64_t H, int64_t Lq,
                        int64_t Lk, int64_t D, const int64_t* strides, float scale,
                        int is_causal, const float* bias, int dtype);

/*
 * sdpa_fwd_splitkv -- sdpa_fwd (no mask) with the keys of every head split into chunks
 * that separate workgroups process in parallel, for problems with few query rows per head
 * and many keys (decoding: one or a few new queries against a long key sequence), where
 * one workgroup per (head, query tile) would leave most of the chip idle.  Each chunk's
 * workgroup writes its rows' softmax-normalised partial output and partial lse to
 * `workspace`; a second kernel merges them exactly through the lse (the same merge that
 * combines attention over disjoint key sets, which the exported lse of the pages' fused
 * forward exists for):  lse = log sum_s exp(lse_s),  out = sum_s exp(lse_s - lse) out_s.
 * The result equals sdpa_fwd's up to the order of the floating-point sums.
 *
 *   q, k, v, out, lse, rank, B..D, scale, is_causal, dtype, stream
 *                 as in sdpa_fwd (all three causal modes); there is no mask.
 *   strides       4*rank element strides: q, k, v, out.
 *   num_splits    requested number of key chunks, 1..1024, or 0 for the library's choice
 *                 (enough workgroups to fill the chip, at least 512 keys per chunk, at most
 *                 64 chunks).  Chunks hold a multiple of 64 keys, so fewer may be used.
 *   workspace     device memory of at least sdpa_fwd_splitkv_workspace(...) bytes,
 *                 16-byte aligned, owned by the caller; its contents on entry do not
 *                 matter and on return are scratch.  Calls that share a workspace must not
 *                 overlap in time.
 *   workspace_bytes  its size (SDPA_ERR_WORKSPACE if smaller than needed).
 *
 * Two launches on `stream` (chunks, then the merge); nothing allocated or synchronised.
 */
int sdpa_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                     int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                     const int64_t* strides, float scale, int is_causal, int64_t num_splits,
                     void* workspace, int64_t workspace_bytes, int dtype, void* stream);

/* sdpa_fwd_splitkv_check -- the host-side validation of sdpa_fwd_splitkv alone. */
int sdpa_fwd_splitkv_check(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, int rank, int64_t B, int64_t H, int64_t Lq,
                           int64_t Lk, int64_t D, const int64_t* strides, float scale,
                           int is_causal, int64_t num_splits, const void* workspace,
                           int64_t workspace_bytes, int dtype);

/* sdpa_fwd_splitkv_workspace -- workspace bytes sdpa_fwd_splitkv needs for these sizes and
 * requested num_splits (0 = the library's choice): nsplit * B*H * Lq * (D + 1) * 4.
 * Returns minus an sdpa_status for invalid sizes. */
int64_t sdpa_fwd_splitkv_workspace(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                                   int64_t num_splits, int dtype);

/* Bytes of the static split-key workspace of sdpa_fwd_splitkv_noalloc (per device). */
#define SDPA_STATIC_WORKSPACE_BYTES (16ll << 20)

/*
 * sdpa_fwd_splitkv_noalloc -- sdpa_fwd_splitkv for callers that cannot allocate device
 * memory: code being captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc.  It takes no workspace argument; the partial outputs and lse go to a static
 * device array of SDPA_STATIC_WORKSPACE_BYTES (16 MiB) that the library holds on every
 * device it runs on until the process ends.  The library allocates and frees nothing; the
 * array's device address is looked up once per device, on the first call there.
 *
 *   arguments     as sdpa_fwd_splitkv, without workspace / workspace_bytes.
 *   limit         problems needing more than SDPA_STATIC_WORKSPACE_BYTES (that is,
 *                 sdpa_fwd_splitkv_workspace(B, H, Lq, Lk, D, num_splits, dtype) bytes) are
 *                 rejected with SDPA_ERR_STATIC_WORKSPACE before anything is launched.
 *   sharing       every call on one device uses that device's one array, whose contents
 *                 each call overwrites (nothing in it needs to start at zero): calls that
 *                 overlap in time on one device race, e.g. calls on two streams that are not
 *                 ordered by an event; calls on one stream are ordered and safe.
 *
 * Two launches on `stream` (chunks, then the merge); the result is the same as
 * sdpa_fwd_splitkv's for the same num_splits, bit for bit.
 */
int sdpa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                             int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                             const int64_t* strides, float scale, int is_causal,
                             int64_t num_splits, int dtype, void* stream);

/*
 * sdpa_fwd_varlen -- the fused forward over a batch of sequences of different lengths
 * packed along the token axis (the cu_seqlens layout of the packed-document kernels in
 * "[flashinfer] FlashInfer, Cake DSA 커널 최적화: Sparse Attention 성능 2배 향상", section 3,
 * Varlen 인덱스 준비 최적화).  Sequence s owns query tokens cu_seqlens_q[s] ..
 * cu_seqlens_q[s+1]-1 and key tokens cu_seqlens_k[s] .. cu_seqlens_k[s+1]-1; each of its
 * heads is the problem of sdpa_fwd on those rows alone (no attention across sequences),
 * with the causal mode applied per sequence (bottom-right uses that sequence's own lengths).
 *
 *   q, out        device [total_q, H, D], k, v device [total_k, H, D], of `dtype`, any token
 *                 and head strides, unit dim stride, bases and strides (bytes) multiples of
 *                 16.  q/out may be NULL when nothing is computed, k/v when total_k == 0.
 *   lse           NULL, or device [H, total_q] contiguous floats (natural log, -inf for
 *                 rows with no visible key), 4-byte aligned.
 *   cu_seqlens_q, cu_seqlens_k
 *                 device int32 arrays of nseq + 1 non-decreasing offsets from 0 to total_q
 *                 (total_k), 4-byte aligned.  Their contents are not validated on the host;
 *                 the kernel clamps every offset into [0, total] and makes them
 *                 non-decreasing, so any contents keep every access in bounds (rows of a
 *                 sequence past the clamped range are then left unwritten).
 *   nseq          number of sequences (>= 0).
 *   max_seqlen_q  an upper bound of every cu_seqlens_q[s+1] - cu_seqlens_q[s], at most
 *                 total_q (it sizes the launch; query rows past it are not written).
 *   total_q, total_k, H, D
 *                 sizes; D in {32, 64, 96, 128, 256}; (total_k + 64) times the token
 *                 stride of k (and of v) must stay below 2 GiB.
 *   strides       12 element strides: (token, head, dim) for q, k, v, out.
 *   scale, causal, dtype, stream
 *                 as in sdpa_fwd (causal: an sdpa_causal mode).
 *
 * One kernel launch; nothing allocated, freed or synchronised.  Returns a status as
 * sdpa_fwd does; nseq * H * total_q * max_seqlen_q == 0 is a no-op returning SDPA_OK.
 */
int sdpa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t nseq,
                    int64_t max_seqlen_q, int64_t total_q, int64_t total_k, int64_t H, int64_t D,
                    const int64_t* strides, float scale, int causal, int dtype, void* stream);

/* sdpa_fwd_varlen_check -- the host-side validation of sdpa_fwd_varlen alone (no stream,
 * no HIP call, no device read). */
int sdpa_fwd_varlen_check(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, int64_t nseq, int64_t max_seqlen_q,
                          int64_t total_q, int64_t total_k, int64_t H, int64_t D,
                          const int64_t* strides, float scale, int causal, int dtype);

/*
 * sdpa_bwd -- gradients dq, dk, dv of sdpa_fwd for an upstream gradient dout.
 *
 * The derivative of the forward above by the chain rule through its steps.  The pages
 * define no backward; it reuses the forward's exported lse, as the fused forward of
 * "[flashinfer] FlashInfer, Cake DSA 커널 최적화: Sparse Attention 성능 2배 향상" returns its
 * lse for its backward (section 2, In-place Strided dout 처리, which also takes a strided
 * dout without copying it, as here):
 *
 *   P[i,j]  = exp(scale * q_i.k_j - lse[i]) for visible (i,j), else 0  (all 0 if lse = -inf)
 *   dv[j,:] = sum_i P[i,j] dout[i,:]
 *   dP[i,j] = dout[i,:].v[j,:],   delta[i] = sum_d dout[i,d] out[i,d]  (= sum_j P[i,j] dP[i,j])
 *   dS[i,j] = P[i,j] (dP[i,j] - delta[i])
 *   dq[i,:] = scale * sum_j dS[i,j] k[j,:],   dk[j,:] = scale * sum_i dS[i,j] q[i,:]
 *
 * bf16 and fp16 at D <= 128 (tiled matrix-core kernels): P and dS are rounded to the input
 * type (nearest-even) before their products (for dk, dS is formed from the rounded P);
 * every product accumulates in fp32, and dq, dk, dv are rounded to the input type once at
 * the end.  fp32 inputs (every D) and D = 256 (every dtype) take row-by-row kernels on the
 * vector ALU: one wave per query row, then one per key row, every value and sum in fp32
 * (P and dS not rounded), dq, dk, dv rounded to the input type at the end; correct for
 * every shape, not tuned for speed.  Deterministic: no atomics, every
 * output element is written by exactly one lane.  A query row with no
 * visible key gets dq = 0 and contributes nothing to dk, dv; a key seen by no query gets
 * dk = dv = 0.
 *
 *   q, k, v, out, dout, dq, dk, dv
 *                 device pointers to `dtype`.  q, out, dout, dq are [B,H,Lq,D] / [N,Lq,D];
 *                 k, v, dk, dv are [B,H,Lk,D] / [N,Lk,D]; any layout with unit innermost
 *                 stride.  Bases and non-innermost strides (in bytes) multiples of 16.
 *                 dq, dk, dv must not overlap each other or any input.  q/out/dout/dq
 *                 may be NULL when B*H*Lq == 0, k/v/dk/dv when B*H*Lk == 0.
 *   lse           device pointer to the B*H*Lq contiguous floats sdpa_fwd wrote for this
 *                 same problem (natural log, -inf for empty rows); required when
 *                 B*H*Lq > 0.
 *   delta         device pointer to B*H*Lq contiguous floats of caller-owned scratch,
 *                 4-byte aligned; receives delta[i] above (fp32).  Required when
 *                 B*H*Lq > 0.
 *   rank, B..D    as in sdpa_fwd (D in {32, 64, 96, 128, 256}); additionally (Lq + 64) times the row
 *                 stride of q (and of dout) must stay below 2 GiB.
 *   strides       9*rank element strides, tensor-major: q, k, v, out, dout, dq, dk, dv,
 *                 mask, each in its own axis order as in sdpa_fwd.
 *   scale, is_causal, mask
 *                 exactly as passed to sdpa_fwd (all three causal modes).
 *   dtype         SDPA_F32, SDPA_BF16 or SDPA_F16 (anything else: SDPA_ERR_DTYPE).
 *   stream        a hipStream_t (NULL = the null stream of the current device).
 *
 * Launches two kernels on `stream` (dq and delta first, then dk and dv); allocates,
 * frees and synchronises nothing.  Ownership and errors as for sdpa_fwd.
 */
int sdpa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta, int rank, int64_t B,
             int64_t H, int64_t Lq, int64_t Lk, int64_t D, const int64_t* strides, float scale,
             int is_causal, const uint8_t* mask, int dtype, void* stream);

/* sdpa_bwd_check -- the host-side validation of sdpa_bwd alone (no stream, no HIP call,
 * no device read).  Returns the status sdpa_bwd would return before launching. */
int sdpa_bwd_check(const void* q, const void* k, const void* v, const void* out,
                   const void* dout, const float* lse, const void* dq, const void* dk,
                   const void* dv, const float* delta, int rank, int64_t B, int64_t H,
                   int64_t Lq, int64_t Lk, int64_t D, const int64_t* strides, float scale,
                   int is_causal, const uint8_t* mask, int dtype);

/*
 * sdpa_bwd_bias -- gradients dq, dk, dv of sdpa_fwd_bias, with the additive mask held
 * constant (no gradient is formed for it).
 *
 * sdpa_bwd's chain rule with the forward's scores scale * q_i.k_j + bias[b,h,i,j]: only P
 * changes, P[i,j] = exp(scale * q_i.k_j + bias[b,h,i,j] - lse[i]) (0 where the bias is
 * -inf); dv, dP, delta, dS, dq and dk then follow as in sdpa_bwd.  The forward it
 * differentiates is sdpa_fwd_bias: the naive module's masked fill before the softmax (the
 * Hungarian edition of "Profiling in PyTorch" part 3), with the mask's entries generalised
 * from 0 / -inf to any finite value or -inf.  The pages define no backward; this is the
 * chain rule through that forward.
 *
 *   bias          device fp32, 4-byte aligned, addressed with the mask strides of
 *                 `strides` (rank entries each, 0 broadcasts an axis, innermost 1); the
 *                 same tensor, with the same values, that sdpa_fwd_bias used for lse.
 *                 Entries must be finite or -inf.  NULL is the bias-free sdpa_bwd.
 *   everything else
 *                 exactly as in sdpa_bwd (lse from sdpa_fwd_bias on the same problem).
 *
 * Two kernel launches on `stream`, as sdpa_bwd; nothing allocated, freed or synchronised.
 * Deterministic.  With all-zero bias the result equals sdpa_bwd's, bit for bit.
 */
int sdpa_bwd_bias(const void* q, const void* k, const void* v, const void* out,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  float* delta, int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                  int64_t D, const int64_t* strides, float scale, int is_causal,
                  const float* bias, int dtype, void* stream);

/* sdpa_bwd_bias_check -- the host-side validation of sdpa_bwd_bias alone (no stream, no
 * HIP call, no device read). */
int sdpa_bwd_bias_check(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, const void* dq, const void* dk,
                        const void* dv, const float* delta, int rank, int64_t B, int64_t H,
                        int64_t Lq, int64_t Lk, int64_t D, const int64_t* strides, float scale,
                        int is_causal, const float* bias, int dtype);

/*
 * sdpa_bwd_varlen -- gradients dq, dk, dv of sdpa_fwd_varlen (packed sequences).
 *
 * Each (sequence, head) is sdpa_bwd's problem on that sequence's rows alone, with the
 * causal mode applied per sequence as in sdpa_fwd_varlen; no gradient flows across
 * sequences.  Same rounding and determinism as sdpa_bwd.
 *
 *   q, out, dout, dq
 *                 device [total_q, H, D] of `dtype` (fp32, bf16 or fp16); k, v, dk, dv device
 *                 [total_k, H, D].  Any token and head strides, unit dim stride; bases and
 *                 strides (bytes) multiples of 16.  Outputs must not overlap each other or
 *                 any input.  The query-side tensors may be NULL when total_q == 0, the
 *                 key-side ones when total_k == 0.
 *   lse           device [H, total_q] contiguous floats written by sdpa_fwd_varlen for this
 *                 problem.
 *   delta         device [H, total_q] contiguous floats of caller-owned scratch (fp32
 *                 delta[i] = sum_d dout[i,d] out[i,d]).
 *   cu_seqlens_q, cu_seqlens_k, nseq
 *                 as in sdpa_fwd_varlen (contents clamped on the device, never read out of
 *                 bounds).
 *   max_seqlen_q, max_seqlen_k
 *                 upper bounds of every sequence's query and key length, at most total_q
 *                 and total_k; they size the launches.  Rows of a longer sequence past them
 *                 are not written.
 *   total_q, total_k, H, D
 *                 sizes; D in {32, 64, 96, 128, 256}; (total + 64) times the token stride of q,
 *                 dout, k and v (each with its own total) must stay below 2 GiB.
 *   strides       24 element strides: (token, head, dim) for q, k, v, out, dout, dq, dk, dv.
 *   scale, causal, dtype, stream
 *                 as in sdpa_bwd (causal: an sdpa_causal mode).
 *
 * Two kernel launches on `stream`; nothing allocated, freed or synchronised.  Returns a
 * status as sdpa_bwd does; nseq * H == 0 or max_seqlen_q + max_seqlen_k == 0 is a no-op.
 */
int sdpa_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    float* delta, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int64_t nseq, int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t total_q,
                    int64_t total_k, int64_t H, int64_t D, const int64_t* strides, float scale,
                    int causal, int dtype, void* stream);

/* sdpa_bwd_varlen_check -- the host-side validation of sdpa_bwd_varlen alone (no stream,
 * no HIP call, no device read). */
int sdpa_bwd_varlen_check(const void* q, const void* k, const void* v, const void* out,
                          const void* dout, const float* lse, const void* dq, const void* dk,
                          const void* dv, const float* delta, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, int64_t nseq, int64_t max_seqlen_q,
                          int64_t max_seqlen_k, int64_t total_q, int64_t total_k, int64_t H,
                          int64_t D, const int64_t* strides, float scale, int causal,
                          int dtype);

/*
 * Launch plan (host-only introspection of the tile scheduler of sdpa_fwd; sdpa_fwd_bias
 * takes the same tiles).
 *
 * A work item is one (b*H + h, query tile) pair: block_m query rows of one head, which
 * walk the key/value tiles of block_n keys.  16-bit inputs take one of three tiles:
 *   - 256 rows and 512 threads (two waves per SIMD in alternating matrix / vector phases),
 *     for D = 96 and 128 when the problem has more than 512 items of 256 rows (at D = 128
 *     with is_causal: more than 1024 such items, or more than 2048 keys);
 *   - 128 rows and 512 threads, the key split (two groups of four waves walk the two halves
 *     of the item's key tiles in alternating phases and merge their rows; one workgroup
 *     per CU, lds_bytes twice the 128-row tile's), for causal problems at D <= 64 with at
 *     most 256 items of 128 rows and at least 1024 keys, or at most 512 such items and at
 *     least 2048 keys;
 *   - 128 rows and 256 threads (one wave per SIMD; two such workgroups share a CU up to
 *     D = 128) otherwise: every other problem at D <= 64, problems of at most 512 items of
 *     256 rows at D = 96 and 128, causal problems at D = 128 of at most 1024 such items and
 *     2048 keys, and D = 256.
 * fp32 inputs: 128 rows, 256 threads.  (sdpa_fwd_varlen always takes the 256-row tile up to
 * D = 128; sdpa_fwd_splitkv the 128-row tile when Lq <= 128.)  With is_causal the items are
 * issued heaviest-first (last query tile of every head first), so the long items start
 * early and the short ones fill the tail.  Without it the items are issued query-tile-major
 * with heads innermost, so the heads that share a broadcast mask tile run back to back.
 */
typedef struct sdpa_plan {
  int64_t block_m;      /* query rows per work item                                    */
  int64_t block_n;      /* keys per inner step                                         */
  int64_t threads;      /* threads per workgroup (wave64)                              */
  int64_t q_tiles;      /* ceil(Lq / block_m)                                          */
  int64_t bh;           /* B*H                                                         */
  int64_t items;        /* bh * q_tiles = workgroups launched                          */
  int64_t lds_bytes;    /* LDS per workgroup                                           */
  int64_t is_causal;    /* issue order: 1 heaviest-first, 0 tile-major                 */
} sdpa_plan_t;

/* Fill `plan` for a problem that sdpa_check accepts (pointers are not needed). Returns
 * SDPA_ERR_NULL for plan == NULL, or the validation status of the sizes and dtype. */
int sdpa_plan(int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
              int is_causal, int dtype, sdpa_plan_t* plan);

/* The work item that workgroup `block` (0 <= block < plan->items) runs: its flat head
 * index b*H + h and its query tile.  This is the decode the kernel performs on the GPU.
 * Returns SDPA_ERR_SHAPE for a block out of range. */
int sdpa_plan_item(const sdpa_plan_t* plan, int64_t block, int64_t* bh, int64_t* q_tile);

#ifdef __cplusplus
}
#endif

#endif /* SDPA_MI355X_H_ */
