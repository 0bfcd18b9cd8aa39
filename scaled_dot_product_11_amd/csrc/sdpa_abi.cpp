// sdpa_abi.cpp -- the exported C ABI: validation, the rank-3/rank-4 stride normaliser,
// the launch plan, status strings, and the one launch per call.
//
// Rank handling follows the PyTorch 2.14 note on rank-3 SDPA inputs: a folded or missing
// batch dimension is the same computation, so a rank-3 [N,L,D] problem is rewritten as
// the rank-4 problem [1,N,L,D] (batch stride 0) before anything else happens, and both
// ranks reach the same fused kernel with the same arguments.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/sdpa.h"
#include "sdpa_internal.h"

namespace {

constexpr int64_t kMaxDim = (int64_t(1) << 31) - 1;
static_assert(SDPA_STATIC_WORKSPACE_BYTES == sdpa::kStaticWorkspaceBytes,
              "header and library disagree on the static workspace size");

bool aligned(const void* p, int64_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// A one-dimensional launch of `blocks` workgroups of `threads` work-items fits HIP's limits:
// at most 2^31 - 1 workgroups and fewer than 2^32 work-items in the dimension.
bool launch_fits(int64_t blocks, int64_t threads) {
  return blocks <= kMaxDim && blocks * threads <= int64_t(UINT32_MAX);
}

// Workgroups and threads of the forward kernel for `rows` query rows per head: the tile
// sdpa::fwd_groups picks for this problem (dense, split-key or packed).
void fwd_tile(int dtype, int64_t D, bool dense, bool split, bool causal, int64_t bh,
              int64_t rows, int64_t keys, int64_t* q_tiles, int64_t* threads) {
  const int groups = sdpa::fwd_groups(dtype, D, dense, causal, bh, rows, keys, split);
  const bool ks = sdpa::fwd_key_split(dtype, D, dense, causal, bh, rows, keys);
  const int64_t bm = dtype != SDPA_F32 ? (ks ? 128 : 128 * groups) : sdpa::kBlockMF32;
  *q_tiles = (rows + bm - 1) / bm;
  *threads = dtype != SDPA_F32 ? (ks ? 512 : 256 * groups) : sdpa::kThreadsF32;
}

// One tensor's `rank` strides as canonical (b, h, row, col) strides: rank 3 [N,L,*] is
// [1,N,L,*] with batch stride 0.  No stride may be negative; the innermost must be 1.
int canon_strides(int rank, const int64_t* s, int64_t out[4]) {
  if (rank == 4) {
    for (int a = 0; a < 4; ++a) out[a] = s[a];
  } else {
    out[0] = 0;
    out[1] = s[0];
    out[2] = s[1];
    out[3] = s[2];
  }
  for (int a = 0; a < 4; ++a)
    if (out[a] < 0) return SDPA_ERR_STRIDE;
  if (out[3] != 1) return SDPA_ERR_STRIDE;
  return SDPA_OK;
}

// The backward's checks of the sizes, head dim (its kernels take 32, 64, 96 and 128) and
// scale.
// The two backward launches (dq, then dk/dv) of `heads` heads with at most `rows` query and
// `keys` key rows each fit HIP's grid limits: the tiled 16-bit kernels, or the row-by-row
// kernels (fp32 inputs, D = 256) with one wave per row.
bool bwd_grids_fit(int dtype, int64_t D, int64_t heads, int64_t rows, int64_t keys) {
  if (heads == 0) return true;
  const bool gen = sdpa::bwd_generic(dtype, D);
  const int64_t bq = gen ? sdpa::kBwdGenRows : sdpa::kBwdBlockQ;
  const int64_t bk = gen ? sdpa::kBwdGenRows : sdpa::kBwdBlockK;
  const int64_t tq = (rows + bq - 1) / bq, tk = (keys + bk - 1) / bk;
  return tq <= kMaxDim / heads && tk <= kMaxDim / heads &&
         launch_fits(heads * tq, gen ? sdpa::kThreadsBwdGen : sdpa::kThreadsBwdQ) &&
         launch_fits(heads * tk, gen ? sdpa::kThreadsBwdGen : sdpa::kThreadsBwdK);
}

int check_sizes(int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D, float scale) {
  if (rank != 3 && rank != 4) return SDPA_ERR_RANK;
  if (rank == 3 && B != 1) return SDPA_ERR_RANK;
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0) return SDPA_ERR_SHAPE;
  if (Lq > kMaxDim || Lk > kMaxDim || B > kMaxDim || H > kMaxDim) return SDPA_ERR_SHAPE;
  if (B != 0 && H > kMaxDim / B) return SDPA_ERR_SHAPE;
  if (!sdpa::bwd_head_dim_ok(D)) return SDPA_ERR_HEAD_DIM;
  if (!isfinite(scale)) return SDPA_ERR_SCALE;
  return SDPA_OK;
}

// Validate the arguments and build the canonical (b, h, row, col) problem.
int normalise(const void* q, const void* k, const void* v, const void* out, const float* lse,
              int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
              const int64_t* strides, float scale, int is_causal, const uint8_t* mask,
              int dtype, sdpa::Problem* p) {
  if (rank != 3 && rank != 4) return SDPA_ERR_RANK;
  if (rank == 3 && B != 1) return SDPA_ERR_RANK;
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0) return SDPA_ERR_SHAPE;
  if (Lq > kMaxDim || Lk > kMaxDim || B > kMaxDim || H > kMaxDim) return SDPA_ERR_SHAPE;
  if (B != 0 && H > kMaxDim / B) return SDPA_ERR_SHAPE;
  if (!sdpa::fwd_head_dim_ok(D)) return SDPA_ERR_HEAD_DIM;
  if (dtype != SDPA_F32 && dtype != SDPA_BF16 && dtype != SDPA_F16) return SDPA_ERR_DTYPE;
  if (!strides) return SDPA_ERR_NULL;
  if (!isfinite(scale)) return SDPA_ERR_SCALE;
  if (is_causal < SDPA_CAUSAL_NONE || is_causal > SDPA_CAUSAL_BOTTOM_RIGHT) return SDPA_ERR_CAUSAL;

  const int64_t bh = B * H;
  int64_t q_tiles, threads;
  fwd_tile(dtype, D, true, false, is_causal != SDPA_CAUSAL_NONE, bh, Lq, Lk, &q_tiles, &threads);
  if (bh != 0 && (q_tiles > kMaxDim / bh || !launch_fits(bh * q_tiles, threads)))
    return SDPA_ERR_SHAPE;  // grid size
  const bool any_rows = bh * Lq != 0;
  const bool reads_kv = any_rows && Lk != 0;

  // strides: q, k, v, out, mask; each `rank` entries in its own axis order.
  int64_t s4[5][4];
  for (int t = 0; t < 5; ++t) {
    const int64_t* s = strides + t * rank;
    if (t == 4 && !mask) {
      s4[t][0] = s4[t][1] = s4[t][2] = s4[t][3] = 0;
      continue;
    }
    const int st = canon_strides(rank, s, s4[t]);
    if (st != SDPA_OK) return st;
  }

  if (any_rows && (!q || !out)) return SDPA_ERR_NULL;
  if (reads_kv && (!k || !v)) return SDPA_ERR_NULL;

  const int64_t esize = dtype == SDPA_F32 ? 4 : 2;
  const void* bases[4] = {q, k, v, out};
  for (int t = 0; t < 4; ++t) {
    const bool used = (t == 1 || t == 2) ? reads_kv : any_rows;
    if (!used) continue;
    if (!aligned(bases[t], 16)) return SDPA_ERR_ALIGN;
    for (int a = 0; a < 3; ++a)
      if ((s4[t][a] * esize) % 16 != 0) return SDPA_ERR_ALIGN;
  }
  if (lse && !aligned(lse, 4)) return SDPA_ERR_ALIGN;
  // K and V rows are addressed with 32-bit byte offsets from the head's base: the rows of
  // one head plus one tile of overrun must span less than 2 GiB.
  if (reads_kv)
    for (int t = 1; t <= 2; ++t)
      if (s4[t][2] > kMaxDim / esize / (Lk + sdpa::block_n(dtype))) return SDPA_ERR_SHAPE;

  if (p) {
    p->q = q;
    p->k = k;
    p->v = v;
    p->out = const_cast<void*>(out);
    p->lse = const_cast<float*>(lse);
    p->mask = mask;
    p->bias = nullptr;
    p->B = B;
    p->H = H;
    p->Lq = Lq;
    p->Lk = Lk;
    p->D = D;
    memcpy(p->sq, s4[0], sizeof p->sq);
    memcpy(p->sk, s4[1], sizeof p->sk);
    memcpy(p->sv, s4[2], sizeof p->sv);
    memcpy(p->so, s4[3], sizeof p->so);
    memcpy(p->sm, s4[4], sizeof p->sm);
    p->scale = scale;
    p->causal = is_causal;
    p->varlen = 0;
    p->cu_q = p->cu_k = nullptr;
    p->nseq = p->max_seqlen_q = 0;
    p->nsplit = p->split_len = 0;
    p->ws_o = p->ws_lse = nullptr;
    p->dtype = dtype;
  }
  return SDPA_OK;
}

// Validate the backward's arguments and build its canonical problem.  Tensor order of
// the strides: q, k, v, out, dout, dq, dk, dv, mask.
int normalise_bwd(const void* q, const void* k, const void* v, const void* out,
                  const void* dout, const float* lse, const void* dq, const void* dk,
                  const void* dv, const float* delta, int rank, int64_t B, int64_t H,
                  int64_t Lq, int64_t Lk, int64_t D, const int64_t* strides, float scale,
                  int is_causal, const uint8_t* mask, int dtype, sdpa::BwdProblem* p) {
  int st = check_sizes(rank, B, H, Lq, Lk, D, scale);
  if (st != SDPA_OK) return st;
  if (dtype != SDPA_F32 && dtype != SDPA_BF16 && dtype != SDPA_F16) return SDPA_ERR_DTYPE;
  if (!strides) return SDPA_ERR_NULL;
  if (is_causal < SDPA_CAUSAL_NONE || is_causal > SDPA_CAUSAL_BOTTOM_RIGHT) return SDPA_ERR_CAUSAL;
  const int64_t bh = B * H;
  if (!bwd_grids_fit(dtype, D, bh, Lq, Lk)) return SDPA_ERR_SHAPE;
  const int64_t esize = dtype == SDPA_F32 ? 4 : 2;
  const bool rows = bh * Lq != 0;  // the dq kernel runs (and reads q, out, dout, lse)
  const bool keys = bh * Lk != 0;  // the dkdv kernel runs (and reads k, v, writes dk, dv)

  enum { Q, K, V, O, DO, DQ, DK, DV, M, NT };
  int64_t s4[NT][4];
  for (int t = 0; t < NT; ++t) {
    if (t == M && !mask) {
      s4[t][0] = s4[t][1] = s4[t][2] = s4[t][3] = 0;
      continue;
    }
    st = canon_strides(rank, strides + t * rank, s4[t]);
    if (st != SDPA_OK) return st;
  }
  // Every tensor is read or written when either kernel runs (q and dout are also staged
  // by the dkdv kernel, k and v by the dq kernel), except that with Lk == 0 nothing of
  // k, v, dk, dv exists and with Lq == 0 nothing of q, out, dout, dq, lse, delta.
  const void* bases[8] = {q, k, v, out, dout, dq, dk, dv};
  for (int t = 0; t < 8; ++t) {
    const bool key_side = t == K || t == V || t == DK || t == DV;
    if (!(key_side ? keys : rows)) continue;
    if (!bases[t]) return SDPA_ERR_NULL;
  }
  if (rows && (!lse || !delta)) return SDPA_ERR_NULL;
  for (int t = 0; t < 8; ++t) {
    const bool key_side = t == K || t == V || t == DK || t == DV;
    if (!(key_side ? keys : rows)) continue;
    if (!aligned(bases[t], 16)) return SDPA_ERR_ALIGN;
    for (int a = 0; a < 3; ++a)
      if ((s4[t][a] * esize) % 16 != 0) return SDPA_ERR_ALIGN;
  }
  if ((lse && !aligned(lse, 4)) || (delta && !aligned(delta, 4))) return SDPA_ERR_ALIGN;
  // Streamed tiles are addressed with 32-bit byte offsets from the head's base: K and V
  // rows (dq kernel) and q and dout rows (dkdv kernel), plus one tile of overrun.
  if (rows && keys) {
    for (int t : {K, V})
      if (s4[t][2] > kMaxDim / 2 / (Lk + sdpa::kBwdStep)) return SDPA_ERR_SHAPE;
    for (int t : {Q, DO})
      if (s4[t][2] > kMaxDim / 2 / (Lq + sdpa::kBwdStep)) return SDPA_ERR_SHAPE;
  }

  if (p) {
    p->q = q;
    p->k = k;
    p->v = v;
    p->out = out;
    p->dout = dout;
    p->lse = lse;
    p->delta = const_cast<float*>(delta);
    p->dq = const_cast<void*>(dq);
    p->dk = const_cast<void*>(dk);
    p->dv = const_cast<void*>(dv);
    p->mask = mask;
    p->B = B;
    p->H = H;
    p->Lq = Lq;
    p->Lk = Lk;
    p->D = D;
    memcpy(p->sq, s4[Q], sizeof p->sq);
    memcpy(p->sk, s4[K], sizeof p->sk);
    memcpy(p->sv, s4[V], sizeof p->sv);
    memcpy(p->so, s4[O], sizeof p->so);
    memcpy(p->sdo, s4[DO], sizeof p->sdo);
    memcpy(p->sdq, s4[DQ], sizeof p->sdq);
    memcpy(p->sdk, s4[DK], sizeof p->sdk);
    memcpy(p->sdv, s4[DV], sizeof p->sdv);
    memcpy(p->sm, s4[M], sizeof p->sm);
    p->bias = nullptr;
    p->cu_q = p->cu_k = nullptr;
    p->nseq = p->max_seqlen_q = p->max_seqlen_k = 0;
    p->scale = scale;
    p->causal = is_causal;
    p->dtype = dtype;
    p->varlen = 0;
  }
  return SDPA_OK;
}

// The backward with an additive mask: sdpa_bwd's validation with the bias in the mask's
// place (same stride rules); fp32, 4-byte aligned.
int normalise_bwd_bias(const void* q, const void* k, const void* v, const void* out,
                       const void* dout, const float* lse, const void* dq, const void* dk,
                       const void* dv, const float* delta, int rank, int64_t B, int64_t H,
                       int64_t Lq, int64_t Lk, int64_t D, const int64_t* strides, float scale,
                       int is_causal, const float* bias, int dtype, sdpa::BwdProblem* p) {
  const int st = normalise_bwd(q, k, v, out, dout, lse, dq, dk, dv, delta, rank, B, H, Lq, Lk,
                               D, strides, scale, is_causal,
                               reinterpret_cast<const uint8_t*>(bias), dtype, p);
  if (st != SDPA_OK) return st;
  if (bias && !aligned(bias, 4)) return SDPA_ERR_ALIGN;
  if (p) {
    p->mask = nullptr;
    p->bias = bias;
  }
  return SDPA_OK;
}

// The backward of packed sequences: tensors [tokens, H, D] with (token, head, dim) strides
// for q, k, v, out, dout, dq, dk, dv; lse and delta [H, total_q].
int normalise_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                         const void* dout, const float* lse, const void* dq, const void* dk,
                         const void* dv, const float* delta, const int32_t* cu_q,
                         const int32_t* cu_k, int64_t nseq, int64_t max_seqlen_q,
                         int64_t max_seqlen_k, int64_t total_q, int64_t total_k, int64_t H,
                         int64_t D, const int64_t* strides, float scale, int causal, int dtype,
                         sdpa::BwdProblem* p) {
  if (nseq < 0 || H < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return SDPA_ERR_SHAPE;
  if (nseq >= kMaxDim || H > kMaxDim || total_q > kMaxDim || total_k > kMaxDim)
    return SDPA_ERR_SHAPE;
  if (nseq != 0 && H > kMaxDim / nseq) return SDPA_ERR_SHAPE;
  if (max_seqlen_q > total_q || max_seqlen_k > total_k) return SDPA_ERR_SHAPE;
  if (H != 0 && total_q > kMaxDim / H) return SDPA_ERR_SHAPE;  // lse / delta [H, total_q]
  if (!sdpa::bwd_head_dim_ok(D)) return SDPA_ERR_HEAD_DIM;
  if (dtype != SDPA_F32 && dtype != SDPA_BF16 && dtype != SDPA_F16) return SDPA_ERR_DTYPE;
  if (!strides) return SDPA_ERR_NULL;
  if (!isfinite(scale)) return SDPA_ERR_SCALE;
  if (causal < SDPA_CAUSAL_NONE || causal > SDPA_CAUSAL_BOTTOM_RIGHT) return SDPA_ERR_CAUSAL;
  const int64_t heads = nseq * H;
  if (!bwd_grids_fit(dtype, D, heads, max_seqlen_q, max_seqlen_k)) return SDPA_ERR_SHAPE;
  const int64_t esize = dtype == SDPA_F32 ? 4 : 2;
  // the dq kernel runs when some sequence may have query rows, the dkdv kernel when some
  // may have keys; each reads the other side's rows too
  const bool rows = heads != 0 && max_seqlen_q != 0;
  const bool keys = heads != 0 && max_seqlen_k != 0;
  const bool any = rows || keys;

  enum { Q, K, V, O, DO, DQ, DK, DV, NT };
  int64_t s4[NT][4];
  for (int t = 0; t < NT; ++t) {
    const int64_t* st = strides + 3 * t;
    s4[t][0] = 0;
    s4[t][1] = st[1];
    s4[t][2] = st[0];
    s4[t][3] = st[2];
    for (int a = 0; a < 4; ++a)
      if (s4[t][a] < 0) return SDPA_ERR_STRIDE;
    if (s4[t][3] != 1) return SDPA_ERR_STRIDE;
  }
  if (any && (!cu_q || !cu_k)) return SDPA_ERR_NULL;
  const void* bases[8] = {q, k, v, out, dout, dq, dk, dv};
  for (int t = 0; t < 8; ++t) {
    const bool key_side = t == K || t == V || t == DK || t == DV;
    if (!any || (key_side ? total_k : total_q) == 0) continue;
    if (!bases[t]) return SDPA_ERR_NULL;
    if (!aligned(bases[t], 16)) return SDPA_ERR_ALIGN;
    for (int a = 1; a < 3; ++a)
      if ((s4[t][a] * esize) % 16 != 0) return SDPA_ERR_ALIGN;
  }
  if (any && total_q != 0 && (!lse || !delta)) return SDPA_ERR_NULL;
  if ((lse && !aligned(lse, 4)) || (delta && !aligned(delta, 4)) ||
      (cu_q && !aligned(cu_q, 4)) || (cu_k && !aligned(cu_k, 4)))
    return SDPA_ERR_ALIGN;
  // a sequence's streamed rows are addressed with 32-bit byte offsets from its first row
  if (any) {
    for (int t : {K, V})
      if (s4[t][2] > kMaxDim / 2 / (total_k + sdpa::kBwdStep)) return SDPA_ERR_SHAPE;
    for (int t : {Q, DO})
      if (s4[t][2] > kMaxDim / 2 / (total_q + sdpa::kBwdStep)) return SDPA_ERR_SHAPE;
  }

  if (p) {
    p->q = q;
    p->k = k;
    p->v = v;
    p->out = out;
    p->dout = dout;
    p->lse = lse;
    p->delta = const_cast<float*>(delta);
    p->dq = const_cast<void*>(dq);
    p->dk = const_cast<void*>(dk);
    p->dv = const_cast<void*>(dv);
    p->mask = nullptr;
    p->bias = nullptr;
    p->cu_q = cu_q;
    p->cu_k = cu_k;
    p->B = 1;
    p->H = H;
    p->Lq = total_q;
    p->Lk = total_k;
    p->D = D;
    p->nseq = nseq;
    p->max_seqlen_q = max_seqlen_q;
    p->max_seqlen_k = max_seqlen_k;
    memcpy(p->sq, s4[Q], sizeof p->sq);
    memcpy(p->sk, s4[K], sizeof p->sk);
    memcpy(p->sv, s4[V], sizeof p->sv);
    memcpy(p->so, s4[O], sizeof p->so);
    memcpy(p->sdo, s4[DO], sizeof p->sdo);
    memcpy(p->sdq, s4[DQ], sizeof p->sdq);
    memcpy(p->sdk, s4[DK], sizeof p->sdk);
    memcpy(p->sdv, s4[DV], sizeof p->sdv);
    memset(p->sm, 0, sizeof p->sm);
    p->scale = scale;
    p->causal = causal;
    p->dtype = dtype;
    p->varlen = 1;
  }
  return SDPA_OK;
}

// Validate a packed variable-length forward and build its problem.  Tensors are
// [tokens, H, D]; strides holds (token, head, dim) for q, k, v, out.
int normalise_varlen(const void* q, const void* k, const void* v, const void* out,
                     const float* lse, const int32_t* cu_q, const int32_t* cu_k, int64_t nseq,
                     int64_t max_seqlen_q, int64_t total_q, int64_t total_k, int64_t H,
                     int64_t D, const int64_t* strides, float scale, int causal, int dtype,
                     sdpa::Problem* p) {
  if (nseq < 0 || H < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0) return SDPA_ERR_SHAPE;
  if (nseq >= kMaxDim || H > kMaxDim || total_q > kMaxDim || total_k > kMaxDim)
    return SDPA_ERR_SHAPE;
  if (max_seqlen_q > total_q) return SDPA_ERR_SHAPE;
  if (!sdpa::fwd_head_dim_ok(D)) return SDPA_ERR_HEAD_DIM;
  if (dtype != SDPA_F32 && dtype != SDPA_BF16 && dtype != SDPA_F16) return SDPA_ERR_DTYPE;
  if (!strides) return SDPA_ERR_NULL;
  if (!isfinite(scale)) return SDPA_ERR_SCALE;
  if (causal < SDPA_CAUSAL_NONE || causal > SDPA_CAUSAL_BOTTOM_RIGHT) return SDPA_ERR_CAUSAL;
  const int64_t heads = nseq * H;
  int64_t q_tiles, threads;
  fwd_tile(dtype, D, false, false, causal != SDPA_CAUSAL_NONE, heads, max_seqlen_q, 0, &q_tiles,
           &threads);
  if (heads != 0 && (q_tiles > kMaxDim / heads || !launch_fits(heads * q_tiles, threads)))
    return SDPA_ERR_SHAPE;  // grid size
  const bool any_rows = heads != 0 && total_q != 0 && max_seqlen_q != 0;

  int64_t s4[4][4];
  for (int t = 0; t < 4; ++t) {
    const int64_t* st = strides + 3 * t;
    s4[t][0] = 0;
    s4[t][1] = st[1];
    s4[t][2] = st[0];
    s4[t][3] = st[2];
    for (int a = 0; a < 4; ++a)
      if (s4[t][a] < 0) return SDPA_ERR_STRIDE;
    if (s4[t][3] != 1) return SDPA_ERR_STRIDE;
  }
  if (any_rows && (!q || !out || !cu_q || !cu_k)) return SDPA_ERR_NULL;
  if (any_rows && total_k != 0 && (!k || !v)) return SDPA_ERR_NULL;
  const int64_t esize = dtype == SDPA_F32 ? 4 : 2;
  const void* bases[4] = {q, k, v, out};
  for (int t = 0; t < 4; ++t) {
    if (!any_rows || (!bases[t] && (t == 1 || t == 2) && total_k == 0)) continue;
    if (!aligned(bases[t], 16)) return SDPA_ERR_ALIGN;
    for (int a = 1; a < 3; ++a)
      if ((s4[t][a] * esize) % 16 != 0) return SDPA_ERR_ALIGN;
  }
  if ((lse && !aligned(lse, 4)) || (cu_q && !aligned(cu_q, 4)) || (cu_k && !aligned(cu_k, 4)))
    return SDPA_ERR_ALIGN;
  // a sequence's K/V rows are addressed with 32-bit byte offsets from its first row
  if (any_rows)
    for (int t = 1; t <= 2; ++t)
      if (s4[t][2] > kMaxDim / esize / (total_k + sdpa::block_n(dtype))) return SDPA_ERR_SHAPE;

  if (p) {
    p->q = q;
    p->k = k;
    p->v = v;
    p->out = const_cast<void*>(out);
    p->lse = const_cast<float*>(lse);
    p->mask = nullptr;
    p->bias = nullptr;
    p->cu_q = cu_q;
    p->cu_k = cu_k;
    p->B = 1;
    p->H = H;
    p->Lq = total_q;
    p->Lk = total_k;
    p->D = D;
    p->nseq = nseq;
    p->max_seqlen_q = max_seqlen_q;
    memcpy(p->sq, s4[0], sizeof p->sq);
    memcpy(p->sk, s4[1], sizeof p->sk);
    memcpy(p->sv, s4[2], sizeof p->sv);
    memcpy(p->so, s4[3], sizeof p->so);
    memset(p->sm, 0, sizeof p->sm);
    p->scale = scale;
    p->causal = causal;
    p->varlen = 1;
    p->nsplit = p->split_len = 0;
    p->ws_o = p->ws_lse = nullptr;
    p->dtype = dtype;
  }
  return SDPA_OK;
}

// Split keys: the dense forward's validation (4 tensors, no mask), then the split plan and
// the workspace: [nsplit][B*H][Lq][D] partial outputs followed by [nsplit][B*H][Lq] lse,
// fp32.  Returns the bytes needed through *need (also on SDPA_ERR_WORKSPACE).
constexpr int64_t kMaxSplits = 1024;

int splitkv_sizes(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D, int64_t num_splits,
                  int dtype, int64_t* nsplit, int64_t* split_len, int64_t* need) {
  if (num_splits < 0 || num_splits > kMaxSplits) return SDPA_ERR_SHAPE;
  const int64_t bh = B * H;
  const int64_t bm = sdpa::block_m(dtype, int(D));
  sdpa::splitkv_plan(bh, (Lq + bm - 1) / bm, Lk, num_splits, nsplit, split_len);
  int64_t q_tiles, threads;
  fwd_tile(dtype, D, false, true, false, bh, Lq, Lk, &q_tiles, &threads);
  // the chunk launch, and the merge launch of one 64-lane wave per query row
  if (bh != 0 && (q_tiles > kMaxDim / bh / *nsplit || !launch_fits(bh * q_tiles * *nsplit, threads) ||
                  !launch_fits((bh * Lq + 3) / 4, 256)))
    return SDPA_ERR_SHAPE;  // grid sizes
  *need = *nsplit * bh * Lq * (D + 1) * 4;
  return SDPA_OK;
}

int normalise_splitkv(const void* q, const void* k, const void* v, const void* out,
                      const float* lse, int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                      int64_t D, const int64_t* strides, float scale, int is_causal,
                      int64_t num_splits, const void* workspace, int64_t workspace_bytes,
                      int dtype, sdpa::Problem* p) {
  if (!strides) return SDPA_ERR_NULL;
  if (rank != 3 && rank != 4) return SDPA_ERR_RANK;
  int64_t s5[20] = {0};
  for (int i = 0; i < 4 * rank; ++i) s5[i] = strides[i];
  int st = normalise(q, k, v, out, lse, rank, B, H, Lq, Lk, D, s5, scale, is_causal, nullptr,
                     dtype, p);
  if (st != SDPA_OK) return st;
  int64_t nsplit, split_len, need;
  st = splitkv_sizes(B, H, Lq, Lk, D, num_splits, dtype, &nsplit, &split_len, &need);
  if (st != SDPA_OK) return st;
  if (B * H * Lq != 0) {
    if (!workspace) return SDPA_ERR_NULL;
    if (!aligned(workspace, 16)) return SDPA_ERR_ALIGN;
    if (workspace_bytes < need) return SDPA_ERR_WORKSPACE;
  }
  if (p) {
    p->nsplit = nsplit;
    p->split_len = split_len;
    p->ws_o = static_cast<float*>(const_cast<void*>(workspace));
    p->ws_lse = p->ws_o ? p->ws_o + nsplit * B * H * Lq * D : nullptr;
  }
  return SDPA_OK;
}

// Additive mask: the dense forward's validation with the bias in the mask's place (its
// strides follow the mask's rules: innermost 1, none negative, 0 to broadcast); fp32,
// 4-byte aligned.
int normalise_bias(const void* q, const void* k, const void* v, const void* out,
                   const float* lse, int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                   int64_t D, const int64_t* strides, float scale, int is_causal,
                   const float* bias, int dtype, sdpa::Problem* p) {
  const int st = normalise(q, k, v, out, lse, rank, B, H, Lq, Lk, D, strides, scale, is_causal,
                           reinterpret_cast<const uint8_t*>(bias), dtype, p);
  if (st != SDPA_OK) return st;
  if (bias && !aligned(bias, 4)) return SDPA_ERR_ALIGN;
  if (p) {
    p->mask = nullptr;
    p->bias = bias;
  }
  return SDPA_OK;
}

// The device `stream` runs on (the current device for the null stream); false on failure.
bool stream_device(hipStream_t stream, int* dev) {
  *dev = 0;
  if (stream) return hipStreamGetDevice(stream, dev) == hipSuccess;
  return hipGetDevice(dev) == hipSuccess;
}

// The code object holds gfx950 machine code only; refuse other devices up front.
// Cached per device id (the only global state of the library besides the static split-key
// workspace of sdpa_fwd_splitkv_noalloc).
bool device_is_gfx950(hipStream_t stream) {
  int dev = 0;
  if (!stream_device(stream, &dev)) return false;
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static signed char verdict[kMaxDevices];  // 0 unknown, 1 gfx950, -1 other
  if (dev < 0 || dev >= kMaxDevices) return false;
  std::lock_guard<std::mutex> lock(mu);
  if (verdict[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return false;
    verdict[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
  }
  return verdict[dev] == 1;
}

}  // namespace

extern "C" {

int sdpa_check(const void* q, const void* k, const void* v, const void* out, const float* lse,
               int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
               const int64_t* strides, float scale, int is_causal, const uint8_t* mask,
               int dtype) {
  return normalise(q, k, v, out, lse, rank, B, H, Lq, Lk, D, strides, scale, is_causal, mask,
                   dtype, nullptr);
}

int sdpa_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int rank,
             int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D, const int64_t* strides,
             float scale, int is_causal, const uint8_t* mask, int dtype, void* stream) {
  sdpa::Problem p;
  const int st = normalise(q, k, v, out, lse, rank, B, H, Lq, Lk, D, strides, scale, is_causal,
                           mask, dtype, &p);
  if (st != SDPA_OK) return st;
  if (p.B * p.H * p.Lq == 0) return SDPA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!device_is_gfx950(s)) return SDPA_ERR_DEVICE;
  return sdpa::launch_fwd(p, s) == hipSuccess ? SDPA_OK : SDPA_ERR_DEVICE;
}

int sdpa_fwd_bias_check(const void* q, const void* k, const void* v, const void* out,
                        const float* lse, int rank, int64_t B, int64_t H, int64_t Lq,
                        int64_t Lk, int64_t D, const int64_t* strides, float scale,
                        int is_causal, const float* bias, int dtype) {
  return normalise_bias(q, k, v, out, lse, rank, B, H, Lq, Lk, D, strides, scale, is_causal,
                        bias, dtype, nullptr);
}

int sdpa_fwd_bias(const void* q, const void* k, const void* v, void* out, float* lse, int rank,
                  int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                  const int64_t* strides, float scale, int is_causal, const float* bias,
                  int dtype, void* stream) {
  sdpa::Problem p;
  const int st = normalise_bias(q, k, v, out, lse, rank, B, H, Lq, Lk, D, strides, scale,
                                is_causal, bias, dtype, &p);
  if (st != SDPA_OK) return st;
  if (p.B * p.H * p.Lq == 0) return SDPA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!device_is_gfx950(s)) return SDPA_ERR_DEVICE;
  return sdpa::launch_fwd(p, s) == hipSuccess ? SDPA_OK : SDPA_ERR_DEVICE;
}

int64_t sdpa_fwd_splitkv_workspace(int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                                   int64_t num_splits, int dtype) {
  if (B < 0 || H < 0 || Lq < 0 || Lk < 0 || B > kMaxDim || H > kMaxDim || Lq > kMaxDim ||
      Lk > kMaxDim || (B != 0 && H > kMaxDim / B))
    return -SDPA_ERR_SHAPE;
  if (!sdpa::fwd_head_dim_ok(D)) return -SDPA_ERR_HEAD_DIM;
  if (dtype != SDPA_F32 && dtype != SDPA_BF16 && dtype != SDPA_F16) return -SDPA_ERR_DTYPE;
  int64_t nsplit, split_len, need;
  const int st = splitkv_sizes(B, H, Lq, Lk, D, num_splits, dtype, &nsplit, &split_len, &need);
  return st != SDPA_OK ? -st : need;
}

int sdpa_fwd_splitkv_check(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, int rank, int64_t B, int64_t H, int64_t Lq,
                           int64_t Lk, int64_t D, const int64_t* strides, float scale,
                           int is_causal, int64_t num_splits, const void* workspace,
                           int64_t workspace_bytes, int dtype) {
  return normalise_splitkv(q, k, v, out, lse, rank, B, H, Lq, Lk, D, strides, scale, is_causal,
                           num_splits, workspace, workspace_bytes, dtype, nullptr);
}

int sdpa_fwd_splitkv(const void* q, const void* k, const void* v, void* out, float* lse,
                     int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                     const int64_t* strides, float scale, int is_causal, int64_t num_splits,
                     void* workspace, int64_t workspace_bytes, int dtype, void* stream) {
  sdpa::Problem p;
  const int st = normalise_splitkv(q, k, v, out, lse, rank, B, H, Lq, Lk, D, strides, scale,
                                   is_causal, num_splits, workspace, workspace_bytes, dtype, &p);
  if (st != SDPA_OK) return st;
  if (p.B * p.H * p.Lq == 0) return SDPA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!device_is_gfx950(s)) return SDPA_ERR_DEVICE;
  return sdpa::launch_fwd(p, s) == hipSuccess ? SDPA_OK : SDPA_ERR_DEVICE;
}

int sdpa_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* out, float* lse,
                             int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D,
                             const int64_t* strides, float scale, int is_causal,
                             int64_t num_splits, int dtype, void* stream) {
  // sdpa_fwd_splitkv's validation with a stand-in workspace that is large enough, then the
  // bytes this problem needs against the static workspace
  alignas(16) static const char stand_in[16] = {0};
  sdpa::Problem p;
  int st = normalise_splitkv(q, k, v, out, lse, rank, B, H, Lq, Lk, D, strides, scale, is_causal,
                             num_splits, stand_in, INT64_MAX, dtype, &p);
  if (st != SDPA_OK) return st;
  int64_t nsplit, split_len, need;
  st = splitkv_sizes(B, H, Lq, Lk, D, num_splits, dtype, &nsplit, &split_len, &need);
  if (st != SDPA_OK) return st;
  if (need > sdpa::kStaticWorkspaceBytes) return SDPA_ERR_STATIC_WORKSPACE;
  if (p.B * p.H * p.Lq == 0) return SDPA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!device_is_gfx950(s)) return SDPA_ERR_DEVICE;
  int dev = 0;
  void* ws = nullptr;
  if (!stream_device(s, &dev) || sdpa::static_workspace(dev, &ws) != hipSuccess)
    return SDPA_ERR_DEVICE;
  p.ws_o = static_cast<float*>(ws);
  p.ws_lse = p.ws_o + p.nsplit * p.B * p.H * p.Lq * p.D;
  return sdpa::launch_fwd(p, s) == hipSuccess ? SDPA_OK : SDPA_ERR_DEVICE;
}

int sdpa_fwd_varlen_check(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, int64_t nseq, int64_t max_seqlen_q,
                          int64_t total_q, int64_t total_k, int64_t H, int64_t D,
                          const int64_t* strides, float scale, int causal, int dtype) {
  return normalise_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, nseq, max_seqlen_q,
                          total_q, total_k, H, D, strides, scale, causal, dtype, nullptr);
}

int sdpa_fwd_varlen(const void* q, const void* k, const void* v, void* out, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int64_t nseq,
                    int64_t max_seqlen_q, int64_t total_q, int64_t total_k, int64_t H, int64_t D,
                    const int64_t* strides, float scale, int causal, int dtype, void* stream) {
  sdpa::Problem p;
  const int st = normalise_varlen(q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, nseq,
                                  max_seqlen_q, total_q, total_k, H, D, strides, scale, causal,
                                  dtype, &p);
  if (st != SDPA_OK) return st;
  if (p.nseq * p.H * p.Lq * p.max_seqlen_q == 0) return SDPA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!device_is_gfx950(s)) return SDPA_ERR_DEVICE;
  return sdpa::launch_fwd(p, s) == hipSuccess ? SDPA_OK : SDPA_ERR_DEVICE;
}

int sdpa_bwd_check(const void* q, const void* k, const void* v, const void* out,
                   const void* dout, const float* lse, const void* dq, const void* dk,
                   const void* dv, const float* delta, int rank, int64_t B, int64_t H,
                   int64_t Lq, int64_t Lk, int64_t D, const int64_t* strides, float scale,
                   int is_causal, const uint8_t* mask, int dtype) {
  return normalise_bwd(q, k, v, out, dout, lse, dq, dk, dv, delta, rank, B, H, Lq, Lk, D,
                       strides, scale, is_causal, mask, dtype, nullptr);
}

int sdpa_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, float* delta, int rank, int64_t B,
             int64_t H, int64_t Lq, int64_t Lk, int64_t D, const int64_t* strides, float scale,
             int is_causal, const uint8_t* mask, int dtype, void* stream) {
  sdpa::BwdProblem p;
  const int st = normalise_bwd(q, k, v, out, dout, lse, dq, dk, dv, delta, rank, B, H, Lq, Lk,
                               D, strides, scale, is_causal, mask, dtype, &p);
  if (st != SDPA_OK) return st;
  if (p.B * p.H * (p.Lq + p.Lk) == 0) return SDPA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!device_is_gfx950(s)) return SDPA_ERR_DEVICE;
  return sdpa::launch_bwd(p, s) == hipSuccess ? SDPA_OK : SDPA_ERR_DEVICE;
}

int sdpa_bwd_bias_check(const void* q, const void* k, const void* v, const void* out,
                        const void* dout, const float* lse, const void* dq, const void* dk,
                        const void* dv, const float* delta, int rank, int64_t B, int64_t H,
                        int64_t Lq, int64_t Lk, int64_t D, const int64_t* strides, float scale,
                        int is_causal, const float* bias, int dtype) {
  return normalise_bwd_bias(q, k, v, out, dout, lse, dq, dk, dv, delta, rank, B, H, Lq, Lk, D,
                            strides, scale, is_causal, bias, dtype, nullptr);
}

int sdpa_bwd_bias(const void* q, const void* k, const void* v, const void* out,
                  const void* dout, const float* lse, void* dq, void* dk, void* dv,
                  float* delta, int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk,
                  int64_t D, const int64_t* strides, float scale, int is_causal,
                  const float* bias, int dtype, void* stream) {
  sdpa::BwdProblem p;
  const int st = normalise_bwd_bias(q, k, v, out, dout, lse, dq, dk, dv, delta, rank, B, H, Lq,
                                    Lk, D, strides, scale, is_causal, bias, dtype, &p);
  if (st != SDPA_OK) return st;
  if (p.B * p.H * (p.Lq + p.Lk) == 0) return SDPA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!device_is_gfx950(s)) return SDPA_ERR_DEVICE;
  return sdpa::launch_bwd(p, s) == hipSuccess ? SDPA_OK : SDPA_ERR_DEVICE;
}

int sdpa_bwd_varlen_check(const void* q, const void* k, const void* v, const void* out,
                          const void* dout, const float* lse, const void* dq, const void* dk,
                          const void* dv, const float* delta, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, int64_t nseq, int64_t max_seqlen_q,
                          int64_t max_seqlen_k, int64_t total_q, int64_t total_k, int64_t H,
                          int64_t D, const int64_t* strides, float scale, int causal,
                          int dtype) {
  return normalise_bwd_varlen(q, k, v, out, dout, lse, dq, dk, dv, delta, cu_seqlens_q,
                              cu_seqlens_k, nseq, max_seqlen_q, max_seqlen_k, total_q, total_k,
                              H, D, strides, scale, causal, dtype, nullptr);
}

int sdpa_bwd_varlen(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv,
                    float* delta, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                    int64_t nseq, int64_t max_seqlen_q, int64_t max_seqlen_k, int64_t total_q,
                    int64_t total_k, int64_t H, int64_t D, const int64_t* strides, float scale,
                    int causal, int dtype, void* stream) {
  sdpa::BwdProblem p;
  const int st = normalise_bwd_varlen(q, k, v, out, dout, lse, dq, dk, dv, delta, cu_seqlens_q,
                                      cu_seqlens_k, nseq, max_seqlen_q, max_seqlen_k, total_q,
                                      total_k, H, D, strides, scale, causal, dtype, &p);
  if (st != SDPA_OK) return st;
  if (p.nseq * p.H == 0 || p.max_seqlen_q + p.max_seqlen_k == 0) return SDPA_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (!device_is_gfx950(s)) return SDPA_ERR_DEVICE;
  return sdpa::launch_bwd(p, s) == hipSuccess ? SDPA_OK : SDPA_ERR_DEVICE;
}

const char* sdpa_strerror(int status) {
  switch (status) {
    case SDPA_OK: return "success";
    case SDPA_ERR_NULL: return "a required pointer is NULL";
    case SDPA_ERR_RANK: return "rank must be 3 or 4 (rank 3 requires B == 1)";
    case SDPA_ERR_SHAPE:
      return "negative size, a size beyond the supported maximum, or one head's k/v rows "
             "spanning 2 GiB or more";
    case SDPA_ERR_HEAD_DIM:
      return "head dim D must be 32, 64, 96, 128 or 256 (the backward: 32, 64, 96 or 128)";
    case SDPA_ERR_DTYPE:
      return "dtype must be SDPA_F32, SDPA_BF16 or SDPA_F16 (the backward: SDPA_BF16 or SDPA_F16)";
    case SDPA_ERR_STRIDE: return "innermost strides must be 1 and no stride may be negative";
    case SDPA_ERR_ALIGN:
      return "q/k/v/out base pointers and outer strides must be 16-byte aligned, lse 4-byte";
    case SDPA_ERR_SCALE: return "scale must be finite";
    case SDPA_ERR_DEVICE: return "device is not gfx950 or the kernel launch failed";
    case SDPA_ERR_CAUSAL:
      return "causal mode must be 0 (none), 1 (top-left) or 2 (bottom-right)";
    case SDPA_ERR_WORKSPACE:
      return "workspace smaller than sdpa_fwd_splitkv_workspace() bytes";
    case SDPA_ERR_STATIC_WORKSPACE:
      return "the split-key workspace this problem needs exceeds the 16 MiB static workspace "
             "of sdpa_fwd_splitkv_noalloc";
    default: return "unknown sdpa status";
  }
}

int sdpa_plan(int rank, int64_t B, int64_t H, int64_t Lq, int64_t Lk, int64_t D, int is_causal,
              int dtype, sdpa_plan_t* plan) {
  if (!plan) return SDPA_ERR_NULL;
  // Validate the sizes only: fake, aligned, non-NULL pointers and unit-innermost strides.
  int64_t strides[20];
  for (int t = 0; t < 5; ++t)
    for (int a = 0; a < rank && a < 4; ++a) strides[t * rank + a] = (a == rank - 1) ? 1 : 0;
  static const float dummy[4] __attribute__((aligned(16))) = {0, 0, 0, 0};
  const int st = normalise(dummy, dummy, dummy, dummy, nullptr, rank, B, H, Lq, Lk, D, strides,
                           1.0f, is_causal, nullptr, dtype, nullptr);
  if (st != SDPA_OK) return st;
  // small 16-bit problems take the one-group tile, or the key split (two streams of tiles)
  const bool causal = is_causal != SDPA_CAUSAL_NONE;
  const bool ks = sdpa::fwd_key_split(dtype, D, true, causal, B * H, Lq, Lk);
  int64_t q_tiles = 0, threads = 0;
  fwd_tile(dtype, D, true, false, causal, B * H, Lq, Lk, &q_tiles, &threads);
  plan->block_m = dtype != SDPA_F32
                      ? (ks ? 128 : 128 * sdpa::fwd_groups(dtype, D, true, causal, B * H, Lq, Lk, false))
                      : sdpa::block_m(dtype, int(D));
  plan->block_n = sdpa::block_n(dtype);
  plan->threads = threads;
  plan->q_tiles = q_tiles;
  plan->bh = B * H;
  plan->items = plan->bh * plan->q_tiles;
  plan->lds_bytes = dtype == SDPA_F32 ? sdpa::lds_bytes_f32(int(D))
                                      : (ks ? 2 : 1) * sdpa::lds_bytes_bf16(int(D));
  plan->is_causal = is_causal ? 1 : 0;
  return SDPA_OK;
}

int sdpa_plan_item(const sdpa_plan_t* plan, int64_t block, int64_t* bh, int64_t* q_tile) {
  if (!plan || !bh || !q_tile) return SDPA_ERR_NULL;
  if (block < 0 || block >= plan->items) return SDPA_ERR_SHAPE;
  sdpa::decode_item(block, plan->bh, plan->q_tiles, plan->is_causal != 0, bh, q_tile);
  return SDPA_OK;
}

}  // extern "C"
