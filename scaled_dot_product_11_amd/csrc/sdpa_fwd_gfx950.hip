// sdpa_fwd_gfx950.hip -- fused scaled-dot-product-attention forward for MI355X (gfx950).
//
// One kernel computes, for every query row i of every head,
//   out[i,:] = sum_j softmax_j(scale * q_i.k_j over the visible keys) v_j     and
//   lse[i]   = log sum_{visible j} exp(scale * q_i.k_j),
// the five primitive steps of "Profiling in PyTorch (part 3): attention" (naive causal
// attention: q.k^T, scale, masked positions to -inf, softmax, attn.v) fused as that
// article's flash and efficient backends fuse them: the [L, L] score matrix never leaves
// the chip, key/value tiles are streamed with an online softmax, causal tiles above the
// diagonal are never computed, and a row with no visible key yields zeros (the math
// backend's safe softmax).
//
// Work decomposition (16-bit and fp32 kernels alike):
//   * a workgroup owns a tile of query rows of one (b, h): 256 rows in 8 waves (bf16, fp16;
//     128 rows in 4 waves at D = 256) or 128 rows in 4 waves (fp32); each wave owns 32 query
//     rows;
//   * lane l serves query row (l % 32) and half h = l / 32 of every key tile, so all
//     per-row softmax state (running max, running sum, rescale factor) is a per-lane
//     scalar;
//   * the scores are computed transposed, S^T = K . Q^T, on 32x32 MFMA tiles: the
//     accumulator of a 32x32 tile gives each lane 16 keys of its own query row;
//   * the output is accumulated transposed, O^T += V^T . P^T, so P^T comes straight from
//     the score registers and each lane again owns its query's column;
//   * K and V tiles of 64 keys are double-buffered through LDS: each tile is loaded from
//     global memory a whole key step before it is written to the other LDS stage;
//   * the output tile of each wave goes through LDS at the end, so that its global stores
//     cover whole rows.
#include <math.h>

#include <mutex>

#include "sdpa_internal.h"

namespace sdpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Kernel arguments: canonical (b, h, row) strides in elements; the innermost stride is 1.
// Packed variable-length problems use the row stride for tokens and the head stride for
// heads; Lq and Lk are then the total token counts and bh_count = sequences * H.
struct Args {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const uint8_t* mask;
  const float* bias;    // additive mask (fp32), addressed with the mask strides
  const int32_t* cu_q;  // variable-length only: sequence s owns query tokens cu_q[s] ..
  const int32_t* cu_k;  // cu_q[s+1]-1 and key tokens cu_k[s] .. cu_k[s+1]-1
  int64_t sq[3], sk[3], sv[3], so[3], sm[3];
  int32_t H, Lq, Lk, q_tiles, bh_count;
  float scale_log2;  // scale * log2(e): scores are kept in base-2 units
  int32_t mask_vec8; // mask rows may be read 8 bytes at a time
  int32_t bias_vec4; // bias rows may be read 16 bytes at a time
  int32_t bottom_right;  // causal alignment: key j visible iff j <= i + (Lk - Lq)
  float* ws_o;           // split keys only: normalised partial outputs [split][bh][Lq][D]
  float* ws_lse;         // and their lse [split][bh][Lq] (fp32, natural log)
  int32_t split_len;     // keys per split, a multiple of the key tile
};

// How a launch maps workgroups to rows: dense (b, h) heads, packed variable-length
// sequences, or dense heads whose keys are split into chunks of split_len, one chunk per
// workgroup, each writing a partial result that a second kernel merges.
enum { kDense = 0, kVarlen = 1, kSplit = 2 };

// The rows one work item serves: the element offsets of row 0 of its head in q, k, v, out
// and the mask, the index of row 0's lse, its row counts, and the causal offset (key j is
// visible to query i iff j <= i + coff: 0 aligns the triangle top-left, Lk - Lq
// bottom-right).  Dense problems: head (b, h) of the strided tensors.  Packed
// variable-length problems: head h of sequence s of the [tokens, H, D] tensors, the lse
// laid out [H, total query tokens]; the sequence offsets are clamped into [0, total] and
// made non-decreasing, so that any contents of cu_q / cu_k keep every access in bounds.
struct Item {
  int64_t q, k, v, o, m, lse;
  int Lq, Lk, coff;
};

template <int MODE>
__device__ inline Item item_of(const Args& a, int64_t bh, int split) {
  Item it;
  if (MODE != kVarlen) {
    const int64_t b = bh / a.H, h = bh - (bh / a.H) * a.H;
    it.q = b * a.sq[0] + h * a.sq[1];
    it.k = b * a.sk[0] + h * a.sk[1];
    it.v = b * a.sv[0] + h * a.sv[1];
    it.o = b * a.so[0] + h * a.so[1];
    it.m = b * a.sm[0] + h * a.sm[1];
    it.lse = bh * a.Lq;
    it.Lq = a.Lq;
    it.Lk = a.Lk;
  } else {
    const int64_t s = bh / a.H, h = bh - (bh / a.H) * a.H;
    const int q_lo = min(max(a.cu_q[s], 0), a.Lq), q_hi = min(max(a.cu_q[s + 1], q_lo), a.Lq);
    const int k_lo = min(max(a.cu_k[s], 0), a.Lk), k_hi = min(max(a.cu_k[s + 1], k_lo), a.Lk);
    it.q = q_lo * a.sq[2] + h * a.sq[1];
    it.o = q_lo * a.so[2] + h * a.so[1];
    it.k = k_lo * a.sk[2] + h * a.sk[1];
    it.v = k_lo * a.sv[2] + h * a.sv[1];
    it.m = 0;
    it.lse = h * a.Lq + q_lo;
    it.Lq = q_hi - q_lo;
    it.Lk = k_hi - k_lo;
  }
  it.coff = a.bottom_right ? it.Lk - it.Lq : 0;
  if (MODE == kSplit) {  // keys ks .. ks + split_len - 1, renumbered from 0
    const int ks = split * a.split_len;
    it.k += int64_t(ks) * a.sk[2];
    it.v += int64_t(ks) * a.sv[2];
    it.Lk = max(0, min(it.Lk - ks, a.split_len));
    it.coff -= ks;
  }
  return it;
}

// Work item (head, query tile) and key split of this workgroup.
__device__ inline void decode_split(const Args& a, bool causal, int mode, int64_t* bh,
                                    int64_t* qt, int* split) {
  int64_t blk = blockIdx.x;
  *split = 0;
  if (mode == kSplit) {
    const int64_t per = int64_t(a.bh_count) * a.q_tiles;
    *split = int(blk / per);
    blk -= int64_t(*split) * per;
  }
  decode_item(blk, a.bh_count, a.q_tiles, causal, bh, qt);
}

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// max / sum of a per-lane value with the lane 32 positions away (the other key half of
// the same query row).  permlane32_swap exchanges the upper half of one copy with the
// lower half of the other; combining both results symmetrically gives every lane
// op(x[l], x[l ^ 32]), bit-identical in both halves.
__device__ inline float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// s_waitcnt immediate (gfx9 encoding) that waits for all vector-memory loads only:
// vmcnt = 0, expcnt and lgkmcnt left at their maxima.
constexpr int kWaitVmcnt0 = 0x0F70;

// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

// Word 3 of a raw buffer resource on gfx9: 32-bit data format, no swizzle, no stride;
// reads past num_records return zero.
constexpr int kBufferFlags = 0x00020000;

// Row permutation of a 32-key K sub-tile in LDS: swapping bits 2 and 3 of the row index
// makes the score accumulator hold, in half h of the lanes, keys 8h..8h+7 in registers
// 0..7 and keys 16+8h..16+8h+7 in registers 8..15, i.e. runs of 8 consecutive keys --
// exactly the operand layout the P^T side of the second product needs.  It is an
// involution, so the same map is used to store and to interpret.
__device__ inline int perm5(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

// ---------------------------------------------------------------------------------------
// 16-bit kernel (bf16 or fp16 inputs): 32x32x16 MFMA of that type for both products, fp32
// accumulation and softmax, P rounded to the input type.
//
// A workgroup is 8 waves owning 256 query rows of one (b, h), 32 rows per wave; each
// SIMD hosts two of its waves, one from each of two groups.  Per key tile t of 64 keys,
// a wave's work splits into a matrix phase M(t) = { O += V(t-1) P(t-1); S(t) = K(t) Q^T }
// and a vector phase V(t) = { softmax of S(t) -> P(t) }, and the two groups run them
// out of step, separated by workgroup barriers:
//     phase A of step t:  group 0 runs M(t),   group 1 runs V(t-1)
//     phase B of step t:  group 0 runs V(t),   group 1 runs M(t)
// so on every SIMD one wave feeds the matrix cores while the other feeds the vector
// ALU.  The groups take alternating 32-row slices, so under a causal mask their numbers
// of live key tiles differ by at most one.
//
// LDS per workgroup: two K stages and two V stages, each a plain row-major copy of 64
// keys x D.  Rows are padded so that the operand reads below hit distinct banks of the
// 64-bank LDS: K by 16 bytes (the 16 rows a b128 read touches start 4 banks apart), V by
// 64 bytes (the four rows of a transposing read start 16 or 48 banks apart, so the two
// 16-lane groups reading 32 bytes each from them never share a bank).  Rows of a 32-key
// K sub-tile are stored with bits 2 and 3 of the row index swapped (perm5), so that the
// score accumulator of half h of the lanes holds keys 8h..8h+7 (registers 0..7) and
// 16+8h..16+8h+7 (registers 8..15) -- runs of 8 consecutive keys, exactly the operand
// layout P^T needs in the second product.  The V^T operand is read with the gfx950
// transposing LDS read (ds_read_b64_tr_b16): within each group of 16 lanes, lane i
// receives element i mod 4 of the 8-byte pieces addressed by lanes 4e + i/4 (e = 0..3);
// addressing V[key0 + e][d0 + 4q] from lane 4e + q therefore hands lane i the column
// d0 + i of four consecutive keys.
// ---------------------------------------------------------------------------------------
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// The 16-bit element types of the matrix-core kernel: bf16 (8 significand bits, fp32's
// range) or IEEE fp16 (11 bits, range to 65504).  Both use the same 32x32x16 product shape
// and operand layouts; only the product instruction and the rounding of P differ.
template <typename E> struct Vec16;
template <> struct Vec16<__bf16> { typedef bf16x8 v8; typedef bf16x2 v2; };
template <> struct Vec16<_Float16> { typedef f16x8 v8; typedef f16x2 v2; };

__device__ inline f32x16 mfma16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mfma16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
typedef float f32x2 __attribute__((ext_vector_type(2)));

// The running max used as the exponent reference may lag the true row max by up to this
// many base-2 units before O and l are rescaled: p = 2^(x - m_ref) then stays <= 256, far
// inside the range of fp32, bf16 and fp16 (whose largest finite value is 65504), and
// the final O / l is unchanged because both carry the same reference.
constexpr float kRescaleSlack = 8.0f;
constexpr float kRescaleBound = 256.0f;  // 2^kRescaleSlack


__device__ inline s16x4 ds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// MK: 0 no mask, 1 boolean mask, 2 additive mask (POS is then false: the scale is applied
// to the scores before the bias is added).
//
// Key split (KS, two groups, dense rows only): the workgroup holds 128 query rows, and its
// two groups walk the two halves of the item's key tiles, each staging its own K and V tiles
// in its own half of the LDS, in the same alternating phases; at the end group 1 hands its
// row state (O, exponent reference, row sum) to group 0 through LDS, which merges the two
// and stores the rows.  It shortens the longest items of small causal problems.
template <typename E, int D, bool CAUSAL, int MK, bool POS, int MODE, int G = groups_16(D),
          bool KS = false>
__global__ __launch_bounds__(256 * G) __attribute__((amdgpu_waves_per_eu(waves_16(D), waves_16(D))))
void fwd_mfma(Args a) {
  constexpr bool MASK = MK == 1, BIAS = MK == 2;
  static_assert(!(BIAS && POS), "an additive mask needs the scores scaled first");
  typedef typename Vec16<E>::v8 v8;
  typedef typename Vec16<E>::v2 v2;
  static_assert(G == 1 || G == 2, "one or two phase groups");
  static_assert(!KS || (G == 2 && MODE == kDense), "the key split runs two groups on dense rows");
  constexpr int BN = kBlockNBf16;
  constexpr int BM = KS ? 128 : 128 * G;   // query rows per workgroup
  constexpr int NT = KS ? 256 : 256 * G;   // threads staging one stream of K and V tiles
  constexpr int DG = D / 8;                // 16-byte chunks per row
  constexpr int CH = (BN * DG + NT - 1) / NT;  // chunks per thread per K (or V) tile
  constexpr bool CH_FULL = CH * NT == BN * DG;  // every thread stages CH chunks
  constexpr int NKF = 2 * (D / 16);        // K operand fragments of one tile's S
  constexpr int KPRE = (MK ? 2 : 4) < NKF ? (MK ? 2 : 4) : NKF;  // read ahead of M(t)
  constexpr int KP = k_pitch_bf16(D);      // K row pitch in LDS (bytes)
  constexpr int VP = v_pitch_bf16(D);      // V row pitch in LDS (bytes)
  constexpr int KT = BN * KP;              // bytes of one K stage
  constexpr int VT = BN * VP;              // bytes of one V stage
  static_assert(D % 32 == 0 && BM == 32 * 4 * (KS ? 1 : G) && NT == 64 * 4 * (KS ? 1 : G),
                "tile shape");
  constexpr int GLDS = 2 * KT + 2 * VT;    // two stages of K and of V: one stream of tiles
  static_assert(GLDS == lds_bytes_bf16(D), "plan and kernel disagree on LDS");
  static_assert(4 * G * 32 * KP <= GLDS, "the epilogue's output tiles fit the LDS");
  static_assert((32 * DG) % 64 == 0, "the epilogue's row chunks split evenly over a wave");
  __shared__ __attribute__((aligned(16))) char lds_all[(KS ? 2 : 1) * GLDS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;  // 0..4G-1; SIMD = wave % 4
  const int grp = G == 2 ? wave >> 2 : 0;  // phase group
  // 32-row slice of the rows; with the key split both groups hold the same 128 rows
  const int slice = KS ? wave & 3 : G == 2 ? 2 * (wave & 3) + grp : wave;
  const int tid = KS ? threadIdx.x & 255 : threadIdx.x;  // index among the stream's stagers
  char* const lds = lds_all + (KS ? grp * GLDS : 0);     // the stages of this group's stream
  const int li = lane & 31;
  const int hf = lane >> 5;

  int64_t bh, qt;
  int split;
  decode_split(a, CAUSAL, MODE, &bh, &qt, &split);
  const Item it = item_of<MODE>(a, bh, split);
  const int Lq = it.Lq, Lk = it.Lk, coff = it.coff;
  const int q0 = int(qt) * BM;
  if (MODE == kVarlen && q0 >= Lq) return;  // a tile past this sequence's rows (whole workgroup)
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + it.q;
  const char* kb = static_cast<const char*>(a.k) + 2 * it.k;
  const char* vb = static_cast<const char*>(a.v) + 2 * it.v;
  uint16_t* ob = static_cast<uint16_t*>(a.out) + it.o;
  const uint8_t* mb = MASK ? a.mask + it.m : nullptr;
  const float* bb = BIAS ? a.bias + it.m : nullptr;

  const int qw = q0 + 32 * slice;  // first query row of this wave
  const int qi = qw + li;          // this lane's query row
  const bool q_ok = qi < Lq;
  const bool wave_live = qw < Lq;

  // Q^T operand fragments, held for the whole key walk: chunk c covers head dims
  // 16c..16c+15, half hf supplies dims 16c+8hf..16c+8hf+7.
  v8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4 w = {0, 0, 0, 0};
    if (q_ok) w = ld16(qb + int64_t(qi) * a.sq[2] + 16 * c + 8 * hf);
    qf[c] = __builtin_bit_cast(v8, w);
  }
  // (the Q loads stay in flight with the first K tile's: both are retired before the key loop)

  // Key tiles the workgroup stages (keys that can be visible to some stored row), and
  // the tiles this wave computes on (with a causal mask: tiles 0 .. (qw + 31 + coff) / 64).
  int kend = Lk;
  if (CAUSAL) kend = max(0, min(kend, min(q0 + BM, Lq) + coff));
  const int ntiles_all = (kend + BN - 1) / BN;
  const int wlast = qw + 31 + coff;  // last key any row of the wave may see (causal)
  const int wtiles_all = !wave_live ? 0
                         : CAUSAL   ? (wlast < 0 ? 0 : min(ntiles_all, wlast / BN + 1))
                                    : ntiles_all;
  // The key tiles of this group's walk: all of them, or with the key split tiles [0, n0)
  // for group 0 and [n0, ntiles_all) for group 1.  Below, t is the index within the walk
  // and kt0 + t the tile's index among the keys (positions, masks, loads).
  const int n0 = KS ? (ntiles_all + 1) / 2 : ntiles_all;
  const int kt0 = KS && grp ? n0 : 0;
  const int ntiles = KS && grp ? ntiles_all - n0 : n0;
  const int wtiles = KS ? min(max(wtiles_all - kt0, 0), ntiles) : wtiles_all;

  // ---- global -> register -> LDS staging of K and V tiles.  All threads stage: K(t+1) is
  // written to LDS at the end of phase A of step t and K(t+2) loaded right after; V(t) is
  // written at the end of phase B and V(t+1) loaded right after.  Each phase carries half
  // of the store traffic, and every load has a whole step to arrive.  The loads are buffer loads whose whole byte offset (tile, row and
  // column) is in the per-lane offset, which the hardware checks against the buffer's
  // extent: rows past the end of the head read as zero, and tiles past the staged range
  // are given an offset beyond the extent, so they read zeros without touching memory.
  // Loads and stores are therefore unconditional, and the memory-counter waits before
  // the stores are exact.  Offsets stay below 2^31: the caller guarantees that
  // (Lk + 64) rows of K and of V span less than 2 GiB. ----
  const int k_rowb = int(a.sk[2]) * 2, v_rowb = int(a.sv[2]) * 2;  // row strides, bytes
  const int k_ext = Lk > 0 ? (Lk - 1) * k_rowb + 2 * D : 0;
  const int v_ext = Lk > 0 ? (Lk - 1) * v_rowb + 2 * D : 0;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kb, 0, k_ext, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, v_ext, kBufferFlags);
  // Chunk p of this thread is chunk tid + p * NT of the tile (row-major, DG per row).  When
  // the tile splits evenly (D = 64, 128, 256) chunk p sits ROWS rows below chunk 0;
  // otherwise (D = 32, 96) each chunk's row and column are computed, and chunks past the
  // tile's end are neither loaded nor stored -- a whole-wave condition, since BN * DG is a
  // multiple of 64 there.
  constexpr bool EVEN = CH_FULL && NT % DG == 0;
  constexpr int ROWS = EVEN ? NT / DG : 0;   // tile rows covered by one chunk pass
  auto chunk_ok = [&](int p) { return EVEN || tid + p * NT < BN * DG; };
  const int ld_row = tid / DG, ld_col = tid % DG;  // this thread's first chunk
  const int k_goff = ld_row * k_rowb + ld_col * 16;
  const int v_goff = ld_row * v_rowb + ld_col * 16;
  const int k_soff = ((ld_row & ~31) | perm5(ld_row & 31)) * KP + ld_col * 16;
  const int v_soff = ld_row * VP + ld_col * 16;
  // byte offsets of chunk p within a tile: global (row stride rowb; chunk 0's offset is in
  // the tile base when the tile splits evenly) and LDS (K or V layout)
  auto g_off = [&](int p, int rowb) {
    if (EVEN) return p * ROWS * rowb;
    const int c = tid + p * NT;
    return (c / DG) * rowb + (c % DG) * 16;
  };
  auto k_sto = [&](int p) {
    // perm5 acts within 32-row sub-tiles: a chunk pass of a multiple of 32 rows leaves it
    // unchanged (D = 64, 128); a pass of 8 rows (D = 256) does not
    if (EVEN && ROWS % 32 == 0) return k_soff + p * ROWS * KP;
    const int c = tid + p * NT, r = c / DG;
    return ((r & ~31) | perm5(r & 31)) * KP + (c % DG) * 16;
  };
  auto v_sto = [&](int p) {
    if (EVEN) return v_soff + p * ROWS * VP;
    const int c = tid + p * NT;
    return (c / DG) * VP + (c % DG) * 16;
  };
  u32x4 kreg[CH], vreg[CH];
  auto load_k = [&](int t) {
    const int base = (EVEN ? k_goff : 0) + (t < ntiles ? (kt0 + t) * BN * k_rowb : k_ext);
#pragma unroll
    for (int p = 0; p < CH; ++p)
      if (chunk_ok(p))
        kreg[p] = __builtin_amdgcn_raw_buffer_load_b128(krs, base + g_off(p, k_rowb), 0, 0);
  };
  auto load_v = [&](int t) {
    const int base = (EVEN ? v_goff : 0) + (t < ntiles ? (kt0 + t) * BN * v_rowb : v_ext);
#pragma unroll
    for (int p = 0; p < CH; ++p)
      if (chunk_ok(p))
        vreg[p] = __builtin_amdgcn_raw_buffer_load_b128(vrs, base + g_off(p, v_rowb), 0, 0);
  };
  auto store_k = [&](int st) {
#pragma unroll
    for (int p = 0; p < CH; ++p)
      if (chunk_ok(p)) *reinterpret_cast<u32x4*>(lds + st * KT + k_sto(p)) = kreg[p];
  };
  auto store_v = [&](int st) {
#pragma unroll
    for (int p = 0; p < CH; ++p)
      if (chunk_ok(p)) *reinterpret_cast<u32x4*>(lds + 2 * KT + st * VT + v_sto(p)) = vreg[p];
  };

  // Per-lane operand addresses (stage and tile offsets are immediates).
  const int kfrag = li * KP + hf * 16;
  const int g16 = lane >> 4, e4 = (lane >> 2) & 3, q4 = lane & 3;
  const int vfrag = (8 * (g16 >> 1) + e4) * VP + (16 * (g16 & 1) + 4 * q4) * 2;
  const float c2 = POS ? a.scale_log2 : 1.f;

  // Mask bytes (boolean mask) and bias values (additive mask) of this lane's keys of key
  // tile t: runs of 8 keys at 64t + 32kt + 16g + 8hf, run 2kt + g.  They are loaded ahead
  // of the vector phase that uses them, so that the latency of the loads is covered by the
  // phases in between: the mask bytes of tile t + 1 are loaded at the start of V(t) (eight
  // registers), the bias values of tile t + 1 at the end of V(t), into the registers V(t)
  // has just consumed (a second set of 32 would not fit beside the D = 128 accumulators,
  // and measured no faster at D = 64).  Lanes past the last query row, and tiles past the
  // wave's last one, load nothing (all keys visible, zero bias).
  constexpr int NMB = MASK ? 4 : 1, NBV = BIAS ? 32 : 1;
  uint64_t mcur[NMB];
  float bcur[NBV];
  auto load_mask = [&](uint64_t* m, int t) {
    const uint8_t* mrow = mb + int64_t(qi) * a.sm[2];
#pragma unroll
    for (int run = 0; run < 4; ++run) {
      const int key0 = t * BN + 32 * (run >> 1) + 16 * (run & 1) + 8 * hf;
      if (a.mask_vec8 && key0 + 8 <= Lk) {
        m[run] = *reinterpret_cast<const uint64_t*>(mrow + key0);
      } else {
        uint64_t w = 0;
        for (int e = 0; e < 8; ++e)
          if (key0 + e < Lk) w |= uint64_t(mrow[key0 + e]) << (8 * e);
        m[run] = w;
      }
    }
  };
  auto load_bias = [&](float* bv, int t) {
    const float* brow = bb + int64_t(qi) * a.sm[2];
#pragma unroll
    for (int run = 0; run < 4; ++run) {
      const int key0 = t * BN + 32 * (run >> 1) + 16 * (run & 1) + 8 * hf;
      if (a.bias_vec4 && key0 + 8 <= Lk) {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(brow + key0);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(brow + key0 + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bv[8 * run + e] = lo[e];
          bv[8 * run + e + 4] = hi[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) bv[8 * run + e] = key0 + e < Lk ? brow[key0 + e] : 0.f;
      }
    }
  };
#pragma unroll
  for (int i = 0; i < NMB; ++i) mcur[i] = ~0ull;
#pragma unroll
  for (int i = 0; i < NBV; ++i) bcur[i] = 0.f;
  if (MASK && q_ok && wtiles > 0) load_mask(mcur, kt0);
  if (BIAS && q_ok && wtiles > 0) load_bias(bcur, kt0);

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_ref = -INFINITY;  // exponent reference (base-2 units), may lag the row max
  float l_run = 0.f;        // sum of 2^(x - m_ref) over this lane's key half
  f32x16 s[2];              // scores of tile t; sub-tile kt, register r = key
                            // 32kt + 16(r/8) + 8hf + r%8
  v8 pf[4];             // P^T operand of tile t: chunk c = keys 16c + 8hf .. +7
  v8 kpre[KPRE];        // first K fragments of the next S, read ahead in the vector phase

  // K operand fragment i of a tile's S, in the order the products consume them:
  // i = 2c + kt is head-dim chunk c (dims 16c..16c+15) of key sub-tile kt (NKF of them).
  auto kfrag_off = [](int i) { return (i & 1) * 32 * KP + (i >> 1) * 32; };

  // The first KPRE K fragments of tile t's S, read at the end of the vector phase that
  // precedes M(t) (K(t) is staged by then), so M(t) starts on the matrix cores at once.
  auto prefetch_k = [&](int t) {
    if (t >= wtiles) return;
    const char* kfp = lds + (t & 1) * KT + kfrag;
#pragma unroll
    for (int i = 0; i < KPRE; ++i) kpre[i] = __builtin_bit_cast(v8, ld16(kfp + kfrag_off(i)));
  };

  // Matrix phase M(t): S^T(t) = K(t) Q^T, then O^T += V^T(t-1) P^T(t-1).  It runs at
  // raised wave priority: the wave of the other group on this SIMD issues a dense
  // stream of independent vector instructions, and without priority it would take every
  // issue slot and hold the matrix products back.  Consecutive products always go to
  // different accumulators (the two score sub-tiles alternate; the four output blocks
  // rotate): a product that accumulates onto the previous one's result waits for it to
  // retire, about 40 instead of 32 cycles per 32x32x16 product.
  auto mphase = [&](int t) {
    __builtin_amdgcn_s_setprio(1);
    if (t < wtiles) {
      const char* kfp = lds + (t & 1) * KT + kfrag;
      v8 kf[NKF];
#pragma unroll
      for (int i = 0; i < NKF; ++i)
        kf[i] = i < KPRE ? kpre[i] : __builtin_bit_cast(v8, ld16(kfp + kfrag_off(i)));
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
#pragma unroll
      for (int i = 0; i < NKF; ++i)
        s[i & 1] = mfma16(kf[i], qf[i >> 1], s[i & 1]);
      // Up to four reads first, then one product per read until the reads are issued,
      // then the remaining products.
      constexpr int R0 = NKF - KPRE < 4 ? NKF - KPRE : 4;
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, R0, 0);
#pragma unroll
      for (int i = 0; i < NKF - KPRE - R0; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, NKF - (NKF - KPRE - R0), 0);
    }
    if (t >= 1 && t - 1 < wtiles) {
      // the V^T operand of key chunk c comes from two transposing reads (keys
      // 16c + 8hf + 0..3 and + 4..7, head dims 32dt + li)
      const char* vfp = lds + 2 * KT + ((t - 1) & 1) * VT + vfrag;
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const s16x4 lo = ds_read_tr(vfp + (16 * c) * VP + 64 * dt);
          const s16x4 hi = ds_read_tr(vfp + (16 * c + 4) * VP + 64 * dt);
          const s16x4 both[2] = {lo, hi};
          const v8 vf = __builtin_bit_cast(v8, both);
          o[dt] = mfma16(vf, pf[c], o[dt]);
        }
      // Keep LDS reads ahead of the products: the first 8 reads, then one product per
      // two reads, then the remaining products.
      __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 8, 0);
#pragma unroll
      for (int i = 0; i < 2 * (D / 32) * 4 / 2 - 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      }
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 4, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // Vector phase V(t): the online softmax of S(t) into P(t).
  auto vphase = [&](int t) {
    if (t < 0 || t >= wtiles) return;
    const int k0 = (kt0 + t) * BN;
    // Scores in the comparison domain: raw q.k when the scale is positive (the scale is
    // folded into the exponent), else scale * q.k.  Invisible keys -> -inf.
    if (!POS) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] *= a.scale_log2;
    }
    const bool pre = q_ok && t + 1 < wtiles;  // this lane loads tile t + 1's mask / bias
    uint64_t mnext[NMB];
    if (MASK) {
#pragma unroll
      for (int i = 0; i < NMB; ++i) mnext[i] = ~0ull;
      if (pre) load_mask(mnext, kt0 + t + 1);
    }
    if (BIAS) {
      // additive mask of this lane's keys, in base-2 units; keys past Lk are hidden below
#pragma unroll
      for (int run = 0; run < 4; ++run)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          s[run >> 1][8 * (run & 1) + e] =
              __builtin_fmaf(bcur[8 * run + e], kLog2e, s[run >> 1][8 * (run & 1) + e]);
    }
    // Hidden keys -> -inf: on the tiles that cross the causal diagonal or the end of the
    // keys, by position (and mask byte); on the others, with a mask, by mask byte only.
    auto mask_byte = [&](int kt, int r) {  // 32-bit halves: byte tests, not 64-bit compares
      const uint64_t w = mcur[2 * kt + (r >> 3)];
      const uint32_t half = (r & 4) ? uint32_t(w >> 32) : uint32_t(w);
      return (half >> (8 * (r & 3))) & 0xffu;
    };
    const bool edge = (CAUSAL && k0 + BN - 1 > qw + coff) || (k0 + BN > Lk);
    if (edge) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kt + 16 * (r >> 3) + 8 * hf + (r & 7);
          bool hide = key >= Lk;
          if (CAUSAL) hide = hide || key > qi + coff;
          if (MASK) hide = hide || mask_byte(kt, r) == 0;
          if (hide) s[kt][r] = -INFINITY;
        }
    } else if (MASK) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (mask_byte(kt, r) == 0) s[kt][r] = -INFINITY;
    }
    // With a boolean mask, whether any key of this tile is visible to the lane's row by its
    // mask bytes (keys past Lk have byte 0; keys hidden by position alone still count).
    bool mvis = true;
    if (MASK) {
      uint32_t any = 0;
#pragma unroll
      for (int i = 0; i < NMB; ++i) any |= uint32_t(mcur[i]) | uint32_t(mcur[i] >> 32);
      mvis = any != 0;
#pragma unroll
      for (int i = 0; i < NMB; ++i) mcur[i] = mnext[i];
    }
    if (BIAS && pre) load_bias(bcur, kt0 + t + 1);
    // Online softmax with a lagging reference.  p = 2^(x - m_ref), rounded to the input type
    // two at a time into the P^T operand; the row sum adds the fp32 values (the lse needs
    // them unrounded) in two independent chains.
    auto exps = [&](float mu, float* psum) {
      float ps[2];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 8 * (c & 1) + 2 * e;
          const f32x2 pp = {exp2_fast(__builtin_fmaf(s[c >> 1][r], c2, -mu)),
                            exp2_fast(__builtin_fmaf(s[c >> 1][r + 1], c2, -mu))};
          ps[c & 1] = c < 2 && e == 0 ? pp[0] + pp[1] : ps[c & 1] + pp[0] + pp[1];
          w[e] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pp, v2));
        }
        pf[c] = __builtin_bit_cast(v8, w);
      }
      *psum = ps[0] + ps[1];
    };
    // Fast path: the exponentials against the current reference, no row max.  A lane whose
    // 32 values sum to at most 2^kRescaleSlack has every p <= 2^kRescaleSlack, i.e. no score
    // above the reference by more than the slack, so no rescale is due.  A row with no
    // reference yet takes the fast path only when none of its keys in the tile is visible
    // (boolean mask: all of the lane's mask bytes zero), against reference 0: every p is 0,
    // as the slow path would give.  Otherwise the wave takes the slow path: the row maxima
    // (a chain of 3-input maxima and one permlane32 swap), the rescale of O and l where some
    // row's max grew by more than the slack, and the exponentials again.  Both paths make
    // the same rescale decisions as always computing the maxima, so the result does not
    // depend on which path ran.
    float lt = 0.f;
    bool slow = true;
    const bool noref = m_ref == -INFINITY;
    if (!MASK) {
      if (!__builtin_amdgcn_ballot_w64(noref)) {
        exps(m_ref, &lt);
        slow = !(lt <= kRescaleBound);
      }
    } else if (!__builtin_amdgcn_ballot_w64(noref && mvis)) {
      exps(noref ? 0.f : m_ref, &lt);
      slow = !noref && !(lt <= kRescaleBound);
    }
    if (__builtin_amdgcn_ballot_w64(slow)) {
      float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
      for (int i = 2; i < 32; i += 2)
        mx = fmaxf(fmaxf(mx, s[i >> 4][i & 15]), s[i >> 4][(i + 1) & 15]);
      mx = pair_max(mx) * c2;  // base-2 units
      if (__builtin_amdgcn_ballot_w64(mx > m_ref + kRescaleSlack)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = m_ref == -INFINITY ? 0.f : exp2_fast(m_ref - m_new);
        m_ref = m_new;
        l_run *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
      }
      exps(m_ref == -INFINITY ? 0.f : m_ref, &lt);
    }
    l_run += lt;
  };

  // ---- two-phase pipeline over key tiles ----
  // Step t:  phase A: group 0 runs M(t); group 1 runs V(t-1) and reads ahead for its M(t);
  //                   then every thread writes K(t+1) to LDS
  //                   and loads K(t+2)
  //          phase B: group 0 runs V(t) and reads ahead for M(t+1); group 1 runs M(t);
  //                   then every thread writes V(t) to LDS and loads V(t+1)
  // M(t) reads K(t) (stage t&1) and V(t-1) (stage (t-1)&1); K(t+1) and V(t) go to the
  // other stages, whose previous tiles step t-1 finished with.
  // Prologue: the Q, first mask / bias, K(0) and V(0) loads are in flight together;
  // retiring all of them here (on every path) leaves only K(1) outstanding at the loop's
  // entry, so the memory-counter waits in the loop cover just the tiles they need.  Each K
  // and V tile is then loaded right after its predecessor is written to LDS, a whole step
  // before its own store.
  load_k(0);
  load_v(0);
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  store_k(0);
  load_k(1);
  __syncthreads();
  if (G == 1) {
    // One wave per SIMD (D = 256): each wave runs M(t) then V(t).  K(t+1) and V(t) go to
    // the stages that held K(t-1) and V(t-2), whose last reader, M(t-1), every wave
    // finished before the previous barrier; one barrier per step publishes them.
    for (int t = 0; t <= ntiles; ++t) {
      prefetch_k(t);
      mphase(t);
      vphase(t);
      store_k((t + 1) & 1);
      load_k(t + 2);
      store_v(t & 1);
      load_v(t + 1);
      __syncthreads();
    }
  } else {
    // (with the key split both groups run the longer walk's n0 + 1 steps; tiles past a
    // group's own walk read as zeros and are not computed on)
    if (grp == 0) prefetch_k(0);
    for (int t = 0; t <= n0; ++t) {
      if (grp == 0) {
        mphase(t);
      } else {
        vphase(t - 1);
        prefetch_k(t);
      }
      store_k((t + 1) & 1);
      load_k(t + 2);
      __syncthreads();
      if (grp == 0) {
        vphase(t);
        prefetch_k(t + 1);
      } else {
        mphase(t);
      }
      store_v(t & 1);
      load_v(t + 1);
      __syncthreads();
    }
  }

  if (KS) {
    // Group 1 hands its row state to the group 0 wave of the same slice through LDS (free
    // after the loop's last barrier): O register-major, each 16-byte piece of a register
    // quartet at lane * 16 of its own 1 KB block, then the reference and the row sum.  Group
    // 0 rescales both to the larger reference and adds them.
    constexpr int NR4 = D / 32 * 4;  // register quartets of O
    char* xo = lds_all + slice * NR4 * 1024 + lane * 16;
    float* xm = reinterpret_cast<float*>(lds_all + 4 * NR4 * 1024) + 2 * (slice * 64 + lane);
    if (grp == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *reinterpret_cast<f32x4*>(xo + (4 * dt + g) * 1024) =
              f32x4{o[dt][4 * g], o[dt][4 * g + 1], o[dt][4 * g + 2], o[dt][4 * g + 3]};
      xm[0] = m_ref;
      xm[1] = l_run;
    }
    __syncthreads();
    if (grp == 0) {
      const float m1 = xm[0], l1 = xm[1];
      const float m = fmaxf(m_ref, m1);
      const float a0 = m_ref == -INFINITY ? 0.f : exp2_fast(m_ref - m);
      const float a1 = m1 == -INFINITY ? 0.f : exp2_fast(m1 - m);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 w = *reinterpret_cast<const f32x4*>(xo + (4 * dt + g) * 1024);
#pragma unroll
          for (int e = 0; e < 4; ++e) o[dt][4 * g + e] = o[dt][4 * g + e] * a0 + w[e] * a1;
        }
      l_run = l_run * a0 + l1 * a1;
      m_ref = m;
    }
    __syncthreads();  // the exchange area is read before the output tiles reuse it
  }
  // ---- epilogue: normalise, safe-softmax zeros, store O and the LSE ----
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (MODE == kSplit) {
    if (q_ok) {
      const int64_t prow = (int64_t(split) * a.bh_count + bh) * Lq + qi;
      float* orow = a.ws_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const f32x4 w = {o[dt][4 * g] * inv, o[dt][4 * g + 1] * inv, o[dt][4 * g + 2] * inv,
                           o[dt][4 * g + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * g + 4 * hf) = w;
        }
      if (hf == 0)
        a.ws_lse[prow] = l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
  } else {
    // The wave's 32 x D output tile goes through LDS (free after the key loop's last
    // barrier; each wave uses its own 32 rows of pitch KP), so that the global stores write
    // whole rows: lane l stores 16-byte chunks l, l + 64, ... of the tile in row-major order,
    // four rows of D = 128 per instruction, instead of 8-byte pieces of 32 rows.
    char* ot = lds_all + wave * 32 * KP;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // registers 4g..4g+3 hold head dims 32dt + 8g + 4hf + 0..3
        uint32_t w[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const E lo = static_cast<E>(o[dt][4 * g + 2 * e] * inv);
          const E hi = static_cast<E>(o[dt][4 * g + 2 * e + 1] * inv);
          w[e] = uint32_t(__builtin_bit_cast(uint16_t, lo)) |
                 (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        *reinterpret_cast<u32x2*>(ot + li * KP + (32 * dt + 8 * g + 4 * hf) * 2) =
            u32x2{w[0], w[1]};
      }
    __syncthreads();
    const bool stores = !KS || grp == 0;  // with the key split, group 0 holds the merged rows
    if (stores) {
#pragma unroll
      for (int i = 0; i < 32 * DG / 64; ++i) {
        const int c = i * 64 + lane, r = c / DG, col = c % DG;
        const u32x4 w = *reinterpret_cast<const u32x4*>(ot + r * KP + col * 16);
        if (qw + r < Lq) *reinterpret_cast<u32x4*>(ob + int64_t(qw + r) * a.so[2] + col * 8) = w;
      }
    }
    if (stores && q_ok && a.lse && hf == 0)
      a.lse[it.lse + qi] =
          l_tot > 0.f ? (m_ref + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}


// ---------------------------------------------------------------------------------------
// fp32 kernel: fp32 MFMA 32x32x2 (true fp32 products, fp32 accumulation) for both
// products; same decomposition as the 16-bit kernel, probabilities stay fp32.
// ---------------------------------------------------------------------------------------
template <int D, bool CAUSAL, int MK, int MODE>
__global__ __launch_bounds__(kThreadsF32) void fwd_f32(Args a) {
  constexpr bool MASK = MK == 1, BIAS = MK == 2;
  constexpr int DG = D / 4;                             // 16-byte groups per row
  constexpr int CH = kBlockNF32 * DG / kThreadsF32;           // chunks per thread per tile
  constexpr int KROW = D + 1;                           // odd pitch: conflict-free column reads
  constexpr int K_ELEMS = kBlockNF32 * KROW;
  constexpr int V_ELEMS = kBlockNF32 * D;
  constexpr int STAGE = K_ELEMS + V_ELEMS;
  constexpr int NS = stages_f32(D);  // LDS stages: 2 (double-buffered) or 1 (D = 256)
  static_assert(CH * kThreadsF32 == kBlockNF32 * DG, "tile must split evenly over threads");
  static_assert(NS * STAGE * 4 == lds_bytes_f32(D), "plan and kernel disagree on LDS");
  __shared__ __attribute__((aligned(16))) float lds[NS * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int hf = lane >> 5;

  int64_t bh, qt;
  int split;
  decode_split(a, CAUSAL, MODE, &bh, &qt, &split);
  const Item it = item_of<MODE>(a, bh, split);
  const int Lq = it.Lq, Lk = it.Lk, coff = it.coff;
  const int q0 = int(qt) * kBlockMF32;
  if (MODE == kVarlen && q0 >= Lq) return;  // a tile past this sequence's rows (whole workgroup)
  const float* qb = static_cast<const float*>(a.q) + it.q;
  const float* kb = static_cast<const float*>(a.k) + it.k;
  const float* vb = static_cast<const float*>(a.v) + it.v;
  float* ob = static_cast<float*>(a.out) + it.o;
  const uint8_t* mb = MASK ? a.mask + it.m : nullptr;
  const float* bb = BIAS ? a.bias + it.m : nullptr;

  const int qw = q0 + wave * 32;
  const int qi = qw + li;
  const bool q_ok = qi < Lq;
  const bool wave_live = qw < Lq;

  // Q^T operand: chunk c supplies head dim 2c + hf.
  float qf[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qf[c] = q_ok ? qb[int64_t(qi) * a.sq[2] + 2 * c + hf] : 0.f;

  int kend = Lk;
  if (CAUSAL) kend = max(0, min(kend, min(q0 + kBlockMF32, Lq) + coff));
  const int ntiles = (kend + kBlockNF32 - 1) / kBlockNF32;

  u32x4 kreg[CH], vreg[CH];
  auto load_tile = [&](int t) {
    const int k0 = t * kBlockNF32;
#pragma unroll
    for (int p = 0; p < CH; ++p) {
      const int c = tid + p * kThreadsF32;
      const int row = c / DG, col = (c % DG) * 4;
      const int key = k0 + row;
      const bool ok = key < Lk;
      kreg[p] = ok ? ld16(kb + int64_t(key) * a.sk[2] + col) : u32x4{0, 0, 0, 0};
      vreg[p] = ok ? ld16(vb + int64_t(key) * a.sv[2] + col) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    float* ks = lds + buf * STAGE;
    float* vs = ks + K_ELEMS;
#pragma unroll
    for (int p = 0; p < CH; ++p) {
      const int c = tid + p * kThreadsF32;
      const int row = c / DG, col = (c % DG) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) ks[row * KROW + col + e] = __uint_as_float(kreg[p][e]);
      *reinterpret_cast<u32x4*>(vs + row * D + col) = vreg[p];
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;
  float l_run = 0.f;

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = NS == 2 ? t & 1 : 0;
    if (NS == 2 && t + 1 < ntiles) load_tile(t + 1);
    const float* ks = lds + buf * STAGE;
    const float* vs = ks + K_ELEMS;
    const int k0 = t * kBlockNF32;
    const bool tile_live = wave_live && (!CAUSAL || k0 <= qw + 31 + coff);

    if (tile_live) {
      // S^T = K . Q^T ; lane (li, hf) register r of sub-tile kt holds key
      // k0 + 32kt + 8(r/4) + 4hf + r%4 of query row qi.
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
        const bool sub_live = !CAUSAL || (k0 + 32 * kt <= qw + 31 + coff);
        if (sub_live) {
#pragma unroll
          for (int c = 0; c < D / 2; ++c)
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[(32 * kt + li) * KROW + 2 * c + hf],
                                                         qf[c], s[kt], 0, 0, 0);
        }
      }

      float x[2][16];
      const bool edge = (CAUSAL && k0 + kBlockNF32 - 1 > qw + coff) || (k0 + kBlockNF32 > Lk);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float xv = s[kt][r] * a.scale_log2;
          const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (BIAS && q_ok && key < Lk)  // additive mask, in base-2 units
            xv = __builtin_fmaf(bb[int64_t(qi) * a.sm[2] + key], kLog2e, xv);
          if (edge || MASK) {
            bool hide = key >= Lk;
            if (CAUSAL) hide = hide || key > qi + coff;
            if (MASK && !hide && q_ok) hide = mb[int64_t(qi) * a.sm[2] + key] == 0;
            if (hide) xv = -INFINITY;
          }
          x[kt][r] = xv;
        }

      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, x[kt][r]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2_fast(m_run - m_use);
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float p = exp2_fast(x[kt][r] - m_use);
          x[kt][r] = p;
          psum += p;
        }
      l_run = l_run * alpha + psum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;

      // O^T += V^T . P^T, two keys (one per lane half) per MFMA.
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x2f32(vs[key * D + 32 * dt + li], x[kt][r],
                                                         o[dt], 0, 0, 0);
          }
    }

    if (NS == 2) {
      if (t + 1 < ntiles) store_tile(buf ^ 1);
      __syncthreads();
    } else if (t + 1 < ntiles) {  // one stage: every wave is done with it before the refill
      load_tile(t + 1);
      __syncthreads();
      store_tile(0);
      __syncthreads();
    }
  }

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (MODE == kSplit) {
    if (q_ok) {
      const int64_t prow = (int64_t(split) * a.bh_count + bh) * Lq + qi;
      float* orow = a.ws_o + prow * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(o[dt][4 * g + e] * inv);
          *reinterpret_cast<u32x4*>(orow + 32 * dt + 8 * g + 4 * hf) = w;
        }
      if (hf == 0)
        a.ws_lse[prow] = l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
  } else if (q_ok) {
    float* orow = ob + int64_t(qi) * a.so[2];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(o[dt][4 * g + e] * inv);
        *reinterpret_cast<u32x4*>(orow + 32 * dt + 8 * g + 4 * hf) = w;
      }
    if (a.lse && hf == 0)
      a.lse[it.lse + qi] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------
// Merge of split-key partial results.  Split s of a row holds o_s = its softmax-weighted
// sum of values over its keys, normalised by its own sum, and lse_s = log of that sum;
// the row's result is the same quantity over all keys:
//   lse = log sum_s exp(lse_s),   out = sum_s exp(lse_s - lse) o_s,
// computed around m = max_s lse_s (splits with no visible key have lse_s = -inf and
// weight 0; a row with none at all gets out = 0, lse = -inf).  One wave per row, lane l
// holding head dims l, l + 64, ...
// ---------------------------------------------------------------------------------------
constexpr int kCombineRows = 4;  // rows (waves) per workgroup

template <int D, typename T>
__global__ __launch_bounds__(64 * kCombineRows) void splitkv_combine(Args a, int nsplit) {
  const int lane = threadIdx.x & 63;
  const int64_t rows = int64_t(a.bh_count) * a.Lq;
  const int64_t row = int64_t(blockIdx.x) * kCombineRows + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int64_t bh = row / a.Lq, i = row - bh * a.Lq;
  float m = -INFINITY;
  for (int sp = 0; sp < nsplit; ++sp) m = fmaxf(m, a.ws_lse[sp * rows + row]);
  constexpr int E = (D + 63) / 64;  // head dims per lane: lane + 64e for lane + 64e < D
  float acc[E];
#pragma unroll
  for (int e = 0; e < E; ++e) acc[e] = 0.f;
  float wsum = 0.f;
  if (m != -INFINITY) {
    for (int sp = 0; sp < nsplit; ++sp) {
      const float w = exp2_fast((a.ws_lse[sp * rows + row] - m) * kLog2e);
      wsum += w;
      const float* o = a.ws_o + (sp * rows + row) * D;
#pragma unroll
      for (int e = 0; e < E; ++e)
        if (lane + 64 * e < D) acc[e] = __builtin_fmaf(w, o[lane + 64 * e], acc[e]);
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t b = bh / a.H, h = bh - b * a.H;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    if (lane + 64 * e >= D) break;
    const int64_t off = b * a.so[0] + h * a.so[1] + i * a.so[2] + lane + 64 * e;
    static_cast<T*>(a.out)[off] = static_cast<T>(acc[e] * inv);
  }
  if (a.lse && lane == 0)
    a.lse[row] = wsum > 0.f ? m + __builtin_amdgcn_logf(wsum) * kLn2 : -INFINITY;
}

template <int D, bool CAUSAL, int MK, int MODE>
hipError_t launch(const Args& a, int dtype, int groups, bool key_split, unsigned grid,
                  hipStream_t stream) {
  void* args[] = {const_cast<Args*>(&a)};
  const void* fn;
  constexpr bool POS_OK = MK != 2;  // an additive mask takes the explicitly scaled path
  const bool pos = POS_OK && a.scale_log2 > 0.f;
  // the key split for small causal dense problems at D <= 64 (fwd_key_split)
  if constexpr (MODE == kDense && CAUSAL && D <= 64) {
    if (key_split && dtype != 0) {
      if (dtype == 1)
        fn = pos ? reinterpret_cast<const void*>(&fwd_mfma<__bf16, D, CAUSAL, MK, POS_OK, MODE, 2, true>)
                 : reinterpret_cast<const void*>(&fwd_mfma<__bf16, D, CAUSAL, MK, false, MODE, 2, true>);
      else
        fn = pos ? reinterpret_cast<const void*>(&fwd_mfma<_Float16, D, CAUSAL, MK, POS_OK, MODE, 2, true>)
                 : reinterpret_cast<const void*>(&fwd_mfma<_Float16, D, CAUSAL, MK, false, MODE, 2, true>);
      return hipLaunchKernel(fn, dim3(grid), dim3(512), args, 0, stream);
    }
  }
  // the one-group tile for small dense problems and decode-shaped split keys (fwd_groups)
  if constexpr ((MODE == kDense || MODE == kSplit) && D <= 128) {
    if (groups == 1 && dtype != 0) {
      if (dtype == 1)
        fn = pos ? reinterpret_cast<const void*>(&fwd_mfma<__bf16, D, CAUSAL, MK, POS_OK, MODE, 1>)
                 : reinterpret_cast<const void*>(&fwd_mfma<__bf16, D, CAUSAL, MK, false, MODE, 1>);
      else
        fn = pos ? reinterpret_cast<const void*>(&fwd_mfma<_Float16, D, CAUSAL, MK, POS_OK, MODE, 1>)
                 : reinterpret_cast<const void*>(&fwd_mfma<_Float16, D, CAUSAL, MK, false, MODE, 1>);
      return hipLaunchKernel(fn, dim3(grid), dim3(256), args, 0, stream);
    }
  }
  if (dtype == 1)
    fn = pos ? reinterpret_cast<const void*>(&fwd_mfma<__bf16, D, CAUSAL, MK, POS_OK, MODE>)
             : reinterpret_cast<const void*>(&fwd_mfma<__bf16, D, CAUSAL, MK, false, MODE>);
  else if (dtype == 2)
    fn = pos ? reinterpret_cast<const void*>(&fwd_mfma<_Float16, D, CAUSAL, MK, POS_OK, MODE>)
             : reinterpret_cast<const void*>(&fwd_mfma<_Float16, D, CAUSAL, MK, false, MODE>);
  else
    fn = reinterpret_cast<const void*>(&fwd_f32<D, CAUSAL, MK, MODE>);
  return hipLaunchKernel(fn, dim3(grid), dim3(block_threads(dtype, D)), args, 0, stream);
}

template <int D>
hipError_t launch_d(const Args& a, int dtype, int groups, bool ks, bool causal, int mode,
                    unsigned grid, hipStream_t s) {
  if (mode == kVarlen)  // packed sequences take no mask
    return causal ? launch<D, true, 0, kVarlen>(a, dtype, groups, ks, grid, s)
                  : launch<D, false, 0, kVarlen>(a, dtype, groups, ks, grid, s);
  if (mode == kSplit)  // neither do split keys
    return causal ? launch<D, true, 0, kSplit>(a, dtype, groups, ks, grid, s)
                  : launch<D, false, 0, kSplit>(a, dtype, groups, ks, grid, s);
  if (a.mask)
    return causal ? launch<D, true, 1, kDense>(a, dtype, groups, ks, grid, s) : launch<D, false, 1, kDense>(a, dtype, groups, ks, grid, s);
  if (a.bias)
    return causal ? launch<D, true, 2, kDense>(a, dtype, groups, ks, grid, s) : launch<D, false, 2, kDense>(a, dtype, groups, ks, grid, s);
  return causal ? launch<D, true, 0, kDense>(a, dtype, groups, ks, grid, s) : launch<D, false, 0, kDense>(a, dtype, groups, ks, grid, s);
}

template <int D>
hipError_t launch_combine(const Args& a, int dtype, int nsplit, hipStream_t s) {
  const int64_t rows = int64_t(a.bh_count) * a.Lq;
  const unsigned grid = unsigned((rows + kCombineRows - 1) / kCombineRows);
  int ns = nsplit;
  void* args[] = {const_cast<Args*>(&a), &ns};
  const void* fn = dtype == 1   ? reinterpret_cast<const void*>(&splitkv_combine<D, __bf16>)
                   : dtype == 2 ? reinterpret_cast<const void*>(&splitkv_combine<D, _Float16>)
                                : reinterpret_cast<const void*>(&splitkv_combine<D, float>);
  return hipLaunchKernel(fn, dim3(grid), dim3(64 * kCombineRows), args, 0, s);
}

}  // namespace

// ---------------------------------------------------------------------------------------
// Split-key workspace of sdpa_fwd_splitkv_noalloc, for callers that cannot allocate: a
// file-scope device array of kStaticWorkspaceBytes, held by every device the library runs
// on until the process ends.  In host code the array's name is only a host-side stand-in;
// its address on a device comes from hipGetSymbolAddress with that device current, taken
// once per device and kept, and only that address is ever handed to a kernel.
// ---------------------------------------------------------------------------------------
namespace {
static __device__ __align__(256) char scratch[kStaticWorkspaceBytes];
}  // namespace

hipError_t static_workspace(int device, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    int current = 0;
    hipError_t e = hipGetDevice(&current);
    if (e != hipSuccess) return e;
    if (current != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (current != device) {
      const hipError_t back = hipSetDevice(current);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    if (!a) return hipErrorInvalidSymbol;
    addr[device] = a;
  }
  *ptr = addr[device];
  return hipSuccess;
}

hipError_t launch_fwd(const Problem& p, hipStream_t stream) {
  Args a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.out = p.out;
  a.lse = p.lse;
  a.mask = p.mask;
  a.bias = p.bias;
  a.cu_q = p.cu_q;
  a.cu_k = p.cu_k;
  for (int i = 0; i < 3; ++i) {
    a.sq[i] = p.sq[i];
    a.sk[i] = p.sk[i];
    a.sv[i] = p.sv[i];
    a.so[i] = p.so[i];
    a.sm[i] = p.sm[i];
  }
  a.H = int32_t(p.H);
  a.Lq = int32_t(p.Lq);
  a.Lk = int32_t(p.Lk);
  // dense: B*H heads of Lq rows; packed: nseq*H heads of up to max_seqlen_q rows
  const int64_t rows = p.varlen ? p.max_seqlen_q : p.Lq;
  const int mode = p.varlen ? kVarlen : p.nsplit > 0 ? kSplit : kDense;
  const int groups = fwd_groups(p.dtype, p.D, mode == kDense, p.causal != 0, p.B * p.H, p.Lq,
                                p.Lk, mode == kSplit);
  const bool ks = fwd_key_split(p.dtype, p.D, mode == kDense, p.causal != 0, p.B * p.H, p.Lq, p.Lk);
  const int bm = p.dtype != 0 ? (ks ? 128 : 128 * groups) : kBlockMF32;
  a.q_tiles = int32_t((rows + bm - 1) / bm);
  a.bh_count = int32_t((p.varlen ? p.nseq : p.B) * p.H);
  a.scale_log2 = p.scale * kLog2e;
  a.mask_vec8 = p.mask && (reinterpret_cast<uintptr_t>(p.mask) % 8 == 0) && p.sm[0] % 8 == 0 &&
                p.sm[1] % 8 == 0 && p.sm[2] % 8 == 0;
  a.bias_vec4 = p.bias && (reinterpret_cast<uintptr_t>(p.bias) % 16 == 0) && p.sm[0] % 4 == 0 &&
                p.sm[1] % 4 == 0 && p.sm[2] % 4 == 0;
  a.bottom_right = p.causal == 2;
  a.ws_o = p.ws_o;
  a.ws_lse = p.ws_lse;
  a.split_len = int32_t(p.split_len);
  const unsigned grid =
      unsigned(int64_t(a.q_tiles) * a.bh_count * (mode == kSplit ? p.nsplit : 1));
  const bool causal = p.causal != 0;
  hipError_t e;
  switch (p.D) {
    case 32: e = launch_d<32>(a, p.dtype, groups, ks, causal, mode, grid, stream); break;
    case 64: e = launch_d<64>(a, p.dtype, groups, ks, causal, mode, grid, stream); break;
    case 96: e = launch_d<96>(a, p.dtype, groups, ks, causal, mode, grid, stream); break;
    case 128: e = launch_d<128>(a, p.dtype, groups, ks, causal, mode, grid, stream); break;
    case 256: e = launch_d<256>(a, p.dtype, groups, ks, causal, mode, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || mode != kSplit) return e;
  const int ns = int(p.nsplit);
  switch (p.D) {
    case 32: return launch_combine<32>(a, p.dtype, ns, stream);
    case 64: return launch_combine<64>(a, p.dtype, ns, stream);
    case 96: return launch_combine<96>(a, p.dtype, ns, stream);
    case 128: return launch_combine<128>(a, p.dtype, ns, stream);
    default: return launch_combine<256>(a, p.dtype, ns, stream);
  }
}

}  // namespace sdpa
