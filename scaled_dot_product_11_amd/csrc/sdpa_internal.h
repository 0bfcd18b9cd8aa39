// sdpa_internal.h -- the canonical problem handed from the C ABI to the gfx950 kernels,
// the tile constants, and the work-item decode shared by host and device.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

// Tile shapes.  16-bit kernel: keys advance 64 at a time and each wave of 64 lanes owns
// 32 query rows.  For D <= 128 a workgroup is 8 waves (256 rows) forming two groups that
// alternate between matrix and vector phases, two waves per SIMD; at D = 256 a wave's
// accumulators, Q fragments and staging registers need more than the 256 registers a wave
// gets at two waves per SIMD, so the workgroup is 4 waves (128 rows), one per SIMD, each
// running its matrix and vector work in turn.  fp32 kernel: 4 waves, 32 rows each (128
// per workgroup), 64 keys at a time.
constexpr int kBlockNBf16 = 64;
constexpr int kThreadsF32 = 256;
constexpr int kBlockMF32 = 128;
constexpr int kBlockNF32 = 64;
// Head dims of the forward kernels (every dtype) and of the backward kernels (at D = 256
// the backward's accumulators and operands exceed two waves' registers per SIMD).
constexpr bool fwd_head_dim_ok(int64_t D) {
  return D == 32 || D == 64 || D == 96 || D == 128 || D == 256;
}
constexpr bool bwd_head_dim_ok(int64_t D) {
  return D == 32 || D == 64 || D == 96 || D == 128 || D == 256;
}
// Phase groups of the 16-bit kernel at head dim D (2: paired waves alternate phases).
constexpr int groups_16(int D) { return D <= 128 ? 2 : 1; }
// Waves per SIMD of a 16-bit workgroup of G groups: two (one per group, or one from each of
// two co-resident one-group workgroups) up to D = 128, else one.
constexpr int waves_16(int D) { return D <= 128 ? 2 : 1; }
// dtype: 0 = fp32, 1 = bf16, 2 = fp16 (the values of sdpa_dtype); both 16-bit types run
// the same matrix-core kernel and tiles
constexpr int block_m(int dtype, int D) { return dtype != 0 ? 128 * groups_16(D) : kBlockMF32; }
constexpr int block_n(int dtype) { return dtype != 0 ? kBlockNBf16 : kBlockNF32; }
constexpr int block_threads(int dtype, int D) {
  return dtype != 0 ? 256 * groups_16(D) : kThreadsF32;
}

// Phase groups of a 16-bit launch.  The two-group tile (two waves per SIMD in alternating
// matrix and vector phases, 256 rows) pays off where the matrix work is large and the key
// walks long: D = 96 and 128 with more than two 256-row items per CU.  Elsewhere the one-group
// tile (one wave per SIMD, 128 rows, two workgroups per CU whose matrix and vector work
// overlap unsynchronised) is faster: at D <= 64 the vector work dominates and needs no
// phase partner; with few items the launch takes as long as its longest item, which the
// shorter 128-row items halve (measured: [1,32,8192,D] causal, 1024 items: D = 32 -12 %,
// D = 64 -7 %, D = 96 +9 %, D = 128 +4 %; 512 and 256 items at D = 64 and 128: -4 % to -19 %).
// Short causal walks at D = 128 take it too, up to four 256-row items per CU: each item of
// the two-group tile runs its first and last key steps half empty and waits for its first
// tiles, a fixed cost that walks of at most 2048 keys do not amortise, while two one-group
// workgroups per CU hide each other's (measured, bf16 causal: [16,16,1024] -6 %,
// [8,16,1536] -4 %, [8,16,2048] -2 %; with 1536 or more items, or without the causal mask,
// the two-group tile stays ahead by 1 to 18 %).
// Split-key launches of decode shapes (at most 128 query rows) take the one-group tile too:
// their workgroups stream K and V for a single live query tile, and two of them per CU keep
// twice as many tile loads in flight.
constexpr int64_t kSmallProblemItems = 512;
constexpr int64_t kShortWalkItems = 1024;
constexpr int64_t kShortWalkKeys = 2048;
constexpr int64_t kDecodeRows = 128;
constexpr int fwd_groups(int dtype, int64_t D, bool dense, bool causal, int64_t bh, int64_t Lq,
                         int64_t Lk, bool split) {
  return dtype != 0 && D <= 128 &&
                 ((dense && (D <= 64 || bh * ((Lq + 255) / 256) <= kSmallProblemItems ||
                             (D == 128 && causal && Lk <= kShortWalkKeys &&
                              bh * ((Lq + 255) / 256) <= kShortWalkItems))) ||
                  (split && Lq <= kDecodeRows))
             ? 1
             : (dtype != 0 ? groups_16(int(D)) : 1);
}

// The key split (dense causal 16-bit problems at D <= 64): 8-wave workgroups of 128 rows
// whose two groups walk the two halves of an item's key tiles and merge their row states,
// one workgroup per CU (each group stages its own tiles).  Where the launch lasts as long as
// its longest items it halves them: with at most 256 such items (one round) and walks of at
// least 1024 keys, or at most 512 items and walks of at least 2048 keys.  Measured, bf16
// causal D = 64 against the one-group tile: [1,16,1024] -12 %, [2,16,1024] -12 %,
// [1,8,2048] -20 %, [1,32,2048] -5 %, [2,8,4096] -17 %, [1,8,8192] -23 %, the additive-mask
// pass [2,8,4096] -6.5 %, with a boolean mask +1 %, D = 32 [2,16,1024] -10 %,
// [1,8,4096] -20 %; and outside the rule [3,16,1024] +4 %, [4,16,1024] +13 %,
// [8,16,512] +34 % (two rounds of short walks).  The decision depends on (B*H, Lq, Lk, D)
// only, so rank-3 and rank-4 inputs of one problem take the same path.
constexpr int64_t kKeySplitOneRound = 256;
constexpr int64_t kKeySplitTwoRounds = 512;
constexpr int64_t kKeySplitKeys = 1024;
constexpr int64_t kKeySplitLongKeys = 2048;
constexpr bool fwd_key_split(int dtype, int64_t D, bool dense, bool causal, int64_t bh,
                             int64_t Lq, int64_t Lk) {
  return dtype != 0 && dense && causal && D <= 64 &&
         (bh * ((Lq + 127) / 128) <= kKeySplitOneRound
              ? Lk >= kKeySplitKeys
              : bh * ((Lq + 127) / 128) <= kKeySplitTwoRounds && Lk >= kKeySplitLongKeys);
}

// Rank-3 [N,L,D] and rank-4 [B,H,L,D] inputs both become this (b, h, row, col) view;
// every stride is in elements of the tensor's own type.  Packed variable-length inputs
// [tokens, H, D] use the h and row strides (b stride 0), Lq / Lk are the token totals,
// and cu_q / cu_k (device, nseq + 1 entries) delimit the sequences.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const uint8_t* mask;
  const float* bias;  // additive mask (fp32) through the mask strides sm; never with mask
  const int32_t* cu_q;
  const int32_t* cu_k;
  int64_t B, H, Lq, Lk, D;
  int64_t nseq, max_seqlen_q;  // packed only
  // split keys (dense, no mask): nsplit > 0 chunks of split_len keys, partial results in
  // ws_o [nsplit][B*H][Lq][D] and ws_lse [nsplit][B*H][Lq] (fp32), merged by a second kernel
  int64_t nsplit, split_len;
  float* ws_o;
  float* ws_lse;
  int64_t sq[4], sk[4], sv[4], so[4], sm[4];
  float scale;
  int causal;  // 0 none, 1 top-left (j <= i), 2 bottom-right (j <= i + Lk - Lq)
  int varlen;
  int dtype;
};

// Work item of workgroup `block`: causal problems run the heaviest query tiles first
// (the last tile of every head, then the one before, ...); the others run tile-major
// with the head index innermost.  Either way consecutive workgroups belong to different
// heads and workgroup i lands on XCD i % 8, so when B*H is a multiple of 8 all tiles of
// a head stay on one XCD and share its L2.
__host__ __device__ inline void decode_item(int64_t block, int64_t bh_count, int64_t q_tiles,
                                            bool causal, int64_t* bh, int64_t* q_tile) {
  const int64_t rank = block / bh_count;
  *bh = block - rank * bh_count;
  *q_tile = causal ? (q_tiles - 1 - rank) : rank;
}

// LDS row pitches (bytes) of the bf16 kernel's K and V tiles, and LDS bytes per
// workgroup of each kernel (two stages of K and two of V).
constexpr int k_pitch_bf16(int D) { return 2 * D + 16; }
constexpr int v_pitch_bf16(int D) { return 2 * D + 64; }
constexpr int64_t lds_bytes_bf16(int D) {
  return 2 * int64_t(kBlockNBf16) * (k_pitch_bf16(D) + v_pitch_bf16(D));
}
// The fp32 kernel double-buffers its K/V tiles up to D = 128; at D = 256 two stages would
// exceed the 160 KiB of LDS, and it runs with one.
constexpr int stages_f32(int D) { return D <= 128 ? 2 : 1; }
constexpr int64_t lds_bytes_f32(int D) {
  return stages_f32(D) * (int64_t(kBlockNF32) * (D + 1) * 4 + int64_t(kBlockNF32) * D * 4);
}

// Launches the kernel matching p.dtype / p.D / p.causal / mask on `stream` (and, with
// split keys, the merge kernel after it).  p must already be validated.  Returns a
// hipError_t.
hipError_t launch_fwd(const Problem& p, hipStream_t stream);

// Split keys: the number of splits used for a requested count (0 = automatic: enough
// workgroups to fill the chip, at least 512 keys per split, at most 64 splits) and the
// keys per split (a multiple of the 64-key tile).
inline void splitkv_plan(int64_t bh, int64_t q_tiles, int64_t Lk, int64_t requested,
                         int64_t* nsplit, int64_t* split_len) {
  int64_t want = requested;
  if (want <= 0) {
    const int64_t items = bh * q_tiles > 0 ? bh * q_tiles : 1;
    want = (512 + items - 1) / items;
    const int64_t by_keys = (Lk + 511) / 512;
    if (want > by_keys) want = by_keys;
    if (want > 64) want = 64;
    if (want < 1) want = 1;
  }
  int64_t len = (Lk + want - 1) / want;
  len = len < 64 ? 64 : (len + 63) / 64 * 64;
  *split_len = len;
  *nsplit = Lk > 0 ? (Lk + len - 1) / len : 1;
}

// sdpa_fwd_splitkv_noalloc: the split-key workspace lives in a static device array of this
// many bytes per device (partial outputs and their lse, nsplit * B*H * Lq * (D + 1) * 4).
constexpr int64_t kStaticWorkspaceBytes = int64_t(16) << 20;

// The device address of that array on `device` (looked up once per device, with the device
// made current for the lookup).  Returns a hipError_t.
hipError_t static_workspace(int device, void** ptr);

// ---- backward (bf16) ----
// Two kernels of 8 waves (two per SIMD): the dQ kernel owns 256 query rows of one (b, h)
// and walks key tiles of 64; the dK/dV kernel owns 128 keys and walks query tiles of 64.
// The dQ kernel runs first and also writes delta = rowsum(dO * O), which the dK/dV kernel
// reads.
constexpr int kThreadsBwdQ = 512;
constexpr int kThreadsBwdK = 512;
constexpr int kBwdBlockQ = 256;
constexpr int kBwdBlockK = 128;
constexpr int kBwdStep = 64;
// fp32 inputs and D = 256 take the row-by-row backward kernels: one wave per query row,
// then one per key row, kBwdGenRows rows per workgroup.
constexpr int kBwdGenRows = 4;
constexpr int kThreadsBwdGen = 64 * kBwdGenRows;
constexpr bool bwd_generic(int dtype, int64_t D) { return dtype == 0 || D == 256; }
// LDS per workgroup of the two backward kernels.  dQ: two stages, each holding the K tile
// in row-read layout (pitch k_pitch_bf16) and in transposed-read layout (pitch
// v_pitch_bf16), and the V tile in row-read layout.
constexpr int64_t lds_bytes_bwd_dq(int D) {
  return 2 * int64_t(kBwdStep) * (2 * k_pitch_bf16(D) + v_pitch_bf16(D));
}
constexpr int64_t lds_bytes_bwd_dkdv(int D) {
  // three stages of Q and dO in one swizzled copy (rows of 4, 8 or 16 slots of 16 bytes)
  // with the tile's lse and delta, then two tiles of P (32 keys x kBwdStep queries,
  // 16-bit) per SIMD
  return 3 * (int64_t(kBwdStep) * 2 * 16 * (D <= 32 ? 4 : D <= 64 ? 8 : 16) + 8 * kBwdStep) +
         2 * 4 * 32 * kBwdStep * 2;
}

struct BwdProblem {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  float* delta;
  void* dq;
  void* dk;
  void* dv;
  const uint8_t* mask;
  const float* bias;     // additive mask, addressed with the sm strides (never with mask)
  const int32_t* cu_q;   // packed sequences (varlen != 0): nseq + 1 query offsets
  const int32_t* cu_k;   // and key offsets; Lq / Lk are then the total token counts
  int64_t B, H, Lq, Lk, D;
  int64_t nseq, max_seqlen_q, max_seqlen_k;
  // dense: (batch, head, row, dim) strides; packed: (0, head, token, dim)
  int64_t sq[4], sk[4], sv[4], so[4], sdo[4], sdq[4], sdk[4], sdv[4], sm[4];
  float scale;
  int causal;
  int dtype;  // 0 fp32, 1 bf16, 2 fp16
  int varlen;
};

// Launches the dQ kernel and then the dK/dV kernel on `stream` (each only when it has
// rows to cover).  p must already be validated.  Returns a hipError_t.
hipError_t launch_bwd(const BwdProblem& p, hipStream_t stream);

}  // namespace sdpa
