// sdpa_internal.h -- the canonical problem handed from the C ABI to the gfx950 kernels,
// the tile constants, and the work-item decode shared by host and device.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

// Tile shapes.  bf16 kernel: a workgroup is 8 waves of 64 lanes, each wave owns 32 query
// rows (256 per workgroup), keys advance 64 at a time; the waves form two groups that
// alternate between matrix and vector phases.  fp32 kernel: 4 waves, 32 rows each (128
// per workgroup), 64 keys at a time.
constexpr int kThreadsBf16 = 512;
constexpr int kBlockMBf16 = 256;
constexpr int kBlockNBf16 = 64;
constexpr int kThreadsF32 = 256;
constexpr int kBlockMF32 = 128;
constexpr int kBlockNF32 = 64;
// dtype: 1 = bf16, 0 = fp32 (the values of sdpa_dtype)
constexpr int block_m(int dtype) { return dtype == 1 ? kBlockMBf16 : kBlockMF32; }
constexpr int block_n(int dtype) { return dtype == 1 ? kBlockNBf16 : kBlockNF32; }
constexpr int block_threads(int dtype) { return dtype == 1 ? kThreadsBf16 : kThreadsF32; }

// Rank-3 [N,L,D] and rank-4 [B,H,L,D] inputs both become this (b, h, row, col) view;
// every stride is in elements of the tensor's own type.
struct Problem {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const uint8_t* mask;
  int64_t B, H, Lq, Lk, D;
  int64_t sq[4], sk[4], sv[4], so[4], sm[4];
  float scale;
  int causal;
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
constexpr int64_t lds_bytes_f32(int D) {
  return 2 * (int64_t(kBlockNF32) * (D + 1) * 4 + int64_t(kBlockNF32) * D * 4);
}

// Launches the kernel matching p.dtype / p.D / p.causal / mask on `stream`.
// p must already be validated.  Returns a hipError_t.
hipError_t launch_fwd(const Problem& p, hipStream_t stream);

}  // namespace sdpa
