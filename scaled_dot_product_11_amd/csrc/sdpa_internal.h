// sdpa_internal.h -- the canonical problem handed from the C ABI to the gfx950 kernels,
// the tile constants, and the work-item decode shared by host and device.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdpa {

// Tile shape of the bf16 and fp32 kernels: 4 waves of 64 lanes, each wave owning 32
// query rows, so a workgroup owns 128 query rows and steps through 64 keys at a time.
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBlockM = 32 * kWaves;
constexpr int kBlockN = 64;

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

// LDS bytes per workgroup of each kernel (two stages of K and V tiles).
constexpr int64_t lds_bytes_bf16(int D) {
  return 2 * (int64_t(kBlockN) * (D + 8) * 2 + int64_t(D) * kBlockN * 2);
}
constexpr int64_t lds_bytes_f32(int D) {
  return 2 * (int64_t(kBlockN) * (D + 1) * 4 + int64_t(kBlockN) * D * 4);
}

// Launches the kernel matching p.dtype / p.D / p.causal / mask on `stream`.
// p must already be validated.  Returns a hipError_t.
hipError_t launch_fwd(const Problem& p, hipStream_t stream);

}  // namespace sdpa
