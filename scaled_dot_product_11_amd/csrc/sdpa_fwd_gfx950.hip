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
// Work decomposition (bf16 and fp32 kernels alike):
//   * a workgroup is 4 waves of 64 lanes and owns 128 query rows of one (b, h);
//   * each wave owns 32 query rows; lane l serves query row (l % 32) and half h = l / 32
//     of every key tile, so all per-row softmax state (running max m, running sum l,
//     rescale factor) is a per-lane scalar;
//   * the scores are computed transposed, S^T = K . Q^T, on 32x32 MFMA tiles: the
//     accumulator of a 32x32 tile gives each lane 16 keys of its own query row;
//   * the output is accumulated transposed, O^T += V^T . P^T, so P^T comes straight from
//     the score registers (rounded to bf16) and each lane again owns its query's column;
//   * K and V tiles of 64 keys are double-buffered through LDS: the global loads of tile
//     t+1 are issued before the matrix work on tile t and written to the other LDS stage
//     after it, with one barrier per tile.
#include <math.h>

#include "sdpa_internal.h"

namespace sdpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Kernel arguments: canonical (b, h, row) strides in elements; the innermost stride is 1.
struct Args {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;
  const uint8_t* mask;
  int64_t sq[3], sk[3], sv[3], so[3], sm[3];
  int32_t H, Lq, Lk, q_tiles, bh_count;
  float scale_log2;  // scale * log2(e): scores are kept in base-2 units
  int32_t mask_vec8; // mask rows may be read 8 bytes at a time
};

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

// Row permutation of a 32-key K sub-tile in LDS: swapping bits 2 and 3 of the row index
// makes the score accumulator hold, in half h of the lanes, keys 8h..8h+7 in registers
// 0..7 and keys 16+8h..16+8h+7 in registers 8..15, i.e. runs of 8 consecutive keys --
// exactly the operand layout the P^T side of the second product needs.  It is an
// involution, so the same map is used to store and to interpret.
__device__ inline int perm5(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

// XOR swizzle of the 16-byte chunks of a transposed V row (row = head-dim index d,
// 8 chunks of 8 keys) so that both the transposing stores and the operand loads of
// the second product spread over all LDS banks.
__device__ inline int vswz(int d) { return (d ^ (d >> 3)) & 7; }

// ---------------------------------------------------------------------------------------
// bf16 kernel: bf16 MFMA 32x32x16 for both products, fp32 accumulation and softmax.
// ---------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void fwd_bf16(Args a) {
  constexpr int DG = D / 8;                             // 16-byte groups per row
  constexpr int KCH = kBlockN * DG / kThreads;          // K chunks per thread per tile
  constexpr int VUNITS = (kBlockN / 4) * DG;            // (4 keys x 8 cols) V units per tile
  constexpr int KROW = D + 8;                           // K row pitch in LDS (elements)
  constexpr int K_ELEMS = kBlockN * KROW;
  constexpr int V_ELEMS = D * kBlockN;                  // transposed V: D rows of 64 keys
  constexpr int STAGE = K_ELEMS + V_ELEMS;
  static_assert(KCH * kThreads == kBlockN * DG, "K tile must split evenly over threads");
  static_assert(VUNITS <= kThreads, "one V unit per thread at most");
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int hf = lane >> 5;

  int64_t bh, qt;
  decode_item(blockIdx.x, a.bh_count, a.q_tiles, CAUSAL, &bh, &qt);
  const int64_t b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + b * a.sq[0] + h * a.sq[1];
  const uint16_t* kb = static_cast<const uint16_t*>(a.k) + b * a.sk[0] + h * a.sk[1];
  const uint16_t* vb = static_cast<const uint16_t*>(a.v) + b * a.sv[0] + h * a.sv[1];
  uint16_t* ob = static_cast<uint16_t*>(a.out) + b * a.so[0] + h * a.so[1];
  const uint8_t* mb = MASK ? a.mask + b * a.sm[0] + h * a.sm[1] : nullptr;

  const int q0 = int(qt) * kBlockM;
  const int qw = q0 + wave * 32;  // first query row of this wave
  const int qi = qw + li;         // this lane's query row
  const bool q_ok = qi < a.Lq;
  const bool wave_live = qw < a.Lq;

  // Q^T operand fragments, held in registers for the whole key walk:
  // chunk c covers head dims 16c..16c+15, half hf supplies dims 16c+8hf..16c+8hf+7.
  bf16x8 qf[D / 16];
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4 w = {0, 0, 0, 0};
    if (q_ok) w = ld16(qb + int64_t(qi) * a.sq[2] + 16 * c + 8 * hf);
    qf[c] = __builtin_bit_cast(bf16x8, w);
  }

  // Keys that can be visible to some stored row of this workgroup.
  int kend = a.Lk;
  if (CAUSAL) kend = min(kend, min(q0 + kBlockM, a.Lq));
  const int ntiles = (kend + kBlockN - 1) / kBlockN;

  // ---- global -> register staging of one K/V tile ----
  u32x4 kreg[KCH];
  u32x4 vreg[4];
  const int v_kg = tid % 16;  // V unit: keys 4*v_kg..+3 of the tile
  const int v_dg = tid / 16;  //         head dims 8*v_dg..+7
  auto load_tile = [&](int t) {
    const int k0 = t * kBlockN;
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      const int c = tid + p * kThreads;
      const int row = c / DG, col = (c % DG) * 8;
      const int key = k0 + row;
      kreg[p] = key < a.Lk ? ld16(kb + int64_t(key) * a.sk[2] + col) : u32x4{0, 0, 0, 0};
    }
    if (tid < VUNITS) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = k0 + 4 * v_kg + r;
        vreg[r] = key < a.Lk ? ld16(vb + int64_t(key) * a.sv[2] + 8 * v_dg) : u32x4{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    uint16_t* ks = lds + buf * STAGE;
    uint16_t* vt = ks + K_ELEMS;
#pragma unroll
    for (int p = 0; p < KCH; ++p) {
      const int c = tid + p * kThreads;
      const int row = c / DG, col = (c % DG) * 8;
      const int prow = (row & ~31) | perm5(row & 31);
      *reinterpret_cast<u32x4*>(ks + prow * KROW + col) = kreg[p];
    }
    if (tid < VUNITS) {
      // 4 keys x 8 dims -> 8 rows (dims) of 4 consecutive keys each.
#pragma unroll
      for (int e2 = 0; e2 < 4; ++e2) {
        const uint32_t r0 = vreg[0][e2], r1 = vreg[1][e2], r2 = vreg[2][e2], r3 = vreg[3][e2];
        const int d_lo = 8 * v_dg + 2 * e2;
        const u32x2 lo = {(r0 & 0xffffu) | (r1 << 16), (r2 & 0xffffu) | (r3 << 16)};
        const u32x2 hi = {(r0 >> 16) | (r1 & 0xffff0000u), (r2 >> 16) | (r3 & 0xffff0000u)};
        const int lc = v_kg >> 1, half = v_kg & 1;
        *reinterpret_cast<u32x2*>(vt + d_lo * kBlockN + ((lc ^ vswz(d_lo)) * 8) + half * 4) = lo;
        *reinterpret_cast<u32x2*>(vt + (d_lo + 1) * kBlockN + ((lc ^ vswz(d_lo + 1)) * 8) +
                                  half * 4) = hi;
      }
    }
  };

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY;  // running max of the base-2 scores of this row
  float l_run = 0.f;        // running sum over this lane's key half, relative to m_run

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const uint16_t* ks = lds + buf * STAGE;
    const uint16_t* vt = ks + K_ELEMS;
    const int k0 = t * kBlockN;
    // Wave-uniform: does any key of this tile reach any row of this wave?
    const bool tile_live = wave_live && (!CAUSAL || k0 <= qw + 31);

    if (tile_live) {
      // Mask bytes of this lane's keys: runs of 8 at k0 + 32kt + 16g + 8hf.
      uint64_t mbits[4] = {~0ull, ~0ull, ~0ull, ~0ull};
      if (MASK && q_ok) {
        const uint8_t* mrow = mb + int64_t(qi) * a.sm[2];
#pragma unroll
        for (int run = 0; run < 4; ++run) {
          const int key0 = k0 + 32 * (run >> 1) + 16 * (run & 1) + 8 * hf;
          if (a.mask_vec8 && key0 + 8 <= a.Lk) {
            mbits[run] = *reinterpret_cast<const uint64_t*>(mrow + key0);
          } else {
            uint64_t w = 0;
            for (int e = 0; e < 8; ++e)
              if (key0 + e < a.Lk) w |= uint64_t(mrow[key0 + e]) << (8 * e);
            mbits[run] = w;
          }
        }
      }

      // S^T = K . Q^T for the two 32-key sub-tiles.
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
        const bool sub_live = !CAUSAL || (k0 + 32 * kt <= qw + 31);
        if (sub_live) {
#pragma unroll
          for (int c = 0; c < D / 16; ++c) {
            const bf16x8 kf = __builtin_bit_cast(
                bf16x8, ld16(ks + (32 * kt + li) * KROW + 16 * c + 8 * hf));
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[c], s[kt], 0, 0, 0);
          }
        }
      }

      // Scale into base-2 units and hide invisible keys.
      float x[2][16];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) x[kt][r] = s[kt][r] * a.scale_log2;
      const bool edge = (CAUSAL && k0 + kBlockN - 1 > qw) || (k0 + kBlockN > a.Lk);
      if (edge || MASK) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kt + 16 * (r >> 3) + 8 * hf + (r & 7);
            bool hide = key >= a.Lk;
            if (CAUSAL) hide = hide || key > qi;
            if (MASK) hide = hide || ((mbits[2 * kt + (r >> 3)] >> (8 * (r & 7))) & 0xff) == 0;
            if (hide) x[kt][r] = -INFINITY;
          }
      }

      // Online softmax: new running max over both key halves, rescale, exponentiate.
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

      // P^T operand: chunk c holds keys 16c + 8hf .. 16c + 8hf + 7 of this lane's row.
      bf16x8 pf[4];
#pragma unroll
      for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int u = 0; u < 8; ++u) pf[c][u] = static_cast<__bf16>(x[c >> 1][8 * (c & 1) + u]);

      // O^T += V^T . P^T
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int d = 32 * dt + li;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const bf16x8 vf = __builtin_bit_cast(
              bf16x8, ld16(vt + d * kBlockN + (((2 * c + hf) ^ vswz(d)) * 8)));
          o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[c], o[dt], 0, 0, 0);
        }
      }
    }

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: normalise, safe-softmax zeros, store O and the LSE ----
  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
    uint16_t* orow = ob + int64_t(qi) * a.so[2];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        // registers 4g..4g+3 hold head dims 32dt + 8g + 4hf + 0..3
        uint32_t w[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const __bf16 lo = static_cast<__bf16>(o[dt][4 * g + 2 * e] * inv);
          const __bf16 hi = static_cast<__bf16>(o[dt][4 * g + 2 * e + 1] * inv);
          w[e] = uint32_t(__builtin_bit_cast(uint16_t, lo)) |
                 (uint32_t(__builtin_bit_cast(uint16_t, hi)) << 16);
        }
        *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * g + 4 * hf) = u32x2{w[0], w[1]};
      }
    if (a.lse && hf == 0)
      a.lse[bh * a.Lq + qi] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}

// ---------------------------------------------------------------------------------------
// fp32 kernel: fp32 MFMA 32x32x2 (true fp32 products, fp32 accumulation) for both
// products; same decomposition as the bf16 kernel, probabilities stay fp32.
// ---------------------------------------------------------------------------------------
template <int D, bool CAUSAL, bool MASK>
__global__ __launch_bounds__(kThreads) void fwd_f32(Args a) {
  constexpr int DG = D / 4;                             // 16-byte groups per row
  constexpr int CH = kBlockN * DG / kThreads;           // chunks per thread per tile
  constexpr int KROW = D + 1;                           // odd pitch: conflict-free column reads
  constexpr int K_ELEMS = kBlockN * KROW;
  constexpr int V_ELEMS = kBlockN * D;
  constexpr int STAGE = K_ELEMS + V_ELEMS;
  static_assert(CH * kThreads == kBlockN * DG, "tile must split evenly over threads");
  __shared__ __attribute__((aligned(16))) float lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int hf = lane >> 5;

  int64_t bh, qt;
  decode_item(blockIdx.x, a.bh_count, a.q_tiles, CAUSAL, &bh, &qt);
  const int64_t b = bh / a.H, h = bh - (bh / a.H) * a.H;
  const float* qb = static_cast<const float*>(a.q) + b * a.sq[0] + h * a.sq[1];
  const float* kb = static_cast<const float*>(a.k) + b * a.sk[0] + h * a.sk[1];
  const float* vb = static_cast<const float*>(a.v) + b * a.sv[0] + h * a.sv[1];
  float* ob = static_cast<float*>(a.out) + b * a.so[0] + h * a.so[1];
  const uint8_t* mb = MASK ? a.mask + b * a.sm[0] + h * a.sm[1] : nullptr;

  const int q0 = int(qt) * kBlockM;
  const int qw = q0 + wave * 32;
  const int qi = qw + li;
  const bool q_ok = qi < a.Lq;
  const bool wave_live = qw < a.Lq;

  // Q^T operand: chunk c supplies head dim 2c + hf.
  float qf[D / 2];
#pragma unroll
  for (int c = 0; c < D / 2; ++c) qf[c] = q_ok ? qb[int64_t(qi) * a.sq[2] + 2 * c + hf] : 0.f;

  int kend = a.Lk;
  if (CAUSAL) kend = min(kend, min(q0 + kBlockM, a.Lq));
  const int ntiles = (kend + kBlockN - 1) / kBlockN;

  u32x4 kreg[CH], vreg[CH];
  auto load_tile = [&](int t) {
    const int k0 = t * kBlockN;
#pragma unroll
    for (int p = 0; p < CH; ++p) {
      const int c = tid + p * kThreads;
      const int row = c / DG, col = (c % DG) * 4;
      const int key = k0 + row;
      const bool ok = key < a.Lk;
      kreg[p] = ok ? ld16(kb + int64_t(key) * a.sk[2] + col) : u32x4{0, 0, 0, 0};
      vreg[p] = ok ? ld16(vb + int64_t(key) * a.sv[2] + col) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_tile = [&](int buf) {
    float* ks = lds + buf * STAGE;
    float* vs = ks + K_ELEMS;
#pragma unroll
    for (int p = 0; p < CH; ++p) {
      const int c = tid + p * kThreads;
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
    const int buf = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const float* ks = lds + buf * STAGE;
    const float* vs = ks + K_ELEMS;
    const int k0 = t * kBlockN;
    const bool tile_live = wave_live && (!CAUSAL || k0 <= qw + 31);

    if (tile_live) {
      // S^T = K . Q^T ; lane (li, hf) register r of sub-tile kt holds key
      // k0 + 32kt + 8(r/4) + 4hf + r%4 of query row qi.
      f32x16 s[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kt][r] = 0.f;
        const bool sub_live = !CAUSAL || (k0 + 32 * kt <= qw + 31);
        if (sub_live) {
#pragma unroll
          for (int c = 0; c < D / 2; ++c)
            s[kt] = __builtin_amdgcn_mfma_f32_32x32x2f32(ks[(32 * kt + li) * KROW + 2 * c + hf],
                                                         qf[c], s[kt], 0, 0, 0);
        }
      }

      float x[2][16];
      const bool edge = (CAUSAL && k0 + kBlockN - 1 > qw) || (k0 + kBlockN > a.Lk);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float xv = s[kt][r] * a.scale_log2;
          if (edge || MASK) {
            const int key = k0 + 32 * kt + 8 * (r >> 2) + 4 * hf + (r & 3);
            bool hide = key >= a.Lk;
            if (CAUSAL) hide = hide || key > qi;
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

    if (t + 1 < ntiles) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = pair_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (q_ok) {
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
      a.lse[bh * a.Lq + qi] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}

template <int D, bool CAUSAL, bool MASK>
hipError_t launch(const Args& a, int dtype, unsigned grid, hipStream_t stream) {
  void* args[] = {const_cast<Args*>(&a)};
  const void* fn = dtype == 1 ? reinterpret_cast<const void*>(&fwd_bf16<D, CAUSAL, MASK>)
                              : reinterpret_cast<const void*>(&fwd_f32<D, CAUSAL, MASK>);
  return hipLaunchKernel(fn, dim3(grid), dim3(kThreads), args, 0, stream);
}

template <int D>
hipError_t launch_d(const Args& a, int dtype, bool causal, unsigned grid, hipStream_t s) {
  const bool m = a.mask != nullptr;
  if (causal) return m ? launch<D, true, true>(a, dtype, grid, s) : launch<D, true, false>(a, dtype, grid, s);
  return m ? launch<D, false, true>(a, dtype, grid, s) : launch<D, false, false>(a, dtype, grid, s);
}

}  // namespace

hipError_t launch_fwd(const Problem& p, hipStream_t stream) {
  Args a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.out = p.out;
  a.lse = p.lse;
  a.mask = p.mask;
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
  a.q_tiles = int32_t((p.Lq + kBlockM - 1) / kBlockM);
  a.bh_count = int32_t(p.B * p.H);
  a.scale_log2 = p.scale * kLog2e;
  a.mask_vec8 = p.mask && (reinterpret_cast<uintptr_t>(p.mask) % 8 == 0) && p.sm[0] % 8 == 0 &&
                p.sm[1] % 8 == 0 && p.sm[2] % 8 == 0;
  const unsigned grid = unsigned(int64_t(a.q_tiles) * a.bh_count);
  if (p.D == 64) return launch_d<64>(a, p.dtype, p.causal != 0, grid, stream);
  return launch_d<128>(a, p.dtype, p.causal != 0, grid, stream);
}

}  // namespace sdpa
