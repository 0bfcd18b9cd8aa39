// sdpa_bwd_gfx950.hip -- gradients of the fused scaled-dot-product attention for MI355X
// (gfx950), bf16 or fp16 inputs and outputs.
//
// The forward is out = P v with P the row softmax of S = scale * q.k^T over the visible
// keys ("Profiling in PyTorch (part 3): attention", naive causal attention, five steps).
// Its derivative for an upstream gradient dO, by the chain rule through those steps:
//   dV = P^T dO,   dP = dO v^T,   dS = P * (dP - delta),   delta_i = sum_j P_ij dP_ij,
//   dQ = scale * dS k,   dK = scale * dS^T q.
// Because out = P v, delta_i also equals sum_d dO_id out_id, which costs one pass over
// dO and out instead of a pass over P.  P itself is rebuilt from the scores and the
// per-row log-sum-exp the forward exported (the fused forward of "[flashinfer] FlashInfer,
// Cake DSA 커널 최적화: Sparse Attention 성능 2배 향상" returns its lse for the backward,
// section 2): P_ij = exp(scale q_i.k_j - lse_i), zero at hidden positions and
// in rows with lse = -inf (no visible key), so the [L, L] matrices never reach memory.
//
// Two kernels, launched back to back on one stream, with no atomics and no workspace
// beyond delta:
//   * dq kernel: a workgroup owns 256 query rows of one (b, h), 32 per wave, and walks
//     the key tiles; lane = query, exactly as in the forward: S^T = K Q^T and
//     dP^T = V dO^T give each lane 16 keys of its own row, so lse and delta are per-lane
//     scalars, and dQ^T += K^T dS^T accumulates in registers.  It also computes delta
//     from its dO and out rows and stores it for the second kernel.
//   * dkdv kernel: a workgroup owns 128 keys, 32 per pair of waves, and walks the query
//     tiles; lane = key: S = Q K^T and dP = dO V^T give each lane 16 queries of its own
//     key's column; one wave of the pair accumulates dV^T += dO^T P, the other
//     dK^T += Q^T dS.
// Each of the streamed tiles (K, V in the first kernel; Q, dO in the second) is the
// left operand of one product (rows of 16 bytes, ds_read_b128) and, for K, Q and dO,
// the transposed left operand of another (ds_read_b64_tr_b16).  The two read patterns
// want different LDS row paddings for conflict-free banks, so such a tile is stored
// twice per stage, once in each layout.
#include <math.h>

#include <type_traits>

#include "sdpa_internal.h"

namespace sdpa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

constexpr float kLog2e = 1.4426950408889634f;
// Word 3 of a raw buffer resource on gfx9: 32-bit data format, no swizzle, no stride;
// reads past num_records return zero.
constexpr int kBufferFlags = 0x00020000;
constexpr int kWaitVmcnt0 = 0x0F70;

struct BwdArgs {
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
  const float* bias;     // additive mask (fp32), addressed with the mask strides
  const int32_t* cu_q;   // packed sequences: sequence s owns query tokens cu_q[s] ..
  const int32_t* cu_k;   // cu_q[s+1]-1 and key tokens cu_k[s] .. cu_k[s+1]-1
  int64_t sq[3], sk[3], sv[3], so[3], sdo[3], sdq[3], sdk[3], sdv[3], sm[3];
  int32_t H, Lq, Lk, q_items, k_items, bh_count;
  float scale;       // multiplies dQ and dK
  float scale_log2;  // scale * log2(e): scores in base-2 units
  int32_t mask_vec8; // mask rows may be read 8 bytes at a time
  int32_t coff;      // causal (dense heads): key j visible to query i iff j <= i + coff
  int32_t bottom_right;  // causal alignment of packed sequences, per sequence
  int32_t bias_vec4;     // bias rows may be read 16 bytes at a time
};

// How a launch maps work items to rows: dense (b, h) heads of the strided tensors, or
// head h of packed sequence s of [tokens, H, D] tensors (lse and delta laid out [H, total
// query tokens]).  MK: 0 no mask, 1 boolean mask, 2 additive mask (dense heads only).
enum { kBwdDense = 0, kBwdVarlen = 1 };

// The rows of one (sequence or batch entry, head): element offsets of row 0 in each
// tensor, of the mask, and of its lse / delta, its row counts and causal offset.  Packed
// offsets are clamped into [0, total] and made non-decreasing, so that any contents of
// cu_q / cu_k keep every access in bounds.
struct BwdItem {
  int64_t q, k, v, o, dO, dq, dk, dv, m, lse;
  int Lq, Lk, coff;
};

template <int MODE>
__device__ inline BwdItem bwd_item(const BwdArgs& a, int64_t bh) {
  BwdItem it;
  const int64_t s = bh / a.H, h = bh - (bh / a.H) * a.H;
  if (MODE == kBwdDense) {
    it.q = s * a.sq[0] + h * a.sq[1];
    it.o = s * a.so[0] + h * a.so[1];
    it.dO = s * a.sdo[0] + h * a.sdo[1];
    it.dq = s * a.sdq[0] + h * a.sdq[1];
    it.k = s * a.sk[0] + h * a.sk[1];
    it.v = s * a.sv[0] + h * a.sv[1];
    it.dk = s * a.sdk[0] + h * a.sdk[1];
    it.dv = s * a.sdv[0] + h * a.sdv[1];
    it.m = s * a.sm[0] + h * a.sm[1];
    it.lse = bh * a.Lq;
    it.Lq = a.Lq;
    it.Lk = a.Lk;
    it.coff = a.coff;
  } else {
    const int q_lo = min(max(a.cu_q[s], 0), a.Lq), q_hi = min(max(a.cu_q[s + 1], q_lo), a.Lq);
    const int k_lo = min(max(a.cu_k[s], 0), a.Lk), k_hi = min(max(a.cu_k[s + 1], k_lo), a.Lk);
    it.q = q_lo * a.sq[2] + h * a.sq[1];
    it.o = q_lo * a.so[2] + h * a.so[1];
    it.dO = q_lo * a.sdo[2] + h * a.sdo[1];
    it.dq = q_lo * a.sdq[2] + h * a.sdq[1];
    it.k = k_lo * a.sk[2] + h * a.sk[1];
    it.v = k_lo * a.sv[2] + h * a.sv[1];
    it.dk = k_lo * a.sdk[2] + h * a.sdk[1];
    it.dv = k_lo * a.sdv[2] + h * a.sdv[1];
    it.m = 0;
    it.lse = h * a.Lq + q_lo;
    it.Lq = q_hi - q_lo;
    it.Lk = k_hi - k_lo;
    it.coff = a.bottom_right ? it.Lk - it.Lq : 0;
  }
  return it;
}

__device__ inline u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// A raw buffer resource (base, no stride, extent in bytes) as four scalar registers, for
// the loads below that are written in asm.
__device__ inline u32x4 buffer_desc(const void* base, int extent) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  return u32x4{uint32_t(b), uint32_t(b >> 32) & 0xFFFFu, uint32_t(extent), uint32_t(kBufferFlags)};
}
// A 16-byte buffer load per lane that writes the LDS instead of registers: lane l fills
// bytes lds_dst + 16l .. +15 (lds_dst wave-uniform), offsets past the extent fill zeros.
// The compiler does not see the LDS write: the caller waits for the memory counter before
// the barrier that publishes the data, and issues no such load into LDS still being read.
// On gfx9 an LDS-writing load reads M0 one wait state after a scalar write of it at the
// earliest (the compiler keeps that distance for its own such loads), hence the s_nop.
// M0 is named as clobbered although the compiler reserves it (and warns so): nothing in
// these kernels reads M0 but these loads.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void buffer_to_lds16(const u32x4& desc, uint32_t lds_dst, int offset) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds_dst), "v"(offset), "s"(desc) : "memory", "m0");
}
#pragma clang diagnostic pop
// LDS address of a shared-memory pointer, as the 32-bit value the hardware takes.
__device__ inline uint32_t lds_addr(const void* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)p));
}

__device__ inline float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ inline s16x4 ds_read_tr(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p));
}

// Swaps bits 2 and 3 of a row index within 32 rows.  Reading the rows of a left operand
// in this order makes the 32x32 accumulator hold, in half h of the lanes, rows 8h..8h+7
// in registers 0..7 and 16+8h..16+8h+7 in registers 8..15: runs of 8 consecutive rows,
// the operand layout the next product needs along its reduction dimension.
__device__ inline int perm5(int m) { return (m & 0x13) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Base-2 log-sum-exp of a row, from the forward's natural-log value; rows with no
// visible key (lse = -inf) get +inf so that every probability of the row is 2^-inf = 0.
__device__ inline float lse_base2(float lse) { return lse == -INFINITY ? INFINITY : lse * kLog2e; }

// The 16-bit input types (bf16 or fp16): operand vectors, the 32x32x16 product of that
// type, and two fp32 values rounded to it (nearest-even) and packed low-first.
template <typename E> struct Vec16;
template <> struct Vec16<__bf16> { typedef bf16x8 v8; typedef bf16x2 v2; };
template <> struct Vec16<_Float16> { typedef f16x8 v8; typedef f16x2 v2; };

__device__ inline f32x16 mfma16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ inline f32x16 mfma16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

template <typename E>
__device__ inline uint32_t pack2(float lo, float hi) {
  const f32x2 p = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(p, typename Vec16<E>::v2));
}
template <typename E>
__device__ inline f32x2 unpack2(uint32_t w) {
  return __builtin_convertvector(__builtin_bit_cast(typename Vec16<E>::v2, w), f32x2);
}

// The transposed operand of a 32x32x16 product from a row-major tile in LDS: rows are
// the reduction index, columns the output rows.  Within each group of 16 lanes, lane i of
// ds_read_b64_tr_b16 receives element i mod 4 of the 8-byte pieces addressed by lanes
// 4e + i/4 (e = 0..3); addressing tile[row0 + e][col0 + 4q] from lane 4e + q therefore
// hands lane i column col0 + i of four consecutive rows.  `tfrag` is that per-lane
// address for row0 = 8 * (lane / 32), col0 = 16 * ((lane / 16) % 2); the operand of
// reduction chunk c (rows 16c + 8h + 0..7 in half h) and output block dt (columns
// 32dt + lane % 32) is two such reads, 4 rows apart.
template <typename V, int PITCH>
__device__ inline V tr_operand(const char* tfrag, int c, int dt) {
  const s16x4 lo = ds_read_tr(tfrag + (16 * c) * PITCH + 64 * dt);
  const s16x4 hi = ds_read_tr(tfrag + (16 * c + 4) * PITCH + 64 * dt);
  const s16x4 both[2] = {lo, hi};
  return __builtin_bit_cast(V, both);
}

__device__ inline int tr_lane_offset(int lane, int pitch) {
  const int g16 = lane >> 4, e4 = (lane >> 2) & 3, q4 = lane & 3;
  return (8 * (g16 >> 1) + e4) * pitch + (16 * (g16 & 1) + 4 * q4) * 2;
}

// Stores a wave's 32 x D accumulator block set (registers 4g..4g+3 of block dt hold
// columns 32dt + 8g + 4h + 0..3 of the lane's row), multiplied by `mul`, in the 16-bit type
// E, through LDS so that the global stores cover whole rows: tile_to_lds puts the 32 rows
// (pitch P bytes) into `ot`; after a workgroup barrier, rows_to_global stores them, lane l
// taking 16-byte chunks l, l + 64, ... of the row-major tile, rows row0 + r < nrows only.
template <typename E, int D, int P>
__device__ inline void tile_to_lds(char* ot, const f32x16 (&acc)[D / 32], float mul, int li,
                                   int hf) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t w0 = pack2<E>(acc[dt][4 * g] * mul, acc[dt][4 * g + 1] * mul);
      const uint32_t w1 = pack2<E>(acc[dt][4 * g + 2] * mul, acc[dt][4 * g + 3] * mul);
      *reinterpret_cast<u32x2*>(ot + li * P + (32 * dt + 8 * g + 4 * hf) * 2) = u32x2{w0, w1};
    }
}
template <int D, int P>
__device__ inline void rows_to_global(const char* ot, int lane, int row0, int nrows,
                                      uint16_t* base, int64_t stride) {
  constexpr int DG = D / 8;
  static_assert((32 * DG) % 64 == 0, "row chunks split evenly over a wave");
#pragma unroll
  for (int i = 0; i < 32 * DG / 64; ++i) {
    const int c = i * 64 + lane, r = c / DG, col = c % DG;
    const u32x4 w = *reinterpret_cast<const u32x4*>(ot + r * P + col * 16);
    if (row0 + r < nrows) *reinterpret_cast<u32x4*>(base + int64_t(row0 + r) * stride + col * 8) = w;
  }
}

// Staging map of a streamed tile of R rows x DG 16-byte chunks over NT threads: chunk p of
// thread tid is chunk tid + p * NT of the row-major tile, at byte offset off(p, pitch) for a
// row pitch of `pitch` bytes (in global memory or LDS).  When the tile splits evenly
// (NT a multiple of DG and of the tile) chunk p sits NT / DG rows below chunk 0; otherwise
// (D = 32, 96) the chunks past the tile's end are skipped -- whole waves, since R * DG is a
// multiple of 64.
template <int R, int DG, int NT>
struct StageMap {
  static constexpr bool kEven = (R * DG) % NT == 0 && NT % DG == 0;
  int tid, row0, col0;
  __device__ explicit StageMap(int t) : tid(t), row0(t / DG), col0(t % DG) {}
  __device__ bool ok(int p) const { return kEven || tid + p * NT < R * DG; }
  __device__ int off(int p, int pitch) const { return row(p) * pitch + col(p) * 16; }
  __device__ int row(int p) const { return kEven ? row0 + p * (NT / DG) : (tid + p * NT) / DG; }
  __device__ int col(int p) const { return kEven ? col0 : (tid + p * NT) % DG; }
};

// ---------------------------------------------------------------------------------------
// dq kernel.  Workgroup: 256 query rows of one (b, h) in 8 waves, two per SIMD, so that
// one wave's vector work and operand reads overlap the other's products; wave w owns
// rows q0 + 32w + 0..31,
// lane (li, hf) row q0 + 32w + li and head-dim half hf of each 16-wide chunk.  Per key
// tile of 64 (two 32-key sub-tiles kt):
//   S^T[kt]  = K[kt] Q^T        (K rows read in perm5 order: register r of half hf is key
//   dP^T[kt] = V[kt] dO^T        32kt + 16(r/8) + 8hf + r%8)
//   dS^T     = P^T * (dP^T - delta),  P^T = 2^(S^T scale log2e - lse2), hidden -> 0
//   dQ^T    += K^T dS^T          (K^T by transposed reads, dS^T rounded to the input type)
// LDS stage: K row copy | K transposed-read copy | V row copy.
// ---------------------------------------------------------------------------------------
template <typename E, int D, bool CAUSAL, int MK, int MODE>
__global__ __launch_bounds__(kThreadsBwdQ) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dq(BwdArgs a) {
  constexpr bool MASK = MK == 1, BIAS = MK == 2;
  typedef typename Vec16<E>::v8 v8;
  constexpr int BN = kBwdStep;
  constexpr int NT = kThreadsBwdQ;
  constexpr int DG = D / 8;           // 16-byte chunks per row
  constexpr int CH = (BN * DG + NT - 1) / NT;  // chunks per thread per tile
  constexpr int RP = k_pitch_bf16(D); // row-read pitch (bytes)
  constexpr int TP = v_pitch_bf16(D); // transposed-read pitch (bytes)
  constexpr int OFF_KT = BN * RP;
  constexpr int OFF_V = OFF_KT + BN * TP;
  constexpr int STAGE = OFF_V + BN * RP;
  static_assert(2 * STAGE == lds_bytes_bwd_dq(D), "plan and kernel disagree on LDS");
  __shared__ __attribute__((aligned(16))) char lds[2 * STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int li = lane & 31;
  const int hf = lane >> 5;

  int64_t bh, qt;
  decode_item(blockIdx.x, a.bh_count, a.q_items, CAUSAL, &bh, &qt);
  const BwdItem it = bwd_item<MODE>(a, bh);
  const int Lq = it.Lq, Lk = it.Lk;
  const int q0 = int(qt) * kBwdBlockQ;
  if (MODE == kBwdVarlen && q0 >= Lq) return;  // a tile past this sequence's rows
  const uint16_t* qb = static_cast<const uint16_t*>(a.q) + it.q;
  const uint16_t* ob = static_cast<const uint16_t*>(a.out) + it.o;
  const uint16_t* dob = static_cast<const uint16_t*>(a.dout) + it.dO;
  const char* kb = static_cast<const char*>(a.k) + 2 * it.k;
  const char* vb = static_cast<const char*>(a.v) + 2 * it.v;
  uint16_t* dqb = static_cast<uint16_t*>(a.dq) + it.dq;
  const uint8_t* mb = MASK ? a.mask + it.m : nullptr;
  const float* bb = BIAS ? a.bias + it.m : nullptr;

  const int qw = q0 + 32 * wave;
  const int qi = qw + li;
  const bool q_ok = qi < Lq;
  const bool wave_live = qw < Lq;

  // Q^T and dO^T operands (chunk c = head dims 16c..16c+15, half hf supplies 8 of them),
  // and delta = dO . out of this row from the same halves of dO and out.
  v8 qf[D / 16], dof[D / 16];
  float dpart = 0.f;
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    u32x4 wq = {0, 0, 0, 0}, wd = {0, 0, 0, 0}, wo = {0, 0, 0, 0};
    if (q_ok) {
      wq = ld16(qb + int64_t(qi) * a.sq[2] + 16 * c + 8 * hf);
      wd = ld16(dob + int64_t(qi) * a.sdo[2] + 16 * c + 8 * hf);
      wo = ld16(ob + int64_t(qi) * a.so[2] + 16 * c + 8 * hf);
    }
    qf[c] = __builtin_bit_cast(v8, wq);
    dof[c] = __builtin_bit_cast(v8, wd);
    const v8 of = __builtin_bit_cast(v8, wo);
#pragma unroll
    for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf(float(dof[c][e]), float(of[e]), dpart);
  }
  const float delta = pair_sum(dpart);
  const float lse2 = q_ok ? lse_base2(a.lse[it.lse + qi]) : INFINITY;
  if (q_ok && hf == 0) a.delta[it.lse + qi] = delta;
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  const int coff = it.coff;
  int kend = Lk;
  if (CAUSAL) kend = max(0, min(kend, min(q0 + kBwdBlockQ, Lq) + coff));
  const int ntiles = (kend + BN - 1) / BN;
  const int wlast = qw + 31 + coff;  // last key any row of the wave may see (causal)
  const int wtiles = !wave_live ? 0 : CAUSAL ? (wlast < 0 ? 0 : min(ntiles, wlast / BN + 1)) : ntiles;

  // Staging of K and V: buffer loads with the whole byte offset in the per-lane offset,
  // checked by the hardware against the head's extent (rows past the end read zero; a
  // tile index past the staged range is sent beyond the extent).  Offsets stay below
  // 2^31: (Lk + 64) rows of K and of V span less than 2 GiB.
  const int k_rowb = int(a.sk[2]) * 2, v_rowb = int(a.sv[2]) * 2;
  const int k_ext = Lk > 0 ? (Lk - 1) * k_rowb + 2 * D : 0;
  const int v_ext = Lk > 0 ? (Lk - 1) * v_rowb + 2 * D : 0;
  const __amdgpu_buffer_rsrc_t krs = __builtin_amdgcn_make_buffer_rsrc((void*)kb, 0, k_ext, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc((void*)vb, 0, v_ext, kBufferFlags);
  const StageMap<BN, DG, NT> sm_(tid);
  u32x4 kreg[CH], vreg[CH];
  auto load = [&](int t) {
    const int kbase = t < ntiles ? t * BN * k_rowb : k_ext;
    const int vbase = t < ntiles ? t * BN * v_rowb : v_ext;
#pragma unroll
    for (int p = 0; p < CH; ++p)
      if (sm_.ok(p)) {
        kreg[p] = __builtin_amdgcn_raw_buffer_load_b128(krs, kbase + sm_.off(p, k_rowb), 0, 0);
        vreg[p] = __builtin_amdgcn_raw_buffer_load_b128(vrs, vbase + sm_.off(p, v_rowb), 0, 0);
      }
  };
  auto store = [&](int st) {
    char* s = lds + st * STAGE;
#pragma unroll
    for (int p = 0; p < CH; ++p)
      if (sm_.ok(p)) {
        *reinterpret_cast<u32x4*>(s + sm_.off(p, RP)) = kreg[p];
        *reinterpret_cast<u32x4*>(s + OFF_KT + sm_.off(p, TP)) = kreg[p];
        *reinterpret_cast<u32x4*>(s + OFF_V + sm_.off(p, RP)) = vreg[p];
      }
  };

  const int rfrag = perm5(li) * RP + hf * 16;  // left-operand row of this lane
  const int tfrag = tr_lane_offset(lane, TP);
  const float c2 = a.scale_log2;

  f32x16 dq[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) dq[dt][r] = 0.f;

  auto compute = [&](int t) {
    const char* st = lds + (t & 1) * STAGE;
    const int k0 = t * BN;
    f32x16 s[2], dp[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kt][r] = dp[kt][r] = 0.f;
    // Products i = 4c + 2kt + {0: S, 1: dP}, their K or V operand read two products
    // ahead; the fences keep that order.
    constexpr int NP = 4 * (D / 16);
    v8 fa[3];
    auto fread = [&](int i) {
      const int c = i >> 2, kt = (i >> 1) & 1;
      fa[i % 3] = __builtin_bit_cast(
          v8, ld16(st + ((i & 1) ? OFF_V : 0) + rfrag + kt * 32 * RP + 32 * c));
    };
    __builtin_amdgcn_sched_barrier(0);
    fread(0);
    fread(1);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + 2 < NP) fread(i + 2);
      const int c = i >> 2, kt = (i >> 1) & 1;
      if (i & 1) dp[kt] = mfma16(fa[i % 3], dof[c], dp[kt]);
      else s[kt] = mfma16(fa[i % 3], qf[c], s[kt]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // x = S scale log2e (+ bias log2e) - lse2 in base-2 units; hidden keys -> -inf.
    float x[2][16];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) x[kt][r] = __builtin_fmaf(s[kt][r], c2, -lse2);
    if (BIAS && q_ok) {
      // the lane's runs of 8 keys: register r of sub-tile kt is key k0 + 32kt + 16(r/8) +
      // 8hf + r%8; keys past Lk read nothing (they are hidden below)
      const float* brow = bb + int64_t(qi) * a.sm[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int g = 0; g < 2; ++g) {
          const int key0 = k0 + 32 * kt + 16 * g + 8 * hf;
          if (a.bias_vec4 && key0 + 8 <= Lk) {
            const f32x4 lo = *reinterpret_cast<const f32x4*>(brow + key0);
            const f32x4 hi = *reinterpret_cast<const f32x4*>(brow + key0 + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              x[kt][8 * g + e] = __builtin_fmaf(lo[e], kLog2e, x[kt][8 * g + e]);
              x[kt][8 * g + e + 4] = __builtin_fmaf(hi[e], kLog2e, x[kt][8 * g + e + 4]);
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e)
              if (key0 + e < Lk)
                x[kt][8 * g + e] = __builtin_fmaf(brow[key0 + e], kLog2e, x[kt][8 * g + e]);
          }
        }
    }
    const bool edge = (CAUSAL && k0 + BN - 1 > qw + coff) || (k0 + BN > Lk);
    if (edge || MASK) {
      uint64_t mbits[4] = {~0ull, ~0ull, ~0ull, ~0ull};
      if (MASK && q_ok) {
        const uint8_t* mrow = mb + int64_t(qi) * a.sm[2];
#pragma unroll
        for (int run = 0; run < 4; ++run) {
          const int key0 = k0 + 32 * (run >> 1) + 16 * (run & 1) + 8 * hf;
          if (a.mask_vec8 && key0 + 8 <= Lk) {
            mbits[run] = *reinterpret_cast<const uint64_t*>(mrow + key0);
          } else {
            uint64_t w = 0;
            for (int e = 0; e < 8; ++e)
              if (key0 + e < Lk) w |= uint64_t(mrow[key0 + e]) << (8 * e);
            mbits[run] = w;
          }
        }
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kt + 16 * (r >> 3) + 8 * hf + (r & 7);
          bool hide = key >= Lk;
          if (CAUSAL) hide = hide || key > qi + coff;
          if (MASK) hide = hide || ((mbits[2 * kt + (r >> 3)] >> (8 * (r & 7))) & 0xff) == 0;
          if (hide) x[kt][r] = -INFINITY;
        }
    }
    // dS^T operand: chunk c = keys 16c + 8hf + 0..7 (registers 8(c%2) .. +7 of kt = c/2)
    v8 dsf[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      u32x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kt = c >> 1, r = 8 * (c & 1) + 2 * e;
        const float d0 = exp2_fast(x[kt][r]) * (dp[kt][r] - delta);
        const float d1 = exp2_fast(x[kt][r + 1]) * (dp[kt][r + 1] - delta);
        w[e] = pack2<E>(d0, d1);
      }
      dsf[c] = __builtin_bit_cast(v8, w);
    }
    // dQ^T += K^T dS^T, operands two products ahead (i = c * (D / 32) + dt)
    const char* ktr = st + OFF_KT + tfrag;
    constexpr int NQ = 4 * (D / 32);
    v8 ta[3];
    auto tread = [&](int i) { ta[i % 3] = tr_operand<v8, TP>(ktr, i / (D / 32), i % (D / 32)); };
    __builtin_amdgcn_sched_barrier(0);
    tread(0);
    tread(1);
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      if (i + 2 < NQ) tread(i + 2);
      dq[i % (D / 32)] = mfma16(ta[i % 3], dsf[i / (D / 32)],
                                                                 dq[i % (D / 32)]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Each tile is loaded right after its predecessor is written to LDS, a whole step
  // before its own store.  The second wave of each SIMD (waves 4..7) stages at the start of
  // the step, while the first one's products hold the matrix core, the first wave at the
  // end, while the second one's products run; stage (t + 1) & 1 was last read at step t - 1.
  load(0);
  store(0);
  load(1);
  __syncthreads();
  const bool stage_first = __builtin_amdgcn_readfirstlane(wave) >= 4;
  for (int t = 0; t < ntiles; ++t) {
    if (stage_first) {
      store((t + 1) & 1);
      load(t + 2);
    }
    if (t < wtiles) compute(t);
    if (!stage_first) {
      store((t + 1) & 1);
      load(t + 2);
    }
    __syncthreads();
  }

  static_assert(8 * 32 * RP <= 2 * STAGE, "the output tiles fit the LDS");
  char* ot = lds + wave * 32 * RP;
  tile_to_lds<E, D, RP>(ot, dq, a.scale, li, hf);
  __syncthreads();
  rows_to_global<D, RP>(ot, lane, qw, Lq, dqb, a.sdq[2]);
}

// ---------------------------------------------------------------------------------------
// Single-copy staging layout of the dK/dV kernel.  A streamed [64 x D] tile is read two
// ways: along a row (16-byte reads of head dims, left operands of S and dP) and down the
// columns (ds_read_b64_tr_b16, left operands of dV^T and dK^T).  Rows have a power-of-two
// number of 16-byte slots (4, 8 or 16; D = 96 takes 16 slots for its 12 chunks), and chunk
// j of row r sits in slot j ^ sw(r).  Within the 16 lanes of one row-read pass (16 rows,
// one chunk) and within the 32 lanes of one transposed-read pass (4 consecutive rows from
// a multiple of 4, 4 consecutive chunks from a multiple of 4) every lane then reaches a
// different 16-byte bank group of the 256-byte bank space; the staging writes (consecutive
// chunks of consecutive rows) do as well.
template <int D>
struct BwdSwz {
  static constexpr int DG = D / 8;                              // 16-byte chunks per row
  static constexpr int SL = DG <= 4 ? 4 : (DG <= 8 ? 8 : 16);   // slots per row
  static constexpr int RB = 16 * SL;                            // row pitch (bytes)
  static constexpr int SH = SL == 16 ? 0 : (SL == 8 ? 1 : 2);
  __device__ static int sw(int r) { return ((r >> 2) & 3) | (((r & 3) >> SH) << 2); }
  __device__ static int at(int r, int j) { return r * RB + 16 * (j ^ sw(r)); }
};

// ---------------------------------------------------------------------------------------
// dkdv kernel.  Workgroup: 128 keys of one (b, h) in 8 waves, two per SIMD.  The two waves
// of a SIMD own the same 32 keys k0 + 32(w % 4) + 0..31 (lane (li, hf): key
// k0 + 32(w % 4) + li) and split the four products of each 64-query tile between them,
// two each, with P handed from one to the other through LDS:
//   P wave:   S[qs] = Q[qs] K^T         (Q rows read in perm5 order: register r of half hf
//                                         is query 32qs + 16(r/8) + 8hf + r%8)
//             P = 2^(S scale log2e - lse2[query]), hidden -> 0, rounded to the input type
//             and written to LDS;  dV^T += dO^T P   (dO^T by transposed reads)
//   dS wave, one tile behind:
//             dP[qs] - delta = dO[qs] V^T + (-delta[query])  (accumulators start at -delta)
//             dS = P * (dP - delta) with P from LDS,  dK^T += Q^T dS   (Q^T by transposed reads)
// Each wave holds one accumulator block and one of K, V, and the two waves of a SIMD meet
// only at the one barrier per tile, so one's vector work (the exponentials; dS) runs under
// the other's products.  Only on the causal diagonal (or with a mask) does the P wave
// test elements.  The dS waves load the Q and dO tiles, the P waves the rows' lse and delta.
// LDS: three stages of [Q | dO | lse2[64] | -delta[64]] in the layout above (the tile the
// P waves compute on, the one the dS waves compute on, the next), then P of two tiles
// (4 KB per SIMD each).  Q and dO go from memory straight into their stage (buffer loads
// that write the LDS), issued by the dS waves at the start of the step before the one in
// which the P waves compute on them.
// ---------------------------------------------------------------------------------------
template <typename E, int D, bool CAUSAL, int MK, int MODE>
__global__ __launch_bounds__(kThreadsBwdK) __attribute__((amdgpu_waves_per_eu(2, 2)))
void bwd_dkdv(BwdArgs a) {
  constexpr bool MASK = MK == 1, BIAS = MK == 2;
  typedef typename Vec16<E>::v8 v8;
  typedef BwdSwz<D> SW;
  constexpr int BQ = kBwdStep;
  constexpr int DG = D / 8;
  constexpr int RB = SW::RB;
  // Stage k: Q at k TILE, dO at (3 + k) TILE, lse2 and -delta at ROWS + k ROWB; then P.
  // Every operand read in the loop is a per-lane base (which includes the Q or dO region)
  // plus an immediate below 64 KB.
  constexpr int NSTAGE = 3;
  constexpr int TILE = BQ * RB;
  constexpr int OFF_DO = NSTAGE * TILE;
  constexpr int ROWS = 2 * NSTAGE * TILE;
  constexpr int ROWB = 8 * BQ;  // lse2[BQ] | -delta[BQ]
  constexpr int OFF_P = ROWS + NSTAGE * ROWB;
  constexpr int PBYTES = 32 * BQ * 2;  // one SIMD's P tile in the input type
  constexpr int LDS_BYTES = OFF_P + 2 * 4 * PBYTES;
  static_assert(LDS_BYTES == lds_bytes_bwd_dkdv(D), "plan and kernel disagree on LDS");
  __shared__ __attribute__((aligned(16))) char lds[LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const bool ds_wave = wave >= 4;  // wave-uniform role
  const int li = lane & 31;
  const int hf = lane >> 5;

  // Key tiles in index order, heads innermost: under a causal mask the first key tiles
  // see the most queries, so the heaviest items are issued first.
  int64_t bh, kt_idx;
  decode_item(blockIdx.x, a.bh_count, a.k_items, false, &bh, &kt_idx);
  const BwdItem it = bwd_item<MODE>(a, bh);
  const int Lq = it.Lq, Lk = it.Lk;
  const int k0 = int(kt_idx) * kBwdBlockK;
  if (MODE == kBwdVarlen && k0 >= Lk) return;  // a tile past this sequence's keys
  const char* qb = static_cast<const char*>(a.q) + 2 * it.q;
  const char* dob = static_cast<const char*>(a.dout) + 2 * it.dO;
  const uint16_t* kb = static_cast<const uint16_t*>(a.k) + it.k;
  const uint16_t* vb = static_cast<const uint16_t*>(a.v) + it.v;
  uint16_t* dkb = static_cast<uint16_t*>(a.dk) + it.dk;
  uint16_t* dvb = static_cast<uint16_t*>(a.dv) + it.dv;
  const uint8_t* mb = MASK ? a.mask + it.m : nullptr;
  const float* bb = BIAS ? a.bias + it.m : nullptr;
  const float* lse_h = a.lse + it.lse;
  const float* del_h = a.delta + it.lse;

  const int kw = k0 + 32 * (wave & 3);
  const int kj = kw + li;
  const bool k_ok = kj < Lk;
  const bool wave_live = kw < Lk;

  // Right operand of the wave's first product: K^T (S, P wave) or V^T (dP, dS wave);
  // column = this lane's key, half hf supplies head dims 16c + 8hf .. +7 of chunk c.
  v8 kvf[D / 16];
  {
    const uint16_t* src = ds_wave ? vb : kb;
    const int64_t rs = ds_wave ? a.sv[2] : a.sk[2];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      u32x4 w = {0, 0, 0, 0};
      if (k_ok) w = ld16(src + int64_t(kj) * rs + 16 * c + 8 * hf);
      kvf[c] = __builtin_bit_cast(v8, w);
    }
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);

  // Query tiles of the walk: with a causal mask, queries i with i + coff < k0 see none of
  // the keys.
  const int coff = it.coff;
  const int ntiles = (Lq + BQ - 1) / BQ;
  const int tbeg = CAUSAL ? min(max(0, k0 - coff) / BQ, ntiles) : 0;

  const int q_rowb = int(a.sq[2]) * 2, d_rowb = int(a.sdo[2]) * 2;
  const int q_ext = Lq > 0 ? (Lq - 1) * q_rowb + 2 * D : 0;
  const int d_ext = Lq > 0 ? (Lq - 1) * d_rowb + 2 * D : 0;
  // A tile of Q (dO) fills RB * BQ / 1024 blocks of 1 KB of its stage, block b loaded by
  // dS wave b % 4: lane l of the load writes bytes 16l..16l+15 of the block and reads the
  // chunk that the swizzled layout puts there (row r, slot s hold chunk s ^ sw(r)); slots
  // past the row's DG chunks read past the extent, zeros.
  constexpr int NDMA = RB * BQ / 4096;  // blocks per loading (dS) wave and tensor
  static_assert(RB * BQ % 4096 == 0, "whole blocks for every loading wave");
  int qoff[NDMA], doff[NDMA];
#pragma unroll
  for (int p = 0; p < NDMA; ++p) {
    const int pos = (4 * p + (wave & 3)) * 1024 + 16 * lane;
    const int r = pos / RB, j = (pos % RB) / 16 ^ SW::sw(r);
    qoff[p] = j < DG ? r * q_rowb + 16 * j : -1;
    doff[p] = j < DG ? r * d_rowb + 16 * j : -1;
  }
  const u32x4 qdesc = buffer_desc(qb, q_ext), ddesc = buffer_desc(dob, d_ext);
  const uint32_t dma_base = lds_addr(lds) + uint32_t((wave & 3) * 1024);
  // Q and dO of tile t into stage st (dS waves; the LDS address must be wave-uniform)
  auto load_tile = [&](int t, int st) {
#pragma unroll
    for (int p = 0; p < NDMA; ++p) {
      const uint32_t dst =
          __builtin_amdgcn_readfirstlane(dma_base + uint32_t(st * TILE + 4 * p * 1024));
      buffer_to_lds16(qdesc, dst, qoff[p] >= 0 ? t * BQ * q_rowb + qoff[p] : q_ext);
      buffer_to_lds16(ddesc, dst + OFF_DO, doff[p] >= 0 ? t * BQ * d_rowb + doff[p] : d_ext);
    }
  };
  // threads 0..63: lse of row tid; 64..127: delta of row tid - 64 (as loaded; converted
  // when stored, so the load is waited for one tile later)
  float rowval = 0.f;
  auto load = [&](int t) {
    const bool live = t < ntiles;
    if (tid < 2 * BQ) {
      const int row = t * BQ + (tid & (BQ - 1));
      const bool ok = live && row < Lq;
      if (tid < BQ) rowval = ok ? lse_h[row] : -INFINITY;
      else rowval = ok ? del_h[row] : 0.f;
    }
  };
  auto store = [&](int st) {
    // lse2 of the rows, and -delta (the initial value of the dP accumulators)
    if (tid < 2 * BQ)
      reinterpret_cast<float*>(lds + ROWS + st * ROWB)[tid] = tid < BQ ? lse_base2(rowval) : -rowval;
  };

  // Row reads: lane row perm5(li) (+ 32qs), chunk 2c + hf.  Transposed reads: rows
  // 16c + 8(lane / 32) + 4h + (lane / 4) % 4, chunks 4dt + 2((lane / 16) % 2) + (lane % 4) / 2.
  // Row reads (Q for the P wave, dO for the dS wave) and transposed reads (dO for the P
  // wave, Q for the dS wave): per-lane bases into the stage the wave computes on (moved to
  // the next stage after each step), plus immediates below 64 KB.  The empty asm keeps the
  // compiler from rebuilding the bases from the loop-invariant parts (a register each).
  int raddr[D / 16];
  {
    const int r = perm5(li), region = ds_wave ? OFF_DO : 0;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      raddr[c] = region + SW::at(r, 2 * c + hf);
      asm("" : "+v"(raddr[c]));
    }
  }
  int taddr[2][D / 32];
  {
    const int g16 = lane >> 4, e4 = (lane >> 2) & 3, q4 = lane & 3;
    const int region = ds_wave ? 0 : OFF_DO;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        taddr[h][dt] = region + 8 * (q4 & 1) +
                       SW::at(8 * (g16 >> 1) + 4 * h + e4, 4 * dt + 2 * (g16 & 1) + (q4 >> 1));
        asm("" : "+v"(taddr[h][dt]));
      }
  }
  const float c2 = a.scale_log2;
  // P of tile t: slot t % 2, chunk c at + c * 1024
  char* pex0 = lds + OFF_P + (wave & 3) * PBYTES + lane * 16;

  // dV^T (P wave) or dK^T (dS wave)
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;

  // The wave's product over head dims for sub-tile qs: S (P wave, Q rows) or dP (dS wave,
  // dO rows); operands are read two chunks ahead, fenced so the scheduler keeps that order.
  auto dim_product2 = [&](f32x16 (&x)[2]) {
    const char* rows = lds;
    constexpr int NR = 2 * (D / 16);  // reads, i = 2c + qs
    v8 opa[4];
    auto read = [&](int i) {
      opa[i % 4] = __builtin_bit_cast(v8, ld16(rows + raddr[i / 2] + (i % 2) * 32 * RB));
    };
    read(0);
    read(1);
    read(2);
#pragma unroll
    for (int i = 0; i < NR; ++i) {
      if (i + 3 < NR) read(i + 3);
      x[i % 2] = mfma16(opa[i % 4], kvf[i / 2], x[i % 2]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // acc += T^T op over the tile's 64 queries, T = dO (P wave) or Q (dS wave) by transposed
  // reads; op chunk c = queries 16c + 8hf + 0..7 (P or dS in the input type).
  auto query_product = [&](const v8 (&op)[4]) {
    const char* rows = lds;
    constexpr int NP = 4 * (D / 32);  // products, i = c * (D / 32) + dt
    v8 ta[3];
    auto tread = [&](int i) {
      const int c = i / (D / 32), dt = i % (D / 32);
      const s16x4 lo = ds_read_tr(rows + taddr[0][dt] + 16 * c * RB);
      const s16x4 hi = ds_read_tr(rows + taddr[1][dt] + 16 * c * RB);
      const s16x4 both[2] = {lo, hi};
      ta[i % 3] = __builtin_bit_cast(v8, both);
    };
    __builtin_amdgcn_sched_barrier(0);
    tread(0);
    tread(1);
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + 2 < NP) tread(i + 2);
      acc[i % (D / 32)] = mfma16(ta[i % 3], op[i / (D / 32)], acc[i % (D / 32)]);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  // A wave's keys are visible to some query of tile t iff the tile's last query + coff >= kw.
  auto tile_live = [&](int t) { return wave_live && (!CAUSAL || t * BQ + BQ - 1 + coff >= kw); };
  // Points the operand bases at stage k (from stage 0) / moves them on from stage k to the
  // next one.
  auto bases_add = [&](int bytes) {
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      raddr[c] += bytes;
      asm("" : "+v"(raddr[c]));
    }
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        taddr[h][dt] += bytes;
        asm("" : "+v"(taddr[h][dt]));
      }
  };
  auto bases_next = [&](int k) { bases_add(k == NSTAGE - 1 ? -(NSTAGE - 1) * TILE : TILE); };

  // The roles run separate loops with the same one barrier per step.  Step t: the P waves
  // compute tile t (P into slot t % 2) and stage the rows' lse and delta of tile t + 1
  // (through registers, loaded a step earlier); the dS waves load Q and dO of tile t + 1
  // into its stage, compute tile t - 1 and wait for their loads.  The barrier publishes P
  // of tile t and stage t + 1; stage (t + 1) % 3 was last read at step t - 1 (tile t - 2).
  if (!ds_wave) {
    load(tbeg);
    store(tbeg % NSTAGE);
    load(tbeg + 1);
    __syncthreads();
    int k = tbeg % NSTAGE;  // stage of tile t
    bases_add(k * TILE);
    for (int t = tbeg; t <= ntiles; ++t) {
      const int kn = k == NSTAGE - 1 ? 0 : k + 1;
      char* pex = pex0 + (t & 1) * 4 * PBYTES;
      const bool live = t < ntiles && tile_live(t);
      v8 pf[4];  // P, chunk c = queries 16c + 8hf + 0..7
      const int qt0 = t * BQ;
      const float* lse2s = reinterpret_cast<const float*>(lds + ROWS + k * ROWB);
      // One tile of P; HIDE: some element may be hidden (causal diagonal, mask, bias).
      auto p_tile = [&](auto hide_tag) {
        constexpr bool HIDE = decltype(hide_tag)::value;
        f32x16 sc2[2];
#pragma unroll
        for (int r = 0; r < 16; ++r) sc2[0][r] = sc2[1][r] = 0.f;
        dim_product2(sc2);
#pragma unroll
        for (int qs = 0; qs < 2; ++qs) {
          const f32x16 sc = sc2[qs];
#pragma unroll
          for (int g = 0; g < 2; ++g) {
            const int c = 2 * qs + g;
            const int qc = 16 * c + 8 * hf;  // first query of the run, within the tile
            const f32x4 l0 = *reinterpret_cast<const f32x4*>(lse2s + qc);
            const f32x4 l1 = *reinterpret_cast<const f32x4*>(lse2s + qc + 4);
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float o[2];
#pragma unroll
              for (int u = 0; u < 2; ++u) {
                const int i = 2 * e + u, r = 8 * g + i;
                const int qrow = qt0 + qc + i;
                float xv = __builtin_fmaf(sc[r], c2, -(i < 4 ? l0[i] : l1[i - 4]));
                if (HIDE) {
                  if (BIAS && k_ok && qrow < Lq)  // additive mask, in base-2 units
                    xv = __builtin_fmaf(bb[int64_t(qrow) * a.sm[2] + kj], kLog2e, xv);
                  bool hide = false;
                  if (CAUSAL) hide = kj > qrow + coff;
                  if (MASK) hide = hide || !k_ok || qrow >= Lq || mb[int64_t(qrow) * a.sm[2] + kj] == 0;
                  if (hide) xv = -INFINITY;
                }
                o[u] = exp2_fast(xv);
              }
              w[e] = pack2<E>(o[0], o[1]);
            }
            pf[c] = __builtin_bit_cast(v8, w);
            *reinterpret_cast<u32x4*>(pex + c * 1024) = w;
          }
        }
      };
      if (live) {
        if (MASK || BIAS || (CAUSAL && qt0 + coff < kw + 31))
          p_tile(std::true_type{});
        else
          p_tile(std::false_type{});
      }
      if (live) query_product(pf);
      if (t + 1 < ntiles) store(kn);
      load(t + 2);
      bases_next(k);
      k = kn;
      __syncthreads();  // P of tile t written; tile t + 1 staged; tile t - 1 read
    }
  } else {
    if (tbeg < ntiles) load_tile(tbeg, tbeg % NSTAGE);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    // tile u = t - 1, one step behind the P waves, on stage k = u % 3
    int k = (tbeg + NSTAGE - 1) % NSTAGE;
    bases_add(k * TILE);
    for (int t = tbeg; t <= ntiles; ++t) {
      if (t + 1 < ntiles) load_tile(t + 1, (t + 1) % NSTAGE);
      const int u = t - 1;
      const char* pex = pex0 + (u & 1) * 4 * PBYTES;
      if (u >= tbeg && tile_live(u)) {
        // dP - delta: the accumulators start at -delta of their rows (register r of half hf
        // is query 32qs + 16(r/8) + 8hf + r%8), then P of the tile
        const float* ndel = reinterpret_cast<const float*>(lds + ROWS + k * ROWB + 4 * BQ);
        f32x16 dp[2];
#pragma unroll
        for (int qs = 0; qs < 2; ++qs)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const f32x4 d = *reinterpret_cast<const f32x4*>(ndel + 32 * qs + 16 * (g >> 1) + 8 * hf + 4 * (g & 1));
#pragma unroll
            for (int e = 0; e < 4; ++e) dp[qs][4 * g + e] = d[e];
          }
        u32x4 pw[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) pw[c] = *reinterpret_cast<const u32x4*>(pex + c * 1024);
        dim_product2(dp);
        v8 dsf[4];  // dS, chunk c = queries 16c + 8hf + 0..7
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          u32x4 w;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const f32x2 p = unpack2<E>(pw[c][e]);
            const int r = 8 * (c & 1) + 2 * e;
            w[e] = pack2<E>(p[0] * dp[c >> 1][r], p[1] * dp[c >> 1][r + 1]);
          }
          dsf[c] = __builtin_bit_cast(v8, w);
        }
        query_product(dsf);
      }
      bases_next(k);
      k = k == NSTAGE - 1 ? 0 : k + 1;
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's loads of tile t + 1
      __syncthreads();
    }
  }
  // dV (P waves) and dK (dS waves) of the same 32 keys per SIMD, written as whole rows
  constexpr int RP = k_pitch_bf16(D);
  static_assert(8 * 32 * RP <= LDS_BYTES, "the output tiles fit the LDS");
  char* ot = lds + wave * 32 * RP;
  tile_to_lds<E, D, RP>(ot, acc, ds_wave ? a.scale : 1.f, li, hf);
  __syncthreads();
  if (ds_wave)
    rows_to_global<D, RP>(ot, lane, kw, Lk, dkb, a.sdk[2]);
  else
    rows_to_global<D, RP>(ot, lane, kw, Lk, dvb, a.sdv[2]);
}

// ---------------------------------------------------------------------------------------
// Row-by-row backward for fp32 inputs and for D = 256 (any input type): the formulas of the
// two kernels above, one wave per query row (dq and delta), then one wave per key row (dk
// and dv), on the vector ALU with every value and sum in fp32 (P and dS are not rounded).
// For a run of 64 keys (queries) lane l first forms the score and dP of key (query) l
// from the row's values, which the wave keeps in its own slot of LDS and reads back as
// broadcasts, four head dims at a time; the lanes then
// switch to head dims l, l + 64, ... and add the run's contributions to the row's
// gradients in key (query) order.  Deterministic; no workgroup barrier, so a wave past
// its item's rows leaves at once.
// ---------------------------------------------------------------------------------------
constexpr int kGenDims = 4;  // head dims per lane (D <= 256)

// Four consecutive elements as floats (16-byte aligned for fp32, 8-byte for 16-bit types).
template <typename E>
__device__ inline f32x4 load4f(const E* p) {
  if constexpr (sizeof(E) == 4) {
    return *reinterpret_cast<const f32x4*>(p);
  } else {
    const u32x2 w = *reinterpret_cast<const u32x2*>(p);
    const auto h = [](uint32_t b) { return float(__builtin_bit_cast(E, uint16_t(b))); };
    return f32x4{h(w[0] & 0xFFFFu), h(w[0] >> 16), h(w[1] & 0xFFFFu), h(w[1] >> 16)};
  }
}

// Publishes a wave's LDS writes to its own later reads (no other wave reads them).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Score of (i, j) in natural-log units with the additive mask, -inf where (i, j) is hidden
// by the boolean mask; position rules are the caller's.
template <int MK>
__device__ inline float gen_score(const BwdArgs& a, const BwdItem& it, int i, int j, float qk) {
  float x = qk * a.scale;
  if (MK == 1 && a.mask[it.m + int64_t(i) * a.sm[2] + j] == 0) x = -INFINITY;
  if (MK == 2) x += a.bias[it.m + int64_t(i) * a.sm[2] + j];
  return x;
}

__device__ inline float gen_prob(float x, float lse) {
  return x > -INFINITY && lse > -INFINITY ? expf(x - lse) : 0.f;
}

template <typename E, bool CAUSAL, int MK, int MODE>
__global__ __launch_bounds__(kThreadsBwdGen) void bwd_rows_gen(BwdArgs a, int D) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = blockIdx.x / a.q_items;
  const int i = int(blockIdx.x - bh * a.q_items) * kBwdGenRows + int(threadIdx.x >> 6);
  const BwdItem it = bwd_item<MODE>(a, bh);
  if (i >= it.Lq) return;
  const E* q = static_cast<const E*>(a.q) + it.q + int64_t(i) * a.sq[2];
  const E* o = static_cast<const E*>(a.out) + it.o + int64_t(i) * a.so[2];
  const E* dO = static_cast<const E*>(a.dout) + it.dO + int64_t(i) * a.sdo[2];
  const E* kb = static_cast<const E*>(a.k) + it.k;
  const E* vb = static_cast<const E*>(a.v) + it.v;
  float qv[kGenDims], dov[kGenDims], dqv[kGenDims];
  float part = 0.f;
#pragma unroll
  for (int c = 0; c < kGenDims; ++c) {
    const int d = lane + 64 * c;
    const bool ok = d < D;
    qv[c] = ok ? float(q[d]) : 0.f;
    dov[c] = ok ? float(dO[d]) : 0.f;
    part += ok ? dov[c] * float(o[d]) : 0.f;
    dqv[c] = 0.f;
  }
  const float delta = wave_sum(part);
  const float lse = a.lse[it.lse + i];
  // the row's q and dout values in this wave's LDS slot, read back as broadcasts
  __shared__ __attribute__((aligned(16))) float rows_lds[kBwdGenRows][2][64 * kGenDims];
  float* const qs = rows_lds[threadIdx.x >> 6][0];
  float* const dos = rows_lds[threadIdx.x >> 6][1];
#pragma unroll
  for (int c = 0; c < kGenDims; ++c) {
    const int d = lane + 64 * c;
    if (d < D) {
      qs[d] = qv[c];
      dos[d] = dov[c];
    }
  }
  wave_lds_sync();
  int kend = it.Lk;
  if (CAUSAL) kend = max(0, min(kend, i + it.coff + 1));
  for (int j0 = 0; j0 < kend; j0 += 64) {
    const int j = j0 + lane;
    const bool act = j < kend;
    const E* kr = kb + int64_t(act ? j : j0) * a.sk[2];
    const E* vr = vb + int64_t(act ? j : j0) * a.sv[2];
    float qk = 0.f, dp = 0.f;
    for (int d = 0; d < D; d += 4) {
      const f32x4 q4 = *reinterpret_cast<const f32x4*>(qs + d);
      const f32x4 o4 = *reinterpret_cast<const f32x4*>(dos + d);
      const f32x4 k4 = load4f(kr + d), v4 = load4f(vr + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qk += q4[e] * k4[e];
        dp += o4[e] * v4[e];
      }
    }
    const float p = act ? gen_prob(gen_score<MK>(a, it, i, j, qk), lse) : 0.f;
    const float ds = p * (dp - delta);
    const int n = min(64, kend - j0);
    for (int e = 0; e < n; ++e) {
      const float dse = __shfl(ds, e);
      const E* kr2 = kb + int64_t(j0 + e) * a.sk[2];
#pragma unroll
      for (int c = 0; c < kGenDims; ++c) {
        const int d = lane + 64 * c;
        if (d < D) dqv[c] += dse * float(kr2[d]);
      }
    }
  }
  E* dq = static_cast<E*>(a.dq) + it.dq + int64_t(i) * a.sdq[2];
#pragma unroll
  for (int c = 0; c < kGenDims; ++c) {
    const int d = lane + 64 * c;
    if (d < D) dq[d] = static_cast<E>(dqv[c] * a.scale);
  }
  if (lane == 0) a.delta[it.lse + i] = delta;
}

template <typename E, bool CAUSAL, int MK, int MODE>
__global__ __launch_bounds__(kThreadsBwdGen) void bwd_keys_gen(BwdArgs a, int D) {
  const int lane = threadIdx.x & 63;
  const int64_t bh = blockIdx.x / a.k_items;
  const int j = int(blockIdx.x - bh * a.k_items) * kBwdGenRows + int(threadIdx.x >> 6);
  const BwdItem it = bwd_item<MODE>(a, bh);
  if (j >= it.Lk) return;
  const E* kr = static_cast<const E*>(a.k) + it.k + int64_t(j) * a.sk[2];
  const E* vr = static_cast<const E*>(a.v) + it.v + int64_t(j) * a.sv[2];
  const E* qb = static_cast<const E*>(a.q) + it.q;
  const E* db = static_cast<const E*>(a.dout) + it.dO;
  float kv[kGenDims], vv[kGenDims], dkv[kGenDims], dvv[kGenDims];
#pragma unroll
  for (int c = 0; c < kGenDims; ++c) {
    const int d = lane + 64 * c;
    const bool ok = d < D;
    kv[c] = ok ? float(kr[d]) : 0.f;
    vv[c] = ok ? float(vr[d]) : 0.f;
    dkv[c] = dvv[c] = 0.f;
  }
  // the key row's k and v values in this wave's LDS slot, read back as broadcasts
  __shared__ __attribute__((aligned(16))) float rows_lds[kBwdGenRows][2][64 * kGenDims];
  float* const ks = rows_lds[threadIdx.x >> 6][0];
  float* const vs = rows_lds[threadIdx.x >> 6][1];
#pragma unroll
  for (int c = 0; c < kGenDims; ++c) {
    const int d = lane + 64 * c;
    if (d < D) {
      ks[d] = kv[c];
      vs[d] = vv[c];
    }
  }
  wave_lds_sync();
  // the queries that can see key j: i >= j - coff under a causal mask
  const int istart = CAUSAL ? min(max(0, j - it.coff), it.Lq) : 0;
  for (int i0 = istart; i0 < it.Lq; i0 += 64) {
    const int i = i0 + lane;
    const bool act = i < it.Lq;
    const E* qr = qb + int64_t(act ? i : i0) * a.sq[2];
    const E* dr = db + int64_t(act ? i : i0) * a.sdo[2];
    float qk = 0.f, dp = 0.f;
    for (int d = 0; d < D; d += 4) {
      const f32x4 k4 = *reinterpret_cast<const f32x4*>(ks + d);
      const f32x4 v4 = *reinterpret_cast<const f32x4*>(vs + d);
      const f32x4 q4 = load4f(qr + d), o4 = load4f(dr + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        qk += k4[e] * q4[e];
        dp += v4[e] * o4[e];
      }
    }
    float p = 0.f, ds = 0.f;
    if (act) {
      p = gen_prob(gen_score<MK>(a, it, i, j, qk), a.lse[it.lse + i]);
      ds = p * (dp - a.delta[it.lse + i]);
    }
    const int n = min(64, it.Lq - i0);
    for (int e = 0; e < n; ++e) {
      const float pe = __shfl(p, e), dse = __shfl(ds, e);
      const E* q2 = qb + int64_t(i0 + e) * a.sq[2];
      const E* d2 = db + int64_t(i0 + e) * a.sdo[2];
#pragma unroll
      for (int c = 0; c < kGenDims; ++c) {
        const int d = lane + 64 * c;
        if (d < D) {
          dvv[c] += pe * float(d2[d]);
          dkv[c] += dse * float(q2[d]);
        }
      }
    }
  }
  E* dk = static_cast<E*>(a.dk) + it.dk + int64_t(j) * a.sdk[2];
  E* dv = static_cast<E*>(a.dv) + it.dv + int64_t(j) * a.sdv[2];
#pragma unroll
  for (int c = 0; c < kGenDims; ++c) {
    const int d = lane + 64 * c;
    if (d < D) {
      dk[d] = static_cast<E>(dkv[c] * a.scale);
      dv[d] = static_cast<E>(dvv[c]);
    }
  }
}

template <typename E, bool CAUSAL, int MK, int MODE>
hipError_t launch_gen_pair(const BwdArgs& a, int D, unsigned grid_q, unsigned grid_k,
                           hipStream_t s) {
  void* args[] = {const_cast<BwdArgs*>(&a), &D};
  if (grid_q) {
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void*>(&bwd_rows_gen<E, CAUSAL, MK, MODE>),
                        dim3(grid_q), dim3(kThreadsBwdGen), args, 0, s);
    if (e != hipSuccess) return e;
  }
  if (grid_k)
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_keys_gen<E, CAUSAL, MK, MODE>),
                           dim3(grid_k), dim3(kThreadsBwdGen), args, 0, s);
  return hipSuccess;
}

template <typename E, bool CAUSAL>
hipError_t launch_gen_c(const BwdArgs& a, bool varlen, int D, unsigned gq, unsigned gk,
                        hipStream_t s) {
  if (varlen) return launch_gen_pair<E, CAUSAL, 0, kBwdVarlen>(a, D, gq, gk, s);
  if (a.mask) return launch_gen_pair<E, CAUSAL, 1, kBwdDense>(a, D, gq, gk, s);
  if (a.bias) return launch_gen_pair<E, CAUSAL, 2, kBwdDense>(a, D, gq, gk, s);
  return launch_gen_pair<E, CAUSAL, 0, kBwdDense>(a, D, gq, gk, s);
}

template <typename E>
hipError_t launch_gen(const BwdArgs& a, bool causal, bool varlen, int D, unsigned gq,
                      unsigned gk, hipStream_t s) {
  return causal ? launch_gen_c<E, true>(a, varlen, D, gq, gk, s)
                : launch_gen_c<E, false>(a, varlen, D, gq, gk, s);
}

template <typename E, int D, bool CAUSAL, int MK, int MODE>
hipError_t launch_pair(const BwdArgs& a, unsigned grid_q, unsigned grid_k, hipStream_t s) {
  void* args[] = {const_cast<BwdArgs*>(&a)};
  if (grid_q) {
    const hipError_t e =
        hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dq<E, D, CAUSAL, MK, MODE>),
                        dim3(grid_q), dim3(kThreadsBwdQ), args, 0, s);
    if (e != hipSuccess) return e;
  }
  if (grid_k)
    return hipLaunchKernel(reinterpret_cast<const void*>(&bwd_dkdv<E, D, CAUSAL, MK, MODE>),
                           dim3(grid_k), dim3(kThreadsBwdK), args, 0, s);
  return hipSuccess;
}

template <typename E, int D, bool CAUSAL>
hipError_t launch_bwd_c(const BwdArgs& a, bool varlen, unsigned gq, unsigned gk, hipStream_t s) {
  if (varlen) return launch_pair<E, D, CAUSAL, 0, kBwdVarlen>(a, gq, gk, s);
  if (a.mask) return launch_pair<E, D, CAUSAL, 1, kBwdDense>(a, gq, gk, s);
  if (a.bias) return launch_pair<E, D, CAUSAL, 2, kBwdDense>(a, gq, gk, s);
  return launch_pair<E, D, CAUSAL, 0, kBwdDense>(a, gq, gk, s);
}

template <typename E, int D>
hipError_t launch_bwd_d(const BwdArgs& a, bool causal, bool varlen, unsigned gq, unsigned gk,
                        hipStream_t s) {
  return causal ? launch_bwd_c<E, D, true>(a, varlen, gq, gk, s)
                : launch_bwd_c<E, D, false>(a, varlen, gq, gk, s);
}

}  // namespace

hipError_t launch_bwd(const BwdProblem& p, hipStream_t stream) {
  BwdArgs a;
  a.q = p.q;
  a.k = p.k;
  a.v = p.v;
  a.out = p.out;
  a.dout = p.dout;
  a.lse = p.lse;
  a.delta = p.delta;
  a.dq = p.dq;
  a.dk = p.dk;
  a.dv = p.dv;
  a.mask = p.mask;
  a.bias = p.bias;
  a.cu_q = p.cu_q;
  a.cu_k = p.cu_k;
  for (int i = 0; i < 3; ++i) {
    a.sq[i] = p.sq[i];
    a.sk[i] = p.sk[i];
    a.sv[i] = p.sv[i];
    a.so[i] = p.so[i];
    a.sdo[i] = p.sdo[i];
    a.sdq[i] = p.sdq[i];
    a.sdk[i] = p.sdk[i];
    a.sdv[i] = p.sdv[i];
    a.sm[i] = p.sm[i];
  }
  a.H = int32_t(p.H);
  a.Lq = int32_t(p.Lq);
  a.Lk = int32_t(p.Lk);
  // dense: B*H heads of Lq query and Lk key rows; packed: nseq*H heads of at most
  // max_seqlen_q / max_seqlen_k rows
  const int64_t qrows = p.varlen ? p.max_seqlen_q : p.Lq;
  const int64_t krows = p.varlen ? p.max_seqlen_k : p.Lk;
  a.bh_count = int32_t((p.varlen ? p.nseq : p.B) * p.H);
  const bool gen = bwd_generic(p.dtype, p.D);  // the row-by-row kernels
  a.q_items = int32_t((qrows + (gen ? kBwdGenRows : kBwdBlockQ) - 1) /
                      (gen ? kBwdGenRows : kBwdBlockQ));
  a.k_items = int32_t((krows + (gen ? kBwdGenRows : kBwdBlockK) - 1) /
                      (gen ? kBwdGenRows : kBwdBlockK));
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  a.mask_vec8 = p.mask && (reinterpret_cast<uintptr_t>(p.mask) % 8 == 0) && p.sm[0] % 8 == 0 &&
                p.sm[1] % 8 == 0 && p.sm[2] % 8 == 0;
  a.coff = p.causal == 2 ? int32_t(p.Lk - p.Lq) : 0;
  a.bottom_right = p.causal == 2;
  a.bias_vec4 = p.bias && (reinterpret_cast<uintptr_t>(p.bias) % 16 == 0) && p.sm[0] % 4 == 0 &&
                p.sm[1] % 4 == 0 && p.sm[2] % 4 == 0;
  const unsigned gq = unsigned(int64_t(a.q_items) * a.bh_count);
  const unsigned gk = unsigned(int64_t(a.k_items) * a.bh_count);
  const bool causal = p.causal != 0;
  if (gen) {
    const int D = int(p.D);
    if (p.dtype == 0) return launch_gen<float>(a, causal, p.varlen != 0, D, gq, gk, stream);
    if (p.dtype == 2) return launch_gen<_Float16>(a, causal, p.varlen != 0, D, gq, gk, stream);
    return launch_gen<__bf16>(a, causal, p.varlen != 0, D, gq, gk, stream);
  }
  if (p.dtype == 2)
    switch (p.D) {
      case 32: return launch_bwd_d<_Float16, 32>(a, causal, p.varlen != 0, gq, gk, stream);
      case 64: return launch_bwd_d<_Float16, 64>(a, causal, p.varlen != 0, gq, gk, stream);
      case 96: return launch_bwd_d<_Float16, 96>(a, causal, p.varlen != 0, gq, gk, stream);
      default: return launch_bwd_d<_Float16, 128>(a, causal, p.varlen != 0, gq, gk, stream);
    }
  switch (p.D) {
    case 32: return launch_bwd_d<__bf16, 32>(a, causal, p.varlen != 0, gq, gk, stream);
    case 64: return launch_bwd_d<__bf16, 64>(a, causal, p.varlen != 0, gq, gk, stream);
    case 96: return launch_bwd_d<__bf16, 96>(a, causal, p.varlen != 0, gq, gk, stream);
    default: return launch_bwd_d<__bf16, 128>(a, causal, p.varlen != 0, gq, gk, stream);
  }
}

}  // namespace sdpa
