// Device helpers shared by the HIP translation units of libtq (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "tq_internal.h"

namespace tq {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(8))) int i32x8;

constexpr int kWave = 64;
constexpr int kBlock = 256;   // 4 waves per workgroup

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float flip_sign(float v, uint32_t bit) {
  return __uint_as_float(__float_as_uint(v) ^ (bit << 31));
}

// The p-th odd-popcount subset of R index bits, in increasing order (the order in which
// the host lists the parity planes and their coefficients).
template <int R>
__host__ __device__ constexpr uint32_t pmask_c(int p) {
  int n = 0;
  for (uint32_t S = 1; S < (1u << R); ++S) {
    if (__builtin_popcount(S) % 2 == 0) continue;
    if (n == p) return S;
    ++n;
  }
  return 0;
}

struct EncodeArgs {
  SubDev s;
  const void* x;
  int64_t n;
  int64_t ldx;
  uint8_t* codes;
  int rec_bytes;
  int is_bf16;
  int vec_load;   // rows 16-byte aligned and no channel gather: vector loads
  uint16_t* rw_hi;  // two-pass encode (long vectors): residual limbs [n][D], high and low
  uint16_t* rw_lo;
  // Groups (grid z): group g encodes rows g n .. g n + n - 1 into its records, or into the
  // cache rows out_index[g n ..] (rows outside [0, out_cap) are skipped); plans with one
  // channel list per head gather with the list of head g % n_heads.
  int n_heads;
  const int64_t* out_index;
  int64_t out_cap;
};

// This workgroup's group: its input rows, its output records (or cache-row indices) and its
// head's channel list.
__device__ __forceinline__ void encode_group_view(EncodeArgs& a) {
  const int64_t g = blockIdx.z;
  const int es = a.is_bf16 ? 2 : 4;
  a.x = static_cast<const uint8_t*>(a.x) + g * a.n * a.ldx * es;
  if (a.out_index)
    a.out_index += g * a.n;
  else
    a.codes += g * a.n * a.rec_bytes;
  if (a.s.chan) a.s.chan += (g % a.n_heads) * a.s.d;
}

// Record of local row `row` (null when an append's cache row lies outside the cache).
__device__ __forceinline__ uint8_t* encode_record(const EncodeArgs& a, int64_t row) {
  if (a.out_index == nullptr) return a.codes + row * a.rec_bytes + a.s.rec_off;
  const int64_t r = a.out_index[row];
  return (r >= 0 && r < a.out_cap) ? a.codes + r * a.rec_bytes + a.s.rec_off : nullptr;
}

// D = 128 inner-product plans with bf16 input and the 32x32 operand tables (encode128.hip).
int launch_encode128(const EncodeArgs& ea, hipStream_t st, int64_t n_groups);
// Compute units of the current device (cached per device; 256 if the query fails).
int compute_units();
// Scorer on decoded fp16 key tiles (score_f16.hip): one inner-product sub-plan with D >= 256
// and at least kScoreF16MinQueries queries per group.  yrot and w are the queries' y' and
// S y' (fp32, [rows][D]); img (n_groups x ceil(nq_per_group / 32) x 32 rows x 2D fp16) and
// isc ([rows]) are its workspace.
constexpr int64_t kScoreF16MinQueries = 128;
bool score_f16_applies(const PlanDev& p, int64_t nq_per_group);
int launch_score_f16(const PlanDev& p, const float* yrot, const float* w, uint16_t* img,
                     float* isc, int64_t nq_per_group, int64_t n_groups, const uint8_t* codes,
                     int64_t n, float* scores, hipStream_t st);

constexpr int kEncWaves = 8;

__device__ __forceinline__ uint32_t or_over_lane_groups(uint32_t v) {
  auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  const uint32_t x = a[0] | a[1];
  auto b = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return b[0] | b[1];
}

__device__ __forceinline__ float sum_over_lane_groups(float v) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  const float x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ bf16x8 bf16x8_from_words(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const u32x4 u = {w0, w1, w2, w3};
  return __builtin_bit_cast(bf16x8, u);
}

__device__ __forceinline__ f16x8 f16x8_from_words(uint32_t w0, uint32_t w1, uint32_t w2, uint32_t w3) {
  typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
  const u32x4 u = {w0, w1, w2, w3};
  return __builtin_bit_cast(f16x8, u);
}

// Copies an operand table of N 16-byte pieces into LDS with a block of NT threads, every
// global load issued before the first LDS store: the block waits for one round of memory
// latency instead of one per loop trip, which is most of a short call's time.
template <int N, int NT>
__device__ __forceinline__ void table_to_lds(uint4* dst, const uint4* src) {
  constexpr int J = (N + NT - 1) / NT;
  uint4 t[J];
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = threadIdx.x + j * NT;
    if (N % NT == 0 || i < N) t[j] = src[i];
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int i = threadIdx.x + j * NT;
    if (N % NT == 0 || i < N) dst[i] = t[j];
  }
}

// Two bf16 values (one word), times a power of two when SCALE, as two fp16 values (one
// word).  Exact when the (scaled) values lie in the fp16 normal range; smaller ones round
// toward zero on the fp16 subnormal grid (absolute error below 2^-24).
template <bool SCALE>
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t w, float scale) {
  float lo = __uint_as_float(w << 16), hi = __uint_as_float(w & 0xFFFF0000u);
  if constexpr (SCALE) {
    lo *= scale;
    hi *= scale;
  }
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  typedef __attribute__((ext_vector_type(2))) float f32x2;
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
#define pack2_bf16 pack_bf16_rne

// v - (one half of the packed bf16 pair hp), exact when that half is v rounded to bf16: one
// bf16 dot product hp . sel + v with sel = -1 in the chosen half and 0 in the other, which
// reads the packed pair directly instead of unpacking it first.
__device__ __forceinline__ float residual_below_bf16(uint32_t hp, uint32_t sel, float v) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, hp),
                                         __builtin_bit_cast(bf16x2, sel), v, false);
}

// The selector (-1, 0) as a register value.  Written as a constant it is folded into the
// inline constant -1.0, which this instruction reads as the pair (0, -1): the wrong half.
__device__ __forceinline__ uint32_t neg_one_low_half() {
  uint32_t v;
  asm("v_mov_b32 %0, 0xbf80" : "=v"(v));
  return v;
}

// Per-lane building blocks of the bucketize.  The select and the shift-in are written out
// as single instructions, so that chains of them stay a fixed sequence (the compiler
// otherwise rebuilds the selects into an integer index and compare chains).  The comparison,
// which reads the matrix-core results, stays a builtin: the compiler inserts the wait states
// a read of an MFMA result needs, which it does not do for an inline-assembly operand.
// Lane mask of |z| >= t (one v_cmp with the abs modifier; 3 = ordered greater-or-equal).
__device__ __forceinline__ uint64_t abs_ge_mask(float z, float t) {
  return __builtin_amdgcn_fcmpf(__builtin_fabsf(z), t, 3);
}
// Per lane: m ? b : a.
__device__ __forceinline__ float select_mask(uint64_t m, float a, float b) {
  float r;
  asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "s"(m));
  return r;
}
// w = 2 w + (this lane's bit of m).
__device__ __forceinline__ uint32_t shift_in_mask(uint32_t w, uint64_t m) {
  uint64_t carry;
  asm("v_addc_co_u32_e64 %0, %1, %0, %0, %2" : "+v"(w), "=s"(carry) : "s"(m));
  return w;
}
// w = 2 w + sign bit of f.
__device__ __forceinline__ uint32_t shift_in_sign(uint32_t w, float f) {
  return __builtin_amdgcn_alignbit(w, __float_as_uint(f), 31);
}

// One coordinate of the symmetric Lloyd-Max quantizer.  The codebook is mirror-symmetric
// with its middle threshold at 0, so idx = 2^(R-1) [z >= 0] + (z >= 0 ? j : 2^(R-1) - 1 - j)
// with j the cell of |z| among the positive thresholds tp[] (levels ap[]).  The sign goes to
// P (bit set = negative), the bits of j to J[R-2..0]; the index planes are formed per word
// afterwards: plane R-1 = ~P, plane m = J[m] ^ P.  Returns the residual z - c[idx].
// (|z| equal to a threshold may land in either neighbouring cell; such a coordinate is
// within rounding of the boundary in any precision.)
template <int R>
__device__ __forceinline__ float bucket_sym(float z, const float* tp, const float* ap,
                                            uint32_t& P, uint32_t* J) {
  constexpr int H = 1 << (R - 1);
  float tc[H > 1 ? H - 1 : 1], lc[H];
#pragma unroll
  for (int j = 0; j < H - 1; ++j) tc[j] = tp[j];
#pragma unroll
  for (int j = 0; j < H; ++j) lc[j] = ap[j];
#pragma unroll
  for (int m = R - 2; m >= 0; --m) {
    const int half = 1 << m;                 // thresholds left: 2 half - 1, middle half - 1
    const uint64_t mk = abs_ge_mask(z, tc[half - 1]);
    J[m] = shift_in_mask(J[m], mk);
#pragma unroll
    for (int j = 0; j < half - 1; ++j) tc[j] = select_mask(mk, tc[j], tc[half + j]);
#pragma unroll
    for (int j = 0; j < half; ++j) lc[j] = select_mask(mk, lc[j], lc[half + j]);
  }
  P = shift_in_sign(P, z);
  return z - copysignf(lc[0], z);
}


// ----------------------------------------------------------------- bit-sliced scorer images
// For a symmetric codebook the level of an R-bit index expands over the parity planes of odd
// subsets of its bits: c[idx] = sum_S a_S (2 p_S - 1).  The MSE term of a key becomes
// 2 sum_S a_S <y', p_S> - A0 sum y', and the QJL term 2 <w, beta> - sum w: binary dot
// products.  Keys are fed to the MFMA as fp4 values 0 / 0.5 straight from their bits; the
// query side is an fp8 image holding three limbs of a_S y' (or w) per query, so that the
// four queries of a group and their three limbs fill the 16 rows of one MFMA tile.
//
// A-operand (fp8, 16 x 128) lane layout of v_mfma_scale_f32_16x16x128_f8f6f4 on gfx950:
// row = lane % 16; element e of lane group G = lane / 16 is K = 16 G + e (e < 16) or
// K = 64 + 16 G + (e - 16).  B-operand (fp4, 128 x 16): column = lane % 16, element e of
// lane group G is K = 32 G + e.  A key plane word W of chunk G gives the B dwords
// (W >> j) & 0x11111111, j = 0..3: nibble m of dword j is coordinate 32 G + 4 m + j at
// K = 32 G + 8 j + m.

__device__ __forceinline__ int bitslice_coord(int K) {
  const int G = K >> 5, j = (K & 31) >> 3, m = K & 7;
  return 32 * G + 4 * m + j;
}

struct QFusedArgs {
  SubDev s;
  const void* q;
  int64_t ldq;
  int is_bf16;
  int64_t nq;            // total query rows
  int64_t nq_per_group;
  int n_qtiles;
  int n_heads;           // group g gathers with the channel list of head g % n_heads
  uint32_t* img;         // [groups*qtiles][n_planes+1][64][8]
  float* ec;             // [groups*qtiles][4][4]
};

// ============================================================================ scorers
// est = n (<y', c[idx]> + gamma sqrt(pi/2)/k <w, 2 beta - 1>), summed over sub-plans
// (technical overview §1.2.3 unbiased two-stage estimate, §4.2.2 per-coordinate centroid
// lookup with the query under the same rotation).

struct ScoreArgs {
  PlanDev p;
  const uint8_t* codes;
  int64_t n;
  int64_t nq_per_group;
  int n_qtiles;
  int vec_out;           // score rows 16-byte aligned (scores and n % 4): vector stores
  float* scores;
  const uint32_t* img[2];
  const float* ec[2];
  const float* yrot[2];
  const float* w[2];
};

template <int NP> struct PlaneImg { i32x8 a[NP + 1]; };

__device__ __forceinline__ i32x8 fp4_operand(uint32_t W) {
  i32x8 b;
  b[0] = (int)(W & 0x11111111u);
  b[1] = (int)((W >> 1) & 0x11111111u);
  b[2] = (int)((W >> 2) & 0x11111111u);
  b[3] = (int)((W >> 3) & 0x11111111u);
  b[4] = 0; b[5] = 0; b[6] = 0; b[7] = 0;
  return b;
}

// Bit-sliced scorer for sub-plans with D <= 128 (score128.hip): query images, then scores.
int launch_qprep_bitslice(const QFusedArgs& fa, int D, int64_t nq, hipStream_t st);
bool dispatch_bitslice(const ScoreArgs& sa, int64_t n_gt, hipStream_t st);

}  // namespace tq
