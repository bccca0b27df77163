// C ABI of libtq: argument validation, plan construction (host tables + one device
// allocation), and dispatch to the kernel launchers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <vector>

#include "tq_internal.h"

using namespace tq;

namespace {

int padded_length(int d) {
  int D = kMinD;
  while (D < d) D *= 2;
  return D;
}

int record_bytes_of(int D, int R) { return 4 * (R + 1) * (D / 32) + 8; }
int record_bytes_mse_of(int D, int R) { return 4 * R * (D / 32) + 4; }

bool current_device(int* dev) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count < 1) return false;
  return hipGetDevice(dev) == hipSuccess;
}

bool plan_device_ok(const tq_plan* p) {
  int dev = -1;
  return hipGetDevice(&dev) == hipSuccess && dev == p->device;
}

tq_status from_hip(int rc) {
  if (rc == 0) return TQ_OK;
  if (rc == (int)hipErrorOutOfMemory || rc == (int)hipErrorMemoryAllocation) return TQ_ENOMEM;
  return TQ_EDEVICE;
}

// Host description of one sub-plan before upload.
struct SubHost {
  int d, D, R;
  std::vector<int32_t> chan;     // empty = identity
  std::vector<double> lev, thr;
  std::vector<uint32_t> signs;   // [3][D/32]
  std::vector<uint16_t> S;       // [D][D]
  std::vector<uint16_t> rotk;    // MFMA operand tables (D <= 128)
  std::vector<uint16_t> rotk16;  // K in one fp16 limb, when every |K| <= 2048 (else empty)
  std::vector<uint16_t> rotkt16; // K^T the same way (dequantization), with rotk16
  std::vector<uint16_t> sperm;
  std::vector<uint16_t> k16_32;  // operands of the D = 128 32x32 encoder (may stay empty)
  std::vector<uint16_t> s16_32;
  std::vector<uint8_t> s8_32;
  std::vector<uint16_t> kf16;    // 32x32 encoder, channel selection folded in (per head)
  std::vector<uint32_t> xmask;   // the selected columns of each head, for the norm
};

constexpr int kMfmaMaxD = 128;

// The rotation as an integer matrix: K = H S3 H S2 H S1 = D^(3/2) Pi (H the Sylvester
// Hadamard matrix, S_r the +-1 diagonals), column i = the transform of e_i.  |K| <= D^2.
std::vector<int64_t> rotation_integer_matrix(const std::vector<uint32_t>& signs, int D) {
  std::vector<int64_t> K((size_t)D * D);
  std::vector<int64_t> v(D);
  for (int i = 0; i < D; ++i) {
    for (int j = 0; j < D; ++j) v[j] = (j == i);
    for (int r = 0; r < 3; ++r) {
      for (int j = 0; j < D; ++j)
        if ((signs[r * (D / 32) + j / 32] >> (j % 32)) & 1u) v[j] = -v[j];
      for (int h = 1; h < D; h <<= 1)
        for (int a = 0; a < D; a += 2 * h)
          for (int b = a; b < a + h; ++b) {
            const int64_t x = v[b], y = v[b + h];
            v[b] = x + y;
            v[b + h] = x - y;
          }
    }
    for (int j = 0; j < D; ++j) K[(size_t)j * D + i] = v[j];
  }
  return K;
}

// Operand tables of the MFMA encode (16x16x32 bf16: lane l holds row l%16 and the 8
// consecutive k values 8*(l/16)..+7 of a 32-wide k step; the 16x16 result puts row
// 4*(l/16) + e of a tile in lane l).  Output rows are permuted so that lane group G of
// tile jt, element e, receives coordinate G*D/4 + 4*jt + e: each lane group then holds D/4
// consecutive coordinates, a whole 32-bit code word when D = 128.
//  rotk: K (rows permuted as above) split into two bf16 limbs (exact: |K| <= 2^14 for
//        D <= 128); k steps of 32 input coordinates.
//  rotk16: the same K as a single fp16 limb (16x16x32 f16 operands), present when every
//        |K| <= 2048 so that each entry is an exact fp16 integer.  With K ~ D N(0,1) per
//        entry this holds for any practical seed; the bf16 pair remains the fallback.
//  sperm: S with rows permuted the same way and columns ordered as the residual registers:
//        k element e of lane group G in step ks is coordinate G*D/4 + 8*ks + e.
int permuted_row(int D, int tile, int row_in_tile) {
  return (row_in_tile / 4) * (D / 4) + 4 * tile + row_in_tile % 4;
}

// Output rows of the dequantization table (K^T): lane group G = row/4 of tile jt, element
// e = row%4, receives input coordinate 32 (jt/2) + 8 G + 4 (jt%2) + e, so that every 32
// consecutive coordinates are split over the four lane groups, 8 each: one store instruction
// then writes 4 x 8 adjacent coordinates of a vector.
int dequant_row(int tile, int row_in_tile) {
  return 32 * (tile / 2) + 8 * (row_in_tile / 4) + 4 * (tile % 2) + row_in_tile % 4;
}

// fp16 bit pattern of an integer with |v| <= 2048 (exact).
uint16_t fp16_bits_of_small_int(int64_t v) {
  if (v == 0) return 0;
  const uint16_t sign = v < 0 ? 0x8000u : 0u;
  uint64_t a = (uint64_t)(v < 0 ? -v : v);
  int e = 63 - __builtin_clzll(a);                 // a = 2^e * (1.f), e <= 11
  const uint32_t mant = (uint32_t)((a << (10 - e)) & 0x3FFu);
  return (uint16_t)(sign | (uint32_t)(e + 15) << 10 | mant);
}

void mfma32_operand_tables(SubHost& h, const std::vector<int64_t>& K);

void mfma_operand_tables(SubHost& h) {
  const int D = h.D, NJT = D / 16, NKS = D / 32;
  const std::vector<int64_t> K = rotation_integer_matrix(h.signs, D);
  h.rotk.assign((size_t)2 * NJT * NKS * 64 * 8, 0);
  if (!h.S.empty()) h.sperm.assign((size_t)NJT * NKS * 64 * 8, 0);
  int64_t kmax = 0;
  for (int64_t v : K) kmax = std::max<int64_t>(kmax, v < 0 ? -v : v);
  if (kmax <= 2048) {
    h.rotk16.assign((size_t)NJT * NKS * 64 * 8, 0);
    h.rotkt16.assign((size_t)NJT * NKS * 64 * 8, 0);
  }
  for (int jt = 0; jt < NJT; ++jt)
    for (int ks = 0; ks < NKS; ++ks)
      for (int l = 0; l < 64; ++l)
        for (int e = 0; e < 8; ++e) {
          const int row = permuted_row(D, jt, l % 16), G = l / 16;
          const double kv = (double)K[(size_t)row * D + 32 * ks + 8 * G + e];
          const uint16_t hi = bf16_rne_from_double(kv);
          uint32_t hb = (uint32_t)hi << 16;
          float hf;
          memcpy(&hf, &hb, 4);
          const uint16_t lo = bf16_rne_from_double(kv - (double)hf);
          const size_t at = (((size_t)jt * NKS + ks) * 64 + l) * 8 + e;
          h.rotk[at] = hi;
          h.rotk[(size_t)NJT * NKS * 64 * 8 + at] = lo;
          if (!h.rotk16.empty()) {
            h.rotk16[at] = fp16_bits_of_small_int(K[(size_t)row * D + 32 * ks + 8 * G + e]);
            // K^T: output (input-domain) coordinate, rotated coordinate as the k index
            const int orow = dequant_row(jt, l % 16);
            h.rotkt16[at] = fp16_bits_of_small_int(K[(size_t)(32 * ks + 8 * G + e) * D + orow]);
          }
          const int col = G * (D / 4) + 8 * ks + e;
          if (!h.S.empty()) h.sperm[at] = h.S[(size_t)row * D + col];
        }
  mfma32_operand_tables(h, K);
}

// Output row rho of a 32-row tile t of the 32x32 encoder (lane half h' = (rho / 4) % 2,
// accumulator element 4 i + j with i = rho / 8, j = rho % 4) is coordinate
// 64 h' + 16 t + 4 i + j: each lane half then holds 64 consecutive coordinates.
int permuted_row32(int tile, int rho) {
  return 64 * ((rho >> 2) & 1) + 16 * tile + 4 * (rho >> 3) + (rho & 3);
}

// Sub-plans of split and layer plans whose channels come from rows of at most 128 columns
// (a multiple of 8): the rotation with the channel selection folded in, K_h = K P_h, where
// P_h sends column c of the input row to coordinate i when chan_h[i] = c (the other columns
// get zero weight), in fp16 with k = the input column, one table per head; and per head the
// 16-bit lane masks of the selected columns, with which the encoder zeroes the unselected
// columns before the norm.  The encoder then reads whole rows with 16-byte loads instead of
// gathering channels.  D = 128 (with the 32x32 tables): the 32x32 encoder's layout, masks
// [k step of 16][lane half][word]; D <= 64 (with rotk16): rotk16's layout over 4 k steps of
// 32 columns, masks [k step][lane group][word] (word w: columns 2w and 2w + 1 of the 8 a lane
// reads).
void folded_operand_tables(SubHost& h, const std::vector<int64_t>& K, int n_heads, int cols) {
  if (h.chan.empty() || cols > 128 || cols % 8 != 0) return;
  const int D = h.D;
  const bool wide = D == 128 && !h.k16_32.empty();
  const bool narrow = D <= 64 && !h.rotk16.empty() && !h.S.empty();
  if (!wide && !narrow) return;
  const size_t per = wide ? (size_t)4 * 8 * 64 * 8 : (size_t)(D / 16) * 4 * 64 * 8;
  h.kf16.assign(per * n_heads, 0);
  h.xmask.assign((size_t)64 * n_heads, 0);
  std::vector<int> inv(cols);
  auto kval = [&](int row, int col) -> uint16_t {
    const int i = col < cols ? inv[col] : -1;
    return i >= 0 ? fp16_bits_of_small_int(K[(size_t)row * D + i]) : 0;
  };
  auto mask_word = [&](int c0) -> uint32_t {
    const uint32_t lo = (c0 < cols && inv[c0] >= 0) ? 0xFFFFu : 0u;
    const uint32_t hi = (c0 + 1 < cols && inv[c0 + 1] >= 0) ? 0xFFFF0000u : 0u;
    return lo | hi;
  };
  for (int hd = 0; hd < n_heads; ++hd) {
    std::fill(inv.begin(), inv.end(), -1);
    for (int i = 0; i < h.d; ++i) inv[h.chan[(size_t)hd * h.d + i]] = i;
    uint16_t* kf = h.kf16.data() + per * hd;
    uint32_t* mw = h.xmask.data() + (size_t)64 * hd;
    if (wide) {
      for (int t = 0; t < 4; ++t)
        for (int l = 0; l < 64; ++l)
          for (int ks = 0; ks < 8; ++ks)
            for (int e = 0; e < 8; ++e)
              kf[(((size_t)t * 8 + ks) * 64 + l) * 8 + e] =
                  kval(permuted_row32(t, l % 32), 16 * ks + 8 * (l / 32) + e);
      for (int ks = 0; ks < 8; ++ks)
        for (int hh = 0; hh < 2; ++hh)
          for (int w = 0; w < 4; ++w) mw[(ks * 2 + hh) * 4 + w] = mask_word(16 * ks + 8 * hh + 2 * w);
    } else {
      for (int jt = 0; jt < D / 16; ++jt)
        for (int ks = 0; ks < 4; ++ks)
          for (int l = 0; l < 64; ++l)
            for (int e = 0; e < 8; ++e)
              kf[(((size_t)jt * 4 + ks) * 64 + l) * 8 + e] =
                  kval(permuted_row(D, jt, l % 16), 32 * ks + 8 * (l / 16) + e);
      for (int ks = 0; ks < 4; ++ks)
        for (int G = 0; G < 4; ++G)
          for (int w = 0; w < 4; ++w) mw[(ks * 4 + G) * 4 + w] = mask_word(32 * ks + 8 * G + 2 * w);
    }
  }
}

// fp16 bit pattern of v when v is exactly representable (normal or subnormal), else false.
bool fp16_bits_exact(double v, uint16_t* out) {
  if (v == 0.0) { *out = std::signbit(v) ? 0x8000u : 0u; return true; }
  const uint16_t sign = v < 0 ? 0x8000u : 0u;
  const double a = std::fabs(v);
  int e;
  const double m = std::frexp(a, &e);             // a = m 2^e, m in [0.5, 1)
  if (e > 16) return false;                       // beyond the largest fp16
  if (e >= -13) {                                 // normal: 11 significant bits
    const double q = std::ldexp(m, 11);
    if (q != std::floor(q)) return false;
    *out = (uint16_t)(sign | (uint32_t)(e - 1 + 15) << 10 | ((uint32_t)q & 0x3FFu));
    return true;
  }
  const double q = std::ldexp(a, 24);             // subnormal: multiples of 2^-24
  if (q != std::floor(q) || q >= 1024.0) return false;
  *out = (uint16_t)(sign | (uint32_t)q);
  return true;
}

// fp8 e4m3 (bias 7, 3 mantissa bits, subnormals in steps of 2^-9, largest 448), rounded to
// nearest with ties to even; magnitudes past 448 saturate.
uint8_t e4m3_rne_bits(double v) {
  const uint8_t sign = std::signbit(v) ? 0x80u : 0u;
  double a = std::fabs(v);
  if (a >= 448.0) return sign | 0x7Eu;
  int e;
  std::frexp(a, &e);                              // a in [2^(e-1), 2^e)
  int ex = e - 1;                                 // unbiased exponent of a
  if (ex < -6) ex = -6;                           // subnormal range shares 2^-6's step
  const double step = std::ldexp(1.0, ex - 3);
  double q = std::nearbyint(a / step);            // ties to even (default rounding mode)
  double r = q * step;
  if (r == 0.0) return sign;
  std::frexp(r, &e);
  const int er = e - 1;
  if (er < -6) return sign | (uint8_t)(int)std::ldexp(r, 9);           // subnormal: m 2^-9
  const int mant = (int)(std::ldexp(r, -er) * 8.0) - 8;
  return sign | (uint8_t)((er + 7) << 3) | (uint8_t)mant;
}

// Operand tables of the D = 128 32x32 encoder (see encode128.hip); left empty when K or
// 2^8 S is not exact in fp16 (the 16x16 encoder then serves the plan).
void mfma32_operand_tables(SubHost& h, const std::vector<int64_t>& K) {
  if (h.D != 128 || h.S.empty() || h.rotk16.empty()) return;
  const int D = 128;
  std::vector<uint16_t> k16((size_t)4 * 8 * 64 * 8), s16((size_t)4 * 8 * 64 * 8);
  std::vector<uint8_t> s8((size_t)4 * 2 * 64 * 32);
  for (int t = 0; t < 4; ++t)
    for (int l = 0; l < 64; ++l) {
      const int row = permuted_row32(t, l % 32), hh = l / 32;
      for (int ks = 0; ks < 8; ++ks)
        for (int e = 0; e < 8; ++e) {
          const size_t at = (((size_t)t * 8 + ks) * 64 + l) * 8 + e;
          k16[at] = fp16_bits_of_small_int(K[(size_t)row * D + 16 * ks + 8 * hh + e]);
          const uint32_t sb = (uint32_t)h.S[(size_t)row * D + 64 * hh + 8 * ks + e] << 16;
          float sf;
          memcpy(&sf, &sb, 4);
          if (!fp16_bits_exact(256.0 * (double)sf, &s16[at])) return;
        }
      for (int q = 0; q < 2; ++q)
        for (int e = 0; e < 32; ++e) {
          const uint32_t sb = (uint32_t)h.S[(size_t)row * D + 64 * hh + 32 * q + e] << 16;
          float sf;
          memcpy(&sf, &sb, 4);
          s8[(((size_t)t * 2 + q) * 64 + l) * 32 + e] = e4m3_rne_bits((double)sf);
        }
    }
  h.k16_32 = std::move(k16);
  h.s16_32 = std::move(s16);
  h.s8_32 = std::move(s8);
}

// Coefficients a_S of the parity planes of odd subsets S of the R index bits:
// c[idx] = sum_S a_S * chi_S(idx), chi_S = prod_{m in S} (2 b_m - 1), exact for a
// codebook symmetric about zero (even subsets have zero weight).
bool plane_coefficients(const std::vector<double>& lev, int R, float* coef, uint8_t* mask,
                        int* n_planes, float* coef_sum) {
  const int L = 1 << R;
  int np = 0;
  double sum = 0.0;
  std::vector<double> a(L, 0.0);
  for (int S = 1; S < L; ++S) {
    double acc = 0.0;
    for (int idx = 0; idx < L; ++idx) {
      int chi = 1;
      for (int m = 0; m < R; ++m)
        if ((S >> m) & 1) chi *= ((idx >> m) & 1) ? 1 : -1;
      acc += lev[idx] * chi;
    }
    a[S] = acc / L;
  }
  for (int S = 1; S < L; ++S) {
    if (__builtin_popcount(S) % 2 == 0) continue;
    coef[np] = (float)a[S];
    mask[np] = (uint8_t)S;
    sum += a[S];
    ++np;
  }
  // reconstruct every level from the odd planes
  for (int idx = 0; idx < L; ++idx) {
    double v = 0.0;
    for (int S = 1; S < L; ++S) {
      if (__builtin_popcount(S) % 2 == 0) continue;
      int chi = 1;
      for (int m = 0; m < R; ++m)
        if ((S >> m) & 1) chi *= ((idx >> m) & 1) ? 1 : -1;
      v += a[S] * chi;
    }
    if (std::fabs(v - lev[idx]) > 1e-12) return false;
  }
  *n_planes = np;
  *coef_sum = (float)sum;
  return true;
}

}  // namespace

extern "C" {

const char* tq_status_string(tq_status status) {
  switch (status) {
    case TQ_OK: return "ok";
    case TQ_EINVAL: return "invalid argument";
    case TQ_ENOMEM: return "out of memory";
    case TQ_EDEVICE: return "HIP device error";
    case TQ_EUNSUPPORTED: return "unsupported";
  }
  return "unknown status";
}

tq_status tq_codebook(int D, int R, double* levels, double* thresholds) {
  if (D < 3 || D > 65536 || R < 1 || R > 8 || !levels || !thresholds) return TQ_EINVAL;
  solve_codebook(D, R, levels, thresholds);
  return TQ_OK;
}

tq_status tq_rotation_signs(uint64_t seed, int subset, int D, int8_t* signs) {
  if (D < 32 || D > 65536 || (D & (D - 1)) || subset < 0 || subset > 1 || !signs) return TQ_EINVAL;
  std::vector<uint32_t> w(3 * (D / 32));
  sign_words(seed, subset, D, w.data());
  for (int r = 0; r < 3; ++r)
    for (int i = 0; i < D; ++i)
      signs[r * D + i] = ((w[r * (D / 32) + i / 32] >> (i % 32)) & 1u) ? -1 : 1;
  return TQ_OK;
}

tq_status tq_qjl_matrix(uint64_t seed, int subset, int k, int D, uint16_t* S_bf16) {
  if (k < 1 || k > 65536 || D < 1 || D > 65536 || subset < 0 || subset > 1 || !S_bf16)
    return TQ_EINVAL;
  qjl_matrix_bf16(seed, subset, k, D, S_bf16);
  return TQ_OK;
}

}  // extern "C"

namespace {

// Both plan kinds: inner-product (R = b - 1 index bits + QJL signs) and TurboQuant-MSE
// (R = b index bits, no QJL matrix).  Arguments are validated by the callers.
// outlier_mask: [n_heads][d] (one mask per head of a layer plan; every head selects the same
// number of channels), or null with n_heads = 1.
tq_status create_plan(int d, int bits, uint64_t seed, const uint8_t* outlier_mask,
                      int outlier_bits, bool mse, tq_plan** out, int n_heads = 1) {
  *out = nullptr;
  std::vector<SubHost> subs;
  if (outlier_mask) {
    if (outlier_bits < 2 || outlier_bits > kMaxR + 1) return TQ_EINVAL;
    SubHost reg, out_s;
    int n_out = -1;
    for (int h = 0; h < n_heads; ++h) {
      const uint8_t* m = outlier_mask + (size_t)h * d;
      int cnt = 0;
      for (int c = 0; c < d; ++c) {
        (m[c] ? out_s.chan : reg.chan).push_back(c);
        cnt += m[c] ? 1 : 0;
      }
      if (n_out >= 0 && cnt != n_out) return TQ_EINVAL;   // every head: the same count
      n_out = cnt;
    }
    reg.d = (int)reg.chan.size() / n_heads; reg.R = bits - 1;
    out_s.d = (int)out_s.chan.size() / n_heads; out_s.R = outlier_bits - 1;
    if (reg.d == 0 || out_s.d == 0) return TQ_EINVAL;
    subs.push_back(std::move(reg));
    subs.push_back(std::move(out_s));
  } else {
    SubHost s;
    s.d = d; s.R = mse ? bits : bits - 1;
    subs.push_back(std::move(s));
  }
  int dev = -1;
  if (!current_device(&dev)) return TQ_EDEVICE;

  tq_plan* plan = new (std::nothrow) tq_plan();
  if (!plan) return TQ_ENOMEM;
  plan->device = dev;
  plan->seed = seed;
  plan->bits[0] = bits;
  plan->bits[1] = outlier_mask ? outlier_bits : 0;
  PlanDev& pd = plan->dev;
  pd.d = d;
  pd.nsub = (int)subs.size();
  pd.rec_bytes = 0;
  pd.n_heads = n_heads;

  // host tables and device layout
  size_t bytes = 0;
  size_t off_sign[2] = {0, 0}, off_S[2] = {0, 0}, off_chan[2] = {0, 0};
  size_t off_rotk[2] = {0, 0}, off_rotk16[2] = {0, 0}, off_rotkt16[2] = {0, 0}, off_sperm[2] = {0, 0};
  size_t off_k16_32[2] = {0, 0}, off_s16_32[2] = {0, 0}, off_s8_32[2] = {0, 0};
  size_t off_kf16[2] = {0, 0}, off_xmask[2] = {0, 0};
  auto take = [&](size_t b) { size_t o = bytes; bytes += (b + 255) / 256 * 256; return o; };
  for (int i = 0; i < pd.nsub; ++i) {
    SubHost& h = subs[i];
    h.D = padded_length(h.d);
    const int L = 1 << h.R;
    h.lev.resize(L);
    h.thr.resize(L - 1);
    solve_codebook(h.D, h.R, h.lev.data(), h.thr.data());
    h.signs.resize(3 * (h.D / 32));
    sign_words(seed, i, h.D, h.signs.data());
    if (!mse) {
      h.S.resize((size_t)h.D * h.D);
      qjl_matrix_bf16(seed, i, h.D, h.D, h.S.data());
    }
    SubDev& s = pd.sub[i];
    memset(&s, 0, sizeof(s));
    s.d = h.d;
    s.D = h.D;
    s.logD = __builtin_ctz(h.D);
    s.R = h.R;
    s.k = mse ? 0 : h.D;
    s.mse = mse ? 1 : 0;
    s.rec_off = pd.rec_bytes;
    s.rec_sub = mse ? record_bytes_mse_of(h.D, h.R) : record_bytes_of(h.D, h.R);
    pd.rec_bytes += s.rec_sub;
    s.inv_scale = (float)std::pow((double)h.D, -1.5);
    for (int l = 0; l < L; ++l) s.lev[l] = (float)h.lev[l];
    for (int j = 0; j < L - 1; ++j) s.thr[j] = (float)h.thr[j];
    if (!plane_coefficients(h.lev, h.R, s.coef, s.plane_mask, &s.n_planes, &s.coef_sum)) {
      delete plan;
      return TQ_EDEVICE;
    }
    off_sign[i] = take(h.signs.size() * 4);
    if (!h.S.empty()) off_S[i] = take(h.S.size() * 2);
    if (!h.chan.empty()) off_chan[i] = take(h.chan.size() * 4);
    if (h.D <= kMfmaMaxD) {
      mfma_operand_tables(h);
      if (!h.chan.empty())
        folded_operand_tables(h, rotation_integer_matrix(h.signs, h.D), n_heads, d);
      off_rotk[i] = take(h.rotk.size() * 2);
      off_rotk16[i] = take(h.rotk16.size() * 2);
      off_rotkt16[i] = take(h.rotkt16.size() * 2);
      off_sperm[i] = take(h.sperm.size() * 2);
      off_k16_32[i] = take(h.k16_32.size() * 2);
      off_s16_32[i] = take(h.s16_32.size() * 2);
      off_s8_32[i] = take(h.s8_32.size());
      off_kf16[i] = take(h.kf16.size() * 2);
      off_xmask[i] = take(h.xmask.size() * 4);
    }
  }
  void* mem = nullptr;
  hipError_t e = hipMalloc(&mem, bytes);
  if (e != hipSuccess) {
    delete plan;
    return e == hipErrorOutOfMemory ? TQ_ENOMEM : TQ_EDEVICE;
  }
  plan->dev_alloc = mem;
  uint8_t* base = static_cast<uint8_t*>(mem);
  for (int i = 0; i < pd.nsub; ++i) {
    SubHost& h = subs[i];
    SubDev& s = pd.sub[i];
    e = hipMemcpy(base + off_sign[i], h.signs.data(), h.signs.size() * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.S.empty())
      e = hipMemcpy(base + off_S[i], h.S.data(), h.S.size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.chan.empty())
      e = hipMemcpy(base + off_chan[i], h.chan.data(), h.chan.size() * 4, hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.rotk.empty())
      e = hipMemcpy(base + off_rotk[i], h.rotk.data(), h.rotk.size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.rotk16.empty())
      e = hipMemcpy(base + off_rotk16[i], h.rotk16.data(), h.rotk16.size() * 2,
                    hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.rotkt16.empty())
      e = hipMemcpy(base + off_rotkt16[i], h.rotkt16.data(), h.rotkt16.size() * 2,
                    hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.sperm.empty())
      e = hipMemcpy(base + off_sperm[i], h.sperm.data(), h.sperm.size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.k16_32.empty())
      e = hipMemcpy(base + off_k16_32[i], h.k16_32.data(), h.k16_32.size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.s16_32.empty())
      e = hipMemcpy(base + off_s16_32[i], h.s16_32.data(), h.s16_32.size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.s8_32.empty())
      e = hipMemcpy(base + off_s8_32[i], h.s8_32.data(), h.s8_32.size(), hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.kf16.empty())
      e = hipMemcpy(base + off_kf16[i], h.kf16.data(), h.kf16.size() * 2, hipMemcpyHostToDevice);
    if (e == hipSuccess && !h.xmask.empty())
      e = hipMemcpy(base + off_xmask[i], h.xmask.data(), h.xmask.size() * 4, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(mem);
      delete plan;
      return TQ_EDEVICE;
    }
    s.signs = reinterpret_cast<const uint32_t*>(base + off_sign[i]);
    s.S = h.S.empty() ? nullptr : reinterpret_cast<const uint16_t*>(base + off_S[i]);
    s.chan = h.chan.empty() ? nullptr : reinterpret_cast<const int32_t*>(base + off_chan[i]);
    s.rotk = h.rotk.empty() ? nullptr : reinterpret_cast<const uint16_t*>(base + off_rotk[i]);
    s.rotk16 = h.rotk16.empty() ? nullptr : reinterpret_cast<const uint16_t*>(base + off_rotk16[i]);
    s.rotkt16 = h.rotkt16.empty() ? nullptr : reinterpret_cast<const uint16_t*>(base + off_rotkt16[i]);
    s.sperm = h.sperm.empty() ? nullptr : reinterpret_cast<const uint16_t*>(base + off_sperm[i]);
    const bool e32 = !h.k16_32.empty() && !h.s16_32.empty() && !h.s8_32.empty();
    s.k16_32 = e32 ? reinterpret_cast<const uint16_t*>(base + off_k16_32[i]) : nullptr;
    s.s16_32 = e32 ? reinterpret_cast<const uint16_t*>(base + off_s16_32[i]) : nullptr;
    s.s8_32 = e32 ? reinterpret_cast<const uint8_t*>(base + off_s8_32[i]) : nullptr;
    const bool fold = !h.kf16.empty() && !h.xmask.empty();
    s.kfold = fold ? reinterpret_cast<const uint16_t*>(base + off_kf16[i]) : nullptr;
    s.xmask = fold ? reinterpret_cast<const uint32_t*>(base + off_xmask[i]) : nullptr;
    s.x_cols = fold ? d : 0;
  }
  *out = plan;
  return TQ_OK;
}

bool is_mse(const tq_plan* p) { return p->dev.sub[0].mse != 0; }

}  // namespace

extern "C" {

tq_status tq_plan_create(int d, int bits, uint64_t seed, const uint8_t* outlier_mask,
                         int outlier_bits, tq_plan** out) {
  if (!out) return TQ_EINVAL;
  *out = nullptr;
  if (d < 1 || d > kMaxD || bits < 2 || bits > kMaxR + 1) return TQ_EINVAL;
  if (outlier_mask && (outlier_bits < 2 || outlier_bits > kMaxR + 1)) return TQ_EINVAL;
  return create_plan(d, bits, seed, outlier_mask, outlier_bits, false, out);
}

tq_status tq_plan_create_heads(int d, int bits, uint64_t seed, int n_heads,
                               const uint8_t* outlier_masks, int outlier_bits, tq_plan** out) {
  if (!out) return TQ_EINVAL;
  *out = nullptr;
  if (d < 2 || d > kMfmaMaxD || bits < 2 || bits > kMaxR + 1 || n_heads < 1 ||
      n_heads > kMaxHeads || !outlier_masks || outlier_bits < 2 || outlier_bits > kMaxR + 1)
    return TQ_EINVAL;
  return create_plan(d, bits, seed, outlier_masks, outlier_bits, false, out, n_heads);
}

tq_status tq_plan_create_mse(int d, int bits, uint64_t seed, tq_plan** out) {
  if (!out) return TQ_EINVAL;
  *out = nullptr;
  if (d < 1 || d > kMaxD || bits < 1 || bits > kMaxR) return TQ_EINVAL;
  return create_plan(d, bits, seed, nullptr, 0, true, out);
}

void tq_plan_destroy(tq_plan* plan) {
  if (!plan) return;
  if (plan->dev_alloc) (void)hipFree(plan->dev_alloc);
  delete plan;
}

tq_status tq_plan_info(const tq_plan* plan, tq_plan_desc* desc) {
  if (!plan || !desc) return TQ_EINVAL;
  memset(desc, 0, sizeof(*desc));
  desc->d = plan->dev.d;
  desc->n_subplans = plan->dev.nsub;
  desc->record_bytes = plan->dev.rec_bytes;
  desc->mode = is_mse(plan) ? TQ_MODE_MSE : TQ_MODE_INNER_PRODUCT;
  desc->n_heads = plan->dev.n_heads;
  for (int i = 0; i < plan->dev.nsub; ++i) {
    const SubDev& s = plan->dev.sub[i];
    desc->sub[i].d = s.d;
    desc->sub[i].D = s.D;
    desc->sub[i].R = s.R;
    desc->sub[i].k = s.k;
    desc->sub[i].record_offset = s.rec_off;
    desc->sub[i].record_bytes = s.rec_sub;
  }
  return TQ_OK;
}

tq_status tq_encode_groups(const tq_plan* plan, const void* x, tq_dtype dt, int64_t n_groups,
                           int64_t n_per_group, int64_t ldx, void* codes, void* stream) {
  if (!plan || n_groups < 0 || n_per_group < 0 || (dt != TQ_F32 && dt != TQ_BF16))
    return TQ_EINVAL;
  if (n_groups == 0 || n_per_group == 0) return TQ_OK;
  const int es = dt == TQ_BF16 ? 2 : 4;
  if (!x || !codes || ldx < plan->dev.d || (uintptr_t)x % es || (uintptr_t)codes % 16)
    return TQ_EINVAL;
  if (n_groups > 65535) return TQ_EINVAL;
  if (!plan_device_ok(plan)) return TQ_EINVAL;
  bool grouped_ok = true;   // the group grid runs on the D <= 128 encoders
  for (int i = 0; i < plan->dev.nsub; ++i) grouped_ok = grouped_ok && plan->dev.sub[i].D <= kMfmaMaxD;
  if (!grouped_ok && n_groups > 1) {
    if (plan->dev.n_heads > 1) return TQ_EUNSUPPORTED;
    // one channel list: the groups are simply consecutive rows
    for (int i = 0; i < plan->dev.nsub; ++i) {
      const int rc = launch_encode(plan->dev, i, x, (int)dt, n_groups * n_per_group, ldx,
                                   static_cast<uint8_t*>(codes), stream);
      if (rc) return from_hip(rc);
    }
    return TQ_OK;
  }
  for (int i = 0; i < plan->dev.nsub; ++i) {
    const int rc = launch_encode(plan->dev, i, x, (int)dt, n_per_group, ldx,
                                 static_cast<uint8_t*>(codes), stream, n_groups);
    if (rc) return from_hip(rc);
  }
  return TQ_OK;
}

tq_status tq_encode(const tq_plan* plan, const void* x, tq_dtype dt, int64_t n, int64_t ldx,
                    void* codes, void* stream) {
  if (!plan || n < 0 || (dt != TQ_F32 && dt != TQ_BF16)) return TQ_EINVAL;
  if (plan->dev.n_heads > 1) return TQ_EINVAL;   // a layer plan's rows need their head
  if (n == 0) return TQ_OK;
  const int es = dt == TQ_BF16 ? 2 : 4;
  if (!x || !codes || ldx < plan->dev.d || (uintptr_t)x % es || (uintptr_t)codes % 16)
    return TQ_EINVAL;
  if (!plan_device_ok(plan)) return TQ_EINVAL;
  for (int i = 0; i < plan->dev.nsub; ++i) {
    const int rc = launch_encode(plan->dev, i, x, (int)dt, n, ldx, static_cast<uint8_t*>(codes), stream);
    if (rc) return from_hip(rc);
  }
  return TQ_OK;
}

tq_status tq_score(const tq_plan* plan, const void* q, tq_dtype dt, int64_t nq_per_group,
                   int64_t n_groups, int64_t ldq, const void* codes, int64_t n, float* scores,
                   void* stream) {
  if (!plan || nq_per_group < 0 || n_groups < 0 || n < 0 || (dt != TQ_F32 && dt != TQ_BF16))
    return TQ_EINVAL;
  if (nq_per_group == 0 || n_groups == 0 || n == 0) return TQ_OK;
  const int es = dt == TQ_BF16 ? 2 : 4;
  if (!q || !codes || !scores || ldq < plan->dev.d || (uintptr_t)q % es || (uintptr_t)codes % 16 ||
      (uintptr_t)scores % 4)
    return TQ_EINVAL;
  if (nq_per_group * n_groups > (int64_t)1 << 31 || n_groups > 65535 * 64) return TQ_EINVAL;
  if (n_groups % plan->dev.n_heads) return TQ_EINVAL;   // group g reads head g % n_heads
  if (!plan_device_ok(plan)) return TQ_EINVAL;
  return from_hip(launch_score(plan->dev, q, (int)dt, nq_per_group, n_groups, ldq,
                               static_cast<const uint8_t*>(codes), n, scores, stream));
}

tq_status tq_score_noalloc(const tq_plan* plan, const void* q, tq_dtype dt, int64_t nq_per_group,
                           int64_t n_groups, int64_t ldq, const void* codes, int64_t n,
                           float* scores, void* stream) {
  if (!plan || nq_per_group < 0 || n_groups < 0 || n < 0 || (dt != TQ_F32 && dt != TQ_BF16))
    return TQ_EINVAL;
  if (nq_per_group == 0 || n_groups == 0 || n == 0) return TQ_OK;
  const int es = dt == TQ_BF16 ? 2 : 4;
  if (!q || !codes || !scores || ldq < plan->dev.d || (uintptr_t)q % es || (uintptr_t)codes % 16 ||
      (uintptr_t)scores % 4)
    return TQ_EINVAL;
  if (nq_per_group * n_groups > (int64_t)1 << 31 || n_groups > 65535 * 64) return TQ_EINVAL;
  if (n_groups % plan->dev.n_heads) return TQ_EINVAL;   // group g reads head g % n_heads
  if (!plan_device_ok(plan)) return TQ_EINVAL;
  const int rc = launch_score_noalloc(plan->dev, q, (int)dt, nq_per_group, n_groups, ldq,
                                      static_cast<const uint8_t*>(codes), n, scores, stream);
  if (rc == (int)hipErrorOutOfMemory) return TQ_EINVAL;   // workspace beyond the fixed array
  return from_hip(rc);
}

tq_status tq_topk(const float* scores, int64_t nq, int64_t n, int k, int64_t* ids, float* vals,
                  void* stream) {
  if (nq < 0 || n < 0 || k < 1 || k > 64 || k > n || n >= ((int64_t)1 << 31)) return TQ_EINVAL;
  if (nq == 0) return TQ_OK;
  if (!scores || !ids || !vals || (uintptr_t)scores % 4 || (uintptr_t)ids % 8 || (uintptr_t)vals % 4)
    return TQ_EINVAL;
  int dev;
  if (hipGetDevice(&dev) != hipSuccess) return TQ_EDEVICE;
  return from_hip(launch_topk(scores, nq, n, k, ids, vals, stream));
}

tq_status tq_score_topk(const tq_plan* plan, const void* q, tq_dtype dt, int64_t nq_per_group,
                        int64_t n_groups, int64_t ldq, const void* codes, int64_t n, int k,
                        int64_t* ids, float* vals, void* stream) {
  if (!plan || nq_per_group < 0 || n_groups < 0 || (dt != TQ_F32 && dt != TQ_BF16) || k < 1 ||
      k > 64 || k > n || n >= ((int64_t)1 << 31))
    return TQ_EINVAL;
  if (nq_per_group == 0 || n_groups == 0) return TQ_OK;
  const int es = dt == TQ_BF16 ? 2 : 4;
  if (!q || !codes || !ids || !vals || ldq < plan->dev.d || (uintptr_t)q % es ||
      (uintptr_t)codes % 16 || (uintptr_t)ids % 8 || (uintptr_t)vals % 4)
    return TQ_EINVAL;
  if (nq_per_group * n_groups > (int64_t)1 << 31 || n_groups > 65535 * 64) return TQ_EINVAL;
  if (n_groups % plan->dev.n_heads) return TQ_EINVAL;
  if (!plan_device_ok(plan)) return TQ_EINVAL;
  return from_hip(launch_score_topk(plan->dev, q, (int)dt, nq_per_group, n_groups, ldq,
                                    static_cast<const uint8_t*>(codes), n, k, ids, vals, stream));
}

tq_status tq_dequantize(const tq_plan* plan, const void* codes, int64_t n, void* x, tq_dtype dt,
                        int64_t ldx, void* stream) {
  if (!plan || n < 0 || (dt != TQ_F32 && dt != TQ_BF16)) return TQ_EINVAL;
  if (n == 0) return TQ_OK;
  const int es = dt == TQ_BF16 ? 2 : 4;
  if (!codes || !x || ldx < plan->dev.d || (uintptr_t)codes % 16 || (uintptr_t)x % es)
    return TQ_EINVAL;
  if (plan->dev.n_heads > 1) return TQ_EUNSUPPORTED;
  if (!plan_device_ok(plan)) return TQ_EINVAL;
  return from_hip(launch_dequantize(plan->dev, static_cast<const uint8_t*>(codes), n, x, (int)dt,
                                    ldx, stream));
}

tq_status tq_attend(const tq_plan* vplan, const float* logits, int64_t nq_per_group,
                    int64_t n_groups, int64_t n, float scale, const void* vcodes, void* out,
                    tq_dtype dt, int64_t ldo, void* stream) {
  if (!vplan || nq_per_group < 0 || n_groups < 0 || n < 1 || (dt != TQ_F32 && dt != TQ_BF16) ||
      !std::isfinite(scale))
    return TQ_EINVAL;
  if (nq_per_group == 0 || n_groups == 0) return TQ_OK;
  if (vplan->dev.nsub != 1 || vplan->dev.sub[0].R > 4) return TQ_EUNSUPPORTED;
  const int es = dt == TQ_BF16 ? 2 : 4;
  if (!logits || !vcodes || !out || ldo < vplan->dev.d || (uintptr_t)logits % 4 ||
      (uintptr_t)vcodes % 16 || (uintptr_t)out % es)
    return TQ_EINVAL;
  if (n_groups > 65535 || (nq_per_group + 3) / 4 > 65535 || (n + 1023) / 1024 > ((int64_t)1 << 31))
    return TQ_EINVAL;
  // one combine workgroup per query row; at most 4 (chunk run, group, row tile) items per
  // pass-1 workgroup
  const int64_t rows = nq_per_group * n_groups;
  if (rows > 0x7FFFFFFF || ((n + 1023) / 1024) > ((int64_t)1 << 33) / rows) return TQ_EINVAL;
  if (vplan->dev.n_heads > 1) return TQ_EUNSUPPORTED;
  if (!plan_device_ok(vplan)) return TQ_EINVAL;
  return from_hip(launch_attend(vplan->dev, logits, nq_per_group, n_groups, n, scale,
                                static_cast<const uint8_t*>(vcodes), out, (int)dt, ldo, stream));
}

tq_status tq_calibrate_outliers(const void* x, tq_dtype dt, int64_t n, int64_t ldx, int d,
                                int n_out, double* var, uint8_t* mask, void* stream) {
  if (n < 1 || d < 1 || d > 65536 || n_out < 0 || n_out > d || (dt != TQ_F32 && dt != TQ_BF16))
    return TQ_EINVAL;
  const int es = dt == TQ_BF16 ? 2 : 4;
  if (!x || !var || !mask || ldx < d || (uintptr_t)x % es || (uintptr_t)var % 8) return TQ_EINVAL;
  int dev;
  if (hipGetDevice(&dev) != hipSuccess) return TQ_EDEVICE;
  return from_hip(launch_calibrate_outliers(x, dt == TQ_BF16, n, ldx, d, n_out, var, mask, stream));
}

tq_status tq_encode_scatter(const tq_plan* plan, const void* x, tq_dtype dt, int64_t n, int64_t ldx,
                            void* cache, int64_t cache_rows, const int64_t* index, void* stream) {
  if (!plan || n < 0 || cache_rows < 0 || (dt != TQ_F32 && dt != TQ_BF16)) return TQ_EINVAL;
  if (n == 0) return TQ_OK;
  const int es = dt == TQ_BF16 ? 2 : 4;
  if (!x || !cache || !index || ldx < plan->dev.d || (uintptr_t)x % es || (uintptr_t)cache % 16 ||
      (uintptr_t)index % 8)
    return TQ_EINVAL;
  if (!plan_device_ok(plan)) return TQ_EINVAL;
  if (plan->dev.n_heads > 1 && n > 65535) return TQ_EINVAL;
  return from_hip(launch_encode_scatter(plan->dev, x, (int)dt, n, ldx, static_cast<uint8_t*>(cache),
                                        cache_rows, index, stream));
}

tq_status tq_rerank(const void* q, tq_dtype qdt, int64_t nq, int64_t ldq, const void* x,
                    tq_dtype xdt, int64_t n, int64_t ldx, int d, const int64_t* cand, int kc, int k,
                    int64_t* ids, float* vals, void* stream) {
  if (nq < 0 || n < 0 || d < 1 || d > 8192 || kc < 1 || kc > 256 || k < 1 || k > kc ||
      (qdt != TQ_F32 && qdt != TQ_BF16) || (xdt != TQ_F32 && xdt != TQ_BF16))
    return TQ_EINVAL;
  if (nq == 0) return TQ_OK;
  const int qs = qdt == TQ_BF16 ? 2 : 4, xs = xdt == TQ_BF16 ? 2 : 4;
  if (!q || !cand || !ids || !vals || (n > 0 && !x) || ldq < d || ldx < d || (uintptr_t)q % qs ||
      (uintptr_t)x % xs || (uintptr_t)cand % 8 || (uintptr_t)ids % 8 || (uintptr_t)vals % 4)
    return TQ_EINVAL;
  int dev;
  if (hipGetDevice(&dev) != hipSuccess) return TQ_EDEVICE;
  return from_hip(launch_rerank(q, qdt == TQ_BF16, nq, ldq, x, xdt == TQ_BF16, n, ldx, d, cand,
                                kc, k, ids, vals, stream));
}

tq_status tq_qjl(const tq_plan* plan, int subplan, const float* r, int64_t n, uint32_t* beta,
                 void* stream) {
  if (!plan || subplan < 0 || subplan >= plan->dev.nsub || n < 0) return TQ_EINVAL;
  if (n == 0) return TQ_OK;
  if (!r || !beta || (uintptr_t)r % 4 || (uintptr_t)beta % 4) return TQ_EINVAL;
  if (plan->dev.n_heads > 1) return TQ_EUNSUPPORTED;
  if (!plan_device_ok(plan)) return TQ_EINVAL;
  if (is_mse(plan)) return TQ_EUNSUPPORTED;
  return from_hip(launch_qjl(plan->dev.sub[subplan], r, n, beta, stream));
}

}  // extern "C"
