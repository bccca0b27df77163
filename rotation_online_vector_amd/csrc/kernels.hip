// HIP kernels for gfx950 (CDNA4, wave64): encode (norm split, randomized Hadamard rotation,
// Lloyd-Max bucketize, bit-plane packing, QJL signs on bf16 MFMA), query preparation,
// scoring (bit-sliced fp8 x fp4 MFMA for D <= 128, a vector-unit scorer otherwise) and
// top-k.  The method is the one of the TurboQuant technical overview (intelliparadigm.com)
// and the TurboQuant deep dive (blog.hotdry.top); section references are given per kernel.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "device_common.h"

namespace tq {


// ============================================================================ encode
// Norm split, rotation z = Pi x / ||x|| with Pi = Ht S3 Ht S2 Ht S1 (TurboQuant technical
// overview §2.1.1-2.1.2; diagonal then transform, three rounds), Lloyd-Max bucketize
// idx = #{t_j <= z} (§1.2.2), residual r = z - c[idx] and its norm (§2.3.1), QJL signs
// beta = [S r >= 0] (§2.3.2) computed on bf16 MFMA with r split into two bf16 limbs.
//
// Layout inside a workgroup: a vector of length D is held by TPV = D/EPT lanes, each lane
// owning EPT consecutive coordinates, so the Walsh-Hadamard butterflies over the low
// log2(EPT) index bits stay in registers and the rest are lane exchanges.

template <int D> struct EncCfg {
  static constexpr int EPT = (D >= 2048) ? 32 : 16;      // coordinates per lane
  static constexpr int TPV = D / EPT;                      // lanes per vector
  static constexpr int VPP = kWave / TPV;                  // vectors per wave pass
  static constexpr int V = (D <= 32) ? 128 : (D <= 512) ? 64 : (D == 1024 ? 32 : 16);  // per tile
  static constexpr int RSTRIDE = D + 8;                    // bf16 row stride of residual limbs
};

// In-register + cross-lane fast Walsh-Hadamard transform (unnormalized) of one vector.
template <int EPT, int TPV>
__device__ __forceinline__ void fwht_lanes(float (&v)[EPT], int t) {
#pragma unroll
  for (int h = 1; h < EPT; h <<= 1) {
#pragma unroll
    for (int i = 0; i < EPT; i += 2 * h) {
#pragma unroll
      for (int j = i; j < i + h; ++j) {
        const float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int m = 1; m < TPV; m <<= 1) {
    const float sgn = (t & m) ? -1.0f : 1.0f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const float p = __shfl_xor(v[e], m);
      v[e] = fmaf(sgn, v[e], p);   // lower lane: v + p ; upper lane: p - v
    }
  }
}

template <int TPV>
__device__ __forceinline__ float lane_group_sum(float x) {
#pragma unroll
  for (int m = 1; m < TPV; m <<= 1) x += __shfl_xor(x, m);
  return x;
}

// QJL sign stage for V vectors whose residual limbs are in LDS.  Writes each 32-row word of
// signs to words[v * vstride + g * gstride + goff] (LDS).
template <int D, int V>
__device__ __forceinline__ void qjl_signs_mfma(const SubDev& s, const uint16_t* rhi,
                                               const uint16_t* rlo, uint32_t* words, int vstride,
                                               int gstride, int goff) {
  constexpr int RS = D + 8;
  constexpr int NG = D / 32;
  constexpr int NT = (V / 16) * NG;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  for (int task = wave; task < NT; task += kBlock / kWave) {
    const int vt = task / NG, g = task % NG;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const uint16_t* ah = rhi + (vt * 16 + col) * RS + 8 * grp;
    const uint16_t* al = rlo + (vt * 16 + col) * RS + 8 * grp;
    const uint16_t* b0p = s.S + (size_t)(32 * g + col) * D + 8 * grp;
    const uint16_t* b1p = b0p + (size_t)16 * D;
#pragma unroll 2
    for (int i0 = 0; i0 < D; i0 += 32) {
      const bf16x8 a_hi = *reinterpret_cast<const bf16x8*>(ah + i0);
      const bf16x8 a_lo = *reinterpret_cast<const bf16x8*>(al + i0);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(b0p + i0);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(b1p + i0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, b1, acc1, 0, 0, 0);
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, b1, acc1, 0, 0, 0);
    }
    // acc_T[e] at lane l: P[vector 4*(l/16)+e][row 32g + 16T + l%16]
    const uint64_t b00 = __ballot(acc0[0] >= 0.f), b01 = __ballot(acc0[1] >= 0.f);
    const uint64_t b02 = __ballot(acc0[2] >= 0.f), b03 = __ballot(acc0[3] >= 0.f);
    const uint64_t b10 = __ballot(acc1[0] >= 0.f), b11 = __ballot(acc1[1] >= 0.f);
    const uint64_t b12 = __ballot(acc1[2] >= 0.f), b13 = __ballot(acc1[3] >= 0.f);
    if (lane < 16) {
      const int v = lane, q = v >> 2, e = v & 3;
      const uint64_t b0 = e == 0 ? b00 : e == 1 ? b01 : e == 2 ? b02 : b03;
      const uint64_t b1 = e == 0 ? b10 : e == 1 ? b11 : e == 2 ? b12 : b13;
      const uint32_t lo = (uint32_t)(b0 >> (16 * q)) & 0xFFFFu;
      const uint32_t hi = (uint32_t)(b1 >> (16 * q)) & 0xFFFFu;
      words[(vt * 16 + v) * vstride + g * gstride + goff] = lo | (hi << 16);
    }
  }
}


// SPLIT: the QJL stage is left to qjl_gemm_kernel; the residual limbs go to a.rw_hi/rw_lo
// instead of LDS and the sign words of the records are written by that kernel.
// MSE: TurboQuant-MSE records (R = b index bits, then the norm): no residual, no QJL stage.
template <int D, int R, bool SPLIT = false, bool MSE = false>
__global__ void __launch_bounds__(kBlock) encode_kernel(EncodeArgs a) {
  using C = EncCfg<D>;
  constexpr int EPT = C::EPT, TPV = C::TPV, VPP = C::VPP, V = C::V, RS = C::RSTRIDE;
  constexpr int L = 1 << R;
  constexpr int W = MSE ? R : R + 1;   // words per 32-coordinate chunk of a record
  const SubDev& s = a.s;
  const int recw = s.rec_sub / 4;   // words per sub-record
  __shared__ __attribute__((aligned(16))) uint16_t rhi[SPLIT || MSE ? 8 : V * RS];
  __shared__ __attribute__((aligned(16))) uint16_t rlo[SPLIT || MSE ? 8 : V * RS];
  __shared__ __attribute__((aligned(16))) uint32_t rec[V * ((4 * (R + 1) * D / 32 + 8) / 4)];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = lane % TPV;                 // lane within its vector
  const int c0 = t * EPT;                   // first coordinate owned by this lane
  const int64_t tile0 = (int64_t)blockIdx.x * V;

  // sign bits of this lane's coordinates for the three rounds
  uint32_t sw[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) sw[r] = s.signs[r * (D / 32) + c0 / 32] >> (c0 % 32);

  constexpr int PASSES = V / (4 * VPP);
#pragma unroll 1
  for (int pass = 0; pass < PASSES; ++pass) {
    const int vl = wave * (V / 4) + pass * VPP + lane / TPV;   // vector within the tile
    const int64_t row = tile0 + vl;
    const bool live = row < a.n;
    float v[EPT];
    // ---- load (zero padding beyond d) ----
    if (live && a.vec_load && c0 + EPT <= s.d) {
      if (a.is_bf16) {
        const uint4* p = reinterpret_cast<const uint4*>(
            reinterpret_cast<const uint16_t*>(a.x) + row * a.ldx + c0);
#pragma unroll
        for (int q = 0; q < EPT / 8; ++q) {
          const uint4 u = p[q];
          const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            v[8 * q + 2 * h] = __uint_as_float(w[h] << 16);
            v[8 * q + 2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
          }
        }
      } else {
        const float4* p = reinterpret_cast<const float4*>(
            reinterpret_cast<const float*>(a.x) + row * a.ldx + c0);
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q) {
          const float4 u = p[q];
          v[4 * q] = u.x; v[4 * q + 1] = u.y; v[4 * q + 2] = u.z; v[4 * q + 3] = u.w;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = c0 + e;
        float val = 0.f;
        if (live && i < s.d) {
          const int64_t ch = s.chan ? s.chan[i] : i;
          if (a.is_bf16)
            val = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.x)[row * a.ldx + ch]);
          else
            val = reinterpret_cast<const float*>(a.x)[row * a.ldx + ch];
        }
        v[e] = val;
      }
    }
    // ---- norm ----
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) ss = fmaf(v[e], v[e], ss);
    ss = lane_group_sum<TPV>(ss);
    const float nrm = sqrtf(ss);
    // ---- rotation: three rounds of (+-1 diagonal, Walsh-Hadamard) ----
#pragma unroll
    for (int r = 0; r < 3; ++r) {
#pragma unroll
      for (int e = 0; e < EPT; ++e) v[e] = flip_sign(v[e], (sw[r] >> e) & 1u);
      fwht_lanes<EPT, TPV>(v, t);
    }
    const float scale = nrm > 0.f ? s.inv_scale / nrm : 0.f;
    // ---- bucketize (idx = #{t_j <= z}), residual ----
    float thr[L - 1], lev[L];
#pragma unroll
    for (int j = 0; j < L - 1; ++j) thr[j] = s.thr[j];
#pragma unroll
    for (int j = 0; j < L; ++j) lev[j] = s.lev[j];
    uint32_t planes[R];
#pragma unroll
    for (int m = 0; m < R; ++m) planes[m] = 0;
    float gg = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      const float z = v[e] * scale;
      int idx = 0;
      float lv = lev[0];
#pragma unroll
      for (int j = 0; j < L - 1; ++j) {
        const bool ge = z >= thr[j];
        idx += ge ? 1 : 0;
        lv = ge ? lev[j + 1] : lv;
      }
      const float rr = z - lv;
      gg = fmaf(rr, rr, gg);
      v[e] = rr;
#pragma unroll
      for (int m = 0; m < R; ++m) planes[m] |= (uint32_t)((idx >> m) & 1) << e;
    }
    if constexpr (!MSE) gg = lane_group_sum<TPV>(gg);
    // ---- residual limbs to LDS ----
    if constexpr (!MSE) {
      uint32_t hi[EPT / 2], lo[EPT / 2];
      const uint32_t sel_lo = neg_one_low_half();
#pragma unroll
      for (int e = 0; e < EPT; e += 2) {
        // two hardware round-to-nearest-even conversions per pair; the remainders read the
        // packed high limbs in place
        hi[e / 2] = pack_bf16_rne(v[e], v[e + 1]);
        lo[e / 2] = pack_bf16_rne(residual_below_bf16(hi[e / 2], sel_lo, v[e]),
                                  residual_below_bf16(hi[e / 2], 0xBF800000u, v[e + 1]));
      }
      uint4* ph;
      uint4* pl;
      if constexpr (SPLIT) {
        const int64_t rrow = live ? row : a.n - 1;   // dead lanes rewrite a real row's limbs...
        ph = reinterpret_cast<uint4*>(a.rw_hi + rrow * D + c0);
        pl = reinterpret_cast<uint4*>(a.rw_lo + rrow * D + c0);
      } else {
        ph = reinterpret_cast<uint4*>(rhi + vl * RS + c0);
        pl = reinterpret_cast<uint4*>(rlo + vl * RS + c0);
      }
      if (!SPLIT || live) {                           // ...so they store nothing instead
#pragma unroll
        for (int q = 0; q < EPT / 8; ++q) {
          ph[q] = make_uint4(hi[4 * q], hi[4 * q + 1], hi[4 * q + 2], hi[4 * q + 3]);
          pl[q] = make_uint4(lo[4 * q], lo[4 * q + 1], lo[4 * q + 2], lo[4 * q + 3]);
        }
      }
    }
    // ---- index bit-planes, norm and gamma into the staged record ----
    uint32_t* myrec = rec + vl * recw;
    if (EPT == 32) {
#pragma unroll
      for (int m = 0; m < R; ++m) myrec[(c0 / 32) * W + m] = planes[m];
    } else {
#pragma unroll
      for (int m = 0; m < R; ++m) {
        const uint32_t other = __shfl_xor(planes[m], 1);
        if ((t & 1) == 0) myrec[(c0 / 32) * W + m] = planes[m] | (other << 16);
      }
    }
    if (t == 0) {
      myrec[(D / 32) * W] = __float_as_uint(nrm);
      if constexpr (!MSE) myrec[(D / 32) * W + 1] = __float_as_uint(sqrtf(gg));
    }
  }
  __syncthreads();
  if constexpr (!SPLIT && !MSE) {
    qjl_signs_mfma<D, V>(s, rhi, rlo, rec, recw, R + 1, R);
    __syncthreads();
  }
  // ---- write records ----
  const int64_t nv = (a.n - tile0 < V) ? (a.n - tile0) : V;
  if (s.rec_sub == a.rec_bytes) {
    const int nw = (int)nv * recw;
    uint32_t* dst = reinterpret_cast<uint32_t*>(a.codes + tile0 * a.rec_bytes);
    if ((nw & 3) == 0) {
      for (int i = threadIdx.x; i < nw / 4; i += kBlock)
        reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(rec)[i];
    } else {
      for (int i = threadIdx.x; i < nw; i += kBlock) dst[i] = rec[i];
    }
  } else {
    for (int i = threadIdx.x; i < (int)nv * recw; i += kBlock) {
      const int vv = i / recw, w = i % recw;
      reinterpret_cast<uint32_t*>(a.codes + (tile0 + vv) * a.rec_bytes + s.rec_off)[w] = rec[i];
    }
  }
}

// ------------------------------------------------------------ QJL signs as a tiled GEMM
// For long vectors (D >= 1024) the projection P = R S^T of a batch of residuals R (two bf16
// limbs each, written by encode_kernel<.., SPLIT>) is one large product: streaming all of S
// (8 MiB at D = 2048) for every 16 vectors, as the fused kernel does, would move far more
// than the residuals themselves.  Block tile: 128 vectors x 256 rows of S, k steps of 32
// coordinates through double-buffered LDS; 8 waves, each 64 vectors x 64 rows (4 x 4 MFMA
// tiles, both limbs into one accumulator); a 1-D grid mapped to tiles per XCD (in the
// kernel).  The signs go straight into the records.  An LDS
// row is four 16-byte pieces stored at piece q ^ ((row / 2) % 4): the 16-byte stores of two
// consecutive rows and the fragment reads of eight consecutive rows then fall in distinct
// banks.
constexpr int kQgBN = 128, kQgBM = 256, kQgKS = 32, kQgRS = kQgKS;   // LDS row: 64 B, pieces swizzled
constexpr int kQgNQ = kQgKS / 8;          // 16-byte pieces per row and k step
constexpr int kQgNI = kQgBM * kQgNQ / 512; // pieces per thread, A and B alike

struct QjlGemmArgs {
  const uint16_t* rh;    // [nv][D]
  const uint16_t* rl;
  const uint16_t* S;     // [D][D] bf16
  uint8_t* codes;        // record of the batch's first vector
  int64_t nv;
  int rec_bytes, rec_off, R;
};

template <int D>
__global__ void __launch_bounds__(512) qjl_gemm_kernel(QjlGemmArgs a) {
  static_assert(D % kQgBM == 0 && D % kQgKS == 0, "whole blocks and k steps");
  static_assert(2 * kQgBN == kQgBM, "A (two limbs) and B have the same piece count");
  static_assert(kQgKS == 32, "four 16-byte pieces per row");
  __shared__ __attribute__((aligned(16))) uint16_t As[2][2][kQgBN * kQgRS];   // [buf][limb]
  __shared__ __attribute__((aligned(16))) uint16_t Bs[2][kQgBM * kQgRS];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int vh = wave & 1, rq = wave >> 1;
  // block b runs on XCD b % 8 (workgroups are dealt round-robin); XCD x takes the key tiles
  // kt = x (mod 8), each with all NR row tiles of S, so that every limb tile is fetched by
  // one XCD and each XCD's L2 holds the 8 limb tiles and NR row tiles in use
  constexpr int NR = D / kQgBM;
  const int b = blockIdx.x, jx = b >> 3;
  const int64_t kt = (int64_t)(jx / NR) * 8 + (b & 7);
  if (kt * kQgBN >= a.nv) return;            // padding of the grid to whole groups of 8
  const int64_t v0 = kt * kQgBN;
  const int r0 = (jx % NR) * kQgBM;
  // global -> LDS pieces: A (limb, vector, 16-byte piece) and B (row, piece)
  const uint16_t* asrc[kQgNI];
  const uint16_t* bsrc[kQgNI];
  int adst[kQgNI], bdst[kQgNI];
#pragma unroll
  for (int i = 0; i < kQgNI; ++i) {
    const int it = tid + 512 * i;
    const int limb = it / (kQgBN * kQgNQ), vv = (it / kQgNQ) % kQgBN, q = it % kQgNQ;
    int64_t v = v0 + vv;
    v = v < a.nv ? v : a.nv - 1;            // past the batch: a real row, never stored
    asrc[i] = (limb ? a.rl : a.rh) + v * D + 8 * q;
    adst[i] = limb * kQgBN * kQgRS + vv * kQgRS + 8 * (q ^ ((vv >> 1) & 3));
    const int rr = it / kQgNQ;
    bsrc[i] = a.S + (size_t)(r0 + rr) * D + 8 * q;
    bdst[i] = rr * kQgRS + 8 * (q ^ ((rr >> 1) & 3));
  }
  uint4 ra[kQgNI], rb[kQgNI];
#define TQ_QG_LOAD(k0)                                                     \
  _Pragma("unroll") for (int i = 0; i < kQgNI; ++i) {                      \
    ra[i] = *reinterpret_cast<const uint4*>(asrc[i] + (k0));               \
    rb[i] = *reinterpret_cast<const uint4*>(bsrc[i] + (k0));               \
  }
#define TQ_QG_STORE(buf)                                                   \
  _Pragma("unroll") for (int i = 0; i < kQgNI; ++i) {                      \
    *reinterpret_cast<uint4*>(&As[buf][0][0] + adst[i]) = ra[i];           \
    *reinterpret_cast<uint4*>(&Bs[buf][0] + bdst[i]) = rb[i];              \
  }
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = (f32x4){0.f, 0.f, 0.f, 0.f};
  TQ_QG_LOAD(0)
  TQ_QG_STORE(0)
  __syncthreads();
  constexpr int NK = D / kQgKS;
  for (int ks = 0; ks < NK; ++ks) {
    const int buf = ks & 1;
    if (ks + 1 < NK) { TQ_QG_LOAD(kQgKS * (ks + 1)) }   // next step's tiles, in flight
    {
      bf16x8 bo[4];
#pragma unroll
      for (int rt = 0; rt < 4; ++rt)
        bo[rt] = *reinterpret_cast<const bf16x8*>(
            &Bs[buf][(64 * rq + 16 * rt + col) * kQgRS + 8 * (grp ^ ((col >> 1) & 3))]);
#pragma unroll
      for (int vt = 0; vt < 4; ++vt) {
        const int arow = (64 * vh + 16 * vt + col) * kQgRS + 8 * (grp ^ ((col >> 1) & 3));
        const bf16x8 ah = *reinterpret_cast<const bf16x8*>(&As[buf][0][arow]);
        const bf16x8 al = *reinterpret_cast<const bf16x8*>(&As[buf][1][arow]);
#pragma unroll
        for (int rt = 0; rt < 4; ++rt) {
          acc[vt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bo[rt], acc[vt][rt], 0, 0, 0);
          acc[vt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bo[rt], acc[vt][rt], 0, 0, 0);
        }
      }
    }
    if (ks + 1 < NK) { TQ_QG_STORE(buf ^ 1) }        // buf ^ 1 was last read before the
    __syncthreads();                                   // previous barrier
  }
#undef TQ_QG_LOAD
#undef TQ_QG_STORE
  // acc[vt][rt][e] at lane l: P[vector 16 vt + 4 (l / 16) + e][row 16 rt + l % 16]
#pragma unroll
  for (int vt = 0; vt < 4; ++vt)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint64_t b0[4], b1[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        b0[e] = __ballot(acc[vt][2 * h][e] >= 0.f);
        b1[e] = __ballot(acc[vt][2 * h + 1][e] >= 0.f);
      }
      if (lane < 16) {
        const int q = lane >> 2, e = lane & 3;
        const uint64_t x0 = e == 0 ? b0[0] : e == 1 ? b0[1] : e == 2 ? b0[2] : b0[3];
        const uint64_t x1 = e == 0 ? b1[0] : e == 1 ? b1[1] : e == 2 ? b1[2] : b1[3];
        const uint32_t word = ((uint32_t)(x0 >> (16 * q)) & 0xFFFFu) |
                              (((uint32_t)(x1 >> (16 * q)) & 0xFFFFu) << 16);
        const int64_t v = v0 + 64 * vh + 16 * vt + lane;
        const int g = (r0 + 64 * rq + 32 * h) / 32;
        if (v < a.nv)
          reinterpret_cast<uint32_t*>(a.codes + v * a.rec_bytes + a.rec_off)[g * (a.R + 1) + a.R] = word;
      }
    }
}

// ---------------------------------------------------------------------------- MFMA encode
// For D <= 128 the rotation is applied as one dense, exact product on bf16 MFMA instead of
// three Walsh-Hadamard rounds on the vector ALU (which, at 3 D log2 D additions per vector,
// would bound the kernel well above the memory time):
//     z_raw = K x,   K = H S3 H S2 H S1 = D^(3/2) Pi   (integers, |K| <= D^2 <= 2^14)
// K is stored as two bf16 limbs that add up to it exactly; a bf16 input is its own exact
// bf16 limb (an fp32 input is split exactly into three), and every product is exact in the
// fp32 accumulator.  z = z_raw / ||z_raw|| (||z_raw|| = D^(3/2) ||x||).  The comparisons
// run on z_raw against thresholds scaled by ||z_raw||, and the residual stays in the
// accumulator registers, which are already laid out as the k values the QJL product needs
// (its matrix columns are permuted to match on the host).
//
// Lane layout (16x16x32 bf16: A[row][k] and B[k][col] at lane row/col + 16 (k / 8)):
// rotation tile = K rows (output coordinates) x x^T (16 vectors as columns).  The host
// permutes K's rows so that lane l then holds vector l % 16 and coordinates
// G D/4 + 4 jt + e (G = l / 16, tile jt, e < 4): a lane group holds D/4 consecutive
// coordinates, i.e. one whole code word at D = 128 (two or four lane groups share a word at
// D = 64 or 32 and are combined with lane-group swaps).  The QJL rows are permuted alike.


// 8 consecutive input elements of one row (zero beyond d), as XL exact bf16 limbs packed
// two per word: limbs[l][w] holds elements 2w, 2w+1 of limb l.  `row` must be a valid row
// (callers clamp: a column of the tile past the last row repeats a real vector and is never
// stored; columns of the products are independent).
// VEC: rows are 16-byte aligned, d = D and no channel gather, so every lane's 8 elements
// are one vector load; otherwise element-wise.
// For XL > 1 (fp32 input) the squares of the 8 values are added to ss.
// Not VEC: chl (LDS) holds the input channel of each coordinate, -1 past d.
template <int XL, bool VEC>
__device__ __forceinline__ void load_x8(const EncodeArgs& a, int64_t row, int c0,
                                        uint32_t (&limbs)[XL][4], float& ss, const int* chl) {
  float v[8];
  if (VEC) {
    if constexpr (XL == 1) {       // bf16 input: its own exact limb
      const uint4 u = *reinterpret_cast<const uint4*>(
          reinterpret_cast<const uint16_t*>(a.x) + row * a.ldx + c0);
      limbs[0][0] = u.x; limbs[0][1] = u.y; limbs[0][2] = u.z; limbs[0][3] = u.w;
      return;
    } else {
      const float4* p = reinterpret_cast<const float4*>(
          reinterpret_cast<const float*>(a.x) + row * a.ldx + c0);
      const float4 u0 = p[0], u1 = p[1];
      v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w;
      v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
    }
  } else {
    const int4 c4a = reinterpret_cast<const int4*>(chl + c0)[0];
    const int4 c4b = reinterpret_cast<const int4*>(chl + c0)[1];
    const int chs[8] = {c4a.x, c4a.y, c4a.z, c4a.w, c4b.x, c4b.y, c4b.z, c4b.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float val = 0.f;
      if (chs[e] >= 0) {
        if constexpr (XL == 1)
          val = bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.x)[row * a.ldx + chs[e]]);
        else
          val = reinterpret_cast<const float*>(a.x)[row * a.ldx + chs[e]];
      }
      v[e] = val;
    }
  }
  if constexpr (XL > 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(v[e], v[e], ss);
  }
  // exact split: truncate to 8 significant bits twice, the remainder fits the third limb
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    float r0 = v[2 * w], r1 = v[2 * w + 1];
#pragma unroll
    for (int l = 0; l < XL; ++l) {
      uint32_t h0, h1;
      if (l + 1 < XL) {
        h0 = __float_as_uint(r0) >> 16;
        h1 = __float_as_uint(r1) >> 16;
        r0 -= __uint_as_float(h0 << 16);
        r1 -= __uint_as_float(h1 << 16);
      } else {
        const uint32_t pk = pack_bf16_rne(r0, r1);
        h0 = pk & 0xFFFFu;
        h1 = pk >> 16;
      }
      limbs[l][w] = h0 | (h1 << 16);
    }
  }
}


// A lane's partial code word holds its D/4 bits at the top of the order fed (bit 0 = its
// first coordinate); place it at its offset in the 32-bit word and merge the lane groups
// that share the word (D = 64: pairs, D = 32: all four).
template <int D>
__device__ __forceinline__ uint32_t combine_word(uint32_t part, int G) {
  if constexpr (D >= 128) {
    return part;
  } else if constexpr (D == 64) {
    const uint32_t v = part << (16 * (G & 1));
    auto a = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return a[0] | a[1];
  } else {
    return or_over_lane_groups(part << (8 * G));
  }
}

// F16 (bf16 input only): the rotation runs as one fp16 product with the exact fp16 K and a
// copy of x scaled per vector by a power of two (2^14 / 2^ceil(log2 ||x||), so every scaled
// element is below 2^14 and the bf16 values convert exactly unless they sit 2^28 below the
// norm), in place of two bf16 products with K split in two limbs.
// MSE: TurboQuant-MSE records (R = b index bits, then the norm): no residual, no QJL stage.
// FOLD (D <= 64, bf16 rows of at most 128 columns, fp16 K): the whole input row is read in
// 16-byte pieces and the channel selection is folded into the rotation table of the vector's
// head (kfold, 4 k steps of 32 columns), the unselected columns masked to zero before the norm
// (xmask); without it a split plan's channels are gathered one element at a time.
template <int D, int R, int XL, bool VEC, bool F16, bool MSE, bool FOLD = false>
__global__ void __launch_bounds__(kEncWaves * kWave) encode_mfma_kernel(EncodeArgs a) {
  encode_group_view(a);
  static_assert(!FOLD || (D <= 64 && XL == 1 && VEC && F16 && !MSE), "folded rows");
  constexpr int NJT = D / 16;        // 16-row tiles of coordinates
  constexpr int NKS = D / 32;        // 32-wide k steps
  constexpr int NKX = FOLD ? 4 : NKS;  // k steps of the rotation over the input row
  constexpr int H = 1 << (R - 1);    // cells of |z|
  constexpr int NT = 2;              // 16-vector tiles per wave iteration
  constexpr uint32_t kPartMask = D >= 128 ? 0xFFFFFFFFu : (1u << (D / 4)) - 1u;
  static_assert(!F16 || XL == 1, "fp16 rotation takes bf16 input");
  constexpr int KLIMBS = F16 ? 1 : 2;
  constexpr int W = MSE ? R : R + 1;  // words per 32-coordinate chunk of a record
  __shared__ uint4 kop[KLIMBS * NJT * NKX * 64];
  __shared__ uint4 sop[MSE ? 1 : NJT * NKS * 64];
  __shared__ uint4 xm[FOLD ? 16 : 1];
  const SubDev& s = a.s;
  if constexpr (FOLD) {
    const int head = (int)(blockIdx.z % a.n_heads);
    table_to_lds<NJT * NKX * 64, kEncWaves * kWave>(
        kop, reinterpret_cast<const uint4*>(s.kfold) + (size_t)head * NJT * NKX * 64);
    if (threadIdx.x < 16) xm[threadIdx.x] = reinterpret_cast<const uint4*>(s.xmask)[head * 16 + threadIdx.x];
  } else {
    table_to_lds<KLIMBS * NJT * NKX * 64, kEncWaves * kWave>(
        kop, reinterpret_cast<const uint4*>(F16 ? s.rotk16 : s.rotk));
  }
  if constexpr (!MSE)
    table_to_lds<NJT * NKS * 64, kEncWaves * kWave>(sop, reinterpret_cast<const uint4*>(s.sperm));
  __shared__ __attribute__((aligned(16))) int chl[VEC ? 8 : D];   // input channel per coordinate
  if constexpr (!VEC) {
    for (int i = threadIdx.x; i < D; i += kEncWaves * kWave)
      chl[i] = i < s.d ? (s.chan ? s.chan[i] : i) : -1;
  }
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, G = lane >> 4;
  // positive half of the symmetric codebook
  float tpos[H > 1 ? H - 1 : 1], apos[H];
#pragma unroll
  for (int j = 0; j < H - 1; ++j) tpos[j] = s.thr[H + j];
#pragma unroll
  for (int j = 0; j < H; ++j) apos[j] = s.lev[H + j];
  const float kscale = 1.f / s.inv_scale;   // D^(3/2)
  const uint32_t sel_lo = neg_one_low_half();

  for (int64_t v0 = ((int64_t)blockIdx.x * kEncWaves + wave) * 16 * NT; v0 < a.n;
       v0 += (int64_t)gridDim.x * kEncWaves * 16 * NT) {
    // ---- x^T operands (columns past the last vector repeat the last one) ----
    uint32_t xw[NT][NKX][XL][4];
    float ss[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      ss[t] = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKX; ++ks) {
        uint32_t lb[XL][4];
        const int64_t row = v0 + 16 * t + col;
        if constexpr (FOLD) {
          // columns past the row carry zero weight; the head's unselected ones are masked
          lb[0][0] = lb[0][1] = lb[0][2] = lb[0][3] = 0u;
          if (32 * ks + 8 * G < s.x_cols)
            load_x8<1, true>(a, row < a.n ? row : a.n - 1, 32 * ks + 8 * G, lb, ss[t], chl);
          const uint4 m = xm[ks * 4 + G];
          lb[0][0] &= m.x; lb[0][1] &= m.y; lb[0][2] &= m.z; lb[0][3] &= m.w;
        } else {
          load_x8<XL, VEC>(a, row < a.n ? row : a.n - 1, 32 * ks + 8 * G, lb, ss[t], chl);
        }
#pragma unroll
        for (int l = 0; l < XL; ++l)
#pragma unroll
          for (int w = 0; w < 4; ++w) xw[t][ks][l][w] = lb[l][w];
      }
    }
    // ---- norms first (so the bucketize can follow the rotation row tile by row tile):
    // bf16 input: diagonal of the Gram matrix x^T x on MFMA; fp32 input: the squares ----
    float nrm[NT], sc[NT], xs[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float xx;
      if constexpr (XL == 1) {
        f32x4 gram = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKX; ++ks) {
          const bf16x8 xb = bf16x8_from_words(xw[t][ks][0][0], xw[t][ks][0][1], xw[t][ks][0][2],
                                              xw[t][ks][0][3]);
          gram = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xb, xb, gram, 0, 0, 0);
        }
        // entry (c, c) sits in lane 16 (c / 4) + c, element c % 4
        xx = __shfl(gram[col & 3], 16 * (col >> 2) + col, 64);
      } else {
        xx = sum_over_lane_groups(ss[t]);
      }
      nrm[t] = __builtin_amdgcn_sqrtf(xx);       // hardware square root (about 1 ulp)
      float zn = nrm[t] * kscale;                // ||z_raw|| = D^(3/2) ||x||
      if constexpr (F16) {
        // x is rotated as x * 2^(14 - e) with ||x|| < 2^e, so z_raw carries the same factor
        const int e = __builtin_amdgcn_frexp_expf(nrm[t]);
        xs[t] = __builtin_amdgcn_ldexpf(1.f, 14 - (e < -100 ? -100 : e));
      }
      sc[t] = zn > 0.f ? zn : 1.f;
    }
    uint32_t xh[F16 ? NT : 1][NKX][4];   // fp16 copy of x (F16 only)
    if constexpr (F16) {
      // Unscaled when every norm of the wave lies in [2^-4, 2^14): elements then stay below
      // the fp16 maximum, and the subnormal rounding (< 2^-24) is below 2^-20 ||x||.
      bool plain = true;
#pragma unroll
      for (int t = 0; t < NT; ++t) plain = plain && nrm[t] >= 0.0625f && nrm[t] < 16384.f;
      if (__all(plain)) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
#pragma unroll
          for (int ks = 0; ks < NKX; ++ks)
#pragma unroll
            for (int w = 0; w < 4; ++w) xh[t][ks][w] = bf16x2_to_f16x2<false>(xw[t][ks][0][w], 1.f);
      } else {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int ks = 0; ks < NKX; ++ks)
#pragma unroll
            for (int w = 0; w < 4; ++w) xh[t][ks][w] = bf16x2_to_f16x2<true>(xw[t][ks][0][w], xs[t]);
          sc[t] *= xs[t];              // z_raw carries the factor (zero vectors: harmless)
        }
      }
    }
    // the positive half of the codebook scaled by ||z_raw||
    float Ts[NT][H > 1 ? H - 1 : 1], As[NT][H];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
      for (int j = 0; j < H - 1; ++j) Ts[t][j] = tpos[j] * sc[t];
#pragma unroll
      for (int j = 0; j < H; ++j) As[t][j] = apos[j] * sc[t];
    }
    // ---- z_raw = K x one 16-row tile at a time, highest first; the tile rotated in the
    // previous step is bucketized meanwhile (independent work for the vector ALUs while the
    // matrix cores run).  This lane's D/4 coordinates sit at bits 4 jt + e of its part of a
    // code word; fed from the highest, each word shifts left by one per coordinate. ----
    f32x4 acc[NT][NJT];
    uint32_t P[NT], J[NT][R > 1 ? R - 1 : 1];
    float g2[NT];
    bf16x8 rhi[NT][NKS], rlo[NT][NKS];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      P[t] = 0;
      g2[t] = 0.f;
#pragma unroll
      for (int m = 0; m < R - 1; ++m) J[t][m] = 0;
    }
#pragma unroll
    for (int step = 0; step <= NJT; ++step) {
      const int jr = NJT - 1 - step;      // row tile rotated in this step
      const int jb = jr + 1;              // row tile bucketized in this step
      if (jr >= 0) {
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[t][jr] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKX; ++ks) {
          if constexpr (F16) {
            const uint4 uk = kop[(jr * NKX + ks) * 64 + lane];
            const f16x8 kh = f16x8_from_words(uk.x, uk.y, uk.z, uk.w);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              const f16x8 xb = f16x8_from_words(xh[t][ks][0], xh[t][ks][1], xh[t][ks][2], xh[t][ks][3]);
              acc[t][jr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kh, xb, acc[t][jr], 0, 0, 0);
            }
            continue;
          }
          const uint4 uh = kop[(jr * NKX + ks) * 64 + lane];
          const uint4 ul = kop[((NJT + jr) * NKX + ks) * 64 + lane];
          const bf16x8 khi = bf16x8_from_words(uh.x, uh.y, uh.z, uh.w);
          const bf16x8 klo = bf16x8_from_words(ul.x, ul.y, ul.z, ul.w);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
#pragma unroll
            for (int l = 0; l < XL; ++l) {
              const bf16x8 xb = bf16x8_from_words(xw[t][ks][l][0], xw[t][ks][l][1],
                                                  xw[t][ks][l][2], xw[t][ks][l][3]);
              acc[t][jr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(khi, xb, acc[t][jr], 0, 0, 0);
              if (l < 2)   // the low limbs' product is below fp32 resolution
                acc[t][jr] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(klo, xb, acc[t][jr], 0, 0, 0);
            }
          }
        }
      }
      if (jb < NJT) {
#pragma unroll
        for (int t = 0; t < NT; ++t) {
#pragma unroll
          for (int e = 3; e >= 0; --e) {
            const float r = bucket_sym<R>(acc[t][jb][e], Ts[t], As[t], P[t], J[t]);
            if constexpr (!MSE) {
              g2[t] = fmaf(r, r, g2[t]);
              acc[t][jb][e] = r;
            }
          }
          if (!MSE && jb % 2 == 0) {
            // residual limbs of k step ks: element e' = tile 2 ks + e'/4, element e' % 4
            const int ks = jb / 2;
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const int e0 = 2 * w, e1 = 2 * w + 1;
              const float r0 = acc[t][2 * ks + (e0 >> 2)][e0 & 3];
              const float r1 = acc[t][2 * ks + (e1 >> 2)][e1 & 3];
              const uint32_t hp = pack2_bf16(r0, r1);
              hw[w] = hp;
              lw[w] = pack2_bf16(residual_below_bf16(hp, sel_lo, r0),
                                 residual_below_bf16(hp, 0xBF800000u, r1));
            }
            rhi[t][ks] = bf16x8_from_words(hw[0], hw[1], hw[2], hw[3]);
            rlo[t][ks] = bf16x8_from_words(lw[0], lw[1], lw[2], lw[3]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t words[NT][R + 1];          // this lane group's code word of each plane
    float gam[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      words[t][R - 1] = combine_word<D>(~P[t] & kPartMask, G);
#pragma unroll
      for (int m = 0; m < R - 1; ++m) words[t][m] = combine_word<D>((J[t][m] ^ P[t]) & kPartMask, G);
      if constexpr (!MSE)
        gam[t] = __builtin_amdgcn_sqrtf(sum_over_lane_groups(g2[t])) * __builtin_amdgcn_rcpf(sc[t]);
    }
    // ---- QJL: P^T = S_perm R^T and its signs, four row tiles at a time, highest first ----
    uint32_t B[NT];                     // sign bits of the projections (set = negative)
#pragma unroll
    for (int t = 0; t < NT; ++t) B[t] = 0;
#pragma unroll
    for (int jq = NJT - 4 < 0 ? 0 : NJT - 4; jq >= 0 && !MSE; jq -= 4) {
      constexpr int NQ = NJT < 4 ? NJT : 4;
      f32x4 qa[NT][NQ];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int h = 0; h < NQ; ++h) qa[t][h] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
        for (int h = 0; h < NQ; ++h) {
          const uint4 us = sop[((jq + h) * NKS + ks) * 64 + lane];
          const bf16x8 sa = bf16x8_from_words(us.x, us.y, us.z, us.w);
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            qa[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa, rhi[t][ks], qa[t][h], 0, 0, 0);
            qa[t][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa, rlo[t][ks], qa[t][h], 0, 0, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int h = NQ - 1; h >= 0; --h)
#pragma unroll
          for (int e = 3; e >= 0; --e) B[t] = shift_in_sign(B[t], qa[t][h][e]);
    }
    if constexpr (!MSE) {
#pragma unroll
      for (int t = 0; t < NT; ++t) words[t][R] = combine_word<D>(~B[t] & kPartMask, G);
    }
    // ---- store: lane group G writes code word G of its vector, group 0 the norms ----
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t row = v0 + 16 * t + col;
      uint32_t* rec = row < a.n ? reinterpret_cast<uint32_t*>(encode_record(a, row)) : nullptr;
      if (rec != nullptr) {
        if ((G * (D / 4)) % 32 == 0) {          // first lane group of its code word
          const int g = G * D / 128;
#pragma unroll
          for (int m = 0; m < W; ++m) rec[g * W + m] = words[t][m];
        }
        if (G == 0) {
          rec[(D / 32) * W] = __float_as_uint(nrm[t]);
          if constexpr (!MSE) rec[(D / 32) * W + 1] = __float_as_uint(gam[t]);
        }
      }
    }
  }
}

// Standalone QJL stage: residuals already rotated, fp32 [n][D] -> sign words [n][D/32].
template <int D>
__global__ void __launch_bounds__(kBlock) qjl_kernel(SubDev s, const float* r, int64_t n,
                                                     uint32_t* beta) {
  using C = EncCfg<D>;
  constexpr int V = C::V, RS = C::RSTRIDE;
  __shared__ __attribute__((aligned(16))) uint16_t rhi[V * RS];
  __shared__ __attribute__((aligned(16))) uint16_t rlo[V * RS];
  __shared__ uint32_t words[V * (D / 32)];
  const int64_t tile0 = (int64_t)blockIdx.x * V;
  for (int i = threadIdx.x; i < V * D; i += kBlock) {
    const int vv = i / D, c = i % D;
    const float x = (tile0 + vv < n) ? r[(tile0 + vv) * D + c] : 0.f;
    const uint32_t h = f32_to_bf16_rne(x);
    rhi[vv * RS + c] = (uint16_t)h;
    rlo[vv * RS + c] = (uint16_t)f32_to_bf16_rne(x - bf16_bits_to_f32(h));
  }
  __syncthreads();
  qjl_signs_mfma<D, V>(s, rhi, rlo, words, D / 32, 1, 0);
  __syncthreads();
  for (int i = threadIdx.x; i < V * (D / 32); i += kBlock) {
    const int vv = i / (D / 32);
    if (tile0 + vv < n) beta[tile0 * (D / 32) + i] = words[i];
  }
}

// ============================================================================ dequantize
// xhat = n * (Pi^T c[idx])[:d]: the centroids of a record's cells taken back through the
// rotation and scaled by its norm (technical overview §4.1.2: dequantize in one batch before
// the attention step; Pi is orthogonal, so its inverse is Pi^T = S1 Ht S2 Ht S3 Ht).  For an
// inner-product record this is the reconstruction of its (b-1)-bit first stage.  Lanes hold
// EPT consecutive rotated coordinates of a vector as in the encoder; the waves of a block
// walk the vectors in a grid-stride loop whose trip count is the same for every lane of a
// wave (the transform exchanges values between lanes).
struct DequantArgs {
  SubDev s;
  const uint8_t* codes;
  int rec_bytes;        // bytes per vector record, all sub-plans
  int64_t n;
  void* out;
  int64_t ldo;          // output row stride, elements
  int out_bf16;
  int vec_store;        // 16-byte aligned rows, identity channels: vector stores
};

template <int D, int R>
__global__ void __launch_bounds__(kBlock) dequant_kernel(DequantArgs a) {
  using C = EncCfg<D>;
  constexpr int EPT = C::EPT, TPV = C::TPV, VPP = C::VPP;
  constexpr int VPB = (kBlock / kWave) * VPP;         // vectors per block and pass
  const SubDev& s = a.s;
  const int W = s.mse ? R : R + 1;                    // words per 32-coordinate chunk
  __shared__ float lev[1 << R];
  if (threadIdx.x < (1 << R)) lev[threadIdx.x] = s.lev[threadIdx.x];
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = lane % TPV, c0 = t * EPT;
  uint32_t sw[3];
#pragma unroll
  for (int r = 0; r < 3; ++r) sw[r] = s.signs[r * (D / 32) + c0 / 32] >> (c0 % 32);
  for (int64_t base = (int64_t)blockIdx.x * VPB + wave * VPP; base < a.n;
       base += (int64_t)gridDim.x * VPB) {
    const int64_t row = base + lane / TPV;
    const bool live = row < a.n;
    const uint32_t* rec = reinterpret_cast<const uint32_t*>(
        a.codes + (live ? row : a.n - 1) * a.rec_bytes + s.rec_off);
    uint32_t pw[R];
#pragma unroll
    for (int m = 0; m < R; ++m) pw[m] = rec[(c0 / 32) * W + m] >> (c0 % 32);
    const float nrm = __uint_as_float(rec[(D / 32) * W]);
    float v[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
      int idx = 0;
#pragma unroll
      for (int m = 0; m < R; ++m) idx |= (int)((pw[m] >> e) & 1u) << m;
      v[e] = lev[idx];
    }
#pragma unroll
    for (int r = 2; r >= 0; --r) {
      fwht_lanes<EPT, TPV>(v, t);
#pragma unroll
      for (int e = 0; e < EPT; ++e) v[e] = flip_sign(v[e], (sw[r] >> e) & 1u);
    }
    const float sc = nrm * s.inv_scale;
#pragma unroll
    for (int e = 0; e < EPT; ++e) v[e] *= sc;
    if (!live) continue;
    if (a.vec_store && c0 + EPT <= s.d) {
      if (a.out_bf16) {
        uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + row * a.ldo + c0);
#pragma unroll
        for (int q = 0; q < EPT / 8; ++q) {
          uint32_t w[4];
#pragma unroll
          for (int h = 0; h < 4; ++h)
            w[h] = pack_bf16_rne(v[8 * q + 2 * h], v[8 * q + 2 * h + 1]);
          o[q] = make_uint4(w[0], w[1], w[2], w[3]);
        }
      } else {
        float4* o = reinterpret_cast<float4*>(static_cast<float*>(a.out) + row * a.ldo + c0);
#pragma unroll
        for (int q = 0; q < EPT / 4; ++q)
          o[q] = make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      }
    } else {
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int i = c0 + e;
        if (i >= s.d) continue;
        const int64_t at = row * a.ldo + (s.chan ? s.chan[i] : i);
        if (a.out_bf16)
          static_cast<uint16_t*>(a.out)[at] = (uint16_t)pack_bf16_rne(v[e], 0.f);
        else
          static_cast<float*>(a.out)[at] = v[e];
      }
    }
  }
}

// D <= 128 with the exact fp16 K: the inverse transform on the matrix cores,
// Pi^T c = D^(-3/2) K^T c, with c (the centroids of a vector's cells, scaled by 2^10) in two
// fp16 limbs, hi = fp16(c) and lo = fp16(c - hi): K^T c_hi + K^T c_lo accumulated in fp32
// (the fp16 products are exact; the sums round like an fp32 transform).  A lane's B operand
// covers 8 rotated coordinates of one vector; both limbs of a pair of coordinates come from
// one 8-byte entry of an LDS table indexed by the pair's 2R index bits.  Every B operand of
// the iteration is built before the first product.  Output rows are permuted so that lane
// group G holds input coordinates 32 q + 8 G + (0..7), q = 0 .. D/32 - 1, of its column's
// vector (tile jt = 2 q + i/4, element i%4): each store covers 32 adjacent coordinates.
constexpr float kDequantLevelScale = 1024.f;   // keeps the low limbs of the levels normal

constexpr int kDqWaves = 4;     // waves per workgroup of the matrix-core reconstruction

template <int D, int R>
__global__ void __launch_bounds__(kDqWaves * kWave) dequant_mfma_kernel(DequantArgs a) {
  constexpr int NJT = D / 16, NKS = D / 32, NT = 2;
  constexpr int NPAIR = 1 << (2 * R);
  __shared__ uint4 kt[NJT * NKS * 64];
  __shared__ uint2 pair_tab[NPAIR];
  const SubDev& s = a.s;
  table_to_lds<NJT * NKS * 64, kDqWaves * kWave>(kt, reinterpret_cast<const uint4*>(s.rotkt16));
  // entry i: coordinate A has index bits i_0, i_2, i_4, ..., coordinate B i_1, i_3, ...
  for (int i = threadIdx.x; i < NPAIR; i += kDqWaves * kWave) {
    int ia = 0, ib = 0;
#pragma unroll
    for (int m = 0; m < R; ++m) {
      ia |= ((i >> (2 * m)) & 1) << m;
      ib |= ((i >> (2 * m + 1)) & 1) << m;
    }
    const float ca = s.lev[ia] * kDequantLevelScale, cb = s.lev[ib] * kDequantLevelScale;
    typedef __attribute__((ext_vector_type(2))) __fp16 f16x2;
    const f16x2 hv = __builtin_amdgcn_cvt_pkrtz(ca, cb);
    const uint32_t hi = __builtin_bit_cast(uint32_t, hv);
    const uint32_t lo = __builtin_bit_cast(
        uint32_t, __builtin_amdgcn_cvt_pkrtz(ca - (float)hv[0], cb - (float)hv[1]));
    pair_tab[i] = make_uint2(hi, lo);
  }
  __syncthreads();
  const int W = s.mse ? R : R + 1;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, G = lane >> 4;
  const float osc = s.inv_scale / kDequantLevelScale;
  const int64_t step = (int64_t)gridDim.x * kDqWaves * 16 * NT;
  // this iteration's record words (index planes, norm), loaded one iteration ahead
  uint32_t rw[NT][NKS][R], rn[NT];
  auto load_records = [&](int64_t v0, uint32_t (&pw)[NT][NKS][R], uint32_t (&pn)[NT]) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t row = v0 + 16 * t + col;
      const int64_t rr = row < a.n ? row : a.n - 1;
      const uint32_t* rec = reinterpret_cast<const uint32_t*>(a.codes + rr * a.rec_bytes + s.rec_off);
      pn[t] = rec[NKS * W];
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int m = 0; m < R; ++m) pw[t][ks][m] = rec[ks * W + m];
    }
  };
  int64_t v0 = ((int64_t)blockIdx.x * kDqWaves + wave) * 16 * NT;
  if (v0 < a.n) load_records(v0, rw, rn);
  for (; v0 < a.n; v0 += step) {
    uint32_t cw[NT][NKS][R];
    float nrm[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      nrm[t] = __uint_as_float(rn[t]);
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
        for (int m = 0; m < R; ++m) cw[t][ks][m] = rw[t][ks][m] >> (8 * G);  // coordinate 8 G + e at bit e
    }
    // the next iteration's records, in flight during this one
    if (v0 + step < a.n) load_records(v0 + step, rw, rn);
    // ---- K^T c, both limbs into one accumulator, k step by k step ----
    f32x4 acc[NT][NJT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) acc[t][jt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      f16x8 bh[NT], bl[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          uint32_t pi = 0;
#pragma unroll
          for (int m = 0; m < R; ++m) pi |= ((cw[t][ks][m] >> (2 * w)) & 3u) << (2 * m);
          const uint2 e = pair_tab[pi];
          hw[w] = e.x;
          lw[w] = e.y;
        }
        bh[t] = f16x8_from_words(hw[0], hw[1], hw[2], hw[3]);
        bl[t] = f16x8_from_words(lw[0], lw[1], lw[2], lw[3]);
      }
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        const uint4 ua = kt[(jt * NKS + ks) * 64 + lane];
        const f16x8 A = f16x8_from_words(ua.x, ua.y, ua.z, ua.w);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          acc[t][jt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bh[t], acc[t][jt], 0, 0, 0);
          acc[t][jt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, bl[t], acc[t][jt], 0, 0, 0);
        }
      }
    }
    // ---- scale and store: lane group G writes coordinates 32 q + 8 G .. + 7 ----
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t row = v0 + 16 * t + col;
      if (row >= a.n) continue;
      const float sc = nrm[t] * osc;
#pragma unroll
      for (int q = 0; q < NKS; ++q) {
        float v[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = acc[t][2 * q + i / 4][i % 4] * sc;
        const int c0 = 32 * q + 8 * G;
        if (a.vec_store && c0 + 8 <= s.d) {
          if (a.out_bf16) {
            uint4* o = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out) + row * a.ldo + c0);
            *o = make_uint4(pack_bf16_rne(v[0], v[1]), pack_bf16_rne(v[2], v[3]),
                            pack_bf16_rne(v[4], v[5]), pack_bf16_rne(v[6], v[7]));
          } else {
            float4* o = reinterpret_cast<float4*>(static_cast<float*>(a.out) + row * a.ldo + c0);
            o[0] = make_float4(v[0], v[1], v[2], v[3]);
            o[1] = make_float4(v[4], v[5], v[6], v[7]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int i = c0 + e;
            if (i >= s.d) continue;
            const int64_t at = row * a.ldo + (s.chan ? s.chan[i] : i);
            if (a.out_bf16)
              static_cast<uint16_t*>(a.out)[at] = (uint16_t)pack_bf16_rne(v[e], 0.f);
            else
              static_cast<float*>(a.out)[at] = v[e];
          }
        }
      }
    }
  }
}

// ============================================================================ queries
// y' = Pi pad(y) (same rotation as the keys: technical overview §4.2.2; the query is kept in
// full precision: deep dive §3), w = S y', and the sums used by the estimate.

struct QPrepArgs {
  SubDev s;
  const void* q;
  int64_t ldq;
  int is_bf16;
  float* yrot;    // [nq][D]
  float* w;       // [nq][D]
  float* sums;    // [nq][2]: sum y', sum w
};

__global__ void __launch_bounds__(kBlock) qprep_kernel(QPrepArgs a) {
  const SubDev& s = a.s;
  const int D = s.D;
  const int64_t qi = blockIdx.x;
  __shared__ float y[kMaxD];
  __shared__ float red[2][kBlock / kWave];
  for (int i = threadIdx.x; i < D; i += kBlock) {
    float val = 0.f;
    if (i < s.d) {
      const int64_t ch = s.chan ? s.chan[i] : i;
      val = a.is_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qi * a.ldq + ch])
                      : reinterpret_cast<const float*>(a.q)[qi * a.ldq + ch];
    }
    y[i] = val;
  }
  __syncthreads();
  for (int r = 0; r < 3; ++r) {
    for (int i = threadIdx.x; i < D; i += kBlock)
      y[i] = flip_sign(y[i], (s.signs[r * (D / 32) + i / 32] >> (i % 32)) & 1u);
    __syncthreads();
    for (int h = 1; h < D; h <<= 1) {
      for (int p = threadIdx.x; p < D / 2; p += kBlock) {
        const int i = (p / h) * 2 * h + (p % h);
        const float u = y[i], v = y[i + h];
        y[i] = u + v;
        y[i + h] = u - v;
      }
      __syncthreads();
    }
  }
  float sy = 0.f;
  for (int i = threadIdx.x; i < D; i += kBlock) {
    const float v = y[i] * s.inv_scale;
    y[i] = v;
    a.yrot[qi * D + i] = v;
    sy += v;
  }
  for (int m = 32; m >= 1; m >>= 1) sy += __shfl_xor(sy, m);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) red[0][wave] = sy;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t0 = 0.f;
    for (int i = 0; i < kBlock / kWave; ++i) t0 += red[0][i];
    a.sums[qi * 2] = t0;
  }
}

// w = S y' on the matrix cores (32x32x16 bf16).  S is exact in bf16 and y' is split into
// three bf16 limbs (together y' to within 2^-24 of its value), so every product is exact
// and the fp32 accumulation gives w to fp32 rounding.  A workgroup takes 64 queries and
// kProjCols rows of S; each wave 32 queries and 64 rows (two output tiles sharing one limb
// split of y').  The workgroup writes its share of each query's sum of w to
// part[query][blockIdx.y], and qsum_kernel adds the shares in order, so that the sums do not
// depend on scheduling.
constexpr int kProjCols = 128;
constexpr int kProjRows = 64;
typedef __attribute__((ext_vector_type(16))) float f32x16;

__global__ void __launch_bounds__(kBlock) qproj_mfma_kernel(QPrepArgs a, int64_t nq, float* part) {
  const SubDev& s = a.s;
  const int D = s.D, K = s.k;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 31, h = lane >> 5;
  const int wq = wave & 1, wj = wave >> 1;
  const int64_t q0 = (int64_t)blockIdx.x * kProjRows + 32 * wq;
  const int jw = blockIdx.y * kProjCols + 64 * wj;
  __shared__ float wsum[kBlock / kWave][32];
  f32x16 acc[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
  const bool ok0 = jw + c < K, ok1 = jw + 32 + c < K;
  if (jw < K) {
    // A: query q0 + c (the last query past the end); B: rows jw + c and jw + 32 + c of S
    // (the last row past K)
    const float* yr = a.yrot + (q0 + c < nq ? q0 + c : nq - 1) * D + 8 * h;
    const uint16_t* S0 = s.S + (size_t)(ok0 ? jw + c : K - 1) * D + 8 * h;
    const uint16_t* S1 = s.S + (size_t)(ok1 ? jw + 32 + c : K - 1) * D + 8 * h;
    for (int i0 = 0; i0 < D; i0 += 16) {
      const float4 ya = *reinterpret_cast<const float4*>(yr + i0);
      const float4 yb = *reinterpret_cast<const float4*>(yr + i0 + 4);
      const uint4 s0 = *reinterpret_cast<const uint4*>(S0 + i0);
      const uint4 s1 = *reinterpret_cast<const uint4*>(S1 + i0);
      const float v[8] = {ya.x, ya.y, ya.z, ya.w, yb.x, yb.y, yb.z, yb.w};
      uint32_t hw[4], mw[4], lw[4];
#pragma unroll
      for (int pr = 0; pr < 4; ++pr) {
        const float x0 = v[2 * pr], x1 = v[2 * pr + 1];
        const uint32_t hp = pack_bf16_rne(x0, x1);
        const float r0 = x0 - __uint_as_float(hp << 16), r1 = x1 - __uint_as_float(hp & 0xFFFF0000u);
        const uint32_t mp = pack_bf16_rne(r0, r1);
        const float t0 = r0 - __uint_as_float(mp << 16), t1 = r1 - __uint_as_float(mp & 0xFFFF0000u);
        hw[pr] = hp;
        mw[pr] = mp;
        lw[pr] = pack_bf16_rne(t0, t1);
      }
      const bf16x8 ah = bf16x8_from_words(hw[0], hw[1], hw[2], hw[3]);
      const bf16x8 am = bf16x8_from_words(mw[0], mw[1], mw[2], mw[3]);
      const bf16x8 al = bf16x8_from_words(lw[0], lw[1], lw[2], lw[3]);
      const bf16x8 b0 = bf16x8_from_words(s0.x, s0.y, s0.z, s0.w);
      const bf16x8 b1 = bf16x8_from_words(s1.x, s1.y, s1.z, s1.w);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b0, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ah, b1, acc[1], 0, 0, 0);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, b0, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(am, b1, acc[1], 0, 0, 0);
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b0, acc[0], 0, 0, 0);
      acc[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(al, b1, acc[1], 0, 0, 0);
    }
  }
  // element i of tile t in this lane: query q0 + 8 (i / 4) + 4 h + i % 4, output jw + 32 t + c
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t q = q0 + 8 * (i / 4) + 4 * h + i % 4;
    if (q < nq) {
      if (ok0) a.w[q * D + jw + c] = acc[0][i];
      if (ok1) a.w[q * D + jw + 32 + c] = acc[1][i];
    }
    float t = (ok0 ? acc[0][i] : 0.f) + (ok1 ? acc[1][i] : 0.f);
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) t += __shfl_xor(t, m);
    if (c == 0) wsum[wave][8 * (i / 4) + 4 * h + i % 4] = t;
  }
  __syncthreads();
  // query r of the workgroup: waves (r / 32) and (r / 32) + 2 hold its two column halves
  if (threadIdx.x < kProjRows) {
    const int r = threadIdx.x;
    const int64_t q = (int64_t)blockIdx.x * kProjRows + r;
    if (q < nq) part[q * gridDim.y + blockIdx.y] = wsum[r / 32][r % 32] + wsum[r / 32 + 2][r % 32];
  }
}

// sum of w per query: the workgroups' shares in order
__global__ void __launch_bounds__(kBlock) qsum_kernel(float* sums, const float* part, int64_t nq,
                                                      int nparts) {
  const int64_t q = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (q >= nq) return;
  float t = 0.f;
  for (int b = 0; b < nparts; ++b) t += part[q * nparts + b];
  sums[q * 2 + 1] = t;
}

// ------------------------------------------------------------ bit-sliced scorer, D > 128
// The same binary-plane form for long vectors and many queries per group (retrieval): the
// 128-coordinate chunks of a key are MFMA steps of one accumulation, and a 16-row image
// tile holds eight queries in two fp8 limbs each (row 2 q + limb), which keeps every
// coordinate to about 2^-10 of its value (the score tolerance is 1e-3 ||q|| ||x||).
constexpr int kWideQT = 8;        // queries per image tile
constexpr int kWideKT = 8;        // 16-key tiles per wave (128 keys per block)

struct WideImgArgs {
  SubDev s;
  const float* yrot;     // [nq][D]
  const float* w;        // [nq][D]
  const float* sums;     // [nq][2]
  int64_t nq_per_group;
  int n_qtiles;          // tiles of kWideQT queries per group
  uint32_t* img;         // [groups*qtiles][D/128][n_planes+1][64][8]
  float* ec;             // [groups*qtiles][kWideQT][4]
};

// One workgroup per image tile: per-query maxima, power-of-two scales, both limbs of every
// plane image of every chunk, the epilogue constants.
__global__ void __launch_bounds__(kBlock) qimage_wide_kernel(WideImgArgs a) {
  const SubDev& s = a.s;
  const int D = s.D, np = s.n_planes, nch = D / 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t gt = blockIdx.x;
  const int64_t grp = gt / a.n_qtiles, qt = gt % a.n_qtiles;
  __shared__ float mx[kWideQT][2][kBlock / kWave];
  __shared__ float scl[kWideQT][2];
  int valid = (int)(a.nq_per_group - qt * kWideQT);
  valid = valid > kWideQT ? kWideQT : valid;
  for (int q = 0; q < kWideQT; ++q) {
    float my = 0.f, mw = 0.f;
    if (q < valid) {
      const int64_t qi = grp * a.nq_per_group + qt * kWideQT + q;
      for (int i = tid; i < D; i += kBlock) {
        my = fmaxf(my, fabsf(a.yrot[qi * D + i]));
        mw = fmaxf(mw, fabsf(a.w[qi * D + i]));
      }
    }
    for (int m = 32; m >= 1; m >>= 1) {
      my = fmaxf(my, __shfl_xor(my, m));
      mw = fmaxf(mw, __shfl_xor(mw, m));
    }
    if (lane == 0) {
      mx[q][0][wave] = my;
      mx[q][1][wave] = mw;
    }
  }
  __syncthreads();
  if (tid < kWideQT) {
    float my = 0.f, mw = 0.f;
    for (int w = 0; w < kBlock / kWave; ++w) {
      my = fmaxf(my, mx[tid][0][w]);
      mw = fmaxf(mw, mx[tid][1][w]);
    }
    float cmax = 0.f;
    for (int p = 0; p < np; ++p) cmax = fmaxf(cmax, fabsf(s.coef[p]));
    const float M1 = my * cmax;
    // powers of two putting the largest image magnitude in (128, 256]
    const float sc_mse = M1 > 0.f ? ldexpf(1.f, 8 - (int)ceilf(log2f(M1))) : 1.f;
    const float sc_qjl = mw > 0.f ? ldexpf(1.f, 8 - (int)ceilf(log2f(mw))) : 1.f;
    scl[tid][0] = sc_mse;
    scl[tid][1] = sc_qjl;
    float* e = a.ec + ((size_t)gt * kWideQT + tid) * 4;
    if (tid < valid) {
      const int64_t qi = grp * a.nq_per_group + qt * kWideQT + tid;
      const float K = sqrtf(0.5f * (float)M_PI) / (float)s.k;
      e[0] = -s.coef_sum * a.sums[qi * 2];
      e[1] = 4.f / sc_mse;
      e[2] = -K * a.sums[qi * 2 + 1];
      e[3] = 4.f * K / sc_qjl;
    } else {
      e[0] = e[1] = e[2] = e[3] = 0.f;
    }
  }
  __syncthreads();
  // image dword (chunk, plane, lane, word): row = lane % 16 = 2 q + limb, lane group G
  const int total = nch * (np + 1) * 64 * 8;
  for (int it = tid; it < total; it += kBlock) {
    const int wd = it & 7, ln = (it >> 3) & 63, cp = it >> 9;
    const int p = cp % (np + 1), c = cp / (np + 1);
    const int row = ln & 15, Ga = ln >> 4, q = row >> 1, limb = row & 1;
    uint32_t word = 0;
    if (q < valid) {
      const int64_t qi = grp * a.nq_per_group + qt * kWideQT + q;
      const float cf = p < np ? s.coef[p] * scl[q][0] : scl[q][1];
      const float* src = (p < np ? a.yrot : a.w) + qi * D + 128 * c;
      float rem[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int e = 4 * wd + b;
        const int K = e < 16 ? 16 * Ga + e : 64 + 16 * Ga + (e - 16);
        rem[b] = cf * src[bitslice_coord(K)];
      }
      // limb l = fp8 e4m3 (round to nearest even) of what limbs 0..l-1 left over
      for (int l = 0; l <= limb; ++l) {
        word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(rem[0], rem[1], 0, false);
        word = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(rem[2], rem[3], (int)word, true);
        rem[0] -= __builtin_amdgcn_cvt_f32_fp8((int)word, 0);
        rem[1] -= __builtin_amdgcn_cvt_f32_fp8((int)word, 1);
        rem[2] -= __builtin_amdgcn_cvt_f32_fp8((int)word, 2);
        rem[3] -= __builtin_amdgcn_cvt_f32_fp8((int)word, 3);
      }
    }
    a.img[(size_t)gt * total + it] = word;
  }
}

// One estimate from the MFMA sums of one (query, key) pair and the query's epilogue constants
// e = (-c_sum * sum y', 4 / image scale, -K * sum w, 4 K / image scale): the same expression
// for the score matrix and for the fused top-k, so both see identical values.
__device__ __forceinline__ float wide_estimate(const float (&e)[4], float sm, float sq, float nrm,
                                               float gam) {
  return nrm * fmaf(gam, fmaf(e[3], sq, e[2]), fmaf(e[1], sm, e[0]));
}

// Fused top-k on the wide scorer (the quantized first stage of two-stage retrieval, technical
// overview §4.2.2, without materializing the score matrix).  Each wave keeps, per query of
// its image tile, a list in LDS of the scores that beat the query's running k-th best; a key
// block appends at most 128 entries per query, and a list that could overflow is cut back to
// its best k (order (-value, index)), which also raises the query's threshold.  The keys a
// wave visits arrive in increasing index order, so a later score equal to the threshold
// loses to every kept entry and a strict comparison drops nothing that could be selected.
struct WideTopk {
  int k;
  int64_t n_slices;      // = gridDim.y: per query, n_slices lists of k candidates
  float* cv;             // [rows][n_slices][k]
  int* ci;               // [rows][n_slices][k]
};

constexpr int kListCap = 2 * kWideKT * 16;            // k kept (k <= 128) + one key block
constexpr int kListPer = kListCap / kWave;            // entries per lane while cutting
static_assert(kListCap - kWideKT * 16 >= 64, "a cut list plus one key block must fit");

__device__ __forceinline__ bool better(float v, int i, float w, int j) {
  return v > w || (v == w && i < j);
}

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                         __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Unsigned key with the order of the float values (both zeros map to the key of +0, since
// they compare equal); no NaN.
__device__ __forceinline__ uint32_t order_key(float v) {
  const uint32_t b = v == 0.f ? 0u : __float_as_uint(v);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t t) {
  return __uint_as_float((t & 0x80000000u) ? (t & 0x7FFFFFFFu) : ~t);
}

// Cut one query's list of cnt > k entries down to its best k (unordered, at the front of the
// list).  Called by a whole wave.  The k-th best value T is found bit by bit on the order
// keys, counting entries with ballots; entries above T stay, and of those equal to T the
// ones with the smallest indices (a second bit-by-bit search when there are more than
// needed).  Returns T, the query's new threshold.
__device__ float wide_list_cut(float* lv, int* li, int cnt, int k, int lane) {
  // entries written by other lanes of this wave must be visible to this lane's loads
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  float v[kListPer];
  int id[kListPer];
  uint32_t key[kListPer];
#pragma unroll
  for (int s = 0; s < kListPer; ++s) {
    const int j = lane + kWave * s;
    const bool ok = j < cnt;
    v[s] = ok ? lv[j] : 0.f;
    id[s] = ok ? li[j] : 0x7FFFFFFF;
    key[s] = ok ? order_key(v[s]) : 0u;        // below every real key
  }
  uint32_t T = 0;                              // largest key with >= k entries at or above it
  for (int b = 31; b >= 0; --b) {
    const uint32_t c = T | (1u << b);
    int n = 0;
#pragma unroll
    for (int s = 0; s < kListPer; ++s) n += __popcll(__ballot(key[s] >= c));
    if (n >= k) T = c;
  }
  int above = 0, equal = 0;
#pragma unroll
  for (int s = 0; s < kListPer; ++s) {
    above += __popcll(__ballot(key[s] > T));
    equal += __popcll(__ballot(key[s] == T));
  }
  const int need = k - above;                  // 1 <= need <= equal
  uint32_t X = 0x7FFFFFFFu;                    // equal entries with index <= X stay
  if (equal > need) {
    X = 0;                                     // largest X with fewer than `need` below it
    for (int b = 30; b >= 0; --b) {
      const uint32_t c = X | (1u << b);
      int n = 0;
#pragma unroll
      for (int s = 0; s < kListPer; ++s) n += __popcll(__ballot(key[s] == T && (uint32_t)id[s] < c));
      if (n < need) X = c;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  int base = 0;
#pragma unroll
  for (int s = 0; s < kListPer; ++s) {
    const bool keep = key[s] > T || (key[s] == T && (uint32_t)id[s] <= X);
    const uint64_t m = __ballot(keep);
    if (keep) {
      const int pos = base + lanes_below(m);
      lv[pos] = v[s];
      li[pos] = id[s];
    }
    base += __popcll(m);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  return key_value(T);
}

// grid.x = (group, block of 4 image tiles), fastest, so that the blocks reading the same keys
// run together and share them through the caches; grid.y strides over 128-key blocks.  Each
// wave owns one image tile (8 queries) and 8 key tiles, whose accumulators stay in registers
// across the chunks; per chunk it loads the plane images once for its 8 key tiles.
// TOPK = false writes the score matrix; TOPK = true keeps the best k per query instead.
template <int R, bool TOPK>
__global__ void __launch_bounds__(kBlock) score_wide_kernel(ScoreArgs a, int64_t n_qblocks,
                                                            WideTopk tk) {
  constexpr int NP = 1 << (R - 1);
  const SubDev& s = a.p.sub[0];
  const int nch = s.D / 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int G = lane >> 4, col = lane & 15;
  const int64_t grp = blockIdx.x / n_qblocks;
  const int64_t qt = (blockIdx.x % n_qblocks) * (kBlock / kWave) + wave;
  if (qt >= a.n_qtiles) return;
  const int64_t gt = grp * a.n_qtiles + qt;
  const int64_t nkb = (a.n + kWideKT * 16 - 1) / (kWideKT * 16);
  const uint8_t* codes = a.codes + grp * a.n * (int64_t)a.p.rec_bytes;
  // epilogue constants of this lane's two queries (rows 4 G .. 4 G + 3 = queries 2 G, 2 G + 1)
  float ea[4], eb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ea[i] = a.ec[0][((size_t)gt * kWideQT + 2 * G) * 4 + i];
    eb[i] = a.ec[0][((size_t)gt * kWideQT + 2 * G + 1) * 4 + i];
  }
  const int64_t qa = qt * kWideQT + 2 * G;
  const bool qa_ok = qa < a.nq_per_group, qb_ok = qa + 1 < a.nq_per_group;
  float* out_a = a.scores + (grp * a.nq_per_group + qa) * a.n;
  float* out_b = out_a + a.n;
  const uint32_t* img = a.img[0] + (size_t)gt * nch * (NP + 1) * 64 * 8 + lane * 8;
  // top-k state: this wave's lists (query q at q * kCap) and, per lane, the count and the
  // threshold of its two queries (equal across the 16 lanes of a lane group)
  constexpr int kCap = kListCap;
  __shared__ float list_v[TOPK ? (kBlock / kWave) * kWideQT * kCap : 1];
  __shared__ int list_i[TOPK ? (kBlock / kWave) * kWideQT * kCap : 1];
  float* lv = list_v + (TOPK ? wave * kWideQT * kCap : 0);
  int* li = list_i + (TOPK ? wave * kWideQT * kCap : 0);
  int cnt_a = 0, cnt_b = 0;
  float thr_a = -INFINITY, thr_b = -INFINITY;
  const uint64_t gmask = 0xFFFFull << (16 * G);
  for (int64_t kb = blockIdx.y; kb < nkb; kb += gridDim.y) {
    const int64_t k0 = kb * kWideKT * 16;
    f32x4 am[kWideKT], aq[kWideKT];
    const uint32_t* rec[kWideKT];                // this lane's key of each tile (clamped: a
#pragma unroll                                    // real key past the end, never stored)
    for (int t = 0; t < kWideKT; ++t) {
      am[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
      aq[t] = (f32x4){0.f, 0.f, 0.f, 0.f};
      int64_t key = k0 + 16 * t + col;
      key = key < a.n ? key : a.n - 1;
      rec[t] = reinterpret_cast<const uint32_t*>(codes + key * a.p.rec_bytes) + G * (R + 1);
    }
    for (int c = 0; c < nch; ++c) {
      i32x8 A[NP + 1];
#pragma unroll
      for (int p = 0; p <= NP; ++p) {
        const uint4* src = reinterpret_cast<const uint4*>(img + ((size_t)c * (NP + 1) + p) * 64 * 8);
        const uint4 u0 = src[0], u1 = src[1];
        A[p][0] = u0.x; A[p][1] = u0.y; A[p][2] = u0.z; A[p][3] = u0.w;
        A[p][4] = u1.x; A[p][5] = u1.y; A[p][6] = u1.z; A[p][7] = u1.w;
      }
      // code chunk 4 c + G of every tile's key: all loads issued before the first use
      uint32_t wd[kWideKT][R + 1];
#pragma unroll
      for (int t = 0; t < kWideKT; ++t)
#pragma unroll
        for (int m = 0; m <= R; ++m) wd[t][m] = rec[t][4 * c * (R + 1) + m];
#pragma unroll
      for (int t = 0; t < kWideKT; ++t) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          uint32_t P = 0;
#pragma unroll
          for (int m = 0; m < R; ++m)
            if ((pmask_c<R>(p) >> m) & 1) P ^= wd[t][m];
          am[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[p], fp4_operand(P), am[t], 0, 4, 0, 127, 0, 127);
        }
        aq[t] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[NP], fp4_operand(wd[t][R]), aq[t], 0, 4, 0, 127, 0, 127);
      }
    }
#pragma unroll
    for (int t = 0; t < kWideKT; ++t) {
      const int64_t key = k0 + 16 * t + col;
      const bool key_ok = key < a.n;
      const int64_t ks = key_ok ? key : a.n - 1;
      const uint32_t* tail = reinterpret_cast<const uint32_t*>(codes + ks * a.p.rec_bytes +
                                                               (s.D / 32) * (R + 1) * 4);
      const float nrm = __uint_as_float(tail[0]), gam = __uint_as_float(tail[1]);
      float est_a = wide_estimate(ea, am[t][0] + am[t][1], aq[t][0] + aq[t][1], nrm, gam);
      float est_b = wide_estimate(eb, am[t][2] + am[t][3], aq[t][2] + aq[t][3], nrm, gam);
      // full-wave region: keep the MFMA results from being sunk into the masked stores
      asm volatile("" : "+v"(est_a), "+v"(est_b));
      if constexpr (!TOPK) {
        if (key_ok && qa_ok) out_a[key] = est_a;
        if (key_ok && qb_ok) out_b[key] = est_b;
      } else {
        const bool pa = key_ok && qa_ok && est_a > thr_a;
        const bool pb = key_ok && qb_ok && est_b > thr_b;
        const uint64_t ma = __ballot(pa), mb = __ballot(pb);
        if ((ma | mb) != 0) {
          if (pa) {
            const int pos = cnt_a + lanes_below(ma & gmask);
            lv[(2 * G) * kCap + pos] = est_a;
            li[(2 * G) * kCap + pos] = (int)key;
          }
          if (pb) {
            const int pos = cnt_b + lanes_below(mb & gmask);
            lv[(2 * G + 1) * kCap + pos] = est_b;
            li[(2 * G + 1) * kCap + pos] = (int)key;
          }
          cnt_a += __popcll(ma & gmask);
          cnt_b += __popcll(mb & gmask);
        }
      }
    }
    if constexpr (TOPK) {
      // cut every list that the next key block could overflow
      const int lim = kCap - kWideKT * 16;
      if (__ballot(cnt_a > lim || cnt_b > lim) != 0) {
#pragma unroll
        for (int q = 0; q < kWideQT; ++q) {
          const int c = __builtin_amdgcn_readlane((q & 1) ? cnt_b : cnt_a, 16 * (q >> 1));
          if (c > lim) {
            const float th = wide_list_cut(lv + q * kCap, li + q * kCap, c, tk.k, lane);
            if ((q >> 1) == G) {
              if (q & 1) { cnt_b = tk.k; thr_b = th; } else { cnt_a = tk.k; thr_a = th; }
            }
          }
        }
      }
    }
  }
  if constexpr (TOPK) {
    // final cut, then this wave's k candidates per query (padding: -inf, index 2^31 - 1)
#pragma unroll
    for (int q = 0; q < kWideQT; ++q) {
      int c = __builtin_amdgcn_readlane((q & 1) ? cnt_b : cnt_a, 16 * (q >> 1));
      if (c > tk.k) {
        wide_list_cut(lv + q * kCap, li + q * kCap, c, tk.k, lane);
        c = tk.k;
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
      const int64_t qi = qt * kWideQT + q;
      if (qi < a.nq_per_group) {
        const size_t o = (((size_t)(grp * a.nq_per_group + qi)) * tk.n_slices + blockIdx.y) * tk.k;
        for (int r = lane; r < tk.k; r += kWave) {
          tk.cv[o + r] = r < c ? lv[q * kCap + r] : -INFINITY;
          tk.ci[o + r] = r < c ? li[q * kCap + r] : 0x7FFFFFFF;
        }
      }
    }
  }
}

// Vector-unit scorer for any D: one key per thread, up to kQT queries of a group per block,
// rotated query and its projection staged in LDS (2 kQT sum(D) floats <= 64 KiB).
template <int kQT>
__global__ void __launch_bounds__(kBlock) score_generic_kernel(ScoreArgs a) {
  extern __shared__ float smem[];   // per sub-plan: y'[QT][D], w[QT][D]
  const int gt = blockIdx.y;
  const int64_t grp = gt / a.n_qtiles, qt = gt % a.n_qtiles;
  const int64_t q0 = qt * kQT;
  const int nq = (int)((a.nq_per_group - q0 < kQT) ? (a.nq_per_group - q0) : kQT);
  int off = 0;
  for (int sb = 0; sb < a.p.nsub; ++sb) {
    const int D = a.p.sub[sb].D;
    for (int i = threadIdx.x; i < kQT * D; i += kBlock) {
      const int qq = i / D, c = i % D;
      const int64_t qi = grp * a.nq_per_group + q0 + qq;
      smem[off + i] = qq < nq ? a.yrot[sb][qi * D + c] : 0.f;
      smem[off + kQT * D + i] = qq < nq ? a.w[sb][qi * D + c] : 0.f;
    }
    off += 2 * kQT * D;
  }
  __syncthreads();
  const int64_t key = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  if (key >= a.n) return;
  const uint8_t* rec0 = a.codes + (grp * a.n + key) * (int64_t)a.p.rec_bytes;
  float est[kQT];
#pragma unroll
  for (int q = 0; q < kQT; ++q) est[q] = 0.f;
  off = 0;
  for (int sb = 0; sb < a.p.nsub; ++sb) {
    const SubDev& s = a.p.sub[sb];
    const int D = s.D, R = s.R;
    const uint32_t* rec = reinterpret_cast<const uint32_t*>(rec0 + s.rec_off);
    const float* ys = smem + off;
    const float* ws = smem + off + kQT * D;
    float am[kQT], aq[kQT];
#pragma unroll
    for (int q = 0; q < kQT; ++q) { am[q] = 0.f; aq[q] = 0.f; }
    for (int g = 0; g < D / 32; ++g) {
      uint32_t wd[kMaxR + 1];
      for (int m = 0; m <= R; ++m) wd[m] = rec[g * (R + 1) + m];
      for (int t = 0; t < 32; ++t) {
        int idx = 0;
        for (int m = 0; m < R; ++m) idx |= ((wd[m] >> t) & 1) << m;
        const float lv = s.lev[idx];
        const float sg = ((wd[R] >> t) & 1) ? 1.f : -1.f;
        const int i = 32 * g + t;
#pragma unroll
        for (int q = 0; q < kQT; ++q) {
          am[q] = fmaf(ys[q * D + i], lv, am[q]);
          aq[q] = fmaf(ws[q * D + i], sg, aq[q]);
        }
      }
    }
    const float nrm = __uint_as_float(rec[(D / 32) * (R + 1)]);
    const float gam = __uint_as_float(rec[(D / 32) * (R + 1) + 1]);
    const float K = sqrtf(0.5f * (float)M_PI) / (float)s.k;
#pragma unroll
    for (int q = 0; q < kQT; ++q) est[q] += nrm * (am[q] + gam * K * aq[q]);
    off += 2 * kQT * D;
  }
  for (int q = 0; q < nq; ++q) a.scores[(grp * a.nq_per_group + q0 + q) * a.n + key] = est[q];
}

// ============================================================================ top-k
// Per row, the k largest (value, index) pairs ordered by (-value, index): the quantized first
// stage of two-stage retrieval (technical overview §4.2.2).  One workgroup streams its row
// and appends every pair that beats the current k-th best to a candidate buffer in LDS.
// Before the buffer could overflow, an exact radix select over 64-bit keys (ordered value
// bits, then the complemented index) finds the k-th best of the buffer, keeps the k best and
// raises the threshold to that pair.  Once the threshold has risen, nearly every element is
// rejected by one comparison and the row streams at the rate its loads allow.
constexpr int kSelRound = kBlock * 16;            // pairs one round of loads brings in
constexpr int kSelCap = kSelRound + 768;          // buffer entries (4 workgroups per CU)
constexpr int kSelKMax = 64;
static_assert(kSelCap - kSelRound >= kSelKMax, "a compacted buffer plus one round must fit");

struct SelShared {
  float v[kSelCap];
  int i[kSelCap];
  alignas(16) int hist[256];
  float kv[kSelKMax];
  int ki[kSelKMax];
  int cnt, nk, digit, above, bin;
  float tv;
  int ti;
};

// Larger key = better pair; -0 ranks as +0, since the two compare equal.
__device__ __forceinline__ uint64_t sel_key(float v, int i) {
  uint32_t b = __float_as_uint(v);
  if ((b & 0x7FFFFFFFu) == 0) b = 0;
  b = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
  return ((uint64_t)b << 32) | (uint32_t)(0x7FFFFFFF - i);
}

// Keep the k best of the cnt buffered pairs at the front of the buffer and return the k-th
// best as the new threshold.  Radix select, 8 bits a pass from the top of the key, until the
// bin that holds the k-th key holds no more keys than are still needed.  Called by the whole
// workgroup with cnt = sh.cnt >= k; ends with a barrier.
__device__ void sel_compact(SelShared& sh, int cnt, int k, float& tv, int& ti) {
  static_assert(kBlock == 256, "one histogram bin per thread");
  const int t = threadIdx.x, lane = t & (kWave - 1);
  uint64_t prefix = 0, mask = 0;
  int need = k;
  for (int shift = 56; shift >= 0; shift -= 8) {
    sh.hist[t] = 0;
    if (t == 0) sh.nk = 0;
    __syncthreads();
    for (int e = t; e < cnt; e += kBlock) {
      const uint64_t key = sel_key(sh.v[e], sh.i[e]);
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(int)(key >> shift) & 255], 1);
    }
    __syncthreads();
    if (t < kWave) {
      // lane l holds bins 4l .. 4l + 3; suf = keys in bins >= 4l
      const int4 h = reinterpret_cast<const int4*>(sh.hist)[lane];
      const int s = h.x + h.y + h.z + h.w;
      int suf = s;
      for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_down(suf, off);
        if (lane + off < kWave) suf += o;
      }
      int run = suf - s;
      if (run < need && need <= suf) {
        const int hb[4] = {h.x, h.y, h.z, h.w};
        for (int b = 3; b >= 0; --b) {
          if (run + hb[b] >= need) {
            sh.digit = 4 * lane + b;
            sh.above = run;
            sh.bin = hb[b];
            break;
          }
          run += hb[b];
        }
      }
    }
    __syncthreads();
    need -= sh.above;
    prefix |= (uint64_t)sh.digit << shift;
    mask |= (uint64_t)0xFF << shift;
    if (sh.bin == need) break;
  }
  // the kept pairs: every key whose top bits exceed the selected prefix, and the whole
  // selected bin (exactly k pairs, the indices being distinct)
  for (int e = t; e < cnt; e += kBlock) {
    const float v = sh.v[e];
    const int i = sh.i[e];
    if ((sel_key(v, i) & mask) >= prefix) {
      const int p = atomicAdd(&sh.nk, 1);
      if (p < kSelKMax) { sh.kv[p] = v; sh.ki[p] = i; }
    }
  }
  __syncthreads();
  if (t < kWave) {
    float v = INFINITY;
    int i = -1;  // ranks above every pair
    if (t < k) {
      v = sh.kv[t];
      i = sh.ki[t];
      sh.v[t] = v;
      sh.i[t] = i;
    }
    for (int m = kWave / 2; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(v, m);
      const int oi = __shfl_xor(i, m);
      if (better(v, i, ov, oi)) { v = ov; i = oi; }
    }
    if (t == 0) { sh.tv = v; sh.ti = i; sh.cnt = k; }
  }
  __syncthreads();
  tv = sh.tv;
  ti = sh.ti;
}

// One round's 16 pairs per thread.  MODE 0: a score row read as float4 (16-byte aligned, n a
// multiple of 4); MODE 1: a score row read as floats; MODE 2: candidate (value, index) lists.
// Pairs past the end get a NaN value, which never beats the threshold.
template <int MODE>
__device__ __forceinline__ void sel_load(const float* x, const int* xi, int64_t n, int64_t base,
                                         float (&v)[16], int (&id)[16]) {
  const int t = threadIdx.x;
  if constexpr (MODE == 0) {
    const float4* x4 = reinterpret_cast<const float4*>(x);
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int64_t j = (base >> 2) + b * kBlock + t;
      const float4 u = 4 * j < n ? x4[j] : make_float4(NAN, NAN, NAN, NAN);
      v[4 * b] = u.x;
      v[4 * b + 1] = u.y;
      v[4 * b + 2] = u.z;
      v[4 * b + 3] = u.w;
#pragma unroll
      for (int c = 0; c < 4; ++c) id[4 * b + c] = (int)(4 * j) + c;
    }
  } else {
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      const int64_t j = base + b * kBlock + t;
      v[b] = j < n ? x[j] : NAN;
      if constexpr (MODE == 2)
        id[b] = j < n ? xi[j] : 0;
      else
        id[b] = (int)j;
    }
  }
}

template <int MODE>
__global__ void __launch_bounds__(kBlock) select_kernel(const float* x, const int* xi, int64_t n,
                                                        int k, int64_t* ids, float* vals) {
  __shared__ SelShared sh;
  const int64_t row = blockIdx.x;
  x += row * n;
  if (MODE == 2) xi += row * n;
  ids += row * k;
  vals += row * k;
  const int t = threadIdx.x, lane = t & (kWave - 1);
  if (t == 0) sh.cnt = 0;
  float tv = -INFINITY;
  int ti = 0x7FFFFFFF;
  float v[16], nv[16];
  int id[16], nid[16];
  sel_load<MODE>(x, xi, n, 0, v, id);
  __syncthreads();
  for (int64_t base = 0; base < n; base += kSelRound) {
    sel_load<MODE>(x, xi, n, base + kSelRound, nv, nid);
    bool pass[16];
    bool any = false;
#pragma unroll
    for (int b = 0; b < 16; ++b) {
      pass[b] = better(v[b], id[b], tv, ti);
      any |= pass[b];
    }
    if (__ballot(any)) {
#pragma unroll
      for (int b = 0; b < 16; ++b) {
        const uint64_t m = __ballot(pass[b]);
        if (m) {
          int at = 0;
          if (lane == 0) at = atomicAdd(&sh.cnt, __popcll(m));
          at = __shfl(at, 0);
          if (pass[b]) {
            const int pos = at + lanes_below(m);
            sh.v[pos] = v[b];
            sh.i[pos] = id[b];
          }
        }
      }
    }
    __syncthreads();
    // every thread reads the count before any appends again (both branches end in a barrier)
    const int c = sh.cnt;
    if (c > kSelCap - kSelRound)
      sel_compact(sh, c, k, tv, ti);
    else
      __syncthreads();
#pragma unroll
    for (int b = 0; b < 16; ++b) { v[b] = nv[b]; id[b] = nid[b]; }
  }
  int cnt = sh.cnt;
  if (cnt > k) {
    sel_compact(sh, cnt, k, tv, ti);
    cnt = k;
  }
  // rank the k kept pairs; a short row (all but fewer than k values NaN) is padded
  if (t < k) {
    float pv = -INFINITY;
    int pi = 0x7FFFFFFF;
    if (t < cnt) { pv = sh.v[t]; pi = sh.i[t]; }
    int r = 0;
    for (int u = 0; u < k; ++u) {
      const float uv = u < cnt ? sh.v[u] : -INFINITY;
      const int ui = u < cnt ? sh.i[u] : 0x7FFFFFFF;
      r += better(uv, ui, pv, pi) || (uv == pv && ui == pi && u < t);
    }
    ids[r] = pi;
    vals[r] = pv;
  }
}

// ============================================================================ attention
// Decode attention over quantized values: for query row r of group g,
//   out[r] = sum_j softmax(scale * logits[r])_j vhat_j,   vhat_j = n_j Pi^T c[idx_j],
// so out[r] = Pi^T (sum_j p_j n_j c[idx_j]): the weighted centroids are summed in the rotated
// domain and the rotation is undone once per row (technical overview §4.1.2 dequantizes the
// cache for the attention step; here that dequantization folds into one transform per row).
// Pass 1, per 1024-token chunk and query row: a reference point m of scale * logit (the
// chunk's max, or up to kAttnSlack below it), the sum of exp(scale * l - m), and the partial
// sums y[r][i] relative to m (fp32).  Pass 2, per row: chunks merged with exp(m_c - M) factors,
// M the largest reference (as in split-token decoding), then Pi^T in LDS, the 1/sum and
// D^(-3/2) scale, and the first d coordinates stored.
//
// Pass 1 is a contraction over tokens on the matrix cores (16x16x32 fp16, fp32 accumulation):
//   y[r][2q + p] = sum_j w[r][j] c(j, 2q + p),   w = exp(scale * l - m) n_j / nsc,
// nsc the largest norm seen in the chunk so far.  Output row m of an MFMA tile is (parity p,
// weight limb, query row); K slots are (token, level limb) pairs whose dwords hold the two
// parities, so a token's B dwords are its pair-table entry (levels of coordinates 2q and
// 2q + 1, high limbs then low limbs) as read, and the A dword of a slot holds the row's weight
// limb in its parity's half.  Weights and levels are each two fp16 limbs (levels scaled by
// 2^10): the four limb products are exact and summed in fp32.  The plane words of a stage of
// tokens are held in LDS token-contiguous ([chunk][plane][token]), so one 16-byte read gives a
// lane its 4 tokens; a lane keeps one 32-coordinate chunk across up to 4 column tiles (pairs
// k = j LPC + col % LPC of chunk col / LPC), reusing each word read.
constexpr int kAttnChunk = 1024;     // tokens per chunk partial
constexpr float kAttnSlack = 8.f;    // a logit may exceed its row's reference max by this

struct AttnArgs {
  SubDev s;
  const float* logits;       // [rows][n]
  int64_t n;
  int64_t nq_per_group;
  float scale;
  const uint8_t* codes;      // group g's records from g * n
  int rec_bytes;
  int64_t n_chunks;
  int64_t chunks_per_block;  // consecutive chunks streamed by one workgroup (or wave)
  int64_t n_groups;
  float* part;               // [chunk][row][D + 2]: y, then max, then sum
  void* out;
  int64_t ldo;
  int out_bf16;
};

// Staging: thread (tt, cm) reads word slot cm of tokens tt, tt + TPI, .. (CMWP = the words per
// token rounded up to a power of two threads per token, TPI = 256 / CMWP tokens per step).
constexpr int attn_pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}
// tokens per stage: the largest power of two <= 512 whose words fit 32 KiB of LDS and take
// at most 16 loads per thread
constexpr int attn_stage_tokens(int wpt) {
  int t = 512;
  while (t > 16 && (wpt * (t + 4) * 4 > 32768 || t * attn_pow2_at_least(wpt) > 16 * kBlock)) t >>= 1;
  return t;
}

// One 16-token block of the contraction, as two MFMAs of 8 tokens per tile.  K slots are
// (token, level limb) pairs, each a dword holding the two parities: the B dwords of a token
// are its pair-table entry (high limbs, low limbs) as read, and the A dword of a (token, level
// limb) slot holds the weight limb of the lane's row in its parity's half (the same for both
// level limbs), so one product sums w (c_hi + c_lo).  Lane group G takes tokens 4G .. 4G + 3 of
// the block, 4G + 2h + {0, 1} in half h.  B fields: per token, the pair fields of ST tiles from
// one shift and mask per plane word, each field the byte offset (or index) of a table entry.
// wl: [limb][row][token] fp16 (row stride wls); sw: [chunk][plane][token] words (row stride
// sws); tok: the block's first token in the staging; tile0: this lane's first column tile.
template <int R, int RQ, int TW, int ST, int LPC, int REP = 1>
__device__ __forceinline__ void attn_contract16(f32x4 (&acc)[RQ][TW], const uint16_t* wl, int wls,
                                                int nrw, const uint32_t* sw, int sws, int tok,
                                                int tile0, int lane, const unsigned char* tab) {
  constexpr int FW = 2 * LPC;
  constexpr int NPAIR = 1 << (2 * R);
  // REP > 1: entry e of copy c at dword e * REP + c, and lane l reads copy l % REP, so that the
  // lanes of a table read fall in distinct banks
  const unsigned char* ltab = tab + (REP > 1 ? (lane % REP) * 4 : 0);
  constexpr int SH = 2 * R + 2 <= FW ? 2 : 0;
  constexpr uint32_t FMASK = (1u << (2 * R + SH)) - 1u;
  uint32_t pm = 0;
#pragma unroll
  for (int j = 0; j < ST; ++j) pm |= 3u << (FW * j);
  const int col = lane & 15, G = lane >> 4;
  const int am = lane & 15, ap = am >> 3, alimb = (am >> 2) & 1, ar = am & 3;
  const uint32_t sel_a = ap ? 0x01000C0Cu : 0x0C0C0100u;
  const uint32_t sel_b = ap ? 0x03020C0Cu : 0x0C0C0302u;
  const int psh = 2 * (col % LPC);
  f16x8 A[2][RQ];
#pragma unroll
  for (int q = 0; q < RQ; ++q) {
    const uint2 x = *reinterpret_cast<const uint2*>(&wl[(alimb * nrw + 4 * q + ar) * wls + tok + 4 * G]);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t xh = h ? x.y : x.x;
      const uint32_t a0 = __builtin_amdgcn_perm(0u, xh, sel_a), a1 = __builtin_amdgcn_perm(0u, xh, sel_b);
      A[h][q] = f16x8_from_words(a0, a0, a1, a1);
    }
  }
#pragma unroll
  for (int st = 0; st < TW / ST; ++st) {
    const int cch = tile0 + st * ST + col / LPC;      // this lane's chunk
    uint4 wd[R];
#pragma unroll
    for (int m = 0; m < R; ++m)
      wd[m] = *reinterpret_cast<const uint4*>(&sw[(cch * R + m) * sws + tok + 4 * G]);
    uint32_t P[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      uint32_t v = 0;
#pragma unroll
      for (int m = 0; m < R; ++m) {
        const uint32_t wv = u == 0 ? wd[m].x : u == 1 ? wd[m].y : u == 2 ? wd[m].z : wd[m].w;
        v |= ((wv >> psh) & pm) << (2 * m + SH);
      }
      P[u] = v;
    }
#pragma unroll
    for (int j = 0; j < ST; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t e[4];
#pragma unroll
        for (int v = 0; v < 2; ++v) {
          const uint32_t pu = P[2 * h + v];
          const uint32_t off = (SH ? (pu >> (FW * j)) & FMASK : ((pu >> (FW * j)) & FMASK) << 2) * REP;
          e[2 * v] = *reinterpret_cast<const uint32_t*>(ltab + off);
          e[2 * v + 1] = *reinterpret_cast<const uint32_t*>(ltab + NPAIR * REP * 4 + off);
        }
        const f16x8 b = f16x8_from_words(e[0], e[1], e[2], e[3]);
#pragma unroll
        for (int q = 0; q < RQ; ++q)
          acc[q][st * ST + j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[h][q], b, acc[q][st * ST + j], 0, 0, 0);
      }
    }
  }
}

// Pair table in LDS: entry i holds coordinate 2q's level (index bits i_0, i_2, ..) in the
// low fp16 half and 2q + 1's (bits i_1, i_3, ..) in the high half; high limbs, then low limbs.
template <int R, int REP = 1>
__device__ __forceinline__ void attn_pair_table(const SubDev& s, uint32_t* ptab) {
  constexpr int NPAIR = 1 << (2 * R);
  __shared__ float slev[1 << R];                  // the levels, read once per workgroup
  if (threadIdx.x < (1 << R)) slev[threadIdx.x] = s.lev[threadIdx.x] * kDequantLevelScale;
  __syncthreads();
  for (int ic = threadIdx.x; ic < NPAIR * REP; ic += blockDim.x) {
    const int i = ic / REP;
    int ia = 0, ib = 0;
#pragma unroll
    for (int m = 0; m < R; ++m) {
      ia |= ((i >> (2 * m)) & 1) << m;
      ib |= ((i >> (2 * m + 1)) & 1) << m;
    }
    const float ca = slev[ia], cb = slev[ib];
    typedef __attribute__((ext_vector_type(2))) __fp16 f16x2;
    const f16x2 hv = __builtin_amdgcn_cvt_pkrtz(ca, cb);
    ptab[ic] = __builtin_bit_cast(uint32_t, hv);
    ptab[NPAIR * REP + ic] =
        __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(ca - (float)hv[0], cb - (float)hv[1]));
  }
}

// D >= 512: the waves of a workgroup split the column tiles, so they share each stage.  A
// workgroup streams the stages of up to chunks_per_block consecutive chunks of one group and
// row tile: the next stage's plane words, norms and logits are loaded while the current stage
// is contracted.  The softmax max and the norm scale are running values over the chunk (as in
// online softmax): when a stage raises them, the accumulators and the partial sums of the
// exponentials are rescaled.  At the end of each chunk its partial (y, max, sum) is written.
template <int D, int R, int RQ>
__global__ void __launch_bounds__(kBlock) attend_mfma_kernel(AttnArgs a) {
  constexpr int NW = kBlock / kWave;
  constexpr int NJT = D / 32;                       // column tiles of 16 pairs = chunks
  constexpr int ST = NJT < 4 ? NJT : 4;             // tiles sharing a lane's chunk
  constexpr int LPC = 16 / ST;                      // columns per chunk within those tiles
  constexpr int TW = NJT < 16 / RQ ? NJT : 16 / RQ; // tiles per wave
  constexpr int NTG = NJT / TW;                     // tile groups
  static_assert(NTG <= NW && TW % ST == 0, "tile split");
  constexpr int TSP = NW / NTG;                     // waves splitting the tokens of a tile group
  constexpr int CMW = NJT * R;                      // plane words per token
  constexpr int WPT = CMW + 1;                      // and the norm
  constexpr int TS = attn_stage_tokens(WPT);
  constexpr int CMWP = attn_pow2_at_least(WPT);
  constexpr int SPT = CMWP > kBlock ? CMWP / kBlock : 1;   // word slots per thread and token
  constexpr int TPI = CMWP > kBlock ? 1 : kBlock / CMWP;   // tokens per staging step
  static_assert(TS % TPI == 0 && kAttnChunk % TS == 0, "stage split");
  constexpr int NLD = TS / TPI * SPT;               // staged words per thread
  constexpr int LPT = TS >= kBlock ? TS / kBlock : 1;   // stage tokens per thread (logits)
  constexpr int SWS = TS + 4;                       // dword stride of a staged word row
  constexpr int WLS = TS + 8;                       // fp16 stride of a weight row
  constexpr int NRW = 4 * RQ;
  constexpr int SW_BYTES = WPT * SWS * 4;
  constexpr int STAGE_BYTES = SW_BYTES + 2 * NRW * WLS * 2;
  constexpr int RED_BYTES = TSP > 1 ? TSP * NRW * D * 4 : 0;
  constexpr int RAW = STAGE_BYTES > RED_BYTES ? STAGE_BYTES : RED_BYTES;
  constexpr int NPAIR = 1 << (2 * R);
  __shared__ __attribute__((aligned(16))) unsigned char raw[RAW];
  __shared__ uint32_t ptab[2 * NPAIR];              // high limbs, then low limbs
  __shared__ float red[2][NW][NRW + 1];             // per stage (two in flight): maxima
  __shared__ float ered[NW][NRW];                   // sums of the exponentials at a flush
  uint32_t* sw = reinterpret_cast<uint32_t*>(raw);
  const float* snrm = reinterpret_cast<const float*>(sw + CMW * SWS);   // row CMW: the norms
  uint16_t* wl = reinterpret_cast<uint16_t*>(raw + SW_BYTES);
  const SubDev& s = a.s;
  const int W = s.mse ? R : R + 1;
  const int rb = a.rec_bytes;
  const int64_t grp = blockIdx.y;
  const int64_t q0 = (int64_t)blockIdx.z * NRW;
  const int nr = (int)((a.nq_per_group - q0) < NRW ? (a.nq_per_group - q0) : NRW);
  const int64_t cb = (int64_t)blockIdx.x * a.chunks_per_block;
  const int64_t ce = (cb + a.chunks_per_block) < a.n_chunks ? cb + a.chunks_per_block : a.n_chunks;
  const int64_t T0 = cb * kAttnChunk;
  const int64_t T1 = (ce * kAttnChunk) < a.n ? ce * kAttnChunk : a.n;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint8_t* gcodes = a.codes + grp * a.n * (int64_t)rb + s.rec_off;
  const float* glg = a.logits + (grp * a.nq_per_group + q0) * a.n;
  // ---- staging roles; full stages load unconditionally (all loads in flight together) ----
  const int stt = CMWP > kBlock ? 0 : tid / CMWP;
  int sslot[SPT];
  uint32_t svoff[SPT];
#pragma unroll
  for (int i = 0; i < SPT; ++i) {
    sslot[i] = CMWP > kBlock ? tid + kBlock * i : tid % CMWP;
    const int scw = sslot[i] < WPT ? sslot[i] : 0;
    const int sword = scw == CMW ? NJT * W : (scw / R) * W + scw % R;
    svoff[i] = (uint32_t)(stt * rb + sword * 4);
  }
  uint32_t pw[NLD];
  float pl[NRW][LPT];
  auto load_stage = [&](int64_t S) {
    const int ns = (T1 - S) < TS ? (int)(T1 - S) : TS;
    const uint8_t* b0 = gcodes + S * rb;
    if (ns == TS) {
#pragma unroll
      for (int k = 0; k < NLD; ++k)
        pw[k] = *reinterpret_cast<const uint32_t*>(b0 + (int64_t)(TPI * (k / SPT)) * rb + svoff[k % SPT]);
    } else {
#pragma unroll
      for (int k = 0; k < NLD; ++k)
        pw[k] = stt + TPI * (k / SPT) < ns
                    ? *reinterpret_cast<const uint32_t*>(b0 + (int64_t)(TPI * (k / SPT)) * rb +
                                                         svoff[k % SPT])
                    : 0u;
    }
    // logits of this thread's stage tokens, indices clamped and values masked arithmetically
#pragma unroll
    for (int k = 0; k < LPT; ++k) {
      const int t = tid + kBlock * k;
      const int tc = t < ns ? t : ns - 1;
#pragma unroll
      for (int r = 0; r < NRW; ++r) {
        const int rc = r < nr ? r : nr - 1;
        pl[r][k] = fminf(a.scale * glg[rc * a.n + S + tc], (t < ns && r < nr) ? INFINITY : -INFINITY);
      }
    }
  };
  load_stage(T0);
  attn_pair_table<R>(s, ptab);
  const int col = lane & 15, G = lane >> 4;
  const int tg = wave / TSP, ts = wave % TSP;
  const unsigned char* tab = reinterpret_cast<const unsigned char*>(ptab);
  float rm[NRW], esum[NRW];                         // running max of scale * logit, partial sums
  float nsc = 0.f;                                  // running max norm
#pragma unroll
  for (int r = 0; r < NRW; ++r) {
    rm[r] = -INFINITY;
    esum[r] = 0.f;
  }
  f32x4 acc[RQ][TW];
#pragma unroll
  for (int q = 0; q < RQ; ++q)
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[q][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  int par = 0;
  for (int64_t S = T0; S < T1; S += TS, par ^= 1) {
    const int ns = (T1 - S) < TS ? (int)(T1 - S) : TS;
    __syncthreads();                      // the previous stage's LDS reads are done
    // ---- words and norms into LDS; this stage's maxima ----
    float nm = 0.f, mx[NRW];
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      const int sl = sslot[k % SPT];
      if (sl < WPT) {
        sw[sl * SWS + stt + TPI * (k / SPT)] = pw[k];
        if (sl == CMW) nm = fmaxf(nm, __uint_as_float(pw[k]));
      }
    }
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
      mx[r] = pl[r][0];
#pragma unroll
      for (int k = 1; k < LPT; ++k) mx[r] = fmaxf(mx[r], pl[r][k]);
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      nm = fmaxf(nm, __shfl_xor(nm, m));
#pragma unroll
      for (int r = 0; r < NRW; ++r) mx[r] = fmaxf(mx[r], __shfl_xor(mx[r], m));
    }
    if (lane == 0) {
#pragma unroll
      for (int r = 0; r < NRW; ++r) red[par][wave][r] = mx[r];
      red[par][wave][NRW] = nm;
    }
    __syncthreads();
    // ---- running maxima; rescale what was accumulated under the old ones ----
    float nn = nsc;
#pragma unroll
    for (int w = 0; w < NW; ++w) nn = fmaxf(nn, red[par][w][NRW]);
    bool changed = nn != nsc;
    float fr[NRW];
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
      float mn = rm[r];
#pragma unroll
      for (int w = 0; w < NW; ++w) mn = fmaxf(mn, red[par][w][r]);
      const float fe = (r < nr && mn != rm[r]) ? __expf(rm[r] - mn) : 1.f;
      changed |= fe != 1.f;
      esum[r] *= fe;
      fr[r] = fe * (nsc > 0.f ? nsc / nn : 1.f);
      rm[r] = mn;
    }
    if (changed) {
#pragma unroll
      for (int q = 0; q < RQ; ++q)
#pragma unroll
        for (int t = 0; t < TW; ++t)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[q][t][i] *= fr[4 * q + i];
    }
    nsc = nn;
    // ---- weights w = exp(scale l - max) n_j / nsc, two fp16 limbs ----
    const float inv = nsc > 0.f ? 1.f / nsc : 0.f;
#pragma unroll
    for (int k = 0; k < LPT; ++k) {
      const int t = tid + kBlock * k;
      if (t < TS) {
        const float nw = snrm[t] * inv;
#pragma unroll
        for (int r = 0; r < NRW; ++r) {
          const float e = r < nr ? __expf(fmaxf(pl[r][k] - rm[r], -INFINITY)) : 0.f;
          esum[r] += e;
          const float w = e * nw;
          typedef __attribute__((ext_vector_type(2))) __fp16 f16x2;
          const f16x2 h = __builtin_amdgcn_cvt_pkrtz(w, 0.f);
          const f16x2 l = __builtin_amdgcn_cvt_pkrtz(w - (float)h[0], 0.f);
          wl[r * WLS + t] = (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xFFFFu);
          wl[(NRW + r) * WLS + t] = (uint16_t)(__builtin_bit_cast(uint32_t, l) & 0xFFFFu);
        }
      }
    }
    if (S + TS < T1) load_stage(S + TS);    // in flight during the contraction
    __syncthreads();
    // ---- the contraction over this stage's tokens ----
    const int nblk = (ns + 15) >> 4;
    for (int b = ts; b < nblk; b += TSP)
      attn_contract16<R, RQ, TW, ST, LPC>(acc, wl, WLS, NRW, sw, SWS, b * 16, tg * TW, lane, tab);
    // ---- end of a chunk: its partial sums (lane groups G = 2p and 2p + 1 hold the high
    // and low weight limbs of parity p), then a fresh start for the next chunk ----
    const int64_t Se = S + ns;
    if (Se == T1 || Se % kAttnChunk == 0) {
      const int64_t chunk = (Se - 1) / kAttnChunk;
#pragma unroll
      for (int r = 0; r < NRW; ++r) {
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) esum[r] += __shfl_xor(esum[r], m);
      }
      if (lane == 0) {
#pragma unroll
        for (int r = 0; r < NRW; ++r) ered[wave][r] = esum[r];
      }
      __syncthreads();                    // the contraction's LDS reads are done
      const float osc = nsc / kDequantLevelScale;
      float* yb = reinterpret_cast<float*>(raw);
      const size_t rows_total = (size_t)a.nq_per_group * gridDim.y;
      const size_t row0 = (size_t)(grp * a.nq_per_group + q0);
      float* pbase = a.part + ((size_t)chunk * rows_total + row0) * (D + 2);
#pragma unroll
      for (int q = 0; q < RQ; ++q)
#pragma unroll
        for (int t = 0; t < TW; ++t) {
          f32x4 v = acc[q][t];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] += __shfl_xor(v[i], 16);
          const int jt = tg * TW + t;
          const int cch = (jt / ST) * ST + col / LPC;
          const int coord = 32 * cch + 2 * ((jt % ST) * LPC + col % LPC) + (G >> 1);
          if ((G & 1) == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int r = 4 * q + i;
              if (TSP > 1)
                yb[(ts * NRW + r) * D + coord] = v[i];
              else if (r < nr)
                pbase[(size_t)r * (D + 2) + coord] = v[i] * osc;
            }
          }
          acc[q][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
      __syncthreads();
      if (TSP > 1) {
        for (int idx = tid; idx < nr * D; idx += kBlock) {
          const int r = idx / D, i = idx - r * D;
          float y = 0.f;
#pragma unroll
          for (int h = 0; h < TSP; ++h) y += yb[(h * NRW + r) * D + i];
          pbase[(size_t)r * (D + 2) + i] = y * osc;
        }
      }
      if (tid < nr) {
        float sum = 0.f, mrow = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += ered[w][tid];
#pragma unroll
        for (int r = 0; r < NRW; ++r)
          if (r == tid) mrow = rm[r];
        pbase[(size_t)tid * (D + 2) + D] = mrow;
        pbase[(size_t)tid * (D + 2) + D + 1] = sum;
      }
#pragma unroll
      for (int r = 0; r < NRW; ++r) {
        rm[r] = -INFINITY;
        esum[r] = 0.f;
      }
      nsc = 0.f;
    }
  }
}

// D <= 256: each wave owns every column tile of its tokens, so waves need not meet.  A wave
// streams its own run of consecutive chunks (one work item: chunks_per_block chunks of one
// group and row tile) through a private LDS region, in stages of up to 64 tokens whose plane
// words, norms and logits load while the previous stage is contracted; maxima are wave
// reductions; each chunk's partial is written by the wave itself.  The only workgroup
// barrier follows the pair table.
template <int D, int R, int RQ>
__global__ void __launch_bounds__(kBlock)
__attribute__((amdgpu_waves_per_eu(RQ == 1 && D <= 128 && R <= 3 ? 4 : 1))) attend_wave_kernel(AttnArgs a, int64_t n_seq, int64_t n_items) {
  constexpr int NW = kBlock / kWave;
  constexpr int NJT = D / 32;
  constexpr int ST = NJT < 4 ? NJT : 4;
  constexpr int LPC = 16 / ST;
  constexpr int TW = NJT;
  static_assert(TW * RQ <= 16 && TW % ST == 0, "tiles per wave");
  constexpr int CMW = NJT * R;
  constexpr int WPT = CMW + 1;                      // plane words and the norm
  constexpr int CMWP = attn_pow2_at_least(WPT);
  static_assert(CMWP <= kWave, "words per token");
  constexpr int TPI = kWave / CMWP;                 // tokens per staging step
  constexpr int TSW = 16 * TPI < 64 ? 16 * TPI : 64;   // tokens per stage (at most 16 loads)
  constexpr int NLD = TSW / TPI;
  constexpr int SWS = TSW + 4;
  constexpr int WLS = TSW + 8;
  constexpr int NRW = 4 * RQ;
  constexpr int WAVE_BYTES = WPT * SWS * 4 + 2 * NRW * WLS * 2;
  constexpr int NPAIR = 1 << (2 * R);
  constexpr int REP = R <= 3 ? 32 : 1;               // table copies (at most 16 KiB)
  constexpr int PTAB_BYTES = 2 * NPAIR * REP * 4;
  // one LDS object: the pair table first (so that table reads take immediate offsets), then
  // the waves' regions
  __shared__ __attribute__((aligned(16))) unsigned char lds[PTAB_BYTES + NW * WAVE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  attn_pair_table<R, REP>(a.s, reinterpret_cast<uint32_t*>(lds));
  __syncthreads();
  const int64_t item = (int64_t)blockIdx.x * NW + wave;
  if (item >= n_items) return;
  unsigned char* raw = lds + PTAB_BYTES;
  uint32_t* sw = reinterpret_cast<uint32_t*>(raw + wave * WAVE_BYTES);
  const float* snrm = reinterpret_cast<const float*>(sw + CMW * SWS);
  uint16_t* wl = reinterpret_cast<uint16_t*>(raw + wave * WAVE_BYTES + WPT * SWS * 4);
  const unsigned char* tab = lds;
  const SubDev& s = a.s;
  const int W = s.mse ? R : R + 1;
  const int rb = a.rec_bytes;
  const int64_t seq = item % n_seq, rest = item / n_seq;
  const int64_t grp = rest % a.n_groups;
  const int64_t q0 = (rest / a.n_groups) * NRW;
  const int nr = (int)((a.nq_per_group - q0) < NRW ? (a.nq_per_group - q0) : NRW);
  const int64_t cb = seq * a.chunks_per_block;
  const int64_t ce = (cb + a.chunks_per_block) < a.n_chunks ? cb + a.chunks_per_block : a.n_chunks;
  const int64_t T0 = cb * kAttnChunk;
  const int64_t T1 = (ce * kAttnChunk) < a.n ? ce * kAttnChunk : a.n;
  const uint8_t* gcodes = a.codes + grp * a.n * (int64_t)rb + s.rec_off;
  const float* glg = a.logits + (grp * a.nq_per_group + q0) * a.n;
  // staging roles: lane (tt, slot); full stages load unconditionally
  const int stt = lane / CMWP, sl = lane % CMWP;
  const int scw = sl < WPT ? sl : 0;
  const int sword = scw == CMW ? NJT * W : (scw / R) * W + scw % R;
  const uint32_t svoff = (uint32_t)(stt * rb + sword * 4);
  uint32_t pw[NLD];
  float pl[NRW];
  auto load_stage = [&](int64_t S) {
    const int ns = (T1 - S) < TSW ? (int)(T1 - S) : TSW;
    const uint8_t* b0 = gcodes + S * rb;
    // (32-bit lane offsets from a uniform base: one load instruction each)
    if (ns == TSW) {
#pragma unroll
      for (int k = 0; k < NLD; ++k)
        pw[k] = *reinterpret_cast<const uint32_t*>(b0 + (uint32_t)(TPI * k * rb + svoff));
    } else {
#pragma unroll
      for (int k = 0; k < NLD; ++k)
        pw[k] = stt + TPI * k < ns
                    ? *reinterpret_cast<const uint32_t*>(b0 + (uint32_t)(TPI * k * rb + svoff))
                    : 0u;
    }
    const uint32_t tc = (uint32_t)(lane < ns ? lane : ns - 1);
#pragma unroll
    for (int r = 0; r < NRW; ++r) {
      const int rc = r < nr ? r : nr - 1;
      const float* lr = glg + rc * a.n + S;
      pl[r] = fminf(a.scale * lr[tc], (lane < ns && r < nr) ? INFINITY : -INFINITY);
    }
  };
  load_stage(T0);
  float rm[NRW], esum[NRW];
  float nsc = 0.f;
#pragma unroll
  for (int r = 0; r < NRW; ++r) {
    rm[r] = -INFINITY;
    esum[r] = 0.f;
  }
  f32x4 acc[RQ][TW];
#pragma unroll
  for (int q = 0; q < RQ; ++q)
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[q][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int64_t S = T0; S < T1; S += TSW) {
    const int ns = (T1 - S) < TSW ? (int)(T1 - S) : TSW;
    // ---- words and norms into this wave's LDS; the stage maxima by wave reductions ----
    __builtin_amdgcn_wave_barrier();      // the previous stage's LDS reads precede these writes
    float nm = 0.f;
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
      if (sl < WPT) {
        sw[sl * SWS + stt + TPI * k] = pw[k];
        if (sl == CMW) nm = fmaxf(nm, __uint_as_float(pw[k]));
      }
    }
    // The reference max of a row and the norm scale move only when a lane exceeds them (a
    // logit by more than kAttnSlack): the weights stay below e^kAttnSlack, well inside fp16,
    // and a stage without a new maximum needs no reduction.  Any reference point is exact:
    // the partial carries it and the combine weighs chunks by exp(reference - max).
    bool need = nm > nsc;
#pragma unroll
    for (int r = 0; r < NRW; ++r) need |= r < nr && pl[r] > rm[r] + kAttnSlack;
    if (__any(need)) {
      float mx[NRW];
#pragma unroll
      for (int r = 0; r < NRW; ++r) mx[r] = pl[r];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) {
        nm = fmaxf(nm, __shfl_xor(nm, m));
#pragma unroll
        for (int r = 0; r < NRW; ++r) mx[r] = fmaxf(mx[r], __shfl_xor(mx[r], m));
      }
      const float nn = fmaxf(nsc, nm);
      bool changed = nn != nsc;
      float fr[NRW];
#pragma unroll
      for (int r = 0; r < NRW; ++r) {
        const float mn = fmaxf(rm[r], mx[r]);
        const float fe = (r < nr && mn != rm[r]) ? __expf(rm[r] - mn) : 1.f;
        changed |= fe != 1.f;
        esum[r] *= fe;
        fr[r] = fe * (nsc > 0.f ? nsc / nn : 1.f);
        rm[r] = mn;
      }
      if (changed) {
#pragma unroll
        for (int q = 0; q < RQ; ++q)
#pragma unroll
          for (int t = 0; t < TW; ++t)
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[q][t][i] *= fr[4 * q + i];
      }
      nsc = nn;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // ---- this lane's token: weights w = exp(scale l - max) n / nsc in two fp16 limbs ----
    if (lane < TSW) {
      const float nw = snrm[lane] * (nsc > 0.f ? 1.f / nsc : 0.f);
#pragma unroll
      for (int r = 0; r < NRW; ++r) {
        const float e = r < nr ? __expf(fmaxf(pl[r] - rm[r], -INFINITY)) : 0.f;
        esum[r] += e;
        const float w = e * nw;
        typedef __attribute__((ext_vector_type(2))) __fp16 f16x2;
        const f16x2 h = __builtin_amdgcn_cvt_pkrtz(w, 0.f);
        const f16x2 l = __builtin_amdgcn_cvt_pkrtz(w - (float)h[0], 0.f);
        wl[r * WLS + lane] = (uint16_t)(__builtin_bit_cast(uint32_t, h) & 0xFFFFu);
        wl[(NRW + r) * WLS + lane] = (uint16_t)(__builtin_bit_cast(uint32_t, l) & 0xFFFFu);
      }
    }
    if (S + TSW < T1) load_stage(S + TSW);  // in flight during the contraction
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int nblk = (ns + 15) >> 4;
    for (int b = 0; b < nblk; ++b)
      attn_contract16<R, RQ, TW, ST, LPC, REP>(acc, wl, WLS, NRW, sw, SWS, b * 16, 0, lane, tab);
    // ---- end of a chunk: the wave writes its partial and starts afresh ----
    const int64_t Se = S + ns;
    if (Se == T1 || Se % kAttnChunk == 0) {
      const int64_t chunk = (Se - 1) / kAttnChunk;
      const float osc = nsc / kDequantLevelScale;
      const size_t rows_total = (size_t)a.nq_per_group * a.n_groups;
      float* pbase = a.part + ((size_t)chunk * rows_total + (size_t)(grp * a.nq_per_group + q0)) * (D + 2);
      const int col = lane & 15, G = lane >> 4;
#pragma unroll
      for (int q = 0; q < RQ; ++q)
#pragma unroll
        for (int t = 0; t < TW; ++t) {
          f32x4 v = acc[q][t];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] += __shfl_xor(v[i], 16);
          const int cch = (t / ST) * ST + col / LPC;
          const int coord = 32 * cch + 2 * ((t % ST) * LPC + col % LPC) + (G >> 1);
          if ((G & 1) == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (4 * q + i < nr) pbase[(size_t)(4 * q + i) * (D + 2) + coord] = v[i] * osc;
          }
          acc[q][t] = (f32x4){0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
      for (int r = 0; r < NRW; ++r) {
        float e = esum[r];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) e += __shfl_xor(e, m);
        if (lane == 0 && r < nr) {
          pbase[(size_t)r * (D + 2) + D] = rm[r];
          pbase[(size_t)r * (D + 2) + D + 1] = e;
        }
        rm[r] = -INFINITY;
        esum[r] = 0.f;
      }
      nsc = 0.f;
    }
  }
}

template <int D>
__global__ void __launch_bounds__(kBlock) attend_combine_kernel(AttnArgs a, int64_t rows) {
  constexpr int NW = kBlock / kWave;
  constexpr int TPC = D < kBlock ? kBlock / D : 1;     // threads per coordinate (chunk subsets)
  __shared__ float y[D];
  __shared__ float sub[TPC > 1 ? TPC : 1][D < kBlock ? D : 1];
  __shared__ float wred[NW];
  __shared__ float scl[2];
  const SubDev& s = a.s;
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nch = a.n_chunks;
  auto at = [&](int64_t c) { return a.part + ((size_t)c * rows + row) * (D + 2); };
  float m = -INFINITY;
#pragma unroll 4
  for (int64_t c = tid; c < nch; c += kBlock) m = fmaxf(m, at(c)[D]);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k));
  if (lane == 0) wred[wave] = m;
  __syncthreads();
  if (tid == 0) {
    float v = wred[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) v = fmaxf(v, wred[w]);
    scl[0] = v;
  }
  __syncthreads();
  const float M = scl[0];
  float sacc = 0.f;
#pragma unroll 4
  for (int64_t c = tid; c < nch; c += kBlock) sacc += at(c)[D + 1] * __expf(at(c)[D] - M);
#pragma unroll
  for (int k = 32; k >= 1; k >>= 1) sacc += __shfl_xor(sacc, k);
  __syncthreads();
  if (lane == 0) wred[wave] = sacc;
  __syncthreads();
  if (tid == 0) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) v += wred[w];
    scl[1] = v;
  }
  if (TPC > 1) {
    const int i = tid % D, h = tid / D;
    float t = 0.f;
#pragma unroll 8
    for (int64_t c = h; c < nch; c += TPC) t = fmaf(at(c)[i], __expf(at(c)[D] - M), t);
    sub[h][i] = t;
    __syncthreads();
    if (tid < D) {
      float v = 0.f;
#pragma unroll
      for (int q = 0; q < TPC; ++q) v += sub[q][tid];
      y[tid] = v;
    }
  } else {
    for (int i = tid; i < D; i += kBlock) {
      float t = 0.f;
#pragma unroll 8
      for (int64_t c = 0; c < nch; ++c) t = fmaf(at(c)[i], __expf(at(c)[D] - M), t);
      y[i] = t;
    }
  }
  __syncthreads();
  // Pi^T: rounds from the last, each a Walsh-Hadamard transform then that round's diagonal
  for (int r = 2; r >= 0; --r) {
    for (int hh = 1; hh < D; hh <<= 1) {
      for (int p = tid; p < D / 2; p += kBlock) {
        const int i = (p / hh) * 2 * hh + (p % hh);
        const float u = y[i], v = y[i + hh];
        y[i] = u + v;
        y[i + hh] = u - v;
      }
      __syncthreads();
    }
    for (int i = tid; i < D; i += kBlock)
      y[i] = flip_sign(y[i], (s.signs[r * (D / 32) + i / 32] >> (i % 32)) & 1u);
    __syncthreads();
  }
  const float sc = s.inv_scale / scl[1];
  for (int i = tid; i < s.d; i += kBlock) {
    const float v = y[i] * sc;
    if (a.out_bf16)
      static_cast<uint16_t*>(a.out)[row * a.ldo + i] = (uint16_t)pack_bf16_rne(v, 0.f);
    else
      static_cast<float*>(a.out)[row * a.ldo + i] = v;
  }
}

template <int D, int RQ>
static void launch_attend_rq(const AttnArgs& aa, int64_t n_groups, hipStream_t st) {
  const int64_t qtiles = (aa.nq_per_group + 4 * RQ - 1) / (4 * RQ);
  // up to 4 chunks per workgroup while at least 2048 workgroups remain
  AttnArgs ab = aa;
  ab.chunks_per_block = 1;
  while (ab.chunks_per_block < 4 && aa.n_chunks * n_groups * qtiles / (2 * ab.chunks_per_block) >= 2048)
    ab.chunks_per_block *= 2;
  const dim3 g1((unsigned)((aa.n_chunks + ab.chunks_per_block - 1) / ab.chunks_per_block),
                (unsigned)n_groups, (unsigned)qtiles);
  switch (aa.s.R) {
    case 1: hipLaunchKernelGGL((attend_mfma_kernel<D, 1, RQ>), g1, dim3(kBlock), 0, st, ab); break;
    case 2: hipLaunchKernelGGL((attend_mfma_kernel<D, 2, RQ>), g1, dim3(kBlock), 0, st, ab); break;
    case 3: hipLaunchKernelGGL((attend_mfma_kernel<D, 3, RQ>), g1, dim3(kBlock), 0, st, ab); break;
    default: hipLaunchKernelGGL((attend_mfma_kernel<D, 4, RQ>), g1, dim3(kBlock), 0, st, ab); break;
  }
}

template <int D, int RQ>
static void launch_attend_wave(const AttnArgs& aa, int64_t n_groups, hipStream_t st) {
  const int64_t qtiles = (aa.nq_per_group + 4 * RQ - 1) / (4 * RQ);
  // up to 4 chunks per wave while at least 8192 waves remain
  AttnArgs ab = aa;
  ab.chunks_per_block = 1;
  while (ab.chunks_per_block < 4 && aa.n_chunks * n_groups * qtiles / (2 * ab.chunks_per_block) >= 8192)
    ab.chunks_per_block *= 2;
  const int64_t n_seq = (aa.n_chunks + ab.chunks_per_block - 1) / ab.chunks_per_block;
  const int64_t items = n_seq * n_groups * qtiles;
  const dim3 g1((unsigned)((items + kBlock / kWave - 1) / (kBlock / kWave)));
  switch (aa.s.R) {
    case 1: hipLaunchKernelGGL((attend_wave_kernel<D, 1, RQ>), g1, dim3(kBlock), 0, st, ab, n_seq, items); break;
    case 2: hipLaunchKernelGGL((attend_wave_kernel<D, 2, RQ>), g1, dim3(kBlock), 0, st, ab, n_seq, items); break;
    case 3: hipLaunchKernelGGL((attend_wave_kernel<D, 3, RQ>), g1, dim3(kBlock), 0, st, ab, n_seq, items); break;
    default: hipLaunchKernelGGL((attend_wave_kernel<D, 4, RQ>), g1, dim3(kBlock), 0, st, ab, n_seq, items); break;
  }
}

template <int D>
static int launch_attend_d(const AttnArgs& aa, int64_t n_groups, hipStream_t st) {
  if (aa.s.R < 1 || aa.s.R > 4) return (int)hipErrorInvalidValue;
  // two row quads per workgroup when there are more than 4 rows (one at D = 2048, where the
  // accumulators of 8 rows would not fit a wave's share of the tiles)
  if constexpr (D <= 256) {
    if (aa.nq_per_group > 4)
      launch_attend_wave<D, 2>(aa, n_groups, st);
    else
      launch_attend_wave<D, 1>(aa, n_groups, st);
  } else {
    if (aa.nq_per_group > 4 && D <= 1024)
      launch_attend_rq<D, D <= 1024 ? 2 : 1>(aa, n_groups, st);
    else
      launch_attend_rq<D, 1>(aa, n_groups, st);
  }
  const int64_t rows = aa.nq_per_group * n_groups;
  hipLaunchKernelGGL(attend_combine_kernel<D>, dim3((unsigned)rows), dim3(kBlock), 0, st, aa, rows);
  return (int)hipGetLastError();
}

// ------------------------------------------------------------ per-stream workspaces
// The score and attention calls need a short-lived workspace (query images, partial
// results).  A stream-ordered allocation per call costs several microseconds of device time
// between launches, so one buffer per (device, stream) is kept and reused by the next call on
// that stream: the stream runs the two calls' kernels one after the other, so the reuse is
// safe.  The buffer grows when a call needs more (a stream-ordered free of the old one, then
// a new allocation) up to kCachedWorkspaceMax; larger requests, and calls on a stream that is
// being captured into a graph, allocate per call as before.  The lock is held from the
// lookup until the lease ends (after the caller has enqueued its kernels), so a growth on
// another host thread cannot free a buffer before its last use is ordered on its stream.
constexpr size_t kCachedWorkspaceMax = (size_t)256 << 20;

struct CachedWorkspace {
  int dev;
  hipStream_t st;
  void* ptr;
  size_t cap;
};
std::mutex g_ws_mu;
std::vector<CachedWorkspace> g_ws;

class WorkspaceLease {
 public:
  WorkspaceLease() = default;
  WorkspaceLease(const WorkspaceLease&) = delete;
  WorkspaceLease& operator=(const WorkspaceLease&) = delete;
  ~WorkspaceLease() {
    if (own_ != nullptr) (void)hipFreeAsync(own_, st_);
  }
  void* ptr() const { return ptr_; }
  // returns 0 or a hipError_t
  int acquire(size_t bytes, hipStream_t st) {
    st_ = st;
    if (bytes == 0) bytes = 256;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    hipError_t e = hipStreamIsCapturing(st, &cs);
    if (e != hipSuccess) return (int)e;
    if (bytes > kCachedWorkspaceMax || cs != hipStreamCaptureStatusNone) {
      e = hipMallocAsync(&own_, bytes, st);
      if (e != hipSuccess) {
        own_ = nullptr;
        return (int)e;
      }
      ptr_ = own_;
      return 0;
    }
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return (int)e;
    lock_ = std::unique_lock<std::mutex>(g_ws_mu);
    CachedWorkspace* w = nullptr;
    for (auto& c : g_ws)
      if (c.dev == dev && c.st == st) w = &c;
    if (w == nullptr) {
      g_ws.push_back({dev, st, nullptr, 0});
      w = &g_ws.back();
    }
    if (w->cap < bytes) {
      if (w->ptr != nullptr) (void)hipFreeAsync(w->ptr, st);
      w->ptr = nullptr;
      w->cap = 0;
      size_t cap = bytes < ((size_t)1 << 20) ? ((size_t)1 << 20) : bytes;
      e = hipMallocAsync(&w->ptr, cap, st);
      if (e != hipSuccess) {
        w->ptr = nullptr;
        return (int)e;
      }
      w->cap = cap;
    }
    ptr_ = w->ptr;
    return 0;
  }

 private:
  std::unique_lock<std::mutex> lock_;
  hipStream_t st_ = nullptr;
  void* own_ = nullptr;
  void* ptr_ = nullptr;
};

int launch_attend(const PlanDev& p, const float* logits, int64_t nq_per_group, int64_t n_groups,
                  int64_t n, float scale, const uint8_t* codes, void* out, int dt, int64_t ldo,
                  void* stream) {
  if (nq_per_group == 0 || n_groups == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  AttnArgs aa;
  aa.s = p.sub[0];
  aa.logits = logits;
  aa.n = n;
  aa.nq_per_group = nq_per_group;
  aa.scale = scale;
  aa.codes = codes;
  aa.rec_bytes = p.rec_bytes;
  aa.n_chunks = (n + kAttnChunk - 1) / kAttnChunk;
  aa.chunks_per_block = 1;
  aa.n_groups = n_groups;
  aa.out = out;
  aa.ldo = ldo;
  aa.out_bf16 = dt == TQ_BF16;
  const size_t bytes = (size_t)aa.n_chunks * nq_per_group * n_groups * (aa.s.D + 2) * 4;
  WorkspaceLease lease;
  const int wrc = lease.acquire(bytes, st);
  if (wrc) return wrc;
  aa.part = static_cast<float*>(lease.ptr());
  int rc;
  switch (aa.s.D) {
    case 32: rc = launch_attend_d<32>(aa, n_groups, st); break;
    case 64: rc = launch_attend_d<64>(aa, n_groups, st); break;
    case 128: rc = launch_attend_d<128>(aa, n_groups, st); break;
    case 256: rc = launch_attend_d<256>(aa, n_groups, st); break;
    case 512: rc = launch_attend_d<512>(aa, n_groups, st); break;
    case 1024: rc = launch_attend_d<1024>(aa, n_groups, st); break;
    case 2048: rc = launch_attend_d<2048>(aa, n_groups, st); break;
    default: rc = (int)hipErrorInvalidValue;
  }
  return rc;
}

// ============================================================================ re-rank
// Second stage of two-stage retrieval (technical overview §4.2.2): exact inner products of
// each query with its candidates' full-precision vectors, and the k best by (-value, id).
// One workgroup per query: the query in LDS as fp32; each wave scores candidates (lanes
// stride over the coordinates, so a wave reads 64 consecutive elements of a row at a time,
// then a wave-wide sum); wave 0 takes k rounds of wave arg-max, dropping every copy of each
// winner, so a candidate listed twice counts once.  Ids outside [0, n) are skipped; slots
// past the valid candidates get id -1 and value -inf.
constexpr int kRerankMaxD = 8192, kRerankMaxC = 256;

struct RerankArgs {
  const void* q;
  int64_t ldq;
  int q_bf16;
  const void* x;
  int64_t ldx;
  int x_bf16;
  int64_t n;
  int d;
  const int64_t* cand;
  int kc;
  int k;
  int64_t* ids;
  float* vals;
};

__device__ __forceinline__ bool better_id64(float v, int64_t i, float w, int64_t j) {
  return v > w || (v == w && i < j);
}

__global__ void __launch_bounds__(kBlock) rerank_kernel(RerankArgs a) {
  __shared__ float qs[kRerankMaxD];
  __shared__ float cv[kRerankMaxC];
  __shared__ int64_t cid[kRerankMaxC];
  const int64_t qi = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int c = threadIdx.x; c < a.d; c += kBlock)
    qs[c] = a.q_bf16 ? bf16_bits_to_f32(static_cast<const uint16_t*>(a.q)[qi * a.ldq + c])
                     : static_cast<const float*>(a.q)[qi * a.ldq + c];
  __syncthreads();
  for (int j = wave; j < a.kc; j += kBlock / kWave) {
    const int64_t id = a.cand[qi * a.kc + j];
    const bool ok = id >= 0 && id < a.n;
    float acc = 0.f;
    if (ok) {
      if (a.x_bf16) {
        const uint16_t* xr = static_cast<const uint16_t*>(a.x) + id * a.ldx;
        for (int c = lane; c < a.d; c += kWave) acc = fmaf(qs[c], bf16_bits_to_f32(xr[c]), acc);
      } else {
        const float* xr = static_cast<const float*>(a.x) + id * a.ldx;
        for (int c = lane; c < a.d; c += kWave) acc = fmaf(qs[c], xr[c], acc);
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) acc += __shfl_xor(acc, m);
    if (lane == 0) {
      cv[j] = ok ? acc : -INFINITY;
      cid[j] = ok ? id : INT64_MAX;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  constexpr int P = kRerankMaxC / kWave;
  float v[P];
  int64_t id[P];
#pragma unroll
  for (int s2 = 0; s2 < P; ++s2) {
    const int j = lane + kWave * s2;
    v[s2] = j < a.kc ? cv[j] : -INFINITY;
    id[s2] = j < a.kc ? cid[j] : INT64_MAX;
  }
  for (int r = 0; r < a.k; ++r) {
    float bv = v[0];
    int64_t bi = id[0];
#pragma unroll
    for (int s2 = 1; s2 < P; ++s2)
      if (better_id64(v[s2], id[s2], bv, bi)) { bv = v[s2]; bi = id[s2]; }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      const float ov = __shfl_xor(bv, m);
      const int64_t oi = (int64_t)(((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)((uint64_t)bi >> 32), m) << 32) |
                                   (uint32_t)__shfl_xor((int)(uint32_t)bi, m));
      if (better_id64(ov, oi, bv, bi)) { bv = ov; bi = oi; }
    }
    const bool valid = bi != INT64_MAX;
    if (lane == 0) {
      a.ids[qi * a.k + r] = valid ? bi : -1;
      a.vals[qi * a.k + r] = valid ? bv : -INFINITY;
    }
    if (valid) {
#pragma unroll
      for (int s2 = 0; s2 < P; ++s2)
        if (id[s2] == bi) { v[s2] = -INFINITY; id[s2] = INT64_MAX; }
    }
  }
}

int launch_rerank(const void* q, int q_bf16, int64_t nq, int64_t ldq, const void* x, int x_bf16,
                  int64_t n, int64_t ldx, int d, const int64_t* cand, int kc, int k, int64_t* ids,
                  float* vals, void* stream) {
  if (nq == 0) return 0;
  RerankArgs ra;
  ra.q = q; ra.ldq = ldq; ra.q_bf16 = q_bf16;
  ra.x = x; ra.ldx = ldx; ra.x_bf16 = x_bf16; ra.n = n; ra.d = d;
  ra.cand = cand; ra.kc = kc; ra.k = k; ra.ids = ids; ra.vals = vals;
  hipLaunchKernelGGL(rerank_kernel, dim3((unsigned)nq), dim3(kBlock), 0, (hipStream_t)stream, ra);
  return (int)hipGetLastError();
}

// ============================================================================ launchers

static inline int hip_rc(hipError_t e) { return e == hipSuccess ? 0 : (int)e; }

template <int D, bool SPLIT, bool MSE = false>
static int launch_encode_kernel(const EncodeArgs& ea, hipStream_t st) {
  const int64_t tiles = (ea.n + EncCfg<D>::V - 1) / EncCfg<D>::V;
  const dim3 grid((unsigned)tiles), block(kBlock);
  switch (ea.s.R) {
    case 1: hipLaunchKernelGGL((encode_kernel<D, 1, SPLIT, MSE>), grid, block, 0, st, ea); break;
    case 2: hipLaunchKernelGGL((encode_kernel<D, 2, SPLIT, MSE>), grid, block, 0, st, ea); break;
    case 3: hipLaunchKernelGGL((encode_kernel<D, 3, SPLIT, MSE>), grid, block, 0, st, ea); break;
    case 4: hipLaunchKernelGGL((encode_kernel<D, 4, SPLIT, MSE>), grid, block, 0, st, ea); break;
    default: return (int)hipErrorInvalidValue;
  }
  return hip_rc(hipGetLastError());
}

// Long vectors: batches of kSplitBatch vectors, each encoded without its signs (residual
// limbs to a stream-ordered temporary of 4 D bytes per vector) and then signed by the GEMM.
constexpr int64_t kSplitBatch = 32768;

template <int D>
static int launch_encode_d(const EncodeArgs& ea, hipStream_t st) {
  if (ea.s.mse) return launch_encode_kernel<D, false, true>(ea, st);   // one pass, no signs
  if constexpr (D >= 1024) {
    const int64_t nb = ea.n < kSplitBatch ? ea.n : kSplitBatch;
    void* ws = nullptr;
    hipError_t e = hipMallocAsync(&ws, (size_t)nb * D * 4, st);
    if (e != hipSuccess) return (int)e;
    const int es = ea.is_bf16 ? 2 : 4;
    int rc = 0;
    for (int64_t b0 = 0; b0 < ea.n && !rc; b0 += kSplitBatch) {
      EncodeArgs eb = ea;
      eb.n = (ea.n - b0) < kSplitBatch ? (ea.n - b0) : kSplitBatch;
      eb.x = static_cast<const uint8_t*>(ea.x) + b0 * ea.ldx * es;
      eb.codes = ea.codes + b0 * ea.rec_bytes;
      eb.rw_hi = static_cast<uint16_t*>(ws);
      eb.rw_lo = eb.rw_hi + (size_t)eb.n * D;
      rc = launch_encode_kernel<D, true>(eb, st);
      if (rc) break;
      QjlGemmArgs ga;
      ga.rh = eb.rw_hi;
      ga.rl = eb.rw_lo;
      ga.S = ea.s.S;
      ga.codes = eb.codes;
      ga.nv = eb.n;
      ga.rec_bytes = ea.rec_bytes;
      ga.rec_off = ea.s.rec_off;
      ga.R = ea.s.R;
      const int64_t nkt = (eb.n + kQgBN - 1) / kQgBN;
      const dim3 grid((unsigned)(8 * (D / kQgBM) * ((nkt + 7) / 8)));
      hipLaunchKernelGGL(qjl_gemm_kernel<D>, grid, dim3(512), 0, st, ga);
      rc = hip_rc(hipGetLastError());
    }
    e = hipFreeAsync(ws, st);
    if (!rc && e != hipSuccess) rc = (int)e;
    return rc;
  } else {
    return launch_encode_kernel<D, false>(ea, st);
  }
}

template <int D, int XL, bool VEC, bool F16, bool MSE>
static void launch_encode_mfma_dxvfm(const EncodeArgs& ea, hipStream_t st, dim3 grid) {
  const dim3 block(kEncWaves * kWave);
  switch (ea.s.R) {
    case 1: hipLaunchKernelGGL((encode_mfma_kernel<D, 1, XL, VEC, F16, MSE>), grid, block, 0, st, ea); break;
    case 2: hipLaunchKernelGGL((encode_mfma_kernel<D, 2, XL, VEC, F16, MSE>), grid, block, 0, st, ea); break;
    case 3: hipLaunchKernelGGL((encode_mfma_kernel<D, 3, XL, VEC, F16, MSE>), grid, block, 0, st, ea); break;
    case 4: hipLaunchKernelGGL((encode_mfma_kernel<D, 4, XL, VEC, F16, MSE>), grid, block, 0, st, ea); break;
  }
}

template <int D, int XL, bool VEC, bool F16>
static void launch_encode_mfma_dxvf(const EncodeArgs& ea, hipStream_t st, dim3 grid) {
  if (ea.s.mse)
    launch_encode_mfma_dxvfm<D, XL, VEC, F16, true>(ea, st, grid);
  else
    launch_encode_mfma_dxvfm<D, XL, VEC, F16, false>(ea, st, grid);
}

template <int D, int XL, bool VEC>
static void launch_encode_mfma_dxv(const EncodeArgs& ea, hipStream_t st, dim3 grid) {
  if constexpr (XL == 1) {
    if (ea.s.rotk16 != nullptr) {
      launch_encode_mfma_dxvf<D, XL, VEC, true>(ea, st, grid);
      return;
    }
  }
  launch_encode_mfma_dxvf<D, XL, VEC, false>(ea, st, grid);
}

template <int D, int XL>
static void launch_encode_mfma_dx(const EncodeArgs& ea, hipStream_t st, dim3 grid) {
  if constexpr (D <= 64 && XL == 1) {
    const bool aligned = ((uintptr_t)ea.x % 16 == 0) && ((ea.ldx * 2) % 16 == 0);
    if (ea.s.chan != nullptr && ea.s.kfold != nullptr && ea.s.rotk16 != nullptr && !ea.s.mse &&
        aligned) {
      const dim3 block(kEncWaves * kWave);
      switch (ea.s.R) {
        case 1: hipLaunchKernelGGL((encode_mfma_kernel<D, 1, 1, true, true, false, true>), grid, block, 0, st, ea); break;
        case 2: hipLaunchKernelGGL((encode_mfma_kernel<D, 2, 1, true, true, false, true>), grid, block, 0, st, ea); break;
        case 3: hipLaunchKernelGGL((encode_mfma_kernel<D, 3, 1, true, true, false, true>), grid, block, 0, st, ea); break;
        case 4: hipLaunchKernelGGL((encode_mfma_kernel<D, 4, 1, true, true, false, true>), grid, block, 0, st, ea); break;
      }
      return;
    }
  }
  if (ea.vec_load && ea.s.d == D)
    launch_encode_mfma_dxv<D, XL, true>(ea, st, grid);
  else
    launch_encode_mfma_dxv<D, XL, false>(ea, st, grid);
}

static int launch_encode_mfma(const EncodeArgs& ea, hipStream_t st, int64_t n_groups) {
  // one wave iteration encodes 32 vectors; two 8-wave blocks per compute unit (what the
  // registers of the common variants allow), each looping over its share of its group's rows,
  // so the operand tables are loaded once per block rather than once per few iterations
  const int64_t iters = (ea.n + 31) / 32;
  int64_t blocks = (iters + kEncWaves - 1) / kEncWaves;
  const int64_t full = 2 * (int64_t)compute_units();
  const int64_t cap = n_groups > 1 ? (full + n_groups - 1) / n_groups : full;
  if (blocks > cap) blocks = cap;
  const dim3 grid((unsigned)blocks, 1, (unsigned)n_groups);
  switch (ea.s.D * 2 + ea.is_bf16) {
    case 32 * 2 + 1: launch_encode_mfma_dx<32, 1>(ea, st, grid); break;
    case 32 * 2: launch_encode_mfma_dx<32, 3>(ea, st, grid); break;
    case 64 * 2 + 1: launch_encode_mfma_dx<64, 1>(ea, st, grid); break;
    case 64 * 2: launch_encode_mfma_dx<64, 3>(ea, st, grid); break;
    case 128 * 2 + 1: launch_encode_mfma_dx<128, 1>(ea, st, grid); break;
    case 128 * 2: launch_encode_mfma_dx<128, 3>(ea, st, grid); break;
    default: return (int)hipErrorInvalidValue;
  }
  return hip_rc(hipGetLastError());
}

// n rows per group, n_groups groups (grid z); with `index`, record i goes to cache row
// index[i] of a cache of `cap` rows instead (D <= 128 encoders only).
static int launch_encode_to(const PlanDev& p, int sub, const void* x, int dt, int64_t n,
                            int64_t ldx, uint8_t* codes, void* stream, int64_t n_groups,
                            const int64_t* index, int64_t cap) {
  if (n == 0 || n_groups == 0) return 0;
  EncodeArgs ea;
  ea.s = p.sub[sub];
  ea.x = x;
  ea.n = n;
  ea.ldx = ldx;
  ea.codes = codes;
  ea.rec_bytes = p.rec_bytes;
  ea.is_bf16 = dt == TQ_BF16;
  const int es = ea.is_bf16 ? 2 : 4;
  ea.vec_load = (ea.s.chan == nullptr) && ((uintptr_t)x % 16 == 0) && ((ldx * es) % 16 == 0);
  ea.rw_hi = ea.rw_lo = nullptr;
  ea.n_heads = p.n_heads > 0 ? p.n_heads : 1;
  ea.out_index = index;
  ea.out_cap = cap;
  hipStream_t st = (hipStream_t)stream;
  if (ea.s.D == 128 && ea.is_bf16 && ea.s.k16_32 && !ea.s.mse) return launch_encode128(ea, st, n_groups);
  if (ea.s.D <= 128 && ea.s.rotk) return launch_encode_mfma(ea, st, n_groups);
  if (n_groups != 1 || index != nullptr) return (int)hipErrorInvalidValue;
  switch (ea.s.D) {
    case 32: return launch_encode_d<32>(ea, st);
    case 64: return launch_encode_d<64>(ea, st);
    case 128: return launch_encode_d<128>(ea, st);
    case 256: return launch_encode_d<256>(ea, st);
    case 512: return launch_encode_d<512>(ea, st);
    case 1024: return launch_encode_d<1024>(ea, st);
    case 2048: return launch_encode_d<2048>(ea, st);
  }
  return (int)hipErrorInvalidValue;
}

int launch_encode(const PlanDev& p, int sub, const void* x, int dt, int64_t n, int64_t ldx,
                  uint8_t* codes, void* stream, int64_t n_groups) {
  return launch_encode_to(p, sub, x, dt, n, ldx, codes, stream, n_groups, nullptr, 0);
}

template <int D>
static int launch_qjl_d(const SubDev& s, const float* r, int64_t n, uint32_t* beta, hipStream_t st) {
  const int64_t tiles = (n + EncCfg<D>::V - 1) / EncCfg<D>::V;
  hipLaunchKernelGGL(qjl_kernel<D>, dim3((unsigned)tiles), dim3(kBlock), 0, st, s, r, n, beta);
  return hip_rc(hipGetLastError());
}

int launch_qjl(const SubDev& s, const float* r, int64_t n, uint32_t* beta, void* stream) {
  if (n == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  switch (s.D) {
    case 32: return launch_qjl_d<32>(s, r, n, beta, st);
    case 64: return launch_qjl_d<64>(s, r, n, beta, st);
    case 128: return launch_qjl_d<128>(s, r, n, beta, st);
    case 256: return launch_qjl_d<256>(s, r, n, beta, st);
    case 512: return launch_qjl_d<512>(s, r, n, beta, st);
    case 1024: return launch_qjl_d<1024>(s, r, n, beta, st);
    case 2048: return launch_qjl_d<2048>(s, r, n, beta, st);
  }
  return (int)hipErrorInvalidValue;
}


// Top-k request of launch_score_impl: k best per query row instead of (or, on the paths
// without a fused form, after) the score matrix.
struct TopkOut {
  int k;
  int64_t* ids;
  float* vals;
};

template <int R, bool TOPK>
static void launch_wide(dim3 grid, hipStream_t st, const ScoreArgs& sa, int64_t n_qblocks,
                        const WideTopk& tk) {
  hipLaunchKernelGGL((score_wide_kernel<R, TOPK>), grid, dim3(kBlock), 0, st, sa, n_qblocks, tk);
}

template <bool TOPK>
static int dispatch_wide(int R, dim3 grid, hipStream_t st, const ScoreArgs& sa, int64_t n_qblocks,
                         const WideTopk& tk) {
  switch (R) {
    case 1: launch_wide<1, TOPK>(grid, st, sa, n_qblocks, tk); return 0;
    case 2: launch_wide<2, TOPK>(grid, st, sa, n_qblocks, tk); return 0;
    case 3: launch_wide<3, TOPK>(grid, st, sa, n_qblocks, tk); return 0;
    case 4: launch_wide<4, TOPK>(grid, st, sa, n_qblocks, tk); return 0;
  }
  return (int)hipErrorInvalidValue;
}

// ws_ext: a workspace the caller provides (ws_cap bytes) instead of a stream-ordered
// temporary; requests that need more than ws_cap return hipErrorOutOfMemory without
// launching anything.
static int launch_score_impl(const PlanDev& p, const void* q, int dt, int64_t nq_per_group,
                             int64_t n_groups, int64_t ldq, const uint8_t* codes, int64_t n,
                             float* scores, const TopkOut* tko, hipStream_t st,
                             void* ws_ext = nullptr, size_t ws_cap = 0) {
  const int64_t nq = nq_per_group * n_groups;
  bool small = true;
  for (int sb = 0; sb < p.nsub; ++sb) small = small && p.sub[sb].D <= 128;
  const int qt_bs = (int)((nq_per_group + 3) / 4);
  // many queries per group on one long inner-product sub-plan: decoded fp16 key tiles on
  // 32x32 fp16 matrix cores (score_f16.hip), top-k then selected from the stored scores;
  // fewer queries per group: the bit-sliced form over 128-coordinate chunks (wide)
  const bool f16 = !small && score_f16_applies(p, nq_per_group);
  const bool wide = !small && !f16 && p.nsub == 1 && nq_per_group >= kWideQT &&
                    p.sub[0].D % 128 == 0;
  const int qt_w = (int)((nq_per_group + kWideQT - 1) / kWideQT);
  const int64_t n_qblocks = (qt_w + kBlock / kWave - 1) / (kBlock / kWave);
  const int64_t nkb = (n + kWideKT * 16 - 1) / (kWideKT * 16);
  // fused top-k on the wide scorer: about 16384 workgroups, each walking a slice of the key
  // blocks (measured on the 10^6-key retrieval shape: 4096 longer-lived workgroups run the
  // same scorer 1.5 times slower, while 65536 pay more in list cuts and merging); otherwise
  // the scores go to a temporary and the top-k kernel reads them back
  const bool fused = tko != nullptr && wide;
  int64_t n_slices = 0;
  if (fused) {
    const int64_t gx = n_groups * n_qblocks;
    n_slices = (16384 + gx - 1) / gx;
    n_slices = n_slices > nkb ? nkb : n_slices;
    n_slices = n_slices > 65535 ? 65535 : n_slices;
  }
  // workspace: per sub-plan y', w, sums, images, epilogue constants
  size_t bytes = 0;
  size_t off_y[2], off_w[2], off_s[2], off_p[2], off_img[2], off_ec[2], off_sc = 0, off_cv = 0, off_ci = 0;
  size_t off_i16 = 0, off_isc = 0;
  auto take = [&](size_t b) { size_t o = bytes; bytes += (b + 255) / 256 * 256; return o; };
  if (fused) {
    off_cv = take((size_t)nq * n_slices * tko->k * 4);
    off_ci = take((size_t)nq * n_slices * tko->k * 4);
  } else if (tko != nullptr) {
    off_sc = take((size_t)nq * n * 4);
  }
  for (int sb = 0; sb < p.nsub; ++sb) {
    const size_t D = p.sub[sb].D;
    // y', w and their sums live in global memory only on the long-vector paths (the
    // bit-sliced query preparation keeps them in LDS)
    off_y[sb] = small ? 0 : take(nq * D * 4);
    off_w[sb] = small ? 0 : take(nq * D * 4);
    off_s[sb] = small ? 0 : take(nq * 2 * 4);
    off_p[sb] = small ? 0 : take(nq * ((p.sub[sb].k + kProjCols - 1) / kProjCols) * 4);
    if (small) {
      off_img[sb] = take((size_t)n_groups * qt_bs * (p.sub[sb].n_planes + 1) * 64 * 32);
      off_ec[sb] = take((size_t)n_groups * qt_bs * 16 * 4);
    } else if (wide) {
      off_img[sb] = take((size_t)n_groups * qt_w * (D / 128) * (p.sub[sb].n_planes + 1) * 64 * 32);
      off_ec[sb] = take((size_t)n_groups * qt_w * kWideQT * 4 * 4);
    }
  }
  if (f16) {
    off_i16 = take((size_t)n_groups * ((nq_per_group + 31) / 32) * 32 * 2 * p.sub[0].D * 2);
    off_isc = take((size_t)nq * 4);
  }
  void* ws = nullptr;
  WorkspaceLease lease;
  if (ws_ext != nullptr) {
    if (bytes > ws_cap) return (int)hipErrorOutOfMemory;
    ws = ws_ext;
  } else {
    const int wrc = lease.acquire(bytes, st);
    if (wrc) return wrc;
    ws = lease.ptr();
  }
  uint8_t* wb = static_cast<uint8_t*>(ws);
  if (tko != nullptr && !fused) scores = reinterpret_cast<float*>(wb + off_sc);
  ScoreArgs sa;
  sa.p = p;
  sa.codes = codes;
  sa.n = n;
  sa.nq_per_group = nq_per_group;
  sa.scores = scores;
  sa.vec_out = ((uintptr_t)scores % 16 == 0) && (n % 4 == 0);
  for (int sb = 0; sb < 2; ++sb) { sa.img[sb] = nullptr; sa.ec[sb] = nullptr; sa.yrot[sb] = nullptr; sa.w[sb] = nullptr; }
  for (int sb = 0; sb < p.nsub; ++sb) {
    QPrepArgs qa;
    qa.s = p.sub[sb];
    qa.q = q;
    qa.ldq = ldq;
    qa.is_bf16 = dt == TQ_BF16;
    qa.yrot = reinterpret_cast<float*>(wb + off_y[sb]);
    qa.w = reinterpret_cast<float*>(wb + off_w[sb]);
    qa.sums = reinterpret_cast<float*>(wb + off_s[sb]);
    sa.yrot[sb] = qa.yrot;
    sa.w[sb] = qa.w;
    if (small) {
      QFusedArgs fa;
      fa.s = p.sub[sb];
      fa.q = q;
      fa.ldq = ldq;
      fa.is_bf16 = dt == TQ_BF16;
      fa.nq = nq;
      fa.nq_per_group = nq_per_group;
      fa.n_qtiles = qt_bs;
      fa.n_heads = p.n_heads > 0 ? p.n_heads : 1;
      fa.img = reinterpret_cast<uint32_t*>(wb + off_img[sb]);
      fa.ec = reinterpret_cast<float*>(wb + off_ec[sb]);
      const int prc = launch_qprep_bitslice(fa, p.sub[sb].D, nq, st);
      if (prc) return prc;
      sa.img[sb] = fa.img;
      sa.ec[sb] = fa.ec;
    } else {
      hipLaunchKernelGGL(qprep_kernel, dim3((unsigned)nq), dim3(kBlock), 0, st, qa);
      if (p.sub[sb].k > 0) {               // w = S y' (an MSE plan has no projection)
        const int nparts = (p.sub[sb].k + kProjCols - 1) / kProjCols;
        float* part = reinterpret_cast<float*>(wb + off_p[sb]);
        hipLaunchKernelGGL(qproj_mfma_kernel, dim3((unsigned)((nq + kProjRows - 1) / kProjRows), (unsigned)nparts),
                           dim3(kBlock), 0, st, qa, nq, part);
        hipLaunchKernelGGL(qsum_kernel, dim3((unsigned)((nq + kBlock - 1) / kBlock)), dim3(kBlock), 0,
                           st, qa.sums, part, nq, nparts);
      } else {
        sa.w[sb] = nullptr;
      }
      if (wide) {
        WideImgArgs wa;
        wa.s = p.sub[sb];
        wa.yrot = qa.yrot;
        wa.w = qa.w;
        wa.sums = qa.sums;
        wa.nq_per_group = nq_per_group;
        wa.n_qtiles = qt_w;
        wa.img = reinterpret_cast<uint32_t*>(wb + off_img[sb]);
        wa.ec = reinterpret_cast<float*>(wb + off_ec[sb]);
        hipLaunchKernelGGL(qimage_wide_kernel, dim3((unsigned)(n_groups * qt_w)), dim3(kBlock), 0,
                           st, wa);
        sa.img[sb] = wa.img;
        sa.ec[sb] = wa.ec;
      }
    }
  }
  int rc = 0;
  if (small) {
    sa.n_qtiles = qt_bs;
    if (!dispatch_bitslice(sa, n_groups * qt_bs, st)) rc = (int)hipErrorInvalidValue;
  } else if (f16) {
    rc = launch_score_f16(p, sa.yrot[0], sa.w[0], reinterpret_cast<uint16_t*>(wb + off_i16),
                          reinterpret_cast<float*>(wb + off_isc), nq_per_group, n_groups, codes, n,
                          scores, st);
  } else if (wide) {
    sa.n_qtiles = qt_w;
    WideTopk tk;
    tk.k = fused ? tko->k : 0;
    tk.n_slices = n_slices;
    tk.cv = fused ? reinterpret_cast<float*>(wb + off_cv) : nullptr;
    tk.ci = fused ? reinterpret_cast<int*>(wb + off_ci) : nullptr;
    const int64_t gy = fused ? n_slices : (nkb < 65535 ? nkb : 65535);
    const dim3 grid((unsigned)(n_groups * n_qblocks), (unsigned)gy);
    const int R = p.sub[0].R;
    rc = fused ? dispatch_wide<true>(R, grid, st, sa, n_qblocks, tk)
               : dispatch_wide<false>(R, grid, st, sa, n_qblocks, tk);
    if (!rc && fused) {
      const int64_t m = n_slices * tko->k;
      hipLaunchKernelGGL(select_kernel<2>, dim3((unsigned)nq), dim3(kBlock), 0, st, tk.cv,
                         tk.ci, m, tko->k, tko->ids, tko->vals);
    }
  } else {
    int sumD = 0;
    for (int sb = 0; sb < p.nsub; ++sb) sumD += p.sub[sb].D;
    const int qt = (2 * 8 * sumD * 4 <= 65536) ? 8 : (2 * 4 * sumD * 4 <= 65536 ? 4 : 2);
    sa.n_qtiles = (int)((nq_per_group + qt - 1) / qt);
    const size_t lds = 2 * (size_t)qt * sumD * 4;
    const int64_t kblocks = (n + kBlock - 1) / kBlock;
    const dim3 grid((unsigned)kblocks, (unsigned)(n_groups * sa.n_qtiles));
    if (qt == 8)
      hipLaunchKernelGGL(score_generic_kernel<8>, grid, dim3(kBlock), lds, st, sa);
    else if (qt == 4)
      hipLaunchKernelGGL(score_generic_kernel<4>, grid, dim3(kBlock), lds, st, sa);
    else
      hipLaunchKernelGGL(score_generic_kernel<2>, grid, dim3(kBlock), lds, st, sa);
  }
  if (!rc) rc = hip_rc(hipGetLastError());
  if (!rc && tko != nullptr && !fused)
    rc = launch_topk(scores, nq, n, tko->k, tko->ids, tko->vals, st);
  return rc;
}

int launch_score(const PlanDev& p, const void* q, int dt, int64_t nq_per_group, int64_t n_groups,
                 int64_t ldq, const uint8_t* codes, int64_t n, float* scores, void* stream) {
  if (n == 0 || nq_per_group == 0 || n_groups == 0) return 0;
  return launch_score_impl(p, q, dt, nq_per_group, n_groups, ldq, codes, n, scores, nullptr,
                           (hipStream_t)stream);
}

// ------------------------------------------------------- scoring without any allocation
// A fixed device array serves as the query workspace of tq_score_noalloc, for callers that
// cannot allocate (HIP graph capture, serving loops, harnesses that forbid hipMalloc).  Each
// device holds its own copy for the life of the process; its address is looked up once per
// device (with that device current) and only that address is handed to kernels (the array's
// name in host code is a host-side stand-in, not a device address).  Calls that overlap on
// one device share the array and race; the kernels write every byte they later read, so
// nothing needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[kScoreScratchBytes];

namespace {
constexpr int kScratchMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kScratchMaxDevices] = {};
}  // namespace

// The current device's address of `scratch`, resolved on first use.
static int scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kScratchMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

int launch_score_noalloc(const PlanDev& p, const void* q, int dt, int64_t nq_per_group,
                         int64_t n_groups, int64_t ldq, const uint8_t* codes, int64_t n,
                         float* scores, void* stream) {
  if (n == 0 || nq_per_group == 0 || n_groups == 0) return 0;
  void* ws = nullptr;
  const int rc = scratch_address(&ws);
  if (rc) return rc;
  return launch_score_impl(p, q, dt, nq_per_group, n_groups, ldq, codes, n, scores, nullptr,
                           (hipStream_t)stream, ws, kScoreScratchBytes);
}

int launch_score_topk(const PlanDev& p, const void* q, int dt, int64_t nq_per_group,
                      int64_t n_groups, int64_t ldq, const uint8_t* codes, int64_t n, int k,
                      int64_t* ids, float* vals, void* stream) {
  if (nq_per_group == 0 || n_groups == 0) return 0;
  const TopkOut tko{k, ids, vals};
  return launch_score_impl(p, q, dt, nq_per_group, n_groups, ldq, codes, n, nullptr, &tko,
                           (hipStream_t)stream);
}

template <int D>
static int launch_dequant_mfma_d(const DequantArgs& da, hipStream_t st) {
  const int64_t iters = (da.n + 31) / 32;
  int64_t blocks = (iters + kDqWaves - 1) / kDqWaves;
  if (blocks > 4096) blocks = 4096;
  const dim3 grid((unsigned)blocks), block(kDqWaves * kWave);
  switch (da.s.R) {
    case 1: hipLaunchKernelGGL((dequant_mfma_kernel<D, 1>), grid, block, 0, st, da); break;
    case 2: hipLaunchKernelGGL((dequant_mfma_kernel<D, 2>), grid, block, 0, st, da); break;
    case 3: hipLaunchKernelGGL((dequant_mfma_kernel<D, 3>), grid, block, 0, st, da); break;
    case 4: hipLaunchKernelGGL((dequant_mfma_kernel<D, 4>), grid, block, 0, st, da); break;
    default: return (int)hipErrorInvalidValue;
  }
  return hip_rc(hipGetLastError());
}

template <int D>
static int launch_dequant_d(const DequantArgs& da, hipStream_t st) {
  constexpr int VPB = (kBlock / kWave) * EncCfg<D>::VPP;
  int64_t blocks = (da.n + VPB - 1) / VPB;
  if (blocks > 8192) blocks = 8192;
  const dim3 grid((unsigned)blocks), block(kBlock);
  switch (da.s.R) {
    case 1: hipLaunchKernelGGL((dequant_kernel<D, 1>), grid, block, 0, st, da); break;
    case 2: hipLaunchKernelGGL((dequant_kernel<D, 2>), grid, block, 0, st, da); break;
    case 3: hipLaunchKernelGGL((dequant_kernel<D, 3>), grid, block, 0, st, da); break;
    case 4: hipLaunchKernelGGL((dequant_kernel<D, 4>), grid, block, 0, st, da); break;
    default: return (int)hipErrorInvalidValue;
  }
  return hip_rc(hipGetLastError());
}

int launch_dequantize(const PlanDev& p, const uint8_t* codes, int64_t n, void* out, int dt,
                      int64_t ldo, void* stream) {
  if (n == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  const int es = dt == TQ_BF16 ? 2 : 4;
  for (int sb = 0; sb < p.nsub; ++sb) {
    DequantArgs da;
    da.s = p.sub[sb];
    da.codes = codes;
    da.rec_bytes = p.rec_bytes;
    da.n = n;
    da.out = out;
    da.ldo = ldo;
    da.out_bf16 = dt == TQ_BF16;
    da.vec_store = da.s.chan == nullptr && (uintptr_t)out % 16 == 0 && (ldo * es) % 16 == 0;
    int rc;
    if (da.s.rotkt16 != nullptr && da.s.D <= 128) {
      switch (da.s.D) {
        case 32: rc = launch_dequant_mfma_d<32>(da, st); break;
        case 64: rc = launch_dequant_mfma_d<64>(da, st); break;
        default: rc = launch_dequant_mfma_d<128>(da, st); break;
      }
      if (rc) return rc;
      continue;
    }
    switch (da.s.D) {
      case 32: rc = launch_dequant_d<32>(da, st); break;
      case 64: rc = launch_dequant_d<64>(da, st); break;
      case 128: rc = launch_dequant_d<128>(da, st); break;
      case 256: rc = launch_dequant_d<256>(da, st); break;
      case 512: rc = launch_dequant_d<512>(da, st); break;
      case 1024: rc = launch_dequant_d<1024>(da, st); break;
      case 2048: rc = launch_dequant_d<2048>(da, st); break;
      default: rc = (int)hipErrorInvalidValue;
    }
    if (rc) return rc;
  }
  return 0;
}

int launch_topk(const float* scores, int64_t nq, int64_t n, int k, int64_t* ids, float* vals,
                void* stream) {
  if (nq == 0) return 0;
  hipStream_t st = (hipStream_t)stream;
  if ((reinterpret_cast<uintptr_t>(scores) & 15) == 0 && (n & 3) == 0)
    hipLaunchKernelGGL(select_kernel<0>, dim3((unsigned)nq), dim3(kBlock), 0, st, scores,
                       (const int*)nullptr, n, k, ids, vals);
  else
    hipLaunchKernelGGL(select_kernel<1>, dim3((unsigned)nq), dim3(kBlock), 0, st, scores,
                       (const int*)nullptr, n, k, ids, vals);
  return hip_rc(hipGetLastError());
}

// ============================================================================ KV-cache policy
// Outlier channels by variance (technical overview §4.1.1: about a quarter of a head's channels
// kept at a higher bit width; here the channels of largest variance over a calibration sample).
// Two passes over the sample, each writing per-(row block, channel) fp64 partials that a
// second kernel sums in a fixed order: sum_x, then sum (x - mean)^2; var = that / n.
constexpr int kVarRows = 256;          // rows per partial

__global__ void __launch_bounds__(kBlock) chan_partial_kernel(const void* x, int x_bf16, int64_t n,
                                                              int64_t ldx, int d, int64_t rows_per,
                                                              const double* mean, double* part) {
  const int c = blockIdx.x * kBlock + threadIdx.x;
  if (c >= d) return;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per;
  const int64_t r1 = (r0 + rows_per) < n ? r0 + rows_per : n;
  const double mu = mean ? mean[c] : 0.0;
  double acc = 0.0;
  for (int64_t r = r0; r < r1; ++r) {
    const double v = x_bf16 ? (double)__uint_as_float((uint32_t)static_cast<const uint16_t*>(x)[r * ldx + c] << 16)
                            : (double)static_cast<const float*>(x)[r * ldx + c];
    acc += mean ? (v - mu) * (v - mu) : v;
  }
  part[(size_t)blockIdx.y * d + c] = acc;
}

__global__ void __launch_bounds__(kBlock) chan_sum_kernel(const double* part, int nblk, int d, int64_t n,
                                                          double* out) {
  const int c = blockIdx.x * kBlock + threadIdx.x;
  if (c >= d) return;
  double s = 0.0;
  for (int b = 0; b < nblk; ++b) s += part[(size_t)b * d + c];
  out[c] = s / (double)n;
}

// channel i is an outlier when fewer than n_out channels come before it in the order
// (-variance, channel)
__global__ void __launch_bounds__(kBlock) outlier_rank_kernel(const double* var, int d, int n_out,
                                                              uint8_t* mask) {
  __shared__ double tile[kBlock];
  const int i = blockIdx.x * kBlock + threadIdx.x;
  const double vi = i < d ? var[i] : 0.0;
  int before = 0;
  for (int j0 = 0; j0 < d; j0 += kBlock) {
    __syncthreads();
    tile[threadIdx.x] = j0 + (int)threadIdx.x < d ? var[j0 + threadIdx.x] : 0.0;
    __syncthreads();
    const int m = (d - j0) < kBlock ? d - j0 : kBlock;
    for (int t = 0; t < m; ++t) {
      const double vj = tile[t];
      before += (vj > vi || (vj == vi && j0 + t < i)) ? 1 : 0;
    }
  }
  if (i < d) mask[i] = before < n_out ? 1 : 0;
}

int launch_calibrate_outliers(const void* x, int x_bf16, int64_t n, int64_t ldx, int d, int n_out,
                              double* var, uint8_t* mask, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  // at most 4 M fp64 partials (32 MiB) and at least kVarRows rows per partial
  int64_t nblk = (n + kVarRows - 1) / kVarRows;
  const int64_t cap = ((int64_t)4 << 20) / d > 1 ? ((int64_t)4 << 20) / d : 1;
  if (nblk > cap) nblk = cap;
  if (nblk > 65535) nblk = 65535;
  const int64_t rows_per = (n + nblk - 1) / nblk;
  nblk = (n + rows_per - 1) / rows_per;
  double* ws = nullptr;
  hipError_t e = hipMallocAsync(reinterpret_cast<void**>(&ws), (size_t)(nblk * d + d) * sizeof(double), st);
  if (e != hipSuccess) return (int)e;
  double* part = ws;
  double* mean = ws + nblk * d;
  const dim3 g((unsigned)((d + kBlock - 1) / kBlock), (unsigned)nblk);
  const dim3 g1((unsigned)((d + kBlock - 1) / kBlock));
  hipLaunchKernelGGL(chan_partial_kernel, g, dim3(kBlock), 0, st, x, x_bf16, n, ldx, d, rows_per,
                     (const double*)nullptr, part);
  hipLaunchKernelGGL(chan_sum_kernel, g1, dim3(kBlock), 0, st, (const double*)part, (int)nblk, d, n, mean);
  hipLaunchKernelGGL(chan_partial_kernel, g, dim3(kBlock), 0, st, x, x_bf16, n, ldx, d, rows_per,
                     (const double*)mean, part);
  hipLaunchKernelGGL(chan_sum_kernel, g1, dim3(kBlock), 0, st, (const double*)part, (int)nblk, d, n, var);
  hipLaunchKernelGGL(outlier_rank_kernel, g1, dim3(kBlock), 0, st, (const double*)var, d, n_out, mask);
  int rc = (int)hipGetLastError();
  e = hipFreeAsync(ws, st);
  if (!rc && e != hipSuccess) rc = (int)e;
  return rc;
}

// Streaming append (technical overview §4.1.2: the cache grows by one record per head and
// decode step): records encoded into a temporary are copied to their cache rows, word by word
// (records are 4-byte multiples); rows outside [0, cap) are skipped.
__global__ void __launch_bounds__(kBlock) scatter_records_kernel(const uint32_t* src, int64_t n, int words,
                                                                 const int64_t* index, int64_t cap,
                                                                 uint32_t* cache) {
  const int64_t i = (int64_t)blockIdx.x * (kBlock / kWave) + (threadIdx.x >> 6);
  if (i >= n) return;
  const int64_t row = index[i];
  if (row < 0 || row >= cap) return;
  for (int w = threadIdx.x & 63; w < words; w += kWave) cache[row * words + w] = src[i * words + w];
}

int launch_encode_scatter(const PlanDev& p, const void* x, int dt, int64_t n, int64_t ldx,
                          uint8_t* cache, int64_t cap, const int64_t* index, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  bool direct = true;
  for (int i = 0; i < p.nsub; ++i) direct = direct && p.sub[i].D <= 128 && p.sub[i].rotk != nullptr;
  if (direct) {
    // the D <= 128 encoders write each record straight to its cache row: one launch per
    // sub-plan; with one channel list per head, vector i is its own group (head i % n_heads)
    const bool per_head = p.n_heads > 1;
    int rc = 0;
    for (int i = 0; i < p.nsub && !rc; ++i)
      rc = launch_encode_to(p, i, x, dt, per_head ? 1 : n, ldx, cache, stream, per_head ? n : 1,
                            index, cap);
    return rc;
  }
  if (p.n_heads > 1) return (int)hipErrorInvalidValue;
  void* tmp = nullptr;
  hipError_t e = hipMallocAsync(&tmp, (size_t)n * p.rec_bytes, st);
  if (e != hipSuccess) return (int)e;
  int rc = 0;
  for (int i = 0; i < p.nsub && !rc; ++i)
    rc = launch_encode(p, i, x, dt, n, ldx, static_cast<uint8_t*>(tmp), stream);
  if (!rc) {
    const dim3 g((unsigned)((n + kBlock / kWave - 1) / (kBlock / kWave)));
    hipLaunchKernelGGL(scatter_records_kernel, g, dim3(kBlock), 0, st, (const uint32_t*)tmp, n,
                       p.rec_bytes / 4, index, cap, reinterpret_cast<uint32_t*>(cache));
    rc = (int)hipGetLastError();
  }
  e = hipFreeAsync(tmp, st);
  if (!rc && e != hipSuccess) rc = (int)e;
  return rc;
}

}  // namespace tq
