// Bit-sliced scorer for sub-plans with D <= 128 (gfx950): per-query fp8 images of the
// rotated query and of its QJL projection, then est = n (<y', c[idx]> + gamma sqrt(pi/2)/k
// <w, 2 beta - 1>) for every key of the group as binary dot products on fp8 x fp4 MFMAs
// (TurboQuant technical overview §1.2.3, §4.2.2; deep dive §三).  TurboQuant-MSE records
// (overview §4.1.1, §4.2.1) are scored by the first term alone, est = n <y', c[idx]>.  The
// image layout and the parity-plane expansion are described with bitslice_coord in
// device_common.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "device_common.h"

namespace tq {

// Query preparation for the bit-sliced scorer (every sub-plan D <= 128): one workgroup per
// query.  Wave 0 computes y' (rotation in registers: lane l holds coordinates l and l + 64);
// then two threads per row compute w = S y' (each half a row, all loads of S in flight at
// once); the block reduces the sums and maxima, writes the query's three image rows per
// plane and its epilogue constants; the first query of a tile also clears the rows of tile
// slots past the last query.
template <int D>
__global__ void __launch_bounds__(kBlock) qprep_bitslice_kernel(QFusedArgs a) {
  static_assert(D == 32 || D == 64 || D == 128, "bit-sliced scorer lengths");
  const SubDev& s = a.s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ float ys[128], ws[128];
  __shared__ float red[kBlock / kWave][4];
  const int64_t qi = blockIdx.x;
  const int64_t grp = qi / a.nq_per_group, qq = qi % a.nq_per_group;
  const int qt = (int)(qq / 4), q = (int)(qq % 4);
  const int64_t gt = grp * a.n_qtiles + qt;
  const int np = s.n_planes;
  // the row halves of S this thread multiplies below, loaded first so that their latency
  // overlaps the query's rotation
  constexpr int HALF = D / 2;
  const int row = tid >> 1, half = tid & 1;
  const bool proj = s.k > 0;              // an MSE plan has no projection: w = 0
  uint4 u[HALF / 8];
  if (row < D && proj) {
    const uint16_t* Sj = s.S + (size_t)row * D + half * HALF;
#pragma unroll
    for (int c = 0; c < HALF / 8; ++c) u[c] = reinterpret_cast<const uint4*>(Sj)[c];
  }
  // ---- y' = Pi pad(y) (wave 0); the query and the three rounds' sign words are loaded
  // together before any arithmetic ----
  if (wave == 0) {
    float v[2];
    uint32_t sw[3][2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = lane + 64 * e;
#pragma unroll
      for (int r = 0; r < 3; ++r) sw[r][e] = i < D ? s.signs[r * (D / 32) + i / 32] : 0u;
      float val = 0.f;
      if (i < s.d) {
        const int64_t ch = s.chan ? s.chan[(grp % a.n_heads) * s.d + i] : i;
        val = a.is_bf16 ? bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qi * a.ldq + ch])
                        : reinterpret_cast<const float*>(a.q)[qi * a.ldq + ch];
      }
      v[e] = val;
    }
    constexpr int lanes_used = D < 64 ? D : 64;
#pragma unroll
    for (int r = 0; r < 3; ++r) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int i = lane + 64 * e;
        if (i < D) v[e] = flip_sign(v[e], (sw[r][e] >> (i % 32)) & 1u);
      }
#pragma unroll
      for (int h = 1; h < lanes_used; h <<= 1) {
        const float sgn = (lane & h) ? -1.f : 1.f;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float pv = __shfl_xor(v[e], h);
          v[e] = fmaf(sgn, v[e], pv);
        }
      }
      if (D == 128) {
        const float x0 = v[0], x1 = v[1];
        v[0] = x0 + x1;
        v[1] = x0 - x1;
      }
    }
    float sy = 0.f, my = 0.f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int i = lane + 64 * e;
      if (i < D) {
        v[e] *= s.inv_scale;
        ys[i] = v[e];
        sy += v[e];
        my = fmaxf(my, fabsf(v[e]));
      }
    }
    for (int m = 32; m >= 1; m >>= 1) {
      sy += __shfl_xor(sy, m);
      my = fmaxf(my, __shfl_xor(my, m));
    }
    if (lane == 0) {
      red[0][0] = sy;
      red[0][1] = my;
    }
  }
  __syncthreads();
  // ---- w = S y' : thread pair (2 row, 2 row + 1) shares row tid / 2, k = D rows ----
  float acc = 0.f;
  if (row < D && proj) {
    const float* yh = ys + half * HALF;
#pragma unroll
    for (int c = 0; c < HALF / 8; ++c) {
      const uint32_t wv[4] = {u[c].x, u[c].y, u[c].z, u[c].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        acc = fmaf(__uint_as_float(wv[h] << 16), yh[8 * c + 2 * h], acc);
        acc = fmaf(__uint_as_float(wv[h] & 0xFFFF0000u), yh[8 * c + 2 * h + 1], acc);
      }
    }
  }
  acc += __shfl_xor(acc, 1);
  float sw = 0.f, mw = 0.f;
  if (row < D && half == 0) {
    ws[row] = acc;
    sw = acc;
    mw = fabsf(acc);
  }
  for (int m = 32; m >= 1; m >>= 1) {
    sw += __shfl_xor(sw, m);
    mw = fmaxf(mw, __shfl_xor(mw, m));
  }
  if (lane == 0) {
    red[wave][2] = sw;
    red[wave][3] = mw;
  }
  __syncthreads();
  const float sy = red[0][0], my = red[0][1];
  float swt = 0.f, mwt = 0.f;
#pragma unroll
  for (int w = 0; w < kBlock / kWave; ++w) {
    swt += red[w][2];
    mwt = fmaxf(mwt, red[w][3]);
  }
  float cmax = 0.f;
  for (int p = 0; p < np; ++p) cmax = fmaxf(cmax, fabsf(s.coef[p]));
  const float M1 = my * cmax;
  // powers of two putting the largest image magnitude in (128, 256]
  const float sc_mse = M1 > 0.f ? ldexpf(1.f, 8 - (int)ceilf(log2f(M1))) : 1.f;
  const float sc_qjl = mwt > 0.f ? ldexpf(1.f, 8 - (int)ceilf(log2f(mwt))) : 1.f;
  // ---- image rows 4q .. 4q+3 of every plane: (plane, limb row, lane group, word) items ----
  for (int it = tid; it < (np + 1) * 128; it += kBlock) {
    const int p = it >> 7, limb = (it >> 5) & 3, Ga = (it >> 3) & 3, wd = it & 7;
    uint32_t* img = a.img + ((size_t)gt * (np + 1) + p) * 64 * 8;
    const float cf = p < np ? s.coef[p] * sc_mse : sc_qjl;
    const float* src = p < np ? ys : ws;
    uint32_t word = 0;
    if (limb < 3) {
      float rem[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int e = 4 * wd + b;
        const int K = e < 16 ? 16 * Ga + e : 64 + 16 * Ga + (e - 16);
        const int c = bitslice_coord(K);
        rem[b] = c < D ? cf * src[c] : 0.f;
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
    img[(16 * Ga + 4 * q + limb) * 8 + wd] = word;
  }
  if (tid == 0) {
    const float K = sqrtf(0.5f * (float)M_PI) / (float)D;
    float* e = a.ec + ((size_t)gt * 4 + q) * 4;
    e[0] = -s.coef_sum * sy;
    e[1] = 4.f / sc_mse;
    e[2] = -K * swt;
    e[3] = 4.f * K / sc_qjl;
  }
  // ---- clear tile slots past the last query (done by the tile's first query) ----
  if (q == 0) {
    const int valid = (int)((a.nq_per_group - 4 * qt) < 4 ? (a.nq_per_group - 4 * qt) : 4);
    for (int qz = valid; qz < 4; ++qz) {
      for (int it = tid; it < (np + 1) * 128; it += kBlock) {
        const int p = it >> 7, limb = (it >> 5) & 3, Ga = (it >> 3) & 3, wd = it & 7;
        uint32_t* img = a.img + ((size_t)gt * (np + 1) + p) * 64 * 8;
        img[(16 * Ga + 4 * qz + limb) * 8 + wd] = 0u;
      }
      if (tid < 4) a.ec[((size_t)gt * 4 + qz) * 4 + tid] = 0.f;
    }
  }
}

// One sub-plan's share of a 16-key step (R index bits, D <= 128); lane l handles key column
// l % 16 and code word l / 16.  The MFMA reads the B registers of every lane, so all lanes
// must reach it with defined operands: loads are branch-free from an always-valid record
// (`key_safe`) and masked by selects.  MSE records hold R index words per chunk and the norm
// (no sign word, no gamma).
template <int R> struct KeyWords {
  uint32_t wd[R + 1];
  float nrm, gam;
};

template <int R, bool MSE = false>
__device__ __forceinline__ KeyWords<R> load_key_words(const SubDev& s, const uint8_t* codes,
                                                      int rec_bytes, int64_t key_safe, bool key_ok) {
  constexpr int W = MSE ? R : R + 1;      // words per 32-coordinate chunk
  const int G = (threadIdx.x & 63) >> 4;
  const bool chunk_ok = 32 * G < s.D;
  const uint8_t* rec = codes + key_safe * rec_bytes + s.rec_off;
  const uint32_t* pw = reinterpret_cast<const uint32_t*>(rec) + (chunk_ok ? G : 0) * W;
  KeyWords<R> k;
#pragma unroll
  for (int m = 0; m < W; ++m) {
    const uint32_t v = pw[m];
    k.wd[m] = (key_ok && chunk_ok) ? v : 0u;
  }
  const uint32_t* tail = reinterpret_cast<const uint32_t*>(rec + (s.D / 32) * W * 4);
  if constexpr (MSE) {
    const uint32_t t0 = tail[0];
    k.nrm = key_ok ? __uint_as_float(t0) : 0.f;
    k.wd[R] = 0u;
    k.gam = 0.f;
  } else {
    const uint32_t t0 = tail[0], t1 = tail[1];
    k.nrm = key_ok ? __uint_as_float(t0) : 0.f;
    k.gam = key_ok ? __uint_as_float(t1) : 0.f;
  }
  return k;
}

// est = n (<y', c[idx]> + gamma sqrt(pi/2)/k <w, 2 beta - 1>); an MSE record gives the first
// term alone, n <y', c[idx]> (overview §4.2.2's quantized distance with the norm of §4.2.1)
template <int R, bool MSE = false>
__device__ __forceinline__ float bitslice_estimate(const KeyWords<R>& k, const i32x8* A,
                                                   const float* e4) {
  constexpr int NP = 1 << (R - 1);
  f32x4 am = {0.f, 0.f, 0.f, 0.f}, aq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    uint32_t P = 0;
#pragma unroll
    for (int m = 0; m < R; ++m)
      if ((pmask_c<R>(p) >> m) & 1) P ^= k.wd[m];
    am = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[p], fp4_operand(P), am, 0, 4, 0, 127, 0, 127);
  }
  // the sign plane's product issues before the index planes' sums are read
  if constexpr (!MSE)
    aq = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A[NP], fp4_operand(k.wd[R]), aq, 0, 4, 0, 127, 0, 127);
  const float msum = am[0] + am[1] + am[2];
  if constexpr (MSE) return k.nrm * fmaf(e4[1], msum, e4[0]);
  const float qsum = aq[0] + aq[1] + aq[2];
  return k.nrm * (fmaf(e4[1], msum, e4[0]) + k.gam * fmaf(e4[3], qsum, e4[2]));
}

constexpr int kScoreSteps = 4;   // 16-key steps whose loads are issued together
// Logits leave through a 1 KiB LDS slot per wave: after the 4 steps a lane holds one query's
// logits of keys 16 u + col; read back as 4 consecutive keys per lane, they go out as one
// 16-byte non-temporal store (the logits are written once and not read by this kernel).

template <int R0, int R1, bool MSE = false>
__global__ void __launch_bounds__(kBlock) score_bitslice_kernel(ScoreArgs a, int keys_per_block) {
  static_assert(!MSE || R1 == 0, "MSE plans have one sub-plan");
  constexpr int NP0 = 1 << (R0 - 1);
  constexpr int NP1 = R1 > 0 ? (1 << (R1 - 1)) : 0;
  constexpr int U = kScoreSteps;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int gt = blockIdx.y;                           // group * n_qtiles + qtile
  const int64_t grp = gt / a.n_qtiles, qt = gt % a.n_qtiles;
  const int G = lane >> 4, col = lane & 15;
  i32x8 A0[NP0 + 1];
  i32x8 A1[NP1 + 1];
  {
    const uint32_t* base = a.img[0] + (size_t)gt * (NP0 + 1) * 64 * 8 + lane * 8;
#pragma unroll
    for (int p = 0; p <= NP0; ++p) {
      const uint4 u0 = reinterpret_cast<const uint4*>(base + p * 64 * 8)[0];
      const uint4 u1 = reinterpret_cast<const uint4*>(base + p * 64 * 8)[1];
      A0[p][0] = u0.x; A0[p][1] = u0.y; A0[p][2] = u0.z; A0[p][3] = u0.w;
      A0[p][4] = u1.x; A0[p][5] = u1.y; A0[p][6] = u1.z; A0[p][7] = u1.w;
    }
  }
  if constexpr (R1 > 0) {
    const uint32_t* base = a.img[1] + (size_t)gt * (NP1 + 1) * 64 * 8 + lane * 8;
#pragma unroll
    for (int p = 0; p <= NP1; ++p) {
      const uint4 u0 = reinterpret_cast<const uint4*>(base + p * 64 * 8)[0];
      const uint4 u1 = reinterpret_cast<const uint4*>(base + p * 64 * 8)[1];
      A1[p][0] = u0.x; A1[p][1] = u0.y; A1[p][2] = u0.z; A1[p][3] = u0.w;
      A1[p][4] = u1.x; A1[p][5] = u1.y; A1[p][6] = u1.z; A1[p][7] = u1.w;
    }
  }
  float e0[4], e1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) e0[i] = a.ec[0][((size_t)gt * 4 + G) * 4 + i];
  if constexpr (R1 > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) e1[i] = a.ec[1][((size_t)gt * 4 + G) * 4 + i];
  }
  __shared__ __attribute__((aligned(16))) float xpose[kBlock / kWave][4 * 64];
  const int64_t qq = qt * 4 + G;
  const bool q_ok = qq < a.nq_per_group;
  float* out = a.scores + (grp * a.nq_per_group + qq) * a.n;
  const uint8_t* codes = a.codes + grp * a.n * (int64_t)a.p.rec_bytes;
  const int64_t kb0 = (int64_t)blockIdx.x * keys_per_block;
  const int64_t kend = (kb0 + keys_per_block < a.n) ? kb0 + keys_per_block : a.n;
  for (int64_t k0 = kb0 + wave * 16 * U; k0 < kend; k0 += 16 * U * (kBlock / kWave)) {
    KeyWords<R0> w0[U];
    KeyWords<(R1 > 0 ? R1 : 1)> w1[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t key = k0 + 16 * u + col;
      const bool key_ok = key < kend;
      const int64_t key_safe = key_ok ? key : kend - 1;
      w0[u] = load_key_words<R0, MSE>(a.p.sub[0], codes, a.p.rec_bytes, key_safe, key_ok);
      if constexpr (R1 > 0)
        w1[u] = load_key_words<R1>(a.p.sub[1], codes, a.p.rec_bytes, key_safe, key_ok);
    }
    // the wave's 4 x 64 logits through LDS, so that each lane stores 4 consecutive keys of
    // its query with one 16-byte write
    float* tr = xpose[wave];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float est = bitslice_estimate<R0, MSE>(w0[u], A0, e0);
      if constexpr (R1 > 0) est += bitslice_estimate<R1>(w1[u], A1, e1);
      asm volatile("" : "+v"(est));
      tr[G * 64 + 16 * u + col] = est;
    }
    __builtin_amdgcn_wave_barrier();
    const float4 v4 = *reinterpret_cast<const float4*>(tr + G * 64 + 4 * col);
    __builtin_amdgcn_wave_barrier();
    const int64_t kfirst = k0 + 4 * col;
    if (q_ok) {
      if (a.vec_out && kfirst + 4 <= kend) {
        typedef __attribute__((ext_vector_type(4))) float f4;
        const f4 v = {v4.x, v4.y, v4.z, v4.w};
        __builtin_nontemporal_store(v, reinterpret_cast<f4*>(out + kfirst));
      } else {
        const float vv[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (kfirst + j < kend) out[kfirst + j] = vv[j];
      }
    }
  }
}

template <int R0, int R1, bool MSE = false>
static void launch_bitslice(const ScoreArgs& sa, int64_t n_gt, hipStream_t st) {
  // 2048 keys per block when that still gives ~2048 blocks; fewer (down to one 256-key batch
  // per block) for short code sets, so that small problems still spread over the chip
  const int64_t per_gt = n_gt >= 2048 ? 1 : 2048 / n_gt;
  int64_t kpb = (sa.n + per_gt - 1) / per_gt;
  kpb = (kpb + 255) / 256 * 256;
  kpb = kpb < 256 ? 256 : (kpb > 2048 ? 2048 : kpb);
  const int64_t kblocks = (sa.n + kpb - 1) / kpb;
  hipLaunchKernelGGL((score_bitslice_kernel<R0, R1, MSE>), dim3((unsigned)kblocks, (unsigned)n_gt),
                     dim3(kBlock), 0, st, sa, (int)kpb);
}

bool dispatch_bitslice(const ScoreArgs& sa, int64_t n_gt, hipStream_t st) {
  const int r0 = sa.p.sub[0].R, r1 = sa.p.nsub > 1 ? sa.p.sub[1].R : 0;
  if (sa.p.sub[0].mse) {
    if (sa.p.nsub != 1) return false;
    switch (r0) {
      case 1: launch_bitslice<1, 0, true>(sa, n_gt, st); return true;
      case 2: launch_bitslice<2, 0, true>(sa, n_gt, st); return true;
      case 3: launch_bitslice<3, 0, true>(sa, n_gt, st); return true;
      case 4: launch_bitslice<4, 0, true>(sa, n_gt, st); return true;
      default: return false;
    }
  }
#define TQ_BS(A, B) if (r0 == A && r1 == B) { launch_bitslice<A, B>(sa, n_gt, st); return true; }
  TQ_BS(1, 0) TQ_BS(2, 0) TQ_BS(3, 0) TQ_BS(4, 0)
  TQ_BS(1, 1) TQ_BS(1, 2) TQ_BS(1, 3) TQ_BS(1, 4)
  TQ_BS(2, 1) TQ_BS(2, 2) TQ_BS(2, 3) TQ_BS(2, 4)
  TQ_BS(3, 1) TQ_BS(3, 2) TQ_BS(3, 3) TQ_BS(3, 4)
  TQ_BS(4, 1) TQ_BS(4, 2) TQ_BS(4, 3) TQ_BS(4, 4)
#undef TQ_BS
  return false;
}

int launch_qprep_bitslice(const QFusedArgs& fa, int D, int64_t nq, hipStream_t st) {
  const dim3 qgrid((unsigned)nq);
  switch (D) {
    case 32: hipLaunchKernelGGL(qprep_bitslice_kernel<32>, qgrid, dim3(kBlock), 0, st, fa); break;
    case 64: hipLaunchKernelGGL(qprep_bitslice_kernel<64>, qgrid, dim3(kBlock), 0, st, fa); break;
    case 128: hipLaunchKernelGGL(qprep_bitslice_kernel<128>, qgrid, dim3(kBlock), 0, st, fa); break;
    default: return (int)hipErrorInvalidValue;
  }
  return 0;
}

}  // namespace tq
