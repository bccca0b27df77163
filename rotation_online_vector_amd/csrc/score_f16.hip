// Scorer for long vectors with many queries per group (D >= 256, one inner-product sub-plan),
// and for every TurboQuant-MSE plan with D >= 256 (centroid terms only, see below):
// the estimate est = n (<y', c[idx]> + gamma sqrt(pi/2)/k <w, 2 beta - 1>) (TurboQuant
// technical overview §1.2.3, §4.2.2; deep dive §三) as one fp16 matrix product over 2D terms
// per (query, key): the key side holds, per 32-coordinate chunk, the 32 centroid values
// c[idx] and the 32 signed QJL weights +-gamma sqrt(pi/2)/k, decoded once per workgroup from
// the record into LDS; the query side holds y' and w in fp16 at a per-query power-of-two
// scale.  This does 2D multiply-accumulates per score on fp16 matrix cores, where the
// bit-sliced form needs (2^(R-1) + 1) planes x 2 limbs x D binary ones on fp8 x fp4.
//
// Workgroup: 256 queries x 128 keys of one group; wave w takes queries 64w .. 64w + 63 (two
// 32-row tiles) against the 128 keys (four 32-column tiles) on v_mfma_f32_32x32x16_f16.  Per
// chunk of 32 coordinates the 256 threads decode the 128 keys' next chunk (thread t: key t/2,
// coordinates 16 (t%2) .. +15 of both halves) into the other LDS buffer while the waves
// multiply the current one.  Query blocks vary fastest over the grid, so with up to 8 of them
// per group each of the chip's 8 L2 slices (workgroups go round-robin over them) serves a
// fixed subset of the query images.
//
// MSE records (R index words per chunk and the norm; overview §4.2.1's index vectors) give
// est = n <y', c[idx]> (the quantized distance of §4.2.2): the decode writes the centroid k
// steps only and the product runs over D terms.  There is no other long-vector path for them,
// so any query count takes this one (a group's rows pad to whole 32-row tiles).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "device_common.h"

namespace tq {

namespace {

typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kMT = 2;               // 32-query tiles per wave
constexpr int kFQ = 4 * 32 * kMT;    // queries per workgroup
constexpr int kFK = 128;             // keys per workgroup (4 tiles of 32)
constexpr float kSignUp = 4096.f;    // 2^12: the key's sign weights are scaled up by it and
constexpr float kSignDown = 1.f / 4096.f;   // the query's w down, keeping both in fp16 range

__device__ __forceinline__ uint32_t f16_bits(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)v);
}

}  // namespace

// One workgroup per query row: the row's image in fp16, per chunk the 32 values of sigma y'
// and then the 32 of sigma w 2^-12, with sigma the power of two that puts the largest
// magnitude in [2^13, 2^14); isc = 1 / sigma (0 rows: sigma = 1).  The image is stored as the
// scorer's A fragments, [32-row tile][chunk][k step][lane][8]: lane l of a fragment holds row
// l % 32 of the tile and the 8 values 16 k + 8 (l / 32) .. +7 of the chunk, so that one load
// instruction reads 1 KiB of consecutive memory.
__global__ void __launch_bounds__(kBlock) qimage_f16_kernel(const float* yrot, const float* w,
                                                            int D, int64_t nq_per_group,
                                                            uint16_t* img, float* isc) {
  const int64_t q = blockIdx.x;
  const float* y = yrot + q * D;
  const float* wq = w ? w + q * D : nullptr;     // none for an MSE plan: its half of the image is 0
  __shared__ float red[kBlock / kWave];
  float m = 0.f;
  for (int i = threadIdx.x; i < D; i += kBlock)
    m = fmaxf(m, fmaxf(fabsf(y[i]), wq ? fabsf(wq[i]) * kSignDown : 0.f));
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  m = 0.f;
#pragma unroll
  for (int i = 0; i < kBlock / kWave; ++i) m = fmaxf(m, red[i]);
  const float sigma = m > 0.f ? ldexpf(1.f, 14 - __builtin_amdgcn_frexp_expf(m)) : 1.f;
  // the row's place: tiles are counted per group (a group's rows start a new tile), lane r
  // (first half) or r + 32 (second half) of each fragment
  const int64_t tpg = (nq_per_group + 31) / 32;
  const int64_t grp = q / nq_per_group, qi = q % nq_per_group;
  uint16_t* tile = img + (grp * tpg + (qi >> 5)) * 64 * (int64_t)D;   // 32 rows x 2D values
  const int r = (int)(qi & 31);
  for (int i = threadIdx.x; i < 2 * D; i += kBlock) {
    const int g = i >> 6, e = i & 63;                       // chunk, image entry
    const float v = e < 32 ? y[32 * g + e] * sigma
                           : (wq ? wq[32 * g + e - 32] * (sigma * kSignDown) : 0.f);
    const int ks = e >> 4, hh = (e >> 3) & 1, j = e & 7;
    tile[((g * 4 + ks) * 64 + r + 32 * hh) * 8 + j] = (uint16_t)f16_bits(v);
  }
  if (threadIdx.x == 0) isc[q] = 1.f / sigma;
}

struct ScoreF16Args {
  SubDev s;
  const uint16_t* img;     // query images as A fragments: [group][row tile of 32][D/32 chunks][4][64][8]
  const float* isc;        // [rows] 1 / sigma
  const uint8_t* codes;    // group g's records from record g * n
  int rec_bytes;
  int64_t n;
  int64_t nq_per_group;
  int64_t n_qblocks;       // query blocks of kFQ per group
  float* scores;           // [n_groups * nq_per_group][n]
};

template <int R, bool MSE>
__global__ void __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2)))
score_f16_kernel(ScoreF16Args a) {
  static_assert(kBlock == 256 && kFK == 128, "thread t decodes half a chunk of key t / 2");
  constexpr int W = MSE ? R : R + 1;       // words per chunk: R index planes (, the sign word)
  constexpr int KS = MSE ? 2 : 4;          // k steps per chunk: centroids (, sign weights)
  constexpr int NPAIR = 1 << (2 * R);
  const SubDev& s = a.s;
  const int D = s.D, NC = D / 32;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t grp = blockIdx.y;
  const int qb = (int)(blockIdx.x % a.n_qblocks);
  const int64_t k0 = (int64_t)(blockIdx.x / a.n_qblocks) * kFK;
  const int64_t qrow0 = grp * a.nq_per_group;               // the group's first query row
  // pair table: entry i = fp16 levels of two coordinates whose index bits interleave in i
  // (bit 2m: the first coordinate's bit m, bit 2m + 1: the second's)
  __shared__ uint32_t ptab[NPAIR];
  // B fragments of a chunk: [buffer][k step][key tile][lane], k steps 0, 1 = centroids of
  // coordinates 0-15, 16-31, k steps 2, 3 = sign weights of QJL rows 0-15, 16-31
  __shared__ uint4 bfr[2][4][4][64];
  __shared__ float knorm[kFK];
  for (int i = tid; i < NPAIR; i += kBlock) {
    int ia = 0, ib = 0;
#pragma unroll
    for (int m = 0; m < R; ++m) {
      ia |= ((i >> (2 * m)) & 1) << m;
      ib |= ((i >> (2 * m + 1)) & 1) << m;
    }
    ptab[i] = f16_bits(s.lev[ia]) | (f16_bits(s.lev[ib]) << 16);
  }
  // ---- this thread's decode role: key kk (clamped to the group), coordinates 16 h .. +15 ----
  const int kk = tid >> 1, h = tid & 1;
  const int64_t key = k0 + kk < a.n ? k0 + kk : a.n - 1;
  const uint8_t* rec = a.codes + (grp * a.n + key) * (int64_t)a.rec_bytes + s.rec_off;
  const uint32_t* rw = reinterpret_cast<const uint32_t*>(rec);
  uint32_t G2;                                               // +gamma K 2^12, both halves
  {
    const float* tail = reinterpret_cast<const float*>(rec + NC * W * 4);
    const float nk = tail[0], gam = MSE ? 0.f : tail[1];
    const float K = sqrtf(0.5f * (float)M_PI) / (float)D;
    const uint32_t g16 = f16_bits(gam * K * kSignUp);
    G2 = g16 | (g16 << 16);
    if (h == 0) knorm[kk] = (k0 + kk < a.n) ? nk : 0.f;
  }
  const int nt = kk >> 5, col = kk & 31;
  auto decode = [&](const uint32_t (&wd0)[W], int buf) {
    // this thread's 16 coordinates moved to bits 0..15, so every position below is a constant
    uint32_t wd[W];
#pragma unroll
    for (int m = 0; m < W; ++m) wd[m] = wd0[m] >> (16 * h);
    uint32_t z = 0u;
    if constexpr (!MSE) {
      const uint32_t nb = ~wd[R];                          // set bit = beta 0 = weight -G
      // sign bit 2j + 1 moved to 2j + 16, so that one shift puts pair j's two bits at 15, 31
      z = (nb & 0x5555u) | ((nb & 0xAAAAu) << 15);
    }
    // planes 0 and 1 of pair j side by side: nibble j / 2 of pq[j % 2]
    uint32_t pq[2] = {0u, 0u};
    if constexpr (R >= 2) {
      pq[0] = (wd[0] & 0x3333u) | ((wd[1] << 2) & 0xCCCCu);
      pq[1] = ((wd[0] >> 2) & 0x3333u) | (wd[1] & 0xCCCCu);
    }
    uint32_t cw[8], sw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t idx;
      if constexpr (R >= 2) idx = (pq[j & 1] >> (4 * (j >> 1))) & 15u;
      else idx = (wd[0] >> (2 * j)) & 3u;
#pragma unroll
      for (int m = 2; m < R; ++m) idx |= ((wd[m] >> (2 * j)) & 3u) << (2 * m);
      cw[j] = ptab[idx];
      sw[j] = ((z << (15 - 2 * j)) & 0x80008000u) | G2;
    }
    bfr[buf][h][nt][col] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    bfr[buf][h][nt][col + 32] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    if constexpr (!MSE) {
      bfr[buf][2 + h][nt][col] = make_uint4(sw[0], sw[1], sw[2], sw[3]);
      bfr[buf][2 + h][nt][col + 32] = make_uint4(sw[4], sw[5], sw[6], sw[7]);
    }
  };
  auto load_words = [&](int g, uint32_t (&wd)[W]) {
#pragma unroll
    for (int m = 0; m < W; ++m) wd[m] = rw[g * W + m];
  };
  // ---- this lane's query rows: tiles mt = 0, 1 of wave w, row 32 mt + lane % 32 ----
  const int half = lane >> 5, c32 = lane & 31;
  // (the query rows are padded to a whole 32-row tile in the image; rows past the group's
  // last query hold what the image kernel left there and are never stored)
  const uint4* arow[kMT];
  const int64_t tpg = (a.nq_per_group + 31) / 32;          // image tiles per group
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt) {
    int64_t t32 = ((int64_t)qb * kFQ + 32 * kMT * wave + 32 * mt) >> 5;
    t32 = t32 < tpg ? t32 : tpg - 1;                       // past the group's rows: not stored
    arow[mt] = reinterpret_cast<const uint4*>(a.img + (grp * tpg + t32) * 64 * (int64_t)D) + lane;
  }
  auto load_a = [&](int g, uint4 (&av)[kMT][4]) {
#pragma unroll
    for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) av[mt][ks] = arow[mt][(g * 4 + ks) * 64];
  };
  f32x16 acc[kMT][4];
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[mt][t][i] = 0.f;
  uint4 a0[kMT][4], a1[kMT][4];
  uint32_t w0[W], w1[W];                                   // record words, two chunks ahead
  load_a(0, a0);
  load_words(0, w0);
  __syncthreads();                                         // the pair table
  decode(w0, 0);
  if (NC > 1) load_words(1, w1);
  __syncthreads();
  // One chunk: the MFMAs of chunk g on the query rows av (loaded during chunk g - 1) and the
  // keys in bfr[g % 2], while chunk g + 1's rows load into an, chunk g + 2's record words into
  // wl, and chunk g + 1's keys (words wd, loaded during chunk g - 1) are decoded into the
  // other buffer (last read before the previous barrier).  The B fragments of k step ks + 1
  // are read from LDS while the MFMAs of step ks issue, one read per two MFMAs, so that each
  // read has about eight MFMAs of time to land.
  auto chunk = [&](int g, const uint4 (&av)[kMT][4], uint4 (&an)[kMT][4], uint32_t (&wl)[W],
                   const uint32_t (&wd)[W]) {
    const int buf = g & 1;
    const bool more = g + 1 < NC;
    if (more) load_a(g + 1, an);
    if (g + 2 < NC) load_words(g + 2, wl);
    uint4 bc[4], bn[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) bc[t] = bfr[buf][0][t][lane];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks < KS - 1)
#pragma unroll
        for (int t = 0; t < 4; ++t) bn[t] = bfr[buf][ks + 1][t][lane];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const f16x8 bv = f16x8_from_words(bc[t].x, bc[t].y, bc[t].z, bc[t].w);
#pragma unroll
        for (int mt = 0; mt < kMT; ++mt)
          acc[mt][t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
              f16x8_from_words(av[mt][ks].x, av[mt][ks].y, av[mt][ks].z, av[mt][ks].w), bv,
              acc[mt][t], 0, 0, 0);
      }
      if (ks < KS - 1)
#pragma unroll
        for (int t = 0; t < 4; ++t) bc[t] = bn[t];
    }
    // issue order: the 4 reads of step 0, then (1 LDS read, 2 MFMAs) x 4 (KS - 1), then the
    // last 8
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // 0x100: LDS reads
#pragma unroll
    for (int i = 0; i < 4 * (KS - 1); ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);   // 0x008: matrix instructions
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    if (more) decode(wd, buf ^ 1);
    __syncthreads();
  };
  // two chunks per trip with the row and word buffers swapped (D / 32 is even), so that no
  // registers are copied between chunks
  for (int g = 0; g < NC; g += 2) {
    chunk(g, a0, a1, w0, w1);
    chunk(g + 1, a1, a0, w1, w0);
  }
  // ---- epilogue: element i of tile (mt, t) is query 32 mt + 8 (i / 4) + 4 half + i % 4 of
  // the wave, key 32 t + lane % 32 ----
#pragma unroll
  for (int mt = 0; mt < kMT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t q = (int64_t)qb * kFQ + 32 * kMT * wave + 32 * mt + 8 * (i >> 2) + 4 * half + (i & 3);
      if (q >= a.nq_per_group) continue;
      const float sc = a.isc[qrow0 + q];
      float* out = a.scores + (qrow0 + q) * a.n + k0;
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kc = 32 * t + c32;
        if (k0 + kc < a.n) out[kc] = acc[mt][t][i] * sc * knorm[kc];
      }
    }
}

bool score_f16_applies(const PlanDev& p, int64_t nq_per_group) {
  const SubDev& s = p.sub[0];
  if (p.nsub != 1 || s.D < 256 || s.R < 1 || s.R > 4) return false;
  if (s.mse) return true;                  // the only long-vector path for MSE records
  return s.k == s.D && nq_per_group >= kScoreF16MinQueries;
}

int launch_score_f16(const PlanDev& p, const float* yrot, const float* w, uint16_t* img,
                     float* isc, int64_t nq_per_group, int64_t n_groups, const uint8_t* codes,
                     int64_t n, float* scores, hipStream_t st) {
  const SubDev& s = p.sub[0];
  const int64_t rows = nq_per_group * n_groups;
  hipLaunchKernelGGL(qimage_f16_kernel, dim3((unsigned)rows), dim3(kBlock), 0, st, yrot, w, s.D,
                     nq_per_group, img, isc);
  ScoreF16Args fa;
  fa.s = s;
  fa.img = img;
  fa.isc = isc;
  fa.codes = codes;
  fa.rec_bytes = p.rec_bytes;
  fa.n = n;
  fa.nq_per_group = nq_per_group;
  fa.n_qblocks = (nq_per_group + kFQ - 1) / kFQ;
  fa.scores = scores;
  const int64_t nkb = (n + kFK - 1) / kFK;
  const dim3 grid((unsigned)(nkb * fa.n_qblocks), (unsigned)n_groups);
#define TQ_F16(RR)                                                                          \
  case RR:                                                                                  \
    if (s.mse)                                                                              \
      hipLaunchKernelGGL((score_f16_kernel<RR, true>), grid, dim3(kBlock), 0, st, fa);      \
    else                                                                                    \
      hipLaunchKernelGGL((score_f16_kernel<RR, false>), grid, dim3(kBlock), 0, st, fa);     \
    break;
  switch (s.R) {
    TQ_F16(1)
    TQ_F16(2)
    TQ_F16(3)
    TQ_F16(4)
    default: return (int)hipErrorInvalidValue;
  }
#undef TQ_F16
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? 0 : (int)e;
}

}  // namespace tq
