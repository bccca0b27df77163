// Internal declarations shared by the host code and the HIP kernels of libtq.
#pragma once
#include <cstdint>

#include "../../include/tq.h"

namespace tq {

constexpr int kMaxR = 4;         // index bits per coordinate: b - 1 with b <= 5
constexpr int kMinD = 32;
constexpr int kMaxD = 2048;
constexpr int kMaxHeads = 1024;  // heads of a layer plan (one channel list each)

// Host tables (host_tables.cpp)
void philox4x32_10(uint64_t block, uint32_t domain, uint64_t seed, uint32_t out[4]);
void sign_words(uint64_t seed, int subset, int D, uint32_t* words);
uint16_t bf16_rne_from_double(double x);
void qjl_matrix_bf16(uint64_t seed, int subset, int k, int D, uint16_t* S);
int solve_codebook(int D, int R, double* levels, double* thresholds);

// Per-sub-plan parameters handed to kernels by value.
struct SubDev {
  int d;            // channels of this sub-plan
  int D;            // rotated length (power of two)
  int logD;
  int R;            // index bits
  int k;            // QJL rows (= D)
  int rec_off;      // byte offset of the sub-record inside a vector record
  int rec_sub;      // bytes of the sub-record
  int mse;          // 1: TurboQuant-MSE record (R words per chunk, then the norm; k = 0)
  int n_planes;     // 2^(R-1) odd-subset planes used by the bit-sliced scorer
  float inv_scale;  // D^(-3/2): the three normalized transforms folded into one multiply
  float thr[15];    // 2^R - 1 thresholds (ascending)
  float lev[16];    // 2^R levels (ascending)
  float coef[8];    // coefficient of each odd-subset parity plane (scorer)
  uint8_t plane_mask[8];  // bit m set = index bit m enters the parity plane
  float coef_sum;   // sum of coef
  const uint32_t* signs;  // device [3][D/32]; bit set = -1
  const uint16_t* S;      // device [k][D] bf16 bit patterns
  const int32_t* chan;    // device [n_heads][d] input channel of each coordinate (one list per
                          // head of a layer plan), or null (identity)
  // D <= 128 only: the rotation and the QJL matrix pre-arranged as MFMA A operands
  // (16x16x32 bf16 tiles, 64 lanes x 8 values each)
  const uint16_t* rotk;   // [2 limbs][D/16 row tiles][D/32 k steps][64][8]: D^(3/2) Pi
  const uint16_t* rotk16; // [D/16][D/32][64][8]: the same in one exact fp16 limb, or null
  const uint16_t* rotkt16; // [D/16][D/32][64][8]: K^T likewise (rows = input coordinates,
                           // lane group G of tile jt, element e: 32 (jt/2) + 8 G + 4 (jt%2) + e;
                           // k = rotated coordinate), with rotk16
  const uint16_t* sperm;  // [D/16][D/32][64][8]: S with columns in the residual register order
  // D = 128 inner-product plans whose K is exact in fp16 and whose 2^8 S is exact in fp16:
  // operands of the 32x32 encoder (encode128.hip; layouts described there), else null
  const uint16_t* k16_32;  // [4][8][64][8] fp16 K
  const uint16_t* s16_32;  // [4][8][64][8] fp16 2^8 S
  const uint8_t* s8_32;    // [4][2][64][32] e4m3 S
  // Split and layer plans whose input rows have at most 128 columns (a multiple of 8), for
  // D = 128 sub-plans with the 32x32 operands above and D <= 64 sub-plans with rotk16: per
  // head h, K in fp16 with the channel selection folded in (k = the input column; unselected
  // columns zero) and the masks of the selected columns, else null
  const uint16_t* kfold;   // D = 128: [n_heads][4][8][64][8] (32x32 encoder layout);
                           // D <= 64: [n_heads][D/16][4][64][8] (rotk16 layout, 4 k steps)
  const uint32_t* xmask;   // [n_heads][64 words]: D = 128 [8 k steps][2 halves][4 words],
                           // D <= 64 [4 k steps][4 lane groups][4 words]
  int x_cols;              // columns of the input rows the folded tables expect
};

struct PlanDev {
  int d;
  int nsub;
  int rec_bytes;
  int n_heads;      // channel lists per sub-plan (a layer plan with one outlier mask per head)
  SubDev sub[2];
};

}  // namespace tq

struct tq_plan {
  tq::PlanDev dev;      // device pointers inside
  int device;           // HIP device the tables live on
  void* dev_alloc;      // single device allocation holding every table
  uint64_t seed;
  int bits[2];
};

// Kernel launchers (kernels.hip).  Return 0 or a HIP error code.
namespace tq {
int launch_encode(const PlanDev& p, int sub, const void* x, int dt, int64_t n, int64_t ldx,
                  uint8_t* codes, void* stream, int64_t n_groups = 1);
int launch_qjl(const SubDev& s, const float* r, int64_t n, uint32_t* beta, void* stream);
int launch_score(const PlanDev& p, const void* q, int dt, int64_t nq_per_group, int64_t n_groups,
                 int64_t ldq, const uint8_t* codes, int64_t n, float* scores, void* stream);
// Bytes of the fixed per-device array behind launch_score_noalloc; a request whose query
// workspace exceeds it returns hipErrorOutOfMemory before any launch.
constexpr size_t kScoreScratchBytes = (size_t)16 << 20;
int launch_score_noalloc(const PlanDev& p, const void* q, int dt, int64_t nq_per_group,
                         int64_t n_groups, int64_t ldq, const uint8_t* codes, int64_t n,
                         float* scores, void* stream);
int launch_topk(const float* scores, int64_t nq, int64_t n, int k, int64_t* ids, float* vals,
                void* stream);
int launch_dequantize(const PlanDev& p, const uint8_t* codes, int64_t n, void* out, int dt,
                      int64_t ldo, void* stream);
int launch_attend(const PlanDev& p, const float* logits, int64_t nq_per_group, int64_t n_groups,
                  int64_t n, float scale, const uint8_t* codes, void* out, int dt, int64_t ldo,
                  void* stream);
int launch_rerank(const void* q, int q_bf16, int64_t nq, int64_t ldq, const void* x, int x_bf16,
                  int64_t n, int64_t ldx, int d, const int64_t* cand, int kc, int k, int64_t* ids,
                  float* vals, void* stream);
int launch_calibrate_outliers(const void* x, int x_bf16, int64_t n, int64_t ldx, int d, int n_out,
                              double* var, uint8_t* mask, void* stream);
int launch_encode_scatter(const PlanDev& p, const void* x, int dt, int64_t n, int64_t ldx,
                          uint8_t* cache, int64_t cap, const int64_t* index, void* stream);
int launch_score_topk(const PlanDev& p, const void* q, int dt, int64_t nq_per_group,
                      int64_t n_groups, int64_t ldq, const uint8_t* codes, int64_t n, int k,
                      int64_t* ids, float* vals, void* stream);
}  // namespace tq
