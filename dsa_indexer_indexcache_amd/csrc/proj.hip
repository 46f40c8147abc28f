// Upstream of the indexer: its projections, the key LayerNorm, rotary encoding of the
// indexer query/key, the folded score scales, and the decode-time cache append.
//
// [IDX] §6.4 (the GLM indexer of the Transformers implementation): the indexer query
// is a projection of the low-rank query latent split into H^I heads of d_I, the key a
// projection of the hidden state followed by a LayerNorm over d_I, the head weights a
// projection of the hidden state times (H^I)^-1/2; the score carries d_I^-1/2 and the
// query/key get rotary position encoding on their rotary part.  [IDX] §4 (the memory
// view of the six-step data flow): each new token is written into the caches before
// it is read.
//
// Reading of the open points: the rotary part is the first rope_dim dimensions in the
// half-split form (dimension j pairs with j + rope_dim/2, angle pos * base^(-2j/rope_dim));
// the projections have no bias; the LayerNorm has weight and bias; d_I^-1/2 is a positive
// factor of the score and is folded into the head weights together with (H^I)^-1/2.
//
// GEMM core: C[n, N] = X[n, K] . W[N, K]^T (nn.Linear weight layout, both operands
// K-contiguous), bf16 in, fp32 accumulate, with v_mfma_f32_16x16x32_bf16.  A workgroup
// of 4 waves computes a 128 x 128 tile (wave (wr, wc) a 64 x 64 quarter: 4 x 4 MFMA
// tiles); K advances 64 at a time through a ring of LDS stages of 128 rows x 64 columns
// for each operand, filled by direct global->LDS copies stages - 1 ahead; rows are 128 bytes
// with their eight 16-byte granules XOR-swizzled by (row & 7), so the 16 rows of a
// fragment read land on distinct banks.  The fp32 tile then goes through LDS to the
// epilogue, which sees whole 128-column rows (one indexer head, or the key).
#include <math.h>

#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kPT = 128;          // tile rows and columns
constexpr int kPK = 64;           // K per stage
constexpr int kPStage = kPT * kPK * 2;  // bytes of one operand's stage (16 KB)

// Two stages for the query projection (two workgroups per CU hide the copy latency);
// four for the key / head-weight projection, whose grid has a workgroup for every 128 rows
// only and whose K (the hidden size) takes a hundred steps, each of them short next to
// the latency of the copies it waits for.
template <int STAGES>
struct ProjSmem {
  union {
    uint8_t stage[STAGES][2][kPStage];  // [stage][operand: 0 = X, 1 = W]
    float tile[kPT][kPT + 1];           // accumulators for the epilogue (+1: no bank conflicts)
  };
};

// Copies 128 rows x 64 bf16 columns (K offset k0) of a row-major [rows, K] bf16 matrix
// into one LDS stage; rows past `rows` re-read the last row (in bounds; never stored).
// Copy j (16 per stage, 4 per wave) fills rows 8 j .. 8 j + 7: lane l lands in row
// 8 j + l / 8 at position l % 8 and fetches granule (l % 8) ^ (row & 7).
__device__ __forceinline__ void stage_copy(const uint16_t* __restrict__ m, int64_t rows, int64_t ld, int64_t row0,
                                           int k0, uint8_t* dst, int wave, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int j = wave + 4 * u;
    const int r = 8 * j + (lane >> 3);
    int64_t gr = row0 + r;
    if (gr > rows - 1) gr = rows - 1;
    const uint16_t* src = m + gr * ld + k0 + 8 * ((lane & 7) ^ (r & 7));
    dma16(src, lds_u32(dst + 1024 * j));
  }
}

// The 128 x 128 fp32 tile C[row0 .., col0 ..] of X . W^T into sm.tile (K % 64 == 0).
template <int STAGES>
__device__ void gemm_tile(const uint16_t* __restrict__ x, int64_t n, const uint16_t* __restrict__ w, int64_t nout,
                          int K, int64_t row0, int64_t col0, ProjSmem<STAGES>& sm) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g = lane >> 4;
  const int wr = wave >> 1, wc = wave & 1;
  f32x4 acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nst = K / kPK;
  // each stage is 8 copies per wave (4 per operand): "stage s landed" with later stages
  // in flight is a fixed vmcnt
  static_assert(STAGES >= 2 && STAGES <= 4, "vmcnt waits below");
  for (int s = 0; s < STAGES - 1 && s < nst; ++s) {
    stage_copy(x, n, K, row0, s * kPK, sm.stage[s][0], wave, lane);
    stage_copy(w, nout, K, col0, s * kPK, sm.stage[s][1], wave, lane);
  }
  for (int s = 0; s < nst; ++s) {
    // this wave's copies of stage s landed; after the barrier every wave's have, and
    // the buffer of stage s - 1 is no longer read
    const int later = min(STAGES - 2, nst - 1 - s);
    if (later >= 2)
      __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16)
    else if (later == 1)
      __builtin_amdgcn_s_waitcnt(0x0F78);  // vmcnt(8)
    else
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    const int sn = s + STAGES - 1;
    if (sn < nst) {
      stage_copy(x, n, K, row0, sn * kPK, sm.stage[sn % STAGES][0], wave, lane);
      stage_copy(w, nout, K, col0, sn * kPK, sm.stage[sn % STAGES][1], wave, lane);
    }
    const uint8_t* xs = sm.stage[s % STAGES][0];
    const uint8_t* ws = sm.stage[s % STAGES][1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x4 af[4], bf[4];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int r = 64 * wr + 16 * a + c;
        af[a] = *reinterpret_cast<const i32x4*>(xs + r * 128 + 16 * ((4 * ks + g) ^ (r & 7)));
      }
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int r = 64 * wc + 16 * b + c;
        bf[b] = *reinterpret_cast<const i32x4*>(ws + r * 128 + 16 * ((4 * ks + g) ^ (r & 7)));
      }
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = mfma_bf16_16x16x32(af[a], bf[b], acc[a][b]);
    }
  }
  __syncthreads();  // every wave is done with the stages: the tile reuses their memory
  // lane holds C[16 a + 4 g + r][16 b + c] of the wave's quarter
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) sm.tile[64 * wr + 16 * a + 4 * g + r][64 * wc + 16 * b + c] = acc[a][b][r];
  __syncthreads();
}

// Rotary frequencies in turns: f[j] = base^(-2 j / rope_dim) / (2 pi), j < rope_dim / 2,
// computed once on the host in fp64 and passed by value.
struct RopeTurns {
  double f[32];
};

// cos and sin of the angle pos * base^(-2 j / rope_dim).  The angle in turns is reduced to
// [-1/2, 1/2] in fp64 (positions reach 2e5 radians, about 3e4 turns: fp32 would lose about
// 1e-2 of the angle), then the hardware sine and cosine, which take turns, give fp32 values.
__device__ __forceinline__ void rope_angle(int64_t pos, double turns_per_pos, float* cs, float* sn) {
  const double a = (double)pos * turns_per_pos;
  const float f = (float)(a - rint(a));
  *cs = __builtin_amdgcn_cosf(f);
  *sn = __builtin_amdgcn_sinf(f);
}

// Epilogue for the query projection: the tile is one indexer head (128 dims) of 128
// tokens.  Thread t takes token t / 2 and columns 64 (t % 2) ..: the first half holds the
// whole rotary part (rope_dim <= 64) and rotates pairs (j, j + rope_dim / 2).
template <int RD>
__global__ __launch_bounds__(256) void proj_q_kernel(const uint16_t* __restrict__ q_lat, int64_t n, int K,
                                                     const uint16_t* __restrict__ wq, int H,
                                                     const int32_t* __restrict__ pos, RopeTurns turns,
                                                     uint16_t* __restrict__ q_idx) {
  __shared__ ProjSmem<2> sm;
  const int64_t row0 = (int64_t)blockIdx.x * kPT;
  const int head = blockIdx.y;
  gemm_tile<2>(q_lat, n, wq, (int64_t)H * kPT, K, row0, (int64_t)head * kPT, sm);
  const int t = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int64_t row = row0 + t;
  if (row >= n) return;
  float v[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) v[j] = sm.tile[t][64 * half + j];
  if (RD > 0 && half == 0) {
    constexpr int hr = RD / 2;
    const int64_t p = pos[row];
#pragma unroll
    for (int j = 0; j < hr; ++j) {
      float cs, sn;
      rope_angle(p, turns.f[j], &cs, &sn);
      const float a = v[j], b = v[j + hr];
      v[j] = a * cs - b * sn;
      v[j + hr] = a * sn + b * cs;
    }
  }
  uint16_t* dst = q_idx + (row * H + head) * kPT + 64 * half;
#pragma unroll
  for (int j = 0; j < 64; j += 8) {
    const uint4 pk = make_uint4(pack_bf16x2(v[j], v[j + 1]), pack_bf16x2(v[j + 2], v[j + 3]),
                                pack_bf16x2(v[j + 4], v[j + 5]), pack_bf16x2(v[j + 6], v[j + 7]));
    *reinterpret_cast<uint4*>(dst + j) = pk;
  }
}

// Epilogue for the key / head-weight projection.  blockIdx.y == 0: the tile is the key
// (128 dims) of 128 tokens: LayerNorm over the row (two threads per row, combined by a
// lane swap), weight and bias, then the rotary part.  blockIdx.y == 1: columns 0 .. H-1
// are the head weights, times wscale = H^-1/2 d^-1/2.
template <int RD>
__global__ __launch_bounds__(256) void proj_kw_kernel(const uint16_t* __restrict__ h, int64_t n, int K,
                                                      const uint16_t* __restrict__ wk,
                                                      const float* __restrict__ gamma, const float* __restrict__ beta,
                                                      float eps, const uint16_t* __restrict__ ww, int H, float wscale,
                                                      const int32_t* __restrict__ pos, RopeTurns turns,
                                                      uint16_t* __restrict__ k_idx, uint16_t* __restrict__ w_out) {
  __shared__ ProjSmem<4> sm;
  const int64_t row0 = (int64_t)blockIdx.x * kPT;
  const bool key = blockIdx.y == 0;
  if (key)
    gemm_tile<4>(h, n, wk, kPT, K, row0, 0, sm);
  else
    gemm_tile<4>(h, n, ww, H, K, row0, 0, sm);
  const int t = threadIdx.x >> 1, half = threadIdx.x & 1;
  const int64_t row = row0 + t;
  // both threads of a row stay to the end (they exchange partial sums)
  float v[64];
#pragma unroll
  for (int j = 0; j < 64; ++j) v[j] = sm.tile[t][64 * half + j];
  if (!key) {
    if (row >= n) return;
    for (int j = 0; j < 64; ++j) {
      const int col = 64 * half + j;
      if (col < H) w_out[row * H + col] = (uint16_t)f32_to_bf16_bits(v[j] * wscale);
    }
    return;
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 64; ++j) s += v[j];
  s += __shfl_xor(s, 1);
  const float mu = s * (1.f / kPT);
  float q2 = 0.f;
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const float dv = v[j] - mu;
    q2 = fmaf(dv, dv, q2);
  }
  q2 += __shfl_xor(q2, 1);
  const float rs = 1.f / sqrtf(q2 * (1.f / kPT) + eps);
#pragma unroll
  for (int j = 0; j < 64; ++j) {
    const int col = 64 * half + j;
    v[j] = (v[j] - mu) * rs * gamma[col] + beta[col];
  }
  // the rotary part (rope_dim <= 64) lies in the first half: each pair (j, j + rope_dim / 2)
  // belongs to the half-0 thread of the row
  if (row >= n) return;
  if (RD > 0 && half == 0) {
    constexpr int hr = RD / 2;
    const int64_t p = pos[row];
#pragma unroll
    for (int j = 0; j < hr; ++j) {
      float cs, sn;
      rope_angle(p, turns.f[j], &cs, &sn);
      const float a = v[j], b = v[j + hr];
      v[j] = a * cs - b * sn;
      v[j + hr] = a * sn + b * cs;
    }
  }
  uint16_t* dst = k_idx + row * kPT + 64 * half;
#pragma unroll
  for (int j = 0; j < 64; j += 8) {
    const uint4 pk = make_uint4(pack_bf16x2(v[j], v[j + 1]), pack_bf16x2(v[j + 2], v[j + 3]),
                                pack_bf16x2(v[j + 4], v[j + 5]), pack_bf16x2(v[j + 6], v[j + 7]));
    *reinterpret_cast<uint4*>(dst + j) = pk;
  }
}

// Row copy: rows[b] (row_bytes each) to cache + dst_row[b] * row_bytes.  A workgroup per
// new row; 16-byte accesses when the row size and both addresses allow, else bytes.  A
// destination outside [0, cache_rows) is skipped (nothing is written for that row).
__global__ __launch_bounds__(256) void cache_append_kernel(uint8_t* __restrict__ cache, int64_t cache_rows,
                                                           const int64_t* __restrict__ dst_row,
                                                           const uint8_t* __restrict__ rows, int64_t row_bytes,
                                                           bool vec) {
  const int64_t b = blockIdx.x;
  const int64_t d = dst_row[b];
  if (d < 0 || d >= cache_rows) return;
  uint8_t* dst = cache + d * row_bytes;
  const uint8_t* src = rows + b * row_bytes;
  if (vec) {
    for (int64_t j = threadIdx.x; j < row_bytes / 16; j += 256)
      reinterpret_cast<uint4*>(dst)[j] = reinterpret_cast<const uint4*>(src)[j];
  } else {
    for (int64_t j = threadIdx.x; j < row_bytes; j += 256) dst[j] = src[j];
  }
}

}  // namespace

hipError_t launch_indexer_project(const ProjectArgs& a, hipStream_t st) {
  const dim3 gq((unsigned)((a.n + kPT - 1) / kPT), (unsigned)a.H);
  const dim3 gk((unsigned)((a.n + kPT - 1) / kPT), 2u);
  RopeTurns turns = {};
  for (int j = 0; 2 * j < a.rope_dim && j < 32; ++j)
    turns.f[j] = pow((double)a.rope_base, -2.0 * j / a.rope_dim) / (2.0 * M_PI);
  const float wscale = (float)(1.0 / sqrt((double)a.H) / sqrt((double)kPT));
#define DSA_PROJ(RDv)                                                                                        \
  if (a.rope_dim == RDv) {                                                                                   \
    hipLaunchKernelGGL(proj_q_kernel<RDv>, gq, dim3(256), 0, st, a.q_lat, a.n, a.r, a.wq, a.H, a.pos, turns,   \
                       a.q_idx);                                                                             \
    hipError_t e = hipGetLastError();                                                                        \
    if (e != hipSuccess) return e;                                                                           \
    hipLaunchKernelGGL(proj_kw_kernel<RDv>, gk, dim3(256), 0, st, a.h, a.n, a.hidden, a.wk, a.gamma, a.beta, \
                       a.eps, a.ww, a.H, wscale, a.pos, turns, a.k_idx, a.w);                                  \
    return hipGetLastError();                                                                                \
  }
  DSA_PROJ(0) DSA_PROJ(32) DSA_PROJ(64)
#undef DSA_PROJ
  return hipErrorInvalidValue;
}

hipError_t launch_cache_append(void* cache, int64_t cache_rows, const int64_t* dst_row, const void* rows,
                               int64_t n_rows, int64_t row_bytes, hipStream_t st) {
  const bool vec = row_bytes % 16 == 0 && ((uintptr_t)cache & 15u) == 0 && ((uintptr_t)rows & 15u) == 0;
  hipLaunchKernelGGL(cache_append_kernel, dim3((unsigned)n_rows), dim3(256), 0, st, (uint8_t*)cache, cache_rows,
                     dst_row, (const uint8_t*)rows, row_bytes, vec);
  return hipGetLastError();
}

}  // namespace dsa
