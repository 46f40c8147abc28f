// KV compression into blocks for compressed sparse attention (DeepSeek-V4 CSA).
//
// Jerry's Blog, "注意力机制中的 Index：从位置下标到预算检索", §5.1: every m tokens become one compressed entry by a
// gated pooling over an overlapping window.  Entry i pools the a-half rows m i .. m i + m - 1
// (values C^a, gate logits Z^a + B^a) together with the b-half rows m (i-1) .. m i - 1
// (values C^b, gate logits Z^b + B^b); the gate is a softmax along the row axis taken
// separately for every feature column.  Entry 0 has no b-half (its window would start
// before the first token) and pools the a-half alone.
//
// The work is elementwise over feature columns and reads every input row once (a-half
// rows by one entry, b-half rows by the next), so the kernel is HBM-bound: one thread
// per (entry, 8 consecutive columns) with 16-byte loads, and a running (online) softmax
// so nothing but the 8 columns' max / sum / weighted sum is held.
#include "dsa_device.h"
#include "launch.h"

namespace dsa {
namespace {

constexpr int kCsaThreads = 256;

struct Pool8 {
  float mx[8], sum[8], acc[8];
};

__device__ __forceinline__ void pool_row(Pool8& p, const uint16_t* z, const uint16_t* v, const float* bias) {
  const i32x4 zr = *reinterpret_cast<const i32x4*>(z);
  const i32x4 vr = *reinterpret_cast<const i32x4*>(v);
  const f32x4 b0 = *reinterpret_cast<const f32x4*>(bias);
  const f32x4 b1 = *reinterpret_cast<const f32x4*>(bias + 4);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t zw = (uint32_t)zr[e >> 1], vw = (uint32_t)vr[e >> 1];
    const float zf = __uint_as_float((e & 1) ? (zw & 0xFFFF0000u) : (zw << 16));
    const float vf = __uint_as_float((e & 1) ? (vw & 0xFFFF0000u) : (vw << 16));
    const float x = zf + (e < 4 ? b0[e & 3] : b1[e & 3]);
    const float m = fmaxf(p.mx[e], x);
    const float a = __expf(p.mx[e] - m), w = __expf(x - m);
    p.sum[e] = fmaf(p.sum[e], a, w);
    p.acc[e] = fmaf(p.acc[e], a, w * vf);
    p.mx[e] = m;
  }
}

template <bool BF16_OUT>
__global__ __launch_bounds__(kCsaThreads) void csa_compress_kernel(
    const uint16_t* __restrict__ ca, const uint16_t* __restrict__ cb, const uint16_t* __restrict__ za,
    const uint16_t* __restrict__ zb, const float* __restrict__ ba, const float* __restrict__ bb, int c, int m,
    int64_t block0, int64_t n_out, void* __restrict__ out) {
  const int cg = c >> 3;
  const int64_t gid = (int64_t)blockIdx.x * kCsaThreads + threadIdx.x;
  if (gid >= n_out * cg) return;
  const int64_t o = gid / cg;
  const int col = (int)(gid - o * cg) * 8;
  const int64_t blk = block0 + o;
  Pool8 p;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    p.mx[e] = -INFINITY;
    p.sum[e] = 0.f;
    p.acc[e] = 0.f;
  }
  // first row: mx = -inf gives a = exp(-inf) = 0 and w = exp(0) = 1
  const int64_t ra = blk * m;
  for (int j = 0; j < m; ++j)
    pool_row(p, za + (ra + j) * c + col, ca + (ra + j) * c + col, ba + (int64_t)j * c + col);
  if (blk > 0) {
    const int64_t rb = ra - m;
    for (int j = 0; j < m; ++j)
      pool_row(p, zb + (rb + j) * c + col, cb + (rb + j) * c + col, bb + (int64_t)j * c + col);
  }
  float r[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = p.acc[e] / p.sum[e];
  if constexpr (BF16_OUT) {
    uint16_t* dst = (uint16_t*)out + o * c + col;
    *reinterpret_cast<i32x4*>(dst) = i32x4{(int)pack_bf16x2(r[0], r[1]), (int)pack_bf16x2(r[2], r[3]),
                                           (int)pack_bf16x2(r[4], r[5]), (int)pack_bf16x2(r[6], r[7])};
  } else {
    float* dst = (float*)out + o * c + col;
    *reinterpret_cast<f32x4*>(dst) = f32x4{r[0], r[1], r[2], r[3]};
    *reinterpret_cast<f32x4*>(dst + 4) = f32x4{r[4], r[5], r[6], r[7]};
  }
}

}  // namespace

hipError_t launch_csa_compress(const CsaArgs& a, hipStream_t st) {
  const int64_t n_out = a.n / a.m - a.block0;
  if (n_out <= 0) return hipSuccess;
  const int64_t threads = n_out * (a.c / 8);
  dim3 grid((unsigned)((threads + kCsaThreads - 1) / kCsaThreads));
  if (a.out_dtype == DSA_BF16)
    hipLaunchKernelGGL(csa_compress_kernel<true>, grid, dim3(kCsaThreads), 0, st, a.ca, a.cb, a.za, a.zb, a.ba,
                       a.bb, a.c, a.m, a.block0, n_out, a.out);
  else
    hipLaunchKernelGGL(csa_compress_kernel<false>, grid, dim3(kCsaThreads), 0, st, a.ca, a.cb, a.za, a.zb, a.ba,
                       a.bb, a.c, a.m, a.block0, n_out, a.out);
  return hipGetLastError();
}

}  // namespace dsa
