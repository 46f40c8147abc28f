// Sparse MLA attention over the selected latent rows.
//
// [IDX] §2: alpha_hat = softmax over S_t only, o_t = sum alpha_hat v_s; §4: DSA reads
// only the MLA latent rows c_s, s in S_t, and each latent row is shared by every
// query head (MQA), so one gathered row serves all n_h heads of the query.
// Here key = c[s, :576], value = c[s, :512], and the score is scale * q . key.
//
// One workgroup per query row (prefill) or per (row, split of the index list)
// (decode, followed by a combine kernel).  Each wave owns 16*HG heads (HG = 1).
// Per block of 32 selected rows:
//   gather  : 32 latent rows -> LDS, row-major (keys for QK) and transposed
//             (first 512 columns, values for PV), invalid slots read as zeros;
//   QK      : S^T[key][head] = K . Q^T with v_mfma_f32_16x16x32_bf16, A = K rows
//             from LDS, B = the wave's Q slice held in registers for the whole row;
//             the output puts one head per lane, keys in registers;
//   softmax : online, in the exp2 domain; the running max is only raised when a
//             block exceeds it by more than 2^8 (bounded growth of p), so O is
//             rescaled rarely; p is rounded to bf16 once and both O and the
//             normaliser use the rounded value;
//   PV      : O[head][v] += P . V with P (bf16) as the A operand straight from the
//             QK registers and V^T rows from LDS as the B operand; the key order
//             inside the MFMA's K slots is the same permutation for both operands.
#include <type_traits>

#include "dsa_device.h"
#include "launch.h"

namespace dsa {

constexpr int kDqk = 576;
constexpr int kDv = 512;
constexpr int kBlk = 32;                 // selected rows per block
constexpr int kKsStride = kDqk + 8;      // bf16 elements per LDS key row (pad: conflict-free b128 reads)
constexpr int kVtStride = kBlk + 4;      // bf16 elements per LDS V^T row
constexpr float kLazy = 8.0f;            // log2-domain slack before the running max moves

struct AttnSmem {
  uint16_t ks[kBlk * kKsStride];
  uint16_t vt[kDv * kVtStride];
  int valid[kBlk];
};

template <int HG>
__global__ __launch_bounds__(512) void sparse_attn_kernel(const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ latent,
                                                          const int32_t* __restrict__ idx, int n_h, int k,
                                                          float scale_log2, dsa_seqs seqs, int64_t n_q, int splits,
                                                          float* __restrict__ out_f32, uint16_t* __restrict__ out_bf16,
                                                          float* __restrict__ part_o, float* __restrict__ part_ml) {
  __shared__ AttnSmem sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x;
  const int64_t i = blockIdx.x / splits;
  const int split = blockIdx.x % splits;
  if (i >= n_q) return;
  const int b = seq_of_row(seqs, i);
  const int64_t p = row_last(seqs, b, i);
  const int64_t krow0 = seqs.k_start[b];
  const int c = lane & 15, g = lane >> 4;
  const int head0 = 16 * HG * wave;

  const int nblk_total = (k + kBlk - 1) / kBlk;
  const int per = (nblk_total + splits - 1) / splits;
  const int blk_lo = split * per;
  const int blk_hi = min(nblk_total, blk_lo + per);

  // Q slice: B operand of the QK MFMA, lane -> head (16hg + c), K slice 8g within each 32-column step.
  i32x4 qf[HG][kDqk / 32];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const uint16_t* qrow = q + (i * n_h + head0 + 16 * hg + c) * kDqk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) qf[hg][ks] = *reinterpret_cast<const i32x4*>(qrow + 32 * ks);
  }

  f32x4 o[HG][kDv / 16];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg)
#pragma unroll
    for (int vt = 0; vt < kDv / 16; ++vt) o[hg][vt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[HG], l[HG];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    m[hg] = -INFINITY;
    l[hg] = 0.f;
  }

  const int32_t* irow = idx + i * (int64_t)k;
  for (int blk = blk_lo; blk < blk_hi; ++blk) {
    // ---- gather 32 latent rows (row pairs so V^T can be written as packed pairs)
    for (int task = tid; task < (kBlk / 2) * (kDqk / 8); task += nthreads) {
      const int rp = task / (kDqk / 8), ch = task % (kDqk / 8);
      i32x4 v[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int slot = blk * kBlk + 2 * rp + e;
        const int32_t s = slot < k ? irow[slot] : -1;
        const bool ok = s >= 0 && s <= p;
        if (ch == 0) sm.valid[2 * rp + e] = ok;
        v[e] = ok ? *reinterpret_cast<const i32x4*>(latent + (krow0 + s) * kDqk + 8 * ch) : i32x4{0, 0, 0, 0};
        *reinterpret_cast<i32x4*>(&sm.ks[(2 * rp + e) * kKsStride + 8 * ch]) = v[e];
      }
      if (ch < kDv / 8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t x0 = (uint32_t)v[0][e], x1 = (uint32_t)v[1][e];
          // columns 8ch+2e and 8ch+2e+1 of rows 2rp and 2rp+1
          *reinterpret_cast<uint32_t*>(&sm.vt[(8 * ch + 2 * e) * kVtStride + 2 * rp]) = (x0 & 0xFFFFu) | (x1 << 16);
          *reinterpret_cast<uint32_t*>(&sm.vt[(8 * ch + 2 * e + 1) * kVtStride + 2 * rp]) = (x0 >> 16) | (x1 & 0xFFFF0000u);
        }
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for two 16-key tiles
    f32x4 st[HG][2];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) st[hg][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDqk / 32; ++ks) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const i32x4 kf = *reinterpret_cast<const i32x4*>(&sm.ks[(16 * kt + c) * kKsStride + 32 * ks + 8 * g]);
#pragma unroll
        for (int hg = 0; hg < HG; ++hg) st[hg][kt] = mfma_bf16_16x16x32(kf, qf[hg][ks], st[hg][kt]);
      }
    }

    // ---- online softmax; lane holds head (16hg + c), keys 16kt + 4g + r
    bool okr[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) okr[kt][r] = sm.valid[16 * kt + 4 * g + r] != 0;
    i32x4 pf[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      float x[2][4];
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[kt][r] = okr[kt][r] ? st[hg][kt][r] * scale_log2 : -INFINITY;
          bmax = fmaxf(bmax, x[kt][r]);
        }
      bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
      bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
      const bool raise = bmax > m[hg] + kLazy;
      if (__any(raise)) {
        const float mnew = fmaxf(m[hg], bmax);
        const float alpha = (m[hg] == -INFINITY) ? 0.f : exp2f(m[hg] - mnew);
        m[hg] = mnew;
        l[hg] *= alpha;
        // alpha for the O layout: lane holds heads 4g + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float ar = __shfl(alpha, 4 * g + r);
#pragma unroll
          for (int vt = 0; vt < kDv / 16; ++vt) o[hg][vt][r] *= ar;
        }
      }
      // p enters the PV product as bf16; the normaliser sums the same rounded values,
      // so the rounding of the weights cancels in O / l (a lone dominant key is exact).
      uint32_t pb[2][4];
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float pr = (m[hg] == -INFINITY) ? 0.f : exp2f(x[kt][r] - m[hg]);
          pb[kt][r] = f32_to_bf16_bits(pr);
          psum += __uint_as_float(pb[kt][r] << 16);
        }
      l[hg] += psum;
      pf[hg] = i32x4{(int)(pb[0][0] | (pb[0][1] << 16)), (int)(pb[0][2] | (pb[0][3] << 16)),
                     (int)(pb[1][0] | (pb[1][1] << 16)), (int)(pb[1][2] | (pb[1][3] << 16))};
    }

    // ---- O += P V ; B operand lane -> value column 16vt + c, K slots {4g..4g+3, 16+4g..16+4g+3}
#pragma unroll
    for (int vt = 0; vt < kDv / 16; ++vt) {
      __builtin_amdgcn_sched_barrier(0);
      const uint16_t* vrow = &sm.vt[(16 * vt + c) * kVtStride];
      const uint64_t lo = *reinterpret_cast<const uint64_t*>(vrow + 4 * g);
      const uint64_t hi = *reinterpret_cast<const uint64_t*>(vrow + 16 + 4 * g);
      const i32x4 vf = i32x4{(int)(uint32_t)lo, (int)(uint32_t)(lo >> 32), (int)(uint32_t)hi, (int)(uint32_t)(hi >> 32)};
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) o[hg][vt] = mfma_bf16_16x16x32(pf[hg], vf, o[hg][vt]);
    }
    __syncthreads();
  }

  // ---- finish: per-head sums across the four lane groups
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    float lt = l[hg];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (splits == 1) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ir = __shfl(inv, 4 * g + r);
        const int64_t orow = (i * n_h + head0 + 16 * hg + 4 * g + r) * kDv;
#pragma unroll
        for (int vt = 0; vt < kDv / 16; ++vt) {
          const float val = o[hg][vt][r] * ir;
          if (out_f32)
            out_f32[orow + 16 * vt + c] = val;
          else
            out_bf16[orow + 16 * vt + c] = (uint16_t)f32_to_bf16_bits(val);
        }
      }
    } else {
      const int64_t pbase = (i * splits + split) * (int64_t)n_h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t orow = (pbase + head0 + 16 * hg + 4 * g + r) * kDv;
#pragma unroll
        for (int vt = 0; vt < kDv / 16; ++vt) part_o[orow + 16 * vt + c] = o[hg][vt][r];
      }
      if (g == 0) {
        part_ml[(pbase + head0 + 16 * hg + c) * 2 + 0] = m[hg];
        part_ml[(pbase + head0 + 16 * hg + c) * 2 + 1] = lt;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Paired-wave variant (n_h a multiple of 32, k <= kIdxMax).
//
// A pair of waves owns 16*HG heads.  QK is split over the 576 latent columns in
// alternating 32-column steps (wave vh takes steps 2 ks + vh), so each wave keeps
// only half of its heads' q in registers; the two partial score tiles are summed
// through LDS, after which both waves hold identical scores and run the same
// softmax.  PV is split over alternating 16-column value tiles (wave vh takes
// tiles 2 vt + vh), so each wave's O accumulator is 16*HG x 256.
// Latent rows are gathered with direct global->LDS copies issued from asm (no
// registers), one block ahead of the block being computed, into a row-major tile;
// the copies are awaited by an explicit vmcnt wait before the block barrier.  V is
// read back column-wise with the LDS transpose read, so no transposed copy is
// written.
// ----------------------------------------------------------------------------
// LDS tile of one block: 9 column groups of 128 bytes (8 granules of 16 B) x 32
// rows; inside a row the 8 granules are XOR-swizzled by (row & 7), so 16 rows
// read at one column land on distinct banks (pairs of rows 8 apart share).
constexpr int kCg = kDqk / 64;                    // 9 column groups
constexpr int kTileBytes = kCg * kBlk * 128;      // 36864
constexpr int kTileIns = kTileBytes / 1024;       // 36 64-lane x 16-byte copies per block
constexpr int kNBuf = 2;
constexpr int kIdxMax = 2048;
constexpr int kMaxWaves = 8;
// Prefetch depths of the paired kernel's LDS reads (QK: 32-column steps; PV: column
// groups).  Eight waves (two per SIMD, 256 registers each, q and O taking 200) have room
// for two steps (three K steps spill and take 30% longer); four waves (one per SIMD) keep
// more reads in flight.
template <int NW> constexpr int pf_k() { return NW >= 8 ? 2 : 3; }
template <int NW> constexpr int pf_v() { return NW >= 8 ? 2 : 2; }

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef v4i16 __attribute__((address_space(3))) lds_v4i16;

template <int HG, int NW>
struct PairSmem {
  uint8_t tile[kNBuf][kTileBytes];
  f32x4 xs[NW][2 * HG][64];     // partial score exchange, [wave][register quad][lane]
  int idx[kIdxMax];             // the split's selected positions (-1 = skip)
  float bias[kIdxMax];          // 0 for a usable slot, -inf for a skipped one
};


// LDS transpose read (4 x b16).  The gather into LDS is issued from asm, so the
// compiler, which does not see it, schedules these reads with no wait for it.
__device__ __forceinline__ v4i16 tr16(const uint8_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(const __attribute__((address_space(3))) void*)p);
}
__device__ __forceinline__ i32x4 pack_tr4(v4i16 lo, v4i16 hi) {
  const uint64_t a = __builtin_bit_cast(uint64_t, lo), b = __builtin_bit_cast(uint64_t, hi);
  return i32x4{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)(uint32_t)b, (int)(uint32_t)(b >> 32)};
}


__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return (uint32_t)((chunk >> 3) * (kBlk * 128) + row * 128 + 16 * ((chunk & 7) ^ (row & 7)));
}

// Grid order: rows in blocks of 8; workgroup b takes row 8 rb + b % 8 of row block rb,
// head group hg and split sp with b = ((sp * n_rb + rb) * hgroups + hg) * 8 + b % 8.
// Workgroups go round-robin over the 8 XCDs, so all head groups (and, for one row
// block, all splits) of a row run on one XCD close together in time and re-read the
// row's gathered latent rows from that XCD's L2.
template <int HG, int NW>
__global__ __launch_bounds__(64 * NW) void sparse_attn_pair_kernel(const uint16_t* __restrict__ q,
                                                                   const uint16_t* __restrict__ latent,
                                                                   const int32_t* __restrict__ idx, int n_h, int k,
                                                                   float scale_log2, dsa_seqs seqs, int64_t n_q,
                                                                   int hgroups, int splits,
                                                                   float* __restrict__ out_f32,
                                                                   uint16_t* __restrict__ out_bf16,
                                                                   float* __restrict__ part_o,
                                                                   float* __restrict__ part_ml) {
  __shared__ PairSmem<HG, NW> sm;
  // the wave index is uniform: kept in a scalar register, so are the values derived from it
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int nwaves = NW;
  const int pair = wave >> 1, vh = wave & 1;
  const uint32_t n_rb = (uint32_t)((n_q + 7) / 8);  // the grid is 8 n_rb hgroups splits < 2^32 workgroups
  const uint32_t rest = blockIdx.x >> 3;
  const int hgi = (int)(rest % (uint32_t)hgroups);
  const uint32_t rs = rest / (uint32_t)hgroups;
  const int64_t i = (int64_t)(rs % n_rb) * 8 + (blockIdx.x & 7);
  const int split = (int)(rs / n_rb);
  if (i >= n_q || split >= splits) return;
  const int b = seq_of_row(seqs, i);
  const int64_t p = row_last(seqs, b, i);
  const uint16_t* lat = latent + seqs.k_start[b] * kDqk;
  const int c = lane & 15, g = lane >> 4;
  const int head0 = 8 * HG * NW * hgi + 16 * HG * pair;

  const int nblk_total = (k + kBlk - 1) / kBlk;
  const int per = (nblk_total + splits - 1) / splits;
  const int blk_lo = min(nblk_total, split * per);
  const int blk_hi = min(nblk_total, blk_lo + per);

  // this split's part of the row's index list, invisible or out-of-range entries marked -1;
  // the entries are loaded (clamped positions, no load in a branch), then q, then staged
  // in LDS, so one wait for memory covers them all
  const int32_t* irow = idx + i * (int64_t)k;
  constexpr int kStage = kIdxMax / (64 * NW);
  const int j_lo = blk_lo * kBlk, j_hi = blk_hi * kBlk;
  int32_t sv[kStage];
#pragma unroll
  for (int u = 0; u < kStage; ++u)
    if (j_lo + 64 * NW * u < j_hi) sv[u] = irow[min(j_lo + tid + 64 * NW * u, k - 1)];

  // q slice: B operand of QK; lane -> head (16hg + c); this wave takes the 32-column
  // steps 2 ks + vh (columns 64 ks + 32 vh + 8 g .. +8)
  i32x4 qf[HG][9];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    const uint16_t* qrow = q + (i * n_h + head0 + 16 * hg + c) * kDqk + 32 * vh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) qf[hg][ks] = *reinterpret_cast<const i32x4*>(qrow + 64 * ks);
  }
#pragma unroll
  for (int u = 0; u < kStage; ++u) {
    const int j = j_lo + tid + 64 * NW * u;
    if (j < j_hi) {
      const int32_t s = j < k ? sv[u] : -1;
      const bool ok = s >= 0 && s <= p;
      sm.idx[j] = ok ? s : -1;
      sm.bias[j] = ok ? 0.f : -INFINITY;
    }
  }
  f32x4 o[HG][16];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg)
#pragma unroll
    for (int vt = 0; vt < 16; ++vt) o[hg][vt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m[HG], l[HG];
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    m[hg] = -INFINITY;
    l[hg] = 0.f;
  }
  __syncthreads();

  // direct global->LDS gather of block blk into buffer bi (invalid slots load row 0
  // of the sequence, which always exists; their scores are masked below)
  // copy j fills column group j/4, rows 8(j%4) .. +8; lane l lands in row
  // 8(j%4) + l/8 at swizzled position l%8, i.e. it fetches granule (l%8) ^ (row & 7)
  const int lrow = lane >> 3, lpos = lane & 7;
  // NW % 4 == 0: copies j = wave + NW m all fill rows 8 (wave % 4) .. +8, so one index
  // read and one byte offset serve all of a wave's copies of a block; copy m starts NW/4
  // column groups (16 NW elements) further along the row, which is the instruction's
  // immediate offset (32 NW m bytes).  The offset counts from the sequence's first latent
  // row (rows * 1152 B < 2^32 is checked on the host).
  constexpr int kWaveCopies = (kTileIns + NW - 1) / NW;
  auto gather_off = [&](int blk) -> uint32_t {
    const int ln = lane_id_here();
    const int r = 8 * (wave & 3) + (ln >> 3);
    const int s = sm.idx[blk * kBlk + r];
    return __umul24((uint32_t)(s >= 0 ? s : 0), 2u * kDqk) +
           (uint32_t)(16 * (8 * (wave >> 2) + ((ln & 7) ^ (r & 7))));
  };
  auto gather_copy = [&](auto mc, uint32_t off, int bi) {
    constexpr int M = decltype(mc)::value;
    if (kTileIns % NW == 0 || wave + NW * M < kTileIns)
      dma16_s<32 * NW * M>(lat, off, lds_u32(&sm.tile[bi][1024 * (wave + NW * M)]));
  };
  auto gather = [&](int blk, int bi) {
    if constexpr (NW % 4 == 0) {
      const uint32_t off = gather_off(blk);
      static_for<0, kWaveCopies>([&](auto mc) { gather_copy(mc, off, bi); });
    } else {
      for (int j = wave; j < kTileIns; j += nwaves) {
        const int r = 8 * (j & 3) + lrow;
        const int chunk = 8 * (j >> 2) + (lpos ^ (r & 7));
        const int s = sm.idx[blk * kBlk + r];
        const uint16_t* src = lat + (int64_t)(s >= 0 ? s : 0) * kDqk + 8 * chunk;
        dma16(src, lds_u32(&sm.tile[bi][1024 * j]));
      }
    }
  };

  if (blk_lo < blk_hi) gather(blk_lo, 0);
  for (int blk = blk_lo; blk < blk_hi; ++blk) {
    const int bi = (blk - blk_lo) & 1;
    // This wave's copies of block blk landed (an explicit wait: the compiler does not
    // reliably wait for direct-to-LDS copies at a barrier); after the barrier every
    // wave's have, and buffer bi^1 (block blk-1) is no longer read.
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    // The next block's gather: with NW % 4 == 0 its copies are spread over the QK steps
    // below (issued together they stall the wave until the memory pipeline takes them).
    const bool more = blk + 1 < blk_hi;
    uint32_t goff = 0;
    if constexpr (NW % 4 == 0) {
      if (more) goff = gather_off(blk + 1);
    } else {
      if (more) gather(blk + 1, bi ^ 1);
    }
    const uint8_t* tile = sm.tile[bi];

    // ---- partial S^T over this wave's 288 columns, for two 16-key tiles
    f32x4 st[HG][2];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) st[hg][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // K fragment of step ks: column group ks, granule 4 vh + g of row 16 kt + c.  The
    // fragments are read kPfK steps ahead of their MFMAs (scheduling barriers keep the
    // order), so several LDS reads are in flight while the matrix core works.
    constexpr int kPfK = pf_k<NW>();
    const uint8_t* kbase = tile + c * 128 + 16 * ((4 * vh + g) ^ (c & 7));
    i32x4 kf[kPfK + 1][2];
#pragma unroll
    for (int j = 0; j < kPfK; ++j)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) kf[j][kt] = *reinterpret_cast<const i32x4*>(kbase + j * (kBlk * 128) + kt * 2048);
    // copy m of the next block's gather goes out at step ks = m * 9 / kWaveCopies
    static_for<0, 9>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NW % 4 == 0) {
        static_for<0, kWaveCopies>([&](auto mc) {
          if constexpr (decltype(mc)::value * 9 / kWaveCopies == ks)
            if (more) gather_copy(mc, goff, bi ^ 1);
        });
      }
      if (ks + kPfK < 9) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          kf[(ks + kPfK) % (kPfK + 1)][kt] =
              *reinterpret_cast<const i32x4*>(kbase + (ks + kPfK) * (kBlk * 128) + kt * 2048);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int hg = 0; hg < HG; ++hg)
          st[hg][kt] = mfma_bf16_16x16x32(kf[ks % (kPfK + 1)][kt], qf[hg][ks], st[hg][kt]);
    });
    __builtin_amdgcn_sched_barrier(0);
    // ---- exchange partial scores with the partner wave
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) sm.xs[wave][2 * hg + kt][lane] = st[hg][kt];
    lds_barrier();  // waits for LDS traffic only, not for the next block's gather
#pragma unroll
    for (int hg = 0; hg < HG; ++hg)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) st[hg][kt] += sm.xs[wave ^ 1][2 * hg + kt][lane];

    // ---- online softmax (identical in both waves of the pair); skipped slots get
    // -inf through an additive bias
    f32x4 bias[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) bias[kt] = *reinterpret_cast<const f32x4*>(&sm.bias[blk * kBlk + 16 * kt + 4 * g]);
    i32x4 pf[HG];
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      float x[2][4];
      float bmax = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          x[kt][r] = fmaf(st[hg][kt][r], scale_log2, bias[kt][r]);
          bmax = fmaxf(bmax, x[kt][r]);
        }
      bmax = max_over_rows(bmax);
      if (__any(bmax > m[hg] + kLazy)) {
        const float mnew = fmaxf(m[hg], bmax);
        const float alpha = (m[hg] == -INFINITY) ? 0.f : exp2f(m[hg] - mnew);
        m[hg] = mnew;
        l[hg] *= alpha;
        float ar[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
        for (int vt = 0; vt < 16; ++vt)
#pragma unroll
          for (int r = 0; r < 4; ++r) o[hg][vt][r] *= ar[r];
      }
      // p = 2^(x - m) (x = -inf gives 0), rounded once to bf16 pairs; the
      // normaliser sums the rounded values (a bf16 dot product with ones)
      const float mu = (m[hg] == -INFINITY) ? 0.f : m[hg];
      const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
      float psum = 0.f;
      uint32_t pk[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int kt = e >> 1, r = 2 * (e & 1);
        const bf16x2 v = {(__bf16)__builtin_amdgcn_exp2f(x[kt][r] - mu),
                          (__bf16)__builtin_amdgcn_exp2f(x[kt][r + 1] - mu)};
        pk[e] = __builtin_bit_cast(uint32_t, v);
        psum = __builtin_amdgcn_fdot2_f32_bf16(v, ones, psum, false);
      }
      l[hg] += psum;
      pf[hg] = i32x4{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
    }

    // ---- O += P V over this wave's value tiles 2 vt + vh (columns 32 vt + 16 vh + ..).
    // B operand via transpose reads: in 16-lane group g, lane a + 4j reads 4 columns
    // (.. + 4a) of key row 4g + j (K slots 0-3) and of row 16 + 4g + j (slots 4-7).
    const int ta = c & 3, tj = c >> 2;
    const int r0 = 4 * g + tj;
    const uint8_t* vb0 = tile + r0 * 128 + 16 * ((2 * vh + (ta >> 1)) ^ (r0 & 7)) + 8 * (ta & 1);
    const uint8_t* vb1 = tile + r0 * 128 + 16 * ((4 + 2 * vh + (ta >> 1)) ^ (r0 & 7)) + 8 * (ta & 1);
    // tiles vt (even: base 0) and vt + 1 (odd: base 1) share column group vt / 2; the
    // transpose reads run kPfV column groups ahead of their MFMAs
    constexpr int kPfV = pf_v<NW>();
    v4i16 vr[kPfV + 1][4];
    auto vread = [&](int it, v4i16 (&d)[4]) {
      const int cgo = it * (kBlk * 128);
      d[0] = tr16(vb0 + cgo);
      d[1] = tr16(vb0 + cgo + 2048);
      d[2] = tr16(vb1 + cgo);
      d[3] = tr16(vb1 + cgo + 2048);
    };
#pragma unroll
    for (int j = 0; j < kPfV; ++j) vread(j, vr[j]);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      __builtin_amdgcn_sched_barrier(0);
      if (it + kPfV < 8) vread(it + kPfV, vr[(it + kPfV) % (kPfV + 1)]);
      const v4i16 (&cur)[4] = vr[it % (kPfV + 1)];
      const i32x4 vfe = pack_tr4(cur[0], cur[1]);
      const i32x4 vfo = pack_tr4(cur[2], cur[3]);
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        o[hg][2 * it] = mfma_bf16_16x16x32(pf[hg], vfe, o[hg][2 * it]);
        o[hg][2 * it + 1] = mfma_bf16_16x16x32(pf[hg], vfo, o[hg][2 * it + 1]);
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }

  // ---- finish
#pragma unroll
  for (int hg = 0; hg < HG; ++hg) {
    float lt = l[hg];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    if (splits == 1) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ir = __shfl(inv, 4 * g + r);
        const int64_t orow = (i * n_h + head0 + 16 * hg + 4 * g + r) * kDv + 16 * vh + c;
#pragma unroll
        for (int vt = 0; vt < 16; ++vt) {
          const float val = o[hg][vt][r] * ir;
          if (out_f32)
            out_f32[orow + 32 * vt] = val;
          else
            out_bf16[orow + 32 * vt] = (uint16_t)f32_to_bf16_bits(val);
        }
      }
    } else {
      const int64_t pbase = (i * splits + split) * (int64_t)n_h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t orow = (pbase + head0 + 16 * hg + 4 * g + r) * kDv + 16 * vh + c;
#pragma unroll
        for (int vt = 0; vt < 16; ++vt) part_o[orow + 32 * vt] = o[hg][vt][r];
      }
      if (vh == 0 && g == 0) {
        part_ml[(pbase + head0 + 16 * hg + c) * 2 + 0] = m[hg];
        part_ml[(pbase + head0 + 16 * hg + c) * 2 + 1] = lt;
      }
    }
  }
}

// ----------------------------------------------------------------------------
// Paired-wave variant for 32 heads per pair (HG = 2), pipelined by one block.
//
// The work split of QK and PV is the one above, but the softmax is not computed twice:
// wave vh normalises only its own 16 heads and hands the other wave its bf16 P and its
// rescale factor through LDS.  PV of block j runs in the next iteration, after QK of
// block j + 1: the next block barrier orders the hand-over, the matrix core gets the QK
// and PV products back to back, and between two blocks there is one exchange barrier and
// half of the softmax.  Three tile buffers: block j (QK), block j - 1 (PV) and block
// j + 1 (gather in flight).  In registers, head group 0 is the wave's own (heads
// 16 vh ..) and group 1 its partner's.  Each O accumulator goes through the same
// operations in the same order as in the kernel above (rescale by the block's factor,
// then add its P V), so both kernels give identical results.
// With 8 waves, waves w and w + 4 share a SIMD and the first four win the issue
// arbitration, finishing QK first.  So that one group's softmax overlaps the other's
// matrix work, waves 0-3 run PV of block j - 1 before the exchange barrier and waves
// 4-7 after it (each still passes one exchange barrier per block); P and the factor are
// kept per block parity, because a wave of the second group may write its P of block j
// while its partner still reads its P of block j - 1.
template <int NW>
struct Pair2Smem {
  uint8_t tile[3][kTileBytes];
  f32x4 xs[NW][2][64];  // partial scores of the partner's head group, [wave][key tile][lane]
  i32x4 px[2][NW][64];  // a wave's bf16 P of its own heads, [block parity][wave][lane]
  float pa[2][NW][64];  // its rescale factor for that block (1 where the running max held)
  int idx[kIdxMax];
  float bias[kIdxMax];
};
static_assert(sizeof(Pair2Smem<8>) <= 160 * 1024, "LDS of one workgroup");  // exactly 160 KB at 8 waves

template <int NW>
__global__ __launch_bounds__(64 * NW) void sparse_attn_pair2_kernel(const uint16_t* __restrict__ q,
                                                                    const uint16_t* __restrict__ latent,
                                                                    const int32_t* __restrict__ idx, int n_h, int k,
                                                                    float scale_log2, dsa_seqs seqs, int64_t n_q,
                                                                    int hgroups, int splits,
                                                                    float* __restrict__ out_f32,
                                                                    uint16_t* __restrict__ out_bf16,
                                                                    float* __restrict__ part_o,
                                                                    float* __restrict__ part_ml) {
  __shared__ Pair2Smem<NW> sm;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave >> 1, vh = wave & 1;
  const bool late = NW == 8 && wave >= 4;  // runs PV after the exchange barrier
  const uint32_t n_rb = (uint32_t)((n_q + 7) / 8);  // same grid order as the kernel above
  const uint32_t rest = blockIdx.x >> 3;
  const int hgi = (int)(rest % (uint32_t)hgroups);
  const uint32_t rs = rest / (uint32_t)hgroups;
  const int64_t i = (int64_t)(rs % n_rb) * 8 + (blockIdx.x & 7);
  const int split = (int)(rs / n_rb);
  if (i >= n_q || split >= splits) return;
  const int b = seq_of_row(seqs, i);
  const int64_t p = row_last(seqs, b, i);
  const uint16_t* lat = latent + seqs.k_start[b] * kDqk;
  const int c = lane & 15, g = lane >> 4;
  const int head0 = 16 * NW * hgi + 32 * pair;
  const int hgl[2] = {vh, vh ^ 1};  // the pair's head group held as register group 0, 1

  const int nblk_total = (k + kBlk - 1) / kBlk;
  const int per = (nblk_total + splits - 1) / splits;
  const int blk_lo = min(nblk_total, split * per);
  const int blk_hi = min(nblk_total, blk_lo + per);
  const int nblk = blk_hi - blk_lo;

  // The split's index entries (at most kIdxMax, kStage per thread) are loaded from clamped
  // positions with no load in a branch, so one wait for memory covers them all before they
  // are staged in LDS; q is loaded after that (its latency overlaps the first gather's, and
  // the entries' registers are free again under the eight-wave register budget).
  const int32_t* irow = idx + i * (int64_t)k;
  constexpr int kStage = kIdxMax / (64 * NW);
  const int j_lo = blk_lo * kBlk, j_hi = blk_hi * kBlk;
  {
    int32_t sv[kStage];
#pragma unroll
    for (int u = 0; u < kStage; ++u) sv[u] = irow[min(j_lo + tid + 64 * NW * u, k - 1)];
#pragma unroll
    for (int u = 0; u < kStage; ++u) {
      const int j = j_lo + tid + 64 * NW * u;
      if (j < j_hi) {
        const int32_t s = j < k ? sv[u] : -1;
        const bool ok = s >= 0 && s <= p;
        sm.idx[j] = ok ? s : -1;
        sm.bias[j] = ok ? 0.f : -INFINITY;
      }
    }
  }

  i32x4 qf[2][9];
#pragma unroll
  for (int lg = 0; lg < 2; ++lg) {
    const uint16_t* qrow = q + (i * n_h + head0 + 16 * hgl[lg] + c) * kDqk + 32 * vh + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 9; ++ks) qf[lg][ks] = *reinterpret_cast<const i32x4*>(qrow + 64 * ks);
  }
  f32x4 o[2][16];
#pragma unroll
  for (int lg = 0; lg < 2; ++lg)
#pragma unroll
    for (int vt = 0; vt < 16; ++vt) o[lg][vt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_own = -INFINITY, l_own = 0.f;
  __syncthreads();

  // gather of block blk into buffer bi, as in the kernel above
  constexpr int kWaveCopies = (kTileIns + NW - 1) / NW;
  const int lrow = lane >> 3, lpos = lane & 7;
  auto gather_off = [&](int blk) -> uint32_t {
    const int ln = lane_id_here();
    const int r = 8 * (wave & 3) + (ln >> 3);
    const int s = sm.idx[blk * kBlk + r];
    return __umul24((uint32_t)(s >= 0 ? s : 0), 2u * kDqk) +
           (uint32_t)(16 * (8 * (wave >> 2) + ((ln & 7) ^ (r & 7))));
  };
  auto gather_copy = [&](auto mc, uint32_t off, int bi) {
    constexpr int M = decltype(mc)::value;
    if (kTileIns % NW == 0 || wave + NW * M < kTileIns)
      dma16_s<32 * NW * M>(lat, off, lds_u32(&sm.tile[bi][1024 * (wave + NW * M)]));
  };
  auto gather = [&](int blk, int bi) {
    if constexpr (NW % 4 == 0) {
      const uint32_t off = gather_off(blk);
      static_for<0, kWaveCopies>([&](auto mc) { gather_copy(mc, off, bi); });
    } else {
      for (int j = wave; j < kTileIns; j += NW) {
        const int r = 8 * (j & 3) + lrow;
        const int chunk = 8 * (j >> 2) + (lpos ^ (r & 7));
        const int s = sm.idx[blk * kBlk + r];
        const uint16_t* src = lat + (int64_t)(s >= 0 ? s : 0) * kDqk + 8 * chunk;
        dma16(src, lds_u32(&sm.tile[bi][1024 * j]));
      }
    }
  };

  // O += P V of one block for both register groups (P operands pa_[0], pa_[1]); the
  // partner's group is first rescaled by its owner's factor for that block
  auto pv_block = [&](const uint8_t* tile, int par) {
    const i32x4 pown = sm.px[par][wave][lane];
    const i32x4 ppar = sm.px[par][wave ^ 1][lane];
    const float apar = sm.pa[par][wave ^ 1][lane];
    if (__any(apar != 1.f)) {
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(apar, 4 * g + r);
#pragma unroll
      for (int vt = 0; vt < 16; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[1][vt][r] *= ar[r];
    }
    const int ta = c & 3, tj = c >> 2;
    const int r0 = 4 * g + tj;
    const uint8_t* vb0 = tile + r0 * 128 + 16 * ((2 * vh + (ta >> 1)) ^ (r0 & 7)) + 8 * (ta & 1);
    const uint8_t* vb1 = tile + r0 * 128 + 16 * ((4 + 2 * vh + (ta >> 1)) ^ (r0 & 7)) + 8 * (ta & 1);
    constexpr int kPfV = pf_v<NW>();
    v4i16 vr[kPfV + 1][4];
    auto vread = [&](int it, v4i16 (&d)[4]) {
      const int cgo = it * (kBlk * 128);
      d[0] = tr16(vb0 + cgo);
      d[1] = tr16(vb0 + cgo + 2048);
      d[2] = tr16(vb1 + cgo);
      d[3] = tr16(vb1 + cgo + 2048);
    };
#pragma unroll
    for (int j = 0; j < kPfV; ++j) vread(j, vr[j]);
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      __builtin_amdgcn_sched_barrier(0);
      if (it + kPfV < 8) vread(it + kPfV, vr[(it + kPfV) % (kPfV + 1)]);
      const v4i16 (&cur)[4] = vr[it % (kPfV + 1)];
      const i32x4 vfe = pack_tr4(cur[0], cur[1]);
      const i32x4 vfo = pack_tr4(cur[2], cur[3]);
      o[0][2 * it] = mfma_bf16_16x16x32(pown, vfe, o[0][2 * it]);
      o[0][2 * it + 1] = mfma_bf16_16x16x32(pown, vfo, o[0][2 * it + 1]);
      o[1][2 * it] = mfma_bf16_16x16x32(ppar, vfe, o[1][2 * it]);
      o[1][2 * it + 1] = mfma_bf16_16x16x32(ppar, vfo, o[1][2 * it + 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  if (nblk > 0) gather(blk_lo, 0);
  int bcur = 0;  // buffer of block j; j - 1 in (bcur + 2) % 3, j + 1 in (bcur + 1) % 3
  for (int j = 0; j < nblk; ++j) {
    const int blk = blk_lo + j;
    const int bnext = bcur == 2 ? 0 : bcur + 1;
    const int bprev = bcur == 0 ? 2 : bcur - 1;
    // block j's copies landed; every wave's P of block j - 1 is in LDS; buffer bnext
    // (block j - 2) is no longer read
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
    const bool more = j + 1 < nblk;
    uint32_t goff = 0;
    if constexpr (NW % 4 == 0) {
      if (more) goff = gather_off(blk + 1);
    } else {
      if (more) gather(blk + 1, bnext);
    }
    const uint8_t* tile = sm.tile[bcur];

    // ---- partial S^T of block j over this wave's 288 columns (both head groups)
    f32x4 st[2][2];
#pragma unroll
    for (int lg = 0; lg < 2; ++lg)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) st[lg][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int kPfK = pf_k<NW>();
    const uint8_t* kbase = tile + c * 128 + 16 * ((4 * vh + g) ^ (c & 7));
    i32x4 kf[kPfK + 1][2];
#pragma unroll
    for (int jj = 0; jj < kPfK; ++jj)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) kf[jj][kt] = *reinterpret_cast<const i32x4*>(kbase + jj * (kBlk * 128) + kt * 2048);
    static_for<0, 9>([&](auto ksc) {
      constexpr int ks = decltype(ksc)::value;
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (NW % 4 == 0) {
        static_for<0, kWaveCopies>([&](auto mc) {
          if constexpr (decltype(mc)::value * 9 / kWaveCopies == ks)
            if (more) gather_copy(mc, goff, bnext);
        });
      }
      if (ks + kPfK < 9) {
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          kf[(ks + kPfK) % (kPfK + 1)][kt] =
              *reinterpret_cast<const i32x4*>(kbase + (ks + kPfK) * (kBlk * 128) + kt * 2048);
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int lg = 0; lg < 2; ++lg)
          st[lg][kt] = mfma_bf16_16x16x32(kf[ks % (kPfK + 1)][kt], qf[lg][ks], st[lg][kt]);
    });
    __builtin_amdgcn_sched_barrier(0);
    // the partner's group: this wave's partial goes to its owner
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) sm.xs[wave][kt][lane] = st[1][kt];

    // ---- PV of block j - 1 (before or after the exchange barrier: see above)
    if (!late && j > 0) pv_block(sm.tile[bprev], (j - 1) & 1);
    lds_barrier();  // partial scores exchanged (LDS traffic only, not the gather)
    if (late && j > 0) pv_block(sm.tile[bprev], (j - 1) & 1);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) st[0][kt] += sm.xs[wave ^ 1][kt][lane];

    // ---- online softmax of the own head group (as in the kernel above)
    f32x4 bias[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) bias[kt] = *reinterpret_cast<const f32x4*>(&sm.bias[blk * kBlk + 16 * kt + 4 * g]);
    float x[2][4];
    float bmax = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        x[kt][r] = fmaf(st[0][kt][r], scale_log2, bias[kt][r]);
        bmax = fmaxf(bmax, x[kt][r]);
      }
    bmax = max_over_rows(bmax);
    float alpha = 1.f;
    if (__any(bmax > m_own + kLazy)) {
      const float mnew = fmaxf(m_own, bmax);
      alpha = (m_own == -INFINITY) ? 0.f : exp2f(m_own - mnew);
      m_own = mnew;
      l_own *= alpha;
      float ar[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) ar[r] = __shfl(alpha, 4 * g + r);
#pragma unroll
      for (int vt = 0; vt < 16; ++vt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[0][vt][r] *= ar[r];
    }
    const float mu = (m_own == -INFINITY) ? 0.f : m_own;
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
    float psum = 0.f;
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int kt = e >> 1, r = 2 * (e & 1);
      const bf16x2 v = {(__bf16)__builtin_amdgcn_exp2f(x[kt][r] - mu),
                        (__bf16)__builtin_amdgcn_exp2f(x[kt][r + 1] - mu)};
      pk[e] = __builtin_bit_cast(uint32_t, v);
      psum = __builtin_amdgcn_fdot2_f32_bf16(v, ones, psum, false);
    }
    l_own += psum;
    sm.px[j & 1][wave][lane] = i32x4{(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
    sm.pa[j & 1][wave][lane] = alpha;
    bcur = bnext;
  }
  __syncthreads();  // the last block's P of every wave is in LDS
  if (nblk > 0) pv_block(sm.tile[bcur == 0 ? 2 : bcur - 1], (nblk - 1) & 1);

  // ---- finish: the owner's normaliser (and running max) of each group
  float lt_own = l_own;
  lt_own += __shfl_xor(lt_own, 16);
  lt_own += __shfl_xor(lt_own, 32);
  sm.xs[wave][0][lane] = f32x4{lt_own, m_own, 0.f, 0.f};
  __syncthreads();
  const f32x4 mlp = sm.xs[wave ^ 1][0][lane];
  const float ltg[2] = {lt_own, mlp[0]};
#pragma unroll
  for (int lg = 0; lg < 2; ++lg) {
    const float lt = ltg[lg];
    const int hh = head0 + 16 * hgl[lg];
    if (splits == 1) {
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float ir = __shfl(inv, 4 * g + r);
        const int64_t orow = (i * n_h + hh + 4 * g + r) * kDv + 16 * vh + c;
#pragma unroll
        for (int vt = 0; vt < 16; ++vt) {
          const float val = o[lg][vt][r] * ir;
          if (out_f32)
            out_f32[orow + 32 * vt] = val;
          else
            out_bf16[orow + 32 * vt] = (uint16_t)f32_to_bf16_bits(val);
        }
      }
    } else {
      const int64_t pbase = (i * splits + split) * (int64_t)n_h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t orow = (pbase + hh + 4 * g + r) * kDv + 16 * vh + c;
#pragma unroll
        for (int vt = 0; vt < 16; ++vt) part_o[orow + 32 * vt] = o[lg][vt][r];
      }
      if (lg == 0 && g == 0) {
        part_ml[(pbase + hh + c) * 2 + 0] = m_own;
        part_ml[(pbase + hh + c) * 2 + 1] = lt;
      }
    }
  }
}

// Merge split partials: M = max m_s, L = sum l_s 2^(m_s - M), O = sum O_s 2^(m_s - M) / L.
// A wave per (row, head, half of the 512 value columns): lane l streams columns
// 256 half + 4 l .. + 4 (16-byte loads) over the splits.  The values, maxima and sums of
// eight splits are loaded before any is used, together with the maxima of the remaining
// splits, so a call with up to eight splits waits for memory once.  Splits are summed in
// order.
constexpr int kCombGroup = 8;
__global__ __launch_bounds__(256) void sparse_attn_combine_kernel(const float* __restrict__ part_o,
                                                                  const float* __restrict__ part_ml, int n_h,
                                                                  int splits, int64_t n_q, float* __restrict__ out_f32,
                                                                  uint16_t* __restrict__ out_bf16) {
  const int64_t wv = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (row, head, half)
  const int half = (int)(wv & 1);
  const int64_t rh = wv >> 1;
  const int lane = threadIdx.x & 63;
  const int64_t i = rh / n_h;
  const int h = (int)(rh % n_h);
  if (i >= n_q) return;
  const float* ml = part_ml + (i * splits * (int64_t)n_h + h) * 2;
  const int64_t mstride = (int64_t)n_h * 2;
  const float* po = part_o + (i * splits * (int64_t)n_h + h) * kDv + 256 * half + 4 * lane;
  const int64_t sstride = (int64_t)n_h * kDv;
  f32x4 v[kCombGroup];
  float ms[kCombGroup], ls[kCombGroup];
  auto load_group = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kCombGroup; ++u)
      if (s0 + u < splits) {
        v[u] = *reinterpret_cast<const f32x4*>(po + (s0 + u) * sstride);
        ms[u] = ml[(s0 + u) * mstride];
        ls[u] = ml[(s0 + u) * mstride + 1];
      }
  };
  load_group(0);
  float M = -INFINITY;
  for (int s = kCombGroup; s < splits; ++s) M = fmaxf(M, ml[s * mstride]);
#pragma unroll
  for (int u = 0; u < kCombGroup; ++u)
    if (u < splits) M = fmaxf(M, ms[u]);
  float L = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < splits; s0 += kCombGroup) {
    if (s0 > 0) load_group(s0);
#pragma unroll
    for (int u = 0; u < kCombGroup; ++u)
      if (s0 + u < splits) {
        const float wgt = ms[u] == -INFINITY ? 0.f : exp2f(ms[u] - M);
        L = fmaf(ls[u], wgt, L);
        acc += v[u] * wgt;
      }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  acc *= inv;
  const int64_t o = (i * n_h + h) * kDv + 256 * half + 4 * lane;
  if (out_f32)
    *reinterpret_cast<f32x4*>(out_f32 + o) = acc;
  else
    *reinterpret_cast<uint2*>(out_bf16 + o) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
}

// Work split of one call.  Prefill (many rows): one workgroup per row with every head.
// Few rows (decode): the heads are cut into groups of 32 (two wave pairs of 16) and the
// row's index list into splits, so that the grid has about 256 workgroups.  Each split
// writes an fp32 partial of its heads that the combine pass merges; head groups keep that
// partial small (64 KB per split and group at 32 heads) where a split over all 128 heads
// would write 256 KB, and the groups of a row re-read its latent rows from one L2.
struct AttnPlan {
  bool paired;
  int nw, hg, hgroups, splits;
};

AttnPlan attn_plan(const AttnArgs& a) {
  AttnPlan pl;
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  const int nblk = (a.k + kBlk - 1) / kBlk;
  pl.paired = (a.n_h == 32 || a.n_h == 64 || a.n_h == 128) && a.k <= kIdxMax;
  pl.splits = 1;
  pl.hgroups = 1;
  if (pl.paired) {
    pl.hg = 2;
    pl.nw = a.n_h / 16;
  } else {
    pl.hg = 1;
    pl.nw = a.n_h / 16;
  }
  if (n_q >= 512 || nblk <= 1) return pl;  // many rows: one workgroup per row with every head
  if (pl.paired) {
    pl.hg = 1;       // a pair per 16 heads, two pairs per workgroup
    pl.nw = 4;
    pl.hgroups = a.n_h / 32;
  }
  // about 256 workgroups, and at most 8 splits: past 8, a split's fixed cost in this kernel
  // outweighs the blocks it takes off each workgroup (one row of 2048 entries: 72 us as 64
  // one-block splits, 28.5 us as 16, 24 us as 8 splits of 8 blocks); 8 is also the number
  // of splits the combine reads with one wait for memory
  const int64_t per_split = n_q * pl.hgroups;
  int s = (int)((256 + per_split - 1) / per_split);
  if (s > nblk) s = nblk;
  if (s > kCombGroup) s = kCombGroup;
  pl.splits = s < 1 ? 1 : s;
  return pl;
}

int attn_splits(const AttnArgs& a) { return attn_plan(a).splits; }

size_t attn_ws_bytes(const AttnArgs& a) {
  const int s = attn_splits(a);
  if (s == 1) return 0;
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  return (size_t)n_q * s * a.n_h * (kDv + 2) * sizeof(float) + 256;
}

hipError_t launch_sparse_attn(const AttnArgs& a, void* ws, hipStream_t st) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  if (n_q == 0) return hipSuccess;
  const AttnPlan pl = attn_plan(a);
  const int splits = pl.splits;
  const float scale_log2 = a.scale * 1.4426950408889634f;
  float* out_f32 = a.out_dtype == DSA_FP32 ? (float*)a.out : nullptr;
  uint16_t* out_bf16 = a.out_dtype == DSA_BF16 ? (uint16_t*)a.out : nullptr;
  float* part_o = nullptr;
  float* part_ml = nullptr;
  if (splits > 1) {
    part_o = (float*)ws;
    part_ml = part_o + (size_t)n_q * splits * a.n_h * kDv;
  }
  // the paired kernel takes rows in blocks of 8 (see its grid order), the other one row each
  const int64_t rows_grid = pl.paired ? (n_q + 7) / 8 * 8 : n_q;
  dim3 grid((unsigned)(rows_grid * pl.hgroups * splits));
  float* of = splits == 1 ? out_f32 : nullptr;
  uint16_t* ob = splits == 1 ? out_bf16 : nullptr;
  if (pl.paired) {
#define DSA_PAIR(HGv, NWv)                                                                                     \
  hipLaunchKernelGGL((sparse_attn_pair_kernel<HGv, NWv>), grid, dim3(64 * NWv), 0, st, a.q, a.latent, a.idx, \
                     a.n_h, a.k, scale_log2, a.seqs, n_q, pl.hgroups, splits, of, ob, part_o, part_ml)
#define DSA_PAIR2(NWv)                                                                                        \
  hipLaunchKernelGGL((sparse_attn_pair2_kernel<NWv>), grid, dim3(64 * NWv), 0, st, a.q, a.latent, a.idx, a.n_h, \
                     a.k, scale_log2, a.seqs, n_q, pl.hgroups, splits, of, ob, part_o, part_ml)
    if (pl.hg == 1 && pl.nw == 4)
      DSA_PAIR(1, 4);
    else if (pl.nw == 2)
      DSA_PAIR2(2);
    else if (pl.nw == 4)
      DSA_PAIR2(4);
    else
      DSA_PAIR2(8);
#undef DSA_PAIR
#undef DSA_PAIR2
  } else {
    // 16 heads per wave: the Q slice (72 VGPRs) and the O accumulator (128) stay
    // resident with two waves per SIMD and no spills.
    hipLaunchKernelGGL(sparse_attn_kernel<1>, grid, dim3(64 * pl.nw), 0, st, a.q, a.latent, a.idx, a.n_h, a.k,
                       scale_log2, a.seqs, n_q, splits, of, ob, part_o, part_ml);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || splits == 1) return e;
  hipLaunchKernelGGL(sparse_attn_combine_kernel, dim3((unsigned)((2 * n_q * a.n_h + 3) / 4)), dim3(256), 0, st, part_o,
                     part_ml, a.n_h, splits, n_q, out_f32, out_bf16);
  return hipGetLastError();
}

}  // namespace dsa
