// Fused lightning indexer + streaming top-k for prefill (one sequence, many queries).
//
// Score ([IDX] §4 lightning-indexer equation) I[t,s] = sum_j w[t,j] ReLU(q_idx[t,j,:] . k_idx[s,:])
// for the visible keys s <= t, and S_t = the k best (score desc, position asc)
// ([IDX] §2 TopK; §6.5 deterministic), without ever writing the score matrix.
//
// Workgroup: 8 waves, one query row per wave (8 consecutive rows), heaviest rows
// first.  Keys stream through LDS in tiles of 256 (fp8) or 64 (bf16) keys by direct
// global->LDS copies issued tiles ahead, one workgroup barrier per tile; every wave
// scores its query against each 64-key sub-tile:
//   MFMA   rows = 16 indexer heads, columns = 16 keys, K = head dim (fp8: one
//          v_mfma_f32_16x16x128_f8f6f4 per 16x16 tile; bf16: d/32 x 16x16x32);
//   head sum: lane (g, c) holds heads 4g+r of key c; it folds ReLU and w in
//          registers, and two permlane32 swaps plus one permlane16 swap finish the
//          sum so that lane l ends with the score of key 64T + l;
//   filter: a key is a candidate only if its order key exceeds the current
//          threshold; candidates are appended to a per-wave pending list in LDS.
// The exact top-k state (2048 (key, position) pairs) lives in registers, 32 per
// lane.  When the pending list fills, a wave-level radix select on the 64-bit key
// (order(score) << 32 | ~position) over state + pending finds the k-th best, keeps
// exactly the k best and raises the threshold to that element's score key.
// Keys arrive in increasing position, so a later key that ties the threshold
// score always loses the tie: the strict filter is exact.
#include "dsa_device.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kFT = 64;         // keys per sub-tile (one score per lane)
constexpr int kFW = 8;          // waves (= query rows) per workgroup
constexpr int kSlots = 32;      // state slots per lane: 2048 per wave
constexpr int kPendCap = 1344;  // pending candidates per wave (LDS: 158 KB in all for fp8)

// Keys per tile (between workgroup barriers) = kFT x tm: fp8 key rows are small
// enough for 256-key tiles, a quarter of the barriers per key of 64-key tiles.
template <bool FP8, int D>
struct FCfg {
  static constexpr int tm = FP8 ? 4 : 1;                      // sub-tiles per tile
  static constexpr int tile_keys = kFT * tm;
  static constexpr int row_bytes = FP8 ? D : 2 * D;           // one key row in LDS
  static constexpr int tile_bytes = tile_keys * row_bytes;
  static constexpr int dma_per_tile = tile_bytes / 1024;     // 64 lanes x 16 B copies
  static constexpr int gran = row_bytes / 16;
};

// key tiles in LDS (the one being scored + ring-1 in flight): 2 fp8 tiles of 32 KB,
// 2 bf16 tiles of 16 KB (d = 128) or 4 of 8 KB (d = 64)
template <bool FP8, int D>
constexpr int ring_of() {
  return FP8 ? 2 : FCfg<FP8, D>::tile_bytes <= 8192 ? 4 : 2;
}

template <bool FP8, int D>
struct FusedSmem {
  uint8_t tile[ring_of<FP8, D>()][FCfg<FP8, D>::tile_bytes];
  float kscale[ring_of<FP8, D>()][FCfg<FP8, D>::tile_keys];
  uint32_t pkey[kFW][kPendCap];
  uint32_t ppos[kFW][kPendCap];
  uint32_t hist[kFW][256];
  int need[2][kFW];  // per-wave "pending list nearly full" votes, by tile parity
};

__device__ __forceinline__ uint64_t key64(uint32_t key, uint32_t pos) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - pos);
}

__device__ __forceinline__ float key_to_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Moves pending entries [0, n) into the free (key == 0) state slots, lane by lane.
__device__ __forceinline__ void fill_free(uint32_t (&skey)[kSlots], uint32_t (&spos)[kSlots], const uint32_t* pkey,
                                          const uint32_t* ppos, int n, int lane) {
  int freec = 0;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) freec += skey[j] == 0u;
  // exclusive prefix of free counts over lanes
  int incl = freec;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  int cur = incl - freec;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    if (skey[j] == 0u && cur < n) {
      skey[j] = pkey[cur];
      spos[j] = ppos[cur];
      ++cur;
    }
  }
}

// Keeps exactly the k best of state + pending and returns the new threshold key.
// Wave-level; uses this wave's histogram and pending areas of LDS only.
template <bool NARROW>
__device__ uint32_t compact(uint32_t (&skey)[kSlots], uint32_t (&spos)[kSlots], uint32_t* pkey, uint32_t* ppos,
                           uint32_t* hist, int n_pend, int& n_state, uint32_t theta, int k, int lane) {
  if (n_state + n_pend <= k) {
    fill_free(skey, spos, pkey, ppos, n_pend, lane);
    n_state += n_pend;
    return theta;
  }
  // radix select of the k-th largest 64-bit key, 8 bits at a time, most significant
  // first.  NARROW: start at the highest bit where the candidates differ (their min
  // and max agree above it, so the passes above would put every key into one bin and
  // every lane's histogram atomic onto one LDS address); used where registers allow.
  int shift = 56;
  uint64_t pmask = 0ull, prefix = 0ull;
  if constexpr (NARROW) {
    uint64_t lo = ~0ull, hi = 0ull;
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      if (skey[j] != 0u) {
        const uint64_t kk = key64(skey[j], spos[j]);
        lo = kk < lo ? kk : lo;
        hi = kk > hi ? kk : hi;
      }
    }
    for (int p = lane; p < n_pend; p += 64) {
      const uint64_t kk = key64(pkey[p], ppos[p]);
      lo = kk < lo ? kk : lo;
      hi = kk > hi ? kk : hi;
    }
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint64_t olo = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(lo >> 32), d) << 32) |
                           (uint32_t)__shfl_xor((int)(uint32_t)lo, d);
      const uint64_t ohi = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(hi >> 32), d) << 32) |
                           (uint32_t)__shfl_xor((int)(uint32_t)hi, d);
      lo = olo < lo ? olo : lo;
      hi = ohi > hi ? ohi : hi;
    }
    const int top = 63 - __clzll((long long)(lo ^ hi));
    shift = top >= 7 ? top - 7 : 0;
    pmask = shift + 8 >= 64 ? 0ull : ~0ull << (shift + 8);
    prefix = hi & pmask;
  }
  uint32_t remaining = (uint32_t)k;
  for (;; shift -= 8) {
    if (shift < 0) shift = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) hist[4 * lane + b] = 0u;
#pragma unroll
    for (int j = 0; j < kSlots; ++j) {
      const uint64_t kk = key64(skey[j], spos[j]);
      if (skey[j] != 0u && (kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
    }
    for (int p = lane; p < n_pend; p += 64) {
      const uint64_t kk = key64(pkey[p], ppos[p]);
      if ((kk & pmask) == prefix) atomicAdd(&hist[(kk >> shift) & 255u], 1u);
    }
    uint32_t h[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) h[b] = hist[4 * lane + b];
    const uint32_t local = h[0] + h[1] + h[2] + h[3];
    uint32_t incl = local;  // suffix sum over lanes: bins >= 4 lane
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_down(incl, d);
      if (lane + d < 64) incl += o;
    }
    uint32_t above = incl - local;  // bins > 4 lane + 3
    int found = -1;
    uint32_t f_above = 0, f_cnt = 0;
#pragma unroll
    for (int b = 3; b >= 0; --b) {
      if (found < 0 && above < remaining && remaining <= above + h[b]) {
        found = 4 * lane + b;
        f_above = above;
        f_cnt = h[b];
      }
      above += h[b];
    }
    const uint64_t ball = __ballot(found >= 0);
    const int src = __ffsll((long long)ball) - 1;
    const uint32_t digit = (uint32_t)__shfl(found, src);
    const uint32_t ab = __shfl(f_above, src);
    const uint32_t cnt = __shfl(f_cnt, src);
    prefix |= (uint64_t)digit << shift;
    pmask |= (uint64_t)0xFFu << shift;
    remaining -= ab;
    if (cnt == remaining || shift == 0) break;  // every key in this bin is selected
  }
  const uint64_t th = prefix;  // selected  <=>  key64 >= th  (exactly k keys)
#pragma unroll
  for (int j = 0; j < kSlots; ++j)
    if (skey[j] != 0u && key64(skey[j], spos[j]) < th) skey[j] = 0u;
  // pack the selected pending entries to the front, in place (writes trail reads)
  int kept = 0;
  for (int base = 0; base < n_pend; base += 64) {
    const int p = base + lane;
    uint32_t kk = 0, pp = 0;
    bool sel = false;
    if (p < n_pend) {
      kk = pkey[p];
      pp = ppos[p];
      sel = key64(kk, pp) >= th;
    }
    const uint64_t m = __ballot(sel);
    if (sel) {
      const int dst = kept + (int)__popcll(m & ((1ull << lane) - 1ull));
      pkey[dst] = kk;
      ppos[dst] = pp;
    }
    kept += (int)__popcll(m);
  }
  fill_free(skey, spos, pkey, ppos, kept, lane);
  n_state = k;
  return (uint32_t)(th >> 32);
}

template <int HB, bool FP8, int D>
__global__ __launch_bounds__(512) void idx_topk_fused_kernel(const void* __restrict__ q_idx,
                                                             const float* __restrict__ q_scale,
                                                             const void* __restrict__ k_idx,
                                                             const float* __restrict__ k_scale,
                                                             const uint16_t* __restrict__ w, int H, int k,
                                                             dsa_seqs seqs, int64_t n_groups, int bf16_scores,
                                                             int32_t* __restrict__ idx_out,
                                                             float* __restrict__ score_out) {
  using C = FCfg<FP8, D>;
  constexpr int kRing = ring_of<FP8, D>();
  __shared__ FusedSmem<FP8, D> sm;
  // the wave index is uniform: kept in a scalar register, so are the values derived from it
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g = lane >> 4;
  // Groups of kFW consecutive rows of one sequence (the rows of a group share its key
  // tiles, so a group never spans two sequences): sequence b owns ceil(nq_b / kFW) groups,
  // numbered in packed order; the grid takes them from the last (heaviest rows first).
  const int64_t grp = n_groups - 1 - (int64_t)blockIdx.x;
  int b = 0;
  int64_t g0 = 0;
  for (; b + 1 < seqs.B; ++b) {
    const int64_t ng = (seqs.q_start[b + 1] - seqs.q_start[b] + kFW - 1) / kFW;
    if (grp < g0 + ng) break;
    g0 += ng;
  }
  const int64_t n_q = seqs.q_start[b + 1] - seqs.q_start[b];   // rows of this sequence
  const int64_t q_pos0 = seqs.q_pos0[b], k_row0 = seqs.k_start[b];
  const int64_t n_keys = seqs.k_start[b + 1] - k_row0;
  const int block = seqs.block;
  const int64_t i0 = (grp - g0) * kFW;                        // sequence-local first row
  const bool row_ok = i0 + wave < n_q;
  const int64_t i = seqs.q_start[b] + (row_ok ? i0 + wave : n_q - 1);   // packed row
  // last visible key of a sequence-local row: its position, or its last visible
  // compressed block (floor(t / block) - 1, -1 for none) with block > 1
  auto last_key = [&](int64_t r) { return block > 1 ? (q_pos0 + r) / block - 1 : q_pos0 + r; };
  const int64_t t = row_ok ? last_key(i0 + wave) : -1;
  const int64_t t_max = last_key(i0 + kFW - 1 < n_q ? i0 + kFW - 1 : n_q - 1);
  constexpr int kTK = FCfg<FP8, D>::tile_keys;
  const int n_tiles = (int)((t_max + kTK) / kTK);
  const uint8_t* kbytes = (const uint8_t*)k_idx + k_row0 * C::row_bytes;
  const float* kscale_g = FP8 ? k_scale + k_row0 : nullptr;

  // ---- this row's q (A operand) and head weights w' = w * q_scale (heads 16hb + 4g + r)
  constexpr int KS = FP8 ? 1 : D / 32;
  i32x4 qa[HB][FP8 ? 2 : KS];
  float wl[HB][4];
  const int64_t qi = i;
  // padded heads (H < 16 HB) read a real head's q and get weight 0
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int head = min(16 * hb + c, H - 1);
    if constexpr (FP8) {
      const i32x4* src = reinterpret_cast<const i32x4*>((const uint8_t*)q_idx + (qi * H + head) * D + 32 * g);
      qa[hb][0] = src[0];
      qa[hb][1] = src[1];
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qa[hb][ks] = *reinterpret_cast<const i32x4*>((const uint16_t*)q_idx + (qi * H + head) * D + 32 * ks + 8 * g);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int hh = 16 * hb + 4 * g + r;
      const int hc = min(hh, H - 1);
      float wv = bf16_to_f32(w[qi * H + hc]);
      if constexpr (FP8) wv *= q_scale[qi * H + hc];
      wl[hb][r] = hh < H ? wv : 0.f;
    }
  }

  // ---- key tiles: copy j of a tile covers LDS bytes [1024 j, 1024 j + 1024); lane l
  // fills granule slot (l % gran) of row (1024 j / row_bytes + l / gran), holding the
  // row's granule slot ^ (row & 7) (XOR swizzle: conflict-free B-operand reads)
  // Every wave issues the same number of copies per tile (kDmaPerWave), so the
  // wait for tile T with later tiles in flight is a fixed vmcnt.
  constexpr int kDmaPerWave = C::dma_per_tile / kFW + (FP8 ? 1 : 0);
  static_assert(C::dma_per_tile % kFW == 0, "tile copies must spread evenly over the waves");
  auto issue_tile = [&](int T) {
    const int bi = T % kRing;
    if ((int64_t)T * kTK + kTK <= n_keys) {
      // a whole tile of keys: the tile's base is uniform (scalar registers) and each copy
      // needs only a 32-bit lane offset
      const uint8_t* tb = kbytes + (int64_t)T * kTK * C::row_bytes;
      const int ln = lane_id_here();
#pragma unroll
      for (int m = 0; m < C::dma_per_tile / kFW; ++m) {
        const int j = wave + kFW * m;
        const int r = j * (1024 / C::row_bytes) + ln / C::gran;
        const uint32_t off = (uint32_t)(r * C::row_bytes + 16 * ((ln % C::gran) ^ (r & 7)));
        dma16_s<0>(tb, off, lds_u32(&sm.tile[bi][1024 * j]));
      }
    } else {
      for (int j = wave; j < C::dma_per_tile; j += kFW) {
        const int r = j * (1024 / C::row_bytes) + lane / C::gran;
        const int slot = lane % C::gran;
        int64_t s = (int64_t)T * kTK + r;
        if (s > n_keys - 1) s = n_keys - 1;  // tail rows past the keys: in-bounds, masked later
        const uint8_t* src = kbytes + s * C::row_bytes + 16 * (slot ^ (r & 7));
        dma16(src, lds_u32(&sm.tile[bi][1024 * j]));
      }
    }
    if constexpr (FP8) {
      // wave w copies the scales of keys (kTK/8) w .. of the tile (kTK/8 lanes active)
      if (lane < kTK / kFW) {
        int64_t s = (int64_t)T * kTK + (kTK / kFW) * wave + lane;
        if (s > n_keys - 1) s = n_keys - 1;
        dma4(kscale_g + s, lds_u32(&sm.kscale[bi][(kTK / kFW) * wave]));
      }
    }
  };
  // s_waitcnt vmcnt(n) with the other counters unconstrained (n <= 15)
  auto wait_vm = [&](int n) {
    switch (n) {
      case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
      case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
      case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
      case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
      case 4: __builtin_amdgcn_s_waitcnt(0x0F74); break;
      case 5: __builtin_amdgcn_s_waitcnt(0x0F75); break;
      case 6: __builtin_amdgcn_s_waitcnt(0x0F76); break;
      default: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    }
  };

  uint32_t skey[kSlots], spos[kSlots];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    skey[j] = 0u;
    spos[j] = 0u;
  }
  uint32_t* pkey = sm.pkey[wave];
  uint32_t* ppos = sm.ppos[wave];
  uint32_t* hist = sm.hist[wave];
  int n_pend = 0, n_state = 0;
  uint32_t theta = 0u;  // order keys of real scores are > 0: everything passes at first

  for (int T = 0; T < kRing - 1 && T < n_tiles; ++T) issue_tile(T);
  for (int T = 0; T < n_tiles; ++T) {
    const int bi = T % kRing;
    // this wave's copies of tile T landed (later tiles may still be in flight) ...
    const int later = min(kRing - 2, n_tiles - 1 - T);
    wait_vm(later * kDmaPerWave);
    // ... and every wave's; tile T-1's buffer is no longer read.  LDS-only barrier:
    // waits for this wave's LDS operations, not for the tiles still in flight; the
    // "memory" clobber keeps the compiler from moving LDS accesses across it.
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    if (T + kRing - 1 < n_tiles) issue_tile(T + kRing - 1);
    // One software pipeline over the tile's 4 tm sub-blocks of 16 keys: the MFMAs of
    // sub-block q+2 are issued right after the ReLU-weighted head sum of sub-block q,
    // so the head sums, the cross-lane reduction and the filter of one 64-key
    // sub-tile run while the matrix core works on the next.
    // sub-block q of the tile: 16 keys 16q .. 16q+15 (sub-tile q / 4)
    auto mfma_sub = [&](int q, f32x4 (&acc)[HB]) {
      const int row = 16 * (q & 3) + c;
      const uint8_t* rb = sm.tile[bi] + (q >> 2) * kFT * C::row_bytes + row * C::row_bytes;
      if constexpr (FP8) {
        const i32x4 b0 = *reinterpret_cast<const i32x4*>(rb + 16 * ((2 * g) ^ (row & 7)));
        const i32x4 b1 = *reinterpret_cast<const i32x4*>(rb + 16 * ((2 * g + 1) ^ (row & 7)));
        const i32x8 bf = i32x8{b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          const i32x8 af = i32x8{qa[hb][0][0], qa[hb][0][1], qa[hb][0][2], qa[hb][0][3],
                                 qa[hb][1][0], qa[hb][1][1], qa[hb][1][2], qa[hb][1][3]};
          acc[hb] = mfma_fp8_16x16x128(af, bf, f32x4{0.f, 0.f, 0.f, 0.f});
        }
      } else {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) acc[hb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const i32x4 bf = *reinterpret_cast<const i32x4*>(rb + 16 * ((4 * ks + g) ^ (row & 7)));
#pragma unroll
          for (int hb = 0; hb < HB; ++hb) acc[hb] = mfma_bf16_16x16x32(qa[hb][ks], bf, acc[hb]);
        }
      }
    };
    auto head_sum = [&](const f32x4 (&acc)[HB]) {
      float ph[HB];
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        ph[hb] = wl[hb][0] * relu_bits(acc[hb][0]);
#pragma unroll
        for (int r = 1; r < 4; ++r) ph[hb] = fmaf(wl[hb][r], relu_bits(acc[hb][r]), ph[hb]);
      }
      if constexpr (HB == 4) return (ph[0] + ph[1]) + (ph[2] + ph[3]);
      if constexpr (HB == 2) return ph[0] + ph[1];
      return ph[0];
    };
    // ---- sub-tile sub: finish the head sum (lane (g, c) -> key 16 g + c of the
    // sub-tile, i.e. key 64 sub + lane of the tile) and filter
    auto finish = [&](int sub, const float (&part)[4]) {
      const auto x02 =
          __builtin_amdgcn_permlane32_swap(__float_as_uint(part[0]), __float_as_uint(part[2]), false, false);
      const auto x13 =
          __builtin_amdgcn_permlane32_swap(__float_as_uint(part[1]), __float_as_uint(part[3]), false, false);
      const float s02 = __uint_as_float(x02[0]) + __uint_as_float(x02[1]);
      const float s13 = __uint_as_float(x13[0]) + __uint_as_float(x13[1]);
      const auto y = __builtin_amdgcn_permlane16_swap(__float_as_uint(s02), __float_as_uint(s13), false, false);
      float score = __uint_as_float(y[0]) + __uint_as_float(y[1]);
      if constexpr (FP8) score *= sm.kscale[bi][kFT * sub + lane];
      if (bf16_scores) score = __uint_as_float(f32_to_bf16_bits(score) << 16);

      // ---- filter into the pending list
      const int64_t s = (int64_t)T * kTK + kFT * sub + lane;
      const uint32_t key = order_key(score);
      const bool pass = s <= t && key > theta;
      const uint64_t m = __ballot(pass);
      if (pass) {
        const int dst = n_pend + (int)__popcll(m & ((1ull << lane) - 1ull));
        pkey[dst] = key;
        ppos[dst] = (uint32_t)s;
      }
      n_pend += (int)__popcll(m);
    };
    constexpr int NQ = 4 * C::tm;
    f32x4 acc[2][HB];
    float part[4];
    mfma_sub(0, acc[0]);
    mfma_sub(1, acc[1]);
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      part[q & 3] = head_sum(acc[q & 1]);
      if (q + 2 < NQ) mfma_sub(q + 2, acc[q & 1]);
      if ((q & 3) == 3) finish(q >> 2, part);
    }
    // vote: compact every wave together (at the next tile) when any list is nearly
    // full, so one wave's compaction does not hold the others at the barrier
    // repeatedly.  Lists fill by at most kTK per tile, so one tile of delay is safe.
    if (lane == 0) sm.need[T & 1][wave] = n_pend > kPendCap - 2 * kTK;
    if (T > 0) {
      int any = 0;
#pragma unroll
      for (int w2 = 0; w2 < kFW; ++w2) any |= sm.need[(T - 1) & 1][w2];
      if (any && n_pend > 0) {
        theta = compact<FP8>(skey, spos, pkey, ppos, hist, n_pend, n_state, theta, k, lane);
        n_pend = 0;
      }
    }
  }
  if (n_pend > 0) theta = compact<FP8>(skey, spos, pkey, ppos, hist, n_pend, n_state, theta, k, lane);
  if (!row_ok) return;

  // ---- write the row (valid entries first, unordered; a row sort follows)
  int v = 0;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) v += skey[j] != 0u;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int o = __shfl_up(incl, d);
    if (lane >= d) incl += o;
  }
  int pos = incl - v;
  int32_t* orow = idx_out + i * (int64_t)k;
  float* srow = score_out ? score_out + i * (int64_t)k : nullptr;
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    if (skey[j] != 0u) {
      orow[pos] = (int32_t)spos[j];
      if (srow) srow[pos] = key_to_score(skey[j]);
      ++pos;
    }
  }
  for (int j = n_state + lane; j < k; j += 64) {
    orow[j] = -1;
    if (srow) srow[j] = 0.f;
  }
}

// Puts the valid prefix of each index row in position order (scores follow).  One
// workgroup per row.  The entries are distinct positions, so an entry's slot is the number
// of selected positions below it: a bitmap over the row's position range marks the
// selection and a prefix sum of its word popcounts gives every entry its slot, with no
// comparison sort.  Rows whose largest position reaches past the bitmap (2^18 positions)
// take a bitonic sort in LDS instead.
constexpr int kOrdThreads = 256;
constexpr int kOrdWords = 8192;                 // bitmap words: positions < 262144
constexpr int kOrdPer = 2048 / kOrdThreads;     // entries per thread (k <= 2048)

union OrdSmem {
  struct {
    uint32_t bits[kOrdWords];
    uint32_t pre[kOrdWords];
  } bm;
  struct {
    int32_t sp[2048];
    float ss[2048];
  } bt;
};

__global__ __launch_bounds__(kOrdThreads) void idx_row_order_kernel(int32_t* __restrict__ idx,
                                                                    float* __restrict__ score, int k, int64_t n_q) {
  __shared__ OrdSmem sm;
  __shared__ int32_t red[kOrdThreads / 64];
  __shared__ uint32_t tot[kOrdThreads / 64];
  const int64_t i = blockIdx.x;
  if (i >= n_q) return;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  int32_t* row = idx + i * (int64_t)k;
  float* srow = score ? score + i * (int64_t)k : nullptr;

  int32_t p[kOrdPer];
  float sc[kOrdPer];
  int32_t mx = -1;
#pragma unroll
  for (int u = 0; u < kOrdPer; ++u) {
    const int j = t + kOrdThreads * u;
    p[u] = j < k ? row[j] : -1;
    sc[u] = (j < k && srow) ? srow[j] : 0.f;
    mx = max(mx, p[u]);
  }
  for (int d = 32; d > 0; d >>= 1) mx = max(mx, __shfl_xor(mx, d));
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = max(max(red[0], red[1]), max(red[2], red[3]));
  if (mx < 0) return;                         // nothing selected: the row is all -1 already
  const int W = mx / 32 + 1;

  if (W <= kOrdWords) {
    for (int w = t; w < W; w += kOrdThreads) sm.bm.bits[w] = 0u;
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kOrdPer; ++u)
      if (p[u] >= 0) atomicOr(&sm.bm.bits[p[u] >> 5], 1u << (p[u] & 31));
    __syncthreads();
    // exclusive prefix of the word popcounts: thread t owns words [t c, t c + c)
    const int c = (W + kOrdThreads - 1) / kOrdThreads;
    const int w0 = t * c, w1 = min(W, w0 + c);
    uint32_t own = 0;
    for (int w = w0; w < w1; ++w) own += __popc(sm.bm.bits[w]);
    uint32_t incl = own;
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = __shfl_up(incl, d);
      if (lane >= d) incl += o;
    }
    if (lane == 63) tot[wv] = incl;
    __syncthreads();
    uint32_t base = incl - own;
    for (int w2 = 0; w2 < wv; ++w2) base += tot[w2];
    for (int w = w0; w < w1; ++w) {
      sm.bm.pre[w] = base;
      base += __popc(sm.bm.bits[w]);
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kOrdPer; ++u) {
      if (p[u] < 0) continue;
      const int w = p[u] >> 5;
      const uint32_t slot = sm.bm.pre[w] + __popc(sm.bm.bits[w] & ((1u << (p[u] & 31)) - 1u));
      row[slot] = p[u];
      if (srow) srow[slot] = sc[u];
    }
    return;
  }

  // bitonic fallback over the next power of two >= k
  int n = 1;
  while (n < k) n <<= 1;
  for (int j = t; j < n; j += kOrdThreads) {
    sm.bt.sp[j] = INT32_MAX;
    sm.bt.ss[j] = 0.f;
  }
  __syncthreads();
#pragma unroll
  for (int u = 0; u < kOrdPer; ++u) {
    const int j = t + kOrdThreads * u;
    if (j < k) {
      sm.bt.sp[j] = p[u] < 0 ? INT32_MAX : p[u];
      sm.bt.ss[j] = sc[u];
    }
  }
  __syncthreads();
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int j = t; j < n / 2; j += kOrdThreads) {
        const int lo = 2 * j - (j & (stride - 1));
        const int hi = lo + stride;
        const bool up = (lo & size) == 0;
        const int32_t a = sm.bt.sp[lo], b = sm.bt.sp[hi];
        if ((a > b) == up) {
          sm.bt.sp[lo] = b;
          sm.bt.sp[hi] = a;
          const float fa = sm.bt.ss[lo];
          sm.bt.ss[lo] = sm.bt.ss[hi];
          sm.bt.ss[hi] = fa;
        }
      }
      __syncthreads();
    }
  }
  for (int j = t; j < k; j += kOrdThreads) {
    const int32_t q = sm.bt.sp[j];
    row[j] = q == INT32_MAX ? -1 : q;
    if (srow) srow[j] = q == INT32_MAX ? 0.f : sm.bt.ss[j];
  }
}

}  // namespace

// Prefill-shaped calls: at least 256 rows and on average at least 8 rows per sequence
// (a group of 8 rows shares its key tiles; decode-shaped calls, one row per sequence,
// take the score slab and the wide select instead).
bool indexer_fused_ok(const IndexerArgs& a) {
  if (a.k > kSlots * 64) return false;
  const int64_t n_q = a.seqs.q_start[a.seqs.B] - a.seqs.q_start[0];
  if (n_q < 256 || n_q < (int64_t)kFW * a.seqs.B) return false;
  if (a.qk_dtype == DSA_FP8_E4M3) return a.d == 128;
  return a.d == 64 || a.d == 128;
}

hipError_t launch_indexer_fused(const IndexerArgs& a, hipStream_t st) {
  const int64_t n_q = a.seqs.q_start[a.seqs.B];
  int64_t n_groups = 0;
  for (int b = 0; b < a.seqs.B; ++b) n_groups += (a.seqs.q_start[b + 1] - a.seqs.q_start[b] + kFW - 1) / kFW;
  if (n_groups == 0) return hipSuccess;
  const int HB = a.H <= 16 ? 1 : a.H <= 32 ? 2 : 4;
  dim3 grid((unsigned)n_groups);
  const bool fp8 = a.qk_dtype == DSA_FP8_E4M3;
#define DSA_FUSED(HBv, F8, Dv)                                                                                 \
  if (HB == HBv && fp8 == F8 && a.d == Dv) {                                                                  \
    hipLaunchKernelGGL((idx_topk_fused_kernel<HBv, F8, Dv>), grid, dim3(64 * kFW), 0, st, a.q_idx, a.q_scale,   \
                       a.k_idx, a.k_scale, a.w, a.H, a.k, a.seqs, n_groups, a.flags & DSA_TOPK_BF16_SCORES,  \
                       a.idx_out, a.score_out);                                                              \
    found = true;                                                                                            \
  }
  bool found = false;
  DSA_FUSED(1, true, 128) DSA_FUSED(2, true, 128) DSA_FUSED(4, true, 128)
  DSA_FUSED(1, false, 128) DSA_FUSED(2, false, 128) DSA_FUSED(4, false, 128)
  DSA_FUSED(1, false, 64) DSA_FUSED(2, false, 64) DSA_FUSED(4, false, 64)
#undef DSA_FUSED
  if (!found) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(idx_row_order_kernel, dim3((unsigned)n_q), dim3(kOrdThreads), 0, st, a.idx_out, a.score_out,
                     a.k, n_q);
  return hipGetLastError();
}

}  // namespace dsa
