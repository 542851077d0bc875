// Exact top-k building blocks for one workgroup of 256 threads (4 waves):
// a radix select of the k-th largest 32-bit key over LDS histograms, and an
// order-preserving emission of the selected ids using wave ballots and
// mbcnt prefix counts.
#pragma once

#include "common.hpp"

namespace qsa {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

// key and id sources of the selection routines: arrays in LDS or memory
struct KeyArray {
  const uint32_t* k;
  __device__ __forceinline__ uint32_t operator()(int e) const { return k[e]; }
};
struct IdArray {
  const int32_t* id;
  __device__ __forceinline__ int32_t operator()(int e) const { return id[e]; }
};

struct SelShared {
  alignas(16) uint32_t hist[3][256];  // radix_kth: hist[0]; radix_kth_regs rotates all three
  uint32_t wcnt[2][kSelWaves];
  uint32_t bc[4];
};

// Thread-contiguous data read from memory in coalesced order.  The
// selection routines want thread t to hold 128 contiguous bytes (16-byte
// chunks 8t .. 8t + 7); read that way, every wave load touches 64 cache
// lines.  stage_chunks reads chunk 256 j + t in step j instead (a wave's
// load covers 1 KB contiguous), and transposes through a 32 KB LDS area in
// which chunk c sits at stage_pos(c): the chunks of each thread permuted
// among themselves so that the coalesced writes (consecutive chunks across
// lanes) and the thread-contiguous reads (lanes 128 bytes apart) both fall
// on distinct banks.
constexpr int kStageChunks = 8;  // 16-byte chunks per thread (32 KB per workgroup)

__device__ __forceinline__ int stage_pos(int c) {
  const int t = c >> 3;
  return c ^ ((t & 7) ^ ((t >> 3) & 1));
}

// out[i] = chunk kStageChunks * t + i for thread t, where load(c) returns
// chunk c.  Contains one workgroup barrier; the caller keeps the staging
// area untouched until every thread is past a later barrier.
template <class Load>
__device__ __forceinline__ void stage_chunks(const Load& load, uint4* stage,
                                             uint4 (&out)[kStageChunks]) {
  uint4 v[kStageChunks];
#pragma unroll
  for (int j = 0; j < kStageChunks; ++j) v[j] = load(j * kSelThreads + (int)threadIdx.x);
#pragma unroll
  for (int j = 0; j < kStageChunks; ++j)
    stage[stage_pos(j * kSelThreads + (int)threadIdx.x)] = v[j];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kStageChunks; ++i)
    out[i] = stage[stage_pos(kStageChunks * (int)threadIdx.x + i)];
}

// Exclusive prefix sum of one value per thread over the workgroup.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, SelShared& sh,
                                                    uint32_t& total) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  uint32_t incl = wave_incl_scan(v);
  if (lane == kWave - 1) sh.wcnt[0][wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    uint32_t c = sh.wcnt[0][w];
    base += (w < wave) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + incl - v;
}

// ---------------------------------------------------------------- register-resident selection

// Inclusive prefix sum over the wave with DPP: row shifts inside each
// 16-lane row, then row broadcasts carry the row totals upward.
__device__ __forceinline__ uint32_t wave_incl_scan_dpp(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
  return v;
}

// Sum over the wave, in every lane.
__device__ __forceinline__ uint32_t wave_sum_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_dpp(v), kWave - 1);
}

// Exact top-k of at most 64 * EPW keys held by one wave, element jj at lane
// jj % 64, slot jj / 64 (key 0 = no element; real keys are >= 1), elements
// in ascending id order by jj.  The k-th largest key T is found bit by bit
// (a count over the wave per bit, no barriers); then the keys above T and
// the first of the keys equal to T, in element order, are written to out in
// element order (k ids; at least k elements must be present).
// The k-th largest key T of the nonzero keys a wave holds (at least k of
// them), found bit by bit (a count over the wave per bit, no barriers);
// kk receives how many keys equal to T belong to the k largest.
template <int EPW>
__device__ __forceinline__ uint32_t wave_kth(const uint32_t (&key)[EPW], int k, uint32_t& kk) {
  uint32_t mx = 0u, nmn = 0u;
#pragma unroll
  for (int i = 0; i < EPW; ++i) {
    if (key[i] != 0u) {
      mx = max(mx, key[i]);
      nmn = max(nmn, ~key[i]);
    }
  }
  mx = wave_max_u32(mx);
  const uint32_t mn = ~wave_max_u32(nmn);
  uint32_t T = mx;
  kk = (uint32_t)k;
  if (mx != mn) {
    const int hi = 31 - __clz(mx ^ mn);  // highest bit where the keys differ
    T = hi == 31 ? 0u : (mx & ~((2u << hi) - 1u));
    for (int bit = hi; bit >= 0; --bit) {
      const uint32_t cand = T | (1u << bit);
      const uint32_t msk = ~((1u << bit) - 1u);  // the bits at and above `bit`
      uint32_t cnt = 0;
#pragma unroll
      for (int i = 0; i < EPW; ++i) cnt += (key[i] & msk) == cand ? 1u : 0u;
      cnt = wave_sum_u32(cnt);
      if (cnt >= kk) T = cand; else kk -= cnt;
    }
  }
  return T;
}

// A lower bound of the k-th largest nonzero key a wave holds (at least k
// of them): the bits of the k-th key from the highest bit where the wave's
// keys differ down to `bits` bits below it, the lower bits cleared.  At
// least k keys are >= the result, and it is within 2^-bits of the wave's
// key range below the k-th key.
template <int EPW>
__device__ __forceinline__ uint32_t wave_kth_floor(const uint32_t (&key)[EPW], int k, int bits) {
  uint32_t mx = 0u, nmn = 0u;
#pragma unroll
  for (int i = 0; i < EPW; ++i) {
    if (key[i] != 0u) {
      mx = max(mx, key[i]);
      nmn = max(nmn, ~key[i]);
    }
  }
  mx = wave_max_u32(mx);
  const uint32_t mn = ~wave_max_u32(nmn);
  if (mx == mn) return mx;
  const int hi = 31 - __clz(mx ^ mn);
  const int lo = hi - bits + 1 > 0 ? hi - bits + 1 : 0;
  uint32_t T = hi == 31 ? 0u : (mx & ~((2u << hi) - 1u));
  uint32_t kk = (uint32_t)k;
  for (int bit = hi; bit >= lo; --bit) {
    const uint32_t cand = T | (1u << bit);
    const uint32_t msk = ~((1u << bit) - 1u);
    uint32_t cnt = 0;
#pragma unroll
    for (int i = 0; i < EPW; ++i) cnt += (key[i] & msk) == cand ? 1u : 0u;
    cnt = wave_sum_u32(cnt);
    if (cnt >= kk) T = cand; else kk -= cnt;
  }
  return T;
}

template <int EPW>
__device__ __forceinline__ void wave_topk_ordered(const uint32_t (&key)[EPW],
                                                  const int32_t (&id)[EPW], int k,
                                                  int32_t* out) {
  uint32_t kk;
  const uint32_t T = wave_kth<EPW>(key, k, kk);
  // in element order: keys above T, and the first kk keys equal to T
  uint32_t eq_before = 0, taken = 0;
#pragma unroll
  for (int i = 0; i < EPW; ++i) {
    const uint64_t me = __ballot(key[i] == T);
    const bool tk = key[i] > T || (key[i] == T && eq_before + lanes_below(me) < kk);
    const uint64_t mt = __ballot(tk);
    if (tk) out[taken + lanes_below(mt)] = id[i];
    eq_before += (uint32_t)__popcll(me);
    taken += (uint32_t)__popcll(mt);
  }
}

// Inclusive prefix sum of one value per thread over the workgroup (one
// barrier pair).  total receives the workgroup sum.
__device__ __forceinline__ uint32_t block_incl_scan(uint32_t v, SelShared& sh, uint32_t& total) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const uint32_t incl = wave_incl_scan_dpp(v);
  if (lane == kWave - 1) sh.wcnt[0][wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint32_t c = sh.wcnt[0][w];
    base += (w < wave) ? c : 0u;
    tot += c;
  }
  __syncthreads();
  total = tot;
  return base + incl;
}

// The maxima of a and of b over the workgroup in one exchange.
__device__ __forceinline__ void block_max2_u32(uint32_t& a, uint32_t& b, SelShared& sh) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  a = wave_max_u32(a);
  b = wave_max_u32(b);
  if (lane == 0) {
    sh.wcnt[0][wave] = a;
    sh.wcnt[1][wave] = b;
  }
  __syncthreads();
  a = 0u;
  b = 0u;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    a = max(a, sh.wcnt[0][w]);
    b = max(b, sh.wcnt[1][w]);
  }
  __syncthreads();
}

__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, SelShared& sh) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  v = wave_max_u32(v);
  if (lane == 0) sh.wcnt[1][wave] = v;
  __syncthreads();
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) m = max(m, sh.wcnt[1][w]);
  __syncthreads();
  return m;
}

// Finds T, the k-th largest key among get(0..n-1) (1 <= k <= n), and r, the
// number of elements equal to T that belong to the k largest (ties are
// later resolved by index order).  The digits are 8 bits wide, starting
// below the bits common to all keys; each pass histograms (LDS atomics)
// the elements still matching the digits fixed so far.  With max_passes
// too small to reach bit 0, T is the k-th largest key with its unresolved
// low bits cleared, a lower bound of it.
template <class Get>
__device__ void radix_kth(const Get& get, int n, int k, SelShared& sh,
                          uint32_t& T, int& r, int max_passes = 4) {
  const int tid = threadIdx.x;
  // bits above the highest bit where the largest and smallest keys differ
  // are common to all keys: the digits start below them
  uint32_t mx = 0u, nmn = 0u;
#pragma unroll 4
  for (int e = tid; e < n; e += kSelThreads) {
    const uint32_t key = get(e);
    mx = max(mx, key);
    nmn = max(nmn, ~key);
  }
  mx = block_max_u32(mx, sh);
  const uint32_t mn = ~block_max_u32(nmn, sh);
  if (mx == mn) {
    T = mx;
    r = k;
    return;
  }
  int hi = 31 - __clz(mx ^ mn);
  uint32_t prefix = (hi == 31) ? 0u : (mx & ~((2u << hi) - 1u));
  uint32_t mask = (hi == 31) ? 0u : ~((2u << hi) - 1u);
  uint32_t kk = (uint32_t)k;
  for (int pass = 0; pass < max_passes; ++pass) {
    const int shift = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (1u << (hi - shift + 1)) - 1u;
    sh.hist[0][tid] = 0u;
    __syncthreads();
#pragma unroll 4
    for (int e = tid; e < n; e += kSelThreads) {
      const uint32_t key = get(e);
      if ((key & mask) == prefix) atomicAdd(&sh.hist[0][(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread t looks at digit 255 - t: counts from the top down
    const uint32_t d = 255u - (uint32_t)tid;
    const uint32_t h = sh.hist[0][d];
    uint32_t tot;
    const uint32_t incl = block_incl_scan(h, sh, tot);
    if (incl - h < kk && kk <= incl) {
      sh.bc[0] = d;
      sh.bc[1] = kk - (incl - h);
    }
    __syncthreads();
    prefix |= sh.bc[0] << shift;
    mask |= dmask << shift;
    kk = sh.bc[1];
    __syncthreads();
    if (shift == 0) break;
    hi = shift - 1;
  }
  T = prefix;
  r = (int)kk;
}

// Writes id(e) for every selected e, in increasing e, to out[0..k): e is
// selected when get(e) > T, or get(e) == T and fewer than r earlier elements
// equal T (writes past out_cap are dropped).  Each wave walks one contiguous quarter of 0..n-1 in steps of 64;
// ballots give the in-step ranks, per-wave counts give the wave offsets.
template <class Get, class Id>
__device__ void emit_topk(const Get& get, const Id& id, int n, uint32_t T,
                          int r, int32_t* out, int out_cap, SelShared& sh) {
  const int wave = threadIdx.x / kWave, lane = lane_id();
  const int per = (((n + kSelWaves - 1) / kSelWaves) + kWave - 1) / kWave * kWave;
  const int beg = wave * per;
  const int end = min(n, beg + per);
  uint32_t gt = 0, eq = 0;
  for (int base = beg; base < end; base += kWave) {
    int e = base + lane;
    bool valid = e < end;
    uint32_t key = valid ? get(e) : 0u;
    gt += __popcll(ballot(valid && key > T));
    eq += __popcll(ballot(valid && key == T));
  }
  if (lane == 0) {
    sh.wcnt[0][wave] = gt;
    sh.wcnt[1][wave] = eq;
  }
  __syncthreads();
  uint32_t tie_base = 0, sel_base = 0;
  for (int w = 0; w < wave; ++w) {
    uint32_t g = sh.wcnt[0][w], q = sh.wcnt[1][w];
    uint32_t take = (uint32_t)r > tie_base ? min(q, (uint32_t)r - tie_base) : 0u;
    sel_base += g + take;
    tie_base += q;
  }
  __syncthreads();
  for (int base = beg; base < end; base += kWave) {
    int e = base + lane;
    bool valid = e < end;
    uint32_t key = valid ? get(e) : 0u;
    bool is_eq = valid && key == T;
    uint64_t eqm = ballot(is_eq);
    uint32_t tie_rank = tie_base + lanes_below(eqm);
    bool take = valid && (key > T || (is_eq && tie_rank < (uint32_t)r));
    uint64_t tm = ballot(take);
    const uint32_t at = sel_base + lanes_below(tm);
    if (take && at < (uint32_t)out_cap) out[at] = id(e);
    tie_base += __popcll(eqm);
    sel_base += __popcll(tm);
  }
}

// k-th largest key (1 <= k <= n) of the keys held in registers: thread t
// holds key[i] for element t * EPT + i, valid when that index is below n.
// The bits above the highest bit in which the largest and smallest keys
// differ are common to all keys; the radix digits start below them, 8 bits
// per pass, for at most max_passes passes.  On return T is the k-th largest
// key with any unresolved low bits cleared (a lower bound of it) and r the
// number of keys equal to T among the k largest (meaningful only when
// resolved is set).
//
// One workgroup barrier per pass: three histograms rotate (pass p counts
// into histogram p % 3 and clears the one pass p + 1 uses, whose last
// readers finished before pass p - 1's barrier), and every wave scans the
// whole histogram itself, so that no second exchange is needed to share the
// digit found.  The waves may still read the last pass's histogram on
// return; the next writer of a histogram clears it after a barrier.
template <int EPT>
__device__ void radix_kth_regs(const uint32_t (&key)[EPT], int n, int k, SelShared& sh,
                               uint32_t& T, int& r, bool& resolved, int max_passes = 4) {
  const int base_e = threadIdx.x * EPT;
  const int lane = lane_id();
  uint32_t mx = 0u, nmn = 0u;  // max and (~min)
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    if (base_e + i < n) {
      mx = max(mx, key[i]);
      nmn = max(nmn, ~key[i]);
    }
  }
  {
    // the maximum and (~minimum) over the workgroup; between the two
    // barriers every wave is past any earlier use of the histograms, and the
    // first pass's is cleared
    const int wave = threadIdx.x / kWave;
    mx = wave_max_u32(mx);
    nmn = wave_max_u32(nmn);
    if (lane == 0) {
      sh.wcnt[0][wave] = mx;
      sh.wcnt[1][wave] = nmn;
    }
    __syncthreads();
    sh.hist[0][threadIdx.x] = 0u;
    mx = 0u;
    nmn = 0u;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      mx = max(mx, sh.wcnt[0][w]);
      nmn = max(nmn, sh.wcnt[1][w]);
    }
    __syncthreads();
  }
  const uint32_t mn = ~nmn;
  if (mx == mn) {
    T = mx;
    r = k;
    resolved = true;
    return;
  }
  int hi = 31 - __clz(mx ^ mn);  // highest differing bit
  uint32_t prefix = (hi == 31) ? 0u : (mx & ~((2u << hi) - 1u));
  uint32_t mask = (hi == 31) ? 0u : ~((2u << hi) - 1u);
  uint32_t kk = (uint32_t)k;
  resolved = false;
  for (int pass = 0; pass < max_passes; ++pass) {
    const int shift = hi >= 7 ? hi - 7 : 0;
    const uint32_t dmask = (1u << (hi - shift + 1)) - 1u;
    const uint32_t* hist = sh.hist[pass % 3];
    sh.hist[(pass + 1) % 3][threadIdx.x] = 0u;
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      if (base_e + i < n && (key[i] & mask) == prefix)
        atomicAdd(&sh.hist[pass % 3][(key[i] >> shift) & dmask], 1u);
    }
    __syncthreads();
    // lane l: digits 255 - 4l .. 252 - 4l, counted from the top down
    const uint4 h = reinterpret_cast<const uint4*>(hist)[kWave - 1 - lane];
    const uint32_t cnt = h.x + h.y + h.z + h.w;
    const uint32_t incl = wave_incl_scan_dpp(cnt);
    // the lane in whose digits the count from the top first reaches kk (the
    // counts total at least kk: every key matches in the first pass, and
    // the digit chosen by a pass holds at least the kk keys the next needs)
    const uint64_t at = ballot(incl - cnt < kk && kk <= incl);
    const int src = __ffsll((unsigned long long)at) - 1;
    uint32_t c = incl - cnt;
    uint32_t d = 252u - 4u * (uint32_t)lane, left = kk - c;
    if (c + h.w >= kk) {
      d += 3u;
    } else if ((c += h.w) + h.z >= kk) {
      d += 2u;
      left = kk - c;
    } else if ((c += h.z) + h.y >= kk) {
      d += 1u;
      left = kk - c;
    } else {
      left = kk - (c + h.y);
    }
    d = (uint32_t)__builtin_amdgcn_readlane((int)d, src);
    kk = (uint32_t)__builtin_amdgcn_readlane((int)left, src);
    prefix |= d << shift;
    mask |= dmask << shift;
    if (shift == 0) {
      resolved = true;
      break;
    }
    hi = shift - 1;
  }
  T = prefix;
  r = (int)kk;
}

// Ordered emission for register-held keys and ids (thread t holds elements
// t * EPT + i, in increasing index order): element e is selected when its
// key > T, or key == T and fewer than r earlier elements equal T; the
// selected ids are written to out[0..) in index order (writes past out_cap
// are dropped).
template <int EPT>
__device__ void emit_regs(const uint32_t (&key)[EPT], const int32_t (&id)[EPT], int n,
                          uint32_t T, int r, int32_t* out, int out_cap, SelShared& sh) {
  static_assert(EPT * kSelThreads < 65536, "counts fit 16 bits");
  const int base_e = threadIdx.x * EPT;
  // the selected elements before thread t: every key above T, and the first
  // r keys equal to T -- one scan of both counts, packed (equal << 16 | above)
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const bool valid = base_e + i < n;
    gt += (valid && key[i] > T) ? 1u : 0u;
    eq += (valid && key[i] == T) ? 1u : 0u;
  }
  uint32_t tot;
  const uint32_t packed = (eq << 16) | gt;
  const uint32_t before = block_incl_scan(packed, sh, tot) - packed;
  uint32_t tie_before = before >> 16;
  uint32_t at = (before & 0xffffu) + min(tie_before, (uint32_t)r);
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const bool valid = base_e + i < n;
    const bool is_eq = valid && key[i] == T;
    const bool take = valid && (key[i] > T || (is_eq && tie_before < (uint32_t)r));
    tie_before += is_eq ? 1u : 0u;
    if (take) {
      if (at < (uint32_t)out_cap) out[at] = id[i];
      ++at;
    }
  }
}

}  // namespace qsa
