// Exact top-k building blocks for one workgroup of 256 threads (4 waves):
// a radix select of the k-th largest 32-bit key over LDS histograms, and an
// order-preserving emission of the selected ids using wave ballots and
// mbcnt prefix counts.
#pragma once

#include "common.hpp"

namespace qsa {

constexpr int kSelThreads = 256;
constexpr int kSelWaves = kSelThreads / kWave;

struct SelShared {
  uint32_t hist[256];
  uint32_t wcnt[2][kSelWaves];
  uint32_t bc[4];
};

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

// Finds T, the k-th largest key among get(0..n-1) (1 <= k <= n), and r, the
// number of elements equal to T that belong to the k largest (ties are
// later resolved by index order).  Four passes of 8-bit digits, most
// significant first; each pass histograms the elements still matching the
// digits fixed so far.
template <class Get>
__device__ void radix_kth(const Get& get, int n, int k, SelShared& sh,
                          uint32_t& T, int& r) {
  const int tid = threadIdx.x;
  uint32_t prefix = 0, mask = 0;
  uint32_t kk = (uint32_t)k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    sh.hist[tid] = 0u;
    __syncthreads();
    for (int e = tid; e < n; e += kSelThreads) {
      uint32_t key = get(e);
      if ((key & mask) == prefix) atomicAdd(&sh.hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      const int l = tid;
      uint32_t h[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) h[j] = sh.hist[4 * l + j];
      uint32_t s = h[0] + h[1] + h[2] + h[3];
      // suffix sums from the top digit down: lanes above l
      uint32_t incl = s;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        uint32_t o = (uint32_t)__shfl_down((int)incl, off);
        if (l + off < kWave) incl += o;
      }
      uint32_t above = incl - s;
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (above < kk && kk <= above + h[j]) {
          sh.bc[0] = (uint32_t)(4 * l + j);
          sh.bc[1] = kk - above;
        }
        above += h[j];
      }
    }
    __syncthreads();
    uint32_t d = sh.bc[0];
    kk = sh.bc[1];
    prefix |= d << shift;
    mask |= 0xffu << shift;
    __syncthreads();
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

}  // namespace qsa
