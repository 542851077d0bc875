// Device helpers shared by the libqsa kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

using bf16_t = uint16_t;  // bfloat16 storage (upper half of a binary32)

constexpr int kWave = 64;

// ---------------------------------------------------------------- dtypes

__device__ __forceinline__ float bf16_to_f32(uint32_t h) {
  return __uint_as_float(h << 16);
}

// binary32 -> bfloat16, round to nearest, ties to even (NaN stays NaN).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (bf16_t)((u >> 16) | 0x40u);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

template <typename T> struct Vec;
// 16-byte vector of T, widened to float.
template <> struct Vec<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void load(const float* p, float (&f)[4]) {
    float4 v = *reinterpret_cast<const float4*>(p);
    f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
  }
  __device__ __forceinline__ static void store(float* p, const float (&f)[4]) {
    *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
  }
};
template <> struct Vec<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const uint4& v, float (&f)[8]) {
    f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xffff0000u);
    f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xffff0000u);
    f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xffff0000u);
    f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xffff0000u);
  }
  __device__ __forceinline__ static void load(const bf16_t* p, float (&f)[8]) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    unpack(v, f);
  }
  __device__ __forceinline__ static void store(bf16_t* p, const float (&f)[8]) {
    uint4 v;
    v.x = (uint32_t)f32_to_bf16(f[0]) | ((uint32_t)f32_to_bf16(f[1]) << 16);
    v.y = (uint32_t)f32_to_bf16(f[2]) | ((uint32_t)f32_to_bf16(f[3]) << 16);
    v.z = (uint32_t)f32_to_bf16(f[4]) | ((uint32_t)f32_to_bf16(f[5]) << 16);
    v.w = (uint32_t)f32_to_bf16(f[6]) | ((uint32_t)f32_to_bf16(f[7]) << 16);
    *reinterpret_cast<uint4*>(p) = v;
  }
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return bf16_to_f32(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) { return f32_to_bf16(x); }

// -0.0 -> +0.0 so that equal scores get equal keys.
__device__ __forceinline__ float canon_zero(float s) {
  return __float_as_uint(s) == 0x80000000u ? 0.0f : s;
}

// Order-preserving map float -> uint32 (larger float -> larger key).  Key 0
// lies below every real score and marks "no element".
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(canon_zero(s));
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ---------------------------------------------------------------- debug checks

// Built with -DQSA_DEBUG (libqsa_debug.so), the kernels check the device data
// the host cannot see: a page id outside [0, n_pages), a sequence id or
// position outside its range, and a selection length or selected id a row
// may not use.  Each such value sets a bit of a per-translation-unit error
// word (qsa_debug_take reports and clears them) and is replaced by one that
// keeps every access inside the caller's buffers (page 0; the clamped
// sequence id or position; the selection entry skipped), the same
// replacement the release build makes for everything but page ids.
// Without QSA_DEBUG the checks compile to nothing.
#ifdef QSA_DEBUG
static __device__ uint32_t g_debug_flags;  // this translation unit's error bits
__device__ __forceinline__ void debug_flag(uint32_t bit) { atomicOr(&g_debug_flags, bit); }
void debug_register(uint32_t (*take)());   // api.hip: the units' readers
namespace {
uint32_t debug_take_unit() {
  uint32_t v = 0, z = 0;
  (void)hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_flags), sizeof v, 0, hipMemcpyDeviceToHost);
  (void)hipMemcpyToSymbol(HIP_SYMBOL(g_debug_flags), &z, sizeof z, 0, hipMemcpyHostToDevice);
  return v;
}
struct DebugUnit {
  DebugUnit() { debug_register(&debug_take_unit); }
} debug_unit_registered;
}  // namespace
#else
__device__ __forceinline__ void debug_flag(uint32_t) {}
#endif

// page id read from a block table: checked in debug builds
__device__ __forceinline__ int32_t checked_page(int32_t page, int64_t n_pages) {
#ifdef QSA_DEBUG
  if ((uint64_t)(uint32_t)page >= (uint64_t)n_pages) {
    debug_flag(QSA_DEBUG_BAD_PAGE);
    return 0;
  }
#else
  (void)n_pages;
#endif
  return page;
}

// v clamped to [lo, hi]; in debug builds a value outside sets `bit`
__device__ __forceinline__ int clamp_flag(int v, int lo, int hi, uint32_t bit) {
#ifdef QSA_DEBUG
  if (v < lo || v > hi) debug_flag(bit);
#else
  (void)bit;
#endif
  return v < lo ? lo : (v > hi ? hi : v);
}

// ---------------------------------------------------------------- paging

struct PageMap {
  const int32_t* table;   // [n_seqs][max_pages]
  int32_t max_pages;
  int32_t page_shift;     // log2(page_size)
  int32_t blk_shift;      // log2(tokens per pooled block)
  int64_t n_pages;        // pages in the pool (debug builds check page ids)
  // physical page of logical page i of sequence seq
  __device__ __forceinline__ int32_t page(int seq, int i) const {
    return checked_page(table[(int64_t)seq * max_pages + i], n_pages);
  }
  __device__ __forceinline__ int64_t token_slot(int seq, int tok) const {
    // global token-row index: page * page_size + slot
    int32_t pg = page(seq, tok >> page_shift);
    return ((int64_t)pg << page_shift) + (tok & ((1 << page_shift) - 1));
  }
  // log2(pooled blocks per page)
  __device__ __forceinline__ int bpp_shift() const { return page_shift - blk_shift; }
  // row index of block b of sequence seq in the pooled-key array
  __device__ __forceinline__ int64_t block_slot(int seq, int b) const {
    const int sh = bpp_shift();
    int32_t pg = page(seq, b >> sh);
    return ((int64_t)pg << sh) + (b & ((1 << sh) - 1));
  }
};

// ---------------------------------------------------------------- wave ops

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of m below this lane
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
  uint32_t lo = __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u);
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), lo);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

// Maximum over the wave, returned in every lane: DPP inside each 16-lane
// row, then the four row results read as scalars.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// inclusive prefix sum over the lanes of a wave
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int l = lane_id();
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    uint32_t o = (uint32_t)__shfl_up((int)v, off);
    if (l >= off) v += o;
  }
  return v;
}

// ---------------------------------------------------------------- DPP sums

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over aligned groups of G lanes (G = 1, 2, 4, 8, 16 or 32); every lane
// of a group gets the group's sum.  DPP quad permutes and row mirrors keep
// the data in VGPRs (no LDS crossbar).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += dpp_f32<0xB1>(v);    // quad_perm [1,0,3,2]
  if constexpr (G >= 4) v += dpp_f32<0x4E>(v);    // quad_perm [2,3,0,1]
  if constexpr (G >= 8) v += dpp_f32<0x141>(v);   // row_half_mirror
  if constexpr (G >= 16) v += dpp_f32<0x140>(v);  // row_mirror
  if constexpr (G >= 32) v += __shfl_xor(v, 16);
  return v;
}

// ---------------------------------------------------------------- hand-off

// Data handed from one workgroup of a kernel to another is written with
// agent-scope atomic stores (write-through past the XCD-private L2) and read
// with agent-scope atomic loads, so no L2 write-back fence is needed.
template <typename U>
__device__ __forceinline__ void st_agent(U* p, U v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename U>
__device__ __forceinline__ U ld_agent(const U* p) {
  return __hip_atomic_load(const_cast<U*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Each wave waits until its own memory operations have completed: its
// agent-scope stores have then reached the level every XCD reads, before
// the workgroup's arrival is counted.  (A workgroup-scope fence does not
// wait for them, and a store and a later atomic may travel to different
// memory channels.)
__device__ __forceinline__ void wait_own_stores() { __builtin_amdgcn_s_waitcnt(0); }

// "Last workgroup" hand-off: every workgroup of a group calls this after
// publishing its results with st_agent; exactly one (the last to arrive)
// gets true.  Each wave first waits for its own stores to complete; the
// counter is reset for the next call.  The last workgroup then invalidates
// its caches once (agent-scope acquire), after which ordinary loads see the
// published data and can be issued back to back.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected,
                                            uint32_t* smem_flag) {
  wait_own_stores();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
    bool last = (prev == expected - 1);
    if (last) st_agent(counter, 0u);
    *smem_flag = last ? 1u : 0u;
  }
  __syncthreads();
  const bool last = *smem_flag != 0u;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

// Atomic adds to one address serialize (about 10 ns each here), so a
// hand-off among many workgroups counts in two levels: member idx of n
// first adds to the counter of its group of G members, and only the last
// member of each group adds to the top counter.  ctr[0] is the top counter
// and ctr[stride * (1 + g)] group g's, each on its own cache line.  Same
// guarantees as arrive_last: every counter is reset by its last member,
// and the one workgroup that gets true has seen every member's published
// data (each member's stores completed before its add, and each group's
// last member adds to the top counter after every add of its group).
template <int G>
__device__ __forceinline__ bool arrive_last_tree(uint32_t* ctr, int stride, uint32_t idx,
                                                 uint32_t n, uint32_t* smem_flag) {
  if (n <= (uint32_t)G) return arrive_last(ctr, n, smem_flag);
  wait_own_stores();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t g = idx / G;
    const uint32_t members = min((uint32_t)G, n - g * G);
    const uint32_t groups = (n + G - 1) / G;
    uint32_t* gc = ctr + (int64_t)stride * (1 + g);
    bool last = false;
    if (__hip_atomic_fetch_add(gc, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
        members - 1) {
      st_agent(gc, 0u);
      last = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
             groups - 1;
      if (last) st_agent(ctr, 0u);
    }
    *smem_flag = last ? 1u : 0u;
  }
  __syncthreads();
  const bool last = *smem_flag != 0u;
  if (last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  return last;
}

}  // namespace qsa
