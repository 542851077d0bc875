// Block-sparse (and dense-baseline) attention on gfx950 matrix cores.
//
// Same computation as the generic kernel in attention.hip (the token set of
// a row is its selected 4-token blocks plus its own block, read straight
// from the paged cache, no mask; online softmax tile by tile), for bfloat16
// caches.  A wave works on one KV head and 16 tokens at a time, with the
// next tile's K and V loads in flight while the current one is computed:
//
//   S^T[16 tok x 16 heads] = K[16 x D] . Q^T      v_mfma_f32_16x16x32_bf16
//     A = K rows loaded straight from the cache (16 B per lane per step),
//     B = the group's query heads (padded to 16) held in registers.
//   O^T[D x 16 heads] += V^T[D x 16 tok] . P^T     v_mfma_f32_16x16x16_bf16
//     B = the softmax numerators, used in the registers where S^T left
//     them (lane group g holds tokens 4g..4g+3, which are its four
//     k-slots); A = V^T read from an LDS copy of the tile's V rows.
//
// Workgroups: 4 waves per (row, split).  With n_splits > 1 (the SPLIT
// instances) the split partials go to the workspace and the last split of
// the row merges them.
#include "attention.hpp"

namespace qsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4_t ld16(const bf16_t* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}
__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
// O^T step on 16 tokens: 16x16x16 bf16, k-slot 4g + i of lane group g
__device__ __forceinline__ f32x4_t mfma16k16(u32x2_t a, u32x2_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bfloat16 pair, round to nearest even
// (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
// A column's reference maximum only moves when a new score exceeds it by
// more than this (log2 units): numerators stay below 2^kSlack, and the
// accumulator is rescaled rarely.  Numerators and their sum use the same
// reference, so the result does not depend on it.
constexpr float kSlack = 8.0f;

// Split partials of a row, [split][head] x (D floats of unnormalised acc,
// then (m in log2 units, l)), are written and merged by 256 threads that
// each own one head and D/16 contiguous dims of it (hq <= 16).
template <int D>
struct MergeLane {
  static constexpr int ND = D / 16;  // dims per thread
  int h, d0;
  bool on;
  __device__ MergeLane(int hq) : h(threadIdx.x / 16), d0((threadIdx.x % 16) * ND), on(h < hq) {}
};

__device__ __forceinline__ uint64_t pack2(float lo, float hi) {
  return (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }

constexpr int kMergeBatch = 8;  // splits whose partials are in flight together

// Merge of a row's split partials, run by the last split workgroup after its
// acquire.  Each thread keeps a running (M, L, O[ND]) for its head and dims;
// the partials of the next kMergeBatch splits are loaded while the current
// batch is folded in.
template <int D>
__device__ void merge_splits(const AttnArgs& a, int row, bf16_t* orow) {
  constexpr int ND = MergeLane<D>::ND;
  constexpr int NV = ND / 2;  // 8-byte loads per split
  const MergeLane<D> ml(a.hq);
  if (!ml.on) return;
  const int S = a.n_splits, hq = a.hq;
  const int64_t rb = (int64_t)row * S * hq;
  const uint64_t* pml = reinterpret_cast<const uint64_t*>(a.part_ml) + rb + ml.h;
  const uint64_t* pacc = reinterpret_cast<const uint64_t*>(a.part_acc + (rb + ml.h) * D + ml.d0);
  const int64_t acc_step = (int64_t)hq * D / 2;  // uint64 per split
  float M = -INFINITY, L = 0.0f, O[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) O[j] = 0.0f;
  uint64_t cm[kMergeBatch], cv[kMergeBatch][NV];
  auto load = [&](int s0) {
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const bool ok = s0 + u < S;
      cm[u] = ok ? pml[(int64_t)(s0 + u) * hq] : pack2(-INFINITY, 0.0f);
#pragma unroll
      for (int j = 0; j < NV; ++j) cv[u][j] = ok ? pacc[(s0 + u) * acc_step + j] : 0ull;
    }
  };
  load(0);
  for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
    uint64_t bm[kMergeBatch], bv[kMergeBatch][NV];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      bm[u] = cm[u];
#pragma unroll
      for (int j = 0; j < NV; ++j) bv[u][j] = cv[u][j];
    }
    if (s0 + kMergeBatch < S) load(s0 + kMergeBatch);
    float Mc = M;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) Mc = fmaxf(Mc, lo_f(bm[u]));
    if (Mc == -INFINITY) continue;  // nothing attended yet
    const float rs = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mc);
    L *= rs;
#pragma unroll
    for (int j = 0; j < ND; ++j) O[j] *= rs;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float mu = lo_f(bm[u]);
      const float f = (mu == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mu - Mc);
      L = fmaf(hi_f(bm[u]), f, L);
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        O[2 * j] = fmaf(lo_f(bv[u][j]), f, O[2 * j]);
        O[2 * j + 1] = fmaf(hi_f(bv[u][j]), f, O[2 * j + 1]);
      }
    }
    M = Mc;
  }
  const float inv = 1.0f / L;
  bf16_t* o = orow + ml.h * D + ml.d0;
#pragma unroll
  for (int j = 0; j < ND; ++j) o[j] = f32_to_bf16(O[j] * inv);
}

template <int D, bool DENSE, bool SPLIT>
__global__ void __launch_bounds__(256, SPLIT ? 2 : 3) attn_mfma_kernel(AttnArgs a) {
  constexpr int NDT = D / 16;  // 16-wide d tiles of the output
  constexpr int KS = D / 32;   // 32-wide k steps of Q.K
  // per list entry: element offset of its first token's row (a multiple of
  // Hkv*D >= 32) with the number of its tokens to attend (0..4) in the low
  // bits; padded to whole tiles with empty entries
  __shared__ int64_t ent_off[kMfmaEntChunk];
  constexpr int kStage = 4 * kMfmaTileTok * kVPitch;   // per-wave V tiles
  constexpr int kMerge = 4 * 16 * (D + 2) * 4;         // per-wave results
  __shared__ __align__(16) unsigned char lds[kStage > kMerge ? kStage : kMerge];
  __shared__ uint32_t flag;
  const int w = threadIdx.x / kWave, l = lane_id(), g = l / 16, c16 = l % 16;
  const int hkv = a.hkv, hq = a.hq, G = hq / hkv;
  const int wph = 4 / hkv;  // waves per KV head
  const int hk = w % hkv, wsub = w / hkv;
  const int row = blockIdx.y, split = blockIdx.x;

  const int seq = min(max(a.seq_id[row], 0), a.n_seqs - 1);
  const int t = min(max(a.pos[row], 0), a.max_pos);
  const int b_own = t / kBlock;
  const int n_list = DENSE ? b_own : min(max(a.n_sel[row], 0), a.top_k);
  const int n_entries = n_list + 1;
  const int* sel_row = DENSE ? nullptr : a.sel + (int64_t)row * a.top_k;
  const int e_beg = split * a.eps;
  const int e_end = min(n_entries, e_beg + a.eps);
  const int tail = (t % kBlock) + 1;  // tokens of the own block

  const bf16_t* kg = static_cast<const bf16_t*>(a.k) + hk * D;
  const bf16_t* vg = static_cast<const bf16_t*>(a.v) + hk * D;
  const int64_t rstride = (int64_t)hkv * D;
  const int64_t own_row = a.pm.token_slot(seq, b_own * kBlock);  // always present
  const int64_t own_off = own_row * rstride;
  const int64_t k_ti = (c16 % 4) * rstride;  // K: token c16 % 4 of an entry
  const int64_t v_ti = g * rstride;          // V: token g of an entry

  // this lane's B fragment of Q^T: head c16 of the group, dims 32s + 8g .. +8
  // at step s (K uses the same order, so one load instruction reads 64
  // contiguous bytes of each token row)
  u32x4_t qf[KS];
  {
    const bf16_t* qh = static_cast<const bf16_t*>(a.q) + ((int64_t)row * hq + hk * G + c16) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = (c16 < G) ? ld16(qh + 32 * s + 8 * g) : u32x4_t{0u, 0u, 0u, 0u};
  }
  const float sl2 = a.scale * 1.4426950408889634f;  // scores in log2 units
  float m = -INFINITY, lsum = 0.0f;
  f32x4_t acc[NDT];
#pragma unroll
  for (int n = 0; n < NDT; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  unsigned char* vs = lds + w * kMfmaTileTok * kVPitch;

  for (int cb = e_beg; cb < e_end; cb += kMfmaEntChunk) {
    const int nloc = min(e_end, cb + kMfmaEntChunk) - cb;
    __syncthreads();
    const int npad = (nloc + kMfmaTileEnt - 1) / kMfmaTileEnt * kMfmaTileEnt;
    for (int i = threadIdx.x; i < npad; i += blockDim.x) {
      const int E = cb + i;
      const bool own = (E == n_list);
      const int b = i >= nloc ? -1 : (own ? b_own : (DENSE ? E : sel_row[E]));
      const bool ok = i < nloc && (own || (b >= 0 && b < b_own));
      ent_off[i] = ok ? (a.pm.token_slot(seq, b * kBlock) * rstride) | (own ? tail : kBlock)
                      : own_row * rstride;
    }
    __syncthreads();
    const int n_tiles = (nloc + kMfmaTileEnt - 1) / kMfmaTileEnt;
    // A tile is 16 tokens (4 entries).  The K fragments (A operand: token
    // c16, dims 32s + 8g) and the V rows (token g + 4i, 16-byte chunk
    // c16) of the wave's next tile are loaded while the current one is
    // computed.
    //
    // Loads are unconditional (straight-line code keeps the prefetch in
    // flight): a token that is not attended -- past the own block's tail,
    // or of an invalid list entry -- is read from the row's own first
    // token instead, which is always in the cache; its score is masked to
    // -inf and its numerator is 0, so it contributes nothing.
    auto load_tile = [&](int tile, u32x4_t (&kf)[KS], u32x4_t (&vf)[4]) {
      const int e0 = tile * kMfmaTileEnt;
      {
        const int64_t v = ent_off[e0 + c16 / 4];
        const int64_t off = (c16 % 4) < (int)(v & 7) ? (v & ~7ll) + k_ti : own_off;
        const bf16_t* p = kg + off + 8 * g;
#pragma unroll
        for (int s2 = 0; s2 < KS; ++s2) kf[s2] = ld16(p + 32 * s2);
      }
      const int cv = c16 < D / 8 ? c16 : 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t v = ent_off[e0 + i];
        const int64_t off = g < (int)(v & 7) ? (v & ~7ll) + v_ti : own_off;
        vf[i] = ld16(vg + off + 8 * cv);
      }
    };
    // one tile: S^T, online softmax, O^T update
    auto compute = [&](int tile, const u32x4_t (&kf)[KS], const u32x4_t (&vf)[4]) {
      const int e0 = tile * kMfmaTileEnt;
      // S^T: lane holds tokens 4g + r (entry e0 + g) for head c16
      f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s2 = 0; s2 < KS; ++s2) sc = mfma16(kf[s2], qf[s2], sc);
      if (c16 < D / 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<u32x4_t*>(vs + (g + 4 * i) * kVPitch + 16 * c16) = vf[i];
      }
      float x[4];
      float mx = -INFINITY;
      {
        const int nt = (int)(ent_off[e0 + g] & 7);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = r < nt ? sc[r] * sl2 : -INFINITY;
          x[r] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      // move the reference maximum (and rescale) only when some column
      // needs it
      const bool grow = mx > m + kSlack;
      if (__ballot(grow) != 0ull) {
        const float m_new = grow ? mx : m;
        const float corr = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - m_new);
        lsum *= corr;
#pragma unroll
        for (int n = 0; n < NDT; ++n) acc[n] = acc[n] * corr;
        m = m_new;
      }
      float p[4];
      float psum = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        // m is -inf only while every score so far was masked (then x is too)
        p[j] = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(x[j] - m);
        psum += p[j];
      }
      lsum += psum;
      const u32x2_t pb = {cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])};
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // O^T += V^T . P^T; k-slot i of lane group g is token 4g + i
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        const unsigned char* col = vs + 2 * (16 * n + c16);
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          h[j] = *reinterpret_cast<const uint16_t*>(col + (4 * g + j) * kVPitch);
        const u32x2_t va = {h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
        acc[n] = mfma16k16(va, pb, acc[n]);
      }
      __builtin_amdgcn_wave_barrier();
    };
    // two register sets alternate: the loads of the wave's next tile go to
    // the set not being computed (the last tile reloads itself, so every
    // step issues the same loads and the wait before a product covers only
    // the current tile's)
    u32x4_t ka[KS], va4[4], kb[KS], vb4[4];
    if (wsub < n_tiles) load_tile(wsub, ka, va4);
    for (int tile = wsub; tile < n_tiles; tile += 2 * wph) {
      const int t1 = tile + wph;
      load_tile(t1 < n_tiles ? t1 : tile, kb, vb4);
      compute(tile, ka, va4);
      if (t1 >= n_tiles) break;
      const int t2 = t1 + wph;
      load_tile(t2 < n_tiles ? t2 : t1, ka, va4);
      compute(t1, kb, vb4);
    }
  }
  lsum += __shfl_xor(lsum, 16);
  lsum += __shfl_xor(lsum, 32);
  __syncthreads();
  // per-wave results to LDS: [wave][head][D + 2] (acc, then m, l)
  float* mrg = reinterpret_cast<float*>(lds);
  if (c16 < G) {
    float* o = mrg + (w * 16 + c16) * (D + 2);
#pragma unroll
    for (int n = 0; n < NDT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[16 * n + 4 * g + i] = acc[n][i];
    if (g == 0) {
      o[D] = m;
      o[D + 1] = lsum;
    }
  }
  __syncthreads();
  bf16_t* orow = static_cast<bf16_t*>(a.out) + (int64_t)row * hq * D;
  // combine the waves of each KV head: thread = (head, D/16 dims)
  const MergeLane<D> lane(hq);
  constexpr int ND = MergeLane<D>::ND;
  if (lane.on) {
    const int hk_ = lane.h / G, hh = lane.h % G;
    float M = -INFINITY;
    for (int j = 0; j < wph; ++j) M = fmaxf(M, mrg[((hk_ + j * hkv) * 16 + hh) * (D + 2) + D]);
    float L = 0.0f, O[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) O[i] = 0.0f;
    for (int j = 0; j < wph; ++j) {
      const float* o = mrg + ((hk_ + j * hkv) * 16 + hh) * (D + 2);
      const float f = (o[D] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(o[D] - M);
      L = fmaf(o[D + 1], f, L);
#pragma unroll
      for (int i = 0; i < ND; ++i) O[i] = fmaf(o[lane.d0 + i], f, O[i]);
    }
    if constexpr (!SPLIT) {
      const float inv = 1.0f / L;
#pragma unroll
      for (int i = 0; i < ND; ++i) orow[lane.h * D + lane.d0 + i] = f32_to_bf16(O[i] * inv);
    } else {
      // partials are read by another workgroup: agent-scope stores, 8 bytes
      // at a time
      const int64_t pbase = ((int64_t)row * a.n_splits + split) * hq + lane.h;
      uint64_t* pacc = reinterpret_cast<uint64_t*>(a.part_acc + pbase * D + lane.d0);
#pragma unroll
      for (int i = 0; i < ND / 2; ++i) st_agent(pacc + i, pack2(O[2 * i], O[2 * i + 1]));
      if (lane.d0 == 0) st_agent(reinterpret_cast<uint64_t*>(a.part_ml) + pbase, pack2(M, L));
    }
  }
  if constexpr (SPLIT) {
    if (!arrive_last(a.cnt + row, (uint32_t)a.n_splits, &flag)) return;
    merge_splits<D>(a, row, orow);
  }
}

bool attn_mfma_supported(int dtype, int hq, int hkv, int d) {
  return dtype == QSA_BF16 && (d == 64 || d == 128) && (hkv == 1 || hkv == 2 || hkv == 4) &&
         hq % hkv == 0 && hq <= 16;
}

void run_attention_mfma(const AttnArgs& a, int d, bool dense, int n_rows, hipStream_t st) {
  dim3 grid((unsigned)a.n_splits, (unsigned)n_rows);
  const bool split = a.n_splits > 1;
#define QSA_ATTN_LAUNCH(DD, DN, SP) \
  hipLaunchKernelGGL((attn_mfma_kernel<DD, DN, SP>), grid, dim3(256), 0, st, a)
  if (d == 128) {
    if (dense) {
      if (split) QSA_ATTN_LAUNCH(128, true, true); else QSA_ATTN_LAUNCH(128, true, false);
    } else {
      if (split) QSA_ATTN_LAUNCH(128, false, true); else QSA_ATTN_LAUNCH(128, false, false);
    }
  } else {
    if (dense) {
      if (split) QSA_ATTN_LAUNCH(64, true, true); else QSA_ATTN_LAUNCH(64, true, false);
    } else {
      if (split) QSA_ATTN_LAUNCH(64, false, true); else QSA_ATTN_LAUNCH(64, false, false);
    }
  }
#undef QSA_ATTN_LAUNCH
}

}  // namespace qsa
