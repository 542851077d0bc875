// Block-sparse (and dense-baseline) attention on gfx950 matrix cores.
//
// Same computation as the generic kernel in attention.hip (the token set of
// a row is its selected 4-token blocks plus its own block, read straight
// from the paged cache, no mask; online softmax tile by tile), for bfloat16
// caches.  A wave works on one KV head and 32 tokens at a time:
//
//   S^T[32 tok x 16 heads] = K[32 x D] . Q^T      v_mfma_f32_16x16x32_bf16
//     A = K rows loaded straight from the cache (16 B per lane per step),
//     B = the group's query heads (padded to 16) held in registers.
//   O^T[D x 16 heads] += V^T[D x 32 tok] . P^T     v_mfma_f32_16x16x32_bf16
//     B = the softmax numerators, used in the registers where S^T left
//     them: the token order inside the 32-wide contraction is chosen so
//     that lane l's eight k-slots are exactly the eight tokens whose scores
//     lane l holds; A = V^T read from an LDS copy of the tile's V rows.
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
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

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
__global__ void __launch_bounds__(256) attn_mfma_kernel(AttnArgs a) {
  constexpr int NDT = D / 16;  // 16-wide d tiles of the output
  constexpr int KS = D / 32;   // 32-wide k steps of Q.K
  __shared__ int32_t ent_row[kMfmaEntChunk];
  __shared__ __align__(16) unsigned char lds[4 * kMfmaTileTok * kVPitch];
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

  // this lane's B fragment of Q^T: head c16 of the group, dims (D/4)g+8s..+8
  // (lane group g covers the contiguous quarter (D/4)g .. (D/4)(g+1) of the
  // head dimension across the KS steps; K uses the same order)
  u32x4_t qf[KS];
  {
    const bf16_t* qh = static_cast<const bf16_t*>(a.q) + ((int64_t)row * hq + hk * G + c16) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = (c16 < G) ? ld16(qh + (D / 4) * g + 8 * s) : u32x4_t{0u, 0u, 0u, 0u};
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
    for (int i = threadIdx.x; i < nloc; i += blockDim.x) {
      const int E = cb + i;
      const bool own = (E == n_list);
      const int b = own ? b_own : (DENSE ? E : sel_row[E]);
      const bool ok = own || (b >= 0 && b < b_own);
      ent_row[i] = ok ? (int32_t)a.pm.token_slot(seq, b * kBlock) : -1;
    }
    __syncthreads();
    const int n_tiles = (nloc + kMfmaTileEnt - 1) / kMfmaTileEnt;
    for (int tile = wsub; tile < n_tiles; tile += wph) {
      const int e0 = tile * kMfmaTileEnt;
      // K fragments: tokens 16*st + c16 of the tile, dims (D/4)g .. +D/4
      u32x4_t kf[2][KS];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int tau = 16 * st + c16, el = e0 + tau / 4, ti = tau % 4;
        const int r0 = el < nloc ? ent_row[el] : -1;
        const bool ok = r0 >= 0 && ti < ((cb + el == n_list) ? tail : kBlock);
        const bf16_t* p = kg + (int64_t)(r0 + ti) * rstride + (D / 4) * g;
#pragma unroll
        for (int s = 0; s < KS; ++s) kf[st][s] = ok ? ld16(p + 8 * s) : u32x4_t{0u, 0u, 0u, 0u};
      }
      // V rows of the tile: token g + 4i, 16-byte chunk c16 (c16 < D/8)
      u32x4_t vf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int tau = g + 4 * i, el = e0 + tau / 4, ti = tau % 4;
        const int r0 = el < nloc ? ent_row[el] : -1;
        const bool ok = c16 < D / 8 && r0 >= 0 && ti < ((cb + el == n_list) ? tail : kBlock);
        vf[i] = ok ? ld16(vg + (int64_t)(r0 + ti) * rstride + 8 * c16) : u32x4_t{0u, 0u, 0u, 0u};
      }
      // S^T: lane holds tokens 16*st + 4g + r for head c16
      f32x4_t sc[2];
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        sc[st] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < KS; ++s) sc[st] = mfma16(kf[st][s], qf[s], sc[st]);
      }
      if (c16 < D / 8) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          *reinterpret_cast<u32x4_t*>(vs + (g + 4 * i) * kVPitch + 16 * c16) = vf[i];
      }
      // online softmax (log2 domain)
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const int el = e0 + 4 * st + g;  // entry of tokens 16*st + 4g .. +3
        const int r0 = el < nloc ? ent_row[el] : -1;
        const int nt = r0 < 0 ? 0 : ((cb + el == n_list) ? tail : kBlock);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = r < nt ? sc[st][r] * sl2 : -INFINITY;
          x[4 * st + r] = v;
          mx = fmaxf(mx, v);
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m, mx);
      float corr = 1.0f, psum = 0.0f;
      float p[8];
      if (m_new == -INFINITY) {
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = 0.0f;
      } else {
        corr = __builtin_amdgcn_exp2f(m - m_new);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = __builtin_amdgcn_exp2f(x[j] - m_new);
          psum += p[j];
        }
      }
      lsum = lsum * corr + psum;
      m = m_new;
      const u32x4_t pb = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3]), pack_bf16(p[4], p[5]),
                          pack_bf16(p[6], p[7])};
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      // O^T += V^T . P^T; k-slot j of lane group g is token 4g + j (j < 4)
      // or 16 + 4g + (j - 4)
#pragma unroll
      for (int n = 0; n < NDT; ++n) {
        const unsigned char* col = vs + 2 * (16 * n + c16);
        uint32_t h[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int tok = (j < 4) ? (4 * g + j) : (16 + 4 * g + j - 4);
          h[j] = *reinterpret_cast<const uint16_t*>(col + tok * kVPitch);
        }
        const u32x4_t va = {h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16),
                            h[6] | (h[7] << 16)};
        acc[n] = acc[n] * corr;
        acc[n] = mfma16(va, pb, acc[n]);
      }
      __builtin_amdgcn_wave_barrier();
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
