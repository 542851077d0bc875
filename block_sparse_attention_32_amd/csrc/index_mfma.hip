// Prefill-side indexer and exact top-k on gfx950 matrix cores (bfloat16
// pooled keys, Di 64 or 128, up to 4 indexer heads).
//
// What is computed is exactly what index.hip computes -- the pooled-key
// scores s[b] = sum_h w[h] * max(0, q_idx[h] . kbar[b]) of every candidate
// block of every query row, and per row the top_k blocks (ties to the lower
// id, ascending ids) -- following keieiax.jp glossary "Qwen Sparse
// Attention", section 4トークンずつまとめて (a lightweight learned indexer
// rates each 4-token block; at most 512 blocks are kept per query).
//
// Many query rows share one sequence's pooled keys, so scoring is a dense
// contraction [rows x heads] x [Di x blocks]:
//   v_mfma_f32_16x16x32_bf16 with A = q_idx rows ordered (query, head) --
//   4 queries x 4 heads = 16 rows -- and B = 16 pooled-key rows.  Lane l of
//   the 16x16 result holds the four head dot products of query l/16 with
//   block l%16, so the ReLU and the weighted head sum are in-lane.
// A workgroup (8 waves x 16 queries) stages 256 pooled keys (one "group")
// at a time in LDS and runs them against its 128 queries.
//
// Exact top-k in four launches per batch of rows:
//   P1  sampled groups only (every s-th): for each (query, lane) the largest
//       key of the group -> the row's "union" of group maxima;
//   P2  per row: tau = the k'-th largest union key, k' = ceil(1.5 k / s),
//       its low bits cleared (k' = k without sampling: then tau is a lower
//       bound of the k-th key; with sampling about 1.5 k keys reach it);
//   P3  all groups: keys >= tau (the survivors; stored as block id and
//       score bits) appended per (row, split) in block order;
//   P4  per row: survivors gathered in block order -> exact radix select and
//       ordered emission (select.hpp); a row whose survivors overflowed its
//       slots, or number fewer than k, is listed for the exact fallback:
//       one streaming pass over its pooled keys keeps every key at or above
//       a guaranteed lower bound of the k-th (from its union), then the same
//       exact select.
#include <type_traits>

#include "index_device.hpp"
#include "select.hpp"

namespace qsa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

namespace {

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

template <int DI>
struct PGeom {
  static constexpr int KS = DI / 32;              // MFMA k steps
  static constexpr int ROWB = DI * 2;             // bytes per pooled key
  static constexpr int VPR = ROWB / 16;           // 16-byte vectors per row
  static constexpr int BUF = kPGrp * ROWB;        // LDS bytes of one staged group
  // LDS rows are unpadded; 16-byte chunk c of row r sits at position
  // c ^ swz(r), so that the 16 rows one operand read touches (the same
  // chunk of each) fall on 16 distinct groups of four banks (64 banks of
  // 4 bytes: two rows of Di 64, or one of Di 128, per 256 bytes)
  __device__ static constexpr int swz(int r) { return (r / (256 / ROWB)) % VPR; }
};

struct TileMeta {
  int32_t seq[kPQT];
  int32_t n[kPQT];
  uint32_t tau[kPQT];
  uint8_t active[kPQT];
  uint8_t done[kPQT];
  int cur_seq, n_hi, n_lo;
};

// Rows of the tile: sequence and candidate count (0 for rows past the
// batch).  Returns false if the tile has no rows.
__device__ __forceinline__ void load_tile_meta(const PIdxArgs& a, int tile, TileMeta& tm,
                                               bool with_tau) {
  for (int i = threadIdx.x; i < kPQT; i += blockDim.x) {
    const int rl = tile * kPQT + i;
    const bool ok = rl < a.rows;
    const int row = a.row0 + rl;
    tm.seq[i] = ok ? a.idx.seq_of(row) : -1;
    tm.n[i] = ok ? a.idx.pos_of(row) >> a.idx.pm.blk_shift : 0;
    tm.tau[i] = (ok && with_tau) ? a.tau[rl] : 0u;
    tm.done[i] = ok ? 0 : 1;
  }
  __syncthreads();
}

// Next sequence of the tile still to process (rows of one sequence share
// the staged pooled keys); false when every row is done.
__device__ __forceinline__ bool next_pass(TileMeta& tm) {
  if (threadIdx.x == 0) {
    int cur = -1;
    for (int i = 0; i < kPQT; ++i)
      if (!tm.done[i]) {
        cur = tm.seq[i];
        break;
      }
    tm.cur_seq = cur;
  }
  __syncthreads();
  const int cur = tm.cur_seq;
  if (cur < 0) return false;
  for (int i = threadIdx.x; i < kPQT; i += blockDim.x) {
    const bool act = !tm.done[i] && tm.seq[i] == cur;
    tm.active[i] = act;
    if (act) tm.done[i] = 1;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int hi = 0, lo = 0x7fffffff;
    for (int i = 0; i < kPQT; ++i)
      if (tm.active[i]) {
        hi = max(hi, tm.n[i]);
        lo = min(lo, tm.n[i]);
      }
    tm.n_hi = hi;
    tm.n_lo = lo;
  }
  __syncthreads();
  return true;
}

// sample stride of a pass: the largest power of two s <= kPMaxStride with
// ceil(n_lo / 256 / s) * 16 >= top_k (or 1): the sampled union still holds
// at least k maxima (a sparser sample leaves more rows short of k
// survivors, which the exact fallback then serves)
__device__ __forceinline__ int pass_stride(int n_lo, int top_k) {
  int s = 1;
  while (s < kPMaxStride && ((n_lo + kPGrp * 2 * s - 1) / (kPGrp * 2 * s)) * 16 >= top_k)
    s *= 2;
  return s;
}

// Order-preserving key of a score, as score_key() but in four operations:
// adding +0.0 turns -0.0 into +0.0; non-negative floats get the sign bit
// set, negative ones are inverted.  Every key of a real score is >= 1.
__device__ __forceinline__ uint32_t ordered_key(float s) {
  const uint32_t u = __float_as_uint(s + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

}  // namespace

// Inverse of ordered_key: the float whose key is k (k >= 1).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

// P1 (FILTER = false) and P3 (FILTER = true).  Grid (splits, tiles); 8 waves
// of 16 queries (4 MFMA tiles of 4 queries x 4 heads) per workgroup.
template <int DI, bool FILTER>
__global__ void __launch_bounds__(kPThreads, DI == 64 ? 4 : 2) pidx_kernel(PIdxArgs a) {
  using Gm = PGeom<DI>;
  constexpr int AT = kPQT / (kPThreads / kWave) / 4;  // MFMA tiles per wave
  // two staged groups of pooled keys: the next group is loaded (straight
  // into LDS) while the current one is scored
  __shared__ __align__(16) unsigned char kst[2 * Gm::BUF];
  __shared__ TileMeta tm;
  const int split = blockIdx.x, tile = blockIdx.y;
  const int w = threadIdx.x / kWave, l = lane_id(), g = l / 16, c16 = l % 16;
  if (tile * kPQT >= a.rows) return;
  load_tile_meta(a, tile, tm, FILTER);
  const bf16_t* kbar = static_cast<const bf16_t*>(a.idx.kbar);
  const bf16_t* qidx = static_cast<const bf16_t*>(a.idx.q_idx);
  const int hi_n = a.idx.hi;
  const float kNegInf = -__builtin_inff();
  while (next_pass(tm)) {
    const int seq = tm.cur_seq;
    const int n_groups = (tm.n_hi + kPGrp - 1) / kPGrp;
    const int s = FILTER ? 1 : a.tile_stride[tile];
    if (!FILTER && threadIdx.x == 0 && split == 0) {
      // the stride of this pass is a property of its rows; P2 reads it
      for (int i = 0; i < kPQT; ++i)
        if (tm.active[i]) a.row_stride[tile * kPQT + i] = s;
    }
    const int gps = (n_groups + a.splits - 1) / a.splits;
    const int g0 = split * gps, g1 = min(n_groups, g0 + gps);
    // A fragments of this wave's AT tiles of 4 queries x 4 heads, and for the
    // lane's query (C rows): weights, threshold as a float (-inf keeps
    // everything, NaN nothing) and survivor count
    u32x4_t af[AT][Gm::KS];
    float wq[AT][4], tf[AT], lmax[AT];
    uint32_t run[AT];
#pragma unroll
    for (int at = 0; at < AT; ++at) {
      const int qa = w * (4 * AT) + at * 4 + c16 / 4, ha = c16 % 4;  // A row: query, head
      const bool oka = tm.active[qa] && ha < hi_n;
      const bf16_t* qp = qidx + ((int64_t)(a.row0 + tile * kPQT + qa) * hi_n + ha) * DI;
#pragma unroll
      for (int ks = 0; ks < Gm::KS; ++ks)
        af[at][ks] = oka ? *reinterpret_cast<const u32x4_t*>(qp + 32 * ks + 8 * g)
                         : u32x4_t{0u, 0u, 0u, 0u};
      const int qc = w * (4 * AT) + at * 4 + g;
      const bool okc = tm.active[qc];
      const float* wp = a.idx.w + (int64_t)(a.row0 + tile * kPQT + qc) * hi_n;
#pragma unroll
      for (int h = 0; h < 4; ++h) wq[at][h] = (okc && h < hi_n) ? wp[h] : 0.0f;
      const uint32_t tk = tm.tau[qc];
      tf[at] = !okc ? __builtin_nanf("") : (tk == 0u ? kNegInf : key_float(tk));
      run[at] = 0u;
      lmax[at] = kNegInf;
    }
    const int region = kPSurvCap / a.splits;
    const int bpp_sh = a.idx.pm.bpp_shift();  // log2(blocks per page)
    const int n_hi = tm.n_hi;
    // blocks at or past a row's candidate count only occur in tiles that
    // reach past the pass's smallest count
    const int n_lo_pass = __builtin_amdgcn_readfirstlane(tm.n_lo);
    // A group is staged by VPT wave loads per wave, each 64 lanes x 16 bytes
    // written straight to 1 KB of LDS (global_load_lds_dwordx4): lane l of
    // wave load j fills LDS vector (w VPT + j) 64 + l of the group, i.e.
    // row vi / VPR at position vi % VPR, with the chunk that the row's
    // swizzle puts there.  Rows past the pass's largest candidate count read
    // the last candidate's key (finite; never a candidate of any row).
    constexpr int VPT = kPGrp * Gm::VPR / kPThreads;
    const int64_t tbase = (int64_t)seq * a.idx.pm.max_pages;
    const int bmask = (1 << bpp_sh) - 1;
    auto first_group = [&](int G) {
      while (G < g1 && !FILTER && (G % s) != 0) ++G;
      return G;
    };
    int32_t pgn[VPT];  // page ids of the rows this lane loads for the next group
    auto load_pages = [&](int G) {
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int vi = (w * VPT + j) * kWave + l;
        const int b = min(G * kPGrp + vi / Gm::VPR, n_hi - 1);
        pgn[j] = a.idx.pm.table[tbase + (b >> bpp_sh)];
      }
    };
    auto stage = [&](int G, int buf) {
#pragma unroll
      for (int j = 0; j < VPT; ++j) {
        const int vi = (w * VPT + j) * kWave + l;
        const int r = vi / Gm::VPR, c = (vi % Gm::VPR) ^ Gm::swz(r);
        const int b = min(G * kPGrp + r, n_hi - 1);
        const int64_t slot =
            ((int64_t)checked_page(pgn[j], a.idx.pm.n_pages) << bpp_sh) + (b & bmask);
        __builtin_amdgcn_global_load_lds(
            static_cast<const void*>(kbar + slot * DI + c * 8),
            (__attribute__((address_space(3))) void*)(kst + buf * Gm::BUF +
                                                      (w * VPT + j) * kWave * 16),
            16, 0, 0);
      }
    };
    int G = first_group(g0);
    if (G < g1) {
      load_pages(G);
      stage(G, 0);
    }
    int Gn = G < g1 ? first_group(G + 1) : g1;
    if (Gn < g1) load_pages(Gn);
    for (int buf = 0; G < g1; buf ^= 1) {
      const int b0 = G * kPGrp;
      // this wave's loads of group G have landed; after the barrier every
      // wave's have, and every wave is done reading the other buffer
      wait_own_stores();
      __syncthreads();
      const int Gnn = Gn < g1 ? first_group(Gn + 1) : g1;
      if (Gn < g1) {
        stage(Gn, buf ^ 1);
        if (Gnn < g1) load_pages(Gnn);
      }
      const unsigned char* kcur = kst + buf * Gm::BUF;
      // four steps of 16 keys per loop iteration: the compiler interleaves
      // one step's products with the previous step's epilogue
#pragma unroll 4
      for (int t16 = 0; t16 < kPGrp / 16; ++t16) {
        u32x4_t bf[Gm::KS];
        const int kr = t16 * 16 + c16;
        const unsigned char* rowp = kcur + kr * Gm::ROWB;
#pragma unroll
        for (int ks = 0; ks < Gm::KS; ++ks)
          bf[ks] = *reinterpret_cast<const u32x4_t*>(rowp + 16 * ((4 * ks + g) ^ Gm::swz(kr)));
        const int b = b0 + t16 * 16 + c16;
        f32x4_t c[AT];
#pragma unroll
        for (int at = 0; at < AT; ++at) {
          c[at] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < Gm::KS; ++ks) c[at] = mfma_bf16(af[at][ks], bf[ks], c[at]);
        }
        // per tile: ReLU, weighted head sum, then the union maximum (P1) or
        // the survivor test (P3); IN_RANGE: every block is a candidate of
        // every row of the pass
        auto epilogue = [&](auto in_range) {
#pragma unroll
          for (int at = 0; at < AT; ++at) {
            float sc = 0.0f;
#pragma unroll
            for (int h = 0; h < 4; ++h)
              sc = fmaf(wq[at][h], __builtin_amdgcn_fmed3f(c[at][h], 0.0f, 3.0e38f), sc);
            bool in = true;
            if constexpr (!decltype(in_range)::value) in = b < tm.n[w * (4 * AT) + at * 4 + g];
            if (!FILTER) {
              lmax[at] = in ? fmaxf(lmax[at], sc) : lmax[at];
            } else {
              // a float compare is the key compare: -0 and +0 compare
              // equal, and NaN thresholds (rows not in this pass) keep nothing
              const bool sv = in && sc >= tf[at];
              const uint64_t m = ballot(sv);
              if (m != 0ull) {
                const uint64_t gm = m & (0xffffull << (16 * g));
                const uint32_t pos = run[at] + lanes_below(gm);
                if (sv && pos < (uint32_t)region) {
                  const int rl = tile * kPQT + w * (4 * AT) + at * 4 + g;
                  a.surv[((int64_t)rl * a.splits + split) * region + pos] =
                      ((uint64_t)(uint32_t)b << 32) | __float_as_uint(sc);
                }
                run[at] += (uint32_t)__popcll(gm);
              }
            }
          }
        };
        if (b0 + t16 * 16 + 16 <= n_lo_pass)  // wave-uniform
          epilogue(std::true_type{});
        else
          epilogue(std::false_type{});
      }
      if (!FILTER) {
        // union entry (G / s) * 16 + lane of the lane's query; key 0 where
        // the lane saw no candidate
#pragma unroll
        for (int at = 0; at < AT; ++at) {
          const int qc = w * (4 * AT) + at * 4 + g;
          const int rl = tile * kPQT + qc;
          const int u = (G / s) * 16 + c16;
          const uint32_t key = lmax[at] == kNegInf ? 0u : ordered_key(lmax[at]);
          if (tm.active[qc] && u < kPUnion) a.uni[(int64_t)rl * kPUnion + u] = key;
          lmax[at] = kNegInf;
        }
      }
      G = Gn;
      Gn = Gnn;
    }
    if (FILTER && c16 == 0) {
#pragma unroll
      for (int at = 0; at < AT; ++at) {
        const int qc = w * (4 * AT) + at * 4 + g;
        if (tm.active[qc]) a.surv_cnt[(int64_t)(tile * kPQT + qc) * a.splits + split] = run[at];
      }
    }
  }
}

// Sample stride per tile: from the smallest candidate count of the tile's
// first sequence (P1 of a tile uses one stride for all its passes).
__global__ void __launch_bounds__(256) pidx_stride_kernel(PIdxArgs a) {
  __shared__ int lo;
  const int tile = blockIdx.x;
  if (threadIdx.x == 0) lo = 0x7fffffff;
  __syncthreads();
  for (int i = threadIdx.x; i < kPQT; i += blockDim.x) {
    const int rl = tile * kPQT + i;
    if (rl < a.rows) atomicMin(&lo, a.idx.pos_of(a.row0 + rl) >> a.idx.pm.blk_shift);
  }
  __syncthreads();
  if (threadIdx.x == 0) a.tile_stride[tile] = pass_stride(lo, a.top_k);
}

// P2: tau per row from its union of group maxima: the k'-th largest union
// key, k' = ceil(1.5 k / s) for sampling stride s (k' = k when every group
// was sampled), its low bits cleared (see below).  Each union key is a
// distinct key of the row, so at least k' keys are >= tau; the unsampled groups hold about (s - 1) times as many
// again, so about 1.5 k keys survive.  For s = 1 this is a guaranteed lower
// bound of the k-th key; otherwise P4 checks that at least k keys survived
// and falls back to an exact select when they did not.
//
// One wave per row (four rows per workgroup): the k'-th largest of the
// row's un union entries, empty entries (key 0) included, found bit by bit
// over the wave without barriers (lane l holds entries l, l + 64, ...), to
// kTauBits bits below the highest bit where the union's keys differ, the
// lower bits cleared: still a lower bound of the k'-th key (the keys it
// admits beyond it lie within 1/4096 of the union's key range), in about
// half the passes.
constexpr int kTauBits = 12;
template <int EPW>
__device__ __forceinline__ uint32_t union_kth_wave(const PIdxArgs& a, int rl, int un, int kq) {
  const int l = lane_id();
  const uint32_t* src = a.uni + (int64_t)rl * kPUnion;
  uint32_t key[EPW];
  uint32_t nz = 0;
#pragma unroll
  for (int i = 0; i < EPW; ++i) {
    const int jj = i * kWave + l;
    key[i] = jj < un ? src[jj] : 0u;
    nz += key[i] != 0u ? 1u : 0u;
  }
  // fewer than kq nonzero entries: the kq-th largest entry is an empty one
  if (wave_sum_u32(nz) < (uint32_t)kq) return 0u;
  return wave_kth_floor<EPW>(key, kq, kTauBits);
}

__global__ void __launch_bounds__(256) pidx_tau_wave_kernel(PIdxArgs a) {
  const int rl = blockIdx.x * (256 / kWave) + (int)threadIdx.x / kWave;
  if (rl >= a.rows) return;  // whole waves
  const int row = a.row0 + rl;
  const int n = a.idx.pos_of(row) >> a.idx.pm.blk_shift;
  if (n <= a.top_k) return;
  const int s = a.row_stride[rl];
  const int n_groups = (n + kPGrp - 1) / kPGrp;
  const int un = min(kPUnion, ((n_groups + s - 1) / s) * 16);
  const int kq = s == 1 ? a.top_k : max(1, min(a.top_k, (3 * a.top_k + 2 * s - 1) / (2 * s)));
  uint32_t tau = 0u;
  if (un >= kq) {
    if (un <= 16 * kWave) tau = union_kth_wave<16>(a, rl, un, kq);
    else if (un <= 32 * kWave) tau = union_kth_wave<32>(a, rl, un, kq);
    else tau = union_kth_wave<kPUnion / kWave>(a, rl, un, kq);
  }
  if (lane_id() == 0) a.tau[rl] = tau;
}

// Key of candidate e recomputed by this lane alone (P4's rare fallback).
template <int DI>
struct PRecomputed {
  const PIdxArgs* a;
  int row, seq;
  __device__ __forceinline__ uint32_t operator()(int e) const {
    const bf16_t* kb = static_cast<const bf16_t*>(a->idx.kbar) + a->idx.pm.block_slot(seq, e) * DI;
    const bf16_t* qr = static_cast<const bf16_t*>(a->idx.q_idx) + (int64_t)row * a->idx.hi * DI;
    float s = 0.0f;
    for (int h = 0; h < a->idx.hi; ++h) {
      float d = 0.0f;
      for (int c = 0; c < DI; ++c) d = fmaf(to_f32(qr[h * DI + c]), to_f32(kb[c]), d);
      s = fmaf(a->idx.w[(int64_t)row * a->idx.hi + h], fmaxf(d, 0.0f), s);
    }
    return score_key(s);
  }
};

struct IdSelf {
  __device__ __forceinline__ int32_t operator()(int e) const { return e; }
};
// P4 for the common case, one wave per row: rows whose survivors fit
// kPWave per lane (and are at least top_k, none lost to a full region).
// Survivor jj of the row (splits in order, each in block order) is held by
// lane jj % 64 as its element jj / 64 (wave_topk_ordered).  Rows it does
// not take are left to pidx_select_kernel (done = 0).
__global__ void __launch_bounds__(256) pidx_select_wave_kernel(PIdxArgs a) {
  const int wv = threadIdx.x / kWave, l = lane_id();
  const int rl = blockIdx.x * (256 / kWave) + wv;
  if (rl >= a.rows) return;  // whole waves
  const int row = a.row0 + rl;
  const int n = a.idx.pos_of(row) >> a.idx.pm.blk_shift;
  int32_t* sel_row = a.sel + (int64_t)row * a.top_k;
  if (n <= a.top_k) {
    for (int j = l; j < a.top_k; j += kWave) sel_row[j] = j < n ? j : -1;
    if (l == 0) {
      a.n_sel[row] = n;
      a.done[rl] = 1u;
    }
    return;
  }
  // survivor counts of the splits (lane s: split s) -> offsets
  const int region = kPSurvCap / a.splits;
  const uint32_t c = l < a.splits ? a.surv_cnt[(int64_t)rl * a.splits + l] : 0u;
  const uint32_t incl = wave_incl_scan_dpp(c);
  const uint32_t m = (uint32_t)__builtin_amdgcn_readlane((int)incl, kWave - 1);
  if (ballot(c > (uint32_t)region) != 0ull || m > (uint32_t)(kWave * kPWave) ||
      m < (uint32_t)a.top_k)
    return;  // the fallback kernel takes the row
  // survivor jj lives at slot jj + sum over splits s >= 1 with jj >= offs[s]
  // of (region - count[s - 1]) of the row's regions
  uint32_t so[kPMaxSplits], dl[kPMaxSplits];
#pragma unroll
  for (int sp = 1; sp < kPMaxSplits; ++sp) {
    const int q = sp < a.splits ? sp : 0;
    so[sp] = sp < a.splits ? (uint32_t)__builtin_amdgcn_readlane((int)(incl - c), q) : 0xffffffffu;
    dl[sp] = (uint32_t)region - (uint32_t)__builtin_amdgcn_readlane((int)c, sp - 1);
  }
  const uint64_t* rs = a.surv + (int64_t)rl * a.splits * region;
  uint32_t key[kPWave];
  int32_t id[kPWave];
#pragma unroll
  for (int i = 0; i < kPWave; ++i) {
    const uint32_t jj = (uint32_t)(i * kWave + l);
    const bool ok = jj < m;
    uint32_t slot = jj;
#pragma unroll
    for (int sp = 1; sp < kPMaxSplits; ++sp) slot += jj >= so[sp] ? dl[sp] : 0u;
    const uint64_t v = ok ? rs[slot] : 0ull;
    key[i] = ok ? ordered_key(__uint_as_float((uint32_t)v)) : 0u;
    id[i] = ok ? (int32_t)(v >> 32) : 0;
  }
  wave_topk_ordered<kPWave>(key, id, a.top_k, sel_row);
  if (l == 0) {
    a.n_sel[row] = a.top_k;
    a.done[rl] = 1u;
  }
}

// P4: gather, exact select, ordered emission (the rows the one-wave select
// left: more survivors than it holds, a full region, or fewer than k).
template <int DI>
__global__ void __launch_bounds__(256) pidx_select_kernel(PIdxArgs a) {
  __shared__ uint32_t offs[kPMaxSplits + 1];
  __shared__ SelShared sh;
  const int rl = blockIdx.x, row = a.row0 + rl;
  {
    const bool done = a.done[rl] != 0u;
    __syncthreads();
    if (done) {
      if (threadIdx.x == 0) a.done[rl] = 0u;  // cleared for the next call
      return;
    }
  }
  const int n = a.idx.pos_of(row) >> a.idx.pm.blk_shift;
  int32_t* sel_row = a.sel + (int64_t)row * a.top_k;
  if (n <= a.top_k) {
    for (int j = threadIdx.x; j < a.top_k; j += blockDim.x) sel_row[j] = j < n ? j : -1;
    if (threadIdx.x == 0) a.n_sel[row] = n;
    return;
  }
  const int region = kPSurvCap / a.splits;
  if (threadIdx.x == 0) {
    uint32_t o = 0;
    bool over = false;
    for (int sp = 0; sp < a.splits; ++sp) {
      const uint32_t c = a.surv_cnt[(int64_t)rl * a.splits + sp];
      over |= c > (uint32_t)region;
      offs[sp] = o;
      o += c;
    }
    offs[a.splits] = (over || o > (uint32_t)kPSelCap) ? 0xffffffffu : o;
  }
  __syncthreads();
  const uint32_t m = offs[a.splits];
  if (m != 0xffffffffu && m >= (uint32_t)a.top_k) {
    // survivor j of the row (splits in order, each in block order) is
    // entry j - offs[sp] of split sp's region, offs[sp] <= j < offs[sp + 1].
    // Thread t holds survivors [EPT t, EPT t + EPT) in registers (loads all
    // in flight), then the register radix select and ordered emission.
    constexpr int EPT = kPSelCap / 256;
    const uint64_t* rs = a.surv + (int64_t)rl * a.splits * region;
    const int base = (int)threadIdx.x * EPT;
    int sp = 0;
    while (sp + 1 < a.splits && offs[sp + 1] <= (uint32_t)base) ++sp;
    uint32_t start = offs[sp];
    uint32_t next = sp + 1 < a.splits ? offs[sp + 1] : m;
    uint64_t v[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const uint32_t jj = (uint32_t)(base + i);
      if (jj < m) {
        while (jj >= next) {  // the next split (empty splits are skipped)
          ++sp;
          start = next;
          next = sp + 1 < a.splits ? offs[sp + 1] : m;
        }
        v[i] = rs[sp * region + (jj - start)];  // (block << 32) | score bits
      }
    }
    uint32_t key[EPT];
    int32_t id[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
      const bool ok = (uint32_t)(base + i) < m;
      key[i] = ok ? ordered_key(__uint_as_float((uint32_t)v[i])) : 0u;
      id[i] = ok ? (int32_t)(v[i] >> 32) : 0;
    }
    uint32_t thr;
    int r;
    bool resolved;
    radix_kth_regs<EPT>(key, (int)m, a.top_k, sh, thr, r, resolved);
    emit_regs<EPT>(key, id, (int)m, thr, r, sel_row, a.top_k, sh);
  } else {
    // survivors overflowed their slots or the select's LDS, or the sampled
    // threshold kept fewer than k: the row is listed for the exact
    // fallback (pidx_fallback_kernel)
    if (threadIdx.x == 0) {
      const uint32_t i = atomicAdd(a.fb_cnt, 1u);
      a.fb_list[i] = rl;
    }
    return;
  }
  if (threadIdx.x == 0) a.n_sel[row] = a.top_k;
}

// LDS of the exact fallback: one chunk of recomputed keys and its pages.
struct FallbackShared {
  uint32_t keys[kChunk];
  int32_t pages[kChunk];
  uint32_t wcnt[kSelWaves];
};

// The exact fallback of one row.  tau_low = the k-th largest key of the
// row's union of group maxima is a lower bound of the row's k-th key (the
// union holds distinct keys of the row, so at least k keys reach it).  One
// streaming pass recomputes the row's keys chunk by chunk with the decode
// indexer's vector path (chunk_scores: same exact scores), keeps the keys
// >= tau_low with their block ids in block order -- in the row's own
// survivor region, free once the row is listed -- and the exact radix
// select and ordered emission pick the k best.  Returns false (nothing
// written) when more keys reach tau_low than the region holds, or fewer
// than k do.
template <int DI>
__device__ bool fallback_row(const PIdxArgs& a, int rl, int row, int n, int32_t* sel_row,
                             FallbackShared& fs, SelShared& sh) {
  const int seq = a.idx.seq_of(row);
  const int s = max(a.row_stride[rl], 1);
  const int n_groups = (n + kPGrp - 1) / kPGrp;
  const int un = min(kPUnion, ((n_groups + s - 1) / s) * 16);
  uint32_t tau = 1u;  // a union smaller than k bounds nothing: every key is kept
  if (un >= a.top_k) {
    constexpr int EPT = kPUnion / kSelThreads;
    const uint32_t* src = a.uni + (int64_t)rl * kPUnion + threadIdx.x * EPT;
    uint32_t key[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) key[i] = src[i];
    int r;
    bool resolved;
    radix_kth_regs<EPT>(key, un, a.top_k, sh, tau, r, resolved);
    tau = max(tau, 1u);
  }
  // candidate (key, id) list in the row's survivor region: keys, then ids
  const int cap = min(kPSelCap, a.splits * (kPSurvCap / a.splits));
  uint32_t* ck = reinterpret_cast<uint32_t*>(a.surv + (int64_t)rl * a.splits * (kPSurvCap / a.splits));
  int32_t* cid = reinterpret_cast<int32_t*>(ck + cap);
  typename RowQuery<bf16_t, DI, 4>::type iq;
  load_row_query<bf16_t, DI, 4>(iq, a.idx, row);
  const int wave = threadIdx.x / kWave, lane = lane_id();
  int total = 0;
  for (int c0 = 0; c0 < n; c0 += kChunk) {
    chunk_scores<bf16_t, DI, 4>(a.idx, seq, n, c0, iq, fs.pages, fs.keys);  // ends with a barrier
    // wave w keeps keys [256 w, 256 w + 256) of the chunk, in order
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      cnt += (uint32_t)__popcll(ballot(fs.keys[wave * 256 + 64 * j + lane] >= tau));
    if (lane == 0) fs.wcnt[wave] = cnt;
    __syncthreads();
    int base = total, next = total;
#pragma unroll
    for (int w = 0; w < kSelWaves; ++w) {
      base += w < wave ? (int)fs.wcnt[w] : 0;
      next += (int)fs.wcnt[w];
    }
    if (next > cap) return false;  // uniform: every thread sees the same counts
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = wave * 256 + 64 * j + lane;
      const uint32_t kk = fs.keys[e];
      const bool hit = kk >= tau;
      const uint64_t m = ballot(hit);
      if (hit) {
        ck[base + (int)lanes_below(m)] = kk;
        cid[base + (int)lanes_below(m)] = c0 + e;
      }
      base += (int)__popcll(m);
    }
    total = next;
    __syncthreads();  // the chunk's LDS is reused by the next chunk
  }
  // the keys recomputed here come from the vector path, the bound from the
  // matrix-core keys: on inputs where the two round differently, fewer than
  // k keys may reach it (then the select over keys recomputed per pass)
  if (total < a.top_k) return false;
  // the list was written by this workgroup's threads through memory
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  uint32_t thr;
  int r;
  radix_kth(KeyArray{ck}, total, a.top_k, sh, thr, r);
  emit_topk(KeyArray{ck}, IdArray{cid}, total, thr, r, sel_row, a.top_k, sh);
  return true;
}

// P4's exact fallback for the rows the select kernels listed: a fixed grid
// of workgroups takes the listed rows in turn (the list is complete: the
// select kernel finished before this launch).  A row whose candidates do
// not fit its region takes the select over keys recomputed per pass.  The
// last workgroup to finish clears the list's counter for the next call.
template <int DI>
__global__ void __launch_bounds__(256) pidx_fallback_kernel(PIdxArgs a) {
  __shared__ FallbackShared fs;
  __shared__ SelShared sh;
  __shared__ uint32_t flag;
  const uint32_t count = ld_agent(a.fb_cnt);
  for (uint32_t i = blockIdx.x; i < count; i += gridDim.x) {
    const int rl = ld_agent(a.fb_list + i);
    const int row = a.row0 + rl;
    const int n = a.idx.pos_of(row) >> a.idx.pm.blk_shift;
    int32_t* sel_row = a.sel + (int64_t)row * a.top_k;
    if (!fallback_row<DI>(a, rl, row, n, sel_row, fs, sh)) {
      const PRecomputed<DI> get{&a, row, a.idx.seq_of(row)};
      uint32_t thr;
      int r;
      radix_kth(get, n, a.top_k, sh, thr, r);
      emit_topk(get, IdSelf{}, n, thr, r, sel_row, a.top_k, sh);
    }
    if (threadIdx.x == 0) a.n_sel[row] = a.top_k;
    __syncthreads();
  }
  if (arrive_last(a.fb_cnt + 1, gridDim.x, &flag) && threadIdx.x == 0) st_agent(a.fb_cnt, 0u);
}

bool pidx_supported(int dtype, int di, int hi) {
  return dtype == QSA_BF16 && (di == 64 || di == 128) && hi >= 1 && hi <= 4;
}

void run_pidx(const PIdxArgs& a, int di, hipStream_t st) {
  const int tiles = (a.rows + kPQT - 1) / kPQT;
  dim3 grid((unsigned)a.splits, (unsigned)tiles);
  const dim3 wave_grid((unsigned)((a.rows + 3) / 4));  // four rows (waves) per workgroup
  hipLaunchKernelGGL(pidx_stride_kernel, dim3(tiles), dim3(256), 0, st, a);
  if (di == 64) {
    hipLaunchKernelGGL((pidx_kernel<64, false>), grid, dim3(kPThreads), 0, st, a);
    hipLaunchKernelGGL(pidx_tau_wave_kernel, wave_grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((pidx_kernel<64, true>), grid, dim3(kPThreads), 0, st, a);
    hipLaunchKernelGGL(pidx_select_wave_kernel, wave_grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((pidx_select_kernel<64>), dim3(a.rows), dim3(256), 0, st, a);
    hipLaunchKernelGGL((pidx_fallback_kernel<64>), dim3(kPFallbackWgs), dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((pidx_kernel<128, false>), grid, dim3(kPThreads), 0, st, a);
    hipLaunchKernelGGL(pidx_tau_wave_kernel, wave_grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((pidx_kernel<128, true>), grid, dim3(kPThreads), 0, st, a);
    hipLaunchKernelGGL(pidx_select_wave_kernel, wave_grid, dim3(256), 0, st, a);
    hipLaunchKernelGGL((pidx_select_kernel<128>), dim3(a.rows), dim3(256), 0, st, a);
    hipLaunchKernelGGL((pidx_fallback_kernel<128>), dim3(kPFallbackWgs), dim3(256), 0, st, a);
  }
}

}  // namespace qsa
