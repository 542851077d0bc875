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
//     k-slots); A = V^T, read with ds_read_b64_tr_b16 from an LDS copy of
//     the tile's V rows.  A product with a ones operand sums the
//     numerators (the softmax denominator) on the matrix core as well.
//
// Workgroups: the SPLIT instances (few rows) run 8 waves per (row, split),
// waves w and w + Hkv on the same KV head; the split partials go to the
// workspace and the last split of the row merges them.  The per-row
// instances (many rows) run 4 waves per (row, KV head): workgroup
// row * Hkv + head, so that with the round-robin placement of workgroups on
// the 8 XCDs (Hkv dividing 8) every XCD serves one KV head only, and its L2
// holds twice as many blocks of that head as it would of both.  The PAIR
// instances serve two neighbouring rows per workgroup (pair * Hkv + head):
// the query heads of both rows fill the 16 product columns, a block both
// rows list is staged once, and each staged token carries a visibility bit
// per row, so every tile masks by column.
#include <type_traits>

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
// then (m in log2 units, l)), are written and merged by the NT threads of a
// workgroup, each owning one head and D/(NT/16) contiguous dims of it
// (hq <= 16).
template <int D, int NT>
struct MergeLane {
  static constexpr int LPH = NT / 16;  // threads per head
  static constexpr int ND = D / LPH;   // dims per thread
  int h, d0;
  bool on;
  __device__ MergeLane(int hq) : h(threadIdx.x / LPH), d0((threadIdx.x % LPH) * ND), on(h < hq) {}
};

__device__ __forceinline__ uint64_t pack2(float lo, float hi) {
  return (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
}
__device__ __forceinline__ float lo_f(uint64_t v) { return __uint_as_float((uint32_t)v); }
__device__ __forceinline__ float hi_f(uint64_t v) { return __uint_as_float((uint32_t)(v >> 32)); }

// Merge of a row's split partials, run by the last split workgroup after its
// acquire.  Each thread keeps a running (M, L, O[ND]) for its head and dims.
// Per batch of kMergeBatch splits, lane j of a head's LPH threads loads the
// (m, l) pair of split j once and the group shares it by lane shuffles,
// each thread loads its ND floats of every split in one or two 16-byte
// loads, and the next batch's loads are in flight while the current batch
// is folded in.
template <int D, int NT>
__device__ void merge_splits(const AttnArgs& a, int row, bf16_t* orow) {
  constexpr int ND = MergeLane<D, NT>::ND;
  constexpr int LPH = MergeLane<D, NT>::LPH;
  constexpr int NV = ND / 4 > 0 ? ND / 4 : 1;  // 16-byte loads per split (8-byte if ND == 2)
  constexpr int kMergeBatch = 16;
  static_assert(LPH >= kMergeBatch, "a head's threads hold one batch of (m, l) pairs");
  static_assert(ND == 2 || ND % 4 == 0, "dims per thread");
  const MergeLane<D, NT> ml(a.hq);
  if (!ml.on) return;  // whole head groups leave together
  const int S = a.n_splits, hq = a.hq;
  const int j = (int)threadIdx.x % LPH;                  // lane within the head's group
  const int gbase = (lane_id() / LPH) * LPH;             // the group's first lane
  const int64_t rb = (int64_t)row * S * hq;
  const uint64_t* pml = reinterpret_cast<const uint64_t*>(a.part_ml) + rb + ml.h;
  const float* pacc = a.part_acc + (rb + ml.h) * D + ml.d0;
  const int64_t acc_step = (int64_t)hq * D;  // floats per split
  float M = -INFINITY, L = 0.0f, O[ND];
#pragma unroll
  for (int q = 0; q < ND; ++q) O[q] = 0.0f;
  uint64_t cm;              // (m, l) of split s0 + j of the batch
  float cv[kMergeBatch][ND];
  auto load = [&](int s0) {
    cm = (j < kMergeBatch && s0 + j < S) ? pml[(int64_t)(s0 + j) * hq] : pack2(-INFINITY, 0.0f);
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const bool ok = s0 + u < S;
      const float* src = pacc + (int64_t)(s0 + u) * acc_step;
      if constexpr (ND == 2) {
        const float2 v = ok ? *reinterpret_cast<const float2*>(src) : make_float2(0.f, 0.f);
        cv[u][0] = v.x;
        cv[u][1] = v.y;
      } else {
#pragma unroll
        for (int q = 0; q < NV; ++q) {
          const float4 v = ok ? *reinterpret_cast<const float4*>(src + 4 * q)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
          cv[u][4 * q] = v.x;
          cv[u][4 * q + 1] = v.y;
          cv[u][4 * q + 2] = v.z;
          cv[u][4 * q + 3] = v.w;
        }
      }
    }
  };
  load(0);
  for (int s0 = 0; s0 < S; s0 += kMergeBatch) {
    const uint64_t bm_own = cm;
    float bv[kMergeBatch][ND];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u)
#pragma unroll
      for (int q = 0; q < ND; ++q) bv[u][q] = cv[u][q];
    if (s0 + kMergeBatch < S) load(s0 + kMergeBatch);
    // the batch's (m, l) pairs, from the lanes that loaded them
    float bm[kMergeBatch], bl[kMergeBatch];
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      bm[u] = __shfl(lo_f(bm_own), gbase + u);
      bl[u] = __shfl(hi_f(bm_own), gbase + u);
    }
    float Mc = M;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) Mc = fmaxf(Mc, bm[u]);
    if (Mc == -INFINITY) continue;  // nothing attended yet
    const float rs = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mc);
    L *= rs;
#pragma unroll
    for (int q = 0; q < ND; ++q) O[q] *= rs;
#pragma unroll
    for (int u = 0; u < kMergeBatch; ++u) {
      const float f = (bm[u] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(bm[u] - Mc);
      L = fmaf(bl[u], f, L);
#pragma unroll
      for (int q = 0; q < ND; ++q) O[q] = fmaf(bv[u][q], f, O[q]);
    }
    M = Mc;
  }
  const float inv = 1.0f / L;
  bf16_t* o = orow + ml.h * D + ml.d0;
#pragma unroll
  for (int q = 0; q < ND; ++q) o[q] = f32_to_bf16(O[q] * inv);
}

// K/V row offsets are kept as 32-bit byte offsets while both arrays are
// smaller than this; larger caches take the WIDE instances, which keep row
// indices and form 64-bit addresses.
constexpr int64_t kNarrowCacheBytes = (1ll << 32) - (1ll << 16);

typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// Waves per workgroup: 4, or 8 for the split instances (few rows: twice the
// entries per split, half the partials to merge).
template <bool SPLIT>
constexpr int attn_waves() { return SPLIT ? 8 : 4; }

template <int D, bool DENSE, bool SPLIT, bool WIDE, bool PAIR>
__global__ void __launch_bounds__(attn_waves<SPLIT>() * 64, SPLIT ? 2 : 3)
    attn_mfma_kernel(AttnArgs a) {
  constexpr int NW = attn_waves<SPLIT>(), NT = NW * kWave;
  constexpr int NDT = D / 16;  // 16-wide d tiles of the output
  constexpr int KS = D / 32;   // 32-wide k steps of Q.K
  // LDS bytes per staged V row: 32 bytes more than the row, so that the 8
  // rows one half-wave reads in a transposing load start 8 banks apart
  constexpr int VP = 2 * D + 32;
  // K rows are staged unpadded, 16-byte chunk c of tile row r at chunk
  // position c ^ (r mod NCH): the 16 rows of one A-fragment read, all at
  // the same chunk, then fall on distinct banks
  constexpr int KP = 2 * D, NCH = D / 8;
  constexpr int kStage = NW * kMfmaTileTok * (VP + KP);  // per-wave K and V tiles
  constexpr int kMerge = NW * 16 * (D + 2) * 4;         // per-wave results
  // The token rows of the staged list, tile by tile: token p of the list
  // (the tokens of its blocks in list order) is tile row 4i + j of tile
  // p / 16, i = (p % 16) / 4, j = p % 4, kept as [j][i]; each value is the
  // byte offset of the token's row in the K and V arrays (WIDE: its row
  // index).  Tokens not to attend point at the row's own first token.
  __shared__ __align__(16) uint32_t trow[kMfmaListTok];
  __shared__ __align__(16) unsigned char lds[kStage > kMerge ? kStage : kMerge];
  __shared__ int wcnt[NW];
  __shared__ uint32_t flag;
  // PAIR: the union of the two rows' entry lists (block ids and which rows
  // list them: bit 0 row A, bit 1 row B) and each staged token's visibility
  // (the same bits)
  __shared__ int32_t ublk[PAIR ? kPairCap : 1];
  __shared__ uint8_t umem[PAIR ? kPairCap : 4];
  __shared__ __align__(4) uint8_t tmask[PAIR ? kMfmaListTok : 4];
  // the wave index is uniform: read it once so that what derives from it
  // (the KV head, the wave's tiles, the cache base) stays scalar
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int l = lane_id(), g = l / 16, c16 = l % 16;
  const int hkv = a.hkv, hq = a.hq, G = hq / hkv;
  // one KV head per workgroup (per-row instances) or Hkv of them (SPLIT)
  const int wph = SPLIT ? NW / hkv : NW;  // waves per KV head
  const int hk = SPLIT ? w % hkv : (int)(blockIdx.x % (unsigned)hkv);
  const int wsub = SPLIT ? w / hkv : w;
  const int row =
      SPLIT ? (int)blockIdx.y : (int)(blockIdx.x / (unsigned)hkv) * (PAIR ? 2 : 1);
  const int split = SPLIT ? (int)blockIdx.x : 0;
  // PAIR: rows row (A) and row + 1 (B, if present) share the workgroup
  const int rowB = row + 1;
  const bool hasB = PAIR && rowB < a.n_rows;

  // the reads that depend on the row index alone, issued together so that
  // their latencies overlap: sequence, position, selection length, and the
  // first selected id this thread stages (a selection row always holds
  // top_k entries; used only when the row attends its own selection)
  const int e_beg = split * a.eps;
  const int sid_raw = a.seq_id[row];
  const int pos_raw = a.pos[row];
  const int nsel_raw = DENSE ? 0 : a.n_sel[row];
  const int32_t pre =
      DENSE ? -1 : a.sel[(int64_t)row * a.top_k + min(e_beg + (int)threadIdx.x, a.top_k - 1)];
  const int sidB_raw = hasB ? a.seq_id[rowB] : 0;
  const int posB_raw = hasB ? a.pos[rowB] : 0;
  const int nselB_raw = hasB ? a.n_sel[rowB] : 0;
  const int seq = clamp_flag(sid_raw, 0, a.n_seqs - 1, QSA_DEBUG_BAD_ROW);
  const int t = clamp_flag(pos_raw, 0, a.max_pos, QSA_DEBUG_BAD_ROW);
  const RowList rl(a, row, t, DENSE, nsel_raw);
  const int seqB = clamp_flag(sidB_raw, 0, a.n_seqs - 1, QSA_DEBUG_BAD_ROW);
  const int tB = clamp_flag(posB_raw, 0, a.max_pos, QSA_DEBUG_BAD_ROW);
  const int b_own = rl.b_own;
  const int n_entries = rl.e_own + 1;
  const int e_end = min(n_entries, e_beg + a.eps);
  const int bs = a.pm.blk_shift, nb = 1 << bs;  // tokens per block
  const int tail = (t & (nb - 1)) + 1;        // tokens of the own block
  const int epp = kMfmaListTok >> bs;  // entries staged per pass

  const unsigned char* kbase = static_cast<const unsigned char*>(a.k) + hk * D * 2;
  const unsigned char* vbase = static_cast<const unsigned char*>(a.v) + hk * D * 2;
  const int64_t rowbytes = (int64_t)hkv * D * 2;
  const int64_t own_row = a.pm.token_slot(seq, b_own << bs);  // always present
  const uint32_t own_t = WIDE ? (uint32_t)own_row : (uint32_t)(own_row * rowbytes);
  const int cv = c16 < D / 8 ? c16 : 0;
  const uint32_t lane_c = 16 * cv;  // 16-byte chunk cv of a K or V row

  // this lane's B fragment of Q^T: head c16 of the group, dims 32 s + 8 g
  // .. +8 at step s (K uses the same order, so one load instruction reads
  // 64 contiguous bytes of each token row)
  // (PAIR: columns G .. 2G - 1 hold row B's heads)
  const bool colB = PAIR && c16 >= G;
  const uint32_t colbit = !PAIR ? 0u : (c16 < G ? 1u : (c16 < 2 * G ? 2u : 0u));
  u32x4_t qf[KS];
  {
    const bool qok = c16 < G || (colB && c16 < 2 * G && hasB);
    const int64_t qr = colB ? rowB : row;
    const bf16_t* qh =
        static_cast<const bf16_t*>(a.q) + (qr * hq + hk * G + (colB ? c16 - G : c16)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s)
      qf[s] = qok ? ld16(qh + 32 * s + 8 * g) : u32x4_t{0u, 0u, 0u, 0u};
  }
  // Online softmax per head column.  Scores stay raw (q.k); the reference
  // maximum m is kept raw and as m * scale * log2(e), and moves only when a
  // score exceeds it by kSlack in log2 units (mlim, raw).
  const float sl2 = a.scale * 1.4426950408889634f;
  const float slack_raw = kSlack / sl2;
  float m_raw = -INFINITY, msl2 = -INFINITY, mlim = -INFINITY;
  f32x4_t acc[NDT];
#pragma unroll
  for (int n = 0; n < NDT; ++n) acc[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  f32x4_t lacc = f32x4_t{0.f, 0.f, 0.f, 0.f};  // softmax denominator, via a ones operand
  const u32x2_t ones = {0x3F803F80u, 0x3F803F80u};  // bfloat16 1.0 x 4
  unsigned char* vs = lds + w * kMfmaTileTok * (VP + KP);
  unsigned char* ks = vs + kMfmaTileTok * VP;
  // transposing read of V^T (see the O^T step): the lane supplies the
  // address of tile row 4g + c16/4, dims 16n + 4(c16 % 4) .. +4
  const uint32_t tr_off = (4 * g + c16 / 4) * VP + 8 * (c16 % 4);
  // K A-fragment reads: row c16, chunk 4s + g (dims 32s + 8g .. +8, the
  // order of the Q fragments)
  const uint32_t kr_off = c16 * KP;

  // list token p -> its place in trow
  auto tslot = [](int p) { return (p >> 4) * 16 + ((p & 3) << 2) + ((p & 15) >> 2); };
  int ntok = 0;  // tokens staged by the current pass
  // A tile is 16 tokens, tile row 4i + j = entry i, token j.  The K and
  // V rows of the wave's next tile are loaded while the current one is
  // computed, both the same way: load i reads entry i, lane group g its
  // token g, lane c16 its 16-byte chunk, so that 16 lanes read a whole
  // row (whole cache lines; the MFMA operand order, 64 bytes of 16 rows
  // per load, costs the vector cache about twice as much).  Every load
  // reads a row present in the cache (masked tokens read the own block's
  // first token).
  auto load_tile = [&](int tile, u32x4_t (&kf)[4], u32x4_t (&vf)[4]) {
    const u32x4_t tv = *reinterpret_cast<const u32x4_t*>(trow + tile * 16 + 4 * g);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (WIDE) {
        const int64_t o = (int64_t)tv[i] * rowbytes + lane_c;
        kf[i] = *reinterpret_cast<const u32x4_t*>(kbase + o);
        vf[i] = *reinterpret_cast<const u32x4_t*>(vbase + o);
      } else {
        const uint32_t o = tv[i] + lane_c;
        kf[i] = *reinterpret_cast<const u32x4_t*>(kbase + o);
        vf[i] = *reinterpret_cast<const u32x4_t*>(vbase + o);
      }
    }
  };
  // one tile: S^T, online softmax, O^T update.  Only the last tile of
  // the chunk can hold tokens not to attend (the own block's tail, the
  // padding), so only it masks.
  // (masked: wave-uniform, true for the last tile of a pass only)
  auto compute = [&](bool masked, int tile, const u32x4_t (&kf)[4], const u32x4_t (&vf)[4]) {
    // K and V rows to LDS (row 4i + g)
    if (c16 < D / 8) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 4 * i + g;
        *reinterpret_cast<u32x4_t*>(ks + r * KP + 16 * (cv ^ (r % NCH))) = kf[i];
        *reinterpret_cast<u32x4_t*>(vs + (4 * i + g) * VP + 16 * c16) = vf[i];
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // S^T: lane holds tile tokens 4g + r (entry g, token r) for head c16
    f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s2 = 0; s2 < KS; ++s2) {
      const u32x4_t kfr = *reinterpret_cast<const u32x4_t*>(
          ks + kr_off + 16 * ((4 * s2 + g) ^ (c16 % NCH)));
      sc = mfma16(kfr, qf[s2], sc);
    }
    float x[4];
    if constexpr (PAIR) {
      // the column's row sees token 4g + r of the tile
      const uint32_t mk = *reinterpret_cast<const uint32_t*>(tmask + tile * 16 + 4 * g);
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = ((mk >> (8 * r)) & colbit) ? sc[r] : -INFINITY;
    } else if (masked) {
      const int p0 = tile * 16 + 4 * g;  // list token of row r: p0 + r
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = p0 + r < ntok ? sc[r] : -INFINITY;
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) x[r] = sc[r];
    }
    const float mx = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    if (__ballot(mx > mlim) != 0ull) {
      // the column's maximum over the four lane groups (rows 16 apart,
      // then 32 apart)
      float cm = mx;
      {
        const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(cm), __float_as_uint(cm),
                                                        false, false);
        cm = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      {
        const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(cm), __float_as_uint(cm),
                                                        false, false);
        cm = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
      }
      if (cm > mlim) {
        const float msl2_new = cm * sl2;
        const float corr = __builtin_amdgcn_exp2f(msl2 - msl2_new);  // 0 while msl2 = -inf
        lacc = lacc * corr;
#pragma unroll
        for (int n = 0; n < NDT; ++n) acc[n] = acc[n] * corr;
        m_raw = cm;
        msl2 = msl2_new;
        mlim = m_raw + slack_raw;
      }
    }
    // (PAIR: a column whose row has seen no token yet has msl2 = -inf and
    // only masked scores; 0 in place of -msl2 keeps their numerators 0)
    const float nm = (PAIR && msl2 == -INFINITY) ? 0.0f : -msl2;
    float p[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(fmaf(x[r], sl2, nm));
    const u32x2_t pb = {cvt_pk_bf16(p[0], p[1]), cvt_pk_bf16(p[2], p[3])};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    // O^T += V^T . P^T.  A lane's k-slots j are tile tokens 4g + j
    // (where S^T left them); the transposing LDS read gives lane (g, c16)
    // V[4g + j][16n + c16], j = 0..3.
#pragma unroll
    for (int n = 0; n < NDT; ++n) {
      const s16x4_t v4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4_t*)(vs + tr_off + 32 * n));
      acc[n] = mfma16k16(__builtin_bit_cast(u32x2_t, v4), pb, acc[n]);
    }
    lacc = mfma16k16(ones, pb, lacc);
    __builtin_amdgcn_wave_barrier();
  };
  // the current pass's tiles, split among the waves of the KV head
  auto run_tiles = [&]() {
    const int n_tiles = (ntok + 15) / 16;
    const int last = n_tiles - 1;
    // The wave's tiles are wsub + q * wph, q < nmine; the last tile of the
    // pass (masked) is its owner's last.  Two register sets alternate: the
    // loads of the next tile go to the set not being computed (past the end
    // a wave reloads its last tile, so every step issues the same loads and
    // the wait before a product covers only the current tile's).  One loop
    // shape for every tile, the last included, keeps both sets in registers.
    const int nmine = wsub < n_tiles ? (last - wsub) / wph + 1 : 0;
    const bool has_last = nmine > 0 && wsub + (nmine - 1) * wph == last;
    auto T = [&](int q) { return wsub + min(q, nmine - 1) * wph; };
    u32x4_t kA[4], vA[4], kB[4], vB[4];
    if (nmine > 0) {
      load_tile(T(0), kA, vA);
      for (int q = 0; q < nmine; q += 2) {
        load_tile(T(q + 1), kB, vB);
        compute(has_last && q == nmine - 1, T(q), kA, vA);
        if (q + 1 < nmine) {
          load_tile(T(q + 2), kA, vA);
          compute(has_last && q + 1 == nmine - 1, T(q + 1), kB, vB);
        }
      }
    }
  };
  if constexpr (!PAIR) {
    for (int cb = e_beg; cb < e_end; cb += epp) {
      const int nloc = min(e_end, cb + epp) - cb;
      __syncthreads();
      // Stage the valid entries of [cb, cb + nloc) at the front, in list
      // order (a block-wide prefix count of the valid flags), so that every
      // tile but the last holds only tokens to attend.  The own block is the
      // last entry of the list, hence the last valid entry of its chunk.
      int nv = 0;
      for (int i0 = 0; i0 < nloc; i0 += NT) {
        const int i = i0 + (int)threadIdx.x;
        const int E = cb + i;
        const bool own = (E == rl.e_own);
        bool ok = i < nloc;
        int b = b_own;
        if (ok && !own) {
          if (!DENSE && rl.own_sel && cb == e_beg && i0 == 0 && E < rl.n_list) {
            b = pre;
            ok = b >= 0 && b < rl.b_sel;
            if (!ok) debug_flag(QSA_DEBUG_BAD_SEL);
          } else {
            b = rl.block(E, DENSE, ok);
          }
        }
        const uint64_t bal = __ballot(ok);
        if (l == 0) wcnt[w] = __popcll(bal);
        __syncthreads();
        int pos = nv + (int)lanes_below(bal), tot = nv;
  #pragma unroll
        for (int j = 0; j < NW; ++j) {
          const int c = wcnt[j];
          pos += j < w ? c : 0;
          tot += c;
        }
        if (ok) {
          const int64_t r0 = a.pm.token_slot(seq, b << bs);
          const int nt = own ? tail : nb;
          const int p0 = pos << bs;
          if (nb == 4) {  // QSA blocks: four stores, no loop
  #pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int64_t r = j < nt ? r0 + j : own_row;
              trow[tslot(p0 + j)] = WIDE ? (uint32_t)r : (uint32_t)(r * rowbytes);
            }
          } else {
            for (int j = 0; j < nt; ++j) {
              const int64_t r = r0 + j;
              trow[tslot(p0 + j)] = WIDE ? (uint32_t)r : (uint32_t)(r * rowbytes);
            }
          }
        }
        nv = tot;
        __syncthreads();
      }
      const bool own_here = rl.e_own >= cb && rl.e_own < cb + nloc;
      // tokens to attend: whole blocks, the own block's tail last
      ntok = own_here ? ((nv - 1) << bs) + tail : (nv << bs);
      for (int p = ntok + (int)threadIdx.x; p < ((ntok + 15) & ~15); p += NT) trow[tslot(p)] = own_t;
      __syncthreads();
      run_tiles();
    }
  } else {
    // Both rows' entry lists (selected blocks, then the own block; invalid
    // ids as -1) go to la and lb in the K/V staging area, which no tile
    // uses yet.
    int32_t* la = reinterpret_cast<int32_t*>(lds);
    int32_t* lb = la + kPairHalf;
    const RowList rlB(a, hasB ? rowB : row, hasB ? tB : t, false, hasB ? nselB_raw : 0);
    const int nA = rl.n_list + 1;
    const int nB = hasB ? rlB.n_list + 1 : 0;
    bool ok = true;  // this thread's entries are valid and ascending
    for (int e = (int)threadIdx.x; e < nA; e += NT) {
      bool v = true;
      const int b = e < rl.n_list ? rl.block(e, false, v) : b_own;
      la[e] = v ? b : -1;
      ok = ok && v;
    }
    for (int e = (int)threadIdx.x; e < nB; e += NT) {
      bool v = true;
      const int b = e < rlB.n_list ? rlB.block(e, false, v) : rlB.b_own;
      lb[e] = v ? b : -1;
      ok = ok && v;
    }
    __syncthreads();
    for (int e = (int)threadIdx.x + 1; e < nA; e += NT) ok = ok && la[e - 1] < la[e];
    for (int e = (int)threadIdx.x + 1; e < nB; e += NT) ok = ok && lb[e - 1] < lb[e];
    // one sequence, both lists valid and strictly ascending: a block both
    // rows list is staged once (else the lists are staged one after the
    // other, each block for its own row)
    const bool share = (__syncthreads_and(ok ? 1 : 0) != 0) && hasB && seqB == seq;
    auto listed = [](const int32_t* v, int n, int x) {  // x in ascending v[0, n)
      int lo = 0, hi = n;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (v[mid] < x) lo = mid + 1; else hi = mid;
      }
      return lo < n && v[lo] == x;
    };
    // the union: row A's entries, then those of row B's that A does not list
    for (int e = (int)threadIdx.x; e < nA; e += NT) {
      const int b = la[e];
      ublk[e] = b;
      umem[e] = b < 0 ? 0 : (uint8_t)(1u | ((share && listed(lb, nB, b)) ? 2u : 0u));
    }
    int nU = nA;
    for (int i0 = 0; i0 < nB; i0 += NT) {
      const int e = i0 + (int)threadIdx.x;
      const bool keep = e < nB && !(share && listed(la, nA, lb[e]));
      const uint64_t bal = __ballot(keep);
      if (l == 0) wcnt[w] = __popcll(bal);
      __syncthreads();
      int pos = nU + (int)lanes_below(bal), tot = nU;
#pragma unroll
      for (int j = 0; j < NW; ++j) {
        const int c = wcnt[j];
        pos += j < w ? c : 0;
        tot += c;
      }
      if (keep) {
        ublk[pos] = lb[e];
        umem[pos] = lb[e] < 0 ? 0 : 2;
      }
      nU = tot;
      __syncthreads();
    }
    // Passes of epp union entries: every token of an entry is staged with
    // its visibility (the row lists the block and the token is at or before
    // the row's position: the own blocks' tails); invisible tokens read
    // row A's own first token.  All tiles mask by column.
    for (int cb = 0; cb < nU; cb += epp) {
      const int nloc = min(nU, cb + epp) - cb;
      __syncthreads();  // the previous pass's tiles (or the union's reads) are done
      for (int i = (int)threadIdx.x; i < nloc; i += NT) {
        const int b = ublk[cb + i];
        const uint32_t m = umem[cb + i];
        const int64_t r0 = m ? a.pm.token_slot((m & 1u) ? seq : seqB, b << bs) : own_row;
        for (int j = 0; j < nb; ++j) {
          const int pt = (b << bs) + j;
          const uint32_t vis =
              (((m & 1u) && pt <= t) ? 1u : 0u) | (((m & 2u) && pt <= tB) ? 2u : 0u);
          const int64_t r = vis ? r0 + j : own_row;
          trow[tslot((i << bs) + j)] = WIDE ? (uint32_t)r : (uint32_t)(r * rowbytes);
          tmask[(i << bs) + j] = (uint8_t)vis;
        }
      }
      ntok = nloc << bs;
      for (int p = ntok + (int)threadIdx.x; p < ((ntok + 15) & ~15); p += NT) {
        trow[tslot(p)] = own_t;
        tmask[p] = 0;
      }
      __syncthreads();
      run_tiles();
    }
  }
  const float lsum = lacc[0];  // every row of the ones product is the column sum
  __syncthreads();
  // per-wave results to LDS: [wave][head][D + 2] (acc, then m, l)
  float* mrg = reinterpret_cast<float*>(lds);
  if (c16 < (PAIR ? 2 * G : G)) {
    float* o = mrg + (w * 16 + c16) * (D + 2);
#pragma unroll
    for (int n = 0; n < NDT; ++n)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[16 * n + 4 * g + i] = acc[n][i];
    if (g == 0) {
      o[D] = msl2;
      o[D + 1] = lsum;
    }
  }
  __syncthreads();
  bf16_t* orow = static_cast<bf16_t*>(a.out) + (int64_t)row * hq * D;
  // combine the waves of each KV head: thread = (head, its dims); lane.h is
  // the query head (SPLIT) or the head within this workgroup's group
  const MergeLane<D, NT> lane(SPLIT ? hq : (PAIR ? 2 * G : G));
  constexpr int ND = MergeLane<D, NT>::ND;
  if (lane.on) {
    const int hk_ = SPLIT ? lane.h / G : 0, hh = SPLIT ? lane.h % G : lane.h;
    const int wstride = SPLIT ? hkv : 1;  // wave j of the head: hk_ + j * wstride
    float M = -INFINITY;
    for (int j = 0; j < wph; ++j) M = fmaxf(M, mrg[((hk_ + j * wstride) * 16 + hh) * (D + 2) + D]);
    float L = 0.0f, O[ND];
#pragma unroll
    for (int i = 0; i < ND; ++i) O[i] = 0.0f;
    for (int j = 0; j < wph; ++j) {
      const float* o = mrg + ((hk_ + j * wstride) * 16 + hh) * (D + 2);
      const float f = (o[D] == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(o[D] - M);
      L = fmaf(o[D + 1], f, L);
#pragma unroll
      for (int i = 0; i < ND; ++i) O[i] = fmaf(o[lane.d0 + i], f, O[i]);
    }
    if constexpr (!SPLIT) {
      const float inv = 1.0f / L;
      const bool isB = PAIR && lane.h >= G;  // a column of row B
      if (!isB || hasB) {
        bf16_t* oh = (isB ? orow + hq * D : orow) + (hk * G + (isB ? lane.h - G : lane.h)) * D +
                     lane.d0;
#pragma unroll
        for (int i = 0; i < ND; ++i) oh[i] = f32_to_bf16(O[i] * inv);
      }
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
    merge_splits<D, NT>(a, row, orow);
  }
}

bool attn_mfma_supported(int dtype, int hq, int hkv, int d) {
  return dtype == QSA_BF16 && (d == 64 || d == 128) && (hkv == 1 || hkv == 2 || hkv == 4) &&
         hq % hkv == 0 && hq <= 16;
}

void run_attention_mfma(const AttnArgs& a, int d, bool dense, int n_rows, hipStream_t st) {
  const bool split = a.n_splits > 1;
  // rows in pairs: a selection of at most kPairHalf - 1 blocks each, the
  // query heads of both rows in the 16 product columns
  const bool pair = !dense && !split && a.sel_of == nullptr && 2 * (a.hq / a.hkv) <= 16 &&
                    a.top_k + 1 <= kPairHalf && n_rows >= 2;
  // SPLIT: (split, row); per row (pair): one workgroup per (row or pair, KV head)
  const dim3 grid = split ? dim3((unsigned)a.n_splits, (unsigned)n_rows)
                          : dim3((unsigned)(pair ? (n_rows + 1) / 2 : n_rows) * (unsigned)a.hkv);
  const bool wide = a.n_slots * a.hkv * d * 2 > kNarrowCacheBytes;
#define QSA_ATTN_LAUNCH(DD, DN, SP, WD, PR) \
  hipLaunchKernelGGL((attn_mfma_kernel<DD, DN, SP, WD, PR>), grid, dim3(attn_waves<SP>() * 64), 0, \
                     st, a)
#define QSA_ATTN_LAUNCH_W(DD, DN, SP) \
  if (wide) QSA_ATTN_LAUNCH(DD, DN, SP, true, false); else QSA_ATTN_LAUNCH(DD, DN, SP, false, false)
#define QSA_ATTN_LAUNCH_P(DD) \
  if (wide) QSA_ATTN_LAUNCH(DD, false, false, true, true); \
  else QSA_ATTN_LAUNCH(DD, false, false, false, true)
  if (d == 128) {
    if (dense) {
      if (split) { QSA_ATTN_LAUNCH_W(128, true, true); } else { QSA_ATTN_LAUNCH_W(128, true, false); }
    } else {
      if (split) { QSA_ATTN_LAUNCH_W(128, false, true); }
      else if (pair) { QSA_ATTN_LAUNCH_P(128); }
      else { QSA_ATTN_LAUNCH_W(128, false, false); }
    }
  } else {
    if (dense) {
      if (split) { QSA_ATTN_LAUNCH_W(64, true, true); } else { QSA_ATTN_LAUNCH_W(64, true, false); }
    } else {
      if (split) { QSA_ATTN_LAUNCH_W(64, false, true); }
      else if (pair) { QSA_ATTN_LAUNCH_P(64); }
      else { QSA_ATTN_LAUNCH_W(64, false, false); }
    }
  }
#undef QSA_ATTN_LAUNCH_P
#undef QSA_ATTN_LAUNCH_W
#undef QSA_ATTN_LAUNCH
}

}  // namespace qsa
