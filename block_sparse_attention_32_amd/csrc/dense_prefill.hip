// Dense causal GQA flash attention for many query rows (the comparison
// baseline of the sparse prefill; keieiax.jp glossary "Qwen Sparse
// Attention", section 長文AIのコストと応答時間にどう影響する？: the reference
// point is dense grouped-query attention).
//
// Same result as attn_mfma_kernel<D, true, false> (every token 0..pos of
// the row's sequence, softmax(scale q.k) v, fp32 accumulation, round to
// nearest-even), organised for many rows: a workgroup (8 waves) owns 256
// query vectors -- (row, head) pairs of one KV head, G = Hq/Hkv heads per
// row, so 256/G consecutive rows -- and walks the KV tokens 64 at a time.
// Each 64-token tile of K and V (both row-major) is staged in LDS once for
// all 256 vectors, double-buffered: the next tile's global loads are in
// flight while the current tile is computed.
//
// Per wave: 32 query vectors (two 16-column groups).
//   S^T[64 tok x 16 vec] = K[64 x D] . Q^T       v_mfma_f32_16x16x32_bf16
//     A = K rows from LDS, B = the query vectors held in registers
//   O^T[D x 16 vec] += V^T[D x 64 tok] . P^T     v_mfma_f32_16x16x32_bf16
//     B = the softmax numerators in the registers where S^T left them (the
//     32 contraction slots of lane group g are tokens 4g..4g+3 of two
//     16-token tiles); A = V^T in that order, read from the row-major V
//     tile with the gfx950 transposing LDS read ds_read_b64_tr_b16
// Online softmax in log2 units; the sum of the numerators is one more
// product on the matrix core (a ones operand against the same bf16
// numerators the O^T product uses).
#include <type_traits>

#include "attention.hpp"

namespace qsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kFTok = 64;                     // KV tokens per tile
constexpr int kFNC = 2;                       // 16-vector column groups per wave
constexpr int kFWaves = 8;
constexpr int kFThreads = kFWaves * 64;
constexpr int kFVec = kFWaves * kFNC * 16;    // query vectors per workgroup

__device__ __forceinline__ f32x4_t mfma(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// two floats -> packed bfloat16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}
// A column's reference maximum only moves when a score exceeds it by more
// than this (log2 units); numerators stay below 2^kSlack and share the
// reference with their sum, so the result does not depend on it.
constexpr float kSlack = 8.0f;

template <int D>
struct FGeom {
  static constexpr int KS = D / 32;               // k steps of Q.K
  static constexpr int NDT = D / 16;              // 16-dim tiles of the output
  static constexpr int KPITCH = D * 2 + 16;       // bytes per staged K row
  // bytes per staged V row: 32 more than the row, so that the four rows one
  // lane group reads in a transposing load start 8 banks apart
  static constexpr int VPITCH = D * 2 + 32;
  static constexpr int KBYTES = kFTok * KPITCH;
  static constexpr int BUF = KBYTES + kFTok * VPITCH;  // one stage (K then V)
  static constexpr int CPR = D / 8;               // 16-byte chunks per token row
  static constexpr int CPT = kFTok * CPR / kFThreads;  // chunks per thread per tensor
};

struct FTile {
  int32_t seq[kFVec];
  int32_t pos[kFVec];
  uint8_t done[kFVec];
  uint8_t active[kFVec];
  int cur_seq, kv_end, min_pos;
};

}  // namespace

template <int D>
__global__ void __launch_bounds__(kFThreads) dense_flash_kernel(AttnArgs a, int n_rows) {
  using Gm = FGeom<D>;
  __shared__ __align__(16) unsigned char smem[2 * Gm::BUF];
  __shared__ FTile ft;
  const int G = a.hq / a.hkv;
  const int TR = kFVec / G;  // rows per tile
  // heaviest tiles (latest rows) first
  const int tile = (int)gridDim.x - 1 - (int)blockIdx.x;
  const int hk = blockIdx.y;
  const int r0 = tile * TR;
  const int w = threadIdx.x / kWave, l = lane_id(), g = l / 16, c16 = l % 16;

  for (int i = threadIdx.x; i < TR; i += blockDim.x) {
    const int row = r0 + i;
    const bool ok = row < n_rows;
    ft.seq[i] = ok ? clamp_flag(a.seq_id[row], 0, a.n_seqs - 1, QSA_DEBUG_BAD_ROW) : -1;
    ft.pos[i] = ok ? clamp_flag(a.pos[row], 0, a.max_pos, QSA_DEBUG_BAD_ROW) : -1;
    ft.done[i] = ok ? 0 : 1;
  }
  __syncthreads();

  const float sl2 = a.scale * 1.4426950408889634f;
  const int64_t rstride = (int64_t)a.hkv * D;
  const bf16_t* kg = static_cast<const bf16_t*>(a.k) + hk * D;
  const bf16_t* vg = static_cast<const bf16_t*>(a.v) + hk * D;

  // rows of one sequence at a time (a tile normally holds one)
  while (true) {
    if (threadIdx.x == 0) {
      int cur = -1;
      for (int i = 0; i < TR; ++i)
        if (!ft.done[i]) {
          cur = ft.seq[i];
          break;
        }
      int hi = -1, lo = 0x7fffffff;
      for (int i = 0; i < TR; ++i) {
        const bool act = cur >= 0 && !ft.done[i] && ft.seq[i] == cur;
        ft.active[i] = act;
        if (act) {
          ft.done[i] = 1;
          hi = max(hi, ft.pos[i]);
          lo = min(lo, ft.pos[i]);
        }
      }
      ft.cur_seq = cur;
      ft.kv_end = hi + 1;
      ft.min_pos = lo;
    }
    __syncthreads();
    const int seq = ft.cur_seq;
    if (seq < 0) break;
    const int kv_end = ft.kv_end, min_pos = ft.min_pos;

    // this lane's query columns: vector v = w*32 + c*16 + c16 -> (row, head)
    u32x4_t qf[kFNC][Gm::KS];
    int cpos[kFNC];
#pragma unroll
    for (int c = 0; c < kFNC; ++c) {
      const int v = w * (kFNC * 16) + c * 16 + c16;
      const int ri = v / G, hh = v % G;
      const bool act = ri < TR && ft.active[ri];
      cpos[c] = act ? ft.pos[ri] : -1;
      const bf16_t* qp = static_cast<const bf16_t*>(a.q) +
                         ((int64_t)(r0 + ri) * a.hq + hk * G + hh) * D + (D / 4) * g;
#pragma unroll
      for (int s = 0; s < Gm::KS; ++s)
        qf[c][s] = act ? *reinterpret_cast<const u32x4_t*>(qp + 8 * s) : u32x4_t{0u, 0u, 0u, 0u};
    }
    float m[kFNC];
    f32x4_t acc[kFNC][Gm::NDT], lacc[kFNC];
    const u32x4_t ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 x 8
#pragma unroll
    for (int c = 0; c < kFNC; ++c) {
      m[c] = -INFINITY;
      lacc[c] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int n = 0; n < Gm::NDT; ++n) acc[c][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }

    // staging, K and V alike: chunk ch = threadIdx.x + kFThreads i -> token
    // ch / CPR, dims 8 (ch % CPR) .. (16 lanes read one whole row).
    // A tile's token rows come from one page lookup when pages hold whole
    // tiles, else one per token.  Tokens past kv_end read the last token's
    // row instead (they are masked), so every load is unconditional and a
    // tile's loads are all in flight together.
    const bool page_tiles = a.pm.page_shift >= 6;
    u32x4_t pk[Gm::CPT], pv[Gm::CPT];
    auto fetch = [&](int t) {
      const int j0 = t * kFTok;
      const int jl = kv_end - 1 - j0;  // last tile token with data
      int64_t off[Gm::CPT];            // element offsets of the thread's rows
      if (page_tiles) {
        const int64_t base = a.pm.token_slot(seq, j0);
#pragma unroll
        for (int i = 0; i < Gm::CPT; ++i) {
          const int ch = threadIdx.x + kFThreads * i;
          off[i] = (base + min(ch / Gm::CPR, jl)) * rstride + 8 * (ch % Gm::CPR);
        }
      } else {
#pragma unroll
        for (int i = 0; i < Gm::CPT; ++i) {
          const int ch = threadIdx.x + kFThreads * i;
          off[i] = a.pm.token_slot(seq, j0 + min(ch / Gm::CPR, jl)) * rstride + 8 * (ch % Gm::CPR);
        }
      }
#pragma unroll
      for (int i = 0; i < Gm::CPT; ++i) {
        pk[i] = *reinterpret_cast<const u32x4_t*>(kg + off[i]);
        pv[i] = *reinterpret_cast<const u32x4_t*>(vg + off[i]);
      }
    };
    auto park = [&](unsigned char* buf) {
      unsigned char* ks = buf;
      unsigned char* vs = buf + Gm::KBYTES;
#pragma unroll
      for (int i = 0; i < Gm::CPT; ++i) {
        const int ch = threadIdx.x + kFThreads * i;
        const int jt = ch / Gm::CPR, part = ch % Gm::CPR;
        *reinterpret_cast<u32x4_t*>(ks + jt * Gm::KPITCH + part * 16) = pk[i];
        *reinterpret_cast<u32x4_t*>(vs + jt * Gm::VPITCH + part * 16) = pv[i];
      }
    };
    // transposing read of V^T: the lane supplies the address of tile token
    // 4g + c16/4 (plus 32 kk, plus 16 for the upper half), dims
    // 16n + 4(c16 % 4) .. +4; lane (g, c16) receives V[4g + j][16n + c16],
    // j = 0..3
    const uint32_t tr_off = (4 * g + c16 / 4) * Gm::VPITCH + 8 * (c16 % 4);

    const int n_tiles = (kv_end + kFTok - 1) / kFTok;
    fetch(0);
    park(smem);
    __syncthreads();
    for (int t = 0; t < n_tiles; ++t) {
      unsigned char* buf = smem + (t & 1) * Gm::BUF;
      if (t + 1 < n_tiles) fetch(t + 1);
      const unsigned char* ks = buf;
      const unsigned char* vs = buf + Gm::KBYTES;
      // S^T: 4 token tiles x kFNC column groups
      f32x4_t sc[kFNC][4];
#pragma unroll
      for (int c = 0; c < kFNC; ++c)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) sc[c][tt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
        for (int s = 0; s < Gm::KS; ++s) {
          const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(
              ks + (16 * tt + c16) * Gm::KPITCH + ((D / 4) * g + 8 * s) * 2);
#pragma unroll
          for (int c = 0; c < kFNC; ++c) sc[c][tt] = mfma(kf, qf[c][s], sc[c][tt]);
        }
      }
      // online softmax per column; tokens past a column's position (only
      // in tiles that reach past the pass's smallest position) are masked
      const int j0 = t * kFTok;
      const bool need_mask = j0 + kFTok - 1 > min_pos;
      u32x4_t pb[kFNC][2];
      bool rescale = false;
      float corr[kFNC];
      // MASK: tiles reaching past the pass's smallest position mask slots
      // past each column's position; the maximum is taken on raw scores
      // (the scale is positive) and the scale folded into one fma per
      // numerator
      auto softmax = [&](auto mask_c) {
        constexpr bool MASK = decltype(mask_c)::value;
#pragma unroll
        for (int c = 0; c < kFNC; ++c) {
          auto masked = [&](int tt, int i) {
            return MASK && j0 + 16 * tt + 4 * g + i > cpos[c];
          };
          float mr = -INFINITY;
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; ++i) mr = fmaxf(mr, masked(tt, i) ? -INFINITY : sc[c][tt][i]);
          // the column's maximum over the four lane groups (rows 16 apart,
          // then 32 apart) with lane swaps instead of LDS permutes
          {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(mr),
                                                            __float_as_uint(mr), false, false);
            mr = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
          }
          {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(mr),
                                                            __float_as_uint(mr), false, false);
            mr = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
          }
          const float mx = mr * sl2;
          const bool grow = mx > m[c] + kSlack;
          const float m_new = grow ? mx : m[c];
          corr[c] = (!grow || m[c] == -INFINITY) ? (grow ? 0.0f : 1.0f)
                                                  : __builtin_amdgcn_exp2f(m[c] - m_new);
          rescale |= grow;
          m[c] = m_new;
          // (without masking some score is finite, so m_new is)
          const bool none = MASK && m_new == -INFINITY;
          uint32_t pw[8];
#pragma unroll
          for (int tt = 0; tt < 4; ++tt)
#pragma unroll
            for (int i = 0; i < 4; i += 2) {
              float p0 = __builtin_amdgcn_exp2f(fmaf(sc[c][tt][i], sl2, -m_new));
              float p1 = __builtin_amdgcn_exp2f(fmaf(sc[c][tt][i + 1], sl2, -m_new));
              if (MASK) {
                p0 = (none || masked(tt, i)) ? 0.0f : p0;
                p1 = (none || masked(tt, i + 1)) ? 0.0f : p1;
              }
              pw[2 * tt + i / 2] = pack_bf16x2(p0, p1);
            }
          // k-slots of step kk: tokens 32kk + 4g + 0..3, then 32kk + 16 + 4g + 0..3
#pragma unroll
          for (int kk = 0; kk < 2; ++kk)
            pb[c][kk] = u32x4_t{pw[4 * kk], pw[4 * kk + 1], pw[4 * kk + 2], pw[4 * kk + 3]};
        }
      };
      if (need_mask)
        softmax(std::true_type{});
      else
        softmax(std::false_type{});
      if (__ballot(rescale) != 0ull) {
#pragma unroll
        for (int c = 0; c < kFNC; ++c) {
          lacc[c] = lacc[c] * corr[c];
#pragma unroll
          for (int n = 0; n < Gm::NDT; ++n) acc[c][n] = acc[c][n] * corr[c];
        }
      }
      // O^T += V^T . P^T
#pragma unroll
      for (int n = 0; n < Gm::NDT; ++n) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const unsigned char* vp = vs + tr_off + 32 * kk * Gm::VPITCH + 32 * n;
          const u32x2_t lo = __builtin_bit_cast(
              u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)vp));
          const u32x2_t hi = __builtin_bit_cast(
              u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(vp + 16 * Gm::VPITCH)));
          const u32x4_t va = {lo.x, lo.y, hi.x, hi.y};
#pragma unroll
          for (int c = 0; c < kFNC; ++c) acc[c][n] = mfma(va, pb[c][kk], acc[c][n]);
        }
      }
      // column sums of the numerators (every row of the product holds them)
#pragma unroll
      for (int c = 0; c < kFNC; ++c)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) lacc[c] = mfma(ones, pb[c][kk], lacc[c]);
      if (t + 1 < n_tiles) park(smem + ((t + 1) & 1) * Gm::BUF);
      __syncthreads();
    }

    // normalise and write: lane holds dims 16n + 4g + i of its column
#pragma unroll
    for (int c = 0; c < kFNC; ++c) {
      const float L = lacc[c][0];
      if (cpos[c] < 0) continue;
      const int v = w * (kFNC * 16) + c * 16 + c16;
      const int ri = v / G, hh = v % G;
      bf16_t* o = static_cast<bf16_t*>(a.out) + ((int64_t)(r0 + ri) * a.hq + hk * G + hh) * D;
      const float inv = 1.0f / L;
#pragma unroll
      for (int n = 0; n < Gm::NDT; ++n) {
        const u32x2_t pr = {pack_bf16x2(acc[c][n][0] * inv, acc[c][n][1] * inv),
                            pack_bf16x2(acc[c][n][2] * inv, acc[c][n][3] * inv)};
        *reinterpret_cast<u32x2_t*>(o + 16 * n + 4 * g) = pr;
      }
    }
    __syncthreads();
  }
}

bool dense_flash_supported(int dtype, int hq, int hkv, int d) {
  if (dtype != QSA_BF16 || (d != 64 && d != 128)) return false;
  if (hkv < 1 || hq % hkv != 0) return false;
  const int G = hq / hkv;
  return G <= 16 && 16 % G == 0;
}

void run_dense_flash(const AttnArgs& a, int d, int n_rows, hipStream_t st) {
  const int G = a.hq / a.hkv;
  const int tr = kFVec / G;
  dim3 grid((unsigned)((n_rows + tr - 1) / tr), (unsigned)a.hkv);
  if (d == 128)
    hipLaunchKernelGGL(dense_flash_kernel<128>, grid, dim3(kFThreads), 0, st, a, n_rows);
  else
    hipLaunchKernelGGL(dense_flash_kernel<64>, grid, dim3(kFThreads), 0, st, a, n_rows);
}

}  // namespace qsa
