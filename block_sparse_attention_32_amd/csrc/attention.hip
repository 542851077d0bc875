// Block-sparse attention over the selected blocks plus the own (tail) block,
// read straight from the paged cache with no mask, and the dense causal GQA
// baseline on the same cache.
//
//   token set  -- blog.cecily.jp/6295 (PR #30965 digest), paragraph on the
//                 trade-offs: whole 4-token blocks are read, and the budget
//                 is the selected blocks plus the current fractional block.
//   no mask    -- ai-manual.ru, "Экономия VRAM в llama.cpp: что даёт
//                 QSA-выбор без kq_mask", section "QSA-выбор и kq_mask": the
//                 selection is consumed directly, no [queries x keys] table.
//   tiling     -- ai-manual.ru, "llama.cpp получил разреженный Flash
//                 Attention для Qwen4 на CUDA", section "Разреженный Flash
//                 Attention и обычный": attention runs tile by tile with an
//                 online softmax; only (max, sum, accumulator) leave a tile.
//   baseline   -- keieiax.jp glossary, section 長文AIのコストと応答時間にどう影
//                 響する？: the comparison is dense grouped-query attention.
//
// One workgroup handles one (row, split); a split is a contiguous range of
// the row's block list.  With several splits per row the partial
// (max, sum, accumulator) triples go to the workspace and the last split of
// the row to finish merges them.
#include "attention.hpp"

namespace qsa {

template <typename T, int D, bool DENSE>
__global__ void __launch_bounds__(kAttnThreads) attn_kernel(AttnArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int TT = a.tile_tokens;
  const int hq = a.hq, hkv = a.hkv, grp = hq / hkv;
  const int row = blockIdx.y, split = blockIdx.x;
  const int tid = threadIdx.x;
  const AttnLayout L = attn_layout((int)sizeof(T), hq, hkv, D, TT);
  float* qs = reinterpret_cast<float*>(smem + L.q);           // [hq][D]
  float* ss = reinterpret_cast<float*>(smem + L.s);           // [hq][TT]
  float* m_s = reinterpret_cast<float*>(smem + L.m);          // [hq]
  float* l_s = reinterpret_cast<float*>(smem + L.l);          // [hq]
  float* c_s = reinterpret_cast<float*>(smem + L.c);          // [hq]
  int64_t* trow = reinterpret_cast<int64_t*>(smem + L.trow);  // [TT]
  T* ks = reinterpret_cast<T*>(smem + L.k);                   // [TT][hkv][D]
  T* vs = reinterpret_cast<T*>(smem + L.v);                   // [TT][hkv][D]
  __shared__ uint32_t flag;

  const int seq = clamp_flag(a.seq_id[row], 0, a.n_seqs - 1, QSA_DEBUG_BAD_ROW);
  const int t = clamp_flag(a.pos[row], 0, a.max_pos, QSA_DEBUG_BAD_ROW);
  // n_sel is clamped to [0, top_k]; selected ids the row may not attend are
  // skipped
  const RowList rl(a, row, t, DENSE, DENSE ? 0 : a.n_sel[row]);
  const int b_own = rl.b_own;
  const int n_entries = rl.e_own + 1;
  const int e_beg = split * a.eps;
  const int e_end = min(n_entries, e_beg + a.eps);

  const T* qrow = static_cast<const T*>(a.q) + (int64_t)row * hq * D;
  for (int i = tid; i < hq * D; i += kAttnThreads) qs[i] = to_f32(qrow[i]);
  for (int h = tid; h < hq; h += kAttnThreads) {
    m_s[h] = -INFINITY;
    l_s[h] = 0.0f;
  }
  const int n_out = (hq * D + kAttnThreads - 1) / kAttnThreads;
  float acc[kMaxOutPerThread];
#pragma unroll
  for (int j = 0; j < kMaxOutPerThread; ++j) acc[j] = 0.0f;

  const int row_elems = hkv * D;
  constexpr int V = Vec<T>::N;
  const T* kg = static_cast<const T*>(a.k);
  const T* vg = static_cast<const T*>(a.v);
  const int bs = a.pm.blk_shift, nb = 1 << bs;  // tokens per block
  const int ept = TT >> bs;  // entries per tile (TT is a multiple of the block)
  for (int e0 = e_beg; e0 < e_end; e0 += ept) {
    __syncthreads();
    for (int j = tid; j < TT; j += kAttnThreads) {
      const int e = e0 + (j >> bs), i = j & (nb - 1);
      int64_t r = -1;
      if (e < e_end) {
        const bool own = (e == rl.e_own);
        bool ok = true;
        const int b = own ? b_own : rl.block(e, DENSE, ok);
        const int ntok = own ? (t & (nb - 1)) + 1 : nb;
        if (ok && i < ntok) r = a.pm.token_slot(seq, (b << bs) + i);
      }
      trow[j] = r;
    }
    __syncthreads();
    const int vpr = row_elems / V;  // vectors per token row
    for (int i = tid; i < TT * vpr; i += kAttnThreads) {
      const int j = i / vpr, c = i % vpr;
      const int64_t r = trow[j];
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (r >= 0) {
        kv = *reinterpret_cast<const uint4*>(kg + r * row_elems + c * V);
        vv = *reinterpret_cast<const uint4*>(vg + r * row_elems + c * V);
      }
      *reinterpret_cast<uint4*>(ks + (size_t)j * row_elems + c * V) = kv;
      *reinterpret_cast<uint4*>(vs + (size_t)j * row_elems + c * V) = vv;
    }
    __syncthreads();
    for (int i = tid; i < hq * TT; i += kAttnThreads) {
      const int h = i / TT, j = i % TT;
      float s = -INFINITY;
      if (trow[j] >= 0) {
        const float* qh = qs + h * D;
        const T* kr = ks + (size_t)j * row_elems + (h / grp) * D;
        float acc_s = 0.0f;
#pragma unroll 8
        for (int d = 0; d < D; ++d) acc_s = fmaf(qh[d], to_f32(kr[d]), acc_s);
        s = acc_s * a.scale;
      }
      ss[h * TT + j] = s;
    }
    __syncthreads();
    for (int h = tid; h < hq; h += kAttnThreads) {
      float mx = -INFINITY;
      for (int j = 0; j < TT; ++j) mx = fmaxf(mx, ss[h * TT + j]);
      const float m_old = m_s[h];
      const float m_new = fmaxf(m_old, mx);
      float corr = 1.0f, sum = 0.0f;
      if (m_new != -INFINITY) {
        corr = __expf(m_old - m_new);
        for (int j = 0; j < TT; ++j) {
          float p = __expf(ss[h * TT + j] - m_new);
          ss[h * TT + j] = p;
          sum += p;
        }
      } else {
        for (int j = 0; j < TT; ++j) ss[h * TT + j] = 0.0f;
      }
      l_s[h] = l_s[h] * corr + sum;
      m_s[h] = m_new;
      c_s[h] = corr;
    }
    __syncthreads();
#pragma unroll
    for (int jo = 0; jo < kMaxOutPerThread; ++jo) {
      const int o = tid + jo * kAttnThreads;
      if (jo < n_out && o < hq * D) {
        const int h = o / D, d = o % D;
        const T* vc = vs + (h / grp) * D + d;
        const float* ph = ss + h * TT;
        float s = acc[jo] * c_s[h];
        for (int j = 0; j < TT; ++j) s = fmaf(ph[j], to_f32(vc[(size_t)j * row_elems]), s);
        acc[jo] = s;
      }
    }
  }
  __syncthreads();

  T* orow = static_cast<T*>(a.out) + (int64_t)row * hq * D;
  if (a.n_splits == 1) {
#pragma unroll
    for (int jo = 0; jo < kMaxOutPerThread; ++jo) {
      const int o = tid + jo * kAttnThreads;
      if (jo < n_out && o < hq * D) orow[o] = from_f32<T>(acc[jo] / l_s[o / D]);
    }
    return;
  }
  const int64_t pbase = ((int64_t)row * a.n_splits + split) * hq;
#pragma unroll
  for (int jo = 0; jo < kMaxOutPerThread; ++jo) {
    const int o = tid + jo * kAttnThreads;
    if (jo < n_out && o < hq * D) st_agent(a.part_acc + pbase * D + o, acc[jo]);
  }
  for (int h = tid; h < hq; h += kAttnThreads) {
    st_agent(a.part_ml + (pbase + h) * 2 + 0, m_s[h]);
    st_agent(a.part_ml + (pbase + h) * 2 + 1, l_s[h]);
  }
  if (!arrive_last(a.cnt + row, (uint32_t)a.n_splits, &flag)) return;
  // merge: out = sum_s acc_s e^(m_s - M) / sum_s l_s e^(m_s - M)
  for (int jo = 0; jo < n_out; ++jo) {
    const int o = tid + jo * kAttnThreads;
    if (o >= hq * D) continue;
    const int h = o / D;
    float M = -INFINITY;
    for (int s = 0; s < a.n_splits; ++s) {
      const int64_t pb = ((int64_t)row * a.n_splits + s) * hq + h;
      M = fmaxf(M, a.part_ml[pb * 2]);
    }
    float L = 0.0f, O = 0.0f;
    for (int s = 0; s < a.n_splits; ++s) {
      const int64_t pb = ((int64_t)row * a.n_splits + s) * hq + h;
      const float ms = a.part_ml[pb * 2];
      const float ls = a.part_ml[pb * 2 + 1];
      if (ls > 0.0f) {
        const float f = __expf(ms - M);
        L = fmaf(ls, f, L);
        O = fmaf(a.part_acc[pb * D + (o % D)], f, O);
      }
    }
    orow[o] = from_f32<T>(O / L);
  }
}

int attn_tile_tokens(int dtype, int hq, int hkv, int d, int block) {
  const int esz = dtype == QSA_F32 ? 4 : 2;
  const int step = block > 4 ? block : 4;  // tiles hold whole blocks
  for (int tt = 64; tt >= step; tt -= step)
    if (attn_layout(esz, hq, hkv, d, tt).total <= (size_t)kAttnLds) return tt;
  return 0;
}

size_t attn_lds_bytes(int dtype, int hq, int hkv, int d, int tt) {
  return attn_layout(dtype == QSA_F32 ? 4 : 2, hq, hkv, d, tt).total;
}

template <typename T, int D>
static void launch_attn(const AttnArgs& a, bool dense, int n_rows, hipStream_t st) {
  const size_t lds = attn_lds_bytes(sizeof(T) == 4 ? QSA_F32 : QSA_BF16, a.hq, a.hkv, D,
                                    a.tile_tokens);
  dim3 grid((unsigned)a.n_splits, (unsigned)n_rows);
  if (dense)
    hipLaunchKernelGGL((attn_kernel<T, D, true>), grid, dim3(kAttnThreads), lds, st, a);
  else
    hipLaunchKernelGGL((attn_kernel<T, D, false>), grid, dim3(kAttnThreads), lds, st, a);
}

void run_attention(const AttnArgs& a, int dtype, int d, bool dense, int n_rows, hipStream_t st) {
#define QSA_ATTN_D(T)                                             \
  switch (d) {                                                    \
    case 32: launch_attn<T, 32>(a, dense, n_rows, st); break;     \
    case 64: launch_attn<T, 64>(a, dense, n_rows, st); break;     \
    case 128: launch_attn<T, 128>(a, dense, n_rows, st); break;   \
    default: break;                                               \
  }
  if (dtype == QSA_F32) { QSA_ATTN_D(float) } else { QSA_ATTN_D(bf16_t) }
#undef QSA_ATTN_D
}

}  // namespace qsa
