// The indexer's input projections on gfx950 matrix cores.
//
// keieiax.jp glossary "Qwen Sparse Attention", section 4トークンずつまとめて:
// a lightweight *learned* indexer rates the blocks; blog.cecily.jp/6295 (PR
// #30965 digest), paragraph on Raschka's explanation: the indexer works on
// keys of its own, averaged per block.  The pages print no projection; the
// plainest reading is three linear maps of the hidden state x of a token:
//   q_idx[h][d] = x . Wq[h*Di + d]     (indexer queries, Hi heads of Di)
//   kidx[d]     = x . Wk[d]            (the token's indexer key, Di)
//   w[h]        = x . Ww[h]            (per-head weights, float32)
// float32 accumulation of bfloat16 products; q_idx and kidx are rounded to
// nearest-even bfloat16, kidx written into the token's slot of the paged
// cache.
//
// One contraction Y[T x N] = X[T x H] . W^T, W the N = Hi*Di + Di + Hi
// weight rows stacked (Wq, Wk, Ww), on v_mfma_f32_16x16x32_bf16: a
// workgroup of 4 waves owns 64 rows x up to 336 columns; each wave 16 rows
// (A fragments straight from x) against all the columns, whose 64-wide K
// slices are staged in LDS by whole 128-byte rows and shared by the waves.
#include "project.hpp"

namespace qsa {

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_bf16(u32x4_t a, u32x4_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

constexpr int kPM = 64;                 // rows per workgroup
constexpr int kPNT = 21;                // 16-column tiles per workgroup
constexpr int kPN = kPNT * 16;          // columns per workgroup
constexpr int kPK = 64;                 // K slice staged at once
constexpr int kPPitch = kPK * 2 + 16;   // LDS bytes per staged weight row

}  // namespace

__global__ void __launch_bounds__(256) project_kernel(ProjArgs a) {
  __shared__ __align__(16) unsigned char ws[kPN * kPPitch];
  const int w = threadIdx.x / kWave, l = lane_id(), g = l / 16, c16 = l % 16;
  const int m0 = blockIdx.x * kPM + w * 16;
  const int n0 = blockIdx.y * kPN;
  const int H = a.h;
  // this lane's A row (rows past T reload the last row; their results are
  // not stored)
  const bf16_t* xr = a.x + (int64_t)min(m0 + c16, a.rows - 1) * H + 8 * g;
  f32x4_t acc[kPNT];
#pragma unroll
  for (int nt = 0; nt < kPNT; ++nt) acc[nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // weight row n of the stacked [Wq; Wk; Ww], or null past N
  auto wrow = [&](int n) -> const bf16_t* {
    if (n < a.nq) return a.wq + (int64_t)n * H;
    if (n < a.nq + a.nk) return a.wk + (int64_t)(n - a.nq) * H;
    if (n < a.n) return a.ww + (int64_t)(n - a.nq - a.nk) * H;
    return nullptr;
  };
  constexpr int kChunks = kPN * (kPK / 8);                    // 16-byte pieces per slice
  constexpr int kPer = (kChunks + 255) / 256;
  for (int k0 = 0; k0 < H; k0 += kPK) {
    u32x4_t xa[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) xa[s] = *reinterpret_cast<const u32x4_t*>(xr + k0 + 32 * s);
    u32x4_t wv[kPer];
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int ci = (int)threadIdx.x + 256 * j;
      const bf16_t* p = ci < kChunks ? wrow(n0 + ci / 8) : nullptr;
      wv[j] = p ? *reinterpret_cast<const u32x4_t*>(p + k0 + 8 * (ci % 8))
                : u32x4_t{0u, 0u, 0u, 0u};
    }
    __syncthreads();  // the previous slice's reads are done
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int ci = (int)threadIdx.x + 256 * j;
      if (ci < kChunks)
        *reinterpret_cast<u32x4_t*>(ws + (ci / 8) * kPPitch + 16 * (ci % 8)) = wv[j];
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < 2; ++s) {
#pragma unroll
      for (int nt = 0; nt < kPNT; ++nt) {
        const u32x4_t b =
            *reinterpret_cast<const u32x4_t*>(ws + (nt * 16 + c16) * kPPitch + 64 * s + 16 * g);
        acc[nt] = mfma_bf16(xa[s], b, acc[nt]);
      }
    }
  }
  // lane holds rows m0 + 4g + i of column n0 + 16 nt + c16
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int row = m0 + 4 * g + i;
    if (row >= a.rows) continue;
    const int seq = a.seq_of(row), t = a.pos_of(row);
    const int64_t slot = a.pm.token_slot(seq, t);
#pragma unroll
    for (int nt = 0; nt < kPNT; ++nt) {
      const int n = n0 + 16 * nt + c16;
      const float y = acc[nt][i];
      if (n < a.nq) {
        a.q_idx[(int64_t)row * a.nq + n] = f32_to_bf16(y);
      } else if (n < a.nq + a.nk) {
        a.kidx[slot * a.nk + (n - a.nq)] = f32_to_bf16(y);
      } else if (n < a.n) {
        a.w[(int64_t)row * (a.n - a.nq - a.nk) + (n - a.nq - a.nk)] = y;
      }
    }
  }
}

void run_project(const ProjArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.rows + kPM - 1) / kPM), (unsigned)((a.n + kPN - 1) / kPN));
  hipLaunchKernelGGL(project_kernel, grid, dim3(256), 0, st, a);
}

}  // namespace qsa
