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
// weight rows stacked (Wq, Wk, Ww), on v_mfma_f32_16x16x32_bf16.  A
// workgroup of 8 waves owns 128 rows x up to 336 columns: 64-wide K slices
// of its rows of X and of the weight rows are staged in LDS by whole
// 128-byte rows, double-buffered, with the loads of the slice after next
// in flight while the current one is multiplied (one slice of products
// does not cover a memory round trip; the loads are unconditional -- past
// the end they reload the last slice -- so that each wait covers only the
// older slice); wave (wm, wn) computes 64 rows x 5 or 6 column tiles,
// reading both operands from LDS.
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

constexpr int kPM = 128;                // rows per workgroup
constexpr int kPNT = 21;                // 16-column tiles per workgroup
constexpr int kPN = kPNT * 16;          // columns per workgroup
constexpr int kPK = 64;                 // K slice staged at once
constexpr int kPPitch = kPK * 2 + 16;   // LDS bytes per staged row
constexpr int kPRowsL = kPM + kPN;      // staged rows per slice (X rows, then W rows)
constexpr int kPBuf = kPRowsL * kPPitch;
constexpr int kPThr = 512;
constexpr int kPChunks = kPRowsL * (kPK / 8);  // 16-byte pieces per slice
constexpr int kPPer = (kPChunks + kPThr - 1) / kPThr;
constexpr int kPMaxNt = 6;              // column tiles of a wave

}  // namespace

__global__ void __launch_bounds__(kPThr) project_kernel(ProjArgs a) {
  __shared__ __align__(16) unsigned char lds[2 * kPBuf];  // two slices
  const int w = threadIdx.x / kWave, l = lane_id(), g = l / 16, c16 = l % 16;
  const int wm = w / 4, wn = w % 4;
  const int mt0 = blockIdx.x * kPM;
  const int n0 = blockIdx.y * kPN;
  const int H = a.h;
  // this wave's column tiles: 6, 5, 5, 5 of the 21
  const int nt0 = wn == 0 ? 0 : 1 + 5 * wn, ntc = wn == 0 ? 6 : 5;
  // source of staged row r: X rows (past T: the last row, never stored),
  // then weight rows of the stacked [Wq; Wk; Ww] (past N: none)
  auto src_row = [&](int r) -> const bf16_t* {
    if (r < kPM) return a.x + (int64_t)min(mt0 + r, a.rows - 1) * H;
    const int n = n0 + r - kPM;
    if (n < a.nq) return a.wq + (int64_t)n * H;
    if (n < a.nq + a.nk) return a.wk + (int64_t)(n - a.nq) * H;
    if (n < a.n) return a.ww + (int64_t)(n - a.nq - a.nk) * H;
    return nullptr;
  };
  // the thread's staged pieces: source rows (fixed across slices) and
  // their LDS places
  // (pieces past the slice or of rows past N read x's first row and store
  // nothing or zeros: every load is unconditional)
  const bf16_t* sp[kPPer];
  uint32_t live = 0u;  // bit j: the piece's row has data
#pragma unroll
  for (int j = 0; j < kPPer; ++j) {
    const int ci = (int)threadIdx.x + kPThr * j;
    const bf16_t* p = ci < kPChunks ? src_row(ci / 8) : nullptr;
    sp[j] = p ? p + 8 * (ci % 8) : a.x;
    live |= p ? (1u << j) : 0u;
  }
  auto load = [&](int k0, u32x4_t (&st)[kPPer]) {
#pragma unroll
    for (int j = 0; j < kPPer; ++j) st[j] = *reinterpret_cast<const u32x4_t*>(sp[j] + k0);
  };
  auto store = [&](unsigned char* buf, const u32x4_t (&st)[kPPer]) {
#pragma unroll
    for (int j = 0; j < kPPer; ++j) {
      const int ci = (int)threadIdx.x + kPThr * j;
      if (ci < kPChunks)
        *reinterpret_cast<u32x4_t*>(buf + (ci / 8) * kPPitch + 16 * (ci % 8)) =
            (live >> j) & 1u ? st[j] : u32x4_t{0u, 0u, 0u, 0u};
    }
  };
  f32x4_t acc[4][kPMaxNt];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < kPMaxNt; ++nt) acc[mt][nt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int nslice = H / kPK;
  auto compute = [&](const unsigned char* cur) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      u32x4_t af[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
        af[mt] = *reinterpret_cast<const u32x4_t*>(cur + (64 * wm + 16 * mt + c16) * kPPitch +
                                                   64 * s + 16 * g);
#pragma unroll
      for (int nt = 0; nt < kPMaxNt; ++nt) {
        if (nt < ntc) {  // uniform
          const u32x4_t b = *reinterpret_cast<const u32x4_t*>(
              cur + (kPM + 16 * (nt0 + nt) + c16) * kPPitch + 64 * s + 16 * g);
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) acc[mt][nt] = mfma_bf16(af[mt], b, acc[mt][nt]);
        }
      }
    }
  };
  // slice ks is in LDS buffer ks % 2; register sets rA / rB alternate
  // holding the next slice (loaded a whole step earlier) and the one after
  u32x4_t rA[kPPer], rB[kPPer];
  // one step: issue the loads of slice ks + 2, multiply slice ks, store
  // slice ks + 1 (the other register set) into the other buffer
  auto step = [&](int ks, const u32x4_t (&rnext)[kPPer], u32x4_t (&rafter)[kPPer]) {
    load(min(ks + 2, nslice - 1) * kPK, rafter);
    compute(lds + (ks & 1) * kPBuf);
    store(lds + ((ks + 1) & 1) * kPBuf, rnext);
    __syncthreads();
  };
  load(0, rA);
  load(min(1, nslice - 1) * kPK, rB);
  store(lds, rA);
  __syncthreads();
  for (int ks = 0; ks < nslice; ks += 2) {
    step(ks, rB, rA);  // slice ks + 1 is in rB; slice ks + 2 goes to rA
    if (ks + 1 < nslice) step(ks + 1, rA, rB);
  }
  // lane holds rows 4g + i of each row tile, column c16 of each column tile
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = mt0 + 64 * wm + 16 * mt + 4 * g + i;
      if (row >= a.rows) continue;
      const int64_t slot = a.pm.token_slot(a.seq_of(row), a.pos_of(row));
#pragma unroll
      for (int nt = 0; nt < kPMaxNt; ++nt) {
        const int n = n0 + 16 * (nt0 + nt) + c16;
        if (nt >= ntc) continue;
        const float y = acc[mt][nt][i];
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
}

void run_project(const ProjArgs& a, hipStream_t st) {
  dim3 grid((unsigned)((a.rows + kPM - 1) / kPM), (unsigned)((a.n + kPN - 1) / kPN));
  hipLaunchKernelGGL(project_kernel, grid, dim3(kPThr), 0, st, a);
}

}  // namespace qsa
