// Argument block of the indexer projections (project.hip).
#pragma once

#include "common.hpp"

namespace qsa {

struct ProjArgs {
  PageMap pm;
  const bf16_t* x;       // [T][h]
  const bf16_t* wq;      // [nq][h]
  const bf16_t* wk;      // [nk][h]
  const bf16_t* ww;      // [n - nq - nk][h]
  int h, nq, nk, n;      // hidden size; Hi*Di; Di; Hi*Di + Di + Hi
  int rows;              // T
  const int32_t* seq_id;
  const int32_t* pos;
  int n_seqs, max_pos;
  bf16_t* q_idx;         // [T][nq]
  bf16_t* kidx;          // paged cache rows [slot][nk]
  float* w;              // [T][Hi]
  __device__ __forceinline__ int seq_of(int row) const {
    return clamp_flag(seq_id[row], 0, n_seqs - 1, QSA_DEBUG_BAD_ROW);
  }
  __device__ __forceinline__ int pos_of(int row) const {
    return clamp_flag(pos[row], 0, max_pos, QSA_DEBUG_BAD_ROW);
  }
};

constexpr int kProjKStep = 64;  // the hidden size must be a multiple of this

void run_project(const ProjArgs& a, hipStream_t st);

}  // namespace qsa
