// Top-k kernels for bfloat16 caches with indexer dimension 128.
#include "topk.hpp"

namespace qsa {
template void launch_topk_typed<bf16_t, 128>(const TopkArgs& t, int rows, hipStream_t st);
}  // namespace qsa
