// Top-k kernels for bfloat16 caches with indexer dimension 16.
#include "topk.hpp"

namespace qsa {
template void launch_topk_typed<bf16_t, 16>(const TopkArgs& t, int rows, hipStream_t st);
}  // namespace qsa
