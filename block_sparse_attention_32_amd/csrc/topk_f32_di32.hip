// Top-k kernels for float32 caches with indexer dimension 32.
#include "topk.hpp"

namespace qsa {
template void launch_topk_typed<float, 32>(const TopkArgs& t, int rows, hipStream_t st);
}  // namespace qsa
