// Top-k kernels for float32 caches with indexer dimension 128.
#include "topk.hpp"

namespace qsa {
template void launch_topk_typed<float, 128>(const TopkArgs& t, int rows, hipStream_t st);
}  // namespace qsa
