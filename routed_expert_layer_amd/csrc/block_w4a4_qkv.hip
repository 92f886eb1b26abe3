// The block kernel with both the W4A4 experts and the next layer's QKV
// projection fused after the boundary: block.hip built again, with only that
// kernel, in a code object of its own.
#define MB_BLOCK_W4A4 1
#define MB_BLOCK_QKV 1
#include "block.hip"
