// The block kernel's W4A4 variant (MXFP4 activations into the experts):
// block.hip built again, with only that kernel, in a code object of its own.
#define MB_BLOCK_W4A4 1
#include "block.hip"
