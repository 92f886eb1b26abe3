// The block kernel's many-rows instance (the fp64-MFMA router tiles compiled
// in): block.hip built again, with only that kernel, in a code object of its
// own, so that the plain kernel's code stays where it is.
#define MB_BLOCK_MANY 1
#include "block.hip"
