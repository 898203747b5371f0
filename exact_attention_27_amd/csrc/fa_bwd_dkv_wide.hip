// The 256-wide dK/dV kernels (head dims 136..256), compiled as a unit of their own. At that
// width a wave's pinned K fragments and dK, dV accumulators (320 registers) exceed the 256
// architectural VGPRs, so this unit leaves the MFMA register form to the compiler's
// heuristics (accumulators may live in AGPRs) instead of forcing the VGPR form the other
// kernels are built with.
#define FA_DKV_WIDE_UNIT 1
#include "fa_bwd_dkv.hip"
