// The decode.hip kernels for MXFP4 weights (FP4 e2m1 codes, E8M0 scales per 32
// channels): the same source compiled with MOE_WEIGHT_FORMAT = 1.
#define MOE_WEIGHT_FORMAT 1
#include "decode.hip"
