// The scale-before tiled kernel of fc_tile128.hip for MXFP4 expert weights.
#define MOE_WEIGHT_FORMAT 1
#include "fc_tile128.hip"
