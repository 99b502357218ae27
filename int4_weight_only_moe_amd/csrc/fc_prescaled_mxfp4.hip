// The pre-scaled tiled kernel of fc_prescaled.hip for MXFP4 expert weights.
#define MOE_WEIGHT_FORMAT 1
#include "fc_prescaled.hip"
