// The chunk-preparation kernels for fp32 inputs: prep.hip compiled as a
// translation unit of its own that instantiates only its fp32 launchers.
#define GDR_PREP_UNIT 1
#include "prep.hip"
