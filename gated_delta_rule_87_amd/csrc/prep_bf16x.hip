// The chunk-preparation kernels for bf16 inputs with d_k 64 or 256: prep.hip
// compiled as a translation unit of its own that instantiates only those
// launchers.
#define GDR_PREP_UNIT 2
#include "prep.hip"
