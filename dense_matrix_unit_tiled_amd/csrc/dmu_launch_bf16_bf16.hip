// Kernel instantiations and launcher for BF16 inputs with BF16 output.
#define DMU_IN dmu::BF16
#define DMU_OUT dmu::BF16
#define DMU_IN_IS_I8 0
#define DMU_LAUNCH_NAME launch_bf16_bf16
#include "dmu_launch.inc"
