// Kernel instantiations and launcher for FP8 e4m3 inputs with BF16 output.
#define DMU_IN dmu::E4M3
#define DMU_OUT dmu::BF16
#define DMU_IN_IS_F8 1
#define DMU_LAUNCH_NAME launch_e4m3_bf16
#include "dmu_launch.inc"
