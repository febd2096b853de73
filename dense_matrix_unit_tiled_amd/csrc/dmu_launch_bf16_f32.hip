// Kernel instantiations and launcher for BF16 inputs with F32 output.
#define DMU_IN dmu::BF16
#define DMU_OUT dmu::F32
#define DMU_IN_IS_I8 0
#define DMU_LAUNCH_NAME launch_bf16_f32
#include "dmu_launch.inc"
