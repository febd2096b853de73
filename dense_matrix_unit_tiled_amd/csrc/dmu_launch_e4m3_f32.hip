// Kernel instantiations and launcher for FP8 e4m3 inputs with F32 output.
#define DMU_IN dmu::E4M3
#define DMU_OUT dmu::F32
#define DMU_IN_IS_F8 1
#define DMU_LAUNCH_NAME launch_e4m3_f32
#include "dmu_launch.inc"
