// Kernel instantiations and launcher for I8 inputs with I32 output.
#define DMU_IN dmu::I8
#define DMU_OUT dmu::I32
#define DMU_IN_IS_I8 1
#define DMU_LAUNCH_NAME launch_i8_i32
#include "dmu_launch.inc"
