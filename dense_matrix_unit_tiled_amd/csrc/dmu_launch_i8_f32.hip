// Kernel instantiations and launcher for INT8 inputs with F32 output (dequantising).
#define DMU_IN dmu::I8
#define DMU_OUT dmu::F32
#define DMU_IN_IS_I8 1
#define DMU_LAUNCH_NAME launch_i8_f32
#include "dmu_launch.inc"
