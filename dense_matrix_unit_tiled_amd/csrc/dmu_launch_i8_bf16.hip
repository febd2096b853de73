// Kernel instantiations and launcher for INT8 inputs with BF16 output (dequantising).
#define DMU_IN dmu::I8
#define DMU_OUT dmu::BF16
#define DMU_IN_IS_I8 1
#define DMU_LAUNCH_NAME launch_i8_bf16
#include "dmu_launch.inc"
