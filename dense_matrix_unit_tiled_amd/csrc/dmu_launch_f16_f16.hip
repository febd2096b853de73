// Kernel instantiations and launcher for F16 inputs with F16 output.
#define DMU_IN dmu::F16
#define DMU_OUT dmu::F16
#define DMU_IN_IS_I8 0
#define DMU_LAUNCH_NAME launch_f16_f16
#include "dmu_launch.inc"
