// Kernel instantiations of translation unit 24 (the SPG_V lines of variants.inc
// whose first field is 24); the units compile in parallel.
#define SPG_DEFINE_LAUNCHERS
#include "launch.hpp"

#define SPG_V(unit, BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, PERS) SPG_V_##unit(BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, PERS)
#define SPG_V_0(...)
#define SPG_V_1(...)
#define SPG_V_2(...)
#define SPG_V_3(...)
#define SPG_V_4(...)
#define SPG_V_5(...)
#define SPG_V_6(...)
#define SPG_V_7(...)
#define SPG_V_8(...)
#define SPG_V_9(...)
#define SPG_V_10(...)
#define SPG_V_11(...)
#define SPG_V_12(...)
#define SPG_V_13(...)
#define SPG_V_14(...)
#define SPG_V_15(...)
#define SPG_V_16(...)
#define SPG_V_17(...)
#define SPG_V_18(...)
#define SPG_V_19(...)
#define SPG_V_20(...)
#define SPG_V_21(...)
#define SPG_V_22(...)
#define SPG_V_23(...)
#define SPG_V_24(...) SPG_INSTANTIATE_ALL(__VA_ARGS__)
#define SPG_V_25(...)
#include "variants.inc"
