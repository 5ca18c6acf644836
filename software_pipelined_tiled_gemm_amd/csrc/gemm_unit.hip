// Kernel instantiations of one translation unit: the SPG_V lines of variants.inc whose
// first field equals the unit number this file is compiled for.  build.py compiles this
// file once per unit number found in variants.inc, passing -DSPG_UNIT_IS_<n>=~,1, so the
// units build in parallel.
#define SPG_DEFINE_LAUNCHERS
#include "launch.hpp"

#define SPG_CAT_(a, b) a##b
#define SPG_CAT(a, b) SPG_CAT_(a, b)
#define SPG_SECOND_(a, b, ...) b
#define SPG_SECOND(...) SPG_SECOND_(__VA_ARGS__)
// 1 when `u` is this unit's number (SPG_UNIT_IS_<u> expands to "~, 1"), else 0
#define SPG_IS_UNIT(u) SPG_SECOND(SPG_CAT(SPG_UNIT_IS_, u), 0)
#define SPG_WHEN_0(...)
#define SPG_WHEN_1(...) SPG_INSTANTIATE_ALL(__VA_ARGS__)
#define SPG_V(unit, ...) SPG_CAT(SPG_WHEN_, SPG_IS_UNIT(unit))(__VA_ARGS__)
#include "variants.inc"
