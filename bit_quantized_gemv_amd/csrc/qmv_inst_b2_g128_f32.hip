// Kernel instances: 2-bit codes, groups of 128, f32 activations.
#define QMV_BITS 2
#define QMV_GS 128
#define QMV_XF32 true
#define QMV_TABLE qmv_table_b2_g128_f32
#define QMV_WTABLE qmv_wtable_b2_g128_f32
#include "qmv_inst.inc"
