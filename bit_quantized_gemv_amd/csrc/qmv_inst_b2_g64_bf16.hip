// Kernel instances: 2-bit codes, groups of 64, bf16 activations.
#define QMV_BITS 2
#define QMV_GS 64
#define QMV_XF32 false
#define QMV_TABLE qmv_table_b2_g64_bf16
#define QMV_WTABLE qmv_wtable_b2_g64_bf16
#include "qmv_inst.inc"
