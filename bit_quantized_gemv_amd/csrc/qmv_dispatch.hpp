// qmv_dispatch.hpp -- host-side tables of kernel instances, indexed by
// (bits, group size, activation dtype) -> [rows per wavefront][M - 1][scale/bias
// dtype], one table for the instances that stage the whole K at once and one
// for the K-windowed instances (both keep one unit in flight per wavefront).
// Entries not instantiated are null.
#pragma once

#include "qmv_kernel.hpp"

namespace qmv {

using KernelFn = void (*)(Params);
constexpr int kNumR = 4;      // rows per wavefront 1, 2, 3, 4
constexpr int kMaxM = 13;
constexpr int kNumSb = 2;     // scales/biases fp16, bf16

extern const KernelFn qmv_table_b4_g64_bf16[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_table_b4_g64_f32[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_table_b4_g128_bf16[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_table_b4_g128_f32[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_table_b2_g64_bf16[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_table_b2_g64_f32[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_table_b2_g128_bf16[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_table_b2_g128_f32[kNumR][kMaxM][kNumSb];

extern const KernelFn qmv_wtable_b4_g64_bf16[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_wtable_b4_g64_f32[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_wtable_b4_g128_bf16[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_wtable_b4_g128_f32[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_wtable_b2_g64_bf16[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_wtable_b2_g64_f32[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_wtable_b2_g128_bf16[kNumR][kMaxM][kNumSb];
extern const KernelFn qmv_wtable_b2_g128_f32[kNumR][kMaxM][kNumSb];

// Stamped instances (measurement aid): bf16 activations and bf16
// scales/biases, 4-bit codes in groups of 64 and 2-bit codes in groups of
// 128, indexed [K-windowed][rows per wavefront - 1][M - 1].
using TimelineFn = void (*)(Params, uint64_t*);
extern const TimelineFn qmv_timeline_b4_g64_bf16[2][kNumR][kMaxM];
extern const TimelineFn qmv_timeline_b2_g128_bf16[2][kNumR][kMaxM];

}  // namespace qmv
