// qmv_dispatch.hpp -- host-side table of kernel instances, indexed by
// (bits, group size, activation dtype) -> [rows per wavefront][M - 1].
#pragma once

#include "qmv_kernel.hpp"

namespace qmv {

using KernelFn = void (*)(Params);
constexpr int kNumR = 3;      // rows per wavefront 1, 2, 4
constexpr int kMaxM = 13;

extern const KernelFn qmv_table_b4_g64_bf16[kNumR][kMaxM];
extern const KernelFn qmv_table_b4_g64_f32[kNumR][kMaxM];
extern const KernelFn qmv_table_b4_g128_bf16[kNumR][kMaxM];
extern const KernelFn qmv_table_b4_g128_f32[kNumR][kMaxM];
extern const KernelFn qmv_table_b2_g64_bf16[kNumR][kMaxM];
extern const KernelFn qmv_table_b2_g64_f32[kNumR][kMaxM];
extern const KernelFn qmv_table_b2_g128_bf16[kNumR][kMaxM];
extern const KernelFn qmv_table_b2_g128_f32[kNumR][kMaxM];

}  // namespace qmv
