// Stamped kernel instances (a measurement aid): bf16 activations, bf16 scales
// and biases, 4-bit codes in groups of 64 and 2-bit codes in groups of 128,
// every rows-per-wavefront and M the library dispatches to, whole K
// (scale/bias copies in LDS) and K-windowed.  Each is the product instance
// with the per-wavefront stamps added; the entry point that launches them is
// qmv_affine_timeline.
#include "qmv_kernel.hpp"
#include "qmv_dispatch.hpp"

namespace qmv {

#define QMV_T(B, G, R, M, WIN) &qmv_affine_kernel<B, G, R, M, 1, false, true, WIN, uint64_t*>
#define QMV_T_M(B, G, R, WIN)                                                                 \
    {QMV_T(B, G, R, 1, WIN), QMV_T(B, G, R, 2, WIN), QMV_T(B, G, R, 3, WIN),                   \
     QMV_T(B, G, R, 4, WIN), QMV_T(B, G, R, 5, WIN), QMV_T(B, G, R, 6, WIN),                   \
     QMV_T(B, G, R, 7, WIN), QMV_T(B, G, R, 8, WIN), QMV_T(B, G, R, 9, WIN),                   \
     QMV_T(B, G, R, 10, WIN), QMV_T(B, G, R, 11, WIN), QMV_T(B, G, R, 12, WIN),                \
     QMV_T(B, G, R, 13, WIN)}
#define QMV_T_NONE                                                                            \
    {nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, \
     nullptr, nullptr, nullptr}

extern const TimelineFn qmv_timeline_b4_g64_bf16[2][kNumR][kMaxM] = {
    {QMV_T_M(4, 64, 1, false), QMV_T_M(4, 64, 2, false), QMV_T_M(4, 64, 3, false), QMV_T_M(4, 64, 4, false)},
    {QMV_T_M(4, 64, 1, true), QMV_T_M(4, 64, 2, true), QMV_T_M(4, 64, 3, true), QMV_T_M(4, 64, 4, true)}};

// (2-bit codes have one- and two-row instances only)
extern const TimelineFn qmv_timeline_b2_g128_bf16[2][kNumR][kMaxM] = {
    {QMV_T_M(2, 128, 1, false), QMV_T_M(2, 128, 2, false), QMV_T_NONE, QMV_T_NONE},
    {QMV_T_M(2, 128, 1, true), QMV_T_M(2, 128, 2, true), QMV_T_NONE, QMV_T_NONE}};

}  // namespace qmv
