// Stamped kernel instances (a measurement aid): 4-bit codes, groups of 64,
// bf16 activations, bf16 scales and biases, every rows-per-wavefront and M
// the library dispatches to, whole K (scale/bias copies in LDS) and
// K-windowed.  Each is the product instance with the per-wavefront stamps
// added; the entry point that launches them is qmv_affine_timeline.
#include "qmv_kernel.hpp"
#include "qmv_dispatch.hpp"

namespace qmv {

#define QMV_T(R, M, WIN) &qmv_affine_kernel<4, 64, R, M, 1, false, true, WIN, uint64_t*>
#define QMV_T_M(R, WIN)                                                                      \
    {QMV_T(R, 1, WIN), QMV_T(R, 2, WIN), QMV_T(R, 3, WIN), QMV_T(R, 4, WIN), QMV_T(R, 5, WIN), \
     QMV_T(R, 6, WIN), QMV_T(R, 7, WIN), QMV_T(R, 8, WIN), QMV_T(R, 9, WIN), QMV_T(R, 10, WIN), \
     QMV_T(R, 11, WIN), QMV_T(R, 12, WIN), QMV_T(R, 13, WIN)}

extern const TimelineFn qmv_timeline_b4_g64_bf16[2][kNumR][kMaxM] = {
    {QMV_T_M(1, false), QMV_T_M(2, false), QMV_T_M(3, false), QMV_T_M(4, false)},
    {QMV_T_M(1, true), QMV_T_M(2, true), QMV_T_M(3, true), QMV_T_M(4, true)}};

}  // namespace qmv
