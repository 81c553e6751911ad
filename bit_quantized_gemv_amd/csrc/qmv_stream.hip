// qmv_stream.hip -- streaming-read ceiling: the bandwidth a one-launch,
// load-and-discard kernel reaches on a buffer of the size qmv streams, with
// the same 128-bit non-temporal loads (one 1 KiB run per wavefront
// instruction, the qmv's per-instruction layout).  The qmv's own fraction of
// the HBM peak is read against this figure.
//
// The launch shape is a parameter, so that the ceiling can be swept over
// workgroups per compute unit, wavefronts per workgroup, loads in flight per
// lane and the order in which wavefronts walk the buffer:
//   * contiguous: wavefront w owns the 1 KiB runs [w*J, (w+1)*J) and reads
//     them in order, `batch` loads in flight;
//   * interleaved: run j*TW + w in instruction j (TW = wavefronts in the
//     grid), so at any moment the chip reads one contiguous span.
// Each wavefront XOR-reduces the words it read.  With `checksum` set the
// wavefront XORs that into *out with one atomic (all wavefronts hit one
// address, which serializes them: for checking only); otherwise it stores it
// to *out only if it equals an arbitrary constant, which keeps the loads live
// at no cost.  A call launches one kernel and nothing else, so it can be
// captured in a HIP graph.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv.h"

namespace {

constexpr int kWave = 64;
constexpr int kMaxThreads = 1024;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int B>
__global__ __launch_bounds__(kMaxThreads) void stream_read_kernel(const u32x4* __restrict__ buf,
                                                                 long long nchunks, int J,
                                                                 int interleave,
                                                                 uint32_t* __restrict__ out,
                                                                 int checksum)
{
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = blockDim.x / kWave;
    const long long gw = (long long)blockIdx.x * waves + threadIdx.x / kWave;
    const long long tw = (long long)gridDim.x * waves;
    // wavefront-uniform: a wavefront whose first run lies past the end has nothing to read
    if ((interleave ? gw : gw * J) * kWave >= nchunks) return;
    uint32_t acc = 0;
    for (int j0 = 0; j0 < J; j0 += B) {
        u32x4 v[B];
        bool ok[B];
#pragma unroll
        for (int k = 0; k < B; ++k) {
            const long long run = interleave ? (long long)(j0 + k) * tw + gw : gw * J + j0 + k;
            const long long c = run * kWave + lane;
            ok[k] = (j0 + k < J) && c < nchunks;
            // lanes past the end re-read the last chunk and are masked below
            v[k] = __builtin_nontemporal_load(buf + (c < nchunks ? c : nchunks - 1));
        }
#pragma unroll
        for (int k = 0; k < B; ++k)
            if (ok[k]) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
    }
    // wavefront XOR
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) acc ^= __shfl_xor(acc, d, kWave);
    if (lane == 0) {
        if (checksum)
            atomicXor(out, acc);
        else if (acc == 0x9e3779b9u)
            *out = acc;
    }
}

using StreamFn = void (*)(const u32x4*, long long, int, int, uint32_t*, int);

StreamFn stream_fn(int batch)
{
    switch (batch) {
    case 1: return stream_read_kernel<1>;
    case 2: return stream_read_kernel<2>;
    case 4: return stream_read_kernel<4>;
    case 8: return stream_read_kernel<8>;
    case 16: return stream_read_kernel<16>;
    default: return nullptr;
    }
}

}  // namespace

extern "C" int qmv_stream_read_ex(const void* buf, long long bytes, uint32_t* out, int checksum,
                                  int wg_per_cu, int waves_per_wg, int batch, int interleave,
                                  void* stream)
{
    if (!buf || !out) return QMV_E_NULL;
    if (bytes <= 0 || bytes % 16 != 0) return QMV_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(buf) % 16) != 0 || (reinterpret_cast<uintptr_t>(out) % 4) != 0)
        return QMV_E_ALIGN;
    if (wg_per_cu < 1 || wg_per_cu > 32 || waves_per_wg < 1 || waves_per_wg > kMaxThreads / kWave ||
        (interleave != 0 && interleave != 1))
        return QMV_E_SHAPE;
    const StreamFn fn = stream_fn(batch);
    if (!fn) return QMV_E_SHAPE;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QMV_E_LAUNCH;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return QMV_E_LAUNCH;
    const long long nchunks = bytes / 16;
    const long long grid = (long long)wg_per_cu * cus;
    const long long runs = (nchunks + kWave - 1) / kWave;                 // 1 KiB runs
    const long long waves = grid * waves_per_wg;
    const long long J = (runs + waves - 1) / waves;                       // runs per wavefront
    if (J > (1 << 20)) return QMV_E_SHAPE;
    hipLaunchKernelGGL(fn, dim3((unsigned)grid), dim3(waves_per_wg * kWave), 0,
                       static_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf), nchunks,
                       (int)J, interleave, out, checksum);
    return hipGetLastError() == hipSuccess ? QMV_OK : QMV_E_LAUNCH;
}

// The default shape: four 8-wavefront workgroups per compute unit, four loads
// in flight per lane, each wavefront on its own contiguous span.
extern "C" int qmv_stream_read(const void* buf, long long bytes, uint32_t* out, int checksum, void* stream)
{
    return qmv_stream_read_ex(buf, bytes, out, checksum, 4, 8, 4, 0, stream);
}
