// qmv_stream.hip -- streaming-read ceiling: the bandwidth a one-launch,
// load-and-discard kernel reaches on a buffer of the size qmv streams, with
// the launch shape of the one-vector qmv (8-wavefront workgroups, four per
// compute unit) and the same 128-bit non-temporal loads.  The qmv's own
// fraction of the HBM peak is read against this figure.
//
// Wavefront w owns chunks [w*J*64, (w+1)*J*64) of the buffer's 16-byte
// chunks; its instruction j reads chunks (w*J + j)*64 + lane, one 1 KiB run
// per instruction (the qmv's per-instruction layout).  Each wavefront
// XOR-reduces the words it read.  With `checksum` set the wavefront XORs that
// into *out with one atomic (all wavefronts hit one address, which serializes
// them: for checking only); otherwise it stores it to *out only if it equals
// an arbitrary constant, which keeps the loads live at no cost.  The call
// launches one kernel and nothing else, so it can be captured in a HIP graph.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmv.h"

namespace {

constexpr int kWave = 64;
constexpr int kWaves = 8;      // wavefronts per workgroup
constexpr int kBatch = 4;      // loads in flight per lane

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kWaves * kWave) void stream_read_kernel(const u32x4* __restrict__ buf,
                                                                    long long nchunks, int J,
                                                                    uint32_t* __restrict__ out,
                                                                    int checksum)
{
    const int lane = threadIdx.x & (kWave - 1);
    const long long wave = (long long)blockIdx.x * kWaves + threadIdx.x / kWave;
    if (wave * J * kWave >= nchunks) return;       // wavefront-uniform: nothing left to read
    uint32_t acc = 0;
    for (int j0 = 0; j0 < J; j0 += kBatch) {
        u32x4 v[kBatch];
        bool ok[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; ++k) {
            const long long c = (wave * J + j0 + k) * kWave + lane;
            ok[k] = (j0 + k < J) && c < nchunks;
            // lanes past the end re-read the last chunk and are masked below
            v[k] = __builtin_nontemporal_load(buf + (c < nchunks ? c : nchunks - 1));
        }
#pragma unroll
        for (int k = 0; k < kBatch; ++k)
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

}  // namespace

extern "C" int qmv_stream_read(const void* buf, long long bytes, uint32_t* out, int checksum, void* stream)
{
    if (!buf || !out) return QMV_E_NULL;
    if (bytes <= 0 || bytes % 16 != 0) return QMV_E_SHAPE;
    if ((reinterpret_cast<uintptr_t>(buf) % 16) != 0 || (reinterpret_cast<uintptr_t>(out) % 4) != 0)
        return QMV_E_ALIGN;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QMV_E_LAUNCH;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        return QMV_E_LAUNCH;
    const long long nchunks = bytes / 16;
    const long long grid = 4LL * cus;                          // four 8-wavefront workgroups per CU
    const long long per_wave = (long long)kWave;               // chunks per instruction
    const long long J = (nchunks + grid * kWaves * per_wave - 1) / (grid * kWaves * per_wave);
    if (J > (1 << 20)) return QMV_E_SHAPE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)grid), dim3(kWaves * kWave), 0, s,
                       static_cast<const u32x4*>(buf), nchunks, (int)J, out, checksum);
    return hipGetLastError() == hipSuccess ? QMV_OK : QMV_E_LAUNCH;
}
