// qlin_scaled_mm_noalloc: scaled_mm / block_scaled_mm for callers that cannot
// allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid hipMalloc).  The split-K workspace is a file-scope
// device array, one copy per GPU, held until the process ends; the call
// itself allocates nothing.
//
// Host code never passes `scratch` itself to a kernel or a copy: in host
// code that name is a host-side stand-in, not a device address.  The device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per
// device with that device current, and only that address is used.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qlin_internal.h"

namespace qlin {

const size_t kScratchBytes = size_t(32) << 20;   // counters (128 KiB) + split partials

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

const int kMaxDevices = 64;

// Zeroes the counter region (the split partials need no clearing: every
// partial a call reads was written by the same call).
__global__ void __launch_bounds__(256) k_zero_counters(int4 *p, int n16)
{
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n16)
        p[i] = int4{0, 0, 0, 0};
}

struct DeviceScratch {
    void *ptr = nullptr;     // device address of this GPU's copy of `scratch`
    bool cleared = false;    // counters known to be zero (cleared outside any capture)
};

std::mutex g_mu;
DeviceScratch g_dev[kMaxDevices];

// The device address of `dev`'s copy, taken with `dev` current.
hipError_t symbol_address(int dev, void **out)
{
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess)
        return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess)
        return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
        const hipError_t e2 = hipSetDevice(cur);
        if (e == hipSuccess)
            e = e2;
    }
    if (e == hipSuccess && !p)
        e = hipErrorInvalidSymbol;
    *out = p;
    return e;
}

// This call's workspace on the stream's GPU.  The first call on a GPU clears
// the counter region with a kernel on the caller's stream (ordered before
// the call's GEMM); a call under stream capture records that clearing kernel
// into the graph, so every replay clears first, and leaves the region marked
// uncleared for the next eager call.
qlin_status scratch_for(hipStream_t stream, void **ws)
{
    int dev = -1;
    if (hipStreamGetDevice(stream, &dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return QLIN_ERR_HIP;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess)
        return QLIN_ERR_HIP;
    std::lock_guard<std::mutex> lk(g_mu);
    DeviceScratch &d = g_dev[dev];
    if (!d.ptr && symbol_address(dev, &d.ptr) != hipSuccess) {
        d.ptr = nullptr;
        return QLIN_ERR_HIP;
    }
    if (!d.cleared) {
        const int n16 = (int)(counter_bytes() / 16);
        hipLaunchKernelGGL(k_zero_counters, dim3((n16 + 255) / 256), dim3(256), 0, stream,
                           static_cast<int4 *>(d.ptr), n16);
        if (hipGetLastError() != hipSuccess)
            return QLIN_ERR_HIP;
        if (cap == hipStreamCaptureStatusNone)
            d.cleared = true;
    }
    *ws = d.ptr;
    return QLIN_OK;
}

}  // namespace
}  // namespace qlin

using namespace qlin;

extern "C" qlin_status qlin_scaled_mm_noalloc(qlin_scaling sc, qlin_dtype dt, int64_t M, int64_t N,
                                              int64_t K, const void *A, int64_t lda,
                                              const float *a_scale, const void *B, int64_t ldb,
                                              const float *b_scale, void *Y, int64_t ldy,
                                              void *stream)
{
    if ((sc != QLIN_TOKEN_CHANNEL && sc != QLIN_BLOCK128) || (dt != QLIN_E4M3 && dt != QLIN_INT8) ||
        (sc == QLIN_BLOCK128 && dt != QLIN_E4M3))
        return QLIN_ERR_BAD_ARGUMENT;
    const int fmt = dt == QLIN_INT8 ? FMT_INT8 : FMT_E4M3;
    const int scal = sc == QLIN_BLOCK128 ? SC_BLOCK : SC_TC;
    Problem pb = problem(fmt, scal, M, N, K, A, lda, a_scale, B, ldb, b_scale, Y, ldy, nullptr, 0,
                         stream);
    qlin_status st = check_problem(pb);
    if (st != QLIN_OK || M == 0 || N == 0)
        return st;
    const size_t need = selected_workspace_bytes(fmt, scal, M, N, K);
    if (need > kScratchBytes)
        return QLIN_ERR_WORKSPACE;
    if (need) {
        void *ws = nullptr;
        if ((st = scratch_for(static_cast<hipStream_t>(stream), &ws)) != QLIN_OK)
            return st;
        pb.ws = ws;
        pb.ws_bytes = kScratchBytes;
    }
    return run_problem(pb, nullptr);
}
