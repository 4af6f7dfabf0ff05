// Host-side dispatch cost of the C ABI, and what graph replay does to it.
//
// The pages report that the DSL's Python-side dispatch costs tens of
// microseconds per call outside CUDA graphs, which is why they replay graphs
// ("Building a High-Performance and Portable vLLM Linear Backend with
// Helion", section "Kernel Implementation", and the techfeed.io summary's
// hybrid-dispatch section).  This program measures the same quantities for
// libqlinear.so, from C:
//   select_us   qlin_select_config (table lookup) per call
//   reject_us   a call that fails validation (argument checks only)
//   launch_us   host time per qlin_scaled_mm call that launches, enqueued
//               in bursts of BURST calls behind a ~2 ms busy kernel (so the
//               GPU consumes nothing while the host enqueues), median over
//               bursts
//   empty_launch_us  the same for an empty kernel (HIP's own floor)
//   args_launch_us   the same for an empty kernel with a GEMM-sized argument
//                    block and a GEMM-sized grid
//   graph_launch_us  host time of one hipGraphLaunch of a graph of BURST calls
//   graph_gpu_us_per_call  GPU time per call inside the replayed graph
// Prints one JSON line.  Usage: qlin_dispatch_bench [M N K]  (W8A8_INT8).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "qlinear.h"

#define CK(x)                                                                        \
    do {                                                                             \
        hipError_t e_ = (x);                                                         \
        if (e_ != hipSuccess) {                                                      \
            std::fprintf(stderr, "HIP error %s at line %d\n", hipGetErrorString(e_), \
                         __LINE__);                                                  \
            std::exit(1);                                                            \
        }                                                                            \
    } while (0)

__global__ void k_empty() {}

// An empty kernel taking an argument block the size of the GEMM kernels'.
struct ArgBlock {
    void *p[8];
    int v[14];
};
__global__ void k_args(ArgBlock a)
{
    if (a.v[0] == 12345)
        static_cast<int *>(a.p[0])[0] = a.v[1];
}

// Keeps the GPU busy for about `cycles` shader clocks (bounded loop).
__global__ void k_busy(long long cycles)
{
    const long long t0 = clock64();
    while (clock64() - t0 < cycles) {
    }
}

static double now_us()
{
    return std::chrono::duration<double, std::micro>(
               std::chrono::steady_clock::now().time_since_epoch())
        .count();
}

static double median(std::vector<double> v)
{
    std::sort(v.begin(), v.end());
    return v[v.size() / 2];
}

int main(int argc, char **argv)
{
    const int64_t M = argc > 3 ? std::atoll(argv[1]) : 1;
    const int64_t N = argc > 3 ? std::atoll(argv[2]) : 2048;
    const int64_t K = argc > 3 ? std::atoll(argv[3]) : 2048;
    const int BURST = 256, REPS = 21;

    hipStream_t s;
    CK(hipStreamCreate(&s));
    void *A, *B, *Y, *ws;
    float *sA, *sB;
    CK(hipMalloc(&A, M * K));
    CK(hipMalloc(&B, N * K));
    CK(hipMalloc(&Y, M * N * 2));
    CK(hipMalloc(&sA, M * 4));
    CK(hipMalloc(&sB, N * 4));
    CK(hipMemset(A, 1, M * K));
    CK(hipMemset(B, 1, N * K));
    CK(hipMemset(sA, 0, M * 4));
    CK(hipMemset(sB, 0, N * 4));
    const size_t wsb = qlin_workspace_size(QLIN_TOKEN_CHANNEL, QLIN_INT8, M, N, K, nullptr);
    CK(hipMalloc(&ws, wsb > 0 ? wsb : 256));
    CK(hipMemset(ws, 0, wsb > 0 ? wsb : 256));
    qlin_config cfg;
    if (qlin_select_config(QLIN_TOKEN_CHANNEL, QLIN_INT8, M, N, K, &cfg) != QLIN_OK)
        return 1;

    auto call = [&]() {
        return qlin_scaled_mm(QLIN_INT8, M, N, K, A, K, sA, B, K, sB, Y, N, ws, wsb, s);
    };
    if (call() != QLIN_OK)
        return 1;
    CK(hipStreamSynchronize(s));

    // table lookup and validation-only cost
    const int NQ = 200000;
    double t0 = now_us();
    for (int i = 0; i < NQ; ++i)
        qlin_select_config(QLIN_TOKEN_CHANNEL, QLIN_INT8, M, N, K, &cfg);
    const double select_us = (now_us() - t0) / NQ;
    t0 = now_us();
    for (int i = 0; i < NQ; ++i)
        qlin_scaled_mm(QLIN_INT8, M, N, 24, A, K, sA, B, K, sB, Y, N, ws, wsb, s);   // K % 16 != 0
    const double reject_us = (now_us() - t0) / NQ;

    // launching calls: enqueue a burst while the GPU is held by a busy
    // kernel, so the host time is the enqueue cost alone
    const long long busy = 5000000;                       // ~2 ms of shader clocks
    std::vector<double> per;
    for (int r = 0; r < REPS; ++r) {
        hipLaunchKernelGGL(k_busy, dim3(1), dim3(64), 0, s, busy);
        t0 = now_us();
        for (int i = 0; i < BURST; ++i)
            call();
        per.push_back((now_us() - t0) / BURST);
        CK(hipStreamSynchronize(s));
    }
    const double launch_us = median(per);
    per.clear();
    for (int r = 0; r < REPS; ++r) {
        hipLaunchKernelGGL(k_busy, dim3(1), dim3(64), 0, s, busy);
        t0 = now_us();
        for (int i = 0; i < BURST; ++i)
            hipLaunchKernelGGL(k_empty, dim3(1), dim3(64), 0, s);
        per.push_back((now_us() - t0) / BURST);
        CK(hipStreamSynchronize(s));
    }
    const double empty_us = median(per);
    per.clear();
    ArgBlock ab{};
    for (int r = 0; r < REPS; ++r) {
        hipLaunchKernelGGL(k_busy, dim3(1), dim3(64), 0, s, busy);
        t0 = now_us();
        for (int i = 0; i < BURST; ++i)
            hipLaunchKernelGGL(k_args, dim3(128), dim3(512), 0, s, ab);
        per.push_back((now_us() - t0) / BURST);
        CK(hipStreamSynchronize(s));
    }
    const double args_us = median(per);

    // graph of BURST calls: host cost of one replay, GPU time per call
    hipGraph_t g;
    hipGraphExec_t ge;
    CK(hipStreamBeginCapture(s, hipStreamCaptureModeGlobal));
    for (int i = 0; i < BURST; ++i)
        call();
    CK(hipStreamEndCapture(s, &g));
    CK(hipGraphInstantiate(&ge, g, nullptr, nullptr, 0));
    CK(hipGraphLaunch(ge, s));
    CK(hipStreamSynchronize(s));
    hipEvent_t e0, e1;
    CK(hipEventCreate(&e0));
    CK(hipEventCreate(&e1));
    std::vector<double> host, gpu;
    for (int r = 0; r < REPS; ++r) {
        CK(hipEventRecord(e0, s));
        t0 = now_us();
        CK(hipGraphLaunch(ge, s));
        host.push_back(now_us() - t0);
        CK(hipEventRecord(e1, s));
        CK(hipStreamSynchronize(s));
        float ms;
        CK(hipEventElapsedTime(&ms, e0, e1));
        gpu.push_back(ms * 1e3 / BURST);
    }
    std::printf("{\"shape\": \"W8A8_INT8 M=%lld N=%lld K=%lld\", \"kernel\": %d, \"split_k\": %d, "
                "\"select_us\": %.4f, \"reject_us\": %.4f, \"launch_us\": %.3f, "
                "\"empty_launch_us\": %.3f, \"args_launch_us\": %.3f, \"graph_launch_us\": %.2f, "
                "\"graph_calls\": %d, "
                "\"graph_gpu_us_per_call\": %.3f}\n",
                (long long)M, (long long)N, (long long)K, cfg.kernel, cfg.split_k, select_us,
                reject_us, launch_us, empty_us, args_us, median(host), BURST, median(gpu));
    CK(hipGraphExecDestroy(ge));
    CK(hipGraphDestroy(g));
    return 0;
}
