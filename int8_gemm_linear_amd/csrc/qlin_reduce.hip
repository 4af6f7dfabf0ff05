// Second pass of Split-K: sums the split partials of each output element in
// split order 0..split_k-1 (so the result does not depend on which split
// finished first) and applies the scale-and-round epilogue.
#include "qlin_device.h"

namespace qlin {

template <int FMT, int SCAL>
__global__ void __launch_bounds__(256) k_reduce(KArgs p)
{
    typedef typename AccT<FMT>::v4 A4;
    typedef typename AccT<FMT>::scalar AS;
    const int n4 = (p.N + 3) >> 2;
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)p.M * n4)
        return;
    const int t = (int)(idx / n4);
    const int n = (int)(idx % n4) * 4;
    A4 sum = A4{0, 0, 0, 0};
    if (n + 3 < p.N && (p.N & 3) == 0) {
        for (int s = 0; s < p.split_k; ++s)
            sum += *reinterpret_cast<const A4 *>(part_ptr<FMT>(p, s, t, n));
        store_final4<FMT, SCAL>(p, t, n, sum);
    } else {
        for (int s = 0; s < p.split_k; ++s)
            for (int v = 0; v < 4; ++v)
                if (n + v < p.N)
                    sum[v] += *part_ptr<FMT>(p, s, t, n + v);
        for (int v = 0; v < 4; ++v)
            if (n + v < p.N)
                store_final<FMT, SCAL>(p, t, n + v, sum[v]);
    }
}

hipError_t launch_reduce(int fmt, int scal, const KArgs &a, hipStream_t s)
{
    const int64_t total = (int64_t)a.M * ((a.N + 3) / 4);
    const dim3 grid((unsigned)((total + 255) / 256));
    if (fmt == FMT_INT8)
        hipLaunchKernelGGL((k_reduce<FMT_INT8, SC_TC>), grid, dim3(256), 0, s, a);
    else if (scal == SC_BLOCK)
        hipLaunchKernelGGL((k_reduce<FMT_E4M3, SC_BLOCK>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((k_reduce<FMT_E4M3, SC_TC>), grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace qlin
