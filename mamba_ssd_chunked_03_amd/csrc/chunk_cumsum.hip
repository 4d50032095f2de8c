// chunk_cumsum.hip -- stage 0 of the block decomposition: chunk-local log decays.
//
// Structured summary of arXiv 2405.21060, section "The Block-Decomposition SSD
// Algorithm", step 0 (partition into ceil(T/Q) chunks) and the 1-SS mask of section
// "The 1-Semiseparable Matrix": entries a_j ... a_{i+1} become exp(cs_j - cs_i) with
// cs the running sum of log a = dt*A inside the chunk.
//
// One workgroup of Q threads per (b, h, chunk).  Thread i reads dt[b, cQ+i, h] (all H
// heads of a chunk read the same cache lines, so L2 serves the strided reads), writes the
// chunk-major copy dt_chunk[b][h][c][i] that the later kernels read contiguously, and the
// inclusive prefix sum of dt*A over the chunk: a wave-level shuffle scan, then the
// wave totals through LDS.  HBM-bound and tiny (two fp32 values per token and head).
#include "ssd_internal.h"

namespace ssd {
namespace {

template <int Q>
__global__ __launch_bounds__(Q) void chunk_cumsum_kernel(const float* __restrict__ dt,
                                                          const float* __restrict__ A,
                                                          float* __restrict__ dtc,
                                                          float* __restrict__ cs, int T, int H,
                                                          int nC) {
    constexpr int kWaves = Q / 64;
    __shared__ float wave_sum[kWaves];
    const int c = blockIdx.x % nC;
    const int bh = blockIdx.x / nC;
    const int h = bh % H;
    const int b = bh / H;
    const int i = threadIdx.x;
    const int t = c * Q + i;
    const float v = t < T ? dt[((size_t)b * T + t) * H + h] : 0.0f;
    float run = v * A[h];
    // inclusive scan inside the 64-wide wave
    const int lane = i & 63;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const float o = __shfl_up(run, off, 64);
        if (lane >= off) run += o;
    }
    if (kWaves > 1) {
        if (lane == 63) wave_sum[i >> 6] = run;
        __syncthreads();
        float carry = 0.0f;
        for (int w = 0; w < (i >> 6); ++w) carry += wave_sum[w];
        run += carry;
    }
    const size_t o = ((size_t)bh * nC + c) * Q + i;
    dtc[o] = v;
    cs[o] = run;
}

}  // namespace

hipError_t launch_chunk_cumsum(const Shape& s, const float* dt, const float* A, float* dtc,
                               float* cs, hipStream_t st) {
    const unsigned blocks = (unsigned)((size_t)s.B * s.H * s.nC);
    if (blocks == 0) return hipSuccess;
    switch (s.Q) {
        case 64:
            chunk_cumsum_kernel<64><<<blocks, 64, 0, st>>>(dt, A, dtc, cs, s.T, s.H, s.nC);
            break;
        case 128:
            chunk_cumsum_kernel<128><<<blocks, 128, 0, st>>>(dt, A, dtc, cs, s.T, s.H, s.nC);
            break;
        case 256:
            chunk_cumsum_kernel<256><<<blocks, 256, 0, st>>>(dt, A, dtc, cs, s.T, s.H, s.nC);
            break;
        default:
            return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssd
