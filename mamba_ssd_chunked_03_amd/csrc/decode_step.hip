// decode_step.hip -- one recurrent step of the SSD layer for a batch of sequences.
//
// "Mamba-2: Attention's Distant Cousin" (docsaid.org), section "Working Through Four
// Tokens": the recurrent (linear) form carries a fixed-size state forward one token at a
// time, which is the form generation uses.  For every (b, h), with g = h / (H / G):
//     S <- exp(dt A) S + dt B x^T,      y = C^T S + D x
// with S the N x P state ([N][P], fp32, updated in place) -- the same arithmetic as one
// step of the oracle's recurrence.  The step is bound by HBM: the state is read and
// written once, everything else is a few hundred bytes per (b, h).
//
// One workgroup of 256 threads per (b, h).  A state row of P fp32 values is P/4 16-byte
// segments; thread t takes segment t % (P/4) of rows t / (P/4), t / (P/4) + 256 / (P/4),
// ... so that consecutive threads write consecutive bytes.  Each thread keeps the four
// partial sums of y for its columns over its rows; the 256 / (P/4) row groups are then
// added through LDS.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ float4 load_x4(const float* p) {
    return *reinterpret_cast<const float4*>(p);
}
__device__ __forceinline__ float4 load_x4(const __bf16* p) {
    const uint2 w = *reinterpret_cast<const uint2*>(p);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

template <typename T>
__global__ __launch_bounds__(kThreads) void decode_step_kernel(
    const T* __restrict__ x, const float* __restrict__ dt, const float* __restrict__ A,
    const T* __restrict__ Bm, const T* __restrict__ Cm, const float* __restrict__ D,
    float* __restrict__ state, T* __restrict__ y, int H, int G, int P, int N) {
    __shared__ float red[kThreads * 4];  // [row group][P]: 1024 floats for any P
    const int bh = blockIdx.x;
    const int h = bh % H, b = bh / H;
    const int g = h / (H / G);
    const int segs = P / 4;           // 16-byte segments per state row
    const int rpp = kThreads / segs;  // rows per pass
    const int tid = threadIdx.x;
    const int seg = tid % segs, r0 = tid / segs;
    const int p0 = seg * 4;

    const float d = dt[bh];
    const float a = expf(d * A[h]);
    const float4 xv = load_x4(x + (size_t)bh * P + p0);
    const float4 dx = make_float4(d * xv.x, d * xv.y, d * xv.z, d * xv.w);
    const T* Bg = Bm + ((size_t)b * G + g) * N;
    const T* Cg = Cm + ((size_t)b * G + g) * N;
    float* S = state + (size_t)bh * N * P;

    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int n = r0; n < N; n += rpp) {
        float4* sp = reinterpret_cast<float4*>(S + (size_t)n * P + p0);
        const float4 s = *sp;
        const float bn = to_f32(Bg[n]), cn = to_f32(Cg[n]);
        float4 o;
        o.x = fmaf(a, s.x, bn * dx.x);
        o.y = fmaf(a, s.y, bn * dx.y);
        o.z = fmaf(a, s.z, bn * dx.z);
        o.w = fmaf(a, s.w, bn * dx.w);
        *sp = o;
        acc.x = fmaf(cn, o.x, acc.x);
        acc.y = fmaf(cn, o.y, acc.y);
        acc.z = fmaf(cn, o.z, acc.z);
        acc.w = fmaf(cn, o.w, acc.w);
    }
    *reinterpret_cast<float4*>(&red[r0 * P + p0]) = acc;
    __syncthreads();
    if (tid < P) {
        float s = 0.f;
        for (int r = 0; r < rpp; ++r) s += red[r * P + tid];
        y[(size_t)bh * P + tid] = from_f32<T>(s + D[h] * to_f32(x[(size_t)bh * P + tid]));
    }
}

}  // namespace

hipError_t launch_decode_step(const Shape& s, ssd_dtype dtype, const void* x, const float* dt,
                              const float* A, const void* Bm, const void* Cm, const float* D,
                              float* state, void* y, hipStream_t st) {
    const unsigned blocks = (unsigned)((size_t)s.B * s.H);
    if (blocks == 0) return hipSuccess;
    if (dtype == SSD_F32)
        decode_step_kernel<float><<<blocks, kThreads, 0, st>>>(
            (const float*)x, dt, A, (const float*)Bm, (const float*)Cm, D, state, (float*)y,
            s.H, s.G, s.P, s.N);
    else
        decode_step_kernel<__bf16><<<blocks, kThreads, 0, st>>>(
            (const __bf16*)x, dt, A, (const __bf16*)Bm, (const __bf16*)Cm, D, state,
            (__bf16*)y, s.H, s.G, s.P, s.N);
    return hipGetLastError();
}

}  // namespace ssd
