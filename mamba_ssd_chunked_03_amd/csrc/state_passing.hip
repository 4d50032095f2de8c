// state_passing.hip -- stage 3 of the block decomposition: carry states across chunks.
//
// Structured summary of arXiv 2405.21060, section "The Block-Decomposition SSD
// Algorithm", stage 3 ("Propagate states between chunks"): the true state after chunk c
// is a 1-SS matrix applied to the sequence of chunk states, i.e. the scalar recurrence
// (section "The 1-Semiseparable Matrix", equation 7) run over chunks with the chunk's
// total decay as the scalar:
//     E_0 = init,   E_{c+1} = exp(cs[c][Q-1]) * E_c + S_c,   final = E_nC.
// The pages' subscripts for this chunk decay are garbled; this is the reading that
// reproduces the token recurrence (checked against the oracle's boundary states).
//
// Every (b, h, p, n) element is an independent lane of a length-nC sequential scan.  A
// workgroup of 256 threads covers 1024 elements of one (b, h) state, four consecutive
// elements per thread.  The loads of kUnroll chunks are issued before the dependent
// multiply-adds so that several requests per thread are in flight; the kernel is bound by
// HBM (it reads S and writes E once each, both in the input dtype).  The initial and final
// states are [N][P] where the chunk states are [P][N]: where a workgroup's 1024 elements are
// whole rows of p (N * P a multiple of 1024), they pass through LDS and are read and written
// as 16-byte runs along p, instead of four 4-byte accesses 4P bytes apart per thread.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

__device__ __forceinline__ float4 fma4(float a, float4 s, float4 v) {
    return make_float4(fmaf(a, s.x, v.x), fmaf(a, s.y, v.y), fmaf(a, s.z, v.z), fmaf(a, s.w, v.w));
}

__device__ __forceinline__ float4 load4(const float* src) {
    return *reinterpret_cast<const float4*>(src);
}
__device__ __forceinline__ float4 load4(const __bf16* src) {
    const uint2 w = *reinterpret_cast<const uint2*>(src);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u));
}

__device__ __forceinline__ void store4(float* dst, float4 v) {
    *reinterpret_cast<float4*>(dst) = v;
}
__device__ __forceinline__ void store4(__bf16* dst, float4 v) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 o;
    o[0] = (__bf16)v.x;
    o[1] = (__bf16)v.y;
    o[2] = (__bf16)v.z;
    o[3] = (__bf16)v.w;
    *reinterpret_cast<bf16x4*>(dst) = o;
}

// T: element type of the chunk states read and of the entry states written (fp32, or bf16
// on the bf16 path, where both are matrix-core operands or their source); the running
// state stays fp32.
// REV walks the chunks last to first: the backward pass carries the entry-state gradients
// the same way, dE_c = Z_c + exp(cs[c][Q-1]) dE_{c+1} from dE_nC = dL/d final state, and
// stores dE_{c+1} (the gradient of chunk c's end state) for chunk c.
template <typename T, bool REV>
__global__ __launch_bounds__(kThreads) void state_passing_kernel(
    const T* __restrict__ states, const float* __restrict__ cs,
    const float* __restrict__ init, T* __restrict__ entry, float* __restrict__ final_state,
    int nC, int Q, int P, int N, int tiles_per_state) {
    constexpr int TILE = kThreads * 4;  // elements per workgroup
    __shared__ __align__(16) float xs[TILE];
    const int NP = N * P;
    const int bh = blockIdx.x / tiles_per_state;
    const int tile = blockIdx.x % tiles_per_state;
    const int e = (tile * kThreads + threadIdx.x) * 4;  // element in the [P][N] state
    // whole rows of p per workgroup, and 16-byte aligned states (the same for every
    // workgroup of the launch, so the barriers below are uniform)
    const bool staged = NP % TILE == 0;
    const bool stage_in = staged && init && ((uintptr_t)init & 15u) == 0;
    const bool stage_out = staged && final_state && ((uintptr_t)final_state & 15u) == 0;
    if (!staged && e >= NP) return;
    const int p = e / N, n = e % N;  // N % 4 == 0, so the four elements share p
    // staged transfers: the workgroup's R = TILE / N rows of p from p0; thread t moves the
    // 16-byte run at n = 4t / R, p = p0 + 4t % R of the [N][P] state (R is a multiple of 4)
    const int R = TILE / N, p0 = tile * R;
    const int tn = (int)(threadIdx.x * 4) / R, tr = (int)(threadIdx.x * 4) % R;

    float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
    if (init) {
        const float* in = init + (size_t)bh * NP;  // [N][P]
        if (stage_in) {
            const float4 v = *reinterpret_cast<const float4*>(in + (size_t)tn * P + p0 + tr);
            xs[(tr + 0) * N + tn] = v.x;  // LDS in the workgroup's [p][n] order
            xs[(tr + 1) * N + tn] = v.y;
            xs[(tr + 2) * N + tn] = v.z;
            xs[(tr + 3) * N + tn] = v.w;
            __syncthreads();
            s = *reinterpret_cast<const float4*>(xs + (e - tile * TILE));
        } else {
            s = make_float4(in[(n + 0) * P + p], in[(n + 1) * P + p], in[(n + 2) * P + p],
                            in[(n + 3) * P + p]);
        }
    }
    const size_t base = (size_t)bh * nC * NP + e;
    const float* csl = cs + (size_t)bh * nC * Q + (Q - 1);  // each chunk's total log decay
    // k-th chunk visited
    auto at = [&](int k) { return REV ? nC - 1 - k : k; };

    int c = 0;
    for (; c + kUnroll <= nC; c += kUnroll) {
        float4 v[kUnroll];
        float a[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            v[k] = load4(states + base + (size_t)at(c + k) * NP);
            a[k] = csl[(size_t)at(c + k) * Q];
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            store4(entry + base + (size_t)at(c + k) * NP, s);
            s = fma4(expf(a[k]), s, v[k]);
        }
    }
    for (; c < nC; ++c) {
        const float4 v = load4(states + base + (size_t)at(c) * NP);
        store4(entry + base + (size_t)at(c) * NP, s);
        s = fma4(expf(csl[(size_t)at(c) * Q]), s, v);
    }
    if (final_state) {
        float* out = final_state + (size_t)bh * NP;  // [N][P]
        if (stage_out) {
            if (stage_in) __syncthreads();  // every thread has read its initial state
            *reinterpret_cast<float4*>(xs + (e - tile * TILE)) = s;
            __syncthreads();
            *reinterpret_cast<float4*>(out + (size_t)tn * P + p0 + tr) =
                make_float4(xs[(tr + 0) * N + tn], xs[(tr + 1) * N + tn], xs[(tr + 2) * N + tn],
                            xs[(tr + 3) * N + tn]);
        } else {
            out[(n + 0) * P + p] = s.x;
            out[(n + 1) * P + p] = s.y;
            out[(n + 2) * P + p] = s.z;
            out[(n + 3) * P + p] = s.w;
        }
    }
}

template <bool REV>
hipError_t launch_passing_t(const Shape& s, ssd_dtype dtype, const void* states, const float* cs,
                            const float* init, void* entry, float* final_state, hipStream_t st) {
    const int NP = s.N * s.P;
    const int tiles = (NP + kThreads * 4 - 1) / (kThreads * 4);
    const unsigned blocks = (unsigned)((size_t)s.B * s.H * tiles);
    if (blocks == 0) return hipSuccess;
    if (dtype == SSD_BF16)
        state_passing_kernel<__bf16, REV><<<blocks, kThreads, 0, st>>>(
            (const __bf16*)states, cs, init, (__bf16*)entry, final_state, s.nC, s.Q, s.P, s.N,
            tiles);
    else
        state_passing_kernel<float, REV><<<blocks, kThreads, 0, st>>>(
            (const float*)states, cs, init, (float*)entry, final_state, s.nC, s.Q, s.P, s.N,
            tiles);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_state_passing(const Shape& s, ssd_dtype dtype, const void* states,
                                const float* cs, const float* init, void* entry,
                                float* final_state, hipStream_t st) {
    return launch_passing_t<false>(s, dtype, states, cs, init, entry, final_state, st);
}

hipError_t launch_state_passing_rev(const Shape& s, ssd_dtype dtype, const void* dstates,
                                    const float* cs, const float* d_final, void* exit_grads,
                                    float* d_init, hipStream_t st) {
    return launch_passing_t<true>(s, dtype, dstates, cs, d_final, exit_grads, d_init, st);
}

}  // namespace ssd
