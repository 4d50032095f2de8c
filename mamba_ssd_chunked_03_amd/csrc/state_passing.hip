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
// workgroup of 256 threads covers a tile of one (b, h) state, 16 bytes of consecutive
// elements per thread (8 in bf16, 4 in fp32), so that every chunk state read and entry state
// written is one 16-byte access.  The loads of kUnroll chunks are issued before the
// dependent multiply-adds so that several requests per thread are in flight; the kernel is
// bound by HBM (it reads S and writes E once each, both in the input dtype).  The initial
// and final states are [N][P] where the chunk states are [P][N]: where a tile is whole rows
// of p (N * P a multiple of the tile), they pass through LDS and are read and written as
// 16-byte runs along p, instead of 4-byte accesses 4P bytes apart per thread.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 8;

// EPT consecutive elements of a state row, one access: 16 bytes (8 bf16 or 4 fp32) or, for
// bf16 with EPT = 4, 8 bytes
template <typename T, int EPT>
__device__ __forceinline__ void load_run(const T* src, float (&v)[EPT]) {
    if constexpr (sizeof(T) == 2) {
        static_assert(EPT == 4 || EPT == 8, "bf16 runs are 4 or 8 elements");
        uint32_t u[EPT / 2];
        if constexpr (EPT == 8) {
            const uint4 w = *reinterpret_cast<const uint4*>(src);
            u[0] = w.x; u[1] = w.y; u[2] = w.z; u[3] = w.w;
        } else {
            const uint2 w = *reinterpret_cast<const uint2*>(src);
            u[0] = w.x; u[1] = w.y;
        }
#pragma unroll
        for (int i = 0; i < EPT / 2; ++i) {
            v[2 * i] = __uint_as_float(u[i] << 16);
            v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
        }
    } else {
        static_assert(EPT == 4, "fp32 runs are 4 elements");
        const float4 w = *reinterpret_cast<const float4*>(src);
        v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
    }
}
template <typename T, int EPT>
__device__ __forceinline__ void store_run(T* dst, const float (&v)[EPT]) {
    if constexpr (sizeof(T) == 2) {
        typedef __bf16 bf16xe_t __attribute__((ext_vector_type(EPT)));
        bf16xe_t o;
#pragma unroll
        for (int i = 0; i < EPT; ++i) o[i] = (__bf16)v[i];
        *reinterpret_cast<bf16xe_t*>(dst) = o;
    } else {
        *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// T: element type of the chunk states read and of the entry states written (fp32, or bf16
// on the bf16 path, where both are matrix-core operands or their source); the running
// state stays fp32.  A thread carries EPT consecutive elements of a row of p: 4, or 8 in
// bf16 where the chunks are few (16-byte accesses; over runs of 64 chunks and more, with
// few (b, h) states, the 8-byte form measured faster: twice the threads in flight).
// REV walks the chunks last to first: the backward pass carries the entry-state gradients
// the same way, dE_c = Z_c + exp(cs[c][Q-1]) dE_{c+1} from dE_nC = dL/d final state, and
// stores dE_{c+1} (the gradient of chunk c's end state) for chunk c.
template <typename T, int EPT, bool REV>
__global__ __launch_bounds__(kThreads) void state_passing_kernel(
    const T* __restrict__ states, const float* __restrict__ cs,
    const float* __restrict__ init, T* __restrict__ entry, float* __restrict__ final_state,
    int nC, int Q, int P, int N, int tiles_per_state) {
    constexpr int TILE = kThreads * EPT;  // elements per workgroup
    constexpr int RUNS = EPT / 4;         // 16-byte fp32 runs of a thread's elements
    __shared__ __align__(16) float xs[TILE];
    const int NP = N * P;
    const int bh = blockIdx.x / tiles_per_state;
    const int tile = blockIdx.x % tiles_per_state;
    const int e = (tile * kThreads + threadIdx.x) * EPT;  // element in the [P][N] state
    // whole rows of p per workgroup, and 16-byte aligned states (the same for every
    // workgroup of the launch, so the barriers below are uniform)
    const bool staged = NP % TILE == 0;
    const bool stage_in = staged && init && ((uintptr_t)init & 15u) == 0;
    const bool stage_out = staged && final_state && ((uintptr_t)final_state & 15u) == 0;
    if (!staged && e >= NP) return;
    const int p = e / N, n = e % N;  // N % EPT == 0, so the elements share p
    // staged transfers: the workgroup's R = TILE / N rows of p from p0; for run k the thread
    // moves the 16 bytes at flat f = 4 (t + k kThreads) of the tile in [n][p] order, i.e.
    // n = f / R, p = p0 + f % R (R is a multiple of 4)
    const int R = TILE / N, p0 = tile * R;

    float s[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) s[i] = 0.f;
    if (init) {
        const float* in = init + (size_t)bh * NP;  // [N][P]
        if (stage_in) {
#pragma unroll
            for (int k = 0; k < RUNS; ++k) {
                const int f = 4 * ((int)threadIdx.x + k * kThreads), tn = f / R, tr = f % R;
                const float4 v = *reinterpret_cast<const float4*>(in + (size_t)tn * P + p0 + tr);
                xs[(tr + 0) * N + tn] = v.x;  // LDS in the workgroup's [p][n] order
                xs[(tr + 1) * N + tn] = v.y;
                xs[(tr + 2) * N + tn] = v.z;
                xs[(tr + 3) * N + tn] = v.w;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < EPT; ++i) s[i] = xs[e - tile * TILE + i];
        } else {
#pragma unroll
            for (int i = 0; i < EPT; ++i) s[i] = in[(n + i) * P + p];
        }
    }
    const size_t base = (size_t)bh * nC * NP + e;
    const float* csl = cs + (size_t)bh * nC * Q + (Q - 1);  // each chunk's total log decay
    // k-th chunk visited
    auto at = [&](int k) { return REV ? nC - 1 - k : k; };

    int c = 0;
    for (; c + kUnroll <= nC; c += kUnroll) {
        float v[kUnroll][EPT];
        float a[kUnroll];
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            load_run<T, EPT>(states + base + (size_t)at(c + k) * NP, v[k]);
            a[k] = csl[(size_t)at(c + k) * Q];
        }
#pragma unroll
        for (int k = 0; k < kUnroll; ++k) {
            store_run<T, EPT>(entry + base + (size_t)at(c + k) * NP, s);
            const float d = expf(a[k]);
#pragma unroll
            for (int i = 0; i < EPT; ++i) s[i] = fmaf(d, s[i], v[k][i]);
        }
    }
    for (; c < nC; ++c) {
        float v[EPT];
        load_run<T, EPT>(states + base + (size_t)at(c) * NP, v);
        store_run<T, EPT>(entry + base + (size_t)at(c) * NP, s);
        const float d = expf(csl[(size_t)at(c) * Q]);
#pragma unroll
        for (int i = 0; i < EPT; ++i) s[i] = fmaf(d, s[i], v[i]);
    }
    if (final_state) {
        float* out = final_state + (size_t)bh * NP;  // [N][P]
        if (stage_out) {
            if (stage_in) __syncthreads();  // every thread has read its initial state
#pragma unroll
            for (int i = 0; i < EPT; ++i) xs[e - tile * TILE + i] = s[i];
            __syncthreads();
#pragma unroll
            for (int k = 0; k < RUNS; ++k) {
                const int f = 4 * ((int)threadIdx.x + k * kThreads), tn = f / R, tr = f % R;
                *reinterpret_cast<float4*>(out + (size_t)tn * P + p0 + tr) =
                    make_float4(xs[(tr + 0) * N + tn], xs[(tr + 1) * N + tn],
                                xs[(tr + 2) * N + tn], xs[(tr + 3) * N + tn]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < EPT; ++i) out[(n + i) * P + p] = s[i];
        }
    }
}

// bf16 states over at most kLongRun chunks take 8 elements per thread, longer runs 4
constexpr int kLongRun = 32;

template <typename T, int EPT, bool REV>
hipError_t launch_passing_e(const Shape& s, const void* states, const float* cs,
                            const float* init, void* entry, float* final_state, hipStream_t st) {
    const int NP = s.N * s.P;
    const int tiles = (NP + kThreads * EPT - 1) / (kThreads * EPT);
    const unsigned blocks = (unsigned)((size_t)s.B * s.H * tiles);
    if (blocks == 0) return hipSuccess;
    state_passing_kernel<T, EPT, REV><<<blocks, kThreads, 0, st>>>(
        (const T*)states, cs, init, (T*)entry, final_state, s.nC, s.Q, s.P, s.N, tiles);
    return hipGetLastError();
}

template <bool REV>
hipError_t launch_passing_t(const Shape& s, ssd_dtype dtype, const void* states, const float* cs,
                            const float* init, void* entry, float* final_state, hipStream_t st) {
    if (dtype != SSD_BF16)
        return launch_passing_e<float, 4, REV>(s, states, cs, init, entry, final_state, st);
    if (s.nC <= kLongRun)
        return launch_passing_e<__bf16, 8, REV>(s, states, cs, init, entry, final_state, st);
    return launch_passing_e<__bf16, 4, REV>(s, states, cs, init, entry, final_state, st);
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
