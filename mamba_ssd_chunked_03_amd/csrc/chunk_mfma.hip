// chunk_mfma.hip -- stage 2 (chunk_state) on gfx950 bf16 MFMA.
//
// Summary of arXiv 2405.21060, section "The Block-Decomposition SSD Algorithm", stage 2
// (the linear-attention contraction order of equation 15):
//     S[n][p] = sum_i B[i][n] x'[i][p],   x'[i][p] = exp(cs_last - cs_i) dt_i x[i][p]
// x' is formed in fp32 and rounded once to bf16.  v_mfma_f32_16x16x32_bf16 contracts over
// time, which runs along the slow (row) dimension of B and x in HBM, so 32-step slices
// are staged through LDS in a transposed [feature][time] layout (two time steps packed
// per 32-bit LDS word), double-buffered through registers.  One workgroup (4 waves) per
// (b, h, chunk); wave w owns state rows n in [w N/4, (w+1) N/4) and all of p.
#include "ssd_internal.h"

namespace ssd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int KB = 32;  // time steps per LDS slice = k of one MFMA
constexpr int LDT = KB + 8;  // row stride (bf16) of the transposed [feature][time] slices

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }

// Workgroup barrier for data exchanged through LDS only.  __syncthreads() is a full
// workgroup fence that also waits for every outstanding global load and store
// (vmcnt(0)), which would drain the register prefetch of the next slice or head at
// every barrier; here only this wave's LDS operations are waited for.  The empty asm
// with a memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// two fp32 -> packed bf16 pair (round to nearest even), as one 32-bit word
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// v if keep, else zeros -- per component, so that it stays a register select
__device__ __forceinline__ uint4 keep_or_zero(bool keep, uint4 v) {
    return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

// element k (0..7) of a 16-byte vector of bf16, as raw 16 bits in the low half
__device__ __forceinline__ uint32_t bits_of(const uint4& v, int k) {
    const uint32_t w = k < 2 ? v.x : k < 4 ? v.y : k < 6 ? v.z : v.w;
    return (k & 1) ? (w >> 16) : (w & 0xffffu);
}

// ============================================================================ chunk_state

template <int Q, int N, int P>
__global__ __launch_bounds__(256) void chunk_state_mfma_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Bm, const float* __restrict__ dtc,
    const float* __restrict__ cs, float* __restrict__ states, int T, int H, int G, int nC) {
    constexpr int NTH = 256;
    constexpr int NB = Q / KB;
    constexpr int PT = P / 16;
    constexpr int NTW = N / 64;                   // 16-row n-tiles per wave
    constexpr int BTASK = 16 * (N / 8);           // (row pair, 8-column group) tasks for B
    constexpr int XTASK = 16 * (P / 8);           // ... and for x
    constexpr int BPT = (BTASK + NTH - 1) / NTH;  // tasks per thread
    constexpr int XPT = (XTASK + NTH - 1) / NTH;
    static_assert(N % 64 == 0 && P % 16 == 0, "tile shape");

    __shared__ __align__(16) __bf16 Bt[2][N][LDT];
    __shared__ __align__(16) __bf16 Xt[2][P][LDT];
    __shared__ float s_w[Q];

    const int c = blockIdx.x % nC;
    const int bh = blockIdx.x / nC;
    const int h = bh % H;
    const int b = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const size_t cbase = ((size_t)bh * nC + c) * Q;
    const int t0 = c * Q;

    // decay to the chunk end times dt, per step (fp32)
    const float cs_last = cs[cbase + Q - 1];
    for (int i = tid; i < Q; i += NTH) s_w[i] = expf(cs_last - cs[cbase + i]) * dtc[cbase + i];

    uint4 rb[BPT][2], rx[XPT][2];
    auto load = [&](int ib) {
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int e = tid + q * NTH;
            const int rp = e % 16, cg = e / 16;
            const int t = t0 + ib * KB + 2 * rp;
            rb[q][0] = rb[q][1] = make_uint4(0, 0, 0, 0);
            if (e < BTASK) {
                const __bf16* src = Bm + ((size_t)(b * T + t) * G + g) * N + cg * 8;
                if (t < T) rb[q][0] = *reinterpret_cast<const uint4*>(src);
                if (t + 1 < T) rb[q][1] = *reinterpret_cast<const uint4*>(src + (size_t)G * N);
            }
        }
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int e = tid + q * NTH;
            const int rp = e % 16, cg = e / 16;
            const int t = t0 + ib * KB + 2 * rp;
            rx[q][0] = rx[q][1] = make_uint4(0, 0, 0, 0);
            if (e < XTASK) {
                const __bf16* src = x + ((size_t)(b * T + t) * H + h) * P + cg * 8;
                if (t < T) rx[q][0] = *reinterpret_cast<const uint4*>(src);
                if (t + 1 < T) rx[q][1] = *reinterpret_cast<const uint4*>(src + (size_t)H * P);
            }
        }
    };
    auto store = [&](int buf, int ib) {
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int e = tid + q * NTH;
            if (e >= BTASK) continue;
            const int rp = e % 16, cg = e / 16;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t w = bits_of(rb[q][0], k) | (bits_of(rb[q][1], k) << 16);
                *reinterpret_cast<uint32_t*>(&Bt[buf][cg * 8 + k][2 * rp]) = w;
            }
        }
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int e = tid + q * NTH;
            if (e >= XTASK) continue;
            const int rp = e % 16, cg = e / 16;
            const float w0 = s_w[ib * KB + 2 * rp], w1 = s_w[ib * KB + 2 * rp + 1];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float v0 = __uint_as_float(bits_of(rx[q][0], k) << 16) * w0;
                const float v1 = __uint_as_float(bits_of(rx[q][1], k) << 16) * w1;
                *reinterpret_cast<uint32_t*>(&Xt[buf][cg * 8 + k][2 * rp]) = pack_bf16(v0, v1);
            }
        }
    };

    f32x4 acc[NTW][PT];
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
        for (int p = 0; p < PT; ++p) acc[a][p] = f32x4{0.f, 0.f, 0.f, 0.f};

    load(0);
    lds_barrier();  // s_w ready
    store(0, 0);
    lds_barrier();
    for (int ib = 0; ib < NB; ++ib) {
        const int buf = ib & 1;
        if (ib + 1 < NB) load(ib + 1);
        bf16x8 bx[PT];
#pragma unroll
        for (int p = 0; p < PT; ++p)
            bx[p] = *reinterpret_cast<const bf16x8*>(&Xt[buf][p * 16 + l16][8 * g4]);
#pragma unroll
        for (int a = 0; a < NTW; ++a) {
            const bf16x8 ba =
                *reinterpret_cast<const bf16x8*>(&Bt[buf][(wave * NTW + a) * 16 + l16][8 * g4]);
#pragma unroll
            for (int p = 0; p < PT; ++p) acc[a][p] = mfma16(ba, bx[p], acc[a][p]);
        }
        if (ib + 1 < NB) store(buf ^ 1, ib + 1);
        lds_barrier();
    }
    // lane holds S[n = tile*16 + 4*g4 + r][p = pt*16 + l16]; layout [p][n]
    float* out = states + ((size_t)bh * nC + c) * P * N;
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            const int n0 = (wave * NTW + a) * 16 + 4 * g4;
            const int pp = p * 16 + l16;
            *reinterpret_cast<float4*>(out + (size_t)pp * N + n0) =
                make_float4(acc[a][p][0], acc[a][p][1], acc[a][p][2], acc[a][p][3]);
        }
}

// ---------------------------------------------------------------- dispatch tables

template <int Q, int N, int P>
hipError_t launch_state_t(const Shape& s, const void* x, const void* Bm, const float* dtc,
                          const float* cs, float* states, hipStream_t st) {
    const unsigned blocks = (unsigned)((size_t)s.B * s.H * s.nC);
    chunk_state_mfma_kernel<Q, N, P><<<blocks, 256, 0, st>>>(
        (const __bf16*)x, (const __bf16*)Bm, dtc, cs, states, s.T, s.H, s.G, s.nC);
    return hipGetLastError();
}

// Heads of one (batch, group, chunk) unit are split into `ranges` workgroups so that the
// grid covers the GPU's 256 CUs at least once, keeping >= 4 heads per workgroup where the
// group has that many (each workgroup pays one C B^T setup for its range).
inline void scan_split(const Shape& s, int* heads_per_wg, int* ranges) {
    const long units = (long)s.B * s.G * s.nC;
    const int hpg = s.H / s.G;
    int want = (int)((256 + units - 1) / units);  // >= 256 pairs = 2 workgroups per CU
    int maxr = hpg / 4 > 0 ? hpg / 4 : 1;
    int r = want < maxr ? want : maxr;
    if (r < 1) r = 1;
    *heads_per_wg = (hpg + r - 1) / r;
    *ranges = (hpg + *heads_per_wg - 1) / *heads_per_wg;
}

#define SSD_FOR_P(F, Q, N)                                   \
    switch (s.P) {                                           \
        case 16: return F<Q, N, 16>;                         \
        case 32: return F<Q, N, 32>;                         \
        case 64: return F<Q, N, 64>;                         \
        case 128: return F<Q, N, 128>;                       \
    }                                                        \
    break;

using StateFn = hipError_t (*)(const Shape&, const void*, const void*, const float*, const float*,
                               float*, hipStream_t);

template <int Q>
StateFn pick_state_q(const Shape& s) {
    switch (s.N) {
        case 64: SSD_FOR_P(launch_state_t, Q, 64)
        case 128: SSD_FOR_P(launch_state_t, Q, 128)
        case 256: SSD_FOR_P(launch_state_t, Q, 256)
    }
    return nullptr;
}

StateFn pick_state(const Shape& s) {
    switch (s.Q) {
        case 64: return pick_state_q<64>(s);
        case 128: return pick_state_q<128>(s);
        case 256: return pick_state_q<256>(s);
    }
    return nullptr;
}

}  // namespace

bool chunk_state_mfma_supported(const Shape& s) { return pick_state(s) != nullptr; }

hipError_t launch_chunk_state_mfma(const Shape& s, const void* x, const void* Bm,
                                   const float* dtc, const float* cs, float* states,
                                   hipStream_t st) {
    StateFn f = pick_state(s);
    if (!f) return hipErrorInvalidValue;
    if ((size_t)s.B * s.H * s.nC == 0) return hipSuccess;
    return f(s, x, Bm, dtc, cs, states, st);
}

}  // namespace ssd
