// chunk_mfma.hip -- stages 2 (chunk_state) and 1+4+5 (chunk_scan) on gfx950 bf16 MFMA.
//
// Both contractions run on v_mfma_f32_16x16x32_bf16 (one wave: D[16x16] += A[16x32] B[32x16],
// fp32 accumulate).  Lane l of a wave supplies row/column (l % 16) of A/B and the eight
// k-slots of lane group l / 16; it receives D rows 4*(l/16)..+3 of column l % 16.  Any
// relabelling of k works as long as A and B use the same one, which the kernels exploit
// to feed MFMA outputs straight back in as operands.
//
// The contraction index of both stages that sum over time runs along the slow (row)
// dimension of the [time][feature] tensors in HBM, so 32-step slices are staged through
// LDS in a transposed [feature][time] layout (two time steps packed per 32-bit LDS
// word), double-buffered: the global loads of slice k+1 are in flight while the MFMAs
// of slice k run.
//
// chunk_state (summary of arXiv 2405.21060, section "The Block-Decomposition SSD
// Algorithm", stage 2; the linear-attention contraction order of equation 15):
//     S[n][p] = sum_i B[i][n] x'[i][p],   x'[i][p] = exp(cs_last - cs_i) dt_i x[i][p]
// x' is formed in fp32 and rounded once to bf16.  One workgroup (4 waves) per
// (b, h, chunk); wave w owns state rows n in [w N/4, (w+1) N/4) and all of p.
//
// chunk_scan (same section, stages 1, 4, 5; the quadratic order (L o C B^T) X of
// equation 16 inside the chunk):  with the output kept transposed, Y^T[p][j],
//     Y^T  = exp(cs_j) * (E^T C^T)                          (entry state read out by C)
//          + sum over 32-step blocks of X^T (Gm^T)          (masked quadratic form)
//     Gm^T[i][j] = (B_i . C_j) exp(cs_j - cs_i) dt_i  for i <= j, else 0
// G^T = B C^T comes out of the MFMA with each lane holding four consecutive i of one
// column j -- exactly the k-slots the next MFMA (X^T Gm^T, contraction over i) needs, so
// the masked block never leaves registers.  The decay is masked before exponentiation
// (the exponent is never positive).  For blocks that lie wholly below a 16-row tile it
// is factored at the block end e, exp(cs_j - cs_e) * exp(cs_e - cs_i) -- both factors
// are <= 1 -- so only one exp per lane per block is needed there; diagonal blocks take
// one exp per element.  One workgroup of Q/32 waves per (b, h, chunk); wave w owns the
// 16-row tiles w and 2*Q/32-1-w, which balances the causal triangle's work across
// waves.  The D skip is added in the epilogue in fp32 before y is rounded to bf16.
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

// two fp32 -> packed bf16 pair (round to nearest even), as one 32-bit word
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
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
    __syncthreads();  // s_w ready
    store(0, 0);
    __syncthreads();
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
        __syncthreads();
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

// ============================================================================ chunk_scan

template <int Q, int N, int P>
__global__ __launch_bounds__(Q * 2) void chunk_scan_mfma_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Bm, const __bf16* __restrict__ Cm,
    const float* __restrict__ dtc, const float* __restrict__ cs, const float* __restrict__ D,
    const float* __restrict__ E, __bf16* __restrict__ y, int T, int H, int G, int nC) {
    constexpr int NTH = Q * 2;
    constexpr int NW = Q / 32;
    constexpr int NB = Q / KB;
    constexpr int PT = P / 16;
    constexpr int NK = N / 32;
    constexpr int LDB = N + 8;                    // row stride (bf16) of B slices and of E
    constexpr int BTASK = KB * (N / 8);           // 16-byte pieces of a B slice
    constexpr int XTASK = 16 * (P / 8);           // (row pair, 8-column group) of an x slice
    constexpr int BPT = (BTASK + NTH - 1) / NTH;
    constexpr int XPT = (XTASK + NTH - 1) / NTH;
    static_assert(N % 32 == 0 && P % 16 == 0 && Q % 64 == 0, "tile shape");

    __shared__ __align__(16) __bf16 Bs[2][KB][LDB];
    __shared__ __align__(16) __bf16 Xt[2][P][LDT];
    __shared__ __align__(16) __bf16 Es[P][LDB];
    __shared__ float s_cs[Q];  // chunk-local prefix sums of dt*A, times log2(e)
    __shared__ float s_dt[Q];
    __shared__ float s_v[Q];   // exp(cs_e - cs_i) dt_i, e = last step of i's 32-step block

    const int c = blockIdx.x % nC;
    const int bh = blockIdx.x / nC;
    const int h = bh % H;
    const int b = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const size_t cbase = ((size_t)bh * nC + c) * Q;
    const int t0 = c * Q;
    const int jt[2] = {wave, 2 * NW - 1 - wave};

    for (int i = tid; i < Q; i += NTH) {
        const float ci = cs[cbase + i];
        const float di = dtc[cbase + i];
        s_cs[i] = ci * kLog2e;
        s_dt[i] = di;
        s_v[i] = exp2_fast((cs[cbase + (i | (KB - 1))] - ci) * kLog2e) * di;
    }
    {   // entry state, fp32 [p][n] -> bf16
        const float* src = E + ((size_t)bh * nC + c) * P * N;
        for (int e = tid; e < P * N / 8; e += NTH) {
            const int p = e / (N / 8), n = (e % (N / 8)) * 8;
            const float4 u = *reinterpret_cast<const float4*>(src + (size_t)p * N + n);
            const float4 v = *reinterpret_cast<const float4*>(src + (size_t)p * N + n + 4);
            uint4 w;
            w.x = pack_bf16(u.x, u.y);
            w.y = pack_bf16(u.z, u.w);
            w.z = pack_bf16(v.x, v.y);
            w.w = pack_bf16(v.z, v.w);
            *reinterpret_cast<uint4*>(&Es[p][n]) = w;
        }
    }
    // C rows of the wave's two tiles, held as B-operand fragments for the whole kernel
    bf16x8 cf[2][NK];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int tt = t0 + jt[t] * 16 + l16;
        const __bf16* src = Cm + ((size_t)(b * T + tt) * G + g) * N + 8 * g4;
#pragma unroll
        for (int k = 0; k < NK; ++k) {
            uint4 v = make_uint4(0, 0, 0, 0);
            if (tt < T) v = *reinterpret_cast<const uint4*>(src + 32 * k);
            cf[t][k] = __builtin_bit_cast(bf16x8, v);
        }
    }

    uint4 rb[BPT], rx[XPT][2];
    auto load = [&](int ib) {
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int e = tid + q * NTH;
            const int r = e / (N / 8), cg = e % (N / 8);
            const int t = t0 + ib * KB + r;
            rb[q] = make_uint4(0, 0, 0, 0);
            if (e < BTASK && t < T)
                rb[q] = *reinterpret_cast<const uint4*>(Bm + ((size_t)(b * T + t) * G + g) * N + cg * 8);
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
    auto store = [&](int buf) {
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int e = tid + q * NTH;
            if (e >= BTASK) continue;
            const int r = e / (N / 8), cg = e % (N / 8);
            *reinterpret_cast<uint4*>(&Bs[buf][r][cg * 8]) = rb[q];
        }
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int e = tid + q * NTH;
            if (e >= XTASK) continue;
            const int rp = e % 16, cg = e / 16;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t w = bits_of(rx[q][0], k) | (bits_of(rx[q][1], k) << 16);
                *reinterpret_cast<uint32_t*>(&Xt[buf][cg * 8 + k][2 * rp]) = w;
            }
        }
    };

    load(0);
    store(0);
    __syncthreads();

    // stage 4: the entry state read out by C, decayed from the chunk start to row j
    f32x4 acc[2][PT];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            f32x4 a4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const bf16x8 ea = *reinterpret_cast<const bf16x8*>(&Es[p * 16 + l16][32 * k + 8 * g4]);
                a4 = mfma16(ea, cf[t][k], a4);
            }
            acc[t][p] = a4;
        }
        const float sc = exp2_fast(s_cs[jt[t] * 16 + l16]);
#pragma unroll
        for (int p = 0; p < PT; ++p) acc[t][p] *= sc;
    }

    // stage 1: the masked quadratic form over 32-step blocks of the chunk
    for (int ib = 0; ib < NB; ++ib) {
        const int buf = ib & 1;
        if (ib + 1 < NB) load(ib + 1);
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const int tile = jt[t];
            if (2 * ib > tile) continue;  // block wholly above this tile's rows
            f32x4 g0 = f32x4{0.f, 0.f, 0.f, 0.f}, g1 = g0;
#pragma unroll
            for (int k = 0; k < NK; ++k) {
                const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&Bs[buf][l16][32 * k + 8 * g4]);
                const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&Bs[buf][16 + l16][32 * k + 8 * g4]);
                g0 = mfma16(a0, cf[t][k], g0);
                g1 = mfma16(a1, cf[t][k], g1);
            }
            // g0[r] = G^T[i0 + r][j], g1[r] = G^T[i0 + 16 + r][j]
            const int j = tile * 16 + l16;
            const int i0 = ib * KB + 4 * g4;
            const float csj = s_cs[j];
            float m[8];
            if (2 * ib + 1 < tile) {
                const float f = exp2_fast(csj - s_cs[ib * KB + KB - 1]);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    m[r] = g0[r] * s_v[i0 + r] * f;
                    m[4 + r] = g1[r] * s_v[i0 + 16 + r] * f;
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int ia = i0 + r, ibb = i0 + 16 + r;
                    m[r] = ia <= j ? g0[r] * exp2_fast(csj - s_cs[ia]) * s_dt[ia] : 0.f;
                    m[4 + r] = ibb <= j ? g1[r] * exp2_fast(csj - s_cs[ibb]) * s_dt[ibb] : 0.f;
                }
            }
            uint4 mw;
            mw.x = pack_bf16(m[0], m[1]);
            mw.y = pack_bf16(m[2], m[3]);
            mw.z = pack_bf16(m[4], m[5]);
            mw.w = pack_bf16(m[6], m[7]);
            const bf16x8 bm = __builtin_bit_cast(bf16x8, mw);
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                const uint2 lo = *reinterpret_cast<const uint2*>(&Xt[buf][p * 16 + l16][4 * g4]);
                const uint2 hi = *reinterpret_cast<const uint2*>(&Xt[buf][p * 16 + l16][16 + 4 * g4]);
                const bf16x8 xa = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                acc[t][p] = mfma16(xa, bm, acc[t][p]);
            }
        }
        if (ib + 1 < NB) store(buf ^ 1);
        __syncthreads();
    }

    // stage 5 and the skip: y[j][p] = acc + D x[j][p]; lane holds p = pt*16 + 4*g4 + r
    const float dh = D[h];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int tt = t0 + jt[t] * 16 + l16;
        if (tt >= T) continue;
        const size_t row = ((size_t)(b * T + tt) * H + h) * P;
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            const int p0 = p * 16 + 4 * g4;
            const uint2 xv = *reinterpret_cast<const uint2*>(x + row + p0);
            uint2 out;
            out.x = pack_bf16(acc[t][p][0] + dh * bf16_lo(xv.x), acc[t][p][1] + dh * bf16_hi(xv.x));
            out.y = pack_bf16(acc[t][p][2] + dh * bf16_lo(xv.y), acc[t][p][3] + dh * bf16_hi(xv.y));
            *reinterpret_cast<uint2*>(y + row + p0) = out;
        }
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

template <int Q, int N, int P>
hipError_t launch_scan_t(const Shape& s, const void* x, const void* Bm, const void* Cm,
                         const float* dtc, const float* cs, const float* D, const float* E,
                         void* y, hipStream_t st) {
    const unsigned blocks = (unsigned)((size_t)s.B * s.H * s.nC);
    chunk_scan_mfma_kernel<Q, N, P><<<blocks, Q * 2, 0, st>>>(
        (const __bf16*)x, (const __bf16*)Bm, (const __bf16*)Cm, dtc, cs, D, E, (__bf16*)y, s.T,
        s.H, s.G, s.nC);
    return hipGetLastError();
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
using ScanFn = hipError_t (*)(const Shape&, const void*, const void*, const void*, const float*,
                              const float*, const float*, const float*, void*, hipStream_t);

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

template <int Q>
ScanFn pick_scan_q(const Shape& s) {
    switch (s.N) {
        case 32: SSD_FOR_P(launch_scan_t, Q, 32)
        case 64: SSD_FOR_P(launch_scan_t, Q, 64)
        case 128: SSD_FOR_P(launch_scan_t, Q, 128)
        case 256: SSD_FOR_P(launch_scan_t, Q, 256)
    }
    return nullptr;
}

ScanFn pick_scan(const Shape& s) {
    switch (s.Q) {
        case 64: return pick_scan_q<64>(s);
        case 128: return pick_scan_q<128>(s);
        case 256: return pick_scan_q<256>(s);
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

bool chunk_scan_mfma_supported(const Shape& s) { return pick_scan(s) != nullptr; }

hipError_t launch_chunk_scan_mfma(const Shape& s, const void* x, const void* Bm, const void* Cm,
                                  const float* dtc, const float* cs, const float* D,
                                  const float* entry, void* y, hipStream_t st) {
    ScanFn f = pick_scan(s);
    if (!f) return hipErrorInvalidValue;
    if ((size_t)s.B * s.H * s.nC == 0) return hipSuccess;
    return f(s, x, Bm, Cm, dtc, cs, D, entry, y, st);
}

}  // namespace ssd
