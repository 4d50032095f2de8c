// block.hip -- the Mamba-2 block around the SSD layer, between the projections: the
// prologue (causal depthwise conv1d + SiLU on the x, B, C channels, softplus step sizes)
// and the epilogue (output gate and per-token group normalisation).
//
// "Mamba-2: Attention's Distant Cousin", section "The Mamba-2 Block" (Figure 6): one
// projection yields x, B, C and the step size together, and after the SSM the output is
// multiplied by the gate and normalised before the output projection.  Structured summary
// of arXiv 2405.21060, section "The Mamba-2 Architecture": gate y * Swish(z), GroupNorm
// after it, Swish/SiLU as the feature map on B and C; section 6.4: the convolution is
// depthwise, one-dimensional, of width 3-4.
//
// Both kernels are HBM-bound streams (a few flops per byte):
//   block_prologue_kernel: one thread per 16-byte vector of channels and 32 consecutive
//     steps of one sequence.  It walks the steps in batches of 8 loads (the next batch in
//     flight while the current one is computed), keeps the K - 1 previous inputs in
//     registers (the causal window), and writes the SiLU'd result
//     straight into x, B or C (a vector never straddles two of them: H*P and G*N are
//     multiples of 16).  The tile's threads also turn dt_raw into softplus(dt_raw + bias)
//     for the same steps, a few independent elements each.  Every input byte is read once
//     (plus the K - 1 step halo of each 32-step tile) and every output byte written once.
//   block_epilogue_kernel: a team of lanes (a power of two up to a wave) per (token,
//     normalisation group).  Its lanes read consecutive 16-byte vectors of y and z, form
//     y * silu(z) in registers, reduce the mean and then the squared deviations across the
//     team (two passes over registers), and write the normalised, scaled output.  Groups
//     too large for registers take a streaming variant that reads them three times.
#include "mfma_common.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

using mfma::bf16_hi;
using mfma::bf16_lo;
using mfma::exp2_fast;
using mfma::kLog2e;
using mfma::pack_bf16;

constexpr int kPrologueTile = 32;  // steps per prologue thread

__device__ __forceinline__ float sigmoid_fast(float v) {
    // 1 / (1 + exp(-v)); exp overflows to +inf for v < -88 and the reciprocal gives 0
    return __builtin_amdgcn_rcpf(1.f + exp2_fast(-v * kLog2e));
}
__device__ __forceinline__ float silu_f(float v) { return v * sigmoid_fast(v); }

// V consecutive elements as floats (V = 8 for bf16 and 4 for fp32 are one 16-byte access)
template <typename T, int V>
__device__ __forceinline__ void load_vec(const T* p, float (&o)[V]) {
    if constexpr (V == 8 && sizeof(T) == 2) {
        const uint4 u = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = bf16_lo(w[i]);
            o[2 * i + 1] = bf16_hi(w[i]);
        }
    } else if constexpr (V % 4 == 0 && sizeof(T) == 4) {
#pragma unroll
        for (int q = 0; q < V / 4; ++q) {
            const float4 u = *reinterpret_cast<const float4*>(p + 4 * q);
            o[4 * q] = u.x; o[4 * q + 1] = u.y; o[4 * q + 2] = u.z; o[4 * q + 3] = u.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) o[i] = to_f32(p[i]);
    }
}
template <typename T, int V>
__device__ __forceinline__ void store_vec(T* p, const float (&o)[V]) {
    if constexpr (V == 8 && sizeof(T) == 2) {
        *reinterpret_cast<uint4*>(p) = make_uint4(pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3]),
                                                  pack_bf16(o[4], o[5]), pack_bf16(o[6], o[7]));
    } else if constexpr (V == 4 && sizeof(T) == 4) {
        *reinterpret_cast<float4*>(p) = make_float4(o[0], o[1], o[2], o[3]);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) p[i] = from_f32<T>(o[i]);
    }
}

// The raw 16-byte (or element) load of V values, unpacked to floats when used
template <typename T, int V>
struct Raw {
    T v[V];
};
template <>
struct Raw<__bf16, 8> {
    uint4 u;
};
template <>
struct Raw<float, 4> {
    float4 u;
};
template <typename T, int V>
__device__ __forceinline__ Raw<T, V> load_raw(const T* p) {
    Raw<T, V> r;
    if constexpr (V == 8 && sizeof(T) == 2) {
        r.u = *reinterpret_cast<const uint4*>(p);
    } else if constexpr (V == 4 && sizeof(T) == 4) {
        r.u = *reinterpret_cast<const float4*>(p);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) r.v[i] = p[i];
    }
    return r;
}
template <typename T, int V>
__device__ __forceinline__ void unpack(const Raw<T, V>& r, float (&o)[V]) {
    if constexpr (V == 8 && sizeof(T) == 2) {
        const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            o[2 * i] = bf16_lo(w[i]);
            o[2 * i + 1] = bf16_hi(w[i]);
        }
    } else if constexpr (V == 4 && sizeof(T) == 4) {
        o[0] = r.u.x; o[1] = r.u.y; o[2] = r.u.z; o[3] = r.u.w;
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) o[i] = to_f32(r.v[i]);
    }
}

// One thread's steps [t0, tend) of one channel vector: batches of 8 steps, the loads of
// batch i + 1 issued before batch i is computed, in two buffers whose roles alternate at
// compile time (the batch loop is unrolled, so no register copies make a batch wait for
// its successor's loads).  FULL: tend - t0 == kPrologueTile, no bounds tests.
template <typename T, int V, int K, bool FULL>
__device__ __forceinline__ void prologue_tile(const T* src, long long xstride, T* dst,
                                              int dstride_o, int t0, int tend,
                                              const float (&wr)[K][V], const float (&bias)[V]) {
    constexpr int NB = kPrologueTile / 8;
    Raw<T, V> buf[2][8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
        if (FULL || t0 + j < tend) buf[0][j] = load_raw<T, V>(src + (long long)(t0 + j) * xstride);
    // win[0 .. K-2]: the K - 1 steps before the next output step; win[K-1]: that step
    float win[K][V];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
        const int t = t0 - (K - 1) + k;
        if (t >= 0) {
            unpack<T, V>(load_raw<T, V>(src + (long long)t * xstride), win[k]);
        } else {
#pragma unroll
            for (int i = 0; i < V; ++i) win[k][i] = 0.f;
        }
    }
#pragma unroll
    for (int bi = 0; bi < NB; ++bi) {
        const int tb = t0 + 8 * bi;
        if (!FULL && tb >= tend) break;
        if (bi + 1 < NB) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (FULL || tb + 8 + j < tend)
                    buf[(bi + 1) & 1][j] = load_raw<T, V>(src + (long long)(tb + 8 + j) * xstride);
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (FULL || tb + j < tend) {
                unpack<T, V>(buf[bi & 1][j], win[K - 1]);
                float o[V];
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    float a = bias[i];
#pragma unroll
                    for (int k = 0; k < K; ++k) a = fmaf(wr[k][i], win[k][i], a);
                    o[i] = silu_f(a);
                }
                store_vec<T, V>(dst + (long long)(tb + j) * dstride_o, o);
#pragma unroll
                for (int k = 0; k < K - 1; ++k)
#pragma unroll
                    for (int i = 0; i < V; ++i) win[k][i] = win[k + 1][i];
            }
        }
    }
}

template <typename T, int V, int K>
__device__ __forceinline__ void prologue_conv(const T* __restrict__ xbc, long long xstride,
                                              const float* __restrict__ w,
                                              const float* __restrict__ cb, T* __restrict__ xo,
                                              T* __restrict__ bo, T* __restrict__ co, int b,
                                              int Tn, int d, int gn, int t0, int tend, int c0) {
    T* dst;
    int dstride_o;
    if (c0 < d) {
        dst = xo + c0;
        dstride_o = d;
    } else if (c0 < d + gn) {
        dst = bo + (c0 - d);
        dstride_o = gn;
    } else {
        dst = co + (c0 - d - gn);
        dstride_o = gn;
    }
    const T* src = xbc + (long long)b * Tn * xstride + c0;
    dst += (long long)b * Tn * dstride_o;
    float wr[K][V], bias[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        bias[i] = cb ? cb[c0 + i] : 0.f;
#pragma unroll
        for (int k = 0; k < K; ++k) wr[k][i] = w[(c0 + i) * K + k];
    }
    if (tend - t0 == kPrologueTile)
        prologue_tile<T, V, K, true>(src, xstride, dst, dstride_o, t0, tend, wr, bias);
    else
        prologue_tile<T, V, K, false>(src, xstride, dst, dstride_o, t0, tend, wr, bias);
}

// grid: x = ceil(ncv / 64) conv columns, y = B * ceil(T / kPrologueTile); the step sizes
// of a tile are spread over all of its threads (a few independent loads each).
template <typename T, int V, int K>
__global__ __launch_bounds__(64) void block_prologue_kernel(
    const T* __restrict__ xbc, long long xstride, const float* __restrict__ w,
    const float* __restrict__ cb, const T* __restrict__ dt_raw, long long dstride,
    const float* __restrict__ dt_bias, T* __restrict__ xo, T* __restrict__ bo,
    T* __restrict__ co, float* __restrict__ dto, int Tn, int H, int d, int gn, int ntile) {
    const int b = blockIdx.y / ntile;
    const int t0 = (blockIdx.y % ntile) * kPrologueTile;
    const int tend = min(t0 + kPrologueTile, Tn);
    const int ncv = (d + 2 * gn) / V;
    const int cv = blockIdx.x * 64 + threadIdx.x;
    if (cv < ncv)
        prologue_conv<T, V, K>(xbc, xstride, w, cb, xo, bo, co, b, Tn, d, gn, t0, tend, cv * V);
    // the step sizes of these steps, spread over the tile's threads: all loads first (none
    // when the caller makes them elsewhere: dto null)
    const int n = dto ? (tend - t0) * H : 0, nthr = gridDim.x * 64;
    for (int e0 = cv; e0 < n; e0 += 8 * nthr) {
        float v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int e = e0 + q * nthr;
            v[q] = e < n ? to_f32(dt_raw[((long long)b * Tn + t0 + e / H) * dstride + e % H]) : 0.f;
        }
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int e = e0 + q * nthr;
            if (e < n) {
                const int h = e % H;
                const float u = dt_bias ? v[q] + dt_bias[h] : v[q];
                dto[((long long)b * Tn + t0 + e / H) * H + h] = softplus_step(u);
            }
        }
    }
}

// sum over the `lpg` lanes of an aligned team (lpg a power of two up to 64)
__device__ __forceinline__ float team_sum(float v, int lpg) {
    for (int o = 1; o < lpg; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// One team of lpg lanes per (row, group); a lane owns the vectors i * lpg + lane of its
// group (nv of them).  NVMAX > 0: exactly NVMAX = nv vectors per lane, whose gated values
// stay in registers (the count is a compile-time constant, so all loads are issued
// before the first is used); NVMAX == 0: they are re-read for each pass.
template <typename T, int V, int NVMAX>
__global__ __launch_bounds__(256) void block_epilogue_kernel(
    const T* __restrict__ y, const T* __restrict__ z, long long zstride,
    const float* __restrict__ nw, const float* __restrict__ nb, T* __restrict__ out,
    long long nteams, int d, int groups, int lpg, int nv, int rms, float eps) {
    const int lane = threadIdx.x & 63;
    const long long team =
        ((long long)blockIdx.x * 4 + (threadIdx.x >> 6)) * (64 / lpg) + lane / lpg;
    if (team >= nteams) return;  // every lane of a team leaves together
    const int tl = lane % lpg;
    const long long row = team / groups;
    const int gs = d / groups;
    const int cbase = (int)(team % groups) * gs;
    const T* yr = y + row * d + cbase;
    const T* zr = z + row * zstride + cbase;
    T* orow = out + row * d + cbase;
    const float inv_gs = 1.f / (float)gs;
    auto gated = [&](int i, float (&v)[V]) {
        const int c = (i * lpg + tl) * V;
        float zv[V];
        load_vec<T, V>(yr + c, v);
        load_vec<T, V>(zr + c, zv);
#pragma unroll
        for (int k = 0; k < V; ++k) v[k] *= silu_f(zv[k]);
    };
    const bool shift = nb && !rms;
    auto emit = [&](int i, const float (&v)[V], float mean, float rstd) {
        const int c = (i * lpg + tl) * V;
        float wv[V], bv[V];
        load_vec<float, V>(nw + cbase + c, wv);
        if (shift) {
            load_vec<float, V>(nb + cbase + c, bv);
        } else {
#pragma unroll
            for (int k = 0; k < V; ++k) bv[k] = 0.f;
        }
        float o[V];
#pragma unroll
        for (int k = 0; k < V; ++k) o[k] = fmaf((v[k] - mean) * rstd, wv[k], bv[k]);
        store_vec<T, V>(orow + c, o);
    };
    if constexpr (NVMAX > 0) {
        Raw<T, V> ry[NVMAX], rz[NVMAX];
#pragma unroll
        for (int i = 0; i < NVMAX; ++i) {
            const int c = (i * lpg + tl) * V;
            ry[i] = load_raw<T, V>(yr + c);
            rz[i] = load_raw<T, V>(zr + c);
        }
        float v[NVMAX][V];
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < NVMAX; ++i) {
            float zv[V];
            unpack<T, V>(ry[i], v[i]);
            unpack<T, V>(rz[i], zv);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                v[i][k] *= silu_f(zv[k]);
                s += v[i][k];
            }
        }
        const float mean = rms ? 0.f : team_sum(s, lpg) * inv_gs;
        float q = 0.f;
#pragma unroll
        for (int i = 0; i < NVMAX; ++i)
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float dv = v[i][k] - mean;
                q = fmaf(dv, dv, q);
            }
        const float rstd = rsqrtf(team_sum(q, lpg) * inv_gs + eps);
#pragma unroll
        for (int i = 0; i < NVMAX; ++i) emit(i, v[i], mean, rstd);
    } else {
        float s = 0.f;
        for (int i = 0; i < nv; ++i) {
            float v[V];
            gated(i, v);
#pragma unroll
            for (int k = 0; k < V; ++k) s += v[k];
        }
        const float mean = rms ? 0.f : team_sum(s, lpg) * inv_gs;
        float q = 0.f;
        for (int i = 0; i < nv; ++i) {
            float v[V];
            gated(i, v);
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const float dv = v[k] - mean;
                q = fmaf(dv, dv, q);
            }
        }
        const float rstd = rsqrtf(team_sum(q, lpg) * inv_gs + eps);
        for (int i = 0; i < nv; ++i) {
            float v[V];
            gated(i, v);
            emit(i, v, mean, rstd);
        }
    }
}

template <typename T, int V, int K>
hipError_t launch_prologue_k(const Shape& s, const BlockPrologueArgs& a, hipStream_t st) {
    const int d = s.H * s.P, gn = s.G * s.N;
    const int ncv = (d + 2 * gn) / V;
    const int ntile = (s.T + kPrologueTile - 1) / kPrologueTile;
    const dim3 grid((unsigned)((ncv + 63) / 64), (unsigned)(s.B * ntile));
    block_prologue_kernel<T, V, K><<<grid, 64, 0, st>>>(
        (const T*)a.xbc, a.xbc_stride, a.conv_w, a.conv_b, (const T*)a.dt_raw, a.dt_stride,
        a.dt_bias, (T*)a.x, (T*)a.Bm, (T*)a.Cm, a.dt, s.T, s.H, d, gn, ntile);
    return hipGetLastError();
}

template <typename T, int V>
hipError_t launch_prologue_v(const Shape& s, const BlockPrologueArgs& a, hipStream_t st) {
    switch (a.conv_k) {
        case 1: return launch_prologue_k<T, V, 1>(s, a, st);
        case 2: return launch_prologue_k<T, V, 2>(s, a, st);
        case 3: return launch_prologue_k<T, V, 3>(s, a, st);
        case 4: return launch_prologue_k<T, V, 4>(s, a, st);
        case 5: return launch_prologue_k<T, V, 5>(s, a, st);
        case 6: return launch_prologue_k<T, V, 6>(s, a, st);
        case 7: return launch_prologue_k<T, V, 7>(s, a, st);
        case 8: return launch_prologue_k<T, V, 8>(s, a, st);
    }
    return hipErrorInvalidValue;
}

template <typename T, int V, int NVMAX>
hipError_t launch_epilogue_n(const Shape& s, const BlockEpilogueArgs& a, int lpg, int nv,
                             hipStream_t st) {
    const long long nteams = (long long)s.B * s.T * a.groups;
    const long long per_block = 4LL * (64 / lpg);
    const long long blocks = (nteams + per_block - 1) / per_block;
    block_epilogue_kernel<T, V, NVMAX><<<(unsigned)blocks, 256, 0, st>>>(
        (const T*)a.y, (const T*)a.z, a.z_stride, a.norm_w, a.norm_b, (T*)a.out, nteams,
        s.H * s.P, a.groups, lpg, nv, a.rms, a.eps);
    return hipGetLastError();
}

template <typename T, int V>
hipError_t launch_epilogue_v(const Shape& s, const BlockEpilogueArgs& a, hipStream_t st) {
    const int gs = s.H * s.P / a.groups;
    const int nvec = gs / V;
    int lpg = 64;
    while (nvec % lpg != 0) lpg >>= 1;  // the largest power of two up to 64 dividing nvec
    const int nv = nvec / lpg;
    switch (nv) {  // exact counts up to 16 per lane, then the streaming variant
#define SSD_NV(K) \
    case K: return launch_epilogue_n<T, V, K>(s, a, lpg, nv, st);
        SSD_NV(1) SSD_NV(2) SSD_NV(3) SSD_NV(4) SSD_NV(5) SSD_NV(6) SSD_NV(7) SSD_NV(8)
        SSD_NV(9) SSD_NV(10) SSD_NV(11) SSD_NV(12) SSD_NV(13) SSD_NV(14) SSD_NV(15) SSD_NV(16)
#undef SSD_NV
    }
    return launch_epilogue_n<T, V, 0>(s, a, lpg, nv, st);
}

bool aligned16p(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace

hipError_t launch_block_prologue(const Shape& s, ssd_dtype dtype, const BlockPrologueArgs& a,
                                 hipStream_t st) {
    if ((long long)s.B * s.T == 0) return hipSuccess;
    const int V = dtype == SSD_BF16 ? 8 : 4;
    const bool vec = aligned16p(a.xbc) && a.xbc_stride % V == 0;
    if (dtype == SSD_BF16)
        return vec ? launch_prologue_v<__bf16, 8>(s, a, st) : launch_prologue_v<__bf16, 1>(s, a, st);
    return vec ? launch_prologue_v<float, 4>(s, a, st) : launch_prologue_v<float, 1>(s, a, st);
}

hipError_t launch_block_epilogue(const Shape& s, ssd_dtype dtype, const BlockEpilogueArgs& a,
                                 hipStream_t st) {
    if ((long long)s.B * s.T == 0) return hipSuccess;
    const int V = dtype == SSD_BF16 ? 8 : 4;
    const int gs = s.H * s.P / a.groups;
    // the vector path reads z, and the norm parameters, as 16-byte runs
    const bool vec = aligned16p(a.z) && a.z_stride % V == 0 && gs % V == 0 &&
                     aligned16p(a.norm_w) && (a.norm_b == nullptr || aligned16p(a.norm_b));
    if (dtype == SSD_BF16)
        return vec ? launch_epilogue_v<__bf16, 8>(s, a, st) : launch_epilogue_v<__bf16, 1>(s, a, st);
    return vec ? launch_epilogue_v<float, 4>(s, a, st) : launch_epilogue_v<float, 1>(s, a, st);
}

}  // namespace ssd
