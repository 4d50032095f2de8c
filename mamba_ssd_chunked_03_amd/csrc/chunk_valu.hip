// chunk_valu.hip -- stages 1, 2, 4 and 5 with plain fp32 vector arithmetic.
//
// These kernels cover every supported size and both input dtypes, accumulating in fp32
// from fp32 operands, so they are the path for fp32 inputs (where bf16 operand rounding
// would cost more accuracy than the fp32 contract allows) and for sizes the MFMA kernels
// are not instantiated for.  They follow the same formulas as the MFMA kernels:
//
// chunk_state (summary of arXiv 2405.21060, section "The Block-Decomposition SSD
// Algorithm", stage 2): S_c[p][n] = sum_i x'[i][p] B[i][n], x' = exp(cs_last - cs_i) dt_i x_i.
// One workgroup per (b, h, chunk, 64x64 output tile); 32-row slabs of x' and B staged in
// LDS; each thread owns a 4x4 block of the tile.
//
// chunk_scan (same section, stages 1, 4, 5; dual form of section "The Scalar-Identity
// SSM", M = L o (C B^T)): one workgroup per (b, h, chunk, 16-row tile).  Phase one puts
// the masked, decayed, dt-scaled block Gm[j][i] = (C_j . B_i) exp(cs_j - cs_i) dt_i
// (i <= j, computed only there so the exponent is never positive) in LDS; phase two
// forms y[j][p] = sum_i Gm[j][i] x[i][p] + exp(cs_j) C_j . E[p] + D x[j][p].
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;

// REV: the backward pass's mirror (C for B, dy for x, weight exp(cs_i)), see chunk_mfma.hip
template <typename Tin, bool REV>
__global__ __launch_bounds__(kThreads) void chunk_state_valu_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ Bm, const float* __restrict__ dtc,
    const float* __restrict__ cs, Tin* __restrict__ states, int T, int H, int G, int P, int N,
    int Q, int nC, int tilesP, int tilesN) {
    __shared__ float xs[32][64 + 1];
    __shared__ float bs[32][64 + 1];
    __shared__ float ws[32];
    int k = blockIdx.x;
    const int tn = k % tilesN; k /= tilesN;
    const int tp = k % tilesP; k /= tilesP;
    const int c = k % nC; k /= nC;
    const int h = k % H;
    const int b = k / H;
    const int g = h / (H / G);
    const int p0 = tp * 64, n0 = tn * 64;
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const size_t cbase = ((size_t)(b * H + h) * nC + c) * Q;
    const float cs_last = cs[cbase + Q - 1];

    float acc[4][4] = {};
    for (int i0 = 0; i0 < Q; i0 += 32) {
        if (threadIdx.x < 32) {
            const int i = i0 + threadIdx.x;
            ws[threadIdx.x] =
                REV ? expf(cs[cbase + i]) : expf(cs_last - cs[cbase + i]) * dtc[cbase + i];
        }
        __syncthreads();
        for (int e = threadIdx.x; e < 32 * 64; e += kThreads) {
            const int r = e / 64, col = e % 64;
            const int t = c * Q + i0 + r;
            float xv = 0.f, bv = 0.f;
            if (t < T) {
                if (p0 + col < P) xv = to_f32(x[((size_t)(b * T + t) * H + h) * P + p0 + col]);
                if (n0 + col < N) bv = to_f32(Bm[((size_t)(b * T + t) * G + g) * N + n0 + col]);
            }
            xs[r][col] = ws[r] * xv;
            bs[r][col] = bv;
        }
        __syncthreads();
        for (int r = 0; r < 32; ++r) {
            float xa[4], ba[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                xa[q] = xs[r][ty * 4 + q];
                ba[q] = bs[r][tx * 4 + q];
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int q = 0; q < 4; ++q) acc[a][q] = fmaf(xa[a], ba[q], acc[a][q]);
        }
        __syncthreads();
    }
    Tin* out = states + ((size_t)(b * H + h) * nC + c) * P * N;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int p = p0 + ty * 4 + a;
        if (p >= P) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + tx * 4 + q;
            if (n < N) out[(size_t)p * N + n] = from_f32<Tin>(acc[a][q]);
        }
    }
}

constexpr int kRows = 16;  // chunk_scan rows per workgroup

template <typename Tin>
__global__ __launch_bounds__(kThreads) void chunk_scan_valu_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ Bm, const Tin* __restrict__ Cm,
    const float* __restrict__ dtc, const float* __restrict__ cs, const float* __restrict__ D,
    const Tin* __restrict__ entry, Tin* __restrict__ y, int T, int H, int G, int P, int N,
    int Q, int nC) {
    __shared__ float gm[kRows][256];
    __shared__ float cj[kRows][256];
    const int rtiles = Q / kRows;
    int k = blockIdx.x;
    const int rt = k % rtiles; k /= rtiles;
    const int c = k % nC; k /= nC;
    const int h = k % H;
    const int b = k / H;
    const int g = h / (H / G);
    const int j0 = rt * kRows;
    const int t0 = c * Q;
    if (t0 + j0 >= T) return;
    const size_t cbase = ((size_t)(b * H + h) * nC + c) * Q;
    const int iend = j0 + kRows;  // columns i < iend can be unmasked for these rows

    for (int e = threadIdx.x; e < kRows * N; e += kThreads) {
        const int r = e / N, n = e % N;
        const int t = t0 + j0 + r;
        cj[r][n] = t < T ? to_f32(Cm[((size_t)(b * T + t) * G + g) * N + n]) : 0.f;
    }
    __syncthreads();
    for (int e = threadIdx.x; e < kRows * iend; e += kThreads) {
        const int r = e / iend, i = e % iend;
        const int j = j0 + r;
        float v = 0.f;
        if (i <= j && t0 + i < T) {
            const Tin* bi = Bm + ((size_t)(b * T + t0 + i) * G + g) * N;
            float dot = 0.f;
            for (int n = 0; n < N; ++n) dot = fmaf(cj[r][n], to_f32(bi[n]), dot);
            v = dot * expf(cs[cbase + j] - cs[cbase + i]) * dtc[cbase + i];
        }
        gm[r][i] = v;
    }
    __syncthreads();
    const Tin* E = entry + ((size_t)(b * H + h) * nC + c) * P * N;
    const float dh = D[h];
    for (int e = threadIdx.x; e < kRows * P; e += kThreads) {
        const int r = e / P, p = e % P;
        const int j = j0 + r;
        const int t = t0 + j;
        if (t >= T) continue;
        float acc = 0.f;
        for (int i = 0; i <= j; ++i)
            acc = fmaf(gm[r][i], to_f32(x[((size_t)(b * T + t0 + i) * H + h) * P + p]), acc);
        float off = 0.f;
        for (int n = 0; n < N; ++n) off = fmaf(cj[r][n], to_f32(E[(size_t)p * N + n]), off);
        const float xv = to_f32(x[((size_t)(b * T + t) * H + h) * P + p]);
        acc += expf(cs[cbase + j]) * off + dh * xv;
        y[((size_t)(b * T + t) * H + h) * P + p] = from_f32<Tin>(acc);
    }
}

template <bool REV>
hipError_t launch_state_valu_t(const Shape& s, ssd_dtype dt, const void* x, const void* Bm,
                               const float* dtc, const float* cs, void* states, hipStream_t st) {
    const int tilesP = (s.P + 63) / 64, tilesN = (s.N + 63) / 64;
    const unsigned blocks = (unsigned)((size_t)s.B * s.H * s.nC * tilesP * tilesN);
    if (blocks == 0) return hipSuccess;
    if (dt == SSD_F32)
        chunk_state_valu_kernel<float, REV><<<blocks, kThreads, 0, st>>>(
            (const float*)x, (const float*)Bm, dtc, cs, (float*)states, s.T, s.H, s.G, s.P, s.N,
            s.Q, s.nC, tilesP, tilesN);
    else
        chunk_state_valu_kernel<__bf16, REV><<<blocks, kThreads, 0, st>>>(
            (const __bf16*)x, (const __bf16*)Bm, dtc, cs, (__bf16*)states, s.T, s.H, s.G, s.P,
            s.N, s.Q, s.nC, tilesP, tilesN);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_state_valu(const Shape& s, ssd_dtype dt, const void* x, const void* Bm,
                                   const float* dtc, const float* cs, void* states,
                                   hipStream_t st) {
    return launch_state_valu_t<false>(s, dt, x, Bm, dtc, cs, states, st);
}

hipError_t launch_chunk_dstate_valu(const Shape& s, ssd_dtype dt, const void* dy, const void* Cm,
                                    const float* cs, void* dstates, hipStream_t st) {
    return launch_state_valu_t<true>(s, dt, dy, Cm, cs, cs, dstates, st);
}

hipError_t launch_chunk_scan_valu(const Shape& s, ssd_dtype dt, const void* x, const void* Bm,
                                  const void* Cm, const float* dtc, const float* cs,
                                  const float* D, const void* entry, void* y, hipStream_t st) {
    const unsigned blocks = (unsigned)((size_t)s.B * s.H * s.nC * (s.Q / kRows));
    if (blocks == 0) return hipSuccess;
    if (dt == SSD_F32)
        chunk_scan_valu_kernel<float><<<blocks, kThreads, 0, st>>>(
            (const float*)x, (const float*)Bm, (const float*)Cm, dtc, cs, D, (const float*)entry, (float*)y, s.T,
            s.H, s.G, s.P, s.N, s.Q, s.nC);
    else
        chunk_scan_valu_kernel<__bf16><<<blocks, kThreads, 0, st>>>(
            (const __bf16*)x, (const __bf16*)Bm, (const __bf16*)Cm, dtc, cs, D, (const __bf16*)entry, (__bf16*)y,
            s.T, s.H, s.G, s.P, s.N, s.Q, s.nC);
    return hipGetLastError();
}

}  // namespace ssd
