// varlen.hip -- packed variable-length rows: several sequences laid end to end in one row
// of steps, each starting from a zero state (a state belongs to one sequence: "Mamba-2:
// Attention's Distant Cousin", section "Working Through Four Tokens", starts from zero; the
// reproduction page for arXiv 2405.21060 describes context parallelism as passing states
// between contiguous pieces of one sequence).
//
// The forward stages run unchanged on the row: chunk_cumsum is given the sequence offsets
// and drops the running log-decay sum by a fixed gap at each start, which zeroes every
// decay across a start (see chunk_cumsum.hip).  Here, for fp32 and for the sizes without a
// bf16 matrix-core instantiation (chunk_mfma.hip has the MFMA one):
//   varlen_final_kernel the state after each sequence's last step t_s, in chunk c:
//     final_s = exp(cs[t_s]) E_c + sum_{i <= t_s in chunk c} exp(cs[t_s] - cs_i) dt_i B_i x_i^T
//     (E_c the chunk's entry state; with the gaps in cs, the entry state and the steps of
//     earlier sequences drop out by themselves).  One workgroup per (sequence, head, 64 x 64
//     tile of the N x P state), 32-step slabs of the weighted x and of B staged in LDS.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;

template <typename Tin>
__global__ __launch_bounds__(kThreads) void varlen_final_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ Bm, const float* __restrict__ dtc,
    const float* __restrict__ cs, const Tin* __restrict__ entry, const int* __restrict__ cu,
    float* __restrict__ finals, int T, int H, int G, int P, int N, int Q, int nC, int tilesP,
    int tilesN) {
    __shared__ float xs[32][64 + 1];
    __shared__ float bs[32][64 + 1];
    __shared__ float ws[32];
    int k = blockIdx.x;
    const int tn = k % tilesN; k /= tilesN;
    const int tp = k % tilesP; k /= tilesP;
    const int h = k % H;
    const int sq = k / H;
    const int g = h / (H / G);
    const int p0 = tp * 64, n0 = tn * 64;
    const int tx = threadIdx.x % 16, ty = threadIdx.x / 16;
    const int beg = cu[sq], end = cu[sq + 1];  // steps [beg, end)
    float acc[4][4] = {};
    if (end > beg) {
        const int te = end - 1;
        const int c = te / Q, off = te - c * Q;
        const size_t cbase = ((size_t)h * nC + c) * Q;
        const float cs_e = cs[cbase + off];
        // the chunk's entry state decayed to the last step ([P][N] in the input dtype)
        const Tin* E = entry + ((size_t)h * nC + c) * P * N;
        const float de = expf(cs_e);
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int p = p0 + ty * 4 + a, n = n0 + tx * 4 + q;
                if (p < P && n < N) acc[a][q] = de * to_f32(E[(size_t)p * N + n]);
            }
        for (int i0 = 0; i0 <= off; i0 += 32) {
            if (threadIdx.x < 32) {
                const int i = i0 + threadIdx.x;
                ws[threadIdx.x] = i <= off ? expf(cs_e - cs[cbase + i]) * dtc[cbase + i] : 0.f;
            }
            __syncthreads();
            for (int e = threadIdx.x; e < 32 * 64; e += kThreads) {
                const int r = e / 64, col = e % 64;
                const int i = i0 + r;
                const int t = c * Q + i;
                float xv = 0.f, bv = 0.f;
                if (i <= off) {
                    if (p0 + col < P) xv = to_f32(x[((size_t)t * H + h) * P + p0 + col]);
                    if (n0 + col < N) bv = to_f32(Bm[((size_t)t * G + g) * N + n0 + col]);
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
    }
    float* out = finals + ((size_t)sq * H + h) * N * P;  // [N][P]
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int p = p0 + ty * 4 + a;
        if (p >= P) continue;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int n = n0 + tx * 4 + q;
            if (n < N) out[(size_t)n * P + p] = acc[a][q];
        }
    }
}

}  // namespace

hipError_t launch_varlen_final(const Shape& s, ssd_dtype dtype, const void* x, const void* Bm,
                               const float* dtc, const float* cs, const void* entry,
                               const int* cu, int nseq, float* finals, hipStream_t st) {
    const int tilesP = (s.P + 63) / 64, tilesN = (s.N + 63) / 64;
    const unsigned blocks = (unsigned)((size_t)nseq * s.H * tilesP * tilesN);
    if (blocks == 0) return hipSuccess;
    if (dtype == SSD_F32)
        varlen_final_kernel<float><<<blocks, kThreads, 0, st>>>(
            (const float*)x, (const float*)Bm, dtc, cs, (const float*)entry, cu, finals, s.T,
            s.H, s.G, s.P, s.N, s.Q, s.nC, tilesP, tilesN);
    else
        varlen_final_kernel<__bf16><<<blocks, kThreads, 0, st>>>(
            (const __bf16*)x, (const __bf16*)Bm, dtc, cs, (const __bf16*)entry, cu, finals,
            s.T, s.H, s.G, s.P, s.N, s.Q, s.nC, tilesP, tilesN);
    return hipGetLastError();
}

}  // namespace ssd
