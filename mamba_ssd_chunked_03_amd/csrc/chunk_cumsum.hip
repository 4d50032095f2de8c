// chunk_cumsum.hip -- stage 0 of the block decomposition: chunk-local log decays.
//
// Structured summary of arXiv 2405.21060, section "The Block-Decomposition SSD
// Algorithm", step 0 (partition into ceil(T/Q) chunks) and the 1-SS mask of section
// "The 1-Semiseparable Matrix": entries a_j ... a_{i+1} become exp(cs_j - cs_i) with
// cs the running sum of log a = dt*A inside the chunk.
//
// One workgroup of 16 waves per (b, chunk, block of 16 heads).  dt is [B][T][H], so a
// chunk's steps for a block of heads are Q rows of 64 contiguous bytes: the workgroup
// reads them coalesced into an LDS tile [head][time], then wave w takes head w: a lane
// holds Q/64 consecutive steps, scans them serially, and a 64-wide DPP scan adds the
// carry of the lanes before it.  It writes the chunk-major copy dt_chunk[b][h][c][i] that
// the later kernels read contiguously, and the inclusive prefix sum cs of dt*A over the
// chunk, both as contiguous rows (one vector store per lane each).  The kernel is
// latency-bound: every load is issued before any is used, and all heads of the block are
// scanned at once.
//
// Step sizes fused in (the block path): instead of dt, the kernel can read the raw step
// sizes straight from the rows of the block's projection output and make them positive
// itself, softplus(raw + bias), the block prologue's map ("Mamba-2: Attention's Distant
// Cousin", section "The Mamba-2 Block": the step size comes out of the input projection
// with x, B and C).  The block then never writes or reads a dt tensor.
//
// Packed variable-length rows (cu != null, batch 1): a step where a sequence s >= 1 begins
// (cu[s]) adds -kSeqGap to the running sum.  Every decay exp(cs_j - cs_i) between two steps of
// different sequences then carries a factor exp(-kSeqGap) or smaller, which is 0 in fp32,
// while inside one sequence the offsets cancel.  The later stages thereby drop every
// cross-sequence term with no change of their own: pair terms inside a chunk, a chunk
// state's steps before the last sequence start, the carry across a chunk with a start in
// it, and the entry state's read-out after a start.
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kHB = 16;  // heads per workgroup, one wave each
constexpr int kThreads = kHB * 64;
// log-decay gap at a packed sequence start: exp2(-kSeqGap log2 e) is below the smallest
// fp32 subnormal, so every decay across a start is exactly zero
constexpr float kSeqGap = 120.f;

// Where the step sizes come from: dt [B][T][H] fp32 as given, or raw rows of the block's
// projection output (in bf16 or fp32), made positive here by softplus(raw + bias) -- the
// block's step-size map fused into this pass, so that the block never writes dt.
enum class DtSource { kF32, kRawBf16, kRawF32 };

template <DtSource SRC>
__device__ __forceinline__ float step_size(const float* dt, const void* raw, long long stride,
                                           const float* bias, int b, int T, int H, int t,
                                           int h) {
    if constexpr (SRC == DtSource::kF32) {
        return dt[((size_t)b * T + t) * H + h];
    } else {
        const long long at = ((long long)b * T + t) * stride + h;
        const float v = SRC == DtSource::kRawBf16
                            ? to_f32(reinterpret_cast<const __bf16*>(raw)[at])
                            : reinterpret_cast<const float*>(raw)[at];
        return softplus_step(bias ? v + bias[h] : v);
    }
}

// v moved by a DPP control CTRL (row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 =
// 0x143) in the rows of ROWS (a 4-bit row mask); 0 in lanes without a source and in the
// rows left out
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or_zero(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false));
}

template <int Q, DtSource SRC>
__global__ __launch_bounds__(kThreads) void chunk_cumsum_kernel(
    const float* __restrict__ dt, const void* __restrict__ raw, long long raw_stride,
    const float* __restrict__ bias, const float* __restrict__ A, const int* __restrict__ cu,
    int nseq, float* __restrict__ dtc, float* __restrict__ cs, int T, int H, int nC) {
    constexpr int E = Q / 64;       // steps per lane
    constexpr int LD = Q + 4;       // padded row: 16-byte aligned, conflict-free writes
    __shared__ __align__(16) float tile[kHB][LD];
    __shared__ float gap[Q];  // -kSeqGap where a packed sequence starts, else 0
    const int hblocks = (H + kHB - 1) / kHB;
    const int hb = blockIdx.x % hblocks;
    const int bc = blockIdx.x / hblocks;
    const int c = bc % nC;
    const int b = bc / nC;
    const int h0 = hb * kHB;
    const int nh = min(kHB, H - h0);
    const int t0 = c * Q;
    const int Lc = min(Q, T - t0);
    const int tid = threadIdx.x;
    // element e = tid + kThreads k of the Q x 16 tile
    constexpr int L = Q * kHB / kThreads;
    float v_in[L];
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const int e = tid + kThreads * k;
        const int t = e / kHB, hh = e % kHB;
        v_in[k] = (t < Lc && hh < nh)
                      ? step_size<SRC>(dt, raw, raw_stride, bias, b, T, H, t0 + t, h0 + hh)
                      : 0.0f;
    }
#pragma unroll
    for (int k = 0; k < L; ++k) {
        const int e = tid + kThreads * k;
        tile[e % kHB][e / kHB] = v_in[k];
    }
    if (tid < Q) gap[tid] = 0.f;
    __syncthreads();
    if (cu && tid == 0) {  // the sequence starts inside this chunk (batch 1)
        int lo = 1, hi = nseq;  // first s >= 1 with cu[s] >= t0 (cu is non-decreasing)
        while (lo < hi) {
            const int mid = (lo + hi) / 2;
            if (cu[mid] < t0) lo = mid + 1;
            else hi = mid;
        }
        for (int q = lo; q < nseq && cu[q] < t0 + Lc; ++q) gap[cu[q] - t0] = -kSeqGap;
    }
    __syncthreads();
    const int hh = tid >> 6, lane = tid & 63;
    if (hh >= nh) return;
    const int h = h0 + hh;
    const float a = A[h];
    float v[E], run[E];
#pragma unroll
    for (int k = 0; k < E; ++k) v[k] = tile[hh][lane * E + k];
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < E; ++k) {
        acc += fmaf(v[k], a, gap[lane * E + k]);
        run[k] = acc;
    }
    // exclusive carry from the lanes before this one: an inclusive scan of the lane totals
    // by DPP (VALU, no LDS round trips): shifts by 1, 2, 4, 8 inside each 16-lane row, then
    // row 0's total into row 1 and row 2's into row 3 (row_bcast:15), then the first two
    // rows' total into rows 2 and 3 (row_bcast:31)
    float incl = acc;
    incl += dpp_or_zero<0x111, 0xF>(incl);
    incl += dpp_or_zero<0x112, 0xF>(incl);
    incl += dpp_or_zero<0x114, 0xF>(incl);
    incl += dpp_or_zero<0x118, 0xF>(incl);
    incl += dpp_or_zero<0x142, 0xA>(incl);
    incl += dpp_or_zero<0x143, 0xC>(incl);
    const float carry = incl - acc;
#pragma unroll
    for (int k = 0; k < E; ++k) run[k] += carry;
    // rows of Q floats: the lane's E steps are contiguous and 4 E-byte aligned
    const size_t o = (((size_t)b * H + h) * nC + c) * Q + lane * E;
    if constexpr (E == 4) {
        *reinterpret_cast<float4*>(dtc + o) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(cs + o) = make_float4(run[0], run[1], run[2], run[3]);
    } else if constexpr (E == 2) {
        *reinterpret_cast<float2*>(dtc + o) = make_float2(v[0], v[1]);
        *reinterpret_cast<float2*>(cs + o) = make_float2(run[0], run[1]);
    } else {
#pragma unroll
        for (int k = 0; k < E; ++k) {
            dtc[o + k] = v[k];
            cs[o + k] = run[k];
        }
    }
}


template <int Q, DtSource SRC>
void launch_q(unsigned blocks, const Shape& s, const float* dt, const DtRaw* raw, const float* A,
              const int* cu, int nseq, float* dtc, float* cs, hipStream_t st) {
    chunk_cumsum_kernel<Q, SRC><<<blocks, kThreads, 0, st>>>(
        dt, raw ? raw->p : nullptr, raw ? raw->stride : 0, raw ? raw->bias : nullptr, A, cu,
        nseq, dtc, cs, s.T, s.H, s.nC);
}

template <DtSource SRC>
hipError_t launch_src(unsigned blocks, const Shape& s, const float* dt, const DtRaw* raw,
                      const float* A, const int* cu, int nseq, float* dtc, float* cs,
                      hipStream_t st) {
    switch (s.Q) {
        case 64: launch_q<64, SRC>(blocks, s, dt, raw, A, cu, nseq, dtc, cs, st); break;
        case 128: launch_q<128, SRC>(blocks, s, dt, raw, A, cu, nseq, dtc, cs, st); break;
        case 256: launch_q<256, SRC>(blocks, s, dt, raw, A, cu, nseq, dtc, cs, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_chunk_cumsum(const Shape& s, const float* dt, const float* A, float* dtc,
                               float* cs, hipStream_t st, const int* cu, int nseq,
                               const DtRaw* raw) {
    const size_t hblocks = (size_t)(s.H + kHB - 1) / kHB;
    const unsigned blocks = (unsigned)((size_t)s.B * s.nC * hblocks);
    if (blocks == 0) return hipSuccess;
    if (!raw) return launch_src<DtSource::kF32>(blocks, s, dt, raw, A, cu, nseq, dtc, cs, st);
    if (raw->dtype == SSD_BF16)
        return launch_src<DtSource::kRawBf16>(blocks, s, dt, raw, A, cu, nseq, dtc, cs, st);
    return launch_src<DtSource::kRawF32>(blocks, s, dt, raw, A, cu, nseq, dtc, cs, st);
}

}  // namespace ssd
