// chunk_mfma.hip -- stage 2 (chunk_state) on gfx950 bf16 MFMA.
//
// Summary of arXiv 2405.21060, section "The Block-Decomposition SSD Algorithm", stage 2
// (the linear-attention contraction order of equation 15):
//     S[n][p] = sum_i B[i][n] x'[i][p],   x'[i][p] = exp(cs_last - cs_i) dt_i x[i][p]
// with fp32 accumulation.  v_mfma_f32_16x16x32_bf16 contracts over time, which runs along
// the slow (row) dimension of B and x in HBM, so both operands pass through LDS.
//
// Two kernels:
//   chunk_state_pipe_kernel (N = 128 or 256, P <= 64; N = 64, P in {32, 64}): persistent
//     and pipelined.  A workgroup per CU walks a run of (unit, head) items, a unit being
//     one (batch, group, chunk).  The unit's B chunk is copied into LDS once and read out
//     through transpose reads into register fragments (one 16-row n-tile per wave, two at
//     N = 256, all 32-step blocks), after which the next unit's B is copied in behind it.
//     At N = 256 the B chunk (128 KB at Q = 256) passes in two column slices of 128, the
//     second copied when the unit begins, so that the LDS holds one slice and two items.  Each item's x, cs and dt are copied into
//     a double-buffered LDS while the previous item computes.  The per-step weight
//     exp(cs_last - cs_i) dt_i is applied to the B fragments (rounded to bf16 once per
//     item), and x^T comes out of LDS through transpose reads.
//     At Q = 256 the workgroup that meets a unit's first head also writes the unit's
//     C B^T blocks for the chunk scan (what chunk_gram does): the B chunk is already in
//     LDS, so only C rows are read (wave w: row tiles w and 15 - w, the blocks below them).
//   chunk_state_mfma_kernel (other shapes): one workgroup per (b, h, chunk); 32-step slices
//     of B and x are transposed through registers into LDS ([feature][time], two time
//     steps per 32-bit word) and double-buffered; x' is formed in fp32 and rounded once.
//
// With REV set, the same kernels compute the backward pass's mirror of stage 2: the
// gradient of the entry state of every chunk through the chunk's own outputs,
//     Z[n][p] = sum_i C[i][n] exp(cs_i) dy[i][p]
// (y_i reads the entry state through exp(cs_i) C_i, so dL/dE = sum_i exp(cs_i) C_i dy_i^T):
// C takes the place of B, dy that of x, and the per-step weight is exp(cs_i).
#include "mfma_common.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

using namespace mfma;

constexpr int LDT = KB + 8;  // row stride (bf16) of the transposed [feature][time] slices

// element k (0..7) of a 16-byte vector of bf16, as raw 16 bits in the low half
__device__ __forceinline__ uint32_t bits_of(const uint4& v, int k) {
    const uint32_t w = k < 2 ? v.x : k < 4 ? v.y : k < 6 ? v.z : v.w;
    return (k & 1) ? (w >> 16) : (w & 0xffffu);
}

// ============================================================================ pipelined
template <int Q, int N, int P>
struct StateCfg {
    static constexpr int NW = N < 128 ? N / 16 : 8;  // waves
    static constexpr int NTW = N / 16 / NW;           // 16-row n-tiles per wave
    static constexpr int NTH = NW * 64;
    static constexpr int NB = Q / KB;
    static constexpr int PT = P / 16, PPR = P / 8;
    // B passes through LDS in column slices of at most 128 (one slice per n-tile of a wave)
    static constexpr int BW = N < 128 ? N : 128, NS = N / BW, BPR = BW / 8;
    static constexpr unsigned XB = Q * P * 2, BB = Q * BW * 2, FB = Q * 4;
    static constexpr unsigned ITEM = XB + 2 * FB;  // x, cs, dt
    static constexpr unsigned LDS = BB + 2 * ITEM + FB;
    // 16-byte state stores (PT / 2 per n-tile) in the forward; in the reverse-weight variant
    // (the backward's state gradients) they measured slower (55.0 -> 59.1 us at 2.7B, the
    // forward's 53.1 -> 51.4 us), so it keeps PT 8-byte stores per n-tile
    static constexpr bool PAIRED(bool rev) { return PT % 2 == 0 && !rev; }
    static constexpr int STORES(bool rev) { return (PAIRED(rev) ? PT / 2 : PT) * NTW; }
    static_assert(NS == NTW, "one B slice per n-tile of a wave");
};

template <int Q, int N, int P>
__device__ __forceinline__ void state_issue_x(const __bf16* x, const float* cs, const float* dtc,
                                              int slot, int hpg, int T, int H, int G, int nC,
                                              uint32_t lds, int wave, int lane) {
    using C_ = StateCfg<Q, N, P>;
    const int unit = slot / hpg;
    const int c = unit % nC, g = (unit / nC) % G, b = unit / nC / G;
    const int h = g * hpg + slot % hpg;
    const int Lc = min(Q, T - c * Q);
    const unsigned rowb = (unsigned)(H * P * 2);
    const u32x4 xr = raw_rsrc(x + ((size_t)(b * T + c * Q) * H + h) * P, (unsigned)Lc * rowb);
    constexpr int XI = Q * C_::PPR / 64;
#pragma unroll
    for (int k = wave; k < XI; k += C_::NW) {
        const int m = k * 64 + lane;
        const int r = m / C_::PPR, sl = m % C_::PPR;
        dma16(xr, lds + k * 1024, (unsigned)r * rowb + (unsigned)(sl ^ (r & (C_::PPR - 1))) * 16u);
    }
    const size_t sb = ((size_t)(b * H + h) * nC + c) * Q;
    if (wave == 0 && lane < Q / 4) dma16(raw_rsrc(cs + sb, C_::FB), lds + C_::XB, lane * 16u);
    if (wave == 1 && lane < Q / 4) dma16(raw_rsrc(dtc + sb, C_::FB), lds + C_::XB + C_::FB, lane * 16u);
}

// columns [BW sl, BW sl + BW) of the unit's B chunk into the B region ([time][BW], swizzled)
template <int Q, int N, int P>
__device__ __forceinline__ void state_issue_b(const __bf16* Bm, int unit, int slice, int T, int G,
                                              int nC, uint32_t lds, int wave, int lane) {
    using C_ = StateCfg<Q, N, P>;
    const int c = unit % nC, g = (unit / nC) % G, b = unit / nC / G;
    const int Lc = min(Q, T - c * Q);
    const unsigned rowb = (unsigned)(G * N * 2);
    const u32x4 br = raw_rsrc(Bm + ((size_t)(b * T + c * Q) * G + g) * N, (unsigned)Lc * rowb);
    const unsigned col0 = (unsigned)slice * C_::BW * 2u;
    constexpr int BI = Q * C_::BPR / 64;
#pragma unroll
    for (int k = wave; k < BI; k += C_::NW) {
        const int m = k * 64 + lane;
        const int r = m / C_::BPR, sl = m % C_::BPR;
        dma16(br, lds + k * 1024,
              (unsigned)r * rowb + col0 + (unsigned)(sl ^ (r & (C_::BPR - 1))) * 16u);
    }
}

// pair index of (16-row tile t, 32-step block ib <= t/2) in tile-major order (the chunk
// scan's layout of the C B^T blocks)
__device__ __forceinline__ int gram_pair_base(int t) {
    return (t & 1) ? (t / 2 + 1) * (t / 2 + 1) : (t / 2) * (t / 2 + 1);
}

template <int Q, int N, int P, bool REV>
__global__ __launch_bounds__((StateCfg<Q, N, P>::NTH)) void chunk_state_pipe_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Bm, const float* __restrict__ dtc,
    const float* __restrict__ cs, __bf16* __restrict__ states, const __bf16* __restrict__ Cm,
    uint4* __restrict__ gram, int T, int H, int G, int nC, int nslots) {
    using C_ = StateCfg<Q, N, P>;
    constexpr int NB = C_::NB, PT = C_::PT, PPR = C_::PPR, BPR = C_::BPR, NTW = C_::NTW;
    extern __shared__ __align__(16) unsigned char smem[];
    const uint32_t lds0 = lds_addr(smem);
    unsigned char* const sB = smem;                    // a B slice of the unit, [time][BW]
    unsigned char* const sX = smem + C_::BB;           // two item buffers: x, cs, dt
    float* const s_w = reinterpret_cast<float*>(smem + C_::BB + 2 * C_::ITEM);

    // a contiguous run of items per workgroup, neighbouring runs on the same XCD
    const int nwg = gridDim.x;
    const int wp = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int per = (nslots + nwg - 1) / nwg;
    const int lo = wp * per, hi = min(nslots, lo + per);
    if (lo >= hi) return;

    const int hpg = H / G;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;

    // transpose-read offsets (rows 4 g4 + l16 / 4 of a 32-step block, column 4 (l16 % 4)
    // within a 16-wide tile); the swizzle depends only on the row mod pieces-per-row.  The
    // wave's n-tile k is wave + NW k, at the same columns of B slice k.
    const unsigned boff = swz_off(4 * g4 + (l16 >> 2), wave * 16 + 4 * (l16 & 3), BPR);
    unsigned xoff[PT];
#pragma unroll
    for (int p = 0; p < PT; ++p) xoff[p] = swz_off(4 * g4 + (l16 >> 2), p * 16 + 4 * (l16 & 3), PPR);
    constexpr unsigned BBLK = KB * BPR * 16, BHALF = 16 * BPR * 16;
    constexpr unsigned XBLK = KB * PPR * 16, XHALF = 16 * PPR * 16;

    bf16x8 bt[NTW][NB];  // B^T fragments of this wave's n-tiles, every 32-step block
    int cur_unit = -1;

    state_issue_b<Q, N, P>(Bm, lo / hpg, 0, T, G, nC, lds0, wave, lane);
    state_issue_x<Q, N, P>(x, cs, dtc, lo, hpg, T, H, G, nC, lds0 + C_::BB, wave, lane);
#pragma unroll 1
    for (int sl = lo; sl < hi; ++sl) {
        const int n = sl - lo;
        const int buf = n & 1;
        const unsigned char* bx = sX + buf * C_::ITEM;
        const float* b_cs = reinterpret_cast<const float*>(bx + C_::XB);
        const float* b_dt = b_cs + Q;
        // this item's copies have landed once only the previous item's stores are pending
        if (n == 0)
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(C_::STORES(REV)) : "memory");
        const int unit = sl / hpg;
        if (unit != cur_unit) {  // the B region holds slice 0 of this unit
            cur_unit = unit;
#pragma unroll
            for (int k = 0; k < NTW; ++k) {
                if (k > 0) {  // slice k: copy it in now and wait for it
                    lds_barrier();  // every wave has read slice k - 1
                    state_issue_b<Q, N, P>(Bm, unit, k, T, G, nC, lds0, wave, lane);
                    dma_barrier();
                }
#pragma unroll
                for (int ib = 0; ib < NB; ++ib) {
                    const unsigned char* bp = sB + boff + ib * BBLK;
                    const uint2 lo2 = lds_read_tr16(bp);
                    const uint2 hi2 = lds_read_tr16(bp + BHALF);
                    bt[k][ib] = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
                }
            }
            constexpr bool kGram = (Q == 256 && (N == 64 || N == 128) && !REV);
            if (kGram && gram != nullptr && sl == unit * hpg) {
                // C B^T blocks of this unit (this workgroup holds its first head): wave w
                // takes the row tile pairs (tp, 15 - tp), tp = w, w + NW, ..., and every
                // block at or below them
                const int c = unit % nC, g = (unit / nC) % G, b = unit / nC / G;
                const int Lc = min(Q, T - c * Q);
                const unsigned crow = (unsigned)(G * N * 2);
                const __amdgpu_buffer_rsrc_t cr =
                    make_rsrc(Cm + ((size_t)(b * T + c * Q) * G + g) * N, (unsigned)Lc * crow);
                constexpr int NK = N / 32, NPAIR = 72;
#pragma unroll 1
                for (int tp = wave; tp < 8; tp += C_::NW) {
                const int ta = tp, tb = 15 - tp;
                const int na = ta / 2 + 1, nb = tb / 2 + 1;
                bf16x8 ca[NK], cb[NK];
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    const unsigned col = (32 * kk + 8 * g4) * 2u;
                    ca[kk] = __builtin_bit_cast(bf16x8, buf_load16(cr, (unsigned)(ta * 16 + l16) * crow + col));
                    cb[kk] = __builtin_bit_cast(bf16x8, buf_load16(cr, (unsigned)(tb * 16 + l16) * crow + col));
                }
                uint4* gu = gram + (size_t)unit * NPAIR * 64 + lane;
#pragma unroll 1
                for (int ib = 0; ib < nb; ++ib) {
                    bf16x8 r0[NK], r1[NK];  // B rows 32 ib + l16 and + 16, n-slice kk
#pragma unroll
                    for (int kk = 0; kk < NK; ++kk) {
                        r0[kk] = *reinterpret_cast<const bf16x8*>(
                            sB + swz_off(ib * KB + l16, 32 * kk + 8 * g4, BPR));
                        r1[kk] = *reinterpret_cast<const bf16x8*>(
                            sB + swz_off(ib * KB + 16 + l16, 32 * kk + 8 * g4, BPR));
                    }
                    auto emit = [&](const bf16x8* cc, int t) {
                        f32x4 g0 = f32x4{0.f, 0.f, 0.f, 0.f}, g1 = g0;
#pragma unroll
                        for (int kk = 0; kk < NK; ++kk) {
                            g0 = mfma16(r0[kk], cc[kk], g0);
                            g1 = mfma16(r1[kk], cc[kk], g1);
                        }
                        gu[(size_t)(gram_pair_base(t) + ib) * 64] =
                            make_uint4(pack_bf16(g0[0], g0[1]), pack_bf16(g0[2], g0[3]),
                                       pack_bf16(g1[0], g1[1]), pack_bf16(g1[2], g1[3]));
                    };
                    if (ib < na) emit(ca, ta);
                    emit(cb, tb);
                }
                }
            }
            lds_barrier();  // every wave holds its fragments: the region is free
            const int nxt = (unit + 1) * hpg;
            if (nxt < hi) state_issue_b<Q, N, P>(Bm, unit + 1, 0, T, G, nC, lds0, wave, lane);
        }
        if (tid < Q) {
            const float ci = b_cs[tid];
            s_w[tid] = REV ? exp2_fast(ci * kLog2e)
                           : exp2_fast((b_cs[Q - 1] - ci) * kLog2e) * b_dt[tid];
        }
        lds_barrier();
        if (sl + 1 < hi)
            state_issue_x<Q, N, P>(x, cs, dtc, sl + 1, hpg, T, H, G, nC,
                                   lds0 + C_::BB + (buf ^ 1) * C_::ITEM, wave, lane);

        f32x4 acc[NTW][PT];
#pragma unroll
        for (int k = 0; k < NTW; ++k)
#pragma unroll
            for (int p = 0; p < PT; ++p) acc[k][p] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) {
            // B^T fragments weighted by exp(cs_last - cs_i) dt_i over their k-slots
            const int i0 = ib * KB + 4 * g4;
            const float4 wa = *reinterpret_cast<const float4*>(&s_w[i0]);
            const float4 wb = *reinterpret_cast<const float4*>(&s_w[i0 + 16]);
            bf16x8 a[NTW];
#pragma unroll
            for (int k = 0; k < NTW; ++k) {
                const uint4 r = __builtin_bit_cast(uint4, bt[k][ib]);
                a[k] = __builtin_bit_cast(
                    bf16x8, make_uint4(pack_bf16(bf16_lo(r.x) * wa.x, bf16_hi(r.x) * wa.y),
                                       pack_bf16(bf16_lo(r.y) * wa.z, bf16_hi(r.y) * wa.w),
                                       pack_bf16(bf16_lo(r.z) * wb.x, bf16_hi(r.z) * wb.y),
                                       pack_bf16(bf16_lo(r.w) * wb.z, bf16_hi(r.w) * wb.w)));
            }
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                const unsigned char* xp = bx + xoff[p] + ib * XBLK;
                const uint2 lo2 = lds_read_tr16(xp);
                const uint2 hi2 = lds_read_tr16(xp + XHALF);
                const bf16x8 xf = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
#pragma unroll
                for (int k = 0; k < NTW; ++k) acc[k][p] = mfma16(a[k], xf, acc[k][p]);
            }
        }
        // lane holds S[n = (wave + NW k)*16 + 4*g4 + r][p = pt*16 + l16]; layout [p][n]
        const int c = unit % nC, g = (unit / nC) % G, b = unit / nC / G;
        const int h = g * hpg + sl % hpg;
        __bf16* out = states + ((size_t)(b * H + h) * nC + c) * P * N;
#pragma unroll
        for (int k = 0; k < NTW; ++k) {
            uint2 o[PT];
#pragma unroll
            for (int p = 0; p < PT; ++p)
                o[p] = make_uint2(pack_bf16(acc[k][p][0], acc[k][p][1]),
                                  pack_bf16(acc[k][p][2], acc[k][p][3]));
            if constexpr (C_::PAIRED(REV)) {
                // 16-byte stores (pair_runs over p-tiles 2q, 2q + 1): rows 16 (2q + g4 % 2)
                // + l16, n-tile elements 8 (g4 / 2) .. +7
#pragma unroll
                for (int q = 0; q < PT / 2; ++q)
                    *reinterpret_cast<uint4*>(out + (size_t)((2 * q + (g4 & 1)) * 16 + l16) * N +
                                              (wave + C_::NW * k) * 16 + 8 * (g4 >> 1)) =
                        pair_runs(o[2 * q], o[2 * q + 1]);
            } else {
#pragma unroll
                for (int p = 0; p < PT; ++p)
                    *reinterpret_cast<uint2*>(out + (size_t)(p * 16 + l16) * N +
                                              (wave + C_::NW * k) * 16 + 4 * g4) = o[p];
            }
        }
    }
}

// ============================================================================ chunk_state

// FIN: packed variable-length rows (batch 1); a workgroup per (sequence, head) takes the
// state after the sequence's last step te, in chunk c = te / Q at offset off:
//     exp(cs_off) E_c + sum_{i <= off} exp(cs_off - cs_i) dt_i B_i x_i^T
// (E_c the chunk's entry state, [P][N] in bf16), written as fp32 [N][P] to `finals`; an
// empty sequence gets zeros.  The log-decay gaps at sequence starts (chunk_cumsum.hip) drop
// the entry state and the steps of earlier sequences by themselves.
template <int Q, int N, int P, bool REV, bool FIN = false>
__global__ __launch_bounds__(256) void chunk_state_mfma_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Bm, const float* __restrict__ dtc,
    const float* __restrict__ cs, __bf16* __restrict__ states, int T, int H, int G, int nC,
    const int* __restrict__ cu = nullptr, const __bf16* __restrict__ entry = nullptr,
    float* __restrict__ finals = nullptr) {
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

    int c, bh, te = 0, sq = 0;
    if constexpr (FIN) {
        sq = blockIdx.x / H;
        bh = blockIdx.x % H;  // batch 1
        te = cu[sq + 1] - 1;  // the sequence's last step (beg > te: empty)
        c = te >= 0 ? te / Q : 0;
    } else {
        c = blockIdx.x % nC;
        bh = blockIdx.x / nC;
    }
    const int h = bh % H;
    const int b = bh / H;
    const int g = h / (H / G);
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const size_t cbase = ((size_t)bh * nC + c) * Q;
    const int t0 = c * Q;
    // FIN: steps t0 .. te (empty: none); else the whole chunk
    const bool empty = FIN && cu[sq + 1] <= cu[sq];
    const int off = FIN ? (empty ? -1 : te - t0) : Q - 1;
    const int tlim = FIN ? t0 + off : T - 1;  // last step read

    // decay to the last step times dt, per step (fp32)
    const float cs_last = off >= 0 ? cs[cbase + off] : 0.f;
    for (int i = tid; i < Q; i += NTH)
        s_w[i] = i > off ? 0.f
                 : REV   ? expf(cs[cbase + i])
                         : expf(cs_last - cs[cbase + i]) * dtc[cbase + i];

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
                if (t <= tlim) rb[q][0] = *reinterpret_cast<const uint4*>(src);
                if (t + 1 <= tlim) rb[q][1] = *reinterpret_cast<const uint4*>(src + (size_t)G * N);
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
                if (t <= tlim) rx[q][0] = *reinterpret_cast<const uint4*>(src);
                if (t + 1 <= tlim) rx[q][1] = *reinterpret_cast<const uint4*>(src + (size_t)H * P);
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
    if constexpr (FIN) {  // the entry state decayed to the last step
        if (!empty) {
            const float de = expf(cs_last);
            const __bf16* E = entry + ((size_t)bh * nC + c) * P * N;
#pragma unroll
            for (int a = 0; a < NTW; ++a)
#pragma unroll
                for (int p = 0; p < PT; ++p) {
                    const int n0 = (wave * NTW + a) * 16 + 4 * g4;
                    const uint2 e2 =
                        *reinterpret_cast<const uint2*>(E + (size_t)(p * 16 + l16) * N + n0);
                    acc[a][p] = f32x4{de * bf16_lo(e2.x), de * bf16_hi(e2.x),
                                      de * bf16_lo(e2.y), de * bf16_hi(e2.y)};
                }
        }
    }
    // 32-step blocks that hold a step to take
    const int nbk = FIN ? (off + KB) / KB : NB;

    load(0);
    lds_barrier();  // s_w ready
    store(0, 0);
    lds_barrier();
    for (int ib = 0; ib < nbk; ++ib) {
        const int buf = ib & 1;
        if (ib + 1 < nbk) load(ib + 1);
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
        if (ib + 1 < nbk) store(buf ^ 1, ib + 1);
        lds_barrier();
    }
    if constexpr (FIN) {  // fp32 [N][P] per (sequence, head)
        float* out = finals + ((size_t)sq * H + h) * N * P;
#pragma unroll
        for (int a = 0; a < NTW; ++a)
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                const int n0 = (wave * NTW + a) * 16 + 4 * g4;
                const int pp = p * 16 + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) out[(size_t)(n0 + r) * P + pp] = acc[a][p][r];
            }
        return;
    }
    // lane holds S[n = tile*16 + 4*g4 + r][p = pt*16 + l16]; layout [p][n]
    __bf16* out = states + ((size_t)bh * nC + c) * P * N;
#pragma unroll
    for (int a = 0; a < NTW; ++a)
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            const int n0 = (wave * NTW + a) * 16 + 4 * g4;
            const int pp = p * 16 + l16;
            *reinterpret_cast<uint2*>(out + (size_t)pp * N + n0) =
                make_uint2(pack_bf16(acc[a][p][0], acc[a][p][1]), pack_bf16(acc[a][p][2], acc[a][p][3]));
        }
}

// ---------------------------------------------------------------- dispatch tables

template <int Q, int N, int P>
hipError_t launch_final_t(const Shape& s, const void* x, const void* Bm, const float* dtc,
                          const float* cs, const void* entry, const int* cu, int nseq,
                          float* finals, hipStream_t st) {
    chunk_state_mfma_kernel<Q, N, P, false, true><<<(unsigned)((size_t)nseq * s.H), 256, 0, st>>>(
        (const __bf16*)x, (const __bf16*)Bm, dtc, cs, nullptr, s.T, s.H, s.G, s.nC, cu,
        (const __bf16*)entry, finals);
    return hipGetLastError();
}
using FinalFn = hipError_t (*)(const Shape&, const void*, const void*, const float*,
                               const float*, const void*, const int*, int, float*, hipStream_t);
template <int Q>
FinalFn pick_final_q(const Shape& s) {
    switch (s.N) {
#define SSD_FIN_N(NV)                                         \
    case NV:                                                  \
        switch (s.P) {                                        \
            case 16: return launch_final_t<Q, NV, 16>;        \
            case 32: return launch_final_t<Q, NV, 32>;        \
            case 64: return launch_final_t<Q, NV, 64>;        \
            case 128: return launch_final_t<Q, NV, 128>;      \
        }                                                     \
        break;
        SSD_FIN_N(64)
        SSD_FIN_N(128)
        SSD_FIN_N(256)
#undef SSD_FIN_N
    }
    return nullptr;
}
FinalFn pick_final(const Shape& s) {
    switch (s.Q) {
        case 64: return pick_final_q<64>(s);
        case 128: return pick_final_q<128>(s);
        case 256: return pick_final_q<256>(s);
    }
    return nullptr;
}

template <int Q, int N, int P, bool REV>
hipError_t launch_state_t(const Shape& s, const void* x, const void* Bm, const float* dtc,
                          const float* cs, void* states, const void*, void*, hipStream_t st) {
    const unsigned blocks = (unsigned)((size_t)s.B * s.H * s.nC);
    chunk_state_mfma_kernel<Q, N, P, REV><<<blocks, 256, 0, st>>>(
        (const __bf16*)x, (const __bf16*)Bm, dtc, cs, (__bf16*)states, s.T, s.H, s.G, s.nC);
    return hipGetLastError();
}

#define SSD_FOR_P(F, Q, N)                                   \
    switch (s.P) {                                           \
        case 16: return F<Q, N, 16, REV>;                    \
        case 32: return F<Q, N, 32, REV>;                    \
        case 64: return F<Q, N, 64, REV>;                    \
        case 128: return F<Q, N, 128, REV>;                  \
    }                                                        \
    break;

using StateFn = hipError_t (*)(const Shape&, const void*, const void*, const float*, const float*,
                               void*, const void*, void*, hipStream_t);

template <int Q, bool REV>
StateFn pick_state_q(const Shape& s) {
    switch (s.N) {
        case 64: SSD_FOR_P(launch_state_t, Q, 64)
        case 128: SSD_FOR_P(launch_state_t, Q, 128)
        case 256: SSD_FOR_P(launch_state_t, Q, 256)
    }
    return nullptr;
}

template <int Q, int N, int P, bool REV>
hipError_t launch_state_pipe_t(const Shape& s, const void* x, const void* Bm, const float* dtc,
                               const float* cs, void* states, const void* Cm, void* gram,
                               hipStream_t st) {
    using C_ = StateCfg<Q, N, P>;
    const auto kern = chunk_state_pipe_kernel<Q, N, P, REV>;
    static DeviceSlots grid_of;  // per device: resident workgroups, a multiple of 8
    int grid = 0;
    const hipError_t e = resident_grid((const void*)kern, C_::NTH, C_::LDS, grid_of, &grid);
    if (e != hipSuccess) return e;
    const int nslots = s.B * s.G * s.nC * (s.H / s.G);
    kern<<<grid, C_::NTH, C_::LDS, st>>>((const __bf16*)x, (const __bf16*)Bm, dtc, cs,
                                                  (__bf16*)states, (const __bf16*)Cm, (uint4*)gram, s.T,
                                                  s.H, s.G, s.nC, nslots);
    return hipGetLastError();
}

template <int Q, bool REV>
StateFn pick_state_pipe_q(const Shape& s) {
    if (s.N == 128) {
        switch (s.P) {
            case 16: return launch_state_pipe_t<Q, 128, 16, REV>;
            case 32: return launch_state_pipe_t<Q, 128, 32, REV>;
            case 64: return launch_state_pipe_t<Q, 128, 64, REV>;
        }
    } else if (s.N == 64) {  // four waves: P up to 64 keeps the copy counts per wave even
        switch (s.P) {
            case 32: return launch_state_pipe_t<Q, 64, 32, REV>;
            case 64: return launch_state_pipe_t<Q, 64, 64, REV>;
        }
    } else if (s.N == 256) {  // two n-tiles per wave, B copied in two column slices
        switch (s.P) {
            case 16: return launch_state_pipe_t<Q, 256, 16, REV>;
            case 32: return launch_state_pipe_t<Q, 256, 32, REV>;
            case 64: return launch_state_pipe_t<Q, 256, 64, REV>;
        }
    }
    return nullptr;
}

bool state_offsets_fit(const Shape& s) {
    // buffer resources address one chunk of x and B with 32-bit byte offsets
    return (size_t)s.Q * s.H * s.P * 2 < ((size_t)1 << 31) &&
           (size_t)s.Q * s.G * s.N * 2 < ((size_t)1 << 31);
}

template <bool REV>
StateFn pick_state(const Shape& s) {
    if (state_offsets_fit(s)) {
        StateFn f = nullptr;
        switch (s.Q) {
            case 64: f = pick_state_pipe_q<64, REV>(s); break;
            case 128: f = pick_state_pipe_q<128, REV>(s); break;
            case 256: f = pick_state_pipe_q<256, REV>(s); break;
        }
        if (f) return f;
    }
    switch (s.Q) {
        case 64: return pick_state_q<64, REV>(s);
        case 128: return pick_state_q<128, REV>(s);
        case 256: return pick_state_q<256, REV>(s);
    }
    return nullptr;
}

}  // namespace

bool chunk_state_mfma_supported(const Shape& s) { return pick_state<false>(s) != nullptr; }

bool varlen_final_mfma_supported(const Shape& s) { return pick_final(s) != nullptr; }

hipError_t launch_varlen_final_mfma(const Shape& s, const void* x, const void* Bm,
                                    const float* dtc, const float* cs, const void* entry,
                                    const int* cu, int nseq, float* finals, hipStream_t st) {
    const FinalFn f = pick_final(s);
    if (!f) return hipErrorInvalidValue;
    if (nseq <= 0 || s.H <= 0) return hipSuccess;
    return f(s, x, Bm, dtc, cs, entry, cu, nseq, finals, st);
}

bool chunk_state_writes_gram(const Shape& s) {
    return state_offsets_fit(s) && s.Q == 256 && (s.N == 64 || s.N == 128) &&
           pick_state_pipe_q<256, false>(s) != nullptr;
}

hipError_t launch_chunk_state_mfma(const Shape& s, const void* x, const void* Bm,
                                   const float* dtc, const float* cs, void* states,
                                   const void* Cm, void* gram, hipStream_t st) {
    StateFn f = pick_state<false>(s);
    if (!f) return hipErrorInvalidValue;
    if ((size_t)s.B * s.H * s.nC == 0) return hipSuccess;
    const bool fuse = gram != nullptr && Cm != nullptr && chunk_state_writes_gram(s);
    return f(s, x, Bm, dtc, cs, states, fuse ? Cm : nullptr, fuse ? gram : nullptr, st);
}

hipError_t launch_chunk_dstate_mfma(const Shape& s, const void* dy, const void* Cm,
                                    const float* cs, void* dstates, hipStream_t st) {
    StateFn f = pick_state<true>(s);
    if (!f) return hipErrorInvalidValue;
    if ((size_t)s.B * s.H * s.nC == 0) return hipSuccess;
    // the weights need only cs; the step sizes are not read (cs stands in for them)
    return f(s, dy, Cm, cs, cs, dstates, nullptr, nullptr, st);
}

}  // namespace ssd
