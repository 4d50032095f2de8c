// chunk_scan_mfma.hip -- stages 1, 4 and 5 of the block decomposition on gfx950 bf16 MFMA.
//
// Summary of arXiv 2405.21060, section "The Block-Decomposition SSD Algorithm": inside a
// chunk the output is the quadratic (attention-like) form of the dual, Y = (L o C B^T) X
// (section "The Scalar-Identity SSM", equation 16); the state carried into the chunk is
// read out by C and decayed (stage 4); the two add up (stage 5).  Per chunk row j and
// head h, with cs the chunk-local prefix sums of dt*A:
//     y[j] = sum_{i<=j} (C_j . B_i) exp(cs_j - cs_i) dt_i x[i] + exp(cs_j) C_j . E + D x[j]
//
// Two kernels:
//   chunk_gram   C B^T once per (batch, group, chunk): the heads of a group share B and C
//                (summary section "The Mamba-2 Architecture", head patterns), so the Gram
//                blocks are computed once and kept, rounded to bf16, in a small workspace
//                laid out as the per-lane MFMA fragments the scan consumes.
//   chunk_scan   persistent: a workgroup per CU walks a run of (batch, head, chunk) items
//                with a double-buffered LDS, copying the next item's x and entry state
//                from HBM while it computes the current one (details at the kernel).  The
//                MFMA operands that run over time come out of LDS through transpose reads;
//                the output is kept transposed, Y^T[p][j], so the Gram block for (row
//                tile, 32-step block), masked and decayed in registers, is directly the B
//                operand of X^T Gm^T.  The decay is masked before exponentiation (never a
//                positive exponent); blocks wholly below a tile factor it at the block end
//                e as exp(cs_j - cs_e) exp(cs_e - cs_i), both factors <= 1, so they need
//                one exp per lane instead of one per element.
#include <type_traits>

#include "mfma_common.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

using namespace mfma;

// pair index of (16-row tile t, 32-step block ib <= t/2) in tile-major order
__host__ __device__ constexpr int pair_base(int t) {
    return (t & 1) ? (t / 2 + 1) * (t / 2 + 1) : (t / 2) * (t / 2 + 1);
}
__host__ __device__ constexpr int npairs(int Q) { return pair_base(Q / 16); }


// ============================================================================ chunk_gram
// gram[unit][pair][lane] (16 bytes): for lane l of tile t, block ib, column j = 16t + l%16
// and g = l/16, the bf16 values C_j . B_i for i = 32ib + 4g + {0..3}, 32ib + 16 + 4g + {0..3}.
// One workgroup per unit.  B and C pass through LDS in column slices of up to 64
// (double-buffered: the next slice is copied while this one is used), and wave w sums the
// blocks of row tiles w and NT - 1 - w over the slices, so each unit's B and C are read from
// HBM once.  The sum over n runs in 32-column steps in order, as in the states kernel's own
// C B^T blocks.
template <int Q, int N>
struct GramCfg {
    static constexpr int NT = Q / 16, NW = NT / 2, NTH = NW * 64;
    static constexpr int BW = N < 64 ? N : 64;          // columns per slice
    static constexpr int NS = N / BW, SPR = BW / 8;     // slices; 16-byte pieces per row
    static constexpr int KS = BW / 32;                  // MFMA k-steps per slice
    static constexpr unsigned SB = Q * BW * 2;          // one slice of B (or of C)
    static constexpr unsigned LDS = 4 * SB;             // (B, C) x two buffers
    static constexpr int NI = Q * SPR / 64;             // copy instructions per slice matrix
    static_assert(N % 32 == 0 && NI * 64 == Q * SPR, "slice shape");
};

template <int Q, int N>
__global__ __launch_bounds__((GramCfg<Q, N>::NTH)) void chunk_gram_kernel(
    const __bf16* __restrict__ Bm, const __bf16* __restrict__ Cm, uint4* __restrict__ gram,
    int T, int G, int nC) {
    using C_ = GramCfg<Q, N>;
    constexpr int NT = C_::NT, KS = C_::KS, SPR = C_::SPR;
    extern __shared__ __align__(16) unsigned char smem[];
    const uint32_t lds0 = lds_addr(smem);
    const int unit = blockIdx.x;
    const int c = unit % nC, g = (unit / nC) % G, b = unit / nC / G;
    const int Lc = min(Q, T - c * Q);
    const unsigned rowb = (unsigned)(G * N * 2);
    const size_t base = ((size_t)(b * T + c * Q) * G + g) * N;
    const u32x4 br = raw_rsrc(Bm + base, (unsigned)Lc * rowb);
    const u32x4 cr = raw_rsrc(Cm + base, (unsigned)Lc * rowb);
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    // slice k of B and C into buffer k & 1 (B at 2 SB u, C after it), swizzled rows
    auto issue = [&](int k) {
        const uint32_t lb = lds0 + (unsigned)(k & 1) * 2u * C_::SB;
#pragma unroll
        for (int i = wave; i < C_::NI; i += C_::NW) {
            const int m = i * 64 + lane;
            const int r = m / SPR, sl = m % SPR;
            const unsigned off =
                (unsigned)r * rowb + (unsigned)(k * C_::BW) * 2u + (unsigned)(sl ^ (r & (SPR - 1))) * 16u;
            dma16(br, lb + (unsigned)i * 1024u, off);
            dma16(cr, lb + C_::SB + (unsigned)i * 1024u, off);
        }
    };
    const int ta = wave, tb = NT - 1 - wave;
    const int na = ta / 2 + 1, nb = tb / 2 + 1;
    f32x4 ga[NT / 4][2], gb[NT / 2][2];
#pragma unroll
    for (int i = 0; i < NT / 4; ++i) ga[i][0] = ga[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NT / 2; ++i) gb[i][0] = gb[i][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    issue(0);
#pragma unroll 1
    for (int k = 0; k < C_::NS; ++k) {
        // slice k has landed for every wave, and slice k - 1's buffer is no longer read
        dma_barrier();
        if (k + 1 < C_::NS) issue(k + 1);
        const unsigned char* sb = smem + (unsigned)(k & 1) * 2u * C_::SB;
        const unsigned char* sc = sb + C_::SB;
        bf16x8 ca[KS], cb[KS];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            ca[kk] = *reinterpret_cast<const bf16x8*>(sc + swz_off(ta * 16 + l16, 32 * kk + 8 * g4, SPR));
            cb[kk] = *reinterpret_cast<const bf16x8*>(sc + swz_off(tb * 16 + l16, 32 * kk + 8 * g4, SPR));
        }
#pragma unroll
        for (int ib = 0; ib < NT / 2; ++ib) {
            if (ib < nb) {
                bf16x8 r0[KS], r1[KS];  // B rows 32 ib + l16 and + 16
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    r0[kk] = *reinterpret_cast<const bf16x8*>(sb + swz_off(ib * KB + l16, 32 * kk + 8 * g4, SPR));
                    r1[kk] = *reinterpret_cast<const bf16x8*>(sb + swz_off(ib * KB + 16 + l16, 32 * kk + 8 * g4, SPR));
                }
                if (ib < NT / 4 && ib < na) {
#pragma unroll
                    for (int kk = 0; kk < KS; ++kk) {
                        ga[ib < NT / 4 ? ib : 0][0] = mfma16(r0[kk], ca[kk], ga[ib < NT / 4 ? ib : 0][0]);
                        ga[ib < NT / 4 ? ib : 0][1] = mfma16(r1[kk], ca[kk], ga[ib < NT / 4 ? ib : 0][1]);
                    }
                }
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    gb[ib][0] = mfma16(r0[kk], cb[kk], gb[ib][0]);
                    gb[ib][1] = mfma16(r1[kk], cb[kk], gb[ib][1]);
                }
            }
        }
    }
    uint4* gu = gram + (size_t)unit * npairs(Q) * 64 + lane;
    auto put = [&](const f32x4* gg, int t, int ib) {
        gu[(size_t)(pair_base(t) + ib) * 64] =
            make_uint4(pack_bf16(gg[0][0], gg[0][1]), pack_bf16(gg[0][2], gg[0][3]),
                       pack_bf16(gg[1][0], gg[1][1]), pack_bf16(gg[1][2], gg[1][3]));
    };
#pragma unroll
    for (int ib = 0; ib < NT / 4; ++ib)
        if (ib < na) put(ga[ib], ta, ib);
#pragma unroll
    for (int ib = 0; ib < NT / 2; ++ib)
        if (ib < nb) put(gb[ib], tb, ib);
}

// ============================================================================ chunk_scan
// Persistent and software-pipelined: each workgroup walks a contiguous run of (unit, head)
// items, consecutive heads of one unit first, from the run's end to its start (the chunk
// state kernel walks the same runs forwards, so the x rows it read last, the likeliest to
// still sit in the Infinity Cache, are read first).  Wave w of the NT/2 waves owns the 16-row
// tiles w and NT-1-w (the same share of the causal triangle for every wave).  While the
// unit stays the same, a wave keeps its tiles' C rows and Gram fragments in registers, so
// the compute needs no global loads at all; meanwhile the next item's x, entry state, cs
// and dt are copied from HBM into the other half of a double-buffered LDS.  The copies are
// issued through inline asm so that the compiler does not make later LDS reads wait for
// them; the one wait that is needed (the next item's copies, not the stores of the item
// just finished) is explicit: vector memory operations complete in issue order, so waiting
// until only this item's stores are outstanding means that everything before them landed.
template <int Q, int N, int P>
struct ScanCfg {
    static constexpr int NT = Q / 16;   // 16-row tiles per chunk
    static constexpr int NW = NT / 2;   // waves per workgroup
    static constexpr int NTH = NW * 64;
    static constexpr int NB = Q / KB;   // 32-step blocks per chunk
    static constexpr int NB0 = NT / 4;  // most blocks the first tile of a wave has
    static constexpr int PT = P / 16, NK = N / 32, PPR = P / 8, NPR = N / 8;
    static constexpr unsigned XB = Q * P * 2, EB = P * N * 2, FB = Q * 4;
    static constexpr unsigned ITEM = XB + EB + 2 * FB;  // x, entry state, cs, dt
    static constexpr unsigned TAIL = 3 * FB;  // cs*log2(e); weights to block and half-block ends
    // copy instructions per wave per item: PT for x (Q P / 512 over Q / 32 waves), the
    // entry state's share, and cs / dt on waves 0 / 1
    static constexpr int EI = P * NPR / 64;
    static constexpr bool EVEN = EI % NW == 0;
    static constexpr int DMA_LO = PT + EI / NW, DMA_HI = DMA_LO + 1;
    // three buffers (copies two items ahead) where they fit and the per-wave copy counts
    // are known, else two, else one
    static constexpr int NBUF = (EVEN && 3 * ITEM + TAIL <= 160u * 1024u) ? 3
                              : (2 * ITEM + TAIL <= 160u * 1024u)         ? 2
                                                                          : 1;
    static constexpr unsigned LDS = NBUF * ITEM + TAIL;
    // y stores per wave per item: two row tiles, each as PT / 2 16-byte stores per lane
    // (PT 8-byte stores where PT is odd)
    static constexpr int STORES = PT % 2 == 0 ? PT : 2 * PT;
};

template <int Q, int N, int P>
__device__ __forceinline__ void issue_item(const __bf16* x, const __bf16* E, const float* cs,
                                           const float* dtc, int slot, int hpg, int T, int H,
                                           int G, int nC, uint32_t lds, int wave, int lane) {
    using C_ = ScanCfg<Q, N, P>;
    const int unit = slot / hpg;
    const int c = unit % nC, g = (unit / nC) % G, b = unit / nC / G;
    const int h = g * hpg + slot % hpg;
    const int Lc = min(Q, T - c * Q);
    const unsigned rowb = (unsigned)(H * P * 2);
    const u32x4 xr = raw_rsrc(x + ((size_t)(b * T + c * Q) * H + h) * P, (unsigned)Lc * rowb);
    constexpr int XI = Q * C_::PPR / 64;
#pragma unroll
    for (int k = wave; k < XI; k += C_::NW) {
        const int m = k * 64 + lane;  // LDS piece
        const int r = m / C_::PPR, sl = m % C_::PPR;
        dma16(xr, lds + k * 1024, (unsigned)r * rowb + (unsigned)(sl ^ (r & (C_::PPR - 1))) * 16u);
    }
    const size_t sb = (size_t)(b * H + h) * nC + c;
    const u32x4 er = raw_rsrc(E + sb * P * N, C_::EB);
    constexpr int EI = P * C_::NPR / 64;
#pragma unroll
    for (int k = wave; k < EI; k += C_::NW) {
        const int m = k * 64 + lane;
        const int p = m / C_::NPR, sl = m % C_::NPR;
        dma16(er, lds + C_::XB + k * 1024,
              (unsigned)(p * N + (sl ^ (p & (C_::NPR - 1))) * 8) * 2u);
    }
    if (wave == 0 && lane < Q / 4)
        dma16(raw_rsrc(cs + sb * Q, C_::FB), lds + C_::XB + C_::EB, lane * 16u);
    if (wave == (C_::NW > 1 ? 1 : 0) && lane < Q / 4)
        dma16(raw_rsrc(dtc + sb * Q, C_::FB), lds + C_::XB + C_::EB + C_::FB, lane * 16u);
}

// With GATE set, the store applies the block's gate and normalisation (GateNorm) and
// writes the block output in place of y.
template <int Q, int N, int P, bool GATE = false>
__global__ __launch_bounds__((ScanCfg<Q, N, P>::NTH)) void chunk_scan_mfma_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Cm, const float* __restrict__ dtc,
    const float* __restrict__ cs, const float* __restrict__ D, const __bf16* __restrict__ E,
    const uint4* __restrict__ gram, __bf16* __restrict__ y, int T, int H, int G, int nC,
    int nslots, GateNorm gn) {
    using C_ = ScanCfg<Q, N, P>;
    constexpr int PT = C_::PT, NK = C_::NK, PPR = C_::PPR, NPR = C_::NPR, NB = C_::NB,
                  NB0 = C_::NB0;
    static_assert(N % 32 == 0 && P % 16 == 0 && Q % 64 == 0, "tile shape");
    extern __shared__ __align__(16) unsigned char smem[];
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
    float* s_c2 = reinterpret_cast<float*>(smem + C_::NBUF * C_::ITEM);
    float* s_v = s_c2 + Q;   // exp(cs_e - cs_i) dt_i, e = end of i's 32-step block
    float* s_vh = s_v + Q;   // the same with e = end of i's 16-step half block

    // this workgroup's items: a contiguous run, neighbouring runs on the same XCD (the GPU
    // deals consecutive workgroups round-robin to its 8 XCDs)
    const int nwg = gridDim.x;
    const int wp = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    const int per = (nslots + nwg - 1) / nwg;
    const int lo = wp * per, hi = min(nslots, lo + per);
    if (lo >= hi) return;  // whole workgroup

    const int hpg = H / G;
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int tile0 = wave, tile1 = C_::NT - 1 - wave;
    const int nblk0 = tile0 / 2 + 1, nblk1 = tile1 / 2 + 1;
    const int j0 = tile0 * 16 + l16, j1 = tile1 * 16 + l16;
    const unsigned rowb = (unsigned)(H * P * 2);
    const unsigned crow = (unsigned)(G * N * 2);

    constexpr unsigned XBLK = KB * PPR * 16;   // bytes of 32 rows of x
    constexpr unsigned XHALF = 16 * PPR * 16;  // bytes of 16 rows

    // C rows j0, j1 of the current unit: held across items where they fit (N <= 128), else
    // loaded for every item, at the end of the item before it
    constexpr bool CRES = N <= 128;
    bf16x8 cf0[NK], cf1[NK];
    auto load_c = [&](int slot) {
        const int u = slot / hpg;
        const int cc = u % nC, gg = (u / nC) % G, bb = u / nC / G;
        const __amdgpu_buffer_rsrc_t cr = make_rsrc(Cm + ((size_t)(bb * T + cc * Q) * G + gg) * N,
                                                    (unsigned)min(Q, T - cc * Q) * crow);
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const unsigned col = (32 * kk + 8 * g4) * 2u;
            cf0[kk] = __builtin_bit_cast(bf16x8, buf_load16(cr, (unsigned)j0 * crow + col));
            cf1[kk] = __builtin_bit_cast(bf16x8, buf_load16(cr, (unsigned)j1 * crow + col));
        }
    };
    // GATE: rows j0, j1 of the item's z (each lane's 4 channels of each p-tile), loaded at
    // the end of the item before, after its stores
    uint2 zq0[GATE ? PT : 1], zq1[GATE ? PT : 1];
    const unsigned zrowb = (unsigned)(gn.z_stride * 2);
    auto load_z = [&](int slot) {
        const int u = slot / hpg;
        const int cc = u % nC, gg = (u / nC) % G, bb = u / nC / G;
        const int hh = gg * hpg + slot % hpg;
        const int tt = cc * Q;
        const __amdgpu_buffer_rsrc_t zr = make_rsrc(
            reinterpret_cast<const __bf16*>(gn.z) + ((size_t)bb * T + tt) * gn.z_stride +
                (size_t)hh * P,
            (unsigned)min(Q, T - tt) * zrowb);
#pragma unroll
        for (int p = 0; p < PT; ++p) {
            const unsigned col = (unsigned)(p * 16 + 4 * g4) * 2u;
            zq0[p] = buf_load8(zr, (unsigned)j0 * zrowb + col);
            zq1[p] = buf_load8(zr, (unsigned)j1 * zrowb + col);
        }
    };
    uint4 gf0[NB0], gf1[NB];  // Gram fragments of (tile0, ib), (tile1, ib)
    int cur_unit = -1;

    issue_item<Q, N, P>(x, E, cs, dtc, hi - 1, hpg, T, H, G, nC, lds0, wave, lane);
    if (C_::NBUF == 3 && lo + 1 < hi)
        issue_item<Q, N, P>(x, E, cs, dtc, hi - 2, hpg, T, H, G, nC, lds0 + C_::ITEM, wave, lane);
    if constexpr (!CRES) load_c(hi - 1);
    if constexpr (GATE) load_z(hi - 1);
    int buf = 0;  // buffer of the current item
#pragma unroll 1
    for (int n = 0; n < hi - lo; ++n) {
        const int sl = hi - 1 - n;
        unsigned char* bx = smem + buf * C_::ITEM;
        const float* b_cs = reinterpret_cast<const float*>(bx + C_::XB + C_::EB);
        const float* b_dt = b_cs + Q;
        // This item's copies have landed once only what was issued after them is pending:
        // with three buffers the next item's copies and the previous item's stores, with
        // two the previous item's stores.
        // (Where the C rows are not held, this item's were issued last, after all of that.)
        constexpr int CX = CRES ? 0 : 2 * NK;
        if constexpr (GATE) {
            // the item's z rows were issued last: wait for everything, then mark them ready
            // here, so that no later wait (the compiler's, at their use) also covers the
            // copies issued during this item
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
#pragma unroll
            for (int p = 0; p < PT; ++p)
                asm volatile("" ::"v"(zq0[p].x), "v"(zq0[p].y), "v"(zq1[p].x), "v"(zq1[p].y));
        } else if (C_::NBUF == 3) {
            const bool more = n + 1 < hi - lo;
            if (n == 0 && !more)
                asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
            else if (n == 0 && wave < 2)
                asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(C_::DMA_HI + CX) : "memory");
            else if (n == 0)
                asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(C_::DMA_LO + CX) : "memory");
            else if (!more)
                asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(C_::STORES + CX) : "memory");
            else if (wave < 2)
                asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(C_::DMA_HI + C_::STORES + CX)
                             : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(C_::DMA_LO + C_::STORES + CX)
                             : "memory");
        } else if (n == 0 || C_::NBUF == 1) {
            asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(C_::STORES + CX) : "memory");
        }

        const int unit = sl / hpg;
        const int c = unit % nC, g = (unit / nC) % G, b = unit / nC / G;
        const int h = g * hpg + sl % hpg;
        const int t0 = c * Q;
        const int Lc = min(Q, T - t0);
        // block counts re-read each item (opaque copies): the compiler would otherwise
        // hoist every block's branch condition out of the loop into spilled SGPR masks
        // Lane-derived offsets and masks are recomputed every item from an opaque copy of
        // the lane id, and the block counts re-read: otherwise the compiler hoists them
        // (and every block's branch condition and diagonal mask) out of the loop, and the
        // registers they hold push the kernel into spills.
        int nb0 = nblk0, nb1 = nblk1, ln = lane;
        asm volatile("" : "+s"(nb0), "+s"(nb1), "+v"(ln));
        const int ql16 = ln & 15, qg4 = ln >> 4;
        // x^T operand of block ib: rows 32 ib + 4 g4 + l16 / 4 (and + 16), column
        // p * 16 + 4 (l16 % 4); the swizzle depends only on the row mod PPR, which a whole
        // block does not change
        unsigned xoff[PT];
#pragma unroll
        for (int p = 0; p < PT; ++p)
            xoff[p] = swz_off(4 * qg4 + (ql16 >> 2), p * 16 + 4 * (ql16 & 3), PPR);
        // Mask of the 16 x 16 block on the diagonal, as 4 bits: a tile's 16 rows j meet its
        // diagonal 32-step block in one 16-step half (the first for an even tile, the
        // second for an odd one); k-slot q of that half (step 4 g4 + q of it) is at or
        // below row j iff bit q is set.  The same bits serve both tiles of the wave.
        unsigned dq = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) dq |= (unsigned)(q <= ql16 - 4 * qg4) << q;
        if (tid < Q) {
            const float ci = b_cs[tid];
            s_c2[tid] = ci * kLog2e;
            s_v[tid] = exp2_fast((b_cs[tid | (KB - 1)] - ci) * kLog2e) * b_dt[tid];
            s_vh[tid] = exp2_fast((b_cs[tid | 15] - ci) * kLog2e) * b_dt[tid];
        }
        if (unit != cur_unit) {  // C rows and Gram fragments of the new unit
            cur_unit = unit;
            if constexpr (CRES) load_c(sl);
            // fragments past a tile's last block read outside the buffer: zeros
            const __amdgpu_buffer_rsrc_t gr = make_rsrc(
                gram + (size_t)unit * npairs(Q) * 64, (unsigned)(npairs(Q) * 64 * 16));
            const unsigned go0 = (unsigned)(pair_base(tile0) * 64 + lane) * 16u;
            const unsigned go1 = (unsigned)(pair_base(tile1) * 64 + lane) * 16u;
#pragma unroll
            for (int i = 0; i < NB0; ++i)
                gf0[i] = buf_load16(gr, i < nblk0 ? go0 + i * 1024u : 0x40000000u);
#pragma unroll
            for (int i = 0; i < NB; ++i)
                gf1[i] = buf_load16(gr, i < nblk1 ? go1 + i * 1024u : 0x40000000u);
            // wait here (vmcnt 0, as a compiler-visible wait) rather than at each first use,
            // where the wait would also cover the next item's copies issued below
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        if constexpr (!CRES) __builtin_amdgcn_s_waitcnt(0x0F70);  // C rows (issued earlier)
        lds_barrier();
        if (C_::NBUF == 3 && n + 2 < hi - lo) {  // into the buffer of the previous item
            const int b2 = buf == 0 ? 2 : buf - 1;
            issue_item<Q, N, P>(x, E, cs, dtc, sl - 2, hpg, T, H, G, nC, lds0 + b2 * C_::ITEM,
                                wave, lane);
        }
        if (C_::NBUF == 2 && n + 1 < hi - lo)
            issue_item<Q, N, P>(x, E, cs, dtc, sl - 1, hpg, T, H, G, nC,
                                lds0 + (buf ^ 1) * C_::ITEM, wave, lane);

        // stage 4: the entry state read out by C, then decayed from the chunk start
        f32x4 acc0[PT], acc1[PT];
#pragma unroll
        for (int p = 0; p < PT; ++p) acc0[p] = acc1[p] = f32x4{0.f, 0.f, 0.f, 0.f};
        const unsigned char* be = bx + C_::XB;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                const bf16x8 ea = *reinterpret_cast<const bf16x8*>(
                    be + swz_off(p * 16 + l16, 32 * kk + 8 * g4, NPR));
                acc0[p] = mfma16(ea, cf0[kk], acc0[p]);
                acc1[p] = mfma16(ea, cf1[kk], acc1[p]);
            }
        }
        const float csj0 = s_c2[j0], csj1 = s_c2[j1];
        {
            const float sc0 = exp2_fast(csj0), sc1 = exp2_fast(csj1);
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                acc0[p] *= sc0;
                acc1[p] *= sc1;
            }
        }

        // stage 1: masked quadratic form, one 32-step block at a time
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) {
            if (ib >= nb1) break;  // nb1 >= nb0
            bf16x8 xa[PT];
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                const unsigned char* xp = bx + xoff[p] + ib * XBLK;
                const uint2 lo2 = lds_read_tr16(xp);
                const uint2 hi2 = lds_read_tr16(xp + XHALF);
                xa[p] = __builtin_bit_cast(bf16x8, make_uint4(lo2.x, lo2.y, hi2.x, hi2.y));
            }
            const int i0 = ib * KB + 4 * g4;
            // masked, decayed Gram block of one tile -> MFMA operand
            // The tile's own block.  Its 16 x 16 quarter on the diagonal is masked through
            // the exponent (-inf above the diagonal, selected bit by bit by the
            // sign-extended mask bit); for an even tile the other half lies wholly above the
            // rows (zero), for an odd tile wholly below them (the decay factored at the end
            // of that half, like a block below).  ODD is the tile's parity (wave-uniform).
            auto diag = [&](auto odd_tag, const uint4 gv4, float csj, float* m) {
                constexpr bool ODD = decltype(odd_tag)::value;
                constexpr int hd = ODD ? 16 : 0;  // the diagonal half
                const float4 cd = *reinterpret_cast<const float4*>(&s_c2[i0 + hd]);
                const float4 dd = *reinterpret_cast<const float4*>(&b_dt[i0 + hd]);
                const float cdv[4] = {cd.x, cd.y, cd.z, cd.w};
                const float ddv[4] = {dd.x, dd.y, dd.z, dd.w};
                const uint32_t w0 = ODD ? gv4.z : gv4.x, w1 = ODD ? gv4.w : gv4.y;
                const float gd[4] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1)};
                const unsigned ninf = 0xff800000u;
                unsigned dbl = dq;  // opaque here too: masks are made where used
                asm volatile("" : "+v"(dbl));
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const unsigned mq = (unsigned)__builtin_amdgcn_sbfe((int)dbl, q, 1);
                    const float e = __uint_as_float((__float_as_uint(csj - cdv[q]) & mq) | (ninf & ~mq));
                    m[hd / 4 + q] = gd[q] * exp2_fast(e) * ddv[q];
                }
                if (ODD) {
                    const float f = exp2_fast(csj - s_c2[ib * KB + 15]);
                    const float4 vh = *reinterpret_cast<const float4*>(&s_vh[i0]);
                    m[0] = bf16_lo(gv4.x) * (vh.x * f); m[1] = bf16_hi(gv4.x) * (vh.y * f);
                    m[2] = bf16_lo(gv4.y) * (vh.z * f); m[3] = bf16_hi(gv4.y) * (vh.w * f);
                } else {
                    m[4] = m[5] = m[6] = m[7] = 0.f;
                }
            };
            auto block = [&](const uint4 gv4, int nblk, bool odd, float csj) -> bf16x8 {
                float m[8];
                if (ib < nblk - 1) {  // wholly below the tile: decay factored at block end
                    const float f = exp2_fast(csj - s_c2[ib * KB + KB - 1]);
                    const float4 va = *reinterpret_cast<const float4*>(&s_v[i0]);
                    const float4 vb = *reinterpret_cast<const float4*>(&s_v[i0 + 16]);
                    m[0] = bf16_lo(gv4.x) * (va.x * f); m[1] = bf16_hi(gv4.x) * (va.y * f);
                    m[2] = bf16_lo(gv4.y) * (va.z * f); m[3] = bf16_hi(gv4.y) * (va.w * f);
                    m[4] = bf16_lo(gv4.z) * (vb.x * f); m[5] = bf16_hi(gv4.z) * (vb.y * f);
                    m[6] = bf16_lo(gv4.w) * (vb.z * f); m[7] = bf16_hi(gv4.w) * (vb.w * f);
                } else if (odd) {
                    diag(std::true_type{}, gv4, csj, m);
                } else {
                    diag(std::false_type{}, gv4, csj, m);
                }
                return __builtin_bit_cast(
                    bf16x8, make_uint4(pack_bf16(m[0], m[1]), pack_bf16(m[2], m[3]),
                                       pack_bf16(m[4], m[5]), pack_bf16(m[6], m[7])));
            };
            if (ib < NB0 && ib < nb0) {
                const bf16x8 bm = block(gf0[ib < NB0 ? ib : 0], nb0, (tile0 & 1) != 0, csj0);
#pragma unroll
                for (int p = 0; p < PT; ++p) acc0[p] = mfma16(xa[p], bm, acc0[p]);
            }
            {
                const bf16x8 bm = block(gf1[ib], nb1, (tile1 & 1) != 0, csj1);
#pragma unroll
                for (int p = 0; p < PT; ++p) acc1[p] = mfma16(xa[p], bm, acc1[p]);
            }
        }

        // stage 5 and the skip: lane holds y[j][p*16 + 4*g4 + 0..3]; rows past the end of
        // the sequence fall outside the buffer resource and are dropped
        const float dh = D[h];
        const __amdgpu_buffer_rsrc_t yr =
            make_rsrc(y + ((size_t)(b * T + t0) * H + h) * P, (unsigned)Lc * rowb);
        auto store_tile = [&](const f32x4* acc, int j) {
            uint2 o[PT];
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                const int p0 = p * 16 + 4 * g4;
                const uint2 xv = *reinterpret_cast<const uint2*>(bx + swz_off(j, p0, PPR));
                o[p].x = pack_bf16(acc[p][0] + dh * bf16_lo(xv.x), acc[p][1] + dh * bf16_hi(xv.x));
                o[p].y = pack_bf16(acc[p][2] + dh * bf16_lo(xv.y), acc[p][3] + dh * bf16_hi(xv.y));
            }
            if constexpr (PT % 2 == 0) {
                // 16-byte stores (pair_runs over p-tiles 2q, 2q + 1): each writes 64
                // contiguous bytes of 16 rows
#pragma unroll
                for (int q = 0; q < PT / 2; ++q) {
                    const int p0 = 32 * q + 16 * (g4 & 1) + 8 * (g4 >> 1);
                    buf_store16(yr, (unsigned)j * rowb + p0 * 2u,
                                pair_runs(o[2 * q], o[2 * q + 1]));
                }
            } else {
#pragma unroll
                for (int p = 0; p < PT; ++p)
                    buf_store8(yr, (unsigned)j * rowb + (p * 16 + 4 * g4) * 2u, o[p]);
            }
        };
        if constexpr (GATE) {
            // out = norm(y * SiLU(z)) per token over groups of S = P / gph channels: a row's
            // P channels sit in the four lane groups of its lanes (p-tile p, channels
            // p * 16 + 4 g4 + 0..3), so a group's sums are per-lane sums over its p-tiles,
            // summed over the lane groups (colsum); mean, then the squared deviations
            const int gph = gn.groups_per_head;
            const int ppg = PT / gph;  // p-tiles per group
            const float inv_s = 1.f / (float)(16 * ppg);
            const float* wh = gn.w + (size_t)h * P;
            const float* bh = gn.b ? gn.b + (size_t)h * P : nullptr;
            auto gate_tile = [&](const f32x4* acc, const uint2* zt, int j) {
                float v[PT][4];
#pragma unroll
                for (int p = 0; p < PT; ++p) {
                    const int p0 = p * 16 + 4 * g4;
                    const uint2 xv = *reinterpret_cast<const uint2*>(bx + swz_off(j, p0, PPR));
                    const uint2 zq = zt[p];
                    const float xs[4] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
                    const float zs[4] = {bf16_lo(zq.x), bf16_hi(zq.x), bf16_lo(zq.y), bf16_hi(zq.y)};
#pragma unroll
                    for (int e = 0; e < 4; ++e)  // SiLU(z) = z / (1 + exp(-z)), v_rcp_f32
                        v[p][e] = fmaf(dh, xs[e], acc[p][e]) *
                                  (zs[e] * __builtin_amdgcn_rcpf(1.f + __expf(-zs[e])));
                }
                // group sums over the tile's p-tiles (the group of p-tile p is p / ppg)
                auto group_sum = [&](const float (&ps)[PT], float (&gs)[PT]) {
#pragma unroll
                    for (int p = 0; p < PT; ++p) {
                        float t = 0.f;
#pragma unroll
                        for (int q2 = 0; q2 < PT; ++q2)
                            t += (q2 / ppg == p / ppg) ? ps[q2] : 0.f;
                        gs[p] = t;
                    }
                };
                float ps[PT], mean[PT], var[PT];
#pragma unroll
                for (int p = 0; p < PT; ++p) {
                    ps[p] = gn.rms ? 0.f : colsum((v[p][0] + v[p][1]) + (v[p][2] + v[p][3]));
                }
                group_sum(ps, mean);
#pragma unroll
                for (int p = 0; p < PT; ++p) {
                    mean[p] *= inv_s;
                    float sq = 0.f;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const float dv = v[p][e] - mean[p];
                        sq = fmaf(dv, dv, sq);
                    }
                    ps[p] = colsum(sq);
                }
                group_sum(ps, var);
                uint2 o[PT];
#pragma unroll
                for (int p = 0; p < PT; ++p) {
                    const int p0 = p * 16 + 4 * g4;
                    const float rstd = __builtin_amdgcn_rsqf(var[p] * inv_s + gn.eps);
                    const float4 w4 = *reinterpret_cast<const float4*>(wh + p0);
                    const float4 b4 = (bh && !gn.rms) ? *reinterpret_cast<const float4*>(bh + p0)
                                                      : make_float4(0.f, 0.f, 0.f, 0.f);
                    const float wv[4] = {w4.x, w4.y, w4.z, w4.w};
                    const float bv[4] = {b4.x, b4.y, b4.z, b4.w};
                    float ov[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ov[e] = fmaf((v[p][e] - mean[p]) * rstd, wv[e], bv[e]);
                    o[p] = make_uint2(pack_bf16(ov[0], ov[1]), pack_bf16(ov[2], ov[3]));
                }
                if constexpr (PT % 2 == 0) {
#pragma unroll
                    for (int q = 0; q < PT / 2; ++q) {
                        const int p0 = 32 * q + 16 * (g4 & 1) + 8 * (g4 >> 1);
                        buf_store16(yr, (unsigned)j * rowb + p0 * 2u,
                                    pair_runs(o[2 * q], o[2 * q + 1]));
                    }
                } else {
#pragma unroll
                    for (int p = 0; p < PT; ++p)
                        buf_store8(yr, (unsigned)j * rowb + (p * 16 + 4 * g4) * 2u, o[p]);
                }
            };
            gate_tile(acc0, zq0, j0);
            gate_tile(acc1, zq1, j1);
        } else {
            store_tile(acc0, j0);
            store_tile(acc1, j1);
        }
        if constexpr (!CRES)
            if (n + 1 < hi - lo) load_c(sl - 1);
        if constexpr (GATE)
            if (n + 1 < hi - lo) load_z(sl - 1);
        if (C_::NBUF == 1 && n + 1 < hi - lo) {
            lds_barrier();  // every wave is done with the buffer
            issue_item<Q, N, P>(x, E, cs, dtc, sl - 1, hpg, T, H, G, nC, lds0, wave, lane);
        }
        buf = (C_::NBUF == 1) ? 0 : (buf + 1 == C_::NBUF ? 0 : buf + 1);
    }
}

// ---------------------------------------------------------------- dispatch

template <int Q, int N, int P, bool GATE = false>
hipError_t launch_scan_t(const Shape& s, const void* x, const void* Cm, const float* dtc,
                         const float* cs, const float* D, const void* E, const void* gram,
                         void* y, hipStream_t st, const GateNorm* gate) {
    using C_ = ScanCfg<Q, N, P>;
    const auto kern = chunk_scan_mfma_kernel<Q, N, P, GATE>;
    const GateNorm gn = gate ? *gate : GateNorm{nullptr, 0, nullptr, nullptr, 1, 0, 0.f};
    // per device: allow the dynamic LDS size, and size the persistent grid to what is
    // resident at once (a multiple of 8 workgroups, one run of items each)
    static DeviceSlots grid_of;
    int grid = 0;
    const hipError_t e = resident_grid((const void*)kern, C_::NTH, C_::LDS, grid_of, &grid);
    if (e != hipSuccess) return e;
    const int nslots = s.B * s.G * s.nC * (s.H / s.G);
    kern<<<grid, C_::NTH, C_::LDS, st>>>(
        (const __bf16*)x, (const __bf16*)Cm, dtc, cs, D, (const __bf16*)E, (const uint4*)gram,
        (__bf16*)y, s.T, s.H, s.G, s.nC, nslots, gn);
    return hipGetLastError();
}

template <int Q, int N>
hipError_t launch_gram_t(const Shape& s, const void* Bm, const void* Cm, void* gram,
                         hipStream_t st) {
    using C_ = GramCfg<Q, N>;
    const auto kern = chunk_gram_kernel<Q, N>;
    static DeviceSlots attr_set;
    const hipError_t e = allow_lds((const void*)kern, C_::LDS, attr_set);
    if (e != hipSuccess) return e;
    const unsigned blocks = (unsigned)((size_t)s.B * s.G * s.nC);
    kern<<<blocks, C_::NTH, C_::LDS, st>>>((const __bf16*)Bm, (const __bf16*)Cm, (uint4*)gram,
                                           s.T, s.G, s.nC);
    return hipGetLastError();
}

using ScanFn = hipError_t (*)(const Shape&, const void*, const void*, const float*, const float*,
                              const float*, const void*, const void*, void*, hipStream_t,
                              const GateNorm*);
using GramFn = hipError_t (*)(const Shape&, const void*, const void*, void*, hipStream_t);

template <int Q, int N>
ScanFn pick_scan_qn(const Shape& s) {
    switch (s.P) {
        case 16: return launch_scan_t<Q, N, 16>;
        case 32: return launch_scan_t<Q, N, 32>;
        case 64: return launch_scan_t<Q, N, 64>;
        case 128: return launch_scan_t<Q, N, 128>;
    }
    return nullptr;
}
template <int Q>
ScanFn pick_scan_q(const Shape& s) {
    switch (s.N) {
        case 32: return pick_scan_qn<Q, 32>(s);
        case 64: return pick_scan_qn<Q, 64>(s);
        case 128: return pick_scan_qn<Q, 128>(s);
        case 256: return pick_scan_qn<Q, 256>(s);
    }
    return nullptr;
}
// the gated store: head sizes whose p-tiles split into 1, 2 or 4 groups of 16 channels or more
template <int Q, int N>
ScanFn pick_scan_gate_qn(const Shape& s) {
    switch (s.P) {
        case 32: return launch_scan_t<Q, N, 32, true>;
        case 64: return launch_scan_t<Q, N, 64, true>;
    }
    return nullptr;
}
template <int Q>
ScanFn pick_scan_gate_q(const Shape& s) {
    switch (s.N) {
        case 32: return pick_scan_gate_qn<Q, 32>(s);
        case 64: return pick_scan_gate_qn<Q, 64>(s);
        case 128: return pick_scan_gate_qn<Q, 128>(s);
        case 256: return pick_scan_gate_qn<Q, 256>(s);
    }
    return nullptr;
}
template <int Q>
GramFn pick_gram_q(const Shape& s) {
    switch (s.N) {
        case 32: return launch_gram_t<Q, 32>;
        case 64: return launch_gram_t<Q, 64>;
        case 128: return launch_gram_t<Q, 128>;
        case 256: return launch_gram_t<Q, 256>;
    }
    return nullptr;
}

bool scan_offsets_fit(const Shape& s) {
    // buffer resources address one chunk of x / y (and B, C) with 32-bit byte offsets
    return (size_t)s.Q * s.H * s.P * 2 < ((size_t)1 << 31) &&
           (size_t)s.Q * s.G * s.N * 2 < ((size_t)1 << 31);
}

ScanFn pick_scan(const Shape& s) {
    if (!scan_offsets_fit(s)) return nullptr;
    switch (s.Q) {
        case 64: return pick_scan_q<64>(s);
        case 128: return pick_scan_q<128>(s);
        case 256: return pick_scan_q<256>(s);
    }
    return nullptr;
}
ScanFn pick_scan_gate(const Shape& s) {
    if (!scan_offsets_fit(s)) return nullptr;
    switch (s.Q) {
        case 64: return pick_scan_gate_q<64>(s);
        case 128: return pick_scan_gate_q<128>(s);
        case 256: return pick_scan_gate_q<256>(s);
    }
    return nullptr;
}
GramFn pick_gram(const Shape& s) {
    if (!scan_offsets_fit(s)) return nullptr;
    switch (s.Q) {
        case 64: return pick_gram_q<64>(s);
        case 128: return pick_gram_q<128>(s);
        case 256: return pick_gram_q<256>(s);
    }
    return nullptr;
}

}  // namespace

bool chunk_scan_mfma_supported(const Shape& s) { return pick_scan(s) != nullptr; }

bool chunk_scan_gate_supported(const Shape& s, int groups_per_head) {
    const int pt = s.P / 16;
    return pick_scan_gate(s) != nullptr && groups_per_head >= 1 && groups_per_head <= pt &&
           pt % groups_per_head == 0;
}

size_t chunk_gram_bytes(const Shape& s) {
    if (!chunk_scan_mfma_supported(s)) return 0;
    return (size_t)s.B * s.G * s.nC * npairs(s.Q) * 64 * 16;
}

hipError_t launch_chunk_gram(const Shape& s, const void* Bm, const void* Cm, void* gram,
                             hipStream_t st) {
    GramFn f = pick_gram(s);
    if (!f) return hipErrorInvalidValue;
    if ((size_t)s.B * s.G * s.nC == 0) return hipSuccess;
    return f(s, Bm, Cm, gram, st);
}

hipError_t launch_chunk_scan_mfma(const Shape& s, const void* x, const void* Cm, const float* dtc,
                                  const float* cs, const float* D, const void* entry,
                                  const void* gram, void* y, hipStream_t st,
                                  const GateNorm* gate) {
    ScanFn f = gate ? pick_scan_gate(s) : pick_scan(s);
    if (!f || (gate && !chunk_scan_gate_supported(s, gate->groups_per_head)))
        return hipErrorInvalidValue;
    if ((size_t)s.B * s.G * s.nC == 0) return hipSuccess;
    return f(s, x, Cm, dtc, cs, D, entry, gram, y, st, gate);
}

}  // namespace ssd
