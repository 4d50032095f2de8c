// chunk_bwd_mfma.hip -- the in-chunk backward on gfx950 bf16 MFMA (headdim 64 with dstate 64,
// 128 or 256, headdim 32 with dstate 32, 64 or 128; any supported chunk length).
//
// It computes what chunk_bwd_valu.hip computes (the formulas are stated there): dx, the
// head-summed dB and dC, and per head the explicit step-size gradient and dL/dcs.
//
// One workgroup of eight waves per (batch, group, chunk, block J of 64 rows), looping over
// the heads of the group.  Waves w and w + 4 own the 16 columns j = j0 + 16 w + (0..15) of
// J and share a SIMD: wave w (a "strip" wave) does the products inside the chunk, wave w + 4
// (a "state" wave) those through the carried states, and they meet in LDS once per head
// (the state wave's (F B_j) tiles and per-row sums go to the strip wave, which finishes dx)
// and once per workgroup (the strip wave's W goes to the state wave, which holds dB, dC).
// The two roles run in separate branches with the same barriers, so neither role's
// registers are held while the other's code runs.  With
// M = dy x^T, W[t][i] = dt_i exp(cs_t - cs_i) M[t][i] (t >= i) is the matrix whose
// head sum gives both diagonal-block products, dC_j += sum_i W[j][i] B_i and
// dB_j += sum_t W[t][j] C_t.  For its columns a wave needs
//   the row strip  W^T[i][j], i <= j   (rows i of W^T, from M^T = x dy^T)  -> dC_j
//   the column strip W[t][j],  t >= j  (rows t, from M = dy x^T)          -> dB_j, dx_j
// taken as whole 32-row blocks covering rows [0, j0 + 64) and [j0, Q): Q / 16 + 4 tiles of
// 16 x 16 for every wave and every J.  W is accumulated over the heads in registers (fp32),
// so dB and dC cost two products per workgroup rather than per head.  Outside J the decays
// factor through a row of J (row_factors): the product tiles' rows are scaled by one
// factor each, so only the four blocks inside J need work per element.
//
// Everything is computed transposed so that the output rows (j) are MFMA columns: a lane
// holds 4 consecutive p (or n) of one row j, which makes every per-row scalar a column sum
// over the four lane groups (stores pair two such runs into 16 bytes, pair_runs):
//   dx^T[p][j]  = D dy + dt_j (sum_t dy[t][p] U[t][j] + exp(cs_last - cs_j) (F B_j)[p])
//                 with U[t][j] = exp(cs_t - cs_j) (C_t . B_j)
//   dB^T[n][j] += sum_p F[p][n] (dt_j exp(cs_last - cs_j) x_j[p])   (+ sum_t C[t][n] W[t][j])
//   dC^T[n][j] += sum_p E[p][n] (exp(cs_j) dy_j[p])                  (+ sum_i B[i][n] W^T[i][j])
// MFMA operand layouts are those of mfma_common.h: contractions over time (t, i) and over
// p use the 8-slot relabelling so that accumulator tiles feed the next product directly;
// contractions over n (the C B^T tiles, F B_j) read natural 8-element runs.
//
// Per head the x rows [0, j0 + 64) and dy rows [j0, Q) (one array of Q + 64 rows), E, F,
// cs and dt are copied into LDS straight from HBM (buffer_load ... lds), double-buffered
// so that the next head's copy runs under this head's products.  The state waves issue
// the copy; at the end of a head each waits for its own share and a workgroup barrier
// follows (two barriers per head: this one and the hand-off).  The group's B and C
// chunks pass through the same LDS before the loop (for C B^T and the B_j, C_j operands;
// in column slices where whole chunks do not fit) and after it (for the two W products).
//
// At dstate 256 the terms through E and F are formed first, by chunk_bwd_carried_kernel
// (at the end of this file), and this kernel takes them from HBM (BwdCfg::EXT).
#include "mfma_common.h"
#include "ssd_internal.h"

namespace ssd {
namespace {

using namespace mfma;

// 8 bf16 at the natural k-slots 32kb + 8g .. +7
__device__ __forceinline__ bf16x8 frag_nat(const unsigned char* base, int row, int kb, int g4,
                                          int ppr) {
    return *reinterpret_cast<const bf16x8*>(base + swz_off(row, 32 * kb + 8 * g4, ppr));
}
// Row rb + rl of a swizzled [rows][8 ppr] bf16 matrix, with rb a multiple of 16 and rl < 16:
// the swizzle (by row % min(ppr, 16), as issue_rows writes it) depends only on rl, so a
// lane's part of the byte offset is computed once per head and the row base is a uniform
// offset (an immediate where it is a constant).
__device__ __forceinline__ unsigned lane_part(int rl, int col, int ppr) {
    return (unsigned)(rl * ppr + ((col >> 3) ^ (rl & (ppr - 1)))) * 16u + (unsigned)(col & 7) * 2u;
}
__device__ __forceinline__ const unsigned char* rows_at(const unsigned char* base, int rb, int ppr) {
    return base + rb * ppr * 16;
}
// relabelled k-slots (two 8-byte halves at lane parts lo, hi)
__device__ __forceinline__ bf16x8 ld_rl(const unsigned char* p, unsigned lo, unsigned hi) {
    const uint2 a = *reinterpret_cast<const uint2*>(p + lo);
    const uint2 b = *reinterpret_cast<const uint2*>(p + hi);
    return __builtin_bit_cast(bf16x8, make_uint4(a.x, a.y, b.x, b.y));
}
__device__ __forceinline__ bf16x8 ld_nat(const unsigned char* p, unsigned off) {
    return *reinterpret_cast<const bf16x8*>(p + off);
}
// transpose read of a 32-row block: rows 0..15 at p + off, rows 16..31 at p + off + plus16
__device__ __forceinline__ bf16x8 ld_tr(const unsigned char* p, unsigned off, unsigned plus16) {
    const uint2 lo = lds_read_tr16(p + off);
    const uint2 hi = lds_read_tr16(p + off + plus16);
    return __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
}
__device__ __forceinline__ bf16x8 scale8(bf16x8 v, float s) {
    const uint4 r = __builtin_bit_cast(uint4, v);
    return __builtin_bit_cast(
        bf16x8, make_uint4(pack_bf16(bf16_lo(r.x) * s, bf16_hi(r.x) * s),
                           pack_bf16(bf16_lo(r.y) * s, bf16_hi(r.y) * s),
                           pack_bf16(bf16_lo(r.z) * s, bf16_hi(r.z) * s),
                           pack_bf16(bf16_lo(r.w) * s, bf16_hi(r.w) * s)));
}
__device__ __forceinline__ float dot8(bf16x8 a, bf16x8 b) {
    const uint4 x = __builtin_bit_cast(uint4, a), y = __builtin_bit_cast(uint4, b);
    float s = bf16_lo(x.x) * bf16_lo(y.x);
    s = fmaf(bf16_hi(x.x), bf16_hi(y.x), s);
    s = fmaf(bf16_lo(x.y), bf16_lo(y.y), s);
    s = fmaf(bf16_hi(x.y), bf16_hi(y.y), s);
    s = fmaf(bf16_lo(x.z), bf16_lo(y.z), s);
    s = fmaf(bf16_hi(x.z), bf16_hi(y.z), s);
    s = fmaf(bf16_lo(x.w), bf16_lo(y.w), s);
    return fmaf(bf16_hi(x.w), bf16_hi(y.w), s);
}
// v plus v from another lane of its 16-lane row, by a DPP row permutation
template <int CTRL>
__device__ __forceinline__ float add_dpp(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF,
                                                          false));
}
// Sum over the wave, the same value in every lane: the lane groups, then inside a row the
// pairs (quad_perm [1,0,3,2]), the quads' halves ([2,3,0,1]), the two quads of each half
// row (row_half_mirror) and the two halves (row_mirror).
__device__ __forceinline__ float wavesum(float v) {
    v = colsum(v);
    v = add_dpp<0xB1>(v);
    v = add_dpp<0x4E>(v);
    v = add_dpp<0x141>(v);
    return add_dpp<0x140>(v);
}

// nrows rows of a [rows][feat] bf16 matrix (row stride rowb bytes in HBM, from row
// src_row0, from byte colb of each row) into LDS rows dst_row0.. (PPRX 16-byte pieces per
// row), swizzled.  Each instruction fills 64 consecutive 16-byte LDS slots (lane L at its
// base + 16 L), so the swizzle is applied on the source side: slot `sl` of LDS row dr
// receives piece sl ^ (dr % 16) (dr % PPRX for rows of fewer than 16 pieces; the XOR keeps
// a piece inside its aligned group of 16, and lane_part's row offset rl < 16 reads the
// same swizzle).  nrows * PPRX is a multiple of 64.  A wave's successive instructions
// are NW * 64 / PPRX rows apart, a multiple of the swizzle period, so the lane's source
// offset only advances by that many rows: it is formed once and then stepped.
template <int PPRX, int NW>
__device__ __forceinline__ void issue_rows(u32x4 rsrc, unsigned rowb, int src_row0, uint32_t lds,
                                           int dst_row0, int nrows, int wave, int lane,
                                           unsigned colb = 0) {
    constexpr int SWM = (PPRX < 16 ? PPRX : 16) - 1;
    constexpr int RSTEP = NW * 64 / PPRX;  // rows between a wave's instructions
    static_assert(NW * 64 % PPRX == 0 && RSTEP % (SWM + 1) == 0, "stepped offsets");
    const int ninst = nrows * PPRX / 64;
    const uint32_t base = lds + (unsigned)dst_row0 * PPRX * 16u;
    const int m = wave * 64 + lane;
    const int r = m / PPRX, sl = m % PPRX;
    unsigned voff =
        (unsigned)(src_row0 + r) * rowb + colb + (unsigned)(sl ^ ((dst_row0 + r) & SWM)) * 16u;
    const unsigned vstep = (unsigned)RSTEP * rowb;
    for (int k = wave; k < ninst; k += NW) {
        dma16(rsrc, base + (unsigned)k * 1024u, voff);
        voff += vstep;
    }
}

// Makes an accumulator update happen where it is written: otherwise the compiler sinks
// the updates of a head to the end of the loop and keeps every product they use live
// across the rest of the head.
__device__ __forceinline__ void pin(f32x4& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void pin(float& v) { asm volatile("" : "+v"(v)); }

template <int Q, int N, int P>
struct BwdCfg {
    static constexpr int NW = 8, NTH = 512;         // 4 strip waves + 4 state waves
    static constexpr int NJ = Q / 64;               // row blocks per chunk
    static constexpr int PAIRS = Q / 32 + 2;        // 32-row blocks of strip per wave
    static constexpr int PPR = P / 8, NPR = N / 8;  // 16-byte pieces per row
    static constexpr int NKB = N / 32, PKB = P / 32;
    static constexpr int NT = N / 16, PT = P / 16;
    // dstate 256: the terms through the carried states come from chunk_bwd_carried_kernel
    // (E and F are not copied here), B and C pass through LDS in column slices for C B^T
    // and in two halves of n for the W products, and the state waves' dB, dC accumulators
    // start from that kernel's sums
    static constexpr bool EXT = N > 128;
    static constexpr int HN = EXT ? 128 : N;        // columns of B / C per W-product pass
    static constexpr int NHP = N / HN;
    static constexpr unsigned XYB = (Q + 64) * P * 2;  // x rows [0, j0+64), dy rows [j0, Q)
    static constexpr unsigned EB = EXT ? 0 : P * N * 2;  // E or F, [p][n]
    static constexpr unsigned FB = Q * 4;              // cs or dt
    static constexpr unsigned ITEM = XYB + 2 * EB + 2 * FB;
    // columns of B / C per C B^T slice: whole chunks where both fit the two item buffers
    // (all of n for headdim 64 below dstate 256)
    static constexpr int SLN = EXT ? 64
                               : 2u * Q * N * 2 <= 2 * ITEM ? N
                               : 2u * Q * 64 * 2 <= 2 * ITEM ? 64 : 32;
    static constexpr bool SLICED = SLN < N;
    static constexpr int NSL = N / SLN;
    static constexpr unsigned BCB = Q * SLN * 2;       // one B or C chunk (slice)
    // exchange from the state waves to the strip waves, after the two item buffers
    static constexpr unsigned X_BF = 2 * ITEM;                // (F B_j) tiles, bf16 [4][PT][64]
    static constexpr unsigned X_OB = X_BF + 4 * PT * 64 * 8;  // ob, oc per column [2][64]
    static constexpr unsigned X_EF = X_OB + 2 * 64 * 4;       // <E, F> share per wave [4]
    static constexpr unsigned X_SH = X_EF + 16;               // workgroup shares [2][4][2]
    // each strip wave's row factors of its head (the Q - 64 rows outside J) [4][Q - 64]
    static constexpr unsigned X_RF = X_SH + 64;
    static constexpr unsigned X_END = X_RF + 4 * (Q - 64) * 4;
    // the W accumulators (bf16) travel from the strip waves after the B/C rows at the end:
    // inside the item buffers where they fit, else past the exchange area
    static constexpr unsigned WB = 4u * PAIRS * 64 * 16;
    static constexpr bool W_IN_ITEMS = !EXT && (Q + 64) * N * 2 + WB <= 2 * ITEM;
    static constexpr unsigned X_W =
        W_IN_ITEMS ? (Q + 64) * N * 2
                   : ((Q + 64) * HN * 2 > X_END ? (Q + 64) * HN * 2 : X_END);
    static constexpr unsigned LDS = W_IN_ITEMS ? X_END : X_W + WB;
    static_assert((P == 64 && (N == 64 || N == 128 || N == 256)) ||
                      (P == 32 && (N == 32 || N == 64 || N == 128)),
                  "shape");
    static_assert(2 * BCB <= 2 * ITEM, "B and C chunks fit the item buffers");
    static_assert(X_W % 16 == 0 && LDS <= 160 * 1024, "LDS");
};

// One head's rows, states and step sizes, copied by the four state waves (iw = 0..3): their
// own vector-memory count then covers the whole copy, so they can wait for it without a
// barrier with the strip waves.
template <int Q, int N, int P>
__device__ __forceinline__ void issue_item(const __bf16* x, const __bf16* dy, const __bf16* entry,
                                           const __bf16* exitg, const float* cs, const float* dtc,
                                           int b, int h, int c, int j0, int Lc, int T, int H,
                                           int nC, uint32_t lds, int iw, int lane) {
    using C_ = BwdCfg<Q, N, P>;
    constexpr int NW = 4;
    const int wave = iw;
    const unsigned rowb = (unsigned)(H * P * 2);
    const size_t xo = ((size_t)(b * T + c * Q) * H + h) * P;
    const u32x4 xr = raw_rsrc(x + xo, (unsigned)Lc * rowb);
    const u32x4 yr = raw_rsrc(dy + xo, (unsigned)Lc * rowb);
    // x rows [0, j0 + 64) at LDS rows 0.., dy rows [j0, Q) at LDS rows j0 + 64..
    issue_rows<C_::PPR, NW>(xr, rowb, 0, lds, 0, j0 + 64, wave, lane);
    issue_rows<C_::PPR, NW>(yr, rowb, j0, lds, j0 + 64, Q - j0, wave, lane);
    if constexpr (!C_::EXT) {
        const size_t so = ((size_t)(b * H + h) * nC + c) * P * N;
        issue_rows<C_::NPR, NW>(raw_rsrc(entry + so, C_::EB), N * 2, 0, lds + C_::XYB, 0, P,
                                wave, lane);
        issue_rows<C_::NPR, NW>(raw_rsrc(exitg + so, C_::EB), N * 2, 0, lds + C_::XYB + C_::EB,
                                0, P, wave, lane);
    }
    const size_t cb = ((size_t)(b * H + h) * nC + c) * Q;
    if (wave == 0 && lane < Q / 4)
        dma16(raw_rsrc(cs + cb, C_::FB), lds + C_::XYB + 2 * C_::EB, lane * 16u);
    if (wave == 1 && lane < Q / 4)
        dma16(raw_rsrc(dtc + cb, C_::FB), lds + C_::XYB + 2 * C_::EB + C_::FB, lane * 16u);
}

// B and C of the group's chunk, columns [part * cols, +cols) (cols = SLN for whole chunks,
// HN for the rows of the W products; all of n below dstate 256)
template <int Q, int N, int P>
__device__ __forceinline__ void issue_bc(const __bf16* Bm, const __bf16* Cm, int b, int g, int t0,
                                         int Lc, int T, int G, int j0, bool rows_only,
                                         uint32_t lds, int wave, int lane, int part = 0) {
    using C_ = BwdCfg<Q, N, P>;
    constexpr int SPR = C_::SLN / 8, HPR = C_::HN / 8;  // pieces per staged row
    const unsigned rowb = (unsigned)(G * N * 2);
    const size_t bo = ((size_t)(b * T + t0) * G + g) * N;
    const u32x4 br = raw_rsrc(Bm + bo, (unsigned)Lc * rowb);
    const u32x4 cr = raw_rsrc(Cm + bo, (unsigned)Lc * rowb);
    if (!rows_only) {  // whole chunks: B at 0, C at BCB
        const unsigned colb = (unsigned)part * C_::SLN * 2u;
        issue_rows<SPR, C_::NW>(br, rowb, 0, lds, 0, Q, wave, lane, colb);
        issue_rows<SPR, C_::NW>(cr, rowb, 0, lds + C_::BCB, 0, Q, wave, lane, colb);
    } else {  // B rows [0, j0 + 64) at rows 0.., C rows [j0, Q) at rows j0 + 64..
        const unsigned colb = (unsigned)part * C_::HN * 2u;
        issue_rows<HPR, C_::NW>(br, rowb, 0, lds, 0, j0 + 64, wave, lane, colb);
        issue_rows<HPR, C_::NW>(cr, rowb, j0, lds, j0 + 64, Q - j0, wave, lane, colb);
    }
}

// ------------------------------------------------------------------ decays factored per row
// Outside J the causal decay factors through a fixed row of the chunk: for i < j0 <= j,
// exp(cs_j - cs_i) = exp(cs_j - cs_j0) exp(cs_j0 - cs_i), and for t > j0 + 63 >= j,
// exp(cs_t - cs_j) = exp(cs_t - cs_j0+63) exp(cs_j0+63 - cs_j), every factor <= 1.  Per
// head, each strip wave forms the row factors (with dt_i for the row strip) of the Q - 64
// rows outside J in its own LDS slice, rf[i] = dt_i exp(cs_j0 - cs_i) for rows i < j0 and
// rf[t - 64] = exp(cs_t - cs_j0+63) for rows t > j0 + 63, and applies them to the rows of
// its product tiles (and to the C B^T operand of dx), so only the blocks inside J need work
// per element.  The slice is the wave's own (a wave's LDS accesses complete in order), so
// no workgroup barrier stands between forming and reading it.
template <int Q, int N, int P>
__device__ __forceinline__ void row_factors(const unsigned char* sXY, float* rf, int j0,
                                            int lane) {
    const float* s_cs = reinterpret_cast<const float*>(sXY + BwdCfg<Q, N, P>::XYB +
                                                       2 * BwdCfg<Q, N, P>::EB);
    const float* s_dt = s_cs + Q;
    const float cs_a = s_cs[j0], cs_b = s_cs[j0 + 63];
    for (int i = lane; i < Q - 64; i += 64) {
        if (i < j0) {
            rf[i] = s_dt[i] * exp2_fast((cs_a - s_cs[i]) * kLog2e);
        } else {
            const int t = i + 64;
            rf[i] = exp2_fast((s_cs[t] - cs_b) * kLog2e);
        }
    }
}

// the four row factors of rows r .. r + 3 (r a multiple of 4)
__device__ __forceinline__ float4 rf4(const float* rf, int r) {
    return *reinterpret_cast<const float4*>(rf + r);
}
// 4 bf16 (a uint2) times 4 factors, rounded back to bf16
__device__ __forceinline__ uint2 scale4(uint2 v, float4 f) {
    return make_uint2(pack_bf16(bf16_lo(v.x) * f.x, bf16_hi(v.x) * f.y),
                      pack_bf16(bf16_lo(v.y) * f.z, bf16_hi(v.y) * f.w));
}

// Everything both roles need to know about their workgroup
struct BwdCtx {
    int b, g, c, rj, j0, t0, Lc, hpg, T, H, G, nC;
    int wave, cw, lane;   // wave 0..7, column tile 0..3 of the block, lane
    uint32_t lds0;
};

// ------------------------------------------------------------------ strip waves
// M strips, W accumulated over heads, C B^T on the strips, the W.G sums, the diagonal part
// of dx; they finish dx and the per-row results of every head.  Instantiated per row block
// (RJ) and column tile (CW), so that the block layout and which tiles inside J are causal,
// masked or diagonal are known at compile time:
//   row strip  blocks k < RSP: x rows [32k, 32k + 32), the last two inside J
//   column strip blocks k < CSP: dy rows [j0 + 32k, +32), the first two inside J
template <int Q, int N, int P, int RJ, int CW>
__device__ __forceinline__ void bwd_strip_role(
    const BwdCtx& k_, unsigned char* smem, const __bf16* x, const __bf16* Bm, const __bf16* Cm,
    const float* dtc, const float* cs, const float* D, const __bf16* entry, const __bf16* exitg,
    const __bf16* dy, __bf16* dx, float* dcs, float* direct, float* xs, float* lt_part,
    float* dd_part) {
    using C_ = BwdCfg<Q, N, P>;
    constexpr int NJ = C_::NJ, PAIRS = C_::PAIRS, PPR = C_::PPR, NPR = C_::NPR;
    constexpr int NKB = C_::NKB, PKB = C_::PKB, PT = C_::PT;
    constexpr int j0 = 64 * RJ;
    constexpr int RSO = 2 * RJ, RSP = RSO + 2;   // row strip: blocks before J, all
    constexpr int CSP = (Q - j0) / 32;           // column strip blocks
    static_assert(RSP + CSP == PAIRS, "layout");
    const int b = k_.b, g = k_.g, c = k_.c, t0 = k_.t0, Lc = k_.Lc;
    const int hpg = k_.hpg, T = k_.T, H = k_.H, G = k_.G, nC = k_.nC;
    const int wave = k_.wave, lane = k_.lane;
    constexpr int cw = CW;
    float* const shares = reinterpret_cast<float*>(smem + C_::X_SH);

    // C B^T on the strips, rounded to bf16: G^T[i][j] = B_i . C_j and G[t][j] = C_t . B_j
    uint2 gt[2 * PAIRS];
    if constexpr (C_::SLICED) {
        // summed in fp32 over column slices of B and C
        constexpr int SPR = C_::SLN / 8, SKB = C_::SLN / 32;
        const int l16 = lane & 15, g4 = lane >> 4;
        const int jl = j0 + 16 * cw + l16;
        const unsigned char* sBc = smem;
        const unsigned char* sCc = smem + C_::BCB;
        f32x4 ga[2 * PAIRS];
#pragma unroll
        for (int s = 0; s < 2 * PAIRS; ++s) ga[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
        for (int sl = 0; sl < C_::NSL; ++sl) {
            issue_bc<Q, N, P>(Bm, Cm, b, g, t0, Lc, T, G, j0, false, k_.lds0, wave, lane, sl);
            dma_barrier();
            bf16x8 bj[SKB], cj[SKB];
#pragma unroll
            for (int kb = 0; kb < SKB; ++kb) {
                bj[kb] = frag_nat(sBc, jl, kb, g4, SPR);
                cj[kb] = frag_nat(sCc, jl, kb, g4, SPR);
            }
#pragma unroll
            for (int k = 0; k < PAIRS; ++k) {
                const bool isrs = k < RSP;
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int row = (isrs ? 32 * k : j0 + 32 * (k - RSP)) + 16 * u + l16;
                    const unsigned char* src = isrs ? sBc : sCc;
#pragma unroll
                    for (int kb = 0; kb < SKB; ++kb)
                        ga[2 * k + u] = mfma16(frag_nat(src, row, kb, g4, SPR),
                                               isrs ? cj[kb] : bj[kb], ga[2 * k + u]);
                }
            }
            lds_barrier();  // this slice is no longer read
        }
#pragma unroll
        for (int s = 0; s < 2 * PAIRS; ++s)
            gt[s] = make_uint2(pack_bf16(ga[s][0], ga[s][1]), pack_bf16(ga[s][2], ga[s][3]));
    } else {
        issue_bc<Q, N, P>(Bm, Cm, b, g, t0, Lc, T, G, j0, false, k_.lds0, wave, lane);
        dma_barrier();
        const int l16 = lane & 15, g4 = lane >> 4;
        const int jl = j0 + 16 * cw + l16;
        const unsigned char* sBc = smem;
        const unsigned char* sCc = smem + C_::BCB;
        bf16x8 bj[NKB], cj[NKB];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            bj[kb] = frag_nat(sBc, jl, kb, g4, NPR);
            cj[kb] = frag_nat(sCc, jl, kb, g4, NPR);
        }
#pragma unroll
        for (int k = 0; k < PAIRS; ++k) {
            const bool isrs = k < RSP;
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int row = (isrs ? 32 * k : j0 + 32 * (k - RSP)) + 16 * u + l16;
                const unsigned char* src = isrs ? sBc : sCc;
                f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
                    acc = mfma16(frag_nat(src, row, kb, g4, NPR), isrs ? cj[kb] : bj[kb], acc);
                gt[2 * k + u] = make_uint2(pack_bf16(acc[0], acc[1]), pack_bf16(acc[2], acc[3]));
            }
        }
        lds_barrier();  // B and C are no longer read: the item buffers are free
    }

    f32x4 wacc[2 * PAIRS];  // W over the strips, summed over the heads
#pragma unroll
    for (int s = 0; s < 2 * PAIRS; ++s) wacc[s] = f32x4{0.f, 0.f, 0.f, 0.f};

    dma_barrier();  // the first head's rows have landed (copied by the state waves)
#pragma unroll 1
    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        const int buf = hh & 1;
        // (this head's copies have landed: the barrier at the end of the previous head)
        if (!C_::EXT && hh > 0 && wave == 0 && lane == 0) {
            const float* sh = shares + (buf ^ 1) * 8;
            const size_t pi = ((size_t)(b * H + h - 1) * nC + c) * NJ + RJ;
            lt_part[pi] = (sh[0] + sh[2]) + (sh[4] + sh[6]);
            dd_part[pi] = (sh[1] + sh[3]) + (sh[5] + sh[7]);
        }
        unsigned char* sXY = smem + buf * C_::ITEM;
        const float* s_cs = reinterpret_cast<const float*>(sXY + C_::XYB + 2 * C_::EB);
        const float* s_dt = s_cs + Q;
        float* const rfw = reinterpret_cast<float*>(smem + C_::X_RF) + cw * (Q - 64);
        row_factors<Q, N, P>(sXY, rfw, j0, lane);
        asm volatile("" ::: "memory");  // the factors are read below by this wave only
        const float* s_rf = rfw;
        // lane-dependent values re-derived every head from an opaque copy of the lane
        // index: the compiler recomputes the LDS addresses instead of keeping them live
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int l16 = ln & 15, g4 = ln >> 4;
        const int jb = j0 + 16 * cw, jl = jb + l16;
        const bool vj = jl < Lc;
        const float cs_last = s_cs[Q - 1];
        const float csj = s_cs[jl], dtj = s_dt[jl];
        const float fj = exp2_fast((cs_last - csj) * kLog2e);
        const float k1 = exp2_fast((csj - s_cs[j0]) * kLog2e);       // exp(cs_j - cs_j0)
        const float k2 = exp2_fast((s_cs[j0 + 63] - csj) * kLog2e);  // exp(cs_j0+63 - cs_j)
        // the lane's parts of its LDS offsets (see lane_part)
        // contractions over p feed no further product, so they read 8 consecutive p
        // (natural slots: one 16-byte read per fragment)
        unsigned pnp[PKB], ptp[PT], pac[PT];
#pragma unroll
        for (int kb = 0; kb < PKB; ++kb) pnp[kb] = lane_part(l16, 32 * kb + 8 * g4, PPR);
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            ptp[pt] = lane_part(4 * g4 + (l16 >> 2), 16 * pt + 4 * (l16 & 3), PPR);
            pac[pt] = lane_part(l16, 16 * pt + 4 * g4, PPR);
        }
        constexpr unsigned R16 = 16u * PPR * 16u;  // 16 rows of x / dy

        bf16x8 xj[PKB], yj[PKB];  // x_j, dy_j over p, unscaled rows of J
#pragma unroll
        for (int kb = 0; kb < PKB; ++kb) {
            xj[kb] = ld_nat(rows_at(sXY, jb, PPR), pnp[kb]);
            yj[kb] = ld_nat(rows_at(sXY, jb + 64, PPR), pnp[kb]);
        }
        // per-column sums of W.G (W[t][i] G[t][i], i.e. the terms of dL/dcs):
        //   rsb[s]  row j's pairs with columns i in the 64-row block s before J
        //   rs_in   row j's pairs with columns i in J (fp32 from unscaled operands)
        //   csu     column j's pairs with rows t in J, without the factor dt_j (likewise)
        //   cpx     column j's pairs with rows t after J, without dt_j
        // A pair inside J enters dL/dcs twice with opposite signs (row t and column i), so
        // both of its copies are formed to fp32 accuracy and cancel; pairs across a block
        // boundary are kept apart (xs) and summed once.
        float rsb[RJ > 0 ? RJ : 1];
#pragma unroll
        for (int s2 = 0; s2 < (RJ > 0 ? RJ : 1); ++s2) rsb[s2] = 0.f;
        float rs_in = 0.f, csu = 0.f;
        f32x4 dxa[PT];  // sum_t dy[t][p] U[t][j], first as the part after J without k2
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) dxa[pt] = f32x4{0.f, 0.f, 0.f, 0.f};

        // column strip after J: W[t][j] (rows scaled by their factors) into the
        // accumulators, and (C B^T) dy with C B^T scaled by the same factors
        {
            bf16x8 xk[PKB];
#pragma unroll
            for (int kb = 0; kb < PKB; ++kb) xk[kb] = scale8(xj[kb], dtj * k2);
#pragma unroll
            for (int k = RSP + 2; k < PAIRS; ++k) {
                const int rt = j0 + 32 * (k - RSP);  // chunk row of the block
                const int rho = rt + 64;              // its LDS row
                float4 f[2];
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    f[u] = rf4(s_rf, rt - 64 + 16 * u + 4 * g4);
                    f32x4 w = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < PKB; ++kb)
                        w = mfma16(ld_nat(rows_at(sXY, rho, PPR) + u * R16, pnp[kb]), xk[kb], w);
                    wacc[2 * k + u][0] = fmaf(f[u].x, w[0], wacc[2 * k + u][0]);
                    wacc[2 * k + u][1] = fmaf(f[u].y, w[1], wacc[2 * k + u][1]);
                    wacc[2 * k + u][2] = fmaf(f[u].z, w[2], wacc[2 * k + u][2]);
                    wacc[2 * k + u][3] = fmaf(f[u].w, w[3], wacc[2 * k + u][3]);
                    pin(wacc[2 * k + u]);
                }
                const uint2 g0 = scale4(gt[2 * k], f[0]), g1 = scale4(gt[2 * k + 1], f[1]);
                const bf16x8 gb = __builtin_bit_cast(bf16x8, make_uint4(g0.x, g0.y, g1.x, g1.y));
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    dxa[pt] = mfma16(ld_tr(rows_at(sXY, rho, PPR), ptp[pt], R16), gb, dxa[pt]);
                    pin(dxa[pt]);
                }
            }
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) dxa[pt] *= k2;
        }
        // cpx_j = x_j . (sum over t after J of U[t][j] dy_t)
        float cpx = 0.f;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            const uint2 xq = *reinterpret_cast<const uint2*>(rows_at(sXY, jb, PPR) + pac[pt]);
            cpx = fmaf(bf16_lo(xq.x), dxa[pt][0], cpx);
            cpx = fmaf(bf16_hi(xq.x), dxa[pt][1], cpx);
            cpx = fmaf(bf16_lo(xq.y), dxa[pt][2], cpx);
            cpx = fmaf(bf16_hi(xq.y), dxa[pt][3], cpx);
        }
        // row strip before J: W^T[i][j] with its rows scaled by their factors, its W.G sums
        // per 64-row block
        {
            bf16x8 yk[PKB];
#pragma unroll
            for (int kb = 0; kb < PKB; ++kb) yk[kb] = scale8(yj[kb], k1);
#pragma unroll
            for (int k = 0; k < RSO; ++k)
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    f32x4 w = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int kb = 0; kb < PKB; ++kb)
                        w = mfma16(ld_nat(rows_at(sXY, 32 * k, PPR) + u * R16, pnp[kb]), yk[kb], w);
                    const float4 f = rf4(s_rf, 32 * k + 16 * u + 4 * g4);
                    w[0] *= f.x;
                    w[1] *= f.y;
                    w[2] *= f.z;
                    w[3] *= f.w;
                    const uint2 gg = gt[2 * k + u];
                    wacc[2 * k + u] += w;
                    pin(wacc[2 * k + u]);
                    float& r_ = rsb[k >> 1];
                    r_ = fmaf(w[0], bf16_lo(gg.x), r_);
                    r_ = fmaf(w[1], bf16_hi(gg.x), r_);
                    r_ = fmaf(w[2], bf16_lo(gg.y), r_);
                    r_ = fmaf(w[3], bf16_hi(gg.y), r_);
                    pin(r_);
                }
        }
        // the four blocks inside J, element by element (exact decays, causal mask); x_j and
        // dy_j are read again here (through an opaque zero offset) rather than kept live
        {
            unsigned z = 0;
            asm volatile("" : "+v"(z));
#pragma unroll
            for (int kb = 0; kb < PKB; ++kb) {
                xj[kb] = ld_nat(rows_at(sXY, jb, PPR) + z, pnp[kb]);
                yj[kb] = ld_nat(rows_at(sXY, jb + 64, PPR) + z, pnp[kb]);
            }
        }
        // The role is specialised per column tile: against the wave's 16 columns (tile CW of
        // J), the 16-row tile t of J lies wholly before them (t < CW: every pair causal in
        // W^T, none in V), on the diagonal (t == CW: masked per element) or wholly after
        // (t > CW: the reverse).  Only the diagonal tile needs the mask, and the wholly
        // masked halves (their products, exps and sums) are not formed at all.
#pragma unroll
        for (int k = RSO; k < RSP + 2; ++k) {
            const bool isrs = k < RSP;
            const int kk = isrs ? k - RSO : k - RSP;                 // 32-row block of J
            const int rbase = isrs ? 32 * k : j0 + 32 * (k - RSP);  // chunk row of the block
            const int rho = isrs ? rbase : rbase + 64;              // its LDS row (unscaled)
            uint32_t ub[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int t = 2 * kk + u;  // 16-row tile of J
                if (isrs ? t > CW : t < CW) continue;  // wholly masked
                const bool diag = t == CW;
                f32x4 m = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kb = 0; kb < PKB; ++kb)
                    m = mfma16(ld_nat(rows_at(sXY, rho, PPR) + u * R16, pnp[kb]),
                               isrs ? yj[kb] : xj[kb], m);
                const int r0 = rbase + 16 * u + 4 * g4;  // chunk row of element q = 0
                const float4 csr = *reinterpret_cast<const float4*>(&s_cs[r0]);
                const float4 dtr = *reinterpret_cast<const float4*>(&s_dt[r0]);
                const uint2 gg = gt[2 * k + u];
                const float gq[4] = {bf16_lo(gg.x), bf16_hi(gg.x), bf16_lo(gg.y), bf16_hi(gg.y)};
                const float cr[4] = {csr.x, csr.y, csr.z, csr.w};
                const float dr[4] = {dtr.x, dtr.y, dtr.z, dtr.w};
                float uq[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    if (isrs) {  // W^T[i][j] = dt_i exp(cs_j - cs_i) M^T[i][j], i <= j
                        const float x_ = exp2_fast((csj - cr[q]) * kLog2e);
                        const float e = (!diag || jl - (r0 + q) >= 0) ? x_ : 0.f;
                        const float w = dr[q] * e * m[q];
                        wacc[2 * k + u][q] += w;
                        rs_in = fmaf(w, gq[q], rs_in);
                    } else {  // V[t][j] = exp(cs_t - cs_j) M[t][j], t >= j; W = dt_j V
                        const float x_ = exp2_fast((cr[q] - csj) * kLog2e);
                        const float e = (!diag || (r0 + q) - jl >= 0) ? x_ : 0.f;
                        const float v = e * m[q];
                        wacc[2 * k + u][q] = fmaf(dtj, v, wacc[2 * k + u][q]);
                        csu = fmaf(v, gq[q], csu);
                        uq[q] = e * gq[q];
                    }
                }
                pin(wacc[2 * k + u]);
                pin(rs_in);
                pin(csu);
                if (!isrs) {
                    ub[2 * u] = pack_bf16(uq[0], uq[1]);
                    ub[2 * u + 1] = pack_bf16(uq[2], uq[3]);
                }
            }
            // dx^T[p][j] += sum_t dy[t][p] U[t][j], unless both halves are masked
            if (!isrs && 2 * kk + 1 >= CW) {
                const bf16x8 bu =
                    __builtin_bit_cast(bf16x8, make_uint4(ub[0], ub[1], ub[2], ub[3]));
#pragma unroll
                for (int pt = 0; pt < PT; ++pt) {
                    dxa[pt] = mfma16(ld_tr(rows_at(sXY, rho, PPR), ptp[pt], R16), bu, dxa[pt]);
                    pin(dxa[pt]);
                }
            }
        }
        rs_in = colsum(rs_in);
        csu = colsum(csu);
        cpx = colsum(cpx);
#pragma unroll
        for (int s2 = 0; s2 < RJ; ++s2) rsb[s2] = colsum(rsb[s2]);

        // the state waves' (F B_j) tiles, ob, oc and <E, F> shares are in LDS
        lds_barrier();
        const uint2* xbf = reinterpret_cast<const uint2*>(smem + C_::X_BF) + (cw * PT) * 64 + ln;
        const float* xob = reinterpret_cast<const float*>(smem + C_::X_OB);
        const float ob = xob[16 * cw + l16], oc = xob[64 + 16 * cw + l16];
        if (g4 == 0 && vj) {
            const size_t item = (size_t)(b * H + h) * nC + c;
            const size_t cb = item * Q;
            direct[cb + jl] = (cpx + csu) + ob;
            dcs[cb + jl] = (rs_in - dtj * csu) + (oc - dtj * ob);
            float* xr = xs + item * NJ * Q + jl;
            xr[0] = dtj * cpx;
#pragma unroll
            for (int s2 = 0; s2 < RJ; ++s2) xr[(1 + s2) * Q] = rsb[s2];
        }
        if (vj) {  // (the partner lane group of pair_runs has the same j)
            const float dh = D[h];
            __bf16* dxr = dx + ((size_t)(b * T + t0 + jl) * H + h) * P;
            uint2 o[PT];
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                const uint2 yq = *reinterpret_cast<const uint2*>(rows_at(sXY, jb + 64, PPR) + pac[pt]);
                const uint2 bq = xbf[pt * 64];
                const float v0 = fmaf(dh, bf16_lo(yq.x), dtj * fmaf(fj, bf16_lo(bq.x), dxa[pt][0]));
                const float v1 = fmaf(dh, bf16_hi(yq.x), dtj * fmaf(fj, bf16_hi(bq.x), dxa[pt][1]));
                const float v2 = fmaf(dh, bf16_lo(yq.y), dtj * fmaf(fj, bf16_lo(bq.y), dxa[pt][2]));
                const float v3 = fmaf(dh, bf16_hi(yq.y), dtj * fmaf(fj, bf16_hi(bq.y), dxa[pt][3]));
                o[pt] = make_uint2(pack_bf16(v0, v1), pack_bf16(v2, v3));
            }
#pragma unroll
            for (int q = 0; q < PT / 2; ++q)  // 16-byte stores, p-tiles 2q and 2q + 1
                *reinterpret_cast<uint4*>(dxr + 16 * (2 * q + (g4 & 1)) + 8 * (g4 >> 1)) =
                    pair_runs(o[2 * q], o[2 * q + 1]);
        }
        // this block's shares of the chunk-end term (dt_j ob_j, and exp(cs_last) <E, F> on
        // the first block) and of dD (x_j . dy_j); at dstate 256 the carried-state kernel
        // writes both
        if constexpr (!C_::EXT) {
            float lt = (g4 == 0 && vj) ? dtj * ob : 0.f;
            if (j0 == 0 && ln == 0)
                lt = fmaf(exp2_fast(cs_last * kLog2e),
                          reinterpret_cast<const float*>(smem + C_::X_EF)[cw], lt);
            lt = wavesum(lt);
            if (lane == 0) shares[buf * 8 + 2 * cw] = lt;
        }
        lds_barrier();  // every state wave's copies of the next head have landed, and
                        // every wave is done with this head's buffer and exchange
    }
    dma_barrier();
    if (!C_::EXT && wave == 0 && lane == 0) {
        const float* sh = shares + ((hpg - 1) & 1) * 8;
        const size_t pi = ((size_t)(b * H + g * hpg + hpg - 1) * nC + c) * NJ + k_.rj;
        lt_part[pi] = (sh[0] + sh[2]) + (sh[4] + sh[6]);
        dd_part[pi] = (sh[1] + sh[3]) + (sh[5] + sh[7]);
    }
    issue_bc<Q, N, P>(Bm, Cm, b, g, t0, Lc, T, G, j0, true, k_.lds0, wave, lane);
    // hand W (bf16, as the B operand of the two products) to the state waves
    uint4* xw = reinterpret_cast<uint4*>(smem + C_::X_W) + (cw * PAIRS) * 64 + lane;
#pragma unroll
    for (int k = 0; k < PAIRS; ++k)
        xw[k * 64] = make_uint4(pack_bf16(wacc[2 * k][0], wacc[2 * k][1]),
                                pack_bf16(wacc[2 * k][2], wacc[2 * k][3]),
                                pack_bf16(wacc[2 * k + 1][0], wacc[2 * k + 1][1]),
                                pack_bf16(wacc[2 * k + 1][2], wacc[2 * k + 1][3]));
    dma_barrier();
    if constexpr (C_::EXT) {
        // the other halves of n: the state waves have read the previous half's rows
#pragma unroll 1
        for (int part = 1; part < C_::NHP; ++part) {
            lds_barrier();
            issue_bc<Q, N, P>(Bm, Cm, b, g, t0, Lc, T, G, j0, true, k_.lds0, wave, lane, part);
            dma_barrier();
        }
    }
}

// dB^T and dC^T tiles [n][j] (lane: n = 16 nt + 4 g4 .. +3 of row j) rounded to bf16 and
// stored as 16-byte runs of row j (pair_runs over n-tiles 2q, 2q + 1); row = the offset of
// element 0 of row j in dB and dC
template <int NTL>
__device__ __forceinline__ void store_dbdc(__bf16* dB, __bf16* dC, size_t row, const f32x4* dbacc,
                                           const f32x4* dcacc, int g4) {
#pragma unroll
    for (int q = 0; q < NTL / 2; ++q) {
        const size_t at = row + 16 * (2 * q + (g4 & 1)) + 8 * (g4 >> 1);
        auto pk = [](const f32x4& a) {
            return make_uint2(pack_bf16(a[0], a[1]), pack_bf16(a[2], a[3]));
        };
        *reinterpret_cast<uint4*>(dB + at) = pair_runs(pk(dbacc[2 * q]), pk(dbacc[2 * q + 1]));
        *reinterpret_cast<uint4*>(dC + at) = pair_runs(pk(dcacc[2 * q]), pk(dcacc[2 * q + 1]));
    }
}

// ------------------------------------------------------------------ state waves
// The off-diagonal terms through the carried states E and F: (F B_j) for dx and the
// per-row sums ob, oc (oc_j = exp(cs_j) dy_j . (E C_j) is taken as C_j . (the head's dC^T
// column j), so E C_j itself is never formed); the dB and dC accumulators; the two W
// products at the end.
template <int Q, int N, int P>
__device__ __forceinline__ void bwd_state_role(
    const BwdCtx& k_, unsigned char* smem, const __bf16* x, const __bf16* Bm, const __bf16* Cm,
    const float* dtc, const float* cs, const __bf16* entry, const __bf16* exitg, const __bf16* dy,
    __bf16* dB, __bf16* dC) {
    using C_ = BwdCfg<Q, N, P>;
    constexpr int PAIRS = C_::PAIRS, PPR = C_::PPR, NPR = C_::NPR;
    constexpr int NKB = C_::NKB, PKB = C_::PKB, NT = C_::NT, PT = C_::PT;
    const int b = k_.b, g = k_.g, c = k_.c, j0 = k_.j0, t0 = k_.t0, Lc = k_.Lc;
    const int hpg = k_.hpg, T = k_.T, H = k_.H, G = k_.G, nC = k_.nC;
    const int wave = k_.wave, cw = k_.cw, lane = k_.lane;
    const int rsp = (j0 + 64) / 32;  // row-strip blocks (rows 32 k), then column-strip blocks

    // B_j over n (natural slots, the operand of F B_j) and C_j[16 nt + 4 g4 .. +3] (the
    // lane's n of the dC^T tiles)
    bf16x8 bj[NKB];
    uint2 cq[NT];
    if constexpr (C_::SLICED) {  // the strip waves' C B^T slices, this wave's B_j, C_j parts
        constexpr int SPR = C_::SLN / 8, SKB = C_::SLN / 32, STL = C_::SLN / 16;
        const int l16 = lane & 15, g4 = lane >> 4;
        const int jl = j0 + 16 * cw + l16;
#pragma unroll
        for (int sl = 0; sl < C_::NSL; ++sl) {
            issue_bc<Q, N, P>(Bm, Cm, b, g, t0, Lc, T, G, j0, false, k_.lds0, wave, lane, sl);
            dma_barrier();
#pragma unroll
            for (int kb = 0; kb < SKB; ++kb) bj[sl * SKB + kb] = frag_nat(smem, jl, kb, g4, SPR);
#pragma unroll
            for (int nt = 0; nt < STL; ++nt)
                cq[sl * STL + nt] = *reinterpret_cast<const uint2*>(
                    smem + C_::BCB + swz_off(jl, 16 * nt + 4 * g4, SPR));
            lds_barrier();
        }
    } else {
        issue_bc<Q, N, P>(Bm, Cm, b, g, t0, Lc, T, G, j0, false, k_.lds0, wave, lane);
        dma_barrier();
        const int l16 = lane & 15, g4 = lane >> 4;
        const int jl = j0 + 16 * cw + l16;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) bj[kb] = frag_nat(smem, jl, kb, g4, NPR);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            cq[nt] = *reinterpret_cast<const uint2*>(smem + C_::BCB +
                                                     swz_off(jl, 16 * nt + 4 * g4, NPR));
        lds_barrier();
    }

    f32x4 dbacc[NT], dcacc[NT];  // dB^T, dC^T [n][j]
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) dbacc[nt] = dcacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    issue_item<Q, N, P>(x, dy, entry, exitg, cs, dtc, b, g * hpg, c, j0, Lc, T, H, nC, k_.lds0,
                        wave - 4, lane);
    dma_barrier();
#pragma unroll 1
    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        const int buf = hh & 1;
        // the other buffer (the previous head's) is free: the barrier at the end of that head
        if (hh + 1 < hpg)
            issue_item<Q, N, P>(x, dy, entry, exitg, cs, dtc, b, h + 1, c, j0, Lc, T, H, nC,
                                k_.lds0 + (buf ^ 1) * C_::ITEM, wave - 4, lane);
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int l16 = ln & 15, g4 = ln >> 4;
        const int jb = j0 + 16 * cw, jl = jb + l16;
        unsigned prl[PKB][2], pac[PT], ptn[NT], pnat[NKB];
#pragma unroll
        for (int kb = 0; kb < PKB; ++kb) {
            prl[kb][0] = lane_part(l16, 32 * kb + 4 * g4, PPR);
            prl[kb][1] = lane_part(l16, 32 * kb + 16 + 4 * g4, PPR);
        }
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) pac[pt] = lane_part(l16, 16 * pt + 4 * g4, PPR);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            ptn[nt] = lane_part(4 * g4 + (l16 >> 2), 16 * nt + 4 * (l16 & 3), NPR);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) pnat[kb] = lane_part(l16, 32 * kb + 8 * g4, NPR);
        constexpr unsigned N16 = 16u * NPR * 16u;  // 16 rows of E / F
        const unsigned char* sXY = smem + buf * C_::ITEM;
        const unsigned char* sE = sXY + C_::XYB;
        const unsigned char* sF = sE + C_::EB;
        const float* s_cs = reinterpret_cast<const float*>(sF + C_::EB);
        const float* s_dt = s_cs + Q;
        const float cs_last = s_cs[Q - 1];
        const float csj = s_cs[jl], dtj = s_dt[jl];
        const float ej = exp2_fast(csj * kLog2e), fj = exp2_fast((cs_last - csj) * kLog2e);

        // this head's dC^T[n][j] term, sum_p E[p][n] (exp(cs_j) dy_j[p]), and from it
        // oc_j = exp(cs_j) dy_j . (E C_j) = sum_n C_j[n] (that term)[n][j]
        float oc = 0.f;
        {
            f32x4 dch[NT];
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) dch[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < PKB; ++kb) {
                const bf16x8 ys8 =
                    scale8(ld_rl(rows_at(sXY, jb + 64, PPR), prl[kb][0], prl[kb][1]), ej);
#pragma unroll
                for (int nt = 0; nt < NT; ++nt)
                    dch[nt] = mfma16(ld_tr(rows_at(sE, 32 * kb, NPR), ptn[nt], N16), ys8, dch[nt]);
            }
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                oc = fmaf(bf16_lo(cq[nt].x), dch[nt][0], oc);
                oc = fmaf(bf16_hi(cq[nt].x), dch[nt][1], oc);
                oc = fmaf(bf16_lo(cq[nt].y), dch[nt][2], oc);
                oc = fmaf(bf16_hi(cq[nt].y), dch[nt][3], oc);
                dcacc[nt] += dch[nt];
            }
        }
        // (F B_j)[p] as [p][j] tiles; ob_j = exp(cs_last - cs_j) x_j . (F B_j)
        float ob = 0.f, dd = 0.f;
        uint2* xbf = reinterpret_cast<uint2*>(smem + C_::X_BF) + (cw * PT) * 64 + ln;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            f32x4 bfm = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
                bfm = mfma16(ld_nat(rows_at(sF, 16 * pt, NPR), pnat[kb]), bj[kb], bfm);
            const uint2 xq = *reinterpret_cast<const uint2*>(rows_at(sXY, jb, PPR) + pac[pt]);
            const uint2 yq = *reinterpret_cast<const uint2*>(rows_at(sXY, jb + 64, PPR) + pac[pt]);
            ob = fmaf(bf16_lo(xq.x), bfm[0], ob);
            ob = fmaf(bf16_hi(xq.x), bfm[1], ob);
            ob = fmaf(bf16_lo(xq.y), bfm[2], ob);
            ob = fmaf(bf16_hi(xq.y), bfm[3], ob);
            dd = fmaf(bf16_lo(xq.x), bf16_lo(yq.x), dd);
            dd = fmaf(bf16_hi(xq.x), bf16_hi(yq.x), dd);
            dd = fmaf(bf16_lo(xq.y), bf16_lo(yq.y), dd);
            dd = fmaf(bf16_hi(xq.y), bf16_hi(yq.y), dd);
            xbf[pt * 64] = make_uint2(pack_bf16(bfm[0], bfm[1]), pack_bf16(bfm[2], bfm[3]));
        }
        ob = colsum(ob) * fj;
        oc = colsum(oc);
        dd = wavesum(dd);  // this wave's 16 rows of x_j . dy_j (the dD share)
        if (ln == 0) reinterpret_cast<float*>(smem + C_::X_SH)[buf * 8 + 2 * cw + 1] = dd;
        float* xob = reinterpret_cast<float*>(smem + C_::X_OB);
        if (g4 == 0) {
            xob[16 * cw + l16] = ob;
            xob[64 + 16 * cw + l16] = oc;
        }
        if (j0 == 0) {  // <E, F>, a quarter per state wave
            float ef = 0.f;
            for (int m = cw * 64 + ln; m < P * NPR; m += 256)
                ef += dot8(*reinterpret_cast<const bf16x8*>(sE + 16 * m),
                           *reinterpret_cast<const bf16x8*>(sF + 16 * m));
            ef = wavesum(ef);
            if (ln == 0) reinterpret_cast<float*>(smem + C_::X_EF)[cw] = ef;
        }
        lds_barrier();  // hand-off to the strip waves
        // dB^T[n][j] += sum_p F[p][n] (dt_j exp(cs_last - cs_j) x_j[p])
#pragma unroll
        for (int kb = 0; kb < PKB; ++kb) {
            const bf16x8 xs8 =
                scale8(ld_rl(rows_at(sXY, jb, PPR), prl[kb][0], prl[kb][1]), dtj * fj);
#pragma unroll
            for (int nt = 0; nt < NT; ++nt)
                dbacc[nt] = mfma16(ld_tr(rows_at(sF, 32 * kb, NPR), ptn[nt], N16), xs8, dbacc[nt]);
        }
        // this wave's share of the next head's copies has landed; after the barrier every
        // share has (a wave's vmcnt covers only its own copies, so the barrier is needed)
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
    }
    dma_barrier();
    issue_bc<Q, N, P>(Bm, Cm, b, g, t0, Lc, T, G, j0, true, k_.lds0, wave, lane);
    dma_barrier();  // B / C rows and the strip waves' W are in LDS
    const int l16 = lane & 15, g4 = lane >> 4;
    const int jl = j0 + 16 * cw + l16;
    const uint4* xw = reinterpret_cast<const uint4*>(smem + C_::X_W) + (cw * PAIRS) * 64 + lane;
    unsigned ptn[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
        ptn[nt] = lane_part(4 * g4 + (l16 >> 2), 16 * nt + 4 * (l16 & 3), NPR);
    constexpr unsigned N16 = 16u * NPR * 16u;
    // dC^T[n][j] += sum_i B[i][n] W^T[i][j] over the row-strip blocks, then
    // dB^T[n][j] += sum_t C[t][n] W[t][j] over the column-strip blocks (two loops, so that
    // no accumulator is chosen per block at run time)
#pragma unroll 1
    for (int k = 0; k < rsp; ++k) {
        const bf16x8 w8 = __builtin_bit_cast(bf16x8, xw[k * 64]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            dcacc[nt] = mfma16(ld_tr(rows_at(smem, 32 * k, NPR), ptn[nt], N16), w8, dcacc[nt]);
    }
#pragma unroll 1
    for (int k = rsp; k < PAIRS; ++k) {
        const bf16x8 w8 = __builtin_bit_cast(bf16x8, xw[k * 64]);
        const int rho = j0 + 32 * (k - rsp) + 64;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
            dbacc[nt] = mfma16(ld_tr(rows_at(smem, rho, NPR), ptn[nt], N16), w8, dbacc[nt]);
    }
    if (jl < Lc)
        store_dbdc<NT>(dB, dC, ((size_t)(b * T + t0 + jl) * G + g) * N, dbacc, dcacc, g4);
}

// The state waves at dstate 256.  chunk_bwd_carried_kernel has already formed the terms
// through the carried states, so per head these waves hand its (F B_j) tile and ob, oc to
// the strip waves and issue the copies; after the loop they finish dB and dC from
// that kernel's head sums, one half of n at a time.  The barriers are bwd_state_role's.
template <int Q, int N, int P>
__device__ __forceinline__ void bwd_state_role_ext(
    const BwdCtx& k_, unsigned char* smem, const __bf16* x, const __bf16* Bm, const __bf16* Cm,
    const float* dtc, const float* cs, const __bf16* dy, const __bf16* xfb, const float* direct,
    const float* dcs, const float* dBs, const float* dCs, __bf16* dB, __bf16* dC) {
    using C_ = BwdCfg<Q, N, P>;
    constexpr int PAIRS = C_::PAIRS, PT = C_::PT, HN = C_::HN, HPR = HN / 8, HT = HN / 16;
    const int b = k_.b, g = k_.g, c = k_.c, j0 = k_.j0, t0 = k_.t0, Lc = k_.Lc;
    const int hpg = k_.hpg, T = k_.T, H = k_.H, G = k_.G, nC = k_.nC;
    const int wave = k_.wave, cw = k_.cw, lane = k_.lane;
    const int rsp = (j0 + 64) / 32;  // row-strip blocks (rows 32 k), then column-strip blocks
    const int l16 = lane & 15, g4 = lane >> 4;
    const int jl = j0 + 16 * cw + l16;
    const bool vj = jl < Lc;

#pragma unroll 1
    for (int sl = 0; sl < C_::NSL; ++sl) {  // the strip waves' C B^T slices
        issue_bc<Q, N, P>(Bm, Cm, b, g, t0, Lc, T, G, j0, false, k_.lds0, wave, lane, sl);
        dma_barrier();
        lds_barrier();
    }

    issue_item<Q, N, P>(x, dy, nullptr, nullptr, cs, dtc, b, g * hpg, c, j0, Lc, T, H, nC,
                        k_.lds0, wave - 4, lane);
    dma_barrier();
#pragma unroll 1
    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        const int buf = hh & 1;
        // (F B_j)[p] for p = 16 pt + 4 g4 .. + 3 of column j, and ob_j, oc_j
        const size_t cb = ((size_t)(b * H + h) * nC + c) * Q;
        const __bf16* fr = xfb + ((size_t)(b * T + t0 + jl) * H + h) * P + 4 * g4;
        uint2 fb[PT];
#pragma unroll
        for (int pt = 0; pt < PT; ++pt)
            fb[pt] = vj ? *reinterpret_cast<const uint2*>(fr + 16 * pt) : make_uint2(0u, 0u);
        const float ob = direct[cb + jl], oc = dcs[cb + jl];
        if (hh + 1 < hpg)
            issue_item<Q, N, P>(x, dy, nullptr, nullptr, cs, dtc, b, h + 1, c, j0, Lc, T, H, nC,
                                k_.lds0 + (buf ^ 1) * C_::ITEM, wave - 4, lane);
        uint2* xbf = reinterpret_cast<uint2*>(smem + C_::X_BF) + (cw * PT) * 64 + lane;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) xbf[pt * 64] = fb[pt];
        float* xob = reinterpret_cast<float*>(smem + C_::X_OB);
        if (g4 == 0) {
            xob[16 * cw + l16] = ob;
            xob[64 + 16 * cw + l16] = oc;
        }
        lds_barrier();  // hand-off to the strip waves
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        lds_barrier();
    }
    dma_barrier();
    issue_bc<Q, N, P>(Bm, Cm, b, g, t0, Lc, T, G, j0, true, k_.lds0, wave, lane);
    dma_barrier();  // B / C rows (first half of n) and the strip waves' W are in LDS
    const uint4* xw = reinterpret_cast<const uint4*>(smem + C_::X_W) + (cw * PAIRS) * 64 + lane;
    unsigned ptn[HT];
#pragma unroll
    for (int nt = 0; nt < HT; ++nt)
        ptn[nt] = lane_part(4 * g4 + (l16 >> 2), 16 * nt + 4 * (l16 & 3), HPR);
    constexpr unsigned N16 = 16u * HPR * 16u;
    // dB^T, dC^T [n][j] for n in one half, from the carried-state sums
    auto finish_half = [&](int part) {
        const size_t ro = ((size_t)(b * T + t0 + jl) * G + g) * N + part * HN + 4 * g4;
        f32x4 dbacc[HT], dcacc[HT];
#pragma unroll
        for (int nt = 0; nt < HT; ++nt) {
            dbacc[nt] = vj ? *reinterpret_cast<const f32x4*>(dBs + ro + 16 * nt)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
            dcacc[nt] = vj ? *reinterpret_cast<const f32x4*>(dCs + ro + 16 * nt)
                           : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll 1
        for (int k = 0; k < rsp; ++k) {
            const bf16x8 w8 = __builtin_bit_cast(bf16x8, xw[k * 64]);
#pragma unroll
            for (int nt = 0; nt < HT; ++nt)
                dcacc[nt] = mfma16(ld_tr(rows_at(smem, 32 * k, HPR), ptn[nt], N16), w8, dcacc[nt]);
        }
#pragma unroll 1
        for (int k = rsp; k < PAIRS; ++k) {
            const bf16x8 w8 = __builtin_bit_cast(bf16x8, xw[k * 64]);
            const int rho = j0 + 32 * (k - rsp) + 64;
#pragma unroll
            for (int nt = 0; nt < HT; ++nt)
                dbacc[nt] = mfma16(ld_tr(rows_at(smem, rho, HPR), ptn[nt], N16), w8, dbacc[nt]);
        }
        if (vj) store_dbdc<HT>(dB, dC, ro - 4 * g4, dbacc, dcacc, g4);
    };
    finish_half(0);
    // the other halves of n: every state wave has read the previous half's rows
#pragma unroll 1
    for (int part = 1; part < C_::NHP; ++part) {
        lds_barrier();
        issue_bc<Q, N, P>(Bm, Cm, b, g, t0, Lc, T, G, j0, true, k_.lds0, wave, lane, part);
        dma_barrier();
        finish_half(part);
    }
}

template <int Q, int N, int P>
__global__ __launch_bounds__(512) void chunk_bwd_mfma_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Bm, const __bf16* __restrict__ Cm,
    const float* __restrict__ dtc, const float* __restrict__ cs, const float* __restrict__ D,
    const __bf16* __restrict__ entry, const __bf16* __restrict__ exitg,
    const __bf16* __restrict__ dy, __bf16* __restrict__ dx, __bf16* __restrict__ dB,
    __bf16* __restrict__ dC, float* __restrict__ dcs, float* __restrict__ direct,
    float* __restrict__ xs, float* __restrict__ lt_part, float* __restrict__ dd_part,
    const __bf16* __restrict__ xfb, const float* __restrict__ dBs, const float* __restrict__ dCs,
    int T, int H, int G, int nC) {
    using C_ = BwdCfg<Q, N, P>;
    extern __shared__ __align__(16) unsigned char smem[];
    BwdCtx k_;
    // neighbouring row blocks and chunks on the same XCD (its L2 holds their shared data)
    const int nwg = gridDim.x, blk = blockIdx.x;
    const int wp = (nwg % 8 == 0) ? (blk & 7) * (nwg >> 3) + (blk >> 3) : blk;
    const int unit = wp / C_::NJ;
    k_.rj = wp % C_::NJ;
    k_.c = unit % nC;
    k_.g = (unit / nC) % G;
    k_.b = unit / (nC * G);
    k_.j0 = k_.rj * 64;
    k_.t0 = k_.c * Q;
    k_.Lc = min(Q, T - k_.t0);
    if (k_.j0 >= k_.Lc) return;  // no valid row
    k_.hpg = H / G;
    k_.T = T;
    k_.H = H;
    k_.G = G;
    k_.nC = nC;
    k_.wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    k_.cw = k_.wave & 3;
    k_.lane = threadIdx.x & 63;
    k_.lds0 = lds_addr(smem);
    // the two roles run the same sequence of barriers; the strip role is instantiated per
    // row block and column tile
    if (k_.wave < 4) {
        switch (k_.rj * 4 + k_.cw) {
#define SSD_STRIP(RJ, CW)                                                                    \
    case RJ * 4 + CW:                                                                        \
        if constexpr (RJ < C_::NJ)                                                           \
            bwd_strip_role<Q, N, P, RJ, CW>(k_, smem, x, Bm, Cm, dtc, cs, D, entry, exitg, dy, \
                                            dx, dcs, direct, xs, lt_part, dd_part);          \
        break;
#define SSD_STRIP4(RJ) SSD_STRIP(RJ, 0) SSD_STRIP(RJ, 1) SSD_STRIP(RJ, 2) SSD_STRIP(RJ, 3)
            SSD_STRIP4(0)
            SSD_STRIP4(1)
            SSD_STRIP4(2)
            SSD_STRIP4(3)
#undef SSD_STRIP4
#undef SSD_STRIP
        }
    } else {
        // both roles at the default wave priority: the strip waves' products are the longer
        // chain of every head, and raising the state waves (which issue the copies) above
        // them measured slower
        if constexpr (C_::EXT)
            bwd_state_role_ext<Q, N, P>(k_, smem, x, Bm, Cm, dtc, cs, dy, xfb, direct, dcs, dBs,
                                        dCs, dB, dC);
        else
            bwd_state_role<Q, N, P>(k_, smem, x, Bm, Cm, dtc, cs, entry, exitg, dy, dB, dC);
    }
}

// ------------------------------------------------------------------ carried states, dstate 256
// At dstate 256 the dB and dC accumulators of a 64-row block over all n (two 64 x 256 fp32
// tiles) do not fit beside the strip products, and E, F (64 x 256 bf16 each) do not fit
// double-buffered beside the x / dy rows.  The terms through the carried states therefore
// run first, in this kernel: one workgroup of eight waves per (batch, group, chunk, block J
// of 64 rows), looping over the heads of the group; wave w owns the 16 columns
// j = j0 + 16 (w % 4) + (0..15) and the half w / 4 of n.  Per head it writes
//   xfb[j][p] = (F B_j)[p] rounded to bf16 (the in-chunk kernel's operand for dx),
//   direct_j = ob_j = exp(cs_last - cs_j) x_j . (F B_j),  dcs_j = oc_j = exp(cs_j) dy_j . (E C_j)
//     (the in-chunk kernel reads both and completes them),
//   the block's chunk-end share (sum_j dt_j ob_j, plus its share of exp(cs_last) <E, F>) and
//     dD share (sum_j x_j . dy_j),
// and after the last head the head sums in fp32, where the in-chunk kernel's dB and dC
// accumulators start:
//   dBs^T[n][j] = sum_h dt_j exp(cs_last - cs_j) sum_p F[p][n] x_j[p]
//   dCs^T[n][j] = sum_h exp(cs_j) sum_p E[p][n] dy_j[p].
// The two halves of n meet in LDS once per head and share the finishing: each half hands
// the other the two p-tiles of its (F B_j) partial that the other finishes, and one of its
// two column sums; the lower half then finishes p-tiles 0-1 and ob, the upper half p-tiles
// 2-3 and oc.  E, F, cs and dt are copied into LDS straight from HBM, double-buffered over
// the heads, the next head's E and F copies spread through this head's products; x_j and
// dy_j (8 bytes per lane and p-tile) are loaded to registers one head ahead.
template <int Q>
struct CarryCfg {
    static constexpr int N = 256, P = 64, NPR = N / 8, NJ = Q / 64;
    static constexpr int PT = P / 16, HT = N / 32, HKB = N / 64;  // per half of n
    static constexpr unsigned EB = P * N * 2;   // E or F, [p][n]
    static constexpr unsigned FB = Q * 4;       // cs or dt
    static constexpr unsigned ITEM = 2 * EB + 2 * FB;
    static constexpr int NCI = P * NPR / 64 / 8;                // E (or F) copies per wave: 4
    static constexpr unsigned X_BM = 2 * ITEM;                 // (F B_j) tiles for the other half, f32x4 [8][2][64]
    static constexpr unsigned X_CS = X_BM + 8 * 2 * 64 * 16;   // column sums for the other half [2][64]
    static constexpr unsigned X_EF = X_CS + 2 * 64 * 4;        // <E, F> shares per wave [8]
    static constexpr unsigned X_SH = X_EF + 8 * 4;             // lt (lower), dd (upper) per wave [2][4][2]
    static constexpr unsigned LDS = X_SH + 16 * 4;
    static_assert(NCI * 8 * 64 == P * NPR && LDS <= 160 * 1024, "layout");
};

template <int Q>
__global__ __launch_bounds__(512) void chunk_bwd_carried_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Bm, const __bf16* __restrict__ Cm,
    const float* __restrict__ dtc, const float* __restrict__ cs,
    const __bf16* __restrict__ entry, const __bf16* __restrict__ exitg,
    const __bf16* __restrict__ dy, __bf16* __restrict__ xfb, float* __restrict__ dBs,
    float* __restrict__ dCs, float* __restrict__ dcs, float* __restrict__ direct,
    float* __restrict__ lt_part, float* __restrict__ dd_part, int T, int H, int G, int nC) {
    using K_ = CarryCfg<Q>;
    constexpr int N = K_::N, P = K_::P, NPR = K_::NPR, NJ = K_::NJ;
    constexpr int PT = K_::PT, HT = K_::HT, HKB = K_::HKB, NCI = K_::NCI;
    extern __shared__ __align__(16) unsigned char smem[];
    // the row blocks of a chunk, and neighbouring chunks, on the same XCD
    const int nwg = gridDim.x, blk = blockIdx.x;
    const int wp = (nwg % 8 == 0) ? (blk & 7) * (nwg >> 3) + (blk >> 3) : blk;
    const int unit = wp / NJ, rj = wp % NJ;
    const int c = unit % nC, g = (unit / nC) % G, b = unit / (nC * G);
    const int j0 = 64 * rj, t0 = c * Q;
    const int Lc = min(Q, T - t0);
    if (j0 >= Lc) return;  // no valid row
    const int nvb = (Lc + 63) / 64;  // row blocks with a valid row: they share <E, F>
    const int hpg = H / G;
    const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
    const int cw = wave & 3, nh = wave >> 2;
    const int lane = threadIdx.x & 63, l16 = lane & 15, g4 = lane >> 4;
    const int jl = j0 + 16 * cw + l16;
    const bool vj = jl < Lc;
    const uint32_t lds0 = lds_addr(smem);
    float* const shr = reinterpret_cast<float*>(smem + K_::X_SH);

    // one head's cs and dt into item buffer `buf` (waves 0 and 1)
    auto issue_steps = [&](int h, int buf) {
        const uint32_t base = lds0 + (unsigned)buf * K_::ITEM + 2 * K_::EB;
        const size_t cb = ((size_t)(b * H + h) * nC + c) * Q;
        if (wave == 0 && lane < Q / 4) dma16(raw_rsrc(cs + cb, K_::FB), base, lane * 16u);
        if (wave == 1 && lane < Q / 4) dma16(raw_rsrc(dtc + cb, K_::FB), base + K_::FB, lane * 16u);
    };
    // copy k (0 .. 2 NCI - 1) of this wave's share of one head's E (k < NCI) and F: 64
    // pieces of 16 bytes at LDS slots 64 (wave + 8 i) .., rows of 32 pieces swizzled as
    // issue_rows writes them
    auto issue_ef = [&](const u32x4& er, const u32x4& fr, int buf, int k) {
        const int i = k % NCI, inst = wave + 8 * i;
        const int m = inst * 64 + lane, r = m / NPR, sl = m % NPR;
        const uint32_t dst = lds0 + (unsigned)buf * K_::ITEM + (k < NCI ? 0u : K_::EB) +
                             (unsigned)inst * 1024u;
        dma16(k < NCI ? er : fr, dst, (unsigned)r * (N * 2u) + (unsigned)(sl ^ (r & 15)) * 16u);
    };
    auto ef_rsrc = [&](int h, u32x4& er, u32x4& fr) {
        const size_t so = ((size_t)(b * H + h) * nC + c) * P * N;
        er = raw_rsrc(entry + so, K_::EB);
        fr = raw_rsrc(exitg + so, K_::EB);
    };
    // x_j and dy_j at p = 16 pt + 4 g4 .. + 3 (zeros past the chunk's end)
    auto load_rows = [&](int h, uint2 (&xq)[PT], uint2 (&yq)[PT]) {
        const size_t o = ((size_t)(b * T + t0 + jl) * H + h) * P + 4 * g4;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            xq[pt] = vj ? *reinterpret_cast<const uint2*>(x + o + 16 * pt) : make_uint2(0u, 0u);
            yq[pt] = vj ? *reinterpret_cast<const uint2*>(dy + o + 16 * pt) : make_uint2(0u, 0u);
        }
    };

    // B_j, C_j over this wave's half of n (natural slots)
    bf16x8 bj[HKB], cj[HKB];
    {
        const size_t ro = ((size_t)(b * T + t0 + jl) * G + g) * N + 128 * nh + 8 * g4;
        const bf16x8 z = __builtin_bit_cast(bf16x8, make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
        for (int kb = 0; kb < HKB; ++kb) {
            bj[kb] = vj ? *reinterpret_cast<const bf16x8*>(Bm + ro + 32 * kb) : z;
            cj[kb] = vj ? *reinterpret_cast<const bf16x8*>(Cm + ro + 32 * kb) : z;
        }
    }
    // lane parts of the LDS offsets: transposed E / F reads for the [n][j] products, natural
    // reads for the [p][j] ones
    unsigned ptn[HT], pnat[HKB];
#pragma unroll
    for (int nt = 0; nt < HT; ++nt)
        ptn[nt] = lane_part(4 * g4 + (l16 >> 2), 128 * nh + 16 * nt + 4 * (l16 & 3), NPR);
#pragma unroll
    for (int kb = 0; kb < HKB; ++kb) pnat[kb] = lane_part(l16, 128 * nh + 32 * kb + 8 * g4, NPR);
    constexpr unsigned N16 = 16u * NPR * 16u;  // 16 rows of E / F

    f32x4 dbacc[HT], dcacc[HT];
#pragma unroll
    for (int nt = 0; nt < HT; ++nt) dbacc[nt] = dcacc[nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    uint2 xq[PT], yq[PT];
    load_rows(g * hpg, xq, yq);
    {
        u32x4 er, fr;
        ef_rsrc(g * hpg, er, fr);
#pragma unroll
        for (int k = 0; k < 2 * NCI; ++k) issue_ef(er, fr, 0, k);
        issue_steps(g * hpg, 0);
    }
#pragma unroll 1
    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        const int buf = hh & 1;
        const bool more = hh + 1 < hpg;
        // this head's copies and rows have landed (the wait is visible to the compiler, so it
        // adds none of its own for the rows); the previous head's exchange has been read
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
        dma_barrier();
        if (hh > 0 && wave == 0 && lane == 0) {
            const float* sh = shr + (buf ^ 1) * 8;
            const size_t pi = ((size_t)(b * H + h - 1) * nC + c) * NJ + rj;
            lt_part[pi] = (sh[0] + sh[2]) + (sh[4] + sh[6]);
            dd_part[pi] = (sh[1] + sh[3]) + (sh[5] + sh[7]);
        }
        uint2 xn[PT], yn[PT];
        u32x4 er, fr;
        if (more) {
            load_rows(h + 1, xn, yn);
            ef_rsrc(h + 1, er, fr);
            issue_steps(h + 1, buf ^ 1);
        }
        const unsigned char* sE = smem + buf * K_::ITEM;
        const unsigned char* sF = sE + K_::EB;
        const float* s_cs = reinterpret_cast<const float*>(sF + K_::EB);
        const float* s_dt = s_cs + Q;
        const float cs_last = s_cs[Q - 1];
        const float csj = vj ? s_cs[jl] : cs_last, dtj = vj ? s_dt[jl] : 0.f;
        const float ej = exp2_fast(csj * kLog2e), fj = exp2_fast((cs_last - csj) * kLog2e);

        // dC^T[n][j] += sum_p E[p][n] (exp(cs_j) dy_j[p]); dB^T[n][j] += sum_p F[p][n]
        // (dt_j exp(cs_last - cs_j) x_j[p]); operands over p in the relabelled slots.  The
        // next head's E and F copies are issued between the products, one per two tiles.
#pragma unroll
        for (int kb = 0; kb < P / 32; ++kb) {
            const bf16x8 y8 = __builtin_bit_cast(
                bf16x8, make_uint4(yq[2 * kb].x, yq[2 * kb].y, yq[2 * kb + 1].x, yq[2 * kb + 1].y));
            const bf16x8 x8 = __builtin_bit_cast(
                bf16x8, make_uint4(xq[2 * kb].x, xq[2 * kb].y, xq[2 * kb + 1].x, xq[2 * kb + 1].y));
            const bf16x8 ys8 = scale8(y8, ej), xs8 = scale8(x8, dtj * fj);
#pragma unroll
            for (int nt = 0; nt < HT; ++nt) {
                dcacc[nt] = mfma16(ld_tr(rows_at(sE, 32 * kb, NPR), ptn[nt], N16), ys8, dcacc[nt]);
                dbacc[nt] = mfma16(ld_tr(rows_at(sF, 32 * kb, NPR), ptn[nt], N16), xs8, dbacc[nt]);
                if ((nt & 1) && more) issue_ef(er, fr, buf ^ 1, kb * (HT / 2) + nt / 2);
            }
        }
        // (F B_j)[p] and (E C_j)[p] over this half of n, as [p][j] tiles; this half's parts
        // of ob, oc (before their decays) and, in the upper half, x_j . dy_j
        f32x4 bfm[PT];
        float obp = 0.f, ocp = 0.f, dd = 0.f;
#pragma unroll
        for (int pt = 0; pt < PT; ++pt) {
            f32x4 cem = f32x4{0.f, 0.f, 0.f, 0.f};
            bfm[pt] = cem;
#pragma unroll
            for (int kb = 0; kb < HKB; ++kb) {
                bfm[pt] = mfma16(ld_nat(rows_at(sF, 16 * pt, NPR), pnat[kb]), bj[kb], bfm[pt]);
                cem = mfma16(ld_nat(rows_at(sE, 16 * pt, NPR), pnat[kb]), cj[kb], cem);
            }
            const uint2 xv = xq[pt], yv = yq[pt];
            const float xs[4] = {bf16_lo(xv.x), bf16_hi(xv.x), bf16_lo(xv.y), bf16_hi(xv.y)};
            const float ys[4] = {bf16_lo(yv.x), bf16_hi(yv.x), bf16_lo(yv.y), bf16_hi(yv.y)};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                obp = fmaf(xs[q], bfm[pt][q], obp);
                ocp = fmaf(ys[q], cem[q], ocp);
                if (nh == 1) dd = fmaf(xs[q], ys[q], dd);
            }
        }
        obp = colsum(obp);
        ocp = colsum(ocp);
        // hand the other half its two p-tiles and column sum (the lower half finishes
        // p-tiles 0-1 and ob, the upper half p-tiles 2-3 and oc)
        f32x4* xbm = reinterpret_cast<f32x4*>(smem + K_::X_BM);
        float* xcs = reinterpret_cast<float*>(smem + K_::X_CS);
        float* xef = reinterpret_cast<float*>(smem + K_::X_EF);
        const int give = 2 * (1 - nh);
        xbm[(wave * 2) * 64 + lane] = bfm[give];
        xbm[(wave * 2 + 1) * 64 + lane] = bfm[give + 1];
        if (g4 == 0) xcs[64 * nh + 16 * cw + l16] = nh == 0 ? ocp : obp;
        // <E, F>: the valid row blocks of the chunk take a share each, an eighth per wave
        {
            float ef = 0.f;
            for (int m = rj * 512 + (int)threadIdx.x; m < P * NPR; m += 512 * nvb)
                ef += dot8(*reinterpret_cast<const bf16x8*>(sE + 16 * m),
                           *reinterpret_cast<const bf16x8*>(sF + 16 * m));
            ef = wavesum(ef);
            if (lane == 0) xef[wave] = ef;
        }
        lds_barrier();
        {
            const int other = wave ^ 4, own = 2 * nh;
            __bf16* xo = xfb + ((size_t)(b * T + t0 + jl) * H + h) * P;
            uint2 o[2];
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const f32x4 v = bfm[own + u] + xbm[(other * 2 + u) * 64 + lane];
                o[u] = make_uint2(pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3]));
            }
            // one 16-byte store per lane (p-tiles own, own + 1; the partner group has the same j)
            const uint4 pr = pair_runs(o[0], o[1]);
            if (vj)
                *reinterpret_cast<uint4*>(xo + 16 * (own + (g4 & 1)) + 8 * (g4 >> 1)) = pr;
            const size_t cb = ((size_t)(b * H + h) * nC + c) * Q;
            float share;
            if (nh == 0) {
                const float ob = (obp + xcs[64 + 16 * cw + l16]) * fj;
                if (g4 == 0 && vj) direct[cb + jl] = ob;
                share = (g4 == 0 && vj) ? dtj * ob : 0.f;
                if (lane == 0)
                    share = fmaf(exp2_fast(cs_last * kLog2e), xef[cw] + xef[cw + 4], share);
            } else {
                const float oc = (ocp + xcs[16 * cw + l16]) * ej;
                if (g4 == 0 && vj) dcs[cb + jl] = oc;
                share = dd;  // this wave's 16 rows of x_j . dy_j
            }
            share = wavesum(share);
            if (lane == 0) shr[buf * 8 + 2 * cw + nh] = share;
        }
        if (more) {
#pragma unroll
            for (int pt = 0; pt < PT; ++pt) {
                xq[pt] = xn[pt];
                yq[pt] = yn[pt];
            }
        }
    }
    dma_barrier();
    if (wave == 0 && lane == 0) {
        const float* sh = shr + ((hpg - 1) & 1) * 8;
        const size_t pi = ((size_t)(b * H + g * hpg + hpg - 1) * nC + c) * NJ + rj;
        lt_part[pi] = (sh[0] + sh[2]) + (sh[4] + sh[6]);
        dd_part[pi] = (sh[1] + sh[3]) + (sh[5] + sh[7]);
    }
    if (vj) {
        const size_t ro = ((size_t)(b * T + t0 + jl) * G + g) * N + 128 * nh + 4 * g4;
#pragma unroll
        for (int nt = 0; nt < HT; ++nt) {
            *reinterpret_cast<f32x4*>(dBs + ro + 16 * nt) = dbacc[nt];
            *reinterpret_cast<f32x4*>(dCs + ro + 16 * nt) = dcacc[nt];
        }
    }
}

template <int Q, int N, int P>
hipError_t launch_bwd_mfma_t(const Shape& s, const BwdArgs& a, hipStream_t st) {
    using C_ = BwdCfg<Q, N, P>;
    const unsigned blocks = (unsigned)((size_t)s.B * s.G * s.nC * C_::NJ);
    hipError_t e;
    if constexpr (C_::EXT) {
        if (!a.xfb || !a.dBs || !a.dCs) return hipErrorInvalidValue;
        const auto ck = chunk_bwd_carried_kernel<Q>;
        static DeviceSlots carried_set;
        e = allow_lds((const void*)ck, CarryCfg<Q>::LDS, carried_set);
        if (e != hipSuccess) return e;
        ck<<<blocks, 512, CarryCfg<Q>::LDS, st>>>(
            (const __bf16*)a.x, (const __bf16*)a.Bm, (const __bf16*)a.Cm, a.dtc, a.cs,
            (const __bf16*)a.entry, (const __bf16*)a.exitg, (const __bf16*)a.dy, (__bf16*)a.xfb,
            a.dBs, a.dCs, a.dcs, a.direct, a.lt_part, a.dd_part, s.T, s.H, s.G, s.nC);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const auto kern = chunk_bwd_mfma_kernel<Q, N, P>;
    static DeviceSlots attr_set;
    e = allow_lds((const void*)kern, C_::LDS, attr_set);
    if (e != hipSuccess) return e;
    kern<<<blocks, C_::NTH, C_::LDS, st>>>(
        (const __bf16*)a.x, (const __bf16*)a.Bm, (const __bf16*)a.Cm, a.dtc, a.cs, a.D,
        (const __bf16*)a.entry, (const __bf16*)a.exitg, (const __bf16*)a.dy, (__bf16*)a.dx,
        (__bf16*)a.dB, (__bf16*)a.dC, a.dcs, a.direct, a.xs, a.lt_part, a.dd_part,
        (const __bf16*)a.xfb, a.dBs, a.dCs, s.T, s.H, s.G, s.nC);
    return hipGetLastError();
}

using BwdFn = hipError_t (*)(const Shape&, const BwdArgs&, hipStream_t);

template <int Q>
BwdFn pick_bwd_q(const Shape& s) {
    if (s.P == 64) {
        switch (s.N) {
            case 64: return launch_bwd_mfma_t<Q, 64, 64>;
            case 128: return launch_bwd_mfma_t<Q, 128, 64>;
            case 256: return launch_bwd_mfma_t<Q, 256, 64>;
        }
    } else if (s.P == 32) {
        switch (s.N) {
            case 32: return launch_bwd_mfma_t<Q, 32, 32>;
            case 64: return launch_bwd_mfma_t<Q, 64, 32>;
            case 128: return launch_bwd_mfma_t<Q, 128, 32>;
        }
    }
    return nullptr;
}

BwdFn pick_bwd(const Shape& s) {
    // buffer resources address one chunk of x / dy and of B / C with 32-bit byte offsets
    if ((size_t)s.Q * s.H * s.P * 2 >= ((size_t)1 << 31) ||
        (size_t)s.Q * s.G * s.N * 2 >= ((size_t)1 << 31))
        return nullptr;
    switch (s.Q) {
        case 64: return pick_bwd_q<64>(s);
        case 128: return pick_bwd_q<128>(s);
        case 256: return pick_bwd_q<256>(s);
    }
    return nullptr;
}

}  // namespace

bool chunk_bwd_mfma_supported(const Shape& s) { return pick_bwd(s) != nullptr; }
bool chunk_bwd_mfma_carried(const Shape& s) { return s.N > 128 && pick_bwd(s) != nullptr; }
int chunk_bwd_mfma_rows() { return 64; }

hipError_t launch_chunk_bwd_mfma(const Shape& s, const BwdArgs& a, hipStream_t st) {
    BwdFn f = pick_bwd(s);
    if (!f) return hipErrorInvalidValue;
    if ((size_t)s.B * s.nC == 0) return hipSuccess;
    return f(s, a, st);
}

}  // namespace ssd
