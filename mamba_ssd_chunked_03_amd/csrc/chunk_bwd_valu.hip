// chunk_bwd_valu.hip -- the backward pass inside each chunk, and the per-step and
// per-head parameter gradients, in plain fp32 vector arithmetic (any supported size,
// fp32 or bf16 inputs).
//
// The forward is the block decomposition of the SSD layer (structured summary of arXiv
// 2405.21060, section "The Block-Decomposition SSD Algorithm"): inside chunk c, with cs the
// chunk-local inclusive prefix sums of dt*A and E the state entering the chunk,
//     y_j = sum_{i<=j} (C_j.B_i) exp(cs_j - cs_i) dt_i x_i + exp(cs_j) E^T C_j + D x_j
//     S_c = sum_i exp(cs_last - cs_i) dt_i B_i x_i^T,    E_next = exp(cs_last) E + S_c.
// Its gradient, given dy and F = dL/dE_next (the carried gradient of the chunk's end state,
// from the reverse inter-chunk pass), with M[t][i] = dy_t . x_i and G[t][i] = C_t . B_i:
//     dx_j  = D dy_j + dt_j [ sum_{t>=j} exp(cs_t - cs_j) G[t][j] dy_t
//                            + exp(cs_last - cs_j) F^T B_j ]
//     dC_j += sum_{i<=j} dt_i exp(cs_j - cs_i) M[j][i] B_i + exp(cs_j) E dy_j
//     dB_j += dt_j [ sum_{t>=j} exp(cs_t - cs_j) M[t][j] C_t + exp(cs_last - cs_j) F x_j ]
// summed over the heads of the group for dB and dC.  The step sizes enter through dt_j
// directly and through every cs_k with k >= j (cs_k = A sum_{m<=k} dt_m), so
//     ddt_j = direct_j + A R_j,   R_j = sum_{k>=j} dL/dcs_k,   dA = sum_j dt_j R_j,
// where direct_j = B_j . (dL/dS_j) x_j is the explicit derivative and, per head,
//     dL/dcs_k = C_k . dC_k(head) - B_k . dB_k(head)   (+ <E_next, F> at the chunk's end)
// because cs_k enters every term as exp(+cs_k) where C_k reads and exp(-cs_k) where B_k
// writes.  These identities follow from differentiating the decomposition term by term;
// the fp64 oracle differentiates the token recurrence instead, and the two agree.
//
// Kernels
//   chunk_bwd_valu_kernel: one workgroup per (b, g, chunk, 16-row tile J), looping over
//     the heads of the group so that dB and dC are summed in registers with no atomics.
//     Per head it forms the row strip W[j][i] (i <= j) and the column strip V[t][j]
//     (t >= j) of the decayed M for j in J, the dx weights U[t][j] = exp(cs_t - cs_j) G[t][j],
//     and from them dx (written per head), the dB/dC contributions and dL/dcs, direct.
//   bwd_ddt_kernel: one wave per (b, h, chunk), a workgroup per 16 heads of a (b, chunk):
//     the suffix sums R, ddt (written as runs of consecutive heads) and dA's share.
//   bwd_param_kernel: one workgroup per head: dA and dD summed over batch and chunks in a
//     fixed order (results do not depend on scheduling).
#include "ssd_internal.h"

namespace ssd {
namespace {

constexpr int kThreads = 256;
constexpr int kRows = 16;   // rows of a tile
constexpr int kMaxNQ = 16;  // N / 16 for N <= 256

template <typename Tin>
__device__ __forceinline__ float ld(const Tin* p, size_t i) { return to_f32(p[i]); }

// Cross-lane sums and scans in VALU operations (DPP row permutations and the gfx950 lane
// swaps) rather than LDS-routed shuffles; a row is 16 aligned lanes.
// v moved by the DPP control CTRL; 0 in lanes without a source
template <int CTRL>
__device__ __forceinline__ float dpp0(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_value(float v, int lane) {  // v of one lane, uniform
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}
// sum over the lane's row (every lane of it gets the total): pairs (quad_perm [1,0,3,2]),
// quad halves ([2,3,0,1]), the two quads of each half row (row_half_mirror), the halves
// (row_mirror)
__device__ __forceinline__ float sum16(float v) {
    v += dpp0<0xB1>(v);
    v += dpp0<0x4E>(v);
    v += dpp0<0x141>(v);
    return v + dpp0<0x140>(v);
}
// v plus v of the same lane in the other row of its pair (rows 0-1, 2-3): v_permlane16_swap
// of v with itself gives the even row's v and the odd row's v in every lane of both
__device__ __forceinline__ float add_row_pair(float v) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
// v plus v of the same lane in the other half of the wave (v_permlane32_swap likewise)
__device__ __forceinline__ float add_half(float v) {
    const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float sum64(float v) { return add_half(add_row_pair(sum16(v))); }
// inclusive suffix sum inside the lane's row (row_shl:1, 2, 4, 8)
__device__ __forceinline__ float row_suffix(float v) {
    v += dpp0<0x101>(v);
    v += dpp0<0x102>(v);
    v += dpp0<0x104>(v);
    return v + dpp0<0x108>(v);
}
// inclusive suffix sum inside the lane's block of LPB lanes (16, 32 or 64)
template <int LPB>
__device__ __forceinline__ float block_suffix(float v, int lane) {
    v = row_suffix(v);
    if constexpr (LPB == 16) {
        return v;
    } else {
        // the rows' totals sit in their first lanes
        const float t1 = lane_value(v, 16), t2 = lane_value(v, 32), t3 = lane_value(v, 48);
        const int row = lane >> 4;
        if constexpr (LPB == 32) return v + (row == 0 ? t1 : row == 2 ? t3 : 0.f);
        else return v + (row == 0 ? t1 + (t2 + t3) : row == 1 ? t2 + t3 : row == 2 ? t3 : 0.f);
    }
}
// sum over the lane's block of LPB lanes
template <int LPB>
__device__ __forceinline__ float block_sum(float v) {
    v = sum16(v);
    if constexpr (LPB >= 32) v = add_row_pair(v);
    if constexpr (LPB == 64) v = add_half(v);
    return v;
}
// sum of v over the lanes of the blocks (LPB lanes each) after the lane's block
template <int LPB>
__device__ __forceinline__ float later_blocks(float v, int lane) {
    if constexpr (LPB == 64) {
        return 0.f;
    } else {
        const float s = sum16(v);
        const float r1 = lane_value(s, 16), r2 = lane_value(s, 32), r3 = lane_value(s, 48);
        const int row = lane >> 4;
        if constexpr (LPB == 32) return row < 2 ? r2 + r3 : 0.f;
        else return row == 0 ? r1 + (r2 + r3) : row == 1 ? r2 + r3 : row == 2 ? r3 : 0.f;
    }
}

template <typename Tin>
__global__ __launch_bounds__(kThreads) void chunk_bwd_valu_kernel(
    const Tin* __restrict__ x, const Tin* __restrict__ Bm, const Tin* __restrict__ Cm,
    const float* __restrict__ dtc, const float* __restrict__ cs, const float* __restrict__ D,
    const Tin* __restrict__ entry, const Tin* __restrict__ exitg, const Tin* __restrict__ dy,
    Tin* __restrict__ dx, Tin* __restrict__ dB, Tin* __restrict__ dC, float* __restrict__ dcs,
    float* __restrict__ direct, float* __restrict__ lt_part, float* __restrict__ dd_part,
    int T, int H, int G, int P, int N, int Q, int nC) {
    extern __shared__ float sm[];
    float* Grow = sm;               // [16][Q]  G[j0 + r][i]
    float* Gcol = Grow + kRows * Q; // [Q][16]  G[t][j0 + r]
    float* Wrow = Gcol + kRows * Q; // [16][Q]  dt_i exp(cs_j - cs_i) M[j][i], i <= j
    float* Vcol = Wrow + kRows * Q; // [Q][16]  exp(cs_t - cs_j) M[t][j], t >= j
    float* Ucol = Vcol + kRows * Q; // [Q][16]  exp(cs_t - cs_j) G[t][j], t >= j
    float* xJ = Ucol + kRows * Q;   // [16][P]
    float* dyJ = xJ + kRows * P;    // [16][P]
    float* red = dyJ + kRows * P;   // [2][4] wave partials

    const int ntiles = Q / kRows;
    int k = blockIdx.x;
    const int rt = k % ntiles; k /= ntiles;
    const int c = k % nC; k /= nC;
    const int g = k % G;
    const int b = k / G;
    const int j0 = rt * kRows, t0 = c * Q;
    if (t0 + j0 >= T) return;  // no valid row: nothing of this tile is read back
    const int Lc = min(Q, T - t0);  // valid rows of the chunk
    const int iend = j0 + kRows;
    const int hpg = H / G;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ro = tid / 16, l16 = tid % 16;  // owned row of the tile and lane in its group
    const int jo = j0 + ro;
    const bool vrow = jo < Lc;
    const int NQ = N / 16;

    auto brow = [&](int i) { return Bm + ((size_t)(b * T + t0 + i) * G + g) * N; };
    auto crow = [&](int i) { return Cm + ((size_t)(b * T + t0 + i) * G + g) * N; };

    // the group's C_j . B_i strips, shared by every head
    for (int e = tid; e < kRows * iend; e += kThreads) {
        const int i = e / kRows, r = e % kRows;
        float v = 0.f;
        if (j0 + r < Lc && i < Lc) {
            const Tin* cr = crow(j0 + r);
            const Tin* br = brow(i);
            for (int n = 0; n < N; ++n) v = fmaf(ld(cr, n), ld(br, n), v);
        }
        Grow[r * Q + i] = v;
    }
    for (int e = tid; e < (Q - j0) * kRows; e += kThreads) {
        const int t = j0 + e / kRows, r = e % kRows;
        float v = 0.f;
        if (t < Lc && j0 + r < Lc) {
            const Tin* cr = crow(t);
            const Tin* br = brow(j0 + r);
            for (int n = 0; n < N; ++n) v = fmaf(ld(cr, n), ld(br, n), v);
        }
        Gcol[t * kRows + r] = v;
    }
    float accB[kMaxNQ], accC[kMaxNQ], bj[kMaxNQ], cj[kMaxNQ];
#pragma unroll
    for (int q = 0; q < kMaxNQ; ++q) {
        accB[q] = accC[q] = 0.f;
        const int n = l16 + 16 * q;
        bj[q] = (q < NQ && vrow) ? ld(brow(jo), n) : 0.f;
        cj[q] = (q < NQ && vrow) ? ld(crow(jo), n) : 0.f;
    }
    __syncthreads();

    for (int hh = 0; hh < hpg; ++hh) {
        const int h = g * hpg + hh;
        const size_t cb = ((size_t)(b * H + h) * nC + c) * Q;
        const float* csh = cs + cb;
        const float* dth = dtc + cb;
        const float cs_last = csh[Q - 1];
        auto xrow = [&](int i) { return x + ((size_t)(b * T + t0 + i) * H + h) * P; };
        auto dyrow = [&](int i) { return dy + ((size_t)(b * T + t0 + i) * H + h) * P; };

        for (int e = tid; e < kRows * P; e += kThreads) {
            const int r = e / P, p = e % P;
            const bool v = j0 + r < Lc;
            xJ[e] = v ? ld(xrow(j0 + r), p) : 0.f;
            dyJ[e] = v ? ld(dyrow(j0 + r), p) : 0.f;
        }
        __syncthreads();
        for (int e = tid; e < kRows * iend; e += kThreads) {
            const int i = e / kRows, r = e % kRows;
            const int j = j0 + r;
            float w = 0.f;
            if (i <= j && j < Lc) {
                const Tin* xi = xrow(i);
                float m = 0.f;
                for (int p = 0; p < P; ++p) m = fmaf(dyJ[r * P + p], ld(xi, p), m);
                w = dth[i] * expf(csh[j] - csh[i]) * m;
            }
            Wrow[r * Q + i] = w;
        }
        for (int e = tid; e < (Q - j0) * kRows; e += kThreads) {
            const int t = j0 + e / kRows, r = e % kRows;
            const int j = j0 + r;
            float v = 0.f, u = 0.f;
            if (t >= j && t < Lc) {
                const Tin* dyt = dyrow(t);
                float m = 0.f;
                for (int p = 0; p < P; ++p) m = fmaf(ld(dyt, p), xJ[r * P + p], m);
                const float dec = expf(csh[t] - csh[j]);
                v = dec * m;
                u = dec * Gcol[t * kRows + r];
            }
            Vcol[t * kRows + r] = v;
            Ucol[t * kRows + r] = u;
        }
        __syncthreads();

        const float cs_j = vrow ? csh[jo] : cs_last;
        const float dtj = vrow ? dth[jo] : 0.f;
        const float e_j = expf(cs_j), f_j = expf(cs_last - cs_j);
        float rs = 0.f, ccol = 0.f, oc = 0.f, ob = 0.f;
        for (int i = l16; i < iend; i += 16) rs = fmaf(Wrow[ro * Q + i], Grow[ro * Q + i], rs);
        for (int t = j0 + l16; t < Q; t += 16)
            ccol = fmaf(Vcol[t * kRows + ro], Gcol[t * kRows + ro], ccol);
        const Tin* E = entry + ((size_t)(b * H + h) * nC + c) * P * N;  // [P][N]
        const Tin* F = exitg + ((size_t)(b * H + h) * nC + c) * P * N;  // [P][N]
        const int imax = min(iend, Lc);
#pragma unroll
        for (int q = 0; q < kMaxNQ; ++q) {
            if (q >= NQ) break;
            const int n = l16 + 16 * q;
            float sC = 0.f, sB = 0.f, edy = 0.f, fx = 0.f;
            for (int i = 0; i < imax; ++i) sC = fmaf(Wrow[ro * Q + i], ld(brow(i), n), sC);
            for (int t = j0; t < Lc; ++t) sB = fmaf(Vcol[t * kRows + ro], ld(crow(t), n), sB);
            for (int p = 0; p < P; ++p) {
                edy = fmaf(ld(E, (size_t)p * N + n), dyJ[ro * P + p], edy);
                fx = fmaf(ld(F, (size_t)p * N + n), xJ[ro * P + p], fx);
            }
            accC[q] += sC + e_j * edy;
            accB[q] += dtj * (sB + f_j * fx);
            oc = fmaf(cj[q], e_j * edy, oc);
            ob = fmaf(bj[q], f_j * fx, ob);
        }
        rs = sum16(rs);
        ccol = sum16(ccol);
        oc = sum16(oc);
        ob = sum16(ob);

        const float dh = D[h];
        for (int p = l16; p < P; p += 16) {
            float sx = 0.f, bf = 0.f;
            for (int t = jo; t < Lc; ++t) sx = fmaf(Ucol[t * kRows + ro], ld(dyrow(t), p), sx);
            if (vrow) {
                const Tin* bjr = brow(jo);
                for (int n = 0; n < N; ++n) bf = fmaf(ld(bjr, n), ld(F, (size_t)p * N + n), bf);
                dx[((size_t)(b * T + t0 + jo) * H + h) * P + p] =
                    from_f32<Tin>(dh * dyJ[ro * P + p] + dtj * (sx + f_j * bf));
            }
        }
        if (l16 == 0 && vrow) {
            direct[cb + jo] = ccol + ob;
            dcs[cb + jo] = rs + oc - dtj * (ccol + ob);
        }

        // this tile's shares of the chunk-end term and of dD
        float lt = (l16 == 0 && vrow) ? dtj * ob : 0.f;
        if (rt == 0) {
            float ef = 0.f;
            for (int e = tid; e < N * P; e += kThreads) ef = fmaf(ld(E, e), ld(F, e), ef);
            lt = fmaf(expf(cs_last), ef, lt);
        }
        float dd = 0.f;
        for (int p = l16; p < P; p += 16) dd = fmaf(xJ[ro * P + p], dyJ[ro * P + p], dd);
        lt = sum64(lt);
        dd = sum64(dd);
        if (lane == 0) {
            red[wave] = lt;
            red[4 + wave] = dd;
        }
        __syncthreads();
        if (tid == 0) {
            const size_t pi = ((size_t)(b * H + h) * nC + c) * ntiles + rt;
            lt_part[pi] = (red[0] + red[1]) + (red[2] + red[3]);
            dd_part[pi] = (red[4] + red[5]) + (red[6] + red[7]);
        }
        // next head overwrites the strips and the staged rows
        __syncthreads();
    }
    if (vrow) {
        Tin* db = dB + ((size_t)(b * T + t0 + jo) * G + g) * N;
        Tin* dc = dC + ((size_t)(b * T + t0 + jo) * G + g) * N;
#pragma unroll
        for (int q = 0; q < kMaxNQ; ++q) {
            if (q >= NQ) break;
            db[l16 + 16 * q] = from_f32<Tin>(accB[q]);
            dc[l16 + 16 * q] = from_f32<Tin>(accC[q]);
        }
    }
}

// One wave per (b, h, chunk).  R_j = sum_{k >= j} dL/dcs_k within the chunk, plus the
// chunk-end term (summed from the row tiles' shares); ddt_j = direct_j + A R_j and this
// chunk's share of dA, sum_j dt_j R_j.  rows: rows per tile of the kernel that wrote the
// shares.
// R_j = sum_{k >= j} dL/dcs_k is a sum over the chunk's pairs (t, i) with i < j <= t of
// W[t][i] G[t][i] (each pair enters dL/dcs_t with + and dL/dcs_i with -), plus the terms
// through the carried states.  dcs holds what a plain suffix sum takes: the state terms, and
// pair terms whose two copies are formed to fp32 accuracy.  With xs (64-row blocks Jb), the
// pairs across a block boundary arrive apart and are summed once each:
//   R_j += sum_{k in Jb, k >= j} (rp_k - cp_k) + CP[Jb] + K[Jb],
// rp_k = sum_{s < blk(k)} xs[1 + s][k]   (row k with the columns of earlier blocks)
// cp_k = xs[0][k], CP[Jb] = sum_{k in Jb} cp_k   (column k with the rows of later blocks)
// K[Jb] = sum_{s < Jb} sum_{k >= 64 (Jb + 1)} xs[1 + s][k]   (later rows, earlier columns)
// L consecutive floats (L = 1, 2, 4) at a 4L-byte aligned address
template <int L>
__device__ __forceinline__ void load_run(const float* p, float (&o)[4]) {
    if constexpr (L == 4) {
        const float4 u = *reinterpret_cast<const float4*>(p);
        o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
    } else if constexpr (L == 2) {
        const float2 u = *reinterpret_cast<const float2*>(p);
        o[0] = u.x; o[1] = u.y; o[2] = o[3] = 0.f;
    } else {
        o[0] = p[0]; o[1] = o[2] = o[3] = 0.f;
    }
}

constexpr int kDdtHeads = 16;  // heads per workgroup of the ddt kernel, one wave each
constexpr int kDdtThreads = 64 * kDdtHeads;

// One workgroup per (b, chunk, block of 16 heads); a wave per head, a lane L = Q/64
// consecutive positions (each wave's work is a chain of dependent cross-lane scans, in DPP
// and lane-swap operations: many waves hide it).  The ddt rows of the block's heads are
// staged in LDS and written as 64-byte runs of consecutive heads ([B][T][H] is head-minor).
template <int Q>
__global__ __launch_bounds__(kDdtThreads) void bwd_ddt_kernel(
    const float* __restrict__ dcs, const float* __restrict__ direct,
    const float* __restrict__ xs, const float* __restrict__ lt_part,
    const float* __restrict__ dtc, const float* __restrict__ A, float* __restrict__ ddt,
    float* __restrict__ dA_part, int T, int H, int nC, int rows) {
    constexpr int L = Q / 64;           // positions per lane, consecutive
    constexpr int NJ = Q / 64, lpb = 64 / L;  // 64-row blocks, lanes per block
    __shared__ float tile[Q][kDdtHeads + 1];
    const int hblocks = (H + kDdtHeads - 1) / kDdtHeads;
    const int hb = blockIdx.x % hblocks;
    const int bc = blockIdx.x / hblocks;
    const int c = bc % nC, b = bc / nC;
    const int h0 = hb * kDdtHeads, nh = min(kDdtHeads, H - h0);
    const int Lc = min(Q, T - c * Q);
    const int ntiles = Q / rows;
    const int nvalid = (Lc + rows - 1) / rows;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int k0 = lane * L;
    const int blk = lane / lpb;
    for (int hh = wave; hh < nh; hh += kDdtThreads / 64) {
        const int h = h0 + hh;
        const size_t item = ((size_t)b * H + h) * nC + c;
        const size_t cb = item * Q;
        float lt = 0.f;
        for (int k = 0; k < nvalid; ++k) lt += lt_part[item * ntiles + k];
        // positions past the chunk's end hold no results: zero them
        auto valid = [&](int m) { return m < L && k0 + m < Lc; };
        float v[4], dv[4], tv[4];
        load_run<L>(dcs + cb + k0, v);
        load_run<L>(direct + cb + k0, dv);
        load_run<L>(dtc + cb + k0, tv);
        float seg = 0.f;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            if (!valid(m)) v[m] = 0.f;
            seg += v[m];
        }
        // inclusive suffix sum of the lanes' segment sums
        const float suf = block_suffix<64>(seg, lane);
        float r = (suf - seg) + lt;
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (xs) {
            const float* xr = xs + item * NJ * Q;
            float pl[NJ][4];  // plane 0: cp; plane 1 + s: row sums over block s
#pragma unroll
            for (int s2 = 0; s2 < NJ; ++s2) load_run<L>(xr + (size_t)s2 * Q + k0, pl[s2]);
            float segb = 0.f, segcp = 0.f;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                if (!valid(m)) continue;
                float rp = 0.f;
#pragma unroll
                for (int s2 = 0; s2 + 1 < NJ; ++s2)
                    if (s2 < blk) rp += pl[1 + s2][m];
                bv[m] = rp - pl[0][m];
                segb += bv[m];
                segcp += pl[0][m];
            }
            // suffix of rp - cp within the block, and the block's total of cp
            const float sufb = block_suffix<lpb>(segb, lane);
            segcp = block_sum<lpb>(segcp);
            // K: for each plane s, the suffix over the lanes after this block
            float ks = 0.f;
#pragma unroll
            for (int s2 = 0; s2 + 1 < NJ; ++s2) {
                float ps = 0.f;
                if (blk > s2) {
#pragma unroll
                    for (int m = 0; m < 4; ++m)
                        if (valid(m)) ps += pl[1 + s2][m];
                }
                const float after = later_blocks<lpb>(ps, lane);  // the later blocks
                if (s2 < blk) ks += after;
            }
            r += (sufb - segb) + segcp + ks;
        }
        const float Ah = A[h];
        float da = 0.f;
#pragma unroll
        for (int m = 3; m >= 0; --m) {
            if (m >= L) continue;
            r += v[m] + bv[m];
            if (valid(m)) {
                tile[k0 + m][hh] = dv[m] + Ah * r;
                da = fmaf(tv[m], r, da);
            }
        }
        da = sum64(da);
        if (lane == 0) dA_part[item] = da;
    }
    __syncthreads();
    // rows of nh consecutive heads
    for (int e = threadIdx.x; e < Lc * nh; e += kDdtThreads) {
        const int j = e / nh, hh = e % nh;
        ddt[((size_t)b * T + c * Q + j) * H + h0 + hh] = tile[j][hh];
    }
}

// One workgroup per head: dA[h] and dD[h] summed over every (b, chunk) in a fixed order.
__global__ __launch_bounds__(kThreads) void bwd_param_kernel(
    const float* __restrict__ dA_part, const float* __restrict__ dd_part, float* __restrict__ dA,
    float* __restrict__ dD, int Bsz, int T, int H, int Q, int nC, int rows) {
    __shared__ float red[2][kThreads];
    const int h = blockIdx.x;
    const int ntiles = Q / rows;
    const int items = Bsz * nC;
    float sa = 0.f, sd = 0.f;
    for (int k = threadIdx.x; k < items; k += kThreads) {
        const int b = k / nC, c = k % nC;
        const size_t item = (size_t)(b * H + h) * nC + c;
        sa += dA_part[item];
        const int Lc = min(Q, T - c * Q);
        const int nvalid = (Lc + rows - 1) / rows;
        for (int t = 0; t < nvalid; ++t) sd += dd_part[item * ntiles + t];
    }
    red[0][threadIdx.x] = sa;
    red[1][threadIdx.x] = sd;
    __syncthreads();
    for (int o = kThreads / 2; o > 0; o >>= 1) {
        if (threadIdx.x < o) {
            red[0][threadIdx.x] += red[0][threadIdx.x + o];
            red[1][threadIdx.x] += red[1][threadIdx.x + o];
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        dA[h] = red[0][0];
        dD[h] = red[1][0];
    }
}

size_t bwd_valu_lds(const Shape& s) {
    return (size_t)(5 * kRows * s.Q + 2 * kRows * s.P + 8) * sizeof(float);
}

template <typename Tin>
hipError_t launch_bwd_valu_t(const Shape& s, const BwdArgs& a, hipStream_t st) {
    const auto kern = chunk_bwd_valu_kernel<Tin>;
    const size_t lds = bwd_valu_lds(s);
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    const unsigned blocks = (unsigned)((size_t)s.B * s.G * s.nC * (s.Q / kRows));
    kern<<<blocks, kThreads, lds, st>>>(
        (const Tin*)a.x, (const Tin*)a.Bm, (const Tin*)a.Cm, a.dtc, a.cs, a.D, (const Tin*)a.entry,
        (const Tin*)a.exitg, (const Tin*)a.dy, (Tin*)a.dx, (Tin*)a.dB, (Tin*)a.dC, a.dcs,
        a.direct, a.lt_part, a.dd_part, s.T, s.H, s.G, s.P, s.N, s.Q, s.nC);
    return hipGetLastError();
}

}  // namespace

int chunk_bwd_valu_rows() { return kRows; }

hipError_t launch_chunk_bwd_valu(const Shape& s, ssd_dtype dtype, const BwdArgs& a,
                                 hipStream_t st) {
    if ((size_t)s.B * s.nC == 0) return hipSuccess;
    return dtype == SSD_F32 ? launch_bwd_valu_t<float>(s, a, st)
                            : launch_bwd_valu_t<__bf16>(s, a, st);
}

hipError_t launch_bwd_finalize(const Shape& s, const BwdArgs& a, int rows, hipStream_t st) {
    const int items = s.B * s.H * s.nC;
    if (items > 0) {
        const unsigned blocks =
            (unsigned)((size_t)s.B * s.nC * ((s.H + kDdtHeads - 1) / kDdtHeads));
        switch (s.Q) {
#define SSD_DDT(QV)                                                                          \
    case QV:                                                                                 \
        bwd_ddt_kernel<QV><<<blocks, kDdtThreads, 0, st>>>(a.dcs, a.direct, a.xs, a.lt_part, \
                                                        a.dtc, a.A, a.ddt, a.dA_part, s.T,   \
                                                        s.H, s.nC, rows);                    \
        break;
            SSD_DDT(64)
            SSD_DDT(128)
            SSD_DDT(256)
#undef SSD_DDT
            default:
                return hipErrorInvalidValue;
        }
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    bwd_param_kernel<<<s.H, kThreads, 0, st>>>(a.dA_part, a.dd_part, a.dA, a.dD, s.B, s.T, s.H,
                                               s.Q, s.nC, rows);
    return hipGetLastError();
}

}  // namespace ssd
