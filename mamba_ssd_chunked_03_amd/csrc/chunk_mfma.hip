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

// ============================================================================ chunk_scan

// One workgroup per (batch, group, chunk, range of heads).  The heads of a group share B
// and C, so C B^T for the chunk is computed once and kept in registers (rounded to bf16)
// for every head of the range; per head only the decay mask, the X^T Gm^T products and
// the entry-state readout remain.  Wave w owns the 16-row tile w of the chunk and the
// w/2+1 32-step blocks of the causal triangle under it.  While one head computes, the
// next head's x, entry state, cs and dt are already in flight into registers.
template <int Q, int N, int P>
__global__ __launch_bounds__(Q * 4, 1) void chunk_scan_mfma_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Bm, const __bf16* __restrict__ Cm,
    const float* __restrict__ dtc, const float* __restrict__ cs, const float* __restrict__ D,
    const __bf16* __restrict__ E, __bf16* __restrict__ y, int T, int H, int G, int nC,
    int heads_per_wg, int ranges) {
    constexpr int NTH = Q * 4;                    // one wave per 16-row tile
    constexpr int NB = Q / KB;
    constexpr int PT = P / 16;
    constexpr int NK = N / 32;
    constexpr int LDB = N + 8;                    // row stride (bf16) of B and of E in LDS
    constexpr int LDX = Q + 4;                    // row stride (bf16) of the transposed x chunk
    constexpr int BTASK = Q * (N / 8);            // 16-byte pieces of the B chunk
    constexpr int XTASK = (Q / 2) * (P / 8);      // (row pair, 8-column group) of the x chunk
    constexpr int ETASK = P * N / 8;              // 16-byte pieces of the entry state
    constexpr int BPT = (BTASK + NTH - 1) / NTH;
    constexpr int XPT = (XTASK + NTH - 1) / NTH;
    constexpr int EPT = (ETASK + NTH - 1) / NTH;
    constexpr int B_BYTES = Q * LDB * 2;
    constexpr int H_BYTES = P * LDX * 2 + P * LDB * 2;
    constexpr int U_BYTES = B_BYTES > H_BYTES ? B_BYTES : H_BYTES;
    static_assert(N % 32 == 0 && P % 16 == 0 && Q % 64 == 0, "tile shape");

    // B chunk during setup; afterwards the current head's transposed x and entry state
    __shared__ __align__(16) unsigned char smem[U_BYTES];
    __shared__ float s_cs[Q];  // chunk-local prefix sums of dt*A, times log2(e)
    __shared__ float s_dt[Q];
    __shared__ float s_v[Q];   // exp(cs_e - cs_i) dt_i, e = last step of i's 32-step block
    constexpr int LDY = P + 8;
    __shared__ __align__(16) __bf16 Ys[Q][LDY];  // y rows of the head, staged for 16-byte stores
    typedef __bf16 RowB[LDB];
    typedef __bf16 RowX[LDX];
    RowB* Bs = reinterpret_cast<RowB*>(smem);
    RowX* Xt = reinterpret_cast<RowX*>(smem);
    RowB* Es = reinterpret_cast<RowB*>(smem + P * LDX * 2);

    const int r = blockIdx.x % ranges;
    const int unit = blockIdx.x / ranges;  // (b, g, c)
    const int c = unit % nC;
    const int bg = unit / nC;
    const int g = bg % G;
    const int b = bg / G;
    const int hpg = H / G;
    const int h_first = g * hpg + r * heads_per_wg;
    const int nh = min(heads_per_wg, hpg - r * heads_per_wg);
    if (nh <= 0) return;
    const int tid = threadIdx.x;
    const int tile = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
    const int nblk = tile / 2 + 1;  // 32-step blocks with i <= some row of the tile
    const int t0 = c * Q;
    const int j = tile * 16 + l16;  // this lane's row of the chunk (column of Y^T)
    const int tj = t0 + j;

    // ---------------- per-head inputs: registers first, then LDS.  Loads use a scalar base
    // and 32-bit byte offsets, and rows past the end of the sequence are zeroed only when
    // stored, so that issuing the prefetch never waits for it.
    uint4 rx[XPT][2], re[EPT];
    float rcs = 0.f, rce = 0.f, rdt = 0.f;
    const uint4 z4 = make_uint4(0, 0, 0, 0);
    const bool cs_wave = tile < Q / 64;  // the waves that carry cs / dt (tid < Q)
    auto load_head = [&](int h) {
        // an opaque copy of tid: offsets are recomputed per head instead of being kept
        // (or spilled, and reloaded through the same counter as the prefetch) across heads
        int tix = tid;
        asm volatile("" : "+v"(tix));
        if (cs_wave) {
            const float* csb = cs + ((size_t)(b * H + h) * nC + c) * Q;
            const float* dtb = dtc + ((size_t)(b * H + h) * nC + c) * Q;
            rcs = csb[tix];
            rce = csb[tix | (KB - 1)];
            rdt = dtb[tix];
        }
        const char* xb = reinterpret_cast<const char*>(x + (size_t)h * P);
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int e = tix + q * NTH;
            const int rp = e % (Q / 2), cg = e / (Q / 2);
            const int t = t0 + 2 * rp;
            if (XTASK % NTH == 0 || e < XTASK) {
                // rows past the end read row T-1 (in bounds); store_head zeroes them
                const unsigned ta = (unsigned)(b * T + min(t, T - 1)), tb = (unsigned)(b * T + min(t + 1, T - 1));
                const unsigned rowb = (unsigned)(H * P * 2);
                rx[q][0] = *reinterpret_cast<const uint4*>(xb + ta * rowb + cg * 16u);
                rx[q][1] = *reinterpret_cast<const uint4*>(xb + tb * rowb + cg * 16u);
            }
        }
        const __bf16* esrc = E + ((size_t)(b * H + h) * nC + c) * P * N;
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
            const int e = tix + q * NTH;
            if (ETASK % NTH == 0 || e < ETASK) re[q] = *reinterpret_cast<const uint4*>(esrc + (size_t)e * 8);
        }
    };
    auto store_head = [&]() {
#pragma unroll
        for (int q = 0; q < XPT; ++q) {
            const int e = tid + q * NTH;
            if (XTASK % NTH != 0 && e >= XTASK) continue;
            const int rp = e % (Q / 2), cg = e / (Q / 2);
            const int t = t0 + 2 * rp;
            const uint4 va = keep_or_zero(t < T, rx[q][0]), vb = keep_or_zero(t + 1 < T, rx[q][1]);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t w = bits_of(va, k) | (bits_of(vb, k) << 16);
                *reinterpret_cast<uint32_t*>(&Xt[cg * 8 + k][2 * rp]) = w;
            }
        }
#pragma unroll
        for (int q = 0; q < EPT; ++q) {
            const int e = tid + q * NTH;
            if (ETASK % NTH != 0 && e >= ETASK) continue;
            const int p = e / (N / 8), n = (e % (N / 8)) * 8;
            *reinterpret_cast<uint4*>(&Es[p][n]) = re[q];
        }
        if (cs_wave) {
            s_cs[tid] = rcs * kLog2e;
            s_dt[tid] = rdt;
            s_v[tid] = exp2_fast((rce - rcs) * kLog2e) * rdt;
        }
    };

    // ---------------- setup: C fragments of this wave's rows, the B chunk, C B^T
    bf16x8 cf[NK];
    {
        const __bf16* src = Cm + ((size_t)(b * T + min(tj, T - 1)) * G + g) * N + 8 * g4;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const uint4 v = *reinterpret_cast<const uint4*>(src + 32 * kk);
            cf[kk] = __builtin_bit_cast(bf16x8, keep_or_zero(tj < T, v));
        }
    }
    {
        uint4 rb[BPT];
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int e = tid + q * NTH;
            const int row = e / (N / 8), cg = e % (N / 8);
            const int t = t0 + row;
            const uint4 v = *reinterpret_cast<const uint4*>(
                Bm + ((size_t)(b * T + min(t, T - 1)) * G + g) * N + cg * 8);
            rb[q] = keep_or_zero((BTASK % NTH == 0 || e < BTASK) && t < T, v);
        }
        load_head(h_first);
#pragma unroll
        for (int q = 0; q < BPT; ++q) {
            const int e = tid + q * NTH;
            if (BTASK % NTH != 0 && e >= BTASK) continue;
            const int row = e / (N / 8), cg = e % (N / 8);
            *reinterpret_cast<uint4*>(&Bs[row][cg * 8]) = rb[q];
        }
    }
    lds_barrier();
    // G^T rows (32ib + 4*g4 + 0..3, 32ib + 16 + 4*g4 + 0..3) of column j, as bf16: gq[ib]
    // for the blocks wholly below the tile (ib < nblk - 1), gd for the diagonal block
    // (ib = nblk - 1, the only block that crosses the tile's rows)
    auto cbt = [&](int ib) {
        f32x4 g0 = f32x4{0.f, 0.f, 0.f, 0.f}, g1 = g0;
#pragma unroll
        for (int kk = 0; kk < NK; ++kk) {
            const bf16x8 a0 = *reinterpret_cast<const bf16x8*>(&Bs[ib * KB + l16][32 * kk + 8 * g4]);
            const bf16x8 a1 = *reinterpret_cast<const bf16x8*>(&Bs[ib * KB + 16 + l16][32 * kk + 8 * g4]);
            g0 = mfma16(a0, cf[kk], g0);
            g1 = mfma16(a1, cf[kk], g1);
        }
        return make_uint4(pack_bf16(g0[0], g0[1]), pack_bf16(g0[2], g0[3]),
                          pack_bf16(g1[0], g1[1]), pack_bf16(g1[2], g1[3]));
    };
    const int ibd = nblk - 1;
    uint4 gq[NB - 1 > 0 ? NB - 1 : 1];
#pragma unroll
    for (int ib = 0; ib < NB - 1; ++ib) gq[ib] = ib < ibd ? cbt(ib) : z4;
    uint4 gd = cbt(ibd);

    // ---------------- heads
    for (int hh = 0; hh < nh; ++hh) {
        const int h = h_first + hh;
        lds_barrier();  // all reads of the previous contents of smem / s_* are done
        store_head();
        lds_barrier();
        // prefetch the next head (the last head re-reads itself: an unconditional load keeps
        // the wait for it at the loop top from also waiting for this head's y stores)
        load_head(hh + 1 < nh ? h + 1 : h);
        // C B^T stays packed in bf16: an empty asm per head stops the compiler from hoisting
        // the unpacked fp32 copies out of the head loop (which would double its registers)
#pragma unroll
        for (int ib = 0; ib < NB - 1; ++ib)
            asm volatile("" : "+v"(gq[ib].x), "+v"(gq[ib].y), "+v"(gq[ib].z), "+v"(gq[ib].w));
        asm volatile("" : "+v"(gd.x), "+v"(gd.y), "+v"(gd.z), "+v"(gd.w));

        // stage 4: the entry state read out by C, decayed from the chunk start to row j
        f32x4 acc[PT];
        const float csj = s_cs[j];
        {
            const float sc = exp2_fast(csj);
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                f32x4 a4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kk = 0; kk < NK; ++kk) {
                    const bf16x8 ea =
                        *reinterpret_cast<const bf16x8*>(&Es[p * 16 + l16][32 * kk + 8 * g4]);
                    a4 = mfma16(ea, cf[kk], a4);
                }
                acc[p] = a4 * sc;
            }
        }

        // stage 1: the masked quadratic form over the 32-step blocks under this tile
        auto xprod = [&](int ib, const float* m) {
            const uint4 mw = make_uint4(pack_bf16(m[0], m[1]), pack_bf16(m[2], m[3]),
                                        pack_bf16(m[4], m[5]), pack_bf16(m[6], m[7]));
            const bf16x8 bm = __builtin_bit_cast(bf16x8, mw);
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                const uint2 lo = *reinterpret_cast<const uint2*>(&Xt[p * 16 + l16][ib * KB + 4 * g4]);
                const uint2 hi = *reinterpret_cast<const uint2*>(&Xt[p * 16 + l16][ib * KB + 16 + 4 * g4]);
                const bf16x8 xa = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
                acc[p] = mfma16(xa, bm, acc[p]);
            }
        };
        // blocks wholly below the tile: the decay factors at the block end e,
        // exp(cs_j - cs_e) * exp(cs_e - cs_i) dt_i, both factors <= 1
#pragma unroll
        for (int ib = 0; ib < NB - 1; ++ib) {
            if (ib >= ibd) continue;
            const int i0 = ib * KB + 4 * g4;
            const float f = exp2_fast(csj - s_cs[ib * KB + KB - 1]);
            const float4 va = *reinterpret_cast<const float4*>(&s_v[i0]);
            const float4 vb = *reinterpret_cast<const float4*>(&s_v[i0 + 16]);
            const uint4 gw = gq[ib];
            float m[8];
            m[0] = bf16_lo(gw.x) * va.x * f; m[1] = bf16_hi(gw.x) * va.y * f;
            m[2] = bf16_lo(gw.y) * va.z * f; m[3] = bf16_hi(gw.y) * va.w * f;
            m[4] = bf16_lo(gw.z) * vb.x * f; m[5] = bf16_hi(gw.z) * vb.y * f;
            m[6] = bf16_lo(gw.w) * vb.z * f; m[7] = bf16_hi(gw.w) * vb.w * f;
            xprod(ib, m);
            // keep unrolled blocks from hoisting each other's operand loads
            __builtin_amdgcn_sched_barrier(0);
        }
        {   // the diagonal block: mask above the diagonal through the exponent (2^-inf = 0)
            const int i0 = ibd * KB + 4 * g4;
            const float4 ca = *reinterpret_cast<const float4*>(&s_cs[i0]);
            const float4 cb = *reinterpret_cast<const float4*>(&s_cs[i0 + 16]);
            const float4 da = *reinterpret_cast<const float4*>(&s_dt[i0]);
            const float4 db = *reinterpret_cast<const float4*>(&s_dt[i0 + 16]);
            const float cav[4] = {ca.x, ca.y, ca.z, ca.w}, cbv[4] = {cb.x, cb.y, cb.z, cb.w};
            const float dav[4] = {da.x, da.y, da.z, da.w}, dbv[4] = {db.x, db.y, db.z, db.w};
            const float gv[8] = {bf16_lo(gd.x), bf16_hi(gd.x), bf16_lo(gd.y), bf16_hi(gd.y),
                                 bf16_lo(gd.z), bf16_hi(gd.z), bf16_lo(gd.w), bf16_hi(gd.w)};
            const float ninf = -__builtin_inff();
            float m[8];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float ea = i0 + q <= j ? csj - cav[q] : ninf;
                const float ec = i0 + 16 + q <= j ? csj - cbv[q] : ninf;
                m[q] = gv[q] * exp2_fast(ea) * dav[q];
                m[4 + q] = gv[4 + q] * exp2_fast(ec) * dbv[q];
            }
            xprod(ibd, m);
        }

        // stage 5 and the skip: y[j][p] = acc + D x[j][p]; lane holds p = pt*16 + 4*g4 + q.
        // x comes from the LDS copy (a global load here would make the wait for it also wait
        // for the next head's prefetch and for every earlier store).  The wave's 16 rows go
        // through LDS so that the stores are whole 16-byte pieces of whole rows.
        {
            const float dh = D[h];
#pragma unroll
            for (int p = 0; p < PT; ++p) {
                const int p0 = p * 16 + 4 * g4;
                float xv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) xv[q] = (float)Xt[p0 + q][j];
                uint2 out;
                out.x = pack_bf16(acc[p][0] + dh * xv[0], acc[p][1] + dh * xv[1]);
                out.y = pack_bf16(acc[p][2] + dh * xv[2], acc[p][3] + dh * xv[3]);
                *reinterpret_cast<uint2*>(&Ys[j][p0]) = out;
            }
            // the wave reads back only its own rows: no workgroup barrier needed
            constexpr int PIECES = 16 * P / 8;  // 16-byte pieces in the wave's 16 rows
#pragma unroll
            for (int q = 0; q < (PIECES + 63) / 64; ++q) {
                const int e = lane + q * 64;
                if (PIECES % 64 != 0 && e >= PIECES) continue;
                const int rr = e / (P / 8), pc = (e % (P / 8)) * 8;
                const int jj = tile * 16 + rr;
                const uint4 v = *reinterpret_cast<const uint4*>(&Ys[jj][pc]);
                if (t0 + jj < T)
                    *reinterpret_cast<uint4*>(y + ((size_t)(b * T + t0 + jj) * H + h) * P + pc) = v;
            }
        }
    }
}

// Per-(b, h, chunk) variant for shapes whose chunks do not fit the shared-C B^T kernel's
// LDS: C B^T is recomputed per head, and B and x stream through LDS in double-buffered
// 32-step slices, so LDS stays small at any (Q, N, P).
template <int Q, int N, int P>
__global__ __launch_bounds__(Q * 2) void chunk_scan_mfma_head_kernel(
    const __bf16* __restrict__ x, const __bf16* __restrict__ Bm, const __bf16* __restrict__ Cm,
    const float* __restrict__ dtc, const float* __restrict__ cs, const float* __restrict__ D,
    const __bf16* __restrict__ E, __bf16* __restrict__ y, int T, int H, int G, int nC) {
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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
    const int lane = tid & 63, l16 = lane & 15, g4 = lane >> 4;
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
    {   // entry state, bf16 [p][n]
        const __bf16* src = E + ((size_t)bh * nC + c) * P * N;
        for (int e = tid; e < P * N / 8; e += NTH) {
            const int p = e / (N / 8), n = (e % (N / 8)) * 8;
            *reinterpret_cast<uint4*>(&Es[p][n]) =
                *reinterpret_cast<const uint4*>(src + (size_t)p * N + n);
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
    lds_barrier();

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
        lds_barrier();
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

// Heads of one (batch, group, chunk) unit are split into `ranges` workgroups so that the
// grid covers the GPU's 256 CUs at least once, keeping >= 4 heads per workgroup where the
// group has that many (each workgroup pays one C B^T setup for its range).
inline void scan_split(const Shape& s, int* heads_per_wg, int* ranges) {
    const long units = (long)s.B * s.G * s.nC;
    const int hpg = s.H / s.G;
    int want = (int)((256 + units - 1) / units);
    int maxr = hpg / 4 > 0 ? hpg / 4 : 1;
    int r = want < maxr ? want : maxr;
    if (r < 1) r = 1;
    *heads_per_wg = (hpg + r - 1) / r;
    *ranges = (hpg + *heads_per_wg - 1) / *heads_per_wg;
}

// LDS bytes of the shared-C B^T chunk scan at (Q, N, P); it is used where this fits.
constexpr int scan_shared_lds(int Q, int N, int P) {
    return (Q * (N + 8) * 2 > P * (Q + 4) * 2 + P * (N + 8) * 2
                ? Q * (N + 8) * 2
                : P * (Q + 4) * 2 + P * (N + 8) * 2) +
           3 * Q * 4 + Q * (P + 8) * 2;
}
constexpr int kLdsBytes = 160 * 1024;

template <int Q, int N, int P>
hipError_t launch_scan_t(const Shape& s, const void* x, const void* Bm, const void* Cm,
                         const float* dtc, const float* cs, const float* D, const void* E,
                         void* y, hipStream_t st) {
    if constexpr (scan_shared_lds(Q, N, P) > kLdsBytes) {
        const unsigned blocks = (unsigned)((size_t)s.B * s.H * s.nC);
        chunk_scan_mfma_head_kernel<Q, N, P><<<blocks, Q * 2, 0, st>>>(
            (const __bf16*)x, (const __bf16*)Bm, (const __bf16*)Cm, dtc, cs, D,
            (const __bf16*)E, (__bf16*)y, s.T, s.H, s.G, s.nC);
        return hipGetLastError();
    } else {
    int hpw, ranges;
    scan_split(s, &hpw, &ranges);
    const unsigned blocks = (unsigned)((size_t)s.B * s.G * s.nC * ranges);
    chunk_scan_mfma_kernel<Q, N, P><<<blocks, Q * 4, 0, st>>>(
        (const __bf16*)x, (const __bf16*)Bm, (const __bf16*)Cm, dtc, cs, D, (const __bf16*)E,
        (__bf16*)y, s.T, s.H, s.G, s.nC, hpw, ranges);
    return hipGetLastError();
    }
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
                              const float*, const float*, const void*, void*, hipStream_t);

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
                                  const void* entry, void* y, hipStream_t st) {
    ScanFn f = pick_scan(s);
    if (!f) return hipErrorInvalidValue;
    if ((size_t)s.B * s.H * s.nC == 0) return hipSuccess;
    return f(s, x, Bm, Cm, dtc, cs, D, entry, y, st);
}

}  // namespace ssd
