// ssd_internal.h -- shapes, element access and kernel launchers shared by libssd's
// translation units.  Not part of the public ABI (that is include/ssd.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "ssd.h"

namespace ssd {

// Problem shape after validation; every size fits in int.
struct Shape {
    int B, T, H, P, N, G, Q, nC;
    int heads_per_group() const { return H / G; }
};

// ---- per-device launch state --------------------------------------------------------
// The only state the library keeps between calls: per kernel instantiation and device,
// whether the kernel's dynamic-LDS limit has been raised and how many of its workgroups
// are resident at once.  Both are computed on the kernel's first launch on a device.  Two
// threads making that first launch together both compute the same value; the slots are
// atomics, and a slot is published only after the attribute is set, so a thread that reads
// a nonzero slot launches after the attribute call of the thread that wrote it.
constexpr int kMaxDevices = 64;
using DeviceSlots = std::atomic<int>[kMaxDevices];

// Raise kern's dynamic LDS limit to `lds` bytes on the current device (once per device) and
// return in *grid the number of workgroups of `threads` threads resident at once, rounded
// down to a multiple of 8 (at least 8): the grid of a persistent kernel.
inline hipError_t resident_grid(const void* kern, int threads, unsigned lds,
                                DeviceSlots& slots, int* grid) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    int g = slots[dev].load(std::memory_order_acquire);
    if (g == 0) {
        e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        int ncu = 0, occ = 0;
        e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess) return e;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kern, threads, lds);
        if (e != hipSuccess) return e;
        const int g8 = (ncu * (occ > 0 ? occ : 1)) / 8;
        g = (g8 > 0 ? g8 : 1) * 8;
        slots[dev].store(g, std::memory_order_release);
    }
    *grid = g;
    return hipSuccess;
}

// Raise kern's dynamic LDS limit to `lds` bytes on the current device, once per device.
inline hipError_t allow_lds(const void* kern, unsigned lds, DeviceSlots& slots) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    if (slots[dev].load(std::memory_order_acquire) == 0) {
        e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) return e;
        slots[dev].store(1, std::memory_order_release);
    }
    return hipSuccess;
}

// ---- element access ---------------------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(__bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return (__bf16)v; }

// The step size's positivity map, softplus(v) = log(1 + exp(v)), written so that exp never
// overflows; the block prologue and the chunk cumsum share it, so both give the same bits.
__device__ __forceinline__ float softplus_step(float v) {
    return fmaxf(v, 0.f) + log1pf(expf(-fabsf(v)));
}

// ---- launchers (each returns the launch status) -------------------------------------
// Raw step sizes: rows of the projection output (row b*T + t at `stride` elements, H values
// in dtype) plus a per-head bias (may be null); the step size is softplus(raw + bias).
struct DtRaw {
    const void* p;
    long long stride;
    const float* bias;
    ssd_dtype dtype;
};
// cu (optional, device [nseq + 1], batch 1): packed sequence offsets; at every sequence
// start the running sum drops by a gap that zeroes every decay across the start.
// raw (optional): take the step sizes from raw rows instead of dt (which is then unused).
hipError_t launch_chunk_cumsum(const Shape& s, const float* dt, const float* A, float* dtc,
                               float* cs, hipStream_t st, const int* cu = nullptr,
                               int nseq = 0, const DtRaw* raw = nullptr);
// chunk states are read and entry states written in dtype (fp32 or bf16); the carried
// state is fp32
hipError_t launch_state_passing(const Shape& s, ssd_dtype dtype, const void* states,
                                const float* cs, const float* init, void* entry,
                                float* final_state, hipStream_t st);

// Plain fp32-accumulate VALU kernels: any supported size, fp32 or bf16 inputs.  Chunk
// states are written in the input dtype.
hipError_t launch_chunk_state_valu(const Shape& s, ssd_dtype dt, const void* x, const void* Bm,
                                   const float* dtc, const float* cs, void* states,
                                   hipStream_t st);
// entry states are read in the input dtype
hipError_t launch_chunk_scan_valu(const Shape& s, ssd_dtype dt, const void* x, const void* Bm,
                                  const void* Cm, const float* dtc, const float* cs,
                                  const float* D, const void* entry, void* y, hipStream_t st);

// bf16 MFMA kernels (gfx950 v_mfma_f32_16x16x32_bf16); *_supported says whether a shape
// has an instantiation.
bool chunk_state_mfma_supported(const Shape& s);
// With Cm and gram given, where chunk_state_writes_gram(s) the same launch also writes the
// chunk scan's C B^T blocks (else it ignores them).
bool chunk_state_writes_gram(const Shape& s);
hipError_t launch_chunk_state_mfma(const Shape& s, const void* x, const void* Bm,
                                   const float* dtc, const float* cs, void* states,
                                   const void* Cm, void* gram, hipStream_t st);
bool chunk_scan_mfma_supported(const Shape& s);
// The block's gate and normalisation applied in the chunk scan's store, where every norm
// group lies inside one head (S = H P / norm_groups channels, S a multiple of 16 dividing P):
// out = norm(y * SiLU(z)) over each group of a token's channels, written where y would be.
struct GateNorm {
    const void* z;        // rows of z in the input dtype, z_stride elements apart
    long long z_stride;
    const float* w;       // [H P], 16-byte aligned
    const float* b;       // [H P] or null (unused with rms), 16-byte aligned
    int groups_per_head;  // P / S
    int rms;
    float eps;
};
bool chunk_scan_gate_supported(const Shape& s, int groups_per_head);
// one recurrent step for every (b, h): state [B][H][N][P] fp32 in place; x, y [B][H][P] and
// B, C [B][G][N] in dtype (Shape's T and Q are not used)
hipError_t launch_decode_step(const Shape& s, ssd_dtype dtype, const void* x, const float* dt,
                              const float* A, const void* Bm, const void* Cm, const float* D,
                              float* state, void* y, hipStream_t st);
// bytes of the C B^T blocks the MFMA chunk scan reads (0 where the shape has no MFMA scan)
size_t chunk_gram_bytes(const Shape& s);
hipError_t launch_chunk_gram(const Shape& s, const void* Bm, const void* Cm, void* gram,
                             hipStream_t st);
hipError_t launch_chunk_scan_mfma(const Shape& s, const void* x, const void* Cm, const float* dtc,
                                  const float* cs, const float* D, const void* entry,
                                  const void* gram, void* y, hipStream_t st,
                                  const GateNorm* gate = nullptr);

// ---- backward ------------------------------------------------------------------------
// The gradient of every chunk's entry state through that chunk's own outputs,
// Z[c][p][n] = sum_i exp(cs_i) C_i[n] dy_i[p] (the chunk_state kernels with C for B, dy for
// x and weight exp(cs_i)); [B][H][nC][P][N] in dtype.
hipError_t launch_chunk_dstate_valu(const Shape& s, ssd_dtype dt, const void* dy, const void* Cm,
                                    const float* cs, void* dstates, hipStream_t st);
hipError_t launch_chunk_dstate_mfma(const Shape& s, const void* dy, const void* Cm,
                                    const float* cs, void* dstates, hipStream_t st);
// the inter-chunk carry run last chunk first: exit_grads[c] = dL/d(end state of chunk c),
// d_init = dL/d init_state ([N][P] fp32, may be NULL), from d_final (NULL = zero)
hipError_t launch_state_passing_rev(const Shape& s, ssd_dtype dtype, const void* dstates,
                                    const float* cs, const float* d_final, void* exit_grads,
                                    float* d_init, hipStream_t st);

// Everything the in-chunk backward and its finishing kernels read and write.
struct BwdArgs {
    const void *x, *Bm, *Cm, *dy;          // inputs, dtype
    const float *dtc, *cs, *A, *D;         // fp32
    const void *entry, *exitg;             // entry states and exit gradients, [P][N], dtype
    void *dx, *dB, *dC;                    // outputs, dtype
    float *ddt, *dA, *dD;                  // outputs, fp32
    float *dcs, *direct;                   // [B][H][nC][Q]: dL/dcs and the explicit dL/ddt
    // [B][H][nC][Q / 64][Q], MFMA path only (null otherwise): the in-chunk pair terms that
    // cross a 64-row block boundary, kept apart from dcs so that no pair is summed twice
    // (plane 0: per column, its pairs with rows in later blocks; plane 1 + s: per row, its
    // pairs with columns in block s)
    float* xs;
    float *lt_part, *dd_part;              // [B][H][nC][Q / rows]: per row tile
    float* dA_part;                        // [B][H][nC]
    // MFMA path at dstate 256 only (null otherwise): the terms through the carried states,
    // formed by a kernel of their own before the in-chunk one -- (F B_j) per step and head
    // ([B][T][H][P], bf16) and the head sums of the dB, dC terms ([B][T][G][N], fp32)
    void* xfb;
    float *dBs, *dCs;
};
int chunk_bwd_valu_rows();
hipError_t launch_chunk_bwd_valu(const Shape& s, ssd_dtype dtype, const BwdArgs& a,
                                 hipStream_t st);
// bf16 MFMA in-chunk backward (headdim 64 with dstate 64, 128 or 256; headdim 32 with
// dstate 32, 64 or 128), same outputs; rows per tile 64.  At dstate 256 it also needs
// BwdArgs' xfb, dBs and dCs (chunk_bwd_mfma_carried).
bool chunk_bwd_mfma_supported(const Shape& s);
bool chunk_bwd_mfma_carried(const Shape& s);
int chunk_bwd_mfma_rows();
hipError_t launch_chunk_bwd_mfma(const Shape& s, const BwdArgs& a, hipStream_t st);
// ddt and dA, dD from the per-chunk and per-tile shares (rows: rows per tile)
hipError_t launch_bwd_finalize(const Shape& s, const BwdArgs& a, int rows, hipStream_t st);

// ---- packed variable-length rows (varlen.hip) -------------------------------------------
// the same on bf16 MFMA (the per-item chunk-state kernel in its final-state mode), for the
// sizes it is instantiated for
bool varlen_final_mfma_supported(const Shape& s);
hipError_t launch_varlen_final_mfma(const Shape& s, const void* x, const void* Bm,
                                    const float* dtc, const float* cs, const void* entry,
                                    const int* cu, int nseq, float* finals, hipStream_t st);
// each sequence's state after its last step, [nseq][H][N][P] fp32 (zeros for an empty one)
hipError_t launch_varlen_final(const Shape& s, ssd_dtype dtype, const void* x, const void* Bm,
                               const float* dtc, const float* cs, const void* entry,
                               const int* cu, int nseq, float* finals, hipStream_t st);

// ---- the block around the layer (block.hip) -------------------------------------------
struct BlockPrologueArgs {
    const void* xbc;            // [B][T] rows of H*P + 2*G*N channels, in dtype
    long long xbc_stride;       // elements between rows
    const float *conv_w, *conv_b;  // [H*P + 2GN][conv_k], [H*P + 2GN] (conv_b may be null)
    int conv_k;                 // 1..8
    const void* dt_raw;         // [B][T] rows of H, in dtype
    long long dt_stride;
    const float* dt_bias;       // [H] or null
    void *x, *Bm, *Cm;          // [B][T][H][P], [B][T][G][N] x2, in dtype
    float* dt;                  // [B][T][H]
};
hipError_t launch_block_prologue(const Shape& s, ssd_dtype dtype, const BlockPrologueArgs& a,
                                 hipStream_t st);
struct BlockEpilogueArgs {
    const void* y;              // [B][T][H*P], in dtype
    const void* z;              // [B][T] rows of H*P, in dtype
    long long z_stride;
    const float *norm_w, *norm_b;  // [H*P] (norm_b may be null)
    int groups, rms;
    float eps;
    void* out;                  // [B][T][H*P], in dtype
};
hipError_t launch_block_epilogue(const Shape& s, ssd_dtype dtype, const BlockEpilogueArgs& a,
                                 hipStream_t st);

}  // namespace ssd
