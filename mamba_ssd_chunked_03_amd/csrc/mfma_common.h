// mfma_common.h -- gfx950 building blocks shared by the bf16 MFMA kernels.
//
// MFMA: v_mfma_f32_16x16x32_bf16 (one wave: D[16x16] += A[16x32] B[32x16], fp32 accumulate).
// Lane l supplies row/column (l % 16) of A/B and the eight k-slots of lane group l / 16;
// it receives D rows 4*(l/16)..+3 of column l % 16.  Any relabelling of k works as long as
// A and B use the same one.  The kernels label the eight k-slots of lane group g as
// {4g..4g+3, 16+4g..16+4g+3} of a 32-step block: exactly the rows a lane holds in the two
// 16x16 outputs that cover 32 rows, so an MFMA output can be fed straight back as an
// operand of the next contraction over those rows.
//
// LDS transpose read (ds_read_b64_tr_b16): inside each group of 16 lanes, lane i receives
// element i % 4 of the four 8-byte chunks addressed by lanes 4q + i/4 (q = 0..3).  With
// lane a of the group addressing row r0 + a/4, column c0 + 4*(a % 4) of a row-major bf16
// matrix, lane i receives rows r0..r0+3 of column c0 + i: a 4 x 16 block transposed.  Two
// such reads give the eight time-ordered k-slots above straight from [time][feature] data.
//
// Data movement: buffer resources bound each access to the rows of one chunk; loads past
// the bound read zeros and stores past it are dropped (the ragged last chunk needs no
// branches).  buffer_load ... lds copies 16 bytes per lane from HBM straight into LDS
// (lane L of an instruction lands at its LDS base + 16 L), so the staging costs no VGPRs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {
namespace mfma {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int KB = 32;  // time steps per block = k of one MFMA

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float v) { return __builtin_amdgcn_exp2f(v); }

// two fp32 -> packed bf16 pair (round to nearest even), as one 32-bit word
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    bf16x2 p;
    p[0] = (__bf16)lo;
    p[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, p);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Workgroup barrier for data exchanged through LDS only.  __syncthreads() is a full
// workgroup fence that also waits for every outstanding global load and store; here only
// this wave's LDS operations are waited for.  The memory clobber keeps the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
// Wait until this wave's global/buffer loads (including copies into LDS) have landed,
// then barrier, so that every wave's copies are visible to all.
__device__ __forceinline__ void dma_barrier() {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                             0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, unsigned off, uint2 v) {
    const u32x2 w = {v.x, v.y};
    __builtin_amdgcn_raw_buffer_store_b64(w, r, (int)off, 0, 0);
}
__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t r, unsigned off, uint4 v) {
    const u32x4 w = {v.x, v.y, v.z, v.w};
    __builtin_amdgcn_raw_buffer_store_b128(w, r, (int)off, 0, 0);
}
// 16 bytes per lane from a buffer straight into LDS at lds_base + 16 * lane
__device__ __forceinline__ void buf_to_lds16(__amdgpu_buffer_rsrc_t r, void* lds_base,
                                             unsigned off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)lds_base, 16, off, 0, 0, 0);
}
// Lane groups g = lane / 16 and g ^ 1 each hold, for two tiles a and b, a run of 4 bf16
// (8 bytes) at element 4 g of a 16-element span.  After one exchange the even group holds
// tile a's elements 8 (g / 2) .. +7 and the odd group tile b's, so each lane makes one
// 16-byte store where it made two 8-byte ones (8-byte pieces spread over 16 rows write at
// about 60% of the rate of 16-byte ones).  Returns the lane's 16 bytes, to be stored in tile
// (g odd ? b : a) at element 8 (g / 2).  The exchange is v_permlane16_swap, which trades
// the odd 16-lane rows of its first operand for the even rows of its second: with (a, b) as
// the operands, an even row gets (its a, the odd row's a) and an odd row (the even row's b,
// its b), both in the order of the returned pair.
__device__ __forceinline__ uint4 pair_runs(uint2 ra, uint2 rb) {
    const auto x = __builtin_amdgcn_permlane16_swap(ra.x, rb.x, false, false);
    const auto y = __builtin_amdgcn_permlane16_swap(ra.y, rb.y, false, false);
    return make_uint4(x[0], y[0], x[1], y[1]);
}
// transpose read: see the header comment
// Sum over the four lane groups (lanes l, l ^ 16, l ^ 32, l ^ 48), the same value in every
// lane.  Two VALU exchanges instead of LDS-routed shuffles: v_permlane32_swap of v with
// itself yields (lower half, upper half) in every lane, so their sum is v + (v at l ^ 32);
// v_permlane16_swap likewise pairs the even and odd 16-lane rows.
__device__ __forceinline__ float colsum(float v) {
    const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                    false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ uint2 buf_load8(__amdgpu_buffer_rsrc_t r, unsigned off) {
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s16x4*)(p));
    return __builtin_bit_cast(uint2, v);
}

// Copies into LDS issued through inline asm: 16 bytes per lane from a buffer resource
// into LDS at lds + 16 * lane.  The compiler does not see these as writes to LDS, so it
// never makes later LDS reads wait for them; callers wait explicitly (s_waitcnt vmcnt)
// and barrier before reading what they copied.
// The LDS address travels in M0, which the compiler writes with a scalar instruction just
// before the asm block.  On gfx950 an LDS copy needs one wait state after an M0 write, or
// it may still see the previous M0 and land at the previous copy's address; the compiler
// inserts that wait for the copies it emits itself but does not look inside asm, so the
// block begins with it.
__device__ __forceinline__ void dma16(u32x4 r, uint32_t lds, uint32_t voff) {
    asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(r),
                 "{m0}"(lds)
                 : "memory");
}
// raw buffer resource words: base, stride 0, size in bytes (reads past it return zeros)
__device__ __forceinline__ u32x4 raw_rsrc(const void* base, unsigned bytes) {
    const uint64_t a = (uint64_t)base;
    return u32x4{(unsigned)a, (unsigned)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}
// LDS byte address of a pointer into shared memory
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const unsigned char*)p;
}

// Row-major bf16 matrices in LDS are stored as rows of 16-byte pieces with the piece
// index XOR-swizzled by the row (piece c of row r sits at slot c ^ (r % pieces_per_row)),
// which spreads the column reads of consecutive rows over the LDS banks.  Byte offset of
// element (r, col) for a power-of-two pieces_per_row:
__device__ __forceinline__ unsigned swz_off(int r, int col, int ppr) {
    return (unsigned)(r * ppr + ((col >> 3) ^ (r & (ppr - 1)))) * 16u + (unsigned)(col & 7) * 2u;
}

}  // namespace mfma
}  // namespace ssd
