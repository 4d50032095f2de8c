// ssd_api.hip -- libssd's C ABI: argument validation, workspace layout and dispatch.
//
// Every entry point validates all of its arguments before enqueuing anything, returns a
// status code (no exceptions cross the ABI) and never synchronises.  Dispatch: bf16
// inputs take the MFMA kernels when the shape has an instantiation, everything else the
// fp32 VALU kernels.
#include <string.h>

#include <atomic>
#include <initializer_list>

#include "ssd_internal.h"

using ssd::Shape;

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 31;  // int indexing inside kernels

bool supported_chunk(int q) { return q == 64 || q == 128 || q == 256; }
bool supported_dstate(int64_t n) { return n == 16 || n == 32 || n == 64 || n == 128 || n == 256; }
bool supported_headdim(int64_t p) { return p == 16 || p == 32 || p == 64 || p == 128; }
bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Whether the product of non-negative factors is below kMaxElems.  Each factor is checked
// against what is left of the budget by division, so no intermediate product can overflow.
bool product_fits(std::initializer_list<int64_t> factors) {
    for (int64_t f : factors)
        if (f == 0) return true;
    int64_t acc = 1;
    for (int64_t f : factors) {
        if (f > (kMaxElems - 1) / acc) return false;  // acc * f would reach kMaxElems
        acc *= f;
    }
    return true;
}

ssd_status make_shape(const ssd_dims* d, int chunk_len, Shape* s) {
    if (!d) return SSD_ERR_NULL;
    if (d->batch < 0 || d->seqlen < 0 || d->nheads < 1 || d->headdim < 1 || d->dstate < 1 ||
        d->ngroups < 1 || d->nheads % d->ngroups != 0)
        return SSD_ERR_DIMS;
    if (!supported_chunk(chunk_len) || !supported_dstate(d->dstate) ||
        !supported_headdim(d->headdim))
        return SSD_ERR_UNSUPPORTED;
    // every size below 2^31 first (so that the int casts and the chunk count cannot
    // overflow), then every tensor below 2^31 elements; ngroups <= nheads since it divides it
    if (d->batch >= kMaxElems || d->seqlen >= kMaxElems || d->nheads > 65536)
        return SSD_ERR_DIMS;
    const int64_t nC = (d->seqlen + chunk_len - 1) / chunk_len;
    const int64_t tpad = nC * chunk_len;
    if (!product_fits({d->batch, tpad, d->nheads, d->headdim}) ||
        !product_fits({d->batch, tpad, d->ngroups, d->dstate}) ||
        !product_fits({d->batch, d->nheads, nC, d->headdim, d->dstate}))
        return SSD_ERR_DIMS;
    s->B = (int)d->batch;
    s->T = (int)d->seqlen;
    s->H = (int)d->nheads;
    s->P = (int)d->headdim;
    s->N = (int)d->dstate;
    s->G = (int)d->ngroups;
    s->Q = chunk_len;
    s->nC = (int)nC;
    return SSD_OK;
}

bool valid_dtype(ssd_dtype t) { return t == SSD_F32 || t == SSD_BF16; }

constexpr size_t kAlign = 256;
size_t round_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

struct Workspace {
    float *dtc, *cs;
    void* states;  // chunk states, in the input dtype
    void* entry;  // entry states, in the input dtype
    void* gram;   // C B^T blocks of the MFMA chunk scan (empty where unused)
};

size_t workspace_bytes(const Shape& s, Workspace* w, char* base) {
    const size_t chunk_elems = (size_t)s.B * s.H * s.nC * s.Q;
    const size_t state_elems = (size_t)s.B * s.H * s.nC * s.P * s.N;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += round_up(bytes);
        return (float*)p;
    };
    Workspace ws;
    ws.dtc = take(chunk_elems * sizeof(float));
    ws.cs = take(chunk_elems * sizeof(float));
    ws.states = take(state_elems * sizeof(float));
    ws.entry = take(state_elems * sizeof(float));  // fp32 size: enough for either dtype
    ws.gram = take(ssd::chunk_gram_bytes(s));
    if (w) *w = ws;
    return off;
}

ssd_status hip_status(hipError_t e) { return e == hipSuccess ? SSD_OK : SSD_ERR_HIP; }

bool any_misaligned(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return true;
    return false;
}

// fp32 tensors read one element at a time (dt, A, D, init_state, final_state)
bool any_misaligned4(std::initializer_list<const void*> ptrs) {
    for (const void* p : ptrs)
        if (p && ((uintptr_t)p & 3u) != 0) return true;
    return false;
}

bool uses_gram(const Shape& s, ssd_dtype dtype) {
    return dtype == SSD_BF16 && ssd::chunk_scan_mfma_supported(s);
}

// chunk states; with C and gram given (and a gram buffer in use for the shape) also the
// chunk scan's C B^T blocks, in the same launch where the kernel can, else right after
ssd_status run_chunk_state(const Shape& s, ssd_dtype dtype, const void* x, const void* B,
                           const float* dtc, const float* cs, void* states, const void* C,
                           void* gram, hipStream_t st) {
    const bool want_gram = C != nullptr && gram != nullptr && uses_gram(s, dtype);
    if (dtype == SSD_BF16 && ssd::chunk_state_mfma_supported(s)) {
        ssd_status r = hip_status(ssd::launch_chunk_state_mfma(
            s, x, B, dtc, cs, states, want_gram ? C : nullptr, want_gram ? gram : nullptr, st));
        if (r != SSD_OK || !want_gram || ssd::chunk_state_writes_gram(s)) return r;
    } else {
        ssd_status r = hip_status(ssd::launch_chunk_state_valu(s, dtype, x, B, dtc, cs, states, st));
        if (r != SSD_OK || !want_gram) return r;
    }
    return hip_status(ssd::launch_chunk_gram(s, B, C, gram, st));
}

// Backward workspace: the forward intermediates it recomputes (dt_chunk, cs, chunk states --
// reused for the chunk entry-state gradients --, entry states), the exit gradients, and
// the per-step / per-tile / per-chunk shares the finishing kernels reduce.
struct BwdWorkspace {
    float *dtc, *cs;
    void *states, *entry, *exitg;
    float *dcs, *direct, *xs, *lt_part, *dd_part, *dA_part;
    void* xfb;            // the carried-state terms at dstate 256 (null otherwise)
    float *dBs, *dCs;
};

size_t bwd_workspace_bytes(const Shape& s, BwdWorkspace* w, char* base) {
    const size_t chunk_elems = (size_t)s.B * s.H * s.nC * s.Q;
    const size_t state_elems = (size_t)s.B * s.H * s.nC * s.P * s.N;
    const size_t tile_elems = (size_t)s.B * s.H * s.nC * (s.Q / ssd::chunk_bwd_valu_rows());
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += round_up(bytes);
        return (float*)p;
    };
    BwdWorkspace ws;
    ws.dtc = take(chunk_elems * sizeof(float));
    ws.cs = take(chunk_elems * sizeof(float));
    ws.states = take(state_elems * sizeof(float));  // fp32 size: enough for either dtype
    ws.entry = take(state_elems * sizeof(float));
    ws.exitg = take(state_elems * sizeof(float));
    ws.dcs = take(chunk_elems * sizeof(float));
    ws.direct = take(chunk_elems * sizeof(float));
    ws.xs = take(chunk_elems * (size_t)(s.Q / 64 > 0 ? s.Q / 64 : 1) * sizeof(float));
    ws.lt_part = take(tile_elems * sizeof(float));
    ws.dd_part = take(tile_elems * sizeof(float));
    ws.dA_part = take((size_t)s.B * s.H * s.nC * sizeof(float));
    ws.xfb = nullptr;
    ws.dBs = ws.dCs = nullptr;
    if (ssd::chunk_bwd_mfma_carried(s)) {  // sized by shape: the dtype is not known here
        const size_t tokens = (size_t)s.B * s.T;
        ws.xfb = take(tokens * s.H * s.P * 2);
        ws.dBs = take(tokens * s.G * s.N * sizeof(float));
        ws.dCs = take(tokens * s.G * s.N * sizeof(float));
    }
    if (w) *w = ws;
    return off;
}

ssd_status run_chunk_scan(const Shape& s, ssd_dtype dtype, const void* x, const void* B,
                          const void* C, const float* dtc, const float* cs, const float* D,
                          const void* entry, const void* gram, void* y, hipStream_t st,
                          const ssd::GateNorm* gate = nullptr) {
    if (uses_gram(s, dtype))
        return hip_status(
            ssd::launch_chunk_scan_mfma(s, x, C, dtc, cs, D, entry, gram, y, st, gate));
    if (gate) return SSD_ERR_UNSUPPORTED;
    return hip_status(ssd::launch_chunk_scan_valu(s, dtype, x, B, C, dtc, cs, D, entry, y, st));
}

}  // namespace

extern "C" {

const char* ssd_status_string(ssd_status status) {
    switch (status) {
        case SSD_OK: return "SSD_OK";
        case SSD_ERR_NULL: return "SSD_ERR_NULL: a required pointer is NULL";
        case SSD_ERR_DIMS: return "SSD_ERR_DIMS: sizes out of range or nheads % ngroups != 0";
        case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: chunk_len/dstate/headdim/dtype not supported";
        case SSD_ERR_ALIGN: return "SSD_ERR_ALIGN: a pointer is not aligned as required";
        case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing or too small";
        case SSD_ERR_HIP: return "SSD_ERR_HIP: the HIP runtime reported a launch error";
    }
    return "SSD_ERR_UNKNOWN";
}

size_t ssd_fwd_workspace_size(const ssd_dims* dims, int chunk_len) {
    Shape s;
    if (make_shape(dims, chunk_len, &s) != SSD_OK) return 0;
    return workspace_bytes(s, nullptr, nullptr);
}

ssd_status ssd_chunk_cumsum(const ssd_dims* dims, int chunk_len, const float* dt, const float* A,
                            float* dt_chunk, float* cs, void* stream) {
    Shape s;
    ssd_status r = make_shape(dims, chunk_len, &s);
    if (r != SSD_OK) return r;
    if ((size_t)s.B * s.T > 0 && (!dt || !A || !dt_chunk || !cs)) return SSD_ERR_NULL;
    if (any_misaligned({dt_chunk, cs}) || any_misaligned4({dt, A})) return SSD_ERR_ALIGN;
    return hip_status(ssd::launch_chunk_cumsum(s, dt, A, dt_chunk, cs, (hipStream_t)stream));
}

ssd_status ssd_chunk_state(const ssd_dims* dims, ssd_dtype dtype, int chunk_len, const void* x,
                           const void* B, const float* dt_chunk, const float* cs, void* states,
                           const void* C, void* gram, void* stream) {
    Shape s;
    ssd_status r = make_shape(dims, chunk_len, &s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if ((size_t)s.B * s.T > 0 && (!x || !B || !dt_chunk || !cs || !states)) return SSD_ERR_NULL;
    const bool want_gram = gram != nullptr && uses_gram(s, dtype);
    if ((size_t)s.B * s.T > 0 && want_gram && !C) return SSD_ERR_NULL;
    if (any_misaligned({x, B, dt_chunk, cs, states, C, gram})) return SSD_ERR_ALIGN;
    return run_chunk_state(s, dtype, x, B, dt_chunk, cs, states, want_gram ? C : nullptr,
                           want_gram ? gram : nullptr, (hipStream_t)stream);
}

ssd_status ssd_state_passing(const ssd_dims* dims, ssd_dtype dtype, int chunk_len,
                             const void* states, const float* cs, const float* init_state,
                             void* entry_states, float* final_state, void* stream) {
    Shape s;
    ssd_status r = make_shape(dims, chunk_len, &s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if ((size_t)s.B * s.T > 0 && (!states || !cs || !entry_states)) return SSD_ERR_NULL;
    if (any_misaligned({states, cs, entry_states}) || any_misaligned4({init_state, final_state}))
        return SSD_ERR_ALIGN;
    if (states && (const void*)states == entry_states && s.nC > 0) return SSD_ERR_DIMS;
    return hip_status(ssd::launch_state_passing(s, dtype, states, cs, init_state, entry_states,
                                                final_state, (hipStream_t)stream));
}

size_t ssd_chunk_gram_size(const ssd_dims* dims, ssd_dtype dtype, int chunk_len) {
    Shape s;
    if (make_shape(dims, chunk_len, &s) != SSD_OK || !valid_dtype(dtype)) return 0;
    return uses_gram(s, dtype) ? ssd::chunk_gram_bytes(s) : 0;
}

ssd_status ssd_chunk_gram(const ssd_dims* dims, ssd_dtype dtype, int chunk_len, const void* B,
                          const void* C, void* gram, void* stream) {
    Shape s;
    ssd_status r = make_shape(dims, chunk_len, &s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if (!uses_gram(s, dtype) || (size_t)s.B * s.T == 0) return SSD_OK;  // nothing to compute
    if (!B || !C || !gram) return SSD_ERR_NULL;
    if (any_misaligned({B, C, gram})) return SSD_ERR_ALIGN;
    return hip_status(ssd::launch_chunk_gram(s, B, C, gram, (hipStream_t)stream));
}

ssd_status ssd_chunk_scan(const ssd_dims* dims, ssd_dtype dtype, int chunk_len, const void* x,
                          const void* B, const void* C, const float* dt_chunk, const float* cs,
                          const float* D, const void* entry_states, const void* gram, void* y,
                          void* stream) {
    Shape s;
    ssd_status r = make_shape(dims, chunk_len, &s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if ((size_t)s.B * s.T > 0 && (!x || !B || !C || !dt_chunk || !cs || !D || !entry_states || !y))
        return SSD_ERR_NULL;
    if ((size_t)s.B * s.T > 0 && uses_gram(s, dtype) && !gram) return SSD_ERR_NULL;
    if (any_misaligned({x, B, C, dt_chunk, cs, entry_states, gram, y}) || any_misaligned4({D}))
        return SSD_ERR_ALIGN;
    return run_chunk_scan(s, dtype, x, B, C, dt_chunk, cs, D, entry_states, gram, y,
                          (hipStream_t)stream);
}

}  // extern "C"

// ssd_fwd_noalloc's stage buffers: one array per GPU, in the code object, allocated by the
// runtime when the library's code is loaded on that GPU and held until the process ends.
// On the host, `scratch` names only a stand-in: its device address comes from
// hipGetSymbolAddress, once per device with that device current, and is kept per device
// (scratch_of_current_device).  The stage kernels fully write every buffer before they read
// it, so nothing in it needs clearing between calls.
static __device__ __align__(256) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];

namespace {
// Arguments of ssd_fwd other than the workspace: checked, and the shape made.
ssd_status fwd_check(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                     const float* A, const void* B, const void* C, const float* D, int chunk_len,
                     const float* init_state, const void* y, const float* final_state, Shape* s) {
    ssd_status r = make_shape(dims, chunk_len, s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    const bool has_tokens = (size_t)s->B * s->T > 0;
    if (has_tokens && (!x || !dt || !A || !B || !C || !D || !y)) return SSD_ERR_NULL;
    if (any_misaligned({x, B, C, y}) || any_misaligned4({dt, A, D, init_state, final_state}))
        return SSD_ERR_ALIGN;
    return SSD_OK;
}

// The forward's launches, on the stage buffers of ws.  raw (optional): the step sizes are
// made from raw projection rows inside the cumsum pass instead of being read from dt.
ssd_status fwd_run(const Shape& s, ssd_dtype dtype, const void* x, const float* dt,
                   const float* A, const void* B, const void* C, const float* D,
                   const float* init_state, void* y, float* final_state, const Workspace& ws,
                   hipStream_t st, const ssd::DtRaw* raw = nullptr,
                   const ssd::GateNorm* gate = nullptr) {
    ssd_status r;
    const bool has_tokens = (size_t)s.B * s.T > 0;
    if (s.B == 0) return SSD_OK;
    if (has_tokens) {
        r = hip_status(ssd::launch_chunk_cumsum(s, dt, A, ws.dtc, ws.cs, st, nullptr, 0, raw));
        if (r != SSD_OK) return r;
        r = run_chunk_state(s, dtype, x, B, ws.dtc, ws.cs, ws.states, C, ws.gram, st);
        if (r != SSD_OK) return r;
    }
    // with T == 0 this only copies init_state (or zeros) to final_state
    r = hip_status(ssd::launch_state_passing(s, dtype, ws.states, ws.cs, init_state, ws.entry,
                                             final_state, st));
    if (r != SSD_OK || !has_tokens) return r;
    return run_chunk_scan(s, dtype, x, B, C, ws.dtc, ws.cs, D, ws.entry, ws.gram, y, st, gate);
}

// ---- scratch for callers that cannot allocate ------------------------------------------
std::atomic<void*> scratch_addr[ssd::kMaxDevices];  // per device: the address of `scratch`

ssd_status scratch_of_current_device(void** out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    if (dev < 0 || dev >= ssd::kMaxDevices) return SSD_ERR_HIP;
    void* p = scratch_addr[dev].load(std::memory_order_acquire);
    if (!p) {
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return SSD_ERR_HIP;
        scratch_addr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return SSD_OK;
}

// The stage buffers packed tightly for the scratch array: the chunk and entry states take
// the input dtype's size (ssd_fwd's workspace reserves fp32 for either dtype).
size_t tight_workspace_bytes(const Shape& s, ssd_dtype dtype, Workspace* w, char* base) {
    const size_t chunk_elems = (size_t)s.B * s.H * s.nC * s.Q;
    const size_t state_bytes = (size_t)s.B * s.H * s.nC * s.P * s.N * (dtype == SSD_BF16 ? 2 : 4);
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += round_up(bytes);
        return (float*)p;
    };
    Workspace ws;
    ws.dtc = take(chunk_elems * sizeof(float));
    ws.cs = take(chunk_elems * sizeof(float));
    ws.states = take(state_bytes);
    ws.entry = take(state_bytes);
    ws.gram = take(uses_gram(s, dtype) ? ssd::chunk_gram_bytes(s) : 0);
    if (w) *w = ws;
    return off;
}
}  // namespace

extern "C" {

ssd_status ssd_fwd(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                   const float* A, const void* B, const void* C, const float* D, int chunk_len,
                   const float* init_state, void* y, float* final_state, void* workspace,
                   size_t workspace_bytes_given, void* stream) {
    Shape s;
    ssd_status r = fwd_check(dims, dtype, x, dt, A, B, C, D, chunk_len, init_state, y,
                             final_state, &s);
    if (r != SSD_OK) return r;
    if (any_misaligned({workspace})) return SSD_ERR_ALIGN;
    Workspace ws;
    const size_t need = workspace_bytes(s, &ws, (char*)workspace);
    if (need > 0 && (!workspace || workspace_bytes_given < need)) return SSD_ERR_WORKSPACE;
    return fwd_run(s, dtype, x, dt, A, B, C, D, init_state, y, final_state, ws,
                   (hipStream_t)stream);
}

ssd_status ssd_fwd_noalloc(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                           const float* A, const void* B, const void* C, const float* D,
                           int chunk_len, const float* init_state, void* y, float* final_state,
                           void* stream) {
    Shape s;
    ssd_status r = fwd_check(dims, dtype, x, dt, A, B, C, D, chunk_len, init_state, y,
                             final_state, &s);
    if (r != SSD_OK) return r;
    if (tight_workspace_bytes(s, dtype, nullptr, nullptr) > (size_t)SSD_NOALLOC_SCRATCH_BYTES)
        return SSD_ERR_WORKSPACE;
    if (s.B == 0) return SSD_OK;
    void* base = nullptr;
    r = scratch_of_current_device(&base);
    if (r != SSD_OK) return r;
    Workspace ws;
    tight_workspace_bytes(s, dtype, &ws, (char*)base);
    return fwd_run(s, dtype, x, dt, A, B, C, D, init_state, y, final_state, ws,
                   (hipStream_t)stream);
}

size_t ssd_bwd_workspace_size(const ssd_dims* dims, int chunk_len) {
    Shape s;
    if (make_shape(dims, chunk_len, &s) != SSD_OK) return 0;
    return bwd_workspace_bytes(s, nullptr, nullptr);
}

}  // extern "C"

namespace {
// fwd_ws: the workspace of an ssd_fwd call on the same inputs (its log decays and entry
// states are read instead of recomputed), or null
ssd_status bwd_impl(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                    const float* A, const void* B, const void* C, const float* D, int chunk_len,
                    const float* init_state, const void* dy, const float* d_final,
                    const void* fwd_ws, void* dx, float* ddt, float* dA, void* dB, void* dC,
                    float* dD, float* d_init, void* workspace, size_t workspace_bytes_given,
                    void* stream) {
    Shape s;
    ssd_status r = make_shape(dims, chunk_len, &s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    const bool has_tokens = (size_t)s.B * s.T > 0;
    if (!dA || !dD) return SSD_ERR_NULL;
    if (has_tokens && (!x || !dt || !A || !B || !C || !D || !dy || !dx || !ddt || !dB || !dC))
        return SSD_ERR_NULL;
    if (any_misaligned({x, B, C, dy, dx, dB, dC, workspace, fwd_ws}) ||
        any_misaligned4({dt, A, D, init_state, d_final, ddt, dA, dD, d_init}))
        return SSD_ERR_ALIGN;
    BwdWorkspace ws;
    const size_t need = bwd_workspace_bytes(s, &ws, (char*)workspace);
    if (need > 0 && (!workspace || workspace_bytes_given < need)) return SSD_ERR_WORKSPACE;
    if (fwd_ws) {  // the forward's own log decays and entry states
        Workspace fws;
        workspace_bytes(s, &fws, (char*)const_cast<void*>(fwd_ws));
        ws.dtc = fws.dtc;
        ws.cs = fws.cs;
        ws.entry = fws.entry;
    }
    hipStream_t st = (hipStream_t)stream;
    const bool mfma_state = dtype == SSD_BF16 && ssd::chunk_state_mfma_supported(s);
    if (has_tokens) {
        if (!fwd_ws) {
            // the forward intermediates: log decays, chunk states, entry states
            r = hip_status(ssd::launch_chunk_cumsum(s, dt, A, ws.dtc, ws.cs, st));
            if (r != SSD_OK) return r;
            r = run_chunk_state(s, dtype, x, B, ws.dtc, ws.cs, ws.states, nullptr, nullptr, st);
            if (r != SSD_OK) return r;
            r = hip_status(ssd::launch_state_passing(s, dtype, ws.states, ws.cs, init_state,
                                                     ws.entry, nullptr, st));
            if (r != SSD_OK) return r;
        }
        // the entry-state gradient of every chunk through its own outputs (into the chunk
        // state buffer, no longer needed)
        r = hip_status(mfma_state
                           ? ssd::launch_chunk_dstate_mfma(s, dy, C, ws.cs, ws.states, st)
                           : ssd::launch_chunk_dstate_valu(s, dtype, dy, C, ws.cs, ws.states, st));
        if (r != SSD_OK) return r;
    }
    // carried backwards over the chunks; with T == 0 this copies d_final (or zeros) to d_init
    r = hip_status(ssd::launch_state_passing_rev(s, dtype, ws.states, ws.cs, d_final, ws.exitg,
                                                 d_init, st));
    if (r != SSD_OK) return r;
    ssd::BwdArgs a;
    a.x = x; a.Bm = B; a.Cm = C; a.dy = dy;
    a.dtc = ws.dtc; a.cs = ws.cs; a.A = A; a.D = D;
    a.entry = ws.entry; a.exitg = ws.exitg;
    a.dx = dx; a.dB = dB; a.dC = dC;
    a.ddt = ddt; a.dA = dA; a.dD = dD;
    a.dcs = ws.dcs; a.direct = ws.direct;
    a.lt_part = ws.lt_part; a.dd_part = ws.dd_part; a.dA_part = ws.dA_part;
    a.xfb = ws.xfb; a.dBs = ws.dBs; a.dCs = ws.dCs;
    const bool mfma_bwd = dtype == SSD_BF16 && ssd::chunk_bwd_mfma_supported(s);
    a.xs = mfma_bwd ? ws.xs : nullptr;
    const int rows = mfma_bwd ? ssd::chunk_bwd_mfma_rows() : ssd::chunk_bwd_valu_rows();
    if (has_tokens) {
        r = hip_status(mfma_bwd ? ssd::launch_chunk_bwd_mfma(s, a, st)
                                : ssd::launch_chunk_bwd_valu(s, dtype, a, st));
        if (r != SSD_OK) return r;
    }
    // dA and dD are written even with no tokens (zeros)
    return hip_status(ssd::launch_bwd_finalize(s, a, rows, st));
}
}  // namespace

extern "C" {

ssd_status ssd_bwd(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                   const float* A, const void* B, const void* C, const float* D, int chunk_len,
                   const float* init_state, const void* dy, const float* d_final, void* dx,
                   float* ddt, float* dA, void* dB, void* dC, float* dD, float* d_init,
                   void* workspace, size_t workspace_bytes_given, void* stream) {
    return bwd_impl(dims, dtype, x, dt, A, B, C, D, chunk_len, init_state, dy, d_final, nullptr,
                    dx, ddt, dA, dB, dC, dD, d_init, workspace, workspace_bytes_given, stream);
}

ssd_status ssd_bwd_saved(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                         const float* A, const void* B, const void* C, const float* D,
                         int chunk_len, const float* init_state, const void* dy,
                         const float* d_final, const void* fwd_workspace, void* dx, float* ddt,
                         float* dA, void* dB, void* dC, float* dD, float* d_init,
                         void* workspace, size_t workspace_bytes_given, void* stream) {
    if (!fwd_workspace) return SSD_ERR_NULL;
    return bwd_impl(dims, dtype, x, dt, A, B, C, D, chunk_len, init_state, dy, d_final,
                    fwd_workspace, dx, ddt, dA, dB, dC, dD, d_init, workspace,
                    workspace_bytes_given, stream);
}

ssd_status ssd_decode_step(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                           const float* A, const void* B, const void* C, const float* D,
                           float* state, void* y, void* stream) {
    if (!dims) return SSD_ERR_NULL;
    ssd_dims one = *dims;
    one.seqlen = 1;  // the sizes are checked as for a one-step sequence
    Shape s;
    ssd_status r = make_shape(&one, 64, &s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if (s.B == 0) return SSD_OK;
    if (!x || !dt || !A || !B || !C || !D || !state || !y) return SSD_ERR_NULL;
    if (any_misaligned({x, state}) || any_misaligned4({dt, A, B, C, D, y})) return SSD_ERR_ALIGN;
    return hip_status(ssd::launch_decode_step(s, dtype, x, dt, A, B, C, D, state, y,
                                              (hipStream_t)stream));
}

// ---- the block around the layer -----------------------------------------------------

static bool aligned_elem(const void* p, ssd_dtype dtype) {
    return ((uintptr_t)p & (dtype == SSD_BF16 ? 1u : 3u)) == 0;
}

ssd_status ssd_block_prologue(const ssd_dims* dims, ssd_dtype dtype, const void* xbc,
                              int64_t xbc_stride, const float* conv_w, const float* conv_b,
                              int conv_k, const void* dt_raw, int64_t dt_stride,
                              const float* dt_bias, void* x, void* B, void* C, float* dt,
                              void* stream) {
    Shape s;
    ssd_status r = make_shape(dims, 64, &s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype) || conv_k < 1 || conv_k > 8) return SSD_ERR_UNSUPPORTED;
    const int64_t cdim = (int64_t)s.H * s.P + 2 * (int64_t)s.G * s.N;
    if (xbc_stride < cdim || dt_stride < s.H) return SSD_ERR_DIMS;
    if (!product_fits({s.B, s.T, xbc_stride}) || !product_fits({s.B, s.T, dt_stride}))
        return SSD_ERR_DIMS;
    if ((size_t)s.B * s.T == 0) return SSD_OK;
    if (!xbc || !conv_w || !dt_raw || !x || !B || !C || !dt) return SSD_ERR_NULL;
    if (any_misaligned({x, B, C}) || any_misaligned4({conv_w, conv_b, dt_bias, dt}) ||
        !aligned_elem(xbc, dtype) || !aligned_elem(dt_raw, dtype))
        return SSD_ERR_ALIGN;
    ssd::BlockPrologueArgs a;
    a.xbc = xbc; a.xbc_stride = xbc_stride;
    a.conv_w = conv_w; a.conv_b = conv_b; a.conv_k = conv_k;
    a.dt_raw = dt_raw; a.dt_stride = dt_stride; a.dt_bias = dt_bias;
    a.x = x; a.Bm = B; a.Cm = C; a.dt = dt;
    return hip_status(ssd::launch_block_prologue(s, dtype, a, (hipStream_t)stream));
}

ssd_status ssd_block_epilogue(const ssd_dims* dims, ssd_dtype dtype, const void* y,
                              const void* z, int64_t z_stride, const float* norm_w,
                              const float* norm_b, int norm_groups, int rms, float eps,
                              void* out, void* stream) {
    Shape s;
    ssd_status r = make_shape(dims, 64, &s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    const int64_t d = (int64_t)s.H * s.P;
    if (norm_groups < 1 || d % norm_groups != 0 || z_stride < d || !(eps >= 0.f) ||
        !product_fits({s.B, s.T, z_stride}))
        return SSD_ERR_DIMS;
    if ((size_t)s.B * s.T == 0) return SSD_OK;
    if (!y || !z || !norm_w || !out) return SSD_ERR_NULL;
    if (any_misaligned({y, out}) || any_misaligned4({norm_w, norm_b}) ||
        !aligned_elem(z, dtype))
        return SSD_ERR_ALIGN;
    ssd::BlockEpilogueArgs a;
    a.y = y; a.z = z; a.z_stride = z_stride;
    a.norm_w = norm_w; a.norm_b = norm_b;
    a.groups = norm_groups; a.rms = rms ? 1 : 0; a.eps = eps;
    a.out = out;
    return hip_status(ssd::launch_block_epilogue(s, dtype, a, (hipStream_t)stream));
}

namespace {
struct BlockWorkspace {
    void *x, *B, *C, *y;
    char* fwd;
    size_t fwd_bytes;
};

// Norm groups per head where ssd_block_fwd applies the gate and the norm in the chunk scan
// (each group S = H P / norm_groups channels inside one head, S a multiple of 16 dividing
// P, bf16 on the matrix-core scan, 8-byte aligned projection rows), else 0.
int norm_groups_per_head(const Shape& s, ssd_dtype dtype, int norm_groups) {
    const int64_t d = (int64_t)s.H * s.P;
    if (dtype != SSD_BF16 || norm_groups < 1 || d % norm_groups != 0) return 0;
    const int64_t gsize = d / norm_groups;
    if (gsize % 16 != 0 || s.P % gsize != 0) return 0;
    const int gph = (int)(s.P / gsize);
    const int64_t width = 2 * d + 2 * (int64_t)s.G * s.N + s.H;
    // the scan addresses a chunk of z rows with 32-bit byte offsets
    if ((width * 2) % 8 != 0 || (int64_t)s.Q * width * 2 >= ((int64_t)1 << 31) ||
        !uses_gram(s, dtype) || !ssd::chunk_scan_gate_supported(s, gph))
        return 0;
    return gph;
}

size_t block_workspace_bytes(const Shape& s, ssd_dtype dtype, BlockWorkspace* w, char* base) {
    const size_t e = dtype == SSD_BF16 ? 2 : 4;
    const size_t bt = (size_t)s.B * s.T;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char* p = base ? base + off : nullptr;
        off += round_up(bytes);
        return p;
    };
    BlockWorkspace ws;
    ws.x = take(bt * s.H * s.P * e);
    ws.y = take(bt * s.H * s.P * e);
    ws.B = take(bt * s.G * s.N * e);
    ws.C = take(bt * s.G * s.N * e);
    ws.fwd_bytes = workspace_bytes(s, nullptr, nullptr);
    ws.fwd = take(ws.fwd_bytes);
    if (w) *w = ws;
    return off;
}
}  // namespace

int ssd_block_fwd_norm_in_scan(const ssd_dims* dims, ssd_dtype dtype, int chunk_len,
                               int norm_groups) {
    Shape s;
    if (make_shape(dims, chunk_len, &s) != SSD_OK || !valid_dtype(dtype)) return 0;
    return norm_groups_per_head(s, dtype, norm_groups) > 0 ? 1 : 0;
}

size_t ssd_block_fwd_workspace_size(const ssd_dims* dims, ssd_dtype dtype, int chunk_len) {
    Shape s;
    if (make_shape(dims, chunk_len, &s) != SSD_OK || !valid_dtype(dtype)) return 0;
    return block_workspace_bytes(s, dtype, nullptr, nullptr);
}

ssd_status ssd_block_fwd(const ssd_dims* dims, ssd_dtype dtype, const void* zxbcdt,
                         const float* conv_w, const float* conv_b, int conv_k,
                         const float* dt_bias, const float* A, const float* D, int chunk_len,
                         const float* init_state, const float* norm_w, const float* norm_b,
                         int norm_groups, int rms, float eps, void* out, float* final_state,
                         void* workspace, size_t workspace_bytes_given, void* stream) {
    Shape s;
    ssd_status r = make_shape(dims, chunk_len, &s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype) || conv_k < 1 || conv_k > 8) return SSD_ERR_UNSUPPORTED;
    const int64_t d = (int64_t)s.H * s.P, gn = (int64_t)s.G * s.N;
    const int64_t width = 2 * d + 2 * gn + s.H;
    if (norm_groups < 1 || d % norm_groups != 0 || !(eps >= 0.f) ||
        !product_fits({s.B, s.T, width}))
        return SSD_ERR_DIMS;
    const bool has_tokens = (size_t)s.B * s.T > 0;
    if (has_tokens && (!zxbcdt || !conv_w || !A || !D || !norm_w || !out)) return SSD_ERR_NULL;
    if (any_misaligned({zxbcdt, out, workspace}) ||
        any_misaligned4({conv_w, conv_b, dt_bias, A, D, init_state, norm_w, norm_b,
                         final_state}))
        return SSD_ERR_ALIGN;
    BlockWorkspace ws;
    const size_t need = block_workspace_bytes(s, dtype, &ws, (char*)workspace);
    if (need > 0 && (!workspace || workspace_bytes_given < need)) return SSD_ERR_WORKSPACE;
    const size_t e = dtype == SSD_BF16 ? 2 : 4;
    const char* zx = (const char*)zxbcdt;
    hipStream_t st = (hipStream_t)stream;
    Workspace fws;
    workspace_bytes(s, &fws, ws.fwd);
    if (!has_tokens)  // only copies init_state (or zeros) to final_state
        return fwd_run(s, dtype, nullptr, nullptr, A, nullptr, nullptr, D, init_state, nullptr,
                       final_state, fws, st);
    // the convolution and SiLU of x, B and C; the step sizes are made in the cumsum pass
    ssd::BlockPrologueArgs pa;
    pa.xbc = zx + d * e; pa.xbc_stride = width;
    pa.conv_w = conv_w; pa.conv_b = conv_b; pa.conv_k = conv_k;
    pa.dt_raw = nullptr; pa.dt_stride = width; pa.dt_bias = nullptr;
    pa.x = ws.x; pa.Bm = ws.B; pa.Cm = ws.C; pa.dt = nullptr;
    r = hip_status(ssd::launch_block_prologue(s, dtype, pa, st));
    if (r != SSD_OK) return r;
    const ssd::DtRaw raw{zx + (2 * d + 2 * gn) * e, width, dt_bias, dtype};
    // norm groups inside a head: the gate and the norm in the chunk scan's store, which
    // writes `out` (y is never stored and no epilogue pass runs)
    const int gph = norm_groups_per_head(s, dtype, norm_groups);
    if (gph > 0 && !any_misaligned({norm_w, norm_b})) {
        const ssd::GateNorm gate{zxbcdt, width, norm_w, norm_b, gph, rms, eps};
        return fwd_run(s, dtype, ws.x, nullptr, A, ws.B, ws.C, D, init_state, out, final_state,
                       fws, st, &raw, &gate);
    }
    r = fwd_run(s, dtype, ws.x, nullptr, A, ws.B, ws.C, D, init_state, ws.y, final_state, fws, st,
                &raw);
    if (r != SSD_OK) return r;
    return ssd_block_epilogue(dims, dtype, ws.y, zxbcdt, width, norm_w, norm_b, norm_groups,
                              rms, eps, out, stream);
}

// ---- packed variable-length rows ------------------------------------------------------

size_t ssd_fwd_varlen_workspace_size(const ssd_dims* dims, int chunk_len) {
    Shape s;
    if (make_shape(dims, chunk_len, &s) != SSD_OK || dims->batch != 1) return 0;
    return workspace_bytes(s, nullptr, nullptr);
}

ssd_status ssd_fwd_varlen(const ssd_dims* dims, ssd_dtype dtype, const void* x, const float* dt,
                          const float* A, const void* B, const void* C, const float* D,
                          int chunk_len, const int32_t* cu_seqlens, int64_t nseq, void* y,
                          float* final_states, void* workspace, size_t workspace_bytes_given,
                          void* stream) {
    Shape s;
    ssd_status r = make_shape(dims, chunk_len, &s);
    if (r != SSD_OK) return r;
    if (!valid_dtype(dtype)) return SSD_ERR_UNSUPPORTED;
    if (dims->batch != 1 || nseq < 1 || nseq >= ((int64_t)1 << 30)) return SSD_ERR_DIMS;
    const bool has_tokens = s.T > 0;
    if (!cu_seqlens) return SSD_ERR_NULL;
    if (has_tokens && (!x || !dt || !A || !B || !C || !D || !y)) return SSD_ERR_NULL;
    if (any_misaligned({x, B, C, y, workspace}) ||
        any_misaligned4({dt, A, D, cu_seqlens, final_states}))
        return SSD_ERR_ALIGN;
    Workspace ws;
    const size_t need = workspace_bytes(s, &ws, (char*)workspace);
    if (need > 0 && (!workspace || workspace_bytes_given < need)) return SSD_ERR_WORKSPACE;
    hipStream_t st = (hipStream_t)stream;
    const int ns = (int)nseq;
    if (has_tokens) {
        r = hip_status(ssd::launch_chunk_cumsum(s, dt, A, ws.dtc, ws.cs, st, cu_seqlens, ns));
        if (r != SSD_OK) return r;
        r = run_chunk_state(s, dtype, x, B, ws.dtc, ws.cs, ws.states, C, ws.gram, st);
        if (r != SSD_OK) return r;
        r = hip_status(ssd::launch_state_passing(s, dtype, ws.states, ws.cs, nullptr, ws.entry,
                                                 nullptr, st));
        if (r != SSD_OK) return r;
        r = run_chunk_scan(s, dtype, x, B, C, ws.dtc, ws.cs, D, ws.entry, ws.gram, y, st);
        if (r != SSD_OK) return r;
    }
    if (!final_states) return SSD_OK;
    if (dtype == SSD_BF16 && has_tokens && ssd::varlen_final_mfma_supported(s))
        return hip_status(ssd::launch_varlen_final_mfma(s, x, B, ws.dtc, ws.cs, ws.entry,
                                                        cu_seqlens, ns, final_states, st));
    return hip_status(ssd::launch_varlen_final(s, dtype, x, B, ws.dtc, ws.cs, ws.entry,
                                               cu_seqlens, ns, final_states, st));
}

}  // extern "C"
