// The decode step for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
// mla_sparse_decode_noalloc runs the same kernels as mla_get_sched_meta +
// mla_sparse_decode_fwd + mla_splitkv_combine, with the plan records, the
// split prefix and the split partials in one file-scope device array instead
// of caller buffers.
//
// The array is `scratch` below (64 MiB).  Each GPU the library runs on holds
// its own copy until the process ends.  Host code never uses the array's name
// as an address: on the first call on a device (with that device current)
// hipGetSymbolAddress gives that device's address, which is kept per device
// and passed to the kernels like any workspace pointer.  Every call on a GPU
// shares that GPU's array, so calls that overlap on one GPU (different
// streams, or host threads) race; calls on one stream are ordered.  Nothing a
// call leaves in the array is read by the next: the plan is rewritten (or
// evaluated in closed form), and every split partial and its lse are written
// by the decode before the combine reads them, so no clearing is needed.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "mla.h"
#include "mla_internal.h"

namespace mla {
int host_fail(int code, const char* msg);
int host_hip_status(hipError_t e, const char* what);
int check_decode_args_noalloc(const mla_decode_args* a, ResolvedShape* rs, DecodeParams* p);
}  // namespace mla

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;

static __device__ __attribute__((aligned(256))) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Device address of `scratch` on the current device (looked up once per device).
int scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return mla::host_hip_status(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return mla::host_fail(MLA_ERR_UNSUPPORTED, "device index beyond 63");
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_dev[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return mla::host_hip_status(e, "hipGetSymbolAddress(scratch)");
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return MLA_OK;
}

}  // namespace

extern "C" int mla_sparse_decode_noalloc(const mla_decode_args* args, void* stream) {
    mla::ResolvedShape r;
    mla::DecodeParams p;
    int st = mla::check_decode_args_noalloc(args, &r, &p);
    if (st != MLA_OK) return st;
    // Array layout: [plan records][split prefix] (only with a per-request
    // cost; with none the kernels evaluate the plan in closed form), then the
    // split partials (packed bf16, 128 KB per split and query column, for the
    // cache formats alike) and their base-2 lse.
    const bool sched = r.overhead != 0;
    const size_t meta_b = sched ? align256((size_t)r.num_parts * sizeof(mla_sched_part)) : 0;
    const size_t prefix_b = sched ? align256((size_t)(r.b + 1) * sizeof(int32_t)) : 0;
    const size_t splits = (size_t)(r.b + r.num_parts) * r.s_q;     // pieces are at most b + num_parts
    const size_t o_b = align256(splits * 128 * 512 * 2);
    const size_t l_b = align256(splits * r.h_q * sizeof(float));
    const size_t need = meta_b + prefix_b + o_b + l_b;
    if (need > kScratchBytes) {
        char msg[160];
        snprintf(msg, sizeof msg, "this shape needs %zu bytes of split workspace; the no-allocation array holds %zu",
                 need, kScratchBytes);
        return mla::host_fail(MLA_ERR_WORKSPACE, msg);
    }
    void* base = nullptr;
    st = scratch_address(&base);
    if (st != MLA_OK) return st;
    uint8_t* b = static_cast<uint8_t*>(base);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (sched) {
        int32_t* meta = reinterpret_cast<int32_t*>(b);
        int32_t* prefix = reinterpret_cast<int32_t*>(b + meta_b);
        st = mla::host_hip_status(mla::launch_sched(r, nullptr, meta, prefix, s), "sched kernel launch");
        if (st != MLA_OK) return st;
        p.sched_meta = meta;
        p.num_splits = prefix;
    }
    p.o_accum = reinterpret_cast<float*>(b + meta_b + prefix_b);
    p.lse_accum = reinterpret_cast<float*>(b + meta_b + prefix_b + o_b);
    st = mla::host_hip_status(mla::launch_decode(p, r.kv_format, r.num_parts, s), "decode kernel launch");
    if (st != MLA_OK) return st;
    return mla::host_hip_status(mla::launch_combine(p, s), "combine kernel launch");
}
