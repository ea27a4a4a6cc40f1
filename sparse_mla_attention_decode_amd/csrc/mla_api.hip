// Host side of libmla: argument validation, default resolution, scheduler
// export and kernel launches behind the C ABI declared in include/mla.h.
// Validation happens before anything touches the device, so every error path
// can be exercised without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "mla.h"
#include "mla_internal.h"
#include "indexer_internal.h"
#include "sched_plan.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = '\0';
    return MLA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validate `in` and fill `out` with every default resolved.
int resolve(const mla_shape* in, mla::ResolvedShape* out) {
    if (!in) return fail(MLA_ERR_INVALID_ARG, "shape is NULL");
    const mla_shape& s = *in;
    if (s.b < 1) return fail(MLA_ERR_INVALID_ARG, "b must be >= 1 (got %d)", s.b);
    if (s.s_q < 1) return fail(MLA_ERR_INVALID_ARG, "s_q must be >= 1 (got %d)", s.s_q);
    if (s.s_q > 65535) return fail(MLA_ERR_INVALID_ARG, "s_q must be <= 65535 (got %d)", s.s_q);
    if ((int64_t)s.b * s.s_q > (1 << 24))
        return fail(MLA_ERR_INVALID_ARG, "b * s_q must be <= 2^24 (got %lld)", (long long)s.b * s.s_q);
    if (s.topk < 1) return fail(MLA_ERR_INVALID_ARG, "topk must be >= 1 (got %d)", s.topk);
    if (s.h_q < 1) return fail(MLA_ERR_INVALID_ARG, "h_q must be >= 1 (got %d)", s.h_q);
    if (s.h_q != 64 && s.h_q != 128) return fail(MLA_ERR_UNSUPPORTED, "h_q must be 64 or 128 (got %d)", s.h_q);
    if (s.h_kv != 1) return fail(MLA_ERR_UNSUPPORTED, "h_kv must be 1 (got %d)", s.h_kv);
    if (s.kv_format != MLA_KV_FP8_656 && s.kv_format != MLA_KV_BF16_576 && s.kv_format != MLA_KV_V4_584 &&
        s.kv_format != MLA_KV_V41_528)
        return fail(MLA_ERR_INVALID_ARG, "unknown kv_format %d", s.kv_format);
    const bool model1 = s.kv_format == MLA_KV_V4_584 || s.kv_format == MLA_KV_V41_528;
    if (s.d_qk != (model1 ? 512 : 576))
        return fail(MLA_ERR_UNSUPPORTED, "d_qk must be %d for this kv_format (got %d)", model1 ? 512 : 576, s.d_qk);
    if (s.d_v != 512) return fail(MLA_ERR_UNSUPPORTED, "d_v must be 512 (got %d)", s.d_v);
    if (s.num_kv_tokens < 1 || s.num_kv_tokens > INT32_MAX)
        return fail(MLA_ERR_INVALID_ARG, "num_kv_tokens must be in [1, 2^31) (got %lld)",
                    (long long)s.num_kv_tokens);
    int P = 1;
    if (s.kv_format != MLA_KV_BF16_576) {                    // paged formats
        P = s.page_block_size;
        if (P < 1) return fail(MLA_ERR_INVALID_ARG, "page_block_size must be >= 1 (got %d)", P);
        if (s.num_kv_tokens % P != 0)
            return fail(MLA_ERR_INVALID_ARG, "num_kv_tokens (%lld) is not a multiple of page_block_size (%d)",
                        (long long)s.num_kv_tokens, P);
    }
    int block = s.split_granularity == 0 ? 64 : s.split_granularity;
    if (block < 32 || block % 32 != 0)
        return fail(MLA_ERR_INVALID_ARG, "split_granularity must be a positive multiple of 32 (got %d)",
                    s.split_granularity);
    if ((int64_t)s.b * ((s.topk + block - 1) / block) >= (int64_t)1 << 30)
        return fail(MLA_ERR_INVALID_ARG, "b * ceil(topk / split_granularity) must be below 2^30");
    int overhead = s.fixed_overhead < 0 ? 5 : s.fixed_overhead;
    if (overhead > (1 << 20)) return fail(MLA_ERR_INVALID_ARG, "fixed_overhead too large (%d)", overhead);
    int parts = s.num_parts;
    if (parts < 0) return fail(MLA_ERR_INVALID_ARG, "num_parts must be >= 0 (got %d)", parts);
    if (parts == 0) {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) {
            (void)hipGetLastError();
            return fail(MLA_ERR_NO_DEVICE, "num_parts = 0 needs a device to read its CU count");
        }
        // the decode kernel (128-head layout for 64 or 128 heads, every cache
        // format) needs all of a CU's LDS: one work-group per CU
        parts = cus / s.s_q;
        if (parts < 1) parts = 1;
    }
    if (parts > 65535) return fail(MLA_ERR_INVALID_ARG, "num_parts must be <= 65535 (got %d)", parts);
    out->b = s.b;
    out->s_q = s.s_q;
    out->h_q = s.h_q;
    out->topk = s.topk;
    out->page_block_size = P;
    out->kv_format = s.kv_format;
    out->num_kv_tokens = s.num_kv_tokens;
    out->num_parts = parts;
    out->block = block;
    out->overhead = overhead;
    return MLA_OK;
}

void workspace_bytes(const mla::ResolvedShape& r, size_t* o, size_t* l) {
    const size_t rows = (size_t)(r.b + r.num_parts) * r.s_q * r.h_q;
    if (o) *o = rows * 512 * sizeof(float);
    if (l) *l = rows * sizeof(float);
}

// Validate `a` and fill the kernel parameters.  With caller_buffers false (the
// no-allocation entry point) the plan and workspace pointers must be NULL:
// the library's own array supplies them afterwards.
// need_indices: the sparse decode reads them; the combine does not, and dense
// decode takes a block table instead (it checks that indices is NULL itself).
int check_decode_args(const mla_decode_args* a, mla::ResolvedShape* rs, mla::DecodeParams* p,
                      bool caller_buffers = true, bool need_indices = true) {
    if (!a) return fail(MLA_ERR_INVALID_ARG, "args is NULL");
    int st = resolve(&a->shape, rs);
    if (st != MLA_OK) return st;
    const mla::ResolvedShape& r = *rs;
    if (!a->q || !a->kv || (need_indices && !a->indices) || !a->out || !a->lse)
        return fail(MLA_ERR_INVALID_ARG, "q, kv, indices, out and lse must be non-NULL");
    const bool inline_plan = !a->sched_meta && !a->num_splits;
    if (!caller_buffers && (!inline_plan || a->o_accum || a->lse_accum))
        return fail(MLA_ERR_INVALID_ARG,
                    "sched_meta, num_splits, o_accum and lse_accum must be NULL: the library's array holds them");
    if (!inline_plan && (!a->sched_meta || !a->num_splits))
        return fail(MLA_ERR_INVALID_ARG, "sched_meta and num_splits must both be set (mla_get_sched_meta) or both NULL");
    if (caller_buffers && inline_plan && r.overhead != 0)
        return fail(MLA_ERR_INVALID_ARG, "a NULL plan (closed form) needs fixed_overhead 0, got %d", r.overhead);
    if ((a->attn_sink && !aligned(a->attn_sink, 4)) || (a->topk_length && !aligned(a->topk_length, 4)))
        return fail(MLA_ERR_INVALID_ARG, "attn_sink and topk_length must be 4-byte aligned");
    if (!aligned(a->q, 16) || a->q_stride_h % 8 || a->q_stride_s % 8 || a->q_stride_b % 8)
        return fail(MLA_ERR_INVALID_ARG, "q must be 16-byte aligned with strides that are multiples of 8 elements");
    const int d_qk = a->shape.d_qk;                          // 576, or 512 for V4 / V4.1 (resolve)
    if (a->q_stride_h < d_qk && r.h_q > 1)
        return fail(MLA_ERR_INVALID_ARG, "q_stride_h (%lld) < d_qk (%d)", (long long)a->q_stride_h, d_qk);
    if (!aligned(a->kv, 16) || a->kv_stride_block % 16)
        return fail(MLA_ERR_INVALID_ARG, "kv must be 16-byte aligned and kv_stride_block a multiple of 16");
    if (r.kv_format == MLA_KV_FP8_656 && a->kv_stride_block < (int64_t)r.page_block_size * 656)
        return fail(MLA_ERR_INVALID_ARG, "kv_stride_block (%lld) < page_block_size * 656",
                    (long long)a->kv_stride_block);
    if (r.kv_format == MLA_KV_V4_584 || r.kv_format == MLA_KV_V41_528) {
        const int64_t tok_b = r.kv_format == MLA_KV_V4_584 ? 584 : 528;
        if ((int64_t)r.page_block_size * tok_b >= (1ll << 31))
            return fail(MLA_ERR_INVALID_ARG, "page_block_size * %lld bytes must be below 2^31", (long long)tok_b);
        if (a->kv_stride_block < (int64_t)r.page_block_size * tok_b)
            return fail(MLA_ERR_INVALID_ARG, "kv_stride_block (%lld) < page_block_size * %lld",
                        (long long)a->kv_stride_block, (long long)tok_b);
    }
    if (r.kv_format == MLA_KV_BF16_576 && a->kv_stride_block < 1152)
        return fail(MLA_ERR_INVALID_ARG, "kv_stride_block (%lld) < 1152 bytes per bf16 row",
                    (long long)a->kv_stride_block);
    if (!aligned(a->indices, 4)) return fail(MLA_ERR_INVALID_ARG, "indices must be 4-byte aligned");
    if (!aligned(a->out, 16) || a->out_stride_h % 8 || a->out_stride_s % 8 || a->out_stride_b % 8)
        return fail(MLA_ERR_INVALID_ARG, "out must be 16-byte aligned with strides that are multiples of 8 elements");
    if (!aligned(a->lse, 4)) return fail(MLA_ERR_INVALID_ARG, "lse must be 4-byte aligned");
    if (!aligned(a->sched_meta, 4) || !aligned(a->num_splits, 4))
        return fail(MLA_ERR_INVALID_ARG, "sched_meta / num_splits must be 4-byte aligned");
    if (caller_buffers) {
        size_t need_o = 0, need_l = 0;
        workspace_bytes(r, &need_o, &need_l);
        if (!a->o_accum || !a->lse_accum || a->o_accum_bytes < need_o || a->lse_accum_bytes < need_l)
            return fail(MLA_ERR_WORKSPACE, "workspace too small: need o_accum %zu and lse_accum %zu bytes", need_o,
                        need_l);
        if (!aligned(a->o_accum, 16) || !aligned(a->lse_accum, 4))
            return fail(MLA_ERR_INVALID_ARG, "o_accum must be 16-byte aligned, lse_accum 4-byte aligned");
    }
    float sm = a->sm_scale > 0.f ? a->sm_scale : 1.0f / std::sqrt((float)d_qk);
    if (!std::isfinite(sm)) return fail(MLA_ERR_INVALID_ARG, "sm_scale must be finite");

    p->q = static_cast<const uint16_t*>(a->q);
    p->q_sb = a->q_stride_b;
    p->q_ss = a->q_stride_s;
    p->q_sh = a->q_stride_h;
    p->kv = static_cast<const uint8_t*>(a->kv);
    p->kv_block_stride = a->kv_stride_block;
    p->indices = a->indices;
    p->idx_sb = a->idx_stride_b;
    p->idx_ss = a->idx_stride_s;
    p->out = static_cast<uint16_t*>(a->out);
    p->out_sb = a->out_stride_b;
    p->out_ss = a->out_stride_s;
    p->out_sh = a->out_stride_h;
    p->lse = a->lse;
    p->sched_meta = static_cast<const int32_t*>(a->sched_meta);
    p->num_splits = a->num_splits;
    p->o_accum = a->o_accum;
    p->lse_accum = a->lse_accum;
    p->attn_sink = a->attn_sink;
    p->topk_length = a->topk_length;
    p->block_table = nullptr;
    p->bt_stride = 0;
    p->causal = 0;
    p->n_pages = (uint32_t)(r.num_kv_tokens / r.page_block_size);
    p->n_tok = r.num_kv_tokens;
    p->n_tok32 = (uint32_t)(r.num_kv_tokens < INT32_MAX ? r.num_kv_tokens : INT32_MAX);
    p->b = r.b;
    p->s_q = r.s_q;
    p->h_q = r.h_q;
    p->topk = r.topk;
    p->page_block_size = r.page_block_size;
    {
        // division by the page size as a multiply-high: l = ceil(log2 P),
        // magic = floor(2^32 (2^l - P) / P) + 1 is exact for every t < 2^31
        const uint64_t P = (uint64_t)r.page_block_size;
        int l = 0;
        while ((1ull << l) < P) ++l;
        p->page_mshift = l;
        p->page_magic = (uint32_t)(((1ull << 32) * ((1ull << l) - P)) / P + 1);
    }
    p->x_kv = nullptr;                                        // no extra cache (mla_sparse_decode_extra_fwd)
    p->x_indices = nullptr;
    p->x_topk_length = nullptr;
    p->x_block_stride = 0;
    p->x_idx_sb = p->x_idx_ss = 0;
    p->main_topk = r.topk;
    p->x_topk = 0;
    p->x_page_block_size = 1;
    p->x_page_mshift = 0;
    p->x_page_magic = 0;
    p->x_scale_off = 0;
    p->x_n_tok32 = 0;
    p->soa_scale_off = r.kv_format == MLA_KV_V4_584    ? (uint32_t)(r.page_block_size * 576)
                       : r.kv_format == MLA_KV_V41_528 ? (uint32_t)(r.page_block_size * 512)
                                                       : 0u;
    p->kv_flat = r.kv_format == MLA_KV_FP8_656 && a->kv_stride_block == (int64_t)r.page_block_size * 656 &&
                 r.num_kv_tokens < (1ll << 24) && r.num_kv_tokens * 656 < (1ll << 32);
    p->block = r.block;
    {
        // closed-form plan constants (used by the kernels only when the plan
        // pointers are NULL); resolve() keeps b * B below 2^30
        const int64_t B = (r.topk + r.block - 1) / r.block, T = (int64_t)r.b * B;
        const int64_t P = (T + r.num_parts - 1) / r.num_parts;
        int64_t x = B, y = P;
        while (y) {
            const int64_t t = x % y;
            x = y;
            y = t;
        }
        p->plan_nblk = (uint32_t)B;
        p->plan_total = (uint32_t)T;
        p->plan_payload = (uint32_t)P;
        p->plan_gb = (uint32_t)(B / x);
        p->plan_gp = (uint32_t)(P / x);
        p->div_nblk = mla::make_fastdiv(p->plan_nblk);
        p->div_payload = mla::make_fastdiv(p->plan_payload);
        p->div_gb = mla::make_fastdiv(p->plan_gb);
        p->div_gp = mla::make_fastdiv(p->plan_gp);
    }
    p->c = sm * 1.4426950408889634f;
    p->threshold = mla::kRefGapLog2;
    return MLA_OK;
}

int hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MLA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

namespace mla {
int host_fail(int code, const char* msg) { return fail(code, "%s", msg); }
int host_ok() { return ok(); }
int host_hip_status(hipError_t e, const char* what) { return hip_status(e, what); }
int check_decode_args_noalloc(const mla_decode_args* a, ResolvedShape* rs, DecodeParams* p) {
    return check_decode_args(a, rs, p, false);
}
}  // namespace mla

extern "C" {

int mla_resolve_shape(mla_shape* shape) {
    mla::ResolvedShape r;
    int st = resolve(shape, &r);
    if (st != MLA_OK) return st;
    shape->num_parts = r.num_parts;
    shape->split_granularity = r.block;
    shape->fixed_overhead = r.overhead;
    if (shape->kv_format == MLA_KV_BF16_576) shape->page_block_size = 1;
    return ok();
}

int mla_sched_meta_size(const mla_shape* shape, size_t* meta_bytes, size_t* num_splits_bytes) {
    mla::ResolvedShape r;
    int st = resolve(shape, &r);
    if (st != MLA_OK) return st;
    if (meta_bytes) *meta_bytes = (size_t)r.num_parts * sizeof(mla_sched_part);
    if (num_splits_bytes) *num_splits_bytes = (size_t)(r.b + 1) * sizeof(int32_t);
    return ok();
}

int mla_workspace_size(const mla_shape* shape, size_t* o_accum_bytes, size_t* lse_accum_bytes) {
    mla::ResolvedShape r;
    int st = resolve(shape, &r);
    if (st != MLA_OK) return st;
    workspace_bytes(r, o_accum_bytes, lse_accum_bytes);
    return ok();
}

static int plan_host(const mla_shape* shape, const int32_t* lengths, void* sched_meta_host,
                     int32_t* num_splits_host) {
    mla::ResolvedShape r;
    int st = resolve(shape, &r);
    if (st != MLA_OK) return st;
    if (!sched_meta_host || !num_splits_host)
        return fail(MLA_ERR_INVALID_ARG, "sched_meta_host and num_splits_host must be non-NULL");
    mla::plan_schedule(r.b, r.topk, r.block, r.overhead, r.num_parts, lengths,
                       static_cast<int32_t*>(sched_meta_host), num_splits_host,
                       [](int32_t* p, int32_t v) { *p = v; });
    return ok();
}

int mla_plan_sched_meta_host(const mla_shape* shape, void* sched_meta_host, int32_t* num_splits_host) {
    return plan_host(shape, nullptr, sched_meta_host, num_splits_host);
}

int mla_plan_sched_meta_len_host(const mla_shape* shape, const int32_t* topk_length_host,
                                 void* sched_meta_host, int32_t* num_splits_host) {
    if (!topk_length_host) return fail(MLA_ERR_INVALID_ARG, "topk_length_host must be non-NULL");
    return plan_host(shape, topk_length_host, sched_meta_host, num_splits_host);
}

static int plan_dev(const mla_shape* shape, const int32_t* lengths, void* sched_meta_dev,
                    int32_t* num_splits_dev, void* stream) {
    mla::ResolvedShape r;
    int st = resolve(shape, &r);
    if (st != MLA_OK) return st;
    if (!sched_meta_dev || !num_splits_dev)
        return fail(MLA_ERR_INVALID_ARG, "sched_meta_dev and num_splits_dev must be non-NULL");
    if (!aligned(sched_meta_dev, 4) || !aligned(num_splits_dev, 4))
        return fail(MLA_ERR_INVALID_ARG, "sched buffers must be 4-byte aligned");
    return hip_status(mla::launch_sched(r, lengths, static_cast<int32_t*>(sched_meta_dev), num_splits_dev,
                                        static_cast<hipStream_t>(stream)),
                      "sched kernel launch");
}

int mla_get_sched_meta(const mla_shape* shape, void* sched_meta_dev, int32_t* num_splits_dev, void* stream) {
    return plan_dev(shape, nullptr, sched_meta_dev, num_splits_dev, stream);
}

int mla_get_sched_meta_len(const mla_shape* shape, const int32_t* topk_length_dev, void* sched_meta_dev,
                           int32_t* num_splits_dev, void* stream) {
    if (!topk_length_dev || !aligned(topk_length_dev, 4))
        return fail(MLA_ERR_INVALID_ARG, "topk_length_dev must be non-NULL and 4-byte aligned");
    return plan_dev(shape, topk_length_dev, sched_meta_dev, num_splits_dev, stream);
}

int mla_sparse_decode_fwd(const mla_decode_args* args, void* stream) {
    mla::ResolvedShape r;
    mla::DecodeParams p;
    int st = check_decode_args(args, &r, &p);
    if (st != MLA_OK) return st;
    return hip_status(mla::launch_decode(p, r.kv_format, r.num_parts, static_cast<hipStream_t>(stream)),
                      "decode kernel launch");
}

int mla_sparse_decode_extra_fwd(const mla_decode_args* args, const mla_extra_kv* x, void* stream) {
    mla::ResolvedShape r;
    mla::DecodeParams p;
    int st = check_decode_args(args, &r, &p);
    if (st != MLA_OK) return st;
    if (r.kv_format != MLA_KV_V41_528)
        return fail(MLA_ERR_UNSUPPORTED, "an FP4 extra cache goes with the V4.1 main cache (kv_format %d)", r.kv_format);
    if (!x) return fail(MLA_ERR_INVALID_ARG, "extra is NULL");
    if (x->extra_topk < 1 || x->extra_topk >= r.topk)
        return fail(MLA_ERR_INVALID_ARG, "extra_topk must be in [1, shape.topk) (got %d of %d)", x->extra_topk, r.topk);
    const int64_t P = x->page_block_size;
    if (P < 1 || P * 288 >= (1ll << 31))
        return fail(MLA_ERR_INVALID_ARG, "extra page_block_size must be >= 1 with P * 288 < 2^31 (got %lld)",
                    (long long)P);
    if (x->num_kv_tokens < 1 || x->num_kv_tokens >= INT32_MAX || x->num_kv_tokens % P != 0)
        return fail(MLA_ERR_INVALID_ARG, "extra num_kv_tokens must be a multiple of its page size in [1, 2^31)");
    if (!x->kv || !aligned(x->kv, 16) || x->kv_stride_block % 16 || x->kv_stride_block < P * 288)
        return fail(MLA_ERR_INVALID_ARG,
                    "extra kv must be 16-byte aligned with kv_stride_block >= page_block_size * 288, a multiple of 16");
    if (!x->indices || !aligned(x->indices, 4) || (x->topk_length && !aligned(x->topk_length, 4)))
        return fail(MLA_ERR_INVALID_ARG, "extra indices (and topk_length) must be non-NULL, 4-byte aligned");
    p.main_topk = r.topk - x->extra_topk;
    p.x_topk = x->extra_topk;
    p.x_kv = static_cast<const uint8_t*>(x->kv);
    p.x_block_stride = x->kv_stride_block;
    p.x_indices = x->indices;
    p.x_idx_sb = x->idx_stride_b;
    p.x_idx_ss = x->idx_stride_s;
    p.x_topk_length = x->topk_length;
    p.x_page_block_size = (int)P;
    {
        int l = 0;                                            // division by P as a multiply-high (as above)
        while ((1ll << l) < P) ++l;
        p.x_page_mshift = l;
        p.x_page_magic = (uint32_t)(((1ull << 32) * ((1ull << l) - (uint64_t)P)) / (uint64_t)P + 1);
    }
    p.x_scale_off = (uint32_t)(P * 256);
    p.x_n_tok32 = (uint32_t)x->num_kv_tokens;
    return hip_status(mla::launch_decode(p, r.kv_format, r.num_parts, static_cast<hipStream_t>(stream)),
                      "decode kernel launch");
}

int mla_dense_decode_fwd(const mla_decode_args* args, const int32_t* block_table, int64_t block_table_stride,
                         int causal, void* stream) {
    mla::ResolvedShape r;
    mla::DecodeParams p;
    int st = check_decode_args(args, &r, &p, true, false);
    if (st != MLA_OK) return st;
    if (args->indices)
        return fail(MLA_ERR_INVALID_ARG, "dense decode walks the block table: args->indices must be NULL");
    if (r.kv_format != MLA_KV_FP8_656)
        return fail(MLA_ERR_UNSUPPORTED, "dense decode reads the FP8 656-byte paged cache only");
    if (r.page_block_size != 64)
        return fail(MLA_ERR_UNSUPPORTED, "dense decode reads 64-token pages (got page_block_size %d)",
                    r.page_block_size);
    if (args->kv_stride_block >= ((int64_t)1 << 32))
        return fail(MLA_ERR_UNSUPPORTED, "dense decode needs a page stride below 4 GiB");
    if (r.topk % r.page_block_size != 0)
        return fail(MLA_ERR_INVALID_ARG, "dense decode: topk (%d, tokens a block-table row can hold) must be a "
                    "multiple of page_block_size (%d)", r.topk, r.page_block_size);
    if (!args->topk_length)
        return fail(MLA_ERR_INVALID_ARG, "dense decode needs the cache lengths in args->topk_length");
    if (!block_table || !aligned(block_table, 4))
        return fail(MLA_ERR_INVALID_ARG, "block_table must be non-NULL and 4-byte aligned");
    if (block_table_stride < r.topk / r.page_block_size)
        return fail(MLA_ERR_INVALID_ARG, "block_table_stride (%lld) < topk / page_block_size (%d)",
                    (long long)block_table_stride, r.topk / r.page_block_size);
    if (causal != 0 && causal != 1) return fail(MLA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
    p.block_table = block_table;
    p.bt_stride = block_table_stride;
    p.causal = causal;
    return hip_status(mla::launch_decode(p, r.kv_format, r.num_parts, static_cast<hipStream_t>(stream)),
                      "dense decode kernel launch");
}

int mla_splitkv_combine(const mla_decode_args* args, void* stream) {
    mla::ResolvedShape r;
    mla::DecodeParams p;
    int st = check_decode_args(args, &r, &p, true, false);
    if (st != MLA_OK) return st;
    // closed-form plan with partitions of whole requests (payload a multiple
    // of the request's block count): no request is split, nothing to merge
    if (!p.sched_meta && p.plan_payload % p.plan_nblk == 0) return ok();
    return hip_status(mla::launch_combine(p, static_cast<hipStream_t>(stream)), "combine kernel launch");
}

int mla_debug_gather_dequant(const mla_decode_args* args, void* k_rows, void* v_rows, void* stream) {
    mla::ResolvedShape r;
    mla::DecodeParams p;
    int st = check_decode_args(args, &r, &p);
    if (st != MLA_OK) return st;
    if (!k_rows || !aligned(k_rows, 16) || (v_rows && !aligned(v_rows, 2)))
        return fail(MLA_ERR_INVALID_ARG, "k_rows must be non-NULL and 16-byte aligned");
    if (r.kv_format != MLA_KV_FP8_656 && r.kv_format != MLA_KV_BF16_576)
        return fail(MLA_ERR_UNSUPPORTED, "the gather check covers the 656-byte and bf16 caches only");
    return hip_status(mla::launch_gather(p, r.kv_format, static_cast<uint16_t*>(k_rows),
                                         static_cast<uint16_t*>(v_rows), static_cast<hipStream_t>(stream)),
                      "gather kernel launch");
}

const char* mla_last_error(void) { return g_err; }

const char* mla_version(void) { return "libmla 0.1 gfx950"; }

}  // extern "C"

static int indexer_params(const mla_indexer_args* a, mla::IndexerParams* p, bool need_scores_in) {
    if (!a) return fail(MLA_ERR_INVALID_ARG, "args is NULL");
    if (a->b < 0 || a->b > 65535) return fail(MLA_ERR_INVALID_ARG, "b must be in [0, 65535] (got %d)", a->b);
    if (a->n_heads != 32 && a->n_heads != 64)
        return fail(MLA_ERR_UNSUPPORTED, "n_heads must be 32 or 64 (got %d)", a->n_heads);
    if (a->topk < 1) return fail(MLA_ERR_INVALID_ARG, "topk must be >= 1 (got %d)", a->topk);
    if (a->max_pages < 1 || (int64_t)a->max_pages * 64 > (1ll << 30))
        return fail(MLA_ERR_INVALID_ARG, "max_pages must be in [1, 2^24] (got %d)", a->max_pages);
    if (a->num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages must be >= 1 (got %d)", a->num_pages);
    if (!a->page_table || !a->seq_len || !a->scores || !aligned(a->page_table, 4) || !aligned(a->seq_len, 4) ||
        !aligned(a->scores, 16))
        return fail(MLA_ERR_INVALID_ARG, "page_table, seq_len (4-byte) and scores (16-byte) must be aligned, non-NULL");
    if (need_scores_in) {
        if (!a->q || !a->weights || !a->kcache || !aligned(a->q, 16) || !aligned(a->kcache, 16) ||
            !aligned(a->weights, 4))
            return fail(MLA_ERR_INVALID_ARG, "q and kcache must be 16-byte aligned, weights 4-byte, all non-NULL");
    } else if (!a->indices || !aligned(a->indices, 4)) {
        return fail(MLA_ERR_INVALID_ARG, "indices must be non-NULL and 4-byte aligned");
    }
    p->b = a->b; p->n_heads = a->n_heads; p->max_pages = a->max_pages; p->num_pages = a->num_pages;
    p->topk = a->topk;
    p->q = static_cast<const uint8_t*>(a->q);
    p->weights = a->weights;
    p->kcache = static_cast<const uint8_t*>(a->kcache);
    p->page_table = a->page_table;
    p->seq_len = a->seq_len;
    p->scores = static_cast<uint16_t*>(a->scores);
    p->indices = a->indices;
    return MLA_OK;
}

int mla_indexer_scores(const mla_indexer_args* args, void* stream) {
    mla::IndexerParams p;
    int st = indexer_params(args, &p, true);
    if (st != MLA_OK) return st;
    return hip_status(mla::launch_indexer_scores(p, static_cast<hipStream_t>(stream)), "indexer score launch");
}

int mla_indexer_topk(const mla_indexer_args* args, void* stream) {
    mla::IndexerParams p;
    int st = indexer_params(args, &p, false);
    if (st != MLA_OK) return st;
    return hip_status(mla::launch_indexer_topk(p, static_cast<hipStream_t>(stream)), "indexer top-k launch");
}
