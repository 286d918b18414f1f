// C-ABI entry points of libtwotower_attn: argument validation (pure host code,
// run before anything is launched), workspace sizing and dispatch.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>

#include "tt_internal.h"

namespace {

// ---- per-device CU count, cached on first use --------------------------------
constexpr int kMaxDevices = 64;
std::atomic<int> g_cu_count[kMaxDevices];

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int n = g_cu_count[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    int cu = 0;
    if (hipDeviceGetAttribute(&cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cu <= 0) cu = 256;
    g_cu_count[dev].store(cu, std::memory_order_relaxed);
    return cu;
}

bool log_enabled() {
    static const bool on = [] {
        const char* v = getenv("TT_LOG");
        return v && v[0] && v[0] != '0';
    }();
    return on;
}

// Fault injection for tests of the error path: with TT_INJECT_HIP_ERROR set (and not "0"),
// every entry point that would launch returns TT_ERR_HIP after validation, launching nothing.
bool inject_hip_error() {
    static const bool on = [] {
        const char* v = getenv("TT_INJECT_HIP_ERROR");
        return v && v[0] && v[0] != '0';
    }();
    return on;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t esize(int dtype) { return dtype == TT_BF16 ? 2 : 4; }

// strides (elements) of a head_dim-contiguous tensor must keep 16-byte alignment;
// the kernels hold them in 32 bits
bool stride_ok(int64_t st, int dtype) {
    return st >= 0 && st < ((int64_t)1 << 31) && (st * (int64_t)esize(dtype)) % 16 == 0;
}

tt_status validate_attn(const tt_block_attn_params* p) {
    if (!p) return TT_ERR_NULL;
    if (p->dtype != TT_BF16 && p->dtype != TT_F32) return TT_ERR_DTYPE;
    if (p->o_dtype != p->dtype && p->o_dtype != TT_F32) return TT_ERR_DTYPE;
    if (p->B < 0 || p->S < 1 || p->S > 64 || p->Hq < 1 || p->Hkv < 1 || p->Hq % p->Hkv != 0) return TT_ERR_SHAPE;
    if (p->head_dim != 64 && p->head_dim != 128) return TT_ERR_UNSUPPORTED;
    if (!(p->softmax_scale > 0.f) || !isfinite(p->softmax_scale)) return TT_ERR_ARG;
    if (p->max_ctx_len < 0) return TT_ERR_SHAPE;
    if (p->B == 0) return TT_OK;
    if (!p->Q || !p->O) return TT_ERR_NULL;
    if ((p->Kden == nullptr) != (p->Vden == nullptr)) return TT_ERR_NULL;
    if (p->max_ctx_len > 0) {
        if (!p->Kctx || !p->Vctx || !p->page_table || !p->ctx_len) return TT_ERR_NULL;
        if (p->page_size < 16 || p->page_size % 16 != 0) return TT_ERR_SHAPE;
        if (p->num_pages < 1 || p->max_pages < 1) return TT_ERR_SHAPE;
        if ((int64_t)p->max_pages * p->page_size < p->max_ctx_len) return TT_ERR_SHAPE;
        if ((int64_t)p->B * p->max_pages >= ((int64_t)1 << 30)) return TT_ERR_UNSUPPORTED;
        if (!aligned16(p->Kctx) || !aligned16(p->Vctx)) return TT_ERR_UNSUPPORTED;
    }
    if (!aligned16(p->Q) || !aligned16(p->O)) return TT_ERR_UNSUPPORTED;
    if (!stride_ok(p->q_stride_b, p->dtype) || !stride_ok(p->q_stride_s, p->dtype) ||
        !stride_ok(p->q_stride_h, p->dtype))
        return TT_ERR_UNSUPPORTED;
    if (!stride_ok(p->o_stride_b, p->o_dtype) || !stride_ok(p->o_stride_s, p->o_dtype) ||
        !stride_ok(p->o_stride_h, p->o_dtype))
        return TT_ERR_UNSUPPORTED;
    if (p->Kden) {
        if (!aligned16(p->Kden) || !aligned16(p->Vden)) return TT_ERR_UNSUPPORTED;
        if (!stride_ok(p->den_stride_b, p->dtype) || !stride_ok(p->den_stride_s, p->dtype) ||
            !stride_ok(p->den_stride_h, p->dtype))
            return TT_ERR_UNSUPPORTED;
    }
    // offsets inside one sequence are 32-bit byte offsets in the kernels
    const int64_t lim = (int64_t)1 << 30;
    if ((int64_t)(p->S - 1) * p->q_stride_s + (int64_t)(p->Hq - 1) * p->q_stride_h + p->head_dim >= lim ||
        (int64_t)(p->S - 1) * p->o_stride_s + (int64_t)(p->Hq - 1) * p->o_stride_h + p->head_dim >= lim)
        return TT_ERR_UNSUPPORTED;
    if (p->Kden &&
        (int64_t)(p->S - 1) * p->den_stride_s + (int64_t)(p->Hkv - 1) * p->den_stride_h + p->head_dim >= lim)
        return TT_ERR_UNSUPPORTED;
    // the bf16 path counts tiles (and the piece-start charge) in 32-bit integers
    const int64_t G = p->Hq / p->Hkv;
    const int64_t n_rb = (p->S * G + tt::kRows - 1) / tt::kRows;
    const int64_t tiles = ((int64_t)p->max_ctx_len + tt::kTile - 1) / tt::kTile + 1 + tt::kPieceCost;
    if ((int64_t)p->B * p->Hkv * n_rb * tiles >= (int64_t)1 << 30) return TT_ERR_SHAPE;
    return TT_OK;
}

tt_status validate_unmask(const tt_conf_unmask_params* p) {
    if (!p) return TT_ERR_NULL;
    if (p->dtype != TT_BF16 && p->dtype != TT_F32) return TT_ERR_DTYPE;
    if (p->B < 0 || p->S < 1 || p->S > 64 || p->V < 1 || p->logits_stride_row < p->V) return TT_ERR_SHAPE;
    if (isnan(p->gamma)) return TT_ERR_ARG;
    if (!(p->temperature > 0.f) || !isfinite(p->temperature)) return TT_ERR_ARG;
    if (p->steps_left < 1) return TT_ERR_ARG;
    if ((int64_t)p->B * p->S >= (int64_t)1 << 31) return TT_ERR_SHAPE;
    if (p->B == 0) return TT_OK;
    // the stochastic draw re-reads one vocabulary split per row through a bounded LDS table
    if (p->uniforms && !tt::unmask_sample_fits(*p, tt::plan_unmask(*p, device_cu_count()))) return TT_ERR_SHAPE;
    if (!p->logits || !p->mask_in || !p->mask_out || !p->tokens) return TT_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(p->logits) % esize(p->dtype)) != 0) return TT_ERR_UNSUPPORTED;
    return TT_OK;
}

tt_status validate_nll(const tt_masked_nll_params* p) {
    if (!p) return TT_ERR_NULL;
    if (p->dtype != TT_BF16 && p->dtype != TT_F32) return TT_ERR_DTYPE;
    if (p->B < 0 || p->S < 1 || p->V < 1 || p->logits_stride_row < p->V) return TT_ERR_SHAPE;
    if ((int64_t)p->B * p->S >= (int64_t)1 << 31) return TT_ERR_SHAPE;
    if (p->B == 0) return TT_OK;
    if (!p->logits || !p->targets || !p->mask || !p->loss) return TT_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(p->logits) % esize(p->dtype)) != 0) return TT_ERR_UNSUPPORTED;
    return TT_OK;
}

tt_status validate_append(const tt_kv_append_params* p) {
    if (!p) return TT_ERR_NULL;
    if (p->dtype != TT_BF16 && p->dtype != TT_F32) return TT_ERR_DTYPE;
    if (p->B < 0 || p->S < 1 || p->S > 64 || p->Hkv < 1 || p->head_dim < 1) return TT_ERR_SHAPE;
    if (p->page_size < 1 || p->num_pages < 1 || p->max_pages < 1) return TT_ERR_SHAPE;
    if ((int64_t)p->B * p->max_pages >= ((int64_t)1 << 30)) return TT_ERR_UNSUPPORTED;
    if (((int64_t)p->head_dim * esize(p->dtype)) % 16 != 0) return TT_ERR_UNSUPPORTED;
    if (p->B == 0) return TT_OK;
    if (!p->Kctx || !p->Vctx || !p->page_table || !p->ctx_len || !p->Knew || !p->Vnew || !p->status)
        return TT_ERR_NULL;
    if ((p->pool == nullptr) != (p->pool_count == nullptr)) return TT_ERR_NULL;
    if (!aligned16(p->Kctx) || !aligned16(p->Vctx) || !aligned16(p->Knew) || !aligned16(p->Vnew))
        return TT_ERR_UNSUPPORTED;
    if (!stride_ok(p->new_stride_b, p->dtype) || !stride_ok(p->new_stride_s, p->dtype) ||
        !stride_ok(p->new_stride_h, p->dtype))
        return TT_ERR_UNSUPPORTED;
    if ((int64_t)p->B * p->S >= ((int64_t)1 << 31)) return TT_ERR_SHAPE;
    return TT_OK;
}

}  // namespace

extern "C" {

int tt_abi_version(void) { return TT_ABI_VERSION; }

const char* tt_status_string(tt_status status) {
    // a C caller may pass any int: read the bits, not a (possibly out-of-range) enum value
    int32_t s;
    memcpy(&s, &status, sizeof s);
    switch (s) {
        case TT_OK: return "TT_OK: success";
        case TT_ERR_NULL: return "TT_ERR_NULL: a required pointer is NULL";
        case TT_ERR_SHAPE: return "TT_ERR_SHAPE: inconsistent or out-of-range sizes or strides";
        case TT_ERR_DTYPE: return "TT_ERR_DTYPE: unsupported element type combination";
        case TT_ERR_UNSUPPORTED: return "TT_ERR_UNSUPPORTED: head_dim or alignment not supported";
        case TT_ERR_WORKSPACE: return "TT_ERR_WORKSPACE: workspace missing or too small";
        case TT_ERR_ARG: return "TT_ERR_ARG: bad scalar argument";
        case TT_ERR_HIP: return "TT_ERR_HIP: the HIP runtime reported an error";
    }
    return "unknown tt_status";
}

size_t tt_block_attn_workspace_bytes(const tt_block_attn_params* p) {
    if (validate_attn(p) != TT_OK || p->B == 0 || p->dtype != TT_BF16) return 0;
    return tt::plan_attn_bf16(*p, device_cu_count()).ws_total;
}

tt_status tt_block_attn(const tt_block_attn_params* p, void* workspace, size_t ws_bytes, hipStream_t stream) {
    const tt_status v = validate_attn(p);
    if (v != TT_OK || p->B == 0) return v;
    try {
        if (p->dtype == TT_F32) {
            if (log_enabled())
                fprintf(stderr, "[tt] block_attn f32 B=%d S=%d Hq=%d Hkv=%d d=%d Lmax=%d\n", p->B, p->S, p->Hq,
                        p->Hkv, p->head_dim, p->max_ctx_len);
            return inject_hip_error() ? TT_ERR_HIP : tt::launch_attn_f32(*p, stream);
        }
        const tt::AttnPlan plan = tt::plan_attn_bf16(*p, device_cu_count());
        if (ws_bytes < plan.ws_total || workspace == nullptr) return TT_ERR_WORKSPACE;
        if (!aligned16(workspace)) return TT_ERR_UNSUPPORTED;
        if (inject_hip_error()) return TT_ERR_HIP;
        if (log_enabled())
            fprintf(stderr, "[tt] block_attn bf16 B=%d S=%d Hq=%d Hkv=%d d=%d Lmax=%d seg=%d pairs=%d ws=%zu\n",
                    p->B, p->S, p->Hq, p->Hkv, p->head_dim, p->max_ctx_len, plan.n_seg, plan.n_pairs,
                    plan.ws_total);
        return tt::launch_attn_bf16(*p, plan, workspace, stream);
    } catch (...) {
        return TT_ERR_HIP;
    }
}

tt_status tt_block_attn_noalloc(const tt_block_attn_params* p, hipStream_t stream) {
    const tt_status v = validate_attn(p);
    if (v != TT_OK || p->B == 0) return v;
    try {
        if (p->dtype == TT_F32) return inject_hip_error() ? TT_ERR_HIP : tt::launch_attn_f32(*p, stream);
        const tt::AttnPlan plan = tt::plan_attn_bf16(*p, device_cu_count());
        if (plan.ws_total > tt::kNoallocScratchBytes) {
            if (log_enabled())
                fprintf(stderr, "[tt] block_attn_noalloc: needs %zu bytes of scratch, the library holds %zu\n",
                        plan.ws_total, tt::kNoallocScratchBytes);
            return TT_ERR_WORKSPACE;
        }
        if (inject_hip_error()) return TT_ERR_HIP;
        tt_status st = TT_OK;
        void* ws = tt::noalloc_scratch(&st);
        if (!ws) return st;
        if (log_enabled())
            fprintf(stderr, "[tt] block_attn_noalloc bf16 B=%d S=%d Hq=%d Hkv=%d d=%d Lmax=%d seg=%d ws=%zu\n", p->B,
                    p->S, p->Hq, p->Hkv, p->head_dim, p->max_ctx_len, plan.n_seg, plan.ws_total);
        return tt::launch_attn_bf16(*p, plan, ws, stream);
    } catch (...) {
        return TT_ERR_HIP;
    }
}

tt_status tt_lse_merge(int P, const float* O_parts, const float* lse_parts, int B, int S, int Hq, int d,
                       void* O_out, tt_dtype o_dtype_arg, float* lse_out, hipStream_t stream) {
    // a C caller may pass any int: read the bits, not a (possibly out-of-range) enum value
    int32_t o_dtype;
    memcpy(&o_dtype, &o_dtype_arg, sizeof o_dtype);
    if (P < 1 || B < 0 || S < 1 || Hq < 1 || d < 4 || d % 4 != 0) return TT_ERR_SHAPE;
    if (o_dtype != TT_F32 && o_dtype != TT_BF16) return TT_ERR_DTYPE;
    if (B == 0) return TT_OK;
    if (!O_parts || !lse_parts || !O_out) return TT_ERR_NULL;
    if (!aligned16(O_parts) || !aligned16(O_out)) return TT_ERR_UNSUPPORTED;
    if (o_dtype == TT_BF16 && d % 8 != 0) return TT_ERR_UNSUPPORTED;
    try {
        if (inject_hip_error()) return TT_ERR_HIP;
        return tt::launch_lse_merge(P, O_parts, lse_parts, B, S, Hq, d, O_out, o_dtype, lse_out, stream);
    } catch (...) {
        return TT_ERR_HIP;
    }
}

size_t tt_conf_unmask_workspace_bytes(const tt_conf_unmask_params* p) {
    if (validate_unmask(p) != TT_OK || p->B == 0) return 0;
    return tt::plan_unmask(*p, device_cu_count()).ws_total;
}

tt_status tt_conf_unmask(const tt_conf_unmask_params* p, void* workspace, size_t ws_bytes, hipStream_t stream) {
    const tt_status v = validate_unmask(p);
    if (v != TT_OK || p->B == 0) return v;
    try {
        const tt::UnmaskPlan plan = tt::plan_unmask(*p, device_cu_count());
        if (ws_bytes < plan.ws_total || workspace == nullptr) return TT_ERR_WORKSPACE;
        if (!aligned16(workspace)) return TT_ERR_UNSUPPORTED;
        if (log_enabled())
            fprintf(stderr, "[tt] conf_unmask B=%d S=%d V=%d vsplit=%d gamma=%g T=%g R=%d\n", p->B, p->S, p->V,
                    plan.n_vsplit, p->gamma, p->temperature, p->steps_left);
        if (inject_hip_error()) return TT_ERR_HIP;
        return tt::launch_unmask(*p, plan, workspace, stream);
    } catch (...) {
        return TT_ERR_HIP;
    }
}

tt_status tt_kv_append(const tt_kv_append_params* p, hipStream_t stream) {
    const tt_status v = validate_append(p);
    if (v != TT_OK || p->B == 0) return v;
    try {
        if (log_enabled())
            fprintf(stderr, "[tt] kv_append B=%d S=%d Hkv=%d d=%d page=%d pages=%d\n", p->B, p->S, p->Hkv,
                    p->head_dim, p->page_size, p->num_pages);
        if (inject_hip_error()) return TT_ERR_HIP;
        return tt::launch_kv_append(*p, stream);
    } catch (...) {
        return TT_ERR_HIP;
    }
}

size_t tt_masked_nll_workspace_bytes(const tt_masked_nll_params* p) {
    if (validate_nll(p) != TT_OK || p->B == 0) return 0;
    return tt::plan_nll(*p, device_cu_count()).ws_total;
}

tt_status tt_masked_nll(const tt_masked_nll_params* p, void* workspace, size_t ws_bytes, hipStream_t stream) {
    const tt_status v = validate_nll(p);
    if (v != TT_OK || p->B == 0) return v;
    try {
        const tt::UnmaskPlan plan = tt::plan_nll(*p, device_cu_count());
        if (ws_bytes < plan.ws_total || workspace == nullptr) return TT_ERR_WORKSPACE;
        if (!aligned16(workspace)) return TT_ERR_UNSUPPORTED;
        if (log_enabled())
            fprintf(stderr, "[tt] masked_nll B=%d S=%d V=%d vsplit=%d\n", p->B, p->S, p->V, plan.n_vsplit);
        if (inject_hip_error()) return TT_ERR_HIP;
        return tt::launch_nll(*p, plan, workspace, stream);
    } catch (...) {
        return TT_ERR_HIP;
    }
}

}  // extern "C"
