// C entry points of libaqd: argument validation, error reporting, dispatch.
// Every check runs on the host before anything is enqueued, so a failing call
// has no side effect on the device.
#include <string>

#include "aqd_internal.h"

namespace aqd {

static thread_local std::string g_last_error;

void set_error(const std::string& s) { g_last_error = s; }

static aqd_status fail(aqd_status st, const std::string& msg) {
    g_last_error = msg;
    return st;
}

static aqd_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return AQD_OK;
    return fail(AQD_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static bool aligned2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }

constexpr int64_t MAX_DIM = int64_t(1) << 24;

static aqd_status check_layer(const aqd_layer* L) {
    if (!L) return fail(AQD_ERR_NULL, "layer is NULL");
    if (L->group != GROUP || L->code_bits != 8)
        return fail(AQD_ERR_UNSUPPORTED, "only group = 8 and code_bits = 8 are supported");
    if (L->d_out < 0 || L->d_out > MAX_DIM) return fail(AQD_ERR_SHAPE, "d_out out of range");
    if (L->d_in < 0 || L->d_in > MAX_DIM || L->d_in % GROUP != 0)
        return fail(AQD_ERR_SHAPE, "d_in must be a multiple of 8 in [0, 2^24]");
    if (L->M < 1 || L->M > MAX_M) return fail(AQD_ERR_SHAPE, "M must be in [1, 8]");
    return AQD_OK;
}

}  // namespace aqd

using namespace aqd;

extern "C" {

int aqd_abi_version(void) { return 1; }

const char* aqd_status_string(int st) {
    switch (st) {
        case AQD_OK: return "ok";
        case AQD_ERR_NULL: return "null pointer";
        case AQD_ERR_SHAPE: return "bad shape";
        case AQD_ERR_K: return "k outside [1, M]";
        case AQD_ERR_BLOCK: return "bad Hadamard block";
        case AQD_ERR_DTYPE: return "unsupported dtype";
        case AQD_ERR_ALIGN: return "misaligned pointer";
        case AQD_ERR_UNSUPPORTED: return "unsupported layer format";
        case AQD_ERR_WORKSPACE: return "workspace missing or too small";
        case AQD_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* aqd_last_error(void) { return g_last_error.c_str(); }

size_t aqd_packed_codes_bytes(const aqd_layer* layer) {
    if (check_layer(layer) != AQD_OK) return 0;
    Geometry g = geometry(*layer);
    return (size_t)(g.plane_bytes * g.M);
}

aqd_status aqd_pack_codes(const uint8_t* codes, uint8_t* packed, const aqd_layer* layer, void* stream) {
    aqd_status st = check_layer(layer);
    if (st != AQD_OK) return st;
    Geometry g = geometry(*layer);
    if (g.plane_bytes == 0) return AQD_OK;
    if (!packed || (!codes && g.d_out * g.G > 0)) return fail(AQD_ERR_NULL, "codes or packed is NULL");
    if (!aligned16(packed)) return fail(AQD_ERR_ALIGN, "packed must be 16-byte aligned");
    return hip_status(launch_pack(codes, packed, g, (hipStream_t)stream), "aqd_pack_codes");
}

aqd_status aqd_unpack_codes(const uint8_t* packed, uint8_t* codes, const aqd_layer* layer, void* stream) {
    aqd_status st = check_layer(layer);
    if (st != AQD_OK) return st;
    Geometry g = geometry(*layer);
    if (g.d_out * g.G == 0) return AQD_OK;
    if (!packed || !codes) return fail(AQD_ERR_NULL, "codes or packed is NULL");
    if (!aligned16(packed)) return fail(AQD_ERR_ALIGN, "packed must be 16-byte aligned");
    return hip_status(launch_unpack(packed, codes, g, (hipStream_t)stream), "aqd_unpack_codes");
}

static bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }

static aqd_status hadamard_rotate(const void* x, void* x_rot, int in_dtype, int out_dtype, int64_t batch,
                                  int64_t d_in, int32_t block, const uint8_t* signs, bool want_signs,
                                  void* stream, const char* name) {
    if (in_dtype != AQD_F16 && in_dtype != AQD_BF16 && in_dtype != AQD_F32)
        return fail(AQD_ERR_DTYPE, "in_dtype must be F16, BF16 or F32");
    if (out_dtype != AQD_F16 && out_dtype != AQD_BF16 && out_dtype != AQD_F32 && out_dtype != AQD_BF16X2)
        return fail(AQD_ERR_DTYPE, "out_dtype must be F16, BF16, F32 or BF16X2");
    if (batch < 0 || batch > MAX_DIM || d_in < 0 || d_in > MAX_DIM)
        return fail(AQD_ERR_SHAPE, "batch or d_in out of range");
    if (block != 64 && block != 128 && block != 256)
        return fail(AQD_ERR_BLOCK, "block must be 64, 128 or 256");
    if (d_in % block != 0) return fail(AQD_ERR_BLOCK, "block must divide d_in");
    if (batch * d_in == 0) return AQD_OK;
    if (!x || !x_rot) return fail(AQD_ERR_NULL, "x or x_rot is NULL");
    if (want_signs && !signs) return fail(AQD_ERR_NULL, "signs is NULL");
    if (!aligned16(x) || !aligned16(x_rot)) return fail(AQD_ERR_ALIGN, "x and x_rot must be 16-byte aligned");
    if (want_signs && !aligned8(signs)) return fail(AQD_ERR_ALIGN, "signs must be 8-byte aligned");
    if (x == x_rot && (in_dtype != out_dtype || out_dtype == AQD_BF16X2))
        return fail(AQD_ERR_DTYPE, "in-place rotation needs equal in/out dtypes");
    return hip_status(launch_hadamard(x, x_rot, in_dtype, out_dtype, batch, d_in, block,
                                      want_signs ? signs : nullptr, (hipStream_t)stream),
                      name);
}

aqd_status aqd_hadamard_rotate(const void* x, void* x_rot, int in_dtype, int out_dtype, int64_t batch,
                               int64_t d_in, int32_t block, void* stream) {
    return hadamard_rotate(x, x_rot, in_dtype, out_dtype, batch, d_in, block, nullptr, false, stream,
                           "aqd_hadamard_rotate");
}

aqd_status aqd_hadamard_rotate_signed(const void* x, void* x_rot, int in_dtype, int out_dtype, int64_t batch,
                                      int64_t d_in, int32_t block, const uint8_t* signs, void* stream) {
    return hadamard_rotate(x, x_rot, in_dtype, out_dtype, batch, d_in, block, signs, true, stream,
                           "aqd_hadamard_rotate_signed");
}

size_t aqd_gemv_workspace_bytes(const aqd_layer* layer, int32_t batch) {
    if (check_layer(layer) != AQD_OK || batch < 1 || batch > 8) return 0;
    return gemv_workspace_bytes(geometry(*layer), batch);
}

static aqd_status check_product(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales,
                                int32_t k, const void* x, const void* y, const aqd_layer* layer, void* ws,
                                size_t ws_bytes, size_t ws_needed, bool* nothing_to_do) {
    aqd_status st = check_layer(layer);
    if (st != AQD_OK) return st;
    if (k < 1 || k > layer->M) return fail(AQD_ERR_K, "k must be in [1, M]");
    *nothing_to_do = layer->d_out == 0;
    if (*nothing_to_do) return AQD_OK;
    if (!y || !scales) return fail(AQD_ERR_NULL, "y or scales is NULL");
    if (layer->d_in > 0 && (!packed || !codebooks || !x))
        return fail(AQD_ERR_NULL, "packed_codes, codebooks or x_rot is NULL");
    if ((packed && !aligned16(packed)) || (codebooks && !aligned16(codebooks)) || (x && !aligned16(x)))
        return fail(AQD_ERR_ALIGN, "packed_codes, codebooks and x_rot must be 16-byte aligned");
    if (!aligned2(scales) || !aligned2(y)) return fail(AQD_ERR_ALIGN, "scales and y must be 2-byte aligned");
    if (ws_needed > 0) {
        if (!ws || ws_bytes < ws_needed) return fail(AQD_ERR_WORKSPACE, "workspace missing or too small");
        if (!aligned16(ws)) return fail(AQD_ERR_ALIGN, "workspace must be 16-byte aligned");
    }
    return AQD_OK;
}

aqd_status aqd_gemv(const uint8_t* packed_codes, const uint16_t* codebooks, const uint16_t* scales, int32_t k,
                    const uint16_t* x_rot, uint16_t* y, int32_t batch, const aqd_layer* layer, void* workspace,
                    size_t workspace_bytes, void* stream) {
    if (batch < 1 || batch > 8) return fail(AQD_ERR_SHAPE, "aqd_gemv batch must be in [1, 8]");
    bool nothing = false;
    size_t need = layer ? aqd_gemv_workspace_bytes(layer, batch) : 0;
    aqd_status st = check_product(packed_codes, codebooks, scales, k, x_rot, y, layer, workspace,
                                  workspace_bytes, need, &nothing);
    if (st != AQD_OK || nothing) return st;
    return hip_status(launch_gemv(packed_codes, codebooks, scales, k, x_rot, y, batch, geometry(*layer),
                                  workspace, (hipStream_t)stream),
                      "aqd_gemv");
}

}  // extern "C"

namespace aqd {

// aqd_gemv's checks for an entry point that supplies a workspace of ws_bytes itself (the no-alloc
// entry point): everything except the workspace pointer, plus the size limit.
aqd_status check_gemv_args(const uint8_t* packed, const uint16_t* codebooks, const uint16_t* scales, int32_t k,
                           const uint16_t* x_rot, const uint16_t* y, int32_t batch, const aqd_layer* layer,
                           size_t ws_bytes, size_t* need, bool* nothing) {
    if (batch < 1 || batch > 8) return fail(AQD_ERR_SHAPE, "batch must be in [1, 8]");
    *need = layer ? aqd_gemv_workspace_bytes(layer, batch) : 0;
    // the workspace pointer is the caller's to check: none is required here
    aqd_status st = check_product(packed, codebooks, scales, k, x_rot, y, layer, nullptr, 0, 0, nothing);
    if (st != AQD_OK || *nothing) return st;
    if (*need > ws_bytes) return fail(AQD_ERR_WORKSPACE, "layer and batch need more workspace than the fixed limit");
    return AQD_OK;
}

aqd_status hip_fail(hipError_t e, const char* what) { return hip_status(e, what); }

}  // namespace aqd

extern "C" {

static aqd_status check_group(const aqd_linear* lins, int32_t n, int64_t d_in, aqd_layer* layers) {
    if (!lins) return fail(AQD_ERR_NULL, "linears is NULL");
    if (n < 1 || n > AQD_MAX_GROUP) return fail(AQD_ERR_SHAPE, "n_linears must be in [1, AQD_MAX_GROUP]");
    for (int i = 0; i < n; ++i) {
        layers[i] = aqd_layer{lins[i].d_out, d_in, lins[i].M, 8, 8};
        aqd_status st = check_layer(&layers[i]);
        if (st != AQD_OK) return st;
    }
    return AQD_OK;
}

size_t aqd_gemv_grouped_workspace_bytes(const aqd_linear* linears, int32_t n_linears, int64_t d_in) {
    aqd_layer layers[AQD_MAX_GROUP];
    if (check_group(linears, n_linears, d_in, layers) != AQD_OK) return 0;
    int64_t d_out[AQD_MAX_GROUP];
    for (int i = 0; i < n_linears; ++i) d_out[i] = linears[i].d_out;
    return gemv_lut_grouped_workspace_bytes(d_out, n_linears);
}

static aqd_status gemv_grouped(const aqd_linear* linears, int32_t n_linears, int32_t k, const uint16_t* x,
                               int64_t d_in, void* workspace, size_t workspace_bytes, void* stream, int block,
                               const uint8_t* signs, const char* name);

aqd_status aqd_gemv_grouped(const aqd_linear* linears, int32_t n_linears, int32_t k, const uint16_t* x_rot,
                            int64_t d_in, void* workspace, size_t workspace_bytes, void* stream) {
    return gemv_grouped(linears, n_linears, k, x_rot, d_in, workspace, workspace_bytes, stream, 0, nullptr,
                        "aqd_gemv_grouped");
}

aqd_status aqd_rotate_gemv_grouped(const aqd_linear* linears, int32_t n_linears, int32_t k, const uint16_t* x,
                                   int64_t d_in, int32_t block, void* workspace, size_t workspace_bytes,
                                   void* stream) {
    if (block != 64 && block != 128 && block != 256) return fail(AQD_ERR_BLOCK, "block must be 64, 128 or 256");
    if (d_in % block) return fail(AQD_ERR_BLOCK, "block must divide d_in");
    return gemv_grouped(linears, n_linears, k, x, d_in, workspace, workspace_bytes, stream, block, nullptr,
                        "aqd_rotate_gemv_grouped");
}

aqd_status aqd_rotate_gemv_grouped_signed(const aqd_linear* linears, int32_t n_linears, int32_t k,
                                          const uint16_t* x, int64_t d_in, int32_t block, const uint8_t* signs,
                                          void* workspace, size_t workspace_bytes, void* stream) {
    if (block != 64 && block != 128 && block != 256) return fail(AQD_ERR_BLOCK, "block must be 64, 128 or 256");
    if (d_in % block) return fail(AQD_ERR_BLOCK, "block must divide d_in");
    if (d_in > 0 && !signs) return fail(AQD_ERR_NULL, "signs is NULL");
    if (d_in > 0 && !aligned8(signs)) return fail(AQD_ERR_ALIGN, "signs must be 8-byte aligned");
    return gemv_grouped(linears, n_linears, k, x, d_in, workspace, workspace_bytes, stream, block, signs,
                        "aqd_rotate_gemv_grouped_signed");
}

static aqd_status gemv_grouped(const aqd_linear* linears, int32_t n_linears, int32_t k, const uint16_t* x_rot,
                               int64_t d_in, void* workspace, size_t workspace_bytes, void* stream, int block,
                               const uint8_t* signs, const char* name) {
    aqd_layer layers[AQD_MAX_GROUP];
    aqd_status st = check_group(linears, n_linears, d_in, layers);
    if (st != AQD_OK) return st;
    const size_t need = aqd_gemv_grouped_workspace_bytes(linears, n_linears, d_in);
    bool any = false;
    for (int i = 0; i < n_linears; ++i) {
        bool nothing = false;
        st = check_product(linears[i].packed_codes, linears[i].codebooks, linears[i].scales, k, x_rot,
                           linears[i].y, &layers[i], workspace, workspace_bytes, need, &nothing);
        if (st != AQD_OK) return st;
        any = any || !nothing;
    }
    if (!any) return AQD_OK;
    if (d_in == 0) {        // empty input: every y is zero (no tables to build)
        for (int i = 0; i < n_linears; ++i) {
            if (linears[i].d_out == 0) continue;
            st = aqd_gemv(linears[i].packed_codes, linears[i].codebooks, linears[i].scales, k, x_rot,
                          linears[i].y, 1, &layers[i], workspace, workspace_bytes, stream);
            if (st != AQD_OK) return st;
        }
        return AQD_OK;
    }
    int64_t d_outs[AQD_MAX_GROUP];
    for (int i = 0; i < n_linears; ++i) d_outs[i] = linears[i].d_out;
    if (!gemv_lut_grouped_supported(d_in / 8, k, d_outs, n_linears))
        return fail(AQD_ERR_UNSUPPORTED, "input too wide or a linear with too many rows for one grouped launch");
    LutLinearRef refs[AQD_MAX_GROUP];
    for (int i = 0; i < n_linears; ++i)
        refs[i] = LutLinearRef{linears[i].packed_codes, linears[i].codebooks, linears[i].scales, linears[i].y,
                               linears[i].d_out};
    return hip_status(launch_gemv_lut_grouped(refs, n_linears, k, x_rot, d_in, workspace, (hipStream_t)stream,
                                              block, signs),
                      name);
}

size_t aqd_gemm_small_batch_workspace_bytes(const aqd_layer* layer, int32_t batch) {
    if (check_layer(layer) != AQD_OK || batch < 1 || batch > 64) return 0;
    return gemm_sb_workspace_bytes(geometry(*layer), batch);
}

aqd_status aqd_gemm_small_batch(const uint8_t* packed_codes, const uint16_t* codebooks, const uint16_t* scales,
                                int32_t k, const void* x_rot, int x_dtype, float* y, int32_t batch,
                                const aqd_layer* layer, void* workspace, size_t workspace_bytes, void* stream) {
    if (batch < 1 || batch > 64) return fail(AQD_ERR_SHAPE, "aqd_gemm_small_batch batch must be in [1, 64]");
    if (x_dtype != AQD_F16 && x_dtype != AQD_BF16 && x_dtype != AQD_BF16X2)
        return fail(AQD_ERR_DTYPE, "x_dtype must be F16, BF16 or BF16X2");
    bool nothing = false;
    size_t need = layer ? aqd_gemm_small_batch_workspace_bytes(layer, batch) : 0;
    aqd_status st = check_product(packed_codes, codebooks, scales, k, x_rot, y, layer, workspace,
                                  workspace_bytes, need, &nothing);
    if (st != AQD_OK || nothing) return st;
    if (reinterpret_cast<uintptr_t>(y) % 4) return fail(AQD_ERR_ALIGN, "y must be 4-byte aligned");
    return hip_status(launch_gemm_sb(packed_codes, codebooks, scales, k, x_rot, x_dtype, y, batch,
                                     geometry(*layer), workspace, (hipStream_t)stream),
                      "aqd_gemm_small_batch");
}

aqd_status aqd_gemm_small_batch_tiered(const uint8_t* packed_codes, const uint16_t* codebooks,
                                       const uint16_t* scales, const int32_t* ks, const uint16_t* x_rot,
                                       float* y, int32_t batch, const aqd_layer* layer,
                                       void* workspace, size_t workspace_bytes, void* stream) {
    if (batch < 1 || batch > 64) return fail(AQD_ERR_SHAPE, "aqd_gemm_small_batch_tiered batch must be in [1, 64]");
    if (!ks) return fail(AQD_ERR_NULL, "ks is NULL");
    aqd_status st = check_layer(layer);
    if (st != AQD_OK) return st;
    int kmax = 1;
    for (int n = 0; n < batch; ++n) {
        if (ks[n] < 1 || ks[n] > layer->M) return fail(AQD_ERR_K, "every ks[n] must be in [1, M]");
        kmax = ks[n] > kmax ? ks[n] : kmax;
    }
    bool nothing = false;
    const size_t need = aqd_gemm_small_batch_workspace_bytes(layer, batch);
    st = check_product(packed_codes, codebooks, scales, kmax, x_rot, y, layer, workspace, workspace_bytes, need,
                       &nothing);
    if (st != AQD_OK || nothing) return st;
    if (reinterpret_cast<uintptr_t>(y) % 4) return fail(AQD_ERR_ALIGN, "y must be 4-byte aligned");
    return hip_status(launch_gemm_sb_tiered(packed_codes, codebooks, scales, ks, x_rot, y, batch, geometry(*layer),
                                            workspace, (hipStream_t)stream),
                      "aqd_gemm_small_batch_tiered");
}

size_t aqd_gemm_prefill_workspace_bytes(const aqd_layer* layer, int32_t batch) {
    if (check_layer(layer) != AQD_OK || batch < 1 || batch > AQD_PREFILL_MAX_BATCH) return 0;
    return gemm_pf_workspace_bytes(geometry(*layer), batch);
}

aqd_status aqd_gemm_prefill(const uint8_t* packed_codes, const uint16_t* codebooks, const uint16_t* scales,
                            int32_t k, const uint16_t* x_rot, float* y, int32_t batch, const aqd_layer* layer,
                            void* workspace, size_t workspace_bytes, void* stream) {
    if (batch < 1 || batch > AQD_PREFILL_MAX_BATCH)
        return fail(AQD_ERR_SHAPE, "aqd_gemm_prefill batch must be in [1, AQD_PREFILL_MAX_BATCH]");
    bool nothing = false;
    const size_t need = layer ? aqd_gemm_prefill_workspace_bytes(layer, batch) : 0;
    aqd_status st = check_product(packed_codes, codebooks, scales, k, x_rot, y, layer, workspace, workspace_bytes,
                                  need, &nothing);
    if (st != AQD_OK || nothing) return st;
    if (reinterpret_cast<uintptr_t>(y) % 4) return fail(AQD_ERR_ALIGN, "y must be 4-byte aligned");
    return hip_status(launch_gemm_pf(packed_codes, codebooks, scales, k, x_rot, y, batch, geometry(*layer),
                                     workspace, (hipStream_t)stream),
                      "aqd_gemm_prefill");
}

aqd_status aqd_encode_greedy(const float* target, const uint16_t* codebooks, int32_t M, int64_t d_out,
                             int64_t d_in, uint8_t* codes, void* stream) {
    if (M < 1 || M > MAX_M) return fail(AQD_ERR_SHAPE, "M must be in [1, 8]");
    if (d_out < 0 || d_out > MAX_DIM || d_in < 0 || d_in > MAX_DIM) return fail(AQD_ERR_SHAPE, "d_out or d_in out of range");
    if (d_in % 8) return fail(AQD_ERR_SHAPE, "d_in must be a multiple of 8");
    if (d_out * d_in == 0) return AQD_OK;
    if ((d_out * (d_in / 8) + 255) / 256 > 0x7FFFFFFF) return fail(AQD_ERR_SHAPE, "too many groups for one launch");
    if (!target || !codebooks || !codes) return fail(AQD_ERR_NULL, "target, codebooks or codes is NULL");
    if (!aligned16(target)) return fail(AQD_ERR_ALIGN, "target must be 16-byte aligned");
    if (!aligned2(codebooks)) return fail(AQD_ERR_ALIGN, "codebooks must be 2-byte aligned");
    return hip_status(launch_encode_greedy(target, codebooks, M, d_out, d_in, codes, (hipStream_t)stream),
                      "aqd_encode_greedy");
}

}  // extern "C"
