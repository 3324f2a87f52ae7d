// C ABI of the library (declared in include/tsd_attn.h): argument checks on
// the host, then dispatch to the kernels' launchers. No device memory is
// allocated here and no call synchronises.
#include "tsd_attn.h"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <mutex>

#include "kernels.h"

namespace {

thread_local char g_last_error[512] = "";

attn_status_t fail(attn_status_t st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

attn_status_t from_hip(hipError_t e, const char *what)
{
    if (e == hipSuccess) return ATTN_OK;
    return fail(ATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return na && nb && x < y + nb && y < x + na;
}

size_t dtype_bytes(int32_t dt) { return dt == ATTN_F32 ? 4 : 2; }

constexpr long long kI32Max = 0x7fffffffLL;

}  // namespace

extern "C" {

attn_status_t attn_fwd_ex(const void *Q, const void *K, const void *V, int32_t mask_kind, const int32_t *valid_lens,
                          float scale, void *O, float *lse, int32_t batch, int32_t heads, int32_t kv_heads,
                          int32_t seq_q, int32_t seq_k, int32_t head_dim, int32_t in_dtype, int32_t out_dtype,
                          void *stream)
{
    g_last_error[0] = '\0';
    if (batch < 0 || heads < 0 || seq_q < 0 || seq_k < 0 || head_dim <= 0)
        return fail(ATTN_EINVAL, "attn_fwd: negative size or head_dim <= 0 (batch=%d heads=%d seq_q=%d seq_k=%d "
                                 "head_dim=%d)", batch, heads, seq_q, seq_k, head_dim);
    if (kv_heads <= 0 || (heads > 0 && heads % kv_heads != 0))
        return fail(ATTN_EINVAL, "attn_fwd: kv_heads must be positive and divide heads (heads=%d kv_heads=%d)", heads,
                    kv_heads);
    if (mask_kind != ATTN_MASK_NONE && mask_kind != ATTN_MASK_CAUSAL && mask_kind != ATTN_MASK_PADDING &&
        mask_kind != ATTN_MASK_CAUSAL_PADDING)
        return fail(ATTN_EINVAL, "attn_fwd: unknown mask_kind %d", mask_kind);
    if ((in_dtype != ATTN_F32 && in_dtype != ATTN_BF16) || (out_dtype != ATTN_F32 && out_dtype != ATTN_BF16))
        return fail(ATTN_EINVAL, "attn_fwd: unknown dtype (in %d, out %d)", in_dtype, out_dtype);
    if (!isfinite(scale)) return fail(ATTN_EINVAL, "attn_fwd: scale is not finite");
    if (scale < 0.f) return fail(ATTN_EUNSUPPORTED, "attn_fwd: negative scale");
    if (in_dtype == ATTN_BF16 && head_dim != 64 && head_dim != 128)
        return fail(ATTN_EUNSUPPORTED, "attn_fwd: bf16 supports head_dim 64 or 128, got %d", head_dim);
    if (in_dtype == ATTN_F32 && head_dim != 16 && head_dim != 32 && head_dim != 64 && head_dim != 128)
        return fail(ATTN_EUNSUPPORTED, "attn_fwd: f32 supports head_dim 16, 32, 64 or 128, got %d", head_dim);
    if (in_dtype == ATTN_F32 && out_dtype != ATTN_F32)
        return fail(ATTN_EUNSUPPORTED, "attn_fwd: f32 inputs need an f32 output");
    const bool causal = mask_kind == ATTN_MASK_CAUSAL || mask_kind == ATTN_MASK_CAUSAL_PADDING;
    const bool padding = mask_kind == ATTN_MASK_PADDING || mask_kind == ATTN_MASK_CAUSAL_PADDING;
    if (causal && seq_q != seq_k)
        return fail(ATTN_EUNSUPPORTED, "attn_fwd: causal mask needs seq_q == seq_k (%d != %d)", seq_q, seq_k);
    const long long bh = (long long)batch * heads;
    if (bh > kI32Max) return fail(ATTN_EINVAL, "attn_fwd: batch*heads too large");

    const size_t ib = dtype_bytes(in_dtype), ob = dtype_bytes(out_dtype);
    const size_t nq = (size_t)bh * seq_q * head_dim, nk = (size_t)batch * kv_heads * seq_k * head_dim;
    const size_t nl = (size_t)bh * seq_q * sizeof(float);
    if (nq == 0) return ATTN_OK;  // no output element
    if (!Q || !O) return fail(ATTN_EINVAL, "attn_fwd: null Q or O");
    if (nk && (!K || !V)) return fail(ATTN_EINVAL, "attn_fwd: null K or V");
    if (padding && !valid_lens) return fail(ATTN_EINVAL, "attn_fwd: padding mask needs valid_lens");
    if (!aligned(Q, 16) || !aligned(O, 16) || (nk && (!aligned(K, 16) || !aligned(V, 16))))
        return fail(ATTN_EINVAL, "attn_fwd: Q, K, V and O must be 16-byte aligned");
    if (valid_lens && padding && !aligned(valid_lens, 4))
        return fail(ATTN_EINVAL, "attn_fwd: valid_lens must be 4-byte aligned");
    if (lse && !aligned(lse, 4)) return fail(ATTN_EINVAL, "attn_fwd: lse must be 4-byte aligned");
    if (overlaps(O, nq * ob, Q, nq * ib) || overlaps(O, nq * ob, K, nk * ib) || overlaps(O, nq * ob, V, nk * ib))
        return fail(ATTN_EINVAL, "attn_fwd: O overlaps an input");
    if (lse && (overlaps(lse, nl, Q, nq * ib) || overlaps(lse, nl, K, nk * ib) || overlaps(lse, nl, V, nk * ib) ||
                overlaps(lse, nl, O, nq * ob)))
        return fail(ATTN_EINVAL, "attn_fwd: lse overlaps an input or O");

    const tsd::AttnHeads hd{kv_heads, heads > 0 ? heads / kv_heads : 1, lse};
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (in_dtype == ATTN_BF16)
        e = tsd::launch_attn_bf16(Q, K, V, mask_kind, valid_lens, scale, O, out_dtype == ATTN_F32, tsd::kOutBHND,
                                  batch, heads, seq_q, seq_k, head_dim, hd, s);
    else
        e = tsd::launch_attn_f32((const float *)Q, (const float *)K, (const float *)V, mask_kind, valid_lens, scale,
                                 (float *)O, batch, heads, seq_q, seq_k, head_dim, hd, s);
    return from_hip(e, "attn_fwd launch");
}

attn_status_t attn_fwd(const void *Q, const void *K, const void *V, int32_t mask_kind, const int32_t *valid_lens,
                       float scale, void *O, int32_t batch, int32_t heads, int32_t seq_q, int32_t seq_k,
                       int32_t head_dim, int32_t in_dtype, int32_t out_dtype, void *stream)
{
    return attn_fwd_ex(Q, K, V, mask_kind, valid_lens, scale, O, nullptr, batch, heads, heads > 0 ? heads : 1, seq_q,
                       seq_k, head_dim, in_dtype, out_dtype, stream);
}

attn_status_t attn_weights(const void *Q, const void *K, int32_t mask_kind, const int32_t *valid_lens, float scale,
                           float *A, int32_t batch, int32_t heads, int32_t kv_heads, int32_t seq_q, int32_t seq_k,
                           int32_t head_dim, int32_t dtype, void *stream)
{
    g_last_error[0] = '\0';
    if (batch < 0 || heads < 0 || seq_q < 0 || seq_k < 0 || head_dim <= 0)
        return fail(ATTN_EINVAL, "attn_weights: negative size or head_dim <= 0");
    if (kv_heads <= 0 || (heads > 0 && heads % kv_heads != 0))
        return fail(ATTN_EINVAL, "attn_weights: kv_heads must be positive and divide heads (heads=%d kv_heads=%d)",
                    heads, kv_heads);
    if (mask_kind < ATTN_MASK_NONE || mask_kind > ATTN_MASK_CAUSAL_PADDING)
        return fail(ATTN_EINVAL, "attn_weights: unknown mask_kind %d", mask_kind);
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_EINVAL, "attn_weights: unknown dtype %d", dtype);
    if (!isfinite(scale)) return fail(ATTN_EINVAL, "attn_weights: scale is not finite");
    if (scale < 0.f) return fail(ATTN_EUNSUPPORTED, "attn_weights: negative scale");
    if (head_dim > 256) return fail(ATTN_EUNSUPPORTED, "attn_weights: head_dim %d > 256", head_dim);
    if (seq_k > tsd::kAttnWeightsMaxKeys)
        return fail(ATTN_EUNSUPPORTED, "attn_weights: seq_k %d > %d (the weights are formed only for short key "
                                       "sequences)", seq_k, tsd::kAttnWeightsMaxKeys);
    const bool causal = mask_kind == ATTN_MASK_CAUSAL || mask_kind == ATTN_MASK_CAUSAL_PADDING;
    const bool padding = mask_kind == ATTN_MASK_PADDING || mask_kind == ATTN_MASK_CAUSAL_PADDING;
    if (causal && seq_q != seq_k)
        return fail(ATTN_EUNSUPPORTED, "attn_weights: causal mask needs seq_q == seq_k (%d != %d)", seq_q, seq_k);
    const long long bh = (long long)batch * heads;
    if (bh > kI32Max) return fail(ATTN_EINVAL, "attn_weights: batch*heads too large");
    const size_t eb = dtype_bytes(dtype);
    const size_t nq = (size_t)bh * seq_q * head_dim * eb, nk = (size_t)batch * kv_heads * seq_k * head_dim * eb;
    const size_t na = (size_t)bh * seq_q * seq_k * sizeof(float);
    if (na == 0) return ATTN_OK;  // no weight to write
    if (!Q || !K || !A) return fail(ATTN_EINVAL, "attn_weights: null Q, K or A");
    if (padding && !valid_lens) return fail(ATTN_EINVAL, "attn_weights: padding mask needs valid_lens");
    if (!aligned(Q, eb) || !aligned(K, eb) || !aligned(A, 4) || (padding && !aligned(valid_lens, 4)))
        return fail(ATTN_EINVAL, "attn_weights: misaligned pointer");
    if (overlaps(A, na, Q, nq) || overlaps(A, na, K, nk)) return fail(ATTN_EINVAL, "attn_weights: A overlaps Q or K");
    const tsd::AttnHeads hd{kv_heads, heads > 0 ? heads / kv_heads : 1, nullptr};
    return from_hip(tsd::launch_attn_weights(Q, K, mask_kind, valid_lens, scale, A, dtype == ATTN_BF16, batch, heads,
                                             seq_q, seq_k, head_dim, hd, (hipStream_t)stream),
                    "attn_weights launch");
}

size_t attn_bwd_workspace_bytes(int32_t batch, int32_t heads, int32_t seq_q)
{
    if (batch < 0 || heads < 0 || seq_q < 0) return 0;
    // per query row, padded to whole 64-row tiles: lse * log2(e) and dO_i . O_i, float32
    const size_t n = 2 * (size_t)batch * heads * (((size_t)seq_q + 63) / 64 * 64) * sizeof(float);
    return (n + 255) / 256 * 256;
}

}  // extern "C"

namespace {

// Every argument check of attn_bwd except the workspace's (done on the host, before any HIP call).
attn_status_t bwd_check(const void *Q, const void *K, const void *V, const void *O, const void *dO, const float *lse,
                        int32_t mask_kind, const int32_t *valid_lens, float scale, void *dQ, void *dK, void *dV,
                        int32_t batch, int32_t heads, int32_t kv_heads, int32_t seq_q, int32_t seq_k,
                        int32_t head_dim, int32_t dtype, bool *empty)
{
    *empty = false;
    if (batch < 0 || heads < 0 || seq_q < 0 || seq_k < 0 || head_dim <= 0)
        return fail(ATTN_EINVAL, "attn_bwd: negative size or head_dim <= 0 (batch=%d heads=%d seq_q=%d seq_k=%d "
                                 "head_dim=%d)", batch, heads, seq_q, seq_k, head_dim);
    if (kv_heads <= 0 || (heads > 0 && heads % kv_heads != 0))
        return fail(ATTN_EINVAL, "attn_bwd: kv_heads must be positive and divide heads (heads=%d kv_heads=%d)", heads,
                    kv_heads);
    if (mask_kind < ATTN_MASK_NONE || mask_kind > ATTN_MASK_CAUSAL_PADDING)
        return fail(ATTN_EINVAL, "attn_bwd: unknown mask_kind %d", mask_kind);
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_EINVAL, "attn_bwd: unknown dtype %d", dtype);
    if (!isfinite(scale)) return fail(ATTN_EINVAL, "attn_bwd: scale is not finite");
    if (scale < 0.f) return fail(ATTN_EUNSUPPORTED, "attn_bwd: negative scale");
    if (dtype != ATTN_BF16) return fail(ATTN_EUNSUPPORTED, "attn_bwd: only bf16 is supported");
    if (head_dim != 64 && head_dim != 128)
        return fail(ATTN_EUNSUPPORTED, "attn_bwd: bf16 supports head_dim 64 or 128, got %d", head_dim);
    const bool causal = mask_kind == ATTN_MASK_CAUSAL || mask_kind == ATTN_MASK_CAUSAL_PADDING;
    const bool padding = mask_kind == ATTN_MASK_PADDING || mask_kind == ATTN_MASK_CAUSAL_PADDING;
    if (causal && seq_q != seq_k)
        return fail(ATTN_EUNSUPPORTED, "attn_bwd: causal mask needs seq_q == seq_k (%d != %d)", seq_q, seq_k);
    const long long bh = (long long)batch * heads, bhk = (long long)batch * kv_heads;
    if (bh > kI32Max || bhk > kI32Max) return fail(ATTN_EINVAL, "attn_bwd: batch*heads too large");
    const size_t nq = (size_t)bh * seq_q * head_dim * 2, nk = (size_t)bhk * seq_k * head_dim * 2;
    const size_t nl = (size_t)bh * seq_q * sizeof(float);
    if (nq == 0 && nk == 0) {
        *empty = true;
        return ATTN_OK;
    }
    if ((nq && (!Q || !O || !dO || !lse || !dQ)) || (nk && (!K || !V || !dK || !dV)))
        return fail(ATTN_EINVAL, "attn_bwd: null pointer");
    if (padding && !valid_lens) return fail(ATTN_EINVAL, "attn_bwd: padding mask needs valid_lens");
    const void *a16[] = {Q, K, V, O, dO, dQ, dK, dV};
    for (const void *p : a16)
        if (p && !aligned(p, 16)) return fail(ATTN_EINVAL, "attn_bwd: tensors must be 16-byte aligned");
    if ((lse && !aligned(lse, 4)) || (valid_lens && padding && !aligned(valid_lens, 4)))
        return fail(ATTN_EINVAL, "attn_bwd: lse and valid_lens must be 4-byte aligned");
    const void *ins[] = {Q, K, V, O, dO, lse};
    const size_t in_n[] = {nq, nk, nk, nq, nq, nl};
    const void *outs[] = {dQ, dK, dV};
    const size_t out_n[] = {nq, nk, nk};
    for (int i = 0; i < 3; ++i) {
        for (int j = 0; j < 6; ++j)
            if (overlaps(outs[i], out_n[i], ins[j], in_n[j]))
                return fail(ATTN_EINVAL, "attn_bwd: an output overlaps an input");
        for (int j = i + 1; j < 3; ++j)
            if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return fail(ATTN_EINVAL, "attn_bwd: outputs overlap");
    }
    return ATTN_OK;
}

// Scratch of attn_bwd_noalloc: the per-row terms of one call (dO_i . O_i and lse_i in base 2), in a
// file-scope device array that every GPU the library runs on holds until the process ends. Host code uses
// the per-device address that hipGetSymbolAddress returns, never the array's name.
constexpr size_t kNoAllocScratchBytes = (size_t)8 << 20;
__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of the scratch array, looked up once per device (with that device current).
attn_status_t device_scratch(void **out)
{
    int dev = -1;
    const hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return fail(ATTN_EHIP, "attn_bwd_noalloc: hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return fail(ATTN_EINVAL, "attn_bwd_noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (g != hipSuccess || !p)
            return fail(ATTN_EHIP, "attn_bwd_noalloc: hipGetSymbolAddress: %s", hipGetErrorString(g));
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return ATTN_OK;
}

}  // namespace

extern "C" {

attn_status_t attn_bwd(const void *Q, const void *K, const void *V, const void *O, const void *dO, const float *lse,
                       int32_t mask_kind, const int32_t *valid_lens, float scale, void *dQ, void *dK, void *dV,
                       int32_t batch, int32_t heads, int32_t kv_heads, int32_t seq_q, int32_t seq_k,
                       int32_t head_dim, int32_t dtype, void *workspace, size_t workspace_bytes, void *stream)
{
    g_last_error[0] = '\0';
    bool empty = false;
    const attn_status_t st = bwd_check(Q, K, V, O, dO, lse, mask_kind, valid_lens, scale, dQ, dK, dV, batch, heads,
                                       kv_heads, seq_q, seq_k, head_dim, dtype, &empty);
    if (st != ATTN_OK || empty) return st;
    const size_t need = attn_bwd_workspace_bytes(batch, heads, seq_q);
    if (need && (!workspace || workspace_bytes < need))
        return fail(ATTN_EINVAL, "attn_bwd: workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (workspace && !aligned(workspace, 256)) return fail(ATTN_EINVAL, "attn_bwd: workspace must be 256-byte aligned");
    const size_t nq = (size_t)batch * heads * seq_q * head_dim * 2, nk = (size_t)batch * kv_heads * seq_k * head_dim * 2;
    const size_t nl = (size_t)batch * heads * seq_q * sizeof(float);
    const void *bufs[] = {Q, K, V, O, dO, lse, dQ, dK, dV};
    const size_t buf_n[] = {nq, nk, nk, nq, nq, nl, nq, nk, nk};
    for (int j = 0; j < 9; ++j)
        if (overlaps(workspace, need, bufs[j], buf_n[j]))
            return fail(ATTN_EINVAL, "attn_bwd: the workspace overlaps an input or an output");
    const hipError_t e = tsd::launch_attn_bwd_bf16(Q, K, V, O, dO, lse, mask_kind, valid_lens, scale, dQ, dK, dV, batch,
                                                   heads, kv_heads, seq_q, seq_k, head_dim, (float *)workspace,
                                                   (hipStream_t)stream);
    return from_hip(e, "attn_bwd launch");
}

size_t attn_bwd_noalloc_max_scratch_bytes(void) { return kNoAllocScratchBytes; }

attn_status_t attn_bwd_noalloc(const void *Q, const void *K, const void *V, const void *O, const void *dO,
                               const float *lse, int32_t mask_kind, const int32_t *valid_lens, float scale, void *dQ,
                               void *dK, void *dV, int32_t batch, int32_t heads, int32_t kv_heads, int32_t seq_q,
                               int32_t seq_k, int32_t head_dim, int32_t dtype, void *stream)
{
    g_last_error[0] = '\0';
    bool empty = false;
    const attn_status_t st = bwd_check(Q, K, V, O, dO, lse, mask_kind, valid_lens, scale, dQ, dK, dV, batch, heads,
                                       kv_heads, seq_q, seq_k, head_dim, dtype, &empty);
    if (st != ATTN_OK || empty) return st;
    const size_t need = attn_bwd_workspace_bytes(batch, heads, seq_q);
    if (need > kNoAllocScratchBytes)
        return fail(ATTN_EINVAL, "attn_bwd_noalloc: these sizes need %zu bytes of scratch, more than the %zu the "
                                 "library holds (batch * heads * seq_q rounded up to 64 must stay <= %zu)",
                    need, kNoAllocScratchBytes, kNoAllocScratchBytes / 8);
    void *ws = nullptr;
    const attn_status_t sst = device_scratch(&ws);
    if (sst != ATTN_OK) return sst;
    // every scratch value a call reads is first written by that call (its dQ kernel writes the row terms of
    // every padded row before the dK/dV kernel reads them), so nothing needs clearing between calls
    const hipError_t e = tsd::launch_attn_bwd_bf16(Q, K, V, O, dO, lse, mask_kind, valid_lens, scale, dQ, dK, dV, batch,
                                                   heads, kv_heads, seq_q, seq_k, head_dim, (float *)ws,
                                                   (hipStream_t)stream);
    return from_hip(e, "attn_bwd_noalloc launch");
}

static attn_status_t mha_check(int32_t batch, int32_t seq, int32_t d_model, int32_t h, int32_t dtype)
{
    if (batch < 0 || seq < 0 || d_model <= 0 || h <= 0)
        return fail(ATTN_EINVAL, "mha_fwd: bad sizes (batch=%d seq=%d d_model=%d h=%d)", batch, seq, d_model, h);
    if (dtype != ATTN_F32 && dtype != ATTN_BF16) return fail(ATTN_EINVAL, "mha_fwd: unknown dtype %d", dtype);
    if (d_model % h != 0) return fail(ATTN_EINVAL, "mha_fwd: d_model %% h != 0 (%d, %d)", d_model, h);
    if (dtype != ATTN_BF16) return fail(ATTN_EUNSUPPORTED, "mha_fwd: only bf16 is supported");
    const int dk = d_model / h;
    if (dk != 64 && dk != 128) return fail(ATTN_EUNSUPPORTED, "mha_fwd: d_model/h must be 64 or 128, got %d", dk);
    if (d_model % 64 != 0) return fail(ATTN_EUNSUPPORTED, "mha_fwd: d_model must be a multiple of 64");
    if ((long long)batch * seq > kI32Max || (long long)batch * h > kI32Max)
        return fail(ATTN_EINVAL, "mha_fwd: batch*seq too large");
    return ATTN_OK;
}

size_t mha_workspace_bytes(int32_t batch, int32_t seq, int32_t d_model, int32_t h, int32_t dtype)
{
    char saved[sizeof g_last_error];
    snprintf(saved, sizeof saved, "%s", g_last_error);
    const attn_status_t st = mha_check(batch, seq, d_model, h, dtype);
    snprintf(g_last_error, sizeof g_last_error, "%s", saved);
    if (st != ATTN_OK) return 0;
    const size_t tok = (size_t)batch * seq * d_model;
    return (3 * tok + tok) * 2;  // q, k, v split into heads + concatenated head outputs, bf16
}

attn_status_t mha_fwd(const void *X, const void *W_qkv, const void *W_o, int32_t h, void *O, int32_t batch,
                      int32_t seq, int32_t d_model, int32_t dtype, void *workspace, size_t workspace_bytes,
                      void *stream)
{
    g_last_error[0] = '\0';
    const attn_status_t st = mha_check(batch, seq, d_model, h, dtype);
    if (st != ATTN_OK) return st;
    const size_t tok = (size_t)batch * seq * d_model;
    if (tok == 0) return ATTN_OK;
    if (!X || !W_qkv || !W_o || !O || !workspace) return fail(ATTN_EINVAL, "mha_fwd: null pointer");
    const size_t need = mha_workspace_bytes(batch, seq, d_model, h, dtype);
    if (workspace_bytes < need)
        return fail(ATTN_EINVAL, "mha_fwd: workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (!aligned(X, 16) || !aligned(W_qkv, 16) || !aligned(W_o, 16) || !aligned(O, 16) || !aligned(workspace, 256))
        return fail(ATTN_EINVAL, "mha_fwd: tensors must be 16-byte aligned, workspace 256-byte aligned");
    const size_t wb = (size_t)d_model * d_model * 2;
    if (overlaps(O, tok * 2, X, tok * 2) || overlaps(O, tok * 2, W_qkv, 3 * wb) || overlaps(O, tok * 2, W_o, wb) ||
        overlaps(workspace, need, X, tok * 2) || overlaps(workspace, need, O, tok * 2) ||
        overlaps(workspace, need, W_qkv, 3 * wb) || overlaps(workspace, need, W_o, wb))
        return fail(ATTN_EINVAL, "mha_fwd: output or workspace overlaps another buffer");

    hipStream_t s = (hipStream_t)stream;
    uint16_t *qkv = (uint16_t *)workspace;  // [3][batch][h][seq][dk]
    uint16_t *ctx = qkv + 3 * tok;          // [batch][seq][h*dk]
    const int dk = d_model / h;
    hipError_t e = tsd::launch_gemm_bf16_qkv_split(X, W_qkv, qkv, batch, seq, d_model, h, s);
    if (e != hipSuccess) return from_hip(e, "mha_fwd projection GEMM");
    e = tsd::launch_attn_bf16(qkv, qkv + tok, qkv + 2 * tok, tsd::kMaskNone, nullptr, 1.0f / sqrtf((float)dk), ctx,
                              0, tsd::kOutBNHD, batch, h, seq, seq, dk, tsd::AttnHeads{h, 1, nullptr}, s);
    if (e != hipSuccess) return from_hip(e, "mha_fwd attention");
    e = tsd::launch_gemm_bf16(ctx, W_o, O, batch * seq, d_model, d_model, s);
    return from_hip(e, "mha_fwd output GEMM");
}

size_t mha_cross_workspace_bytes(int32_t batch, int32_t seq_q, int32_t seq_kv, int32_t d_model, int32_t h,
                                 int32_t dtype)
{
    char saved[sizeof g_last_error];
    snprintf(saved, sizeof saved, "%s", g_last_error);
    const attn_status_t st = seq_kv < 0 ? ATTN_EINVAL : mha_check(batch, seq_q, d_model, h, dtype);
    const attn_status_t st2 = st == ATTN_OK ? mha_check(batch, seq_kv, d_model, h, dtype) : st;
    snprintf(g_last_error, sizeof g_last_error, "%s", saved);
    if (st2 != ATTN_OK) return 0;
    const size_t tq = (size_t)batch * seq_q * d_model, tk = (size_t)batch * seq_kv * d_model;
    return (2 * tq + 2 * tk) * 2;  // q and k, v split into heads + concatenated head outputs, bf16
}

attn_status_t mha_cross_fwd(const void *Xq, const void *Xkv, const void *W_qkv, const void *W_o, int32_t h,
                            int32_t mask_kind, const int32_t *valid_lens, void *O, int32_t batch, int32_t seq_q,
                            int32_t seq_kv, int32_t d_model, int32_t dtype, void *workspace, size_t workspace_bytes,
                            void *stream)
{
    g_last_error[0] = '\0';
    if (seq_kv < 0) return fail(ATTN_EINVAL, "mha_cross_fwd: negative seq_kv");
    attn_status_t st = mha_check(batch, seq_q, d_model, h, dtype);
    if (st != ATTN_OK) return st;
    if (mask_kind != ATTN_MASK_NONE && mask_kind != ATTN_MASK_PADDING)
        return fail(mask_kind == ATTN_MASK_CAUSAL || mask_kind == ATTN_MASK_CAUSAL_PADDING ? ATTN_EUNSUPPORTED
                                                                                            : ATTN_EINVAL,
                    "mha_cross_fwd: mask_kind must be none or padding (got %d)", mask_kind);
    if ((long long)batch * seq_kv > kI32Max) return fail(ATTN_EINVAL, "mha_cross_fwd: batch*seq_kv too large");
    const size_t tq = (size_t)batch * seq_q * d_model, tk = (size_t)batch * seq_kv * d_model;
    if (tq == 0) return ATTN_OK;  // no output row
    const bool padding = mask_kind == ATTN_MASK_PADDING;
    if (!Xq || !W_qkv || !W_o || !O || !workspace || (tk && !Xkv))
        return fail(ATTN_EINVAL, "mha_cross_fwd: null pointer");
    if (padding && !valid_lens) return fail(ATTN_EINVAL, "mha_cross_fwd: padding mask needs valid_lens");
    const size_t need = mha_cross_workspace_bytes(batch, seq_q, seq_kv, d_model, h, dtype);
    if (workspace_bytes < need)
        return fail(ATTN_EINVAL, "mha_cross_fwd: workspace of %zu bytes, need %zu", workspace_bytes, need);
    if (!aligned(Xq, 16) || (Xkv && !aligned(Xkv, 16)) || !aligned(W_qkv, 16) || !aligned(W_o, 16) ||
        !aligned(O, 16) || !aligned(workspace, 256) || (padding && !aligned(valid_lens, 4)))
        return fail(ATTN_EINVAL, "mha_cross_fwd: tensors must be 16-byte aligned, workspace 256-byte aligned");
    const size_t wb = (size_t)d_model * d_model * 2;
    const void *ins[] = {Xq, Xkv, W_qkv, W_o};
    const size_t in_n[] = {tq * 2, tk * 2, 3 * wb, wb};
    for (int j = 0; j < 4; ++j)
        if (overlaps(O, tq * 2, ins[j], in_n[j]) || overlaps(workspace, need, ins[j], in_n[j]))
            return fail(ATTN_EINVAL, "mha_cross_fwd: output or workspace overlaps an input");
    if (overlaps(workspace, need, O, tq * 2)) return fail(ATTN_EINVAL, "mha_cross_fwd: workspace overlaps O");

    hipStream_t s = (hipStream_t)stream;
    const int dk = d_model / h;
    uint16_t *qh = (uint16_t *)workspace;  // [batch][h][seq_q][dk]
    uint16_t *kvh = qh + tq;               // [2][batch][h][seq_kv][dk]
    uint16_t *ctx = kvh + 2 * tk;          // [batch][seq_q][h*dk]
    hipError_t e = tsd::launch_gemm_bf16_heads(Xq, W_qkv, 3 * d_model, qh, batch, seq_q, d_model, d_model, h, s);
    if (e != hipSuccess) return from_hip(e, "mha_cross_fwd query projection GEMM");
    if (tk) {
        e = tsd::launch_gemm_bf16_heads(Xkv, (const uint16_t *)W_qkv + d_model, 3 * d_model, kvh, batch, seq_kv,
                                        2 * d_model, d_model, h, s);
        if (e != hipSuccess) return from_hip(e, "mha_cross_fwd key/value projection GEMM");
    }
    e = tsd::launch_attn_bf16(qh, kvh, kvh + tk, mask_kind, valid_lens, 1.0f / sqrtf((float)dk), ctx, 0, tsd::kOutBNHD,
                              batch, h, seq_q, seq_kv, dk, tsd::AttnHeads{h, 1, nullptr}, s);
    if (e != hipSuccess) return from_hip(e, "mha_cross_fwd attention");
    e = tsd::launch_gemm_bf16(ctx, W_o, O, batch * seq_q, d_model, d_model, s);
    return from_hip(e, "mha_cross_fwd output GEMM");
}

const char *attn_status_string(int32_t status)
{
    switch (status) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported configuration";
    case ATTN_EHIP: return "HIP error";
    default: return "unknown status";
    }
}

const char *attn_last_error(void) { return g_last_error; }

}  // extern "C"
