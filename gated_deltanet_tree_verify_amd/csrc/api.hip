// C-ABI front end of libgdntree.so: host-side argument validation, kernel
// selection and asynchronous launch on the caller's stream.  The declared
// contract (layouts, ownership, errors) is in include/gdn_tree.h.
#include <stdint.h>

#include <atomic>

#include "internal.hpp"

namespace {

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool dim_ok(int d) { return d >= 8 && d <= GDN_MAX_DIM && d % 8 == 0; }

gdn_status shape_status(int batch, int n, int H, int dk, int dv) {
    if (batch < 1 || n < 1 || H < 1 || dk < 1 || dv < 1) return GDN_ERR_INVALID_ARG;
    if (n > GDN_MAX_NODES || !dim_ok(dk) || !dim_ok(dv)) return GDN_ERR_UNSUPPORTED;
    // element offsets are formed in 64-bit, but grid.x = batch * H must fit
    if ((long long)batch * H > 0x7fffffffLL) return GDN_ERR_UNSUPPORTED;
    return GDN_OK;
}

gdn_status from_hip(hipError_t e) { return e == hipSuccess ? GDN_OK : GDN_ERR_HIP; }

}  // namespace

namespace gdn {

int device_cu_count() {
    constexpr int kMaxDevices = 64;
    static std::atomic<int> cache[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
    int v = cache[dev].load(std::memory_order_relaxed);
    if (v <= 0) {
        if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            v <= 0)
            v = 256;
        cache[dev].store(v, std::memory_order_relaxed);
    }
    return v;
}

}  // namespace gdn

extern "C" {

gdn_status gdn_tree_verify(const void *q, const void *k, const void *v, gdn_dtype qkv_dtype,
                           const float *alpha, const float *beta, const int32_t *parent,
                           const float *S0, float *out, int batch, int n, int H, int d_k,
                           int d_v, int32_t *status, void *stream) {
    if (!q || !k || !v || !alpha || !beta || !parent || !S0 || !out) return GDN_ERR_INVALID_ARG;
    if (qkv_dtype != GDN_DTYPE_F32 && qkv_dtype != GDN_DTYPE_BF16) return GDN_ERR_INVALID_ARG;
    const void *ptrs[] = {q, k, v, alpha, beta, parent, S0, out, status};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;
    const gdn_status st = shape_status(batch, n, H, d_k, d_v);
    if (st != GDN_OK) return st;
    gdn::VerifyArgs a{q, k, v, qkv_dtype, alpha, beta, parent, S0, out,
                      batch, n, H, d_k, d_v, status};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (gdn::verify_split_supports(a)) return from_hip(gdn::launch_verify_split(a, s));
    if (gdn::verify_mfma_supports(a)) return from_hip(gdn::launch_verify_mfma(a, s));
    if (gdn::verify_mfma128_supports(a)) return from_hip(gdn::launch_verify_mfma128(a, s));
    if (gdn::verify_f32_supports(a)) return from_hip(gdn::launch_verify_f32(a, s));
    return from_hip(gdn::launch_verify_generic(a, s));
}

gdn_status gdn_branch_verify(const void *q, const void *k, const void *v, gdn_dtype qkv_dtype,
                             const float *alpha, const float *beta, const int32_t *parent,
                             const float *S0, float *out, int batch, int n, int H, int d_k,
                             int d_v, int32_t *status, void *stream) {
    if (!q || !k || !v || !alpha || !beta || !parent || !S0 || !out) return GDN_ERR_INVALID_ARG;
    if (qkv_dtype != GDN_DTYPE_F32 && qkv_dtype != GDN_DTYPE_BF16) return GDN_ERR_INVALID_ARG;
    const void *ptrs[] = {q, k, v, alpha, beta, parent, S0, out, status};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;
    const gdn_status st = shape_status(batch, n, H, d_k, d_v);
    if (st != GDN_OK) return st;
    gdn::VerifyArgs a{q, k, v, qkv_dtype, alpha, beta, parent, S0, out,
                      batch, n, H, d_k, d_v, status};
    return from_hip(gdn::launch_branch_verify(a, static_cast<hipStream_t>(stream)));
}

gdn_status gdn_tree_commit(float *S, const int32_t *path, const int32_t *path_len, int max_path,
                           const void *k, const void *v, gdn_dtype qkv_dtype, const float *alpha,
                           const float *beta, const int32_t *parent, int batch, int n, int H,
                           int d_k, int d_v, int32_t *status, void *stream) {
    if (!S || !path || !path_len || !k || !v || !alpha || !beta || !parent)
        return GDN_ERR_INVALID_ARG;
    if (qkv_dtype != GDN_DTYPE_F32 && qkv_dtype != GDN_DTYPE_BF16) return GDN_ERR_INVALID_ARG;
    if (max_path < 1) return GDN_ERR_INVALID_ARG;
    const void *ptrs[] = {S, path, path_len, k, v, alpha, beta, parent, status};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;
    const gdn_status st = shape_status(batch, n, H, d_k, d_v);
    if (st != GDN_OK) return st;
    gdn::CommitArgs a{S, path, path_len, max_path, k, v, qkv_dtype, alpha, beta, parent,
                      batch, n, H, d_k, d_v, status};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (gdn::commit_split_supports(a)) return from_hip(gdn::launch_commit_split(a, s));
    if (gdn::commit_mfma_supports(a)) return from_hip(gdn::launch_commit_mfma(a, s));
    if (gdn::commit_f32_supports(a)) return from_hip(gdn::launch_commit_f32(a, s));
    return from_hip(gdn::launch_commit(a, s));
}

gdn_status gdn_tree_commit_verify(float *S, const int32_t *path, const int32_t *path_len,
                                  int max_path, const void *k_prev, const void *v_prev,
                                  const float *alpha_prev, const float *beta_prev,
                                  const int32_t *parent_prev, const void *u_prev, int n_prev,
                                  const void *q, const void *k, const void *v,
                                  gdn_dtype qkv_dtype, const float *alpha, const float *beta,
                                  const int32_t *parent, float *out, void *u_out,
                                  gdn_dtype u_dtype, int batch, int n, int H, int d_k, int d_v,
                                  int32_t *status, void *stream) {
    if (!S || !path || !path_len || !k_prev || !v_prev || !alpha_prev || !beta_prev ||
        !parent_prev || !q || !k || !v || !alpha || !beta || !parent || !out)
        return GDN_ERR_INVALID_ARG;
    if (qkv_dtype != GDN_DTYPE_F32 && qkv_dtype != GDN_DTYPE_BF16) return GDN_ERR_INVALID_ARG;
    if (max_path < 1) return GDN_ERR_INVALID_ARG;
    if ((u_prev || u_out) && u_dtype != GDN_DTYPE_F32 && u_dtype != GDN_DTYPE_F16)
        return GDN_ERR_INVALID_ARG;
    const void *ptrs[] = {S,    path, path_len, k_prev, v_prev, alpha_prev, beta_prev, parent_prev,
                          u_prev, q,  k,        v,      alpha,  beta,       parent,    out,
                          u_out, status};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;
    gdn_status st = shape_status(batch, n_prev, H, d_k, d_v);
    if (st == GDN_OK) st = shape_status(batch, n, H, d_k, d_v);
    if (st != GDN_OK) return st;
    gdn::CommitVerifyArgs a{
        {S, path, path_len, max_path, k_prev, v_prev, qkv_dtype, alpha_prev, beta_prev,
         parent_prev, batch, n_prev, H, d_k, d_v, status},
        {q, k, v, qkv_dtype, alpha, beta, parent, S, out, batch, n, H, d_k, d_v, status, true},
        u_prev,
        u_out,
        u_dtype == GDN_DTYPE_F16};
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (gdn::commit_verify_split_supports(a))
        return from_hip(gdn::launch_commit_verify_split(a, s));
    if (gdn::commit_verify_mfma_supports(a)) return from_hip(gdn::launch_commit_verify_mfma(a, s));
    // 65..128 new nodes: one launch, the commit solving for its
    // pseudo-values (u_prev not needed)
    if (gdn::commit_verify_mfma128_supports(a))
        return from_hip(gdn::launch_commit_verify_mfma128(a, s));
    if (u_out) return GDN_ERR_UNSUPPORTED;
    // other shapes: the two halves as separate launches on the same stream
    // (the commit solves for the pseudo-values itself, so u_prev is not
    // needed), the verify ORing its flag into what the commit wrote
    const hipError_t e = gdn::commit_mfma_supports(a.c) ? gdn::launch_commit_mfma(a.c, s)
                         : gdn::commit_f32_supports(a.c) ? gdn::launch_commit_f32(a.c, s)
                                                         : gdn::launch_commit(a.c, s);
    if (e != hipSuccess) return GDN_ERR_HIP;
    if (gdn::verify_mfma128_supports(a.v)) return from_hip(gdn::launch_verify_mfma128(a.v, s));
    if (gdn::verify_f32_supports(a.v)) return from_hip(gdn::launch_verify_f32(a.v, s));
    return from_hip(gdn::launch_verify_generic(a.v, s));
}

gdn_status gdn_tree_path(const int32_t *parent, const int32_t *accepted, int32_t *path,
                         int32_t *path_len, int batch, int n, int max_path, int32_t *status,
                         void *stream) {
    if (!parent || !accepted || !path || !path_len) return GDN_ERR_INVALID_ARG;
    if (batch < 1 || n < 1 || max_path < 1) return GDN_ERR_INVALID_ARG;
    if (n > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    const void *ptrs[] = {parent, accepted, path, path_len, status};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;
    return from_hip(gdn::launch_path(parent, accepted, path, path_len, batch, n, max_path, status,
                                     static_cast<hipStream_t>(stream)));
}

gdn_status gdn_tree_build(const float *cand_logp, const int32_t *cand_tok, const int32_t *root_tok,
                          int32_t *parent, int32_t *token, float *score, int32_t *n_built,
                          int batch, int n, int K, int width, int max_depth, void *stream) {
    if (!cand_logp || !cand_tok || !parent || !token || !score) return GDN_ERR_INVALID_ARG;
    if (batch < 1 || n < 1 || K < 1 || width < 1 || max_depth < 0) return GDN_ERR_INVALID_ARG;
    if (n > GDN_MAX_NODES || K > GDN_MAX_CANDIDATES) return GDN_ERR_UNSUPPORTED;
    const void *ptrs[] = {cand_logp, cand_tok, root_tok, parent, token, score, n_built};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;
    return from_hip(gdn::launch_tree_build(cand_logp, cand_tok, root_tok, parent, token, score,
                                           n_built, batch, n, K, width, max_depth,
                                           static_cast<hipStream_t>(stream)));
}

gdn_status gdn_tree_accept(const int32_t *parent, const int32_t *draft_tok,
                           const int32_t *verify_tok, int32_t *accepted, int32_t *accept_len,
                           int32_t *bonus_tok, int batch, int n, int32_t *status, void *stream) {
    if (!parent || !draft_tok || !verify_tok || !accepted) return GDN_ERR_INVALID_ARG;
    if (batch < 1 || n < 1) return GDN_ERR_INVALID_ARG;
    if (n > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    const void *ptrs[] = {parent, draft_tok, verify_tok, accepted, accept_len, bonus_tok, status};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;
    return from_hip(gdn::launch_accept(parent, draft_tok, verify_tok, accepted, accept_len,
                                       bonus_tok, batch, n, status,
                                       static_cast<hipStream_t>(stream)));
}

gdn_status gdn_tree_index(const int32_t *parent, int32_t *depth, uint32_t *anc, int batch, int n,
                          int32_t *status, void *stream) {
    if (!parent || !depth || !anc) return GDN_ERR_INVALID_ARG;
    if (batch < 1 || n < 1) return GDN_ERR_INVALID_ARG;
    if (n > GDN_MAX_NODES) return GDN_ERR_UNSUPPORTED;
    const void *ptrs[] = {parent, depth, anc, status};
    for (const void *p : ptrs)
        if (p && !aligned16(p)) return GDN_ERR_INVALID_ARG;
    return from_hip(gdn::launch_index(parent, depth, anc, batch, n, status,
                                      static_cast<hipStream_t>(stream)));
}

const char *gdn_status_string(int status) {
    switch (status) {
        case GDN_OK: return "ok";
        case GDN_ERR_INVALID_ARG: return "invalid argument (null or misaligned pointer, bad size)";
        case GDN_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case GDN_ERR_HIP: return "HIP runtime error at launch";
        default: return "unknown status";
    }
}

int gdn_tree_abi_version(void) { return GDN_TREE_ABI_VERSION; }

}  // extern "C"
