// Internal interface between the C-ABI front end (api.hip) and the kernel
// launchers.  Not installed; the public surface is include/gdn_tree.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gdn_tree.h"

namespace gdn {

struct VerifyArgs {
    const void *q, *k, *v;
    gdn_dtype dtype;
    const float *alpha, *beta;
    const int32_t *parent;
    const float *S0;
    float *out;
    int batch, n, H, dk, dv;
    int32_t *status;
    bool status_or = false;   // OR the flags into status[b] instead of overwriting it
};

struct CommitArgs {
    float *S;
    const int32_t *path, *path_len;
    int max_path;
    const void *k, *v;
    gdn_dtype dtype;
    const float *alpha, *beta;
    const int32_t *parent;
    int batch, n, H, dk, dv;
    int32_t *status;
};

// commit of a previous tree's path, then verify of the next tree from the
// committed state (c.S is the verify's S0); both halves share batch, H, d
struct CommitVerifyArgs {
    CommitArgs c;
    VerifyArgs v;
    const void *u_prev;    // previous tree's pseudo-values, or null (solve for them)
    void *u_out;           // this tree's pseudo-values, or null
    bool u_half;           // u_prev / u_out hold fp16 (else fp32)
};

// number of compute units of the current device (cached per device); only
// used to shape work placement, never for correctness
int device_cu_count();

// every launcher returns the launch's hipError_t (hipGetLastError after it)
hipError_t launch_verify_generic(const VerifyArgs &a, hipStream_t s);
hipError_t launch_branch_verify(const VerifyArgs &a, hipStream_t s);
bool verify_split_supports(const VerifyArgs &a);
hipError_t launch_verify_split(const VerifyArgs &a, hipStream_t s);
bool verify_mfma_supports(const VerifyArgs &a);
hipError_t launch_verify_mfma(const VerifyArgs &a, hipStream_t s);
bool verify_mfma128_supports(const VerifyArgs &a);
hipError_t launch_verify_mfma128(const VerifyArgs &a, hipStream_t s);
bool verify_f32_supports(const VerifyArgs &a);
hipError_t launch_verify_f32(const VerifyArgs &a, hipStream_t s);
hipError_t launch_commit(const CommitArgs &a, hipStream_t s);
bool commit_split_supports(const CommitArgs &a);
hipError_t launch_commit_split(const CommitArgs &a, hipStream_t s);
bool commit_mfma_supports(const CommitArgs &a);
hipError_t launch_commit_mfma(const CommitArgs &a, hipStream_t s);
bool commit_f32_supports(const CommitArgs &a);
hipError_t launch_commit_f32(const CommitArgs &a, hipStream_t s);
bool commit_verify_split_supports(const CommitVerifyArgs &a);
hipError_t launch_commit_verify_split(const CommitVerifyArgs &a, hipStream_t s);
bool commit_verify_mfma_supports(const CommitVerifyArgs &a);
hipError_t launch_commit_verify_mfma(const CommitVerifyArgs &a, hipStream_t s);
bool commit_verify_mfma128_supports(const CommitVerifyArgs &a);
hipError_t launch_commit_verify_mfma128(const CommitVerifyArgs &a, hipStream_t s);
hipError_t launch_path(const int32_t *parent, const int32_t *accepted,
                       int32_t *path, int32_t *path_len, int batch, int n,
                       int max_path, int32_t *status, hipStream_t s);
hipError_t launch_accept(const int32_t *parent, const int32_t *draft, const int32_t *verify,
                         int32_t *accepted, int32_t *accept_len, int32_t *bonus, int batch, int n,
                         int32_t *status, hipStream_t s);
hipError_t launch_tree_build(const float *cand_logp, const int32_t *cand_tok,
                             const int32_t *root_tok, int32_t *parent, int32_t *token,
                             float *score, int32_t *n_built, int batch, int n, int K, int width,
                             int max_depth, hipStream_t s);
hipError_t launch_index(const int32_t *parent, int32_t *depth, uint32_t *anc,
                        int batch, int n, int32_t *status, hipStream_t s);

}  // namespace gdn
