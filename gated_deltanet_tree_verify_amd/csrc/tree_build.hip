// Width-w best-first draft-tree construction (DFlash-TfM page, tree
// construction section): the tree grows from a candidate heap, and each
// round takes the top-w candidates and expands them together, so a budget of
// B nodes takes ceil(B / w) sequential rounds.
//
// Inputs: row i of the candidate table holds the K child candidates that the
// i-th inserted node proposes (log-probabilities, -inf when absent, token
// ids); node ids are insertion order, so every row is known up front.  A
// node's score is its parent's score plus its candidate's log-probability
// (one fp32 addition); candidates deeper than max_depth are not proposed; a
// round pops up to w candidates, best first (higher score, then earlier
// push: lower node id, then lower slot), and the new nodes propose only from
// the next round on.
//
// One wave per sequence.  Every table row is sorted once (descending score,
// ties by slot) into LDS, so a node's best remaining candidate is the head
// of its sorted row: the heap becomes "best head over the live nodes", one
// wave-wide argmax per popped candidate.  Lane l owns nodes l and 64 + l and
// keeps their head value in registers.
#include "device_common.hpp"
#include "internal.hpp"

namespace gdn {
namespace {

constexpr int kMaxN = GDN_MAX_NODES;
constexpr int kMaxK = GDN_MAX_CANDIDATES;

struct Cand {
    float v;   // score of the node's best remaining candidate (-inf: none)
    int key;   // node * 64 + original slot (ties: lower key first)
};

__device__ __forceinline__ bool better(float v, int key, float bv, int bkey) {
    return v > bv || (v == bv && key < bkey);
}

// one DPP step of the wave-wide (value, key) maximum: take the candidate the
// DPP pattern moves into this lane when it is better (lanes with no source
// see the (-inf, max) sentinel)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ void dpp_best(float &bv, int &bk) {
    const float ov = __int_as_float(__builtin_amdgcn_update_dpp(
        (int)0xff800000, __float_as_int(bv), CTRL, ROW_MASK, 0xf, false));
    const int ok = __builtin_amdgcn_update_dpp(0x7fffffff, bk, CTRL, ROW_MASK, 0xf, false);
    if (better(ov, ok, bv, bk)) {
        bv = ov;
        bk = ok;
    }
}

// best (value, key) over the wave, returned uniform: row_shr 1, 2, 4, 8 leave
// each 16-lane row's best in its lane 15; row_bcast 15 and 31 carry those
// into lane 63, which is read out
__device__ __forceinline__ void wave_best(float &bv, int &bk) {
    dpp_best<0x111, 0xf>(bv, bk);
    dpp_best<0x112, 0xf>(bv, bk);
    dpp_best<0x114, 0xf>(bv, bk);
    dpp_best<0x118, 0xf>(bv, bk);
    dpp_best<0x142, 0xa>(bv, bk);
    dpp_best<0x143, 0xc>(bv, bk);
    bv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(bv), 63));
    bk = __builtin_amdgcn_readlane(bk, 63);
}

__global__ __launch_bounds__(64) void tree_build_kernel(
    const float *__restrict__ cand_logp, const int32_t *__restrict__ cand_tok,
    const int32_t *__restrict__ root_tok, int32_t *__restrict__ parent_out,
    int32_t *__restrict__ token_out, float *__restrict__ score_out,
    int32_t *__restrict__ n_built_out, int n, int K, int width, int max_depth) {
    __shared__ float s_lp[kMaxN][kMaxK];          // sorted log-probs of each row
    __shared__ unsigned char s_j[kMaxN][kMaxK];   // their original slots
    __shared__ float s_raw[kMaxN * kMaxK];        // the table as read
    const int b = blockIdx.x, l = threadIdx.x;
    const float *lp = cand_logp + (size_t)b * n * K;

    // ---- stage the table in LDS (coalesced), then sort every row: the rank
    //      of slot j is the number of slots that come before it
    for (int e = l; e < n * K; e += 64) s_raw[e] = lp[e];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    for (int e = l; e < n * K; e += 64) {
        const int i = e / K, j = e % K;
        const float v = s_raw[e];
        const bool fin = isfinite(v);
        int rank = 0;
        for (int t = 0; t < K; ++t) {
            const float u = s_raw[i * K + t];
            const bool ufin = isfinite(u);
            // finite slots first, by descending value, ties by slot
            if (ufin && (!fin || u > v || (u == v && t < j))) ++rank;
            else if (!ufin && !fin && t < j) ++rank;
        }
        s_lp[i][rank] = fin ? v : -INFINITY;
        s_j[i][rank] = (unsigned char)j;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    // ---- per node (two per lane): live flag, head, depth, score, parent, slot
    bool live[2] = {false, false};
    int head[2] = {0, 0}, dep[2] = {0, 0}, par[2] = {-1, -1}, slot[2] = {-1, -1};
    float sc[2] = {0.f, 0.f};
    Cand cur[2];
    auto refresh = [&](int u) {
        const int i = 64 * u + l;
        cur[u].v = -INFINITY;
        cur[u].key = 0x7fffffff;
        if (live[u] && dep[u] + 1 <= max_depth && head[u] < K && i < n) {
            const float x = s_lp[i][head[u]];
            if (x != -INFINITY) {
                cur[u].v = sc[u] + x;   // one fp32 addition, parent score first
                cur[u].key = i * 64 + s_j[i][head[u]];
            }
        }
    };
    if (l == 0) live[0] = true;   // node 0: the root, score 0, depth 0
    refresh(0);
    refresh(1);

    int nn = 1;
    bool dry = false;
    while (nn < n && !dry) {
        const int cnt = min(width, n - nn);
        int popped = 0;
        for (; popped < cnt; ++popped) {
            // best head over the live nodes
            float bv = cur[0].v;
            int bk = cur[0].key;
            if (better(cur[1].v, cur[1].key, bv, bk)) { bv = cur[1].v; bk = cur[1].key; }
            wave_best(bv, bk);
            if (bv == -INFINITY) break;   // nothing left this round
            const int pnode = bk >> 6, pslot = bk & 63;
            const int id = nn + popped;
            // the parent's depth, from the lane that owns it
            const int pdep = __builtin_amdgcn_readlane(pnode < 64 ? dep[0] : dep[1], pnode & 63);
            // the new node's lane records it (live only from the next round)
            if ((id & 63) == l) {
                const int u = id >> 6;
                par[u] = pnode;
                slot[u] = pslot;
                sc[u] = bv;
                dep[u] = pdep + 1;
                head[u] = 0;
            }
            // the parent's lane advances its head
            if ((pnode & 63) == l) {
                const int u = pnode >> 6;
                ++head[u];
                refresh(u);
            }
        }
        // the round's nodes become live
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = 64 * u + l;
            if (i >= nn && i < nn + popped) {
                live[u] = true;
                refresh(u);
            }
        }
        nn += popped;
        // a round that found nothing at all leaves nothing for later rounds
        dry = popped == 0;
    }

    // ---- outputs (rows past the built count: parent -1, token -1, -inf)
    const size_t row0 = (size_t)b * n;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = 64 * u + l;
        if (i >= n) continue;
        if (i == 0) {
            parent_out[row0] = -1;
            token_out[row0] = root_tok ? root_tok[b] : -1;
            score_out[row0] = 0.f;
        } else if (i < nn) {
            parent_out[row0 + i] = par[u];
            token_out[row0 + i] = cand_tok[((size_t)b * n + par[u]) * K + slot[u]];
            score_out[row0 + i] = sc[u];
        } else {
            parent_out[row0 + i] = -1;
            token_out[row0 + i] = -1;
            score_out[row0 + i] = -INFINITY;
        }
    }
    if (l == 0 && n_built_out) n_built_out[b] = nn;
}

}  // namespace

hipError_t launch_tree_build(const float *cand_logp, const int32_t *cand_tok,
                             const int32_t *root_tok, int32_t *parent, int32_t *token,
                             float *score, int32_t *n_built, int batch, int n, int K, int width,
                             int max_depth, hipStream_t s) {
    hipLaunchKernelGGL(tree_build_kernel, dim3((unsigned)batch), dim3(64), 0, s, cand_logp,
                       cand_tok, root_tok, parent, token, score, n_built, n, K, width, max_depth);
    return hipGetLastError();
}

}  // namespace gdn
