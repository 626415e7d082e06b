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
// ties by slot) into LDS, and put in pop order when its node is inserted
// (entries whose scores round to the same value ordered by slot), so a
// node's best remaining candidate is the head of its row: the heap becomes "best head over the live nodes", one
// wave-wide maximum per popped candidate.  Lane l owns nodes l and 64 + l
// and keeps their heads, and the entries after them, in registers; a
// candidate is one 64-bit word whose unsigned order is the pop order, and
// its maximum takes a 32-bit pass over the scores plus, on a tie, one over
// the keys.
#include "device_common.hpp"
#include "internal.hpp"

namespace gdn {
namespace {

constexpr int kMaxN = GDN_MAX_NODES;
constexpr int kMaxK = GDN_MAX_CANDIDATES;

// A candidate as one 64-bit word whose unsigned order is the pop order:
// the high half is the score mapped to an order-preserving integer (higher
// score, larger word), the low half (8191 - key) << 8 | depth, so a lower key
// (node * 64 + original slot, the earlier push) wins a tie; the depth of the
// proposing node rides along in the low byte (keys are unique, so it never
// decides).  0 means "no candidate": every real score maps above it.
__device__ __forceinline__ unsigned long long pack(float v, int key, int dep) {
    const uint32_t b = __float_as_uint(v + 0.f);   // -0 -> +0: equal scores, equal words
    const uint32_t o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)o << 32) | ((uint32_t)(8191 - key) << 8) | (uint32_t)dep;
}

__device__ __forceinline__ float unpack_score(unsigned long long w) {
    const uint32_t o = (uint32_t)(w >> 32);
    return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

// one DPP step of a wave-wide maximum of a 32-bit unsigned value (lanes
// with no source see 0, the identity); wave_max32: row_shr 1, 2, 4, 8 leave
// each 16-lane row's maximum in its lane 15, row_bcast 15 and 31 carry
// those into lane 63, which is read out (uniform)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max32(uint32_t x) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xf, false);
    return o > x ? o : x;
}

__device__ __forceinline__ uint32_t wave_max32(uint32_t x) {
    x = dpp_max32<0x111, 0xf>(x);
    x = dpp_max32<0x112, 0xf>(x);
    x = dpp_max32<0x114, 0xf>(x);
    x = dpp_max32<0x118, 0xf>(x);
    x = dpp_max32<0x142, 0xa>(x);
    x = dpp_max32<0x143, 0xc>(x);
    return __builtin_amdgcn_readlane((int)x, 63);
}

// The wave maximum of a 64-bit candidate word in two 32-bit passes: the
// high halves (the scores) first; the low halves only among the lanes that
// hold that score, and when one lane alone holds it (the usual case) its
// word is read directly.  Same word as a 64-bit maximum.
__device__ __forceinline__ unsigned long long wave_max_2level(unsigned long long x) {
    const uint32_t hi = (uint32_t)(x >> 32), lo = (uint32_t)x;
    const uint32_t mhi = wave_max32(hi);
    const unsigned long long tied = __ballot(hi == mhi);
    uint32_t mlo;
    if (__popcll(tied) == 1)
        mlo = __builtin_amdgcn_readlane((int)lo, __ffsll((long long)tied) - 1);
    else
        mlo = wave_max32(hi == mhi ? lo : 0u);
    return ((unsigned long long)mhi << 32) | mlo;
}

// Puts one row of the sorted table in pop order for a node of score sc:
// (rounded score sc + x descending, slot ascending), entries with no
// candidate (x = -inf) last, by slot.  Called only when two distinct
// log-probs of the row may round to the same score (see make_live); kept
// out of line so that the build's round loop does not carry its code.
__device__ __attribute__((noinline)) void pop_order_row(float *lp, unsigned char *js, float sc,
                                                        int K) {
    bool tie = false;
    for (int t = 1; t < K; ++t)
        tie |= lp[t] != -INFINITY && sc + lp[t] == sc + lp[t - 1];
    if (!tie) return;
    float xv[kMaxK];
    int jv[kMaxK];
    for (int t = 0; t < K; ++t) {
        xv[t] = lp[t];
        jv[t] = js[t];
    }
    for (int t = 0; t < K; ++t) {
        const bool ct = xv[t] != -INFINITY;
        const float st = sc + xv[t];
        int rank = 0;
        for (int t2 = 0; t2 < K; ++t2) {
            const bool c2 = xv[t2] != -INFINITY;
            const float s2 = sc + xv[t2];
            const bool before =
                (c2 && !ct) ||
                (c2 == ct && ((c2 && s2 > st) || ((!c2 || s2 == st) && jv[t2] < jv[t])));
            rank += before ? 1 : 0;
        }
        lp[rank] = xv[t];
        js[rank] = (unsigned char)jv[t];
    }
}

// One tree node owned by a lane.  x / j: log-probability and original slot
// of its best remaining candidate (the head of its sorted row); xn / jn: the
// entry after it, read ahead so that advancing the head waits for no LDS.
struct Node {
    bool live;
    int head, dep, par, slot;
    float sc, x, xn;
    int j, jn;
};

// KB: a compile-time bound on K (8, 16 or 32), so that the per-row sort
// unrolls to it with no per-slot branch
template <int KB>
__global__ __launch_bounds__(64) void tree_build_kernel(
    const float *__restrict__ cand_logp, const int32_t *__restrict__ cand_tok,
    const int32_t *__restrict__ root_tok, int32_t *__restrict__ parent_out,
    int32_t *__restrict__ token_out, float *__restrict__ score_out,
    int32_t *__restrict__ n_built_out, int n, int K, int width, int max_depth) {
    __shared__ float s_lp[kMaxN][kMaxK + 2];          // sorted log-probs of each row, -inf padded
    __shared__ unsigned char s_j[kMaxN][kMaxK + 2];   // their original slots
    __shared__ float s_raw[kMaxN * kMaxK];            // the table as read
    __shared__ int32_t s_tok[kMaxN * kMaxK];          // the token ids, for the outputs
    __shared__ unsigned long long s_pop[kMaxN];       // the current round's popped words
    __shared__ float2 s_gap[kMaxN];   // per row: smallest gap between distinct finite
                                      // log-probs, largest |log-prob| (see pop_order)
    const int b = blockIdx.x, l = threadIdx.x;
    const float *lp = cand_logp + (size_t)b * n * K;
    const int32_t *tk = cand_tok + (size_t)b * n * K;

    // ---- stage the table and the token ids in LDS (coalesced; the token
    //      ids are needed only for the outputs, so their loads run under the
    //      whole build), then sort every row: the rank of slot j is the
    //      number of slots that come before it
    for (int e = l; e < n * K; e += 64) {
        s_raw[e] = lp[e];
        s_tok[e] = tk[e];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    // lane l sorts rows l and 64 + l: slot j's rank is the number of slots
    // whose sort word is larger.  The word orders finite slots first, by
    // descending value, then by slot; non-finite slots after them, by slot.
    auto sort_word = [](float v, int j) -> unsigned long long {
        const uint32_t b = __float_as_uint(v + 0.f);   // -0 -> +0
        const uint32_t o = isfinite(v) ? ((b & 0x80000000u) ? ~b : (b | 0x80000000u)) : 0u;
        return ((unsigned long long)o << 32) | (uint32_t)(255 - j);
    };
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = 64 * u + l;
        const bool row = i < n;
        // every slot read at once, from an index clamped into the table (no
        // branch between the reads, so one wait covers them all); slots past
        // K get the word 0, below every slot's word, so they never count
        float v[KB];
        unsigned long long w[KB];
#pragma unroll
        for (int t = 0; t < KB; ++t) v[t] = s_raw[min(i * K + t, kMaxN * kMaxK - 1)];
#pragma unroll
        for (int t = 0; t < KB; ++t) w[t] = (t < K && row) ? sort_word(v[t], t) : 0ull;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
            int rank = 0;
#pragma unroll
            for (int t = 0; t < KB; ++t) rank += w[t] > w[j] ? 1 : 0;
            if (j < K && row) {
                s_lp[i][rank] = isfinite(v[j]) ? v[j] : -INFINITY;
                s_j[i][rank] = (unsigned char)j;
            }
        }
    }
    // two -inf entries past the end of every row, so reading ahead of the
    // head never leaves the row
    for (int i = l; i < n; i += 64) {
        s_lp[i][K] = s_lp[i][K + 1] = -INFINITY;
        s_j[i][K] = s_j[i][K + 1] = 0;
    }
    // per row (the lane's own, sorted above): the smallest gap between
    // adjacent distinct finite log-probs and the largest |log-prob|, for
    // the tie check of pop_order
    for (int i = l; i < n; i += 64) {
        float gap = INFINITY, vmax = 0.f, prev = s_lp[i][0];
        if (prev != -INFINITY) vmax = fabsf(prev);
#pragma unroll
        for (int t = 1; t < KB; ++t) {
            const float x = t < K ? s_lp[i][t] : -INFINITY;
            if (x != -INFINITY) {
                if (x < prev) gap = fminf(gap, prev - x);
                vmax = fmaxf(vmax, fabsf(x));
            }
            prev = x;
        }
        s_gap[i] = make_float2(gap, vmax);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");

    // ---- lane l owns nodes l (u = 0) and 64 + l (u = 1)
    Node nd[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) nd[u] = Node{false, 0, 0, -1, -1, 0.f, -INFINITY, -INFINITY, 0, 0};
    // the candidate word of node u (0: none): live, below the depth cap and
    // with a finite head
    auto cand = [&](int u) -> unsigned long long {
        const Node &d = nd[u];
        const int i = 64 * u + l;
        if (!d.live || d.dep + 1 > max_depth || d.x == -INFINITY) return 0ull;
        return pack(d.sc + d.x, i * 64 + d.j, d.dep);   // one fp32 addition, parent score first
    };
    // Node u becomes live with its head at slot rank 0.  Its row was sorted
    // by log-probability (descending, ties by slot), which gives
    // non-increasing scores sc + x; but two entries whose scores round to the
    // same fp32 value pop by slot (the earlier push), whatever their
    // log-probabilities, and then the row is put in pop order first
    // (pop_order_row).  That can only happen when two distinct log-probs of
    // the row lie closer than the spacing of fp32 values at the scores'
    // magnitude, at most (|sc| + max |x|) 2^-23: the row's smallest gap
    // above twice that rules it out (an infinite score never passes).
    auto make_live = [&](int u) {
        const int i = 64 * u + l;
        nd[u].live = i < n;
        nd[u].head = 0;
        if (i < n) {
            const float2 gp = s_gap[i];
            if (!(gp.x > (fabsf(nd[u].sc) + gp.y) * 0x1p-22f))
                pop_order_row(s_lp[i], s_j[i], nd[u].sc, K);
            nd[u].x = s_lp[i][0];
            nd[u].j = s_j[i][0];
            nd[u].xn = s_lp[i][1];
            nd[u].jn = s_j[i][1];
        }
    };
    // node u's head moves one rank on; the entry after it is read ahead
    auto advance = [&](int u) {
        const int i = 64 * u + l;
        Node &d = nd[u];
        ++d.head;
        d.x = d.xn;
        d.j = d.jn;
        const int r = min(d.head + 1, K + 1);
        d.xn = s_lp[i][r];
        d.jn = s_j[i][r];
    };
    if (l == 0) make_live(0);   // node 0: the root, score 0, depth 0
    unsigned long long c0 = cand(0), c1 = cand(1);

    int nn = 1;
    bool dry = false;
    while (nn < n && !dry) {
        const int cnt = min(width, n - nn);
        int popped = 0;
        for (; popped < cnt; ++popped) {
            const unsigned long long best = wave_max_2level(c0 > c1 ? c0 : c1);
            if (best == 0ull) break;   // nothing left this round
            const int pnode = (8191 - (int)(((uint32_t)best >> 8) & 0xffffffu)) >> 6;
            // the new node (live only from the next round) is recorded by
            // its lane after the round, from this word
            if (l == 0) s_pop[popped] = best;
            // the parent's lane advances its head (u is uniform)
            if ((pnode & 63) == l) {
                if (pnode < 64) {
                    advance(0);
                    c0 = cand(0);
                } else {
                    advance(1);
                    c1 = cand(1);
                }
            }
        }
        // the round's nodes: each lane records its own from the popped
        // words, and they become live
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            const int i = 64 * u + l;
            if (i >= nn && i < nn + popped) {
                const unsigned long long wd = s_pop[i - nn];
                const int key = 8191 - (int)(((uint32_t)wd >> 8) & 0xffffffu);
                nd[u].par = key >> 6;
                nd[u].slot = key & 63;
                nd[u].sc = unpack_score(wd);
                nd[u].dep = (int)(wd & 0xffu) + 1;
                make_live(u);
            }
        }
        c0 = cand(0);
        c1 = cand(1);
        nn += popped;
        // a round that found nothing at all leaves nothing for later rounds
        dry = popped == 0;
    }

    // ---- outputs (rows past the built count: parent -1, token -1, -inf)
    const size_t row0 = (size_t)b * n;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int i = 64 * u + l;
        if (i >= n) {
        } else if (i == 0) {
            parent_out[row0] = -1;
            token_out[row0] = root_tok ? root_tok[b] : -1;
            score_out[row0] = 0.f;
        } else if (i < nn) {
            parent_out[row0 + i] = nd[u].par;
            token_out[row0 + i] = s_tok[nd[u].par * K + nd[u].slot];
            score_out[row0 + i] = nd[u].sc;
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
    if (K <= 8)
        hipLaunchKernelGGL(tree_build_kernel<8>, dim3((unsigned)batch), dim3(64), 0, s, cand_logp,
                           cand_tok, root_tok, parent, token, score, n_built, n, K, width,
                           max_depth);
    else if (K <= 16)
        hipLaunchKernelGGL(tree_build_kernel<16>, dim3((unsigned)batch), dim3(64), 0, s,
                           cand_logp, cand_tok, root_tok, parent, token, score, n_built, n, K,
                           width, max_depth);
    else
        hipLaunchKernelGGL(tree_build_kernel<kMaxK>, dim3((unsigned)batch), dim3(64), 0, s,
                           cand_logp, cand_tok, root_tok, parent, token, score, n_built, n, K,
                           width, max_depth);
    return hipGetLastError();
}

}  // namespace gdn
