/*
 * rra.h -- C ABI of librra.so: RRAttention block-sparse causal prefill
 * attention on AMD Instinct MI355X (gfx950).
 *
 * The method is the one described in "RRAttention: Dynamic Block Sparse
 * Attention via Per-Head Round-Robin Shifts for Long-Context Inference"
 * (arXiv 2602.05853).  Section references below are to that page.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Pointers named q, k, v, kagg, score, mask, idx, cnt, out, workspace are
 *    DEVICE pointers to memory the caller allocated and owns.  The library
 *    never allocates or frees device memory, never synchronises, and keeps no
 *    mutable global state, so calls on different streams may run concurrently
 *    as long as their output buffers do not overlap.  The one exception is
 *    rra_estimate_noalloc, whose intermediates live in a device array of the
 *    library (see there).
 *  - Every call is asynchronous on `stream` (a hipStream_t; NULL is the null
 *    stream).  A successful return means the kernels were enqueued.
 *  - Layouts are dense row-major:
 *        q, out   [Bz, H,   L, d]     bfloat16
 *        k, v     [Bz, Hkv, L, d]     bfloat16
 *        kagg     [Bz, Hkv, Ns, d]    bfloat16, Ns = ceil(L / S)
 *        score    [Bz, H, Nb, Nb]     float32,  Nb = ceil(L / Bk) (§2.1)
 *        mask     [Bz, H, Nb, Nb]     uint8 (1 = key block selected)
 *        idx      [Bz, H, Nb, Nb]     int32, first cnt entries of each row valid
 *        cnt      [Bz, H, Nb]         int32
 *    Query head h reads KV head h / (H / Hkv) (grouped-query attention).
 *    Base pointers of bf16/float/int32 arrays must be 16-byte aligned.
 *  - Every entry point first validates its parameters on the host
 *    (rra_validate) and its pointers; on failure it returns the status and
 *    enqueues nothing.  A failed launch returns RRA_ERR_HIP.  No C++
 *    exception crosses this interface.
 */
#ifndef RRA_H_
#define RRA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RRA_ABI_VERSION 3

typedef enum rra_status {
  RRA_OK = 0,
  RRA_ERR_INVALID_ARG = 1, /* a parameter or pointer is invalid            */
  RRA_ERR_UNSUPPORTED = 2, /* valid for the method but not built (shapes)  */
  RRA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required   */
  RRA_ERR_HIP = 4          /* the HIP runtime reported an error            */
} rra_status_t;

/* Round-robin strategies (§4.3 Round-Robin Strategy ablation: head-RR,
 * layer-RR, hybrid-RR and no RR; the page names them without formulas).
 * The offset o(h) of the sampled query inside every stride, for query head h
 * of layer l = rr_layer, is read as:
 *   RRA_RR_HEAD    o = h mod S              (the method's default, §3.1)
 *   RRA_RR_LAYER   o = l mod S              (same for every head of a layer)
 *   RRA_RR_HYBRID  o = (h + l) mod S
 *   RRA_RR_NONE    o = rr_offset            (fixed, 0 <= rr_offset < S)     */
typedef enum rra_rr_mode {
  RRA_RR_HEAD = 0,
  RRA_RR_LAYER = 1,
  RRA_RR_HYBRID = 2,
  RRA_RR_NONE = 3
} rra_rr_mode_t;

/* Problem description (§2.1: Q, K of one head are L x d, split into
 * ceil(L / Bk) blocks of Bk tokens, the last one possibly partial, with a
 * finer sampling stride S; §3.3: threshold tau; causal prefill, §4.1, or
 * causal = 0 for attention without a causal mask).  Supported: H % Hkv == 0;
 * d in {64, 128}; Bk in {64, 128}; Bk % S == 0 and Bk / S <= 32;
 * ceil(L / Bk) <= 4096; 0 < tau <= 1; causal in {0, 1}; protect_last in
 * {0, 1}; rr_mode in rra_rr_mode_t; rr_layer >= 0; 0 <= rr_offset < S.
 * A zero-filled tail (rr_mode = rr_layer = rr_offset = 0) is head-RR.
 * batch == 0 or seq_len == 0 is a valid empty problem: every entry point
 * returns RRA_OK without touching memory. */
typedef struct rra_params {
  int32_t batch;        /* Bz                                              */
  int32_t num_heads;    /* H, query heads                                  */
  int32_t num_kv_heads; /* Hkv, key/value heads                            */
  int32_t seq_len;      /* L                                               */
  int32_t head_dim;     /* d                                               */
  int32_t stride;       /* S, sampling stride (§2.1)                       */
  int32_t block;        /* Bk, query and key block size (§2.1's B)         */
  float tau;            /* Top-tau threshold (§3.3); 1 keeps every block   */
  int32_t causal;       /* 1: causal (prefill); 0: every key visible       */
  int32_t protect_last; /* 1: the last query-block row keeps every causal
                           key block (§4.3, last query block protection)  */
  float sm_scale;       /* softmax scale; <= 0 means 1/sqrt(head_dim)      */
  int32_t rr_mode;      /* rra_rr_mode_t, 0 = head round-robin             */
  int32_t rr_layer;     /* layer index l for RRA_RR_LAYER / RRA_RR_HYBRID  */
  int32_t rr_offset;    /* fixed offset for RRA_RR_NONE                    */
} rra_params_t;

/* RRA_ABI_VERSION of the loaded library. */
int rra_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* rra_status_str(rra_status_t status);

/* Host-only parameter check; makes no HIP call. */
rra_status_t rra_validate(const rra_params_t* p);

/* Bytes of device workspace rra_estimate needs (*bytes is written). */
rra_status_t rra_estimate_workspace_size(const rra_params_t* p, size_t* bytes);

/* Bytes of the optional device workspace of rra_sparse_attn and
 * rra_dense_attn (*bytes is written; the same for every valid problem). */
rra_status_t rra_attn_workspace_size(const rra_params_t* p, size_t* bytes);

/* Round n float32 values to bfloat16, round to nearest even (used when
 * inputs arrive in float32; the method itself runs on bf16). */
rra_status_t rra_cast_f32_to_bf16(const float* src, void* dst_bf16, int64_t n, void* stream);

/* Stride key aggregation (§3.2: the sum of the key vectors of each stride,
 * normalised by 1/S): kagg[b,g,j,:] = bf16_rne( (sum_{t=jS}^{min(jS+S,L)-1} k[b,g,t,:]) / S ).
 * The sum is formed exactly (float64) and rounded once to bf16; a last
 * partial stride sums the keys it has (still divided by S). */
rra_status_t rra_stride_aggregate(const rra_params_t* p, const void* k, void* kagg, void* stream);

/* Round-robin sampled stride scores, stride softmax and block pooling
 * (§3.1, §3.2, §2.2 query independence).  For query head h the query of
 * stride i is taken at position P(i,h) = i*S + o(h), o(h) = h mod S for
 * head-RR (other strategies: rra_rr_mode_t); its scores
 * s[i,j] = sm_scale * <q[P(i,h)], kagg[j]> over strides j <= i (every j
 * when causal = 0) are softmax normalised per sampled query, and pooled:
 *   score[b,h,I,J] = (1/r_I) * sum_{i in block I} sum_{j in block J, j <= i} p[i,j],
 * r_I the number of sampled queries of block I (Bk / S, fewer in a last
 * partial block, where P(i,h) >= L samples nothing), so every row sums to 1;
 * a block with no sampled query gets a zero row.  Causal: entries with
 * J > I are written as 0. */
rra_status_t rra_block_scores(const rra_params_t* p, const void* q, const void* kagg, float* score,
                              void* stream);

/* Adaptive Top-tau block selection (§3.3; same rule as XAttention's
 * threshold selection).  For each row (b,h,I): order the candidates J in
 * [0, I] ([0, Nb) when causal = 0) by (score desc, J asc) and keep the
 * shortest prefix whose cumulative score reaches tau * (row total); keep
 * every candidate when tau >= 1, when protect_last is set and I == Nb - 1,
 * or when the row total is 0 (no estimate).  Writes the whole mask row (0
 * above the diagonal when causal), idx[b,h,I,0:cnt] strictly ascending, and
 * cnt[b,h,I]. */
rra_status_t rra_top_tau(const rra_params_t* p, const float* score, uint8_t* mask, int32_t* idx,
                         int32_t* cnt, void* stream);

/* The whole estimator: rra_stride_aggregate -> rra_block_scores ->
 * rra_top_tau.  workspace must hold rra_estimate_workspace_size() bytes
 * (kagg, and the score matrix when `score` is NULL).  `score` is optional. */
rra_status_t rra_estimate(const rra_params_t* p, const void* q, const void* k, void* workspace,
                          size_t workspace_bytes, uint8_t* mask, int32_t* idx, int32_t* cnt,
                          float* score, void* stream);

/* Size of the device array behind rra_estimate_noalloc, per GPU. */
#define RRA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

/* rra_estimate for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same kernels and results as rra_estimate, with no workspace argument.
 * Its intermediates (the aggregated keys, and the block scores when `score`
 * is NULL) go to a file-scope device array of RRA_NOALLOC_SCRATCH_BYTES that
 * each GPU the library runs on holds from its first use until the process
 * ends.  Needs Bz*Hkv*ceil(L/S)*d*2 bytes with `score` given, that rounded up
 * to 256 plus Bz*H*Nb*Nb*4 with `score` NULL; a larger problem returns
 * RRA_ERR_WORKSPACE and enqueues nothing.  Calls on one GPU share its array
 * (the last call's contents stay there; nothing in it needs clearing), so
 * calls that overlap in time on the same GPU race: serialise them.  Other
 * arguments, checks and outputs as rra_estimate.  No allocating call is made
 * (the array's device address is looked up once per device). */
rra_status_t rra_estimate_noalloc(const rra_params_t* p, const void* q, const void* k, uint8_t* mask,
                                  int32_t* idx, int32_t* cnt, float* score, void* stream);

/* XAttention's antidiagonal block scores, the comparison estimator for
 * pattern-search time (RR §2.2, §4.2; XAttention summary): inside each S x S
 * cell the lower-left to upper-right antidiagonal of the token scores is
 * summed,
 *   a[i,j] = (sm_scale / S) * sum_{o<S} q[b,h,iS+S-1-o] . k[b,g,jS+o],
 * then softmax per query stride over j <= i and pooled exactly as
 * rra_block_scores does (1/r, r = Bk / S); rows sum to 1, J > I is 0.
 * Run rra_top_tau on the result for XAttention's selection.  Built for
 * L % Bk == 0, causal == 1 and (Bk, S) in {(128,16), (128,8), (128,4),
 * (64,8), (64,4)}; other valid shapes return RRA_ERR_UNSUPPORTED.  The
 * round-robin fields are not used. */
rra_status_t rra_xattn_block_scores(const rra_params_t* p, const void* q, const void* k, float* score,
                                    void* stream);

/* Exact block masses of full causal attention, the reference the estimated
 * block scores approximate (§3.2 with S = 1: every query sampled, every key
 * its own stride; §3.3 Top-tau on it is the exact selection):
 *   mass[b,h,I,J] = (1/n_I) * sum_{t in block I} sum_{u in block J, u <= t} p[t,u],
 *   p[t,u] = softmax over u <= t of sm_scale * q_t . k_u,
 * n_I the tokens of block I (Bk, fewer in a last partial block), every row
 * summing to 1, J > I written as 0 (causal = 0: every key u < L).  mass is float32
 * [Bz, H, Nb, Nb]; S, tau and the round-robin fields are not used.  bf16
 * MFMA, float32 softmax and sums (two passes over the causal keys).  Used to
 * score the estimator's selections (precision / recall against the exact
 * Top-tau set, and the attention mass they keep). */
rra_status_t rra_block_mass(const rra_params_t* p, const void* q, const void* k, float* mass, void* stream);

/* Block-sparse causal flash attention (§4.1, prefill): for query t < L of
 * block I of head h,
 *   out[b,h,t] = sum_{u in A(t)} softmax_u(sm_scale * q_t . k_u) v_u,
 *   A(t) = { u <= t, u < L : block(u) in idx[b,h,I,0:cnt[b,h,I]] }
 * (without u <= t when causal = 0).  idx rows must be strictly ascending
 * key-block indices in [0, I] ([0, Nb) when causal = 0) with
 * 1 <= cnt <= I + 1 (Nb) (rra_top_tau's output satisfies this).  The lists
 * are device data and are not checked: the kernel reads the K / V rows of
 * whatever blocks they name, so an index outside the range reads outside K
 * and V, and a repeated one counts its block twice; cnt = 0 gives a zero
 * output row.  bf16 MFMA, float32 accumulation and online softmax; out is
 * rounded to bf16.
 *
 * workspace (optional, rra_attn_workspace_size() bytes, 16-byte aligned)
 * holds the counters of a dynamic schedule: a fixed set of resident
 * workgroups takes the (b, h, I) rows from one queue per XCD and, once its
 * own queue is empty, from the others, so XCDs that run slower (their clocks
 * differ under the power limit) are not left to finish the launch alone.
 * Its contents on entry do not matter and are unspecified on return; calls
 * that may run at the same time need distinct workspaces.  workspace = NULL
 * launches one workgroup per row instead.  The output is bitwise the same
 * either way.  A workspace smaller than required returns RRA_ERR_WORKSPACE. */
rra_status_t rra_sparse_attn(const rra_params_t* p, const void* q, const void* k, const void* v,
                             const int32_t* idx, const int32_t* cnt, void* out, void* workspace,
                             size_t workspace_bytes, void* stream);

/* Dense flash attention: rra_sparse_attn with every causal key block (every
 * key block when causal = 0) selected (the FlashAttention baseline of
 * §4.1), same kernel and the same optional workspace. */
rra_status_t rra_dense_attn(const rra_params_t* p, const void* q, const void* k, const void* v,
                            void* out, void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RRA_H_ */
