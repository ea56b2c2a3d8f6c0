/*
 * drafter_attn.h -- C ABI of the MI355X (gfx950) drafter block-attention library.
 *
 * What is computed (TensorRT-LLM PR #20532 "Share Kimi K3 FP4 modeling and add NVFP4
 * support on SM103", Conversation: the commit adding k3_drafter_attn and
 * k3_drafter_attn_qknorm, and the commit after it that adds their contracts):
 *
 *   batch     R <= 8 requests with T <= 8 draft tokens each (one block per request)
 *   heads     Hq = 6 * Hkv query heads over Hkv KV heads, head_dim 64; the layouts
 *             the contracts test are 6/1 and 24/4
 *   keys      for each request, its L_r context tokens, kept in HND pages of 64 tokens
 *             named by its page-table row, followed by its b_r block tokens, whose k
 *             and v columns are taken from the packed qkv rows (the pool is never
 *             written)
 *   mask      none: each block token sees every key of its own request
 *   qknorm    drafter_attn_qknorm RMS-normalises each q and k head of the block
 *             (eps 1e-5) and applies the NeoX rotation (base 10000) before attending;
 *             drafter_attn expects q and k already processed
 *   replay    the kernels read lengths, page-table rows, positions and qkv from device
 *             memory at run time, so a call captured in a HIP graph stays correct when
 *             those buffers are rewritten in place between replays
 *   ranges    the contracts test lengths 0 to 2041, dense and padded page-table
 *             strides, and int32 and int64 positions
 *
 * For request r, block token t < b_r, query head h (KV head g = h / 6):
 *
 *   out[r*T+t, h*64:(h+1)*64] = sum_j softmax_j(scale * <q, key_j>) * value_j
 *
 * over the L_r context tokens (token c: slot c%64 of page page_table[r][c/64])
 * followed by the b_r block tokens (k and v heads g of qkv rows r*T .. r*T+b_r-1).
 * In the qknorm variant q and the block's k are first replaced by
 * rope(rmsnorm(x, w), position); context K/V and every v are used as stored.
 *
 * Layouts (bf16 = IEEE bfloat16 bit patterns, little endian):
 *   qkv        [R*T rows][qkv_row_stride elements]; row r*T+t holds q heads
 *              0..Hq-1, then k heads 0..Hkv-1, then v heads 0..Hkv-1, 64 each.
 *   k_pool     page p at k_pool + p*pool_page_stride elements, laid out
 *              [Hkv][64 slots][64 dims] (HND).  v_pool likewise, same stride
 *              (a fused [P][2][Hkv][64][64] pool is v_pool = k_pool + Hkv*4096,
 *              pool_page_stride = 2*Hkv*4096).
 *   page_table int32 [R][page_table_stride], all of it readable memory.  The
 *              kernel loads the entries of each split's page range (see
 *              drafter_attn_plan) before it has the row's length, so any entry of row
 *              r may be loaded; only the first ceil(L_r/64) are used as page ids.  The
 *              others may hold anything: their values are never used.
 *   out        [R*T rows][out_row_stride elements] bf16; rows t >= b_r are
 *              written as zeros.
 *   positions  int32 or int64 [R*T], read per token (row order of qkv).
 *
 * Pointers: every array argument is a DEVICE pointer owned by the caller, except
 * that `stream` is a hipStream_t (NULL = the null stream) and `yarn` a host
 * pointer to a small parameter struct read during the call.  The library
 * allocates nothing and never synchronises the host with the device: calls are
 * asynchronous in `stream` order and may be captured into a HIP graph.
 * The attention calls write only `out`, `workspace` and `status_word`; qkv, the
 * pools and the page table are left bit-identical.  drafter_qk_norm_rope writes
 * the q and k columns of qkv in place and nothing else; drafter_kv_append writes
 * the block's slots of the pools (and status_word) and nothing else.
 *
 * Errors: every shape, stride, alignment, aliasing and workspace check runs on
 * the host before any launch and returns a negative da_status with a message
 * retrievable through drafter_attn_last_error() (thread-local).  Values that
 * live on the device (lengths, page ids, block lengths) cannot be checked
 * without a synchronisation: the kernel clamps them into range so that it never
 * reads outside the arrays described above, and ORs a DA_FLAG_* bit into
 * *status_word when one was out of contract (status_word may be NULL).
 */
#ifndef DRAFTER_ATTN_H
#define DRAFTER_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum da_status {
  DA_OK = 0,
  DA_EINVAL = -1,        /* an argument is outside the contract */
  DA_EUNSUPPORTED = -2,  /* head_dim / page_size / GQA ratio other than 64 / 64 / 6 */
  DA_EWORKSPACE = -3,    /* workspace missing, not 256-byte aligned, or smaller than
                            drafter_attn_workspace_bytes() */
  DA_ELAUNCH = -4        /* the HIP runtime refused the launch (no device, bad stream, ...) */
} da_status;

enum { DA_POS_INT32 = 0, DA_POS_INT64 = 1 };

/* Bits ORed into *status_word by the kernel. */
enum {
  DA_FLAG_CONTEXT_LEN = 1, /* some L_r < 0 or > page_table_stride*64 (clamped) */
  DA_FLAG_PAGE_ID = 2,     /* some referenced page id outside [0, num_pages) (clamped) */
  DA_FLAG_BLOCK_LEN = 4    /* some b_r outside [1, T] (clamped) */
};

/* Hard limits of the contract. */
#define DA_MAX_REQUESTS 8
#define DA_MAX_TOKENS 8
#define DA_MAX_KV_HEADS 16
#define DA_HEAD_DIM 64
#define DA_PAGE_SIZE 64
#define DA_GQA 6
#define DA_MAX_NORM_TOKENS 65536 /* rows per drafter_qk_norm_rope call */

/*
 * Bytes of workspace a call with these sizes needs (0 for arguments outside the
 * contract, a head_dim other than 64 included).  The workspace holds one fp32
 * partial (running max, weight sum, unnormalised output) per (request, KV head,
 * context split) and one 256-byte line of arrival counters per (request, KV head)
 * (word 0; words 1..8 too where a request's splits are combined in two levels).  The workspace must be 256-byte aligned (as hipMalloc returns).
 * The counters must be zero before the first call on a workspace (zero the whole
 * buffer once after allocating it); every call leaves them zero again.  Two calls
 * in flight on one workspace race.
 */
size_t drafter_attn_workspace_bytes(int32_t num_requests, int32_t tokens_per_block,
                                    int32_t num_q_heads, int32_t num_kv_heads,
                                    int32_t head_dim, int32_t page_table_stride);

/*
 * The static split-KV plan for these sizes: S = *num_splits workgroups per
 * (request, KV head), each covering Ps = *pages_per_split pages of the
 * page-table row.  It depends only on these host values.  On the device a request
 * uses only the ranges its context length reaches (at least the first, which also
 * holds the block's own keys).
 *
 * Length-aware schedule: when S > 1 and Ps >= 32, the kernel reads every request's
 * length and may take a balanced plan instead.  With npg_i = ceil(L_i / 64), N =
 * sum npg_i and Pb = the smallest multiple of 8 (at least 8) that is >= ceil(N /
 * (R (S - 1))) and >= ceil(max npg_i / 32), the balanced plan is taken when Pb <=
 * 3 Ps / 4 (rounded down to a multiple of 8).  Request i is then cut into
 * k_i = max(1, ceil(npg_i / Pb)) splits of Pb pages (consecutive entries, at most
 * R * S in all) spread over the same grid of workgroups, so that long requests no
 * longer leave most workgroups idle.  The workspace size is the same for both plans.
 *
 * Either way the schedule is a function of the lengths and the host sizes, so the
 * same inputs always take the same path and the same reduction order: results are
 * bit-identical across reruns and graph replays.  Under the static plan a request's
 * output bits depend only on its own inputs.  Under the balanced plan they also
 * depend on Pb, i.e. on the other requests' lengths: rewriting another request's
 * rows, pages or positions, or its length without moving Pb, leaves them
 * bit-identical; a length that moves Pb moves every request's split boundaries,
 * which changes the last bits of their outputs (within rounding).
 * Returns DA_OK or DA_EINVAL.
 */
int drafter_attn_plan(int32_t num_requests, int32_t num_kv_heads, int32_t page_table_stride,
                      int32_t* num_splits, int32_t* pages_per_split);

/*
 * k3_drafter_attn: q and the block's k are used as given (already normalised and
 * rotated).  scale must be finite and > 0 (usually 1/sqrt(64)).
 * Alignment: qkv, k_pool, v_pool and out 16-byte aligned; page_table,
 * context_lens, block_lens and status_word 4-byte aligned; qkv_row_stride,
 * out_row_stride and pool_page_stride multiples of 8 elements.
 * out must not overlap any input or the workspace.
 */
int drafter_attn(const void* qkv, int64_t qkv_row_stride,
                 const void* k_pool, const void* v_pool, int64_t pool_page_stride,
                 int32_t num_pages,
                 const int32_t* page_table, int32_t page_table_stride,
                 const int32_t* context_lens, const int32_t* block_lens /* NULL = all T */,
                 int32_t num_requests, int32_t tokens_per_block,
                 int32_t num_q_heads, int32_t num_kv_heads,
                 int32_t head_dim, int32_t page_size,
                 float scale,
                 void* workspace, size_t workspace_bytes,
                 void* out, int64_t out_row_stride,
                 int32_t* status_word /* NULL = off */,
                 void* stream /* hipStream_t */);

/*
 * k3_drafter_attn_qknorm: as drafter_attn, but q and the block's k are first
 * normalised, x * w / sqrt(mean(x^2) + eps) over each head's 64 values (q heads
 * use q_norm_weight, k heads k_norm_weight; bf16 [64] each), then rotated NeoX
 * style: dims i and i+32 (i < 32) turn by pos * rope_base^(-2i/64) with pos =
 * positions[r*T+t].  The block's v and the paged context are not touched.
 * eps must be finite and >= 0, rope_base finite and > 0; positions_dtype is
 * DA_POS_INT32 or DA_POS_INT64, and positions aligned to its element size.  The angle is formed and reduced in fp64, the
 * rotation and the norm are computed in fp32, and q/k are rounded to bf16 once
 * before the contractions.
 */
int drafter_attn_qknorm(const void* qkv, int64_t qkv_row_stride,
                        const void* k_pool, const void* v_pool, int64_t pool_page_stride,
                        int32_t num_pages,
                        const int32_t* page_table, int32_t page_table_stride,
                        const int32_t* context_lens, const int32_t* block_lens,
                        int32_t num_requests, int32_t tokens_per_block,
                        int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t head_dim, int32_t page_size,
                        float scale,
                        const void* positions, int32_t positions_dtype,
                        const void* q_norm_weight, const void* k_norm_weight,
                        float eps, float rope_base,
                        void* workspace, size_t workspace_bytes,
                        void* out, int64_t out_row_stride,
                        int32_t* status_word,
                        void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): drafter_attn_qknorm without
 * the workspace arguments.  Arguments, layouts, results, errors and status flags are
 * drafter_attn_qknorm's, bit for bit.  The split partials and arrival counters live in
 * DA_NOALLOC_SCRATCH_BYTES of device memory that the library holds, one array per
 * GPU, kept until the process ends; the call allocates nothing.
 *
 * Limit: 32768 bytes of counters plus R * Hkv * S partial slots of 12,672 bytes (S from
 * drafter_attn_plan; each of the two partial regions rounded up to 256 bytes) must
 * fit in DA_NOALLOC_SCRATCH_BYTES, i.e. at most 1,321 slots (8 x 8 tokens at 24/4 heads
 * with 32k-token contexts uses 256, with 1M-token contexts 1,024).  Larger sizes return
 * DA_EWORKSPACE before anything is launched.
 *
 * The first call on a device (the current device; `stream` must belong to it) looks up
 * the array's device address and clears its counters on `stream`; it must not be under
 * stream capture (DA_EINVAL).  Later calls may be captured.  All calls on one GPU share
 * its array: two calls whose kernels overlap on one GPU (other streams, other host
 * threads) race and give wrong results.
 */
#define DA_NOALLOC_SCRATCH_BYTES (16u << 20)

int drafter_attn_qknorm_noalloc(const void* qkv, int64_t qkv_row_stride,
                                const void* k_pool, const void* v_pool, int64_t pool_page_stride,
                                int32_t num_pages,
                                const int32_t* page_table, int32_t page_table_stride,
                                const int32_t* context_lens, const int32_t* block_lens,
                                int32_t num_requests, int32_t tokens_per_block,
                                int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t page_size,
                                float scale,
                                const void* positions, int32_t positions_dtype,
                                const void* q_norm_weight, const void* k_norm_weight,
                                float eps, float rope_base,
                                void* out, int64_t out_row_stride,
                                int32_t* status_word,
                                void* stream);

/*
 * fused_qk_norm_rope, the drafter's cell (TensorRT-LLM PR #20532, Conversation,
 * the commit adding fused_qk_norm_rope's drafter cell: head_dim 64, 6 query heads
 * per KV head, 1 to 64 tokens, eps 1e-5, base 10000, NeoX; the attention commit
 * says k3_drafter_attn_qknorm uses this op's arithmetic).  In place on qkv: in
 * each of the num_tokens rows every query head is RMS-normalised with
 * q_norm_weight and every key head with k_norm_weight (x * w / sqrt(mean(x^2) +
 * eps), fp32), then NeoX-rotated (dims i and i + 32 by pos * base^(-2i/64), the
 * angle reduced in fp64), and rounded to bf16 once.  Value heads and columns past
 * the heads are not touched.  The arithmetic is the one drafter_attn_qknorm
 * applies to the block's q and k, so drafter_attn on rows processed here gives
 * bit-identical output to drafter_attn_qknorm on the original rows.
 *
 *   qkv        bf16 [num_tokens][qkv_row_stride] (device, read and written)
 *   positions  int32 or int64 [num_tokens] (device, aligned to its element)
 *   q_norm_weight, k_norm_weight  bf16 [64] (device, 16-byte aligned)
 *
 * num_tokens in [1, DA_MAX_NORM_TOKENS]; num_q_heads = 6 * num_kv_heads,
 * num_kv_heads in [1, 16]; head_dim 64 (else DA_EUNSUPPORTED); qkv 16-byte
 * aligned, qkv_row_stride a multiple of 8 elements and >= (Hq + 2*Hkv) * 64;
 * positions and the weights must not overlap qkv; eps finite >= 0, rope_base
 * finite > 0.  Errors are returned before any launch (DA_EINVAL, DA_EUNSUPPORTED,
 * DA_ELAUNCH) with a message in drafter_attn_last_error().  Asynchronous in
 * `stream`; capturable.
 */
int drafter_qk_norm_rope(void* qkv, int64_t qkv_row_stride, int32_t num_tokens,
                         int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                         const void* positions, int32_t positions_dtype,
                         const void* q_norm_weight, const void* k_norm_weight,
                         float eps, float rope_base,
                         void* stream /* hipStream_t */);

/*
 * YaRN rotary scaling.  The drafter checkpoint is named with "YaRN 4.0" (page
 * "K3 DFlash Sequence-Compaction GB300 Validation", Scope and results) and no
 * other parameter, so the caller supplies them.  The method is the published one
 * (Peng, Quesnelle, Fan, Shippole, "YaRN: Efficient Context Window Extension of
 * Large Language Models", 2023, Section 3): rotary pair i (frequency
 * f_i = base^(-2i/64)) turns r_i = original_max_position * f_i / (2 pi) times over
 * the original context; a weight gamma_i of its unscaled frequency, 1 for pairs that
 * turn at least beta times and 0 for pairs that turn at most alpha times, gives the
 * frequency (1 - gamma_i) * f_i / factor + gamma_i * f_i; the rotated q and k are
 * both multiplied by mscale (default 0.1 * ln(factor) + 1, the temperature: logits
 * divided by t).  Between alpha and beta, gamma is linear in
 *   DA_YARN_RAMP_TURNS (0, the paper's):  gamma_i = clamp((r_i - alpha) / (beta - alpha), 0, 1);
 *   DA_YARN_RAMP_INDEX (1):  the pair index: with i(rho) = 32 ln(L / (2 pi rho)) / ln(base)
 *     the fractional pair that turns rho times, lo = floor(i(beta)) and hi = ceil(i(alpha)),
 *     each clamped to [0, 31], gamma_i = 1 - clamp((i - lo) / (hi - lo), 0, 1) -- the
 *     shape checkpoint configurations commonly use;
 *   DA_YARN_RAMP_INDEX_UNROUNDED (2):  the same with lo = i(beta), hi = i(alpha) (clamped,
 *     not rounded).
 * Where the clamped bounds meet (hi <= lo), pairs i <= lo keep f_i and the others take
 * f_i / factor.  The index ramps need rope_base > 1 (frequencies falling along the
 * pairs); a ramp outside the three, a negative or non-finite mscale, or an index ramp
 * with rope_base <= 1 returns DA_EINVAL.  factor 1 with the default mscale is the plain
 * rotation, bit for bit.
 * A zero-filled tail (ramp 0, mscale 0) is the paper's ramp and temperature.
 */
#define DA_YARN_RAMP_TURNS 0
#define DA_YARN_RAMP_INDEX 1
#define DA_YARN_RAMP_INDEX_UNROUNDED 2

typedef struct da_yarn {
  float factor;                  /* >= 1, finite ("YaRN 4.0": 4) */
  int32_t original_max_position; /* >= 1: the context the base rotation was trained on */
  float alpha;                   /* ramp start in turns, >= 0 (published: 1) */
  float beta;                    /* ramp end in turns, > alpha (published: 32) */
  int32_t ramp;                  /* DA_YARN_RAMP_TURNS, _INDEX or _INDEX_UNROUNDED */
  float mscale;                  /* factor on the rotated q and k, finite; 0 = 0.1 ln(factor) + 1
                                    (a checkpoint that folds the temperature into the softmax
                                    scale passes 1 and that scale as `scale`) */
} da_yarn;

/*
 * drafter_attn_qknorm with YaRN-scaled rotation.  Arguments as drafter_attn_qknorm,
 * plus `yarn` (a HOST pointer, read during the call; NULL = the plain rotation,
 * i.e. drafter_attn_qknorm).  Out-of-range YaRN parameters return DA_EINVAL
 * before any launch.
 */
int drafter_attn_qknorm_yarn(const void* qkv, int64_t qkv_row_stride,
                             const void* k_pool, const void* v_pool, int64_t pool_page_stride,
                             int32_t num_pages,
                             const int32_t* page_table, int32_t page_table_stride,
                             const int32_t* context_lens, const int32_t* block_lens,
                             int32_t num_requests, int32_t tokens_per_block,
                             int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t page_size,
                             float scale,
                             const void* positions, int32_t positions_dtype,
                             const void* q_norm_weight, const void* k_norm_weight,
                             float eps, float rope_base, const da_yarn* yarn,
                             void* workspace, size_t workspace_bytes,
                             void* out, int64_t out_row_stride,
                             int32_t* status_word,
                             void* stream);

/*
 * drafter_qk_norm_rope with YaRN-scaled rotation (same arithmetic as
 * drafter_attn_qknorm_yarn's prologue, so drafter_attn on rows processed here
 * equals drafter_attn_qknorm_yarn on the original rows, bit for bit).  `yarn` as
 * there (host pointer, NULL = plain).
 */
int drafter_qk_norm_rope_yarn(void* qkv, int64_t qkv_row_stride, int32_t num_tokens,
                              int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                              const void* positions, int32_t positions_dtype,
                              const void* q_norm_weight, const void* k_norm_weight,
                              float eps, float rope_base, const da_yarn* yarn,
                              void* stream /* hipStream_t */);

/*
 * The path the fused op replaces, built here as an A/B baseline (TensorRT-LLM PR
 * #20532, Conversation, the attention commit: the fused kernel reads the block's
 * K/V from qkv instead of appending them to the cache with append_paged_kv_cache
 * and then running a non-causal context kernel).  Run as drafter_qk_norm_rope (in
 * the qknorm case), drafter_kv_append, then drafter_paged_attn with kv_lens = L + b,
 * it computes the same attention as drafter_attn(_qknorm) on the original rows, at
 * the cost of three launches and pool writes.
 *
 * drafter_kv_append: for every request r, token t < b_r (block_lens, NULL = all T)
 * and KV head g, copies the block's K row (qkv columns (Hq + g) * 64 ..) and V row
 * (columns (Hq + Hkv + g) * 64 ..) to slot (L_r + t) % 64 of page
 * page_table[r * page_table_stride + (L_r + t) / 64] of k_pool / v_pool (device,
 * written).  Layouts, alignment and size limits as for drafter_attn;
 * page_table_stride >= 1.  The pools must not overlap qkv, the page table, the
 * lengths or status_word.  On the device, a request whose L_r + b_r exceeds
 * page_table_stride * 64 is skipped (DA_FLAG_CONTEXT_LEN), a token whose page id
 * is out of [0, num_pages) is skipped (DA_FLAG_PAGE_ID), a b_r outside [1, T] is
 * clamped (DA_FLAG_BLOCK_LEN).  Distinct requests must name distinct pages for
 * their appended slots (two writers of one slot race).
 */
int drafter_kv_append(const void* qkv, int64_t qkv_row_stride,
                      void* k_pool, void* v_pool, int64_t pool_page_stride,
                      int32_t num_pages,
                      const int32_t* page_table, int32_t page_table_stride,
                      const int32_t* context_lens, const int32_t* block_lens /* NULL = all T */,
                      int32_t num_requests, int32_t tokens_per_block,
                      int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, int32_t page_size,
                      int32_t* status_word /* NULL = off */,
                      void* stream /* hipStream_t */);

/*
 * drafter_paged_attn: non-causal paged attention of the block's query rows (q
 * columns of qkv; its k/v columns are not read) over the first kv_lens[r] tokens
 * of each request's paged row only -- no own-block keys are added.  Arguments,
 * layouts, workspace, errors and flags as for drafter_attn, with kv_lens in place
 * of context_lens (kv_lens[r] <= page_table_stride * 64).  A request with no key
 * gets zero rows; rows past the block length are zero.
 */
int drafter_paged_attn(const void* qkv, int64_t qkv_row_stride,
                       const void* k_pool, const void* v_pool, int64_t pool_page_stride,
                       int32_t num_pages,
                       const int32_t* page_table, int32_t page_table_stride,
                       const int32_t* kv_lens, const int32_t* block_lens /* NULL = all T */,
                       int32_t num_requests, int32_t tokens_per_block,
                       int32_t num_q_heads, int32_t num_kv_heads,
                       int32_t head_dim, int32_t page_size,
                       float scale,
                       void* workspace, size_t workspace_bytes,
                       void* out, int64_t out_row_stride,
                       int32_t* status_word /* NULL = off */,
                       void* stream /* hipStream_t */);

/* Message for the last non-DA_OK return on this thread ("" if none). */
const char* drafter_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* DRAFTER_ATTN_H */
