/*
 * sjsa.h - C ABI of the MI355X (gfx950) JSSA sparse-decode library (libsjsa.so).
 *
 * One decode step of token-level top-k sparse attention for GQA, in the joint
 * query-key subspace form of the JSSA article ("JSSA 完全拆解:联合 query-key
 * 子空间打分与 gather-free 内核,训练无关的 token 级稀疏解码"). For every
 * sequence b and KV head h:
 *   q_bar = mean of the G query heads of KV head h        (section 打分误差的定义)
 *   q_hat = M_h q_bar,  s_j = q_hat . Kproj[b,h,j]  for j < n_b
 *   S     = the k positions with the largest s_j          (section JSSA 的整体结构)
 *   out_g = softmax attention of query head g over S, reading the original bf16
 *           K and V in place, with no gather              (section 原理详解(二))
 * The G query heads of a KV head share its index set; each KV head has its own.
 *
 * Conventions shared by every entry point
 *   - Tensors are row-major and contiguous. bf16 is passed as 16-bit patterns.
 *       q      [B, H_q, d]        bf16, H_q = H_kv * G, query head hq -> KV head hq / G
 *       K, V   [B, H_kv, cap, d]  bf16
 *       Kproj  [B, H_kv, cap, r]  bf16 (projected scoring cache, K M^T), or one-byte
 *                                 FP8 E4M3 values with SJSA_FLAG_KPROJ_FP8
 *       M      [H_kv, r, d]       fp32, orthonormal rows (one basis per KV head)
 *       seq_len[B]                int32: tokens valid in each sequence's cache
 *       idx    [B, H_kv, k]       int32
 *       out    [B, H_q, d]        bf16, or fp32 with SJSA_FLAG_OUT_F32
 *   - Every tensor pointer is a DEVICE pointer except the sjsa_shape pointer,
 *     which is host memory. The caller owns every buffer, including the
 *     workspace; the library never allocates, frees or keeps device memory.
 *   - d (head_dim) must be 128; r (rank) 16, 32 or 64; G (group) 1, 2, 4 or 8.
 *   - All device pointers must be 16-byte aligned; the workspace 256-byte aligned.
 *   - seq_len values are read on the device and clamped to [0, cap]; n_b below
 *     means min(max(seq_len[b], 0), cap).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream)
 *     and runs asynchronously; no call synchronizes with the host.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     failed check returns a negative status and enqueues nothing. A launch
 *     failure reported by the HIP runtime returns SJSA_ERR_HIP.
 *   - Calls that share a workspace must not overlap (use one stream or order
 *     them). What one call hands to the next (a unit's step count, the
 *     candidates of the scan) lives in the caller's workspace; the only
 *     process-wide state is the device address of the static scratch array of
 *     sjsa_decode_step_append_noalloc, looked up once per device and kept.
 *   - Results are deterministic: identical inputs give bit-identical outputs.
 */
#ifndef SJSA_H
#define SJSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sjsa_status {
  SJSA_OK = 0,
  SJSA_ERR_NULL = -1,        /* a required pointer is NULL */
  SJSA_ERR_DIMS = -2,        /* a size is out of range */
  SJSA_ERR_UNSUPPORTED = -3, /* d, r, G or flags outside the supported set */
  SJSA_ERR_K = -4,           /* k < 1 or above SJSA_MAX_K */
  SJSA_ERR_WORKSPACE = -5,   /* workspace smaller than the size query returns */
  SJSA_ERR_HIP = -6,         /* the HIP runtime reported a launch error */
  SJSA_ERR_ALIGN = -7,       /* a pointer is not aligned as required */
  SJSA_ERR_SCRATCH = -8      /* the step needs more than the static scratch array holds */
} sjsa_status;

/* sjsa_shape.flags bits.
 * SJSA_FLAG_OUT_F32: `out` is fp32 instead of bf16.
 * SJSA_FLAG_WRITE_SCORES: the score scan also stores every fp32 score in the
 *   workspace (for inspection; see sjsa_score). Results do not change.
 * SJSA_FLAG_KPROJ_FP8: the projected scoring cache Kproj holds OCP FP8 E4M3 values
 *   (one byte each, unscaled, saturating at +-448; the JSSA article's section
 *   投影打分缓存与校准成本 keeps the cache in FP8) instead of bf16. Appends round the
 *   fp32 projection to nearest (ties to even); scoring decodes exactly. */
#define SJSA_FLAG_OUT_F32 1
#define SJSA_FLAG_WRITE_SCORES 2
#define SJSA_FLAG_KPROJ_FP8 4
/* Largest supported token budget per call, and largest cache capacity. */
#define SJSA_MAX_K (1 << 20)
#define SJSA_MAX_CAPACITY ((int64_t)1 << 30)
#define SJSA_MAX_SELECT_UNITS 4096   /* unit (block) budget of the gated and block-sparse steps */
#define SJSA_MAX_BLOCK_SIZE 4096     /* positions per key block of the block-sparse step */
#define SJSA_MAX_FUSED_WAIT_US 1000000  /* largest sjsa_shape.fused_wait_us */

typedef struct sjsa_shape {
  int32_t batch;      /* B >= 1 */
  int32_t n_kv_heads; /* H_kv >= 1 */
  int32_t group;      /* G: query heads per KV head (1, 2, 4, 8) */
  int32_t head_dim;   /* d: must be 128 */
  int32_t rank;       /* r: 16, 32 or 64 */
  int32_t flags;      /* 0 or SJSA_FLAG_* bits */
  int64_t capacity;   /* cap: token slots per (b, h) in K, V, Kproj; 1 .. SJSA_MAX_CAPACITY */
  int32_t fused_wait_us; /* longest wait, in microseconds, of a scan workgroup of the fused
                            prep + scan launch for what its unit's prep publishes (see
                            sjsa_prep_scan): 0 = the default 200; negative = the scan
                            workgroups do not take what the prep publishes at all, so every
                            unit is selected by the exact path (for testing and measuring
                            it); at most SJSA_MAX_FUSED_WAIT_US. Results never depend on it. */
} sjsa_shape;

/*
 * Append n_new tokens per (sequence, KV head) to the caches.
 * Source: JSSA article, section 投影打分缓存与校准成本 (the auxiliary scoring
 * cache Kproj = K M^T sits next to the original KV cache) and section 组件级拆解
 * (projecting each new key is the pipeline's cheapest stage).
 *   k_new, v_new [B, H_kv, n_new, d] bf16 (device)
 *   M            [H_kv, r, d] fp32 (device)
 *   pos          [B] int32 (device): first slot written for sequence b
 * Writes K[b,h,pos_b+t] = k_new[b,h,t], V likewise, and
 * Kproj[b,h,pos_b+t,i] = bf16_rne(sum_c M[h,i,c] * k_new[b,h,t,c]) (fp32 dot).
 * Rows whose slot falls outside [0, cap) are skipped (nothing is written).
 * Errors: SJSA_ERR_NULL, _DIMS (n_new < 1), _UNSUPPORTED, _ALIGN, _HIP.
 */
int sjsa_append_kv(const sjsa_shape* shape, const void* k_new, const void* v_new,
                   int32_t n_new, const float* M, const int32_t* pos,
                   void* K, void* V, void* Kproj, void* stream);

/*
 * Bytes of device workspace that sjsa_decode_step / the stage calls need for
 * this shape and budget k. Returns 0 if the shape or k is invalid.
 */
size_t sjsa_decode_workspace_size(const sjsa_shape* shape, int32_t k);

/*
 * One sparse decode step: the whole pipeline of the JSSA article's section
 * 组件级拆解 (scoring prep, candidate scoring, top-k selection, sparse
 * attention) on one stream. Equivalent to sjsa_score, then sjsa_select, then
 * sjsa_attend on the same workspace.
 *   q [B, H_q, d] bf16; K, V [B, H_kv, cap, d] bf16; Kproj [B, H_kv, cap, r] bf16
 *   M [H_kv, r, d] fp32; seq_len [B] int32; k >= 1 (token budget per KV head)
 *   sm_scale: softmax scale of the final attention; 0 selects 1/sqrt(d)
 *   out [B, H_q, d] (bf16, or fp32 with SJSA_FLAG_OUT_F32); idx [B, H_kv, k]
 * idx[b,h] holds the min(k, n_b) selected positions in ascending order, then -1.
 * Ranking: larger score first, equal scores by lower position, -0 == +0, NaN
 * last. out is zero where n_b = 0.
 * Cost: a unit whose scan candidates cannot be used (more than 16384 of them,
 * which is always so for k > 16384 and n_b > k; fewer than k; or a scan
 * workgroup that gave up waiting, see fused_wait_us) has its scores recomputed
 * and selected exactly: the same result, at about 1.4 times the step's time when
 * every unit of the 128K-token batch-16 step takes that path, and 1.25-1.3 times when
 * the 8 units of one sequence do (a padded slot whose queries are zero, say: all
 * its scores tie, every row is a candidate).
 * Errors: SJSA_ERR_NULL, _DIMS, _UNSUPPORTED, _K, _WORKSPACE, _ALIGN, _HIP.
 */
int sjsa_decode_step(const sjsa_shape* shape, const void* q, const void* K, const void* V,
                     const void* Kproj, const float* M, const int32_t* seq_len,
                     int32_t k, float sm_scale, void* out, int32_t* idx,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * A decode step that first appends the step's new token: the same as
 * sjsa_append_kv with n_new = 1 followed by sjsa_decode_step, with identical
 * results (the K, V and Kproj rows written are bit-identical to the append
 * call's), but the append is done by the first kernel of the step instead of a
 * launch of its own. Source: JSSA article, section 局限 (the current token is
 * appended first and then competes like any other position) and section
 * 投影打分缓存与校准成本 (the scoring cache is extended on append).
 *   k_new, v_new [B, H_kv, 1, d] bf16; pos [B] int32: slot of the new token (a
 *   slot outside [0, cap) writes nothing); seq_len normally pos + 1.
 *   Other arguments as sjsa_decode_step; K, V and Kproj are written.
 * Errors: as sjsa_decode_step.
 */
int sjsa_decode_step_append(const sjsa_shape* shape, const void* k_new, const void* v_new,
                            const int32_t* pos, const void* q, void* K, void* V, void* Kproj,
                            const float* M, const int32_t* seq_len, int32_t k, float sm_scale,
                            void* out, int32_t* idx, void* workspace, size_t workspace_bytes,
                            void* stream);

/*
 * sjsa_decode_step_append with no workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid allocation. The step's scratch memory is a static array
 * inside the library, SJSA_NOALLOC_SCRATCH_BYTES on each GPU the library is loaded
 * on, held until the process ends; the call itself allocates and frees nothing.
 * A shape whose workspace (sjsa_decode_workspace_size(shape, k)) is larger is
 * rejected with SJSA_ERR_SCRATCH before anything is enqueued (with 131072 token
 * slots, r = 32 and k = 4096 that allows up to 58 (sequence, KV head) pairs; one
 * sequence of 32768 tokens with 8 KV heads and k = 2048 needs 2.8 MiB).
 * Every call on one GPU uses that GPU's one array, which keeps the previous call's
 * contents (the step, like a fresh workspace, needs nothing cleared): calls that
 * overlap on one GPU (on different streams, or from host threads without ordering)
 * race and give undefined results. `stream` must belong to the current device.
 * Arguments and results as sjsa_decode_step_append, bit for bit.
 * Errors: as sjsa_decode_step_append, and SJSA_ERR_SCRATCH.
 */
#define SJSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int sjsa_decode_step_append_noalloc(const sjsa_shape* shape, const void* k_new, const void* v_new,
                                    const int32_t* pos, const void* q, void* K, void* V, void* Kproj,
                                    const float* M, const int32_t* seq_len, int32_t k, float sm_scale,
                                    void* out, int32_t* idx, void* stream);

/*
 * Stage 1+2 of the step: scoring prep (q_bar, q_hat; section 打分误差的定义)
 * and the full-context score scan over Kproj (section 原理详解(二): scoring
 * still scans every candidate position). The scan keeps, per (b, h), only the
 * positions whose score reaches a threshold placed by the prep stage from a
 * sample of 2048 rows (one adjacent pair in each of 1024 equal strata, at an
 * offset drawn anew for every unit and step), low enough that the exact top k is
 * among them in all but misjudged cases (which sjsa_select detects and resolves
 * exactly: it then recomputes the unit's scores and selects over all of them);
 * hence the budget k is an argument. With SJSA_FLAG_WRITE_SCORES the
 * scan also stores every fp32 score: that of (b, h, j) is at float offset
 * sjsa_workspace_scores_offset(shape)/4 + (b*H_kv + h)*stride + j, stride =
 * sjsa_workspace_score_stride(shape).
 * Errors: as sjsa_decode_step.
 */
int sjsa_score(const sjsa_shape* shape, const void* q, const void* Kproj, const float* M,
               const int32_t* seq_len, int32_t k, void* workspace, size_t workspace_bytes, void* stream);

/* sjsa_score in two launches, for callers that time the stages separately:
 * sjsa_prep (q_bar, q_hat, the candidate threshold) then sjsa_scan (the score
 * scan over Kproj). Same workspace rules as sjsa_score. */
int sjsa_prep(const sjsa_shape* shape, const void* q, const float* M, const void* Kproj,
              const int32_t* seq_len, int32_t k, void* workspace, size_t workspace_bytes, void* stream);
/* sjsa_prep that first appends the step's new token, as sjsa_decode_step_append
 * does (arguments as there). */
int sjsa_prep_append(const sjsa_shape* shape, const void* k_new, const void* v_new, const int32_t* pos,
                     const void* q, void* K, void* V, void* Kproj, const float* M,
                     const int32_t* seq_len, int32_t k, void* workspace, size_t workspace_bytes,
                     void* stream);
int sjsa_scan(const sjsa_shape* shape, const void* Kproj, const int32_t* seq_len, void* workspace,
              size_t workspace_bytes, void* stream);
/* Stages 1+2 as the decode steps run them: sjsa_prep (or, with k_new non-NULL,
 * sjsa_prep_append with k_new, v_new, pos, K, V as there) and sjsa_scan in one
 * launch, whose scan workgroups take q_hat, the threshold and the appended row
 * from the prep workgroups as soon as each is published. A scan workgroup waits
 * at most shape->fused_wait_us for them (200 us by default; a negative value
 * means it never takes them); past that it marks its tile unusable and
 * sjsa_select handles that unit exactly, so results never depend on the limit. Results are those of
 * the separate calls. The published words are tagged with each unit's step count,
 * kept in the workspace and advanced by sjsa_select: every call of this function
 * must therefore be followed by sjsa_select on the same workspace before the next
 * call of this function there (the decode steps always pair them). The workspace
 * needs no initialisation. With SJSA_FLAG_WRITE_SCORES it makes the two separate
 * launches.
 * Errors: as sjsa_prep_append (K, V, Kproj and pos are checked only when k_new is
 * non-NULL). */
int sjsa_prep_scan(const sjsa_shape* shape, const void* q, const float* M, void* Kproj,
                   const int32_t* seq_len, int32_t k, const void* k_new, const void* v_new,
                   const int32_t* pos, void* K, void* V, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Stage 3: top-k per (b, h) from what sjsa_score left in the workspace -> idx
 * [B, H_kv, k] (Kproj is read again only for a unit whose sampled threshold
 * misjudged the scores). Source: JSSA article, section JSSA 的整体结构
 * (per-KV-head top-k shared by the group's query heads). */
int sjsa_select(const sjsa_shape* shape, const void* Kproj, const int32_t* seq_len, int32_t k,
                int32_t* idx, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Stage 4: gather-free indexed attention (JSSA article, section 原理详解(二):
 * one launch per layer, per-KV-head index sets resolved inside the kernel, K and
 * V read in place). idx [B, H_kv, k] may come from any source: entries < 0 or
 * >= n_b are skipped, and duplicates count as often as they appear.
 */
int sjsa_attend(const sjsa_shape* shape, const void* q, const void* K, const void* V,
                const int32_t* idx, int32_t k, const int32_t* seq_len, float sm_scale,
                void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Top-k of caller-provided fp32 scores: scores [B, H_kv, score_stride], the first
 * n_b entries of each row valid; score_stride >= cap, a multiple of 4. Same
 * ranking and output as sjsa_select. Uses the same workspace as decode.
 */
int sjsa_topk(const sjsa_shape* shape, const float* scores, int64_t score_stride,
              const int32_t* seq_len, int32_t k, int32_t* idx,
              void* workspace, size_t workspace_bytes, void* stream);

/* Workspace layout helpers for reading scores stored with SJSA_FLAG_WRITE_SCORES
 * (host only). */
size_t sjsa_workspace_scores_offset(const sjsa_shape* shape);
int64_t sjsa_workspace_score_stride(const sjsa_shape* shape);

/*
 * Gated-logit sparse decode step. Source: SAS article ("SAS：用门控稀疏注意力把
 * 上下文排序端到端对齐 LM 损失"), section 2.1 (each unit's gate enters the
 * attention logits in log form), section 2.2 (b) (normalized softmax gates; the
 * current block is always kept) and section 2.3 (decode attends only over the
 * units with the largest gates).
 * The cache is split into context units of unit_size consecutive positions; unit
 * i covers [i*unit_size, (i+1)*unit_size). Sequence b has U_b = ceil(n_b/unit_size)
 * units; the last one, which holds position n_b - 1, is the current unit.
 *   q [B, H_q, d] bf16; K, V [B, H_kv, cap, d] bf16; seq_len [B] int32
 *   gate_scores [B, H_kv, gate_stride] fp32: the selector's score u of every unit
 *     (gate_stride >= ceil(cap/unit_size)); the gates are g = softmax(u) over the
 *     U_b units of the sequence. Scores are finite or -inf: a score of -inf gives
 *     its unit a gate of 0, so its positions get zero weight (lambda = 0 drops the
 *     gate term altogether); a query head whose kept positions all have zero weight
 *     gets a zero output. Each sequence with n_b > 0 needs one finite score. NaN and
 *     +inf are not supported (NaN ranks lowest; the output is then unspecified).
 *   Kept units: every unit when U_b <= k_units, else the current unit plus the
 *     k_units - 1 other units with the largest scores (equal scores: lower unit).
 *   idx [B, H_kv, k_units*unit_size]: the kept units' positions below n_b,
 *     ascending, then -1.
 *   out [B, H_q, d]: per query head, the softmax over the kept positions j of
 *     sm_scale * q.k_j + lambda * ln g(unit of j), applied to their V rows
 *     (bf16, or fp32 with SJSA_FLAG_OUT_F32); zero where n_b = 0.
 *   shape: rank and SJSA_FLAG_KPROJ_FP8 are ignored (no scoring cache is read).
 *   1 <= k_units <= SJSA_MAX_SELECT_UNITS, unit_size >= 1,
 *   k_units * unit_size <= SJSA_MAX_K; lambda and sm_scale finite (sm_scale 0
 *   selects 1/sqrt(d)).
 * The workspace (caller-owned, sjsa_gated_workspace_size bytes, 256-byte aligned)
 * holds each position's logit term and the attention partials.
 * Errors: SJSA_ERR_NULL, _DIMS, _UNSUPPORTED, _K, _WORKSPACE, _ALIGN, _HIP.
 */
size_t sjsa_gated_workspace_size(const sjsa_shape* shape, int32_t unit_size, int32_t k_units);
int sjsa_gated_decode_step(const sjsa_shape* shape, const void* q, const void* K, const void* V,
                           const float* gate_scores, int64_t gate_stride, const int32_t* seq_len,
                           int32_t unit_size, int32_t k_units, float lambda, float sm_scale,
                           void* out, int32_t* idx, void* workspace, size_t workspace_bytes,
                           void* stream);

/*
 * Block-sparse decode: block keys, selection of whole key blocks, attention over
 * the kept blocks. Sources: the NSA tutorial page ("稀疏注意力:每个 query 只挑一部分
 * 历史去读"): a block's summary key exists once the block is complete; a block's
 * score is the softmax of q . key / sqrt(head_size) over the visible blocks, summed
 * over the query heads sharing the K/V head, which select together; the current
 * block, the first block and the local blocks are always selected. The
 * SpotAttention abstract page ("SpotAttention: Plug-In Block-Sparse Routing for
 * Pretrained Long-Context Transformers"): the selector's key cache may be INT4.
 * Block j of a sequence covers positions [j*bs, (j+1)*bs); it is complete once
 * n_b >= (j+1)*bs. Block keys are parameter-free: the mean of the block's keys
 * (fp32 sum in position order, divided by bs, rounded to bf16).
 *   Kc [B, H_kv, floor(cap/bs), d] bf16 block keys, and/or the INT4 form:
 *   Kq [B, H_kv, floor(cap/bs), d/2] uint8 (two 4-bit two's-complement codes per
 *   byte, element 2i in the low nibble) with Ks [B, H_kv, floor(cap/bs), d/64] fp16
 *   scales: per group of 64 elements, scale = fp16(absmax / 7) (saturating at 65504)
 *   and code = clamp(rint(x / scale), -7, 7) (0 when the scale is 0), x the bf16 key.
 *   1 <= bs <= SJSA_MAX_BLOCK_SIZE; rank and the Kproj flag of shape are ignored.
 */

/* Keys of every complete block of each sequence (n_b = seq_len[b]). Kc, or Kq with
 * Ks, or all three. Errors: SJSA_ERR_NULL, _DIMS, _UNSUPPORTED, _ALIGN, _HIP. */
int sjsa_block_keys(const sjsa_shape* shape, int32_t block_size, const void* K, const int32_t* seq_len,
                    void* Kc, void* Kq, void* Ks, void* stream);

/* Append n_new tokens per (b, h) at slots pos[b] .. pos[b]+n_new-1 (K and V rows as
 * in sjsa_append_kv, slots outside [0, cap) skipped), then write the keys of the
 * blocks these rows complete (reading the blocks' earlier rows from K).
 * Errors: as sjsa_block_keys, and _DIMS for n_new < 1. */
int sjsa_block_append(const sjsa_shape* shape, int32_t block_size, const void* k_new, const void* v_new,
                      int32_t n_new, const int32_t* pos, void* K, void* V, void* Kc, void* Kq, void* Ks,
                      void* stream);

/* Workspace bytes of sjsa_block_decode_step; 0 if the arguments are invalid. */
size_t sjsa_block_workspace_size(const sjsa_shape* shape, int32_t block_size, int32_t k_blocks);

/*
 * One block-sparse decode step. Scores the complete blocks with the bf16 keys Kc
 * (or, when Kc is NULL, with the INT4 keys Kq, Ks), keeps the forced blocks (the
 * first n_init blocks, and the n_local blocks ending with the current block, the
 * one holding position n_b - 1) and the highest-scoring other complete blocks
 * until k_blocks are kept (equal scores: lower block; every block when a sequence
 * has at most k_blocks), then runs exact softmax attention of every query head
 * over the kept blocks' positions, K and V read in place.
 *   q [B, H_q, d] bf16; K, V [B, H_kv, cap, d] bf16; seq_len [B] int32
 *   idx [B, H_kv, k_blocks*bs]: kept positions below n_b, ascending, then -1
 *   out [B, H_q, d] (bf16, or fp32 with SJSA_FLAG_OUT_F32); zero where n_b = 0
 *   sm_scale scales both the block logits and the attention (0 selects 1/sqrt(d))
 *   1 <= k_blocks <= SJSA_MAX_SELECT_UNITS, k_blocks*bs <= SJSA_MAX_K,
 *   n_init, n_local >= 0 with n_init + n_local <= k_blocks.
 * Errors: SJSA_ERR_NULL, _DIMS, _UNSUPPORTED, _K, _WORKSPACE, _ALIGN, _HIP.
 */
int sjsa_block_decode_step(const sjsa_shape* shape, int32_t block_size, const void* q, const void* K,
                           const void* V, const void* Kc, const void* Kq, const void* Ks,
                           const int32_t* seq_len, int32_t k_blocks, int32_t n_init, int32_t n_local,
                           float sm_scale, void* out, int32_t* idx, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * Calibration of the scoring basis. Source: JSSA article, section 校准:一次前向 +
 * 一次特征分解 (one dense prefill per calibration sequence accumulates, per layer
 * and KV head, the second moments of the group-mean query and of the key; then one
 * eigendecomposition per layer and KV head), section 迹归一化 (unit-trace
 * normalization of each moment) and section 闭式谱解 (basis rows = top-r
 * eigenvectors of the sum of the normalized moments).
 *
 * sjsa_calib_accumulate adds one prefill's sums to fp64 accumulators (device):
 *   q [B, H_q, T, d] bf16 (the prefill's queries), k [B, H_kv, T, d] bf16 (its keys)
 *   SQ[h] += sum over (b, t) of q_bar q_bar^T, q_bar = the decode step's group-mean
 *            query (fp32 sum of the G heads in head order, divided by G)
 *   SK[h] += sum over (b, t) of k k^T          (SQ, SK: [H_kv, d, d] fp64, d = 128)
 * Products are summed in fp32 over at most 256 positions, then in fp64, in a fixed
 * order (deterministic). Only batch, n_kv_heads, group and head_dim of shape are
 * used. The workspace holds per-workgroup fp64 partials
 * (sjsa_calib_workspace_size bytes, 8-byte aligned).
 * Errors: SJSA_ERR_NULL, _DIMS, _UNSUPPORTED, _WORKSPACE, _ALIGN, _HIP.
 */
size_t sjsa_calib_workspace_size(const sjsa_shape* shape, int64_t n_tokens);
int sjsa_calib_accumulate(const sjsa_shape* shape, const void* q, const void* k, int64_t n_tokens,
                          double* SQ, double* SK, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Host (no GPU work): the basis of every KV head from accumulated sums (host
 * memory). A = SQ/tr(SQ) + SK/tr(SK) (symmetrized; the sample count cancels), its
 * eigendecomposition by cyclic Jacobi rotations in fp64, and M[h] = the eigenvectors
 * of the r largest eigenvalues as rows (descending; each row's largest-magnitude
 * component made positive), written as fp32 [H_kv, r, d]. eigenvalues (optional,
 * [H_kv, d] fp64) receives all eigenvalues in descending order.
 * Errors: SJSA_ERR_NULL, _DIMS (r outside 1..d, or a zero or non-finite trace).
 */
int sjsa_calib_basis(const double* SQ, const double* SK, int32_t n_kv_heads, int32_t d, int32_t r, float* M,
                     double* eigenvalues);

/* Static message for a status code. */
const char* sjsa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* SJSA_H */
