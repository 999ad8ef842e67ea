// C ABI of libsjsa: host-side argument validation, workspace layout and launch
// sequencing on the caller's stream. Nothing here allocates device memory.
#include <math.h>
#include <string.h>

#include <atomic>

#include "sjsa_internal.h"

namespace sjsa {
namespace {

constexpr size_t WS_ALIGN = 256;
constexpr int ATT_TARGET_WGS = 1024;   // attention workgroups to aim for (4 per CU)
constexpr int ATT_ALIGN = 64;          // attention splits hold a multiple of 64 entries
// Shortest attention split of the token-level step: a split of 64 rows is one pass of
// its slots, and costs more to start and to merge than it saves (at 8 units, 32 splits
// of 128 rows took the step from 51.5 to 48.2 us; at 16 units from 64.1 to 59.7 us).
constexpr int ATT_MIN_CHUNK = 128;
// The gated step's splits: each repeats its unit's gated selection, and 64-entry splits
// measured faster there (16.2 against 17.2 us graph-replayed at 8 units)
constexpr int GATE_ATT_MIN_CHUNK = 64;
constexpr int ATT_MAX_CHUNK = 1024;    // the attention kernel stages one chunk of indices in LDS
constexpr int BLOCK_ATT_MIN_CHUNK = 128;

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// with_rank = false: the call reads no scoring cache, so rank is not checked.
int check_shape(const sjsa_shape* s, bool with_rank = true) {
  if (!s) return SJSA_ERR_NULL;
  if (s->batch < 1 || s->n_kv_heads < 1 || s->capacity < 1 || s->capacity > SJSA_MAX_CAPACITY) return SJSA_ERR_DIMS;
  if ((int64_t)s->batch * s->n_kv_heads > 65535) return SJSA_ERR_DIMS;     // grid.y limit
  if (s->head_dim != HEAD_DIM) return SJSA_ERR_UNSUPPORTED;
  if (with_rank && s->rank != 16 && s->rank != 32 && s->rank != 64) return SJSA_ERR_UNSUPPORTED;
  if (s->group != 1 && s->group != 2 && s->group != 4 && s->group != 8) return SJSA_ERR_UNSUPPORTED;
  if (s->flags & ~(SJSA_FLAG_OUT_F32 | SJSA_FLAG_WRITE_SCORES | SJSA_FLAG_KPROJ_FP8)) return SJSA_ERR_UNSUPPORTED;
  if (s->fused_wait_us > SJSA_MAX_FUSED_WAIT_US) return SJSA_ERR_DIMS;
  return SJSA_OK;
}

int check_k(int32_t k) { return (k < 1 || k > SJSA_MAX_K) ? SJSA_ERR_K : SJSA_OK; }

float resolve_scale(float sm_scale) {
  return sm_scale != 0.f ? sm_scale : (float)(1.0 / sqrt((double)HEAD_DIM));
}

int status_of(hipError_t e) { return e == hipSuccess ? SJSA_OK : SJSA_ERR_HIP; }

}  // namespace

namespace {

Layout make_layout_split(const sjsa_shape& s, int k, int min_chunk) {
  Layout L;
  L.units = (int64_t)s.batch * s.n_kv_heads;
  L.score_stride = (int64_t)align_up((size_t)s.capacity, 64);
  const int64_t max_split = (k + min_chunk - 1) / min_chunk;
  int64_t want = (ATT_TARGET_WGS + L.units - 1) / L.units;
  want = want < 1 ? 1 : (want > max_split ? max_split : want);
  int64_t chunk = (k + want - 1) / want;
  chunk = (int64_t)align_up((size_t)chunk, ATT_ALIGN);
  if (chunk > ATT_MAX_CHUNK) chunk = ATT_MAX_CHUNK;
  L.chunk = (int)chunk;
  L.nsplit = (int)((k + chunk - 1) / chunk);
  L.tile_rows = tile_rows(s.rank * ((s.flags & SJSA_FLAG_KPROJ_FP8) != 0 ? 1 : 2));
  L.ntile = (s.capacity + L.tile_rows - 1) / L.tile_rows;
  const int64_t rows_min = tile_rows(s.rank * 2);
  L.ntile_cap = (s.capacity + rows_min - 1) / rows_min;
  L.cand_stride = (s.capacity + TILE_ROWS_MAX - 1) / TILE_ROWS_MAX * TILE_ROWS_MAX;
  size_t off = 0;
  L.off_qhat = off;
  off = align_up(off + (size_t)L.units * QHAT_STRIDE * sizeof(float), WS_ALIGN);
  L.off_tlow = off;
  off = align_up(off + (size_t)L.units * 2 * sizeof(uint32_t), WS_ALIGN);
  L.off_epoch = off;
  off = align_up(off + (size_t)L.units * sizeof(uint32_t), WS_ALIGN);
  L.off_sync = off;
  off = align_up(off + (size_t)L.units * SYNC_WORDS * sizeof(uint64_t), WS_ALIGN);
  L.off_counts = off;
  off = align_up(off + (size_t)L.units * L.ntile_cap * sizeof(uint64_t), WS_ALIGN);
  L.off_arrive = off;
  off = align_up(off + (size_t)L.units * sizeof(uint32_t), WS_ALIGN);
  L.off_parthist = off;
  off = align_up(off + (size_t)L.units * EXACT_WGS * HIST_BINS * sizeof(uint32_t), WS_ALIGN);
  L.off_cand = off;
  off = align_up(off + (size_t)L.units * L.cand_stride * sizeof(uint32_t), WS_ALIGN);
  L.off_scores = off;
  off = align_up(off + (size_t)L.units * L.score_stride * sizeof(float), WS_ALIGN);
  L.scores_end = off;
  L.off_partials = off;
  const size_t part = L.nsplit > 1 ? (size_t)L.units * L.nsplit * s.group * PART_STRIDE * sizeof(float) : 0;
  off = align_up(off + part, WS_ALIGN);
  L.total = off;
  return L;
}

}  // namespace

Layout make_layout(const sjsa_shape& s, int k) { return make_layout_split(s, k, ATT_MIN_CHUNK); }

Layout make_gated_layout(const sjsa_shape& s, int ktok) {
  const Layout A = make_layout_split(s, ktok, GATE_ATT_MIN_CHUNK);   // attention split of a ktok-entry index list
  Layout L;
  L.units = A.units;
  L.nsplit = A.nsplit;
  L.chunk = A.chunk;
  size_t off = 0;
  L.off_bias = off;
  off = align_up(off + (size_t)L.units * ktok * sizeof(float), WS_ALIGN);
  L.off_partials = off;
  const size_t part = L.nsplit > 1 ? (size_t)L.units * L.nsplit * s.group * PART_STRIDE * sizeof(float) : 0;
  off = align_up(off + part, WS_ALIGN);
  L.scores_end = L.off_partials;
  L.total = off;
  return L;
}

BlockLayout make_block_layout(const sjsa_shape& s, int block_size, int k_blocks) {
  BlockLayout B;
  const int ktok = block_size * k_blocks;
  const Layout A = make_layout(s, ktok);
  B.nblk_cap = s.capacity / block_size;
  B.zstride = (int64_t)align_up((size_t)B.nblk_cap, 64);
  B.ntile = (int)((B.nblk_cap + 63) / 64);
  const size_t units = (size_t)A.units;
  size_t off = 0;
  B.off_z = off;
  off = align_up(off + units * s.group * B.zstride * sizeof(float), WS_ALIGN);
  B.off_ms = off;
  off = align_up(off + units * B.ntile * s.group * 2 * sizeof(float), WS_ALIGN);
  B.att.units = A.units;
  // splits of at least BLOCK_ATT_MIN_CHUNK entries: the block step's G = 8 attention
  // splits cost more to start and to merge than their share of a short list saves
  // (at 4 x 8 units, 1024 entries: 8 splits took the step from 32.7 to 30.9 us, 4
  // made it 33.2)
  B.att.chunk = A.chunk < BLOCK_ATT_MIN_CHUNK && BLOCK_ATT_MIN_CHUNK <= ktok ? BLOCK_ATT_MIN_CHUNK : A.chunk;
  B.att.nsplit = (ktok + B.att.chunk - 1) / B.att.chunk;
  B.att.off_partials = off;
  const size_t part = B.att.nsplit > 1 ? units * B.att.nsplit * s.group * PART_STRIDE * sizeof(float) : 0;
  off = align_up(off + part, WS_ALIGN);
  B.att.total = off;
  B.total = off;
  return B;
}

}  // namespace sjsa

using namespace sjsa;

namespace {

int check_blocks(const sjsa_shape* shape, int32_t block_size) {
  int st = check_shape(shape, false);
  if (st) return st;
  if (block_size < 1 || block_size > SJSA_MAX_BLOCK_SIZE) return SJSA_ERR_DIMS;
  return SJSA_OK;
}

int check_gated(const sjsa_shape* shape, int32_t unit_size, int32_t k_units) {
  int st = check_shape(shape, false);
  if (st) return st;
  if (unit_size < 1 || k_units < 1 || k_units > SJSA_MAX_SELECT_UNITS) return SJSA_ERR_DIMS;
  if ((int64_t)unit_size * k_units > SJSA_MAX_K) return SJSA_ERR_K;
  return SJSA_OK;
}

}  // namespace

extern "C" {

const char* sjsa_status_string(int status) {
  switch (status) {
    case SJSA_OK: return "ok";
    case SJSA_ERR_NULL: return "a required pointer is NULL";
    case SJSA_ERR_DIMS: return "a size is out of range";
    case SJSA_ERR_UNSUPPORTED: return "head_dim, rank, group or flags outside the supported set";
    case SJSA_ERR_K: return "k is below 1 or above SJSA_MAX_K";
    case SJSA_ERR_WORKSPACE: return "workspace is smaller than required";
    case SJSA_ERR_HIP: return "the HIP runtime reported a launch error";
    case SJSA_ERR_ALIGN: return "a pointer is not aligned as required";
    case SJSA_ERR_SCRATCH:
      return "the step needs more scratch memory than the library's static array holds (SJSA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

size_t sjsa_decode_workspace_size(const sjsa_shape* shape, int32_t k) {
  if (check_shape(shape) != SJSA_OK || check_k(k) != SJSA_OK) return 0;
  return make_layout(*shape, k).total;
}

size_t sjsa_workspace_scores_offset(const sjsa_shape* shape) {
  if (check_shape(shape) != SJSA_OK) return 0;
  return make_layout(*shape, 1).off_scores;
}

int64_t sjsa_workspace_score_stride(const sjsa_shape* shape) {
  if (check_shape(shape) != SJSA_OK) return 0;
  return make_layout(*shape, 1).score_stride;
}

int sjsa_append_kv(const sjsa_shape* shape, const void* k_new, const void* v_new, int32_t n_new,
                   const float* M, const int32_t* pos, void* K, void* V, void* Kproj, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if (!k_new || !v_new || !M || !pos || !K || !V || !Kproj) return SJSA_ERR_NULL;
  if (n_new < 1) return SJSA_ERR_DIMS;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(K, 16) || !aligned(V, 16) ||
      !aligned(Kproj, 16) || !aligned(M, 16) || !aligned(pos, 4))
    return SJSA_ERR_ALIGN;
  if ((n_new + 63) / 64 > 2147483647) return SJSA_ERR_DIMS;
  return status_of(launch_append(*shape, (const uint16_t*)k_new, (const uint16_t*)v_new, n_new, M, pos,
                                 (uint16_t*)K, (uint16_t*)V, Kproj, (hipStream_t)stream));
}

}  // extern "C"

namespace {

// Validation shared by the fused append entry points (one new token per sequence).
int check_append_one(const void* k_new, const void* v_new, const int32_t* pos, const void* K, const void* V,
                     const void* Kproj) {
  if (!k_new || !v_new || !pos || !K || !V || !Kproj) return SJSA_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(pos, 4)) return SJSA_ERR_ALIGN;
  return SJSA_OK;
}

PrepAppend make_append(const void* k_new, const void* v_new, const int32_t* pos, void* K, void* V, void* Kproj) {
  PrepAppend ap;
  ap.k_new = (const uint16_t*)k_new;
  ap.v_new = (const uint16_t*)v_new;
  ap.pos = pos;
  ap.K = (uint16_t*)K;
  ap.V = (uint16_t*)V;
  ap.Kproj = (unsigned char*)Kproj;
  return ap;
}

}  // namespace

extern "C" {

int sjsa_score(const sjsa_shape* shape, const void* q, const void* Kproj, const float* M,
               const int32_t* seq_len, int32_t k, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if (!q || !Kproj || !M || !seq_len || !workspace) return SJSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(Kproj, 16) || !aligned(M, 16) || !aligned(seq_len, 4) ||
      !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  const Layout L = make_layout(*shape, k);
  if (workspace_bytes < L.scores_end) return SJSA_ERR_WORKSPACE;
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_prep(*shape, L, (const uint16_t*)q, M, (const void*)Kproj, seq_len, k, ws, s);
  if (e == hipSuccess) e = launch_score(*shape, L, (const void*)Kproj, seq_len, ws, s);
  return status_of(e);
}

int sjsa_prep(const sjsa_shape* shape, const void* q, const float* M, const void* Kproj, const int32_t* seq_len,
              int32_t k, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if (!q || !M || !Kproj || !seq_len || !workspace) return SJSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(M, 16) || !aligned(Kproj, 16) || !aligned(seq_len, 4) ||
      !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  const Layout L = make_layout(*shape, k);
  if (workspace_bytes < L.scores_end) return SJSA_ERR_WORKSPACE;
  return status_of(launch_prep(*shape, L, (const uint16_t*)q, M, (const void*)Kproj, seq_len, k,
                               (unsigned char*)workspace, (hipStream_t)stream));
}

int sjsa_prep_append(const sjsa_shape* shape, const void* k_new, const void* v_new, const int32_t* pos,
                     const void* q, void* K, void* V, void* Kproj, const float* M, const int32_t* seq_len,
                     int32_t k, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if ((st = check_append_one(k_new, v_new, pos, K, V, Kproj))) return st;
  if (!q || !M || !seq_len || !workspace) return SJSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(M, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(Kproj, 16) ||
      !aligned(seq_len, 4) || !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  const Layout L = make_layout(*shape, k);
  if (workspace_bytes < L.scores_end) return SJSA_ERR_WORKSPACE;
  const PrepAppend ap = make_append(k_new, v_new, pos, K, V, Kproj);
  return status_of(launch_prep(*shape, L, (const uint16_t*)q, M, (const void*)Kproj, seq_len, k,
                               (unsigned char*)workspace, (hipStream_t)stream, &ap));
}

int sjsa_scan(const sjsa_shape* shape, const void* Kproj, const int32_t* seq_len, void* workspace,
              size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if (!Kproj || !seq_len || !workspace) return SJSA_ERR_NULL;
  if (!aligned(Kproj, 16) || !aligned(seq_len, 4) || !aligned(workspace, WS_ALIGN)) return SJSA_ERR_ALIGN;
  const Layout L = make_layout(*shape, 1);
  if (workspace_bytes < L.scores_end) return SJSA_ERR_WORKSPACE;
  return status_of(launch_score(*shape, L, (const void*)Kproj, seq_len, (unsigned char*)workspace,
                                (hipStream_t)stream));
}

int sjsa_prep_scan(const sjsa_shape* shape, const void* q, const float* M, void* Kproj, const int32_t* seq_len,
                   int32_t k, const void* k_new, const void* v_new, const int32_t* pos, void* K, void* V,
                   void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if (k_new && (st = check_append_one(k_new, v_new, pos, K, V, Kproj))) return st;
  if (!q || !M || !Kproj || !seq_len || !workspace) return SJSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(M, 16) || !aligned(Kproj, 16) || !aligned(seq_len, 4) ||
      !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  if (k_new && (!aligned(K, 16) || !aligned(V, 16))) return SJSA_ERR_ALIGN;
  const Layout L = make_layout(*shape, k);
  if (workspace_bytes < L.scores_end) return SJSA_ERR_WORKSPACE;
  const PrepAppend ap = make_append(k_new, v_new, pos, K, V, Kproj);
  return status_of(launch_prep_scan(*shape, L, (const uint16_t*)q, M, (const void*)Kproj, seq_len, k,
                                    (unsigned char*)workspace, (hipStream_t)stream, k_new ? &ap : nullptr));
}

int sjsa_select(const sjsa_shape* shape, const void* Kproj, const int32_t* seq_len, int32_t k, int32_t* idx,
                void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if (!Kproj || !seq_len || !idx || !workspace) return SJSA_ERR_NULL;
  if (!aligned(Kproj, 16) || !aligned(seq_len, 4) || !aligned(idx, 4) || !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  const Layout L = make_layout(*shape, k);
  if (workspace_bytes < L.scores_end) return SJSA_ERR_WORKSPACE;
  return status_of(launch_select(*shape, L, nullptr, 0, (const void*)Kproj, seq_len, k, idx,
                                 (unsigned char*)workspace, (hipStream_t)stream));
}

int sjsa_topk(const sjsa_shape* shape, const float* scores, int64_t score_stride, const int32_t* seq_len,
              int32_t k, int32_t* idx, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if (!scores || !seq_len || !idx || !workspace) return SJSA_ERR_NULL;
  if (score_stride < shape->capacity || (score_stride % 4) != 0) return SJSA_ERR_DIMS;
  if (!aligned(scores, 16) || !aligned(seq_len, 4) || !aligned(idx, 4) || !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  const Layout L = make_layout(*shape, k);
  if (workspace_bytes < L.scores_end) return SJSA_ERR_WORKSPACE;
  return status_of(launch_select(*shape, L, scores, score_stride, nullptr, seq_len, k, idx,
                                 (unsigned char*)workspace, (hipStream_t)stream));
}

int sjsa_attend(const sjsa_shape* shape, const void* q, const void* K, const void* V, const int32_t* idx,
                int32_t k, const int32_t* seq_len, float sm_scale, void* out, void* workspace,
                size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if (!q || !K || !V || !idx || !seq_len || !out || !workspace) return SJSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(idx, 4) || !aligned(seq_len, 4) ||
      !aligned(out, 16) || !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  if (!isfinite(sm_scale)) return SJSA_ERR_DIMS;
  const Layout L = make_layout(*shape, k);
  if (workspace_bytes < L.total) return SJSA_ERR_WORKSPACE;
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const hipError_t e = launch_attend(*shape, L, (const uint16_t*)q, (const uint16_t*)K, (const uint16_t*)V, idx, k,
                                     seq_len, resolve_scale(sm_scale), out, ws, s);
  return status_of(e);
}

int sjsa_decode_step(const sjsa_shape* shape, const void* q, const void* K, const void* V, const void* Kproj,
                     const float* M, const int32_t* seq_len, int32_t k, float sm_scale, void* out, int32_t* idx,
                     void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if (!q || !K || !V || !Kproj || !M || !seq_len || !out || !idx || !workspace) return SJSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(Kproj, 16) || !aligned(M, 16) ||
      !aligned(seq_len, 4) || !aligned(idx, 4) || !aligned(out, 16) || !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  if (!isfinite(sm_scale)) return SJSA_ERR_DIMS;
  const Layout L = make_layout(*shape, k);
  if (workspace_bytes < L.total) return SJSA_ERR_WORKSPACE;
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_prep_scan(*shape, L, (const uint16_t*)q, M, (const void*)Kproj, seq_len, k, ws, s);
  if (e == hipSuccess) e = launch_select(*shape, L, nullptr, 0, (const void*)Kproj, seq_len, k, idx, ws, s);
  if (e == hipSuccess)
    e = launch_attend(*shape, L, (const uint16_t*)q, (const uint16_t*)K, (const uint16_t*)V, idx, k, seq_len,
                      resolve_scale(sm_scale), out, ws, s);
  return status_of(e);
}

int sjsa_decode_step_append(const sjsa_shape* shape, const void* k_new, const void* v_new, const int32_t* pos,
                            const void* q, void* K, void* V, void* Kproj, const float* M, const int32_t* seq_len,
                            int32_t k, float sm_scale, void* out, int32_t* idx, void* workspace,
                            size_t workspace_bytes, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if ((st = check_append_one(k_new, v_new, pos, K, V, Kproj))) return st;
  if (!q || !M || !seq_len || !out || !idx || !workspace) return SJSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(Kproj, 16) || !aligned(M, 16) ||
      !aligned(seq_len, 4) || !aligned(idx, 4) || !aligned(out, 16) || !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  if (!isfinite(sm_scale)) return SJSA_ERR_DIMS;
  const Layout L = make_layout(*shape, k);
  if (workspace_bytes < L.total) return SJSA_ERR_WORKSPACE;
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const PrepAppend ap = make_append(k_new, v_new, pos, K, V, Kproj);
  hipError_t e = launch_prep_scan(*shape, L, (const uint16_t*)q, M, (const void*)Kproj, seq_len, k, ws, s, &ap);
  if (e == hipSuccess) e = launch_select(*shape, L, nullptr, 0, (const void*)Kproj, seq_len, k, idx, ws, s);
  if (e == hipSuccess)
    e = launch_attend(*shape, L, (const uint16_t*)q, (const uint16_t*)K, (const uint16_t*)V, idx, k, seq_len,
                      resolve_scale(sm_scale), out, ws, s);
  return status_of(e);
}

}  // extern "C"

namespace {

// Scratch memory of sjsa_decode_step_append_noalloc: a static device array, one copy
// per GPU the library is loaded on. In host code `scratch` names a host-side stand-in,
// not device memory: kernels get the device address from hipGetSymbolAddress, taken
// once per device (with that device current) and kept here.
__device__ __align__(256) unsigned char scratch[SJSA_NOALLOC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_scratch_ptr[MAX_DEVICES];

// Device address of the current device's scratch array (null on failure). Threads
// that race on a device's first call both store the same address.
void* scratch_ptr(int dev) {
  if (dev < 0 || dev >= MAX_DEVICES) return nullptr;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  void* q = nullptr;
  if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) return nullptr;
  g_scratch_ptr[dev].store(q, std::memory_order_release);
  return q;
}

}  // namespace

extern "C" {

int sjsa_decode_step_append_noalloc(const sjsa_shape* shape, const void* k_new, const void* v_new,
                                    const int32_t* pos, const void* q, void* K, void* V, void* Kproj,
                                    const float* M, const int32_t* seq_len, int32_t k, float sm_scale,
                                    void* out, int32_t* idx, void* stream) {
  int st = check_shape(shape);
  if (st) return st;
  if ((st = check_k(k))) return st;
  if (make_layout(*shape, k).total > SJSA_NOALLOC_SCRATCH_BYTES) return SJSA_ERR_SCRATCH;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return SJSA_ERR_HIP;
  if (stream) {
    hipDevice_t sdev = -1;
    if (hipStreamGetDevice((hipStream_t)stream, &sdev) != hipSuccess || sdev != dev) return SJSA_ERR_HIP;
  }
  void* ws = scratch_ptr(dev);
  if (!ws) return SJSA_ERR_HIP;
  return sjsa_decode_step_append(shape, k_new, v_new, pos, q, K, V, Kproj, M, seq_len, k, sm_scale, out, idx, ws,
                                 SJSA_NOALLOC_SCRATCH_BYTES, stream);
}

size_t sjsa_gated_workspace_size(const sjsa_shape* shape, int32_t unit_size, int32_t k_units) {
  if (check_gated(shape, unit_size, k_units) != SJSA_OK) return 0;
  return make_gated_layout(*shape, unit_size * k_units).total;
}

int sjsa_gated_decode_step(const sjsa_shape* shape, const void* q, const void* K, const void* V,
                           const float* gate_scores, int64_t gate_stride, const int32_t* seq_len,
                           int32_t unit_size, int32_t k_units, float lambda, float sm_scale, void* out,
                           int32_t* idx, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_gated(shape, unit_size, k_units);
  if (st) return st;
  if (!q || !K || !V || !gate_scores || !seq_len || !out || !idx || !workspace) return SJSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(gate_scores, 4) ||
      !aligned(seq_len, 4) || !aligned(idx, 4) || !aligned(out, 16) || !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  if (gate_stride < (shape->capacity + unit_size - 1) / unit_size) return SJSA_ERR_DIMS;
  if (!isfinite(sm_scale) || !isfinite(lambda)) return SJSA_ERR_DIMS;
  const int ktok = unit_size * k_units;
  const Layout L = make_gated_layout(*shape, ktok);
  if (workspace_bytes < L.total) return SJSA_ERR_WORKSPACE;
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  if ((shape->capacity + unit_size - 1) / unit_size <= GATE_FUSED_UNITS_MAX && k_units <= GATE_FUSED_KEPT_MAX) {
    // every attention workgroup makes its unit's selection itself: no selection launch
    GatedSelect g;
    g.gate_scores = gate_scores;
    g.gate_stride = gate_stride;
    g.unit_size = unit_size;
    g.k_units = k_units;
    g.lambda = lambda;
    g.idx = idx;
    return status_of(launch_attend(*shape, L, (const uint16_t*)q, (const uint16_t*)K, (const uint16_t*)V, idx, ktok,
                                   seq_len, resolve_scale(sm_scale), out, ws, s, nullptr, &g));
  }
  float* bias = reinterpret_cast<float*>(ws + L.off_bias);
  hipError_t e = launch_gate_select(*shape, gate_scores, gate_stride, seq_len, unit_size, k_units, lambda, idx,
                                    bias, s);
  if (e == hipSuccess)
    e = launch_attend(*shape, L, (const uint16_t*)q, (const uint16_t*)K, (const uint16_t*)V, idx, ktok, seq_len,
                      resolve_scale(sm_scale), out, ws, s, bias);
  return status_of(e);
}

int sjsa_block_keys(const sjsa_shape* shape, int32_t block_size, const void* K, const int32_t* seq_len, void* Kc,
                    void* Kq, void* Ks, void* stream) {
  int st = check_blocks(shape, block_size);
  if (st) return st;
  if (!K || !seq_len || (!Kc && !(Kq && Ks)) || (!Kq != !Ks)) return SJSA_ERR_NULL;
  if (!aligned(K, 16) || !aligned(seq_len, 4) || !aligned(Kc, 16) || !aligned(Kq, 4) || !aligned(Ks, 2))
    return SJSA_ERR_ALIGN;
  return status_of(launch_block_keys(*shape, block_size, (const uint16_t*)K, seq_len, nullptr, 0, (uint16_t*)Kc,
                                     (unsigned char*)Kq, (uint16_t*)Ks, (hipStream_t)stream));
}

int sjsa_block_append(const sjsa_shape* shape, int32_t block_size, const void* k_new, const void* v_new,
                      int32_t n_new, const int32_t* pos, void* K, void* V, void* Kc, void* Kq, void* Ks,
                      void* stream) {
  int st = check_blocks(shape, block_size);
  if (st) return st;
  if (!k_new || !v_new || !pos || !K || !V || (!Kc && !(Kq && Ks)) || (!Kq != !Ks)) return SJSA_ERR_NULL;
  if (n_new < 1) return SJSA_ERR_DIMS;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(pos, 4) ||
      !aligned(Kc, 16) || !aligned(Kq, 4) || !aligned(Ks, 2))
    return SJSA_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = launch_kv_rows(*shape, (const uint16_t*)k_new, (const uint16_t*)v_new, n_new, pos, (uint16_t*)K,
                                (uint16_t*)V, s);
  if (e == hipSuccess)
    e = launch_block_keys(*shape, block_size, (const uint16_t*)K, nullptr, pos, n_new, (uint16_t*)Kc,
                          (unsigned char*)Kq, (uint16_t*)Ks, s);
  return status_of(e);
}

size_t sjsa_block_workspace_size(const sjsa_shape* shape, int32_t block_size, int32_t k_blocks) {
  if (check_blocks(shape, block_size) != SJSA_OK) return 0;
  if (k_blocks < 1 || k_blocks > SJSA_MAX_SELECT_UNITS || (int64_t)k_blocks * block_size > SJSA_MAX_K) return 0;
  return make_block_layout(*shape, block_size, k_blocks).total;
}

int sjsa_block_decode_step(const sjsa_shape* shape, int32_t block_size, const void* q, const void* K, const void* V,
                           const void* Kc, const void* Kq, const void* Ks, const int32_t* seq_len, int32_t k_blocks,
                           int32_t n_init, int32_t n_local, float sm_scale, void* out, int32_t* idx,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_blocks(shape, block_size);
  if (st) return st;
  if (k_blocks < 1 || k_blocks > SJSA_MAX_SELECT_UNITS) return SJSA_ERR_DIMS;
  if ((int64_t)k_blocks * block_size > SJSA_MAX_K) return SJSA_ERR_K;
  if (n_init < 0 || n_local < 0 || (int64_t)n_init + n_local > k_blocks) return SJSA_ERR_DIMS;
  if (!q || !K || !V || !seq_len || !out || !idx || !workspace || (!Kc && !(Kq && Ks))) return SJSA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(Kc, 16) || !aligned(Kq, 4) ||
      !aligned(Ks, 2) || !aligned(seq_len, 4) || !aligned(idx, 4) || !aligned(out, 16) ||
      !aligned(workspace, WS_ALIGN))
    return SJSA_ERR_ALIGN;
  if (!isfinite(sm_scale)) return SJSA_ERR_DIMS;
  const BlockLayout L = make_block_layout(*shape, block_size, k_blocks);
  if (workspace_bytes < L.total) return SJSA_ERR_WORKSPACE;
  unsigned char* ws = (unsigned char*)workspace;
  hipStream_t s = (hipStream_t)stream;
  const float scale = resolve_scale(sm_scale);
  const int ktok = k_blocks * block_size;
  hipError_t e = launch_block_select(*shape, L, block_size, (const uint16_t*)q, (const uint16_t*)Kc,
                                     Kc ? nullptr : (const unsigned char*)Kq, Kc ? nullptr : (const uint16_t*)Ks,
                                     seq_len, k_blocks, n_init, n_local, scale, idx, ws, s);
  if (e == hipSuccess)
    e = launch_attend(*shape, L.att, (const uint16_t*)q, (const uint16_t*)K, (const uint16_t*)V, idx, ktok, seq_len,
                      scale, out, ws, s);
  return status_of(e);
}

}  // extern "C"
