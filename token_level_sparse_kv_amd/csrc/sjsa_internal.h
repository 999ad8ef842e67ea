// Internal host-side declarations of libsjsa: workspace layout and kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "sjsa.h"

namespace sjsa {

constexpr int HEAD_DIM = 128;
constexpr int HIST_BINS = 4096;      // first radix digit: top 12 bits of the score key
constexpr int HIST_SHIFT = 20;
constexpr int QHAT_STRIDE = 64;      // floats reserved per unit for q_hat (r <= 64)
constexpr int SEG_ROWS = 128;        // rows per scan segment (one wave iteration)
// Rows per scan workgroup (one candidate region each): about 128 KB of projected rows
// per tile, between 1024 and 4096 rows. Longer tiles leave a longer end of the launch
// in which few workgroups still run; shorter ones add per-workgroup cost.
constexpr int TILE_BYTES = 128 * 1024;
constexpr int TILE_ROWS_MIN = 1024;
constexpr int TILE_ROWS_MAX = 4096;
__host__ __device__ constexpr int tile_rows(int row_bytes) {
  return row_bytes <= 0 || TILE_BYTES / row_bytes > TILE_ROWS_MAX ? TILE_ROWS_MAX
         : (TILE_BYTES / row_bytes < TILE_ROWS_MIN ? TILE_ROWS_MIN : TILE_BYTES / row_bytes);
}
constexpr uint32_t TILE_OVERFLOW = 0xffffffffu;   // tile count: the tile's candidates are not usable
// Words a unit's prep hands to the scan workgroups of the same launch when the two
// run as one kernel: 64-bit words (tag << 32 | value), the tag naming the launch.
constexpr int SYNC_WORDS = 128;      // per unit
constexpr int SYNC_THR = 64;         // word: threshold key ([0, r) hold q_hat)
constexpr int SYNC_ROW = 96;         // words: the appended token's projected row (r*KB/4 <= 32)
// A candidate entry holds its key relative to the unit's threshold key,
// rel = (key - threshold) >> shift clamped to CAND_KEY_BITS bits, above the row's
// offset inside its scan tile (at most 2^CAND_ROW_BITS rows). The prep picks the
// unit's shift so that four times the sampled keys' range above the threshold fits
// the CAND_KEY_BITS bits (shift <= CAND_ROW_BITS, since keys have 32 bits): the
// selection ranks by rel and recomputes the exact score only of the entries that
// share the boundary's rel, which at this resolution is rarely more than one.
constexpr int CAND_ROW_BITS = 12;
constexpr int CAND_KEY_BITS = 32 - CAND_ROW_BITS;
constexpr uint32_t CAND_ROW_MASK = (1u << CAND_ROW_BITS) - 1u;
constexpr uint32_t CAND_REL_MAX = (1u << CAND_KEY_BITS) - 1u;
static_assert(TILE_ROWS_MAX == 1 << CAND_ROW_BITS, "a tile offset fits the entry's low bits");
__host__ __device__ constexpr uint32_t cand_rel(uint32_t key, uint32_t tkey, uint32_t shift) {
  return key <= tkey ? 0u : ((key - tkey) >> shift < CAND_REL_MAX ? (key - tkey) >> shift : CAND_REL_MAX);
}
__host__ __device__ constexpr uint32_t cand_entry(uint32_t rel, int row) {
  return (rel << CAND_ROW_BITS) | ((uint32_t)row & CAND_ROW_MASK);
}
// tlow[2u + 1]: bit 0 = every position is taken (k >= n); bits 8.. = the unit's shift
constexpr int TLOW_SHIFT_POS = 8;
constexpr int CAND_HEADROOM = 2;      // log2 of the relative keys' span over the sampled range
constexpr int PART_STRIDE = HEAD_DIM + 2;   // acc[d], running max, running sum
// Most workgroups of the selection launch per unit (fewer when the units alone fill the
// GPU): the first selects from the candidates; when the unit takes the exact path (scores
// recomputed from the projected cache), all of them recompute one part of its rows and
// the last to finish selects.
constexpr int EXACT_WGS = 4;

struct Layout {
  int64_t units = 0;          // B * H_kv
  int64_t score_stride = 0;   // floats per unit row of the score buffer
  int nsplit = 1;             // attention splits per unit
  int chunk = 0;              // selected indices per split
  // The workspace's offsets do not depend on the projected cache's format (stage calls
  // that do not name it share one workspace): count words and candidate regions are
  // sized for the format with the most tiles.
  int64_t tile_rows = 0;      // rows per scan tile of this shape's format
  int64_t ntile = 0;          // scan tiles per unit of this shape's format (capacity / tile_rows, up)
  int64_t ntile_cap = 0;      // count words per unit (tiles of the bf16 cache, the most of any format)
  int64_t cand_stride = 0;    // 4-byte candidate entries per unit (capacity rounded up to TILE_ROWS_MAX)
  size_t off_qhat = 0, off_tlow = 0, off_counts = 0, off_cand = 0, off_scores = 0, off_partials = 0;
  size_t off_sync = 0;        // SYNC_WORDS 64-bit words per unit
  size_t off_epoch = 0;       // one u32 per unit: steps completed on this workspace
  size_t off_arrive = 0;      // one u32 per unit: workgroups of its exact path done (reset by the prep)
  size_t off_parthist = 0;    // [units, EXACT_WGS, HIST_BINS] u32: the exact path's partial histograms
  size_t off_bias = 0;        // gated step: per-position logit terms
  size_t scores_end = 0, total = 0;
};

Layout make_layout(const sjsa_shape& s, int k);
// Workspace of the gated step: logit terms [units, ktok] fp32, then attention partials.
Layout make_gated_layout(const sjsa_shape& s, int ktok);

// Kernel launchers (device pointers; host-validated arguments).
hipError_t launch_append(const sjsa_shape& s, const uint16_t* k_new, const uint16_t* v_new, int n_new,
                         const float* M, const int32_t* pos, uint16_t* K, uint16_t* V, void* Kproj,
                         hipStream_t st);
// The new token of a decode step, appended by the prep kernel (one token per sequence).
struct PrepAppend {
  const uint16_t* k_new = nullptr;   // [B, H_kv, d]
  const uint16_t* v_new = nullptr;
  const int32_t* pos = nullptr;      // [B]
  uint16_t* K = nullptr;
  uint16_t* V = nullptr;
  unsigned char* Kproj = nullptr;     // bf16 or fp8 elements (SJSA_FLAG_KPROJ_FP8)
};
// ap != nullptr: the prep kernel also appends the new token (see PrepAppend).
hipError_t launch_prep(const sjsa_shape& s, const Layout& L, const uint16_t* q, const float* M,
                       const void* kproj, const int32_t* seq_len, int k, unsigned char* ws, hipStream_t st,
                       const PrepAppend* ap = nullptr);
hipError_t launch_score(const sjsa_shape& s, const Layout& L, const void* kproj, const int32_t* seq_len,
                        unsigned char* ws, hipStream_t st);
// prep and scan as one launch (the scan workgroups take q_hat and the threshold from
// the prep workgroups as they are published); falls back to the two launches when the
// one-dimensional grid would not fit or dense scores are requested.
hipError_t launch_prep_scan(const sjsa_shape& s, const Layout& L, const uint16_t* q, const float* M,
                            const void* kproj, const int32_t* seq_len, int k, unsigned char* ws, hipStream_t st,
                            const PrepAppend* ap = nullptr);
// scores == nullptr: select from the scan's candidates in the workspace (recomputing a
// unit's scores from kproj/qhat when needed); else exact top-k of the given dense scores.
hipError_t launch_select(const sjsa_shape& s, const Layout& L, const float* scores, int64_t stride,
                         const void* kproj, const int32_t* seq_len, int k, int32_t* idx, unsigned char* ws,
                         hipStream_t st);
// The gated-logit selection, when the attention launch makes it itself (gsel below).
struct GatedSelect {
  const float* gate_scores = nullptr;   // [B * H_kv, gate_stride] unit scores
  int64_t gate_stride = 0;
  int unit_size = 1;
  int k_units = 1;
  float lambda = 0.f;
  int32_t* idx = nullptr;               // [B * H_kv, k_units * unit_size] output
};
// Largest unit count and budget the attention launch selects for itself.
constexpr int GATE_FUSED_UNITS_MAX = 2048;
constexpr int GATE_FUSED_KEPT_MAX = 512;
// bias != nullptr: one exp2-domain logit term per index entry, laid out like idx.
// gsel != nullptr: every attention workgroup makes its unit's gated selection first
// (k = k_units * unit_size; idx and bias are not read, the index list is written).
hipError_t launch_attend(const sjsa_shape& s, const Layout& L, const uint16_t* q, const uint16_t* K,
                         const uint16_t* V, const int32_t* idx, int k, const int32_t* seq_len,
                         float sm_scale, void* out, unsigned char* ws, hipStream_t st,
                         const float* bias = nullptr, const GatedSelect* gsel = nullptr);
// Block-sparse step: workspace of the block logits and the tiles' softmax partials,
// then the attention partials (att).
struct BlockLayout {
  Layout att;                 // attention split and partials for k_blocks * block_size entries
  int64_t nblk_cap = 0;       // block keys per (b, h): capacity / block_size
  int64_t zstride = 0;        // floats per (unit, head) row of block logits
  int ntile = 0;              // scoring tiles per unit
  size_t off_z = 0, off_ms = 0, total = 0;
};
BlockLayout make_block_layout(const sjsa_shape& s, int block_size, int k_blocks);
hipError_t launch_kv_rows(const sjsa_shape& s, const uint16_t* k_new, const uint16_t* v_new, int n_new,
                          const int32_t* pos, uint16_t* K, uint16_t* V, hipStream_t st);
// pos == nullptr: keys of every complete block of each sequence; else of the blocks
// completed by the rows [pos_b, pos_b + n_new) just written. Kc / Kq+Ks may be null.
hipError_t launch_block_keys(const sjsa_shape& s, int bs, const uint16_t* K, const int32_t* seq_len,
                             const int32_t* pos, int n_new, uint16_t* Kc, unsigned char* Kq, uint16_t* Ks,
                             hipStream_t st);
// Kc != nullptr: bf16 block keys; else INT4 codes Kq and fp16 scales Ks.
hipError_t launch_block_select(const sjsa_shape& s, const BlockLayout& L, int bs, const uint16_t* q,
                               const uint16_t* Kc, const unsigned char* Kq, const uint16_t* Ks,
                               const int32_t* seq_len, int k_blocks, int n_init, int n_local, float sm_scale,
                               int32_t* idx, unsigned char* ws, hipStream_t st);
// Gated-logit unit selection: idx and bias [B * H_kv, k_units * unit_size].
hipError_t launch_gate_select(const sjsa_shape& s, const float* gate_scores, int64_t gate_stride,
                              const int32_t* seq_len, int unit_size, int k_units, float lambda, int32_t* idx,
                              float* bias, hipStream_t st);

}  // namespace sjsa
