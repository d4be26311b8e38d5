// spb_launch.h -- host-side launchers of the gfx950 kernels (internal to libspb).
// Implemented in spb_attention.hip and spb_score.hip; called by spb_host.cpp
// after every argument has been validated.  Each returns 0 or a hipError_t
// value and never allocates.
#pragma once
#include <stddef.h>
#include <stdint.h>

#include "spb_head_layout.h"

namespace spb {

struct AttnLaunch {
  const void *q, *k, *v;
  void *o;
  int in_dtype, out_dtype;   // spb_dtype values
  int hq, hkv, head_dim;
  float scale;               // softmax scale (already resolved)
  float s_q, s_k, s_v;       // fp8 dequantisation scales (1 otherwise)
  int n_tokens, n_tiles;
  const void *rows, *tiles, *branches;  // device pointers into the metadata blob
  const void *items[3], *bchunks;       // work items at 32, 64, 128 rows; their branch chunks
  int n_items[3];
  void *v_wide;              // e4m3 inputs: bf16 copy of V (n_tokens x hkv x d), or NULL
};

struct ScoreLaunch {
  const void *hidden;
  int h_dtype, hidden_dim;
  const void *lm_head;
  int vocab;
  int n_scored, n_targets, n_branches, n_options;
  const void *scored, *tgt_off, *tgt_tok, *branches, *opt_step_off, *step_slot, *step_row;
  float *part;   // workspace: [n_scored][n_slices][2] (max, sum of exp) per vocabulary slice
  float *tz;     // workspace: [n_targets] captured logits
  float *lse;    // workspace: [n_scored]
  void *hg;      // workspace: gathered hidden states, bf16 [m_pad][hidden_dim]
  float *lp, *p, *residual;
  void *ev_begin, *ev_end;  // optional hipEvent_t around the GEMM kernel
  int kind;                 // lm-head output kind (SPB_HEAD_*)
};


// Several passes' scored rows through one lm-head stream: pass i's rows
// occupy combined rows m_off[i] .. +n_scored and its targets combined
// targets t_off[i] .. (the per-pass fields of pass[i] describe its
// metadata and outputs; its workspace fields are unused).
constexpr int kMaxBatchPasses = 64;
struct ScoreBatchLaunch {
  int n;
  ScoreLaunch pass[kMaxBatchPasses];
  int m_off[kMaxBatchPasses], t_off[kMaxBatchPasses];
  int m_tot, t_tot;
  int h_dtype, hidden_dim;
  const void *lm_head;
  int vocab;
  float *part, *tz, *lse;  // workspace, combined rows / targets
  void *hg;
  int32_t *ctgt_off, *ctgt_tok;  // workspace: combined target CSR
  int kind;                      // lm-head output kind (SPB_HEAD_*)
  void *ev_begin, *ev_end;
};

// Decoder-stack kernels (spb_layer.hip).
struct NormLaunch {
  const float *x;          // [rows][dim] f32 residual stream
  const uint16_t *gain;    // [dim] bf16
  uint16_t *out;           // [rows][dim] bf16
  long long rows;
  int dim;
  float eps;
};

// Y^T = W . X^T over tiles of 256 W rows x 32*kLinearMB X rows, then one of
// the epilogues (SPB_LINEAR_* values).
constexpr int kLinearMB = 7;
struct LinearLaunch {
  const uint16_t *x;       // [m][k] bf16
  const uint16_t *w;       // [n][k] bf16
  int m, n, k;
  int mode;
  uint16_t *y;             // BF16: [m][n]; SILU_GATE: [m][n/2]
  float *yf;               // F32: [m][n]
  float *resid;            // RESIDUAL: [m][n] f32, added to in place
  uint16_t *q, *kk, *v;    // QKV_ROPE: [m][hq*d], [m][hkv*d], [m][hkv*d]
  int hq, hkv, head_dim;
  const int32_t *pos;      // QKV_ROPE: [m] positions
  const float *rope;       // QKV_ROPE: [n_pos][d/2] (cos, sin) pairs
  int n_pos;
  void *ev_begin, *ev_end; // optional hipEvent_t around the kernel
  int fp8;                 // x and w are e4m3 bytes; the products are scaled by `scale`
  float scale;             // s_x * s_w
};

struct QuantLaunch {       // dst = e4m3(src * inv_scale)
  const float *src_f32;    // one of the two
  const uint16_t *src_bf16;
  uint8_t *dst;
  long long n;
  float inv_scale;
};
int launch_quantize_e4m3(const QuantLaunch &a, void *stream);

int launch_rmsnorm(const NormLaunch &a, void *stream);

// Slot decoding kernels (spb_decode.hip).
constexpr int kMaxTopK = 16;       // candidates per row
constexpr int kMaxBeams = 16;      // beams per slot
constexpr int kMaxSlotRanges = 16; // key ranges of a slot's prefix

struct TopkLaunch {
  const float *z;            // [rows][vocab] logits
  long long rows;
  int vocab, k;
  const uint32_t *masks;     // [n_masks][ceil(vocab/32)] allowed-token bits, or NULL
  const int32_t *mask_of_row;// [rows] mask index, -1 all tokens (NULL: all rows all tokens)
  const int32_t *stop_of_row;// [rows] a token always allowed (NULL: none)
  int32_t *ids;              // [rows][k]
  float *lp;                 // [rows][k] z - LSE
  float *lse;                // [rows]
  void *workspace;           // topk_workspace_bytes(rows, vocab)
};
// The top-k workspace: one partial per (row, vocabulary span of kTopkSpan
// entries), each a running (max, sum of exp) and its best kMaxTopK candidates.
constexpr int kTopkSpan = 8192;  // vocabulary entries per work group of the first kernel
struct Cand {
  float v;
  int id;
};
struct TopkPart {  // one work group's partial of one row
  float m, s;
  Cand best[kMaxTopK];
};
inline size_t topk_workspace_bytes(long long rows, int vocab) {
  const int n_parts = (vocab + kTopkSpan - 1) / kTopkSpan;
  return (size_t)rows * n_parts * sizeof(TopkPart);
}

struct DecodeAttnLaunch {
  const uint16_t *q;         // [R][hq][d] bf16
  const uint16_t *kp, *vp;   // pass cache of the layer: [n_pass_rows][hkv][d]
  const uint16_t *kd, *vd;   // decode cache of the layer: [t_cap * R][hkv][d]
  uint16_t *o;               // [R][hq][d]
  int R, beams, hq, hkv, head_dim;
  const int32_t *ranges;     // [n_slots][kMaxSlotRanges][2] (first pass row, count)
  const int32_t *n_ranges;   // [n_slots]
  const int32_t *path;       // [R][t_cap] decode-cache rows of the ancestors
  int t_cap, n_path;         // ancestors per row this step; own row = n_path * R + r
  int n_pass_rows, n_dec_rows;  // bounds the kernel clamps row indices to
  float scale;
};

struct BeamLaunch {
  int n_slots, beams, k, t_cap, step, stop_any;
  const int32_t *stop;       // [n_slots]
  const int32_t *ids;        // [rows][k] candidates (rows: n_slots at step 0, else n_slots * beams)
  const float *lp;
  const int32_t *tok_in, *len_in, *fin_in, *path_in, *nb_in;   // state before the step
  const float *score_in;
  int32_t *tok_out, *len_out, *fin_out, *path_out, *nb_out;    // state after
  float *score_out;
  int32_t *feed;             // [n_slots * beams] token each beam feeds next
};

struct GatherLaunch {
  const uint16_t *src;       // [*][dim] bf16
  const int32_t *idx;        // [rows], clamped into [0, n_src)
  long long rows;
  int n_src;
  int dim;
  float *dst_f32;            // one of the two
  uint16_t *dst_bf16;
  int32_t *pos;              // optional: pos[r] = pos_base[r / per] + pos_add
  const int32_t *pos_base;
  int per, pos_add;
};

int launch_topk_lse(const TopkLaunch &a, void *stream);
int launch_decode_attention(const DecodeAttnLaunch &a, void *stream);
int launch_beam_step(const BeamLaunch &a, void *stream);
int launch_gather_rows(const GatherLaunch &a, void *stream);
int launch_linear(const LinearLaunch &a, void *stream);

int launch_attention(const AttnLaunch &a, void *stream);
int launch_score(const ScoreLaunch &a, void *stream);
// The allocation-free head's workspace: a device array of this many bytes per
// GPU; score_scratch gives the current device's address of it (taken once per
// device), or returns a hipError_t value.
constexpr size_t kScoreScratchBytes = size_t(64) << 20;
int score_scratch(void **out);
// The MFMA calibration loop: work_groups x 256 threads, each wave 16 x iters
// MFMA 32x32x16 bf16; writes work_groups * 256 floats to out.
int launch_mfma_calibration(float *out, int work_groups, int iters, int random, void *stream);
int launch_score_batch(const ScoreBatchLaunch &a, void *stream);
const char *hip_error_string(int err);

}  // namespace spb
