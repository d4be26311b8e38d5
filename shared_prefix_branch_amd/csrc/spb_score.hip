// spb_score.hip -- the scored-row lm head for gfx950 (CDNA4).
//
// Only the rows whose next-token distribution is needed are fed to the head:
// each template's last row (it predicts the options' first tokens) and each
// option-trie node.  For each such row the head needs the vocab-wide
// log-softmax at a handful of tokens: an option's log-probability, then p
// renormalised over the options and the residual mass outside them [article
// "Bulk classification and decision inference on one GPU", the response
// example and the paragraph after it].  Logits are f32, the pages' default
// lm-head precision [man page "spinf-serve", PARAMETERS: --lm-head f32out].
//
// Kernel 0 (gather_hidden_kernel): packs the scored rows' hidden states as
//   bf16 rows, zero-padded to the GEMM's row tiling.
// Kernel 1 (head_lse_kernel): Z^T[v, m] = W[v, :] . h[m, :] on MFMA 32x32x16
//   bf16 with f32 accumulation, one work group per (256-row vocabulary slice,
//   32..256 scored rows), each wave a 64-row vocabulary strip against all the
//   group's rows; W and h tiles of 64 hidden elements are copied global ->
//   LDS asynchronously into XOR-swizzled rings.  Logits never leave
//   registers: the epilogue writes, per (row, slice), the slice max and sum
//   of exp(z - max), and stores the logits of the option tokens the row
//   predicts.
// Kernel 2 (finalize_kernel): one wave per branch merges a row's slices in
//   slice order into LSE, sums each option's chain of log-probabilities in
//   token order, and renormalises.
//
// Batch invariance: z[v, m] depends only on W[v] and h[m] (fixed K order), the
// slice width is a constant, and every merge runs in a fixed order, so a row's
// results do not depend on how many rows share the pass.
#define SPB_HD __host__ __device__
#include "spb_meta.h"
#include "spb_launch.h"
#include "spb_dev.h"
#include "spb_gemm.h"
#include "../../include/spb.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

namespace spb {
namespace {

using gemm::bf16x8_t;
using gemm::f32x16;
using gemm::u32x4;
using gemm::kKT;
using gemm::kThreads;
using gemm::swz;

constexpr float kNegInf = -__builtin_inff();
static_assert(gemm::kWRows == kVocabTile, "one lm-head slice per GEMM tile");

__device__ inline uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}


struct GatherParams {
  const void *hidden;
  const int32_t *scored;
  uint16_t *hg;
  int H, M;        // this call's scored rows
  int planes;      // bf16 planes per gathered row: 1, or 3 (hi, mid, lo) for the fp32 head
  int row0;        // their first row in hg
  int zero_end;    // rows row0 + M .. zero_end are zeroed (padding)
  // batched calls: copy this pass's target CSR into the combined one
  const int32_t *tgt_off, *tgt_tok;
  int32_t *ctgt_off, *ctgt_tok;
  int t_base, t_end;  // the pass's first target in the combined CSR; total targets (last pass only: -1 otherwise)
};

__device__ inline float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// x = hi + mid + lo exactly for an f32 x: each term is the bf16 (nearest
// even) of what the previous ones left; the differences are exact in f32.
__device__ inline void split3(float x, uint32_t &hi, uint32_t &mid, uint32_t &lo) {
  hi = f2bf(x);
  const float r1 = x - bf2f(hi);
  mid = f2bf(r1);
  lo = f2bf(r1 - bf2f(mid));
}

// hg[row0 + m] = bf16(hidden[scored[m]]) for m < M, zero rows up to
// zero_end; with three planes, row m holds hi | mid | lo of the f32 row (a
// bf16 row: itself | 0 | 0).  With a combined CSR, also its rows' target
// ranges and tokens.
template <int HIN>
__global__ __launch_bounds__(256) void gather_hidden_kernel(GatherParams g) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;  // one 8-element unit
  const int per_row = g.H / 8;
  const int n_rows = g.zero_end - g.row0;
  if (i >= (long long)n_rows * per_row) return;
  const int m = (int)(i / per_row), k = (int)(i % per_row) * 8;
  uint4 v = {0u, 0u, 0u, 0u}, v2 = {0u, 0u, 0u, 0u}, v3 = {0u, 0u, 0u, 0u};
  if (m < g.M) {
    const long long row = g.scored[m];
    if constexpr (HIN == SPB_BF16) {
      v = *(const uint4 *)((const uint16_t *)g.hidden + row * g.H + k);
    } else {
      const float4 *s = (const float4 *)((const float *)g.hidden + row * g.H + k);
      const float4 a = s[0], b = s[1];
      const float x[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
      uint32_t h[8], md[8], lw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (g.planes == 3) {
          split3(x[j], h[j], md[j], lw[j]);
        } else {
          h[j] = f2bf(x[j]);
          md[j] = lw[j] = 0u;
        }
      }
      v = uint4{h[0] | (h[1] << 16), h[2] | (h[3] << 16), h[4] | (h[5] << 16), h[6] | (h[7] << 16)};
      v2 = uint4{md[0] | (md[1] << 16), md[2] | (md[3] << 16), md[4] | (md[5] << 16), md[6] | (md[7] << 16)};
      v3 = uint4{lw[0] | (lw[1] << 16), lw[2] | (lw[3] << 16), lw[4] | (lw[5] << 16), lw[6] | (lw[7] << 16)};
    }
    if (g.ctgt_off && k == 0) {
      const int t0 = g.tgt_off[m], t1 = g.tgt_off[m + 1];
      g.ctgt_off[g.row0 + m] = g.t_base + t0;
      for (int t = t0; t < t1; ++t) g.ctgt_tok[g.t_base + t] = g.tgt_tok[t];
      if (m == g.M - 1 && g.t_end >= 0) g.ctgt_off[g.row0 + g.M] = g.t_end;
    }
  }
  uint16_t *dst = g.hg + (long long)(g.row0 + m) * g.planes * g.H + k;
  *(uint4 *)dst = v;
  if (g.planes == 3) {
    *(uint4 *)(dst + g.H) = v2;
    *(uint4 *)(dst + 2 * g.H) = v3;
  }
}

struct HeadParams {
  const uint16_t *hg;  // gathered hidden states [M_pad][Hrow] bf16
  const uint16_t *W;
  int H, V, M;
  int Hrow;       // hg row length: H, or 3H (planes hi | mid | lo) for the fp32 head
  int SW;         // stages per sweep of W (H / 64); Hrow / 64 stages in all
  int round_bf16; // bf16 head: each logit rounded to bf16 before the epilogue uses it
  int n_slices, n_mchunks;
  const int32_t *tgt_off, *tgt_tok;
  float *part, *tz;
};

template <int MB>
using HeadTile = gemm::Tile<MB>;

// Work group: 256 vocabulary rows x TM = 32*MB scored rows, on the shared K
// loop (spb_gemm.h); the h tile is small and shared by every work group, so
// L2-resident.
template <int MB>
__global__ __launch_bounds__(kThreads, 1) void head_lse_kernel(HeadParams p) {
  using T = HeadTile<MB>;
  constexpr int TM = T::TM;
  __shared__ __attribute__((aligned(1024))) char lds[T::LDS];
  static_assert(4 * TM * 2 * 4 <= T::LDS, "epilogue buffer must fit in the ring");

  // XCD-aware order: work groups are dealt round-robin to the 8 XCDs, so the
  // M chunks of one vocabulary slice get consecutive slots of one XCD and
  // stream the same W rows through its L2 together.
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int slice = (slot / p.n_mchunks) * 8 + xcd;
  const int mchunk = slot % p.n_mchunks;
  if (slice >= p.n_slices) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform within the wave
  const int qi = lane & 31, half = lane >> 5;
  const int v0 = slice * kVocabTile;
  const int m0 = mchunk * TM;

  uint32_t woff[8], hoff[MB];
  gemm::tile_offsets<MB>(
      woff, hoff, [&](int r) { return v0 + r < p.V ? v0 + r : p.V - 1; }, [&](int r) { return m0 + r; }, p.H,
      p.Hrow, wave, lane);
  f32x16 acc[2][MB];
  gemm::k_loop<MB>(acc, lds, p.W, p.hg, woff, hoff, p.Hrow / kKT, p.SW, wave, qi, half);

  // epilogue; the ring is free.  LDS: the four waves' (max, sum) per row,
  // then the group's target CSR (offsets relative to its first target) and,
  // when they fit, its target tokens, staged in one round trip so the
  // capture below waits on LDS, not on a global load per target.
  float (*red)[TM][2] = (float (*)[TM][2])lds;  // [4][TM][2]
  int *s_off = (int *)(lds + 4 * TM * 2 * 4);   // [TM + 1]
  int *s_tok = s_off + TM + 1;
  constexpr int kTokCap = (T::LDS - 4 * TM * 2 * 4) / 4 - (TM + 1);
  static_assert(kTokCap >= 4 * TM, "room for several targets per row");
  const int tb = p.tgt_off[m0 < p.M ? m0 : p.M];
  const int te = p.tgt_off[m0 + TM < p.M ? m0 + TM : p.M];
  const bool staged = te - tb <= kTokCap;
  for (int i = tid; i <= TM; i += kThreads) s_off[i] = p.tgt_off[m0 + i < p.M ? m0 + i : p.M] - tb;
  if (staged)
    for (int i = tid; i < te - tb; i += kThreads) s_tok[i] = p.tgt_tok[tb + i];
  __syncthreads();

  // Lane holds column m = m0 + mb*32 + qi; register r of block vb holds
  // vocabulary row v0 + wave*64 + vb*32 + (r/4)*8 + half*4 + r%4.
  const int vw0 = v0 + wave * 64;
  const int nvalid = p.V - vw0;      // rows past the vocabulary (last slice only) are excluded
  const bool full = nvalid >= 64;    // uniform: every strip but the vocabulary's tail
  constexpr float kL2e = 1.44269504088896340736f;
  // one 32-row block at a time, so only its two accumulators leave the
  // accumulation registers at once
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    f32x16 z[2] = {acc[0][mb], acc[1][mb]};
    asm volatile("" : "+v"(z[0]), "+v"(z[1]));  // the copy out of acc happens here, not at the loop exit
    if (p.round_bf16) {
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) z[vb][r] = bf2f(f2bf(z[vb][r]));
    }
    float mx = kNegInf;
    if (full) {
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, z[vb][r]);
    } else {
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int vr = vb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
          mx = fmaxf(mx, vr < nvalid ? z[vb][r] : kNegInf);
        }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float se = 0.f;
    if (mx != kNegInf) {
      // exp(z - mx) as 2^(z log2e - mx log2e): one fma and one v_exp_f32
      const float nm = -mx * kL2e;
      if (full) {
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) se += __builtin_amdgcn_exp2f(__builtin_fmaf(z[vb][r], kL2e, nm));
      } else {
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int vr = vb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
            se += vr < nvalid ? __builtin_amdgcn_exp2f(__builtin_fmaf(z[vb][r], kL2e, nm)) : 0.f;
          }
      }
    }
    se = se + __shfl_xor(se, 32);
    const int ml = mb * 32 + qi;
    if (half == 0) {
      red[wave][ml][0] = mx;
      red[wave][ml][1] = se;
    }
    // capture the logits of the tokens this row predicts
    const int m = m0 + ml;
    if (m < p.M) {
      const int t0 = s_off[ml], t1 = s_off[ml + 1];
      for (int t = t0; t < t1; ++t) {
        const int rel = (staged ? s_tok[t] : p.tgt_tok[tb + t]) - vw0;
        if (rel < 0 || rel >= 64) continue;
        const int rr = rel & 31;
        if (((rr >> 2) & 1) != half) continue;
        const int vbt = rel >> 5, rt = (rr >> 3) * 4 + (rr & 3);
        float val = 0.f;
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) val = (vb == vbt && r == rt) ? z[vb][r] : val;
        p.tz[tb + t] = val;
      }
    }
  }
  __syncthreads();
  // merge the four waves' (max, sum) in wave order
  for (int ml = tid; ml < TM; ml += kThreads) {
    const int m = m0 + ml;
    if (m < p.M) {
      float M = red[0][ml][0], S = red[0][ml][1];
#pragma unroll
      for (int w = 1; w < 4; ++w) {
        const float a = red[w][ml][0];
        const float Mn = fmaxf(M, a);
        S = (M == kNegInf ? 0.f : S * __expf(M - Mn)) + (a == kNegInf ? 0.f : red[w][ml][1] * __expf(a - Mn));
        M = Mn;
      }
      float *dst = p.part + ((size_t)m * p.n_slices + slice) * 2;
      dst[0] = M;
      dst[1] = S;
    }
  }
}

struct FinParams {
  const SpbBranch *branches;
  const int32_t *opt_step_off, *step_slot, *step_row;
  const float *tz, *lse;
  float *lp, *p, *residual;
};

__device__ inline void merge(float &M, float &S, float m2, float s2) {
  float Mn = fmaxf(M, m2);
  float a = M == kNegInf ? 0.f : S * __expf(M - Mn);
  float b = m2 == kNegInf ? 0.f : s2 * __expf(m2 - Mn);
  M = Mn;
  S = a + b;
}

struct LseParams {
  int n_slices, M;
  const float *part;  // [M][n_slices] (max, sum of exp) pairs
  float *lse;         // [M]
};

// LSE of every scored row, one wave per row: each lane merges slices lane,
// lane + 64, ... in increasing order (its loads issued eight at a time ahead
// of the merges), then a butterfly whose pairwise merges are commutative, so
// every lane agrees and the order is fixed.
__global__ __launch_bounds__(256) void lse_kernel(LseParams a) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.M) return;
  const int lane = threadIdx.x & 63;
  const float2 *pp = (const float2 *)(a.part + (size_t)row * a.n_slices * 2);
  float M = kNegInf, S = 0.f;
  for (int i0 = lane; i0 < a.n_slices; i0 += 64 * 8) {
    float2 v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int i = i0 + 64 * j;
      v[j] = i < a.n_slices ? pp[i] : make_float2(kNegInf, 0.f);  // (-inf, 0) merges as nothing
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) merge(M, S, v[j].x, v[j].y);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    float m2 = __shfl_xor(M, off), s2 = __shfl_xor(S, off);
    merge(M, S, m2, s2);
  }
  if (lane == 0) a.lse[row] = M + __logf(S);
}

// One wave per branch, after lse_kernel: option chains and renormalisation.
__global__ __launch_bounds__(64) void finalize_kernel(FinParams f) {
  const SpbBranch br = f.branches[blockIdx.x];
  const int lane = threadIdx.x;
  // option log-probabilities: chain rule in token order
  float mx = kNegInf;
  for (int o = lane; o < br.n_opt; o += 64) {
    const int opt = br.opt0 + o;
    float acc = 0.f;
    for (int st = f.opt_step_off[opt]; st < f.opt_step_off[opt + 1]; ++st)
      acc += f.tz[f.step_slot[st]] - f.lse[f.step_row[st]];
    f.lp[opt] = acc;
    mx = fmaxf(mx, acc);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  __threadfence_block();
  float se = 0.f;
  for (int o = lane; o < br.n_opt; o += 64) se += __expf(f.lp[br.opt0 + o] - mx);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) se += __shfl_xor(se, off);
  const float inv = 1.f / se;
  for (int o = lane; o < br.n_opt; o += 64) f.p[br.opt0 + o] = __expf(f.lp[br.opt0 + o] - mx) * inv;
  if (lane == 0) f.residual[blockIdx.x] = -expm1f(mx + __logf(se));
}

}  // namespace

namespace {

int launch_gather(const GatherParams &g, int h_dtype, hipStream_t s) {
  const long long units = (long long)(g.zero_end - g.row0) * (g.H / 8);
  if (units <= 0) return 0;
  const unsigned blocks = (unsigned)((units + 255) / 256);
  if (h_dtype == SPB_BF16)
    hipLaunchKernelGGL(gather_hidden_kernel<SPB_BF16>, dim3(blocks), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL(gather_hidden_kernel<SPB_F32>, dim3(blocks), dim3(256), 0, s, g);
  return (int)hipGetLastError();
}

// The GEMM + slice partials over M gathered rows, bracketed by the optional
// timing events.
int launch_head(const HeadParams &p0, int mb, void *ev_begin, void *ev_end, hipStream_t s) {
  HeadParams p = p0;
  long long groups = (long long)((p.n_slices + 7) / 8) * 8 * p.n_mchunks;
  if (groups > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  dim3 grid((unsigned)groups), block(kThreads);
  int e;
  if (ev_begin) {
    e = (int)hipEventRecord((hipEvent_t)ev_begin, s);
    if (e) return e;
  }
  switch (mb) {
    case 1: hipLaunchKernelGGL(head_lse_kernel<1>, grid, block, 0, s, p); break;
    case 2: hipLaunchKernelGGL(head_lse_kernel<2>, grid, block, 0, s, p); break;
    case 3: hipLaunchKernelGGL(head_lse_kernel<3>, grid, block, 0, s, p); break;
    case 4: hipLaunchKernelGGL(head_lse_kernel<4>, grid, block, 0, s, p); break;
    case 5: hipLaunchKernelGGL(head_lse_kernel<5>, grid, block, 0, s, p); break;
    case 6: hipLaunchKernelGGL(head_lse_kernel<6>, grid, block, 0, s, p); break;
    case 7: hipLaunchKernelGGL(head_lse_kernel<7>, grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL(head_lse_kernel<8>, grid, block, 0, s, p); break;
  }
  e = (int)hipGetLastError();
  if (e) return e;
  if (ev_end) {
    e = (int)hipEventRecord((hipEvent_t)ev_end, s);
    if (e) return e;
  }
  return 0;
}

int launch_lse(int n_slices, int M, const float *part, float *lse, hipStream_t s) {
  if (M <= 0) return 0;
  LseParams a{n_slices, M, part, lse};
  hipLaunchKernelGGL(lse_kernel, dim3((unsigned)((M + 3) / 4)), dim3(256), 0, s, a);
  return (int)hipGetLastError();
}

int launch_finalize(const FinParams &f, int n_branches, hipStream_t s) {
  if (n_branches <= 0) return 0;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)n_branches), dim3(64), 0, s, f);
  return (int)hipGetLastError();
}

}  // namespace

int launch_score(const ScoreLaunch &a, void *stream) {
  hipStream_t s = (hipStream_t)stream;
  int n_chunks = 0, mb = 0;
  head_m_layout(a.n_scored, &n_chunks, &mb);
  GatherParams g{};
  g.hidden = a.hidden;
  g.scored = (const int32_t *)a.scored;
  g.hg = (uint16_t *)a.hg;
  g.H = a.hidden_dim;
  g.M = a.n_scored;
  g.planes = head_planes(a.kind);
  g.row0 = 0;
  g.zero_end = n_chunks * 32 * mb;
  int e = launch_gather(g, a.h_dtype, s);
  if (e) return e;

  HeadParams p;
  p.hg = (const uint16_t *)a.hg;
  p.W = (const uint16_t *)a.lm_head;
  p.H = a.hidden_dim;
  p.V = a.vocab;
  p.M = a.n_scored;
  p.Hrow = a.hidden_dim * head_planes(a.kind);
  p.SW = a.hidden_dim / kKT;
  p.round_bf16 = a.kind == SPB_HEAD_BF16;
  p.n_slices = n_vocab_slices(a.vocab);
  p.n_mchunks = n_chunks;
  p.tgt_off = (const int32_t *)a.tgt_off;
  p.tgt_tok = (const int32_t *)a.tgt_tok;
  p.part = a.part;
  p.tz = a.tz;
  e = launch_head(p, mb, a.ev_begin, a.ev_end, s);
  if (e) return e;

  FinParams f;
  f.branches = (const SpbBranch *)a.branches;
  f.opt_step_off = (const int32_t *)a.opt_step_off;
  f.step_slot = (const int32_t *)a.step_slot;
  f.step_row = (const int32_t *)a.step_row;
  f.tz = a.tz;
  f.lse = a.lse;
  f.lp = a.lp;
  f.p = a.p;
  f.residual = a.residual;
  e = launch_lse(p.n_slices, a.n_scored, a.part, a.lse, s);
  if (e) return e;
  return launch_finalize(f, a.n_branches, s);
}

int launch_score_batch(const ScoreBatchLaunch &a, void *stream) {
  hipStream_t s = (hipStream_t)stream;
  int n_chunks = 0, mb = 0;
  head_m_layout(a.m_tot, &n_chunks, &mb);
  const int m_pad = n_chunks * 32 * mb;
  int e;
  for (int i = 0; i < a.n; ++i) {
    const ScoreLaunch &P = a.pass[i];
    const bool last = i == a.n - 1;
    GatherParams g{};
    g.hidden = P.hidden;
    g.scored = (const int32_t *)P.scored;
    g.hg = (uint16_t *)a.hg;
    g.H = a.hidden_dim;
    g.M = P.n_scored;
    g.planes = head_planes(a.kind);
    g.row0 = a.m_off[i];
    g.zero_end = last ? m_pad : a.m_off[i] + P.n_scored;
    g.tgt_off = (const int32_t *)P.tgt_off;
    g.tgt_tok = (const int32_t *)P.tgt_tok;
    g.ctgt_off = a.ctgt_off;
    g.ctgt_tok = a.ctgt_tok;
    g.t_base = a.t_off[i];
    g.t_end = last ? a.t_tot : -1;
    e = launch_gather(g, a.h_dtype, s);
    if (e) return e;
  }
  HeadParams p;
  p.hg = (const uint16_t *)a.hg;
  p.W = (const uint16_t *)a.lm_head;
  p.H = a.hidden_dim;
  p.V = a.vocab;
  p.M = a.m_tot;
  p.Hrow = a.hidden_dim * head_planes(a.kind);
  p.SW = a.hidden_dim / kKT;
  p.round_bf16 = a.kind == SPB_HEAD_BF16;
  p.n_slices = n_vocab_slices(a.vocab);
  p.n_mchunks = n_chunks;
  p.tgt_off = a.ctgt_off;
  p.tgt_tok = a.ctgt_tok;
  p.part = a.part;
  p.tz = a.tz;
  e = launch_head(p, mb, a.ev_begin, a.ev_end, s);
  if (e) return e;
  e = launch_lse(p.n_slices, a.m_tot, a.part, a.lse, s);  // the passes' rows lie back to back
  if (e) return e;
  for (int i = 0; i < a.n; ++i) {
    const ScoreLaunch &P = a.pass[i];
    FinParams f;
    f.branches = (const SpbBranch *)P.branches;
    f.opt_step_off = (const int32_t *)P.opt_step_off;
    f.step_slot = (const int32_t *)P.step_slot;
    f.step_row = (const int32_t *)P.step_row;
    f.tz = a.tz + a.t_off[i];
    f.lse = a.lse + a.m_off[i];
    f.lp = P.lp;
    f.p = P.p;
    f.residual = P.residual;
    e = launch_finalize(f, P.n_branches, s);
    if (e) return e;
  }
  return 0;
}

// ------------------------------------------------------ MFMA calibration
// The rate the head's MFMA (32x32x16 bf16, f32 accumulation) sustains with
// nothing else to do: each wave runs 16 independent accumulators through
// `iters` rounds of 16 MFMAs, operands rotating through 16 registers each,
// no memory traffic in the loop.  Operands are random bf16 values (random) or
// small integers whose products leave most multiplier bits idle; with random
// data the chip's power limit lowers the clock, so the two bound what the
// head can reach.  One float per thread is written so nothing is eliminated.
namespace {
__global__ __launch_bounds__(256) void mfma_calibration_kernel(float *out, int iters, int random) {
  f32x16 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x16{0.f};
  u32x4 a[16], b[16];
#pragma unroll
  for (int k = 0; k < 16; ++k)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t x = (threadIdx.x + 1u) * 2654435761u ^ (uint32_t)(i * 40503 + k * 0x9E3779B9u);
      x ^= x >> 13; x *= 0x85EBCA6Bu; x ^= x >> 16;
      uint32_t y = (threadIdx.x + 7u) * 2246822519u ^ (uint32_t)(i * 97 + k * 0x7F4A7C15u);
      y ^= y >> 15; y *= 0xC2B2AE35u; y ^= y >> 13;
      // random: bf16 pairs of either sign below 2 in magnitude; else the
      // small integers 0..7 (exact bf16, few mantissa bits set)
      a[k][i] = random ? (x & 0xBF7FBF7Fu) : (f2bf((float)(x & 7u)) | (f2bf((float)((x >> 8) & 7u)) << 16));
      b[k][i] = random ? (y & 0xBF7FBF7Fu) : (f2bf((float)(y & 7u)) | (f2bf((float)((y >> 8) & 7u)) << 16));
    }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j)
      acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(bf16x8_t *)&a[j], *(bf16x8_t *)&b[(j * 5 + 3) & 15], acc[j],
                                                        0, 0, 0);
  }
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += acc[j][r];
  out[blockIdx.x * 256 + threadIdx.x] = sum;
}
}  // namespace

int launch_mfma_calibration(float *out, int work_groups, int iters, int random, void *stream) {
  hipLaunchKernelGGL(mfma_calibration_kernel, dim3((unsigned)work_groups), dim3(256), 0, (hipStream_t)stream, out,
                     iters, random);
  return (int)hipGetLastError();
}

// ------------------------------------------------------ allocation-free head
// The workspace of spb_score_options_noalloc: one file-scope device array per
// GPU (each device that loads the library holds its own copy until the
// process ends).  Host code never passes the array's name to a kernel or a
// copy: in host code it is a host-side stand-in.  Its device address is taken
// once per device, with that device current, and kept.
namespace {
__device__ __align__(256) unsigned char scratch[kScoreScratchBytes];
constexpr int kScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch[kScratchDevices] = {};
}  // namespace

int score_scratch(void **out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kScratchDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void *ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!ptr || (uintptr_t)ptr % 256) return (int)hipErrorInvalidSymbol;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return 0;
}

}  // namespace spb
