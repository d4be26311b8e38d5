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
// Kernel 1 (head_lse_kernel): Z^T[v, m] = W[v, :] . h[m, :] on MFMA 32x32x16
//   bf16 with f32 accumulation, one work group per (256-row vocabulary slice,
//   128 scored rows).  Logits never leave registers: the epilogue writes, per
//   (row, slice), the slice max and sum of exp(z - max), and stores the logits
//   of the option tokens the row predicts.
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
#include "../../include/spb.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spb {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kNegInf = -__builtin_inff();
constexpr int kMT = 128;      // scored rows per work group
constexpr int kKT = 64;       // hidden elements per K stage
constexpr int kHP = kKT + 8;  // LDS pitch of the hidden tile (bf16)
constexpr int kThreads = 256; // 4 waves x 64 vocabulary rows

__device__ inline uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

struct HeadParams {
  const void *hidden;
  const uint16_t *W;
  int H, V, M;
  int n_slices, n_mchunks;
  const int32_t *scored, *tgt_off, *tgt_tok;
  float *part, *tz;
};

template <int HIN>
__device__ inline uint4 load_hidden8(const void *hidden, int row, int H, int k) {
  if constexpr (HIN == SPB_BF16) {
    return *(const uint4 *)((const uint16_t *)hidden + (size_t)row * H + k);
  } else {
    const float4 *s = (const float4 *)((const float *)hidden + (size_t)row * H + k);
    float4 a = s[0], b = s[1];
    uint4 u;
    u.x = f2bf(a.x) | (f2bf(a.y) << 16);
    u.y = f2bf(a.z) | (f2bf(a.w) << 16);
    u.z = f2bf(b.x) | (f2bf(b.y) << 16);
    u.w = f2bf(b.z) | (f2bf(b.w) << 16);
    return u;
  }
}

template <int HIN>
__global__ __launch_bounds__(kThreads) void head_lse_kernel(HeadParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t Hs[2][kMT * kHP];
  __shared__ float red[4][kMT][2];

  // XCD-aware order: work groups are dealt round-robin to the 8 XCDs, so the
  // M chunks of one vocabulary slice are given consecutive slots of one XCD
  // and stream the same W rows through its L2 together.
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  const int slice = (slot / p.n_mchunks) * 8 + xcd;
  const int mchunk = slot % p.n_mchunks;
  if (slice >= p.n_slices) return;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int qi = lane & 31, half = lane >> 5;
  const int v_w0 = slice * kVocabTile + wave * 64;  // this wave's 64 vocabulary rows
  const int m0 = mchunk * kMT;

  // W row pointers (rows past the vocabulary read row 0 and are masked later)
  const uint16_t *wrow[2];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb) {
    int v = v_w0 + vb * 32 + qi;
    wrow[vb] = p.W + (size_t)(v < p.V ? v : 0) * p.H + half * 8;
  }
  // hidden tile: 128 rows x 64 k per stage, 16-byte units (4 per thread)
  int hrow[4], hm[4], hk[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    int unit = tid + u * kThreads;
    hm[u] = unit >> 3;
    hk[u] = (unit & 7) * 8;
    int m = m0 + hm[u];
    hrow[u] = m < p.M ? p.scored[m] : -1;
  }

  f32x16 acc[2][4];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[vb][mb] = f32x16{0.f};

  const int S = p.H / kKT;
  bf16x8_t wcur[2][4], wnext[2][4];
  uint4 hreg[4];
#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) wcur[vb][ks] = *(const bf16x8_t *)(wrow[vb] + ks * 16);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    uint4 val = hrow[u] >= 0 ? load_hidden8<HIN>(p.hidden, hrow[u], p.H, hk[u]) : uint4{0u, 0u, 0u, 0u};
    *(uint4 *)(&Hs[0][hm[u] * kHP + hk[u]]) = val;
  }
  __syncthreads();

  for (int s = 0; s < S; ++s) {
    const int k1 = (s + 1) * kKT;
    const bool more = s + 1 < S;
    if (more) {
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) wnext[vb][ks] = *(const bf16x8_t *)(wrow[vb] + k1 + ks * 16);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        hreg[u] = hrow[u] >= 0 ? load_hidden8<HIN>(p.hidden, hrow[u], p.H, k1 + hk[u]) : uint4{0u, 0u, 0u, 0u};
    }
    const uint16_t *Hb = Hs[s & 1];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        bf16x8_t bfrag = *(const bf16x8_t *)(Hb + (mb * 32 + qi) * kHP + ks * 16 + half * 8);
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
          acc[vb][mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wcur[vb][ks], bfrag, acc[vb][mb], 0, 0, 0);
      }
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < 4; ++u) *(uint4 *)(&Hs[(s + 1) & 1][hm[u] * kHP + hk[u]]) = hreg[u];
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) wcur[vb][ks] = wnext[vb][ks];
    }
    __syncthreads();
  }

  // epilogue.  Lane holds column m = mb*32 + qi; register r of block vb holds
  // vocabulary row v_w0 + vb*32 + (r/4)*8 + half*4 + r%4.
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    float mx = kNegInf;
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int v = v_w0 + vb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
        if (v >= p.V) acc[vb][mb][r] = kNegInf;
        mx = fmaxf(mx, acc[vb][mb][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    float se = 0.f;
    if (mx != kNegInf) {
#pragma unroll
      for (int vb = 0; vb < 2; ++vb)
#pragma unroll
        for (int r = 0; r < 16; ++r) se += __expf(acc[vb][mb][r] - mx);
    }
    se = se + __shfl_xor(se, 32);
    if (half == 0) {
      red[wave][mb * 32 + qi][0] = mx;
      red[wave][mb * 32 + qi][1] = se;
    }
    // capture the logits of the tokens this row predicts
    const int m = m0 + mb * 32 + qi;
    if (m < p.M) {
      const int t0 = p.tgt_off[m], t1 = p.tgt_off[m + 1];
      for (int t = t0; t < t1; ++t) {
        const int rel = p.tgt_tok[t] - v_w0;
        if (rel < 0 || rel >= 64) continue;
        const int rr = rel & 31;
        if (((rr >> 2) & 1) != half) continue;
        const int vbt = rel >> 5, rt = (rr >> 3) * 4 + (rr & 3);
        float val = 0.f;
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) val = (vb == vbt && r == rt) ? acc[vb][mb][r] : val;
        p.tz[t] = val;
      }
    }
  }
  __syncthreads();
  if (tid < kMT) {
    const int m = m0 + tid;
    if (m < p.M) {
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, red[w][tid][0]);
      float Ssum = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        float mw = red[w][tid][0];
        Ssum += mw == kNegInf ? 0.f : red[w][tid][1] * __expf(mw - M);
      }
      float *dst = p.part + ((size_t)m * p.n_slices + slice) * 2;
      dst[0] = M;
      dst[1] = Ssum;
    }
  }
}

struct FinParams {
  int n_slices;
  const SpbBranch *branches;
  const int32_t *opt_step_off, *step_slot, *step_row;
  const float *part, *tz;
  float *lse, *lp, *p, *residual;
};

__device__ inline void merge(float &M, float &S, float m2, float s2) {
  float Mn = fmaxf(M, m2);
  float a = M == kNegInf ? 0.f : S * __expf(M - Mn);
  float b = m2 == kNegInf ? 0.f : s2 * __expf(m2 - Mn);
  M = Mn;
  S = a + b;
}

__global__ __launch_bounds__(64) void finalize_kernel(FinParams f) {
  const SpbBranch br = f.branches[blockIdx.x];
  const int lane = threadIdx.x;
  // LSE of each scored row of the branch: slices in order per lane, then a
  // butterfly whose pairwise merges are commutative, so every lane agrees
  for (int s = br.scored0; s < br.scored0 + br.n_scored; ++s) {
    float M = kNegInf, S = 0.f;
    const float *pp = f.part + (size_t)s * f.n_slices * 2;
    for (int i = lane; i < f.n_slices; i += 64) merge(M, S, pp[2 * i], pp[2 * i + 1]);
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      float m2 = __shfl_xor(M, off), s2 = __shfl_xor(S, off);
      merge(M, S, m2, s2);
    }
    if (lane == 0) f.lse[s] = M + __logf(S);
  }
  __threadfence_block();
  __syncthreads();
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

int launch_score(const ScoreLaunch &a, void *stream) {
  hipStream_t s = (hipStream_t)stream;
  HeadParams p;
  p.hidden = a.hidden;
  p.W = (const uint16_t *)a.lm_head;
  p.H = a.hidden_dim;
  p.V = a.vocab;
  p.M = a.n_scored;
  p.n_slices = n_vocab_slices(a.vocab);
  p.n_mchunks = (a.n_scored + kMT - 1) / kMT;
  p.scored = (const int32_t *)a.scored;
  p.tgt_off = (const int32_t *)a.tgt_off;
  p.tgt_tok = (const int32_t *)a.tgt_tok;
  p.part = a.part;
  p.tz = a.tz;
  long long groups = (long long)((p.n_slices + 7) / 8) * 8 * p.n_mchunks;
  if (groups > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  if (a.h_dtype == SPB_BF16)
    hipLaunchKernelGGL(head_lse_kernel<SPB_BF16>, dim3((unsigned)groups), dim3(kThreads), 0, s, p);
  else
    hipLaunchKernelGGL(head_lse_kernel<SPB_F32>, dim3((unsigned)groups), dim3(kThreads), 0, s, p);
  int e = (int)hipGetLastError();
  if (e) return e;
  FinParams f;
  f.n_slices = p.n_slices;
  f.branches = (const SpbBranch *)a.branches;
  f.opt_step_off = (const int32_t *)a.opt_step_off;
  f.step_slot = (const int32_t *)a.step_slot;
  f.step_row = (const int32_t *)a.step_row;
  f.part = a.part;
  f.tz = a.tz;
  f.lse = a.lse;
  f.lp = a.lp;
  f.p = a.p;
  f.residual = a.residual;
  hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)a.n_branches), dim3(64), 0, s, f);
  return (int)hipGetLastError();
}

}  // namespace spb
