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
//   bf16 with f32 accumulation over tiles of (256-row vocabulary slice,
//   32..256 scored rows), each wave a 64-row vocabulary strip against all the
//   tile's rows.  One resident work group per compute unit walks its list of
//   tiles as one stream of 64-element K stages, copied global -> LDS
//   asynchronously into XOR-swizzled rings, so a tile's first stages load
//   during the previous tile's epilogue.  Logits never leave registers: the
//   epilogue writes, per (row, slice), the slice max and sum of exp(z - max),
//   and stores the logits of the option tokens the row predicts.
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

#include <algorithm>
#include <atomic>
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

// A work group stays resident and computes a list of 256 x TM tiles (256
// vocabulary rows x TM = 32*MB scored rows) as one continuous stream of
// 64-element K stages: stage g of the stream is stage g mod S of tile g / S
// (S = Hrow / 64).  The W and h rings of the K loop (spb_gemm.h) rotate over
// the whole stream, so the copies of a tile's first stages are issued during
// the previous tile's last stages and land while its epilogue runs; a tile
// never starts by waiting on memory, and no work group is launched per tile.
//
// XCD-aware order: work groups are dealt round-robin to the 8 XCDs, so block
// b runs on XCD b mod 8 as its (b / 8)-th of P groups there.  The XCD's tile
// slots are k = 0, 1, ... with slice (k / n_mchunks) * 8 + xcd and row chunk
// k mod n_mchunks; group j takes slots j, j + P, j + 2P, ...  The P groups of
// an XCD move through their lists at the same pace, so the row chunks of one
// vocabulary slice run side by side there and share its W lines in that
// XCD's L2.
template <int MB>
__global__ __launch_bounds__(kThreads, 1) void head_lse_kernel(HeadParams p) {
  using T = HeadTile<MB>;
  constexpr int TM = T::TM;
  constexpr int NH = T::NH, NW = T::NW;
  __shared__ __attribute__((aligned(1024))) char lds[T::LDS];

  const int b = blockIdx.x;
  const int xcd = b & 7, j = b >> 3, P = (int)(gridDim.x >> 3);
  const int slots = ((p.n_slices - xcd + 7) >> 3) * p.n_mchunks;
  const int n_tiles = j < slots ? (slots - j + P - 1) / P : 0;
  if (n_tiles == 0) return;
  auto slice_of = [&](int t) { return ((j + t * P) / p.n_mchunks) * 8 + xcd; };
  auto m0_of = [&](int t) { return ((j + t * P) % p.n_mchunks) * TM; };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform within the wave
  const int qi = lane & 31, half = lane >> 5;
  const int dr = lane >> 3;

  // Copy offsets (bytes): one DMA instruction moves 8 rows x 128 bytes, lane
  // t filling LDS position t%8 of row r8 + t/8, i.e. chunk (t%8) ^ ((r/2)%8)
  // of that row (swz).  h rows are offsets from the tile's first row; W rows
  // past the vocabulary (its last slice) are clamped onto its last row.
  uint32_t hoff[MB], woff[8];
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = (wave * MB + i) * 8 + dr;
    hoff[i] = ((uint32_t)r * (uint32_t)p.Hrow + (uint32_t)((lane & 7) ^ ((r >> 1) & 7)) * 8) * 2;
  }
  auto w_offsets = [&](int v0) {
    const int rmax = p.V - 1 - v0;
    int l = lane;
    asm volatile("" : "+v"(l));  // recomputed from the lane here, not kept in registers across the loop
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = wave * 64 + i * 8 + (l >> 3);
      woff[i] = ((uint32_t)min(r, rmax) * (uint32_t)p.H + (uint32_t)((l & 7) ^ ((r >> 1) & 7)) * 8) * 2;
    }
  };

  char *const wring = lds;
  const uint32_t lds0 = lds_addr(&lds[0]);
  const uint32_t hring0 = lds0 + T::RW * T::WBYTES;
  // Copy i of a stage: the stage's base pointer and the wave's first LDS row
  // in the slot are scalars, the lane's offset is fixed.
  auto copy_h = [&](int i, const uint16_t *xs, uint32_t lbase) { dma16(xs, hoff[i], lbase + i * 8 * 128); };
  auto copy_w = [&](int i, const uint16_t *ws, uint32_t lbase) { dma16(ws, woff[i], lbase + i * 8 * 128); };
  auto h_stage = [&](const uint16_t *xb, int xk) { return xb + xk * kKT; };
  auto w_stage = [&](const uint16_t *wb, int wk) {
    int ws = wk;  // the fp32 kind sweeps W once per plane of h
    if (ws >= p.SW) ws -= p.SW;
    if (ws >= p.SW) ws -= p.SW;
    return wb + ws * kKT;
  };
  auto h_lds = [&](int sl) {
    return __builtin_amdgcn_readfirstlane(hring0 + (uint32_t)sl * T::HBYTES + wave * NH * 8 * 128);
  };
  auto w_lds = [&](int sl) { return __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)sl * T::WBYTES + wave * 64 * 128); };

  // The stream position of the next h copies (tile xt, stage xk) and of the
  // next W copies (wt, wk).  Past the stream's last stage they stay on it:
  // those copies reload it into a slot nothing reads again, so every trip
  // has the same copies in flight.
  const int S = p.Hrow / kKT;
  int xt = 0, xk = 0, wt = 0, wk = 0;
  const uint16_t *xb = p.hg + (size_t)m0_of(0) * p.Hrow;
  int v0w = slice_of(0) * kVocabTile;
  const uint16_t *wb = p.W + (size_t)v0w * p.H;
  w_offsets(v0w);
  auto next_x = [&]() {
    if (xk + 1 < S) {
      ++xk;
    } else if (xt + 1 < n_tiles) {
      ++xt;
      xk = 0;
      xb = p.hg + (size_t)m0_of(xt) * p.Hrow;
    }
  };
  auto next_w = [&]() {
    if (wk + 1 < S) {
      ++wk;
    } else if (wt + 1 < n_tiles) {
      ++wt;
      wk = 0;
      v0w = slice_of(wt) * kVocabTile;
      wb = p.W + (size_t)v0w * p.H;
      w_offsets(v0w);
    }
  };

  f32x16 acc[2][MB];

  // Epilogue of tile t, in the 32 KB W slot R that the stream's stage just
  // finished with (the next copy into it is issued on the next trip).  R
  // holds the four waves' (max, sum) per row, then the tile's target CSR and,
  // when they fit, its target tokens, copied in asynchronously while the
  // slice statistics are computed, so no step waits on a global load.
  constexpr int kOffN = (TM + 1 + 63) / 64 * 64;
  constexpr int kTokCap = ((T::WBYTES - 4 * TM * 2 * 4 - 4 * kOffN) / 4) / 64 * 64;
  static_assert(kTokCap >= 4 * TM, "room for several targets per row");
  // A tile's first and end target positions (tb, te) are scalar loads (the
  // CSR is constant while the kernel runs) issued one epilogue ahead, so no
  // epilogue waits on them.
  typedef const __attribute__((address_space(4))) int32_t *const_i32;
  const const_i32 csr = (const_i32)p.tgt_off;
  auto tile_targets = [&](int t, int &tb, int &te) {
    const int m0 = m0_of(t);
    tb = csr[min(m0, p.M)];
    te = csr[min(m0 + TM, p.M)];
  };
  int tb_next = 0, te_next = 0;
  tile_targets(0, tb_next, te_next);
  auto epilogue = [&](int t, char *R) {
    const int v0 = slice_of(t) * kVocabTile, m0 = m0_of(t);
    float (*red)[TM][2] = (float (*)[TM][2])R;  // [4][TM][2]
    int *s_off = (int *)(R + 4 * TM * 2 * 4);   // [kOffN]: the CSR entries of rows m0 .. m0 + TM, raw
    int *s_tok = s_off + kOffN;                 // [kTokCap]
    const int tb = tb_next, te = te_next;
    if (t + 1 < n_tiles) tile_targets(t + 1, tb_next, te_next);
    const int n_tok = te - tb;
    const bool staged = n_tok <= kTokCap;
    for (int i0 = wave * 64; i0 < kOffN; i0 += 256)
      dma4(p.tgt_off, (uint32_t)min(m0 + i0 + lane, p.M) * 4, lds_addr(s_off + i0));
    if (staged)
      for (int i0 = wave * 64; i0 < n_tok; i0 += 256)
        dma4(p.tgt_tok, (uint32_t)(tb + min(i0 + lane, n_tok - 1)) * 4, lds_addr(s_tok + i0));

    // Lane holds column m = m0 + mb*32 + qi; register r of block vb holds
    // vocabulary row v0 + wave*64 + vb*32 + (r/4)*8 + half*4 + r%4.
    const int vw0 = v0 + wave * 64;
    const int nvalid = p.V - vw0;    // rows past the vocabulary (last slice only) are excluded
    const bool full = nvalid >= 64;  // uniform: every strip but the vocabulary's tail
    constexpr float kL2e = 1.44269504088896340736f;
    auto logits = [&](int mb, f32x16 (&z)[2]) {
      z[0] = acc[0][mb];
      z[1] = acc[1][mb];
      asm volatile("" : "+v"(z[0]), "+v"(z[1]));  // the copy out of acc happens here
      if (p.round_bf16) {
#pragma unroll
        for (int vb = 0; vb < 2; ++vb)
#pragma unroll
          for (int r = 0; r < 16; ++r) z[vb][r] = bf2f(f2bf(z[vb][r]));
      }
    };
    // one 32-row block at a time, so only its two accumulators leave the
    // accumulation registers at once
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      f32x16 z[2];
      logits(mb, z);
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
      if (half == 0) {
        red[wave][mb * 32 + qi][0] = mx;
        red[wave][mb * 32 + qi][1] = se;
      }
    }
    wait_vmcnt<0>();  // the CSR and token copies (and the stream's W copies before them) landed
    lds_barrier();

    // capture the logits of the tokens each row predicts
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int ml = mb * 32 + qi;
      if (m0 + ml < p.M) {
        const int t0 = s_off[ml] - tb, t1 = s_off[ml + 1] - tb;
        for (int t = t0; t < t1; ++t) {
          const int rel = (staged ? s_tok[t] : p.tgt_tok[tb + t]) - vw0;
          if (rel < 0 || rel >= 64) continue;
          const int rr = rel & 31;
          if (((rr >> 2) & 1) != half) continue;
          const int vbt = rel >> 5, rt = (rr >> 3) * 4 + (rr & 3);
          f32x16 z[2];
          logits(mb, z);
          float val = 0.f;
#pragma unroll
          for (int vb = 0; vb < 2; ++vb)
#pragma unroll
            for (int r = 0; r < 16; ++r) val = (vb == vbt && r == rt) ? z[vb][r] : val;
          p.tz[tb + t] = val;
        }
      }
    }
    // merge the four waves' (max, sum) in wave order
    for (int ml = tid; ml < TM; ml += kThreads) {
      const int m = m0 + ml;
      if (m < p.M) {
        float M = red[0][ml][0], Ssum = red[0][ml][1];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const float a = red[w][ml][0];
          const float Mn = fmaxf(M, a);
          Ssum = (M == kNegInf ? 0.f : Ssum * __expf(M - Mn)) + (a == kNegInf ? 0.f : red[w][ml][1] * __expf(a - Mn));
          M = Mn;
        }
        float *dst = p.part + ((size_t)m * p.n_slices + v0 / kVocabTile) * 2;
        dst[0] = M;
        dst[1] = Ssum;
      }
    }
    lds_barrier();  // R is free again for the stream's copies
  };

  // Trip g: K steps 0-2 of stage g, the hand-off, then K step 3, whose MFMAs
  // carry the reads of stage g+1's first fragments.  The copies are spread
  // evenly over the trip, a group after every few MFMAs, so the L2 -> LDS
  // stream never comes in bursts: the first half of h(g+2) over K step 3
  // (stage g's h slot is free once the barrier has passed), its second half
  // over the next trip's K step 0, and W(g+2), two stages ahead, over K steps
  // 1 and 2.  The barrier follows every read of stage g (its lgkmcnt(0)), so
  // stage g's slots are free after it.  A result element sees the same MFMAs
  // in the same order as in a loop over one tile: its W row and h row, K
  // stage by stage, 16 elements per MFMA.
  constexpr int NXA = (NH + 1) / 2, NXB = NH - NXA;  // h copies over K step 3, then the next K step 0
  constexpr int NWA = NW / 2;                          // W copies over K step 1 (the rest over K step 2)
  using SXA = gemm::Spread<MB, NXA>;
  using SXB = gemm::Spread<MB, NXB>;
  using SW1 = gemm::Spread<MB, NWA>;
  using SW2 = gemm::Spread<MB, NW - NWA>;
  const u32x4 *const wr = (const u32x4 *)wring;
  const u32x4 *const hr = (const u32x4 *)(lds + T::RW * T::WBYTES);
  constexpr int WQ = T::WBYTES / 16, HQ = T::HBYTES / 16;  // slot sizes in 16-byte units

  // Prologue: h(0), W(0), W(1), then the first half of h(1).
  {
    const uint16_t *xs = h_stage(xb, xk);
    const uint32_t xl = h_lds(0);
#pragma unroll
    for (int i = 0; i < NH; ++i) copy_h(i, xs, xl);
    next_x();
#pragma unroll
    for (int s1 = 0; s1 < 2; ++s1) {
      const uint16_t *ws = w_stage(wb, wk);
      const uint32_t wl = w_lds(s1);
#pragma unroll
      for (int i = 0; i < NW; ++i) copy_w(i, ws, wl);
      next_w();
    }
  }
  wait_vmcnt<NW>();  // h(0), W(0) landed (this wave's copies)
  lds_barrier();
  const uint16_t *pxs = h_stage(xb, xk);  // the h stage whose copies are under way
  uint32_t pxl = h_lds(1);
#pragma unroll
  for (int i = 0; i < NXA; ++i) copy_h(i, pxs, pxl);

  gemm::Frags<MB> f0, f1;
  gemm::frags<MB>(f0, wr, hr, 0, wave, qi, half);
  int sw = 0, sh = 0;  // ring slots of the stream's current stage
  for (int tt = 0; tt < n_tiles; ++tt) {
    int sw_done = 0;
    for (int kst = 0; kst < S; ++kst) {
      const u32x4 *Wb = wr + sw * WQ;
      const u32x4 *Hb = hr + sh * HQ;
      const uint16_t *cws = w_stage(wb, wk);
      const uint32_t cwl = w_lds(sw == 0 ? 2 : sw - 1);  // slot of the stage two ahead (= one behind, mod 3)
      const uint16_t *cxs = pxs;
      const uint32_t cxl = pxl;
      auto copy_x = [&](int c) { copy_h(c, cxs, cxl); };
      auto copy_wc = [&](int c) { copy_w(c, cws, cwl); };
      __builtin_amdgcn_sched_barrier(0);
      if (kst == 0)  // a tile's first K step starts its accumulators
        gemm::k_step<MB, true, SXB::CPS, decltype(copy_x), true, SXB::STRIDE>(acc, f0, f1, Wb, Hb, 1, wave, qi,
                                                                               half, copy_x, NXA, NH);
      else
        gemm::k_step<MB, true, SXB::CPS, decltype(copy_x), false, SXB::STRIDE>(acc, f0, f1, Wb, Hb, 1, wave, qi,
                                                                                half, copy_x, NXA, NH);
      next_x();
      gemm::k_step<MB, true, SW1::CPS, decltype(copy_wc), false, SW1::STRIDE>(acc, f1, f0, Wb, Hb, 2, wave, qi, half,
                                                                              copy_wc, 0, NWA);
      gemm::k_step<MB, true, SW2::CPS, decltype(copy_wc), false, SW2::STRIDE>(acc, f0, f1, Wb, Hb, 3, wave, qi, half,
                                                                              copy_wc, NWA, NW);
      next_w();
      wait_vmcnt<NW>();  // the next stage's h and W copies landed
      lds_barrier();
      sw_done = sw;
      sw = sw == 2 ? 0 : sw + 1;
      pxs = h_stage(xb, xk);  // h(g+2) goes into stage g's h slot
      pxl = h_lds(sh);
      sh ^= 1;
      const uint16_t *nxs = pxs;
      const uint32_t nxl = pxl;
      auto copy_nx = [&](int c) { copy_h(c, nxs, nxl); };
      gemm::k_step<MB, true, SXA::CPS, decltype(copy_nx), false, SXA::STRIDE>(acc, f1, f0, wr + sw * WQ,
                                                                              hr + sh * HQ, 0, wave, qi, half,
                                                                              copy_nx, 0, NXA);
    }
    // The next stage's first fragments are read again after the epilogue
    // (its slots are not the one the epilogue uses), so they hold no
    // registers during it.
    epilogue(tt, wring + sw_done * T::WBYTES);
    gemm::frags<MB>(f0, wr + sw * WQ, hr + sh * HQ, 0, wave, qi, half);
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
// Compute units of the current device (cached per device).
int device_cus() {
  static std::atomic<int> cached[16];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

int launch_head(const HeadParams &p0, int mb, void *ev_begin, void *ev_end, hipStream_t s) {
  HeadParams p = p0;
  // one resident work group per compute unit, P per XCD, each walking its
  // list of tiles (never more groups than an XCD has tile slots)
  const long long slots = (long long)((p.n_slices + 7) / 8) * p.n_mchunks;
  if (slots > 0x7FFFFFFFll / 8) return (int)hipErrorInvalidValue;
  const long long per_xcd = std::max(1, device_cus() / 8);
  const long long groups = 8 * std::min(per_xcd, slots);
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
