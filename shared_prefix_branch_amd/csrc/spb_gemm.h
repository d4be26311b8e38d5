// spb_gemm.h -- the MFMA K steps shared by the lm head and the decoder
// stack's linear layers, and the linears' K loop (gfx950).  The lm head runs
// the same K steps in a stream over many tiles (head_lse_kernel).
//
// One work group (4 waves) computes a 256 x TM tile of Y^T = W . X^T: 256
// rows of W (vocabulary rows, or output features) against TM = 32 * MB rows
// of X (scored rows, or tokens), both K-contiguous bf16.  Wave w owns W rows
// w*64 .. +64 (two 32-row blocks) against all TM rows, on
// v_mfma_f32_32x32x16_bf16 with f32 accumulation.  Each K stage is 64
// elements, so every tile row is one 128-byte line.  Stage j's W tile is
// copied global -> LDS into ring slot j % 3 two stages ahead of use (each wave
// copies the 64 rows only it reads); its X tile into slot j % 2 one stage
// ahead.  Both are XOR-swizzled so fragment reads are free of bank conflicts.
// The loop is scheduled by hand (k_step): each MFMA of K step t is followed
// by one LDS read of step t+1's fragments and, in a stage's first two steps,
// one tile copy (X copies in the first, W copies in the second), so no queue
// takes a burst that holds up MFMA issue.
//
// Accumulator layout: acc[vb][mb] register r of lane (qi, half) holds
// W row w*64 + vb*32 + (r/4)*8 + half*4 + r%4 against X row mb*32 + qi.
//
// A result element depends only on its W row and X row, in a K order that
// is fixed (stage by stage, 16 elements per MFMA), so it does not depend on
// how many rows the launch covers.
#pragma once

#include "spb_dev.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spb {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr int kKT = 64;        // K elements per stage (128-byte LDS rows: one cache line)
constexpr int kThreads = 256;  // 4 waves
constexpr int kWRows = 256;    // W rows per work group

// LDS position, in 16-byte units, of chunk c (0..7) of row r of a tile with
// 128-byte rows.  A fragment read has 16 lanes in flight on 16 consecutive
// rows at one chunk; the XOR by (r/2)%8 puts them on 16 distinct 16-byte bank
// groups of the 64 banks.
__device__ inline int swz(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

template <int MB>
struct Tile {
  static constexpr int TM = 32 * MB;                // X rows per work group
  static constexpr int WBYTES = kWRows * 128;       // W stage: 256 rows x 64 bf16
  static constexpr int HBYTES = TM * 128;           // X stage: TM rows x 64 bf16
  static constexpr int RW = 3;                      // W ring: two stages in flight
  static constexpr int RH = 2;                      // X ring: one stage in flight
  static constexpr int LDS = RW * WBYTES + RH * HBYTES;  // <= 160 KB
  static constexpr int NW = 8;                      // W copies per wave per stage (its own 64 rows)
  static constexpr int NH = MB;                     // X copies per wave per stage
  static_assert(LDS <= 160 * 1024, "LDS ring too large");
};

// Fragments of one 16-element K step: A = the wave's 2 W blocks, B = the MB
// X blocks.
template <int MB>
struct Frags {
  bf16x8_t a[2];
  bf16x8_t b[MB];
};

// K step ks (0..3) of a 64-element stage: lane (qi, half) takes elements
// 16 ks + 8 half .. +8 of its row, i.e. chunk 2 ks + half.
template <int MB>
__device__ __attribute__((always_inline)) inline void frags(Frags<MB> &f, const u32x4 *Wb, const u32x4 *Hb, int ks,
                                                            int wave, int qi, int half) {
#pragma unroll
  for (int vb = 0; vb < 2; ++vb) {
    u32x4 u = Wb[swz(wave * 64 + vb * 32 + qi, ks * 2 + half)];
    f.a[vb] = *(bf16x8_t *)&u;
  }
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    u32x4 u = Hb[swz(mb * 32 + qi, ks * 2 + half)];
    f.b[mb] = *(bf16x8_t *)&u;
  }
}

// Piece j (0..MB+1) of a K step's fragments: the wave's W blocks, then the
// X blocks.
template <int MB>
__device__ __attribute__((always_inline)) inline void frag_piece(Frags<MB> &f, const u32x4 *Wb, const u32x4 *Hb,
                                                                 int ks, int j, int wave, int qi, int half) {
  if (j < 2) {
    u32x4 u = Wb[swz(wave * 64 + j * 32 + qi, ks * 2 + half)];
    f.a[j] = *(bf16x8_t *)&u;
  } else {
    u32x4 u = Hb[swz((j - 2) * 32 + qi, ks * 2 + half)];
    f.b[j - 2] = *(bf16x8_t *)&u;
  }
}

// One K step, scheduled by hand: its 2 MB MFMAs in the order of mfma(), and
// after MFMA j, piece j of the next step's fragments (when READ; pieces past
// the last MFMA follow it) and tile copies c0 + j*CPS .. +CPS (those below
// c1).  One MFMA, one read and a copy
// per slot keep the MFMA pipe fed while the LDS and memory queues take the
// rest; a burst of either would hold up MFMA issue.
// With ZERO, the step starts the accumulators (acc = A.B, not acc + A.B).
// With STRIDE > 1 the copies go out in groups of CPS after every STRIDE-th
// MFMA only (group q after MFMA q * STRIDE).
template <int MB, bool READ, int CPS, typename Copy, bool ZERO = false, int STRIDE = 1>
__device__ __attribute__((always_inline)) inline void k_step(f32x16 (&acc)[2][MB], const Frags<MB> &fc,
                                                             Frags<MB> &fn, const u32x4 *Wb, const u32x4 *Hb,
                                                             int ks_next, int wave, int qi, int half, Copy copy,
                                                             int c0, int c1) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int vb = 0; vb < 2; ++vb) {
      const int j = mb * 2 + vb;
      acc[vb][mb] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(fc.a[vb], fc.b[mb], ZERO ? f32x16{0.f} : acc[vb][mb], 0, 0, 0);
      if (READ && j < 2 + MB) frag_piece<MB>(fn, Wb, Hb, ks_next, j, wave, qi, half);
      if (j % STRIDE == 0) {
#pragma unroll
        for (int c = c0 + (j / STRIDE) * CPS; c < c0 + (j / STRIDE + 1) * CPS; ++c)
          if (c < c1) copy(c);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  // MB = 1: three pieces, two MFMAs
#pragma unroll
  for (int j = 2 * MB; j < 2 + MB; ++j)
    if (READ) frag_piece<MB>(fn, Wb, Hb, ks_next, j, wave, qi, half);
}

// N copies spread evenly over the 2 MB MFMA slots of one K step: a group of
// CPS copies after every STRIDE-th MFMA.
template <int MB, int N>
struct Spread {
  static constexpr int SLOTS = 2 * MB;
  static constexpr int STRIDE = (N > 0 && SLOTS / N > 0) ? SLOTS / N : 1;
  static constexpr int GROUPS = SLOTS / STRIDE;
  static constexpr int CPS = N > 0 ? (N + GROUPS - 1) / GROUPS : 0;
};

// Per-lane global byte offsets of the tile copies: one DMA instruction moves
// 8 rows x 128 bytes, lane t filling LDS position t%8 of row r8 + t/8, which
// swz() maps to chunk (t%8) ^ ((r/2)%8).  w_row(r) / x_row(r) give the global
// row of tile row r (already clamped into the operand); ldw / ldx are the
// operands' row lengths in elements.
template <int MB, typename WRow, typename XRow>
__device__ __attribute__((always_inline)) inline void tile_offsets(uint32_t (&woff)[8], uint32_t (&hoff)[MB],
                                                                   WRow w_row, XRow x_row, int ldw, int ldx,
                                                                   int wave, int lane) {
  const int dr = lane >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = wave * 64 + i * 8 + dr;
    const uint32_t c = (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    woff[i] = ((uint32_t)w_row(r) * (uint32_t)ldw + c * 8) * 2;
  }
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = (wave * MB + i) * 8 + dr;
    const uint32_t c = (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    hoff[i] = ((uint32_t)x_row(r) * (uint32_t)ldx + c * 8) * 2;
  }
}

// acc += W tile . X tile^T over S stages of 64 K elements.  W's K position
// wraps every SW stages (SW = S, except for the lm head's three-plane fp32
// kind, which sweeps W once per plane of X).  Ends with every copy landed and
// the LDS ring free for reuse.
template <int MB>
__device__ __attribute__((always_inline)) inline void k_loop(f32x16 (&acc)[2][MB], char *lds, const uint16_t *W,
                                                             const uint16_t *X, const uint32_t (&woff)[8],
                                                             const uint32_t (&hoff)[MB], int S, int SW, int wave,
                                                             int qi, int half) {
  using T = Tile<MB>;
  char *const wring = lds;
  char *const hring = lds + T::RW * T::WBYTES;
  const uint32_t lds0 = lds_addr(&lds[0]);
  auto copy_w = [&](int i, int stage, int sl) {  // W copy i (0..7) of a stage
    int ws = stage;
    if (ws >= SW) ws -= SW;
    if (ws >= SW) ws -= SW;
    const uint32_t kb = (uint32_t)ws * kKT * 2;
    const uint32_t s0 = lds0 + (uint32_t)sl * T::WBYTES;
    dma16(W, woff[i] + kb, __builtin_amdgcn_readfirstlane(s0 + (wave * 64 + i * 8) * 128));
  };
  auto copy_h = [&](int i, int stage, int sl) {  // X copy i (0..MB-1) of a stage
    const uint32_t kb = (uint32_t)stage * kKT * 2;
    const uint32_t s0 = lds0 + T::RW * T::WBYTES + (uint32_t)sl * T::HBYTES;
    dma16(X, hoff[i] + kb, __builtin_amdgcn_readfirstlane(s0 + (wave * T::NH + i) * 8 * 128));
  };
  auto issue_w = [&](int stage, int sl) {
#pragma unroll
    for (int i = 0; i < T::NW; ++i) copy_w(i, stage, sl);
  };
  auto issue_h = [&](int stage, int sl) {
#pragma unroll
    for (int i = 0; i < T::NH; ++i) copy_h(i, stage, sl);
  };

#pragma unroll
  for (int vb = 0; vb < 2; ++vb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[vb][mb] = f32x16{0.f};

  const int last = S - 1;
  // Copies past the last stage reload it into a slot nothing reads again, so
  // the count of copies in flight is the same on every trip.
  // The copies are spread evenly over each trip, a group after every few
  // MFMAs, so the L2 -> LDS stream never comes in bursts: the first half of
  // X(s+2) over K step 3 of trip s (stage s's X slot is free once the barrier
  // has passed), its second half over K step 0 of trip s+1, and W(s+2), two
  // stages ahead, over K steps 1 and 2.  At a trip's end only W(s+2) may be
  // in flight.
  constexpr int NH = T::NH, NW = T::NW;
  constexpr int NXA = (NH + 1) / 2;  // X copies over K step 3 (the rest over the next K step 0)
  constexpr int NWA = NW / 2;        // W copies over K step 1 (the rest over K step 2)
  using SXA = Spread<MB, NXA>;
  using SXB = Spread<MB, NH - NXA>;
  using SW1 = Spread<MB, NWA>;
  using SW2 = Spread<MB, NW - NWA>;
  issue_h(0, 0);
  issue_w(0, 0);
  issue_w(min(1, last), 1);
  wait_vmcnt<NW>();  // X(0), W(0) landed (this wave's copies)
  lds_barrier();
  int xst = min(1, last), xsl = 1;  // the X stage whose copies are under way, and its slot
#pragma unroll
  for (int i = 0; i < NXA; ++i) copy_h(i, xst, xsl);

  // The stage hand-off (copies landed, barrier) comes before the last K
  // step, whose MFMAs carry the reads of the next stage's first fragments, so
  // no stage starts by waiting on LDS.  The barrier follows every read of
  // stage s (its lgkmcnt(0)), so the copies after it may overwrite its slots.
  // After the last stage those reads fetch landed copies of the last stage,
  // unused.
  Frags<MB> f0, f1;
  frags<MB>(f0, (const u32x4 *)wring, (const u32x4 *)hring, 0, wave, qi, half);
  int sw = 0, sh = 0;  // ring slots of stage s
  for (int s = 0; s < S; ++s) {
    const u32x4 *Wb = (const u32x4 *)(wring + sw * T::WBYTES);
    const u32x4 *Hb = (const u32x4 *)(hring + sh * T::HBYTES);
    const int sw2 = sw == 0 ? 2 : sw - 1;  // slot of stage s + 2 (= s - 1 mod 3)
    const int sx2 = min(s + 2, last);
    const int cxst = xst, cxsl = xsl;
    auto copy_x = [&](int c) { copy_h(c, cxst, cxsl); };
    auto copy_wc = [&](int c) { copy_w(c, sx2, sw2); };
    __builtin_amdgcn_sched_barrier(0);
    k_step<MB, true, SXB::CPS, decltype(copy_x), false, SXB::STRIDE>(acc, f0, f1, Wb, Hb, 1, wave, qi, half, copy_x,
                                                                     NXA, NH);
    k_step<MB, true, SW1::CPS, decltype(copy_wc), false, SW1::STRIDE>(acc, f1, f0, Wb, Hb, 2, wave, qi, half,
                                                                      copy_wc, 0, NWA);
    k_step<MB, true, SW2::CPS, decltype(copy_wc), false, SW2::STRIDE>(acc, f0, f1, Wb, Hb, 3, wave, qi, half,
                                                                      copy_wc, NWA, NW);
    wait_vmcnt<NW>();  // X(s+1) and W(s+1) landed
    lds_barrier();
    xst = sx2;  // X(s+2) goes into stage s's X slot
    xsl = sh;
    sw = sw == 2 ? 0 : sw + 1;
    sh ^= 1;
    const int nxst = xst, nxsl = xsl;
    auto copy_nx = [&](int c) { copy_h(c, nxst, nxsl); };
    k_step<MB, true, SXA::CPS, decltype(copy_nx), false, SXA::STRIDE>(
        acc, f1, f0, (const u32x4 *)(wring + sw * T::WBYTES), (const u32x4 *)(hring + sh * T::HBYTES), 0, wave, qi,
        half, copy_nx, 0, NXA);
  }
  wait_vmcnt<0>();  // no copy may land after the ring is reused or released
  lds_barrier();
}

}  // namespace gemm
}  // namespace spb
