// spb_gemm8.h -- the K loop of spb_gemm.h on OCP e4m3 operands (gfx950).
//
// Same tile, rings, swizzle and copies as the bf16 loop: a stage is
// still one 128-byte line per tile row, now 128 K elements, and each stage is
// two K steps of v_mfma_scale_f32_32x32x64_f8f6f4 (e4m3 x e4m3, f32
// accumulation, scale operands neutral).  Lane (qi, half) of a K step holds
// the 32 bytes 32 * half .. +32 of its row's 64-element step, i.e. the
// 16-byte chunks 4 ks + 2 half and 4 ks + 2 half + 1 of the stage.  The K
// order of every result element is fixed, as in the bf16 loop.
#pragma once

#include "spb_gemm.h"

namespace spb {
namespace gemm {

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kKT8 = 128;  // e4m3 K elements per stage (128-byte rows)

template <int MB>
struct Frags8 {
  i32x8 a[2];
  i32x8 b[MB];
};

__device__ __attribute__((always_inline)) inline i32x8 frag8(const u32x4 *T, int row, int c) {
  const u32x4 u0 = T[swz(row, c)], u1 = T[swz(row, c + 1)];
  return i32x8{(int)u0.x, (int)u0.y, (int)u0.z, (int)u0.w, (int)u1.x, (int)u1.y, (int)u1.z, (int)u1.w};
}

template <int MB>
__device__ __attribute__((always_inline)) inline void frags8(Frags8<MB> &f, const u32x4 *Wb, const u32x4 *Hb, int ks,
                                                             int wave, int qi, int half) {
  const int c = ks * 4 + half * 2;
#pragma unroll
  for (int vb = 0; vb < 2; ++vb) f.a[vb] = frag8(Wb, wave * 64 + vb * 32 + qi, c);
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) f.b[mb] = frag8(Hb, mb * 32 + qi, c);
}

// A K step scheduled by hand, as k_step: after MFMA j, piece j of the next
// step's fragments (two 16-byte reads) when READ, and copies c0 + j*CPS ..
// +CPS below c1.
template <int MB, bool READ, int CPS, typename Copy>
__device__ __attribute__((always_inline)) inline void k_step8(f32x16 (&acc)[2][MB], const Frags8<MB> &fc,
                                                              Frags8<MB> &fn, const u32x4 *Wb, const u32x4 *Hb,
                                                              int ks_next, int wave, int qi, int half, Copy copy,
                                                              int c0, int c1) {
  const int c = ks_next * 4 + half * 2;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int vb = 0; vb < 2; ++vb) {
      const int j = mb * 2 + vb;
      acc[vb][mb] =
          __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(fc.a[vb], fc.b[mb], acc[vb][mb], 0, 0, 0, 0, 0, 0);
      if (READ && j < 2 + MB) {
        if (j < 2)
          fn.a[j] = frag8(Wb, wave * 64 + j * 32 + qi, c);
        else
          fn.b[j - 2] = frag8(Hb, (j - 2) * 32 + qi, c);
      }
#pragma unroll
      for (int k = c0 + j * CPS; k < c0 + (j + 1) * CPS; ++k)
        if (k < c1) copy(k);
      __builtin_amdgcn_sched_barrier(0);
    }
  // MB = 1: three pieces, two MFMAs
#pragma unroll
  for (int j = 2 * MB; j < 2 + MB; ++j)
    if (READ) fn.b[j - 2] = frag8(Hb, (j - 2) * 32 + qi, c);
}

// Byte offsets of the tile copies for 1-byte elements (see tile_offsets).
template <int MB, typename WRow, typename XRow>
__device__ __attribute__((always_inline)) inline void tile_offsets8(uint32_t (&woff)[8], uint32_t (&hoff)[MB],
                                                                    WRow w_row, XRow x_row, int ldw, int ldx,
                                                                    int wave, int lane) {
  const int dr = lane >> 3;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int r = wave * 64 + i * 8 + dr;
    const uint32_t c = (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    woff[i] = (uint32_t)w_row(r) * (uint32_t)ldw + c * 16;
  }
#pragma unroll
  for (int i = 0; i < MB; ++i) {
    const int r = (wave * MB + i) * 8 + dr;
    const uint32_t c = (uint32_t)((lane & 7) ^ ((r >> 1) & 7));
    hoff[i] = (uint32_t)x_row(r) * (uint32_t)ldx + c * 16;
  }
}

// acc += W tile . X tile^T over S stages of 128 e4m3 K elements; ends with
// every copy landed and the LDS ring free.
template <int MB>
__device__ __attribute__((always_inline)) inline void k_loop8(f32x16 (&acc)[2][MB], char *lds, const uint8_t *W,
                                                              const uint8_t *X, const uint32_t (&woff)[8],
                                                              const uint32_t (&hoff)[MB], int S, int wave, int qi,
                                                              int half) {
  using T = Tile<MB>;
  char *const wring = lds;
  char *const hring = lds + T::RW * T::WBYTES;
  const uint32_t lds0 = lds_addr(&lds[0]);
  auto copy_w = [&](int i, int stage, int sl) {
    const uint32_t s0 = lds0 + (uint32_t)sl * T::WBYTES;
    dma16(W, woff[i] + (uint32_t)stage * 128, __builtin_amdgcn_readfirstlane(s0 + (wave * 64 + i * 8) * 128));
  };
  auto copy_h = [&](int i, int stage, int sl) {
    const uint32_t s0 = lds0 + T::RW * T::WBYTES + (uint32_t)sl * T::HBYTES;
    dma16(X, hoff[i] + (uint32_t)stage * 128, __builtin_amdgcn_readfirstlane(s0 + (wave * T::NH + i) * 8 * 128));
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
  // the copy schedule of k_loop: trip s issues X(s+1) then W(s+2)
  issue_h(0, 0);
  issue_w(0, 0);
  issue_w(min(1, last), 1);
  wait_vmcnt<T::NW>();
  lds_barrier();
  // per stage: X(s+1) over the slots of the first K step, whose MFMAs also
  // carry the second step's fragment reads, then W(s+2) over the second
  constexpr int NC = T::NH + T::NW;
  constexpr int CPSX = (T::NH + 2 * MB - 1) / (2 * MB);
  constexpr int CPSW = (T::NW + 2 * MB - 1) / (2 * MB);
  int sw = 0, sh = 0;
  for (int s = 0; s < S; ++s) {
    const u32x4 *Wb = (const u32x4 *)(wring + sw * T::WBYTES);
    const u32x4 *Hb = (const u32x4 *)(hring + sh * T::HBYTES);
    Frags8<MB> f0, f1;
    frags8<MB>(f0, Wb, Hb, 0, wave, qi, half);
    const int sw2 = sw == 0 ? 2 : sw - 1;
    const int sx = min(s + 1, last), sx2 = min(s + 2, last);
    auto copy = [&](int c) {
      if (c < T::NH)
        copy_h(c, sx, sh ^ 1);
      else
        copy_w(c - T::NH, sx2, sw2);
    };
    __builtin_amdgcn_sched_barrier(0);
    k_step8<MB, true, CPSX>(acc, f0, f1, Wb, Hb, 1, wave, qi, half, copy, 0, T::NH);
    k_step8<MB, false, CPSW>(acc, f1, f0, Wb, Hb, 0, wave, qi, half, copy, T::NH, NC);
    wait_vmcnt<T::NW>();
    lds_barrier();
    sw = sw == 2 ? 0 : sw + 1;
    sh ^= 1;
  }
  wait_vmcnt<0>();
  lds_barrier();
}

}  // namespace gemm
}  // namespace spb
