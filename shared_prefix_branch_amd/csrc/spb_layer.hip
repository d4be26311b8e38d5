// spb_layer.hip -- the decoder stack around branch attention (gfx950):
// rmsnorm and the linear layers with their fused epilogues.
//
// The engine runs a whole decoder model over the packed pass and feeds its
// last hidden states to the head [PyPI "spinf-serve 0.1.1", "Layout": one
// packed forward].  The layer taken here is the plain pre-norm decoder layer
// (rmsnorm, q/k/v projections with rotary position embedding at each row's
// root-path position, branch attention, output projection, silu-gated MLP,
// residual adds in f32); every kernel works row by row or element by
// element of the packed pass, so a row's results do not depend on the rest
// of the pass.
//
// rmsnorm_kernel: one wave per row; the sum of squares runs lane by lane in
//   index order, then over a fixed butterfly (identical on every lane).
// linear_kernel<MODE>: Y^T = W . X^T on the K loop shared with the lm head
//   (spb_gemm.h), 256 W rows x 224 tokens per work group; the accumulators
//   are staged through LDS as f32 so that every global store is a whole
//   16-byte run of a token's row.  Epilogues:
//     BF16       y = bf16(x W^T)
//     RESIDUAL   resid += bf16(x W^T)                      (f32 residual stream)
//     SILU_GATE  y = bf16(silu(x Wg^T) * (x Wu^T)), W holding Wg and Wu
//                interleaved in blocks of 32 rows (gate block, then up block)
//     QKV_ROPE   q, k, v = split(x [Wq; Wk; Wv]^T), q and k rotated at the
//                row's position (pairs (2i, 2i+1), angle pos * theta_i, from
//                a (cos, sin) table), each rounded once to bf16
//     F32        y = x W^T in f32 (the lm head's logits for decoded rows)
#define SPB_HD __host__ __device__
#include "spb_meta.h"
#include "spb_launch.h"
#include "spb_dev.h"
#include "spb_gemm.h"
#include "spb_gemm8.h"
#include "../../include/spb.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spb {
namespace {

using gemm::f32x16;
using gemm::kKT;
using gemm::kThreads;
using gemm::kWRows;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ inline uint32_t f2bf(float f) {  // round to nearest even (finite inputs)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ inline float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// ------------------------------------------------------------------ rmsnorm

__global__ __launch_bounds__(256) void rmsnorm_kernel(NormLaunch a) {
  const long long row = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const float4 *x = (const float4 *)(a.x + row * a.dim);
  const int n4 = a.dim >> 2;
  float ss = 0.f;
  for (int i = lane; i < n4; i += 64) {
    const float4 v = x[i];
    ss = __builtin_fmaf(v.x, v.x, ss);
    ss = __builtin_fmaf(v.y, v.y, ss);
    ss = __builtin_fmaf(v.z, v.z, ss);
    ss = __builtin_fmaf(v.w, v.w, ss);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  const float inv = 1.0f / sqrtf(ss / (float)a.dim + a.eps);
  const u32x2 *g = (const u32x2 *)a.gain;
  u32x2 *out = (u32x2 *)(a.out + row * a.dim);
  for (int i = lane; i < n4; i += 64) {
    const float4 v = x[i];
    const u32x2 gg = g[i];
    const float y0 = v.x * inv * bf2f(gg.x & 0xFFFFu), y1 = v.y * inv * bf2f(gg.x >> 16);
    const float y2 = v.z * inv * bf2f(gg.y & 0xFFFFu), y3 = v.w * inv * bf2f(gg.y >> 16);
    out[i] = u32x2{f2bf(y0) | (f2bf(y1) << 16), f2bf(y2) | (f2bf(y3) << 16)};
  }
}

// ------------------------------------------------------------------ linear

constexpr int kMB = kLinearMB;
constexpr int kGroupM = 8;  // token chunks per group of the tile order (see the block mapping)

struct LinParams {
  LinearLaunch a;
  int n_wtiles, n_mchunks, per_xcd;
};

// One work group: W rows wt*256 .. +256 against tokens mchunk*224 .. +224.
// Tiles are ordered in groups of kGroupM token chunks x every W tile (token
// chunk fastest), and that order is cut into 8 contiguous ranges, one per
// XCD (work groups are dealt round-robin to the XCDs, block b to XCD b % 8).
// So every XCD gets the same number of tiles, and the 32 work groups an XCD
// runs at once cover 8 token chunks x 4 W tiles, sharing both through its L2.
template <int MODE, bool FP8>
__global__ __launch_bounds__(kThreads, 1) void linear_kernel(LinParams P) {
  using T = gemm::Tile<kMB>;
  constexpr int TM = T::TM;
  __shared__ __attribute__((aligned(1024))) char lds[T::LDS];
  const LinearLaunch &p = P.a;

  const int b = blockIdx.x;
  const int pid = (b & 7) * P.per_xcd + (b >> 3);
  if (pid >= P.n_wtiles * P.n_mchunks) return;
  const int span = kGroupM * P.n_wtiles;
  const int first_m = (pid / span) * kGroupM;
  const int gm = P.n_mchunks - first_m < kGroupM ? P.n_mchunks - first_m : kGroupM;
  const int mchunk = first_m + (pid % span) % gm;
  const int wt = (pid % span) / gm;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qi = lane & 31, half = lane >> 5;
  const int w0 = wt * kWRows;
  const int m0 = mchunk * TM;

  uint32_t woff[8], hoff[kMB];
  f32x16 acc[2][kMB];
  auto w_row = [&](int r) { return w0 + r < p.n ? w0 + r : p.n - 1; };
  auto x_row = [&](int r) { return m0 + r < p.m ? m0 + r : p.m - 1; };
  if constexpr (FP8) {
    // e4m3 operands; the products are scaled back by s_x * s_w
    gemm::tile_offsets8<kMB>(woff, hoff, w_row, x_row, p.k, p.k, wave, lane);
    gemm::k_loop8<kMB>(acc, lds, (const uint8_t *)p.w, (const uint8_t *)p.x, woff, hoff, p.k / gemm::kKT8, wave, qi,
                       half);
#pragma unroll
    for (int vb = 0; vb < 2; ++vb)
#pragma unroll
      for (int mb = 0; mb < kMB; ++mb) acc[vb][mb] *= p.scale;
  } else {
    gemm::tile_offsets<kMB>(woff, hoff, w_row, x_row, p.k, p.k, wave, lane);
    gemm::k_loop<kMB>(acc, lds, p.w, p.x, woff, hoff, p.k / kKT, p.k / kKT, wave, qi, half);
  }

  // ---- epilogue: f32 staging of up to 128 tokens at a time, [token][feature]
  constexpr bool GLU = MODE == SPB_LINEAR_SILU_GATE;
  constexpr int NF = GLU ? kWRows / 2 : kWRows;  // output features of the tile
  constexpr int PITCH = NF + 4;                  // floats per staged token row
  static_assert(128 * PITCH * 4 <= T::LDS, "staging must fit in the ring");
  float *st = (float *)lds;
  const int f0 = GLU ? wt * (kWRows / 2) : w0;   // first output feature of the tile
  const int nout = GLU ? p.n / 2 : p.n;
#pragma unroll
  for (int mb0 = 0; mb0 < kMB; mb0 += 4) {
    // registers -> LDS
#pragma unroll
    for (int mb = mb0; mb < mb0 + 4 && mb < kMB; ++mb) {
      float *row = st + ((mb - mb0) * 32 + qi) * PITCH;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        if constexpr (GLU) {
          float4 v;
          float *vv = (float *)&v;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float gt = acc[0][mb][g4 * 4 + j], up = acc[1][mb][g4 * 4 + j];
            vv[j] = gt / (1.0f + __expf(-gt)) * up;
          }
          *(float4 *)(row + wave * 32 + g4 * 8 + half * 4) = v;
        } else {
#pragma unroll
          for (int vb = 0; vb < 2; ++vb) {
            const float4 v = {acc[vb][mb][g4 * 4], acc[vb][mb][g4 * 4 + 1], acc[vb][mb][g4 * 4 + 2],
                              acc[vb][mb][g4 * 4 + 3]};
            *(float4 *)(row + wave * 64 + vb * 32 + g4 * 8 + half * 4) = v;
          }
        }
      }
    }
    __syncthreads();
    // LDS -> global: 8 consecutive features of one token per step
    const int ntok = (kMB - mb0 < 4 ? kMB - mb0 : 4) * 32;
    for (int u = tid; u < ntok * (NF / 8); u += kThreads) {
      const int tl = u / (NF / 8), c8 = u % (NF / 8);
      const int m = m0 + mb0 * 32 + tl;
      const int f = f0 + c8 * 8;
      if (m >= p.m || f >= nout) continue;
      const float4 a0 = *(const float4 *)(st + tl * PITCH + c8 * 8);
      const float4 a1 = *(const float4 *)(st + tl * PITCH + c8 * 8 + 4);
      float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      if constexpr (MODE == SPB_LINEAR_F32) {
        float4 *yf = (float4 *)(p.yf + (size_t)m * p.n + f);
        yf[0] = a0;
        yf[1] = a1;
      } else if constexpr (MODE == SPB_LINEAR_RESIDUAL) {
        float4 *r = (float4 *)(p.resid + (size_t)m * p.n + f);
        float4 r0 = r[0], r1 = r[1];
        r0.x += bf2f(f2bf(v[0])); r0.y += bf2f(f2bf(v[1])); r0.z += bf2f(f2bf(v[2])); r0.w += bf2f(f2bf(v[3]));
        r1.x += bf2f(f2bf(v[4])); r1.y += bf2f(f2bf(v[5])); r1.z += bf2f(f2bf(v[6])); r1.w += bf2f(f2bf(v[7]));
        r[0] = r0;
        r[1] = r1;
      } else {
        uint16_t *dst;
        if constexpr (MODE == SPB_LINEAR_QKV_ROPE) {
          const int d = p.head_dim, qd = p.hq * d, kd = p.hkv * d;
          if (f < qd + kd) {
            int ps = p.pos[m];
            ps = ps < 0 ? 0 : (ps >= p.n_pos ? p.n_pos - 1 : ps);
            const int i0 = (f % d) >> 1;
            const float4 *cs = (const float4 *)(p.rope + ((size_t)ps * (d >> 1) + i0) * 2);
            const float4 c01 = cs[0], c23 = cs[1];
            const float c[4] = {c01.x, c01.z, c23.x, c23.z}, s[4] = {c01.y, c01.w, c23.y, c23.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const float x0 = v[2 * j], x1 = v[2 * j + 1];
              v[2 * j] = x0 * c[j] - x1 * s[j];
              v[2 * j + 1] = x0 * s[j] + x1 * c[j];
            }
          }
          dst = f < qd ? p.q + (size_t)m * qd + f
                       : (f < qd + kd ? p.kk + (size_t)m * kd + (f - qd) : p.v + (size_t)m * kd + (f - qd - kd));
        } else {
          dst = p.y + (size_t)m * nout + f;
        }
        *(u32x4 *)dst = u32x4{f2bf(v[0]) | (f2bf(v[1]) << 16), f2bf(v[2]) | (f2bf(v[3]) << 16),
                              f2bf(v[4]) | (f2bf(v[5]) << 16), f2bf(v[6]) | (f2bf(v[7]) << 16)};
      }
    }
    __syncthreads();
  }
}

template <int MODE, bool FP8>
int launch_linear_mode(const LinearLaunch &a, hipStream_t s) {
  LinParams P;
  P.a = a;
  P.n_wtiles = (a.n + kWRows - 1) / kWRows;
  P.n_mchunks = (a.m + 32 * kMB - 1) / (32 * kMB);
  const long long tiles = (long long)P.n_wtiles * P.n_mchunks;
  if (tiles > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  P.per_xcd = (int)((tiles + 7) / 8);
  const long long blocks = 8ll * P.per_xcd;
  if (blocks > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  if (a.ev_begin) {
    hipError_t e = hipEventRecord((hipEvent_t)a.ev_begin, s);
    if (e != hipSuccess) return (int)e;
  }
  hipLaunchKernelGGL((linear_kernel<MODE, FP8>), dim3((unsigned)blocks), dim3(kThreads), 0, s, P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  if (a.ev_end) return (int)hipEventRecord((hipEvent_t)a.ev_end, s);
  return 0;
}

}  // namespace

int launch_rmsnorm(const NormLaunch &a, void *stream) {
  if (a.rows == 0) return 0;
  const long long blocks = (a.rows + 3) / 4;
  if (blocks > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(rmsnorm_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

namespace {

template <bool FP8>
int launch_linear_t(const LinearLaunch &a, hipStream_t s) {
  switch (a.mode) {
    case SPB_LINEAR_BF16: return launch_linear_mode<SPB_LINEAR_BF16, FP8>(a, s);
    case SPB_LINEAR_RESIDUAL: return launch_linear_mode<SPB_LINEAR_RESIDUAL, FP8>(a, s);
    case SPB_LINEAR_SILU_GATE: return launch_linear_mode<SPB_LINEAR_SILU_GATE, FP8>(a, s);
    case SPB_LINEAR_QKV_ROPE: return launch_linear_mode<SPB_LINEAR_QKV_ROPE, FP8>(a, s);
    case SPB_LINEAR_F32: return launch_linear_mode<SPB_LINEAR_F32, FP8>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

// ---------------------------------------------------------- e4m3 quantize

// OCP e4m3fn code of v (finite): the nearest value, ties to the even
// significand, saturated to +-448.
__device__ inline uint32_t f32_to_e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 31) << 7;
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {  // below 2^-6: subnormal steps of 2^-9 (8 steps reach 2^-6, code 8)
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    int e;
    const float m = frexpf(a, &e);        // a = m 2^e, 0.5 <= m < 1
    float q = __builtin_rintf(m * 16.0f);  // 8 .. 16: 1.fff with 3 fraction bits
    int E = e - 1;
    if (q == 16.0f) {
      q = 8.0f;
      ++E;
    }
    code = ((uint32_t)(E + 7) << 3) | ((uint32_t)q - 8u);
  }
  return sign | code;
}

// dst[i] = e4m3(src[i] * inv_scale), 8 elements per thread.
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(QuantLaunch a) {
  const long long i0 = ((long long)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i0 >= a.n) return;
  if (i0 + 8 <= a.n) {
    float v[8];
    if (a.src_f32) {
      const float4 u0 = *(const float4 *)(a.src_f32 + i0), u1 = *(const float4 *)(a.src_f32 + i0 + 4);
      v[0] = u0.x; v[1] = u0.y; v[2] = u0.z; v[3] = u0.w; v[4] = u1.x; v[5] = u1.y; v[6] = u1.z; v[7] = u1.w;
    } else {
      const u32x4 u = *(const u32x4 *)(a.src_bf16 + i0);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf2f(w[j] & 0xFFFFu);
        v[2 * j + 1] = bf2f(w[j] >> 16);
      }
    }
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      lo |= f32_to_e4m3(v[j] * a.inv_scale) << (8 * j);
      hi |= f32_to_e4m3(v[4 + j] * a.inv_scale) << (8 * j);
    }
    *(u32x2 *)(a.dst + i0) = u32x2{lo, hi};
  } else {
    for (long long i = i0; i < a.n; ++i) {
      const float v = a.src_f32 ? a.src_f32[i] : bf2f(a.src_bf16[i]);
      a.dst[i] = (uint8_t)f32_to_e4m3(v * a.inv_scale);
    }
  }
}

}  // namespace

int launch_quantize_e4m3(const QuantLaunch &a, void *stream) {
  if (a.n == 0) return 0;
  const long long blocks = (a.n + 2047) / 2048;
  if (blocks > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(quantize_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_linear(const LinearLaunch &a, void *stream) {
  if (a.m == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  return a.fp8 ? launch_linear_t<true>(a, s) : launch_linear_t<false>(a, s);
}

}  // namespace spb
