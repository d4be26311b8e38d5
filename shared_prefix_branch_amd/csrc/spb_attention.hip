// spb_attention.hip -- branch-masked packed attention for gfx950 (CDNA4).
//
// Computes, for every packed row x and query head h, softmax attention over
// the keys on x's root path only: its own content (causal for content rows,
// all of it for branch rows), its own template prefix and its own option-trie
// ancestors.  This is the pages' "content read once, every question a branch
// of the same pass" [PyPI "spinf-serve 0.1.1", "What it does"], with answers
// equal to running each content + question as its own prompt [PyPI, "Speed
// and scale"].
//
// Work item: up to 32*RW consecutive rows of one 128-row tile (rows of one
// segment) and one KV head.  Wave w handles 32 query rows for query head
// kvh*G + w%G; the G query heads of a KV group share every staged K/V chunk.
//
// Per chunk of 64 keys staged in LDS (K row-major, V transposed to d-major):
//   S^T = K Q^T      (MFMA 32x32x16 bf16, or 32x32x64 OCP e4m3 for fp8 Q/K)
//   online softmax   (each lane owns one query; f32, base-2 exponent)
//   O^T += V^T P^T   (MFMA 32x32x16 bf16, P rounded to bf16)
//
// Batch invariance: a row consumes its content keys in 64-key chunks aligned
// to its content start, then its branch keys in 64-key chunks aligned to its
// branch start.  Slot i of a chunk always holds chunk-relative key i, every
// masked slot contributes an exact zero and leaves the running max unchanged
// (alpha = 1), and every per-row sum runs in a fixed slot order.  So a row's
// bits depend on its own root path only, not on where its input was packed.
#define SPB_HD __host__ __device__
#include "spb_meta.h"
#include "spb_launch.h"
#include "../../include/spb.h"

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace spb {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

__device__ inline uint32_t f2bf(float f) {  // round to nearest even (inputs finite)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ inline float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// OCP e4m3fn byte -> bf16 bits (exact: every e4m3 value is a bf16 value).
__device__ inline uint32_t e4m3_to_bf(uint32_t b) {
  uint32_t s = (b & 0x80u) << 8;
  uint32_t e = (b >> 3) & 0xFu;
  uint32_t m = b & 0x7u;
  uint32_t normal = s | ((e + 120u) << 7) | (m << 4);
  uint32_t sub = s | (__float_as_uint((float)m * 0.001953125f) >> 16);  // m * 2^-9
  return e ? normal : sub;
}

struct AttnParams {
  const void *q, *k, *v;
  void *o;
  int hq, hkv, n_tokens;
  float sc;   // softmax scale * log2(e) * s_q * s_k
  float s_v;  // applied to the output
  const SpbRow *rows;
  const SpbTile *tiles;
  const SpbBranch *branches;
};

template <int D, int G, int IN>
struct Cfg {
  static constexpr int RW = G == 4 ? 2 : 4;      // 32-row groups per work item
  static constexpr int NW = RW * G;              // waves
  static constexpr int NT = NW * 64;
  static constexpr int ROWS = 32 * RW;
  static constexpr int SPLITS = 128 / ROWS;      // work items per 128-row tile
  static constexpr int KPAD = IN == SPB_FP8_E4M3 ? D + 16 : D + 8;  // K row pitch (elements)
  static constexpr int KBYTES = 64 * KPAD * (IN == SPB_FP8_E4M3 ? 1 : 2);
  static constexpr int VPAD = 68;                // V^T row pitch (bf16): 64 keys + 4
  static constexpr int VBYTES = D * VPAD * 2;
};

// ----------------------------------------------------------------- staging

template <int D, int G, int IN>
__device__ inline void stage_chunk(const AttnParams &p, int kvh, int key0, unsigned char *Ks, uint16_t *Vt) {
  using C = Cfg<D, G, IN>;
  const int tid = threadIdx.x;
  const int n = p.n_tokens;
  if constexpr (IN == SPB_FP8_E4M3) {
    const unsigned char *kp = (const unsigned char *)p.k;
    constexpr int KU = 64 * D / 16;
    for (int u = tid; u < KU; u += C::NT) {
      int key = u / (D / 16), dc = u % (D / 16);
      int y = key0 + key;
      uint4 val = {0u, 0u, 0u, 0u};
      if (y < n) val = *(const uint4 *)(kp + ((size_t)y * p.hkv + kvh) * D + dc * 16);
      *(uint4 *)(Ks + key * C::KPAD + dc * 16) = val;
    }
  } else {
    uint16_t *Kd = (uint16_t *)Ks;
    constexpr int KU = 64 * D / 8;
    for (int u = tid; u < KU; u += C::NT) {
      int key = u / (D / 8), dc = u % (D / 8);
      int y = key0 + key;
      uint4 val = {0u, 0u, 0u, 0u};
      if (y < n) {
        if constexpr (IN == SPB_BF16) {
          val = *(const uint4 *)((const uint16_t *)p.k + ((size_t)y * p.hkv + kvh) * D + dc * 8);
        } else {
          const float4 *src = (const float4 *)((const float *)p.k + ((size_t)y * p.hkv + kvh) * D + dc * 8);
          float4 a = src[0], b = src[1];
          val.x = f2bf(a.x) | (f2bf(a.y) << 16);
          val.y = f2bf(a.z) | (f2bf(a.w) << 16);
          val.z = f2bf(b.x) | (f2bf(b.y) << 16);
          val.w = f2bf(b.z) | (f2bf(b.w) << 16);
        }
      }
      *(uint4 *)(Kd + key * C::KPAD + dc * 8) = val;
    }
  }
  // V^T: each unit is 4 keys x 8 dims, written as 8 rows of 4 keys
  constexpr int VU = 16 * (D / 8);
  for (int u = tid; u < VU; u += C::NT) {
    int kg = u / (D / 8), dc = u % (D / 8);
    uint32_t e[4][8];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      int y = key0 + kg * 4 + kk;
      bool in = y < n;
      size_t base = ((size_t)(in ? y : 0) * p.hkv + kvh) * D + dc * 8;
      if constexpr (IN == SPB_BF16) {
        uint4 w = in ? *(const uint4 *)((const uint16_t *)p.v + base) : uint4{0u, 0u, 0u, 0u};
        uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[kk][2 * i] = ww[i] & 0xFFFFu;
          e[kk][2 * i + 1] = ww[i] >> 16;
        }
      } else if constexpr (IN == SPB_F32) {
        const float4 *src = (const float4 *)((const float *)p.v + base);
        float4 a = in ? src[0] : float4{0.f, 0.f, 0.f, 0.f};
        float4 b = in ? src[1] : float4{0.f, 0.f, 0.f, 0.f};
        e[kk][0] = f2bf(a.x); e[kk][1] = f2bf(a.y); e[kk][2] = f2bf(a.z); e[kk][3] = f2bf(a.w);
        e[kk][4] = f2bf(b.x); e[kk][5] = f2bf(b.y); e[kk][6] = f2bf(b.z); e[kk][7] = f2bf(b.w);
      } else {
        uint2 w = in ? *(const uint2 *)((const unsigned char *)p.v + base) : uint2{0u, 0u};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          e[kk][i] = e4m3_to_bf((w.x >> (8 * i)) & 0xFFu);
          e[kk][4 + i] = e4m3_to_bf((w.y >> (8 * i)) & 0xFFu);
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint2 w;
      w.x = e[0][i] | (e[1][i] << 16);
      w.y = e[2][i] | (e[3][i] << 16);
      *(uint2 *)(Vt + (dc * 8 + i) * C::VPAD + kg * 4) = w;
    }
  }
}

// ----------------------------------------------------------------- one chunk

template <int D, int IN>
struct QFrag {
  static constexpr int STEPS = IN == SPB_FP8_E4M3 ? D / 64 : D / 16;
  typename std::conditional<IN == SPB_FP8_E4M3, i32x8, bf16x8_t>::type f[STEPS];
};

struct RowState {
  float m;   // running max (base-2 logits)
  float l;   // this lane's partial row sum
};

template <int D, int G, int IN>
__device__ inline void chunk_step(const unsigned char *Ks, const uint16_t *Vt, const QFrag<D, IN> &qf,
                                  uint64_t mask, float sc, RowState &st, f32x16 (&o)[D / 32]) {
  using C = Cfg<D, G, IN>;
  const int lane = threadIdx.x & 63;
  const int qi = lane & 31, half = lane >> 5;
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{0.f};
    if constexpr (IN == SPB_FP8_E4M3) {
#pragma unroll
      for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
        const unsigned char *src = Ks + (kb * 32 + qi) * C::KPAD + t * 64 + half * 32;
        i32x8 a;
        uint4 a0 = *(const uint4 *)src, a1 = *(const uint4 *)(src + 16);
        a[0] = a0.x; a[1] = a0.y; a[2] = a0.z; a[3] = a0.w;
        a[4] = a1.x; a[5] = a1.y; a[6] = a1.z; a[7] = a1.w;
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf.f[t], s[kb], 0, 0, 0, 0, 0, 0);
      }
    } else {
      const uint16_t *Kd = (const uint16_t *)Ks;
#pragma unroll
      for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
        bf16x8_t a = *(const bf16x8_t *)(Kd + (kb * 32 + qi) * C::KPAD + t * 16 + half * 8);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf.f[t], s[kb], 0, 0, 0);
      }
    }
  }
  // online softmax: lane owns query qi; register r of block kb holds key
  // kb*32 + (r/4)*8 + half*4 + r%4
  float mloc = kNegInf;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      int key = kb * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
      float t = ((mask >> key) & 1ull) ? s[kb][r] * sc : kNegInf;
      s[kb][r] = t;
      mloc = fmaxf(mloc, t);
    }
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  float mnew = fmaxf(st.m, mloc);
  float alpha = mnew == kNegInf ? 1.f : exp2f(st.m - mnew);
  uint32_t pk[2][8];
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      float p0 = s[kb][r] == kNegInf ? 0.f : exp2f(s[kb][r] - mnew);
      float p1 = s[kb][r + 1] == kNegInf ? 0.f : exp2f(s[kb][r + 1] - mnew);
      uint32_t b0 = f2bf(p0), b1 = f2bf(p1);
      lsum += bf2f(b0);
      lsum += bf2f(b1);
      pk[kb][r >> 1] = b0 | (b1 << 16);
    }
  st.l = st.l * alpha + lsum;
  st.m = mnew;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
  // O^T += V^T P^T: k-step j covers keys 16j + half*4 + {0..3} and 16j + 8 + half*4 + {0..3}
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int kb = j >> 1, rb = (j & 1) * 4;
    union {
      uint32_t u[4];
      bf16x8_t v;
    } b;
    b.u[0] = pk[kb][rb]; b.u[1] = pk[kb][rb + 1]; b.u[2] = pk[kb][rb + 2]; b.u[3] = pk[kb][rb + 3];
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const uint16_t *row = Vt + (db * 32 + qi) * C::VPAD + 16 * j + half * 4;
      union {
        uint2 u[2];
        bf16x8_t v;
      } a;
      a.u[0] = *(const uint2 *)row;
      a.u[1] = *(const uint2 *)(row + 8);
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, o[db], 0, 0, 0);
    }
  }
}

__device__ inline uint64_t range_mask(int n) {  // bits [0, n), n clamped to [0, 64]
  n = n < 0 ? 0 : (n > 64 ? 64 : n);
  return n == 64 ? ~0ull : ((1ull << n) - 1ull);
}

// ----------------------------------------------------------------- kernel

template <int D, int G, int IN, int OUT>
__global__ __launch_bounds__((Cfg<D, G, IN>::NT)) void branch_attention_kernel(AttnParams p) {
  using C = Cfg<D, G, IN>;
  __shared__ __attribute__((aligned(16))) unsigned char Ks[C::KBYTES];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[C::VBYTES / 2];

  const int w = blockIdx.x;
  const int kvh = w % p.hkv;
  const int rest = w / p.hkv;
  const int split = rest % C::SPLITS;
  const SpbTile tile = p.tiles[rest / C::SPLITS];
  const int sub0 = tile.row0 + split * C::ROWS;
  const int sub_n = min(C::ROWS, tile.row0 + tile.nrows - sub0);
  if (sub_n <= 0) return;  // uniform over the work group

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int rw = wave / G, gh = wave % G;
  const int h = kvh * G + gh;
  const int qi = lane & 31, half = lane >> 5;
  const int local = rw * 32 + qi;
  const bool active = local < sub_n;
  const int x = sub0 + local;

  SpbRow row;
  if (active) {
    row = p.rows[x];
  } else {
    row.cvis = 0; row.seg = 0; row.br = -1; row.e = 0; row.L = 0; row.depth = 0; row.anc01 = 0; row.anc23 = 0;
  }

  QFrag<D, IN> qf;
  if constexpr (IN == SPB_FP8_E4M3) {
    const unsigned char *qp = (const unsigned char *)p.q + ((size_t)x * p.hq + h) * D;
#pragma unroll
    for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
      uint4 a0 = {0u, 0u, 0u, 0u}, a1 = {0u, 0u, 0u, 0u};
      if (active) {
        a0 = *(const uint4 *)(qp + t * 64 + half * 32);
        a1 = *(const uint4 *)(qp + t * 64 + half * 32 + 16);
      }
      qf.f[t][0] = a0.x; qf.f[t][1] = a0.y; qf.f[t][2] = a0.z; qf.f[t][3] = a0.w;
      qf.f[t][4] = a1.x; qf.f[t][5] = a1.y; qf.f[t][6] = a1.z; qf.f[t][7] = a1.w;
    }
  } else {
#pragma unroll
    for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
      union {
        uint4 u;
        bf16x8_t v;
      } a;
      a.u = uint4{0u, 0u, 0u, 0u};
      if (active) {
        if constexpr (IN == SPB_BF16) {
          a.u = *(const uint4 *)((const uint16_t *)p.q + ((size_t)x * p.hq + h) * D + t * 16 + half * 8);
        } else {
          const float4 *src = (const float4 *)((const float *)p.q + ((size_t)x * p.hq + h) * D + t * 16 + half * 8);
          float4 b0 = src[0], b1 = src[1];
          a.u.x = f2bf(b0.x) | (f2bf(b0.y) << 16);
          a.u.y = f2bf(b0.z) | (f2bf(b0.w) << 16);
          a.u.z = f2bf(b1.x) | (f2bf(b1.y) << 16);
          a.u.w = f2bf(b1.z) | (f2bf(b1.w) << 16);
        }
      }
      qf.f[t] = a.v;
    }
  }

  RowState st{kNegInf, 0.f};
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{0.f};

  // content phase: chunks aligned to the content start
  for (int c = 0; c < tile.ncc; ++c) {
    __syncthreads();
    stage_chunk<D, G, IN>(p, kvh, tile.seg + c * kChunk, Ks, Vt);
    __syncthreads();
    uint64_t mask = range_mask(row.cvis - c * kChunk);
    if (__ballot(mask != 0ull)) chunk_step<D, G, IN>(Ks, Vt, qf, mask, p.sc, st, o);
  }
  // branch phase: chunks aligned to each branch start
  for (int b = tile.b_lo; b < tile.b_hi; ++b) {
    const SpbBranch br = p.branches[b];
    if (br.start + br.E <= sub0 || br.start >= sub0 + sub_n) continue;
    const int last = min(br.start + br.E, sub0 + sub_n) - 1 - br.start;
    const bool mine = row.br == br.start;
    for (int c = 0; c * kChunk <= last; ++c) {
      __syncthreads();
      stage_chunk<D, G, IN>(p, kvh, br.start + c * kChunk, Ks, Vt);
      __syncthreads();
      uint64_t mask = 0ull;
      if (mine) {
        const int lo = c * kChunk;
        mask = range_mask(min(row.e + 1, row.L) - lo);
#pragma unroll
        for (int i = 0; i < kMaxDepth; ++i) {
          int a = anc_of(row, i) - lo;
          if (i < row.depth && a >= 0 && a < kChunk) mask |= 1ull << a;
        }
      }
      if (__ballot(mask != 0ull)) chunk_step<D, G, IN>(Ks, Vt, qf, mask, p.sc, st, o);
    }
  }

  // normalise and store: lane holds d = db*32 + (r/4)*8 + half*4 + r%4
  float l = st.l + __shfl_xor(st.l, 32);
  float inv = p.s_v / l;
  if (active) {
    if constexpr (OUT == SPB_F32) {
      float *op = (float *)p.o + ((size_t)x * p.hq + h) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          float4 v = {o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
          *(float4 *)(op + db * 32 + g * 8 + half * 4) = v;
        }
    } else {
      uint16_t *op = (uint16_t *)p.o + ((size_t)x * p.hq + h) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          uint2 v;
          v.x = f2bf(o[db][4 * g] * inv) | (f2bf(o[db][4 * g + 1] * inv) << 16);
          v.y = f2bf(o[db][4 * g + 2] * inv) | (f2bf(o[db][4 * g + 3] * inv) << 16);
          *(uint2 *)(op + db * 32 + g * 8 + half * 4) = v;
        }
    }
  }
}

template <int D, int G, int IN, int OUT>
int launch_t(const AttnLaunch &a, hipStream_t s) {
  using C = Cfg<D, G, IN>;
  AttnParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o;
  p.hq = a.hq; p.hkv = a.hkv; p.n_tokens = a.n_tokens;
  p.sc = a.scale * kLog2e * a.s_q * a.s_k;
  p.s_v = a.s_v;
  p.rows = (const SpbRow *)a.rows;
  p.tiles = (const SpbTile *)a.tiles;
  p.branches = (const SpbBranch *)a.branches;
  long long items = (long long)a.n_tiles * C::SPLITS * a.hkv;
  if (items > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL((branch_attention_kernel<D, G, IN, OUT>), dim3((unsigned)items), dim3(C::NT), 0, s, p);
  return (int)hipGetLastError();
}

template <int D, int G>
int launch_dtypes(const AttnLaunch &a, hipStream_t s) {
  if (a.in_dtype == SPB_BF16)
    return a.out_dtype == SPB_F32 ? launch_t<D, G, SPB_BF16, SPB_F32>(a, s) : launch_t<D, G, SPB_BF16, SPB_BF16>(a, s);
  if (a.in_dtype == SPB_F32)
    return a.out_dtype == SPB_F32 ? launch_t<D, G, SPB_F32, SPB_F32>(a, s) : launch_t<D, G, SPB_F32, SPB_BF16>(a, s);
  if constexpr (D == 128)
    return a.out_dtype == SPB_F32 ? launch_t<D, G, SPB_FP8_E4M3, SPB_F32>(a, s)
                                  : launch_t<D, G, SPB_FP8_E4M3, SPB_BF16>(a, s);
  return (int)hipErrorInvalidValue;
}

}  // namespace

int launch_attention(const AttnLaunch &a, void *stream) {
  hipStream_t s = (hipStream_t)stream;
  int g = a.hq / a.hkv;
  if (a.head_dim == 128) {
    if (g == 1) return launch_dtypes<128, 1>(a, s);
    if (g == 2) return launch_dtypes<128, 2>(a, s);
    if (g == 4) return launch_dtypes<128, 4>(a, s);
  } else if (a.head_dim == 64) {
    if (g == 1) return launch_dtypes<64, 1>(a, s);
    if (g == 2) return launch_dtypes<64, 2>(a, s);
    if (g == 4) return launch_dtypes<64, 4>(a, s);
  }
  return (int)hipErrorInvalidValue;
}

const char *hip_error_string(int err) { return hipGetErrorString((hipError_t)err); }

}  // namespace spb
