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
// Keys are visited as a list of chunks built per work item: content chunks of
// 64 keys aligned to the content start, then for each branch that meets the
// work item's rows, chunks of 32 keys aligned to the branch start (template
// rows, then option-trie nodes).  Each chunk is staged row-major in LDS (K and
// V, rows padded against bank conflicts), double-buffered, loaded into
// registers one chunk ahead:
//   S^T = K Q^T      (MFMA 32x32x16 bf16, or 32x32x64 OCP e4m3 for fp8 Q/K)
//   online softmax   (each lane owns one query; f32, base-2 exponent)
//   O^T += V^T P^T   (MFMA 32x32x16 bf16 with P in bf16; the V^T operand is
//                     read from row-major V with the LDS transpose read)
//
// Batch invariance: a row sees its content keys in 64-key chunks aligned to
// its content start and its branch keys in 32-key chunks aligned to its branch
// start.  Slot i of a chunk always holds chunk-relative key i, every masked
// slot contributes an exact zero and leaves the running max unchanged
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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kMaxChunks = kMaxTileChunks;  // chunk-list capacity per work item (checked on the host)

__device__ inline uint32_t pack_bf16(float a, float b) {  // round to nearest even
  bf16x2_t v = __builtin_convertvector(f32x2{a, b}, bf16x2_t);
  return *(uint32_t *)&v;
}

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
  static constexpr bool FP8 = IN == SPB_FP8_E4M3;
  static constexpr int RW = G == 4 ? 2 : 4;   // 32-row groups per work item
  static constexpr int NW = RW * G;           // waves
  static constexpr int NT = NW * 64;
  static constexpr int ROWS = 32 * RW;
  static constexpr int SPLITS = 128 / ROWS;   // work items per 128-row tile
  static constexpr int KROWB = FP8 ? D : 2 * D;  // bytes per staged K row
  static constexpr int KCH = KROWB / 16;         // 16-byte chunks per K row
  static constexpr int VCH = 2 * D / 16;         // V is staged as bf16
  static constexpr int KPT = (64 * KCH + NT - 1) / NT;  // K units per thread (64-key chunk)
  static constexpr int VPT = (64 * VCH + NT - 1) / NT;
  // LDS row pitches (bytes).  K: +16 so the 16 rows a quarter-wave reads at
  // one column rotate through all banks.  V: +64 so the 4 rows of one
  // transpose read fall in disjoint quarters of the banks.
  static constexpr int KPITCH = KROWB + 16;
  static constexpr int VPITCH = 2 * D + 64;
};

template <int D, int IN>
struct QFrag {
  static constexpr int STEPS = IN == SPB_FP8_E4M3 ? D / 64 : D / 16;
  typename std::conditional<IN == SPB_FP8_E4M3, i32x8, bf16x8_t>::type f[STEPS];
};

template <int D, int G, int IN>
struct Stage {  // one chunk's K and V units held by this thread
  u32x4 k[Cfg<D, G, IN>::KPT];
  u32x4 v[Cfg<D, G, IN>::VPT];
};

// Global -> registers: rows key0 .. key0 + nrows of K and V for KV head kvh.
template <int D, int G, int IN>
__device__ inline void stage_load(Stage<D, G, IN> &st, const AttnParams &p, int kvh, int key0, int nrows) {
  using C = Cfg<D, G, IN>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::KPT; ++i) {
    const int u = tid + i * C::NT;
    const int r = u / C::KCH, c = u % C::KCH;
    const int y = key0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r < nrows && y < p.n_tokens) {
      const size_t row = (size_t)y * p.hkv + kvh;
      if constexpr (IN == SPB_FP8_E4M3) {
        val = *(const u32x4 *)((const unsigned char *)p.k + row * D + c * 16);
      } else if constexpr (IN == SPB_BF16) {
        val = *(const u32x4 *)((const uint16_t *)p.k + row * D + c * 8);
      } else {
        const float *src = (const float *)p.k + row * D + c * 8;
        u32x4 a = *(const u32x4 *)src, b = *(const u32x4 *)(src + 4);
        val = u32x4{pack_bf16(__uint_as_float(a.x), __uint_as_float(a.y)),
                    pack_bf16(__uint_as_float(a.z), __uint_as_float(a.w)),
                    pack_bf16(__uint_as_float(b.x), __uint_as_float(b.y)),
                    pack_bf16(__uint_as_float(b.z), __uint_as_float(b.w))};
      }
    }
    st.k[i] = val;
  }
#pragma unroll
  for (int i = 0; i < C::VPT; ++i) {
    const int u = tid + i * C::NT;
    const int r = u / C::VCH, c = u % C::VCH;
    const int y = key0 + r;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r < nrows && y < p.n_tokens) {
      const size_t row = (size_t)y * p.hkv + kvh;
      if constexpr (IN == SPB_FP8_E4M3) {
        u32x2 w = *(const u32x2 *)((const unsigned char *)p.v + row * D + c * 8);
        val = u32x4{e4m3_to_bf(w.x & 0xFFu) | (e4m3_to_bf((w.x >> 8) & 0xFFu) << 16),
                    e4m3_to_bf((w.x >> 16) & 0xFFu) | (e4m3_to_bf(w.x >> 24) << 16),
                    e4m3_to_bf(w.y & 0xFFu) | (e4m3_to_bf((w.y >> 8) & 0xFFu) << 16),
                    e4m3_to_bf((w.y >> 16) & 0xFFu) | (e4m3_to_bf(w.y >> 24) << 16)};
      } else if constexpr (IN == SPB_BF16) {
        val = *(const u32x4 *)((const uint16_t *)p.v + row * D + c * 8);
      } else {
        const float *src = (const float *)p.v + row * D + c * 8;
        u32x4 a = *(const u32x4 *)src, b = *(const u32x4 *)(src + 4);
        val = u32x4{pack_bf16(__uint_as_float(a.x), __uint_as_float(a.y)),
                    pack_bf16(__uint_as_float(a.z), __uint_as_float(a.w)),
                    pack_bf16(__uint_as_float(b.x), __uint_as_float(b.y)),
                    pack_bf16(__uint_as_float(b.z), __uint_as_float(b.w))};
      }
    }
    st.v[i] = val;
  }
}

// registers -> LDS buffers (swizzled)
template <int D, int G, int IN>
__device__ inline void stage_store(const Stage<D, G, IN> &st, char *Ks, char *Vs, int nrows) {
  using C = Cfg<D, G, IN>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::KPT; ++i) {
    const int u = tid + i * C::NT;
    const int r = u / C::KCH, c = u % C::KCH;
    if (r < nrows) *(u32x4 *)(Ks + r * C::KPITCH + c * 16) = st.k[i];
  }
#pragma unroll
  for (int i = 0; i < C::VPT; ++i) {
    const int u = tid + i * C::NT;
    const int r = u / C::VCH, c = u % C::VCH;
    if (r < nrows) *(u32x4 *)(Vs + r * C::VPITCH + c * 16) = st.v[i];
  }
}

__device__ inline void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct RowState {
  float m;  // running max of the scaled (base-2) logits
  float l;  // this lane's partial row sum
};

// Which keys of a chunk this lane's query sees.  Register r of block kb
// holds chunk key kb*32 + (r/4)*8 + half*4 + r%4; with the lane's half folded
// into the thresholds, every test compares a compile-time slot offset
// kb*32 + (r/4)*8 + r%4 against per-lane values:
//   visible = slot < thr  ||  slot is one of anc[0..3]  (ANC only)
struct Vis {
  int thr;        // keys [0, thr + 4*half) visible
  int anc[kMaxDepth];  // option-trie ancestor keys minus 4*half, or -1000
};

// One chunk of NKB*32 keys.  MODE 0: every key visible to every lane;
// 1: prefix test only; 2: prefix test and ancestor keys.
template <int D, int G, int IN, int NKB, int MODE>
__device__ inline void chunk_step(const char *Ks, const char *Vs, const QFrag<D, IN> &qf, const Vis &vis,
                                  float sc, RowState &st, f32x16 (&o)[D / 32]) {
  using C = Cfg<D, G, IN>;
  const int lane = threadIdx.x & 63;
  const int qi = lane & 31, half = lane >> 5;
  f32x16 s[NKB];
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
    asm volatile("" ::: "memory");  // keeps each block's LDS reads next to its MFMAs
    s[kb] = f32x16{0.f};
    const int r = kb * 32 + qi;
    if constexpr (C::FP8) {
#pragma unroll
      for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
        const char *src = Ks + r * C::KPITCH + t * 64 + half * 32;
        u32x4 a0 = *(const u32x4 *)src, a1 = *(const u32x4 *)(src + 16);
        i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf.f[t], s[kb], 0, 0, 0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
        u32x4 u = *(const u32x4 *)(Ks + r * C::KPITCH + t * 32 + half * 16);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(bf16x8_t *)&u, qf.f[t], s[kb], 0, 0, 0);
      }
    }
  }
  // online softmax: lane owns query qi; register r of block kb holds key
  // kb*32 + (r/4)*8 + half*4 + r%4
  if constexpr (MODE != 0) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int slot = kb * 32 + (r >> 2) * 8 + (r & 3);
        bool v = slot < vis.thr;
        if constexpr (MODE == 2) {
#pragma unroll
          for (int a = 0; a < kMaxDepth; ++a) v = v || slot == vis.anc[a];
        }
        s[kb][r] = v ? s[kb][r] : kNegInf;
      }
  }
  float mloc = kNegInf;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[kb][r]);
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  const float mnew = fmaxf(st.m, mloc * sc);
  const bool none = mnew == kNegInf;  // nothing visible yet: p = 0, alpha = 1
  const float alpha = none ? 1.f : __builtin_amdgcn_exp2f(st.m - mnew);
  const float negm = none ? 0.f : -mnew;
  uint32_t pk[NKB][8];
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], sc, negm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r + 1], sc, negm));
      lsum += p0;
      lsum += p1;
      pk[kb][r >> 1] = pack_bf16(p0, p1);
    }
  st.l = st.l * alpha + lsum;
  st.m = mnew;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
  }
  // O^T += V^T P^T.  k-step j covers keys 16j + half*4 + {0..3} and
  // 16j + 8 + half*4 + {0..3}: the P^T operand is registers 8(j%2) .. +8 of
  // block j/2, the V^T operand two transpose reads of 4 rows each.
  const int g = qi >> 4, l16 = lane & 15;
#pragma unroll
  for (int j = 0; j < 2 * NKB; ++j) {
    asm volatile("" ::: "memory");
    const int kb = j >> 1, rb = (j & 1) * 4;
    union {
      uint32_t u[4];
      bf16x8_t v;
    } b;
    b.u[0] = pk[kb][rb]; b.u[1] = pk[kb][rb + 1]; b.u[2] = pk[kb][rb + 2]; b.u[3] = pk[kb][rb + 3];
    // lane reads 4 bf16 at row 16j + half*4 + l16/4 (and +8), column
    // db*32 + g*16 + 4*(l16%4); the transpose hands it column db*32 + qi
    const char *vrow = Vs + (16 * j + half * 4 + (l16 >> 2)) * C::VPITCH + (g * 16 + 4 * (l16 & 3)) * 2;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      union {
        i16x4 h[2];
        bf16x8_t v;
      } a;
      a.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vrow + db * 64));
      a.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vrow + 8 * C::VPITCH + db * 64));
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, o[db], 0, 0, 0);
    }
  }
}

// ----------------------------------------------------------------- kernel

template <int D, int G, int IN, int OUT>
__global__ __launch_bounds__((Cfg<D, G, IN>::NT)) void branch_attention_kernel(AttnParams p) {
  using C = Cfg<D, G, IN>;
  __shared__ __attribute__((aligned(16))) char Ks[2][64 * C::KPITCH];
  __shared__ __attribute__((aligned(16))) char Vs[2][64 * C::VPITCH];
  __shared__ int2 chunks[kMaxChunks];  // (key0, info): info < 0 content chunk -1-c; else branch << 10 | c
  __shared__ int n_chunks_s;

  const int w = blockIdx.x;
  const int kvh = w % p.hkv;
  const int rest = w / p.hkv;
  const int split = rest % C::SPLITS;
  const SpbTile tile = p.tiles[rest / C::SPLITS];
  const int sub0 = tile.row0 + split * C::ROWS;
  const int sub_n = min(C::ROWS, tile.row0 + tile.nrows - sub0);
  if (sub_n <= 0) return;  // uniform over the work group

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rw = wave / G, gh = wave % G;
  const int h = kvh * G + gh;
  const int qi = lane & 31, half = lane >> 5;
  const int local = rw * 32 + qi;
  const bool active = local < sub_n;
  const int x = sub0 + local;

  // chunk list (wave 0): content chunks, then the chunks of each branch that
  // meets rows [sub0, sub0 + sub_n)
  if (wave == 0) {
    for (int c = lane; c < tile.ncc && c < kMaxChunks; c += 64) chunks[c] = int2{tile.seg + c * kChunk, -1 - c};
    int n = tile.ncc;
    for (int b0 = tile.b_lo; b0 < tile.b_hi; b0 += 64) {
      const int b = b0 + lane;
      int cnt = 0, start = 0;
      if (b < tile.b_hi) {
        const SpbBranch br = p.branches[b];
        start = br.start;
        if (br.start + br.E > sub0 && br.start < sub0 + sub_n) {
          const int last = min(br.start + br.E, sub0 + sub_n) - 1 - br.start;
          cnt = last / kBranchChunk + 1;
        }
      }
      int incl = cnt;  // inclusive prefix sum over the wave
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int t = __shfl_up(incl, off);
        if (lane >= off) incl += t;
      }
      const int base = n + incl - cnt;
      for (int c = 0; c < cnt; ++c)
        if (base + c < kMaxChunks) chunks[base + c] = int2{start + c * kBranchChunk, (b << 10) | c};
      n += __shfl(incl, 63);
    }
    if (lane == 0) n_chunks_s = n < kMaxChunks ? n : kMaxChunks;
  }

  SpbRow row;
  if (active) {
    row = p.rows[x];
  } else {
    row.cvis = 0; row.seg = 0; row.br = -1; row.e = 0; row.L = 0; row.depth = 0; row.anc01 = 0; row.anc23 = 0;
  }

  QFrag<D, IN> qf;
  if constexpr (C::FP8) {
    const unsigned char *qp = (const unsigned char *)p.q + ((size_t)x * p.hq + h) * D;
#pragma unroll
    for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
      u32x4 a0 = {0u, 0u, 0u, 0u}, a1 = {0u, 0u, 0u, 0u};
      if (active) {
        a0 = *(const u32x4 *)(qp + t * 64 + half * 32);
        a1 = *(const u32x4 *)(qp + t * 64 + half * 32 + 16);
      }
      qf.f[t] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
    }
  } else {
#pragma unroll
    for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
      u32x4 a = {0u, 0u, 0u, 0u};
      if (active) {
        if constexpr (IN == SPB_BF16) {
          a = *(const u32x4 *)((const uint16_t *)p.q + ((size_t)x * p.hq + h) * D + t * 16 + half * 8);
        } else {
          const float *src = (const float *)p.q + ((size_t)x * p.hq + h) * D + t * 16 + half * 8;
          u32x4 f0 = *(const u32x4 *)src, f1 = *(const u32x4 *)(src + 4);
          a = u32x4{pack_bf16(__uint_as_float(f0.x), __uint_as_float(f0.y)),
                    pack_bf16(__uint_as_float(f0.z), __uint_as_float(f0.w)),
                    pack_bf16(__uint_as_float(f1.x), __uint_as_float(f1.y)),
                    pack_bf16(__uint_as_float(f1.z), __uint_as_float(f1.w))};
        }
      }
      qf.f[t] = *(bf16x8_t *)&a;
    }
  }

  RowState st{kNegInf, 0.f};
  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{0.f};

  __syncthreads();  // chunk list ready
  const int nch = n_chunks_s;

  // Prefetch loads are issued on every trip (past the end they reload the
  // last chunk), so no branch changes the count of outstanding loads and each
  // LDS store waits only for the chunk it writes.
  auto nrows_of = [&](int i) { return chunks[i].y < 0 ? kChunk : kBranchChunk; };
  Stage<D, G, IN> stg;
  if (nch > 0) {
    stage_load<D, G, IN>(stg, p, kvh, chunks[0].x, nrows_of(0));
    stage_store<D, G, IN>(stg, Ks[0], Vs[0], nrows_of(0));
    lds_barrier();
    const int i1 = min(1, nch - 1);
    stage_load<D, G, IN>(stg, p, kvh, chunks[i1].x, nrows_of(i1));
  }

  for (int i = 0; i < nch; ++i) {
    const int buf = i & 1;
    const int2 ch = chunks[i];
    Vis vis;
#pragma unroll
    for (int a = 0; a < kMaxDepth; ++a) vis.anc[a] = -1000;
    if (ch.y < 0) {  // content chunk c: keys [c*64, c*64 + 64) of the content
      const int c = -1 - ch.y;
      const int nvis = row.cvis - c * kChunk;
      vis.thr = nvis - 4 * half;
      if (__ballot(nvis > 0)) {
        if (__ballot(nvis < kChunk))
          chunk_step<D, G, IN, 2, 1>(Ks[buf], Vs[buf], qf, vis, p.sc, st, o);
        else
          chunk_step<D, G, IN, 2, 0>(Ks[buf], Vs[buf], qf, vis, p.sc, st, o);
      }
    } else {  // branch chunk c: extended keys [c*32, c*32 + 32) of the branch
      const int c = ch.y & 1023;
      const int lo = c * kBranchChunk;
      const bool mine = row.br == ch.x - lo;
      int nt = mine ? min(min(row.e + 1, row.L) - lo, kBranchChunk) : 0;
      bool any = nt > 0;
      const bool node = mine && row.depth > 0;
      if (node) {
#pragma unroll
        for (int a = 0; a < kMaxDepth; ++a) {
          const int e = anc_of(row, a) - lo;
          if (a < row.depth && e >= 0 && e < kBranchChunk) {
            vis.anc[a] = e - 4 * half;
            any = true;
          }
        }
      }
      vis.thr = nt - 4 * half;
      if (__ballot(any)) {
        if (__ballot(node))
          chunk_step<D, G, IN, 1, 2>(Ks[buf], Vs[buf], qf, vis, p.sc, st, o);
        else
          chunk_step<D, G, IN, 1, 1>(Ks[buf], Vs[buf], qf, vis, p.sc, st, o);
      }
    }
    const int i1 = min(i + 1, nch - 1), i2 = min(i + 2, nch - 1);
    stage_store<D, G, IN>(stg, Ks[buf ^ 1], Vs[buf ^ 1], nrows_of(i1));
    lds_barrier();
    stage_load<D, G, IN>(stg, p, kvh, chunks[i2].x, nrows_of(i2));
  }

  // normalise and store: lane holds d = db*32 + (r/4)*8 + half*4 + r%4
  const float l = st.l + __shfl_xor(st.l, 32);
  const float inv = p.s_v / l;
  if (active) {
    if constexpr (OUT == SPB_F32) {
      float *op = (float *)p.o + ((size_t)x * p.hq + h) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          float4 v = {o[db][4 * gg] * inv, o[db][4 * gg + 1] * inv, o[db][4 * gg + 2] * inv, o[db][4 * gg + 3] * inv};
          *(float4 *)(op + db * 32 + gg * 8 + half * 4) = v;
        }
    } else {
      uint16_t *op = (uint16_t *)p.o + ((size_t)x * p.hq + h) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          u32x2 v = {pack_bf16(o[db][4 * gg] * inv, o[db][4 * gg + 1] * inv),
                     pack_bf16(o[db][4 * gg + 2] * inv, o[db][4 * gg + 3] * inv)};
          *(u32x2 *)(op + db * 32 + gg * 8 + half * 4) = v;
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
