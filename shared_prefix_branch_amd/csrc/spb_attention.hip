// spb_attention.hip -- branch-masked packed attention for gfx950 (CDNA4).
//
// Computes, for every packed row x and query head h, softmax attention over
// the keys on x's root path only: its own content (causal for content rows,
// all of it for branch rows), its own template prefix and its own option-trie
// ancestors.  So each content is read once and all of its questions ride in
// the same pass as branches [PyPI "spinf-serve 0.1.1", "What it does"], with answers
// equal to running each content + question as its own prompt [PyPI, "Speed
// and scale"].
//
// Work item: up to 128 consecutive rows of one 128-row tile (rows of one
// segment) and one KV head.  Keys are visited as a list of chunks per work
// item: content chunks of 64 keys aligned to the content start, then for each
// branch that meets the work item's rows, chunks of 32 keys aligned to the
// branch start (template rows, then option-trie nodes).  Per chunk:
//   S^T = K Q^T      (MFMA 32x32x16 bf16, or 32x32x64 OCP e4m3 for fp8 Q/K)
//   online softmax   (each lane owns one query; f32, base-2 exponent, the
//                     exponent reference moved lazily)
//   O^T += V^T P^T   (MFMA 32x32x16 bf16 with P in bf16; the V^T operand is
//                     read from row-major V with the LDS transpose read)
//
// Two kernels share that chunk step:
//  * bf16 inputs (dma kernel): four waves, two work groups per CU.  The work
//    item's chunk list comes from the pass metadata (items of 32, 64 or 128
//    rows).  K and V rows are copied straight from global memory into a
//    two-slot LDS ring (XOR-swizzled rows, no staging registers), one chunk
//    ahead; every LDS fragment read is issued ahead of the MFMAs that use it.
//    A wave owns 32 query rows of one query head (two heads for d = 64,
//    sharing every K/V fragment read and visibility test).  Q rows and bf16
//    O rows also pass through LDS, so that their global accesses are whole
//    16-byte pieces of consecutive rows rather than one row per lane pair.
//  * f32 / fp8 inputs (staged kernel): K and V pass through registers, where
//    f32 is rounded to bf16 and e4m3 V is widened to bf16, into a
//    double-buffered padded LDS layout; one head per wave; the chunk list is
//    built in the kernel from the tile and branch tables.
// Both run one chunk step per chunk (a single instance in the loop, so the
// O accumulators keep their registers).
//
// Batch invariance: a row sees its content keys in 64-key chunks aligned to
// its content start and its branch keys in 32-key chunks aligned to its branch
// start.  Slot i of a chunk always holds chunk-relative key i, every masked
// slot contributes an exact zero, the exponent reference follows only the
// row's own chunk maxima, and every per-row sum runs in a fixed slot order.
// So a row's bits depend on its own root path only, not on where its input
// was packed.
#define SPB_HD __host__ __device__
#include "spb_meta.h"
#include "spb_launch.h"
#include "spb_dev.h"
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
  const SpbItem *items;      // the item table of the kernel's row granularity
  const SpbChunk *bchunks;   // stem and branch chunks of the items
  int n_work;                // items x KV heads
};

template <int D, int IN>
struct QFrag {
  static constexpr int STEPS = IN == SPB_FP8_E4M3 ? D / 64 : D / 16;
  typename std::conditional<IN == SPB_FP8_E4M3, i32x8, bf16x8_t>::type f[STEPS];
};

// Per-lane LDS byte offsets of the wave's fragment reads, relative to a K
// block (32 key rows) and to a V k-step (16 key rows).  K: step t, piece pc
// (bf16: one 16-byte piece; e4m3: two).  V: d-block db, first of the two
// transpose reads (the second is 8 rows further).
template <int D, int IN>
struct FragOffsets {
  static constexpr int STEPS = QFrag<D, IN>::STEPS;
  static constexpr int NPC = IN == SPB_FP8_E4M3 ? 2 : 1;
  uint32_t k[STEPS][NPC];
  uint32_t v[D / 32];
};

struct RowState {
  float m;  // exponent reference (scaled, base 2)
  float l;  // this lane's partial row sum
};

// Which keys of a 32-key block this lane's query sees.  Register r of a block
// holds block key (r/4)*8 + half*4 + r%4; with the lane's half folded into the
// per-lane values, every test compares a compile-time slot (r/4)*8 + r%4:
//   visible = slot < thr  ||  slot is one of anc[0..3]
struct Vis {
  int thr;             // block keys [0, thr + 4*half) visible
  int anc[kMaxDepth];  // option-trie ancestor keys minus 4*half, or -1000
};

template <int ANC>
__device__ __attribute__((always_inline)) inline void mask_block(f32x16 &s, const Vis &vis) {
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int slot = (r >> 2) * 8 + (r & 3);
    bool v = slot < vis.thr;
    if constexpr (ANC) {
#pragma unroll
      for (int a = 0; a < kMaxDepth; ++a) v = v || slot == vis.anc[a];
    }
    s[r] = v ? s[r] : kNegInf;
  }
}

// max over the lane pair (i, i ^ 32): v_permlane32_swap hands each lane its
// partner's value without an LDS round trip
__device__ __attribute__((always_inline)) inline float half_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Online softmax over one chunk -- one 32-key block, or two when `two`
// (runtime, uniform over the wave) -- for one head, with a lazily moved
// reference: the row's exponent reference m changes only when the chunk's max
// exceeds it by more than kLazy (log2 units) -- always on the first visible
// chunk, where O and l are still zero -- so p = 2^(s - m) stays at most
// 2^kLazy and O is rescaled (by 2^(m_old - m_new)) only on those rare moves.
// The quotient O / l is the same softmax for any reference.  Returns P as
// bf16 pairs; the row sum runs over block 0 then block 1, registers in order.
constexpr float kLazy = 8.f;

template <int D>
__device__ __attribute__((always_inline)) inline void softmax_chunk(const f32x16 &s0, const f32x16 &s1, bool two,
                                                                     float sc, RowState &st, f32x16 (&o)[D / 32],
                                                                     uint32_t (&pk)[2][8]) {
  float mloc = kNegInf;
#pragma unroll
  for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s0[r]);
  if (two) {
#pragma unroll
    for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s1[r]);
  }
  mloc = half_max(mloc) * sc;
  const bool first = st.m == kNegInf;
  const bool move = !first && mloc > st.m + kLazy;
  const float mnew = (first || move) ? mloc : st.m;
  const float negm = mnew == kNegInf ? 0.f : -mnew;
  float lsum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; r += 2) {
    const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], sc, negm));
    const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r + 1], sc, negm));
    lsum += p0;
    lsum += p1;
    pk[0][r >> 1] = pack_bf16(p0, p1);
  }
  if (two) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], sc, negm));
      const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r + 1], sc, negm));
      lsum += p0;
      lsum += p1;
      pk[1][r >> 1] = pack_bf16(p0, p1);
    }
  }
  if (__ballot(move)) {
    const float alpha = move ? __builtin_amdgcn_exp2f(st.m - mnew) : 1.f;
    st.l *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
  }
  st.l += lsum;
  st.m = mnew;
}

// S^T of one 32-key block for HPW heads: each K fragment read from LDS feeds
// one MFMA per head.  Kblk: the block's first key row in LDS.
template <int D, int IN, int HPW>
__device__ __attribute__((always_inline)) inline void qk_block(const char *Kblk, const FragOffsets<D, IN> &fo,
                                                               const QFrag<D, IN> (&qf)[HPW], f32x16 (&s)[HPW]) {
  constexpr int STEPS = QFrag<D, IN>::STEPS;
#pragma unroll
  for (int j = 0; j < HPW; ++j) s[j] = f32x16{0.f};
  if constexpr (IN == SPB_FP8_E4M3) {
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      asm volatile("" ::: "memory");
      u32x4 a0 = *(const u32x4 *)(Kblk + fo.k[t][0]), a1 = *(const u32x4 *)(Kblk + fo.k[t][1]);
      i32x8 a = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
      for (int j = 0; j < HPW; ++j)
        s[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[j].f[t], s[j], 0, 0, 0, 0, 0, 0);
    }
  } else {
    constexpr int GRP = STEPS < 4 ? STEPS : 4;
#pragma unroll
    for (int t0 = 0; t0 < STEPS; t0 += GRP) {
      asm volatile("" ::: "memory");  // keeps each group's LDS reads next to its MFMAs
      u32x4 a[GRP];
#pragma unroll
      for (int t = 0; t < GRP; ++t) a[t] = *(const u32x4 *)(Kblk + fo.k[t0 + t][0]);
#pragma unroll
      for (int t = 0; t < GRP; ++t)
#pragma unroll
        for (int j = 0; j < HPW; ++j)
          s[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t *)&a[t], qf[j].f[t0 + t], s[j], 0, 0, 0);
    }
  }
}

// O^T += V^T P^T over one 32-key block (two k-steps of 16 keys).
// k-step j covers block keys 16(j%2) + half*4 + {0..3} and +8: the P^T
// operand is registers 8(j%2) .. +8 of the block, the V^T operand two
// transpose reads of 4 rows each, shared by the HPW heads.  VSTRIDE: bytes
// per V row in LDS.
template <int D, int IN, int HPW, int VSTRIDE>
__device__ __attribute__((always_inline)) inline void pv_block(const char *Vblk, const FragOffsets<D, IN> &fo,
                                                               const uint32_t (&pk)[HPW][8],
                                                               f32x16 (&o)[HPW][D / 32]) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    asm volatile("" ::: "memory");  // keeps each k-step's transpose reads next to its MFMAs
    const int rb = jj * 4;
    const char *vstep = Vblk + 16 * jj * VSTRIDE;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      union {
        i16x4 h[2];
        bf16x8_t v;
      } a;
      a.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vstep + fo.v[db]));
      a.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vstep + fo.v[db] + 8 * VSTRIDE));
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        union {
          uint32_t u[4];
          bf16x8_t v;
        } b;
        b.u[0] = pk[h][rb]; b.u[1] = pk[h][rb + 1]; b.u[2] = pk[h][rb + 2]; b.u[3] = pk[h][rb + 3];
        o[h][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a.v, b.v, o[h][db], 0, 0, 0);
      }
    }
  }
}

// bf16 with K and V in 16-byte-swizzled LDS rows of ROWB bytes: the chunk's
// S^T (one or two 32-key blocks) and its O^T update with every LDS read
// issued ahead of the MFMAs that use it.  K fragments go in groups of four
// 16-element steps, the next group read while the current one multiplies; V^T
// fragments go one 16-key k-step ahead, the first k-step read before the
// softmax (read_v_step).  Each output element accumulates in the same order
// as in qk_block / pv_block.
template <int D>
struct VStep {
  bf16x8_t v[D / 32];
};

template <int D, int ROWB>
__device__ __attribute__((always_inline)) inline void read_k_group(const char *Kb, const FragOffsets<D, SPB_BF16> &fo,
                                                                   int gi, u32x4 (&a)[4]) {
  constexpr int NG = D / 64;  // groups per 32-key block
  const char *base = Kb + (gi / NG) * 32 * ROWB;
#pragma unroll
  for (int t = 0; t < 4; ++t) a[t] = *(const u32x4 *)(base + fo.k[(gi % NG) * 4 + t][0]);
}

template <int D, int HPW, int ROWB>
__device__ __attribute__((always_inline)) inline void qk_chunk(const char *Kb, const FragOffsets<D, SPB_BF16> &fo,
                                                               const QFrag<D, SPB_BF16> (&qf)[HPW], f32x16 (&s0)[HPW],
                                                               f32x16 (&s1)[HPW], bool two) {
  constexpr int NG = D / 64;
#pragma unroll
  for (int j = 0; j < HPW; ++j) s0[j] = f32x16{0.f};
  if (two) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) s1[j] = f32x16{0.f};
  }
  u32x4 a[2][4];
  read_k_group<D, ROWB>(Kb, fo, 0, a[0]);
#pragma unroll
  for (int gi = 0; gi < 2 * NG; ++gi) {
    if (gi == NG && !two) break;
    asm volatile("" ::: "memory");  // reads of group gi + 2 stay behind this point
    if (gi + 1 < NG || (gi + 1 < 2 * NG && two)) read_k_group<D, ROWB>(Kb, fo, gi + 1, a[(gi + 1) & 1]);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        const bf16x8_t av = *(const bf16x8_t *)&a[gi & 1][t];
        if (gi < NG)
          s0[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[j].f[(gi % NG) * 4 + t], s0[j], 0, 0, 0);
        else
          s1[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[j].f[(gi % NG) * 4 + t], s1[j], 0, 0, 0);
      }
  }
}

// V^T operands of k-step ks (keys 16 ks .. 16 ks + 16 of the chunk)
template <int D, int ROWB, typename FO>
__device__ __attribute__((always_inline)) inline void read_v_step(const char *Vb, const FO &fo, int ks, VStep<D> &f) {
  const char *vstep = Vb + 16 * ks * ROWB;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    union {
      i16x4 h[2];
      bf16x8_t v;
    } a;
    a.h[0] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vstep + fo.v[db]));
    a.h[1] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(vstep + fo.v[db] + 8 * ROWB));
    f.v[db] = a.v;
  }
}

template <int D, int HPW, int ROWB, typename FO>
__device__ __attribute__((always_inline)) inline void pv_chunk(const char *Vb, const FO &fo,
                                                               const uint32_t (&pk)[HPW][2][8],
                                                               f32x16 (&o)[HPW][D / 32], bool two,
                                                               const VStep<D> &first) {
  VStep<D> f[2];
  f[0] = first;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (ks == 2 && !two) break;
    asm volatile("" ::: "memory");  // reads of k-step ks + 2 stay behind this point
    if (ks + 1 < 2 || (ks + 1 < 4 && two)) read_v_step<D, ROWB>(Vb, fo, ks + 1, f[(ks + 1) & 1]);
    const int blk = ks >> 1, rb = (ks & 1) * 4;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        union {
          uint32_t u[4];
          bf16x8_t v;
        } b;
        b.u[0] = pk[h][blk][rb]; b.u[1] = pk[h][blk][rb + 1]; b.u[2] = pk[h][blk][rb + 2]; b.u[3] = pk[h][blk][rb + 3];
        o[h][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[ks & 1].v[db], b.v, o[h][db], 0, 0, 0);
      }
  }
}

// Chunk list of a work item in LDS: its content chunks, then its stem and
// branch chunks from the item table.  Entry: (first key row, info, pre,
// post | nvis << 24); info < 0 for content chunk -1 - info, else the table's.
__device__ inline void load_chunk_list(const AttnParams &p, const SpbItem &it, int4 *chunks, int tid, int nt) {
  const int nch = it.ncc + it.bn;
  for (int i = tid; i < nch; i += nt) {
    if (i < it.ncc) {
      chunks[i] = int4{it.seg + i * kChunk, -1 - i, 0, 0};
    } else {
      const SpbChunk c = p.bchunks[it.boff + i - it.ncc];
      chunks[i] = int4{c.key0, c.info, c.pre, c.post_nvis};
    }
  }
}

// The row a lane works on; lanes past the item's rows get a row that sees
// nothing (no content, no stem, no branch).
__device__ inline SpbRow load_row(const AttnParams &p, int x, bool active) {
  if (active) return p.rows[x];
  SpbRow r{};
  r.br = -1;
  r.spre = -1;
  return r;
}

// Q fragments of row x, query head h (zeros for inactive lanes).
template <int D, int IN>
__device__ inline void load_q(QFrag<D, IN> &qf, const AttnParams &p, int x, int h, bool active, int half) {
  if constexpr (IN == SPB_FP8_E4M3) {
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
}

// normalise and store: lane holds d = db*32 + (r/4)*8 + half*4 + r%4
template <int D, int OUT>
__device__ inline void store_o(const AttnParams &p, int x, int h, int half, const RowState &st,
                               const f32x16 (&o)[D / 32]) {
  const float l = st.l + __shfl_xor(st.l, 32);
  const float inv = p.s_v / l;
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

// What one wave does with one chunk.  Content chunk c (keys [c*64, c*64 + 64)
// of the content) is two 32-key blocks, the second skipped when no lane sees
// past key 32; stem chunk c (tokens [c*32, c*32 + nvis) of a shared template
// stem) and branch chunk c (extended keys [c*32, c*32 + 32) of the branch)
// are one block each.  A stem row sees its own stem causally; a row whose
// path runs through a stem (its DFS number falls in the stem's interval) sees
// all of it.  A chunk is skipped by a wave none of whose lanes sees a key of
// it.  ch = (first key row, info, pre, post | nvis << 24): info < 0 for
// content chunk -1 - info, kStemChunk | stem << 10 | c for a stem chunk,
// else branch << 10 | c.  Calls ballots: every lane of the wave takes part.
struct ChunkStep {
  bool run;     // some lane sees a key of the chunk
  bool two;     // content chunk whose second block some lane sees
  bool masked;  // some lane sees only part of the chunk
  bool anc;     // some lane is an option-trie node of the chunk's branch
  Vis vis;
};

__device__ __attribute__((always_inline)) inline ChunkStep chunk_step(int4 ch, const SpbRow &row, int half) {
  int thr;  // keys of the chunk this lane sees as a prefix
  int anc[kMaxDepth];
  bool any, node = false;
#pragma unroll
  for (int a = 0; a < kMaxDepth; ++a) anc[a] = -1000;
  if (ch.y < 0) {
    thr = row.cvis - (-1 - ch.y) * kChunk;
    any = thr > 0;
  } else if (ch.y & kStemChunk) {
    const int lo = (ch.y & 1023) * kBranchChunk;
    const int nvis = (int)((uint32_t)ch.w >> 24);
    const bool own = row.br == ch.x - lo;
    const bool below = ch.z <= row.spre && row.spre < (ch.w & 0xFFFFFF);
    thr = own ? min(row.e + 1 - lo, nvis) : below ? nvis : 0;
    any = thr > 0;
  } else {
    const int c = ch.y & 1023;
    const int lo = c * kBranchChunk;
    const bool mine = row.br == ch.x - lo;
    thr = mine ? min(min(row.e + 1, row.L) - lo, kBranchChunk) : 0;
    any = thr > 0;
    node = mine && row.depth > 0;
    if (node) {
#pragma unroll
      for (int a = 0; a < kMaxDepth; ++a) {
        const int e = anc_of(row, a) - lo;
        if (a < row.depth && e >= 0 && e < kBranchChunk) {
          anc[a] = e;
          any = true;
        }
      }
    }
  }
  ChunkStep cs;
  cs.run = __ballot(any) != 0;
  cs.two = ch.y < 0 && __ballot(thr > 32) != 0;
  cs.anc = __ballot(node) != 0;
  cs.vis.thr = thr - 4 * half;
#pragma unroll
  for (int a = 0; a < kMaxDepth; ++a) cs.vis.anc[a] = anc[a] - 4 * half;
  cs.masked = cs.anc || __ballot(thr < (cs.two ? 64 : 32)) != 0;
  return cs;
}

// The chunk walk of the staged kernel: block(i, vis, two, masked, anc) runs
// chunk i -- S^T, mask, softmax, O^T update over one or two blocks -- and
// appears once in the loop, so the accumulators keep their registers;
// advance(i) hands the LDS buffers on to chunk i + 1.
template <typename Block, typename Advance>
__device__ __attribute__((always_inline)) inline void walk_chunks(const int4 *chunks, int nch, const SpbRow &row,
                                                                  int half, Block &&block, Advance &&advance) {
  for (int i = 0; i < nch; ++i) {
    const ChunkStep cs = chunk_step(chunks[i], row, half);
    if (cs.run) block(i, cs.vis, cs.two, cs.masked, cs.anc);
    advance(i);
  }
}

// S^T of one chunk for e4m3 K and Q on the fp8 MFMA (32x32x64), K in
// 16-byte-swizzled LDS rows of ROWB bytes: block 0, then block 1 when `two`,
// each over the 64-element K steps in order -- the same MFMAs in the same
// order as qk_block, so the same bits.
template <int D, int HPW, int ROWB>
__device__ __attribute__((always_inline)) inline void qk_chunk_fp8(const char *Kb,
                                                                   const FragOffsets<D, SPB_FP8_E4M3> &fo,
                                                                   const QFrag<D, SPB_FP8_E4M3> (&qf)[HPW],
                                                                   f32x16 (&s0)[HPW], f32x16 (&s1)[HPW], bool two) {
  constexpr int STEPS = QFrag<D, SPB_FP8_E4M3>::STEPS;
  u32x4 a[2][STEPS][2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    if (blk == 1 && !two) break;
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      a[blk][t][0] = *(const u32x4 *)(Kb + blk * 32 * ROWB + fo.k[t][0]);
      a[blk][t][1] = *(const u32x4 *)(Kb + blk * 32 * ROWB + fo.k[t][1]);
    }
  }
#pragma unroll
  for (int j = 0; j < HPW; ++j) s0[j] = f32x16{0.f};
  if (two) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) s1[j] = f32x16{0.f};
  }
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    if (blk == 1 && !two) break;
#pragma unroll
    for (int t = 0; t < STEPS; ++t) {
      const u32x4 a0 = a[blk][t][0], a1 = a[blk][t][1];
      const i32x8 k8 = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
#pragma unroll
      for (int j = 0; j < HPW; ++j) {
        if (blk == 0)
          s0[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k8, qf[j].f[t], s0[j], 0, 0, 0, 0, 0, 0);
        else
          s1[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(k8, qf[j].f[t], s1[j], 0, 0, 0, 0, 0, 0);
      }
    }
  }
}

// e4m3 V -> bf16 V (exact), 16 elements per thread, for the fp8 dma kernel.
__global__ __launch_bounds__(256) void widen_v_kernel(const unsigned char *v8, uint32_t *v16, long long n16) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const u32x4 w = ((const u32x4 *)v8)[i];
  uint32_t out[8];
  const uint32_t src[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    out[2 * q] = e4m3_to_bf(src[q] & 0xFFu) | (e4m3_to_bf((src[q] >> 8) & 0xFFu) << 16);
    out[2 * q + 1] = e4m3_to_bf((src[q] >> 16) & 0xFFu) | (e4m3_to_bf(src[q] >> 24) << 16);
  }
  u32x4 *dst = (u32x4 *)v16 + 2 * i;
  dst[0] = u32x4{out[0], out[1], out[2], out[3]};
  dst[1] = u32x4{out[4], out[5], out[6], out[7]};
}

// ------------------------------------------------------- bf16: dma kernel

template <int D, int G, int HPW_, int RG_, int IN_ = SPB_BF16>
struct DmaCfg {
  static constexpr int HPW = HPW_;            // query heads per wave
  static constexpr int HG = G / HPW;          // waves per 32-row group
  static constexpr int RG = RG_;              // 32-row groups per work item
  static constexpr int NW = RG * HG;          // waves
  static constexpr int NT = 64 * NW;
  static constexpr int GRAN = RG == 1 ? 0 : RG == 2 ? 1 : 2;  // work items of 32 << GRAN rows
  static constexpr bool FP8 = IN_ == SPB_FP8_E4M3;  // e4m3 K (fp8 MFMA for S), bf16 V (widened beforehand)
  static constexpr int ROWB_K = FP8 ? D : 2 * D;    // bytes per K row in LDS
  static constexpr int ROWB = 2 * D;                // bytes per V row (and per K row for bf16)
  static constexpr int BUFK = 64 * ROWB_K;          // one chunk of K
  static constexpr int BUF = 64 * ROWB;             // one chunk of V
  static constexpr int SLOT = BUFK + BUF;           // ring slot: K of a chunk, then its V
  // Q rows of a wave (32 rows x HPW heads, QROWB bytes each) are copied
  // into the 1 KB blocks of ring slot 1 that the wave itself later fills
  // with chunk 1, when they fit there.
  static constexpr int QROWB = FP8 ? D : 2 * D;
  static constexpr int QBLK = 32 * HPW * QROWB / 1024;  // Q blocks per wave
  static constexpr bool QLDS = QBLK * NW * 1024 <= SLOT;
  // bf16 output rows of a wave (32 rows x HPW heads) staged in the ring
  static constexpr int OROWB = 2 * HPW * D;
  // copies per wave per tensor for a 64-key and a 32-key chunk
  static constexpr int QK64 = 64 * ROWB_K / 1024 / NW;
  static constexpr int QK32 = 32 * ROWB_K / 1024 / NW;
  static constexpr int Q64 = 64 * ROWB / 1024 / NW;
  static constexpr int Q32 = 32 * ROWB / 1024 / NW;
  // work groups per CU the registers are budgeted for: two (at most 256 per
  // lane) with one query head per wave
  static constexpr int MINWG = HPW == 1 ? 2 : 1;
  static_assert(G % HPW == 0 && (RG == 1 || RG == 2 || RG == 4), "work item shape");
  static_assert(Q32 >= 1 && Q32 * NW * 1024 == 32 * ROWB, "a 32-key chunk must give every wave whole copies");
  static_assert(QK32 >= 1 && QK32 * NW * 1024 == 32 * ROWB_K, "a 32-key chunk must give every wave whole copies");
  static_assert(!FP8 || D == 128, "e4m3 inputs need head_dim 128");
  static_assert(NW * 32 * OROWB <= 2 * SLOT && (OROWB == 128 || OROWB == 256), "output staging must fit the ring");
  static_assert(QROWB == 128 || QROWB == 256, "Q rows of 128 or 256 bytes");
};

// LDS row swizzles (16-byte chunk c of row r lives at chunk c ^ f(r)).  K: a
// fragment read has 16 lanes on 16 consecutive rows at one chunk; V: a
// transpose read has 32 lanes on 4 consecutive rows at 4 consecutive chunks.
// Both spread those over all 64 banks.
template <int ROWB>
__device__ inline int swz_k(int r) { return ROWB == 256 ? (r & 15) : ((r >> 1) & 7); }
template <int ROWB>
__device__ inline int swz_v(int r) { return ROWB == 256 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// One work item (an item of the table, one KV head) per work group, two
// work groups per CU.  The item's chunk list (content chunks, then the
// chunks of the branches meeting its rows) is taken from the item table.  K
// and V of the chunks are copied global -> LDS into a two-slot ring, the copy
// of chunk i + 1 running while chunk i is computed.
template <int D, int G, int HPW_, int RG_, int OUT, int IN = SPB_BF16>
__global__ __launch_bounds__((DmaCfg<D, G, HPW_, RG_, IN>::NT), (DmaCfg<D, G, HPW_, RG_, IN>::MINWG)) void
branch_attention_dma(AttnParams p) {
  using C = DmaCfg<D, G, HPW_, RG_, IN>;
  constexpr int HPW = C::HPW;
  // ring slot s: K of chunk s (mod 2) at ring + s * SLOT, its V BUFK bytes on
  __shared__ __attribute__((aligned(1024))) char ring[2 * C::SLOT];
  __shared__ int4 chunks[kMaxChunks];

  const int w = blockIdx.x;
  const int kvh = w % p.hkv;
  const SpbItem it = p.items[w / p.hkv];
  const int nch = it.ncc + it.bn;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int rg = wave / C::HG, hgi = wave % C::HG;
  const int h0 = kvh * G + hgi * HPW;  // the wave's first query head
  const int qi = lane & 31, half = lane >> 5;
  const int local = rg * 32 + qi;
  const bool active = local < it.nrows;
  const int x = it.row0 + local;

  const uint32_t k_lds = lds_addr(&ring[0]), v_lds = k_lds + C::BUFK;

  // Copies chunk i (64 or 32 key rows; rows past the pass repeat its last
  // row, so every slot holds finite data) into ring slot i % 2.  Copy qq of
  // this wave moves slot bytes (qq*NW + wave)*1024 .. +1024 of each tensor:
  // lane t fills row r0 + qq*RSTEP at 16-byte position pos, where r0 and pos
  // do not depend on qq, and neither does the row swizzle (RSTEP is a
  // multiple of its period), so only the source row changes per copy.
  // (For e4m3 K, whose rows are half as long, K has its own row step and
  // lane positions; copy qq of K moves its own 1,024 bytes the same way.)
  constexpr int RSTEP = C::NW * 1024 / C::ROWB;
  constexpr int RSTEPK = C::NW * 1024 / C::ROWB_K;
  static_assert(RSTEP % 16 == 0 && RSTEPK % 16 == 0, "copy rounds must keep the swizzle phase");
  const int r0 = (wave * 1024 + lane * 16) / C::ROWB;
  const int pos = ((lane * 16) % C::ROWB) >> 4;
  const int r0k = (wave * 1024 + lane * 16) / C::ROWB_K;
  const int posk = ((lane * 16) % C::ROWB_K) >> 4;
  const uint32_t kofs = (uint32_t)(kvh * C::ROWB_K + ((posk ^ swz_k<C::ROWB_K>(r0k)) << 4));
  const uint32_t vofs = (uint32_t)(kvh * C::ROWB + ((pos ^ swz_v<C::ROWB>(r0)) << 4));
  const uint32_t ystride = (uint32_t)(p.hkv * C::ROWB);
  const uint32_t ystridek = (uint32_t)(p.hkv * C::ROWB_K);
  auto copy_k = [&](int key0, int slot, int qq) {
    const int y = min(key0 + r0k + qq * RSTEPK, p.n_tokens - 1);
    dma16(p.k, (uint32_t)y * ystridek + kofs, k_lds + (uint32_t)slot * C::SLOT + (uint32_t)(qq * C::NW + wave) * 1024);
  };
  auto copy_v = [&](int key0, int slot, int qq) {
    const int y = min(key0 + r0 + qq * RSTEP, p.n_tokens - 1);
    dma16(p.v, (uint32_t)y * ystride + vofs, v_lds + (uint32_t)slot * C::SLOT + (uint32_t)(qq * C::NW + wave) * 1024);
  };
  auto copy_chunk = [&](int key0, int slot, bool content) {
    if (content) {
#pragma unroll
      for (int qq = 0; qq < C::Q64; ++qq) {
        if (qq < C::QK64) copy_k(key0, slot, qq);
        copy_v(key0, slot, qq);
      }
    } else {
#pragma unroll
      for (int qq = 0; qq < C::Q32; ++qq) {
        if (qq < C::QK32) copy_k(key0, slot, qq);
        copy_v(key0, slot, qq);
      }
    }
  };
  auto issue = [&](int i) { copy_chunk(chunks[i].x, i & 1, chunks[i].y < 0); };

  // An item's content chunk 0 starts at its content start, so its copy needs
  // no chunk list: it goes out first, ahead of the list, row and Q loads.
  const bool early = it.ncc > 0;
  if (early) copy_chunk(it.seg, 0, true);

  // Q block b of this wave (rows 32 j + r of its heads, j = head, r = row of
  // its 32, RPB rows per block) is ring block NW * b + wave of slot 1: the
  // blocks this wave's own copies of chunk 1 overwrite, so no other wave
  // reads or writes them in between.  Rows are swizzled like K rows; lanes
  // past the item copy the pass's last row (finite; their rows see no key).
  constexpr int RPB = 1024 / C::QROWB;
  const uint32_t q_lds = k_lds + C::SLOT;
  if constexpr (C::QLDS) {
    // offsets from the wave's first row (64-bit base), so Q may exceed 4 GiB
    const int xb = min(it.row0 + rg * 32, p.n_tokens - 1);
    const char *qb = (const char *)p.q + ((size_t)xb * p.hq + h0) * C::QROWB;
#pragma unroll
    for (int b = 0; b < C::QBLK; ++b) {
      const int rr = b * RPB + lane / (C::QROWB / 16);  // 32 j + r
      const int pc = lane % (C::QROWB / 16);
      const int xr = min(it.row0 + rg * 32 + (rr & 31), p.n_tokens - 1);
      const int c = pc ^ swz_k<C::QROWB>(rr);
      const uint32_t off = ((uint32_t)(xr - xb) * (uint32_t)p.hq + (uint32_t)(rr >> 5)) * C::QROWB + (uint32_t)c * 16;
      dma16(qb, off, q_lds + (uint32_t)(b * C::NW + wave) * 1024);
    }
  }

  load_chunk_list(p, it, chunks, tid, C::NT);
  const SpbRow row = load_row(p, x, active);
  QFrag<D, IN> qf[HPW];
  if constexpr (!C::QLDS) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) load_q<D, IN>(qf[j], p, x, h0 + j, active, half);
  }

  // fragment offsets in the swizzled layout
  FragOffsets<D, IN> fo;
#pragma unroll
  for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
    if constexpr (C::FP8) {  // 64 elements per step: 16-byte chunks 4t + 2half, +1
      fo.k[t][0] = qi * C::ROWB_K + (((4 * t + 2 * half) ^ swz_k<C::ROWB_K>(qi)) << 4);
      fo.k[t][1] = qi * C::ROWB_K + (((4 * t + 2 * half + 1) ^ swz_k<C::ROWB_K>(qi)) << 4);
    } else {
      fo.k[t][0] = qi * C::ROWB + (((2 * t + half) ^ swz_k<C::ROWB>(qi)) << 4);
    }
  }
  {
    const int g = qi >> 4, l16 = lane & 15;
    const int rr = half * 4 + (l16 >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int cv = 2 * g + ((l16 & 3) >> 1) + 4 * db;
      fo.v[db] = rr * C::ROWB + ((cv ^ swz_v<C::ROWB>(rr)) << 4) + (l16 & 1) * 8;
    }
  }

  RowState st[HPW];
  f32x16 o[HPW][D / 32];
#pragma unroll
  for (int j = 0; j < HPW; ++j) {
    st[j] = RowState{kNegInf, 0.f};
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[j][db] = f32x16{0.f};
  }
  __syncthreads();  // chunk list in LDS
  if (!early) issue(0);
  wait_all_loads();  // chunk 0, the row and the Q rows
  lds_barrier();
  if constexpr (C::QLDS) {
    // Q fragments: the K fragment pieces of row 32 j + qi of the Q blocks
    const char *qbase = ring + C::SLOT;
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const int rr = j * 32 + qi;
      const char *rowp = qbase + ((rr / RPB) * C::NW + wave) * 1024 + (rr % RPB) * C::QROWB;
#pragma unroll
      for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
        if constexpr (C::FP8) {
          const u32x4 a0 = *(const u32x4 *)(rowp + (((4 * t + 2 * half) ^ swz_k<C::QROWB>(rr)) << 4));
          const u32x4 a1 = *(const u32x4 *)(rowp + (((4 * t + 2 * half + 1) ^ swz_k<C::QROWB>(rr)) << 4));
          qf[j].f[t] = i32x8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        } else {
          const u32x4 a = *(const u32x4 *)(rowp + (((2 * t + half) ^ swz_k<C::QROWB>(rr)) << 4));
          qf[j].f[t] = *(const bf16x8_t *)&a;
        }
      }
    }
    // the reads are done before this wave's copies of chunk 1 reuse the blocks
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  }
  if (nch > 1) issue(1);

  auto block = [&](int slot, const Vis &vis, bool two, bool masked, bool anc) {
    const char *Kb = ring + slot * C::SLOT;
    const char *Vb = Kb + C::BUFK;
    f32x16 s0[HPW], s1[HPW];
    if constexpr (C::FP8)
      qk_chunk_fp8<D, HPW, C::ROWB_K>(Kb, fo, qf, s0, s1, two);
    else
      qk_chunk<D, HPW, C::ROWB>(Kb, fo, qf, s0, s1, two);
    if (masked) {
      if (anc) {
#pragma unroll
        for (int j = 0; j < HPW; ++j) mask_block<1>(s0[j], vis);
      } else {
#pragma unroll
        for (int j = 0; j < HPW; ++j) mask_block<0>(s0[j], vis);
        if (two) {
          Vis v1 = vis;
          v1.thr -= 32;
#pragma unroll
          for (int j = 0; j < HPW; ++j) mask_block<0>(s1[j], v1);
        }
      }
    }
    VStep<D> v0;
    read_v_step<D, C::ROWB>(Vb, fo, 0, v0);
    uint32_t pk[HPW][2][8];
#pragma unroll
    for (int j = 0; j < HPW; ++j) softmax_chunk<D>(s0[j], s1[j], two, p.sc, st[j], o[j], pk[j]);
    pv_chunk<D, HPW, C::ROWB>(Vb, fo, pk, o, two, v0);
  };

  for (int i = 0; i < nch; ++i) {
    const ChunkStep cs = chunk_step(chunks[i], row, half);
    if (cs.run) block(i & 1, cs.vis, cs.two, cs.masked, cs.anc);
    // chunk i + 1 has landed and every wave is done with slot i % 2
    wait_vmcnt<0>();
    lds_barrier();
    if (i + 2 < nch) issue(i + 2);
  }

  if constexpr (OUT == SPB_BF16) {
    // bf16 O through LDS, so that each global store writes whole 16-byte
    // pieces of 4 (or 8) consecutive rows: row r of the wave's 32 (heads
    // h0 .. h0 + HPW - 1 side by side, OROWB bytes) at ring + wave * 32 *
    // OROWB, 16-byte pieces swizzled by row.  The loop's last barrier has
    // freed the ring; each wave reads back only what it wrote.
    constexpr int NP = C::OROWB / 16;
    char *tile = ring + wave * 32 * C::OROWB;
    if (nch == 0) lds_barrier();  // no loop barrier: other waves may still read their Q blocks
#pragma unroll
    for (int j = 0; j < HPW; ++j) {
      const float l = st[j].l + __shfl_xor(st[j].l, 32);
      const float inv = p.s_v / l;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int gg = 0; gg < 4; ++gg) {
          const int piece = (j * D + db * 32 + gg * 8) / 8;  // d = db*32 + gg*8 + half*4 .. +4
          const u32x2 v = {pack_bf16(o[j][db][4 * gg] * inv, o[j][db][4 * gg + 1] * inv),
                           pack_bf16(o[j][db][4 * gg + 2] * inv, o[j][db][4 * gg + 3] * inv)};
          *(u32x2 *)(tile + qi * C::OROWB + ((piece ^ swz_k<C::OROWB>(qi)) << 4) + half * 8) = v;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int b = 0; b < 32 * C::OROWB / 1024; ++b) {
      const int r = b * (1024 / C::OROWB) + lane / NP, pc = lane % NP;
      const u32x4 v = *(const u32x4 *)(tile + r * C::OROWB + ((pc ^ swz_k<C::OROWB>(r)) << 4));
      if (rg * 32 + r < it.nrows)
        *(u32x4 *)((char *)p.o + ((size_t)(it.row0 + rg * 32 + r) * p.hq + h0) * (2 * D) + pc * 16) = v;
    }
  } else if (active) {
#pragma unroll
    for (int j = 0; j < HPW; ++j) store_o<D, OUT>(p, x, h0 + j, half, st[j], o[j]);
  }
}

// ------------------------------------------------- f32 / fp8: staged kernel

template <int D, int G, int IN>
struct StagedCfg {
  static constexpr bool FP8 = IN == SPB_FP8_E4M3;
  static constexpr int RW = G == 4 ? 2 : 4;   // 32-row groups per work item
  static constexpr int NW = RW * G;           // waves, one query head each
  static constexpr int NT = NW * 64;
  static constexpr int ROWS = 32 * RW;
  static constexpr int GRAN = RW == 2 ? 1 : 2;  // work items of 32 << GRAN rows
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

template <int D, int G, int IN>
struct Stage {  // one chunk's K and V units held by this thread
  u32x4 k[StagedCfg<D, G, IN>::KPT];
  u32x4 v[StagedCfg<D, G, IN>::VPT];
};

// Global -> registers: rows key0 .. key0 + nrows of K and V for KV head kvh;
// rows past nrows (or past the pass) are zeros.
template <int D, int G, int IN>
__device__ inline void stage_load(Stage<D, G, IN> &st, const AttnParams &p, int kvh, int key0, int nrows) {
  using C = StagedCfg<D, G, IN>;
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

// registers -> LDS buffers; every one of the 64 rows is written (zeros past
// the chunk), so no slot ever holds a stale or uninitialised value.
template <int D, int G, int IN>
__device__ inline void stage_store(const Stage<D, G, IN> &st, char *Ks, char *Vs) {
  using C = StagedCfg<D, G, IN>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < C::KPT; ++i) {
    const int u = tid + i * C::NT;
    if (u < 64 * C::KCH) *(u32x4 *)(Ks + (u / C::KCH) * C::KPITCH + (u % C::KCH) * 16) = st.k[i];
  }
#pragma unroll
  for (int i = 0; i < C::VPT; ++i) {
    const int u = tid + i * C::NT;
    if (u < 64 * C::VCH) *(u32x4 *)(Vs + (u / C::VCH) * C::VPITCH + (u % C::VCH) * 16) = st.v[i];
  }
}

template <int D, int G, int IN, int OUT>
__global__ __launch_bounds__((StagedCfg<D, G, IN>::NT)) void branch_attention_staged(AttnParams p) {
  using C = StagedCfg<D, G, IN>;
  __shared__ __attribute__((aligned(16))) char Ks[2][64 * C::KPITCH];
  __shared__ __attribute__((aligned(16))) char Vs[2][64 * C::VPITCH];
  __shared__ int4 chunks[kMaxChunks];

  const int w = blockIdx.x;
  const int kvh = w % p.hkv;
  const SpbItem it = p.items[w / p.hkv];
  const int nch = it.ncc + it.bn;
  const int sub0 = it.row0, sub_n = it.nrows;

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rw = wave / G, gh = wave % G;
  const int h = kvh * G + gh;
  const int qi = lane & 31, half = lane >> 5;
  const int local = rw * 32 + qi;
  const bool active = local < sub_n;
  const int x = sub0 + local;

  load_chunk_list(p, it, chunks, tid, C::NT);
  const SpbRow row = load_row(p, x, active);
  QFrag<D, IN> qf[1];
  load_q<D, IN>(qf[0], p, x, h, active, half);

  FragOffsets<D, IN> fo;
#pragma unroll
  for (int t = 0; t < QFrag<D, IN>::STEPS; ++t) {
    if constexpr (C::FP8) {
      fo.k[t][0] = qi * C::KPITCH + t * 64 + half * 32;
      fo.k[t][1] = fo.k[t][0] + 16;
    } else {
      fo.k[t][0] = qi * C::KPITCH + t * 32 + half * 16;
    }
  }
  {
    const int g = qi >> 4, l16 = lane & 15;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      fo.v[db] = (half * 4 + (l16 >> 2)) * C::VPITCH + (g * 16 + 4 * (l16 & 3)) * 2 + db * 64;
  }

  RowState st[1] = {RowState{kNegInf, 0.f}};
  f32x16 o[1][D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[0][db] = f32x16{0.f};

  __syncthreads();  // chunk list ready

  // Prefetch loads are issued on every trip (past the end they reload the
  // last chunk), so no branch changes the count of outstanding loads and each
  // LDS store waits only for the chunk it writes.
  auto nrows_of = [&](int i) { return chunks[i].y < 0 ? kChunk : kBranchChunk; };
  Stage<D, G, IN> stg;
  if (nch > 0) {
    stage_load<D, G, IN>(stg, p, kvh, chunks[0].x, nrows_of(0));
    stage_store<D, G, IN>(stg, Ks[0], Vs[0]);
    lds_barrier();
    const int i1 = min(1, nch - 1);
    stage_load<D, G, IN>(stg, p, kvh, chunks[i1].x, nrows_of(i1));
  }

  auto block = [&](int i, const Vis &vis, bool two, bool masked, bool anc) {
    const char *Kb = Ks[i & 1];
    const char *Vb = Vs[i & 1];
    f32x16 s0[1], s1[1];
    qk_block<D, IN, 1>(Kb, fo, qf, s0);
    if (two) qk_block<D, IN, 1>(Kb + 32 * C::KPITCH, fo, qf, s1);
    if (masked) {
      if (anc) {
        mask_block<1>(s0[0], vis);
      } else {
        mask_block<0>(s0[0], vis);
        if (two) {
          Vis v1 = vis;
          v1.thr -= 32;
          mask_block<0>(s1[0], v1);
        }
      }
    }
    uint32_t pk[2][8];
    softmax_chunk<D>(s0[0], s1[0], two, p.sc, st[0], o[0], pk);
    {
      uint32_t pb[1][8];
#pragma unroll
      for (int r = 0; r < 8; ++r) pb[0][r] = pk[0][r];
      pv_block<D, IN, 1, C::VPITCH>(Vb, fo, pb, o);
    }
    if (two) {
      uint32_t pb[1][8];
#pragma unroll
      for (int r = 0; r < 8; ++r) pb[0][r] = pk[1][r];
      pv_block<D, IN, 1, C::VPITCH>(Vb + 32 * C::VPITCH, fo, pb, o);
    }
  };
  auto advance = [&](int i) {  // stage chunk i+1 into the other buffer, start loading chunk i+2
    const int i2 = min(i + 2, nch - 1);
    stage_store<D, G, IN>(stg, Ks[(i & 1) ^ 1], Vs[(i & 1) ^ 1]);
    lds_barrier();
    stage_load<D, G, IN>(stg, p, kvh, chunks[i2].x, nrows_of(i2));
  };
  walk_chunks(chunks, nch, row, half, block, advance);

  if (active) store_o<D, OUT>(p, x, h, half, st[0], o[0]);
}

// ------------------------------------------------------------------ launch

AttnParams make_params(const AttnLaunch &a) {
  AttnParams p;
  p.q = a.q; p.k = a.k; p.v = a.v; p.o = a.o;
  p.hq = a.hq; p.hkv = a.hkv; p.n_tokens = a.n_tokens;
  p.sc = a.scale * kLog2e * a.s_q * a.s_k;
  p.s_v = a.s_v;
  p.rows = (const SpbRow *)a.rows;
  p.bchunks = (const SpbChunk *)a.bchunks;
  return p;
}

// Work-item shapes of the dma kernel: (query heads per wave, 32-row groups).
// One head per wave and up to eight waves (two per SIMD); d = 64 rows are too
// short for eight waves to split a 32-key chunk into whole copies, so there
// the two heads of a wave share the K/V reads and four waves suffice.
template <int D, int G>
struct DmaShape {  // four waves per work group
  static constexpr int HPW = (G >= 2 && D == 64) ? 2 : 1;
  static constexpr int RG = 4 / (G / HPW);
};

template <int D, int G, int OUT, int IN = SPB_BF16>
int launch_dma(const AttnLaunch &a, hipStream_t s) {
  using Sh = DmaShape<D, G>;
  using C = DmaCfg<D, G, Sh::HPW, Sh::RG, IN>;
  const long long work = (long long)a.n_items[C::GRAN] * a.hkv;
  if (work > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  // the copies address K/V with 32-bit byte offsets
  if ((long long)a.n_tokens * a.hkv * C::ROWB > 0xFFFFFFFFll) return (int)hipErrorInvalidValue;
  AttnParams p = make_params(a);
  if constexpr (C::FP8) {
    // V widened to bf16 into the workspace first (every row of the pass)
    const long long n16 = (long long)a.n_tokens * a.hkv * D / 16;
    if (n16 > 0) {
      hipLaunchKernelGGL(widen_v_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                         (const unsigned char *)a.v, (uint32_t *)a.v_wide, n16);
      const int e = (int)hipGetLastError();
      if (e) return e;
    }
    p.v = a.v_wide;
  }
  if (work == 0) return 0;
  p.items = (const SpbItem *)a.items[C::GRAN];
  p.n_work = (int)work;
  hipLaunchKernelGGL((branch_attention_dma<D, G, Sh::HPW, Sh::RG, OUT, IN>), dim3((unsigned)work), dim3(C::NT), 0, s,
                     p);
  return (int)hipGetLastError();
}

template <int D, int G, int IN, int OUT>
int launch_staged(const AttnLaunch &a, hipStream_t s) {
  using C = StagedCfg<D, G, IN>;
  const long long work = (long long)a.n_items[C::GRAN] * a.hkv;
  if (work > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  if (work == 0) return 0;
  AttnParams p = make_params(a);
  p.items = (const SpbItem *)a.items[C::GRAN];
  p.n_work = (int)work;
  hipLaunchKernelGGL((branch_attention_staged<D, G, IN, OUT>), dim3((unsigned)work), dim3(C::NT), 0, s, p);
  return (int)hipGetLastError();
}

template <int D, int G>
int launch_dtypes(const AttnLaunch &a, hipStream_t s) {
  if (a.in_dtype == SPB_BF16)
    return a.out_dtype == SPB_F32 ? launch_dma<D, G, SPB_F32>(a, s) : launch_dma<D, G, SPB_BF16>(a, s);
  if (a.in_dtype == SPB_F32)
    return a.out_dtype == SPB_F32 ? launch_staged<D, G, SPB_F32, SPB_F32>(a, s)
                                  : launch_staged<D, G, SPB_F32, SPB_BF16>(a, s);
  if constexpr (D == 128) {
    if (a.v_wide)
      return a.out_dtype == SPB_F32 ? launch_dma<D, G, SPB_F32, SPB_FP8_E4M3>(a, s)
                                    : launch_dma<D, G, SPB_BF16, SPB_FP8_E4M3>(a, s);
    return a.out_dtype == SPB_F32 ? launch_staged<D, G, SPB_FP8_E4M3, SPB_F32>(a, s)
                                  : launch_staged<D, G, SPB_FP8_E4M3, SPB_BF16>(a, s);
  }
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
