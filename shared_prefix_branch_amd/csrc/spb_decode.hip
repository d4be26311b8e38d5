// spb_decode.hip -- searched decoding of extraction slots (gfx950).
//
// A slot ({*} text, {n} a number, {$} an amount) is decoded from the same
// read as the scored questions, with its answers' probabilities [PyPI
// "spinf-serve 0.1.1", "What it does": Extraction and generation], the slots
// of many inputs together [PyPI "Speed and scale"].  The search is a beam
// search of width B over the model's vocab-wide log-probabilities, proposing
// only the slot kind's tokens (and the stop token).  One decode step, for the
// B beams of every slot of a pass at once:
//
//   gather_rows_kernel      the fed tokens' embedding rows (and positions)
//   (decoder stack)         rmsnorm / linear kernels of spb_layer.hip
//   decode_attention_kernel each new row over its slot's prefix in the pass's
//                           KV cache, then its own beam's decoded rows
//   (lm head)               linear kernel, f32 logits
//   topk_part_kernel,       per row: LSE over the vocabulary and the k best
//   topk_merge_kernel       allowed tokens (8192-entry parts, merged in order)
//   beam_step_kernel        per slot: the B best candidates, the new beams
//
// Every choice is taken in a total order (score, then beam, then token id),
// and every sum runs in a fixed order, so a slot's answers do not depend on
// which other slots are decoded with it.
#define SPB_HD __host__ __device__
#include "spb_meta.h"
#include "spb_launch.h"
#include "../../include/spb.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace spb {
namespace {

constexpr float kNegInf = -__builtin_inff();

__device__ inline float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
__device__ inline uint32_t f2bf(float f) {  // round to nearest even (finite inputs)
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// (value, id) with the order: larger value first, then smaller id.
__device__ inline bool better(const Cand &a, const Cand &b) { return a.v > b.v || (a.v == b.v && a.id < b.id); }

// ------------------------------------------------------------ row gather

__global__ __launch_bounds__(256) void gather_rows_kernel(GatherLaunch a) {
  const long long r = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= a.rows) return;
  const int lane = threadIdx.x & 63;
  const int sr = min(max(a.idx[r], 0), a.n_src - 1);
  const uint16_t *src = a.src + (size_t)sr * a.dim;
  if (a.dst_f32) {
    float *dst = a.dst_f32 + (size_t)r * a.dim;
    for (int i = lane; i < a.dim; i += 64) dst[i] = bf2f(src[i]);
  } else {
    uint16_t *dst = a.dst_bf16 + (size_t)r * a.dim;
    for (int i = lane; i < a.dim; i += 64) dst[i] = src[i];
  }
  if (a.pos && lane == 0) a.pos[r] = a.pos_base[r / a.per] + a.pos_add;
}

// ------------------------------------------------------------ top-k + LSE

constexpr int kTopkThreads = 256;

// Merges two (max, sum of exp) partials.
__device__ inline void lse_merge(float &m, float &s, float m2, float s2) {
  const float mn = fmaxf(m, m2);
  s = (m == kNegInf ? 0.f : s * __expf(m - mn)) + (m2 == kNegInf ? 0.f : s2 * __expf(m2 - mn));
  m = mn;
}

// Inserts c into the sorted list L (best first) if it belongs there.
__device__ __attribute__((always_inline)) inline void topk_insert(Cand (&L)[kMaxTopK], const Cand &c) {
  if (!better(c, L[kMaxTopK - 1])) return;
  L[kMaxTopK - 1] = c;
#pragma unroll
  for (int j = kMaxTopK - 1; j > 0; --j)
    if (better(L[j], L[j - 1])) {
      const Cand t = L[j];
      L[j] = L[j - 1];
      L[j - 1] = t;
    }
}

// Tree merge of the work group's 256 partials (fixed pairs), result in slot 0.
__device__ inline void topk_tree(float *sm, float *ss, Cand (*sl)[kMaxTopK], int tid) {
  for (int w = kTopkThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) {
      float m = sm[tid], s = ss[tid];
      lse_merge(m, s, sm[tid + w], ss[tid + w]);
      sm[tid] = m;
      ss[tid] = s;
      Cand out[kMaxTopK];
      int i1 = 0, i2 = 0;
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) {
        const Cand c1 = sl[tid][i1], c2 = sl[tid + w][i2];
        if (better(c2, c1)) {
          out[j] = c2;
          ++i2;
        } else {
          out[j] = c1;
          ++i1;
        }
      }
#pragma unroll
      for (int j = 0; j < kMaxTopK; ++j) sl[tid][j] = out[j];
    }
    __syncthreads();
  }
}

// First kernel: work group (row, part) covers vocabulary entries
// part*8192 .. +8192; each thread reads 8 entries per round (two 16-byte
// loads in flight) and keeps a running (max, sum of exp) and its best
// kMaxTopK allowed tokens.
__global__ __launch_bounds__(kTopkThreads) void topk_part_kernel(TopkLaunch a, TopkPart *parts, int n_parts) {
  const long long row = blockIdx.x / n_parts;
  const int part = blockIdx.x % n_parts;
  const int tid = threadIdx.x;
  const float *z = a.z + (size_t)row * a.vocab;
  const int mi = a.mask_of_row ? a.mask_of_row[row] : -1;
  const uint32_t *mask = (a.masks && mi >= 0) ? a.masks + (size_t)mi * ((a.vocab + 31) / 32) : nullptr;
  const int stop = a.stop_of_row ? a.stop_of_row[row] : -1;
  const int lo = part * kTopkSpan, hi = min(lo + kTopkSpan, a.vocab);
  float m = kNegInf, s = 0.f;
  Cand best[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) best[j] = Cand{kNegInf, 0x7FFFFFFF};
  auto take = [&](int i, float v) {
    if (v > m) {
      s = s * __expf(m - v) + 1.f;
      m = v;
    } else {
      s += __expf(v - m);
    }
    const bool ok = !mask || i == stop || ((mask[i >> 5] >> (i & 31)) & 1u);
    if (ok) topk_insert(best, Cand{v, i});
  };
  const bool vec = (a.vocab & 3) == 0;  // rows 16-byte aligned
  for (int i0 = lo + tid * 8; i0 < hi; i0 += kTopkThreads * 8) {
    if (vec && i0 + 8 <= hi) {
      const float4 u0 = *(const float4 *)(z + i0), u1 = *(const float4 *)(z + i0 + 4);
      const float v[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) take(i0 + j, v[j]);
    } else {
      for (int j = 0; j < 8 && i0 + j < hi; ++j) take(i0 + j, z[i0 + j]);
    }
  }
  __shared__ float sm[kTopkThreads], ss[kTopkThreads];
  __shared__ Cand sl[kTopkThreads][kMaxTopK];
  sm[tid] = m;
  ss[tid] = s;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) sl[tid][j] = best[j];
  __syncthreads();
  topk_tree(sm, ss, sl, tid);
  if (tid == 0) {
    TopkPart &P = parts[blockIdx.x];
    P.m = sm[0];
    P.s = ss[0];
#pragma unroll
    for (int j = 0; j < kMaxTopK; ++j) P.best[j] = sl[0][j];
  }
}

// Second kernel: one wave per row merges the row's parts in part order.
__global__ __launch_bounds__(64) void topk_merge_kernel(TopkLaunch a, const TopkPart *parts, int n_parts) {
  const long long row = blockIdx.x;
  if (threadIdx.x != 0) return;
  const TopkPart *P = parts + row * n_parts;
  float m = P[0].m, s = P[0].s;
  Cand best[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) best[j] = P[0].best[j];
  for (int q = 1; q < n_parts; ++q) {
    lse_merge(m, s, P[q].m, P[q].s);
    for (int j = 0; j < kMaxTopK; ++j) {
      const Cand c = P[q].best[j];
      if (!better(c, best[kMaxTopK - 1])) break;  // the part's list is sorted
      topk_insert(best, c);
    }
  }
  const float lse = m + __logf(s);
  a.lse[row] = lse;
  for (int j = 0; j < a.k; ++j) {
    const Cand c = best[j];
    a.ids[row * a.k + j] = c.v == kNegInf ? -1 : c.id;
    a.lp[row * a.k + j] = c.v == kNegInf ? kNegInf : c.v - lse;
  }
}

// ------------------------------------------------------- decode attention

// One wave per (decoded row, KV head), the G = hq / hkv query heads of the
// group together.  Keys: the slot's prefix ranges in the pass cache, then
// the row's ancestors in the decode cache, then the row itself.  Lane j
// scores key j of each 64-key chunk (q . k in f32, its key row read with all
// 16-byte loads in flight); the online softmax's max and sum run over a fixed
// butterfly; the chunk's V rows are staged in LDS, and for P.V lane l owns
// dimensions l * D / 64 .. of every head.
template <int D, int G>
__global__ __launch_bounds__(64) void decode_attention_kernel(DecodeAttnLaunch a) {
  constexpr int DL = D / 64;  // dimensions per lane in P.V
  constexpr int PR = D / 8;   // 16-byte pieces per key row
  const int r = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int lane = threadIdx.x;
  const int slot = r / a.beams;
  __shared__ float qs[G][D];
  __shared__ __attribute__((aligned(16))) uint16_t vs[64][D];  // the chunk's V rows
  for (int i = lane; i < G * D; i += 64) {
    const int h = i / D, dd = i % D;
    qs[h][dd] = bf2f(a.q[((size_t)r * a.hq + g * G + h) * D + dd]);
  }
  __syncthreads();
  float m[G], l[G], o[G][DL];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    m[h] = kNegInf;
    l[h] = 0.f;
#pragma unroll
    for (int j = 0; j < DL; ++j) o[h][j] = 0.f;
  }
  const int nr = min(max(a.n_ranges[slot], 0), kMaxSlotRanges);
  const int32_t *rg = a.ranges + (size_t)slot * kMaxSlotRanges * 2;
  int total = 0;
  for (int i = 0; i < nr; ++i) total += max(rg[2 * i + 1], 0);
  const int n_keys = total + a.n_path + 1;
  const size_t kstride = (size_t)a.hkv * D;
  // key index -> row offset in its cache (pass cache, then decode cache)
  auto key_at = [&](int kidx, bool &dec) -> size_t {
    if (kidx < total) {
      int i = 0;
      while (i < nr - 1 && kidx >= max(rg[2 * i + 1], 0)) {
        kidx -= max(rg[2 * i + 1], 0);
        ++i;
      }
      dec = false;
      return (size_t)min(max(rg[2 * i] + kidx, 0), a.n_pass_rows - 1) * kstride + (size_t)g * D;
    }
    kidx -= total;
    const int own = a.n_path * a.R + r;
    int crow = kidx < a.n_path ? a.path[(size_t)r * a.t_cap + kidx] : own;
    if (crow < 0 || crow >= a.n_dec_rows) crow = own;  // a finished beam's unused row
    dec = true;
    return (size_t)crow * kstride + (size_t)g * D;
  };
  for (int c0 = 0; c0 < n_keys; c0 += 64) {
    const int kidx = c0 + lane;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = kNegInf;
    if (kidx < n_keys) {
      bool dec;
      const size_t off = key_at(kidx, dec);
      const uint16_t *kr = (dec ? a.kd : a.kp) + off;
      uint4 u[PR];
#pragma unroll
      for (int pc = 0; pc < PR; ++pc) u[pc] = *(const uint4 *)(kr + pc * 8);
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
#pragma unroll
      for (int pc = 0; pc < PR; ++pc) {
        const uint32_t w[4] = {u[pc].x, u[pc].y, u[pc].z, u[pc].w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = bf2f(w[e] & 0xFFFFu), k1 = bf2f(w[e] >> 16);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h] = __builtin_fmaf(qs[h][pc * 8 + 2 * e], k0, acc[h]);
            acc[h] = __builtin_fmaf(qs[h][pc * 8 + 2 * e + 1], k1, acc[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = acc[h] * a.scale;
    }
    // the chunk's V rows into LDS: piece p of the chunk is row p / PR, 16 bytes p % PR
    const int nk = n_keys - c0 < 64 ? n_keys - c0 : 64;
    {
      uint4 vv[PR];
#pragma unroll
      for (int i = 0; i < PR; ++i) {
        const int pcs = lane + 64 * i, kr = pcs / PR, pc = pcs % PR;
        vv[i] = uint4{0u, 0u, 0u, 0u};
        if (kr < nk) {
          bool dec;
          const size_t off = key_at(c0 + kr, dec);
          vv[i] = *(const uint4 *)((dec ? a.vd : a.vp) + off + pc * 8);
        }
      }
#pragma unroll
      for (int i = 0; i < PR; ++i) {
        const int pcs = lane + 64 * i;
        *(uint4 *)&vs[pcs / PR][(pcs % PR) * 8] = vv[i];
      }
    }
    float p[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float cm = sc[h];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) cm = fmaxf(cm, __shfl_xor(cm, off));
      const float mn = fmaxf(m[h], cm);
      const float alpha = m[h] == kNegInf ? 0.f : __expf(m[h] - mn);
      p[h] = sc[h] == kNegInf ? 0.f : __expf(sc[h] - mn);
      float ps = p[h];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) ps += __shfl_xor(ps, off);
      l[h] = l[h] * alpha + ps;
#pragma unroll
      for (int j = 0; j < DL; ++j) o[h][j] *= alpha;
      m[h] = mn;
    }
    __syncthreads();  // V rows in LDS
    for (int j = 0; j < nk; ++j) {
      float vf[DL];
#pragma unroll
      for (int e = 0; e < DL; ++e) vf[e] = bf2f(vs[j][lane * DL + e]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pj = __shfl(p[h], j);
#pragma unroll
        for (int e = 0; e < DL; ++e) o[h][e] = __builtin_fmaf(pj, vf[e], o[h][e]);
      }
    }
    __syncthreads();  // before the next chunk overwrites vs
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    uint16_t *dst = a.o + ((size_t)r * a.hq + g * G + h) * D + lane * DL;
#pragma unroll
    for (int e = 0; e < DL; ++e) dst[e] = (uint16_t)f2bf(o[h][e] / l[h]);
  }
}

// ------------------------------------------------------------ beam step

// One wave per slot.  Candidates: every finished beam as itself (token -1),
// every live beam b extended by its k best tokens; the B best in the order
// (score desc, beam asc, token asc) become the new beams.  At step 0 the
// single parent is the slot's template row.
__global__ __launch_bounds__(64) void beam_step_kernel(BeamLaunch a) {
  const int s = blockIdx.x, lane = threadIdx.x;
  const int B = a.beams, K = a.k, T = a.t_cap;
  const int stop = a.stop[s];
  constexpr int PER = kMaxBeams * kMaxTopK / 64;  // candidates per lane (<= 4)
  float cs[PER];
  int cb[PER], cx[PER];
  const int nb = a.step == 0 ? 1 : a.nb_in[s];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int c = lane * PER + i;  // candidate c = parent b * K + j
    const int b = c / K, j = c % K;
    cs[i] = kNegInf;
    cb[i] = 0x7FFFFFFF;
    cx[i] = 0x7FFFFFFF;
    if (b >= nb) continue;
    if (a.step > 0 && a.fin_in[s * B + b]) {
      if (j == 0) {
        cs[i] = a.score_in[s * B + b];
        cb[i] = b;
        cx[i] = -1;
      }
      continue;
    }
    const int row = a.step == 0 ? s : s * B + b;
    const int x = a.ids[row * K + j];
    if (x < 0) continue;
    cs[i] = (a.step == 0 ? 0.f : a.score_in[s * B + b]) + a.lp[row * K + j];
    cb[i] = b;
    cx[i] = x;
  }
  int n_new = 0;
  for (int nbk = 0; nbk < B; ++nbk) {
    // the best remaining candidate of the wave
    float bs = kNegInf;
    int bb = 0x7FFFFFFF, bx = 0x7FFFFFFF, bl = -1, bi = -1;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool bt = cb[i] != 0x7FFFFFFF &&
                      (bl < 0 || cs[i] > bs || (cs[i] == bs && (cb[i] < bb || (cb[i] == bb && cx[i] < bx))));
      if (bt) {
        bs = cs[i];
        bb = cb[i];
        bx = cx[i];
        bl = lane;
        bi = i;
      }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float os = __shfl_xor(bs, off);
      const int ob = __shfl_xor(bb, off), ox = __shfl_xor(bx, off), ol = __shfl_xor(bl, off);
      const bool take = ol >= 0 && (bl < 0 || os > bs || (os == bs && (ob < bb || (ob == bb && ox < bx))));
      if (take) {
        bs = os;
        bb = ob;
        bx = ox;
        bl = ol;
      }
    }
    if (bl < 0) break;  // no candidates left
    if (lane == bl) {
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (i == bi) cb[i] = 0x7FFFFFFF;  // taken
    }
    // write new beam nbk from parent bb (+ token bx)
    const int o = s * B + nbk;
    const int pi = s * B + bb;
    const int plen = a.step == 0 ? 0 : a.len_in[pi];
    for (int t = lane; t < T; t += 64) {
      int tok = -1, pth = -1;
      if (a.step > 0) {
        tok = t < plen ? a.tok_in[(size_t)pi * T + t] : -1;
        pth = a.path_in[(size_t)pi * T + t];
      }
      if (bx >= 0 && t == plen) tok = bx;
      // the parent's row fed this step (depth plen) joins the path
      if (bx >= 0 && a.step > 0 && t == plen - 1) pth = (plen - 1) * (a.n_slots * B) + pi;
      a.tok_out[(size_t)o * T + t] = tok;
      a.path_out[(size_t)o * T + t] = pth;
    }
    if (lane == 0) {
      const int len = bx >= 0 ? plen + 1 : plen;
      a.len_out[o] = len;
      a.fin_out[o] = bx < 0 ? 1 : (bx == stop ? 1 : 0);
      a.score_out[o] = bs;
      a.feed[o] = bx >= 0 ? bx : stop;
    }
    ++n_new;
  }
  if (lane == 0) a.nb_out[s] = n_new;
  __syncthreads();  // beam 0's state is read back below
  // beams past n_new (fewer candidates than B): inert copies of beam 0
  for (int nbk = n_new; nbk < B; ++nbk) {
    const int o = s * B + nbk, src = s * B;
    for (int t = lane; t < T; t += 64) {
      a.tok_out[(size_t)o * T + t] = a.tok_out[(size_t)src * T + t];
      a.path_out[(size_t)o * T + t] = a.path_out[(size_t)src * T + t];
    }
    if (lane == 0) {
      a.len_out[o] = a.len_out[src];
      a.fin_out[o] = 1;
      a.score_out[o] = kNegInf;
      a.feed[o] = a.feed[src];
    }
  }
}

template <int D>
int launch_decode_d(const DecodeAttnLaunch &a, hipStream_t s) {
  const int G = a.hq / a.hkv;
  const long long blocks = (long long)a.R * a.hkv;
  if (blocks > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  if (G == 1) hipLaunchKernelGGL((decode_attention_kernel<D, 1>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  else if (G == 2) hipLaunchKernelGGL((decode_attention_kernel<D, 2>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  else if (G == 4) hipLaunchKernelGGL((decode_attention_kernel<D, 4>), dim3((unsigned)blocks), dim3(64), 0, s, a);
  else return (int)hipErrorInvalidValue;
  return (int)hipGetLastError();
}

}  // namespace

int launch_gather_rows(const GatherLaunch &a, void *stream) {
  if (a.rows == 0) return 0;
  const long long blocks = (a.rows + 3) / 4;
  if (blocks > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(gather_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

int launch_topk_lse(const TopkLaunch &a, void *stream) {
  if (a.rows == 0) return 0;
  const int n_parts = (a.vocab + kTopkSpan - 1) / kTopkSpan;
  const long long blocks = a.rows * n_parts;
  if (blocks > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  TopkPart *parts = (TopkPart *)a.workspace;
  hipLaunchKernelGGL(topk_part_kernel, dim3((unsigned)blocks), dim3(kTopkThreads), 0, (hipStream_t)stream, a, parts,
                     n_parts);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return (int)e;
  hipLaunchKernelGGL(topk_merge_kernel, dim3((unsigned)a.rows), dim3(64), 0, (hipStream_t)stream, a, parts, n_parts);
  return (int)hipGetLastError();
}

int launch_decode_attention(const DecodeAttnLaunch &a, void *stream) {
  if (a.R == 0) return 0;
  if (a.head_dim == 128) return launch_decode_d<128>(a, (hipStream_t)stream);
  if (a.head_dim == 64) return launch_decode_d<64>(a, (hipStream_t)stream);
  return (int)hipErrorInvalidValue;
}

int launch_beam_step(const BeamLaunch &a, void *stream) {
  if (a.n_slots == 0) return 0;
  hipLaunchKernelGGL(beam_step_kernel, dim3((unsigned)a.n_slots), dim3(64), 0, (hipStream_t)stream, a);
  return (int)hipGetLastError();
}

}  // namespace spb
