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
//   topk_lse_kernel         per row: LSE over the vocabulary and the k best
//                           allowed tokens
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
struct Cand {
  float v;
  int id;
};
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

// One work group per row.  Thread t walks elements t, t + 256, ... keeping a
// running (max, sum of exp) and its own best kMaxTopK allowed tokens; the 256
// partials are merged pairwise in a fixed tree.
__global__ __launch_bounds__(kTopkThreads) void topk_lse_kernel(TopkLaunch a) {
  const long long row = blockIdx.x;
  const int tid = threadIdx.x;
  const float *z = a.z + (size_t)row * a.vocab;
  const int mi = a.mask_of_row ? a.mask_of_row[row] : -1;
  const uint32_t *mask = (a.masks && mi >= 0) ? a.masks + (size_t)mi * ((a.vocab + 31) / 32) : nullptr;
  const int stop = a.stop_of_row ? a.stop_of_row[row] : -1;

  float m = kNegInf, s = 0.f;
  Cand best[kMaxTopK];
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) best[j] = Cand{kNegInf, 0x7FFFFFFF};
  for (int i = tid; i < a.vocab; i += kTopkThreads) {
    const float v = z[i];
    if (v > m) {
      s = s * __expf(m - v) + 1.f;
      m = v;
    } else {
      s += __expf(v - m);
    }
    const bool ok = !mask || i == stop || ((mask[i >> 5] >> (i & 31)) & 1u);
    const Cand c{v, i};
    if (ok && better(c, best[kMaxTopK - 1])) {
      best[kMaxTopK - 1] = c;
#pragma unroll
      for (int j = kMaxTopK - 1; j > 0; --j)
        if (better(best[j], best[j - 1])) {
          const Cand t = best[j];
          best[j] = best[j - 1];
          best[j - 1] = t;
        }
    }
  }
  __shared__ float sm[kTopkThreads], ss[kTopkThreads];
  __shared__ Cand sl[kTopkThreads][kMaxTopK];
  sm[tid] = m;
  ss[tid] = s;
#pragma unroll
  for (int j = 0; j < kMaxTopK; ++j) sl[tid][j] = best[j];
  __syncthreads();
  for (int w = kTopkThreads / 2; w >= 1; w >>= 1) {
    if (tid < w) {
      const float m1 = sm[tid], m2 = sm[tid + w];
      const float mn = fmaxf(m1, m2);
      ss[tid] = (m1 == kNegInf ? 0.f : ss[tid] * __expf(m1 - mn)) + (m2 == kNegInf ? 0.f : ss[tid + w] * __expf(m2 - mn));
      sm[tid] = mn;
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
  if (tid == 0) {
    const float lse = sm[0] + __logf(ss[0]);
    a.lse[row] = lse;
    for (int j = 0; j < a.k; ++j) {
      const Cand c = sl[0][j];
      a.ids[row * a.k + j] = c.v == kNegInf ? -1 : c.id;
      a.lp[row * a.k + j] = c.v == kNegInf ? kNegInf : c.v - lse;
    }
  }
}

// ------------------------------------------------------- decode attention

// One wave per (decoded row, KV head), the G = hq / hkv query heads of the
// group together.  Keys: the slot's prefix ranges in the pass cache, then
// the row's ancestors in the decode cache, then the row itself.  Lane j
// scores key j of each 64-key chunk (q . k in f32); the online softmax's max
// and sum run over a fixed butterfly; for P.V lane l owns dimensions
// l * D / 64 .. of every head.
template <int D, int G>
__global__ __launch_bounds__(64) void decode_attention_kernel(DecodeAttnLaunch a) {
  constexpr int DL = D / 64;  // dimensions per lane in P.V
  const int r = blockIdx.x / a.hkv, g = blockIdx.x % a.hkv;
  const int lane = threadIdx.x;
  const int slot = r / a.beams;
  __shared__ float qs[G][D];
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
  // key index -> row pointer (pass cache, then decode cache)
  auto key_row = [&](int kidx, bool v) -> const uint16_t * {
    if (kidx < total) {
      int i = 0;
      while (i < nr - 1 && kidx >= max(rg[2 * i + 1], 0)) {
        kidx -= max(rg[2 * i + 1], 0);
        ++i;
      }
      const int prow = min(max(rg[2 * i] + kidx, 0), a.n_pass_rows - 1);
      return (v ? a.vp : a.kp) + (size_t)prow * kstride + (size_t)g * D;
    }
    kidx -= total;
    const int own = a.n_path * a.R + r;
    int crow = kidx < a.n_path ? a.path[(size_t)r * a.t_cap + kidx] : own;
    if (crow < 0 || crow >= a.n_dec_rows) crow = own;  // a finished beam's unused row
    return (v ? a.vd : a.kd) + (size_t)crow * kstride + (size_t)g * D;
  };
  for (int c0 = 0; c0 < n_keys; c0 += 64) {
    const int kidx = c0 + lane;
    float sc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) sc[h] = kNegInf;
    if (kidx < n_keys) {
      const uint16_t *kr = key_row(kidx, false);
      float acc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
      for (int dd = 0; dd < D; dd += 8) {
        const uint4 u = *(const uint4 *)(kr + dd);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = bf2f(w[e] & 0xFFFFu), k1 = bf2f(w[e] >> 16);
#pragma unroll
          for (int h = 0; h < G; ++h) {
            acc[h] = __builtin_fmaf(qs[h][dd + 2 * e], k0, acc[h]);
            acc[h] = __builtin_fmaf(qs[h][dd + 2 * e + 1], k1, acc[h]);
          }
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = acc[h] * a.scale;
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
    const int nk = n_keys - c0 < 64 ? n_keys - c0 : 64;
    for (int j = 0; j < nk; ++j) {
      const uint16_t *vr = key_row(c0 + j, true);
      float vv[DL];
#pragma unroll
      for (int e = 0; e < DL; ++e) vv[e] = bf2f(vr[lane * DL + e]);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pj = __shfl(p[h], j);
#pragma unroll
        for (int e = 0; e < DL; ++e) o[h][e] = __builtin_fmaf(pj, vv[e], o[h][e]);
      }
    }
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
  if (a.rows > 0x7FFFFFFFll) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(topk_lse_kernel, dim3((unsigned)a.rows), dim3(kTopkThreads), 0, (hipStream_t)stream, a);
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
