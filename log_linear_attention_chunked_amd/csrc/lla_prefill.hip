// lla_prefill.hip — hand-over from a prompt to the decoding step: the level-state cache of
// loglinear_attn_decode_step after position P = T - 1, built directly from the prompt's k, v
// and log_a ("Log-Linear Attention": per-level states of the recurrent form, study notes
// sections 2-2 and 3-6; the level of a pair is the Fenwick level bit_length(t XOR s)).
//
// After position P the live levels are 0 (position P itself) and l = j + 1 for each set bit j of
// P, holding the aligned block of 2^j positions [(P >> l) << l, + 2^j), decayed to P:
//   S_l = sum_{s in block} exp(A_P - A_s) k_s v_s^T.
// Workgroups over (head, item): item 0 writes the rank-one factors (k_P, v_P) of level 0 into the
// cache's parity P & 1 and the log-scale row of that parity; every other item is a segment of
// up to kSeg positions of a live level's block (the large blocks split so that no workgroup
// walks a long block alone), contracted on MFMA in tiles of 64 positions taken from the
// segment's end backwards, so every decay weight exp(A_P - A_s) is built from sums of
// log_a <= 0 and never exceeds 1. A block of one segment is written to its level directly; the
// segments of a longer block go to a scratch array and a second kernel adds them in segment
// order (deterministic). The weighted
// operand is split into bf16 hi + lo parts (bf16 inputs), as in the backward pass: the state is
// read by every later step. The contract is documented in include/loglinear_attn.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "loglinear_attn.h"
#include "lla_bwd.hpp"
#include "lla_host.hpp"

namespace lla {
namespace prefill {

constexpr int kTile = 64;          // positions per tile
constexpr int kWaves = 4;
constexpr int kMaxLevels = 25;     // as the decoding step's cache
constexpr int kSeg = 256;          // positions per segment of a live level's block

struct Params {
  const void* k;
  const void* v;
  const float* log_a;
  float* state;     // [BH][Lc][dk][dv]
  float* lscale;    // [BH][2][Lc]
  float* scratch;   // [BH][nslot][dk][dv]: the segments of the blocks longer than kSeg
  int T, Lc, dv, nslot;
};

// segments of level l's block (2^(l-1) positions)
__host__ __device__ inline int seg_count(int l) { return l - 1 > 8 ? 1 << (l - 1 - 8) : 1; }
static_assert(kSeg == 1 << 8, "segments of 2^8 positions");

// item (>= 1) -> live level l, segment index, and the segment's scratch slot (-1: one segment,
// written to the level itself); levels in increasing order, each with its segments
__device__ inline void item_of(long long P, int item, int& l, int& seg, int& slot) {
  int base = 1, sbase = 0;
  for (l = 1; l < kMaxLevels; ++l) {
    if (!((P >> (l - 1)) & 1)) continue;
    const int ns = seg_count(l);
    if (item < base + ns) {
      seg = item - base;
      slot = ns > 1 ? sbase + seg : -1;
      return;
    }
    base += ns;
    if (ns > 1) sbase += ns;
  }
  l = 0; seg = 0; slot = -1;   // not reached for items of the launch
}

template <typename T, int DK, int DV>
__global__ void __launch_bounds__(64 * kWaves) prefill_kernel(Params p) {
  constexpr int NT = 64 * kWaves, ES = (int)sizeof(T), RK = DK + 16 / ES, RV = DV + 16 / ES;
  constexpr int AB = cdiv(DK / 16, kWaves), NB = DV / 16;
  __shared__ __attribute__((aligned(16))) T ks[kTile * RK];
  __shared__ __attribute__((aligned(16))) T vs[kTile * RV];
  __shared__ float wt[kTile];
  __shared__ float red[NT];
  const int bh = blockIdx.x, item = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, jj = lane & 15, g4 = lane >> 4;
  const long long P = (long long)p.T - 1;
  const size_t row0 = (size_t)bh * p.T;
  const T* kg = reinterpret_cast<const T*>(p.k) + row0 * DK;
  const T* vg = reinterpret_cast<const T*>(p.v) + row0 * DV;
  const float* lg = p.log_a + row0;
  float* ls = p.lscale + ((size_t)bh * 2 + (P & 1)) * p.Lc;
  if (item == 0) {
    // level 0: the factors of position P at parity P & 1; every log-scale of that parity is 0
    // (live levels are stored unscaled, the others are never read)
    float* f0 = p.state + (size_t)bh * p.Lc * DK * DV + (size_t)(P & 1) * (DK + DV);
    for (int i = tid; i < DK + DV; i += NT)
      f0[i] = i < DK ? (float)kg[(size_t)P * DK + i] : (float)vg[(size_t)P * DV + (i - DK)];
    for (int i = tid; i < p.Lc; i += NT) ls[i] = 0.f;
    return;
  }
  int l, seg, slot;
  item_of(P, item, l, seg, slot);
  float* st = slot < 0 ? p.state + ((size_t)bh * p.Lc + l) * DK * DV
                       : p.scratch + ((size_t)bh * p.nslot + slot) * DK * DV;
  // the segment [b0, bend) of the block [(P >> l) << l, + 2^(l-1))
  const long long n = 1LL << (l - 1), sn = n < kSeg ? n : kSeg;
  const long long b0 = ((P >> l) << l) + seg * sn, bend = b0 + sn;

  // R = sum of log_a over (end of the current tile, P]: first over [bend, P], in a fixed order
  float part = 0.f;
  for (long long r = bend + tid; r <= P; r += NT) part += lg[r];
  red[tid] = part;
  __syncthreads();
  float R = 0.f;
  for (int i = 0; i < NT; ++i) R += red[i];

  f32x4 acc[AB][NB];
#pragma unroll
  for (int x = 0; x < AB; ++x)
#pragma unroll
    for (int y = 0; y < NB; ++y) acc[x][y] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (long long t1 = bend; t1 > b0; t1 -= kTile) {
    const long long t0 = t1 - kTile > b0 ? t1 - kTile : b0;
    const int m = (int)(t1 - t0);               // positions in this tile, rows [0, m)
    __syncthreads();                            // the previous tile is no longer read
    constexpr int EPV = 16 / ES;
    for (int idx = tid; idx < kTile * (DK / EPV); idx += NT) {
      const int r = idx / (DK / EPV), c = (idx % (DK / EPV)) * EPV;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (r < m) x = *reinterpret_cast<const u32x4*>(kg + (size_t)(t0 + r) * DK + c);
      *reinterpret_cast<u32x4*>(ks + r * RK + c) = x;
    }
    for (int idx = tid; idx < kTile * (DV / EPV); idx += NT) {
      const int r = idx / (DV / EPV), c = (idx % (DV / EPV)) * EPV;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (r < m) x = *reinterpret_cast<const u32x4*>(vg + (size_t)(t0 + r) * DV + c);
      *reinterpret_cast<u32x4*>(vs + r * RV + c) = x;
    }
    // weights exp(R + sum of log_a over (s, t1 - 1]) by a suffix scan in wave 0
    if (w == 0) {
      const float x = lane < m - 1 ? lg[t0 + lane + 1] : 0.f;   // log_a[s + 1] for row s = lane
      float suf = x;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const float y = __shfl_down(suf, d);
        if (lane + d < 64) suf += y;
      }
      wt[lane] = lane < m ? __expf(R + suf) : 0.f;
      // the next tile ends where this one starts: add this tile's log_a[t0 + 1 .. t1 - 1]
      // and log_a[t0] (the decay from t0 - 1 to t0)
      const float tot = __shfl(suf, 0) + lg[t0];
      if (lane == 0) red[0] = tot;
    }
    __syncthreads();
    R += red[0];
#pragma unroll
    for (int x = 0; x < AB; ++x) {
      const int ab = w + kWaves * x;
      if (ab >= DK / 16) break;
#pragma unroll
      for (int y = 0; y < NB; ++y)
#pragma unroll
        for (int s0 = 0; s0 < kTile; s0 += 32) {
          const Frag<T> a = bwd::frag_col<T, kTile>(ks, RK, s0 + 8 * g4, ab * 16 + jj);
          Frag<T> bhi, blo;
          bwd::frag_col_split<T, kTile>(vs, RV, s0 + 8 * g4, y * 16 + jj, wt, bhi, blo);
          mma(acc[x][y], a, bhi);
          if constexpr (ES == 2) mma(acc[x][y], a, blo);
        }
    }
  }
#pragma unroll
  for (int x = 0; x < AB; ++x) {
    const int ab = w + kWaves * x;
    if (ab >= DK / 16) break;
#pragma unroll
    for (int y = 0; y < NB; ++y)
#pragma unroll
      for (int r = 0; r < 4; ++r) st[(size_t)(ab * 16 + 4 * g4 + r) * DV + y * 16 + jj] = acc[x][y][r];
  }
}

// the segments of every block longer than kSeg, added in segment order: one workgroup per (head,
// such level), 16-byte pieces of the state per thread
template <int DK, int DV>
__global__ void __launch_bounds__(256) prefill_reduce_kernel(Params p) {
  const int bh = blockIdx.x;
  const long long P = (long long)p.T - 1;
  int m = blockIdx.y, l = 1, sbase = 0;
  for (; l < kMaxLevels; ++l) {          // the m-th live level with more than one segment
    if (!((P >> (l - 1)) & 1) || seg_count(l) == 1) continue;
    if (m-- == 0) break;
    sbase += seg_count(l);
  }
  const int ns = seg_count(l);
  const f32x4* src = reinterpret_cast<const f32x4*>(p.scratch + ((size_t)bh * p.nslot + sbase) * DK * DV);
  f32x4* dst = reinterpret_cast<f32x4*>(p.state + ((size_t)bh * p.Lc + l) * DK * DV);
  for (int i = threadIdx.x; i < DK * DV / 4; i += 256) {
    f32x4 acc = src[i];
    for (int s = 1; s < ns; ++s) acc += src[(size_t)s * (DK * DV / 4) + i];
    dst[i] = acc;
  }
}

template <typename T, int DK>
const void* pick_dv(int dv) {
  switch (dv) {
    case 16: return reinterpret_cast<const void*>(&prefill_kernel<T, DK, 16>);
    case 32: return reinterpret_cast<const void*>(&prefill_kernel<T, DK, 32>);
    case 64: return reinterpret_cast<const void*>(&prefill_kernel<T, DK, 64>);
    case 128: return reinterpret_cast<const void*>(&prefill_kernel<T, DK, 128>);
  }
  return nullptr;
}

template <typename T>
const void* pick(int dk, int dv) {
  switch (dk) {
    case 16: return pick_dv<T, 16>(dv);
    case 32: return pick_dv<T, 32>(dv);
    case 64: return pick_dv<T, 64>(dv);
    case 128: return pick_dv<T, 128>(dv);
  }
  return nullptr;
}

template <int DK>
const void* pick_reduce_dv(int dv) {
  switch (dv) {
    case 16: return reinterpret_cast<const void*>(&prefill_reduce_kernel<DK, 16>);
    case 32: return reinterpret_cast<const void*>(&prefill_reduce_kernel<DK, 32>);
    case 64: return reinterpret_cast<const void*>(&prefill_reduce_kernel<DK, 64>);
    case 128: return reinterpret_cast<const void*>(&prefill_reduce_kernel<DK, 128>);
  }
  return nullptr;
}
const void* pick_reduce(int dk, int dv) {
  switch (dk) {
    case 16: return pick_reduce_dv<16>(dv);
    case 32: return pick_reduce_dv<32>(dv);
    case 64: return pick_reduce_dv<64>(dv);
    case 128: return pick_reduce_dv<128>(dv);
  }
  return nullptr;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

}  // namespace prefill
}  // namespace lla

extern "C" int loglinear_attn_decode_prefill(const lla_prefill_args* a, lla_stream_t stream) {
  using namespace lla::prefill;
  if (!a) return LLA_ERR_INVALID_ARG;
  if (a->B < 0 || a->H < 0 || a->T < 1 || a->Lc < 1) return LLA_ERR_INVALID_ARG;
  if (a->dtype != LLA_DTYPE_BF16 && a->dtype != LLA_DTYPE_F32) return LLA_ERR_UNSUPPORTED;
  const void* fn = a->dtype == LLA_DTYPE_BF16 ? pick<lla::bf16>(a->dk, a->dv) : pick<float>(a->dk, a->dv);
  if (!fn) return LLA_ERR_UNSUPPORTED;
  if (a->Lc > kMaxLevels) return LLA_ERR_UNSUPPORTED;
  // the first step after the prompt is at position T: levels 0 .. bit_length(T) are needed
  int need = 1;
  for (long long t = a->T; t; t >>= 1) ++need;
  if (need > a->Lc) return LLA_ERR_INVALID_ARG;
  const long long BH = (long long)a->B * a->H;
  if (BH == 0) return LLA_OK;
  if (BH > 0x7fffffffLL) return LLA_ERR_UNSUPPORTED;
  if (!a->k || !a->v || !a->log_a || !a->state || !a->log_scale) return LLA_ERR_INVALID_ARG;
  if (((uintptr_t)a->k | (uintptr_t)a->v) & 15) return LLA_ERR_INVALID_ARG;
  if (((uintptr_t)a->log_a | (uintptr_t)a->state | (uintptr_t)a->log_scale) & 3) return LLA_ERR_INVALID_ARG;
  const size_t es = a->dtype == LLA_DTYPE_BF16 ? 2 : 4;
  const size_t nk = (size_t)BH * a->T * a->dk * es, nv = (size_t)BH * a->T * a->dv * es;
  const size_t nla = (size_t)BH * a->T * 4;
  const size_t nst = (size_t)BH * a->Lc * a->dk * a->dv * 4, nls = (size_t)BH * 2 * a->Lc * 4;
  const void* ins[] = {a->k, a->v, a->log_a};
  const size_t nin[] = {nk, nv, nla};
  for (int i = 0; i < 3; ++i)
    if (overlaps(a->state, nst, ins[i], nin[i]) || overlaps(a->log_scale, nls, ins[i], nin[i]))
      return LLA_ERR_INVALID_ARG;
  if (overlaps(a->state, nst, a->log_scale, nls)) return LLA_ERR_INVALID_ARG;
  Params p;
  memset(&p, 0, sizeof(p));
  p.k = a->k; p.v = a->v; p.log_a = a->log_a; p.state = a->state; p.lscale = a->log_scale;
  p.T = a->T; p.Lc = a->Lc; p.dv = a->dv;
  // items: level 0, then the segments of each live level; scratch slots for the blocks of more
  // than one segment
  const long long P = a->T - 1;
  int items = 1, multi = 0;
  for (int l = 1; l < kMaxLevels && (P >> (l - 1)); ++l) {
    if (!((P >> (l - 1)) & 1)) continue;
    items += seg_count(l);
    if (seg_count(l) > 1) {
      p.nslot += seg_count(l);
      ++multi;
    }
  }
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  void* scratch = nullptr;
  if (p.nslot > 0) {
    if (lla::workspace_alloc(&scratch, (size_t)BH * p.nslot * a->dk * a->dv * 4, s) != hipSuccess)
      return LLA_ERR_NO_MEMORY;
    p.scratch = static_cast<float*>(scratch);
  }
  void* args[] = {&p};
  int st = LLA_OK;
  if (hipLaunchKernel(fn, dim3((unsigned)BH, (unsigned)items), dim3(64 * kWaves), args, 0, s) != hipSuccess)
    st = LLA_ERR_HIP;
  if (st == LLA_OK && multi > 0) {
    const void* red = pick_reduce(a->dk, a->dv);
    if (!red || hipLaunchKernel(red, dim3((unsigned)BH, (unsigned)multi), dim3(256), args, 0, s) != hipSuccess)
      st = LLA_ERR_HIP;
  }
  if (scratch && hipFreeAsync(scratch, s) != hipSuccess && st == LLA_OK) st = LLA_ERR_HIP;
  return st;
}
