// lla_decode.hip — one decoding step of log-linear Mamba-2 attention: the recurrent form with one
// dk x dv state per Fenwick level ("Log-Linear Attention", arXiv 2506.04761; study notes
// dimensionstp.github.io/study-concept/log_linear_attention, sections 2-2 and 3-6: states per
// power-of-two bucket, merged like a carry when the lower buckets fill; gist.science zh lay
// summary, the "drawer" merging). The contract is documented in include/loglinear_attn.h.
//
// Step t (c = ctz(t) for t > 0): the states of levels 0..c after t-1 are merged into level c+1,
// every state is multiplied by a_t = exp(log_a_t), level 0 becomes k_t v_t^T, and
//   o_t = sum_l lambda_t[l] S_l^T q_t   over the levels live after t
// (level 0, and level j+1 for each set bit j of t).
//
// Cache layout (fp32): state[b][h][l][dk][dv] holds level l >= 1 up to a scale,
// S_l = state[b][h][l] * exp(log_scale[b][h][t & 1][l]), so the per-step multiplication by a_t
// touches Lc scalars instead of every state; level 0 is rank one and state[b][h][0] keeps its
// factors, (k, v) of the last even position in floats [0, dk+dv) and of the last odd one in
// [dk+dv, 2(dk+dv)). Both parities exist so that the workgroups of one head, which split the
// value columns, read step t-1's factors and scales while step t's are written elsewhere.
// A level is read only while it is live (the bits of t say which), so the cache never needs
// clearing. Level c+1 is not live after t-1 (bit c of t-1 is clear), so writing the merged
// state there races with no read.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include <stdint.h>
#include <string.h>

#include "loglinear_attn.h"

namespace lla_decode {

constexpr int kMaxLevels = 25;   // state levels a cache may have (positions below 2^24)
constexpr int kCols = 16;        // value columns per workgroup

template <typename T> __device__ __forceinline__ float to_f32(T x);
template <> __device__ __forceinline__ float to_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ float to_f32<__hip_bfloat16>(__hip_bfloat16 x) { return __bfloat162float(x); }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ __hip_bfloat16 from_f32<__hip_bfloat16>(float x) { return __float2bfloat16(x); }

struct Params {
  const void* q; const void* k; const void* v;
  const float* log_a; const float* lam;
  void* out;
  float* state; float* lscale;
  int dv, Lc, H;
  long long t;                 // the position of every (b, h), or the largest one when t_seq is set
  const long long* t_seq;      // per-sequence positions [B] (device), or null
};

// Row groups: thread (rg, col) owns rows rg*RG .. rg*RG+RG-1 of column 16*blockIdx.y + col.
template <int DK> constexpr int row_groups() { return DK >= 64 ? 32 : 16; }

template <typename T, int DK>
__global__ __launch_bounds__(kCols * row_groups<DK>()) void lla_decode_kernel(Params p) {
  constexpr int NRG = row_groups<DK>(), RG = DK / NRG, NT = kCols * NRG;
  const int tid = threadIdx.x;
  const int col = tid % kCols, rg = tid / kCols;
  const int bh = blockIdx.x, cb = blockIdx.y;
  const int dv = p.dv, Lc = p.Lc;
  const int vc = cb * kCols + col;
  // this sequence's position: a negative one takes no step (nothing is read or written); one past
  // the largest the call declared (the cache was sized for) writes NaN and leaves the cache alone
  const long long t = p.t_seq ? p.t_seq[bh / p.H] : p.t;
  if (t < 0) return;
  if (t > p.t) {
    if (tid < kCols) reinterpret_cast<T*>(p.out)[(size_t)bh * dv + cb * kCols + tid] = from_f32<T>(__builtin_nanf(""));
    return;
  }
  const int par = (int)(t & 1);

  __shared__ float qs[DK], ks[DK], lam[kMaxLevels], sig[kMaxLevels], red[NRG][kCols];
  const T* qg = reinterpret_cast<const T*>(p.q) + (size_t)bh * DK;
  const T* kg = reinterpret_cast<const T*>(p.k) + (size_t)bh * DK;
  const T* vg = reinterpret_cast<const T*>(p.v) + (size_t)bh * dv;
  float* st = p.state + (size_t)bh * Lc * DK * dv;
  float* ls = p.lscale + (size_t)bh * 2 * Lc;

  // The live levels of t-1 (which depend on t alone) are loaded first, together with the
  // token's vectors: one memory round trip per step.
  const long long tm = t - 1;
  const int c = t > 0 ? __builtin_ctzll((unsigned long long)t) : 0;
  const int top = t > 1 ? 64 - __builtin_clzll((unsigned long long)tm) : 0;   // bit_length(t-1)
  float X[kMaxLevels - 1][RG];
#pragma unroll
  for (int l = 1; l < kMaxLevels; ++l) {
    if (l <= top && ((tm >> (l - 1)) & 1)) {
      const float* sl = st + ((size_t)l * DK + rg * RG) * dv + vc;
#pragma unroll
      for (int i = 0; i < RG; ++i) X[l - 1][i] = sl[(size_t)i * dv];
    }
  }
  float F0[RG], vprev = 0.f;          // level 0 after t-1: rank one, factors of parity 1 - par
  if (t > 0) {
    const float* f0 = st + (size_t)(1 - par) * (DK + dv);
    vprev = f0[DK + vc];
#pragma unroll
    for (int i = 0; i < RG; ++i) F0[i] = f0[rg * RG + i];
  }
  if (tid < DK) {
    qs[tid] = to_f32<T>(qg[tid]);
    ks[tid] = to_f32<T>(kg[tid]);
  }
  if (tid < Lc) {
    lam[tid] = p.lam[(size_t)bh * Lc + tid];
    sig[tid] = t > 0 ? ls[(1 - par) * Lc + tid] : 0.f;
  }
  const float la = p.log_a[bh];
  const float v_t = to_f32<T>(vg[vc]);
  __syncthreads();

  float part = 0.f;                          // this thread's rows of sum_l w_l S_l^T q
  if (t > 0) {
    float M[RG];
#pragma unroll
    for (int i = 0; i < RG; ++i) M[i] = __expf(sig[0]) * F0[i] * vprev;
    // live levels 1..top of t-1; 1..c merge into c+1, the ones above c+1 are read out
#pragma unroll
    for (int l = 1; l < kMaxLevels; ++l) {
      if (l <= top && ((tm >> (l - 1)) & 1)) {
        if (l <= c) {
          const float e = __expf(sig[l]);
#pragma unroll
          for (int i = 0; i < RG; ++i) M[i] += e * X[l - 1][i];
        } else {
          float y = 0.f;
#pragma unroll
          for (int i = 0; i < RG; ++i) y += X[l - 1][i] * qs[rg * RG + i];
          part += lam[l] * __expf(sig[l] + la) * y;
        }
      }
    }
    // merged state: level c+1, scale a_t (its log-scale becomes log_a_t below)
    float ym = 0.f;
    float* sm = st + ((size_t)(c + 1) * DK + rg * RG) * dv + vc;
#pragma unroll
    for (int i = 0; i < RG; ++i) {
      sm[(size_t)i * dv] = M[i];
      ym += M[i] * qs[rg * RG + i];
    }
    part += lam[c + 1] * __expf(la) * ym;
  }
  red[rg][col] = part;
  __syncthreads();

  if (rg == 0) {
    float o = 0.f;
#pragma unroll
    for (int g = 0; g < NRG; ++g) o += red[g][col];
    float qk = 0.f;
#pragma unroll
    for (int r = 0; r < DK; ++r) qk += qs[r] * ks[r];
    o += lam[0] * qk * v_t;
    reinterpret_cast<T*>(p.out)[(size_t)bh * dv + vc] = from_f32<T>(o);
    st[(size_t)par * (DK + dv) + DK + vc] = v_t;     // level-0 factors of step t
  }
  if (cb == 0) {
    if (tid < DK) st[(size_t)par * (DK + dv) + tid] = ks[tid];
    if (tid < Lc) {
      // log-scales after t: level 0 fresh, level c+1 just merged, the others decay by a_t
      const int cm = t > 0 ? c : -1;
      ls[par * Lc + tid] = tid == 0 ? 0.f : tid == cm + 1 ? la : sig[tid] + la;
    }
  }
}

template <typename T, int DK>
hipError_t launch_dk(const Params& p, int BH, hipStream_t stream) {
  constexpr int NT = kCols * row_groups<DK>();
  Params q = p;
  void* args[] = {&q};
  return hipLaunchKernel(reinterpret_cast<const void*>(&lla_decode_kernel<T, DK>),
                         dim3((unsigned)BH, (unsigned)(p.dv / kCols)), dim3(NT), args, 0, stream);
}

template <typename T>
hipError_t launch(const Params& p, int BH, int dk, hipStream_t stream) {
  switch (dk) {
    case 16: return launch_dk<T, 16>(p, BH, stream);
    case 32: return launch_dk<T, 32>(p, BH, stream);
    case 64: return launch_dk<T, 64>(p, BH, stream);
    default: return launch_dk<T, 128>(p, BH, stream);
  }
}

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

}  // namespace lla_decode

extern "C" int loglinear_attn_decode_step(const lla_decode_args* a, lla_stream_t stream) {
  using namespace lla_decode;
  if (!a) return LLA_ERR_INVALID_ARG;
  if (a->B < 0 || a->H < 0 || a->t < 0 || a->Lc < 1) return LLA_ERR_INVALID_ARG;
  if (a->dtype != LLA_DTYPE_BF16 && a->dtype != LLA_DTYPE_F32) return LLA_ERR_UNSUPPORTED;
  if (!dim_ok(a->dk) || !dim_ok(a->dv)) return LLA_ERR_UNSUPPORTED;
  if (a->Lc > kMaxLevels) return LLA_ERR_UNSUPPORTED;
  // levels live after t: 0 .. bit_length(t)
  const int need = (a->t > 0 ? 64 - __builtin_clzll((unsigned long long)a->t) : 0) + 1;
  if (need > a->Lc) return LLA_ERR_INVALID_ARG;
  const long long BH = (long long)a->B * a->H;
  if (BH == 0) return LLA_OK;
  if (BH > 0x7fffffffLL) return LLA_ERR_UNSUPPORTED;
  if (!a->q || !a->k || !a->v || !a->log_a || !a->lambda || !a->out || !a->state || !a->log_scale)
    return LLA_ERR_INVALID_ARG;
  if ((uintptr_t)a->t_seq % 8) return LLA_ERR_INVALID_ARG;
  const size_t es = a->dtype == LLA_DTYPE_BF16 ? 2 : 4;
  const void* eptr[] = {a->q, a->k, a->v, a->out};
  for (const void* x : eptr)
    if ((uintptr_t)x % es) return LLA_ERR_INVALID_ARG;                 // element alignment
  const void* fptr[] = {a->log_a, a->lambda, a->state, a->log_scale};
  for (const void* x : fptr)
    if ((uintptr_t)x % 4) return LLA_ERR_INVALID_ARG;
  const size_t n_out = (size_t)BH * a->dv * es;
  const size_t n_state = (size_t)BH * a->Lc * a->dk * a->dv * 4, n_ls = (size_t)BH * 2 * a->Lc * 4;
  const void* ins[] = {a->q, a->k, a->v, a->log_a, a->lambda};
  const size_t nin[] = {(size_t)BH * a->dk * es, (size_t)BH * a->dk * es, (size_t)BH * a->dv * es,
                        (size_t)BH * 4, (size_t)BH * a->Lc * 4};
  for (int i = 0; i < 5; ++i)
    if (overlaps(a->out, n_out, ins[i], nin[i]) || overlaps(a->state, n_state, ins[i], nin[i]) ||
        overlaps(a->log_scale, n_ls, ins[i], nin[i]))
      return LLA_ERR_INVALID_ARG;
  if (overlaps(a->out, n_out, a->state, n_state) || overlaps(a->out, n_out, a->log_scale, n_ls) ||
      overlaps(a->state, n_state, a->log_scale, n_ls))
    return LLA_ERR_INVALID_ARG;

  Params p;
  memset(&p, 0, sizeof(p));
  p.q = a->q; p.k = a->k; p.v = a->v; p.log_a = a->log_a; p.lam = a->lambda; p.out = a->out;
  p.state = a->state; p.lscale = a->log_scale;
  p.dv = a->dv; p.Lc = a->Lc; p.t = a->t; p.H = a->H;
  p.t_seq = a->t_seq;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = a->dtype == LLA_DTYPE_BF16 ? launch<__hip_bfloat16>(p, (int)BH, a->dk, s)
                                                  : launch<float>(p, (int)BH, a->dk, s);
  return e == hipSuccess ? LLA_OK : LLA_ERR_HIP;
}
