// lla_bwd_api.hip — C ABI of the backward pass: argument validation, plan (chunk, tree and
// workspace layout) and the stream-ordered launch sequence bwd_states -> bwd_rn -> bwd_gsum ->
// bwd_tree -> bwd_grads -> bwd_dloga. The contract is documented in include/loglinear_attn.h.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include "loglinear_attn.h"
#include "lla_bwd.hpp"
#include "lla_host.hpp"

namespace lla {
namespace bwd {

// ----------------------------------------------------------------------------------------
// bwd_gsum: total log decay of every block (one workgroup per head)
// ----------------------------------------------------------------------------------------

__global__ void __launch_bounds__(256) bwd_gsum_kernel(BwdParams p) {
  const int bh = blockIdx.x;
  float* gs = p.gsum + (size_t)bh * p.nslot;
  for (int i = 1; i < p.nl; ++i) {
    const int nprev = (p.N + (1 << (i - 1)) - 1) >> (i - 1), nb = (p.N + (1 << i) - 1) >> i;
    const int o_prev = slot_of(p.N, i - 1, 0), o = slot_of(p.N, i, 0);
    for (int m = threadIdx.x; m < nb; m += blockDim.x) {
      const float l = gs[o_prev + 2 * m];
      gs[o + m] = 2 * m + 1 < nprev ? l + gs[o_prev + 2 * m + 1] : l;
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------------------
// bwd_tree: 64 state elements of one head per workgroup, 16 waves splitting the blocks of a level.
//   up-sweep, levels i = 1 .. nl-1: node(i,m) = exp(G(i-1,2m+1)) node(i-1,2m) + node(i-1,2m+1).
//   down-sweep, levels i = nl-1 .. 0: Out(i, m) = what the chunks of block (i, m) receive from
//     later blocks at levels >= i, decayed to the end of (i, m):
//       left child with a right sibling Y: Out = exp(G(Y)) Out(parent) + RN(i, Y), RN(i, Y) the
//       sum of Y's sub-block states (bwd_rn), each decayed over the sub-blocks before it;
//       otherwise: Out = Out(parent); the parent of the top level holds nothing.
//     Out(0, c) is the combined right-sibling state of chunk c.
// ----------------------------------------------------------------------------------------

constexpr int kTreeWaves = 16;

// LDS: every block value of the 64 elements, [slot][64] floats (up-sweep nodes, then the
// down-sweep's values), when that fits; otherwise the up-sweep reads level i-1 back from the
// node array and the down-sweep keeps every level in the outs array.
// E: the element type of the copies the gradient kernel reads (node_e, u_e)
template <typename E, bool LDS>
__global__ void __launch_bounds__(64 * kTreeWaves) bwd_tree_kernel(BwdParams p, int SZ) {
  extern __shared__ __attribute__((aligned(16))) float tl[];
  const int bh = blockIdx.y, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 64 + lane, w = threadIdx.x >> 6;
  // the grid has exactly SZ / 64 columns of workgroups (SZ = dk*dv is a multiple of 64)
  const float* __restrict__ gsg = p.gsum + (size_t)bh * p.nslot;
  // on chip, the block decays sit after the block values: no level waits on a decay load
  float* gsl = tl + (size_t)p.nslot * 64;
  if (LDS)
    for (int i = threadIdx.x; i < p.nslot; i += blockDim.x) gsl[i] = gsg[i];
  const float* gs = LDS ? gsl : gsg;
  // on chip the waves exchange values through shared memory only: the barrier then waits for
  // shared-memory accesses alone, and the loads issued ahead for the next level stay in flight
  auto bar = [&]() {
    if (LDS) lds_barrier();
    else __syncthreads();
  };
  float* __restrict__ nd = p.node + (size_t)bh * p.nslot * SZ + e;
  const float* __restrict__ rp = p.rnp + (size_t)bh * p.items * SZ + e;
  float* __restrict__ ou = p.outs + (size_t)bh * p.nslot * SZ + e;
  E* __restrict__ ne = reinterpret_cast<E*>(p.node_e) + (size_t)bh * p.nslot * SZ + e;
  E* __restrict__ ue = reinterpret_cast<E*>(p.u_e) + (size_t)bh * p.N * SZ + e;
  // bf16 copies also keep their low parts, x - bf16(x)
  constexpr bool SPLIT = sizeof(E) == 2;
  E* __restrict__ nlo = reinterpret_cast<E*>(p.node_lo) + (size_t)bh * p.nslot * SZ + e;
  E* __restrict__ ulo = reinterpret_cast<E*>(p.u_lo) + (size_t)bh * p.N * SZ + e;
  auto put = [&](E* hi, E* lo, size_t at, float x) {
    const E h = (E)x;
    hi[at] = h;
    if (SPLIT) lo[at] = (E)(x - (float)h);
  };
  for (int m = w; m < p.N; m += kTreeWaves) {
    const float x = nd[(size_t)m * SZ];
    // the gradient kernel reads node (j, (c >> j) - 1) for set bits j of c: even nodes only
    if (!(m & 1)) put(ne, nlo, (size_t)m * SZ, x);
    if (LDS) tl[m * 64 + lane] = x;
  }
  bar();
  for (int i = 1; i < p.nl; ++i) {
    const int nprev = (p.N + (1 << (i - 1)) - 1) >> (i - 1), nb = (p.N + (1 << i) - 1) >> i;
    const int o_prev = slot_of(p.N, i - 1, 0), o = slot_of(p.N, i, 0);
    for (int m = w; m < nb; m += kTreeWaves) {
      const bool right = 2 * m + 1 < nprev;
      const int sl = o_prev + 2 * m;
      const float lhs = LDS ? tl[sl * 64 + lane] : nd[(size_t)sl * SZ];
      const float rhs = right ? (LDS ? tl[(sl + 1) * 64 + lane] : nd[(size_t)(sl + 1) * SZ]) : 0.f;
      const float gr = right ? gs[sl + 1] : 0.f;
      const float val = right ? __expf(gr) * lhs + rhs : lhs;
      if (!(m & 1)) put(ne, nlo, (size_t)(o + m) * SZ, val);
      if (LDS) tl[(o + m) * 64 + lane] = val;
      else nd[(size_t)(o + m) * SZ] = val;
    }
    bar();
  }
  // down-sweep; a wave takes KB of its blocks at a time and loads all their right-block states
  // before it uses any of them; the first KB of the next level are loaded while this level is
  // worked on (they depend on nothing the sweep writes)
  constexpr int KB = 8;
  auto fetch = [&](int i, int m0, float (&rn)[KB]) {
    const int nb = (p.N + (1 << i) - 1) >> i;
    const int s = sub_log(i), b = i - s, os = slot_of(p.N, s, 0);
    const int nsub = (p.N + (1 << s) - 1) >> s;
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int m = m0 + u * kTreeWaves;
      rn[u] = 0.f;
      if (m < nb && !(m & 1) && m + 1 < nb) {
        const int sb0 = (m + 1) << b, sb1 = min((m + 2) << b, nsub);
        if (sb1 - sb0 == 1) {
          rn[u] = rp[(size_t)(p.rn_off[i] + item_of_sub(i, sb0)) * SZ];
        } else {
          float dec = 0.f;
          for (int sb = sb0; sb < sb1; ++sb) {
            rn[u] += __expf(dec) * rp[(size_t)(p.rn_off[i] + item_of_sub(i, sb)) * SZ];
            dec += gs[os + sb];
          }
        }
      }
    }
  };
  float rn_next[KB];
  if (p.nl > 0) fetch(p.nl - 1, w, rn_next);
  for (int i = p.nl - 1; i >= 0; --i) {
    float rn_first[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) rn_first[u] = rn_next[u];
    if (i > 0) fetch(i - 1, w, rn_next);
    const int nb = (p.N + (1 << i) - 1) >> i;
    const int o = slot_of(p.N, i, 0);
    const bool top = i + 1 >= p.nl;
    const int op = top ? 0 : slot_of(p.N, i + 1, 0);
    for (int m0 = w; m0 < nb; m0 += kTreeWaves * KB) {
      float rn[KB];
      if (m0 == w) {
#pragma unroll
        for (int u = 0; u < KB; ++u) rn[u] = rn_first[u];
      } else {
        fetch(i, m0, rn);
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int m = m0 + u * kTreeWaves;
        if (m >= nb) break;
        const int ps = op + (m >> 1);
        const float par = top ? 0.f : (LDS ? tl[ps * 64 + lane] : ou[(size_t)ps * SZ]);
        const float val = (!(m & 1) && m + 1 < nb) ? __expf(gs[o + m + 1]) * par + rn[u] : par;
        // the level-i slots of tl held nodes that are no longer read: level i+1 was read above,
        // and the up-sweep is over
        if (LDS) tl[(o + m) * 64 + lane] = val;
        else ou[(size_t)(o + m) * SZ] = val;
        if (i == 0) put(ue, ulo, (size_t)m * SZ, val);
      }
    }
    bar();
  }
}

// ----------------------------------------------------------------------------------------
// bwd_dloga: dlog_a[r] = sum_{t >= r} dA_t (one workgroup per head, fixed order)
// ----------------------------------------------------------------------------------------

__global__ void __launch_bounds__(256) bwd_dloga_kernel(BwdParams p) {
  __shared__ float part[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int per = (p.T + 255) / 256;
  const int lo = tid * per, hi = min(p.T, lo + per);
  const float* dA = p.dA + (size_t)bh * p.T;
  float* out = p.glog_a + (size_t)bh * p.T;
  float s = 0.f;
  for (int t = hi - 1; t >= lo; --t) s += dA[t];
  part[tid] = s;
  __syncthreads();
  // suffix of the segment sums: threads above this one
  if (tid == 0) {
    float run = 0.f;
    for (int u = 255; u >= 0; --u) {
      const float x = part[u];
      part[u] = run;
      run += x;
    }
  }
  __syncthreads();
  float run = part[tid];
  for (int t = hi - 1; t >= lo; --t) {
    run += dA[t];
    out[t] = run;
  }
}

}  // namespace bwd
}  // namespace lla

namespace {

using lla::bwd::BwdKernels;
using lla::bwd::BwdParams;

inline bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
inline int bit_len(unsigned x) { int n = 0; while (x) { ++n; x >>= 1; } return n; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kLdsPerWorkgroup = 160 * 1024;

struct BwdPlan {
  int C, N, nl, nslot, L, esize, smem_states, smem_grads, tree_smem;
  long BH;
  int items, rn_off[lla::kLamCap + 1];
  size_t off_node, off_gsum, off_rnp, off_outs, off_node_e, off_u_e, off_node_lo, off_u_lo, off_dA, ws_bytes;
};

const BwdKernels* bwd_kernels(int dtype, int C, int DK, int DV) {
  if (dtype == LLA_DTYPE_BF16) {
    switch (C) {
      case 16: return lla::bwd::bwd_kernels_bf16_c16(DK, DV);
      case 32: return lla::bwd::bwd_kernels_bf16_c32(DK, DV);
      case 64: return lla::bwd::bwd_kernels_bf16_c64(DK, DV);
    }
  } else if (dtype == LLA_DTYPE_F32) {
    switch (C) {
      case 16: return lla::bwd::bwd_kernels_f32_c16(DK, DV);
      case 32: return lla::bwd::bwd_kernels_f32_c32(DK, DV);
      case 64: return lla::bwd::bwd_kernels_f32_c64(DK, DV);
    }
  }
  return nullptr;
}

int grads_smem(int esize, int C, int dk, int dv) {
  return lla::bwd::bwd_smem(esize, C, dk, dv, true).total;
}

// 16 for head dims up to 16; otherwise the largest of 64, 32, 16 whose gradient kernel fits the
// shared memory of one workgroup
int bwd_default_chunk(int dk, int dv, int esize) {
  if (dk <= 16 && dv <= 16) return 16;
  for (int C = 64; C >= 16; C /= 2)
    if (grads_smem(esize, C, dk, dv) <= kLdsPerWorkgroup) return C;
  return 16;
}

int make_bwd_plan(int B, int H, int T, int dk, int dv, int chunk, int dtype, BwdPlan& pl) {
  if (dtype != LLA_DTYPE_BF16 && dtype != LLA_DTYPE_F32) return LLA_ERR_INVALID_ARG;
  if (B < 0 || H < 0 || T < 0) return LLA_ERR_INVALID_ARG;
  if (!supported_dim(dk) || !supported_dim(dv)) return LLA_ERR_UNSUPPORTED;
  if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64) return LLA_ERR_UNSUPPORTED;
  pl.esize = dtype == LLA_DTYPE_BF16 ? 2 : 4;
  const int C = chunk ? chunk : bwd_default_chunk(dk, dv, pl.esize);
  const long BH = (long)B * H;
  if (BH > 65535) return LLA_ERR_UNSUPPORTED;
  pl.C = C;
  pl.BH = BH;
  pl.L = T > 0 ? bit_len((unsigned)(T - 1)) + 1 : 0;
  if (pl.L > lla::kLamCap) return LLA_ERR_UNSUPPORTED;
  pl.N = (T + C - 1) / C;
  if ((long long)pl.N * BH > 0x7fffffffLL) return LLA_ERR_UNSUPPORTED;   // one workgroup per chunk
  pl.nl = pl.N > 1 ? bit_len((unsigned)(pl.N - 1)) : 0;
  pl.nslot = 0;
  for (int i = 0; i < (pl.nl > 0 ? pl.nl : 0); ++i) pl.nslot += (pl.N + (1 << i) - 1) >> i;
  const size_t SZ = (size_t)dk * dv;
  size_t off = 0;
  pl.off_node = off; off = align256(off + (size_t)BH * pl.nslot * SZ * 4);
  pl.off_gsum = off; off = align256(off + (size_t)BH * pl.nslot * 4);
  pl.items = 0;
  for (int j = 0; j <= lla::kLamCap; ++j) {
    pl.rn_off[j] = pl.items;
    if (j < pl.nl) pl.items += lla::bwd::items_of_level(pl.N, j);
  }
  if ((long long)pl.items * BH > 0x7fffffffLL) return LLA_ERR_UNSUPPORTED;   // one workgroup each
  pl.off_rnp = off;  off = align256(off + (size_t)BH * pl.items * SZ * 4);
  // the tree keeps its block values in shared memory when they fit: then the fp32 nodes above
  // level 0 and the down-sweep's values never reach memory (the node region is still laid out
  // per head with every slot; the outs region is not needed)
  pl.tree_smem = (size_t)pl.nslot * 65 * 4 <= (size_t)kLdsPerWorkgroup ? pl.nslot * 65 * 4 : 0;
  pl.off_outs = off; off = align256(off + (pl.tree_smem ? 0 : (size_t)BH * pl.nslot * SZ * 4));
  pl.off_node_e = off; off = align256(off + (size_t)BH * pl.nslot * SZ * pl.esize);
  pl.off_u_e = off;  off = align256(off + (pl.nl > 0 ? (size_t)BH * pl.N * SZ * pl.esize : 0));
  const bool split = dtype == LLA_DTYPE_BF16;   // bf16 copies keep their low parts
  pl.off_node_lo = off; off = align256(off + (split ? (size_t)BH * pl.nslot * SZ * pl.esize : 0));
  pl.off_u_lo = off; off = align256(off + (split && pl.nl > 0 ? (size_t)BH * pl.N * SZ * pl.esize : 0));
  pl.off_dA = off;   off = align256(off + (size_t)BH * T * 4);
  pl.ws_bytes = off;
  pl.smem_states = lla::bwd::bwd_smem(pl.esize, C, dk, dv, false).total;
  pl.smem_grads = grads_smem(pl.esize, C, dk, dv);
  if (pl.smem_grads > kLdsPerWorkgroup) return LLA_ERR_UNSUPPORTED;
  return LLA_OK;
}

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return na && nb && x < y + nb && y < x + na;
}

int validate(const lla_bwd_args& a, const BwdPlan& pl) {
  if (!a.q || !a.k || !a.v || !a.log_a || !a.lambda || !a.grad_out || !a.grad_q || !a.grad_k ||
      !a.grad_v || !a.grad_log_a || !a.grad_lambda)
    return LLA_ERR_INVALID_ARG;
  if (a.lambda_bf16 != 0 && a.lambda_bf16 != 1) return LLA_ERR_INVALID_ARG;
  const size_t es = (size_t)pl.esize, nt = (size_t)pl.BH * a.T;
  const size_t nq = nt * a.dk * es, nv = nt * a.dv * es, nla = nt * 4, nlam = nt * pl.L * 4;
  const size_t nlam_in = nt * pl.L * (a.lambda_bf16 ? 2 : 4);
  if (((uintptr_t)a.q | (uintptr_t)a.k | (uintptr_t)a.v | (uintptr_t)a.grad_out |
       (uintptr_t)a.grad_q | (uintptr_t)a.grad_k | (uintptr_t)a.grad_v) & 15)
    return LLA_ERR_INVALID_ARG;
  if (((uintptr_t)a.log_a | (uintptr_t)a.grad_log_a | (uintptr_t)a.grad_lambda) & 3)
    return LLA_ERR_INVALID_ARG;
  if ((uintptr_t)a.lambda & (a.lambda_bf16 ? 1 : 3)) return LLA_ERR_INVALID_ARG;
  const void* in[6] = {a.q, a.k, a.v, a.log_a, a.lambda, a.grad_out};
  const size_t nin[6] = {nq, nq, nv, nla, nlam_in, nv};
  const void* out[5] = {a.grad_q, a.grad_k, a.grad_v, a.grad_log_a, a.grad_lambda};
  const size_t nout[5] = {nq, nq, nv, nla, nlam};
  for (int o = 0; o < 5; ++o) {
    for (int i = 0; i < 6; ++i)
      if (overlaps(out[o], nout[o], in[i], nin[i])) return LLA_ERR_INVALID_ARG;
    for (int o2 = o + 1; o2 < 5; ++o2)
      if (overlaps(out[o], nout[o], out[o2], nout[o2])) return LLA_ERR_INVALID_ARG;
  }
  return LLA_OK;
}

hipError_t set_smem(const void* fn, int bytes) {
  return bytes > 65536 ? hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes)
                       : hipSuccess;
}

int launch_bwd(const lla_bwd_args& a, const BwdPlan& pl, void* ws, hipStream_t stream) {
  const BwdKernels* ks = bwd_kernels(a.dtype, pl.C, a.dk, a.dv);
  if (!ks) return LLA_ERR_UNSUPPORTED;
  int dev = 0, max_smem = 0;
  if (hipGetDevice(&dev) != hipSuccess) return LLA_ERR_HIP;
  if (hipDeviceGetAttribute(&max_smem, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess)
    return LLA_ERR_HIP;
  if (pl.smem_grads > max_smem) return LLA_ERR_UNSUPPORTED;

  BwdParams p;
  memset(&p, 0, sizeof(p));
  p.q = a.q; p.k = a.k; p.v = a.v; p.dout = a.grad_out; p.log_a = a.log_a; p.lam = a.lambda;
  p.lam_bf16 = a.lambda_bf16;
  p.gq = a.grad_q; p.gk = a.grad_k; p.gv = a.grad_v; p.glog_a = a.grad_log_a; p.glam = a.grad_lambda;
  char* w = static_cast<char*>(ws);
  p.node = reinterpret_cast<float*>(w + pl.off_node);
  p.gsum = reinterpret_cast<float*>(w + pl.off_gsum);
  p.rnp = reinterpret_cast<float*>(w + pl.off_rnp);
  p.items = pl.items;
  for (int j = 0; j <= lla::kLamCap; ++j) p.rn_off[j] = pl.rn_off[j];
  p.outs = reinterpret_cast<float*>(w + pl.off_outs);
  p.node_e = w + pl.off_node_e;
  p.u_e = w + pl.off_u_e;
  p.node_lo = w + pl.off_node_lo;
  p.u_lo = w + pl.off_u_lo;
  p.dA = reinterpret_cast<float*>(w + pl.off_dA);
  p.BH = (int)pl.BH; p.T = a.T; p.L = pl.L; p.N = pl.N; p.nl = pl.nl; p.nslot = pl.nslot;
  void* args[] = {&p};
  auto mark = [&](int i) {
    return a.stage_events[i] ? hipEventRecord(reinterpret_cast<hipEvent_t>(a.stage_events[i]), stream)
                             : hipSuccess;
  };
  const int NT = 64 * (pl.C >= 64 ? 4 : pl.C / 16);
  const dim3 chunks((unsigned)pl.N, (unsigned)pl.BH);

  if (mark(0) != hipSuccess) return LLA_ERR_HIP;
  if (pl.nl > 0) {
    if (set_smem(ks->states, pl.smem_states) != hipSuccess) return LLA_ERR_HIP;
    if (hipLaunchKernel(ks->states, chunks, dim3(NT), args, pl.smem_states, stream) != hipSuccess)
      return LLA_ERR_HIP;
    if (set_smem(ks->rn, pl.smem_states) != hipSuccess) return LLA_ERR_HIP;
    if (hipLaunchKernel(ks->rn, dim3((unsigned)((long long)pl.items * pl.BH)), dim3(NT), args,
                        pl.smem_states, stream) != hipSuccess)
      return LLA_ERR_HIP;
    if (pl.nl > 1) {
      hipLaunchKernelGGL(lla::bwd::bwd_gsum_kernel, dim3((unsigned)pl.BH), dim3(256), 0, stream, p);
      if (hipGetLastError() != hipSuccess) return LLA_ERR_HIP;
    }
    const int SZ = a.dk * a.dv;   // a multiple of 64: the tree grid covers it exactly
    const dim3 tgrid((unsigned)(SZ / 64), (unsigned)pl.BH), tblock(64 * lla::bwd::kTreeWaves);
    const bool bf = a.dtype == LLA_DTYPE_BF16;
    if (pl.tree_smem > 0) {
      const void* fn = bf ? reinterpret_cast<const void*>(&lla::bwd::bwd_tree_kernel<lla::bf16, true>)
                          : reinterpret_cast<const void*>(&lla::bwd::bwd_tree_kernel<float, true>);
      if (set_smem(fn, pl.tree_smem) != hipSuccess) return LLA_ERR_HIP;
      if (bf)
        hipLaunchKernelGGL((lla::bwd::bwd_tree_kernel<lla::bf16, true>), tgrid, tblock, pl.tree_smem, stream, p, SZ);
      else
        hipLaunchKernelGGL((lla::bwd::bwd_tree_kernel<float, true>), tgrid, tblock, pl.tree_smem, stream, p, SZ);
    } else if (bf) {
      hipLaunchKernelGGL((lla::bwd::bwd_tree_kernel<lla::bf16, false>), tgrid, tblock, 0, stream, p, SZ);
    } else {
      hipLaunchKernelGGL((lla::bwd::bwd_tree_kernel<float, false>), tgrid, tblock, 0, stream, p, SZ);
    }
    if (hipGetLastError() != hipSuccess) return LLA_ERR_HIP;
  }
  if (mark(1) != hipSuccess) return LLA_ERR_HIP;
  if (set_smem(ks->grads, pl.smem_grads) != hipSuccess) return LLA_ERR_HIP;
  // one-dimensional: the kernel maps workgroups to (chunk, head) so that each XCD keeps to its heads
  if (hipLaunchKernel(ks->grads, dim3((unsigned)(pl.N * pl.BH)), dim3(NT), args, pl.smem_grads,
                      stream) != hipSuccess)
    return LLA_ERR_HIP;
  if (mark(2) != hipSuccess) return LLA_ERR_HIP;
  hipLaunchKernelGGL(lla::bwd::bwd_dloga_kernel, dim3((unsigned)pl.BH), dim3(256), 0, stream, p);
  if (hipGetLastError() != hipSuccess) return LLA_ERR_HIP;
  if (mark(3) != hipSuccess) return LLA_ERR_HIP;
  return LLA_OK;
}

int backward(const lla_bwd_args& a, hipStream_t stream) {
  BwdPlan pl;
  int st = make_bwd_plan(a.B, a.H, a.T, a.dk, a.dv, a.chunk, a.dtype, pl);
  if (st != LLA_OK) return st;
  if (pl.BH == 0 || a.T == 0) return LLA_OK;
  st = validate(a, pl);
  if (st != LLA_OK) return st;
  void* ws = a.workspace;
  bool owned = false;
  if (ws) {
    if (a.workspace_bytes < pl.ws_bytes) return LLA_ERR_WORKSPACE;
    if ((uintptr_t)ws & 255) return LLA_ERR_INVALID_ARG;
  } else {
    if (lla::workspace_alloc(&ws, pl.ws_bytes, stream) != hipSuccess) return LLA_ERR_NO_MEMORY;
    owned = true;
  }
  st = launch_bwd(a, pl, ws, stream);
  if (owned && hipFreeAsync(ws, stream) != hipSuccess && st == LLA_OK) st = LLA_ERR_HIP;
  return st;
}

}  // namespace

extern "C" {

int loglinear_attn_bwd(const lla_bwd_args* args, lla_stream_t stream) {
  if (!args) return LLA_ERR_INVALID_ARG;
  return backward(*args, reinterpret_cast<hipStream_t>(stream));
}

size_t loglinear_attn_bwd_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, int dtype) {
  BwdPlan pl;
  if (make_bwd_plan(B, H, T, dk, dv, chunk, dtype, pl) != LLA_OK) return 0;
  return pl.ws_bytes;
}

int loglinear_attn_bwd_default_chunk(int dk, int dv, int dtype) {
  if (!supported_dim(dk) || !supported_dim(dv)) return 0;
  if (dtype != LLA_DTYPE_BF16 && dtype != LLA_DTYPE_F32) return 0;
  return bwd_default_chunk(dk, dv, dtype == LLA_DTYPE_BF16 ? 2 : 4);
}

}  // extern "C"
