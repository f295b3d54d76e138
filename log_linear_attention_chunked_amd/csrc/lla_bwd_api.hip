// lla_bwd_api.hip — C ABI of the backward pass: argument validation, plan (chunk, tree and
// workspace layout) and the stream-ordered launch sequence bwd_states -> bwd_rn -> bwd_gsum ->
// bwd_gtree (or bwd_tree) -> bwd_grads -> bwd_dloga. The contract is documented in
// include/loglinear_attn.h.
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
    const int o_prev = p.lvl[i - 1], o = p.lvl[i];
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

// For trees too large for bwd_gtree's shared memory: the up-sweep reads level i-1 back from
// the node array and the down-sweep keeps every level in the outs array.
// E: the element type of the copies the gradient kernel reads (node_e, u_e)
// at most 64 registers per lane: two workgroups of 16 waves share a compute unit (8 waves per SIMD)
template <typename E>
__global__ void __launch_bounds__(64 * kTreeWaves) __attribute__((amdgpu_waves_per_eu(8)))
bwd_tree_kernel(BwdParams p, int SZ) {
  const int bh = blockIdx.y, lane = threadIdx.x & 63;
  const int e = blockIdx.x * 64 + lane, w = threadIdx.x >> 6;
  // the grid has exactly SZ / 64 columns of workgroups (SZ = dk*dv is a multiple of 64)
  const float* __restrict__ gs = p.gsum + (size_t)bh * p.nslot;
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
  // level 0, KB chunks of a wave at a time: all their loads (unconditional, clamped to the last
  // chunk) are issued before any value is used, so a batch costs one memory round trip
  constexpr int KB = 8;
  for (int m0 = w; m0 < p.N; m0 += kTreeWaves * KB) {
    float x[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) x[u] = nd[(size_t)min(m0 + u * kTreeWaves, p.N - 1) * SZ];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int m = m0 + u * kTreeWaves;
      if (m >= p.N) break;
      // the gradient kernel reads node (j, (c >> j) - 1) for set bits j of c: even nodes only
      if (!(m & 1)) put(ne, nlo, (size_t)m * SZ, x[u]);
    }
  }
  __syncthreads();
  for (int i = 1; i < p.nl; ++i) {
    const int nprev = (p.N + (1 << (i - 1)) - 1) >> (i - 1), nb = (p.N + (1 << i) - 1) >> i;
    const int o_prev = p.lvl[i - 1], o = p.lvl[i];
    for (int m0 = w; m0 < nb; m0 += kTreeWaves * KB) {
      // both children of KB blocks (clamped to valid slots of level i-1) before any is used
      float lhs[KB], rhs[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int sl = o_prev + min(2 * (m0 + u * kTreeWaves), nprev - 1);
        const int sr = o_prev + min(2 * (m0 + u * kTreeWaves) + 1, nprev - 1);
        lhs[u] = nd[(size_t)sl * SZ];
        rhs[u] = nd[(size_t)sr * SZ];
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int m = m0 + u * kTreeWaves;
        if (m >= nb) break;
        const bool right = 2 * m + 1 < nprev;
        const float val = right ? __expf(gs[o_prev + 2 * m + 1]) * lhs[u] + rhs[u] : lhs[u];
        if (!(m & 1)) put(ne, nlo, (size_t)(o + m) * SZ, val);
        nd[(size_t)(o + m) * SZ] = val;
      }
    }
    __syncthreads();
  }
  // down-sweep; a wave takes KB of its blocks at a time and loads all their right-block states
  // before it uses any of them; the first KB of the next level are loaded while this level is
  // worked on (they depend on nothing the sweep writes). Every load is unconditional from a
  // clamped, valid item (a block with no right sibling multiplies it by zero), so the counted
  // waits stay exact; a right block of several sub-blocks (levels past kSubLog) is summed KB
  // sub-blocks at a time, their loads again issued together.
  auto fetch = [&](int i, int m0, float (&rn)[KB]) {
    const int nb = (p.N + (1 << i) - 1) >> i;
    const int s = sub_log(i), b = i - s, os = p.lvl[s];
    const int nsub = (p.N + (1 << s) - 1) >> s;
    const int nit = items_of_level(p.N, i);
    const float* rpl = rp + (size_t)p.rn_off[i] * SZ;
    if (b == 0) {   // one sub-block per right block
      float x[KB];
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int m = m0 + u * kTreeWaves;
        // an odd block has no right sibling: every such lane reads item 0
        x[u] = rpl[(m & 1) ? 0 : (size_t)min(item_of_sub(i, min(m + 1, nsub - 1)), nit - 1) * SZ];
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int m = m0 + u * kTreeWaves;
        rn[u] = (m < nb && !(m & 1) && m + 1 < nb) ? x[u] : 0.f;
      }
      return;
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int m = m0 + u * kTreeWaves;
      rn[u] = 0.f;
      if (m < nb && !(m & 1) && m + 1 < nb) {
        const int sb0 = (m + 1) << b, sb1 = min((m + 2) << b, nsub);
        float dec = 0.f;
        for (int t0 = sb0; t0 < sb1; t0 += KB) {
          float x[KB];
#pragma unroll
          for (int e = 0; e < KB; ++e) x[e] = rpl[(size_t)item_of_sub(i, min(t0 + e, sb1 - 1)) * SZ];
#pragma unroll
          for (int e = 0; e < KB; ++e) {
            if (t0 + e < sb1) {
              rn[u] += __expf(dec) * x[e];
              dec += gs[os + t0 + e];
            }
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
    const int o = p.lvl[i];
    const bool top = i + 1 >= p.nl;
    const int op = top ? 0 : p.lvl[i + 1];
    for (int m0 = w; m0 < nb; m0 += kTreeWaves * KB) {
      float rn[KB];
      if (m0 == w) {
#pragma unroll
        for (int u = 0; u < KB; ++u) rn[u] = rn_first[u];
      } else {
        fetch(i, m0, rn);
      }
      // the parents' values (level i+1, clamped to its valid slots) before any is used
      float par[KB];
      const int npar = (p.N + (2 << i) - 1) >> (i + 1);
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int ps = op + min((m0 + u * kTreeWaves) >> 1, npar - 1);
        par[u] = top ? 0.f : ou[(size_t)ps * SZ];
      }
#pragma unroll
      for (int u = 0; u < KB; ++u) {
        const int m = m0 + u * kTreeWaves;
        if (m >= nb) break;
        const float val = (!(m & 1) && m + 1 < nb) ? __expf(gs[o + m + 1]) * par[u] + rn[u] : par[u];
        ou[(size_t)(o + m) * SZ] = val;
        if (i == 0) put(ue, ulo, (size_t)m * SZ, val);
      }
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------------------------------------
// bwd_gtree: the same tree, with each wave owning a run of 2^wl consecutive groups of 8 chunks
// (bwd_rn's sub-blocks; wl >= 1, the least that covers every group with the kTreeWaves waves).
// Levels 0..3 of a group (its chunks, pairs, quads and the group itself) are combined in
// registers, up and down; a pair of groups (level 4) is combined by its wave as it goes; only the
// levels above go through shared memory. A right block of several groups (level i >= 4) receives,
// from each of its groups g, the contribution exp(decay from the block's start to g's start) *
// P(i, g) (P: bwd_rn's sub-block state); a wave sums the contributions of its groups per unit of
// min(2^(i-3), 2^wl) groups (a unit lies inside one wave's run and one block) and the down-sweep
// sums a block's units in order. Every global load a workgroup makes (the first group's chunk
// states, right blocks' states and contributions, and the block decays) is issued before the
// first wait.
// Shared memory: the block decays (floats); then slots of VE floats per lane: per level
// i >= 4 (below nl) the block values (up-sweep values later overwritten by the down-sweep's); per
// level i >= 4 the contributions, one per unit of a right block (in unit order).
// ----------------------------------------------------------------------------------------

constexpr int kGrpLog = 3;            // 8 chunks per group
static_assert(kGrpLog == kSubLog, "a group is one of bwd_rn's sub-blocks");
constexpr int kGtCt = 6;              // levels >= 4 whose contributions a wave prefetches
// Each lane holds VE (4, else 2 or 1 where the shared memory would not fit) consecutive state
// elements: 16-byte loads, 8-byte bf16 stores and 16-byte shared-memory slots at VE = 4, where a
// workgroup covers 256 elements and the scalar work of a group (its addresses, levels and
// branches, the same for every element) is shared by four times the data.

// log2 of the groups a wave owns: at least 2 (a pair of groups), a power of two, and enough for
// kTreeWaves waves to cover the ng groups
__host__ __device__ inline int gtree_wave_log(int ng) {
  int wl = 1;
  while ((kTreeWaves << wl) < ng) ++wl;
  return wl;
}
// log2 of the unit (in groups) over which a wave sums the level-i contributions, and the units
// of right blocks at level i (unit t lies in block t >> (i - 3 - a), a right block when odd)
__host__ __device__ inline int gtree_unit_log(int i, int wl) { return i - 3 < wl ? i - 3 : wl; }
__host__ __device__ inline int gtree_units(int ng, int i, int wl) {
  const int a = gtree_unit_log(i, wl), b = i - 3 - a;
  const int M = (ng + (1 << a) - 1) >> a;
  const int rem = M & ((2 << b) - 1);
  return ((M >> (b + 1)) << b) + (rem > (1 << b) ? rem - (1 << b) : 0);
}
// the k-th unit of right blocks at level i: unit t (bit b of t set, b = i - 3 - a)
__host__ __device__ inline int gtree_unit_item(int i, int wl, int t) {
  const int b = i - 3 - gtree_unit_log(i, wl);
  return ((t >> (b + 1)) << b) | (t & ((1 << b) - 1));
}
// first slot of level i's block values (4 <= i <= nl) and of level i's contributions
// (4 <= i <= nl; i = nl gives the total) in the value region, which follows the block decays
__host__ __device__ inline int gtree_lv(int N, int i) {
  int off = 0;
  for (int a = 4; a < i; ++a) off += (N + (1 << a) - 1) >> a;
  return off;
}
__host__ __device__ inline int gtree_ct(int N, int nl, int i) {
  const int ng = (N + 7) >> kGrpLog, wl = gtree_wave_log(ng);
  int off = gtree_lv(N, nl > 4 ? nl : 4);
  for (int a = 4; a < i; ++a) off += gtree_units(ng, a, wl);
  return off;
}
// the decays, then every level's block values and contributions, VE * 64 floats per slot
__host__ __device__ inline int gtree_floats(int N, int nl, int nslot, int VE) {
  return ((nslot + 63) & ~63) + gtree_ct(N, nl, nl > 4 ? nl : 4) * VE * 64;
}

// GROUPED: bwd_statesg has done levels 0..3 of every group (nodes written, the group in fp32 at
// its level-3 slot); the tree then starts from the groups
// DOUT: the down-sweep stops at the groups and writes what each group receives
// from the levels above 2, in fp32, to ud; the gradient kernel finishes it per chunk from the
// group's target-side blocks of levels 0..2 (which this kernel then never reads)
template <typename E, bool GROUPED, int VE, bool DOUT = false>
__global__ void __launch_bounds__(64 * kTreeWaves) __attribute__((amdgpu_waves_per_eu(VE > 1 ? 4 : 8)))
bwd_gtree_kernel(BwdParams p, int SZ) {
  extern __shared__ __attribute__((aligned(16))) float tl[];
  constexpr int SW = 64 * VE;   // elements per workgroup (one shared-memory slot)
  typedef float FV __attribute__((ext_vector_type(VE)));
  typedef E EV __attribute__((ext_vector_type(VE)));
  // the wave index is uniform (read from lane 0), so every group and block index below is, and
  // each access is a uniform base plus the lane's bytes
  const int bh = blockIdx.y, lane = threadIdx.x & 63;
  const unsigned ul = threadIdx.x & 63;   // the lane as an unsigned (zero-extended) offset
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int e0 = blockIdx.x * SW;
  const int N = p.N, nl = p.nl, ng = (N + 7) >> kGrpLog;
  const float* __restrict__ gsg = p.gsum + (size_t)bh * p.nslot;
  float* gs = tl;                        // block decays first
  float* tv = tl + ((p.nslot + 63) & ~63);   // then the block values, SW floats per slot
  const float* __restrict__ nd = p.node + (size_t)bh * p.nslot * SZ + e0;
  const float* __restrict__ rp = p.rnp + (size_t)bh * p.items * SZ + e0;
  E* __restrict__ ne = reinterpret_cast<E*>(p.node_e) + (size_t)bh * p.nslot * SZ + e0;
  E* __restrict__ ue = reinterpret_cast<E*>(p.u_e) + (size_t)bh * N * SZ + e0;
  constexpr bool SPLIT = sizeof(E) == 2;
  E* __restrict__ nlo = reinterpret_cast<E*>(p.node_lo) + (size_t)bh * p.nslot * SZ + e0;
  E* __restrict__ ulo = reinterpret_cast<E*>(p.u_lo) + (size_t)bh * N * SZ + e0;
  auto put = [&](E* hi, E* lo, size_t at, const FV& x) {
    EV h, l;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      h[e] = (E)x[e];
      l[e] = (E)(x[e] - (float)h[e]);
    }
    reinterpret_cast<__attribute__((address_space(1))) EV*>(uniform_ptr(hi + at))[ul] = h;
    if (SPLIT) reinterpret_cast<__attribute__((address_space(1))) EV*>(uniform_ptr(lo + at))[ul] = l;
  };
  // the lane's elements of the state in slot i of a region
  auto ld = [&](const float* base, int i) {
    return reinterpret_cast<const __attribute__((address_space(1))) FV*>(uniform_ptr(base + (size_t)i * SZ))[ul];
  };
  // the lane's elements of block-value slot s (shared memory)
  auto tvs = [&](int s) -> FV& { return *reinterpret_cast<FV*>(tv + s * SW + VE * lane); };
  auto nb = [&](int i) { return (N + (1 << i) - 1) >> i; };
  // item index of right block sb at level i, or item 0 (read, then multiplied by nothing) when
  // there is none
  auto item = [&](int i, int sb, bool ok) {
    return ok ? p.rn_off[i] + item_of_sub(i, sb) : 0;
  };
  const FV zero = (FV)(0.f);

  // one group's loads: its chunk states (zero past N), the right-block states of levels 0..3
  // inside it, and its contributions to right blocks of levels 4 .. 3 + kGtCt
  struct GLoads {
    FV x[GROUPED ? 1 : 8], r0[4], r1[2], r2, r3, ct[kGtCt];
  };
  auto load_group = [&](int g, GLoads& d) {
    const int c0 = g << kGrpLog;
    if constexpr (GROUPED) {
      d.x[0] = ld(nd, 3 < nl ? slot_p(p, 3, g) : 0);
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) d.x[k] = ld(nd, min(c0 + k, N - 1));
    }
    if constexpr (!DOUT) {
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const int sb = c0 + 2 * h + 1;                     // level 0: chunk 2h+1 of the group
        d.r0[h] = ld(rp, item(0, sb, 0 < nl && sb < N));
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int sb = 4 * g + 2 * h + 1;
        d.r1[h] = ld(rp, item(1, sb, 1 < nl && sb < nb(1)));
      }
      d.r2 = ld(rp, item(2, 2 * g + 1, 2 < nl && 2 * g + 1 < nb(2)));
    }
    d.r3 = ld(rp, item(3, g + 1, 3 < nl && !(g & 1) && g + 1 < ng));
#pragma unroll
    for (int u = 0; u < kGtCt; ++u) {
      const int i = 4 + u;
      d.ct[u] = ld(rp, item(i, g, i < nl && ((g >> (i - 3)) & 1)));
    }
  };

  // the decays go to shared memory first (one value per thread for up to 1024 blocks, the rest,
  // for larger trees, in a loop afterwards); the first group's loads are issued beside them
  const float gv = gsg[min((int)threadIdx.x, p.nslot - 1)];
  // this wave's groups [gb, ge)
  const int wl = gtree_wave_log(ng);
  const int gb = w << wl, ge = min(gb + (1 << wl), ng);
  GLoads first;
  if (gb < ng) load_group(gb, first);
  if ((int)threadIdx.x < p.nslot) gs[threadIdx.x] = gv;
  for (int i = threadIdx.x + 64 * kTreeWaves; i < p.nslot; i += 64 * kTreeWaves) gs[i] = gsg[i];
  __syncthreads();
  // decay of block m at level i (0 where the block does not exist: it then holds zeros)
  auto G = [&](int i, int m) { return (i < nl && m < nb(i)) ? gs[slot_p(p, i, m)] : 0.f; };

  // up-sweep inside a group; returns the group's value at level 3
  auto up_group = [&](int g, const GLoads& d) -> FV {
    if constexpr (GROUPED) {
      return d.x[0];
    } else {
      const int c0 = g << kGrpLog;
      FV x[8], y1[4], y2[2];
#pragma unroll
      for (int k = 0; k < 8; ++k) x[k] = c0 + k < N ? d.x[k] : zero;
#pragma unroll
      for (int h = 0; h < 4; ++h) y1[h] = __expf(G(0, c0 + 2 * h + 1)) * x[2 * h] + x[2 * h + 1];
#pragma unroll
      for (int h = 0; h < 2; ++h) y2[h] = __expf(G(1, 4 * g + 2 * h + 1)) * y1[2 * h] + y1[2 * h + 1];
      const FV y3 = __expf(G(2, 2 * g + 1)) * y2[0] + y2[1];
      // the gradient kernel reads node (j, (c >> j) - 1) for set bits j of c: even nodes only
#pragma unroll
      for (int h = 0; h < 4; ++h)
        if (0 < nl && c0 + 2 * h < N) put(ne, nlo, (size_t)(c0 + 2 * h) * SZ, x[2 * h]);
#pragma unroll
      for (int h = 0; h < 2; ++h)
        if (1 < nl && 4 * g + 2 * h < nb(1)) put(ne, nlo, (size_t)slot_p(p, 1, 4 * g + 2 * h) * SZ, y1[2 * h]);
      if (2 < nl && 2 * g < nb(2)) put(ne, nlo, (size_t)slot_p(p, 2, 2 * g) * SZ, y2[0]);
      if (3 < nl && !(g & 1)) put(ne, nlo, (size_t)slot_p(p, 3, g) * SZ, y3);
      return y3;
    }
  };
  // the pair of groups g >> 1 (a level-4 block): the left group's value waits in the block's
  // slot for its right sibling, which the same wave takes next
  auto up_pair = [&](int g, const FV& y3) {
    if (4 < nl) {
      FV& v = tvs(p.gtlv[4] + (g >> 1));
      if (!(g & 1)) v = y3;
      else v = __expf(G(3, g)) * v + y3;
      if (((g & 1) || g + 1 == ng) && !((g >> 1) & 1)) put(ne, nlo, (size_t)slot_p(p, 4, g >> 1) * SZ, v);
    }
  };
  // contributions of a group to the right blocks above level 3 that hold it, summed over the
  // groups of each unit (the unit's first group sets its slot, the others add, in group order)
  auto contribute = [&](int g, const GLoads& d) {
#pragma unroll
    for (int u = 0; u < kGtCt; ++u) {
      const int i = 4 + u;
      if (i < nl && ((g >> (i - 3)) & 1)) {
        float dec = 0.f;
        for (int g2 = (g >> (i - 3)) << (i - 3); g2 < g; ++g2) dec += gs[slot_p(p, 3, g2)];
        const int a = gtree_unit_log(i, wl);
        FV& c = tvs(p.gtct[i] + gtree_unit_item(i, wl, g >> a));
        const FV t = __expf(dec) * d.ct[u];
        if (g & ((1 << a) - 1)) c += t;
        else c = t;
      }
    }
  };
  for (int g = gb; g < ge; ++g) {
    if (g == gb) {
      contribute(g, first);
      up_pair(g, up_group(g, first));
    } else {
      GLoads d;
      load_group(g, d);
      contribute(g, d);
      up_pair(g, up_group(g, d));
    }
  }
  __syncthreads();

  // levels >= 5, up: block values from the level below
  for (int i = 5; i < nl; ++i) {
    for (int m = w; m < nb(i); m += kTreeWaves) {
      const bool right = 2 * m + 1 < nb(i - 1);
      const FV l0 = tvs(p.gtlv[i - 1] + 2 * m);
      const FV v = right ? __expf(G(i - 1, 2 * m + 1)) * l0 + tvs(p.gtlv[i - 1] + 2 * m + 1) : l0;
      tvs(p.gtlv[i] + m) = v;
      if (!(m & 1)) put(ne, nlo, (size_t)slot_p(p, i, m) * SZ, v);
    }
    __syncthreads();
  }
  // levels >= 4, down (each block's value replaces its up-sweep value): what the block's
  // chunks receive from later blocks at its level and above, decayed to the block's end
  for (int i = nl - 1; i >= 4; --i) {
    for (int m = w; m < nb(i); m += kTreeWaves) {
      const FV par = i + 1 < nl ? tvs(p.gtlv[i + 1] + (m >> 1)) : zero;
      FV v = par;
      if (!(m & 1) && m + 1 < nb(i)) {
        FV rn = zero;
        const int a = gtree_unit_log(i, wl);
        const int t0 = ((m + 1) << (i - 3)) >> a, t1 = (min((m + 2) << (i - 3), ng) + (1 << a) - 1) >> a;
        for (int t = t0; t < t1; ++t) rn += tvs(p.gtct[i] + gtree_unit_item(i, wl, t));
        v = __expf(G(i, m + 1)) * par + rn;
      }
      tvs(p.gtlv[i] + m) = v;
    }
    __syncthreads();
  }
  // levels 3..0 of each group, down; the chunks' combined right-sibling states
  auto down_group = [&](int g, const GLoads& d) {
    const int c0 = g << kGrpLog;
    const FV par3 = 4 < nl ? tvs(p.gtlv[4] + (g >> 1)) : zero;
    const FV d3 = (3 < nl && !(g & 1) && g + 1 < ng) ? __expf(G(3, g + 1)) * par3 + d.r3 : par3;
    if constexpr (DOUT) {
      reinterpret_cast<__attribute__((address_space(1))) FV*>(
          uniform_ptr(p.ud + ((size_t)bh * ng + g) * SZ + e0))[ul] = d3;
      return;
    }
    FV d2[2], d1[4];
    d2[0] = (2 < nl && 2 * g + 1 < nb(2)) ? __expf(G(2, 2 * g + 1)) * d3 + d.r2 : d3;
    d2[1] = d3;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int m = 4 * g + 2 * h;
      d1[2 * h] = (1 < nl && m + 1 < nb(1)) ? __expf(G(1, m + 1)) * d2[h] + d.r1[h] : d2[h];
      d1[2 * h + 1] = d2[h];
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      const int c = c0 + 2 * h;
      const FV d0 = (0 < nl && c + 1 < N) ? __expf(G(0, c + 1)) * d1[h] + d.r0[h] : d1[h];
      if (c < N) put(ue, ulo, (size_t)c * SZ, d0);
      if (c + 1 < N) put(ue, ulo, (size_t)(c + 1) * SZ, d1[h]);
    }
  };
  for (int g = gb; g < ge; ++g) {
    if (g == gb) {
      down_group(g, first);
    } else {
      GLoads d;
      load_group(g, d);
      down_group(g, d);
    }
  }
}

// ----------------------------------------------------------------------------------------
// bwd_dloga: dlog_a[r] = sum_{t >= r} dA_t (fixed order)
// ----------------------------------------------------------------------------------------

// one workgroup per segment of a head's positions (gridDim.x segments): the sum of every dA after
// the segment by a block reduction, then the segment's own reverse prefix on top of it
__global__ void __launch_bounds__(256) bwd_dloga_kernel(BwdParams p) {
  __shared__ float wtot[4];
  const int bh = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int seglen = (p.T + gridDim.x - 1) / gridDim.x;
  const int s0 = min(p.T, (int)blockIdx.x * seglen), s1 = min(p.T, s0 + seglen);
  const float* dA = p.dA + (size_t)bh * p.T;
  float* out = p.glog_a + (size_t)bh * p.T;
  // the positions after the segment
  float after = 0.f;
  for (int t = s1 + tid; t < p.T; t += 256) after += dA[t];
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) after += __shfl_xor(after, d);
  if (lane == 0) wtot[w] = after;
  __syncthreads();
  after = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  __syncthreads();
  // the segment: per-thread runs, their suffix over the threads above by wave shuffles and the
  // waves above through shared memory, all in a fixed order
  const int per = (s1 - s0 + 255) / 256;
  const int lo = min(s1, s0 + tid * per), hi = min(s1, lo + per);
  float s = 0.f;
  for (int t = hi - 1; t >= lo; --t) s += dA[t];
  float incl = s;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_down(incl, d);
    if (lane + d < 64) incl += y;
  }
  if (lane == 0) wtot[w] = incl;
  __syncthreads();
  float run = incl - s + after;
  for (int u = 3; u > w; --u) run += wtot[u];
  for (int t = hi - 1; t >= lo; --t) {
    run += dA[t];
    out[t] = run;
  }
}

}  // namespace bwd
}  // namespace lla

namespace {

// the group tree's instance for an element type, a grouped start and VE elements per lane (at
// most 2 without the grouped start, whose eight chunk states per group would not fit the
// registers at 4)
template <typename E, bool GROUPED, bool DOUT = false>
const void* gtree_fn_ve(int ve) {
  using namespace lla::bwd;
  if constexpr (GROUPED)
    if (ve == 4) return reinterpret_cast<const void*>(&bwd_gtree_kernel<E, GROUPED, 4, DOUT>);
  if (ve == 2) return reinterpret_cast<const void*>(&bwd_gtree_kernel<E, GROUPED, 2, DOUT>);
  if (ve == 1) return reinterpret_cast<const void*>(&bwd_gtree_kernel<E, GROUPED, 1, DOUT>);
  return nullptr;
}
// dout: the down-sweep stops at the groups (grouped only)
const void* gtree_fn(bool bf, bool grouped, int ve, bool dout) {
  if (bf) {
    if (!grouped) return dout ? gtree_fn_ve<lla::bf16, false, true>(ve) : gtree_fn_ve<lla::bf16, false>(ve);
    return dout ? gtree_fn_ve<lla::bf16, true, true>(ve) : gtree_fn_ve<lla::bf16, true>(ve);
  }
  if (!grouped) return dout ? gtree_fn_ve<float, false, true>(ve) : gtree_fn_ve<float, false>(ve);
  return dout ? gtree_fn_ve<float, true, true>(ve) : gtree_fn_ve<float, true>(ve);
}

using lla::bwd::BwdKernels;
using lla::bwd::BwdParams;

inline bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
inline int bit_len(unsigned x) { int n = 0; while (x) { ++n; x >>= 1; } return n; }
inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int kLdsPerWorkgroup = 160 * 1024;

struct BwdPlan {
  int C, N, nl, nslot, L, esize, smem_states, smem_grads;
  int gtree_smem;   // > 0: the group tree (bwd_gtree) runs, with this much shared memory
  int gtree_ve;     // and this many state elements per lane
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
  // the group tree when its contributions are all prefetched (levels up to 3 + kGtCt) and its
  // shared memory fits; otherwise the level-by-level tree
  pl.gtree_smem = 0;
  pl.gtree_ve = 0;
  for (int ve = 4; ve >= 1 && pl.nl > 0 && pl.nl <= 4 + lla::bwd::kGtCt && !pl.gtree_smem; ve >>= 1) {
    const size_t b = (size_t)lla::bwd::gtree_floats(pl.N, pl.nl, pl.nslot, ve) * 4;
    if (b <= (size_t)kLdsPerWorkgroup) {
      pl.gtree_smem = (int)b;
      pl.gtree_ve = ve;
    }
  }
  pl.off_outs = off; off = align256(off + (pl.gtree_smem ? 0 : (size_t)BH * pl.nslot * SZ * 4));
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
  {
    // the gradient kernel's per-wave dlambda shares of the node levels, in its score images
    const lla::bwd::BwdSmem g = lla::bwd::bwd_smem(pl.esize, C, dk, dv, true);
    const int nw = C >= 64 ? 4 : C / 16;
    if ((long long)nw * pl.nl * C * 4 > g.lam - g.p1) return LLA_ERR_UNSUPPORTED;
  }
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
  // the group states when the gradient kernel forms U_c itself, in U's region (ceil(N/8) fp32
  // states per head take no more room than N element-type ones for N >= 2)
  p.ud = reinterpret_cast<float*>(w + pl.off_u_e);
  p.dA = reinterpret_cast<float*>(w + pl.off_dA);
  p.BH = (int)pl.BH; p.T = a.T; p.L = pl.L; p.N = pl.N; p.nl = pl.nl; p.nslot = pl.nslot;
  for (int i = 0; i <= lla::kLamCap; ++i) {
    p.lvl[i] = i <= pl.nl ? lla::bwd::slot_of(pl.N, i, 0) : pl.nslot;
    p.gtlv[i] = i >= 4 && i <= pl.nl ? lla::bwd::gtree_lv(pl.N, i) : 0;
    p.gtct[i] = i >= 4 && i <= pl.nl ? lla::bwd::gtree_ct(pl.N, pl.nl, i) : 0;
  }
  void* args[] = {&p};
  auto mark = [&](int i) {
    return a.stage_events[i] ? hipEventRecord(reinterpret_cast<hipEvent_t>(a.stage_events[i]), stream)
                             : hipSuccess;
  };
  const int NT = 64 * (pl.C >= 64 ? 4 : pl.C / 16);
  const dim3 chunks((unsigned)pl.N, (unsigned)pl.BH);

  // the chunk states: by groups of 8 chunks with the groups' part of the up-sweep when the
  // group tree runs and the kernel exists for the shape, else one workgroup per chunk; whenever
  // the group tree runs, it hands over group states and the gradient kernel forms each chunk's
  // combined right-sibling state (the level-by-level tree still writes U_c)
  const bool grouped = pl.nl > 0 && pl.gtree_smem > 0 && ks->statesg;
  const bool dmode = pl.nl > 0 && pl.gtree_smem > 0 && ks->grads_d;
  const void* grads = dmode ? ks->grads_d : ks->grads;
  if (mark(0) != hipSuccess) return LLA_ERR_HIP;
  if (pl.nl > 0) {
    const long long ng = (pl.N + 7) / 8;
    if (grouped) {
      if (set_smem(ks->statesg, pl.smem_states) != hipSuccess) return LLA_ERR_HIP;
      if (hipLaunchKernel(ks->statesg, dim3((unsigned)(ng * pl.BH)), dim3(NT), args, pl.smem_states,
                          stream) != hipSuccess)
        return LLA_ERR_HIP;
    } else {
      if (set_smem(ks->states, pl.smem_states) != hipSuccess) return LLA_ERR_HIP;
      if (hipLaunchKernel(ks->states, chunks, dim3(NT), args, pl.smem_states, stream) != hipSuccess)
        return LLA_ERR_HIP;
    }
    // the target-side sub-block states: one workgroup per group of 8 chunks where its
    // accumulators fit, else one per sub-block and level
    if (ks->rng) {
      if (set_smem(ks->rng, pl.smem_states) != hipSuccess) return LLA_ERR_HIP;
      if (hipLaunchKernel(ks->rng, dim3((unsigned)(ng * pl.BH)), dim3(NT), args, pl.smem_states,
                          stream) != hipSuccess)
        return LLA_ERR_HIP;
    } else {
      if (set_smem(ks->rn, pl.smem_states) != hipSuccess) return LLA_ERR_HIP;
      if (hipLaunchKernel(ks->rn, dim3((unsigned)((long long)pl.items * pl.BH)), dim3(NT), args,
                          pl.smem_states, stream) != hipSuccess)
        return LLA_ERR_HIP;
    }
    if (pl.nl > 1) {
      hipLaunchKernelGGL(lla::bwd::bwd_gsum_kernel, dim3((unsigned)pl.BH), dim3(256), 0, stream, p);
      if (hipGetLastError() != hipSuccess) return LLA_ERR_HIP;
    }
    const int SZ = a.dk * a.dv;   // a multiple of 256: the tree grids cover it exactly
    const dim3 tgrid((unsigned)(SZ / 64), (unsigned)pl.BH), tblock(64 * lla::bwd::kTreeWaves);
    const bool bf = a.dtype == LLA_DTYPE_BF16;
    if (pl.gtree_smem > 0) {
      // the shared memory planned for VE elements per lane covers any smaller VE
      const int ve = grouped || pl.gtree_ve < 2 ? pl.gtree_ve : 2;
      const void* fn = gtree_fn(bf, grouped, ve, dmode);
      if (!fn) return LLA_ERR_UNSUPPORTED;
      if (set_smem(fn, pl.gtree_smem) != hipSuccess) return LLA_ERR_HIP;
      void* targs[] = {&p, const_cast<int*>(&SZ)};
      if (hipLaunchKernel(fn, dim3((unsigned)(SZ / (64 * ve)), (unsigned)pl.BH), tblock, targs,
                          pl.gtree_smem, stream) != hipSuccess)
        return LLA_ERR_HIP;
    } else if (bf) {
      hipLaunchKernelGGL((lla::bwd::bwd_tree_kernel<lla::bf16>), tgrid, tblock, 0, stream, p, SZ);
    } else {
      hipLaunchKernelGGL((lla::bwd::bwd_tree_kernel<float>), tgrid, tblock, 0, stream, p, SZ);
    }
    if (hipGetLastError() != hipSuccess) return LLA_ERR_HIP;
  }
  if (mark(1) != hipSuccess) return LLA_ERR_HIP;
  if (set_smem(grads, pl.smem_grads) != hipSuccess) return LLA_ERR_HIP;
  // one-dimensional: the kernel maps workgroups to (chunk, head) so that each XCD keeps to its heads
  if (hipLaunchKernel(grads, dim3((unsigned)(pl.N * pl.BH)), dim3(NT), args, pl.smem_grads,
                      stream) != hipSuccess)
    return LLA_ERR_HIP;
  if (mark(2) != hipSuccess) return LLA_ERR_HIP;
  // segments of about 1024 positions per head
  hipLaunchKernelGGL(lla::bwd::bwd_dloga_kernel, dim3((unsigned)((a.T + 1023) / 1024), (unsigned)pl.BH),
                     dim3(256), 0, stream, p);
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
