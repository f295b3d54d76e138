// lla_bwd.hpp — gfx950 backward pass of chunkwise log-linear Mamba-2 attention.
//
// Gradients of L = sum_t do_t . o_t for the forward operation
//   o_t = sum_{s<=t} lambda[t, l(t,s)] * exp(A_t - A_s) * (q_t . k_s) * v_s,  l = bit_length(t ^ s).
// ("Log-Linear Attention": the pages name training speed and the lambda gradient as the hard
// part of the backward pass, study notes sections 3-5 and 4-5.) With M[t,s] the mask weight
// lambda * exp(A_t - A_s), S = q.k and W[t,s] = do_t . v_s:
//   dq_t = sum_s M W k_s        dk_s = sum_t M W q_t        dv_s = sum_t M S do_t
//   dlambda[t, l] = sum_{s : l(t,s) = l} exp(A_t - A_s) S W
//   dA_t = q_t . dq_t - k_t . dk_t,   dlog_a[r] = sum_{t >= r} dA_t
// (A_t is the later end of every pair (t, s) and the earlier end of every pair (t', t); summing
// M S W over either index gives the two dot products.)
//
// Chunk structure (chunk C = 2^J, N chunks, chunk levels j = 0 .. nl-1, nl = bit_length(N-1)).
// For t in chunk c and s in an earlier chunk c', l(t,s) = J + 1 + j with j the highest bit of
// c ^ c'. The query side is the forward pass's: target c reads, for each set bit j, the Fenwick
// node (j, (c >> j) - 1) = sum_{s in block} exp(A_end - A_s) k_s v_s^T, decayed over the blocks
// of c's lower set bits. The source side is its mirror image: source chunk c receives, for each
// clear bit j, the right sibling block Y = (j, (c >> j) + 1) through
//   RN(j, Y) = sum_{t in Y} lambda[t, J+1+j] exp(A_t - A_start(Y)) q_t do_t^T,
// decayed over the right siblings of c's lower clear bits. lambda sits on the target here, so
// RN cannot be built from the blocks below it like a forward node: it is contracted from the
// block's own q and do rows, level by level.
//
// Kernels, in stream order (bwd_gsum, bwd_gtree / bwd_tree and bwd_dloga, which do not depend on
// the chunk or the head dims, live in lla_bwd_api.hip):
//   bwd_states  (chunk, head): F(c) = sum_s exp(g_c - A_s) k_s v_s^T (tree slot (0, c)) and g_c;
//   bwd_rn      (sub-block, head): the right blocks of level j split into sub-blocks of up to 8
//               chunks; each sub-block's lambda-weighted, decayed q do^T on MFMA;
//   bwd_gsum    (head): total log decay of every block (j, m), pairwise from the chunks;
//   bwd_gtree   (64 state elements, head): the forward up-sweep of the nodes, then a down-sweep
//               that gives every chunk its combined right-sibling state; each wave owns groups
//               of 8 chunks (tree levels 0..3 in registers), the levels above go through shared
//               memory; sums in fp32, and a copy in the element type of what the gradient kernel
//               reads (it rounds its MFMA operands to that type in any case). bwd_tree does the
//               same level by level through the workspace, for trees too large for bwd_gtree;
//   bwd_grads   (chunk, head): intra-chunk gradients on MFMA (masked S and W tiles, dlambda of
//               the levels inside the chunk), node read-outs for dq and dlambda, the combined
//               right-sibling state for dk and dv, dA;
//   bwd_dloga   (head): dlog_a as the reverse prefix sum of dA.
// Every sum runs in a fixed order: the gradients are bitwise deterministic.
//
// MFMA conventions as in the forward kernels: 16x16 output tiles, lane (j = lane & 15,
// g = lane >> 4) holds rows 4g..4g+3 of column j; a K = 32 operand fragment gives lane (j, g)
// the contraction indices 8g..8g+7 of its row j. Here every product is written
// out[m][n] = sum_k A[m][k] Bt[n][k], with both operands read by row m (n) and index k.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lla_kernels.hpp"

namespace lla {
namespace bwd {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* log_a;
  const void* lam;  // float32, or bfloat16 when lam_bf16
  int lam_bf16;
  void* gq;
  void* gk;
  void* gv;
  float* glog_a;
  float* glam;
  float* node;    // [BH][nslot][dk*dv]: forward Fenwick nodes over chunks, all block levels
  float* gsum;    // [BH][nslot]: total log decay of each block
  float* rnp;     // [BH][items][dk*dv]: target-side block states, one per sub-block (see bwd_rn)
  float* outs;    // [BH][nslot][dk*dv]: down-sweep values (only when the tree cannot keep them on chip)
  void* node_e;   // [BH][nslot][dk*dv] in the element type: the nodes as the gradient kernel reads them
  void* u_e;      // [BH][N][dk*dv] in the element type: each chunk's combined right-sibling state
  void* node_lo;  // bf16 only: node - bf16(node), so that hi + lo carries ~16 mantissa bits
  void* u_lo;     // bf16 only: the same for the combined right-sibling states
  float* ud;      // [BH][ceil(N/8)][dk*dv], in place of u_e when the gradient kernel forms U_c
                  // itself: what each group of 8 chunks receives from the levels above 2
  float* dA;      // [BH][T]
  int BH, T, L, N, nl, nslot;
  int items;                  // sub-blocks per head over all levels
  int rn_off[kLamCap + 1];    // first sub-block of each level
  int lvl[kLamCap + 1];       // first tree slot of each level (slot_of(N, i, 0))
  int gtlv[kLamCap + 1];      // bwd_gtree: first shared slot of level i's block values (i >= 3)
  int gtct[kLamCap + 1];      // bwd_gtree: first shared slot of level i's contributions (i >= 4)
};

// slot of block (i, m) from the level offsets the host computed (no loop over the levels)
__device__ __forceinline__ int slot_p(const BwdParams& p, int i, int m) { return p.lvl[i] + m; }

// lambda element i (float32, or bfloat16 widened exactly)
__device__ __forceinline__ float lambda_at(const BwdParams& p, size_t i) {
  if (p.lam_bf16) {
    const unsigned short b = reinterpret_cast<const unsigned short*>(p.lam)[i];
    return __builtin_bit_cast(float, (unsigned)b << 16);
  }
  return reinterpret_cast<const float*>(p.lam)[i];
}

// Sub-blocks of the target side. At chunk level j the right blocks (2^j chunks) are split into
// sub-blocks of 2^s chunks, s = min(j, kSubLog): sub-block sb (chunks sb << s ..) belongs to a
// right block when bit j - s of sb is set. The k-th such sub-block of level j:
constexpr int kSubLog = 3;
__host__ __device__ inline int sub_log(int j) { return j < kSubLog ? j : kSubLog; }
__host__ __device__ inline int sub_of_item(int j, int k) {
  const int b = j - sub_log(j);
  return ((k >> b) << (b + 1)) | (1 << b) | (k & ((1 << b) - 1));
}
__host__ __device__ inline int item_of_sub(int j, int sb) {
  const int b = j - sub_log(j);
  return ((sb >> (b + 1)) << b) | (sb & ((1 << b) - 1));
}
// sub-blocks of level j that hold at least one of the N chunks (bit j - s set in [0, ceil(N/2^s)))
__host__ __device__ inline int items_of_level(int N, int j) {
  const int s = sub_log(j), b = j - s;
  const int M = (N + (1 << s) - 1) >> s;
  const int rem = M & ((2 << b) - 1);
  return ((M >> (b + 1)) << b) + (rem > (1 << b) ? rem - (1 << b) : 0);
}

// bwd_rn's processing order (the items' places in the workspace are unchanged): group by group
// of 8 chunks, each group's items of levels 0..2 (its odd chunks, odd pairs, odd quad) and then
// the levels >= 3 whose right blocks hold it, so that every read of a group's q and dO rows after
// the first comes from L2. Position x of the order -> level j and sub-block sb: the group by a
// binary search over the closed-form count of items before each group (every group but the
// last is whole), then the item inside it.
__host__ __device__ inline int rn_items_before(int nl, int g) {
  int n = g * ((nl > 0 ? 4 : 0) + (nl > 1 ? 2 : 0) + (nl > 2 ? 1 : 0));
  for (int j = 3; j < nl; ++j) {   // groups g' < g with bit j - 3 set
    const int b = j - 3, rem = (g & ((2 << b) - 1)) - (1 << b);
    n += ((g >> (b + 1)) << b) + (rem > 0 ? rem : 0);
  }
  return n;
}
__host__ __device__ inline void rn_item_at(int N, int nl, int x, int& j, int& sb) {
  int lo = 0, hi = ((N + 7) >> 3) - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (rn_items_before(nl, mid) <= x) lo = mid;
    else hi = mid - 1;
  }
  const int g = lo;
  int r = x - rn_items_before(nl, g);
  for (int h = 0; h < 4 && nl > 0; ++h)
    if (8 * g + 2 * h + 1 < N && r-- == 0) { j = 0; sb = 8 * g + 2 * h + 1; return; }
  for (int h = 0; h < 2 && nl > 1; ++h)
    if (4 * g + 2 * h + 1 < ((N + 1) >> 1) && r-- == 0) { j = 1; sb = 4 * g + 2 * h + 1; return; }
  if (nl > 2 && 2 * g + 1 < ((N + 3) >> 2) && r-- == 0) { j = 2; sb = 2 * g + 1; return; }
  for (j = 3; j < nl; ++j)
    if (((g >> (j - 3)) & 1) && r-- == 0) { sb = g; return; }
  j = 0; sb = 0;   // not reached for x < items
}

// slot of block (i, m) in the per-head tree: blocks of level i' < i come first
__host__ __device__ inline int slot_of(int N, int i, int m) {
  int o = 0;
  for (int a = 0; a < i; ++a) o += (N + (1 << a) - 1) >> a;
  return o + m;
}

// shared-memory layout of bwd_states / bwd_grads (host and device agree)
struct BwdSmem {
  int q, k, v, o, p1, p2, lam, al, ea, ws, ust, cg, dqd, total;
};

__host__ __device__ inline BwdSmem bwd_smem(int es, int C, int DK, int DV, bool grads) {
  BwdSmem s{};
  int off = 0;
  auto take = [&](int bytes) { const int o = off; off += (bytes + 15) & ~15; return o; };
  const int rk = DK + 16 / es, rv = DV + 16 / es, rc = C + 16 / es;
  s.q = take(C * rk * es);
  s.k = take(C * rk * es);
  s.v = take(C * rv * es);
  s.o = take(C * rv * es);
  s.p1 = grads ? take(C * rc * es) : off;
  // P2, and (bf16) once the intra-chunk products are done, the low part of a [dk][dv] state image
  s.p2 = grads ? take((es == 2 && DK * rv > C * rc ? DK * rv : C * rc) * es) : off;
  s.lam = take(C * kLamCap * 4);
  s.al = take(C * 4);
  s.ea = take(C * 4);
  s.ws = take(C * 4);
  // a [dk][dv] state image: the combined right-sibling state
  s.ust = grads ? take(DK * rv * es) : off;
  s.cg = grads ? take(4 * C * 4) : off;   // per-wave column sums of G = M S W
  s.dqd = grads ? take(C * 4) : off;       // q . (dq from the nodes), per position
  s.total = (off + 255) & ~255;
  return s;
}

template <int C>
struct Waves {
  static constexpr int NW = C >= 64 ? 4 : C / 16;   // waves per workgroup
  static constexpr int RB = C / 16 / NW;             // 16-row blocks of positions per wave
};

// ----------------------------------------------------------------------------------------
// fragments
// ----------------------------------------------------------------------------------------

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

// X[r][k .. k+7] of a row-major shared-memory image with row stride RS (k a multiple of 8);
// indices at or past K read as zero
template <typename T, int K>
__device__ __forceinline__ Frag<T> frag_row(const T* img, int RS, int r, int k) {
  if (k >= K) return zero_frag<T>();
  const T* p = img + r * RS + k;
  if constexpr (sizeof(T) == 2) {
    Frag<T> f;
    f.v = *reinterpret_cast<const bf16x8*>(p);
    return f;
  } else {
    Frag<T> f;
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 4);
    return f;
  }
}

// X[k .. k+7][c] (a column of the image), each element times sc[k + e] when sc is given
// (k a multiple of 8, the same in each 16-lane group; c = c0 + (lane & 15) with c0 a multiple of
// 16). bf16: two transposing reads (ds_read_tr16_b64). In each 16-lane group such a read gives
// lane i, as its element e, element i % 4 of the 4-element piece addressed by lane 4e + i / 4;
// so lane L addresses row k + L / 4 (then k + 4 + L / 4), columns c0 + 4 (L % 4) .. + 3.
// f32: element-wise reads.
template <typename T, int K>
__device__ __forceinline__ Frag<T> frag_col(const T* img, int RS, int k, int c,
                                            const float* sc = nullptr) {
  const bool ok = k < K;
  const int kk = ok ? k : 0;
  f32x4 lo, hi;
  if constexpr (sizeof(T) == 2) {
    const int L = c & 15, c0 = c - L;
    const T* p = img + (kk + (L >> 2)) * RS + c0 + 4 * (L & 3);
    const s16x4 a = ds_read_tr(reinterpret_cast<const unsigned char*>(p));
    const s16x4 b = ds_read_tr(reinterpret_cast<const unsigned char*>(p + 4 * RS));
    Frag<T> f;
    f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    if (!ok) return zero_frag<T>();
    if (!sc) return f;
    frag_to_f32(f, lo, hi);
  } else {
    if (!ok) return zero_frag<T>();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = to_f(img[(k + e) * RS + c]);
      hi[e] = to_f(img[(k + 4 + e) * RS + c]);
    }
    if (!sc) return frag_from<T>(lo, hi);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    lo[e] *= sc[k + e];
    hi[e] *= sc[k + 4 + e];
  }
  return frag_from<T>(lo, hi);
}

// x * sc (a scaled column fragment) as hi + lo with hi = bf16(x sc), lo = bf16(x sc - hi), so
// that a product with it keeps ~16 mantissa bits of the weights; fp32: lo = 0
template <typename T, int K>
__device__ __forceinline__ void frag_col_split(const T* img, int RS, int k, int c, const float* sc,
                                               Frag<T>& hi, Frag<T>& lo) {
  const Frag<T> f = frag_col<T, K>(img, RS, k, c, sc);
  if constexpr (sizeof(T) == 2) {
    // recompute the exact products in fp32 from the unscaled elements
    const Frag<T> u = frag_col<T, K>(img, RS, k, c);
    f32x4 ulo, uhi, hlo, hhi;
    frag_to_f32(u, ulo, uhi);
    frag_to_f32(f, hlo, hhi);
    if (k < K) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ulo[e] = ulo[e] * sc[k + e] - hlo[e];
        uhi[e] = uhi[e] * sc[k + 4 + e] - hhi[e];
      }
    }
    hi = f;
    lo = frag_from<T>(ulo, uhi);
  } else {
    hi = f;
    lo = zero_frag<T>();
  }
}

// a row-major float state in global memory, g[r][k .. k+7] (row stride RS), as an operand
template <typename T, int K>
__device__ __forceinline__ Frag<T> frag_grow(const float* g, int RS, int r, int k) {
  if (k >= K) return zero_frag<T>();
  const float* p = g + (size_t)r * RS + k;
  const f32x4 lo = *reinterpret_cast<const f32x4*>(p);
  const f32x4 hi = *reinterpret_cast<const f32x4*>(p + 4);
  return frag_from<T>(lo, hi);
}

// lane l's value of x (a scalar read: every lane gets the same value)
__device__ __forceinline__ float lane_f(float x, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), l));
}
__device__ __forceinline__ int lane_i(int x, int l) { return __builtin_amdgcn_readlane(x, l); }

// x summed over the four 16-lane rows (lanes l, l ^ 16, l ^ 32, l ^ 48): exchanging the odd rows
// of x with the even rows of a copy (v_permlane16_swap) leaves x[l] and x[l ^ 16] in the two
// registers of every lane; the same with the wave's halves (v_permlane32_swap) for l ^ 32
__device__ __forceinline__ float sum_rows(float x) {
  const unsigned xi = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane16_swap(xi, xi, false, false);
  const unsigned a0 = r[0], a1 = r[1];   // copied out before the casts (element reads)
  const float y = __builtin_bit_cast(float, a0) + __builtin_bit_cast(float, a1);
  const unsigned yi = __builtin_bit_cast(unsigned, y);
  const auto r2 = __builtin_amdgcn_permlane32_swap(yi, yi, false, false);
  const unsigned b0 = r2[0], b1 = r2[1];
  return __builtin_bit_cast(float, b0) + __builtin_bit_cast(float, b1);
}

// x from another lane of the same 16-lane row through a DPP move (the vector unit, not the
// shared-memory permute that a generic shuffle compiles to): quad_perm patterns 0xB1 ([1,0,3,2])
// and 0x4E ([2,3,0,1]); row_ror:4 = 0x124, row_ror:8 = 0x128
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}

// a wave-uniform global address as the compiler's uniform value (both halves read from lane 0;
// global address space): an access at it plus a lane offset then takes the scalar-base form
// instead of a 64-bit address per lane
template <typename P>
__device__ __forceinline__ __attribute__((address_space(1))) P* uniform_ptr(P* ptr) {
  const uint64_t a = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  return (__attribute__((address_space(1))) P*)(((uint64_t)hi << 32) | lo);
}

// x from lane (lane ^ 4) of the same row: half_mirror (lane 7 - i of each 8) then quad_perm
// [3,2,1,0] (lane i ^ 3)
__device__ __forceinline__ float dpp_xor4(float x) { return dpp_f<0x1B>(dpp_f<0x141>(x)); }

// sum over the 16 lanes of a row (lane & 15 varies), in every lane: pairs, quads, then the
// quads 4 and 8 lanes around the row
__device__ __forceinline__ float sum16(float x) {
  x += dpp_f<0xB1>(x);
  x += dpp_f<0x4E>(x);
  x += dpp_f<0x124>(x);
  x += dpp_f<0x128>(x);
  return x;
}

// four row values x[0..3] (rows 0..3 of a lane's row group) each summed over the 16 lanes of the
// row; lane j receives the sum of row j & 3. Two exchange steps halve the values a lane carries
// (lanes j, j ^ 1 keep rows of opposite low bit; then j, j ^ 2 of opposite high bit), two
// rotations add the lanes 4 and 8 apart: 11 vector instructions instead of four sums of 4 DPP
// adds each
__device__ __forceinline__ float sum16x4(const float (&x)[4], int jj) {
  const bool b0 = jj & 1, b1 = jj & 2;
  const float y0 = (b0 ? x[1] : x[0]) + dpp_f<0xB1>(b0 ? x[0] : x[1]);
  const float y1 = (b0 ? x[3] : x[2]) + dpp_f<0xB1>(b0 ? x[2] : x[3]);
  float z = (b1 ? y1 : y0) + dpp_f<0x4E>(b1 ? y0 : y1);
  z += dpp_f<0x124>(z);
  z += dpp_f<0x128>(z);
  return z;
}

// kernel table of one (dtype, chunk, dk, dv)
struct BwdKernels {
  const void* states;   // bwd_states_kernel<T, C, DK, DV>
  const void* statesg;  // bwd_statesg_kernel<T, C, DK, DV> where its states fit, else null
  const void* rn;       // bwd_rn_kernel<T, C, DK, DV>
  const void* rng;      // bwd_rng_kernel<T, C, DK, DV> where its accumulators fit, else null
  const void* grads;    // bwd_grads_kernel<T, C, DK, DV>
  const void* grads_d;  // bwd_grads_kernel<T, C, DK, DV, true>: forms U_c from the tree's group states
};

// per (dtype, chunk) tables, one instantiation unit each; nullptr outside {16,32,64,128}
const BwdKernels* bwd_kernels_bf16_c16(int DK, int DV);
const BwdKernels* bwd_kernels_bf16_c32(int DK, int DV);
const BwdKernels* bwd_kernels_bf16_c64(int DK, int DV);
const BwdKernels* bwd_kernels_f32_c16(int DK, int DV);
const BwdKernels* bwd_kernels_f32_c32(int DK, int DV);
const BwdKernels* bwd_kernels_f32_c64(int DK, int DV);

// ----------------------------------------------------------------------------------------
// shared staging of one chunk: q, k, v, do images, lambda rows, decays
// ----------------------------------------------------------------------------------------

template <typename T, int C, int DK, int DV>
struct Chunk {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int RK = DK + 16 / ES, RV = DV + 16 / ES;
  T *q, *k, *v, *o;
  float *lam, *al, *ea, *ws;
  float g;   // total log decay of the chunk

  __device__ void bind(unsigned char* sm, const BwdSmem& L) {
    q = reinterpret_cast<T*>(sm + L.q);
    k = reinterpret_cast<T*>(sm + L.k);
    v = reinterpret_cast<T*>(sm + L.v);
    o = reinterpret_cast<T*>(sm + L.o);
    lam = reinterpret_cast<float*>(sm + L.lam);
    al = reinterpret_cast<float*>(sm + L.al);
    ea = reinterpret_cast<float*>(sm + L.ea);
    ws = reinterpret_cast<float*>(sm + L.ws);
  }

  // one image's rows [0, nv) in registers on their way into shared memory, in 16-byte pieces
  // (rows past nv are written as zeros). Every load is unconditional, from a clamped row of the
  // chunk (nv >= 1): with no load under a branch the compiler's counted waits stay exact, so a
  // wait for these loads never drains loads issued after them.
  template <int D, int NT>
  struct Rows {
    static constexpr int EPV = 16 / ES, NVR = D / EPV, RS = D + 16 / ES, NP = C * NVR;
    static constexpr int PER = (NP + NT - 1) / NT;
    u32x4 r[PER];
    __device__ __forceinline__ void fetch(const T* g, int nv, int tid) {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int idx = min(tid + u * NT, NP - 1), row = min(idx / NVR, nv - 1);
        r[u] = *reinterpret_cast<const u32x4*>(g + (size_t)row * D + (idx % NVR) * EPV);
      }
    }
    __device__ __forceinline__ void put(T* img, int nv, int tid) const {
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int idx = tid + u * NT;
        if (idx < NP)
          *reinterpret_cast<u32x4*>(img + (idx / NVR) * RS + (idx % NVR) * EPV) =
              idx / NVR < nv ? r[u] : u32x4{0u, 0u, 0u, 0u};
      }
    }
  };

  // everything of chunk c of head bh: fetch() issues every global load into registers (raw words,
  // unconditional, from clamped indices), put() writes the images, the lambda rows and (wave 0,
  // after its chunk-local scan of log_a) the decays, without a barrier. Between the two a caller
  // may issue loads of its own; the chunk then costs one memory round trip whatever else is in
  // flight. A = chunk-local inclusive prefix of log_a, ea = exp(A), ws = exp(g - A) (decay from
  // a position to the chunk's end).
  // KV: k and v images; QO: q and do images; LAM: all lambda rows (else none)
  template <int NT, bool KV = true, bool QO = true, bool LAM = true>
  struct Staged {
    static_assert(C <= 64, "one lane per position in the log_a scan");
    static constexpr int PL = (C * kLamCap + NT - 1) / NT;
    Rows<DK, NT> rq, rk;
    Rows<DV, NT> rv, ro;
    unsigned lm[LAM ? PL : 1];   // lambda: float32 bits, or bfloat16 bits in the low half
    float la;
    int nv, L, bf;

    __device__ __forceinline__ void fetch(const BwdParams& p, int bh, int c, int nv_, int tid) {
      nv = nv_;
      L = p.L;
      bf = p.lam_bf16;
      const size_t row0 = (size_t)bh * p.T + (size_t)c * C;
      // lambda first: its two kinds of loads sit in the two arms of a branch, and a wait the
      // compiler puts at the start of one arm then has nothing else to drain
      if (LAM) {
        const size_t base = row0 * p.L;
        if (bf) {
          const unsigned short* lp = reinterpret_cast<const unsigned short*>(p.lam) + base;
#pragma unroll
          for (int u = 0; u < PL; ++u) {
            const int i = min(tid + u * NT, C * kLamCap - 1);
            lm[u] = lp[(size_t)min(i / kLamCap, nv - 1) * p.L + min(i % kLamCap, p.L - 1)];
          }
        } else {
          const unsigned* lp = reinterpret_cast<const unsigned*>(p.lam) + base;
#pragma unroll
          for (int u = 0; u < PL; ++u) {
            const int i = min(tid + u * NT, C * kLamCap - 1);
            lm[u] = lp[(size_t)min(i / kLamCap, nv - 1) * p.L + min(i % kLamCap, p.L - 1)];
          }
        }
      }
      la = p.log_a[row0 + min(tid, nv - 1)];
      if (QO) rq.fetch(reinterpret_cast<const T*>(p.q) + row0 * DK, nv, tid);
      if (KV) rk.fetch(reinterpret_cast<const T*>(p.k) + row0 * DK, nv, tid);
      if (KV) rv.fetch(reinterpret_cast<const T*>(p.v) + row0 * DV, nv, tid);
      if (QO) ro.fetch(reinterpret_cast<const T*>(p.dout) + row0 * DV, nv, tid);
    }

    __device__ __forceinline__ void put(Chunk& ch, int tid) const {
      if (QO) rq.put(ch.q, nv, tid);
      if (KV) rk.put(ch.k, nv, tid);
      if (KV) rv.put(ch.v, nv, tid);
      if (QO) ro.put(ch.o, nv, tid);
      // every level slot is written: rows past nv and levels past L are zero weights
      if (LAM)
#pragma unroll
        for (int u = 0; u < PL; ++u) {
          const int i = tid + u * NT;
          const float x = __builtin_bit_cast(float, bf ? lm[u] << 16 : lm[u]);
          if (i < C * kLamCap) ch.lam[i] = (i / kLamCap < nv && i % kLamCap < L) ? x : 0.f;
        }
      if (tid < 64) {
        const float incl = wave_scan<false>((tid < C && tid < nv) ? la : 0.f);
        const float tot = lane_f(incl, 63);
        if (tid < C) {
          ch.al[tid] = incl;
          ch.ea[tid] = __expf(incl);
          ch.ws[tid] = __expf(tot - incl);
        }
      }
    }
  };

  // after put() and a barrier: the chunk's total log decay
  __device__ __forceinline__ void finish() { g = al[C - 1]; }

  // fetch, put, barrier
  template <int NT, bool KV = true, bool QO = true, bool LAM = true>
  __device__ void load(const BwdParams& p, int bh, int c, int nv, int tid) {
    Staged<NT, KV, QO, LAM> st;
    st.fetch(p, bh, c, nv, tid);
    st.put(*this, tid);
    __syncthreads();
    finish();
  }
};

// Tiles of a DK x DV product out[a][b] = sum_k A[k][a] B'[k][b] whose B' is a scaled (and, in
// bf16, hi + lo split) operand: the waves split the b (column) dimension first, so that each
// wave scales the columns it uses once per contraction step and reuses them for every a block
// it holds (splitting a first would have every wave scale every column). Wave w holds YPW
// column blocks y(w, ya) and, for each, APW row blocks ab(w, b) (possibly past DK / 16 when
// there are more waves than tiles: such tiles are computed on zeros and not stored); tile
// ya * APW + b of its accumulators.
template <int DK, int DV, int NW>
struct ScaledTiles {
  static constexpr int NAT = DK / 16, NYT = DV / 16;
  static constexpr bool BYCOL = NYT >= NW;                     // every wave its own columns
  static constexpr int YPW = BYCOL ? NYT / NW : 1;
  static constexpr int APW = BYCOL ? NAT : cdiv(NAT, NW / NYT);
  static constexpr int TPW = YPW * APW;
  __device__ static constexpr int y(int w, int ya) { return BYCOL ? w + NW * ya : w % NYT; }
  __device__ static constexpr int ab(int w, int b) { return BYCOL ? b : w / NYT + (NW / NYT) * b; }
  // the wave's tiles, row-major with row stride LD floats
  template <int LD>
  __device__ static void store(float* dst, const f32x4* acc, int w, int lane) {
    const int jj = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int ya = 0; ya < YPW; ++ya)
#pragma unroll
      for (int b = 0; b < APW; ++b) {
        const int a0 = ab(w, b);
        if (a0 >= NAT) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          dst[(size_t)(a0 * 16 + 4 * g4 + r) * LD + y(w, ya) * 16 + jj] = acc[ya * APW + b][r];
      }
  }
};

// x (8 contraction elements as float, lo = first 4) times sc[0..7] as an MFMA operand pair
// hi + lo: hi = x sc rounded to T, lo = the rounding error rounded to T (zero for float32)
template <typename T>
__device__ __forceinline__ void scale_split(const f32x4& ulo, const f32x4& uhi, const float* sc,
                                            Frag<T>& hi, Frag<T>& lo) {
  f32x4 xa, xb;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    xa[e] = ulo[e] * sc[e];
    xb[e] = uhi[e] * sc[4 + e];
  }
  hi = frag_from<T>(xa, xb);
  if constexpr (sizeof(T) == 2) {
    f32x4 ha, hb;
    frag_to_f32(hi, ha, hb);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      xa[e] -= ha[e];
      xb[e] -= hb[e];
    }
    lo = frag_from<T>(xa, xb);
  } else {
    lo = zero_frag<T>();
  }
}

// ----------------------------------------------------------------------------------------
// bwd_states: chunk state F(c) and the right-block partials Z(c, j)
// ----------------------------------------------------------------------------------------

// out[a][b] = sum_s X[s][a] * sc[s] * Y[s][b] over the chunk's positions (a < DA, b < DB),
// stored row-major into dst (fp32); the waves split the tiles as ScaledTiles (the scaled
// Y columns once per wave)
template <typename T, int C, int DA, int DB, int NW>
__device__ __forceinline__ void outer_store(const T* X, int RX, const T* Y, int RY, const float* sc,
                                            float* __restrict__ dst, int w, int lane) {
  using TM = ScaledTiles<DA, DB, NW>;
  const int jj = lane & 15, g4 = lane >> 4;
  f32x4 acc[TM::TPW];
#pragma unroll
  for (int i = 0; i < TM::TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s0 = 0; s0 < C; s0 += 32) {
    const int k = s0 + 8 * g4;
    Frag<T> a[TM::APW];
#pragma unroll
    for (int b = 0; b < TM::APW; ++b) {
      const int ab = TM::ab(w, b);
      a[b] = ab < DA / 16 ? frag_col<T, C>(X, RX, k, ab * 16 + jj) : zero_frag<T>();
    }
#pragma unroll
    for (int ya = 0; ya < TM::YPW; ++ya) {
      const Frag<T> uy = frag_col<T, C>(Y, RY, k, TM::y(w, ya) * 16 + jj);
      f32x4 ulo, uhi;
      frag_to_f32(uy, ulo, uhi);
      Frag<T> bh, bl;
      scale_split<T>(ulo, uhi, sc + (k < C ? k : 0), bh, bl);
#pragma unroll
      for (int b = 0; b < TM::APW; ++b) {
        mma(acc[ya * TM::APW + b], a[b], bh);
        if constexpr (sizeof(T) == 2) mma(acc[ya * TM::APW + b], a[b], bl);
      }
    }
  }
  TM::template store<DB>(dst, acc, w, lane);
}

template <typename T, int C, int DK, int DV>
__global__ void __launch_bounds__(64 * Waves<C>::NW)
bwd_states_kernel(BwdParams p) {
  constexpr int NW = Waves<C>::NW, NT = 64 * NW;
  using CH = Chunk<T, C, DK, DV>;
  extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int nv = min(C, p.T - c * C);
  const BwdSmem Lo = bwd_smem((int)sizeof(T), C, DK, DV, false);
  CH ch;
  ch.bind(sm, Lo);
  ch.template load<NT, true, false, false>(p, bh, c, nv, tid);
  const size_t SZ = (size_t)DK * DV;
  // F(c): keys weighted by their decay to the chunk's end
  outer_store<T, C, DK, DV, NW>(ch.k, CH::RK, ch.v, CH::RV, ch.ws,
                                p.node + ((size_t)bh * p.nslot + c) * SZ, w, lane);
  if (tid == 0) p.gsum[(size_t)bh * p.nslot + c] = ch.g;
}

// ----------------------------------------------------------------------------------------
// bwd_statesg: the chunk states by groups of 8 chunks (a sub-block of level 3) and head, with
// the group's part of the forward nodes' up-sweep. Chunk by chunk, F(c) on MFMA; then in
// registers node(1, m) = exp(G(0, 2m+1)) node(0, 2m) + node(0, 2m+1), and the same for levels
// 2 and 3 (chunks past N are zero states with zero decay, so a block without its right half
// keeps its left one; the block decays are formed as bwd_gsum forms them). Every even node of
// levels 0..3 is written as the gradient kernel's MFMA operands (element type; bf16 as high and
// low parts), the group itself (level 3) also in fp32 for the levels above it; g_c into the
// block decays. Used with bwd_gtree, where its four states fit the registers.
// ----------------------------------------------------------------------------------------

template <typename T, int C, int DK, int DV>
__global__ void __launch_bounds__(64 * Waves<C>::NW) __attribute__((amdgpu_waves_per_eu(2)))
bwd_statesg_kernel(BwdParams p) {
  constexpr int NW = Waves<C>::NW, NT = 64 * NW;
  using TM = ScaledTiles<DK, DV, NW>;
  constexpr int TPW = TM::TPW;
  constexpr int ES = (int)sizeof(T), EPV = 16 / ES;
  constexpr int PK = C * DK / EPV, PV = C * DV / EPV;        // 16-byte pieces of the k, v rows
  constexpr int NKP = cdiv(PK, NT), NVP = cdiv(PV, NT);
  constexpr bool SPLIT = ES == 2;
  using CH = Chunk<T, C, DK, DV>;
  extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
  const int ng = (p.N + 7) >> 3;
  // one-dimensional grid in XCD order, as in bwd_grads
  const int Lw = blockIdx.x, q8 = Lw >> 3;
  const bool xcd = (p.BH & 7) == 0;
  const int g = xcd ? q8 % ng : Lw % ng;
  const int bh = xcd ? ((q8 / ng) << 3) + (Lw & 7) : Lw / ng;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, jj = lane & 15, g4 = lane >> 4;
  const int c0 = g << 3, c1 = min(c0 + 8, p.N);
  const BwdSmem Lo = bwd_smem(ES, C, DK, DV, false);
  CH ch;
  ch.bind(sm, Lo);
  const size_t SZ = (size_t)DK * DV;
  T* ne = reinterpret_cast<T*>(p.node_e) + (size_t)bh * p.nslot * SZ;
  T* nlo = reinterpret_cast<T*>(p.node_lo) + (size_t)bh * p.nslot * SZ;
  float* gsum = p.gsum + (size_t)bh * p.nslot;
  auto nb = [&](int i) { return (p.N + (1 << i) - 1) >> i; };
  // the wave's tiles of a state into slot s, as MFMA operands in the element type (a uniform
  // base per tile and row step, the lane's offset added last)
  const unsigned lofs = (unsigned)(4 * g4 * DV + jj);
  auto put = [&](int s, const f32x4* X) {
#pragma unroll
    for (int ya = 0; ya < TM::YPW; ++ya)
#pragma unroll
      for (int b = 0; b < TM::APW; ++b) {
        const int a0 = TM::ab(w, b);
        if (a0 >= DK / 16) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const size_t at = (size_t)s * SZ + (size_t)(a0 * 16 + r) * DV + TM::y(w, ya) * 16;
          const float x = X[ya * TM::APW + b][r];
          const T hv = (T)x;
          uniform_ptr(ne + at)[lofs] = hv;
          if constexpr (SPLIT) uniform_ptr(nlo + at)[lofs] = (T)(x - (float)hv);
        }
      }
  };

  // the next chunk's k and v rows and log_a, in registers (unconditional, clamped)
  u32x4 rk[NKP], rv[NVP];
  float rla = 0.f;
  auto fetch = [&](int c) {
    const int nv = min(C, p.T - c * C);
    const size_t row0 = (size_t)bh * p.T + (size_t)c * C;
    const u32x4* gk = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.k) + row0 * DK);
    const u32x4* gv = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.v) + row0 * DV);
#pragma unroll
    for (int u = 0; u < NKP; ++u) {
      const int idx = min(tid + u * NT, PK - 1);
      rk[u] = gk[min(idx / (DK / EPV), nv - 1) * (DK / EPV) + idx % (DK / EPV)];
    }
#pragma unroll
    for (int u = 0; u < NVP; ++u) {
      const int idx = min(tid + u * NT, PV - 1);
      rv[u] = gv[min(idx / (DV / EPV), nv - 1) * (DV / EPV) + idx % (DV / EPV)];
    }
    rla = p.log_a[row0 + min(lane, nv - 1)];
  };
  fetch(c0);
  f32x4 F[TPW], K0[TPW], K1[TPW], K2[TPW];
  float gl0 = 0.f, G1L = 0.f, G2L = 0.f;   // decays of the left chunk, pair and quad
#pragma unroll 1
  for (int l = 0; l < 8; ++l) {
    const int c = c0 + l;
    float gc = 0.f;
#pragma unroll
    for (int i = 0; i < TPW; ++i) F[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (c < c1) {
      const int nv = min(C, p.T - c * C);
      if (l > 0) __syncthreads();   // the previous chunk's images are no longer read
#pragma unroll
      for (int u = 0; u < NKP; ++u) {
        const int idx = tid + u * NT;
        if (idx < PK) {
          const int r = idx / (DK / EPV), f = (idx % (DK / EPV)) * EPV;
          *reinterpret_cast<u32x4*>(ch.k + r * CH::RK + f) = r < nv ? rk[u] : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < NVP; ++u) {
        const int idx = tid + u * NT;
        if (idx < PV) {
          const int r = idx / (DV / EPV), f = (idx % (DV / EPV)) * EPV;
          *reinterpret_cast<u32x4*>(ch.v + r * CH::RV + f) = r < nv ? rv[u] : u32x4{0u, 0u, 0u, 0u};
        }
      }
      // every wave scans the chunk's log_a; wave 0 writes the weights exp(g_c - A_s)
      const float incl = wave_scan<false>(lane < nv ? rla : 0.f);
      gc = lane_f(incl, 63);
      if (w == 0 && lane < C) ch.ws[lane] = __expf(gc - incl);
      __syncthreads();
      if (c + 1 < c1) fetch(c + 1);
      // F(c) = k^T (ws * v), the wave's tiles
#pragma unroll
      for (int s0 = 0; s0 < C; s0 += 32) {
        const int k = s0 + 8 * g4;
        Frag<T> a[TM::APW];
#pragma unroll
        for (int b = 0; b < TM::APW; ++b) {
          const int ab = TM::ab(w, b);
          a[b] = ab < DK / 16 ? frag_col<T, C>(ch.k, CH::RK, k, ab * 16 + jj) : zero_frag<T>();
        }
#pragma unroll
        for (int ya = 0; ya < TM::YPW; ++ya) {
          const Frag<T> uy = frag_col<T, C>(ch.v, CH::RV, k, TM::y(w, ya) * 16 + jj);
          f32x4 ulo, uhi;
          frag_to_f32(uy, ulo, uhi);
          Frag<T> bh_, bl_;
          scale_split<T>(ulo, uhi, ch.ws + (k < C ? k : 0), bh_, bl_);
#pragma unroll
          for (int b = 0; b < TM::APW; ++b) {
            mma(F[ya * TM::APW + b], a[b], bh_);
            if constexpr (SPLIT) mma(F[ya * TM::APW + b], a[b], bl_);
          }
        }
      }
      if (tid == 0) gsum[c] = gc;
    }
    // the group's up-sweep (levels 0..3): even nodes out, the left halves kept
    if (!(l & 1)) {
      if (c < c1) put(c, F);
#pragma unroll
      for (int i = 0; i < TPW; ++i) K0[i] = F[i];
      gl0 = gc;
      continue;
    }
    const float eg1 = __expf(gc);
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) F[i][r] = eg1 * K0[i][r] + F[i][r];   // node(1, c >> 1)
    const float G1 = c < c1 ? gl0 + gc : gl0;
    const int m1 = c >> 1;
    if (!(l & 2)) {
      if (1 < p.nl && m1 < nb(1)) put(slot_p(p, 1, m1), F);
#pragma unroll
      for (int i = 0; i < TPW; ++i) K1[i] = F[i];
      G1L = G1;
      continue;
    }
    const bool right1 = (m1 < nb(1));   // the right pair holds at least one chunk
    const float eg2 = __expf(right1 ? G1 : 0.f);
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) F[i][r] = eg2 * K1[i][r] + F[i][r];   // node(2, c >> 2)
    const float G2 = right1 ? G1L + G1 : G1L;
    const int m2 = c >> 2;
    if (!(l & 4)) {
      if (2 < p.nl && m2 < nb(2)) put(slot_p(p, 2, m2), F);
#pragma unroll
      for (int i = 0; i < TPW; ++i) K2[i] = F[i];
      G2L = G2;
      continue;
    }
    const bool right2 = (m2 < nb(2));
    const float eg3 = __expf(right2 ? G2 : 0.f);
#pragma unroll
    for (int i = 0; i < TPW; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) F[i][r] = eg3 * K2[i][r] + F[i][r];   // the group: node(3, g)
    if (3 < p.nl) {
      if (!(g & 1)) put(slot_p(p, 3, g), F);
      TM::template store<DV>(p.node + ((size_t)bh * p.nslot + slot_p(p, 3, g)) * SZ, F, w, lane);
    }
  }
  (void)G2L;
}

// ----------------------------------------------------------------------------------------
// bwd_rn: one target-side sub-block state per workgroup,
//   P(j, sb) = sum over the positions t of sub-block sb of lambda[t, J+1+j] exp(A_t - A_0) q_t do_t^T
// with A_0 the prefix decay just before the sub-block, accumulated chunk by chunk on MFMA
// ----------------------------------------------------------------------------------------

template <typename T, int C, int DK, int DV>
__global__ void __launch_bounds__(64 * Waves<C>::NW)
bwd_rn_kernel(BwdParams p) {
  constexpr int NW = Waves<C>::NW, NT = 64 * NW, J = ilog2(C);
  using TM = ScaledTiles<DK, DV, NW>;
  constexpr int ES = (int)sizeof(T), EPV = 16 / ES;
  constexpr int PQ = C * DK / EPV, PO = C * DV / EPV;        // 16-byte pieces of the q, do rows
  constexpr int NQ = cdiv(PQ, NT), NO = cdiv(PO, NT);
  using CH = Chunk<T, C, DK, DV>;
  extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
  // one-dimensional grid in XCD order, as in bwd_grads: XCD x takes heads x, x + 8, ... (B*H a
  // multiple of 8), a head's items in the group-major order of rn_item_at, so the q and dO rows
  // of a group, read by up to 7 + (nl - 3) items, come from its L2 after the first time
  const int Lw = blockIdx.x, q8 = Lw >> 3;
  const bool xcd = (p.BH & 7) == 0;
  const int x = xcd ? q8 % p.items : Lw % p.items;   // place in the group-major order
  const int bh = xcd ? ((q8 / p.items) << 3) + (Lw & 7) : Lw / p.items;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, jj = lane & 15, g4 = lane >> 4;
  int j, sb;
  rn_item_at(p.N, p.nl, x, j, sb);
  const int item = p.rn_off[j] + item_of_sub(j, sb);
  const int c0 = sb << sub_log(j), c1 = min(c0 + (1 << sub_log(j)), p.N);
  const BwdSmem Lo = bwd_smem(ES, C, DK, DV, false);
  CH ch;
  ch.bind(sm, Lo);
  float* sc = ch.lam;   // per-position weights of the current chunk
  f32x4 acc[TM::TPW];
#pragma unroll
  for (int i = 0; i < TM::TPW; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  // the next chunk's q and do rows, log_a and lambda of level J+1+j, in registers: issued before
  // the current chunk's products so that their latency hides behind them
  u32x4 rq[NQ], ro[NO];
  float rla = 0.f, rlm = 0.f;
  auto fetch = [&](int c) {
    const int nv = min(C, p.T - c * C);
    const size_t row0 = (size_t)bh * p.T + (size_t)c * C;
    const u32x4* gq = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.q) + row0 * DK);
    const u32x4* go = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.dout) + row0 * DV);
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int idx = tid + u * NT;
      rq[u] = (idx < PQ && idx / (DK / EPV) < nv) ? gq[idx] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int idx = tid + u * NT;
      ro[u] = (idx < PO && idx / (DV / EPV) < nv) ? go[idx] : u32x4{0u, 0u, 0u, 0u};
    }
    rla = lane < nv ? p.log_a[row0 + lane] : 0.f;
    rlm = lane < nv ? lambda_at(p, (row0 + lane) * p.L + J + 1 + j) : 0.f;
  };
  fetch(c0);
  float eoff = 0.f;     // log decay from the sub-block's start to the current chunk's start
  for (int c = c0; c < c1; ++c) {
    if (c > c0) __syncthreads();   // the previous chunk's images and weights are no longer read
#pragma unroll
    for (int u = 0; u < NQ; ++u) {
      const int idx = tid + u * NT;
      if (idx < PQ) {
        const int r = idx / (DK / EPV), f = (idx % (DK / EPV)) * EPV;
        *reinterpret_cast<u32x4*>(ch.q + r * CH::RK + f) = rq[u];
      }
    }
#pragma unroll
    for (int u = 0; u < NO; ++u) {
      const int idx = tid + u * NT;
      if (idx < PO) {
        const int r = idx / (DV / EPV), f = (idx % (DV / EPV)) * EPV;
        *reinterpret_cast<u32x4*>(ch.o + r * CH::RV + f) = ro[u];
      }
    }
    // every wave scans the chunk's log_a (C <= 64 positions, one per lane); wave 0 writes the
    // weights lambda * exp(decay from the sub-block's start)
    const float incl = wave_scan<false>(lane < C ? rla : 0.f);
    if (w == 0 && lane < C) sc[lane] = rlm * __expf(eoff + incl);
    eoff += lane_f(incl, C - 1);
    __syncthreads();
    if (c + 1 < c1) fetch(c + 1);
    // the wave's tiles: its do columns scaled and split once per contraction step
#pragma unroll
    for (int s0 = 0; s0 < C; s0 += 32) {
      const int k = s0 + 8 * g4;
      Frag<T> a[TM::APW];
#pragma unroll
      for (int b = 0; b < TM::APW; ++b) {
        const int ab = TM::ab(w, b);
        a[b] = ab < DK / 16 ? frag_col<T, C>(ch.q, CH::RK, k, ab * 16 + jj) : zero_frag<T>();
      }
#pragma unroll
      for (int ya = 0; ya < TM::YPW; ++ya) {
        const Frag<T> uo = frag_col<T, C>(ch.o, CH::RV, k, TM::y(w, ya) * 16 + jj);
        f32x4 ulo, uhi;
        frag_to_f32(uo, ulo, uhi);
        Frag<T> bh_, bl_;
        scale_split<T>(ulo, uhi, sc + (k < C ? k : 0), bh_, bl_);
#pragma unroll
        for (int b = 0; b < TM::APW; ++b) {
          mma(acc[ya * TM::APW + b], a[b], bh_);
          if constexpr (sizeof(T) == 2) mma(acc[ya * TM::APW + b], a[b], bl_);
        }
      }
    }
  }
  TM::template store<DV>(p.rnp + ((size_t)bh * p.items + item) * ((size_t)DK * DV), acc, w, lane);
}

// ----------------------------------------------------------------------------------------
// bwd_rng: the same sub-block states as bwd_rn, with one workgroup per group of 8 chunks (a
// sub-block of every level >= 3) and head, chunk by chunk: the group's q and do rows are read
// once, and every state its chunks belong to is accumulated at the same time. Slots 0..2: the
// right blocks of levels 0, 1, 2 inside the group (a chunk takes part in level j when bit j of
// its index is set; a block's state is stored when its last chunk is done and the slot starts
// over); slots 3..: the group itself, for up to kRgHigh levels j >= 3 whose right blocks hold it
// (bit j - 3 of the group index set), stored at the end; more such levels take another pass
// over the group. The weights of a slot are lambda[t, J+1+j] exp(A_t - A_0), A_0 the prefix
// decay just before the slot's block (the group's start for slots 3..).
// ----------------------------------------------------------------------------------------

constexpr int kRgHigh = 4;

// whether the 3 + kRgHigh accumulators of one wave fit its registers (at most 4 tiles each)
template <int C, int DK, int DV>
constexpr bool rng_fits() {
  return ScaledTiles<DK, DV, Waves<C>::NW>::TPW <= 4;
}

template <typename T, int C, int DK, int DV>
__global__ void __launch_bounds__(64 * Waves<C>::NW) __attribute__((amdgpu_waves_per_eu(2)))
bwd_rng_kernel(BwdParams p) {
  constexpr int NW = Waves<C>::NW, NT = 64 * NW, J = ilog2(C);
  using TM = ScaledTiles<DK, DV, NW>;
  constexpr int TPW = TM::TPW;
  constexpr int ES = (int)sizeof(T), EPV = 16 / ES;
  constexpr int PQ = C * DK / EPV, PO = C * DV / EPV;        // 16-byte pieces of the q, do rows
  constexpr int NQ = cdiv(PQ, NT), NO = cdiv(PO, NT);
  constexpr int NS = 3 + kRgHigh;                            // accumulator slots
  static_assert(NS * C <= C * kLamCap, "slot weights fit the lambda rows");
  using CH = Chunk<T, C, DK, DV>;
  extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
  const int ng = (p.N + 7) >> 3;
  // one-dimensional grid in XCD order, as in bwd_grads
  const int Lw = blockIdx.x, q8 = Lw >> 3;
  const bool xcd = (p.BH & 7) == 0;
  const int g = xcd ? q8 % ng : Lw % ng;
  const int bh = xcd ? ((q8 / ng) << 3) + (Lw & 7) : Lw / ng;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, jj = lane & 15, g4 = lane >> 4;
  const int c0 = g << 3, c1 = min(c0 + 8, p.N);
  const BwdSmem Lo = bwd_smem(ES, C, DK, DV, false);
  CH ch;
  ch.bind(sm, Lo);
  float* scw = ch.lam;   // [slot][position] weights of the current chunk
  const size_t SZ = (size_t)DK * DV;
  float* rnp = p.rnp + (size_t)bh * p.items * SZ;

  // the levels above 2 whose right blocks hold this group
  int nh = 0;
  for (int j = 3; j < p.nl; ++j) nh += (g >> (j - 3)) & 1;
  const int npass = nh > kRgHigh ? cdiv(nh, kRgHigh) : 1;

  for (int pass = 0; pass < npass; ++pass) {
    // this pass's levels per slot (-1: unused): low slots in the first pass only
    int lev[NS];
#pragma unroll
    for (int u = 0; u < 3; ++u) lev[u] = (pass == 0 && u < p.nl) ? u : -1;
#pragma unroll
    for (int u = 3; u < NS; ++u) {   // the (pass * kRgHigh + u - 3)-th such level, if any
      const int want = pass * kRgHigh + u - 3;
      int k = 0, found = -1;
      for (int j = 3; j < p.nl; ++j)
        if ((g >> (j - 3)) & 1) {
          if (k == want) found = j;
          ++k;
        }
      lev[u] = found;
    }
    f32x4 acc[NS][TPW];
#pragma unroll
    for (int u = 0; u < NS; ++u)
#pragma unroll
      for (int i = 0; i < TPW; ++i) acc[u][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // the next chunk's q and do rows, log_a and the slots' lambda values, in registers (every
    // load unconditional, from clamped valid indices)
    u32x4 rq[NQ], ro[NO];
    float rla = 0.f, rlm[NS];
    auto fetch = [&](int c) {
      const int nv = min(C, p.T - c * C);
      const size_t row0 = (size_t)bh * p.T + (size_t)c * C;
      const u32x4* gq = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.q) + row0 * DK);
      const u32x4* go = reinterpret_cast<const u32x4*>(reinterpret_cast<const T*>(p.dout) + row0 * DV);
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int idx = min(tid + u * NT, PQ - 1);
        rq[u] = gq[min(idx / (DK / EPV), nv - 1) * (DK / EPV) + idx % (DK / EPV)];
      }
#pragma unroll
      for (int u = 0; u < NO; ++u) {
        const int idx = min(tid + u * NT, PO - 1);
        ro[u] = go[min(idx / (DV / EPV), nv - 1) * (DV / EPV) + idx % (DV / EPV)];
      }
      const size_t r = row0 + min(lane, nv - 1);
      rla = p.log_a[r];
#pragma unroll
      for (int u = 0; u < NS; ++u) rlm[u] = lambda_at(p, r * p.L + min(J + 1 + max(lev[u], 0), p.L - 1));
    };
    fetch(c0);
    float eoff = 0.f;     // log decay from the group's start to the current chunk's start
    float base[3] = {0.f, 0.f, 0.f};
    for (int c = c0; c < c1; ++c) {
      const int nv = min(C, p.T - c * C);
      if (c > c0) __syncthreads();   // the previous chunk's images and weights are no longer read
#pragma unroll
      for (int u = 0; u < NQ; ++u) {
        const int idx = tid + u * NT;
        if (idx < PQ) {
          const int r = idx / (DK / EPV), f = (idx % (DK / EPV)) * EPV;
          *reinterpret_cast<u32x4*>(ch.q + r * CH::RK + f) = r < nv ? rq[u] : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < NO; ++u) {
        const int idx = tid + u * NT;
        if (idx < PO) {
          const int r = idx / (DV / EPV), f = (idx % (DV / EPV)) * EPV;
          *reinterpret_cast<u32x4*>(ch.o + r * CH::RV + f) = r < nv ? ro[u] : u32x4{0u, 0u, 0u, 0u};
        }
      }
      // every wave scans the chunk's log_a (C <= 64 positions, one per lane); wave 0 writes the
      // weights of the active slots
      const float incl = wave_scan<false>(lane < nv ? rla : 0.f);
      bool act[NS];
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        act[u] = lev[u] >= 0 && ((c >> u) & 1);
        if (act[u] && !(c & ((1 << u) - 1))) base[u] = eoff;   // first chunk of its right block
      }
#pragma unroll
      for (int u = 3; u < NS; ++u) act[u] = lev[u] >= 0;
      if (w == 0 && lane < C) {
#pragma unroll
        for (int u = 0; u < NS; ++u)
          if (act[u]) scw[u * C + lane] = lane < nv ? rlm[u] * __expf(eoff - (u < 3 ? base[u] : 0.f) + incl) : 0.f;
      }
      eoff += lane_f(incl, C - 1);
      __syncthreads();
      if (c + 1 < c1) fetch(c + 1);
      // the wave's tiles: do columns (the scaled operand) scaled and split once per slot and
      // contraction step, then used against every q column block the wave holds
#pragma unroll
      for (int s0 = 0; s0 < C; s0 += 32) {
        const int k = s0 + 8 * g4;
        Frag<T> a[TM::APW];
#pragma unroll
        for (int b = 0; b < TM::APW; ++b) {
          const int ab = TM::ab(w, b);
          a[b] = ab < DK / 16 ? frag_col<T, C>(ch.q, CH::RK, k, ab * 16 + jj) : zero_frag<T>();
        }
#pragma unroll
        for (int ya = 0; ya < TM::YPW; ++ya) {
          const Frag<T> uo = frag_col<T, C>(ch.o, CH::RV, k, TM::y(w, ya) * 16 + jj);
          f32x4 ulo, uhi;
          frag_to_f32(uo, ulo, uhi);
#pragma unroll
          for (int u = 0; u < NS; ++u) {
            if (!act[u]) continue;
            // past C (chunk 16) the operands are zero; the weights are read in range
            const float* sc = scw + u * C + (k < C ? k : 0);
            Frag<T> bh_, bl_;
            scale_split<T>(ulo, uhi, sc, bh_, bl_);
#pragma unroll
            for (int b = 0; b < TM::APW; ++b) {
              mma(acc[u][ya * TM::APW + b], a[b], bh_);
              if constexpr (sizeof(T) == 2) mma(acc[u][ya * TM::APW + b], a[b], bl_);
            }
          }
        }
      }
      // store (and restart) each low slot whose right block ends with this chunk
#pragma unroll
      for (int u = 0; u < 3; ++u) {
        if (!act[u] || (c + 1 < c1 && ((c + 1) >> u) & 1)) continue;
        TM::template store<DV>(rnp + (size_t)(p.rn_off[u] + item_of_sub(u, c >> u)) * SZ, acc[u], w, lane);
#pragma unroll
        for (int i = 0; i < TPW; ++i) acc[u][i] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
    // the group's states of the levels above 2
#pragma unroll
    for (int u = 3; u < NS; ++u) {
      if (lev[u] < 0) continue;
      TM::template store<DV>(rnp + (size_t)(p.rn_off[lev[u]] + item_of_sub(lev[u], g)) * SZ, acc[u], w, lane);
    }
    if (pass + 1 < npass) __syncthreads();   // the images are rewritten by the next pass
  }
}

// ----------------------------------------------------------------------------------------
// bwd_grads: all gradients of one chunk
// ----------------------------------------------------------------------------------------

// one or two [DK][DV] states stored in the element type T into shared images (row stride RV), in
// 16-byte pieces; every load is issued before any shared-memory write
template <typename T, int DK, int DV, int RV, int NT, bool TWO = false>
__device__ __forceinline__ void stage_state(T* img, const T* __restrict__ g, int tid, T* img2 = nullptr,
                                            const T* __restrict__ g2 = nullptr) {
  constexpr int EPV = 16 / (int)sizeof(T), NP = DK * DV / EPV, PER = (NP + NT - 1) / NT;
  u32x4 r[PER], r2[TWO ? PER : 1];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = tid + u * NT;
    if (idx < NP) r[u] = reinterpret_cast<const u32x4*>(g)[idx];
    if (TWO && idx < NP) r2[u] = reinterpret_cast<const u32x4*>(g2)[idx];
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int idx = tid + u * NT;
    const int a = (idx * EPV) / DV, b = (idx * EPV) % DV;
    if (idx < NP) *reinterpret_cast<u32x4*>(img + a * RV + b) = r[u];
    if (TWO && idx < NP) *reinterpret_cast<u32x4*>(img2 + a * RV + b) = r2[u];
  }
}

// dq tiles (row block of the C positions, column block of DK) dealt to the NW = C / 16 waves by
// column, so that a wave reads only the node rows of its own columns: WIDE (DK / 16 >= NW) gives
// wave w the column blocks w, w + NW, ... and every row block; otherwise wave w has column block
// w % NK and the row blocks congruent to w / NK modulo NW / NK. Tile index a * RBW + b.
template <int C, int DK>
struct DqTiles {
  static constexpr int NW = Waves<C>::NW, NK = DK / 16;
  static_assert(C / 16 == NW, "one 16-row block per wave");
  static constexpr bool WIDE = NK >= NW;
  static constexpr int TA = WIDE ? NK / NW : 1;     // column blocks per wave
  static constexpr int RBW = WIDE ? NW : NK;        // row blocks per wave
  __device__ static constexpr int t(int w, int a) { return WIDE ? w + NW * a : w % NK; }
  __device__ static constexpr int rb(int w, int b) { return WIDE ? b : w / NK + (NW / NK) * b; }
  __device__ static constexpr bool holds(int w, int R) { return WIDE || (R % (NW / NK)) == w / NK; }
};

// X[r][k .. k+7] of a row-major state in global memory (row stride RS elements, element type),
// as an MFMA operand; the load is unconditional (from a clamped column when k >= K) and ok
// tells the caller whether to use it or zeros
template <typename T, int K>
__device__ __forceinline__ Frag<T> frag_gload(const T* g, int RS, int r, int k, bool& ok) {
  ok = K % 32 == 0 || k < K;   // steps of 32 over a multiple of 32 never pass K
  const T* p = g + (size_t)r * RS + (ok ? k : K - 8);
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
  } else {
    f.lo = *reinterpret_cast<const f32x4*>(p);
    f.hi = *reinterpret_cast<const f32x4*>(p + 4);
  }
  return f;
}

// two waves per SIMD (at most 256 registers per lane, accumulation registers included) where two
// workgroups' shared memory fits a compute unit (states up to 64 x 64); fewer would leave half
// of it idle
template <int DK, int DV>
constexpr int grads_waves_per_eu() { return DK * DV <= 64 * 64 ? 2 : 1; }

// whether the gradient kernel stages nodes through shared memory (each thread's share of a node
// in 1..4 16-byte pieces), rather than reading them by columns of dq
template <typename T, int C, int DK, int DV>
constexpr bool grads_staged() {
  constexpr int NPF = DK * DV / (16 / (int)sizeof(T)) / (64 * Waves<C>::NW);
  return NPF >= 1 && NPF <= 4 && NPF * (64 * Waves<C>::NW) * (16 / (int)sizeof(T)) == DK * DV;
}

// LATER: the head has more than one chunk (p.nl > 0), so there are later chunks and Fenwick
// nodes; the body is compiled once for each case so that none of its loads sits under a branch
template <typename T, int C, int DK, int DV, bool LATER, bool DM>
__device__ __forceinline__ void grads_body(const BwdParams& p, unsigned char* sm) {
  constexpr int NW = Waves<C>::NW, RB = Waves<C>::RB, NT = 64 * NW, J = ilog2(C);
  constexpr int ES = (int)sizeof(T), RC = C + 16 / ES;
  constexpr int NK = DK / 16, NV = DV / 16;
  using CH = Chunk<T, C, DK, DV>;
  // workgroups go to the 8 XCDs in turn: with B*H a multiple of 8, XCD x gets heads x, x + 8, ...
  // chunk after chunk, so the Fenwick nodes that consecutive chunks share stay in its L2
  const int L = blockIdx.x;
  const int q8 = L >> 3;
  const bool xcd = (p.BH & 7) == 0;
  const int c = xcd ? q8 % p.N : L % p.N;
  const int bh = xcd ? ((q8 / p.N) << 3) + (L & 7) : L / p.N;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, jj = lane & 15, g4 = lane >> 4;
  const int nv = min(C, p.T - c * C);
  const BwdSmem Lo = bwd_smem(ES, C, DK, DV, true);
  CH ch;
  ch.bind(sm, Lo);
  T* P1 = reinterpret_cast<T*>(sm + Lo.p1);     // M * W  [i][j]
  T* P2 = reinterpret_cast<T*>(sm + Lo.p2);     // M * S  [i][j]
  T* Ust = reinterpret_cast<T*>(sm + Lo.ust);   // combined right-sibling state [a][b]
  const size_t SZ = (size_t)DK * DV;
  const size_t row0 = (size_t)bh * p.T + (size_t)c * C;
  // the combined right-sibling state, written by the down-sweep (zero for the last chunk);
  // its loads are issued with the chunk's
  constexpr bool later = LATER;
  // bf16: the cross-chunk states are read as hi + lo (two bf16 MFMAs per read-out), so that
  // their rounding, shared by every position that reads a state, stays far below the inputs'
  constexpr bool SPLIT = ES == 2;
  T* Plo = P2;                                   // low part of the state image (after step 2)
  const T* node_e = reinterpret_cast<const T*>(p.node_e) + (size_t)bh * p.nslot * SZ;
  const T* node_lo = reinterpret_cast<const T*>(p.node_lo) + (size_t)bh * p.nslot * SZ;
  const T* u_lo = reinterpret_cast<const T*>(p.u_lo) + ((size_t)bh * p.N + c) * SZ;
  const T* u_e = reinterpret_cast<const T*>(p.u_e) + ((size_t)bh * p.N + c) * SZ;
  // the chunk's loads are issued first, then the combined right-sibling state's and the first
  // node of step 4 (prefetched into registers), and only then is anything written to shared
  // memory: one memory round trip for all of it
  typename CH::template Staged<NT> st;
  st.fetch(p, bh, c, nv, tid);
  constexpr int EPV = 16 / ES;
  constexpr int NPF = DK * DV / EPV / NT;
  constexpr bool PF = grads_staged<T, C, DK, DV>();
  static_assert(PF == (NPF >= 1 && NPF <= 4 && NPF * NT * EPV == DK * DV), "staged path");
  // step 4 by columns of dq when a node is too large for the staging's register prefetch
  constexpr bool COLQ = !PF;
  // jl past the last set bit (nothing left to read) loads a valid slot that is never used: the
  // node just read (cur, still in L2), or for chunk 0 slot 0.
  // rows of dq: the whole node, every thread its share, on its way into shared memory
  u32x4 pf[PF ? NPF : 1], pf2[PF && SPLIT ? NPF : 1];
  auto prefetch = [&](int sl) {
    const size_t off = (size_t)sl * SZ;
    const u32x4* src = reinterpret_cast<const u32x4*>(node_e + off);
    const u32x4* src2 = reinterpret_cast<const u32x4*>(node_lo + off);
#pragma unroll
    for (int u = 0; u < (PF ? NPF : 1); ++u) pf[u] = src[tid + u * NT];
    if constexpr (SPLIT)
#pragma unroll
      for (int u = 0; u < (PF ? NPF : 1); ++u) pf2[u] = src2[tid + u * NT];
  };
  // columns of dq: the node rows this wave's dq columns need (hi and lo parts), straight into
  // operand registers
  using QT = DqTiles<C, DK>;
  constexpr int NKS = DV >= 32 ? DV / 32 : 1;           // contraction steps over dv
  constexpr int NBF = QT::TA * NKS;                      // operand fragments per node
  auto load_node = [&](int sl, Frag<T>* hi, Frag<T>* lo, bool* ok) {
    const size_t off = (size_t)sl * SZ;
#pragma unroll
    for (int a = 0; a < QT::TA; ++a)
#pragma unroll
      for (int kb = 0; kb < NKS; ++kb) {
        const int r = QT::t(w, a) * 16 + jj, kk = kb * 32 + 8 * g4;
        hi[a * NKS + kb] = frag_gload<T, DV>(node_e + off, DV, r, kk, ok[a * NKS + kb]);
        if constexpr (SPLIT) lo[a * NKS + kb] = frag_gload<T, DV>(node_lo + off, DV, r, kk, ok[a * NKS + kb]);
      }
  };
  Frag<T> bhi[NBF], blo[NBF];
  bool bok[NBF];
  auto put = [&](T* img, const u32x4* r) {
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      const int idx = tid + u * NT;
      const int a = (idx * EPV) / DV, b = (idx * EPV) % DV;
      *reinterpret_cast<u32x4*>(img + a * CH::RV + b) = r[u];
    }
  };
  u32x4 uhi[PF ? NPF : 1], ulo[PF && SPLIT ? NPF : 1];
  if (PF && later && !DM)
#pragma unroll
    for (int u = 0; u < NPF; ++u) uhi[u] = reinterpret_cast<const u32x4*>(u_e)[tid + u * NT];
  if (PF && SPLIT && later && !DM)
#pragma unroll
    for (int u = 0; u < NPF; ++u) ulo[u] = reinterpret_cast<const u32x4*>(u_lo)[tid + u * NT];
  // DM: U_c is formed here, in fp32, as the tree's down-sweep would: from what the chunk's group
  // of 8 receives from the levels above 2 (ud) and, for each clear bit j < 3 of c, the right
  // sibling block at level j inside the group (a target-side state of bwd_rng), decayed:
  // U = D, then for j = 2, 1, 0 where that sibling exists, U = exp(G(sibling)) U + RN(sibling).
  // Each thread forms the elements of its own 16-byte pieces: on the staged path with every
  // load issued beside the prologue's others, on the column path in batches (form_u_img).
  constexpr int NF4 = DM && PF ? NPF * EPV / 4 : 1;   // float4s of a state per thread
  f32x4 udv[NF4], urn[3][NF4];
  bool uin[3] = {false, false, false};
  float ugs[3] = {0.f, 0.f, 0.f};
  const float* dsrc = p.ud;
  const float* rsrc[3] = {p.rnp, p.rnp, p.rnp};
  if constexpr (DM && LATER) {
    dsrc = p.ud + ((size_t)bh * ((p.N + 7) >> 3) + (c >> 3)) * SZ;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const int m = c >> j;
      uin[j] = j < p.nl && !(m & 1) && m + 1 < ((p.N + (1 << j) - 1) >> j);
      const int it = uin[j] ? p.rn_off[j] + item_of_sub(j, m + 1) : 0;
      rsrc[j] = p.rnp + ((size_t)bh * p.items + it) * SZ;
      ugs[j] = p.gsum[(size_t)bh * p.nslot + (uin[j] ? slot_p(p, j, m + 1) : 0)];
    }
  }
  // the column path (states too large to hold in registers at once): U_c's high or low parts
  // formed in batches of UB 16-byte pieces per thread straight into a shared-memory image,
  // each batch's loads issued together
  auto form_u_img = [&](T* img, bool lo) {
    constexpr int NP = DK * DV / EPV, PER = (NP + NT - 1) / NT, UB = 2, Q = EPV / 4;
    float ue[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) ue[j] = __expf(ugs[j]);
    for (int u0 = 0; u0 < PER; u0 += UB) {
      f32x4 x[UB][Q], r[3][UB][Q];
#pragma unroll
      for (int b = 0; b < UB; ++b) {
        const int idx = min(tid + (u0 + b) * NT, NP - 1);
#pragma unroll
        for (int q = 0; q < Q; ++q) {
          const size_t at = (size_t)idx * EPV + 4 * q;
          x[b][q] = *reinterpret_cast<const f32x4*>(dsrc + at);
#pragma unroll
          for (int j = 0; j < 3; ++j)
            if (uin[j]) r[j][b][q] = *reinterpret_cast<const f32x4*>(rsrc[j] + at);
        }
      }
#pragma unroll
      for (int b = 0; b < UB; ++b) {
        const int idx = tid + (u0 + b) * NT;
        if (u0 + b >= PER || idx >= NP) continue;
        uint32_t wd[4];
#pragma unroll
        for (int e = 0; e < EPV; ++e) {
          float v = x[b][e / 4][e % 4];
#pragma unroll
          for (int j = 2; j >= 0; --j)
            if (uin[j]) v = ue[j] * v + r[j][b][e / 4][e % 4];
          if constexpr (SPLIT) {
            const T h = (T)v;
            const uint32_t bits = __builtin_bit_cast(uint16_t, lo ? (T)(v - (float)h) : h);
            if (e & 1) wd[e / 2] |= bits << 16;
            else wd[e / 2] = bits;
          } else {
            wd[e] = __builtin_bit_cast(uint32_t, v);
          }
        }
        const int a = (idx * EPV) / DV, bcol = (idx * EPV) % DV;
        *reinterpret_cast<u32x4*>(img + a * CH::RV + bcol) = u32x4{wd[0], wd[1], wd[2], wd[3]};
      }
    }
  };
  if constexpr (DM && LATER && PF) {
#pragma unroll
    for (int u = 0; u < NPF; ++u)
#pragma unroll
      for (int q = 0; q < EPV / 4; ++q) {
        const size_t at = (size_t)(tid + u * NT) * EPV + 4 * q;
        udv[u * (EPV / 4) + q] = *reinterpret_cast<const f32x4*>(dsrc + at);
        // only the blocks that exist (a uniform branch: every one of these loads is waited for
        // before the first shared-memory write anyway)
#pragma unroll
        for (int j = 0; j < 3; ++j)
          if (uin[j]) urn[j][u * (EPV / 4) + q] = *reinterpret_cast<const f32x4*>(rsrc[j] + at);
      }
  }
  // the nodes of step 4 are (j, (c >> j) - 1) for the set bits j of c (c < N <= 2^nl), lowest
  // first. Lane l < nl holds node l's slot (slot 0 where bit l is clear) and its block decay
  // (zero where clear), loaded with the rest; step 4 turns them into each node's decay to the
  // chunk's start, so that its loop reads neither the kernel arguments nor memory for them
  // (the row path only: the column path, short of registers, reads them in its loop)
  const int first_set = c ? __builtin_ctz((unsigned)c) : p.nl;
  int nslot_l = 0;
  float gsl = 0.f;
  auto node_table = [&]() {
#pragma unroll
    for (int l = 0; l < kLamCap; ++l)
      if (lane == l && l < p.nl) nslot_l = slot_p(p, l, max((c >> l) - 1, 0));
    gsl = later ? p.gsum[(size_t)bh * p.nslot + nslot_l] : 0.f;
  };
  if constexpr (!COLQ) node_table();
  // the next set bit after jl, or nl past the last
  auto next_set = [&](int jl) {
    const int rest = c >> (jl + 1);
    return rest ? jl + 1 + __builtin_ctz((unsigned)rest) : p.nl;
  };
  // node jl's slot, or (past the last node) node cur's, still in L2
  auto slot_at = [&](int jl, int cur) { return lane_i(nslot_l, jl < p.nl ? jl : cur); };
  // the first node's slot (slot 0 for chunk 0, which has none)
  const int sl0 = first_set < p.nl ? slot_p(p, first_set, (c >> first_set) - 1) : 0;
  if constexpr (COLQ) {
    if (later) load_node(sl0, bhi, blo, bok);
  } else {
    if (later) prefetch(sl0);
  }
  if constexpr (DM && LATER && PF) {
    float ue[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) ue[j] = __expf(ugs[j]);
#pragma unroll
    for (int k = 0; k < NF4; ++k) {
      f32x4 x = udv[k];
#pragma unroll
      for (int j = 2; j >= 0; --j)
        if (uin[j]) x = ue[j] * x + urn[j][k];
      udv[k] = x;
    }
    // hi = x rounded to T, lo = the rounding error rounded to T, packed as the copies would be
#pragma unroll
    for (int u = 0; u < NPF; ++u) {
      uint32_t hw[4], lw[4];
#pragma unroll
      for (int e = 0; e < EPV; ++e) {
        const float x = udv[u * (EPV / 4) + e / 4][e % 4];
        uint32_t hb, lb = 0;
        if constexpr (SPLIT) {
          const T h = (T)x;
          hb = __builtin_bit_cast(uint16_t, h);
          lb = __builtin_bit_cast(uint16_t, (T)(x - (float)h));
          if (e & 1) { hw[e / 2] |= hb << 16; lw[e / 2] |= lb << 16; }
          else { hw[e / 2] = hb; lw[e / 2] = lb; }
        } else {
          hw[e] = __builtin_bit_cast(uint32_t, x);
        }
      }
      uhi[u] = u32x4{hw[0], hw[1], hw[2], hw[3]};
      if constexpr (SPLIT) ulo[u] = u32x4{lw[0], lw[1], lw[2], lw[3]};
    }
  }
  st.put(ch, tid);
  if (later) {
    if constexpr (PF) put(Ust, uhi);
    else if constexpr (DM) form_u_img(Ust, false);
    else stage_state<T, DK, DV, CH::RV, NT>(Ust, u_e, tid);
  }
  __syncthreads();
  ch.finish();

  // 1. masked score tiles: wave w takes 16-row blocks rb = w + NW*x of query positions i.
  //    dlambda of the levels inside the chunk is summed per (row, level) in registers: in a tile
  //    off the diagonal every pair has level 4 + bit_length(rb ^ cb); on it, bit_length(i ^ j).
  static_assert(RB == 1, "one 16-row block of positions per wave");
  float* colp = reinterpret_cast<float*>(sm + Lo.cg);   // [wave][position]
  float rowg[4] = {0.f, 0.f, 0.f, 0.f};   // per-lane partial row sums of G = P1 * S (fp32)
  // dlambda of levels 5..J of row 4 g4 + (jj & 3) of the block (each lane's row of sum16x4)
  float bins[RB][J + 1];
  for (int x = 0; x < RB; ++x)
#pragma unroll
    for (int l = 0; l <= J; ++l) bins[x][l] = 0.f;
#pragma unroll
  for (int x = 0; x < RB; ++x) {
    const int rb = w + NW * x;
#pragma unroll
    for (int cb = 0; cb < C / 16; ++cb) {
      f32x4 s = {0.f, 0.f, 0.f, 0.f}, wv = {0.f, 0.f, 0.f, 0.f};
      if (cb <= rb) {
#pragma unroll
        for (int a0 = 0; a0 < DK; a0 += 32)
          mma(s, frag_row<T, DK>(ch.q, CH::RK, rb * 16 + jj, a0 + 8 * g4),
              frag_row<T, DK>(ch.k, CH::RK, cb * 16 + jj, a0 + 8 * g4));
#pragma unroll
        for (int b0 = 0; b0 < DV; b0 += 32)
          mma(wv, frag_row<T, DV>(ch.o, CH::RV, rb * 16 + jj, b0 + 8 * g4),
              frag_row<T, DV>(ch.v, CH::RV, cb * 16 + jj, b0 + 8 * g4));
      }
      float u[4], colg = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rb * 16 + 4 * g4 + r, j = cb * 16 + jj;
        float p1 = 0.f, p2 = 0.f;
        u[r] = 0.f;
        if (j <= i) {
          const float d = __expf(ch.al[i] - ch.al[j]);
          const float m = ch.lam[i * kLamCap + bit_length((unsigned)(i ^ j))] * d;
          p1 = m * wv[r];
          p2 = m * s[r];
          u[r] = d * s[r] * wv[r];
        }
        P1[i * RC + j] = (T)p1;
        P2[i * RC + j] = (T)p2;
        rowg[r] += p1 * s[r];
        colg += p1 * s[r];
      }
      // this wave's rows of column j: the four row groups of the lane's column
      colg = sum_rows(colg);
      if (g4 == 0) colp[w * C + cb * 16 + jj] = colg;
      if (cb < rb) {
        const int lv = 4 + bit_length((unsigned)(rb ^ cb));
        const float su = sum16x4(u, jj);
#pragma unroll
        for (int l = 5; l <= J; ++l)
          if (l == lv) bins[x][l] += su;
      } else if (cb == rb) {
        // levels 0..4 lie inside this diagonal tile: with u_j the row's value at lane j, the
        // partial sums P1_x = u_x + u_{x^1}, P2_x = P1_x + P1_{x^2}, P3_x = P2_x + P2_{x^4} give
        // row i (= 4 g4 + r, local) its level sums at lane i: u_i, u_{i^1}, P1_{i^2}, P2_{i^4},
        // P3_{i^8} (u is zero above the diagonal); that lane parks them in the lambda rows'
        // slots of those levels (read already, by this wave only) until step 6 stores them
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float v = u[r];
          const float p1 = v + dpp_f<0xB1>(v);
          const float p2 = p1 + dpp_f<0x4E>(p1);
          const float p3 = p2 + dpp_xor4(p2);
          const float s1 = dpp_f<0xB1>(v), s2 = dpp_f<0x4E>(p1), s3 = dpp_xor4(p2), s4 = dpp_f<0x128>(p3);
          if (jj == 4 * g4 + r) {
            float* dl = ch.lam + (rb * 16 + jj) * kLamCap;
            dl[0] = v;
            dl[1] = s1;
            dl[2] = s2;
            dl[3] = s3;
            dl[4] = s4;
          }
        }
      }
    }
    // dlambda of the levels across the diagonal tiles (5..J), parked the same way
    if (jj < 4)
#pragma unroll
      for (int l = 5; l <= J; ++l) ch.lam[(rb * 16 + 4 * g4 + jj) * kLamCap + l] = bins[x][l];
  }
  __syncthreads();

  // 2. intra-chunk products: dq = P1 K (the wave's dq tiles: the rows of block rb, or by columns
  //    as step 4 takes them), dk = P1^T Q, dv = P2^T dO (rows: positions of block rb)
  f32x4 aq[NK], ak[RB][NK], av[RB][NV];
#pragma unroll
  for (int a = 0; a < (COLQ ? QT::TA : 1); ++a)
#pragma unroll
    for (int b = 0; b < (COLQ ? QT::RBW : NK); ++b) {
      const int R = COLQ ? QT::rb(w, b) : w, t = COLQ ? QT::t(w, a) : b;
      f32x4 zq = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s0 = 0; s0 < C; s0 += 32)
        mma(zq, frag_row<T, C>(P1, RC, R * 16 + jj, s0 + 8 * g4),
            frag_col<T, C>(ch.k, CH::RK, s0 + 8 * g4, t * 16 + jj));
      aq[COLQ ? a * QT::RBW + b : b] = zq;
    }
#pragma unroll
  for (int x = 0; x < RB; ++x) {
    const int rb = w + NW * x;
#pragma unroll
    for (int t = 0; t < NK; ++t) {
      f32x4 zk = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s0 = 0; s0 < C; s0 += 32)
        mma(zk, frag_col<T, C>(P1, RC, s0 + 8 * g4, rb * 16 + jj),
            frag_col<T, C>(ch.q, CH::RK, s0 + 8 * g4, t * 16 + jj));
      ak[x][t] = zk;
    }
#pragma unroll
    for (int t = 0; t < NV; ++t) {
      f32x4 zv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s0 = 0; s0 < C; s0 += 32)
        mma(zv, frag_col<T, C>(P2, RC, s0 + 8 * g4, rb * 16 + jj),
            frag_col<T, C>(ch.o, CH::RV, s0 + 8 * g4, t * 16 + jj));
      av[x][t] = zv;
    }
  }

  // 3. later chunks, source side: dk += w_s (V U^T), dv += w_s (K U), w_s = exp(g - A_s),
  //    U the combined right-sibling state staged at the start (its low part now, in P2's place);
  //    pk collects k . (that part of dk)
  float pk[4] = {0.f, 0.f, 0.f, 0.f};
  if (SPLIT && later) {
    __syncthreads();   // P2 is no longer read
    if constexpr (PF) put(Plo, ulo);
    else if constexpr (DM) form_u_img(Plo, true);
    else stage_state<T, DK, DV, CH::RV, NT>(Plo, u_lo, tid);
    __syncthreads();
  }
  if (later) {
#pragma unroll
    for (int x = 0; x < RB; ++x) {
      const int rb = w + NW * x;
      float wsr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) wsr[r] = ch.ws[rb * 16 + 4 * g4 + r];
#pragma unroll
      for (int t = 0; t < NK; ++t) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b0 = 0; b0 < DV; b0 += 32) {
          const Frag<T> av_ = frag_row<T, DV>(ch.v, CH::RV, rb * 16 + jj, b0 + 8 * g4);
          mma(y, av_, frag_row<T, DV>(Ust, CH::RV, t * 16 + jj, b0 + 8 * g4));
          if constexpr (SPLIT) mma(y, av_, frag_row<T, DV>(Plo, CH::RV, t * 16 + jj, b0 + 8 * g4));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          ak[x][t][r] += wsr[r] * y[r];
          pk[r] += wsr[r] * y[r] * to_f(ch.k[(rb * 16 + 4 * g4 + r) * CH::RK + t * 16 + jj]);
        }
      }
#pragma unroll
      for (int t = 0; t < NV; ++t) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int a0 = 0; a0 < DK; a0 += 32) {
          const Frag<T> ak_ = frag_row<T, DK>(ch.k, CH::RK, rb * 16 + jj, a0 + 8 * g4);
          mma(y, ak_, frag_col<T, DK>(Ust, CH::RV, a0 + 8 * g4, t * 16 + jj));
          if constexpr (SPLIT) mma(y, ak_, frag_col<T, DK>(Plo, CH::RV, a0 + 8 * g4, t * 16 + jj));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) av[x][t][r] += wsr[r] * y[r];
      }
    }
  }

  // 4. earlier chunks, query side: for each set bit j of c the node (j, (c>>j) - 1), decayed
  //    over the nodes of the lower set bits; Y = dO node^T gives dq (weighted by lambda) and,
  //    as its row dot with q, dlambda of level J+1+j (parked in that level's slot of the lambda
  //    rows, which nothing reads again, and stored in step 6); q . (dq from the nodes) goes to
  //    dqd for dA. Two ways, chosen by what measured faster:
  //    - a node of at most 4 16-byte pieces per thread: staged into shared memory (the next
  //      node's pieces in flight in registers meanwhile), every wave reading it whole for the
  //      dq rows of its block;
  //    - larger nodes, which the staging could not prefetch: by columns of dq, each wave loading
  //      only the node rows of its own dq columns straight into operand registers, one node
  //      ahead, with no barrier in the loop; the waves' dlambda shares are summed afterwards.
  float* dqd = reinterpret_cast<float*>(sm + Lo.dqd);
  if constexpr (!COLQ) {
    // decay factor from the end of node l to the start of chunk c: exp of the block decays of
    // the nodes of the lower set bits (an exclusive prefix sum over the lanes)
    const float gl = (lane < p.nl && ((c >> lane) & 1)) ? gsl : 0.f;
    const float ej = __expf(wave_scan<false>(gl) - gl);
    T* Nst = Ust;   // the state image, free once step 3 is done
    const int rb = w;
    const int ro = jj & 3, io = rb * 16 + 4 * g4 + ro;   // the row whose sums this lane receives
    float eai[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) eai[r] = ch.ea[rb * 16 + 4 * g4 + r];
    const float eao = ro == 0 ? eai[0] : ro == 1 ? eai[1] : ro == 2 ? eai[2] : eai[3];
    float dq_dot = 0.f;   // row io's q . (dq from the nodes)
    // bf16: the lane's q elements of the row dots below, read once, two per register (rows
    // 4 g4 + 2h and + 2h + 1 of column t 16 + jj in qp[2t + h], low and high halves)
    constexpr bool QREG = ES == 2;
    uint32_t qp[QREG ? 2 * NK : 1];
    if constexpr (QREG)
#pragma unroll
      for (int t = 0; t < NK; ++t)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = rb * 16 + 4 * g4 + 2 * h;
          const uint32_t a = __builtin_bit_cast(uint16_t, ch.q[i * CH::RK + t * 16 + jj]);
          const uint32_t b = __builtin_bit_cast(uint16_t, ch.q[(i + 1) * CH::RK + t * 16 + jj]);
          qp[2 * t + h] = a | (b << 16);
        }
    auto qval = [&](int t, int r) {
      if constexpr (QREG) {
        const uint32_t v = qp[2 * t + (r >> 1)];
        return __builtin_bit_cast(float, (r & 1) ? (v & 0xffff0000u) : (v << 16));
      } else {
        return to_f(ch.q[(rb * 16 + 4 * g4 + r) * CH::RK + t * 16 + jj]);
      }
    };
    for (int jl = first_set; jl < p.nl;) {
      const int nx = next_set(jl);
      __syncthreads();   // the previous reads of the state image are done
      put(Nst, pf);
      if constexpr (SPLIT) put(Plo, pf2);
      prefetch(slot_at(nx, jl));
      __syncthreads();
      const float dj = lane_f(ej, jl);
      float part[4] = {0.f, 0.f, 0.f, 0.f};
      float scl[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rb * 16 + 4 * g4 + r;
        scl[r] = ch.lam[i * kLamCap + J + 1 + jl] * eai[r] * dj;
      }
#pragma unroll
      for (int t = 0; t < NK; ++t) {
        f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b0 = 0; b0 < DV; b0 += 32) {
          const Frag<T> ao_ = frag_row<T, DV>(ch.o, CH::RV, rb * 16 + jj, b0 + 8 * g4);
          mma(y, ao_, frag_row<T, DV>(Nst, CH::RV, t * 16 + jj, b0 + 8 * g4));
          if constexpr (SPLIT) mma(y, ao_, frag_row<T, DV>(Plo, CH::RV, t * 16 + jj, b0 + 8 * g4));
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          aq[t][r] += scl[r] * y[r];
          part[r] += y[r] * qval(t, r);
        }
      }
      const float tot = sum16x4(part, jj);
      const float so = ro == 0 ? scl[0] : ro == 1 ? scl[1] : ro == 2 ? scl[2] : scl[3];
      dq_dot += so * tot;
      if (jj < 4) ch.lam[io * kLamCap + J + 1 + jl] = eao * dj * tot;
      jl = nx;
    }
    if (jj < 4) dqd[io] = dq_dot;
  } else {
    __syncthreads();
    const float* gs = p.gsum + (size_t)bh * p.nslot;
    float* red = reinterpret_cast<float*>(sm + Lo.p1);   // [wave][node][position]
    {
      float dlow = 0.f;   // log decay from the end of the current node to the start of chunk c
      int kn = 0;         // nodes done
      Frag<T> nhi[NBF], nlo[NBF];
      bool nok[NBF];
      for (int jl = first_set; jl < p.nl; ++jl) {
        if (!((c >> jl) & 1)) continue;
        int nx = jl + 1;
        while (nx < p.nl && !((c >> nx) & 1)) ++nx;
        const int sl = slot_p(p, jl, (c >> jl) - 1);
        load_node(nx < p.nl ? slot_p(p, nx, (c >> nx) - 1) : sl, nhi, nlo, nok);
        const float dj = __expf(dlow);
#pragma unroll
        for (int b = 0; b < QT::RBW; ++b) {
          const int R = QT::rb(w, b);
          float scl[4], part[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = R * 16 + 4 * g4 + r;
            scl[r] = ch.lam[i * kLamCap + J + 1 + jl] * ch.ea[i] * dj;
            part[r] = 0.f;
          }
#pragma unroll
          for (int a = 0; a < QT::TA; ++a) {
            f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kb = 0; kb < NKS; ++kb) {
              const Frag<T> ao_ = frag_row<T, DV>(ch.o, CH::RV, R * 16 + jj, kb * 32 + 8 * g4);
              const int f = a * NKS + kb;
              mma(y, ao_, bok[f] ? bhi[f] : zero_frag<T>());
              if constexpr (SPLIT) mma(y, ao_, bok[f] ? blo[f] : zero_frag<T>());
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = R * 16 + 4 * g4 + r;
              aq[a * QT::RBW + b][r] += scl[r] * y[r];
              part[r] += y[r] * to_f(ch.q[i * CH::RK + QT::t(w, a) * 16 + jj]);
            }
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float sum = sum16(part[r]);
            if (jj == r) red[(w * p.nl + kn) * C + R * 16 + 4 * g4 + r] = sum;
          }
        }
#pragma unroll
        for (int f = 0; f < NBF; ++f) {
          bhi[f] = nhi[f];
          if constexpr (SPLIT) blo[f] = nlo[f];
          bok[f] = nok[f];
        }
        dlow += gs[sl];
        ++kn;
      }
    }
    // the waves' shares summed in wave order, one position per thread: dlambda of each node
    // level (parked as above) and q . (dq from the nodes) for dA
    __syncthreads();
    if (tid < C) {
      const int i = tid, R = i >> 4;
      float dl = 0.f, acc = 0.f;
      int kn = 0;
      for (int jl = first_set; jl < p.nl; jl = next_set(jl)) {
        float sum = 0.f;
        for (int u = 0; u < NW; ++u)
          if (QT::holds(u, R)) sum += red[(u * p.nl + kn) * C + i];
        const float e = ch.ea[i] * __expf(dl);
        acc += ch.lam[i * kLamCap + J + 1 + jl] * e * sum;
        ch.lam[i * kLamCap + J + 1 + jl] = e * sum;
        dl += gs[slot_p(p, jl, (c >> jl) - 1)];
        ++kn;
      }
      dqd[i] = acc;
    }
  }

  // 5. the stores: dq, dk, dv go through the q, k, v images (no longer read) so that every
  //    thread writes whole 16-byte pieces of rows; then dA_t = q.dq - k.dk = (row sum - column
  //    sum of G inside the chunk, in fp32 from the score tiles) + q . (dq from the nodes)
  //    - k . (dk from the later chunks)
  __syncthreads();
#pragma unroll
  for (int a = 0; a < (COLQ ? QT::TA : 1); ++a)
#pragma unroll
    for (int b = 0; b < (COLQ ? QT::RBW : NK); ++b) {
      const int R = COLQ ? QT::rb(w, b) : w, t = COLQ ? QT::t(w, a) : b;
#pragma unroll
      for (int r = 0; r < 4; ++r)
        ch.q[(R * 16 + 4 * g4 + r) * CH::RK + t * 16 + jj] = (T)aq[COLQ ? a * QT::RBW + b : b][r];
    }
#pragma unroll
  for (int x = 0; x < RB; ++x) {
    const int rb = w + NW * x;
#pragma unroll
    for (int t = 0; t < NK; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = rb * 16 + 4 * g4 + r, a = t * 16 + jj;
        ch.k[i * CH::RK + a] = (T)ak[x][t][r];
      }
#pragma unroll
    for (int t = 0; t < NV; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) ch.v[(rb * 16 + 4 * g4 + r) * CH::RV + t * 16 + jj] = (T)av[x][t][r];
  }
  __syncthreads();
  {
    constexpr int EPV = 16 / ES;
    for (int idx = tid; idx < C * (DK / EPV); idx += NT) {
      const int r = idx / (DK / EPV), cc = (idx % (DK / EPV)) * EPV;
      if (r < nv) {
        *reinterpret_cast<u32x4*>(reinterpret_cast<T*>(p.gq) + (row0 + r) * DK + cc) =
            *reinterpret_cast<const u32x4*>(ch.q + r * CH::RK + cc);
        *reinterpret_cast<u32x4*>(reinterpret_cast<T*>(p.gk) + (row0 + r) * DK + cc) =
            *reinterpret_cast<const u32x4*>(ch.k + r * CH::RK + cc);
      }
    }
    for (int idx = tid; idx < C * (DV / EPV); idx += NT) {
      const int r = idx / (DV / EPV), cc = (idx % (DV / EPV)) * EPV;
      if (r < nv)
        *reinterpret_cast<u32x4*>(reinterpret_cast<T*>(p.gv) + (row0 + r) * DV + cc) =
            *reinterpret_cast<const u32x4*>(ch.v + r * CH::RV + cc);
    }
  }
#pragma unroll
  for (int x = 0; x < RB; ++x) {
    const int rb = w + NW * x;
    {
      float d[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) d[r] = rowg[r] - pk[r];
      const float rs = sum16x4(d, jj);   // row 4 g4 + (jj & 3)
      const int i = rb * 16 + 4 * g4 + (jj & 3);
      float colsum = 0.f;
      for (int u = 0; u < NW; ++u) colsum += colp[u * C + i];
      if (jj < 4 && i < nv) p.dA[row0 + i] = rs + dqd[i] - colsum;
    }

    // 6. dlambda of this block's rows: levels 0..J and the levels of step 4's node read-outs
    //    from where steps 1 and 4 parked them, zero for every other level (lane jj writes levels
    //    jj, jj + 16)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = rb * 16 + 4 * g4 + r;
      if (i >= nv) continue;
      for (int l = jj; l < p.L; l += 16) {
        float val = 0.f;
        if (l <= J) {
          val = ch.lam[i * kLamCap + l];
        } else {
          const int jl = l - J - 1;
          if (jl < p.nl && ((c >> jl) & 1)) val = ch.lam[i * kLamCap + l];
        }
        p.glam[(row0 + i) * p.L + l] = val;
      }
    }
  }
}

// DM: the gradient kernel forms each chunk's combined right-sibling state itself (from the
// group's state in ud and the group's own target-side blocks)
template <typename T, int C, int DK, int DV, bool DM = false>
__global__ void __launch_bounds__(64 * Waves<C>::NW)
__attribute__((amdgpu_waves_per_eu(grads_waves_per_eu<DK, DV>())))
bwd_grads_kernel(BwdParams p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char sm[];
  if (p.nl > 0) grads_body<T, C, DK, DV, true, DM>(p, sm);
  else grads_body<T, C, DK, DV, false, false>(p, sm);
}

}  // namespace bwd
}  // namespace lla

namespace lla {
namespace bwd {

template <typename TY, int C, int DK, int DV>
BwdKernels make_bwd() {
  const void* rng = nullptr;
  const void* sg = nullptr;
  const void* gd = nullptr;
  if constexpr (rng_fits<C, DK, DV>()) {
    rng = reinterpret_cast<const void*>(&bwd_rng_kernel<TY, C, DK, DV>);
    sg = reinterpret_cast<const void*>(&bwd_statesg_kernel<TY, C, DK, DV>);
  }
  gd = reinterpret_cast<const void*>(&bwd_grads_kernel<TY, C, DK, DV, true>);
  return BwdKernels{reinterpret_cast<const void*>(&bwd_states_kernel<TY, C, DK, DV>), sg,
                    reinterpret_cast<const void*>(&bwd_rn_kernel<TY, C, DK, DV>), rng,
                    reinterpret_cast<const void*>(&bwd_grads_kernel<TY, C, DK, DV>), gd};
}

template <typename TY, int C, int DK_>
void bwd_fill_row(BwdKernels (&r)[4]) {
  r[0] = make_bwd<TY, C, DK_, 16>();
  r[1] = make_bwd<TY, C, DK_, 32>();
  r[2] = make_bwd<TY, C, DK_, 64>();
  r[3] = make_bwd<TY, C, DK_, 128>();
}

template <typename TY, int C>
const BwdKernels* bwd_table(int DK, int DV) {
  static const struct Table {
    BwdKernels t[4][4];
    Table() {
      bwd_fill_row<TY, C, 16>(t[0]);
      bwd_fill_row<TY, C, 32>(t[1]);
      bwd_fill_row<TY, C, 64>(t[2]);
      bwd_fill_row<TY, C, 128>(t[3]);
    }
  } table;
  const int di = DK == 16 ? 0 : DK == 32 ? 1 : DK == 64 ? 2 : DK == 128 ? 3 : -1;
  const int vi = DV == 16 ? 0 : DV == 32 ? 1 : DV == 64 ? 2 : DV == 128 ? 3 : -1;
  if (di < 0 || vi < 0) return nullptr;
  return &table.t[di][vi];
}

}  // namespace bwd
}  // namespace lla
