// lla_kernels.hpp — gfx950 (CDNA4) kernels of the chunkwise log-linear Mamba-2 forward pass.
//
// Operation, per (b,h) and position t:
//   o_t = sum_{s<=t} lambda[t, l(t,s)] * exp(A_t - A_s) * (q_t . k_s) * v_s,
//   l(t,s) = bit_length(t ^ s),  A_t = sum_{r<=t} log_a[r].
// ("Log-Linear Attention": level-weighted states over a Fenwick partition, study notes
// sections 2-2, 3-2, 3-3; hierarchical mask times the Mamba-2 decay mask, sections
// 3-4, 3-5; chunkwise evaluation, gist.science zh technical summary section 2.3.)
//
// Chunk structure. With chunk size C = 2^J, positions in the same chunk have level <= J
// and are handled densely (intra-chunk block). For s in an earlier chunk c' of the
// chunk c holding t, l(t,s) = J + 1 + floor(log2(c ^ c')), so the level depends on the
// chunk pair only, and the source chunks of level J+1+j are the aligned block of 2^j
// chunks that ends where the blocks of c's lower set bits begin: a node of a Fenwick
// tree over chunks. Its contribution to t is
//   lambda[t, J+1+j] * exp(A_t - A_end) * q_t^T N,   N = sum_{s in block} exp(A_end - A_s) k_s v_s^T
// with A_end the prefix decay at the block's last position.
//
// Work split. A workgroup walks a "sweep" of R = 2^m consecutive chunks of one head.
// Fenwick nodes inside the sweep are built on the fly in registers (carry merging as the
// walk advances); nodes made of whole earlier sweeps come from a Fenwick tree over sweep
// totals built by two small kernels beforehand:
//   lla_sweep_state_kernel : per sweep, H = sum_s exp(A_sweep_end - A_s) k_s v_s^T and its
//                            total log decay G (reads k, v, log_a).
//   lla_fenwick_kernel     : in-place Fenwick up-sweep over the sweep totals of a head; emits
//                            each node in bf16/f32 MFMA-operand order plus its log decay.
//   lla_query_kernel       : per sweep, chunk by chunk: dense masked block on MFMA, decayed
//                            chunk state on MFMA, level-fused read-out of the live Fenwick
//                            nodes on MFMA, output store.
//
// MFMA operand convention. All products use 16x16 output tiles. A K=32 operand fragment
// gives lane (j = lane & 15, g = lane >> 4) eight values e = 0..7 at contraction index
//   pi(g, e) = 4g + (e & 3) + 16 (e >> 2).
// With this numbering the 16x16 accumulator layout (lane (j,g) holds rows 4g..4g+3 of
// column j) of two vertically stacked tiles is exactly one operand fragment, so scores and
// states produced by one MFMA feed the next one from registers. bf16 uses one
// v_mfma_f32_16x16x32_bf16 per fragment, f32 eight v_mfma_f32_16x16x4_f32.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lla {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMaxThreads = 512;   // 8 waves: one per 16 output columns, dv <= 128

// ----------------------------------------------------------------------------------------
// fragments and MFMA
// ----------------------------------------------------------------------------------------

template <typename T> struct Frag;
template <> struct Frag<bf16> { bf16x8 v; };
template <> struct Frag<float> { f32x4 lo, hi; };

__device__ __forceinline__ void mma(f32x4& c, const Frag<bf16>& a, const Frag<bf16>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, c, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4& c, const Frag<float>& a, const Frag<float>& b) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[0], b.lo[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[1], b.lo[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[2], b.lo[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.lo[3], b.lo[3], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[0], b.hi[0], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[1], b.hi[1], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[2], b.hi[2], c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(a.hi[3], b.hi[3], c, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ Frag<T> frag_from(const f32x4& lo, const f32x4& hi);
template <> __device__ __forceinline__ Frag<bf16> frag_from<bf16>(const f32x4& lo, const f32x4& hi) {
  Frag<bf16> f;
  f.v[0] = (bf16)lo[0]; f.v[1] = (bf16)lo[1]; f.v[2] = (bf16)lo[2]; f.v[3] = (bf16)lo[3];
  f.v[4] = (bf16)hi[0]; f.v[5] = (bf16)hi[1]; f.v[6] = (bf16)hi[2]; f.v[7] = (bf16)hi[3];
  return f;
}
template <> __device__ __forceinline__ Frag<float> frag_from<float>(const f32x4& lo, const f32x4& hi) {
  Frag<float> f; f.lo = lo; f.hi = hi; return f;
}

__device__ __forceinline__ void frag_to_f32(const Frag<bf16>& f, f32x4& lo, f32x4& hi) {
  lo[0] = (float)f.v[0]; lo[1] = (float)f.v[1]; lo[2] = (float)f.v[2]; lo[3] = (float)f.v[3];
  hi[0] = (float)f.v[4]; hi[1] = (float)f.v[5]; hi[2] = (float)f.v[6]; hi[3] = (float)f.v[7];
}
__device__ __forceinline__ void frag_to_f32(const Frag<float>& f, f32x4& lo, f32x4& hi) {
  lo = f.lo; hi = f.hi;
}

// 4 consecutive elements of a fragment (one half: e0 = 0 or 4)
template <typename T> struct Quad;
template <> struct Quad<bf16> { typedef bf16x4 type; };
template <> struct Quad<float> { typedef f32x4 type; };

__device__ __forceinline__ int bit_length(unsigned x) { return 32 - __clz((int)x); }

// ----------------------------------------------------------------------------------------
// shared-memory layout of one chunk (byte offsets; host and device agree)
// ----------------------------------------------------------------------------------------

struct ChunkSmem {
  int qf, kf, pf, ktf, vtf, lam, aloc, total;
};

// slots: one slot = one fragment for all 64 lanes (64 * 8 elements)
template <typename T>
__host__ __device__ inline ChunkSmem chunk_smem(int C, int DK, int DV, int L, bool with_q,
                                                bool alias_p) {
  const int slot = 64 * 8 * (int)sizeof(T);
  const int nqb = C / 16, nks_c = (C + 31) / 32, nks_d = (DK + 31) / 32;
  const int ndkb = DK / 16, ndvb = DV / 16;
  ChunkSmem s;
  int off = 0;
  s.qf = off;  off += with_q ? nqb * nks_d * slot : 0;
  s.kf = off;  int kbytes = with_q ? nqb * nks_d * slot : 0;
  int pbytes = with_q ? nqb * nks_c * slot : 0;
  if (alias_p) { s.pf = off; off += (kbytes > pbytes ? kbytes : pbytes); }
  else { off += kbytes; s.pf = off; off += pbytes; }
  s.ktf = off; off += ndkb * nks_c * slot;
  s.vtf = off; off += ndvb * nks_c * slot;
  s.lam = off; off += with_q ? C * L * 4 : 0;
  s.aloc = off; off += C * 4 + 16;
  s.total = (off + 255) & ~255;
  return s;
}

// ----------------------------------------------------------------------------------------
// loading one chunk into operand fragments
// ----------------------------------------------------------------------------------------

// Writes 4 consecutive contraction elements (k = k0..k0+3, k0 % 4 == 0, k0 < 32) of the
// fragment row/column `rc` (0..15) of fragment slot `slot`.
template <typename T>
__device__ __forceinline__ void put_quad(T* base, int slot, int rc, int k0,
                                         const typename Quad<T>::type& q4) {
  const int hidx = k0 >> 2;
  const int g = hidx & 3, e0 = (hidx >> 2) * 4;
  T* p = base + ((size_t)slot * 64 + rc + 16 * g) * 8 + e0;
  *reinterpret_cast<typename Quad<T>::type*>(p) = q4;
}

// 16-byte global piece: 8 bf16 or 4 f32
template <typename T> struct Piece { static constexpr int n = 16 / sizeof(T); };

template <typename T>
__device__ __forceinline__ uint4 load_piece(const T* p, bool valid) {
  if (!valid) return make_uint4(0, 0, 0, 0);
  return *reinterpret_cast<const uint4*>(p);
}

template <typename T>
__device__ __forceinline__ typename Quad<T>::type quad_of(const uint4& u, int h);
template <>
__device__ __forceinline__ bf16x4 quad_of<bf16>(const uint4& u, int h) {
  uint2 w = h ? make_uint2(u.z, u.w) : make_uint2(u.x, u.y);
  return *reinterpret_cast<bf16x4*>(&w);
}
template <>
__device__ __forceinline__ f32x4 quad_of<float>(const uint4& u, int) {
  return *reinterpret_cast<const f32x4*>(&u);
}

template <typename T>
__device__ __forceinline__ T elem_of(const uint4& u, int i) {
  return reinterpret_cast<const T*>(&u)[i];
}


// Loads rows [0, valid) of a [C, df] block (row stride df, rows past `valid` read as 0) and
// writes them as
//   rowf: row-major operand fragments, slot = (row / 16) * ceil(df/32) + col / 32
//         (rows = positions, contraction = features: q and k for the scores, q for read-outs)
//   trf : transposed operand fragments, slot = (col / 16) * ceil(C/32) + row / 32
//         (rows = features, contraction = positions: k and v for states, v for P.V)
// Each thread moves 4 consecutive positions x one 16-byte feature piece, so the transposed
// fragments get 4-element (8- or 16-byte) shared-memory stores.
template <typename T, int C, bool ROW, bool TR>
__device__ __forceinline__ void load_block(const T* __restrict__ g, int df, int valid,
                                           T* rowf, T* trf, int tid, int nthreads) {
  constexpr int EPP = Piece<T>::n;
  constexpr int NKS_C = (C + 31) / 32;
  typedef typename Quad<T>::type Q4;
  const Q4 zero4 = {};
  const int ppr = df / EPP;
  const int nks_d = (df + 31) / 32;
  for (int p = tid; p < (C / 4) * ppr; p += nthreads) {
    const int tg = p / ppr, fp = p - tg * ppr;
    const int r0 = 4 * tg, f0 = fp * EPP;
    uint4 x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = load_piece<T>(g + (size_t)(r0 + i) * df + f0, r0 + i < valid);
    if (ROW) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = r0 + i;
#pragma unroll
        for (int h = 0; h < EPP / 4; ++h) {
          const int col = f0 + 4 * h;
          put_quad<T>(rowf, (r >> 4) * nks_d + (col >> 5), r & 15, col & 31, quad_of<T>(x[i], h));
          if (df < 32) put_quad<T>(rowf, (r >> 4) * nks_d, r & 15, (col & 31) + 16, zero4);
        }
      }
    }
    if (TR) {
      const int k0 = r0 & 31, ks = r0 >> 5;
#pragma unroll
      for (int i = 0; i < EPP; ++i) {
        const int f = f0 + i;
        Q4 q4;
        q4[0] = elem_of<T>(x[0], i); q4[1] = elem_of<T>(x[1], i);
        q4[2] = elem_of<T>(x[2], i); q4[3] = elem_of<T>(x[3], i);
        put_quad<T>(trf, (f >> 4) * NKS_C + ks, f & 15, k0, q4);
        if (C < 32) put_quad<T>(trf, (f >> 4) * NKS_C + ks, f & 15, k0 + 16, zero4);
      }
    }
  }
}

// Inclusive prefix sum of log_a over one chunk (run by one wave) into aloc[0..C-1];
// positions past `valid` count as 0. Fixed summation order: bitwise reproducible.
template <int C>
__device__ __forceinline__ void chunk_cumsum(const float* __restrict__ la, int valid,
                                             float* aloc, int lane) {
  constexpr int E = C > 64 ? C / 64 : 1;      // positions per lane
  float x[E];
  float run = 0.f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane * E + e;
    run += (i < C && i < valid) ? la[i] : 0.f;
    x[e] = run;
  }
  float tot = run;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(tot, d, 64);
    if (lane >= d) tot += y;
  }
  const float excl = tot - run;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int i = lane * E + e;
    if (i < C) aloc[i] = excl + x[e];
  }
}

// ----------------------------------------------------------------------------------------
// per-wave building blocks
// ----------------------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ Frag<T> lds_frag(const T* base, int slot, int lane) {
  return reinterpret_cast<const Frag<T>*>(base)[slot * 64 + lane];
}

// Decayed chunk state for the wave's 16 value columns, as 16x16 tiles F[dk block]:
//   F = sum_{s in chunk} exp(gtot - A_s) k_s v_s^T   (gtot = A at the chunk's last position)
template <typename T, int C, int DK>
__device__ __forceinline__ void chunk_state(const T* ktf, const Frag<T> (&vfr)[(C + 31) / 32],
                                            const float* aloc, float gtot, int lane,
                                            f32x4 (&F)[DK / 16]) {
  constexpr int NKS_C = (C + 31) / 32;
  constexpr int NDKB = DK / 16;
  const int g = lane >> 4;
#pragma unroll
  for (int b = 0; b < NDKB; ++b) F[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS_C; ++ks) {
    f32x4 wlo, whi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int tlo = 32 * ks + 4 * g + e, thi = tlo + 16;
      wlo[e] = tlo < C ? __expf(gtot - aloc[min(tlo, C - 1)]) : 0.f;
      whi[e] = thi < C ? __expf(gtot - aloc[min(thi, C - 1)]) : 0.f;
    }
#pragma unroll
    for (int b = 0; b < NDKB; ++b) {
      f32x4 lo, hi;
      frag_to_f32(lds_frag<T>(ktf, b * NKS_C + ks, lane), lo, hi);
      mma(F[b], frag_from<T>(lo * wlo, hi * whi), vfr[ks]);
    }
  }
}

// Read-out operand (rows = value columns, contraction = key features) of a state kept as
// 16x16 accumulator tiles: tiles 2s and 2s+1 are exactly fragment s.
template <typename T, int DK>
__device__ __forceinline__ Frag<T> node_frag(const f32x4 (&N)[DK / 16], int s) {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return frag_from<T>(N[2 * s], (2 * s + 1 < DK / 16) ? N[2 * s + 1] : z);
}

// One Fenwick node read out by every query of the chunk (level-weighted, decayed):
//   O[qb] += lambda[i, lev] * exp(aloc[i] + doff) * (N^T q_i)
// doff = log decay from the node's last position to the chunk's first position (<= 0).
template <typename T, int C, int DK>
__device__ __forceinline__ void node_readout(const Frag<T> (&A)[(DK + 31) / 32], const T* qf,
                                             const float* lam, int L, const float* aloc,
                                             int lev, float doff, int lane, f32x4 (&O)[C / 16]) {
  constexpr int NQB = C / 16;
  constexpr int NKS_D = (DK + 31) / 32;
  const int j = lane & 15;
  f32x4 Y[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) Y[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NKS_D; ++s) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) mma(Y[qb], A[s], lds_frag<T>(qf, qb * NKS_D + s, lane));
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qi = 16 * qb + j;
    const float sc = lam[qi * L + lev] * __expf(aloc[qi] + doff);
    O[qb] += sc * Y[qb];
  }
}

// Masked score unit (query block qb, key step ks): the two 16x16 score tiles of keys
// 32ks..32ks+31 against queries 16qb..16qb+15, masked by
//   lambda[i, bit_length(i ^ s)] * exp(A_i - A_s) for s <= i (chunk-local i, s), else 0,
// returned as the P^T operand fragment of the value product.
template <typename T, int C, int DK>
__device__ __forceinline__ Frag<T> score_unit(const T* qf, const T* kf, const float* lam, int L,
                                              const float* aloc, int qb, int ks, int lane) {
  constexpr int NKS_D = (DK + 31) / 32;
  const int j = lane & 15, g = lane >> 4;
  const int kb0 = 2 * ks, kb1 = 2 * ks + 1;
  const bool has1 = kb1 <= qb;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NKS_D; ++s) {
    const Frag<T> bq = lds_frag<T>(qf, qb * NKS_D + s, lane);
    mma(s0, lds_frag<T>(kf, kb0 * NKS_D + s, lane), bq);
    if (has1) mma(s1, lds_frag<T>(kf, kb1 * NKS_D + s, lane), bq);
  }
  const int qi = 16 * qb + j;
  const float aq = aloc[qi];
  const float* lrow = lam + qi * L;
  f32x4 p0, p1;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int key0 = 16 * kb0 + 4 * g + r, key1 = key0 + 16;
    const int l0 = min(bit_length((unsigned)(qi ^ key0)), L - 1);
    const int l1 = min(bit_length((unsigned)(qi ^ key1)), L - 1);
    p0[r] = key0 <= qi ? s0[r] * lrow[l0] * __expf(aq - aloc[key0]) : 0.f;
    p1[r] = (has1 && key1 <= qi) ? s1[r] * lrow[l1] * __expf(aq - aloc[min(key1, C - 1)]) : 0.f;
  }
  return frag_from<T>(p0, p1);
}

template <typename T> __device__ __forceinline__ void store_quad(T* p, const f32x4& v);
template <> __device__ __forceinline__ void store_quad<bf16>(bf16* p, const f32x4& v) {
  bf16x4 b;
  b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = b;
}
template <> __device__ __forceinline__ void store_quad<float>(float* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }
constexpr int num_units(int nqb) { return nqb <= 0 ? 0 : num_units(nqb - 1) + (nqb - 1) / 2 + 1; }
// local Fenwick levels kept in registers per sweep: sweeps of up to 8 chunks (4 for dk=128)
template <int DK> struct SweepCap { static constexpr int LMAX = DK >= 128 ? 2 : 3; };

// ----------------------------------------------------------------------------------------
// kernels
// ----------------------------------------------------------------------------------------

struct Params {
  const void* q; const void* k; const void* v;
  const float* log_a; const float* lam;
  void* out;
  int BH, T, DV, L;
  int nchunks;      // ceil(T / C)
  int sweep;        // R: consecutive chunks per workgroup (power of two)
  int m;            // log2(R)
  int nsweep;       // ceil(nchunks / R)
  float* hbuf;      // [BH][nsweep-1][DV/16][DK/16][64] f32x4: sweep totals -> Fenwick nodes
  float* gbuf;      // [BH][nsweep-1]: sweep log decays -> Fenwick node log decays
  void* nodes;      // [BH][nsweep-1][DV/16][ceil(DK/32)][64] Frag<T>: nodes as read-out operands
  int xcd_per;      // query grid: workgroups per XCD slice
};

// Sweep totals. Grid (nsweep-1, BH): only whole sweeps before the last one are needed.
//   H = sum_{s in sweep} exp(A_end - A_s) k_s v_s^T,  G = A_end - A_{start-1}
template <typename T, int C, int DK>
__global__ __launch_bounds__(kMaxThreads) void lla_sweep_state_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int NDKB = DK / 16, NKS_C = (C + 31) / 32;
  const int tid = threadIdx.x, nthreads = blockDim.x;
  const int lane = tid & 63, w = tid >> 6;
  const int sw = blockIdx.x, bh = blockIdx.y;
  const int DV = p.DV, ns = p.nsweep - 1;
  const ChunkSmem S = chunk_smem<T>(C, DK, DV, p.L, false, false);
  T* ktf = reinterpret_cast<T*>(smem + S.ktf);
  T* vtf = reinterpret_cast<T*>(smem + S.vtf);
  float* aloc = reinterpret_cast<float*>(smem + S.aloc);

  const size_t hoff = (size_t)bh * p.T;
  const T* kg = reinterpret_cast<const T*>(p.k) + hoff * DK;
  const T* vg = reinterpret_cast<const T*>(p.v) + hoff * DV;
  const float* lag = p.log_a + hoff;

  f32x4 H[NDKB];
#pragma unroll
  for (int b = 0; b < NDKB; ++b) H[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float G = 0.f;
  for (int u = 0; u < p.sweep; ++u) {
    const int t0 = (sw * p.sweep + u) * C;
    if (u) __syncthreads();
    load_block<T, C, false, true>(kg + (size_t)t0 * DK, DK, C, nullptr, ktf, tid, nthreads);
    load_block<T, C, false, true>(vg + (size_t)t0 * DV, DV, C, nullptr, vtf, tid, nthreads);
    if (w == 0) chunk_cumsum<C>(lag + t0, C, aloc, lane);
    __syncthreads();
    const float gtot = aloc[C - 1];
    Frag<T> vfr[NKS_C];
#pragma unroll
    for (int ks = 0; ks < NKS_C; ++ks) vfr[ks] = lds_frag<T>(vtf, w * NKS_C + ks, lane);
    f32x4 F[NDKB];
    chunk_state<T, C, DK>(ktf, vfr, aloc, gtot, lane, F);
    const float d = __expf(gtot);
#pragma unroll
    for (int b = 0; b < NDKB; ++b) H[b] = d * H[b] + F[b];
    G += gtot;
  }
  f32x4* hb = reinterpret_cast<f32x4*>(p.hbuf) + (((size_t)bh * ns + sw) * (DV / 16) + w) * NDKB * 64;
#pragma unroll
  for (int b = 0; b < NDKB; ++b) hb[b * 64 + lane] = H[b];
  if (tid == 0) p.gbuf[(size_t)bh * ns + sw] = G;
}

// In-place Fenwick up-sweep over the ns = nsweep-1 sweep totals of a head: afterwards slot e
// holds the node of the lowbit(e+1) sweeps ending at e, decayed to its last position, and
// gbuf[e] its total log decay. Then every node is written as read-out fragments (Frag<T>).
// Grid (ceil(DV/16 * ceil(DK/32) * 64 / blockDim), BH); thread = (value block, dk step, lane).
template <typename T, int DK>
__global__ __launch_bounds__(256) void lla_fenwick_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  float* gsh = reinterpret_cast<float*>(smem);
  constexpr int NDKB = DK / 16, NKS_D = (DK + 31) / 32;
  const int ns = p.nsweep - 1;
  const int bh = blockIdx.y;
  const int ndvb = p.DV / 16;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = idx < ndvb * NKS_D * 64;
  const int lane = idx & 63, s = (idx >> 6) % NKS_D, w = (idx >> 6) / NKS_D;
  const int b0 = 2 * s, b1 = 2 * s + 1;
  const bool has1 = b1 < NDKB;

  float* gb = p.gbuf + (size_t)bh * ns;
  for (int i = threadIdx.x; i < ns; i += blockDim.x) gsh[i] = gb[i];
  __syncthreads();

  f32x4* hb = reinterpret_cast<f32x4*>(p.hbuf) + (size_t)bh * ns * ndvb * NDKB * 64;
  auto tile = [&](int e, int b) -> f32x4* { return hb + (((size_t)e * ndvb + w) * NDKB + b) * 64 + lane; };

  for (int half = 1; half < ns; half <<= 1) {
    if (active) {
      for (int e = 2 * half - 1; e < ns; e += 2 * half) {
        const float d = __expf(gsh[e]);     // decay across the right half (slot e as it is)
        *tile(e, b0) = d * *tile(e - half, b0) + *tile(e, b0);
        if (has1) *tile(e, b1) = d * *tile(e - half, b1) + *tile(e, b1);
      }
    }
    __syncthreads();
    for (int e = 2 * half - 1 + 2 * half * threadIdx.x; e < ns; e += 2 * half * blockDim.x)
      gsh[e] += gsh[e - half];
    __syncthreads();
  }
  if (active) {
    Frag<T>* nd = reinterpret_cast<Frag<T>*>(p.nodes);
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    for (int e = 0; e < ns; ++e) {
      const f32x4 lo = *tile(e, b0);
      const f32x4 hi = has1 ? *tile(e, b1) : z;
      nd[((((size_t)bh * ns + e) * ndvb + w) * NKS_D + s) * 64 + lane] = frag_from<T>(lo, hi);
    }
  }
  if (blockIdx.x == 0)
    for (int i = threadIdx.x; i < ns; i += blockDim.x) gb[i] = gsh[i];
}

// The output kernel: one workgroup walks the R chunks of one sweep of one head.
// Workgroup ids are dealt round-robin to the 8 XCDs; consecutive sweeps of a head are mapped
// to the same XCD so that the Fenwick nodes they share stay in one L2.
// ALIAS: the masked scores reuse the key fragments' shared memory (needed when C=128 and
// the head dims are 128); each wave then holds its score units in registers across a barrier.
template <typename T, int C, int DK, bool ALIAS>
__global__ __launch_bounds__(kMaxThreads) void lla_query_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int NQB = C / 16, NKS_C = (C + 31) / 32, NKS_D = (DK + 31) / 32, NDKB = DK / 16;
  constexpr int J = ilog2(C);
  constexpr int LMAX = SweepCap<DK>::LMAX;
  constexpr int NUNITS = num_units(NQB);
  constexpr int UHOLD = ALIAS ? 4 : 1;

  const int total = p.nsweep * p.BH;
  const int lin = (blockIdx.x & 7) * p.xcd_per + (blockIdx.x >> 3);
  if (lin >= total) return;
  const int bh = lin / p.nsweep, sw = lin - bh * p.nsweep;

  const int tid = threadIdx.x, nthreads = blockDim.x;
  const int lane = tid & 63, w = tid >> 6, nw = nthreads >> 6;
  const int j = lane & 15, g = lane >> 4;
  const int DV = p.DV, L = p.L, ns = p.nsweep - 1;
  const ChunkSmem S = chunk_smem<T>(C, DK, DV, L, true, ALIAS);
  T* qf = reinterpret_cast<T*>(smem + S.qf);
  T* kf = reinterpret_cast<T*>(smem + S.kf);
  T* pf = reinterpret_cast<T*>(smem + S.pf);
  T* ktf = reinterpret_cast<T*>(smem + S.ktf);
  T* vtf = reinterpret_cast<T*>(smem + S.vtf);
  float* lam = reinterpret_cast<float*>(smem + S.lam);
  float* aloc = reinterpret_cast<float*>(smem + S.aloc);

  const size_t hoff = (size_t)bh * p.T;
  const T* qg = reinterpret_cast<const T*>(p.q) + hoff * DK;
  const T* kg = reinterpret_cast<const T*>(p.k) + hoff * DK;
  const T* vg = reinterpret_cast<const T*>(p.v) + hoff * DV;
  const float* lag = p.log_a + hoff;
  const float* lamg = p.lam + hoff * L;
  T* og = reinterpret_cast<T*>(p.out) + hoff * DV;

  const int c0 = sw * p.sweep;
  const int nch = min(p.sweep, p.nchunks - c0);

  f32x4 LN[LMAX][NDKB];   // local Fenwick nodes (this wave's value columns)
  float LD[LMAX];         // log decay from each node's last position to the current chunk start
#pragma unroll
  for (int a = 0; a < LMAX; ++a) {
    LD[a] = 0.f;
#pragma unroll
    for (int b = 0; b < NDKB; ++b) LN[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  float gam = 0.f;        // log decay from the sweep's first position to the current chunk start

  for (int u = 0; u < nch; ++u) {
    const int t0 = (c0 + u) * C;
    const int valid = min(C, p.T - t0);
    if (u) __syncthreads();
    load_block<T, C, true, false>(qg + (size_t)t0 * DK, DK, valid, qf, nullptr, tid, nthreads);
    load_block<T, C, true, true>(kg + (size_t)t0 * DK, DK, valid, kf, ktf, tid, nthreads);
    load_block<T, C, false, true>(vg + (size_t)t0 * DV, DV, valid, nullptr, vtf, tid, nthreads);
    for (int i = tid; i < C * L; i += nthreads)
      lam[i] = i < valid * L ? lamg[(size_t)t0 * L + i] : 0.f;
    if (w == 0) chunk_cumsum<C>(lag + t0, valid, aloc, lane);
    __syncthreads();
    const float gtot = aloc[C - 1];

    // masked scores -> P^T fragments
    if (!ALIAS) {
      for (int un = w; un < NUNITS; un += nw) {
        int qb = 0, ks = un;
        while (ks >= qb / 2 + 1) { ks -= qb / 2 + 1; ++qb; }
        const Frag<T> f = score_unit<T, C, DK>(qf, kf, lam, L, aloc, qb, ks, lane);
        reinterpret_cast<Frag<T>*>(pf)[(qb * NKS_C + ks) * 64 + lane] = f;
      }
    } else {
      Frag<T> held[UHOLD];
      int where[UHOLD];
#pragma unroll
      for (int h = 0; h < UHOLD; ++h) {
        const int un = w + h * nw;
        where[h] = -1;
        if (un < NUNITS) {
          int qb = 0, ks = un;
          while (ks >= qb / 2 + 1) { ks -= qb / 2 + 1; ++qb; }
          held[h] = score_unit<T, C, DK>(qf, kf, lam, L, aloc, qb, ks, lane);
          where[h] = qb * NKS_C + ks;
        }
      }
      __syncthreads();
#pragma unroll
      for (int h = 0; h < UHOLD; ++h)
        if (where[h] >= 0) reinterpret_cast<Frag<T>*>(pf)[where[h] * 64 + lane] = held[h];
    }
    __syncthreads();

    // intra-chunk values
    Frag<T> vfr[NKS_C];
#pragma unroll
    for (int ks = 0; ks < NKS_C; ++ks) vfr[ks] = lds_frag<T>(vtf, w * NKS_C + ks, lane);
    f32x4 O[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      O[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks <= qb / 2; ++ks) mma(O[qb], vfr[ks], lds_frag<T>(pf, qb * NKS_C + ks, lane));
    }

    // Fenwick nodes inside the sweep (levels J+1 .. J+m)
#pragma unroll
    for (int a = 0; a < LMAX; ++a) {
      if ((u >> a) & 1) {
        Frag<T> A[NKS_D];
#pragma unroll
        for (int s = 0; s < NKS_D; ++s) A[s] = node_frag<T, DK>(LN[a], s);
        node_readout<T, C, DK>(A, qf, lam, L, aloc, J + 1 + a, LD[a], lane, O);
      }
    }
    // Fenwick nodes made of whole earlier sweeps (levels J+m+1 ..)
    if (sw > 0) {
      const Frag<T>* nd = reinterpret_cast<const Frag<T>*>(p.nodes);
      float dext = 0.f;
      for (int jb = 0; (sw >> jb) != 0; ++jb) {
        if (!((sw >> jb) & 1)) continue;
        const int e = ((sw >> jb) << jb) - 1;
        Frag<T> A[NKS_D];
#pragma unroll
        for (int s = 0; s < NKS_D; ++s)
          A[s] = nd[((((size_t)bh * ns + e) * (DV / 16) + w) * NKS_D + s) * 64 + lane];
        node_readout<T, C, DK>(A, qf, lam, L, aloc, J + 1 + p.m + jb, gam + dext, lane, O);
        dext += p.gbuf[(size_t)bh * ns + e];
      }
    }
    // store rows [0, valid)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qi = 16 * qb + j;
      if (qi < valid) store_quad<T>(og + (size_t)(t0 + qi) * DV + 16 * w + 4 * g, O[qb]);
    }

    // carry the chunk's state into the sweep's Fenwick nodes
    if (u + 1 < nch) {
      f32x4 F[NDKB];
      chunk_state<T, C, DK>(ktf, vfr, aloc, gtot, lane, F);
      const int cz = __builtin_ctz(u + 1);
#pragma unroll
      for (int a = 0; a < LMAX; ++a) {
        LD[a] += gtot;
        if (a < cz) {
          const float d = __expf(LD[a]);
#pragma unroll
          for (int b = 0; b < NDKB; ++b) F[b] += d * LN[a][b];
        }
      }
#pragma unroll
      for (int a = 0; a < LMAX; ++a) {
        if (a == cz) {
          LD[a] = 0.f;
#pragma unroll
          for (int b = 0; b < NDKB; ++b) LN[a][b] = F[b];
        }
      }
    }
    gam += gtot;
  }
}

}  // namespace lla
