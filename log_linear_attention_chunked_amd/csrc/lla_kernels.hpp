// lla_kernels.hpp — gfx950 (CDNA4) forward kernel of chunkwise log-linear Mamba-2.
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
// Work split. One kernel, one workgroup per "sweep" of R consecutive chunks of one head (R = 1
// or 2, all of them resident in shared memory at once), one wave per 16 value columns.
// Workgroups take a ticket from an atomic counter and map it sweep-major, so every sweep
// they wait for belongs to a workgroup that started earlier.
//   load:    node flags, log_a, k, v, lambda and q of the sweep go straight from HBM into
//            shared memory (global_load_lds; q, k, v as swizzled images), in that order, with
//            counted waits: wave 0 scans log_a once it lands, phase A starts once k and v
//            have, while q is still arriving.
//   phase A: chunk states k^T (w v) on MFMA (w: decay to the chunk end); the sweep total plus
//            the nodes of earlier sweeps it absorbs (a Fenwick tree over sweeps) is published
//            as this sweep's node; the state of chunk 0 is kept for chunk 1 (level J+1).
//   phase B: per chunk: masked scores on MFMA -> P^T, P.V on MFMA, read-out of the live
//            Fenwick nodes on MFMA (inside the sweep from registers, earlier sweeps from the
//            published nodes), output store.
// A node is published per wave (16 value columns) with device-scope stores, then a flag;
// readers poll the flag (bounded: on timeout the outputs are set to NaN so that a broken
// dependency can never hang the device) and then read the node (see node_st below).
//
// MFMA conventions. 16x16 output tiles; the accumulator gives lane (j = lane & 15,
// g = lane >> 4) rows 4g..4g+3 of column j. A K=32 operand fragment gives lane (j, g) the
// contraction indices 8g..8g+7 of its row/column j (bf16: one v_mfma_f32_16x16x32_bf16; f32:
// eight v_mfma_f32_16x16x4_f32). Tiles whose rows are later used as a contraction index are
// computed in pairs with permuted rows,
//   tile 2s+h, row i  <->  index 32s + 8(i/4) + 4h + (i%4),
// so that the two accumulators a lane holds are exactly its operand fragment for indices
// 32s..32s+31: masked scores become P^T and chunk states become read-out operands without
// leaving registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lla {

typedef __bf16 bf16;
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) void lds_void;

// Copies from global into shared memory (global_load_lds: each lane's 4 or 16 bytes land at
// M0 + lane * size), written as inline assembly. Through the builtin the compiler tracks them
// as shared-memory stores of unknown extent and waits for every one of them (vmcnt 0) before
// any later shared-memory read, which would hold phase A back until the q images arrive; it
// adds no waits for these. Every read of copied data in this file is preceded by an explicit
// wait_vm (copies complete in issue order) and, across waves, a barrier. The shared-memory
// address, wave-uniform, is passed in M0.
// a flat shared-memory address is the shared aperture's base plus the offset: its low 32 bits
__device__ __forceinline__ unsigned lds_off(const void* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)p);
}
__device__ __forceinline__ void copy_lds16(const void* src, const void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds_off(dst)) : "memory");
#else
  (void)src; (void)dst;
#endif
}
__device__ __forceinline__ void copy_lds4(const void* src, const void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds_off(dst)) : "memory");
#else
  (void)src; (void)dst;
#endif
}
// 2 bytes per lane, zero-extended into the lane's 4-byte slot at M0 + lane * 4 (bfloat16 lambda:
// the slot then holds the bf16 bits in its low half)
__device__ __forceinline__ void copy_lds2(const void* src, const void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_lds_ushort %0, off" ::"v"(src), "{m0}"(lds_off(dst)) : "memory");
#else
  (void)src; (void)dst;
#endif
}
// the same, device scope (sc1): node flags, coherent across XCDs like the flag polls
__device__ __forceinline__ void copy_lds4_device(const void* src, const void* dst) {
#if defined(__HIP_DEVICE_COMPILE__)
  asm volatile("global_load_lds_dword %0, off sc1" ::"v"(src), "{m0}"(lds_off(dst)) : "memory");
#else
  (void)src; (void)dst;
#endif
}

constexpr int kLamCap = 24;       // lambda levels held per position (T <= 2^23)
constexpr int kMaxSweep = 2;      // chunks resident per workgroup

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) { static_for_impl<0, N>(f); }
constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

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

template <typename T> __device__ __forceinline__ Frag<T> zero_frag() {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return frag_from<T>(z, z);
}

__device__ __forceinline__ int bit_length(unsigned x) { return 32 - __clz((int)x); }

// ----------------------------------------------------------------------------------------
// shared-memory images
// ----------------------------------------------------------------------------------------
// Every q, k, v image is row-major (row = position) in 16-byte vectors whose place in the
// row is XOR-swizzled at 16-byte granularity, so that global_load_lds can write an image
// directly (one 16-byte piece per lane). ES = element bytes, NV = vectors per row.
//   row images (q, k): conflict-free operand-fragment reads (16 rows x one vector) and, for
//                      bf16 k, conflict-free transposing reads of chunk states (4 rows x quads
//                      2c+h, c = 0..3);
//   value images (v):  bf16: conflict-free transposing reads (4 rows x 4 consecutive quads);
//                      f32: read element-wise with the row swizzle.
template <int ES, int NV>
__host__ __device__ constexpr int swz_row(int r) {
  return ES == 2 ? (NV == 2 ? (r >> 3) & 1
                  : NV == 4 ? (r >> 2) & 3
                  : NV == 8 ? ((((r >> 1) & 1) << 2) | ((r >> 2) & 3))
                            : (((r & 3) << 2) | ((r >> 2) & 3)))
                 : (NV == 4 ? (r >> 2) & 3 : NV == 8 ? (r >> 1) & 7 : r & 15);
}
template <int ES, int NV>
__host__ __device__ constexpr int swz_val(int r) {
  return ES == 2 ? (2 * (r & 3)) & (NV - 1) : swz_row<ES, NV>(r);
}

// byte offset of element f (feature) of row r in an image with NV vectors per row
template <int ES, int NV, bool VAL>
__device__ __forceinline__ int elem_off(int r, int f) {
  constexpr int EPV = 16 / ES;
  const int x = VAL ? swz_val<ES, NV>(r) : swz_row<ES, NV>(r);
  return r * NV * 16 + (((f / EPV) ^ x) << 4) + (f % EPV) * ES;
}

// Shared-memory layout of the forward kernel (host and device agree). Per resident chunk u:
// q, k, v images, lambda rows (C x L floats, row stride L), A / e^A / e^-A / state weights (the
// weights' slot first receives the chunk's log_a), a flag word and the chunk's total log decay,
// and the P^T fragments of its masked scores; then copies of each wave's node flags, and the
// workgroup ticket.
struct Smem {
  int q[kMaxSweep], k[kMaxSweep], v[kMaxSweep], lam[kMaxSweep], dec[kMaxSweep], flag[kMaxSweep],
      pf[kMaxSweep], flg, ticket, total;
};
constexpr int kFlagCopy = 8;      // node flags copied per wave (at least the register budget)
__host__ __device__ inline Smem smem_layout(int es, int C, int DK, int DV, int NB) {
  Smem s;
  int off = 0;
  const int nqb = C / 16, nks_c = cdiv(C, 32);
  for (int u = 0; u < kMaxSweep; ++u) {
    const bool on = u < NB;
    s.q[u] = off;    off += on ? C * DK * es : 0;
    s.k[u] = off;    off += on ? C * DK * es : 0;
    s.v[u] = off;    off += on ? C * DV * es : 0;
    s.lam[u] = off;  off += on ? C * kLamCap * 4 : 0;
    s.dec[u] = off;  off += on ? 4 * C * 4 : 0;
    s.flag[u] = off; off += on ? 16 : 0;
    s.pf[u] = off;   off += on ? nqb * nks_c * 64 * 8 * es : 0;
  }
  s.flg = off; off += 8 * kFlagCopy * 4;   // up to 8 waves
  s.ticket = off; off += 16;
  s.total = (off + 255) & ~255;
  return s;
}

// ----------------------------------------------------------------------------------------
// staging: HBM -> shared memory
// ----------------------------------------------------------------------------------------

// One [C, DF] block (row stride DF; rows past `valid` replaced by row valid-1) into an image
// by global_load_lds: slot p of the image (row p/NV, physical vector p%NV) receives logical
// vector (p%NV) ^ swizzle(row) of that row. Wave w issues the 1 KB blocks i*NW + w; lanes
// past the image end issue nothing.
// The per-lane part of the source offsets is computed once per kernel (the images of all
// chunks share it); a ragged chunk (valid < C) takes the clamping path.
template <typename T, int C, int DF, int NW, bool VAL>
struct DmaPlan {
  static constexpr int ES = (int)sizeof(T), NV = DF * ES / 16, SLOTS = C * NV;
  static constexpr int ITERS = cdiv(SLOTS, 64 * NW);
  int row[ITERS], col[ITERS];      // source row, element offset of the piece within the row
  __device__ __forceinline__ void init(int w, int lane) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int p = (it * NW + w) * 64 + lane;
      const int r = min(p / NV, C - 1), pv = p % NV;
      row[it] = r;
      col[it] = (pv ^ (VAL ? swz_val<ES, NV>(r) : swz_row<ES, NV>(r))) * (16 / ES);
    }
  }
  __device__ __forceinline__ void issue(unsigned char* img, const T* __restrict__ g, int valid,
                                        int w, int lane) const {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int blk = it * NW + w;
      // images made of whole 64-lane rounds issue unconditionally, so the compiler can count
      // them when it places waits for earlier loads
      if (SLOTS % (64 * NW) == 0 || blk * 64 + lane < SLOTS) {
        const int r = valid == C ? row[it] : min(row[it], valid - 1);
        const T* src = g + (size_t)(r * DF + col[it]);
        copy_lds16(src, img + blk * 1024);
      }
    }
  }
};

// lambda rows of one chunk (n_total = C*L contiguous floats, a multiple of 4, n_valid of them
// real) by global_load_lds: float i lands at lam[i]. A whole chunk with a 16-byte aligned source
// moves in 16-byte pieces; otherwise 4-byte pieces, and past the real floats the last one is
// repeated (those rows belong to positions past T, whose outputs are not stored).
__device__ __forceinline__ void dma_lambda(float* lam, const float* __restrict__ g, int n_valid,
                                           int n_total, int w, int nw, int lane) {
  if (n_valid == n_total && (reinterpret_cast<uintptr_t>(g) & 15) == 0) {
    for (int blk = w; blk * 256 < n_total; blk += nw) {
      const int i = (blk * 64 + lane) * 4;
      if (i < n_total) {
        copy_lds16(g + i, lam + blk * 256);
      }
    }
    return;
  }
  for (int blk = w; blk * 64 < n_total; blk += nw) {
    const int i = blk * 64 + lane;
    if (i < n_total) {
      const float* src = g + min(i, n_valid - 1);
      copy_lds4(src, lam + blk * 64);
    }
  }
}

// bfloat16 lambda rows of one chunk (n_total = C*L elements, n_valid of them real): element i lands
// zero-extended in the 4-byte slot lam[i] (past the real elements the last one is repeated), one
// element per lane, so no alignment is assumed; lambda_widen turns the slots into floats once
// they have landed.
__device__ __forceinline__ void dma_lambda_bf16(float* lam, const unsigned short* __restrict__ g, int n_valid,
                                                int n_total, int w, int nw, int lane) {
  for (int blk = w; blk * 64 < n_total; blk += nw) {
    const int i = blk * 64 + lane;
    if (i < n_total) copy_lds2(g + min(i, n_valid - 1), lam + blk * 64);
  }
}
// the elements wave w copied by dma_lambda_bf16 (after they landed): bf16 bits -> float
__device__ __forceinline__ void lambda_widen(float* lam, int n_total, int w, int nw, int lane) {
  unsigned* u = reinterpret_cast<unsigned*>(lam);
  for (int blk = w; blk * 64 < n_total; blk += nw) {
    const int i = blk * 64 + lane;
    if (i < n_total) u[i] = u[i] << 16;
  }
}

// global_load_lds instructions wave w issues for one [C, DF] image (DmaPlan::issue)
template <typename T, int C, int DF, int NW>
__host__ __device__ constexpr int dma_count(int w) {
  constexpr int SLOTS = C * DF * (int)sizeof(T) / 16;
  int n = 0;
  for (int it = 0; it * NW + w < cdiv(SLOTS, 64); ++it) ++n;
  return n;
}

// s_waitcnt vmcnt(min(N, 63)) alone (expcnt and lgkmcnt left at their maxima); the counter
// never exceeds 63, so the clamp only waits longer
template <int N0>
__device__ __forceinline__ void wait_vm() {
  constexpr int N = N0 > 63 ? 63 : N0;
  static_assert(N >= 0, "vmcnt");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Workgroup barrier for shared memory only: this wave's shared-memory accesses complete, then
// s_barrier. (__syncthreads would also wait for every outstanding global access, including
// copies still meant to be in flight.)
__device__ __forceinline__ void lds_barrier() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Inclusive prefix (sum or max) over the 64 lanes of a wave, by DPP: shifts by 1, 2, 4, 8
// lanes inside each row of 16, then row 0's last lane into row 1 and row 2's into row 3, then
// lane 31 into rows 2 and 3 (row_shr:n = 0x110 + n, row_bcast:15 = 0x142, row_bcast:31 =
// 0x143). Lanes a step gives no source add the identity. A fixed order: bitwise reproducible.
template <bool MAX>
__device__ __forceinline__ float wave_scan(float x) {
  const int id = __builtin_bit_cast(int, MAX ? -__builtin_inff() : 0.f);
  auto step = [&](int y) {
    const float v = __builtin_bit_cast(float, y);
    x = MAX ? fmaxf(x, v) : x + v;
  };
  const int xi0 = __builtin_bit_cast(int, x);
  step(__builtin_amdgcn_update_dpp(id, xi0, 0x111, 0xf, 0xf, false));
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, x), 0x112, 0xf, 0xf, false));
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, x), 0x114, 0xf, 0xf, false));
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, x), 0x118, 0xf, 0xf, false));
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, x), 0x142, 0xa, 0xf, false));
  step(__builtin_amdgcn_update_dpp(id, __builtin_bit_cast(int, x), 0x143, 0xc, 0xf, false));
  return x;
}

// log_a of one chunk in a wave's registers (lane l holds positions E*l .. E*l+E-1), and the
// chunk-local inclusive prefix sum A (same layout); wave 0 computes it for every chunk.
template <int C>
struct DecayRegs {
  static constexpr int E = C > 64 ? C / 64 : 1;
  float x[E];
  float a[E];

  // from the chunk's log_a copied into shared memory (positions past `valid` count as 0)
  __device__ __forceinline__ void fetch_lds(const float* la, int valid, int lane) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lane * E + e;
      x[e] = (i < C && i < valid) ? la[i] : 0.f;
    }
  }
  // fixed summation order: bitwise reproducible
  __device__ __forceinline__ void scan(int lane) {
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) { run += x[e]; a[e] = run; }
    (void)lane;
    const float tot = wave_scan<false>(run);
    const float excl = tot - run;
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] += excl;
  }
  // total log decay of the chunk (all lanes of the wave must call it together)
  __device__ __forceinline__ float total() const {
    return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a[E - 1]), 63));
  }
  // wave 0: publish A, e^A, e^-A, the state weights exp(g - A) (over the log_a copy: each lane
  // reads its own positions before writing them), whether the factorised decay e^{A_i} e^{-A_s}
  // is safe (|A| < 40), and the total g
  __device__ __forceinline__ void publish(float* dec, int* flag, float g, int lane) const {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lane * E + e;
      if (i < C) {
        dec[i] = a[e];
        dec[C + i] = __expf(a[e]);
        dec[2 * C + i] = __expf(-a[e]);
        dec[3 * C + i] = __expf(g - a[e]);
        amax = fmaxf(amax, fabsf(a[e]));
      }
    }
    amax = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wave_scan<true>(amax)), 63));
    if (lane == 0) {
      flag[0] = amax < 40.f ? 1 : 0;
      flag[1] = __builtin_bit_cast(int, g);
    }
  }
};

// ----------------------------------------------------------------------------------------
// operand fragments from shared memory
// ----------------------------------------------------------------------------------------

// Row operand: row r of a row image, contraction features 32s + 8g .. +7 (zero past DF).
template <typename T, int DF>
__device__ __forceinline__ Frag<T> row_frag(const unsigned char* img, int r, int s, int lane) {
  constexpr int ES = (int)sizeof(T), NV = DF * ES / 16;
  const int g = lane >> 4;
  Frag<T> f;
  if constexpr (ES == 2) {
    const int v = 4 * s + g;
    const bool ok = NV >= 4 || v < NV;
    const int x = swz_row<2, NV>(r);
    u32x4 d = *reinterpret_cast<const u32x4*>(img + r * NV * 16 + (((ok ? v : 0) ^ x) << 4));
    if (!ok) d = u32x4{0u, 0u, 0u, 0u};
    f.v = __builtin_bit_cast(bf16x8, d);
  } else {
    const int v0 = 8 * s + 2 * g;
    const bool ok = NV >= 8 || v0 < NV;
    const int x = swz_row<4, NV>(r);
    const int vv = ok ? v0 : 0;
    f.lo = *reinterpret_cast<const f32x4*>(img + r * NV * 16 + ((vv ^ x) << 4));
    f.hi = *reinterpret_cast<const f32x4*>(img + r * NV * 16 + (((vv + 1) ^ x) << 4));
    if (!ok) { f.lo = f32x4{0.f, 0.f, 0.f, 0.f}; f.hi = f.lo; }
  }
  return f;
}

__device__ __forceinline__ s16x4 ds_read_tr(const unsigned char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)p);
}

// Position-contracted operand: rows = 16 features, contraction = positions 32ks + 8g + e.
// Output row i holds feature 16fsel + i of a value image (VAL), or feature
// 32fsel + 8(i/4) + 4h + (i%4) of a key image (state tile (fsel, h)). bf16 by two transposing
// reads: in each 16-lane group the read returns to lane i, element c, element i%4 of the quad
// addressed by lane 4c + i/4, so lane k addresses position base + k/4 and the quad of output
// rows 4(k%4)..4(k%4)+3. f32 element-wise. Positions >= C (C = 16) and features >= DF are 0.
template <typename T, int C, int DF, bool VAL>
__device__ __forceinline__ Frag<T> col_frag(const unsigned char* img, int fsel, int h, int ks,
                                            int lane) {
  constexpr int ES = (int)sizeof(T), NV = DF * ES / 16;
  const int k = lane & 15, g = lane >> 4;
  const bool tok = C >= 32 || g < 2;
  Frag<T> f;
  if constexpr (ES == 2) {
    const int qa = VAL ? 4 * fsel + (k & 3) : 8 * fsel + 2 * (k & 3) + h;    // addressed by k
    const int qo = VAL ? 4 * fsel + (k >> 2) : 8 * fsel + 2 * (k >> 2) + h;  // of k's output rows
    const bool qaok = qa < 2 * NV, qook = qo < 2 * NV;
    const int t = tok ? 32 * ks + 8 * g + (k >> 2) : 0;
    const int q = qaok ? qa : 0;
    const int x0 = VAL ? swz_val<2, NV>(t) : swz_row<2, NV>(t);
    const int x1 = VAL ? swz_val<2, NV>(t + 4) : swz_row<2, NV>(t + 4);
    const s16x4 a = ds_read_tr(img + t * NV * 16 + (((q >> 1) ^ x0) << 4) + ((q & 1) << 3));
    const s16x4 b = ds_read_tr(img + (t + 4) * NV * 16 + (((q >> 1) ^ x1) << 4) + ((q & 1) << 3));
    f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    if (!(tok && qook)) f = zero_frag<bf16>();
  } else {
    const int feat = VAL ? 16 * fsel + k : 32 * fsel + 8 * (k >> 2) + 4 * h + (k & 3);
    const bool fok = feat < DF;
    float e[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int t = 32 * ks + 8 * g + i;
      const bool ok = tok && fok && t < C;
      const float val = *reinterpret_cast<const float*>(img + elem_off<4, NV, VAL>(ok ? t : 0, fok ? feat : 0));
      e[i] = ok ? val : 0.f;
    }
    f.lo = f32x4{e[0], e[1], e[2], e[3]};
    f.hi = f32x4{e[4], e[5], e[6], e[7]};
  }
  return f;
}

// fragment multiplied element-wise by (w0, w1)
__device__ __forceinline__ Frag<bf16> frag_scale(const Frag<bf16>& f, const f32x4& w0, const f32x4& w1) {
  f32x4 lo, hi;
  frag_to_f32(f, lo, hi);
  return frag_from<bf16>(lo * w0, hi * w1);
}
__device__ __forceinline__ Frag<float> frag_scale(const Frag<float>& f, const f32x4& w0, const f32x4& w1) {
  Frag<float> r; r.lo = f.lo * w0; r.hi = f.hi * w1; return r;
}

// Operand reads of one chunk's images. bf16: byte offsets per lane computed once for the
// whole kernel (a row's swizzle depends only on its low 4 bits, so query blocks, key steps and
// tile halves are immediate offsets; images differ only by their base). f32: the generic
// element-wise reads above.
template <typename T, int C, int DK, int DV> struct Reader;

template <int C, int DK, int DV>
struct Reader<bf16, C, DK, DV> {
  static constexpr int NVK = DK / 8, NVV = DV / 8, RBK = NVK * 16, RBV = NVV * 16;
  static constexpr int NKS_D = cdiv(DK, 32);
  int oq[NKS_D];        // q row j, features 32s + 8g ..            (+ 16qb rows)
  int ok[2][NKS_D];     // k row 8(j/4) + 4t + j%4 of score tile t  (+ 32ks rows)
  int okt[2][NKS_D];    // k^T, state tile (s, .), read r: row 8g + k/4 + 4r, quad 8s + 2(k%4) (+ 32ks rows, + h quads)
  int ovt;              // v^T, value block w: row 8g + k/4, quad 4w + k%4 (+ 32ks rows, + 4 rows for read 1)
  bool fq;              // the lane's 8-feature vector exists (dk = 16: g < 2)
  bool fkt;             // the lane's state-tile output rows exist (dk = 16: k/4 < 2)
  bool tv;              // the lane group's positions exist (C = 16: g < 2)

  __device__ __forceinline__ void init(int lane, int w) {
    const int k = lane & 15, g = lane >> 4, b = k >> 2, c = k & 3;
    fq = NVK >= 4 || g < 2;
    fkt = NVK >= 4 || b < 2;
    tv = C >= 32 || g < 2;
#pragma unroll
    for (int s = 0; s < NKS_D; ++s) {
      const int v = fq ? 4 * s + g : 0;
      oq[s] = k * RBK + ((v ^ swz_row<2, NVK>(k)) << 4);
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int r = min(8 * b + 4 * t + c, C - 1);
        ok[t][s] = r * RBK + ((v ^ swz_row<2, NVK>(r)) << 4);
      }
      const int vk = (4 * s + c < NVK) ? 4 * s + c : 0;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = tv ? 8 * g + b + 4 * r : 0;
        okt[r][s] = row * RBK + ((vk ^ swz_row<2, NVK>(row)) << 4);
      }
    }
    const int row = tv ? 8 * g + b : 0;
    ovt = row * RBV + (((2 * w + (c >> 1)) ^ swz_val<2, NVV>(row)) << 4) + 8 * (c & 1);
  }
  __device__ __forceinline__ static Frag<bf16> frag16(const unsigned char* p, bool ok) {
    u32x4 d = *reinterpret_cast<const u32x4*>(p);
    if (!ok) d = u32x4{0u, 0u, 0u, 0u};
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8, d);
    return f;
  }
  __device__ __forceinline__ static Frag<bf16> frag_tr(const unsigned char* p0, const unsigned char* p1, bool ok) {
    const s16x4 a = ds_read_tr(p0), b = ds_read_tr(p1);
    Frag<bf16> f;
    f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
    if (!ok) f = zero_frag<bf16>();
    return f;
  }
  __device__ __forceinline__ Frag<bf16> q(const unsigned char* img, int qb, int s) const {
    return frag16(img + oq[s] + 16 * qb * RBK, fq);
  }
  __device__ __forceinline__ Frag<bf16> k(const unsigned char* img, int t, int ks, int s) const {
    return frag16(img + ok[t][s] + 32 * ks * RBK, fq);
  }
  __device__ __forceinline__ Frag<bf16> kt(const unsigned char* img, int s, int h, int ks) const {
    return frag_tr(img + okt[0][s] + 32 * ks * RBK + 8 * h, img + okt[1][s] + 32 * ks * RBK + 8 * h, tv && fkt);
  }
  __device__ __forceinline__ Frag<bf16> vt(const unsigned char* img, int ks) const {
    return frag_tr(img + ovt + 32 * ks * RBV, img + ovt + (32 * ks + 4) * RBV, tv);
  }
};

template <int C, int DK, int DV>
struct Reader<float, C, DK, DV> {
  int lane, w;
  __device__ __forceinline__ void init(int lane_, int w_) { lane = lane_; w = w_; }
  __device__ __forceinline__ Frag<float> q(const unsigned char* img, int qb, int s) const {
    return row_frag<float, DK>(img, 16 * qb + (lane & 15), s, lane);
  }
  __device__ __forceinline__ Frag<float> k(const unsigned char* img, int t, int ks, int s) const {
    const int j = lane & 15;
    return row_frag<float, DK>(img, min(32 * ks + 8 * (j >> 2) + 4 * t + (j & 3), C - 1), s, lane);
  }
  __device__ __forceinline__ Frag<float> kt(const unsigned char* img, int s, int h, int ks) const {
    return col_frag<float, C, DK, false>(img, s, h, ks, lane);
  }
  __device__ __forceinline__ Frag<float> vt(const unsigned char* img, int ks) const {
    return col_frag<float, C, DV, true>(img, w, 0, ks, lane);
  }
};

// ----------------------------------------------------------------------------------------
// per-wave building blocks
// ----------------------------------------------------------------------------------------

// Decayed chunk state for the wave's 16 value columns, as 2*ceil(DK/32) tiles with permuted
// key-feature rows (tiles 2s, 2s+1 hold features 32s..32s+31):
//   F = sum_{s in chunk} exp(g - A_s) k_s v_s^T   (weights applied to the value operand)
template <typename T, int C, int DK, int DV>
__device__ __forceinline__ void chunk_state(const Reader<T, C, DK, DV>& rd, const unsigned char* kimg,
                                            const unsigned char* vimg, const float* wts, int lane,
                                            f32x4 (&F)[2 * cdiv(DK, 32)]) {
  constexpr int NKS_C = cdiv(C, 32), NKS_D = cdiv(DK, 32);
  const int g = lane >> 4;
#pragma unroll
  for (int b = 0; b < 2 * NKS_D; ++b) F[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS_C; ++ks) {
    const int p0 = min(32 * ks + 8 * g, C - 8);
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(wts + p0);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(wts + p0 + 4);
    const Frag<T> vf = frag_scale(rd.vt(vimg, ks), w0, w1);
#pragma unroll
    for (int s = 0; s < NKS_D; ++s) {
      mma(F[2 * s], rd.kt(kimg, s, 0, ks), vf);
      mma(F[2 * s + 1], rd.kt(kimg, s, 1, ks), vf);
    }
  }
}

// Read-out operand of a state kept as permuted tile pairs: tiles 2s, 2s+1 are fragment s.
template <typename T, int DK>
__device__ __forceinline__ Frag<T> node_frag(const f32x4 (&N)[2 * cdiv(DK, 32)], int s) {
  return frag_from<T>(N[2 * s], N[2 * s + 1]);
}

// One Fenwick node read out by every query of the chunk (level-weighted, decayed):
//   O[qb] += lambda[i, lev] * e^{A_i} * edoff * (N^T q_i)
// edoff = exp(log decay from the node's last position to the chunk's first position).
template <typename T, int C, int DK>
__device__ __forceinline__ void node_readout(const Frag<T> (&A)[cdiv(DK, 32)],
                                             const Frag<T> (&qf)[C / 16][cdiv(DK, 32)],
                                             const float* lam, int LS, const float (&eaq)[C / 16],
                                             int lev, float edoff, int lane, f32x4 (&O)[C / 16]) {
  constexpr int NQB = C / 16, NKS_D = cdiv(DK, 32);
  const int j = lane & 15;
  f32x4 Y[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) Y[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NKS_D; ++s) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) mma(Y[qb], A[s], qf[qb][s]);
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb)
    O[qb] += (lam[(16 * qb + j) * LS + lev] * eaq[qb] * edoff) * Y[qb];
}

// Masked score unit (query block qb, key step ks) as the P^T operand fragment of the value
// product: lane (j, g) element e = 4t + r holds key 32ks + 8g + e against query 16qb + j,
//   lambda[i, bit_length(i ^ s)] * exp(A_i - A_s) * (q_i . k_s)  for s <= i, else 0
// (chunk-local i, s). The two score tiles use permuted key rows (tile t, row i <-> key
// 32ks + 8(i/4) + 4t + i%4). exp(A_i - A_s) is e^{A_i} e^{-A_s} when the chunk's |A| < 40
// (`fact`), else taken directly. The key block 2ks + g/2 decides per lane: below the query
// block one level for the row, equal per-element levels, above masked.
template <typename T, int C, int DK, int DV>
__device__ __forceinline__ Frag<T> score_unit(const Reader<T, C, DK, DV>& rd, const unsigned char* qimg,
                                              const unsigned char* kimg, const float* lam, int LS,
                                              const float* dec, bool fact, int qb, int ks, int lane) {
  constexpr int NKS_D = cdiv(DK, 32);
  const int j = lane & 15, g = lane >> 4;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NKS_D; ++s) {
    const Frag<T> qfr = rd.q(qimg, qb, s);
    mma(s0, rd.k(kimg, 0, ks, s), qfr);
    mma(s1, rd.k(kimg, 1, ks, s), qfr);
  }
  const int qi = 16 * qb + j;
  const int kblk = 2 * ks + (g >> 1);
  const int key0 = min(32 * ks + 8 * g, C - 8);      // keys key0 .. key0+7 (in range when used)
  const float* lrow = lam + qi * LS;
  f32x4 d0, d1;
  if (fact) {
    const float eq = dec[C + qi];
    d0 = eq * *reinterpret_cast<const f32x4*>(dec + 2 * C + key0);
    d1 = eq * *reinterpret_cast<const f32x4*>(dec + 2 * C + key0 + 4);
  } else {
    const float aq = dec[qi];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      d0[r] = __expf(fminf(aq - dec[key0 + r], 0.f));
      d1[r] = __expf(fminf(aq - dec[key0 + 4 + r], 0.f));
    }
  }
  f32x4 p0, p1;
  if (kblk < qb) {
    const float lv = lrow[min(4 + bit_length((unsigned)(kblk ^ qb)), LS - 1)];
    p0 = (lv * s0) * d0;
    p1 = (lv * s1) * d1;
  } else if (kblk == qb) {
    const int kl = 8 * (g & 1);                       // first key of the lane inside the 16-block
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int k0 = kl + r, k1 = kl + 4 + r;
      const float l0 = lrow[min(bit_length((unsigned)(j ^ k0)), LS - 1)];
      const float l1 = lrow[min(bit_length((unsigned)(j ^ k1)), LS - 1)];
      p0[r] = k0 <= j ? s0[r] * l0 * d0[r] : 0.f;
      p1[r] = k1 <= j ? s1[r] * l1 * d1[r] : 0.f;
    }
  } else {
    p0 = f32x4{0.f, 0.f, 0.f, 0.f};
    p1 = p0;
  }
  return frag_from<T>(p0, p1);
}

// Output rows are written once and never read in the launch: non-temporal stores, which keep
// them from filling the L2 with dirty lines that the end of the launch must write back. The
// streamed input copies keep the default policy (non-temporal copies measured slower).
template <typename T> __device__ __forceinline__ void store_quad(T* p, const f32x4& v);
template <> __device__ __forceinline__ void store_quad<bf16>(bf16* p, const f32x4& v) {
  bf16x4 b;
  b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
  __builtin_nontemporal_store(b, reinterpret_cast<bf16x4*>(p));
}
template <> __device__ __forceinline__ void store_quad<float>(float* p, const f32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
// four output values into shared memory (8 bytes as bf16, 16 as float)
template <typename T> __device__ __forceinline__ void stage_quad(unsigned char* p, const f32x4& v);
template <> __device__ __forceinline__ void stage_quad<bf16>(unsigned char* p, const f32x4& v) {
  bf16x4 b;
  b[0] = (bf16)v[0]; b[1] = (bf16)v[1]; b[2] = (bf16)v[2]; b[3] = (bf16)v[3];
  *reinterpret_cast<bf16x4*>(p) = b;
}
template <> __device__ __forceinline__ void stage_quad<float>(unsigned char* p, const f32x4& v) {
  *reinterpret_cast<f32x4*>(p) = v;
}

// Score units (qb, ks), ks <= qb/2: the ones holding a diagonal block (ks = qb/2, the most
// work) first, one per wave, then the rest round-robin.
constexpr int num_units(int nqb) { return nqb <= 0 ? 0 : num_units(nqb - 1) + (nqb - 1) / 2 + 1; }
__device__ __forceinline__ void unit_decode(int un, int nqb, int& qb, int& ks) {
  if (un < nqb) { qb = un; ks = un / 2; return; }
  un -= nqb;                                  // off-diagonal units: (qb, ks), ks < qb/2
  qb = 2;
  ks = un;
  while (ks >= qb / 2) { ks -= qb / 2; ++qb; }
}

// ----------------------------------------------------------------------------------------
// node records between workgroups
// ----------------------------------------------------------------------------------------
// Node records pass between workgroups of one launch, possibly on different XCDs (each XCD has
// its own L2). A record is written once per launch, with device-scope (sc1) stores that write
// through to memory; the wave then waits until its stores have completed and sets its flag
// (device-scope atomic). Readers poll the flag with device-scope loads and then read the
// record with ordinary, cacheable loads: no cache can hold an older copy, since nothing reads
// a record before its flag is set and caches are invalidated between kernel launches, so
// later readers of a node on the same XCD share its L2 lines.
constexpr int kCpolDevice = 16;   // cache-policy immediate: sc1 (device scope)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t node_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
// 16-byte multiples (a bf16 or f32 operand fragment), contiguous at byte_off
template <typename V>
__device__ __forceinline__ void node_st(void* base, int byte_off, const V& x) {
  static_assert(sizeof(V) % 16 == 0, "16-byte node accesses");
  struct W { u32x4 r[sizeof(V) / 16]; };
  const W wv = __builtin_bit_cast(W, x);
#pragma unroll
  for (int i = 0; i < (int)(sizeof(V) / 16); ++i)
    __builtin_amdgcn_raw_buffer_store_b128(wv.r[i], node_rsrc(base), byte_off + 16 * i, 0, kCpolDevice);
}
// node decays share cache lines between records: device-scope accesses only
__device__ __forceinline__ float node_ld_f(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void node_st_f(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// after a wave's node writes, before its flag store: every access of the wave has completed
__device__ __forceinline__ void node_publish_fence() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ----------------------------------------------------------------------------------------
// the kernel
// ----------------------------------------------------------------------------------------

constexpr int kFlagBase = 64;   // ints ahead of the node flags (the ticket counter, alone in its line)

struct Params {
  const void* q; const void* k; const void* v;
  const float* log_a; const void* lam;
  void* out;
  int BH, T, L;
  int lam_bf16;     // lambda is bfloat16 (else float32)
  int nchunks;      // ceil(T / C)
  int sweep;        // R: chunks per workgroup (the kernel's NB)
  int m;            // log2(R)
  int nsweep;       // ceil(nchunks / R)
  int* sync;        // [0..1]: ticket counter (epoch << 32 | count); [kFlagBase + (bh*ns + e)*NW + w]: node flags
  float* gnode;     // [BH][ns][NW]: log decay across node e (one copy per wave)
  void* nodeT;      // [BH][ns][NW][ceil(DK/32)][64] Frag<T>: node e as read-out operands
  int spin_limit;   // polls of a node flag before the wait is abandoned
  // Variable-length batches (cu_seqlens non-null): head index bh = n * vH + h is sequence n of
  // head h, positions [cu_seqlens[n], cu_seqlens[n+1]) of the packed [vH, T, .] tensors (T is
  // then the packed length); nchunks and nsweep are those of the longest sequence. Tickets
  // enumerate only the (sweep, sequence, head) that exist; vtotal is their number when the
  // host knows it (the grid), else 0 (the grid is vN * vH * nsweep and the surplus leaves).
  const int* cu_seqlens;
  int vH, vN, vtotal;
};

// Node flags, data and decays are indexed by (head, node = sweep index e, wave).
__device__ __forceinline__ size_t node_slot(int bh, int ns, int e, int nw, int w) {
  return ((size_t)bh * ns + e) * nw + w;
}

// Variable-length batch: length of sequence n, clamped into the packed rows and to the longest
// length the grid was sized for (as the kernel reads it), and its number of sweeps.
template <int C, int NB>
__device__ __forceinline__ int varlen_sweeps(const Params& p, int n) {
  const int s0 = min(max(p.cu_seqlens[n], 0), p.T);
  const int s1 = min(max(p.cu_seqlens[n + 1], s0), min(s0 + p.nchunks * C, p.T));
  return cdiv(cdiv(s1 - s0, C), NB);
}

// Sum over the 64 lanes of a wave (DPP inclusive scan, read from the last lane): all lanes call.
__device__ __forceinline__ int wave_sum_int(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);
  return __builtin_amdgcn_readlane(x, 63);
}

// Variable-length batch: this workgroup's ticket, mapped sweep-major onto the (sweep, sequence,
// head) that exist. Tickets t in [P(s), P(s+1)) belong to sweep s, P(s) = H sum_n min(nsw_n, s);
// within a sweep, sequences in order, heads fastest. Wave 0 works it out (one sequence per lane,
// a binary search over s) and hands it to the other waves through `tk` (4 words). Returns false
// when the workgroup has no ticket and must leave at once; else sets the sweep, the virtual head
// and the value of a published flag in this launch, and `poisoned` when the counter was past the
// ticket count (a workspace that was never zero-filled: the sweep's rows are then written as NaN).
template <int C, int NB>
__device__ bool varlen_ticket(const Params& p, unsigned* tk, int tid, int blk, bool counted,
                              int& sw, int& bh, int& flagv, bool& poisoned) {
  if (tid < 64) {
    const int lane = tid;
    const int N = p.vN, H = p.vH;
    const int own = lane < N ? varlen_sweeps<C, NB>(p, lane) : 0;     // sequences 0..63
    auto P = [&](int s) {             // H * sum_n min(nsw_n, s)
      int acc = min(own, s);
      for (int n = 64 + lane; n - lane < N; n += 64) acc += n < N ? min(varlen_sweeps<C, NB>(p, n), s) : 0;
      return H * wave_sum_int(acc);
    };
    const int total = P(p.nsweep);
    bool ok = p.vtotal ? p.vtotal == total : blk < total;   // surplus workgroups, or a host count
    int t = blk;                                             // that disagrees: nothing is drawn
    unsigned ep = 0;
    bool nan_rows = false;
    if (ok && counted) {
      unsigned lo = 0, hi = 0;
      if (lane == 0) {
        unsigned long long* ctr = reinterpret_cast<unsigned long long*>(p.sync);
        const unsigned long long old = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lo = (unsigned)old;
        hi = (unsigned)(old >> 32);
        if (lo == (unsigned)total - 1u) {            // epochs skip 2^32 - 1 (flag value 0)
          const unsigned nep = hi + 1u == 0xffffffffu ? 0u : hi + 1u;
          __hip_atomic_store(ctr, (unsigned long long)nep << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
      const unsigned cnt = __builtin_amdgcn_readlane(lo, 0);
      ep = __builtin_amdgcn_readlane(hi, 0);
      // a count past the tickets: a workspace never zero-filled. The counts drawn then run over
      // consecutive values, so (count - total) mod total meets every ticket once; that sweep's
      // rows are written as NaN.
      nan_rows = cnt >= (unsigned)total;
      t = nan_rows ? (int)((cnt - (unsigned)total) % (unsigned)total) : (int)cnt;
    }
    int s = 0, n = 0, h = 0;
    if (ok) {
      int lo = 0, hi = p.nsweep;                     // the largest s with P(s) <= t
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (P(mid) <= t) lo = mid; else hi = mid;
      }
      s = lo;
      const int r = t - P(s);
      int i = r / H;
      h = r - i * H;
      for (int b = 0; b * 64 < N; ++b) {             // the i-th sequence that has sweep s
        const int m = b * 64 + lane;
        const bool act = m < N && (b == 0 ? own : varlen_sweeps<C, NB>(p, m)) > s;
        const unsigned long long mask = __ballot(act);
        const int cnt = __popcll(mask);
        if (i < cnt) {
          const int rank = __builtin_amdgcn_mbcnt_hi((unsigned)(mask >> 32),
                                                     __builtin_amdgcn_mbcnt_lo((unsigned)mask, 0u));
          n = b * 64 + __ffsll((long long)__ballot(act && rank == i)) - 1;
          break;
        }
        i -= cnt;
      }
    }
    if (lane == 0) {
      tk[0] = ok ? (nan_rows ? 2u : 1u) : 0u;
      tk[1] = ep + 1u;
      tk[2] = (unsigned)s;
      tk[3] = (unsigned)(n * H + h);
    }
  }
  __syncthreads();
  flagv = (int)__builtin_amdgcn_readfirstlane(tk[1]);
  sw = (int)__builtin_amdgcn_readfirstlane(tk[2]);
  bh = (int)__builtin_amdgcn_readfirstlane(tk[3]);
  const unsigned st = __builtin_amdgcn_readfirstlane(tk[0]);
  poisoned = st == 2u;
  return st != 0u;
}

// The forward pass: one workgroup per sweep of NB chunks of one head, one wave per 16 value
// columns; ns = nsweep - 1 sweeps per head publish a node (the last one has no reader).
//
// Node of sweep e: the Fenwick node over sweeps that ends at e, i.e. the lowbit(e+1) sweeps
// (e - lowbit(e+1), e], decayed to the end of e:
//   node(e) = H_e + sum_{i < ctz(e+1)} exp(gacc_i) node(e - 2^i),
// H_e = sum_{s in sweep e} exp(A_end(e) - A_s) k_s v_s^T, gacc_i the log decay from the end of
// node(e - 2^i) to the end of e. Sweep sw reads the nodes ending at ((sw >> j) << j) - 1 for
// each set bit j of sw (level J + 1 + m + j); the first ctz(sw+1) of them are exactly the
// children of its own node. VL: a variable-length batch (p.cu_seqlens), a separate instance so
// that the fixed-length kernel carries none of its code.
template <typename T, int C, int DK, int DV, int NB, bool VL>
__global__ __launch_bounds__(4 * DV, 2) void lla_fwd_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int ES = (int)sizeof(T);
  constexpr int NT = 4 * DV, NW = DV / 16;
  constexpr int NQB = C / 16, NKS_C = cdiv(C, 32), NKS_D = cdiv(DK, 32), NTF = 2 * NKS_D;
  constexpr int J = ilog2(C);
  constexpr int NUNITS = num_units(NQB);
  constexpr int XREG = DK >= 128 ? 2 : 5;   // nodes over earlier sweeps held in registers
  static_assert(NB >= 1 && NB <= kMaxSweep, "one or two resident chunks");
  static_assert(XREG <= kFlagCopy && NW <= 8, "node flag copies");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index: uniform
  const int j = lane & 15, g = lane >> 4;
  const int L = p.L, ns = p.nsweep - 1;
  const Smem S = smem_layout(ES, C, DK, DV, NB);

  // ticket -> (head, sweep), sweep-major. The counter holds (epoch << 32) | count: the
  // workgroup that draws the last ticket of a launch resets the count and moves to the next
  // epoch, and node flags hold epoch + 1, so a workspace that was zero-filled once stays valid
  // for every later launch without being cleared again.
  int t = blockIdx.x;
  int flagv = 1;                      // value of a published flag in this launch
  int vsw = 0, vbh = 0;               // variable-length batch: the ticket's sweep and head
  bool poisoned = false;              // counter past the tickets: write the sweep's rows as NaN
  if constexpr (VL) {
    if (!varlen_ticket<C, NB>(p, reinterpret_cast<unsigned*>(smem + S.ticket), tid, blockIdx.x, ns > 0,
                              vsw, vbh, flagv, poisoned))
      return;
  } else if (ns > 0) {
    const unsigned total = (unsigned)p.BH * (unsigned)p.nsweep;
    unsigned* tk = reinterpret_cast<unsigned*>(smem + S.ticket);
    if (tid == 0) {
      unsigned long long* ctr = reinterpret_cast<unsigned long long*>(p.sync);
      const unsigned long long old = __hip_atomic_fetch_add(ctr, 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const unsigned cnt = (unsigned)old, ep = (unsigned)(old >> 32);
      if (cnt == total - 1) {         // epochs skip 2^32 - 1, whose flag value would be 0
        const unsigned nep = ep + 1u == 0xffffffffu ? 0u : ep + 1u;
        __hip_atomic_store(ctr, (unsigned long long)nep << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      tk[0] = cnt;
      tk[1] = ep;
    }
    __syncthreads();
    const unsigned cnt = __builtin_amdgcn_readfirstlane(tk[0]);
    flagv = (int)(__builtin_amdgcn_readfirstlane(tk[1]) + 1u);
    // A count past the tickets: a workspace that was never zero-filled. The counts drawn are
    // consecutive, so (count - total) mod total meets every ticket once; that sweep's rows are
    // written as NaN (no node is read or published) and the workspace stays in that state until
    // it is zero-filled again.
    poisoned = cnt >= total;
    t = poisoned ? (int)((cnt - total) % total) : (int)cnt;
  }
  const int sw = VL ? vsw : t / p.BH, bh = VL ? vbh : t - (t / p.BH) * p.BH;

  // this head's sequence: its length, first row in the tensors, chunk count
  int Tn = p.T, nchunks = p.nchunks;
  size_t hoff = (size_t)bh * p.T;
  if constexpr (VL) {
    const int n = bh / p.vH, h = bh - n * p.vH;
    // clamped into the packed rows and to the longest length the grid was sized for
    const int s0 = min(max(p.cu_seqlens[n], 0), p.T);
    const int s1 = min(max(p.cu_seqlens[n + 1], s0), min(s0 + p.nchunks * C, p.T));
    Tn = s1 - s0;
    nchunks = cdiv(Tn, C);
    hoff = (size_t)h * p.T + s0;
  }

  const T* qg = reinterpret_cast<const T*>(p.q) + hoff * DK;
  const T* kg = reinterpret_cast<const T*>(p.k) + hoff * DK;
  const T* vg = reinterpret_cast<const T*>(p.v) + hoff * DV;
  const float* lag = p.log_a + hoff;
  const size_t lam_off = hoff * L;       // lambda element offset of this head's rows
  T* og = reinterpret_cast<T*>(p.out) + hoff * DV;

  const int c0 = sw * NB;
  const int nch = min(NB, nchunks - c0);
  const int next = __builtin_popcount((unsigned)sw);

  if (poisoned) {
    const f32x4 nan4 = {__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    for (int u = 0; u < nch; ++u) {
      const int t0 = (c0 + u) * C;
      const int valid = min(C, Tn - t0);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qi = 16 * qb + j;
        if (qi < valid) store_quad<T>(og + (size_t)(t0 + qi) * DV + 16 * w + 4 * g, nan4);
      }
    }
    return;
  }

  Reader<T, C, DK, DV> rd;
  rd.init(lane, w);

  // ---------------- Fenwick nodes over earlier sweeps ----------------
  // The x-th node of sw (x-th set bit j of sw, lowest first) ends at sweep ((sw >> j) << j) - 1
  // and has level J + 1 + m + j; the first XREG of them are tabulated once.
  auto node_index_slow = [&](int x) {
    unsigned m = (unsigned)sw;
    for (int i = 0; i < x && m; ++i) m &= m - 1;
    return m ? ((sw >> __builtin_ctz(m)) << __builtin_ctz(m)) - 1 : 0;
  };
  auto node_level_slow = [&](int x) {
    unsigned m = (unsigned)sw;
    for (int i = 0; i < x && m; ++i) m &= m - 1;
    return m ? J + 1 + p.m + __builtin_ctz(m) : 0;
  };
  int NE[XREG], NLV[XREG];
  {
    unsigned m = (unsigned)sw;
#pragma unroll
    for (int x = 0; x < XREG; ++x) {
      const int tz = m ? __builtin_ctz(m) : 0;
      NE[x] = m ? ((sw >> tz) << tz) - 1 : 0;
      NLV[x] = J + 1 + p.m + tz;
      m &= m - 1;
    }
  }
  auto node_index = [&](int x) { return x < XREG ? NE[x] : node_index_slow(x); };
  auto node_level = [&](int x) { return x < XREG ? NLV[x] : node_level_slow(x); };
  const Frag<T>* ndT = reinterpret_cast<const Frag<T>*>(p.nodeT);
  auto node_base = [&](int e) { return ndT + node_slot(bh, ns, e, NW, w) * NKS_D * 64; };
  auto flag_set = [&](int e) {
    const int* f = p.sync + kFlagBase + node_slot(bh, ns, e, NW, w);
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) == flagv;
  };
  int bad = 0;                       // a flag never came: outputs become NaN (wave-uniform)
  auto wait_node = [&](int e) {
    int n = 0;
    while (!flag_set(e)) {
      if (++n > p.spin_limit) { bad = 1; break; }
      __builtin_amdgcn_s_sleep(2);
    }
  };
  // node operands of the first XREG nodes in registers; bit x of `loaded` once X[x] is there
  Frag<T> X[XREG][NKS_D];
  float XD[XREG];            // log decay across each node
  unsigned loaded = 0;
  auto load_x = [&](auto xc) {
    constexpr int x = decltype(xc)::value;
    const Frag<T>* nb = node_base(NE[x]);
#pragma unroll
    for (int s = 0; s < NKS_D; ++s) X[x][s] = nb[s * 64 + lane];
    XD[x] = node_ld_f(p.gnode + node_slot(bh, ns, NE[x], NW, w));
    loaded |= 1u << x;
  };


  // ---------------- load the sweep: every input read is issued here ----------------
  // Everything moves by global_load_lds straight into shared memory, in this order: each wave's
  // node flags (device scope, like the flag polls: usually already set, those sweeps started long
  // before), the chunks' log_a (wave 0), the k and v images (phase A), the lambda rows and the q
  // images (phase B). The copies complete in issue order, so "no more than the copies issued
  // after X outstanding" means X has landed. Nothing is loaded into registers before phase A:
  // the compiler drains every outstanding copy before it uses a register loaded alongside them,
  // which would hold phase A back until the q images arrive.
  int* flc = reinterpret_cast<int*>(smem + S.flg) + w * kFlagCopy;
  if (ns > 0 && lane < XREG) {
    int e = NE[0];                      // lane x copies the flag of the x-th node (selects, not
    static_for<XREG>([&](auto xc) {     // a dynamic register index)
      constexpr int x = decltype(xc)::value;
      if (lane == x) e = NE[x];
    });
    const int* src = p.sync + kFlagBase + node_slot(bh, ns, e, NW, w);
    copy_lds4_device(src, flc);
  }
  int t0s[NB], valids[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int uc = u < nch ? u : 0;                 // a missing last chunk re-reads chunk 0
    t0s[u] = (c0 + uc) * C;
    valids[u] = min(C, Tn - t0s[u]);
  }
  if (w == 0) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      float* la = reinterpret_cast<float*>(smem + S.dec[u]) + 3 * C;
#pragma unroll
      for (int b = 0; b < cdiv(C, 64); ++b) {
        if (b * 64 + lane < C) {
          const float* src = lag + t0s[u] + min(b * 64 + lane, valids[u] - 1);
          copy_lds4(src, la + b * 64);
        }
      }
    }
  }
  DmaPlan<T, C, DK, NW, false> dk_plan;
  DmaPlan<T, C, DV, NW, true> dv_plan;
  dk_plan.init(w, lane);
  dv_plan.init(w, lane);
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    dk_plan.issue(smem + S.k[u], kg + (size_t)t0s[u] * DK, valids[u], w, lane);
    dv_plan.issue(smem + S.v[u], vg + (size_t)t0s[u] * DV, valids[u], w, lane);
  }
  const bool lbf = p.lam_bf16 != 0;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    float* lam = reinterpret_cast<float*>(smem + S.lam[u]);
    const size_t off = lam_off + (size_t)t0s[u] * L;
    if (lbf)
      dma_lambda_bf16(lam, reinterpret_cast<const unsigned short*>(p.lam) + off, valids[u] * L, C * L, w, NW, lane);
    else
      dma_lambda(lam, reinterpret_cast<const float*>(p.lam) + off, valids[u] * L, C * L, w, NW, lane);
  }
#pragma unroll
  for (int u = 0; u < NB; ++u) dk_plan.issue(smem + S.q[u], qg + (size_t)t0s[u] * DK, valids[u], w, lane);
  if (w == 0) {
    // log_a landed (k, v and q copies of wave 0 follow it, lambda's at least none): scan, publish
    wait_vm<NB * (2 * dma_count<T, C, DK, NW>(0) + dma_count<T, C, DV, NW>(0))>();
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      DecayRegs<C> ar;
      float* dec = reinterpret_cast<float*>(smem + S.dec[u]);
      ar.fetch_lds(dec + 3 * C, valids[u], lane);
      ar.scan(lane);
      ar.publish(dec, reinterpret_cast<int*>(smem + S.flag[u]), ar.total(), lane);
    }
  }
  wait_vm<NB * dma_count<T, C, DK, NW>(NW - 1)>();   // this wave's flags, k, v, lambda landed
  if (lbf) {                  // the wave's own bf16 lambda copies -> floats; read after a barrier
#pragma unroll
    for (int u = 0; u < NB; ++u) lambda_widen(reinterpret_cast<float*>(smem + S.lam[u]), C * L, w, NW, lane);
  }
  lds_barrier();
  float gch[NB];                        // total log decay of each chunk
#pragma unroll
  for (int u = 0; u < NB; ++u)
    gch[u] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(reinterpret_cast<const int*>(smem + S.flag[u])[1]));
  int fl0[XREG];
#pragma unroll
  for (int x = 0; x < XREG; ++x) fl0[x] = x < next ? flc[x] : 0;

  // published nodes over earlier sweeps: into registers now, their latency hides behind phase A
  static_for<XREG>([&](auto xc) {
    constexpr int x = decltype(xc)::value;
    if (x < next && __builtin_amdgcn_readfirstlane(fl0[x]) == flagv) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      load_x(xc);
    }
  });

  // ---------------- phase A: chunk states, chunk 0's state, the sweep total ----------------
  Frag<T> SL[NKS_D];              // state of chunk 0 (decayed to its end), level J+1 for chunk 1
  f32x4 H[NTF];
#pragma unroll
  for (int b = 0; b < NTF; ++b) H[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float G = 0.f;
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    if (u < nch) {
      f32x4 F[NTF];
      chunk_state<T, C, DK, DV>(rd, smem + S.k[u], smem + S.v[u],
                                reinterpret_cast<const float*>(smem + S.dec[u]) + 3 * C, lane, F);
      const float d = __expf(gch[u]);
#pragma unroll
      for (int b = 0; b < NTF; ++b) H[b] = d * H[b] + F[b];
      G += gch[u];
      if (u == 0 && NB > 1) {
#pragma unroll
        for (int s = 0; s < NKS_D; ++s) SL[s] = node_frag<T, DK>(F, s);
      }
    }
  }

  // Own node: the sweep total plus its children (the first kc nodes of sw), published right
  // away when the children are already in registers, else after the intra-chunk work.
  const int kc = sw < ns ? __builtin_ctz((unsigned)(sw + 1)) : 0;
  bool published = sw >= ns;
  auto publish = [&]() {            // children x < min(kc, XREG) are loaded
    float gacc = G;
    static_for<XREG>([&](auto xc) {
      constexpr int x = decltype(xc)::value;
      if (x < kc) {
        const float d = __expf(gacc);
#pragma unroll
        for (int s = 0; s < NKS_D; ++s) {
          f32x4 lo, hi;
          frag_to_f32(X[x][s], lo, hi);
          H[2 * s] += d * lo;
          H[2 * s + 1] += d * hi;
        }
        gacc += XD[x];
      }
    });
    for (int x = XREG; x < kc; ++x) {   // beyond the registers: wait and read on demand
      const int e = node_index(x);
      wait_node(e);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      const Frag<T>* nb = node_base(e);
      const float d = __expf(gacc);
#pragma unroll
      for (int s = 0; s < NKS_D; ++s) {
        f32x4 lo, hi;
        frag_to_f32(nb[s * 64 + lane], lo, hi);
        H[2 * s] += d * lo;
        H[2 * s + 1] += d * hi;
      }
      gacc += node_ld_f(p.gnode + node_slot(bh, ns, e, NW, w));
    }
    if (__builtin_amdgcn_readfirstlane(bad)) {
#pragma unroll
      for (int b = 0; b < NTF; ++b) H[b] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
    const size_t me = node_slot(bh, ns, sw, NW, w);
    Frag<T>* oT = reinterpret_cast<Frag<T>*>(p.nodeT) + me * NKS_D * 64;
#pragma unroll
    for (int s = 0; s < NKS_D; ++s)
      node_st<Frag<T>>(oT, (s * 64 + lane) * (int)sizeof(Frag<T>), node_frag<T, DK>(H, s));
    if (lane == 0) node_st_f(p.gnode + me, gacc);
    node_publish_fence();
    if (lane == 0) __hip_atomic_store(p.sync + kFlagBase + me, flagv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  if (!published && kc <= XREG) {
    const unsigned need = (1u << kc) - 1u;
    if ((loaded & need) == need) {
      publish();
      published = true;
    }
  }

  wait_vm<0>();                         // this wave's q images landed
  lds_barrier();

  // ---------------- phase B, intra-sweep part: scores, P.V, the node inside the sweep ----------------
  f32x4 O[NB][NQB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    if (u < nch) {
      const unsigned char* qimg = smem + S.q[u];
      const unsigned char* kimg = smem + S.k[u];
      const float* lam = reinterpret_cast<const float*>(smem + S.lam[u]);
      const float* dec = reinterpret_cast<const float*>(smem + S.dec[u]);
      Frag<T>* pf = reinterpret_cast<Frag<T>*>(smem + S.pf[u]);
      const bool fact = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int*>(smem + S.flag[u])) != 0;

      // masked scores -> P^T fragments (shared by all waves)
      for (int un = w; un < NUNITS; un += NW) {
        int qb, ks;
        unit_decode(un, NQB, qb, ks);
        pf[(qb * NKS_C + ks) * 64 + lane] = score_unit<T, C, DK, DV>(rd, qimg, kimg, lam, L, dec, fact, qb, ks, lane);
      }
      lds_barrier();

      Frag<T> vfr[NKS_C];
#pragma unroll
      for (int ks = 0; ks < NKS_C; ++ks) vfr[ks] = rd.vt(smem + S.v[u], ks);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        O[u][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks <= qb / 2; ++ks) mma(O[u][qb], vfr[ks], pf[(qb * NKS_C + ks) * 64 + lane]);
      }

      // chunk 0 of the sweep, read by chunk 1 (level J+1; adjacent, so no decay in between)
      if (NB > 1 && u == 1) {
        Frag<T> qf[NQB][NKS_D];
        float eaq[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          eaq[qb] = dec[C + 16 * qb + j];
#pragma unroll
          for (int s = 0; s < NKS_D; ++s) qf[qb][s] = rd.q(qimg, qb, s);
        }
        node_readout<T, C, DK>(SL, qf, lam, L, eaq, J + 1, 1.f, lane, O[u]);
      }
    }
  }

  // ---------------- nodes that were not there yet; own node if it waited for them ----------------
  // Each round polls the flags of every node still missing at once and loads all that are
  // published, until the nodes in `need` are there: first the children (later sweeps wait
  // for this node), then the rest.
  const int nreg = min(next, XREG);
  auto gather = [&](unsigned need) {
    int n = 0;
    while (!bad && (loaded & need) != need) {
      int fl[XREG];
#pragma unroll
      for (int x = 0; x < XREG; ++x)
        fl[x] = (x < nreg && !((loaded >> x) & 1u))
                    ? __hip_atomic_load(p.sync + kFlagBase + node_slot(bh, ns, NE[x], NW, w),
                                        __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : 0;
      static_for<XREG>([&](auto xc) {
        constexpr int x = decltype(xc)::value;
        if (x < nreg && !((loaded >> x) & 1u) && __builtin_amdgcn_readfirstlane(fl[x]) == flagv) {
          __atomic_signal_fence(__ATOMIC_SEQ_CST);
          load_x(xc);
        }
      });
      if ((loaded & need) == need) break;
      if (++n > p.spin_limit) { bad = 1; break; }
      __builtin_amdgcn_s_sleep(2);
    }
  };
  gather((1u << min(kc, XREG)) - 1u);
  if (!published) publish();
  gather((1u << nreg) - 1u);
  for (int x = XREG; x < next; ++x) wait_node(node_index(x));
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  // ---------------- phase B, read-out of earlier sweeps and store ----------------
  float gam = 0.f;           // log decay from the sweep's first position to the current chunk start
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    if (u < nch) {
      const int t0 = (c0 + u) * C;
      const int valid = min(C, Tn - t0);
      const unsigned char* qimg = smem + S.q[u];
      const float* lam = reinterpret_cast<const float*>(smem + S.lam[u]);
      const float* dec = reinterpret_cast<const float*>(smem + S.dec[u]);
      if (next > 0) {
        Frag<T> qf[NQB][NKS_D];
        float eaq[NQB];
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb) {
          eaq[qb] = dec[C + 16 * qb + j];
#pragma unroll
          for (int s = 0; s < NKS_D; ++s) qf[qb][s] = rd.q(qimg, qb, s);
        }
        // Fenwick nodes made of whole earlier sweeps (levels J+m+1 ..), lowest bit first
        float dext = 0.f;
#pragma unroll
        for (int x = 0; x < XREG; ++x) {
          if (x < next) {
            node_readout<T, C, DK>(X[x], qf, lam, L, eaq, node_level(x), __expf(gam + dext), lane, O[u]);
            dext += XD[x];
          }
        }
        for (int x = XREG; x < next; ++x) {    // beyond the register budget: load on demand
          const int e = node_index(x);
          const Frag<T>* nb = node_base(e);
          Frag<T> A[NKS_D];
#pragma unroll
          for (int s = 0; s < NKS_D; ++s) A[s] = nb[s * 64 + lane];
          node_readout<T, C, DK>(A, qf, lam, L, eaq, node_level(x), __expf(gam + dext), lane, O[u]);
          dext += node_ld_f(p.gnode + node_slot(bh, ns, e, NW, w));
        }
      }
      // store rows [0, valid); NaN if a node never arrived. A wave holds 16 columns of every row,
      // so the rows go through shared memory (the first chunk's k image onwards, 16-byte units
      // XOR-swizzled by row) and leave as whole rows, each 16-byte piece by one lane:
      // non-temporal stores of whole cache lines. The stage is free once every wave is past the
      // second chunk's score barrier (the first chunk's k and v images are read before it) and,
      // for the second chunk, once the first chunk's rows are copied out; a sweep of one chunk
      // has no second score barrier, so it takes a barrier of its own (its stage may reach into
      // the v image that P.V reads when dv > dk)
      unsigned char* stage = smem + S.k[0];
      constexpr int RB = DV * ES, VR = RB / 16;   // row bytes, 16-byte units per row
      if (u > 0 || nch < 2) lds_barrier();
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qi = 16 * qb + j;
        if (__builtin_amdgcn_readfirstlane(bad)) O[u][qb] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
        const int cb = (16 * w + 4 * g) * ES;      // the lane's bytes in the row
        stage_quad<T>(stage + qi * RB + (((cb >> 4) ^ (qi & (VR - 1))) << 4) + (cb & 15), O[u][qb]);
      }
      lds_barrier();
      for (int v = tid; v < C * VR; v += NT) {
        const int r = v / VR, c16 = v % VR;
        if (r < valid) {
          const u32x4 x = *reinterpret_cast<const u32x4*>(stage + r * RB + ((c16 ^ (r & (VR - 1))) << 4));
          __builtin_nontemporal_store(x, reinterpret_cast<u32x4*>(reinterpret_cast<unsigned char*>(og + (size_t)(t0 + r) * DV) + c16 * 16));
        }
      }
      gam += gch[u];
    }
  }
}

}  // namespace lla
