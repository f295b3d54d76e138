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
// Work split. One kernel, one workgroup per "sweep" of R = 2^m consecutive chunks of one head
// (lla_fused_kernel). Workgroups take a ticket from an atomic counter and map it sweep-major,
// so every sweep they wait for belongs to a workgroup that started earlier.
//   phase A: chunk states of the sweep (decayed k^T v on MFMA); the Fenwick nodes inside the
//            sweep are kept in registers; the sweep total plus the nodes of earlier sweeps it
//            absorbs (a Fenwick tree over sweeps) is published as this sweep's node.
//   phase B: chunk by chunk: dense masked block on MFMA, read-out of the live Fenwick nodes
//            (inside the sweep from registers, earlier sweeps from the published nodes),
//            output store.
// A node is published per wave (16 value columns): data stores, an agent-scope release fence,
// then a flag; readers poll the flag (bounded: on timeout the outputs are set to NaN so that
// a broken dependency can never hang the device) and take an agent-scope acquire fence.
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

__device__ __forceinline__ Frag<bf16> frag_select_impl(bool c, const Frag<bf16>& a, const Frag<bf16>& b) {
  Frag<bf16> r; r.v = c ? a.v : b.v; return r;
}
__device__ __forceinline__ Frag<float> frag_select_impl(bool c, const Frag<float>& a, const Frag<float>& b) {
  Frag<float> r; r.lo = c ? a.lo : b.lo; r.hi = c ? a.hi : b.hi; return r;
}
template <typename T> __device__ __forceinline__ Frag<T> zero_frag() {
  const f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return frag_from<T>(z, z);
}
template <typename T>
__device__ __forceinline__ Frag<T> frag_select(bool c, const Frag<T>& a, const Frag<T>& b) {
  return frag_select_impl(c, a, b);
}

// 4 consecutive elements of a fragment (one half: e0 = 0 or 4)
template <typename T> struct Quad;
template <> struct Quad<bf16> { typedef bf16x4 type; };
template <> struct Quad<float> { typedef f32x4 type; };

__device__ __forceinline__ int bit_length(unsigned x) { return 32 - __clz((int)x); }


constexpr int kLamCap = 24;       // lambda levels held per position (T <= 2^23)
constexpr int kSweepCap = 4;      // chunks per sweep: Fenwick nodes inside a sweep in registers

// bf16 operands contracted over positions (v, decayed k) are read with the gfx950 transposing
// LDS read from a row-major image; f32 ones are stored in fragment order instead.
template <typename T> struct TrNative { static constexpr bool value = sizeof(T) == 2; };

// ----------------------------------------------------------------------------------------
// shared-memory images of one chunk
// ----------------------------------------------------------------------------------------
// A [C, DF] block is kept row-major in 4-element quads whose place inside a row is XOR-swizzled:
//   TR = false: quad q of row r sits at q ^ (r mod 16). A fragment read takes one quad of
//               16 consecutive rows per 16 lanes: 16 distinct bank groups.
//   TR = true : quad q of row r sits at q ^ 4 (r mod 4). A transposing read takes 4 quads of
//               4 consecutive rows per 16 lanes: 16 distinct bank groups.
template <typename T, int DF, bool TR>
struct Img {
  static constexpr int NQ = DF / 4;                  // quads per row
  static constexpr int QB = 4 * (int)sizeof(T);      // bytes per quad
  static constexpr int ROWB = DF * (int)sizeof(T);   // bytes per row
  __device__ __forceinline__ static int swz(int r) {
    return TR ? ((4 * (r & 3)) & (NQ - 1)) : (r & (NQ - 1) & 15);
  }
  __device__ __forceinline__ static int off(int r, int q) { return r * ROWB + (q ^ swz(r)) * QB; }
};

struct ChunkSmem {
  int qimg, kimg, pf, kt, vt, lam, aloc, ea, eb, flag, total;
};

// Byte offsets of one chunk's shared memory (host and device agree). A fragment slot is one
// operand fragment for all 64 lanes (64 x 8 elements). with_q: the query-side images (q, k,
// masked scores, lambda); with_kt: the decayed-key operand of chunk states.
template <typename T>
__host__ __device__ inline ChunkSmem chunk_smem(int C, int DK, int DV, int L, bool with_q,
                                                bool with_kt) {
  const int es = (int)sizeof(T);
  const int slot = 64 * 8 * es;
  const int nqb = C / 16, nks_c = (C + 31) / 32;
  const bool trn = es == 2;
  ChunkSmem s;
  int off = 0;
  s.qimg = off; off += with_q ? C * DK * es : 0;
  s.kimg = off; off += with_q ? C * DK * es : 0;
  s.pf = off;   off += with_q ? nqb * nks_c * slot : 0;
  s.kt = off;   off += with_kt ? (trn ? C * DK * es : (DK / 16) * nks_c * slot) : 0;
  s.vt = off;   off += trn ? C * DV * es : (DV / 16) * nks_c * slot;
  s.lam = off;  off += with_q ? ((C * L * 4 + 15) & ~15) : 0;
  s.aloc = off; off += C * 4;
  s.ea = off;   off += C * 4;
  s.eb = off;   off += C * 4;
  s.flag = off; off += 16;
  s.total = (off + 255) & ~255;
  return s;
}

// Shared memory of the fused kernel: the phase A and phase B layouts overlap from offset 0;
// the workgroup ticket sits after both.
template <typename T>
__host__ __device__ inline int fused_ticket_offset(int C, int DK, int DV, int L) {
  const int a = chunk_smem<T>(C, DK, DV, L, false, true).total;
  const int b = chunk_smem<T>(C, DK, DV, L, true, false).total;
  return a > b ? a : b;
}
template <typename T>
__host__ __device__ inline int fused_smem_bytes(int C, int DK, int DV, int L) {
  return fused_ticket_offset<T>(C, DK, DV, L) + 16;
}

// ----------------------------------------------------------------------------------------
// global -> registers -> shared memory staging of one chunk
// ----------------------------------------------------------------------------------------

template <typename T> struct Pair;
template <> struct Pair<bf16> { typedef bf16 __attribute__((ext_vector_type(2))) type; };
template <> struct Pair<float> { typedef float __attribute__((ext_vector_type(2))) type; };

template <typename T>
__device__ __forceinline__ uint4 load_piece(const T* p, bool valid) {
  if (!valid) return make_uint4(0, 0, 0, 0);
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ unsigned word_of(const uint4& u, int i) {
  return i == 0 ? u.x : i == 1 ? u.y : i == 2 ? u.z : u.w;
}

// element i of a 16-byte piece, as float
template <typename T> __device__ __forceinline__ float elemf(const uint4& u, int i);
template <> __device__ __forceinline__ float elemf<bf16>(const uint4& u, int i) {
  const unsigned w = word_of(u, i >> 1);
  return __builtin_bit_cast(float, (i & 1) ? (w & 0xffff0000u) : (w << 16));
}
template <> __device__ __forceinline__ float elemf<float>(const uint4& u, int i) {
  return __builtin_bit_cast(float, word_of(u, i));
}

// a 16-byte piece with every element multiplied by w (rounded back to T)
template <typename T> __device__ __forceinline__ uint4 scale_piece(const uint4& u, float w);
template <> __device__ __forceinline__ uint4 scale_piece<bf16>(const uint4& u, float w) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)(elemf<bf16>(u, i) * w);
  const u32x4 x = __builtin_bit_cast(u32x4, r);
  return make_uint4(x[0], x[1], x[2], x[3]);
}
template <> __device__ __forceinline__ uint4 scale_piece<float>(const uint4& u, float w) {
  return make_uint4(__builtin_bit_cast(unsigned, elemf<float>(u, 0) * w),
                    __builtin_bit_cast(unsigned, elemf<float>(u, 1) * w),
                    __builtin_bit_cast(unsigned, elemf<float>(u, 2) * w),
                    __builtin_bit_cast(unsigned, elemf<float>(u, 3) * w));
}

// Writes one 16-byte piece (features f0..f0+EPP-1 of row r) into a swizzled image.
template <typename T, int DF, bool TR>
__device__ __forceinline__ void put_piece(unsigned char* img, int r, int f0, const uint4& x) {
  typedef Img<T, DF, TR> I;
  if (sizeof(T) == 2) {
    // two quads 2p, 2p+1 land on an aligned pair, swapped when the swizzle flips bit 0
    const int q = f0 / 4;
    const int phys = q ^ I::swz(r);
    uint4 y = (phys & 1) ? make_uint4(x.z, x.w, x.x, x.y) : x;
    *reinterpret_cast<uint4*>(img + r * I::ROWB + (phys & ~1) * I::QB) = y;
  } else {
    *reinterpret_cast<uint4*>(img + I::off(r, f0 / 4)) = x;
  }
}

// Writes 2 consecutive contraction elements k0, k0+1 (k0 even) of fragment row/column rc of
// fragment slot `slot` (fragment-order storage, f32 position-contracted operands).
template <typename T>
__device__ __forceinline__ void put_pair(T* base, int slot, int rc, int k0,
                                         const typename Pair<T>::type& p2) {
  const int hidx = k0 >> 2;
  const int g = hidx & 3, e = (hidx >> 2) * 4 + (k0 & 3);
  *reinterpret_cast<typename Pair<T>::type*>(base + ((size_t)slot * 64 + rc + 16 * g) * 8 + e) = p2;
}

// One [C, DF] block (row stride DF; rows past `valid` read as 0) in registers: units of 2
// consecutive rows x one 16-byte piece, dealt round-robin to the NT threads.
template <typename T, int C, int DF, int NT>
struct BlockRegs {
  static constexpr int EPP = 16 / (int)sizeof(T);
  static constexpr int PPR = DF / EPP;
  static constexpr int UNITS = (C / 2) * PPR;
  static constexpr int ITERS = (UNITS + NT - 1) / NT;
  uint4 x[ITERS][2];

  __device__ __forceinline__ static int row0(int tid, int it) {
    const int u = tid + it * NT;
    return u < UNITS ? 2 * (u / PPR) : 0;
  }

  // Branch-free: every lane issues its loads at a clamped, in-bounds address and zeroes what
  // lies past `valid` (valid >= 1), so the compiler can count outstanding loads exactly.
  __device__ __forceinline__ void fetch(const T* __restrict__ g, int valid, int tid) {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int u = tid + it * NT;
      const bool ok = (UNITS % NT == 0) || u < UNITS;
      const int uc = ok ? u : 0;
      const int r0 = 2 * (uc / PPR), f0 = (uc % PPR) * EPP;
      const int ra = min(r0, valid - 1), rb = min(r0 + 1, valid - 1);
      const uint4 a = *reinterpret_cast<const uint4*>(g + (size_t)ra * DF + f0);
      const uint4 b = *reinterpret_cast<const uint4*>(g + (size_t)rb * DF + f0);
      const uint4 z = make_uint4(0, 0, 0, 0);
      x[it][0] = (ok && r0 < valid) ? a : z;
      x[it][1] = (ok && r0 + 1 < valid) ? b : z;
    }
  }

  // row-major swizzled image; ws[it][i] (if given) scales row r0+i of unit it
  template <bool TR, bool SCALE>
  __device__ __forceinline__ void commit_image(unsigned char* img, int tid, const float (*ws)[2]) const {
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int u = tid + it * NT;
      if (u >= UNITS) break;
      const int r0 = 2 * (u / PPR), f0 = (u % PPR) * EPP;
#pragma unroll
      for (int i = 0; i < 2; ++i)
        put_piece<T, DF, TR>(img, r0 + i, f0, SCALE ? scale_piece<T>(x[it][i], ws[it][i]) : x[it][i]);
    }
  }

  // fragment-order storage of the position-contracted operand (rows = features)
  template <bool SCALE>
  __device__ __forceinline__ void commit_frags(T* trf, int tid, const float (*ws)[2]) const {
    constexpr int NKS_C = (C + 31) / 32;
    typedef typename Pair<T>::type P2;
    const P2 zero2 = {};
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const int u = tid + it * NT;
      if (u >= UNITS) break;
      const int r0 = 2 * (u / PPR), f0 = (u % PPR) * EPP;
      const int k0 = r0 & 31, ks = r0 >> 5;
      const float w0 = SCALE ? ws[it][0] : 1.f, w1 = SCALE ? ws[it][1] : 1.f;
#pragma unroll
      for (int i = 0; i < EPP; ++i) {
        const int f = f0 + i;
        P2 p2;
        p2[0] = (T)(elemf<T>(x[it][0], i) * w0);
        p2[1] = (T)(elemf<T>(x[it][1], i) * w1);
        put_pair<T>(trf, (f >> 4) * NKS_C + ks, f & 15, k0, p2);
        if (C < 32) put_pair<T>(trf, (f >> 4) * NKS_C + ks, f & 15, k0 + 16, zero2);
      }
    }
  }
};

// lambda rows of one chunk (C*L contiguous floats) in registers: NF floats per thread, each
// loaded at a clamped in-bounds index (branch-free) and zeroed past the chunk's valid rows.
template <int C, int NT>
struct LamRegs {
  static constexpr int NF = (C * kLamCap + NT - 1) / NT;
  float x[NF];

  __device__ __forceinline__ void fetch(const float* __restrict__ g, int nvalid, int tid) {
#pragma unroll
    for (int it = 0; it < NF; ++it) {
      const int i = tid + it * NT;
      const float v = g[min(i, nvalid - 1)];
      x[it] = i < nvalid ? v : 0.f;
    }
  }

  __device__ __forceinline__ void commit(float* lam, int ntotal, int tid) const {
#pragma unroll
    for (int it = 0; it < NF; ++it) {
      const int i = tid + it * NT;
      if (i < ntotal) lam[i] = x[it];
    }
  }
};

// log_a of one chunk in every wave's registers (lane l holds positions E*l .. E*l+E-1), and
// the chunk-local inclusive prefix sum A (same layout), computed by each wave on its own.
template <int C>
struct DecayRegs {
  static constexpr int E = C > 64 ? C / 64 : 1;
  float x[E];
  float a[E];

  __device__ __forceinline__ void fetch(const float* __restrict__ la, int valid, int lane) {
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lane * E + e;
      const float v = la[min(i, valid - 1)];
      x[e] = (i < C && i < valid) ? v : 0.f;
    }
  }
  // fixed summation order: bitwise reproducible
  __device__ __forceinline__ void scan(int lane) {
    float run = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) { run += x[e]; a[e] = run; }
    float tot = run;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(tot, d, 64);
      if (lane >= d) tot += y;
    }
    const float excl = tot - run;
#pragma unroll
    for (int e = 0; e < E; ++e) a[e] += excl;
  }
  // A at chunk position r (all lanes of the wave must call it together)
  __device__ __forceinline__ float at(int r) const {
    if (E == 1) return __shfl(a[0], r, 64);
    const float lo = __shfl(a[0], r / E, 64);
    const float hi = __shfl(a[E - 1], r / E, 64);
    return (r % E) ? hi : lo;
  }
  // wave 0: publish A, e^A, e^-A and whether the factorised decay is safe (|A| < 40)
  __device__ __forceinline__ void publish(float* aloc, float* ea, float* eb, int* flag, int lane) const {
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int i = lane * E + e;
      if (i < C) {
        aloc[i] = a[e];
        ea[i] = __expf(a[e]);
        eb[i] = __expf(-a[e]);
        amax = fmaxf(amax, fabsf(a[e]));
      }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) amax = fmaxf(amax, __shfl_xor(amax, d, 64));
    if (lane == 0) *flag = amax < 40.f ? 1 : 0;
  }
};

// ----------------------------------------------------------------------------------------
// operand fragments from shared memory
// ----------------------------------------------------------------------------------------

template <typename T>
__device__ __forceinline__ Frag<T> lds_frag(const T* base, int slot, int lane) {
  return reinterpret_cast<const Frag<T>*>(base)[slot * 64 + lane];
}

template <typename T> __device__ __forceinline__ typename Quad<T>::type lds_quad(const unsigned char* p) {
  return *reinterpret_cast<const typename Quad<T>::type*>(p);
}

// Row-major operand fragment (rows = positions rb*16.., contraction = features 32s..32s+31)
template <typename T, int DF>
__device__ __forceinline__ Frag<T> row_frag(const unsigned char* img, int rb, int s, int lane) {
  typedef Img<T, DF, false> I;
  typedef typename Quad<T>::type Q4;
  const int r = 16 * rb + (lane & 15), g = lane >> 4;
  const int q0 = 8 * s + g, q1 = q0 + 4;
  const Q4 z = {};
  const Q4 lo = lds_quad<T>(img + I::off(r, q0));
  const Q4 hi = (q1 < I::NQ) ? lds_quad<T>(img + I::off(r, q1)) : z;
  Frag<T> f;
  if constexpr (sizeof(T) == 2) {
    f.v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  } else {
    f.lo = lo; f.hi = hi;
  }
  return f;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Position-contracted operand fragment (rows = features fb*16.., contraction = positions
// 32ks..32ks+31) from a row-major TR-swizzled bf16 image, by two transposing LDS reads:
// in each 16-lane group the read returns to lane i, element b, element i%4 of the quad read
// by lane 4b + i/4; so lane k of group g reads row 32ks + 16h + 4g + k/4, quad 4fb + k%4.
template <int C, int DF>
__device__ __forceinline__ Frag<bf16> tr_frag(const unsigned char* img, int fb, int ks, int lane) {
  typedef Img<bf16, DF, true> I;
  const int k = lane & 15, g = lane >> 4;
  const int q = 4 * fb + (k & 3);
  const int t0 = 32 * ks + 4 * g + (k >> 2);
  const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(img + I::off(t0, q)));
  s16x4 v1 = {0, 0, 0, 0};
  if (C >= 32)
    v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(img + I::off(t0 + 16, q)));
  Frag<bf16> f;
  f.v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
  return f;
}

// position-contracted operand: transposing read (bf16) or fragment-order slot (f32)
template <typename T, int C, int DF>
__device__ __forceinline__ Frag<T> col_frag(const unsigned char* base, int fb, int ks, int lane) {
  if constexpr (TrNative<T>::value) {
    return tr_frag<C, DF>(base, fb, ks, lane);
  } else {
    constexpr int NKS_C = (C + 31) / 32;
    return lds_frag<T>(reinterpret_cast<const T*>(base), fb * NKS_C + ks, lane);
  }
}

// ----------------------------------------------------------------------------------------
// per-wave building blocks
// ----------------------------------------------------------------------------------------

// Decayed chunk state for the wave's 16 value columns, as 16x16 tiles F[dk block]:
//   F = sum_{s in chunk} exp(gtot - A_s) k_s v_s^T   (the decay is already applied to k~)
template <typename T, int C, int DK>
__device__ __forceinline__ void chunk_state(const unsigned char* kt, const Frag<T> (&vfr)[(C + 31) / 32],
                                            int lane, f32x4 (&F)[DK / 16]) {
  constexpr int NKS_C = (C + 31) / 32;
  constexpr int NDKB = DK / 16;
#pragma unroll
  for (int b = 0; b < NDKB; ++b) F[b] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < NKS_C; ++ks) {
#pragma unroll
    for (int b = 0; b < NDKB; ++b) mma(F[b], col_frag<T, C, DK>(kt, b, ks, lane), vfr[ks]);
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
//   O[qb] += lambda[i, lev] * exp(A_i) * edoff * (N^T q_i)
// edoff = exp(log decay from the node's last position to the chunk's first position).
template <typename T, int C, int DK>
__device__ __forceinline__ void node_readout(const Frag<T> (&A)[(DK + 31) / 32], const unsigned char* qimg,
                                             const float* lam, int L, const float* ea,
                                             int lev, float edoff, int lane, f32x4 (&O)[C / 16]) {
  constexpr int NQB = C / 16;
  constexpr int NKS_D = (DK + 31) / 32;
  const int j = lane & 15;
  f32x4 Y[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) Y[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NKS_D; ++s) {
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) mma(Y[qb], A[s], row_frag<T, DK>(qimg, qb, s, lane));
  }
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qi = 16 * qb + j;
    O[qb] += (lam[qi * L + lev] * ea[qi] * edoff) * Y[qb];
  }
}

// Masked score unit (query block qb, key step ks): the two 16x16 score tiles of keys
// 32ks..32ks+31 against queries 16qb..16qb+15, masked by
//   lambda[i, bit_length(i ^ s)] * exp(A_i - A_s) for s <= i (chunk-local i, s), else 0,
// returned as the P^T operand fragment of the value product. exp(A_i - A_s) is taken as
// e^{A_i} e^{-A_s} when the chunk's |A| < 40 (`fact`), else directly.
template <typename T, int C, int DK>
__device__ __forceinline__ Frag<T> score_unit(const unsigned char* qimg, const unsigned char* kimg,
                                              const float* lam, int L, const float* aloc,
                                              const float* ea, const float* eb, bool fact,
                                              int qb, int ks, int lane) {
  constexpr int NKS_D = (DK + 31) / 32;
  const int j = lane & 15, g = lane >> 4;
  const int kb0 = 2 * ks, kb1 = 2 * ks + 1;
  const bool has1 = kb1 <= qb;
  f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NKS_D; ++s) {
    const Frag<T> bq = row_frag<T, DK>(qimg, qb, s, lane);
    mma(s0, row_frag<T, DK>(kimg, kb0, s, lane), bq);
    if (has1) mma(s1, row_frag<T, DK>(kimg, kb1, s, lane), bq);
  }
  const int qi = 16 * qb + j;
  const float* lrow = lam + qi * L;
  const int key0 = 16 * kb0 + 4 * g;
  f32x4 d0, d1;
  if (fact) {
    const float eq = ea[qi];
    d0 = eq * *reinterpret_cast<const f32x4*>(eb + key0);
    d1 = has1 ? eq * *reinterpret_cast<const f32x4*>(eb + key0 + 16) : f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    const float aq = aloc[qi];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      d0[r] = key0 + r <= qi ? __expf(aq - aloc[key0 + r]) : 0.f;
      d1[r] = (has1 && key0 + 16 + r <= qi) ? __expf(aq - aloc[min(key0 + 16 + r, C - 1)]) : 0.f;
    }
  }
  f32x4 p0, p1;
  if (kb0 < qb) {
    // whole tile below the diagonal: one level for the row
    const float lv = lrow[min(4 + bit_length((unsigned)(kb0 ^ qb)), L - 1)];
    p0 = (lv * s0) * d0;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + r;
      p0[r] = key <= qi ? s0[r] * lrow[min(bit_length((unsigned)(qi ^ key)), L - 1)] * d0[r] : 0.f;
    }
  }
  if (!has1) {
    p1 = f32x4{0.f, 0.f, 0.f, 0.f};
  } else if (kb1 < qb) {
    const float lv = lrow[min(4 + bit_length((unsigned)(kb1 ^ qb)), L - 1)];
    p1 = (lv * s1) * d1;
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = key0 + 16 + r;
      p1[r] = key <= qi ? s1[r] * lrow[min(bit_length((unsigned)(qi ^ key)), L - 1)] * d1[r] : 0.f;
    }
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

__device__ __forceinline__ void unit_decode(int un, int& qb, int& ks) {
  qb = 0;
  ks = un;
  while (ks >= qb / 2 + 1) { ks -= qb / 2 + 1; ++qb; }
}

// Stages one chunk: v as the position-contracted operand (P.V, states) and log_a -> (wave 0)
// A, e^A, e^-A; WITH_Q: q, k as row-major images (scores, read-outs) and lambda rows; KT:
// k~ = exp(g - A_s) k_s as position-contracted operand (chunk states).
template <typename T, int C, int DK, int DV, int NT, bool WITH_Q, bool KT>
struct ChunkStage {
  BlockRegs<T, C, DK, NT> qr, kr;
  BlockRegs<T, C, DV, NT> vr;
  LamRegs<C, NT> lr;
  DecayRegs<C> ar;

  __device__ __forceinline__ void fetch(const T* qg, const T* kg, const T* vg, const float* lamg,
                                        const float* lag, int L, int valid, int tid, int lane) {
    if (WITH_Q) {
      qr.fetch(qg, valid, tid);
      lr.fetch(lamg, valid * L, tid);
    }
    kr.fetch(kg, valid, tid);
    vr.fetch(vg, valid, tid);
    ar.fetch(lag, valid, lane);
  }

  __device__ __forceinline__ void commit(const ChunkSmem& S, unsigned char* smem, int L, int tid,
                                         int lane, int w) {
    ar.scan(lane);
    if (KT) {
      const float g = ar.at(C - 1);
      typedef BlockRegs<T, C, DK, NT> KR;
      float ws[KR::ITERS][2];
#pragma unroll
      for (int it = 0; it < KR::ITERS; ++it) {
        const int r0 = KR::row0(tid, it);
        ws[it][0] = __expf(g - ar.at(r0));
        ws[it][1] = __expf(g - ar.at(r0 + 1));
      }
      if constexpr (TrNative<T>::value)
        kr.template commit_image<true, true>(smem + S.kt, tid, ws);
      else
        kr.template commit_frags<true>(reinterpret_cast<T*>(smem + S.kt), tid, ws);
    }
    if (WITH_Q) {
      qr.template commit_image<false, false>(smem + S.qimg, tid, nullptr);
      kr.template commit_image<false, false>(smem + S.kimg, tid, nullptr);
      lr.commit(reinterpret_cast<float*>(smem + S.lam), C * L, tid);
    }
    if constexpr (TrNative<T>::value)
      vr.template commit_image<true, false>(smem + S.vt, tid, nullptr);
    else
      vr.template commit_frags<false>(reinterpret_cast<T*>(smem + S.vt), tid, nullptr);
    if (w == 0)
      ar.publish(reinterpret_cast<float*>(smem + S.aloc), reinterpret_cast<float*>(smem + S.ea),
                 reinterpret_cast<float*>(smem + S.eb), reinterpret_cast<int*>(smem + S.flag), lane);
  }
};

// ----------------------------------------------------------------------------------------
// kernels
// ----------------------------------------------------------------------------------------

// Node records pass between workgroups of one launch, possibly on different XCDs (each XCD has
// its own L2). Two schemes, chosen at compile time:
//   kScopedNodeIO = false: plain loads and stores of node data, an agent-scope release fence
//                          (L2 write-back) before the flag store and an agent-scope acquire
//                          fence (L2 invalidate) after the flag is seen;
//   kScopedNodeIO = true : node data is written and read with device-scope (sc1) buffer
//                          accesses, which are coherent across XCDs without touching the rest
//                          of L2; the flag is stored once those writes have completed.
#ifndef LLA_SCOPED_NODE_IO
#define LLA_SCOPED_NODE_IO 1
#endif
constexpr bool kScopedNodeIO = LLA_SCOPED_NODE_IO != 0;
constexpr int kCpolDevice = 16;   // cache-policy immediate: sc1 (device scope)

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Buffer descriptor over a wave-uniform base address (raw, unstrided).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t node_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7fffffff, 0x00020000);
}
// 16-byte multiples (an f32x4 tile quad, a bf16 or f32 operand fragment), contiguous at byte_off
template <typename V>
__device__ __forceinline__ V node_ld(const void* base, int byte_off) {
  static_assert(sizeof(V) % 16 == 0, "16-byte node accesses");
  if constexpr (kScopedNodeIO) {
    u32x4 r[sizeof(V) / 16];
#pragma unroll
    for (int i = 0; i < (int)(sizeof(V) / 16); ++i)
      r[i] = __builtin_amdgcn_raw_buffer_load_b128(node_rsrc(base), byte_off + 16 * i, 0, kCpolDevice);
    return __builtin_bit_cast(V, r);
  } else {
    return *reinterpret_cast<const V*>(reinterpret_cast<const char*>(base) + byte_off);
  }
}
template <typename V>
__device__ __forceinline__ void node_st(void* base, int byte_off, const V& x) {
  static_assert(sizeof(V) % 16 == 0, "16-byte node accesses");
  if constexpr (kScopedNodeIO) {
    struct W { u32x4 r[sizeof(V) / 16]; };
    const W wv = __builtin_bit_cast(W, x);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(V) / 16); ++i)
      __builtin_amdgcn_raw_buffer_store_b128(wv.r[i], node_rsrc(base), byte_off + 16 * i, 0, kCpolDevice);
  } else {
    *reinterpret_cast<V*>(reinterpret_cast<char*>(base) + byte_off) = x;
  }
}
__device__ __forceinline__ float node_ld_f(const float* p) {
  if constexpr (kScopedNodeIO) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
__device__ __forceinline__ void node_st_f(float* p, float x) {
  if constexpr (kScopedNodeIO) __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = x;
}
// after a wave's node writes, before its flag store
__device__ __forceinline__ void node_publish_fence() {
  if constexpr (kScopedNodeIO) {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0);     // every outstanding access of this wave has completed
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
  } else {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
  }
}
// after the flags a wave waits for were seen set, before its node reads
__device__ __forceinline__ void node_acquire_fence() {
  if constexpr (kScopedNodeIO) __atomic_signal_fence(__ATOMIC_SEQ_CST);
  else __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

constexpr int kFlagBase = 64;   // ints ahead of the node flags (the ticket counter, alone in its line)

struct Params {
  const void* q; const void* k; const void* v;
  const float* log_a; const float* lam;
  void* out;
  int BH, T, L;
  int nchunks;      // ceil(T / C)
  int sweep;        // R: consecutive chunks per workgroup (power of two, <= kSweepCap)
  int m;            // log2(R)
  int nsweep;       // ceil(nchunks / R)
  int* sync;        // [0]: workgroup ticket counter; [kFlagBase + (bh*ns + e)*NW + w]: node flags
  float* gnode;     // [BH][ns][NW]: log decay across node e (one copy per wave)
  float* node32;    // [BH][ns][NW][DK/16][64] f32x4: node e as float32 accumulator tiles
  void* nodeT;      // [BH][ns][NW][ceil(DK/32)][64] Frag<T>: node e as read-out operands
  int spin_limit;   // polls of a node flag before the wait is abandoned
};

// Node flags, data and decays are indexed by (head, node = sweep index e, wave).
__device__ __forceinline__ size_t node_slot(int bh, int ns, int e, int nw, int w) {
  return ((size_t)bh * ns + e) * nw + w;
}

// The forward pass. One workgroup per sweep of R chunks of one head, one wave per 16 value
// columns; ns = nsweep - 1 sweeps per head publish a node (the last one has no reader).
//
// Node of sweep e: the Fenwick node over sweeps that ends at e, i.e. the lowbit(e+1) sweeps
// (e - lowbit(e+1), e], decayed to the end of e:
//   node(e) = H_e + sum_{i < ctz(e+1)} exp(gacc_i) node(e - 2^i),
// H_e = sum_{s in sweep e} exp(A_end(e) - A_s) k_s v_s^T, gacc_i the log decay from the end of
// node(e - 2^i) to the end of e. Sweep sw reads the nodes ending at ((sw >> j) << j) - 1 for
// each set bit j of sw (level J + 1 + m + j); the first ctz(sw+1) of them are exactly the
// children of its own node.
//
// Global loads are issued branch-free where possible, so that waits count exactly: the
// inputs of the next chunk are loaded into registers right after the current chunk is staged
// in shared memory, and the first chunk of phase B while the last chunk of phase A is
// computed.
template <typename T, int C, int DK, int DV>
__global__ __launch_bounds__(4 * DV, 2) void lla_fused_kernel(Params p) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  constexpr int NT = 4 * DV, NW = DV / 16;
  constexpr int NQB = C / 16, NKS_C = (C + 31) / 32, NKS_D = (DK + 31) / 32, NDKB = DK / 16;
  constexpr int J = ilog2(C);
  constexpr int LMAX = ilog2(kSweepCap);
  constexpr int NSLOT = kSweepCap - 1;
  constexpr int NUNITS = num_units(NQB);
  constexpr int XREG = DK >= 128 ? 2 : 5;   // nodes over earlier sweeps held in registers
  static_assert(kSweepCap <= 4, "slot u of a sweep is the running total or chunk u alone only for R <= 4");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index: uniform
  const int j = lane & 15, g = lane >> 4;
  const int L = p.L, ns = p.nsweep - 1;
  const ChunkSmem SA = chunk_smem<T>(C, DK, DV, L, false, true);
  const ChunkSmem SB = chunk_smem<T>(C, DK, DV, L, true, false);

  // ticket -> (head, sweep), sweep-major
  int t = blockIdx.x;
  if (ns > 0) {
    int* tk = reinterpret_cast<int*>(smem + fused_ticket_offset<T>(C, DK, DV, L));
    if (tid == 0) *tk = __hip_atomic_fetch_add(p.sync, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    t = __builtin_amdgcn_readfirstlane(*tk);
  }
  const int sw = t / p.BH, bh = t - sw * p.BH;

  const size_t hoff = (size_t)bh * p.T;
  const T* qg = reinterpret_cast<const T*>(p.q) + hoff * DK;
  const T* kg = reinterpret_cast<const T*>(p.k) + hoff * DK;
  const T* vg = reinterpret_cast<const T*>(p.v) + hoff * DV;
  const float* lag = p.log_a + hoff;
  const float* lamg = p.lam + hoff * L;
  T* og = reinterpret_cast<T*>(p.out) + hoff * DV;

  const int c0 = sw * p.sweep;
  const int nch = min(p.sweep, p.nchunks - c0);
  const int next = __builtin_popcount((unsigned)sw);

  auto node_index = [&](int x) {      // sweep index the x-th node of sw ends at (0 if none)
    unsigned m = (unsigned)sw;
    for (int i = 0; i < x && m; ++i) m &= m - 1;
    return m ? ((sw >> __builtin_ctz(m)) << __builtin_ctz(m)) - 1 : 0;
  };
  auto node_level = [&](int x) {
    unsigned m = (unsigned)sw;
    for (int i = 0; i < x && m; ++i) m &= m - 1;
    return m ? J + 1 + p.m + __builtin_ctz(m) : 0;
  };
  const Frag<T>* ndT = reinterpret_cast<const Frag<T>*>(p.nodeT);
  auto load_node = [&](Frag<T> (&A)[NKS_D], int e) {
    const Frag<T>* base = ndT + node_slot(bh, ns, e, NW, w) * NKS_D * 64;
#pragma unroll
    for (int s = 0; s < NKS_D; ++s) A[s] = node_ld<Frag<T>>(base, (s * 64 + lane) * (int)sizeof(Frag<T>));
  };

  ChunkStage<T, C, DK, DV, NT, false, true> sa;
  ChunkStage<T, C, DK, DV, NT, true, false> sb;
  auto fetch_a = [&](int u) {
    const int t0 = (c0 + u) * C;
    const int valid = min(C, p.T - t0);
    sa.fetch(nullptr, kg + (size_t)t0 * DK, vg + (size_t)t0 * DV, nullptr, lag + t0, 0, valid, tid, lane);
  };
  auto fetch_b = [&](int u) {
    const int t0 = (c0 + u) * C;
    const int valid = min(C, p.T - t0);
    sb.fetch(qg + (size_t)t0 * DK, kg + (size_t)t0 * DK, vg + (size_t)t0 * DV, lamg + (size_t)t0 * L,
             lag + t0, L, valid, tid, lane);
  };

  // ---------------- phase A: chunk states -> slots inside the sweep, sweep total ----------------
  // Slot s (s < R-1) is the Fenwick node over the chunks of the sweep that ends at chunk s; for
  // R <= 4 it is the running total when s+1 is a power of two and chunk s's own state otherwise.
  Frag<T> SL[NSLOT][NKS_D];
#pragma unroll
  for (int s = 0; s < NSLOT; ++s)
#pragma unroll
    for (int s2 = 0; s2 < NKS_D; ++s2) SL[s][s2] = zero_frag<T>();
  f32x4 H[NDKB];
#pragma unroll
  for (int b = 0; b < NDKB; ++b) H[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  float G = 0.f;
  auto body_a = [&](int u) {
    const float gtot = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(
        __builtin_bit_cast(int, reinterpret_cast<const float*>(smem + SA.aloc)[C - 1])));
    Frag<T> vfr[NKS_C];
#pragma unroll
    for (int ks = 0; ks < NKS_C; ++ks) vfr[ks] = col_frag<T, C, DV>(smem + SA.vt, w, ks, lane);
    f32x4 F[NDKB];
    chunk_state<T, C, DK>(smem + SA.kt, vfr, lane, F);
    const float d = __expf(gtot);
#pragma unroll
    for (int b = 0; b < NDKB; ++b) H[b] = d * H[b] + F[b];
    G += gtot;
    // value selects, not conditional stores: the slots must stay in registers
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
      const bool hit = u == s;
      const bool whole = ((s + 1) & s) == 0;
#pragma unroll
      for (int s2 = 0; s2 < NKS_D; ++s2)
        SL[s][s2] = frag_select<T>(hit, whole ? node_frag<T, DK>(H, s2) : node_frag<T, DK>(F, s2), SL[s][s2]);
    }
  };
  fetch_a(0);
  for (int u = 0; u + 1 < nch; ++u) {
    if (u) __syncthreads();
    sa.commit(SA, smem, L, tid, lane, w);
    __syncthreads();
    fetch_a(u + 1);
    body_a(u);
  }
  if (nch > 1) __syncthreads();
  sa.commit(SA, smem, L, tid, lane, w);
  __syncthreads();
  fetch_b(0);
  body_a(nch - 1);

  // ---------------- nodes of earlier sweeps: wait, absorb children, publish ----------------
  bool bad = false;
  for (int x = 0; x < next; ++x) {
    const int* f = p.sync + kFlagBase + node_slot(bh, ns, node_index(x), NW, w);
    int n = 0;
    while (__hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
      if (++n > p.spin_limit) { bad = true; break; }
      __builtin_amdgcn_s_sleep(2);
    }
  }
  if (next > 0) node_acquire_fence();

  if (sw < ns) {
    const int kc = __builtin_ctz((unsigned)(sw + 1));   // children: nodes x < kc of sw
    const f32x4* n32 = reinterpret_cast<const f32x4*>(p.node32);
    float gacc = G;
    for (int x = 0; x < kc; ++x) {
      const size_t e = node_slot(bh, ns, node_index(x), NW, w);
      const float d = __expf(gacc);
#pragma unroll
      for (int b = 0; b < NDKB; ++b) H[b] += d * node_ld<f32x4>(n32 + e * NDKB * 64, (b * 64 + lane) * 16);
      gacc += node_ld_f(p.gnode + e);
    }
    if (bad) {
#pragma unroll
      for (int b = 0; b < NDKB; ++b) H[b] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
    }
    const size_t me = node_slot(bh, ns, sw, NW, w);
    f32x4* o32 = reinterpret_cast<f32x4*>(p.node32) + me * NDKB * 64;
#pragma unroll
    for (int b = 0; b < NDKB; ++b) node_st<f32x4>(o32, (b * 64 + lane) * 16, H[b]);
    Frag<T>* oT = reinterpret_cast<Frag<T>*>(p.nodeT) + me * NKS_D * 64;
#pragma unroll
    for (int s = 0; s < NKS_D; ++s) node_st<Frag<T>>(oT, (s * 64 + lane) * (int)sizeof(Frag<T>), node_frag<T, DK>(H, s));
    if (lane == 0) node_st_f(p.gnode + me, gacc);
    node_publish_fence();
    if (lane == 0) __hip_atomic_store(p.sync + kFlagBase + me, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  Frag<T> X[XREG][NKS_D];
  float XD[XREG];            // log decay across each node
  if (ns > 0) {
#pragma unroll
    for (int x = 0; x < XREG; ++x) {
      const int e = node_index(x);
      load_node(X[x], e);
      XD[x] = node_ld_f(p.gnode + node_slot(bh, ns, e, NW, w));
    }
  }

  // ---------------- phase B: outputs, chunk by chunk ----------------
  const unsigned char* qimg = smem + SB.qimg;
  const unsigned char* kimg = smem + SB.kimg;
  T* pf = reinterpret_cast<T*>(smem + SB.pf);
  const float* lam = reinterpret_cast<const float*>(smem + SB.lam);
  const float* aloc = reinterpret_cast<const float*>(smem + SB.aloc);
  const float* ea = reinterpret_cast<const float*>(smem + SB.ea);
  const float* eb = reinterpret_cast<const float*>(smem + SB.eb);
  const int* flag = reinterpret_cast<const int*>(smem + SB.flag);

  float SD[NSLOT];           // log decay from the end of slot s to the current chunk start
#pragma unroll
  for (int s = 0; s < NSLOT; ++s) SD[s] = 0.f;
  float gam = 0.f;           // log decay from the sweep's first position to the current chunk start

  for (int u = 0; u < nch; ++u) {
    const int t0 = (c0 + u) * C;
    const int valid = min(C, p.T - t0);
    __syncthreads();
    sb.commit(SB, smem, L, tid, lane, w);
    __syncthreads();
    fetch_b(u + 1 < nch ? u + 1 : u);     // unconditional: re-reads this chunk after the last
    const float gtot = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, aloc[C - 1])));
    const bool fact = __builtin_amdgcn_readfirstlane(*flag) != 0;

    // masked scores -> P^T fragments
    for (int un = w; un < NUNITS; un += NW) {
      int qb, ks;
      unit_decode(un, qb, ks);
      const Frag<T> f = score_unit<T, C, DK>(qimg, kimg, lam, L, aloc, ea, eb, fact, qb, ks, lane);
      reinterpret_cast<Frag<T>*>(pf)[(qb * NKS_C + ks) * 64 + lane] = f;
    }
    __syncthreads();

    // intra-chunk values
    Frag<T> vfr[NKS_C];
#pragma unroll
    for (int ks = 0; ks < NKS_C; ++ks) vfr[ks] = col_frag<T, C, DV>(smem + SB.vt, w, ks, lane);
    f32x4 O[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      O[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks <= qb / 2; ++ks) mma(O[qb], vfr[ks], lds_frag<T>(pf, qb * NKS_C + ks, lane));
    }

    // Fenwick nodes inside the sweep (levels J+1 .. J+m): chunk u reads slot ((u>>a)<<a) - 1
    // for each set bit a of u
#pragma unroll
    for (int s = 0; s < NSLOT; ++s) {
#pragma unroll
      for (int a = 0; a < LMAX; ++a) {
        if (((u >> a) & 1) && ((u >> a) << a) - 1 == s)
          node_readout<T, C, DK>(SL[s], qimg, lam, L, ea, J + 1 + a, __expf(SD[s]), lane, O);
      }
    }

    // Fenwick nodes made of whole earlier sweeps (levels J+m+1 ..), lowest bit first
    {
      float dext = 0.f;
#pragma unroll
      for (int x = 0; x < XREG; ++x) {
        if (x < next) {
          node_readout<T, C, DK>(X[x], qimg, lam, L, ea, node_level(x), __expf(gam + dext), lane, O);
          dext += XD[x];
        }
      }
      for (int x = XREG; x < next; ++x) {    // beyond the register budget: load on demand
        Frag<T> A[NKS_D];
        const int e = node_index(x);
        load_node(A, e);
        node_readout<T, C, DK>(A, qimg, lam, L, ea, node_level(x), __expf(gam + dext), lane, O);
        dext += node_ld_f(p.gnode + node_slot(bh, ns, e, NW, w));
      }
    }
    // store rows [0, valid); NaN if a node never arrived
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      const int qi = 16 * qb + j;
      if (bad) O[qb] = f32x4{__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""), __builtin_nanf("")};
      if (qi < valid) store_quad<T>(og + (size_t)(t0 + qi) * DV + 16 * w + 4 * g, O[qb]);
    }
#pragma unroll
    for (int s = 0; s < NSLOT; ++s)
      if (s < u) SD[s] += gtot;
    gam += gtot;
  }
}

}  // namespace lla
