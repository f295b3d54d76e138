// lla_gdn.hpp — gfx950 kernels of the chunkwise forward pass of log-linear Gated DeltaNet.
//
// Operation, per (b,h) and position t (Gated DeltaNet's attention matrix under the Fenwick
// hierarchical mask; the model's own transition carries every level state — study notes,
// section 3-5; gist.science de technical summary, "Kernidee" and "Anwendung auf bestehende
// Modelle"; zh technical summary, section 2.4):
//   o_t = sum_{s<=t} lambda[t, l(t,s)] beta_s q_t^T A_t ... A_{s+1} k_s v_s,
//   A_r = a_r (I - beta_r k_r k_r^T),  a_r = exp(log_a[r]),  l(t,s) = bit_length(t ^ s).
//
// Chunk structure (chunk C = 2^J, local positions i, j; a_i = chunk-local inclusive prefix of
// log_a, g = a_{C-1}, Gam[i,j] = exp(a_i - a_j)). With Tm = I + strict_lower(diag(beta)(K K^T *
// Gam)) (the delta rule inside the chunk in its triangular, "UT" form):
//   W = Tm^{-1} diag(beta e^a) K,  U = Tm^{-1} diag(beta) V
//   intra-chunk:  O_intra = ((Lqk Tm^{-1} diag(beta)) * Lambda) V,  Lqk = (Q K^T * Gam) on j <= i
//                 ((Lqk Tm^{-1} diag(beta))[i,j] = beta_j q_i^T A_i..A_{j+1} k_j, the attention
//                 matrix inside the chunk);
//   transport of a query to the chunk start: X0 = diag(e^a) Q - Lqk W
//                 (row i is q_i^T A_i ... A_{c0}, c0 the chunk's first position);
//   the chunk as a Fenwick leaf: its state N = Khat^T U and its transition Phi = e^g I - Khat^T W,
//                 Khat = diag(e^{g-a}) K (the chunk's inputs, and A over the whole chunk).
// Fenwick nodes over chunks (level j, block m of 2^j chunks): N(j,m) = Phi_R N_L + N_R and
// Phi(j,m) = Phi_R Phi_L (children L = (j-1, 2m), R = (j-1, 2m+1)). Chunk c reads, for each set
// bit j of c from the lowest, the node (j, (c >> j) - 1) at level J+1+j with X the query rows
// carried to that node's end: O += lambda[:, J+1+j] * (X N), then X <- X Phi of that node.
//
// Kernels (stream order): gdn_chunk (one workgroup per chunk and head), the up-sweep (for
// dk <= 64 gdn_upsweep2, two tree levels per launch, one workgroup per node of the upper level
// and head, and a last odd level's even nodes on their own; at dk = 128 gdn_upsweep, one launch
// per level with workgroups over node and head or over node, head and a 16-column panel),
// gdn_query (one workgroup per chunk and head). Products run on the matrix cores from shared
// memory, in float32 — except, for bfloat16 inputs, K K^T and Q K^T of gdn_chunk on bf16
// operands (exact) and, with dk >= 32, gdn_query's and gdn_upsweep2's in split bf16 (high and
// low parts, three bf16 products); Tm^{-1} is formed blockwise (16 x 16 diagonal blocks by
// forward substitution, then doubled); inputs may be bfloat16 or float32, the output is in their
// type.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lla {
namespace gdn {

typedef __bf16 bf16;
constexpr int kNT = 256;          // threads per workgroup
constexpr int kLamCapG = 24;      // lambda levels held per position (T <= 2^23)

struct GdnParams {
  const void* q; const void* k; const void* v;
  const float* log_a; const float* beta; const void* lam;
  void* out;
  int lam_bf16;
  int BH, T, L;
  int nchunks;      // ceil(T / C)
  int nslot;        // tree slots per head: sum over levels j of (nchunks >> j)
  float* oi;        // [BH][nchunks*C][DV]: intra-chunk outputs
  float* x0;        // [BH][nchunks*C][DK]: query rows carried to their chunk's start
  float* node;      // [BH][nslot][DK][DV]: Fenwick node states
  float* phi;       // [BH][nslot][DK][DK]: Fenwick node transitions
  int level;        // up-sweep: the level being built (>= 1)
  int off_prev;     // up-sweep: first slot of level-1
  int off_cur;      // up-sweep: first slot of level
  int off_next;     // up-sweep of two levels: first slot of level + 1
  int ncur;         // up-sweep: nodes at level (nchunks >> level)
  int two;          // gdn_upsweep2: 1 = levels level and level + 1; 0 = level's even nodes only
};

__device__ __forceinline__ int bit_length(unsigned x) { return 32 - __clz((int)x); }

template <typename T> __device__ __forceinline__ float to_f(T x) { return (float)x; }

__device__ __forceinline__ float lambda_at(const GdnParams& p, size_t i) {
  if (p.lam_bf16) {
    const unsigned short b = reinterpret_cast<const unsigned short*>(p.lam)[i];
    return __builtin_bit_cast(float, (unsigned)b << 16);
  }
  return reinterpret_cast<const float*>(p.lam)[i];
}

// Tree nodes in the workspace: float32 matrices, or, for bfloat16 inputs with 32 <= dk <= 64 (where
// every product that reads them runs in split bf16), each slot's matrix as its high bf16 parts
// followed by its low parts (the same 4 bytes per element), copied into the split-bf16 images
// without conversion.
template <typename T, int DK>
constexpr bool nodes_split() { return std::is_same<T, bf16>::value && DK >= 32 && DK <= 64; }
// element i of an n-element matrix stored at `at` as its high parts, then its low parts
__device__ __forceinline__ void put_split(float* at, int n, int i, float x) {
  bf16* h = reinterpret_cast<bf16*>(at);
  const bf16 hi = (bf16)x;
  h[i] = hi;
  h[n + i] = (bf16)(x - (float)hi);
}

// out(i, j) = sum_k A(i, k) B(k, j) for an M x N output over a K-long contraction, operands in
// shared memory (float32): A(i, k) = TA ? A[k*lda + i] : A[i*lda + k], B(k, j) = TB ?
// B[j*ldb + k] : B[k*ldb + j], times kscale[k] when kscale is given. On the matrix cores in
// float32 (v_mfma_f32_16x16x4_f32): 16 x 16 output tiles dealt to the waves in turn; per step,
// lane (j, g) (j = lane % 16, g = lane / 16) supplies A(16ti + j, k + g) and B(k + g, 16tj + j),
// and the accumulator gives it rows 16ti + 4g .. +3 of column 16tj + j. Every output value is
// handed once to epi(i, j, value).
template <int M, int N, int K, bool TA, bool TB, typename AT, typename BT, typename Epi>
__device__ __forceinline__ void gemm_f32(const AT* A, int lda, const BT* B, int ldb, int tid,
                                         Epi&& epi, const float* kscale = nullptr) {
  static_assert(M % 16 == 0 && N % 16 == 0 && K % 4 == 0, "16 x 16 tiles, 4-deep steps");
  constexpr int TN = N / 16, NTILE = (M / 16) * TN, NWAVE = kNT / 64;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int j = lane & 15, g = lane >> 4;
  for (int tile = w; tile < NTILE; tile += NWAVE) {
    const int i0 = (tile / TN) * 16, j0 = (tile % TN) * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
    for (int k = 0; k < K; k += 4) {
      const int kk = k + g;
      const float a = to_f(TA ? A[kk * lda + i0 + j] : A[(i0 + j) * lda + kk]);
      float b = to_f(TB ? B[(j0 + j) * ldb + kk] : B[kk * ldb + j0 + j]);
      if (kscale) b *= kscale[kk];
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) epi(i0 + 4 * g + r, j0 + j, acc[r]);
  }
}

// Split-bf16 products (bfloat16 inputs): a float32 operand x is held as hi = bf16(x) and
// lo = bf16(x - hi) (~16 mantissa bits), and a product as hi*hi + hi*lo + lo*hi on the bf16
// matrix cores (v_mfma_f32_16x16x32_bf16, K = 32 per step), the dropped lo*lo term about 2^-16 of
// it: float32-grade sums at a fraction of the float32 products' cost.
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4g __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4g lds_s16x4g;

// A(i, k..k+7): row i of a row-major bf16 image, 8 consecutive contraction elements
__device__ __forceinline__ bf16x8 frag_rows(const bf16* img, int ld, int i, int k) {
  return *reinterpret_cast<const bf16x8*>(img + i * ld + k);
}
// B(k..k+7, n): column n of a row-major bf16 image over 8 consecutive rows, by two transposing
// reads (ds_read_b64_tr_b16: lane L of a 16-lane group addresses row k + L/4, columns
// n0 + 4 (L % 4) .. + 3, and receives column n0 + L of rows k .. k + 3)
__device__ __forceinline__ bf16x8 frag_cols(const bf16* img, int ld, int k, int n) {
  const int L = n & 15, n0 = n - L;
  const bf16* q = img + (k + (L >> 2)) * ld + n0 + 4 * (L & 3);
  const s16x4g a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4g*)q);
  const s16x4g b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4g*)(q + 4 * ld));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Node images 64 elements wide (128-byte rows, no padding) with their 32-byte windows permuted
// per row: window w of row r sits at w ^ swz_win(r). A transposing read takes 32-byte pieces of
// rows k + {0..3} + 8g; the permutation (row bits 1 and 3) sends the even and the odd ones of
// every 8 rows that one pass serves to 4 different windows, so they meet no bank twice (padded
// 144-byte rows gave those rows overlapping banks).
__device__ __forceinline__ int swz_win(int r) { return ((r >> 1) & 1) | (((r >> 3) & 1) << 1); }
__device__ __forceinline__ int swz_col(int r, int col) { return col ^ (swz_win(r) << 4); }
__device__ __forceinline__ bf16x8 frag_cols_sw(const bf16* img, int k, int n) {
  constexpr int ld = 64;
  const int L = n & 15, n0 = n - L, r = k + (L >> 2), col = n0 + 4 * (L & 3);
  const s16x4g a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4g*)(img + r * ld + swz_col(r, col)));
  const s16x4g b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4g*)(img + (r + 4) * ld + swz_col(r + 4, col)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
template <bool SW>
__device__ __forceinline__ bf16x8 frag_cols_b(const bf16* img, int ld, int k, int n) {
  if constexpr (SW) return frag_cols_sw(img, k, n);
  else return frag_cols(img, ld, k, n);
}

// out(i, j) = sum_k A(i, k) B(k, j) over an M x N output and a K-long contraction, A and B
// row-major in shared memory as high and low bf16 images (row strides lda, ldb elements, each a
// multiple of 8); 16 x 16 tiles dealt to the waves in turn, the epilogue as gemm_f32's
template <int M, int N, int K, bool SWB = false, typename Epi>
__device__ __forceinline__ void gemm_bf3(const bf16* Ah, const bf16* Al, int lda, const bf16* Bh,
                                         const bf16* Bl, int ldb, int tid, Epi&& epi) {
  static_assert(M % 16 == 0 && N % 16 == 0 && K % 32 == 0, "16 x 16 tiles, 32-deep steps");
  constexpr int TN = N / 16, NTILE = (M / 16) * TN, NWAVE = kNT / 64;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int j = lane & 15, g = lane >> 4;
  for (int tile = w; tile < NTILE; tile += NWAVE) {
    const int i0 = (tile / TN) * 16, j0 = (tile % TN) * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; k += 32) {
      const bf16x8 ah = frag_rows(Ah, lda, i0 + j, k + 8 * g), al = frag_rows(Al, lda, i0 + j, k + 8 * g);
      const bf16x8 bh = frag_cols_b<SWB>(Bh, ldb, k + 8 * g, j0 + j), bl = frag_cols_b<SWB>(Bl, ldb, k + 8 * g, j0 + j);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) epi(i0 + 4 * g + r, j0 + j, acc[r]);
  }
}

// out(i, j) = sum_k A(i, k) B(j, k) for operands whose values are bf16 (inputs): A and B row-major
// bf16 images in shared memory, one v_mfma_f32_16x16x32_bf16 per 32-deep step (products exact,
// sums in float32); tiles and epilogue as gemm_bf3's
template <int M, int N, int K, typename Epi>
__device__ __forceinline__ void gemm_bf1_nt(const bf16* A, int lda, const bf16* B, int ldb, int tid, Epi&& epi) {
  static_assert(M % 16 == 0 && N % 16 == 0 && K % 32 == 0, "16 x 16 tiles, 32-deep steps");
  constexpr int TN = N / 16, NTILE = (M / 16) * TN, NWAVE = kNT / 64;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int j = lane & 15, g = lane >> 4;
  for (int tile = w; tile < NTILE; tile += NWAVE) {
    const int i0 = (tile / TN) * 16, j0 = (tile % TN) * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; k += 32)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(frag_rows(A, lda, i0 + j, k + 8 * g),
                                                    frag_rows(B, ldb, j0 + j, k + 8 * g), acc, 0, 0, 0);
#pragma unroll
    for (int r = 0; r < 4; ++r) epi(i0 + 4 * g + r, j0 + j, acc[r]);
  }
}

// out(i, j) = sum_k A(k, i) B(k, j): A an exact-bf16 row-major image read transposed (its columns
// by the transposing reads), B as high and low bf16 images, row-major; A has no low part, so a
// 32-deep step is two v_mfma_f32_16x16x32_bf16 (A hi + A lo). Tiles and epilogue as gemm_bf3's.
template <int M, int N, int K, typename Epi>
__device__ __forceinline__ void gemm_bf2_tn(const bf16* A, int lda, const bf16* Bh, const bf16* Bl, int ldb,
                                            int tid, Epi&& epi) {
  static_assert(M % 16 == 0 && N % 16 == 0 && K % 32 == 0, "16 x 16 tiles, 32-deep steps");
  constexpr int TN = N / 16, NTILE = (M / 16) * TN, NWAVE = kNT / 64;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int j = lane & 15, g = lane >> 4;
  for (int tile = w; tile < NTILE; tile += NWAVE) {
    const int i0 = (tile / TN) * 16, j0 = (tile % TN) * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; k += 32) {
      const bf16x8 a = frag_cols(A, lda, k + 8 * g, i0 + j);
      const bf16x8 bh = frag_cols(Bh, ldb, k + 8 * g, j0 + j), bl = frag_cols(Bl, ldb, k + 8 * g, j0 + j);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bl, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) epi(i0 + 4 * g + r, j0 + j, acc[r]);
  }
}

// out(i, j) = sum_k A(i, k) B(k, j): A row-major as high and low bf16 images, B an exact-bf16
// row-major image; two v_mfma_f32_16x16x32_bf16 per 32-deep step (A hi + A lo against B), tiles
// and epilogue as gemm_bf3's
template <int M, int N, int K, typename Epi>
__device__ __forceinline__ void gemm_bf2_nn(const bf16* Ah, const bf16* Al, int lda, const bf16* B, int ldb,
                                            int tid, Epi&& epi) {
  static_assert(M % 16 == 0 && N % 16 == 0 && K % 32 == 0, "16 x 16 tiles, 32-deep steps");
  constexpr int TN = N / 16, NTILE = (M / 16) * TN, NWAVE = kNT / 64;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int j = lane & 15, g = lane >> 4;
  for (int tile = w; tile < NTILE; tile += NWAVE) {
    const int i0 = (tile / TN) * 16, j0 = (tile % TN) * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; k += 32) {
      const bf16x8 ah = frag_rows(Ah, lda, i0 + j, k + 8 * g), al = frag_rows(Al, lda, i0 + j, k + 8 * g);
      const bf16x8 b = frag_cols(B, ldb, k + 8 * g, j0 + j);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, b, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, b, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) epi(i0 + 4 * g + r, j0 + j, acc[r]);
  }
}

// gemm_bf3 with the epilogue told the tile's place among the wave's (t < gemm_tiles_per_wave) and
// the accumulator row r, so that a caller can keep the outputs in registers across products
template <int M, int N>
constexpr int gemm_tiles_per_wave() { return ((M / 16) * (N / 16) + kNT / 64 - 1) / (kNT / 64); }
template <int M, int N, int K, bool SWB = false, typename Epi>
__device__ __forceinline__ void gemm_bf3_t(const bf16* Ah, const bf16* Al, int lda, const bf16* Bh,
                                           const bf16* Bl, int ldb, int tid, Epi&& epi) {
  static_assert(M % 16 == 0 && N % 16 == 0 && K % 32 == 0, "16 x 16 tiles, 32-deep steps");
  constexpr int TN = N / 16, NTILE = (M / 16) * TN, NWAVE = kNT / 64, PERW = gemm_tiles_per_wave<M, N>();
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int j = lane & 15, g = lane >> 4;
#pragma unroll
  for (int t = 0; t < PERW; ++t) {
    const int tile = w + t * NWAVE;
    if (tile >= NTILE) break;
    const int i0 = (tile / TN) * 16, j0 = (tile % TN) * 16;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < K; k += 32) {
      const bf16x8 ah = frag_rows(Ah, lda, i0 + j, k + 8 * g), al = frag_rows(Al, lda, i0 + j, k + 8 * g);
      const bf16x8 bh = frag_cols_b<SWB>(Bh, ldb, k + 8 * g, j0 + j), bl = frag_cols_b<SWB>(Bl, ldb, k + 8 * g, j0 + j);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) epi(t, r, i0 + 4 * g + r, j0 + j, acc[r]);
  }
}

// An R x CC row-major block (source row stride src_ld elements) on its way into shared-memory
// floats dst[r * ldd + c], rows at or past nv read as zeros: load() issues the thread's 16-byte
// vector loads into registers, store() converts and writes them. Several blocks loaded before
// any is stored cost one memory round trip together.
template <typename T, int R, int CC>
struct StagedBlock {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  static constexpr int EPV = 16 / (int)sizeof(T), VPR = CC / EPV, NVEC = R * VPR;
  static constexpr int PER = (NVEC + kNT - 1) / kNT;
  static_assert(CC % EPV == 0, "whole 16-byte vectors per row");
  u32x4 buf[PER];

  __device__ __forceinline__ void load(const T* src, size_t src_ld, int nv, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * kNT, r = v / VPR;
      buf[i] = u32x4{0u, 0u, 0u, 0u};
      if (v < NVEC && r < nv) buf[i] = *reinterpret_cast<const u32x4*>(src + (size_t)r * src_ld + (v % VPR) * EPV);
    }
  }
  // float32 blocks only: each element as high and low bf16 parts into two images
  __device__ __forceinline__ void store_split(bf16* hi, bf16* lo, int ldd, int tid) const {
    static_assert(sizeof(T) == 4, "float32 sources");
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * kNT;
      if (v >= NVEC) break;
      const int at = (v / VPR) * ldd + (v % VPR) * EPV;
      unsigned hw[2], lw[2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const unsigned word = buf[i][e];
        const float x = __builtin_bit_cast(float, word);
        const bf16 h = (bf16)x;
        const unsigned hb = __builtin_bit_cast(unsigned short, h);
        const unsigned lb = __builtin_bit_cast(unsigned short, (bf16)(x - (float)h));
        if (e & 1) { hw[e / 2] |= hb << 16; lw[e / 2] |= lb << 16; }
        else { hw[e / 2] = hb; lw[e / 2] = lb; }
      }
      typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
      *reinterpret_cast<u32x2*>(hi + at) = u32x2{hw[0], hw[1]};
      *reinterpret_cast<u32x2*>(lo + at) = u32x2{lw[0], lw[1]};
    }
  }
  // bf16 blocks only: the vectors as they are into a bf16 image (row stride ldd, a multiple of 8)
  __device__ __forceinline__ void store_raw(bf16* dst, int ldd, int tid) const {
    static_assert(sizeof(T) == 2, "bf16 sources");
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * kNT;
      if (v >= NVEC) break;
      *reinterpret_cast<u32x4*>(dst + (v / VPR) * ldd + (v % VPR) * EPV) = buf[i];
    }
  }
  // bf16 blocks only: into a 64-wide node image with the 32-byte windows permuted per row
  // (swz_col)
  __device__ __forceinline__ void store_raw_sw(bf16* dst, int tid) const {
    static_assert(sizeof(T) == 2 && CC <= 64, "bf16 sources, rows within the 64-wide image");
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * kNT;
      if (v >= NVEC) break;
      const int r = v / VPR;
      *reinterpret_cast<u32x4*>(dst + r * 64 + swz_col(r, (v % VPR) * EPV)) = buf[i];
    }
  }
  __device__ __forceinline__ void store(float* dst, int ldd, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int v = tid + i * kNT;
      if (v >= NVEC) break;
      float* d = dst + (v / VPR) * ldd + (v % VPR) * EPV;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        // the element is copied to a scalar first: a bit cast applied to the vector element
        // itself compiles to a read of element 0 whatever e is
        const unsigned word = buf[i][e];
        if constexpr (sizeof(T) == 4) {
          d[e] = __builtin_bit_cast(float, word);
        } else {
          d[2 * e] = __builtin_bit_cast(float, word << 16);
          d[2 * e + 1] = __builtin_bit_cast(float, word & 0xffff0000u);
        }
      }
    }
  }
};

template <typename T, int R, int CC>
__device__ __forceinline__ void stage_block(float* dst, int ldd, const T* src, size_t src_ld, int nv, int tid) {
  StagedBlock<T, R, CC> b;
  b.load(src, src_ld, nv, tid);
  b.store(dst, ldd, tid);
}

// levels L0 .. L0 + LW - 1 of the lambda rows of positions [row0, row0 + C), bound for
// lam[r * LW + l - L0] (rows past nv and levels past L are zero weights), loaded and stored like
// StagedBlock
template <int C, int LW = kLamCapG, int L0 = 0>
struct StagedLambda {
  static constexpr int PER = (C * LW + kNT - 1) / kNT;
  float buf[PER];
  __device__ __forceinline__ void load(const GdnParams& p, size_t row0, int nv, int tid) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * kNT, r = idx / LW, l = L0 + idx % LW;
      buf[i] = (idx < C * LW && r < nv && l < p.L) ? lambda_at(p, (row0 + r) * p.L + l) : 0.f;
    }
  }
  __device__ __forceinline__ void store(float* lam, int tid) const {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int idx = tid + i * kNT;
      if (idx < C * LW) lam[idx] = buf[i];
    }
  }
};

// Shared-memory bytes of the three kernels (host and device agree; the host refuses shapes past
// 160 KB).
// gdn_chunk reads the in-chunk lambda levels only (bit_length(i ^ j) <= log2 C)
__host__ __device__ constexpr int chunk_lw(int C) { return C == 16 ? 5 : C == 32 ? 6 : 7; }
// QB: bfloat16 inputs keep q and k as bf16 images (rows padded by 8 elements; their values are
// exact in bf16, and K K^T, Q K^T run on the bf16 matrix cores), and Khat then takes the float32
// buffers of Lqk and Tm^{-1} (free by then) where they hold it: at chunk 32 and d = 64, 57.6 ->
// 46.8 KB, three workgroups per compute unit instead of two
__host__ __device__ constexpr bool chunk_qb(bool bf, int C, int DK) { return bf && 2 * (C + 1) >= DK + 1 && DK % 32 == 0; }
// LB (QB with chunks of 32 or 64): the leaf's products run on the bf16 matrix cores. Since
// Khat = diag(e^{g-a}) K, the row scale moves onto U and W (U' = diag(e^{g-a}) U, W'' likewise),
// K^T stays exact in bf16, U' and W'' are held as high and low bf16 images (rows padded by 8), and
// each 32-deep step is K^T hi + K^T lo: two v_mfma_f32_16x16x32_bf16 instead of eight float32 steps.
// U' takes U's buffer (grown to C (dv + 8) floats), W'' the buffers of q (low parts) and Lqk
// (high parts), free by then. v is then kept as a bf16 image too, and the in-chunk attention
// matrix as high and low bf16 images (its product with v: two bf16 steps per 32, v exact).
__host__ __device__ constexpr bool chunk_lb(bool bf, int C, int DK) { return chunk_qb(bf, C, DK) && C % 32 == 0; }
__host__ __device__ constexpr int chunk_smem_bytes(int C, int DK, int DV, bool bf = false) {
  return 4 * ((chunk_qb(bf, C, DK) ? C * (DK + 8) : 2 * C * (DK + 1)) +
              (chunk_lb(bf, C, DK) ? C * (DV + 8) / 2 + C * (C + 8) + 2 * C * (C + 1)
                                   : C * (DV + 1) + 3 * C * (C + 1)) +
              C * (DK + 1) + (chunk_lb(bf, C, DK) ? C * (DV + 8) : C * (DV + 1)) + C * chunk_lw(C) + 3 * C);
}
// up-sweep panel width: the whole [N | Phi] row (WHOLE: one workgroup per node, the right
// child's transition read once; for dk <= 64, at levels with enough nodes to fill the device) or
// 16 columns (more, shorter workgroups, each reading the transition again)
__host__ __device__ constexpr int up_panel(int DK, int DV, bool whole) { return whole ? DV + DK : 16; }
__host__ __device__ constexpr int up_smem_bytes(int DK, int DV, bool whole) {
  return 4 * (DK * (DK + 1) + DK * (up_panel(DK, DV, whole) + 1));
}
// the two-level up-sweep: one transition and one whole [N | Phi] row block, in float32 or (BF3)
// as high and low bf16 images with rows padded by 8 elements
__host__ __device__ constexpr int up2_smem_bytes(int DK, int DV, bool bf3) {
  return bf3 ? 2 * 2 * (DK * (DK + 8) + DK * (DV + DK + 8)) : 4 * (DK * (DK + 1) + DK * (DV + DK + 1));
}
__host__ __device__ constexpr int query_smem_bytes_f32(int C, int DK, int DV) {
  return 4 * (2 * C * (DK + 1) + C * (DV + 1) + DK * ((DK > DV ? DK : DV) + 1) + C * kLamCapG);
}
// bfloat16 inputs (dk >= 32): the query rows (two, each high and low parts) and the node matrix
// (high and low parts) in bf16, rows padded by 8 elements, and the lambda rows' levels above the
// chunk in fp32 (the outputs stay in the registers): 39.2 KB at chunk 32, d = 64, four workgroups
// per compute unit
__host__ __device__ constexpr int query_jlev(int C) { return C == 16 ? 5 : C == 32 ? 6 : 7; }
// node images 64 wide are unpadded (their windows permuted per row instead)
__host__ __device__ constexpr int query_node_ld(int DK, int DV) {
  return (DK > DV ? DK : DV) == 64 ? 64 : (DK > DV ? DK : DV) + 8;
}
__host__ __device__ constexpr int query_smem_bytes_bf3(int C, int DK, int DV) {
  return 2 * 2 * C * (DK + 8) + 2 * 2 * DK * query_node_ld(DK, DV) + 4 * C * (kLamCapG - query_jlev(C));
}
__host__ __device__ constexpr int query_smem_bytes(int C, int DK, int DV, bool bf) {
  return bf && DK >= 32 ? query_smem_bytes_bf3(C, DK, DV) : query_smem_bytes_f32(C, DK, DV);
}
// the larger of the two (the shape checks, which do not depend on the input type)
__host__ __device__ constexpr int query_smem_bytes(int C, int DK, int DV) {
  return query_smem_bytes_f32(C, DK, DV) > query_smem_bytes_bf3(C, DK, DV) ? query_smem_bytes_f32(C, DK, DV)
                                                                           : query_smem_bytes_bf3(C, DK, DV);
}

// shared-memory layout of gdn_chunk (floats; float32 row strides padded by one)
template <int C, int DK, int DV, bool BF>
struct ChunkSmem {
  static constexpr bool QB = chunk_qb(BF, C, DK), LB = chunk_lb(BF, C, DK);
  static constexpr int SK = DK + 1, SV = DV + 1, SC = C + 1, SQ = QB ? DK + 8 : SK, LW = chunk_lw(C);
  static constexpr int SU = LB ? DV + 8 : SV, SW = DK + 8;   // U or U' (bf16 images), W'' images
  static constexpr int SVB = DV + 8, SM = C + 8;   // (LB) v's bf16 image, the attention matrix's images
  static constexpr int Q = 0, K = Q + (QB ? C * SQ / 2 : C * SK), V = K + (QB ? C * SQ / 2 : C * SK),
                       M1 = V + (LB ? C * SVB / 2 : C * SV), M2 = M1 + (LB ? C * SM : C * SC), Y = M2 + C * SC, W = Y + C * SC, U = W + C * SK,
                       LAM = U + C * SU, AL = LAM + C * LW, BT = AL + C, BE = BT + C, TOTAL = BE + C;
  static constexpr int KH = QB ? M2 : Q;   // Khat (float32, stride SK), where the leaf needs it (!LB)
  static constexpr int BYTES = TOTAL * 4;
  static_assert(BYTES == chunk_smem_bytes(C, DK, DV, BF), "layout and size formula agree");
  static_assert(LB || !QB || KH + C * SK <= W, "Khat fits the buffers of Lqk and Tm^{-1}");
  static_assert(!LB || (2 * C * SW <= 2 * 4 * C * SC && C * SW == 2 * (K - Q)),
                "W'' high parts fit the buffers of Lqk and Tm^{-1}, its low parts q's");
  static_assert(K % 2 == 0 && M2 % 2 == 0 && U % 2 == 0 && (C * SU) % 4 == 0,
                "bf16 images start on 8-byte boundaries (transposing reads)");
  static_assert(!LB || (V % 4 == 0 && M1 % 4 == 0 && (C * SM) % 8 == 0),
                "v's image and the attention matrix's start on 16-byte boundaries");
};

// gdn_chunk: per (chunk, head) the intra-chunk output, the query rows carried to the chunk's
// start, and the chunk's Fenwick leaf (state and transition). Rows past T are zero inputs with
// beta = 0 and log_a = 0 (A = I there), so they change nothing and their outputs are not stored.
template <typename T, int C, int DK, int DV>
__global__ __launch_bounds__(kNT) void gdn_chunk_kernel(GdnParams p) {
  static_assert(C <= 64, "one lane per position in the log_a scan");
  using S = ChunkSmem<C, DK, DV, std::is_same<T, bf16>::value>;
  constexpr int SK = S::SK, SV = S::SV, SC = S::SC, SQ = S::SQ;
  extern __shared__ __attribute__((aligned(16))) float sm[];
  // q, k: bf16 images (QB) or float32 (row stride SQ); Khat: float32, in q's buffer or (QB) those
  // of Lqk and Tm^{-1}
  typedef typename std::conditional<S::QB, bf16, float>::type QT;
  QT* Qs = reinterpret_cast<QT*>(sm + S::Q);
  QT* Ks = reinterpret_cast<QT*>(sm + S::K);
  float* Kh = sm + S::KH;
  float* Vs = sm + S::V;
  float* M1 = sm + S::M1; float* M2 = sm + S::M2; float* Ti = sm + S::Y;
  float* Ws = sm + S::W;  float* Us = sm + S::U;  float* lam = sm + S::LAM;
  float* al = sm + S::AL; float* bt = sm + S::BT; float* be = sm + S::BE;

  const int tid = threadIdx.x;
  const int c = blockIdx.x % p.nchunks, bh = blockIdx.x / p.nchunks;
  const int t0 = c * C;
  const int nv = min(C, p.T - t0);
  const size_t row0 = (size_t)bh * p.T + t0;          // first input row of the chunk
  const size_t wrow0 = ((size_t)bh * p.nchunks + c) * C;   // first workspace row of the chunk
  const T* qg = reinterpret_cast<const T*>(p.q);
  const T* kg = reinterpret_cast<const T*>(p.k);
  const T* vg = reinterpret_cast<const T*>(p.v);

  {
    StagedBlock<T, C, DK> sq, sk;
    StagedBlock<T, C, DV> sv;
    StagedLambda<C, S::LW> sl;
    sq.load(qg + row0 * DK, DK, nv, tid);
    sk.load(kg + row0 * DK, DK, nv, tid);
    sv.load(vg + row0 * DV, DV, nv, tid);
    sl.load(p, row0, nv, tid);
    if constexpr (S::QB) {
      sq.store_raw(Qs, SQ, tid);
      sk.store_raw(Ks, SQ, tid);
    } else {
      sq.store(Qs, SK, tid);
      sk.store(Ks, SK, tid);
    }
    if constexpr (S::LB) sv.store_raw(reinterpret_cast<bf16*>(Vs), S::SVB, tid);
    else sv.store(Vs, SV, tid);
    sl.store(lam, tid);
  }
  if (tid < 64) {      // chunk-local inclusive prefix of log_a, one position per lane
    float x = tid < nv ? p.log_a[row0 + tid] : 0.f;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const float y = __shfl_up(x, d);
      if (tid >= d) x += y;
    }
    if (tid < C) {
      const float b = tid < nv ? p.beta[row0 + tid] : 0.f;
      al[tid] = x;
      bt[tid] = b;
      be[tid] = b * __expf(x);
    }
  }
  for (int i = tid; i < C * C; i += kNT) Ti[(i / C) * SC + (i % C)] = 0.f;
  __syncthreads();
  const float g = al[C - 1];

  // Tm = I + M1, M1 its strictly lower part; exp of a difference of prefixes, never above 1
  auto tm_lower = [&](int i, int j, float x) { M1[i * SC + j] = j < i ? bt[i] * x * __expf(al[i] - al[j]) : 0.f; };
  if constexpr (S::QB) gemm_bf1_nt<C, C, DK>(Ks, SQ, Ks, SQ, tid, tm_lower);
  else gemm_f32<C, C, DK, false, true>(Ks, SQ, Ks, SQ, tid, tm_lower);
  __syncthreads();

  // Ti = Tm^{-1} (unit lower triangular): the 16 x 16 diagonal blocks by forward substitution,
  // one column per thread; then blocks doubled, [A 0; B D]^{-1} = [A^{-1} 0; -D^{-1} B A^{-1}
  // D^{-1}], with M2 as scratch for B A^{-1}
  if (tid < C) {
    const int b0 = (tid / 16) * 16, col = tid % 16;
    float x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float r = i == col ? 1.f : 0.f;
      const float* mrow = M1 + (b0 + i) * SC + b0;
#pragma unroll
      for (int j = 0; j < i; ++j) r -= mrow[j] * x[j];
      x[i] = r;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Ti[(b0 + i) * SC + b0 + col] = x[i];
  }
  __syncthreads();
  auto merge = [&](auto nc) {
    constexpr int n = decltype(nc)::value;
    for (int p0 = 0; p0 < C; p0 += 2 * n) {
      gemm_f32<n, n, n, false, false>(M1 + (p0 + n) * SC + p0, SC, Ti + p0 * SC + p0, SC, tid,
                                      [&](int i, int j, float x) { M2[i * SC + j] = x; });
      __syncthreads();
      gemm_f32<n, n, n, false, false>(Ti + (p0 + n) * SC + p0 + n, SC, M2, SC, tid,
                                      [&](int i, int j, float x) { Ti[(p0 + n + i) * SC + p0 + j] = -x; });
      __syncthreads();
    }
  };
  if constexpr (C > 16) merge(std::integral_constant<int, 16>{});
  if constexpr (C > 32) merge(std::integral_constant<int, 32>{});

  // W = Ti diag(beta e^a) K, U = Ti diag(beta) V; Lqk into M2 (its scratch use is over)
  gemm_f32<C, DK, C, false, false>(Ti, SC, Ks, SQ, tid, [&](int i, int d, float x) { Ws[i * SK + d] = x; }, be);
  if constexpr (S::LB) {   // U' = diag(e^{g-a}) U as high and low bf16 images
    bf16* Uh = reinterpret_cast<bf16*>(Us);
    gemm_f32<C, DV, C, false, false>(Ti, SC, reinterpret_cast<const bf16*>(Vs), S::SVB, tid, [&](int i, int e, float x) {
      const float y = __expf(g - al[i]) * x;
      const bf16 h = (bf16)y;
      Uh[i * S::SU + e] = h;
      Uh[C * S::SU + i * S::SU + e] = (bf16)(y - (float)h);
    }, bt);
  } else {
    gemm_f32<C, DV, C, false, false>(Ti, SC, Vs, SV, tid, [&](int i, int e, float x) { Us[i * SV + e] = x; }, bt);
  }
  auto lqk = [&](int i, int j, float x) { M2[i * SC + j] = j <= i ? x * __expf(al[i] - al[j]) : 0.f; };
  if constexpr (S::QB) gemm_bf1_nt<C, C, DK>(Qs, SQ, Ks, SQ, tid, lqk);
  else gemm_f32<C, C, DK, false, true>(Qs, SQ, Ks, SQ, tid, lqk);
  __syncthreads();

  // X0 = diag(e^a) Q - Lqk W (to the workspace); M1 <- (Lqk Ti diag(beta)) * Lambda, the
  // attention matrix inside the chunk under the level weights (Tm is no longer read). X0 and the
  // intra-chunk outputs are read only by the query kernel, after the up-sweep: stored
  // non-temporally, they leave the caches to the leaves the up-sweep reads next
  float* x0g = p.x0 + wrow0 * DK;
  gemm_f32<C, DK, C, false, false>(M2, SC, Ws, SK, tid, [&](int i, int d, float x) {
    __builtin_nontemporal_store(__expf(al[i]) * to_f(Qs[i * SQ + d]) - x, &x0g[(size_t)i * DK + d]);
  });
  gemm_f32<C, C, C, false, false>(M2, SC, Ti, SC, tid, [&](int i, int j, float x) {
    const float y = j <= i ? x * bt[j] * lam[i * S::LW + bit_length((unsigned)(i ^ j))] : 0.f;
    if constexpr (S::LB) {   // high and low bf16 images
      bf16* Mh = reinterpret_cast<bf16*>(M1);
      const bf16 h = (bf16)y;
      Mh[i * S::SM + j] = h;
      Mh[C * S::SM + i * S::SM + j] = (bf16)(y - (float)h);
    } else {
      M1[i * SC + j] = y;
    }
  });
  __syncthreads();

  // O_intra = M1 V (to the workspace); Khat = diag(e^{g-a}) K, or (LB) W'' = diag(e^{g-a}) W as
  // high and low bf16 images (q, Lqk and Tm^{-1} are done)
  float* oig = p.oi + wrow0 * DV;
  auto put_oi = [&](int i, int e, float x) { __builtin_nontemporal_store(x, &oig[(size_t)i * DV + e]); };
  if constexpr (S::LB) {
    const bf16* Mh = reinterpret_cast<const bf16*>(M1);
    gemm_bf2_nn<C, DV, C>(Mh, Mh + C * S::SM, S::SM, reinterpret_cast<const bf16*>(Vs), S::SVB, tid, put_oi);
  } else {
    gemm_f32<C, DV, C, false, false>(M1, SC, Vs, SV, tid, put_oi);
  }
  bf16* Wh = reinterpret_cast<bf16*>(sm + S::M2);
  bf16* Wl = reinterpret_cast<bf16*>(sm + S::Q);
  for (int i = tid; i < C * DK; i += kNT) {
    const int r = i / DK, d = i % DK;
    if constexpr (S::LB) {
      const float y = __expf(g - al[r]) * Ws[r * SK + d];
      const bf16 h = (bf16)y;
      Wh[r * S::SW + d] = h;
      Wl[r * S::SW + d] = (bf16)(y - (float)h);
    } else {
      Kh[r * SK + d] = __expf(g - al[r]) * to_f(Ks[r * SQ + d]);
    }
  }
  __syncthreads();

  // the chunk's leaf: N = Khat^T U, Phi = e^g I - Khat^T W
  const size_t slot = (size_t)bh * p.nslot + c;
  float* ng = p.node + slot * DK * DV;
  float* pg = p.phi + slot * DK * DK;
  // split nodes: high and low parts straight from the accumulators (staging them through shared
  // memory for 16-byte stores cost more in barriers than it saved)
  constexpr bool NSPLIT = nodes_split<T, DK>();
  auto put_n = [&](int d, int e, float x) {
    if constexpr (NSPLIT) put_split(ng, DK * DV, d * DV + e, x);
    else ng[(size_t)d * DV + e] = x;
  };
  const float eg = __expf(g);
  auto put_phi = [&](int d, int d2, float x) {
    const float y = (d == d2 ? eg : 0.f) - x;
    if constexpr (NSPLIT) put_split(pg, DK * DK, d * DK + d2, y);
    else pg[(size_t)d * DK + d2] = y;
  };
  if constexpr (S::LB) {   // N = K^T U', Phi = e^g I - K^T W''
    const bf16* Kb = reinterpret_cast<const bf16*>(Ks);
    const bf16* Uh = reinterpret_cast<const bf16*>(Us);
    gemm_bf2_tn<DK, DV, C>(Kb, SQ, Uh, Uh + C * S::SU, S::SU, tid, put_n);
    gemm_bf2_tn<DK, DK, C>(Kb, SQ, Wh, Wl, S::SW, tid, put_phi);
  } else {
    gemm_f32<DK, DV, C, true, false>(Kh, SK, Us, SV, tid, put_n);
    gemm_f32<DK, DK, C, true, false>(Kh, SK, Ws, SK, tid, put_phi);
  }
}

// shared-memory layout of gdn_upsweep: the right child's transition and one panel of the left
// child's [N | Phi]
template <int DK, int DV, bool WHOLE>
struct UpSmem {
  static constexpr int SP = DK + 1, PW = up_panel(DK, DV, WHOLE), SW = PW + 1;
  static constexpr int PHI = 0, PAN = PHI + DK * SP, TOTAL = PAN + DK * SW;
  static constexpr int BYTES = TOTAL * 4;
  static_assert(BYTES == up_smem_bytes(DK, DV, WHOLE), "layout and size formula agree");
};

// gdn_upsweep (level j >= 1): node (j, m) from its children L = (j-1, 2m), R = (j-1, 2m+1):
//   [N | Phi](j, m) = Phi_R [N_L | Phi_L] + [N_R | 0]
// one workgroup per (node, head, panel of [N | Phi]); WHOLE: the panel is the whole row.
template <int DK, int DV, bool WHOLE>
__global__ __launch_bounds__(kNT) void gdn_upsweep_kernel(GdnParams p) {
  using S = UpSmem<DK, DV, WHOLE>;
  constexpr int SP = S::SP, PW = S::PW, SW = S::SW, NPAN = (DV + DK) / PW;
  extern __shared__ float sm[];
  float* Pr = sm + S::PHI;
  float* Pan = sm + S::PAN;
  const int tid = threadIdx.x;
  const int pan = blockIdx.x % NPAN;
  const int rest = blockIdx.x / NPAN;
  const int m = rest % p.ncur, bh = rest / p.ncur;
  const size_t base = (size_t)bh * p.nslot;
  const size_t sl = base + p.off_prev + 2 * m, sr = sl + 1, so = base + p.off_cur + m;
  const float* nr = p.node + sr * DK * DV;
  if constexpr (WHOLE) {
    {
      StagedBlock<float, DK, DK> sp, sf;
      StagedBlock<float, DK, DV> sn;
      sp.load(p.phi + sr * DK * DK, DK, DK, tid);
      sn.load(p.node + sl * DK * DV, DV, DK, tid);
      sf.load(p.phi + sl * DK * DK, DK, DK, tid);
      sp.store(Pr, SP, tid);
      sn.store(Pan, SW, tid);
      sf.store(Pan + DV, SW, tid);
    }
    __syncthreads();
    float* on = p.node + so * DK * DV;
    float* of = p.phi + so * DK * DK;
    // the N columns, then the Phi columns (two products, each over its own output tiles)
    gemm_f32<DK, DV, DK, false, false>(Pr, SP, Pan, SW, tid, [&](int r, int cc, float x) {
      on[(size_t)r * DV + cc] = x + nr[(size_t)r * DV + cc];
    });
    gemm_f32<DK, DK, DK, false, false>(Pr, SP, Pan + DV, SW, tid, [&](int r, int cc, float x) {
      of[(size_t)r * DK + cc] = x;
    });
  } else {
    const bool isN = pan * PW < DV;                      // panel of N (else of Phi)
    const int col0 = isN ? pan * PW : pan * PW - DV;
    {
      StagedBlock<float, DK, DK> sp;
      StagedBlock<float, DK, PW> sc;
      sp.load(p.phi + sr * DK * DK, DK, DK, tid);
      if (isN) sc.load(p.node + sl * DK * DV + col0, DV, DK, tid);
      else sc.load(p.phi + sl * DK * DK + col0, DK, DK, tid);
      sp.store(Pr, SP, tid);
      sc.store(Pan, SW, tid);
    }
    __syncthreads();
    if (isN) {
      float* out = p.node + so * DK * DV;
      gemm_f32<DK, PW, DK, false, false>(Pr, SP, Pan, SW, tid, [&](int r, int cc, float x) {
        out[(size_t)r * DV + col0 + cc] = x + nr[(size_t)r * DV + col0 + cc];
      });
    } else {
      float* out = p.phi + so * DK * DK;
      gemm_f32<DK, PW, DK, false, false>(Pr, SP, Pan, SW, tid, [&](int r, int cc, float x) {
        out[(size_t)r * DK + col0 + cc] = x;
      });
    }
  }
}

// gdn_upsweep2 (levels j and j + 1 in one launch; dk <= 64): node (j + 1, m) as the fold of its
// four grandchildren G0..G3 = (j - 1, 4m .. 4m + 3) in order, X <- Phi_G X + [N_G | 0] from
// X = [N_G0 | Phi_G0] (the same products as the two levels' merges, associated from the left):
// after G1, X is node (j, 2m), stored because the query reads the even nodes of every level;
// after G3 it is node (j + 1, m), stored. The odd node (j, 2m + 1), read by nothing but its
// parent, is never formed, and the level-j nodes are never read back. One workgroup per node
// (j + 1, m) and head, plus, where level j has an odd node count, one that folds G0, G1 only
// (level j's last node, which has no sibling). Each product's output tiles stay in the
// registers until every wave has read X, then overwrite it in place. BF3 (bfloat16 inputs,
// dk >= 32): the nodes are stored split (nodes_split), Phi_G and X are held as high and low bf16
// images (copied in as stored) and multiplied in split bf16 as in gemm_bf3, N_G goes through the
// images' state columns to be added in float32, and a stored node is copied out of the images.
template <int DK, int DV, bool BF3>
struct Up2Smem {
  static constexpr int NC = DV + DK;
  static constexpr int SP = BF3 ? DK + 8 : DK + 1, SW = BF3 ? NC + 8 : NC + 1;   // row strides
  static constexpr int ABYTES = BF3 ? DK * SP * 2 : DK * SP * 4, XBYTES = BF3 ? DK * SW * 2 : DK * SW * 4;
  // A (high), [A low], X (high), [X low]
  static constexpr int A = 0, AL = A + ABYTES, X = AL + (BF3 ? ABYTES : 0), XL = X + XBYTES,
                       TOTAL = XL + (BF3 ? XBYTES : 0);
  static_assert(TOTAL == up2_smem_bytes(DK, DV, BF3), "layout and size formula agree");
  static_assert(!BF3 || (ABYTES % 16 == 0 && XBYTES % 16 == 0), "16-byte aligned images");
};

template <int DK, int DV, bool BF3>
__global__ __launch_bounds__(kNT) __attribute__((amdgpu_waves_per_eu(3))) void gdn_upsweep2_kernel(GdnParams p) {
  static_assert(!BF3 || DK % 32 == 0, "32-deep split-bf16 steps");
  using S = Up2Smem<DK, DV, BF3>;
  constexpr int SP = S::SP, NC = S::NC, SW = S::SW;
  // wave w: row tile w % RT (its A fragments loaded once per step of the contraction) and
  // column tiles w / RT + WPR * t, t < PERW (those past TN skipped)
  constexpr int TN = NC / 16, RT = DK / 16, NWAVE = kNT / 64;
  constexpr int WPR = NWAVE / RT, PERW = (TN + WPR - 1) / WPR;
  static_assert(NWAVE % RT == 0, "whole row tiles per wave");
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  extern __shared__ __attribute__((aligned(16))) unsigned char smu[];
  float* A = reinterpret_cast<float*>(smu + S::A);
  float* X = reinterpret_cast<float*>(smu + S::X);
  bf16* Ah = reinterpret_cast<bf16*>(smu + S::A);
  bf16* Al = reinterpret_cast<bf16*>(smu + S::AL);
  bf16* Xh = reinterpret_cast<bf16*>(smu + S::X);
  bf16* Xl = reinterpret_cast<bf16*>(smu + S::XL);
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jl = lane & 15, g = lane >> 4;
  // two levels: one workgroup per node (j + 1, m) plus one for level j's unpaired last node;
  // one level (the top one): its even nodes only (nothing reads the odd ones)
  const int npair = p.two ? p.ncur >> 1 : 0;
  const int nwg = p.two ? npair + (p.ncur & 1) : (p.ncur + 1) >> 1;
  const int m = blockIdx.x % nwg, bh = blockIdx.x / nwg;
  const int steps = m < npair ? 3 : 1;
  const size_t base = (size_t)bh * p.nslot;
  const size_t g0 = base + p.off_prev + 4 * m;
  const int i0 = (w % RT) * 16, c0 = w / RT;
  auto col_tile = [&](int t) { return c0 + WPR * t; };
  // BF3: the nodes are stored as high and low bf16 parts, copied into the images as they are
  auto hi_of = [](const float* at) { return reinterpret_cast<const bf16*>(at); };
  if constexpr (BF3) {
    StagedBlock<bf16, DK, DV> snh, snl;
    StagedBlock<bf16, DK, DK> sfh, sfl, sah, sal;
    snh.load(hi_of(p.node + g0 * DK * DV), DV, DK, tid);
    snl.load(hi_of(p.node + g0 * DK * DV) + DK * DV, DV, DK, tid);
    sfh.load(hi_of(p.phi + g0 * DK * DK), DK, DK, tid);
    sfl.load(hi_of(p.phi + g0 * DK * DK) + DK * DK, DK, DK, tid);
    sah.load(hi_of(p.phi + (g0 + 1) * DK * DK), DK, DK, tid);
    sal.load(hi_of(p.phi + (g0 + 1) * DK * DK) + DK * DK, DK, DK, tid);
    snh.store_raw(Xh, SW, tid);
    snl.store_raw(Xl, SW, tid);
    sfh.store_raw(Xh + DV, SW, tid);
    sfl.store_raw(Xl + DV, SW, tid);
    sah.store_raw(Ah, SP, tid);
    sal.store_raw(Al, SP, tid);
  } else {
    StagedBlock<float, DK, DV> sn;
    StagedBlock<float, DK, DK> sf, sa;
    sn.load(p.node + g0 * DK * DV, DV, DK, tid);
    sf.load(p.phi + g0 * DK * DK, DK, DK, tid);
    sa.load(p.phi + (g0 + 1) * DK * DK, DK, DK, tid);
    sn.store(X, SW, tid);
    sf.store(X + DV, SW, tid);
    sa.store(A, SP, tid);
  }
  __syncthreads();
  for (int s = 1; s <= steps; ++s) {
    const size_t gs = g0 + s;
    // N of G_s for the state columns and the next transition, in flight during the product
    // float32: the lane's elements of N_G directly; split: N_G's 16-byte vectors, which go
    // through the images' state columns once the product has read them
    float nadd[BF3 ? 1 : PERW][4];
    if constexpr (!BF3) {
#pragma unroll
      for (int t = 0; t < PERW; ++t) {
        const int j0 = col_tile(t) * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          nadd[t][r] = j0 < DV ? p.node[gs * DK * DV + (size_t)(i0 + 4 * g + r) * DV + j0 + jl] : 0.f;
      }
    }
    StagedBlock<bf16, DK, BF3 ? DV : 16> nah, nal;
    if constexpr (BF3) {
      nah.load(hi_of(p.node + gs * DK * DV), DV, DK, tid);
      nal.load(hi_of(p.node + gs * DK * DV) + DK * DV, DV, DK, tid);
    }
    StagedBlock<float, DK, BF3 ? 16 : DK> nxt;      // float32 transitions
    StagedBlock<bf16, DK, BF3 ? DK : 16> nxh, nxl;   // split transitions
    if (s < steps) {
      if constexpr (BF3) {
        nxh.load(hi_of(p.phi + (gs + 1) * DK * DK), DK, DK, tid);
        nxl.load(hi_of(p.phi + (gs + 1) * DK * DK) + DK * DK, DK, DK, tid);
      } else {
        nxt.load(p.phi + (gs + 1) * DK * DK, DK, DK, tid);
      }
    }
    f32x4 acc[PERW];
#pragma unroll
    for (int t = 0; t < PERW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (BF3) {
#pragma unroll 1
      for (int k = 0; k < DK; k += 32) {
        const bf16x8 ah = frag_rows(Ah, SP, i0 + jl, k + 8 * g), al = frag_rows(Al, SP, i0 + jl, k + 8 * g);
#pragma unroll
        for (int t = 0; t < PERW; ++t) {
          if (col_tile(t) < TN) {
            const int j0 = col_tile(t) * 16;
            const bf16x8 bh = frag_cols(Xh, SW, k + 8 * g, j0 + jl), bl = frag_cols(Xl, SW, k + 8 * g, j0 + jl);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc[t], 0, 0, 0);
          }
        }
      }
    } else {
#pragma unroll 1
      for (int k = 0; k < DK; k += 4) {
        const float a = A[(i0 + jl) * SP + k + g];
#pragma unroll
        for (int t = 0; t < PERW; ++t)
          if (col_tile(t) < TN)
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x4f32(a, X[(k + g) * SW + col_tile(t) * 16 + jl], acc[t], 0, 0, 0);
      }
    }
    __syncthreads();   // every wave has read A and X
    if constexpr (BF3) {
      // N_G into the state columns of the images (read back below by the lane that owns each
      // element), the next transition into A's
      nah.store_raw(Xh, SW, tid);
      nal.store_raw(Xl, SW, tid);
      if (s < steps) {
        nxh.store_raw(Ah, SP, tid);
        nxl.store_raw(Al, SP, tid);
      }
      __syncthreads();
    }
    const bool out = s != 2;
    const size_t slot = s == 1 ? base + p.off_cur + 2 * m : base + p.off_next + m;
#pragma unroll
    for (int t = 0; t < PERW; ++t) {
      if (col_tile(t) < TN) {
        const int j0 = col_tile(t) * 16, col = j0 + jl;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = i0 + 4 * g + r;
          if constexpr (BF3) {
            float x = acc[t][r];
            if (j0 < DV) x += (float)Xh[row * SW + col] + (float)Xl[row * SW + col];
            const bf16 h = (bf16)x;
            Xh[row * SW + col] = h;
            Xl[row * SW + col] = (bf16)(x - (float)h);
          } else {
            const float x = acc[t][r] + nadd[t][r];
            X[row * SW + col] = x;
            if (out) {
              if (j0 < DV) p.node[slot * DK * DV + (size_t)row * DV + col] = x;
              else p.phi[slot * DK * DK + (size_t)row * DK + col - DV] = x;
            }
          }
        }
      }
    }
    if constexpr (!BF3) {
      if (s < steps) nxt.store(A, SP, tid);
    }
    __syncthreads();
    if constexpr (BF3) {
      // the stored node's high and low parts from the images, 16 bytes at a time (the next
      // product only reads the images)
      if (out) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        constexpr int VR = NC / 8;   // 16-byte vectors per image row
        bf16* nh = reinterpret_cast<bf16*>(p.node + slot * DK * DV);
        bf16* fh = reinterpret_cast<bf16*>(p.phi + slot * DK * DK);
        for (int v = tid; v < 2 * DK * VR; v += kNT) {
          const int part = v / (DK * VR), row = (v / VR) % DK, col = (v % VR) * 8;
          const u32x4 x = *reinterpret_cast<const u32x4*>((part ? Xl : Xh) + row * SW + col);
          if (col < DV) *reinterpret_cast<u32x4*>(nh + part * DK * DV + row * DV + col) = x;
          else *reinterpret_cast<u32x4*>(fh + part * DK * DK + row * DK + col - DV) = x;
        }
      }
    }
  }
}

// gdn_query's (chunk, head) of this workgroup. Consecutive workgroups go to the 8 XCDs in turn,
// each with its own L2; where the heads divide evenly, head h's chunks all run on XCD h % 8 (in
// chunk order), so the nodes a head's chunks share are read through one L2.
__device__ __forceinline__ void query_block(const GdnParams& p, int& c, int& bh) {
  const int b = blockIdx.x;
  if (p.BH % 8 == 0) {
    const int k = b >> 3;
    bh = (b & 7) + 8 * (k / p.nchunks);
    c = k % p.nchunks;
  } else {
    c = b % p.nchunks;
    bh = b / p.nchunks;
  }
}

// shared-memory layout of gdn_query: query rows (two copies, for X <- X Phi), outputs, one node
// matrix at a time, lambda rows
template <int C, int DK, int DV>
struct QuerySmem {
  static constexpr int SK = DK + 1, SV = DV + 1, MD = DK > DV ? DK : DV, SM = MD + 1;
  static constexpr int X = 0, XN = X + C * SK, O = XN + C * SK, MAT = O + C * SV,
                       LAM = MAT + DK * SM, TOTAL = LAM + C * kLamCapG;
  static constexpr int BYTES = TOTAL * 4;
  static_assert(BYTES == query_smem_bytes_f32(C, DK, DV), "layout and size formula agree");
};

// shared-memory layout of gdn_query's split-bf16 form (bytes): the query rows (two, high and
// low parts), outputs (fp32), one node matrix (high and low parts), lambda rows (fp32)
template <int C, int DK, int DV>
struct QuerySmemB {
  static constexpr int SX = DK + 8, MD = DK > DV ? DK : DV, SMB = query_node_ld(DK, DV);
  static constexpr bool SW = MD == 64;   // node images with permuted windows (swz_col)
  static constexpr int J1 = query_jlev(C), LW = kLamCapG - J1;   // lambda levels J1 .. 23
  static constexpr int XB = C * SX * 2, MB = DK * SMB * 2;
  static constexpr int X = 0, MH = X + 2 * XB, ML = MH + MB, LAM = ML + MB, TOTAL = LAM + C * LW * 4;
  static_assert(TOTAL == query_smem_bytes_bf3(C, DK, DV), "layout and size formula agree");
  static_assert(XB % 16 == 0 && MB % 16 == 0, "16-byte aligned images");
};

// gdn_query for bfloat16 inputs (dk >= 32): the same read-outs, every product in split bf16
// (gemm_bf3); the carried query rows are kept as high and low parts between nodes
template <int C, int DK, int DV>
__device__ __forceinline__ void gdn_query_bf3(const GdnParams& p, unsigned char* smb) {
  using S = QuerySmemB<C, DK, DV>;
  constexpr int SX = S::SX, SMB = S::SMB, LW = S::LW;
  constexpr int OPW = gemm_tiles_per_wave<C, DV>(), OTN = DV / 16, NOT = (C / 16) * OTN;
  // the carried query rows, updated in place (each wave's new tiles wait in its registers until
  // every wave has read the old rows)
  bf16* xh = reinterpret_cast<bf16*>(smb + S::X);
  bf16* xl = reinterpret_cast<bf16*>(smb + S::X + S::XB);
  bf16* Mh = reinterpret_cast<bf16*>(smb + S::MH);
  bf16* Ml = reinterpret_cast<bf16*>(smb + S::ML);
  float* lam = reinterpret_cast<float*>(smb + S::LAM);
  const int tid = threadIdx.x;
  int c, bh;
  query_block(p, c, bh);
  const int t0 = c * C;
  const int nv = min(C, p.T - t0);
  const size_t row0 = (size_t)bh * p.T + t0;
  const size_t wrow0 = ((size_t)bh * p.nchunks + c) * C;
  auto slot_of = [&](int j, int m) {
    int off = 0;
    for (int i = 0; i < j; ++i) off += p.nchunks >> i;
    return (size_t)bh * p.nslot + off + m;
  };
  auto next_bit = [&](int j) {
    const unsigned rest = (unsigned)c >> (j + 1);
    return rest ? j + 1 + __builtin_ctz(rest) : -1;
  };
  // up to d = 64 the next node's state and transition travel in registers meanwhile, as the
  // high and low bf16 parts the tree stores them in, copied into the images as they are
  constexpr bool PRE = DK <= 64;
  static_assert(PRE == nodes_split<bf16, DK>(), "split nodes exactly where they are prefetched");
  auto hi_of = [](const float* at) { return reinterpret_cast<const bf16*>(at); };
  StagedBlock<bf16, DK, PRE ? DV : 16> nbh, nbl;
  StagedBlock<bf16, DK, PRE ? DK : 16> fbh, fbl;
  auto load_node = [&](size_t slot, bool phi) {
    nbh.load(hi_of(p.node + slot * DK * DV), DV, DK, tid);
    nbl.load(hi_of(p.node + slot * DK * DV) + DK * DV, DV, DK, tid);
    if (phi) {
      fbh.load(hi_of(p.phi + slot * DK * DK), DK, DK, tid);
      fbl.load(hi_of(p.phi + slot * DK * DK) + DK * DK, DK, DK, tid);
    }
  };
  int j = c ? __builtin_ctz((unsigned)c) : -1;
  // the outputs in the registers, in gemm_bf3_t's places: tile w + 4t of the C x DV output, row
  // 4g + r of it, column (lane % 16); from the intra-chunk outputs
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, jl = lane & 15, g4 = 4 * (lane >> 4);
  float oacc[OPW][4];
#pragma unroll
  for (int t = 0; t < OPW; ++t) {
    const int tile = w + t * (kNT / 64), i0 = (tile / OTN) * 16, j0 = (tile % OTN) * 16;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      oacc[t][r] = tile < NOT ? p.oi[(wrow0 + i0 + g4 + r) * DV + j0 + jl] : 0.f;
  }
  {
    StagedBlock<float, C, DK> sx;
    StagedLambda<C, LW, S::J1> sl;
    sx.load(p.x0 + wrow0 * DK, DK, C, tid);
    sl.load(p, row0, nv, tid);
    if constexpr (PRE) {
      if (j >= 0) load_node(slot_of(j, (c >> j) - 1), next_bit(j) >= 0);
    }
    sx.store_split(xh, xl, SX, tid);
    sl.store(lam, tid);
  }
  __syncthreads();
  constexpr int XPW = gemm_tiles_per_wave<C, DK>(), XTN = DK / 16, NXT = (C / 16) * XTN;
  float xt[XPW][4];
  while (j >= 0) {
    const size_t slot = slot_of(j, (c >> j) - 1);
    const int jn = next_bit(j);
    if constexpr (S::SW) {
      nbh.store_raw_sw(Mh, tid);
      nbl.store_raw_sw(Ml, tid);
    } else if constexpr (PRE) {
      nbh.store_raw(Mh, SMB, tid);
      nbl.store_raw(Ml, SMB, tid);
    } else {
      StagedBlock<float, DK, DV> b;
      b.load(p.node + slot * DK * DV, DV, DK, tid);
      b.store_split(Mh, Ml, SMB, tid);
    }
    __syncthreads();
    // level J + 1 + j, at j of the staged levels
    gemm_bf3_t<C, DV, DK, S::SW>(xh, xl, SX, Mh, Ml, SMB, tid, [&](int t, int r, int i, int e, float x) {
      oacc[t][r] += lam[i * LW + j] * x;
    });
    __syncthreads();
    if (jn >= 0) {           // a higher node follows: X <- X Phi of this node
      if constexpr (S::SW) {
        fbh.store_raw_sw(Mh, tid);
        fbl.store_raw_sw(Ml, tid);
        load_node(slot_of(jn, (c >> jn) - 1), next_bit(jn) >= 0);
      } else if constexpr (PRE) {
        fbh.store_raw(Mh, SMB, tid);
        fbl.store_raw(Ml, SMB, tid);
        load_node(slot_of(jn, (c >> jn) - 1), next_bit(jn) >= 0);
      } else {
        StagedBlock<float, DK, DK> b;
        b.load(p.phi + slot * DK * DK, DK, DK, tid);
        b.store_split(Mh, Ml, SMB, tid);
      }
      __syncthreads();
      gemm_bf3_t<C, DK, DK, S::SW>(xh, xl, SX, Mh, Ml, SMB, tid,
                                   [&](int t, int r, int i, int d, float x) { xt[t][r] = x; });
      __syncthreads();
      // every read of the old rows and of the transition is done: the new rows go in place (the
      // next node's state joins them in this phase, and the loop's barrier follows)
#pragma unroll
      for (int t = 0; t < XPW; ++t) {
        const int tile = w + t * (kNT / 64), i0 = (tile / XTN) * 16, d0 = (tile % XTN) * 16;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (tile < NXT) {
            const bf16 h = (bf16)xt[t][r];
            xh[(i0 + g4 + r) * SX + d0 + jl] = h;
            xl[(i0 + g4 + r) * SX + d0 + jl] = (bf16)(xt[t][r] - (float)h);
          }
      }
    }
    j = jn;
  }
  // the outputs leave as whole rows: staged through the query rows' images (every read of them
  // ended at the last barrier) and written with 16-byte non-temporal stores, so that no partly
  // written line is left in L2 to be merged (rows past T are not stored)
  constexpr int SO = DV + 8, VR = DV / 8;   // staged row stride (bf16 elements), 16-byte pieces a row
  static_assert(C * SO * 2 <= S::LAM && DV % 8 == 0, "staged outputs fit the query rows' and nodes' images");
  bf16* st = reinterpret_cast<bf16*>(smb + S::X);
#pragma unroll
  for (int t = 0; t < OPW; ++t) {
    const int tile = w + t * (kNT / 64), i0 = (tile / OTN) * 16, j0 = (tile % OTN) * 16;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (tile < NOT) st[(i0 + g4 + r) * SO + j0 + jl] = (bf16)oacc[t][r];
  }
  __syncthreads();
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  bf16* og = reinterpret_cast<bf16*>(p.out);
  for (int v = tid; v < C * VR; v += kNT) {
    const int r = v / VR, c8 = (v % VR) * 8;
    if (r < nv)
      __builtin_nontemporal_store(*reinterpret_cast<const u32x4*>(st + r * SO + c8),
                                  reinterpret_cast<u32x4*>(og + (row0 + r) * DV + c8));
  }
}

// gdn_query: per (chunk, head) the Fenwick nodes of the chunk's set bits, lowest first, read out
// with the query rows carried to each node's end; plus the intra-chunk output; store.
// the split-bf16 query kernel up to chunk 32 and dk, dv = 64, where five workgroups' shared memory
// fits a compute unit (27 KB at chunk 32, d = 64), has its registers held to five waves per SIMD
// (at chunk 64 the bound would spill, and the shared memory allows four anyway)
template <typename T, int C, int DK, int DV>
constexpr int query_min_waves() {
  return std::is_same<T, bf16>::value && C <= 32 && DK >= 32 && DK <= 64 && DV <= 64 &&
                 5 * query_smem_bytes_bf3(C, DK, DV) <= 160 * 1024 ? 5 : 1;
}
template <typename T, int C, int DK, int DV>
__global__ __launch_bounds__(kNT, (query_min_waves<T, C, DK, DV>())) void gdn_query_kernel(GdnParams p) {
  if constexpr (std::is_same<T, bf16>::value && DK >= 32) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smq[];
    gdn_query_bf3<C, DK, DV>(p, smq);
    return;
  }
  using S = QuerySmem<C, DK, DV>;
  constexpr int SK = S::SK, SV = S::SV, SM = S::SM;
  constexpr int J = C == 16 ? 4 : C == 32 ? 5 : 6;
  extern __shared__ float sm[];
  float* Xa = sm + S::X;
  float* Xb = sm + S::XN;
  float* Os = sm + S::O;
  float* Ms = sm + S::MAT;
  float* lam = sm + S::LAM;
  const int tid = threadIdx.x;
  int c, bh;
  query_block(p, c, bh);
  const int t0 = c * C;
  const int nv = min(C, p.T - t0);
  const size_t row0 = (size_t)bh * p.T + t0;
  const size_t wrow0 = ((size_t)bh * p.nchunks + c) * C;
  // slot of node (j, m) of this head: the levels below j come first
  auto slot_of = [&](int j, int m) {
    int off = 0;
    for (int i = 0; i < j; ++i) off += p.nchunks >> i;
    return (size_t)bh * p.nslot + off + m;
  };
  // the set bit of c after j (the next node), or -1
  auto next_bit = [&](int j) {
    const unsigned rest = (unsigned)c >> (j + 1);
    return rest ? j + 1 + __builtin_ctz(rest) : -1;
  };
  // up to d = 64 the next node's state and transition travel in registers while the current one
  // is read out (one memory round trip per node instead of two, none for the first)
  constexpr bool PRE = DK <= 64;
  StagedBlock<float, DK, PRE ? DV : 16> nb;
  StagedBlock<float, DK, PRE ? DK : 16> fb;
  int j = c ? __builtin_ctz((unsigned)c) : -1;
  {
    StagedBlock<float, C, DK> sx;
    StagedBlock<float, C, DV> so;
    StagedLambda<C> sl;
    sx.load(p.x0 + wrow0 * DK, DK, C, tid);
    so.load(p.oi + wrow0 * DV, DV, C, tid);
    sl.load(p, row0, nv, tid);
    if constexpr (PRE) {
      if (j >= 0) {
        const size_t slot = slot_of(j, (c >> j) - 1);
        nb.load(p.node + slot * DK * DV, DV, DK, tid);
        if (next_bit(j) >= 0) fb.load(p.phi + slot * DK * DK, DK, DK, tid);
      }
    }
    sx.store(Xa, SK, tid);
    so.store(Os, SV, tid);
    sl.store(lam, tid);
  }
  __syncthreads();
  while (j >= 0) {
    const size_t slot = slot_of(j, (c >> j) - 1);
    const int jn = next_bit(j);
    if constexpr (PRE) nb.store(Ms, SM, tid);
    else stage_block<float, DK, DV>(Ms, SM, p.node + slot * DK * DV, DV, DK, tid);
    __syncthreads();
    const int lev = J + 1 + j;
    gemm_f32<C, DV, DK, false, false>(Xa, SK, Ms, SM, tid, [&](int i, int e, float x) {
      Os[i * SV + e] += lam[i * kLamCapG + lev] * x;
    });
    __syncthreads();
    if (jn >= 0) {           // a higher node follows: X <- X Phi of this node
      if constexpr (PRE) {
        fb.store(Ms, SM, tid);
        const size_t sn = slot_of(jn, (c >> jn) - 1);
        nb.load(p.node + sn * DK * DV, DV, DK, tid);
        if (next_bit(jn) >= 0) fb.load(p.phi + sn * DK * DK, DK, DK, tid);
      } else {
        stage_block<float, DK, DK>(Ms, SM, p.phi + slot * DK * DK, DK, DK, tid);
      }
      __syncthreads();
      gemm_f32<C, DK, DK, false, false>(Xa, SK, Ms, SM, tid, [&](int i, int d, float x) {
        Xb[i * SK + d] = x;
      });
      __syncthreads();
      float* tmp = Xa; Xa = Xb; Xb = tmp;
    }
    j = jn;
  }
  T* og = reinterpret_cast<T*>(p.out);
  for (int i = tid; i < C * DV; i += kNT) {
    const int r = i / DV, e = i % DV;
    if (r < nv) og[(row0 + r) * DV + e] = (T)Os[r * SV + e];
  }
}

}  // namespace gdn
}  // namespace lla

namespace lla {
namespace gdn {

// per (dtype, chunk) tables of the chunk and query kernels, indexed by (dk, dv); entries whose
// shared memory would exceed 160 KB are null
struct GdnKernels {
  const void* chunk;
  const void* query;
};
const GdnKernels* kernels_bf16_c16(int DK, int DV);
const GdnKernels* kernels_bf16_c32(int DK, int DV);
const GdnKernels* kernels_bf16_c64(int DK, int DV);
const GdnKernels* kernels_f32_c16(int DK, int DV);
const GdnKernels* kernels_f32_c32(int DK, int DV);
const GdnKernels* kernels_f32_c64(int DK, int DV);

inline int dim_index(int x) { return x == 16 ? 0 : x == 32 ? 1 : x == 64 ? 2 : x == 128 ? 3 : -1; }

// One (dtype, chunk) table: every (dk, dv) whose kernels fit shared memory.
template <typename T, int C>
struct GdnTable {
  GdnKernels k[4][4];
  template <int DK, int DV>
  static constexpr bool fits() {
    return chunk_smem_bytes(C, DK, DV) <= 160 * 1024 && query_smem_bytes(C, DK, DV) <= 160 * 1024;
  }
  template <int DK, int DV>
  void set() {
    if constexpr (fits<DK, DV>()) {
      k[dim_index(DK)][dim_index(DV)] = {reinterpret_cast<const void*>(&gdn_chunk_kernel<T, C, DK, DV>),
                                         reinterpret_cast<const void*>(&gdn_query_kernel<T, C, DK, DV>)};
    } else {
      k[dim_index(DK)][dim_index(DV)] = {nullptr, nullptr};
    }
  }
  template <int DK>
  void row() { set<DK, 16>(); set<DK, 32>(); set<DK, 64>(); set<DK, 128>(); }
  GdnTable() { row<16>(); row<32>(); row<64>(); row<128>(); }
  const GdnKernels* get(int DK, int DV) const {
    const int a = dim_index(DK), b = dim_index(DV);
    if (a < 0 || b < 0 || !k[a][b].chunk) return nullptr;
    return &k[a][b];
  }
};

}  // namespace gdn
}  // namespace lla
